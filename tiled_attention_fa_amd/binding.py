"""ctypes binding of libmiattn (the C ABI in include/libmiattn.h).

The functions ``fa_fwd``, ``fa_bwd``, ``fa_block_mask_build`` and the
helpers mirror the C entry points one to one and take raw device pointers.
``forward``, ``backward`` and ``build_block_mask`` are conveniences on top:
they allocate outputs with torch, pass ``data_ptr()`` and the current stream,
and raise ``FaError`` on a non-zero status.  No arithmetic of the method runs
here; if the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmiattn.so")

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED = 0, -1, -2, -3
FA_ERR_ALIGN, FA_ERR_PARAM, FA_ERR_WORKSPACE, FA_ERR_LAUNCH, FA_ERR_SCRATCH = -4, -5, -6, -7, -8
FA_NOALLOC_SCRATCH_BYTES = 16 << 20
FA_BF16, FA_F32 = 0, 1
MASK_NONE, MASK_CAUSAL, MASK_SLIDING_WINDOW, MASK_DOCUMENT = 0, 1, 2, 3
MOD_NONE, MOD_ALIBI, MOD_SOFTCAP, MOD_LOCAL_BOOST, MOD_REL_BIAS = 0, 1, 2, 3, 4
TILE_EMPTY, TILE_PARTIAL, TILE_FULL = 0, 1, 2
BLOCK = 128

FA_BWD_DELTA, FA_BWD_DKDV, FA_BWD_DQ = 1, 2, 4

FA_VERSION = 200  # the header's FA_VERSION: the struct layouts below
EXPORTED = ("fa_fwd", "fa_fwd_kv_step", "fa_bwd", "fa_bwd_phase", "fa_bwd_noalloc", "fa_bwd_workspace_bytes",
            "fa_bwd_ds_workspace_bytes",
            "fa_bwd_rel_bias_workspace_bytes",
            "fa_block_mask_bytes", "fa_block_mask_layout", "fa_block_mask_build", "fa_fp8_quantize", "fa_fwd_fp8",
            "fa_status_str", "fa_version")


class FaMaskParams(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("doc_ids", ctypes.c_void_p), ("visited", ctypes.c_void_p),
                ("work_queue", ctypes.c_void_p), ("wg_trace", ctypes.c_void_p)]


class FaModParams(ctypes.Structure):
    _fields_ = [("alibi_slopes", ctypes.c_void_p), ("softcap", ctypes.c_float),
                ("boost_radius", ctypes.c_int32), ("boost_factor", ctypes.c_float),
                ("rel_bias", ctypes.c_void_p), ("rel_bias_grad", ctypes.c_void_p),
                ("rel_bias_ws", ctypes.c_void_p), ("rel_bias_ws_bytes", ctypes.c_size_t)]


class FaBlockMask(ctypes.Structure):
    _fields_ = [("block_q", ctypes.c_int32), ("block_kv", ctypes.c_int32),
                ("n_q", ctypes.c_int32), ("n_kv", ctypes.c_int32), ("n_b", ctypes.c_int32),
                ("tile_state", ctypes.c_void_p), ("kv_count", ctypes.c_void_p),
                ("kv_index", ctypes.c_void_p), ("q_count", ctypes.c_void_p),
                ("q_index", ctypes.c_void_p), ("q_order", ctypes.c_void_p),
                ("kv_order", ctypes.c_void_p)]


class FaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {fa_status_str(status)} (status {status})")
        self.status = status


_LIB = None
_P = ctypes.c_void_p
_I = ctypes.c_int


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m tiled_attention_fa_amd.build`")
        L = declare_prototypes(ctypes.CDLL(LIB_PATH))
        if L.fa_version() != FA_VERSION:
            raise RuntimeError(f"{LIB_PATH} is version {L.fa_version()}, this binding needs {FA_VERSION} "
                               "(the parameter structs differ): rebuild it with `python -m tiled_attention_fa_amd.build`")
        _LIB = L
    return _LIB


def declare_prototypes(L: ctypes.CDLL) -> ctypes.CDLL:
    """Set the argument and result types of every entry point on a loaded
    copy of the library; returns it."""
    L.fa_fwd.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float,
                         _I, ctypes.POINTER(FaMaskParams), _I, ctypes.POINTER(FaModParams),
                         ctypes.POINTER(FaBlockMask), _P]
    L.fa_fwd.restype = _I
    L.fa_bwd.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                         _I, _I, _I, _I, _I, _I, _I, ctypes.c_float,
                         _I, ctypes.POINTER(FaMaskParams), _I, ctypes.POINTER(FaModParams),
                         ctypes.POINTER(FaBlockMask), _P]
    L.fa_bwd.restype = _I
    L.fa_bwd_phase.argtypes = [_I] + L.fa_bwd.argtypes
    L.fa_bwd_phase.restype = _I
    L.fa_bwd_noalloc.argtypes = L.fa_bwd.argtypes[:9] + L.fa_bwd.argtypes[11:]
    L.fa_bwd_noalloc.restype = _I
    L.fa_bwd_workspace_bytes.argtypes = [_I, _I, _I, _I]
    L.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.fa_bwd_ds_workspace_bytes.argtypes = [_I, _I, _I, _I, _I, _I]
    L.fa_bwd_ds_workspace_bytes.restype = ctypes.c_size_t
    L.fa_bwd_rel_bias_workspace_bytes.argtypes = [_I, _I, _I, _I]
    L.fa_bwd_rel_bias_workspace_bytes.restype = ctypes.c_size_t
    L.fa_block_mask_bytes.argtypes = [_I, _I, _I, _I, _I, _I]
    L.fa_block_mask_bytes.restype = ctypes.c_size_t
    L.fa_block_mask_layout.argtypes = [_P, _I, _I, _I, _I, _I, _I, ctypes.POINTER(FaBlockMask)]
    L.fa_block_mask_layout.restype = _I
    L.fa_block_mask_build.argtypes = [_I, ctypes.POINTER(FaMaskParams), _I, _I, _I,
                                      ctypes.POINTER(FaBlockMask), _P]
    L.fa_block_mask_build.restype = _I
    L.fa_status_str.argtypes = [_I]
    L.fa_status_str.restype = ctypes.c_char_p
    L.fa_fwd_kv_step.argtypes = [_I, _I]
    L.fa_fwd_kv_step.restype = _I
    L.fa_version.argtypes = []
    L.fa_version.restype = _I
    L.fa_fp8_quantize.argtypes = [_P, _P, _P, _I, _I, _I, _P, _P]
    L.fa_fp8_quantize.restype = _I
    L.fa_fwd_fp8.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float,
                             _I, ctypes.POINTER(FaMaskParams), _P]
    L.fa_fwd_fp8.restype = _I
    return L


# ---------------------------------------------------------------- raw C calls

def fa_fwd(*args) -> int:
    return lib().fa_fwd(*args)


def fa_bwd(*args) -> int:
    return lib().fa_bwd(*args)


def fa_bwd_noalloc(*args) -> int:
    return lib().fa_bwd_noalloc(*args)


def fa_bwd_phase(*args) -> int:
    return lib().fa_bwd_phase(*args)


def fa_block_mask_build(*args) -> int:
    return lib().fa_block_mask_build(*args)


def fa_bwd_workspace_bytes(B: int, Hq: int, Sq: int, D: int) -> int:
    return int(lib().fa_bwd_workspace_bytes(B, Hq, Sq, D))


def fa_bwd_ds_workspace_bytes(B: int, Hq: int, Sq: int, Skv: int, D: int, mask: int) -> int:
    return int(lib().fa_bwd_ds_workspace_bytes(B, Hq, Sq, Skv, D, mask))


def fa_bwd_rel_bias_workspace_bytes(B: int, Hq: int, Sq: int, Skv: int) -> int:
    return int(lib().fa_bwd_rel_bias_workspace_bytes(B, Hq, Sq, Skv))


def fa_fwd_kv_step(D: int, dtype: int) -> int:
    return int(lib().fa_fwd_kv_step(D, dtype))


def fa_status_str(status: int) -> str:
    return lib().fa_status_str(status).decode()


def fa_version() -> int:
    return int(lib().fa_version())


# ---------------------------------------------------------------- torch conveniences

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dense(t, what, shape=None, dtypes=None, device=None):
    """Check that ``t`` (if given) is a dense row-major tensor of ``shape``
    (None entries are free) with a dtype in ``dtypes`` on ``device``; the C
    ABI reads plain arrays from the data pointer, so a strided view or a
    tensor of another shape would be read as the wrong elements."""
    if t is None:
        return None
    if shape is not None and (t.dim() != len(shape) or
                              any(w is not None and w != g for w, g in zip(shape, t.shape))):
        raise ValueError(f"{what}: shape {tuple(t.shape)} does not match {tuple(shape)}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{what}: dtype {t.dtype} not in {tuple(dtypes)}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{what}: on {t.device}, expected {device}")
    return t


def _check_qkv(q, k, v):
    """Shapes (B, Hq, Hkv, Sq, Skv, D) of q [B,Hq,Sq,D], k and v [B,Hkv,Skv,D]."""
    torch = _torch()
    _dense(q, "q", (None, None, None, None), (torch.bfloat16, torch.float32))
    B, Hq, Sq, D = q.shape
    _dense(k, "k", (B, None, None, D), (q.dtype,), q.device)
    Hkv, Skv = k.shape[1], k.shape[2]
    _dense(v, "v", (B, Hkv, Skv, D), (q.dtype,), q.device)
    return B, Hq, Hkv, Sq, Skv, D


def _check_mod_tensors(q, Hq, Sq, Skv, doc_ids, alibi_slopes, rel_bias):
    torch = _torch()
    _dense(doc_ids, "doc_ids", (q.shape[0], Sq), (torch.int32,), q.device)
    _dense(alibi_slopes, "alibi_slopes", (Hq,), (torch.float32,), q.device)
    _dense(rel_bias, "rel_bias", (Hq, Sq + Skv - 1), (torch.float32,), q.device)


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def default_scale(D: int) -> float:
    """1/sqrt(D) as the float32 value the kernel receives."""
    return float(ctypes.c_float(1.0 / math.sqrt(D)).value)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _params(mask, window, doc_ids, visited, mod, alibi_slopes, softcap, boost_radius, boost_factor,
            rel_bias=None, rel_bias_grad=None, rel_bias_ws=None, work_queue=None, wg_trace=None):
    ptr = lambda t: None if t is None else t.data_ptr()
    mp = FaMaskParams(int(window), ptr(doc_ids), ptr(visited), ptr(work_queue), ptr(wg_trace))
    ws_bytes = 0 if rel_bias_ws is None else rel_bias_ws.numel() * rel_bias_ws.element_size()
    op = FaModParams(ptr(alibi_slopes), float(softcap), int(boost_radius), float(boost_factor),
                     ptr(rel_bias), ptr(rel_bias_grad), ptr(rel_bias_ws), int(ws_bytes))
    return mp, op


FA_WORK_QUEUE_INTS = 288


def new_work_queue(device="cuda"):
    """A zeroed work queue for the persistent forward (fa_mask_params.work_queue)."""
    return _torch().zeros(FA_WORK_QUEUE_INTS, dtype=_torch().int32, device=device)


FA_WG_TRACE_WORDS = 4


def new_wg_trace(B, Hq, Sq, device="cuda", Hkv=None, Skv=None):
    """A zeroed workgroup-trace buffer (fa_mask_params.wg_trace): for fa_fwd,
    or with Hkv and Skv given for fa_bwd (dK/dV records, then dQ records)."""
    n = B * Hq * -(-Sq // BLOCK)
    if Hkv is not None:
        n += B * Hkv * -(-(Skv if Skv is not None else Sq) // BLOCK)
    return _torch().zeros((n, FA_WG_TRACE_WORDS), dtype=_torch().int64, device=device)


def decode_wg_trace(rec):
    """Records of a wg_trace buffer (host array [n, 4]) as dicts, skipping the
    entries no tile wrote: start/end in us of the 100 MHz clock, the XCD (XCC_ID
    bits 3:0), a compute-unit key unique on the chip (XCD, and HW_ID bits 15:8:
    CU, shader array and shader engine), the static index P, rows and steps."""
    out = []
    for p, (t0, t1, loc, size) in enumerate(rec.tolist()):
        if t0 == 0 and t1 == 0:
            continue
        xcc, hw = (loc >> 32) & 0xF, loc & 0xFFFFFFFF
        out.append({"P": p, "start_us": t0 / 100.0, "end_us": t1 / 100.0, "xcd": xcc,
                    "cu": (xcc << 8) | ((hw >> 8) & 0xFF), "rows": size >> 32, "steps": size & 0xFFFFFFFF})
    return out


FP8_BLOCK = 128  # rows per FP8 quantization block


def quantize_fp8(x, signs=None, *, out=None, scales=None, stream=None):
    """E4M3 codes and per-128-row E8M0 scale bytes of a bf16 [B, H, S, D]
    tensor; with ``signs`` (float32 [D] of +-1) the rows are first multiplied
    by diag(signs) H / sqrt(D) (incoherent processing)."""
    torch = _torch()
    _dense(x, "x", (None, None, None, None), (torch.bfloat16,))
    B, H, S, D = x.shape
    _dense(signs, "signs", (D,), (torch.float32,), x.device)
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((B, H, -(-S // FP8_BLOCK)), dtype=torch.uint8, device=x.device)
    _dense(out, "out", tuple(x.shape), (torch.uint8,), x.device)
    _dense(scales, "scales", None, (torch.uint8,), x.device)
    if scales.numel() < B * H * -(-S // FP8_BLOCK):
        raise ValueError(f"scales: {scales.numel()} bytes, need {B * H * -(-S // FP8_BLOCK)}")
    rc = lib().fa_fp8_quantize(_ptr(x), _ptr(out), _ptr(scales), int(B * H), int(S), int(D), _ptr(signs),
                               _stream(stream))
    if rc != FA_OK:
        raise FaError(rc, "fa_fp8_quantize")
    return out, scales


def forward_fp8(q8, k8, v8, q_scale, k_scale, v_scale, *, scale=None, mask=MASK_NONE, window=0,
                return_lse=False, out=None, lse=None, stream=None):
    """bf16 O (and LSE) from E4M3 q8 [B,Hq,Sq,D], k8/v8 [B,Hkv,Skv,D] with their
    block scales (masks: none, causal, sliding window)."""
    torch = _torch()
    u8 = (torch.uint8,)
    _dense(q8, "q8", (None, None, None, None), u8)
    B, Hq, Sq, D = q8.shape
    _dense(k8, "k8", (B, None, None, D), u8, q8.device)
    Hkv, Skv = k8.shape[1], k8.shape[2]
    _dense(v8, "v8", (B, Hkv, Skv, D), u8, q8.device)
    for t, what, rows, n in ((q_scale, "q_scale", B * Hq, Sq), (k_scale, "k_scale", B * Hkv, Skv),
                             (v_scale, "v_scale", B * Hkv, Skv)):
        _dense(t, what, None, u8, q8.device)
        if t is not None and t.numel() < rows * -(-n // FP8_BLOCK):
            raise ValueError(f"{what}: {t.numel()} bytes, need {rows * -(-n // FP8_BLOCK)}")
    if out is None:
        out = torch.empty((B, Hq, Sq, D), dtype=torch.bfloat16, device=q8.device)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q8.device)
    _dense(out, "out", (B, Hq, Sq, D), (torch.bfloat16,), q8.device)
    _dense(lse if return_lse else None, "lse", (B, Hq, Sq), (torch.float32,), q8.device)
    mp, _ = _params(mask, window, None, None, MOD_NONE, None, 0.0, 0, 1.0)
    sc = default_scale(D) if scale is None else float(scale)
    rc = lib().fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), _ptr(out),
                          _ptr(lse), int(B), int(Hq), int(Hkv), int(Sq), int(Skv), int(D), sc, int(mask),
                          ctypes.byref(mp), _stream(stream))
    if rc != FA_OK:
        raise FaError(rc, "fa_fwd_fp8")
    return (out, lse) if return_lse else out


def fa_block_mask_bytes(n_b: int, Sq: int, Skv: int, with_orders: bool = True) -> int:
    return int(lib().fa_block_mask_bytes(n_b, Sq, Skv, BLOCK, BLOCK, int(with_orders)))


class BlockMask:
    """Device arrays of a 128 x 128 block mask, carved from one allocation
    by fa_block_mask_layout; the attributes are torch views of it."""

    def __init__(self, n_b, n_q, n_kv, device, orders=True):
        torch = _torch()
        self.n_b, self.n_q, self.n_kv = n_b, n_q, n_kv
        Sq, Skv = n_q * BLOCK, n_kv * BLOCK
        nbytes = fa_block_mask_bytes(n_b, Sq, Skv, orders)
        if nbytes == 0:
            raise FaError(FA_ERR_SHAPE, "fa_block_mask_bytes")
        self.buffer = torch.empty(nbytes, dtype=torch.uint8, device=device)
        s = FaBlockMask()
        rc = lib().fa_block_mask_layout(ctypes.c_void_p(self.buffer.data_ptr()), n_b, Sq, Skv, BLOCK, BLOCK,
                                        int(orders), ctypes.byref(s))
        if rc != FA_OK:
            raise FaError(rc, "fa_block_mask_layout")
        base = self.buffer.data_ptr()

        def view(addr, count, dtype, shape):
            if addr is None:
                return None
            o = addr - base
            n = count * (4 if dtype == torch.int32 else 1)
            return self.buffer[o:o + n].view(dtype).view(shape)

        nq1, nkv1 = max(n_q, 1), max(n_kv, 1)
        self.tile_state = view(s.tile_state, n_b * n_q * n_kv, torch.uint8, (n_b, n_q, n_kv))
        self.kv_count = view(s.kv_count, n_b * n_q, torch.int32, (n_b, n_q))
        self.kv_index = view(s.kv_index, n_b * n_q * nkv1, torch.int32, (n_b, n_q, nkv1))
        self.q_count = view(s.q_count, n_b * n_kv, torch.int32, (n_b, n_kv))
        self.q_index = view(s.q_index, n_b * nkv1 * nq1, torch.int32, (n_b, nkv1, nq1))
        # schedule orders of the tiles (optional in the C struct)
        self.q_order = view(s.q_order, n_b * nq1, torch.int32, (n_b, nq1)) if orders else None
        self.kv_order = view(s.kv_order, n_b * nkv1, torch.int32, (n_b, nkv1)) if orders else None

    def struct(self) -> FaBlockMask:
        ptr = lambda t: None if t is None else t.data_ptr()
        return FaBlockMask(BLOCK, BLOCK, self.n_q, self.n_kv, self.n_b,
                           self.tile_state.data_ptr(), self.kv_count.data_ptr(), self.kv_index.data_ptr(),
                           self.q_count.data_ptr(), self.q_index.data_ptr(), ptr(self.q_order),
                           ptr(self.kv_order))


def build_block_mask(mask: int, B: int, Sq: int, Skv: int, *, window: int = 0, doc_ids=None,
                     device="cuda", stream=None, into: BlockMask | None = None, orders: bool = True) -> BlockMask:
    """Build (or rebuild ``into``, allocating nothing) the block mask of a mask kind;
    ``orders`` adds the tile orders the kernels schedule by (longest first,
    the tiles of one document together)."""
    n_b = B if mask == MASK_DOCUMENT else 1
    if doc_ids is not None:
        _dense(doc_ids, "doc_ids", (B, Sq), (_torch().int32,))
    bm = into if into is not None else BlockMask(n_b, -(-Sq // BLOCK), -(-Skv // BLOCK), device, orders)
    mp, _ = _params(mask, window, doc_ids, None, MOD_NONE, None, 0.0, 0, 1.0)
    s = bm.struct()
    rc = fa_block_mask_build(int(mask), ctypes.byref(mp), int(B), int(Sq), int(Skv), ctypes.byref(s), _stream(stream))
    if rc != FA_OK:
        raise FaError(rc, "fa_block_mask_build")
    return bm


def forward(q, k, v, *, scale=None, mask=MASK_NONE, window=0, doc_ids=None, mod=MOD_NONE,
            alibi_slopes=None, softcap=0.0, boost_radius=0, boost_factor=1.0, rel_bias=None,
            block_mask=None, return_lse=False, out=None, lse=None, visited=None, work_queue=None, wg_trace=None,
            stream=None):
    """O (and LSE if ``return_lse``) for q [B,Hq,Sq,D], k/v [B,Hkv,Skv,D] on the GPU.

    ``rel_bias`` (MOD_REL_BIAS): float32 [Hq, Sq + Skv - 1] on the device.
    ``work_queue``: int32 [FA_WORK_QUEUE_INTS] on the device, zero before its
    first use (``new_work_queue()``): the persistent, dynamically scheduled
    kernel takes its query tiles from it and leaves it zero.
    ``wg_trace``: int64 [B * Hq * ceil(Sq / 128), FA_WG_TRACE_WORDS] on the
    device (``new_wg_trace()``), debug records of where and when each query
    tile ran."""
    torch = _torch()
    B, Hq, Hkv, Sq, Skv, D = _check_qkv(q, k, v)
    _check_mod_tensors(q, Hq, Sq, Skv, doc_ids, alibi_slopes, rel_bias)
    _dense(visited, "visited", None, (torch.int32,), q.device)
    _dense(work_queue, "work_queue", (FA_WORK_QUEUE_INTS,), (torch.int32,), q.device)
    _dense(wg_trace, "wg_trace", (B * Hq * -(-Sq // BLOCK), FA_WG_TRACE_WORDS), (torch.int64,), q.device)
    if out is None:
        out = torch.empty((B, Hq, Sq, D), dtype=q.dtype, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    _dense(out, "out", (B, Hq, Sq, D), (q.dtype,), q.device)
    _dense(lse if return_lse else None, "lse", (B, Hq, Sq), (torch.float32,), q.device)
    mp, op = _params(mask, window, doc_ids, visited, mod, alibi_slopes, softcap, boost_radius, boost_factor,
                     rel_bias, work_queue=work_queue, wg_trace=wg_trace)
    bms = block_mask.struct() if block_mask is not None else None
    rc = fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse) if return_lse else None,
                B, Hq, Hkv, Sq, Skv, D, _dtype_code(q), float(default_scale(D) if scale is None else scale),
                int(mask), ctypes.byref(mp), int(mod), ctypes.byref(op),
                ctypes.byref(bms) if bms is not None else None, _stream(stream))
    if rc != FA_OK:
        raise FaError(rc, "fa_fwd")
    return (out, lse) if return_lse else out


def backward(q, k, v, out, dout, lse, *, scale=None, mask=MASK_NONE, window=0, doc_ids=None,
             mod=MOD_NONE, alibi_slopes=None, softcap=0.0, boost_radius=0, boost_factor=1.0,
             rel_bias=None, rel_bias_grad=None, rel_bias_ws=None,
             block_mask=None, workspace=None, grads=None, stream=None,
             phases=FA_BWD_DELTA | FA_BWD_DKDV | FA_BWD_DQ, noalloc=False, store_ds=False, wg_trace=None):
    """(dq, dk, dv) of sum(O * dout), recomputing P from ``lse``.

    ``phases`` selects which backward phases run (all by default, which is
    fa_bwd; the row pass and dQ in one call share one launch).  ``noalloc``: call fa_bwd_noalloc, whose
    workspace is the library's fixed device scratch (all phases; with
    ``grads`` given and no relative-bias gradient nothing is allocated).
    ``store_ds``: allocate the stored-dS workspace (fa_bwd_ds_workspace_bytes)
    when none is given, so dQ is computed from the dS the dK/dV phase
    stores (unmasked and causal attention).  With MOD_REL_BIAS, ``rel_bias_grad`` (float32
    [Hq, Sq + Skv - 1], or True to allocate it) receives the gradient of the
    bias table; its scratch ``rel_bias_ws`` is allocated when not given.  The
    return value is then (dq, dk, dv, rel_bias_grad).  ``wg_trace``
    (``new_wg_trace(B, Hq, Sq, Hkv=Hkv, Skv=Skv)``): debug records of the
    dK/dV and dQ workgroups."""
    torch = _torch()
    B, Hq, Hkv, Sq, Skv, D = _check_qkv(q, k, v)
    _check_mod_tensors(q, Hq, Sq, Skv, doc_ids, alibi_slopes, rel_bias)
    qs, kvs = (B, Hq, Sq, D), (B, Hkv, Skv, D)
    _dense(out, "out", qs, (q.dtype,), q.device)
    _dense(dout, "dout", qs, (q.dtype,), q.device)
    _dense(lse, "lse", (B, Hq, Sq), (torch.float32,), q.device)
    if grads is None:
        grads = (torch.empty(qs, dtype=q.dtype, device=q.device), torch.empty(kvs, dtype=q.dtype, device=q.device),
                 torch.empty(kvs, dtype=q.dtype, device=q.device))
    dq, dk, dv = grads
    for t, what, shape in ((dq, "dq", qs), (dk, "dk", kvs), (dv, "dv", kvs)):
        _dense(t, what, shape, (q.dtype,), q.device)
    if noalloc:
        if workspace is not None or phases != FA_BWD_DELTA | FA_BWD_DKDV | FA_BWD_DQ:
            raise ValueError("noalloc: the workspace is the library's own, and every phase runs")
    else:
        ws_bytes = fa_bwd_workspace_bytes(B, Hq, Sq, D)
        if store_ds:
            ws_bytes = max(ws_bytes, fa_bwd_ds_workspace_bytes(B, Hq, Sq, Skv, D, mask))
        if workspace is None:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
        _dense(workspace, "workspace", None, None, q.device)
    want_bias_grad = rel_bias_grad is not None
    if rel_bias_grad is True:
        rel_bias_grad = torch.empty((Hq, Sq + Skv - 1), dtype=torch.float32, device=q.device)
    if want_bias_grad and rel_bias_ws is None:
        rel_bias_ws = torch.empty(max(fa_bwd_rel_bias_workspace_bytes(B, Hq, Sq, Skv), 16), dtype=torch.uint8,
                                  device=q.device)
    _dense(rel_bias_grad, "rel_bias_grad", (Hq, Sq + Skv - 1), (torch.float32,), q.device)
    _dense(rel_bias_ws, "rel_bias_ws", None, None, q.device)
    _dense(wg_trace, "wg_trace", (B * Hkv * -(-Skv // BLOCK) + B * Hq * -(-Sq // BLOCK), FA_WG_TRACE_WORDS),
           (torch.int64,), q.device)
    mp, op = _params(mask, window, doc_ids, None, mod, alibi_slopes, softcap, boost_radius, boost_factor,
                     rel_bias, rel_bias_grad, rel_bias_ws, wg_trace=wg_trace)
    bms = block_mask.struct() if block_mask is not None else None
    tail = (B, Hq, Hkv, Sq, Skv, D, _dtype_code(q), float(default_scale(D) if scale is None else scale),
            int(mask), ctypes.byref(mp), int(mod), ctypes.byref(op),
            ctypes.byref(bms) if bms is not None else None, _stream(stream))
    tensors = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv))
    if noalloc:
        rc = fa_bwd_noalloc(*tensors, *tail)
        if rc != FA_OK:
            raise FaError(rc, "fa_bwd_noalloc")
    else:
        rc = fa_bwd_phase(int(phases), *tensors, _ptr(workspace), workspace.numel() * workspace.element_size(), *tail)
        if rc != FA_OK:
            raise FaError(rc, "fa_bwd_phase")
    if want_bias_grad:
        return dq, dk, dv, rel_bias_grad
    return dq, dk, dv


_ATTENTION_FN = None


def _attention_fn():
    """The torch.autograd.Function behind attention(), made on first use
    (the binding imports torch lazily)."""
    global _ATTENTION_FN
    if _ATTENTION_FN is None:
        torch = _torch()

        class _Attention(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, rel_bias, opts):
                o, lse = forward(q, k, v, rel_bias=rel_bias, return_lse=True, **opts)
                ctx.save_for_backward(q, k, v, o, lse, rel_bias)
                ctx.opts = opts
                return o

            @staticmethod
            def backward(ctx, dout):
                q, k, v, o, lse, rel_bias = ctx.saved_tensors
                want_bias = rel_bias is not None and ctx.needs_input_grad[3]
                res = backward(q, k, v, o, dout.contiguous(), lse, rel_bias=rel_bias,
                               rel_bias_grad=True if want_bias else None, **ctx.opts)
                return res[0], res[1], res[2], (res[3] if want_bias else None), None

        _ATTENTION_FN = _Attention
    return _ATTENTION_FN


def attention(q, k, v, *, scale=None, mask=MASK_NONE, window=0, doc_ids=None, mod=MOD_NONE, alibi_slopes=None,
              softcap=0.0, boost_radius=0, boost_factor=1.0, rel_bias=None, block_mask=None):
    """O = softmax(mod(scale q k^T) masked) v as a differentiable torch
    operation: fa_fwd (keeping its LSE) in the forward, fa_bwd in the backward,
    giving dq, dk, dv (dk, dv summed over each GQA group) and, with MOD_REL_BIAS
    and a ``rel_bias`` that requires grad, the bias table's gradient.  The other
    arguments are those of forward() and carry no gradient.  The backward takes
    bf16 inputs, like fa_bwd."""
    opts = dict(scale=scale, mask=mask, window=window, doc_ids=doc_ids, mod=mod, alibi_slopes=alibi_slopes,
                softcap=softcap, boost_radius=boost_radius, boost_factor=boost_factor, block_mask=block_mask)
    return _attention_fn().apply(q, k, v, rel_bias, opts)
