"""The C ABI on the host: the library loads, exports every symbol the header
declares, and rejects invalid arguments before touching the GPU (CPU only;
no call here reaches a kernel launch)."""
import ctypes
import os
import re
import subprocess

import pytest

import tiled_attention_fa_amd as fa
from tiled_attention_fa_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libmiattn.h")


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(binding.LIB_PATH):
        from tiled_attention_fa_amd import build
        build.build()
    alt = os.environ.get("MIATTN_ABI_TEST_LIB")
    if alt:
        # The validation layer built on its own with the host sanitizers and
        # launchers that only report failure (tests/test_abi_sanitized.py):
        # the calls below exercise it instead of the GPU library's copy.
        binding._LIB = binding.declare_prototypes(ctypes.CDLL(alt))
        yield binding._LIB
        binding._LIB = None
        return
    yield fa.lib()


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for name in declared():
        assert name in syms, name
        assert hasattr(fa.lib(), name)


def test_host_helpers():
    assert fa.fa_version() == binding.FA_VERSION
    assert fa.fa_status_str(0) == "ok"
    assert "workspace" in fa.fa_status_str(fa.FA_ERR_WORKSPACE)
    assert fa.fa_fwd_kv_step(128, fa.FA_BF16) == 64
    assert fa.fa_fwd_kv_step(64, fa.FA_F32) == 32
    assert fa.fa_fwd_kv_step(96, fa.FA_BF16) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_bwd_workspace_bytes(2, 16, 8192, 128) == 2 * (2 * 16 * 8192 * 4)
    assert fa.fa_bwd_workspace_bytes(1, 1, 10, 64) == 2 * 256
    assert fa.fa_bwd_workspace_bytes(0, 1, 3, 64) == 256


P = ctypes.c_void_p(0x100000)      # never dereferenced: every call below fails validation
MIS = ctypes.c_void_p(0x100008)    # not 16-byte aligned


def fwd(q=P, k=P, v=P, o=P, lse=None, B=1, Hq=2, Hkv=2, Sq=16, Skv=16, D=64, dtype=0, scale=0.125,
        mask=0, mp=None, mod=0, op=None, bm=None):
    return fa.fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, D, dtype, scale, mask,
                     ctypes.byref(mp) if mp else None, mod, ctypes.byref(op) if op else None,
                     ctypes.byref(bm) if bm else None, None)


def test_fwd_rejects_bad_shapes():
    assert fwd(D=96) == fa.FA_ERR_UNSUPPORTED
    assert fwd(dtype=7) == fa.FA_ERR_UNSUPPORTED
    assert fwd(Hq=3, Hkv=2) == fa.FA_ERR_SHAPE
    assert fwd(B=-1) == fa.FA_ERR_SHAPE
    assert fwd(Sq=-5) == fa.FA_ERR_SHAPE
    assert fwd(Hkv=0) == fa.FA_ERR_SHAPE
    assert fwd(Sq=1 << 23) == fa.FA_ERR_SHAPE


def test_fwd_rejects_misaligned_work_queue():
    assert fwd(mp=fa.FaMaskParams(0, None, None, 0x100002)) == fa.FA_ERR_ALIGN


def test_fwd_rejects_misaligned_wg_trace():
    assert fwd(mp=fa.FaMaskParams(0, None, None, None, 0x100004)) == fa.FA_ERR_ALIGN


def test_header_constants_match_binding():
    defines = dict(re.findall(r"^#define\s+(FA_\w+)\s+(.+)$", open(HEADER).read(), flags=re.M))
    assert int(defines["FA_VERSION"]) == binding.FA_VERSION
    assert int(defines["FA_WORK_QUEUE_INTS"]) == fa.FA_WORK_QUEUE_INTS
    assert int(defines["FA_WG_TRACE_WORDS"]) == fa.FA_WG_TRACE_WORDS
    assert eval(defines["FA_NOALLOC_SCRATCH_BYTES"].replace("(size_t)", "")) == fa.FA_NOALLOC_SCRATCH_BYTES


def test_struct_layouts_match_header(tmp_path):
    """sizeof and every field offset of the parameter structs, from a C
    program compiled against the header, equal the ctypes binding's."""
    structs = {"fa_mask_params": fa.FaMaskParams, "fa_mod_params": fa.FaModParams,
               "fa_block_mask": fa.FaBlockMask}
    src = ["#include <stdio.h>", "#include <stddef.h>", f'#include "{HEADER}"', "int main(void) {"]
    for cname, cls in structs.items():
        src.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in cls._fields_:
            src.append(f'printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    src += ["return 0;", "}"]
    (tmp_path / "layout.c").write_text("\n".join(src) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", str(tmp_path / "layout.c"), "-o", str(exe)], check=True)
    got = {}
    for line in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines():
        cname, what, val = line.split()
        got[(cname, what)] = int(val)
    for cname, cls in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(cls), cname
        for fname, _ in cls._fields_:
            assert got[(cname, fname)] == getattr(cls, fname).offset, (cname, fname)


def test_fwd_rejects_bad_pointers():
    assert fwd(q=None) == fa.FA_ERR_NULL
    assert fwd(o=None) == fa.FA_ERR_NULL
    assert fwd(k=None) == fa.FA_ERR_NULL
    assert fwd(q=MIS) == fa.FA_ERR_ALIGN
    assert fwd(v=MIS) == fa.FA_ERR_ALIGN
    assert fwd(lse=ctypes.c_void_p(0x100002)) == fa.FA_ERR_ALIGN


def test_fwd_rejects_bad_params():
    assert fwd(scale=-1.0) == fa.FA_ERR_PARAM
    assert fwd(scale=float("nan")) == fa.FA_ERR_PARAM
    assert fwd(mask=2) == fa.FA_ERR_NULL
    assert fwd(mask=2, mp=fa.FaMaskParams(0, None, None)) == fa.FA_ERR_PARAM
    assert fwd(mask=3, mp=fa.FaMaskParams(0, None, None)) == fa.FA_ERR_NULL
    assert fwd(mask=3, mp=fa.FaMaskParams(0, 0x200000, None), Skv=32) == fa.FA_ERR_SHAPE
    assert fwd(mask=9) == fa.FA_ERR_UNSUPPORTED
    assert fwd(mod=2) == fa.FA_ERR_NULL
    assert fwd(mod=2, op=fa.FaModParams(None, 0.0, 0, 1.0)) == fa.FA_ERR_PARAM
    assert fwd(mod=2, op=fa.FaModParams(None, float("inf"), 0, 1.0)) == fa.FA_ERR_PARAM
    # scale log2(e) and 2 scale log2(e) / softcap must be finite in fp32
    assert fwd(scale=3.0e38) == fa.FA_ERR_PARAM
    assert fwd(mod=2, op=fa.FaModParams(None, 1e-40, 0, 1.0)) == fa.FA_ERR_PARAM
    assert fwd(mod=3, op=fa.FaModParams(None, 0.0, -1, 1.1)) == fa.FA_ERR_PARAM
    assert fwd(mod=3, op=fa.FaModParams(None, 0.0, 5, float("nan"))) == fa.FA_ERR_PARAM
    assert fwd(mod=8) == fa.FA_ERR_UNSUPPORTED


def test_fwd_rejects_bad_block_mask():
    good = dict(block_q=128, block_kv=128, n_q=1, n_kv=1, n_b=1, tile_state=0x300000, kv_count=0x300100,
                kv_index=0x300200, q_count=0x300300, q_index=0x300400)
    assert fwd(bm=fa.FaBlockMask(**{**good, "block_q": 64})) == fa.FA_ERR_UNSUPPORTED
    assert fwd(bm=fa.FaBlockMask(**{**good, "n_q": 2})) == fa.FA_ERR_SHAPE
    assert fwd(bm=fa.FaBlockMask(**{**good, "n_b": 3})) == fa.FA_ERR_SHAPE
    assert fwd(bm=fa.FaBlockMask(**{**good, "kv_index": None})) == fa.FA_ERR_NULL
    assert fwd(bm=fa.FaBlockMask(**{**good, "kv_count": 0x300102})) == fa.FA_ERR_ALIGN


def test_fwd_empty_batch_is_noop():
    assert fwd(B=0, q=None, k=None, v=None, o=None) == fa.FA_OK
    assert fwd(Sq=0, q=None, o=None) == fa.FA_OK


def bwd(dtype=0, lse=P, ws=P, ws_bytes=1 << 20, dq=P, B=1, Hq=2, Hkv=2, S=16, D=64):
    return fa.fa_bwd(P, P, P, P, P, lse, dq, P, P, ws, ws_bytes, B, Hq, Hkv, S, S, D, dtype, 0.125,
                     0, None, 0, None, None, None)


def test_bwd_validation():
    assert bwd(dtype=1) == fa.FA_ERR_UNSUPPORTED
    assert bwd(lse=None) == fa.FA_ERR_NULL
    assert bwd(ws=None) == fa.FA_ERR_WORKSPACE
    assert bwd(ws_bytes=100) == fa.FA_ERR_WORKSPACE
    assert bwd(ws=MIS) == fa.FA_ERR_ALIGN
    assert bwd(dq=MIS) == fa.FA_ERR_ALIGN
    assert bwd(D=80) == fa.FA_ERR_UNSUPPORTED
    assert bwd(B=0) == fa.FA_OK
    args = (P, P, P, P, P, P, P, P, P, P, 1 << 20, 1, 2, 2, 16, 16, 64, 0, 0.125, 0, None, 0, None, None, None)
    assert fa.fa_bwd_phase(0, *args) == fa.FA_ERR_PARAM
    assert fa.fa_bwd_phase(8, *args) == fa.FA_ERR_PARAM
    assert fa.fa_bwd_phase(fa.FA_BWD_DQ, *args[:16], 96, *args[17:]) == fa.FA_ERR_UNSUPPORTED


def test_block_mask_build_validation():
    bm = fa.FaBlockMask(128, 128, 1, 1, 1, 0x300000, 0x300100, 0x300200, 0x300300, 0x300400)
    mp = fa.FaMaskParams(0, 0x200000, None)
    assert fa.fa_block_mask_build(3, ctypes.byref(mp), 2, 100, 100, ctypes.byref(bm), None) == fa.FA_ERR_SHAPE
    assert fa.fa_block_mask_build(1, None, 1, 100, 100, None, None) == fa.FA_ERR_NULL
    assert fa.fa_block_mask_build(1, None, 0, 100, 100, ctypes.byref(bm), None) == fa.FA_ERR_SHAPE
    bad = fa.FaBlockMask(128, 128, 2, 1, 1, 0x300000, 0x300100, 0x300200, 0x300300, 0x300400)
    assert fa.fa_block_mask_build(1, None, 1, 100, 100, ctypes.byref(bad), None) == fa.FA_ERR_SHAPE
    no_q = fa.FaBlockMask(128, 128, 1, 1, 1, 0x300000, 0x300100, 0x300200, None, None)
    assert fa.fa_block_mask_build(1, None, 1, 100, 100, ctypes.byref(no_q), None) == fa.FA_ERR_NULL


def fp8_fwd(q=P, k=P, v=P, qs=P, ks=P, vs=P, o=P, lse=None, B=1, Hq=2, Hkv=2, Sq=16, Skv=16, D=64,
            scale=0.125, mask=0, mp=None):
    L = fa.lib()
    return L.fa_fwd_fp8(q, k, v, qs, ks, vs, o, lse, B, Hq, Hkv, Sq, Skv, D, scale, mask,
                        ctypes.byref(mp) if mp else None, None)


def test_fp8_fwd_validation():
    assert fp8_fwd(D=96) == fa.FA_ERR_UNSUPPORTED
    assert fp8_fwd(mask=3, mp=fa.FaMaskParams(0, 0x200000, None)) == fa.FA_ERR_UNSUPPORTED
    assert fp8_fwd(mask=2) == fa.FA_ERR_NULL
    assert fp8_fwd(mask=2, mp=fa.FaMaskParams(0, None, None)) == fa.FA_ERR_PARAM
    assert fp8_fwd(Hq=3, Hkv=2) == fa.FA_ERR_SHAPE
    assert fp8_fwd(scale=-1.0) == fa.FA_ERR_PARAM
    assert fp8_fwd(q=None) == fa.FA_ERR_NULL
    assert fp8_fwd(ks=None) == fa.FA_ERR_NULL
    assert fp8_fwd(qs=None) == fa.FA_ERR_NULL
    assert fp8_fwd(k=MIS) == fa.FA_ERR_ALIGN
    assert fp8_fwd(lse=ctypes.c_void_p(0x100002)) == fa.FA_ERR_ALIGN
    assert fp8_fwd(B=0, q=None, k=None, v=None, o=None, qs=None, ks=None, vs=None) == fa.FA_OK


def test_fp8_quantize_validation():
    L = fa.lib()
    assert L.fa_fp8_quantize(P, P, P, 2, 16, 96, None, None) == fa.FA_ERR_UNSUPPORTED
    assert L.fa_fp8_quantize(P, P, P, -1, 16, 64, None, None) == fa.FA_ERR_SHAPE
    assert L.fa_fp8_quantize(None, P, P, 2, 16, 64, None, None) == fa.FA_ERR_NULL
    assert L.fa_fp8_quantize(P, P, None, 2, 16, 64, None, None) == fa.FA_ERR_NULL
    assert L.fa_fp8_quantize(MIS, P, P, 2, 16, 64, None, None) == fa.FA_ERR_ALIGN
    assert L.fa_fp8_quantize(P, P, P, 2, 16, 64, ctypes.c_void_p(0x100002), None) == fa.FA_ERR_ALIGN
    assert L.fa_fp8_quantize(None, None, None, 0, 16, 64, None, None) == fa.FA_OK


def test_rel_bias_validation():
    """Relative-bias modifier: table required and aligned; its gradient needs
    an aligned output and enough scratch (fa_bwd_rel_bias_workspace_bytes)."""
    assert fa.fa_bwd_rel_bias_workspace_bytes(2, 16, 8192, 8192) == 2 * 16 * 64 * (8192 + 128) * 4
    assert fa.fa_bwd_rel_bias_workspace_bytes(1, 2, 300, 100) == 1 * 2 * 3 * (100 + 128) * 4
    assert fa.fa_bwd_rel_bias_workspace_bytes(0, 2, 300, 100) == 0
    assert fa.fa_bwd_rel_bias_workspace_bytes(1, 2, 0, 100) == 0
    table = 0x500000
    assert fwd(mod=4) == fa.FA_ERR_NULL
    assert fwd(mod=4, op=fa.FaModParams(None, 0.0, 0, 1.0, None)) == fa.FA_ERR_NULL
    assert fwd(mod=4, op=fa.FaModParams(None, 0.0, 0, 1.0, 0x500002)) == fa.FA_ERR_ALIGN
    need = fa.fa_bwd_rel_bias_workspace_bytes(1, 2, 16, 16)

    def bwd_rel(grad, ws, ws_bytes, phase=7):
        op = fa.FaModParams(None, 0.0, 0, 1.0, table, grad, ws, ws_bytes)
        return fa.fa_bwd_phase(phase, P, P, P, P, P, P, P, P, P, P, 1 << 20, 1, 2, 2, 16, 16, 64, 0, 0.125,
                               0, None, 4, ctypes.byref(op), None, None)

    assert bwd_rel(0x600000, None, 0) == fa.FA_ERR_WORKSPACE
    assert bwd_rel(0x600000, 0x700000, need - 4) == fa.FA_ERR_WORKSPACE
    assert bwd_rel(0x600002, 0x700000, need) == fa.FA_ERR_ALIGN
    assert bwd_rel(0x600000, 0x700008, need) == fa.FA_ERR_ALIGN
    # other validation still comes first
    op = fa.FaModParams(None, 0.0, 0, 1.0, None, 0x600000, 0x700000, need)
    assert fa.fa_bwd(P, P, P, P, P, P, P, P, P, P, 1 << 20, 1, 2, 2, 16, 16, 64, 0, 0.125, 0, None, 4,
                     ctypes.byref(op), None, None) == fa.FA_ERR_NULL


def test_block_mask_bytes_and_layout():
    """One allocation holds every block-mask array, each on a 256-byte boundary."""
    L = fa.lib()
    # S = 1000: 8 blocks; n_b = 2
    parts = [2 * 8 * 8, 2 * 8 * 4, 2 * 8 * 8 * 4, 2 * 8 * 4, 2 * 8 * 8 * 4, 2 * 8 * 4, 2 * 8 * 4]
    rnd = lambda n: (n + 255) // 256 * 256
    assert fa.fa_block_mask_bytes(2, 1000, 1000, True) == sum(rnd(n) for n in parts)
    assert fa.fa_block_mask_bytes(2, 1000, 1000, False) == sum(rnd(n) for n in parts[:5])
    assert L.fa_block_mask_bytes(2, 1000, 1000, 64, 128, 1) == 0
    assert L.fa_block_mask_bytes(0, 1000, 1000, 128, 128, 1) == 0
    assert L.fa_block_mask_bytes(1, -1, 1000, 128, 128, 1) == 0
    base = 0x10000000
    s = fa.FaBlockMask()
    assert L.fa_block_mask_layout(ctypes.c_void_p(base), 2, 1000, 1000, 128, 128, 1, ctypes.byref(s)) == fa.FA_OK
    assert (s.block_q, s.block_kv, s.n_q, s.n_kv, s.n_b) == (128, 128, 8, 8, 2)
    ptrs = [s.tile_state, s.kv_count, s.kv_index, s.q_count, s.q_index, s.q_order, s.kv_order]
    off = 0
    for p, n in zip(ptrs, parts):
        assert p == base + off and p % 256 == 0
        off += rnd(n)
    s2 = fa.FaBlockMask()
    assert L.fa_block_mask_layout(ctypes.c_void_p(base), 1, 300, 200, 128, 128, 0, ctypes.byref(s2)) == fa.FA_OK
    assert s2.q_order is None and s2.kv_order is None and (s2.n_q, s2.n_kv) == (3, 2)
    assert L.fa_block_mask_layout(None, 1, 300, 200, 128, 128, 0, ctypes.byref(s2)) == fa.FA_ERR_NULL
    assert L.fa_block_mask_layout(ctypes.c_void_p(base + 16), 1, 300, 200, 128, 128, 0, ctypes.byref(s2)) == fa.FA_ERR_ALIGN
    assert L.fa_block_mask_layout(ctypes.c_void_p(base), 1, 300, 200, 128, 64, 0, ctypes.byref(s2)) == fa.FA_ERR_SHAPE


def test_binding_rejects_strided_or_mismatched_tensors():
    """The torch conveniences check layouts before calling the library: the C
    ABI reads dense arrays, so a strided view or a mismatched tensor would be
    read as the wrong elements (these checks run before any HIP call)."""
    import pytest
    import torch
    q = torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="contiguous"):
        fa.forward(q.transpose(2, 3).contiguous().transpose(2, 3), k, k)
    with pytest.raises(ValueError, match="shape"):
        fa.forward(q, torch.zeros(1, 2, 16, 128, dtype=torch.bfloat16), k)
    with pytest.raises(ValueError, match="dtype"):
        fa.forward(q, k, k.float())
    with pytest.raises(ValueError, match="doc_ids"):
        fa.forward(q, k, k, mask=fa.MASK_DOCUMENT, doc_ids=torch.zeros(1, 15, dtype=torch.int32))
    with pytest.raises(ValueError, match="lse"):
        fa.backward(q, k, k, q, q, torch.zeros(1, 2, 15))
    with pytest.raises(ValueError, match="dk"):
        fa.backward(q, k, k, q, q, torch.zeros(1, 2, 16), grads=(q, k[:, :1], k))
