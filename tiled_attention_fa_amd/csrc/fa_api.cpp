// C ABI of libmiattn: argument validation (before any HIP call) and
// dispatch to the template instantiations.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "../../include/libmiattn.h"
#include "fa_args.h"
#include "fa_launch.h"

using namespace miattn;

namespace {

constexpr long long kMaxSeq = 1LL << 22;    // 4M tokens per sequence
constexpr long long kMaxGrid = 0x7fffffffLL;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
long long cdiv(long long a, long long b) { return (a + b - 1) / b; }

int check_shapes(int B, int Hq, int Hkv, int Sq, int Skv, int D) {
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  if (B < 0 || Sq < 0 || Skv < 0 || Hq < 1 || Hkv < 1) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (Sq > kMaxSeq || Skv > kMaxSeq || Hq > 65536) return FA_ERR_SHAPE;
  const long long heads = (long long)B * Hq;
  if (heads * cdiv(Sq, kTileQ) > kMaxGrid || (long long)B * Hkv * cdiv(Skv, kTileQ) > kMaxGrid) return FA_ERR_SHAPE;
  return FA_OK;
}

// scale * log2(e), the multiplier from raw scores to log2 units.  A zero
// scale maps to the smallest normal-range positive value used here, 1e-30:
// the kernels may then keep masked raw scores at -inf (-inf * 0 would be NaN),
// and every admissible probability still rounds to exactly 1 (|s| * 1e-30 is
// far below fp32 resolution), as with a zero scale.
float log2_multiplier(float scale) {
  const float c = (float)((double)scale * 1.4426950408889634);
  return c > 0.0f ? c : 1e-30f;
}

// Checks shared by the forward and backward passes; fills the mask and
// modifier argument blocks.
int check_variant(int B, int Hq, int Sq, int Skv, float scale, int mask_kind, const fa_mask_params* mp,
                  int mod_kind, const fa_mod_params* op, MaskArgs& mask, ModArgs& mod) {
  // The kernels multiply raw scores by scale log2(e), which must stay finite.
  if (!std::isfinite(scale) || scale < 0.0f || !std::isfinite(log2_multiplier(scale))) return FA_ERR_PARAM;
  mask = MaskArgs{0, nullptr};
  mod = ModArgs{nullptr, 1.0f, 0, 1.0f, nullptr, nullptr, nullptr, 0.0f, -1.0f};
  switch (mask_kind) {
    case FA_MASK_NONE:
    case FA_MASK_CAUSAL: break;
    case FA_MASK_SLIDING_WINDOW:
      if (!mp) return FA_ERR_NULL;
      if (mp->window < 1) return FA_ERR_PARAM;
      // Every admissible pair has i - j < max(Sq, Skv), so a larger window
      // admits the same pairs; the clamp keeps the kernels' range arithmetic
      // (first key + tile + window) far from int overflow.
      mask.window = (int)std::min<long long>(mp->window, std::max<long long>(std::max(Sq, Skv), 1));
      break;
    case FA_MASK_DOCUMENT:
      if (!mp || !mp->doc_ids) return FA_ERR_NULL;
      if (!aligned(mp->doc_ids, 4)) return FA_ERR_ALIGN;
      if (Sq != Skv) return FA_ERR_SHAPE;
      mask.doc_ids = mp->doc_ids;
      break;
    default: return FA_ERR_UNSUPPORTED;
  }
  switch (mod_kind) {
    case FA_MOD_NONE: break;
    case FA_MOD_ALIBI:
      if (op && op->alibi_slopes) {
        if (!aligned(op->alibi_slopes, 4)) return FA_ERR_ALIGN;
        mod.slopes = op->alibi_slopes;
      }
      break;
    case FA_MOD_SOFTCAP:
      if (!op) return FA_ERR_NULL;
      if (!std::isfinite(op->softcap) || !(op->softcap > 0.0f)) return FA_ERR_PARAM;
      mod.softcap = op->softcap;
      mod.softcap_k = (float)(2.0 * (double)scale * 1.4426950408889634 / (double)op->softcap);
      mod.softcap_m = (float)(-2.0 * (double)op->softcap * 1.4426950408889634);
      if (!std::isfinite(mod.softcap_k) || !std::isfinite(mod.softcap_m)) return FA_ERR_PARAM;
      break;
    case FA_MOD_LOCAL_BOOST:
      if (!op) return FA_ERR_NULL;
      if (op->boost_radius < 0 || !std::isfinite(op->boost_factor)) return FA_ERR_PARAM;
      // Every pair has |i - j| < max(Sq, Skv), so a larger radius selects the
      // same pairs; the clamp keeps the kernels' band arithmetic (2 R and
      // first-row + R) far from int overflow.  R = 0 selects no pair.
      mod.boost_radius = (int)std::min<long long>(op->boost_radius, std::max<long long>(std::max(Sq, Skv), 1));
      mod.boost_factor = op->boost_factor;
      break;
    case FA_MOD_REL_BIAS:
      if (!op || !op->rel_bias) return FA_ERR_NULL;
      if (!aligned(op->rel_bias, 4)) return FA_ERR_ALIGN;
      mod.rel_bias = op->rel_bias;
      break;
    default: return FA_ERR_UNSUPPORTED;
  }
  (void)B;
  (void)Hq;
  return FA_OK;
}

// The modifier the kernels run: a local boost of radius 0 boosts no pair,
// which is the unmodified score (and gradient), so it takes that path.
int kernel_mod(int mod_kind, const ModArgs& mod) {
  return (mod_kind == FA_MOD_LOCAL_BOOST && mod.boost_radius == 0) ? FA_MOD_NONE : mod_kind;
}

int check_block_mask(const fa_block_mask* bm, int mask_kind, int B, int Sq, int Skv, bool need_q_lists,
                     BlockMaskArgs& out) {
  out = BlockMaskArgs{nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0, 0, nullptr, nullptr};
  if (!bm) return FA_OK;
  if (bm->block_q != kMaskBlock || bm->block_kv != kMaskBlock) return FA_ERR_UNSUPPORTED;
  if (bm->n_q != cdiv(Sq, kMaskBlock) || bm->n_kv != cdiv(Skv, kMaskBlock)) return FA_ERR_SHAPE;
  if (!(bm->n_b == 1 || bm->n_b == B)) return FA_ERR_SHAPE;
  if (mask_kind == FA_MASK_DOCUMENT && bm->n_b != B) return FA_ERR_SHAPE;
  if (!bm->tile_state || !bm->kv_count || !bm->kv_index) return FA_ERR_NULL;
  if (need_q_lists && (!bm->q_count || !bm->q_index)) return FA_ERR_NULL;
  if (!aligned(bm->kv_count, 4) || !aligned(bm->kv_index, 4)) return FA_ERR_ALIGN;
  if (need_q_lists && (!aligned(bm->q_count, 4) || !aligned(bm->q_index, 4))) return FA_ERR_ALIGN;
  if (!aligned(bm->q_order, 4) || !aligned(bm->kv_order, 4)) return FA_ERR_ALIGN;
  out = BlockMaskArgs{bm->tile_state, bm->kv_count, bm->kv_index, bm->q_count, bm->q_index,
                      bm->n_b, bm->n_q, bm->n_kv, bm->q_order, bm->kv_order};
  return FA_OK;
}

int check_tensor(const void* p, bool nonempty) {
  if (!nonempty) return FA_OK;
  if (!p) return FA_ERR_NULL;
  if (!aligned(p, 16)) return FA_ERR_ALIGN;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_version(void) { return FA_VERSION; }

const char* fa_status_str(int s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "sizes are negative, inconsistent or too large";
    case FA_ERR_UNSUPPORTED: return "head dim, dtype or combination not supported";
    case FA_ERR_ALIGN: return "a device pointer is misaligned";
    case FA_ERR_PARAM: return "a mask or modifier parameter is out of range";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_SCRATCH: return "problem needs more than fa_bwd_noalloc's fixed device scratch";
    default: return "unknown status";
  }
}

int fa_fwd_kv_step(int D, int dtype) {
  if ((D != 64 && D != 128) || (dtype != FA_BF16 && dtype != FA_F32)) return FA_ERR_UNSUPPORTED;
  return fwd_kv_step(dtype == FA_F32);
}

int fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv, int Sq,
           int Skv, int D, int dtype, float scale, int mask_kind, const fa_mask_params* mask_params,
           int score_mod_kind, const fa_mod_params* mod_params, const fa_block_mask* block_mask, void* stream) {
  if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  int rc = check_shapes(B, Hq, Hkv, Sq, Skv, D);
  if (rc) return rc;
  FwdArgs a{};
  rc = check_variant(B, Hq, Sq, Skv, scale, mask_kind, mask_params, score_mod_kind, mod_params, a.mask, a.mod);
  if (rc) return rc;
  rc = check_block_mask(block_mask, mask_kind, B, Sq, Skv, false, a.bm);
  if (rc) return rc;
  const bool has_q = (long long)B * Sq > 0, has_kv = (long long)B * Skv > 0;
  if ((rc = check_tensor(q, has_q)) || (rc = check_tensor(out, has_q)) || (rc = check_tensor(k, has_kv)) ||
      (rc = check_tensor(v, has_kv)))
    return rc;
  if (lse && !aligned(lse, 4)) return FA_ERR_ALIGN;
  int32_t* visited = mask_params ? mask_params->visited : nullptr;
  if (visited && !aligned(visited, 4)) return FA_ERR_ALIGN;
  int32_t* queue = mask_params ? mask_params->work_queue : nullptr;
  if (queue && !aligned(queue, 4)) return FA_ERR_ALIGN;
  int64_t* trace = mask_params ? mask_params->wg_trace : nullptr;
  if (trace && !aligned(trace, 8)) return FA_ERR_ALIGN;
  if (!has_q) return FA_OK;
  if (queue && device_cu_count(&a.n_cu) != hipSuccess) return FA_ERR_LAUNCH;
  a.queue = queue;

  a.q = q;
  a.k = k;
  a.v = v;
  a.o = out;
  a.lse = lse;
  a.visited = visited;
  a.trace = trace;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.Sq = Sq;
  a.Skv = Skv;
  a.n_qt = (int)cdiv(Sq, kTileQ);
  a.scale = scale;
  a.scale_log2 = log2_multiplier(scale);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int mod = kernel_mod(score_mod_kind, a.mod);
  hipError_t e;
  if (dtype == FA_BF16)
    e = D == 128 ? launch_fwd_dt<128, false>(a, mask_kind, mod, st) : launch_fwd_dt<64, false>(a, mask_kind, mod, st);
  else
    e = D == 128 ? launch_fwd_dt<128, true>(a, mask_kind, mod, st) : launch_fwd_dt<64, true>(a, mask_kind, mod, st);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// Workspace: two [B][Hq][Sq] float arrays (row sums of dO * O, and LSE in
// log2 units), each starting on a 256-byte boundary.
static size_t ws_half(int B, int Hq, int Sq) {
  const size_t n = (size_t)B * Hq * Sq * sizeof(float);
  return (n + 255) & ~(size_t)255;
}

int fa_fp8_quantize(const void* x, void* x8, uint8_t* scales, int rows, int S, int D, const float* signs,
                    void* stream) {
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  if (rows < 0 || S < 0 || S > kMaxSeq || rows > 65535) return FA_ERR_SHAPE;
  const bool any = (long long)rows * S > 0;
  int rc;
  if ((rc = check_tensor(x, any)) || (rc = check_tensor(x8, any))) return rc;
  if (any && !scales) return FA_ERR_NULL;
  if (signs && !aligned(signs, 4)) return FA_ERR_ALIGN;
  if (!any) return FA_OK;
  const hipError_t e = launch_fp8_quantize(x, x8, scales, rows, S, D, signs, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd_fp8(const void* q8, const void* k8, const void* v8, const uint8_t* q_scale, const uint8_t* k_scale,
               const uint8_t* v_scale, void* out, float* lse, int B, int Hq, int Hkv, int Sq, int Skv, int D,
               float scale, int mask_kind, const fa_mask_params* mask_params, void* stream) {
  int rc = check_shapes(B, Hq, Hkv, Sq, Skv, D);
  if (rc) return rc;
  if (mask_kind == FA_MASK_DOCUMENT) return FA_ERR_UNSUPPORTED;
  MaskArgs mask;
  ModArgs mod;
  rc = check_variant(B, Hq, Sq, Skv, scale, mask_kind, mask_params, FA_MOD_NONE, nullptr, mask, mod);
  if (rc) return rc;
  const bool has_q = (long long)B * Sq > 0, has_kv = (long long)B * Skv > 0;
  if ((rc = check_tensor(q8, has_q)) || (rc = check_tensor(out, has_q)) || (rc = check_tensor(k8, has_kv)) ||
      (rc = check_tensor(v8, has_kv)))
    return rc;
  if ((has_q && !q_scale) || (has_kv && (!k_scale || !v_scale))) return FA_ERR_NULL;
  if (lse && !aligned(lse, 4)) return FA_ERR_ALIGN;
  if (!has_q) return FA_OK;
  Fp8FwdArgs a{};
  a.q8 = (const uint8_t*)q8;
  a.k8 = (const uint8_t*)k8;
  a.v8 = (const uint8_t*)v8;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.o = out;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.Sq = Sq;
  a.Skv = Skv;
  a.D = D;
  a.n_qt = (int)cdiv(Sq, kTileQ);
  a.window = mask.window;
  a.scale_log2 = log2_multiplier(scale);
  const hipError_t e = launch_fp8_fwd(a, mask_kind, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int Sq, int D) {
  (void)D;
  if (B <= 0 || Hq <= 0 || Sq <= 0) return 256;
  return 2 * ws_half(B, Hq, Sq);
}

size_t fa_bwd_ds_workspace_bytes(int B, int Hq, int Sq, int Skv, int D, int mask_kind) {
  if (B <= 0 || Hq <= 0 || Sq <= 0 || Skv <= 0 || (D != 64 && D != 128)) return 0;
  if (Sq > kMaxSeq || Skv > kMaxSeq) return 0;
  const int n_qs = (int)cdiv(Sq, 32), n_kt = (int)cdiv(Skv, kTileQ);
  long blocks;
  if (mask_kind == FA_MASK_NONE)
    blocks = ds_block<MASK_NONE>(n_kt, 0, n_qs);
  else if (mask_kind == FA_MASK_CAUSAL)
    blocks = ds_block<MASK_CAUSAL>(n_kt, 4 * n_kt, n_qs);
  else
    return 0;
  return fa_bwd_workspace_bytes(B, Hq, Sq, D) + (size_t)B * Hq * (size_t)blocks * kDsBlock * sizeof(uint16_t);
}

size_t fa_bwd_rel_bias_workspace_bytes(int B, int Hq, int Sq, int Skv) {
  if (B <= 0 || Hq <= 0 || Sq <= 0 || Skv < 0) return 0;
  return (size_t)B * Hq * (size_t)cdiv(Sq, kTileQ) * ((size_t)Skv + kBiasRowPad) * sizeof(float);
}

}  // extern "C"

// The backward entry points.  workspace == nullptr with use_scratch: the
// workspace is the library's fixed device array (fa_bwd_noalloc), whose
// address is looked up only after every argument has passed validation.
static int bwd_entry(int phase, const void* q, const void* k, const void* v, const void* out, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                     bool use_scratch, int B, int Hq, int Hkv, int Sq, int Skv, int D, int dtype, float scale,
                     int mask_kind, const fa_mask_params* mask_params, int score_mod_kind,
                     const fa_mod_params* mod_params, const fa_block_mask* block_mask, void* stream) {
  if (phase <= 0 || (phase & ~(FA_BWD_DELTA | FA_BWD_DKDV | FA_BWD_DQ)) != 0) return FA_ERR_PARAM;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  int rc = check_shapes(B, Hq, Hkv, Sq, Skv, D);
  if (rc) return rc;
  BwdArgs a{};
  rc = check_variant(B, Hq, Sq, Skv, scale, mask_kind, mask_params, score_mod_kind, mod_params, a.mask, a.mod);
  if (rc) return rc;
  rc = check_block_mask(block_mask, mask_kind, B, Sq, Skv, true, a.bm);
  if (rc) return rc;
  const bool has_q = (long long)B * Sq > 0, has_kv = (long long)B * Skv > 0;
  if ((rc = check_tensor(q, has_q)) || (rc = check_tensor(out, has_q)) || (rc = check_tensor(dout, has_q)) ||
      (rc = check_tensor(dq, has_q)) || (rc = check_tensor(k, has_kv)) || (rc = check_tensor(v, has_kv)) ||
      (rc = check_tensor(dk, has_kv)) || (rc = check_tensor(dv, has_kv)))
    return rc;
  if (has_q) {
    if (!lse) return FA_ERR_NULL;
    if (!aligned(lse, 4)) return FA_ERR_ALIGN;
    if (use_scratch) {
      if (fa_bwd_workspace_bytes(B, Hq, Sq, D) > kScratchBytes) return FA_ERR_SCRATCH;
    } else {
      if (!workspace || ws_bytes < fa_bwd_workspace_bytes(B, Hq, Sq, D)) return FA_ERR_WORKSPACE;
      if (!aligned(workspace, 16)) return FA_ERR_ALIGN;
    }
  }
  // Relative-bias gradient: output table and the per-tile scratch.
  const bool bias_grad = score_mod_kind == FA_MOD_REL_BIAS && mod_params->rel_bias_grad != nullptr &&
                         (phase & FA_BWD_DQ) && (long long)Sq + Skv > 1;
  if (bias_grad) {
    if (!aligned(mod_params->rel_bias_grad, 4)) return FA_ERR_ALIGN;
    if ((long long)Hq * cdiv((long long)Sq + Skv - 1, 256) > kMaxGrid) return FA_ERR_SHAPE;
    const size_t need = fa_bwd_rel_bias_workspace_bytes(B, Hq, Sq, Skv);
    if (need > 0) {
      if (!mod_params->rel_bias_ws || mod_params->rel_bias_ws_bytes < need) return FA_ERR_WORKSPACE;
      if (!aligned(mod_params->rel_bias_ws, 16)) return FA_ERR_ALIGN;
      a.mod.rel_bias_part = mod_params->rel_bias_ws;
    }
    a.mod.rel_bias_grad = mod_params->rel_bias_grad;
  }
  int64_t* trace = mask_params ? mask_params->wg_trace : nullptr;
  if (trace && !aligned(trace, 8)) return FA_ERR_ALIGN;
  if (B == 0 && !bias_grad) return FA_OK;
  if (use_scratch && scratch_address(&workspace) != hipSuccess) return FA_ERR_LAUNCH;

  a.trace = trace;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = out;
  a.dout = dout;
  a.lse = lse;
  a.delta = (float*)workspace;
  a.lse2 = (const float*)((char*)workspace + ws_half(B, Hq, Sq));
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.Sq = Sq;
  a.Skv = Skv;
  a.n_qt = (int)cdiv(Sq, kTileQ);
  a.n_kt = (int)cdiv(Skv, kTileQ);
  a.n_qs = (int)cdiv(Sq, 32);
  a.scale = scale;
  a.scale_log2 = log2_multiplier(scale);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int mod = kernel_mod(score_mod_kind, a.mod);
  // Stored dS: a workspace of fa_bwd_ds_workspace_bytes holds the dS tiles
  // after the row arrays, and the dQ launch reads them instead of
  // recomputing S and dP (no mask or causal, no block mask, no relative bias).
  if (!use_scratch && B > 0 && Sq > 0 && Skv > 0 && !block_mask && mod != FA_MOD_REL_BIAS &&
      (mask_kind == FA_MASK_NONE || mask_kind == FA_MASK_CAUSAL)) {
    const size_t need = fa_bwd_ds_workspace_bytes(B, Hq, Sq, Skv, D, mask_kind);
    if (need > 0 && ws_bytes >= need) {
      a.ds = (uint16_t*)((char*)workspace + 2 * ws_half(B, Hq, Sq));
      a.ds_blocks = mask_kind == FA_MASK_CAUSAL ? ds_block<MASK_CAUSAL>(a.n_kt, 4 * a.n_kt, a.n_qs)
                                                : ds_block<MASK_NONE>(a.n_kt, 0, a.n_qs);
    }
  }
  const hipError_t e = D == 128 ? launch_bwd_d<128>(a, mask_kind, mod, phase, st)
                                : launch_bwd_d<64>(a, mask_kind, mod, phase, st);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" {

int fa_bwd_phase(int phase, const void* q, const void* k, const void* v, const void* out, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes, int B, int Hq,
                 int Hkv, int Sq, int Skv, int D, int dtype, float scale, int mask_kind,
                 const fa_mask_params* mask_params, int score_mod_kind, const fa_mod_params* mod_params,
                 const fa_block_mask* block_mask, void* stream) {
  return bwd_entry(phase, q, k, v, out, dout, lse, dq, dk, dv, workspace, ws_bytes, false, B, Hq, Hkv, Sq, Skv, D,
                   dtype, scale, mask_kind, mask_params, score_mod_kind, mod_params, block_mask, stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
           void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes, int B, int Hq, int Hkv, int Sq, int Skv,
           int D, int dtype, float scale, int mask_kind, const fa_mask_params* mask_params, int score_mod_kind,
           const fa_mod_params* mod_params, const fa_block_mask* block_mask, void* stream) {
  return fa_bwd_phase(FA_BWD_DELTA | FA_BWD_DKDV | FA_BWD_DQ, q, k, v, out, dout, lse, dq, dk, dv, workspace,
                      ws_bytes, B, Hq, Hkv, Sq, Skv, D, dtype, scale, mask_kind, mask_params, score_mod_kind,
                      mod_params, block_mask, stream);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Skv, int D, int dtype,
                   float scale, int mask_kind, const fa_mask_params* mask_params, int score_mod_kind,
                   const fa_mod_params* mod_params, const fa_block_mask* block_mask, void* stream) {
  return bwd_entry(FA_BWD_DELTA | FA_BWD_DKDV | FA_BWD_DQ, q, k, v, out, dout, lse, dq, dk, dv, nullptr, 0, true, B,
                   Hq, Hkv, Sq, Skv, D, dtype, scale, mask_kind, mask_params, score_mod_kind, mod_params, block_mask,
                   stream);
}


// Sizes of the block-mask arrays in fa_block_mask_layout's order; false for
// invalid arguments.
static bool block_mask_parts(int n_b, int Sq, int Skv, int block_q, int block_kv, int with_orders, size_t (&part)[7],
                             int& n_parts) {
  if (block_q != kMaskBlock || block_kv != kMaskBlock) return false;
  if (n_b < 1 || n_b > 65535 || Sq < 0 || Skv < 0 || Sq > kMaxSeq || Skv > kMaxSeq) return false;
  const size_t nb = (size_t)n_b, nq = (size_t)cdiv(Sq, kMaskBlock), nkv = (size_t)cdiv(Skv, kMaskBlock);
  const size_t nq1 = nq > 0 ? nq : 1, nkv1 = nkv > 0 ? nkv : 1;
  part[0] = nb * nq * nkv;                    // tile_state, u8
  part[1] = nb * nq * 4;                      // kv_count
  part[2] = nb * nq * nkv1 * 4;               // kv_index
  part[3] = nb * nkv * 4;                     // q_count
  part[4] = nb * nkv1 * nq1 * 4;              // q_index
  part[5] = with_orders ? nb * nq1 * 4 : 0;   // q_order
  part[6] = with_orders ? nb * nkv1 * 4 : 0;  // kv_order
  n_parts = with_orders ? 7 : 5;
  return true;
}

size_t fa_block_mask_bytes(int n_b, int Sq, int Skv, int block_q, int block_kv, int with_orders) {
  size_t part[7];
  int n;
  if (!block_mask_parts(n_b, Sq, Skv, block_q, block_kv, with_orders, part, n)) return 0;
  size_t total = 0;
  for (int i = 0; i < n; ++i) total += (part[i] + 255) & ~(size_t)255;
  return total > 0 ? total : 256;
}

int fa_block_mask_layout(void* base, int n_b, int Sq, int Skv, int block_q, int block_kv, int with_orders,
                         fa_block_mask* out) {
  if (!base || !out) return FA_ERR_NULL;
  if (!aligned(base, 256)) return FA_ERR_ALIGN;
  size_t part[7];
  int n;
  if (!block_mask_parts(n_b, Sq, Skv, block_q, block_kv, with_orders, part, n)) return FA_ERR_SHAPE;
  void* p[7] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  char* c = static_cast<char*>(base);
  for (int i = 0; i < n; ++i) {
    p[i] = c;
    c += (part[i] + 255) & ~(size_t)255;
  }
  out->block_q = block_q;
  out->block_kv = block_kv;
  out->n_q = (int)cdiv(Sq, kMaskBlock);
  out->n_kv = (int)cdiv(Skv, kMaskBlock);
  out->n_b = n_b;
  out->tile_state = static_cast<uint8_t*>(p[0]);
  out->kv_count = static_cast<int32_t*>(p[1]);
  out->kv_index = static_cast<int32_t*>(p[2]);
  out->q_count = static_cast<int32_t*>(p[3]);
  out->q_index = static_cast<int32_t*>(p[4]);
  out->q_order = static_cast<int32_t*>(p[5]);
  out->kv_order = static_cast<int32_t*>(p[6]);
  return FA_OK;
}

int fa_block_mask_build(int mask_kind, const fa_mask_params* mask_params, int B, int Sq, int Skv,
                        const fa_block_mask* out, void* stream) {
  if (!out) return FA_ERR_NULL;
  if (B < 1 || Sq < 0 || Skv < 0 || Sq > kMaxSeq || Skv > kMaxSeq) return FA_ERR_SHAPE;
  MaskArgs mask;
  ModArgs mod;
  int rc = check_variant(B, 1, Sq, Skv, 1.0f, mask_kind, mask_params, FA_MOD_NONE, nullptr, mask, mod);
  if (rc) return rc;
  BlockMaskArgs m;
  rc = check_block_mask(out, mask_kind, B, Sq, Skv, true, m);
  if (rc) return rc;
  if (m.n_b > 65535) return FA_ERR_SHAPE;
  const hipError_t e = launch_block_mask(mask_kind, mask.window, mask.doc_ids, Sq, Skv, m,
                                         reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"
