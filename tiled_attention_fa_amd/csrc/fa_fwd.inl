// Forward attention kernels for gfx950.
//
// What is computed: O = softmax(mod(scale * Q K^T) masked) V and optionally
// LSE, for every query row, with an online softmax over key tiles: a
// running row max m, a running normaliser l and an output accumulator
// rescaled by 2^(m_old - m_new) whenever the max grows ("FlashAttention 설명"
// page, §4-§5 online softmax; §6 tiling).  The score matrix never leaves
// registers ("FlashAttention-3 (KO)" page, background: fusing the two matrix
// products and the softmax into one kernel).
//
// Work split: one workgroup of 4 waves per (batch, query head, 128-row query
// tile), each wave owning 32 query rows; the key/value tiles are shared
// through LDS ("FlashAttention-2" page, §3-§4: query blocks spread over the
// warps, key/value blocks traversed together).  Per key step of 64 keys:
//   1. K and V tiles (64 x D bf16) stream from HBM into one of two LDS
//      stages with 16-byte loads; the next step's loads are in flight while
//      the current step computes.
//   2. S^T = K Q^T on 32x32x16 bf16 MFMA: each lane owns one query column,
//      so the row max and row sum are in-lane plus one v_permlane32_swap.
//   3. scores -> modifier -> mask (only on partial tiles) -> exp2 domain.
//   4. O^T += V^T P^T: P is repacked to bf16 in registers and used directly
//      as the B operand; V^T comes from LDS through ds_read_b64_tr_b16.
// The fp32 variant uses 32x32x2 fp32 MFMA with the same data flow.
#include <type_traits>

#include "fa_device.h"

namespace miattn {

template <bool F32>
struct FwdCfg {
  static constexpr int BN = F32 ? 32 : 64;  // keys per step
  static constexpr int NT = BN / 32;        // 32-key subtiles per step
};

template <int D, bool F32>
struct FwdSmem {
  static constexpr int ROW = F32 ? (D + 1) * 4 : D * 2;  // bytes per LDS row
  static constexpr int TILE = FwdCfg<F32>::BN * ROW;     // one K or V tile
  static constexpr int STAGES = F32 ? 1 : 2;
  static constexpr int BYTES = STAGES * 2 * TILE;
};

template <int D, bool F32, int MASK, int MOD>
__global__ __launch_bounds__(256) void fwd_kernel(FwdArgs a) {
  using Cfg = FwdCfg<F32>;
  using Sm = FwdSmem<D, F32>;
  constexpr int BN = Cfg::BN, NT = Cfg::NT;
  constexpr int ROW = Sm::ROW, TILE = Sm::TILE;
  constexpr int DT = D / 32;                 // 32-row d tiles of O^T
  constexpr int KC = F32 ? D / 2 : D / 16;   // MFMA k-chunks of the S product
  constexpr int NCH = F32 ? D / 4 : D / 8;   // 16-byte chunks per global row
  constexpr int LOADS = BN * NCH / 256;      // 16-byte chunks per thread per tensor
  static_assert(LOADS * 256 == BN * NCH, "tile load must divide evenly");

  __shared__ __attribute__((aligned(16))) char smem[Sm::BYTES];
  __shared__ int sdoc[Sm::STAGES][BN];

  int b, hq, qt;
  decode_work(blockIdx.x, a.B, a.Hq, a.Hkv, a.n_qt, MASK == MASK_CAUSAL || MASK == MASK_DOCUMENT, b,
              hq, qt);
  const int hk = hq / a.G;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int Sq = a.Sq, Skv = a.Skv;
  const int q0 = qt * kTileQ;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + l32;
  const bool row_ok = qi < Sq;
  const int window = a.mask.window;

  typedef typename std::conditional<F32, float, uint16_t>::type elem_t;
  const elem_t* Q = (const elem_t*)a.q + (size_t)(b * a.Hq + hq) * Sq * D;
  const elem_t* K = (const elem_t*)a.k + (size_t)(b * a.Hkv + hk) * Skv * D;
  const elem_t* V = (const elem_t*)a.v + (size_t)(b * a.Hkv + hk) * Skv * D;
  const int32_t* doc = nullptr;
  int doc_i = 0;
  if constexpr (MASK == MASK_DOCUMENT) {
    doc = a.mask.doc_ids + (size_t)b * Skv;
    doc_i = row_ok ? doc[qi] : -1;
  }
  const float slope = head_slope<MOD>(a.mod, hq, a.Hq);

  // ---- query fragments (B operand of S^T = K Q^T), resident for the whole loop
  u32x4 qf[F32 ? 1 : KC];
  float qs[F32 ? KC : 1];
  if constexpr (F32) {
    const float* src = (const float*)Q + (size_t)(row_ok ? qi : 0) * D;
#pragma unroll
    for (int c = 0; c < KC; ++c) qs[c] = row_ok ? src[2 * c + hh] : 0.0f;
  } else {
    const u32x4* src = (const u32x4*)(Q + (size_t)(row_ok ? qi : 0) * D);
#pragma unroll
    for (int c = 0; c < KC; ++c) qf[c] = row_ok ? src[2 * c + hh] : u32x4{0, 0, 0, 0};
  }

  // ---- key steps: analytic range, or the block mask's list of non-empty blocks
  constexpr int STEPS_PER_BLOCK = kMaskBlock / BN;
  const bool use_bm = a.bm.tile_state != nullptr;
  int step_lo = 0, n_steps = 0;
  const int32_t* bm_list = nullptr;
  const uint8_t* bm_state = nullptr;
  if (use_bm) {
    const int bb = a.bm.n_b == 1 ? 0 : b;
    const int row = bb * a.bm.n_q + qt;
    n_steps = a.bm.kv_count[row] * STEPS_PER_BLOCK;
    bm_list = a.bm.kv_index + (size_t)row * a.bm.n_kv;
    bm_state = a.bm.tile_state + (size_t)row * a.bm.n_kv;
  } else {
    int lo, hi;
    key_range<MASK>(q0, min(q0 + kTileQ, Sq), Skv, window, lo, hi);
    if (hi > lo) {
      step_lo = lo / BN;
      n_steps = (hi + BN - 1) / BN - step_lo;
    }
  }
  auto step_k0 = [&](int s) -> int {
    if (use_bm) return bm_list[s / STEPS_PER_BLOCK] * kMaskBlock + (s % STEPS_PER_BLOCK) * BN;
    return (step_lo + s) * BN;
  };

  // ---- global -> register staging of one K/V tile
  u32x4 kr[LOADS], vr[LOADS];
  int dr = -1;
  auto gload = [&](int k0) {
#pragma unroll
    for (int p = 0; p < LOADS; ++p) {
      const int id = tid + 256 * p, r = id / NCH, c = id % NCH, j = k0 + r;
      if (j < Skv) {
        kr[p] = *(const u32x4*)((const char*)K + ((size_t)j * D) * sizeof(elem_t) + c * 16);
        vr[p] = *(const u32x4*)((const char*)V + ((size_t)j * D) * sizeof(elem_t) + c * 16);
      } else {
        kr[p] = u32x4{0, 0, 0, 0};
        vr[p] = u32x4{0, 0, 0, 0};
      }
    }
    if constexpr (MASK == MASK_DOCUMENT) {
      if (tid < BN) dr = (k0 + tid < Skv) ? doc[k0 + tid] : -2;
    }
  };
  auto lstore = [&](int stage) {
    char* ks = smem + stage * 2 * TILE;
    char* vs = ks + TILE;
#pragma unroll
    for (int p = 0; p < LOADS; ++p) {
      const int id = tid + 256 * p, r = id / NCH, c = id % NCH;
      if constexpr (F32) {
        float* kd = (float*)(ks + r * ROW) + 4 * c;
        float* vd = (float*)(vs + r * ROW) + 4 * c;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kd[e] = __uint_as_float(kr[p][e]);
          vd[e] = __uint_as_float(vr[p][e]);
        }
      } else {
        *(u32x4*)(ks + r * ROW + swz<D>(r, c) * 16) = kr[p];
        *(u32x4*)(vs + r * ROW + swz<D>(r, c) * 16) = vr[p];
      }
    }
    if constexpr (MASK == MASK_DOCUMENT) {
      if (tid < BN) sdoc[stage][tid] = dr;
    }
  };

  float m = kNegInf, l = 0.0f;  // m: running max in log2 units; l: this lane's partial sum
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};

  int visited = 0;
  if (n_steps > 0) {
    gload(step_k0(0));
    lstore(0);
  }
  __syncthreads();

  for (int s = 0; s < n_steps; ++s) {
    const int cur = F32 ? 0 : (s & 1);
    const int k0 = step_k0(s);
    const bool have_next = s + 1 < n_steps;
    if (!F32 && have_next) gload(step_k0(s + 1));
    if (k0 < Skv) ++visited;

    int cls;
    if (use_bm) {
      cls = (k0 >= Skv) ? TILE_EMPTY
                        : (bm_state[bm_list[s / STEPS_PER_BLOCK]] == TILE_FULL ? TILE_FULL : TILE_PARTIAL);
    } else {
      cls = block_class<MASK>(qw0, 32, k0, BN, Skv, window);
    }
    if (qw0 >= Sq) cls = TILE_EMPTY;

    if (cls != TILE_EMPTY) {
      const char* ks = smem + cur * 2 * TILE;
      const char* vs = ks + TILE;
      // ---- S^T = K Q^T  (lane: query column qi; register r: key 8(r/4) + 4hh + r%4)
      f32x16 st[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        st[t] = f32x16{};
        const int r = 32 * t + l32;
        const char* krow = ks + r * ROW;
        if constexpr (F32) {
#pragma unroll
          for (int c = 0; c < KC; ++c) st[t] = mfma_f32(((const float*)krow)[2 * c + hh], qs[c], st[t]);
        } else {
#pragma unroll
          for (int c = 0; c < KC; ++c)
            st[t] = mfma_bf16(*(const u32x4*)(krow + swz<D>(r, 2 * c + hh) * 16), qf[c], st[t]);
        }
      }
      // ---- scores to log2 units, modifier, mask; block max
      float mb = kNegInf;
      const bool plain = (MOD == MOD_NONE) && cls == TILE_FULL;
      if (plain) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) mb = fmaxf(mb, st[t][r]);
        mb = mb * a.scale_log2;
      } else {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int jr = 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
            const int j = k0 + jr;
            float x;
            if constexpr (MOD == MOD_NONE) {
              x = st[t][r] * a.scale_log2;
            } else {
              x = apply_mod<MOD>(st[t][r] * a.scale, qi, j, slope, a.mod) * kLog2e;
            }
            if (cls == TILE_PARTIAL) {
              int dj = 0;
              if constexpr (MASK == MASK_DOCUMENT) dj = sdoc[cur][jr];
              const bool ok = j < Skv && mask_ok<MASK>(qi, j, window, doc_i, dj);
              x = ok ? x : kNegInf;
            }
            st[t][r] = x;
            mb = fmaxf(mb, x);
          }
      }
      mb = half_swap_max(mb);
      const float m_new = fmaxf(m, mb);
      const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
      const float alpha = fast_exp2(m - m_use);
      // ---- probabilities, row sum
      float ps = 0.0f;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = plain ? fast_exp2(__builtin_fmaf(st[t][r], a.scale_log2, -m_use))
                                : fast_exp2(st[t][r] - m_use);
          st[t][r] = p;
          ps += p;
        }
      l = l * alpha + ps;
      m = m_new;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
      }
      // ---- O^T += V^T P^T
      if constexpr (F32) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int jr = 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
              const float vv = ((const float*)(vs + jr * ROW))[32 * dt + l32];
              acc[dt] = mfma_f32(vv, st[t][r], acc[dt]);
            }
      } else {
        u32x4 pb[NT][2];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int cc = 0; cc < 2; ++cc)
            pb[t][cc] = u32x4{pack_bf16(st[t][8 * cc + 0], st[t][8 * cc + 1]),
                              pack_bf16(st[t][8 * cc + 2], st[t][8 * cc + 3]),
                              pack_bf16(st[t][8 * cc + 4], st[t][8 * cc + 5]),
                              pack_bf16(st[t][8 * cc + 6], st[t][8 * cc + 7])};
        const int gi = lane & 15, g = (lane >> 4) & 1;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int ch = 4 * dt + 2 * g + ((gi & 3) >> 1);
          const int half = (gi & 1) * 8;
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
              const int r0 = 32 * t + 16 * cc + 4 * hh + (gi >> 2), r1 = r0 + 8;
              const u32x2 lo = lds_read_tr16(vs + r0 * ROW + swz<D>(r0, ch) * 16 + half);
              const u32x2 hi = lds_read_tr16(vs + r1 * ROW + swz<D>(r1, ch) * 16 + half);
              acc[dt] = mfma_bf16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb[t][cc], acc[dt]);
            }
        }
      }
    }

    if (F32) {
      __syncthreads();
      if (have_next) {
        gload(step_k0(s + 1));
        lstore(0);
      }
      __syncthreads();
    } else {
      if (have_next) lstore(cur ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: O = acc / l, LSE = ln 2 (m + log2 l)
  const float lt = half_swap_sum(l);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (row_ok) {
    elem_t* Orow = (elem_t*)a.o + ((size_t)(b * a.Hq + hq) * Sq + qi) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = 32 * dt + 8 * rq + 4 * hh;
        const float o0 = acc[dt][4 * rq + 0] * inv, o1 = acc[dt][4 * rq + 1] * inv;
        const float o2 = acc[dt][4 * rq + 2] * inv, o3 = acc[dt][4 * rq + 3] * inv;
        if constexpr (F32) {
          *(f32x4*)((float*)Orow + d0) = f32x4{o0, o1, o2, o3};
        } else {
          *(u32x2*)((uint16_t*)Orow + d0) = u32x2{pack_bf16(o0, o1), pack_bf16(o2, o3)};
        }
      }
    if (a.lse != nullptr && hh == 0)
      a.lse[(size_t)(b * a.Hq + hq) * Sq + qi] = lt > 0.0f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : kNegInf;
  }
  if (a.visited != nullptr && tid == 0) atomicAdd(&a.visited[(size_t)(b * a.Hq + hq) * a.n_qt + qt], visited);
}

template <int D, bool F32, int MASK>
static hipError_t launch_mod(const FwdArgs& a, int mod, hipStream_t st) {
  const dim3 grid((unsigned)(a.B * a.Hq * a.n_qt)), block(256);
  switch (mod) {
    case MOD_NONE: hipLaunchKernelGGL((fwd_kernel<D, F32, MASK, MOD_NONE>), grid, block, 0, st, a); break;
    case MOD_ALIBI: hipLaunchKernelGGL((fwd_kernel<D, F32, MASK, MOD_ALIBI>), grid, block, 0, st, a); break;
    case MOD_SOFTCAP: hipLaunchKernelGGL((fwd_kernel<D, F32, MASK, MOD_SOFTCAP>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((fwd_kernel<D, F32, MASK, MOD_BOOST>), grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

template <int D, bool F32>
hipError_t launch_fwd_dt(const FwdArgs& a, int mask, int mod, hipStream_t st) {
  switch (mask) {
    case MASK_NONE: return launch_mod<D, F32, MASK_NONE>(a, mod, st);
    case MASK_CAUSAL: return launch_mod<D, F32, MASK_CAUSAL>(a, mod, st);
    case MASK_WINDOW: return launch_mod<D, F32, MASK_WINDOW>(a, mod, st);
    default: return launch_mod<D, F32, MASK_DOCUMENT>(a, mod, st);
  }
}

}  // namespace miattn
