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
//   1. K and V tiles (64 x D bf16) stream from HBM straight into one of two
//      LDS stages (buffer loads to LDS, zero-filled past the last key); the
//      next step's loads are in flight while the current step computes.
//   2. S^T = K Q^T on 32x32x16 bf16 MFMA: each lane owns one query column,
//      so the row max and row sum are in-lane plus one v_permlane32_swap.
//   3. scores -> modifier -> mask (only on partial tiles) -> exp2 domain.
//   4. O^T += V^T P^T: P is repacked to bf16 in registers and used directly
//      as the B operand; V^T comes from LDS through ds_read_b64_tr_b16.
// The fp32 variant uses 32x32x2 fp32 MFMA with the same data flow.
#include <type_traits>

#include "fa_device.h"

namespace miattn {

// ---------------------------------------------------------------- score transform
// Turns one wave's raw scores of a key step (st[t][r]: query qi of this lane,
// key k0 + c + 4hh with c = 32t + 8(r/4) + r%4) into values x, in place, and
// a multiplier `mult` such that a pair's probability against a row max m (log2
// units) is exp2(x * mult - m); masked pairs get x * mult = -inf.  Returns the
// lane's max of x * mult (log2 units, before the two half-waves combine).
// Each modifier takes the form with the fewest vector instructions per score:
//   none:    x = the raw score, mult = scale log2(e): the scale folds into the
//            exponent's FMA and masked scores are -inf in raw units;
//   ALiBi:   x = raw scale log2(e) + slope log2(e) (j - i), the bias from one
//            per-4-keys base plus one add, mult = 1;
//   softcap: c tanh(s / c) = c - 2c / (1 + e^(2s/c)) and softmax ignores the
//            constant c, so x = 1 / (1 + 2^(k raw)), k = 2 scale log2(e) / c,
//            mult = -2c log2(e) < 0, masked x = +inf, and the row max is
//            mult * min x (the epilogue adds c back to the LSE);
//   boost:   steps with no pair in the band |i - j| < radius take the
//            unmodified form; band steps x = raw scale log2(e) (factor or 1);
//   relative bias: x = raw scale + T[h][i - j + Skv - 1] (natural units),
//            mult = log2(e).
// partial: 0 = no masking (full tile), 1 = the pair is admissible iff j < Skv
// and j <= qi, 3 = iff also qi - j < window, 2 = admissible iff ok(j, x),
// x = aux(jr) the entry (document id) of the key at in-step offset
// jr = c + 4hh; with GROUP4 aux4(jr0) gives the entries of four consecutive
// keys jr0 .. jr0 + 3 at once (one 16-byte LDS read for four scores; off
// where the registers for them would spill).  bias(c):
// relative-bias entry of in-step key offset c + 4hh.  qw0: first row of the wave.
template <int MOD, int NT, bool GROUP4, typename Ok, typename Aux, typename Aux4, typename Bias>
__device__ __forceinline__ float transform_scores(f32x16 (&st)[NT], int partial, int k0, int qi, int qw0, int hh,
                                                  int Skv, float slope, const FwdArgs& a, Ok ok, Aux aux,
                                                  Aux4 aux4, Bias bias, float& mult) {
  const float c1 = a.scale_log2;
  float mb = kNegInf;
  bool plain = MOD == MOD_NONE;
  if constexpr (MOD == MOD_BOOST) {
    // Steps with no pair in the band |i - j| < R (none at all when R = 0).
    const int R = a.mod.boost_radius;
    plain = R <= 0 || !(k0 + 32 * NT - 1 > qw0 - R && k0 < qw0 + 31 + R);
  }
  // Elementwise mask, one branch per mode for the whole step.
  // Modes 1 and 3 compare the in-step offset c (a constant per register)
  // with per-lane bounds taken once per step, relative to k0 + 4hh.
  auto mask_all = [&](float masked) __attribute__((always_inline)) {
    const int base = k0 + 4 * hh;
    if (partial == 1) {
      const int hi = min(qi, Skv - 1) - base;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 32 * t + 8 * (r >> 2) + (r & 3);
          st[t][r] = c <= hi ? st[t][r] : masked;
        }
    } else if (partial == 3) {
      // lo <= c <= hi as one unsigned compare; lo is clamped to the step's
      // first key (no overflow for any window), and a row without keys
      // here gets an empty range.
      int lo = max(qi - a.mask.window + 1, base) - base;
      int span = min(qi, Skv - 1) - base - lo;
      if (span < 0) {
        lo = 1 << 30;
        span = 0;
      }
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 32 * t + 8 * (r >> 2) + (r & 3);
          st[t][r] = (unsigned)(c - lo) <= (unsigned)span ? st[t][r] : masked;
        }
    } else if (partial == 2) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int jr0 = 32 * t + 8 * q + 4 * hh;
          if constexpr (GROUP4) {
            const i32x4 x = aux4(jr0);
#pragma unroll
            for (int e = 0; e < 4; ++e) st[t][4 * q + e] = ok(k0 + jr0 + e, x[e]) ? st[t][4 * q + e] : masked;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              st[t][4 * q + e] = ok(k0 + jr0 + e, aux(jr0 + e)) ? st[t][4 * q + e] : masked;
          }
        }
    }
  };
  if (plain) {
    mask_all(kNegInf);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mb = fmaxf(mb, st[t][r]);
    mult = c1;
    return mb * c1;
  }
  if constexpr (MOD == MOD_SOFTCAP) {
    const float k = a.mod.softcap_k;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) st[t][r] = fast_rcp(1.0f + fast_exp2(st[t][r] * k));
    mask_all(__builtin_inff());
    float rmin = __builtin_inff();
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) rmin = fminf(rmin, st[t][r]);
    mult = a.mod.softcap_m;
    return rmin * mult;
  } else {
    // ALiBi, boost inside the band, relative bias.
    const float s2 = slope * kLog2e;
    const float s2e[4] = {0.0f, s2, 2.0f * s2, 3.0f * s2};
    const int d0 = k0 + 4 * hh - qi;  // j - i at c = 0
    const float cf = c1 * a.mod.boost_factor;
    const int R = a.mod.boost_radius;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float bq = 0.0f;
        if constexpr (MOD == MOD_ALIBI) bq = s2 * (float)(d0 + 32 * t + 8 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * q + e, c = 32 * t + 8 * q + e;
          float x;
          if constexpr (MOD == MOD_ALIBI) {
            x = __builtin_fmaf(st[t][r], c1, e ? bq + s2e[e] : bq);
          } else if constexpr (MOD == MOD_BOOST) {
            // |d| < R as one unsigned compare: d + R - 1 in [0, 2R - 2].
            // Valid for R >= 1 (R = 0 took the plain form above); the host
            // clamps R to max(Sq, Skv), so 2R - 1 cannot overflow.
            const int d = d0 + c;  // j - i
            x = st[t][r] * ((unsigned)(d + R - 1) < (unsigned)(2 * R - 1) ? cf : c1);
          } else {
            x = __builtin_fmaf(st[t][r], a.scale, bias(c));
          }
          st[t][r] = x;
        }
      }
    mask_all(kNegInf);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mb = fmaxf(mb, st[t][r]);
    if constexpr (MOD == MOD_REL_BIAS) {
      mult = kLog2e;
      return mb * kLog2e;
    }
    mult = 1.0f;
    return mb;
  }
}

template <bool F32>
struct FwdCfg {
  static constexpr int BN = F32 ? 32 : 64;  // keys per step
  static constexpr int NT = BN / 32;        // 32-key subtiles per step
};

template <int D, bool F32>
struct FwdSmem {
  static constexpr int ROW = F32 ? (D + 1) * 4 : D * 2;  // bytes per LDS row
  static constexpr int TILE = FwdCfg<F32>::BN * ROW;     // one K or V tile
};

// One 128-row query tile (b, hq, qt) of the 4-wave forward: the whole
// online-softmax pass over its key steps and the epilogue.  Every wave of the
// workgroup calls it; on return every read of the LDS stages has finished.
// `at_last_step` runs at the start of the tile's last key step, after that
// step's loads are issued (persistent kernels take their next tile there, so
// the queue's latency hides behind the step).
template <int D, bool F32, int MASK, int MOD, bool BM, typename AtLast>
__device__ __forceinline__ void fwd_tile(const FwdArgs& a, int P, uint64_t t0, int b, int hq, int qt,
                                         AtLast at_last_step) {
  using Cfg = FwdCfg<F32>;
  using Sm = FwdSmem<D, F32>;
  constexpr int BN = Cfg::BN, NT = Cfg::NT;
  constexpr int ROW = Sm::ROW, TILE = Sm::TILE;
  constexpr int DT = D / 32;                 // 32-row d tiles of O^T
  constexpr int KC = F32 ? D / 2 : D / 16;   // MFMA k-chunks of the S product
  constexpr int NCH = F32 ? D / 4 : D / 8;   // 16-byte chunks per global row
  constexpr int LOADS = BN * NCH / 256;      // 16-byte chunks per thread per tensor (fp32 path)
  static_assert(LOADS * 256 == BN * NCH, "tile load must divide evenly");

  // Two LDS stages as separate objects: the step reading one stage never
  // waits on the loads in flight into the other.
  __shared__ __attribute__((aligned(16))) char sK0[TILE], sV0[TILE];
  __shared__ __attribute__((aligned(16))) char sK1[F32 ? 16 : TILE], sV1[F32 ? 16 : TILE];
  __shared__ __attribute__((aligned(16))) int sD0[BN], sD1[BN];
  // Relative-bias diagonals of one key step: 128 + BN - 1 entries, in 64-float chunks.
  constexpr bool REL = MOD == MOD_REL_BIAS;
  constexpr int NB = (kTileQ + BN + 62) / 64 * 64;
  __shared__ __attribute__((aligned(16))) float sB0[REL ? NB : 1], sB1[REL && !F32 ? NB : 1];

  const int hk = hq / a.G;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = wave_uniform(tid >> 6);  // uniform: per-wave branches stay scalar
  const int Sq = a.Sq, Skv = a.Skv;
  const int q0 = qt * kTileQ;
  const int qw0 = q0 + wave * 32;
  const int tlen = Sq + Skv - 1;
  const float* T = nullptr;
  if constexpr (REL) T = uniform_ptr(a.mod.rel_bias + (size_t)hq * tlen);
  // First table entry of the bias slice of the key step at k0.
  auto bias_i0 = [&](int k0) { return q0 - k0 - (BN - 1) + (Skv - 1); };
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
  constexpr bool use_bm = BM;
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
  // Block-mask path: list entry (block index) of step s.  Analytic path:
  // the first key of step s.
  auto fetch_blk = [&](int s) -> int {
    if (s >= n_steps) return 0;
    if constexpr (BM) return bm_list[s / STEPS_PER_BLOCK];
    return step_lo + s;
  };
  auto key0 = [&](int s, int blk) -> int {
    if constexpr (BM) return blk * kMaskBlock + (s % STEPS_PER_BLOCK) * BN;
    return blk * BN;
  };

  // ---- tile loads.  bf16: straight from memory into an LDS stage (buffer
  // loads, zero past Skv).  fp32: through registers into the single stage.
  auto issue = [&](int k0, char* ks, char* vs, int* ds, float* bs) {
    if constexpr (!F32) {
      tile_load<D, BN>(rows_rsrc(K, Skv, k0, D * 2), ks, wave, lane);
      tile_load<D, BN>(rows_rsrc(V, Skv, k0, D * 2), vs, wave, lane);
      if constexpr (MASK == MASK_DOCUMENT) {
        if (wave == 0) ints_to_lds(doc, Skv, k0, ds, lane);
      }
      if constexpr (REL) {
        if (wave < NB / 64) bias_chunk_to_lds(T, tlen, bias_i0(k0), bs, wave, lane);
      }
    }
  };
  auto load_f32 = [&](int k0) {
    if constexpr (F32) {
      u32x4 kr[LOADS], vr[LOADS];
      int dr = -1;
#pragma unroll
      for (int p = 0; p < LOADS; ++p) {
        const int id = tid + 256 * p, r = id / NCH, c = id % NCH, j = k0 + r;
        const bool ok = j < Skv;
        kr[p] = ok ? *(const u32x4*)((const float*)K + (size_t)j * D + 4 * c) : u32x4{0, 0, 0, 0};
        vr[p] = ok ? *(const u32x4*)((const float*)V + (size_t)j * D + 4 * c) : u32x4{0, 0, 0, 0};
      }
      if constexpr (MASK == MASK_DOCUMENT) {
        if (tid < BN) dr = (k0 + tid < Skv) ? doc[k0 + tid] : -2;
      }
      float br = 0.0f;
      if constexpr (REL) {
        const int idx = bias_i0(k0) + tid;
        if (tid < NB && idx >= 0 && idx < tlen) br = T[idx];
      }
#pragma unroll
      for (int p = 0; p < LOADS; ++p) {
        const int id = tid + 256 * p, r = id / NCH, c = id % NCH;
        float* kd = (float*)(sK0 + r * ROW) + 4 * c;
        float* vd = (float*)(sV0 + r * ROW) + 4 * c;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kd[e] = __uint_as_float(kr[p][e]);
          vd[e] = __uint_as_float(vr[p][e]);
        }
      }
      if constexpr (MASK == MASK_DOCUMENT) {
        if (tid < BN) sD0[tid] = dr;
      }
      if constexpr (REL) {
        if (tid < NB) sB0[tid] = br;
      }
    }
  };

  float m = kNegInf, l = 0.0f;  // m: running max in log2 units; l: this lane's partial sum
  float lc = 0.0f;              // compensation of l
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  int visited = 0;

  // One key step on the stage (ks, vs, ds); the next step's tiles go to
  // (kn, vn, dn).  The block index of this step and the next, and the block
  // state of this step, are in registers.  Block-mask reads for later steps
  // (list entry two steps ahead, state one step ahead) are issued after the
  // tile loads and only consumed in the next step, after its wait.
  int blk_c = 0, blk_n = 0, st_c = 0, st_n = 0;
  auto step = [&](int s, const char* ks, const char* vs, const int* ds, const float* bs, char* kn, char* vn, int* dn,
                  float* bn) {
    const int k0 = key0(s, blk_c);
    const bool have_next = s + 1 < n_steps;
    if (have_next) issue(key0(s + 1, blk_n), kn, vn, dn, bn);
    const int blk_nn = fetch_blk(s + 2);
    if constexpr (BM) st_n = have_next ? bm_state[blk_n] : 0;
    if (k0 < Skv) ++visited;
    if (!have_next) at_last_step();

    int cls;
    if constexpr (BM) {
      cls = (k0 >= Skv) ? TILE_EMPTY : (st_c == TILE_FULL ? TILE_FULL : TILE_PARTIAL);
      // A partial 128 x 128 tile is refined per wave and step with the
      // analytic bounds of the mask: the wave's 32 x BN block may hold no
      // admissible pair (above the diagonal, or below a window), or, for
      // causal and window masks, only admissible pairs.  Document masks are
      // causal within a document, so the causal bound applies to them too.
      if constexpr (MASK != MASK_NONE) {
        if (cls == TILE_PARTIAL) {
          const int c2 = block_class<MASK == MASK_DOCUMENT ? MASK_CAUSAL : MASK>(qw0, 32, k0, BN, Skv, window);
          if (c2 == TILE_EMPTY) cls = TILE_EMPTY;
          if constexpr (MASK != MASK_DOCUMENT) {
            if (c2 == TILE_FULL) cls = TILE_FULL;
          }
        }
      }
    } else {
      cls = block_class<MASK>(qw0, 32, k0, BN, Skv, window);
    }
    if (qw0 >= Sq) cls = TILE_EMPTY;

    if (cls != TILE_EMPTY) {
      // ---- S^T = K Q^T  (lane: query column qi; register r: key 8(r/4) + 4hh + r%4)
      f32x16 st[NT];
      if constexpr (F32) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          st[t] = f32x16{};
          const char* krow = ks + (32 * t + l32) * ROW;
#pragma unroll
          for (int c = 0; c < KC; ++c) st[t] = mfma_f32(((const float*)krow)[2 * c + hh], qs[c], st[t]);
        }
      } else {
        // The NT accumulation chains alternate; LDS reads run 4 ahead of the MFMAs.
#pragma unroll
        for (int t = 0; t < NT; ++t) st[t] = f32x16{};
#pragma unroll
        for (int c = 0; c < KC; ++c)
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const int r = 32 * t + l32;
            st[t] = mfma_bf16(*(const u32x4*)(ks + r * ROW + swz<D>(r, 2 * c + hh) * 16), qf[c], st[t]);
          }
        constexpr int NM = KC * NT;
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < NM - 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
      // ---- scores to log2 units (relative bias: natural units), modifier, mask; block max
      // bl[CMAX - c] is the bias of key k0 + c + 4hh (c = 32t + 8(r/4) + r%4).
      constexpr int CMAX = 32 * (NT - 1) + 27;
      const float* bl = bs + (32 * wave + l32 + 4 - 4 * hh);
      // Mask mode: a partial step whose keys and rows all carry one document
      // id needs only the causal test (the usual case: a diagonal tile inside
      // a document).  Checked per step from the staged key ids and the rows'.
      int mode = cls == TILE_PARTIAL ? 2 : 0;
      if constexpr (MASK == MASK_DOCUMENT) {
        if (mode == 2) {
          const int ref = wave_uniform(doc_i);
          const bool keys_one = __builtin_amdgcn_ballot_w64(lane >= BN || ds[lane] == ref) == ~0ull;
          const bool rows_one = __builtin_amdgcn_ballot_w64(doc_i == ref) == ~0ull;
          // One document: only the causal test is left, and none at all
          // when every key precedes every row of the wave.
          if (keys_one && rows_one) mode = k0 + BN - 1 <= qw0 && k0 + BN <= Skv && qw0 + 31 < Sq ? 0 : 1;
        }
      } else if constexpr (MASK == MASK_CAUSAL) {
        mode = mode ? 1 : 0;
      } else if constexpr (MASK == MASK_WINDOW) {
        mode = mode ? 3 : 0;
      }
      float mult;
      float mb = transform_scores<MOD, NT, !(MASK == MASK_DOCUMENT && MOD == MOD_BOOST)>(
          st, mode, k0, qi, qw0, hh, Skv, slope, a,
          [&](int j, int dj) { return j < Skv && mask_ok<MASK>(qi, j, window, doc_i, dj); },
          [&](int jr) { return MASK == MASK_DOCUMENT ? ds[jr] : 0; },
          [&](int jr0) { return MASK == MASK_DOCUMENT ? *(const i32x4*)(ds + jr0) : i32x4{0, 0, 0, 0}; },
          [&](int c) { return REL ? bl[CMAX - c] : 0.0f; }, mult);
      mb = half_swap_max(mb);
      const float m_new = fmaxf(m, mb);
      const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
      const float alpha = fast_exp2(m - m_use);
      // ---- probabilities, row sum
      float ps = 0.0f;  // the first term starts the sum (no add of 0)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(__builtin_fmaf(st[t][r], mult, -m_use));
          st[t][r] = p;
          ps = (t == 0 && r == 0) ? p : ps + p;
        }
      row_sum_update(l, lc, alpha, ps);
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
        // Transposing reads run two MFMAs (4 reads) ahead.
        constexpr int NM = DT * NT * 2;
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
        for (int i = 0; i < NM - 2; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
      }
    }

    if constexpr (F32) {
      __syncthreads();
      if (have_next) load_f32(key0(s + 1, blk_n));
      __syncthreads();
    } else {
      wait_loads();
      __syncthreads();
    }
    blk_c = blk_n;
    st_c = st_n;
    blk_n = blk_nn;
  };

  blk_c = fetch_blk(0);
  blk_n = fetch_blk(1);
  if constexpr (BM) st_c = n_steps > 0 ? bm_state[blk_c] : 0;
  if (n_steps > 0) {
    if constexpr (F32) {
      load_f32(key0(0, blk_c));
    } else {
      issue(key0(0, blk_c), sK0, sV0, sD0, sB0);
      wait_loads();
    }
  }
  __syncthreads();
  if constexpr (F32) {
    for (int s = 0; s < n_steps; ++s) step(s, sK0, sV0, sD0, sB0, sK0, sV0, sD0, sB0);
  } else {
    for (int s = 0; s < n_steps; s += 2) {
      step(s, sK0, sV0, sD0, sB0, sK1, sV1, sD1, sB1);
      if (s + 1 < n_steps) step(s + 1, sK1, sV1, sD1, sB1, sK0, sV0, sD0, sB0);
    }
  }

  // ---- epilogue: O = acc / l, LSE = ln 2 (m + log2 l) (+ the constant the
  // softcap form leaves out)
  const float lt = half_swap_sum(l - lc);
  const float lse_shift = MOD == MOD_SOFTCAP ? a.mod.softcap : 0.0f;
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
      a.lse[(size_t)(b * a.Hq + hq) * Sq + qi] = lt > 0.0f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 + lse_shift : kNegInf;
  }
  if (a.visited != nullptr && tid == 0) atomicAdd(&a.visited[(size_t)(b * a.Hq + hq) * a.n_qt + qt], visited);
  trace_end(a.trace, P, t0, wave == 0, kTileQ, n_steps);
}

// Query tile of the static schedule's workgroup P: XCD-pinned (batch, kv
// head) units, heaviest causal tiles first, or the block mask's
// schedule order.
template <int MASK, bool BM>
__device__ __forceinline__ void fwd_tile_of(const FwdArgs& a, int P, int& b, int& hq, int& qt) {
  decode_work(P, a.B, a.Hq, a.Hkv, a.n_qt, (MASK == MASK_CAUSAL || MASK == MASK_DOCUMENT) && !(BM && a.bm.q_order),
              b, hq, qt);
  if constexpr (BM) qt = ordered_tile(a.bm.q_order, a.bm.n_b, b, a.bm.n_q, qt, qt);
}

template <int D, bool F32, int MASK, int MOD, bool BM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_kernel(FwdArgs a) {
  const uint64_t t0 = trace_clock(a.trace);
  int b, hq, qt;
  fwd_tile_of<MASK, BM>(a, blockIdx.x, b, hq, qt);
  fwd_tile<D, F32, MASK, MOD, BM>(a, blockIdx.x, t0, b, hq, qt, [] {});
}

// Persistent, dynamically scheduled form of fwd_kernel (the role of a
// hardware tile scheduler with persistent workgroups on the "PyTorch
// FlexAttention, FlashAttention-4" page, 섹션별 상세, and the persistent
// scheduling of the "FlashInfer SM120" page, §4): about two workgroups per
// compute unit, each taking query tiles from a work queue in caller memory
// until it is empty.  The queue holds one counter per XCD over that XCD's
// share of the static schedule (its (batch, kv-head) units, longest tiles
// first); a workgroup drains its own XCD's counter, keeping K/V in that L2,
// then takes leftovers from the others.  Results are those of fwd_kernel,
// bit for bit: the same per-tile code runs, only the order of tiles differs.
template <int D, bool F32, int MASK, int MOD, bool BM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_persist_kernel(FwdArgs a) {
  __shared__ int sUnit;
  const WorkQueue wq = work_queue_shape(a.B, a.Hq, a.Hkv, a.n_qt);
  const int home = (int)(blockIdx.x % kXcds);
  int P = finish_pull(a.queue, wq, home, -1, &sUnit);
  while (P >= 0) {
    int b, hq, qt;
    fwd_tile_of<MASK, BM>(a, P, b, hq, qt);
    // The next tile's index is taken (thread 0) when this tile's last step
    // starts and read after the tile, when the step's loads have landed.
    int i_next = -1;
    fwd_tile<D, F32, MASK, MOD, BM>(a, -1, 0, b, hq, qt, [&] {
      if (threadIdx.x == 0) i_next = take_home(a.queue, wq, home);
    });
    P = finish_pull(a.queue, wq, home, i_next, &sUnit);
  }
  release_queue(a.queue);
}

// ---------------------------------------------------------------- ping-pong forward
// bf16, analytic masks (none, causal, sliding window), every score modifier.
// Workgroup: 8 waves in two groups of 4 over 256 query rows; group g owns
// rows [q0 + 128 g, q0 + 128 g + 128), 32 per wave, and both groups walk the
// same key tiles, held once in LDS for all 8 waves.  Each SIMD hosts one wave
// of each group and the groups run half a step apart:
//   phase 2j:   group 0: O += V_{j-1}^T P_{j-1} and S_j = K_j Q^T (MFMA)
//               group 1: softmax of S_{j-1} (VALU, exp)
//   phase 2j+1: group 0: softmax of S_j;  group 1: the MFMA work of step j
// separated by workgroup barriers, so the exponentials of one wave overlap
// the matrix products of the other wave on the same SIMD: the warpgroup
// ping-pong of the "FlashAttention-3 (KO)" page (intra-consumer overlap of
// softmax and GEMM), built from the one workgroup barrier of CDNA.  Every
// wave runs the same sequence (MFMA work of step j, barrier, softmax of
// step j, barrier); group 1 passes one extra barrier first and group 0 one
// at the end, which puts the groups half a step apart without a group-
// dependent code path (two such paths double the live registers).
// LDS: two K slots and two V slots.  Group 0 issues K_{j+1} and V_j at the
// start of its phase 2j (into the slots that steps j-1 and j-2 no longer
// use) and waits for them at the end of phase 2j+1.
template <int D, int MASK, int MOD>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_pp_kernel(FwdArgs a) {
  static_assert(MASK != MASK_DOCUMENT, "document masks take fwd_kernel");
  constexpr int BN = 64, NT = 2, ROW = D * 2, TILE = BN * ROW;
  constexpr int DT = D / 32, KC = D / 16;
  constexpr int QT = 2 * kTileQ;  // query rows per workgroup
  constexpr bool REL = MOD == MOD_REL_BIAS;
  __shared__ __attribute__((aligned(16))) char sK0[TILE], sK1[TILE], sV0[TILE], sV1[TILE];
  // Relative-bias diagonals of one key step: QT + BN - 1 entries (5 chunks of 64).
  __shared__ __attribute__((aligned(16))) float sB0[REL ? 320 : 1], sB1[REL ? 320 : 1];

  const uint64_t t0 = trace_clock(a.trace);
  int b, hq, qt;
  decode_work(blockIdx.x, a.B, a.Hq, a.Hkv, (a.Sq + QT - 1) / QT, MASK == MASK_CAUSAL, b, hq, qt);
  const int hk = hq / a.G;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = wave_uniform(tid >> 6), grp = wave >> 2;
  const int Sq = a.Sq, Skv = a.Skv, window = a.mask.window;
  const int q0 = qt * QT, qg0 = q0 + kTileQ * grp, qw0 = qg0 + 32 * (wave & 3), qi = qw0 + l32;
  const bool row_ok = qi < Sq;

  const uint16_t* Q = (const uint16_t*)a.q + (size_t)(b * a.Hq + hq) * Sq * D;
  const uint16_t* K = uniform_ptr((const uint16_t*)a.k + (size_t)(b * a.Hkv + hk) * Skv * D);
  const uint16_t* V = uniform_ptr((const uint16_t*)a.v + (size_t)(b * a.Hkv + hk) * Skv * D);
  const float slope = head_slope<MOD>(a.mod, hq, a.Hq);
  const int tlen = Sq + Skv - 1;
  const float* T = nullptr;
  if constexpr (REL) T = uniform_ptr(a.mod.rel_bias + (size_t)hq * tlen);

  u32x4 qf[KC];
  {
    const u32x4* src = (const u32x4*)(Q + (size_t)(row_ok ? qi : 0) * D);
#pragma unroll
    for (int c = 0; c < KC; ++c) qf[c] = row_ok ? src[2 * c + hh] : u32x4{0, 0, 0, 0};
  }

  // Key steps of the whole workgroup (union of both groups' ranges).
  int step_lo = 0, n_steps = 0;
  {
    int lo, hi;
    key_range<MASK>(q0, min(q0 + QT, Sq), Skv, window, lo, hi);
    if (hi > lo) {
      step_lo = lo / BN;
      n_steps = (hi + BN - 1) / BN - step_lo;
    }
  }
  auto wave_class = [&](int j) __attribute__((always_inline)) -> int {
    if (qw0 >= Sq) return TILE_EMPTY;
    return block_class<MASK>(qw0, 32, (step_lo + j) * BN, BN, Skv, window);
  };
  // Tile loads are issued by the 4 waves of group 0.
  auto issue_k = [&](int j, char* ks) { tile_load<D, BN>(rows_rsrc(K, Skv, (step_lo + j) * BN, ROW), ks, wave & 3, lane); };
  auto issue_v = [&](int j, char* vs) { tile_load<D, BN>(rows_rsrc(V, Skv, (step_lo + j) * BN, ROW), vs, wave & 3, lane); };
  // Bias diagonals of step j (entry e: i - j = q0 - k0 - (BN - 1) + e), by
  // the 4 waves of group 1, which issue no tile loads.
  auto issue_b = [&](int j, float* bs) {
    const int i0 = q0 - (step_lo + j) * BN - (BN - 1) + (Skv - 1);
    bias_chunk_to_lds(T, tlen, i0, bs, wave & 3, lane);
    if ((wave & 3) == 0) bias_chunk_to_lds(T, tlen, i0, bs, 4, lane);
  };

  float m = kNegInf, l = 0.0f;  // running max (log2 units), this lane's partial row sum
  float lc = 0.0f;              // compensation of l
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  f32x16 st[NT];
  u32x4 pb[NT][2];
  int cls_s = TILE_EMPTY;  // class of the step whose scores / probabilities are held
  const int gi = lane & 15, g16 = (lane >> 4) & 1;

  // MFMA work of step j: O^T += V_{j-1}^T P_{j-1}^T, then S_j^T = K_j Q^T.
  auto m_phase = [&](int j, const char* ks, const char* vs) __attribute__((always_inline)) {
    if (cls_s != TILE_EMPTY) {
      const int half = (gi & 1) * 8;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int ch = 4 * dt + 2 * g16 + ((gi & 3) >> 1);
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
      constexpr int NM = DT * NT * 2;
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
      for (int i = 0; i < NM - 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
    }
    cls_s = j < n_steps ? wave_class(j) : TILE_EMPTY;
    if (cls_s != TILE_EMPTY) {
#pragma unroll
      for (int t = 0; t < NT; ++t) st[t] = f32x16{};
#pragma unroll
      for (int c = 0; c < KC; ++c)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int r = 32 * t + l32;
          st[t] = mfma_bf16(*(const u32x4*)(ks + r * ROW + swz<D>(r, 2 * c + hh) * 16), qf[c], st[t]);
        }
      constexpr int NM = KC * NT;
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < NM - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
  };

  // Softmax of step j's scores: running max, rescale of O, P packed to bf16.
  // With the relative bias, scores stay in natural units until the exp.
  auto v_phase = [&](int j, const float* bs) __attribute__((always_inline)) {
    if (j < 0 || j >= n_steps || cls_s == TILE_EMPTY) return;
    const int k0 = (step_lo + j) * BN;
    // bl[59 - c] is the bias of key k0 + c + 4hh (c = 32t + 8(r/4) + r%4).
    const float* bl = bs + (qi - q0 + 4 - 4 * hh);
    float mult;
    float mb = transform_scores<MOD, NT, false>(
        st, cls_s == TILE_PARTIAL ? (MASK == MASK_CAUSAL ? 1 : MASK == MASK_WINDOW ? 3 : 2) : 0, k0, qi, qw0, hh,
        Skv, slope, a,
        [&](int j, int) { return j < Skv && mask_ok<MASK>(qi, j, window, 0, 0); },
        [](int) { return 0; }, [](int) { return i32x4{0, 0, 0, 0}; }, [&](int c) { return REL ? bl[59 - c] : 0.0f; },
        mult);
    mb = half_swap_max(mb);
    const float m_new = fmaxf(m, mb);
    const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = fast_exp2(m - m_use);
    float ps = 0.0f;  // the first term starts the sum (no add of 0)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(st[t][r], mult, -m_use));
        st[t][r] = p;
        ps = (t == 0 && r == 0) ? p : ps + p;
      }
    row_sum_update(l, lc, alpha, ps);
    m = m_new;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
        pb[t][cc] = u32x4{pack_bf16(st[t][8 * cc + 0], st[t][8 * cc + 1]), pack_bf16(st[t][8 * cc + 2], st[t][8 * cc + 3]),
                          pack_bf16(st[t][8 * cc + 4], st[t][8 * cc + 5]), pack_bf16(st[t][8 * cc + 6], st[t][8 * cc + 7])};
  };

  // Step j of this wave.  (kc: K_j, vp: V_{j-1}; kn, vc: where K_{j+1}, V_j
  // go; bc: bias of step j; bn: where group 1 loads the bias of step j + 1.
  // Group 1 is half a step behind, so that slot's last readers, the softmax
  // phases of step j - 1, are done when it starts its step j.)
  auto step = [&](int j, const char* kc, const char* vp, char* kn, char* vc, const float* bc, float* bn)
      __attribute__((always_inline)) {
    if (grp == 0) {
      if (j + 1 < n_steps) issue_k(j + 1, kn);
      if (j < n_steps) issue_v(j, vc);
    } else if constexpr (REL) {
      if (j + 1 < n_steps) issue_b(j + 1, bn);
    }
    m_phase(j, kc, vp);
    phase_barrier();
    v_phase(j, bc);
    wait_loads();
    phase_barrier();
  };

  if (grp == 0 && n_steps > 0) issue_k(0, sK0);
  if constexpr (REL) {
    if (grp == 1 && n_steps > 0) issue_b(0, sB0);
  }
  wait_loads();
  __syncthreads();
  if (grp == 1) phase_barrier();
  for (int j = 0; j <= n_steps; j += 2) {
    step(j, sK0, sV1, sK1, sV0, sB0, sB1);
    if (j + 1 <= n_steps) step(j + 1, sK1, sV0, sK0, sV1, sB1, sB0);
  }
  if (grp == 0) phase_barrier();

  // ---- epilogue: O = acc / l, LSE = ln 2 (m + log2 l) (+ the constant the
  // softcap form leaves out)
  const float lt = half_swap_sum(l - lc);
  const float lse_shift = MOD == MOD_SOFTCAP ? a.mod.softcap : 0.0f;
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (row_ok) {
    uint16_t* Orow = (uint16_t*)a.o + ((size_t)(b * a.Hq + hq) * Sq + qi) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = 32 * dt + 8 * rq + 4 * hh;
        *(u32x2*)(Orow + d0) = u32x2{pack_bf16(acc[dt][4 * rq + 0] * inv, acc[dt][4 * rq + 1] * inv),
                                     pack_bf16(acc[dt][4 * rq + 2] * inv, acc[dt][4 * rq + 3] * inv)};
      }
    if (a.lse != nullptr && hh == 0)
      a.lse[(size_t)(b * a.Hq + hq) * Sq + qi] = lt > 0.0f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 + lse_shift : kNegInf;
  }
  // Debug count per 128-row query tile: key steps holding an admissible pair.
  if (a.visited != nullptr && (tid & 255) == 0 && qg0 < Sq) {
    int vis = 0;
    for (int j = 0; j < n_steps; ++j) {
      const int k0 = (step_lo + j) * BN;
      if (k0 < Skv && block_class<MASK>(qg0, min(kTileQ, Sq - qg0), k0, BN, Skv, window) != TILE_EMPTY) ++vis;
    }
    atomicAdd(&a.visited[(size_t)(b * a.Hq + hq) * a.n_qt + qg0 / kTileQ], vis);
  }
  trace_end(a.trace, blockIdx.x, t0, wave == 0, QT, n_steps);
}

template <int D, int MASK>
static hipError_t launch_pp(const FwdArgs& a, int mod, hipStream_t st) {
  const dim3 grid((unsigned)(a.B * a.Hq * ((a.Sq + 2 * kTileQ - 1) / (2 * kTileQ)))), block(512);
  switch (mod) {
    case MOD_NONE: hipLaunchKernelGGL((fwd_pp_kernel<D, MASK, MOD_NONE>), grid, block, 0, st, a); break;
    case MOD_ALIBI: hipLaunchKernelGGL((fwd_pp_kernel<D, MASK, MOD_ALIBI>), grid, block, 0, st, a); break;
    case MOD_SOFTCAP: hipLaunchKernelGGL((fwd_pp_kernel<D, MASK, MOD_SOFTCAP>), grid, block, 0, st, a); break;
    case MOD_REL_BIAS: hipLaunchKernelGGL((fwd_pp_kernel<D, MASK, MOD_REL_BIAS>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((fwd_pp_kernel<D, MASK, MOD_BOOST>), grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

template <int D, bool F32, int MASK, bool BM, int MOD>
static void launch_one(const FwdArgs& a, hipStream_t st) {
  const int tiles = a.B * a.Hq * a.n_qt;
  if (a.queue != nullptr) {
    // Two workgroups per compute unit, but no more than there are tiles.
    const int grid = min(tiles, 2 * a.n_cu);
    hipLaunchKernelGGL((fwd_persist_kernel<D, F32, MASK, MOD, BM>), dim3((unsigned)grid), dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((fwd_kernel<D, F32, MASK, MOD, BM>), dim3((unsigned)tiles), dim3(256), 0, st, a);
  }
}

template <int D, bool F32, int MASK, bool BM>
static hipError_t launch_mod(const FwdArgs& a, int mod, hipStream_t st) {
  switch (mod) {
    case MOD_NONE: launch_one<D, F32, MASK, BM, MOD_NONE>(a, st); break;
    case MOD_ALIBI: launch_one<D, F32, MASK, BM, MOD_ALIBI>(a, st); break;
    case MOD_SOFTCAP: launch_one<D, F32, MASK, BM, MOD_SOFTCAP>(a, st); break;
    case MOD_REL_BIAS: launch_one<D, F32, MASK, BM, MOD_REL_BIAS>(a, st); break;
    default: launch_one<D, F32, MASK, BM, MOD_BOOST>(a, st); break;
  }
  return hipGetLastError();
}

template <int D, bool F32, int MASK>
static hipError_t launch_bm(const FwdArgs& a, int mod, hipStream_t st) {
  if (a.bm.tile_state != nullptr) return launch_mod<D, F32, MASK, true>(a, mod, st);
  // The ping-pong kernel walks the union of the key ranges of 256 rows; for
  // short windows that union is up to 25% longer than a 128-row tile's
  // range, and the 4-wave kernel is faster (1024-key window: 0.42 vs
  // 0.44 ms at B2 Hq32 S8192).
  // Up to 1024 keys a query tile has at most 16 key steps, and the 4-wave
  // kernel, two workgroups per compute unit, hides each one's prologue and
  // epilogue behind the other's steps: causal B16 H16 S1024 0.123 against
  // 0.134 ms (equal at S = 2048, the ping-pong kernel 3-5 % ahead from 4096).
  if constexpr (!F32 && MASK != MASK_DOCUMENT) {
    if (a.queue == nullptr && a.Skv > 1024 && (MASK != MASK_WINDOW || a.mask.window > 2048))
      return launch_pp<D, MASK>(a, mod, st);
  }
  return launch_mod<D, F32, MASK, false>(a, mod, st);
}

template <int D, bool F32>
hipError_t launch_fwd_dt(const FwdArgs& a, int mask, int mod, hipStream_t st) {
  switch (mask) {
    case MASK_NONE: return launch_bm<D, F32, MASK_NONE>(a, mod, st);
    case MASK_CAUSAL: return launch_bm<D, F32, MASK_CAUSAL>(a, mod, st);
    case MASK_WINDOW: return launch_bm<D, F32, MASK_WINDOW>(a, mod, st);
    default: return launch_bm<D, F32, MASK_DOCUMENT>(a, mod, st);
  }
}

}  // namespace miattn
