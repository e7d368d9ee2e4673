// Backward attention kernels for gfx950 (included by fa_bwd_d*.hip).
//
// The backward pass recomputes the probabilities from Q, K and the saved
// LSE instead of storing the score matrix ("FlashAttention-2" page, §3
// recomputation and §4 backward).  The gradient formulas are not on the
// pages; they are the chain rule of the forward definition:
//   P = exp(mod(scale q.k) - LSE), dV = P^T dO, dP = dO V^T,
//   delta_i = rowsum(dO_i * O_i), dS = P (dP - delta) mod',
//   dQ = scale dS K, dK = scale dS^T Q.
// Three phases on one stream: the row pass (delta and LSE in log2 units), a
// key-stationary kernel that owns 128 keys and loops over every query head of
// its GQA group and every query step (dK, dV accumulated in registers,
// written once), and a query-stationary kernel for dQ (like the forward
// pass).  When one call asks for the row pass and dQ, the dQ kernel does the
// row pass for its own rows and runs first (two launches instead of three).  Nothing is accumulated with atomics, so the results are
// deterministic.  Q/dO (resp. K/V) tiles go straight from memory into
// per-stage LDS objects, with the step loop unrolled by two.
#include <type_traits>

#include "fa_device.h"

namespace miattn {

// ---------------------------------------------------------------- row pass
// delta[row] = rowsum(dO * O); lse2[row] = LSE * log2(e), or +inf for rows
// with no admissible key (their probabilities are all zero).
//
// A row's delta is the sum of D / 8 partials over 16-byte chunks (dot8_bf16,
// chunk c = elements 8c .. 8c + 7), combined as a halving tree: partial c
// with partial c + D / 16, then c with c + D / 32, ... down to chunks 0 and 1.
// Both the row pass below and the dQ kernel's fused row pass (fuse_rows)
// follow exactly this order, so they give the same bits.
__device__ __forceinline__ float dot8_bf16(const u32x4& x, const u32x4& y) {
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) s += bf16_lo(x[e]) * bf16_lo(y[e]) + bf16_hi(x[e]) * bf16_hi(y[e]);
  return s;
}
__device__ __forceinline__ float lse_log2(float L) { return (L == kNegInf) ? __builtin_inff() : L * kLog2e; }

template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t* __restrict__ o,
                                                        const uint16_t* __restrict__ dout,
                                                        const float* __restrict__ lse, float* __restrict__ delta,
                                                        float* __restrict__ lse2, long rows) {
  constexpr int LPR = D / 8;  // lanes per row, 16 bytes each
  const long row = (long)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  float s = 0.0f;
  if (row < rows) s = dot8_bf16(*(const u32x4*)(o + row * D + c * 8), *(const u32x4*)(dout + row * D + c * 8));
  // Lane c adds lane c ^ w: the halving tree (addition is commutative).
#pragma unroll
  for (int w = LPR / 2; w >= 1; w >>= 1) s += __shfl_xor(s, w, LPR);
  if (row < rows && c == 0) {
    delta[row] = s;
    lse2[row] = lse_log2(lse[row]);
  }
}

// Probability, and the factor that turns dP - delta into dS, for one
// (query i, key j) score: p = 2^(x2 - lse2) with x2 the modified score in
// log2 units, the subtraction folded into the exponent's FMA.  `bias` is the
// relative-bias table entry of the pair (MOD_REL_BIAS only).  Softcap uses
// r = 1 / (1 + 2^(k raw)), k = 2 scale log2(e) / c: tanh(s / c) = 1 - 2r, so
// x2 = c log2(e) + (-2c log2(e)) r and the derivative 1 - tanh^2 = 4r(1 - r).
template <int MOD>
__device__ __forceinline__ void recompute_p(float sraw, int i, int j, float slope, float bias, const BwdArgs& a,
                                            float lse2, float& p, float& grad) {
  grad = 1.0f;
  if constexpr (MOD == MOD_NONE) {
    p = fast_exp2(__builtin_fmaf(sraw, a.scale_log2, -lse2));
  } else if constexpr (MOD == MOD_REL_BIAS) {
    p = fast_exp2(__builtin_fmaf(__builtin_fmaf(sraw, a.scale, bias), kLog2e, -lse2));
  } else if constexpr (MOD == MOD_ALIBI) {
    p = fast_exp2(__builtin_fmaf(sraw, a.scale_log2, __builtin_fmaf(slope * kLog2e, (float)(j - i), -lse2)));
  } else if constexpr (MOD == MOD_SOFTCAP) {
    const float r = fast_rcp(1.0f + fast_exp2(sraw * a.mod.softcap_k));
    p = fast_exp2(__builtin_fmaf(r, a.mod.softcap_m, -0.5f * a.mod.softcap_m - lse2));
    grad = 4.0f * __builtin_fmaf(-r, r, r);
  } else {
    int d = i - j;
    d = d < 0 ? -d : d;
    grad = d < a.mod.boost_radius ? a.mod.boost_factor : 1.0f;
    p = fast_exp2(__builtin_fmaf(sraw, a.scale_log2 * grad, -lse2));
  }
}

__device__ __forceinline__ u32x4 pack8(const f32x16& v, int base) {
  return u32x4{pack_bf16(v[base + 0], v[base + 1]), pack_bf16(v[base + 2], v[base + 3]),
               pack_bf16(v[base + 4], v[base + 5]), pack_bf16(v[base + 6], v[base + 7])};
}

// The dK/dV and dQ steps issue their LDS operand reads ahead of the matrix
// products (scheduling groups) where the registers allow it: every variant
// but the document mask, the relative bias, and local boost over a block
// mask, which would spill with the extra fragments in flight.
template <int MASK, int MOD, bool BM>
constexpr bool bwd_read_ahead() {
  return MASK != MASK_DOCUMENT && MOD != MOD_REL_BIAS && !(BM && MOD == MOD_BOOST);
}

// ---------------------------------------------------------------- dK, dV
// Workgroup: 4 waves own keys [k0, k0 + 128), 32 per wave (one key column
// per lane).  K rows stay in registers; the workgroup's 128 V rows sit in
// LDS for the whole kernel.  Per step: 32 query rows of one query head, Q
// and dO tiles in LDS.  S = Q K^T and dP = dO V^T come out key-column-per-
// lane, so P and dS are repacked in registers as the B operands of
// dV^T += dO^T P and dK^T += Q^T dS, whose A operands are transposing LDS
// reads.  Two workgroups fit per CU (2 waves per SIMD).
// DS: also store each step's bf16 dS (32 queries x this wave's 32 keys, in
// the register layout: lane l holds 16 queries of key kw0 + l % 32) as a
// 2 KB piece of block ds_block(kt, q0 / 32), zeros where the wave skips the
// step, for the dQ kernel that reads dS instead of recomputing it.
template <int D, int MASK, int MOD, bool BM, bool DS = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int BK = 128, BQ = 32;
  constexpr int ROW = D * 2, TILE = BQ * ROW;
  constexpr int KC = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(16))) char sV[BK * ROW];
  __shared__ __attribute__((aligned(16))) char sQ0[TILE], sO0[TILE], sQ1[TILE], sO1[TILE];
  // 64 entries each: one per lane of the loading wave (the last 32 are unused).
  __shared__ __attribute__((aligned(16))) float sL0[64], sE0[64], sL1[64], sE1[64];
  __shared__ __attribute__((aligned(16))) int sD0[64], sD1[64];
  // Relative-bias diagonals of one step: BQ + BK - 1 = 159 entries, 3 chunks of 64.
  constexpr bool REL = MOD == MOD_REL_BIAS;
  __shared__ __attribute__((aligned(16))) float sB0[REL ? 192 : 1], sB1[REL ? 192 : 1];

  const uint64_t t0 = trace_clock(a.trace);
  int b, hk, kt;
  decode_work(blockIdx.x, a.B, a.Hkv, a.Hkv, a.n_kt, false, b, hk, kt);
  if constexpr (BM) kt = ordered_tile(a.bm.kv_order, a.bm.n_b, b, a.bm.n_kv, kt, kt);
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = wave_uniform(tid >> 6);  // uniform: per-wave branches stay scalar
  const int gi = lane & 15, g16 = (lane >> 4) & 1;
  const int Sq = a.Sq, Skv = a.Skv, G = a.G, window = a.mask.window;
  const int k0 = kt * BK, kw0 = k0 + 32 * wave, kj = kw0 + l32;
  const bool col_ok = kj < Skv;
  const int vrow = 32 * wave + l32;  // this lane's key row in sV

  const uint16_t* Kh = (const uint16_t*)a.k + (size_t)(b * a.Hkv + hk) * Skv * D;
  const uint16_t* Vh = (const uint16_t*)a.v + (size_t)(b * a.Hkv + hk) * Skv * D;
  u32x4 kf[KC];
  {
    const u32x4* ks = (const u32x4*)(Kh + (size_t)(col_ok ? kj : 0) * D);
#pragma unroll
    for (int c = 0; c < KC; ++c) kf[c] = col_ok ? ks[2 * c + hh] : u32x4{0, 0, 0, 0};
  }
  const int32_t* doc = (MASK == MASK_DOCUMENT) ? a.mask.doc_ids + (size_t)b * Skv : nullptr;
  int doc_j = 0;
  if constexpr (MASK == MASK_DOCUMENT) doc_j = col_ok ? doc[kj] : -3;

  // query steps per head: analytic range or the block mask's q list of this key block
  constexpr int STEPS_PER_BLOCK = kMaskBlock / BQ;
  int qs_lo = 0, n_qs = 0;
  const int32_t* bm_list = nullptr;
  const uint8_t* bm_state = nullptr;
  if constexpr (BM) {
    const int bb = a.bm.n_b == 1 ? 0 : b;
    n_qs = a.bm.q_count[bb * a.bm.n_kv + kt] * STEPS_PER_BLOCK;
    bm_list = a.bm.q_index + (size_t)(bb * a.bm.n_kv + kt) * a.bm.n_q;
    bm_state = a.bm.tile_state + (size_t)bb * a.bm.n_q * a.bm.n_kv + kt;  // + qb * n_kv
  } else {
    int lo = 0, hi = Sq;
    if constexpr (MASK != MASK_NONE) lo = min(k0, Sq);
    if constexpr (MASK == MASK_WINDOW) hi = min(Sq, k0 + BK - 1 + window);
    if (hi > lo) {
      qs_lo = lo / BQ;
      n_qs = (hi + BQ - 1) / BQ - qs_lo;
    }
  }
  const int n_steps = G * n_qs;
  // Position of a step: query head g of the GQA group, query step j of that
  // head.  Steps run g-major; positions advance by counting, not dividing.
  struct Pos {
    int g, j;
  };
  auto advance = [&](Pos p) -> Pos {
    if (++p.j == n_qs) {
      p.j = 0;
      ++p.g;
    }
    return p;
  };
  // Block index (block-mask path) or query-step index (analytic) of step s.
  auto fetch_blk = [&](int s, Pos p) -> int {
    if (s >= n_steps) return 0;
    if constexpr (BM) return bm_list[p.j / STEPS_PER_BLOCK];
    return qs_lo + p.j;
  };
  auto query0 = [&](Pos p, int blk) -> int {
    if constexpr (BM) return blk * kMaskBlock + (p.j % STEPS_PER_BLOCK) * BQ;
    return blk * BQ;
  };

  const int tlen = Sq + Skv - 1;
  auto issue = [&](Pos p, int blk, char* qn, char* on, float* ln, float* en, int* dn, float* bn) {
    const int hq = hk * G + p.g, q0 = query0(p, blk);
    const size_t head = (size_t)(b * a.Hq + hq) * Sq;
    tile_load<D, BQ>(rows_rsrc((const uint16_t*)a.q + head * D, Sq, q0, ROW), qn, wave, lane);
    tile_load<D, BQ>(rows_rsrc((const uint16_t*)a.dout + head * D, Sq, q0, ROW), on, wave, lane);
    if (wave == 0) ints_to_lds(a.lse2 + head, Sq, q0, (int*)ln, lane);
    if (wave == 1) ints_to_lds(a.delta + head, Sq, q0, (int*)en, lane);
    if constexpr (MASK == MASK_DOCUMENT) {
      if (wave == 2) ints_to_lds(doc, Skv, q0, dn, lane);
    }
    if constexpr (REL) {
      // Entry e: i - j = q0 - k0 - (BK - 1) + e.
      if (wave < 3)
        bias_chunk_to_lds(uniform_ptr(a.mod.rel_bias + (size_t)hq * tlen), tlen, q0 - k0 - (BK - 1) + (Skv - 1), bn,
                          wave, lane);
    }
  };

  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }

  int blk_c = 0, blk_n = 0, st_c = 0, st_n = 0;
  Pos pc{0, 0};
  Pos pn = advance(pc);
  Pos pnn = advance(pn);
  auto step = [&](int s, const char* qs, const char* ds, const float* ls, const float* es, const int* dcs,
                  const float* bs, char* qn, char* on, float* ln, float* en, int* dn, float* bn) {
    const bool have_next = s + 1 < n_steps;
    if (have_next) issue(pn, blk_n, qn, on, ln, en, dn, bn);
    const int blk_nn = fetch_blk(s + 2, pnn);
    if constexpr (BM) st_n = have_next ? bm_state[(size_t)blk_n * a.bm.n_kv] : 0;
    const int hq = hk * G + pc.g;
    const int q0 = query0(pc, blk_c);
    int cls;
    if constexpr (BM) {
      cls = st_c == TILE_FULL ? TILE_FULL : TILE_PARTIAL;
    } else {
      cls = block_class<MASK>(q0, BQ, kw0, 32, Skv, window);
    }
    if (q0 + BQ > Sq && cls == TILE_FULL) cls = TILE_PARTIAL;
    if (kw0 >= Skv || q0 >= Sq) cls = TILE_EMPTY;
    u32x4* dsp = nullptr;
    if constexpr (DS)
      dsp = (u32x4*)(a.ds + ((size_t)(b * a.Hq + hq) * a.ds_blocks + ds_block<MASK>(kt, q0 / BQ, a.n_qs)) * kDsBlock) +
            2 * (wave * 64 + lane);

    if (cls != TILE_EMPTY) {
      const float slope = head_slope<MOD>(a.mod, hq, a.Hq);
      const int ch = 2 * g16 + ((gi & 3) >> 1);
      const int half = (gi & 1) * 8;
      // LDS operand offsets, rebuilt each step from two bases (XOR on the
      // chunk index, row_base) rather than held as one register per chunk:
      // row reads of chunk 2c + hh of row l32 (Q, dO; the V rows of this wave
      // share them, 32 rows further per wave), and transposing reads of rows
      // 16 cc + r00 (+ 8), chunk 4 dt + ch, at (t ^ 64 dt) + 16 cc ROW.
      const int qrow = opaque(row_base<D>(l32) ^ (16 * hh));
      const char* vw = sV + 32 * wave * ROW;
      f32x16 sp = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const int o = qrow ^ (32 * c);
        sp = mfma_bf16(*(const u32x4*)(qs + o), kf[c], sp);
        dp = mfma_bf16(*(const u32x4*)(ds + o), *(const u32x4*)(vw + o), dp);
      }
      // LDS operands read ahead of the matrix products: 4 reads first, then
      // per pair of products the next three (Q, dO, V of the next chunk).
      if constexpr (bwd_read_ahead<MASK, MOD, BM>()) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < KC - 2; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
      }
      // P and dS (register r: query q0 + 8(r/4) + 4hh + r%4).  Full tiles
      // take a branch without the mask test.  bl[8 rq + e] is the bias of
      // query q0 + 8 rq + 4hh + e and this lane's key.
      const float* bl = bs + (BK - 1 - 32 * wave - l32 + 4 * hh);
      // Row offsets 8 rq + 4 hh + e are rebuilt from this each step rather
      // than kept in 16 registers across the loop.
      const int hh4 = opaque(4 * hh);
      auto pds = [&](auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int ir = 8 * rq + hh4;
          const f32x4 L4 = *(const f32x4*)&ls[ir];
          const f32x4 E4 = *(const f32x4*)&es[ir];
          // Document ids of the four query rows, one 16-byte read.
          i32x4 D4 = {0, 0, 0, 0};
          if constexpr (MASKED && MASK == MASK_DOCUMENT) D4 = *(const i32x4*)&dcs[ir];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = q0 + ir + e;
            float p, grad;
            recompute_p<MOD>(sp[4 * rq + e], i, kj, slope, REL ? bl[8 * rq + e] : 0.0f, a, L4[e], p, grad);
            if constexpr (MASKED) {
              int di = 0;
              if constexpr (MASK == MASK_DOCUMENT) di = D4[e];
              const bool ok = col_ok && i < Sq && mask_ok<MASK>(i, kj, window, di, doc_j);
              p = ok ? p : 0.0f;
            }
            sp[4 * rq + e] = p;
            dp[4 * rq + e] = p * (dp[4 * rq + e] - E4[e]) * grad;
          }
        }
      };
      if (cls == TILE_PARTIAL) {
        pds(std::true_type{});
      } else {
        pds(std::false_type{});
      }
      const u32x4 pb0 = pack8(sp, 0), pb1 = pack8(sp, 8);
      const u32x4 sb0 = pack8(dp, 0), sb1 = pack8(dp, 8);
      const int r00 = 4 * hh + (gi >> 2);
      const int t0 = opaque((row_base<D>(r00) | half) ^ (16 * ch));
      const int t1 = opaque((row_base<D>(r00 + 8) | half) ^ (16 * ch));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int o0 = (t0 ^ (64 * dt)) + 16 * cc * ROW;
          const int o1 = (t1 ^ (64 * dt)) + 16 * cc * ROW;
          const u32x2 dlo = lds_read_tr16(ds + o0), dhi = lds_read_tr16(ds + o1);
          dv[dt] = mfma_bf16(u32x4{dlo[0], dlo[1], dhi[0], dhi[1]}, cc ? pb1 : pb0, dv[dt]);
          const u32x2 qlo = lds_read_tr16(qs + o0), qhi = lds_read_tr16(qs + o1);
          dk[dt] = mfma_bf16(u32x4{qlo[0], qlo[1], qhi[0], qhi[1]}, cc ? sb1 : sb0, dk[dt]);
        }
      if constexpr (DS) {
        dsp[0] = sb0;
        dsp[1] = sb1;
      }
    } else if constexpr (DS) {
      dsp[0] = u32x4{0, 0, 0, 0};
      dsp[1] = u32x4{0, 0, 0, 0};
    }
    if constexpr (DS) {
      // The next stage's loads (issued at the start of this step) have
      // landed; this step's two dS stores may still be in flight.
      wait_loads_not_last2();
      phase_barrier();
    } else {
      wait_loads();
      __syncthreads();
    }
    blk_c = blk_n;
    st_c = st_n;
    blk_n = blk_nn;
    pc = pn;
    pn = pnn;
    pnn = advance(pnn);
  };

  blk_c = fetch_blk(0, pc);
  blk_n = fetch_blk(1, pn);
  if constexpr (BM) st_c = n_steps > 0 ? bm_state[(size_t)blk_c * a.bm.n_kv] : 0;
  if (n_steps > 0) {
    tile_load<D, BK>(rows_rsrc(Vh, Skv, k0, ROW), sV, wave, lane);
    issue(pc, blk_c, sQ0, sO0, sL0, sE0, sD0, sB0);
    wait_loads();
  }
  __syncthreads();
  for (int s = 0; s < n_steps; s += 2) {
    step(s, sQ0, sO0, sL0, sE0, sD0, sB0, sQ1, sO1, sL1, sE1, sD1, sB1);
    if (s + 1 < n_steps) step(s + 1, sQ1, sO1, sL1, sE1, sD1, sB1, sQ0, sO0, sL0, sE0, sD0, sB0);
  }

  if (col_ok) {
    uint16_t* dK = (uint16_t*)a.dk + ((size_t)(b * a.Hkv + hk) * Skv + kj) * D;
    uint16_t* dV = (uint16_t*)a.dv + ((size_t)(b * a.Hkv + hk) * Skv + kj) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = 32 * dt + 8 * rq + 4 * hh;
        *(u32x2*)(dK + d0) = u32x2{pack_bf16(dk[dt][4 * rq] * a.scale, dk[dt][4 * rq + 1] * a.scale),
                                   pack_bf16(dk[dt][4 * rq + 2] * a.scale, dk[dt][4 * rq + 3] * a.scale)};
        *(u32x2*)(dV + d0) = u32x2{pack_bf16(dv[dt][4 * rq], dv[dt][4 * rq + 1]),
                                   pack_bf16(dv[dt][4 * rq + 2], dv[dt][4 * rq + 3])};
      }
  }
  trace_end(a.trace, blockIdx.x, t0, wave == 0, BK, n_steps);
}

// ---------------------------------------------------------------- dQ
// Workgroup: 4 waves own 128 query rows of one head, 32 per wave (one query
// column per lane, as in the forward kernel).  Per step: 64 keys, K and V
// tiles in LDS.  S^T = K Q^T and dP^T = V dO^T give dS^T with a query per
// lane; dQ^T += K^T dS^T takes K^T from transposing LDS reads.
//
// Relative-bias gradient (rel_bias_part set): the gradient of table entry
// i - j + Skv - 1 sums dS' over that diagonal.  Each step adds its dS'
// values into per-(wave, half-wave) LDS slices indexed by diagonal, with no
// two lanes of one instruction on the same entry, so the sums are
// deterministic.  At the start of the next step the slices are summed in a
// fixed order into a 256-entry ring indexed by the diagonal mod 256.  Keys
// only grow from step to step, so the diagonals above the next step's range
// are complete: they leave the ring into this tile's partial row, each
// written exactly once (never-touched diagonals are written as zero).
template <int D, int MASK, int MOD, bool BM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(BwdArgs a) {
  constexpr int BN = 64, NT = BN / 32;
  constexpr int ROW = D * 2, TILE = BN * ROW;
  constexpr int KC = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(16))) char sK0[TILE], sV0[TILE], sK1[TILE], sV1[TILE];
  __shared__ __attribute__((aligned(16))) int sD0[BN], sD1[BN];
  // Relative bias: diagonals of one step (128 + BN - 1 = 191 entries, 3 chunks).
  constexpr bool REL = MOD == MOD_REL_BIAS;
  __shared__ __attribute__((aligned(16))) float sB0[REL ? 192 : 1], sB1[REL ? 192 : 1];
  // Gradient slices [stage][wave][half][96] and the ring of open diagonals.
  constexpr int GS = 96;
  __shared__ __attribute__((aligned(16))) float sG[REL ? 2 * 8 * GS : 1], sRing[REL ? 256 : 1];

  const uint64_t t0 = trace_clock(a.trace);
  int b, hq, qt;
  decode_work(blockIdx.x, a.B, a.Hq, a.Hkv, a.n_qt,
              (MASK == MASK_CAUSAL || MASK == MASK_DOCUMENT) && !(BM && a.bm.q_order), b, hq, qt);
  if constexpr (BM) qt = ordered_tile(a.bm.q_order, a.bm.n_b, b, a.bm.n_q, qt, qt);
  const int hk = hq / a.G;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = wave_uniform(tid >> 6);  // uniform: per-wave branches stay scalar
  const int gi = lane & 15, g16 = (lane >> 4) & 1;
  const int Sq = a.Sq, Skv = a.Skv, window = a.mask.window;
  const int q0 = qt * kTileQ, qw0 = q0 + 32 * wave, qi = qw0 + l32;
  const bool row_ok = qi < Sq;

  const size_t ri = (size_t)(b * a.Hq + hq) * Sq + (row_ok ? qi : 0);
  const uint16_t* Qrow = (const uint16_t*)a.q + ri * D;
  const uint16_t* dOrow = (const uint16_t*)a.dout + ri * D;
  u32x4 qf[KC], of[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    qf[c] = row_ok ? ((const u32x4*)Qrow)[2 * c + hh] : u32x4{0, 0, 0, 0};
    of[c] = row_ok ? ((const u32x4*)dOrow)[2 * c + hh] : u32x4{0, 0, 0, 0};
  }
  float lse2, del;
  if (a.fuse_rows) {
    // The row pass for this lane's row: this lane holds chunks 2c + hh of
    // dO (c < KC), the other half-wave the rest.  The halving tree over the
    // chunk index pairs chunk 2c + hh with 2(c + w) + hh for w = KC/2 .. 1
    // in-lane, then the two half-waves.
    const uint16_t* Orow = (const uint16_t*)a.o + ri * D;
    float part[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c)
      part[c] = dot8_bf16(row_ok ? ((const u32x4*)Orow)[2 * c + hh] : u32x4{0, 0, 0, 0}, of[c]);
#pragma unroll
    for (int w = KC / 2; w >= 1; w >>= 1)
#pragma unroll
      for (int c = 0; c < w; ++c) part[c] += part[c + w];
    del = half_swap_sum(part[0]);
    lse2 = row_ok ? lse_log2(a.lse[ri]) : __builtin_inff();
    if (row_ok && hh == 0) {
      a.delta[ri] = del;
      const_cast<float*>(a.lse2)[ri] = lse2;
    }
  } else {
    lse2 = row_ok ? a.lse2[ri] : __builtin_inff();
    del = row_ok ? a.delta[ri] : 0.0f;
  }
  const uint16_t* K = (const uint16_t*)a.k + (size_t)(b * a.Hkv + hk) * Skv * D;
  const uint16_t* V = (const uint16_t*)a.v + (size_t)(b * a.Hkv + hk) * Skv * D;
  const int32_t* doc = nullptr;
  int doc_i = 0;
  if constexpr (MASK == MASK_DOCUMENT) {
    doc = a.mask.doc_ids + (size_t)b * Skv;
    doc_i = row_ok ? doc[qi] : -1;
  }
  const float slope = head_slope<MOD>(a.mod, hq, a.Hq);
  const int tlen = Sq + Skv - 1;
  const float* T = nullptr;
  if constexpr (REL) T = uniform_ptr(a.mod.rel_bias + (size_t)hq * tlen);
  const bool want_grad = REL && a.mod.rel_bias_part != nullptr;

  constexpr int STEPS_PER_BLOCK = kMaskBlock / BN;
  int step_lo = 0, n_steps = 0;
  const int32_t* bm_list = nullptr;
  const uint8_t* bm_state = nullptr;
  if constexpr (BM) {
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
  auto fetch_blk = [&](int s) -> int {
    if (s >= n_steps) return 0;
    if constexpr (BM) return bm_list[s / STEPS_PER_BLOCK];
    return step_lo + s;
  };
  auto key0 = [&](int s, int blk) -> int {
    if constexpr (BM) return blk * kMaskBlock + (s % STEPS_PER_BLOCK) * BN;
    return blk * BN;
  };

  auto issue = [&](int k0, char* kn, char* vn, int* dn, float* bn) {
    tile_load<D, BN>(rows_rsrc(K, Skv, k0, ROW), kn, wave, lane);
    tile_load<D, BN>(rows_rsrc(V, Skv, k0, ROW), vn, wave, lane);
    if constexpr (MASK == MASK_DOCUMENT) {
      if (wave == 0) ints_to_lds(doc, Skv, k0, dn, lane);
    }
    if constexpr (REL) {
      // Entry e: i - j = q0 - k0 - (BN - 1) + e.
      if (wave < 3) bias_chunk_to_lds(T, tlen, q0 - k0 - (BN - 1) + (Skv - 1), bn, wave, lane);
    }
  };

  // ---- relative-bias gradient: this tile's partial row and its flushes
  float* part = nullptr;
  if constexpr (REL) {
    if (want_grad) part = a.mod.rel_bias_part + ((size_t)(b * a.Hq + hq) * a.n_qt + qt) * (size_t)(Skv + kBiasRowPad);
  }
  int open_hi = q0 + kTileQ - 1;  // highest diagonal not yet written to the partial row
  // Close the step that started at key kp (its slices in g): diagonals above
  // next_hi are final.  Also writes zeros for never-touched diagonals in
  // (next_hi, open_hi].  Entry d of the row sits at d - q0 + Skv - 1.
  auto flush = [&](float* g, int kp, int next_hi) {
    const int lo = q0 - kp - (BN - 1), hi = q0 + kTileQ - 1 - kp;
    if (tid < kTileQ + BN - 1) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int e = tid - 32 * w;
        if (e >= 0 && e < 32 + BN - 1) {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            float* x = g + (2 * w + h2) * GS + e;
            v += *x;
            *x = 0.0f;
          }
        }
      }
      const int d = lo + tid;
      float* r = sRing + (d & 255);
      if (d > next_hi) {
        const int pos = d - q0 + Skv - 1;
        if (pos >= 0) part[pos] = *r + v;
        *r = 0.0f;
      } else {
        *r += v;
      }
    }
    for (int d = open_hi - tid; d > next_hi; d -= 256) {
      const int pos = d - q0 + Skv - 1;
      if ((d < lo || d > hi) && pos >= 0) part[pos] = 0.0f;
    }
    open_hi = next_hi;
  };

  f32x16 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = f32x16{};

  int blk_c = 0, blk_n = 0, st_c = 0, st_n = 0, k_prev = 0;
  auto step = [&](int s, const char* ks, const char* vs, const int* dcs, const float* bs, float* gs, float* gp,
                  char* kn, char* vn, int* dn, float* bn) {
    const int k0 = key0(s, blk_c);
    const bool have_next = s + 1 < n_steps;
    if (have_next) issue(key0(s + 1, blk_n), kn, vn, dn, bn);
    if constexpr (REL) {
      if (want_grad && s > 0) flush(gp, k_prev, q0 + kTileQ - 1 - k0);
      k_prev = k0;
    }
    const int blk_nn = fetch_blk(s + 2);
    if constexpr (BM) st_n = have_next ? bm_state[blk_n] : 0;
    int cls;
    if constexpr (BM) {
      cls = (k0 >= Skv) ? TILE_EMPTY : (st_c == TILE_FULL ? TILE_FULL : TILE_PARTIAL);
    } else {
      cls = block_class<MASK>(qw0, 32, k0, BN, Skv, window);
    }
    if (qw0 >= Sq) cls = TILE_EMPTY;

    if (cls != TILE_EMPTY) {
      const int ch = 2 * g16 + ((gi & 3) >> 1);
      const int half = (gi & 1) * 8;
      // bl[59 - c]: bias of key k0 + c + 4hh; gl[59 - c]: its gradient slot
      // in this (wave, half-wave) slice (c = 32t + 8(r/4) + r%4).
      const float* bl = bs + (32 * wave + l32 + 4 - 4 * hh);
      float* gl = gs + (2 * wave + hh) * GS + (l32 + 4 - 4 * hh);
      // LDS operand offsets, rebuilt each step from a few bases (XOR on the
      // chunk index, row_base) rather than held as one register per chunk:
      // row reads of chunk 2c + hh of row 32t + l32 (K, V), and transposing
      // reads of rows 32t + 16cc + r00 (+ 8), chunk 4dt + ch, of K.
      const int krow = opaque(row_base<D>(l32) ^ (16 * hh));
      const int r00 = 4 * hh + (gi >> 2);
      const int t0 = opaque((row_base<D>(r00) | half) ^ (16 * ch));
      const int t1 = opaque((row_base<D>(r00 + 8) | half) ^ (16 * ch));
      // One 32-key subtile at a time keeps the live registers low.
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x16 st = f32x16{}, dpt = f32x16{};
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const int o = (krow ^ (32 * c)) + 32 * t * ROW;
          st = mfma_bf16(*(const u32x4*)(ks + o), qf[c], st);
          dpt = mfma_bf16(*(const u32x4*)(vs + o), of[c], dpt);
        }
        // K and V fragments read four products ahead.
        if constexpr (bwd_read_ahead<MASK, MOD, BM>()) {
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
          for (int i = 0; i < 2 * KC - 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
        // Full tiles take a branch without the mask test.
        auto pds = [&](auto masked) {
          constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            // Document ids of four consecutive keys, one 16-byte read.
            i32x4 D4 = {0, 0, 0, 0};
            if constexpr (MASKED && MASK == MASK_DOCUMENT) D4 = *(const i32x4*)&dcs[32 * t + 8 * g4 + 4 * hh];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int rr = 4 * g4 + e;
              const int c = 32 * t + 8 * g4 + e;
              const int jr = c + 4 * hh;
              const int j = k0 + jr;
              float p, grad;
              recompute_p<MOD>(st[rr], qi, j, slope, REL ? bl[59 - c] : 0.0f, a, lse2, p, grad);
              if constexpr (MASKED) {
                int dj = 0;
                if constexpr (MASK == MASK_DOCUMENT) dj = D4[e];
                const bool ok = j < Skv && mask_ok<MASK>(qi, j, window, doc_i, dj);
                p = ok ? p : 0.0f;
              }
              dpt[rr] = p * (dpt[rr] - del) * grad;
              if constexpr (REL) {
                if (want_grad)
                  __hip_atomic_fetch_add(gl + (59 - c), dpt[rr], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
              }
            }
          }
        };
        if (cls == TILE_PARTIAL) {
          pds(std::true_type{});
        } else {
          pds(std::false_type{});
        }
        const u32x4 sb0 = pack8(dpt, 0), sb1 = pack8(dpt, 8);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const int rows = (32 * t + 16 * cc) * ROW;
            const u32x2 lo = lds_read_tr16(ks + ((t0 ^ (64 * dt)) + rows));
            const u32x2 hi = lds_read_tr16(ks + ((t1 ^ (64 * dt)) + rows));
            dq[dt] = mfma_bf16(u32x4{lo[0], lo[1], hi[0], hi[1]}, cc ? sb1 : sb0, dq[dt]);
          }
        // Transposing K reads two products ahead.
        if constexpr (bwd_read_ahead<MASK, MOD, BM>()) {
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
          for (int i = 0; i < 2 * DT - 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
      }
    }
    wait_loads();
    __syncthreads();
    blk_c = blk_n;
    st_c = st_n;
    blk_n = blk_nn;
  };

  blk_c = fetch_blk(0);
  blk_n = fetch_blk(1);
  if constexpr (BM) st_c = n_steps > 0 ? bm_state[blk_c] : 0;
  if constexpr (REL) {
    if (want_grad) {
      for (int x = tid; x < 2 * 8 * GS; x += 256) sG[x] = 0.0f;
      sRing[tid] = 0.0f;
    }
  }
  if (n_steps > 0) {
    issue(key0(0, blk_c), sK0, sV0, sD0, sB0);
    wait_loads();
  }
  __syncthreads();
  for (int s = 0; s < n_steps; s += 2) {
    step(s, sK0, sV0, sD0, sB0, sG, sG + 8 * GS, sK1, sV1, sD1, sB1);
    if (s + 1 < n_steps) step(s + 1, sK1, sV1, sD1, sB1, sG + 8 * GS, sG, sK0, sV0, sD0, sB0);
  }
  if constexpr (REL) {
    if (want_grad) {
      // Close the last step (its slices are in stage (n_steps - 1) & 1) and
      // write every remaining diagonal down to q0 - Skv + 1.
      if (n_steps > 0) {
        flush(sG + ((n_steps - 1) & 1) * 8 * GS, k_prev, q0 - Skv);
      } else {
        for (int d = open_hi - tid; d > q0 - Skv; d -= 256) part[d - q0 + Skv - 1] = 0.0f;
      }
    }
  }

  if (row_ok) {
    uint16_t* dQ = (uint16_t*)a.dq + ri * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = 32 * dt + 8 * rq + 4 * hh;
        *(u32x2*)(dQ + d0) = u32x2{pack_bf16(dq[dt][4 * rq] * a.scale, dq[dt][4 * rq + 1] * a.scale),
                                   pack_bf16(dq[dt][4 * rq + 2] * a.scale, dq[dt][4 * rq + 3] * a.scale)};
      }
  }
  trace_end(a.trace == nullptr ? nullptr : a.trace + (size_t)a.B * a.Hkv * a.n_kt * FA_WG_TRACE_WORDS, blockIdx.x,
            t0, wave == 0, kTileQ, n_steps);
}

// ---------------------------------------------------------------- dQ from stored dS
// dQ = scale dS K with dS read back from the blocks the dK/dV kernel stored
// (no mask or the causal mask, no relative bias): nothing is recomputed.
// Workgroup: 4 waves own the 128 query rows of (b, hq, qt), wave w the query
// step 4 qt + w.  Per step of 64 keys, straight into LDS: the K rows
// (swizzled, as everywhere) and, per wave, its 64 x 32 piece of dS, gathered
// so that LDS row j holds key j's two 32-byte lane chunks (the 16 queries of
// half 0, then of half 1): 64-byte rows, which the transposing reads below
// access without bank conflicts.  dQ^T += K^T dS^T takes both operands from
// transposing reads with the same key rows, so their k orders agree; the
// output column of lane l is position p = l % 32 of those rows, i.e. query
// 8 ((p % 16) / 4) + 4 (p / 16) + p % 4 of the wave's step.
template <int D, int MASK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_ds_kernel(BwdArgs a) {
  static_assert(MASK == MASK_NONE || MASK == MASK_CAUSAL, "stored dS covers the unmasked and causal cases");
  constexpr int BN = 64, ROW = D * 2, TILE = BN * ROW, DT = D / 32;
  constexpr int SROW = 64, SWAVE = BN * SROW;  // one wave's dS piece: 4 KB
  __shared__ __attribute__((aligned(16))) char sK0[TILE], sK1[TILE];
  __shared__ __attribute__((aligned(16))) char sS0[4 * SWAVE], sS1[4 * SWAVE];

  const uint64_t t0 = trace_clock(a.trace);
  int b, hq, qt;
  decode_work(blockIdx.x, a.B, a.Hq, a.Hkv, a.n_qt, MASK == MASK_CAUSAL, b, hq, qt);
  const int hk = hq / a.G;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = wave_uniform(tid >> 6);
  const int gi = lane & 15, g16 = (lane >> 4) & 1;
  const int Sq = a.Sq, Skv = a.Skv;
  const int q0 = qt * kTileQ, qw0 = q0 + 32 * wave;
  const bool wave_ok = qw0 < Sq;  // steps past Sq were never stored
  const int qs = qw0 / 32;

  const uint16_t* K = uniform_ptr((const uint16_t*)a.k + (size_t)(b * a.Hkv + hk) * Skv * D);
  const uint16_t* dsh = uniform_ptr(a.ds + (size_t)(b * a.Hq + hq) * a.ds_blocks * kDsBlock);
  const int hi = MASK == MASK_CAUSAL ? min(Skv, q0 + kTileQ) : Skv;
  const int n_steps = hi > 0 ? (hi + BN - 1) / BN : 0;

  // Gather offsets (bytes within a 4 KB half block) of this lane's chunks:
  // load k writes LDS rows 16 k + lane / 4; chunk (lane % 4) of a row is
  // 16 bytes of lane chunk (key, half (lane % 4) / 2), part lane % 2.
  // A wave whose step lies past Sq reads through an empty resource: zeros.
  auto issue = [&](int s, char* kb, char* sb) {
    tile_load<D, BN>(rows_rsrc(K, Skv, s * BN, ROW), kb, wave, lane);
    const long blk = wave_ok ? ds_block<MASK>(s >> 1, qs, a.n_qs) : 0;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(dsh + (size_t)blk * kDsBlock + (size_t)(s & 1) * (kDsBlock / 2),
                                               wave_ok ? kDsBlock : 0);  // 4 KB: half of the block
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int j = 16 * k + (lane >> 2), w2 = j >> 5, jl = j & 31;
      const uint32_t off = (uint32_t)((w2 * 64 + jl + 32 * ((lane & 3) >> 1)) * 32 + 16 * (lane & 1));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(sb + wave * SWAVE + 1024 * k), 16, off, 0, 0, 0);
    }
  };

  f32x16 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = f32x16{};

  const int ch = 2 * g16 + ((gi & 3) >> 1);
  const int half = (gi & 1) * 8;
  auto step = [&](int s, const char* kb, const char* sb, char* kn, char* sn) {
    if (s + 1 < n_steps) issue(s + 1, kn, sn);
    {
      // K^T rows 32t + 16cc + r00 (+ 8), chunk 4dt + ch: (t ^ 64 dt) + row offset
      // (as in the other backward kernels); dS^T: the same key rows of the
      // 64-byte rows of this wave's piece, chunk ch.
      const int r00 = 4 * hh + (gi >> 2);
      const int t0 = opaque((row_base<D>(r00) | half) ^ (16 * ch));
      const int t1 = opaque((row_base<D>(r00 + 8) | half) ^ (16 * ch));
      const char* sw = sb + opaque(wave * SWAVE + r00 * SROW + ch * 16 + half);
#pragma unroll
      for (int kc = 0; kc < BN / 16; ++kc) {
        const u32x2 slo = lds_read_tr16(sw + 16 * kc * SROW), shi = lds_read_tr16(sw + (16 * kc + 8) * SROW);
        const u32x4 bfrag = u32x4{slo[0], slo[1], shi[0], shi[1]};
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int rows = 16 * kc * ROW;
          const u32x2 lo = lds_read_tr16(kb + ((t0 ^ (64 * dt)) + rows));
          const u32x2 hi2 = lds_read_tr16(kb + ((t1 ^ (64 * dt)) + rows));
          dq[dt] = mfma_bf16(u32x4{lo[0], lo[1], hi2[0], hi2[1]}, bfrag, dq[dt]);
        }
      }
    }
    wait_loads();
    __syncthreads();
  };

  if (n_steps > 0) {
    issue(0, sK0, sS0);
    wait_loads();
  }
  __syncthreads();
  for (int s = 0; s < n_steps; s += 2) {
    step(s, sK0, sS0, sK1, sS1);
    if (s + 1 < n_steps) step(s + 1, sK1, sS1, sK0, sS0);
  }

  // Lane l holds position p = l % 32: query 8 ((p % 16) / 4) + 4 (p / 16) + p % 4.
  const int qi = qw0 + 8 * ((l32 & 15) >> 2) + 4 * (l32 >> 4) + (l32 & 3);
  if (qi < Sq) {
    uint16_t* dQ = (uint16_t*)a.dq + ((size_t)(b * a.Hq + hq) * Sq + qi) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = 32 * dt + 8 * rq + 4 * hh;
        *(u32x2*)(dQ + d0) = u32x2{pack_bf16(dq[dt][4 * rq] * a.scale, dq[dt][4 * rq + 1] * a.scale),
                                   pack_bf16(dq[dt][4 * rq + 2] * a.scale, dq[dt][4 * rq + 3] * a.scale)};
      }
  }
  trace_end(a.trace == nullptr ? nullptr : a.trace + (size_t)a.B * a.Hkv * a.n_kt * FA_WG_TRACE_WORDS, blockIdx.x,
            t0, wave == 0, kTileQ, n_steps);
}

// ---------------------------------------------------------------- bias gradient
// grad[h][r] = sum over batches b and query tiles qt of the dQ workgroups'
// partial rows, entry r - 128 qt of row (b, h, qt), in that fixed order, so
// the result is deterministic.  Tile qt's row covers table entries
// [128 qt, 128 qt + Skv + 126].  (Templated on the head dimension only so
// that each translation unit has its own instance.)
template <int D>
__global__ __launch_bounds__(256) void bias_grad_reduce_kernel(const float* __restrict__ part,
                                                               float* __restrict__ grad, int B, int Hq, int n_qt,
                                                               int Skv, int tlen, int blocks_per_head) {
  const int h = blockIdx.x / blocks_per_head;
  const int r = (blockIdx.x - h * blocks_per_head) * 256 + threadIdx.x;
  if (r >= tlen) return;
  const size_t row = (size_t)Skv + kBiasRowPad;
  const int first = r - (Skv + kTileQ - 2);
  const int qt_lo = first > 0 ? (first + kTileQ - 1) / kTileQ : 0;
  const int qt_hi = min(n_qt - 1, r / kTileQ);
  float s = 0.0f;
  for (int b = 0; b < B; ++b) {
    const float* p = part + (size_t)(b * Hq + h) * n_qt * row;
    for (int qt = qt_lo; qt <= qt_hi; ++qt) s += p[(size_t)qt * row + (r - qt * kTileQ)];
  }
  grad[(size_t)h * tlen + r] = s;
}

template <int D, int MASK, int MOD, bool BM>
static hipError_t launch_bwd_mm(const BwdArgs& a_in, int phases, hipStream_t st) {
  BwdArgs a = a_in;
  const long rows = (long)a.B * a.Hq * a.Sq;
  const int rows_per_block = 256 / (D / 8);
  // Stored dS (the host sets a.ds only for these variants): the dK/dV kernel
  // writes dS and the dQ kernel reads it.
  constexpr bool DS_OK = (MASK == MASK_NONE || MASK == MASK_CAUSAL) && !BM && MOD != MOD_REL_BIAS;
  const bool use_ds = DS_OK && a.ds != nullptr;
  // The row pass and the recomputing dQ kernel in one call: one launch, the
  // dQ kernel doing the row pass for its own rows (and writing them for a
  // dK/dV launch that follows).  Same bits as the two launches.
  const int asked = phases;
  if ((phases & 5) == 5 && !use_ds && rows > 0) {
    a.fuse_rows = 1;
    hipLaunchKernelGGL((bwd_dq_kernel<D, MASK, MOD, BM>), dim3((unsigned)(a.B * a.Hq * a.n_qt)), dim3(256), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.fuse_rows = 0;
    phases &= ~5;
  }
  if ((phases & 1) && rows > 0) {
    hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)),
                       dim3(256), 0, st, (const uint16_t*)a.o, (const uint16_t*)a.dout, a.lse, a.delta,
                       const_cast<float*>(a.lse2), rows);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // dK, dV are written for every key (zero when no query sees it).
  if ((phases & 2) && (long)a.B * a.Hkv * a.n_kt > 0) {
    const dim3 grid((unsigned)(a.B * a.Hkv * a.n_kt));
    if constexpr (DS_OK) {
      if (use_ds) {
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, MASK, MOD, BM, true>), grid, dim3(256), 0, st, a);
      } else {
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, MASK, MOD, BM>), grid, dim3(256), 0, st, a);
      }
    } else {
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, MASK, MOD, BM>), grid, dim3(256), 0, st, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((phases & 4) && rows > 0) {
    const dim3 grid((unsigned)(a.B * a.Hq * a.n_qt));
    if constexpr (DS_OK) {
      if (use_ds) {
        hipLaunchKernelGGL((bwd_dq_ds_kernel<D, MASK>), grid, dim3(256), 0, st, a);
      } else {
        hipLaunchKernelGGL((bwd_dq_kernel<D, MASK, MOD, BM>), grid, dim3(256), 0, st, a);
      }
    } else {
      hipLaunchKernelGGL((bwd_dq_kernel<D, MASK, MOD, BM>), grid, dim3(256), 0, st, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if constexpr (MOD == MOD_REL_BIAS) {
    // The table gradient (also when there are no rows: then it is zero).
    const int tlen = a.Sq + a.Skv - 1;
    if ((asked & 4) && a.mod.rel_bias_grad != nullptr && tlen > 0) {
      const int per_head = (tlen + 255) / 256;
      hipLaunchKernelGGL((bias_grad_reduce_kernel<D>), dim3((unsigned)(a.Hq * per_head)), dim3(256), 0, st,
                         a.mod.rel_bias_part, a.mod.rel_bias_grad, rows > 0 ? a.B : 0, a.Hq, a.n_qt, a.Skv, tlen,
                         per_head);
      return hipGetLastError();
    }
  }
  return hipSuccess;
}

template <int D, int MASK, int MOD>
static hipError_t launch_bwd_bm(const BwdArgs& a, int phases, hipStream_t st) {
  return a.bm.tile_state != nullptr ? launch_bwd_mm<D, MASK, MOD, true>(a, phases, st)
                                    : launch_bwd_mm<D, MASK, MOD, false>(a, phases, st);
}

template <int D, int MASK>
static hipError_t launch_bwd_mask(const BwdArgs& a, int mod, int phases, hipStream_t st) {
  switch (mod) {
    case MOD_NONE: return launch_bwd_bm<D, MASK, MOD_NONE>(a, phases, st);
    case MOD_ALIBI: return launch_bwd_bm<D, MASK, MOD_ALIBI>(a, phases, st);
    case MOD_SOFTCAP: return launch_bwd_bm<D, MASK, MOD_SOFTCAP>(a, phases, st);
    case MOD_REL_BIAS: return launch_bwd_bm<D, MASK, MOD_REL_BIAS>(a, phases, st);
    default: return launch_bwd_bm<D, MASK, MOD_BOOST>(a, phases, st);
  }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, int mask, int mod, int phases, hipStream_t st) {
  switch (mask) {
    case MASK_NONE: return launch_bwd_mask<D, MASK_NONE>(a, mod, phases, st);
    case MASK_CAUSAL: return launch_bwd_mask<D, MASK_CAUSAL>(a, mod, phases, st);
    case MASK_WINDOW: return launch_bwd_mask<D, MASK_WINDOW>(a, mod, phases, st);
    default: return launch_bwd_mask<D, MASK_DOCUMENT>(a, mod, phases, st);
  }
}

}  // namespace miattn
