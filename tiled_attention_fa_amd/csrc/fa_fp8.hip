// FP8 path ("FlashAttention-3 (KO)" page, technical innovation 3: FP8
// doubles the matrix throughput of 16-bit formats; incoherent processing
// multiplies Q and K by a random orthogonal matrix such as a Hadamard matrix
// before quantizing, which spreads outliers and leaves Q K^T unchanged).
//
// Format: OCP E4M3 (gfx950's FP8 conversions and MFMA).  Every tensor is
// quantized in blocks of 128 rows of one (batch, head) with one power-of-two
// scale per block, stored as an E8M0 byte (e + 127); the matrix cores apply
// these scales themselves (v_mfma_scale_f32_32x32x64_f8f6f4), so the kernel
// spends no vector instructions on dequantization.
//
// fp8_quantize_kernel: one workgroup per (row group, 128-row block), one
// thread per row.  Optional incoherence transform x -> (x * signs) H / sqrt(D)
// (H the Sylvester Hadamard matrix, applied as an in-register fast
// Walsh-Hadamard transform), block max, the smallest 2^e with
// max <= 448 * 2^e, then round-to-nearest-even to E4M3 of x / 2^e.
//
// fwd_fp8_kernel: the 4-wave forward of fwd_kernel with both products on
// 32x32x64 FP8 MFMA.  Per 64-key step: S^T = K Q^T (two MFMAs per 32-key
// subtile at D = 128), the softmax as in the bf16 kernel, P rounded to E4M3
// (P <= 1 relative to the running max) and packed in the order the S^T
// accumulator holds the keys, and O^T += V^T P^T with V^T assembled by
// ds_read_b64_tr_b8 reads so that every k-slot carries the same key in both
// operands.  The row sum takes the unrounded probabilities.
#include "fa_device.h"
#include "fa_launch.h"

namespace miattn {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

// FP8 tile rows are D bytes: (256 / D) rows share one 256-byte bank window.
// The 16-byte chunk c of row r is stored at chunk c ^ f(m), m = r / (256 /
// D) mod (D / 16).  The K reads (16 lanes of 16 bytes per LDS pass: 16
// consecutive rows at one chunk) need f one-to-one on every 8 (D = 128) or
// 4 (D = 64) consecutive m.  The transposing V reads (32 lanes of 8 bytes
// per pass) take two adjacent chunks c, c ^ 1 of 8 rows; at D = 128 those
// rows are the pairs m0 + {0, 1, 4, 5} (m0 = 0, 2 mod 8), so f / 2 must
// also differ over each such set: f swaps the two low bits of m, which
// keeps f a permutation and meets both.  At D = 64, f = m serves both.
template <int D>
__device__ __forceinline__ int swz8(int r, int c) {
  if constexpr (D == 128) {
    const int m = (r >> 1) & 7;
    return c ^ (((m & 1) << 1) | ((m >> 1) & 1) | (m & 4));
  } else {
    return c ^ ((r / (256 / D)) & (D / 16 - 1));
  }
}

// ROWS rows of an FP8 [rows][D] matrix into an LDS tile in the swz8 layout
// (buffer loads straight to LDS, zero past the resource's end); 4 waves.
template <int D, int ROWS>
__device__ __forceinline__ void tile_load8(__amdgpu_buffer_rsrc_t rsrc, char* tile, int wave, int lane) {
  constexpr int PER_WAVE = ROWS * D / 1024 / 4;
  static_assert(PER_WAVE * 4 * 1024 == ROWS * D, "tile must split into 1 KB loads over 4 waves");
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int byte = (wave * PER_WAVE + i) * 1024 + lane * 16;
    const int r = byte / D, p = (byte % D) / 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void*)(tile + (wave * PER_WAVE + i) * 1024), 16,
        (uint32_t)(r * D + swz8<D>(r, p) * 16), 0, 0, 0);
  }
}

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c, int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, scale_b);
}

// Two floats (|x| <= 448) -> two E4M3 codes in the low (HI false) or high
// half of `old`.
template <bool HI>
__device__ __forceinline__ int pack_fp8(float x, float y, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(x, y, old, HI);
}

// ---------------------------------------------------------------- quantize
template <int D>
__global__ __launch_bounds__(128) void fp8_quantize_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ x8,
                                                           uint8_t* __restrict__ scales, int S, int nblk,
                                                           const float* __restrict__ signs) {
  const int blk = blockIdx.x, grp = blockIdx.y, t = threadIdx.x;
  const int row = blk * 128 + t;
  const bool ok = row < S;
  const size_t base = ((size_t)grp * S + (ok ? row : 0)) * D;
  float v[D];
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const u32x4 w = ok ? *(const u32x4*)(x + base + 8 * c) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[8 * c + 2 * e] = bf16_lo(w[e]);
      v[8 * c + 2 * e + 1] = bf16_hi(w[e]);
    }
  }
  if (signs != nullptr) {
#pragma unroll
    for (int d = 0; d < D; ++d) v[d] *= signs[d];
#pragma unroll
    for (int h = 1; h < D; h <<= 1)
#pragma unroll
      for (int i = 0; i < D; ++i)
        if ((i & h) == 0) {
          const float p = v[i], q = v[i + h];
          v[i] = p + q;
          v[i + h] = p - q;
        }
    const float rs = D == 64 ? 0.125f : 0.088388347648318440550f;  // 1 / sqrt(D)
#pragma unroll
    for (int d = 0; d < D; ++d) v[d] *= rs;
  }
  // The block scale comes from the finite values; a NaN stays NaN (E4M3's
  // NaN code) and +-Inf saturates at +-448 like any value out of range.
  float amax = 0.0f;
#pragma unroll
  for (int d = 0; d < D; ++d) amax = fmaxf(amax, __builtin_isfinite(v[d]) ? fabsf(v[d]) : 0.0f);
  __shared__ float s_max[2];
  for (int w = 32; w >= 1; w >>= 1) amax = fmaxf(amax, __shfl_xor(amax, w));
  if ((t & 63) == 0) s_max[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(s_max[0], s_max[1]);
  // smallest e with amax <= 448 * 2^e (exact: powers of two)
  int e = 0;
  if (amax > 0.0f) {
    int e2;
    (void)frexpf(amax, &e2);
    e = e2 - 9;
    while (amax > ldexpf(448.0f, e)) ++e;
    while (e > -127 && amax <= ldexpf(448.0f, e - 1)) --e;
    e = max(-127, min(127, e));
  }
  if (ok) {
    uint8_t* out = x8 + base;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      u32x4 w;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float f[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float y = ldexpf(v[16 * c + 4 * k + i], -e);
          f[i] = y != y ? y : fminf(fmaxf(y, -448.0f), 448.0f);
        }
        const int lo = pack_fp8<false>(f[0], f[1], 0);
        w[k] = (uint32_t)pack_fp8<true>(f[2], f[3], lo);
      }
      *(u32x4*)(out + 16 * c) = w;
    }
  }
  if (t == 0) scales[(size_t)grp * nblk + blk] = (uint8_t)(e + 127);
}

// ---------------------------------------------------------------- forward
template <int D, int MASK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_fp8_kernel(Fp8FwdArgs a) {
  constexpr int BN = 64, NT = 2, TILE = BN * D;
  constexpr int KC = D / 64;  // 64-wide k chunks of one S product
  constexpr int DT = D / 32;  // 32-row d tiles of O^T
  __shared__ __attribute__((aligned(16))) char sK0[TILE], sV0[TILE];
  __shared__ __attribute__((aligned(16))) char sK1[TILE], sV1[TILE];

  int b, hq, qt;
  decode_work(blockIdx.x, a.B, a.Hq, a.Hkv, a.n_qt, MASK == MASK_CAUSAL, b, hq, qt);
  const int hk = hq / a.G;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = wave_uniform(tid >> 6);
  const int Sq = a.Sq, Skv = a.Skv, window = a.window;
  const int q0 = qt * kTileQ, qw0 = q0 + 32 * wave, qi = qw0 + l32;
  const bool row_ok = qi < Sq;
  const int nbq = (Sq + 127) / 128, nbk = (Skv + 127) / 128;

  const uint8_t* Q = a.q8 + (size_t)(b * a.Hq + hq) * Sq * D;
  const uint8_t* K = uniform_ptr(a.k8 + (size_t)(b * a.Hkv + hk) * Skv * D);
  const uint8_t* V = uniform_ptr(a.v8 + (size_t)(b * a.Hkv + hk) * Skv * D);
  const int sq = a.q_scale[(size_t)(b * a.Hq + hq) * nbq + qt];  // the 128-row query tile is one block
  const uint8_t* KS = a.k_scale + (size_t)(b * a.Hkv + hk) * nbk;
  const uint8_t* VS = a.v_scale + (size_t)(b * a.Hkv + hk) * nbk;

  // Q fragments (B operand of S^T): bytes 64c + 32hh .. +31 of this lane's row.
  i32x8 qf[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    const u32x4* src = (const u32x4*)(Q + (size_t)(row_ok ? qi : 0) * D + 64 * c + 32 * hh);
    const u32x4 x0 = row_ok ? src[0] : u32x4{0, 0, 0, 0}, x1 = row_ok ? src[1] : u32x4{0, 0, 0, 0};
    qf[c] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
  }

  int step_lo = 0, n_steps = 0;
  {
    int lo, hi;
    key_range<MASK>(q0, min(q0 + kTileQ, Sq), Skv, window, lo, hi);
    if (hi > lo) {
      step_lo = lo / BN;
      n_steps = (hi + BN - 1) / BN - step_lo;
    }
  }
  auto issue = [&](int s, char* ks, char* vs) {
    const int k0 = (step_lo + s) * BN;
    tile_load8<D, BN>(rows_rsrc(K, Skv, k0, D), ks, wave, lane);
    tile_load8<D, BN>(rows_rsrc(V, Skv, k0, D), vs, wave, lane);
  };

  float m = kNegInf, l = 0.0f, lc = 0.0f;  // lc: compensation of l
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  // Per-lane constants of the transposing V^T reads: this lane addresses key
  // kappa(8q + L/2) of the step (L = lane within its 16-lane group), d bytes
  // 16 g + 8 (L % 2) of each 32-wide d tile (g = 16-lane group within the half).
  const int L = lane & 15, g16 = (lane >> 4) & 1;

  auto step = [&](int s, const char* ks, const char* vs, char* kn, char* vn) {
    const int k0 = (step_lo + s) * BN;
    if (s + 1 < n_steps) issue(s + 1, kn, vn);
    int cls = qw0 >= Sq ? TILE_EMPTY : block_class<MASK>(qw0, 32, k0, BN, Skv, window);
    if (cls != TILE_EMPTY) {
      const int skb = KS[k0 / 128], svb = VS[k0 / 128];
      // ---- S^T = K Q^T (block scales applied by the MFMA)
      f32x16 st[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        st[t] = f32x16{};
        const int r = 32 * t + l32;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const int ch = 4 * c + 2 * hh;
          const u32x4 y0 = *(const u32x4*)(ks + r * D + swz8<D>(r, ch) * 16);
          const u32x4 y1 = *(const u32x4*)(ks + r * D + swz8<D>(r, ch + 1) * 16);
          const i32x8 kf = i32x8{(int)y0[0], (int)y0[1], (int)y0[2], (int)y0[3], (int)y1[0], (int)y1[1], (int)y1[2], (int)y1[3]};
          st[t] = mfma_fp8(kf, qf[c], st[t], skb, sq);
        }
      }
      // ---- V^T fragments of the whole step, read before the softmax so their
      // latency hides behind it.  A-operand byte p of a lane is V[kappa(hh, p)][d].
      i32x8 vf[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int qv = 0; qv < 4; ++qv) {
          const int pk = 8 * qv + (L >> 1);                 // k-slot this lane addresses
          const int key = 32 * (pk >> 4) + 8 * ((pk & 15) >> 2) + 4 * hh + (pk & 3);
          const int ch = 2 * dt + g16;
          const char* addr = vs + key * D + swz8<D>(key, ch) * 16 + 8 * (L & 1);
          typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
          const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (lds_i32x2*)((const __attribute__((address_space(3))) char*)(addr)));
          vf[dt][2 * qv] = x[0];
          vf[dt][2 * qv + 1] = x[1];
        }
      // ---- softmax (as the bf16 kernel)
      // Raw scores stay raw: masked pairs become -inf in place (the log2
      // multiplier is > 0) and the multiplier folds into the exponent's FMA,
      // one register flow for full and partial tiles.
      float mb = kNegInf;
      if (cls == TILE_PARTIAL) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = k0 + 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
            st[t][r] = (j < Skv && mask_ok<MASK>(qi, j, window, 0, 0)) ? st[t][r] : kNegInf;
          }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mb = fmaxf(mb, st[t][r]);
      mb = half_swap_max(mb * a.scale_log2);
      const float m_new = fmaxf(m, mb);
      const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
      const float alpha = fast_exp2(m - m_use);
      const float mult = a.scale_log2;
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
      // ---- P to E4M3: byte p of the B operand is key kappa(hh, p) =
      // 32 (p / 16) + 8 ((p % 16) / 4) + 4 hh + p % 4, i.e. st[p / 16][p % 16].
      i32x8 pb;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int t = w >> 2, r0 = 4 * (w & 3);
        // The first conversion writes the low half-word and the second the
        // high one, so the first's other half may start as anything: a
        // register an empty asm statement claims to define, rather than a
        // zero moved into place.
        int any;
        asm volatile("" : "=v"(any));
        const int lo = pack_fp8<false>(st[t][r0], st[t][r0 + 1], any);
        pb[w] = pack_fp8<true>(st[t][r0 + 2], st[t][r0 + 3], lo);
      }
      // ---- O^T += V^T P^T
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] = mfma_fp8(vf[dt], pb, acc[dt], svb, 127);
    }
    wait_loads();
    __syncthreads();
  };

  if (n_steps > 0) {
    issue(0, sK0, sV0);
    wait_loads();
  }
  __syncthreads();
  for (int s = 0; s < n_steps; s += 2) {
    step(s, sK0, sV0, sK1, sV1);
    if (s + 1 < n_steps) step(s + 1, sK1, sV1, sK0, sV0);
  }

  const float lt = half_swap_sum(l - lc);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (row_ok) {
    uint16_t* Orow = (uint16_t*)a.o + ((size_t)(b * a.Hq + hq) * Sq + qi) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = 32 * dt + 8 * rq + 4 * hh;
        *(u32x2*)(Orow + d0) = u32x2{pack_bf16(acc[dt][4 * rq] * inv, acc[dt][4 * rq + 1] * inv),
                                     pack_bf16(acc[dt][4 * rq + 2] * inv, acc[dt][4 * rq + 3] * inv)};
      }
    if (a.lse != nullptr && hh == 0)
      a.lse[(size_t)(b * a.Hq + hq) * Sq + qi] = lt > 0.0f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : kNegInf;
  }
}

template <int D>
static hipError_t launch_fp8_fwd_d(const Fp8FwdArgs& a, int mask, hipStream_t st) {
  const dim3 grid((unsigned)(a.B * a.Hq * a.n_qt)), block(256);
  switch (mask) {
    case MASK_NONE: hipLaunchKernelGGL((fwd_fp8_kernel<D, MASK_NONE>), grid, block, 0, st, a); break;
    case MASK_CAUSAL: hipLaunchKernelGGL((fwd_fp8_kernel<D, MASK_CAUSAL>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((fwd_fp8_kernel<D, MASK_WINDOW>), grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_fp8_fwd(const Fp8FwdArgs& a, int mask, hipStream_t st) {
  return a.D == 128 ? launch_fp8_fwd_d<128>(a, mask, st) : launch_fp8_fwd_d<64>(a, mask, st);
}

hipError_t launch_fp8_quantize(const void* x, void* x8, uint8_t* scales, int rows, int S, int D, const float* signs,
                               hipStream_t st) {
  const int nblk = (S + 127) / 128;
  const dim3 grid((unsigned)nblk, (unsigned)rows), block(128);
  if (D == 128)
    hipLaunchKernelGGL((fp8_quantize_kernel<128>), grid, block, 0, st, (const uint16_t*)x, (uint8_t*)x8, scales, S,
                       nblk, signs);
  else
    hipLaunchKernelGGL((fp8_quantize_kernel<64>), grid, block, 0, st, (const uint16_t*)x, (uint8_t*)x8, scales, S,
                       nblk, signs);
  return hipGetLastError();
}

}  // namespace miattn
