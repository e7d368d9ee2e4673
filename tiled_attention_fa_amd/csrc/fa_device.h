// Device helpers for the gfx950 attention kernels: MFMA wrappers, exp2,
// bf16 packing, cross-half wave reductions, LDS swizzles, masks, score
// modifiers and the workgroup-to-tile schedule.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/libmiattn.h"
#include "fa_args.h"

namespace miattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------- MFMA
// 32x32x16 bf16 -> fp32.  Lane l supplies A[l%32][k-slot l/32] and
// B[k-slot l/32][l%32] (8 bf16 each); the accumulator register r of lane l
// holds C[8(r/4) + 4(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
// 32x32x2 fp32: one value per lane, same accumulator layout.
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// The value of the first active lane, held in a scalar register: tells the
// compiler that a per-wave quantity (e.g. the wave index) is uniform.  Kept
// in a device function so kernel bodies name no target builtin directly.
__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// x, hidden from the optimizer (an empty asm that claims to modify it):
// values derived from it are recomputed where they are used, inside the loop
// that calls this, instead of being hoisted out of the loop, each into a
// register of its own.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Combine a value with the one in lane l ^ 32 (v_permlane32_swap).
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Transposing LDS read: within each 16-lane group, lane i receives element
// i%4 of the 8-byte chunk addressed by lane 4j + i/4, for j = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* lds_byte_ptr) {
  typedef __attribute__((address_space(3))) bf16x4_t lds_v4;
  const __attribute__((address_space(3))) char* p =
      (const __attribute__((address_space(3))) char*)(lds_byte_ptr);
  bf16x4_t t = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)p);
  return __builtin_bit_cast(u32x2, t);
}

// ---------------------------------------------------------------- LDS swizzle
// A row of D bf16 values is D/8 chunks of 16 bytes; chunk c of row r is
// stored at chunk c ^ f(r).  Two read patterns must be bank-conflict free:
//  * row reads (MFMA operand rows): 16 lanes read the same chunk of 16
//    consecutive rows -> f must be a bijection on those rows;
//  * transposing reads (lds_read_tr16): 32 lanes read 4 consecutive chunks
//    (64 bytes) of 4 consecutive rows -> the four rows must land their
//    64-byte groups in different quarters of the 256-byte bank window.
// D = 128 (256-byte rows): f(r) swaps the two low 2-bit fields of r.
// D = 64 (128-byte rows, two rows per window): f(r) = bit 1 of r moved to
// bit 2, bits 2..3 of r in bits 0..1.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (D == 128) return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
  return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Byte offset of chunk 0 of swizzled row r.  Because the swizzle is an XOR
// on the chunk index, and chunk bits (4 .. log2(ROW) - 1) never carry into
// the row bits, chunk c of row r sits at row_base(r) ^ (16 c).
template <int D>
__device__ __forceinline__ int row_base(int r) {
  return r * (2 * D) + swz<D>(r, 0) * 16;
}

// ---------------------------------------------------------------- global -> LDS
// Buffer resource over `bytes` bytes at `base` (raw buffer, no stride): loads
// at offsets >= bytes return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Buffer resource over rows [r0, n_rows) of a row-major matrix with
// `row_bytes` bytes per row: offset 0 is the start of row r0, and offsets at
// or past row n_rows read as zeros.  r0 is wave-uniform, so the resource is
// built with scalar instructions and per-lane offsets stay loop-invariant.
// `base` must be held in scalar registers (see uniform_ptr).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int n_rows, int r0, int row_bytes) {
  r0 = __builtin_amdgcn_readfirstlane(r0);
  const int left = n_rows > r0 ? n_rows - r0 : 0;
  return make_rsrc((const char*)base + (size_t)r0 * (size_t)row_bytes, (uint32_t)left * (uint32_t)row_bytes);
}

// A wave-uniform pointer moved to scalar registers.  Pointers derived from
// values the compiler computes in vector registers (e.g. a head index from
// an integer division) would otherwise make it wrap each buffer load in a
// per-lane loop; apply once, outside the loops.
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (const T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// ROWS rows of a bf16 [rows][D] matrix into an LDS tile in the swizzled
// layout, straight from memory to LDS (buffer_load ... lds, no registers).
// Each load instruction fills 1 KB of the tile, lane l writing bytes
// 16 l .. 16 l + 15, so lane l fetches the global chunk that the swizzle
// places there.  The rows come from a rows_rsrc resource, so the per-lane
// offsets depend only on the wave and the lane and stay loop-invariant.
// All NW waves of the workgroup take part, each issuing PER_WAVE loads;
// `wave` must be wave-uniform (wave_uniform).
template <int D, int ROWS, int NW = 4>
__device__ __forceinline__ void tile_load(__amdgpu_buffer_rsrc_t rsrc, char* tile, int wave, int lane) {
  constexpr int ROW = D * 2, PER_WAVE = ROWS * ROW / 1024 / NW;
  static_assert(PER_WAVE * NW * 1024 == ROWS * ROW, "tile must split into 1 KB loads over the waves");
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int byte = (wave * PER_WAVE + i) * 1024 + lane * 16;
    const int r = byte / ROW, p = (byte % ROW) / 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void*)(tile + (wave * PER_WAVE + i) * 1024), 16,
        (uint32_t)(r * ROW + swz<D>(r, p) * 16), 0, 0, 0);
  }
}

// 64 int32 values src[i0 .. i0 + 63] (zeros at or past index n) into LDS by
// one wave.
__device__ __forceinline__ void ints_to_lds(const void* src, int n, int i0, int* dst, int lane) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rows_rsrc(src, n, i0, 4), (__attribute__((address_space(3))) void*)dst, 4,
                                            (uint32_t)(lane * 4), 0, 0, 0);
}

// Chunk c (64 floats) of a slice table[i0 .. ) of a relative-position bias
// table into dst[64 c .. 64 c + 63], by one wave, straight to LDS.  Entries
// outside [0, len) read as zero: i0 may be negative (the slice of a key tile
// that runs past the last key), and such lanes get an offset past the end of
// the resource.  i0 is wave-uniform; `table` must be in scalar registers.
__device__ __forceinline__ void bias_chunk_to_lds(const float* table, int len, int i0, float* dst, int c, int lane) {
  const int base = i0 > 0 ? i0 : 0;
  const int idx = i0 + 64 * c + lane;
  const uint32_t off = idx >= base ? (uint32_t)(idx - base) * 4u : 0x7ffffff0u;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rows_rsrc(table, len, base, 4),
                                            (__attribute__((address_space(3))) void*)(dst + 64 * c), 4, off, 0, 0, 0);
}

// Wait until every load this wave issued has landed (vmcnt = 0).
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0); }

// Wait until every vector memory operation of this wave but the two most
// recent (vmcnt(2); they complete in issue order) has completed, and every
// LDS access: the stage loads issued earlier in a step have landed while the
// step's two trailing stores may still be in flight.
__device__ __forceinline__ void wait_loads_not_last2() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0072);  // vmcnt 2, expcnt 7 (no wait), lgkmcnt 0
  asm volatile("" ::: "memory");
}

// Workgroup barrier without a memory fence: unlike __syncthreads it does not
// wait for this wave's loads in flight into other LDS buffers.  The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void phase_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------- masks
// Admissibility of (query i, key j), absolute indices.  `doc_i` / `doc_j`
// are the document ids (only read for MASK_DOCUMENT).
template <int MASK>
__device__ __forceinline__ bool mask_ok(int i, int j, int window, int doc_i, int doc_j) {
  if constexpr (MASK == MASK_NONE) return true;
  if constexpr (MASK == MASK_CAUSAL) return j <= i;
  if constexpr (MASK == MASK_WINDOW) return j <= i && i - j < window;
  return j <= i && doc_i == doc_j;
}

// Key range [lo, hi) that can be admissible for query rows [q0, q1).
template <int MASK>
__device__ __forceinline__ void key_range(int q0, int q1, int Skv, int window, int& lo, int& hi) {
  lo = 0;
  hi = Skv;
  if constexpr (MASK != MASK_NONE) hi = min(Skv, q1);
  if constexpr (MASK == MASK_WINDOW) lo = max(0, q0 - window + 1);
}

// Class of the block [q0, q0+nq) x [k0, k0+nk) under an analytic mask:
// TILE_EMPTY, TILE_PARTIAL or TILE_FULL (every pair in range and admissible).
template <int MASK>
__device__ __forceinline__ int block_class(int q0, int nq, int k0, int nk, int Skv, int window) {
  const int q1 = q0 + nq - 1, k1 = k0 + nk - 1;
  const bool in_range = k0 + nk <= Skv;
  if constexpr (MASK == MASK_NONE) return in_range ? TILE_FULL : TILE_PARTIAL;
  if (k0 > q1) return TILE_EMPTY;
  if constexpr (MASK == MASK_WINDOW) {
    if (k1 < q0 - window + 1) return TILE_EMPTY;
    return (in_range && k1 <= q0 && q1 - k0 < window) ? TILE_FULL : TILE_PARTIAL;
  }
  if constexpr (MASK == MASK_CAUSAL) return (in_range && k1 <= q0) ? TILE_FULL : TILE_PARTIAL;
  return TILE_PARTIAL;
}

// ---------------------------------------------------------------- score modifiers
template <int MOD>
__device__ __forceinline__ float head_slope(const ModArgs& m, int h, int Hq) {
  if constexpr (MOD == MOD_ALIBI) {
    if (m.slopes) return m.slopes[h];
    return fast_exp2(-8.0f * (float)(h + 1) / (float)Hq);
  }
  return 0.0f;
}

// ---------------------------------------------------------------- schedule
// Workgroups are handed to the 8 XCDs round-robin by id.  When the number
// of (batch, kv-head) units is a multiple of 8, every unit is pinned to one
// XCD so its K/V stream stays in that XCD's L2, and within an XCD the tile
// rank advances slowest so the heaviest tiles (largest index under causal
// masks) start first.  Returns the batch, query head and tile index.
__device__ __forceinline__ void decode_work(int P, int B, int Hq, int Hkv, int n_tiles,
                                            bool heavy_first, int& b, int& hq, int& tile) {
  const int G = Hq / Hkv;
  const int NU = B * Hkv;
  int r;
  if ((NU & 7) == 0) {
    const int xcd = P & 7, s = P >> 3;
    const int per_rank = (NU >> 3) * G;
    r = s / per_rank;
    const int rem = s - r * per_rank;
    const int ul = rem / G, g = rem - ul * G;
    const int u = ul * 8 + xcd;
    b = u / Hkv;
    hq = (u - b * Hkv) * G + g;
  } else {
    const int heads = B * Hq;
    r = P / heads;
    const int hh = P - r * heads;
    b = hh / Hq;
    hq = hh - b * Hq;
  }
  tile = heavy_first ? (n_tiles - 1 - r) : r;
}

// ---------------------------------------------------------------- workgroup trace
// Debug records of fa_mask_params.wg_trace (kernels of the static schedule):
// the constant-rate clock at a tile's start (read into scalar registers
// when the tile starts) and end, where it ran (the XCC_ID and HW_ID
// hardware registers, read with s_getreg: id 20 and id 4, all 32 bits) and
// its size, all four words written at the end by lane 0 of the workgroup's
// first wave (`first`: a wave-uniform test, so no thread index stays live
// through the tile).  Plain vector stores; nothing when `tr` is null or
// P < 0.
__device__ __forceinline__ uint64_t trace_clock(const int64_t* tr) {
  return tr != nullptr ? __builtin_amdgcn_s_memrealtime() : 0;
}

__device__ __forceinline__ void trace_end(int64_t* tr, int P, uint64_t t0, bool first, int rows, int steps) {
  if (tr == nullptr || P < 0 || !first) return;
  const unsigned lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  if (lane == 0) {
    int64_t* e = tr + (size_t)P * FA_WG_TRACE_WORDS;
    const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
    const uint32_t xcc = (uint32_t)__builtin_amdgcn_s_getreg((31 << 11) | 20);
    const uint32_t hw = (uint32_t)__builtin_amdgcn_s_getreg((31 << 11) | 4);
    e[0] = (int64_t)t0;
    e[1] = (int64_t)t1;
    e[2] = (int64_t)(((uint64_t)xcc << 32) | hw);
    e[3] = (int64_t)(((uint64_t)(uint32_t)rows << 32) | (uint32_t)steps);
  }
}

// ---------------------------------------------------------------- work queue
// Persistent kernels take the static schedule's workgroup indices P from a
// queue of counters in caller memory (int32[kQueueInts], zero at launch).
// When the (batch, kv-head) units pin to XCDs (decode_work), there is one
// counter per XCD over P = 8 i + x; otherwise one counter over P = i.  A last
// counter counts finished workgroups; the last to finish zeroes them all.
// Each counter has a 128-byte line of its own.
constexpr int kXcds = 8;
constexpr int kQueueStride = 32;                   // ints per counter
constexpr int kQueueInts = (kXcds + 1) * kQueueStride;
constexpr int kQueueDone = kXcds * kQueueStride;   // the finished-workgroup count

static_assert(kQueueInts == FA_WORK_QUEUE_INTS, "the header states the queue length");

struct WorkQueue {
  int n_queues;   // 8 (XCD-pinned) or 1
  int per_queue;  // workgroup indices per counter
};

__device__ __forceinline__ WorkQueue work_queue_shape(int B, int Hq, int Hkv, int n_tiles) {
  const int NU = B * Hkv;
  if ((NU & 7) == 0) return WorkQueue{kXcds, (NU >> 3) * (Hq / Hkv) * n_tiles};
  return WorkQueue{1, B * Hq * n_tiles};
}

__device__ __forceinline__ int queue_home(const WorkQueue& wq, int home) { return wq.n_queues == 1 ? 0 : home; }

// Raw index from the workgroup's own counter (one device-scope atomic; the
// caller may issue it early and consume the result later).
__device__ __forceinline__ int take_home(int32_t* q, const WorkQueue& wq, int home) {
  return __hip_atomic_fetch_add(q + queue_home(wq, home) * kQueueStride, 1, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
}

// The workgroup's next index P, or -1 once every counter is past its end.
// Thread 0 decides: `i_home` is an index already taken from the own counter
// (or -1 if none was taken); when it is past the end, the other counters are
// tried in turn.  The workgroup reads the result through `slot`.  Counters
// only grow, so every workgroup ends.
__device__ __forceinline__ int finish_pull(int32_t* q, const WorkQueue& wq, int home, int i_home, int* slot) {
  if (threadIdx.x == 0) {
    int P = -1;
    if (i_home < 0) i_home = take_home(q, wq, home);
    if (i_home < wq.per_queue) {
      P = i_home * wq.n_queues + queue_home(wq, home);
    } else {
      for (int k = 1; k < wq.n_queues; ++k) {
        int32_t* c = q + ((home + k) & (kXcds - 1)) * kQueueStride;
        if (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= wq.per_queue) continue;
        const int i = __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (i < wq.per_queue) {
          P = i * wq.n_queues + ((home + k) & (kXcds - 1));
          break;
        }
      }
    }
    *slot = P;
  }
  __syncthreads();
  const int P = *slot;
  __syncthreads();  // the slot is rewritten by the next pull
  return P;
}

// End of a persistent workgroup: count it as finished; the last one zeroes
// the queue (every other workgroup has made its last pull by then), so the
// next launch, or a graph replay, starts from zero without a clearing pass.
__device__ __forceinline__ void release_queue(int32_t* q) {
  if (threadIdx.x == 0) {
    const int done = __hip_atomic_fetch_add(q + kQueueDone, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (done == (int)gridDim.x - 1) {
      for (int x = 0; x <= kXcds; ++x)
        __hip_atomic_store(q + x * kQueueStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Running row sum with compensation (Kahan): l is the sum, c the negated
// low-order part lost so far, so the sum is l - c.  After every key step,
// l <- alpha l + ps with ps the step's sum.  Over 10^5 steps of nearly equal
// step sums (millions of keys with one score) a plain fp32 sum drifts by up
// to ~1e-3 relative; the compensated one stays at rounding level.
__device__ __forceinline__ void row_sum_update(float& l, float& c, float alpha, float ps) {
  const float ls = l * alpha;
  c *= alpha;
  const float y = ps - c;
  const float t = ls + y;
  c = (t - ls) - y;
  l = t;
}

// Tile at position r of a block mask's schedule order, or `fallback`
// when the mask carries no order.  The entry is clamped into [0, n).
__device__ __forceinline__ int ordered_tile(const int32_t* order, int n_b, int b, int n, int r, int fallback) {
  if (order == nullptr) return fallback;
  const int v = order[(size_t)(n_b == 1 ? 0 : b) * n + r];
  return min(max(v, 0), n - 1);
}

}  // namespace miattn
