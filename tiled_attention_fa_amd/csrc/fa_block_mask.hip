// Block-mask construction ("PyTorch FlexAttention, FlashAttention-4" page,
// 섹션별 상세: block-sparse iteration lets the kernel skip blocks that the
// mask empties; blocks are 128 x 128).
//
// Tile (qt, kt) covers queries [128 qt, 128 qt + 128) and keys
// [128 kt, 128 kt + 128).  EMPTY: no in-range pair is admissible.  FULL:
// every pair is in range and admissible.  PARTIAL: otherwise.
//
// Kernel 1: one workgroup per (batch row, query tile); each thread
// classifies one key tile per pass of 256 tiles.  Analytic masks are
// classified in closed form.  Document tiles are first decided from the id
// range of each 128-token block: disjoint ranges -> EMPTY; both blocks
// holding one and the same id -> the causal class of the tile.  The tiles
// that remain (blocks straddling a document boundary) are checked pair by
// pair, one tile per wave.  A workgroup prefix sum
// writes the non-empty tiles in ascending order.
// Kernel 2: one workgroup per (batch row, key tile), one thread per query
// tile; a prefix sum writes the ascending list of non-empty query tiles.
// Kernel 3 (when the caller asks for them): the schedule orders (longest
// first, tiles of one document together).
#include "fa_device.h"
#include "fa_launch.h"

namespace miattn {

// Minimum and maximum of doc[i0 .. i0 + n) (0 <= n <= 128) over the 32
// lanes of a half wave: coalesced loads, then a butterfly over the half.
// Every load is issued (index clamped into doc[0 .. len)) and the range
// test is a select, so the loads stay in flight together.
__device__ __forceinline__ void id_range32(const int32_t* doc, int len, int i0, int n, int l32, int& lo, int& hi) {
  int d[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) d[e] = doc[min(max(i0 + e * 32 + l32, 0), len - 1)];
  lo = 0x7fffffff;
  hi = -0x7fffffff - 1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bool in = e * 32 + l32 < n;
    lo = in ? min(lo, d[e]) : lo;
    hi = in ? max(hi, d[e]) : hi;
  }
#pragma unroll
  for (int w = 16; w >= 1; w >>= 1) {
    lo = min(lo, __shfl_xor(lo, w, 32));
    hi = max(hi, __shfl_xor(hi, w, 32));
  }
}

// Exclusive prefix sum of `flag` over the 256 threads; returns this thread's
// offset and stores the total in `total`.
__device__ __forceinline__ int block_scan(bool flag, int* s_wave, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t bal = __builtin_amdgcn_ballot_w64(flag);
  const int below = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
  __syncthreads();  // s_wave free from the previous pass
  if (lane == 0) s_wave[wave] = __builtin_popcountll(bal);
  __syncthreads();
  int off = 0;
  total = 0;
  for (int w = 0; w < 4; ++w) {
    off += w < wave ? s_wave[w] : 0;
    total += s_wave[w];
  }
  return off + below;
}

__global__ __launch_bounds__(256) void block_mask_rows_kernel(int mask_kind, int window, const int32_t* doc_ids,
                                                              int Sq, int Skv, BlockMaskArgs m) {
  const int qt = blockIdx.x, bb = blockIdx.y;
  const int tid = threadIdx.x;
  const int q0 = qt * kMaskBlock;
  const int nq = min(kMaskBlock, Sq - q0);
  const int q_last = q0 + nq - 1;
  __shared__ int srow[kMaskBlock];
  __shared__ __attribute__((aligned(16))) int scol[4 * kMaskBlock];  // key ids of the tile each wave checks
  __shared__ int s_nbf, s_wave[4];
  __shared__ int s_bf[256];       // tiles of this pass that need the pair check (thread index)
  __shared__ uint8_t s_st[256];   // their resolved state
  __shared__ int s_lo[256], s_hi[256];  // id range of each key block of this pass
  const int32_t* doc = mask_kind == MASK_DOCUMENT ? doc_ids + (size_t)bb * Skv : nullptr;
  const int lane = tid & 63, half = (tid >> 5) & 1, wave = tid >> 6;
  int qlo = 0, qhi = 0;
  if (doc) {
    if (tid < kMaskBlock) {
      const int d = doc[min(q0 + tid, Skv - 1)];
      srow[tid] = q0 + tid < Sq ? d : -1;
    }
    id_range32(doc, Skv, q0, nq, lane & 31, qlo, qhi);  // every half wave computes the same range
  }
  const bool quni = qlo == qhi;

  uint8_t* state = m.tile_state + ((size_t)bb * m.n_q + qt) * m.n_kv;
  int32_t* list = m.kv_index + ((size_t)bb * m.n_q + qt) * m.n_kv;
  int count = 0;
  for (int kt0 = 0; kt0 < m.n_kv; kt0 += 256) {
    const int kt = kt0 + tid;
    int st = TILE_EMPTY;
    bool need_pairs = false;
    if (doc) {
      // id ranges of this pass's key blocks: half wave h of wave w takes
      // blocks 2w + h, 2w + h + 8, ...
      for (int blk0 = 2 * wave + half; blk0 < 256 && kt0 + blk0 < m.n_kv; blk0 += 32) {
        int lo[4], hi[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {  // four blocks' loads in flight together
          const int blk = blk0 + 8 * u;
          const int k0 = (kt0 + blk) * kMaskBlock;
          const int n = (blk < 256 && kt0 + blk < m.n_kv) ? min(kMaskBlock, Skv - k0) : 0;
          id_range32(doc, Skv, k0, n, lane & 31, lo[u], hi[u]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int blk = blk0 + 8 * u;
          if ((lane & 31) == 0 && blk < 256 && kt0 + blk < m.n_kv) {
            s_lo[blk] = lo[u];
            s_hi[blk] = hi[u];
          }
        }
      }
      __syncthreads();
    }
    if (kt < m.n_kv) {
      const int k0 = kt * kMaskBlock;
      const int nk = min(kMaskBlock, Skv - k0);
      const bool full_extent = nq == kMaskBlock && nk == kMaskBlock;
      switch (mask_kind) {
        case MASK_NONE: st = full_extent ? TILE_FULL : TILE_PARTIAL; break;
        case MASK_CAUSAL: {
          const int c = block_class<MASK_CAUSAL>(q0, nq, k0, nk, Skv, window);
          st = (c == TILE_FULL && !full_extent) ? TILE_PARTIAL : c;
          break;
        }
        case MASK_WINDOW: {
          const int c = block_class<MASK_WINDOW>(q0, nq, k0, nk, Skv, window);
          st = (c == TILE_FULL && !full_extent) ? TILE_PARTIAL : c;
          break;
        }
        default: {
          if (k0 > q_last) break;  // causal part empties the tile
          const int klo = s_lo[tid], khi = s_hi[tid];
          if (khi < qlo || klo > qhi) break;  // no shared document id
          if (quni && klo == khi) {           // one id on both sides, the same one
            st = (k0 + nk - 1 <= q0 && full_extent) ? TILE_FULL : TILE_PARTIAL;
            break;
          }
          need_pairs = true;
          break;
        }
      }
    }
    // Pair check of the undecided tiles: each wave takes one tile at a time
    // (lane l: query rows l and l + 64 against the tile's 128 key ids).
    if (doc) {
      if (tid == 0) s_nbf = 0;
      __syncthreads();
      if (need_pairs) s_bf[atomicAdd(&s_nbf, 1)] = tid;
      __syncthreads();
      const int nbf = s_nbf;
      for (int u = wave; u < nbf; u += 4) {
        const int k0 = (kt0 + s_bf[u]) * kMaskBlock;
        const int nk = min(kMaskBlock, Skv - k0);
        const int c0 = doc[min(k0 + lane, Skv - 1)], c1 = doc[min(k0 + 64 + lane, Skv - 1)];
        scol[wave * kMaskBlock + lane] = lane < nk ? c0 : -2;
        scol[wave * kMaskBlock + 64 + lane] = 64 + lane < nk ? c1 : -2;
        __builtin_amdgcn_wave_barrier();
        // A tile that gets here has two different ids in one of its blocks,
        // so it cannot be FULL: find one admissible pair (key c of the tile
        // is admissible for row i iff c <= min(nk - 1, i - k0) and the ids
        // agree), stopping at the first.
        const int i0 = q0 + lane, i1 = i0 + 64;
        const int d0 = srow[lane], d1 = srow[lane + 64];
        const int cmax0 = i0 < Sq ? min(nk - 1, i0 - k0) : -1;
        const int cmax1 = i1 < Sq ? min(nk - 1, i1 - k0) : -1;
        bool any = false;
        for (int c = 0; c < kMaskBlock; c += 8) {
          typedef int i32x4 __attribute__((ext_vector_type(4)));
          const i32x4 ka = *(const i32x4*)&scol[wave * kMaskBlock + c];  // same address on every lane
          const i32x4 kb = *(const i32x4*)&scol[wave * kMaskBlock + c + 4];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int kid = e < 4 ? ka[e] : kb[e - 4];
            any |= (c + e <= cmax0 && d0 == kid) | (c + e <= cmax1 && d1 == kid);
          }
          if (__builtin_amdgcn_ballot_w64(any) != 0) break;
        }
        const bool w_any = __builtin_amdgcn_ballot_w64(any) != 0;
        if (lane == 0) s_st[s_bf[u]] = (uint8_t)(w_any ? TILE_PARTIAL : TILE_EMPTY);
        __builtin_amdgcn_wave_barrier();  // this wave's scol slice is free again
      }
      __syncthreads();
      if (need_pairs) st = s_st[tid];
    }
    if (kt < m.n_kv) state[kt] = (uint8_t)st;
    int total;
    const int pos = block_scan(st != TILE_EMPTY, s_wave, total);
    if (st != TILE_EMPTY) list[count + pos] = kt;
    count += total;
  }
  for (int kt = count + tid; kt < m.n_kv; kt += 256) list[kt] = -1;
  if (tid == 0) m.kv_count[bb * m.n_q + qt] = count;
}

__global__ __launch_bounds__(256) void block_mask_cols_kernel(BlockMaskArgs m) {
  const int kt = blockIdx.x, bb = blockIdx.y, tid = threadIdx.x;
  __shared__ int s_wave[4];
  const uint8_t* state = m.tile_state + (size_t)bb * m.n_q * m.n_kv + kt;
  int32_t* list = m.q_index + ((size_t)bb * m.n_kv + kt) * m.n_q;
  int count = 0;
  for (int qt0 = 0; qt0 < m.n_q; qt0 += 256) {
    const int qt = qt0 + tid;
    const bool ne = qt < m.n_q && state[(size_t)qt * m.n_kv] != TILE_EMPTY;
    int total;
    const int pos = block_scan(ne, s_wave, total);
    if (ne) list[count + pos] = qt;
    count += total;
  }
  for (int qt = count + tid; qt < m.n_q; qt += 256) list[qt] = -1;
  if (tid == 0) m.q_count[bb * m.n_kv + kt] = count;
}

// Kernel 3: for each batch row, the q tiles (grid y = 0) and the kv tiles
// (y = 1) in a schedule order: longest list first, ties by index.  Under a
// document mask (`group`), tiles whose lists share their first kv tile (q
// tiles) or their last q tile (kv tiles), i.e. the tiles of one document,
// which stream the same key (or query) rows, are kept together: groups go
// heaviest first (weight: the longest list in the group), ties by ascending
// group key, and inside a group longest first, ties by index.  Workgroups
// that run together then share their rows in L2, while the longest work
// still starts first.  Item t goes to position #{u : key(u) < key(t)} for
// the strict total order key = (-weight, group, -count, index) (without
// `group`, every tile is its own group of weight = count): a permutation,
// so every position is written exactly once.
// Rows of more tiles than this (sequences over 256K tokens) get the identity
// order: the quadratic ranking below would cost more than it balances.
constexpr int kOrderMax = 2048;

__global__ __launch_bounds__(256) void block_mask_order_kernel(BlockMaskArgs m, int group) {
  const int bb = blockIdx.x, which = blockIdx.y;
  const int n = which == 0 ? m.n_q : m.n_kv;      // tiles to order
  const int len = which == 0 ? m.n_kv : m.n_q;    // list capacity of each tile
  const int32_t* c = which == 0 ? m.kv_count + (size_t)bb * m.n_q : m.q_count + (size_t)bb * m.n_kv;
  const int32_t* lists = which == 0 ? m.kv_index + (size_t)bb * m.n_q * m.n_kv : m.q_index + (size_t)bb * m.n_kv * m.n_q;
  int32_t* order = which == 0 ? m.q_order : m.kv_order;
  if (order == nullptr) return;
  order += (size_t)bb * n;
  if (n > kOrderMax) {
    for (int t = threadIdx.x; t < n; t += 256) order[t] = t;
    return;
  }
  // Group keys lie in [0, len] (len: empty lists); a document mask has
  // len == n.  Longer lists (never under a document mask) are not grouped.
  const bool grouped = group && len <= kOrderMax;
  __shared__ int sw[kOrderMax + 1];                  // group weights by group key
  __shared__ unsigned long long skey[kOrderMax];     // the packed sort keys
  for (int g = threadIdx.x; g <= kOrderMax; g += 256) sw[g] = 0;
  __syncthreads();
  // (65535 - weight, group, 65535 - count, index) packs into 16-bit fields
  // of one 64-bit key (counts clamped to 65535: past 8M keys the order of
  // such tiles among themselves is by index; the unique index field keeps
  // the ranking a permutation).
  int ct_[kOrderMax / 256], gt_[kOrderMax / 256];
#pragma unroll
  for (int i = 0; i < kOrderMax / 256; ++i) {
    const int t = threadIdx.x + 256 * i;
    if (t < n) {
      const int ct = min(max(c[t], 0), len);
      const int gt = !grouped ? t : ct == 0 ? len : min(max(lists[(size_t)t * len + (which == 0 ? 0 : ct - 1)], 0), len);
      ct_[i] = ct;
      gt_[i] = gt;
      if (grouped) atomicMax(&sw[gt], ct);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kOrderMax / 256; ++i) {
    const int t = threadIdx.x + 256 * i;
    if (t < n) {
      const int w = min(grouped ? sw[gt_[i]] : ct_[i], 65535), ct = min(ct_[i], 65535);
      skey[t] = (unsigned long long)(65535 - w) << 48 | (unsigned long long)gt_[i] << 32 |
                (unsigned long long)(65535 - ct) << 16 | (unsigned long long)t;
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < n; t += 256) {
    const unsigned long long kt = skey[t];
    int pos = 0;
    for (int u = 0; u < n; ++u) pos += skey[u] < kt;
    order[pos] = t;
  }
}

hipError_t launch_block_mask(int mask_kind, int window, const int32_t* doc_ids, int Sq, int Skv,
                             const BlockMaskArgs& m, hipStream_t st) {
  if (m.n_q > 0) {
    hipLaunchKernelGGL(block_mask_rows_kernel, dim3((unsigned)m.n_q, (unsigned)m.n_b), dim3(256), 0, st, mask_kind,
                       window, doc_ids, Sq, Skv, m);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (m.n_kv > 0) {
    hipLaunchKernelGGL(block_mask_cols_kernel, dim3((unsigned)m.n_kv, (unsigned)m.n_b), dim3(256), 0, st, m);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((m.q_order != nullptr || m.kv_order != nullptr) && (m.n_q > 0 || m.n_kv > 0)) {
    hipLaunchKernelGGL(block_mask_order_kernel, dim3((unsigned)m.n_b, 2u), dim3(256), 0, st, m,
                       mask_kind == MASK_DOCUMENT ? 1 : 0);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace miattn
