// Block-mask construction ("PyTorch FlexAttention, FlashAttention-4" page,
// 섹션별 상세: block-sparse iteration lets the kernel skip blocks that the
// mask empties; blocks are 128 x 128).
//
// Tile (qt, kt) covers queries [128 qt, 128 qt + 128) and keys
// [128 kt, 128 kt + 128).  EMPTY: no in-range pair is admissible.  FULL:
// every pair is in range and admissible.  PARTIAL: otherwise.
//
// Kernel 1: one workgroup per (batch row, query tile).  Analytic masks are
// classified in closed form; document masks by checking all pairs of the
// tile (256 threads, 64 pairs each) with a workgroup-wide any/all, skipping
// tiles the causal part already empties.  The workgroup walks the key tiles
// in order, so its list of non-empty tiles is ascending.
// Kernel 2: one thread per (batch row, key tile) scans the states of its
// column and writes the ascending list of non-empty query tiles.
#include "fa_device.h"
#include "fa_launch.h"

namespace miattn {

__global__ __launch_bounds__(256) void block_mask_rows_kernel(int mask_kind, int window, const int32_t* doc_ids,
                                                              int Sq, int Skv, BlockMaskArgs m) {
  const int qt = blockIdx.x, bb = blockIdx.y;
  const int tid = threadIdx.x;
  const int q0 = qt * kMaskBlock;
  __shared__ int srow[kMaskBlock];
  __shared__ int scol[kMaskBlock];
  __shared__ int s_any, s_all;
  const int32_t* doc = mask_kind == MASK_DOCUMENT ? doc_ids + (size_t)bb * Skv : nullptr;
  if (doc && tid < kMaskBlock) srow[tid] = (q0 + tid < Sq) ? doc[q0 + tid] : -1;

  uint8_t* state = m.tile_state + ((size_t)bb * m.n_q + qt) * m.n_kv;
  int32_t* list = m.kv_index + ((size_t)bb * m.n_q + qt) * m.n_kv;
  const int nq = min(kMaskBlock, Sq - q0);
  int count = 0;
  for (int kt = 0; kt < m.n_kv; ++kt) {
    const int k0 = kt * kMaskBlock;
    const int nk = min(kMaskBlock, Skv - k0);
    const bool full_extent = nq == kMaskBlock && nk == kMaskBlock;
    int st;
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
        if (k0 > q0 + nq - 1) {
          st = TILE_EMPTY;
          break;
        }
        __syncthreads();  // previous tile's readers of scol / s_any are done
        if (tid < kMaskBlock) scol[tid] = (k0 + tid < Skv) ? doc[k0 + tid] : -2;
        if (tid == 0) {
          s_any = 0;
          s_all = 1;
        }
        __syncthreads();
        const int r = tid & (kMaskBlock - 1), c0 = (tid >> 7) * 64;
        const int i = q0 + r;
        int any = 0, all = 1;
        for (int c = c0; c < c0 + 64; ++c) {
          const int j = k0 + c;
          const bool ok = i < Sq && j < Skv && j <= i && srow[r] == scol[c];
          any |= ok;
          all &= ok;
        }
        if (any) s_any = 1;
        if (!all) s_all = 0;
        __syncthreads();
        st = s_any ? (s_all && full_extent ? TILE_FULL : TILE_PARTIAL) : TILE_EMPTY;
        break;
      }
    }
    if (tid == 0) {
      state[kt] = (uint8_t)st;
      if (st != TILE_EMPTY) list[count] = kt;
    }
    count += st != TILE_EMPTY;
  }
  for (int kt = count + tid; kt < m.n_kv; kt += 256) list[kt] = -1;
  if (tid == 0) m.kv_count[bb * m.n_q + qt] = count;
}

__global__ __launch_bounds__(256) void block_mask_cols_kernel(BlockMaskArgs m) {
  const int id = blockIdx.x * 256 + threadIdx.x;
  if (id >= m.n_b * m.n_kv) return;
  const int bb = id / m.n_kv, kt = id - bb * m.n_kv;
  const uint8_t* state = m.tile_state + (size_t)bb * m.n_q * m.n_kv;
  int32_t* list = m.q_index + ((size_t)bb * m.n_kv + kt) * m.n_q;
  int count = 0;
  for (int qt = 0; qt < m.n_q; ++qt)
    if (state[(size_t)qt * m.n_kv + kt] != TILE_EMPTY) list[count++] = qt;
  for (int qt = count; qt < m.n_q; ++qt) list[qt] = -1;
  m.q_count[bb * m.n_kv + kt] = count;
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
    const int n = m.n_b * m.n_kv;
    hipLaunchKernelGGL(block_mask_cols_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, m);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace miattn
