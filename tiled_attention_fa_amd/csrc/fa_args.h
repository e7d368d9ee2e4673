// Kernel argument blocks shared by the host dispatcher and the kernels.
#pragma once
#include <stdint.h>

namespace miattn {

enum { MASK_NONE = 0, MASK_CAUSAL = 1, MASK_WINDOW = 2, MASK_DOCUMENT = 3 };
enum { MOD_NONE = 0, MOD_ALIBI = 1, MOD_SOFTCAP = 2, MOD_BOOST = 3, MOD_REL_BIAS = 4 };
enum { TILE_EMPTY = 0, TILE_PARTIAL = 1, TILE_FULL = 2 };

// Query rows per workgroup and the block-mask granularity; the forward,
// backward and block-mask kernels all use 128-row query tiles.
constexpr int kTileQ = 128;
constexpr int kMaskBlock = 128;

struct MaskArgs {
  int window;
  const int32_t* doc_ids;  // [B][S]
};

struct ModArgs {
  const float* slopes;  // [Hq] or null: 2^(-8(h+1)/Hq)
  float softcap;
  int boost_radius;
  float boost_factor;
  // Relative-position bias: s + rel_bias[h][i - j + Skv - 1], [Hq][Sq + Skv - 1].
  const float* rel_bias;
  // Backward only, may be null: per-(batch, head, query tile) partial sums of
  // the table gradient ([B][Hq][n_qt][Skv + kBiasRowPad], written by the dQ
  // kernel) and the gradient itself ([Hq][Sq + Skv - 1], their sum).
  float* rel_bias_part;
  float* rel_bias_grad;
  // Softcap in the forward's shifted form (see the forward kernels):
  // k = 2 scale log2(e) / softcap, m = -2 softcap log2(e).
  float softcap_k, softcap_m;
};

// A dQ workgroup's partial row covers the diagonals i - j of its 128 query
// rows: [q0 - Skv + 1, q0 + 127], Skv + 127 entries, padded to Skv + 128.
constexpr int kBiasRowPad = 128;

struct BlockMaskArgs {
  uint8_t* tile_state;  // null: tile ranges follow from the mask kind
  int32_t* kv_count;    // the attention kernels only read these arrays;
  int32_t* kv_index;    // the block-mask builder writes them
  int32_t* q_count;
  int32_t* q_index;
  int n_b, n_q, n_kv;
  int32_t* q_order;   // optional: q tiles in schedule order (longest first, documents together)
  int32_t* kv_order;  // optional: kv tiles in schedule order
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int32_t* visited;
  int B, Hq, Hkv, G, Sq, Skv;
  int n_qt;  // query tiles of kTileQ rows
  float scale, scale_log2;
  MaskArgs mask;
  ModArgs mod;
  BlockMaskArgs bm;
  int32_t* queue;  // null: static schedule; else the work queue of a persistent launch
  int n_cu;        // compute units of the device (persistent grid size)
  int64_t* trace;  // null, or FA_WG_TRACE_WORDS words per tile (debug)
};

// FP8 forward: E4M3 tensors with one E8M0 scale byte per 128-row block of
// each (batch, head).
struct Fp8FwdArgs {
  const uint8_t* q8;
  const uint8_t* k8;
  const uint8_t* v8;
  const uint8_t* q_scale;  // [B][Hq][ceil(Sq/128)]
  const uint8_t* k_scale;  // [B][Hkv][ceil(Skv/128)]
  const uint8_t* v_scale;
  void* o;                 // bf16 [B][Hq][Sq][D]
  float* lse;
  int B, Hq, Hkv, G, Sq, Skv, D;
  int n_qt;
  int window;
  float scale_log2;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* delta;       // [B][Hq][Sq] workspace: rowsum(dO * O)
  const float* lse2;  // [B][Hq][Sq] workspace: LSE * log2(e), +inf for empty rows
  void* dq;
  void* dk;
  void* dv;
  int B, Hq, Hkv, G, Sq, Skv;
  int n_qt, n_kt;
  float scale, scale_log2;
  MaskArgs mask;
  ModArgs mod;
  BlockMaskArgs bm;
  // Stored-dS backward (null: the dQ kernel recomputes S and dP): bf16 dS
  // tiles written by the dK/dV kernel and read by the dQ kernel, blocks of
  // 32 query rows x 128 keys (ds_block), ds_blocks per (batch, query head).
  uint16_t* ds;
  long ds_blocks;
  int n_qs;  // query steps of 32 rows
  // Debug records (fa_mask_params.wg_trace): the dK/dV workgroups' first,
  // then the dQ workgroups' from record B * Hkv * n_kt on.
  int64_t* trace;
  // Set by the launcher, not the caller: the dQ kernel computes delta and
  // lse2 of its own rows and writes them for the dK/dV kernel that follows
  // (no separate row pass).
  int fuse_rows;
};

// Elements of one stored dS block: 4 waves x 64 lanes x 16 bf16.
constexpr int kDsBlock = 4096;

// Index of the stored dS block of key tile kt (128 keys) and query step qs
// (32 rows) within one (batch, query head), for n_qs query steps.  Without
// a mask every pair of (kt, qs) has a block; under the causal mask key tile
// kt has the query steps qs >= 4 kt (the steps the dK/dV kernel visits), and
// the blocks are packed tile after tile.  ds_block(n_kt, 4 n_kt, n_qs) is
// the number of blocks per (batch, query head).  (constexpr: host and device.)
template <int MASK>
constexpr long ds_block(int kt, int qs, int n_qs) {
  if constexpr (MASK == MASK_CAUSAL) {
    const long m = kt < (n_qs + 3) / 4 ? kt : (n_qs + 3) / 4;
    return m * n_qs - 2 * m * (m - 1) + (qs - 4L * kt);
  } else {
    return (long)kt * n_qs + qs;
  }
}

}  // namespace miattn
