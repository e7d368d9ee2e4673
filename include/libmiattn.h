/*
 * libmiattn: fused exact attention for AMD Instinct MI355X (gfx950).
 *
 * Computes O = softmax(mod(scale * Q K^T) masked) V tile by tile with an
 * online softmax (running row max, running normaliser, rescaled output
 * accumulator), so the Sq x Skv score matrix never reaches device memory.
 *
 * Sources for what is computed (web pages, cited by title and section):
 *  - "FlashAttention 설명" (FlashAttention explainer), §1: the definition
 *    softmax(QK^T/sqrt(d))V; §3-§6: never materialise the score matrix,
 *    online softmax with running max / normaliser / output, tiling through
 *    on-chip memory, result identical to the plain definition.
 *  - "FlashAttention-2 — GPU attention의 사실상 표준", §3-§4: Q row tiles,
 *    K/V column tiles, backward pass recomputes the scores.
 *  - "PyTorch FlexAttention, FlashAttention-4 백엔드 도입" (섹션별 상세):
 *    score modifiers receive (score, batch, head, q_idx, kv_idx); ALiBi,
 *    sliding window, document masking, tanh soft-cap, local boost; block-
 *    sparse iteration skips fully masked blocks; 128x128 mask blocks.
 *  - "FlashInfer SM120 NVFP4 어텐션 최적화" §1-§2: separate query/output
 *    and key/value head counts, optional LSE output [B, Hq, S] float32.
 *
 * Conventions (all entry points):
 *  - Layout: Q, O [B][Hq][Sq][D]; K, V [B][Hkv][Skv][D]; contiguous, D
 *    innermost.  LSE [B][Hq][Sq] float32, natural-log units.  The tensor
 *    pointers (Q, K, V, O, dO, dQ, dK, dV) and the workspace must be 16-byte
 *    aligned; float and int32 arrays 4-byte aligned.
 *  - Ownership: the caller owns every buffer.  The library allocates no
 *    device memory, keeps no mutable global state, and is re-entrant.
 *    Parameter structs are host memory read during the call only; the
 *    arrays they point to (doc_ids, alibi_slopes, rel_bias and its gradient
 *    and scratch, block-mask arrays) are device memory.
 *  - Errors: an fa_status is returned.  All argument validation happens
 *    before any HIP call, so an invalid call has no device side effect.
 *    A failed launch maps to FA_ERR_LAUNCH.  Nothing is thrown or aborted.
 *  - Execution is asynchronous on `stream` (a hipStream_t; NULL = the
 *    default stream).  The library never synchronises.
 *  - GQA / MQA: G = Hq / Hkv; query head h uses key/value head h / G.
 *  - Indices in masks and modifiers are absolute (query i in [0,Sq), key j
 *    in [0,Skv)); causal means j <= i even when Sq != Skv.
 */
#ifndef LIBMIATTN_H
#define LIBMIATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = -2,       /* sizes negative, inconsistent or too large */
  FA_ERR_UNSUPPORTED = -3, /* head dim / dtype / combination not built */
  FA_ERR_ALIGN = -4,       /* a device pointer is not 16-byte aligned */
  FA_ERR_PARAM = -5,       /* mask or modifier parameter out of range */
  FA_ERR_WORKSPACE = -6,   /* workspace missing or too small */
  FA_ERR_LAUNCH = -7,      /* the kernel launch failed */
  FA_ERR_SCRATCH = -8      /* fa_bwd_noalloc: the problem's workspace exceeds
                              FA_NOALLOC_SCRATCH_BYTES */
} fa_status;

typedef enum { FA_BF16 = 0, FA_F32 = 1 } fa_dtype;

/* Masks ("PyTorch FlexAttention, FlashAttention-4" page, 섹션별 상세 and
 * 핵심 요약: sliding window and document masking as mask_mod examples). */
typedef enum {
  FA_MASK_NONE = 0,           /* every key */
  FA_MASK_CAUSAL = 1,         /* j <= i */
  FA_MASK_SLIDING_WINDOW = 2, /* j <= i and i - j < window */
  FA_MASK_DOCUMENT = 3        /* doc_ids[b][i] == doc_ids[b][j] and j <= i */
} fa_mask_kind;

/* Score modifiers, applied to the scaled score s = scale * q_i . k_j (same
 * page: score_mod(score, b, h, q_idx, kv_idx); the soft-cap and local_boost
 * code examples; ALiBi named in the summary). */
typedef enum {
  FA_MOD_NONE = 0,
  FA_MOD_ALIBI = 1,       /* s + slope[h] * (j - i) */
  FA_MOD_SOFTCAP = 2,     /* softcap * tanh(s / softcap) */
  FA_MOD_LOCAL_BOOST = 3, /* |i - j| < boost_radius ? s * boost_factor : s */
  FA_MOD_REL_BIAS = 4     /* s + rel_bias[h][i - j + Skv - 1]: a learnable
                             relative-position bias (the same page lists the
                             gradients of learnable bias tensors among
                             FlexAttention's limits; fa_bwd returns it) */
} fa_mod_kind;

typedef struct {
  int32_t window;          /* FA_MASK_SLIDING_WINDOW: keys per query, >= 1
                              (any value up to INT32_MAX; from max(Sq, Skv)
                              on, the causal mask) */
  const int32_t* doc_ids;  /* FA_MASK_DOCUMENT: device int32 [B][S] */
  int32_t* visited;        /* optional debug output, device int32
                              [B][Hq][ceil(Sq/128)]: fa_fwd ADDS the number of
                              key steps (of fa_fwd_kv_step() columns) each
                              128-row query tile processed.  NULL in production. */
  int32_t* work_queue;     /* optional, device int32[FA_WORK_QUEUE_INTS], all
                              zero before its first use.  fa_fwd then runs a
                              persistent, dynamically scheduled kernel whose
                              workgroups take query tiles from these counters
                              (one per XCD, longest tiles first, leftovers
                              shared) until none is left; the last workgroup
                              zeroes them again, so repeated calls and graph
                              replays need no clearing.  Calls that overlap in
                              time need separate arrays.  Results are
                              bit-identical to the static schedule's.  NULL:
                              the static schedule.  Ignored by fa_bwd. */
  int64_t* wg_trace;       /* optional debug output, device int64
                              [B * Hq * ceil(Sq/128)][FA_WG_TRACE_WORDS]:
                              fa_fwd writes one record per query tile it
                              processes, at the tile's index P in the static
                              schedule (0 <= P < the number of tiles, which is
                              B * Hq * ceil(Sq/256) for the 256-row kernel
                              that bf16 forwards of more than 1024 keys with
                              analytic masks take; records past it are left
                              untouched): [0] the GPU's constant 100 MHz
                              clock (s_memrealtime) when the tile starts,
                              [1] the same after its last output is issued,
                              [2] the XCC_ID hardware register << 32 | the
                              HW_ID register of the workgroup's first wave,
                              [3] the tile's query rows << 32 | its key
                              steps.  Static schedule only: ignored with a
                              work_queue.  fa_bwd (all its forms) writes the
                              same records for its dK/dV workgroups (key
                              tiles: [3] holds 128 << 32 | the query steps)
                              at 0 <= P < B * Hkv * ceil(Skv/128), then for
                              its dQ workgroups from that index on (room:
                              B * Hkv * ceil(Skv/128) + B * Hq * ceil(Sq/128)
                              records).  NULL in production. */
} fa_mask_params;

/* Words per record of fa_mask_params.wg_trace. */
#define FA_WG_TRACE_WORDS 4

/* Length of fa_mask_params.work_queue. */
#define FA_WORK_QUEUE_INTS 288

typedef struct {
  const float* alibi_slopes; /* device float [Hq]; NULL: 2^(-8(h+1)/Hq) */
  float softcap;             /* FA_MOD_SOFTCAP: > 0 */
  int32_t boost_radius;      /* FA_MOD_LOCAL_BOOST: >= 0; 0 boosts no pair, and
                                any value >= max(Sq, Skv) boosts every pair */
  float boost_factor;        /* FA_MOD_LOCAL_BOOST: finite */
  const float* rel_bias;     /* FA_MOD_REL_BIAS: device float [Hq][Sq + Skv - 1],
                                entry i - j + Skv - 1 is added to the scaled
                                score of (query i, key j) of query head h */
  float* rel_bias_grad;      /* fa_bwd / fa_bwd_phase with FA_MOD_REL_BIAS (DQ
                                phase): NULL, or device float [Hq][Sq + Skv - 1]
                                that is overwritten with d(sum O * dout) /
                                d rel_bias, summed over the batch in a fixed
                                order (deterministic) */
  float* rel_bias_ws;        /* required with rel_bias_grad: device scratch of
                                at least rel_bias_ws_bytes bytes, 16-byte
                                aligned, contents need not be initialised */
  size_t rel_bias_ws_bytes;  /* >= fa_bwd_rel_bias_workspace_bytes(B, Hq, Sq, Skv) */
} fa_mod_params;

/* Tile states of a block mask. */
enum { FA_TILE_EMPTY = 0, FA_TILE_PARTIAL = 1, FA_TILE_FULL = 2 };

/* Block mask at block_q x block_kv granularity ("PyTorch FlexAttention,
 * FlashAttention-4" page, 섹션별 상세: block-sparse iteration skips masked
 * blocks; 128x128 blocks).  A tile is EMPTY when no in-range pair is
 * admissible, FULL when every pair is in range and admissible, PARTIAL
 * otherwise.  The arrays are device memory owned by the caller.
 * n_b is 1 (one mask for every batch row) or B (document masks). */
typedef struct {
  int32_t block_q, block_kv; /* must both be 128 */
  int32_t n_q, n_kv;         /* ceil(Sq/block_q), ceil(Skv/block_kv) */
  int32_t n_b;               /* 1 or B */
  uint8_t* tile_state;       /* [n_b][n_q][n_kv] FA_TILE_* */
  int32_t* kv_count;         /* [n_b][n_q]  non-empty kv tiles per q tile */
  int32_t* kv_index;         /* [n_b][n_q][n_kv] ascending, first kv_count valid */
  int32_t* q_count;          /* [n_b][n_kv] non-empty q tiles per kv tile */
  int32_t* q_index;          /* [n_b][n_kv][n_q] ascending, first q_count valid */
  int32_t* q_order;          /* [n_b][n_q] or NULL: the q tiles in schedule order,
                                by descending kv_count, ties by ascending index.
                                Under a document mask, tiles whose kv lists
                                start at the same kv tile (one document) stay
                                together: such groups go by descending weight
                                (their longest kv_count), ties by ascending
                                first kv tile, and inside a group by descending
                                kv_count, ties by ascending index.  The query-
                                stationary kernels start their tiles in this
                                order: the longest first, so the hardware's
                                in-order dispatch to free compute units
                                balances uneven rows, and one document's tiles
                                together, so they share its key rows in L2.
                                Rows of more than 2048 tiles get the identity
                                order.  NULL: the default order. */
  int32_t* kv_order;         /* [n_b][n_kv] or NULL: the kv tiles in the same
                                kind of order (document groups by the last q
                                tile of their q lists), for the key-stationary
                                dK/dV kernel */
} fa_block_mask;

/* Forward pass.  q, k, v, out: device, dtype elements in the layout above.
 * lse: device float [B][Hq][Sq] or NULL (no LSE written).  scale multiplies
 * q . k before the modifier; it must be finite and >= 0 with scale * log2(e)
 * finite in fp32 (and 2 scale log2(e) / softcap for FA_MOD_SOFTCAP), else
 * FA_ERR_PARAM.  mask_params / mod_params: host structs, may be
 * NULL when the kind needs no parameter.  block_mask: NULL (tile ranges
 * derived from the mask kind) or a mask built for this (mask, B, Sq, Skv);
 * when given, only its non-empty tiles are visited and FULL tiles skip the
 * elementwise mask.  Rows with no admissible key get O = 0, LSE = -inf.
 * B == 0 or Sq == 0 is a valid no-op.  Supported: D in {64, 128}; dtype
 * FA_BF16 or FA_F32 (fp32 inputs/outputs, fp32 products). */
int fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
           int B, int Hq, int Hkv, int Sq, int Skv, int D, int dtype, float scale,
           int mask_kind, const fa_mask_params* mask_params,
           int score_mod_kind, const fa_mod_params* mod_params,
           const fa_block_mask* block_mask, void* stream);

/* Width in keys of one forward key step (the unit of fa_mask_params.visited). */
int fa_fwd_kv_step(int D, int dtype);

/* Backward pass with recomputation ("FlashAttention-2" page §3-§4: the
 * backward pass recomputes the scores instead of storing them).  Given the
 * forward's out and lse (lse is required) and dout, writes dq [B][Hq][Sq][D]
 * and dk, dv [B][Hkv][Skv][D] (summed over each GQA group), accumulating in
 * float32 and rounding once.  workspace: device, at least
 * fa_bwd_workspace_bytes(B, Hq, Sq, D) bytes, 16-byte aligned, contents
 * need not be initialised (it receives two [B][Hq][Sq] float arrays: the
 * row sums of dout * out and the LSE in log2 units).  Supported: dtype
 * FA_BF16, D in {64, 128}, every mask and modifier.  With FA_MOD_REL_BIAS
 * and mod_params->rel_bias_grad set, the DQ phase also writes the bias
 * table's gradient (see fa_mod_params). */
int fa_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
           int B, int Hq, int Hkv, int Sq, int Skv, int D, int dtype, float scale,
           int mask_kind, const fa_mask_params* mask_params,
           int score_mod_kind, const fa_mod_params* mod_params,
           const fa_block_mask* block_mask, void* stream);

/* The phases of fa_bwd, any subset per call (a bit mask): FA_BWD_DELTA
 * writes rowsum(dout * out) and the LSE in log2 units into the workspace;
 * FA_BWD_DKDV writes dk and dv; FA_BWD_DQ writes dq.  Same arguments and
 * validation as fa_bwd.  With a workspace of fa_bwd_workspace_bytes, DKDV
 * and DQ only read what DELTA wrote, so once DELTA has finished they may run
 * concurrently on different streams; with the stored-dS workspace
 * (fa_bwd_ds_workspace_bytes) DQ reads what DKDV wrote and must follow it.
 * A call holding both DELTA and DQ (without stored dS) runs them as one
 * launch, the dQ kernel computing the row sums of its own rows, then DKDV if
 * asked; fa_bwd is that call with all three.  Every split of the phases over
 * calls in the order DELTA, DKDV, DQ (or DELTA + DQ, then DKDV) on one stream
 * gives the same bits as fa_bwd. */
enum { FA_BWD_DELTA = 1, FA_BWD_DKDV = 2, FA_BWD_DQ = 4 };
int fa_bwd_phase(int phase, const void* q, const void* k, const void* v, const void* out,
                 const void* dout, const float* lse, void* dq, void* dk, void* dv, void* workspace,
                 size_t ws_bytes, int B, int Hq, int Hkv, int Sq, int Skv, int D, int dtype,
                 float scale, int mask_kind, const fa_mask_params* mask_params,
                 int score_mod_kind, const fa_mod_params* mod_params,
                 const fa_block_mask* block_mask, void* stream);

size_t fa_bwd_workspace_bytes(int B, int Hq, int Sq, int D);

/* Workspace size of the stored-dS backward: fa_bwd_workspace_bytes plus room
 * for the bf16 dS tiles the dK/dV phase computes anyway (2 bytes per query-
 * key pair it visits: B * Hq * Sq * Skv * 2 without a mask, about half that
 * under the causal mask; 2.2 GB at B=2, Hq=16, S=8192 causal).  Given a
 * workspace at least this large, fa_bwd / fa_bwd_phase store dS in the DKDV
 * phase and the DQ phase computes dQ = scale dS K from it instead of
 * recomputing the scores and dO V^T (FA_MASK_NONE or FA_MASK_CAUSAL, no block
 * mask, any modifier but FA_MOD_REL_BIAS; other calls ignore the extra
 * space).  Then DQ reads what DKDV wrote, so DQ must run after DKDV.  Results
 * meet the same bars as the recomputing path (not the same bits: dS comes
 * from the other kernel's accumulation order) and are deterministic.
 * Returns 0 for other mask kinds or invalid sizes. */
size_t fa_bwd_ds_workspace_bytes(int B, int Hq, int Sq, int Skv, int D, int mask_kind);

/* Size of the fixed device scratch of fa_bwd_noalloc: 16 MiB per GPU, which
 * holds the backward workspace of up to B * Hq * Sq = 2^21 query rows. */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* fa_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops, harnesses
 * that forbid allocation).  The workspace fa_bwd takes from the caller
 * (fa_bwd_workspace_bytes(B, Hq, Sq, D) bytes) lives instead in a device
 * array of FA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends; its address is looked up on the first
 * call on each device.  Nothing is allocated by the call (the relative-bias
 * gradient still takes its scratch from mod_params, as in fa_bwd).  Returns
 * FA_ERR_SCRATCH, before any HIP call, when the workspace would exceed
 * FA_NOALLOC_SCRATCH_BYTES; otherwise the same validation, results and
 * errors as fa_bwd (identical bits: the same kernels).  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (e.g. on
 * two streams) race and must be serialised by the caller.  The array needs
 * no clearing: each call overwrites what it reads. */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* out, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv,
                   int B, int Hq, int Hkv, int Sq, int Skv, int D, int dtype, float scale,
                   int mask_kind, const fa_mask_params* mask_params,
                   int score_mod_kind, const fa_mod_params* mod_params,
                   const fa_block_mask* block_mask, void* stream);

/* Size of the scratch a relative-bias gradient needs (fa_mod_params
 * rel_bias_ws): one float row of Skv + 128 per (batch, query head, 128-row
 * query tile), the per-tile diagonal sums that a fixed-order reduction then
 * adds up.  It grows as B Hq Sq Skv / 32 bytes: 68 MB at B=2, Hq=16,
 * Sq=Skv=8192; 2.2 GB at B=1, Hq=16, Sq=Skv=65536.  0 when any size is 0. */
size_t fa_bwd_rel_bias_workspace_bytes(int B, int Hq, int Sq, int Skv);

/* FP8 path ("FlashAttention-3 (KO)" page, technical innovation 3: FP8
 * doubles the matrix throughput of 16-bit formats; incoherent processing
 * multiplies Q and K by a random orthogonal matrix before quantizing, which
 * spreads outliers while Q K^T is unchanged).  Format: OCP E4M3 (sign, 4
 * exponent bits with bias 7, 3 mantissa bits, largest finite 448).  Every
 * tensor carries one power-of-two scale per block of 128 rows of each
 * (batch, head), stored as the byte e + 127 (E8M0): row value ~= E4M3 value
 * * 2^e, 2^e the smallest power of two with the block's max |value| <= 448
 * * 2^e. */

/* Quantize x (bf16 [rows][S][D], rows = B * H, contiguous) to E4M3 codes x8
 * (uint8, same layout) and scale bytes (uint8 [rows][ceil(S/128)]), rounding
 * to nearest even.  signs: device float [D] of +-1, or NULL.  When given,
 * each row is first replaced by (row * signs) H / sqrt(D), H the Sylvester
 * Hadamard matrix (orthogonal, so applying the same signs to Q and K leaves
 * Q K^T unchanged).  D in {64, 128}; x and x8 16-byte aligned.  Returns an
 * fa_status; rows * S == 0 is a no-op. */
int fa_fp8_quantize(const void* x, void* x8, uint8_t* scales, int rows, int S, int D, const float* signs,
                    void* stream);

/* Forward pass from E4M3 tensors: q8 [B][Hq][Sq][D], k8 and v8
 * [B][Hkv][Skv][D] with their scale bytes (q_scale [B][Hq][ceil(Sq/128)],
 * k_scale and v_scale [B][Hkv][ceil(Skv/128)]), as written by
 * fa_fp8_quantize.  Writes out (bf16 [B][Hq][Sq][D]) and, if lse is not
 * NULL, LSE (float [B][Hq][Sq], natural log).  Both products run on FP8
 * matrix cores with float32 accumulation; the probabilities of each 64-key
 * step are rounded to E4M3 (relative to the running row max) for the P V
 * product, while the row sum uses them unrounded.  scale multiplies the
 * dequantized q . k.  Masks: FA_MASK_NONE, FA_MASK_CAUSAL,
 * FA_MASK_SLIDING_WINDOW (FA_MASK_DOCUMENT -> FA_ERR_UNSUPPORTED); no score
 * modifier.  Of mask_params only window is read (no visited counters, work
 * queue or workgroup trace on this path).  D in {64, 128}; tensors 16-byte
 * aligned. */
int fa_fwd_fp8(const void* q8, const void* k8, const void* v8, const uint8_t* q_scale, const uint8_t* k_scale,
               const uint8_t* v_scale, void* out, float* lse, int B, int Hq, int Hkv, int Sq, int Skv, int D,
               float scale, int mask_kind, const fa_mask_params* mask_params, void* stream);

/* Build a block mask for (mask_kind, mask_params, B, Sq, Skv) into the
 * caller's arrays described by *out (block sizes, n_q, n_kv, n_b and the five
 * list pointers must be set; q_order and kv_order are filled when not NULL;
 * n_b must be B for FA_MASK_DOCUMENT and may be 1 otherwise).  One
 * stream-ordered pass; every entry of every array is written (unused list
 * slots are set to -1). */
/* Bytes of one device allocation that holds every array of a block mask
 * with n_b mask rows (1, or B for document masks) for sequence lengths Sq and
 * Skv at 128 x 128 blocks, each array starting on a 256-byte boundary;
 * with_orders adds q_order and kv_order.  block_q and block_kv must be 128.
 * Returns 0 for invalid sizes (n_b < 1, lengths < 0 or too large, blocks
 * other than 128). */
size_t fa_block_mask_bytes(int n_b, int Sq, int Skv, int block_q, int block_kv, int with_orders);

/* Fill *out (block sizes, counts and every array pointer) for a block mask
 * carved from `base`, an allocation of at least fa_block_mask_bytes(...)
 * bytes, 256-byte aligned, in the order tile_state, kv_count, kv_index,
 * q_count, q_index[, q_order, kv_order].  Host only: no device access, no
 * HIP call.  Returns FA_ERR_NULL, FA_ERR_ALIGN or FA_ERR_SHAPE on bad
 * arguments, else FA_OK. */
int fa_block_mask_layout(void* base, int n_b, int Sq, int Skv, int block_q, int block_kv, int with_orders,
                         fa_block_mask* out);

int fa_block_mask_build(int mask_kind, const fa_mask_params* mask_params,
                        int B, int Sq, int Skv, const fa_block_mask* out, void* stream);

const char* fa_status_str(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH: FA_VERSION of the
 * header it was built from.  0.2.0: fa_mask_params gained work_queue and
 * wg_trace (a caller built against an older header passes a shorter
 * struct, so check fa_version() == FA_VERSION first). */
#define FA_VERSION 200
int fa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LIBMIATTN_H */
