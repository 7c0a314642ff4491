/*
 * pisa.h - C ABI of the MI355X (gfx950) implementation of PISA:
 * the mean-pooled key pyramid, coarse-to-fine pyramid Top-K block selection
 * with LogSumExp scoring, the flat BSA selector it is compared with,
 * block-sparse attention over the selected blocks and its backward with the
 * block lists held fixed, pyramid upkeep for decode, and a GQA decode step.
 *
 * Source of the method: "Block Sparse Attention with Log-Linear Complexity"
 * (PISA), as laid out by the close-reading page "论文精读 · Block Sparse
 * Attention with Log-Linear Complexity (PISA)"; sections and equations below
 * refer to that page.
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * - All functions are extern "C", never throw, and return a pisa_status.
 * - Every tensor argument is a DEVICE pointer to contiguous row-major memory,
 *   16-byte aligned, owned by the caller.  The alignment is checked for the
 *   tensors the kernels access with 16-byte vector loads and stores (Q, K, V,
 *   O, the pyramid, the caches, the gradients and the workspace): an address
 *   off it returns PISA_ERR_INVALID before any launch; block_idx,
 *   block_score, row_lse and cache_len need only their elements' alignment.
 *   The library allocates no device or
 *   host memory and keeps no state between calls; calls are re-entrant.  The
 *   one exception is pisa_select_noalloc, which uses a fixed device array of
 *   the library's (see there).
 * - Layouts (B batch, Hq query heads, Hkv KV heads, N tokens, d head dim,
 *   K budget, R pyramid rows):
 *     Q, O        [B, Hq,  N, d]   dtype = problem.dtype
 *     K, V        [B, Hkv, N, d]   dtype = problem.dtype
 *     pyramid     [B, Hkv, R, d]   float32; level l occupies rows
 *                                  row_offsets[l-1] .. row_offsets[l]-1
 *     block_idx   [B, Hkv, N, K]   int32, each row ascending, padded with -1
 *     block_score [B, Hkv, N, K]   float32: the score that ranked the entry;
 *                                  +inf for entries kept without ranking
 *                                  (forced, or all candidates kept); -inf for
 *                                  padding
 *     row_lse     [B, Hq, N]       float32 natural-log softmax normaliser
 *   Query head h reads KV head h / (Hq / Hkv).
 * - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *   asynchronously; outputs are valid once the stream has been synchronised.
 * - Validation happens before anything is enqueued: on any error the function
 *   returns < 0 and has written nothing.  A failed launch returns PISA_ERR_HIP;
 *   pisa_last_error() then describes it (thread-local text).
 * - Outputs are bitwise reproducible run to run (no floating-point atomics).
 * - No call clears memory with hipMemsetAsync (workspaces are initialised by
 *   the library's own kernels) or waits on the host, so the launches an entry
 *   point enqueues can be captured into a HIP graph and replayed.  Exceptions:
 *   the per-kernel events of pisa_profile_enable, and pisa_select_noalloc's
 *   first call on a device, which looks its scratch up (make one call before
 *   capturing).
 *
 * Supported now: d in {64, 128}; C in {16, 32, 64}; g = 2; 1 <= K <= 32;
 * K >= 3 with PISA_FORCE_FIRST_PREV (K >= 1 otherwise); Hq % Hkv == 0 with
 * Hq / Hkv <= 16; PISA_FORCE_FIRST_PREV requires PISA_CAUSAL.
 */
#ifndef PISA_H_
#define PISA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PISA_OK = 0,
  PISA_ERR_INVALID = -1,     /* null pointer, bad shape or flag combination  */
  PISA_ERR_UNSUPPORTED = -2, /* valid but outside the supported d/C/K/g/G    */
  PISA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required   */
  PISA_ERR_HIP = -4          /* a HIP call or kernel launch failed           */
} pisa_status;

typedef enum { PISA_F32 = 0, PISA_BF16 = 1 } pisa_dtype;

enum {
  /* Causal prefill/decode (§5.3): nodes entirely after the current leaf are
     dropped, the node holding the current leaf is kept without being ranked,
     and attention masks tokens after t inside the current block. */
  PISA_CAUSAL = 1u,
  /* Also keep leaf 0 and leaf c-1 (and their ancestors) for query t in leaf c,
     as the NSA/FLA policy of §5.3; they take slots of the budget K. */
  PISA_FORCE_FIRST_PREV = 2u,
  /* Rank candidates by a truncation of eq. (8) (§4.3 eq. (9)) instead of eq.
     (7)'s LSE: PISA-1 scores a node by the mean of its children's logits,
     PISA-2 by that mean plus half their population variance (at the leaf
     level, over the raw keys).  At most one of the two.  Used by pisa_select
     (per-query selector; PISA_SELECT_TWO_STAGE is then unsupported) and
     pisa_decode_step; the other entry points ignore them. */
  PISA_SCORE_MEAN = 4u,
  PISA_SCORE_MEAN_VAR = 8u
};

enum { PISA_MAX_LEVELS = 32 };

typedef struct {
  int32_t batch;     /* B */
  int32_t heads_q;   /* Hq */
  int32_t heads_kv;  /* Hkv */
  int32_t seq_len;   /* N (prefill) or cache capacity (decode) */
  int32_t head_dim;  /* d */
  int32_t block;     /* C, leaf block size */
  int32_t topk;      /* K, blocks kept per query and KV head */
  int32_t branch;    /* g, must be 2 */
  uint32_t flags;    /* PISA_CAUSAL | PISA_FORCE_FIRST_PREV | PISA_SCORE_* */
  int32_t dtype;     /* pisa_dtype of Q/K/V/O */
  float scale;       /* logit scale; <= 0 selects 1/sqrt(d) */
} pisa_problem;

/* Operations for pisa_workspace_bytes. */
enum {
  PISA_OP_PYRAMID = 0,
  PISA_OP_SELECT = 1,
  PISA_OP_BSA = 2,
  PISA_OP_ATTN = 3,
  PISA_OP_DECODE = 4,
  PISA_OP_ATTN_BWD = 5
};

/* Selection strategies for pisa_select (problem-independent hint). */
enum {
  PISA_SELECT_AUTO = 0,      /* library picks (two-stage when it pays) */
  PISA_SELECT_FUSED = 1,     /* one kernel per query, leaf level included */
  PISA_SELECT_TWO_STAGE = 2  /* intermediate levels per query, then leaf
                                blocks scored once per group of queries */
};

/* Pyramid geometry of eq. (3) (§4.1): M_1 = ceil(N/C), M_{l+1} = ceil(M_l/2)
 * until one node remains.  Host-only, touches no device.
 *   levels:      out, number of levels L (may be NULL)
 *   row_offsets: out, L+1 entries: level l starts at row_offsets[l-1]; the
 *                last entry is R, the total row count (may be NULL)
 *   max_offsets: capacity of row_offsets (>= L+1 when row_offsets != NULL)
 * Errors: PISA_ERR_INVALID for N < 1, C < 1, g != 2 or too small a buffer. */
int pisa_pyramid_layout(int32_t seq_len, int32_t block, int32_t branch, int32_t* levels,
                        int64_t* row_offsets, int32_t max_offsets);

/* Device workspace (bytes) that `op` needs for this problem; 0 means none.
 * Pass a buffer at least this large as `ws` / `ws_bytes`.  Host-only. */
int pisa_workspace_bytes(const pisa_problem* problem, int32_t op, size_t* bytes);

/* Key pyramid (§4.1 eqs. (3), (4)): level 1 row i is the mean of keys
 * [iC, min((i+1)C, N)); level l+1 row i is the mean of the existing level-l
 * rows {2i, 2i+1}.  Reads K once, writes every level of `pyramid`.
 *   k:        [B, Hkv, N, d] dtype
 *   pyramid:  [B, Hkv, R, d] float32, out */
int pisa_build_pyramid(const pisa_problem* problem, const void* k, float* pyramid, void* stream);

/* Pyramid cache upkeep for decode (§5.3, decode cache; §4.1 eqs. (3), (4)):
 * for each sequence b, the key of token t = cache_len[b] - 1 is already in
 * k_cache; the rows on t's path (leaf t / C and every ancestor) are rewritten
 * to those of the pyramid over exactly t + 1 tokens: the leaf is the mean of
 * keys [cC, t], each ancestor the mean of its existing children.  The rows
 * written equal bit for bit what pisa_build_pyramid writes for a sequence of
 * t + 1 tokens; rows off the path are not touched.  O(C d + L d) per
 * (sequence, KV head).  Call once per appended token, after writing it.
 *   problem.seq_len: cache capacity (the pyramid's layout); flags and topk
 *                    are not used
 *   cache_len: [B] int32 device, length after the append; values outside
 *              [1, capacity] leave that sequence's pyramid unchanged
 *   k_cache:   [B, Hkv, capacity, d] dtype
 *   pyramid:   [B, Hkv, R(capacity), d] float32, updated in place
 * Errors: as pisa_build_pyramid; PISA_ERR_INVALID for NULL pointers. */
int pisa_pyramid_append(const pisa_problem* problem, const int32_t* cache_len,
                        const void* k_cache, float* pyramid, void* stream);

/* PISA selection (§4.2 eqs. (5), (6); §4.3 eq. (7); §4.4 eq. (11); §5.3):
 * per (b, kv head, t), descend from the root; at each level drop future nodes,
 * keep all candidates if there are at most K, else keep the forced nodes plus
 * the best K-#F others by sum over the group's heads of
 * LSE_r(scale * q . kbar_r) over the node's children (raw keys at level 1),
 * ties to the lower index; expand kept nodes to their children.
 *   q:           [B, Hq, N, d] dtype
 *   k:           [B, Hkv, N, d] dtype (leaf level scores raw keys)
 *   pyramid:     from pisa_build_pyramid
 *   block_idx:   [B, Hkv, N, K] int32, out
 *   block_score: [B, Hkv, N, K] float32, out, may be NULL
 *   strategy:    PISA_SELECT_*
 *   ws/ws_bytes: workspace of pisa_workspace_bytes(PISA_OP_SELECT) bytes
 * Tuning (two-stage path; environment, read per call): PISA_S2_ITEM_ROWS, the
 * (query, head) columns served by one load of a level-3 node's keys (power of
 * two in [64, 4096], default 1024; the workspace size follows it), and
 * PISA_S2_BATCH_ROWS, the columns staged per batch (32, 64 or 128; default 64
 * with one query head per KV head, else 128), and PISA_S1_TILE_ROWS, the child
 * rows per window of the first stage with 16 query heads per KV head (multiple
 * of 64 in [64, 8192], default 8192).  Results do not depend on them. */
int pisa_select(const pisa_problem* problem, const void* q, const void* k, const float* pyramid,
                int32_t* block_idx, float* block_score, int32_t strategy, void* ws,
                size_t ws_bytes, void* stream);

/* pisa_select for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same selection, bit for bit, with the two-stage selector's workspace taken
 * from a fixed array of PISA_NOALLOC_SCRATCH_BYTES that the library keeps on
 * each device it runs on until the process ends.  No allocation, no memset.
 *   arguments:  as pisa_select, without ws / ws_bytes
 *   limits:     a problem whose two-stage workspace
 *               (pisa_workspace_bytes(PISA_OP_SELECT)) exceeds the scratch is
 *               rejected with PISA_ERR_WORKSPACE before anything is enqueued
 *               (PISA_SELECT_FUSED needs no scratch and has no such limit)
 *   stream:     must belong to the current device (the scratch used is the
 *               current device's)
 *   concurrency: every call on one device shares that device's scratch and
 *               leaves the last call's contents in it; calls that overlap on
 *               one device (different streams or threads) race. */
#define PISA_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int pisa_select_noalloc(const pisa_problem* problem, const void* q, const void* k,
                        const float* pyramid, int32_t* block_idx, float* block_score,
                        int32_t strategy, void* stream);

/* BSA flat selection (§02 eq. (1)): s_{t,i} = sum over the group's heads of
 * scale * q . kbar_i over every eligible leaf summary (level 1 of `pyramid`),
 * written in full to the workspace, then the forced blocks plus the best
 * K-#F others (same forcing, causal and tie rules as pisa_select).
 *   q, pyramid, block_idx, block_score: as pisa_select
 *   ws/ws_bytes: pisa_workspace_bytes(PISA_OP_BSA) bytes (holds the scores:
 *                B * Hkv * N * M1 fp32, M1 = ceil(N / C), plus the bf16 planes)
 * Up to 4096 leaf blocks for every supported shape; beyond that only for bf16,
 * a power-of-two group and M1 a multiple of 4 (else PISA_ERR_UNSUPPORTED). */
int pisa_bsa_select(const pisa_problem* problem, const void* q, const float* pyramid,
                    int32_t* block_idx, float* block_score, void* ws, size_t ws_bytes,
                    void* stream);

/* Block-sparse attention (§02 eq. (2); mask of §5.3): for each query head h
 * and position t, softmax(scale * q . k_j) weighted sum of v_j over the
 * tokens of the blocks in block_idx[b, h / G, t, :] (-1 entries skipped),
 * restricted to j <= t when PISA_CAUSAL is set.
 *   q, k, v:   as above
 *   block_idx: [B, Hkv, N, K] int32 leaf indices; rows need not be sorted;
 *              entries < 0 or >= ceil(N/C) are skipped; duplicates are
 *              not allowed (they would be counted twice); a row whose blocks
 *              hold no attendable token gets zeros and row_lse = -inf
 *   out:       [B, Hq, N, d] dtype, out
 *   row_lse:   [B, Hq, N] float32, out, may be NULL
 *   ws/ws_bytes: pisa_workspace_bytes(PISA_OP_ATTN) bytes */
int pisa_block_sparse_attn(const pisa_problem* problem, const void* q, const void* k,
                           const void* v, const int32_t* block_idx, void* out, float* row_lse,
                           void* ws, size_t ws_bytes, void* stream);

/* Backward of pisa_block_sparse_attn with block_idx held fixed (§5.3,
 * "backward": the selected indices do not move and gradients flow only
 * through the attention entries they select).  For every query head h and row
 * t with token set J (the tokens pisa_block_sparse_attn attends), with
 * P_j = exp(scale q.k_j - row_lse) and D = dout . out:
 *   dq      = scale * sum_j P_j (dout . v_j - D) k_j
 *   dk_j   += scale * P_j (dout . v_j - D) q
 *   dv_j   += P_j dout
 * dk and dv sum over every query head of the KV group and every row whose
 * list holds the key's block; keys no row attends get zeros.
 *   q, k, v, block_idx: the forward's inputs (same rules for block_idx)
 *   out, row_lse:       the forward's outputs for exactly these inputs
 *                       (row_lse is required)
 *   dout:      [B, Hq, N, d] dtype, gradient of the loss w.r.t. out
 *   dq:        [B, Hq, N, d] dtype, out (every row written)
 *   dk, dv:    [B, Hkv, N, d] dtype, out (every row written)
 *   ws/ws_bytes: pisa_workspace_bytes(PISA_OP_ATTN_BWD) bytes
 * Supported: every shape pisa_block_sparse_attn supports with ceil(N / C) <=
 * 8192 (PISA_ERR_UNSUPPORTED otherwise); bf16 with C = 64 and a power-of-two
 * Hq / Hkv runs on the matrix cores, the rest on fp32 vector arithmetic.
 * Deterministic: each block's rows are visited in row order and every sum has
 * a fixed order. */
int pisa_block_sparse_attn_backward(const pisa_problem* problem, const void* q, const void* k,
                                    const void* v, const int32_t* block_idx, const void* out,
                                    const float* row_lse, const void* dout, void* dq, void* dk,
                                    void* dv, void* ws, size_t ws_bytes, void* stream);

/* One decode step (§5.1: single fused stage for decode; §5.3 pyramid cache):
 * for each sequence b the new query sits at t = cache_len[b] - 1 and its key
 * and value are already in the caches and the pyramid.  Selection and
 * attention are those of pisa_select / pisa_block_sparse_attn at row t.
 *   problem.seq_len: cache capacity; PISA_CAUSAL must be set
 *   cache_len: [B] int32 device, 1 <= cache_len[b] <= capacity (values out
 *              of range produce -1 indices and zero outputs for that row)
 *   q:         [B, Hq, d] dtype
 *   k_cache, v_cache: [B, Hkv, capacity, d] dtype
 *   pyramid:   [B, Hkv, R(capacity), d] float32 built over the cache
 *   block_idx: [B, Hkv, K] int32, out;  block_score: same, may be NULL
 *   out:       [B, Hq, d] dtype, out;   row_lse: [B, Hq] float32, may be NULL
 *   ws/ws_bytes: pisa_workspace_bytes(PISA_OP_DECODE) bytes */
int pisa_decode_step(const pisa_problem* problem, const int32_t* cache_len, const void* q,
                     const void* k_cache, const void* v_cache, const float* pyramid,
                     int32_t* block_idx, float* block_score, void* out, float* row_lse,
                     void* ws, size_t ws_bytes, void* stream);

/* Per-kernel timing (diagnostics).  While enabled, every kernel the library
 * launches is bracketed by two HIP events recorded on its stream (the library
 * creates and keeps these events; timing is off by default).  Host-only. */
int pisa_profile_enable(int enable);

/* Waits for the recorded events, aggregates elapsed time by kernel name in
 * order of first launch, and forgets the records.
 *   names:     out, '\n'-terminated kernel names (truncated to names_len)
 *   total_ms:  out [max_kernels], summed milliseconds per kernel
 *   counts:    out [max_kernels], launches per kernel
 *   n_kernels: out, number of distinct kernels recorded (may exceed max)
 * Returns PISA_ERR_HIP if an event could not be read. */
int pisa_profile_report(char* names, size_t names_len, float* total_ms, int32_t* counts,
                        int32_t max_kernels, int32_t* n_kernels);

/* Static text for a status code. */
const char* pisa_status_string(int status);

/* Detail of the last error on the calling thread ("" if none). */
const char* pisa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PISA_H_ */
