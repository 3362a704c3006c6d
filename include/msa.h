/*
 * msa.h -- C ABI of libmsa: causal sliding-window + mean-pooled-landmark
 * sparse attention for AMD Instinct MI355X (gfx950).
 *
 * The operation is the fused local-window + landmark ("Flash-MSA") attention
 * described on the page "Scaling GPU Cluster for Million Token Context",
 * sections "Why Sparse Attention Changes the Game" (a local window of recent
 * tokens plus landmark tokens that summarise distant context) and "What is
 * Flash-MSA Sparse Attention in GPU Clusters?" (one fused, tiled pass that
 * never writes the score matrix to HBM), made precise as:
 *
 *   landmark b   : Kbar_b = mean(K[b*L .. b*L+L-1]),  Vbar_b likewise,
 *                  L = n / G;
 *   row i sees   : key j        iff  i - w < j <= i,
 *                  landmark b   iff  (b+1)*L - 1 <= i - w;
 *   output       : one softmax over everything row i sees, with scores
 *                  scale * q_i . k;  O_i = sum p v,
 *                  LSE_i = m_i + ln(sum exp(s - m_i))   (natural log).
 *
 * Decode evaluates the same for the single row i = ctx-1 of a cache, split
 * into chunks whose partial results are merged by log-sum-exp -- the
 * single-GPU form of the softmax-statistics aggregation of Ring Attention on
 * the page "Training at 1M+ Token Context: Ring Attention, YaRN, NTK-Aware
 * Scaling GPU Cost" (Ring Attention paragraph).
 *
 * Conventions for every entry point
 *  - Tensors are dense, row-major, and live in device memory unless stated.
 *      Q, O      [B][Hq][n][d]      K, V        [B][Hkv][n][d]
 *      Kbar,Vbar [B][Hkv][G][d]     LSE         [B][Hq][n]   (float32)
 *      decode q, O [B][Hq][d]       decode LSE  [B][Hq]      (float32)
 *      caches    [B][Hkv][ctx][d]
 *    Query head h reads KV head h / (Hq / Hkv).
 *  - Device pointers must be 16-byte aligned.
 *  - The caller owns every buffer.  The library allocates no device memory,
 *    keeps no pointer after returning, and holds no state between calls.
 *  - Compute calls are asynchronous: kernels are enqueued on `stream` (a
 *    hipStream_t; NULL = the null stream).  Results are valid once the
 *    caller synchronises that stream.  Calls on different streams that
 *    write the same buffers race.
 *  - Arguments are validated before anything is enqueued; on any error
 *    nothing is written and nothing is launched.  Error detail is in
 *    msa_last_error() (thread-local).  A launch failure reported by the HIP
 *    runtime returns MSA_ERR_HIP.
 *  - Inputs with NaN or Inf give unspecified results.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 1: pooling, prefill, static decode and plans.  2: adds incremental
 * decode (msa_decode_fwd_varlen, msa_append_kv, msa_plan_decode_varlen, and
 * the paged msa_decode_fwd_paged, msa_append_kv_paged),
 * the backward (msa_attn_bwd_workspace_size, msa_attn_bwd) and block-sparse
 * lists (msa_attn_fwd_blocksparse). */
#define MSA_ABI_VERSION 3

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment ...      */
  MSA_ERR_UNSUPPORTED = 2, /* valid but not implemented (head_dim, dtype)    */
  MSA_ERR_WORKSPACE = 3,   /* decode workspace too small                      */
  MSA_ERR_HIP = 4,         /* the HIP runtime reported an error               */
  MSA_ERR_CAPACITY = 5     /* output array of a plan query too small          */
} msa_status;

typedef enum { MSA_DTYPE_F32 = 0, MSA_DTYPE_BF16 = 1 } msa_dtype;

/* Decode schedule (see msa_decode_fwd): chosen from the problem's shape, or
 * forced. */
typedef enum { MSA_DECODE_AUTO = 0, MSA_DECODE_SPLIT = 1, MSA_DECODE_FUSED = 2 } msa_decode_schedule;

/* Prefill problem.  head_dim in {64, 128}.  window >= 1 (a window >= n is
 * plain causal attention).  num_landmarks G >= 0; G > 0 requires n % G == 0.
 * in_dtype is the dtype of Q, K, V, Kbar, Vbar; out_dtype that of O
 * (bf16 inputs may write float32 O; float32 inputs write float32 O).
 * With bf16 inputs one head's K or V, seq_len*head_dim*2 bytes, must be
 * < 2 GiB (MSA_ERR_UNSUPPORTED otherwise). */
typedef struct {
  int32_t batch;
  int32_t heads_q;
  int32_t heads_kv;
  int32_t seq_len;
  int32_t head_dim;
  int32_t window;
  int32_t num_landmarks;
  float scale; /* score scale, usually 1/sqrt(head_dim); finite and > 0 */
  int32_t in_dtype;  /* msa_dtype */
  int32_t out_dtype; /* msa_dtype */
} msa_attn_desc;

/* Decode problem: one new query per sequence at position ctx_len-1, whose
 * own K/V are already in the cache.  Landmarks are those of the whole cache
 * (L = ctx_len / G).  num_splits >= 1 chunks of the visible list.  Query
 * heads per KV head (heads_q / heads_kv) must be <= 16. */
typedef struct {
  int32_t batch;
  int32_t heads_q;
  int32_t heads_kv;
  int32_t ctx_len;
  int32_t head_dim;
  int32_t window;
  int32_t num_landmarks;
  int32_t num_splits;
  float scale; /* finite and > 0 */
  int32_t in_dtype;
  int32_t out_dtype;
  int32_t schedule; /* msa_decode_schedule */
} msa_decode_desc;

/* Landmark pooling.  Reads K, V [B][Hkv][n][d] (n = desc->seq_len) and
 * writes Kbar, Vbar [B][Hkv][G][d]: the mean of each block of L = n/G rows,
 * accumulated in float32 in a fixed order (deterministic) and rounded to
 * nearest-even into in_dtype.  Fields read: batch, heads_kv, seq_len,
 * head_dim, num_landmarks, in_dtype.  G == 0 is a no-op (pointers may be
 * NULL).  For a decode cache pass an attn desc with seq_len = ctx_len.
 * Source: the landmark definition above (mean of K and V over each block). */
msa_status msa_pool_landmarks(const msa_attn_desc* desc, const void* K, const void* V,
                              void* Kbar, void* Vbar, void* stream);

/* Sparse-attention prefill: O and LSE for every row of every query head.
 * Kbar/Vbar are the landmarks (from msa_pool_landmarks, or any values of the
 * same layout); they may be NULL when G == 0.  LSE may be NULL.
 * Work is enumerated block-sparsely: each workgroup visits only the key
 * tiles of its rows' windows and the landmark tiles that some row sees.
 * Source: the operation defined at the top of this file; tiling as in
 * "What is Flash-MSA Sparse Attention in GPU Clusters?" and the Flash
 * Attention paragraph of "Training at 1M+ Token Context ...". */
msa_status msa_attn_fwd(const msa_attn_desc* desc, const void* Q, const void* K, const void* V,
                        const void* Kbar, const void* Vbar, void* O, float* LSE, void* stream);

/* ---- Block-sparse lists: the same tiled pass driven by explicit per-block
 * lists instead of the window + landmark closed form.  The pages drive
 * block-sparse kernels by per-block index lists with counts ("Sparse
 * Attention GPU Cluster Implementation: What Actually Works", section on
 * the kernel that applies the pattern; 64-token blocks) and describe
 * patterns such as 128-token blocks each attending to 16 others ("Million
 * Token Context Window Optimization: What Actually Works", indexing
 * section). ---- */

#define MSA_LIST_QUERY_BLOCK 128 /* rows per query block of a list     */
#define MSA_LIST_KEY_BLOCK 64    /* keys per listed key block           */

/* O and LSE where query block t (rows t*128 .. t*128+127) of query head h
 * in batch b sees every key of the key blocks listed for it -- block k
 * covers keys k*64 .. k*64+63, clipped at n -- and, with causal = 1, only
 * keys j <= i; one softmax over what a row sees.  Lists live in device
 * memory: block_counts int32 [B][Hq][T] (T = ceil(n/128)), block_indices
 * int32 [B][Hq][T][max_blocks]; entry c < count of a list is its c-th
 * block (order free).  Counts are clamped to [0, max_blocks] on the
 * device; an index outside [0, ceil(n/64)) is skipped; a block listed
 * twice is seen twice.  A row that sees nothing gets O = 0, LSE = -inf.
 * desc fields read: batch, heads_q, heads_kv, seq_len, head_dim, scale,
 * in_dtype (bf16 only, MSA_ERR_UNSUPPORTED otherwise), out_dtype; window
 * and num_landmarks are not read.  LSE may be NULL.  Other conventions as
 * for msa_attn_fwd. */
msa_status msa_attn_fwd_blocksparse(const msa_attn_desc* desc, const int32_t* block_counts,
                                   const int32_t* block_indices, int32_t max_blocks, int32_t causal,
                                   const void* Q, const void* K, const void* V, void* O, float* LSE,
                                   void* stream);

/* ---- Backward of msa_attn_fwd.  The pages train at these lengths
 * ("Training at 1M+ Token Context: Ring Attention, YaRN, NTK-Aware Scaling
 * GPU Cost", Flash Attention and Block-Sparse Flash Attention paragraphs)
 * but do not write the backward out; it is the chain rule through the
 * operation defined at the top of this file:
 *   P = exp(S - LSE) over the visible entries,  dP = dO V_vis^T,
 *   D_i = sum_d dO_i O_i,  dS = P (dP - D),
 *   dQ = scale dS K_vis,  dK_vis = scale dS^T Q,  dV_vis = P^T dO,
 * summed over the query heads that share a KV head, and each landmark's
 * gradient spread over the L rows of its block with weight 1/L (the
 * landmark is their mean).  dK, dV are the total gradients of K, V through
 * both the window and the landmark paths. ---- */

/* Bytes of device workspace msa_attn_bwd needs for `desc`.  Host only. */
msa_status msa_attn_bwd_workspace_size(const msa_attn_desc* desc, size_t* bytes);

/* Gradients of the prefill.  Inputs: Q, K, V, Kbar, Vbar as given to
 * msa_attn_fwd (Kbar/Vbar may be NULL when G == 0), its outputs O and LSE
 * (LSE required), and dO [B][Hq][n][d].  in_dtype must be bf16
 * (MSA_ERR_UNSUPPORTED otherwise); O and dO are bf16.  Outputs dQ
 * [B][Hq][n][d] and dK, dV [B][Hkv][n][d] in out_dtype (bf16 or f32); every
 * element is written (no accumulation into the caller's buffers).  The
 * workspace is caller-owned scratch of at least msa_attn_bwd_workspace_size
 * bytes.  Arithmetic: bf16 matrix-core products with float32 accumulation;
 * P and dS are rounded to bf16 as operands; each output element is computed
 * by one workgroup in a fixed order (deterministic, no atomics). */
msa_status msa_attn_bwd(const msa_attn_desc* desc, const void* Q, const void* K, const void* V,
                        const void* Kbar, const void* Vbar, const void* O, const float* LSE, const void* dO,
                        void* workspace, size_t workspace_bytes, void* dQ, void* dK, void* dV,
                        void* stream);

/* Bytes of device workspace msa_decode_fwd (and its _varlen and _paged
 * forms) needs: num_splits * batch * heads_q * (head_dim + 1) * 4.  Host
 * only; the 2 GiB limit of contiguous caches is not checked here. */
msa_status msa_decode_workspace_size(const msa_decode_desc* desc, size_t* bytes);

/* Decode with split-KV partial softmax and an LSE merge.
 * The ordered visible list of row ctx-1 (visible landmarks in block order,
 * then the window keys ascending; E entries) is cut into num_splits chunks
 * of s = ceil(E / num_splits) entries; chunk c covers [c*s, min(E,(c+1)*s)).
 * Each chunk's normalised output o_c and log-sum-exp lse_c (an empty chunk
 * has lse_c = -inf, o_c = 0) are merged:
 * LSE = ln sum_c exp(lse_c), O = sum_c exp(lse_c - LSE) o_c.
 * Two schedules compute this, with the same results up to float32 rounding
 * of the merge:
 *  - split: one wavefront per chunk writes (o_c, lse_c) to the workspace --
 *    o_c float32 [S][B][Hq][d] at offset 0, then lse_c float32 [S][B][Hq] --
 *    and a second kernel merges them;
 *  - fused: one workgroup per (sequence, KV head) streams all its chunks,
 *    merging the partials on chip; the workspace is not written.
 * With schedule = MSA_DECODE_AUTO the fused schedule is used when
 * batch*heads_kv >= 2 x (compute units) and num_splits >= 4;
 * MSA_DECODE_SPLIT or MSA_DECODE_FUSED forces one of them (any other value:
 * MSA_ERR_INVALID_ARG).
 * The workspace is caller-owned scratch of at least
 * msa_decode_workspace_size() bytes (required by both schedules).
 * Kbar/Vbar: landmarks of the caches (NULL if G == 0).  LSE may be NULL.
 * in_dtype must be bf16 (MSA_ERR_UNSUPPORTED otherwise); out_dtype bf16 or
 * f32.  One head's cache, ctx_len*head_dim*2 bytes, must be < 2 GiB
 * (MSA_ERR_UNSUPPORTED otherwise). */
msa_status msa_decode_fwd(const msa_decode_desc* desc, const void* q, const void* Kcache,
                          const void* Vcache, const void* Kbar, const void* Vbar, void* workspace,
                          size_t workspace_bytes, void* O, float* LSE, void* stream);

/* Bytes of the library's own device array behind msa_decode_fwd_noalloc. */
#define MSA_NOALLOC_SCRATCH_BYTES (32u << 20)

/* msa_decode_fwd without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops that
 * must not call hipMalloc, harnesses that forbid it.  Arguments, results
 * and errors are those of msa_decode_fwd minus the workspace; the caller
 * still provides q, the caches, the landmarks, O and LSE.  The split
 * schedule's per-chunk partials go to a static device array inside the
 * library, MSA_NOALLOC_SCRATCH_BYTES on every GPU the library runs on, held
 * until the process ends; a problem that runs the split schedule and needs
 * more (num_splits * batch * heads_q * (head_dim + 1) * 4 bytes) is
 * rejected with MSA_ERR_WORKSPACE before any launch (the fused schedule
 * needs none).  Every call on a GPU shares that GPU's array, which keeps the
 * last call's contents: calls that overlap on one GPU (different streams,
 * threads) race, and the caller must serialise them.  Nothing in the array
 * needs clearing: each call overwrites every partial its merge reads.  The
 * array's device address is looked up once per device, on the first call
 * with that device current.  Calls no hipMalloc, hipFree or allocating
 * routine. */
msa_status msa_decode_fwd_noalloc(const msa_decode_desc* desc, const void* q, const void* Kcache,
                                  const void* Vcache, const void* Kbar, const void* Vbar, void* O,
                                  float* LSE, void* stream);

/* ---- Incremental decode: sequences of different lengths in one cache,
 * grown one token per step.  The pages run generation after a long prompt
 * with the KV cache as the per-token state ("Million Token Context Window
 * Optimization: What Actually Works", sections "Flash MSA vs Flash
 * Attention: The real difference" and "Benchmarking your optimization").
 * Here the cache of every sequence has the same capacity C = desc->ctx_len
 * rows ([B][Hkv][C][d], as above), landmark blocks have the fixed length
 * L = C / G (G = desc->num_landmarks slots per sequence, [B][Hkv][G][d]),
 * and a landmark is the mean of its block once the block's L rows are in
 * the cache.  The visibility rule is the one at the top of this file, so a
 * visible landmark is always a complete block. ---- */

/* Decode of sequence b at its own length n_b = ctx_lens[b] (int32 device
 * array [B], 4-byte aligned): its query, at position n_b-1, sees the window
 * keys n_b-w .. n_b-1 and the landmarks b' with (b'+1)*L - 1 <= n_b-1-w.
 * Its visible list is chunked, computed and merged exactly as in
 * msa_decode_fwd (same schedules and schedule field, same workspace size and
 * layout).  Only rows < n_b of the caches and
 * landmark slots < (n_b - w)/L are read.  n_b is clamped to [0, C] on the
 * device (the host cannot read it); n_b = 0 gives O = 0 and LSE = -inf.
 * With every n_b = C this is msa_decode_fwd.  Other arguments and errors as
 * for msa_decode_fwd. */
msa_status msa_decode_fwd_varlen(const msa_decode_desc* desc, const int32_t* ctx_lens, const void* q,
                                 const void* Kcache, const void* Vcache, const void* Kbar,
                                 const void* Vbar, void* workspace, size_t workspace_bytes, void* O,
                                 float* LSE, void* stream);

/* Append one token per sequence: k_new, v_new [B][Hkv][d] (bf16) are stored
 * at row p_b = positions[b] (int32 device array [B], 4-byte aligned) of
 * Kcache and Vcache; when p_b + 1 is a multiple of L, landmark slot
 * (p_b + 1)/L - 1 of Kbar and Vbar is set to the mean of that block's L
 * rows, computed by the same code and in the same order as
 * msa_pool_landmarks, so its bits equal pooling the finished cache.  A
 * position outside [0, C) leaves sequence b untouched (use -1 for an idle
 * slot).  Rows other than p_b and the other landmark slots are not written.
 * Fields read: batch, heads_kv, ctx_len (= C), head_dim, num_landmarks,
 * in_dtype (bf16 only, MSA_ERR_UNSUPPORTED otherwise).  Kbar/Vbar may be
 * NULL when G == 0.  The caller appends position n_b before decoding with
 * length n_b + 1 on the same stream. */
msa_status msa_append_kv(const msa_decode_desc* desc, const int32_t* positions, const void* k_new,
                         const void* v_new, void* Kcache, void* Vcache, void* Kbar, void* Vbar,
                         void* stream);

/* Paged caches (the vLLM-style "PagedAttention" the page "Sparse Attention
 * GPU Cluster Implementation: What Actually Works", FAQ, names for
 * single-node serving): K and V rows live in pools of fixed-size pages,
 * Kpages, Vpages [num_pages][Hkv][page_size][d] bf16, and sequence b's
 * logical page p (rows p*page_size .. +page_size-1) is physical page
 * block_table[b][p] (int32 device array [B][C/page_size], C =
 * desc->ctx_len, the capacity).  page_size is a power of two in [32, 2^20]
 * dividing C.  Landmarks stay contiguous, [B][Hkv][G][d].  A page id
 * outside [0, num_pages) is never dereferenced: decode reads page 0 in its
 * place (the result for that sequence is then meaningless) and append
 * leaves that sequence untouched.  Pools are addressed with 64-bit offsets
 * (no 2 GiB limit).  Otherwise as msa_decode_fwd_varlen / msa_append_kv,
 * with the same results for the same rows. */
msa_status msa_decode_fwd_paged(const msa_decode_desc* desc, int32_t page_size, int32_t num_pages,
                                const int32_t* block_table, const int32_t* ctx_lens, const void* q,
                                const void* Kpages, const void* Vpages, const void* Kbar,
                                const void* Vbar, void* workspace, size_t workspace_bytes, void* O,
                                float* LSE, void* stream);

msa_status msa_append_kv_paged(const msa_decode_desc* desc, int32_t page_size, int32_t num_pages,
                               const int32_t* block_table, const int32_t* positions, const void* k_new,
                               const void* v_new, void* Kpages, void* Vpages, void* Kbar, void* Vbar,
                               void* stream);

/* ---- Host-only introspection: the exact schedule the kernels use.  These
 * make no HIP call and need no GPU; all pointers are host memory. ---- */

/* Per row i in [0, n): win_lo[i] = lowest visible window key, lm_count[i] =
 * number of visible landmarks (they are always landmarks 0..lm_count-1). */
msa_status msa_plan_rows(const msa_attn_desc* desc, int32_t* win_lo, int32_t* lm_count);

/* The tiles msa_attn_fwd visits, in kernel order, as int32 quadruples
 * (query_tile, kind, tile, interior): kind 0 = landmark tile (landmarks
 * tile*bn .. tile*bn+bn-1), 1 = window key tile (keys tile*bn ..);
 * interior = 1 when every (row, key) of the tile is visible so the kernel
 * applies no mask.  Query tile t covers rows t*bm .. min(n, t*bm+bm)-1.
 * Writes *count (always) and *bm, *bn; writes `out` only if capacity >=
 * *count (else MSA_ERR_CAPACITY); out may be NULL to query the count. */
msa_status msa_plan_tiles(const msa_attn_desc* desc, int32_t* out, int64_t capacity,
                          int64_t* count, int32_t* bm, int32_t* bn);

/* Decode schedule: chunk_bounds[0..num_splits] (entry offsets of the
 * chunks), *lm_visible = visible landmarks of row ctx-1, *entries = E. */
msa_status msa_plan_decode(const msa_decode_desc* desc, int32_t* chunk_bounds,
                           int32_t* lm_visible, int32_t* entries);

/* Decode schedule of one sequence of ctx tokens (0 <= ctx <= desc->ctx_len)
 * as msa_decode_fwd_varlen runs it: outputs as for msa_plan_decode. */
msa_status msa_plan_decode_varlen(const msa_decode_desc* desc, int32_t ctx, int32_t* chunk_bounds,
                                  int32_t* lm_visible, int32_t* entries);

/* Static description of a status code. */
const char* msa_status_string(msa_status s);
/* Detail of the last error on the calling thread ("" if none). */
const char* msa_last_error(void);
/* MSA_ABI_VERSION of the loaded library. */
int32_t msa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MSA_H_ */
