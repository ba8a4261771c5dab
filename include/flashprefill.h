/*
 * flashprefill.h -- block-sparse causal prefill attention for MI355X (gfx950).
 *
 * The method (FlashPrefill, gist.science technical summary, section 2; and
 * FlashPrefill V2, abstract):
 *   1. block-mean pooling of Q and K ("Approximation par Blocs", 2.A), and of
 *      V for the mean-correction term;
 *   2. pooled block logits s[h,I,J] = sigma * q_bar[h,I] . k_bar[h/g,J], J <= I,
 *      whose row softmax is the block score (2.A, fused 2D reduction: the
 *      L x L/B score matrix never exists, and the L/B x L/B one stays on chip);
 *   3. max-based dynamic threshold (2.B, threshold equation):
 *      keep J iff Score[I,J] >= alpha * max_{J' <= I} Score[I,J'],
 *      evaluated as s - max(s) >= ln(alpha);
 *   4. one ascending list of kept KV blocks per (query head, query block),
 *      walked by index so skipped blocks cost nothing (2.C, physical skip);
 *   5. flash attention over the kept blocks, plus the mean-correction term of
 *      V2 (abstract): every skipped block J < I enters row i's softmax as one
 *      entry with logit sigma * q_i . k_bar_J + ln n_J and value v_bar_J.
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers unless the name ends in _host.  Device
 *     buffers are contiguous, row-major and 16-byte aligned.
 *   - bf16 tensors are IEEE bfloat16; fp8 tensors are OCP e4m3fn bytes.
 *   - Q is [S, Hq, d] token-major; K and V are [S, Hkv, d]; query head h reads
 *     KV head h / (Hq / Hkv).
 *   - B = block_size; nB = ceil(S / B); n_J = tokens in block J.
 *   - Block lists: kv_idx holds, for each sequence, a triangular region of
 *     Hq * nB * (nB + 1) / 2 int32; the list of (h, I) starts at
 *     h * nB * (nB + 1) / 2 + I * (I + 1) / 2 and has capacity I + 1.  kv_cnt
 *     holds Hq * nB int32 per sequence, entry h * nB + I = list length.  In a
 *     batch, sequence b's regions follow sequence b-1's.
 *   - stream is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on that stream: it never allocates, frees or synchronises,
 *     and keeps no pointer after it returns.  The caller owns every buffer and
 *     keeps it alive until the stream has passed the work.
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued.  On a non-zero return nothing was launched and no output was
 *     written; fp_last_error() then describes the problem.  Faults inside a
 *     kernel surface at the caller's next synchronisation.
 */
#ifndef FLASHPREFILL_H
#define FLASHPREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define FP_OK                   0
#define FP_INVALID_ARGUMENT     1   /* NULL / misaligned pointer, bad size, alpha outside [0,1] ... */
#define FP_UNSUPPORTED          2   /* a valid request this build does not implement (e.g. d = 96) */
#define FP_WORKSPACE_TOO_SMALL  3
#define FP_DEVICE_ERROR         4   /* a launch was rejected by the HIP runtime */

/* Element type of the q/k/v that an attention call reads. */
#define FP_DTYPE_BF16        0
#define FP_DTYPE_FP8_E4M3FN  1

typedef struct {
    int32_t num_q_heads;      /* Hq, a multiple of num_kv_heads */
    int32_t num_kv_heads;     /* Hkv >= 1 */
    int32_t head_dim;         /* d: 64 or 128 */
    int32_t block_size;       /* B: 64 or 128 (query block = KV block = pooling block) */
    float   alpha;            /* threshold ratio, 0 <= alpha <= 1; 0 keeps every causal block */
    float   softmax_scale;    /* sigma for scores and attention; <= 0 means 1/sqrt(d) */
    int32_t mean_correction;  /* 1: add the mean-correction entries of skipped blocks */
    int32_t dtype;            /* FP_DTYPE_*: element type of q/k/v in the attention call */
    int32_t shared_selection; /* 0: one list per query head (steps 1-4 as written);
                                 1: the g = Hq/Hkv query heads of a KV head share one list,
                                 the union of their own lists (every head of a group then
                                 runs on every tile fetched for the group);
                                 2: they share one list scored from the group-pooled query,
                                 the mean of the g heads' q_bar rows, against the KV head's
                                 k_bar (steps 2-4 once per KV head).  pooled_q stays per
                                 query head in every mode. */
    int32_t query_probes;     /* 0: q_bar is the mean of every query of the block (step 1);
                                 P dividing block_size: the mean of the skeleton queries at
                                 offsets 0, st, 2 st, ... of the block, st = block_size / P
                                 (FlashPrefill 2.A); a partial block keeps the probes it has */
} fp_params;

/*
 * Selection: steps 1-4 for one sequence of length seqlen (FlashPrefill 2.A-2.C).
 *   q [S,Hq,d], k [S,Hkv,d], v [S,Hkv,d]: bf16, whatever params->dtype says
 *     (fp8 attention selects on the bf16 data).  v may be NULL when pooled_v
 *     and pooled_kv_bf16 both are (then V is not read).
 *   pooled_q [Hq,nB,d], pooled_k [Hkv,nB,d], pooled_v [Hkv,nB,d]: fp32 outputs,
 *     means over the valid tokens of each block.  pooled_v may be NULL.
 *   pooled_kv_bf16 [2,Hkv,nB,d] bf16 output or NULL: the K and V block means
 *     rounded to bf16 (nearest even), K_bar first.  The mean correction in
 *     fp_sparse_prefill_fwd reads it.
 *   kv_idx, kv_cnt: int32 outputs in the list layout above.
 * Lists are ascending and never empty: the row's best block always passes.
 */
int fp_select_blocks(const fp_params* params,
                     const void* q, const void* k, const void* v, int32_t seqlen,
                     float* pooled_q, float* pooled_k, float* pooled_v, void* pooled_kv_bf16,
                     int32_t* kv_idx, int32_t* kv_cnt, void* stream);

/*
 * fp8 inputs in one pass (FlashPrefill V2 abstract: FP8 inference): reads the
 * bf16 q, k, v of one sequence once and writes
 *   - the e4m3 codes and fp32 scales fp_sparse_prefill_fwd takes in fp8 mode:
 *     per (head, block) scale = amax / 448 of the block's values (1 for an
 *     all-zero block), code = OCP E4M3 ("fn") value nearest to
 *     clamp(x / scale, -448, 448), ties to even; both divisions are correctly
 *     rounded fp32;
 *   - the block means, and then the lists of steps 1-4 exactly as
 *     fp_select_blocks would (selection from the bf16 data).
 *   params: dtype must be FP_DTYPE_FP8_E4M3FN (the attention that follows).
 *   q [S,Hq,d], k, v [S,Hkv,d] bf16.
 *   q8 [S,Hq,d], k8, v8 [S,Hkv,d] uint8 codes, 8-byte aligned (written).
 *   q_scale [Hq,nB], k_scale, v_scale [Hkv,nB] fp32 (written).
 *   pooled_q, pooled_k, pooled_kv_bf16, kv_idx, kv_cnt: as for fp_select_blocks
 *     (pooled_kv_bf16 required when params->mean_correction is 1).
 */
int fp_select_blocks_fp8(const fp_params* params, const void* q, const void* k, const void* v,
                         int32_t seqlen, void* q8, void* k8, void* v8,
                         float* q_scale, float* k_scale, float* v_scale,
                         float* pooled_q, float* pooled_k, void* pooled_kv_bf16,
                         int32_t* kv_idx, int32_t* kv_cnt, void* stream);

/*
 * Attention: step 5 for one sequence, over the lists from fp_select_blocks
 * (FlashPrefill 2.C; V2 abstract for the correction, PackGQA and FP8).
 *   q [S,Hq,d], k, v [S,Hkv,d]: bf16, or e4m3fn bytes when params->dtype is
 *     FP_DTYPE_FP8_E4M3FN; then q_scale [Hq,nB], k_scale, v_scale [Hkv,nB] are
 *     fp32 per-(head, block) scales, x = code * scale, and block = block_size.
 *     The scale pointers are ignored for bf16.
 *   kv_idx, kv_cnt: lists in the layout above.
 *   pooled_kv_bf16: bf16 [2,Hkv,nB,d] block means (K_bar then V_bar) from
 *     fp_select_blocks; required when params->mean_correction is 1, ignored
 *     otherwise.
 *   out [S,Hq,d] bf16 (written); lse [Hq,S] fp32 natural-log sum of exp of
 *     each row's logits (written when not NULL).
 */
int fp_sparse_prefill_fwd(const fp_params* params,
                          const void* q, const void* k, const void* v,
                          const float* q_scale, const float* k_scale, const float* v_scale,
                          int32_t seqlen, const int32_t* kv_idx, const int32_t* kv_cnt,
                          const void* pooled_kv_bf16,
                          void* out, float* lse, void* stream);

/*
 * Continuous batch over a paged KV cache: steps 1-5 for `batch` requests
 * (FlashPrefill V2 abstract: paged KV cache and continuous batching).  Each
 * request is a pure prefill (query length = KV length = its length); blocks
 * start at each request's first token and no request sees another's tokens.
 *   q [T,Hq,d] bf16, T = cu_seqlens_host[batch]: requests packed back to back.
 *   k_cache, v_cache [num_pages, page_size, Hkv, d] bf16.  Token t of request b
 *     lives in page block_table[b * max_pages_per_seq + t / page_size], slot
 *     t % page_size.  block_size must be a multiple of page_size.  Page ids
 *     outside [0, num_pages) read as zeros.
 *   cu_seqlens_host [batch+1] int32, host memory read during the call:
 *     0 = cu[0] <= cu[1] <= ... (request b is tokens cu[b] .. cu[b+1]-1 of q).
 *   kv_idx, kv_cnt: list outputs, regions of consecutive requests concatenated
 *     (sizes from fp_index_capacity / fp_count_entries).
 *   workspace: device scratch of at least fp_varlen_workspace_bytes() bytes
 *     (pooled means); contents on return are unspecified.
 *   out [T,Hq,d] bf16, lse [Hq,T] fp32 or NULL.
 * bf16 only (FP_UNSUPPORTED for fp8; see fp_sparse_prefill_varlen_paged_fp8).
 * batch <= FP_MAX_BATCH.
 */
#define FP_MAX_BATCH 128
int fp_sparse_prefill_varlen_paged(const fp_params* params, const void* q,
                                   const void* k_cache, const void* v_cache,
                                   int32_t page_size, int32_t num_pages,
                                   const int32_t* block_table, int32_t max_pages_per_seq,
                                   const int32_t* cu_seqlens_host, int32_t batch, int32_t* kv_idx, int32_t* kv_cnt,
                                   void* workspace, size_t workspace_bytes,
                                   void* out, float* lse, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation as fp_sparse_prefill_varlen_paged, with the workspace taken
 * from a library-owned device array of FP_NOALLOC_SCRATCH_BYTES per GPU
 * instead of a caller's buffer.  The array lives in the library's code object
 * on every GPU the library runs on, until the process ends.  The call
 * allocates nothing, frees nothing and calls no allocating routine; the
 * caller still passes (and owns) every input and output.
 *   All arguments: as for fp_sparse_prefill_varlen_paged, without workspace.
 *   FP_WORKSPACE_TOO_SMALL when the batch needs more pooled-mean scratch than
 *     FP_NOALLOC_SCRATCH_BYTES (fp_varlen_workspace_bytes gives the need);
 *     nothing is launched then.
 * Every call on one GPU shares that GPU's array and overwrites it (it holds
 * the last call's pooled means; nothing in it needs to start at zero).  Calls
 * that overlap on one GPU (other streams, other threads) race on it: the
 * caller orders them, e.g. by issuing them on one stream.
 */
#define FP_NOALLOC_SCRATCH_BYTES (64u << 20)
int fp_sparse_prefill_varlen_paged_noalloc(const fp_params* params, const void* q,
                                           const void* k_cache, const void* v_cache,
                                           int32_t page_size, int32_t num_pages,
                                           const int32_t* block_table, int32_t max_pages_per_seq,
                                           const int32_t* cu_seqlens_host, int32_t batch,
                                           int32_t* kv_idx, int32_t* kv_cnt,
                                           void* out, float* lse, void* stream);

/*
 * fp8 inference over a paged batch (FlashPrefill V2 abstract: FP8 inference,
 * paged KV cache and continuous batching): the requests of
 * fp_sparse_prefill_varlen_paged, with params->dtype = FP_DTYPE_FP8_E4M3FN.
 * One pass over the bf16 data writes the e4m3 codes with one scale per
 * (head, block) (the recipe of fp_select_blocks_fp8) and the block means;
 * selection runs on the means of the bf16 data; attention runs on the codes,
 * reading K and V from the e4m3 pages.
 *   q, k_cache, v_cache, page_size, num_pages, block_table,
 *     max_pages_per_seq, cu_seqlens_host, batch: as for
 *     fp_sparse_prefill_varlen_paged (bf16 inputs).
 *   k8_cache, v8_cache [num_pages, page_size, Hkv, d] uint8 e4m3 codes, 16-byte
 *     aligned (written): the fp8 paged cache.  Each token's codes go to the
 *     place its bf16 values have in k_cache / v_cache; pages no request
 *     names are left untouched.
 *   k_scale_cache, v_scale_cache [num_pages, Hkv] fp32 (written): the scale of
 *     head h of a block sits at the entry [p][h] of the page p that holds the
 *     block's first token.
 *   kv_idx, kv_cnt: list outputs, as for fp_sparse_prefill_varlen_paged.
 *   workspace: at least fp_varlen_workspace_bytes() bytes for these params
 *     (with dtype fp8 it includes the Q codes and scales).
 *   out [T,Hq,d] bf16, lse [Hq,T] fp32 or NULL.
 * FP_INVALID_ARGUMENT when params->dtype is not fp8.
 */
int fp_sparse_prefill_varlen_paged_fp8(const fp_params* params, const void* q,
                                       const void* k_cache, const void* v_cache,
                                       int32_t page_size, int32_t num_pages,
                                       const int32_t* block_table, int32_t max_pages_per_seq,
                                       const int32_t* cu_seqlens_host, int32_t batch,
                                       void* k8_cache, void* v8_cache,
                                       float* k_scale_cache, float* v_scale_cache,
                                       int32_t* kv_idx, int32_t* kv_cnt,
                                       void* workspace, size_t workspace_bytes,
                                       void* out, float* lse, void* stream);

/*
 * Chunked prefill over a paged KV cache (FlashPrefill V2 abstract and the
 * authors' post: an attention backend with paged KV and continuous
 * batching).  Request b brings q_len = cu_seqlens_q_host[b+1] -
 * cu_seqlens_q_host[b] new queries at the end of a context of
 * kv_len = kv_lens_host[b] tokens whose keys and values, the new ones
 * included, are already in the cache; 0 <= q_len <= kv_len.  Blocks are
 * counted from the start of the context.  Query row r of request b sits at
 * position P0 + r, P0 = kv_len - q_len, and sees every key at or before it
 * (bottom-right causal alignment); its query block I = position / block_size
 * is pooled over the chunk's queries in it (a chunk may start inside a
 * block: that block then pools only the chunk's queries), scored against
 * the block means of the whole context and thresholded as in steps 1-4, and
 * attends as in step 5.  When P0 is a multiple of block_size a chunk's
 * output equals the last q_len rows of a prefill of the whole context;
 * otherwise every row past its first query block still does.  Skeleton
 * queries (query_probes > 0) need P0 to be a multiple of block_size, else
 * FP_UNSUPPORTED.
 *   q [T,Hq,d] bf16, T = cu_seqlens_q_host[batch]: the chunks packed back to back.
 *   k_cache, v_cache, page_size, num_pages, block_table, max_pages_per_seq: as
 *     for fp_sparse_prefill_varlen_paged; block_table covers kv_len tokens.
 *   kv_lens_host [batch] int32, host memory read during the call.
 *   pooled_cache: NULL, or fp32 [2, num_pages, Hkv, d] owned by the caller
 *     and kept between calls: entry [0|1][p][h] holds the K_bar | V_bar of
 *     head h of the block whose first token lives in page p.  Every block
 *     pooled in the call is written there.
 *   prefix_pooled: 1 = the blocks before each chunk were pooled into
 *     pooled_cache by earlier calls (same pages, same contents): their means
 *     are read from it instead of from the cache pages; 0 = pool them now.
 *     1 requires pooled_cache.
 *   kv_idx, kv_cnt: lists of the chunk's query blocks only: request b's
 *     region holds, for each head h, the rows I = first .. nb-1 (first =
 *     floor(P0 / block_size), or nb for an empty chunk; nb = ceil(kv_len /
 *     block_size)), row I
 *     with capacity I + 1; kv_cnt is [Hq, nb - first] per request.  Regions
 *     of consecutive requests are concatenated.  Sizes from fp_chunked_sizes.
 *   workspace: at least the bytes fp_chunked_sizes gives; contents on return
 *     are unspecified.
 *   out [T,Hq,d] bf16, lse [Hq,T] fp32 or NULL (rows of the chunks).
 * bf16 (fp8 attention: fp_sparse_prefill_chunked_paged_fp8).  batch <= FP_MAX_BATCH.
 */
int fp_sparse_prefill_chunked_paged(const fp_params* params, const void* q,
                                    const void* k_cache, const void* v_cache,
                                    int32_t page_size, int32_t num_pages,
                                    const int32_t* block_table, int32_t max_pages_per_seq,
                                    const int32_t* cu_seqlens_q_host, const int32_t* kv_lens_host,
                                    int32_t batch, float* pooled_cache, int32_t prefix_pooled,
                                    int32_t* kv_idx, int32_t* kv_cnt,
                                    void* workspace, size_t workspace_bytes,
                                    void* out, float* lse, void* stream);

/*
 * Chunked prefill with fp8 attention (FlashPrefill V2 abstract: FP8
 * inference, and the attention backend with paged KV and continuous
 * batching of the authors' post).  The chunk, its context, the pooled cache
 * and the lists are those of fp_sparse_prefill_chunked_paged, bit for bit:
 * the block means come from the bf16 pages (the chunks' blocks in the same
 * pass that encodes them, summed in the pooling kernel's order), and the
 * pooled cache receives the same entries.  Attention reads e4m3 pages kept beside
 * them, in the form fp_sparse_prefill_varlen_paged_fp8 writes: codes in the
 * layout of the bf16 pages and one fp32 scale per (page, KV head) at the
 * entry of the page that holds a block's first token.  The call encodes the
 * query blocks first .. nb-1 of each request (blockwise absmax / 448 scales,
 * OCP E4M3 codes): K and V of those blocks whole, from the bf16 pages (the
 * tokens of block first that precede the chunk included), Q over the chunk's
 * queries in each block (workspace).  Blocks 0 .. first-1 are read as they
 * stand, so they must hold the codes of earlier calls of this entry (or of
 * fp_sparse_prefill_varlen_paged_fp8) over the same tokens.  The result then
 * equals fp8 attention over the whole context's blockwise codes, with the
 * chunk's Q blocks encoded over the chunk's queries.
 *   q, k_cache, v_cache, page_size, num_pages, block_table,
 *   max_pages_per_seq, cu_seqlens_q_host, kv_lens_host, batch, pooled_cache,
 *   prefix_pooled, kv_idx, kv_cnt, out, lse: as for
 *   fp_sparse_prefill_chunked_paged.
 *   k8_cache, v8_cache: uint8 [num_pages, page_size, Hkv, d], 16-byte aligned;
 *     k_scale_cache, v_scale_cache: fp32 [num_pages, Hkv].  Read and written.
 *   workspace: at least the bytes fp_chunked_sizes gives for these params
 *     (with dtype fp8 it includes the Q codes and scales).
 * FP_INVALID_ARGUMENT when params->dtype is not fp8.
 */
int fp_sparse_prefill_chunked_paged_fp8(const fp_params* params, const void* q,
                                        const void* k_cache, const void* v_cache,
                                        int32_t page_size, int32_t num_pages,
                                        const int32_t* block_table, int32_t max_pages_per_seq,
                                        const int32_t* cu_seqlens_q_host, const int32_t* kv_lens_host,
                                        int32_t batch, float* pooled_cache, int32_t prefix_pooled,
                                        void* k8_cache, void* v8_cache,
                                        float* k_scale_cache, float* v_scale_cache,
                                        int32_t* kv_idx, int32_t* kv_cnt,
                                        void* workspace, size_t workspace_bytes,
                                        void* out, float* lse, void* stream);

/* Sizes for fp_sparse_prefill_chunked_paged and
 * fp_sparse_prefill_chunked_paged_fp8 (host only): kv_idx entries, kv_cnt
 * entries and workspace bytes, written where the pointers are not NULL.
 * Returns FP_OK or the error the call itself would give for these lengths. */
int fp_chunked_sizes(const fp_params* params, const int32_t* cu_seqlens_q_host,
                     const int32_t* kv_lens_host, int32_t batch,
                     int64_t* index_capacity, int64_t* count_entries, size_t* workspace_bytes);

/* Sizes (host only, no device work).  A single sequence of length S is
 * cu_seqlens_host = {0, S}, batch = 1.  Return -1 / 0 on invalid arguments. */
int64_t fp_index_capacity(const fp_params* params, const int32_t* cu_seqlens_host, int32_t batch);
int64_t fp_count_entries(const fp_params* params, const int32_t* cu_seqlens_host, int32_t batch);
size_t  fp_varlen_workspace_bytes(const fp_params* params, const int32_t* cu_seqlens_host,
                                  int32_t batch);

/* Workgroups the attention kernel is launched with for these arguments
 * (host only, no device work): one per (query block, query head), bf16 and
 * fp8 alike, contiguous (paged = 0, fp_sparse_prefill_fwd) or paged
 * (paged = 1, the paged entries).  Returns -1 on invalid arguments. */
int64_t fp_attention_workgroups(const fp_params* params, const int32_t* cu_seqlens_host, int32_t batch,
                                int32_t paged);

/* Static text for a return code. */
const char* fp_status_string(int status);
/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* fp_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FLASHPREFILL_H */
