// C-ABI entry points of libflashprefill: host-side validation, size queries,
// request tables and kernel launches.  Nothing here allocates, frees or
// synchronises; every call enqueues on the caller's stream.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "flashprefill.h"
#include "fp_launch.h"

#define FP_EXPORT extern "C" __attribute__((visibility("default")))

static_assert(FP_MAX_BATCH <= FP_TABLE_MAX, "request table too small");

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return FP_OK;
}

bool aligned(const void* p, uintptr_t a) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t tri(int64_t n) { return n * (n + 1) / 2; }

int check_params(const fp_params* p) {
    if (!p) return fail(FP_INVALID_ARGUMENT, "params is NULL");
    if (p->num_q_heads < 1 || p->num_kv_heads < 1)
        return fail(FP_INVALID_ARGUMENT, "num_q_heads (%d) and num_kv_heads (%d) must be >= 1", p->num_q_heads,
                    p->num_kv_heads);
    if (p->num_q_heads % p->num_kv_heads != 0)
        return fail(FP_INVALID_ARGUMENT, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)",
                    p->num_q_heads, p->num_kv_heads);
    if (p->num_q_heads / p->num_kv_heads > 32)
        return fail(FP_UNSUPPORTED, "more than 32 query heads per KV head (%d)", p->num_q_heads / p->num_kv_heads);
    if (p->head_dim != 64 && p->head_dim != 128)
        return fail(FP_UNSUPPORTED, "head_dim %d (supported: 64, 128)", p->head_dim);
    if (p->block_size != 64 && p->block_size != 128)
        return fail(FP_UNSUPPORTED, "block_size %d (supported: 64, 128)", p->block_size);
    if (!(p->alpha >= 0.f && p->alpha <= 1.f))
        return fail(FP_INVALID_ARGUMENT, "alpha must lie in [0, 1] (got %g)", (double)p->alpha);
    if (!std::isfinite(p->softmax_scale))
        return fail(FP_INVALID_ARGUMENT, "softmax_scale must be finite");
    if (p->mean_correction != 0 && p->mean_correction != 1)
        return fail(FP_INVALID_ARGUMENT, "mean_correction must be 0 or 1");
    if (p->dtype != FP_DTYPE_BF16 && p->dtype != FP_DTYPE_FP8_E4M3FN)
        return fail(FP_INVALID_ARGUMENT, "unknown dtype %d", p->dtype);
    if (p->shared_selection < 0 || p->shared_selection > 2)
        return fail(FP_INVALID_ARGUMENT, "shared_selection must be 0, 1 or 2");
    if (p->query_probes < 0 || (p->query_probes > 0 && p->block_size % p->query_probes != 0))
        return fail(FP_INVALID_ARGUMENT, "query_probes (%d) must be 0 or divide block_size (%d)", p->query_probes,
                    p->block_size);
    return FP_OK;
}

float sigma_of(const fp_params& p) {
    return p.softmax_scale > 0.f ? p.softmax_scale : (float)(1.0 / std::sqrt((double)p.head_dim));
}

// Validate cu_seqlens_host (query tokens per request) and, for chunked
// prefill, kv_lens_host (context length per request; NULL: equal to the query
// count), and fill the request table.  items_per_tile = 1 counts query
// blocks; n > 1 counts tiles of n query blocks (selection workgroups).
int build_table(const fp_params& p, const int32_t* cu, const int32_t* kv_lens, int32_t batch, int items_per_tile,
                SeqTable& t) {
    if (!cu) return fail(FP_INVALID_ARGUMENT, "cu_seqlens_host is NULL");
    if (batch < 1) return fail(FP_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", batch);
    if (batch > FP_MAX_BATCH) return fail(FP_UNSUPPORTED, "batch %d exceeds %d", batch, FP_MAX_BATCH);
    if (cu[0] != 0) return fail(FP_INVALID_ARGUMENT, "cu_seqlens[0] must be 0");
    const int B = p.block_size;
    std::memset(&t, 0, sizeof t);
    t.batch = batch;
    int64_t blocks = 0, pre = 0, idx = 0;
    std::vector<int64_t> ctx(batch);
    for (int b = 0; b < batch; ++b) {
        if (cu[b + 1] < cu[b]) return fail(FP_INVALID_ARGUMENT, "cu_seqlens not non-decreasing at %d", b + 1);
        const int64_t qlen = (int64_t)cu[b + 1] - cu[b];
        const int64_t len = kv_lens ? (int64_t)kv_lens[b] : qlen;
        if (len < qlen)
            return fail(FP_INVALID_ARGUMENT, "request %d: %lld queries exceed its context of %lld tokens", b,
                        (long long)qlen, (long long)len);
        if (p.query_probes > 0 && (len - qlen) % B != 0)
            return fail(FP_UNSUPPORTED,
                        "request %d: skeleton queries need a chunk that starts on a block boundary (start %lld, "
                        "block %d)", b, (long long)(len - qlen), B);
        const int64_t nb = (len + B - 1) / B;
        // Query blocks are first .. nb-1; the chunk may start inside block first.
        const int64_t first = qlen > 0 ? (len - qlen) / B : nb;
        if (nb > FP_MAX_BLOCKS / 2)
            return fail(FP_UNSUPPORTED, "request %d has %lld blocks (max %d)", b, (long long)nb, FP_MAX_BLOCKS / 2);
        ctx[b] = len;
        t.tok_off[b] = cu[b];
        t.blk_off[b] = (int32_t)blocks;
        t.pre_off[b] = (int32_t)pre;
        t.idx_off[b] = idx;
        t.tail[b] = (int16_t)(nb > 0 ? len - (nb - 1) * B : 0);
        blocks += nb;
        pre += first;
        idx += (int64_t)p.num_q_heads * (tri(nb) - tri(first));
    }
    t.tok_off[batch] = cu[batch];
    t.blk_off[batch] = (int32_t)blocks;
    t.pre_off[batch] = (int32_t)pre;
    t.idx_off[batch] = idx;
    t.total_tokens = cu[batch];
    t.total_blocks = (int32_t)blocks;
    t.total_qblocks = (int32_t)(blocks - pre);
    std::vector<int> ord(batch);
    for (int b = 0; b < batch; ++b) ord[b] = b;
    std::stable_sort(ord.begin(), ord.end(), [&](int x, int y) { return ctx[x] > ctx[y]; });
    int64_t items = 0;
    for (int s = 0; s < batch; ++s) {
        const int b = ord[s];
        const int nq = (t.blk_off[b + 1] - t.blk_off[b]) - (t.pre_off[b + 1] - t.pre_off[b]);
        t.order[s] = (int16_t)b;
        t.item_off[s] = (int32_t)items;
        items += (nq + items_per_tile - 1) / items_per_tile;
    }
    t.item_off[batch] = (int32_t)items;
    t.total_items = (int32_t)items;
    if ((int64_t)items * p.num_q_heads > 0x7fffffff)
        return fail(FP_UNSUPPORTED, "too many work items");
    return FP_OK;
}

int device_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return FP_OK;
    return fail(FP_DEVICE_ERROR, "%s launch failed: %s", what, hipGetErrorString(e));
}

int select_tile(const fp_params& p) { return 32 / (p.num_q_heads / p.num_kv_heads); }

int run_scores(const fp_params& p, const int32_t* cu, const int32_t* kv_lens, int32_t batch, const float* pq,
               const float* pk, int32_t* kv_idx, int32_t* kv_cnt, hipStream_t st);

// Pooling.  pcache: the caller's pooled cache (chunked prefill) or NULL;
// reuse: read the prefix blocks' means from it instead of pooling them;
// prefix_only: K and V of the prefix blocks only (the fused fp8 chunk pass
// pools the chunks' blocks).
int run_pool(const fp_params& p, const SeqTable& t, const void* q, const void* k, const void* v,
             const KVLayout& kv, bool paged, float* pq, float* pk, float* pv, uint16_t* pkv16, float* pcache,
             int reuse, bool prefix_only, hipStream_t st) {
    PoolArgs pa;
    pa.q = static_cast<const uint16_t*>(q);
    pa.k = static_cast<const uint16_t*>(k);
    const bool pool_v = pv || pkv16 || pcache;
    pa.v = pool_v ? static_cast<const uint16_t*>(v) : nullptr;
    pa.pcache = pcache;
    pa.reuse = reuse;
    pa.pq = pq;
    pa.pk = pk;
    pa.pv = pv;
    pa.pkv16 = pkv16;
    pa.kv = kv;
    pa.Hq = p.num_q_heads;
    pa.Hkv = p.num_kv_heads;
    pa.D = p.head_dim;
    pa.B = p.block_size;
    pa.q_stride = p.query_probes > 0 ? p.block_size / p.query_probes : 1;
    pa.q_chunks = p.num_q_heads * p.head_dim / 8;
    pa.k_chunks = p.num_kv_heads * p.head_dim / 8;
    pa.total_chunks = pa.q_chunks + pa.k_chunks * (pool_v ? 2 : 1);
    pa.prefix_only = prefix_only ? 1 : 0;
    return device_status(launch_pool(pa, t, paged, st), "pool");
}

// Pooling and selection.  kv_lens: context lengths (chunked prefill) or NULL.
int run_select(const fp_params& p, const int32_t* cu, const int32_t* kv_lens, int32_t batch, const void* q,
               const void* k, const void* v, const KVLayout& kv, bool paged, float* pq, float* pk, float* pv,
               uint16_t* pkv16, float* pcache, int reuse, int32_t* kv_idx, int32_t* kv_cnt, hipStream_t st) {
    SeqTable t;
    int rc = build_table(p, cu, kv_lens, batch, 1, t);
    if (rc) return rc;
    rc = run_pool(p, t, q, k, v, kv, paged, pq, pk, pv, pkv16, pcache, reuse, false, st);
    if (rc) return rc;
    return run_scores(p, cu, kv_lens, batch, pq, pk, kv_idx, kv_cnt, st);
}

// Scores, threshold and lists from pooled means already in place.
int run_scores(const fp_params& p, const int32_t* cu, const int32_t* kv_lens, int32_t batch, const float* pq,
               const float* pk, int32_t* kv_idx, int32_t* kv_cnt, hipStream_t st) {
    int rc;
    SeqTable ts;
    const int TI = select_tile(p);
    rc = build_table(p, cu, kv_lens, batch, kSelectRowWaves * TI, ts);
    if (rc) return rc;
    SelArgs sa;
    sa.pq = pq;
    sa.pk = pk;
    sa.kv_idx = kv_idx;
    sa.kv_cnt = kv_cnt;
    sa.Hq = p.num_q_heads;
    sa.Hkv = p.num_kv_heads;
    sa.g = p.num_q_heads / p.num_kv_heads;
    sa.D = p.head_dim;
    sa.TI = TI;
    sa.scale = sigma_of(p);
    sa.ln_alpha = p.alpha > 0.f ? (float)std::log((double)p.alpha) : -INFINITY;
    sa.shared = p.shared_selection;
    return device_status(launch_select(sa, ts, st), "select");
}

}  // namespace

FP_EXPORT const char* fp_status_string(int status) {
    switch (status) {
        case FP_OK: return "ok";
        case FP_INVALID_ARGUMENT: return "invalid argument";
        case FP_UNSUPPORTED: return "unsupported";
        case FP_WORKSPACE_TOO_SMALL: return "workspace too small";
        case FP_DEVICE_ERROR: return "device error";
        default: return "unknown status";
    }
}

FP_EXPORT const char* fp_last_error(void) { return g_last_error.c_str(); }

FP_EXPORT int64_t fp_index_capacity(const fp_params* params, const int32_t* cu_seqlens_host, int32_t batch) {
    SeqTable t;
    if (check_params(params) || build_table(*params, cu_seqlens_host, nullptr, batch, 1, t)) return -1;
    return t.idx_off[batch];
}

FP_EXPORT int64_t fp_count_entries(const fp_params* params, const int32_t* cu_seqlens_host, int32_t batch) {
    SeqTable t;
    if (check_params(params) || build_table(*params, cu_seqlens_host, nullptr, batch, 1, t)) return -1;
    return (int64_t)params->num_q_heads * t.total_qblocks;
}

namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
struct WsLayout {
    size_t q, k, kv16;          // fp32 Q_bar, fp32 K_bar, bf16 K_bar | V_bar
    size_t q8, qs;              // fp8 only: e4m3 Q codes [T, Hq, d], fp32 Q scales [Hq, blocks]
    size_t total;
};
WsLayout ws_layout(const fp_params& p, const SeqTable& t) {
    WsLayout w;
    const size_t per = (size_t)t.total_blocks * p.head_dim;
    w.q = 0;
    w.k = align256((size_t)t.total_qblocks * p.head_dim * p.num_q_heads * sizeof(float));
    w.kv16 = w.k + align256(per * p.num_kv_heads * sizeof(float));
    w.q8 = w.kv16 + (p.mean_correction ? align256(2 * per * p.num_kv_heads * sizeof(uint16_t)) : 0);
    w.qs = w.q8;
    w.total = w.q8;
    if (p.dtype == FP_DTYPE_FP8_E4M3FN) {
        w.qs = w.q8 + align256((size_t)t.total_tokens * p.num_q_heads * p.head_dim);
        w.total = w.qs + align256((size_t)t.total_qblocks * p.num_q_heads * sizeof(float));
    }
    return w;
}
}  // namespace

FP_EXPORT int64_t fp_attention_workgroups(const fp_params* params, const int32_t* cu_seqlens_host, int32_t batch,
                                          int32_t paged) {
    SeqTable t;
    if (check_params(params) || build_table(*params, cu_seqlens_host, nullptr, batch, 1, t)) return -1;
    if (paged != 0 && paged != 1) return -1;
    return (int64_t)t.total_items * params->num_q_heads;
}

FP_EXPORT size_t fp_varlen_workspace_bytes(const fp_params* params, const int32_t* cu_seqlens_host, int32_t batch) {
    SeqTable t;
    if (check_params(params) || build_table(*params, cu_seqlens_host, nullptr, batch, 1, t)) return 0;
    return ws_layout(*params, t).total;
}

FP_EXPORT int fp_select_blocks(const fp_params* params, const void* q, const void* k, const void* v, int32_t seqlen,
                               float* pooled_q, float* pooled_k, float* pooled_v, void* pooled_kv_bf16,
                               int32_t* kv_idx, int32_t* kv_cnt, void* stream) {
    int rc = check_params(params);
    if (rc) return rc;
    if (seqlen < 0) return fail(FP_INVALID_ARGUMENT, "seqlen must be >= 0 (got %d)", seqlen);
    if (seqlen == 0) return ok();
    if (!aligned(q, 16) || !aligned(k, 16)) return fail(FP_INVALID_ARGUMENT, "q and k must be non-NULL and 16-byte aligned");
    if (!aligned(pooled_q, 16) || !aligned(pooled_k, 16))
        return fail(FP_INVALID_ARGUMENT, "pooled_q and pooled_k must be non-NULL and 16-byte aligned");
    if (!aligned(kv_idx, 4) || !aligned(kv_cnt, 4))
        return fail(FP_INVALID_ARGUMENT, "kv_idx and kv_cnt must be non-NULL and 4-byte aligned");
    if (pooled_v && (!aligned(pooled_v, 16) || !aligned(v, 16)))
        return fail(FP_INVALID_ARGUMENT, "pooled_v needs a non-NULL, 16-byte aligned v (and itself aligned)");
    if (pooled_kv_bf16 && (!aligned(pooled_kv_bf16, 16) || !aligned(v, 16)))
        return fail(FP_INVALID_ARGUMENT, "pooled_kv_bf16 needs a non-NULL, 16-byte aligned v (and itself aligned)");
    const int32_t cu[2] = {0, seqlen};
    KVLayout kv = {nullptr, 1, 0, 0, 0};
    (void)hipGetLastError();
    rc = run_select(*params, cu, nullptr, 1, q, k, v, kv, false, pooled_q, pooled_k, pooled_v,
                    static_cast<uint16_t*>(pooled_kv_bf16), nullptr, 0, kv_idx, kv_cnt,
                    static_cast<hipStream_t>(stream));
    return rc ? rc : ok();
}

FP_EXPORT int fp_select_blocks_fp8(const fp_params* params, const void* q, const void* k, const void* v,
                                   int32_t seqlen, void* q8, void* k8, void* v8, float* q_scale, float* k_scale,
                                   float* v_scale, float* pooled_q, float* pooled_k, void* pooled_kv_bf16,
                                   int32_t* kv_idx, int32_t* kv_cnt, void* stream) {
    int rc = check_params(params);
    if (rc) return rc;
    const fp_params& p = *params;
    if (p.dtype != FP_DTYPE_FP8_E4M3FN)
        return fail(FP_INVALID_ARGUMENT, "fp_select_blocks_fp8 prepares fp8 attention: params->dtype must be fp8");
    if (seqlen < 0) return fail(FP_INVALID_ARGUMENT, "seqlen must be >= 0 (got %d)", seqlen);
    if (seqlen == 0) return ok();
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
        return fail(FP_INVALID_ARGUMENT, "q, k and v must be non-NULL and 16-byte aligned");
    if (!aligned(q8, 8) || !aligned(k8, 8) || !aligned(v8, 8))
        return fail(FP_INVALID_ARGUMENT, "q8, k8 and v8 must be non-NULL and 8-byte aligned");
    if (!aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4))
        return fail(FP_INVALID_ARGUMENT, "q_scale, k_scale and v_scale must be non-NULL and 4-byte aligned");
    if (!aligned(pooled_q, 16) || !aligned(pooled_k, 16))
        return fail(FP_INVALID_ARGUMENT, "pooled_q and pooled_k must be non-NULL and 16-byte aligned");
    if (p.mean_correction && !aligned(pooled_kv_bf16, 16))
        return fail(FP_INVALID_ARGUMENT, "mean_correction needs a 16-byte aligned pooled_kv_bf16");
    if (!aligned(kv_idx, 4) || !aligned(kv_cnt, 4))
        return fail(FP_INVALID_ARGUMENT, "kv_idx and kv_cnt must be non-NULL and 4-byte aligned");
    const int32_t cu[2] = {0, seqlen};
    SeqTable t;
    rc = build_table(p, cu, nullptr, 1, 1, t);
    if (rc) return rc;
    QuantArgs qa;
    qa.src[0] = static_cast<const uint16_t*>(q);
    qa.src[1] = static_cast<const uint16_t*>(k);
    qa.src[2] = static_cast<const uint16_t*>(v);
    qa.codes[0] = static_cast<uint8_t*>(q8);
    qa.codes[1] = static_cast<uint8_t*>(k8);
    qa.codes[2] = static_cast<uint8_t*>(v8);
    qa.scale[0] = q_scale;
    qa.scale[1] = k_scale;
    qa.scale[2] = v_scale;
    qa.pq = pooled_q;
    qa.pk = pooled_k;
    qa.pkv16 = p.mean_correction ? static_cast<uint16_t*>(pooled_kv_bf16) : nullptr;
    qa.pcache = nullptr;
    qa.H[0] = p.num_q_heads;
    qa.H[1] = qa.H[2] = p.num_kv_heads;
    qa.groups[0] = qa.groups[1] = qa.groups[2] = 0;
    qa.kv = KVLayout{nullptr, 1, 0, 0, 0};
    qa.D = p.head_dim;
    qa.B = p.block_size;
    qa.nB = t.total_blocks;
    qa.q_stride = p.query_probes > 0 ? p.block_size / p.query_probes : 1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    rc = device_status(launch_quant_pool(qa, t, false, false, st), "quantize + pool");
    if (rc) return rc;
    rc = run_scores(p, cu, nullptr, 1, pooled_q, pooled_k, kv_idx, kv_cnt, st);
    return rc ? rc : ok();
}

FP_EXPORT int fp_sparse_prefill_fwd(const fp_params* params, const void* q, const void* k, const void* v,
                                    const float* q_scale, const float* k_scale, const float* v_scale, int32_t seqlen,
                                    const int32_t* kv_idx, const int32_t* kv_cnt, const void* pooled_kv_bf16,
                                    void* out, float* lse, void* stream) {
    int rc = check_params(params);
    if (rc) return rc;
    const fp_params& p = *params;
    if (seqlen < 0) return fail(FP_INVALID_ARGUMENT, "seqlen must be >= 0 (got %d)", seqlen);
    if (seqlen == 0) return ok();
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return fail(FP_INVALID_ARGUMENT, "q, k, v and out must be non-NULL and 16-byte aligned");
    if (!aligned(kv_idx, 4) || !aligned(kv_cnt, 4))
        return fail(FP_INVALID_ARGUMENT, "kv_idx and kv_cnt must be non-NULL and 4-byte aligned");
    if (p.mean_correction && !aligned(pooled_kv_bf16, 16))
        return fail(FP_INVALID_ARGUMENT, "mean_correction needs a 16-byte aligned pooled_kv_bf16");
    if (lse && !aligned(lse, 4)) return fail(FP_INVALID_ARGUMENT, "lse must be 4-byte aligned");
    const bool fp8 = p.dtype == FP_DTYPE_FP8_E4M3FN;
    if (fp8 && (!aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4)))
        return fail(FP_INVALID_ARGUMENT, "fp8 inputs need q_scale, k_scale and v_scale");
    const int32_t cu[2] = {0, seqlen};
    SeqTable t;
    rc = build_table(p, cu, nullptr, 1, 1, t);
    if (rc) return rc;
    AttnArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.q_scale = q_scale;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.kv_idx = kv_idx;
    a.kv_cnt = kv_cnt;
    a.pk16 = static_cast<const uint16_t*>(pooled_kv_bf16);
    a.pv16 = a.pk16 ? a.pk16 + (int64_t)p.num_kv_heads * t.total_blocks * p.head_dim : nullptr;
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    a.kv = KVLayout{nullptr, 1, 0, 0, 0};
    a.Hq = p.num_q_heads;
    a.Hkv = p.num_kv_heads;
    a.g = p.num_q_heads / p.num_kv_heads;
    a.scale_log2 = (float)(sigma_of(p) * 1.4426950408889634);
    a.correction = p.mean_correction;
    (void)hipGetLastError();
    hipStream_t st = static_cast<hipStream_t>(stream);
    rc = fp8 ? device_status(launch_attn_fp8(a, t, p.head_dim, p.block_size, false, st), "attention (fp8)")
             : device_status(launch_attn_bf16(a, t, p.head_dim, p.block_size, false, st), "attention");
    return rc ? rc : ok();
}

namespace {
// e4m3 pages of fp8 chunked prefill: codes in the layout of the bf16 pages,
// one fp32 scale per (page, KV head) at the entry of a block's first page.
struct Fp8Pages {
    void* k8;
    void* v8;
    float* ks;
    float* vs;
};

// The paged entries: pooling, selection and attention of a continuous batch.
// kv_lens NULL: whole prompts; else context lengths (chunked prefill), with
// the pooled cache pcache (may be NULL) and its reuse flag.  f8 non-NULL:
// fp8 attention over the e4m3 pages, whose query blocks' codes and scales
// are written first (chunked prefill; params in fp8).
// log2 of a power of two (a page size divides the block size, 64 or 128, so
// it is one); the kernels address pages with shifts and masks.
static int log2_exact(int v) {
    int s = 0;
    while ((1 << s) < v) ++s;
    return s;
}

int paged_prefill(const fp_params* params, const void* q, const void* k_cache, const void* v_cache, int32_t page_size,
                  int32_t num_pages, const int32_t* block_table, int32_t max_pages_per_seq, const int32_t* cu_q,
                  const int32_t* kv_lens, int32_t batch, float* pcache, int32_t reuse, const Fp8Pages* f8,
                  int32_t* kv_idx, int32_t* kv_cnt, void* workspace, size_t workspace_bytes, void* out, float* lse,
                  void* stream) {
    int rc = check_params(params);
    if (rc) return rc;
    const fp_params& p = *params;
    if (f8 && p.dtype != FP_DTYPE_FP8_E4M3FN)
        return fail(FP_INVALID_ARGUMENT, "fp_sparse_prefill_chunked_paged_fp8: params->dtype must be fp8");
    if (!f8 && p.dtype != FP_DTYPE_BF16) return fail(FP_UNSUPPORTED, "the paged entries read bf16 only");
    SeqTable t;
    rc = build_table(p, cu_q, kv_lens, batch, 1, t);
    if (rc) return rc;
    if (page_size < 1 || p.block_size % page_size != 0)
        return fail(FP_INVALID_ARGUMENT, "page_size (%d) must divide block_size (%d)", page_size, p.block_size);
    if (num_pages < 1) return fail(FP_INVALID_ARGUMENT, "num_pages must be >= 1");
    for (int b = 0; b < batch; ++b) {
        const int64_t len = kv_lens ? (int64_t)kv_lens[b] : (int64_t)cu_q[b + 1] - cu_q[b];
        const int64_t need = (len + page_size - 1) / page_size;
        if (need > max_pages_per_seq)
            return fail(FP_INVALID_ARGUMENT, "request %d needs %lld pages > max_pages_per_seq %d", b,
                        (long long)need, max_pages_per_seq);
    }
    if (t.total_tokens == 0) return ok();
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
        return fail(FP_INVALID_ARGUMENT, "q, k_cache, v_cache and out must be non-NULL and 16-byte aligned");
    if (!aligned(block_table, 4) || !aligned(kv_idx, 4) || !aligned(kv_cnt, 4))
        return fail(FP_INVALID_ARGUMENT, "block_table, kv_idx and kv_cnt must be non-NULL and 4-byte aligned");
    if (lse && !aligned(lse, 4)) return fail(FP_INVALID_ARGUMENT, "lse must be 4-byte aligned");
    if (pcache && !aligned(pcache, 16)) return fail(FP_INVALID_ARGUMENT, "pooled_cache must be 16-byte aligned");
    if (f8 && (!aligned(f8->k8, 16) || !aligned(f8->v8, 16)))
        return fail(FP_INVALID_ARGUMENT, "k8_cache and v8_cache must be non-NULL and 16-byte aligned");
    if (f8 && (!aligned(f8->ks, 4) || !aligned(f8->vs, 4)))
        return fail(FP_INVALID_ARGUMENT, "k_scale_cache and v_scale_cache must be non-NULL and 4-byte aligned");
    const WsLayout ws = ws_layout(p, t);
    if (!aligned(workspace, 256)) return fail(FP_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");
    if (workspace_bytes < ws.total)
        return fail(FP_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, need %zu", workspace_bytes, ws.total);
    char* wsb = static_cast<char*>(workspace);
    float* pq = reinterpret_cast<float*>(wsb + ws.q);
    float* pk = reinterpret_cast<float*>(wsb + ws.k);
    uint16_t* pkv16 = p.mean_correction ? reinterpret_cast<uint16_t*>(wsb + ws.kv16) : nullptr;
    KVLayout kv = {block_table, page_size, num_pages, max_pages_per_seq, log2_exact(page_size)};
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (!f8) {
        rc = run_select(p, cu_q, kv_lens, batch, q, k_cache, v_cache, kv, true, pq, pk, nullptr, pkv16, pcache, reuse,
                        kv_idx, kv_cnt, st);
        if (rc) return rc;
    }
    AttnArgs a;
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.q_scale = a.k_scale = a.v_scale = nullptr;
    if (f8) {
        // The prefix blocks' K/V means (from the pooled cache, or pooled
        // now); then one pass over the chunks' query blocks: Q codes and
        // scales into the workspace, K and V codes into the e4m3 pages
        // (blocks before them were encoded by earlier calls), and their
        // means (the same bits the pooling kernel forms); then selection.
        rc = run_pool(p, t, q, k_cache, v_cache, kv, true, pq, pk, nullptr, pkv16, pcache, reuse, true, st);
        if (rc) return rc;
        uint8_t* q8 = reinterpret_cast<uint8_t*>(wsb + ws.q8);
        float* qs = reinterpret_cast<float*>(wsb + ws.qs);
        QuantArgs qa;
        std::memset(&qa, 0, sizeof qa);
        qa.src[0] = static_cast<const uint16_t*>(q);
        qa.src[1] = static_cast<const uint16_t*>(k_cache);
        qa.src[2] = static_cast<const uint16_t*>(v_cache);
        qa.codes[0] = q8;
        qa.codes[1] = static_cast<uint8_t*>(f8->k8);
        qa.codes[2] = static_cast<uint8_t*>(f8->v8);
        qa.scale[0] = qs;
        qa.scale[1] = f8->ks;
        qa.scale[2] = f8->vs;
        qa.kv = kv;
        qa.H[0] = p.num_q_heads;
        qa.H[1] = qa.H[2] = p.num_kv_heads;
        qa.pq = pq;
        qa.pk = pk;
        qa.pkv16 = pkv16;
        qa.pcache = pcache;
        qa.D = p.head_dim;
        qa.B = p.block_size;
        qa.nB = t.total_qblocks;
        qa.q_stride = p.query_probes > 0 ? p.block_size / p.query_probes : 1;
        rc = device_status(launch_quant_pool(qa, t, true, true, st), "quantize + pool (chunked)");
        if (rc) return rc;
        rc = run_scores(p, cu_q, kv_lens, batch, pq, pk, kv_idx, kv_cnt, st);
        if (rc) return rc;
        a.q = q8;
        a.k = f8->k8;
        a.v = f8->v8;
        a.q_scale = qs;
        a.k_scale = f8->ks;
        a.v_scale = f8->vs;
    }
    a.kv_idx = kv_idx;
    a.kv_cnt = kv_cnt;
    a.pk16 = pkv16;
    a.pv16 = pkv16 ? pkv16 + (int64_t)p.num_kv_heads * t.total_blocks * p.head_dim : nullptr;
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    a.kv = kv;
    a.Hq = p.num_q_heads;
    a.Hkv = p.num_kv_heads;
    a.g = p.num_q_heads / p.num_kv_heads;
    a.scale_log2 = (float)(sigma_of(p) * 1.4426950408889634);
    a.correction = p.mean_correction;
    rc = f8 ? device_status(launch_attn_fp8(a, t, p.head_dim, p.block_size, true, st), "attention (fp8, chunked)")
            : device_status(launch_attn_bf16(a, t, p.head_dim, p.block_size, true, st), "attention (paged)");
    return rc ? rc : ok();
}
}  // namespace

FP_EXPORT int fp_sparse_prefill_varlen_paged(const fp_params* params, const void* q, const void* k_cache,
                                             const void* v_cache, int32_t page_size, int32_t num_pages,
                                             const int32_t* block_table, int32_t max_pages_per_seq,
                                             const int32_t* cu_seqlens_host, int32_t batch,
                                             int32_t* kv_idx, int32_t* kv_cnt, void* workspace,
                                             size_t workspace_bytes, void* out, float* lse, void* stream) {
    return paged_prefill(params, q, k_cache, v_cache, page_size, num_pages, block_table, max_pages_per_seq,
                         cu_seqlens_host, nullptr, batch, nullptr, 0, nullptr, kv_idx, kv_cnt, workspace,
                         workspace_bytes, out, lse, stream);
}

// Scratch of the allocation-free paged entry: one copy per GPU, in the
// library's code object, held until the process ends.  Host code never uses
// the array's name as an address (on the host it names a stand-in, not device
// memory): the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) char scratch[FP_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of this device's scratch array (looked up on the first call
// with that device current), or an FP_* error.
int scratch_on_current_device(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FP_DEVICE_ERROR, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(FP_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(FP_DEVICE_ERROR, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return FP_OK;
}
}  // namespace

FP_EXPORT int fp_sparse_prefill_varlen_paged_noalloc(const fp_params* params, const void* q, const void* k_cache,
                                                     const void* v_cache, int32_t page_size, int32_t num_pages,
                                                     const int32_t* block_table, int32_t max_pages_per_seq,
                                                     const int32_t* cu_seqlens_host, int32_t batch,
                                                     int32_t* kv_idx, int32_t* kv_cnt, void* out, float* lse,
                                                     void* stream) {
    int rc = check_params(params);
    if (rc) return rc;
    SeqTable t;
    rc = build_table(*params, cu_seqlens_host, nullptr, batch, 1, t);
    if (rc) return rc;
    const size_t need = ws_layout(*params, t).total;
    if (need > FP_NOALLOC_SCRATCH_BYTES)
        return fail(FP_WORKSPACE_TOO_SMALL,
                    "the batch needs %zu bytes of pooled-mean scratch; the allocation-free entry holds %zu "
                    "(use fp_sparse_prefill_varlen_paged with a workspace)",
                    need, (size_t)FP_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    rc = scratch_on_current_device(&ws);
    if (rc) return rc;
    return paged_prefill(params, q, k_cache, v_cache, page_size, num_pages, block_table, max_pages_per_seq,
                         cu_seqlens_host, nullptr, batch, nullptr, 0, nullptr, kv_idx, kv_cnt, ws,
                         (size_t)FP_NOALLOC_SCRATCH_BYTES, out, lse, stream);
}

FP_EXPORT int fp_sparse_prefill_varlen_paged_fp8(const fp_params* params, const void* q, const void* k_cache,
                                                 const void* v_cache, int32_t page_size, int32_t num_pages,
                                                 const int32_t* block_table, int32_t max_pages_per_seq,
                                                 const int32_t* cu_seqlens_host, int32_t batch, void* k8_cache,
                                                 void* v8_cache, float* k_scale_cache, float* v_scale_cache,
                                                 int32_t* kv_idx, int32_t* kv_cnt, void* workspace,
                                                 size_t workspace_bytes, void* out, float* lse, void* stream) {
    int rc = check_params(params);
    if (rc) return rc;
    const fp_params& p = *params;
    if (p.dtype != FP_DTYPE_FP8_E4M3FN)
        return fail(FP_INVALID_ARGUMENT, "fp_sparse_prefill_varlen_paged_fp8: params->dtype must be fp8");
    SeqTable t;
    rc = build_table(p, cu_seqlens_host, nullptr, batch, 1, t);
    if (rc) return rc;
    if (page_size < 1 || p.block_size % page_size != 0)
        return fail(FP_INVALID_ARGUMENT, "page_size (%d) must divide block_size (%d)", page_size, p.block_size);
    if (num_pages < 1) return fail(FP_INVALID_ARGUMENT, "num_pages must be >= 1");
    for (int b = 0; b < batch; ++b) {
        const int64_t len = (int64_t)cu_seqlens_host[b + 1] - cu_seqlens_host[b];
        if ((len + page_size - 1) / page_size > max_pages_per_seq)
            return fail(FP_INVALID_ARGUMENT, "request %d needs %lld pages > max_pages_per_seq %d", b,
                        (long long)((len + page_size - 1) / page_size), max_pages_per_seq);
    }
    if (t.total_tokens == 0) return ok();
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
        return fail(FP_INVALID_ARGUMENT, "q, k_cache, v_cache and out must be non-NULL and 16-byte aligned");
    if (!aligned(k8_cache, 16) || !aligned(v8_cache, 16))
        return fail(FP_INVALID_ARGUMENT, "k8_cache and v8_cache must be non-NULL and 16-byte aligned");
    if (!aligned(k_scale_cache, 4) || !aligned(v_scale_cache, 4))
        return fail(FP_INVALID_ARGUMENT, "k_scale_cache and v_scale_cache must be non-NULL and 4-byte aligned");
    if (!aligned(block_table, 4) || !aligned(kv_idx, 4) || !aligned(kv_cnt, 4))
        return fail(FP_INVALID_ARGUMENT, "block_table, kv_idx and kv_cnt must be non-NULL and 4-byte aligned");
    if (lse && !aligned(lse, 4)) return fail(FP_INVALID_ARGUMENT, "lse must be 4-byte aligned");
    const WsLayout ws = ws_layout(p, t);
    if (!aligned(workspace, 256)) return fail(FP_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");
    if (workspace_bytes < ws.total)
        return fail(FP_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, need %zu", workspace_bytes, ws.total);
    char* wsb = static_cast<char*>(workspace);
    float* pq = reinterpret_cast<float*>(wsb + ws.q);
    float* pk = reinterpret_cast<float*>(wsb + ws.k);
    uint16_t* pkv16 = p.mean_correction ? reinterpret_cast<uint16_t*>(wsb + ws.kv16) : nullptr;
    uint8_t* q8 = reinterpret_cast<uint8_t*>(wsb + ws.q8);
    float* qs = reinterpret_cast<float*>(wsb + ws.qs);
    const KVLayout kv = {block_table, page_size, num_pages, max_pages_per_seq, log2_exact(page_size)};
    // One pass over the bf16 data: Q codes and scales into the workspace, K
    // and V codes into the e4m3 pages with their scales, the block means.
    QuantArgs qa;
    qa.src[0] = static_cast<const uint16_t*>(q);
    qa.src[1] = static_cast<const uint16_t*>(k_cache);
    qa.src[2] = static_cast<const uint16_t*>(v_cache);
    qa.codes[0] = q8;
    qa.codes[1] = static_cast<uint8_t*>(k8_cache);
    qa.codes[2] = static_cast<uint8_t*>(v8_cache);
    qa.scale[0] = qs;
    qa.scale[1] = k_scale_cache;
    qa.scale[2] = v_scale_cache;
    qa.pq = pq;
    qa.pk = pk;
    qa.pkv16 = pkv16;
    qa.pcache = nullptr;
    qa.kv = kv;
    qa.H[0] = p.num_q_heads;
    qa.H[1] = qa.H[2] = p.num_kv_heads;
    qa.groups[0] = qa.groups[1] = qa.groups[2] = 0;
    qa.D = p.head_dim;
    qa.B = p.block_size;
    qa.nB = t.total_blocks;
    qa.q_stride = p.query_probes > 0 ? p.block_size / p.query_probes : 1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    rc = device_status(launch_quant_pool(qa, t, true, false, st), "quantize + pool (paged)");
    if (rc) return rc;
    rc = run_scores(p, cu_seqlens_host, nullptr, batch, pq, pk, kv_idx, kv_cnt, st);
    if (rc) return rc;
    AttnArgs a;
    a.q = q8;
    a.k = k8_cache;
    a.v = v8_cache;
    a.q_scale = qs;
    a.k_scale = k_scale_cache;
    a.v_scale = v_scale_cache;
    a.kv_idx = kv_idx;
    a.kv_cnt = kv_cnt;
    a.pk16 = pkv16;
    a.pv16 = pkv16 ? pkv16 + (int64_t)p.num_kv_heads * t.total_blocks * p.head_dim : nullptr;
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    a.kv = kv;
    a.Hq = p.num_q_heads;
    a.Hkv = p.num_kv_heads;
    a.g = p.num_q_heads / p.num_kv_heads;
    a.scale_log2 = (float)(sigma_of(p) * 1.4426950408889634);
    a.correction = p.mean_correction;
    rc = device_status(launch_attn_fp8(a, t, p.head_dim, p.block_size, true, st), "attention (fp8, paged)");
    return rc ? rc : ok();
}

FP_EXPORT int fp_chunked_sizes(const fp_params* params, const int32_t* cu_seqlens_q_host, const int32_t* kv_lens_host,
                               int32_t batch, int64_t* index_capacity, int64_t* count_entries,
                               size_t* workspace_bytes) {
    int rc = check_params(params);
    if (rc) return rc;
    if (!kv_lens_host) return fail(FP_INVALID_ARGUMENT, "kv_lens_host is NULL");
    SeqTable t;
    rc = build_table(*params, cu_seqlens_q_host, kv_lens_host, batch, 1, t);
    if (rc) return rc;
    if (index_capacity) *index_capacity = t.idx_off[batch];
    if (count_entries) *count_entries = (int64_t)params->num_q_heads * t.total_qblocks;
    if (workspace_bytes) *workspace_bytes = ws_layout(*params, t).total;
    return ok();
}

FP_EXPORT int fp_sparse_prefill_chunked_paged(const fp_params* params, const void* q, const void* k_cache,
                                              const void* v_cache, int32_t page_size, int32_t num_pages,
                                              const int32_t* block_table, int32_t max_pages_per_seq,
                                              const int32_t* cu_seqlens_q_host, const int32_t* kv_lens_host,
                                              int32_t batch, float* pooled_cache, int32_t prefix_pooled,
                                              int32_t* kv_idx, int32_t* kv_cnt, void* workspace,
                                              size_t workspace_bytes, void* out, float* lse, void* stream) {
    if (!kv_lens_host) return fail(FP_INVALID_ARGUMENT, "kv_lens_host is NULL");
    if (prefix_pooled != 0 && prefix_pooled != 1) return fail(FP_INVALID_ARGUMENT, "prefix_pooled must be 0 or 1");
    if (prefix_pooled && !pooled_cache) return fail(FP_INVALID_ARGUMENT, "prefix_pooled needs a pooled_cache");
    return paged_prefill(params, q, k_cache, v_cache, page_size, num_pages, block_table, max_pages_per_seq,
                         cu_seqlens_q_host, kv_lens_host, batch, pooled_cache, prefix_pooled, nullptr, kv_idx, kv_cnt,
                         workspace, workspace_bytes, out, lse, stream);
}

FP_EXPORT int fp_sparse_prefill_chunked_paged_fp8(const fp_params* params, const void* q, const void* k_cache,
                                                  const void* v_cache, int32_t page_size, int32_t num_pages,
                                                  const int32_t* block_table, int32_t max_pages_per_seq,
                                                  const int32_t* cu_seqlens_q_host, const int32_t* kv_lens_host,
                                                  int32_t batch, float* pooled_cache, int32_t prefix_pooled,
                                                  void* k8_cache, void* v8_cache, float* k_scale_cache,
                                                  float* v_scale_cache, int32_t* kv_idx, int32_t* kv_cnt,
                                                  void* workspace, size_t workspace_bytes, void* out, float* lse,
                                                  void* stream) {
    if (!kv_lens_host) return fail(FP_INVALID_ARGUMENT, "kv_lens_host is NULL");
    if (prefix_pooled != 0 && prefix_pooled != 1) return fail(FP_INVALID_ARGUMENT, "prefix_pooled must be 0 or 1");
    if (prefix_pooled && !pooled_cache) return fail(FP_INVALID_ARGUMENT, "prefix_pooled needs a pooled_cache");
    const Fp8Pages f8 = {k8_cache, v8_cache, k_scale_cache, v_scale_cache};
    return paged_prefill(params, q, k_cache, v_cache, page_size, num_pages, block_table, max_pages_per_seq,
                         cu_seqlens_q_host, kv_lens_host, batch, pooled_cache, prefix_pooled, &f8, kv_idx, kv_cnt,
                         workspace, workspace_bytes, out, lse, stream);
}
