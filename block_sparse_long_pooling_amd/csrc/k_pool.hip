// Block-mean pooling of Q, K and V (FlashPrefill, gist.science technical
// summary, section 2.A: keys are replaced by their block mean; queries are
// pooled the same way, and V is pooled for the V2 mean-correction term).
// K_bar and V_bar are also written rounded to bf16, the form in which the
// attention kernels consume them.
//
// In chunked prefill the prefix blocks have no queries in the call; their
// K_bar / V_bar are pooled from the cache pages or, when an earlier call
// pooled them, read from the caller's pooled cache (one fp32 entry per page
// that starts a block), and every block pooled here is written back to it.
//
// One workgroup covers one KV block of one request and 256 column chunks
// of 8 bf16 (16 bytes) taken from the concatenated row [Q | K | V].  Each
// thread walks the block's tokens, so a wave reads 1 KiB contiguous per
// token step, with 4 loads in flight per thread.  Sums are fp32, in the
// token tree of the fused fp8 pass (tree_sum below), then divided by n_J.
#include "fp_launch.h"

namespace {

constexpr int kThreads = 256;

// Q, K and V are streamed once here: non-temporal loads (they are not kept in
// the caches for reuse) run the pass about 10% faster.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ntload(const uint16_t* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void add8(float* acc, uint4 x) {
    acc[0] += bf16_lo(x.x); acc[1] += bf16_hi(x.x);
    acc[2] += bf16_lo(x.y); acc[3] += bf16_hi(x.y);
    acc[4] += bf16_lo(x.z); acc[5] += bf16_hi(x.z);
    acc[6] += bf16_lo(x.w); acc[7] += bf16_hi(x.w);
}

// Block sum of one 8-value column chunk, in the order in which the fused fp8
// pass (k_quant.hip) adds the same tokens: partial (w, hf), w = 0..7,
// hf = 0..1, takes tokens 16 s + 2 w + hf in s order; the two halves of a w
// are added, then the w partials in w order.  The means of both kernels are
// then bit-identical (tokens that do not count add nothing; the fused pass
// adds zeros for them, which leaves every partial unchanged).  load(tok)
// gives the chunk of token tok and whether it counts; two values of s are in
// flight at a time (four loads).
template <typename Load>
__device__ __forceinline__ void tree_sum(int B, Load&& load, float* tot) {
    const int ns = B / 16;
#pragma unroll 1
    for (int w = 0; w < 8; ++w) {
        float a0[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float a1[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < ns; s += 2) {
            uint4 x[4];
            bool ok[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) ok[u] = load(16 * (s + (u >> 1)) + 2 * w + (u & 1), x[u]);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (ok[u]) add8((u & 1) ? a1 : a0, x[u]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) tot[i] = w == 0 ? a0[i] + a1[i] : tot[i] + (a0[i] + a1[i]);
    }
}

template <bool PAGED>
__global__ __launch_bounds__(kThreads) void k_pool(PoolArgs a, SeqTable t) {
    const int gb = blockIdx.x;
    // prefix_only: the grid covers the K and V chunks of prefix blocks only.
    const int c = (a.prefix_only ? a.q_chunks : 0) + blockIdx.y * kThreads + threadIdx.x;
    if (c >= a.total_chunks) return;
    const int b = request_of_block(t, gb);
    const int I = gb - t.blk_off[b];
    const int first = first_block(t, b);
    if (a.prefix_only && I >= first) return;
    const int len = context_len(t, b, a.B);
    const int t0 = I * a.B;
    const int n = min(a.B, len - t0);

    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float mean[8];
    if (c < a.q_chunks) {
        // Q: packed rows of this call's queries, never paged.  Prefix blocks
        // (chunked prefill) have no queries here, and a chunk that starts
        // inside its first block holds that block's tokens lo .. n-1 only.
        if (I < first) return;
        const int col = c * 8;
        const int ph = chunk_phase(t, b, a.B);
        const int lo = I == first ? ph : 0;
        // With skeleton queries only every q_stride-th token of the block
        // counts (the host admits them for block-aligned chunks only).
        const int64_t row_elems = (int64_t)a.Hq * a.D;
        // Row 0 of the block is query row q0 (tokens before lo are not in the call).
        const uint16_t* p = a.q + (int64_t)(t.tok_off[b] + (I - first) * a.B - ph) * row_elems + col;
        const int stride = a.q_stride;
        tree_sum(a.B, [&](int tok, uint4& x) {
            const bool ok = tok >= lo && tok < n && tok % stride == 0;
            x = ok ? ntload(p + (int64_t)tok * row_elems) : make_uint4(0, 0, 0, 0);
            return ok;
        }, acc);
        const int nq = (n - lo + stride - 1) / stride;
        const float fn = (float)nq;
#pragma unroll
        for (int i = 0; i < 8; ++i) mean[i] = acc[i] / fn;
        const int64_t off = ((int64_t)(col / a.D) * t.total_qblocks + qblock_row(t, b, I)) * a.D + col % a.D;
        reinterpret_cast<float4*>(a.pq + off)[0] = make_float4(mean[0], mean[1], mean[2], mean[3]);
        reinterpret_cast<float4*>(a.pq + off)[1] = make_float4(mean[4], mean[5], mean[6], mean[7]);
        return;
    }
    int cc = c - a.q_chunks;
    const bool isv = cc >= a.k_chunks;
    if (isv) cc -= a.k_chunks;
    const int col = cc * 8;
    const int h = col / a.D;
    const int dd = col % a.D;
    // Pooled cache entry of this block: the page holding its first token.
    float* cache = nullptr;
    if (PAGED && a.pcache) {
        const int page = a.kv.block_table[(int64_t)b * a.kv.max_pages + a.kv.page_of(t0)];
        if ((unsigned)page < (unsigned)a.kv.num_pages)
            cache = a.pcache + (((int64_t)(isv ? a.kv.num_pages : 0) + page) * a.Hkv + h) * a.D + dd;
    }
    if (PAGED && a.reuse && I < first) {
        // A prefix block pooled by an earlier call.
        float4 m0 = make_float4(0.f, 0.f, 0.f, 0.f), m1 = m0;
        if (cache) {
            m0 = reinterpret_cast<const float4*>(cache)[0];
            m1 = reinterpret_cast<const float4*>(cache)[1];
        }
        mean[0] = m0.x; mean[1] = m0.y; mean[2] = m0.z; mean[3] = m0.w;
        mean[4] = m1.x; mean[5] = m1.y; mean[6] = m1.z; mean[7] = m1.w;
    } else {
        const uint16_t* base = isv ? a.v : a.k;
        const int64_t row_elems = (int64_t)a.Hkv * a.D;
        const int tok0 = t.tok_off[b];
        tree_sum(a.B, [&](int tok, uint4& x) {
            const int64_t row = tok < n ? kv_row<PAGED>(a.kv, b, tok0, t0 + tok) : -1;
            x = row >= 0 ? ntload(base + row * row_elems + col) : make_uint4(0, 0, 0, 0);
            return row >= 0;
        }, acc);
        const float fn = (float)n;
#pragma unroll
        for (int i = 0; i < 8; ++i) mean[i] = acc[i] / fn;
        if (cache) {
            reinterpret_cast<float4*>(cache)[0] = make_float4(mean[0], mean[1], mean[2], mean[3]);
            reinterpret_cast<float4*>(cache)[1] = make_float4(mean[4], mean[5], mean[6], mean[7]);
        }
    }
    const int64_t off = ((int64_t)h * t.total_blocks + gb) * a.D + dd;
    float* dst = isv ? a.pv : a.pk;
    if (dst) {
        reinterpret_cast<float4*>(dst + off)[0] = make_float4(mean[0], mean[1], mean[2], mean[3]);
        reinterpret_cast<float4*>(dst + off)[1] = make_float4(mean[4], mean[5], mean[6], mean[7]);
    }
    if (a.pkv16) {   // the same means rounded to bf16 (nearest even): the correction's operands
        uint16_t* dst16 = a.pkv16 + (isv ? (int64_t)a.Hkv * t.total_blocks * a.D : 0);
        *reinterpret_cast<uint4*>(dst16 + off) =
            make_uint4(pack_bf16(mean[0], mean[1]), pack_bf16(mean[2], mean[3]), pack_bf16(mean[4], mean[5]),
                       pack_bf16(mean[6], mean[7]));
    }
}

}  // namespace

hipError_t launch_pool(const PoolArgs& a, const SeqTable& t, bool paged, hipStream_t s) {
    if (t.total_blocks == 0) return hipSuccess;
    // Blocks vary fastest in the dispatch order, so the workgroups in flight
    // spread over the whole tensors (dispatching a block's three chunk groups
    // together ran 5% slower).
    const int nchunks = a.total_chunks - (a.prefix_only ? a.q_chunks : 0);
    if (nchunks <= 0) return hipSuccess;
    dim3 grid(t.total_blocks, (nchunks + kThreads - 1) / kThreads);
    if (paged)
        hipLaunchKernelGGL(k_pool<true>, grid, dim3(kThreads), 0, s, a, t);
    else
        hipLaunchKernelGGL(k_pool<false>, grid, dim3(kThreads), 0, s, a, t);
    return hipGetLastError();
}
