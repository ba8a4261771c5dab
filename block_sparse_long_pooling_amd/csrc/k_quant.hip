// Fused fp8 quantization and block-mean pooling of Q, K and V in one pass
// over the bf16 data (FlashPrefill V2 abstract: FP8 inference; the fp8
// recipe is one scale per (head, block) = amax / 448, codes = OCP E4M3 of
// clamp(x / scale), and the pooled means that drive selection are those of
// the bf16 data, as in the pooling kernel).
//
// Blocks are those of a request table (one sequence, or a batch whose K and
// V rows may live in a paged cache: codes then go to the same place in an
// e4m3 page pool, and each block's scale to the entry of its first page).
// In chunk mode (chunked prefill over the paged cache) the grid covers only
// the query blocks of each request's chunk: K and V of such a block are
// re-encoded whole from the bf16 pages, the tokens before the chunk
// included, so a block that an earlier chunk left partial ends up encoded as
// a prefill of the whole context would encode it; Q of the block holds only
// the chunk's queries in it.  Its K and V means also go to the caller's
// pooled cache.  The block sums run in a fixed token tree that the pooling
// kernel reproduces (tree_sum in k_pool.hip), so both kernels' means are
// bit-identical.
// A workgroup (8 waves) owns one block of one tensor for a group of heads
// whose chunks of 8 bf16 make 32 chunks per token row (two heads at d 128,
// four at d 64), i.e. 512 contiguous bytes.  Lane l of wave w handles chunk
// l % 32 of tokens 16 s + 2 w + l / 32: a wave reads two full 512-byte rows
// per load, and each thread keeps its B / 16 chunks in registers.  Block sums
// and the per-head absolute maximum are reduced across lanes and waves; the
// means and the scale are written, then the codes are formed from the values
// still in registers (every thread derives its head's scale from the
// waves' maxima itself).  HBM sees one read of the bf16 data and one write of
// the codes.  The scale and x / scale are correctly rounded fp32 divisions,
// so every code is decided in the same precision as the format's reference.
// x / scale takes three operations: with y the correctly rounded 1 / scale
// (one division per head and block), q = x y, the remainder x - q scale
// (exact with an FMA) and q + remainder * y rounded give the correctly
// rounded quotient (Markstein's correction step).  Quotients small enough to
// lose precision as fp32 subnormals lie far below the smallest e4m3 code and
// encode as zero either way.
#include "fp_launch.h"

// The quotient steps below are explicit FMAs; nothing else may be fused.
#pragma clang fp contract(off)

namespace {

constexpr int kWaves = 8;

// Six waves per SIMD (three workgroups per CU): more loads in flight, at
// the cost of a small spill (28 bytes) in the paged variants.
template <int D, int B, bool PAGED, bool CHUNK>
__global__ __launch_bounds__(64 * kWaves, 6) void k_quant_pool(QuantArgs a, SeqTable t) {
    constexpr int CPH = D / 8;             // chunks per head
    constexpr int HPG = 32 / CPH;          // heads per workgroup
    constexpr int NS = B / (2 * kWaves);   // tokens per thread
    __shared__ float psum[kWaves][32][8];
    __shared__ float pmax[kWaves][HPG];

    const int J = blockIdx.x;                       // block of all requests (chunk mode: query block row)
    int g = blockIdx.y, ts = 0;
    if (g >= a.groups[0]) {
        g -= a.groups[0];
        ts = 1;
        if (g >= a.groups[1]) {
            g -= a.groups[1];
            ts = 2;
        }
    }
    const int H = a.H[ts];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int ch = lane & 31, hf = lane >> 5;
    const int hl = ch / CPH;               // head within the group
    const int h = g * HPG + hl;
    const bool hv = h < H;
    int b, I, kvJ;                                  // request, block of request b, block of all requests
    if (CHUNK) {
        b = request_of_qblock(t, J);
        I = first_block(t, b) + J - (t.blk_off[b] - t.pre_off[b]);
        kvJ = t.blk_off[b] + I;
    } else {
        b = request_of_block(t, J);
        I = J - t.blk_off[b];
        kvJ = J;
    }
    const int t0 = I * B;
    const int n = min(B, context_len(t, b, B) - t0);
    // Q rows of a chunk: tokens lo .. n-1 of the block, query row q0 + tok
    // (the chunk may start inside its first block).
    int lo = 0;
    int64_t q0 = (int64_t)t.tok_off[b] + t0;
    if (CHUNK && ts == 0) {
        const int first = first_block(t, b), ph = chunk_phase(t, b, B);
        lo = I == first ? ph : 0;
        q0 = (int64_t)t.tok_off[b] + (I - first) * B - ph;
    }
    const bool pg = PAGED && ts > 0;                // K and V rows live in pages
    const int64_t row = (int64_t)H * D;
    const int64_t col = (int64_t)g * HPG * D + ch * 8;
    // Packed rows: offsets from the block's row 0; paged rows: from the
    // pool's start.
    const int64_t base = pg ? col : q0 * row + col;
    const KVLayout kv = a.kv;
    // Row of token tok of this block relative to the base (-1: a page id out
    // of range, read as zeros and not written).
    auto row_of = [=](int tok) -> int64_t { return pg ? kv_row<true>(kv, b, 0, t0 + tok) : tok; };
    const uint16_t* src = a.src[ts] + base;

    // Q_bar may average only the skeleton queries (every q_stride-th token).
    const int stride = ts == 0 ? a.q_stride : 1;
    // Whole blocks of packed rows with every head of the group present and
    // every token counted (the common case) take a path without per-token
    // tests: unconditional loads and stores at 32-bit offsets from the
    // block's first row.  Only in the packed-layout kernel: in the paged one
    // the second path's registers spilled inside the token loops (2.3x
    // slower).
    const bool full = !PAGED && n == B && stride == 1 && (g + 1) * HPG <= H;
    uint4 x[NS];
    if (full) {
        const char* src8 = reinterpret_cast<const char*>(src);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int tok = 2 * kWaves * s + 2 * w + hf;
            x[s] = *reinterpret_cast<const uint4*>(src8 + (uint32_t)tok * (uint32_t)(row * 2));
        }
    } else {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int tok = 2 * kWaves * s + 2 * w + hf;
            const int64_t r = row_of(min(max(tok, lo), n - 1));
            x[s] = (hv && tok >= lo && tok < n && r >= 0) ? *reinterpret_cast<const uint4*>(src + r * row)
                                                          : make_uint4(0, 0, 0, 0);
        }
    }
    float sum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float amax = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const uint32_t wd[4] = {x[s].x, x[s].y, x[s].z, x[s].w};
        const bool counted = full || (2 * kWaves * s + 2 * w + hf) % stride == 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = bf16_lo(wd[i]), hi = bf16_hi(wd[i]);
            sum[2 * i] += counted ? lo : 0.f;
            sum[2 * i + 1] += counted ? hi : 0.f;
            amax = fmaxf(amax, fmaxf(fabsf(lo), fabsf(hi)));
        }
    }
    // Sums: the two token halves of a wave, then the waves (in wave order,
    // so the sum order is fixed).
#pragma unroll
    for (int i = 0; i < 8; ++i) sum[i] += __shfl_xor(sum[i], 32);
    // amax: the head's chunks within the wave, both halves.
#pragma unroll
    for (int off = 1; off < CPH; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    if (hf == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) psum[w][ch][i] = sum[i];
        if (ch % CPH == 0) pmax[w][hl] = amax;
    }
    __syncthreads();
    if (!hv) return;
    // Every thread forms its head's scale from the waves' maxima itself (the
    // same operations in the same order, so the same bits), so the codes need
    // no second barrier.
    float am = pmax[0][hl];
#pragma unroll
    for (int w2 = 1; w2 < kWaves; ++w2) am = fmaxf(am, pmax[w2][hl]);
    const float sc = am > 0.f ? __fdiv_rn(am, kE4M3Max) : 1.f;
    const float ry = __fdiv_rn(1.f, sc);
    if (w == 0 && hf == 0) {
        {
            float m[8];
            const float cnt = (float)((n - lo + stride - 1) / stride);   // counted tokens (lo = 0 when stride > 1)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float t = psum[0][ch][i];
#pragma unroll
                for (int w2 = 1; w2 < kWaves; ++w2) t += psum[w2][ch][i];
                m[i] = t / cnt;
            }
            // Q means by query-block row J; K and V means by KV block of all requests.
            const int dd = (ch % CPH) * 8;
            const int64_t off = ((int64_t)h * (CHUNK && ts > 0 ? t.total_blocks : a.nB) + (ts > 0 ? kvJ : J)) * D + dd;
            float* dst = ts == 0 ? a.pq : (ts == 1 ? a.pk : nullptr);
            if (dst) {
                reinterpret_cast<float4*>(dst + off)[0] = make_float4(m[0], m[1], m[2], m[3]);
                reinterpret_cast<float4*>(dst + off)[1] = make_float4(m[4], m[5], m[6], m[7]);
            }
            if (ts > 0 && a.pkv16)
                *reinterpret_cast<uint4*>(a.pkv16 + (ts == 2 ? (int64_t)a.H[1] * (CHUNK ? t.total_blocks : a.nB) * D : 0) + off) =
                    make_uint4(pack_bf16(m[0], m[1]), pack_bf16(m[2], m[3]), pack_bf16(m[4], m[5]),
                               pack_bf16(m[6], m[7]));
            if (CHUNK && ts > 0 && a.pcache) {
                // The pooled cache entry of the page that holds the block's first token.
                const int page = a.kv.block_table[(int64_t)b * a.kv.max_pages + t0 / a.kv.page_size];
                if ((unsigned)page < (unsigned)a.kv.num_pages) {
                    float* e = a.pcache + (((int64_t)(ts == 2 ? a.kv.num_pages : 0) + page) * H + h) * D + dd;
                    reinterpret_cast<float4*>(e)[0] = make_float4(m[0], m[1], m[2], m[3]);
                    reinterpret_cast<float4*>(e)[1] = make_float4(m[4], m[5], m[6], m[7]);
                }
            }
        }
        if (ch % CPH == 0) {
            if (pg) {
                // Paged K and V: the scale goes with the page of the block's first token.
                const int page = a.kv.block_table[(int64_t)b * a.kv.max_pages + t0 / a.kv.page_size];
                if ((unsigned)page < (unsigned)a.kv.num_pages) a.scale[ts][(int64_t)page * H + h] = sc;
            } else {
                a.scale[ts][(int64_t)h * a.nB + J] = sc;
            }
        }
    }
    // The correction step turns a quotient of -0 into +0 (-0 + +0 rounds to
    // +0); the sign of x restores it, so -0 inputs encode as -0 like x / scale.
    auto quot = [&](float xv) {
        const float q = xv * ry;
        const float r = fmaf(-q, sc, xv);
        return fminf(fmaxf(copysignf(fmaf(r, ry, q), xv), -kE4M3Max), kE4M3Max);
    };
    uint8_t* dst = a.codes[ts] + base;
    // The codes convert the packed words again: the block's values would
    // otherwise stay unpacked across the barrier (twice the registers).
#pragma unroll
    for (int s = 0; s < NS; ++s) asm volatile("" : "+v"(x[s].x), "+v"(x[s].y), "+v"(x[s].z), "+v"(x[s].w));
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int tok = 2 * kWaves * s + 2 * w + hf;
        if (!full && (tok < lo || tok >= n)) continue;
        const uint32_t wd[4] = {x[s].x, x[s].y, x[s].z, x[s].w};
        uint32_t out[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            float y[4];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                y[2 * k] = quot(bf16_lo(wd[2 * i + k]));
                y[2 * k + 1] = quot(bf16_hi(wd[2 * i + k]));
            }
            int v = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
            v = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], v, true);
            out[i] = (uint32_t)v;
        }
        if (full) {
            *reinterpret_cast<uint2*>(dst + (uint32_t)tok * (uint32_t)row) = make_uint2(out[0], out[1]);
        } else {
            const int64_t r = row_of(tok);
            if (r >= 0) *reinterpret_cast<uint2*>(dst + r * row) = make_uint2(out[0], out[1]);
        }
    }
}

template <int D, int B>
hipError_t launch_t(const QuantArgs& a, const SeqTable& t, bool paged, bool chunk, hipStream_t s) {
    constexpr int HPG = 32 / (D / 8);
    QuantArgs b = a;
    for (int i = 0; i < 3; ++i) b.groups[i] = (a.H[i] + HPG - 1) / HPG;
    const dim3 grid(a.nB, b.groups[0] + b.groups[1] + b.groups[2]);
    if (chunk)
        hipLaunchKernelGGL((k_quant_pool<D, B, true, true>), grid, dim3(64 * kWaves), 0, s, b, t);
    else if (paged)
        hipLaunchKernelGGL((k_quant_pool<D, B, true, false>), grid, dim3(64 * kWaves), 0, s, b, t);
    else
        hipLaunchKernelGGL((k_quant_pool<D, B, false, false>), grid, dim3(64 * kWaves), 0, s, b, t);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_pool(const QuantArgs& a, const SeqTable& t, bool paged, bool chunk, hipStream_t s) {
    if (a.nB == 0) return hipSuccess;
    if (chunk && (!paged || a.nB != t.total_qblocks)) return hipErrorInvalidValue;
    if (a.D == 128 && a.B == 128) return launch_t<128, 128>(a, t, paged, chunk, s);
    if (a.D == 128 && a.B == 64) return launch_t<128, 64>(a, t, paged, chunk, s);
    if (a.D == 64 && a.B == 128) return launch_t<64, 128>(a, t, paged, chunk, s);
    if (a.D == 64 && a.B == 64) return launch_t<64, 64>(a, t, paged, chunk, s);
    return hipErrorInvalidValue;
}
