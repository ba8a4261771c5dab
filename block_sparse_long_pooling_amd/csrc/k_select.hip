// Pooled block scores, max-based dynamic threshold and list compaction
// (FlashPrefill, gist.science technical summary, sections 2.A-2.C).
//
// For query head h and query block I, s[J] = sigma * q_bar[h,I] . k_bar[h/g,J]
// over J <= I.  Block J is kept iff its softmax score is at least alpha times
// the row's largest, i.e. s[J] - max_J s >= ln(alpha).  Kept blocks are
// written in ascending J to the (h, I) list, which is never empty.
//
// A workgroup owns 32 score rows: TI consecutive query blocks x the g query
// heads of one KV head, so every k_bar row it loads serves 32 rows.  The
// (L/B)^2 score matrix is never stored: phase 1 takes each row's max, phase 2
// recomputes the same scores (same instruction sequence, bit-identical) into
// a keep bitmap in LDS, phase 3 compacts it in ascending J.  The dot products run on bf16 MFMA with each
// fp32 operand split into hi + lo bf16 parts (hi*hi + hi*lo + lo*hi), which
// is within ~2^-17 of the fp32 product sum -- far below the 1e-3 band in
// which the threshold decision is allowed to differ from an exact one.
#include "fp_launch.h"

// Scores feed both the row max (pass 1) and the compare s - max (pass 2); no
// multiply may be fused into a later add, or the two passes would disagree.
#pragma clang fp contract(off)

namespace {

__device__ __forceinline__ void split8(const float4& x0, const float4& x1, bf16x8& hi, bf16x8& lo) {
    float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        __bf16 h = (__bf16)x[i];
        hi[i] = h;
        lo[i] = (__bf16)(x[i] - (float)h);
    }
}

// Three independent MFMA chains (hi*hi, hi*lo, lo*hi) summed in a fixed
// order: the same instruction sequence gives the same bits in every pass.
template <int D>
__device__ __forceinline__ f32x16 tile_scores(const bf16x8* qh, const bf16x8* ql, const float4* kb, float scale) {
    f32x16 a0 = {}, a1 = {}, a2 = {};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        bf16x8 kh, kl;
        split8(kb[2 * kk], kb[2 * kk + 1], kh, kl);
        a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qh[kk], kh, a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qh[kk], kl, a1, 0, 0, 0);
        a2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ql[kk], kh, a2, 0, 0, 0);
    }
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = (a0[r] + (a1[r] + a2[r])) * scale;
    return acc;
}

template <int D>
__device__ __forceinline__ void load_kbar(const float* pk, int64_t row0, int J, int nb, int half, float4* kb) {
    if (J < nb) {
        const float4* src = reinterpret_cast<const float4*>(pk + (row0 + J) * D + 8 * half);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            kb[2 * kk] = src[4 * kk];       // d = 8*half + 16*kk .. +3
            kb[2 * kk + 1] = src[4 * kk + 1];
        }
    } else {
#pragma unroll
        for (int i = 0; i < D / 8; ++i) kb[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

constexpr int kWaves = 4;
constexpr int kMaxColTiles = FP_MAX_BLOCKS / 2 / 32;   // 32-block column tiles per row

// One workgroup (4 waves) owns 32 score rows: TI consecutive query blocks x
// the g query heads of one KV head.  The waves split the 32-block column
// tiles (wave w takes tiles w, w+4, ...).  Phase 1: row maxima, combined in
// LDS.  Phase 2: the same scores again, thresholded; each tile's keep bits go
// to an LDS bitmap [tile][row].  Phase 3: each wave compacts 8 rows in
// ascending J with a wave-wide prefix sum over the tiles' popcounts.
template <int D>
__global__ __launch_bounds__(64 * kWaves, 2) void k_select(SelArgs a, SeqTable t) {
    __shared__ uint32_t bits[kMaxColTiles][32];
    __shared__ float pmax[kWaves][32];
    __shared__ float rmax[32];

    const int tid = threadIdx.x;
    const int wv = tid >> 6, lane = tid & 63;
    const int rank = blockIdx.x / a.Hkv;
    const int hk = blockIdx.x % a.Hkv;
    int b, local;
    item_of(t, rank, b, local);
    const int nb = seq_blocks(t, b);
    const int first = first_block(t, b);             // query blocks are first .. nb-1
    const int ntiles = (nb - first + a.TI - 1) / a.TI;
    const int I0 = first + (ntiles - 1 - local) * a.TI;
    const int gblk0 = t.blk_off[b];
    const int rows = a.TI * a.g;
    const int rho = lane & 31;
    const int half = lane >> 5;

    // A operand: row rho = (query block I0 + rho / g, head hk*g + rho % g).
    bf16x8 qh[D / 16], ql[D / 16];
    {
        const int I = I0 + rho / a.g;
        const int h = hk * a.g + rho % a.g;
        const bool valid = rho < rows && I < nb;
        const float4* src = reinterpret_cast<const float4*>(
            a.pq + ((int64_t)h * t.total_qblocks + qblock_row(t, b, valid ? I : I0)) * D + 8 * half);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            float4 x0 = valid ? src[4 * kk] : make_float4(0.f, 0.f, 0.f, 0.f);
            float4 x1 = valid ? src[4 * kk + 1] : make_float4(0.f, 0.f, 0.f, 0.f);
            split8(x0, x1, qh[kk], ql[kk]);
        }
    }
    // Output register r of this lane holds row (r%4) + 8*(r/4) + 4*half.
    int rowI[16];
    bool rowOk[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int rr = (r & 3) + 8 * (r >> 2) + 4 * half;
        rowI[r] = I0 + rr / a.g;
        rowOk[r] = rr < rows && rowI[r] < nb;
    }
    const int ncol = min(nb, I0 + a.TI);
    const int ntile = (ncol + 31) >> 5;
    const int64_t krow0 = (int64_t)hk * t.total_blocks + gblk0;

    // Phase 1: partial row maxima over this wave's tiles.
    float m[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) m[r] = -INFINITY;
    float4 kb[D / 8];
    for (int ct = wv; ct < ntile; ct += kWaves) {
        load_kbar<D>(a.pk, krow0, 32 * ct + rho, nb, half, kb);
        const f32x16 s = tile_scores<D>(qh, ql, kb, a.scale);
        const int J = 32 * ct + rho;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (rowOk[r] && J <= rowI[r]) m[r] = fmaxf(m[r], s[r]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) m[r] = fmaxf(m[r], __shfl_xor(m[r], off));
    }
    if (rho == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) pmax[wv][(r & 3) + 8 * (r >> 2) + 4 * half] = m[r];
    }
    __syncthreads();
    if (tid < 32) {
        float x = pmax[0][tid];
#pragma unroll
        for (int w2 = 1; w2 < kWaves; ++w2) x = fmaxf(x, pmax[w2][tid]);
        rmax[tid] = x;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) m[r] = rmax[(r & 3) + 8 * (r >> 2) + 4 * half];

    // Phase 2: keep bits per (tile, row).
    for (int ct = wv; ct < ntile; ct += kWaves) {
        load_kbar<D>(a.pk, krow0, 32 * ct + rho, nb, half, kb);
        const f32x16 s = tile_scores<D>(qh, ql, kb, a.scale);
        const int J = 32 * ct + rho;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const bool keep = rowOk[r] && J <= rowI[r] && (s[r] - m[r] >= a.ln_alpha);
            const uint64_t mask = __ballot(keep);
            if (lane == 0) {
                const int rr = (r & 3) + 8 * (r >> 2);
                bits[ct][rr] = (uint32_t)mask;
                bits[ct][rr + 4] = (uint32_t)(mask >> 32);
            }
        }
    }
    __syncthreads();

    // Phase 3: ordered compaction, 8 rows per wave, 64 tiles per step.
    for (int rr = wv; rr < 32; rr += kWaves) {
        const int ii = rr / a.g, hi = rr % a.g;
        const int I = I0 + ii;
        if (rr >= rows || I >= nb) continue;                 // wave-uniform
        const int h = hk * a.g + hi;
        int32_t* out = a.kv_idx + list_row(t, b, h, I, nb, first);
        int base = 0;
        for (int c0 = 0; c0 < ntile; c0 += 64) {
            const int ct = c0 + lane;
            uint32_t wbits = 0u;
            if (ct < ntile) {
                if (a.shared) {
                    // Group-shared selection: the union of the g heads' keep bits
                    // of this query block (rows ii*g .. ii*g+g-1 of this workgroup).
                    for (int j = 0; j < a.g; ++j) wbits |= bits[ct][ii * a.g + j];
                } else {
                    wbits = bits[ct][rr];
                }
            }
            const int n = __popc(wbits);
            int incl = n;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(incl, off);
                if (lane >= off) incl += y;
            }
            int pos = base + incl - n;
            uint32_t wb = wbits;
            while (wb) {
                const int bit = __ffs(wb) - 1;
                wb &= wb - 1;
                out[pos++] = 32 * ct + bit;
            }
            base += __shfl(incl, 63);
        }
        if (lane == 0) a.kv_cnt[count_index(t, a.Hq, b, h, I, nb, first)] = base;
    }
}

}  // namespace

hipError_t launch_select(const SelArgs& a, const SeqTable& t, hipStream_t s) {
    if (t.total_items == 0) return hipSuccess;
    dim3 grid(t.total_items * a.Hkv);
    if (a.D == 64)
        hipLaunchKernelGGL(k_select<64>, grid, dim3(64 * kWaves), 0, s, a, t);
    else
        hipLaunchKernelGGL(k_select<128>, grid, dim3(64 * kWaves), 0, s, a, t);
    return hipGetLastError();
}
