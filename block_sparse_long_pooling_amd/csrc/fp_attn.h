// Pieces shared by the bf16 and fp8 attention kernels (gfx950): the LDS-only
// barrier, tile geometry, the online-softmax update and the output store.
// The tile walk and the MFMA loops are in attn_walk.h; k_attn.hip describes
// the overall design.
#pragma once
#include "fp_launch.h"

namespace fp_attn {

// Workgroup barrier that orders LDS accesses only: this wave's LDS
// operations complete (lgkmcnt 0), then all waves meet.  __syncthreads(), and
// any release fence, also waits for every outstanding global access and LDS
// DMA (vmcnt 0), which would stall on tile DMAs and loads that are meant to
// stay in flight across the barrier.  Callers that need a DMA's data wait for
// it explicitly first.  The memory clobber keeps the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

constexpr float kLn2 = 0.69314718055994530942f;

// Row statistics of a query live in lanes l and l ^ 32.  v_permlane32_swap
// exchanges the halves of two copies of v, which then hold the lower and the
// upper half's value in every lane: a register move, where a lane shuffle
// (ds_bpermute) would be an LDS round trip in the middle of the softmax.  Both
// lanes of a pair get the same bits.
__device__ __forceinline__ float pair_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int BLK>
struct Tile {
    static constexpr int NW = BLK / 32;     // waves per workgroup
    static constexpr int NT = 64 * NW;      // threads
    static constexpr int KCH = D / 8;       // 16-byte chunks per K row
    static constexpr int VCH = BLK / 8;     // 16-byte chunks per BLK-key row
    static constexpr int NSUB = BLK / 32;   // 32-key subtiles of S^T
    static constexpr int NDS = D / 32;      // 32-row d subtiles of O^T
};

// Online-softmax update.  s holds raw scores q.k (masked entries -inf); the
// logit in log2 units is s * c + bias.  The running max m only moves when a
// tile raises it by more than kLazy (log2 units): P then stays below 2^kLazy,
// which bf16 and the fp32 accumulators hold exactly enough, and most tiles
// skip rescaling O.  Packs P to bf16 pairs pk[sub][0..7].
#ifndef FP_LAZY_LOG2
#define FP_LAZY_LOG2 8.f
#endif
constexpr float kLazy = FP_LAZY_LOG2;

template <int NSUB, int NDS>
__device__ __forceinline__ void softmax_update(f32x16* s, float c, float bias, float& m, float& l, f32x16* o,
                                               uint32_t (*pk)[8]) {
    float mt = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[sub][r]);
    mt = pair_max(mt);
    const float mt2 = (mt == -INFINITY) ? -INFINITY : fmaf(mt, c, bias);
    const bool grow = mt2 > m + kLazy;
    if (__ballot(grow)) {
        const float m_new = grow ? mt2 : m;
        const float alpha = grow ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[ds][r] *= alpha;
    }
    const float off = bias - (m == -INFINITY ? 0.f : m);
    // The row sum adds the bf16-rounded P pairs (one dot2 per pair), i.e.
    // exactly the weights the PV product applies.
    // Four independent partial sums keep the accumulate chain short.
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(s[sub][2 * i], c, off));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(s[sub][2 * i + 1], c, off));
            pk[sub][i] = pack_bf16(p0, p1);
            part[i & 3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[sub][i]), ones, part[i & 3],
                                                         false);
        }
    }
    l += (part[0] + part[1]) + (part[2] + part[3]);
}

// Normalise O, stage the bf16 tile in LDS (reusing tile buffers: rows
// 0 .. BLK/2-1 in lo_rows, the rest in hi_rows, each [BLK/2][D] bf16) and
// store full rows; write the natural-log sum of exp when requested.
template <int D, int BLK>
__device__ __forceinline__ void store_output(const AttnArgs& a, const SeqTable& t, int h, int q0, int lo, int nI,
                                             int qr, int half, float m, float l, const f32x16* o, uint4* lo_rows,
                                             uint4* hi_rows, int tid) {
    using T = Tile<D, BLK>;
    constexpr int HR = BLK / 2;
    const float l_tot = pair_sum(l);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    __syncthreads();
    uint4* mine = qr < HR ? lo_rows + qr * T::KCH : hi_rows + (qr - HR) * T::KCH;   // uniform per wave
#pragma unroll
    for (int ds = 0; ds < T::NDS; ++ds)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int chunk = 4 * ds + g4;        // d0 = 32 ds + 8 g4 + 4 half
            uint2 v2 = make_uint2(pack_bf16(o[ds][4 * g4] * inv, o[ds][4 * g4 + 1] * inv),
                                  pack_bf16(o[ds][4 * g4 + 2] * inv, o[ds][4 * g4 + 3] * inv));
            reinterpret_cast<uint2*>(&mine[chunk ^ (qr % T::KCH)])[half] = v2;
        }
    __syncthreads();
    for (int i = tid; i < (nI - lo) * T::KCH; i += T::NT) {
        const int row = lo + i / T::KCH, ch = i % T::KCH;
        const uint4* src = row < HR ? lo_rows + row * T::KCH : hi_rows + (row - HR) * T::KCH;
        *reinterpret_cast<uint4*>(a.out + ((int64_t)(q0 + row) * a.Hq + h) * D + ch * 8) =
            src[ch ^ (row % T::KCH)];
    }
    if (a.lse && half == 0 && qr >= lo && qr < nI)
        a.lse[(int64_t)h * t.total_tokens + q0 + qr] = (m + __log2f(l_tot)) * kLn2;
}

}  // namespace fp_attn
