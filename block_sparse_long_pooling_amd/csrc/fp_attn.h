// Tile machinery shared by the bf16 and fp8 attention kernels (gfx950):
// LDS tile layouts, the S^T = K Q^T and O^T += V^T P^T MFMA loops, and the
// online-softmax update.  See k_attn.hip for the overall design.
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

// Swap bits 2 and 3 of a key position inside its 16-key group.
__device__ __forceinline__ int key_perm(int p) { return (p & ~0xC) | ((p & 4) << 1) | ((p & 8) >> 1); }

// 8 rows x 8 bf16 (x[u] = row u) -> 8 columns (y[j] = column j of all rows).
__device__ __forceinline__ void transpose8(const uint4* x, uint4* y) {
    const uint32_t* xs = reinterpret_cast<const uint32_t*>(x);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t w[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t a = xs[(2 * m) * 4 + j / 2];
            const uint32_t c = xs[(2 * m + 1) * 4 + j / 2];
            w[m] = (j & 1) ? ((a >> 16) | (c & 0xffff0000u)) : ((a & 0xffffu) | (c << 16));
        }
        y[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

__device__ __forceinline__ uint4 f32x8_to_bf16(const float4& a, const float4& b) {
    return make_uint4(pack_bf16(a.x, a.y), pack_bf16(a.z, a.w), pack_bf16(b.x, b.y), pack_bf16(b.z, b.w));
}

template <int D, int BLK>
struct Tile {
    static constexpr int NW = BLK / 32;     // waves per workgroup
    static constexpr int NT = 64 * NW;      // threads
    static constexpr int KCH = D / 8;       // 16-byte chunks per K row
    static constexpr int VCH = BLK / 8;     // 16-byte chunks per V^T row
    static constexpr int NSUB = BLK / 32;   // 32-key subtiles of S^T
    static constexpr int NDS = D / 32;      // 32-row d subtiles of O^T
};

// K tile [BLK keys][D] and V^T tile [D][BLK keys (permuted)] of KV block J.
template <int D, int BLK, bool PAGED>
__device__ __forceinline__ void load_kv_tile(const uint16_t* kb, const uint16_t* vb, const KVLayout& L, int b,
                                             int tok0, int len, int J, int Hkv, int hk, uint4* lk, uint4* lv,
                                             int tid) {
    using T = Tile<D, BLK>;
    const int64_t rs = (int64_t)Hkv * D;
    for (int i = tid; i < BLK * T::KCH; i += T::NT) {
        const int row = i / T::KCH, ch = i % T::KCH;
        const int tr = J * BLK + row;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (tr < len) {
            const int64_t r = kv_row<PAGED>(L, b, tok0, tr);
            if (r >= 0) val = *reinterpret_cast<const uint4*>(kb + r * rs + (int64_t)hk * D + ch * 8);
        }
        lk[row * T::KCH + (ch ^ (row % T::KCH))] = val;
    }
    for (int i = tid; i < T::VCH * T::KCH; i += T::NT) {
        const int kg = i / T::KCH, dc = i % T::KCH;
        uint4 x[8], y[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int tr = J * BLK + key_perm(8 * kg + u);
            x[u] = make_uint4(0, 0, 0, 0);
            if (tr < len) {
                const int64_t r = kv_row<PAGED>(L, b, tok0, tr);
                if (r >= 0) x[u] = *reinterpret_cast<const uint4*>(vb + r * rs + (int64_t)hk * D + dc * 8);
            }
        }
        transpose8(x, y);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int drow = 8 * dc + j;
            lv[drow * T::VCH + (kg ^ (drow % T::VCH))] = y[j];
        }
    }
}

// Pooled K_bar / V_bar (bf16) of blocks c0 .. c0+BLK-1 (zero for blocks >= I).
template <int D, int BLK>
__device__ __forceinline__ void load_pooled_tile(const uint16_t* pk, const uint16_t* pv, int64_t prow0, int c0, int I,
                                                 uint4* lk, uint4* lv, int tid) {
    using T = Tile<D, BLK>;
    for (int i = tid; i < BLK * T::KCH; i += T::NT) {
        const int row = i / T::KCH, ch = i % T::KCH;
        const int J = c0 + row;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (J < I) val = *reinterpret_cast<const uint4*>(pk + (prow0 + J) * D + ch * 8);
        lk[row * T::KCH + (ch ^ (row % T::KCH))] = val;
    }
    for (int i = tid; i < T::VCH * T::KCH; i += T::NT) {
        const int kg = i / T::KCH, dc = i % T::KCH;
        uint4 x[8], y[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int J = c0 + key_perm(8 * kg + u);
            x[u] = make_uint4(0, 0, 0, 0);
            if (J < I) x[u] = *reinterpret_cast<const uint4*>(pv + (prow0 + J) * D + dc * 8);
        }
        transpose8(x, y);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int drow = 8 * dc + j;
            lv[drow * T::VCH + (kg ^ (drow % T::VCH))] = y[j];
        }
    }
}

// S^T[sub] = K[32 sub + .., :] Q^T for this wave's 32 queries.
template <int D, int BLK>
__device__ __forceinline__ void qk_tile(const uint4* lk, const bf16x8* qf, int col, int half, f32x16* s) {
    using T = Tile<D, BLK>;
#pragma unroll
    for (int sub = 0; sub < T::NSUB; ++sub) {
        f32x16 acc = {};
        const int row = 32 * sub + col;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            const uint4 a = lk[row * T::KCH + ((half + 2 * kk) ^ (row % T::KCH))];
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[kk], acc, 0, 0, 0);
        }
        s[sub] = acc;
    }
}

// O^T[dsub] += V^T[32 dsub + .., :] P^T.
template <int D, int BLK>
__device__ __forceinline__ void pv_tile(const uint4* lv, const uint32_t (*pk)[8], int col, int half, f32x16* o) {
    using T = Tile<D, BLK>;
#pragma unroll
    for (int ds = 0; ds < T::NDS; ++ds) {
        const int row = 32 * ds + col;
#pragma unroll
        for (int st = 0; st < BLK / 16; ++st) {
            const uint4 a = lv[row * T::VCH + ((half + 2 * st) ^ (row % T::VCH))];
            const uint32_t* p = &pk[st >> 1][4 * (st & 1)];
            const uint4 bp = make_uint4(p[0], p[1], p[2], p[3]);
            o[ds] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                            __builtin_bit_cast(bf16x8, bp), o[ds], 0, 0, 0);
        }
    }
}

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
    mt = fmaxf(mt, __shfl_xor(mt, 32));
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

// Mean-correction pass (FlashPrefill V2 abstract): every skipped block J < I
// enters row i's softmax as one entry with logit sigma*q_i.k_bar_J + ln n_J and
// value v_bar_J.  Pooled K_bar / V_bar tiles of BLK blocks run through the
// bf16 MFMA pipeline with every kept or non-past block masked out.  qf is the
// bf16 Q fragment (B operand layout of qk_tile); c = sigma * log2(e).
template <int D, int BLK>
__device__ __forceinline__ void correction_pass(const AttnArgs& a, const SeqTable& t, int b, int I, int hk, int cnt,
                                                const int32_t* list, const bf16x8* qf, uint4* lk, uint4* lv,
                                                uint32_t* kept_bits, int tid, int col, int half, float c,
                                                float& m, float& l, f32x16* o) {
    using T = Tile<D, BLK>;
    f32x16 s[T::NSUB];
    uint32_t pk[T::NSUB][8];

    const int nwords = (I + 31) >> 5;
    for (int i = tid; i < nwords; i += T::NT) kept_bits[i] = 0u;
    __syncthreads();
    for (int i = tid; i < cnt; i += T::NT) {
        const int J = list[i];
        if (J < I) atomicOr(&kept_bits[J >> 5], 1u << (J & 31));
    }
    __syncthreads();
    const int64_t prow0 = (int64_t)hk * t.total_blocks + t.blk_off[b];
    // Every block J < I of a request is full, so ln n_J = ln BLK (log2 units here).
    const float log2_blk = __log2f((float)BLK);
    for (int c0 = 0; c0 < I; c0 += BLK) {
        // Bit j of skip[sub] <=> block c0 + 32 sub + j is strictly past (< I) and not kept.
        uint32_t skip[T::NSUB];
        int nskip = 0;
#pragma unroll
        for (int sub = 0; sub < T::NSUB; ++sub) {
            const int j0 = c0 + 32 * sub;
            const int nvalid = min(32, max(0, I - j0));
            const uint32_t valid = nvalid >= 32 ? 0xffffffffu : ((1u << nvalid) - 1u);
            skip[sub] = ~kept_bits[j0 >> 5] & valid;
            nskip += __popc(skip[sub]);
        }
        if (nskip == 0) continue;                      // every past block here is kept
        __syncthreads();
        load_pooled_tile<D, BLK>(a.pk16, a.pv16, prow0, c0, I, lk, lv, tid);
        __syncthreads();
        qk_tile<D, BLK>(lk, qf, col, half, s);
#pragma unroll
        for (int sub = 0; sub < T::NSUB; ++sub) {
            const uint32_t bits = skip[sub] >> (4 * half);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[sub][r] = ((bits >> ((r & 3) + 8 * (r >> 2))) & 1u) ? s[sub][r] : -INFINITY;
        }
        softmax_update<T::NSUB, T::NDS>(s, c, log2_blk, m, l, o, pk);
        pv_tile<D, BLK>(lv, pk, col, half, o);
    }
}

// Normalise O, stage the bf16 tile in LDS (reusing the K tile) and store full
// rows; write the natural-log sum of exp when requested.
template <int D, int BLK>
__device__ __forceinline__ void store_output(const AttnArgs& a, const SeqTable& t, int h, int q0, int nI, int qr,
                                             int half, float m, float l, const f32x16* o, uint4* lk, int tid) {
    using T = Tile<D, BLK>;
    const float l_tot = l + __shfl_xor(l, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    __syncthreads();
#pragma unroll
    for (int ds = 0; ds < T::NDS; ++ds)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int chunk = 4 * ds + g4;        // d0 = 32 ds + 8 g4 + 4 half
            uint2 v2 = make_uint2(pack_bf16(o[ds][4 * g4] * inv, o[ds][4 * g4 + 1] * inv),
                                  pack_bf16(o[ds][4 * g4 + 2] * inv, o[ds][4 * g4 + 3] * inv));
            reinterpret_cast<uint2*>(&lk[qr * T::KCH + (chunk ^ (qr % T::KCH))])[half] = v2;
        }
    __syncthreads();
    for (int i = tid; i < nI * T::KCH; i += T::NT) {
        const int row = i / T::KCH, ch = i % T::KCH;
        *reinterpret_cast<uint4*>(a.out + ((int64_t)(q0 + row) * a.Hq + h) * D + ch * 8) =
            lk[row * T::KCH + (ch ^ (row % T::KCH))];
    }
    if (a.lse && half == 0 && qr < nI)
        a.lse[(int64_t)h * t.total_tokens + q0 + qr] = (m + __log2f(l_tot)) * kLn2;
}

}  // namespace fp_attn
