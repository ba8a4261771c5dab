// fp8 (OCP e4m3fn) sparse attention over the kept blocks (FlashPrefill V2
// abstract: FP8 inference), same work decomposition as the bf16 kernel.
//
// Inputs carry one fp32 scale per (head, block): x = code * scale.  Scores
// come from v_mfma_scale_f32_32x32x64_f8f6f4 on the raw codes and are scaled
// by sq[h,I] * sk[h_kv,J] * sigma afterwards.  P (times 2^8, so the row
// maximum 1 is exact) goes to the PV product as two e4m3 terms,
// P_hi = e4m3(p) and P_lo = e4m3(p - P_hi), both on fp8 MFMA into the same
// accumulator: one e4m3 term alone carries up to 2^-4 relative error per
// weight, the pair about 2^-8.  Each tile's V scale is folded into the
// per-tile rescale of the O accumulator: O holds sum P (V8) in units of the
// current tile's scale.
//
// LDS: the K8 tile is [BLK][D] bytes; the V8 tile is stored transposed,
// [D][BLK] bytes, with keys permuted inside each 64-key step so that the
// 32x32 output layout of S^T is directly the byte layout of the PV B operand
// (position p holds key  32*p[4] + 8*p[3:2] + 4*p[5] + p[1:0]).
//
// The mean correction runs on the bf16 pipeline with Q dequantized to bf16:
// the bf16 pooled K_bar / V_bar rows of 64 past blocks at a time arrive by
// DMA into one of two LDS buffers (the tile buffers of the kept walk) while
// the previous 64 are computed, K_bar read row-major and V_bar with the
// transposing LDS read, as in the bf16 kernel.
#include "attn_walk.h"

namespace {
using namespace fp_attn;
using namespace fp_walk;

typedef __attribute__((ext_vector_type(2))) float f32x2;

constexpr int kNeutralScale = 127;   // E8M0 code of 1.0 for the MFMA block scales

__device__ __forceinline__ int key_perm8(int p) {
    const int q = p & 63;
    return (p & ~63) | (((q >> 4) & 1) << 5) | (((q >> 2) & 3) << 3) | (((q >> 5) & 1) << 2) | (q & 3);
}

// 4x4 byte transpose: a[u] byte j -> c[j] byte u.
__device__ __forceinline__ void transpose4b(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, uint32_t* c) {
    const uint32_t t0 = __builtin_amdgcn_perm(a1, a0, 0x05010400u);
    const uint32_t t1 = __builtin_amdgcn_perm(a1, a0, 0x07030602u);
    const uint32_t t2 = __builtin_amdgcn_perm(a3, a2, 0x05010400u);
    const uint32_t t3 = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
    c[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
    c[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
    c[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
    c[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

template <int D, int BLK>
struct Tile8 {
    static constexpr int KCH = D / 16;    // 16-byte chunks per K8 row
    static constexpr int VCH = BLK / 16;  // 16-byte chunks per V8^T row
    static constexpr int NT = 2 * BLK;
};

template <int D, int BLK>
__device__ __forceinline__ void load_kv8_tile(const uint8_t* k8, const uint8_t* v8, int tok0, int len, int J, int Hkv,
                                              int hk, uint4* lk, uint2* lv2, int tid) {
    using T = Tile8<D, BLK>;
    const int64_t rs = (int64_t)Hkv * D;
    for (int i = tid; i < BLK * T::KCH; i += T::NT) {
        const int row = i / T::KCH, ch = i % T::KCH;
        const int tr = J * BLK + row;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (tr < len) val = *reinterpret_cast<const uint4*>(k8 + (tok0 + tr) * rs + (int64_t)hk * D + ch * 16);
        lk[row * T::KCH + (ch ^ (row % T::KCH))] = val;
    }
    // (position group of 8, d group of 8) per thread: 8x8 byte transpose.
    for (int i = tid; i < (BLK / 8) * (D / 8); i += T::NT) {
        const int pg = i / (D / 8), dc = i % (D / 8);
        uint2 x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int tr = J * BLK + key_perm8(8 * pg + u);
            x[u] = make_uint2(0, 0);
            if (tr < len) x[u] = *reinterpret_cast<const uint2*>(v8 + (tok0 + tr) * rs + (int64_t)hk * D + dc * 8);
        }
        uint32_t c0[4], c1[4], c2[4], c3[4];
        transpose4b(x[0].x, x[1].x, x[2].x, x[3].x, c0);   // keys 0-3, d 0-3
        transpose4b(x[0].y, x[1].y, x[2].y, x[3].y, c1);   // keys 0-3, d 4-7
        transpose4b(x[4].x, x[5].x, x[6].x, x[7].x, c2);   // keys 4-7, d 0-3
        transpose4b(x[4].y, x[5].y, x[6].y, x[7].y, c3);   // keys 4-7, d 4-7
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int d = 8 * dc + j;
            const uint2 y = j < 4 ? make_uint2(c0[j], c2[j]) : make_uint2(c1[j - 4], c3[j - 4]);
            lv2[2 * (d * T::VCH + ((pg >> 1) ^ (d % T::VCH))) + (pg & 1)] = y;
        }
    }
}

template <int D, int BLK>
__device__ __forceinline__ i32x8 lds_pair(const uint4* base, int row, int nch, int ch) {
    const uint4 a = base[row * nch + (ch ^ (row % nch))];
    const uint4 b = base[row * nch + ((ch + 1) ^ (row % nch))];
    i32x8 r = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    return r;
}

template <int D, int BLK, int NSUB>
__device__ __forceinline__ void qk8_tile(const uint4* lk, const i32x8* qf, int col, int half, f32x16* s) {
    using T = Tile8<D, BLK>;
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
        f32x16 acc = {};
#pragma unroll
        for (int kk = 0; kk < D / 64; ++kk) {
            const i32x8 a = lds_pair<D, BLK>(lk, 32 * sub + col, T::KCH, 2 * half + 4 * kk);
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[kk], acc, 0, 0, 0, kNeutralScale, 0,
                                                                  kNeutralScale);
        }
        s[sub] = acc;
    }
}

template <int D, int BLK, int NDS>
__device__ __forceinline__ void pv8_tile(const uint4* lv, const uint32_t (*ph)[4], const uint32_t (*pl)[4], int col,
                                         int half, f32x16* o) {
    using T = Tile8<D, BLK>;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
#pragma unroll
        for (int st = 0; st < BLK / 64; ++st) {
            const i32x8 a = lds_pair<D, BLK>(lv, 32 * ds + col, T::VCH, 4 * st + 2 * half);
            const uint32_t* h0 = ph[2 * st];
            const uint32_t* h1 = ph[2 * st + 1];
            const uint32_t* l0 = pl[2 * st];
            const uint32_t* l1 = pl[2 * st + 1];
            const i32x8 bh = {(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3],
                              (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
            const i32x8 bl = {(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3],
                              (int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3]};
            o[ds] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bh, o[ds], 0, 0, 0, kNeutralScale, 0,
                                                                    kNeutralScale);
            o[ds] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bl, o[ds], 0, 0, 0, kNeutralScale, 0,
                                                                    kNeutralScale);
        }
    }
}

// Exact online softmax for fp8 tiles.  c = logit scale of this tile (log2
// units); vr = previous V scale / this tile's V scale.  With e = 2^8 p:
// ph = e4m3(e), pl = e4m3(e - ph); the row sum takes e itself.
template <int NSUB, int NDS>
__device__ __forceinline__ void softmax8_update(f32x16* s, float c, float vr, float& m, float& l, f32x16* o,
                                                uint32_t (*ph)[4], uint32_t (*pl)[4]) {
    float mt = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[sub][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mt2 = (mt == -INFINITY) ? -INFINITY : mt * c;
    const float m_new = fmaxf(m, mt2);
    const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    l *= alpha;
    const float ov = alpha * vr;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[ds][r] *= ov;
    const float off = 8.f - (m == -INFINITY ? 0.f : m);
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float e0 = __builtin_amdgcn_exp2f(fmaf(s[sub][4 * i], c, off));
            const float e1 = __builtin_amdgcn_exp2f(fmaf(s[sub][4 * i + 1], c, off));
            const float e2 = __builtin_amdgcn_exp2f(fmaf(s[sub][4 * i + 2], c, off));
            const float e3 = __builtin_amdgcn_exp2f(fmaf(s[sub][4 * i + 3], c, off));
            int w = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
            w = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, w, true);
            ph[sub][i] = (uint32_t)w;
            const f32x2 d0 = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
            const f32x2 d1 = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
            int r = __builtin_amdgcn_cvt_pk_fp8_f32(e0 - d0.x, e1 - d0.y, 0, false);
            r = __builtin_amdgcn_cvt_pk_fp8_f32(e2 - d1.x, e3 - d1.y, r, true);
            pl[sub][i] = (uint32_t)r;
            l += (e0 + e1) + (e2 + e3);
        }
    }
}

// Mean-correction pass over the skipped past blocks J < I of row block I:
// BLK/2 pooled blocks per step, double-buffered DMA into buf0 / buf1 (each a
// [BLK][D] bf16 tile buffer: BLK/2 K_bar rows, then BLK/2 V_bar rows, chunks
// swizzled per row).
template <int D, int BLK>
__device__ __forceinline__ void correction_dma(const AttnArgs& a, const SeqTable& t, int b, int I, int hk, int cnt,
                                               const int32_t* list, const bf16x8* qf, char* buf0, char* buf1,
                                               uint32_t* kept_bits, int tid, int col, int half, float c, float& m,
                                               float& l, f32x16* o) {
    constexpr int NT = 2 * BLK;                          // threads
    constexpr int HT = BLK / 2;                          // pooled blocks per step
    constexpr int NS = HT / 32;                          // 32-key subtiles per step
    constexpr int HALF = HT * D * 2;                     // bytes of K_bar (or V_bar) rows per step
    const int lane = tid & 63;
    const int nwords = (I + 31) >> 5;
    for (int i = tid; i < nwords; i += NT) kept_bits[i] = 0u;
    __syncthreads();
    for (int i = tid; i < cnt; i += NT) {
        const int J = list[i];
        if (J < I) atomicOr(&kept_bits[J >> 5], 1u << (J & 31));
    }
    __syncthreads();
    const uint16_t* kfirst = a.pk16 + ((int64_t)hk * t.total_blocks + t.blk_off[b]) * D;
    const uint16_t* vfirst = a.pv16 + ((int64_t)hk * t.total_blocks + t.blk_off[b]) * D;
    DmaPlan<D, HT, NT> plan;
    plan.init(tid);
    const int wave_base = __builtin_amdgcn_readfirstlane(64 * (tid >> 6) * 16);
    const float log2_blk = __log2f((float)BLK);          // every block J < I is full
    const int nht = (I + HT - 1) / HT;
    // Skip bits of step hh: bit j of word sub <=> block HT hh + 32 sub + j is past and not kept.
    auto skips = [&](int hh, uint32_t* sk) {
        uint32_t any = 0;
#pragma unroll
        for (int sub = 0; sub < NS; ++sub) {
            const int j0 = HT * hh + 32 * sub;
            const int nvalid = min(32, max(0, I - j0));
            const uint32_t valid = nvalid >= 32 ? 0xffffffffu : ((1u << nvalid) - 1u);
            sk[sub] = __builtin_amdgcn_readfirstlane(~kept_bits[j0 >> 5] & valid);
            any |= sk[sub];
        }
        return any != 0;
    };
    auto next_step = [&](int hh) {
        uint32_t sk[NS];
        for (++hh; hh < nht; ++hh)
            if (skips(hh, sk)) return hh;
        return nht;
    };
    auto issue = [&](int hh, char* dst) {
        const int nvalid = I - HT * hh;
        issue_tile<D, HT, NT, false>(kfirst, nullptr, a.kv, D, hh, nvalid, plan, &kZeroChunk, dst, wave_base);
        issue_tile<D, HT, NT, false>(vfirst, nullptr, a.kv, D, hh, nvalid, plan, &kZeroChunk, dst + HALF, wave_base);
    };
    f32x16 s[NS];
    uint32_t pk[NS][8];
    int cur = next_step(-1);
    if (cur < nht) issue(cur, buf0);
    auto step = [&](char* bcur, char* bnext) {
        __builtin_amdgcn_s_waitcnt(0);                   // this thread's DMA of step cur is done
        lds_barrier();                                   // ... every thread's; the other buffer is free
        const int nxt = next_step(cur);
        if (nxt < nht) issue(nxt, bnext);
        uint32_t sk[NS];
        skips(cur, sk);
        qk<D, BLK, 1, 0, NS>(reinterpret_cast<const uint4*>(bcur), qf, col, half, s);
#pragma unroll
        for (int sub = 0; sub < NS; ++sub) {
            const uint32_t bits = sk[sub] >> (4 * half);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[sub][r] = ((bits >> ((r & 3) + 8 * (r >> 2))) & 1u) ? s[sub][r] : -INFINITY;
        }
        softmax_update<NS, D / 32>(s, c, log2_blk, m, l, o, pk);
        pv<D, BLK, 1, 0, NS>(bcur + HALF, pk, lane, o);
        cur = nxt;
    };
    while (cur < nht) {
        step(buf0, buf1);
        if (cur >= nht) break;
        step(buf1, buf0);
    }
    lds_barrier();                                       // buffers free for the output staging
}

template <int D, int BLK>
__global__ __launch_bounds__(2 * BLK, 2) void k_attn_fp8(AttnArgs a, SeqTable t) {
    using T = Tile<D, BLK>;          // bf16 geometry: LDS sized for the correction tiles
    __shared__ uint4 lk[BLK * T::KCH];
    __shared__ uint4 lv[D * T::VCH];
    __shared__ uint32_t kept_bits[FP_MAX_BLOCKS / 32];

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
    const int rank = blockIdx.x / a.Hq;
    const int h = xcd_head(blockIdx.x % a.Hq, a.Hq);
    int b, local;
    item_of(t, rank, b, local);
    const int nb = seq_blocks(t, b);                   // whole sequences only: no prefix blocks
    const int I = nb - 1 - local;
    const int tok0 = t.tok_off[b];
    const int len = context_len(t, b, BLK);
    const int q0 = tok0 + I * BLK;
    const int nI = min(BLK, len - I * BLK);
    const int hk = h / a.g;
    const int32_t* list = a.kv_idx + list_row(t, b, h, I, nb, 0);
    const int cnt = a.kv_cnt[count_index(t, a.Hq, b, h, I, nb, 0)];
    const int qr = 32 * w + col;
    const uint8_t* q8 = static_cast<const uint8_t*>(a.q);
    const uint8_t* k8 = static_cast<const uint8_t*>(a.k);
    const uint8_t* v8 = static_cast<const uint8_t*>(a.v);
    const int64_t sblk = (int64_t)t.blk_off[b];
    const float sq = a.q_scale[(int64_t)h * t.total_blocks + sblk + I];
    const uint8_t* qrow = q8 + ((int64_t)(q0 + qr) * a.Hq + h) * D;

    i32x8 qf[D / 64];
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk) {
        uint4 x0 = make_uint4(0, 0, 0, 0), x1 = make_uint4(0, 0, 0, 0);
        if (qr < nI) {
            x0 = *reinterpret_cast<const uint4*>(qrow + 32 * half + 64 * kk);
            x1 = *reinterpret_cast<const uint4*>(qrow + 32 * half + 64 * kk + 16);
        }
        qf[kk] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    }
    float m = -INFINITY, l = 0.f;
    f32x16 o[T::NDS];
#pragma unroll
    for (int ds = 0; ds < T::NDS; ++ds) o[ds] = f32x16{};
    f32x16 s[T::NSUB];
    uint32_t ph[T::NSUB][4], pl[T::NSUB][4];
    float sv_prev = 1.f;
    const float cq = sq * a.scale_log2;

    for (int it = 0; it < cnt; ++it) {
        const int J = list[it];
        __syncthreads();
        load_kv8_tile<D, BLK>(k8, v8, tok0, len, J, a.Hkv, hk, lk, reinterpret_cast<uint2*>(lv), tid);
        __syncthreads();
        qk8_tile<D, BLK, T::NSUB>(lk, qf, col, half, s);
        if (J == I) {
#pragma unroll
            for (int sub = 0; sub < T::NSUB; ++sub)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = 32 * sub + (r & 3) + 8 * (r >> 2) + 4 * half;
                    s[sub][r] = key > qr ? -INFINITY : s[sub][r];
                }
        }
        const float sk = a.k_scale[(int64_t)hk * t.total_blocks + sblk + J];
        const float sv = a.v_scale[(int64_t)hk * t.total_blocks + sblk + J];
        softmax8_update<T::NSUB, T::NDS>(s, cq * sk, sv_prev / sv, m, l, o, ph, pl);
        sv_prev = sv;
        pv8_tile<D, BLK, T::NDS>(lv, ph, pl, col, half, o);
    }
    // Back to plain units: O * sv / 2^8, l / 2^8.
    {
        const float f = sv_prev * (1.f / 256.f);
#pragma unroll
        for (int ds = 0; ds < T::NDS; ++ds)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[ds][r] *= f;
        l *= (1.f / 256.f);
    }
    if (a.correction && I > 0) {
        // bf16 Q fragment of the dequantized queries (B operand layout of qk_tile).
        bf16x8 qb[D / 16];
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            uint2 x = make_uint2(0, 0);
            if (qr < nI) x = *reinterpret_cast<const uint2*>(qrow + 8 * half + 16 * kk);
            const f32x2 f0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)x.x, false);
            const f32x2 f1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)x.x, true);
            const f32x2 f2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)x.y, false);
            const f32x2 f3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)x.y, true);
            const uint4 pk = make_uint4(pack_bf16(f0.x * sq, f0.y * sq), pack_bf16(f1.x * sq, f1.y * sq),
                                        pack_bf16(f2.x * sq, f2.y * sq), pack_bf16(f3.x * sq, f3.y * sq));
            qb[kk] = __builtin_bit_cast(bf16x8, pk);
        }
        correction_dma<D, BLK>(a, t, b, I, hk, cnt, list, qb, reinterpret_cast<char*>(lk),
                               reinterpret_cast<char*>(lv), kept_bits, tid, col, half, a.scale_log2, m, l, o);
    }
    store_output<D, BLK>(a, t, h, q0, nI, qr, half, m, l, o, lk, tid);
}

template <int D, int BLK>
hipError_t launch_fp8_t(const AttnArgs& a, const SeqTable& t, hipStream_t s) {
    dim3 grid((unsigned)t.total_items * a.Hq);
    hipLaunchKernelGGL((k_attn_fp8<D, BLK>), grid, dim3(2 * BLK), 0, s, a, t);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fp8(const AttnArgs& a, const SeqTable& t, int D, int B, hipStream_t s) {
    if (t.total_items == 0) return hipSuccess;
    if (D == 128 && B == 128) return launch_fp8_t<128, 128>(a, t, s);
    if (D == 128 && B == 64) return launch_fp8_t<128, 64>(a, t, s);
    if (D == 64 && B == 128) return launch_fp8_t<64, 128>(a, t, s);
    if (D == 64 && B == 64) return launch_fp8_t<64, 64>(a, t, s);
    return hipErrorInvalidValue;
}
