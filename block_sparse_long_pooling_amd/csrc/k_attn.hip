// Sparse flash attention over the kept KV blocks, with the mean-correction
// term (FlashPrefill, gist.science technical summary, section 2.C: the kernel
// walks per-query-block index lists, so skipped blocks cost no work; FlashPrefill
// V2 abstract: mean correction, PackGQA-style memory access, FP8, paged KV).
//
// A workgroup owns one (query head h, query block I) of one request; each of
// its BLK/32 waves owns 32 query rows.  Per kept block J the K tile and the V
// tile go to LDS, then every wave computes
//     S^T = K Q^T        (v_mfma_f32_32x32x16_bf16; lane = query, 16 keys per
//                         32-key subtile in registers)
//     online softmax     (exp2 domain, row statistics are per-lane scalars
//                         combined with the partner lane l ^ 32)
//     O^T += V^T P^T     (P straight from registers; V^T from LDS)
// Transposed products keep the query index on the MFMA column (= lane), so
// neither P nor the softmax statistics ever cross lanes through LDS.  V^T is
// written to LDS through registers (8x8 transposes), with keys permuted inside
// each 16-key group so that the 32x32 output layout of S^T is directly the
// B operand layout of the PV product.
//
// Mean correction: after the kept blocks, the pooled K_bar / V_bar of the
// skipped blocks J < I go through the same pipeline as one more "tile" per
// BLK pooled blocks, with logit sigma*q.k_bar_J + ln n_J and every kept or
// non-past block masked out.  Query heads of one KV head are placed on one
// XCD so their K/V tiles meet in that XCD's L2.
#include "fp_attn.h"

namespace {
using namespace fp_attn;

template <int D, int BLK, bool PAGED>
__global__ __launch_bounds__(2 * BLK, 2) void k_attn_bf16(AttnArgs a, SeqTable t) {
    using T = Tile<D, BLK>;
    __shared__ uint4 lk[BLK * T::KCH];
    __shared__ uint4 lv[D * T::VCH];
    __shared__ uint32_t kept_bits[FP_MAX_BLOCKS / 32];

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
    const int rank = blockIdx.x / a.Hq;
    const int h = xcd_head(blockIdx.x % a.Hq, a.Hq);
    int b, local;
    item_of(t, rank, b, local);
    const int nb = seq_blocks(t, b);
    const int I = nb - 1 - local;
    const int tok0 = t.tok_off[b];
    const int len = t.tok_off[b + 1] - tok0;
    const int q0 = tok0 + I * BLK;
    const int nI = min(BLK, len - I * BLK);
    const int hk = h / a.g;
    const int32_t* list = a.kv_idx + t.idx_off[b] + (int64_t)h * ((int64_t)nb * (nb + 1) / 2) +
                          (int64_t)I * (I + 1) / 2;
    const int cnt = a.kv_cnt[(int64_t)a.Hq * t.blk_off[b] + (int64_t)h * nb + I];
    const int qr = 32 * w + col;
    const uint16_t* qb = static_cast<const uint16_t*>(a.q);
    const uint16_t* kb = static_cast<const uint16_t*>(a.k);
    const uint16_t* vb = static_cast<const uint16_t*>(a.v);

    bf16x8 qf[D / 16];
    {
        const uint16_t* qp = qb + ((int64_t)(q0 + qr) * a.Hq + h) * D + 8 * half;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (qr < nI) x = *reinterpret_cast<const uint4*>(qp + 16 * kk);
            qf[kk] = __builtin_bit_cast(bf16x8, x);
        }
    }
    const float c = a.scale_log2;
    float m = -INFINITY, l = 0.f;
    f32x16 o[T::NDS];
#pragma unroll
    for (int ds = 0; ds < T::NDS; ++ds) o[ds] = f32x16{};
    f32x16 s[T::NSUB];
    uint32_t pk[T::NSUB][8];

    for (int it = 0; it < cnt; ++it) {
        const int J = list[it];
        __syncthreads();
        load_kv_tile<D, BLK, PAGED>(kb, vb, a.kv, b, tok0, len, J, a.Hkv, hk, lk, lv, tid);
        __syncthreads();
        qk_tile<D, BLK>(lk, qf, col, half, s);
        if (J == I) {
#pragma unroll
            for (int sub = 0; sub < T::NSUB; ++sub)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = 32 * sub + (r & 3) + 8 * (r >> 2) + 4 * half;
                    s[sub][r] = key > qr ? -INFINITY : s[sub][r];
                }
        }
        softmax_update<T::NSUB, T::NDS>(s, c, 0.f, m, l, o, pk);
        pv_tile<D, BLK>(lv, pk, col, half, o);
    }

    if (a.correction && I > 0)
        correction_pass<D, BLK>(a, t, b, I, hk, cnt, list, qf, lk, lv, kept_bits, tid, col, half, c, m, l, o);
    store_output<D, BLK>(a, t, h, q0, nI, qr, half, m, l, o, lk, tid);
}

template <int D, int BLK>
hipError_t launch_attn_t(const AttnArgs& a, const SeqTable& t, bool paged, hipStream_t s) {
    dim3 grid((unsigned)t.total_items * a.Hq);
    if (paged)
        hipLaunchKernelGGL((k_attn_bf16<D, BLK, true>), grid, dim3(2 * BLK), 0, s, a, t);
    else
        hipLaunchKernelGGL((k_attn_bf16<D, BLK, false>), grid, dim3(2 * BLK), 0, s, a, t);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, const SeqTable& t, int D, int B, bool paged, hipStream_t s) {
    if (t.total_items == 0) return hipSuccess;
    if (D == 128 && B == 128) return launch_attn_t<128, 128>(a, t, paged, s);
    if (D == 128 && B == 64) return launch_attn_t<128, 64>(a, t, paged, s);
    if (D == 64 && B == 128) return launch_attn_t<64, 128>(a, t, paged, s);
    if (D == 64 && B == 64) return launch_attn_t<64, 64>(a, t, paged, s);
    return hipErrorInvalidValue;
}
