// fp8 (OCP e4m3fn) sparse attention over the kept blocks (FlashPrefill V2
// abstract: FP8 inference).  One workgroup of BLK/32 waves (32 query rows
// each) per (query block, query head), at least two workgroups per CU.
// Query blocks are those of a request table: whole prompts, or the chunks of
// chunked prefill (each chunk at the end of its context, possibly starting
// inside its first query block).
//
// Inputs carry one fp32 scale per (head, block): x = code * scale.  Scores
// come from v_mfma_scale_f32_32x32x64_f8f6f4 on the raw codes and are scaled
// by sq[h,I] * sk[h_kv,J] * sigma afterwards.  P (times 2^8, so the row
// maximum 1 is exact) goes to the PV product as two e4m3 terms,
// P_hi = e4m3(p) and P_lo = e4m3(p - P_hi), both on fp8 MFMA into the same
// accumulator: one e4m3 term alone carries up to 2^-4 relative error per
// weight, the pair about 2^-8.  The row sum l is taken from the same two
// rounded terms (a product of P against a block of ones), so numerator and
// denominator weigh every key alike.  Each tile's V scale is folded into the
// per-tile rescale of the O accumulator: O holds sum P (V8) in units of the
// current tile's scale.
//
// LDS: K8 and V8 tiles are row-major [BLK][D] bytes (16-byte chunks XOR-
// swizzled per row), DMA'd into one of two buffers while the other is
// computed on.  The V^T operand is read with ds_read_b64_tr_b8, gathering per
// lane the keys in the order in which the P registers hold them, so P is the
// PV operand as it stands.
//
// The mean correction runs on the bf16 pipeline with Q dequantized to bf16:
// the bf16 pooled K_bar / V_bar rows of BLK/2 past blocks at a time arrive by
// DMA into one of two LDS buffers (the tile buffers of the kept walk) while
// the previous 64 are computed, K_bar read row-major and V_bar with the
// transposing LDS read, as in the bf16 kernel.
#include "attn_walk.h"

namespace {
using namespace fp_attn;
using namespace fp_walk;

typedef __attribute__((ext_vector_type(2))) float f32x2;

constexpr int kNeutralScale = 127;   // E8M0 code of 1.0 for the MFMA block scales

typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

__device__ __forceinline__ i32x8 cat8(const uint4& x, const uint4& y) {
    return i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
}

// S^T = K8 Q8^T for subtiles SUB0 .. SUB0+NS-1 (64 bytes of d per MFMA).  A
// operand of lane l: key row 32 sub + l%32, d bytes 32 (l/32) + 64 kk .. +31.
template <int D, int SUB0, int NS>
__device__ __forceinline__ void qk8(const uint4* kt, const i32x8* qf, int col, int half, f32x16* s) {
    constexpr int NCH = D / 16;                  // 16-byte chunks per fp8 row
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int row = 32 * (SUB0 + j) + col;
        uint4 av[2 * (D / 64)];
#pragma unroll
        for (int kk = 0; kk < D / 64; ++kk) {
            av[2 * kk] = kt[row * NCH + ((2 * half + 4 * kk) ^ swz<D / 2>(row))];
            av[2 * kk + 1] = kt[row * NCH + ((2 * half + 4 * kk + 1) ^ swz<D / 2>(row))];
        }
        __builtin_amdgcn_sched_barrier(0);       // keep the reads ahead of the MFMA chain
        f32x16 acc = {};
#pragma unroll
        for (int kk = 0; kk < D / 64; ++kk)
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cat8(av[2 * kk], av[2 * kk + 1]), qf[kk], acc, 0, 0,
                                                                  0, kNeutralScale, 0, kNeutralScale);
        s[j] = acc;
    }
}

// O^T[ds] += V^T P^T over the 64-key step ST (keys 64 ST ..).  The A operand
// of lane l (group g = l/16, i = l%16, h = l/32) holds d = 32 ds + 16 (g&1) + i
// and the 32 keys 64 ST + 4 h + 16 t + {0,1,2,3, 8,9,10,11} (t = 0..3) -- the
// order in which the P registers of subtiles 2 ST and 2 ST + 1 hold their
// keys.  ds_read_b64_tr_b8 gives output lane i of a 16-lane group byte i mod 8
// of the 8-byte reads of source lanes (i div 8) + 2m, m = 0..7; so source lane
// 2m + p reads key row m of the set at d bytes 32 ds + 16 (g&1) + 8 p.
template <int D, int ST>
__device__ __forceinline__ void pv8(const char* vt, const uint32_t (*ph)[4], const uint32_t (*pl)[4], int lane,
                                    f32x16* o, f32x16& lsum) {
    const int gl = lane & 15, g = lane >> 4;
    const int h = g >> 1, m = gl >> 1, p = gl & 1;
    const int krow = 64 * ST + 4 * h + (m & 3) + 8 * (m >> 2);
    const i32x8 bh = {(int)ph[0][0], (int)ph[0][1], (int)ph[0][2], (int)ph[0][3],
                      (int)ph[1][0], (int)ph[1][1], (int)ph[1][2], (int)ph[1][3]};
    const i32x8 bl = {(int)pl[0][0], (int)pl[0][1], (int)pl[0][2], (int)pl[0][3],
                      (int)pl[1][0], (int)pl[1][1], (int)pl[1][2], (int)pl[1][3]};
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds) {
        const int dbyte = 32 * ds + 16 * (g & 1) + 8 * p;
        i32x2 part[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int key = krow + 16 * t;
            const char* addr = vt + key * D + (((dbyte >> 4) ^ swz<D / 2>(key)) << 4) + (dbyte & 15);
            part[t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)addr);
        }
        __builtin_amdgcn_sched_barrier(0);       // keep the reads ahead of the MFMAs
        const i32x8 av = {part[0].x, part[0].y, part[1].x, part[1].y, part[2].x, part[2].y, part[3].x, part[3].y};
        o[ds] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bh, o[ds], 0, 0, 0, kNeutralScale, 0,
                                                                kNeutralScale);
        o[ds] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bl, o[ds], 0, 0, 0, kNeutralScale, 0,
                                                                kNeutralScale);
    }
    // Row sums of the two P terms as the products apply them: a V^T block of
    // e4m3 ones (0x38) gives, in every row, sum over the step's keys of
    // P_hi + P_lo for each query.
    const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                        0x38383838, 0x38383838, 0x38383838, 0x38383838};
    lsum = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, bh, lsum, 0, 0, 0, kNeutralScale, 0, kNeutralScale);
    lsum = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, bl, lsum, 0, 0, 0, kNeutralScale, 0, kNeutralScale);
}

template <int NSUB, int NDS>
__device__ __forceinline__ void softmax8_update(f32x16* s, float c, float vr, float& m, float& l, f32x16* o,
                                                uint32_t (*ph)[4], uint32_t (*pl)[4]) {
    float mt = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[sub][r]);
    mt = pair_max(mt);
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
        }
    }
}

template <int D, int BLK, int PG>
__global__ __launch_bounds__(2 * BLK, 2) void k_attn_fp8(AttnArgs a, SeqTable t) {
    constexpr bool PAGED = PG != kContig;
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
    const int nb = seq_blocks(t, b);
    const int first = first_block(t, b);               // query blocks are first .. nb-1
    const int I = nb - 1 - local;
    const int tok0 = t.tok_off[b];
    const int len = context_len(t, b, BLK);
    // Row r of the block is query row q0 + r; a chunk that starts inside its
    // first block has no rows before lo there.
    const int phase = chunk_phase(t, b, BLK);
    const int q0 = tok0 + (I - first) * BLK - phase;
    const int lo = I == first ? phase : 0;
    const int nI = min(BLK, len - I * BLK);
    const int hk = h / a.g;
    const int32_t* list = a.kv_idx + list_row(t, b, h, I, nb, first);
    const int cnt = a.kv_cnt[count_index(t, a.Hq, b, h, I, nb, first)];
    const int J0 = list[min(tid, I)];                    // for the correction's bitmap (capacity I + 1)
    const int qr = 32 * w + col;
    const uint8_t* q8 = static_cast<const uint8_t*>(a.q);
    const uint8_t* k8 = static_cast<const uint8_t*>(a.k);
    const uint8_t* v8 = static_cast<const uint8_t*>(a.v);
    const int64_t sblk = (int64_t)t.blk_off[b];
    const float sq = a.q_scale[(int64_t)h * t.total_qblocks + qblock_row(t, b, I)];
    // Rows outside lo .. nI-1 hold zero queries (their outputs are not
    // stored); their address is clamped to a row of the block.
    const bool qok = qr >= lo && qr < nI;
    const uint8_t* qrow = q8 + ((int64_t)(q0 + min(max(qr, lo), nI - 1)) * a.Hq + h) * D;

    i32x8 qf[D / 64];
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk) {
        uint4 x0 = make_uint4(0, 0, 0, 0), x1 = make_uint4(0, 0, 0, 0);
        if (qok) {
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

    // Kept tiles through two DMA buffers (lk for even steps, lv for odd):
    // K8 rows at the buffer's start, V8 rows after them.
    constexpr int NTH = 2 * BLK;
    constexpr int VOFF = BLK * D;                        // bytes of a K8 (or V8) tile
    DmaPlan<D / 2, BLK, NTH> plan;
    plan.init(tid);
    const int wave_base = __builtin_amdgcn_readfirstlane(64 * w * 16);
    const int64_t rs2 = (int64_t)a.Hkv * D / 2;          // row stride in 2-byte units
    // Contiguous: the request's rows; paged: the pools (page ids per tile).
    const int64_t kvbase = ((PAGED ? 0 : (int64_t)tok0 * a.Hkv) + hk) * D;
    const uint16_t* kfirst = reinterpret_cast<const uint16_t*>(k8 + kvbase);
    const uint16_t* vfirst = reinterpret_cast<const uint16_t*>(v8 + kvbase);
    const int32_t* pages = PAGED ? a.kv.block_table + (int64_t)b * a.kv.max_pages : nullptr;
    // Page ids of a tile: one per DMA row, one per load or one per tile, by
    // the paged form.
    constexpr int NPG = PG == kPagedRows ? DmaPlan<D / 2, BLK, NTH>::NLOAD : 1;
    auto load_pages8 = [&](int J, int* pg) {
        if (PAGED) load_pages_any<PG, D / 2, BLK, NTH>(pages, a.kv, J, len - J * BLK, lane, plan, pg);
    };
    auto issue8_pg = [&](int J, char* dst, const int* pg) {
        issue_tile_any<PG, D / 2, BLK, NTH>(kfirst, pg, a.kv, rs2, J, len - J * BLK, plan, dst, wave_base);
        issue_tile_any<PG, D / 2, BLK, NTH>(vfirst, pg, a.kv, rs2, J, len - J * BLK, plan, dst + VOFF, wave_base);
    };
    auto issue8 = [&](int J, char* dst) {
        int pg[NPG];
        load_pages8(J, pg);
        issue8_pg(J, dst, pg);
    };
    char* buf0 = reinterpret_cast<char*>(lk);
    char* buf1 = reinterpret_cast<char*>(lv);
    // The list and its blocks' K and V scales are read 64 entries at a time,
    // one per lane, and handed out with readlane.  No global load then sits
    // between a tile's DMA and its use: the vector-memory counter is in order,
    // so waiting for such a load would also wait for the DMA issued before it.
    const int64_t srow = (int64_t)hk * t.total_blocks + sblk;
    int wbase = 0, wJ = 0;
    float wsk = 0.f, wsv = 0.f;
    auto load_window = [&](int base) {
        wbase = base;
        const int i = min(base + lane, cnt - 1);
        wJ = list[i];
        if (PAGED) {
            // Paged scales: [num_pages, Hkv], the entry of the block's first page.
            const int page = pages[a.kv.page_of(wJ * BLK)];
            const bool ok = (unsigned)page < (unsigned)a.kv.num_pages;
            // A page id outside the pool reads as zero codes (the DMA's zero
            // chunk) with scale 1, i.e. as a page of zeros.
            const int64_t e = (int64_t)(ok ? page : 0) * a.Hkv + hk;
            wsk = ok ? a.k_scale[e] : 1.f;
            wsv = ok ? a.v_scale[e] : 1.f;
        } else {
            wsk = a.k_scale[srow + wJ];
            wsv = a.v_scale[srow + wJ];
        }
        __builtin_amdgcn_s_waitcnt(0);                   // settled here, not at a later use among DMAs
    };
    auto from_window = [&](int it, int& J, float& sk, float& sv) {
        J = __builtin_amdgcn_readlane(wJ, it - wbase);
        sk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wsk), it - wbase));
        sv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wsv), it - wbase));
    };
    int J = 0;
    float sk = 1.f, sv = 1.f;
    // Paged layout: the walk runs one tile further ahead -- tile it + 1's
    // block, scales and page ids (Ja, ska, sva, pga) are known a step before
    // its DMA, so a step issues the DMA right after the barrier instead of
    // first waiting on the block table.
    int Ja = 0;
    float ska = 1.f, sva = 1.f;
    int pga[NPG];
    if (cnt > 0) {
        load_window(0);
        from_window(0, J, sk, sv);
        issue8(J, buf0);
        if (PAGED && cnt > 1) {
            from_window(1, Ja, ska, sva);
            load_pages8(Ja, pga);
        }
    }
    auto step = [&](int it, char* bcur, char* bnext) {
        __builtin_amdgcn_s_waitcnt(0);                   // this thread's DMA of tile it is done
        lds_barrier();                                   // ... every thread's; the other buffer is free
        int Jn = 0;
        float skn = 1.f, svn = 1.f;
        auto prefetch = [&]() {
            if (PAGED) {
                // The window move waits on memory; nothing else is in flight yet.
                if (it + 2 < cnt && it + 2 - wbase == 64) load_window(it + 2);
                Jn = Ja;
                skn = ska;
                svn = sva;
                if (it + 1 < cnt) issue8_pg(Jn, bnext, pga);
                if (it + 2 < cnt) {
                    from_window(it + 2, Ja, ska, sva);
                    load_pages8(Ja, pga);
                }
            } else if (it + 1 < cnt) {
                if (it + 1 - wbase == 64) load_window(it + 1);
                from_window(it + 1, Jn, skn, svn);
                issue8(Jn, bnext);
            }
        };
        if (!kSerialFill) prefetch();
        qk8<D, 0, T::NSUB>(reinterpret_cast<const uint4*>(bcur), qf, col, half, s);
        if (J == I) {
#pragma unroll
            for (int sub = 0; sub < T::NSUB; ++sub)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = 32 * sub + (r & 3) + 8 * (r >> 2) + 4 * half;
                    s[sub][r] = key > qr ? -INFINITY : s[sub][r];
                }
        }
        softmax8_update<T::NSUB, T::NDS>(s, cq * sk, sv_prev / sv, m, l, o, ph, pl);
        sv_prev = sv;
        f32x16 lsum = {};
        pv8<D, 0>(bcur + VOFF, ph, pl, lane, o, lsum);
        if (BLK == 128) pv8<D, (BLK == 128 ? 1 : 0)>(bcur + VOFF, ph + 2, pl + 2, lane, o, lsum);
        if (kSerialFill) {
            lds_barrier();                               // every wave is done with tile it
            prefetch();
        }
        // Every lane of a query pair got the whole row sum; the lower half
        // keeps it (l is summed over the pair at the end).
        l += half ? 0.f : lsum[0];
        J = Jn;
        sk = skn;
        sv = svn;
    };
    for (int it = 0; it < cnt; it += 2) {
        step(it, buf0, buf1);
        if (it + 1 < cnt) step(it + 1, buf1, buf0);
    }
    lds_barrier();                                       // all reads of the last tile are done
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
        // bf16 Q fragment of the dequantized queries (the B operand of the bf16 qk product).
        bf16x8 qb[D / 16];
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            uint2 x = make_uint2(0, 0);
            if (qok) x = *reinterpret_cast<const uint2*>(qrow + 8 * half + 16 * kk);
            const f32x2 f0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)x.x, false);
            const f32x2 f1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)x.x, true);
            const f32x2 f2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)x.y, false);
            const f32x2 f3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)x.y, true);
            const uint4 pk = make_uint4(pack_bf16(f0.x * sq, f0.y * sq), pack_bf16(f1.x * sq, f1.y * sq),
                                        pack_bf16(f2.x * sq, f2.y * sq), pack_bf16(f3.x * sq, f3.y * sq));
            qb[kk] = __builtin_bit_cast(bf16x8, pk);
        }
        constexpr int HALF = (BLK / 2) * D * 2;          // bytes of BLK/2 pooled bf16 rows
        char* b0 = reinterpret_cast<char*>(lk);
        char* b1 = reinterpret_cast<char*>(lv);
        correction_dma<D, BLK>(a, t, b, I, hk, cnt, list, J0, qb, b0, b0 + HALF, b1, b1 + HALF, kept_bits, tid,
                               col, half, a.scale_log2, m, l, o);
    }
    store_output<D, BLK>(a, t, h, q0, lo, nI, qr, half, m, l, o, lk, lk + (BLK / 2) * T::KCH, tid);
}

template <int D, int BLK>
hipError_t launch_fp8_t(const AttnArgs& a, const SeqTable& t, bool paged, hipStream_t s) {
    dim3 grid((unsigned)t.total_items * a.Hq);
    const int form = paged ? paged_form<BLK, DmaPlan<D / 2, BLK, 2 * BLK>::ROWSTEP>(a.kv.page_size) : kContig;
    if (form == kPagedTiles)
        hipLaunchKernelGGL((k_attn_fp8<D, BLK, kPagedTiles>), grid, dim3(2 * BLK), 0, s, a, t);
    else if (form == kPagedSpans)
        hipLaunchKernelGGL((k_attn_fp8<D, BLK, kPagedSpans>), grid, dim3(2 * BLK), 0, s, a, t);
    else if (paged)
        hipLaunchKernelGGL((k_attn_fp8<D, BLK, kPagedRows>), grid, dim3(2 * BLK), 0, s, a, t);
    else
        hipLaunchKernelGGL((k_attn_fp8<D, BLK, kContig>), grid, dim3(2 * BLK), 0, s, a, t);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fp8(const AttnArgs& a, const SeqTable& t, int D, int B, bool paged, hipStream_t s) {
    if (t.total_items == 0) return hipSuccess;
    if (D == 128 && B == 128) return launch_fp8_t<128, 128>(a, t, paged, s);
    if (D == 128 && B == 64) return launch_fp8_t<128, 64>(a, t, paged, s);
    if (D == 64 && B == 128) return launch_fp8_t<64, 128>(a, t, paged, s);
    if (D == 64 && B == 64) return launch_fp8_t<64, 64>(a, t, paged, s);
    return hipErrorInvalidValue;
}
