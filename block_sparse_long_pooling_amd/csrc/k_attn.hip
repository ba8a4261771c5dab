// Sparse flash attention over the kept KV blocks, with the mean-correction
// term, bf16 (FlashPrefill, gist.science technical summary, section 2.C: the
// kernel walks per-query-block index lists, so skipped blocks cost no work;
// FlashPrefill V2 abstract: mean correction, PackGQA-style memory access,
// paged KV).
//
// One workgroup per (query block I, query head h): BLK/32 waves of 32 query
// rows, at least two workgroups per CU.  The workgroup walks h's ascending
// list of kept blocks as tiles of KT keys (64, or 32 at d = 128 with block
// size 64; BLK/KT tiles per block).  Per tile, each wave computes
//     S^T = K Q^T        v_mfma_f32_32x32x16_bf16, lane = query, 16 keys per
//                        32-key subtile in registers
//     online softmax     exp2 domain; row statistics are per-lane scalars
//                        combined with the partner lane l ^ 32
//     O^T += V^T P^T     P straight from registers; V^T operand read from the
//                        row-major V rows with ds_read_b64_tr_b16
// A tile buffer holds the tile's KT K rows and its KT V rows in two arrays,
// row-major [KT][D] bf16 with 16-byte chunks XOR-swizzled per row (16 KiB
// each for 64 keys at d = 128).  Tiles arrive by buffer loads into LDS (DMA,
// no registers; per-row page addresses by global_load_lds only for pages
// smaller than a load's rows) into two alternating buffers: the next tile's
// DMA is issued right after the one barrier per tile and lands while the
// current tile is computed.  Rows past a request's end re-read its last row
// (a zero chunk with per-row page addresses; a page id outside the pool reads
// as zeros); the causal mask of the diagonal block removes them, and a tile
// that lies wholly past the end (a tile of the last block after its last
// token) is not visited.  On the diagonal block a wave whose rows all precede a tile's keys
// skips it.
//
// With one head per workgroup no wave idles through a tile that only another
// head keeps, and the resident workgroups of a CU hide each other's barrier
// and DMA waits.  Workgroups run longest rows first and the query heads of
// one KV head are placed on one XCD, so a tile several of them keep is read
// from HBM once into that XCD's L2.
//
// Mean correction: after the kept tiles, the bf16 pooled K_bar / V_bar rows
// of BLK/2 past blocks at a time arrive through the same two buffers, with
// logit sigma*q.k_bar_J + ln n_J, masked to the skipped J < I.
#include "attn_walk.h"

namespace {
using namespace fp_walk;

// Keys per tile: 64, or 32 at d = 128 and block size 64, where 64-key
// buffers would leave room for only two 2-wave workgroups per CU (one wave
// per SIMD); with 32-key buffers four fit, two waves per SIMD.
template <int D, int BLK>
constexpr int kTileKeys = (D == 128 && BLK == 64) ? 32 : 64;

template <int D, int BLK, int PG>
__global__ __launch_bounds__(2 * BLK, 2) void k_attn_bf16(AttnArgs a, SeqTable t) {
    constexpr bool PAGED = PG != kContig;
    constexpr int KT = kTileKeys<D, BLK>;               // keys per tile
    constexpr int NH = BLK / KT;                         // tiles per KV block
    constexpr int NT = 2 * BLK;
    constexpr int NDS = D / 32;
    constexpr int NSB = KT / 32;                         // 32-key subtiles per tile
    constexpr int TB = KT * D * 2;                       // bytes of a tile's K (or V) rows
    static_assert(TB >= BLK * D, "a K or V tile buffer also holds BLK/2 pooled rows or output rows");
    // Two tile buffers, each a K array and a V array.  Four separate arrays
    // let the compiler see that the V rows a tile's PV product reads are not
    // the ones the next tile's DMA writes; with K and V in one array it made
    // the product wait for that DMA.
    __shared__ __attribute__((aligned(16))) char kb0[TB];
    __shared__ __attribute__((aligned(16))) char vb0[TB];
    __shared__ __attribute__((aligned(16))) char kb1[TB];
    __shared__ __attribute__((aligned(16))) char vb1[TB];
    __shared__ uint32_t kept_bits[FP_MAX_BLOCKS / 32];   // correction: kept past blocks

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, col = lane & 31, half = lane >> 5;
    // Items run longest first; the query heads of one KV head share an XCD.
    const int rank = blockIdx.x / a.Hq;
    const int h = xcd_head(blockIdx.x % a.Hq, a.Hq);
    int b, local;
    item_of(t, rank, b, local);
    const int nb = seq_blocks(t, b);
    const int first = first_block(t, b);
    const int I = nb - 1 - local;
    const int tok0 = t.tok_off[b];
    const int len = context_len(t, b, BLK);
    const int phase = chunk_phase(t, b, BLK);
    const int q0 = tok0 + (I - first) * BLK - phase;     // query row of the block's row 0
    const int lo = I == first ? phase : 0;               // rows lo .. nI-1 exist
    const int nI = min(BLK, len - I * BLK);
    const int hk = h / a.g;
    const int32_t* list = a.kv_idx + list_row(t, b, h, I, nb, first);
    const int cnt = a.kv_cnt[count_index(t, a.Hq, b, h, I, nb, first)];
    const int qr = 32 * w + col;
    // The list's first window (entries lane, within its capacity I + 1) and
    // entry tid (for the correction's bitmap) load before Q: waiting for the
    // window, which names the first tile, then does not wait for the Q rows
    // as well (the vector-memory counter is in order).
    int wJ = list[min(lane, I)];
    const int J0 = list[min(tid, I)];
    // Rows outside lo .. nI-1 re-read the nearest valid row; they are never stored.
    bf16x8 qf[D / 16];
    {
        const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                             ((int64_t)(q0 + min(max(qr, lo), nI - 1)) * a.Hq + h) * D + 8 * half;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 16 * kk));
    }
    float m = -INFINITY, l = 0.f;
    f32x16 o[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) o[ds] = f32x16{};
    f32x16 s[NSB];
    uint32_t pk[NSB][8];
    const float c = a.scale_log2;

    DmaPlan<D, KT, NT> plan;
    plan.init(tid);
    constexpr int NLOAD = DmaPlan<D, KT, NT>::NLOAD;
    const int wave_base = __builtin_amdgcn_readfirstlane(64 * w * 16);
    const int64_t rs = (int64_t)a.Hkv * D;
    const int64_t base = (PAGED ? 0 : (int64_t)tok0 * rs) + (int64_t)hk * D;
    const uint16_t* kfirst = static_cast<const uint16_t*>(a.k) + base;
    const uint16_t* vfirst = static_cast<const uint16_t*>(a.v) + base;
    const int32_t* pages = PAGED ? a.kv.block_table + (int64_t)b * a.kv.max_pages : nullptr;
    // Tile code = NH J + hh: keys KT code .. KT code + KT - 1 of the request.
    // Paged layout: pg holds the page ids of the next tile to issue (one per
    // DMA row, one per load, or one per tile, by the paged form), loaded a
    // step ahead so the issue does not wait on the block table.
    int pg[PG == kPagedRows ? NLOAD : 1];
    auto load_pages = [&](int code) {
        if (PAGED) load_pages_any<PG, D, KT, NT>(pages, a.kv, code, len - code * KT, lane, plan, pg);
    };
    auto issue = [&](int code, char* kd, char* vd) {
        issue_tile_any<PG, D, KT, NT>(kfirst, pg, a.kv, rs, code, len - code * KT, plan, kd, wave_base);
        issue_tile_any<PG, D, KT, NT>(vfirst, pg, a.kv, rs, code, len - code * KT, plan, vd, wave_base);
    };
    // The list is read 64 entries at a time, one per lane, bounded by its
    // capacity I + 1 (entries past the count are never used).
    int wbase = 0;
    auto load_window = [&](int wb) {
        wbase = wb;
        wJ = list[min(wb + lane, I)];
    };
    // Tile cursor: entry ge of the list, tile gh of its block gJ.
    int ge = -1, gh = NH - 1, gJ = 0;
    auto next_code = [&]() -> int {
        if (gh + 1 < NH && len > (NH * gJ + gh + 1) * KT) {
            ++gh;
        } else {
            if (++ge >= cnt) return -1;
            if (ge - wbase == 64) load_window(ge);
            gJ = __builtin_amdgcn_readlane(wJ, ge - wbase);
            gh = 0;
        }
        return NH * gJ + gh;
    };
    int code = next_code();
    if (code >= 0) {
        load_pages(code);
        issue(code, kb0, vb0);
    }
    int coden = code >= 0 ? next_code() : -1;
    if (coden >= 0) load_pages(coden);

    auto step = [&](char* kc, char* vc, char* kn, char* vn) {
        __builtin_amdgcn_s_waitcnt(0);                   // this thread's DMA of the tile (and next page ids)
        lds_barrier();                                   // ... every thread's; the other buffer is free
        int codenn = -1;
        auto prefetch = [&]() {
            if (coden >= 0) {
                codenn = next_code();
                issue(coden, kn, vn);
                if (codenn >= 0) load_pages(codenn);
            }
        };
        if (!kSerialFill) prefetch();
        const int J = code / NH, hh = code % NH;
        if (J != I || 32 * w + 31 >= KT * hh) {
            qk<D, 0, NSB>(reinterpret_cast<const uint4*>(kc), qf, col, half, s);
            if (J == I) {
                // Causal mask of the diagonal block (opaque limit: the lane
                // masks are computed here, not hoisted and held).
                int lim = qr - 4 * half - KT * hh;
                asm volatile("" : "+v"(lim));
#pragma unroll
                for (int j = 0; j < NSB; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = 32 * j + (r & 3) + 8 * (r >> 2);
                        s[j][r] = key > lim ? -INFINITY : s[j][r];
                    }
            }
            softmax_update<NSB, NDS>(s, c, 0.f, m, l, o, pk);
            pv<D, 0, NSB>(vc, pk, lane, o);
        }
        if (kSerialFill) {
            lds_barrier();                               // every wave is done with the tile
            prefetch();
        }
        code = coden;
        coden = codenn;
    };
    while (code >= 0) {
        step(kb0, vb0, kb1, vb1);
        if (code < 0) break;
        step(kb1, vb1, kb0, vb0);
    }
    lds_barrier();                                       // the last tile is read
    if (a.correction && I > 0)
        correction_dma<D, BLK>(a, t, b, I, hk, cnt, list, J0, qf, kb0, vb0, kb1, vb1, kept_bits, tid, col, half, c,
                               m, l, o);
    store_output<D, BLK>(a, t, h, q0, lo, nI, qr, half, m, l, o, reinterpret_cast<uint4*>(kb0),
                         reinterpret_cast<uint4*>(vb0), tid);
}

template <int D, int BLK>
hipError_t launch_db(const AttnArgs& a, const SeqTable& t, bool paged, hipStream_t s) {
    const dim3 grid((unsigned)(t.total_items * a.Hq));
    constexpr int KT = kTileKeys<D, BLK>;
    const int form = paged ? paged_form<KT, DmaPlan<D, KT, 2 * BLK>::ROWSTEP>(a.kv.page_size) : kContig;
    if (form == kPagedTiles)
        hipLaunchKernelGGL((k_attn_bf16<D, BLK, kPagedTiles>), grid, dim3(2 * BLK), 0, s, a, t);
    else if (form == kPagedSpans)
        hipLaunchKernelGGL((k_attn_bf16<D, BLK, kPagedSpans>), grid, dim3(2 * BLK), 0, s, a, t);
    else if (form == kPagedRows)
        hipLaunchKernelGGL((k_attn_bf16<D, BLK, kPagedRows>), grid, dim3(2 * BLK), 0, s, a, t);
    else
        hipLaunchKernelGGL((k_attn_bf16<D, BLK, kContig>), grid, dim3(2 * BLK), 0, s, a, t);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, const SeqTable& t, int D, int B, bool paged, hipStream_t s) {
    if (t.total_items == 0) return hipSuccess;
    if (D == 128 && B == 128) return launch_db<128, 128>(a, t, paged, s);
    if (D == 128 && B == 64) return launch_db<128, 64>(a, t, paged, s);
    if (D == 64 && B == 128) return launch_db<64, 128>(a, t, paged, s);
    if (D == 64 && B == 64) return launch_db<64, 64>(a, t, paged, s);
    return hipErrorInvalidValue;
}
