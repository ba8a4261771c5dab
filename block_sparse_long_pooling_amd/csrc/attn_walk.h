// Pieces of the tile walk shared by the bf16 and fp8 attention kernels
// (gfx950): the tile DMA plan and issue, the bf16 S = K Q^T and O += V^T P^T
// products on LDS tiles, and the mean-correction pass over the pooled means
// of skipped past blocks (FlashPrefill, gist.science technical summary,
// section 2.C; FlashPrefill V2 abstract).
#pragma once
#include "fp_attn.h"

namespace fp_walk {
using namespace fp_attn;

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Source of DMA chunks for rows that hold no data (out-of-range pages): one
// zero chunk, and one zero row of the widest tile row (d = 128 bf16).
static __device__ const uint4 kZeroChunk = {0u, 0u, 0u, 0u};
static __device__ const uint4 kZeroRow[16] = {};

// XOR swizzle of 16-byte chunks within a row: conflict-free for the MFMA K
// reads (16 consecutive rows, one chunk) and for the transposing V reads
// (4 consecutive rows, 2 adjacent chunks).
template <int D>
__device__ __forceinline__ int swz(int row) {
    if (D == 128) return ((row & 7) << 1) | ((row >> 3) & 1);
    if (D == 64) return (row >> 1) & 7;
    return (row >> 2) & 3;   // D == 32: 64-byte rows of fp8 d = 64 tiles
}

// Per-thread DMA plan for a [ROWS][D] bf16 tile (ROWS keys or pooled
// blocks): load i of this thread fills LDS chunk i*NT + tid, i.e. row
// row0 + i*NT/NCH and chunk position chunk0, which holds logical chunk
// (chunk0 XOR swizzle of the row).  Two registers; the rest is recomputed
// per load.
template <int D, int ROWS, int NT>
struct DmaPlan {
    static constexpr int NCH = D / 8;
    static constexpr int NLOAD = ROWS * NCH / NT;
    static constexpr int ROWSTEP = NT / NCH;
    int row0, chunk0;
    __device__ __forceinline__ void init(int tid) {
        row0 = tid / NCH;
        chunk0 = tid % NCH;
    }
    __device__ __forceinline__ int row(int i) const { return row0 + i * ROWSTEP; }
    __device__ __forceinline__ int coff(int i) const { return (chunk0 ^ swz<D>(row(i))) * 8; }
};

// Raw buffer resource over the 4 GiB from base (stride 0, every offset in
// range; dword 3 selects the 32-bit data format that untyped buffer loads
// need on gfx9-family chips).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, -1, 0x00020000);
}

// Page ids of this thread's DMA rows of tile J (paged layout), all loaded
// before any of the tile's DMAs is issued: the vector-memory counter is in
// order, so a page id loaded between DMAs could only be waited for together
// with the DMAs before it.  Rows past the request's end (row >= nvalid) look
// up its last valid row's page, so the block-table read stays inside the
// pages that cover the request.
template <int D, int ROWS, int NT>
__device__ __forceinline__ void load_tile_pages(const int32_t* pages, const KVLayout& L, int J, int nvalid,
                                                const DmaPlan<D, ROWS, NT>& plan, int* pg) {
#pragma unroll
    for (int i = 0; i < DmaPlan<D, ROWS, NT>::NLOAD; ++i)
        pg[i] = pages[L.page_of(J * ROWS + min(plan.row(i), nvalid - 1))];
}

// DMA ROWS rows starting at `tile` (row stride rs elements; nvalid >= 1 rows
// hold data) by buffer loads into LDS from a resource whose base is the
// tile's first row, with a 32-bit per-lane offset.  (A global_load_lds is a
// FLAT instruction that the compiler counts as an LDS access too, so while one
// is in flight it waits for every outstanding LDS read instead of the one an
// MFMA needs.)
template <int D, int ROWS, int NT>
__device__ __forceinline__ void issue_rows(const char* tile, int rs, int nvalid, const DmaPlan<D, ROWS, NT>& plan,
                                           char* lds, int wave_base) {
    using P = DmaPlan<D, ROWS, NT>;
    static_assert((ROWS * P::NCH) % NT == 0, "tile chunks must split evenly");
    const __amdgpu_buffer_rsrc_t rsrc = tile_rsrc(tile);
    if (nvalid >= ROWS) {
        // Whole tile: load i's row offset is the thread's first row's plus
        // a uniform step, so no multiply per load.  The base is opaque so
        // the compiler keeps one register, not one offset per load.
        int rbase = plan.row0 * rs;
        asm volatile("" : "+v"(rbase));
#pragma unroll
        for (int i = 0; i < P::NLOAD; ++i) {
            const uint32_t off = (uint32_t)(rbase + i * P::ROWSTEP * rs + plan.coff(i)) * 2u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds + (i * NT) * 16 + wave_base), 16, off, 0,
                                                     0, 0);
        }
        return;
    }
    // Rows past the end of the sequence re-read its last row: they occur only
    // on the diagonal block, where the causal mask removes them, and finite
    // values keep 0 * v at 0.  The row index is opaque so the compiler does
    // not keep a precomputed offset per chunk and row stride (it would spill).
#pragma unroll
    for (int i = 0; i < P::NLOAD; ++i) {
        int r = plan.row(i);
        asm volatile("" : "+v"(r));
        const uint32_t off = (uint32_t)(min(r, nvalid - 1) * rs + plan.coff(i)) * 2u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds + (i * NT) * 16 + wave_base), 16, off, 0, 0,
                                                 0);
    }
}

// DMA one tile: rows J*ROWS .. J*ROWS+ROWS-1 of the request whose first row
// is `first` (contiguous), or of its pages pg from load_tile_pages (paged).
// nvalid >= 1 rows of the tile hold data.
template <int D, int ROWS, int NT, bool PAGED>
__device__ __forceinline__ void issue_tile(const uint16_t* first, const int* pg, const KVLayout& L,
                                           int64_t rs, int J, int nvalid, const DmaPlan<D, ROWS, NT>& plan,
                                           const uint4* zero, char* lds, int wave_base) {
    using P = DmaPlan<D, ROWS, NT>;
    if (!PAGED) {
        issue_rows<D, ROWS, NT>(reinterpret_cast<const char*>(first + (int64_t)J * ROWS * rs), (int)rs, nvalid, plan,
                                lds, wave_base);
    } else {
#pragma unroll
        for (int i = 0; i < P::NLOAD; ++i) {
            const int row = plan.row(i);
            const int tr = J * ROWS + row;
            const int page = pg[i];
            // Opaque column offset: keeps the compiler from holding a 64-bit
            // pointer per chunk across the loop (it would spill).
            int co = plan.coff(i);
            asm volatile("" : "+v"(co));
            const uint16_t* p = first + (((int64_t)page << L.page_shift) + L.slot_of(tr)) * rs + co;
            const void* src =
                (row < nvalid && (unsigned)page < (unsigned)L.num_pages) ? (const void*)p : (const void*)zero;
            __builtin_amdgcn_global_load_lds(src, (lds_void*)(lds + (i * NT) * 16 + wave_base), 16, 0, 0);
        }
    }
}

// K/V layout of a kernel's kept tiles: contiguous rows; pages of any size (a
// page id per tile row); pages that hold each DMA load's rows (a page id per
// load, contiguous form); pages that hold whole tiles (one page id per tile,
// contiguous form).
enum { kContig = 0, kPagedRows = 1, kPagedSpans = 2, kPagedTiles = 3 };

// Paged tiles whose loads each fall in one page: load i of every thread of
// the workgroup reads rows i*ROWSTEP .. i*ROWSTEP + ROWSTEP-1 of the tile, and
// with page_size >= ROWSTEP (both powers of two, tiles aligned) those rows are
// consecutive rows of one page.  Each load then takes the contiguous form: a
// uniform base (its page's row) and 32-bit lane offsets, by buffer loads.
// Lane i of pgv holds the page id of load i (load_span_pages, a step ahead).
template <int D, int ROWS, int NT>
__device__ __forceinline__ void load_span_pages(const int32_t* pages, const KVLayout& L, int J, int nvalid, int lane,
                                                int& pgv) {
    using P = DmaPlan<D, ROWS, NT>;
    const int i = min(lane, P::NLOAD - 1);
    // (clamped to the request's last row, so the block-table read stays
    // inside the pages that cover the request)
    pgv = pages[L.page_of(J * ROWS + min(i * P::ROWSTEP, nvalid - 1))];
}

// Rows past the request's end (nvalid >= 1 rows of the tile hold data)
// re-read its last row, which lies in the same load's page when the load
// still holds a valid row; a load wholly past the end, or whose page id is
// outside the pool, reads one zero row (stride 0).
template <int D, int ROWS, int NT>
__device__ __forceinline__ void issue_span_tile(const uint16_t* first, int pgv, const KVLayout& L, int rs, int J,
                                                int nvalid, const DmaPlan<D, ROWS, NT>& plan, const uint4* zero_row,
                                                char* lds, int wave_base) {
    using P = DmaPlan<D, ROWS, NT>;
#pragma unroll
    for (int i = 0; i < P::NLOAD; ++i) {
        const int r0 = i * P::ROWSTEP;                   // the load's first tile row
        const int page = __builtin_amdgcn_readlane(pgv, i);
        const bool ok = r0 < nvalid && (unsigned)page < (unsigned)L.num_pages;
        const uint16_t* base = first + (((int64_t)page << L.page_shift) + L.slot_of(J * ROWS + r0)) * rs;
        const char* src = ok ? reinterpret_cast<const char*>(base) : reinterpret_cast<const char*>(zero_row);
        const int stride = ok ? rs : 0;
        int r = min(plan.row0, nvalid - 1 - r0);         // row within the load's rows
        asm volatile("" : "+v"(r));
        const uint32_t off = (uint32_t)(r * stride + plan.coff(i)) * 2u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(tile_rsrc(src), (lds_void*)(lds + (i * NT) * 16 + wave_base), 16,
                                                 off, 0, 0, 0);
    }
}

// Paged tile that lies in one page (page_size >= ROWS; both are powers of two
// and tiles start at multiples of ROWS): the tile is ROWS consecutive rows of
// page `page` (uniform) from slot (J*ROWS mod page_size), so it takes the
// contiguous form with one uniform base.  Rows past the request's end re-read
// its last row, which lies in the same page.  A page id outside the pool
// reads as zeros: every row then reads one zero row (stride 0).
template <int D, int ROWS, int NT>
__device__ __forceinline__ void issue_page_tile(const uint16_t* first, int page, const KVLayout& L, int rs, int J,
                                                int nvalid, const DmaPlan<D, ROWS, NT>& plan, const uint4* zero_row,
                                                char* lds, int wave_base) {
    const bool ok = (unsigned)page < (unsigned)L.num_pages;
    const uint16_t* base = first + (((int64_t)page << L.page_shift) + L.slot_of(J * ROWS)) * rs;
    issue_rows<D, ROWS, NT>(ok ? reinterpret_cast<const char*>(base) : reinterpret_cast<const char*>(zero_row),
                            ok ? rs : 0, nvalid, plan, lds, wave_base);
}

// Page ids and DMA of one tile in any of the paged forms: pg holds NLOAD page
// ids (kPagedRows) or one value (lane i: load i's page for kPagedSpans; the
// tile's page for kPagedTiles), loaded a step ahead by load_pages_any.
template <int PG, int D, int ROWS, int NT>
__device__ __forceinline__ void load_pages_any(const int32_t* pages, const KVLayout& L, int J, int nvalid, int lane,
                                               const DmaPlan<D, ROWS, NT>& plan, int* pg) {
    if (PG == kPagedRows) load_tile_pages(pages, L, J, nvalid, plan, pg);
    if (PG == kPagedSpans) load_span_pages<D, ROWS, NT>(pages, L, J, nvalid, lane, pg[0]);
    if (PG == kPagedTiles) pg[0] = pages[L.page_of(J * ROWS)];
}

template <int PG, int D, int ROWS, int NT>
__device__ __forceinline__ void issue_tile_any(const uint16_t* first, const int* pg, const KVLayout& L, int64_t rs,
                                               int J, int nvalid, const DmaPlan<D, ROWS, NT>& plan, char* lds,
                                               int wave_base) {
    if (PG == kPagedSpans)
        issue_span_tile<D, ROWS, NT>(first, pg[0], L, (int)rs, J, nvalid, plan, kZeroRow, lds, wave_base);
    else if (PG == kPagedTiles)
        issue_page_tile<D, ROWS, NT>(first, __builtin_amdgcn_readfirstlane(pg[0]), L, (int)rs, J, nvalid, plan,
                                     kZeroRow, lds, wave_base);
    else
        issue_tile<D, ROWS, NT, PG != kContig>(first, pg, L, rs, J, nvalid, plan, &kZeroChunk, lds, wave_base);
}

// The paged form a kernel takes for tiles of ROWS rows DMA'd by plan P.
template <int ROWS, int ROWSTEP>
inline int paged_form(int page_size) {
    return page_size >= ROWS ? kPagedTiles : page_size >= ROWSTEP ? kPagedSpans : kPagedRows;
}

// S^T for subtiles SUB0 .. SUB0+NS-1 (keys 32 SUB0 ..) of this wave's 32
// queries; each subtile's 8 K operands are read before its MFMA chain.
template <int D, int SUB0, int NS>
__device__ __forceinline__ void qk(const uint4* kt, const bf16x8* qf, int col, int half, f32x16* s) {
    constexpr int NCH = D / 8;                   // 16-byte chunks per row
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int row = 32 * (SUB0 + j) + col;
        uint4 av[D / 16];
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) av[kk] = kt[row * NCH + ((half + 2 * kk) ^ swz<D>(row))];
        __builtin_amdgcn_sched_barrier(0);               // keep the reads ahead of the MFMA chain
        f32x16 acc = {};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[kk]), qf[kk], acc, 0, 0, 0);
        s[j] = acc;
    }
}

// O^T[ds] += V^T[32 ds + .., keys of subtiles SUB0 .. SUB0+NS-1] P^T.  A
// operand of key step st for lane (group gi = lane/16, gl = lane%16):
// d = 32 ds + 16 (gi&1) + gl, keys 32 (st/2) + 16 (st&1) + 4 (gi/2) + 8 r + t
// (r = 0, 1; t = 0..3) -- the same key order as the P registers.  Each
// ds_read_b64_tr_b16 reads, per source lane, 4 columns of one key row; the
// hardware transpose hands each lane its column for 4 consecutive keys.
template <int D, int SUB0, int NS>
__device__ __forceinline__ void pv(const char* vt, const uint32_t (*pk)[8], int lane, f32x16* o) {
    const int gl = lane & 15, gi = lane >> 4;
    const int hf = gi >> 1;
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds) {
        const int col_e = 32 * ds + 16 * (gi & 1) + 4 * (gl & 3);
        const int chunk = col_e >> 3, within = (col_e & 7) * 2;
        s16x4 part[2 * NS][2];
#pragma unroll
        for (int st = 0; st < 2 * NS; ++st)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int key = 32 * (SUB0 + (st >> 1)) + 16 * (st & 1) + 4 * hf + 8 * r + (gl >> 2);
                const char* addr = vt + key * (D * 2) + ((chunk ^ swz<D>(key)) << 4) + within;
                part[st][r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)addr);
            }
        __builtin_amdgcn_sched_barrier(0);               // keep the reads ahead of the MFMAs
#pragma unroll
        for (int st = 0; st < 2 * NS; ++st) {
            const uint32_t* p = &pk[st >> 1][4 * (st & 1)];
            const uint4 bp = make_uint4(p[0], p[1], p[2], p[3]);
            const s16x8 av = {part[st][0][0], part[st][0][1], part[st][0][2], part[st][0][3],
                              part[st][1][0], part[st][1][1], part[st][1][2], part[st][1][3]};
            o[ds] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                            __builtin_bit_cast(bf16x8, bp), o[ds], 0, 0, 0);
        }
    }
}

// Mean-correction pass over the skipped past blocks J < I of row block I
// (I > 0); J0 is list entry tid (any value when tid >= cnt):
// BLK/2 pooled blocks per step, double-buffered DMA: step buffers (k0, v0)
// and (k1, v1), each [BLK/2][D] bf16 (K_bar rows in k, V_bar rows in v,
// chunks swizzled per row).
template <int D, int BLK>
__device__ __forceinline__ void correction_dma(const AttnArgs& a, const SeqTable& t, int b, int I, int hk, int cnt,
                                               const int32_t* list, int J0, const bf16x8* qf, char* k0, char* v0,
                                               char* k1, char* v1, uint32_t* kept_bits, int tid, int col, int half,
                                               float c, float& m, float& l, f32x16* o) {
    constexpr int NT = 2 * BLK;                          // threads
    constexpr int HT = BLK / 2;                          // pooled blocks per step
    constexpr int NS = HT / 32;                          // 32-key subtiles per step
    const int lane = tid & 63;
    const uint16_t* kfirst = a.pk16 + ((int64_t)hk * t.total_blocks + t.blk_off[b]) * D;
    const uint16_t* vfirst = a.pv16 + ((int64_t)hk * t.total_blocks + t.blk_off[b]) * D;
    DmaPlan<D, HT, NT> plan;
    plan.init(tid);
    const int wave_base = __builtin_amdgcn_readfirstlane(64 * (tid >> 6) * 16);
    const float log2_blk = __log2f((float)BLK);          // every block J < I is full
    const int nht = (I + HT - 1) / HT;
    auto issue = [&](int hh, char* kd, char* vd) {
        const int nvalid = I - HT * hh;
        issue_tile<D, HT, NT, false>(kfirst, nullptr, a.kv, D, hh, nvalid, plan, &kZeroChunk, kd, wave_base);
        issue_tile<D, HT, NT, false>(vfirst, nullptr, a.kv, D, hh, nvalid, plan, &kZeroChunk, vd, wave_base);
    };
    // The bitmap of kept past blocks is rebuilt from the list: J0, list
    // entry tid, was loaded by the caller long before, so the marks wait on
    // no memory.  Step 0's DMA goes out right after them (an LDS access
    // while a DMA into LDS is in flight would wait for it), before the
    // barrier that publishes the bitmap.  Step 0 (blocks 0 .. HT-1) is taken
    // whether or not it holds a skipped block: a step with every block kept
    // is fully masked and leaves m, l and O as they are.
    const int nwords = (I + 31) >> 5;
    for (int i = tid; i < nwords; i += NT) kept_bits[i] = 0u;
    lds_barrier();
    if (tid < cnt && J0 < I) atomicOr(&kept_bits[J0 >> 5], 1u << (J0 & 31));
    for (int i = tid + NT; i < cnt; i += NT) {
        const int J = list[i];
        if (J < I) atomicOr(&kept_bits[J >> 5], 1u << (J & 31));
    }
    if (!kSerialFill) issue(0, k0, v0);
    lds_barrier();
    if (kSerialFill) issue(0, k0, v0);
    // Skip bits of step hh: bit j of word sub <=> block HT hh + 32 sub + j is past and not kept.
    auto skips = [&](int hh, uint32_t* sk) {
        uint32_t any = 0;
#pragma unroll
        for (int sub = 0; sub < NS; ++sub) {
            const int j0 = HT * hh + 32 * sub;
            const int nvalid = min(32, max(0, I - j0));
            const uint32_t valid = nvalid >= 32 ? 0xffffffffu : ((1u << nvalid) - 1u);
            // (a word past the bitmap can only occur with no valid block in it)
            sk[sub] = __builtin_amdgcn_readfirstlane(~kept_bits[min(j0 >> 5, FP_MAX_BLOCKS / 32 - 1)] & valid);
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
    f32x16 s[NS];
    uint32_t pk[NS][8];
    int cur = 0;
    auto step = [&](char* kc, char* vc, char* kn, char* vn) {
        __builtin_amdgcn_s_waitcnt(0);                   // this thread's DMA of step cur is done
        lds_barrier();                                   // ... every thread's; the other buffers are free
        const int nxt = next_step(cur);
        if (!kSerialFill && nxt < nht) issue(nxt, kn, vn);
        uint32_t sk[NS];
        skips(cur, sk);
        qk<D, 0, NS>(reinterpret_cast<const uint4*>(kc), qf, col, half, s);
        // Element r of a lane in half hf is block 32 sub + (r & 3) + 8 (r >> 2)
        // + 4 hf.  The skip words are uniform, so each element's keep mask is
        // built on the scalar unit as a 64-lane mask and applied with one
        // select.  A step whose blocks are all skipped past blocks (most of
        // them at low density) needs no mask at all.
        uint32_t all = 0xffffffffu;
#pragma unroll
        for (int sub = 0; sub < NS; ++sub) all &= sk[sub];
        if (all != 0xffffffffu) {
#pragma unroll
            for (int sub = 0; sub < NS; ++sub)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int k0 = (r & 3) + 8 * (r >> 2);
                    const uint64_t keep = (((sk[sub] >> k0) & 1u) ? 0xffffffffull : 0ull) |
                                          (((sk[sub] >> (k0 + 4)) & 1u) ? 0xffffffff00000000ull : 0ull);
                    s[sub][r] = __builtin_amdgcn_inverse_ballot_w64(keep) ? s[sub][r] : -INFINITY;
                }
        }
        softmax_update<NS, D / 32>(s, c, log2_blk, m, l, o, pk);
        pv<D, 0, NS>(vc, pk, lane, o);
        if (kSerialFill) {
            lds_barrier();                               // every wave is done with step cur
            if (nxt < nht) issue(nxt, kn, vn);
        }
        cur = nxt;
    };
    while (cur < nht) {
        step(k0, v0, k1, v1);
        if (cur >= nht) break;
        step(k1, v1, k0, v0);
    }
    lds_barrier();                                       // buffers free for the output staging
}

}  // namespace fp_walk
