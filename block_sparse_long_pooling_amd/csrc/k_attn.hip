// Sparse flash attention over the kept KV blocks, with the mean-correction
// term, bf16 (FlashPrefill, gist.science technical summary, section 2.C: the
// kernel walks per-query-block index lists, so skipped blocks cost no work;
// FlashPrefill V2 abstract: mean correction, PackGQA-style memory access,
// paged KV).
//
// Work item: (query block I, HP query heads that share one KV head).  Each
// head's BLK query rows belong to BLK/32 waves, so a workgroup is HP*BLK/32
// waves.  The workgroup walks the union of the HP heads' ascending lists; a
// K/V tile is fetched once and serves every head whose list holds it (the
// others' waves skip it).  Per tile, each active wave computes
//     S^T = K Q^T        v_mfma_f32_32x32x16_bf16, lane = query, 16 keys per
//                        32-key subtile in registers
//     online softmax     exp2 domain; row statistics are per-lane scalars
//                        combined with the partner lane l ^ 32
//     O^T += V^T P^T     P straight from registers; V^T operand read from the
//                        row-major V tile with ds_read_b64_tr_b16
// K and V tiles are row-major [BLK][D] bf16 in LDS, 16-byte chunks XOR-
// swizzled per row.  They are fetched by global_load_lds_dwordx4 (DMA into
// LDS, no registers) into two buffers: the next tile is issued right after
// the one barrier per tile and lands while the current tile is computed.
// Rows past a request's end (and out-of-range pages) read a zero chunk.
//
// Mean correction: after the kept tiles, the pooled K_bar / V_bar rows of
// blocks c0 .. c0+BLK-1 (fp32 -> bf16) form one more tile per BLK blocks,
// with logit sigma*q.k_bar_J + ln n_J, masked per head to its skipped J < I.
// Query heads of one KV head are placed on one XCD so their tiles meet in
// that XCD's L2.
#include <atomic>
#include <type_traits>

#include "fp_attn.h"

namespace {
using namespace fp_attn;

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ const uint4 kZeroChunk = {0u, 0u, 0u, 0u};

// XOR swizzle of 16-byte chunks within a row: conflict-free for the MFMA K
// reads (16 consecutive rows, one chunk) and for the transposing V reads
// (4 consecutive rows, 2 adjacent chunks).
template <int D>
__device__ __forceinline__ int swz(int row) {
    if (D == 128) return ((row & 7) << 1) | ((row >> 3) & 1);
    return (row >> 1) & 7;
}

template <int D, int BLK, int HP>
struct Geo {
    static constexpr int WPH = BLK / 32;          // waves per head
    static constexpr int NW = WPH * HP;           // waves per workgroup
    static constexpr int NT = 64 * NW;            // threads
    static constexpr int NCH = D / 8;             // 16-byte chunks per row
    static constexpr int TILE = BLK * D * 2;      // bytes per K or V tile
    static constexpr int NSUB = BLK / 32;
    static constexpr int NDS = D / 32;
};

// Per-thread DMA plan for a [BLK][D] bf16 tile: load i of this thread fills
// LDS chunk i*NT + tid, i.e. row row0 + i*NT/NCH and chunk position chunk0,
// which holds logical chunk (chunk0 XOR swizzle of the row).  Two registers;
// the rest is recomputed per load.
template <int D, int BLK, int HP>
struct DmaPlan {
    static constexpr int NT = 64 * HP * (BLK / 32);
    static constexpr int NCH = D / 8;
    static constexpr int NLOAD = BLK * NCH / NT;
    static constexpr int ROWSTEP = NT / NCH;
    int row0, chunk0;
    __device__ __forceinline__ void init(int tid) {
        row0 = tid / NCH;
        chunk0 = tid % NCH;
    }
    __device__ __forceinline__ int row(int i) const { return row0 + i * ROWSTEP; }
    __device__ __forceinline__ int coff(int i) const { return (chunk0 ^ swz<D>(row(i))) * 8; }
};

// DMA one tile: rows J*BLK .. of the request whose first row is `first`
// (contiguous) or whose pages are listed in `pages` (paged).
template <int D, int BLK, int HP, bool PAGED>
__device__ __forceinline__ void issue_tile(const uint16_t* first, const int32_t* pages, const KVLayout& L,
                                           int64_t rs, int J, int nvalid, const DmaPlan<D, BLK, HP>& plan,
                                           const uint4* zero, char* lds, int wave_base) {
    using G = Geo<D, BLK, HP>;
    using P = DmaPlan<D, BLK, HP>;
    static_assert((BLK * G::NCH) % G::NT == 0, "tile chunks must split evenly");
    if (!PAGED) {
        // Uniform tile base plus a 32-bit per-lane offset (the scalar-base
        // addressing form).
        const char* tile = reinterpret_cast<const char*>(first + (int64_t)J * BLK * rs);
        // Rows past the end of the sequence re-read its last row: they occur
        // only in the diagonal tile, where the causal mask removes them, and
        // finite values keep 0 * v at 0.  The row index is opaque so the
        // compiler does not keep a precomputed offset per chunk and row stride
        // (it would spill).
#pragma unroll
        for (int i = 0; i < P::NLOAD; ++i) {
            int r = plan.row(i);
            asm volatile("" : "+v"(r));
            const uint32_t off = (uint32_t)(min(r, nvalid - 1) * (int)rs + plan.coff(i)) * 2u;
            __builtin_amdgcn_global_load_lds(tile + off, (lds_void*)(lds + (i * G::NT) * 16 + wave_base), 16, 0, 0);
        }
    } else {
#pragma unroll
        for (int i = 0; i < P::NLOAD; ++i) {
            const int row = plan.row(i);
            const int tr = J * BLK + row;
            const int page = pages[tr / L.page_size];
            // Opaque column offset: keeps the compiler from holding a 64-bit
            // pointer per chunk across the loop (it would spill).
            int co = plan.coff(i);
            asm volatile("" : "+v"(co));
            const uint16_t* p = first + ((int64_t)page * L.page_size + tr % L.page_size) * rs + co;
            const void* src =
                (row < nvalid && (unsigned)page < (unsigned)L.num_pages) ? (const void*)p : (const void*)zero;
            __builtin_amdgcn_global_load_lds(src, (lds_void*)(lds + (i * G::NT) * 16 + wave_base), 16, 0, 0);
        }
    }
}

// S^T for subtiles SUB0 .. SUB0+NS-1 (keys 32 SUB0 ..) of this wave's 32
// queries; each subtile's 8 K operands are read before its MFMA chain.
template <int D, int BLK, int HP, int SUB0, int NS>
__device__ __forceinline__ void qk(const uint4* kt, const bf16x8* qf, int col, int half, f32x16* s) {
    using G = Geo<D, BLK, HP>;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int row = 32 * (SUB0 + j) + col;
        uint4 av[D / 16];
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) av[kk] = kt[row * G::NCH + ((half + 2 * kk) ^ swz<D>(row))];
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
template <int D, int BLK, int HP, int SUB0, int NS>
__device__ __forceinline__ void pv(const char* vt, const uint32_t (*pk)[8], int lane, f32x16* o) {
    using G = Geo<D, BLK, HP>;
    const int gl = lane & 15, gi = lane >> 4;
    const int hf = gi >> 1;
#pragma unroll
    for (int ds = 0; ds < G::NDS; ++ds) {
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

// Ascending-merge cursor over the lists of the HP heads of a workgroup.
template <int HP>
struct Union {
    const int32_t* list[HP];
    int cnt[HP];
    int cap;         // capacity of each list (I + 1): windows never read past it
    int pos[HP];     // entries of list h consumed so far
    int wbase[HP];   // list index held by lane 0 of win[h]
    int win[HP];     // lane l: list[h][wbase[h] + l] (INT_MAX past the end)
    // Lists are read 64 entries at a time, one per lane, so the walk waits
    // on memory once per 64 kept blocks instead of once per block.  A window
    // is bounded by the list's capacity, not its count, so it need not wait
    // for the count; entries past the count are never used.
    __device__ __forceinline__ void load_window(int h) {
        wbase[h] = pos[h];
        const int i = pos[h] + (int)__lane_id();
        win[h] = i < cap ? list[h][i] : INT_MAX;
    }
    __device__ __forceinline__ void init() {
#pragma unroll
        for (int h = 0; h < HP; ++h) {
            pos[h] = 0;
            load_window(h);
        }
    }
    __device__ __forceinline__ int val(int h) const {
        return pos[h] < cnt[h] ? __builtin_amdgcn_readlane(win[h], pos[h] - wbase[h]) : INT_MAX;
    }
    // Next block of the union and the heads that keep it (bit mask); INT_MAX when done.
    __device__ __forceinline__ int next(int& act) {
        int v[HP];
        int J = INT_MAX;
#pragma unroll
        for (int h = 0; h < HP; ++h) {
            v[h] = val(h);
            J = min(J, v[h]);
        }
        act = 0;
#pragma unroll
        for (int h = 0; h < HP; ++h)
            if (J != INT_MAX && v[h] == J) {
                act |= 1 << h;
                if (++pos[h] - wbase[h] == 64) load_window(h);
            }
        return J;
    }
};

// One work item: query block I of one request, HP heads of one KV head.
template <int D, int BLK, int HP, bool PAGED>
struct Item {
    int b, nb, I, tok0, len, q0, nI, hk, h;      // h: this wave's query head
    int nct;                                      // correction tiles (blocks 0 .. I-1 in tiles of BLK)
    int ct;                                       // next correction tile to examine; -1 while kept blocks remain
    Union<HP> u;
    const uint16_t* kfirst;                       // K rows of this request / KV head (or the pool)
    const uint16_t* vfirst;
    const int32_t* pages;                         // block-table row (paged)

    __device__ __forceinline__ void setup(const AttnArgs& a, const SeqTable& t, int idx, int hs) {
        const int npairs = a.Hq / HP;
        const int rank = idx / npairs;
        h = HP * xcd_head(idx % npairs, npairs) + hs;
        int local;
        item_of(t, rank, b, local);
        nb = seq_blocks(t, b);
        I = nb - 1 - local;
        tok0 = t.tok_off[b];
        len = t.tok_off[b + 1] - tok0;
        q0 = tok0 + I * BLK;
        nI = min(BLK, len - I * BLK);
        hk = h / a.g;
        const int64_t rs = (int64_t)a.Hkv * D;
        const int64_t tri = (int64_t)nb * (nb + 1) / 2;
        const int h0 = h - hs;
#pragma unroll
        for (int j = 0; j < HP; ++j) {
            u.list[j] = a.kv_idx + t.idx_off[b] + (int64_t)(h0 + j) * tri + (int64_t)I * (I + 1) / 2;
            u.cnt[j] = a.kv_cnt[(int64_t)a.Hq * t.blk_off[b] + (int64_t)(h0 + j) * nb + I];
        }
        u.cap = I + 1;
        u.init();
        nct = (a.correction && I > 0) ? (I + BLK - 1) / BLK : 0;
        ct = -1;
        const int64_t base = (PAGED ? 0 : (int64_t)tok0 * rs) + (int64_t)hk * D;
        kfirst = static_cast<const uint16_t*>(a.k) + base;
        vfirst = static_cast<const uint16_t*>(a.v) + base;
        pages = PAGED ? a.kv.block_table + (int64_t)b * a.kv.max_pages : nullptr;
    }
};

// Tiles of a work item are coded as ints: a kept KV block J (0 <= J <= I), or
// kCorr + ct for correction tile ct (pooled blocks ct*BLK .. ct*BLK+BLK-1).
constexpr int kCorr = FP_MAX_BLOCKS;

// Persistent: each workgroup takes one work item from each band of G =
// gridDim consecutive items (items run longest first; G is a multiple of 8 so
// an item keeps its XCD).  An item walks its tiles -- the kept blocks of its
// HP heads in ascending order, then the tiles of skipped past blocks whose
// pooled means form the correction -- through one double-buffered DMA
// pipeline.  As soon as the walk ends, the next item's first tile is DMA'd
// into buffer pair 1 while this item's output is normalised and stored.
template <int D, int BLK, int HP, bool PAGED>
__global__ __launch_bounds__(64 * HP * (BLK / 32)) void k_attn_bf16(AttnArgs a, SeqTable t) {
    using G = Geo<D, BLK, HP>;
    using It = Item<D, BLK, HP, PAGED>;
    // Four separate LDS objects: the compiler then sees that a DMA into one
    // buffer does not touch the buffer being read, and does not wait on it.
    __shared__ __attribute__((aligned(16))) char kb0[G::TILE];
    __shared__ __attribute__((aligned(16))) char kb1[G::TILE];
    __shared__ __attribute__((aligned(16))) char vb0[G::TILE];
    __shared__ __attribute__((aligned(16))) char vb1[G::TILE];
    // Bit J of head j: block J < I is kept by head j of the current item.
    __shared__ uint32_t kept_bits[HP][FP_MAX_BLOCKS / 32];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
    const int hs = w / G::WPH;                   // which of the HP heads this wave serves
    const int rw = w % G::WPH;                   // 32-row group inside the query block
    const int nitems = t.total_items * (a.Hq / HP);
    const int64_t rs = (int64_t)a.Hkv * D;
    const float c = a.scale_log2;
    const float log2_blk = __log2f((float)BLK);  // past blocks are full: ln n_J = ln BLK
    // Band k of gridDim items goes to the workgroups rotated by k rows of 8,
    // so a workgroup stays on its XCD (item % 8) but does not always draw the
    // same head pair (heads differ in density).
    const int G8 = gridDim.x % 8 == 0 ? (int)gridDim.x / 8 : 0;
    auto item_index = [&](int k) {
        return G8 ? k * (int)gridDim.x + (((int)blockIdx.x / 8 + k) % G8) * 8 + (int)blockIdx.x % 8
                  : k * (int)gridDim.x + (int)blockIdx.x;
    };
    int band = 0;
    int idx = item_index(0);
    if (idx >= nitems) return;

    // Lane-dependent values.  They are re-derived through an opaque copy of the
    // thread index at the start of each item and of the epilogue, so the
    // compiler keeps only the current phase's LDS addresses in registers
    // instead of hoisting all of them out of the item loop.
    int lane, col, half, qr, tphase;
    auto phase = [&]() {
        tphase = tid;
        asm volatile("" : "+v"(tphase));
        lane = tphase & 63;
        col = lane & 31;
        half = lane >> 5;
        qr = 32 * rw + col;
    };
    phase();

    // Per-thread DMA plan: chunk offsets relative to a tile's first row.
    DmaPlan<D, BLK, HP> plan;
    const uint4* zero = &kZeroChunk;
    const int wave_base = __builtin_amdgcn_readfirstlane(64 * w * 16);
    auto issue = [&](const It& itm, int code, char* kdst, char* vdst) {
        if (code < kCorr) {
            issue_tile<D, BLK, HP, PAGED>(itm.kfirst, itm.pages, a.kv, rs, code, itm.len - code * BLK, plan, zero,
                                          kdst, wave_base);
            issue_tile<D, BLK, HP, PAGED>(itm.vfirst, itm.pages, a.kv, rs, code, itm.len - code * BLK, plan, zero,
                                          vdst, wave_base);
        } else {
            // Pooled rows of this request's blocks for the KV head (contiguous, row stride D).
            const int ct = code - kCorr;
            const int64_t prow = ((int64_t)itm.hk * t.total_blocks + t.blk_off[itm.b]) * D;
            issue_tile<D, BLK, HP, false>(a.pk16 + prow, nullptr, a.kv, D, ct, itm.I - ct * BLK, plan, zero, kdst,
                                          wave_base);
            issue_tile<D, BLK, HP, false>(a.pv16 + prow, nullptr, a.kv, D, ct, itm.I - ct * BLK, plan, zero, vdst,
                                          wave_base);
        }
    };
    // Record a kept block in the bitmap (each wave sets it itself, so its own
    // later reads see it without a barrier).
    auto mark = [&](const It& itm, int code, int act) {
        if (code < itm.I && lane == 0) {
#pragma unroll
            for (int j = 0; j < HP; ++j)
                if ((act >> j) & 1) atomicOr(&kept_bits[j][code >> 5], 1u << (code & 31));
        }
    };
    // Next tile of an item: its kept blocks, then the correction tiles in
    // which some head skips a past block (act: the heads that use the tile).
    auto next_tile = [&](It& itm, int& act) -> int {
        if (itm.ct < 0) {
            const int J = itm.u.next(act);
            if (J != INT_MAX) {
                mark(itm, J, act);
                return J;
            }
            itm.ct = 0;
        }
        while (itm.ct < itm.nct) {
            const int ct = itm.ct++;
            int any = 0;
#pragma unroll
            for (int sub = 0; sub < G::NSUB; ++sub) {
                const int j0 = ct * BLK + 32 * sub;
                const int nvalid = min(32, max(0, itm.I - j0));
                const uint32_t valid = nvalid >= 32 ? 0xffffffffu : ((1u << nvalid) - 1u);
#pragma unroll
                for (int j = 0; j < HP; ++j)
                    if (~kept_bits[j][j0 >> 5] & valid) any |= 1 << j;
            }
            any = __builtin_amdgcn_readfirstlane(any);
            if (any) {
                act = any;
                return kCorr + ct;
            }
        }
        return INT_MAX;
    };
    auto zero_bits = [&](const It& itm) {
        const int nwords = (itm.I + 31) >> 5;
        for (int i = tphase; i < HP * nwords; i += G::NT) kept_bits[i / nwords][i % nwords] = 0u;
    };
    bf16x8 qf[D / 16];
    // Rows past the end of a ragged last block re-read the last valid row:
    // their outputs are never stored, and unconditional loads keep the
    // compiler from waiting on them (and on DMAs issued before) when the
    // registers are written.
    auto load_q = [&](const It& itm) {
        const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                             ((int64_t)(itm.q0 + min(qr, itm.nI - 1)) * a.Hq + itm.h) * D + 8 * half;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 16 * kk));
    };

    It cur;
    cur.setup(a, t, idx, hs);
    int act, act_next;
    plan.init(tphase);
    zero_bits(cur);
    lds_barrier();
    int J = next_tile(cur, act);
    if (J != INT_MAX) issue(cur, J, kb1, vb1);
    load_q(cur);

    float m, l;
    f32x16 o[G::NDS];
    constexpr int SH = G::NSUB > 1 ? G::NSUB / 2 : 1;   // subtiles per half tile
    f32x16 s[SH];
    uint32_t pk[SH][8];

    // One tile: wait for its DMA, release the other buffers by the barrier,
    // prefetch the next tile into them, compute on this one.
    auto step = [&](char* kcur, char* vcur, char* knext, char* vnext) {
        __builtin_amdgcn_s_waitcnt(0);                   // this thread's DMA for tile J is done
        lds_barrier();                                   // ... every thread's; the other buffers are free
        const int Jn = next_tile(cur, act_next);
        if (Jn != INT_MAX) issue(cur, Jn, knext, vnext);
        if ((act >> hs) & 1) {
            const bool corr = J >= kCorr;
            // Correction tile: bit j of skip[sub] <=> pooled block ct*BLK + 32 sub + j
            // is strictly past and not kept by this head.
            uint32_t skip[G::NSUB];
            if (corr) {
#pragma unroll
                for (int sub = 0; sub < G::NSUB; ++sub) {
                    const int j0 = (J - kCorr) * BLK + 32 * sub;
                    const int nvalid = min(32, max(0, cur.I - j0));
                    const uint32_t valid = nvalid >= 32 ? 0xffffffffu : ((1u << nvalid) - 1u);
                    skip[sub] = __builtin_amdgcn_readfirstlane(~kept_bits[hs][j0 >> 5] & valid);
                }
            }
            // Two halves of SH subtiles each: online softmax per half keeps S and
            // P at half size, which leaves registers to read operands ahead.
            auto half_tile = [&](auto sub0) {
                constexpr int S0 = decltype(sub0)::value;
                qk<D, BLK, HP, S0, SH>(reinterpret_cast<const uint4*>(kcur), qf, col, half, s);
                if (corr) {
                    // Element r of a lane in half hf is block 32 sub + (r & 3) + 8 (r >> 2) + 4 hf:
                    // the keep mask is uniform per half, so it is built on the scalar
                    // unit as a 64-lane mask and applied with one select.
#pragma unroll
                    for (int j = 0; j < SH; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int k0 = (r & 3) + 8 * (r >> 2);
                            const uint64_t keep = (((skip[S0 + j] >> k0) & 1u) ? 0xffffffffull : 0ull) |
                                                  (((skip[S0 + j] >> (k0 + 4)) & 1u) ? 0xffffffff00000000ull : 0ull);
                            s[j][r] = __builtin_amdgcn_inverse_ballot_w64(keep) ? s[j][r] : -INFINITY;
                        }
                } else if (J == cur.I) {
                    // Causal mask of the diagonal tile.  The limit is made opaque so
                    // the 16 * SH lane masks are computed here, once per item, instead
                    // of being hoisted out of the loops and held in registers.
                    int lim = qr - 4 * half;
                    asm volatile("" : "+v"(lim));
#pragma unroll
                    for (int j = 0; j < SH; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = 32 * (S0 + j) + (r & 3) + 8 * (r >> 2);
                            s[j][r] = key > lim ? -INFINITY : s[j][r];
                        }
                }
                softmax_update<SH, G::NDS>(s, c, corr ? log2_blk : 0.f, m, l, o, pk);
                pv<D, BLK, HP, S0, SH>(vcur, pk, lane, o);
            };
            half_tile(std::integral_constant<int, 0>());
            if (G::NSUB > SH) half_tile(std::integral_constant<int, (G::NSUB > SH ? SH : 0)>());
        }
        J = Jn;
        act = act_next;
    };

    while (true) {
        phase();
        plan.init(tphase);
        m = -INFINITY;
        l = 0.f;
#pragma unroll
        for (int ds = 0; ds < G::NDS; ++ds) o[ds] = f32x16{};
        // All tiles; the first one is already in pair 1.
        while (J != INT_MAX) {
            step(kb1, vb1, kb0, vb0);
            if (J == INT_MAX) break;
            step(kb0, vb0, kb1, vb1);
        }
        lds_barrier();                                   // all reads of the last tile and the bitmap are done

        // Next item: its lists and first tile (pair 1) go in flight now.
        const int nidx = item_index(band + 1);
        const bool has_next = nidx < nitems;
        It nxt;
        int Jn0 = INT_MAX, actn0 = 0;
        if (has_next) {
            nxt.setup(a, t, nidx, hs);
            zero_bits(nxt);
            Jn0 = nxt.u.next(actn0);                     // a kept block (lists are never empty)
            if (Jn0 != INT_MAX) issue(nxt, Jn0, kb1, vb1);
        }

        // Epilogue: normalise, stage each head's bf16 tile in LDS (kb0 for the
        // first head, vb0 for the second; the next item's first tile is
        // arriving in kb1/vb1), store full rows.  Each buffer is named in a
        // branch of its own, kept apart by distinct empty asm statements, so
        // the compiler sees which object is accessed and does not wait for
        // the DMA.
        phase();
        const float l_tot = l + __shfl_xor(l, 32);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        lds_barrier();                                   // zeroed bitmap; staging buffers free
        if (has_next) mark(nxt, Jn0, actn0);
        auto stage_rows = [&](char* buf) {
            uint4* stage = reinterpret_cast<uint4*>(buf);
#pragma unroll
            for (int ds = 0; ds < G::NDS; ++ds)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int chunk = 4 * ds + g4;       // d0 = 32 ds + 8 g4 + 4 half
                    const uint2 v2 = make_uint2(pack_bf16(o[ds][4 * g4] * inv, o[ds][4 * g4 + 1] * inv),
                                                pack_bf16(o[ds][4 * g4 + 2] * inv, o[ds][4 * g4 + 3] * inv));
                    reinterpret_cast<uint2*>(&stage[qr * G::NCH + (chunk ^ swz<D>(qr))])[half] = v2;
                }
        };
        auto store_rows = [&](const char* buf) {
            const uint4* stage = reinterpret_cast<const uint4*>(buf);
            const int ht = tphase % (64 * G::WPH);       // thread index within this head's waves
            for (int i = ht; i < cur.nI * G::NCH; i += 64 * G::WPH) {
                const int row = i / G::NCH, ch = i % G::NCH;
                *reinterpret_cast<uint4*>(a.out + ((int64_t)(cur.q0 + row) * a.Hq + cur.h) * D + ch * 8) =
                    stage[row * G::NCH + (ch ^ swz<D>(row))];
            }
        };
        if (hs == 0) {
            stage_rows(kb0);
            asm volatile("; staged head 0");
        } else {
            stage_rows(vb0);
            asm volatile("; staged head 1");
        }
        if (has_next) load_q(nxt);                       // O is staged: its registers take the next Q
        lds_barrier();
        if (hs == 0) {
            store_rows(kb0);
            asm volatile("; stored head 0");
        } else {
            store_rows(vb0);
            asm volatile("; stored head 1");
        }
        if (a.lse && half == 0 && qr < cur.nI)
            a.lse[(int64_t)cur.h * t.total_tokens + cur.q0 + qr] = (m + __log2f(l_tot)) * kLn2;
        if (!has_next) break;
        cur = nxt;
        idx = nidx;
        ++band;
        J = Jn0;
        act = actn0;
    }
}

// Persistent grid: as many workgroups as the device holds at once (a multiple
// of the 8 XCDs), at most one per item.  The resident count is computed once
// per kernel and device.
template <typename K>
int persistent_grid(K kernel, int block, int nitems) {
    constexpr int kMaxDev = 64;
    static std::atomic<int> resident[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nitems;
    int n = resident[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        int ncu = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess)
            return nitems;
        n = max(8, (ncu * max(per_cu, 1)) / 8 * 8);
        resident[dev].store(n, std::memory_order_relaxed);
    }
    return max(1, min(nitems, n));
}

template <int D, int BLK, int HP>
hipError_t launch_t(const AttnArgs& a, const SeqTable& t, bool paged, hipStream_t s) {
    const int nitems = t.total_items * (a.Hq / HP);
    const int block = 64 * HP * (BLK / 32);
    if (paged) {
        auto k = k_attn_bf16<D, BLK, HP, true>;
        hipLaunchKernelGGL(k, dim3(persistent_grid(k, block, nitems)), dim3(block), 0, s, a, t);
    } else {
        auto k = k_attn_bf16<D, BLK, HP, false>;
        hipLaunchKernelGGL(k, dim3(persistent_grid(k, block, nitems)), dim3(block), 0, s, a, t);
    }
    return hipGetLastError();
}

template <int D, int BLK>
hipError_t launch_db(const AttnArgs& a, const SeqTable& t, bool paged, hipStream_t s) {
    return (a.g % 2 == 0) ? launch_t<D, BLK, 2>(a, t, paged, s) : launch_t<D, BLK, 1>(a, t, paged, s);
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
