// Work-item walk shared by the attention kernels: the persistent item loop's
// pieces (list cursor, item setup, tile DMA, grid sizing).  A work item is
// (query block I of one request, HP query heads of one KV head); its tiles
// are the union of the heads' kept KV blocks followed by the tiles of pooled
// means that form the correction (FlashPrefill, gist.science technical
// summary, section 2.C; FlashPrefill V2 abstract).
#pragma once
#include <mutex>
#include <type_traits>

#include "fp_attn.h"

namespace fp_walk {
using namespace fp_attn;

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Source of DMA chunks for rows that hold no data (out-of-range pages).
static __device__ const uint4 kZeroChunk = {0u, 0u, 0u, 0u};

// XOR swizzle of 16-byte chunks within a row: conflict-free for the MFMA K
// reads (16 consecutive rows, one chunk) and for the transposing V reads
// (4 consecutive rows, 2 adjacent chunks).
template <int D>
__device__ __forceinline__ int swz(int row) {
    if (D == 128) return ((row & 7) << 1) | ((row >> 3) & 1);
    if (D == 64) return (row >> 1) & 7;
    return (row >> 2) & 3;   // D == 32: 64-byte rows of fp8 d = 64 tiles
}

// Workgroup geometry of the bf16 kernel: 32 query rows per wave.
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
template <int D, int BLK, int NT>
struct DmaPlan {
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

// Page ids of this thread's DMA rows of tile J (paged layout), all loaded
// before any of the tile's DMAs is issued: the vector-memory counter is in
// order, so a page id loaded between DMAs could only be waited for together
// with the DMAs before it.  Rows past the request's end (row >= nvalid) look
// up its last valid row's page, so the block-table read stays inside the
// pages that cover the request.
template <int D, int BLK, int NT>
__device__ __forceinline__ void load_tile_pages(const int32_t* pages, const KVLayout& L, int J, int nvalid,
                                                const DmaPlan<D, BLK, NT>& plan, int* pg) {
#pragma unroll
    for (int i = 0; i < DmaPlan<D, BLK, NT>::NLOAD; ++i)
        pg[i] = pages[(J * BLK + min(plan.row(i), nvalid - 1)) / L.page_size];
}

// DMA one tile: rows J*BLK .. of the request whose first row is `first`
// (contiguous), or of its pages pg from load_tile_pages (paged).
template <int D, int BLK, int NT, bool PAGED>
__device__ __forceinline__ void issue_tile(const uint16_t* first, const int* pg, const KVLayout& L,
                                           int64_t rs, int J, int nvalid, const DmaPlan<D, BLK, NT>& plan,
                                           const uint4* zero, char* lds, int wave_base) {
    using P = DmaPlan<D, BLK, NT>;
    static_assert((BLK * P::NCH) % NT == 0, "tile chunks must split evenly");
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
            __builtin_amdgcn_global_load_lds(tile + off, (lds_void*)(lds + (i * NT) * 16 + wave_base), 16, 0, 0);
        }
    } else {
#pragma unroll
        for (int i = 0; i < P::NLOAD; ++i) {
            const int row = plan.row(i);
            const int tr = J * BLK + row;
            const int page = pg[i];
            // Opaque column offset: keeps the compiler from holding a 64-bit
            // pointer per chunk across the loop (it would spill).
            int co = plan.coff(i);
            asm volatile("" : "+v"(co));
            const uint16_t* p = first + ((int64_t)page * L.page_size + tr % L.page_size) * rs + co;
            const void* src =
                (row < nvalid && (unsigned)page < (unsigned)L.num_pages) ? (const void*)p : (const void*)zero;
            __builtin_amdgcn_global_load_lds(src, (lds_void*)(lds + (i * NT) * 16 + wave_base), 16, 0, 0);
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
    int b, nb, I, tok0, len, q0, lo, nI, hk, h;  // h: this wave's query head; rows lo .. nI-1 exist
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
        const int first = first_block(t, b);          // query blocks are first .. nb-1
        I = nb - 1 - local;
        tok0 = t.tok_off[b];
        len = context_len(t, b, BLK);
        // Row r of the block is query row q0 + r; a chunk that starts inside
        // its first block has no rows before lo there.
        const int ph = chunk_phase(t, b, BLK);
        q0 = tok0 + (I - first) * BLK - ph;
        lo = I == first ? ph : 0;
        nI = min(BLK, len - I * BLK);
        hk = h / a.g;
        const int64_t rs = (int64_t)a.Hkv * D;
        const int h0 = h - hs;
        // The heads' counts and first list windows load together (unconditional
        // loads, lanes past the capacity re-read the last entry and are masked
        // after), so setting up an item waits on memory once.
        int cnt_raw[HP], win_raw[HP];
        u.cap = I + 1;
#pragma unroll
        for (int j = 0; j < HP; ++j) {
            u.list[j] = a.kv_idx + list_row(t, b, h0 + j, I, nb, first);
            cnt_raw[j] = a.kv_cnt[count_index(t, a.Hq, b, h0 + j, I, nb, first)];
            win_raw[j] = u.list[j][min((int)__lane_id(), I)];
        }
        __builtin_amdgcn_sched_barrier(0);               // all four loads before the first use
#pragma unroll
        for (int j = 0; j < HP; ++j) {
            u.cnt[j] = __builtin_amdgcn_readfirstlane(cnt_raw[j]);
            u.pos[j] = 0;
            u.wbase[j] = 0;
            u.win[j] = (int)__lane_id() < u.cap ? win_raw[j] : INT_MAX;
        }
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

// Persistent grid: as many workgroups as the device holds at once (a multiple
// of the 8 XCDs), at most one per item.  The resident count depends on the
// kernel (its registers and LDS) and the block size, so it is computed once
// per (kernel, block size, device) and cached under that key: every
// instantiation of a kernel template has the same function type, so a cache
// keyed by type alone would let the first variant launched size all others.
inline int resident_workgroups(const void* kernel, int block) {
    struct Entry {
        const void* fn;
        int block, dev, n;
    };
    constexpr int kMaxEntries = 256;
    static std::mutex mu;
    static Entry cache[kMaxEntries];
    static int used = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
        if (cache[i].fn == kernel && cache[i].block == block && cache[i].dev == dev) return cache[i].n;
    int ncu = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess)
        return 0;
    const int n = max(8, (ncu * max(per_cu, 1)) / 8 * 8);
    if (used < kMaxEntries) cache[used++] = Entry{kernel, block, dev, n};
    return n;
}

template <typename K>
int persistent_grid(K kernel, int block, int nitems) {
    const int n = resident_workgroups(reinterpret_cast<const void*>(kernel), block);
    return n > 0 ? max(1, min(nitems, n)) : nitems;
}

}  // namespace fp_walk
