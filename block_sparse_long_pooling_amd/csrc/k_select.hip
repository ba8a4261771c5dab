// Pooled block scores, max-based dynamic threshold and list compaction
// (FlashPrefill, gist.science technical summary, sections 2.A-2.C).
//
// For query head h and query block I, s[J] = sigma * q_bar[h,I] . k_bar[h/g,J]
// over J <= I.  Block J is kept iff its softmax score is at least alpha times
// the row's largest, i.e. s[J] - max_J s >= ln(alpha).  Kept blocks are
// written in ascending J to the (h, I) list, which is never empty.
//
// A workgroup of 8 waves owns up to 128 score rows of one KV head: 4 row
// waves, each 32 rows = TI consecutive query blocks x the g query heads, and
// 2 column groups.  A row wave's cost grows with its last query block, so the
// row waves are dealt to workgroups in a snake (the longest with the
// shortest, two middle ones together) and every workgroup gets about the
// same number of (row, column tile) products.  The k_bar rows stream
// through LDS in column tiles of 32 blocks, two tiles per step (one per
// column group), split once per workgroup into bf16 hi + lo parts; every
// tile then serves all the rows of the workgroup.  The rows of the step after
// next are loaded into registers while the current step computes.
//
// The (L/B)^2 score matrix is never stored.  Phase 1 walks the column tiles
// from the last to the first, so a row wave meets its diagonal tile first,
// keeps each row's running max m (shared by the two column groups after
// every step) and writes each (tile, row)'s keep bits s - m >= ln(alpha) to
// a bitmap in LDS.  A bit set against a running max below the final one may
// be wrong; a bit clear stays clear, since the max only grows.  Phase 2
// recomputes the same scores (same instruction sequence, bit-identical) only
// for the tiles holding such words; when the row max lies in the diagonal
// tile, as it does when nearby blocks score highest, there are none.  Phase 3
// compacts the bitmap in ascending J.  The dot products run on bf16 MFMA with each
// fp32 operand split into hi + lo bf16 parts (hi*hi + hi*lo + lo*hi), which
// is within ~2^-17 of the fp32 product sum -- far below the 1e-3 band in
// which the threshold decision is allowed to differ from an exact one.
#include "fp_launch.h"

// Scores feed both the row max (pass 1) and the compare s - max (pass 2); no
// multiply may be fused into a later add, or the two passes would disagree.
#pragma clang fp contract(off)

namespace {

constexpr int kRowWaves = kSelectRowWaves;
constexpr int kColGroups = 2;
constexpr int kWaves = kRowWaves * kColGroups;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowSlots = 32 * kRowWaves;
constexpr int kMaxColTiles = FP_MAX_BLOCKS / 2 / 32;   // 32-block column tiles per row

__device__ __forceinline__ void split8(const float4& x0, const float4& x1, bf16x8& hi, bf16x8& lo) {
    float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        __bf16 h = (__bf16)x[i];
        hi[i] = h;
        lo[i] = (__bf16)(x[i] - (float)h);
    }
}

// LDS stage of one column tile: hi and lo bf16 parts of 32 k_bar rows, row
// J at chunks [J * D/8, (J + 1) * D/8) of 16 bytes, chunk c stored at
// c ^ (J mod D/8) so that the 32 rows' reads of one chunk spread over the
// banks.
template <int D>
struct TileStage {
    uint4 part[2][32 * D / 8];
};

template <int D>
__device__ __forceinline__ int chunk_slot(int J, int c) {
    return J * (D / 8) + (c ^ (J & (D / 8 - 1)));
}

// Staging: thread -> (column group, k_bar row J in the tile, D/8 consecutive
// floats of that row).
template <int D>
struct Stager {
    static constexpr int F = D / 8;            // floats per thread
    int cg, J, seg;
    __device__ __forceinline__ Stager(int tid) : cg(tid / 256), J((tid % 256) / 8), seg(tid % 8) {}
    // Rows past the workgroup's last column block (ncol - 1) re-read that
    // block: they are causally masked for every row that scores them, and an
    // unconditional load keeps the in-flight loads of the other buffer from
    // being waited for.
    __device__ __forceinline__ void load(const float* pk, int64_t krow0, int ct, int ncol, float4* x) const {
        const int blk = min(32 * ct + J, ncol - 1);
        const float4* src = reinterpret_cast<const float4*>(pk + (krow0 + blk) * D + F * seg);
#pragma unroll
        for (int i = 0; i < F / 4; ++i) x[i] = src[i];
    }
    __device__ __forceinline__ void store(TileStage<D>* st, const float4* x) const {
#pragma unroll
        for (int i = 0; i < F / 8; ++i) {
            bf16x8 h, l;
            split8(x[2 * i], x[2 * i + 1], h, l);
            const int slot = chunk_slot<D>(J, (F / 8) * seg + i);
            st[cg].part[0][slot] = __builtin_bit_cast(uint4, h);
            st[cg].part[1][slot] = __builtin_bit_cast(uint4, l);
        }
    }
};

// Transposed scores S^T = K_bar (sigma Q_bar)^T of one column tile: lane
// (rho, half) holds query row rho and, in register r, column block
// (r%4) + 8*(r/4) + 4*half of the tile.  One MFMA chain accumulates
// hi*hi, hi*lo and lo*hi per 16-wide slice of d: the same instruction
// sequence gives the same bits in every pass.  Lane (rho, half) supplies
// k_bar row rho and query row rho, d = 16 kk + 8 half .. + 7.
template <int D>
__device__ __forceinline__ f32x16 tile_scores(const bf16x8* qh, const bf16x8* ql, const TileStage<D>& st, int rho,
                                              int half) {
    // All operand reads go out before the first product.
    bf16x8 kh[D / 16], kl[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        const int slot = chunk_slot<D>(rho, 2 * kk + half);
        kh[kk] = __builtin_bit_cast(bf16x8, st.part[0][slot]);
        kl[kk] = __builtin_bit_cast(bf16x8, st.part[1][slot]);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x16 acc = {};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh[kk], qh[kk], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kl[kk], qh[kk], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh[kk], ql[kk], acc, 0, 0, 0);
    }
    return acc;
}

// Workgroup barrier over LDS only: the next step's global loads stay in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Combine a lane's value with that of lane l ^ 32 (the other half of the
// wave holds the other 16 columns of the same score row).  permlane32_swap
// exchanges the halves of two copies of v, which then hold the lower and the
// upper half's values in every lane: a register move, no LDS round trip.
__device__ __forceinline__ float max_halves(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ uint32_t or_halves(uint32_t v) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return r[0] | r[1];
}

// Workgroup = up to 128 score rows (4 row waves x TI query blocks x g heads)
// of one KV head.  Wave wv: row wave rw = wv / 2, column group cg = wv % 2;
// each step stages two column tiles, and column group cg scores the (cg)-th
// of them for its row wave's rows.  Phase 1 (tiles in descending order):
// running row maxima, exchanged between the column groups every step, and
// each (tile, row)'s keep bits against the running max, in an LDS bitmap
// [tile][row slot].  Phase 2: the tiles with a word formed before its row's
// max last grew are scored again against the final max.  Phase 3: one lane
// per row slot writes the row's list in ascending J.
template <int D>
__global__ __launch_bounds__(kThreads, 1) void k_select(SelArgs a, SeqTable t) {
    __shared__ TileStage<D> stage[2][kColGroups];
    __shared__ uint32_t bits[kMaxColTiles][kRowSlots];
    __shared__ float xch[kColGroups][kRowSlots];      // phase 1: the step's tile maxima
    __shared__ int32_t wstale[kWaves];               // phase 1: the wave holds a stale row
    __shared__ uint32_t need[kMaxColTiles / 32];     // phase 2: tiles some row may keep from
    __shared__ int32_t todo[kMaxColTiles];           // ... in ascending order

    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    // Column groups of a row wave on different SIMDs (waves are dealt to the
    // 4 SIMDs in turn): row waves 0 and 2 on SIMDs 0-1, 1 and 3 on SIMDs 2-3.
    const int rw = wv >> 1, cg = wv & 1;
    const int rank = blockIdx.x / a.Hkv;
    const int hk = blockIdx.x % a.Hkv;
    int b, local;
    item_of(t, rank, b, local);
    const int nb = seq_blocks(t, b);
    const int first = first_block(t, b);             // query blocks are first .. nb-1
    const int TIW = kRowWaves * a.TI;                // query blocks per workgroup
    const int ntiles = (nb - first + TIW - 1) / TIW;
    // Row waves are dealt to workgroups so that every workgroup gets about
    // the same number of column tiles, and each SIMD pair too: with the
    // request's nrw row waves counted from the longest (i = 0), workgroup
    // `local` of K takes i = local (row wave 0), 2K-1-local (1), 4K-1-local
    // (2, the shortest, beside the longest) and 2K+local (3).
    const int nrw = (nb - first + a.TI - 1) / a.TI;
    auto rw_first = [&](int r) {
        const int K = ntiles;
        const int i = r == 0 ? local : r == 1 ? 2 * K - 1 - local : r == 2 ? 4 * K - 1 - local : 2 * K + local;
        return i < nrw ? first + (nrw - 1 - i) * a.TI : nb;     // nb: no rows
    };
    const int gblk0 = t.blk_off[b];
    const int rows = a.TI * a.g;                     // used row slots per row wave
    const int rho = lane & 31;
    const int half = lane >> 5;
    const int Iw0 = rw_first(rw);                    // this row wave's first query block
    const int Iw_end = min(nb, Iw0 + a.TI);          // and one past its last
    const int ntile_w = Iw_end > Iw0 ? (Iw_end - 1) / 32 + 1 : 0;   // column tiles it needs
    const bool rows_full = rows == 32 && Iw0 + a.TI <= nb;

    const int ncol = min(nb, rw_first(0) + a.TI);    // row wave 0 holds the workgroup's last rows
    const int ntile = (ncol + 31) >> 5;
    const int64_t krow0 = (int64_t)hk * t.total_blocks + gblk0;
    const Stager<D> sg(tid);
    if (tid < kMaxColTiles / 32) need[tid] = 0u;

    // Phase 1 stages the column tiles from the last to the first: entry i of
    // the order is tile ntile - 1 - i; past the end, tile ntile, which is
    // staged but never scored.
    auto tile1 = [&](int i) { return i < ntile ? ntile - 1 - i : ntile; };
    // Two register buffers: the rows of step p + 2 load while step p scores.
    float4 x0[Stager<D>::F / 4], x1[Stager<D>::F / 4];

    // Query rows.  Row slot r (row wave r / 32, row rho = r % 32) is query
    // block rw_first(r / 32) + rho / g of head hk*g + rho % g; slots without a
    // query block read the first block and are zeroed by the scale below.
    // Both column groups of a row wave need the same rows, so the
    // workgroup's rows are read from memory once, into LDS (the bitmap's
    // space, unused until phase 1; 16-byte chunks swizzled per row), and
    // every lane takes its fragment from there: d = 16 kk + 8 half .. + 7.
    // With group-pooled lists every row of a query block holds the sum of its
    // g heads' rows, and the scale takes the 1/g of their mean.
    const int rowI = Iw0 + rho / a.g;
    const bool rowOk = rho < rows && rowI < nb;
    const bool pooled = a.shared == 2;
    const int slot = 32 * rw + rho;
    constexpr int QCH = D / 4;                                  // 16-byte chunks per fp32 row
    float4* qstage = reinterpret_cast<float4*>(&bits[0][0]);   // [kRowSlots][QCH]
    auto qpos = [](int r, int c) { return r * QCH + (c ^ (r & (QCH - 1))); };
    sg.load(a.pk, krow0, tile1(sg.cg), ncol, x0);        // phase 1's first two steps
    sg.load(a.pk, krow0, tile1(2 + sg.cg), ncol, x1);
    {
        // All of a thread's loads are issued before the first LDS write, so
        // the gather waits on memory once.
        constexpr int NQ = kRowSlots * QCH / kThreads;
        float4 qv[NQ];
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int e = tid + i * kThreads;
            const int r = e / QCH, c = e % QCH;
            const int rr = r % 32;
            const int I = rw_first(r / 32) + rr / a.g;
            const bool ok = rr < rows && I < nb;
            const int h = hk * a.g + rr % a.g;
            const int64_t qrow = qblock_row(t, b, ok ? I : first);
            qv[i] = reinterpret_cast<const float4*>(a.pq + ((int64_t)h * t.total_qblocks + qrow) * D)[c];
        }
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int e = tid + i * kThreads;
            qstage[qpos(e / QCH, e % QCH)] = qv[i];
        }
    }
    lds_barrier();
    bf16x8 qh[D / 16], ql[D / 16];
    {
        float4 qf[D / 8];
        const int r0 = pooled ? 32 * rw + (rho / a.g) * a.g : slot;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            qf[2 * kk] = qstage[qpos(r0, 4 * kk + 2 * half)];
            qf[2 * kk + 1] = qstage[qpos(r0, 4 * kk + 2 * half + 1)];
        }
        if (pooled) {
            for (int j = 1; j < a.g; ++j) {
#pragma unroll
                for (int kk = 0; kk < D / 8; ++kk) {
                    const float4 x = qstage[qpos(min(r0 + j, 32 * rw + 31), 4 * (kk / 2) + 2 * half + (kk & 1))];
                    qf[kk] = make_float4(qf[kk].x + x.x, qf[kk].y + x.y, qf[kk].z + x.z, qf[kk].w + x.w);
                }
            }
        }
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            const float sc = rowOk ? (pooled ? a.scale / (float)a.g : a.scale) : 0.f;
            const float4 u = qf[2 * kk], v = qf[2 * kk + 1];
            split8(make_float4(u.x * sc, u.y * sc, u.z * sc, u.w * sc),
                   make_float4(v.x * sc, v.y * sc, v.z * sc, v.w * sc), qh[kk], ql[kk]);
        }
    }
    // One pass over column tiles tile_of(0), tile_of(1), ... (a tile index
    // >= ntile is staged but not scored): step p stages entries 2p and
    // 2p + 1, and column group cg calls visit(ct, stage) on entry 2p + cg if
    // its row wave needs that tile.  x0 and x1 hold steps 0 and 1 on entry.
    auto sweep = [&](int nstep, auto&& tile_of, auto&& visit) {
        sg.store(stage[0], x0);
        lds_barrier();
        auto step = [&](int p, float4* xnext, float4* xfree) {
            sg.load(a.pk, krow0, tile_of(2 * (p + 2) + sg.cg), ncol, xfree);
            const int ct = tile_of(2 * p + cg);
            if (ct < ntile_w) visit(ct, stage[p & 1][cg]);
            if (!kSerialFill && p + 1 < nstep) sg.store(stage[(p + 1) & 1], xnext);
            lds_barrier();
            if (kSerialFill) {                           // fill only after every read of this step
                if (p + 1 < nstep) sg.store(stage[(p + 1) & 1], xnext);
                lds_barrier();
            }
        };
        for (int p = 0; p < nstep; p += 2) {
            step(p, x1, x0);
            if (p + 1 < nstep) step(p + 1, x0, x1);
        }
    };
    // Tiles wholly below the row wave's first query block with every row
    // valid need no causal mask.  Column block of register r within a tile:
    auto masked = [&](int ct) { return !(rows_full && 32 * ct + 31 <= Iw0); };
    auto colJ = [&](int r) { return (r & 3) + 8 * (r >> 2) + 4 * half; };
    // Columns of tile ct that this lane's row may keep: J <= rowI, and none
    // for rows without a query block.
    auto colmask = [&](int ct) -> uint32_t {
        if (!masked(ct)) return 0xffffffffu;
        const int lim = rowI - 32 * ct;             // last column the row may keep
        const uint32_t cm = lim >= 31 ? 0xffffffffu : lim < 0 ? 0u : (2u << lim) - 1u;
        return rowOk ? cm : 0u;
    };
    // Keep bits of the row (both halves' columns), branch-free.
    auto keep_bits = [&](const f32x16& s, int ct, float mrow) {
        uint32_t w = 0u;
#pragma unroll
        for (int r = 0; r < 16; ++r) w |= (s[r] - mrow >= a.ln_alpha) ? (1u << colJ(r)) : 0u;
        return or_halves(w) & colmask(ct);
    };

    // Phase 1: per step the two column groups exchange their tile maxima, so
    // m is the row's max over every tile visited so far, and each visited
    // (tile, row) gets its keep bits against that running max.  A word is
    // final unless m grows at a later step and the word holds a bit (a larger
    // max only clears bits): such a row is flagged stale, and phase 2 scores
    // its tiles again.  When the row max lies in the diagonal tile -- the
    // usual case, nearby blocks score highest -- nothing is stale.
    const int nstep1 = (ntile + 1) >> 1;
    float m = -INFINITY;     // running row max (the same in both column groups)
    int last_inc = -1;       // last step at which m grew
    bool nz = false;         // this column group has formed a word with a bit
    bool stale_row = false;  // ... and m grew after that
    sg.store(stage[0], x0);
    lds_barrier();
    auto step1 = [&](int p, float4* xnext, float4* xfree) {
        sg.load(a.pk, krow0, tile1(2 * (p + 2) + sg.cg), ncol, xfree);
        const int ct = tile1(2 * p + cg);
        const bool vis = ct < ntile_w;
        f32x16 s = {};
        float tm = -INFINITY;
        // The next step's rows go into the other stage buffer (its last
        // readers finished before the previous barrier) while this step's
        // products run.
        if (vis) {
            s = tile_scores<D>(qh, ql, stage[p & 1][cg], rho, half);
            if (!kSerialFill && p + 1 < nstep1) sg.store(stage[(p + 1) & 1], xnext);
            if (masked(ct)) {
                const uint32_t cm = colmask(ct);
#pragma unroll
                for (int r = 0; r < 16; ++r) tm = fmaxf(tm, ((cm >> colJ(r)) & 1u) ? s[r] : -INFINITY);
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) tm = fmaxf(tm, s[r]);
            }
            tm = max_halves(tm);
        } else if (!kSerialFill && p + 1 < nstep1) {
            sg.store(stage[(p + 1) & 1], xnext);
        }
        if (half == 0) xch[cg][slot] = tm;
        lds_barrier();
        const float mt = fmaxf(tm, xch[cg ^ 1][slot]);
        if (mt > m) {
            m = mt;
            last_inc = p;
            stale_row = stale_row || nz;
        }
        if (vis) {
            const uint32_t w = keep_bits(s, ct, m);
            if (half == 0) bits[ct][slot] = w;
            nz = nz || w != 0u;
        }
        lds_barrier();
        if (kSerialFill) {                               // fill only after every read of this step
            if (p + 1 < nstep1) sg.store(stage[(p + 1) & 1], xnext);
            lds_barrier();
        }
    };
    for (int p = 0; p < nstep1; p += 2) {
        step1(p, x1, x0);
        if (p + 1 < nstep1) step1(p + 1, x0, x1);
    }
    {
        const bool wave_stale = __ballot(rowOk && stale_row) != 0ull;   // all lanes vote
        if (lane == 0) wstale[wv] = wave_stale ? 1 : 0;
    }
    lds_barrier();
    int any_stale = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) any_stale |= wstale[i];

    if (any_stale) {
        // Tiles to score again: a word formed before its row's max last grew
        // that holds a bit.  Column group 0 of each row wave marks them; the
        // list is compacted in ascending order.
        auto stale = [&](int ct) {
            return rowOk && ((ntile - 1 - ct) >> 1) < last_inc && bits[ct][slot] != 0u;
        };
        if (cg == 0 && (wstale[2 * rw] | wstale[2 * rw + 1])) {
            for (int ct = 0; ct < ntile_w; ++ct)
                if (__ballot(stale(ct)) && lane == 0) atomicOr(&need[ct >> 5], 1u << (ct & 31));
        }
        lds_barrier();
        int nneed = 0;
#pragma unroll
        for (int i = 0; i < kMaxColTiles / 32; ++i) nneed += __popc(need[i]);
        if (tid < ntile) {
            const uint32_t word = need[tid >> 5], below = word & ((1u << (tid & 31)) - 1u);
            if ((word >> (tid & 31)) & 1u) {
                int pos = __popc(below);
                for (int i = 0; i < (tid >> 5); ++i) pos += __popc(need[i]);
                todo[pos] = tid;
            }
        }
        lds_barrier();
        auto todo_tile = [&](int i) { return i < nneed ? todo[i] : ntile; };
        sg.load(a.pk, krow0, todo_tile(sg.cg), ncol, x0);    // phase 2's first two steps
        sg.load(a.pk, krow0, todo_tile(2 + sg.cg), ncol, x1);

        // Phase 2: the listed tiles' words again, against the final max, for
        // the row waves that hold a stale word there.
        sweep((nneed + 1) >> 1, todo_tile, [&](int ct, const TileStage<D>& st) {
            if (__ballot(stale(ct))) {
                const f32x16 s = tile_scores<D>(qh, ql, st, rho, half);
                const uint32_t w = keep_bits(s, ct, m);
                if (half == 0) bits[ct][slot] = w;
            }
        });
    }

    // Phase 3: ordered compaction.  Four lanes per row slot (16 slots per
    // wave), each taking a consecutive quarter of the row's tiles: the lanes
    // count their bits, scan the counts across the four lanes, and write
    // their blocks from that offset, each tile's bits lowest first.
    {
        const int q4 = lane & 3;
        const int slot3 = wv * (kRowSlots / kWaves) + (lane >> 2);
        const int rw3 = slot3 / 32, r3 = slot3 % 32;
        const int ii = r3 / a.g, hi = r3 % a.g;
        const int I = rw_first(rw3) + ii;
        const bool live = r3 < rows && I < nb;
        const int nt = live ? I / 32 + 1 : 0;            // tiles holding J <= I
        const int per = (nt + 3) >> 2;
        const int c0 = min(nt, q4 * per), c1 = min(nt, c0 + per);
        auto word = [&](int ct) -> uint32_t {
            if (a.shared) {
                // Group-shared selection: the union of the g heads' keep bits
                // of this query block (row slots ii*g .. ii*g+g-1 of this row
                // wave); with group-pooled rows the g rows' bits are equal.
                uint32_t w = 0u;
                for (int j = 0; j < a.g; ++j) w |= bits[ct][32 * rw3 + ii * a.g + j];
                return w;
            }
            return bits[ct][slot3];
        };
        int cnt = 0;
        for (int ct = c0; ct < c1; ++ct) cnt += __popc(word(ct));
        int incl = cnt;
        int up = __shfl_up(incl, 1, 4);
        if (q4 >= 1) incl += up;
        up = __shfl_up(incl, 2, 4);
        if (q4 >= 2) incl += up;
        if (live) {
            const int h = hk * a.g + hi;
            int32_t* out = a.kv_idx + list_row(t, b, h, I, nb, first);
            int pos = incl - cnt;
            for (int ct = c0; ct < c1; ++ct) {
                uint32_t w = word(ct);
                while (w) {
                    out[pos++] = 32 * ct + __ffs(w) - 1;
                    w &= w - 1;
                }
            }
            if (q4 == 3) a.kv_cnt[count_index(t, a.Hq, b, h, I, nb, first)] = incl;
        }
    }
}

}  // namespace

hipError_t launch_select(const SelArgs& a, const SeqTable& t, hipStream_t s) {
    if (t.total_items == 0) return hipSuccess;
    dim3 grid(t.total_items * a.Hkv);
    if (a.D == 64)
        hipLaunchKernelGGL(k_select<64>, grid, dim3(kThreads), 0, s, a, t);
    else
        hipLaunchKernelGGL(k_select<128>, grid, dim3(kThreads), 0, s, a, t);
    return hipGetLastError();
}
