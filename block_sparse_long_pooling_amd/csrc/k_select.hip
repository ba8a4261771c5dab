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
// same number of (row, column tile) products.  The k_bar rows stream through LDS in column tiles of 32
// blocks, two tiles per step (one per column group), split once per
// workgroup into bf16 hi + lo parts; every tile then serves all the rows of
// the workgroup.  The rows of the step after next are loaded into registers
// while the current step computes.  The (L/B)^2 score matrix is never stored: phase 1
// takes each row's max, phase 2 recomputes the same scores (same
// instruction sequence, bit-identical) into a keep bitmap in LDS, phase 3
// compacts it in ascending J.  The dot products run on bf16 MFMA with each
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

// Workgroup = up to 128 score rows (4 row waves x TI query blocks x g heads)
// of one KV head.  Wave wv: row wave rw = wv / 2, column group cg = wv % 2;
// each step stages two column tiles (phase 1: tiles 2p and 2p + 1 at step
// p), and column group cg scores the (cg)-th of them for its row wave's
// rows.  Phase 1: row maxima, combined over the
// column groups in LDS.  Phase 2: the same scores again, thresholded; each
// tile's keep bits go to an LDS bitmap [tile][row slot]; tiles whose phase-1
// maximum lies below every row's threshold are not scored again.  Phase 3:
// one lane per row slot writes the row's list in ascending J.
template <int D>
__global__ __launch_bounds__(kThreads, 1) void k_select(SelArgs a, SeqTable t) {
    __shared__ TileStage<D> stage[2][kColGroups];
    __shared__ uint32_t bits[kMaxColTiles][kRowSlots];
    __shared__ float pmax[kColGroups][kRowSlots];
    __shared__ uint32_t need[kMaxColTiles / 32];     // phase 2: tiles some row may keep from
    __shared__ int32_t todo[kMaxColTiles];           // ... in ascending order

    const int tid = threadIdx.x;
    const int wv = tid >> 6, lane = tid & 63;
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

    // This lane's query row rho = (query block Iw0 + rho / g, head hk*g + rho % g);
    // rows without a query block read the first one and are zeroed.  The
    // row is scaled by sigma before it is split.  With group-pooled lists
    // every row of a query block holds the sum of its g heads' rows, and the
    // scale takes the 1/g of their mean.
    const int rowI = Iw0 + rho / a.g;
    const bool rowOk = rho < rows && rowI < nb;
    const bool pooled = a.shared == 2;
    float4 qf[D / 8];
    {
        const int64_t qrow = qblock_row(t, b, rowOk ? rowI : first);
        const int h = hk * a.g + (pooled ? 0 : rho % a.g);
        const float4* src = reinterpret_cast<const float4*>(a.pq + ((int64_t)h * t.total_qblocks + qrow) * D + 8 * half);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            qf[2 * kk] = src[4 * kk];
            qf[2 * kk + 1] = src[4 * kk + 1];
        }
        if (pooled) {
            for (int j = 1; j < a.g; ++j) {
                src += (int64_t)t.total_qblocks * D / 4;       // head h + j
#pragma unroll
                for (int kk = 0; kk < D / 8; ++kk) {
                    const float4 x = src[4 * (kk / 2) + (kk & 1)];
                    qf[kk] = make_float4(qf[kk].x + x.x, qf[kk].y + x.y, qf[kk].z + x.z, qf[kk].w + x.w);
                }
            }
        }
    }
    // Two register buffers: the rows of step p + 2 load while step p scores.
    float4 x0[Stager<D>::F / 4], x1[Stager<D>::F / 4];
    sg.load(a.pk, krow0, sg.cg, ncol, x0);               // phase 1's first two steps
    sg.load(a.pk, krow0, 2 + sg.cg, ncol, x1);
    bf16x8 qh[D / 16], ql[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        const float sc = rowOk ? (pooled ? a.scale / (float)a.g : a.scale) : 0.f;
        const float4 u = qf[2 * kk], v = qf[2 * kk + 1];
        split8(make_float4(u.x * sc, u.y * sc, u.z * sc, u.w * sc), make_float4(v.x * sc, v.y * sc, v.z * sc, v.w * sc),
               qh[kk], ql[kk]);
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
            if (p + 1 < nstep) sg.store(stage[(p + 1) & 1], xnext);
            lds_barrier();
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
    // Between the phases the bitmap words hold the bits of each (tile, row)'s
    // score maximum (-inf for rows without a valid entry in the tile).

    // Phase 1: per tile, this row's max (both halves of the wave), kept in
    // tmax; then the row max over all tiles and both column groups.
    float m = -INFINITY;
    sweep((ntile + 1) >> 1, [](int i) { return i; }, [&](int ct, const TileStage<D>& st) {
        const f32x16 s = tile_scores<D>(qh, ql, st, rho, half);
        float tm = -INFINITY;
        if (masked(ct)) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (rowOk && 32 * ct + colJ(r) <= rowI) tm = fmaxf(tm, s[r]);
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) tm = fmaxf(tm, s[r]);
        }
        tm = fmaxf(tm, __shfl_xor(tm, 32));
        if (half == 0) bits[ct][32 * rw + rho] = __float_as_uint(tm);
        m = fmaxf(m, tm);
    });
    if (half == 0) pmax[cg][32 * rw + rho] = m;
    lds_barrier();
    m = pmax[0][32 * rw + rho];
#pragma unroll
    for (int c2 = 1; c2 < kColGroups; ++c2) m = fmaxf(m, pmax[c2][32 * rw + rho]);

    // Tiles to score again: those where some row's maximum reaches its
    // threshold (s <= tmax implies s - m <= tmax - m in floating point, so
    // no other tile keeps anything).  Column group 0 of each row wave marks
    // them; the list is compacted in ascending order and every other tile's
    // words are cleared.
    if (cg == 0) {
        for (int ct = 0; ct < ntile_w; ++ct) {
            const float tm = __uint_as_float(bits[ct][32 * rw + rho]);
            if (__ballot(rowOk && tm - m >= a.ln_alpha) && lane == 0) atomicOr(&need[ct >> 5], 1u << (ct & 31));
        }
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
    for (int e = tid; e < ntile * kRowSlots; e += kThreads) {
        const int ct = e / kRowSlots;
        if (!((need[ct >> 5] >> (ct & 31)) & 1u)) bits[ct][e % kRowSlots] = 0u;
    }
    lds_barrier();
    auto todo_tile = [&](int i) { return i < nneed ? todo[i] : ntile; };
    sg.load(a.pk, krow0, todo_tile(sg.cg), ncol, x0);    // phase 2's first two steps
    sg.load(a.pk, krow0, todo_tile(2 + sg.cg), ncol, x1);

    // Phase 2: keep bits per listed (tile, row slot); bit j of a word is
    // column block j of the tile.  Row waves whose rows keep nothing in the
    // tile skip the scores.  The two halves of the wave hold alternate groups
    // of 4 columns and are merged before the store.
    sweep((nneed + 1) >> 1, todo_tile, [&](int ct, const TileStage<D>& st) {
        const float tm = __uint_as_float(bits[ct][32 * rw + rho]);
        uint32_t w = 0u;
        if (__ballot(rowOk && tm - m >= a.ln_alpha)) {
            const f32x16 s = tile_scores<D>(qh, ql, st, rho, half);
            const bool mk = masked(ct);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                bool keep = s[r] - m >= a.ln_alpha;
                if (mk) keep = keep && rowOk && 32 * ct + colJ(r) <= rowI;
                w |= keep ? (1u << colJ(r)) : 0u;
            }
            w |= __shfl_xor(w, 32);
        }
        if (half == 0) bits[ct][32 * rw + rho] = w;
    });

    // Phase 3: ordered compaction, one row slot per lane (lanes 0..15 of
    // every wave): the row's tiles in ascending order, each tile's bits
    // lowest first.
    if (lane < kRowSlots / kWaves) {
        const int slot = wv * (kRowSlots / kWaves) + lane;
        const int rw3 = slot / 32, r3 = slot % 32;
        const int ii = r3 / a.g, hi = r3 % a.g;
        const int I = rw_first(rw3) + ii;
        if (r3 < rows && I < nb) {
            const int h = hk * a.g + hi;
            const int nt = I / 32 + 1;                       // tiles holding J <= I
            int32_t* out = a.kv_idx + list_row(t, b, h, I, nb, first);
            int pos = 0;
            for (int ct = 0; ct < nt; ++ct) {
                uint32_t w;
                if (a.shared) {
                    // Group-shared selection: the union of the g heads' keep bits
                    // of this query block (row slots ii*g .. ii*g+g-1 of this row
                    // wave); with group-pooled rows the g rows' bits are equal.
                    w = 0u;
                    for (int j = 0; j < a.g; ++j) w |= bits[ct][32 * rw3 + ii * a.g + j];
                } else {
                    w = bits[ct][slot];
                }
                while (w) {
                    out[pos++] = 32 * ct + __ffs(w) - 1;
                    w &= w - 1;
                }
            }
            a.kv_cnt[count_index(t, a.Hq, b, h, I, nb, first)] = pos;
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
