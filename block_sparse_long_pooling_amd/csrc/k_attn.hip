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
// Rows past a request's end re-read its last row (contiguous layout) or a
// zero chunk (paged layout, also for out-of-range pages); the causal mask
// of the diagonal tile removes them.
//
// Mean correction: after the kept tiles, the bf16 pooled K_bar / V_bar rows
// of blocks c0 .. c0+BLK-1 form one more tile per BLK blocks, fetched through
// the same DMA pipeline, with logit sigma*q.k_bar_J + ln n_J, masked per
// head to its skipped J < I.
// Query heads of one KV head are placed on one XCD so their tiles meet in
// that XCD's L2.
#include "attn_walk.h"

namespace {
using namespace fp_walk;


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
    DmaPlan<D, BLK, G::NT> plan;
    const uint4* zero = &kZeroChunk;
    const int wave_base = __builtin_amdgcn_readfirstlane(64 * w * 16);
    constexpr int NLOAD = DmaPlan<D, BLK, G::NT>::NLOAD;
    // A kept tile's DMAs; K and V rows share their pages: one set of page
    // ids (paged layout) for both.
    auto issue_kept = [&](const It& itm, int code, char* kdst, char* vdst, const int* pg) {
        issue_tile<D, BLK, G::NT, PAGED>(itm.kfirst, pg, a.kv, rs, code, itm.len - code * BLK, plan, zero, kdst,
                                      wave_base);
        issue_tile<D, BLK, G::NT, PAGED>(itm.vfirst, pg, a.kv, rs, code, itm.len - code * BLK, plan, zero, vdst,
                                      wave_base);
    };
    auto issue = [&](const It& itm, int code, char* kdst, char* vdst) {
        if (code < kCorr) {
            int pg[NLOAD];
            if (PAGED) load_tile_pages(itm.pages, a.kv, code, itm.len - code * BLK, plan, pg);
            issue_kept(itm, code, kdst, vdst, pg);
        } else {
            // Pooled rows of this request's blocks for the KV head (contiguous, row stride D).
            const int ct = code - kCorr;
            const int64_t prow = ((int64_t)itm.hk * t.total_blocks + t.blk_off[itm.b]) * D;
            issue_tile<D, BLK, G::NT, false>(a.pk16 + prow, nullptr, a.kv, D, ct, itm.I - ct * BLK, plan, zero, kdst,
                                          wave_base);
            issue_tile<D, BLK, G::NT, false>(a.pv16 + prow, nullptr, a.kv, D, ct, itm.I - ct * BLK, plan, zero, vdst,
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
    // Rows past the end of a ragged last block (or before the start of a
    // chunk) re-read the nearest valid row: their outputs are never stored,
    // and unconditional loads keep the compiler from waiting on them (and on
    // DMAs issued before) when the registers are written.
    auto load_q = [&](const It& itm) {
        const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                             ((int64_t)(itm.q0 + min(max(qr, itm.lo), itm.nI - 1)) * a.Hq + itm.h) * D + 8 * half;
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
    // Paged layout: the walk runs one tile further ahead.  Jn, the tile
    // after J, is known a step before its DMA, and the page ids of its rows
    // (pgn) are loaded then, so a step issues its DMA right after the
    // barrier instead of first waiting on the block table.
    int Jn = INT_MAX, actn = 0;
    int pgn[NLOAD];
    auto ahead = [&](It& itm) {
        Jn = next_tile(itm, actn);
        if (Jn < kCorr) load_tile_pages(itm.pages, a.kv, Jn, itm.len - Jn * BLK, plan, pgn);
    };
    if (PAGED && J != INT_MAX) ahead(cur);
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
        int Jn1;
        auto prefetch = [&]() {
            if (PAGED) {
                Jn1 = Jn;
                act_next = actn;
                if (Jn1 < kCorr)
                    issue_kept(cur, Jn1, knext, vnext, pgn);
                else if (Jn1 != INT_MAX)
                    issue(cur, Jn1, knext, vnext);
                if (Jn1 != INT_MAX) ahead(cur);
            } else {
                Jn1 = next_tile(cur, act_next);
                if (Jn1 != INT_MAX) issue(cur, Jn1, knext, vnext);
            }
        };
        if (!kSerialFill) prefetch();
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
        if (kSerialFill) {
            lds_barrier();                               // every wave is done with tile J
            prefetch();
        }
        J = Jn1;
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
            if (!kSerialFill && Jn0 != INT_MAX) issue(nxt, Jn0, kb1, vb1);
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
        if (PAGED && has_next) ahead(nxt);
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
            for (int i = cur.lo * G::NCH + ht; i < cur.nI * G::NCH; i += 64 * G::WPH) {
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
        if (a.lse && half == 0 && qr >= cur.lo && qr < cur.nI)
            a.lse[(int64_t)cur.h * t.total_tokens + cur.q0 + qr] = (m + __log2f(l_tot)) * kLn2;
        if (kSerialFill) {
            lds_barrier();                               // the staged rows are read
            if (has_next && Jn0 != INT_MAX) issue(nxt, Jn0, kb1, vb1);
        }
        if (!has_next) break;
        cur = nxt;
        idx = nidx;
        ++band;
        J = Jn0;
        act = actn0;
    }
}

template <int D, int BLK, int HP>
int grid_t(const AttnArgs& a, const SeqTable& t, bool paged) {
    const int nitems = t.total_items * (a.Hq / HP);
    const int block = 64 * HP * (BLK / 32);
    return paged ? persistent_grid(k_attn_bf16<D, BLK, HP, true>, block, nitems)
                 : persistent_grid(k_attn_bf16<D, BLK, HP, false>, block, nitems);
}

template <int D, int BLK, int HP>
hipError_t launch_t(const AttnArgs& a, const SeqTable& t, bool paged, hipStream_t s) {
    const int block = 64 * HP * (BLK / 32);
    const dim3 grid(grid_t<D, BLK, HP>(a, t, paged));
    if (paged)
        hipLaunchKernelGGL((k_attn_bf16<D, BLK, HP, true>), grid, dim3(block), 0, s, a, t);
    else
        hipLaunchKernelGGL((k_attn_bf16<D, BLK, HP, false>), grid, dim3(block), 0, s, a, t);
    return hipGetLastError();
}

template <int D, int BLK>
hipError_t launch_db(const AttnArgs& a, const SeqTable& t, bool paged, hipStream_t s) {
    return (a.g % 2 == 0) ? launch_t<D, BLK, 2>(a, t, paged, s) : launch_t<D, BLK, 1>(a, t, paged, s);
}

template <int D, int BLK>
int grid_db(const AttnArgs& a, const SeqTable& t, bool paged) {
    return (a.g % 2 == 0) ? grid_t<D, BLK, 2>(a, t, paged) : grid_t<D, BLK, 1>(a, t, paged);
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

int attn_bf16_grid(const AttnArgs& a, const SeqTable& t, int D, int B, bool paged) {
    if (t.total_items == 0) return 0;
    if (D == 128 && B == 128) return grid_db<128, 128>(a, t, paged);
    if (D == 128 && B == 64) return grid_db<128, 64>(a, t, paged);
    if (D == 64 && B == 128) return grid_db<64, 128>(a, t, paged);
    if (D == 64 && B == 64) return grid_db<64, 64>(a, t, paged);
    return -1;
}
