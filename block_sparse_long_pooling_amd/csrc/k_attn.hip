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
// LDS chunk i*NT + tid, i.e. row row[i], logical chunk (chunk position XOR
// swizzle).  off[i] is that chunk's element offset inside the tile's rows for
// contiguous K/V (row * row_stride + kv head * D + chunk * 8).
template <int D, int BLK, int HP>
struct DmaPlan {
    static constexpr int NLOAD = BLK * (D / 8) / (64 * HP * (BLK / 32));
    int row[NLOAD];
    int coff[NLOAD];   // element offset inside one token row: hk * D + chunk * 8
    __device__ __forceinline__ void init(int tid, int hk) {
        constexpr int NT = 64 * HP * (BLK / 32);
        constexpr int NCH = D / 8;
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            const int p = i * NT + tid;
            row[i] = p / NCH;
            coff[i] = hk * D + ((p % NCH) ^ swz<D>(row[i])) * 8;
        }
    }
};

// DMA one tile: rows J*BLK .. of the request whose first row is `first`
// (contiguous) or whose pages are listed in `pages` (paged).
template <int D, int BLK, int HP, bool PAGED>
__device__ __forceinline__ void issue_tile(const uint16_t* first, const int32_t* pages, const KVLayout& L,
                                           int64_t rs, int J, int nvalid, const DmaPlan<D, BLK, HP>& plan,
                                           const uint4* zero, char* lds, int wave_base) {
    using G = Geo<D, BLK, HP>;
    static_assert((BLK * G::NCH) % G::NT == 0, "tile chunks must split evenly");
#pragma unroll
    for (int i = 0; i < DmaPlan<D, BLK, HP>::NLOAD; ++i) {
        const int row = plan.row[i];
        const void* src;
        if (!PAGED) {
            const uint16_t* p = first + ((int64_t)J * BLK + row) * rs + plan.coff[i];
            src = row < nvalid ? (const void*)p : (const void*)zero;
        } else {
            const int tr = J * BLK + row;
            const int page = pages[tr / L.page_size];
            const uint16_t* p = first + ((int64_t)page * L.page_size + tr % L.page_size) * rs + plan.coff[i];
            src = (row < nvalid && (unsigned)page < (unsigned)L.num_pages) ? (const void*)p : (const void*)zero;
        }
        __builtin_amdgcn_global_load_lds(src, (lds_void*)(lds + (i * G::NT) * 16 + wave_base), 16, 0, 0);
    }
}

// Pooled rows c0 .. c0+BLK-1 (zero for blocks >= I) as bf16 into a tile buffer.
template <int D, int BLK, int HP>
__device__ __forceinline__ void store_pooled_tile(const float* src, int64_t prow0, int c0, int I, uint4* tile,
                                                  int tid) {
    using G = Geo<D, BLK, HP>;
    for (int i = tid; i < BLK * G::NCH; i += G::NT) {
        const int row = i / G::NCH, c = i % G::NCH;
        const int J = c0 + row;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (J < I) {
            const float4* s = reinterpret_cast<const float4*>(src + (prow0 + J) * D + c * 8);
            v = f32x8_to_bf16(s[0], s[1]);
        }
        tile[row * G::NCH + (c ^ swz<D>(row))] = v;
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
    int pos[HP];
    __device__ __forceinline__ int head(int h) const { return pos[h] < cnt[h] ? list[h][pos[h]] : INT_MAX; }
    // Next block of the union and the heads that keep it (bit mask); INT_MAX when done.
    __device__ __forceinline__ int next(int& act) {
        int J = INT_MAX;
#pragma unroll
        for (int h = 0; h < HP; ++h) J = min(J, head(h));
        act = 0;
#pragma unroll
        for (int h = 0; h < HP; ++h)
            if (J != INT_MAX && head(h) == J) { act |= 1 << h; ++pos[h]; }
        return J;
    }
};

template <int D, int BLK, int HP, bool PAGED>
__global__ __launch_bounds__(64 * HP * (BLK / 32)) void k_attn_bf16(AttnArgs a, SeqTable t) {
    using G = Geo<D, BLK, HP>;
    // Four separate LDS objects: the compiler then sees that a DMA into one
    // buffer does not touch the buffer being read, and does not wait on it.
    __shared__ __attribute__((aligned(16))) char kb0[G::TILE];
    __shared__ __attribute__((aligned(16))) char kb1[G::TILE];
    __shared__ __attribute__((aligned(16))) char vb0[G::TILE];
    __shared__ __attribute__((aligned(16))) char vb1[G::TILE];
    __shared__ uint32_t kept_bits[HP][FP_MAX_BLOCKS / 32];

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
    const int hs = w / G::WPH;                   // which of the HP heads this wave serves
    const int rw = w % G::WPH;                   // 32-row group inside the query block
    const int npairs = a.Hq / HP;
    const int rank = blockIdx.x / npairs;
    const int h = HP * xcd_head(blockIdx.x % npairs, npairs) + hs;
    int b, local;
    item_of(t, rank, b, local);
    const int nb = seq_blocks(t, b);
    const int I = nb - 1 - local;
    const int tok0 = t.tok_off[b];
    const int len = t.tok_off[b + 1] - tok0;
    const int q0 = tok0 + I * BLK;
    const int nI = min(BLK, len - I * BLK);
    const int hk = h / a.g;
    const int64_t rs = (int64_t)a.Hkv * D;
    const int64_t tri = (int64_t)nb * (nb + 1) / 2;
    const int h0 = h - hs;

    Union<HP> u;
#pragma unroll
    for (int j = 0; j < HP; ++j) {
        u.list[j] = a.kv_idx + t.idx_off[b] + (int64_t)(h0 + j) * tri + (int64_t)I * (I + 1) / 2;
        u.cnt[j] = a.kv_cnt[(int64_t)a.Hq * t.blk_off[b] + (int64_t)(h0 + j) * nb + I];
        u.pos[j] = 0;
    }
    const int qr = 32 * rw + col;
    // Tile DMA: contiguous K/V start at this request's first row; paged K/V
    // start at the pool and go through the request's block-table row.
    const uint16_t* kfirst = static_cast<const uint16_t*>(a.k) + (PAGED ? 0 : (int64_t)tok0 * rs);
    const uint16_t* vfirst = static_cast<const uint16_t*>(a.v) + (PAGED ? 0 : (int64_t)tok0 * rs);
    const int32_t* pages = PAGED ? a.kv.block_table + (int64_t)b * a.kv.max_pages : nullptr;
    DmaPlan<D, BLK, HP> plan;
    plan.init(tid, hk);
    const uint4* zero = &kZeroChunk;
    const int wave_base = __builtin_amdgcn_readfirstlane(64 * w * 16);

    bf16x8 qf[D / 16];
    {
        const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((int64_t)(q0 + qr) * a.Hq + h) * D + 8 * half;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (qr < nI) x = *reinterpret_cast<const uint4*>(qp + 16 * kk);
            qf[kk] = __builtin_bit_cast(bf16x8, x);
        }
    }
    const float c = a.scale_log2;
    float m = -INFINITY, l = 0.f;
    f32x16 o[G::NDS];
#pragma unroll
    for (int ds = 0; ds < G::NDS; ++ds) o[ds] = f32x16{};
    constexpr int SH = G::NSUB > 1 ? G::NSUB / 2 : 1;   // subtiles per half tile
    f32x16 s[SH];
    uint32_t pk[SH][8];

    int act, act_next;
    int J = u.next(act);
    if (J != INT_MAX) {
        issue_tile<D, BLK, HP, PAGED>(kfirst, pages, a.kv, rs, J, len - J * BLK, plan, zero, kb0, wave_base);
        issue_tile<D, BLK, HP, PAGED>(vfirst, pages, a.kv, rs, J, len - J * BLK, plan, zero, vb0, wave_base);
    }
    // One kept tile: wait for its DMA, release the other buffers by the
    // barrier, prefetch the next tile into them, compute on this one.
    auto step = [&](char* kcur, char* vcur, char* knext, char* vnext) {
        const int Jn = u.next(act_next);
        __builtin_amdgcn_s_waitcnt(0);                   // this thread's DMA for tile J is done
        __syncthreads();                                 // ... every thread's; the other buffers are free
        if (Jn != INT_MAX) {
            issue_tile<D, BLK, HP, PAGED>(kfirst, pages, a.kv, rs, Jn, len - Jn * BLK, plan, zero, knext,
                                          wave_base);
            issue_tile<D, BLK, HP, PAGED>(vfirst, pages, a.kv, rs, Jn, len - Jn * BLK, plan, zero, vnext,
                                          wave_base);
        }
        if ((act >> hs) & 1) {
            // Two halves of SH subtiles each: online softmax per half keeps S and
            // P at half size, which leaves registers to read operands ahead.
            auto half_tile = [&](auto sub0) {
                constexpr int S0 = decltype(sub0)::value;
                qk<D, BLK, HP, S0, SH>(reinterpret_cast<const uint4*>(kcur), qf, col, half, s);
                if (J == I) {
#pragma unroll
                    for (int j = 0; j < SH; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = 32 * (S0 + j) + (r & 3) + 8 * (r >> 2) + 4 * half;
                            s[j][r] = key > qr ? -INFINITY : s[j][r];
                        }
                }
                softmax_update<SH, G::NDS>(s, c, 0.f, m, l, o, pk);
                pv<D, BLK, HP, S0, SH>(vcur, pk, lane, o);
            };
            half_tile(std::integral_constant<int, 0>());
            if (G::NSUB > SH) half_tile(std::integral_constant<int, (G::NSUB > SH ? SH : 0)>());
        }
        J = Jn;
        act = act_next;
    };
    while (J != INT_MAX) {
        step(kb0, vb0, kb1, vb1);
        if (J == INT_MAX) break;
        step(kb1, vb1, kb0, vb0);
    }

    if (a.correction && I > 0) {
        const int nwords = (I + 31) >> 5;
        __syncthreads();                                 // last tile's reads are done
        for (int i = tid; i < HP * nwords; i += G::NT) kept_bits[i / nwords][i % nwords] = 0u;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < HP; ++j)
            for (int i = tid; i < u.cnt[j]; i += G::NT) {
                const int Jk = u.list[j][i];
                if (Jk < I) atomicOr(&kept_bits[j][Jk >> 5], 1u << (Jk & 31));
            }
        __syncthreads();
        const int64_t prow0 = (int64_t)hk * t.total_blocks + t.blk_off[b];
        const float log2_blk = __log2f((float)BLK);      // past blocks are full: ln n_J = ln BLK
        for (int c0 = 0; c0 < I; c0 += BLK) {
            // Bit j of skip[sub] <=> block c0 + 32 sub + j is strictly past and not kept by this head.
            uint32_t skip[G::NSUB];
            int nskip = 0, nany = 0;
#pragma unroll
            for (int sub = 0; sub < G::NSUB; ++sub) {
                const int j0 = c0 + 32 * sub;
                const int nvalid = min(32, max(0, I - j0));
                const uint32_t valid = nvalid >= 32 ? 0xffffffffu : ((1u << nvalid) - 1u);
                skip[sub] = ~kept_bits[hs][j0 >> 5] & valid;
                nskip += __popc(skip[sub]);
#pragma unroll
                for (int j = 0; j < HP; ++j) nany += __popc(~kept_bits[j][j0 >> 5] & valid);
            }
            if (nany == 0) continue;                     // every head keeps every past block here
            __syncthreads();
            store_pooled_tile<D, BLK, HP>(a.pk, prow0, c0, I, reinterpret_cast<uint4*>(kb0), tid);
            store_pooled_tile<D, BLK, HP>(a.pv, prow0, c0, I, reinterpret_cast<uint4*>(vb0), tid);
            __syncthreads();
            if (nskip == 0) continue;
            auto corr_half = [&](auto sub0) {
                constexpr int S0 = decltype(sub0)::value;
                qk<D, BLK, HP, S0, SH>(reinterpret_cast<const uint4*>(kb0), qf, col, half, s);
#pragma unroll
                for (int j = 0; j < SH; ++j) {
                    const uint32_t bits = skip[S0 + j] >> (4 * half);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        s[j][r] = ((bits >> ((r & 3) + 8 * (r >> 2))) & 1u) ? s[j][r] : -INFINITY;
                }
                softmax_update<SH, G::NDS>(s, c, log2_blk, m, l, o, pk);
                pv<D, BLK, HP, S0, SH>(vb0, pk, lane, o);
            };
            corr_half(std::integral_constant<int, 0>());
            if (G::NSUB > SH) corr_half(std::integral_constant<int, (G::NSUB > SH ? SH : 0)>());
        }
    }

    // Epilogue: normalise, stage each head's bf16 tile in LDS, store full rows.
    const float l_tot = l + __shfl_xor(l, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    __syncthreads();
    uint4* stage = reinterpret_cast<uint4*>(hs == 0 ? kb0 : kb1);
#pragma unroll
    for (int ds = 0; ds < G::NDS; ++ds)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int chunk = 4 * ds + g4;               // d0 = 32 ds + 8 g4 + 4 half
            const uint2 v2 = make_uint2(pack_bf16(o[ds][4 * g4] * inv, o[ds][4 * g4 + 1] * inv),
                                        pack_bf16(o[ds][4 * g4 + 2] * inv, o[ds][4 * g4 + 3] * inv));
            reinterpret_cast<uint2*>(&stage[qr * G::NCH + (chunk ^ swz<D>(qr))])[half] = v2;
        }
    __syncthreads();
    const int ht = tid % (64 * G::WPH);                  // thread index within this head's waves
    for (int i = ht; i < nI * G::NCH; i += 64 * G::WPH) {
        const int row = i / G::NCH, ch = i % G::NCH;
        *reinterpret_cast<uint4*>(a.out + ((int64_t)(q0 + row) * a.Hq + h) * D + ch * 8) =
            stage[row * G::NCH + (ch ^ swz<D>(row))];
    }
    if (a.lse && half == 0 && qr < nI)
        a.lse[(int64_t)h * t.total_tokens + q0 + qr] = (m + __log2f(l_tot)) * kLn2;
}

template <int D, int BLK, int HP>
hipError_t launch_t(const AttnArgs& a, const SeqTable& t, bool paged, hipStream_t s) {
    dim3 grid((unsigned)t.total_items * (a.Hq / HP));
    dim3 block(64 * HP * (BLK / 32));
    if (paged)
        hipLaunchKernelGGL((k_attn_bf16<D, BLK, HP, true>), grid, block, 0, s, a, t);
    else
        hipLaunchKernelGGL((k_attn_bf16<D, BLK, HP, false>), grid, block, 0, s, a, t);
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
