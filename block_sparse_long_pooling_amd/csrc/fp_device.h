// Device-side definitions shared by the flashprefill kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// Debug build (-DFP_SERIAL_DMA=1): every fill of an LDS tile buffer (DMA or
// register-staged) is issued only after every wave has finished reading the
// tile before it, so no fill overlaps compute.  The arithmetic and its order
// are unchanged, so results must equal the pipelined build's bit for bit; a
// difference would expose a fill racing with a read.
#ifndef FP_SERIAL_DMA
#define FP_SERIAL_DMA 0
#endif
constexpr bool kSerialFill = FP_SERIAL_DMA != 0;

#define FP_TABLE_MAX 128   // requests per call (kernel-argument tables)
#define FP_MAX_BLOCKS 8192 // query blocks per request (kept-block bitmap in LDS)

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;

// Requests of one launch and the order in which workgroups visit them.
// Request b has a context of kv_len tokens, counted in KV blocks from its
// start; its queries in this call are the last q_len of them (chunked
// prefill; q_len = kv_len for a whole prompt) and start on a block boundary,
// so query blocks are KV blocks first .. nb-1 with first = (kv_len-q_len)/B.
// Work items of request b are counted by the launch over its query blocks
// (query blocks, query block tiles, ...); sorted position s holds request
// order[s], longest context first, and its items start at rank item_off[s].
// Lists and counts are stored for query blocks only:
//   kv_idx row (h, I): idx_off[b] + h (tri(nb) - tri(first)) + tri(I) - tri(first)
//   kv_cnt (h, I):     Hq (blk_off[b] - pre_off[b]) + h (nb - first) + I - first
// with tri(n) = n (n + 1) / 2.  A single sequence is batch = 1, first = 0.
struct SeqTable {
    int64_t idx_off[FP_TABLE_MAX + 1];   // start of request b's kv_idx region
    int32_t tok_off[FP_TABLE_MAX + 1];   // query token offsets (cu_seqlens of the queries)
    int32_t blk_off[FP_TABLE_MAX + 1];   // cumulative KV blocks
    int32_t pre_off[FP_TABLE_MAX + 1];   // cumulative prefix blocks (KV blocks without queries)
    int32_t item_off[FP_TABLE_MAX + 1];
    alignas(4) int16_t order[FP_TABLE_MAX];
    alignas(4) int16_t tail[FP_TABLE_MAX];   // tokens in request b's last KV block (1 .. B)
    int32_t batch;
    int32_t total_tokens;                // query tokens
    int32_t total_blocks;                // KV blocks
    int32_t total_qblocks;               // query blocks (total_blocks - pre_off[batch])
    int32_t total_items;
};

__device__ __forceinline__ int seq_blocks(const SeqTable& t, int b) { return t.blk_off[b + 1] - t.blk_off[b]; }
__device__ __forceinline__ int first_block(const SeqTable& t, int b) { return t.pre_off[b + 1] - t.pre_off[b]; }
// Entry i of a 16-bit table read as part of an aligned 32-bit word: with a
// uniform index that is one scalar load of the kernel arguments (a 16-bit
// load would go through the vector memory path and its counter).
__device__ __forceinline__ int table16(const int16_t* tab, int i) {
    const int w = reinterpret_cast<const int32_t*>(tab)[i >> 1];
    return (i & 1) ? (w >> 16) : (int)(int16_t)w;
}
__device__ __forceinline__ int context_len(const SeqTable& t, int b, int B) {
    const int nb = seq_blocks(t, b);
    return nb > 0 ? (nb - 1) * B + table16(t.tail, b) : 0;
}
// Tokens of query block first_block(t, b) that precede the chunk (0 unless a
// chunk starts inside a block): chunk row 0 is position first * B + phase.
__device__ __forceinline__ int chunk_phase(const SeqTable& t, int b, int B) {
    const int qlen = t.tok_off[b + 1] - t.tok_off[b];
    return qlen > 0 ? context_len(t, b, B) - qlen - first_block(t, b) * B : 0;
}
__device__ __forceinline__ int64_t tri64(int n) { return (int64_t)n * (n + 1) / 2; }
// Start of the kv_idx row of (query head h, query block I); capacity I + 1.
__device__ __forceinline__ int64_t list_row(const SeqTable& t, int b, int h, int I, int nb, int first) {
    return t.idx_off[b] + (int64_t)h * (tri64(nb) - tri64(first)) + tri64(I) - tri64(first);
}
__device__ __forceinline__ int64_t count_index(const SeqTable& t, int Hq, int b, int h, int I, int nb, int first) {
    return (int64_t)Hq * (t.blk_off[b] - t.pre_off[b]) + (int64_t)h * (nb - first) + (I - first);
}
// Row of query block I of request b among all query blocks of the launch.
__device__ __forceinline__ int qblock_row(const SeqTable& t, int b, int I) { return t.blk_off[b] - t.pre_off[b + 1] + I; }
// Query block row r -> request (the last one whose rows start at or before r:
// requests without query blocks are passed over).
__device__ __forceinline__ int request_of_qblock(const SeqTable& t, int r) {
    int lo = 0, hi = t.batch - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (t.blk_off[mid] - t.pre_off[mid] <= r) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Rank (in visiting order) -> (request, item index counted from the request's
// last item, so that long rows go first).
__device__ __forceinline__ void item_of(const SeqTable& t, int rank, int& b, int& local) {
    int lo = 0, hi = t.batch - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (t.item_off[mid] <= rank) lo = mid; else hi = mid - 1;
    }
    b = table16(t.order, lo);
    local = rank - t.item_off[lo];
}

// Global query block -> request.
__device__ __forceinline__ int request_of_block(const SeqTable& t, int gb) {
    int lo = 0, hi = t.batch - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (t.blk_off[mid] <= gb) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair (round to nearest even; hardware convert).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Where the KV rows of a request live: contiguous [T, Hkv, d] or a page pool
// [num_pages * page_size, Hkv, d] addressed through a block table.
struct KVLayout {
    const int32_t* block_table;
    int32_t page_size;
    int32_t num_pages;
    int32_t max_pages;
    int32_t page_shift;          // log2(page_size): a page size divides the block size (64 or 128)
    // Page index and slot of a request's token tr >= 0 (a shift and a mask,
    // where a division by a run-time page size costs a few dozen instructions).
    __device__ __forceinline__ int page_of(int tr) const { return tr >> page_shift; }
    __device__ __forceinline__ int slot_of(int tr) const { return tr & (page_size - 1); }
};

// Row of token tr (0-based inside request b whose packed rows start at tok0);
// -1 when the page id is out of range.
template <bool PAGED>
__device__ __forceinline__ int64_t kv_row(const KVLayout& L, int b, int tok0, int tr) {
    if (!PAGED) return (int64_t)tok0 + tr;
    int page = L.block_table[(int64_t)b * L.max_pages + L.page_of(tr)];
    if ((unsigned)page >= (unsigned)L.num_pages) return -1;
    return ((int64_t)page << L.page_shift) + L.slot_of(tr);
}

// Head permutation that puts the query heads of one KV head on one XCD when
// workgroups are dispatched round-robin over 8 XCDs (slot = blockIdx % 8).
__device__ __forceinline__ int xcd_head(int slot, int Hq) {
    if (Hq % 8 != 0) return slot;
    return (slot % 8) * (Hq / 8) + slot / 8;
}
