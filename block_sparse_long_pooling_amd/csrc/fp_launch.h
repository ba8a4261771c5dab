// Host-side launch interface between the C-ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp_device.h"

struct PoolArgs {
    const uint16_t* q;   // bf16 [T, Hq, d]
    const uint16_t* k;   // bf16 rows (contiguous or paged)
    const uint16_t* v;   // may be null (then not pooled)
    float* pq;           // [Hq, total_qblocks, d]
    float* pk;           // [Hkv, total_blocks, d]
    float* pv;           // [Hkv, total_blocks, d] or null
    uint16_t* pkv16;     // bf16 [2, Hkv, total_blocks, d] (K_bar then V_bar) or null
    float* pcache;       // fp32 [2, num_pages, Hkv, d] by the page of a block's first token, or null
    int32_t reuse;       // prefix blocks: read their means from pcache instead of pooling
    KVLayout kv;
    int32_t Hq, Hkv, D, B;
    int32_t q_stride;    // Q_bar averages the block's tokens 0, q_stride, 2 q_stride, ...
    int32_t q_chunks;    // Hq * d / 8
    int32_t k_chunks;    // Hkv * d / 8
    int32_t total_chunks;
    int32_t prefix_only; // K and V of prefix blocks only (the fused fp8 chunk pass pools the rest)
};

// A selection workgroup holds kSelectRowWaves row waves of 32 score rows, i.e.
// kSelectRowWaves * TI consecutive query blocks of one KV head.
constexpr int kSelectRowWaves = 4;
struct SelArgs {
    const float* pq;
    const float* pk;
    int32_t* kv_idx;
    int32_t* kv_cnt;
    int32_t Hq, Hkv, g, D, TI;   // TI query blocks x g heads per row wave (TI * g <= 32)
    float scale;                 // sigma
    float ln_alpha;              // threshold on s - max s (-inf keeps every causal block)
    int32_t shared;              // 1: the g heads of a query block share the union of their lists;
                                 // 2: they share the list of the mean of their q_bar rows
};

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* q_scale;        // fp8: [Hq, total_qblocks] (by qblock_row)
    const float* k_scale;        // fp8: [Hkv, total_blocks]
    const float* v_scale;
    const int32_t* kv_idx;
    const int32_t* kv_cnt;
    const uint16_t* pk16;        // bf16 pooled K_bar [Hkv, total_blocks, d] (correction)
    const uint16_t* pv16;        // bf16 pooled V_bar, same layout
    uint16_t* out;               // bf16 [T, Hq, d]
    float* lse;                  // [Hq, T] or null
    KVLayout kv;
    int32_t Hq, Hkv, g;
    float scale_log2;            // sigma * log2(e)
    int32_t correction;
};

// Fused fp8 quantization + pooling of one sequence (tensors 0, 1, 2 = Q, K, V).
constexpr float kE4M3Max = 448.f;
struct QuantArgs {
    const uint16_t* src[3];      // bf16 [T, H, d] packed rows; K and V may be pages [num_pages, page, Hkv, d]
    uint8_t* codes[3];           // e4m3 codes in the layout of src
    float* scale[3];             // fp32 [H, nB]; paged K and V: [num_pages, Hkv], entry of a block's first page
    float* pq;                   // fp32 Q_bar [Hq, nB, d] (by query-block row)
    float* pk;                   // fp32 K_bar [Hkv, total_blocks, d]
    uint16_t* pkv16;             // bf16 [2, Hkv, total_blocks, d] (K_bar then V_bar) or null
    float* pcache;               // chunk mode: fp32 [2, num_pages, Hkv, d] pooled cache (K/V means) or null
    KVLayout kv;                 // pages of K and V (used when paged)
    int32_t H[3];                // Hq, Hkv, Hkv
    int32_t groups[3];           // head groups per tensor (set by the launcher)
    int32_t D, B, nB;            // nB: blocks of all requests (chunk mode: query blocks)
    int32_t q_stride;            // Q_bar averages the block's tokens 0, q_stride, 2 q_stride, ...
};

hipError_t launch_pool(const PoolArgs& a, const SeqTable& t, bool paged, hipStream_t s);
// chunk: codes, scales and means of the query blocks of each request's chunk
// only (paged; nB = t.total_qblocks), K/V means also into a.pcache.
hipError_t launch_quant_pool(const QuantArgs& a, const SeqTable& t, bool paged, bool chunk, hipStream_t s);
hipError_t launch_select(const SelArgs& a, const SeqTable& t, hipStream_t s);
hipError_t launch_attn_bf16(const AttnArgs& a, const SeqTable& t, int D, int B, bool paged, hipStream_t s);
hipError_t launch_attn_fp8(const AttnArgs& a, const SeqTable& t, int D, int B, bool paged, hipStream_t s);
