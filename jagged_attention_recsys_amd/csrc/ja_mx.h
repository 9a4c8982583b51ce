// ja_mx.h -- interface of the MXFP8 kernels (quantizer and attention forward).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ja {

constexpr int kMxBlock = 32;   // tokens (and channels) per scale block
constexpr int kMxD = 128;      // head dim of the MXFP8 attention forward
constexpr int kMxBM = 128;     // query rows per work item
constexpr int kMxKT = 128;     // keys per stage (scheduler cost unit)

struct MxQuantArgs {
    const void* x;             // bf16 [T, H, d]
    const int32_t* off;        // [B+1]
    uint8_t* x8;               // [T, H, d] E4M3 codes
    uint8_t* scales;           // [blocks, H, d/32] E8M0
    int32_t* soff;             // [B+1] first block of each sequence (written)
    int32_t* blk_seq;          // [max_blocks] sequence of each block (workspace)
    int32_t B, H, d, T;
    int32_t max_blocks;
};
hipError_t launch_mx_quant(const MxQuantArgs& a, hipStream_t stream);

struct MxFwdArgs {
    const uint8_t* q8;
    const uint8_t* k8;
    const uint8_t* v8;
    const uint8_t* qs;         // [blocks, H, d/32] scales of Q, K, V
    const uint8_t* ks;
    const uint8_t* vs;
    const int32_t* q_soff;     // [B+1] first scale block of each sequence (K and V share k_soff)
    const int32_t* k_soff;
    void* out;                 // bf16 [Tq, H, d]
    float* lse;                // may be null
    const int32_t* q_off;
    const int32_t* k_off;
    const int32_t* items;      // (sequence, 128-row query tile) pairs
    int32_t* counters;
    int32_t H;
    int32_t Tq, Tk;
    int32_t causal, window;
    float scale;
};
hipError_t launch_mx_fwd(const MxFwdArgs& a, int grid, hipStream_t stream);
int mx_fwd_blocks_per_cu();

}  // namespace ja
