// ja_block.h -- interface of the fused block-diagonal attention backward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ja {

// Tokens per tile of the block kernels: a block of at most this many tokens is
// one independent problem (or several, for smaller blocks, inside one tile).
constexpr int kBlkTile = 64;

struct BlkArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    const int32_t* off;    // [B+1] offsets shared by queries, keys and values
    const int32_t* items;  // (sequence, 64-token tile) pairs from the tile scheduler
    const int32_t* counters;
    int32_t cap;           // item capacity in (pair, head) units: H * pairs the list can hold
    int32_t B, H;
    int32_t T;             // tensor extent: rows outside [0, T) are never touched
    int32_t causal;
    int32_t bsh;           // log2 of the block size, at most log2(kBlkTile)
    float scale;
};

bool blk_supported(int dtype, int d, int bsh);
int blk_blocks_per_cu(int d);  // resident workgroups per CU
// Persistent grid: workgroup g takes (tile, head) items g, g + grid, ...
hipError_t launch_blk_bwd(const BlkArgs& a, int d, int grid, hipStream_t stream);

}  // namespace ja
