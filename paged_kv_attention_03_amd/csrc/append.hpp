// Slot-mapped append of this step's K/V rows into the page pool.
//
// Each new token's rows are written in place into the slot its scheduler
// chose: keys and values stay in fixed-size pages that per-request block
// tables locate, so a request grows by filling its pages, never by reshaping
// or copying a cache (vllm-metal v0.4.0 release post, "Replacing attention,
// reusing the rest").  One thread
// moves one 16-byte chunk of a K row and the matching chunk of the V row, so
// the kernel reads and writes exactly the bytes of the new rows, coalesced
// along head_dim.
#pragma once

#include "pkv_device.hpp"

namespace pkv {

struct AppendParams {
    const uint8_t* k_new;
    const uint8_t* v_new;
    uint8_t* k_pool;
    uint8_t* v_pool;
    const int64_t* slots;
    int64_t rows;           // num_tokens * num_kv_heads
    int num_kv_heads;
    int chunks_per_row;     // head_dim * elem_bytes / 16
    int block_size;
    int64_t num_slots;      // num_blocks * block_size
};

__global__ void __launch_bounds__(256) append_kernel(AppendParams p) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t row = gid / p.chunks_per_row;
    if (row >= p.rows) return;
    const int c = (int)(gid - row * p.chunks_per_row);
    const int64_t t = row / p.num_kv_heads;
    const int h = (int)(row - t * p.num_kv_heads);
    const int64_t slot = p.slots[t];
    if (slot < 0 || slot >= p.num_slots) return;
    const int64_t blk = slot / p.block_size;
    const int64_t off = slot - blk * p.block_size;
    const int64_t rb = (int64_t)p.chunks_per_row * 16;
    const int64_t dst = ((blk * p.num_kv_heads + h) * p.block_size + off) * rb + c * 16;
    const int64_t src = row * rb + c * 16;
    st16(p.k_pool + dst, ld16(p.k_new + src));
    st16(p.v_pool + dst, ld16(p.v_new + src));
}

// Whole-page copies inside the pool (K and V, every kv head): the private
// copy a sequence takes of a shared page before writing into it.  One thread
// moves one 16-byte chunk of the K page and the same chunk of the V page;
// pairs naming a page outside the pool are skipped.
struct CopyBlocksParams {
    uint8_t* k_pool;
    uint8_t* v_pool;
    const int32_t* src;
    const int32_t* dst;
    int64_t num_pairs;
    int64_t chunks_per_block;  // num_kv_heads * block_size * head_dim * elem_bytes / 16
    int64_t num_blocks;
};

__global__ void __launch_bounds__(256) copy_blocks_kernel(CopyBlocksParams p) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t i = gid / p.chunks_per_block;
    if (i >= p.num_pairs) return;
    const int64_t c = gid - i * p.chunks_per_block;
    const int64_t s = p.src[i], d = p.dst[i];
    if (s < 0 || s >= p.num_blocks || d < 0 || d >= p.num_blocks) return;
    const int64_t bb = p.chunks_per_block * 16;
    st16(p.k_pool + d * bb + c * 16, ld16(p.k_pool + s * bb + c * 16));
    st16(p.v_pool + d * bb + c * 16, ld16(p.v_pool + s * bb + c * 16));
}

}  // namespace pkv
