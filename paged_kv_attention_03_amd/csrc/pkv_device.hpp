// Device helpers shared by the paged-KV kernels (gfx950, wave64).
//
// Matrix-core conventions used throughout (16x16 output tiles):
//   v_mfma_f32_16x16x32_bf16 : A[16][32], B[32][16] bf16 -> C[16][16] f32
//   v_mfma_f32_16x16x4_f32   : A[16][4],  B[4][16]  f32  -> C[16][16] f32
// Lane l holds A row (l % 16), B column (l % 16), and the k-slots of group
// (l / 16): 8 consecutive slots for bf16, one slot for f32.  The result tile
// gives lane l rows 4*(l/16) .. 4*(l/16)+3 of column (l % 16).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kPage = 16;  // tokens per KV page (block_size)

// Floats per (token, query head) softmax state of a shared-prefix pass:
// unnormalised output [D], running max (log2 units of the scaled logits), sum,
// and two of padding (rows stay 16-byte aligned).
template <int D>
constexpr int kStateStride = D + 4;

struct bf16_t {};  // tag type for bfloat16 storage (raw 16-bit patterns)

template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kBytes = 4;
    static constexpr int kPerChunk = 4;  // elements per 16-byte chunk
};
template <> struct Elem<bf16_t> {
    static constexpr int kBytes = 2;
    static constexpr int kPerChunk = 8;
};

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Two floats -> packed bf16 pair (round to nearest even), low half first.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Buffer resource over `bytes` bytes from base (raw, stride 0; loads past
// the end read zero).  Word 3 selects the 32-bit data format that untyped
// buffer loads on CDNA expect.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// 16-byte buffer load at byte offset off; NT sets the non-temporal hint (the
// data is streamed past the caches instead of displacing reused lines), an
// immediate of the instruction.
template <bool NT>
__device__ __forceinline__ u32x4 buffer_ld16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, NT ? 2 : 0);
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, const u32x4& v) {
    *reinterpret_cast<u32x4*>(p) = v;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// Transposing LDS read: within each 16-lane group, lane i receives element
// (i % 4) of the 4 consecutive 16-bit values that lane 4r + i / 4 points at,
// for r = 0..3 (so 16 lanes pointing at a 4 x 16 block of 16-bit values, 4
// lanes per row, receive its 16 columns).
__device__ __forceinline__ uint2 lds_read_tr16(const uint8_t* addr) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)addr);
    return __builtin_bit_cast(uint2, v);
}

// Max / sum over the four lanes that share a column (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float col_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}
__device__ __forceinline__ float col_sum(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// Keys a sequence attends to, with every device-side value clamped to the
// host bounds so that no index can leave the buffers.
struct SeqRange {
    int L;      // keys (clamped)
    int a;      // first visible key (clamped to [0, L])
    int first_page, end_page;  // pages [first_page, end_page) hold keys [a, L)
};

__device__ __forceinline__ SeqRange seq_range(const int32_t* seq_lens, const int32_t* kv_start,
                                              int s, int max_seqlen_k, int max_blocks) {
    SeqRange r;
    int L = seq_lens[s];
    int cap = min(max_seqlen_k, max_blocks * kPage);
    L = L < 0 ? 0 : (L > cap ? cap : L);
    int a = kv_start ? kv_start[s] : 0;
    a = a < 0 ? 0 : (a > L ? L : a);
    r.L = L;
    r.a = a;
    r.first_page = a / kPage;
    r.end_page = (L + kPage - 1) / kPage;
    return r;
}

__device__ __forceinline__ int64_t safe_block(const int32_t* row, int page, int64_t num_blocks) {
    int64_t b = row[page];
    return (b >= 0 && b < num_blocks) ? b : 0;
}

}  // namespace pkv
