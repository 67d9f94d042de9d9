// Device-side helpers shared by the gfx950 kernels of libxattn.
//
// MFMA lane conventions used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   A (32 x 16, M x K): lane l holds row l%32, k-slots 8*(l/32) .. +8
//   B (16 x 32, K x N): lane l holds col l%32, k-slots 8*(l/32) .. +8
//   C (32 x 32 fp32)  : lane l holds col l%32; acc[4*i + j] is row 8*i + 4*(l/32) + j
// A and B name their k-slots the same way, so any k order the hardware uses
// internally cancels out of every product; only the C layout is relied on.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 128;  // BSA block (tokens)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Addressing of one K (or V) tensor: contiguous varlen or paged.
struct KvView {
  const char* base;            // byte pointer
  const int32_t* block_table;  // [batch, max_blocks] or nullptr
  const int32_t* cu_k;         // [batch+1] (contiguous layout)
  int max_blocks;
  int num_pages;  // paged: pages addressable from base; an entry outside [0, num_pages) is absent
  int kv_heads;
  int head_dim;
  int elem_bytes;
  int y_offset;  // contiguous layout: the array starts at key y_offset of the sequence

  // Byte address of key `y` (sequence-relative), kv head `g`, element 0.
  // Paged: returns nullptr when the page is unallocated (-1) or outside the
  // cache (an entry >= num_pages is never dereferenced).
  __device__ __forceinline__ const char* row(int b, int y, int g) const {
    const long long row_bytes = (long long)kv_heads * head_dim * elem_bytes;
    if (block_table) {
      const int page = block_table[(long long)b * max_blocks + (y >> 7)];
      if (page < 0 || page >= num_pages) return nullptr;
      return base + ((long long)page * kBlock + (y & (kBlock - 1))) * row_bytes +
             (long long)g * head_dim * elem_bytes;
    }
    return base + (long long)(cu_k[b] + y - y_offset) * row_bytes + (long long)g * head_dim * elem_bytes;
  }
};

__device__ __forceinline__ float wave_max_xor32(float v) {
  return fmaxf(v, __shfl_xor(v, 32, 64));
}

}  // namespace xattn
