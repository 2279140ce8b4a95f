// LDS tile layout and score scaling shared by the attention forward and backward kernels,
// so that both stage 64 x 64 bf16 tiles the same way and form bitwise the same scaled
// queries.
#pragma once

#include "rope_math.h"

namespace lcv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kTileBytes = 64 * 128;   // one 64 x 64 bf16 tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Softmax scale 1/sqrt(64) and the change to base 2, carried by the queries into the matrix
// cores: a score of Q' = bf16(Q * log2(e)/8) against K is in log2 units.
constexpr float kScoreToLog2 = kLog2e / 8.0f;

// Byte offset of 16-byte chunk `chunk` of row `row` in a 64 x 64 bf16 tile; chunks are
// XOR-swizzled by swz(row).  The LDS serves 256 bytes (64 banks of 4) per cycle, the 16-byte
// reads of 16 lanes: for one chunk in 16 consecutive rows, the 8 even rows and the 8 odd
// rows (128 bytes further on) must each take 8 distinct chunk slots, so swz is a permutation
// of 0..7 on the even and on the odd rows of every aligned group of 16 rows (a swizzle that
// repeats every 8 rows conflicts two ways on these reads).  The transposing 8-byte reads (a
// chunk pair of 4 consecutive rows per 16 lanes) stay conflict-free: bit 2 of
// swz(r) ^ swz(r + 2) is set on every aligned group of 4 rows.
__device__ __forceinline__ int swz(int row) {
  return (((row & 3) << 1) | ((row >> 2) & 1)) ^ (((row >> 3) & 1) << 1);
}
__device__ __forceinline__ uint32_t tile_off(int row, int chunk) {
  return (uint32_t)(row * 128 + ((chunk ^ swz(row)) << 4));
}

// Raw buffer resource (no stride, 32-bit data format) over `bytes` bytes from the byte address
// `base`, both wave-uniform: buffer loads at offsets past `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(uint64_t base, int bytes) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  bytes = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), 0, bytes, 0x00020000);
}

// 8 bf16 channels -> bf16(value * log2(e)/8), each product in fp32 and rounded to nearest
// even: the forward's query operand, and the backward's (from the same bits, the same
// bits out).
__device__ __forceinline__ u32x4 scale_chunk_log2(u32x4 raw) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = __uint_as_float(raw[e] << 16) * kScoreToLog2;
    const float b = __uint_as_float(raw[e] & 0xffff0000u) * kScoreToLog2;
    raw[e] = pack_bf16x2(a, b);
  }
  return raw;
}

}  // namespace lcv
