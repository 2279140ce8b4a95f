// Partitioned 3D rotary embedding arithmetic shared by the standalone RoPE pass and the
// RoPE fused into the attention kernel's Q/K loads, so both produce identical bits.
//
// A 64-channel head splits into sections [0,16) turning with the frame index t,
// [16,40) with the row y and [40,64) with the column x of the latent token; adjacent
// channels (2p, 2p+1) of a section of width d form one complex number turned by the angle
// pos * theta^(-2p/d) (longcat-video-rs page, section 03 "Partitioned 3D-RoPE
// (16T+24H+24W)").
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace lcv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// cos and sin of pos * theta^(-2p/width), fp32.
__device__ __forceinline__ float2 rope_cos_sin(int32_t pos, int32_t p, int32_t width, float log2_theta) {
  const float freq = exp2f(-(2.0f * (float)p / (float)width) * log2_theta);
  const float ang = (float)pos * freq;
  float s, c;
  sincosf(ang, &s, &c);
  return make_float2(c, s);
}

// Round two fp32 values to a packed bf16 pair (round to nearest even), low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Turn one packed bf16 channel pair (low half = channel 2p, high half = 2p+1).
__device__ __forceinline__ uint32_t rotate_pair(uint32_t w, float2 cs) {
  const float a = __uint_as_float(w << 16);
  const float b = __uint_as_float(w & 0xffff0000u);
  const float ra = fmaf(a, cs.x, -(b * cs.y));
  const float rb = fmaf(a, cs.y, b * cs.x);
  return pack_bf16x2(ra, rb);
}

// Section of the 8-channel chunk c = 0..7 (channels [8c, 8c+8)): axis (0 t, 1 y, 2 x),
// section width and the pair index of its first pair inside the section.
__device__ __forceinline__ void chunk_section(int c, int& axis, int& width, int& p0) {
  if (c < 2) {
    axis = 0; width = 16; p0 = 4 * c;
  } else if (c < 5) {
    axis = 1; width = 24; p0 = 4 * (c - 2);
  } else {
    axis = 2; width = 24; p0 = 4 * (c - 5);
  }
}

}  // namespace lcv
