// Query/key prologue of the self-attention over bf16 [n_outer, n_tokens, 64] (HBM-bound):
// RMSNorm of each head's 64 channels with a per-channel gain, then (optionally) the
// partitioned 3D-RoPE (myzaker article, technical principles: RMSNorm in the self-attention
// module and 3D RoPE on visual tokens; longcat-video-rs page, section 03 "Partitioned
// 3D-RoPE (16T+24H+24W)").
//
// Each thread owns one 8-channel chunk of one token, as in the standalone RoPE pass: the
// eight threads of a token are consecutive lanes, so the row's sum of squares is three
// butterfly exchanges inside the lane group; the thread's gains and cos/sin pairs are loaded
// and computed once and reused for every (batch, head) slice it visits.  Values stay in fp32
// from the load to the single rounding to bf16 at the store.
#include "lcv_internal.h"
#include "rope_math.h"

namespace lcv {
namespace {

constexpr int kThreads = 256;
constexpr int kOuterPerThread = 2;

template <bool ROPE>
__global__ __launch_bounds__(kThreads) void qk_prologue_kernel(const uint16_t* x, uint16_t* y, const float* gamma,
                                                               float eps, int64_t n_outer, int32_t n_tokens,
                                                               int32_t token_offset, FastDiv div_hw, FastDiv div_w,
                                                               float log2_theta) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int32_t tok = (int32_t)(gid >> 3);
  const int c = (int)(gid & 7);
  // the eight lanes of a token leave together, so the exchanges below stay inside live groups
  if (tok >= n_tokens) return;

  // the thread's chunks of its (up to) kOuterPerThread slices are all loaded before any is
  // used, so each thread keeps that many 16-byte loads in flight
  const int64_t o0 = (int64_t)blockIdx.y * kOuterPerThread;
  const int n_o = (int)((o0 + kOuterPerThread < n_outer) ? kOuterPerThread : n_outer - o0);
  u32x4 w[kOuterPerThread];
#pragma unroll
  for (int i = 0; i < kOuterPerThread; ++i) {
    const int64_t o = o0 + (i < n_o ? i : n_o - 1);   // past the last slice: reload it (unused)
    w[i] = *reinterpret_cast<const u32x4*>(x + (o * n_tokens + tok) * 64 + 8 * c);
  }
  float gain[8];
  {
    const float4 g0 = *reinterpret_cast<const float4*>(gamma + 8 * c);
    const float4 g1 = *reinterpret_cast<const float4*>(gamma + 8 * c + 4);
    gain[0] = g0.x; gain[1] = g0.y; gain[2] = g0.z; gain[3] = g0.w;
    gain[4] = g1.x; gain[5] = g1.y; gain[6] = g1.z; gain[7] = g1.w;
  }
  float2 cs[4];
  if constexpr (ROPE) {
    const uint32_t n = (uint32_t)(tok + token_offset);
    const uint32_t t = fast_div(n, div_hw);
    const uint32_t rem = n - t * div_hw.d;
    const uint32_t yy = fast_div(rem, div_w);
    const uint32_t xx = rem - yy * div_w.d;
    int axis, width, p0;
    chunk_section(c, axis, width, p0);
    const int32_t pos = (axis == 0) ? (int32_t)t : (axis == 1) ? (int32_t)yy : (int32_t)xx;
#pragma unroll
    for (int e = 0; e < 4; ++e) cs[e] = rope_cos_sin(pos, p0 + e, width, log2_theta);
  }

#pragma unroll
  for (int i = 0; i < kOuterPerThread; ++i) {
    if (i >= n_o) break;
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[i][e] << 16);
      v[2 * e + 1] = __uint_as_float(w[i][e] & 0xffff0000u);
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    ss += __shfl_xor(ss, 4, 64);
    float inv;
    if (ss <= 3.0e38f && ss >= 1.0e-30f) {
      inv = __builtin_amdgcn_rsqf(ss * (1.0f / 64.0f) + eps);   // v_rsq_f32: ~1 ulp, far below bf16
    } else {
      // Rows whose sum of squares overflows fp32, or is too small to keep its precision (or
      // is zero): redo it on the row scaled by the power of two that brings its largest
      // magnitude into [0.5, 1).  The eight lanes of a token take this branch together.
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
      int k;
      frexpf(amax, &k);   // amax = f * 2^k, f in [0.5, 1); k = 0 for a zero row
      k = k < -126 ? -126 : (k > 126 ? 126 : k);   // keep the scale a normal fp32 number
      const float scale = ldexpf(1.0f, -k);
      float su = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float u = v[e] * scale;
        su = fmaf(u, u, su);
      }
      su += __shfl_xor(su, 1, 64);
      su += __shfl_xor(su, 2, 64);
      su += __shfl_xor(su, 4, 64);
      // x / sqrt(mean(x^2) + eps) = (x * scale) / sqrt(mean(u^2) + eps * scale^2), u = x * scale;
      // eps * scale^2 overflows only for rows so far below sqrt(eps) that mean(x^2) vanishes
      // next to eps in fp32: those are x / sqrt(eps)
      const float es = (eps * scale) * scale;
      if (__builtin_isinf(es)) {
        inv = __builtin_amdgcn_rsqf(eps);
      } else {
        inv = __builtin_amdgcn_rsqf(su * (1.0f / 64.0f) + es);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= scale;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = v[e] * inv * gain[e];
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float a = v[2 * e], b = v[2 * e + 1];
      if constexpr (ROPE) {
        const float ra = fmaf(a, cs[e].x, -(b * cs[e].y));
        const float rb = fmaf(a, cs[e].y, b * cs[e].x);
        a = ra;
        b = rb;
      }
      r[e] = pack_bf16x2(a, b);
    }
    *reinterpret_cast<u32x4*>(y + ((o0 + i) * n_tokens + tok) * 64 + 8 * c) = r;
  }
}

}  // namespace

hipError_t launch_qk_prologue(const uint16_t* x, uint16_t* y, const float* gamma, float eps, int64_t n_outer,
                              int32_t n_tokens, int32_t token_offset, bool rope, int32_t H, int32_t W,
                              float log2_theta, hipStream_t stream) {
  if (n_outer == 0 || n_tokens == 0) return hipSuccess;
  const int64_t threads = (int64_t)n_tokens * 8;
  const dim3 grid((unsigned)((threads + kThreads - 1) / kThreads),
                  (unsigned)((n_outer + kOuterPerThread - 1) / kOuterPerThread));
  const FastDiv dhw = make_fastdiv(rope ? (uint32_t)H * (uint32_t)W : 1u);
  const FastDiv dw = make_fastdiv(rope ? (uint32_t)W : 1u);
  if (rope)
    hipLaunchKernelGGL(qk_prologue_kernel<true>, grid, dim3(kThreads), 0, stream, x, y, gamma, eps, n_outer, n_tokens,
                       token_offset, dhw, dw, log2_theta);
  else
    hipLaunchKernelGGL(qk_prologue_kernel<false>, grid, dim3(kThreads), 0, stream, x, y, gamma, eps, n_outer,
                       n_tokens, token_offset, dhw, dw, log2_theta);
  return hipGetLastError();
}

}  // namespace lcv
