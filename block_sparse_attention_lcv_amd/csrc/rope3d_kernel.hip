// Standalone partitioned 3D-RoPE pass over bf16 [n_outer, n_tokens, 64] (HBM-bound).
//
// Each thread owns one 8-channel chunk of one token: it computes the four cos/sin pairs of
// that chunk once and reuses them for every (batch, head) slice it visits, so the
// trigonometry is amortised over the heads while the 16-byte loads and stores of
// consecutive threads stay contiguous.
#include "lcv_internal.h"
#include "rope_math.h"

namespace lcv {
namespace {

constexpr int kRopeThreads = 256;
constexpr int kRopeOuterPerThread = 2;

__global__ __launch_bounds__(kRopeThreads) void rope3d_kernel(const uint16_t* x, uint16_t* y,
                                                             int64_t n_outer, int32_t n_tokens, int32_t token_offset,
                                                             FastDiv div_hw, FastDiv div_w, float log2_theta) {
  const int64_t gid = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x;
  const int32_t tok = (int32_t)(gid >> 3);
  const int c = (int)(gid & 7);
  if (tok >= n_tokens) return;
  const uint32_t n = (uint32_t)(tok + token_offset);
  const uint32_t t = fast_div(n, div_hw);
  const uint32_t rem = n - t * div_hw.d;
  const uint32_t yy = fast_div(rem, div_w);
  const uint32_t xx = rem - yy * div_w.d;
  int axis, width, p0;
  chunk_section(c, axis, width, p0);
  const int32_t pos = (axis == 0) ? (int32_t)t : (axis == 1) ? (int32_t)yy : (int32_t)xx;
  float2 cs[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) cs[e] = rope_cos_sin(pos, p0 + e, width, log2_theta);

  // the thread's chunks of its (up to) kRopeOuterPerThread slices are all loaded before any
  // is used, so each thread keeps that many 16-byte loads in flight
  const int64_t o0 = (int64_t)blockIdx.y * kRopeOuterPerThread;
  const int n_o = (int)((o0 + kRopeOuterPerThread < n_outer) ? kRopeOuterPerThread : n_outer - o0);
  u32x4 w[kRopeOuterPerThread];
#pragma unroll
  for (int i = 0; i < kRopeOuterPerThread; ++i) {
    const int64_t o = o0 + (i < n_o ? i : n_o - 1);   // past the last slice: reload it (unused)
    w[i] = *reinterpret_cast<const u32x4*>(x + (o * n_tokens + tok) * 64 + 8 * c);
  }
#pragma unroll
  for (int i = 0; i < kRopeOuterPerThread; ++i) {
    if (i >= n_o) break;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[i][e] = rotate_pair(w[i][e], cs[e]);
    *reinterpret_cast<u32x4*>(y + ((o0 + i) * n_tokens + tok) * 64 + 8 * c) = w[i];
  }
}

}  // namespace

hipError_t launch_rope3d(const uint16_t* x, uint16_t* y, int64_t n_outer, int32_t n_tokens, int32_t token_offset,
                         int32_t H, int32_t W, float log2_theta, hipStream_t stream) {
  if (n_outer == 0 || n_tokens == 0) return hipSuccess;
  const int64_t threads = (int64_t)n_tokens * 8;
  const dim3 grid((unsigned)((threads + kRopeThreads - 1) / kRopeThreads),
                  (unsigned)((n_outer + kRopeOuterPerThread - 1) / kRopeOuterPerThread));
  hipLaunchKernelGGL(rope3d_kernel, grid, dim3(kRopeThreads), 0, stream, x, y, n_outer, n_tokens, token_offset,
                     make_fastdiv((uint32_t)H * (uint32_t)W), make_fastdiv((uint32_t)W), log2_theta);
  return hipGetLastError();
}

}  // namespace lcv
