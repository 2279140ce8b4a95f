// Backward of the query/key prologue (HBM-bound): for y = R (x / r * gamma) with
// r = sqrt(mean(x^2) + eps) over each head's 64 channels and R the partitioned 3D-RoPE
// (myzaker article, technical principles: RMSNorm in the self-attention and 3D RoPE on
// visual tokens; longcat-video-rs page, section 03 "Partitioned 3D-RoPE (16T+24H+24W)"),
// the gradients for the upstream gradient dy are, with n = x / r and dy' = R^T dy (each pair
// rotated by minus its angle):
//   dgamma = sum over every row of dy' * n,   dx = (dn - n * mean(dn * n)) / r,  dn = dy' * gamma.
//
// Thread mapping as in the forward prologue: one thread per 8-channel chunk of a token, the
// eight threads of a token consecutive lanes (row sums are three butterfly exchanges); a
// workgroup walks token groups (grid-stride) over a range of (batch, head) slices, two slices
// per iteration with all four 16-byte loads in flight.  Each workgroup writes its 64 partial
// sums of dgamma to the workspace; a second kernel adds them in a fixed order, so the result
// is deterministic.
#include <mutex>

#include "prologue_bwd.h"
#include "rope_math.h"

namespace lcv {
namespace {

constexpr int kThreads = kPrologueBwdThreads;

// 1 / sqrt(mean(v^2) + eps) for the lane group's row, with v rescaled in place by a power of
// two when the fp32 sum of squares would overflow or lose its precision; returns the factor
// that turns the result into 1/r of the unscaled row (v_scaled * inv == v / r).
__device__ __forceinline__ float row_inv_rms(float (&v)[8], float eps, float& unscale) {
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
  ss += __shfl_xor(ss, 1, 64);
  ss += __shfl_xor(ss, 2, 64);
  ss += __shfl_xor(ss, 4, 64);
  unscale = 1.f;
  if (ss <= 3.0e38f && ss >= 1.0e-30f) return __builtin_amdgcn_rsqf(ss * (1.0f / 64.0f) + eps);
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
  int k;
  frexpf(amax, &k);
  k = k < -126 ? -126 : (k > 126 ? 126 : k);
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
  const float es = (eps * scale) * scale;
  if (__builtin_isinf(es)) return __builtin_amdgcn_rsqf(eps);   // mean(x^2) vanishes next to eps
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] *= scale;
  unscale = scale;
  return __builtin_amdgcn_rsqf(su * (1.0f / 64.0f) + es);
}

template <bool ROPE>
__global__ __launch_bounds__(kThreads) void qk_prologue_bwd_kernel(const uint16_t* x, const uint16_t* dy,
                                                                   const float* gamma, float eps, int64_t n_outer,
                                                                   int32_t n_tokens, int32_t token_offset,
                                                                   FastDiv div_hw, FastDiv div_w, float log2_theta,
                                                                   uint16_t* dx, float* partials) {
  __shared__ float red[kThreads / 64][64];
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int c = tid & 7;
  const int64_t o0 = (int64_t)blockIdx.y * kPrologueBwdSlices;
  const int n_o = (int)((o0 + kPrologueBwdSlices < n_outer) ? kPrologueBwdSlices : n_outer - o0);
  float gain[8];
  {
    const float4 g0 = *reinterpret_cast<const float4*>(gamma + 8 * c);
    const float4 g1 = *reinterpret_cast<const float4*>(gamma + 8 * c + 4);
    gain[0] = g0.x; gain[1] = g0.y; gain[2] = g0.z; gain[3] = g0.w;
    gain[4] = g1.x; gain[5] = g1.y; gain[6] = g1.z; gain[7] = g1.w;
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int64_t n_groups = ((int64_t)n_tokens * 8 + kThreads - 1) / kThreads;
  for (int64_t grp = blockIdx.x; grp < n_groups; grp += gridDim.x) {
    const int32_t tok = (int32_t)((grp * kThreads + tid) >> 3);
    if (tok >= n_tokens) continue;   // the eight lanes of a token skip together
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
    for (int i0 = 0; i0 < n_o; i0 += 2) {
      // both slices' x and dy chunks in flight together (a missing second slice re-reads the first)
      u32x4 wx[2], wd[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int64_t o = o0 + (i0 + k < n_o ? i0 + k : i0);
        const int64_t off = (o * n_tokens + tok) * 64 + 8 * c;
        wx[k] = *reinterpret_cast<const u32x4*>(x + off);
        wd[k] = *reinterpret_cast<const u32x4*>(dy + off);
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if (i0 + k >= n_o) break;
        float v[8], g[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = __uint_as_float(wx[k][e] << 16);
          v[2 * e + 1] = __uint_as_float(wx[k][e] & 0xffff0000u);
          float a = __uint_as_float(wd[k][e] << 16), b = __uint_as_float(wd[k][e] & 0xffff0000u);
          if constexpr (ROPE) {
            const float ra = fmaf(a, cs[e].x, b * cs[e].y);    // R^T: rotation by minus the angle
            const float rb = fmaf(b, cs[e].x, -(a * cs[e].y));
            a = ra;
            b = rb;
          }
          g[2 * e] = a;
          g[2 * e + 1] = b;
        }
        float unscale;
        const float inv = row_inv_rms(v, eps, unscale);
        float nrm[8], dn[8], dot = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          nrm[e] = v[e] * inv;
          acc[e] = fmaf(g[e], nrm[e], acc[e]);
          dn[e] = g[e] * gain[e];
          dot = fmaf(dn[e], nrm[e], dot);
        }
        dot += __shfl_xor(dot, 1, 64);
        dot += __shfl_xor(dot, 2, 64);
        dot += __shfl_xor(dot, 4, 64);
        const float mean = dot * (1.0f / 64.0f);
        const float inv_r = inv * unscale;
        u32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          r[e] = pack_bf16x2((dn[2 * e] - nrm[2 * e] * mean) * inv_r, (dn[2 * e + 1] - nrm[2 * e + 1] * mean) * inv_r);
        const int64_t o = o0 + i0 + k;
        *reinterpret_cast<u32x4*>(dx + (o * n_tokens + tok) * 64 + 8 * c) = r;
      }
    }
  }
  // workgroup sum of the gain gradient: lanes of equal chunk (lane bits 3..5), then waves
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    acc[e] += __shfl_xor(acc[e], 8, 64);
    acc[e] += __shfl_xor(acc[e], 16, 64);
    acc[e] += __shfl_xor(acc[e], 32, 64);
  }
  if (lane < 8) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[tid >> 6][8 * lane + e] = acc[e];
  }
  __syncthreads();
  if (tid < 64) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) s += red[w][tid];
    partials[((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * 64 + tid] = s;
  }
}

// dgamma = sum of the workgroups' partials, in a fixed order: 1024 threads, thread t adds the
// partials t/64, t/64 + 16, ... of channel t%64 (eight independent sums, so that eight loads
// are in flight, added in a fixed order), then 16 values per channel.
__global__ __launch_bounds__(1024) void sum_partials_kernel(const float* partials, int64_t n_part, float* dgamma) {
  __shared__ float red[16][64];
  const int tid = (int)threadIdx.x;
  const int ch = tid & 63;
  const int grp = tid >> 6;
  float s8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int64_t p = grp;
  for (; p + 7 * 16 < n_part; p += 8 * 16) {
#pragma unroll
    for (int u = 0; u < 8; ++u) s8[u] += partials[(p + 16 * u) * 64 + ch];
  }
  for (int u = 0; p < n_part; p += 16, ++u) s8[u & 7] += partials[p * 64 + ch];
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) s += s8[u];
  red[grp][ch] = s;
  __syncthreads();
  if (tid < 64) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) t += red[k][tid];
    dgamma[tid] = t;
  }
}

// Scratch of lcv_qk_rmsnorm_rope3d_backward_noalloc: the workgroups' dgamma partials, for
// callers that cannot allocate.  The loader gives every GPU the library runs on its own copy
// with the code object (held until the process ends); in host code the name is only a handle
// for hipGetSymbolAddress, never a device address.  Calls on one GPU share it: overlapping
// calls race.  Every workgroup writes its own partial before the sum kernel reads it, so no
// call needs it cleared.
static __device__ __align__(256) float scratch[kNoAllocPartialFloats];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxScratchDevices] = {};

}  // namespace

hipError_t prologue_bwd_scratch(float** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_qk_prologue_bwd(const uint16_t* x, const uint16_t* dy, const float* gamma, float eps, int64_t n_outer,
                                  int32_t n_tokens, int32_t token_offset, bool rope, int32_t H, int32_t W,
                                  float log2_theta, uint16_t* dx, float* dgamma, float* partials, hipStream_t stream) {
  const PrologueBwdGrid pg = prologue_bwd_grid(n_outer, n_tokens);
  if (pg.x > 0 && pg.y > 0) {
    const dim3 grid((unsigned)pg.x, (unsigned)pg.y);
    const FastDiv dhw = make_fastdiv(rope ? (uint32_t)H * (uint32_t)W : 1u);
    const FastDiv dw = make_fastdiv(rope ? (uint32_t)W : 1u);
    if (rope)
      hipLaunchKernelGGL(qk_prologue_bwd_kernel<true>, grid, dim3(kThreads), 0, stream, x, dy, gamma, eps, n_outer,
                         n_tokens, token_offset, dhw, dw, log2_theta, dx, partials);
    else
      hipLaunchKernelGGL(qk_prologue_bwd_kernel<false>, grid, dim3(kThreads), 0, stream, x, dy, gamma, eps, n_outer,
                         n_tokens, token_offset, dhw, dw, log2_theta, dx, partials);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(sum_partials_kernel, dim3(1), dim3(1024), 0, stream, partials, pg.x * pg.y, dgamma);
  return hipGetLastError();
}

}  // namespace lcv
