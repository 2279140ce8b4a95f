// Merge of attention results computed over disjoint key sets (HBM-bound): per row,
// lse = log(sum_i exp(lse_i)) and out = sum_i exp(lse_i - lse) * out_i, which is the softmax
// attention over the union of the sets.  This is the combine step of context-parallel ring
// attention (myzaker article, technical principles: context-parallel ring block-sparse
// attention), where each step attends the key/value shard held by one peer.
//
// One thread per 8-channel chunk of a row, the eight threads of a row consecutive lanes; each
// thread loads its 16-byte chunk of every part and the row's lse of every part (the same
// 4 bytes for the eight lanes), so all loads of a thread are in flight together.  fp32 math,
// one rounding to bf16 at the store.
#include "lcv_internal.h"
#include "rope_math.h"

namespace lcv {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__global__ __launch_bounds__(kThreads) void attn_merge_kernel(const MergeParams P) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t row = gid >> 3;
  const int c = (int)(gid & 7);
  if (row >= P.rows) return;
  u32x4 w[kMaxMergeParts];
  float l[kMaxMergeParts];
#pragma unroll
  for (int i = 0; i < kMaxMergeParts; ++i) {
    if (i < P.n_parts) {
      w[i] = *reinterpret_cast<const u32x4*>(P.outs[i] + row * 64 + 8 * c);
      l[i] = P.lses[i][row];
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxMergeParts; ++i)
    if (i < P.n_parts) m = fmaxf(m, l[i]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float total = 0.f;
  if (m != -INFINITY) {
#pragma unroll
    for (int i = 0; i < kMaxMergeParts; ++i) {
      if (i < P.n_parts) {
        const float wt = exp2f((l[i] - m) * kLog2e);   // exp(lse_i - max) in [0, 1]; 0 for an empty part
        total += wt;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] = fmaf(wt, __uint_as_float(w[i][e] << 16), acc[2 * e]);
          acc[2 * e + 1] = fmaf(wt, __uint_as_float(w[i][e] & 0xffff0000u), acc[2 * e + 1]);
        }
      }
    }
  }
  const float inv = total > 0.f ? 1.f / total : 0.f;   // total >= 1 unless every part is empty
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
  *reinterpret_cast<u32x4*>(P.out + row * 64 + 8 * c) = r;
  if (P.lse != nullptr && c == 0) P.lse[row] = total > 0.f ? m + log2f(total) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_attn_merge(const MergeParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  const int64_t threads = p.rows * 8;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)((threads + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace lcv
