// Backward of the query/key prologue (RMSNorm + 3D-RoPE): internal declarations.
#pragma once

#include "lcv_internal.h"

namespace lcv {

constexpr int kPrologueBwdThreads = 256;
constexpr int kPrologueBwdSlices = 16;        // (batch, head) slices per workgroup row of the grid
constexpr int kPrologueBwdMaxGroups = 512;    // token-group workgroups per slice range

struct PrologueBwdGrid {
  int64_t x, y;   // workgroups along token groups and along slice ranges
};

inline PrologueBwdGrid prologue_bwd_grid(int64_t n_outer, int32_t n_tokens) {
  const int64_t groups = ((int64_t)n_tokens * 8 + kPrologueBwdThreads - 1) / kPrologueBwdThreads;
  PrologueBwdGrid g;
  g.x = groups < kPrologueBwdMaxGroups ? groups : kPrologueBwdMaxGroups;
  g.y = (n_outer + kPrologueBwdSlices - 1) / kPrologueBwdSlices;
  return g;
}

// fp32 values of the workspace: one 64-value partial gain gradient per workgroup
inline int64_t prologue_bwd_workspace_floats(int64_t n_outer, int32_t n_tokens) {
  const PrologueBwdGrid g = prologue_bwd_grid(n_outer, n_tokens);
  return g.x * g.y * 64;
}

// The allocation-free entry point keeps the workgroups' partials in a static device array of
// this many floats (4 MiB: 16,384 workgroup partials, e.g. 512 (batch, head) slices of up to
// 16,384 tokens each, or 32 slices of any length).
constexpr int64_t kNoAllocPartialFloats = int64_t(1) << 20;

// Address of that array on the current device, looked up once per device.
hipError_t prologue_bwd_scratch(float** ptr);

hipError_t launch_qk_prologue_bwd(const uint16_t* x, const uint16_t* dy, const float* gamma, float eps, int64_t n_outer,
                                  int32_t n_tokens, int32_t token_offset, bool rope, int32_t H, int32_t W,
                                  float log2_theta, uint16_t* dx, float* dgamma, float* partials, hipStream_t stream);

}  // namespace lcv
