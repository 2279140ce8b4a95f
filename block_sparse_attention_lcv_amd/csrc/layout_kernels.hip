// Block layout construction on the GPU: per-row counts, an exclusive scan into row_ptr,
// the ascending col_idx fill, and each attention workgroup's key-block list (the union
// of its query blocks' rows with a per-wavefront membership mask).
//
// Layout rule: longcat-video-rs page, section 02 benchmark table (block=64, local=2,
// stride=4) and section 03 "Block-Sparse & Multi-Audio" (local window plus strided global
// key/value blocks); condition isolation: myzaker article, section on the technical
// principles (condition tokens unaffected by noise tokens).
#include "lcv_internal.h"

namespace lcv {
namespace {

__global__ __launch_bounds__(256) void row_count_kernel(LayoutRule L, int32_t* row_ptr) {
  const int32_t i = blockIdx.x * 256 + threadIdx.x;
  if (i < L.n) row_ptr[i + 1] = row_shape(L, i).len;
  if (i == 0) row_ptr[0] = 0;
}

// In-place inclusive scan of row_ptr[1..n] by one workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void row_scan_kernel(int32_t* row_ptr, int32_t n) {
  __shared__ int32_t wave_tot[16];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int32_t base = 0; base < n; base += 1024) {
    const int32_t i = base + tid;
    int32_t x = (i < n) ? row_ptr[1 + i] : 0;
    // inclusive scan inside the wavefront
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) wave_tot[wave] = x;
    __syncthreads();
    int32_t before = carry_s;
    for (int w = 0; w < wave; ++w) before += wave_tot[w];
    if (i < n) row_ptr[1 + i] = x + before;
    __syncthreads();
    if (tid == 1023) carry_s = before + x;
    __syncthreads();
  }
}

// One workgroup per query block row: col_idx[row_ptr[i] + r] = r-th key block.
__global__ __launch_bounds__(256) void row_fill_kernel(LayoutRule L, const int32_t* row_ptr, int32_t* col_idx) {
  const int32_t i = blockIdx.x;
  const RowShape rs = row_shape(L, i);
  int32_t* dst = col_idx + row_ptr[i];
  for (int32_t r = threadIdx.x; r < rs.len; r += 256) dst[r] = row_elem(L, rs, r);
}

// One thread per attention workgroup: merge the kWaves ascending rows of its query
// blocks into one ascending list of (j << 8) | (bit w set iff row w contains j).
__global__ __launch_bounds__(64) void st_union_kernel(int32_t n, int32_t n_st, const int32_t* row_ptr,
                                                     const int32_t* col_idx, int32_t* st_cnt, int32_t* st_ent) {
  const int32_t st = blockIdx.x * 64 + threadIdx.x;
  if (st >= n_st) return;
  int32_t cur[kWaves], end[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int32_t i = st * kWaves + w;
    cur[w] = (i < n) ? row_ptr[i] : 0;
    end[w] = (i < n) ? row_ptr[i + 1] : 0;
  }
  int32_t* out = st_ent + row_ptr[st * kWaves];
  int32_t cnt = 0;
  for (;;) {
    int32_t jmin = 0x7fffffff;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (cur[w] < end[w]) jmin = min(jmin, col_idx[cur[w]]);
    if (jmin == 0x7fffffff) break;
    int32_t mask = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (cur[w] < end[w] && col_idx[cur[w]] == jmin) {
        mask |= 1 << w;
        ++cur[w];
      }
    }
    out[cnt++] = (jmin << 8) | mask;
  }
  st_cnt[st] = cnt;
}

}  // namespace

hipError_t launch_layout_build(const LayoutRule& L, const LayoutDev& d, hipStream_t stream) {
  hipLaunchKernelGGL(row_count_kernel, dim3((L.n + 255) / 256), dim3(256), 0, stream, L, d.row_ptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(row_scan_kernel, dim3(1), dim3(1024), 0, stream, d.row_ptr, L.n);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(row_fill_kernel, dim3(L.n), dim3(256), 0, stream, L, (const int32_t*)d.row_ptr, d.col_idx);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(st_union_kernel, dim3((d.n_st + 63) / 64), dim3(64), 0, stream, L.n, d.n_st,
                     (const int32_t*)d.row_ptr, (const int32_t*)d.col_idx, d.st_cnt, d.st_ent);
  return hipGetLastError();
}

}  // namespace lcv
