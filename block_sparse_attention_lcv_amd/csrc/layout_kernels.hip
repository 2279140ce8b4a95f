// Block layout construction on the GPU: per-row counts, an exclusive scan into row_ptr, the
// ascending col_idx fill, each attention workgroup's key-block list (the union of its query
// blocks' rows with a per-wavefront membership mask) and the forward's work order, and the
// key-side schedule of the backward (groups of key blocks with the ascending union of their
// columns).  Every list is produced by ballot compaction over candidate blocks, each tested
// in O(1) against the closed-form rule, so no kernel walks a list serially.
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

// In-place inclusive scan of a[1..n] by one workgroup of 1024 threads (a[0] is left as is).
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* a, int32_t n) {
  __shared__ int32_t wave_tot[16];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int32_t base = 0; base < n; base += 1024) {
    const int32_t i = base + tid;
    int32_t x = (i < n) ? a[1 + i] : 0;
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
    if (i < n) a[1 + i] = x + before;
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

// Ascending compaction of the candidates c in [lo, hi] with a nonzero mask(c) by one
// wavefront: writes (c << 8) | mask at out[0 ..) in order; returns the count.
template <typename MaskFn>
__device__ __forceinline__ int32_t compact_wave(int32_t lo, int32_t hi, int32_t* out, MaskFn mask_of) {
  const int lane = threadIdx.x & 63;
  int32_t cnt = 0;
  for (int32_t base = lo; base <= hi; base += 64) {
    const int32_t c = base + lane;
    const int32_t m = (c <= hi) ? mask_of(c) : 0;
    const uint64_t bal = __ballot(m != 0);
    const int32_t before = (int32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (m != 0) out[cnt + before] = (c << 8) | m;
    cnt += (int32_t)__popcll(bal);
  }
  return cnt;
}

// One wavefront per attention workgroup list st: the ascending union of the rows of query
// blocks st*kWaves .. +kWaves-1 with bit w set iff row w holds the key block.  The list goes to
// st_ent + row_ptr[st * kWaves] (the union is no longer than the rows together).
__global__ __launch_bounds__(256) void st_union_kernel(LayoutRule L, int32_t n_st, const int32_t* row_ptr,
                                                       int32_t* st_cnt, int32_t* st_ent) {
  const int32_t st = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (st >= n_st) return;
  RowShape rs[kWaves];
  bool on[kWaves];
  int32_t lo = L.n, hi = -1;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int32_t i = st * kWaves + w;
    on[w] = i < L.n;
    rs[w] = row_shape(L, on[w] ? i : 0);
    if (on[w]) {
      lo = rs[w].lo < lo ? rs[w].lo : lo;
      hi = rs[w].hi > hi ? rs[w].hi : hi;
    }
  }
  if (L.s > 0) {   // global blocks anywhere below the eligibility limits
    lo = 0;
    hi = L.n - 1;
  }
  const int32_t cnt = compact_wave(lo, hi, st_ent + row_ptr[st * kWaves], [&](int32_t j) {
    int32_t m = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (on[w] && row_has(L, rs[w], j)) m |= 1 << w;
    return m;
  });
  if ((threadIdx.x & 63) == 0) st_cnt[st] = cnt;
}

// The forward's work order, one workgroup: the lists by decreasing length class (16 classes
// of the longest list's length, class = cnt * 16 / (max + 1)), in index order inside a class
// (stable compaction, class by class).
__global__ __launch_bounds__(1024) void st_order_kernel(const int32_t* st_cnt, int32_t n_st, int32_t* st_order) {
  __shared__ int32_t red[16];
  __shared__ int32_t cmax_s;
  __shared__ int32_t pos_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t m = 0;
  for (int32_t i = tid; i < n_st; i += 1024) m = st_cnt[i] > m ? st_cnt[i] : m;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const int32_t y = __shfl_xor(m, off, 64);
    m = y > m ? y : m;
  }
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (tid == 0) {
    int32_t c = 0;
    for (int w = 0; w < 16; ++w) c = red[w] > c ? red[w] : c;
    cmax_s = c;
    pos_s = 0;
  }
  __syncthreads();
  const int64_t cmax1 = (int64_t)cmax_s + 1;
  for (int cls = 15; cls >= 0; --cls) {
    for (int32_t base = 0; base < n_st; base += 1024) {
      const int32_t i = base + tid;
      const bool take = i < n_st && (int32_t)((int64_t)st_cnt[i] * 16 / cmax1) == cls;
      const uint64_t bal = __ballot(take);
      const int32_t before = (int32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      if (lane == 0) red[wave] = (int32_t)__popcll(bal);
      __syncthreads();
      int32_t off = pos_s;
      for (int w = 0; w < wave; ++w) off += red[w];
      if (take) st_order[off + before] = i;
      __syncthreads();
      if (tid == 1023) pos_s = off + (int32_t)__popcll(bal);
      __syncthreads();
    }
  }
}

// Key block of position p of the backward's key order: the strided global blocks ascending,
// then the others ascending; -1 past the end.
__device__ __forceinline__ int32_t key_order(const LayoutRule& L, int32_t p) {
  if (p >= L.n) return -1;
  if (L.s <= 0) return p;
  const int32_t n_glob = (L.n + L.s - 1) / L.s;
  if (p < n_glob) return p * L.s;
  const int32_t t = p - n_glob;               // s >= 2 here (s == 1 makes every block global)
  return (t / (L.s - 1)) * L.s + 1 + t % (L.s - 1);
}

// Query blocks attending one of a key group's blocks: rows in [lo, hi] (a local block is only
// in the bands of rows within w of it; a global one in every row).
struct GroupScan {
  int32_t j[kWaves];
  int32_t lo, hi;
};
__device__ __forceinline__ GroupScan group_scan(const LayoutRule& L, int32_t g) {
  GroupScan gs;
  gs.lo = L.n;
  gs.hi = -1;
#pragma unroll
  for (int b = 0; b < kWaves; ++b) {
    gs.j[b] = key_order(L, g * kWaves + b);
    if (gs.j[b] < 0) continue;
    const bool global = L.s > 0 && gs.j[b] % L.s == 0;
    const int32_t lo = global ? 0 : (gs.j[b] - L.w > 0 ? gs.j[b] - L.w : 0);
    const int32_t hi = global ? L.n - 1 : (gs.j[b] + L.w < L.n - 1 ? gs.j[b] + L.w : L.n - 1);
    gs.lo = lo < gs.lo ? lo : gs.lo;
    gs.hi = hi > gs.hi ? hi : gs.hi;
  }
  return gs;
}

__device__ __forceinline__ int32_t group_mask(const LayoutRule& L, const GroupScan& gs, int32_t i) {
  const RowShape rs = row_shape(L, i);
  int32_t m = 0;
#pragma unroll
  for (int b = 0; b < kWaves; ++b)
    if (gs.j[b] >= 0 && row_has(L, rs, gs.j[b])) m |= 1 << b;
  return m;
}

// Pass 1, one wavefront per key group: its key blocks (kg_blk) and the length of the union of
// their columns, into kg_cnt[g] and kg_off[g + 1] (scanned afterwards).
__global__ __launch_bounds__(256) void kg_count_kernel(LayoutRule L, int32_t n_kg, int32_t* kg_blk, int32_t* kg_cnt,
                                                       int32_t* kg_off) {
  const int32_t g = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= n_kg) return;
  const int lane = threadIdx.x & 63;
  const GroupScan gs = group_scan(L, g);
  int32_t cnt = 0;
  for (int32_t base = gs.lo; base <= gs.hi; base += 64) {
    const int32_t i = base + lane;
    const bool hit = i <= gs.hi && group_mask(L, gs, i) != 0;
    cnt += (int32_t)__popcll(__ballot(hit));
  }
  int32_t jb = -1;
#pragma unroll
  for (int b = 0; b < kWaves; ++b) jb = lane == b ? gs.j[b] : jb;
  if (lane < kWaves) kg_blk[g * kWaves + lane] = jb;
  if (lane == 0) {
    kg_cnt[g] = cnt;
    kg_off[g + 1] = cnt;
  }
  if (g == 0 && lane == 0) kg_off[0] = 0;
}

// Pass 2, one wavefront per key group: the ascending union (i << 8) | mask at kg_off[g].
__global__ __launch_bounds__(256) void kg_fill_kernel(LayoutRule L, int32_t n_kg, const int32_t* kg_off,
                                                      int32_t* kg_ent) {
  const int32_t g = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= n_kg) return;
  const GroupScan gs = group_scan(L, g);
  compact_wave(gs.lo, gs.hi, kg_ent + kg_off[g], [&](int32_t i) { return group_mask(L, gs, i); });
}

__global__ void summary_kernel(const int32_t* row_ptr, int32_t n, const int32_t* kg_off, int32_t n_kg,
                               int32_t* summary) {
  if (threadIdx.x == 0) {
    summary[0] = row_ptr[n];
    summary[1] = kg_off[n_kg];
  }
}

}  // namespace

hipError_t launch_layout_build(const LayoutRule& L, const LayoutDev& d, hipStream_t stream) {
  hipError_t e;
  hipLaunchKernelGGL(row_count_kernel, dim3((L.n + 255) / 256), dim3(256), 0, stream, L, d.row_ptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, stream, d.row_ptr, L.n);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(row_fill_kernel, dim3(L.n), dim3(256), 0, stream, L, (const int32_t*)d.row_ptr, d.col_idx);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(st_union_kernel, dim3((d.n_st + 3) / 4), dim3(256), 0, stream, L, d.n_st,
                     (const int32_t*)d.row_ptr, d.st_cnt, d.st_ent);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(st_order_kernel, dim3(1), dim3(1024), 0, stream, (const int32_t*)d.st_cnt, d.n_st, d.st_order);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(kg_count_kernel, dim3((d.n_kg + 3) / 4), dim3(256), 0, stream, L, d.n_kg, d.kg_blk, d.kg_cnt,
                     d.kg_off);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, stream, d.kg_off, d.n_kg);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(kg_fill_kernel, dim3((d.n_kg + 3) / 4), dim3(256), 0, stream, L, d.n_kg,
                     (const int32_t*)d.kg_off, d.kg_ent);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(summary_kernel, dim3(1), dim3(64), 0, stream, (const int32_t*)d.row_ptr, L.n,
                     (const int32_t*)d.kg_off, d.n_kg, d.summary);
  return hipGetLastError();
}

}  // namespace lcv
