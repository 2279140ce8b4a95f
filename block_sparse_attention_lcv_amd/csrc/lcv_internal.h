// Internal declarations shared by the host layer and the gfx950 kernels of liblcv_bsa.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

#include "lcv_bsa.h"

namespace lcv {

constexpr int kHeadDim = 64;
constexpr int kBlock = 64;
// Query blocks per workgroup of the attention kernel (one wavefront per query block).
// The layout's per-workgroup key-block lists are built for this width.
constexpr int kWaves = 4;
// Largest 3D-RoPE table (cos/sin pairs) the attention kernel stages in LDS:
// 8*T + 12*H + 12*W entries of 8 bytes.
constexpr int kMaxRopeEntries = 4096;

// n / d for 0 <= n < 2^31 by multiply-high (round-up magic number, Granlund-Montgomery).
struct FastDiv {
  uint32_t d;
  uint32_t m;
  uint32_t s;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  const uint64_t m = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
  return FastDiv{d, static_cast<uint32_t>(m), s};
}

__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv f) {
  return (__umulhi(n, f.m) + n) >> f.s;
}

// Block rule of the layout (see lcv_bsa.h): query block i attends key block j iff
// |i-j| <= w or j % s == 0, restricted to key blocks holding a condition key when every
// row of block i is a condition row.
struct LayoutRule {
  int32_t N;    // tokens
  int32_t n;    // blocks = ceil(N/64)
  int32_t C;    // condition tokens
  int32_t w;    // window radius in blocks
  int32_t s;    // global stride (0 = none)
  int32_t jc;   // key blocks holding at least one condition key = ceil(C/64)
};

struct RowShape {
  int32_t lo, hi;   // band [lo, hi] (never empty)
  int32_t lim;      // key blocks [0, lim) are eligible
  int32_t pre;      // multiples of s below lo
  int32_t len;      // entries in the row
};

__host__ __device__ inline RowShape row_shape(const LayoutRule& L, int32_t i) {
  RowShape r;
  const int32_t last_row = (64 * i + 63 < L.N - 1) ? 64 * i + 63 : L.N - 1;
  r.lim = (last_row >= L.C) ? L.n : L.jc;
  r.lo = (i - L.w > 0) ? i - L.w : 0;
  int32_t hi = i + L.w;
  if (hi > L.n - 1) hi = L.n - 1;
  if (hi > r.lim - 1) hi = r.lim - 1;
  r.hi = hi;
  const int32_t band = r.hi - r.lo + 1;
  if (L.s > 0) {
    r.pre = (r.lo + L.s - 1) / L.s;
    const int32_t post = (r.lim + L.s - 1) / L.s - (r.hi / L.s + 1);
    r.len = r.pre + band + (post > 0 ? post : 0);
  } else {
    r.pre = 0;
    r.len = band;
  }
  return r;
}

// r-th (ascending) key block of row i, 0 <= r < len.
__host__ __device__ inline int32_t row_elem(const LayoutRule& L, const RowShape& rs, int32_t r) {
  if (r < rs.pre) return r * L.s;
  r -= rs.pre;
  const int32_t band = rs.hi - rs.lo + 1;
  if (r < band) return rs.lo + r;
  r -= band;
  return (rs.hi / L.s + 1 + r) * L.s;
}

__host__ __device__ inline bool row_has(const LayoutRule& L, const RowShape& rs, int32_t j) {
  if (j < 0 || j >= rs.lim) return false;
  if (j >= rs.lo && j <= rs.hi) return true;
  return L.s > 0 && (j % L.s) == 0;
}

// Entries of row i that are < a.
__host__ __device__ inline int32_t row_count_below(const LayoutRule& L, const RowShape& rs, int32_t a) {
  if (a > rs.lim) a = rs.lim;
  if (a <= 0) return 0;
  int32_t c = 0;
  // band part
  const int32_t bh = (a - 1 < rs.hi) ? a - 1 : rs.hi;
  if (bh >= rs.lo) c += bh - rs.lo + 1;
  if (L.s > 0) {
    // multiples below lo (and below a)
    const int32_t lo_cap = (a < rs.lo) ? a : rs.lo;
    c += (lo_cap + L.s - 1) / L.s;
    // multiples in (hi, a)
    if (a - 1 > rs.hi) {
      const int32_t above = (a + L.s - 1) / L.s - (rs.hi / L.s + 1);
      if (above > 0) c += above;
    }
  }
  return c;
}

// Device-side layout owned by a handle.
struct LayoutDev {
  int32_t* row_ptr;   // [n+1]
  int32_t* col_idx;   // [nnz]
  int32_t* st_cnt;    // [n_st] entries of each workgroup's key-block list
  int32_t* st_ent;    // [nnz]   list of workgroup st starts at row_ptr[st*kWaves]: (j << 8) | wave mask
  int32_t* st_order;  // [n_st]  the forward's work order: lists by decreasing length class, index order inside
  int32_t n_st;       // ceil(n / kWaves)
  // Key-side schedule of the backward (column walk): key blocks in groups of kWaves whose
  // columns (attending query blocks) are nearly the same -- the strided global blocks
  // together, the others in runs of consecutive blocks -- and per group the ascending union
  // of its columns, entry (i << 8) | mask (bit b: query block i attends key block kg_blk[4g+b]).
  int32_t* kg_blk;    // [n_kg * kWaves] key block of each slot, -1 for an empty slot
  int32_t* kg_cnt;    // [n_kg]
  int32_t* kg_off;    // [n_kg + 1] first entry of each group's list in kg_ent (kg_off[n_kg] = kg_total)
  int32_t* kg_ent;    // [kg_total] (room for nnz: a group's union is no longer than its columns together)
  int32_t n_kg;
  int64_t kg_total;
  int32_t* summary;   // [2] written by the build: row_ptr[n] and kg_total, read back once
  void* block;        // the one device allocation all of the above live in
};

struct FwdParams {
  const uint16_t* q;        // [BH, q_rows, 64]
  const uint16_t* k;        // [BH, N - kv_split, 64]
  const uint16_t* v;
  const uint16_t* k_cond;   // [BH, kv_split, 64] (cached call)
  const uint16_t* v_cond;
  uint16_t* out;            // [BH, q_rows, 64]
  float* lse;               // [BH, q_rows] or nullptr
  const int32_t* row_ptr;
  const int32_t* st_cnt;
  const int32_t* st_ent;
  int32_t N, C, n_blocks;
  int32_t q_row0;           // first query token of the call (0 full, C cached)
  int32_t q_rows;           // q_end - q_row0 (rows of the q, out and lse tensors)
  int32_t q_end;            // one past the last query token of the call (N unless a row range)
  int32_t kv_split;         // keys < kv_split read from k_cond / v_cond
  int32_t st_first;         // first workgroup list used
  int32_t n_st_active;      // workgroup lists per (batch, head)
  int32_t n_items;          // BH * n_st_active
  int32_t bh_count;         // BH (batch * heads)
  const int32_t* st_order;  // [n_st] the layout's work order of the lists (full calls), or nullptr:
                            // lists st_first, st_first + 1, ... in order
  uint32_t flags;
  int32_t T, H, W;
  FastDiv div_hw, div_w;
  float log2_theta;
  int32_t rope_entries;     // 8T + 12H + 12W when a RoPE flag is set
  // cross-attention only: text keys/values [BH, kv_len, 64], optional per-batch lengths
  int32_t kv_len;
  const int32_t* kv_lens;   // [B] device, or nullptr (all kv_len)
  int32_t heads;
  int32_t q_per_part;       // > 0: query blocks per workgroup of the walk with the text in LDS
                            // (a multiple of 2 * kWaves; n_st_active counts the ranges)
};

struct BwdParams {
  const uint16_t* q;        // [BH, N, 64], as it entered the scores (rotated)
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* out;      // forward output
  const uint16_t* dout;     // upstream gradient
  const float* lse;         // [BH, N] natural-log LSE of the forward
  uint16_t* qs;             // [BH, N, 64] workspace: Q' = bf16(q * log2(e)/8), the forward's operand
  float* lse2;              // [BH, N] workspace: lse * log2(e) (3e38 for an empty row)
  float* delta;             // [BH, N] workspace: rowsum(dout * out)
  uint2* fold_l;            // [BH, N] workspace: the three bf16 parts of -lse2 (the key walk's fold operand)
  uint2* fold_d;            // [BH, N] workspace: the three bf16 parts of -delta
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  const int32_t* row_ptr;
  const int32_t* st_cnt;
  const int32_t* st_ent;
  const int32_t* kg_blk;
  const int32_t* kg_cnt;
  const int32_t* kg_off;
  const int32_t* kg_ent;
  int64_t bh_rows;          // BH * N
  int32_t N, C, n_blocks, n_st, n_kg, bh;
  // cross-attention (text keys/values [BH, kv_len, 64])
  bool cross;               // true: the cross-attention backward (the fields below), false: self-attention
  int32_t kv_len;           // rows per (batch, head) of k and v
  const int32_t* kv_lens;   // [B] valid text tokens, or nullptr
  int32_t heads;
  int32_t n_kv_blocks;      // ceil(kv_len / 64)
  int32_t q_chunk;          // query blocks per key-walk workgroup
  int32_t n_chunks;         // key-walk chunks of the query blocks
  float* part_dk;           // [n_chunks, BH, kv_len, 64] fp32 partial sums
  float* part_dv;
  int32_t q_parts;          // > 0: query-walk workgroups per (batch, head) with the text in LDS
  int32_t q_per_part;       // query blocks per such workgroup (a multiple of 4)
};
// Text blocks a cross-attention query walk keeps resident in LDS (K and V: 128 KB).
constexpr int kCrossResidentBlocks = 8;

hipError_t launch_layout_build(const LayoutRule& L, const LayoutDev& d, hipStream_t stream);
hipError_t launch_bsa_bwd(const BwdParams& p, hipStream_t stream);
hipError_t launch_cross_fwd(const FwdParams& p, hipStream_t stream);

constexpr int kMaxMergeParts = 8;
struct MergeParams {
  const uint16_t* outs[kMaxMergeParts];   // bf16 [rows, 64] per part
  const float* lses[kMaxMergeParts];      // fp32 [rows] per part
  uint16_t* out;
  float* lse;                             // or nullptr
  int64_t rows;
  int32_t n_parts;
};
hipError_t launch_attn_merge(const MergeParams& p, hipStream_t stream);
hipError_t launch_rope3d(const uint16_t* x, uint16_t* y, int64_t n_outer, int32_t n_tokens,
                         int32_t token_offset, int32_t H, int32_t W, float log2_theta, hipStream_t stream);
hipError_t launch_bsa_fwd(const FwdParams& p, hipStream_t stream);
hipError_t launch_qk_prologue(const uint16_t* x, uint16_t* y, const float* gamma, float eps, int64_t n_outer,
                              int32_t n_tokens, int32_t token_offset, bool rope, int32_t H, int32_t W,
                              float log2_theta, hipStream_t stream);

}  // namespace lcv
