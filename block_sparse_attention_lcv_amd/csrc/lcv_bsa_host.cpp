// Host side of liblcv_bsa: argument validation, layout handles and kernel launches.
// Every check runs before anything is launched; see include/lcv_bsa.h for the contract.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "lcv_internal.h"
#include "prologue_bwd.h"

struct lcv_bsa_layout {
  lcv_bsa_layout_info info;
  lcv::LayoutDev dev;
  int device;
};

namespace {

thread_local std::string g_last_error;

lcv_status fail(lcv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

lcv_status ok() {
  g_last_error.clear();
  return LCV_OK;
}

lcv_status hip_fail(hipError_t e, const char* what) {
  return fail(LCV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

lcv_status check_params(const lcv_bsa_layout_params* p) {
  if (p == nullptr) return fail(LCV_ERR_NULL, "params is NULL");
  if (p->block != LCV_BLOCK) return fail(LCV_ERR_INVALID_ARG, "block must be %d (got %d)", LCV_BLOCK, p->block);
  if (p->n_tokens < 1) return fail(LCV_ERR_INVALID_ARG, "n_tokens must be >= 1 (got %d)", p->n_tokens);
  if (p->local_blocks < 0) return fail(LCV_ERR_INVALID_ARG, "local_blocks must be >= 0 (got %d)", p->local_blocks);
  if (p->global_stride < 0) return fail(LCV_ERR_INVALID_ARG, "global_stride must be >= 0 (got %d)", p->global_stride);
  if (p->cond_len < 0 || p->cond_len > p->n_tokens)
    return fail(LCV_ERR_INVALID_ARG, "cond_len must be in [0, n_tokens] (got %d, n_tokens %d)", p->cond_len, p->n_tokens);
  const int64_t n = ((int64_t)p->n_tokens + LCV_BLOCK - 1) / LCV_BLOCK;
  if (n >= (int64_t(1) << 23))
    return fail(LCV_ERR_UNSUPPORTED, "more than 2^23 blocks (%lld) are not supported", (long long)n);
  return LCV_OK;
}

lcv::LayoutRule make_rule(const lcv_bsa_layout_params* p) {
  lcv::LayoutRule L;
  L.N = p->n_tokens;
  L.n = (p->n_tokens + LCV_BLOCK - 1) / LCV_BLOCK;
  L.C = p->cond_len;
  // a window wider than the sequence is the whole sequence
  L.w = p->local_blocks < L.n ? p->local_blocks : L.n;
  L.s = p->global_stride;
  L.jc = (p->cond_len + LCV_BLOCK - 1) / LCV_BLOCK;
  return L;
}

// Closed-form sizes of the layout (host only).
lcv_status compute_info(const lcv_bsa_layout_params* p, lcv_bsa_layout_info* info) {
  const lcv::LayoutRule L = make_rule(p);
  int64_t nnz = 0, pairs = 0;
  int32_t max_len = 0;
  const int32_t last_size = L.N - 64 * (L.n - 1);
  const int32_t fc = L.C / 64;                       // blocks [0, fc) are all condition keys
  const int32_t partial = (fc < L.n) ? (L.C - 64 * fc) : 0;  // condition keys of block fc
  for (int32_t i = 0; i < L.n; ++i) {
    const lcv::RowShape rs = lcv::row_shape(L, i);
    nnz += rs.len;
    if (rs.len > max_len) max_len = rs.len;
    const int32_t size_i = (i == L.n - 1) ? last_size : 64;
    int32_t cond_rows = L.C - 64 * i;
    cond_rows = cond_rows < 0 ? 0 : (cond_rows > size_i ? size_i : cond_rows);
    const int32_t noise_rows = size_i - cond_rows;
    // keys of the row: 64 per block, the last block may be short
    int64_t keys = 64 * (int64_t)rs.len;
    if (lcv::row_has(L, rs, L.n - 1)) keys -= 64 - last_size;
    // condition keys of the row
    int64_t ckeys = 64 * (int64_t)lcv::row_count_below(L, rs, fc);
    if (partial > 0 && lcv::row_has(L, rs, fc)) ckeys += partial;
    pairs += (int64_t)noise_rows * keys + (int64_t)cond_rows * ckeys;
  }
  if (nnz >= (int64_t(1) << 31))
    return fail(LCV_ERR_UNSUPPORTED, "layout has %lld entries; at most 2^31-1 are supported", (long long)nnz);
  info->n_tokens = p->n_tokens;
  info->n_blocks = L.n;
  info->local_blocks = p->local_blocks;
  info->global_stride = p->global_stride;
  info->cond_len = p->cond_len;
  info->max_row_len = max_len;
  info->nnz = nnz;
  info->attended_pairs = pairs;
  return LCV_OK;
}

lcv_status check_grid(const lcv_rope3d_grid* grid) {
  if (grid == nullptr) return fail(LCV_ERR_NULL, "grid is NULL");
  if (grid->T < 1 || grid->H < 1 || grid->W < 1)
    return fail(LCV_ERR_INVALID_ARG, "grid dimensions must be >= 1 (got %d x %d x %d)", grid->T, grid->H, grid->W);
  if (!(grid->theta > 0.f) || !std::isfinite(grid->theta))
    return fail(LCV_ERR_INVALID_ARG, "theta must be finite and > 0");
  if ((int64_t)grid->T * grid->H * grid->W >= (int64_t(1) << 31))
    return fail(LCV_ERR_UNSUPPORTED, "grid has more than 2^31-1 tokens");
  return LCV_OK;
}

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* k_cond;
  const void* v_cond;
  void* out;
  float* lse;
  bool cached;
  int32_t row_begin = 0;    // query rows [row_begin, row_end) of the call (row_end < 0: to N)
  int32_t row_end = -1;
};

lcv_status forward_common(const FwdArgs& a, int32_t batch, int32_t heads, const lcv_bsa_layout* layout,
                          int32_t cond_len, uint32_t flags, const lcv_rope3d_grid* grid, hipStream_t stream) {
  if (layout == nullptr) return fail(LCV_ERR_NULL, "layout is NULL");
  if (batch < 1 || heads < 1) return fail(LCV_ERR_INVALID_ARG, "batch and heads must be >= 1 (got %d, %d)", batch, heads);
  const lcv_bsa_layout_info& info = layout->info;
  if (cond_len != info.cond_len)
    return fail(LCV_ERR_LAYOUT_MISMATCH, "cond_len %d differs from the layout's %d", cond_len, info.cond_len);
  if (flags & ~(LCV_ROPE_Q | LCV_ROPE_K)) return fail(LCV_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  const int32_t N = info.n_tokens, C = info.cond_len;
  const bool has_noise = N > C;
  if (a.cached) {
    if (has_noise && (a.q == nullptr || a.k == nullptr || a.v == nullptr || a.out == nullptr))
      return fail(LCV_ERR_NULL, "q_noise, k_noise, v_noise and out_noise are required when cond_len < n_tokens");
    if (C > 0 && (a.k_cond == nullptr || a.v_cond == nullptr))
      return fail(LCV_ERR_NULL, "k_cond and v_cond are required when cond_len > 0");
  } else if (a.q == nullptr || a.k == nullptr || a.v == nullptr || a.out == nullptr) {
    return fail(LCV_ERR_NULL, "q, k, v and out are required");
  }
  const void* ptrs16[] = {a.q, a.k, a.v, a.k_cond, a.v_cond, a.out};
  for (const void* p : ptrs16)
    if (p != nullptr && !aligned(p, 16)) return fail(LCV_ERR_INVALID_ARG, "bf16 tensors must be 16-byte aligned");
  if (a.lse != nullptr && !aligned(a.lse, 4)) return fail(LCV_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  int32_t rope_entries = 0;
  if (flags) {
    lcv_status st = check_grid(grid);
    if (st != LCV_OK) return st;
    if ((int64_t)grid->T * grid->H * grid->W != N)
      return fail(LCV_ERR_SHAPE, "grid %d x %d x %d has %lld tokens, layout has %d", grid->T, grid->H, grid->W,
                  (long long)grid->T * grid->H * grid->W, N);
    const int64_t entries = 8 * (int64_t)grid->T + 12 * (int64_t)grid->H + 12 * (int64_t)grid->W;
    if (entries > lcv::kMaxRopeEntries)
      return fail(LCV_ERR_UNSUPPORTED, "fused RoPE supports 8T+12H+12W <= %d (got %lld); rotate with lcv_rope3d_apply",
                  lcv::kMaxRopeEntries, (long long)entries);
    rope_entries = (int32_t)entries;
  }
  const int64_t bh = (int64_t)batch * heads;
  const int32_t n = info.n_blocks;
  const int32_t q_row0 = a.cached ? C : a.row_begin;
  const int32_t q_end = a.row_end < 0 ? N : a.row_end;
  if (q_row0 >= q_end) return ok();   // cached call with no noise tokens, or an empty row range
  const int32_t st_first = (q_row0 / 64) / lcv::kWaves;
  const int32_t st_end = ((q_end + 63) / 64 + lcv::kWaves - 1) / lcv::kWaves;
  const int64_t n_items = bh * (st_end - st_first);
  if (n_items >= (int64_t(1) << 31) - 8)
    return fail(LCV_ERR_UNSUPPORTED, "batch*heads*workgroups = %lld is too large", (long long)n_items);

  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != layout->device)
    return fail(LCV_ERR_INVALID_ARG, "layout was built on device %d, current device is %d", layout->device, dev);

  lcv::FwdParams p;
  std::memset(&p, 0, sizeof p);
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.k_cond = static_cast<const uint16_t*>(a.k_cond);
  p.v_cond = static_cast<const uint16_t*>(a.v_cond);
  p.out = static_cast<uint16_t*>(a.out);
  p.lse = a.lse;
  p.row_ptr = layout->dev.row_ptr;
  p.st_cnt = layout->dev.st_cnt;
  p.st_ent = layout->dev.st_ent;
  p.N = N;
  p.C = C;
  p.n_blocks = n;
  p.q_row0 = q_row0;
  p.q_rows = q_end - q_row0;
  p.q_end = q_end;
  p.kv_split = a.cached ? C : 0;
  p.st_first = st_first;
  p.n_st_active = st_end - st_first;
  p.n_items = (int32_t)n_items;
  p.bh_count = (int32_t)bh;
  // the lists by decreasing length when the call covers every query row; a row range or the
  // cached call walks its lists in order
  p.st_order = (q_row0 == 0 && q_end == N) ? layout->dev.st_order : nullptr;
  p.flags = flags;
  if (flags) {
    p.T = grid->T;
    p.H = grid->H;
    p.W = grid->W;
    p.div_hw = lcv::make_fastdiv((uint32_t)grid->H * (uint32_t)grid->W);
    p.div_w = lcv::make_fastdiv((uint32_t)grid->W);
    p.log2_theta = std::log2(grid->theta);
    p.rope_entries = rope_entries;
  }
  e = lcv::launch_bsa_fwd(p, stream);
  if (e != hipSuccess) return hip_fail(e, "bsa_fwd launch");
  return ok();
}

// Workspace of the attention backward, per query row: Q' = bf16(q * log2(e)/8) (64 bf16 = 32
// fp32 slots), then lse * log2(e) and D = rowsum(dO * O) of every row, then the three bf16
// parts of -lse * log2(e) and of -D (8 bytes each) of every row.
constexpr int64_t kBwdRowFloats = 38;

// Work split of the cross-attention backward: the query walk takes four query blocks per
// workgroup; the key walk takes four text blocks and one chunk of the query blocks, with
// enough chunks to give the chip about 512 workgroups; the chunks' fp32 partial dK, dV
// follow the per-row values in the workspace (16-byte aligned).
// workgroups the cross-attention forward with the text in LDS aims for (one per compute unit)
#ifndef LCV_CROSS_FWD_WORKGROUPS
#define LCV_CROSS_FWD_WORKGROUPS 256
#endif

// workgroups the two walks of the cross-attention backward aim for (a few per compute unit)
#ifndef LCV_CROSS_KEY_WALK_WORKGROUPS
#define LCV_CROSS_KEY_WALK_WORKGROUPS 512
#endif
#ifndef LCV_CROSS_QUERY_WALK_WORKGROUPS
#define LCV_CROSS_QUERY_WALK_WORKGROUPS 512
#endif

struct CrossBwdPlan {
  int32_t n_q_blocks, n_kv_blocks, n_st, n_kg, n_chunks, q_chunk;
  int32_t q_parts, q_per_part;   // query walk with the text resident in LDS (q_parts = 0: not)
  int64_t part_offset, part_floats, workspace_floats;
};

CrossBwdPlan cross_bwd_plan(int64_t bh, int32_t n_q, int32_t kv_len) {
  CrossBwdPlan pl{};
  pl.n_q_blocks = (int32_t)(((int64_t)n_q + 63) / 64);
  pl.n_kv_blocks = (int32_t)(((int64_t)kv_len + 63) / 64);
  pl.n_st = (pl.n_q_blocks + lcv::kWaves - 1) / lcv::kWaves;
  const int64_t n_groups = (pl.n_kv_blocks + lcv::kWaves - 1) / lcv::kWaves;
  int64_t chunks = 0;
  if (pl.n_q_blocks > 0 && n_groups > 0) {
    const int64_t per_chunk = bh * n_groups;
    chunks = (LCV_CROSS_KEY_WALK_WORKGROUPS + per_chunk - 1) / per_chunk;
    chunks = chunks < 64 ? chunks : 64;
    chunks = chunks < pl.n_q_blocks ? chunks : pl.n_q_blocks;
    pl.q_chunk = (int32_t)((pl.n_q_blocks + chunks - 1) / chunks);
    chunks = (pl.n_q_blocks + pl.q_chunk - 1) / pl.q_chunk;   // no empty chunk
  }
  pl.n_chunks = (int32_t)chunks;
  // query walk: with the text in LDS, about 512 workgroups, each a range of query blocks as
  // equal as whole blocks allow (its wavefronts share it 32 rows at a time), at least 4 long
  if (pl.n_q_blocks > 0 && pl.n_kv_blocks <= lcv::kCrossResidentBlocks) {
    int64_t parts = (LCV_CROSS_QUERY_WALK_WORKGROUPS + bh - 1) / bh;
    parts = parts < pl.n_st ? parts : pl.n_st;
    const int64_t per = (pl.n_q_blocks + parts - 1) / parts;
    pl.q_per_part = (int32_t)per;
    pl.q_parts = (int32_t)((pl.n_q_blocks + per - 1) / per);
  }
  pl.n_kg = (int32_t)(n_groups * chunks);
  const int64_t rows = bh * n_q;
  pl.part_offset = (kBwdRowFloats * rows + 3) / 4 * 4;
  pl.part_floats = chunks * bh * kv_len * 64;
  pl.workspace_floats = pl.part_offset + 2 * pl.part_floats;
  return pl;
}

// Shared checks and launch of the two prologue backward entry points: the caller's workspace,
// or (static_scratch) the library's static scratch array of the current device, looked up
// after every check has passed.
lcv_status prologue_bwd_common(const void* x, const void* dy, const float* gamma, float eps, int64_t n_outer,
                               int32_t n_tokens, int32_t token_offset, const lcv_rope3d_grid* grid, void* dx,
                               float* dgamma, float* workspace, int64_t workspace_floats, bool static_scratch,
                               hipStream_t stream) {
  if (x == nullptr || dy == nullptr || gamma == nullptr || dx == nullptr || dgamma == nullptr)
    return fail(LCV_ERR_NULL, "x, dy, gamma, dx and dgamma are required");
  if (n_outer < 0 || n_tokens < 0 || token_offset < 0)
    return fail(LCV_ERR_INVALID_ARG, "n_outer, n_tokens and token_offset must be >= 0");
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(LCV_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (!aligned(x, 16) || !aligned(dy, 16) || !aligned(dx, 16))
    return fail(LCV_ERR_INVALID_ARG, "x, dy and dx must be 16-byte aligned");
  if (!aligned(gamma, 16) || !aligned(dgamma, 4) || !aligned(workspace, 4))
    return fail(LCV_ERR_INVALID_ARG, "gamma must be 16-byte aligned, dgamma and workspace 4-byte aligned");
  if (grid != nullptr) {
    lcv_status st = check_grid(grid);
    if (st != LCV_OK) return st;
    const int64_t total = (int64_t)grid->T * grid->H * grid->W;
    if ((int64_t)token_offset + n_tokens > total)
      return fail(LCV_ERR_SHAPE, "tokens [%d, %lld) exceed the grid's %lld tokens", token_offset,
                  (long long)token_offset + n_tokens, (long long)total);
  } else if ((int64_t)token_offset + n_tokens >= (int64_t(1) << 31)) {
    return fail(LCV_ERR_UNSUPPORTED, "token_offset + n_tokens must be below 2^31");
  }
  if (n_outer > (int64_t)65535 * lcv::kPrologueBwdSlices)
    return fail(LCV_ERR_UNSUPPORTED, "n_outer above %lld is not supported", (long long)65535 * lcv::kPrologueBwdSlices);
  const int64_t need = lcv::prologue_bwd_workspace_floats(n_outer, n_tokens);
  if (static_scratch) {
    if (need > lcv::kNoAllocPartialFloats)
      return fail(LCV_ERR_UNSUPPORTED,
                  "n_outer %lld x n_tokens %d needs %lld scratch values; the static scratch holds %lld "
                  "(use lcv_qk_rmsnorm_rope3d_backward with a workspace)",
                  (long long)n_outer, n_tokens, (long long)need, (long long)lcv::kNoAllocPartialFloats);
    const hipError_t se = lcv::prologue_bwd_scratch(&workspace);
    if (se != hipSuccess) return hip_fail(se, "static scratch of the prologue backward");
  } else if (workspace_floats < need) {
    return fail(LCV_ERR_INVALID_ARG, "workspace holds %lld floats, %lld needed", (long long)workspace_floats,
                (long long)need);
  }
  const hipError_t e = lcv::launch_qk_prologue_bwd(
      static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(dy), gamma, eps, n_outer, n_tokens, token_offset,
      grid != nullptr, grid ? grid->H : 1, grid ? grid->W : 1, grid ? std::log2(grid->theta) : 0.f,
      static_cast<uint16_t*>(dx), dgamma, workspace, stream);
  if (e != hipSuccess) return hip_fail(e, "qk prologue backward launch");
  return ok();
}

}  // namespace

extern "C" {

int32_t lcv_abi_version(void) { return LCV_BSA_ABI_VERSION; }

const char* lcv_last_error(void) { return g_last_error.c_str(); }

lcv_status lcv_bsa_layout_query(const lcv_bsa_layout_params* params, lcv_bsa_layout_info* info) {
  lcv_status st = check_params(params);
  if (st != LCV_OK) return st;
  if (info == nullptr) return fail(LCV_ERR_NULL, "info is NULL");
  st = compute_info(params, info);
  if (st != LCV_OK) return st;
  return ok();
}

lcv_status lcv_bsa_build_layout(const lcv_bsa_layout_params* params, hipStream_t stream, lcv_bsa_layout** out) {
  if (out == nullptr) return fail(LCV_ERR_NULL, "out is NULL");
  *out = nullptr;
  lcv_status st = check_params(params);
  if (st != LCV_OK) return st;
  lcv_bsa_layout_info info;
  st = compute_info(params, &info);
  if (st != LCV_OK) return st;

  lcv_bsa_layout* h = new (std::nothrow) lcv_bsa_layout;
  if (h == nullptr) return fail(LCV_ERR_OOM, "host allocation failed");
  std::memset(h, 0, sizeof *h);
  h->info = info;
  hipError_t e = hipGetDevice(&h->device);
  if (e != hipSuccess) {
    delete h;
    return hip_fail(e, "hipGetDevice");
  }
  const int32_t n = info.n_blocks;
  h->dev.n_st = (n + lcv::kWaves - 1) / lcv::kWaves;
  h->dev.n_kg = (n + lcv::kWaves - 1) / lcv::kWaves;
  // one device allocation, carved into 256-byte aligned arrays
  const size_t nnz_alloc = info.nnz > 0 ? (size_t)info.nnz : 1;
  struct {
    int32_t** p;
    size_t count;
  } parts[] = {{&h->dev.row_ptr, (size_t)n + 1},         {&h->dev.col_idx, nnz_alloc},
               {&h->dev.st_cnt, (size_t)h->dev.n_st},    {&h->dev.st_ent, nnz_alloc},
               {&h->dev.st_order, (size_t)h->dev.n_st},  {&h->dev.kg_blk, (size_t)h->dev.n_kg * lcv::kWaves},
               {&h->dev.kg_cnt, (size_t)h->dev.n_kg},    {&h->dev.kg_off, (size_t)h->dev.n_kg + 1},
               {&h->dev.kg_ent, nnz_alloc},              {&h->dev.summary, 2}};
  size_t bytes = 0;
  for (auto& pt : parts) bytes += (pt.count * sizeof(int32_t) + 255) / 256 * 256;
  e = hipMalloc(&h->dev.block, bytes);
  if (e != hipSuccess) {
    lcv_bsa_layout_destroy(h);
    return fail(e == hipErrorOutOfMemory ? LCV_ERR_OOM : LCV_ERR_HIP, "hipMalloc of the layout: %s",
                hipGetErrorString(e));
  }
  size_t at = 0;
  for (auto& pt : parts) {
    *pt.p = reinterpret_cast<int32_t*>(static_cast<char*>(h->dev.block) + at);
    at += (pt.count * sizeof(int32_t) + 255) / 256 * 256;
  }
  const lcv::LayoutRule L = make_rule(params);
  e = lcv::launch_layout_build(L, h->dev, stream);
  int32_t summary[2] = {-1, -1};
  if (e == hipSuccess) e = hipMemcpyAsync(summary, h->dev.summary, sizeof summary, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    lcv_bsa_layout_destroy(h);
    return hip_fail(e, "layout build");
  }
  if (summary[0] != info.nnz || summary[1] < 0 || summary[1] > info.nnz) {
    lcv_bsa_layout_destroy(h);
    return fail(LCV_ERR_HIP, "layout build produced %d entries (expected %lld) and %d key-side entries", summary[0],
                (long long)info.nnz, summary[1]);
  }
  h->dev.kg_total = summary[1];
  *out = h;
  return ok();
}

lcv_status lcv_bsa_layout_get_info(const lcv_bsa_layout* layout, lcv_bsa_layout_info* info) {
  if (layout == nullptr || info == nullptr) return fail(LCV_ERR_NULL, "layout and info are required");
  *info = layout->info;
  return ok();
}

lcv_status lcv_bsa_layout_copy_csr(const lcv_bsa_layout* layout, int32_t* row_ptr, int32_t* col_idx,
                                   hipStream_t stream) {
  if (layout == nullptr || row_ptr == nullptr || col_idx == nullptr)
    return fail(LCV_ERR_NULL, "layout, row_ptr and col_idx are required");
  if (!aligned(row_ptr, 4) || !aligned(col_idx, 4)) return fail(LCV_ERR_INVALID_ARG, "int32 buffers must be 4-byte aligned");
  hipError_t e = hipMemcpyAsync(row_ptr, layout->dev.row_ptr, ((size_t)layout->info.n_blocks + 1) * sizeof(int32_t),
                                hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess && layout->info.nnz > 0)
    e = hipMemcpyAsync(col_idx, layout->dev.col_idx, (size_t)layout->info.nnz * sizeof(int32_t),
                       hipMemcpyDeviceToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "copy csr");
  return ok();
}

void lcv_bsa_layout_destroy(lcv_bsa_layout* layout) {
  if (layout == nullptr) return;
  (void)hipFree(layout->dev.block);
  delete layout;
}

lcv_status lcv_rope3d_apply(const void* x, void* y, int64_t n_outer, int32_t n_tokens, int32_t token_offset,
                            const lcv_rope3d_grid* grid, hipStream_t stream) {
  if (x == nullptr || y == nullptr) return fail(LCV_ERR_NULL, "x and y are required");
  if (n_outer < 0 || n_tokens < 0 || token_offset < 0)
    return fail(LCV_ERR_INVALID_ARG, "n_outer, n_tokens and token_offset must be >= 0");
  lcv_status st = check_grid(grid);
  if (st != LCV_OK) return st;
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(LCV_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
  const int64_t total = (int64_t)grid->T * grid->H * grid->W;
  if ((int64_t)token_offset + n_tokens > total)
    return fail(LCV_ERR_SHAPE, "tokens [%d, %lld) exceed the grid's %lld tokens", token_offset,
                (long long)token_offset + n_tokens, (long long)total);
  if (n_outer > (int64_t)65535 * 2) return fail(LCV_ERR_UNSUPPORTED, "n_outer above 131070 is not supported");
  const hipError_t e = lcv::launch_rope3d(static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), n_outer, n_tokens,
                                          token_offset, grid->H, grid->W, std::log2(grid->theta), stream);
  if (e != hipSuccess) return hip_fail(e, "rope3d launch");
  return ok();
}

lcv_status lcv_qk_rmsnorm_rope3d(const void* x, void* y, const float* gamma, float eps, int64_t n_outer,
                                 int32_t n_tokens, int32_t token_offset, const lcv_rope3d_grid* grid,
                                 hipStream_t stream) {
  if (x == nullptr || y == nullptr || gamma == nullptr) return fail(LCV_ERR_NULL, "x, y and gamma are required");
  if (n_outer < 0 || n_tokens < 0 || token_offset < 0)
    return fail(LCV_ERR_INVALID_ARG, "n_outer, n_tokens and token_offset must be >= 0");
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(LCV_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(LCV_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
  if (!aligned(gamma, 4)) return fail(LCV_ERR_INVALID_ARG, "gamma must be 4-byte aligned");
  if (grid != nullptr) {
    lcv_status st = check_grid(grid);
    if (st != LCV_OK) return st;
    const int64_t total = (int64_t)grid->T * grid->H * grid->W;
    if ((int64_t)token_offset + n_tokens > total)
      return fail(LCV_ERR_SHAPE, "tokens [%d, %lld) exceed the grid's %lld tokens", token_offset,
                  (long long)token_offset + n_tokens, (long long)total);
  } else if ((int64_t)token_offset + n_tokens >= (int64_t(1) << 31)) {
    return fail(LCV_ERR_UNSUPPORTED, "token_offset + n_tokens must be below 2^31");
  }
  if (n_outer > (int64_t)65535 * 2) return fail(LCV_ERR_UNSUPPORTED, "n_outer above 131070 is not supported");
  const hipError_t e = lcv::launch_qk_prologue(
      static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), gamma, eps, n_outer, n_tokens, token_offset,
      grid != nullptr, grid ? grid->H : 1, grid ? grid->W : 1, grid ? std::log2(grid->theta) : 0.f, stream);
  if (e != hipSuccess) return hip_fail(e, "qk prologue launch");
  return ok();
}

int64_t lcv_qk_rmsnorm_rope3d_backward_workspace(int64_t n_outer, int32_t n_tokens) {
  if (n_outer < 0 || n_tokens < 0) return -1;
  return lcv::prologue_bwd_workspace_floats(n_outer, n_tokens);
}

lcv_status lcv_qk_rmsnorm_rope3d_backward(const void* x, const void* dy, const float* gamma, float eps,
                                          int64_t n_outer, int32_t n_tokens, int32_t token_offset,
                                          const lcv_rope3d_grid* grid, void* dx, float* dgamma, float* workspace,
                                          int64_t workspace_floats, hipStream_t stream) {
  if (workspace == nullptr) return fail(LCV_ERR_NULL, "workspace is required");
  return prologue_bwd_common(x, dy, gamma, eps, n_outer, n_tokens, token_offset, grid, dx, dgamma, workspace,
                             workspace_floats, false, stream);
}

lcv_status lcv_qk_rmsnorm_rope3d_backward_noalloc(const void* x, const void* dy, const float* gamma, float eps,
                                                  int64_t n_outer, int32_t n_tokens, int32_t token_offset,
                                                  const lcv_rope3d_grid* grid, void* dx, float* dgamma,
                                                  hipStream_t stream) {
  return prologue_bwd_common(x, dy, gamma, eps, n_outer, n_tokens, token_offset, grid, dx, dgamma, nullptr, 0, true,
                             stream);
}

lcv_status lcv_attn_merge(const void* const* outs, const float* const* lses, int32_t n_parts, int64_t rows,
                          void* out, float* lse, hipStream_t stream) {
  if (outs == nullptr || lses == nullptr || out == nullptr) return fail(LCV_ERR_NULL, "outs, lses and out are required");
  if (n_parts < 1 || n_parts > lcv::kMaxMergeParts)
    return fail(LCV_ERR_INVALID_ARG, "n_parts must be in [1, %d] (got %d)", lcv::kMaxMergeParts, n_parts);
  if (rows < 0 || rows > (int64_t(1) << 40)) return fail(LCV_ERR_INVALID_ARG, "rows must be in [0, 2^40]");
  lcv::MergeParams p;
  std::memset(&p, 0, sizeof p);
  for (int i = 0; i < n_parts; ++i) {
    if (outs[i] == nullptr || lses[i] == nullptr) return fail(LCV_ERR_NULL, "part %d has a NULL pointer", i);
    if (!aligned(outs[i], 16)) return fail(LCV_ERR_INVALID_ARG, "bf16 tensors must be 16-byte aligned");
    if (!aligned(lses[i], 4)) return fail(LCV_ERR_INVALID_ARG, "lse tensors must be 4-byte aligned");
    p.outs[i] = static_cast<const uint16_t*>(outs[i]);
    p.lses[i] = lses[i];
  }
  if (!aligned(out, 16)) return fail(LCV_ERR_INVALID_ARG, "bf16 tensors must be 16-byte aligned");
  if (lse != nullptr && !aligned(lse, 4)) return fail(LCV_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (rows * 8 / 256 >= (int64_t(1) << 31)) return fail(LCV_ERR_UNSUPPORTED, "rows = %lld is too large", (long long)rows);
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.rows = rows;
  p.n_parts = n_parts;
  hipError_t e = lcv::launch_attn_merge(p, stream);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return ok();
}

lcv_status lcv_cross_attention(const void* q, const void* k, const void* v, int32_t batch, int32_t heads,
                               int32_t n_q, int32_t kv_len, const int32_t* kv_lens, void* out, float* lse,
                               hipStream_t stream) {
  if (batch < 1 || heads < 1) return fail(LCV_ERR_INVALID_ARG, "batch and heads must be >= 1 (got %d, %d)", batch, heads);
  if (n_q < 0 || kv_len < 0) return fail(LCV_ERR_INVALID_ARG, "n_q and kv_len must be >= 0 (got %d, %d)", n_q, kv_len);
  if (n_q > 0 && (q == nullptr || out == nullptr)) return fail(LCV_ERR_NULL, "q and out are required when n_q > 0");
  if (n_q > 0 && kv_len > 0 && (k == nullptr || v == nullptr))
    return fail(LCV_ERR_NULL, "k and v are required when n_q > 0 and kv_len > 0");
  for (const void* t : {q, k, v, static_cast<const void*>(out)})
    if (!aligned(t, 16)) return fail(LCV_ERR_INVALID_ARG, "bf16 tensors must be 16-byte aligned");
  if (lse != nullptr && !aligned(lse, 4)) return fail(LCV_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (kv_lens != nullptr && !aligned(kv_lens, 4)) return fail(LCV_ERR_INVALID_ARG, "kv_lens must be 4-byte aligned");
  const int64_t bh = (int64_t)batch * heads;
  const int32_t n_blocks = (int32_t)(((int64_t)n_q + 63) / 64);
  const int32_t n_st = (n_blocks + lcv::kWaves - 1) / lcv::kWaves;
  const int64_t n_items = bh * n_st;
  if (n_items >= (int64_t(1) << 31) - 8 || bh >= (int64_t(1) << 31))
    return fail(LCV_ERR_UNSUPPORTED, "batch*heads*workgroups = %lld is too large", (long long)n_items);
  if (n_q == 0) return ok();
  lcv::FwdParams p;
  std::memset(&p, 0, sizeof p);
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.N = n_q;
  p.C = 0;
  p.n_blocks = n_blocks;
  p.q_row0 = 0;
  p.q_rows = n_q;
  p.q_end = n_q;
  p.kv_split = 0;
  p.st_first = 0;
  p.n_st_active = n_st;
  p.n_items = (int32_t)n_items;
  p.bh_count = (int32_t)bh;
  p.st_order = nullptr;   // every list is the whole text: equal lengths
  p.flags = 0;
  p.kv_len = kv_len;
  p.kv_lens = kv_lens;
  p.heads = heads;
  // With at most kCrossResidentBlocks text blocks the text stays in LDS: about
  // LCV_CROSS_FWD_WORKGROUPS workgroups (one per compute unit), each streaming a range of
  // query blocks past its head's text.  The ranges of a head are as equal as whole blocks
  // allow (the wavefronts of a workgroup share its range block by block), and at least as
  // long as the workgroup has wavefronts.
  if ((int64_t)kv_len <= (int64_t)lcv::kCrossResidentBlocks * 64) {
    constexpr int64_t kRound = 2 * lcv::kWaves;
    const int64_t rounds = (n_blocks + kRound - 1) / kRound;
    int64_t parts = (LCV_CROSS_FWD_WORKGROUPS + bh - 1) / bh;
    parts = parts < rounds ? parts : rounds;
    const int64_t per = (n_blocks + parts - 1) / parts;
    parts = (n_blocks + per - 1) / per;
    p.q_per_part = (int32_t)per;
    p.n_st_active = (int32_t)parts;
    p.n_items = (int32_t)(bh * parts);
  }
  hipError_t e = lcv::launch_cross_fwd(p, stream);
  if (e != hipSuccess) return hip_fail(e, "cross-attention launch");
  return ok();
}

int64_t lcv_cross_attention_backward_workspace(int32_t batch, int32_t heads, int32_t n_q, int32_t kv_len) {
  if (batch < 1 || heads < 1 || n_q < 0 || kv_len < 0) return -1;
  const CrossBwdPlan pl = cross_bwd_plan((int64_t)batch * heads, n_q, kv_len);
  return pl.workspace_floats;
}

lcv_status lcv_cross_attention_backward(const void* q, const void* k, const void* v, const void* out,
                                        const float* lse, const void* dout, int32_t batch, int32_t heads, int32_t n_q,
                                        int32_t kv_len, const int32_t* kv_lens, void* dq, void* dk, void* dv,
                                        float* workspace, int64_t workspace_floats, hipStream_t stream) {
  if (batch < 1 || heads < 1) return fail(LCV_ERR_INVALID_ARG, "batch and heads must be >= 1 (got %d, %d)", batch, heads);
  if (n_q < 0 || kv_len < 0) return fail(LCV_ERR_INVALID_ARG, "n_q and kv_len must be >= 0 (got %d, %d)", n_q, kv_len);
  if (n_q > 0 && (q == nullptr || out == nullptr || lse == nullptr || dout == nullptr || dq == nullptr))
    return fail(LCV_ERR_NULL, "q, out, lse, dout and dq are required when n_q > 0");
  if (kv_len > 0 && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr))
    return fail(LCV_ERR_NULL, "k, v, dk and dv are required when kv_len > 0");
  for (const void* t : {q, k, v, out, dout, static_cast<const void*>(dq), static_cast<const void*>(dk),
                        static_cast<const void*>(dv)})
    if (!aligned(t, 16)) return fail(LCV_ERR_INVALID_ARG, "bf16 tensors must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(workspace, 16))
    return fail(LCV_ERR_INVALID_ARG, "lse must be 4-byte and workspace 16-byte aligned");
  if (kv_lens != nullptr && !aligned(kv_lens, 4)) return fail(LCV_ERR_INVALID_ARG, "kv_lens must be 4-byte aligned");
  const int64_t bh = (int64_t)batch * heads;
  const CrossBwdPlan pl = cross_bwd_plan(bh, n_q, kv_len);
  if (pl.workspace_floats > 0 && workspace == nullptr) return fail(LCV_ERR_NULL, "workspace is required");
  if (workspace_floats < pl.workspace_floats)
    return fail(LCV_ERR_INVALID_ARG, "workspace holds %lld values, %lld are needed", (long long)workspace_floats,
                (long long)pl.workspace_floats);
  const int64_t items = bh * (pl.n_st > pl.n_kg ? pl.n_st : pl.n_kg);
  if (bh >= (int64_t(1) << 31) || items >= (int64_t(1) << 31) - 8 || bh * n_q * 8 >= (int64_t(1) << 40) ||
      bh * kv_len * 8 >= (int64_t(1) << 40))
    return fail(LCV_ERR_UNSUPPORTED, "batch * heads = %lld is too large", (long long)bh);
  if (n_q == 0 && kv_len == 0) return ok();
  hipError_t e;
  lcv::BwdParams p;
  std::memset(&p, 0, sizeof p);
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.out = static_cast<const uint16_t*>(out);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.qs = reinterpret_cast<uint16_t*>(workspace);
  p.lse2 = workspace + 32 * bh * n_q;
  p.delta = p.lse2 + bh * n_q;
  p.fold_l = reinterpret_cast<uint2*>(p.delta + bh * n_q);
  p.fold_d = p.fold_l + bh * n_q;
  p.cross = true;
  p.part_dk = workspace + pl.part_offset;
  p.part_dv = p.part_dk + pl.part_floats;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.bh_rows = bh * n_q;
  p.N = n_q;
  p.C = 0;
  p.n_blocks = pl.n_q_blocks;
  p.n_st = pl.n_st;
  p.n_kg = pl.n_kg;
  p.bh = (int32_t)bh;
  p.kv_len = kv_len;
  p.kv_lens = kv_lens;
  p.heads = heads;
  p.n_kv_blocks = pl.n_kv_blocks;
  p.q_chunk = pl.q_chunk;
  p.n_chunks = pl.n_chunks;
  p.q_parts = pl.q_parts;
  p.q_per_part = pl.q_per_part;
  e = lcv::launch_bsa_bwd(p, stream);
  if (e != hipSuccess) return hip_fail(e, "cross-attention backward launch");
  return ok();
}

int64_t lcv_bsa_backward_workspace(int32_t batch, int32_t heads, int32_t n_tokens) {
  if (batch < 1 || heads < 1 || n_tokens < 1) return -1;
  return kBwdRowFloats * batch * heads * (int64_t)n_tokens;
}

lcv_status lcv_bsa_backward(const void* q, const void* k, const void* v, const void* out, const float* lse,
                            const void* dout, int32_t batch, int32_t heads, const lcv_bsa_layout* layout,
                            int32_t cond_len, void* dq, void* dk, void* dv, float* workspace, int64_t workspace_floats,
                            hipStream_t stream) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || lse == nullptr || dout == nullptr ||
      dq == nullptr || dk == nullptr || dv == nullptr || workspace == nullptr || layout == nullptr)
    return fail(LCV_ERR_NULL, "every tensor, the workspace and the layout are required");
  if (batch < 1 || heads < 1) return fail(LCV_ERR_INVALID_ARG, "batch and heads must be >= 1");
  if (cond_len != layout->info.cond_len)
    return fail(LCV_ERR_LAYOUT_MISMATCH, "cond_len %d differs from the layout's %d", cond_len, layout->info.cond_len);
  for (const void* t : {q, k, v, out, dout, static_cast<const void*>(dq), static_cast<const void*>(dk),
                        static_cast<const void*>(dv)})
    if (!aligned(t, 16)) return fail(LCV_ERR_INVALID_ARG, "bf16 tensors must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(workspace, 16))
    return fail(LCV_ERR_INVALID_ARG, "lse must be 4-byte and workspace 16-byte aligned");
  const int64_t bh = (int64_t)batch * heads;
  const int32_t N = layout->info.n_tokens;
  const int64_t items = bh * (layout->dev.n_st > layout->dev.n_kg ? layout->dev.n_st : layout->dev.n_kg);
  if (bh >= (int64_t(1) << 31) || items >= (int64_t(1) << 31) - 8 || bh * N * 8 >= (int64_t(1) << 40))
    return fail(LCV_ERR_UNSUPPORTED, "batch * heads = %lld is too large", (long long)bh);
  const int64_t need = kBwdRowFloats * bh * N;
  if (workspace_floats < need)
    return fail(LCV_ERR_INVALID_ARG, "workspace holds %lld values, %lld are needed", (long long)workspace_floats,
                (long long)need);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != layout->device)
    return fail(LCV_ERR_INVALID_ARG, "layout was built on device %d, current device is %d", layout->device, dev);
  lcv::BwdParams p;
  std::memset(&p, 0, sizeof p);
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.out = static_cast<const uint16_t*>(out);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.qs = reinterpret_cast<uint16_t*>(workspace);
  p.lse2 = workspace + 32 * bh * N;
  p.delta = p.lse2 + bh * N;
  p.fold_l = reinterpret_cast<uint2*>(p.delta + bh * N);
  p.fold_d = p.fold_l + bh * N;
  p.cross = false;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.row_ptr = layout->dev.row_ptr;
  p.st_cnt = layout->dev.st_cnt;
  p.st_ent = layout->dev.st_ent;
  p.kg_blk = layout->dev.kg_blk;
  p.kg_cnt = layout->dev.kg_cnt;
  p.kg_off = layout->dev.kg_off;
  p.kg_ent = layout->dev.kg_ent;
  p.bh_rows = bh * N;
  p.N = N;
  p.C = cond_len;
  p.n_blocks = layout->info.n_blocks;
  p.n_st = layout->dev.n_st;
  p.n_kg = layout->dev.n_kg;
  p.bh = (int32_t)bh;
  e = lcv::launch_bsa_bwd(p, stream);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return ok();
}

lcv_status lcv_bsa_forward(const void* q, const void* k, const void* v, int32_t batch, int32_t heads,
                           const lcv_bsa_layout* layout, int32_t cond_len, uint32_t flags,
                           const lcv_rope3d_grid* grid, void* out, float* lse, hipStream_t stream) {
  FwdArgs a{q, k, v, nullptr, nullptr, out, lse, false};
  return forward_common(a, batch, heads, layout, cond_len, flags, grid, stream);
}

lcv_status lcv_bsa_forward_rows(const void* q, const void* k, const void* v, int32_t batch, int32_t heads,
                                const lcv_bsa_layout* layout, int32_t cond_len, uint32_t flags,
                                const lcv_rope3d_grid* grid, int32_t row_begin, int32_t row_end, void* out, float* lse,
                                hipStream_t stream) {
  if (layout != nullptr && (row_begin < 0 || row_end < row_begin || row_end > layout->info.n_tokens))
    return fail(LCV_ERR_INVALID_ARG, "row range [%d, %d) is not inside [0, %d]", row_begin, row_end,
                layout->info.n_tokens);
  if (layout != nullptr && row_begin == row_end) return ok();   // empty range: nothing to read or write
  FwdArgs a{q, k, v, nullptr, nullptr, out, lse, false};
  a.row_begin = row_begin;
  a.row_end = row_end;
  return forward_common(a, batch, heads, layout, cond_len, flags, grid, stream);
}

lcv_status lcv_bsa_forward_cached(const void* q_noise, const void* k_noise, const void* v_noise, const void* k_cond,
                                  const void* v_cond, int32_t batch, int32_t heads, const lcv_bsa_layout* layout,
                                  int32_t cond_len, uint32_t flags, const lcv_rope3d_grid* grid, void* out_noise,
                                  float* lse_noise, hipStream_t stream) {
  FwdArgs a{q_noise, k_noise, v_noise, k_cond, v_cond, out_noise, lse_noise, true};
  return forward_common(a, batch, heads, layout, cond_len, flags, grid, stream);
}

}  // extern "C"
