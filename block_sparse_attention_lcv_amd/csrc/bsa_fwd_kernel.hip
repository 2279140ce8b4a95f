// Block-sparse 3D self-attention forward for gfx950 (MI355X).
//
// Method (what is computed): softmax attention of 64-token query blocks over the key
// blocks their layout row lists -- dense inside each attended block pair, sparse between
// blocks (zhichai.net post, section "Block Sparse Attention"; longcat-video-rs page,
// section 03 "Block-Sparse & Multi-Audio") -- with condition queries restricted to
// condition keys (myzaker article, technical principles: block attention with a KV cache)
// and the partitioned 3D-RoPE applied to Q and K as they are loaded (longcat-video-rs
// page, section 03 "Partitioned 3D-RoPE").
//
// Mapping onto CDNA4:
//  * One workgroup = kWaves wavefronts = kWaves consecutive query blocks of one
//    (batch, head).  Each wavefront keeps its 64 query rows resident in VGPRs as bf16
//    MFMA operands (RoPE applied once at load).
//  * The workgroup walks the union of its query blocks' key-block rows (built with the
//    layout, each entry carrying a per-wavefront membership mask).  Each K and V block
//    (64 x 64 bf16) is staged once into LDS for all wavefronts by direct global -> LDS
//    copies: block e+1 is copied into the other stage while block e is processed (K RoPE,
//    when fused, goes through registers instead); one barrier per entry.  Each SIMD runs
//    two wavefronts of different workgroups, whose matrix-core and vector phases overlap.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K from LDS as the A operand, Q as B), so
//    each lane owns one query column: row statistics need only the partner lane l^32.
//  * Online softmax in the log2 domain with a per-row reference that only moves when a half
//    block's probabilities grow too large (lazy rescaling), and then to a multiple of 64,
//    so that it stays 0 for rows whose scores stay near 0; a wavefront with some nonzero
//    reference subtracts it from its scores with the vector ALU.  The common score costs one
//    v_exp_f32 and half a conversion on the vector ALU; the row sums of the probabilities
//    are products on the matrix cores (a 0/1 selection operand against the P operands).
//    Each row's decisions depend on that row alone, so results do not depend on which other
//    rows share the wavefront (the cached call reproduces the full call bit for bit).
//  * O^T += V^T P^T with the same MFMA: P (bf16) comes straight from the S^T registers, V^T
//    operands come from the row-major V tile through ds_read_b64_tr_b16 transposing reads.
//  * Workgroups are numbered so that each XCD (blockIdx % 8 on MI355X) receives a
//    contiguous range of work items, i.e. whole heads: their shared global key blocks stay
//    in that XCD's L2.
#include <type_traits>

#include "attn_tile.h"
#include "lcv_internal.h"

namespace lcv {
namespace {

typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 64 * kWaves;
#ifndef LCV_WAVES_PER_SIMD
#define LCV_WAVES_PER_SIMD 2
#endif
constexpr int kWavesPerSimd = LCV_WAVES_PER_SIMD;  // occupancy the register budget is sized for
// Lazy rescaling with a coarse reference.  A row's reference moves only when its
// probabilities in one 32-key half sum past 2^40, and then to the multiple of 64 nearest the
// row's largest score, which so lies within 32 of it (a row's first block always sets it).
// Every probability therefore stays below 2^40 and a row's sum below 2^56, far inside fp32
// and bf16, the largest probability of a row is at least 2^-32, and a rescale multiplies by
// an exact power of two.  Both lanes of a row get the row's half sum from the matrix cores
// (half_row_sum), so the test needs no partner exchange.
constexpr float kRescaleLimit = 1099511627776.0f;   // 2^40

// Vector instructions of a half's softmax placed after each of the 8 MFMAs it is interleaved
// with (about 52 per half: 32 exponentials, 16 conversions, the tests; 7 measured slightly
// faster than 5, 6, 8 or 9)
#ifndef LCV_VALU_PER_MFMA
#define LCV_VALU_PER_MFMA 7
#endif
constexpr int kValuPerMfma = LCV_VALU_PER_MFMA;
__device__ __forceinline__ float coarse_ref(float m) { return 64.0f * __builtin_rintf(m * (1.0f / 64.0f)); }

__device__ __forceinline__ float partner(float x) { return __shfl_xor(x, 32, 64); }

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Coords {
  uint32_t t, y, x;
};

__device__ __forceinline__ Coords token_coords(uint32_t n, const FwdParams& P) {
  Coords c;
  c.t = fast_div(n, P.div_hw);
  const uint32_t rem = n - c.t * P.div_hw.d;
  c.y = fast_div(rem, P.div_w);
  c.x = rem - c.y * P.div_w.d;
  return c;
}

// Rotate the 8-channel chunk `c` of a token with cos/sin from the LDS table.
__device__ __forceinline__ u32x4 rope_chunk(u32x4 raw, int c, const Coords& xyz, const float2* tab,
                                            const FwdParams& P) {
  int axis, width, p0;
  chunk_section(c, axis, width, p0);
  const int base = (axis == 0) ? (int)xyz.t * 8 + p0
                   : (axis == 1) ? 8 * P.T + (int)xyz.y * 12 + p0
                                 : 8 * P.T + 12 * P.H + (int)xyz.x * 12 + p0;
#pragma unroll
  for (int e = 0; e < 4; ++e) raw[e] = rotate_pair(raw[e], tab[base + e]);
  return raw;
}

// Staging of K/V block j into an LDS stage.  The 8 KB tile is moved as 8 wave-loads of
// 1 KB (8 rows); wavefront w issues loads u = w*kLoadsPerWave + c.  In load u, lane l carries
// row 8u + l/8 and lands at LDS byte 1024u + 16l, i.e. physical chunk l%8 of that row, which
// holds logical chunk (l%8) ^ swz(8u + l/8) under the swizzle of tile_off.  The copies are
// buffer loads straight into LDS: the block's first row is the (wave-uniform) base of a
// buffer resource built with scalar instructions, each lane's byte offset inside the block
// is fixed for the whole walk (computed once), and the resource's size stops at the end of
// the keys, so rows past it read zeros (their scores are masked and their probabilities are
// zero).  The vector ALU computes no address per copy.
constexpr int kLoadsPerWave = 8 / kWaves;
static_assert(8 % kWaves == 0, "a tile is 8 wave-loads");

typedef __attribute__((address_space(4))) const int32_t const_i32;

// s_waitcnt immediate that waits for every LDS operation only (vmcnt 63 in bits 3:0 and
// 15:14, expcnt 7 in bits 6:4, lgkmcnt 0 in bits 11:8)
constexpr int kWaitLdsOnly = 0xC07F;   // scalar loads of the lists

// Buffer resource over `rows` key rows of 128 bytes from the byte address `base`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(uint64_t base, int rows) {
  return uniform_rsrc(base, rows * 128);
}

// Lane offset (bytes) of load c inside a K or V block: row 8u + l/8, physical chunk l%8
// holding logical chunk (l%8) ^ swz(row).
__device__ __forceinline__ uint32_t stage_lane_offset(int wave, int lane, int c) {
  const int u = wave * kLoadsPerWave + c;
  const int row = 8 * u + (lane >> 3);
  return (uint32_t)(row * 128 + 16 * ((lane & 7) ^ swz(row)));
}

// Where the rows of one (batch, head)'s keys and values live, as byte addresses of key row 0
// (wave-uniform, computed once): key row `key` is at cond + 128 key when key < split (the
// condition cache of the cached call), else at noise + 128 key.  Self-attention: the
// [BH, N, 64] tensors (the noise tensor of the cached call holds rows [split, N), so its
// address is taken split rows early); cross-attention: the text tensor [BH, kv_len, 64].
struct KvSrc {
  uint64_t k_cond, v_cond, k_noise, v_noise;
  int split;      // 0 unless cached
  int key_end;    // keys [0, key_end) exist; rows past it read zeros (the K rows rotated in
                  // the kernel: the last row)
};

template <bool CACHED, bool CROSS>
__device__ __forceinline__ KvSrc kv_src(const FwdParams& P, int bh, int key_end) {
  KvSrc s;
  s.key_end = key_end;
  s.split = CACHED ? P.kv_split : 0;
  const int64_t rows = CROSS ? P.kv_len : P.N - s.split;            // rows per (batch, head) of the noise tensor
  const int64_t noise0 = (int64_t)bh * rows - s.split;              // its row index of key 0
  s.k_noise = (uint64_t)(uintptr_t)P.k + (uint64_t)(noise0 * 128);
  s.v_noise = (uint64_t)(uintptr_t)P.v + (uint64_t)(noise0 * 128);
  s.k_cond = CACHED ? (uint64_t)(uintptr_t)P.k_cond + (uint64_t)((int64_t)bh * s.split * 128) : 0;
  s.v_cond = CACHED ? (uint64_t)(uintptr_t)P.v_cond + (uint64_t)((int64_t)bh * s.split * 128) : 0;
  return s;
}

// Row `key` (clamped to key_end - 1) of K (is_k) or V, 16-byte chunk `chunk`; row0 is the
// first key of the lane's 8-row group (wave-uniform): the source tensor is chosen per group,
// per lane only in the group that holds the condition boundary.
template <bool CACHED>
__device__ __forceinline__ const uint16_t* kv_row(const KvSrc& s, bool is_k, int row0, int key, int chunk) {
  key = key < s.key_end ? key : s.key_end - 1;
  uint64_t base = is_k ? s.k_noise : s.v_noise;
  if constexpr (CACHED) {
    if (row0 < s.split) {
      base = is_k ? s.k_cond : s.v_cond;
      if (key >= s.split) base = is_k ? s.k_noise : s.v_noise;
    }
  }
  return reinterpret_cast<const uint16_t*>(base + (uint64_t)key * 128 + 16 * chunk);
}

// Issue the asynchronous copies of block j into a stage's K and V tiles (V always, K too
// unless K is rotated on the way); K chunks to be rotated are loaded into kreg.  In the cached
// call a block lies in the condition cache, in the noise tensor, or (the block holding the
// boundary) in both: then each source is copied by the lanes whose rows it holds.
template <bool ROPE_K, bool CACHED>
__device__ __forceinline__ void stage_issue(const KvSrc& src, unsigned char* kdst, unsigned char* vdst, int j, int wave,
                                            int lane, const uint32_t (&voff)[kLoadsPerWave],
                                            u32x4 (&kreg)[kLoadsPerWave]) {
  const int row0 = 64 * j;
  // copies from the tensors whose key row 0 is at kbase / vbase, rows below `limit`, by the
  // lanes for which on(c) holds
  auto issue = [&](uint64_t kbase, uint64_t vbase, int limit, auto&& on) __attribute__((always_inline)) {
    int rows = limit - row0;
    rows = rows < 0 ? 0 : (rows > 64 ? 64 : rows);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vbase + (uint64_t)row0 * 128, rows);
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kbase + (uint64_t)row0 * 128, rows);
#pragma unroll
    for (int c = 0; c < kLoadsPerWave; ++c) {
      const int u = wave * kLoadsPerWave + c;
      if (on(c)) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vdst + 1024 * u), 16, voff[c], 0, 0, 0);
        if constexpr (!ROPE_K)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kdst + 1024 * u), 16, voff[c], 0, 0, 0);
      }
    }
  };
  auto all = [](int) { return true; };
  if constexpr (!CACHED) {
    issue(src.k_noise, src.v_noise, src.key_end, all);
  } else {
    if (row0 + 64 <= src.split) {
      issue(src.k_cond, src.v_cond, src.split, all);
    } else if (row0 >= src.split) {
      issue(src.k_noise, src.v_noise, src.key_end, all);
    } else {
      auto key = [&](int c) { return row0 + 8 * (wave * kLoadsPerWave + c) + (lane >> 3); };
      issue(src.k_cond, src.v_cond, src.split, [&](int c) { return key(c) < src.split; });
      issue(src.k_noise, src.v_noise, src.key_end, [&](int c) { return key(c) >= src.split; });
    }
  }
  if constexpr (ROPE_K) {
#pragma unroll
    for (int c = 0; c < kLoadsPerWave; ++c) {
      const int u = wave * kLoadsPerWave + c;
      const int gch = (lane & 7) ^ swz(8 * u + (lane >> 3));
      const int key = row0 + 8 * u + (lane >> 3);
      kreg[c] = *reinterpret_cast<const u32x4*>(kv_row<CACHED>(src, true, row0 + 8 * u, key, gch));
    }
  }
}

// Rotate the K chunks loaded into kreg and write them to the stage (fused K RoPE only).
__device__ __forceinline__ void stage_store_k(const FwdParams& P, unsigned char* stage, int j, int wave, int lane,
                                              const float2* tab, const u32x4 (&kreg)[kLoadsPerWave]) {
#pragma unroll
  for (int c = 0; c < kLoadsPerWave; ++c) {
    const int u = wave * kLoadsPerWave + c;
    const int gch = (lane & 7) ^ swz(8 * u + (lane >> 3));
    const int key = 64 * j + 8 * u + (lane >> 3);
    u32x4 kv = kreg[c];
    if (key < P.N) kv = rope_chunk(kv, gch, token_coords((uint32_t)key, P), tab, P);
    *reinterpret_cast<u32x4*>(stage + 1024 * u + 16 * lane) = kv;
  }
}

// p = 2^(s + shift) for the 16 scores of query tile qt held by this lane in one 32-key half
// (the scores already taken relative to the row's reference m), packed to bf16 as the B
// operands of the two 16-key P*V steps: pb[h] holds keys 16h + 8(lane/32) .. +7 of query
// lane % 32.
template <bool SHIFT>
__device__ __forceinline__ void probs(const f32x16& s, float shift, bf16x8 (&pb)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    bf16x2 w[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      float x0 = s[8 * h + 2 * e2], x1 = s[8 * h + 2 * e2 + 1];
      if (SHIFT) {
        x0 += shift;
        x1 += shift;
      }
      const f32x2_t p = {__builtin_amdgcn_exp2f(x0), __builtin_amdgcn_exp2f(x1)};
      w[e2] = __builtin_convertvector(p, bf16x2);
    }
    pb[h] = __builtin_shufflevector(__builtin_shufflevector(w[0], w[1], 0, 1, 2, 3),
                                    __builtin_shufflevector(w[2], w[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// The 0/1 operand of half_row_sum: lane l supplies row l % 16, keys-group l / 16 of the
// 16 x 32 A operand of v_mfma_f32_16x16x32_bf16, and a row of even (odd) index selects the
// key groups of even (odd) index.
__device__ __forceinline__ bf16x8 row_sum_selector(int lane) {
  const uint32_t one2 = 0x3F803F80u;   // two bf16 ones
  const uint32_t v = ((lane & 1) == ((lane >> 4) & 1)) ? one2 : 0u;
  return __builtin_bit_cast(bf16x8, u32x4{v, v, v, v});
}

// Sum of the rounded probabilities of one 32-key half for the lane's query row, on the
// matrix cores.  Read as the B operand of v_mfma_f32_16x16x32_bf16 (lane l: column l % 16,
// key group l / 16), pb[h] holds query n = l % 16 in groups 0 and 2 (keys 0-7 and 8-15 of
// the step) and query n + 16 in groups 1 and 3; so with the selector as A, result rows of even
// index hold the sum of query l % 16 over both steps and odd rows that of query l % 16 + 16.
// Lane l reads its own query l % 32 from result row 0 (l % 32 < 16, upper = false) or 1.
// Both lanes of a query read the same sum.
__device__ __forceinline__ float half_row_sum(const bf16x8 (&pb)[2], const bf16x8& sel, bool upper) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pb[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pb[1], acc, 0, 0, 0);
  return upper ? acc[1] : acc[0];
}

// The attention walk of one workgroup.  CROSS: cross-attention of the video queries over
// text keys/values [BH, kv_len, 64]: every query block attends every text block (dense, no
// RoPE, no condition rule), keys past the batch item's text length are masked.  RESIDENT
// (cross-attention with at most kCrossResidentBlocks text blocks): 2 * kWaves wavefronts
// hold the head's whole text K and V in LDS, loaded once, and each streams a range of query
// blocks past it on its own (no copies, no barriers after the load); otherwise kWaves
// wavefronts walk one workgroup list (or, CROSS, every text block) through a two-stage K/V
// ring.
template <bool ROPE_Q, bool ROPE_K, bool CACHED, bool CROSS, bool RESIDENT>
__device__ __forceinline__ void fwd_body(const FwdParams& P) {
  static_assert(!CROSS || (!ROPE_Q && !ROPE_K && !CACHED), "cross-attention has no RoPE and no cache");
  static_assert(!RESIDENT || CROSS, "only the cross-attention keeps its keys resident");
  // LDS: the K and V tiles of stages 0 and 1 are four separate variables, so the compiler
  // can tell that reads of one stage do not depend on the global -> LDS copies into the
  // other (with one shared array it makes those reads wait for every copy in flight).  The
  // resident walk keeps the K and V tiles of text block j at tiles 2j and 2j + 1 of lds_k0,
  // so that the lane offsets carry the block and the tile bases fit the LDS instructions'
  // immediate offsets.
  constexpr int kBytes0 = RESIDENT ? 2 * kCrossResidentBlocks * kTileBytes : kTileBytes;
  constexpr int kBytes1 = RESIDENT ? 16 : kTileBytes;
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k0[kBytes0];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k1[kBytes1];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v0[kBytes1];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v1[kBytes1];
  // cos/sin table of the fused RoPE (its own variable, so that the compiler can tell its
  // writes apart from the copies into the stages)
  __shared__ __attribute__((aligned(16))) float2 lds_tab[(ROPE_Q || ROPE_K) ? kMaxRopeEntries : 1];
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int l32 = lane & 31;

  // ---- work item (a (batch, head) and a workgroup list of 4 query blocks): XCD x (=
  // blockIdx % 8) runs the x-th contiguous eighth of the items, head after head, so that the
  // key blocks its workgroups share stay in its L2; inside a head the lists come in the
  // layout's work order (longest first, in runs of consecutive lists).  The hardware starts
  // each workgroup as a slot frees up, so the longest lists of a head go first and the
  // shortest fill the end.
  // The resident walk's items are (batch, head, range of q_per_part query blocks), the
  // ranges counted by n_st_active.
  const int per_xcd = (int)(gridDim.x >> 3);
  const int item = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (item >= P.n_items) return;
  const int bh = item / P.n_st_active;
  const int level = item - bh * P.n_st_active;
  const int st = P.st_order != nullptr ? P.st_order[level] : P.st_first + level;
  // keys [0, key_end) exist: the sequence (self-attention) or the batch item's text length
  int key_end = P.N;
  if constexpr (CROSS) {
    key_end = P.kv_len;
    if (P.kv_lens != nullptr) {
      const int len = P.kv_lens[bh / P.heads];
      key_end = len < 0 ? 0 : (len < P.kv_len ? len : P.kv_len);
    }
    key_end = __builtin_amdgcn_readfirstlane(key_end);
  }
  const KvSrc kvs = kv_src<CACHED, CROSS>(P, bh, key_end);

  // the workgroup's list: layout-built (self-attention), or every text block for all four
  // wavefronts (cross-attention)
  const const_i32* ents = CROSS ? nullptr : (const const_i32*)P.st_ent + P.row_ptr[st * kWaves];
  const int cnt = CROSS ? (key_end + 63) >> 6 : P.st_cnt[st];
  auto entry = [&](int e) __attribute__((always_inline)) {
    if constexpr (CROSS)
      return (e << 8) | ((1 << kWaves) - 1);
    else
      return (int)ents[e];
  };

  // List entries are wave-uniform (SGPRs, scalar loads): entry e+1 is known when step e
  // starts (its block is copied during step e) and entry e+2 is loaded during step e.  The
  // copies of the first block go out before the cos/sin table and the query block are
  // prepared, so that the list lookups and the copies overlap that work.
  u32x4 kreg[kLoadsPerWave];
  uint32_t voff[kLoadsPerWave];
#pragma unroll
  for (int c = 0; c < kLoadsPerWave; ++c) voff[c] = stage_lane_offset(wave, lane, c);
  int ent_cur = 0, ent_next = 0;
  if constexpr (RESIDENT) {
    // every text block: wavefront w issues wave-load w of each tile (8 rows), rows past the
    // text read zeros
    const uint32_t off = stage_lane_offset(wave >> 1, lane, wave & 1);
    for (int j = 0; j < cnt; ++j) {
      const int rows = key_end - 64 * j < 64 ? key_end - 64 * j : 64;
      const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kvs.k_noise + (uint64_t)j * kTileBytes, rows);
      const __amdgpu_buffer_rsrc_t rv = tile_rsrc(kvs.v_noise + (uint64_t)j * kTileBytes, rows);
      unsigned char* kt = lds_k0 + 2 * j * kTileBytes + 1024 * wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)kt, 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(kt + kTileBytes), 16, off, 0, 0, 0);
    }
  } else if (cnt > 0) {
    ent_cur = __builtin_amdgcn_readfirstlane(entry(0));
    if (cnt > 1) ent_next = __builtin_amdgcn_readfirstlane(entry(1));
    const int j0 = ent_cur >> 8;
    stage_issue<ROPE_K, CACHED>(kvs, lds_k0, lds_v0, j0, wave, lane, voff, kreg);
  }

  // ---- this wavefront's query block as MFMA B operands: qf[qt][ks] holds rows
  // 32*qt + (lane & 31), channels 16*ks + 8*(lane >> 5) .. +7, scaled by log2(e)/8
  int qblk = 0;
  bool wave_on = false;
  bf16x8 qf[2][4];
  int qtok[2];
  bool qok[2];
  // the rows of query block qb this lane owns, and whether they are computed
  auto query_rows = [&](int qb) __attribute__((always_inline)) {
    qblk = qb;
    wave_on = (qb < P.n_blocks) && (64 * qb + 63 >= P.q_row0) && (64 * qb < P.q_end);
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      qtok[qt] = 64 * qb + 32 * qt + l32;
      qok[qt] = wave_on && qtok[qt] >= P.q_row0 && qtok[qt] < P.q_end;
    }
  };
  // all eight 16-byte loads go out before any is used (rows outside the call's range read a
  // valid row of the tensor and are zeroed afterwards), so the block costs one memory latency
  u32x4 qraw[2][4];
  auto load_query = [&](int qb) __attribute__((always_inline)) {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      int qr = 64 * qb + 32 * qt + l32 - P.q_row0;
      qr = qr < 0 ? 0 : (qr < P.q_rows ? qr : P.q_rows - 1);
      const uint16_t* qrow = P.q + ((int64_t)bh * P.q_rows + qr) * 64;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qraw[qt][ks] = *reinterpret_cast<const u32x4*>(qrow + 8 * (2 * ks + g));
    }
  };
  if constexpr (!RESIDENT) {
    query_rows(st * kWaves + wave);
    load_query(st * kWaves + wave);
  }
  // ---- cos/sin table of every (axis, position, pair) of the grid
  float2* tab = lds_tab;
  if constexpr (ROPE_Q || ROPE_K) {
    for (int e = tid; e < P.rope_entries; e += kThreads) {
      int pos, p, width;
      if (e < 8 * P.T) {
        pos = e >> 3; p = e & 7; width = 16;
      } else if (e < 8 * P.T + 12 * P.H) {
        const int r = e - 8 * P.T;
        pos = r / 12; p = r - 12 * pos; width = 24;
      } else {
        const int r = e - 8 * P.T - 12 * P.H;
        pos = r / 12; p = r - 12 * pos; width = 24;
      }
      tab[e] = rope_cos_sin(pos, p, width, P.log2_theta);
    }
    // the table's LDS writes are visible to the workgroup; the first block's copies stay in
    // flight (a fenced barrier would wait for them here)
    __builtin_amdgcn_s_waitcnt(kWaitLdsOnly);
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
  }

  // rotation (fused Q RoPE) and scaling of the loaded query block
  auto query_operands = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      Coords xyz{0u, 0u, 0u};
      if (ROPE_Q && qok[qt]) xyz = token_coords((uint32_t)qtok[qt], P);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int c = 2 * ks + g;
        u32x4 raw = qraw[qt][ks];
        if constexpr (ROPE_Q) raw = rope_chunk(raw, c, xyz, tab, P);
        raw = scale_chunk_log2(raw);
        if (!qok[qt]) raw = u32x4{0u, 0u, 0u, 0u};
        qf[qt][ks] = __builtin_bit_cast(bf16x8, raw);
      }
    }
  };
  if constexpr (!RESIDENT) query_operands();

  // ---- per-lane LDS offsets (stage, 32-row and 16-row steps become immediates)
  uint32_t ka_off[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) ka_off[ks] = tile_off(l32, 2 * ks + g);
  // transposing reads of V: rows krow0 (low half) and krow0 + 8 (high half, another swizzle)
  uint32_t vb_off[2], vb_off_hi[2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) {
    const int krow0 = 4 * g + ((lane & 15) >> 2);
    const int dcol = 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    vb_off[dt] = tile_off(krow0, dcol >> 3) + (uint32_t)(lane & 1) * 8u;
    vb_off_hi[dt] = tile_off(krow0 + 8, dcol >> 3) + (uint32_t)(lane & 1) * 8u;
  }

  auto shift_offsets = [&](int bytes) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) ka_off[ks] += (uint32_t)bytes;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      vb_off[dt] += (uint32_t)bytes;
      vb_off_hi[dt] += (uint32_t)bytes;
    }
  };

  // ---- state
  const bf16x8 sum_sel = row_sum_selector(lane);   // operand and result row of half_row_sum
  const bool sum_upper = (lane & 16) != 0;
  f32x16 o[2][2];   // O^T tiles [d tile][query tile]
  float mref[2];    // reference of each row (log2 units), -inf = none yet
  float lsum[2];
  bool ref_nonzero;  // some row of the wavefront has a reference other than 0
  auto clear_state = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[a][b][r] = 0.f;
    mref[0] = mref[1] = -INFINITY;
    lsum[0] = lsum[1] = 0.f;
    ref_nonzero = false;
  };
  clear_state();

  // the first block's K rotated into its stage (fused K RoPE), then every copy of it landed
  if constexpr (ROPE_K) {
    if (cnt > 0) stage_store_k(P, lds_k0, ent_cur >> 8, wave, lane, tab, kreg);
  }
  // the resident walk's counter of handed-out query blocks (in the otherwise unused 16 bytes of
  // lds_k1): every wavefront starts on its own block, the next ones are taken from here
  int* const next_block = reinterpret_cast<int*>(lds_k1);
  if constexpr (RESIDENT) {
    if (tid == 0) *next_block = level * P.q_per_part + 2 * kWaves;
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // S^T[key][query] = K Q'^T for the keys 32*kt .. 32*kt+31 of a stage: the K operands, then
  // the products
  auto read_k = [&](const unsigned char* kb, int kt, bf16x8 (&ka)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      ka[ks] = *reinterpret_cast<const bf16x8*>(kb + ka_off[ks] + 4096u * kt);
  };
  auto qk_half = [&](const bf16x8 (&ka)[4], f32x16 (&s)[2]) {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[qt][ks], acc, 0, 0, 0);
      s[qt] = acc;
    }
  };
  // scores relative to the rows' current references (nothing to do while every row of the
  // wavefront keeps the reference 0, or has none yet)
  auto rebase = [&](f32x16 (&s)[2]) {
    if (__builtin_expect(ref_nonzero, 0)) {
      const float f0 = (mref[0] == -INFINITY) ? 0.f : mref[0];
      const float f1 = (mref[1] == -INFINITY) ? 0.f : mref[1];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[0][r] -= f0;
        s[1][r] -= f1;
      }
    }
  };

  // token mask where the block pair crosses the end of the sequence or (full call) the
  // condition boundary: keys >= N, and noise keys for condition queries
  auto mask_half = [&](int key0, int kt, f32x16 (&s)[2]) {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 32 * kt + 8 * (r >> 2) + 4 * g + (r & 3);
        const bool ok = key < key_end && (CROSS || qtok[qt] >= P.C || key < P.C);
        if (!ok) s[qt][r] = -INFINITY;
      }
  };

  // Online softmax of one half: p = 2^(s - m) with the scores s already taken relative to
  // the row's reference m.  The reference only moves when the row's probabilities in this half
  // exceed the limit; the fast path is then one v_exp_f32 and half a conversion per score on
  // the vector ALU, and four small products for the row sums.  The slow path recomputes the half's probabilities against the moved
  // reference (shifted by its change, delta).
  auto softmax_fast = [&](const f32x16 (&s)[2], bf16x8 (&pb)[2][2], float (&psum)[2], bool (&trig)[2]) {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      probs<false>(s[qt], 0.f, pb[qt]);
      psum[qt] = half_row_sum(pb[qt], sum_sel, sum_upper);
      trig[qt] = (mref[qt] == -INFINITY) || !(psum[qt] <= kRescaleLimit);
    }
  };
  auto softmax_slow = [&](const f32x16 (&s)[2], bf16x8 (&pb)[2][2], float (&psum)[2], const bool (&trig)[2],
                          float (&delta)[2]) {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float bm = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) bm = fmaxf(bm, s[qt][r]);
      bm = fmaxf(bm, partner(bm));
      const float m_base = (mref[qt] == -INFINITY) ? 0.f : mref[qt];
      // both lanes of a row take the row's decision (the exchange runs on all lanes: under
      // a short-circuit || the triggered lanes would skip it and their partners would read
      // an inactive lane)
      const int partner_trig = __shfl_xor((int)trig[qt], 32, 64);
      const bool row_trig = trig[qt] || partner_trig != 0;
      const float m_new = row_trig ? fmaxf(mref[qt], coarse_ref(bm + m_base)) : mref[qt];
      const float alpha = (m_new == mref[qt]) ? 1.f : __builtin_amdgcn_exp2f(mref[qt] - m_new);
      o[0][qt] *= alpha;
      o[1][qt] *= alpha;
      lsum[qt] *= alpha;
      mref[qt] = m_new;
      const float m_base_new = (m_new == -INFINITY) ? 0.f : m_new;
      delta[qt] = m_base - m_base_new;
      probs<true>(s[qt], delta[qt], pb[qt]);
      psum[qt] = half_row_sum(pb[qt], sum_sel, sum_upper);
    }
    ref_nonzero = __any((mref[0] != 0.f && mref[0] != -INFINITY) || (mref[1] != 0.f && mref[1] != -INFINITY));
  };

  // O^T[d][query] += V^T P^T over the two 16-key steps of half kt; V^T operands by
  // transposing reads of the row-major V tile
  auto pv_half = [&](const unsigned char* vb, int kt, const bf16x8 (&pb)[2][2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t js_off = 2048u * (2 * kt + h);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vb + vb_off[dt] + js_off));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vb + vb_off_hi[dt] + js_off));
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
          o[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[qt][h], o[dt][qt], 0, 0, 0);
      }
    }
  };

  // One key block, its two halves software-pipelined: the second half's Q K^T is issued
  // with the first half's softmax and the first half's P V with the second half's softmax,
  // interleaved instruction by instruction.  Each half's scores are taken relative to the
  // references as they stand when its softmax starts (after the first half's rescale, if any).
  auto attend = [&](const unsigned char* kb, const unsigned char* vb, auto mask_tag, int j, auto&& copies) {
    // the mask choice: a compile-time tag (two instantiations of the body), or a runtime
    // flag (one body for masked and unmasked blocks)
    bool masked;
    if constexpr (std::is_same_v<decltype(mask_tag), bool>)
      masked = __builtin_expect(mask_tag, false);
    else
      masked = decltype(mask_tag)::value;
    const int key0 = 64 * j;
    f32x16 s0[2], s1[2];
    bf16x8 p0[2][2], p1[2][2];
    float psum[2], delta[2];
    bool trig[2];
    bf16x8 ka0[4], ka1[4];
    read_k(kb, 0, ka0);
    qk_half(ka0, s0);
    read_k(kb, 1, ka1);
    // the next block's copies go out under the first half's matrix-core work, so that the
    // loads of all wavefronts do not queue up at the start of the step
    copies();
    // 4 K reads, the first half's 8 Q K^T MFMAs, the second half's 4 K reads
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    // The wavefront's issue priority is raised while the second half's Q K^T products run
    // interleaved with the first half's softmax, so that where the two wavefronts of a SIMD
    // compete for issue this segment goes first (about 1% less time per launch at 720p;
    // raised over both interleaved segments it gained less, around the matrix-only runs of
    // the block it took longer).  The variants that rotate K in the kernel keep the normal
    // priority: with their K staging through registers it cost 0.5%.
    if constexpr (!ROPE_K) __builtin_amdgcn_s_setprio(1);
    if (masked) mask_half(key0, 0, s0);
    rebase(s0);
    qk_half(ka1, s1);
    softmax_fast(s0, p0, psum, trig);
    // the second half's 8 MFMAs, each followed by vector work of the first half's softmax
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
    }
    if (__builtin_expect(__any(trig[0] || trig[1]), 0)) softmax_slow(s0, p0, psum, trig, delta);
    lsum[0] += psum[0];
    lsum[1] += psum[1];
    if constexpr (!ROPE_K) __builtin_amdgcn_s_setprio(0);
    if (masked) mask_half(key0, 1, s1);
    rebase(s1);
    pv_half(vb, 0, p0);
    softmax_fast(s1, p1, psum, trig);
    // 8 V^T reads, then the first half's 8 P V MFMAs each followed by vector work of the
    // second half's softmax
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
    }
    if (__builtin_expect(__any(trig[0] || trig[1]), 0)) softmax_slow(s1, p1, psum, trig, delta);
    lsum[0] += psum[0];
    lsum[1] += psum[1];
    pv_half(vb, 1, p1);
  };

  auto step = [&](auto stage_tag, int e) {
    constexpr int STAGE = decltype(stage_tag)::value;
    const int ent = ent_cur;
    const int jn = ent_next >> 8;
    // copies of block e+1 into the other stage; past the end of the list they re-read block
    // 0 into that stage, which nothing reads any more
    auto copies = [&]() __attribute__((always_inline)) {
      stage_issue<ROPE_K, CACHED>(kvs, STAGE ? lds_k0 : lds_k1, STAGE ? lds_v0 : lds_v1, jn, wave, lane, voff, kreg);
    };
    // in flight until the barrier below (all lanes load the same entry)
    const int ent_after_raw = (e + 2 < cnt) ? entry(e + 2) : 0;
    if (wave_on && ((ent >> wave) & 1)) {
      const int j = ent >> 8;
      // token mask at the end of the keys and where the block pair crosses the condition
      // boundary (in the cached call the masked rows are not computed: the test is kept the
      // same in every variant because the register allocation of the cached one spilled
      // inside the loop without it)
      const bool need_mask = 64 * j + 63 >= key_end || (64 * qblk < P.C && 64 * j + 63 >= P.C);
      const unsigned char* kb = STAGE ? lds_k1 : lds_k0;
      const unsigned char* vb = STAGE ? lds_v1 : lds_v0;
      if (__builtin_expect(need_mask, 0))
        attend(kb, vb, std::true_type{}, j, copies);
      else
        attend(kb, vb, std::false_type{}, j, copies);
    } else {
      copies();
    }
    if constexpr (ROPE_K) stage_store_k(P, STAGE ? lds_k0 : lds_k1, jn, wave, lane, tab, kreg);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    ent_cur = ent_next;
    ent_next = __builtin_amdgcn_readfirstlane(ent_after_raw);
  };

  // ---- epilogue: O = O~ / l, LSE = (m + log2 l) * ln 2
  auto store_output = [&]() __attribute__((always_inline)) {
    if (wave_on) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const float lt = lsum[qt];   // the row's sum (both lanes of a row hold it)
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        if (qok[qt]) {
          const int64_t row = (int64_t)bh * P.q_rows + (qtok[qt] - P.q_row0);
          uint16_t* orow = P.out + row * 64;
#pragma unroll
          for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int R = 0; R < 4; ++R) {
              const int d = 32 * dt + 8 * R + 4 * g;
              uint2 pk;
              pk.x = pack_bf16x2(o[dt][qt][4 * R] * inv, o[dt][qt][4 * R + 1] * inv);
              pk.y = pack_bf16x2(o[dt][qt][4 * R + 2] * inv, o[dt][qt][4 * R + 3] * inv);
              *reinterpret_cast<uint2*>(orow + d) = pk;
            }
          if (P.lse != nullptr && g == 0) P.lse[row] = lt > 0.f ? (mref[qt] + log2f(lt)) * kLn2 : -INFINITY;
        }
      }
    }
  };

  if constexpr (RESIDENT) {
    // query blocks [blk0, blk1) of the head: wavefront w starts on blk0 + w and then takes the
    // next block not yet handed out.  The two wavefronts of a SIMD do not progress alike (the
    // older one issues first), so with fixed shares the faster one finished about 15% earlier
    // and left its SIMD to the other alone.  A block's result does not depend on which
    // wavefront computes it.  The next block's rows are loaded before this block's output is
    // stored.
    const int blk0 = level * P.q_per_part;
    const int blk1 = blk0 + P.q_per_part < P.n_blocks ? blk0 + P.q_per_part : P.n_blocks;
    int qb = blk0 + wave;
    if (qb < blk1) load_query(qb);
    auto no_copies = []() {};
    while (qb < blk1) {
      query_rows(qb);
      query_operands();
      // the lane offsets step through the text blocks and are set back afterwards
      for (int j = 0; j < cnt; ++j) {
        attend(lds_k0, lds_k0 + kTileBytes, 64 * j + 63 >= key_end, j, no_copies);
        shift_offsets(2 * kTileBytes);
      }
      shift_offsets(-2 * kTileBytes * cnt);
      int taken = 0;
      if (lane == 0) taken = atomicAdd(next_block, 1);
      const int qn = __builtin_amdgcn_readfirstlane(taken);
      if (qn < blk1) load_query(qn);
      store_output();
      clear_state();
      qb = qn;
    }
  } else {
    int e = 0;
    for (; e + 1 < cnt; e += 2) {
      step(std::integral_constant<int, 0>{}, e);
      step(std::integral_constant<int, 1>{}, e + 1);
    }
    if (e < cnt) step(std::integral_constant<int, 0>{}, e);
    store_output();
  }
}

template <bool ROPE_Q, bool ROPE_K, bool CACHED, bool CROSS>
__global__ __launch_bounds__(kThreads, kWavesPerSimd) void bsa_fwd_kernel(const FwdParams P) {
  fwd_body<ROPE_Q, ROPE_K, CACHED, CROSS, false>(P);
}

// Cross-attention over at most kCrossResidentBlocks text blocks: one workgroup of
// 2 * kWaves wavefronts per compute unit (the text takes 128 KB of LDS).
__global__ __launch_bounds__(2 * kThreads, kWavesPerSimd) void bsa_cross_resident_kernel(const FwdParams P) {
  fwd_body<false, false, false, true, true>(P);
}

template <bool ROPE_Q, bool ROPE_K, bool CACHED, bool CROSS = false>
hipError_t launch_variant(const FwdParams& p, unsigned groups, size_t lds, hipStream_t stream) {
  hipLaunchKernelGGL((bsa_fwd_kernel<ROPE_Q, ROPE_K, CACHED, CROSS>), dim3(groups), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

unsigned item_groups(int64_t n_items) { return (unsigned)((n_items + 7) / 8 * 8); }

hipError_t launch_bsa_fwd(const FwdParams& p, hipStream_t stream) {
  if (p.n_items == 0) return hipSuccess;
  const unsigned groups = item_groups(p.n_items);
  const bool rq = (p.flags & LCV_ROPE_Q) != 0, rk = (p.flags & LCV_ROPE_K) != 0, cached = p.kv_split > 0;
  const size_t lds = 0;   // all LDS is static
  const int v = (rq ? 4 : 0) | (rk ? 2 : 0) | (cached ? 1 : 0);
  switch (v) {
    case 0: return launch_variant<false, false, false>(p, groups, lds, stream);
    case 1: return launch_variant<false, false, true>(p, groups, lds, stream);
    case 2: return launch_variant<false, true, false>(p, groups, lds, stream);
    case 3: return launch_variant<false, true, true>(p, groups, lds, stream);
    case 4: return launch_variant<true, false, false>(p, groups, lds, stream);
    case 5: return launch_variant<true, false, true>(p, groups, lds, stream);
    case 6: return launch_variant<true, true, false>(p, groups, lds, stream);
    default: return launch_variant<true, true, true>(p, groups, lds, stream);
  }
}

hipError_t launch_cross_fwd(const FwdParams& p, hipStream_t stream) {
  if (p.n_items == 0) return hipSuccess;
  const unsigned groups = item_groups(p.n_items);
  if (p.q_per_part > 0) {   // the text fits in LDS
    hipLaunchKernelGGL(bsa_cross_resident_kernel, dim3(groups), dim3(2 * kThreads), 0, stream, p);
    return hipGetLastError();
  }
  return launch_variant<false, false, false, true>(p, groups, 0, stream);
}

}  // namespace lcv
