// Block-sparse 3D self-attention backward for gfx950 (MI355X): dQ, dK, dV of the attention
// from the forward's output and LSE, for LoRA training of the model (myzaker article,
// technical principles: the LoRA-trained refinement expert; SimpleTuner quickstart
// "LongCat-Video Edit").  Inputs are Q and K as they entered the scores (already rotated).
//
// With P = exp(S - lse) recomputed from the saved LSE, the gradients are
//   dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D) with D = rowsum(dO * O),
//   dQ = dS K / 8, dK = dS^T Q / 8.
// Both walks score with the forward's own operands: Q' = bf16(Q * log2(e)/8), rounded as the
// forward rounds it, against the unscaled K, so that P = exp2(S' - lse * log2(e)) is the
// forward's probability of the pair (up to the order of the fp32 additions) and agrees with
// the forward's LSE however large the scores.  With S' = Q' K^T the forward's score in log2
// units, dS/dK = Q' ln 2 (the derivative of that score in natural units) and dS/dQ = K / 8.
// Two kernels:
//  * bwd_dq_kernel: the row walk of the forward -- a workgroup of 8 wavefronts owns 4 query
//    blocks (32 rows per wavefront) and streams the K and V blocks of their rows through LDS;
//    it first forms its rows' D = rowsum(dO * O), lse * log2(e) and Q' (row_terms) and
//    stores them in the workspace for the key walk;
//    per 32-key half it forms S^T - lse * log2(e) = K Q'^T and dP^T - D = V dO^T with
//    v_mfma_f32_32x32x16_bf16 (the row's lse and D are folded into one extra MFMA step each),
//    then dS^T = exp2(.) (dP^T - D) and dQ^T += K^T dS^T with K^T read through
//    ds_read_b64_tr_b16;
//  * bwd_dkdv_kernel: the column walk -- a workgroup owns 4 key blocks (32 keys per
//    wavefront) grouped so that their columns nearly coincide (the strided global blocks
//    together) and streams the Q' and dO blocks, lse and D of the union of their columns;
//    S' - lse * log2(e) = Q' K^T and dP - D (both folds one MFMA step), P = exp2(.) with no
//    vector work before the exponential; then dV^T += dO^T P and dK^T += Q'^T dS.
// Every output row is written by exactly one wavefront, with no atomics: results are
// deterministic.
// Cross-attention (CROSS = true): keys and values are the text states [BH, kv_len, 64] with a
// per-batch valid length; the query walk visits every text block, and since every query
// block attends every text block the key walk splits the query blocks into chunks, each
// workgroup writing fp32 partial dK, dV for its chunk, which bwd_cross_reduce_kernel adds in
// chunk order (deterministic).
#include <type_traits>

#include "attn_tile.h"
#include "lcv_internal.h"

namespace lcv {
namespace {

// read-only schedule tables through the constant address space: uniform indexes become scalar
// loads, which neither occupy the vector memory counter nor need a readfirstlane
typedef __attribute__((address_space(4))) const int32_t const_i32;

constexpr int kBwdWaves = 2 * kWaves;         // two wavefronts (32 rows each) per 64-row block
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr float kEmptyRowLse2 = 3.0e38f;   // lse * log2(e) of a row with no key: p = 0
// s_waitcnt operand: vmcnt <= 2 and lgkmcnt == 0, expcnt not waited for (gfx9 field layout)
constexpr int kWaitVm2 = 2 | (7 << 4);
static_assert(kBwdWaves == 8, "a 64 x 64 tile is 8 wave-loads of 1 KB, one per wavefront");

// fp32 value m as three bf16 parts (hi + mid + lo == m to fp32 precision) in slots 0..2 of
// the lanes of channel group 0: with an operand of ones in the same slots, one MFMA step
// adds -m (sign folded) to a whole row or column of an accumulator.
__device__ __forceinline__ bf16x8 fold_neg(float m, int g) {
  const float nm = -m;
  const __bf16 hi = (__bf16)nm;
  const float r1 = nm - (float)hi;
  const __bf16 mid = (__bf16)r1;
  const __bf16 lo = (__bf16)(r1 - (float)mid);
  const __bf16 z = (__bf16)0.0f;
  const bf16x8 v = {hi, mid, lo, z, z, z, z, z};
  const bf16x8 zero = {z, z, z, z, z, z, z, z};
  return g == 0 ? v : zero;
}

// The three parts of fold_neg(m) packed in 8 bytes (hi | mid << 16, lo), as the backward
// stores them per row for the fold steps of its walks.
__device__ __forceinline__ uint2 fold_parts(float m) {
  const bf16x8 v = fold_neg(m, 0);
  const u32x4 w = __builtin_bit_cast(u32x4, v);
  return uint2{w[0], w[1]};
}

__device__ __forceinline__ bf16x8 ones_slots(int g) {
  const __bf16 one = (__bf16)1.0f, z = (__bf16)0.0f;
  return g == 0 ? bf16x8{one, one, one, z, z, z, z, z} : bf16x8{z, z, z, z, z, z, z, z};
}

// A fold step on the 32x32x8 product, which covers the three parts at half the cycles of
// the 32x32x16 one.  Its 4-wide operands: lane l holds slots k = 4 (l / 32) .. +3 of its row
// (A) or column (B); the parts sit in slots 0-2 of the lanes with l / 32 = 0 and meet ones
// there.  fold_rows: the parts of row l % 32 as A (result rows = the folded rows);
// fold_cols: as B (result columns).
__device__ __forceinline__ i16x4 fold4(uint2 parts, int g) {
  return __builtin_bit_cast(i16x4, uint2{g == 0 ? parts.x : 0u, g == 0 ? parts.y : 0u});
}
__device__ __forceinline__ i16x4 ones4(int g) {
  return __builtin_bit_cast(i16x4, uint2{g == 0 ? 0x3F803F80u : 0u, g == 0 ? 0x00003F80u : 0u});
}
__device__ __forceinline__ f32x16 fold_rows(uint2 parts, int g) {
  return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(fold4(parts, g), ones4(g), f32x16{}, 0, 0, 0);
}
__device__ __forceinline__ f32x16 fold_cols(uint2 parts, int g) {
  return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(ones4(g), fold4(parts, g), f32x16{}, 0, 0, 0);
}

// 8 channels (chunk c) of row `row` of a [rows, 64] bf16 tensor as an MFMA operand; zero
// when !ok.
__device__ __forceinline__ bf16x8 load_chunk(const uint16_t* base, int64_t row, int c, bool ok) {
  u32x4 raw{0u, 0u, 0u, 0u};
  if (ok) raw = *reinterpret_cast<const u32x4*>(base + row * 64 + 8 * c);
  return __builtin_bit_cast(bf16x8, raw);
}

// 16 accumulator values (scores of one 32 x 32 tile) -> bf16 MFMA B operands of its two
// 16-wide contraction steps (registers 8h .. 8h+7 of step h).
__device__ __forceinline__ void pack16(const f32x16& x, bf16x8 (&b)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    bf16x2 w[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const f32x2_t p = {x[8 * h + 2 * e2], x[8 * h + 2 * e2 + 1]};
      w[e2] = __builtin_convertvector(p, bf16x2);
    }
    b[h] = __builtin_shufflevector(__builtin_shufflevector(w[0], w[1], 0, 1, 2, 3),
                                   __builtin_shufflevector(w[2], w[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// Offsets of the transposing reads that give the A operand X^T of a contraction over the
// rows of a row-major tile X (the rows in the order in which an accumulator holds them):
// channel tile dt, rows 4g + (lane & 15) / 4 of a 16-row step (plus 8 for the upper half,
// whose swizzle differs), plus 2048 * (2 * half + step) for the step (16 rows: the swizzle
// repeats).
struct TrOff {
  uint32_t lo, hi;
};
__device__ __forceinline__ TrOff tr_off(int lane, int dt) {
  const int g = lane >> 5;
  const int row0 = 4 * g + ((lane & 15) >> 2);
  const int col = 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  return {tile_off(row0, col >> 3) + (uint32_t)(lane & 1) * 8u, tile_off(row0 + 8, col >> 3) + (uint32_t)(lane & 1) * 8u};
}

__device__ __forceinline__ bf16x8 tr_read(const unsigned char* tile, const TrOff& off, uint32_t step) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + off.lo + step));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + off.hi + step));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Asynchronous copy of rows 64*blk .. 64*blk+63 of a [N, 64] bf16 slice into an LDS tile by a
// buffer load straight into LDS: wavefront w moves rows 8w .. 8w+7, lane l row 8w + l/8,
// landing at physical chunk l%8, which holds logical chunk (l%8) ^ swz(row) of the swizzle.
// The block's first row is the base of a buffer resource (scalar arithmetic) whose size ends at
// row N, so rows past the sequence read zeros (their scores are masked, their probabilities and
// dS are zero); the lane's offset inside the block does not depend on the block.
__device__ __forceinline__ void copy_tile(const uint16_t* slice, int32_t N, int blk, unsigned char* dst, int wave,
                                          int lane) {
  const int row = 8 * wave + (lane >> 3);
  const int gch = (lane & 7) ^ swz(row);
  int rows = N - 64 * blk;
  rows = rows < 0 ? 0 : (rows > 64 ? 64 : rows);
  const __amdgpu_buffer_rsrc_t r = uniform_rsrc((uint64_t)(uintptr_t)slice + (uint64_t)blk * kTileBytes, rows * 128);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + 1024 * wave), 16, (uint32_t)(row * 128 + 16 * gch), 0,
                                           0, 0);
}

// Asynchronous copy of the 64 eight-byte row values of block blk into LDS (one wavefront, two
// 4-byte loads per lane), zeros past row N.
__device__ __forceinline__ void copy_rows_u64(const uint2* slice, int32_t N, int blk, uint2* dst, int lane) {
  int rows = N - 64 * blk;
  rows = rows < 0 ? 0 : (rows > 64 ? 64 : rows);
  const __amdgpu_buffer_rsrc_t r = uniform_rsrc((uint64_t)(uintptr_t)(slice + (int64_t)64 * blk), rows * 8);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 4, (uint32_t)(4 * lane), 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(reinterpret_cast<unsigned char*>(dst) + 256), 4,
                                           (uint32_t)(256 + 4 * lane), 0, 0, 0);
}

// The per-row terms of the backward, formed by the query walks (which visit every query row
// once) and stored for the key walk that runs after them: Q' = bf16(Q log2(e)/8) (the
// forward's query operand), lse log2(e) (an empty row's value for lse = -inf) and
// D = rowsum(dO * O), with the fold parts of -lse log2(e) and -D.  The lane holds channel
// chunks 2ks + g (ks = 0..3) of row `row` in qr, orw (O) and dx (dO), the partner lane l ^ 32
// the other four; ok: the row exists (else nothing is stored).  Returns Q' in qx.
__device__ __forceinline__ void row_terms(const BwdParams& P, int64_t row, bool ok, int g, const bf16x8 (&qr)[4],
                                          const bf16x8 (&orw)[4], const bf16x8 (&dx)[4], float l, bf16x8 (&qx)[4],
                                          float& l2, float& d) {
  float sum = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const u32x4 a = __builtin_bit_cast(u32x4, orw[ks]), b = __builtin_bit_cast(u32x4, dx[ks]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sum = fmaf(__uint_as_float(a[e] << 16), __uint_as_float(b[e] << 16), sum);
      sum = fmaf(__uint_as_float(a[e] & 0xffff0000u), __uint_as_float(b[e] & 0xffff0000u), sum);
    }
    const u32x4 sc = scale_chunk_log2(__builtin_bit_cast(u32x4, qr[ks]));
    qx[ks] = __builtin_bit_cast(bf16x8, sc);
    if (ok) *reinterpret_cast<u32x4*>(P.qs + row * 64 + 8 * (2 * ks + g)) = sc;
  }
  d = sum + __shfl_xor(sum, 32, 64);
  l2 = (l == -INFINITY) ? kEmptyRowLse2 : l * kLog2e;
  if (ok && g == 0) {
    P.lse2[row] = l2;
    P.delta[row] = d;
    P.fold_l[row] = fold_parts(l2);
    P.fold_d[row] = fold_parts(d);
  }
}

// End of a pipeline step: this wavefront's copies of the next block have landed in LDS (only
// the two copies issued in this step may still be in flight) and its LDS reads are done;
// then the workgroup barrier.  __syncthreads() would also wait for the copies in flight
// (its release fence covers every outstanding memory operation).
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitVm2);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Work item -> workgroup numbering as in the forward: XCD x (blockIdx % 8) runs the x-th
// contiguous eighth of the items.
__device__ __forceinline__ int xcd_item() {
  const int per_xcd = (int)(gridDim.x >> 3);
  return (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
}

// ------------------------------------------------------------------------------------ dQ
// Valid keys of a (batch, head) row: the sequence, or the batch item's text length.
template <bool CROSS>
__device__ __forceinline__ int key_end_of(const BwdParams& P, int bh) {
  if constexpr (!CROSS) return P.N;
  int len = P.kv_len;
  if (P.kv_lens != nullptr) {
    const int l = P.kv_lens[bh / P.heads];
    len = l < 0 ? 0 : (l < P.kv_len ? l : P.kv_len);
  }
  return __builtin_amdgcn_readfirstlane(len);
}

template <bool CROSS>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dq_kernel(const BwdParams P) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k2[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v2[kTileBytes];
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;

  const int item = xcd_item();
  if (item >= P.bh * P.n_st) return;
  const int bh = item / P.n_st;
  const int st = item - bh * P.n_st;
  const int64_t base = (int64_t)bh * P.N;

  // this wavefront's 32 query rows; the lane's own row is q
  const int qblk = st * kWaves + (wave >> 1);
  const bool wave_on = qblk < P.n_blocks;
  const int q = 64 * qblk + 32 * (wave & 1) + l32;
  const bool qok = wave_on && q < P.N;
  // the row's terms (row_terms: Q', and lse in log2 units and D, which are folded into the
  // S^T and dP^T accumulators by one extra MFMA step each), stored for the key walk
  bf16x8 qf[4], dof[4];
  float lse2, dlt;
  {
    bf16x8 qr[4], orw[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qr[ks] = load_chunk(P.q + base * 64, q, 2 * ks + g, qok);
      orw[ks] = load_chunk(P.out + base * 64, q, 2 * ks + g, qok);
      dof[ks] = load_chunk(P.dout + base * 64, q, 2 * ks + g, qok);
    }
    const float l = qok ? P.lse[base + q] : -INFINITY;
    row_terms(P, base + q, qok, g, qr, orw, dof, l, qf, lse2, dlt);
  }
  const bf16x8 fold_l = fold_neg(lse2, g);
  const bf16x8 fold_d = fold_neg(dlt, g);
  const int key_end = key_end_of<CROSS>(P, bh);                 // keys [0, key_end) exist
  const int64_t kv_base = (int64_t)bh * (CROSS ? P.kv_len : P.N);
  const bf16x8 ones = ones_slots(g);
  uint32_t ka_off[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) ka_off[ks] = tile_off(l32, 2 * ks + g);
  const TrOff tr0 = tr_off(lane, 0), tr1 = tr_off(lane, 1);

  f32x16 dqt[2];   // dQ^T tiles [channel tile]: lane = query, registers = channels
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqt[dt][r] = 0.f;

  // the workgroup's list: the forward's (self-attention), or every text block for all four
  // query blocks (cross-attention)
  const const_i32* ents = CROSS ? nullptr : (const const_i32*)(P.st_ent) + P.row_ptr[st * kWaves];
  const int cnt = CROSS ? (key_end + 63) >> 6 : P.st_cnt[st];
  auto entry = [&](int e) __attribute__((always_inline)) {
    if constexpr (CROSS)
      return (e << 8) | ((1 << kWaves) - 1);
    else
      return (int)ents[e];
  };
  const uint16_t* kslice = P.k + kv_base * 64;
  const uint16_t* vslice = P.v + kv_base * 64;
  // three LDS stages: block e+2 is copied while block e is used and block e+1 lands
  int ent_cur = 0, ent_n1 = 0, ent_n2 = 0;
  if (cnt > 0) {
    ent_cur = entry(0);
    if (cnt > 1) ent_n1 = entry(1);
    if (cnt > 2) ent_n2 = entry(2);
    copy_tile(kslice, key_end, ent_cur >> 8, lds_k0, wave, lane);
    copy_tile(vslice, key_end, ent_cur >> 8, lds_v0, wave, lane);
    copy_tile(kslice, key_end, ent_n1 >> 8, lds_k1, wave, lane);
    copy_tile(vslice, key_end, ent_n1 >> 8, lds_v1, wave, lane);
  }
  stage_barrier();

  // the folded lse and D terms do not change along the walk (the wavefront's queries are
  // fixed): their accumulator tiles are formed once and start every block's products
  const f32x16 dp_init = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, fold_d, f32x16{}, 0, 0, 0);
  const f32x16 s_init = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, fold_l, f32x16{}, 0, 0, 0);

  // S^T and dP^T - D of keys 32kt .. 32kt+31 (registers) against the wavefront's queries
  auto sdp_half = [&](const unsigned char* kb, const unsigned char* vb, int kt, f32x16& s, f32x16& dp)
      __attribute__((always_inline)) {
    bf16x8 ka[4], va[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      ka[ks] = *reinterpret_cast<const bf16x8*>(kb + ka_off[ks] + 4096u * kt);
      va[ks] = *reinterpret_cast<const bf16x8*>(vb + ka_off[ks] + 4096u * kt);
    }
    dp = dp_init;
    s = s_init;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[ks], dof[ks], dp, 0, 0, 0);
    }
  };
  auto mask_half = [&](int j, int kt, f32x16& s) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 64 * j + 32 * kt + 8 * (r >> 2) + 4 * g + (r & 3);
      const bool ok = key < key_end && (q >= P.C || key < P.C);
      s[r] = ok ? s[r] : -INFINITY;
    }
  };
  // dS^T = P^T * (dP^T - D) as the bf16 B operands of the two 16-key steps
  auto ds_half = [&](const f32x16& s, const f32x16& dp, bf16x8 (&dsb)[2]) __attribute__((always_inline)) {
    f32x16 ds;
#pragma unroll
    for (int r = 0; r < 16; ++r) ds[r] = __builtin_amdgcn_exp2f(s[r]) * dp[r];
    pack16(ds, dsb);
  };
  // dQ^T += K^T dS^T over the two 16-key steps of half kt
  auto dq_half = [&](const unsigned char* kb, int kt, const bf16x8 (&dsb)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t so = 2048u * (2 * kt + h);
      dqt[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read(kb, tr0, so), dsb[h], dqt[0], 0, 0, 0);
      dqt[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read(kb, tr1, so), dsb[h], dqt[1], 0, 0, 0);
    }
  };

  // One key block, its halves software-pipelined as in the forward: the second half's S^T
  // and dP^T go to the matrix cores while the vector ALU forms the first half's dS^T, and
  // the first half's dQ^T update runs with the second half's dS^T.
  // (one body for masked and unmasked blocks: with two instantiations the register allocator
  // kept the dQ^T accumulators in different registers on the two paths and copied them at
  // the join, every block)
  auto block = [&](const unsigned char* kb, const unsigned char* vb, int j, bool masked, auto&& copies)
      __attribute__((always_inline)) {
    f32x16 s0, dp0, s1, dp1;
    bf16x8 d0[2], d1[2];
    sdp_half(kb, vb, 0, s0, dp0);
    if (__builtin_expect(masked, 0)) mask_half(j, 0, s0);
    copies();
    // issue priority raised over the interleaved segment, as in the forward
    __builtin_amdgcn_s_setprio(1);
    sdp_half(kb, vb, 1, s1, dp1);
    ds_half(s0, dp0, d0);
    // 8 K/V reads, then the second half's 10 MFMAs each followed by vector work of the first
    // half's dS^T
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 10; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    if (__builtin_expect(masked, 0)) mask_half(j, 1, s1);
    dq_half(kb, 0, d0);
    ds_half(s1, dp1, d1);
    // 8 transposing K reads, then the first half's 4 dQ^T MFMAs each followed by vector work
    // of the second half's dS^T
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
    }
    dq_half(kb, 1, d1);
  };

  auto step = [&](auto stage_tag, int e) __attribute__((always_inline)) {
    constexpr int STAGE = decltype(stage_tag)::value;
    constexpr int SN = (STAGE + 2) % 3;
    unsigned char* const kc = STAGE == 0 ? lds_k0 : STAGE == 1 ? lds_k1 : lds_k2;
    unsigned char* const vc = STAGE == 0 ? lds_v0 : STAGE == 1 ? lds_v1 : lds_v2;
    unsigned char* const kn = SN == 0 ? lds_k0 : SN == 1 ? lds_k1 : lds_k2;
    unsigned char* const vn = SN == 0 ? lds_v0 : SN == 1 ? lds_v1 : lds_v2;
    const int ent = ent_cur;
    const int jn = ent_n2 >> 8;
    const int ent_after_raw = (e + 3 < cnt) ? entry(e + 3) : 0;
    // copies of block e+2 into the stage block e-1 used (past the end of the list they
    // re-read block 0, which nothing reads any more)
    auto copies = [&]() __attribute__((always_inline)) {
      copy_tile(kslice, key_end, jn, kn, wave, lane);
      copy_tile(vslice, key_end, jn, vn, wave, lane);
    };
    if (wave_on && ((ent >> (wave >> 1)) & 1)) {
      const int j = ent >> 8;
      const bool masked = 64 * j + 63 >= key_end || (64 * qblk < P.C && 64 * j + 63 >= P.C);
      block(kc, vc, j, masked, copies);
    } else {
      copies();
    }
    stage_barrier();
    ent_cur = ent_n1;
    ent_n1 = ent_n2;
    ent_n2 = ent_after_raw;
  };
  int e = 0;
  for (; e + 2 < cnt; e += 3) {
    step(std::integral_constant<int, 0>{}, e);
    step(std::integral_constant<int, 1>{}, e + 1);
    step(std::integral_constant<int, 2>{}, e + 2);
  }
  if (e < cnt) step(std::integral_constant<int, 0>{}, e);
  if (e + 1 < cnt) step(std::integral_constant<int, 1>{}, e + 1);
  // the last copies (re-reads into free stages) land before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(0);

  // dQ = dQ^T / 8 (the score scale), rows written as 8-byte stores of 4 channels
  if (qok) {
    uint16_t* row = P.dq + (base + q) * 64;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        uint2 pk;
        pk.x = pack_bf16x2(dqt[dt][4 * R] * 0.125f, dqt[dt][4 * R + 1] * 0.125f);
        pk.y = pack_bf16x2(dqt[dt][4 * R + 2] * 0.125f, dqt[dt][4 * R + 3] * 0.125f);
        *reinterpret_cast<uint2*>(row + 32 * dt + 8 * R + 4 * g) = pk;
      }
  }
}

// ------------------------------------------------------------ dQ of the cross-attention
// With at most kCrossResidentBlocks text blocks (512 tokens) a head's text K and V fit in
// LDS (128 KB): each workgroup loads them once and streams a range of query blocks past
// them in units of 32 query rows (two per query block, as in bwd_dq_kernel), handed out to
// the wavefronts one at a time.
// The walk has no copies and no barriers, so the wavefronts run on their own; each loads its
// next unit's Q, dO, lse and D right after its walk, under its dQ stores and the partner
// wavefront's work.  Per text block the arithmetic is bwd_dq_kernel's (no condition rule).
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dq_cross_resident_kernel(const BwdParams P) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k[kCrossResidentBlocks * kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_v[kCrossResidentBlocks * kTileBytes];
  __shared__ int next_unit;   // the next unit of the range not yet handed out
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;

  const int item = xcd_item();
  if (item >= P.bh * P.q_parts) return;
  const int bh = item / P.q_parts;
  const int part = item - bh * P.q_parts;
  const int64_t base = (int64_t)bh * P.N;
  const int key_end = key_end_of<true>(P, bh);
  const int nkb = (key_end + 63) >> 6;   // <= kCrossResidentBlocks: kv_len is checked on the host
  const int64_t kv_base = (int64_t)bh * P.kv_len;
  const int blk0 = part * P.q_per_part;
  const int blk1 = blk0 + P.q_per_part < P.n_blocks ? blk0 + P.q_per_part : P.n_blocks;

  // the text blocks, rows past the item's length clamped to its last token (masked below)
  for (int j = 0; j < nkb; ++j) {
    copy_tile(P.k + kv_base * 64, key_end, j, lds_k + j * kTileBytes, wave, lane);
    copy_tile(P.v + kv_base * 64, key_end, j, lds_v + j * kTileBytes, wave, lane);
  }
  if (tid == 0) next_unit = kBwdThreads / 64;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  uint32_t ka_off[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) ka_off[ks] = tile_off(l32, 2 * ks + g);
  const TrOff tr0 = tr_off(lane, 0), tr1 = tr_off(lane, 1);

  // The range's work is handed out in units of 32 query rows: unit u is half u & 1 of query
  // block blk0 + u / 2.  Wavefront w starts on unit w and then takes the next unit not yet
  // handed out: the two wavefronts of a SIMD do not progress alike (the older one issues
  // first), and with fixed shares the faster one would finish early and leave its SIMD to the
  // other alone.  A unit's results do not depend on which wavefront computes it.
  // The per-row terms (row_terms) of the 32 rows of unit u; rows past the range or the
  // sequence read zeros and an empty row's lse.
  auto row_ok = [&](int u, int& qq) __attribute__((always_inline)) {
    const int qb = blk0 + (u >> 1);
    qq = 64 * qb + 32 * (u & 1) + l32;
    return qb < blk1 && qq < P.N;
  };
  auto issue_rows = [&](int u, bf16x8 (&qr)[4], bf16x8 (&orw)[4], bf16x8 (&dx)[4], float& l)
      __attribute__((always_inline)) {
    int qq;
    const bool ok = row_ok(u, qq);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qr[ks] = load_chunk(P.q + base * 64, qq, 2 * ks + g, ok);
      orw[ks] = load_chunk(P.out + base * 64, qq, 2 * ks + g, ok);
      dx[ks] = load_chunk(P.dout + base * 64, qq, 2 * ks + g, ok);
    }
    l = ok ? P.lse[base + qq] : -INFINITY;
  };
  auto finish_rows = [&](int u, const bf16x8 (&qr)[4], const bf16x8 (&orw)[4], const bf16x8 (&dx)[4], float l,
                         bf16x8 (&qx)[4], float& l2, float& d) __attribute__((always_inline)) {
    int qq;
    const bool ok = row_ok(u, qq);
    row_terms(P, base + qq, ok, g, qr, orw, dx, l, qx, l2, d);
  };

  int unit = wave;
  bf16x8 qf[4], dof[4];
  float lse2, dlt;
  {
    bf16x8 qr[4], orw[4];
    float l;
    issue_rows(unit, qr, orw, dof, l);
    finish_rows(unit, qr, orw, dof, l, qf, lse2, dlt);
  }
  while (blk0 + (unit >> 1) < blk1) {
    int taken = 0;
    if (lane == 0) taken = atomicAdd(&next_unit, 1);
    const int unext = __builtin_amdgcn_readfirstlane(taken);

    const int q = 64 * (blk0 + (unit >> 1)) + 32 * (unit & 1) + l32;
    const uint2 fold_l = fold_parts(lse2);
    const uint2 fold_d = fold_parts(dlt);
    f32x16 dqt[2];
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) dqt[dt][r] = 0.f;

    auto sdp_half = [&](const unsigned char* kb, const unsigned char* vb, int kt, f32x16& s, f32x16& dp)
        __attribute__((always_inline)) {
      bf16x8 ka[4], va[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        ka[ks] = *reinterpret_cast<const bf16x8*>(kb + ka_off[ks] + 4096u * kt);
        va[ks] = *reinterpret_cast<const bf16x8*>(vb + ka_off[ks] + 4096u * kt);
      }
      dp = fold_cols(fold_d, g);
      s = fold_cols(fold_l, g);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[ks], dof[ks], dp, 0, 0, 0);
      }
    };
    auto mask_half = [&](int j, int kt, f32x16& s) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 64 * j + 32 * kt + 8 * (r >> 2) + 4 * g + (r & 3);
        s[r] = key < key_end ? s[r] : -INFINITY;
      }
    };
    auto ds_half = [&](const f32x16& s, const f32x16& dp, bf16x8 (&dsb)[2]) __attribute__((always_inline)) {
      f32x16 ds;
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] = __builtin_amdgcn_exp2f(s[r]) * dp[r];
      pack16(ds, dsb);
    };
    auto dq_half = [&](const unsigned char* kb, int kt, const bf16x8 (&dsb)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t so = 2048u * (2 * kt + h);
        dqt[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read(kb, tr0, so), dsb[h], dqt[0], 0, 0, 0);
        dqt[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read(kb, tr1, so), dsb[h], dqt[1], 0, 0, 0);
      }
    };
    auto block = [&](const unsigned char* kb, const unsigned char* vb, int j, auto mask_tag)
        __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
      f32x16 s0, dp0, s1, dp1;
      bf16x8 d0[2], d1[2];
      sdp_half(kb, vb, 0, s0, dp0);
      if (MASK) mask_half(j, 0, s0);
      sdp_half(kb, vb, 1, s1, dp1);
      ds_half(s0, dp0, d0);
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 10; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      if (MASK) mask_half(j, 1, s1);
      dq_half(kb, 0, d0);
      ds_half(s1, dp1, d1);
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
      }
      dq_half(kb, 1, d1);
    };
    for (int j = 0; j < nkb; ++j) {
      const unsigned char* kb = lds_k + j * kTileBytes;
      const unsigned char* vb = lds_v + j * kTileBytes;
      if (64 * j + 63 >= key_end)
        block(kb, vb, j, std::true_type{});
      else
        block(kb, vb, j, std::false_type{});
    }

    // the next round's rows, loaded after the walk (holding them through it would spill):
    // they arrive while this round's dQ is stored and the partner wavefront computes
    bf16x8 qr_n[4], or_n[4], dof_n[4];
    float l_n;
    issue_rows(unext, qr_n, or_n, dof_n, l_n);
    // dQ = dQ^T / 8, rows written as 8-byte stores of 4 channels
    if (q < P.N) {
      uint16_t* row = P.dq + (base + q) * 64;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int R = 0; R < 4; ++R) {
          uint2 pk;
          pk.x = pack_bf16x2(dqt[dt][4 * R] * 0.125f, dqt[dt][4 * R + 1] * 0.125f);
          pk.y = pack_bf16x2(dqt[dt][4 * R + 2] * 0.125f, dqt[dt][4 * R + 3] * 0.125f);
          *reinterpret_cast<uint2*>(row + 32 * dt + 8 * R + 4 * g) = pk;
        }
    }
    finish_rows(unext, qr_n, or_n, dof_n, l_n, qf, lse2, dlt);
    unit = unext;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) dof[ks] = dof_n[ks];
  }
}

// ---------------------------------------------------------------------------------- dK, dV
template <bool CROSS>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dkdv_kernel(const BwdParams P) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds_q0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_q1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_o0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_o1[kTileBytes];
  __shared__ __attribute__((aligned(512))) uint2 lds_l0[64];   // fold parts of -lse * log2(e) per query row
  __shared__ __attribute__((aligned(512))) uint2 lds_l1[64];
  __shared__ __attribute__((aligned(512))) uint2 lds_d0[64];   // and of -D
  __shared__ __attribute__((aligned(512))) uint2 lds_d1[64];
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;

  const int item = xcd_item();
  if (item >= P.bh * P.n_kg) return;
  const int bh = item / P.n_kg;
  const int grp = item - bh * P.n_kg;           // self: a key group; cross: (group, chunk)
  const int64_t base = (int64_t)bh * P.N;
  const int key_end = key_end_of<CROSS>(P, bh);
  const int64_t kv_base = (int64_t)bh * (CROSS ? P.kv_len : P.N);
  const int kgroup = CROSS ? grp / P.n_chunks : grp;
  const int chunk = CROSS ? grp - kgroup * P.n_chunks : 0;

  // this wavefront's 32 keys; the lane's own key is key
  int kblk;
  if constexpr (CROSS) {
    kblk = kWaves * kgroup + (wave >> 1);
    kblk = 64 * kblk < key_end ? kblk : -1;   // blocks past the text length: never read back
  } else {
    kblk = __builtin_amdgcn_readfirstlane(P.kg_blk[grp * kWaves + (wave >> 1)]);
  }
  const bool wave_on = kblk >= 0;
  const int key = 64 * kblk + 32 * (wave & 1) + l32;
  const bool kok = wave_on && key < (CROSS ? key_end : P.N);   // padded text rows stay zero
  bf16x8 kf[4], vf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    kf[ks] = load_chunk(P.k + kv_base * 64, key, 2 * ks + g, kok);
    vf[ks] = load_chunk(P.v + kv_base * 64, key, 2 * ks + g, kok);
  }
  uint32_t qa_off[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qa_off[ks] = tile_off(l32, 2 * ks + g);
  const TrOff tr0 = tr_off(lane, 0), tr1 = tr_off(lane, 1);

  f32x16 dvt[2], dkt[2];   // dV^T, dK^T tiles [channel tile]: lane = key, registers = channels
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dvt[dt][r] = 0.f;
      dkt[dt][r] = 0.f;
    }

  // the workgroup's list: the host-built column union (self-attention), or the chunk's query
  // blocks, all of which attend every text block (cross-attention)
  const int32_t* ents = CROSS ? nullptr : P.kg_ent + P.kg_off[grp];
  const int first_q = chunk * P.q_chunk;
  int cnt;
  if constexpr (CROSS) {
    cnt = P.n_blocks - first_q;
    cnt = cnt < P.q_chunk ? cnt : P.q_chunk;
  } else {
    cnt = P.kg_cnt[grp];
  }
  auto entry = [&](int e) __attribute__((always_inline)) {
    if constexpr (CROSS)
      return ((first_q + e) << 8) | ((1 << kWaves) - 1);
    else
      return ents[e];
  };
  const uint16_t* qslice = P.qs + base * 64;
  const uint16_t* oslice = P.dout + base * 64;
  const uint2* lslice = P.fold_l + base;
  const uint2* dslice = P.fold_d + base;
  auto copies = [&](int blk, unsigned char* qd, unsigned char* od, uint2* ld, uint2* dd) __attribute__((always_inline)) {
    copy_tile(qslice, P.N, blk, qd, wave, lane);
    copy_tile(oslice, P.N, blk, od, wave, lane);
    if (wave == 0) copy_rows_u64(lslice, P.N, blk, ld, lane);
    if (wave == 1) copy_rows_u64(dslice, P.N, blk, dd, lane);
  };
  int ent_cur = 0, ent_next = 0;
  if (cnt > 0) {
    ent_cur = __builtin_amdgcn_readfirstlane(entry(0));
    if (cnt > 1) ent_next = __builtin_amdgcn_readfirstlane(entry(1));
    copies(ent_cur >> 8, lds_q0, lds_o0, lds_l0, lds_d0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // S' - lse * log2(e) (S' = Q' K^T, log2 units) and dP - D for queries 32qt .. 32qt+31 (registers) and the wavefront's keys
  // (lanes); the per-query lse and D enter through one folded MFMA step each
  auto sdp_half = [&](const unsigned char* qb, const unsigned char* ob, const uint2* lb, const uint2* db, int qt,
                      f32x16& s, f32x16& dp) __attribute__((always_inline)) {
    bf16x8 qa[4], oa[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qa[ks] = *reinterpret_cast<const bf16x8*>(qb + qa_off[ks] + 4096u * qt);
      oa[ks] = *reinterpret_cast<const bf16x8*>(ob + qa_off[ks] + 4096u * qt);
    }
    s = fold_rows(lb[32 * qt + l32], g);
    dp = fold_rows(db[32 * qt + l32], g);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ks], kf[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[ks], vf[ks], dp, 0, 0, 0);
    }
  };
  auto mask_half = [&](int i, int qt, f32x16& s) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qq = 64 * i + 32 * qt + 8 * (r >> 2) + 4 * g + (r & 3);
      const bool ok = qq < P.N && (CROSS ? key < key_end : (qq >= P.C || key < P.C));
      s[r] = ok ? s[r] : -INFINITY;
    }
  };
  // P and dS = P * (dP - D) as the bf16 B operands of the two 16-query steps
  auto pds_half = [&](const f32x16& s, const f32x16& dp, bf16x8 (&pb)[2], bf16x8 (&dsb)[2])
      __attribute__((always_inline)) {
    f32x16 p, ds;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = __builtin_amdgcn_exp2f(s[r]);
      ds[r] = p[r] * dp[r];
    }
    pack16(p, pb);
    pack16(ds, dsb);
  };
  // dV^T += dO^T P and dK^T += Q'^T dS over the two 16-query steps of half qt
  auto upd_half = [&](const unsigned char* qb, const unsigned char* ob, int qt, const bf16x8 (&pb)[2],
                      const bf16x8 (&dsb)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t so = 2048u * (2 * qt + h);
      dvt[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read(ob, tr0, so), pb[h], dvt[0], 0, 0, 0);
      dvt[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read(ob, tr1, so), pb[h], dvt[1], 0, 0, 0);
      dkt[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read(qb, tr0, so), dsb[h], dkt[0], 0, 0, 0);
      dkt[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read(qb, tr1, so), dsb[h], dkt[1], 0, 0, 0);
    }
  };

  // One query block, its halves software-pipelined: the second half's S and dP go to the
  // matrix cores while the vector ALU forms the first half's P and dS, and the first half's
  // dV^T, dK^T updates run with the second half's P and dS.
  // (one body for masked and unmasked blocks, as in the query walk)
  auto block = [&](const unsigned char* qb, const unsigned char* ob, const uint2* lb, const uint2* db, int i,
                   bool masked, auto&& copies) __attribute__((always_inline)) {
    f32x16 s0, dp0, s1, dp1;
    bf16x8 p0[2], d0[2], p1[2], d1[2];
    sdp_half(qb, ob, lb, db, 0, s0, dp0);
    if (__builtin_expect(masked, 0)) mask_half(i, 0, s0);
    copies();
    __builtin_amdgcn_s_setprio(1);
    sdp_half(qb, ob, lb, db, 1, s1, dp1);
    pds_half(s0, dp0, p0, d0);
    __builtin_amdgcn_sched_group_barrier(0x100, 10, 0);
#pragma unroll
    for (int n = 0; n < 10; ++n) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    if (__builtin_expect(masked, 0)) mask_half(i, 1, s1);
    upd_half(qb, ob, 0, p0, d0);
    pds_half(s1, dp1, p1, d1);
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    }
    upd_half(qb, ob, 1, p1, d1);
  };

  auto step = [&](auto stage_tag, int e) __attribute__((always_inline)) {
    constexpr int STAGE = decltype(stage_tag)::value;
    const unsigned char* const qc = STAGE ? lds_q1 : lds_q0;
    const unsigned char* const oc = STAGE ? lds_o1 : lds_o0;
    const uint2* const lc = STAGE ? lds_l1 : lds_l0;
    const uint2* const dc = STAGE ? lds_d1 : lds_d0;
    const int ent = ent_cur;
    const int in = ent_next >> 8;
    auto next_copies = [&]() __attribute__((always_inline)) {
      if (STAGE)
        copies(in, lds_q0, lds_o0, lds_l0, lds_d0);
      else
        copies(in, lds_q1, lds_o1, lds_l1, lds_d1);
    };
    const int ent_after_raw = (e + 2 < cnt) ? entry(e + 2) : 0;
    if (wave_on && ((ent >> (wave >> 1)) & 1)) {
      const int i = ent >> 8;
      const bool masked = CROSS ? (64 * i + 63 >= P.N || 64 * kblk + 63 >= key_end)
                                : (64 * i + 63 >= P.N || (64 * i < P.C && 64 * kblk + 63 >= P.C));
      block(qc, oc, lc, dc, i, masked, next_copies);
    } else {
      next_copies();
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    ent_cur = ent_next;
    ent_next = __builtin_amdgcn_readfirstlane(ent_after_raw);
  };
  int e = 0;
  for (; e + 1 < cnt; e += 2) {
    step(std::integral_constant<int, 0>{}, e);
    step(std::integral_constant<int, 1>{}, e + 1);
  }
  if (e < cnt) step(std::integral_constant<int, 0>{}, e);

  if constexpr (CROSS) {
    // fp32 partial sums of this chunk, dK already scaled by ln 2: [chunk, BH, kv_len, 64]
    if (kok) {
      const int64_t prow = ((int64_t)chunk * P.bh + bh) * P.kv_len + key;
      float* krow = P.part_dk + prow * 64;
      float* vrow = P.part_dv + prow * 64;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int R = 0; R < 4; ++R) {
          const float4 k4 = {dkt[dt][4 * R] * kLn2, dkt[dt][4 * R + 1] * kLn2, dkt[dt][4 * R + 2] * kLn2,
                             dkt[dt][4 * R + 3] * kLn2};
          const float4 v4 = {dvt[dt][4 * R], dvt[dt][4 * R + 1], dvt[dt][4 * R + 2], dvt[dt][4 * R + 3]};
          *reinterpret_cast<float4*>(krow + 32 * dt + 8 * R + 4 * g) = k4;
          *reinterpret_cast<float4*>(vrow + 32 * dt + 8 * R + 4 * g) = v4;
        }
    }
    return;
  }
  // dK = dK^T ln 2 (Q' carries log2(e)/8), dV = dV^T; key rows written as 8-byte stores of 4
  // channels
  if (kok) {
    uint16_t* krow = P.dk + (base + key) * 64;
    uint16_t* vrow = P.dv + (base + key) * 64;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        uint2 pk, pv;
        pk.x = pack_bf16x2(dkt[dt][4 * R] * kLn2, dkt[dt][4 * R + 1] * kLn2);
        pk.y = pack_bf16x2(dkt[dt][4 * R + 2] * kLn2, dkt[dt][4 * R + 3] * kLn2);
        pv.x = pack_bf16x2(dvt[dt][4 * R], dvt[dt][4 * R + 1]);
        pv.y = pack_bf16x2(dvt[dt][4 * R + 2], dvt[dt][4 * R + 3]);
        *reinterpret_cast<uint2*>(krow + 32 * dt + 8 * R + 4 * g) = pk;
        *reinterpret_cast<uint2*>(vrow + 32 * dt + 8 * R + 4 * g) = pv;
      }
  }
}

// dK, dV of the cross-attention: the chunks' partial sums added in chunk order, rounded to
// bf16; padded text rows (past the batch item's length) are zero.  One thread per 8 channels.
__global__ __launch_bounds__(256) void bwd_cross_reduce_kernel(const BwdParams P) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid >> 3;              // (bh, key)
  const int c = (int)(gid & 7);
  const int64_t rows = (int64_t)P.bh * P.kv_len;
  if (row >= rows) return;
  const int bh = (int)(row / P.kv_len);
  const int key = (int)(row - (int64_t)bh * P.kv_len);
  int len = P.kv_len;
  if (P.kv_lens != nullptr) {
    const int l = P.kv_lens[bh / P.heads];
    len = l < 0 ? 0 : (l < P.kv_len ? l : P.kv_len);
  }
  float dk[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float dv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (key < len) {
    for (int ch = 0; ch < P.n_chunks; ++ch) {
      const int64_t off = (((int64_t)ch * P.bh) * P.kv_len + row) * 64 + 8 * c;
      const float4 k0 = *reinterpret_cast<const float4*>(P.part_dk + off);
      const float4 k1 = *reinterpret_cast<const float4*>(P.part_dk + off + 4);
      const float4 v0 = *reinterpret_cast<const float4*>(P.part_dv + off);
      const float4 v1 = *reinterpret_cast<const float4*>(P.part_dv + off + 4);
      dk[0] += k0.x; dk[1] += k0.y; dk[2] += k0.z; dk[3] += k0.w;
      dk[4] += k1.x; dk[5] += k1.y; dk[6] += k1.z; dk[7] += k1.w;
      dv[0] += v0.x; dv[1] += v0.y; dv[2] += v0.z; dv[3] += v0.w;
      dv[4] += v1.x; dv[5] += v1.y; dv[6] += v1.z; dv[7] += v1.w;
    }
  }
  u32x4 pk, pv;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pk[e] = pack_bf16x2(dk[2 * e], dk[2 * e + 1]);
    pv[e] = pack_bf16x2(dv[2 * e], dv[2 * e + 1]);
  }
  *reinterpret_cast<u32x4*>(P.dk + row * 64 + 8 * c) = pk;
  *reinterpret_cast<u32x4*>(P.dv + row * 64 + 8 * c) = pv;
}

unsigned grid_for(int64_t items) { return (unsigned)((items + 7) / 8 * 8); }

}  // namespace

hipError_t launch_bsa_bwd(const BwdParams& p, hipStream_t stream) {
  const bool cross = p.cross;
  hipError_t e = hipSuccess;
  // the query walks form the per-row terms (row_terms) that the key walk reads
  if (p.bh_rows == 0 && !cross) return hipSuccess;
  if (!cross) {   // self-attention
    hipLaunchKernelGGL(bwd_dq_kernel<false>, dim3(grid_for((int64_t)p.bh * p.n_st)), dim3(kBwdThreads), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dkdv_kernel<false>, dim3(grid_for((int64_t)p.bh * p.n_kg)), dim3(kBwdThreads), 0, stream,
                       p);
    return hipGetLastError();
  }
  // cross-attention; with no query (n_chunks = 0) the reduction writes dK = dV = 0
  if (p.bh_rows > 0) {
    if (p.q_parts > 0)   // the text fits in LDS
      hipLaunchKernelGGL(bwd_dq_cross_resident_kernel, dim3(grid_for((int64_t)p.bh * p.q_parts)), dim3(kBwdThreads),
                         0, stream, p);
    else
      hipLaunchKernelGGL(bwd_dq_kernel<true>, dim3(grid_for((int64_t)p.bh * p.n_st)), dim3(kBwdThreads), 0, stream,
                         p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.n_kg > 0) {
    hipLaunchKernelGGL(bwd_dkdv_kernel<true>, dim3(grid_for((int64_t)p.bh * p.n_kg)), dim3(kBwdThreads), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t reduce_threads = (int64_t)p.bh * p.kv_len * 8;
  if (reduce_threads > 0)
    hipLaunchKernelGGL(bwd_cross_reduce_kernel, dim3((unsigned)((reduce_threads + 255) / 256)), dim3(256), 0, stream,
                       p);
  return hipGetLastError();
}

}  // namespace lcv
