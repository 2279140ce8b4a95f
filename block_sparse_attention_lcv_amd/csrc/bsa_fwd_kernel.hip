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
//    (64 x 64 bf16) is staged once into LDS for all wavefronts: global -> VGPR prefetch of
//    entry e+1 overlaps the MFMA/softmax work on entry e, then goes to the other LDS
//    buffer (K RoPE applied on the way); one barrier per entry.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K from LDS as the A operand, Q as B), so
//    each lane owns one query column: row statistics need only the partner lane l^32.
//  * Online softmax in the log2 domain with a per-row reference max that only moves when a
//    block's probabilities would exceed 2^8 (lazy rescaling): the common block costs one
//    FMA, one v_exp_f32, half a conversion and half a dot2 per score.  Each row's decisions
//    depend on that row alone, so results do not depend on which other rows share the
//    wavefront (the cached call reproduces the full call bit for bit).
//  * O^T += V^T P^T with the same MFMA: P (bf16) comes straight from the S^T registers, V^T
//    operands come from the row-major V tile through ds_read_b64_tr_b16 transposing reads.
//  * Workgroups are numbered so that each XCD (blockIdx % 8 on MI355X) receives a
//    contiguous range of work items, i.e. whole heads: their shared global key blocks stay
//    in that XCD's L2.
#include "lcv_internal.h"
#include "rope_math.h"

namespace lcv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kThreads = 64 * kWaves;
constexpr int kTileBytes = 64 * 128;            // one 64 x 64 bf16 tile
constexpr int kStageBytes = 2 * kTileBytes;     // K tile + V tile
constexpr int kRopeTabOffset = 2 * kStageBytes; // two stages, then the cos/sin table
constexpr int kChunksPerThread = 512 / kThreads; // 16-byte chunks of a tile per thread
constexpr float kScoreToLog2 = 1.4426950408889634f / 8.0f;  // log2(e) / sqrt(64)
constexpr float kRescaleLimit = 256.0f;                     // lazy-rescale threshold 2^8
constexpr float kLn2 = 0.6931471805599453f;

static_assert(512 % kThreads == 0, "tile chunks must split evenly over the workgroup");

// Byte offset of 16-byte chunk `chunk` of row `row` in a 64 x 64 bf16 tile; chunks are
// XOR-swizzled by the row so that column reads of 8 consecutive rows hit distinct banks.
__device__ __forceinline__ uint32_t tile_off(int row, int chunk) {
  return (uint32_t)(row * 128 + ((chunk ^ (row & 7)) << 4));
}

__device__ __forceinline__ float partner(float x) { return __shfl_xor(x, 32, 64); }

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

__device__ __forceinline__ const uint16_t* key_row_ptr(const FwdParams& P, const uint16_t* cond, const uint16_t* noise,
                                                       int bh, int key) {
  if (key < P.kv_split) return cond + ((int64_t)bh * P.kv_split + key) * 64;
  return noise + ((int64_t)bh * (P.N - P.kv_split) + (key - P.kv_split)) * 64;
}

__device__ __forceinline__ void load_kv(const FwdParams& P, int bh, int j, u32x4 (&kreg)[kChunksPerThread],
                                        u32x4 (&vreg)[kChunksPerThread]) {
#pragma unroll
  for (int c = 0; c < kChunksPerThread; ++c) {
    const int id = (int)threadIdx.x + c * kThreads;
    const int row = id >> 3, ch = id & 7;
    const int key = 64 * j + row;
    if (key < P.N) {
      kreg[c] = *reinterpret_cast<const u32x4*>(key_row_ptr(P, P.k_cond, P.k, bh, key) + 8 * ch);
      vreg[c] = *reinterpret_cast<const u32x4*>(key_row_ptr(P, P.v_cond, P.v, bh, key) + 8 * ch);
    } else {
      kreg[c] = u32x4{0u, 0u, 0u, 0u};
      vreg[c] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

__device__ __forceinline__ void store_kv(const FwdParams& P, unsigned char* stage, int j, bool rope_k,
                                         const float2* tab, u32x4 (&kreg)[kChunksPerThread],
                                         const u32x4 (&vreg)[kChunksPerThread]) {
#pragma unroll
  for (int c = 0; c < kChunksPerThread; ++c) {
    const int id = (int)threadIdx.x + c * kThreads;
    const int row = id >> 3, ch = id & 7;
    const int key = 64 * j + row;
    u32x4 kv = kreg[c];
    if (rope_k && key < P.N) kv = rope_chunk(kv, ch, token_coords((uint32_t)key, P), tab, P);
    *reinterpret_cast<u32x4*>(stage + tile_off(row, ch)) = kv;
    *reinterpret_cast<u32x4*>(stage + kTileBytes + tile_off(row, ch)) = vreg[c];
  }
}

// p = 2^(s * log2(e)/8 - mu) for the 32 scores of query tile qt held by this lane, packed to
// bf16 as the B operand of the four 16-key P*V steps; returns the lane's sum of the
// rounded probabilities.  (The bf16 pairs are built as bf16x2 values and fed to the dot2
// intrinsic directly: taking them out of a u32 vector by bit_cast was mis-optimised by the
// compiler into reusing one pair for several dot2 operands.)
__device__ __forceinline__ float probs(const f32x16 (&s)[2][2], int qt, float mu, bf16x8 (&pb)[4]) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int js = 0; js < 4; ++js) {
    const int kt = js >> 1, base = 8 * (js & 1);
    bf16x2 w[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const f32x2_t p = {__builtin_amdgcn_exp2f(fmaf(s[kt][qt][base + 2 * e2], kScoreToLog2, -mu)),
                         __builtin_amdgcn_exp2f(fmaf(s[kt][qt][base + 2 * e2 + 1], kScoreToLog2, -mu))};
      w[e2] = __builtin_convertvector(p, bf16x2);
    }
    acc0 = __builtin_amdgcn_fdot2_f32_bf16(w[0], ones, acc0, false);
    acc1 = __builtin_amdgcn_fdot2_f32_bf16(w[1], ones, acc1, false);
    acc0 = __builtin_amdgcn_fdot2_f32_bf16(w[2], ones, acc0, false);
    acc1 = __builtin_amdgcn_fdot2_f32_bf16(w[3], ones, acc1, false);
    pb[js] = __builtin_shufflevector(__builtin_shufflevector(w[0], w[1], 0, 1, 2, 3),
                                     __builtin_shufflevector(w[2], w[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
  }
  return acc0 + acc1;
}

__global__ __launch_bounds__(kThreads, 2) void bsa_fwd_kernel(const FwdParams P) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int l32 = lane & 31;

  // ---- work item: XCD x (= blockIdx % 8) takes the x-th contiguous slice of items
  const int per_xcd = (int)(gridDim.x >> 3);
  const int item = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (item >= P.n_items) return;
  const int bh = item / P.n_st_active;
  const int st = P.st_first + (item - bh * P.n_st_active);
  const bool rope_q = (P.flags & LCV_ROPE_Q) != 0;
  const bool rope_k = (P.flags & LCV_ROPE_K) != 0;

  // ---- cos/sin table of every (axis, position, pair) of the grid
  float2* tab = reinterpret_cast<float2*>(smem + kRopeTabOffset);
  if (P.flags) {
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
  }
  __syncthreads();

  // ---- this wavefront's query block, resident as MFMA B operands: qf[qt][ks] holds rows
  // 32*qt + (lane & 31), channels 16*ks + 8*(lane >> 5) .. +7
  const int qblk = st * kWaves + wave;
  const bool wave_on = (qblk < P.n_blocks) && (64 * qblk + 63 >= P.q_row0);
  bf16x8 qf[2][4];
  int qtok[2];
  bool qok[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    qtok[qt] = 64 * qblk + 32 * qt + l32;
    qok[qt] = wave_on && qtok[qt] >= P.q_row0 && qtok[qt] < P.N;
    const uint16_t* qrow = P.q + ((int64_t)bh * P.q_rows + (qtok[qt] - P.q_row0)) * 64;
    Coords xyz{0u, 0u, 0u};
    if (rope_q && qok[qt]) xyz = token_coords((uint32_t)qtok[qt], P);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c = 2 * ks + g;
      u32x4 raw{0u, 0u, 0u, 0u};
      if (qok[qt]) {
        raw = *reinterpret_cast<const u32x4*>(qrow + 8 * c);
        if (rope_q) raw = rope_chunk(raw, c, xyz, tab, P);
      }
      qf[qt][ks] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // ---- walk the workgroup's key-block list
  const int32_t* ents = P.st_ent + P.row_ptr[st * kWaves];
  const int cnt = P.st_cnt[st];

  f32x16 o[2][2];   // O^T tiles [d tile][query tile]
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[a][b][r] = 0.f;
  float mref[2] = {-INFINITY, -INFINITY};
  float lsum[2] = {0.f, 0.f};

  u32x4 kreg[kChunksPerThread], vreg[kChunksPerThread];
  if (cnt > 0) {
    const int j0 = ents[0] >> 8;
    load_kv(P, bh, j0, kreg, vreg);
    store_kv(P, smem, j0, rope_k, tab, kreg, vreg);
  }
  __syncthreads();

  for (int e = 0; e < cnt; ++e) {
    const int ent = ents[e];
    const int j = ent >> 8;
    unsigned char* stage = smem + (e & 1) * kStageBytes;
    int jn = 0;
    if (e + 1 < cnt) {
      jn = ents[e + 1] >> 8;
      load_kv(P, bh, jn, kreg, vreg);
    }

    if (wave_on && ((ent >> wave) & 1)) {
      // S^T[key][query] = K Q^T : s[kt][qt] covers keys 32*kt.., queries 32*qt..
      f32x16 s[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        bf16x8 ka[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          ka[ks] = *reinterpret_cast<const bf16x8*>(stage + tile_off(32 * kt + l32, 2 * ks + g));
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          f32x16 acc;
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[qt][ks], acc, 0, 0, 0);
          s[kt][qt] = acc;
        }
      }

      // token mask where the block pair crosses the end of the sequence or the condition
      // boundary: keys >= N, and noise keys for condition queries
      const int key0 = 64 * j;
      if (key0 + 63 >= P.N || (64 * qblk < P.C && key0 + 63 >= P.C)) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = key0 + 32 * kt + 8 * (r >> 2) + 4 * g + (r & 3);
              const bool ok = key < P.N && (qtok[qt] >= P.C || key < P.C);
              if (!ok) s[kt][qt][r] = -INFINITY;
            }
      }

      // online softmax (log2 domain, lazy rescaling)
      bf16x8 pb[2][4];
      float psum[2];
      bool trig[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const bool uninit = mref[qt] == -INFINITY;
        psum[qt] = probs(s, qt, uninit ? 0.f : mref[qt], pb[qt]);
        const float row_sum = psum[qt] + partner(psum[qt]);
        trig[qt] = uninit || !(row_sum <= kRescaleLimit);
      }
      if (__any(trig[0] || trig[1])) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          float bm = -INFINITY;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) bm = fmaxf(bm, s[kt][qt][r]);
          bm = fmaxf(bm, partner(bm)) * kScoreToLog2;
          const float m_new = trig[qt] ? fmaxf(mref[qt], bm) : mref[qt];
          const float alpha = (m_new == mref[qt]) ? 1.f : __builtin_amdgcn_exp2f(mref[qt] - m_new);
          o[0][qt] *= alpha;
          o[1][qt] *= alpha;
          lsum[qt] *= alpha;
          mref[qt] = m_new;
          psum[qt] = probs(s, qt, (m_new == -INFINITY) ? 0.f : m_new, pb[qt]);
        }
      }
      lsum[0] += psum[0];
      lsum[1] += psum[1];

      // O^T[d][query] += V^T P^T : 16-key steps js, d tiles dt
      const unsigned char* vt = stage + kTileBytes;
#pragma unroll
      for (int js = 0; js < 4; ++js) {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const int krow = 16 * js + 4 * g + ((lane & 15) >> 2);
          const int dcol = 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
          const uint32_t sub = (uint32_t)((dcol >> 2) & 1) * 8u;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(vt + tile_off(krow, dcol >> 3) + sub));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(vt + tile_off(krow + 8, dcol >> 3) + sub));
          const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8 va = __builtin_bit_cast(bf16x8, both);
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) o[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[qt][js], o[dt][qt], 0, 0, 0);
        }
      }
    }

    if (e + 1 < cnt) store_kv(P, smem + ((e + 1) & 1) * kStageBytes, jn, rope_k, tab, kreg, vreg);
    __syncthreads();
  }

  // ---- epilogue: O = O~ / l, LSE = (m + log2 l) * ln 2
  if (wave_on) {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const float lt = lsum[qt] + partner(lsum[qt]);
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
}

}  // namespace

hipError_t launch_bsa_fwd(const FwdParams& p, hipStream_t stream) {
  if (p.n_items == 0) return hipSuccess;
  const unsigned groups = (unsigned)(((int64_t)p.n_items + 7) / 8 * 8);
  const size_t lds = (size_t)kRopeTabOffset + (p.flags ? (size_t)p.rope_entries * sizeof(float2) : 0);
  hipLaunchKernelGGL(bsa_fwd_kernel, dim3(groups), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace lcv
