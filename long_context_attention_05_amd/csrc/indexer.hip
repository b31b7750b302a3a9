// indexer.hip -- stage 2a, Lightning Indexer scores (paper notes "DeepSeek-V4: Towards Highly Efficient
// Million-Token Context Intelligence", section 2.3 Eq. 16 and the Indexer excerpt; cosmocat page section 3;
// 67808.cn explainer section 2: 64 indexer heads of dim 128, low-rank queries, FP4).
//
//   s[t][i] = sum_h w[t][h] * max(0, qI[t][h] . kI[i])      for visible i < min(floor(t/m), N)
//
// The per-head dots are a dense contraction [heads x DI] x [DI x entries], so the 64x128 case runs on MFMA
// (v_mfma_f32_32x32x16_bf16): each wave holds 64 keys in registers as the B operand and takes the queries
// (A operand, heads as rows) from LDS, so one key load serves every query of the block (prefill) and the K
// stream is read once (decode).  fp4 keys/queries are widened to bf16 in registers, which is exact (a 2-bit
// significand times a power of two).  Other shapes and fp32 inputs use a vector-ALU kernel.
//
// Every kernel reduces the heads in the same (canonical) order so that exact dots give bit-identical scores: with
// r[h] = max(0, d[h]) and the heads zero padded to a power of two P >= 16, sixteen chains c_j = fl32(w_j r_j)
// followed by fused multiply-adds of heads j + 16, j + 32, ..., then a halving tree c_j += c_(j + L/2) over
// L = 16, 8, 4, 2 (fewer than 16 heads: the products, then the halving tree).  Most of the work is then fused
// multiply-adds within one lane of an MFMA result.  Scores are written to the workspace as order-preserving uint32
// keys.
#include "lca_device.h"
#include "lca_internal.h"

namespace lca {


__host__ __device__ __forceinline__ int nvis_of(long long t, int m, int N) {
  long long v = t / m;
  return (int)(v < N ? v : N);
}

// ------------------------------------------------------------------------------------------------
// vector-ALU kernel: any HI <= 64, DI <= 128, formats F32 / BF16 / FP4
// ------------------------------------------------------------------------------------------------
constexpr int kSimtTile = 32;

__device__ __forceinline__ float load_elem(const lca_tensor& t, long long row, int j) {
  if (t.format == LCA_F32) return ((const float*)t.data)[row * t.dim + j];
  if (t.format == LCA_BF16) return bf16_to_f32(((const uint16_t*)t.data)[row * t.dim + j]);
  // FP4
  uint32_t byte = ((const uint8_t*)t.data)[row * (t.dim / 2) + (j >> 1)];
  uint32_t code = (j & 1) ? (byte >> 4) : (byte & 15u);
  int e = (int)((const uint8_t*)t.scale)[row * (t.dim / kFp4Block) + j / kFp4Block] - 127;
  return fp4_value(code) * exp2i(e);
}

__global__ __launch_bounds__(256) void idx_score_simt(IdxArgs a) {
#pragma clang fp contract(off)
  __shared__ float q_s[64 * 128];
  __shared__ float k_s[kSimtTile * 129];
  __shared__ float p_s[kSimtTile * 65];
  const int b = blockIdx.z, r = blockIdx.y;
  const long long t = seq_position(a.seq_pos, a.q_start, b) + r;
  const int nvis = nvis_of(t, a.m, a.N);
  const int e0 = blockIdx.x * kSimtTile;
  if (e0 >= nvis) return;
  const int HI = a.HI, DI = a.DI;
  const long long qrow0 = ((long long)b * a.Sq + r) * HI;
  for (int x = threadIdx.x; x < HI * DI; x += blockDim.x) q_s[x] = load_elem(a.q, qrow0 + x / DI, x % DI);
  for (int x = threadIdx.x; x < kSimtTile * DI; x += blockDim.x) {
    int e = x / DI, j = x % DI;
    k_s[e * 129 + j] = (e0 + e < nvis) ? load_elem(a.k, tensor_row(a.k, b, e0 + e), j) : 0.0f;
  }
  __syncthreads();
  const float* wr = a.w + ((long long)b * a.Sq + r) * HI;
  const int e = threadIdx.x % kSimtTile;
  for (int h = threadIdx.x / kSimtTile; h < HI; h += blockDim.x / kSimtTile) {
    float d = 0.0f;
    for (int j = 0; j < DI; ++j) d = fmaf(q_s[h * DI + j], k_s[e * 129 + j], d);
    p_s[e * 65 + h] = fmaxf(d, 0.0f);
  }
  __syncthreads();
  // the canonical head sum: with the heads padded to a power of two P, sixteen chains c_j = w_j r_j, then fused
  // multiply-adds of heads j + 16, j + 32, ... (P >= 16), or the P products (P < 16); then a halving tree
  if (threadIdx.x < kSimtTile && e0 + threadIdx.x < nvis) {
    int P = 1;
    while (P < HI) P <<= 1;
    const float* rr = p_s + threadIdx.x * 65;
    float v[64];
    int L = P;
    if (P >= 16) {
      for (int j = 0; j < 16; ++j) {
        float c = (j < HI) ? wr[j] * rr[j] : 0.0f;
        for (int h = j + 16; h < HI; h += 16) c = __builtin_fmaf(wr[h], rr[h], c);
        v[j] = c;
      }
      L = 16;
    } else {
      for (int h = 0; h < P; ++h) v[h] = (h < HI) ? wr[h] * rr[h] : 0.0f;
    }
    for (; L > 1; L >>= 1)
      for (int j = 0; j < L / 2; ++j) v[j] = v[j] + v[j + L / 2];
    a.keys[((long long)b * a.Sq + r) * a.N + e0 + threadIdx.x] = score_key(v[0]);
  }
}

// ------------------------------------------------------------------------------------------------
// MFMA kernel: HI = 64, DI = 128, BF16 or FP4 operands
// ------------------------------------------------------------------------------------------------
// Lane layouts of v_mfma_f32_32x32x16_bf16 (wave64):
//   A (32 x 16): lane l holds A[l % 32][8 * (l / 32) + v], v = 0..7
//   B (16 x 32): lane l holds B[8 * (l / 32) + v][l % 32]
//   D (32 x 32): lane l, register r holds D[8 * (r / 4) + 4 * (l / 32) + (r % 4)][l % 32]
// The contraction index of K-step s (0..7) is mapped to channel 64 * (l / 32) + 8 * s + v, the same for A and
// B, so each lane reads 128 contiguous bytes of one key row.
constexpr int kMfmaEntriesPerWave = 64;
constexpr int kMfmaEntriesPerBlock = 4 * kMfmaEntriesPerWave;
constexpr int kQStride = 136;  // bf16 elements per query head row in LDS (128 + 8 padding: no bank conflicts)


// Eight consecutive fp4 codes (one little-endian uint32) with their scale, widened to eight bf16 (exact).
__device__ __forceinline__ uint4 fp4x8_to_bf16x8(uint32_t codes, int e) {
  const float s = exp2i(e);
  uint4 r;
  r.x = pack_bf16x2(fp4_value(codes & 15u) * s, fp4_value((codes >> 4) & 15u) * s);
  r.y = pack_bf16x2(fp4_value((codes >> 8) & 15u) * s, fp4_value((codes >> 12) & 15u) * s);
  r.z = pack_bf16x2(fp4_value((codes >> 16) & 15u) * s, fp4_value((codes >> 20) & 15u) * s);
  r.w = pack_bf16x2(fp4_value((codes >> 24) & 15u) * s, fp4_value((codes >> 28) & 15u) * s);
  return r;
}

// 64 consecutive channels [64g, 64g + 64) of one row as eight 8-channel chunks.
template <int FMT>
__device__ __forceinline__ void load_row64(const lca_tensor& t, long long row, int g, uint4 (&out)[8]) {
  if (FMT == LCA_BF16) {
    const uint4* p = (const uint4*)((const uint16_t*)t.data + row * 128 + 64 * g);
#pragma unroll
    for (int s = 0; s < 8; ++s) out[s] = p[s];
  } else {
    // channels 64 g .. 64 g + 63 are blocks 2 g and 2 g + 1: chunk s (8 channels) is in block 2 g + s / 4
    const uint4* p = (const uint4*)((const uint8_t*)t.data + row * 64 + 32 * g);
    uint4 c0 = p[0], c1 = p[1];
    const uint32_t sc = *(const uint16_t*)((const uint8_t*)t.scale + row * 4 + 2 * g);
    uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
    for (int s = 0; s < 8; ++s) out[s] = fp4x8_to_bf16x8(cw[s], (int)((sc >> (8 * (s >> 2))) & 255u) - 127);
  }
}

// One query row's 64 x 128 block (bf16; fp4 widened exactly) as 4 chunks of 8 channels per thread of 256.
template <int FMT>
__device__ __forceinline__ void load_qblock(const IdxArgs& a, long long qrow0, u32x4_t (&v)[4]) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int chunk = threadIdx.x + 256 * it;  // 1024 chunks of 8 channels
    const int h = chunk >> 4, c8 = chunk & 15;
    if constexpr (FMT == LCA_BF16) {
      v[it] = *(gbl_u32x4_t*)((const uint16_t*)a.q.data + (qrow0 + h) * 128 + 8 * c8);
    } else {
      const uint32_t codes = *(const uint32_t*)((const uint8_t*)a.q.data + (qrow0 + h) * 64 + 4 * c8);
      const int e = (int)((const uint8_t*)a.q.scale)[(qrow0 + h) * 4 + (c8 >> 2)] - 127;
      const uint4 w = fp4x8_to_bf16x8(codes, e);
      v[it] = u32x4_t{w.x, w.y, w.z, w.w};
    }
  }
}

// Score of key l % 32 from the 32x32 results of the two head tiles (every lane of the key returns it), in the
// canonical order: chain j (heads j, j + 16, j + 32, j + 48) is c_j = w r, then three fused multiply-adds; then
// the halving tree c_j + c_(j+8), + c_(j+4), + c_(j+2), + c_(j+1).  Register k of tile T holds head
// 32 T + 8 (k / 4) + 4 hh + k % 4, so lane half hh holds the whole chains j = 4 hh + r (registers r, 8 + r of both
// tiles) and j = 8 + 4 hh + r (registers 4 + r, 12 + r): the chains and the +8 step run in lane, +4 across the lane
// halves, +2 across them again after the scattered swap, +1 in lane.
__device__ __forceinline__ float head_tree32(const f32x16_t (&acc)[2], const float (&wv)[2][16]) {
  auto relu = [&](int T, int k) { return __int_as_float(max(__float_as_int(acc[T][k]), 0)); };
  float t[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float ca = wv[0][r] * relu(0, r);
    ca = __builtin_fmaf(wv[0][8 + r], relu(0, 8 + r), ca);
    ca = __builtin_fmaf(wv[1][r], relu(1, r), ca);
    ca = __builtin_fmaf(wv[1][8 + r], relu(1, 8 + r), ca);
    float cb = wv[0][4 + r] * relu(0, 4 + r);
    cb = __builtin_fmaf(wv[0][12 + r], relu(0, 12 + r), cb);
    cb = __builtin_fmaf(wv[1][4 + r], relu(1, 4 + r), cb);
    cb = __builtin_fmaf(wv[1][12 + r], relu(1, 12 + r), cb);
    t[r] = ca + cb;  // +8
  }
  // +4 across the lane halves, scattered: the low half keeps classes 0 and 1, the high half 2 and 3
  const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(t[0]), __float_as_uint(t[2]), false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(t[1]), __float_as_uint(t[3]), false, false);
  const float u02 = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
  const float u13 = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
  return xor32_sum(u02) + xor32_sum(u13);  // +2 across the halves, then +1
}

template <int FMT>
__global__ __launch_bounds__(256) void idx_score_mfma(IdxArgs a, int qpb) {
#pragma clang fp contract(off)
  // query blocks double-buffered in LDS: the next row's block is loaded into registers while this row is scored
  __shared__ uint16_t q_s[2][64 * kQStride];
  __shared__ float w_s[2][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int g = lane >> 5, col = lane & 31;
  const int b = blockIdx.z;
  const int e0 = blockIdx.x * kMfmaEntriesPerBlock + wave * kMfmaEntriesPerWave;
  const int r_begin = blockIdx.y * qpb;
  const int r_end = min(r_begin + qpb, a.Sq);
  const long long qpos = seq_position(a.seq_pos, a.q_start, b);
  const int nvis_last = nvis_of(qpos + r_end - 1, a.m, a.N);
  if (blockIdx.x * kMfmaEntriesPerBlock >= nvis_last) return;  // whole block invisible to every query

  // keys of this wave: two 32-entry column tiles, B operand for 8 K-steps each
  bf16x8_t kb[2][8];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = e0 + 32 * u + col;
    uint4 raw[8];
    if (e < nvis_last) {
      load_row64<FMT>(a.k, tensor_row(a.k, b, e), g, raw);
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) raw[s] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) kb[u][s] = __builtin_bit_cast(bf16x8_t, raw[s]);
  }

  u32x4_t qn[4];
  float wn = 0.0f;
  auto stage = [&](int buf) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int chunk = threadIdx.x + 256 * it;
      *(u32x4_t*)&q_s[buf][(chunk >> 4) * kQStride + 8 * (chunk & 15)] = qn[it];
    }
    if (threadIdx.x < 64) w_s[buf][threadIdx.x] = wn;
  };
  load_qblock<FMT>(a, ((long long)b * a.Sq + r_begin) * 64, qn);
  if (threadIdx.x < 64) wn = a.w[((long long)b * a.Sq + r_begin) * 64 + threadIdx.x];
  stage(0);
  __syncthreads();

  for (int r = r_begin; r < r_end; ++r) {
    const int cur = (r - r_begin) & 1;
    {  // the next row's block is in flight while this row is scored (the last row reloads itself, unused)
      const int rn = min(r + 1, r_end - 1);
      load_qblock<FMT>(a, ((long long)b * a.Sq + rn) * 64, qn);
      if (threadIdx.x < 64) wn = a.w[((long long)b * a.Sq + rn) * 64 + threadIdx.x];
    }
    const int nvis = nvis_of(qpos + r, a.m, a.N);
    if (e0 < nvis) {  // wave-uniform
      f32x16_t acc[2][2];
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int x = 0; x < 16; ++x) acc[T][u][x] = 0.0f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
#pragma unroll
        for (int T = 0; T < 2; ++T) {
          const uint4 qv = *(const uint4*)&q_s[cur][(32 * T + col) * kQStride + 64 * g + 8 * s];
          const bf16x8_t qa = __builtin_bit_cast(bf16x8_t, qv);
#pragma unroll
          for (int u = 0; u < 2; ++u)
            acc[T][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kb[u][s], acc[T][u], 0, 0, 0);
        }
      }
      // epilogue: head h = 32T + 8(x/4) + 4g + (x%4) for register x; the canonical reduction over h
      float wv[2][16];
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int x = 0; x < 16; ++x) wv[T][x] = w_s[cur][32 * T + 8 * (x >> 2) + 4 * g + (x & 3)];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const f32x16_t au[2] = {acc[0][u], acc[1][u]};
        const float sc = head_tree32(au, wv);
        const int e = e0 + 32 * u + col;
        if (g == 0 && e < nvis) a.keys[((long long)b * a.Sq + r) * a.N + e] = score_key(sc);
      }
    }
    stage(cur ^ 1);
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------------
// decode kernels (up to kDecodeMaxRows query rows per sequence): the key stream is the whole cost
// ------------------------------------------------------------------------------------------------
// Grid y is the query row b * Sq + r.  With several rows the grid's x extent (key ranges) is rounded up to a multiple
// of eight, the XCD count: the workgroups of a sequence's rows for one key range are then a multiple of eight apart
// in dispatch order, so they run on one XCD at about the same time and the later rows read the keys from its L2
// rather than from memory.  The padding workgroups find no keys and exit.
// Both formats use 16-key MFMA column blocks whose B operand is a run of whole cache rows, so each lane loads its
// operand bytes straight from HBM into registers (no LDS staging, no barriers in the loop).  A wave streams its own
// slab of keys in stages; the next stage's loads are issued, unconditionally, before the current stage is scored,
// so the wait for a stage's data never drains the loads behind it.  Past the end of the workgroup's range the
// addresses clamp to its last key (loaded, scored, never written).
//
// Accumulator layout of both 16x16 MFMAs: lane l, register r holds head 16 T + 4 (l / 16) + r (M-tile T) for key
// l % 16.  The canonical reduction over the 64 heads is then: the chain of head j = 4 (l / 16) + r over T in-lane,
// +8 (lanes l, l ^ 32) and +4 (l, l ^ 16) across lanes, +2 and +1 in-lane.
//
// With a row histogram to fill (decode select), each workgroup counts its keys' bits [31:21] in LDS and adds the
// counts into the row's histogram, zeroed before the launch.  The select that follows reads it instead of making
// its own first pass over the keys.

// In-lane part of the tree for one 16-key group: the canonical chain of head j = 4 (l / 16) + r over heads j + 16 T,
// v[r] = fma(w r (T=3), fma(w r (T=2), fma(w r (T=1), w r (T=0)))).  ReLU is one integer max of the bit pattern
// with 0: non-negative floats order like their bit patterns and every negative one (-0 included) has the sign bit
// set, so the result equals max(x, 0) without the float max's NaN canonicalization.
__device__ __forceinline__ void head_partial(const f32x4_t (&acc)[4], const float (&wv)[4][4], float (&v)[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float c = wv[0][r] * __int_as_float(max(__float_as_int(acc[0][r]), 0));
#pragma unroll
    for (int T = 1; T < 4; ++T) c = __builtin_fmaf(wv[T][r], __int_as_float(max(__float_as_int(acc[T][r]), 0)), c);
    v[r] = c;
  }
}

// Cross-lane part for four groups at once, as a reduce-scatter over the chains: +8 pairs lane rows g and g + 2
// (lanes l, l ^ 32), +4 pairs rows g and g + 1 (l, l ^ 16), then +2 and +1 in-lane.  permlane32_swap(A, B) returns (A.lo, B.lo) and
// (A.hi, B.hi), so one swap and one add leave group 0 (2)'s pair sums in the low (high) half; permlane16_swap does
// the same for rows 0/1 and 2/3.  Row g of the wave ends with group g's four partial sums, and the lane returns the
// score of group g, key l % 16.  The pairs are those of the canonical halving tree over the chains (fp32
// addition is commutative).
__device__ __forceinline__ float head_cross4(const float (&v)[4][4]) {
  float s02[4], s13[4], t[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0][r]), __float_as_uint(v[2][r]), false, false);
    s02[r] = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[1][r]), __float_as_uint(v[3][r]), false, false);
    s13[r] = __uint_as_float(c[0]) + __uint_as_float(c[1]);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const auto d = __builtin_amdgcn_permlane16_swap(__float_as_uint(s02[r]), __float_as_uint(s13[r]), false, false);
    t[r] = __uint_as_float(d[0]) + __uint_as_float(d[1]);
  }
  return (t[0] + t[2]) + (t[1] + t[3]);
}

__device__ __forceinline__ void flush_hist(const int* hist_s, int* gh) {
  __syncthreads();
  if (blockDim.x == 512) {  // every bin's count read at once, then the adds
    int c[kSelBins / 512];
#pragma unroll
    for (int u = 0; u < kSelBins / 512; ++u) c[u] = hist_s[threadIdx.x + 512 * u];
#pragma unroll
    for (int u = 0; u < kSelBins / 512; ++u)
      if (c[u]) atomicAdd(&gh[threadIdx.x + 512 * u], c[u]);
    return;
  }
  for (int i = threadIdx.x; i < kSelBins; i += blockDim.x) {
    const int c = hist_s[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

// Scores of four 16-key groups (lane (g, col) holds group q0 + g's score after the head tree), so that one store
// writes 64 keys.  The store is unconditional -- a lane past the range holds the
// score of the clamped key k1 - 1 and writes that same value there -- and is issued after the next stage's loads,
// so no branch or register reuse separates the loads in flight from their waits.
struct KeyOut {
  uint32_t key;
  int e;
};

__device__ __forceinline__ KeyOut lane_key(int gbase, int g, float s) {
  return KeyOut{score_key(s), gbase + 16 * g + (int)(threadIdx.x & 15)};
}

__device__ __forceinline__ void store_key(const IdxArgs& a, int b, int k1, const KeyOut& o, int* hist_s, bool hist) {
  a.keys[(long long)b * a.N + min(o.e, k1 - 1)] = o.key;
  if (hist && o.e < k1) atomicAdd(&hist_s[o.key >> 21], 1);
}

// Keys [k0, k1) of sequence b for the workgroup; the slab of wave w in stage st starts at k0 + st * 4 * KPW + w * KPW,
// KPW = 16 * groups keys.

// ---- bf16: v_mfma_f32_16x16x32_bf16, A = queries (lane: head 16T + l % 16, channels 8 (l / 16) + 32 s + v),
//      B = keys (lane: key l % 16, the same channels), i.e. 16 bytes at 16 (l / 16) + 64 s of the 256-byte row.
constexpr int kBfGroups = 4;  // 16-key groups per wave per stage (16 KB per wave in flight); the tree takes 4

struct BfStage {
  uint4 c[kBfGroups][4];
};

// Key e of the wave's keys kbase .. kbase + 63 (kbase a multiple of 64) is row b * cap + e of a dense cache; in a
// paged one (blocks of at least 32 rows) it sits in block blk[0] (keys kbase .. + 31) or blk[1] (the rest).
__device__ __forceinline__ void bf_load_stage(BfStage& S, const uint8_t* kd, long long dense0, const int (&blk)[2],
                                              int br, int kbase, int klast, int lane) {
  const int g = lane >> 4, col = lane & 15;
#pragma unroll
  for (int j = 0; j < kBfGroups; ++j) {
    const int e = min(kbase + 16 * j + col, klast);
    const long long row = br ? (long long)blk[j >= 2] * br + (e & (br - 1)) : dense0 + e;
#pragma unroll
    for (int s = 0; s < 4; ++s) S.c[j][s] = *(const uint4*)(kd + row * 256 + 16 * g + 64 * s);
  }
}

// NR query rows (consecutive rows of one sequence) per workgroup: each key stage is loaded once and scored for every
// row.  One row keeps two workgroups per CU (at most 256 registers a wave); two rows hold both rows' query blocks
// and take one workgroup per CU, whose waves may use the whole register file.
template <int NST, int NR>
__global__ __launch_bounds__(256, NR == 1 ? 2 : 1) void idx_score_decode_bf16(IdxArgs a) {
#pragma clang fp contract(off)
  __shared__ int hist_s[NR][kSelBins];
  constexpr int KPW = 16 * kBfGroups;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int g = lane >> 4, col = lane & 15;
  const int qrow0 = blockIdx.y * NR, b = qrow0 / a.Sq;  // query rows qrow0 .. qrow0 + NR - 1, all of sequence b
  const long long pos0 = seq_position(a.seq_pos, a.q_start, b) + (qrow0 - b * a.Sq);
  int nv[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) nv[r] = nvis_of(pos0 + r, a.m, a.N);
  const int nvis = nv[NR - 1];  // the group's last row sees the most entries
  const int k0 = blockIdx.x * (NST * 4 * KPW);
  const int k1 = min(k0 + NST * 4 * KPW, nvis);
  if (k0 >= k1) return;
  const bool hist = a.sel_state != nullptr;
  if (hist)
    for (int i = threadIdx.x; i < NR * kSelBins; i += blockDim.x) (&hist_s[0][0])[i] = 0;
  const uint8_t* kd = (const uint8_t*)a.k.data;
  // paged: every stage's blocks, resolved before the stream starts (wave-uniform table reads)
  const int br = a.k.block_table ? a.k.block_rows : 0;
  const long long dense0 = (long long)b * a.k.cap;
  int blk[NST][2];
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    blk[st][0] = blk[st][1] = 0;
    if (br) {
      const int kbase = k0 + st * 4 * KPW + wave * KPW;
      const int sh = __builtin_ctz((unsigned)br);
      const long long tb = (long long)b * (a.k.cap >> sh);
      const int kl = min(kbase, k1 - 1), kh = min(kbase + 32, k1 - 1);
      blk[st][0] = a.k.block_table[tb + (kl >> sh)];
      blk[st][1] = a.k.block_table[tb + (kh >> sh)];
    }
  }

  BfStage S[2];
  bf_load_stage(S[0], kd, dense0, blk[0], br, k0 + wave * KPW, k1 - 1, lane);
  bf16x8_t qa[NR][4][4];
  float wv[NR][4][4];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      const uint8_t* qp = (const uint8_t*)a.q.data + ((long long)(qrow0 + r) * 64 + 16 * T + col) * 256;
#pragma unroll
      for (int s = 0; s < 4; ++s) qa[r][T][s] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(qp + 16 * g + 64 * s));
#pragma unroll
      for (int x = 0; x < 4; ++x) wv[r][T][x] = a.w[(long long)(qrow0 + r) * 64 + 16 * T + 4 * g + x];
    }
  if (hist) __syncthreads();  // histogram zeroed before any update

  // straight-line stages (fully unrolled): the next stage's loads are in flight while this one is scored, and each
  // stage's keys are stored after the following stage's loads are issued
  KeyOut pend[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) pend[r] = KeyOut{0u, k1};
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    const int kbase = k0 + st * 4 * KPW + wave * KPW;
    if (st + 1 < NST) {
      bf_load_stage(S[(st + 1) & 1], kd, dense0, blk[st + 1], br, kbase + 4 * KPW, k1 - 1, lane);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the scoring
    }
    if (st > 0)
#pragma unroll
      for (int r = 0; r < NR; ++r)
        store_key(a, qrow0 + r, k1, pend[r], hist_s[r], hist && pend[r].e < nv[r]);
    const BfStage& C = S[st & 1];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      float v[kBfGroups][4];
#pragma unroll
      for (int j = 0; j < kBfGroups; ++j) {
        f32x4_t acc[4];
#pragma unroll
        for (int T = 0; T < 4; ++T) acc[T] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8_t kv = __builtin_bit_cast(bf16x8_t, C.c[j][s]);
#pragma unroll
          for (int T = 0; T < 4; ++T)
            acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[r][T][s], kv, acc[T], 0, 0, 0);
        }
        head_partial(acc, wv[r], v[j]);
      }
      pend[r] = lane_key(kbase, g, head_cross4(v));
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) store_key(a, qrow0 + r, k1, pend[r], hist_s[r], hist && pend[r].e < nv[r]);
  if (hist)
#pragma unroll
    for (int r = 0; r < NR; ++r) flush_hist(hist_s[r], a.sel_state + (long long)(qrow0 + r) * kSelStateInts);
}

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;

// ---- fp4 decode scoring with the keys streamed into an LDS ring: one workgroup of eight waves per CU takes NST
// stages of 512 keys.  A stage's codes (32 KB) and scales (2 KB) travel from memory straight into a ring slot with
// buffer loads into LDS (no registers hold data in flight), three stages in flight while one is scored; each slot is
// its own pair of LDS variables and the stage loop is fully unrolled, so every wait is a count fixed at compile
// time.  Each wave moves and scores its own 64 keys of a stage, so waves never wait for each other.  Code rows are
// stored with their four 16-byte chunks XOR-swizzled by bits 2..3 of the key's position in its 16-key group, which
// makes the operand reads bank-conflict free.
//
// Scoring runs on v_mfma_scale_f32_32x32x64_f8f6f4, which takes fp4 operands at twice the rate of the 16x16x128
// form: A = 32 heads (lane l: head l % 32, contraction slots 32 (l / 32) .. + 31), B = 32 keys (lane l: key l % 32,
// the same slots), one E8M0 scale per lane applied to the lane's 32 slots -- exactly the cache's 32-element scale
// block.  Lane half hh takes code chunk (block) c = 2 i + hh in instruction i, both operands with that block's scale
// (the instruction's byte select picks it from the row's scale word), so four instructions (2 head tiles x 2 chunk
// pairs) give the 64 x 32 dots.  Products of fp4 values and their block sums are exact, scaled by powers of two, so
// the per-head dots equal the exact ones whenever they fit fp32 -- the fixed head-reduction order then makes the
// scores bit-reproducible.  Lane l, register k of the 32x32 result holds head 32 T + 8 (k / 4) + 4 hh + k % 4 for
// key l % 32: the chains and the +8 step run in lane, +4 and +2 across the lane halves, +1 in lane -- the same pairs
// as the 16x16 kernels.
constexpr int kF4rWaves = 8;
constexpr int kF4rStage = 64 * kF4rWaves;  // keys per stage
constexpr int kF4rCodeB = kF4rStage * 64;  // 32 KB
constexpr int kF4rScaleB = kF4rStage * 4;  // 2 KB: four scale bytes per key
__shared__ __attribute__((aligned(16))) uint8_t f4r_c0[kF4rCodeB];
__shared__ __attribute__((aligned(16))) uint8_t f4r_c1[kF4rCodeB];
__shared__ __attribute__((aligned(16))) uint8_t f4r_c2[kF4rCodeB];
__shared__ __attribute__((aligned(16))) uint8_t f4r_c3[kF4rCodeB];
__shared__ __attribute__((aligned(16))) uint8_t f4r_s0[kF4rScaleB];
__shared__ __attribute__((aligned(16))) uint8_t f4r_s1[kF4rScaleB];
__shared__ __attribute__((aligned(16))) uint8_t f4r_s2[kF4rScaleB];
__shared__ __attribute__((aligned(16))) uint8_t f4r_s3[kF4rScaleB];
// Row histograms of pass 1 in LDS, one per query row the workgroup scores (with 4 slots of codes and scales, two rows
// take 152 of the 160 KB of a CU's LDS).
constexpr int kF4rMaxRows = 2;
__shared__ int f4r_hist[kF4rMaxRows * kSelBins];

template <int S>
__device__ __forceinline__ uint8_t* f4r_codes() {
  if constexpr (S == 0) return f4r_c0;
  else if constexpr (S == 1) return f4r_c1;
  else if constexpr (S == 2) return f4r_c2;
  else return f4r_c3;
}
template <int S>
__device__ __forceinline__ uint8_t* f4r_scales() {
  if constexpr (S == 0) return f4r_s0;
  else if constexpr (S == 1) return f4r_s1;
  else if constexpr (S == 2) return f4r_s2;
  else return f4r_s3;
}

typedef __attribute__((address_space(3))) void idx_lds_void_t;
typedef __attribute__((address_space(3))) int idx_lds_int_t;

// Adds one to an LDS counter without a result.  Written as an instruction of its own, so that the compiler does not
// wait for the LDS-direct loads in flight before it (it cannot tell that they write other LDS addresses); LDS
// operations complete in order, so the compiler's own counts of outstanding LDS operations stay safe.
__device__ __forceinline__ void lds_count_one(int* p) {
  const uint32_t addr = (uint32_t)(uintptr_t)(idx_lds_int_t*)p;
  asm volatile("ds_add_u32 %0, %1" : : "v"(addr), "v"(1));
}
constexpr int kIdxBufWord3 = 0x00020000;  // buffer descriptor word 3: raw untyped loads

// s_waitcnt immediate for vmcnt(n) with the other counters untouched
__host__ __device__ constexpr int vm_wait_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (0xF << 8) | (7 << 4); }

// Memory operations a wave has issued after the loads of stage st when step st waits for them: the loads of the
// (at most two) stages after it and the key stores of the steps since they were issued (5 loads per stage: 4 code
// rows of 1 KB and one row of 256 scale bytes; nr stores per step, one per query row).
__host__ __device__ constexpr int f4r_wait_count(int st, int nst, int nr) {
  const int later = (st + 2 < nst - 1 ? st + 2 : nst - 1) - st;
  const int stores = st - (st - 3 > 0 ? st - 3 : 0);
  return 5 * later + nr * stores;
}

// Calls f(integral_constant<int, ST>) for ST = ST0 .. NST - 1 in order (a loop whose index is a constant).
template <int ST, int NST, class F>
__device__ __forceinline__ void unroll_steps(F& f) {
  if constexpr (ST < NST) {
    f(std::integral_constant<int, ST>{});
    unroll_steps<ST + 1, NST>(f);
  }
}

// NR query rows (consecutive rows of one sequence) per workgroup: every key stage is loaded once and scored for each
// row, its key operands read from LDS once for all of them.
template <int NST, int NR, bool PAGED>
__global__ __launch_bounds__(kF4rWaves * 64) void idx_score_decode_fp4_ring(IdxArgs a) {
#pragma clang fp contract(off)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int col = lane & 31, hh = lane >> 5;
  const int qrow0 = blockIdx.y * NR, b = qrow0 / a.Sq;  // query rows qrow0 .. qrow0 + NR - 1, all of sequence b
  const long long pos0 = seq_position(a.seq_pos, a.q_start, b) + (qrow0 - b * a.Sq);
  int nv[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) nv[r] = nvis_of(pos0 + r, a.m, a.N);
  const int nvis = nv[NR - 1];  // the group's last row sees the most entries
  const int k0 = blockIdx.x * (NST * kF4rStage);
  const int k1 = min(k0 + NST * kF4rStage, nvis);
  if (k0 >= k1) return;  // block-uniform
  const bool hist = a.sel_state != nullptr;
  for (int i = threadIdx.x; i < NR * kSelBins; i += blockDim.x) f4r_hist[i] = 0;
  if (hist) __syncthreads();  // the histograms are zeroed before any count (nothing is in flight yet)

  // The body in two forms: FAST for a dense cache and a workgroup whose NST stages are all below k1 (every workgroup
  // of a row but its last), which addresses a stage through a descriptor of its own and a constant lane offset (no
  // vector instructions per load); otherwise every key index is clamped to k1 - 1.  One branch per workgroup picks
  // the form, so neither has a branch inside its stage loop.
  auto body = [&](auto FASTC) {
  constexpr bool FAST = decltype(FASTC)::value;
  // queries: head tile T = heads 32 T .. 32 T + 31, lane head 32 T + col; chunks (blocks) hh and 2 + hh of its code
  // row and its scale word.  The raw loads go first and the operands are built after the ring's first loads are
  // issued, so that nothing waits for the queries before the ring starts.
  uint4 qraw[NR][2][2];
  uint32_t sraw[NR][2];
  float wv[NR][2][16];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      const long long row = (long long)(qrow0 + r) * 64 + 32 * T + col;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        qraw[r][T][i] = *(const uint4*)((const uint8_t*)a.q.data + row * 64 + 16 * (2 * i + hh));
      sraw[r][T] = *(const uint32_t*)((const uint8_t*)a.q.scale + row * 4);
      // weights of heads 32 T + 8 a + 4 hh + c, c = 0..3: four consecutive floats per a, one 16-byte load each when
      // the weights start 16-byte aligned
      const float* wrow = a.w + (long long)(qrow0 + r) * 64 + 32 * T + 4 * hh;
      if (((uintptr_t)a.w & 15u) == 0) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 wq = *(const float4*)(wrow + 8 * q4);
          wv[r][T][4 * q4] = wq.x;
          wv[r][T][4 * q4 + 1] = wq.y;
          wv[r][T][4 * q4 + 2] = wq.z;
          wv[r][T][4 * q4 + 3] = wq.w;
        }
      } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) wv[r][T][k] = wrow[8 * (k >> 2) + (k & 3)];
      }
    }
  __builtin_amdgcn_sched_barrier(0);
  i32x8_t qop[NR][2][2];
  int qs[NR][2];  // bytes 0 and 2: the scales of blocks hh and 2 + hh (the operands qop[..][0] and qop[..][1])

  // buffer descriptors over the workgroup's own keys [k0, k1) of a dense cache (offsets stay small whatever the cache
  // size, and the range check covers exactly the keys the workgroup may read), or over the whole pool of a paged one
  // (blocks of at least 32 rows, pool under 2 GiB of codes: checked on the host)
  const int br = PAGED ? a.k.block_rows : 0;
  const long long rb0 = PAGED ? 0 : (long long)b * a.k.cap + k0;
  const long long nrows = PAGED ? a.k.pool_rows : (long long)(k1 - k0);
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)a.k.data + rb0 * 64), 0, (int)(nrows * 64), kIdxBufWord3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)a.k.scale + rb0 * 4), 0, (int)(nrows * 4), kIdxBufWord3);
  // paged: the blocks of each stage's 64 wave keys (keys 0..31 and 32..63 of the slice), read before the ring starts
  int blk[NST][2];
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    blk[st][0] = blk[st][1] = 0;
    if constexpr (PAGED) {
      const int sh = __builtin_ctz((unsigned)br);
      const long long tb = (long long)b * (a.k.cap >> sh);
      const int kl = min(k0 + st * kF4rStage + 64 * wave, k1 - 1), kh = min(kl + 32, k1 - 1);
      blk[st][0] = a.k.block_table[tb + (kl >> sh)];
      blk[st][1] = a.k.block_table[tb + (kh >> sh)];
    }
  }
  // row (relative to the descriptor) of key kst + 64 w + o, o < 64
  auto key_row = [&](int st, int kst, int o) -> int {
    const int key = min(kst + 64 * wave + o, k1 - k0 - 1);
    if constexpr (PAGED) return blk[st][o >= 32] * br + ((k0 + key) & (br - 1));
    else return key;
  };
  // FAST: the lane's offsets within a stage, one per code instruction (kept in registers: an instruction's immediate
  // offset would move its LDS destination as well)
  const int vcode0 = (64 * wave + (lane >> 2)) * 64 + 16 * ((lane & 3) ^ (lane >> 4));
  const int vcode1 = vcode0 + 1024, vcode2 = vcode0 + 2048, vcode3 = vcode0 + 3072;
  const int vscale = (64 * wave + lane) * 4;
  // stage st into slot S: code instruction i of wave w moves keys 64 w + 16 i .. + 15 (lane l: key + l / 4, chunk
  // position l % 4 holding code chunk (l % 4) ^ (l / 16)); the scale instruction moves the wave's 64 scale words
  // (lane l: key 64 w + l).  Keys past k1 repeat key k1 - 1.
  auto issue = [&](auto SC, int st) {
    constexpr int S = decltype(SC)::value;
    const int kst = st * kF4rStage;  // relative to k0
    uint8_t* const lc = f4r_codes<S>() + 64 * wave * 64;
    uint8_t* const ls = f4r_scales<S>() + 64 * wave * 4;
    if constexpr (FAST) {
      // a descriptor over the stage's own 512 keys (scalar arithmetic), all of them below k1
      const __amdgpu_buffer_rsrc_t cst = __builtin_amdgcn_make_buffer_rsrc(
          (void*)((const uint8_t*)a.k.data + (rb0 + kst) * 64), 0, kF4rStage * 64, kIdxBufWord3);
      const __amdgpu_buffer_rsrc_t sst = __builtin_amdgcn_make_buffer_rsrc(
          (void*)((const uint8_t*)a.k.scale + (rb0 + kst) * 4), 0, kF4rStage * 4, kIdxBufWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(cst, (idx_lds_void_t*)lc, 16, vcode0, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(cst, (idx_lds_void_t*)(lc + 1024), 16, vcode1, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(cst, (idx_lds_void_t*)(lc + 2048), 16, vcode2, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(cst, (idx_lds_void_t*)(lc + 3072), 16, vcode3, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sst, (idx_lds_void_t*)ls, 4, vscale, 0, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = key_row(st, kst, 16 * i + (lane >> 2));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, (idx_lds_void_t*)(lc + 16 * i * 64), 16,
                                                 row * 64 + 16 * ((lane & 3) ^ (lane >> 4)), 0, 0, 0);
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (idx_lds_void_t*)ls, 4, key_row(st, kst, lane) * 4, 0, 0, 0);
    }
  };
  // key operands of the wave's key tile u (keys 64 w + 32 u + col of stage slot S); ks holds the scales of blocks
  // hh and 2 + hh in its bytes 0 and 2, which the instruction's byte select picks
  auto kops = [&](auto SC, int u, i32x8_t (&kop)[2], int& ks) {
    constexpr int S = decltype(SC)::value;
    const int kl = 64 * wave + 32 * u + col;
    const uint8_t* cb = f4r_codes<S>() + kl * 64;
    const int sw = (kl >> 2) & 3;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const u32x4_t kc = *(const u32x4_t*)(cb + 16 * ((2 * i + hh) ^ sw));
      kop[i] = i32x8_t{(int)kc[0], (int)kc[1], (int)kc[2], (int)kc[3], 0, 0, 0, 0};
    }
    ks = (int)(*(const uint32_t*)(f4r_scales<S>() + kl * 4) >> (8 * hh));
  };
  // 64 x 32 dots of query row r against one key tile: block hh (byte 0 of both scale words), then block 2 + hh
  // (byte 2)
  auto dots = [&](const i32x8_t (&kop)[2], int ks, int r, f32x16_t (&acc)[2]) {
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      acc[T] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qop[r][T][0], kop[0], f32x16_t{}, 4, 4, 0, qs[r][T], 0,
                                                               ks);
      acc[T] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qop[r][T][1], kop[1], acc[T], 4, 4, 2, qs[r][T], 2, ks);
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  // the query loads above are older than the ring's, so the first wait covers them
  issue(S0{}, 0);
  if constexpr (NST > 1) issue(S1{}, 1);
  if constexpr (NST > 2) issue(S2{}, 2);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int T = 0; T < 2; ++T) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint4 c = qraw[r][T][i];
        qop[r][T][i] = i32x8_t{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
      }
      qs[r][T] = (int)(sraw[r][T] >> (8 * hh));
    }

  // Stage st sits in slot st % 4.  A wave loads exactly the keys it scores, so the ring needs no barrier: step st
  // waits for this wave's own loads of stage st, starts stage st + 3 in the slot this wave finished with in step
  // st - 1, scores it for every row, stores the keys and counts them in the row histograms.
  auto step = [&](auto STC) {
    constexpr int st = decltype(STC)::value;
    using SC = std::integral_constant<int, st % 4>;
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(f4r_wait_count(st, NST, NR)));
    asm volatile("" ::: "memory");
    if constexpr (st + 3 < NST) issue(std::integral_constant<int, (st + 3) % 4>{}, st + 3);
    i32x8_t kop0[2], kop1[2];
    int ks0, ks1;
    kops(SC{}, 0, kop0, ks0);
    kops(SC{}, 1, kop1, ks1);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      f32x16_t acc0[2], acc1[2];
      dots(kop0, ks0, r, acc0);
      __builtin_amdgcn_sched_barrier(0);
      dots(kop1, ks1, r, acc1);
      const float s0 = head_tree32(acc0, wv[r]);
      // the second tile's MFMAs run while the first tile's tree issues between them
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      const float s1 = head_tree32(acc1, wv[r]);
      const uint32_t key0 = score_key(s0), key1 = score_key(s1);
      // lane (col, hh) stores and counts tile hh's key col: 64 keys per store and row (a lane past k1 held key
      // k1 - 1 and writes its score again, uncounted)
      const int e = k0 + st * kF4rStage + 64 * wave + 32 * hh + col;
      const uint32_t key = hh ? key1 : key0;
      a.keys[(long long)(qrow0 + r) * a.N + (FAST ? e : min(e, k1 - 1))] = key;
      if (hist && ((FAST && NR == 1) || e < nv[r])) lds_count_one(&f4r_hist[r * kSelBins + (key >> 21)]);
    }
  };
  unroll_steps<0, NST>(step);
  if (hist) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
      flush_hist(f4r_hist + r * kSelBins, a.sel_state + (long long)(qrow0 + r) * kSelStateInts);
  }
  };
  if (!PAGED && k1 - k0 == NST * kF4rStage) body(std::true_type{});
  else body(std::false_type{});
}

// key ranges of a decode launch: a multiple of the eight XCDs when several rows share them
static int decode_grid_x(int ranges, int Sq) { return Sq > 1 ? (ranges + 7) & ~7 : ranges; }

// A bf16 row costs the decode kernel a whole pass of MFMAs and head tree per key, while the many-row kernel keeps a
// key tile in registers across rows; with three or four bf16 rows of up to kTopkLdsKeys entries (whose selection
// then runs from LDS) the many-row path is the faster one.
bool indexer_uses_decode_kernel(int B, int Sq, int HI, int DI, int N, int q_format, int k_format) {
  (void)B;
  if (Sq < 1 || Sq > kDecodeMaxRows || HI != 64 || DI != 128 || q_format != k_format) return false;
  if (q_format == LCA_FP4) return true;
  return q_format == LCA_BF16 && (Sq <= 2 || N > kTopkLdsKeys);
}

hipError_t launch_indexer_scores(const IdxArgs& a, hipStream_t st, hipEvent_t eb, hipEvent_t ee) {
  const int nvis_max = nvis_of(a.q_start + a.Sq - 1, a.m, a.N);  // q_start is the largest position of the call
  if (nvis_max <= 0) return hipSuccess;
  clear_stale_error();
  const bool mfma = a.HI == 64 && a.DI == 128 && a.q.format == a.k.format &&
                    (a.q.format == LCA_BF16 || a.q.format == LCA_FP4);
  if (indexer_uses_decode_kernel(a.B, a.Sq, a.HI, a.DI, a.N, a.q.format, a.k.format)) {
    const bool fp4 = a.q.format == LCA_FP4;
    if (fp4) {
      // one workgroup per CU where the context allows: the most stages per workgroup that still leave 256; two query
      // rows of a sequence per workgroup when the rows per sequence are even (each key stage loaded once for both)
      const int nr = a.Sq % 2 == 0 ? 2 : 1;
      const long long groups = (long long)a.B * a.Sq / nr;
      int nst = 8;
      while (nst > 1 && groups * ((nvis_max + nst * kF4rStage - 1) / (nst * kF4rStage)) < 256) nst >>= 1;
      const dim3 grid((unsigned)decode_grid_x((nvis_max + nst * kF4rStage - 1) / (nst * kF4rStage), a.Sq / nr),
                      (unsigned)groups);
      const dim3 block(kF4rWaves * 64);
      const bool paged = a.k.block_table != nullptr;
#define LCA_F4R(NS, R, PG) hipExtLaunchKernelGGL((idx_score_decode_fp4_ring<NS, R, PG>), grid, block, 0, st, eb, ee, 0, a)
#define LCA_F4R_NST(R, PG)                \
  do {                                    \
    if (nst == 8) LCA_F4R(8, R, PG);      \
    else if (nst == 4) LCA_F4R(4, R, PG); \
    else if (nst == 2) LCA_F4R(2, R, PG); \
    else LCA_F4R(1, R, PG);               \
  } while (0)
      if (nr == 2) {
        if (paged) LCA_F4R_NST(2, true);
        else LCA_F4R_NST(2, false);
      } else {
        if (paged) LCA_F4R_NST(1, true);
        else LCA_F4R_NST(1, false);
      }
#undef LCA_F4R_NST
#undef LCA_F4R
      return hipGetLastError();
    }
    // a fixed key range per workgroup (NST stages of 4 waves x KPW keys), the grid grows with the context; fewer
    // stages when that leaves fewer than about two workgroups per CU (one per CU for two rows per workgroup, which
    // also allows eight stages)
    const int kpw = 16 * kBfGroups;
    const int nr = a.Sq % 2 == 0 ? 2 : 1;
    const long long groups = (long long)a.B * a.Sq / nr;
    const long long target = nr == 1 ? 512 : 256;
    int nst = nr == 1 ? 4 : 8;
    while (nst > 1 && groups * ((nvis_max + nst * 4 * kpw - 1) / (nst * 4 * kpw)) < target) nst >>= 1;
    const dim3 grid((unsigned)decode_grid_x((nvis_max + nst * 4 * kpw - 1) / (nst * 4 * kpw), a.Sq / nr),
                    (unsigned)groups);
#define LCA_BFD(NS, R) hipExtLaunchKernelGGL((idx_score_decode_bf16<NS, R>), grid, dim3(256), 0, st, eb, ee, 0, a)
    if (nr == 2) {
      if (nst == 8) LCA_BFD(8, 2);
      else if (nst == 4) LCA_BFD(4, 2);
      else if (nst == 2) LCA_BFD(2, 2);
      else LCA_BFD(1, 2);
    } else {
      if (nst == 4) LCA_BFD(4, 1);
      else if (nst == 2) LCA_BFD(2, 1);
      else LCA_BFD(1, 1);
    }
#undef LCA_BFD
  } else if (mfma) {
    const int qpb = a.Sq >= 16 ? 16 : a.Sq;
    dim3 grid((unsigned)((nvis_max + kMfmaEntriesPerBlock - 1) / kMfmaEntriesPerBlock),
              (unsigned)((a.Sq + qpb - 1) / qpb), (unsigned)a.B);
    if (a.q.format == LCA_BF16)
      hipExtLaunchKernelGGL(idx_score_mfma<LCA_BF16>, grid, dim3(256), 0, st, eb, ee, 0, a, qpb);
    else
      hipExtLaunchKernelGGL(idx_score_mfma<LCA_FP4>, grid, dim3(256), 0, st, eb, ee, 0, a, qpb);
  } else {
    dim3 grid((unsigned)((nvis_max + kSimtTile - 1) / kSimtTile), (unsigned)a.Sq, (unsigned)a.B);
    hipExtLaunchKernelGGL(idx_score_simt, grid, dim3(256), 0, st, eb, ee, 0, a);
  }
  return hipGetLastError();
}

}  // namespace lca
