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
// Both kernels reduce the heads the same way so that exact dots give bit-identical scores:
//   p[h] = fl32(w[h] * max(0, d[h])), then a halving tree a[j] += a[j + L/2] over L = 64, 32, ..., 2
// (zero padded to a power of two).  Scores are written to the workspace as order-preserving uint32 keys.
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
  int e = (int)((const uint8_t*)t.scale)[row * (t.dim / 16) + (j >> 4)] - 127;
  return fp4_value(code) * exp2i(e);
}

__global__ __launch_bounds__(256) void idx_score_simt(IdxArgs a) {
#pragma clang fp contract(off)
  __shared__ float q_s[64 * 128];
  __shared__ float k_s[kSimtTile * 129];
  __shared__ float p_s[kSimtTile * 65];
  const int b = blockIdx.z, r = blockIdx.y;
  const long long t = a.q_start + r;
  const int nvis = nvis_of(t, a.m, a.N);
  const int e0 = blockIdx.x * kSimtTile;
  if (e0 >= nvis) return;
  const int HI = a.HI, DI = a.DI;
  const long long qrow0 = ((long long)b * a.Sq + r) * HI;
  for (int x = threadIdx.x; x < HI * DI; x += blockDim.x) q_s[x] = load_elem(a.q, qrow0 + x / DI, x % DI);
  for (int x = threadIdx.x; x < kSimtTile * DI; x += blockDim.x) {
    int e = x / DI, j = x % DI;
    k_s[e * 129 + j] = (e0 + e < nvis) ? load_elem(a.k, (long long)b * a.k.cap + e0 + e, j) : 0.0f;
  }
  __syncthreads();
  const float* wr = a.w + ((long long)b * a.Sq + r) * HI;
  const int e = threadIdx.x % kSimtTile;
  for (int h = threadIdx.x / kSimtTile; h < HI; h += blockDim.x / kSimtTile) {
    float d = 0.0f;
    for (int j = 0; j < DI; ++j) d = fmaf(q_s[h * DI + j], k_s[e * 129 + j], d);
    p_s[e * 65 + h] = wr[h] * fmaxf(d, 0.0f);
  }
  __syncthreads();
  if (threadIdx.x < kSimtTile && e0 + threadIdx.x < nvis) {
    int P = 1;
    while (P < HI) P <<= 1;
    float v[64];
    for (int h = 0; h < P; ++h) v[h] = (h < HI) ? p_s[threadIdx.x * 65 + h] : 0.0f;
    for (int L = P; L > 1; L >>= 1)
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
    const uint4* p = (const uint4*)((const uint8_t*)t.data + row * 64 + 32 * g);
    uint4 c0 = p[0], c1 = p[1];
    uint32_t sc = *(const uint32_t*)((const uint8_t*)t.scale + row * 8 + 4 * g);
    uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
    for (int s = 0; s < 8; ++s) out[s] = fp4x8_to_bf16x8(cw[s], (int)((sc >> (8 * (s >> 1))) & 255u) - 127);
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
      const int e = (int)((const uint8_t*)a.q.scale)[(qrow0 + h) * 8 + (c8 >> 1)] - 127;
      const uint4 w = fp4x8_to_bf16x8(codes, e);
      v[it] = u32x4_t{w.x, w.y, w.z, w.w};
    }
  }
}

// Score of key l % 32 from the 32x32 results of the two head tiles (every lane of the key returns it).
__device__ __forceinline__ float head_tree32(const f32x16_t (&acc)[2], const float (&wv)[2][16]) {
  float a[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const float p0 = wv[0][k] * __int_as_float(max(__float_as_int(acc[0][k]), 0));
    const float p1 = wv[1][k] * __int_as_float(max(__float_as_int(acc[1][k]), 0));
    a[k] = p0 + p1;  // h+32
  }
  float c[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) c[r] = (a[r] + a[r + 8]) + (a[r + 4] + a[r + 12]);  // h+16, then h+8
  // h+4 across the lane halves, scattered: the low half keeps head classes 0 and 1, the high half 2 and 3
  const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(c[0]), __float_as_uint(c[2]), false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(c[1]), __float_as_uint(c[3]), false, false);
  const float d02 = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
  const float d13 = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
  return xor32_sum(d02) + xor32_sum(d13);  // h+2 across the halves, then h+1
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
  const int nvis_last = nvis_of(a.q_start + r_end - 1, a.m, a.N);
  if (blockIdx.x * kMfmaEntriesPerBlock >= nvis_last) return;  // whole block invisible to every query

  // keys of this wave: two 32-entry column tiles, B operand for 8 K-steps each
  bf16x8_t kb[2][8];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = e0 + 32 * u + col;
    uint4 raw[8];
    if (e < nvis_last) {
      load_row64<FMT>(a.k, (long long)b * a.k.cap + e, g, raw);
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
    const int nvis = nvis_of(a.q_start + r, a.m, a.N);
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
      // epilogue: head h = 32T + 8(x/4) + 4g + (x%4) for register x; fixed halving tree over h
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
// l % 16.  The fixed halving tree over the 64 heads is then: h+32 (T, T+2) and h+16 (T, T+1) in-lane, h+8 (lanes
// l, l ^ 32) and h+4 (l, l ^ 16) across lanes, h+2 and h+1 in-lane.
//
// With a row histogram to fill (decode select), each workgroup counts its keys' bits [31:21] in LDS and adds the
// counts into the row's histogram, zeroed before the launch.  The select that follows reads it instead of making
// its own first pass over the keys.

// In-lane part of the tree for one 16-key group: v[r] = ((w relu)(T=0) + (T=2)) + ((T=1) + (T=3)) for the lane's
// heads 4 (l / 16) + r (+ 16 T).  ReLU is one integer max of the bit pattern with 0: non-negative floats order like
// their bit patterns and every negative one (-0 included) has the sign bit set, so the result equals max(x, 0)
// without the float max's NaN canonicalization.
__device__ __forceinline__ void head_partial(const f32x4_t (&acc)[4], const float (&wv)[4][4], float (&v)[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float p[4];
#pragma unroll
    for (int T = 0; T < 4; ++T) p[T] = wv[T][r] * __int_as_float(max(__float_as_int(acc[T][r]), 0));
    v[r] = (p[0] + p[2]) + (p[1] + p[3]);
  }
}

// Cross-lane part for four groups at once, as a reduce-scatter: h+8 pairs lane rows g and g + 2 (lanes l, l ^ 32),
// h+4 pairs rows g and g + 1 (l, l ^ 16), then h+2 and h+1 in-lane.  permlane32_swap(A, B) returns (A.lo, B.lo) and
// (A.hi, B.hi), so one swap and one add leave group 0 (2)'s pair sums in the low (high) half; permlane16_swap does
// the same for rows 0/1 and 2/3.  Row g of the wave ends with group g's four partial sums, and the lane returns the
// score of group g, key l % 16.  The pairs are those of the fixed halving tree (fp32 addition is commutative).
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

__device__ __forceinline__ void bf_load_stage(BfStage& S, const uint8_t* kb, int kbase, int klast, int lane) {
  const int g = lane >> 4, col = lane & 15;
#pragma unroll
  for (int j = 0; j < kBfGroups; ++j) {
    const int e = min(kbase + 16 * j + col, klast);
#pragma unroll
    for (int s = 0; s < 4; ++s) S.c[j][s] = *(const uint4*)(kb + (long long)e * 256 + 16 * g + 64 * s);
  }
}

template <int NST>
__global__ __launch_bounds__(256, 2) void idx_score_decode_bf16(IdxArgs a) {
#pragma clang fp contract(off)
  __shared__ int hist_s[kSelBins];
  constexpr int KPW = 16 * kBfGroups;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int g = lane >> 4, col = lane & 15;
  const int qrow = blockIdx.y, b = qrow / a.Sq;  // query row b * Sq + r
  const int nvis = nvis_of(a.q_start + (qrow - b * a.Sq), a.m, a.N);
  const int k0 = blockIdx.x * (NST * 4 * KPW);
  const int k1 = min(k0 + NST * 4 * KPW, nvis);
  if (k0 >= k1) return;
  const bool hist = a.sel_state != nullptr;
  if (hist)
    for (int i = threadIdx.x; i < kSelBins; i += blockDim.x) hist_s[i] = 0;
  const uint8_t* kb = (const uint8_t*)a.k.data + (long long)b * a.k.cap * 256;

  BfStage S[2];
  bf_load_stage(S[0], kb, k0 + wave * KPW, k1 - 1, lane);
  bf16x8_t qa[4][4];
  float wv[4][4];
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    const uint8_t* qp = (const uint8_t*)a.q.data + ((long long)qrow * 64 + 16 * T + col) * 256;
#pragma unroll
    for (int s = 0; s < 4; ++s) qa[T][s] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(qp + 16 * g + 64 * s));
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[T][r] = a.w[(long long)qrow * 64 + 16 * T + 4 * g + r];
  }
  if (hist) __syncthreads();  // histogram zeroed before any update

  // straight-line stages (fully unrolled): the next stage's loads are in flight while this one is scored, and each
  // stage's keys are stored after the following stage's loads are issued
  KeyOut pend{0u, k1};
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    const int kbase = k0 + st * 4 * KPW + wave * KPW;
    if (st + 1 < NST) {
      bf_load_stage(S[(st + 1) & 1], kb, kbase + 4 * KPW, k1 - 1, lane);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the scoring
    }
    if (st > 0) store_key(a, qrow, k1, pend, hist_s, hist);
    const BfStage& C = S[st & 1];
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
        for (int T = 0; T < 4; ++T) acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[T][s], kv, acc[T], 0, 0, 0);
      }
      head_partial(acc, wv, v[j]);
    }
    pend = lane_key(kbase, g, head_cross4(v));
  }
  store_key(a, qrow, k1, pend, hist_s, hist);
  if (hist) flush_hist(hist_s, a.sel_state + (long long)qrow * kSelStateInts);
}

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;

// ---- fp4 decode scoring with the keys streamed into an LDS ring: one workgroup of eight waves per CU takes NST
// stages of 512 keys.  A stage's codes (32 KB) and scales (4 KB) travel from memory straight into a ring slot with
// buffer loads into LDS (no registers hold data in flight), three stages in flight while one is scored; each slot is
// its own pair of LDS variables and the stage loop is fully unrolled, so every wait is a count fixed at compile
// time.  Each wave moves and scores its own 64 keys of a stage, so waves never wait for each other.  Code rows are
// stored with their four 16-byte chunks XOR-swizzled by bits 2..3 of the key's position in its 16-key group, which
// makes the operand reads bank-conflict free.
//
// Scoring runs on v_mfma_scale_f32_32x32x64_f8f6f4, which takes fp4 operands at twice the rate of the 16x16x128
// form: A = 32 heads (lane l: head l % 32, contraction slots 32 (l / 32) .. + 31), B = 32 keys (lane l: key l % 32,
// the same slots), one E8M0 scale per lane applied to the lane's 32 slots.  The cache scales each 16 elements, so
// lane half hh = l / 32 takes code chunk c = 2 i + hh (groups 2c, 2c + 1) in instruction pair i; the key operand is
// the chunk as loaded and the query operand keeps one of its two groups (h = 0, 1) with that group's scales and
// zeros the other 16 slots, whose products are exact zeros (e2m1 has no infinities or NaNs).  Eight instructions
// (2 head tiles x 2 chunk pairs x 2 groups) give the 64 x 32 dots.  Products of fp4 values and their block sums are
// exact, scaled by powers of two, so the per-head dots equal the exact ones whenever they fit fp32 -- the fixed
// head-reduction order then makes the scores bit-reproducible.  Lane l, register k of the 32x32 result holds head
// 32 T + 8 (k / 4) + 4 hh + k % 4 for key l % 32: the tree's h+32, h+16, h+8 steps run in lane, h+4 and h+2 across
// the lane halves, h+1 in lane -- the same pairs as the 16x16 kernels.
constexpr int kF4rWaves = 8;
constexpr int kF4rStage = 64 * kF4rWaves;  // keys per stage
constexpr int kF4rCodeB = kF4rStage * 64;  // 32 KB
constexpr int kF4rScaleB = kF4rStage * 8;  // 4 KB
__shared__ __attribute__((aligned(16))) uint8_t f4r_c0[kF4rCodeB];
__shared__ __attribute__((aligned(16))) uint8_t f4r_c1[kF4rCodeB];
__shared__ __attribute__((aligned(16))) uint8_t f4r_c2[kF4rCodeB];
__shared__ __attribute__((aligned(16))) uint8_t f4r_c3[kF4rCodeB];
__shared__ __attribute__((aligned(16))) uint8_t f4r_s0[kF4rScaleB];
__shared__ __attribute__((aligned(16))) uint8_t f4r_s1[kF4rScaleB];
__shared__ __attribute__((aligned(16))) uint8_t f4r_s2[kF4rScaleB];
__shared__ __attribute__((aligned(16))) uint8_t f4r_s3[kF4rScaleB];
__shared__ int f4r_hist[kSelBins];

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
constexpr int kIdxBufWord3 = 0x00020000;  // buffer descriptor word 3: raw untyped loads

// s_waitcnt immediate for vmcnt(n) with the other counters untouched
__host__ __device__ constexpr int vm_wait_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (0xF << 8) | (7 << 4); }

// Memory operations a wave has issued after the loads of stage st when step st waits for them: the loads of the
// (at most two) stages after it and the key stores of the steps since they were issued (6 loads per stage: 4 code
// rows of 1 KB and 2 scale rows of 256 bytes; 1 store per step).
__host__ __device__ constexpr int f4r_wait_count(int st, int nst) {
  const int later = (st + 2 < nst - 1 ? st + 2 : nst - 1) - st;
  const int stores = st - (st - 3 > 0 ? st - 3 : 0);
  return 6 * later + stores;
}

// Calls f(integral_constant<int, ST>) for ST = ST0 .. NST - 1 in order (a loop whose index is a constant).
template <int ST, int NST, class F>
__device__ __forceinline__ void unroll_steps(F& f) {
  if constexpr (ST < NST) {
    f(std::integral_constant<int, ST>{});
    unroll_steps<ST + 1, NST>(f);
  }
}


template <int NST>
__global__ __launch_bounds__(kF4rWaves * 64) void idx_score_decode_fp4_ring(IdxArgs a) {
#pragma clang fp contract(off)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int col = lane & 31, hh = lane >> 5;
  const int qrow = blockIdx.y, b = qrow / a.Sq;  // query row b * Sq + r
  const int nvis = nvis_of(a.q_start + (qrow - b * a.Sq), a.m, a.N);
  const int k0 = blockIdx.x * (NST * kF4rStage);
  const int k1 = min(k0 + NST * kF4rStage, nvis);
  if (k0 >= k1) return;  // block-uniform
  const bool hist = a.sel_state != nullptr;
  for (int i = threadIdx.x; i < kSelBins; i += blockDim.x) f4r_hist[i] = 0;

  // query: head tile T = heads 32 T .. 32 T + 31, lane head 32 T + col; chunks hh and 2 + hh of its code row and the
  // matching scale bytes 2 hh, 2 hh + 1, 4 + 2 hh, 5 + 2 hh.  The raw loads go first and the operands are built after
  // the ring's first loads are issued, so that nothing waits for the queries before the ring starts.
  uint4 qraw[2][2];
  uint2 sraw[2];
  float wv[2][16];
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    const long long row = (long long)qrow * 64 + 32 * T + col;
#pragma unroll
    for (int i = 0; i < 2; ++i) qraw[T][i] = *(const uint4*)((const uint8_t*)a.q.data + row * 64 + 16 * (2 * i + hh));
    sraw[T] = *(const uint2*)((const uint8_t*)a.q.scale + row * 8);
#pragma unroll
    for (int k = 0; k < 16; ++k) wv[T][k] = a.w[(long long)qrow * 64 + 32 * T + 8 * (k >> 2) + 4 * hh + (k & 3)];
  }
  __builtin_amdgcn_sched_barrier(0);
  i32x8_t qop[2][2][2];
  int qs[2][2][2];

  // buffer descriptors over the workgroup's own keys [k0, k1): offsets stay small whatever the cache size, and the
  // range check covers exactly the keys the workgroup may read
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)a.k.data + ((long long)b * a.k.cap + k0) * 64), 0, (k1 - k0) * 64, kIdxBufWord3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)a.k.scale + ((long long)b * a.k.cap + k0) * 8), 0, (k1 - k0) * 8, kIdxBufWord3);
  // stage st into slot S: code instruction i of wave w moves keys 64 w + 16 i .. + 15 (lane l: key + l / 4, chunk
  // position l % 4 holding code chunk (l % 4) ^ (l / 16)); scale instruction i moves 32 keys' scale rows.  Keys past
  // k1 repeat key k1 - 1.
  auto issue = [&](auto SC, int st) {
    constexpr int S = decltype(SC)::value;
    const int kst = st * kF4rStage;  // relative to k0
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = min(kst + 64 * wave + 16 * i + (lane >> 2), k1 - k0 - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, (idx_lds_void_t*)(f4r_codes<S>() + (64 * wave + 16 * i) * 64), 16,
                                               key * 64 + 16 * ((lane & 3) ^ (lane >> 4)), 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key = min(kst + 64 * wave + 32 * i + (lane >> 1), k1 - k0 - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (idx_lds_void_t*)(f4r_scales<S>() + (64 * wave + 32 * i) * 8), 4,
                                               key * 8 + 4 * (lane & 1), 0, 0, 0);
    }
  };
  // 64 x 32 dots of the wave's key tile u (keys 64 w + 32 u + col of stage slot S)
  auto dots = [&](auto SC, int u, f32x16_t (&acc)[2]) {
    constexpr int S = decltype(SC)::value;
    const int kl = 64 * wave + 32 * u + col;
    const uint8_t* cb = f4r_codes<S>() + kl * 64;
    const int sw = (kl >> 2) & 3;
    const uint2 s8 = *(const uint2*)(f4r_scales<S>() + kl * 8);
    i32x8_t kop[2];
    int ks[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const u32x4_t kc = *(const u32x4_t*)(cb + 16 * ((2 * i + hh) ^ sw));
      kop[i] = i32x8_t{(int)kc[0], (int)kc[1], (int)kc[2], (int)kc[3], 0, 0, 0, 0};
      const uint32_t sword = i == 0 ? s8.x : s8.y;  // bytes 4i .. 4i + 3
      ks[i][0] = (int)((sword >> (16 * hh)) & 255u);
      ks[i][1] = (int)((sword >> (16 * hh + 8)) & 255u);
    }
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      acc[T] = f32x16_t{};
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          acc[T] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qop[T][i][h], kop[i], acc[T], 4, 4, 0,
                                                                   qs[T][i][h], 0, ks[i][h]);
    }
  };
  // lane (col, hh) returns the key of tile u's key col (both halves hold it)
  auto score = [&](auto SC, int st) -> uint2 {
    f32x16_t acc0[2], acc1[2];
    dots(SC, 0, acc0);
    __builtin_amdgcn_sched_barrier(0);
    dots(SC, 1, acc1);
    const float s0 = head_tree32(acc0, wv);
    // the second tile's MFMAs run while the first tile's tree issues between them
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    const float s1 = head_tree32(acc1, wv);
    (void)st;
    return uint2{score_key(s0), score_key(s1)};
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
  for (int T = 0; T < 2; ++T)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 c = qraw[T][i];
      qop[T][i][0] = i32x8_t{(int)c.x, (int)c.y, 0, 0, 0, 0, 0, 0};
      qop[T][i][1] = i32x8_t{0, 0, (int)c.z, (int)c.w, 0, 0, 0, 0};
      const uint32_t sword = i == 0 ? sraw[T].x : sraw[T].y;
      qs[T][i][0] = (int)((sword >> (16 * hh)) & 255u);
      qs[T][i][1] = (int)((sword >> (16 * hh + 8)) & 255u);
    }

  // Stage st sits in slot st % 4.  A wave loads exactly the keys it scores, so the ring needs no barrier: step st
  // waits for this wave's own loads of stage st, starts stage st + 3 in the slot this wave finished with in step
  // st - 1, scores and stores.  The histogram counts wait until the ring is drained: an LDS atomic while ring loads
  // are in flight would make the compiler wait for all of them.
  uint2 kept[NST];
  auto step = [&](auto STC) {
    constexpr int st = decltype(STC)::value;
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(f4r_wait_count(st, NST)));
    asm volatile("" ::: "memory");
    if constexpr (st + 3 < NST) issue(std::integral_constant<int, (st + 3) % 4>{}, st + 3);
    kept[st] = score(std::integral_constant<int, st % 4>{}, st);
    // lane (col, hh) stores tile hh's key col: 64 keys per store
    const int e = k0 + st * kF4rStage + 64 * wave + 32 * hh + col;
    a.keys[(long long)qrow * a.N + min(e, k1 - 1)] = hh ? kept[st].y : kept[st].x;
  };
  unroll_steps<0, NST>(step);
  if (hist) {
    __syncthreads();  // every wave has zeroed its part of the histogram
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int e = k0 + st * kF4rStage + 64 * wave + 32 * hh + col;
      if (e < k1) atomicAdd(&f4r_hist[(hh ? kept[st].y : kept[st].x) >> 21], 1);
    }
  }
  if (hist) flush_hist(f4r_hist, a.sel_state + (long long)qrow * kSelStateInts);
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

hipError_t launch_indexer_scores(const IdxArgs& a, hipStream_t st) {
  const int nvis_max = nvis_of(a.q_start + a.Sq - 1, a.m, a.N);
  if (nvis_max <= 0) return hipSuccess;
  clear_stale_error();
  const bool mfma = a.HI == 64 && a.DI == 128 && a.q.format == a.k.format &&
                    (a.q.format == LCA_BF16 || a.q.format == LCA_FP4);
  if (indexer_uses_decode_kernel(a.B, a.Sq, a.HI, a.DI, a.N, a.q.format, a.k.format)) {
    const bool fp4 = a.q.format == LCA_FP4;
    if (fp4) {
      // one workgroup per CU where the context allows: the most stages per workgroup that still leave 256
      const long long rows = (long long)a.B * a.Sq;
      int nst = 8;
      while (nst > 1 && rows * ((nvis_max + nst * kF4rStage - 1) / (nst * kF4rStage)) < 256) nst >>= 1;
      const dim3 grid((unsigned)decode_grid_x((nvis_max + nst * kF4rStage - 1) / (nst * kF4rStage), a.Sq),
                      (unsigned)rows);
      const dim3 block(kF4rWaves * 64);
      if (nst == 8) hipLaunchKernelGGL(idx_score_decode_fp4_ring<8>, grid, block, 0, st, a);
      else if (nst == 4) hipLaunchKernelGGL(idx_score_decode_fp4_ring<4>, grid, block, 0, st, a);
      else if (nst == 2) hipLaunchKernelGGL(idx_score_decode_fp4_ring<2>, grid, block, 0, st, a);
      else hipLaunchKernelGGL(idx_score_decode_fp4_ring<1>, grid, block, 0, st, a);
      return hipGetLastError();
    }
    // a fixed key range per workgroup (NST stages of 4 waves x KPW keys), the grid grows with the context; fewer
    // stages when that leaves fewer than about two workgroups per CU
    const int kpw = 16 * kBfGroups;
    const long long rows = (long long)a.B * a.Sq;
    int nst = 4;
    while (nst > 1 && rows * ((nvis_max + nst * 4 * kpw - 1) / (nst * 4 * kpw)) < 512) nst >>= 1;
    const dim3 grid((unsigned)decode_grid_x((nvis_max + nst * 4 * kpw - 1) / (nst * 4 * kpw), a.Sq), (unsigned)rows);
    if (nst == 4) hipLaunchKernelGGL(idx_score_decode_bf16<4>, grid, dim3(256), 0, st, a);
    else if (nst == 2) hipLaunchKernelGGL(idx_score_decode_bf16<2>, grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(idx_score_decode_bf16<1>, grid, dim3(256), 0, st, a);
  } else if (mfma) {
    const int qpb = a.Sq >= 16 ? 16 : a.Sq;
    dim3 grid((unsigned)((nvis_max + kMfmaEntriesPerBlock - 1) / kMfmaEntriesPerBlock),
              (unsigned)((a.Sq + qpb - 1) / qpb), (unsigned)a.B);
    if (a.q.format == LCA_BF16)
      hipLaunchKernelGGL(idx_score_mfma<LCA_BF16>, grid, dim3(256), 0, st, a, qpb);
    else
      hipLaunchKernelGGL(idx_score_mfma<LCA_FP4>, grid, dim3(256), 0, st, a, qpb);
  } else {
    dim3 grid((unsigned)((nvis_max + kSimtTile - 1) / kSimtTile), (unsigned)a.Sq, (unsigned)a.B);
    hipLaunchKernelGGL(idx_score_simt, grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace lca
