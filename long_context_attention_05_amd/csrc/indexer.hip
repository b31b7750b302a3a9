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

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

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

template <int FMT>
__global__ __launch_bounds__(256) void idx_score_mfma(IdxArgs a, int qpb) {
#pragma clang fp contract(off)
  __shared__ uint16_t q_s[64 * kQStride];
  __shared__ float w_s[64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
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

  for (int r = r_begin; r < r_end; ++r) {
    const long long t = a.q_start + r;
    const int nvis = nvis_of(t, a.m, a.N);
    if (blockIdx.x * kMfmaEntriesPerBlock >= nvis) continue;  // block-uniform
    __syncthreads();
    {  // stage the 64 x 128 query block (bf16) in LDS: 256 threads x 4 chunks of 8 channels
      const long long qrow0 = ((long long)b * a.Sq + r) * 64;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int chunk = threadIdx.x + 256 * it;  // 1024 chunks of 8 channels
        const int h = chunk >> 4, c8 = chunk & 15;
        uint4 v;
        if (FMT == LCA_BF16) {
          v = *(const uint4*)((const uint16_t*)a.q.data + (qrow0 + h) * 128 + 8 * c8);
        } else {
          uint32_t codes = *(const uint32_t*)((const uint8_t*)a.q.data + (qrow0 + h) * 64 + 4 * c8);
          int e = (int)((const uint8_t*)a.q.scale)[(qrow0 + h) * 8 + (c8 >> 1)] - 127;
          v = fp4x8_to_bf16x8(codes, e);
        }
        *(uint4*)&q_s[h * kQStride + 8 * c8] = v;
      }
      if (threadIdx.x < 64) w_s[threadIdx.x] = a.w[((long long)b * a.Sq + r) * 64 + threadIdx.x];
    }
    __syncthreads();
    if (e0 >= nvis) continue;  // wave-uniform

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
        const uint4 qv = *(const uint4*)&q_s[(32 * T + col) * kQStride + 64 * g + 8 * s];
        const bf16x8_t qa = __builtin_bit_cast(bf16x8_t, qv);
#pragma unroll
        for (int u = 0; u < 2; ++u) acc[T][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kb[u][s], acc[T][u], 0, 0, 0);
      }
    }
    // epilogue: head h = 32T + 8(x/4) + 4g + (x%4) for register x; fixed halving tree over h
    float wv[2][16];
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int x = 0; x < 16; ++x) wv[T][x] = w_s[32 * T + 8 * (x >> 2) + 4 * g + (x & 3)];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float l1[16];
#pragma unroll
      for (int x = 0; x < 16; ++x) {  // level 1: h + 32
        float p0 = wv[0][x] * fmaxf(acc[0][u][x], 0.0f);
        float p1 = wv[1][x] * fmaxf(acc[1][u][x], 0.0f);
        l1[x] = p0 + p1;
      }
      float l2[8], l3[4], l4[4];
#pragma unroll
      for (int x = 0; x < 8; ++x) l2[x] = l1[x] + l1[x + 8];  // h + 16
#pragma unroll
      for (int x = 0; x < 4; ++x) l3[x] = l2[x] + l2[x + 4];  // h + 8
#pragma unroll
      for (int x = 0; x < 4; ++x) {  // h + 4: the partner lane holds the other 4g half
        float o = __shfl_xor(l3[x], 32, 64);
        l4[x] = (g == 0) ? (l3[x] + o) : (o + l3[x]);
      }
      float l5_0 = l4[0] + l4[2], l5_1 = l4[1] + l4[3];  // h + 2
      float s = l5_0 + l5_1;                             // h + 1
      const int e = e0 + 32 * u + col;
      if (g == 0 && e < nvis) a.keys[((long long)b * a.Sq + r) * a.N + e] = score_key(s);
    }
  }
}

// ------------------------------------------------------------------------------------------------
// decode MFMA kernel (one query row per sequence): the key stream is the whole cost, so keys move in
// fully coalesced 16-byte loads (16 lanes per 256-byte key row) into a double-buffered LDS tile while the
// previous tile is scored; the query block stays in registers for the whole entry range of the workgroup.
// ------------------------------------------------------------------------------------------------
constexpr int kDecTile = 128;      // entries per tile, 32 per wave
constexpr int kKRowB = 272;        // LDS bytes per bf16 key row (256 + 16 padding)
constexpr int kKRowF4 = 80;        // LDS bytes per fp4 key row (64 codes + 8 scales + 8 padding)

template <int FMT>
constexpr int dec_row_bytes() { return FMT == LCA_BF16 ? kKRowB : kKRowF4; }

template <int FMT>
__device__ __forceinline__ void dec_load_tile(const IdxArgs& a, int b, int e0, int nvis, uint4 (&v)[8]) {
  const int tid = threadIdx.x;
  if (FMT == LCA_BF16) {
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int c = tid + 256 * x, e = c >> 4, piece = c & 15;
      v[x] = (e0 + e < nvis)
                 ? *(const uint4*)((const uint8_t*)a.k.data + ((long long)b * a.k.cap + e0 + e) * 256 + 16 * piece)
                 : make_uint4(0, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int c = tid + 256 * x, e = c >> 2, piece = c & 3;
      v[x] = (e0 + e < nvis)
                 ? *(const uint4*)((const uint8_t*)a.k.data + ((long long)b * a.k.cap + e0 + e) * 64 + 16 * piece)
                 : make_uint4(0, 0, 0, 0);
    }
    const int e = tid >> 1, half = tid & 1;
    v[2].x = (e0 + e < nvis) ? *(const uint32_t*)((const uint8_t*)a.k.scale + ((long long)b * a.k.cap + e0 + e) * 8 +
                                                  4 * half)
                             : 0u;
  }
}

template <int FMT>
__device__ __forceinline__ void dec_store_tile(uint8_t* buf, const uint4 (&v)[8]) {
  const int tid = threadIdx.x;
  if (FMT == LCA_BF16) {
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int c = tid + 256 * x, e = c >> 4, piece = c & 15;
      *(uint4*)(buf + e * kKRowB + 16 * piece) = v[x];
    }
  } else {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int c = tid + 256 * x, e = c >> 2, piece = c & 3;
      *(uint4*)(buf + e * kKRowF4 + 16 * piece) = v[x];
    }
    const int e = tid >> 1, half = tid & 1;
    *(uint32_t*)(buf + e * kKRowF4 + 64 + 4 * half) = v[2].x;
  }
}

template <int FMT>
__global__ __launch_bounds__(256, 2) void idx_score_decode(IdxArgs a, int tiles_per_block) {
#pragma clang fp contract(off)
  extern __shared__ __attribute__((aligned(16))) uint8_t dec_lds[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 5, col = lane & 31;
  const int b = blockIdx.y;
  if (a.sel_state && blockIdx.x == 0)  // the select that follows accumulates into this row's state
    for (int i = threadIdx.x; i < kSelStateInts; i += blockDim.x) a.sel_state[(long long)b * kSelStateInts + i] = 0;
  const int nvis = nvis_of(a.q_start, a.m, a.N);
  const int ntiles = (nvis + kDecTile - 1) / kDecTile;
  const int t_begin = blockIdx.x * tiles_per_block;
  const int t_end = min(t_begin + tiles_per_block, ntiles);
  if (t_begin >= t_end) return;
  constexpr int RB = dec_row_bytes<FMT>();

  uint4 pre[8];
  dec_load_tile<FMT>(a, b, t_begin * kDecTile, nvis, pre);

  // query block (64 heads x 128) as the A operand: lane holds head 32T + col, channels 64g + 8s .. + 7
  bf16x8_t qa[2][8];
  float wv[2][16];
  {
    const long long qrow0 = (long long)b * 64;
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      const long long row = qrow0 + 32 * T + col;
      uint4 raw[8];
      load_row64<FMT>(a.q, row, g, raw);
#pragma unroll
      for (int s = 0; s < 8; ++s) qa[T][s] = __builtin_bit_cast(bf16x8_t, raw[s]);
#pragma unroll
      for (int x = 0; x < 16; ++x) wv[T][x] = a.w[(long long)b * 64 + 32 * T + 8 * (x >> 2) + 4 * g + (x & 3)];
    }
  }
  dec_store_tile<FMT>(dec_lds, pre);
  __syncthreads();

  for (int tt = t_begin; tt < t_end; ++tt) {
    const int cur = (tt - t_begin) & 1;
    if (tt + 1 < t_end) dec_load_tile<FMT>(a, b, (tt + 1) * kDecTile, nvis, pre);

    // B operand: the wave's 32 keys, channels 64g + 8s .. + 7
    bf16x8_t kb[8];
    const uint8_t* rowp = dec_lds + cur * (kDecTile * RB) + (32 * wave + col) * RB;
    if (FMT == LCA_BF16) {
#pragma unroll
      for (int s = 0; s < 8; ++s) kb[s] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(rowp + 128 * g + 16 * s));
    } else {
      const uint4 c0 = *(const uint4*)(rowp + 32 * g), c1 = *(const uint4*)(rowp + 32 * g + 16);
      const uint32_t sc = *(const uint32_t*)(rowp + 64 + 4 * g);
      const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
      for (int s = 0; s < 8; ++s)
        kb[s] = __builtin_bit_cast(bf16x8_t, fp4x8_to_bf16x8(cw[s], (int)((sc >> (8 * (s >> 1))) & 255u) - 127));
    }
    f32x16_t acc[2];
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[T][x] = 0.0f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int T = 0; T < 2; ++T) acc[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[T][s], kb[s], acc[T], 0, 0, 0);

    // fixed halving tree over the 64 heads (see the header comment)
    float l1[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const float p0 = wv[0][x] * fmaxf(acc[0][x], 0.0f);
      const float p1 = wv[1][x] * fmaxf(acc[1][x], 0.0f);
      l1[x] = p0 + p1;
    }
    float l2[8], l3[4], l4[4];
#pragma unroll
    for (int x = 0; x < 8; ++x) l2[x] = l1[x] + l1[x + 8];
#pragma unroll
    for (int x = 0; x < 4; ++x) l3[x] = l2[x] + l2[x + 4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const float o = __shfl_xor(l3[x], 32, 64);
      l4[x] = (g == 0) ? (l3[x] + o) : (o + l3[x]);
    }
    const float s = (l4[0] + l4[2]) + (l4[1] + l4[3]);
    const int e = tt * kDecTile + 32 * wave + col;
    if (g == 0 && e < nvis) a.keys[(long long)b * a.N + e] = score_key(s);

    if (tt + 1 < t_end) dec_store_tile<FMT>(dec_lds + (cur ^ 1) * (kDecTile * RB), pre);
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------------
// decode kernel for fp4 keys and queries: block-scaled MFMA on the stored codes
// ------------------------------------------------------------------------------------------------
// v_mfma_scale_f32_16x16x128_f8f6f4 with both operands in fp4 e2m1 applies one E8M0 scale per lane to the lane's
// 32 contraction slots (A: lane l holds row l % 16, slots 32 (l / 16) .. + 31; B: column l % 16, same slots).  The
// cache scales each 16 elements, so each lane fills the first 16 slots of its block with one 16-element group and
// the other 16 with zeros; two instructions (h = 0, 1) cover the 8 groups of a 128-dim row: block b of
// instruction h holds group 2b + h.  Products of fp4 values and their block sums are exact, scaled by powers of
// two, so the per-head dots equal the exact ones whenever they fit fp32 -- the fixed head-reduction order then
// makes the scores bit-reproducible.  The 16x16 accumulator holds heads 16T + 4(l/16) + r for key l % 16.
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;

__device__ __forceinline__ i32x8_t fp4_operand(uint32_t lo, uint32_t hi) {
  i32x8_t v = {(int)lo, (int)hi, 0, 0, 0, 0, 0, 0};
  return v;
}

__global__ __launch_bounds__(256, 2) void idx_score_decode_fp4(IdxArgs a, int tiles_per_block) {
#pragma clang fp contract(off)
  extern __shared__ __attribute__((aligned(16))) uint8_t dec_lds[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, col = lane & 15;
  const int b = blockIdx.y;
  if (a.sel_state && blockIdx.x == 0)  // the select that follows accumulates into this row's state
    for (int i = threadIdx.x; i < kSelStateInts; i += blockDim.x) a.sel_state[(long long)b * kSelStateInts + i] = 0;
  const int nvis = nvis_of(a.q_start, a.m, a.N);
  const int ntiles = (nvis + kDecTile - 1) / kDecTile;
  const int t_begin = blockIdx.x * tiles_per_block;
  const int t_end = min(t_begin + tiles_per_block, ntiles);
  if (t_begin >= t_end) return;
  constexpr int RB = kKRowF4;

  uint4 pre[8];
  dec_load_tile<LCA_FP4>(a, b, t_begin * kDecTile, nvis, pre);

  // query operands: M-tile T = heads 16T .. 16T + 15; lane holds head 16T + col, groups 2g and 2g + 1
  uint32_t qc[4][4];  // [T][0..1] = group 2g codes, [2..3] = group 2g + 1 codes
  int qs[4][2];
  float wv[4][4];
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    const long long row = (long long)b * 64 + 16 * T + col;
    const uint4 c = *(const uint4*)((const uint8_t*)a.q.data + row * 64 + 16 * g);
    qc[T][0] = c.x;
    qc[T][1] = c.y;
    qc[T][2] = c.z;
    qc[T][3] = c.w;
    const uint32_t s2 = *(const uint16_t*)((const uint8_t*)a.q.scale + row * 8 + 2 * g);
    qs[T][0] = (int)(s2 & 255u);
    qs[T][1] = (int)(s2 >> 8);
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[T][r] = a.w[(long long)b * 64 + 16 * T + 4 * g + r];
  }
  dec_store_tile<LCA_FP4>(dec_lds, pre);
  __syncthreads();

  for (int tt = t_begin; tt < t_end; ++tt) {
    const int cur = (tt - t_begin) & 1;
    if (tt + 1 < t_end) dec_load_tile<LCA_FP4>(a, b, (tt + 1) * kDecTile, nvis, pre);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint8_t* rowp = dec_lds + cur * (kDecTile * RB) + (32 * wave + 16 * u + col) * RB;
      const uint4 kc = *(const uint4*)(rowp + 16 * g);
      const uint32_t ks2 = *(const uint16_t*)(rowp + 64 + 2 * g);
      const i32x8_t kop0 = fp4_operand(kc.x, kc.y), kop1 = fp4_operand(kc.z, kc.w);
      const int ks0 = (int)(ks2 & 255u), ks1 = (int)(ks2 >> 8);
      f32x4_t acc[4];
#pragma unroll
      for (int T = 0; T < 4; ++T) {
        acc[T] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        acc[T] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fp4_operand(qc[T][0], qc[T][1]), kop0, acc[T], 4, 4,
                                                                  0, qs[T][0], 0, ks0);
        acc[T] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fp4_operand(qc[T][2], qc[T][3]), kop1, acc[T], 4, 4,
                                                                  0, qs[T][1], 0, ks1);
      }
      // halving tree: h+32 (T, T+2), h+16 (T, T+1) in-lane; h+8 (g, g+2) and h+4 (g, g+1) across lanes;
      // h+2, h+1 in-lane
      float l1[2][4], l2[4], l3[4], l4[4];
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p0 = wv[T][r] * fmaxf(acc[T][r], 0.0f);
          const float p1 = wv[T + 2][r] * fmaxf(acc[T + 2][r], 0.0f);
          l1[T][r] = p0 + p1;
        }
#pragma unroll
      for (int r = 0; r < 4; ++r) l2[r] = l1[0][r] + l1[1][r];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float o = __shfl_xor(l2[r], 32, 64);
        l3[r] = (g < 2) ? (l2[r] + o) : (o + l2[r]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float o = __shfl_xor(l3[r], 16, 64);
        l4[r] = ((g & 1) == 0) ? (l3[r] + o) : (o + l3[r]);
      }
      const float s = (l4[0] + l4[2]) + (l4[1] + l4[3]);
      const int e = tt * kDecTile + 32 * wave + 16 * u + col;
      if (g == 0 && e < nvis) a.keys[(long long)b * a.N + e] = score_key(s);
    }
    if (tt + 1 < t_end) dec_store_tile<LCA_FP4>(dec_lds + (cur ^ 1) * (kDecTile * RB), pre);
    __syncthreads();
  }
}

static bool g_dec_attr[64];

bool indexer_uses_decode_kernel(int B, int Sq, int HI, int DI, int q_format, int k_format) {
  (void)B;
  return Sq == 1 && HI == 64 && DI == 128 && q_format == k_format && (q_format == LCA_BF16 || q_format == LCA_FP4);
}

hipError_t launch_indexer_scores(const IdxArgs& a, hipStream_t st) {
  const int nvis_max = nvis_of(a.q_start + a.Sq - 1, a.m, a.N);
  if (nvis_max <= 0) return hipSuccess;
  clear_stale_error();
  const bool mfma = a.HI == 64 && a.DI == 128 && a.q.format == a.k.format &&
                    (a.q.format == LCA_BF16 || a.q.format == LCA_FP4);
  if (indexer_uses_decode_kernel(a.B, a.Sq, a.HI, a.DI, a.q.format, a.k.format)) {
    const int ntiles = (nvis_max + kDecTile - 1) / kDecTile;
    int bps = (512 + a.B - 1) / a.B;  // about two workgroups per CU over the whole batch
    if (bps > ntiles) bps = ntiles;
    const int tpb = (ntiles + bps - 1) / bps;
    bps = (ntiles + tpb - 1) / tpb;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    if (dev >= 0 && dev < 64 && !g_dec_attr[dev]) {
      hipError_t e = hipFuncSetAttribute((const void*)idx_score_decode<LCA_BF16>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kDecTile * kKRowB);
      if (e != hipSuccess) return e;
      g_dec_attr[dev] = true;
    }
    if (a.q.format == LCA_BF16)
      hipLaunchKernelGGL(idx_score_decode<LCA_BF16>, dim3((unsigned)bps, (unsigned)a.B), dim3(256),
                         2 * kDecTile * kKRowB, st, a, tpb);
    else
      hipLaunchKernelGGL(idx_score_decode_fp4, dim3((unsigned)bps, (unsigned)a.B), dim3(256), 2 * kDecTile * kKRowF4,
                         st, a, tpb);
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
