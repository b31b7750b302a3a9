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
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float l1[16];
#pragma unroll
        for (int x = 0; x < 16; ++x) {  // level 1: h + 32
          const int h = 8 * (x >> 2) + 4 * g + (x & 3);
          const float p0 = w_s[cur][h] * fmaxf(acc[0][u][x], 0.0f);
          const float p1 = w_s[cur][32 + h] * fmaxf(acc[1][u][x], 0.0f);
          l1[x] = p0 + p1;
        }
        float l2[8], l3[4], l4[4];
#pragma unroll
        for (int x = 0; x < 8; ++x) l2[x] = l1[x] + l1[x + 8];  // h + 16
#pragma unroll
        for (int x = 0; x < 4; ++x) l3[x] = l2[x] + l2[x + 4];  // h + 8
#pragma unroll
        for (int x = 0; x < 4; ++x) l4[x] = xor32_sum(l3[x]);  // h + 4: the partner lane holds the other 4g half
        const float l5_0 = l4[0] + l4[2], l5_1 = l4[1] + l4[3];  // h + 2
        const float sc = l5_0 + l5_1;                            // h + 1
        const int e = e0 + 32 * u + col;
        if (g == 0 && e < nvis) a.keys[((long long)b * a.Sq + r) * a.N + e] = score_key(sc);
      }
    }
    stage(cur ^ 1);
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------------
// decode kernels (one query row per sequence): the key stream is the whole cost
// ------------------------------------------------------------------------------------------------
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

__device__ __forceinline__ float head_tree(const f32x4_t (&acc)[4], const float (&wv)[4][4]) {
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
  for (int r = 0; r < 4; ++r) l3[r] = xor32_sum(l2[r]);
#pragma unroll
  for (int r = 0; r < 4; ++r) l4[r] = xor16_sum(l3[r]);
  return (l4[0] + l4[2]) + (l4[1] + l4[3]);
}

__device__ __forceinline__ void flush_hist(const int* hist_s, int* gh) {
  __syncthreads();
  for (int i = threadIdx.x; i < kSelBins; i += blockDim.x) {
    const int c = hist_s[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

// Scores of four 16-key groups (every lane of a key holds its score after the head tree): lane (g, col) takes
// group q0 + g, so that one store writes 64 keys.  The store is unconditional -- a lane past the range holds the
// score of the clamped key k1 - 1 and writes that same value there -- and is issued after the next stage's loads,
// so no branch or register reuse separates the loads in flight from their waits.
struct KeyOut {
  uint32_t key;
  int e;
};

__device__ __forceinline__ KeyOut pick_key4(int gbase, int g, const float (&sc)[4]) {
  const float s = g == 0 ? sc[0] : g == 1 ? sc[1] : g == 2 ? sc[2] : sc[3];
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
constexpr int kBfGroups = 4;  // 16-key groups per wave per stage (16 KB per wave in flight)

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
  const int b = blockIdx.y;
  const int nvis = nvis_of(a.q_start, a.m, a.N);
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
    const uint8_t* qrow = (const uint8_t*)a.q.data + ((long long)b * 64 + 16 * T + col) * 256;
#pragma unroll
    for (int s = 0; s < 4; ++s) qa[T][s] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(qrow + 16 * g + 64 * s));
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[T][r] = a.w[(long long)b * 64 + 16 * T + 4 * g + r];
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
    if (st > 0) store_key(a, b, k1, pend, hist_s, hist);
    const BfStage& C = S[st & 1];
    float sc[kBfGroups];
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
      sc[j] = head_tree(acc, wv);
    }
    pend = pick_key4(kbase, g, sc);
  }
  store_key(a, b, k1, pend, hist_s, hist);
  if (hist) flush_hist(hist_s, a.sel_state + (long long)b * kSelStateInts);
}

// ---- fp4: v_mfma_scale_f32_16x16x128_f8f6f4 with both operands in fp4 e2m1 applies one E8M0 scale per lane to
// the lane's 32 contraction slots (A: lane l holds row l % 16, slots 32 (l / 16) .. + 31; B: column l % 16, same
// slots).  The cache scales each 16 elements, so each lane fills the first 16 slots of its block with one
// 16-element group and the other 16 with zeros; two instructions (h = 0, 1) cover the 8 groups of a 128-dim row:
// block b of instruction h holds group 2b + h.  A lane's operand bytes are 16 bytes at 16 (l / 16) of the key's
// 64-byte code row (groups 2g, 2g + 1) and the two scale bytes at 2 (l / 16) of its 8-byte scale row.  Products of
// fp4 values and their block sums are exact, scaled by powers of two, so the per-head dots equal the exact ones
// whenever they fit fp32 -- the fixed head-reduction order then makes the scores bit-reproducible.
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;

__device__ __forceinline__ i32x8_t fp4_operand(uint32_t lo, uint32_t hi) {
  i32x8_t v = {(int)lo, (int)hi, 0, 0, 0, 0, 0, 0};
  return v;
}

constexpr int kF4Groups = 8;  // 16-key groups per wave per stage (9 KB per wave in flight)

struct F4Stage {
  uint4 c[kF4Groups];
  uint32_t s[kF4Groups];
};

__device__ __forceinline__ void f4_load_stage(F4Stage& S, const uint8_t* codes, const uint8_t* scales, int kbase,
                                              int klast, int lane) {
  const int g = lane >> 4, col = lane & 15;
#pragma unroll
  for (int j = 0; j < kF4Groups; ++j) {
    const int e = min(kbase + 16 * j + col, klast);
    S.c[j] = *(const uint4*)(codes + (long long)e * 64 + 16 * g);
    S.s[j] = *(const uint16_t*)(scales + (long long)e * 8 + 2 * g);
  }
}

template <int NST>
__global__ __launch_bounds__(256, 2) void idx_score_decode_fp4(IdxArgs a) {
#pragma clang fp contract(off)
  __shared__ int hist_s[kSelBins];
  constexpr int KPW = 16 * kF4Groups;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int g = lane >> 4, col = lane & 15;
  const int b = blockIdx.y;
  const int nvis = nvis_of(a.q_start, a.m, a.N);
  const int k0 = blockIdx.x * (NST * 4 * KPW);
  const int k1 = min(k0 + NST * 4 * KPW, nvis);
  if (k0 >= k1) return;
  const bool hist = a.sel_state != nullptr;
  if (hist)
    for (int i = threadIdx.x; i < kSelBins; i += blockDim.x) hist_s[i] = 0;
  const uint8_t* codes = (const uint8_t*)a.k.data + (long long)b * a.k.cap * 64;
  const uint8_t* scales = (const uint8_t*)a.k.scale + (long long)b * a.k.cap * 8;

  F4Stage S[2];
  f4_load_stage(S[0], codes, scales, k0 + wave * KPW, k1 - 1, lane);
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
  if (hist) __syncthreads();  // histogram zeroed before any update

  // straight-line stages as in the bf16 kernel; a stage is two batches of four groups, and each batch's keys are
  // stored once the next batch (or the next stage's loads) is under way
  KeyOut pend{0u, k1};
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    const int kbase = k0 + st * 4 * KPW + wave * KPW;
    if (st + 1 < NST) {
      f4_load_stage(S[(st + 1) & 1], codes, scales, kbase + 4 * KPW, k1 - 1, lane);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the scoring
    }
    const F4Stage& C = S[st & 1];
#pragma unroll
    for (int q = 0; q < kF4Groups / 4; ++q) {
      if (st > 0 || q > 0) store_key(a, b, k1, pend, hist_s, hist);
      float sc[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = 4 * q + jj;
        const uint4 kc = C.c[j];
        const i32x8_t kop0 = fp4_operand(kc.x, kc.y), kop1 = fp4_operand(kc.z, kc.w);
        const int ks0 = (int)(C.s[j] & 255u), ks1 = (int)(C.s[j] >> 8);
        f32x4_t acc[4];
#pragma unroll
        for (int T = 0; T < 4; ++T) {
          acc[T] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
          acc[T] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fp4_operand(qc[T][0], qc[T][1]), kop0, acc[T], 4,
                                                                    4, 0, qs[T][0], 0, ks0);
          acc[T] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fp4_operand(qc[T][2], qc[T][3]), kop1, acc[T], 4,
                                                                    4, 0, qs[T][1], 0, ks1);
        }
        sc[jj] = head_tree(acc, wv);
      }
      pend = pick_key4(kbase + 64 * q, g, sc);
    }
  }
  store_key(a, b, k1, pend, hist_s, hist);
  if (hist) flush_hist(hist_s, a.sel_state + (long long)b * kSelStateInts);
}

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
    // a fixed key range per workgroup (NST stages of 4 waves x KPW keys), the grid grows with the context; fewer
    // stages when that leaves fewer than about two workgroups per CU
    const bool fp4 = a.q.format == LCA_FP4;
    const int kpw = fp4 ? 16 * kF4Groups : 16 * kBfGroups;
    int nst = 4;
    while (nst > 1 && (long long)a.B * ((nvis_max + nst * 4 * kpw - 1) / (nst * 4 * kpw)) < 512) nst >>= 1;
    const dim3 grid((unsigned)((nvis_max + nst * 4 * kpw - 1) / (nst * 4 * kpw)), (unsigned)a.B);
    if (fp4) {
      if (nst == 4) hipLaunchKernelGGL(idx_score_decode_fp4<4>, grid, dim3(256), 0, st, a);
      else if (nst == 2) hipLaunchKernelGGL(idx_score_decode_fp4<2>, grid, dim3(256), 0, st, a);
      else hipLaunchKernelGGL(idx_score_decode_fp4<1>, grid, dim3(256), 0, st, a);
    } else {
      if (nst == 4) hipLaunchKernelGGL(idx_score_decode_bf16<4>, grid, dim3(256), 0, st, a);
      else if (nst == 2) hipLaunchKernelGGL(idx_score_decode_bf16<2>, grid, dim3(256), 0, st, a);
      else hipLaunchKernelGGL(idx_score_decode_bf16<1>, grid, dim3(256), 0, st, a);
    }
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
