// attn.hip -- stages 3 and 4: shared-KV multi-query attention over the sliding window, the compressed entries
// (selected by the indexer for CSA, all visible ones for HCA) and a per-head attention sink.
//
// Paper notes "DeepSeek-V4: Towards Highly Efficient Million-Token Context Intelligence", section 2.3 item 3
// (K and V are the same latent entry) and the Attention.forward excerpt (window indices and compressed indices go
// through one sparse attention kernel with the sink); itsolotime page mechanisms 1 (128-token window) and 3
// (learned per-head sink logit added to the softmax denominator); section 2.4 for the dense HCA variant.
//
//   l_j = scale * q_h . kv_j,   o_h = sum_j e^(l_j - M) kv_j / (e^(z_h - M) + sum_j e^(l_j - M))
//
// Each workgroup takes one query row and one contiguous slice ("split") of that row's entry list (window
// positions first, then compressed entries).  Entries are gathered 32 at a time into LDS; 64 heads share every
// entry, so the work is a dense contraction and runs on MFMA: S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (wave w
// owns heads 16w..16w+15), an online softmax per head, then O^T += V^T P^T with v_mfma_f32_16x16x16_bf16 whose B
// operand is exactly the S^T accumulator layout.  A second layout of the tile (channel-major, 4 entries per 8
// bytes) feeds the V^T operand.  fp8 entries are widened to bf16 exactly and their per-entry scale is applied to
// the logits and folded into P.  A split writes (max, sum, unnormalised o) and a merge kernel folds splits and the
// sink; a single split finishes in place.  Small or fp32 shapes use a vector-ALU kernel with the same contract.
#include "lca_device.h"
#include "lca_internal.h"

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;

namespace lca {


struct RowList {
  long long w0;  // first window position
  int nw;        // window entries
  int nc;        // compressed list length
};

__device__ __forceinline__ RowList row_list(const AttnArgs& a, long long t) {
  RowList L;
  long long w0 = t - a.window + 1;
  if (w0 < 0) w0 = 0;
  L.w0 = w0;
  L.nw = a.window > 0 ? (int)(t - w0 + 1) : 0;
  if (a.hca_m > 0) {
    long long v = t / a.hca_m;
    L.nc = (int)(v < a.N ? v : a.N);
  } else {
    L.nc = a.k;
  }
  return L;
}

// Row (within the tensor) of list position p, or -1 if the position is padding.
__device__ __forceinline__ long long list_row(const AttnArgs& a, const RowList& L, int b, int r, int p) {
  if (p < L.nw) return (long long)b * a.raw.cap + (L.w0 + p - a.raw_start);
  int j = p - L.nw;
  if (j >= L.nc) return -1;
  int e;
  if (a.hca_m > 0) {
    e = j;
  } else {
    e = a.idx[((long long)b * a.Sq + r) * a.k + j];
    if (e < 0 || e >= a.N) return -1;
  }
  return (long long)b * a.comp.cap + e;
}

// ------------------------------------------------------------------------------------------------
// MFMA kernel: H = 64, D = 512, q bf16, KV bf16 or mixed fp8/bf16
// ------------------------------------------------------------------------------------------------
constexpr int kTE = 32;            // entries per LDS tile
constexpr int kRowStride = 520;    // bf16 per entry row in the row-major tile
constexpr int kTStride = 36;       // bf16 per channel in the channel-major tile (32 entries + pad)
constexpr int kAttnThreads = 256;

__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t two) {
  return (uint32_t)f32_to_bf16(fp8_decode(two & 0xFFu)) | ((uint32_t)f32_to_bf16(fp8_decode((two >> 8) & 0xFFu)) << 16);
}

template <int FMT>
__global__ __launch_bounds__(kAttnThreads) void attn_mfma_kernel(AttnArgs a) {
  extern __shared__ uint16_t lds[];
  uint16_t* kt = lds;                                // [kTE][kRowStride]
  uint16_t* vt = lds + kTE * kRowStride;             // [512][kTStride]
  float* scale_s = (float*)(vt + 512 * kTStride);    // [kTE]
  int* valid_s = (int*)(scale_s + kTE);              // [kTE]

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hl = lane & 15, grp = lane >> 4;  // head within the wave's 16, lane group
  const int split = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const long long t = a.q_start + r;
  const RowList L = row_list(a, t);
  const int total = L.nw + L.nc;
  const int p_begin = split * a.split_len;
  const int p_end = min(p_begin + a.split_len, total);
  const int head = 16 * wave + hl;

  // Q^T B operand for 16 K-steps of 32 channels: lane holds q[head][32 s + 8 grp .. + 7]
  bf16x8_t qreg[16];
  {
    const uint16_t* qp = (const uint16_t*)a.q + (((long long)b * a.Sq + r) * 64 + head) * 512 + 8 * grp;
#pragma unroll
    for (int s = 0; s < 16; ++s) qreg[s] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(qp + 32 * s));
  }
  f32x4_t acc_o[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) acc_o[dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;

  const int ge = threadIdx.x & 31, gc = threadIdx.x >> 5;  // gather: entry, 64-channel chunk
  for (int p0 = p_begin; p0 < p_end; p0 += kTE) {
    __syncthreads();
    {  // gather 32 entries: thread (ge, gc) moves channels [64 gc, 64 gc + 64) of entry ge
      const int p = p0 + ge;
      const long long row = (p < p_end) ? list_row(a, L, b, r, p) : -1;
      const bool from_raw = p < L.nw;
      const lca_tensor& src = from_raw ? a.raw : a.comp;
      uint4 v[8];
      float sc = 1.0f;
      if (row >= 0) {
        if (FMT == LCA_BF16) {
          const uint4* gp = (const uint4*)((const uint16_t*)src.data + row * 512 + 64 * gc);
#pragma unroll
          for (int x = 0; x < 8; ++x) v[x] = gp[x];
        } else {
          if (gc < 7) {
            const uint4* gp = (const uint4*)((const uint8_t*)src.data + row * 448 + 64 * gc);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              uint4 c = gp[x];
              v[2 * x] = make_uint4(fp8x2_to_bf16x2(c.x), fp8x2_to_bf16x2(c.x >> 16), fp8x2_to_bf16x2(c.y),
                                    fp8x2_to_bf16x2(c.y >> 16));
              v[2 * x + 1] = make_uint4(fp8x2_to_bf16x2(c.z), fp8x2_to_bf16x2(c.z >> 16), fp8x2_to_bf16x2(c.w),
                                        fp8x2_to_bf16x2(c.w >> 16));
            }
          } else {
            const uint4* gp = (const uint4*)((const uint16_t*)src.rope + row * 64);
#pragma unroll
            for (int x = 0; x < 8; ++x) v[x] = gp[x];
          }
          sc = ((const float*)src.scale)[row];
        }
      } else {
#pragma unroll
        for (int x = 0; x < 8; ++x) v[x] = make_uint4(0, 0, 0, 0);
      }
      uint4* kp = (uint4*)(kt + ge * kRowStride + 64 * gc);
#pragma unroll
      for (int x = 0; x < 8; ++x) kp[x] = v[x];
      const uint16_t* hv = (const uint16_t*)v;
#pragma unroll
      for (int x = 0; x < 64; ++x) vt[(64 * gc + x) * kTStride + ge] = hv[x];
      if (gc == 0) {
        scale_s[ge] = sc;
        valid_s[ge] = row >= 0;
      }
    }
    __syncthreads();

    // S^T = K Q^T for two 16-entry tiles
    float lg[2][4];
#pragma unroll
    for (int et = 0; et < 2; ++et) {
      f32x4_t am = {0.0f, 0.0f, 0.0f, 0.0f}, ar = {0.0f, 0.0f, 0.0f, 0.0f};
      const uint16_t* kp = kt + (16 * et + hl) * kRowStride + 8 * grp;
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, *(const uint4*)(kp + 32 * s));
        if (FMT == LCA_MIXED_FP8 && s >= 14)
          ar = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qreg[s], ar, 0, 0, 0);
        else
          am = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qreg[s], am, 0, 0, 0);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int e = 16 * et + 4 * grp + x;
        float l = (FMT == LCA_MIXED_FP8) ? a.scale * (scale_s[e] * am[x] + ar[x]) : a.scale * am[x];
        lg[et][x] = valid_s[e] ? l : -INFINITY;
      }
    }
    // online softmax for head `head` (lanes hl, hl+16, hl+32, hl+48 hold its 32 logits)
    float mt = fmaxf(fmaxf(fmaxf(lg[0][0], lg[0][1]), fmaxf(lg[0][2], lg[0][3])),
                     fmaxf(fmaxf(lg[1][0], lg[1][1]), fmaxf(lg[1][2], lg[1][3])));
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = (m_new == -INFINITY) ? 1.0f : __expf(m_run - m_new);
    float pv[2][4], psum = 0.0f;
#pragma unroll
    for (int et = 0; et < 2; ++et)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        pv[et][x] = (lg[et][x] == -INFINITY) ? 0.0f : __expf(lg[et][x] - m_new);
        psum += pv[et][x];
      }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) acc_o[dt] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int et = 0; et < 2; ++et) {
      s16x4_t pb, pbs;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        pb[x] = (short)f32_to_bf16(pv[et][x]);
        pbs[x] = (short)f32_to_bf16(pv[et][x] * scale_s[16 * et + 4 * grp + x]);
      }
      const uint16_t* vp = vt + hl * kTStride + 16 * et + 4 * grp;
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) {
        const s16x4_t av = __builtin_bit_cast(s16x4_t, *(const uint2*)(vp + 16 * dt * kTStride));
        const s16x4_t bop = (FMT == LCA_MIXED_FP8 && dt < 28) ? pbs : pb;
        acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bop, acc_o[dt], 0, 0, 0);
      }
    }
  }

  // lane holds o^T[channel 16 dt + 4 grp + x][head]
  const long long item = ((long long)b * a.Sq + r) * a.n_splits + split;
  if (a.n_splits == 1) {
    const float z = a.sink[head];
    const float M = fmaxf(m_run, z);
    float den, f;
    if (M == -INFINITY) {
      den = 0.0f;
      f = 0.0f;
    } else {
      den = ((z == -INFINITY) ? 0.0f : __expf(z - M)) + l_run * ((m_run == -INFINITY) ? 0.0f : __expf(m_run - M));
      f = (m_run == -INFINITY) ? 0.0f : __expf(m_run - M) / den;
    }
    const long long ob = (((long long)b * a.Sq + r) * 64 + head) * 512;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const int c0 = 16 * dt + 4 * grp;
      if (a.out_format == LCA_F32) {
        *(float4*)((float*)a.out + ob + c0) =
            make_float4(acc_o[dt][0] * f, acc_o[dt][1] * f, acc_o[dt][2] * f, acc_o[dt][3] * f);
      } else {
        uint2 w2;
        w2.x = (uint32_t)f32_to_bf16(acc_o[dt][0] * f) | ((uint32_t)f32_to_bf16(acc_o[dt][1] * f) << 16);
        w2.y = (uint32_t)f32_to_bf16(acc_o[dt][2] * f) | ((uint32_t)f32_to_bf16(acc_o[dt][3] * f) << 16);
        *(uint2*)((uint16_t*)a.out + ob + c0) = w2;
      }
    }
    if (a.lse && grp == 0) a.lse[((long long)b * a.Sq + r) * 64 + head] = (M == -INFINITY) ? -INFINITY : M + __logf(den);
  } else {
    float* po = a.part_o + (item * 64 + head) * 512;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt)
      *(float4*)(po + 16 * dt + 4 * grp) = make_float4(acc_o[dt][0], acc_o[dt][1], acc_o[dt][2], acc_o[dt][3]);
    if (grp == 0) {
      a.part_ml[(item * 64 + head) * 2 + 0] = m_run;
      a.part_ml[(item * 64 + head) * 2 + 1] = l_run;
    }
  }
}

// ------------------------------------------------------------------------------------------------
// head-group MFMA kernel (few query rows: decode): H = 64, D = 512, bf16 or mixed fp8/bf16 entries
// ------------------------------------------------------------------------------------------------
// A workgroup owns 16 heads (one head group) of one query row and one slice of the row's entry list; each of its
// four waves takes every fourth 16-entry tile of the slice:
//   S^T = K Q^T     v_mfma_f32_16x16x32_bf16, A = the tile's 16 rows from LDS, B = the 16 heads' queries (LDS)
//   O^T += V^T P^T  v_mfma_f32_16x16x16_bf16, A = V^T read by ds_read_b64_tr_b16 straight from the row-major tile,
//                   B = P^T, which is exactly the S^T accumulator layout (lane: head l % 16, entries 4 (l / 16) + v)
// ds_read_b64_tr_b16: in each 16-lane group, output lane 4a + e takes element e of the 8-byte chunks addressed by
// group lanes a, a + 4, a + 8, a + 12.  Group lane a + 4v addresses entry 4G + v, channels 16 dt + 4a .. + 3, so
// lane 4a + e receives V[4G + v][16 dt + 4a + e] for v = 0..3, the A layout of the 16x16x16 instruction.
// fp8 entries are widened to bf16 exactly when the tile is written to LDS; their per-entry scale multiplies the
// fp8-channel part of the logit and is folded into P for the fp8 channels.
// The four waves' (max, sum, o) are merged in LDS at the end; the four head groups of a (row, slice) pair get
// workgroup ids congruent mod 8 so that they run on one XCD and share its L2 copy of the gathered entries.
constexpr int kHgRow = 520;                                   // bf16 per LDS row (1040 bytes)
constexpr int kHgOStride = 516;                               // floats per head row in the merge buffer

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Each wave owns its own 16-entry LDS tile.  The next tile's 16 rows are loaded into registers (one wave-wide
// 16-byte load per row, fully coalesced) while the current tile is scored, then written over the consumed tile, so
// gathers overlap compute and no workgroup barrier is needed until the final merge.
constexpr int kWTile = 16;
constexpr float kRescaleSlack = 8.0f;
constexpr int kWBufBytes = kWTile * kHgRow * 2;  // 16640
// four wave tiles, then the per-wave (max, sum) of the merge; the merge's 2 x 16 x kHgOStride floats reuse the tiles
// + the 16 heads' queries (shared), the waves' (max, sum) and entry scales
constexpr size_t kHgwLds = (size_t)5 * kWBufBytes + 4 * 16 * 2 * 4 + 4 * 16 * 4;
static_assert((size_t)2 * 16 * kHgOStride * 4 <= (size_t)4 * kWBufBytes, "merge buffer fits the tiles");

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4_t gbl_u32x4_t;

struct WaveTile {
  uint4 v[kWTile];  // lane i: bytes 16 i .. 16 i + 15 of each of the tile's 16 rows
  uint64_t valid;   // bit j: entry j of the tile is real (padding loads a mapped dummy row, masked in the logits)
};

// Loads the 16 rows of list positions [p0, p0 + 16) into registers; each wave-wide 16-byte load reads one whole
// 1 KB row.  Loads go through the global address space (not flat) so that waits on LDS traffic do not also wait
// for these loads.
__device__ __forceinline__ WaveTile wave_load_tile(const AttnArgs& a, const RowList& L, int b, int r, int p0,
                                                   int p_end, int lane) {
  WaveTile T;
  const int p = p0 + (lane & 15);
  long long row = -1;
  if (lane < 16 && p < p_end) row = list_row(a, L, b, r, p);
  const bool valid = row >= 0;
  const unsigned long long base =
      valid ? (unsigned long long)((const uint8_t*)(p < L.nw ? a.raw.data : a.comp.data) + row * 1024)
            : (unsigned long long)((const uint8_t*)a.comp.data + (long long)b * a.comp.cap * 1024);
  T.valid = __ballot(valid) & 0xFFFFull;
#pragma unroll
  for (int j = 0; j < kWTile; ++j) {
    const unsigned long long rb = __shfl(base, j, 64);
    const u32x4_t x = *(gbl_u32x4_t*)(rb + 16 * (unsigned long long)lane);
    T.v[j] = make_uint4(x.x, x.y, x.z, x.w);
  }
  return T;
}

__device__ __forceinline__ void wave_store_tile(uint8_t* buf, int lane, const WaveTile& T) {
#pragma unroll
  for (int j = 0; j < kWTile; ++j) *(uint4*)(buf + j * (kHgRow * 2) + 16 * lane) = T.v[j];
}

typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;

// Four OCP e4m3 codes -> four bf16 (exact: every e4m3 value is a bf16 value), via the hardware fp8 -> f32 conversion.
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t w) {
  const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  uint2 r;
  r.x = (__float_as_uint(lo[0]) >> 16) | (__float_as_uint(lo[1]) & 0xFFFF0000u);
  r.y = (__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xFFFF0000u);
  return r;
}

struct WaveTileMixed {
  uint4 v[kWTile];  // lane c < 28: fp8 chunk c (channels 16c .. 16c + 15); 28 <= c < 36: RoPE chunk c - 28
  float scale;      // lane j < 16: the per-entry fp8 scale of row j
  uint64_t valid;
};

__device__ __forceinline__ WaveTileMixed wave_load_tile_mixed(const AttnArgs& a, const RowList& L, int b, int r,
                                                              int p0, int p_end, int lane) {
  WaveTileMixed T;
  const int p = p0 + (lane & 15);
  long long row = -1;
  if (lane < 16 && p < p_end) row = list_row(a, L, b, r, p);
  const bool valid = row >= 0;
  const bool raw = valid && p < L.nw;
  const long long rr = valid ? row : (long long)b * a.comp.cap;
  const lca_tensor& src = raw ? a.raw : a.comp;
  const unsigned long long fbase = (unsigned long long)((const uint8_t*)src.data + rr * 448);
  const unsigned long long rbase = (unsigned long long)((const uint8_t*)src.rope + rr * 128);
  T.scale = valid ? ((const float*)src.scale)[rr] : 1.0f;
  T.valid = __ballot(valid) & 0xFFFFull;
  const unsigned long long off = lane < 28 ? 16ull * lane : 16ull * (lane - 28);
#pragma unroll
  for (int j = 0; j < kWTile; ++j) {
    const unsigned long long fb = __shfl(fbase, j, 64), rb = __shfl(rbase, j, 64);
    if (lane < 36) {
      const u32x4_t x = *(gbl_u32x4_t*)((lane < 28 ? fb : rb) + off);
      T.v[j] = make_uint4(x.x, x.y, x.z, x.w);
    } else {
      T.v[j] = make_uint4(0, 0, 0, 0);
    }
  }
  return T;
}

__device__ __forceinline__ void wave_store_tile_mixed(uint8_t* buf, float* scale_w, int lane, const WaveTileMixed& T) {
#pragma unroll
  for (int j = 0; j < kWTile; ++j) {
    uint8_t* row = buf + j * (kHgRow * 2);
    if (lane < 28) {
      const uint2 a0 = fp8x4_to_bf16x4(T.v[j].x), a1 = fp8x4_to_bf16x4(T.v[j].y);
      const uint2 a2 = fp8x4_to_bf16x4(T.v[j].z), a3 = fp8x4_to_bf16x4(T.v[j].w);
      *(uint4*)(row + 32 * lane) = make_uint4(a0.x, a0.y, a1.x, a1.y);
      *(uint4*)(row + 32 * lane + 16) = make_uint4(a2.x, a2.y, a3.x, a3.y);
    } else if (lane < 36) {
      *(uint4*)(row + 896 + 16 * (lane - 28)) = T.v[j];
    }
  }
  if (lane < 16) scale_w[lane] = T.scale;
}

template <int FMT>
__global__ __launch_bounds__(256) void attn_hgw_kernel(AttnArgs a, int pairs) {
  extern __shared__ __attribute__((aligned(16))) uint8_t hgw_lds[];
  const int id = blockIdx.x;
  const int hg = (id & 31) >> 3;
  const int pair = (id >> 5) * 8 + (id & 7);
  if (pair >= pairs) return;
  const int S = a.n_splits;
  const int qrow = pair / S, split = pair % S;
  const int b = qrow / a.Sq, r = qrow % a.Sq;
  const long long t = a.q_start + r;
  const RowList L = row_list(a, t);
  const int total = L.nw + L.nc;
  const int p_begin = split * a.split_len;
  const int p_end = min(p_begin + a.split_len, total);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hl = lane & 15, grp = lane >> 4;
  const int head = 16 * hg + hl;
  uint8_t* wbuf = hgw_lds + wave * kWBufBytes;
  uint16_t* q_s = (uint16_t*)(hgw_lds + 4 * kWBufBytes);  // [16 heads][kHgRow]
  float* ml_s = (float*)(hgw_lds + 5 * kWBufBytes);         // [4 waves][16 heads][2]
  float* esc_w = ml_s + 4 * 16 * 2 + 16 * wave;             // [4 waves][16] entry scales (fp8 cache)

  const int ntiles = p_end > p_begin ? (p_end - p_begin + kWTile - 1) / kWTile : 0;
  int tt = wave;
  uint64_t cur = 0;
  if (tt < ntiles) {
    if (FMT == LCA_BF16) {
      const WaveTile T0 = wave_load_tile(a, L, b, r, p_begin + kWTile * tt, p_end, lane);
      wave_store_tile(wbuf, lane, T0);
      cur = T0.valid;
    } else {
      const WaveTileMixed T0 = wave_load_tile_mixed(a, L, b, r, p_begin + kWTile * tt, p_end, lane);
      wave_store_tile_mixed(wbuf, esc_w, lane, T0);
      cur = T0.valid;
    }
  }

  {  // the 16 heads' queries (16 KB), once per workgroup: thread -> 4 chunks of 16 bytes
    const uint8_t* qg = (const uint8_t*)a.q + ((long long)qrow * 64 + 16 * hg) * 1024;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int c = threadIdx.x + 256 * x, h = c >> 6, piece = c & 63;
      *(uint4*)((uint8_t*)q_s + h * (kHgRow * 2) + 16 * piece) = *(const uint4*)(qg + h * 1024 + 16 * piece);
    }
  }
  __syncthreads();
  f32x4_t acc_o[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) acc_o[dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;
  const uint16_t* qsp = q_s + hl * kHgRow + 8 * grp;

  for (; tt < ntiles; tt += 4) {
    // the next tile's rows are in flight while this one is scored (past the slice end: masked dummy rows)
    WaveTile nxt;
    WaveTileMixed nxm;
    if (FMT == LCA_BF16)
      nxt = wave_load_tile(a, L, b, r, p_begin + kWTile * (tt + 4), p_end, lane);
    else
      nxm = wave_load_tile_mixed(a, L, b, r, p_begin + kWTile * (tt + 4), p_end, lane);
    const uint16_t* kt = (const uint16_t*)wbuf;

    f32x4_t am = {0.0f, 0.0f, 0.0f, 0.0f}, ar = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint16_t* kp = kt + hl * kHgRow + 8 * grp;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const bf16x8_t kv = __builtin_bit_cast(bf16x8_t, *(const uint4*)(kp + 32 * s));
      const bf16x8_t qv = __builtin_bit_cast(bf16x8_t, *(const uint4*)(qsp + 32 * s));
      if (FMT == LCA_MIXED_FP8 && s >= 14)  // RoPE channels: bf16, not scaled
        ar = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qv, ar, 0, 0, 0);
      else
        am = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qv, am, 0, 0, 0);
    }
    float lg[4], esc[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      esc[x] = (FMT == LCA_MIXED_FP8) ? esc_w[4 * grp + x] : 1.0f;
      const float l = (FMT == LCA_MIXED_FP8) ? a.scale * (esc[x] * am[x] + ar[x]) : a.scale * am[x];
      lg[x] = ((cur >> (4 * grp + x)) & 1ull) ? l : -INFINITY;
    }
    float mt = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    // The reference max only moves when a logit exceeds it by more than kRescaleSlack (e^8 keeps every weight and
    // sum far inside fp32, and bf16 keeps 8 significant bits at any scale), so the accumulators are rescaled a few
    // times per row instead of on every tile.
    const float m_new = (mt > m_run + kRescaleSlack) ? mt : m_run;
    const float alpha = (m_new == m_run) ? 1.0f : __expf(m_run - m_new);
    float pv[4], psum = 0.0f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      pv[x] = (lg[x] == -INFINITY) ? 0.0f : __expf(lg[x] - m_new);
      psum += pv[x];
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    s16x4_t pb, pbs;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      pb[x] = (short)f32_to_bf16(pv[x]);
      pbs[x] = (FMT == LCA_MIXED_FP8) ? (short)f32_to_bf16(pv[x] * esc[x]) : pb[x];  // fp8 channels carry the scale
    }
    const uint16_t* vp = kt + (4 * grp + (hl >> 2)) * kHgRow + 4 * (hl & 3);
    if (__ballot(alpha != 1.0f)) {  // wave-uniform: some head's reference max moved
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) acc_o[dt] *= alpha;
    }
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const s16x4_t av = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vp + 16 * dt));
      acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, (FMT == LCA_MIXED_FP8 && dt < 28) ? pbs : pb, acc_o[dt],
                                                            0, 0, 0);
    }
    if (FMT == LCA_BF16) {  // the tile's LDS reads are complete: refill in place
      wave_store_tile(wbuf, lane, nxt);
      cur = nxt.valid;
    } else {
      wave_store_tile_mixed(wbuf, esc_w, lane, nxm);
      cur = nxm.valid;
    }
  }

  // merge the four waves (same heads, different entries)
  __syncthreads();
  if (grp == 0) {
    ml_s[(wave * 16 + hl) * 2 + 0] = m_run;
    ml_s[(wave * 16 + hl) * 2 + 1] = l_run;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, ml_s[(w * 16 + hl) * 2 + 0]);
  float Lsum = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mw = ml_s[(w * 16 + hl) * 2 + 0];
    Lsum += (mw == -INFINITY) ? 0.0f : ml_s[(w * 16 + hl) * 2 + 1] * __expf(mw - M);
  }
  const float own = (m_run == -INFINITY) ? 0.0f : __expf(m_run - M);
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) acc_o[dt] *= own;
  float* ob = (float*)hgw_lds;  // [2][16][kHgOStride]
  if (wave >= 2) {
#pragma unroll
    for (int dt = 0; dt < 32; ++dt)
      *(f32x4_t*)(ob + ((wave - 2) * 16 + hl) * kHgOStride + 16 * dt + 4 * grp) = acc_o[dt];
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) acc_o[dt] += *(const f32x4_t*)(ob + (wave * 16 + hl) * kHgOStride + 16 * dt + 4 * grp);
  }
  __syncthreads();
  if (wave == 1) {
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) *(f32x4_t*)(ob + hl * kHgOStride + 16 * dt + 4 * grp) = acc_o[dt];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) acc_o[dt] += *(const f32x4_t*)(ob + hl * kHgOStride + 16 * dt + 4 * grp);

  if (S == 1) {
    const float z = a.sink[head];
    const float Mz = fmaxf(M, z);
    float den = 0.0f, f = 0.0f;
    if (Mz != -INFINITY) {
      den = ((z == -INFINITY) ? 0.0f : __expf(z - Mz)) + ((M == -INFINITY) ? 0.0f : Lsum * __expf(M - Mz));
      f = (M == -INFINITY) ? 0.0f : __expf(M - Mz) / den;
    }
    const long long obase = ((long long)qrow * 64 + head) * 512;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const int c0 = 16 * dt + 4 * grp;
      if (a.out_format == LCA_F32) {
        *(float4*)((float*)a.out + obase + c0) =
            make_float4(acc_o[dt][0] * f, acc_o[dt][1] * f, acc_o[dt][2] * f, acc_o[dt][3] * f);
      } else {
        uint2 w2;
        w2.x = (uint32_t)f32_to_bf16(acc_o[dt][0] * f) | ((uint32_t)f32_to_bf16(acc_o[dt][1] * f) << 16);
        w2.y = (uint32_t)f32_to_bf16(acc_o[dt][2] * f) | ((uint32_t)f32_to_bf16(acc_o[dt][3] * f) << 16);
        *(uint2*)((uint16_t*)a.out + obase + c0) = w2;
      }
    }
    if (a.lse && grp == 0) a.lse[(long long)qrow * 64 + head] = (Mz == -INFINITY) ? -INFINITY : Mz + __logf(den);
  } else {
    const long long item = (long long)qrow * S + split;
    float* po = a.part_o + (item * 64 + head) * 512;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) *(f32x4_t*)(po + 16 * dt + 4 * grp) = acc_o[dt];
    if (grp == 0) {
      a.part_ml[(item * 64 + head) * 2 + 0] = M;
      a.part_ml[(item * 64 + head) * 2 + 1] = Lsum;
    }
  }
}

// ------------------------------------------------------------------------------------------------
// vector-ALU kernel: H * D <= 8192, any supported format (fp32 accumulation)
// ------------------------------------------------------------------------------------------------
constexpr int kSimtTE = 8;

__device__ __forceinline__ float kv_elem(const lca_tensor& t, long long row, int j) {
  if (t.format == LCA_F32) return ((const float*)t.data)[row * t.dim + j];
  if (t.format == LCA_BF16) return bf16_to_f32(((const uint16_t*)t.data)[row * t.dim + j]);
  const int dm = t.dim - t.rope_dims;
  if (j < dm) return fp8_decode(((const uint8_t*)t.data)[row * dm + j]) * ((const float*)t.scale)[row];
  return bf16_to_f32(((const uint16_t*)t.rope)[row * t.rope_dims + (j - dm)]);
}

__global__ __launch_bounds__(256) void attn_simt_kernel(AttnArgs a) {
  __shared__ float o_s[8192];
  __shared__ float kv_s[kSimtTE * 513];
  __shared__ float lg_s[64 * kSimtTE];
  __shared__ float alpha_s[64];
  __shared__ float m_s[64], l_s[64];
  const int H = a.H, D = a.D;
  const int split = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const long long t = a.q_start + r;
  const RowList L = row_list(a, t);
  const int total = L.nw + L.nc;
  const int p_begin = split * a.split_len;
  const int p_end = min(p_begin + a.split_len, total);
  const long long qrow0 = ((long long)b * a.Sq + r) * H;
  for (int x = threadIdx.x; x < H * D; x += blockDim.x) o_s[x] = 0.0f;
  for (int h = threadIdx.x; h < H; h += blockDim.x) {
    m_s[h] = -INFINITY;
    l_s[h] = 0.0f;
  }
  for (int p0 = p_begin; p0 < p_end; p0 += kSimtTE) {
    __syncthreads();
    for (int x = threadIdx.x; x < kSimtTE * D; x += blockDim.x) {
      const int e = x / D, j = x % D;
      const int p = p0 + e;
      const long long row = (p < p_end) ? list_row(a, L, b, r, p) : -1;
      kv_s[e * 513 + j] = row >= 0 ? kv_elem(p < L.nw ? a.raw : a.comp, row, j) : 0.0f;
      if (j == 0) lg_s[e] = row >= 0 ? 1.0f : 0.0f;  // validity flag, overwritten below
    }
    __syncthreads();
    float valid[kSimtTE];
#pragma unroll
    for (int e = 0; e < kSimtTE; ++e) valid[e] = lg_s[e];
    __syncthreads();
    for (int x = threadIdx.x; x < H * kSimtTE; x += blockDim.x) {
      const int h = x / kSimtTE, e = x % kSimtTE;
      float d = 0.0f;
      for (int j = 0; j < D; ++j) {
        float qv = (a.q_format == LCA_F32) ? ((const float*)a.q)[(qrow0 + h) * D + j]
                                           : bf16_to_f32(((const uint16_t*)a.q)[(qrow0 + h) * D + j]);
        d = fmaf(qv, kv_s[e * 513 + j], d);
      }
      lg_s[h * kSimtTE + e] = valid[e] != 0.0f ? a.scale * d : -INFINITY;
    }
    __syncthreads();
    for (int h = threadIdx.x; h < H; h += blockDim.x) {
      float mt = -INFINITY;
      for (int e = 0; e < kSimtTE; ++e) mt = fmaxf(mt, lg_s[h * kSimtTE + e]);
      const float m_new = fmaxf(m_s[h], mt);
      const float al = (m_new == -INFINITY) ? 1.0f : __expf(m_s[h] - m_new);
      float ps = 0.0f;
      for (int e = 0; e < kSimtTE; ++e) {
        float l = lg_s[h * kSimtTE + e];
        float pe = (l == -INFINITY) ? 0.0f : __expf(l - m_new);
        lg_s[h * kSimtTE + e] = pe;
        ps += pe;
      }
      l_s[h] = l_s[h] * al + ps;
      m_s[h] = m_new;
      alpha_s[h] = al;
    }
    __syncthreads();
    for (int x = threadIdx.x; x < H * D; x += blockDim.x) {
      const int h = x / D, j = x % D;
      float acc = o_s[x] * alpha_s[h];
      for (int e = 0; e < kSimtTE; ++e) acc = fmaf(lg_s[h * kSimtTE + e], kv_s[e * 513 + j], acc);
      o_s[x] = acc;
    }
  }
  __syncthreads();
  const long long item = ((long long)b * a.Sq + r) * a.n_splits + split;
  if (a.n_splits == 1) {
    for (int x = threadIdx.x; x < H * D; x += blockDim.x) {
      const int h = x / D;
      const float z = a.sink[h], mr = m_s[h];
      const float M = fmaxf(mr, z);
      float f = 0.0f;
      if (M != -INFINITY && mr != -INFINITY) {
        float den = ((z == -INFINITY) ? 0.0f : __expf(z - M)) + l_s[h] * __expf(mr - M);
        f = __expf(mr - M) / den;
      }
      const float v = o_s[x] * f;
      const long long oi = (qrow0 + h) * D + (x % D);
      if (a.out_format == LCA_F32)
        ((float*)a.out)[oi] = v;
      else
        ((uint16_t*)a.out)[oi] = f32_to_bf16(v);
    }
    if (a.lse) {
      for (int h = threadIdx.x; h < H; h += blockDim.x) {
        const float z = a.sink[h], mr = m_s[h];
        const float M = fmaxf(mr, z);
        float lv = -INFINITY;
        if (M != -INFINITY) {
          float den = ((z == -INFINITY) ? 0.0f : __expf(z - M)) + ((mr == -INFINITY) ? 0.0f : l_s[h] * __expf(mr - M));
          lv = M + __logf(den);
        }
        a.lse[qrow0 + h] = lv;
      }
    }
  } else {
    for (int x = threadIdx.x; x < H * D; x += blockDim.x) a.part_o[item * H * D + x] = o_s[x];
    for (int h = threadIdx.x; h < H; h += blockDim.x) {
      a.part_ml[(item * H + h) * 2 + 0] = m_s[h];
      a.part_ml[(item * H + h) * 2 + 1] = l_s[h];
    }
  }
}

// ------------------------------------------------------------------------------------------------
// merge of splits + sink
// ------------------------------------------------------------------------------------------------
// One workgroup per (head, query row, sequence): combine the splits' (max, sum, o) with the sink.
constexpr int kMergeThreads = 128;
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(AttnArgs a) {
  extern __shared__ float wsplit[];  // [n_splits] weights e^(m_s - M)
  __shared__ float red[kMergeThreads / 64];
  __shared__ float stat[2];
  const int h = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int H = a.H, D = a.D, S = a.n_splits;
  const long long item0 = ((long long)b * a.Sq + r) * S;
  const float z = a.sink[h];
  // M = max(z, m_s)
  float mloc = -INFINITY;
  for (int s = threadIdx.x; s < S; s += blockDim.x) mloc = fmaxf(mloc, a.part_ml[((item0 + s) * H + h) * 2 + 0]);
  mloc = wave_max(mloc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mloc;
  __syncthreads();
  float M = z;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) M = fmaxf(M, red[i]);
  __syncthreads();
  // den = e^(z - M) + sum_s e^(m_s - M) l_s
  float dloc = 0.0f;
  for (int s = threadIdx.x; s < S; s += blockDim.x) {
    const float ms = a.part_ml[((item0 + s) * H + h) * 2 + 0];
    const float wgt = (M == -INFINITY || ms == -INFINITY) ? 0.0f : __expf(ms - M);
    wsplit[s] = wgt;
    dloc += wgt * a.part_ml[((item0 + s) * H + h) * 2 + 1];
  }
  dloc = wave_sum(dloc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = dloc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float den = (M == -INFINITY || z == -INFINITY) ? 0.0f : __expf(z - M);
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) den += red[i];
    stat[0] = den > 0.0f ? 1.0f / den : 0.0f;
    if (a.lse) a.lse[((long long)b * a.Sq + r) * H + h] = (M == -INFINITY) ? -INFINITY : M + __logf(den);
  }
  __syncthreads();
  const float inv = stat[0];
  const long long ob = (((long long)b * a.Sq + r) * H + h) * D;
  for (int x = threadIdx.x; x < D; x += blockDim.x) {
    float acc = 0.0f;
    for (int s = 0; s < S; ++s) acc = fmaf(wsplit[s], a.part_o[((item0 + s) * H + h) * D + x], acc);
    const float v = acc * inv;
    if (a.out_format == LCA_F32)
      ((float*)a.out)[ob + x] = v;
    else
      ((uint16_t*)a.out)[ob + x] = f32_to_bf16(v);
  }
}

constexpr size_t kMfmaLds = (size_t)kTE * kRowStride * 2 + (size_t)512 * kTStride * 2 + kTE * 4 * 2;
static bool g_attn_attr[64];
static bool g_hg_attr[64];

bool attn_uses_mfma(int H, int D, int q_format, int kv_format) {
  return H == 64 && D == 512 && q_format == LCA_BF16 && (kv_format == LCA_BF16 || kv_format == LCA_MIXED_FP8);
}

hipError_t launch_attn(AttnArgs a, hipStream_t st) {
  const bool mfma = attn_uses_mfma(a.H, a.D, a.q_format, a.comp.format);
  dim3 grid((unsigned)a.n_splits, (unsigned)a.Sq, (unsigned)a.B);
  clear_stale_error();
  if (mfma && a.hg_mode) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    if (dev >= 0 && dev < 64 && !g_hg_attr[dev]) {
      hipError_t e = hipFuncSetAttribute((const void*)attn_hgw_kernel<LCA_BF16>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)kHgwLds);
      if (e == hipSuccess)
        e = hipFuncSetAttribute((const void*)attn_hgw_kernel<LCA_MIXED_FP8>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)kHgwLds);
      if (e != hipSuccess) return e;
      g_hg_attr[dev] = true;
    }
    const int pairs = a.B * a.Sq * a.n_splits;
    const dim3 hgrid((unsigned)(((pairs + 7) / 8) * 32));
    if (a.comp.format == LCA_BF16)
      hipLaunchKernelGGL(attn_hgw_kernel<LCA_BF16>, hgrid, dim3(256), kHgwLds, st, a, pairs);
    else
      hipLaunchKernelGGL(attn_hgw_kernel<LCA_MIXED_FP8>, hgrid, dim3(256), kHgwLds, st, a, pairs);
  } else if (mfma) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    if (dev >= 0 && dev < 64 && !g_attn_attr[dev]) {
      hipError_t e = hipFuncSetAttribute((const void*)attn_mfma_kernel<LCA_BF16>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMfmaLds);
      if (e == hipSuccess)
        e = hipFuncSetAttribute((const void*)attn_mfma_kernel<LCA_MIXED_FP8>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMfmaLds);
      if (e != hipSuccess) return e;
      g_attn_attr[dev] = true;
    }
    if (a.comp.format == LCA_BF16)
      hipLaunchKernelGGL(attn_mfma_kernel<LCA_BF16>, grid, dim3(kAttnThreads), kMfmaLds, st, a);
    else
      hipLaunchKernelGGL(attn_mfma_kernel<LCA_MIXED_FP8>, grid, dim3(kAttnThreads), kMfmaLds, st, a);
  } else {
    hipLaunchKernelGGL(attn_simt_kernel, grid, dim3(256), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_splits == 1) return e;
  const size_t lds = sizeof(float) * (size_t)a.n_splits;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)a.H, (unsigned)a.Sq, (unsigned)a.B), dim3(kMergeThreads), lds,
                     st, a);
  return hipGetLastError();
}

}  // namespace lca
