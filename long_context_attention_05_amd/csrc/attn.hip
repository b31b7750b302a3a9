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
    for (int s = 0; s < S; ++s) {
      const float wgt = wsplit[s];
      if (wgt != 0.0f) acc = fmaf(wgt, a.part_o[((item0 + s) * H + h) * D + x], acc);
    }
    const float v = acc * inv;
    if (a.out_format == LCA_F32)
      ((float*)a.out)[ob + x] = v;
    else
      ((uint16_t*)a.out)[ob + x] = f32_to_bf16(v);
  }
}

constexpr size_t kMfmaLds = (size_t)kTE * kRowStride * 2 + (size_t)512 * kTStride * 2 + kTE * 4 * 2;
static bool g_attn_attr[64];

bool attn_uses_mfma(int H, int D, int q_format, int kv_format) {
  return H == 64 && D == 512 && q_format == LCA_BF16 && (kv_format == LCA_BF16 || kv_format == LCA_MIXED_FP8);
}

hipError_t launch_attn(AttnArgs a, hipStream_t st) {
  const bool mfma = attn_uses_mfma(a.H, a.D, a.q_format, a.comp.format);
  dim3 grid((unsigned)a.n_splits, (unsigned)a.Sq, (unsigned)a.B);
  clear_stale_error();
  if (mfma) {
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
