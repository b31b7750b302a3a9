// compress.hip -- stage 1 (KV compression) and the cache codec's quantise-on-write.
//
// KV compression follows the paper notes ("DeepSeek-V4: Towards Highly Efficient Million-Token Context
// Intelligence"), section 2.3 Eq. 11-12 and the Compressor excerpt, and section 2.4 Eq. 22-23: per channel,
// a softmax over the candidates' logits (gate + learned position bias) weights the candidates' values;
// with overlap (CSA) the candidates are the block's own tokens from stream a plus the previous block's tokens
// from stream b.  The work is a pure HBM stream (each input value is read once, 1/m as much is written), so it
// runs on the vector ALU: one workgroup per (entry, sequence), one thread per channel slice, loads coalesced
// along channels, an online softmax in fp32.
//
// The codec (mixed-precision cache: cosmocat page section 3; Mind Observatory page) is applied in the same
// pass: fp32 entries are encoded to bf16 / fp8 e4m3 with a per-entry scale plus bf16 RoPE dims / fp4 e2m1 with
// one power-of-two scale per 32-element block while the row is still in registers.
#include "lca_device.h"
#include "lca_internal.h"

namespace lca {

constexpr int kRowThreads = 256;

struct RowOut {
  int format, dim, rope, rotate;
  long long cap;
  void* data;
  void* rope_data;
  void* scale;
  const int32_t* table;  // paged output: block table [B][cap / block_rows] (else NULL)
  int block_rows;
};

// Storage row of row i of sequence b of the output (see tensor_row).
__device__ __forceinline__ long long out_row(const RowOut& o, int b, long long i) {
  if (!o.table) return (long long)b * o.cap + i;
  const int sh = __builtin_ctz((unsigned)o.block_rows);
  return (long long)o.table[(long long)b * (o.cap >> sh) + (i >> sh)] * o.block_rows + (i & (o.block_rows - 1));
}

__device__ __forceinline__ float block_max_256(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = fmaxf(r, red[i]);
  return r;
}

__device__ __forceinline__ float block_sum_256(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r += red[i];
  return r;
}

constexpr int kRotMaxDim = 1024;

// Orthonormal Sylvester-Hadamard rotation of a row held as v[u] = channel (threadIdx.x + blockDim.x * u)
// (paper notes, the Indexer excerpt: indexer queries and keys are rotated before their FP4 quantisation).
// dim is a power of two <= kRotMaxDim.  Stage h (h = 1, 2, 4, ...) maps the pair (j, j + h), j & h == 0, to
// (x_j + x_{j+h}, x_j - x_{j+h}), the stages with h >= 64 through an LDS ping-pong buffer; after log2(dim) stages every output is the sum of
// all inputs with the signs (-1)^popcount(i & j), and one multiply by 1/sqrt(dim) (exact for even powers of two,
// fl32(sqrt(2)) * 2^-(p+1)/2 for odd p) makes the matrix orthonormal.  All threads of the block take part.
// Stages with h < 64 pair lanes of one wave (channel j ^ h sits in lane ^ h, same u, since blockDim is a multiple of
// 64) and run on shuffles with the same operands as the LDS stages.
template <int CPT>
__device__ void hadamard_row(float (&v)[CPT], int dim, float* buf) {
  const int nt = blockDim.x;
  const int hw = dim < 64 ? dim : 64;
  for (int h = 1; h < hw; h <<= 1) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int j = threadIdx.x + nt * u;
      const float o = __shfl_xor(v[u], h, 64);
      v[u] = (j & h) ? o - v[u] : v[u] + o;
    }
  }
  float* x = buf;
  float* y = buf + kRotMaxDim;
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int j = threadIdx.x + nt * u;
    if (j < dim) x[j] = v[u];
  }
  __syncthreads();
  for (int h = hw; h < dim; h <<= 1) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int j = threadIdx.x + nt * u;
      if (j < dim) {
        const float a = x[j & ~h], b = x[j | h];
        y[j] = (j & h) ? a - b : a + b;
      }
    }
    __syncthreads();
    float* t = x;
    x = y;
    y = t;
  }
  const int p = 31 - __clz(dim);
  const float s = (p & 1) ? ldexpf(1.41421354f, -(p + 1) / 2) : ldexpf(1.0f, -p / 2);
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int j = threadIdx.x + nt * u;
    v[u] = j < dim ? x[j] * s : 0.0f;
  }
  __syncthreads();  // the buffer may be reused by the caller's next row
}

// Encode one row held as v[u] = channel (threadIdx.x + blockDim.x * u), u < CPT, and store it at `row`.
// All threads of the block must call this (block-wide reduction for the fp8 scale; the rotation's exchange).
template <int CPT>
__device__ void store_row(const RowOut& o, long long row, const float (&vin)[CPT], float* red, float* rot) {
  const int c = o.dim;
  const int nt = blockDim.x;
  float v[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) v[u] = vin[u];
  if (o.rotate) hadamard_row<CPT>(v, c, rot);
  if (o.format == LCA_F32) {
    float* d = (float*)o.data + row * c;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      int j = threadIdx.x + nt * u;
      if (j < c) d[j] = v[u];
    }
  } else if (o.format == LCA_BF16) {
    uint16_t* d = (uint16_t*)o.data + row * c;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      int j = threadIdx.x + nt * u;
      if (j < c) d[j] = f32_to_bf16(v[u]);
    }
  } else if (o.format == LCA_MIXED_FP8) {
    const int dm = c - o.rope;
    float am = 0.0f;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      int j = threadIdx.x + nt * u;
      if (j < dm) am = fmaxf(am, fabsf(v[u]));
    }
    am = block_max_256(am, red);
    const float s = (am == 0.0f) ? 1.0f : am / 448.0f;  // IEEE fp32 divide
    uint8_t* d = (uint8_t*)o.data + row * dm;
    uint16_t* rd = (uint16_t*)o.rope_data + row * o.rope;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      int j = threadIdx.x + nt * u;
      if (j < dm) {
        float y = fminf(fmaxf(v[u] / s, -448.0f), 448.0f);
        d[j] = fp8_encode(y);
      } else if (j < c) {
        rd[j - dm] = f32_to_bf16(v[u]);
      }
    }
    if (threadIdx.x == 0) ((float*)o.scale)[row] = s;
  } else {  // LCA_FP4: blocks of 32 consecutive channels live in 32 consecutive lanes
    uint8_t* d = (uint8_t*)o.data + row * (c / 2);
    uint8_t* sc = (uint8_t*)o.scale + row * (c / kFp4Block);
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      int j = threadIdx.x + nt * u;
      float a = (j < c) ? fabsf(v[u]) : 0.0f;
#pragma unroll
      for (int off = 1; off < kFp4Block; off <<= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
      int e = fp4_group_exp(a);
      float y = ldexpf(v[u], -e);
      uint32_t code = fp4_encode(y);
      uint32_t other = __shfl_xor(code, 1, 64);
      if (j < c) {
        if ((j & 1) == 0) d[j >> 1] = (uint8_t)(code | (other << 4));
        if ((j & (kFp4Block - 1)) == 0) sc[j / kFp4Block] = (uint8_t)(e + 127);
      }
    }
  }
}

// The codec for rows that arrive already in memory (lca_encode): one wave per row, four rows per workgroup, a row
// held as v[u] = channel (lane + 64 u), u < CPW.  Every reduction stays inside the wave, and so does the rotation:
// its stages with h < 64 pair lanes (shuffles) and those with h >= 64 pair registers u and u ^ (h / 64) of one lane,
// with the same operands in the same order as hadamard_row (x_j + x_{j+h}, x_j - x_{j+h}).  The codes are those of
// store_row.
constexpr int kEncWaves = 4;

template <int CPW>
__device__ void store_row_wave(const RowOut& o, long long row, float (&v)[CPW]) {
  const int c = o.dim, lane = threadIdx.x & 63;
  if (o.rotate) {
    const int hw = c < 64 ? c : 64;
    for (int h = 1; h < hw; h <<= 1) {
#pragma unroll
      for (int u = 0; u < CPW; ++u) {
        const float x = __shfl_xor(v[u], h, 64);
        v[u] = (lane & h) ? x - v[u] : v[u] + x;
      }
    }
#pragma unroll
    for (int s = 1; s < CPW; s <<= 1) {
      if (64 * s >= c) break;
#pragma unroll
      for (int u = 0; u < CPW; ++u) {
        if (u & s) continue;
        const float x = v[u], y = v[u | s];
        v[u] = x + y;
        v[u | s] = x - y;
      }
    }
    const int p = 31 - __clz(c);
    const float sc = (p & 1) ? ldexpf(1.41421354f, -(p + 1) / 2) : ldexpf(1.0f, -p / 2);
#pragma unroll
    for (int u = 0; u < CPW; ++u) v[u] = (lane + 64 * u < c) ? v[u] * sc : 0.0f;
  }
  if (o.format == LCA_F32) {
    float* d = (float*)o.data + row * c;
#pragma unroll
    for (int u = 0; u < CPW; ++u)
      if (lane + 64 * u < c) d[lane + 64 * u] = v[u];
  } else if (o.format == LCA_BF16) {
    uint16_t* d = (uint16_t*)o.data + row * c;
#pragma unroll
    for (int u = 0; u < CPW; ++u)
      if (lane + 64 * u < c) d[lane + 64 * u] = f32_to_bf16(v[u]);
  } else if (o.format == LCA_MIXED_FP8) {
    const int dm = c - o.rope;
    float am = 0.0f;
#pragma unroll
    for (int u = 0; u < CPW; ++u)
      if (lane + 64 * u < dm) am = fmaxf(am, fabsf(v[u]));
    am = wave_max(am);
    const float s = (am == 0.0f) ? 1.0f : am / 448.0f;  // IEEE fp32 divide
    uint8_t* d = (uint8_t*)o.data + row * dm;
    uint16_t* rd = (uint16_t*)o.rope_data + row * o.rope;
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      const int j = lane + 64 * u;
      if (j < dm) {
        const float y = fminf(fmaxf(v[u] / s, -448.0f), 448.0f);
        d[j] = fp8_encode(y);
      } else if (j < c) {
        rd[j - dm] = f32_to_bf16(v[u]);
      }
    }
    if (lane == 0) ((float*)o.scale)[row] = s;
  } else {  // LCA_FP4: blocks of 32 consecutive channels live in 32 consecutive lanes
    uint8_t* d = (uint8_t*)o.data + row * (c / 2);
    uint8_t* sc = (uint8_t*)o.scale + row * (c / kFp4Block);
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      const int j = lane + 64 * u;
      float a = (j < c) ? fabsf(v[u]) : 0.0f;
#pragma unroll
      for (int off = 1; off < kFp4Block; off <<= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
      const int e = fp4_group_exp(a);
      const uint32_t code = fp4_encode(ldexpf(v[u], -e));
      const uint32_t other = __shfl_xor(code, 1, 64);
      if (j < c) {
        if ((j & 1) == 0) d[j >> 1] = (uint8_t)(code | (other << 4));
        if ((j & (kFp4Block - 1)) == 0) sc[j / kFp4Block] = (uint8_t)(e + 127);
      }
    }
  }
}

// RPW rows per wave (short rows), every row's loads issued before the first is encoded.
template <int CPW, int RPW>
__global__ __launch_bounds__(64 * kEncWaves) void encode_rows_kernel(const float* __restrict__ src, long long rows,
                                                                      long long row0, RowOut o) {
  const long long r0 = ((long long)blockIdx.x * kEncWaves + (threadIdx.x >> 6)) * RPW;
  if (r0 >= rows) return;  // wave-uniform
  const int b = blockIdx.y, lane = threadIdx.x & 63;
  float v[RPW][CPW];
#pragma unroll
  for (int q = 0; q < RPW; ++q) {
    const float* s = src + ((long long)b * rows + min(r0 + q, rows - 1)) * o.dim;
#pragma unroll
    for (int u = 0; u < CPW; ++u) v[q][u] = (lane + 64 * u < o.dim) ? s[lane + 64 * u] : 0.0f;
  }
#pragma unroll
  for (int q = 0; q < RPW; ++q)
    if (r0 + q < rows) store_row_wave<CPW>(o, out_row(o, b, row0 + r0 + q), v[q]);
}

struct CompressArgs {
  const float *Ca, *Cb, *Za, *Zb, *Ba, *Bb, *tCb, *tZb;
  long long n, start_pos;
  const long long* seq_pos;  // nullable [B]: sequence b's start (a ragged batch)
  const int* seq_len;        // nullable [B]: sequence b's tokens among the n given
  int c, m, overlap;
  lca_epilogue epi;
};

// The entry epilogues (RMSNorm, then rotary embedding of the trailing channels at the block's first token) on a row
// held as v[u] = channel (threadIdx.x + blockDim.x * u).  All threads of the block must call this.  A channel pair
// (2i, 2i + 1) lies in lanes l and l ^ 1 of one wave (blockDim.x is a multiple of 64), so each lane takes its
// partner's value with one shuffle.
template <int CPT>
__device__ void entry_epilogue(const lca_epilogue& e, int c, long long entry, int m, float (&v)[CPT], float* red) {
  const int nt = blockDim.x;
  if (e.norm_weight) {
    float ss = 0.0f;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int j = threadIdx.x + nt * u;
      if (j < c) ss += v[u] * v[u];
    }
    ss = block_sum_256(ss, red);
    const float inv = 1.0f / sqrtf(ss / (float)c + e.norm_eps);
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int j = threadIdx.x + nt * u;
      if (j < c) v[u] = v[u] * inv * e.norm_weight[j];
    }
  }
  if (e.rope_dims > 0) {
    const int r0 = c - e.rope_dims;
    const double p = (double)m * (double)entry;
    const double lb = log2((double)e.rope_base);
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int j = threadIdx.x + nt * u;
      const float other = __shfl_xor(v[u], 1, 64);
      if (j >= r0 && j < c) {
        const int i = (j - r0) >> 1;
        const double ang = p * exp2(-2.0 * (double)i / (double)e.rope_dims * lb);
        double sd, cd;
        sincos(ang, &sd, &cd);
        const float sn = (float)sd, cs = (float)cd;
        v[u] = ((j - r0) & 1) ? other * sn + v[u] * cs : v[u] * cs - other * sn;
      }
    }
  }
}

__device__ __forceinline__ void softmax_acc(float l, float x, float& mx, float& den, float& num) {
  float nm = fmaxf(mx, l);
  float sc = __expf(mx - nm);
  float e = __expf(l - nm);
  den = den * sc + e;
  num = num * sc + e * x;
  mx = nm;
}

template <int CPT>
__global__ __launch_bounds__(kRowThreads) void compress_kernel(CompressArgs a, RowOut o) {
  __shared__ float red[kRowThreads / 64];
  __shared__ float rot[2 * kRotMaxDim];
  const long long i = blockIdx.x;  // local entry index
  const int b = blockIdx.y;
  const int c = a.c, m = a.m;
  const long long n_b = a.seq_len ? a.seq_len[b] : a.n;  // this sequence's tokens (rows [0, n_b) of its slice)
  if ((long long)m * i >= n_b) return;                      // block-uniform: no token of this sequence's entry i
  const long long gblock = seq_position(a.seq_pos, a.start_pos, b) / m + i;
  float mx[CPT], den[CPT], num[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    mx[u] = -INFINITY;
    den[u] = 0.0f;
    num[u] = 0.0f;
  }
  const long long base = (long long)b * a.n;
  // stream a: block i's own tokens; stream b: block i-1's tokens (absent for the first block of the sequence).
  // Candidates are taken eight at a time with all their loads issued before the softmax updates (a decode append
  // has at most 2m = 8 of them: one round of loads); loads past the last candidate or channel repeat a valid
  // address and are masked, so no branch separates them.
  const long long pa0 = (long long)m * i;
  const int na = (int)((n_b - pa0) < m ? (n_b - pa0) : m);
  const int nbk = (a.overlap && gblock >= 1) ? m : 0;
  const int ncand = na + nbk;
  constexpr int kBatch = 8;
  for (int r0 = 0; r0 < ncand; r0 += kBatch) {
    float zl[kBatch][CPT], cv[kBatch][CPT];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int rr = min(r0 + q, ncand - 1);
      const bool from_a = rr < na;
      const int r = from_a ? rr : rr - na;
      const float *zr, *cr, *br;
      if (from_a) {
        zr = a.Za + (base + pa0 + r) * c;
        cr = a.Ca + (base + pa0 + r) * c;
        br = a.Ba + (long long)r * c;
      } else if (i >= 1) {
        zr = a.Zb + (base + pa0 - m + r) * c;
        cr = a.Cb + (base + pa0 - m + r) * c;
        br = a.Bb + (long long)r * c;
      } else {
        zr = a.tZb + ((long long)b * m + r) * c;
        cr = a.tCb + ((long long)b * m + r) * c;
        br = a.Bb + (long long)r * c;
      }
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int j = min((int)threadIdx.x + (int)blockDim.x * u, c - 1);
        zl[q][u] = zr[j] + br[j];
        cv[q][u] = cr[j];
      }
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      if (r0 + q < ncand) {
#pragma unroll
        for (int u = 0; u < CPT; ++u) softmax_acc(zl[q][u], cv[q][u], mx[u], den[u], num[u]);
      }
    }
  }
  float v[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) v[u] = num[u] / den[u];
  if (a.epi.norm_weight || a.epi.rope_dims > 0) entry_epilogue<CPT>(a.epi, c, gblock, m, v, red);
  store_row<CPT>(o, out_row(o, b, gblock), v, red, rot);
}

static RowOut row_out(const lca_tensor& t) {
  return RowOut{t.format, t.dim, t.rope_dims, (t.flags & LCA_ROTATE_HADAMARD) ? 1 : 0, t.cap, t.data, t.rope,
                t.scale, t.block_table, t.block_rows};
}

static int threads_for(int c) {
  int nt = ((c + 63) / 64) * 64;
  return nt > kRowThreads ? kRowThreads : nt;
}

hipError_t launch_encode(const float* src, int B, long long rows, long long row0, const lca_tensor& dst,
                         hipStream_t st) {
  const RowOut o = row_out(dst);
  const int cpw = (dst.dim + 63) / 64;  // dim <= 1024 (checked by the caller)
  const int rpw = cpw <= 2 ? 4 : cpw <= 4 ? 2 : 1;  // rows per wave: about 2 KB of each wave's loads in flight
  const long long per_wg = (long long)kEncWaves * rpw;
  const dim3 grid((unsigned)((rows + per_wg - 1) / per_wg), (unsigned)B), block(64 * kEncWaves);
  clear_stale_error();
  if (cpw <= 1)
    hipLaunchKernelGGL((encode_rows_kernel<1, 4>), grid, block, 0, st, src, rows, row0, o);
  else if (cpw <= 2)
    hipLaunchKernelGGL((encode_rows_kernel<2, 4>), grid, block, 0, st, src, rows, row0, o);
  else if (cpw <= 4)
    hipLaunchKernelGGL((encode_rows_kernel<4, 2>), grid, block, 0, st, src, rows, row0, o);
  else if (cpw <= 8)
    hipLaunchKernelGGL((encode_rows_kernel<8, 1>), grid, block, 0, st, src, rows, row0, o);
  else
    hipLaunchKernelGGL((encode_rows_kernel<16, 1>), grid, block, 0, st, src, rows, row0, o);
  return hipGetLastError();
}

hipError_t launch_compress(const float* Ca, const float* Cb, const float* Za, const float* Zb, const float* Ba,
                           const float* Bb, const float* tCb, const float* tZb, int B, long long n, int c, int m,
                           int overlap, long long start_pos, const long long* seq_pos, const int* seq_len,
                           const lca_epilogue& epi, const lca_tensor& out, hipStream_t st) {
  CompressArgs a{Ca, Cb, Za, Zb, Ba, Bb, tCb, tZb, n, start_pos, seq_pos, seq_len, c, m, overlap, epi};
  RowOut o = row_out(out);
  int nt = threads_for(c);
  int cpt = (c + nt - 1) / nt;
  long long nb = (n + m - 1) / m;
  dim3 grid((unsigned)nb, (unsigned)B);
  clear_stale_error();
  if (cpt <= 1)
    hipLaunchKernelGGL(compress_kernel<1>, grid, dim3(nt), 0, st, a, o);
  else if (cpt <= 2)
    hipLaunchKernelGGL(compress_kernel<2>, grid, dim3(nt), 0, st, a, o);
  else
    hipLaunchKernelGGL(compress_kernel<4>, grid, dim3(nt), 0, st, a, o);
  return hipGetLastError();
}

}  // namespace lca
