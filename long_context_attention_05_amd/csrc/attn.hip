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
  long long w0;    // first window position
  long long raw0;  // position of the sequence's raw row 0
  int nw;          // window entries
  int nc;          // compressed list length
};

// The list of query row r of sequence b: its position is the sequence's (ragged batch) or the call's, plus r.
__device__ __forceinline__ RowList row_list(const AttnArgs& a, int b, int r) {
  const long long pos = seq_position(a.seq_pos, a.q_start, b);
  const long long t = pos + r;
  RowList L;
  L.raw0 = a.raw_start + (pos - a.q_start);
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

// Storage row of list position p of query row r of sequence b -- window positions in the raw tensor, the rest in the
// compressed one (through its block table when it is paged) -- or -1 where the position is padding.  Storage rows of
// both tensors are below 2^31.
__device__ __forceinline__ int list_row(const AttnArgs& a, const RowList& L, int b, int r, int p) {
  if (p < L.nw) return (int)((long long)b * a.raw.cap + (L.w0 + p - L.raw0));
  int j = p - L.nw;
  if (j >= L.nc) return -1;
  int e;
  if (a.hca_m > 0) {
    e = j;
  } else {
    e = a.idx[((long long)b * a.Sq + r) * a.k + j];
    if (e < 0 || e >= a.N) return -1;
  }
  return (int)tensor_row(a.comp, b, e);
}

// Rows held by a tensor's arrays: the pool of a paged tensor, B * cap of a dense one.
__host__ __device__ __forceinline__ long long tensor_storage_rows(const lca_tensor& t, int B) {
  return t.block_table ? t.pool_rows : (long long)B * t.cap;
}

// The running softmax max only moves when a logit exceeds it by more than kRescaleSlack (e^8 keeps every weight and
// sum far inside fp32, and bf16 keeps 8 significant bits at any scale), so accumulators are rescaled a few times per
// row instead of on every tile.
constexpr float kRescaleSlack = 8.0f;

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;

// Four OCP e4m3 codes -> four bf16 (exact), via the hardware fp8 -> f32 conversion.
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t w) {
  const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  uint2 r;
  r.x = (__float_as_uint(lo[0]) >> 16) | (__float_as_uint(lo[1]) & 0xFFFF0000u);
  r.y = (__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xFFFF0000u);
  return r;
}

// Writes a prefill workgroup's result for head `head`: lane (head, grp) holds o^T[channel 16 dt + 4 grp + x][head]
// in acc_o[dt][x].  A single split normalises with the sink in place; otherwise (max, sum, o) go to the partials.
__device__ __forceinline__ void pf_finish(const AttnArgs& a, const f32x4_t (&acc_o)[32], float m_run, float l_run,
                                          int b, int r, int split, int head, int grp) {
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
        w2.x = pack_bf16x2(acc_o[dt][0] * f, acc_o[dt][1] * f);
        w2.y = pack_bf16x2(acc_o[dt][2] * f, acc_o[dt][3] * f);
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
// MFMA kernel for many query rows (prefill chunks): H = 64, D = 512, q bf16, KV bf16 or mixed fp8/bf16
// ------------------------------------------------------------------------------------------------
// One workgroup per (query row, slice of its list) with all 64 heads, wave w holding heads [16 w, 16 w + 16).  The
// rows of the slice's list positions are resolved into LDS first; then 32-entry tiles are gathered (all 256 threads,
// 128 contiguous bytes each) into registers one tile ahead, written row-major into a double-buffered LDS tile (fp8
// widened to bf16) and scored with the same MFMA layouts as the head-group kernel: S^T = K Q^T with A = the tile
// rows (ds_read_b128) and B = the wave's queries in registers, then O^T += V^T P^T with A = V^T from
// ds_read_b64_tr_b16 of the row-major tile.  One barrier per tile.
constexpr int kPfTE = 32;                        // entries per tile
constexpr int kPfRow = 520;                      // bf16 per LDS tile row (1040 bytes)
constexpr int kPfTileBytes = kPfTE * kPfRow * 2;  // 33280
constexpr int kAttnThreads = 256;
constexpr size_t kPfScaleOff = (size_t)2 * kPfTileBytes;      // [2][32] entry scales
constexpr size_t kPfValidOff = kPfScaleOff + 2 * kPfTE * 4;    // [2] tile validity masks
constexpr size_t kPfTableOff = kPfValidOff + 2 * 4 + 8;
constexpr size_t kMfmaLds = kPfTableOff + (size_t)kHgSplitMax * 4;

template <int FMT>
__global__ __launch_bounds__(kAttnThreads) void attn_mfma_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t pf_lds[];
  float* scale_s = (float*)(pf_lds + kPfScaleOff);
  uint32_t* valid_s = (uint32_t*)(pf_lds + kPfValidOff);
  int* rows_s = (int*)(pf_lds + kPfTableOff);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hl = lane & 15, grp = lane >> 4;
  const int split = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const RowList L = row_list(a, b, r);
  const int total = L.nw + L.nc;
  const int p_begin = split * a.split_len;
  const int npos = max(min(a.split_len, total - p_begin), 0);
  const int head = 16 * wave + hl;

  for (int i = threadIdx.x; i < npos; i += blockDim.x) {
    const int p = p_begin + i;
    const int row = list_row(a, L, b, r, p);
    rows_s[i] = row;
  }
  // Q^T B operand for 16 K-steps of 32 channels: lane holds q[head][32 s + 8 grp .. + 7]
  bf16x8_t qreg[16];
  {
    const uint8_t* qp = (const uint8_t*)a.q + ((((long long)b * a.Sq + r) * 64 + head) * 512 + 8 * grp) * 2;
#pragma unroll
    for (int s = 0; s < 16; ++s) qreg[s] = __builtin_bit_cast(bf16x8_t, *(gbl_u32x4_t*)(qp + 64 * s));
  }
  __syncthreads();

  // gather: thread (ge, gc) moves channels [64 gc, 64 gc + 64) of tile entry ge
  const int ge = threadIdx.x & 31, gc = threadIdx.x >> 5;
  u32x4_t gv[8];
  float gsc = 1.0f;
  bool gok = false;
  auto gather = [&](int i0) {
    const int i = min(i0 + ge, npos - 1);
    const int row = rows_s[i];
    gok = i0 + ge < npos && row >= 0;
    const bool from_raw = p_begin + i < L.nw;
    const lca_tensor& src = from_raw ? a.raw : a.comp;
    const long long rr = row >= 0 ? row : 0;
    if constexpr (FMT == LCA_BF16) {
      const uint8_t* gp = (const uint8_t*)src.data + rr * 1024 + 128 * gc;
#pragma unroll
      for (int x = 0; x < 8; ++x) gv[x] = *(gbl_u32x4_t*)(gp + 16 * x);
    } else {
      if (gc < 7) {
        const uint8_t* gp = (const uint8_t*)src.data + rr * 448 + 64 * gc;
#pragma unroll
        for (int x = 0; x < 4; ++x) gv[x] = *(gbl_u32x4_t*)(gp + 16 * x);
      } else {
        const uint8_t* gp = (const uint8_t*)src.rope + rr * 128;
#pragma unroll
        for (int x = 0; x < 8; ++x) gv[x] = *(gbl_u32x4_t*)(gp + 16 * x);
      }
      gsc = ((const float*)src.scale)[rr];
    }
  };
  auto stage = [&](int buf) {
    uint8_t* kp = pf_lds + buf * kPfTileBytes + ge * (kPfRow * 2) + 128 * gc;
    if constexpr (FMT == LCA_BF16) {
#pragma unroll
      for (int x = 0; x < 8; ++x) *(u32x4_t*)(kp + 16 * x) = gv[x];
    } else {
      if (gc < 7) {  // 64 fp8 codes -> 64 bf16 (exact)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const uint2 a0 = fp8x4_to_bf16x4(gv[x].x), a1 = fp8x4_to_bf16x4(gv[x].y);
          const uint2 a2 = fp8x4_to_bf16x4(gv[x].z), a3 = fp8x4_to_bf16x4(gv[x].w);
          *(u32x4_t*)(kp + 32 * x) = u32x4_t{a0.x, a0.y, a1.x, a1.y};
          *(u32x4_t*)(kp + 32 * x + 16) = u32x4_t{a2.x, a2.y, a3.x, a3.y};
        }
      } else {
#pragma unroll
        for (int x = 0; x < 8; ++x) *(u32x4_t*)(kp + 16 * x) = gv[x];
      }
      if (gc == 0) scale_s[buf * kPfTE + ge] = gsc;
    }
    const uint64_t vb = __ballot(gok);
    if (threadIdx.x == 0) valid_s[buf] = (uint32_t)vb;  // lanes 0..31 are the tile's entries (gc = 0)
  };

  f32x4_t acc_o[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) acc_o[dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;

  const int ntiles = (npos + kPfTE - 1) / kPfTE;
  if (ntiles > 0) {
    gather(0);
    stage(0);
  }
  __syncthreads();
  for (int tt = 0; tt < ntiles; ++tt) {
    const int cur = tt & 1;
    if (tt + 1 < ntiles) gather(kPfTE * (tt + 1));  // block-uniform: the next tile is in flight
    const uint16_t* kt = (const uint16_t*)(pf_lds + cur * kPfTileBytes);
    const uint32_t valid = valid_s[cur];

    // S^T = K Q^T for the two 16-entry halves
    float lg[2][4], esc[2][4];
#pragma unroll
    for (int et = 0; et < 2; ++et) {
      f32x4_t am = {0.0f, 0.0f, 0.0f, 0.0f}, ar = {0.0f, 0.0f, 0.0f, 0.0f};
      const uint16_t* kp = kt + (16 * et + hl) * kPfRow + 8 * grp;
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(kp + 32 * s));
        if (FMT == LCA_MIXED_FP8 && s >= 14)
          ar = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qreg[s], ar, 0, 0, 0);
        else
          am = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qreg[s], am, 0, 0, 0);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int e = 16 * et + 4 * grp + x;
        esc[et][x] = (FMT == LCA_MIXED_FP8) ? scale_s[cur * kPfTE + e] : 1.0f;
        const float l = (FMT == LCA_MIXED_FP8) ? a.scale * (esc[et][x] * am[x] + ar[x]) : a.scale * am[x];
        lg[et][x] = ((valid >> e) & 1u) ? l : -INFINITY;
      }
    }
    // online softmax for head `head` (lanes hl, hl + 16, hl + 32, hl + 48 hold its 32 logits); the reference max
    // only moves by more than kRescaleSlack, as in the decode kernels
    float mt = fmaxf(fmaxf(fmaxf(lg[0][0], lg[0][1]), fmaxf(lg[0][2], lg[0][3])),
                     fmaxf(fmaxf(lg[1][0], lg[1][1]), fmaxf(lg[1][2], lg[1][3])));
    mt = xor32_max(xor16_max(mt));
    const float m_new = (mt > m_run + kRescaleSlack) ? mt : m_run;
    const float alpha = (m_new == m_run) ? 1.0f : __expf(m_run - m_new);
    float pv[2][4], psum = 0.0f;
#pragma unroll
    for (int et = 0; et < 2; ++et)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        pv[et][x] = (lg[et][x] == -INFINITY) ? 0.0f : __expf(lg[et][x] - m_new);
        psum += pv[et][x];
      }
    psum = xor32_sum(xor16_sum(psum));
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) acc_o[dt] *= alpha;
    }

    // O^T += V^T P^T, 16 entries per product
#pragma unroll
    for (int et = 0; et < 2; ++et) {
      s16x4_t pb, pbs;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        pb[x] = (short)f32_to_bf16(pv[et][x]);
        pbs[x] = (FMT == LCA_MIXED_FP8) ? (short)f32_to_bf16(pv[et][x] * esc[et][x]) : pb[x];
      }
      const uint16_t* vp = kt + (16 * et + 4 * grp + (hl >> 2)) * kPfRow + 4 * (hl & 3);
#pragma unroll
      for (int d0 = 0; d0 < 32; d0 += 8) {
        s16x4_t av[8];
#pragma unroll
        for (int d = 0; d < 8; ++d) av[d] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vp + 16 * (d0 + d)));
#pragma unroll
        for (int d = 0; d < 8; ++d)
          acc_o[d0 + d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
              av[d], (FMT == LCA_MIXED_FP8 && d0 + d < 28) ? pbs : pb, acc_o[d0 + d], 0, 0, 0);
      }
    }
    if (tt + 1 < ntiles) stage(cur ^ 1);
    __syncthreads();
  }

  pf_finish(a, acc_o, m_run, l_run, b, r, split, head, grp);
}

// ------------------------------------------------------------------------------------------------
// LDS tile ring of the bf16 prefill kernel (attn_pfs_kernel below)
// ------------------------------------------------------------------------------------------------
// The tiles travel from memory straight into LDS (buffer_load ... lds: one instruction moves one 1 KB entry row, 16
// bytes per lane), so no registers hold data in flight.  Each ring slot is its own LDS variable and the tile loop is
// unrolled over the slots, so the compiler can tell that a slot's reads do not alias loads still landing in other
// slots; the waits for a slot are explicit counts.
constexpr int kPdRowB = 1024;                    // LDS bytes per tile row
constexpr int kPdTileB = kPfTE * kPdRowB;        // 32768
__shared__ __attribute__((aligned(16))) uint8_t pd_slot0[kPdTileB];
__shared__ __attribute__((aligned(16))) uint8_t pd_slot1[kPdTileB];
__shared__ __attribute__((aligned(16))) uint8_t pd_slot2[kPdTileB];
__shared__ __attribute__((aligned(16))) uint8_t pd_slot3[kPdTileB];
__shared__ int pd_rows[kHgSplitMax];
__shared__ float pd_ml[64][2];

template <int S>
__device__ __forceinline__ uint8_t* pd_slot() {
  if constexpr (S == 0) return pd_slot0;
  else if constexpr (S == 1) return pd_slot1;
  else if constexpr (S == 2) return pd_slot2;
  else return pd_slot3;
}

typedef __attribute__((address_space(3))) void lds_void_t;
// Buffer descriptor word 3 for raw untyped loads (32-bit data format, no swizzle, no index stride).
constexpr int kBufRsrcWord3 = 0x00020000;
// s_waitcnt immediates (vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8])
constexpr int kWaitVm8 = (0xF << 8) | (7 << 4) | 8;  // vmcnt(8)
constexpr int kWaitVm0 = (0xF << 8) | (7 << 4);      // vmcnt(0)
constexpr int kWaitLgkm0 = (3 << 14) | (7 << 4) | 0xF;  // lgkmcnt(0)

// Workgroup barrier for LDS only: the compiler keeps memory accesses on their side of it and no load in flight is
// waited for (the caller has already waited for what it needs).
__device__ __forceinline__ void pd_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // this wave's LDS writes are complete before others read them
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------------------------------------
// bf16 attention for many query rows (prefill; also dense HCA rows split into slices), score and value waves:
// H = 64, D = 512
// ------------------------------------------------------------------------------------------------
// Eight waves in two roles, one of each per SIMD, a tile apart:
//   score waves 0-3: wave g scores head group g (heads 16 g .. 16 g + 15) over all 512 channels,
//                    S^T = K Q^T (A = the tile's K read from LDS, B = the group's queries held in registers),
//                    runs the online softmax of its 16 heads and publishes P^T and the rescale factors;
//   value waves 4-7: wave 4 + v accumulates O^T for channels 128 v .. 128 v + 127 and all 64 heads,
//                    O^T += V^T P^T (A = V^T by transposing LDS reads, B = the published P^T), and moves the
//                    tiles into the LDS ring.
// In step tt the score waves work on tile tt and the value waves on tile tt - 1, so each SIMD overlaps one wave's
// LDS reads and softmax arithmetic with the other's MFMAs; one barrier per step hands P^T(tt) over and
// retires tile tt - 1.  The ring holds four 32-entry tiles (tile tt in slot tt % 4; tiles tt + 1 and tt + 2 in
// flight during step tt).  Entry rows sit 1024 bytes apart with 16-byte chunk c of tile row r stored at chunk
// c ^ (r % 16), which keeps the K reads (16 rows x 4 chunks per instruction) free of bank conflicts (a padded
// 1040-byte pitch halves their rate); the transposing V reads run at the same rate under either layout.  Logits are
// kept in base 2 (scale * log2(e) folded into the one multiply).  Split partials are written in bf16 when the
// launcher asks for them (part_bf16).
constexpr int kPsThreads = 512;
constexpr float kLog2e = 1.4426950408889634f;
__shared__ __attribute__((aligned(16))) u32x4_t ps_p[2][4][64];    // [tile parity][head group][lane]: P^T operands
__shared__ __attribute__((aligned(16))) float ps_alpha[2][16][4];  // [tile parity][head % 16][head / 16]

__global__ __launch_bounds__(kPsThreads) void attn_pfs_kernel(AttnArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hl = lane & 15, grp = lane >> 4;
  const bool scorer = wave < 4;    // wave-uniform role
  const int vw = wave & 3;         // head group (score waves) or channel quarter (value waves)
  const int split = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const RowList L = row_list(a, b, r);
  const int total = L.nw + L.nc;
  const int p_begin = split * a.split_len;
  const int npos = max(min(a.split_len, total - p_begin), 0);
  const int qhead = 16 * vw + hl;  // the head a score lane works on

  // score waves: qreg[s] = channels 32 s + 8 grp .. + 7 of head qhead (loaded first, so that they land while the
  // row table is built)
  bf16x8_t qreg[16];
  {
    const uint8_t* qp =
        (const uint8_t*)a.q + ((((long long)b * a.Sq + r) * 64 + (scorer ? qhead : hl)) * 512 + 8 * grp) * 2;
    if (scorer) {
#pragma unroll
      for (int s = 0; s < 16; ++s) qreg[s] = __builtin_bit_cast(bf16x8_t, *(gbl_u32x4_t*)(qp + 64 * s));
    }
  }
  for (int i = threadIdx.x; i < npos; i += blockDim.x) {
    const int p = p_begin + i;
    const int row = list_row(a, L, b, r, p);
    pd_rows[i] = row;
  }
  // value waves: acc[hg][dt] holds o^T[channel 128 v + 16 dt + 4 grp + x][head 16 hg + hl] in lane (hl, grp)
  f32x4_t acc[4][8];
  float m_run = -INFINITY, l_run = 0.0f;  // score waves: of head qhead, base 2
  const float c2 = a.scale * kLog2e;
  __syncthreads();
  // The two roles run separate loops with the same barriers (one per step), so that the score waves' queries and
  // the value waves' accumulators never share registers.
  if (scorer) {
    // an empty asm re-defines each query register, so that the tile loop does not see registers defined by memory
    // loads from before it
#pragma unroll
    for (int s = 0; s < 16; ++s) asm volatile("" : "+v"(qreg[s]));
  } else {
#pragma unroll
    for (int hg = 0; hg < 4; ++hg)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc[hg][dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  const int ntiles = (npos + kPfTE - 1) / kPfTE;
  if (ntiles > 0) {  // block-uniform
    // descriptors over the whole tensors (the table holds storage rows; the launcher checks both stay under 2 GiB)
    const __amdgpu_buffer_rsrc_t raw_rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.raw.data, 0, (int)(tensor_storage_rows(a.raw, a.B) * 1024), kBufRsrcWord3);
    const __amdgpu_buffer_rsrc_t comp_rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.comp.data, 0, (int)(tensor_storage_rows(a.comp, a.B) * 1024), kBufRsrcWord3);
    // Value wave v moves entries 8 v .. 8 v + 7 of tile tt into ring slot S (lane j takes chunk j ^ (tile row % 16)
    // of the entry into LDS chunk j); positions past the slice repeat its last entry, so every tile issues the same
    // number of loads and the wait counts stay fixed.
    auto issue = [&](auto SC, int tt) {
      constexpr int S = decltype(SC)::value;
      const int ii = min(kPfTE * tt + 8 * vw + (lane & 7), npos - 1);
      const int myrow = pd_rows[ii];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = __builtin_amdgcn_readfirstlane(min(kPfTE * tt + 8 * vw + q, npos - 1));
        const int row = __builtin_amdgcn_readlane(myrow, q);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(p_begin + i < L.nw ? raw_rs : comp_rs,
                                                 (lds_void_t*)(pd_slot<S>() + (8 * vw + q) * kPdRowB), 16,
                                                 16 * (lane ^ ((8 * vw + q) & 15)), max(row, 0) * 1024, 0, 0);
      }
    };
    // Score waves: S^T of tile tt (slot S) for head group vw over all channels, then the softmax; publishes P^T and
    // the rescale factor in buffer tt & 1.  K batch j: K-steps 2 j and 2 j + 1 of both 16-entry halves (four reads,
    // three batches in flight), four independent accumulator chains.
    auto score = [&](auto SC, int tt) {
      constexpr int S = decltype(SC)::value;
      const int iv = kPfTE * tt + (lane & 31);
      const uint32_t valid = (uint32_t)__ballot(iv < npos && pd_rows[min(iv, npos - 1)] >= 0);
      // K-step kk reads chunk 4 kk + grp of rows hl and 16 + hl, stored at chunk (4 kk + grp) ^ hl
      const uint8_t* kp = pd_slot<S>() + hl * kPdRowB;
      const int koff = 16 * (grp ^ (hl & 3)) + 64 * (hl >> 2);
      u32x4_t kb[3][4];
      auto kload = [&](u32x4_t (&dst)[4], int j) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int kk = 2 * j + u;
          const uint8_t* kq = kp + (koff ^ (64 * (kk & 3))) + 256 * (kk >> 2);
          dst[2 * u] = *(const u32x4_t*)kq;
          dst[2 * u + 1] = *(const u32x4_t*)(kq + 16 * kPdRowB);
        }
      };
      f32x4_t am[2][2];
#pragma unroll
      for (int et = 0; et < 2; ++et) am[et][0] = am[et][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      kload(kb[0], 0);
      kload(kb[1], 1);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j + 2 < 8) kload(kb[(j + 2) % 3], j + 2);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int et = 0; et < 2; ++et)
            am[et][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kb[j % 3][2 * u + et]),
                                                                qreg[2 * j + u], am[et][u], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      // softmax: lanes hl, hl + 16, hl + 32, hl + 48 hold head qhead's 32 logits; the reference max only moves by
      // more than kRescaleSlack
      float lg[2][4];
#pragma unroll
      for (int et = 0; et < 2; ++et) {
        const f32x4_t s = am[et][0] + am[et][1];
#pragma unroll
        for (int x = 0; x < 4; ++x) lg[et][x] = s[x] * c2;
      }
      if (valid != 0xFFFFFFFFu) {  // block-uniform: the slice's last tile, or rows without an entry
#pragma unroll
        for (int et = 0; et < 2; ++et)
#pragma unroll
          for (int x = 0; x < 4; ++x)
            if (!((valid >> (16 * et + 4 * grp + x)) & 1u)) lg[et][x] = -INFINITY;
      }
      float mt = fmaxf(fmaxf(fmaxf(lg[0][0], lg[0][1]), fmaxf(lg[0][2], lg[0][3])),
                       fmaxf(fmaxf(lg[1][0], lg[1][1]), fmaxf(lg[1][2], lg[1][3])));
      mt = xor32_max(xor16_max(mt));
      const float m_new = (mt > m_run + kRescaleSlack * kLog2e) ? mt : m_run;
      const float alpha = (m_new == m_run) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      const float m_sub = (m_new == -INFINITY) ? 0.0f : m_new;  // no entry yet: every weight is exp2(-inf) = 0
      float psum = 0.0f;
      u32x4_t pw;
#pragma unroll
      for (int et = 0; et < 2; ++et)
#pragma unroll
        for (int x = 0; x < 4; x += 2) {
          const float p0 = __builtin_amdgcn_exp2f(lg[et][x] - m_sub);
          const float p1 = __builtin_amdgcn_exp2f(lg[et][x + 1] - m_sub);
          psum += p0 + p1;
          pw[2 * et + x / 2] = pack_bf16x2(p0, p1);
        }
      psum = xor32_sum(xor16_sum(psum));
      l_run = l_run * alpha + psum;
      m_run = m_new;
      ps_p[tt & 1][vw][lane] = pw;
      ps_alpha[tt & 1][hl][vw] = alpha;  // the four lanes of a head store the same value
    };
    // Value waves: bring the accumulators to the reference maxima of tile tp (rare: only when some head's reference
    // max moved), then O^T += V^T P^T of tile tp (slot S) for the wave's 128 channels and all 64 heads.
    auto value = [&](auto SC, int tp) {
      constexpr int S = decltype(SC)::value;
      const f32x4_t al = *(const f32x4_t*)&ps_alpha[tp & 1][hl][0];
      if (__ballot(al[0] != 1.0f || al[1] != 1.0f || al[2] != 1.0f || al[3] != 1.0f)) {
#pragma unroll
        for (int hg = 0; hg < 4; ++hg)
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) acc[hg][dt] *= al[hg];
      }
      bf16x8_t pb[4];
#pragma unroll
      for (int hg = 0; hg < 4; ++hg) pb[hg] = __builtin_bit_cast(bf16x8_t, ps_p[tp & 1][hg][lane]);
      // lane 4 a + e of group g reads V[4 g + v][128 w + 16 dt + 4 a + e] (first half) and V[16 + 4 g + v][..]:
      // lane (hl, grp) addresses row R = 4 grp + hl / 4 (and 16 + R), bytes 8 (hl % 4) + 32 dt + 256 w, whose
      // 16-byte chunk C sits at chunk C ^ R
      const int vrow = 4 * grp + (hl >> 2);
      const int vchunk = ((((hl & 3) >> 1) + 16 * vw) ^ vrow) * 16;  // of dt = 0; dt flips chunk bits 1-3
      const uint8_t* vp = pd_slot<S>() + vrow * kPdRowB + 8 * (hl & 1);
      // V batch j: channel tiles 2 j and 2 j + 1 (four reads), the next batch in flight
      s16x4_t vb[2][4];
      auto vload = [&](s16x4_t (&dst)[4], int j) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const uint8_t* vq = vp + (vchunk ^ (32 * (2 * j + u)));
          dst[2 * u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)vq);
          dst[2 * u + 1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vq + 16 * kPdRowB));
        }
      };
      vload(vb[0], 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j + 1 < 4) vload(vb[(j + 1) & 1], j + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bf16x8_t av = __builtin_bit_cast(
              bf16x8_t, __builtin_shufflevector(vb[j & 1][2 * u], vb[j & 1][2 * u + 1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int hg = 0; hg < 4; ++hg)
            acc[hg][2 * j + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[hg], acc[hg][2 * j + u], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    // Step tt (tt >= 1): score tile tt (slot SQ) | value tile tt - 1 (slot SP) and wait for this wave's loads of
    // tile tt + 1; barrier (tile tt + 1 has landed, P^T(tt) is published, tile tt - 1 is retired); start tile
    // tt + 3 in the slot tile tt - 1 used.  The steps run in whole groups of four: up to three tiles past the slice
    // take part with no valid position (P = 0), so that the loop has one shape, every step is entered only from
    // the step before it (the wait counts hold on every path), and the last tile sits in slot 0.
    const int nsteps = 1 + ((ntiles - 1 + 3) & ~3);
    if (scorer) {
      auto sstep = [&](auto SQ, int tt) {
        score(SQ, tt);
        pd_barrier();
      };
      pd_barrier();  // tile 0 has landed
      sstep(S0{}, 0);
      for (int tt = 1; tt < nsteps; tt += 4) {
        sstep(S1{}, tt);
        sstep(S2{}, tt + 1);
        sstep(S3{}, tt + 2);
        sstep(S0{}, tt + 3);
      }
    } else {
      auto vstep = [&](auto SP, int tt) {
        value(SP, tt - 1);
        __builtin_amdgcn_s_waitcnt(kWaitVm8);
        pd_barrier();
        issue(SP, tt + 3);
      };
      issue(S0{}, 0);
      issue(S1{}, 1);
      issue(S2{}, 2);
      __builtin_amdgcn_s_waitcnt((1 << 14) | (0xF << 8) | (7 << 4));  // vmcnt(16): tile 0 has landed
      pd_barrier();
      __builtin_amdgcn_s_waitcnt(kWaitVm8);  // step 0: tile 1 has landed
      pd_barrier();
      issue(S3{}, 3);
      for (int tt = 1; tt < nsteps; tt += 4) {
        vstep(S0{}, tt);
        vstep(S1{}, tt + 1);
        vstep(S2{}, tt + 2);
        vstep(S3{}, tt + 3);
      }
      value(S0{}, nsteps - 1);  // the last tile ((nsteps - 1) % 4 == 0)
      __builtin_amdgcn_s_waitcnt(kWaitVm0);  // the trailing ring loads land before the workgroup can end
    }
  }

  // finish: (max, sum) of every head through LDS (back to natural-log units); each value lane writes 4 heads x 8 x
  // 4 channels
  const long long item = ((long long)b * a.Sq + r) * a.n_splits + split;
  if (scorer && grp == 0) {
    pd_ml[qhead][0] = m_run * (1.0f / kLog2e);
    pd_ml[qhead][1] = l_run;
  }
  __syncthreads();
  if (scorer) return;
  // bf16 rows (the output of a whole row, or a split's unnormalised partial sums, which the merge rescales in
  // fp32) go through the wave's own slot of the idle ring (every load has landed and every wave is past its last
  // tile), so that each store writes whole 256-byte head rows, 1 KB per instruction, instead of 32-byte pieces
  constexpr int kPr = 272;  // LDS bytes per head row: 256 + 16, which spreads the lanes' 8-byte writes over banks
  uint8_t* stage = vw == 0 ? pd_slot0 : vw == 1 ? pd_slot1 : vw == 2 ? pd_slot2 : pd_slot3;
  auto store_rows = [&](uint8_t* dst) {  // dst: head 0 of the wave's 128 channels; head rows 1 KB apart
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int head = 4 * i + (lane >> 4);
      __builtin_nontemporal_store(*(const u32x4_t*)(stage + head * kPr + 16 * (lane & 15)),
                                  (u32x4_t*)(dst + (long long)head * 1024 + 16 * (lane & 15)));
    }
  };
  if (a.n_splits == 1) {
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) {
      const int head = 16 * hg + hl;
      const float m = pd_ml[head][0], l = pd_ml[head][1];
      const float z = a.sink[head];
      const float M = fmaxf(m, z);
      float den, f;
      if (M == -INFINITY) {
        den = 0.0f;
        f = 0.0f;
      } else {
        den = ((z == -INFINITY) ? 0.0f : __expf(z - M)) + l * ((m == -INFINITY) ? 0.0f : __expf(m - M));
        f = (m == -INFINITY) ? 0.0f : __expf(m - M) / den;
      }
      const long long ob = (((long long)b * a.Sq + r) * 64 + head) * 512 + 128 * vw + 4 * grp;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4_t o = acc[hg][dt] * f;
        if (a.out_format == LCA_F32) {
          *(float4*)((float*)a.out + ob + 16 * dt) = make_float4(o[0], o[1], o[2], o[3]);
        } else {
          uint2 w2;
          w2.x = pack_bf16x2(o[0], o[1]);
          w2.y = pack_bf16x2(o[2], o[3]);
          *(uint2*)(stage + head * kPr + 2 * (16 * dt + 4 * grp)) = w2;
        }
      }
      if (a.lse && vw == 0 && grp == 0)
        a.lse[((long long)b * a.Sq + r) * 64 + head] = (M == -INFINITY) ? -INFINITY : M + __logf(den);
    }
    if (a.out_format != LCA_F32)
      store_rows((uint8_t*)a.out + ((((long long)b * a.Sq + r) * 64) * 512 + 128 * vw) * 2);
    return;
  }
  if (vw == 0 && grp == 0) {
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) {
      const int head = 16 * hg + hl;
      a.part_ml[(item * 64 + head) * 2 + 0] = pd_ml[head][0];
      a.part_ml[(item * 64 + head) * 2 + 1] = pd_ml[head][1];
    }
  }
  if (!a.part_bf16) {
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) {
      const long long pi = (item * 64 + 16 * hg + hl) * 512 + 128 * vw + 4 * grp;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *(float4*)(a.part_o + pi + 16 * dt) =
            make_float4(acc[hg][dt][0], acc[hg][dt][1], acc[hg][dt][2], acc[hg][dt][3]);
    }
    return;
  }
#pragma unroll
  for (int hg = 0; hg < 4; ++hg)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint2 w2;
      w2.x = pack_bf16x2(acc[hg][dt][0], acc[hg][dt][1]);
      w2.y = pack_bf16x2(acc[hg][dt][2], acc[hg][dt][3]);
      *(uint2*)(stage + (16 * hg + hl) * kPr + 2 * (16 * dt + 4 * grp)) = w2;
    }
  store_rows((uint8_t*)a.part_o + (item * 64 * 512 + 128 * vw) * 2);
}

// ------------------------------------------------------------------------------------------------
// head-group MFMA kernel (few query rows: decode): H = 64, D = 512, bf16 or mixed fp8/bf16 entries
// ------------------------------------------------------------------------------------------------
// One workgroup per (16-head group, query row, slice of the row's list); each of its four waves streams its own
// 16-entry tiles of the slice and keeps an online softmax for the 16 heads.
//   S^T = K Q^T     v_mfma_f32_16x16x32_bf16, A = the tile (lane: entry l % 16, channels 32 s + 8 (l / 16) + v),
//                   B = the 16 heads' queries (lane: head l % 16, the same channels); both stay in registers.
//   O^T += V^T P^T  v_mfma_f32_16x16x16_bf16, A = V^T read by ds_read_b64_tr_b16 from the tile written row-major
//                   to LDS, B = P^T, which is exactly the S^T accumulator layout (lane: head l % 16, entries
//                   4 (l / 16) + v).
// ds_read_b64_tr_b16: in each 16-lane group, output lane 4a + e takes element e of the 8-byte chunks addressed by
// group lanes a, a + 4, a + 8, a + 12.  Group lane a + 4v addresses entry 4G + v, channels 16 dt + 4a .. + 3, so
// lane 4a + e receives V[4G + v][16 dt + 4a + e] for v = 0..3, the A layout of the 16x16x16 instruction.
// The tile is loaded straight into the S^T operand layout, the next one in flight while a tile is scored; the rows
// of the slice's list
// positions are resolved once into LDS so that a tile's loads never wait on an index load.  fp8 entries are widened
// to bf16 in registers (exact: every e4m3 value is a bf16 value); their per-entry scale multiplies the fp8-channel
// part of the logit and is folded into P for the fp8 channels.  The four waves' (max, sum, o) are merged in LDS at
// the end; the four head groups of a (row, slice) pair get workgroup ids congruent mod 8 so that they run on one
// XCD and share its L2 copy of the gathered entries.
constexpr int kHgRow = 520;                // bf16 per LDS tile row (1040 bytes)
constexpr int kWTile = 16;                 // entries per wave tile
constexpr int kWBufBytes = kWTile * kHgRow * 2;  // 16640
// four wave tiles, the row table (the merge buffer reuses both), the waves' (max, sum) and
// the entry scales
constexpr size_t kHgTableOff = (size_t)4 * kWBufBytes;
// the merge: every wave leaves its 32 channel tiles, [wave][32][64 lanes] x 16 bytes, over the (then dead) tiles and
// row table
constexpr size_t kHgMergeBytes = (size_t)4 * 32 * 64 * 16;
constexpr size_t kHgMlOff = kHgMergeBytes > kHgTableOff + (size_t)kHgSplitMax * 4
                                ? kHgMergeBytes
                                : kHgTableOff + (size_t)kHgSplitMax * 4;
constexpr size_t kHgwLds = kHgMlOff + 4 * 16 * 2 * 4 + 4 * 16 * 4;

// A wave's tile in the S^T operand layout.  bf16: v[s] = bytes 64 s + 16 (l / 16) .. + 15 of entry l % 16's row.
// mixed: f[s] = fp8 bytes 32 s + 8 (l / 16) .. + 7 (s < 14), r[s] = RoPE bf16 bytes 64 s + 16 (l / 16) .. (s < 2).
template <int FMT>
struct HgTile;
template <>
struct HgTile<LCA_BF16> {
  uint4 v[16];
  uint64_t valid;  // bit j: entry j of the tile is real (the others load a clamped row and are masked)
};
template <>
struct HgTile<LCA_MIXED_FP8> {
  uint2 f[14];
  uint4 r[2];
  float scale;     // entry l % 16's fp8 scale
  uint64_t valid;
};

struct HgSlice {
  int b, p_begin, npos, nw;  // list positions [p_begin, p_begin + npos); the first nw of the list are the window
};

template <int FMT>
__device__ __forceinline__ void hg_load(HgTile<FMT>& T, const AttnArgs& a, const HgSlice& sl, const int* rows_s,
                                        int i0, int lane) {
  const int hl = lane & 15, grp = lane >> 4;
  const int i = min(i0 + hl, sl.npos - 1);
  const int row = rows_s[i];
  const bool raw = sl.p_begin + i < sl.nw;
  const lca_tensor& src = raw ? a.raw : a.comp;
  const long long rr = row >= 0 ? row : 0;
  T.valid = __ballot(lane < 16 && i0 + hl < sl.npos && row >= 0) & 0xFFFFull;
  if constexpr (FMT == LCA_BF16) {
    const unsigned long long base = (unsigned long long)((const uint8_t*)src.data + rr * 1024) + 16 * grp;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const u32x4_t x = *(gbl_u32x4_t*)(base + 64 * s);
      T.v[s] = make_uint4(x.x, x.y, x.z, x.w);
    }
  } else {
    HgTile<LCA_MIXED_FP8>& M = T;
    const unsigned long long fb = (unsigned long long)((const uint8_t*)src.data + rr * 448) + 8 * grp;
    const unsigned long long rb = (unsigned long long)((const uint8_t*)src.rope + rr * 128) + 16 * grp;
#pragma unroll
    for (int s = 0; s < 14; ++s) {
      const u32x2_t x = *(gbl_u32x2_t*)(fb + 32 * s);
      M.f[s] = make_uint2(x.x, x.y);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const u32x4_t x = *(gbl_u32x4_t*)(rb + 64 * s);
      M.r[s] = make_uint4(x.x, x.y, x.z, x.w);
    }
    M.scale = ((const float*)src.scale)[rr];
  }
}

// The tile's 8 channels of K-step s as bf16 (the A operand), widened from fp8 for the mixed format.
template <int FMT>
__device__ __forceinline__ uint4 hg_chunk(const HgTile<FMT>& T, int s) {
  if constexpr (FMT == LCA_BF16) {
    return T.v[s];
  } else {
    if (s >= 14) return T.r[s - 14];
    const uint2 lo = fp8x4_to_bf16x4(T.f[s].x), hi = fp8x4_to_bf16x4(T.f[s].y);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
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
  const RowList L = row_list(a, b, r);
  const int total = L.nw + L.nc;
  HgSlice sl;
  sl.b = b;
  sl.p_begin = split * a.split_len;
  sl.npos = max(min(a.split_len, total - sl.p_begin), 0);
  sl.nw = L.nw;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hl = lane & 15, grp = lane >> 4;
  const int head = 16 * hg + hl;
  uint8_t* wbuf = hgw_lds + wave * kWBufBytes;
  int* rows_s = (int*)(hgw_lds + kHgTableOff);
  float* ml_s = (float*)(hgw_lds + kHgMlOff);  // [4 waves][16 heads][2]
  float* esc_w = ml_s + 4 * 16 * 2 + 16 * wave;  // [4 waves][16] entry scales (fp8 cache)

  // rows of the slice's list positions (window positions index the raw tensor, the rest the compressed one; -1:
  // padding)
  for (int i = threadIdx.x; i < sl.npos; i += blockDim.x) {
    const int p = sl.p_begin + i;
    const int row = list_row(a, L, b, r, p);
    rows_s[i] = row;
  }
  // the 16 heads' queries as the B operand: lane holds head 16 hg + hl, channels 32 s + 8 grp .. + 7
  bf16x8_t qv[16];
  {
    const uint8_t* qp = (const uint8_t*)a.q + ((long long)qrow * 64 + head) * 1024 + 16 * grp;
#pragma unroll
    for (int s = 0; s < 16; ++s) qv[s] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(qp + 64 * s));
  }
  __syncthreads();

  f32x4_t acc_o[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) acc_o[dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;
  const uint16_t* kt = (const uint16_t*)wbuf;
  const uint16_t* vp = kt + (4 * grp + (hl >> 2)) * kHgRow + 4 * (hl & 3);

  // Scores tile T, then reuses its registers for the loads of the tile at list offset next_i0.
  auto process = [&](HgTile<FMT>& T, int next_i0) {
    // S^T for the tile's 16 entries x 16 heads; the tile goes to LDS (bf16) for the V^T reads
    f32x4_t am = {0.0f, 0.0f, 0.0f, 0.0f}, ar = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const uint4 c = hg_chunk<FMT>(T, s);
      *(uint4*)(wbuf + hl * (kHgRow * 2) + 64 * s + 16 * grp) = c;
      const bf16x8_t kv = __builtin_bit_cast(bf16x8_t, c);
      if (FMT == LCA_MIXED_FP8 && s >= 14)  // RoPE channels: bf16, not scaled
        ar = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qv[s], ar, 0, 0, 0);
      else
        am = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qv[s], am, 0, 0, 0);
    }
    float esc[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    if constexpr (FMT == LCA_MIXED_FP8) {
      if (lane < 16) esc_w[lane] = T.scale;
#pragma unroll
      for (int x = 0; x < 4; ++x) esc[x] = esc_w[4 * grp + x];
    }
    const uint64_t valid = T.valid;
    // the tile's registers are free: the wave's next tile goes in flight (none past the slice: a load nobody uses
    // would still hold up whatever later reuses its registers)
    if (next_i0 < sl.npos) hg_load<FMT>(T, a, sl, rows_s, next_i0, lane);
    float lg[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const float l = (FMT == LCA_MIXED_FP8) ? a.scale * (esc[x] * am[x] + ar[x]) : a.scale * am[x];
      lg[x] = ((valid >> (4 * grp + x)) & 1ull) ? l : -INFINITY;
    }
    float mt = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    mt = xor32_max(xor16_max(mt));
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
    psum = xor32_sum(xor16_sum(psum));
    l_run = l_run * alpha + psum;
    m_run = m_new;
    s16x4_t pb, pbs;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      pb[x] = (short)f32_to_bf16(pv[x]);
      pbs[x] = (FMT == LCA_MIXED_FP8) ? (short)f32_to_bf16(pv[x] * esc[x]) : pb[x];  // fp8 channels carry the scale
    }
    if (__ballot(alpha != 1.0f)) {  // wave-uniform: some head's reference max moved
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) acc_o[dt] *= alpha;
    }
    // V^T reads eight channel tiles ahead of the products
#pragma unroll
    for (int d0 = 0; d0 < 32; d0 += 8) {
      s16x4_t av[8];
#pragma unroll
      for (int d = 0; d < 8; ++d) av[d] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vp + 16 * (d0 + d)));
#pragma unroll
      for (int d = 0; d < 8; ++d)
        acc_o[d0 + d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
            av[d], (FMT == LCA_MIXED_FP8 && d0 + d < 28) ? pbs : pb, acc_o[d0 + d], 0, 0, 0);
    }
  };

  // the wave's tiles tt = wave, wave + 4, ...: each tile's registers take the next tile's loads as soon as its
  // S^T products are issued, so the loads overlap the softmax and the V^T products
  const int ntiles = (sl.npos + kWTile - 1) / kWTile;
  if (wave < ntiles) {
    HgTile<FMT> T;
    hg_load<FMT>(T, a, sl, rows_s, kWTile * wave, lane);
    for (int tt = wave; tt < ntiles; tt += 4) process(T, kWTile * (tt + 4));
  }

  // merge the four waves (same heads, different entries): wave w finalizes channel tiles [8 w, 8 w + 8)
  __syncthreads();  // every wave is done with its tile: the LDS is reused
  if (grp == 0) {
    ml_s[(wave * 16 + hl) * 2 + 0] = m_run;
    ml_s[(wave * 16 + hl) * 2 + 1] = l_run;
  }
  f32x4_t* mg = (f32x4_t*)hgw_lds;  // [wave][32 channel tiles][64 lanes]
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) mg[(wave * 32 + dt) * 64 + lane] = acc_o[dt];
  __syncthreads();
  float mw[4], M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    mw[w] = ml_s[(w * 16 + hl) * 2 + 0];
    M = fmaxf(M, mw[w]);
  }
  float Lsum = 0.0f, fw[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    fw[w] = (mw[w] == -INFINITY) ? 0.0f : __expf(mw[w] - M);
    Lsum += fw[w] * ml_s[(w * 16 + hl) * 2 + 1];
  }
  f32x4_t res[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    f32x4_t acc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int w = 0; w < 4; ++w) acc += fw[w] * mg[(w * 32 + 8 * wave + k) * 64 + lane];
    res[k] = acc;
  }

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
    for (int k = 0; k < 8; ++k) {
      const int c0 = 16 * (8 * wave + k) + 4 * grp;
      if (a.out_format == LCA_F32) {
        *(float4*)((float*)a.out + obase + c0) =
            make_float4(res[k][0] * f, res[k][1] * f, res[k][2] * f, res[k][3] * f);
      } else {
        uint2 w2;
        w2.x = pack_bf16x2(res[k][0] * f, res[k][1] * f);
        w2.y = pack_bf16x2(res[k][2] * f, res[k][3] * f);
        *(uint2*)((uint16_t*)a.out + obase + c0) = w2;
      }
    }
    if (a.lse && wave == 0 && grp == 0) a.lse[(long long)qrow * 64 + head] = (Mz == -INFINITY) ? -INFINITY : Mz + __logf(den);
  } else {
    const long long item = (long long)qrow * S + split;
    float* po = a.part_o + (item * 64 + head) * 512;
#pragma unroll
    for (int k = 0; k < 8; ++k) *(f32x4_t*)(po + 16 * (8 * wave + k) + 4 * grp) = res[k];
    if (wave == 0 && grp == 0) {
      a.part_ml[(item * 64 + head) * 2 + 0] = M;
      a.part_ml[(item * 64 + head) * 2 + 1] = Lsum;
    }
  }
}

// ------------------------------------------------------------------------------------------------
// wide MFMA kernel (few query rows over many entries: dense HCA decode over the mixed cache): H = 64, D = 512
// (written for bf16 or mixed entries; launched for the mixed cache, since bf16 rows take the many-row kernel)
// ------------------------------------------------------------------------------------------------
// One 512-thread workgroup per (query row, slice of its list) with all 64 heads; wave w owns channels
// [64 w, 64 w + 64) of every entry (for the mixed cache, waves 0..6 hold the 448 fp8 channels and wave 7 the 64 RoPE
// channels), so each entry is read from memory once per workgroup and each wave streams only its 128 bytes of it.
// Two waves share each SIMD, so one wave's LDS and barrier latencies overlap the other's products.  Per 32-entry tile:
//   partial S^T (v_mfma_f32_16x16x32_bf16: A = the wave's channels of the tile, B = those channels of the 64 heads'
//     queries, both in registers; fp8 waves scale it by the entry's scale) -> LDS; barrier;
//   wave w sums the eight partials of heads [8 w, 8 w + 8), runs their online softmax (lazy rescale as in the
//     head-group kernel) and writes P (bf16, and P times the entry's fp8 scale) and the rescale factors to LDS;
//     barrier;
//   O^T += V^T P^T for the wave's channels and all heads (v_mfma_f32_16x16x32_bf16, K = the tile's 32 entries:
//     A = V^T from two ds_read_b64_tr_b16 of the wave's own row-major tile in LDS, B = P^T from LDS).
// The output of a wave's channels needs no cross-wave merge; the heads' (max, sum) come from their owners.
constexpr int kWdWaves = 8;
constexpr int kWdThreads = 64 * kWdWaves;
constexpr int kWdTile = 32;                                 // entries per tile
constexpr int kWdRowB = 144;                                // LDS bytes per tile row (a wave's 64 channels + pad)
constexpr int kWdTileBytes = kWdTile * kWdRowB;             // 4608 per wave
constexpr int kWdSpStride = 36;                             // floats per head row of a wave's partial logits
constexpr int kWdPStride = 40;                              // bf16 per head row of P (32 entries + pad)
constexpr size_t kWdSpOff = (size_t)kWdWaves * kWdTileBytes;
constexpr size_t kWdPOff = kWdSpOff + (size_t)kWdWaves * 64 * kWdSpStride * 4;
constexpr size_t kWdAlphaOff = kWdPOff + (size_t)2 * 64 * kWdPStride * 2;
constexpr size_t kWdTableOff = kWdAlphaOff + 64 * 4;
constexpr size_t kWdMlOff = kWdTableOff + (size_t)kHgSplitMax * 4;
constexpr size_t kWdLds = kWdMlOff + 64 * 2 * 4;
static_assert(kWdLds <= 160 * 1024, "wide kernel LDS");

// A wave's tile: for entry 16 eb + l % 16 and K-step s, channels 64 w + 32 s + 8 (l / 16) .. + 7.
template <int FMT>
struct WdTile;
template <>
struct WdTile<LCA_BF16> {
  uint4 v[2][2];
  uint32_t valid;  // bit j: entry j of the tile is real
};
template <>
struct WdTile<LCA_MIXED_FP8> {
  uint4 c[2][2];   // waves 0..6: the 8 fp8 codes in .x, .y; wave 7: the 8 RoPE channels in bf16
  float scale[2];  // the fp8 scale of entry 16 eb + l % 16
  uint32_t valid;
};

template <int FMT>
__device__ __forceinline__ void wd_load(WdTile<FMT>& T, const AttnArgs& a, const HgSlice& sl, const int* rows_s,
                                        int i0, int wave, int lane) {
  const int hl = lane & 15, grp = lane >> 4;
  uint32_t valid = 0;
#pragma unroll
  for (int eb = 0; eb < 2; ++eb) {
    const int i = min(i0 + 16 * eb + hl, sl.npos - 1);
    const int row = rows_s[i];
    const bool raw = sl.p_begin + i < sl.nw;
    const lca_tensor& src = raw ? a.raw : a.comp;
    const long long rr = row >= 0 ? row : 0;
    valid |= (uint32_t)(__ballot(lane < 16 && i0 + 16 * eb + hl < sl.npos && row >= 0) & 0xFFFFull) << (16 * eb);
    if constexpr (FMT == LCA_BF16) {
      const unsigned long long base = (unsigned long long)((const uint8_t*)src.data + rr * 1024) + 128 * wave + 16 * grp;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const u32x4_t x = *(gbl_u32x4_t*)(base + 64 * s);
        T.v[eb][s] = make_uint4(x.x, x.y, x.z, x.w);
      }
    } else {
      if (wave == 7) {
        const unsigned long long rb = (unsigned long long)((const uint8_t*)src.rope + rr * 128) + 16 * grp;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const u32x4_t x = *(gbl_u32x4_t*)(rb + 64 * s);
          T.c[eb][s] = make_uint4(x.x, x.y, x.z, x.w);
        }
      } else {
        const unsigned long long fb = (unsigned long long)((const uint8_t*)src.data + rr * 448) + 64 * wave + 8 * grp;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const u32x2_t x = *(gbl_u32x2_t*)(fb + 32 * s);
          T.c[eb][s] = make_uint4(x.x, x.y, 0u, 0u);
        }
      }
      T.scale[eb] = ((const float*)src.scale)[rr];
    }
  }
  T.valid = valid;
}

template <int FMT>
__device__ __forceinline__ uint4 wd_chunk(const WdTile<FMT>& T, int eb, int s, int wave) {
  if constexpr (FMT == LCA_BF16) {
    return T.v[eb][s];
  } else {
    if (wave == 7) return T.c[eb][s];
    const uint2 lo = fp8x4_to_bf16x4(T.c[eb][s].x), hi = fp8x4_to_bf16x4(T.c[eb][s].y);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
}

// Exchange with the lane 8 apart inside each 16-lane row (row_ror:8).
__device__ __forceinline__ float xor8_get(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
}

template <int FMT>
__global__ __launch_bounds__(kWdThreads) void attn_wide_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t wd_lds[];
  const int item = blockIdx.x;
  const int S = a.n_splits;
  const int qrow = item / S, split = item % S;
  const int b = qrow / a.Sq, r = qrow % a.Sq;
  const RowList L = row_list(a, b, r);
  const int total = L.nw + L.nc;
  HgSlice sl;
  sl.b = b;
  sl.p_begin = split * a.split_len;
  sl.npos = max(min(a.split_len, total - sl.p_begin), 0);
  sl.nw = L.nw;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hl = lane & 15, grp = lane >> 4;
  const int oh = 8 * wave + (lane & 7), oq = lane >> 3;  // softmax owner lane: head oh, entries 4 oq .. 4 oq + 3
  uint8_t* tbuf = wd_lds + wave * kWdTileBytes;
  float* sp = (float*)(wd_lds + kWdSpOff);             // [8 waves][64 heads][kWdSpStride]
  uint16_t* P_s = (uint16_t*)(wd_lds + kWdPOff);       // [64 heads][kWdPStride]
  uint16_t* Pe_s = P_s + 64 * kWdPStride;              // P times the entry scale (fp8 channels)
  float* alpha_s = (float*)(wd_lds + kWdAlphaOff);     // [64]
  int* rows_s = (int*)(wd_lds + kWdTableOff);
  float* ml_s = (float*)(wd_lds + kWdMlOff);           // [64][2]
  constexpr bool kMixed = FMT == LCA_MIXED_FP8;
  const bool fp8_wave = kMixed && wave < 7;

  for (int i = threadIdx.x; i < sl.npos; i += blockDim.x) {
    const int p = sl.p_begin + i;
    const int row = list_row(a, L, b, r, p);
    rows_s[i] = row;
  }
  // queries (B operand of the partial S^T): lane holds head 16 hb + hl, channels 64 wave + 32 s + 8 grp .. + 7
  bf16x8_t qv[2][4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const uint8_t* qp = (const uint8_t*)a.q + ((long long)qrow * 64 + 16 * hb + hl) * 1024 + 128 * wave + 16 * grp;
#pragma unroll
    for (int s = 0; s < 2; ++s) qv[s][hb] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(qp + 64 * s));
  }
  __syncthreads();

  f32x4_t acc_o[4][4];  // [channel tile mb][head block hb]: channel 64 wave + 16 mb + 4 grp + x, head 16 hb + hl
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) acc_o[mb][hb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;  // of head oh (owned by this wave)

  auto step = [&](WdTile<FMT>& T, int next_i0) {
    // partial S^T of the tile over this wave's channels; the tile goes to LDS (bf16) for the V^T reads
    f32x4_t sacc[2][4];
#pragma unroll
    for (int eb = 0; eb < 2; ++eb)
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) sacc[eb][hb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int eb = 0; eb < 2; ++eb) {
        const uint4 c = wd_chunk<FMT>(T, eb, s, wave);
        *(uint4*)(tbuf + (16 * eb + hl) * kWdRowB + 64 * s + 16 * grp) = c;
        const bf16x8_t kv = __builtin_bit_cast(bf16x8_t, c);
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          sacc[eb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qv[s][hb], sacc[eb][hb], 0, 0, 0);
      }
    if (fp8_wave) {  // the entry scales of the accumulator's entries 16 eb + 4 grp + x (lane 4 grp + x loaded them)
#pragma unroll
      for (int eb = 0; eb < 2; ++eb)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          float sc = 1.0f;
          if constexpr (kMixed) sc = __shfl(T.scale[eb], 4 * grp + x, 64);
#pragma unroll
          for (int hb = 0; hb < 4; ++hb) sacc[eb][hb][x] = sc * sacc[eb][hb][x];
        }
    }
#pragma unroll
    for (int eb = 0; eb < 2; ++eb)
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
        *(f32x4_t*)(sp + (wave * 64 + 16 * hb + hl) * kWdSpStride + 16 * eb + 4 * grp) = sacc[eb][hb];
    // the owner lanes' entry scales (entries 4 oq + x: lane (4 oq + x) % 16 of block (4 oq + x) / 16 loaded them)
    float esc[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    if constexpr (kMixed) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int e = 4 * oq + x;
        const float s0 = __shfl(T.scale[0], e & 15, 64), s1 = __shfl(T.scale[1], e & 15, 64);
        esc[x] = e < 16 ? s0 : s1;
      }
    }
    const uint32_t valid = T.valid;
    if (next_i0 < sl.npos) wd_load<FMT>(T, a, sl, rows_s, next_i0, wave, lane);  // the next tile goes in flight
    __syncthreads();

    // softmax of head oh over the tile's entries 4 oq + x
    f32x4_t s4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int w = 0; w < kWdWaves; ++w) s4 += *(const f32x4_t*)(sp + (w * 64 + oh) * kWdSpStride + 4 * oq);
    float lg[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) lg[x] = ((valid >> (4 * oq + x)) & 1u) ? a.scale * s4[x] : -INFINITY;
    float mt = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    mt = fmaxf(mt, xor8_get(mt));
    mt = xor32_max(xor16_max(mt));
    const float m_new = (mt > m_run + kRescaleSlack) ? mt : m_run;
    const float alpha = (m_new == m_run) ? 1.0f : __expf(m_run - m_new);
    float p[4], psum = 0.0f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      p[x] = (lg[x] == -INFINITY) ? 0.0f : __expf(lg[x] - m_new);
      psum += p[x];
    }
    uint2 pw;
    pw.x = pack_bf16x2(p[0], p[1]);
    pw.y = pack_bf16x2(p[2], p[3]);
    *(uint2*)(P_s + oh * kWdPStride + 4 * oq) = pw;
    if constexpr (kMixed) {
      uint2 pe;
      pe.x = pack_bf16x2(p[0] * esc[0], p[1] * esc[1]);
      pe.y = pack_bf16x2(p[2] * esc[2], p[3] * esc[3]);
      *(uint2*)(Pe_s + oh * kWdPStride + 4 * oq) = pe;
    }
    psum += xor8_get(psum);
    psum = xor32_sum(xor16_sum(psum));
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (lane < 8) alpha_s[oh] = alpha;
    __syncthreads();

    // O^T += V^T P^T over this wave's channels, all 64 heads
    float al[4];
    bool any = false;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      al[hb] = alpha_s[16 * hb + hl];
      any |= al[hb] != 1.0f;
    }
    if (__ballot(any)) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) acc_o[mb][hb] *= al[hb];
    }
    const uint16_t* Pw = fp8_wave ? Pe_s : P_s;  // the fp8 channels carry the entry scale
    bf16x8_t bp[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
      bp[hb] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(Pw + (16 * hb + hl) * kWdPStride + 8 * grp));
    const uint8_t* vrow = tbuf + (8 * grp + (hl >> 2)) * kWdRowB + 8 * (hl & 3);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vrow + 32 * mb));
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vrow + 4 * kWdRowB + 32 * mb));
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
        acc_o[mb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bp[hb], acc_o[mb][hb], 0, 0, 0);
    }
  };

  const int ntiles = (sl.npos + kWdTile - 1) / kWdTile;
  if (ntiles > 0) {  // uniform over the workgroup: every wave takes every tile (its own channels)
    // one tile buffer: the next tile loads as soon as a tile's S^T products are issued (a second buffer costs
    // more registers than two waves per SIMD leave, and a spill reload would drain the loads in flight)
    WdTile<FMT> T;
    wd_load<FMT>(T, a, sl, rows_s, 0, wave, lane);
    for (int tt = 0; tt < ntiles; ++tt) step(T, kWdTile * (tt + 1));
  }

  // every head's (max, sum) from its owner
  if (lane < 8) {
    ml_s[oh * 2 + 0] = m_run;
    ml_s[oh * 2 + 1] = l_run;
  }
  __syncthreads();
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const int head = 16 * hb + hl;
    const float M = ml_s[head * 2 + 0], Ls = ml_s[head * 2 + 1];
    if (S == 1) {
      const float z = a.sink[head];
      const float Mz = fmaxf(M, z);
      float den = 0.0f, f = 0.0f;
      if (Mz != -INFINITY) {
        den = ((z == -INFINITY) ? 0.0f : __expf(z - Mz)) + ((M == -INFINITY) ? 0.0f : Ls * __expf(M - Mz));
        f = (M == -INFINITY) ? 0.0f : __expf(M - Mz) / den;
      }
      const long long obase = ((long long)qrow * 64 + head) * 512 + 64 * wave + 4 * grp;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const f32x4_t o = acc_o[mb][hb];
        if (a.out_format == LCA_F32) {
          *(float4*)((float*)a.out + obase + 16 * mb) = make_float4(o[0] * f, o[1] * f, o[2] * f, o[3] * f);
        } else {
          uint2 w2;
          w2.x = pack_bf16x2(o[0] * f, o[1] * f);
          w2.y = pack_bf16x2(o[2] * f, o[3] * f);
          *(uint2*)((uint16_t*)a.out + obase + 16 * mb) = w2;
        }
      }
      if (a.lse && wave == 2 * hb + (hl >> 3) && grp == 0)
        a.lse[(long long)qrow * 64 + head] = (Mz == -INFINITY) ? -INFINITY : Mz + __logf(den);
    } else {
      // unnormalised partial sums in bf16 (the merge rescales them in fp32; the output is bf16 or checked at bf16
      // precision anyway), half the bytes of the split round trip
      const long long pi = ((long long)item * 64 + head) * 512 + 64 * wave + 4 * grp;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const f32x4_t o = acc_o[mb][hb];
        uint2 w2;
        w2.x = pack_bf16x2(o[0], o[1]);
        w2.y = pack_bf16x2(o[2], o[3]);
        *(uint2*)((uint16_t*)a.part_o + pi + 16 * mb) = w2;
      }
      if (wave == 2 * hb + (hl >> 3) && grp == 0) {
        a.part_ml[((long long)item * 64 + head) * 2 + 0] = M;
        a.part_ml[((long long)item * 64 + head) * 2 + 1] = Ls;
      }
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
  const RowList L = row_list(a, b, r);
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
// sparse decode attention in two passes (few query rows, H = 64, D = 512, bf16 or mixed entries)
// ------------------------------------------------------------------------------------------------
// With one query row per sequence, splitting a row's entry list over workgroups leaves one 64 x 512 partial output
// per split -- more bytes than the split's own entries -- and a merge pass over them.  The decode path instead
// stores the probabilities, which are 64 values per entry:
//   scores (one workgroup per (query row, 32-entry tile), all 64 heads): S^T = scale * K Q^T for the tile with
//     v_mfma_f32_16x16x32_bf16, wave w contracting channels [128 w, 128 w + 128) (fp8 entries widened exactly, the
//     entry scale applied to their part) and the four partial products added in LDS; then per head the tile max
//     m_t, P_t = e^(S - m_t) (bf16, 0 for padding) and l_t = sum P_t.
//   values (one workgroup per (query row, 64 channels, 16 heads)): M = max(z, m_t), den = e^(z - M) +
//     sum_t l_t e^(m_t - M) and the tile weights f_t = e^(m_t - M) / den, then O^T = sum_t f_t V_t^T P_t^T on
//     v_mfma_f32_16x16x32_bf16: wave w of 8 takes tiles w, w + 8, ..., issues every load of its tiles at once, turns
//     each tile's channels into a row-major bf16 tile in its own LDS area (fp8 widened and multiplied by the entry
//     scale) and reads V^T with ds_read_b64_tr_b16; the eight waves' sums are added in LDS at the end.
// The exact normaliser is known before any value is weighted, so no partial output goes through memory.
constexpr int kDecTile = 32;                              // list positions per tile
constexpr int kDecMaxTiles = kDecMaxEntries / kDecTile;   // 64
constexpr int kDsTile = 64;                               // list positions per score workgroup (two value tiles)
constexpr int kDsWaves = 8;                               // waves of a score workgroup
constexpr int kDvRowB = 144;                              // LDS bytes per entry of a value tile (64 bf16 + pad)
constexpr int kDvWaves = 8;                               // waves of a value workgroup

template <int FMT>
__global__ __launch_bounds__(64 * kDsWaves) void attn_dec_score_kernel(AttnArgs a) {
  constexpr bool MX = FMT == LCA_MIXED_FP8;
  // LDS: the 64 x 512 queries (1 KB rows), then the tile's entries (bf16: 1 KB rows; mixed: 448 fp8 bytes, 128
  // RoPE bytes and 16 bytes of padding).  bf16 rows keep 16-byte chunk c of row r at chunk c ^ (r % 16), so that
  // the 16 rows an operand read touches fall on distinct banks; the padded mixed rows do the same by their stride.
  constexpr int KROW = MX ? 592 : 1024;
  __shared__ __attribute__((aligned(16))) uint8_t ds_lds[65536 + kDsTile * KROW];
  __shared__ uint8_t ds_ok[kDsTile];
  __shared__ __attribute__((aligned(16))) float ds_esc[kDsTile];
  uint8_t* const qs = ds_lds;
  uint8_t* const kt = ds_lds + 65536;
  const int qrow = blockIdx.x, tile = blockIdx.y;
  const int b = qrow / a.Sq, r = qrow - b * a.Sq;
  const RowList L = row_list(a, b, r);
  const int total = L.nw + L.nc;
  const int p0 = tile * kDsTile;
  if (p0 >= total) return;  // past this row's list: the value pass does not read these tiles
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int hl = lane & 15, grp = lane >> 4;

  // lane e of every wave resolves tile entry e: its tensor row (row 0 of the compressed tensor for padding), whether
  // it is a window entry and whether it is real; the copies below take these by readlane / ds_bpermute
  // (the index load is unconditional -- a read of the sink array where there is no index -- and its value is used
  // only after the query copies are issued, so that they are not held up by it)
  const int pl = p0 + lane;
  const bool rwl = pl < L.nw;
  const bool sel = !rwl && pl < total;
  const int xl = *(sel ? a.idx + ((long long)qrow * a.k + (pl - L.nw)) : (const int*)a.sink);
  // queries: wave w copies head rows 8 w .. 8 w + 7, 1 KB per instruction
  {
    const uint8_t* qg = (const uint8_t*)a.q + (long long)qrow * 65536;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int h = 8 * wave + i;
      __builtin_amdgcn_global_load_lds((const void*)(qg + h * 1024 + 16 * (lane ^ (h & 15))), (void*)(qs + h * 1024),
                                       16, 0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm8);  // the index load has landed; the eight query copies may still be in flight
  __builtin_amdgcn_sched_barrier(0);
  const int rowl = rwl ? (int)(L.w0 + pl - L.raw0) : ((sel & (xl >= 0) & (xl < a.N)) ? xl : -1);
  const bool okl = rowl >= 0;
  // storage row: the raw tensor is dense; the compressed one may be paged (a dependent table read)
  const long long rabsl = rwl ? (long long)b * a.raw.cap + rowl : tensor_row(a.comp, b, okl ? rowl : 0);
  const int rlo = (int)rabsl, rhi = (int)(rabsl >> 32), rwi = rwl ? 1 : 0;
  // entries
  if constexpr (!MX) {
    // wave w copies entries 8 w .. 8 w + 7, one 1 KB row per instruction
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = 8 * wave + i;
      const long long rabs = ((long long)__builtin_amdgcn_readlane(rhi, e) << 32) |
                             (uint32_t)__builtin_amdgcn_readlane(rlo, e);
      const uint8_t* src = (const uint8_t*)(__builtin_amdgcn_readlane(rwi, e) ? a.raw.data : a.comp.data) +
                           rabs * 1024 + 16 * (lane ^ (e & 15));
      __builtin_amdgcn_global_load_lds((const void*)src, (void*)(kt + e * 1024), 16, 0, 0);
    }
  } else {
    // 37 instructions of 64 16-byte slots: slot s is chunk s % 37 of entry s / 37 (28 fp8 chunks, 8 RoPE chunks,
    // then the padding slot, which copies fp8 chunk 0); wave w issues instructions w, w + 8, ...
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int j = wave + 8 * i;
      const int sl = 64 * min(j, 36) + lane, e = sl / 37, c = sl - 37 * e;
      const long long rabs = ((long long)__builtin_amdgcn_ds_bpermute(4 * e, rhi) << 32) |
                             (uint32_t)__builtin_amdgcn_ds_bpermute(4 * e, rlo);
      const bool rw = __builtin_amdgcn_ds_bpermute(4 * e, rwi) != 0;
      // (fields selected one by one: a lane-dependent choice of the whole tensor struct would be read through
      // per-lane pointers)
      const uint8_t* fb = (const uint8_t*)(rw ? a.raw.data : a.comp.data) + rabs * 448;
      const uint8_t* rb = (const uint8_t*)(rw ? a.raw.rope : a.comp.rope) + rabs * 128;
      const uint8_t* g = c < 28 ? fb + 16 * c : c < 36 ? rb + 16 * (c - 28) : fb;
      if (j < 37) __builtin_amdgcn_global_load_lds((const void*)g, (void*)(kt + 1024 * j), 16, 0, 0);
    }
  }
  if (wave == 0) {
    ds_ok[lane] = okl ? 1 : 0;
    if constexpr (MX) {
      const long long rabs = ((long long)rhi << 32) | (uint32_t)rlo;
      ds_esc[lane] = (rwi ? (const float*)a.raw.scale : (const float*)a.comp.scale)[rabs];
    }
  }
  __syncthreads();  // every copy has landed

  // wave (cs, eh): channels [128 cs, 128 cs + 128) of entries [32 eh, 32 eh + 32) for all 64 heads
  const int cs = wave & 3, eh = wave >> 2;
  f32x4_t acc[2][4], accr[2][4];
#pragma unroll
  for (int eb = 0; eb < 2; ++eb)
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      acc[eb][hb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      accr[eb][hb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int c = 16 * cs + 4 * ks + grp;  // the lane's 16-byte chunk: channels 8 c .. 8 c + 7
    bf16x8_t qb[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
      qb[hb] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(qs + (16 * hb + hl) * 1024 + 16 * (c ^ hl)));
#pragma unroll
    for (int eb = 0; eb < 2; ++eb) {
      const int e = 32 * eh + 16 * eb + hl;
      if constexpr (!MX) {
        const bf16x8_t kv = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(kt + e * 1024 + 16 * (c ^ hl)));
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          acc[eb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qb[hb], acc[eb][hb], 0, 0, 0);
      } else if (128 * cs + 32 * ks < 448) {
        const uint2 f = *(const uint2*)(kt + e * KROW + 8 * c);
        const uint2 lo = fp8x4_to_bf16x4(f.x), hi = fp8x4_to_bf16x4(f.y);
        const bf16x8_t kv = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          acc[eb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qb[hb], acc[eb][hb], 0, 0, 0);
      } else {
        const bf16x8_t kv = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(kt + e * KROW + 448 + 16 * (c - 56)));
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          accr[eb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qb[hb], accr[eb][hb], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // the staged rows are dead: the partial products go over them
  // partials [slot][entry block 2 eh + eb][head block][lane]: slot = channel quarter (mixed: slot 4 = RoPE part)
  f32x4_t* part = (f32x4_t*)ds_lds;
#pragma unroll
  for (int eb = 0; eb < 2; ++eb)
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      part[((cs * 4 + 2 * eh + eb) * 4 + hb) * 64 + lane] = acc[eb][hb];
      if constexpr (MX)
        if (cs == 3) part[((4 * 4 + 2 * eh + eb) * 4 + hb) * 64 + lane] = accr[eb][hb];
    }
  __syncthreads();

  // thread (head h, group g) finishes entries 8 g .. 8 g + 7 of head h: entry 16 B + er of head block h / 16 sits in
  // lane 16 (er / 4) + h % 16, element er % 4, of entry block B
  const int h = tid >> 3, g = tid & 7;
  const int blk = g >> 1, l0 = 32 * (g & 1) + (h & 15), hb = h >> 4;
  float sv[8];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int l = l0 + 16 * half;
    f32x4_t sm = (part[((0 * 4 + blk) * 4 + hb) * 64 + l] + part[((1 * 4 + blk) * 4 + hb) * 64 + l]) +
                 (part[((2 * 4 + blk) * 4 + hb) * 64 + l] + part[((3 * 4 + blk) * 4 + hb) * 64 + l]);
    if constexpr (MX) sm = sm * *(const f32x4_t*)&ds_esc[8 * g + 4 * half] + part[((4 * 4 + blk) * 4 + hb) * 64 + l];
#pragma unroll
    for (int x = 0; x < 4; ++x) sv[4 * half + x] = a.scale * sm[x];
  }
  // per 32-entry value tile (groups g / 4): max, probabilities, sum
  float mt = -INFINITY;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (ds_ok[8 * g + j]) mt = fmaxf(mt, sv[j]);
  mt = fmaxf(mt, __shfl_xor(mt, 1));
  mt = fmaxf(mt, __shfl_xor(mt, 2));
  float pv[8], ls = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    pv[j] = ds_ok[8 * g + j] ? __expf(sv[j] - mt) : 0.0f;
    ls += pv[j];
  }
  ls += __shfl_xor(ls, 1);
  ls += __shfl_xor(ls, 2);
  // P in the value pass's operand order: per (row, head group, tile) 64 lanes x 16 bytes, lane 16 q + (h % 16)
  // holding entries 8 q .. 8 q + 7 of the tile for head h
  const int t = 2 * tile + (g >> 2), q = g & 3;
  const u32x4_t pk = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
                      pack_bf16x2(pv[6], pv[7])};
  *(u32x4_t*)(a.dec_p + ((((long long)qrow * 4 + hb) * a.dec_tiles + t) * 64 + 16 * q + (h & 15)) * 8) = pk;
  if (q == 0) ((float2*)a.dec_ml)[((long long)qrow * a.dec_tiles + t) * 64 + h] = make_float2(mt, ls);
}

// NTI: the most tiles a wave takes (every wave loads all of its tiles at once).  The occupancy is stated so that the
// compiler keeps the loads in distinct registers rather than reusing them at the price of waits: 4 waves per SIMD
// (two workgroups per CU) for short lists, 2 for long ones.
template <int FMT, int NTI>
__global__ __launch_bounds__(64 * kDvWaves) __attribute__((amdgpu_waves_per_eu(NTI <= 4 ? 4 : 2, NTI <= 4 ? 4 : 2)))
void attn_dec_value_kernel(AttnArgs a) {
  constexpr int kGroups = 4 * kDvWaves;  // tile groups of the weight computation (16 heads x kGroups threads)
  constexpr int kPer = kDecMaxTiles / kGroups;
  __shared__ __attribute__((aligned(16))) uint8_t dvt[kDvWaves][kDecTile * kDvRowB];  // each wave's value tile
  __shared__ int drows[kDecMaxEntries];
  __shared__ float dfac[kDecMaxTiles][16];
  __shared__ float dred[kGroups][16];
  const int qrow = blockIdx.x, cb = blockIdx.y, hg = blockIdx.z;
  const int b = qrow / a.Sq, r = qrow - b * a.Sq;
  const RowList L = row_list(a, b, r);
  const int total = L.nw + L.nc;
  const int nt = (total + kDecTile - 1) / kDecTile;
  const int T = a.dec_tiles;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int hl = lane & 15, grp = lane >> 4;

  // rows of all T * 32 list positions (-1: padding or past the list)
  for (int p = tid; p < T * kDecTile; p += 64 * kDvWaves) {
    drows[p] = p < total ? list_row(a, L, b, r, p) : -1;
  }
  // this thread's tiles' (m_t, l_t) for head 16 hg + (tid % 16) and that head's sink; both read before the value
  // loads (a load issued after them could only be waited for together with all of them), tiles past the list
  // reading the last tile and dropped below
  const int hh = tid & 15, tg = tid >> 4;
  const int head = 16 * hg + hh;
  float2 mlv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    mlv[i] = ((const float2*)a.dec_ml)[((long long)qrow * T + min(tg + kGroups * i, T - 1)) * 64 + head];
  const float z = a.sink[head];
  __syncthreads();

  // wave w: tiles w, w + kDvWaves, ... (nti of them); acc[d] = O^T for channels 64 cb + 16 d + 4 grp + x, head
  // 16 hg + hl
  const int nti = nt > wave ? (nt - wave + kDvWaves - 1) / kDvWaves : 0;
  f32x4_t acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) acc[d] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  uint8_t* vt = dvt[wave];
  const uint16_t* pbase = a.dec_p + (((long long)qrow * 4 + hg) * T * 64 + lane) * 8;
  // the V^T reads: rows 8 grp + 4 half + hl / 4, channels 16 d + 4 (hl % 4)
  const uint8_t* vtr = vt + (8 * grp + (hl >> 2)) * kDvRowB + 8 * (hl & 3);

  // The body twice, for bf16 channels and for fp8 channels (the mixed cache's blocks 0..6), so that neither has a
  // branch between its loads.
  auto run = [&](auto f8c) {
    constexpr bool F8 = decltype(f8c)::value;
    u32x4_t vr[NTI][4];
    float es[NTI][2];
    bool ok[NTI][4];
    u32x4_t pr[NTI];
    // every load of the wave's tiles (slots past its last tile repeat a valid tile, so that the count is fixed)
#pragma unroll
    for (int i = 0; i < NTI; ++i) {
      const int t = min(wave + kDvWaves * min(i, max(nti, 1) - 1), T - 1);
      pr[i] = *(gbl_u32x4_t*)(pbase + 512 * t);
      if constexpr (!F8) {
        // entries (lane / 8) + 8 k, 16 bytes (8 channels) at chunk lane % 8
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int p = 32 * t + (lane >> 3) + 8 * k;
          const int row = drows[p];
          ok[i][k] = row >= 0;
          const bool rw = p < L.nw;
          // (fields selected one by one: a lane-dependent choice of the whole tensor struct would be read through
          // per-lane pointers)
          const long long rabs = row >= 0 ? row : 0;
          const uint8_t* vp = FMT == LCA_MIXED_FP8
                                  ? (const uint8_t*)(rw ? a.raw.rope : a.comp.rope) + rabs * 128
                                  : (const uint8_t*)(rw ? a.raw.data : a.comp.data) + rabs * 1024 + 128 * cb;
          vr[i][k] = *(gbl_u32x4_t*)(vp + 16 * (lane & 7));
        }
      } else {
        // entries (lane / 4) + 16 k, 16 fp8 channels at chunk lane % 4, and the entry scales
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int p = 32 * t + (lane >> 2) + 16 * k;
          const int row = drows[p];
          ok[i][k] = row >= 0;
          const bool rw = p < L.nw;
          const long long rabs = row >= 0 ? row : 0;
          vr[i][k] = *(gbl_u32x4_t*)((const uint8_t*)(rw ? a.raw.data : a.comp.data) + rabs * 448 + 64 * cb +
                                     16 * (lane & 3));
          es[i][k] = ((const float*)(rw ? a.raw.scale : a.comp.scale))[rabs];
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // while the loads are in flight: M = max(z, m_t), den = e^(z - M) + sum_t l_t e^(m_t - M) and
    // f_t = e^(m_t - M) / den per head of the group (LDS-only barriers: the loads are not waited for)
    {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (tg + kGroups * i < nt) mx = fmaxf(mx, mlv[i].x);
      dred[tg][hh] = mx;
      pd_barrier();
      float M = z;
#pragma unroll
      for (int gi = 0; gi < kGroups; ++gi) M = fmaxf(M, dred[gi][hh]);
      float d = 0.0f;
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (tg + kGroups * i < nt && mlv[i].x != -INFINITY) d += mlv[i].y * __expf(mlv[i].x - M);
      pd_barrier();
      dred[tg][hh] = d;
      pd_barrier();
      float den = (z == -INFINITY) ? 0.0f : __expf(z - M);
#pragma unroll
      for (int gi = 0; gi < kGroups; ++gi) den += dred[gi][hh];
      const float inv = den > 0.0f ? 1.0f / den : 0.0f;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int t = tg + kGroups * i;
        if (t < nt) dfac[t][hh] = (mlv[i].x == -INFINITY) ? 0.0f : __expf(mlv[i].x - M) * inv;
      }
      if (cb == 0 && tg == 0 && a.lse)
        a.lse[(long long)qrow * 64 + head] = (M == -INFINITY) ? -INFINITY : M + __logf(den);
      pd_barrier();
    }

#pragma unroll
    for (int i = 0; i < NTI; ++i) {
      if (i < nti) {
        const int t = wave + kDvWaves * i;
        // the tile's channels, row-major bf16 (padding rows zero: their probabilities are zero, and zero times an
        // unwritten row must not make a NaN); the empty asm keeps each use of the loaded data below the barriers
        if constexpr (!F8) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            u32x4_t v = vr[i][k];
            asm volatile("" : "+v"(v));
            const u32x4_t zero = {0u, 0u, 0u, 0u};
            *(u32x4_t*)(vt + ((lane >> 3) + 8 * k) * kDvRowB + 16 * (lane & 7)) = ok[i][k] ? v : zero;
          }
        } else {
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            u32x4_t v = vr[i][k];
            asm volatile("" : "+v"(v));
            const float sc = ok[i][k] ? es[i][k] : 0.0f;
            uint32_t w[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[q], false);
              const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[q], true);
              w[2 * q] = pack_bf16x2(lo[0] * sc, lo[1] * sc);
              w[2 * q + 1] = pack_bf16x2(hi[0] * sc, hi[1] * sc);
            }
            uint8_t* dst = vt + ((lane >> 2) + 16 * k) * kDvRowB + 32 * (lane & 3);
            *(u32x4_t*)dst = u32x4_t{w[0], w[1], w[2], w[3]};
            *(u32x4_t*)(dst + 16) = u32x4_t{w[4], w[5], w[6], w[7]};
          }
        }
        const float f = dfac[t][hl];
        const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pr[i]);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vtr + 32 * d));
          const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vtr + 4 * kDvRowB + 32 * d));
          const bf16x8_t av = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
          const f32x4_t pvt =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
          acc[d] += f * pvt;
        }
      }
    }
  };
  if (FMT == LCA_MIXED_FP8 && cb < 7)
    run(std::true_type{});
  else
    run(std::false_type{});

  // the eight waves' sums: wave w < 4 finishes channel block 16 w of the 64
  f32x4_t* mg = (f32x4_t*)dvt[wave];
#pragma unroll
  for (int d = 0; d < 4; ++d) mg[d * 64 + lane] = acc[d];
  __syncthreads();
  if (wave >= 4) return;
  f32x4_t o = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int w = 0; w < kDvWaves; ++w) o += ((const f32x4_t*)dvt[w])[wave * 64 + lane];
  const long long oi = ((long long)qrow * 64 + 16 * hg + hl) * 512 + 64 * cb + 16 * wave + 4 * grp;
  if (a.out_format == LCA_F32) {
    *(f32x4_t*)((float*)a.out + oi) = o;
  } else {
    uint2 w2;
    w2.x = pack_bf16x2(o[0], o[1]);
    w2.y = pack_bf16x2(o[2], o[3]);
    *(uint2*)((uint16_t*)a.out + oi) = w2;
  }
}

// ------------------------------------------------------------------------------------------------
// sparse decode attention in one pass per 64-entry tile, then the merge (few query rows, H = 64, D = 512)
// ------------------------------------------------------------------------------------------------
// One workgroup per (query row, 64 list positions), all 64 heads.  Since K = V = the entry, the tile that the
// scores were computed from is still in LDS when its probabilities are known, so the same workgroup forms the
// tile's partial output:
//   S^T = scale * K Q^T on v_mfma_f32_16x16x32_bf16: queries (64 KB) and entries are copied into LDS with
//   row-contiguous global_load_lds (1 KB per instruction, 16-byte chunks XOR-swizzled by row so that operand reads
//   are conflict-free), wave w contracts channels [128 (w % 4), + 128) of entries [32 (w / 4), + 32) for all heads
//   (fp8 entries widened exactly, the entry scale applied to their part), and the four channel quarters are added
//   in LDS in a fixed order;
//   m = the tile's max per head, P = e^(S - m) (0 for padding), l = sum P;
//   O^T = V^T P^T on v_mfma_f32_16x16x32_bf16, wave w taking channels [64 w, 64 w + 64) of all heads; V^T is read
//   with ds_read_b64_tr_b16 from the tile's bf16 rows (the mixed format's fp8 part widened and multiplied by the
//   entry scale into bf16 rows first), P^T from LDS in the operand layout;
//   O (bf16) and (m, l) go to the split partials, and attn_merge_kernel folds the tiles and the sink with LSE
//   weights.
// Against two passes (scores for the whole list, then values weighted by the exact normaliser) this saves a launch
// and the second gather of every entry, for a merge over 64 KB of bf16 partials per tile.
constexpr int kDfRowB = 1040;  // LDS bytes per head row of the output staging (1024 + 16)

template <int FMT>
__global__ __launch_bounds__(64 * kDsWaves) void attn_dec_fused_kernel(AttnArgs a) {
  constexpr bool MX = FMT == LCA_MIXED_FP8;
  // LDS: [0, 64 KB) the queries, then the channel partials 0-3, then (mixed) the widened value rows, then the output
  // staging (64 head rows of kDfRowB bytes, reaching into the entry area once that is dead); the entries (bf16: 1 KB
  // rows, 16-byte chunk c of row r at chunk c ^ (r % 16); mixed: 448 fp8 bytes, 128 RoPE bytes, 16 bytes of padding);
  // (mixed) the RoPE partials; P^T as [entry block][head block][64 lanes] x 16 bytes.
  constexpr int KROW = MX ? 592 : 1024;
  constexpr int kEnt = 65536;
  constexpr int kRope = kEnt + kDsTile * KROW;
  constexpr int kP = kRope + (MX ? 16384 : 0);
  __shared__ __attribute__((aligned(16))) uint8_t df_lds[kP + 8192];
  __shared__ uint8_t df_ok[kDsTile];
  __shared__ __attribute__((aligned(16))) float df_esc[kDsTile];
  static_assert(64 * kDfRowB <= kEnt + kDsTile * KROW, "output staging");
  uint8_t* const qs = df_lds;
  uint8_t* const kt = df_lds + kEnt;
  const int qrow = blockIdx.x, tile = blockIdx.y;
  const int b = qrow / a.Sq, r = qrow - b * a.Sq;
  const RowList L = row_list(a, b, r);
  const int total = L.nw + L.nc;
  const int p0 = tile * kDsTile;  // a tile past the row's list runs with every position masked: O = 0, m = -inf
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int hl = lane & 15, grp = lane >> 4;
  const long long item = (long long)qrow * a.n_splits + tile;

  // lane e of every wave resolves tile entry e: its tensor row (row 0 of the compressed tensor for padding), whether
  // it is a window entry and whether it is real; the copies below take these by readlane / ds_bpermute (the index
  // load is unconditional -- a read of the sink array where there is no index -- and its value is used only after
  // the query copies are issued, so that they are not held up by it)
  const int pl = p0 + lane;
  const bool rwl = pl < L.nw;
  const bool sel = !rwl && pl < total;
  const int xl = *(sel ? a.idx + ((long long)qrow * a.k + (pl - L.nw)) : (const int*)a.sink);
  {
    const uint8_t* qg = (const uint8_t*)a.q + (long long)qrow * 65536;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int h = 8 * wave + i;
      __builtin_amdgcn_global_load_lds((const void*)(qg + h * 1024 + 16 * (lane ^ (h & 15))), (void*)(qs + h * 1024),
                                       16, 0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm8);  // the index load has landed; the eight query copies may still be in flight
  __builtin_amdgcn_sched_barrier(0);
  const int rowl = rwl ? (int)(L.w0 + pl - L.raw0) : ((sel & (xl >= 0) & (xl < a.N)) ? xl : -1);
  const bool okl = rowl >= 0;
  const long long rabsl = rwl ? (long long)b * a.raw.cap + rowl : tensor_row(a.comp, b, okl ? rowl : 0);
  const int rlo = (int)rabsl, rhi = (int)(rabsl >> 32), rwi = rwl ? 1 : 0;
  if constexpr (!MX) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = 8 * wave + i;
      const long long rabs = ((long long)__builtin_amdgcn_readlane(rhi, e) << 32) |
                             (uint32_t)__builtin_amdgcn_readlane(rlo, e);
      const uint8_t* src = (const uint8_t*)(__builtin_amdgcn_readlane(rwi, e) ? a.raw.data : a.comp.data) +
                           rabs * 1024 + 16 * (lane ^ (e & 15));
      __builtin_amdgcn_global_load_lds((const void*)src, (void*)(kt + e * 1024), 16, 0, 0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int j = wave + 8 * i;
      const int sl = 64 * min(j, 36) + lane, e = sl / 37, c = sl - 37 * e;
      const long long rabs = ((long long)__builtin_amdgcn_ds_bpermute(4 * e, rhi) << 32) |
                             (uint32_t)__builtin_amdgcn_ds_bpermute(4 * e, rlo);
      const bool rw = __builtin_amdgcn_ds_bpermute(4 * e, rwi) != 0;
      const uint8_t* fb = (const uint8_t*)(rw ? a.raw.data : a.comp.data) + rabs * 448;
      const uint8_t* rb = (const uint8_t*)(rw ? a.raw.rope : a.comp.rope) + rabs * 128;
      const uint8_t* g = c < 28 ? fb + 16 * c : c < 36 ? rb + 16 * (c - 28) : fb;
      if (j < 37) __builtin_amdgcn_global_load_lds((const void*)g, (void*)(kt + 1024 * j), 16, 0, 0);
    }
  }
  if (wave == 0) {
    df_ok[lane] = okl ? 1 : 0;
    if constexpr (MX) {
      const long long rabs = ((long long)rhi << 32) | (uint32_t)rlo;
      df_esc[lane] = (rwi ? (const float*)a.raw.scale : (const float*)a.comp.scale)[rabs];
    }
  }
  __syncthreads();  // every copy has landed

  // S^T: wave (cs, eh) takes channels [128 cs, 128 cs + 128) of entries [32 eh, 32 eh + 32) for all 64 heads
  const int cs = wave & 3, eh = wave >> 2;
  f32x4_t acc[2][4], accr[2][4];
#pragma unroll
  for (int eb = 0; eb < 2; ++eb)
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      acc[eb][hb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      accr[eb][hb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int c = 16 * cs + 4 * ks + grp;
    bf16x8_t qb[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
      qb[hb] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(qs + (16 * hb + hl) * 1024 + 16 * (c ^ hl)));
#pragma unroll
    for (int eb = 0; eb < 2; ++eb) {
      const int e = 32 * eh + 16 * eb + hl;
      if constexpr (!MX) {
        const bf16x8_t kv = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(kt + e * 1024 + 16 * (c ^ hl)));
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          acc[eb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qb[hb], acc[eb][hb], 0, 0, 0);
      } else if (128 * cs + 32 * ks < 448) {
        const uint2 f = *(const uint2*)(kt + e * KROW + 8 * c);
        const uint2 lo = fp8x4_to_bf16x4(f.x), hi = fp8x4_to_bf16x4(f.y);
        const bf16x8_t kv = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          acc[eb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qb[hb], acc[eb][hb], 0, 0, 0);
      } else {
        const bf16x8_t kv = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(kt + e * KROW + 448 + 16 * (c - 56)));
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          accr[eb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qb[hb], accr[eb][hb], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // the queries are dead: the channel partials go over them
  // partials [slot][entry block 2 eh + eb][head block][lane]: slot = channel quarter; mixed: the RoPE part apart
  f32x4_t* part = (f32x4_t*)qs;
  f32x4_t* partr = (f32x4_t*)(df_lds + kRope);
#pragma unroll
  for (int eb = 0; eb < 2; ++eb)
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      part[((cs * 4 + 2 * eh + eb) * 4 + hb) * 64 + lane] = acc[eb][hb];
      if constexpr (MX)
        if (cs == 3) partr[((2 * eh + eb) * 4 + hb) * 64 + lane] = accr[eb][hb];
    }
  if constexpr (!MX) {
    // padding rows of the value tile become zero (their probabilities are zero, and zero times an unloaded row must
    // not make a NaN): wave w clears its own rows 8 w .. 8 w + 7
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = 8 * wave + i;
      if (!df_ok[e]) *(u32x4_t*)(kt + e * 1024 + 16 * lane) = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  __syncthreads();

  // thread (head h, group g) finishes entries 8 g .. 8 g + 7 of head h
  const int h = tid >> 3, g = tid & 7;
  const int blk = g >> 1, l0 = 32 * (g & 1) + (h & 15), hb = h >> 4;
  float sv[8];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int l = l0 + 16 * half;
    f32x4_t sm = (part[((0 * 4 + blk) * 4 + hb) * 64 + l] + part[((1 * 4 + blk) * 4 + hb) * 64 + l]) +
                 (part[((2 * 4 + blk) * 4 + hb) * 64 + l] + part[((3 * 4 + blk) * 4 + hb) * 64 + l]);
    if constexpr (MX) sm = sm * *(const f32x4_t*)&df_esc[8 * g + 4 * half] + partr[(blk * 4 + hb) * 64 + l];
#pragma unroll
    for (int x = 0; x < 4; ++x) sv[4 * half + x] = a.scale * sm[x];
  }
  // the tile's max per head (the 8 groups of a head are 8 neighbouring lanes), probabilities and sum
  float mt = -INFINITY;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (df_ok[8 * g + j]) mt = fmaxf(mt, sv[j]);
  mt = fmaxf(mt, __shfl_xor(mt, 1));
  mt = fmaxf(mt, __shfl_xor(mt, 2));
  mt = fmaxf(mt, __shfl_xor(mt, 4));
  float pv[8], ls = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    pv[j] = df_ok[8 * g + j] ? __expf(sv[j] - mt) : 0.0f;
    ls += pv[j];
  }
  ls += __shfl_xor(ls, 1);
  ls += __shfl_xor(ls, 2);
  ls += __shfl_xor(ls, 4);
  // P^T operand of entry block g / 4, head block h / 16: lane 16 (g % 4) + h % 16 holds entries 8 g .. 8 g + 7
  u32x4_t* const pt = (u32x4_t*)(df_lds + kP);
  pt[((g >> 2) * 4 + hb) * 64 + 16 * (g & 3) + (h & 15)] =
      u32x4_t{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
              pack_bf16x2(pv[6], pv[7])};
  if (g == 0) ((float2*)a.part_ml)[item * 64 + h] = make_float2(mt, ls);
  __syncthreads();  // the channel partials are read and P^T is written

  uint8_t* vbase = kt;
  if constexpr (MX) {
    // the value rows in bf16 over the dead partials: thread t widens chunks (t % 8) + 8 i of entry t / 8 (fp8 times
    // the entry scale; padding rows zero), stored at chunk c ^ (e % 16) of a 1 KB row
    const int e = tid >> 3;
    const float sc = df_ok[e] ? df_esc[e] : 0.0f;
    const uint8_t* src = kt + e * KROW;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = (tid & 7) + 8 * i;
      u32x4_t w;
      if (c < 56) {
        const uint2 f = *(const uint2*)(src + 8 * c);
        const f32x2_t a0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)f.x, false);
        const f32x2_t a1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)f.x, true);
        const f32x2_t a2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)f.y, false);
        const f32x2_t a3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)f.y, true);
        w = u32x4_t{pack_bf16x2(a0[0] * sc, a0[1] * sc), pack_bf16x2(a1[0] * sc, a1[1] * sc),
                    pack_bf16x2(a2[0] * sc, a2[1] * sc), pack_bf16x2(a3[0] * sc, a3[1] * sc)};
      } else {
        const u32x4_t v = *(const u32x4_t*)(src + 448 + 16 * (c - 56));
        const u32x4_t zero = {0u, 0u, 0u, 0u};
        w = df_ok[e] ? v : zero;
      }
      *(u32x4_t*)(qs + e * 1024 + 16 * (c ^ (e & 15))) = w;
    }
    __syncthreads();
    vbase = qs;
  }

  // O^T += V^T P^T: wave w, channels 64 w + 16 dt + 4 grp + x (dt < 4) of head 16 hb + hl in oacc[hb][dt].  The A
  // operand's K slots 8 grp .. 8 grp + 7 are entries 8 grp .. 8 grp + 7 of the entry block, as in P^T: lane (hl, grp)
  // addresses rows R1 = 8 grp + hl / 4 and R2 = R1 + 4 at bytes 8 (hl % 4) + 32 dt + 128 w, so ds_read_b64_tr_b16
  // hands lane 4 a + e of the group channel 4 a + e of four consecutive entries.  Logical chunk C of row R sits at
  // chunk C ^ (R % 16); dt flips chunk bits 1-2, which the lane's chunk at dt = 0 leaves clear.
  f32x4_t oacc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[i][dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  {
    const int r1 = 8 * grp + (hl >> 2), r2 = r1 + 4;
    const int cb = ((hl & 3) >> 1) + 8 * wave;
    const uint8_t* vp1 = vbase + r1 * 1024 + 8 * (hl & 1);
    const uint8_t* vp2 = vbase + r2 * 1024 + 8 * (hl & 1);
    const int vc1 = 16 * (cb ^ (r1 & 15)), vc2 = 16 * (cb ^ (r2 & 15));
#pragma unroll
    for (int eb = 0; eb < 2; ++eb) {
      bf16x8_t pb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[i] = __builtin_bit_cast(bf16x8_t, pt[(eb * 4 + i) * 64 + lane]);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const s16x4_t v0 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vp1 + eb * 32 * 1024 + (vc1 ^ (32 * dt))));
        const s16x4_t v1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vp2 + eb * 32 * 1024 + (vc2 ^ (32 * dt))));
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int i = 0; i < 4; ++i)
          oacc[i][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[i], oacc[i][dt], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // every value and P^T read is done: the staging goes over the value rows
  // the tile's partial output in bf16 through LDS, so that each store writes a whole 1 KB head row
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      uint2 w2;
      w2.x = pack_bf16x2(oacc[i][dt][0], oacc[i][dt][1]);
      w2.y = pack_bf16x2(oacc[i][dt][2], oacc[i][dt][3]);
      *(uint2*)(qs + (16 * i + hl) * kDfRowB + 2 * (64 * wave + 16 * dt + 4 * grp)) = w2;
    }
  __syncthreads();
  uint8_t* const po = (uint8_t*)a.part_o + item * (64 * 512 * 2);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int head = 8 * wave + i;
    __builtin_nontemporal_store(*(const u32x4_t*)(qs + head * kDfRowB + 16 * lane), (u32x4_t*)(po + head * 1024 + 16 * lane));
  }
}

// ------------------------------------------------------------------------------------------------
// merge of splits + sink
// ------------------------------------------------------------------------------------------------
// One workgroup per (head, query row, sequence): combine the splits' (max, sum, o) with the sink.
constexpr int kMergeThreads = 128;
// bf16 partials of at most 16 splits over 512 channels: one wave per (head, row), eight channels per lane
__host__ __device__ inline bool merge_one_wave(const AttnArgs& a) {
  return a.part_bf16 && a.n_splits <= 16 && a.D == 512;
}
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(AttnArgs a) {
  extern __shared__ float wsplit[];  // [n_splits] weights e^(m_s - M)
  __shared__ float red[kMergeThreads / 64];
  __shared__ float stat[2];
  const int h = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int H = a.H, D = a.D, S = a.n_splits;
  const long long item0 = ((long long)b * a.Sq + r) * S;
  const float z = a.sink[h];
  if (merge_one_wave(a)) {
    // bf16 partials, at most 16 splits, one wave: lane t's eight channels of every split are loaded at once (a batch
    // of NS >= S loads, the last split's repeated), behind the splits' (max, sum); lane s < S forms split s's weight,
    // which the channel sums read from it by lane broadcast
    auto merge_wave = [&](auto NSC) {
      constexpr int NS = decltype(NSC)::value;
      const int tid = threadIdx.x;
      const long long sstride = (long long)H * D;
      const uint16_t* pb = (const uint16_t*)a.part_o + (item0 * H + h) * D + 8 * tid;
      const float2 ml = ((const float2*)a.part_ml)[(item0 + min(tid, S - 1)) * H + h];
      uint4 pv[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) pv[s] = *(const uint4*)(pb + min(s, S - 1) * sstride);
      const float ms = tid < S ? ml.x : -INFINITY;
      const float M = fmaxf(z, wave_max(ms));
      const float wgt = (M == -INFINITY || ms == -INFINITY) ? 0.0f : __expf(ms - M);
      const float den = wave_sum(tid < S ? wgt * ml.y : 0.0f) +
                        ((M == -INFINITY || z == -INFINITY) ? 0.0f : __expf(z - M));
      if (tid == 0 && a.lse)
        a.lse[((long long)b * a.Sq + r) * H + h] = (M == -INFINITY) ? -INFINITY : M + __logf(den);
      const float inv = den > 0.0f ? 1.0f / den : 0.0f;
      f32x4_t lo = {0.0f, 0.0f, 0.0f, 0.0f}, hi = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s < S) {
          const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), s));
          const uint4 w = pv[s];
          lo += ws * f32x4_t{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                             __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
          hi += ws * f32x4_t{__uint_as_float(w.z << 16), __uint_as_float(w.z & 0xFFFF0000u),
                             __uint_as_float(w.w << 16), __uint_as_float(w.w & 0xFFFF0000u)};
        }
      }
      lo *= inv;
      hi *= inv;
      const long long ob = (((long long)b * a.Sq + r) * H + h) * D + 8 * tid;
      if (a.out_format == LCA_F32) {
        *(f32x4_t*)((float*)a.out + ob) = lo;
        *(f32x4_t*)((float*)a.out + ob + 4) = hi;
      } else {
        *(uint4*)((uint16_t*)a.out + ob) = make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                                                      pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3]));
      }
    };
    if (S <= 8) merge_wave(std::integral_constant<int, 8>{});
    else merge_wave(std::integral_constant<int, 16>{});
    return;
  }
  if (a.part_bf16 && S <= 32 && D == 4 * kMergeThreads) {
    // bf16 partials, at most 32 splits: thread t's four channels of every split are loaded at once (in a batch of
    // NS >= S loads, the last split's repeated), behind the splits' (max, sum) (loaded unconditionally, so that the
    // wait for them does not cover the partials), and the weights are formed while the partials are in flight
    auto merge_bf16 = [&](auto NSC) {
      constexpr int NS = decltype(NSC)::value;
      const int tid = threadIdx.x;
      const long long sstride = (long long)H * D;
      const uint16_t* pb = (const uint16_t*)a.part_o + (item0 * H + h) * D + 4 * tid;
      const float2 ml = ((const float2*)a.part_ml)[(item0 + min(tid, S - 1)) * H + h];
      uint2 pv[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) pv[s] = *(const uint2*)(pb + min(s, S - 1) * sstride);
      const float ms = tid < S ? ml.x : -INFINITY;
      float mloc = wave_max(ms);
      if ((tid & 63) == 0) red[tid >> 6] = mloc;
      __syncthreads();
      float M = z;
      for (int i = 0; i < kMergeThreads / 64; ++i) M = fmaxf(M, red[i]);
      const float wgt = (M == -INFINITY || ms == -INFINITY) ? 0.0f : __expf(ms - M);
      if (tid < S) wsplit[tid] = wgt;
      float dloc = wave_sum(tid < S ? wgt * ml.y : 0.0f);
      __syncthreads();
      if ((tid & 63) == 0) red[tid >> 6] = dloc;
      __syncthreads();
      float den = (M == -INFINITY || z == -INFINITY) ? 0.0f : __expf(z - M);
      for (int i = 0; i < kMergeThreads / 64; ++i) den += red[i];
      if (tid == 0 && a.lse)
        a.lse[((long long)b * a.Sq + r) * H + h] = (M == -INFINITY) ? -INFINITY : M + __logf(den);
      const float inv = den > 0.0f ? 1.0f / den : 0.0f;
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s < S) {
          const uint2 w = pv[s];
          acc += wsplit[s] * f32x4_t{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                                     __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
        }
      }
      acc *= inv;
      const long long ob = (((long long)b * a.Sq + r) * H + h) * D + 4 * tid;
      if (a.out_format == LCA_F32) {
        *(f32x4_t*)((float*)a.out + ob) = acc;
      } else {
        uint2 w2;
        w2.x = pack_bf16x2(acc[0], acc[1]);
        w2.y = pack_bf16x2(acc[2], acc[3]);
        *(uint2*)((uint16_t*)a.out + ob) = w2;
      }
    };
    if (S <= 8) merge_bf16(std::integral_constant<int, 8>{});
    else if (S <= 16) merge_bf16(std::integral_constant<int, 16>{});
    else if (S <= 24) merge_bf16(std::integral_constant<int, 24>{});
    else merge_bf16(std::integral_constant<int, 32>{});
    return;
  }
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
  if ((D & 3) == 0) {
    // four channels per thread, eight (fp32) or sixteen (bf16) splits' loads in flight at a time
    const long long sstride = (long long)H * D;
    const float* po = a.part_o + (item0 * H + h) * D;
    const uint16_t* pb = (const uint16_t*)a.part_o + (item0 * H + h) * D;
    // split s's four channels c .. c + 3 (bf16 partials widened exactly); the format is a template flag of the loop
    // so that its loads carry no branch between them
    auto merge = [&](auto bfc) {
      constexpr bool BF = decltype(bfc)::value;
      auto part = [&](int s, int c) -> f32x4_t {
        if constexpr (BF) {
          const uint2 w = *(const uint2*)(pb + s * sstride + c);
          return f32x4_t{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                         __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
        } else {
          return *(const f32x4_t*)(po + s * sstride + c);
        }
      };
      constexpr int NB = BF ? 16 : 8;  // splits whose loads are in flight together
      for (int c = 4 * threadIdx.x; c < D; c += 4 * blockDim.x) {
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
        int s0 = 0;
        for (; s0 + NB <= S; s0 += NB) {
          f32x4_t v[NB];
#pragma unroll
          for (int u = 0; u < NB; ++u) v[u] = part(s0 + u, c);
#pragma unroll
          for (int u = 0; u < NB; ++u) acc += wsplit[s0 + u] * v[u];
        }
        for (; s0 < S; ++s0) acc += wsplit[s0] * part(s0, c);
        acc *= inv;
        if (a.out_format == LCA_F32) {
          *(f32x4_t*)((float*)a.out + ob + c) = acc;
        } else {
          uint2 w2;
          w2.x = pack_bf16x2(acc[0], acc[1]);
          w2.y = pack_bf16x2(acc[2], acc[3]);
          *(uint2*)((uint16_t*)a.out + ob + c) = w2;
        }
      }
    };
    if (a.part_bf16)
      merge(std::true_type{});
    else
      merge(std::false_type{});
    return;
  }
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

// The value pass with the smallest per-wave load round that holds a wave's nti tiles (at most 8 per round).
template <int FMT>
void launch_dec_value(int nti, dim3 grid, hipStream_t st, hipEvent_t ee, const AttnArgs& a) {
  const dim3 blk(64 * kDvWaves);
  switch (nti <= 1 ? 1 : nti >= 7 ? 8 : nti) {
    case 1: hipExtLaunchKernelGGL((attn_dec_value_kernel<FMT, 1>), grid, blk, 0, st, nullptr, ee, 0, a); break;
    case 2: hipExtLaunchKernelGGL((attn_dec_value_kernel<FMT, 2>), grid, blk, 0, st, nullptr, ee, 0, a); break;
    case 3: hipExtLaunchKernelGGL((attn_dec_value_kernel<FMT, 3>), grid, blk, 0, st, nullptr, ee, 0, a); break;
    case 4: hipExtLaunchKernelGGL((attn_dec_value_kernel<FMT, 4>), grid, blk, 0, st, nullptr, ee, 0, a); break;
    case 5: hipExtLaunchKernelGGL((attn_dec_value_kernel<FMT, 5>), grid, blk, 0, st, nullptr, ee, 0, a); break;
    case 6: hipExtLaunchKernelGGL((attn_dec_value_kernel<FMT, 6>), grid, blk, 0, st, nullptr, ee, 0, a); break;
    default: hipExtLaunchKernelGGL((attn_dec_value_kernel<FMT, 8>), grid, blk, 0, st, nullptr, ee, 0, a); break;
  }
}

bool attn_uses_mfma(int H, int D, int q_format, int kv_format) {
  return H == 64 && D == 512 && q_format == LCA_BF16 && (kv_format == LCA_BF16 || kv_format == LCA_MIXED_FP8);
}

hipError_t launch_attn(AttnArgs a, hipStream_t st, hipEvent_t eb, hipEvent_t ee) {
  const bool mfma = attn_uses_mfma(a.H, a.D, a.q_format, a.comp.format);
  dim3 grid((unsigned)a.n_splits, (unsigned)a.Sq, (unsigned)a.B);
  clear_stale_error();
  if (mfma && a.hg_mode == 3) {
    const dim3 sgrid((unsigned)(a.B * a.Sq), (unsigned)(a.dec_tiles / 2));
    const dim3 vgrid((unsigned)(a.B * a.Sq), 8u, 4u);
    const int nti = (a.dec_tiles + kDvWaves - 1) / kDvWaves;  // most tiles a value-pass wave takes
    if (a.comp.format == LCA_BF16) {
      hipExtLaunchKernelGGL(attn_dec_score_kernel<LCA_BF16>, sgrid, dim3(64 * kDsWaves), 0, st, eb, nullptr, 0, a);
      launch_dec_value<LCA_BF16>(nti, vgrid, st, ee, a);
    } else {
      hipExtLaunchKernelGGL(attn_dec_score_kernel<LCA_MIXED_FP8>, sgrid, dim3(64 * kDsWaves), 0, st, eb, nullptr, 0,
                            a);
      launch_dec_value<LCA_MIXED_FP8>(nti, vgrid, st, ee, a);
    }
  } else if (mfma && a.hg_mode == 4) {
    // one workgroup per (row, 64 list positions), bf16 partials, then the merge
    if (a.part_bf16 != 1 || a.n_splits > 32) return hipErrorInvalidValue;
    const dim3 fgrid((unsigned)(a.B * a.Sq), (unsigned)a.n_splits);
    if (a.comp.format == LCA_BF16)
      hipExtLaunchKernelGGL(attn_dec_fused_kernel<LCA_BF16>, fgrid, dim3(64 * kDsWaves), 0, st, eb, ee, 0, a);
    else
      hipExtLaunchKernelGGL(attn_dec_fused_kernel<LCA_MIXED_FP8>, fgrid, dim3(64 * kDsWaves), 0, st, eb, ee, 0, a);
  } else if (mfma && a.hg_mode == 2) {
    // mode 2 is chosen for the mixed cache only (dense HCA rows over a bf16 cache take the many-row kernel)
    if (a.comp.format != LCA_MIXED_FP8) return hipErrorInvalidValue;
    const hipError_t e = ensure_dyn_lds((const void*)attn_wide_kernel<LCA_MIXED_FP8>, (int)kWdLds);
    if (e != hipSuccess) return e;
    const dim3 wgrid((unsigned)(a.B * a.Sq * a.n_splits));
    hipExtLaunchKernelGGL(attn_wide_kernel<LCA_MIXED_FP8>, wgrid, dim3(kWdThreads), kWdLds, st, eb, ee, 0, a);
  } else if (mfma && a.hg_mode == 1) {
    hipError_t e = ensure_dyn_lds((const void*)attn_hgw_kernel<LCA_BF16>, (int)kHgwLds);
    if (e == hipSuccess) e = ensure_dyn_lds((const void*)attn_hgw_kernel<LCA_MIXED_FP8>, (int)kHgwLds);
    if (e != hipSuccess) return e;
    const int pairs = a.B * a.Sq * a.n_splits;
    const dim3 hgrid((unsigned)(((pairs + 7) / 8) * 32));
    if (a.comp.format == LCA_BF16)
      hipExtLaunchKernelGGL(attn_hgw_kernel<LCA_BF16>, hgrid, dim3(256), kHgwLds, st, eb, ee, 0, a, pairs);
    else
      hipExtLaunchKernelGGL(attn_hgw_kernel<LCA_MIXED_FP8>, hgrid, dim3(256), kHgwLds, st, eb, ee, 0, a, pairs);
  } else if (mfma) {
    hipError_t e = ensure_dyn_lds((const void*)attn_mfma_kernel<LCA_BF16>, (int)kMfmaLds);
    if (e == hipSuccess) e = ensure_dyn_lds((const void*)attn_mfma_kernel<LCA_MIXED_FP8>, (int)kMfmaLds);
    if (e != hipSuccess) return e;
    if (a.comp.format == LCA_BF16 && tensor_storage_rows(a.raw, a.B) * 1024 < (1ll << 31) &&
        tensor_storage_rows(a.comp, a.B) * 1024 < (1ll << 31)) {
      a.part_bf16 = 1;  // split partials in bf16, for this kernel and the merge after it
      hipExtLaunchKernelGGL(attn_pfs_kernel, grid, dim3(kPsThreads), 0, st, eb, ee, 0, a);
    }
    else if (a.comp.format == LCA_BF16)
      hipExtLaunchKernelGGL(attn_mfma_kernel<LCA_BF16>, grid, dim3(kAttnThreads), kMfmaLds, st, eb, ee, 0, a);
    else
      hipExtLaunchKernelGGL(attn_mfma_kernel<LCA_MIXED_FP8>, grid, dim3(kAttnThreads), kMfmaLds, st, eb, ee, 0, a);
  } else {
    hipExtLaunchKernelGGL(attn_simt_kernel, grid, dim3(256), 0, st, eb, ee, 0, a);
  }
  hipError_t e = hipGetLastError();
  // mode 3 writes the output itself; mode 4 always leaves partials
  if (e != hipSuccess || a.hg_mode == 3 || (a.n_splits == 1 && a.hg_mode != 4)) return e;
  const size_t lds = sizeof(float) * (size_t)a.n_splits;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)a.H, (unsigned)a.Sq, (unsigned)a.B),
                     dim3(merge_one_wave(a) ? 64 : kMergeThreads), lds, st, a);
  return hipGetLastError();
}

}  // namespace lca
