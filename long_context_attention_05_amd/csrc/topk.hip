// topk.hip -- stage 2b, exact top-k of the indexer scores (paper notes "DeepSeek-V4: Towards Highly Efficient
// Million-Token Context Intelligence", section 2.3 Indexer excerpt: top-k of min(k, visible) entries, k = 512 /
// 1024 per cosmocat page section 3 and 67808.cn explainer section 2).
//
// The selected set is the first k of the order (score descending, entry ascending); it is written in ascending
// entry order.  Scores arrive as order-preserving uint32 keys, so selection is an exact radix select:
//   three histogram passes over key bits [31:21], [20:10], [9:0] find the k-th largest key kappa and how many
//   entries equal to kappa are still needed; a final pass in entry order keeps every key > kappa and the first
//   `need` keys == kappa (lowest entries first), compacting the survivors with wave ballots.
// One 1024-thread workgroup per query row.  Rows up to kLdsKeys entries are staged once in LDS; longer rows are
// re-read from the workspace (L2-resident) on every pass.
#include "lca_device.h"
#include "lca_internal.h"

namespace lca {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kLdsKeys = kTopkLdsKeys;  // 128 KB of keys in LDS
constexpr size_t kSelDynLds = (size_t)kLdsKeys * 4;


constexpr int kBorderCap = 2048;  // keys of the border bin kept in LDS for passes 2 and 3
constexpr int kPerThread = 8;     // entries per thread in the ordered compaction (two 16-byte LDS reads)

// Workgroup barrier for LDS only: this wave's LDS operations complete before it, and no global load in flight is
// waited for (the caller waits for what it needs).
__device__ __forceinline__ void sel_lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((3 << 14) | (7 << 4) | 0xF);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier: LDS-only (LDSB) or a full __syncthreads.
template <bool LDSB>
__device__ __forceinline__ void sel_barrier() {
  if constexpr (LDSB) sel_lds_barrier();
  else __syncthreads();
}

// Exclusive scan over the block (1024 threads, one value each); `tot` receives the block total.
template <bool LDSB = false>
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int& tot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) wsum[w] = incl;
  sel_barrier<LDSB>();
  int before = 0;
  tot = 0;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    int x = wsum[i];
    if (i < w) before += x;
    tot += x;
  }
  sel_barrier<LDSB>();
  return before + incl - v;
}

// Finds, among 2048 histogram bins read in descending order, the bin holding the need-th largest key.
// Returns the bin; *above receives the number of keys in higher bins.
template <bool LDSB = false>
__device__ __forceinline__ int find_bin(const int* hist, int need, int* wsum, int* shared_pair) {
  const int tid = threadIdx.x;
  const int bhi = 2047 - 2 * tid, blo = bhi - 1;
  const int hh = hist[bhi], hl = hist[blo];
  int tot;
  const int before = block_excl_scan<LDSB>(hh + hl, wsum, tot);
  if (before < need && before + hh >= need) {
    shared_pair[0] = bhi;
    shared_pair[1] = before;
  } else if (before + hh < need && before + hh + hl >= need) {
    shared_pair[0] = blo;
    shared_pair[1] = before + hh;
  }
  sel_barrier<LDSB>();
  return shared_pair[0];
}

template <bool kLds>
__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(SelArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t keys_s[];
  __shared__ int hist[2048];
  __shared__ uint32_t border[kBorderCap];
  __shared__ int wsum[kSelWaves];
  __shared__ int pair[2];
  __shared__ int border_n;

  const int row = blockIdx.x;
  const int r = row % a.Sq;
  const long long t = seq_position(a.seq_pos, a.q_start, row / a.Sq) + r;
  const long long nv = t / a.m;
  const int nvis = (int)(nv < a.N ? nv : a.N);
  const int k = a.k;
  int32_t* out = a.idx_out + (long long)row * k;
  float* sout = a.score_out ? a.score_out + (long long)row * k : nullptr;
  const uint32_t* kg = a.keys + (long long)row * a.N;
  const int tid = threadIdx.x;

  if (nvis <= k) {  // every visible entry is selected
    for (int j = tid; j < k; j += kSelThreads) {
      out[j] = j < nvis ? j : -1;
      if (sout) sout[j] = j < nvis ? key_score(kg[j]) : -INFINITY;
    }
    return;
  }
  const uint32_t* K = kLds ? keys_s : kg;

  // pass 1 (key bits [31:21]) fused with staging the row in LDS
  for (int i = tid; i < 2048; i += kSelThreads) hist[i] = 0;
  if (tid == 0) border_n = 0;
  __syncthreads();
  for (int base = 0; base < nvis; base += kSelThreads * kPerThread) {
    uint32_t kv[kPerThread];  // eight independent loads in flight per thread
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int i = base + tid + kSelThreads * u;
      kv[u] = i < nvis ? kg[i] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int i = base + tid + kSelThreads * u;
      if (i < nvis) {
        if (kLds) keys_s[i] = kv[u];
        atomicAdd(&hist[kv[u] >> 21], 1);
      }
    }
  }
  __syncthreads();
  int need = k;
  const int b1 = find_bin(hist, need, wsum, pair);
  need -= pair[1];
  __syncthreads();

  // border bin: the keys sharing the 11-bit prefix b1
  for (int i = tid; i < 2048; i += kSelThreads) hist[i] = 0;
  for (int base = 0; base < nvis; base += kSelThreads * kPerThread) {
    uint32_t kv[kPerThread];
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int i = base + tid + kSelThreads * u;
      kv[u] = i < nvis ? K[i] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int i = base + tid + kSelThreads * u;
      if (i < nvis && (int)(kv[u] >> 21) == b1) {
        const int pos = atomicAdd(&border_n, 1);
        if (pos < kBorderCap) border[pos] = kv[u];
      }
    }
  }
  __syncthreads();
  const int nb = border_n;
  const bool in_lds = nb <= kBorderCap;
  const uint32_t* src = in_lds ? border : K;
  const int n_src = in_lds ? nb : nvis;

  // passes 2 (bits [20:10]) and 3 (bits [9:0]) over the border keys only
  uint32_t prefix = (uint32_t)b1 << 21, mask = 0xFFE00000u;
  for (int pass = 0; pass < 2; ++pass) {
    const int sh = pass == 0 ? 10 : 0;
    const uint32_t digit = pass == 0 ? 0x7FFu : 0x3FFu;
    for (int i = tid; i < n_src; i += kSelThreads) {
      const uint32_t key = src[i];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> sh) & digit], 1);
    }
    __syncthreads();
    const int bn = find_bin(hist, need, wsum, pair);
    need -= pair[1];
    prefix |= (uint32_t)bn << sh;
    mask |= digit << sh;
    __syncthreads();
    if (pass == 0) {
      for (int i = tid; i < 2048; i += kSelThreads) hist[i] = 0;
      __syncthreads();
    }
  }
  const uint32_t kappa = prefix;  // the k-th largest key; `need` of the keys equal to it are selected

  // entry-ordered compaction: every key > kappa, then the first `need` keys == kappa
  int sel_run = 0, eq_run = 0;
  for (int base = 0; base < nvis && sel_run < k; base += kSelThreads * kPerThread) {
    const int i0 = base + tid * kPerThread;
    uint32_t kk[kPerThread];
    if (kLds && i0 + kPerThread <= nvis) {
      // the thread's eight keys in two 16-byte LDS reads (eight 4-byte reads 32 bytes apart across the lanes would
      // each take eight times as long, their lanes meeting in the same banks)
      const uint4 x0 = *(const uint4*)(K + i0), x1 = *(const uint4*)(K + i0 + 4);
      kk[0] = x0.x, kk[1] = x0.y, kk[2] = x0.z, kk[3] = x0.w;
      kk[4] = x1.x, kk[5] = x1.y, kk[6] = x1.z, kk[7] = x1.w;
    } else {
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) kk[j] = (i0 + j < nvis) ? K[i0 + j] : 0u;
    }
    int gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const bool valid = i0 + j < nvis;
      gt += (valid && kk[j] > kappa) ? 1 : 0;
      eq += (valid && kk[j] == kappa) ? 1 : 0;
    }
    int tot;
    const int packed_before = block_excl_scan(gt | (eq << 16), wsum, tot);
    const int gt_before = packed_before & 0xFFFF, eq_before = packed_before >> 16;
    const int rem = need - eq_run > 0 ? need - eq_run : 0;
    int pos = sel_run + gt_before + (eq_before < rem ? eq_before : rem);
    int eq_seen = eq_run + eq_before;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int i = i0 + j;
      if (i >= nvis) break;
      bool sel = kk[j] > kappa;
      if (kk[j] == kappa) {
        sel = eq_seen < need;
        ++eq_seen;
      }
      if (sel) {
        out[pos] = i;
        if (sout) sout[pos] = key_score(kk[j]);
        ++pos;
      }
    }
    const int tot_gt = tot & 0xFFFF, tot_eq = tot >> 16;
    sel_run += tot_gt + (tot_eq < rem ? tot_eq : rem);
    eq_run += tot_eq;
  }
}

// ------------------------------------------------------------------------------------------------
// decode rows (up to kDecodeMaxRows queries per sequence): the scoring kernel has already built each row's
// histogram of key bits [31:21], so pass 1 is a read of 2048 counts instead of a pass over the keys.  Every pass over all the keys runs
// spread over many workgroups; one workgroup per row then works on a few thousand candidates only.
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void sel_zero_kernel(int* state) {
  int4* p = (int4*)(state + (long long)blockIdx.x * kSelStateInts);
  for (int i = threadIdx.x; i < kSelStateInts / 4; i += blockDim.x) p[i] = make_int4(0, 0, 0, 0);
}

hipError_t launch_sel_zero(int* state, int rows, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  clear_stale_error();
  hipLaunchKernelGGL(sel_zero_kernel, dim3((unsigned)rows), dim3(256), 0, st, state);
  return hipGetLastError();
}

__device__ __forceinline__ int sel_row_nvis(const SelArgs& a, int row) {
  const long long t = seq_position(a.seq_pos, a.q_start, row / a.Sq) + row % a.Sq;
  const long long nv = t / a.m;
  return (int)(nv < a.N ? nv : a.N);
}

// Each row is cut into slices of kSliceKeys entries, one 256-thread workgroup per slice.
//   topk_collect_kernel: every slice finds the border bin b1 from the row histogram and writes its keys with
//                        bin >= b1 (a superset of the selection: about k + |border| keys per row) in entry order to
//                        its candidate segment with the segment's length.
//   topk_finish_kernel:  one workgroup per row (a separate launch, so that every slice's writes are visible without
//                        cross-workgroup fences) reads the row histogram, gathers the segments, resolves bits
//                        [20:10] (pass 2) and [9:0] (pass 3) over the candidates and writes the output.
constexpr int kMbThreads = 256;
constexpr int kMbPerThread = kSliceKeys / kMbThreads;  // 16
constexpr int kCandCap = 6144;                         // candidates the finishing workgroup holds in registers

// Exclusive scan over a 256-thread block.
__device__ __forceinline__ int block256_excl_scan(int v, int* wsum, int& tot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int before = 0;
  tot = 0;
#pragma unroll
  for (int i = 0; i < kMbThreads / 64; ++i) {
    const int x = wsum[i];
    if (i < w) before += x;
    tot += x;
  }
  __syncthreads();
  return before + incl - v;
}

// Bin (of 2048, descending order) holding the need-th largest key; *above = keys in higher bins.  256 threads,
// thread t owning bins 2047 - 8t - j, j = 0..7.
__device__ __forceinline__ int find_bin256(const int* hist, int need, int* wsum, int* sh, int* above) {
  const int t = threadIdx.x;
  int loc[8], sum = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    loc[j] = hist[2047 - 8 * t - j];
    sum += loc[j];
  }
  int tot;
  int cum = block256_excl_scan(sum, wsum, tot);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (cum < need && cum + loc[j] >= need) {
      sh[0] = 2047 - 8 * t - j;
      sh[1] = cum;
    }
    cum += loc[j];
  }
  __syncthreads();
  *above = sh[1];
  return sh[0];
}

__global__ __launch_bounds__(kMbThreads) void topk_collect_kernel(SelArgs a) {
  __shared__ __attribute__((aligned(16))) int hist[kSelBins];
  __shared__ int wsum[kMbThreads / 64];
  __shared__ int sh[4];
  const int p = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  const int nvis = sel_row_nvis(a, row);
  const int k = a.k;
  const uint32_t* kg = a.keys + (long long)row * a.N;
  if (nvis <= k) return;  // the finishing kernel writes the whole row
  const int P = (nvis + kSliceKeys - 1) / kSliceKeys;
  if (p >= P) return;
  const int slots = (a.N + kSliceKeys - 1) / kSliceKeys;
  const int s0 = p * kSliceKeys, s1 = min(s0 + kSliceKeys, nvis);

  // thread t takes the slice's keys 16 t .. 16 t + 15 straight into registers (four 16-byte loads when all of them
  // are visible and the row starts 16-byte aligned), with the row histogram's loads in flight beside them
  const int j0 = s0 + kMbPerThread * tid;
  uint32_t kv[kMbPerThread];
  if ((a.N & 3) == 0 && j0 + kMbPerThread <= s1) {
#pragma unroll
    for (int u = 0; u < kMbPerThread / 4; ++u) {
      const uint4 x = *(const uint4*)(kg + j0 + 4 * u);
      kv[4 * u] = x.x;
      kv[4 * u + 1] = x.y;
      kv[4 * u + 2] = x.z;
      kv[4 * u + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int u = 0; u < kMbPerThread; ++u) kv[u] = j0 + u < s1 ? kg[j0 + u] : 0u;
  }
  const int* gh = a.sel_state + (long long)row * kSelStateInts;
  static_assert(kSelBins == 8 * kMbThreads, "eight consecutive bins per thread");
  const int4 h0 = *(const int4*)(gh + 8 * tid), h1 = *(const int4*)(gh + 8 * tid + 4);
  *(int4*)(hist + 8 * tid) = h0;
  *(int4*)(hist + 8 * tid + 4) = h1;
  __syncthreads();
  int above1;
  const int b1 = find_bin256(hist, k, wsum, sh, &above1);

  // this slice's keys with bin >= b1, in entry order
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < kMbPerThread; ++j) cnt += (j0 + j < s1 && (int)(kv[j] >> 21) >= b1) ? 1 : 0;
  int tot;
  int pos = block256_excl_scan(cnt, wsum, tot);
  uint2* seg = a.cand + (long long)row * a.N + s0;
#pragma unroll
  for (int j = 0; j < kMbPerThread; ++j) {
    const uint32_t key = kv[j];
    if (j0 + j < s1 && (int)(key >> 21) >= b1) seg[pos++] = make_uint2(key, (uint32_t)(j0 + j));
  }
  if (tid == 0) a.counts[(long long)row * slots + p] = tot;
}

// Segment of candidate j (row order): the last segment whose start offset is <= j.
__device__ __forceinline__ int cand_segment(const int* seg_off, int nseg, int j) {
  int lo = 0, hi = nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seg_off[mid] <= j) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The finishing workgroup: 1024 threads, so that one round of loads gathers up to kCandCap candidates (6 consecutive
// ones per thread), which stay in registers for the pass-3 count and the one round of the ordered compaction.
constexpr int kFinThreads = 1024;
constexpr int kFinPer = kCandCap / kFinThreads;  // 6
constexpr int kFinMaxSlices = kFinThreads;       // one slice count per thread

__global__ __launch_bounds__(kFinThreads) void topk_finish_kernel(SelArgs a) {
  __shared__ int hist[kSelBins];   // pass 1, then pass 3
  __shared__ int hist2[kSelBins];  // pass 2
  __shared__ int seg_off[kFinMaxSlices];
  __shared__ int wsum[kSelWaves];
  __shared__ int sh[2];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int nvis = sel_row_nvis(a, row);
  const int k = a.k;
  int32_t* out = a.idx_out + (long long)row * k;
  float* sout = a.score_out ? a.score_out + (long long)row * k : nullptr;
  if (nvis <= k) {  // every visible entry is selected
    const uint32_t* kg = a.keys + (long long)row * a.N;
    for (int j = tid; j < k; j += kFinThreads) {
      out[j] = j < nvis ? j : -1;
      if (sout) sout[j] = j < nvis ? key_score(kg[j]) : -INFINITY;
    }
    return;
  }
  const int P = (nvis + kSliceKeys - 1) / kSliceKeys;  // <= kFinMaxSlices (checked at launch)
  const int slots = (a.N + kSliceKeys - 1) / kSliceKeys;
  const int* gh = a.sel_state + (long long)row * kSelStateInts;
  // segment lengths and the pass-1 histogram, all loads in flight together
  const int c = tid < P ? a.counts[(long long)row * slots + tid] : 0;
  int hv[kSelBins / kFinThreads];
#pragma unroll
  for (int u = 0; u < kSelBins / kFinThreads; ++u) hv[u] = gh[tid + kFinThreads * u];
#pragma unroll
  for (int u = 0; u < kSelBins / kFinThreads; ++u) {
    hist[tid + kFinThreads * u] = hv[u];
    hist2[tid + kFinThreads * u] = 0;
  }
  int total;
  const int off = block_excl_scan(c, wsum, total);  // (its barriers also publish the histogram and the zeroed one)
  if (tid < P) seg_off[tid] = off;
  sel_lds_barrier();  // the segment offsets

  const uint2* cseg = a.cand + (long long)row * a.N;
  const bool in_regs = total <= kCandCap;
  auto load_cand = [&](int j) -> uint2 {
    const int sgm = cand_segment(seg_off, P, j);
    return cseg[(long long)sgm * kSliceKeys + (j - seg_off[sgm])];
  };
  // one round of candidate loads: thread t takes candidates 6 t .. 6 t + 5 (indices clamp to the last candidate and
  // are masked below), finding the segment of the first by a search and the others by walking forward, so that the
  // loads issue after one search; they stay in flight while pass 1 resolves from the row histogram behind LDS-only
  // barriers, and in registers for passes 2 and 3 and the ordered output
  const int j0 = kFinPer * tid;
  uint2 cv[kFinPer];
  if (in_regs) {
    int sgm = cand_segment(seg_off, P, min(j0, total - 1));
    int s_lo = seg_off[sgm], s_hi = sgm + 1 < P ? seg_off[sgm + 1] : total;
#pragma unroll
    for (int i = 0; i < kFinPer; ++i) {
      const int j = min(j0 + i, total - 1);
      while (j >= s_hi) {  // the next non-empty segment
        ++sgm;
        s_lo = s_hi;
        s_hi = sgm + 1 < P ? seg_off[sgm + 1] : total;
      }
      cv[i] = cseg[(long long)sgm * kSliceKeys + (j - s_lo)];
    }
  }
  const int b1 = find_bin<true>(hist, k, wsum, sh);
  int need = k - sh[1];
  // pass 2 over the candidates of the border bin b1
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < kFinPer; ++i)
      if (j0 + i < total && (int)(cv[i].x >> 21) == b1) atomicAdd(&hist2[(cv[i].x >> 10) & 0x7FFu], 1);
  } else {
    for (int j = tid; j < total; j += kFinThreads) {
      const uint32_t key = load_cand(j).x;
      if ((int)(key >> 21) == b1) atomicAdd(&hist2[(key >> 10) & 0x7FFu], 1);
    }
  }
#pragma unroll
  for (int u = 0; u < kSelBins / kFinThreads; ++u) hist[tid + kFinThreads * u] = 0;  // pass 3 counts
  __syncthreads();
  const int b2 = find_bin(hist2, need, wsum, sh);
  need -= sh[1];
  const uint32_t prefix12 = ((uint32_t)b1 << 21) | ((uint32_t)b2 << 10);

  // pass 3 over the keys sharing the 21-bit prefix
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < kFinPer; ++i)
      if (j0 + i < total && (cv[i].x & 0xFFFFFC00u) == prefix12) atomicAdd(&hist[cv[i].x & 0x3FFu], 1);
  } else {
    for (int j = tid; j < total; j += kFinThreads) {
      const uint32_t key = load_cand(j).x;
      if ((key & 0xFFFFFC00u) == prefix12) atomicAdd(&hist[key & 0x3FFu], 1);
    }
  }
  __syncthreads();
  const int b3 = find_bin(hist, need, wsum, sh);
  need -= sh[1];
  const uint32_t kappa = prefix12 | (uint32_t)b3;  // the k-th largest key; `need` of the keys equal to it are taken

  // ordered output: candidates > kappa, then the first `need` equal to kappa; thread t takes kFinPer consecutive
  // candidates of each round (one round, from registers, when the row has at most kCandCap candidates)
  int sel_run = 0, eq_run = 0;
  for (int base = 0; base < total && sel_run < k; base += kCandCap) {
    const int jb = base + j0;
    uint2 cw[kFinPer];
    int gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < kFinPer; ++j) {
      const bool v = jb + j < total;
      cw[j] = v ? (in_regs ? cv[j] : load_cand(jb + j)) : make_uint2(0u, 0u);
      gt += (v && cw[j].x > kappa) ? 1 : 0;
      eq += (v && cw[j].x == kappa) ? 1 : 0;
    }
    int ptot;
    const int packed = block_excl_scan(gt | (eq << 16), wsum, ptot);
    const int gt_before = packed & 0xFFFF, eq_before = packed >> 16;
    const int rem = need - eq_run > 0 ? need - eq_run : 0;
    int o = sel_run + gt_before + (eq_before < rem ? eq_before : rem);
    int eq_seen = eq_run + eq_before;
#pragma unroll
    for (int j = 0; j < kFinPer; ++j) {
      if (jb + j >= total) break;
      bool sel = cw[j].x > kappa;
      if (cw[j].x == kappa) {
        sel = eq_seen < need;
        ++eq_seen;
      }
      if (sel) {
        if (o < k) {  // always true for histograms consistent with the keys
          out[o] = (int32_t)cw[j].y;
          if (sout) sout[o] = key_score(cw[j].x);
        }
        ++o;
      }
    }
    const int tg = ptot & 0xFFFF, te = ptot >> 16;
    sel_run += tg + (te < rem ? te : rem);
    eq_run += te;
  }
}

hipError_t launch_topk(const SelArgs& a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  // the longest visible row decides the variant (q_start is the largest position of the call)
  long long nv = (a.q_start + a.Sq - 1) / a.m;
  const int nvis_max = (int)(nv < a.N ? nv : a.N);
  clear_stale_error();
  if (a.sel_state) {
    const int P = (nvis_max + kSliceKeys - 1) / kSliceKeys;
    if (P > kFinMaxSlices) return hipErrorInvalidValue;  // more than 4M entries per row
    if (nvis_max > a.k)
      hipLaunchKernelGGL(topk_collect_kernel, dim3((unsigned)P, (unsigned)a.rows), dim3(kMbThreads), 0, st, a);
    hipLaunchKernelGGL(topk_finish_kernel, dim3((unsigned)a.rows), dim3(kFinThreads), 0, st, a);
  } else if (nvis_max <= kLdsKeys) {
    const hipError_t e = ensure_dyn_lds((const void*)topk_select_kernel<true>, (int)kSelDynLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_select_kernel<true>, dim3((unsigned)a.rows), dim3(kSelThreads), kSelDynLds, st, a);
  } else {
    hipLaunchKernelGGL(topk_select_kernel<false>, dim3((unsigned)a.rows), dim3(kSelThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace lca
