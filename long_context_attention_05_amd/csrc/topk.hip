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
constexpr int kLdsKeys = 32768;  // 128 KB of keys in LDS
constexpr size_t kSelDynLds = (size_t)kLdsKeys * 4;


constexpr int kBorderCap = 2048;  // keys of the border bin kept in LDS for passes 2 and 3
constexpr int kPerThread = 8;     // entries per thread in the ordered compaction

// Exclusive scan over the block (1024 threads, one value each); `tot` receives the block total.
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int& tot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int n = __shfl_up(incl, o, 64);
    if (lane >= o) incl += n;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int before = 0;
  tot = 0;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    int x = wsum[i];
    if (i < w) before += x;
    tot += x;
  }
  __syncthreads();
  return before + incl - v;
}

// Finds, among 2048 histogram bins read in descending order, the bin holding the need-th largest key.
// Returns the bin; *above receives the number of keys in higher bins.
__device__ __forceinline__ int find_bin(const int* hist, int need, int* wsum, int* shared_pair) {
  const int tid = threadIdx.x;
  const int bhi = 2047 - 2 * tid, blo = bhi - 1;
  const int hh = hist[bhi], hl = hist[blo];
  int tot;
  const int before = block_excl_scan(hh + hl, wsum, tot);
  if (before < need && before + hh >= need) {
    shared_pair[0] = bhi;
    shared_pair[1] = before;
  } else if (before + hh < need && before + hh + hl >= need) {
    shared_pair[0] = blo;
    shared_pair[1] = before + hh;
  }
  __syncthreads();
  return shared_pair[0];
}

template <bool kLds>
__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(SelArgs a) {
  extern __shared__ uint32_t keys_s[];
  __shared__ int hist[2048];
  __shared__ uint32_t border[kBorderCap];
  __shared__ int wsum[kSelWaves];
  __shared__ int pair[2];
  __shared__ int border_n;

  const int row = blockIdx.x;
  const int r = row % a.Sq;
  const long long t = a.q_start + r;
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
    int gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      kk[j] = (i0 + j < nvis) ? K[i0 + j] : 0u;
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

static bool g_lds_attr_set = false;

hipError_t launch_topk(const SelArgs& a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  // the longest visible row decides the variant (rows of one call differ only by their causal limit)
  long long nv = (a.q_start + a.Sq - 1) / a.m;
  const int nvis_max = (int)(nv < a.N ? nv : a.N);
  clear_stale_error();
  if (nvis_max <= kLdsKeys) {
    if (!g_lds_attr_set) {
      hipError_t e = hipFuncSetAttribute((const void*)topk_select_kernel<true>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSelDynLds);
      if (e != hipSuccess) return e;
      g_lds_attr_set = true;
    }
    hipLaunchKernelGGL(topk_select_kernel<true>, dim3((unsigned)a.rows), dim3(kSelThreads), kSelDynLds, st, a);
  } else {
    hipLaunchKernelGGL(topk_select_kernel<false>, dim3((unsigned)a.rows), dim3(kSelThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace lca
