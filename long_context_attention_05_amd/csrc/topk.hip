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


// Inclusive scan over the block (1024 threads, one value each); `tot` receives the block total.
__device__ __forceinline__ int block_incl_scan(int v, int* wsum, int& tot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int n = __shfl_up(v, o, 64);
    if (lane >= o) v += n;
  }
  if (lane == 63) wsum[w] = v;
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
  return v + before;
}

template <bool kLds>
__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(SelArgs a) {
  extern __shared__ uint32_t keys_s[];
  __shared__ int hist[2048];
  __shared__ int wsum[kSelWaves];
  __shared__ int cnt[2][2][kSelWaves];
  __shared__ int found_bin, found_above;

  const int row = blockIdx.x;
  const int r = row % a.Sq;
  const long long t = a.q_start + r;
  long long nv = t / a.m;
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
  if (kLds) {
    for (int i = tid; i < nvis; i += kSelThreads) keys_s[i] = kg[i];
  }
  const uint32_t* K = kLds ? keys_s : kg;

  uint32_t prefix = 0, mask = 0;
  int need = k;
  const int shifts[3] = {21, 10, 0};
  const int nbits[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass], nb = 1 << nbits[pass];
    for (int i = tid; i < 2048; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < nvis; i += kSelThreads) {
      uint32_t key = K[i];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> sh) & (nb - 1)], 1);
    }
    __syncthreads();
    // bins in descending order: thread tid owns bins hi = 2047 - 2 tid and lo = hi - 1 (only nb bins exist)
    const int bhi = 2047 - 2 * tid, blo = bhi - 1;
    const int hh = bhi < nb ? hist[bhi] : 0;
    const int hl = blo < nb ? hist[blo] : 0;
    int tot;
    const int incl = block_incl_scan(hh + hl, wsum, tot);
    const int before = incl - hh - hl;
    if (before < need && before + hh >= need) {
      found_bin = bhi;
      found_above = before;
    } else if (before + hh < need && before + hh + hl >= need) {
      found_bin = blo;
      found_above = before + hh;
    }
    __syncthreads();
    prefix |= (uint32_t)found_bin << sh;
    mask |= (uint32_t)(nb - 1) << sh;
    need -= found_above;
    __syncthreads();
  }
  const uint32_t kappa = prefix;

  // entry-ordered compaction: keys > kappa, then the first `need` keys == kappa
  const int lane = tid & 63, w = tid >> 6;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int sel_run = 0, eq_run = 0, parity = 0;
  for (int base = 0; base < nvis && sel_run < k; base += kSelThreads) {
    const int i = base + tid;
    const uint32_t key = i < nvis ? K[i] : 0u;
    const bool gt = i < nvis && key > kappa;
    const bool eq = i < nvis && key == kappa;
    const uint64_t bgt = __ballot(gt), beq = __ballot(eq);
    if (lane == 0) {
      cnt[parity][0][w] = __popcll(bgt);
      cnt[parity][1][w] = __popcll(beq);
    }
    __syncthreads();
    int eq_before = eq_run, sel_before = sel_run, eq_acc = eq_run, sel_acc = sel_run;
    for (int x = 0; x < kSelWaves; ++x) {
      const int cg = cnt[parity][0][x], ce = cnt[parity][1][x];
      int take = need - eq_acc;
      take = take < 0 ? 0 : (take > ce ? ce : take);
      if (x == w) {
        eq_before = eq_acc;
        sel_before = sel_acc;
      }
      eq_acc += ce;
      sel_acc += cg + take;
    }
    const int eqrank = eq_before + __popcll(beq & lt_mask);
    const bool sel = gt || (eq && eqrank < need);
    const uint64_t bsel = __ballot(sel);
    if (sel) {
      const int pos = sel_before + __popcll(bsel & lt_mask);
      out[pos] = i;
      if (sout) sout[pos] = key_score(key);
    }
    eq_run = eq_acc;
    sel_run = sel_acc;
    parity ^= 1;
  }
}

static bool g_lds_attr_set = false;

hipError_t launch_topk(const SelArgs& a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  // the longest visible row decides the variant (rows of one call differ only by their causal limit)
  long long nv = (a.q_start + a.Sq - 1) / a.m;
  const int nvis_max = (int)(nv < a.N ? nv : a.N);
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
