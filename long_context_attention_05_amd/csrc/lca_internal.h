// lca_internal.h -- argument blocks and launchers shared between the entry points (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lca.h"
#include <hip/hip_ext.h>

namespace lca {

// Drops an error left in the runtime by an earlier, unrelated call, so that the status read after a launch
// belongs to that launch.
inline void clear_stale_error() {
  hipError_t e = hipGetLastError();
  (void)e;
}

// The profiling hook's event pair for one timed kernel: kept when both are set and st is not being captured into a
// graph (the hooks time eager launches only), else both null.  The timed kernel is launched with
// hipExtLaunchKernelGGL, which stamps the events with that dispatch's own start and end times.
inline hipError_t hook_pair(hipEvent_t& b, hipEvent_t& e, hipStream_t st) {
  if (!b || !e) {
    b = e = nullptr;
    return hipSuccess;
  }
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const hipError_t r = hipStreamIsCapturing(st, &cs);
  if (r != hipSuccess) return r;
  if (cs != hipStreamCaptureStatusNone) b = e = nullptr;
  return hipSuccess;
}

// Raises a kernel's dynamic LDS limit to `bytes` on the current device, once per (kernel, device); safe to call from
// several host threads at once (api.hip).
hipError_t ensure_dyn_lds(const void* kernel, int bytes);

// stage 1 + codec (compress.hip)
hipError_t launch_encode(const float* src, int B, long long rows, long long row0, const lca_tensor& dst,
                         hipStream_t st);
hipError_t launch_compress(const float* Ca, const float* Cb, const float* Za, const float* Zb, const float* Ba,
                           const float* Bb, const float* tCb, const float* tZb, int B, long long n, int c, int m,
                           int overlap, long long start_pos, const long long* seq_pos, const int* seq_len,
                           const lca_epilogue& epi, const lca_tensor& out, hipStream_t st);

// stage 2a, indexer scores (indexer.hip)
struct IdxArgs {
  lca_tensor q, k;
  const float* w;
  uint32_t* keys;  // [B][Sq][N] order-preserving score keys (workspace)
  int B, Sq, HI, DI, N, m;
  long long q_start;       // the largest query position of the call (row r of sequence b: seq_position + r)
  const long long* seq_pos;  // nullable [B]: each sequence's position (a ragged batch)
  int* sel_state;  // nullable: [B * Sq][kSelStateInts] row histograms the decode kernels add into (zeroed first)
};
// Decode kernels take up to this many query rows per sequence (one token, or a few draft tokens verified together):
// the rows of a sequence score the same keys side by side, so the key stream is read from memory about once.
// fp4 caches: one power-of-two (E8M0) scale per block of 32 consecutive elements -- the 1x32 FP4 sub-blocks with
// their own scale factors of the page "百万token成本暴降90%！DeepSeek-V4揭秘" (question 4), and the block one lane of
// a scaled MFMA applies its scale to.
constexpr int kFp4Block = 32;

constexpr int kDecodeMaxRows = 4;
// Rows of at most this many keys are selected from an LDS copy by the many-row top-k.
constexpr int kTopkLdsKeys = 32768;
// Whether launch_indexer_scores takes the decode kernels (which fill sel_state) for N entries per sequence.
bool indexer_uses_decode_kernel(int B, int Sq, int HI, int DI, int N, int q_format, int k_format);
// ev_begin / ev_end (nullable, from hook_pair): stamped with the scoring kernel's start and end.
hipError_t launch_indexer_scores(const IdxArgs& a, hipStream_t st, hipEvent_t ev_begin = nullptr,
                                 hipEvent_t ev_end = nullptr);

// stage 2b, exact top-k (topk.hip)
struct SelArgs {
  const uint32_t* keys;  // [rows][N]
  int32_t* idx_out;      // [rows][k]
  float* score_out;      // nullable [rows][k]
  int rows, Sq, N, m, k;
  long long q_start;
  const long long* seq_pos;  // nullable [rows / Sq]: each sequence's position (a ragged batch)
  // decode rows: the row histograms written by the scoring kernel, and the multi-workgroup select buffers; all null
  // for the select that makes its own histogram passes
  int* sel_state;  // [rows][kSelStateInts]: histograms of key bits [31:21] (all keys, from the scoring kernel)
  int* counts;     // [rows][slices]
  uint2* cand;     // [rows][N] (key, entry) candidates, slice s at [s * kSliceKeys]
};
constexpr int kSelBins = 2048;
constexpr int kSelStateInts = kSelBins;
constexpr int kSliceKeys = 4096;  // keys per workgroup in the multi-workgroup select
// Zeroes the row histograms [rows][kSelStateInts] (a fill kernel, so that it may be captured in a graph).
hipError_t launch_sel_zero(int* state, int rows, hipStream_t st);
hipError_t launch_topk(const SelArgs& a, hipStream_t st);

// stages 3/4, attention (attn.hip)
struct AttnArgs {
  const void* q;
  int q_format;
  lca_tensor comp, raw;
  int N;
  long long raw_start;
  int S_raw;
  const int32_t* idx;  // sparse mode: [B][Sq][k]
  int k;
  int hca_m;  // > 0: dense over the visible entries
  const float* sink;
  int B, Sq, H, D, window;
  float scale;
  long long q_start;
  const long long* seq_pos;  // nullable [B]: each sequence's position; its raw rows start at raw_start + seq_pos[b] -
                             // q_start
  void* out;
  int out_format;
  float* lse;
  int n_splits, split_len;
  float* part_o;   // [B][Sq][n_splits][H][D] fp32, or bf16 when part_bf16
  float* part_ml;  // [B][Sq][n_splits][H][2]
  int part_bf16;   // split partial outputs stored as bf16 (the wide and the many-row bf16 kernels: half the
                   // partial traffic); set by the launcher for the kernel it takes
  int hg_mode;     // 1: one workgroup per (16-head group, row, split); 2: one per (row, split) with the channels
                   // split over the waves; 3: scores then values in two passes; 4: one pass per (row, 64 list
                   // positions), partials always merged -- 3 and 4 for few rows (decode)
  // mode 3: the score pass's probabilities and per-tile (max, sum)
  int dec_tiles;     // 32-entry tiles per row (an even number: list capacity / 64, rounded up, times 2)
  uint16_t* dec_p;   // [B][Sq][H / 16][dec_tiles][64 lanes][8] bf16 probabilities e^(l - m_t), in the order the
                     // value pass loads its MFMA operand (lane 16 q + h % 16: entries 8 q .. 8 q + 7 of head h)
  float* dec_ml;     // [B][Sq][dec_tiles][H][2] (m_t, l_t)
};
constexpr int kDecMaxEntries = 2048;  // list positions per row in the decode attention (mode 4: 32 partials)
constexpr int kDecTwoPassMax = 512;   // lists up to this long take the two passes (mode 3), whose value pass grows
                                      // with the list where the one pass pays a fixed merge
constexpr int kHgSplitMax = 2048;  // list positions per workgroup slice in the MFMA attention kernels (LDS row table)
bool attn_uses_mfma(int H, int D, int q_format, int kv_format);
// ev_begin / ev_end (nullable, from hook_pair): stamped with the start of the attention's first kernel and the end of
// its last one before the merge of split partials.
hipError_t launch_attn(AttnArgs a, hipStream_t st, hipEvent_t ev_begin = nullptr, hipEvent_t ev_end = nullptr);

// measurement helper (measure.hip)
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* out, int workgroups, hipStream_t st);

}  // namespace lca
