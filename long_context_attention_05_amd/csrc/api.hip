// api.hip -- the extern "C" entry points of liblca.so: host-side validation, workspace layout, dispatch.
// Every check runs before anything is enqueued, so an error return leaves the stream untouched.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "lca_internal.h"


namespace lca {

// (kernel, device) pairs whose LDS limit is raised: a fixed table, so that no call allocates host memory either.
// A pair that does not fit is set again on every launch (the attribute call is idempotent).
hipError_t ensure_dyn_lds(const void* kernel, int bytes) {
  struct Done {
    const void* kernel;
    int device, bytes;
  };
  constexpr int kMaxDone = 1024;
  static std::mutex mu;
  static Done done[kMaxDone];
  static int n_done = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < n_done; ++i)
    if (done[i].kernel == kernel && done[i].device == dev && done[i].bytes >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && n_done < kMaxDone) done[n_done++] = Done{kernel, dev, bytes};
  return e;
}

}  // namespace lca

// Scratch memory of indexer_score_topk_noalloc: one array per device (each device that runs the library holds its
// own copy until the process ends).  Host code never passes this name to a kernel: on the host it stands for no
// device address.  The device address comes from hipGetSymbolAddress, once per device (scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[LCA_NOALLOC_SCRATCH_BYTES];

using namespace lca;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Validates one tensor descriptor: format, dim, pointers and their alignment.
// A writer's rotation: the Sylvester-Hadamard matrix exists for powers of two; the mixed format keeps its RoPE
// channels apart, so a rotation across them is refused.
static bool rotation_ok(const lca_tensor& t) {
  if (!(t.flags & LCA_ROTATE_HADAMARD)) return true;
  return t.format != LCA_MIXED_FP8 && (t.dim & (t.dim - 1)) == 0;
}

int check_tensor(const lca_tensor& t, bool allow_fp4, bool allow_mixed, bool allow_paged = false) {
  if (t.dim <= 0 || t.cap <= 0 || !t.data || (t.flags & ~LCA_ROTATE_HADAMARD)) return LCA_ERR_INVALID_ARG;
  if (t.block_table) {
    if (!allow_paged) return LCA_ERR_INVALID_ARG;
    const long long br = t.block_rows;
    if (br <= 0 || (br & (br - 1)) || t.cap % br || t.pool_rows <= 0 || t.pool_rows % br || t.pool_rows >= (1ll << 31))
      return LCA_ERR_INVALID_ARG;
    if ((uintptr_t)t.block_table & 3u) return LCA_ERR_ALIGNMENT;
  }
  switch (t.format) {
    case LCA_F32:
    case LCA_BF16:
      break;
    case LCA_MIXED_FP8:
      if (!allow_mixed) return LCA_ERR_UNSUPPORTED;
      if (t.rope_dims <= 0 || t.rope_dims >= t.dim || !t.rope || !t.scale) return LCA_ERR_INVALID_ARG;
      if (!aligned16(t.rope) || ((uintptr_t)t.scale & 3u)) return LCA_ERR_ALIGNMENT;
      break;
    case LCA_FP4:
      if (!allow_fp4) return LCA_ERR_UNSUPPORTED;
      if (t.dim % kFp4Block != 0 || !t.scale) return LCA_ERR_INVALID_ARG;
      if ((uintptr_t)t.scale & 3u) return LCA_ERR_ALIGNMENT;
      break;
    default:
      return LCA_ERR_INVALID_ARG;
  }
  if (!aligned16(t.data)) return LCA_ERR_ALIGNMENT;
  return LCA_OK;
}

thread_local hipError_t t_last_hip = hipSuccess;

int hip_status(hipError_t e) {
  if (e != hipSuccess) t_last_hip = e;
  return e == hipSuccess ? LCA_OK : LCA_ERR_HIP;
}

// profiling hooks (per host thread): events stamped with the start and end of the indexer scoring kernel and of the
// attention kernels
thread_local hipEvent_t t_ev_begin = nullptr, t_ev_end = nullptr;
thread_local hipEvent_t t_attn_ev_begin = nullptr, t_attn_ev_end = nullptr;

// Split plan of the attention: rows = B * Sq query rows, each with up to max_entries list positions.
// mode 0: one workgroup per (row, split), all heads; 1 (head-group kernel): four workgroups of 16 heads per (row,
// split); 2 (wide kernel): one workgroup per (row, split) with the channels split over its waves.
// table: the kernel resolves a slice's rows into an LDS table of kHgSplitMax entries (every MFMA kernel), so no
// slice may be longer.
void attn_plan(int B, int Sq, int H, int max_entries, int mode, bool table, int& n_splits, int& split_len) {
  const long long rows = (long long)B * Sq;
  const long long unit = mode == 1 ? 64 : 32;
  long long ns = 1, len = max_entries > 0 ? max_entries : 1;
  if (rows < 256 && max_entries > 64) {
    const long long per_row = mode == 1 ? rows * (H / 16) : rows;
    const long long want = (256 + per_row - 1) / per_row;
    len = (max_entries + want - 1) / want;
    len = (len + unit - 1) / unit * unit;
    if (len < 64) len = 64;
  }
  if (table && len > kHgSplitMax) len = kHgSplitMax;
  ns = (max_entries + len - 1) / len;
  const long long max_splits = 4096;  // the merge keeps one weight per split in LDS
  if (ns > max_splits) {
    ns = max_splits;
    len = (max_entries + ns - 1) / ns;
    len = (len + unit - 1) / unit * unit;
    ns = (max_entries + len - 1) / len;
  }
  if (ns < 1) ns = 1;
  n_splits = (int)ns;
  split_len = (int)len;
}

// The kernel a call takes: few query rows on the MFMA path go to the two-pass decode kernels (sparse lists of up to
// kDecTwoPassMax positions), the one-pass decode kernel and the merge (up to kDecMaxEntries), the head-group kernel
// (longer sparse lists) or, for dense HCA lists over the mixed cache, the wide kernel.  Dense HCA lists over a bf16 cache take the many-row path (mode 0): its LDS ring keeps two
// tiles in flight where the wide kernel holds one in registers, and it splits the list the same way.
int attn_mode(int B, int Sq, int H, int D, int q_format, int kv_format, int hca_m, int max_entries) {
  if (!attn_uses_mfma(H, D, q_format, kv_format) || (long long)B * Sq >= 256) return 0;
  if (hca_m > 0) return kv_format == LCA_BF16 ? 0 : 2;
  return max_entries <= kDecTwoPassMax ? 3 : max_entries <= kDecMaxEntries ? 4 : 1;
}

// 64-entry tiles per row of the decode attention (in mode 4 each leaves one partial output), at least one
int dec_splits(int max_entries) { return max_entries > 0 ? (max_entries + 63) / 64 : 1; }
// 32-entry tiles per row of the two-pass probabilities: whole 64-entry score tiles
int dec_tiles(int max_entries) { return 2 * dec_splits(max_entries); }

size_t attn_ws_plan_size(int B, int Sq, int H, int D, int max_entries, int mode, bool table) {
  if (mode == 3) {  // probabilities [rows][H][tiles * 32] bf16 and (m, l) [rows][tiles][H] float2
    const size_t rows = (size_t)B * Sq, T = (size_t)dec_tiles(max_entries);
    return align_up(rows * H * T * 32 * sizeof(uint16_t)) + align_up(rows * T * H * 2 * sizeof(float));
  }
  if (mode == 4) {  // per 64-entry tile: a bf16 partial output [H][D] and (m, l) [H] float2
    const size_t items = (size_t)B * Sq * dec_splits(max_entries);
    return align_up(items * H * D * sizeof(uint16_t)) + align_up(items * H * 2 * sizeof(float));
  }
  int ns, len;
  attn_plan(B, Sq, H, max_entries, mode, table, ns, len);
  if (ns <= 1) return 0;
  const size_t items = (size_t)B * Sq * ns;
  return align_up(items * H * D * sizeof(float)) + align_up(items * H * 2 * sizeof(float));
}

// Enough for whichever kernel the call will take (the size query does not know the formats).
size_t attn_ws_size(int B, int Sq, int H, int D, int max_entries) {
  // many rows: the plan without a row-table cap (SIMT kernels) or with it (MFMA kernels split longer lists)
  size_t need = attn_ws_plan_size(B, Sq, H, D, max_entries, 0, false);
  const size_t tabled = attn_ws_plan_size(B, Sq, H, D, max_entries, 0, true);
  if (tabled > need) need = tabled;
  if (H == 64 && D == 512 && (long long)B * Sq < 256)  // the few-row kernels (see attn_mode)
    for (int mode = 0; mode <= 4; ++mode) {
      if ((mode == 3 && max_entries > kDecTwoPassMax) || (mode == 4 && max_entries > kDecMaxEntries)) continue;
      const size_t m = attn_ws_plan_size(B, Sq, H, D, max_entries, mode, true);
      if (m > need) need = m;
    }
  return need;
}

int run_attn(const void* q, int q_format, const lca_tensor& comp_in, int N, int hca_m, const lca_tensor& raw,
             long long raw_start, int S_raw, const int32_t* idx, int k, const float* sink, int B, int Sq, int H, int D,
             int window, float scale, long long q_start, void* out, int out_format, float* lse, void* ws,
             size_t ws_bytes, const lca_ragged* ragged, void* stream) {
  if (!q || !sink || !out) return LCA_ERR_INVALID_ARG;
  const long long* seq_pos = ragged ? ragged->pos : nullptr;
  if (seq_pos && ((uintptr_t)seq_pos & 7u)) return LCA_ERR_ALIGNMENT;
  if (B <= 0 || Sq <= 0 || H <= 0 || D <= 0 || window < 0 || N < 0 || q_start < 0) return LCA_ERR_INVALID_ARG;
  if (hca_m == 0 && (k < 0 || (k > 0 && !idx))) return LCA_ERR_INVALID_ARG;
  if (q_format != LCA_F32 && q_format != LCA_BF16) return LCA_ERR_INVALID_ARG;
  if (out_format != LCA_F32 && out_format != LCA_BF16) return LCA_ERR_INVALID_ARG;
  // a window-only call (the ratio-0 layer: no compressed entry can be attended) may leave kv_comp empty; the
  // kernels then take the window's tensor for both roles and never read a compressed row
  lca_tensor comp = comp_in;
  const bool no_comp = (hca_m == 0 && k == 0) || N == 0;
  if (no_comp && !comp.data) {
    if (window <= 0) return LCA_ERR_INVALID_ARG;
    comp = raw;
    N = 0;
  }
  int rc = check_tensor(comp, false, true, comp.data != raw.data);
  if (rc) return rc;
  if (window > 0) {
    rc = check_tensor(raw, false, true);
    if (rc) return rc;
    if (raw.format != comp.format || raw.dim != D || (raw.format == LCA_MIXED_FP8 && raw.rope_dims != comp.rope_dims))
      return LCA_ERR_INVALID_ARG;
    // every window position of every query must be inside the raw span
    long long first_w0 = q_start - window + 1;
    if (first_w0 < 0) first_w0 = 0;
    const long long last_t = q_start + Sq - 1;
    if (S_raw <= 0 || S_raw > raw.cap || first_w0 < raw_start || last_t >= raw_start + S_raw) return LCA_ERR_INVALID_ARG;
  }
  if (comp.dim != D || (long long)N > comp.cap) return LCA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out) || (idx && ((uintptr_t)idx & 3u)) || ((uintptr_t)sink & 3u))
    return LCA_ERR_ALIGNMENT;
  const bool mfma = attn_uses_mfma(H, D, q_format, comp.format);
  if (!mfma) {
    if (H > 64 || D > 512 || (long long)H * D > 8192) return LCA_ERR_UNSUPPORTED;
    if (comp.format == LCA_MIXED_FP8 && (D - comp.rope_dims) <= 0) return LCA_ERR_INVALID_ARG;
  } else if (comp.format == LCA_MIXED_FP8 && comp.rope_dims != 64) {
    return LCA_ERR_UNSUPPORTED;
  }
  const int max_entries = window + (hca_m > 0 ? N : k);
  const int mode = attn_mode(B, Sq, H, D, q_format, comp.format, hca_m, max_entries);
  int ns = 1, len = max_entries;
  if (mode == 4)
    ns = dec_splits(max_entries), len = 64;
  else if (mode != 3)
    attn_plan(B, Sq, H, max_entries, mode, mfma, ns, len);
  if (mfma && len > kHgSplitMax) return LCA_ERR_UNSUPPORTED;  // more than 4096 x 2048 list positions per row
  const size_t need = attn_ws_plan_size(B, Sq, H, D, max_entries, mode, mfma);
  if (need > 0 && (!ws || ws_bytes < need)) return LCA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return LCA_ERR_ALIGNMENT;  // split partials go out in 16-byte stores

  AttnArgs a{};
  a.q = q;
  a.q_format = q_format;
  a.comp = comp;
  a.raw = raw;
  a.N = N;
  a.raw_start = raw_start;
  a.S_raw = S_raw;
  a.idx = idx;
  a.k = k;
  a.hca_m = hca_m;
  a.sink = sink;
  a.B = B;
  a.Sq = Sq;
  a.H = H;
  a.D = D;
  a.window = window;
  a.scale = scale;
  a.q_start = q_start;
  a.out = out;
  a.out_format = out_format;
  a.lse = lse;
  a.seq_pos = seq_pos;
  a.n_splits = ns;
  a.split_len = len;
  a.hg_mode = mode;
  a.part_bf16 = (mode == 2 || mode == 4) ? 1 : 0;  // the wide and the one-pass decode kernels' partials are bf16
  if (mode == 3) {
    a.dec_tiles = dec_tiles(max_entries);
    a.dec_p = (uint16_t*)ws;
    a.dec_ml = (float*)((char*)ws + align_up((size_t)B * Sq * H * a.dec_tiles * 32 * sizeof(uint16_t)));
  } else if (mode == 4) {
    const size_t items = (size_t)B * Sq * ns;
    a.part_o = (float*)ws;
    a.part_ml = (float*)((char*)ws + align_up(items * H * D * sizeof(uint16_t)));
  } else if (ns > 1) {
    const size_t items = (size_t)B * Sq * ns;
    a.part_o = (float*)ws;
    a.part_ml = (float*)((char*)ws + align_up(items * H * D * sizeof(float)));
  }
  hipEvent_t eb = t_attn_ev_begin, ee = t_attn_ev_end;
  const int rh = hip_status(hook_pair(eb, ee, (hipStream_t)stream));
  if (rh) return rh;
  return hip_status(launch_attn(a, (hipStream_t)stream, eb, ee));
}

}  // namespace

extern "C" {

const char* lca_status_string(int status) {
  switch (status) {
    case LCA_OK:
      return "LCA_OK";
    case LCA_ERR_INVALID_ARG:
      return "LCA_ERR_INVALID_ARG: null pointer, bad size or inconsistent arguments";
    case LCA_ERR_UNSUPPORTED:
      return "LCA_ERR_UNSUPPORTED: no kernel for this shape/format combination";
    case LCA_ERR_WORKSPACE:
      return "LCA_ERR_WORKSPACE: workspace missing or too small";
    case LCA_ERR_ALIGNMENT:
      return "LCA_ERR_ALIGNMENT: pointer not 16-byte aligned";
    case LCA_ERR_HIP:
      return "LCA_ERR_HIP: the HIP runtime rejected a launch";
    default:
      return "unknown lca status";
  }
}

int lca_encode(const float* src, int B, long long rows, long long row0, lca_tensor dst, void* stream) {
  if (!src || B <= 0 || rows < 0 || row0 < 0) return LCA_ERR_INVALID_ARG;
  int rc = check_tensor(dst, true, true, true);
  if (rc) return rc;
  if (row0 + rows > dst.cap) return LCA_ERR_INVALID_ARG;
  if (dst.dim > 1024) return LCA_ERR_UNSUPPORTED;
  if (!rotation_ok(dst)) return LCA_ERR_INVALID_ARG;
  if (rows == 0) return LCA_OK;
  return hip_status(launch_encode(src, B, rows, row0, dst, (hipStream_t)stream));
}

int kv_compress(const float* Ca, const float* Cb, const float* Za, const float* Zb, const float* Ba, const float* Bb,
                const float* tail_Cb, const float* tail_Zb, int B, long long n, int c, int m, int overlap,
                long long start_pos, const lca_epilogue* epi, const lca_ragged* ragged, lca_tensor out,
                void* stream) {
  if (!Ca || !Za || !Ba || B <= 0 || n <= 0 || c <= 0 || m <= 0 || start_pos < 0) return LCA_ERR_INVALID_ARG;
  if (overlap && (!Cb || !Zb || !Bb)) return LCA_ERR_INVALID_ARG;
  if (start_pos % m != 0) return LCA_ERR_INVALID_ARG;
  const long long* seq_pos = ragged ? ragged->pos : nullptr;
  const int* seq_len = ragged ? ragged->len : nullptr;
  if ((seq_pos && ((uintptr_t)seq_pos & 7u)) || (seq_len && ((uintptr_t)seq_len & 3u))) return LCA_ERR_ALIGNMENT;
  // a ragged call's sequences may start anywhere up to start_pos: the tail is needed whenever any of them may be > 0
  const bool tail = overlap && (start_pos > 0 || seq_pos);
  if (overlap && start_pos > 0 && (!tail_Cb || !tail_Zb)) return LCA_ERR_INVALID_ARG;
  int rc = check_tensor(out, true, true, true);
  if (rc) return rc;
  if (out.dim != c) return LCA_ERR_INVALID_ARG;
  if (c > 1024) return LCA_ERR_UNSUPPORTED;
  if (!rotation_ok(out)) return LCA_ERR_INVALID_ARG;
  const long long nb = (n + m - 1) / m;
  if (start_pos / m + nb > out.cap) return LCA_ERR_INVALID_ARG;
  lca_epilogue e{nullptr, 0.0f, 0, 0.0f};
  if (epi) {
    e = *epi;
    if (e.rope_dims < 0 || (e.rope_dims & 1) || e.rope_dims > c) return LCA_ERR_INVALID_ARG;
    if (e.rope_dims > 0 && !(e.rope_base > 0.0f && e.rope_base < INFINITY)) return LCA_ERR_INVALID_ARG;
    if (e.norm_weight && !(e.norm_eps >= 0.0f && e.norm_eps < INFINITY)) return LCA_ERR_INVALID_ARG;
    if ((uintptr_t)e.norm_weight & 3u) return LCA_ERR_ALIGNMENT;
  }
  return hip_status(launch_compress(Ca, overlap ? Cb : nullptr, Za, overlap ? Zb : nullptr, Ba, overlap ? Bb : nullptr,
                                    tail ? tail_Cb : nullptr, tail ? tail_Zb : nullptr, B, n, c, m, overlap ? 1 : 0,
                                    start_pos, seq_pos, seq_len, e, out, (hipStream_t)stream));
}

const char* lca_last_hip_error(void) { return hipGetErrorString(t_last_hip); }

int lca_stream_read(const void* src, size_t bytes, uint32_t* out, int workgroups, void* stream) {
  if (!src || !out || bytes == 0 || bytes % 16 != 0 || workgroups <= 0 || workgroups > (1 << 20))
    return LCA_ERR_INVALID_ARG;
  if (!aligned16(src) || ((uintptr_t)out & 3u)) return LCA_ERR_ALIGNMENT;
  return hip_status(launch_stream_read(src, bytes, out, workgroups, (hipStream_t)stream));
}

void lca_set_score_events(void* ev_begin, void* ev_end) {
  t_ev_begin = (hipEvent_t)ev_begin;
  t_ev_end = (hipEvent_t)ev_end;
}

void lca_set_attn_events(void* ev_begin, void* ev_end) {
  t_attn_ev_begin = (hipEvent_t)ev_begin;
  t_attn_ev_end = (hipEvent_t)ev_end;
}

// Workspace of indexer_score_topk: the score keys [B * Sq][N]; for up to kDecodeMaxRows query rows per sequence
// (decode) also the select buffers of the decode path: per-row histograms, per-slice counts and candidate segments.
struct IdxWs {
  size_t keys, state, counts, cand, total;
};
constexpr long long kMaxMultiN = 1024LL * kSliceKeys;  // slices per row <= 1024, one per finishing thread

IdxWs idx_ws_layout(int B, int Sq, int N) {
  IdxWs l{};
  const size_t rows = (size_t)B * Sq;
  l.keys = 0;
  size_t off = align_up(rows * N * sizeof(uint32_t));
  if (Sq <= kDecodeMaxRows && N <= kMaxMultiN) {
    const size_t slots = ((size_t)N + kSliceKeys - 1) / kSliceKeys;
    l.state = off;
    off += align_up(rows * kSelStateInts * sizeof(int));
    l.counts = off;
    off += align_up(rows * slots * sizeof(int));
    l.cand = off;
    off += align_up(rows * N * sizeof(uint2));
  }
  l.total = off > kAlign ? off : kAlign;
  return l;
}

size_t indexer_score_topk_workspace_size(int B, int Sq, int N, int k) {
  (void)k;
  if (B <= 0 || Sq <= 0 || N <= 0) return kAlign;
  return idx_ws_layout(B, Sq, N).total;
}

namespace {

// Device address of this device's `scratch` array, looked up with the device current on its first use and kept.
hipError_t scratch_ptr(void** out) {
  constexpr int kMaxDevices = 256;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

}  // namespace

int indexer_score_topk(lca_tensor qI, const float* w, lca_tensor kI, int B, int Sq, int HI, int DI, int N, int m, int k,
                       long long q_start_pos, int32_t* idx_out, float* score_out, void* ws, size_t ws_bytes,
                       const lca_ragged* ragged, void* stream) {
  if (!w || !idx_out || B <= 0 || Sq <= 0 || HI <= 0 || DI <= 0 || N < 0 || m <= 0 || k <= 0 || q_start_pos < 0)
    return LCA_ERR_INVALID_ARG;
  const long long* seq_pos = ragged ? ragged->pos : nullptr;
  if (seq_pos && ((uintptr_t)seq_pos & 7u)) return LCA_ERR_ALIGNMENT;
  int rc = check_tensor(qI, true, false);
  if (rc) return rc;
  rc = check_tensor(kI, true, false, true);
  if (rc) return rc;
  // the kernels address query row r of sequence b at rows (b * Sq + r) * HI + h: the tensor must be exactly that
  if (qI.dim != DI || kI.dim != DI || qI.cap != (long long)Sq * HI || kI.cap < N) return LCA_ERR_INVALID_ARG;
  if ((qI.format == LCA_FP4) != (kI.format == LCA_FP4)) return LCA_ERR_UNSUPPORTED;
  if (HI > 64 || DI > 128) return LCA_ERR_UNSUPPORTED;
  if (((uintptr_t)w & 3u) || ((uintptr_t)idx_out & 3u) || (score_out && ((uintptr_t)score_out & 3u)))
    return LCA_ERR_ALIGNMENT;
  if (N > 0 && (!ws || ws_bytes < indexer_score_topk_workspace_size(B, Sq, N, k))) return LCA_ERR_WORKSPACE;
  if (N > 0 && !aligned16(ws)) return LCA_ERR_ALIGNMENT;  // keys, histograms and candidates are read 16 bytes at a time
  hipStream_t st = (hipStream_t)stream;
  const IdxWs L = idx_ws_layout(B, Sq, N > 0 ? N : 1);
  const bool multi = N > 0 && Sq <= kDecodeMaxRows && N <= kMaxMultiN &&
                     indexer_uses_decode_kernel(B, Sq, HI, DI, N, qI.format, kI.format);
  // the decode scorers read a paged key cache a wave's 64 keys at a time from at most two blocks, and the fp4 one
  // addresses the pool with 32-bit buffer offsets
  if (kI.block_table && N > 0 && indexer_uses_decode_kernel(B, Sq, HI, DI, N, qI.format, kI.format)) {
    if (kI.block_rows < 32) return LCA_ERR_UNSUPPORTED;
    if (kI.format == LCA_FP4 && kI.pool_rows * (DI / 2) >= (1ll << 31)) return LCA_ERR_UNSUPPORTED;
  }
  char* wsb = (char*)ws;
  int* state = multi ? (int*)(wsb + L.state) : nullptr;
  IdxArgs a{qI, kI, w, (uint32_t*)(wsb + L.keys), B, Sq, HI, DI, N, m, q_start_pos, seq_pos, state};
  if (N > 0) {
    if (state) {  // the decode scoring kernels add into the row histograms
      rc = hip_status(launch_sel_zero(state, B * Sq, st));
      if (rc) return rc;
    }
    hipEvent_t eb = t_ev_begin, ee = t_ev_end;
    rc = hip_status(hook_pair(eb, ee, st));
    if (rc) return rc;
    rc = hip_status(launch_indexer_scores(a, st, eb, ee));
    if (rc) return rc;
  }
  SelArgs s{(const uint32_t*)(wsb + L.keys), idx_out, score_out, B * Sq, Sq, N, m, k, q_start_pos, seq_pos, state,
            multi ? (int*)(wsb + L.counts) : nullptr, multi ? (uint2*)(wsb + L.cand) : nullptr};
  return hip_status(launch_topk(s, st));
}

int indexer_score_topk_noalloc(lca_tensor qI, const float* w, lca_tensor kI, int B, int Sq, int HI, int DI, int N, int m,
                               int k, long long q_start_pos, int32_t* idx_out, float* score_out,
                               const lca_ragged* ragged, void* stream) {
  if (B > 0 && Sq > 0 && N > 0 && indexer_score_topk_workspace_size(B, Sq, N, k) > (size_t)LCA_NOALLOC_SCRATCH_BYTES)
    return LCA_ERR_WORKSPACE;
  void* ws = nullptr;
  const int rc = hip_status(scratch_ptr(&ws));
  if (rc) return rc;
  // the same kernels as indexer_score_topk over the device's scratch array: every buffer that must start at zero
  // (the row histograms) is cleared by a fill kernel inside the call, the rest is written before it is read
  return indexer_score_topk(qI, w, kI, B, Sq, HI, DI, N, m, k, q_start_pos, idx_out, score_out, ws,
                            (size_t)LCA_NOALLOC_SCRATCH_BYTES, ragged, stream);
}

size_t sparse_mqa_attn_workspace_size(int B, int Sq, int H, int D, int max_entries) {
  return attn_ws_size(B, Sq, H, D, max_entries);
}

int sparse_mqa_attn(const void* q, int q_format, lca_tensor kv_comp, int N, lca_tensor kv_raw, long long raw_start_pos,
                    int S_raw, const int32_t* idx, int k, const float* sink, int B, int Sq, int H, int D, int window,
                    float scale, long long q_start_pos, void* out, int out_format, float* lse_out, void* ws,
                    size_t ws_bytes, const lca_ragged* ragged, void* stream) {
  return run_attn(q, q_format, kv_comp, N, 0, kv_raw, raw_start_pos, S_raw, idx, k, sink, B, Sq, H, D, window, scale,
                  q_start_pos, out, out_format, lse_out, ws, ws_bytes, ragged, stream);
}

size_t hca_attn_workspace_size(int B, int Sq, int H, int D, int max_entries) {
  return attn_ws_size(B, Sq, H, D, max_entries);
}

int hca_attn(const void* q, int q_format, lca_tensor kv_comp, int N, int m, lca_tensor kv_raw, long long raw_start_pos,
             int S_raw, const float* sink, int B, int Sq, int H, int D, int window, float scale,
             long long q_start_pos, void* out, int out_format, float* lse_out, void* ws, size_t ws_bytes,
             const lca_ragged* ragged, void* stream) {
  if (m <= 0) return LCA_ERR_INVALID_ARG;
  return run_attn(q, q_format, kv_comp, N, m, kv_raw, raw_start_pos, S_raw, nullptr, 0, sink, B, Sq, H, D, window,
                  scale, q_start_pos, out, out_format, lse_out, ws, ws_bytes, ragged, stream);
}

}  // extern "C"
