/*
 * lca.h -- C ABI of the MI355X (gfx950) hybrid compressed attention library (liblca.so).
 *
 * The layer is the DeepSeek-V4 hybrid attention described on the pages:
 *   - "DeepSeek-V4: Towards Highly Efficient Million-Token Context Intelligence" (paper notes), section 2.3
 *     (CSA: Token-Level Compressor Eq. 11-12, Lightning Indexer Eq. 16, shared-KV MQA) and section 2.4
 *     (HCA, Eq. 22-23, Attention.forward fusing window + compressed entries in one sparse attention);
 *   - "百万token成本暴降90%！DeepSeek-V4揭秘", mechanisms 1-3 (128-token sliding window, overlapped
 *     compression, per-head attention sink) and question 4 (FP4);
 *   - "一个数量级是怎么省的" (cosmocat), sections 3-4 (indexer, top-k, bf16/fp8/fp4 cache, HCA);
 *   - 67808.cn explainer, sections 2-4 (overlap, 64x128 indexer in FP4, top-k <= 1024, HCA < 8000 entries
 *     at 1M tokens, window).
 *
 * Conventions shared by every call
 *   - Every pointer argument is a DEVICE pointer owned by the caller, except where a comment says host.
 *     The library never allocates, frees or synchronises: all work is enqueued on `stream` (a hipStream_t;
 *     NULL = the default stream) and the call returns once it is enqueued.
 *   - Tensors are dense and row-major.  Sequence b of a cache tensor occupies rows [b*cap, (b+1)*cap).
 *   - Every argument is validated on the host before anything is launched; on error nothing is enqueued
 *     and a negative lca_status is returned.  A failed launch returns LCA_ERR_HIP.  Faults inside a kernel
 *     surface at the caller's next synchronisation.
 *   - Positions are absolute token positions; query row r of a call is at q_start_pos + r for every sequence,
 *     unless the call takes a ragged batch (lca_ragged: each sequence at its own position).
 *   - Calls are deterministic: the same inputs give bit-identical outputs.  Calls that share a workspace must
 *     not overlap in time.
 */
#ifndef LCA_H
#define LCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LCA_OK = 0,
  LCA_ERR_INVALID_ARG = -1, /* null pointer, bad size, inconsistent shapes or positions          */
  LCA_ERR_UNSUPPORTED = -2, /* valid request that no kernel of this library implements           */
  LCA_ERR_WORKSPACE = -3,   /* ws NULL or ws_bytes smaller than the matching *_workspace_size    */
  LCA_ERR_ALIGNMENT = -4,   /* a pointer is not 16-byte aligned                                 */
  LCA_ERR_HIP = -5          /* the HIP runtime rejected a launch                                */
} lca_status;

/* Storage formats of a cache tensor (cosmocat page, section 3; Mind Observatory page: RoPE dims in
 * BF16, the rest in FP8, indexer keys in FP4). */
typedef enum {
  LCA_F32 = 0,       /* data: float   [rows][dim]                                                       */
  LCA_BF16 = 1,      /* data: uint16  [rows][dim] bfloat16 bits                                         */
  LCA_MIXED_FP8 = 2, /* data: uint8   [rows][dim - rope_dims] OCP fp8 e4m3 codes of x / s,              */
                     /* scale: float [rows] s = fl32(amax / 448) over those dims (1 if amax = 0),       */
                     /* rope: uint16 [rows][rope_dims] bfloat16 bits of the LAST rope_dims channels     */
  LCA_FP4 = 3        /* data: uint8   [rows][dim / 2] OCP fp4 e2m1 codes of x * 2^-e, element 2j in    */
                     /* the low nibble of byte j; scale: uint8 [rows][dim / 32] E8M0 byte e + 127, one  */
                     /* per block of 32 consecutive elements (dim a multiple of 32), e = smallest       */
                     /* integer with amax(block) <= 6 * 2^e (e = -127 if amax = 0)                      */
} lca_format;

/* Tensor flag LCA_ROTATE_HADAMARD (paper notes, the Indexer excerpt: the indexer's queries, and the keys of its own
 * compressor, are rotated by a Hadamard transform that spreads outliers before they are quantised to FP4).  The
 * rows hold rotated values: writers (lca_encode, kv_compress) multiply each fp32 row x by the orthonormal
 * Sylvester-Hadamard matrix of order dim, y[i] = sum_j (-1)^popcount(i & j) x[j] / sqrt(dim), before encoding.
 * dim must be a power of two and the format not LCA_MIXED_FP8.  Readers use the stored values as they are: the
 * rotation is orthogonal, so dot products of rotated queries and rotated keys equal the unrotated ones up to the
 * encoding.  The writers compute the transform in fp32 (log2(dim) butterfly stages, then one multiply by
 * 1/sqrt(dim) rounded to fp32). */
#define LCA_ROTATE_HADAMARD 1

/* One cache (or query) tensor: `cap` rows per sequence, each row one entry of `dim` channels.
 *
 * Dense tensor (block_table NULL): sequence b owns rows [b * cap, (b + 1) * cap) of the data / rope / scale arrays.
 * Paged tensor (block_table set; itsolotime page, question 5: the compressed cache is managed in fixed blocks of
 * lcm(4, 128) = 128 tokens, i.e. 32 CSA entries or one HCA entry per block): the arrays hold a pool of pool_rows rows
 * in blocks of block_rows rows, and row i of sequence b is pool row
 *     block_table[b * (cap / block_rows) + i / block_rows] * block_rows + i % block_rows.
 * block_table is a DEVICE int32 array [B][cap / block_rows] owned by the caller; its entries must name blocks inside
 * the pool (not checked: they are device data).  Compressed caches and indexer keys may be paged (kv_compress and
 * lca_encode write through the table; the indexer and the attention read through it); query tensors and the raw
 * window may not. */
typedef struct {
  int format;    /* lca_format                                                                       */
  int dim;       /* channels per row                                                                 */
  int rope_dims; /* LCA_MIXED_FP8 only: trailing channels kept in bf16 (0 < rope_dims < dim)         */
  long long cap; /* rows per sequence                                                                */
  void* data;    /* see lca_format                                                                   */
  void* rope;    /* LCA_MIXED_FP8 only, else NULL                                                    */
  void* scale;   /* LCA_MIXED_FP8 / LCA_FP4 only, else NULL                                          */
  int flags;     /* 0 or LCA_ROTATE_HADAMARD; other bits are INVALID_ARG                             */
  const int32_t* block_table; /* NULL: dense; else paged (see above)                                 */
  int block_rows;             /* paged: rows per block, a power of two dividing cap                  */
  long long pool_rows;        /* paged: rows in the pool arrays (a multiple of block_rows, < 2^31)  */
} lca_tensor;

/* A ragged batch: each sequence of a call at its own position.  All pointers are DEVICE arrays of B elements owned
 * by the caller; the struct itself is passed by a host pointer (NULL: every sequence at the call's uniform position).
 *   pos[b] replaces the call's position for sequence b: start_pos of kv_compress (a multiple of m), q_start_pos of
 *     indexer_score_topk, sparse_mqa_attn and hca_attn.  The call's uniform position must then be the largest pos[b]
 *     (it sizes the launch and the host-side checks).  In the attention, sequence b's raw window rows start at
 *     position raw_start_pos + pos[b] - q_start_pos (the same offset from its queries as the call's).
 *   len[b] (kv_compress only, nullable): tokens of sequence b among the n given, 1 <= len[b] <= n; entries
 *     [pos[b] / m, pos[b] / m + ceil(len[b] / m)) of sequence b are written. */
typedef struct {
  const long long* pos;
  const int* len;
} lca_ragged;

/* Human-readable name of a status code (static string). */
const char* lca_status_string(int status);

/* The HIP runtime's message for the last LCA_ERR_HIP returned on the calling host thread (static string). */
const char* lca_last_hip_error(void);

/*
 * lca_stream_read -- measurement helper, not part of the layer: reads `bytes` (a multiple of 16) of device memory at
 * `src` once with 16-byte loads spread over `workgroups` workgroups of 256 threads, and XORs what it read into
 * *out (uint32, device).  Timing it gives the read-stream rate that HBM-bound kernels are compared with, next to
 * the 8 TB/s peak.  Errors: INVALID_ARG (null, bytes 0 or not a multiple of 16, workgroups out of [1, 2^20]),
 * ALIGNMENT (src not 16-byte aligned, out not 4-byte aligned).
 */
int lca_stream_read(const void* src, size_t bytes, uint32_t* out, int workgroups, void* stream);

/*
 * lca_encode -- quantise-on-write: encode fp32 rows into a cache tensor's format (the codec of the
 * mixed-precision cache).  src: float [B][rows][dst.dim].  Writes rows [row0, row0 + rows) of every
 * sequence of dst (row0 + rows <= dst.cap).  Formats as described at lca_format; rounding is to nearest,
 * ties to even, for bf16, fp8 and fp4.
 * With LCA_ROTATE_HADAMARD in dst.flags each row is rotated first (see the flag).
 * Errors: INVALID_ARG (null, rows < 0, row0 < 0, row range beyond cap, fp4 dim % 16 != 0, bad rope_dims,
 *         a rotation with dim not a power of two or the mixed format), UNSUPPORTED (dim > 1024).
 */
int lca_encode(const float* src, int B, long long rows, long long row0, lca_tensor dst, void* stream);

/* Epilogues kv_compress applies to each fp32 entry, in this order, before the output flag's Hadamard rotation and the
 * encoding (paper notes, section 2.3: the Compressor normalises its entries with an RMSNorm over the head dim, and
 * the Indexer excerpt applies rotary position embedding to the trailing channels):
 *   norm_weight != NULL (device, float [c]): y[j] = x[j] / sqrt(mean_j(x[j]^2) + norm_eps) * norm_weight[j];
 *   rope_dims > 0 (even, <= c): channel pair (c - rope_dims + 2i, c - rope_dims + 2i + 1) of entry e (the absolute
 *     entry index) turns by the angle p * rope_base^(-2i / rope_dims) with p = m * e, the position of the first
 *     token of the entry's block: (a, b) -> (a cos - b sin, a sin + b cos).  The angle and its sine and cosine are
 *     computed in double precision, the rotation itself in fp32.
 * The RMS is reduced in fp32. */
typedef struct {
  const float* norm_weight; /* NULL: no normalisation                                                            */
  float norm_eps;           /* >= 0                                                                              */
  int rope_dims;            /* 0: no rotary embedding                                                            */
  float rope_base;          /* > 0 when rope_dims > 0                                                            */
} lca_epilogue;

/*
 * kv_compress -- stage 1, KV compression (paper notes section 2.3 Eq. 11-12 and the Compressor excerpt;
 * section 2.4 Eq. 22-23; itsolotime mechanism 2; 67808.cn section 2).
 * Entry i of a sequence merges the m tokens of block i: per channel j, a softmax over the candidates'
 * logits Z + B weights their values C.  Candidates are block i's tokens from stream a (logit Za[p][j] +
 * Ba[r][j], value Ca[p][j]) and, when overlap != 0 (CSA, m = 4), block i-1's tokens from stream b (logit
 * Zb[p][j] + Bb[r][j], value Cb[p][j]); block -1 contributes nothing.  Entries are computed in fp32 and
 * encoded into out's format (rotated first when out.flags has LCA_ROTATE_HADAMARD).
 *   Ca, Za (and Cb, Zb when overlap): float [B][n][c], tokens start_pos .. start_pos + n - 1.
 *   Ba (and Bb when overlap): float [m][c] position biases.
 *   tail_Cb, tail_Zb: float [B][m][c], stream-b values/logits of block start_pos/m - 1; required when
 *     overlap && start_pos > 0, else ignored (may be NULL).
 *   start_pos must be a multiple of m.  A decode append passes the tokens of the current partial block
 *   again plus the new token.  Writes entries [start_pos/m, start_pos/m + ceil(n/m)) of each sequence of
 *   out (out.dim == c); the last one is provisional when n is not a multiple of m.
 *   epi (HOST pointer, nullable): the entry epilogues (see lca_epilogue); NULL applies none.
 *   ragged (HOST pointer, nullable): per-sequence start positions and token counts (see lca_ragged); with
 *   ragged->pos, a tail is passed whenever overlap (it is read for the sequences whose pos[b] > 0).
 * Errors: INVALID_ARG (null, n <= 0, c != out.dim, m <= 0, start_pos % m, rows beyond out.cap,
 *         missing tail, an epilogue with rope_dims odd, negative or > c, rope_base <= 0, norm_eps < 0 or not
 *         finite), UNSUPPORTED (c > 1024), ALIGNMENT.
 */
int kv_compress(const float* Ca, const float* Cb, const float* Za, const float* Zb, const float* Ba, const float* Bb,
                const float* tail_Cb, const float* tail_Zb, int B, long long n, int c, int m, int overlap,
                long long start_pos, const lca_epilogue* epi, const lca_ragged* ragged, lca_tensor out, void* stream);

/*
 * indexer_score_topk -- stage 2, Lightning Indexer score and exact top-k (paper notes section 2.3 Eq. 16 and
 * the Indexer excerpt; cosmocat section 3; 67808.cn section 2).
 * For query row t = q_start_pos + r and entry i:  s[t][i] = sum_h w[t][h] * max(0, qI[t][h] . kI[i]).
 * Entry i is visible iff i < min(floor(t / m), N): a query never sees its own block.  The k_eff =
 * min(k, visible) entries first in the order (score descending, index ascending) are selected and written
 * to idx_out in ascending entry order, followed by -1 padding.
 *   qI: query tensor with cap = Sq * HI rows per sequence (row r*HI + h), dim = DI; format F32, BF16 or FP4.
 *   w:  float [B][Sq][HI] head weights (already scaled).
 *   kI: key tensor, dim = DI, first N rows of each sequence used; format F32, BF16 or FP4.
 *   idx_out: int32 [B][Sq][k].  score_out (nullable): float [B][Sq][k], the fp32 score of each selected
 *   entry (-inf at padding).
 * Scores are fp32.  The per-head sum is fixed: p[h] = fl32(w[h] * max(0, d[h])) added in a halving tree
 * (a[j] += a[j + L/2], L = next power of two of HI, zero padded), so inputs whose per-head dots are exact in
 * fp32 (e.g. fp4 x fp4 with a bounded scale spread) give bit-reproducible selections.
 * ws: device scratch of at least indexer_score_topk_workspace_size(B, Sq, N, k) bytes, 16-byte aligned (contents
 * ignored).
 * ragged (HOST pointer, nullable): per-sequence query positions (see lca_ragged).
 * Errors: INVALID_ARG (null, sizes <= 0, dims mismatch, qI.cap != Sq * HI, DI % 16 for FP4),
 *         UNSUPPORTED (HI > 64, DI > 128, q/k formats not both float-like or both FP4; a paged kI with blocks of
 *         fewer than 32 rows, or an fp4 pool of 2 GiB of codes or more, on the decode kernels -- 64 heads of 128
 *         dims and up to 4 query rows per sequence), WORKSPACE, ALIGNMENT.
 */
size_t indexer_score_topk_workspace_size(int B, int Sq, int N, int k);

/*
 * lca_set_score_events -- profiling hook for the dominant kernel.  While both are non-NULL, every
 * indexer_score_topk call made from the calling host thread launches its scoring kernel with hipExtLaunchKernel
 * and these two events (hipEvent_t, created by the caller with timing enabled), which the runtime stamps with that
 * dispatch's own start and end, so hipEventElapsedTime(ev_begin, ev_end) is the kernel's duration.  Pass NULL, NULL
 * to stop.  The events are owned by the caller.  Nothing is stamped while the stream is being captured into a graph.
 */
void lca_set_score_events(void* ev_begin, void* ev_end);

/*
 * lca_set_attn_events -- the same hook for the attention: while both are non-NULL, every sparse_mqa_attn and
 * hca_attn call made from the calling host thread has ev_begin stamped with the start of its first attention kernel
 * and ev_end with the end of its last one before the merge of split partials (the decode path's score and value
 * passes are timed together).  Pass NULL, NULL to stop.
 */
void lca_set_attn_events(void* ev_begin, void* ev_end);

int indexer_score_topk(lca_tensor qI, const float* w, lca_tensor kI, int B, int Sq, int HI, int DI, int N, int m, int k,
                       long long q_start_pos, int32_t* idx_out, float* score_out, void* ws, size_t ws_bytes,
                       const lca_ragged* ragged, void* stream);

/*
 * indexer_score_topk_noalloc -- for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): indexer_score_topk with the same arguments, kernels and
 * results, minus ws / ws_bytes.  Its scratch is a fixed device array inside the library of
 * LCA_NOALLOC_SCRATCH_BYTES per device, held by each device that runs it until the process ends; the call itself
 * allocates nothing.  Every call on one device shares that device's array and leaves its contents behind (what
 * must start at zero is cleared inside each call): calls that overlap in time on one device (several streams or
 * host threads) race and give undefined results.
 * Errors: those of indexer_score_topk, and WORKSPACE when indexer_score_topk_workspace_size(B, Sq, N, k) exceeds
 *         LCA_NOALLOC_SCRATCH_BYTES (e.g. the decode workloads fit: 4 x 262144 or 16 x 32768 entries, one or two
 *         query rows; long prefill chunks do not).
 */
#define LCA_NOALLOC_SCRATCH_BYTES (32u << 20)
int indexer_score_topk_noalloc(lca_tensor qI, const float* w, lca_tensor kI, int B, int Sq, int HI, int DI, int N, int m,
                               int k, long long q_start_pos, int32_t* idx_out, float* score_out,
                               const lca_ragged* ragged, void* stream);

/*
 * sparse_mqa_attn -- stage 3, shared-KV multi-query attention over the sliding window, the selected
 * compressed entries and a per-head sink (paper notes section 2.3 item 3 and the Attention.forward excerpt;
 * itsolotime mechanisms 1 and 3; 67808.cn section 4).
 * For query row t and head h the attended set is the raw window positions [max(0, t - window + 1), t]
 * (row p - raw_start_pos of kv_raw) plus the compressed entries idx[b][r][0..k) that lie in [0, N)
 * (other values are padding and are skipped).  Every entry is both key and value:
 *   l_j = scale * q[t][h] . kv_j,  M = max(sink[h], max_j l_j),
 *   o[t][h] = sum_j e^(l_j - M) kv_j / (e^(sink[h] - M) + sum_j e^(l_j - M)).
 * sink[h] = -INFINITY disables the sink.  An empty set without a sink gives o = 0 and lse = -inf.
 *   q: [B][Sq][H][D] in q_format (LCA_F32 or LCA_BF16).
 *   kv_comp, kv_raw: dim = D, formats F32, BF16 or MIXED_FP8 (both the same format).  A window-only call (k = 0,
 *   idx NULL: the ratio-0 pure sliding-window layer of the paper notes' section 2.4 config excerpt) may pass a
 *   kv_comp with data NULL (N is then taken as 0).
 *   The window positions of every query must lie in [raw_start_pos, raw_start_pos + S_raw), and
 *   S_raw <= kv_raw.cap.
 *   out: [B][Sq][H][D] in out_format (LCA_F32 or LCA_BF16).  lse_out (nullable): float [B][Sq][H], the log
 *   of the softmax denominator M + log(den).
 * ws: device scratch of at least sparse_mqa_attn_workspace_size(B, Sq, H, D, window + k) bytes, 16-byte aligned when
 * that size is non-zero.
 * ragged (HOST pointer, nullable): per-sequence query positions (see lca_ragged).
 * Errors: INVALID_ARG, UNSUPPORTED (shape without a kernel: on the float path -- q or the caches not bf16 over
 *         bf16/mixed, or H != 64, or D != 512 -- H > 64, D > 512 or H * D > 8192), WORKSPACE, ALIGNMENT.
 */
size_t sparse_mqa_attn_workspace_size(int B, int Sq, int H, int D, int max_entries);
int sparse_mqa_attn(const void* q, int q_format, lca_tensor kv_comp, int N, lca_tensor kv_raw, long long raw_start_pos,
                    int S_raw, const int32_t* idx, int k, const float* sink, int B, int Sq, int H, int D, int window,
                    float scale, long long q_start_pos, void* out, int out_format, float* lse_out, void* ws,
                    size_t ws_bytes, const lca_ragged* ragged, void* stream);

/*
 * hca_attn -- stage 4, the HCA variant: dense MQA over every visible m:1 entry (i < min(floor(t/m), N)),
 * the sliding window and the sink (paper notes section 2.4; cosmocat section 4; 67808.cn section 3).
 * Same arithmetic, arguments and errors as sparse_mqa_attn with the index list replaced by all visible
 * entries.  ws: at least hca_attn_workspace_size(B, Sq, H, D, window + N) bytes, 16-byte aligned.
 */
size_t hca_attn_workspace_size(int B, int Sq, int H, int D, int max_entries);
int hca_attn(const void* q, int q_format, lca_tensor kv_comp, int N, int m, lca_tensor kv_raw, long long raw_start_pos,
             int S_raw, const float* sink, int B, int Sq, int H, int D, int window, float scale,
             long long q_start_pos, void* out, int out_format, float* lse_out, void* ws, size_t ws_bytes,
             const lca_ragged* ragged, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LCA_H */
