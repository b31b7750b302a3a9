/*
 * oracle.c -- plain, slow CPU reference for the DeepSeek-V4 hybrid compressed attention layer
 * (CSA: 4:1 overlapped compression + Lightning Indexer top-k + sparse MQA with window and sink;
 *  HCA: 128:1 compression + dense MQA with window and sink).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call this file.  Only the
 * test suite, the package smoke check and the benchmark's CPU-baseline leg use it.  It shares no code,
 * header, table or constant generator with the HIP library: every format and every step below is
 * written again from the pages' description and from the published number-format definitions.
 *
 * Arithmetic is IEEE double unless a step is defined in fp32 (the codec's scale/divide steps and the
 * canonical fp32 indexer score).  Build with  gcc -O2 -ffp-contract=off -fopenmp  so that no step is
 * fused or reassociated.
 *
 * Sources (page titles as printed on the pages):
 *   [P1] "百万token成本暴降90%！DeepSeek-V4揭秘" -- sliding-window branch (mechanism 1), overlapped
 *        compression (mechanism 2), attention sink (mechanism 3), FP4 question 4, cache question 5.
 *   [P2] "DeepSeek-V4: Towards Highly Efficient Million-Token Context Intelligence" (paper notes) --
 *        section 2.3 (CSA, Eq. 11-12 text, Eq. 16, Compressor and Indexer code excerpts),
 *        section 2.4 (HCA, Eq. 22-23 text, Attention.forward excerpt).
 *   [P3] "Mind Observatory: Uncovering the technical ledger of DeepSeek-V4" -- mixed-precision cache.
 *   [P4] "一个数量级是怎么省的：DeepSeek-V4 的百万上下文三件套" -- section 3 (indexer, top-k,
 *        low-precision cache), section 4 (HCA).
 *   [P5] DeepSeek-V4 CSA/HCA explainer (67808.cn) -- section 2 (overlap, indexer dims, k), section 3
 *        (HCA entry count), section 4 (window).
 *
 * Parity status of each function is listed in its header comment ("pinned by" = the CPU tests that
 * tie it to something other than itself).
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------------------------------ */
/* Number formats (written from the format definitions, value level first, bits last).               */
/* ------------------------------------------------------------------------------------------------ */

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_MIXED = 2, ORC_FP4 = 3 };

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Round a finite double to a grid of spacing `quantum` (a power of two), ties to the even multiple.
 * nearbyint() uses the default rounding mode, round-half-to-even. */
static double round_to_quantum(double a, double quantum) { return nearbyint(a / quantum) * quantum; }

/* floor(log2(a)) for a > 0, exact via frexp. */
static int floor_log2(double a) {
  int e;
  frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
  return e - 1;
}

/* bfloat16: 8 significant bits, 8-bit exponent (same range as fp32), round to nearest even.
 * pinned by: tests compare every result with torch's float32 -> bfloat16 cast. */
uint16_t orc_bf16_encode1(float x) {
  uint32_t u;
  if (isnan(x)) return 0x7FC0;
  if (x == 0.0f || isinf(x)) {
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16);
  }
  double a = fabs((double)x);
  double quantum = (a < 0x1p-126) ? 0x1p-133 : ldexp(1.0, floor_log2(a) - 7);
  double r = round_to_quantum(a, quantum);
  float rf = (float)r; /* exact: r has at most 8 significant bits (or is FLT overflow -> inf) */
  if (r > (double)FLT_MAX) rf = INFINITY;
  if (signbit(x)) rf = -rf;
  memcpy(&u, &rf, 4);
  return (uint16_t)(u >> 16);
}

double orc_bf16_decode1(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP FP8 E4M3 ("e4m3fn"): exponent bias 7, 3 mantissa bits, no infinities, max finite 448,
 * subnormal spacing 2^-9.  Input must already be clamped to [-448, 448]; rounding is to nearest even.
 * pinned by: every one of the 256 codes round-trips, and encode matches torch.float8_e4m3fn casts. */
uint8_t orc_fp8_encode1(float y) {
  double a = fabs((double)y);
  uint8_t sign = signbit(y) ? 0x80 : 0x00;
  if (a > 448.0) a = 448.0;
  double quantum = (a < 0x1p-6) ? 0x1p-9 : ldexp(1.0, floor_log2(a) - 3);
  double r = round_to_quantum(a, quantum);
  if (r > 448.0) r = 448.0;
  uint8_t code;
  if (r < 0x1p-6) {
    code = (uint8_t)(r / 0x1p-9); /* subnormal: exponent field 0, mantissa r / 2^-9 in 0..7 */
  } else {
    int e = floor_log2(r);
    int mant = (int)((r / ldexp(1.0, e) - 1.0) * 8.0);
    code = (uint8_t)(((e + 7) << 3) | mant);
  }
  return code | sign;
}

double orc_fp8_decode1(uint8_t c) {
  int sgn = (c & 0x80) ? -1 : 1;
  int ef = (c >> 3) & 0xF, mf = c & 7;
  if (ef == 0xF && mf == 7) return NAN;
  double v = (ef == 0) ? ldexp((double)mf, -9) : ldexp(1.0 + mf / 8.0, ef - 7);
  return sgn * v;
}

/* OCP FP4 E2M1: magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}; code = sign<<3 | magnitude index.
 * Nearest value, ties to the even magnitude index, saturating at 6.
 * pinned by: brute-force nearest-value search over the 8 magnitudes in the tests, and torch's
 * float4_e2m1fn_x2 decode table. */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

uint8_t orc_fp4_encode1(double y) {
  double a = fabs(y);
  int best = 0;
  double bd = INFINITY;
  for (int c = 0; c < 8; ++c) {
    double d = fabs(a - kE2M1[c]);
    if (d < bd || (d == bd && (c % 2) == 0)) {
      bd = d;
      best = c;
    }
  }
  return (uint8_t)((signbit(y) ? 8 : 0) | best);
}

double orc_fp4_decode1(uint8_t c) { return ((c & 8) ? -1.0 : 1.0) * kE2M1[c & 7]; }

/* fp4 blocks of ORC_FP4_BLOCK consecutive elements share one power-of-two scale ([P1] question 4: each 1x32 FP4
 * sub-block has its own scale factor): the smallest integer e with amax <= 6 * 2^e over the block (exact
 * comparison), kept in [-127, 127]; amax == 0 gives e = -127.  Stored as the E8M0 byte e + 127. */
#define ORC_FP4_BLOCK 32
static int fp4_group_exponent(double amax) {
  if (amax == 0.0) return -127;
  int e = floor_log2(amax) - 3; /* 6 * 2^e < amax here unless amax is tiny; walk up exactly */
  while (amax > 6.0 * ldexp(1.0, e)) ++e;
  while (e > -127 && amax <= 6.0 * ldexp(1.0, e - 1)) --e;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

/* A cache tensor as the oracle reads it.  Rows are addressed b * cap + r.
 *   F32  : data = float[rows][dim]
 *   BF16 : data = uint16[rows][dim]
 *   MIXED: data = uint8 fp8 codes [rows][dim - rope], scale = float[rows], rope = uint16 bf16 [rows][rope]
 *          (the RoPE dims are the last `rope` channels of the row, [P2] Indexer excerpt applies RoPE to
 *          q[..., -rd:]; [P3]/[P4] sec.3: RoPE dims bf16, the rest fp8)
 *   FP4  : data = uint8 packed [rows][dim/2] (element 2j in the low nibble), scale = uint8 E8M0 [rows][dim/32]
 */
typedef struct {
  int fmt, dim, rope;
  long long cap;
  const void* data;
  const void* rope_data;
  const void* scale;
  /* A paged cache ([P1] question 5: the compressed cache is managed in fixed-size blocks): when table != NULL, entry
   * i of sequence b is row table[b * (cap / block_rows) + i / block_rows] * block_rows + i % block_rows of the
   * arrays above (a pool of blocks); otherwise it is row b * cap + i. */
  const int* table;
  int block_rows;
} orc_cache;

/* Storage row of entry i of sequence b (see orc_cache).
 * pinned by: a cache whose blocks are permuted through its table gives the same scores and outputs as the dense
 * cache. */
static long long cache_row(const orc_cache* c, int b, long long i) {
  if (!c->table) return (long long)b * c->cap + i;
  const long long nblk = c->cap / c->block_rows;
  return (long long)c->table[(long long)b * nblk + i / c->block_rows] * c->block_rows + i % c->block_rows;
}

/* Encode fp32 rows into a cache format (the quantise-on-write of the mixed-precision cache).
 * The fp8 per-row scale is s = fl32(amax / 448) over the row's non-RoPE dims (s = 1 if amax = 0);
 * code = fp8(clamp(fl32(x / s), +-448)).  fp4 per block of ORC_FP4_BLOCK elements: see fp4_group_exponent.
 * pinned by: codec round-trip and torch-cast tests. */
void orc_encode_rows(const float* x, long long rows, int fmt, int dim, int rope, void* data, void* rope_data,
                     void* scale) {
#pragma omp parallel for schedule(static)
  for (long long r = 0; r < rows; ++r) {
    const float* xr = x + r * dim;
    if (fmt == ORC_F32) {
      memcpy((float*)data + r * dim, xr, sizeof(float) * (size_t)dim);
    } else if (fmt == ORC_BF16) {
      uint16_t* o = (uint16_t*)data + r * dim;
      for (int j = 0; j < dim; ++j) o[j] = orc_bf16_encode1(xr[j]);
    } else if (fmt == ORC_MIXED) {
      int dm = dim - rope;
      float amax = 0.0f;
      for (int j = 0; j < dm; ++j) {
        float a = fabsf(xr[j]);
        if (a > amax) amax = a;
      }
      volatile float s = (amax == 0.0f) ? 1.0f : amax / 448.0f; /* fp32 divide */
      ((float*)scale)[r] = s;
      uint8_t* o = (uint8_t*)data + r * dm;
      for (int j = 0; j < dm; ++j) {
        volatile float y = xr[j] / s; /* fp32 divide */
        float yc = y > 448.0f ? 448.0f : (y < -448.0f ? -448.0f : y);
        o[j] = orc_fp8_encode1(yc);
      }
      uint16_t* ro = (uint16_t*)rope_data + r * rope;
      for (int j = 0; j < rope; ++j) ro[j] = orc_bf16_encode1(xr[dm + j]);
    } else { /* FP4 */
      uint8_t* o = (uint8_t*)data + r * (dim / 2);
      uint8_t* sc = (uint8_t*)scale + r * (dim / ORC_FP4_BLOCK);
      for (int g = 0; g < dim / ORC_FP4_BLOCK; ++g) {
        const float* xb = xr + (size_t)ORC_FP4_BLOCK * g;
        double amax = 0.0;
        for (int j = 0; j < ORC_FP4_BLOCK; ++j) {
          double a = fabs((double)xb[j]);
          if (a > amax) amax = a;
        }
        int e = fp4_group_exponent(amax);
        sc[g] = (uint8_t)(e + 127);
        for (int j = 0; j < ORC_FP4_BLOCK; j += 2) {
          uint8_t lo = orc_fp4_encode1(ldexp((double)xb[j], -e));
          uint8_t hi = orc_fp4_encode1(ldexp((double)xb[j + 1], -e));
          o[(ORC_FP4_BLOCK / 2) * g + j / 2] = (uint8_t)(lo | (hi << 4));
        }
      }
    }
  }
}

static void decode_row(const orc_cache* c, long long row, double* out) {
  int dim = c->dim;
  if (c->fmt == ORC_F32) {
    const float* p = (const float*)c->data + row * dim;
    for (int j = 0; j < dim; ++j) out[j] = (double)p[j];
  } else if (c->fmt == ORC_BF16) {
    const uint16_t* p = (const uint16_t*)c->data + row * dim;
    for (int j = 0; j < dim; ++j) out[j] = orc_bf16_decode1(p[j]);
  } else if (c->fmt == ORC_MIXED) {
    int dm = dim - c->rope;
    const uint8_t* p = (const uint8_t*)c->data + row * dm;
    double s = (double)((const float*)c->scale)[row];
    for (int j = 0; j < dm; ++j) out[j] = orc_fp8_decode1(p[j]) * s;
    const uint16_t* rp = (const uint16_t*)c->rope_data + row * c->rope;
    for (int j = 0; j < c->rope; ++j) out[dm + j] = orc_bf16_decode1(rp[j]);
  } else {
    const uint8_t* p = (const uint8_t*)c->data + row * (dim / 2);
    const uint8_t* sc = (const uint8_t*)c->scale + row * (dim / ORC_FP4_BLOCK);
    for (int j = 0; j < dim; ++j) {
      uint8_t byte = p[j / 2];
      uint8_t code = (j & 1) ? (byte >> 4) : (byte & 0xF);
      out[j] = ldexp(orc_fp4_decode1(code), (int)sc[j / ORC_FP4_BLOCK] - 127);
    }
  }
}

void orc_decode_rows(const orc_cache* c, long long row0, long long rows, double* out) {
#pragma omp parallel for schedule(static)
  for (long long r = 0; r < rows; ++r) decode_row(c, row0 + r, out + r * c->dim);
}

/* ------------------------------------------------------------------------------------------------ */
/* Stage 1: KV compression ([P2] sec. 2.3 Eq. 11-12 text and Compressor excerpt; [P2] sec. 2.4        */
/* Eq. 22-23 text; [P1] mechanism 2; [P5] sec. 2 "half-window overlap").                             */
/* ------------------------------------------------------------------------------------------------ */
/* Hadamard rotation of indexer rows ([P2] section 2.3, the Indexer excerpt: the indexer's queries, and the keys
 * its own compressor writes, are rotated by a Hadamard transform before their FP4 quantisation).  The plain
 * definition of the orthonormal Sylvester-Hadamard matrix of order n (a power of two), evaluated as written,
 * O(n^2) per row, in double:
 *   y[i] = sum_j (-1)^popcount(i & j) x[j] / sqrt(n). */
void orc_hadamard_rows(const double* x, long long rows, int n, double* y) {
  const double s = sqrt((double)n);
#pragma omp parallel for schedule(static)
  for (long long r = 0; r < rows; ++r) {
    const double* xr = x + r * n;
    for (int i = 0; i < n; ++i) {
      double acc = 0.0;
      for (int j = 0; j < n; ++j) acc += (__builtin_popcount((unsigned)(i & j)) & 1) ? -xr[j] : xr[j];
      y[r * n + i] = acc / s;
    }
  }
}

/*
 * Entry i (block i of m consecutive tokens), channel j, is a softmax-weighted sum of candidates:
 *   - the tokens of block i from stream a: logit Za[p][j] + Ba[r][j], value Ca[p][j], p = m*i + r;
 *   - with overlap (CSA), the tokens of block i-1 from stream b: logit Zb[p][j] + Bb[r][j], value Cb[p][j].
 * The softmax runs over all candidates of the entry, per channel.  Block -1 does not exist: its
 * candidates are absent (the -inf padding of the missing predecessor).  A partial last block uses
 * the tokens present.  Inputs start at absolute token start_pos (a multiple of m); with overlap and
 * start_pos > 0 the previous block's stream-b tokens come from tail_Cb / tail_Zb [B][m][c].
 * Output: out[B][ceil(n/m)][c] in double.
 * pinned by: constant candidates give the constant (weights sum to 1); one-hot logits select one
 * candidate and show which block each stream feeds; shift invariance of the logits; m = 1 reduces
 * the whole layer to causal attention (checked against torch's scaled_dot_product_attention).
 */
void orc_kv_compress(const float* Ca, const float* Cb, const float* Za, const float* Zb, const float* Ba,
                     const float* Bb, const float* tail_Cb, const float* tail_Zb, int B, long long n, int c, int m,
                     int overlap, long long start_pos, double* out) {
  long long nb = (n + m - 1) / m;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b) {
    for (long long i = 0; i < nb; ++i) {
      double* lg = (double*)malloc(sizeof(double) * 2 * (size_t)m);
      double* vv = (double*)malloc(sizeof(double) * 2 * (size_t)m);
      long long gblock = start_pos / m + i;
      for (int j = 0; j < c; ++j) {
        int cnt = 0;
        for (int r = 0; r < m; ++r) {
          long long p = (long long)m * i + r;
          if (p >= n) break;
          size_t o = ((size_t)b * n + p) * c + j;
          lg[cnt] = (double)Za[o] + (double)Ba[r * c + j];
          vv[cnt] = (double)Ca[o];
          ++cnt;
        }
        if (overlap && gblock >= 1) {
          for (int r = 0; r < m; ++r) {
            double z, v;
            if (i >= 1) {
              size_t o = ((size_t)b * n + (size_t)m * (i - 1) + r) * c + j;
              z = (double)Zb[o];
              v = (double)Cb[o];
            } else {
              size_t o = ((size_t)b * m + r) * c + j;
              z = (double)tail_Zb[o];
              v = (double)tail_Cb[o];
            }
            lg[cnt] = z + (double)Bb[r * c + j];
            vv[cnt] = v;
            ++cnt;
          }
        }
        double mx = -INFINITY;
        for (int q = 0; q < cnt; ++q)
          if (lg[q] > mx) mx = lg[q];
        double num = 0.0, den = 0.0;
        for (int q = 0; q < cnt; ++q) {
          double e = exp(lg[q] - mx);
          num += e * vv[q];
          den += e;
        }
        out[((size_t)b * nb + i) * c + j] = num / den;
      }
      free(lg);
      free(vv);
    }
  }
}

/* Epilogues on compressed entries ([P2] section 2.3: the Compressor holds an RMSNorm over the entry's head_dim; the
 * Indexer excerpt applies rotary position embedding to the trailing rd channels).  Plain definitions, in double.
 *
 * RMS normalisation of each row: y[j] = x[j] / sqrt(mean_j(x[j]^2) + eps) * g[j].
 * pinned by: a hand-computed row; invariance to scaling x (eps = 0); mean(y^2) = 1 for g = 1, eps = 0. */
void orc_rmsnorm_rows(const double* x, long long rows, int c, const float* g, double eps, double* y) {
#pragma omp parallel for schedule(static)
  for (long long r = 0; r < rows; ++r) {
    const double* xr = x + r * c;
    double ss = 0.0;
    for (int j = 0; j < c; ++j) ss += xr[j] * xr[j];
    const double inv = 1.0 / sqrt(ss / c + eps);
    for (int j = 0; j < c; ++j) y[r * c + j] = xr[j] * inv * (double)g[j];
  }
}

/* Rotary position embedding of the trailing rd channels of each row (rd even): channel pair (2j, 2j+1) of that
 * segment is rotated by the angle pos[r] * base^(-2j/rd):
 *   (a, b) -> (a cos - b sin, a sin + b cos).
 * The leading c - rd channels are copied.
 * pinned by: position 0 is the identity; pair norms are preserved; hand-computed angles; composition of positions;
 * dot products of two rotated rows depend only on the difference of their positions. */
void orc_rope_rows(const double* x, long long rows, int c, int rd, const double* pos, double base, double* y) {
#pragma omp parallel for schedule(static)
  for (long long r = 0; r < rows; ++r) {
    const double* xr = x + r * c;
    double* yr = y + r * c;
    for (int j = 0; j < c - rd; ++j) yr[j] = xr[j];
    for (int j = 0; j < rd / 2; ++j) {
      const double ang = pos[r] * pow(base, -2.0 * j / rd);
      const double cs = cos(ang), sn = sin(ang);
      const double a = xr[c - rd + 2 * j], b = xr[c - rd + 2 * j + 1];
      yr[c - rd + 2 * j] = a * cs - b * sn;
      yr[c - rd + 2 * j + 1] = a * sn + b * cs;
    }
  }
}

/* ------------------------------------------------------------------------------------------------ */
/* Stage 2: Lightning Indexer score ([P2] sec. 2.3 Eq. 16 and Indexer excerpt; [P4] sec. 3; [P5]      */
/* sec. 2) and exact top-k.                                                                          */
/* ------------------------------------------------------------------------------------------------ */
/*
 * For query row t (absolute position q_start_pos + row) and compressed entry i:
 *   d[h]  = q[t,h,:] . K[i,:]
 *   s[i]  = sum_h w[t,h] * max(0, d[h])                                       (Eq. 16)
 * Entry i is visible to query t iff i < floor(t / m) and i < N: a query never sees the block it sits
 * in ([P1] mechanism 1, [P5] sec. 4).  Entries that are not visible get s = -inf.
 *
 * s64 receives the double score.  If s32 is non-NULL it receives the canonical fp32 score, defined
 * whenever every d[h] is computed exactly by fp32 arithmetic in any summation order (see
 * orc_dot_is_fp32_exact).  With r[h] = max(0, fl32(d[h])) and the heads padded with zeros (w = r = 0) to a power
 * of two P (the paper notes fix no summation order; this one is the library's, chosen so that most of the
 * reduction is fused multiply-adds that stay within one lane of a matrix unit's result):
 *   P >= 16: sixteen chains, c[j] = fl32(w[j] r[j]), then c[j] <- fma32(w[j + 16 m], r[j + 16 m], c[j]) for
 *            m = 1 .. P/16 - 1 (one rounding per step), then a halving tree over c[0..15];
 *   P < 16:  p[h] = fl32(w[h] r[h]), then a halving tree over p[0..P-1];
 * a halving tree adds level by level a[j] <- a[j] + a[j + L/2] for j < L/2, in fp32.  A -0 result is written
 * as +0.  *inexact counts the (row, entry) pairs with at least one head whose dot is
 * not certified exact; exact_out (optional, [B][nrows][N]) holds 1 for a certified pair, else 0.
 * abs_out (optional) receives sum_h |w[t,h]| * sum_d |q[t,h,d] * K[i,d]|, the scale of the fp32
 * rounding error of any summation order (used to certify near-ties).
 * Rows evaluated: rows[0..nrows) (offsets into [0, Sq)); outputs are [B][nrows][N].  seq_pos (nullable, [B]) puts
 * the rows of sequence b at seq_pos[b] + row instead (a ragged batch).
 * pinned by: dyadic tiny inputs reproduce hand-derivable scores; brute force over tiny inputs; the
 * certificate accepts small-spread fp4 rows and rejects a constructed wide-spread row whose fp32 sum
 * rounds.
 */
/* Certificate that fp32 arithmetic reproduces the dot sum_d q[d] * k[d] exactly in every summation order
 * (and in any grouping, such as a matrix unit's blocks with their own scale factors).  The products are
 * exact in double (fp32 inputs carry at most 24 significant bits).  Let 2^L be the largest power of two
 * dividing every nonzero product and A = sum_d |q[d] k[d]|.  Every partial sum of any subset of products is
 * an integer multiple of 2^L no larger than A in magnitude, so if A < 2^(L + 24) each one has at most 24
 * significant bits and is an fp32 value; L >= -126 keeps them out of the subnormal range.  For fp4 x fp4
 * rows (one scale per 32-element block) this is the bound on the spread of the blocks' scale exponents: a block's
 * products are multiples of 2^(eq + ek - 2) summing to less than 2^(eq + ek + 11). */
int orc_dot_is_fp32_exact(const double* q, const double* k, int n) {
  int L = INT32_MAX;
  double A = 0.0;
  for (int d = 0; d < n; ++d) {
    double p = q[d] * k[d];
    if (p == 0.0) continue;
    int e;
    double f = frexp(fabs(p), &e);            /* |p| = f * 2^e, f in [0.5, 1) */
    uint64_t mant = (uint64_t)ldexp(f, 53);   /* exact: f has at most 53 significant bits */
    int low = e - 53 + __builtin_ctzll(mant); /* exponent of the lowest set bit of p */
    if (low < L) L = low;
    A += fabs(p);
  }
  if (L == INT32_MAX) return 1; /* every product is zero */
  return L >= -126 && A < ldexp(1.0, L + 24);
}

void orc_indexer_scores(const orc_cache* q, const float* w, const orc_cache* K, int B, int Sq, int HI, int DI, int N,
                        int m, long long q_start_pos, const long long* seq_pos, const int* rows, int nrows,
                        double* s64, float* s32, double* abs_out, long long* inexact, unsigned char* exact_out) {
  int P = 1;
  while (P < HI) P <<= 1;
  long long bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1) reduction(+ : bad)
  for (int b = 0; b < B; ++b) {
    for (int rr = 0; rr < nrows; ++rr) {
      int row = rows[rr];
      long long t = (seq_pos ? seq_pos[b] : q_start_pos) + row;
      long long nvis = t / m;
      if (nvis > N) nvis = N;
      double* qd = (double*)malloc(sizeof(double) * (size_t)HI * DI);
      double* kd = (double*)malloc(sizeof(double) * (size_t)DI);
      float* a = (float*)malloc(sizeof(float) * (size_t)P);
      for (int h = 0; h < HI; ++h) decode_row(q, ((long long)b * Sq + row) * HI + h, qd + (size_t)h * DI);
      const float* wr = w + ((size_t)b * Sq + row) * HI;
      size_t ob = ((size_t)b * nrows + rr) * N;
      for (long long i = 0; i < N; ++i) {
        if (i >= nvis) {
          s64[ob + i] = -INFINITY;
          if (s32) s32[ob + i] = -INFINITY;
          if (abs_out) abs_out[ob + i] = 0.0;
          if (exact_out) exact_out[ob + i] = 1;
          continue;
        }
        decode_row(K, cache_row(K, b, i), kd);
        double acc = 0.0, aacc = 0.0;
        int certified = 1;
        for (int h = 0; h < P; ++h) a[h] = 0.0f;
        for (int h = 0; h < HI; ++h) {
          double d = 0.0, ad = 0.0;
          for (int x = 0; x < DI; ++x) {
            d += qd[(size_t)h * DI + x] * kd[x];
            ad += fabs(qd[(size_t)h * DI + x] * kd[x]);
          }
          acc += (double)wr[h] * (d > 0.0 ? d : 0.0);
          aacc += fabs((double)wr[h]) * ad;
          if (s32 || exact_out || inexact) {
            if (!orc_dot_is_fp32_exact(qd + (size_t)h * DI, kd, DI)) certified = 0;
          }
          if (s32) {
            float d32 = (float)d;
            a[h] = d32 > 0.0f ? d32 : 0.0f; /* r[h]; padded heads stay 0 */
          }
        }
        if (!certified) ++bad;
        if (exact_out) exact_out[ob + i] = (unsigned char)certified;
        s64[ob + i] = acc;
        if (abs_out) abs_out[ob + i] = aacc;
        if (s32) {
          int L = P;
          if (P >= 16) {
            for (int j = 0; j < 16; ++j) {
              volatile float c = (j < HI ? wr[j] : 0.0f) * a[j]; /* fp32 multiply, rounded once */
              for (int h = j + 16; h < P; h += 16) {
                volatile float f = fmaf(h < HI ? wr[h] : 0.0f, a[h], c); /* fused: one rounding */
                c = f;
              }
              a[j] = c;
            }
            L = 16;
          } else {
            for (int h = 0; h < P; ++h) {
              volatile float pr = (h < HI ? wr[h] : 0.0f) * a[h];
              a[h] = pr;
            }
          }
          for (; L > 1; L >>= 1) {
            for (int j = 0; j < L / 2; ++j) {
              volatile float sum = a[j] + a[j + L / 2];
              a[j] = sum;
            }
          }
          s32[ob + i] = (a[0] == 0.0f) ? 0.0f : a[0];
        }
      }
      free(qd);
      free(kd);
      free(a);
    }
  }
  if (inexact) *inexact = bad;
}

/* Exact top-k of one score row ([P2] Indexer excerpt: top-k of min(k, visible) entries; ties go to
 * the lower index).  The selected set is written in ascending entry order, then -1 padding.
 * kth_out / next_out receive the k-th and (k+1)-th scores of the total order (score desc, index asc),
 * -inf where they do not exist.
 * pinned by: brute-force sort over tiny inputs with forced ties. */
typedef struct {
  double s;
  int i;
} orc_si;

static int cmp_desc(const void* x, const void* y) {
  const orc_si* a = (const orc_si*)x;
  const orc_si* b = (const orc_si*)y;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->i < b->i) ? -1 : (a->i > b->i);
}

static int cmp_int(const void* x, const void* y) {
  int a = *(const int*)x, b = *(const int*)y;
  return (a > b) - (a < b);
}

void orc_topk_rows(const double* s, long long nrows, int N, const int* nvis, int k, int* idx_out, double* kth_out,
                   double* next_out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (long long r = 0; r < nrows; ++r) {
    int nv = nvis[r];
    orc_si* v = (orc_si*)malloc(sizeof(orc_si) * (size_t)(nv > 0 ? nv : 1));
    for (int i = 0; i < nv; ++i) {
      double x = s[r * N + i];
      v[i].s = (x == 0.0) ? 0.0 : x;
      v[i].i = i;
    }
    qsort(v, (size_t)nv, sizeof(orc_si), cmp_desc);
    int ke = nv < k ? nv : k;
    int* o = idx_out + r * k;
    for (int j = 0; j < ke; ++j) o[j] = v[j].i;
    qsort(o, (size_t)ke, sizeof(int), cmp_int);
    for (int j = ke; j < k; ++j) o[j] = -1;
    if (kth_out) kth_out[r] = (k >= 1 && k <= nv) ? v[k - 1].s : -INFINITY;
    if (next_out) next_out[r] = (k < nv) ? v[k].s : -INFINITY;
    free(v);
  }
}

/* ------------------------------------------------------------------------------------------------ */
/* Stage 3/4: shared-KV MQA over window + compressed entries + sink ([P2] sec. 2.3 item 3 "K and V    */
/* shared", Attention.forward excerpt; [P1] mechanisms 1 and 3; [P5] sec. 4; [P2] sec. 2.4 / [P4]      */
/* sec. 4 for the dense HCA variant).                                                                */
/* ------------------------------------------------------------------------------------------------ */
/*
 * Query row t = q_start_pos + row, head h.  The attended set is
 *   W(t) = raw positions [max(0, t - window + 1), t]  (raw row p - raw_start),
 *   S(t) = sparse mode (hca_m == 0): entries idx[b][row][0..k) that lie in [0, N) (others are padding);
 *          dense mode (hca_m  > 0):  entries [0, min(floor(t / hca_m), N)).
 * Each entry is both key and value.  l_j = scale * q . kv_j.  The sink logit z_h joins the softmax
 * denominator only: M = max(z_h, max l), den = e^(z_h - M) + sum e^(l_j - M), o = sum e^(l_j - M) kv_j / den,
 * lse = M + log(den).  z_h = -inf disables the sink.  An empty set with no sink gives o = 0, lse = -inf.
 * seq_pos (nullable, [B]) places the rows of sequence b at seq_pos[b] + row (a ragged batch); its raw rows then
 * start at position raw_start + seq_pos[b] - q_start_pos.
 * Returns 0, or -1 if a window position falls outside the raw span given.
 * pinned by: m = 1 collapse to causal attention (library routine), the sink closed form
 * o(z) = o(-inf) * S / (S + e^z), invariance to permuting idx, own block invisible.
 */
int orc_attn(const orc_cache* q, const orc_cache* comp, int N, const orc_cache* raw, long long raw_start, int S_raw,
             const int* idx, int k, int hca_m, const float* sink, int B, int Sq, int H, int D, int window,
             double scale, long long q_start_pos, const long long* seq_pos, const int* rows, int nrows, double* out,
             double* lse) {
  int err = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1) reduction(| : err)
  for (int b = 0; b < B; ++b) {
    for (int rr = 0; rr < nrows; ++rr) {
      int row = rows[rr];
      const long long pos_b = seq_pos ? seq_pos[b] : q_start_pos;
      const long long rs = raw_start + (pos_b - q_start_pos); /* sequence b's raw rows keep the same offset */
      long long t = pos_b + row;
      long long w0 = t - window + 1;
      if (w0 < 0) w0 = 0;
      long long nw = (window > 0) ? (t - w0 + 1) : 0;
      if (nw > 0 && (w0 < rs || t >= rs + S_raw)) {
        err |= 1;
        continue;
      }
      long long nc;
      if (hca_m > 0) {
        nc = t / hca_m;
        if (nc > N) nc = N;
      } else {
        nc = k;
      }
      long long tot = nw + nc;
      double* kv = (double*)malloc(sizeof(double) * (size_t)(tot > 0 ? tot : 1) * D);
      char* use = (char*)malloc((size_t)(tot > 0 ? tot : 1));
      long long cnt = 0;
      for (long long p = w0; p < w0 + nw; ++p) {
        decode_row(raw, cache_row(raw, b, p - rs), kv + (size_t)cnt * D);
        use[cnt++] = 1;
      }
      for (long long j = 0; j < nc; ++j) {
        long long e = (hca_m > 0) ? j : idx[((size_t)b * Sq + row) * k + j];
        if (e < 0 || e >= N) {
          use[cnt++] = 0;
          continue;
        }
        decode_row(comp, cache_row(comp, b, e), kv + (size_t)cnt * D);
        use[cnt++] = 1;
      }
      double* qd = (double*)malloc(sizeof(double) * (size_t)D);
      double* lg = (double*)malloc(sizeof(double) * (size_t)(tot > 0 ? tot : 1));
      for (int h = 0; h < H; ++h) {
        decode_row(q, ((long long)b * Sq + row) * H + h, qd);
        double mx = (double)sink[h];
        for (long long j = 0; j < cnt; ++j) {
          if (!use[j]) continue;
          double d = 0.0;
          for (int x = 0; x < D; ++x) d += qd[x] * kv[(size_t)j * D + x];
          lg[j] = scale * d;
          if (lg[j] > mx) mx = lg[j];
        }
        double* o = out + (((size_t)b * nrows + rr) * H + h) * D;
        for (int x = 0; x < D; ++x) o[x] = 0.0;
        if (mx == -INFINITY) {
          lse[((size_t)b * nrows + rr) * H + h] = -INFINITY;
          continue;
        }
        double den = exp((double)sink[h] - mx);
        for (long long j = 0; j < cnt; ++j) {
          if (!use[j]) continue;
          double e = exp(lg[j] - mx);
          den += e;
          for (int x = 0; x < D; ++x) o[x] += e * kv[(size_t)j * D + x];
        }
        for (int x = 0; x < D; ++x) o[x] /= den;
        lse[((size_t)b * nrows + rr) * H + h] = mx + log(den);
      }
      free(qd);
      free(lg);
      free(kv);
      free(use);
    }
  }
  return err ? -1 : 0;
}
