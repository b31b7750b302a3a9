/* Drives every function of the CPU oracle (oracle/oracle.c) on small inputs, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py compiles and runs it).  Exits 0 when every call
 * returned; the sanitizers abort on any out-of-bounds access, use of freed memory or undefined behaviour. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/oracle.c"

static unsigned long long rng_state = 88172645463325252ull;
static double urand(void) { /* xorshift64, uniform in [-1, 1) */
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (double)(rng_state >> 11) / (double)(1ull << 52) - 1.0;
}
static float* frand(size_t n) {
  float* p = (float*)malloc(sizeof(float) * n);
  for (size_t i = 0; i < n; ++i) p[i] = (float)(2.0 * urand());
  return p;
}

int main(void) {
  enum { B = 2, n = 37, c = 32, m = 4, Sq = 3, HI = 4, DI = 32, H = 3, D = 32, k = 5, W = 6 };
  /* codec, all formats */
  for (int code = 0; code < 256; ++code) (void)orc_fp8_decode1((uint8_t)code);
  for (int code = 0; code < 16; ++code) (void)orc_fp4_decode1((uint8_t)code);
  (void)orc_bf16_encode1(INFINITY);
  (void)orc_bf16_encode1(NAN);
  (void)orc_fp8_encode1(1e-9f);
  const int rows = 7;
  float* x = frand((size_t)rows * 128);
  x[5] = 0.0f;
  for (int j = 0; j < 16; ++j) x[128 + j] = 0.0f; /* an all-zero fp4 group */
  for (int fmt = 0; fmt < 4; ++fmt) {
    const int rope = fmt == ORC_MIXED ? 16 : 0;
    void* data = malloc((size_t)rows * 128 * 4);
    void* rd = malloc((size_t)rows * 128 * 2);
    void* sc = malloc((size_t)rows * 128);
    orc_encode_rows(x, rows, fmt, 128, rope, data, rd, sc);
    orc_cache cc = {fmt, 128, rope, rows, data, rd, sc, NULL, 0};
    double* out = (double*)malloc(sizeof(double) * rows * 128);
    orc_decode_rows(&cc, 0, rows, out);
    free(out);
    free(data);
    free(rd);
    free(sc);
  }
  /* compression: CSA with a carried tail, HCA, a ragged chunk */
  float *Ca = frand(B * n * c), *Cb = frand(B * n * c), *Za = frand(B * n * c), *Zb = frand(B * n * c);
  float *Ba = frand(128 * c), *Bb = frand(m * c), *tC = frand(B * m * c), *tZ = frand(B * m * c);
  double* E = (double*)malloc(sizeof(double) * B * ((n + m - 1) / m) * c);
  orc_kv_compress(Ca, Cb, Za, Zb, Ba, Bb, tC, tZ, B, n, c, m, 1, 8, E);
  orc_kv_compress(Ca, NULL, Za, NULL, Ba, NULL, NULL, NULL, B, n, c, 128, 0, 0, E);
  /* epilogues and the rotation */
  double* Y = (double*)malloc(sizeof(double) * B * 10 * c);
  double pos[B * 10];
  for (int i = 0; i < B * 10; ++i) pos[i] = 4.0 * i;
  orc_rmsnorm_rows(E, B * 10, c, Ba, 1e-6, Y);
  orc_rope_rows(Y, B * 10, c, 16, pos, 10000.0, E);
  orc_hadamard_rows(E, B * 10, c, Y);
  /* indexer scores over fp4 and f32 keys, dense, paged and ragged; top-k */
  const int N = 12, cap = 16;
  float* q32 = frand(B * Sq * HI * DI);
  float* k32 = frand(B * cap * DI);
  float* w = frand(B * Sq * HI);
  int table[B * (cap / 4)];
  for (int i = 0; i < B * (cap / 4); ++i) table[i] = B * (cap / 4) - 1 - i;
  orc_cache qc = {ORC_F32, DI, 0, Sq * HI, q32, NULL, NULL, NULL, 0};
  orc_cache kc = {ORC_F32, DI, 0, cap, k32, NULL, NULL, NULL, 0};
  orc_cache kp = {ORC_F32, DI, 0, cap, k32, NULL, NULL, table, 4};
  int rws[Sq] = {0, 1, 2};
  double* s64 = (double*)malloc(sizeof(double) * B * Sq * N);
  float* s32 = (float*)malloc(sizeof(float) * B * Sq * N);
  double* ab = (double*)malloc(sizeof(double) * B * Sq * N);
  unsigned char* ex = (unsigned char*)malloc((size_t)B * Sq * N);
  long long bad = 0, seq_pos[B] = {4 * N, 4 * N - 9};
  orc_indexer_scores(&qc, w, &kc, B, Sq, HI, DI, N, m, 4 * N, NULL, rws, Sq, s64, s32, ab, &bad, ex);
  orc_indexer_scores(&qc, w, &kp, B, Sq, HI, DI, N, m, 4 * N, seq_pos, rws, Sq, s64, s32, ab, &bad, ex);
  int nvis[B * Sq];
  for (int i = 0; i < B * Sq; ++i) nvis[i] = (i % 2) ? N : 3;
  int* idx = (int*)malloc(sizeof(int) * B * Sq * k);
  double kth[B * Sq], nxt[B * Sq];
  orc_topk_rows(s64, B * Sq, N, nvis, k, idx, kth, nxt);
  /* attention: sparse, dense HCA, window only; paged and ragged */
  float* qa = frand(B * Sq * H * D);
  float* comp = frand(B * cap * D);
  float* raw = frand(B * (W + Sq) * D);
  float sink[H] = {-INFINITY, 0.5f, 1.0f};
  orc_cache qa_c = {ORC_F32, D, 0, Sq * H, qa, NULL, NULL, NULL, 0};
  orc_cache cp = {ORC_F32, D, 0, cap, comp, NULL, NULL, table, 4};
  orc_cache rc = {ORC_F32, D, 0, W + Sq, raw, NULL, NULL, NULL, 0};
  double* o = (double*)malloc(sizeof(double) * B * Sq * H * D);
  double* lse = (double*)malloc(sizeof(double) * B * Sq * H);
  const long long q0 = 4 * N;
  int rc1 = orc_attn(&qa_c, &cp, N, &rc, q0 - W + 1, W + Sq, idx, k, 0, sink, B, Sq, H, D, W, 0.3, q0, NULL, rws, Sq,
                     o, lse);
  int rc2 = orc_attn(&qa_c, &cp, N, &rc, q0 - W + 1, W + Sq, NULL, 0, m, sink, B, Sq, H, D, W, 0.3, q0, seq_pos, rws,
                     Sq, o, lse);
  int rc3 = orc_attn(&qa_c, &cp, 0, &rc, q0 - W + 1, W + Sq, NULL, 0, 0, sink, B, Sq, H, D, W, 0.3, q0, NULL, rws, Sq,
                     o, lse);
  printf("oracle calls done: %d %d %d, inexact %lld\n", rc1, rc2, rc3, bad);
  free(x);
  free(Ca);
  free(Cb);
  free(Za);
  free(Zb);
  free(Ba);
  free(Bb);
  free(tC);
  free(tZ);
  free(E);
  free(Y);
  free(q32);
  free(k32);
  free(w);
  free(s64);
  free(s32);
  free(ab);
  free(ex);
  free(idx);
  free(qa);
  free(comp);
  free(raw);
  free(o);
  free(lse);
  return (rc1 | rc2 | rc3) != 0;
}
