/*
 * Drives every function of oracle/oracle.c over random and edge-case inputs
 * with buffers of exactly the documented sizes, so that a build with
 * -fsanitize=address,undefined reports any out-of-bounds access, overflow or
 * undefined operation in the oracle.  Test infrastructure only.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oracle_bf16_to_f32(uint16_t b);
uint16_t oracle_f32_to_bf16(float f);
float oracle_e4m3_to_f32(uint8_t b);
uint8_t oracle_f32_to_e4m3(float y);
int64_t oracle_capacity(int32_t N, int32_t K, int32_t E, int32_t A);
int oracle_layout(int32_t N, int32_t K, int32_t E, int32_t R, int32_t A, const int32_t* topk_idx,
                  int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                  uint8_t* is_token_in_rank, int32_t* expert_slot_offset,
                  int32_t* num_recv_per_expert, int32_t* slot_of);
void oracle_recv_meta(int32_t N, int32_t K, int64_t cap, const int32_t* slot_of,
                      const float* topk_weights, int32_t* recv_src_idx, float* recv_topk_weights);
int oracle_ll_layout(int32_t N, int32_t K, int32_t E, int32_t R, int32_t M, const int32_t* topk_idx,
                     int32_t* recv_count, int32_t* slot_of, int32_t* flags);
void oracle_dispatch_bf16(int32_t N, int32_t K, int32_t H, const uint16_t* x,
                          const int32_t* slot_of, uint16_t* recv_x);
void oracle_quantize_row(int32_t H, const uint16_t* xrow, uint8_t* q, float* scales);
void oracle_dispatch_fp8(int32_t N, int32_t K, int32_t H, const uint16_t* x,
                         const int32_t* slot_of, uint8_t* recv_q, float* recv_scales);
void oracle_dispatch_quantized(int32_t N, int32_t K, int32_t H, const uint8_t* codes,
                               const float* scales, const int32_t* slot_of, uint8_t* recv_q,
                               float* recv_scales);
void oracle_zero_padding(int32_t E, int32_t row_bytes, int32_t G, const int32_t* off,
                         const int32_t* count, uint8_t* recv_x, float* recv_scales);
void oracle_accumulate_stats(int32_t E, const int32_t* count, int64_t* stats);
void oracle_combine(int32_t N, int32_t K, int32_t H, const void* eo, int32_t eo_is_f32,
                    const int32_t* slot_of, const float* topk_weights, uint16_t* y,
                    float* acc_out, const int32_t* tokens, int32_t n_tokens);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {  /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static int32_t rint_in(int32_t lo, int32_t hi) { return lo + (int32_t)(rnd() % (uint32_t)(hi - lo + 1)); }
static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
  return p;
}
#define FAIL(...) do { fprintf(stderr, __VA_ARGS__); fputc('\n', stderr); exit(1); } while (0)

static void codecs(void) {
  for (uint32_t b = 0; b < 65536; b++) {
    float f = oracle_bf16_to_f32((uint16_t)b);
    if (!isnan(f) && oracle_f32_to_bf16(f) != (uint16_t)b) FAIL("bf16 round trip %u", b);
    (void)oracle_f32_to_e4m3(f * 3.0f);
  }
  for (int c = 0; c < 256; c++) (void)oracle_e4m3_to_f32((uint8_t)c);
  const float special[] = {0.0f, -0.0f, INFINITY, -INFINITY, NAN, 1e-45f, 3.4e38f, 448.0f, 464.0f};
  for (size_t i = 0; i < sizeof special / sizeof special[0]; i++) {
    (void)oracle_f32_to_e4m3(special[i]);
    (void)oracle_f32_to_bf16(special[i]);
  }
}

static void one_case(void) {
  const int32_t R = rint_in(1, 4), E = R * rint_in(1, 6), K = rint_in(1, 9);
  const int32_t N = R * rint_in(0, 12), A = rint_in(1, 6), fp8 = (int32_t)(rnd() & 1);
  const int32_t H = fp8 ? 128 * rint_in(1, 2) : 8 * rint_in(1, 40), G = H / 128;
  const int64_t NK = (int64_t)N * K;
  const int64_t cap = oracle_capacity(N, K, E, A);
  if (cap != NK + (int64_t)E * (A - 1)) FAIL("capacity");
  int32_t* idx = xmalloc(sizeof(int32_t) * NK);
  float* w = xmalloc(sizeof(float) * NK);
  uint16_t* x = xmalloc(sizeof(uint16_t) * N * H);
  for (int64_t i = 0; i < NK; i++) {
    idx[i] = rint_in(-2, E);  /* -1 = none, -2 and E are invalid */
    w[i] = (float)rint_in(-1000, 1000) / 500.0f;
  }
  for (int64_t i = 0; i < (int64_t)N * H; i++) x[i] = oracle_f32_to_bf16((float)rint_in(-30000, 30000) / 997.0f);
  int32_t* ntpr = xmalloc(sizeof(int32_t) * R * R);
  int32_t* ntpe = xmalloc(sizeof(int32_t) * R * E);
  uint8_t* in_rank = xmalloc((size_t)N * R);
  int32_t* off = xmalloc(sizeof(int32_t) * (E + 1));
  int32_t* cnt = xmalloc(sizeof(int32_t) * E);
  int32_t* slot_of = xmalloc(sizeof(int32_t) * NK);
  int flags = oracle_layout(N, K, E, R, A, idx, ntpr, ntpe, in_rank, off, cnt, slot_of);
  if (flags < 0) FAIL("layout rejected valid sizes");
  int64_t valid = 0, total = 0;
  for (int64_t i = 0; i < NK; i++) valid += (idx[i] >= 0 && idx[i] < E);
  for (int32_t e = 0; e < E; e++) total += cnt[e];
  if (valid != total) FAIL("counts");
  if (off[E] > cap) FAIL("offsets beyond capacity");

  int32_t* src = xmalloc(sizeof(int32_t) * cap);
  float* rw = xmalloc(sizeof(float) * cap);
  oracle_recv_meta(N, K, cap, slot_of, w, src, rw);
  if (!fp8) {
    uint16_t* recv = xmalloc(sizeof(uint16_t) * cap * H);
    memset(recv, 0, sizeof(uint16_t) * cap * H);
    oracle_dispatch_bf16(N, K, H, x, slot_of, recv);
    oracle_zero_padding(E, 2 * H, 0, off, cnt, (uint8_t*)recv, NULL);
    free(recv);
  } else {
    uint8_t* q = xmalloc((size_t)cap * H);
    float* sc = xmalloc(sizeof(float) * cap * G);
    oracle_dispatch_fp8(N, K, H, x, slot_of, q, sc);
    uint8_t* codes = xmalloc((size_t)N * H);
    float* scales = xmalloc(sizeof(float) * N * G);
    for (int32_t t = 0; t < N; t++) oracle_quantize_row(H, x + (int64_t)t * H, codes + (int64_t)t * H, scales + (int64_t)t * G);
    oracle_dispatch_quantized(N, K, H, codes, scales, slot_of, q, sc);
    oracle_zero_padding(E, H, G, off, cnt, q, sc);
    free(q); free(sc); free(codes); free(scales);
  }
  int64_t* stats = xmalloc(sizeof(int64_t) * E);
  memset(stats, 0, sizeof(int64_t) * E);
  oracle_accumulate_stats(E, cnt, stats);

  uint16_t* eo = xmalloc(sizeof(uint16_t) * cap * H);
  float* eof = xmalloc(sizeof(float) * cap * H);
  for (int64_t i = 0; i < cap * H; i++) {
    eof[i] = (float)rint_in(-5000, 5000) / 1234.0f;
    eo[i] = oracle_f32_to_bf16(eof[i]);
  }
  uint16_t* y = xmalloc(sizeof(uint16_t) * N * H);
  float* acc = xmalloc(sizeof(float) * N * H);
  oracle_combine(N, K, H, eo, 0, slot_of, w, y, acc, NULL, 0);
  oracle_combine(N, K, H, eof, 1, slot_of, w, y, NULL, NULL, 0);
  if (N > 0) {
    int32_t tok[3] = {N - 1, 0, N / 2};   /* y/acc hold N rows */
    oracle_combine(N, K, H, eo, 0, slot_of, w, y, acc, tok, N < 3 ? N : 3);
  }

  const int32_t M = rint_in(1, 5);
  int32_t* rc = xmalloc(sizeof(int32_t) * E * R);
  int32_t* lslot = xmalloc(sizeof(int32_t) * NK);
  int32_t* lflags = xmalloc(sizeof(int32_t) * R);
  if (oracle_ll_layout(N, K, E, R, M, idx, rc, lslot, lflags) < 0) FAIL("ll layout");
  for (int64_t i = 0; i < NK; i++)
    if (lslot[i] >= (int64_t)E * R * M) FAIL("ll slot beyond capacity");

  free(idx); free(w); free(x); free(ntpr); free(ntpe); free(in_rank); free(off); free(cnt);
  free(slot_of); free(src); free(rw); free(stats); free(eo); free(eof); free(y); free(acc);
  free(rc); free(lslot); free(lflags);
}

int main(int argc, char** argv) {
  int cases = argc > 1 ? atoi(argv[1]) : 300;
  codecs();
  for (int i = 0; i < cases; i++) one_case();
  /* invalid sizes are rejected, not read */
  if (oracle_layout(10, 2, 8, 4, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL) != -1) FAIL("N %% R");
  if (oracle_ll_layout(8, 2, 8, 4, 0, NULL, NULL, NULL, NULL) != -1) FAIL("M < 1");
  printf("oracle driver: %d cases clean\n", cases);
  return 0;
}
