/*
 * oracle_mt.c -- threaded driver of the oracle: the CPU baseline that the
 * benchmark reports beside the GPU figures, and the parity checks of the
 * largest workloads.
 *
 * TEST INFRASTRUCTURE ONLY, like oracle.c (only the tests, the smoke check
 * and the CPU-baseline leg of the benchmark load it).
 *
 * Nothing here computes anything itself.  The token range [0, N) is cut into
 * `threads` contiguous pieces and each thread calls the single-threaded
 * oracle function on its piece (pointers offset to the piece's first token).
 * Every output element of dispatch and combine depends on one token only
 * (slots are global, so the receive buffers are shared, but no two tokens
 * write the same slot), so the result is the same bytes as one call over all
 * tokens; the tests check that.  Layout and the per-slot tags stay
 * single-threaded: the layout's queue order is a walk over all tokens.
 *
 * Build: compiled into liboracle.so together with oracle.c (-lpthread).
 */
#include <pthread.h>
#include <stdint.h>

void oracle_dispatch_bf16(int32_t N, int32_t K, int32_t H, const uint16_t* x,
                          const int32_t* slot_of, uint16_t* recv_x);
void oracle_dispatch_fp8(int32_t N, int32_t K, int32_t H, const uint16_t* x,
                         const int32_t* slot_of, uint8_t* recv_q, float* recv_scales);
void oracle_combine(int32_t N, int32_t K, int32_t H, const void* eo, int32_t eo_is_f32,
                    const int32_t* slot_of, const float* topk_weights, uint16_t* y,
                    float* acc_out, const int32_t* tokens, int32_t n_tokens);

enum { OP_DISPATCH_BF16, OP_DISPATCH_FP8, OP_COMBINE };
#define MT_MAX_THREADS 256

typedef struct {
  int op;
  int32_t t0, t1, K, H;
  const uint16_t* x;
  const int32_t* slot_of;
  void* recv_x;
  float* recv_scales;
  const void* eo;
  int32_t eo_is_f32;
  const float* w;
  uint16_t* y;
  float* acc;
} job_t;

static void* run_piece(void* arg) {
  const job_t* j = (const job_t*)arg;
  const int32_t n = j->t1 - j->t0;
  const int64_t t0 = j->t0;
  if (n <= 0) return 0;
  switch (j->op) {
    case OP_DISPATCH_BF16:
      oracle_dispatch_bf16(n, j->K, j->H, j->x + t0 * j->H, j->slot_of + t0 * j->K,
                           (uint16_t*)j->recv_x);
      break;
    case OP_DISPATCH_FP8:
      oracle_dispatch_fp8(n, j->K, j->H, j->x + t0 * j->H, j->slot_of + t0 * j->K,
                          (uint8_t*)j->recv_x, j->recv_scales);
      break;
    default:
      oracle_combine(n, j->K, j->H, j->eo, j->eo_is_f32, j->slot_of + t0 * j->K,
                     j->w + t0 * j->K, j->y ? j->y + t0 * j->H : 0,
                     j->acc ? j->acc + t0 * j->H : 0, 0, 0);
      break;
  }
  return 0;
}

/* Run `proto` over [0, N) in `threads` contiguous pieces; 0 on success, -1 if
 * a thread could not be started (the pieces that did start are joined, the
 * rest run on the calling thread, so the result is complete either way). */
static int run_split(const job_t* proto, int32_t N, int threads) {
  pthread_t th[MT_MAX_THREADS];
  job_t jobs[MT_MAX_THREADS];
  int started[MT_MAX_THREADS];
  int rc = 0;
  if (threads < 1) threads = 1;
  if (threads > MT_MAX_THREADS) threads = MT_MAX_THREADS;
  for (int i = 0; i < threads; i++) {
    jobs[i] = *proto;
    jobs[i].t0 = (int32_t)((int64_t)N * i / threads);
    jobs[i].t1 = (int32_t)((int64_t)N * (i + 1) / threads);
    started[i] = pthread_create(&th[i], 0, run_piece, &jobs[i]) == 0;
    if (!started[i]) rc = -1;
  }
  for (int i = 0; i < threads; i++) {
    if (started[i])
      pthread_join(th[i], 0);
    else
      run_piece(&jobs[i]);
  }
  return rc;
}

int oracle_dispatch_bf16_mt(int32_t N, int32_t K, int32_t H, const uint16_t* x,
                            const int32_t* slot_of, uint16_t* recv_x, int threads) {
  job_t j = {0};
  j.op = OP_DISPATCH_BF16;
  j.K = K;
  j.H = H;
  j.x = x;
  j.slot_of = slot_of;
  j.recv_x = recv_x;
  return run_split(&j, N, threads);
}

int oracle_dispatch_fp8_mt(int32_t N, int32_t K, int32_t H, const uint16_t* x,
                           const int32_t* slot_of, uint8_t* recv_q, float* recv_scales,
                           int threads) {
  job_t j = {0};
  j.op = OP_DISPATCH_FP8;
  j.K = K;
  j.H = H;
  j.x = x;
  j.slot_of = slot_of;
  j.recv_x = recv_q;
  j.recv_scales = recv_scales;
  return run_split(&j, N, threads);
}

int oracle_combine_mt(int32_t N, int32_t K, int32_t H, const void* eo, int32_t eo_is_f32,
                      const int32_t* slot_of, const float* topk_weights, uint16_t* y,
                      float* acc_out, int threads) {
  job_t j = {0};
  j.op = OP_COMBINE;
  j.K = K;
  j.H = H;
  j.eo = eo;
  j.eo_is_f32 = eo_is_f32;
  j.slot_of = slot_of;
  j.w = topk_weights;
  j.y = y;
  j.acc = acc_out;
  return run_split(&j, N, threads);
}
