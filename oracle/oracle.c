/*
 * oracle.c -- plain CPU oracle for MoE expert-parallel dispatch / combine
 * with virtual EP ranks laid out in one address space.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP library and its Python binding) never calls it, links it or shares
 * a line of code with it.
 *
 * Everything here is a single-threaded loop written straight from the
 * definition of the operation, in the order the pages describe it:
 *
 *   - Lesson 14 "DeepSeek DeepEP core architecture and MoE expert-parallel
 *     communication operators" (hsthanb4 hpclearning), practice task: the
 *     dispatch step appends (token, row) to a per-expert queue while walking
 *     tokens in order and their top-k choices in order; the combine step looks
 *     up each (token, expert) result and adds weight * output into a float32
 *     accumulator for that token.
 *   - DeepEP book ch.1 "positioning and version boundaries" (bowenzhou.top),
 *     sec. 1.4: the V1 dispatch takes the layout tensors num_tokens_per_rank,
 *     is_token_in_rank, num_tokens_per_expert and an expert_alignment;
 *     sec. 1.1: the V2 dispatch takes num_experts and expert_alignment.
 *   - DeepEP walkthrough (2kiu.com news 5702702), sec. 2.3: tokens may be
 *     quantised to FP8 before they are sent; FlashMLA/DeepEP/DeepGEMM in
 *     practice (nlpx), sec. 4.1: FP8 data carries a per-block scale that is
 *     multiplied back on use.
 *
 * Readings taken where the pages are silent (each one is listed with its
 * reason in the design notes):
 *   token t belongs to source rank t / (N/R); expert e lives on rank e / (E/R);
 *   expert regions are padded to a multiple of the alignment A; inside a
 *   region the order is (source rank, token, k) ascending; topk_idx == -1 is
 *   "no expert" and is skipped; any other value outside [0, E) sets error bit
 *   0 and is skipped; the FP8 format is OCP E4M3FN with round-to-nearest-even
 *   and saturation to +-448; scale = amax/448 and the quantiser multiplies by
 *   448/amax (both one float32 division); where 448/amax overflows float32 the
 *   group is first multiplied by 2^64 (exact), since the codes only depend on
 *   v/amax; amax == 0 gives scale 1 and signed zero codes; padding slots carry
 *   no payload, source index -1, weight 0.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fPIC -shared oracle.c -lm
 * (no FMA contraction: every float product and sum is rounded on its own).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* number formats                                                      */
/* ------------------------------------------------------------------ */

/* bfloat16 -> float32: the bf16 bits are the top half of the float32. */
float oracle_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* float32 -> bfloat16, round to nearest, ties to even.  The 16 low bits are
 * dropped; the kept part goes up by one ulp when the dropped part is above
 * one half, or exactly one half and the kept part is odd.  A carry out of
 * the mantissa moves into the exponent, which is the correct result
 * (including overflow to infinity).  NaN stays NaN (quiet bit forced). */
uint16_t oracle_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t hi = u >> 16, lo = u & 0xFFFFu;
  if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1u;
  return (uint16_t)hi;
}

/* OCP FP8 E4M3FN decode: sign s, exponent field e (bias 7), mantissa m.
 * e == 0 is subnormal (m/8 * 2^-6); e == 15, m == 7 is NaN; no infinities. */
float oracle_e4m3_to_f32(uint8_t b) {
  int s = b >> 7, e = (b >> 3) & 0xF, m = b & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return s ? -NAN : NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return (float)(s ? -v : v);
}

/* float32 -> OCP FP8 E4M3FN, round to nearest even, saturating.
 * |y| >= 448 (the largest finite code 0x7E) gives +-448: values in [448, 464)
 * round to 448 anyway and anything larger saturates.  Below 2^-6 the step is
 * 2^-9 (subnormals); rounding up to 8 steps yields code 0x08, the smallest
 * normal, which is the right answer.  NaN keeps its sign and becomes 0x7F. */
uint8_t oracle_f32_to_e4m3(float y) {
  uint8_t s = signbit(y) ? 0x80 : 0x00;
  if (isnan(y)) return (uint8_t)(s | 0x7F);
  double a = fabs((double)y);
  if (a >= 448.0) return (uint8_t)(s | 0x7E);
  if (a < ldexp(1.0, -6)) {
    double m = nearbyint(a * 512.0); /* exact scaling; ties to even */
    return (uint8_t)(s | (uint8_t)m);
  }
  int ex;
  double fr = frexp(a, &ex); /* a = fr * 2^ex with fr in [0.5, 1) */
  int E = ex - 1;            /* a = (2 fr) * 2^E with 2 fr in [1, 2) */
  double m = nearbyint((2.0 * fr - 1.0) * 8.0);
  if (m == 8.0) {
    m = 0.0;
    E += 1;
  }
  return (uint8_t)(s | (uint8_t)(((E + 7) << 3) | (int)m));
}

/* array forms used by the tests */
void oracle_bf16_to_f32_n(const uint16_t* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_bf16_to_f32(in[i]);
}
void oracle_f32_to_bf16_n(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_f32_to_bf16(in[i]);
}
void oracle_e4m3_to_f32_n(const uint8_t* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_e4m3_to_f32(in[i]);
}
void oracle_f32_to_e4m3_n(const float* in, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_f32_to_e4m3(in[i]);
}

/* ------------------------------------------------------------------ */
/* layout                                                              */
/* ------------------------------------------------------------------ */

/* Receive capacity that always suffices: every (token, k) pair plus at most
 * A-1 padding slots per expert.  -1 when the arguments make no sense. */
int64_t oracle_capacity(int32_t N, int32_t K, int32_t E, int32_t A) {
  if (N < 0 || K < 1 || E < 1 || A < 1) return -1;
  return (int64_t)N * K + (int64_t)E * (A - 1);
}

/* Routing layout.
 *  num_tokens_per_expert[s][e]  pairs of source rank s routed to expert e
 *  is_token_in_rank[t][r]       1 iff some k routes token t to an expert on r
 *  num_tokens_per_rank[s][r]    tokens of source s with is_token_in_rank set
 *  num_recv_per_expert[e]       pairs received by expert e (all sources)
 *  expert_slot_offset[e]        first slot of expert e; regions padded to A
 *  slot_of[t][k]                slot of pair (t, k), -1 when it has no expert
 * Slots are handed out per expert queue, walking tokens in order and k in
 * order, exactly as the lesson-14 simulator appends to its expert queues;
 * with contiguous source blocks this is (source rank, token, k) order.
 * Returns -1 for bad sizes, else error flags (bit 0: an index outside
 * [-1, E)). */
int oracle_layout(int32_t N, int32_t K, int32_t E, int32_t R, int32_t A,
                  const int32_t* topk_idx, int32_t* num_tokens_per_rank,
                  int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank,
                  int32_t* expert_slot_offset, int32_t* num_recv_per_expert,
                  int32_t* slot_of) {
  if (N < 0 || K < 1 || E < 1 || R < 1 || A < 1) return -1;
  if (E % R != 0 || N % R != 0) return -1;
  int32_t L = E / R; /* experts per rank */
  int32_t T = N / R; /* tokens per source rank */
  int flags = 0;

  memset(num_tokens_per_expert, 0, sizeof(int32_t) * (size_t)R * E);
  memset(num_tokens_per_rank, 0, sizeof(int32_t) * (size_t)R * R);
  memset(is_token_in_rank, 0, (size_t)N * R);

  for (int32_t t = 0; t < N; t++) {
    int32_t src = t / T;
    for (int32_t k = 0; k < K; k++) {
      int32_t e = topk_idx[(int64_t)t * K + k];
      if (e == -1) continue;
      if (e < -1 || e >= E) {
        flags |= 1;
        continue;
      }
      num_tokens_per_expert[(int64_t)src * E + e] += 1;
      is_token_in_rank[(int64_t)t * R + e / L] = 1;
    }
    for (int32_t r = 0; r < R; r++)
      num_tokens_per_rank[(int64_t)src * R + r] += is_token_in_rank[(int64_t)t * R + r];
  }

  expert_slot_offset[0] = 0;
  for (int32_t e = 0; e < E; e++) {
    int32_t cnt = 0;
    for (int32_t s = 0; s < R; s++) cnt += num_tokens_per_expert[(int64_t)s * E + e];
    num_recv_per_expert[e] = cnt;
    int32_t padded = (cnt + A - 1) / A * A;
    expert_slot_offset[e + 1] = expert_slot_offset[e] + padded;
  }

  int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  if (!fill) return -1;
  for (int32_t e = 0; e < E; e++) fill[e] = expert_slot_offset[e];
  for (int32_t t = 0; t < N; t++) {
    for (int32_t k = 0; k < K; k++) {
      int32_t e = topk_idx[(int64_t)t * K + k];
      if (e < 0 || e >= E) {
        slot_of[(int64_t)t * K + k] = -1;
        continue;
      }
      slot_of[(int64_t)t * K + k] = fill[e];
      fill[e] += 1;
    }
  }
  free(fill);
  return flags;
}

/* Per-slot metadata that travels with the payload: the source token and the
 * gate weight of the pair; padding and unused slots get -1 and 0. */
void oracle_recv_meta(int32_t N, int32_t K, int64_t cap, const int32_t* slot_of,
                      const float* topk_weights, int32_t* recv_src_idx,
                      float* recv_topk_weights) {
  for (int64_t s = 0; s < cap; s++) {
    recv_src_idx[s] = -1;
    recv_topk_weights[s] = 0.0f;
  }
  for (int32_t t = 0; t < N; t++)
    for (int32_t k = 0; k < K; k++) {
      int32_t s = slot_of[(int64_t)t * K + k];
      if (s < 0) continue;
      recv_src_idx[s] = t;
      recv_topk_weights[s] = topk_weights[(int64_t)t * K + k];
    }
}

/* Low-latency layout: every expert e owns R sub-blocks of M rows, one per
 * source rank, so slot (e*R + s)*M + j holds the j-th pair of source s routed
 * to e, counting in token order then k order (the lesson-14 queue order,
 * restricted to one source).  Pairs beyond M in a sub-block get no slot and
 * set bit 1 of the source's flags; indices outside [-1, E) set bit 0.
 *   recv_count[e][s]  rows used in sub-block (e, s)  (at most M)
 *   slot_of[t][k]     slot of pair (t, k), -1 when it has none
 *   flags[s]          error bits of source s
 * The capacity is E*R*M slots.  Returns -1 for bad sizes, else the OR of the
 * flags. */
int oracle_ll_layout(int32_t N, int32_t K, int32_t E, int32_t R, int32_t M,
                     const int32_t* topk_idx, int32_t* recv_count, int32_t* slot_of,
                     int32_t* flags) {
  if (N < 0 || K < 1 || E < 1 || R < 1 || M < 1) return -1;
  if (E % R != 0 || N % R != 0) return -1;
  int32_t T = N / R;
  int all = 0;
  int32_t* cnt = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  if (!cnt) return -1;
  for (int32_t s = 0; s < R; s++) {
    int f = 0;
    for (int32_t e = 0; e < E; e++) cnt[e] = 0;
    for (int32_t t = s * T; t < (s + 1) * T; t++) {
      for (int32_t k = 0; k < K; k++) {
        int32_t e = topk_idx[(int64_t)t * K + k];
        int64_t q = (int64_t)t * K + k;
        slot_of[q] = -1;
        if (e == -1) continue;
        if (e < -1 || e >= E) {
          f |= 1;
          continue;
        }
        if (cnt[e] >= M) {
          f |= 2;
          continue;
        }
        slot_of[q] = ((e * R) + s) * M + cnt[e];
        cnt[e] += 1;
      }
    }
    for (int32_t e = 0; e < E; e++) recv_count[(int64_t)e * R + s] = cnt[e];
    flags[s] = f;
    all |= f;
  }
  free(cnt);
  return all;
}

/* ------------------------------------------------------------------ */
/* dispatch                                                            */
/* ------------------------------------------------------------------ */

/* bf16 payload: every pair's slot receives a bit copy of its token row.
 * recv_x is [cap][H]; only slots named by slot_of are written. */
void oracle_dispatch_bf16(int32_t N, int32_t K, int32_t H, const uint16_t* x,
                          const int32_t* slot_of, uint16_t* recv_x) {
  for (int32_t t = 0; t < N; t++)
    for (int32_t k = 0; k < K; k++) {
      int32_t s = slot_of[(int64_t)t * K + k];
      if (s < 0) continue;
      memcpy(recv_x + (int64_t)s * H, x + (int64_t)t * H, sizeof(uint16_t) * (size_t)H);
    }
}

/* FP8 quantisation of one token row, one scale per 128-channel group:
 *   amax = max |v| over the group (v is the exact float of the bf16 value)
 *   scale = amax / 448, inv = 448 / amax (one float32 division each)
 *   q = E4M3FN(v * inv)  (one float32 multiply, then the encoder above)
 * amax == 0 gives scale 1 and +-0 codes.  Dequantisation is q * scale.
 * What the codes approximate is v * 448 / amax, which does not change when
 * the whole group is multiplied by a power of two.  For amax below 448/FLT_MAX
 * (about 1.3e-36) the float32 inverse overflows, so there the values and
 * amax are first multiplied by 2^64 -- exact for every bf16 value, and it
 * leaves the codes of any group whose inverse is finite either way unchanged
 * -- and the codes are those of the scaled group.  The scale is still the
 * float32 quotient amax / 448 of the group as given. */
void oracle_quantize_row(int32_t H, const uint16_t* xrow, uint8_t* q, float* scales) {
  for (int32_t g = 0; g < H / 128; g++) {
    float amax = 0.0f;
    for (int32_t i = 0; i < 128; i++) {
      float a = fabsf(oracle_bf16_to_f32(xrow[128 * g + i]));
      if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
      scales[g] = 1.0f;
      for (int32_t i = 0; i < 128; i++)
        q[128 * g + i] = signbit(oracle_bf16_to_f32(xrow[128 * g + i])) ? 0x80 : 0x00;
      continue;
    }
    float scale = amax / 448.0f;
    float inv = 448.0f / amax;
    int pre = 0; /* power of two applied to the group before the multiply */
    if (isinf(inv)) {
      pre = 64;
      inv = 448.0f / ldexpf(amax, pre);
    }
    scales[g] = scale;
    for (int32_t i = 0; i < 128; i++) {
      float v = ldexpf(oracle_bf16_to_f32(xrow[128 * g + i]), pre);
      float prod = v * inv;
      q[128 * g + i] = oracle_f32_to_e4m3(prod);
    }
  }
}

/* FP8 payload: each token is quantised once, then its codes and scales are
 * copied to every slot of the token.  recv_q is [cap][H] bytes, recv_scales
 * [cap][H/128] float32.  H must be a multiple of 128. */
void oracle_dispatch_fp8(int32_t N, int32_t K, int32_t H, const uint16_t* x,
                         const int32_t* slot_of, uint8_t* recv_q, float* recv_scales) {
  int32_t G = H / 128;
  uint8_t* q = (uint8_t*)malloc((size_t)H);
  float* sc = (float*)malloc(sizeof(float) * (size_t)(G > 0 ? G : 1));
  if (!q || !sc) {
    free(q);
    free(sc);
    return;
  }
  for (int32_t t = 0; t < N; t++) {
    oracle_quantize_row(H, x + (int64_t)t * H, q, sc);
    for (int32_t k = 0; k < K; k++) {
      int32_t s = slot_of[(int64_t)t * K + k];
      if (s < 0) continue;
      memcpy(recv_q + (int64_t)s * H, q, (size_t)H);
      memcpy(recv_scales + (int64_t)s * G, sc, sizeof(float) * (size_t)G);
    }
  }
  free(q);
  free(sc);
}

/* Pre-quantised payload (DeepEP's dispatch also takes x as a pair of codes
 * and scales, DeepEP book ch.1 sec. 1.1 and 1.4): the given codes [N][H] and
 * scales [N][H/128] are copied unchanged to every slot of their token. */
void oracle_dispatch_quantized(int32_t N, int32_t K, int32_t H, const uint8_t* codes,
                               const float* scales, const int32_t* slot_of, uint8_t* recv_q,
                               float* recv_scales) {
  int32_t G = H / 128;
  for (int32_t t = 0; t < N; t++)
    for (int32_t k = 0; k < K; k++) {
      int32_t s = slot_of[(int64_t)t * K + k];
      if (s < 0) continue;
      memcpy(recv_q + (int64_t)s * H, codes + (int64_t)t * H, (size_t)H);
      memcpy(recv_scales + (int64_t)s * G, scales + (int64_t)t * G, sizeof(float) * (size_t)G);
    }
}

/* Zero padding (DeepEP's do_zero_padding): the padding rows of every expert
 * region, slots [off[e] + count[e], off[e+1]), are set to zero bytes; so are
 * their scale rows when scales != NULL.  row_bytes is 2H (bf16) or H (e4m3). */
void oracle_zero_padding(int32_t E, int32_t row_bytes, int32_t G, const int32_t* off,
                         const int32_t* count, uint8_t* recv_x, float* recv_scales) {
  for (int32_t e = 0; e < E; e++)
    for (int64_t s = (int64_t)off[e] + count[e]; s < off[e + 1]; s++) {
      memset(recv_x + s * row_bytes, 0, (size_t)row_bytes);
      if (recv_scales) memset(recv_scales + s * G, 0, sizeof(float) * (size_t)G);
    }
}

/* Running per-expert receive statistics (DeepEP's
 * cumulative_local_expert_recv_stats, book ch.1 sec. 1.1): stats[e] += count[e]. */
void oracle_accumulate_stats(int32_t E, const int32_t* count, int64_t* stats) {
  for (int32_t e = 0; e < E; e++) stats[e] += count[e];
}

/* ------------------------------------------------------------------ */
/* combine                                                             */
/* ------------------------------------------------------------------ */

/* Weighted top-k reduction back into token order:
 *   acc = 0;  for k = 0..K-1 with a slot:  acc = acc + w[t][k] * eo[slot][c]
 * in float32, product and sum rounded separately, then y = bf16(acc) (RNE).
 * eo is bf16 [cap][H] (eo_is_f32 == 0) or float32 [cap][H] (eo_is_f32 != 0).
 * tokens == NULL computes all N tokens into rows 0..N-1 of y/acc; otherwise
 * row i of y/acc is token tokens[i] (n_tokens rows).  y or acc may be NULL. */
void oracle_combine(int32_t N, int32_t K, int32_t H, const void* eo, int32_t eo_is_f32,
                    const int32_t* slot_of, const float* topk_weights, uint16_t* y,
                    float* acc_out, const int32_t* tokens, int32_t n_tokens) {
  int32_t rows = tokens ? n_tokens : N;
  for (int32_t i = 0; i < rows; i++) {
    int32_t t = tokens ? tokens[i] : i;
    for (int32_t c = 0; c < H; c++) {
      float acc = 0.0f;
      for (int32_t k = 0; k < K; k++) {
        int32_t s = slot_of[(int64_t)t * K + k];
        if (s < 0) continue;
        float v = eo_is_f32 ? ((const float*)eo)[(int64_t)s * H + c]
                            : oracle_bf16_to_f32(((const uint16_t*)eo)[(int64_t)s * H + c]);
        float p = topk_weights[(int64_t)t * K + k] * v;
        acc = acc + p;
      }
      if (acc_out) acc_out[(int64_t)i * H + c] = acc;
      if (y) y[(int64_t)i * H + c] = oracle_f32_to_bf16(acc);
    }
  }
}
