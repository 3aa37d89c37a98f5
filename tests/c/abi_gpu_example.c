/*
 * A plain C caller of libepget (no Python, no torch): reads a problem and its
 * inputs from a directory, runs ep_get_layout -> ep_dispatch -> ep_combine on
 * the GPU with buffers from hipMalloc, and writes the outputs back as raw
 * files for the test to compare with the oracle.
 *
 *   abi_gpu_example <dir>
 *   <dir>/problem.txt   N H K E R A use_fp8
 *   <dir>/topk_idx.bin  int32 [N][K]      <dir>/topk_weights.bin  fp32 [N][K]
 *   <dir>/x.bin         bf16  [N][H]      <dir>/expert_out.bin    bf16 [cap][H]
 * writes slot_of.bin, offsets.bin, counts.bin, recv_x.bin, recv_scales.bin
 * (fp8 only), recv_src_idx.bin, y.bin.  Exit status 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ep_get.h"

#define HIP(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
  fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_)); exit(3); } } while (0)
#define EP(x) do { int r_ = (x); if (r_ != EP_OK) { \
  fprintf(stderr, "%s: %s\n", #x, ep_status_str(r_)); exit(4); } } while (0)

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(2); }
  void* p = malloc(bytes ? bytes : 1);
  if (!p || fread(p, 1, bytes, f) != bytes) { fprintf(stderr, "short read %s\n", path); exit(2); }
  fclose(f);
  return p;
}

static void write_file(const char* dir, const char* name, const void* p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(p, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(2); }
  fclose(f);
}

static void* dev_copy(const void* h, size_t bytes) {
  void* d = NULL;
  HIP(hipMalloc(&d, bytes ? bytes : 1));
  if (bytes) HIP(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
  return d;
}

static void* dev_alloc(size_t bytes) {
  void* d = NULL;
  HIP(hipMalloc(&d, bytes ? bytes : 1));
  return d;
}

static void fetch(const char* dir, const char* name, const void* d, size_t bytes) {
  void* h = malloc(bytes ? bytes : 1);
  if (bytes) HIP(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
  write_file(dir, name, h, bytes);
  free(h);
}

int main(int argc, char** argv) {
  if (argc != 2) { fprintf(stderr, "usage: %s <dir>\n", argv[0]); return 1; }
  const char* dir = argv[1];
  char path[4096];
  snprintf(path, sizeof path, "%s/problem.txt", dir);
  FILE* f = fopen(path, "r");
  ep_problem_t p;
  memset(&p, 0, sizeof p);
  if (!f || fscanf(f, "%d %d %d %d %d %d %d", &p.num_tokens, &p.hidden, &p.num_topk,
                   &p.num_experts, &p.num_ranks, &p.expert_alignment, &p.use_fp8) != 7) {
    fprintf(stderr, "bad problem.txt\n");
    return 2;
  }
  fclose(f);
  const size_t N = (size_t)p.num_tokens, H = (size_t)p.hidden, K = (size_t)p.num_topk;
  const size_t E = (size_t)p.num_experts, R = (size_t)p.num_ranks, G = H / 128;
  const int64_t cap = ep_recv_capacity(&p), ws = ep_workspace_bytes(&p);
  if (cap < 0 || ws < 0) { fprintf(stderr, "invalid problem\n"); return 2; }
  const size_t row = p.use_fp8 ? H : 2 * H;

  void* h_idx = read_file(dir, "topk_idx.bin", 4 * N * K);
  void* h_w = read_file(dir, "topk_weights.bin", 4 * N * K);
  void* h_x = read_file(dir, "x.bin", 2 * N * H);
  void* h_eo = read_file(dir, "expert_out.bin", 2 * (size_t)cap * H);
  void* d_idx = dev_copy(h_idx, 4 * N * K);
  void* d_w = dev_copy(h_w, 4 * N * K);
  void* d_x = dev_copy(h_x, 2 * N * H);
  void* d_eo = dev_copy(h_eo, 2 * (size_t)cap * H);
  int32_t* d_ntpr = dev_alloc(4 * R * R);
  int32_t* d_ntpe = dev_alloc(4 * R * E);
  uint8_t* d_in_rank = dev_alloc(N * R);
  int32_t* d_cnt = dev_alloc(4 * E);
  int32_t* d_off = dev_alloc(4 * (E + 1));
  int32_t* d_slot = dev_alloc(4 * N * K);
  void* d_ws = dev_alloc((size_t)ws);
  void* d_recv = dev_alloc(row * (size_t)cap);
  float* d_scales = p.use_fp8 ? dev_alloc(4 * G * (size_t)cap) : NULL;
  int32_t* d_src = dev_alloc(4 * (size_t)cap);
  float* d_rw = dev_alloc(4 * (size_t)cap);
  void* d_y = dev_alloc(2 * N * H);
  hipStream_t st;
  HIP(hipStreamCreate(&st));

  EP(ep_get_layout(&p, d_idx, d_ntpr, d_ntpe, d_in_rank, d_cnt, d_off, d_slot, d_ws, st));
  EP(ep_dispatch(&p, d_x, d_w, d_slot, d_off, d_cnt, d_recv, d_scales, d_src, d_rw, cap, st));
  EP(ep_combine(&p, d_eo, d_slot, d_w, d_y, cap, st));
  int32_t err = -1;
  EP(ep_layout_error(d_ws, &err, st));
  HIP(hipStreamSynchronize(st));

  fetch(dir, "slot_of.bin", d_slot, 4 * N * K);
  fetch(dir, "offsets.bin", d_off, 4 * (E + 1));
  fetch(dir, "counts.bin", d_cnt, 4 * E);
  fetch(dir, "recv_x.bin", d_recv, row * (size_t)cap);
  if (p.use_fp8) fetch(dir, "recv_scales.bin", d_scales, 4 * G * (size_t)cap);
  fetch(dir, "recv_src_idx.bin", d_src, 4 * (size_t)cap);
  fetch(dir, "y.bin", d_y, 2 * N * H);
  printf("abi_gpu_example: N=%zu H=%zu K=%zu E=%zu R=%zu cap=%lld error word=%d\n", N, H, K, E, R,
         (long long)cap, err);
  HIP(hipStreamDestroy(st));
  return 0;
}
