/*
 * Drives the host-side code of libepget (validation, capacity and workspace
 * sizing, error paths) with random and extreme descriptors, in a build with
 * host-only -fsanitize=address,undefined, so that integer overflow or an
 * out-of-bounds access in the host logic is reported.  No call here reaches a
 * device: every one is rejected by validation or is host-only by contract.
 * Test infrastructure only.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "ep_get.h"

static uint64_t st = 0x243F6A8885A308D3ull;
static uint32_t rnd(void) {
  st ^= st >> 12; st ^= st << 25; st ^= st >> 27;
  return (uint32_t)((st * 0x2545F4914F6CDD1Dull) >> 32);
}
static int32_t pick(void) {
  static const int32_t v[] = {-2147483647 - 1, -7, -1, 0, 1, 2, 3, 7, 8, 16, 31, 32, 33, 128, 255,
                              256, 257, 1023, 1024, 1025, 4096, 65536, 1 << 20, 1 << 28,
                              2147483647};
  if (rnd() & 1) return v[rnd() % (sizeof v / sizeof v[0])];
  return (int32_t)(rnd() % 5000);
}
#define FAIL(...) do { fprintf(stderr, __VA_ARGS__); fputc('\n', stderr); exit(1); } while (0)

int main(void) {
  void* fake = (void*)(uintptr_t)256;  /* never dereferenced */
  for (int i = 0; i < 200000; i++) {
    ep_problem_t p = {pick(), pick(), pick(), pick(), pick(), pick(), (int32_t)(rnd() % 3),
                      (int32_t)(rnd() % 10), pick()};
    const int64_t cap = ep_recv_capacity(&p);
    const int64_t ws = ep_workspace_bytes(&p);
    const int64_t llc = ep_ll_capacity(&p, pick());
    if ((cap < 0) != (ws < 0)) FAIL("capacity and workspace disagree on validity");
    if (cap > INT32_MAX || llc > INT32_MAX) FAIL("bound beyond int32");
    if (ws >= 0 && ws % 256) FAIL("workspace not a multiple of 256");
    /* argument errors: misaligned workspace, missing descriptor / pointers */
    if (ep_get_layout(&p, fake, fake, fake, fake, fake, fake, fake, (void*)(uintptr_t)260, NULL) == 0)
      FAIL("misaligned workspace accepted");
    if (ep_dispatch_ex(&p, NULL, NULL) != EP_ERR_INVALID_ARG) FAIL("NULL args accepted");
    ep_dispatch_args_t a = {0};
    a.recv_capacity = (int64_t)pick() - 1;
    a.flags = rnd() % 4;
    const int rc = ep_dispatch_ex(&p, &a, NULL);
    if (rc == EP_OK && p.num_tokens > 0) FAIL("dispatch without buffers accepted");
  }
  if (ep_get_layout(NULL, 0, 0, 0, 0, 0, 0, 0, 0, 0) != EP_ERR_INVALID_ARG) FAIL("NULL descriptor");
  if (ep_combine(NULL, 0, 0, 0, 0, 0, 0) != EP_ERR_INVALID_ARG) FAIL("NULL descriptor");
  if (ep_layout_error(NULL, NULL, NULL) != EP_ERR_INVALID_ARG) FAIL("NULL workspace");
  for (int s = -3; s < 8; s++)
    if (!ep_status_str(s)) FAIL("status string");
  printf("host driver clean\n");
  return 0;
}
