// cvt_sweep.hip -- test helper: runs the gfx950 float32 -> OCP E4M3
// conversion instruction (v_cvt_pk_fp8_f32, round to nearest even,
// saturating) over a contiguous range of float32 bit patterns, so that a test
// can compare every code it produces with the CPU oracle's encoder.  The
// fused-quantisation dispatch kernels rely on this instruction for every
// scaled value they encode (all of them lie below 464 in magnitude).
//
// Lanes take four consecutive bit patterns and pack their codes into one
// 32-bit word the way the dispatch kernels do: the first two through the low
// half (word_sel = false), the next two through the high half (word_sel = true).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {
__global__ __launch_bounds__(256) void cvt_sweep_kernel(uint32_t first, int64_t n_words,
                                                        uint32_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_words) return;
  const uint32_t b = first + (uint32_t)(4 * i);
  const float y0 = __uint_as_float(b), y1 = __uint_as_float(b + 1u);
  const float y2 = __uint_as_float(b + 2u), y3 = __uint_as_float(b + 3u);
  int word = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  word = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, word, true);
  out[i] = (uint32_t)word;
}
}  // namespace

extern "C" {
// Codes of the float32 bit patterns first, first + 1, ..., first + n - 1 into
// out[0, n) (device memory).  n must be a multiple of 4 and the range must
// not wrap past 0xFFFFFFFF.  Returns 0, 1 for bad arguments, 3 for a launch
// failure.
int cvt_e4m3_sweep(uint32_t first, int64_t n, void* out, void* stream) {
  if (n < 0 || n % 4 != 0 || (int64_t)first + n > (int64_t)1 << 32) return 1;
  const int64_t words = n / 4;
  if (words == 0) return 0;
  const int64_t blocks = (words + 255) / 256;
  cvt_sweep_kernel<<<(unsigned)blocks, 256, 0, (hipStream_t)stream>>>(first, words,
                                                                      (uint32_t*)out);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}
}
