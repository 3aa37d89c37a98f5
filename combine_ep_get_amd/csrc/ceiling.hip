// ceiling.hip -- plain kernels that measure what this GPU's HBM delivers for
// the traffic patterns of the EP path, and the known-size reference used to
// scale rocprof FETCH_SIZE / WRITE_SIZE counters.  Not part of the EP path:
// the benchmark times them beside the EP kernels so that each kernel can be
// judged against the best rate its own access pattern reaches on the same
// box, as well as against the 8 TB/s peak.
//
//   copy / write / read : linear sweeps with P 16-byte accesses per thread
//                         (P = 4 or 1: fewer accesses per thread, more
//                         threads, is faster for writes on MI355X);
//   scatter             : dispatch's traffic without its arithmetic or tags:
//                         token row t (R 16-byte chunks) is read once and
//                         written to the K rows map[t][0..K-1] of dst (one
//                         wavefront per token, LDS-staged 2 KiB pieces, and
//                         an XCD-placed item form);
//   gather              : combine's traffic without its arithmetic: the K
//                         rows map[t][0..K-1] of src are read and one row
//                         (their XOR, so that no load is dead) is written
//                         to dst[t], through to memory as combine writes y.
// The map is the real slot map of a workload (slot_of), so the addresses are
// exactly the EP kernels'.  Rows named -1 are skipped (scatter) or read as
// row 0 (gather, like combine's branch-free loads).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {
constexpr int kThreads = 256;

template <int P>
__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, int64_t n16) {
  const int64_t base = ((int64_t)blockIdx.x * kThreads * P) + threadIdx.x;
  u32x4 v[P];
#pragma unroll
  for (int i = 0; i < P; i++) {
    const int64_t j = base + (int64_t)i * kThreads;
    if (j < n16) v[i] = __builtin_nontemporal_load(src + j);
  }
#pragma unroll
  for (int i = 0; i < P; i++) {
    const int64_t j = base + (int64_t)i * kThreads;
    if (j < n16) __builtin_nontemporal_store(v[i], dst + j);
  }
}

template <int P>
__global__ __launch_bounds__(kThreads) void write_kernel(u32x4* __restrict__ dst, int64_t n16,
                                                         uint32_t value) {
  const int64_t base = ((int64_t)blockIdx.x * kThreads * P) + threadIdx.x;
  const u32x4 v = {value, value, value, value};
#pragma unroll
  for (int i = 0; i < P; i++) {
    const int64_t j = base + (int64_t)i * kThreads;
    if (j < n16) __builtin_nontemporal_store(v, dst + j);
  }
}

template <int P>
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ src,
                                                        int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t base = ((int64_t)blockIdx.x * kThreads * P) + threadIdx.x;
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < P; i++) {
    const int64_t j = base + (int64_t)i * kThreads;
    if (j < n16) {
      const u32x4 v = __builtin_nontemporal_load(src + j);
      x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  if (x == 0x9E3779B9u) sink[threadIdx.x] = x;   // keeps the loads; practically never stores
}

// Scatter: one wavefront per token; the row is read into registers once
// (NV chunks per lane) and stored to each of the K rows.
template <int NV>
__global__ __launch_bounds__(kThreads) void scatter_kernel(const u32x4* __restrict__ src,
                                                           u32x4* __restrict__ dst,
                                                           const int32_t* __restrict__ map,
                                                           int N, int K, int R) {
  const int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= N) return;
  const int lane = threadIdx.x & 63;
  const u32x4* row = src + (int64_t)t * R;
  u32x4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; i++) {
    const int c = i * 64 + lane;
    if (c < R) v[i] = row[c];
  }
  for (int k = 0; k < K; k++) {
    const int s = map[(int64_t)t * K + k];
    if (s < 0) continue;
    u32x4* d = dst + (int64_t)s * R;
#pragma unroll
    for (int i = 0; i < NV; i++) {
      const int c = i * 64 + lane;
      if (c < R) __builtin_nontemporal_store(v[i], d + c);
    }
  }
}

// Scatter as (token, k, 128-chunk piece) workgroups of 128 threads, one
// chunk per thread, ordered so that the K workgroups reading one piece are 8
// apart (the hardware deals workgroups to the 8 XCDs round robin, so they
// share an XCD and its L2).  The fastest form of the pattern when the source
// rows are still in the Infinity Cache; from a cold cache it is much slower
// than scatter_kernel (the K reads of a piece are not merged).
__global__ __launch_bounds__(128) void scatter_items_kernel(const u32x4* __restrict__ src,
                                                            u32x4* __restrict__ dst,
                                                            const int32_t* __restrict__ map,
                                                            int N, int K, int R, int P) {
  const int64_t b = blockIdx.x;
  const int64_t lo = b & 7, hi = b >> 3;
  const int k = (int)(hi % K);
  const int64_t tp = (hi / K) * 8 + lo;
  const int t = (int)(tp / P), p = (int)(tp % P);
  if (t >= N) return;
  const int s = map[(int64_t)t * K + k];
  if (s < 0) return;
  const int c = p * 128 + threadIdx.x;
  if (c < R) __builtin_nontemporal_store(src[(int64_t)t * R + c], dst + (int64_t)s * R + c);
}

// Scatter as (token, 128-chunk piece) workgroups of four wavefronts: the
// piece is read once into LDS, then wavefront w stores it to rows
// map[t][w], map[t][w + 4], ... -- the form of the bf16 dispatch kernel.
__global__ __launch_bounds__(256) void scatter_pieces_kernel(const u32x4* __restrict__ src,
                                                             u32x4* __restrict__ dst,
                                                             const int32_t* __restrict__ map,
                                                             int N, int K, int R, int P) {
  __shared__ u32x4 piece[128];
  const int64_t b = blockIdx.x;
  const int t = (int)(b / P), p = (int)(b % P);
  if (t >= N) return;
  const int base = p * 128, n = min(128, R - base);
  if ((int)threadIdx.x < n) piece[threadIdx.x] = src[(int64_t)t * R + base + threadIdx.x];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  for (int k = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6); k < K; k += 4) {
    const int s = __builtin_amdgcn_readfirstlane(map[(int64_t)t * K + k]);
    if (s < 0) continue;
    u32x4* d = dst + (int64_t)s * R + base;
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int c = i * 64 + lane;
      if (c < n) __builtin_nontemporal_store(piece[c], d + c);
    }
  }
}

// Gather: one wavefront per (token, piece of 64 chunks); the K slots are
// uniform loads and all K rows of the piece are requested before any is used
// (K a template parameter, so the loads are unconditional and in flight
// together) -- the form the combine kernel uses.
template <int K>
__global__ __launch_bounds__(64) void gather_kernel(const u32x4* __restrict__ src,
                                                    u32x4* __restrict__ dst,
                                                    const int32_t* __restrict__ map, int N, int R,
                                                    int P) {
  const int64_t b = blockIdx.x;
  const int t = (int)(b / P), c = (int)(b % P) * 64 + threadIdx.x;
  if (t >= N) return;
  const int cc = c < R ? c : R - 1;
  u32x4 v[K];
#pragma unroll
  for (int k = 0; k < K; k++) {
    int s = map[(int64_t)t * K + k];
    s = s < 0 ? 0 : s;
    v[k] = __builtin_nontemporal_load(src + (int64_t)s * R + cc);
  }
  u32x4 x = v[0];
#pragma unroll
  for (int k = 1; k < K; k++) x ^= v[k];
  // written through to memory over the token's row, like the combine kernel
  // (a buffer store with the device-scope cache bit)
  if (c < R) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(dst + (int64_t)t * R, 0, R * 16, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(x, r, c * 16, 0, 16);
  }
}

int64_t blocks_of(int64_t n16, int per) { return (n16 + (int64_t)kThreads * per - 1) / ((int64_t)kThreads * per); }

int launched() { return hipGetLastError() == hipSuccess ? 0 : 3; }
}  // namespace

extern "C" {
// Read `bytes` (multiple of 16, 16-byte aligned) with `per` (1 or 4) 16-byte
// loads per thread; `sink` must hold 256 uint32.
int epc_read_p(const void* src, int64_t bytes, int per, void* sink, void* stream) {
  if (bytes < 0 || bytes % 16 || (uintptr_t)src % 16 || (per != 1 && per != 4)) return 1;
  const int64_t n16 = bytes / 16, blocks = blocks_of(n16, per);
  if (blocks == 0) return 0;
  if (per == 1)
    read_kernel<1><<<(unsigned)blocks, kThreads, 0, (hipStream_t)stream>>>((const u32x4*)src, n16,
                                                                           (uint32_t*)sink);
  else
    read_kernel<4><<<(unsigned)blocks, kThreads, 0, (hipStream_t)stream>>>((const u32x4*)src, n16,
                                                                           (uint32_t*)sink);
  return launched();
}

// Fill `bytes` (multiple of 16, 16-byte aligned) with a 32-bit pattern,
// `per` (1 or 4) 16-byte stores per thread.
int epc_write_p(void* dst, int64_t bytes, uint32_t value, int per, void* stream) {
  if (bytes < 0 || bytes % 16 || (uintptr_t)dst % 16 || (per != 1 && per != 4)) return 1;
  const int64_t n16 = bytes / 16, blocks = blocks_of(n16, per);
  if (blocks == 0) return 0;
  if (per == 1)
    write_kernel<1><<<(unsigned)blocks, kThreads, 0, (hipStream_t)stream>>>((u32x4*)dst, n16, value);
  else
    write_kernel<4><<<(unsigned)blocks, kThreads, 0, (hipStream_t)stream>>>((u32x4*)dst, n16, value);
  return launched();
}

// Copy `bytes` (multiple of 16, 16-byte aligned pointers) from src to dst,
// `per` (1 or 4) 16-byte loads and stores per thread.
int epc_copy_p(void* dst, const void* src, int64_t bytes, int per, void* stream) {
  if (bytes < 0 || bytes % 16 || ((uintptr_t)dst | (uintptr_t)src) % 16 || (per != 1 && per != 4))
    return 1;
  const int64_t n16 = bytes / 16, blocks = blocks_of(n16, per);
  if (blocks == 0) return 0;
  if (per == 1)
    copy_kernel<1><<<(unsigned)blocks, kThreads, 0, (hipStream_t)stream>>>((const u32x4*)src,
                                                                           (u32x4*)dst, n16);
  else
    copy_kernel<4><<<(unsigned)blocks, kThreads, 0, (hipStream_t)stream>>>((const u32x4*)src,
                                                                           (u32x4*)dst, n16);
  return launched();
}

// LDS of the current device: the per-workgroup maximum (what each CU-budget
// workgroup of the EP library reserves: it asks for sharedMemPerBlock) and
// the per-CU total.  Returns 0, or 3 when the properties cannot be read.
int epc_lds_info(int64_t* per_workgroup, int64_t* per_cu) {
  int dev = 0;
  hipDeviceProp_t prop;
  if (!per_workgroup || !per_cu) return 1;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return 3;
  *per_workgroup = (int64_t)prop.sharedMemPerBlock;
  *per_cu = (int64_t)prop.maxSharedMemoryPerMultiProcessor;
  return 0;
}

// Clocks of the current device as the runtime reports them: peak core clock
// and memory clock in kHz, memory bus width in bits.  Returns 0, or 3 when an
// attribute cannot be read.
int epc_clock_info(int64_t* core_khz, int64_t* mem_khz, int64_t* bus_bits) {
  int dev = 0, c = 0, m = 0, w = 0;
  if (!core_khz || !mem_khz || !bus_bits) return 1;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&c, hipDeviceAttributeClockRate, dev) != hipSuccess ||
      hipDeviceGetAttribute(&m, hipDeviceAttributeMemoryClockRate, dev) != hipSuccess ||
      hipDeviceGetAttribute(&w, hipDeviceAttributeMemoryBusWidth, dev) != hipSuccess)
    return 3;
  *core_khz = c;
  *mem_khz = m;
  *bus_bits = w;
  return 0;
}

// The four-access-per-thread forms (the counter-scaling reference).
int epc_read(const void* src, int64_t bytes, void* sink, void* stream) {
  return epc_read_p(src, bytes, 4, sink, stream);
}
int epc_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  return epc_copy_p(dst, src, bytes, 4, stream);
}
int epc_write(void* dst, int64_t bytes, uint32_t value, void* stream) {
  return epc_write_p(dst, bytes, value, 4, stream);
}

// Dispatch's pattern: src [N][row_bytes], dst [rows][row_bytes], map [N][K]
// int32 row indices in [-1, rows).  row_bytes a multiple of 16, at most
// 16 KiB (1024 chunks); pointers 16-byte aligned.  The caller guarantees the
// map's range.
int epc_scatter(const void* src, void* dst, const int32_t* map, int32_t N, int32_t K,
                int64_t row_bytes, void* stream) {
  if (N < 0 || K < 1 || row_bytes <= 0 || row_bytes % 16 || row_bytes > 16384 ||
      ((uintptr_t)src | (uintptr_t)dst) % 16)
    return 1;
  if (N == 0) return 0;
  const int R = (int)(row_bytes / 16);
  const int blocks = (N + kThreads / 64 - 1) / (kThreads / 64);
  hipStream_t st = (hipStream_t)stream;
  const u32x4* s = (const u32x4*)src;
  u32x4* d = (u32x4*)dst;
  if (R <= 64 * 4) scatter_kernel<4><<<blocks, kThreads, 0, st>>>(s, d, map, N, K, R);
  else if (R <= 64 * 8) scatter_kernel<8><<<blocks, kThreads, 0, st>>>(s, d, map, N, K, R);
  else if (R <= 64 * 14) scatter_kernel<14><<<blocks, kThreads, 0, st>>>(s, d, map, N, K, R);
  else scatter_kernel<16><<<blocks, kThreads, 0, st>>>(s, d, map, N, K, R);
  return launched();
}

// The same pattern as LDS-staged (token, piece) workgroups
// (scatter_pieces_kernel).  Same arguments as epc_scatter.
int epc_scatter_pieces(const void* src, void* dst, const int32_t* map, int32_t N, int32_t K,
                       int64_t row_bytes, void* stream) {
  if (N < 0 || K < 1 || row_bytes <= 0 || row_bytes % 16 || ((uintptr_t)src | (uintptr_t)dst) % 16)
    return 1;
  if (N == 0) return 0;
  const int R = (int)(row_bytes / 16);
  const int P = (R + 127) / 128;
  const int64_t blocks = (int64_t)N * P;
  if (blocks > INT32_MAX) return 1;
  scatter_pieces_kernel<<<(unsigned)blocks, 256, 0, (hipStream_t)stream>>>(
      (const u32x4*)src, (u32x4*)dst, map, N, K, R, P);
  return launched();
}

// The same pattern as (token, k, piece) workgroups placed by XCD
// (scatter_items_kernel).  Same arguments as epc_scatter.
int epc_scatter_items(const void* src, void* dst, const int32_t* map, int32_t N, int32_t K,
                      int64_t row_bytes, void* stream) {
  if (N < 0 || K < 1 || row_bytes <= 0 || row_bytes % 16 || ((uintptr_t)src | (uintptr_t)dst) % 16)
    return 1;
  if (N == 0) return 0;
  const int R = (int)(row_bytes / 16);
  const int P = (R + 127) / 128;
  const int64_t blocks = ((int64_t)N * P + 7) / 8 * 8 * K;
  if (blocks > INT32_MAX) return 1;
  scatter_items_kernel<<<(unsigned)blocks, 128, 0, (hipStream_t)stream>>>(
      (const u32x4*)src, (u32x4*)dst, map, N, K, R, P);
  return launched();
}

// Combine's pattern: src [rows][row_bytes] (rows >= 1), map [N][K] in
// [-1, rows), dst [N][row_bytes].  K <= 8, row_bytes a multiple of 16.
int epc_gather(const void* src, void* dst, const int32_t* map, int32_t N, int32_t K,
               int64_t row_bytes, void* stream) {
  if (N < 0 || K < 1 || K > 8 || row_bytes <= 0 || row_bytes % 16 ||
      ((uintptr_t)src | (uintptr_t)dst) % 16)
    return 1;
  if (N == 0) return 0;
  const int R = (int)(row_bytes / 16);
  const int P = (R + 63) / 64;
  const int64_t blocks = (int64_t)N * P;
  if (blocks > INT32_MAX) return 1;
  hipStream_t st = (hipStream_t)stream;
  const u32x4* s = (const u32x4*)src;
  u32x4* d = (u32x4*)dst;
  const unsigned g = (unsigned)blocks;
  switch (K) {
    case 1: gather_kernel<1><<<g, 64, 0, st>>>(s, d, map, N, R, P); break;
    case 2: gather_kernel<2><<<g, 64, 0, st>>>(s, d, map, N, R, P); break;
    case 3: gather_kernel<3><<<g, 64, 0, st>>>(s, d, map, N, R, P); break;
    case 4: gather_kernel<4><<<g, 64, 0, st>>>(s, d, map, N, R, P); break;
    case 5: gather_kernel<5><<<g, 64, 0, st>>>(s, d, map, N, R, P); break;
    case 6: gather_kernel<6><<<g, 64, 0, st>>>(s, d, map, N, R, P); break;
    case 7: gather_kernel<7><<<g, 64, 0, st>>>(s, d, map, N, R, P); break;
    default: gather_kernel<8><<<g, 64, 0, st>>>(s, d, map, N, R, P); break;
  }
  return launched();
}
}
