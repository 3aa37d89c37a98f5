// ep_get.hip -- MoE expert-parallel layout / dispatch / combine for one
// MI355X (gfx950), virtual EP ranks as partitions of one GPU's HBM.
//
// The operations (see include/ep_get.h for the full contract):
//   layout   : per-expert / per-rank histograms, is_token_in_rank, padded
//              expert offsets and a stable slot for every (token, k) pair.
//              DeepEP book ch.1 "positioning and version boundaries",
//              sec. 1.4 names the layout tensors; lesson 14 "DeepSeek DeepEP
//              core architecture", practice task, fixes the queue order.
//   dispatch : bit copy (bf16) or fused per-128-channel E4M3 quantise + copy
//              of each token row into its K slots.  DeepEP walkthrough
//              (2kiu.com) sec. 2.1 and 2.3; FlashMLA/DeepEP/DeepGEMM in
//              practice (nlpx) sec. 4.1 for the per-block scale.
//   combine  : fp32 weighted gather-reduce of the K expert rows, bf16 store.
//              Lesson 14, sec. 3 (top-k weighted sum) and practice task.
//   low-latency dispatch : routing and payload in one launch over fixed
//              (expert, source) sub-blocks (lesson 14 sec. 3; hotdry analysis,
//              "two kernel families").
//   options  : int64 routing indices, pre-quantised e4m3 input, zeroed
//              padding rows, running per-expert counts (DeepEP book ch.1
//              sec. 1.1), and a CU budget that keeps dispatch and combine on
//              a fixed number of CUs (hotdry analysis, "two kernel families").
//
// Nothing here is a contraction, so there is no MFMA: every kernel is bound by
// HBM bandwidth (dispatch, combine) or by latency (layout).  Design points:
//   - payload work in small independent items over the pieces of a row:
//     16-byte accesses, so that one wave instruction moves 1 KiB of a row
//     (fully coalesced 128-byte lines), and enough items to fill 256 CUs;
//   - a piece is read once and stored K times (dispatch: through LDS for
//     bf16, in VGPRs for the fused e4m3 path), or the K rows of a piece are
//     all put in flight before the fp32 accumulation (combine);
//   - streaming data uses non-temporal loads/stores so that the 14 KiB rows do
//     not evict the small metadata from L2 / the Infinity Cache, except that
//     combine writes y through to memory, leaving no dirty lines of it for
//     the next kernel to write back;
//   - no order-dependent atomics decide a slot: in-block ranks come from
//     per-wavefront 64-bit LDS masks (atomic OR, commutative) plus popcount,
//     so every output is deterministic run to run;
//   - no device-wide memset and no host sync: every word of every output is
//     written by some kernel on each call.
//
// Build: hipcc --offload-arch=gfx950 -O3 -ffp-contract=off (products and sums
// in combine are rounded separately, matching the contract bit for bit).

#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "ep_get.h"

// Cache policy of the streaming accesses (measured on MI355X): token rows
// read by dispatch use ordinary loads, expert rows read by combine use
// non-temporal loads; dispatch stores its rows non-temporally, combine writes
// y through to memory (st16y below).
#ifndef EP_DISPATCH_NT_LOAD
#define EP_DISPATCH_NT_LOAD 0
#endif
#ifndef EP_COMBINE_NT_LOAD
#define EP_COMBINE_NT_LOAD 1
#endif

namespace {

#ifndef EP_BLOCK
#define EP_BLOCK 256
#endif
constexpr int kThreads = EP_BLOCK;        // threads per block of the small utility kernels

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- memory ops
template <bool NT>
__device__ __forceinline__ u32x4 ld16(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// Payload stores of dispatch: non-temporal (EP_DISPATCH_STORE 0) or ordinary (1).
template <int POL>
__device__ __forceinline__ void st16p(u32x4* p, u32x4 v) {
  if constexpr (POL == 0) __builtin_nontemporal_store(v, p);
  else *p = v;
}
#ifndef EP_DISPATCH_STORE
#define EP_DISPATCH_STORE 0
#endif
__device__ __forceinline__ void st16(u32x4* p, u32x4 v) { st16p<EP_DISPATCH_STORE>(p, v); }

// Stores of combine's output y: chunk c of a token's row.  EP_COMBINE_STORE 2
// writes it through to memory (device scope) with a buffer store over the row
// (whose base is uniform per wavefront); 0 / 1 as st16p.
// Measured per prefill step (layout + dispatch + combine) with y written
// through instead of non-temporally: 197 -> 193 us back to back and 206 ->
// 201 us after a read pass over 1 GiB, because no dirty lines of y are left
// for the next kernel to write back; 4 us slower after a write pass (dirty
// lines of other data in the caches).  Writing the dispatched rows through as
// well gains another 2 us back to back but loses 3-5 us from a cold cache, so
// dispatch stays non-temporal.
#ifndef EP_COMBINE_STORE
#define EP_COMBINE_STORE 2
#endif
constexpr int kCpolDeviceScope = 16;  // SC1 in the cache-policy operand of gfx950 buffer ops
constexpr int kBufferWord3 = 0x00020000;  // raw buffer, 32-bit data format
__device__ __forceinline__ void st16y(u32x4* row, int H8, int c, u32x4 v) {
  if constexpr (EP_COMBINE_STORE == 2) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(row, 0, H8 * 16, kBufferWord3);
    __builtin_amdgcn_raw_buffer_store_b128(v, r, c * 16, 0, kCpolDeviceScope);
  } else {
    st16p<EP_COMBINE_STORE>(row + c, v);
  }
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ int lane_value(int v, int lane) {
  return __builtin_amdgcn_readlane(v, lane);
}

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// ---------------------------------------------------------------- formats
// bf16 halves of a 32-bit word -> float32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------- layout
// Work split shared by the host (workspace sizing) and the launches: blocks
// never straddle a source rank, so the per-source sums are sums over whole
// blocks.  Block b covers chunk (b % CB) of source (b / CB); a chunk is C
// tokens (the last chunk of a source may be shorter).
struct Plan {
  int32_t C, CB, B;
  int64_t o_err, o_cnt, o_rank, o_berr, bytes;
};

__host__ __device__ inline int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }

// Both layout phases stage the block's routing indices in LDS, a tile of
// whole tokens at a time, issuing every global load of the tile before any of
// them is used: these kernels are latency-bound, and a chain of dependent
// global round trips is what would make them slow.
constexpr int kCountTile = 8192;        // pairs staged per tile in phase 1 (32 KiB of LDS)
constexpr int kAssignTile = 4096;       // pairs staged per tile in phase 2 (16 KiB of LDS)
constexpr int kCountThreads = 512;
constexpr int kFlagBytes = 16384;       // LDS for is_token_in_rank staging

// Load n (1 <= n <= TILE) consecutive pairs of topk_idx into registers without
// branches (the index is clamped, so every lane issues its loads back to
// back), then store them to sidx[0, n).
// Routing indices come as int32 or int64.  An int64 value that does not fit
// in int32 becomes -2, which the kernels treat like every other value outside
// [-1, E): skipped and flagged EP_LAYOUT_ERR_INDEX.
__device__ __forceinline__ int to_expert(int32_t v) { return v; }
__device__ __forceinline__ int to_expert(int64_t v) {
  return (v >= -1 && v <= INT32_MAX) ? (int)v : -2;
}

template <int BLK, int TILE, typename I>
__device__ __forceinline__ void load_idx(int (&v)[TILE / BLK], const I* __restrict__ idx, int n) {
#pragma unroll
  for (int j = 0; j < TILE / BLK; j++)
    v[j] = to_expert(idx[min(j * BLK + (int)threadIdx.x, n - 1)]);
}

template <int BLK, int TILE>
__device__ __forceinline__ void store_idx(int* __restrict__ sidx, const int (&v)[TILE / BLK],
                                          int n) {
#pragma unroll
  for (int j = 0; j < TILE / BLK; j++) {
    const int q = j * BLK + (int)threadIdx.x;
    if (q < n) sidx[q] = v[j];
  }
}

// Phase 1: per-block expert histogram, is_token_in_rank rows and per-block
// per-rank token counts.  LDS atomics only count (order does not matter).
template <typename I>
__global__ __launch_bounds__(kCountThreads) void layout_count_kernel(
    const I* __restrict__ topk_idx, uint8_t* __restrict__ in_rank,
    int32_t* __restrict__ blk_cnt, int32_t* __restrict__ blk_rank, int32_t* __restrict__ blk_err,
    int K, int E, int R, int L, int T, int CB, int C) {
  __shared__ int sidx[kCountTile];
  __shared__ int hist[EP_MAX_EXPERTS];
  __shared__ int rcnt[EP_MAX_RANKS];
  __shared__ uint32_t flagw[kFlagBytes / 4];
  __shared__ int err;
  constexpr int BLK = kCountThreads;
  uint8_t* flags = reinterpret_cast<uint8_t*>(flagw);
  const int tid = threadIdx.x;
  const int b = blockIdx.x, src = b / CB, c = b % CB;
  const int t0 = src * T + c * C;
  const int t1 = src * T + min((c + 1) * C, T);
  const int tok_tile = kCountTile / K;          // whole tokens per tile
  const int tok_sub = kFlagBytes / R;           // tokens per flag pass (>= 64)
  for (int e = tid; e < E; e += BLK) hist[e] = 0;
  for (int r = tid; r < R; r += BLK) rcnt[r] = 0;
  if (tid == 0) err = 0;
  for (int tt = t0; tt < t1; tt += tok_tile) {
    const int ntok = min(tok_tile, t1 - tt);
    const int n = ntok * K;
    int v[kCountTile / BLK];
    load_idx<BLK, kCountTile>(v, topk_idx + (int64_t)tt * K, n);
    __syncthreads();  // previous tile fully consumed; counters initialised
    store_idx<BLK, kCountTile>(sidx, v, n);
#pragma unroll
    for (int j = 0; j < kCountTile / BLK; j++) {
      const int e = v[j];
      if (j * BLK + tid < n) {
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
        else if (e != -1) err = EP_LAYOUT_ERR_INDEX;
      }
    }
    for (int sub = 0; sub < ntok; sub += tok_sub) {
      const int nt = min(tok_sub, ntok - sub);
      for (int q = tid; q < (nt * R + 3) / 4; q += BLK) flagw[q] = 0u;
      __syncthreads();
      for (int q = tid; q < nt * K; q += BLK) {
        const int e = sidx[sub * K + q];
        if (e >= 0 && e < E) flags[(q / K) * R + e / L] = 1;
      }
      __syncthreads();
      // is_token_in_rank rows: 4 bytes per store when rows are word aligned
      uint8_t* out = in_rank + (int64_t)(tt + sub) * R;
      if ((R & 3) == 0 && (reinterpret_cast<uintptr_t>(in_rank) & 3) == 0) {
        for (int q = tid; q < nt * R / 4; q += BLK)
          reinterpret_cast<uint32_t*>(out)[q] = flagw[q];
      } else {
        for (int q = tid; q < nt * R; q += BLK) out[q] = flags[q];
      }
      // per-rank token counts: thread (r, slice) sums a column, one atomic each
      const int slices = BLK / R;  // R <= 256 so at least 2
      if (tid < slices * R) {
        const int r = tid % R, sl = tid / R;
        int cnt = 0;
        for (int t = sl; t < nt; t += slices) cnt += flags[t * R + r];
        if (cnt) atomicAdd(&rcnt[r], cnt);
      }
      __syncthreads();
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += BLK) blk_cnt[(int64_t)b * E + e] = hist[e];
  for (int r = tid; r < R; r += BLK) blk_rank[(int64_t)b * R + r] = rcnt[r];
  if (tid == 0) blk_err[b] = err;
}

// Phase 2: scan and stable slots, 1024 threads per block.  Every block first
// rebuilds, from the per-block histograms of phase 1, what it needs of the
// device-wide scan: its own exclusive prefix over earlier blocks for each
// expert and the per-expert totals, whose padded exclusive scan gives the
// region offsets.  This is redundant per block, but the histogram reads are
// split over 1024/E slices of blocks so that they are all in flight at once
// (together with the block's routing indices and the per-source rank counts),
// which is cheaper than a serial scan in a separate launch.  Block 0
// publishes the offsets, receive counts and error word; the first block of
// each source publishes that source's rows of the count matrices.
//
// Slots: pairs are taken in (token, k) order, 1024 per round; within a
// wavefront each lane ORs its bit into the 64-bit LDS mask of its expert, so
// the rank among equal experts is the popcount of the lower lanes' bits, plus
// the counts of lower wavefronts, plus everything the block and the earlier
// blocks already placed for that expert.
constexpr int kAssignThreads = 1024;
constexpr int kAssignWaves = kAssignThreads / 64;

template <typename I>
__global__ __launch_bounds__(kAssignThreads) void layout_assign_kernel(
    const I* __restrict__ topk_idx, const int32_t* __restrict__ blk_cnt,
    const int32_t* __restrict__ blk_rank, const int32_t* __restrict__ blk_err,
    int32_t* __restrict__ err_word, int32_t* __restrict__ num_tokens_per_rank,
    int32_t* __restrict__ num_tokens_per_expert, int32_t* __restrict__ num_recv,
    int32_t* __restrict__ off, int32_t* __restrict__ slot_of, int K, int E, int R, int T,
    int CB, int C, int B, int A) {
  constexpr int BLK = kAssignThreads;
  __shared__ int sidx[kAssignTile];
  __shared__ int base[EP_MAX_EXPERTS];
  __shared__ int rsum[EP_MAX_RANKS];
  __shared__ int wsum[kAssignWaves];
  // dynamic LDS: the per-wave expert masks [kAssignWaves][E]; its first
  // 3*BLK ints hold the slice partials of step (a)/(b), which are dead before
  // the masks are first written in step (c)
  extern __shared__ unsigned long long masks[];
  int* part_tot = reinterpret_cast<int*>(masks);
  int* part_pre = part_tot + BLK;
  int* part_src = part_pre + BLK;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.x, src = b / CB, c = b % CB;
  const int t0 = src * T + c * C;
  const int t1 = src * T + min((c + 1) * C, T);
  const int tok_tile = kAssignTile / K;
  const int s0 = src * CB, s1 = s0 + CB;

  // (a) loads, all issued before any is consumed and without branches (the
  //     addresses are clamped, the results masked): the first tile of routing
  //     indices, 16 per-block histogram entries per thread (one slice of the
  //     blocks for one expert), the per-source rank counts and the error flags
  constexpr int kPer = kAssignTile / BLK;
  const int ntok0 = min(tok_tile, t1 - t0);
  const int n0 = ntok0 * K;
  int iv[kPer];
  load_idx<BLK, kAssignTile>(iv, topk_idx + (int64_t)t0 * K, n0);
  const int S = BLK / E;  // slices of the block range per expert
  const int e_a = tid % E, sl = tid / E;
  const int bb0 = sl < S ? (int)((int64_t)B * sl / S) : 0;
  const int bb1 = sl < S ? (int)((int64_t)B * (sl + 1) / S) : 0;
  int cv[16];
#pragma unroll
  for (int u = 0; u < 16; u++) cv[u] = blk_cnt[(int64_t)min(bb0 + u, B - 1) * E + e_a];
  const int rv = blk_rank[(int64_t)s0 * R + min(tid, CB * R - 1)];
  const int evv = blk_err[min(tid, B - 1)];
  // consume
  store_idx<BLK, kAssignTile>(sidx, iv, n0);
  for (int r = tid; r < R; r += BLK) rsum[r] = 0;
  int tot = 0, pre = 0, srow = 0;
#pragma unroll
  for (int u = 0; u < 16; u++) {
    const int bi = bb0 + u;
    const int v = (bi < bb1) ? cv[u] : 0;
    tot += v;
    if (bi < b) pre += v;
    if (bi >= s0 && bi < s1) srow += v;
  }
  for (int bi = bb0 + 16; bi < bb1; bi++) {  // only when a slice spans more than 16 blocks
    const int v = blk_cnt[(int64_t)bi * E + e_a];
    tot += v;
    if (bi < b) pre += v;
    if (bi >= s0 && bi < s1) srow += v;
  }
  int ev = (b == 0 && tid < B) ? evv : 0;
  if (b == 0)
    for (int bb = tid + BLK; bb < B; bb += BLK) ev |= blk_err[bb];
  __syncthreads();  // rsum zeroed, sidx staged
  if (c == 0) {
    if (tid < CB * R) atomicAdd(&rsum[tid % R], rv);
    for (int q = tid + BLK; q < CB * R; q += BLK) atomicAdd(&rsum[q % R], blk_rank[(int64_t)s0 * R + q]);
  }
  if (sl < S) {
    part_tot[sl * E + e_a] = tot;
    part_pre[sl * E + e_a] = pre;
    part_src[sl * E + e_a] = srow;
  }
  __syncthreads();
  // (b) thread tid < E owns expert tid: reduce the slices, then a padded
  //     exclusive scan over experts across the whole block
  tot = 0;
  pre = 0;
  srow = 0;
  if (tid < E) {
    for (int k = 0; k < S; k++) {
      tot += part_tot[k * E + tid];
      pre += part_pre[k * E + tid];
      srow += part_src[k * E + tid];
    }
  }
  const int padded = (tid < E) ? (tot + A - 1) / A * A : 0;
  int x = padded;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int wpre = 0;
  for (int ww = 0; ww < w; ww++) wpre += wsum[ww];
  const int incl = wpre + x;
  // (c) publish, and set base[] to this block's first slot per expert
  if (tid < E) {
    const int offe = incl - padded;
    if (b == 0) {
      off[tid] = offe;
      num_recv[tid] = tot;
      if (tid == E - 1) off[E] = incl;
    }
    if (c == 0) num_tokens_per_expert[(int64_t)src * E + tid] = srow;
    base[tid] = offe + pre;
#pragma unroll
    for (int ww = 0; ww < kAssignWaves; ww++) masks[ww * E + tid] = 0ull;
  }
  if (c == 0)
    for (int r = tid; r < R; r += BLK) num_tokens_per_rank[(int64_t)src * R + r] = rsum[r];
  if (b == 0) {
    ev = __syncthreads_or(ev);
    if (tid == 0) *err_word = ev ? EP_LAYOUT_ERR_INDEX : 0;
  }
  __syncthreads();

  // (d) stable ranks, tile by tile (one tile unless the chunk is very large)
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int tt = t0; tt < t1; tt += tok_tile) {
    const int n = min(tok_tile, t1 - tt) * K;
    if (tt != t0) {
      int v[kPer];
      load_idx<BLK, kAssignTile>(v, topk_idx + (int64_t)tt * K, n);
      __syncthreads();
      store_idx<BLK, kAssignTile>(sidx, v, n);
      __syncthreads();
    }
    for (int r0 = 0; r0 < n; r0 += BLK) {
      const int p = r0 + tid;
      const int e = (p < n) ? sidx[p] : -1;
      const bool ok = (e >= 0 && e < E);
      if (ok) atomicOr(&masks[w * E + e], 1ull << lane);
      __syncthreads();
      int slot = -1;
      unsigned long long m = 0;
      if (ok) {
        m = masks[w * E + e];
        int pw = 0;
        for (int w2 = 0; w2 < w; w2++) pw += __popcll(masks[w2 * E + e]);
        slot = base[e] + pw + __popcll(m & below);
      }
      __syncthreads();
      if (ok && (m & below) == 0ull) {  // lowest lane of this expert in this wave
        atomicAdd(&base[e], __popcll(m));
        masks[w * E + e] = 0ull;
      }
      __syncthreads();
      if (p < n) slot_of[(int64_t)tt * K + p] = slot;
    }
  }
}

// floor(n / d) as the high half of n * ceil(2^32 / d): exact whenever
// n * d <= 2^32 (the error of the product is below n / 2^32 <= 1 / d, less than
// the distance from n / d to the next integer).  magic_of is the host side.
__device__ __forceinline__ uint32_t div_magic(uint32_t n, uint64_t magic) {
  return (uint32_t)(((uint64_t)n * magic) >> 32);
}
inline uint64_t magic_of(uint32_t d) { return ((uint64_t(1) << 32) + d - 1) / d; }

// Single-launch layout for problems with N*K <= kFusedMaxPairs, N <= kFlagBytes
// and E <= kFusedMaxExperts (the decode-sized workloads).
// No block needs another block's results: each block reads all N*K routing
// indices (from L2 after the first touch) and files every pair into one of
// four histograms by the position of its token: before the block's source,
// in the source before the block's chunk, from the chunk to the end of the
// source, after the source.  The first two give the block's prefix, all four
// the totals, the middle two the source's row of num_tokens_per_expert.  The
// same pass marks is_token_in_rank for every token of the block's source in
// LDS (N bytes at most), so the first block of a source also counts its rank
// row.  Then the padded scan, publishing and stable ranks run as in phase 2.
// Problems up to this many (token, k) pairs take the single-launch layout
// (measured on MI355X: 5.2 us at 288 pairs, 6.7 us at 8192, 7.6 us at 16384,
// 10.2 us at 32768 and 16.1 us at 65536, where the two-launch layout costs
// 10.0-10.8 us up to 32768 pairs and 11.7 us at 65536).
#ifndef EP_FUSED_MAX_PAIRS
#define EP_FUSED_MAX_PAIRS 32768
#endif
constexpr int kFusedThreads = 1024;
constexpr int kFusedMaxPairs = EP_FUSED_MAX_PAIRS;
constexpr int kFusedMaxExperts = 512;

template <typename I>
__global__ __launch_bounds__(kFusedThreads) void layout_fused_kernel(
    const I* __restrict__ topk_idx, uint8_t* __restrict__ in_rank,
    int32_t* __restrict__ err_word, int32_t* __restrict__ num_tokens_per_rank,
    int32_t* __restrict__ num_tokens_per_expert, int32_t* __restrict__ num_recv,
    int32_t* __restrict__ off, int32_t* __restrict__ slot_of, int N, int K, int E, int R, int T,
    int CB, int C, int A, uint64_t magic_k, uint64_t magic_l) {
  constexpr int BLK = kFusedThreads;
  constexpr int kWv = BLK / 64;
  __shared__ int sidx[kAssignTile];
  __shared__ int hist[4][kFusedMaxExperts];
  __shared__ int base[kFusedMaxExperts];
  __shared__ int rsum[EP_MAX_RANKS];
  __shared__ uint32_t flagw[kFlagBytes / 4];
  __shared__ int wsum[kWv];
  __shared__ int err;
  extern __shared__ unsigned long long masks[];  // [kWv][E]
  uint8_t* flags = reinterpret_cast<uint8_t*>(flagw);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.x, src = b / CB, c = b % CB;
  const int t0 = src * T + c * C;
  const int t1 = src * T + min((c + 1) * C, T);
  const int p0 = t0 * K, np = (t1 - t0) * K;

  // own chunk (<= kAssignTile pairs) first: it is needed last
  int iv[kAssignTile / BLK];
  load_idx<BLK, kAssignTile>(iv, topk_idx + p0, np);
  for (int q = tid; q < 4 * E; q += BLK) (&hist[0][0])[(q / E) * kFusedMaxExperts + q % E] = 0;
  for (int q = tid; q < (T * R + 3) / 4; q += BLK) flagw[q] = 0u;
  if (tid == 0) err = 0;
  __syncthreads();
  store_idx<BLK, kAssignTile>(sidx, iv, np);

  // (a) every pair of the problem, 16 loads in flight per thread; the class
  //     comes from comparing the pair's position with the (token-aligned)
  //     class boundaries.  Token and rank of a pair of the block's source come
  //     from multiplications (div_magic), so the loop reads no LDS and issues
  //     its LDS atomics and flag stores without waiting on any of them.
  const int NK = N * K, ps0 = src * T * K, ps1 = ps0 + T * K;
  for (int pb = 0; pb < NK; pb += 16 * BLK) {
    int v[16];
#pragma unroll
    for (int u = 0; u < 16; u++) v[u] = to_expert(topk_idx[min(pb + u * BLK + tid, NK - 1)]);
#pragma unroll
    for (int u = 0; u < 16; u++) {
      const int p = pb + u * BLK + tid;
      const int e = v[u];
      if (p < NK) {
        if ((unsigned)e < (unsigned)E) {
          const int cls = (p >= ps0) + (p >= p0) + (p >= ps1);
          atomicAdd(&hist[cls][e], 1);
          if (cls == 1 || cls == 2)
            flags[div_magic((uint32_t)(p - ps0), magic_k) * R + div_magic((uint32_t)e, magic_l)] = 1;
        } else if (e != -1) {
          err = EP_LAYOUT_ERR_INDEX;
        }
      }
    }
  }
  __syncthreads();

  // (b) prefix, totals, source row; padded exclusive scan over experts
  int tot = 0, pre = 0, srow = 0;
  if (tid < E) {
    const int h0 = hist[0][tid], h1 = hist[1][tid], h2 = hist[2][tid], h3 = hist[3][tid];
    pre = h0 + h1;
    srow = h1 + h2;
    tot = h0 + h1 + h2 + h3;
  }
  const int padded = (tid < E) ? (tot + A - 1) / A * A : 0;
  int x = padded;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[w] = x;
  // is_token_in_rank rows of this chunk, straight from the source's flags
  {
    const int fo = (t0 - src * T) * R, nb = (t1 - t0) * R;
    uint8_t* out = in_rank + (int64_t)t0 * R;
    if ((fo & 3) == 0 && (nb & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 3) == 0) {
      for (int q = tid; q < nb / 4; q += BLK) reinterpret_cast<uint32_t*>(out)[q] = flagw[fo / 4 + q];
    } else {
      for (int q = tid; q < nb; q += BLK) out[q] = flags[fo + q];
    }
  }
  if (c == 0) {
    for (int r = tid; r < R; r += BLK) rsum[r] = 0;
  }
  __syncthreads();
  if (c == 0) {  // per-rank token counts of the source: column sums, one atomic each
    const int slices = BLK / R;
    if (tid < slices * R) {
      const int r = tid % R, sl = tid / R;
      int cnt = 0;
      for (int t = sl; t < T; t += slices) cnt += flags[t * R + r];
      if (cnt) atomicAdd(&rsum[r], cnt);
    }
  }
  int wpre = 0;
  for (int ww = 0; ww < w; ww++) wpre += wsum[ww];
  const int incl = wpre + x;
  if (tid < E) {
    const int offe = incl - padded;
    if (b == 0) {
      off[tid] = offe;
      num_recv[tid] = tot;
      if (tid == E - 1) off[E] = incl;
    }
    if (c == 0) num_tokens_per_expert[(int64_t)src * E + tid] = srow;
    base[tid] = offe + pre;
#pragma unroll
    for (int ww = 0; ww < kWv; ww++) masks[ww * E + tid] = 0ull;
  }
  if (b == 0 && tid == 0) *err_word = err;
  __syncthreads();
  if (c == 0)
    for (int r = tid; r < R; r += BLK) num_tokens_per_rank[(int64_t)src * R + r] = rsum[r];

  // (c) stable ranks of this chunk
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int r0 = 0; r0 < np; r0 += BLK) {
    const int p = r0 + tid;
    const int e = (p < np) ? sidx[p] : -1;
    const bool ok = (e >= 0 && e < E);
    if (ok) atomicOr(&masks[w * E + e], 1ull << lane);
    __syncthreads();
    int slot = -1;
    unsigned long long m = 0;
    if (ok) {
      m = masks[w * E + e];
      int pw = 0;
      for (int w2 = 0; w2 < w; w2++) pw += __popcll(masks[w2 * E + e]);
      slot = base[e] + pw + __popcll(m & below);
    }
    __syncthreads();
    if (ok && (m & below) == 0ull) {
      atomicAdd(&base[e], __popcll(m));
      masks[w * E + e] = 0ull;
    }
    __syncthreads();
    if (p < np) slot_of[(int64_t)p0 + p] = slot;
  }
}

// N == 0: no blocks of the two kernels above run; publish zero outputs.
__global__ __launch_bounds__(kThreads) void layout_empty_kernel(
    int32_t* __restrict__ err_word, int32_t* __restrict__ num_tokens_per_rank,
    int32_t* __restrict__ num_tokens_per_expert, int32_t* __restrict__ num_recv,
    int32_t* __restrict__ off, int E, int R) {
  const int tid = threadIdx.x;
  for (int e = tid; e <= E; e += kThreads) {
    off[e] = 0;
    if (e < E) num_recv[e] = 0;
  }
  for (int q = tid; q < R * E; q += kThreads) num_tokens_per_expert[q] = 0;
  for (int q = tid; q < R * R; q += kThreads) num_tokens_per_rank[q] = 0;
  if (tid == 0) *err_word = 0;
}

// ---------------------------------------------------------------- dispatch
// Work of a dispatch launch besides the token rows, taken as wavefront items
// by blocks placed after the payload blocks of the grid (or by the items of a
// persistent grid), so that it runs alongside them and costs the payload
// blocks nothing:
//   - padding tags: every slot of [0, cap) that holds no pair gets source -1
//     and weight 0.  Item e < E tags expert e's padding slots
//     [off[e] + cnt[e], off[e+1]) (fewer than A); item E + u tags the slots of
//     [u * kTailSlots, (u+1) * kTailSlots) at or beyond off[E] (unit u exits at
//     once when its range lies below off[E]).  No search and no LDS.
//   - zeroed padding rows (DeepEP's do_zero_padding): item v takes padding
//     row j = v % (A-1) of expert e = v / (A-1), which exists iff
//     j < off[e+1] - off[e] - cnt[e]; consecutive items take consecutive rows
//     of one expert, so items past an expert's padding exit at once.
//   - the running per-expert receive counts (DeepEP's
//     cumulative_local_expert_recv_stats): one item.
// Every range is clamped to [0, cap), so offsets that ep_get_layout did not
// produce cannot send a store out of the buffers.
constexpr int kTailSlots = 512;

struct DispatchAux {
  const int32_t* off;   // [E+1] expert region offsets
  const int32_t* cnt;   // [E] pairs per expert
  int32_t* recv_src;    // tags, or NULL
  float* recv_w;
  u32x4* recv_x;        // zero padding: rows of row16 16-byte chunks
  float* recv_scales;   // and G scales per row (e4m3 payload), or NULL
  int64_t* stats;       // [E], or NULL
  int64_t cap;
  int E, A, row16, G;
  int64_t tag_items, zero_items, stat_items;
  __host__ __device__ int64_t items() const { return tag_items + zero_items + stat_items; }
};

__device__ __forceinline__ void tag_slots(int64_t lo, int64_t hi, const DispatchAux& a) {
  const int lane = threadIdx.x & 63;
  lo = lo < 0 ? 0 : lo;
  hi = hi > a.cap ? a.cap : hi;
  for (int64_t s = lo + lane; s < hi; s += 64) {
    if (a.recv_src) a.recv_src[s] = -1;
    if (a.recv_w) a.recv_w[s] = 0.0f;
  }
}

__device__ __forceinline__ void zero_padding_row(int64_t v, const DispatchAux& a) {
  const int lane = threadIdx.x & 63;
  const int e = (int)(v / (a.A - 1)), j = (int)(v % (a.A - 1));
  if (e >= a.E) return;
  const int64_t row = (int64_t)a.off[e] + a.cnt[e] + j;
  if (row < 0 || row >= a.off[e + 1] || row >= a.cap) return;  // [0, cap) even for foreign offsets
  const u32x4 z = {0u, 0u, 0u, 0u};
  u32x4* dst = a.recv_x + row * a.row16;
  for (int c = lane; c < a.row16; c += 64) st16(dst + c, z);
  if (a.recv_scales)
    for (int g = lane; g < a.G; g += 64) a.recv_scales[row * a.G + g] = 0.0f;
}

// One wavefront's auxiliary item v (0 <= v < a.items()).
__device__ __forceinline__ void aux_item(int64_t v, const DispatchAux& a) {
  if (v < a.tag_items) {
    if (v < a.E) {
      tag_slots((int64_t)a.off[v] + a.cnt[v], a.off[v + 1], a);
    } else {
      const int64_t lo = (v - a.E) * kTailSlots, used = a.off[a.E];
      tag_slots(lo > used ? lo : used, lo + kTailSlots, a);
    }
    return;
  }
  v -= a.tag_items;
  if (v < a.zero_items) {
    zero_padding_row(v, a);
    return;
  }
  for (int e = threadIdx.x & 63; e < a.E; e += 64) a.stats[e] += a.cnt[e];
}

// Blocks b >= 0 of the auxiliary range of a grid with BLK threads per block.
template <int BLK>
__device__ __forceinline__ void aux_block(int64_t b, const DispatchAux& a) {
  const int64_t v = b * (BLK / 64) + (threadIdx.x >> 6);
  if (v < a.items()) aux_item(v, a);
}

// Slot of pair (t, lane) for lanes < K, -1 elsewhere or when out of range.
__device__ __forceinline__ int load_slot(const int32_t* __restrict__ slot_of, int t, int K,
                                         int lane, int64_t cap) {
  int s = -1;
  if (lane < K) {
    s = slot_of[(int64_t)t * K + lane];
    if (s < 0 || (int64_t)s >= cap) s = -1;
  }
  return s;
}

__device__ __forceinline__ void write_meta(int t, int K, int lane, int myslot,
                                           const float* __restrict__ w,
                                           int32_t* __restrict__ recv_src,
                                           float* __restrict__ recv_w) {
  if (lane < K && myslot >= 0) {
    if (recv_src) recv_src[myslot] = t;
    if (recv_w) recv_w[myslot] = w[(int64_t)t * K + lane];
  }
}

// Copy one row (H8 16-byte chunks: bf16 or e4m3 codes) to the slots that
// lanes 0..K-1 of `myslot` name (-1: none).  TPT threads share the row; `vl` is this thread's
// index among them.  The row is read once into VGPRs per pass of NV chunks per
// thread and stored to every slot.
template <int TPT, int NV>
__device__ __forceinline__ void copy_row(const u32x4* __restrict__ row,
                                              u32x4* __restrict__ recv_x, int myslot, int K,
                                              int H8, int vl) {
  for (int base = 0; base < H8; base += TPT * NV) {
    u32x4 v[NV];
#pragma unroll
    for (int i = 0; i < NV; i++) {
      const int c = base + i * TPT + vl;
      if (c < H8) v[i] = ld16<EP_DISPATCH_NT_LOAD>(row + c);
    }
    for (int k = 0; k < K; k++) {
      const int s = lane_value(myslot, k);
      if (s < 0) continue;
      u32x4* dst = recv_x + (int64_t)s * H8;
#pragma unroll
      for (int i = 0; i < NV; i++) {
        const int c = base + i * TPT + vl;
        if (c < H8) st16(dst + c, v[i]);
      }
    }
  }
}

// E4M3 codes of the 16 consecutive channels this lane holds (two 16-byte
// chunks of bf16, v0 then v1), as part of a 128-channel group held by 8
// consecutive lanes 8j..8j+7, whose amax is reduced with xor-shuffles (all 64
// lanes must call this).  Sets `scale` to the group's scale:
//   amax = max |v|, scale = amax/448, inv = 448/amax (fp32 divisions),
//   code = E4M3(v * inv), round to nearest even, saturating; an all-zero
//   group has scale 1 and keeps each zero's sign.
__device__ __forceinline__ u32x4 quant16(u32x4 v0, u32x4 v1, float& scale) {
  float f[16];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    f[2 * j] = bf16_lo(v0[j]);
    f[2 * j + 1] = bf16_hi(v0[j]);
    f[8 + 2 * j] = bf16_lo(v1[j]);
    f[8 + 2 * j + 1] = bf16_hi(v1[j]);
  }
  float am = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; j++) am = fmaxf(am, fabsf(f[j]));
  am = fmaxf(am, __shfl_xor(am, 1));
  am = fmaxf(am, __shfl_xor(am, 2));
  am = fmaxf(am, __shfl_xor(am, 4));
  const bool zero = (am == 0.0f);
  scale = zero ? 1.0f : am / 448.0f;
  float inv = 448.0f / am;
  u32x4 q;
  if (!zero) {
    if (!__builtin_isfinite(inv)) {
      // amax < 448/FLT_MAX: the inverse overflows.  The codes approximate
      // v * 448/amax, which multiplying the whole group by 2^64 (exact for
      // bf16 values) leaves unchanged, so the scaled group is quantised.
      inv = 448.0f / (am * 0x1p64f);
#pragma unroll
      for (int j = 0; j < 16; j++) f[j] *= 0x1p64f;
    }
    // |f * inv| <= 448 (1 + 2^-23) < 464 here, where the hardware
    // conversion (v_cvt_pk_fp8_f32: OCP E4M3, round to nearest even,
    // saturating) is the contract's encoder; a GPU test compares it with the
    // oracle's encoder on every float32 below 464 in magnitude
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const float p0 = f[4 * j] * inv, p1 = f[4 * j + 1] * inv;
      const float p2 = f[4 * j + 2] * inv, p3 = f[4 * j + 3] * inv;
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
      q[j] = (uint32_t)word;
    }
  } else {
    // all-zero group: scale 1, each zero keeps its sign
#pragma unroll
    for (int j = 0; j < 4; j++) {
      uint32_t word = 0;
#pragma unroll
      for (int b = 0; b < 4; b++) word |= ((__float_as_uint(f[4 * j + b]) >> 24) & 0x80u) << (8 * b);
      q[j] = word;
    }
  }
  return q;
}

// Quantise one bf16 row of H channels (H % 128 == 0) to E4M3 with one fp32
// scale per 128-channel group and store codes and scales to the slots that
// lanes 0..K-1 of `myslot` name; one wavefront per row (the CU-budget and
// low-latency kernels).  NI pieces of 1024 channels per pass; after piece i,
// lanes 8i..8i+7 pick up the scales of its groups so that one store per slot
// writes the pass's scales.
template <int NI>
__device__ __forceinline__ void quant_row_fp8(const u32x4* __restrict__ row,
                                              u32x4* __restrict__ recv_q,
                                              float* __restrict__ recv_scales, int myslot, int K,
                                              int H, int lane) {
  const int H16 = H >> 4, G = H >> 7;
  for (int pbase = 0; pbase < H; pbase += NI * 1024) {
    u32x4 v[NI][2];
#pragma unroll
    for (int i = 0; i < NI; i++) {
      const int ch = pbase + i * 1024 + lane * 16;
      if (ch < H) {
        v[i][0] = ld16<EP_DISPATCH_NT_LOAD>(row + (ch >> 3));
        v[i][1] = ld16<EP_DISPATCH_NT_LOAD>(row + (ch >> 3) + 1);
      }
    }
    float my_scale = 0.0f;
#pragma unroll
    for (int i = 0; i < NI; i++) {
      const int ch = pbase + i * 1024 + lane * 16;
      float scale;
      const u32x4 q = quant16(v[i][0], v[i][1], scale);
      const float sv = __shfl(scale, 8 * (lane & 7));
      if ((lane >> 3) == i) my_scale = sv;
      if (ch < H) {
        for (int k = 0; k < K; k++) {
          const int s = lane_value(myslot, k);
          if (s < 0) continue;
          st16(recv_q + (int64_t)s * H16 + (ch >> 4), q);
        }
      }
    }
    const int g = (pbase >> 7) + lane;
    if (lane < NI * 8 && g < G) {
      for (int k = 0; k < K; k++) {
        const int s = lane_value(myslot, k);
        if (s < 0) continue;
        recv_scales[(int64_t)s * G + g] = my_scale;
      }
    }
  }
}

// Fused e4m3 rows as (token, piece) items, one wavefront each: item
// b = t * P + p quantises piece p of token t (1024 channels, 8 groups of 128,
// 16 channels per lane) and stores its codes and 8 scales to each of the
// token's K slots.  Measured on the e4m3 prefill workload: 48.7 us per launch
// (152.8 us per step, 165 us from a cold cache) against 54.1 us (156.5 /
// 167 us) for one wavefront per token walking its row piece by piece; the
// smaller items keep more rows in flight.  Splitting an item's K slots over
// S wavefronts that each quantise the piece again (placed on one XCD so that
// the piece is read from HBM once) gains nothing at S = 2 and loses at S = 4
// (158.3 / 175.3 us).  Lanes past H (when H % 1024 != 0) hold whole groups:
// they load clamped addresses, take part in the shuffles and store nothing.
// A launch holds at most kItemLaunch items; larger problems take several.
constexpr int64_t kItemLaunch = 1 << 30;

__global__ __launch_bounds__(64) void dispatch_fp8_item_kernel(
    const u32x4* __restrict__ x, const float* __restrict__ w, const int32_t* __restrict__ slot_of,
    u32x4* __restrict__ recv_q, float* __restrict__ recv_scales, int32_t* __restrict__ recv_src,
    float* __restrict__ recv_w, int N, int K, int H, int P, int64_t item0, int64_t items,
    int64_t cap, DispatchAux aux) {
  const int64_t b = item0 + blockIdx.x;
  if (b >= items) {
    aux_block<64>(b - items, aux);
    return;
  }
  const int t = (int)(b / P), p = (int)(b % P);
  const int lane = threadIdx.x;
  const int H16 = H >> 4, G = H >> 7;
  const int ch = p * 1024 + lane * 16;
  const int chc = ch < H ? ch : H - 16;
  const u32x4* row = x + (int64_t)t * (H >> 3);
  const u32x4 v0 = ld16<EP_DISPATCH_NT_LOAD>(row + (chc >> 3));
  const u32x4 v1 = ld16<EP_DISPATCH_NT_LOAD>(row + (chc >> 3) + 1);
  const int myslot = load_slot(slot_of, t, K, lane, cap);
  float scale;
  const u32x4 q = quant16(v0, v1, scale);
  for (int k = 0; k < K; k++) {
    const int s = lane_value(myslot, k);
    if (s < 0) continue;
    if (ch < H) {
      st16(recv_q + (int64_t)s * H16 + (ch >> 4), q);
      if ((lane & 7) == 0) recv_scales[(int64_t)s * G + (ch >> 7)] = scale;
    }
  }
  if (p == 0) write_meta(t, K, lane, myslot, w, recv_src, recv_w);
}

// The G scales of token t to each slot lanes 0..K-1 of `myslot` name.
__device__ __forceinline__ void copy_scales(const float* __restrict__ xs, int t, int G,
                                            float* __restrict__ recv_scales, int myslot, int K,
                                            int lane) {
  for (int g0 = 0; g0 < G; g0 += 64) {
    const int g = g0 + lane;
    const float sv = xs[(int64_t)t * G + min(g, G - 1)];
    for (int k = 0; k < K; k++) {
      const int s = lane_value(myslot, k);
      if (s >= 0 && g < G) recv_scales[(int64_t)s * G + g] = sv;
    }
  }
}

// bf16 rows as (token, piece) workgroups of kPieceWaves wavefronts: the piece
// (kPieceChunks 16-byte chunks, 2 KiB) is read from x once, into LDS, then
// wavefront w stores it to the slots of pairs w, w + kPieceWaves, ... and tags
// them on the token's first piece.  Workgroups past the pieces do the
// auxiliary work, after every piece has been issued.
// Measured at the prefill shape (per launch warm / cold, and the whole step
// warm / cold): one wavefront per token holding the row in VGPRs 97 / 112,
// 199 / 213 us; these workgroups 93 / 104, 195 / 206 us.  The piece size and
// the workgroup size both matter from a cold cache (1 KiB pieces: 148 us,
// 2 KiB pieces with 8 wavefronts: 113 us), where the reads of x have to come
// from HBM while the writes stream out.  The K readers of a piece must stay
// one read: (token, k, piece) workgroups that each read the piece win while
// x is in the Infinity Cache (85 us) but lose badly from a cold cache (163
// us), because the K concurrent reads of a piece are not merged into one HBM
// read.
#ifndef EP_PIECE_WAVES
#define EP_PIECE_WAVES 4
#endif
#ifndef EP_PIECE_CHUNKS
#define EP_PIECE_CHUNKS 128
#endif
constexpr int kPieceWaves = EP_PIECE_WAVES;
constexpr int kPieceThreads = 64 * kPieceWaves;
constexpr int kPieceChunks = EP_PIECE_CHUNKS;
static_assert(kPieceChunks % 64 == 0 && kPieceChunks <= kPieceThreads * 4, "piece geometry");

__global__ __launch_bounds__(kPieceThreads) void dispatch_piece_kernel(
    const u32x4* __restrict__ x, const float* __restrict__ w, const int32_t* __restrict__ slot_of,
    u32x4* __restrict__ recv_x, int32_t* __restrict__ recv_src, float* __restrict__ recv_w, int N,
    int K, int R, int P, int64_t item0, int64_t items, int64_t cap, DispatchAux aux) {
  __shared__ u32x4 piece[kPieceChunks];
  const int64_t b = item0 + blockIdx.x;
  if (b >= items) {
    aux_block<kPieceThreads>(b - items, aux);
    return;
  }
  const int t = (int)(b / P), p = (int)(b % P);
  const int tid = threadIdx.x, lane = tid & 63;
  const int base = p * kPieceChunks;
  const int n = min(kPieceChunks, R - base);  // chunks of this piece
  const u32x4* row = x + (int64_t)t * R + base;
#pragma unroll
  for (int j0 = 0; j0 < kPieceChunks; j0 += kPieceThreads) {
    const int j = j0 + tid;
    if (j < n) piece[j] = ld16<EP_DISPATCH_NT_LOAD>(row + j);
  }
  __syncthreads();
  for (int k = uniform(tid >> 6); k < K; k += kPieceWaves) {
    const int s = uniform(slot_of[(int64_t)t * K + k]);
    if (s < 0 || (int64_t)s >= cap) continue;
    u32x4* dst = recv_x + (int64_t)s * R + base;
#pragma unroll
    for (int i = 0; i < kPieceChunks / 64; i++) {
      const int c = i * 64 + lane;
      if (c < n) st16(dst + c, piece[c]);
    }
    if (p == 0 && lane == 0) {
      if (recv_src) recv_src[s] = t;
      if (recv_w) recv_w[s] = w[(int64_t)t * K + k];
    }
  }
}

// Pre-quantised e4m3 rows, one wavefront per token, kTokPerBlock per
// workgroup: the codes are read into VGPRs once (NV 16-byte chunks per lane
// per pass) and stored to each of the token's K slots, with their scales.
// Workgroups past the tokens do the auxiliary work.
constexpr int kTokPerBlock = kThreads / 64;

template <int NV>
__global__ __launch_bounds__(kThreads) void dispatch_token_kernel(
    const u32x4* __restrict__ x, const float* __restrict__ xs, const float* __restrict__ w,
    const int32_t* __restrict__ slot_of, u32x4* __restrict__ recv_x,
    float* __restrict__ recv_scales, int32_t* __restrict__ recv_src, float* __restrict__ recv_w,
    int N, int K, int H, int64_t cap, DispatchAux aux) {
  const int tok_blocks = (N + kTokPerBlock - 1) / kTokPerBlock;
  if ((int)blockIdx.x >= tok_blocks) {
    aux_block<kThreads>((int64_t)blockIdx.x - tok_blocks, aux);
    return;
  }
  const int t = uniform((int)blockIdx.x * kTokPerBlock + (int)(threadIdx.x >> 6));
  if (t >= N) return;
  const int lane = threadIdx.x & 63;
  const int myslot = load_slot(slot_of, t, K, lane, cap);
  copy_row<64, NV>(x + (int64_t)t * (H >> 4), recv_x, myslot, K, H >> 4, lane);
  copy_scales(xs, t, H >> 7, recv_scales, myslot, K, lane);
  write_meta(t, K, lane, myslot, w, recv_src, recv_w);
}

// ---------------------------------------------------------------- CU budget
// DeepEP bounds the SMs its kernels occupy (num_sms) so that expert GEMMs can
// run beside them.  Here the bound is a persistent grid of at most `budget`
// workgroups of 1024 threads, each reserving all of a CU's LDS (160 KiB on
// gfx950), so that no CU holds two of them, nor any other workgroup that uses
// LDS (a GEMM's): the kernel occupies min(budget, work) CUs alone and leaves
// the rest to other streams.  Its 16 wavefronts take work items
// i = blockIdx.x*16 + wave, stepping by gridDim.x*16; an item is one token
// row (dispatch), one token's 64-chunk column group (combine), or one item of
// the auxiliary work (aux_item).  Every item runs the same wavefront code as
// the wavefront-per-token paths, so results are identical.
constexpr int kPersistThreads = 1024;
constexpr int kPersistWaves = kPersistThreads / 64;
constexpr int kCombinePersistNV = 2;  // 16-byte chunks per lane per combine item

template <int MODE, int NV>  // MODE 0: bf16 copy, 1: fused e4m3, 2: pre-quantised e4m3
__global__ __launch_bounds__(kPersistThreads) void dispatch_persist_kernel(
    const u32x4* __restrict__ x, const float* __restrict__ xs, const float* __restrict__ w,
    const int32_t* __restrict__ slot_of, u32x4* __restrict__ recv_x,
    float* __restrict__ recv_scales, int32_t* __restrict__ recv_src, float* __restrict__ recv_w,
    int N, int K, int H, int64_t cap, DispatchAux aux) {
  extern __shared__ int lds[];  // only reserves the CU
  if (N < 0) lds[threadIdx.x] = 0;
  const int lane = threadIdx.x & 63;
  const int64_t n_aux = aux.items();
  const int64_t n_items = n_aux + N;
  for (int64_t i = (int64_t)blockIdx.x * kPersistWaves + (threadIdx.x >> 6); i < n_items;
       i += (int64_t)gridDim.x * kPersistWaves) {
    if (i < n_aux) {
      aux_item(i, aux);
      continue;
    }
    const int t = uniform((int)(i - n_aux));
    const int myslot = load_slot(slot_of, t, K, lane, cap);
    if constexpr (MODE == 0) {
      copy_row<64, NV>(x + (int64_t)t * (H >> 3), recv_x, myslot, K, H >> 3, lane);
    } else if constexpr (MODE == 1) {
      quant_row_fp8<NV>(x + (int64_t)t * (H >> 3), recv_x, recv_scales, myslot, K, H, lane);
    } else {
      copy_row<64, NV>(x + (int64_t)t * (H >> 4), recv_x, myslot, K, H >> 4, lane);
      copy_scales(xs, t, H >> 7, recv_scales, myslot, K, lane);
    }
    write_meta(t, K, lane, myslot, w, recv_src, recv_w);
  }
}

// ---------------------------------------------------------------- low latency
// One launch moves a decode-sized batch: routing and payload together.
// Expert e owns R sub-blocks of M rows, one per source rank; pair (t, k) of
// source s routed to e goes to slot (e*R + s)*M + j, j being its rank among
// source s's pairs routed to e in (token, k) order.  A slot therefore depends
// only on the pairs of its own source, and no device-wide scan is needed.
// Block (s, q) moves the rows of its own kLLWaves tokens, one wavefront per
// token.  The rank of one of its pairs is the number of earlier pairs of the
// source routed to the same expert: pairs of earlier tokens are counted with
// one pass of LDS atomic adds (a count, so their order does not matter), and
// the block's own pairs (at most kLLWaves*K <= 128) are ranked in one round
// of per-wavefront 64-bit masks and popcounts.  Block (s, 0) also counts all
// of the source's pairs, which gives recv_count, the flags and the running
// statistics.  Pairs beyond M in a sub-block get no slot and set
// EP_LAYOUT_ERR_OVERFLOW in the source's flags.
constexpr int kLLThreads = 256;
constexpr int kLLWaves = kLLThreads / 64;

// MODE 0: bf16 rows; 1: fused e4m3 quantisation; 2: pre-quantised e4m3 codes
// (x) and scales (xs) copied unchanged.  stats != NULL: the block (s, 0) adds
// its source's received rows per expert (atomic integer adds, so the sum is
// the same in any order).
template <int MODE, int NV, typename I>
__global__ __launch_bounds__(kLLThreads) void ll_dispatch_kernel(
    const I* __restrict__ topk_idx, const u32x4* __restrict__ x, const float* __restrict__ xs,
    const float* __restrict__ w, int32_t* __restrict__ recv_count, int32_t* __restrict__ slot_of,
    int32_t* __restrict__ flags, u32x4* __restrict__ recv_x, float* __restrict__ recv_scales,
    int32_t* __restrict__ recv_src, float* __restrict__ recv_w, int64_t* __restrict__ stats,
    int K, int E, int R, int T, int M, int H, int Q) {
  __shared__ int sidx[kAssignTile];
  __shared__ int sslot[kLLWaves * EP_MAX_TOPK];
  __shared__ int cnt[EP_MAX_EXPERTS];   // pairs of earlier tokens (q > 0) or all pairs (q == 0)
  __shared__ int ferr;
  extern __shared__ unsigned long long masks[];  // [kLLWaves][E]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int s = blockIdx.x / Q, q = blockIdx.x % Q;
  const int np = T * K;
  const int64_t p0 = (int64_t)s * T * K;
  const int per = (T + Q - 1) / Q;
  const int ta = min(T, q * per), tb = min(T, ta + per);
  const int own0 = ta * K, nown = (tb - ta) * K;
  // pairs this block reads: all of the source for q == 0, else those up to its last token
  const int nread = (q == 0) ? np : tb * K;
  int iv[kAssignTile / kLLThreads];
  if (nread > 0) load_idx<kLLThreads, kAssignTile>(iv, topk_idx + p0, nread);
  // A copied row (bf16 or pre-quantised codes) does not depend on the routing:
  // when it fits one pass, each wavefront requests its token's row now, so
  // the load latency overlaps the ranking below (per <= kLLWaves: at most one
  // token per wavefront).
  constexpr bool kCopy = (MODE != 1);
  const int rowc = (MODE == 2) ? (H >> 4) : (H >> 3);
  const bool prefetch = kCopy && rowc <= 64 * NV;
  const int tl0 = ta + wv;
  u32x4 row[NV];
  if (prefetch && tl0 < tb) {
    const u32x4* src = x + (int64_t)(s * T + tl0) * rowc;
#pragma unroll
    for (int i = 0; i < NV; i++) {
      const int c = i * 64 + lane;
      if (c < rowc) row[i] = ld16<EP_DISPATCH_NT_LOAD>(src + c);
    }
  }
  for (int e = tid; e < E; e += kLLThreads) {
    cnt[e] = 0;
#pragma unroll
    for (int ww = 0; ww < kLLWaves; ww++) masks[ww * E + e] = 0ull;
  }
  if (tid == 0) ferr = 0;
  __syncthreads();
  if (nread > 0) store_idx<kLLThreads, kAssignTile>(sidx, iv, nread);
  __syncthreads();
  // counts: pairs before the block's own tokens (q > 0), every pair (q == 0)
  const int ncount = (q == 0) ? np : own0;
  int myerr = 0;
  for (int p = tid; p < ncount; p += kLLThreads) {
    const int e = sidx[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    else if (e != -1) myerr |= EP_LAYOUT_ERR_INDEX;
  }
  // the block's own pairs: one round of masks (nown <= kLLThreads)
  const int e_own = (tid < nown) ? sidx[own0 + tid] : -1;
  const bool ok = (e_own >= 0 && e_own < E);
  if (ok) atomicOr(&masks[wv * E + e_own], 1ull << lane);
  if (myerr) atomicOr(&ferr, myerr);
  __syncthreads();
  if (q == 0) {
    for (int e = tid; e < E; e += kLLThreads) {
      const int got = min(cnt[e], M);
      recv_count[(int64_t)e * R + s] = got;
      if (stats && got)
        atomicAdd(reinterpret_cast<unsigned long long*>(stats + e), (unsigned long long)got);
      if (cnt[e] > M) atomicOr(&ferr, EP_LAYOUT_ERR_OVERFLOW);
    }
  }
  if (tid < nown) {
    int slot = -1;
    if (ok) {
      const unsigned long long below = (1ull << lane) - 1ull;
      int pw = 0;
      for (int w2 = 0; w2 < wv; w2++) pw += __popcll(masks[w2 * E + e_own]);
      // q == 0 owns the first tokens, so nothing of the source precedes them
      const int before = (q == 0) ? 0 : cnt[e_own];
      const int j = before + pw + __popcll(masks[wv * E + e_own] & below);
      if (j < M) slot = (e_own * R + s) * M + j;
    }
    sslot[tid] = slot;
    slot_of[p0 + own0 + tid] = slot;
  }
  __syncthreads();
  if (q == 0 && tid == 0) flags[s] = ferr;
  if (prefetch) {
    if (tl0 < tb) {
      const int t = uniform(s * T + tl0);
      const int myslot = (lane < K) ? sslot[(tl0 - ta) * K + lane] : -1;
      for (int k = 0; k < K; k++) {
        const int sl = lane_value(myslot, k);
        if (sl < 0) continue;
        u32x4* dst = recv_x + (int64_t)sl * rowc;
#pragma unroll
        for (int i = 0; i < NV; i++) {
          const int c = i * 64 + lane;
          if (c < rowc) st16(dst + c, row[i]);
        }
      }
      if constexpr (MODE == 2) copy_scales(xs, t, H >> 7, recv_scales, myslot, K, lane);
      write_meta(t, K, lane, myslot, w, recv_src, recv_w);
    }
    return;
  }
  for (int tl = ta + wv; tl < tb; tl += kLLWaves) {
    const int t = uniform(s * T + tl);
    const int myslot = (lane < K) ? sslot[(tl - ta) * K + lane] : -1;
    if constexpr (MODE == 1) {
      quant_row_fp8<NV>(x + (int64_t)t * (H >> 3), recv_x, recv_scales, myslot, K, H, lane);
    } else if constexpr (MODE == 2) {
      copy_row<64, NV>(x + (int64_t)t * (H >> 4), recv_x, myslot, K, H >> 4, lane);
      copy_scales(xs, t, H >> 7, recv_scales, myslot, K, lane);
    } else {
      copy_row<64, NV>(x + (int64_t)t * (H >> 3), recv_x, myslot, K, H >> 3, lane);
    }
    write_meta(t, K, lane, myslot, w, recv_src, recv_w);
  }
}

// N == 0 in the low-latency path: zero counts and flags.
__global__ __launch_bounds__(kThreads) void ll_empty_kernel(int32_t* __restrict__ recv_count,
                                                             int32_t* __restrict__ flags, int E,
                                                             int R) {
  for (int q = threadIdx.x; q < E * R; q += kThreads) recv_count[q] = 0;
  for (int q = threadIdx.x; q < R; q += kThreads) flags[q] = 0;
}

// ---------------------------------------------------------------- combine
// Combine: the K expert rows of a token are gathered and accumulated in
// ascending k, acc = acc + w_k * row_k (separately rounded multiply and add,
// matching the contract bit for bit), and stored as bf16 with
// round-to-nearest-even (v_cvt_pk_bf16_f32).  Loads are branch-free (the
// column index is clamped and invalid slots read row 0); only the
// accumulation skips slots that hold no pair.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <int TPT, int NV>
__device__ __forceinline__ void combine_load8(u32x4 (&v)[8][NV], const u32x4* __restrict__ eo,
                                              int myslot, int K, int base, int vl, int H8) {
#pragma unroll
  for (int j = 0; j < 8; j++) {
    int s = (j < K) ? lane_value(myslot, j) : -1;
    s = s < 0 ? 0 : s;
    const u32x4* r = eo + (int64_t)s * H8;
#pragma unroll
    for (int i = 0; i < NV; i++) {
      const int c = min(base + i * TPT + vl, H8 - 1);
      v[j][i] = ld16<EP_COMBINE_NT_LOAD>(r + c);
    }
  }
}

template <int NV>
__device__ __forceinline__ void combine_accum8(float (&acc)[NV][8], const u32x4 (&v)[8][NV],
                                               int myslot, float myw, int K) {
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const int s = (j < K) ? lane_value(myslot, j) : -1;
    if (s < 0) continue;
    const float wk = lane_value(myw, j);
#pragma unroll
    for (int i = 0; i < NV; i++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        acc[i][2 * q] = acc[i][2 * q] + wk * bf16_lo(v[j][i][q]);
        acc[i][2 * q + 1] = acc[i][2 * q + 1] + wk * bf16_hi(v[j][i][q]);
      }
  }
}

template <int TPT, int NV>
__device__ __forceinline__ void combine_store(const float (&acc)[NV][8], u32x4* __restrict__ yrow,
                                              int base, int vl, int H8) {
#pragma unroll
  for (int i = 0; i < NV; i++) {
    const int c = base + i * TPT + vl;
    if (c < H8) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; q++) o[q] = pack_bf16x2(acc[i][2 * q], acc[i][2 * q + 1]);
      st16y(yrow, H8, c, o);
    }
  }
}

template <int TPT, int NV>
__device__ __forceinline__ void combine_pass8(const u32x4 (&v)[8][NV], int myslot, float myw,
                                              int K, u32x4* __restrict__ yrow, int base, int vl,
                                              int H8) {
  float acc[NV][8];
#pragma unroll
  for (int i = 0; i < NV; i++)
#pragma unroll
    for (int j = 0; j < 8; j++) acc[i][j] = 0.0f;
  combine_accum8<NV>(acc, v, myslot, myw, K);
  combine_store<TPT, NV>(acc, yrow, base, vl, H8);
}

// The ordinary launch takes (token, piece) items, one wavefront each: item
// b = t * P + p reduces piece p of the token's rows (64 16-byte chunks, one
// per lane), with all K (or the next 8 of K) rows of the piece requested
// before any is used.  Measured on MI355X at hidden 7168: 85.9 us at the
// prefill shape and 20.1 us at the decode shape, against 88.8 / 23.2 us for
// one 896-thread workgroup per token (the whole rows requested at once) and
// 101 us for one wavefront walking the pieces of its token in turn; the
// reads dominate (eight rows read per row written), and many small
// independent items keep the most of them in flight.  Any row width is P
// pieces; K > 8 goes through groups of 8 rows, accumulated group after group
// so that the order over k is kept.
// KT = K (1..8): the token's slots and weights are uniform loads (scalar) that
// arrive together, so the row loads can all be issued after one wait.
template <int KT>
__global__ __launch_bounds__(64) void combine_piece_k_kernel(
    const u32x4* __restrict__ eo, const int32_t* __restrict__ slot_of,
    const float* __restrict__ w, u32x4* __restrict__ y, int N, int H8, int P, int64_t item0,
    int64_t cap) {
  const int64_t b = item0 + blockIdx.x;
  const int t = (int)(b / P), base = (int)(b % P) * 64;
  if (t >= N) return;
  const int lane = threadIdx.x;
  int s[KT];
  float wk[KT];
#pragma unroll
  for (int k = 0; k < KT; k++) {
    s[k] = slot_of[(int64_t)t * KT + k];
    wk[k] = w[(int64_t)t * KT + k];
    if (s[k] < 0 || (int64_t)s[k] >= cap) s[k] = -1;
  }
  const int c = base + lane;
  const int cc = c < H8 ? c : H8 - 1;
  u32x4 v[KT];
#pragma unroll
  for (int k = 0; k < KT; k++)
    v[k] = ld16<EP_COMBINE_NT_LOAD>(eo + (int64_t)(s[k] < 0 ? 0 : s[k]) * H8 + cc);
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; j++) acc[j] = 0.0f;
#pragma unroll
  for (int k = 0; k < KT; k++) {
    if (s[k] < 0) continue;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      acc[2 * q] = acc[2 * q] + wk[k] * bf16_lo(v[k][q]);
      acc[2 * q + 1] = acc[2 * q + 1] + wk[k] * bf16_hi(v[k][q]);
    }
  }
  if (c < H8) {
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; q++) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    st16y(y + (int64_t)t * H8, H8, c, o);
  }
}

// Any K (used for K > 8): slots per lane, groups of 8 rows.
__global__ __launch_bounds__(64) void combine_piece_kernel(
    const u32x4* __restrict__ eo, const int32_t* __restrict__ slot_of,
    const float* __restrict__ w, u32x4* __restrict__ y, int N, int K, int H8, int P, int64_t item0,
    int64_t cap) {
  const int64_t b = item0 + blockIdx.x;
  const int t = (int)(b / P), base = (int)(b % P) * 64;
  if (t >= N) return;
  const int lane = threadIdx.x;
  const int myslot = load_slot(slot_of, t, K, lane, cap);
  const float myw = (lane < K) ? w[(int64_t)t * K + lane] : 0.0f;
  float acc[1][8];
#pragma unroll
  for (int j = 0; j < 8; j++) acc[0][j] = 0.0f;
  for (int kg = 0; kg < K; kg += 8) {
    u32x4 v[8][1];
    const int slot_g = __shfl_down(myslot, kg);  // lane j now holds pair kg + j
    const float w_g = __shfl_down(myw, kg);
    combine_load8<64, 1>(v, eo, slot_g, K - kg, base, lane, H8);
    combine_accum8<1>(acc, v, slot_g, w_g, K - kg);
  }
  combine_store<64, 1>(acc, y + (int64_t)t * H8, base, lane, H8);
}

// Combine under a CU budget (see dispatch_persist_kernel): an item is one
// token's group of 64*NV 16-byte chunks (NV per lane); K rows of it are
// gathered and reduced in ascending k exactly as in combine_piece_kernel.
template <int NV>
__global__ __launch_bounds__(kPersistThreads) void combine_persist_kernel(
    const u32x4* __restrict__ eo, const int32_t* __restrict__ slot_of,
    const float* __restrict__ w, u32x4* __restrict__ y, int N, int K, int H8, int64_t cap) {
  extern __shared__ int lds[];  // only reserves the CU
  if (N < 0) lds[threadIdx.x] = 0;
  const int lane = threadIdx.x & 63;
  const int Q = (H8 + 64 * NV - 1) / (64 * NV);
  const int64_t n_items = (int64_t)N * Q;
  for (int64_t i = (int64_t)blockIdx.x * kPersistWaves + (threadIdx.x >> 6); i < n_items;
       i += (int64_t)gridDim.x * kPersistWaves) {
    const int t = uniform((int)(i / Q)), base = uniform((int)(i % Q)) * 64 * NV;
    const int myslot = load_slot(slot_of, t, K, lane, cap);
    const float myw = (lane < K) ? w[(int64_t)t * K + lane] : 0.0f;
    float acc[NV][8];
#pragma unroll
    for (int i2 = 0; i2 < NV; i2++)
#pragma unroll
      for (int j = 0; j < 8; j++) acc[i2][j] = 0.0f;
    for (int kg = 0; kg < K; kg += 8) {
      u32x4 v[8][NV];
      const int slot_g = __shfl_down(myslot, kg);
      const float w_g = __shfl_down(myw, kg);
      combine_load8<64, NV>(v, eo, slot_g, K - kg, base, lane, H8);
      combine_accum8<NV>(acc, v, slot_g, w_g, K - kg);
    }
    combine_store<64, NV>(acc, y + (int64_t)t * H8, base, lane, H8);
  }
}

// Combine under a CU budget for rows of at most 16 wavefronts (H8 <= 1024)
// and K <= 8: one workgroup of 64*Q threads per CU takes tokens
// t = blockIdx.x, t + gridDim.x, ...; each thread owns one 16-byte chunk
// column of the row, and gathers the next token's K
// rows while it reduces the current one, so two tokens' rows are in flight.
template <int Q>
__global__ __launch_bounds__(64 * Q) void combine_persist_tok_kernel(
    const u32x4* __restrict__ eo, const int32_t* __restrict__ slot_of,
    const float* __restrict__ w, u32x4* __restrict__ y, int N, int K, int H8, int64_t cap) {
  extern __shared__ int lds[];  // only reserves the CU
  if (N < 0) lds[threadIdx.x] = 0;
  constexpr int TPT = 64 * Q;
  const int vl = threadIdx.x, lane = vl & 63;
  const int G = gridDim.x;
  int t = blockIdx.x;
  if (t >= N) return;
  u32x4 va[8][1], vb[8][1];
  int sa = load_slot(slot_of, t, K, lane, cap);
  float wa = (lane < K) ? w[(int64_t)t * K + lane] : 0.0f;
  combine_load8<TPT, 1>(va, eo, sa, K, 0, vl, H8);
  while (true) {
    // token t is in va; fetch t + G into vb, reduce t
    const int tb = t + G;
    int sb = -1;
    float wb = 0.0f;
    if (tb < N) {
      sb = load_slot(slot_of, tb, K, lane, cap);
      wb = (lane < K) ? w[(int64_t)tb * K + lane] : 0.0f;
      combine_load8<TPT, 1>(vb, eo, sb, K, 0, vl, H8);
    }
    combine_pass8<TPT, 1>(va, sa, wa, K, y + (int64_t)t * H8, 0, vl, H8);
    if (tb >= N) break;
    // token tb is in vb; fetch tb + G into va, reduce tb
    const int ta = tb + G;
    if (ta < N) {
      sa = load_slot(slot_of, ta, K, lane, cap);
      wa = (lane < K) ? w[(int64_t)ta * K + lane] : 0.0f;
      combine_load8<TPT, 1>(va, eo, sa, K, 0, vl, H8);
    }
    combine_pass8<TPT, 1>(vb, sb, wb, K, y + (int64_t)tb * H8, 0, vl, H8);
    if (ta >= N) break;
    t = ta;
  }
}

template <int Q>
void launch_combine_persist_tok(int grid, size_t lds, hipStream_t st, const void* eo,
                                const int32_t* slot_of, const float* w, void* y, int N, int K,
                                int H8, int64_t cap) {
  combine_persist_tok_kernel<Q><<<grid, 64 * Q, lds, st>>>((const u32x4*)eo, slot_of, w,
                                                           (u32x4*)y, N, K, H8, cap);
}

// ---------------------------------------------------------------- host side
bool log_on() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("EP_GET_LOG");
    v = (e && *e && *e != '0') ? 1 : 0;
  }
  return v == 1;
}

#define EP_LOG(...)                          \
  do {                                       \
    if (log_on()) {                          \
      fprintf(stderr, "[ep_get] " __VA_ARGS__); \
      fputc('\n', stderr);                   \
    }                                        \
  } while (0)

int check_device() {
  static std::atomic<int> cache[64];  // 0 unknown, 1 gfx950, 2 other
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return EP_ERR_HIP;
  int c = (dev >= 0 && dev < 64) ? cache[dev].load() : 0;
  if (c == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return EP_ERR_HIP;
    c = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    if (dev >= 0 && dev < 64) cache[dev].store(c);
  }
  return c == 1 ? EP_OK : EP_ERR_UNSUPPORTED;
}

// LDS a persistent workgroup reserves: the whole per-workgroup maximum of
// the current device (cached per device; 0 if it cannot be read).
size_t persist_lds() {
  static std::atomic<long long> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  long long v = (dev >= 0 && dev < 64) ? cache[dev].load() : 0;
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
    v = (long long)prop.sharedMemPerBlock;
    if (dev >= 0 && dev < 64) cache[dev].store(v);
  }
  return (size_t)v;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    EP_LOG("%s: %s", what, hipGetErrorString(e));
    return EP_ERR_HIP;
  }
  return EP_OK;
}

int64_t bound_of(const ep_problem_t* p) {
  return (int64_t)p->num_tokens * p->num_topk + (int64_t)p->num_experts * (p->expert_alignment - 1);
}

int validate_layout(const ep_problem_t* p) {
  if (!p) return EP_ERR_INVALID_ARG;
  const int N = p->num_tokens, K = p->num_topk, E = p->num_experts, R = p->num_ranks,
            A = p->expert_alignment;
  if (N < 0 || K < 1 || K > EP_MAX_TOPK || E < 1 || E > EP_MAX_EXPERTS || R < 1 ||
      R > EP_MAX_RANKS || R > E || A < 1)
    return EP_ERR_INVALID_ARG;
  if (E % R != 0 || N % R != 0) return EP_ERR_INVALID_ARG;
  if (p->topk_idx_bytes != 0 && p->topk_idx_bytes != 4 && p->topk_idx_bytes != 8)
    return EP_ERR_INVALID_ARG;
  if (p->cu_budget < 0) return EP_ERR_INVALID_ARG;
  if (bound_of(p) > INT32_MAX) return EP_ERR_INVALID_ARG;
  return EP_OK;
}

int validate_payload(const ep_problem_t* p) {
  int rc = validate_layout(p);
  if (rc != EP_OK) return rc;
  const int H = p->hidden;
  if (H <= 0 || H > EP_MAX_HIDDEN || H % 8 != 0) return EP_ERR_INVALID_ARG;
  if (p->use_fp8 != 0 && p->use_fp8 != 1) return EP_ERR_INVALID_ARG;
  if (p->use_fp8 && H % 128 != 0) return EP_ERR_INVALID_ARG;
  return EP_OK;
}

Plan make_plan(const ep_problem_t* p) {
  Plan pl{};
  const int64_t N = p->num_tokens, K = p->num_topk, E = p->num_experts, R = p->num_ranks;
  const int64_t T = N / R;
  // at least ~512 pairs per block, and about 64 blocks when N*K is larger
  int64_t C = (512 + K - 1) / K;
  const int64_t C2 = (N * K / 64 + K - 1) / K;
  if (C2 > C) C = C2;
  const int64_t CB = T > 0 ? (T + C - 1) / C : 0;
  pl.C = (int32_t)C;
  pl.CB = (int32_t)CB;
  pl.B = (int32_t)(R * CB);
  int64_t o = 0;
  pl.o_err = o;
  o = align256(o + 4);
  pl.o_cnt = o;
  o = align256(o + 4 * (int64_t)pl.B * E);
  pl.o_rank = o;
  o = align256(o + 4 * (int64_t)pl.B * R);
  pl.o_berr = o;
  o = align256(o + 4 * (int64_t)pl.B);
  pl.bytes = o;
  return pl;
}

template <int NV>
void launch_dispatch_token(int grid, hipStream_t st, const ep_problem_t* p,
                           const ep_dispatch_args_t* a, const DispatchAux& aux) {
  dispatch_token_kernel<NV><<<grid, kThreads, 0, st>>>(
      (const u32x4*)a->x, a->x_scales, a->topk_weights, a->slot_of, (u32x4*)a->recv_x,
      a->recv_scales, a->recv_src_idx, a->recv_topk_weights, p->num_tokens, p->num_topk,
      p->hidden, a->recv_capacity, aux);
}

void launch_dispatch_piece(int grid, hipStream_t st, const ep_problem_t* p,
                           const ep_dispatch_args_t* a, const DispatchAux& aux, int P,
                           int64_t item0, int64_t items) {
  dispatch_piece_kernel<<<grid, kPieceThreads, 0, st>>>(
      (const u32x4*)a->x, a->topk_weights, a->slot_of, (u32x4*)a->recv_x, a->recv_src_idx,
      a->recv_topk_weights, p->num_tokens, p->num_topk, p->hidden / 8, P, item0, items,
      a->recv_capacity, aux);
}

void launch_dispatch_fp8_item(int grid, hipStream_t st, const ep_problem_t* p,
                              const ep_dispatch_args_t* a, const DispatchAux& aux, int P,
                              int64_t item0, int64_t items) {
  dispatch_fp8_item_kernel<<<grid, 64, 0, st>>>(
      (const u32x4*)a->x, a->topk_weights, a->slot_of, (u32x4*)a->recv_x, a->recv_scales,
      a->recv_src_idx, a->recv_topk_weights, p->num_tokens, p->num_topk, p->hidden, P, item0,
      items, a->recv_capacity, aux);
}

template <int MODE, int NV>
void launch_dispatch_persist(int grid, size_t lds, hipStream_t st, const ep_problem_t* p,
                             const ep_dispatch_args_t* a, const DispatchAux& aux) {
  dispatch_persist_kernel<MODE, NV><<<grid, kPersistThreads, lds, st>>>(
      (const u32x4*)a->x, a->x_scales, a->topk_weights, a->slot_of, (u32x4*)a->recv_x,
      a->recv_scales, a->recv_src_idx, a->recv_topk_weights, p->num_tokens, p->num_topk,
      p->hidden, a->recv_capacity, aux);
}

// Layout launches for one index type.
template <typename I>
int run_layout(const ep_problem_t* p, const I* topk_idx, int32_t* num_tokens_per_rank,
               int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank,
               int32_t* num_recv_per_expert, int32_t* expert_slot_offset, int32_t* slot_of,
               void* workspace, int32_t* err_word, hipStream_t st) {
  int rc;
  const int N = p->num_tokens;
  const Plan pl = make_plan(p);
  const int K = p->num_topk, E = p->num_experts, R = p->num_ranks;
  const int T = N / R, L = E / R;
  char* ws = (char*)workspace;
  // the error word: the workspace's own, unless the caller names another
  int32_t* err = err_word ? err_word : (int32_t*)(ws + pl.o_err);
  int32_t* blk_cnt = (int32_t*)(ws + pl.o_cnt);
  int32_t* blk_rank = (int32_t*)(ws + pl.o_rank);
  int32_t* blk_err = (int32_t*)(ws + pl.o_berr);
  EP_LOG("layout N=%d K=%d E=%d R=%d A=%d idx=int%d: blocks=%d chunk=%d tokens", N, K, E, R,
         p->expert_alignment, (int)(8 * sizeof(I)), pl.B, pl.C);
  if (pl.B == 0) {
    layout_empty_kernel<<<1, kThreads, 0, st>>>(err, num_tokens_per_rank, num_tokens_per_expert,
                                                num_recv_per_expert, expert_slot_offset, E, R);
    return check_launch("layout_empty");
  }
  if ((int64_t)N * K <= kFusedMaxPairs && N <= kFlagBytes && E <= kFusedMaxExperts &&
      (int64_t)pl.C * K <= kAssignTile) {
    const size_t mbytes = sizeof(unsigned long long) * (kFusedThreads / 64) * (size_t)E;
    layout_fused_kernel<I><<<pl.B, kFusedThreads, mbytes, st>>>(
        topk_idx, is_token_in_rank, err, num_tokens_per_rank, num_tokens_per_expert,
        num_recv_per_expert, expert_slot_offset, slot_of, N, K, E, R, T, pl.CB, pl.C,
        p->expert_alignment, magic_of((uint32_t)K), magic_of((uint32_t)L));
    return check_launch("layout_fused");
  }
  layout_count_kernel<I><<<pl.B, kCountThreads, 0, st>>>(
      topk_idx, is_token_in_rank, blk_cnt, blk_rank, blk_err, K, E, R, L, T, pl.CB, pl.C);
  if ((rc = check_launch("layout_count")) != EP_OK) return rc;
  size_t mask_bytes = sizeof(unsigned long long) * kAssignWaves * (size_t)E;
  if (mask_bytes < 3 * sizeof(int) * kAssignThreads) mask_bytes = 3 * sizeof(int) * kAssignThreads;
  layout_assign_kernel<I><<<pl.B, kAssignThreads, mask_bytes, st>>>(
      topk_idx, blk_cnt, blk_rank, blk_err, err, num_tokens_per_rank, num_tokens_per_expert,
      num_recv_per_expert, expert_slot_offset, slot_of, K, E, R, T, pl.CB, pl.C, pl.B,
      p->expert_alignment);
  return check_launch("layout_assign");
}

template <int MODE, int NV>
void launch_ll(int grid, size_t lds, hipStream_t st, const ep_problem_t* p,
               const ep_ll_args_t* a, int T, int M, int Q) {
  const int K = p->num_topk, E = p->num_experts, R = p->num_ranks, H = p->hidden;
  if (p->topk_idx_bytes == 8)
    ll_dispatch_kernel<MODE, NV, int64_t><<<grid, kLLThreads, lds, st>>>(
        (const int64_t*)a->topk_idx, (const u32x4*)a->x, a->x_scales, a->topk_weights,
        a->recv_count, a->slot_of, a->flags, (u32x4*)a->recv_x, a->recv_scales, a->recv_src_idx,
        a->recv_topk_weights, a->cumulative_recv_stats, K, E, R, T, M, H, Q);
  else
    ll_dispatch_kernel<MODE, NV, int32_t><<<grid, kLLThreads, lds, st>>>(
        (const int32_t*)a->topk_idx, (const u32x4*)a->x, a->x_scales, a->topk_weights,
        a->recv_count, a->slot_of, a->flags, (u32x4*)a->recv_x, a->recv_scales, a->recv_src_idx,
        a->recv_topk_weights, a->cumulative_recv_stats, K, E, R, T, M, H, Q);
}

}  // namespace

// ------------------------------------------------------------ static scratch
// The layout workspace of ep_get_layout_noalloc, for callers that cannot
// allocate: a file-scope device array, one copy per GPU, held until the
// process ends.  Host code never uses its name as an address (on the host it
// is only a stand-in symbol): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address reaches the kernels.  Every call on one GPU shares the
// array; the layout kernels write every word they later read, so it needs no
// clearing, and calls that overlap on one GPU race.
constexpr int64_t kScratchBytes = EP_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
int scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return EP_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return EP_ERR_UNSUPPORTED;
  void* ptr = cache[dev].load();
  if (!ptr) {
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      EP_LOG("hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      return EP_ERR_HIP;
    }
    cache[dev].store(ptr);
  }
  *out = ptr;
  return EP_OK;
}
}  // namespace

// ===================================================================== C ABI
extern "C" {

int64_t ep_recv_capacity(const ep_problem_t* p) {
  if (validate_layout(p) != EP_OK) return -1;
  return bound_of(p);
}

int64_t ep_workspace_bytes(const ep_problem_t* p) {
  if (validate_layout(p) != EP_OK) return -1;
  return make_plan(p).bytes;
}

int ep_get_layout(const ep_problem_t* p, const void* topk_idx, int32_t* num_tokens_per_rank,
                  int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank,
                  int32_t* num_recv_per_expert, int32_t* expert_slot_offset, int32_t* slot_of,
                  void* workspace, void* stream) {
  int rc = validate_layout(p);
  if (rc != EP_OK) return rc;
  const int N = p->num_tokens;
  if (!num_tokens_per_rank || !num_tokens_per_expert || !num_recv_per_expert ||
      !expert_slot_offset || !workspace)
    return EP_ERR_INVALID_ARG;
  if (N > 0 && (!topk_idx || !is_token_in_rank || !slot_of)) return EP_ERR_INVALID_ARG;
  if (((uintptr_t)workspace & 255) != 0) return EP_ERR_INVALID_ARG;
  rc = check_device();
  if (rc != EP_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  if (p->topk_idx_bytes == 8)
    return run_layout(p, (const int64_t*)topk_idx, num_tokens_per_rank, num_tokens_per_expert,
                      is_token_in_rank, num_recv_per_expert, expert_slot_offset, slot_of,
                      workspace, nullptr, st);
  return run_layout(p, (const int32_t*)topk_idx, num_tokens_per_rank, num_tokens_per_expert,
                    is_token_in_rank, num_recv_per_expert, expert_slot_offset, slot_of,
                    workspace, nullptr, st);
}

int ep_get_layout_noalloc(const ep_problem_t* p, const void* topk_idx,
                          int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                          uint8_t* is_token_in_rank, int32_t* num_recv_per_expert,
                          int32_t* expert_slot_offset, int32_t* slot_of, int32_t* error_word,
                          void* stream) {
  int rc = validate_layout(p);
  if (rc != EP_OK) return rc;
  const int N = p->num_tokens;
  if (!num_tokens_per_rank || !num_tokens_per_expert || !num_recv_per_expert ||
      !expert_slot_offset)
    return EP_ERR_INVALID_ARG;
  if (N > 0 && (!topk_idx || !is_token_in_rank || !slot_of)) return EP_ERR_INVALID_ARG;
  if (make_plan(p).bytes > kScratchBytes) return EP_ERR_SCRATCH;
  rc = check_device();
  if (rc != EP_OK) return rc;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != EP_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  if (p->topk_idx_bytes == 8)
    return run_layout(p, (const int64_t*)topk_idx, num_tokens_per_rank, num_tokens_per_expert,
                      is_token_in_rank, num_recv_per_expert, expert_slot_offset, slot_of, ws,
                      error_word, st);
  return run_layout(p, (const int32_t*)topk_idx, num_tokens_per_rank, num_tokens_per_expert,
                    is_token_in_rank, num_recv_per_expert, expert_slot_offset, slot_of, ws,
                    error_word, st);
}

int ep_dispatch_ex(const ep_problem_t* p, const ep_dispatch_args_t* a, void* stream) {
  int rc = validate_payload(p);
  if (rc != EP_OK) return rc;
  if (!a || (a->flags & ~(uint32_t)EP_DISPATCH_ZERO_PADDING) != 0) return EP_ERR_INVALID_ARG;
  const int64_t cap = a->recv_capacity;
  if (cap < bound_of(p)) return EP_ERR_CAPACITY;
  const int N = p->num_tokens, E = p->num_experts, A = p->expert_alignment, H = p->hidden;
  const bool meta = a->recv_src_idx || a->recv_topk_weights;
  const bool prequant = a->x_scales != nullptr;
  const bool zero = (a->flags & EP_DISPATCH_ZERO_PADDING) && A > 1;
  const bool stats = a->cumulative_recv_stats != nullptr;
  if (prequant && !p->use_fp8) return EP_ERR_INVALID_ARG;
  if (a->recv_topk_weights && N > 0 && !a->topk_weights) return EP_ERR_INVALID_ARG;
  if (N > 0 && (!a->x || !a->slot_of || !a->recv_x)) return EP_ERR_INVALID_ARG;
  if (p->use_fp8 && N > 0 && !a->recv_scales) return EP_ERR_INVALID_ARG;
  if ((meta || zero || stats) && (!a->expert_slot_offset || !a->num_recv_per_expert))
    return EP_ERR_INVALID_ARG;
  if (zero && (!a->recv_x || (p->use_fp8 && !a->recv_scales))) return EP_ERR_INVALID_ARG;
  rc = check_device();
  if (rc != EP_OK) return rc;
  const int K = p->num_topk;
  const int mode = prequant ? 2 : (p->use_fp8 ? 1 : 0);  // 0 bf16, 1 fused e4m3, 2 pre-quantised
  // the work besides the token rows, as wavefront items (aux_item)
  DispatchAux aux{};
  aux.off = a->expert_slot_offset;
  aux.cnt = a->num_recv_per_expert;
  aux.recv_src = a->recv_src_idx;
  aux.recv_w = a->recv_topk_weights;
  aux.recv_x = (u32x4*)a->recv_x;
  aux.recv_scales = p->use_fp8 ? a->recv_scales : nullptr;
  aux.stats = a->cumulative_recv_stats;
  aux.cap = cap;
  aux.E = E;
  aux.A = A;
  aux.row16 = p->use_fp8 ? H / 16 : H / 8;
  aux.G = p->use_fp8 ? H / 128 : 0;
  aux.tag_items = meta ? E + (cap + kTailSlots - 1) / kTailSlots : 0;
  aux.zero_items = zero ? (int64_t)E * (A - 1) : 0;
  aux.stat_items = stats ? 1 : 0;
  const int64_t n_aux = aux.items();
  // 16-byte chunks per lane of one wavefront-per-row pass (1024 channels for e4m3)
  const int q = mode == 0 ? (H / 8 + 63) / 64 : (mode == 2 ? (H / 16 + 63) / 64 : (H + 1023) / 1024);
  hipStream_t st = (hipStream_t)stream;
  if (p->cu_budget > 0) {
    // persistent grid: one 1024-thread workgroup per CU, wavefront work items
    const int64_t n_items = N + n_aux;
    const int64_t want = (n_items + kPersistWaves - 1) / kPersistWaves;
    const int pg = (int)(want < p->cu_budget ? want : p->cu_budget);
    if (pg == 0) return EP_OK;
    const size_t lds = persist_lds();
    EP_LOG("dispatch (CU budget %d) N=%d H=%d K=%d cap=%lld: workgroups=%d items=%lld lds=%zu",
           p->cu_budget, N, H, K, (long long)cap, pg, (long long)n_items, lds);
    if (lds == 0) return EP_ERR_HIP;
#define EP_DP(M, NV) launch_dispatch_persist<M, NV>(pg, lds, st, p, a, aux)
    if (mode == 0) {
      if (q <= 1) EP_DP(0, 1);
      else if (q <= 2) EP_DP(0, 2);
      else if (q <= 4) EP_DP(0, 4);
      else if (q <= 7) EP_DP(0, 7);
      else if (q <= 8) EP_DP(0, 8);
      else if (q <= 14) EP_DP(0, 14);
      else EP_DP(0, 16);
    } else if (mode == 1) {
      if (q <= 1) EP_DP(1, 1);
      else if (q <= 2) EP_DP(1, 2);
      else if (q <= 4) EP_DP(1, 4);
      else if (q <= 7) EP_DP(1, 7);
      else EP_DP(1, 8);
    } else {
      if (q <= 1) EP_DP(2, 1);
      else if (q <= 2) EP_DP(2, 2);
      else if (q <= 4) EP_DP(2, 4);
      else if (q <= 7) EP_DP(2, 7);
      else if (q <= 8) EP_DP(2, 8);
      else EP_DP(2, 16);
    }
#undef EP_DP
    return check_launch("dispatch_persist");
  }
  if (mode == 1) {
    // fused e4m3: (token, 1024-channel piece) items of one wavefront, then
    // the auxiliary blocks
    const int P = (H + 1023) / 1024;
    const int64_t items = (int64_t)N * P;
    if (items + n_aux == 0) return EP_OK;
    EP_LOG("dispatch e4m3 N=%d H=%d K=%d cap=%lld: items=%lld (pieces %d) aux items=%lld", N, H,
           K, (long long)cap, (long long)items, P, (long long)n_aux);
    for (int64_t item0 = 0;; item0 += kItemLaunch) {
      const int64_t left = items - item0;
      const bool last = left <= kItemLaunch;
      const int64_t grid = last ? left + n_aux : kItemLaunch;
      if (grid > INT32_MAX) return EP_ERR_INVALID_ARG;
      launch_dispatch_fp8_item((int)grid, st, p, a, aux, P, item0, items);
      if ((rc = check_launch("dispatch")) != EP_OK || last) return rc;
    }
  }
  if (mode == 0) {
    // bf16: (token, 2 KiB piece) workgroups, then the auxiliary blocks
    const int P = (H / 8 + kPieceChunks - 1) / kPieceChunks;
    const int64_t items = (int64_t)N * P;
    const int64_t aux_blocks = (n_aux + kPieceWaves - 1) / kPieceWaves;
    if (items + aux_blocks == 0) return EP_OK;
    EP_LOG("dispatch bf16 N=%d H=%d K=%d cap=%lld: piece workgroups=%lld (pieces %d) aux items=%lld "
           "(tags %lld, zero rows %lld, stats %lld)", N, H, K, (long long)cap, (long long)items, P,
           (long long)n_aux, (long long)aux.tag_items, (long long)aux.zero_items,
           (long long)aux.stat_items);
    for (int64_t item0 = 0;; item0 += kItemLaunch) {
      const int64_t left = items - item0;
      const bool last = left <= kItemLaunch;
      const int64_t grid = last ? left + aux_blocks : kItemLaunch;
      if (grid > INT32_MAX) return EP_ERR_INVALID_ARG;
      launch_dispatch_piece((int)grid, st, p, a, aux, P, item0, items);
      if ((rc = check_launch("dispatch")) != EP_OK || last) return rc;
    }
  }
  // pre-quantised e4m3: one wavefront per token, then the auxiliary blocks
  const int64_t grid = ((int64_t)N + kTokPerBlock - 1) / kTokPerBlock +
                       (n_aux + kTokPerBlock - 1) / kTokPerBlock;
  if (grid > INT32_MAX) return EP_ERR_INVALID_ARG;
  if (grid == 0) return EP_OK;
  EP_LOG("dispatch pre-quantised e4m3 N=%d H=%d K=%d cap=%lld: token blocks=%d aux items=%lld "
         "(tags %lld, zero rows %lld, stats %lld)", N, H, K, (long long)cap,
         (N + kTokPerBlock - 1) / kTokPerBlock, (long long)n_aux, (long long)aux.tag_items,
         (long long)aux.zero_items, (long long)aux.stat_items);
  const int g = (int)grid;
#define EP_DT(NV) launch_dispatch_token<NV>(g, st, p, a, aux)
  if (q <= 1) EP_DT(1);
  else if (q <= 2) EP_DT(2);
  else if (q <= 4) EP_DT(4);
  else if (q <= 7) EP_DT(7);
  else if (q <= 8) EP_DT(8);
  else EP_DT(16);
#undef EP_DT
  return check_launch("dispatch");
}

int ep_dispatch(const ep_problem_t* p, const void* x, const float* topk_weights,
                const int32_t* slot_of, const int32_t* expert_slot_offset,
                const int32_t* num_recv_per_expert, void* recv_x, float* recv_scales,
                int32_t* recv_src_idx, float* recv_topk_weights, int64_t recv_capacity,
                void* stream) {
  ep_dispatch_args_t a{};
  a.x = x;
  a.topk_weights = topk_weights;
  a.slot_of = slot_of;
  a.expert_slot_offset = expert_slot_offset;
  a.num_recv_per_expert = num_recv_per_expert;
  a.recv_x = recv_x;
  a.recv_scales = recv_scales;
  a.recv_src_idx = recv_src_idx;
  a.recv_topk_weights = recv_topk_weights;
  a.recv_capacity = recv_capacity;
  return ep_dispatch_ex(p, &a, stream);
}

int ep_combine(const ep_problem_t* p, const void* expert_out, const int32_t* slot_of,
               const float* topk_weights, void* y, int64_t recv_capacity, void* stream) {
  int rc = validate_payload(p);
  if (rc != EP_OK) return rc;
  const int N = p->num_tokens;
  if (recv_capacity < 0) return EP_ERR_INVALID_ARG;
  if (N == 0) return EP_OK;
  // the loads are branch-free: a pair without a slot reads row 0, which must exist
  if (recv_capacity < 1 || !slot_of || !topk_weights || !y || !expert_out)
    return EP_ERR_INVALID_ARG;
  rc = check_device();
  if (rc != EP_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  const int H8 = p->hidden / 8;
  const int q = (H8 + 63) / 64;  // wavefronts for one chunk per thread
  if (p->cu_budget > 0 && p->num_topk <= 8 && q <= 16) {
    const int pg = N < p->cu_budget ? N : p->cu_budget;
    const size_t lds = persist_lds();
    EP_LOG("combine (CU budget %d, token pipeline) N=%d H=%d K=%d: workgroups=%d lds=%zu",
           p->cu_budget, N, p->hidden, p->num_topk, pg, lds);
    if (lds < 4 * (2 * (size_t)EP_MAX_EXPERTS + 1)) return EP_ERR_HIP;
#define EP_CPT(QQ) launch_combine_persist_tok<QQ>(pg, lds, st, expert_out, slot_of, topk_weights, \
                                                  y, N, p->num_topk, H8, recv_capacity)
    switch (q) {
      case 1: EP_CPT(1); break;
      case 2: EP_CPT(2); break;
      case 3:
      case 4: EP_CPT(4); break;
      case 5:
      case 6:
      case 7: EP_CPT(7); break;
      case 8: EP_CPT(8); break;
      case 9:
      case 10:
      case 11:
      case 12:
      case 13:
      case 14: EP_CPT(14); break;
      default: EP_CPT(16); break;
    }
#undef EP_CPT
    return check_launch("combine_persist_tok");
  }
  if (p->cu_budget > 0) {
    constexpr int nv = kCombinePersistNV;
    const int64_t items = (int64_t)N * ((H8 + 64 * nv - 1) / (64 * nv));
    const int64_t want = (items + kPersistWaves - 1) / kPersistWaves;
    const int pg = (int)(want < p->cu_budget ? want : p->cu_budget);
    const size_t lds = persist_lds();
    EP_LOG("combine (CU budget %d) N=%d H=%d K=%d: workgroups=%d lds=%zu", p->cu_budget, N,
           p->hidden, p->num_topk, pg, lds);
    if (lds < 4 * (2 * (size_t)EP_MAX_EXPERTS + 1)) return EP_ERR_HIP;
    combine_persist_kernel<nv><<<pg, kPersistThreads, lds, st>>>(
        (const u32x4*)expert_out, slot_of, topk_weights, (u32x4*)y, N, p->num_topk, H8,
        recv_capacity);
    return check_launch("combine_persist");
  }
  // (token, piece) items; a launch holds at most kItemLaunch of them
  const int64_t items = (int64_t)N * q;
  EP_LOG("combine N=%d H=%d K=%d cap=%lld: items=%lld (pieces %d)", N, p->hidden, p->num_topk,
         (long long)recv_capacity, (long long)items, q);
  for (int64_t item0 = 0; item0 < items; item0 += kItemLaunch) {
    const int64_t left = items - item0;
    const int grid = (int)(left < kItemLaunch ? left : kItemLaunch);
    const u32x4* eo = (const u32x4*)expert_out;
    u32x4* yy = (u32x4*)y;
#define EP_CK(KK) combine_piece_k_kernel<KK><<<grid, 64, 0, st>>>(eo, slot_of, topk_weights, yy, N, \
                                                                  H8, q, item0, recv_capacity)
    switch (p->num_topk) {
      case 1: EP_CK(1); break;
      case 2: EP_CK(2); break;
      case 3: EP_CK(3); break;
      case 4: EP_CK(4); break;
      case 5: EP_CK(5); break;
      case 6: EP_CK(6); break;
      case 7: EP_CK(7); break;
      case 8: EP_CK(8); break;
      default:
        combine_piece_kernel<<<grid, 64, 0, st>>>(eo, slot_of, topk_weights, yy, N, p->num_topk,
                                                  H8, q, item0, recv_capacity);
        break;
    }
#undef EP_CK
    if ((rc = check_launch("combine")) != EP_OK) return rc;
  }
  return EP_OK;
}

int64_t ep_ll_capacity(const ep_problem_t* p, int32_t max_tokens_per_rank) {
  if (validate_layout(p) != EP_OK || max_tokens_per_rank < 1) return -1;
  const int64_t cap = (int64_t)p->num_experts * p->num_ranks * max_tokens_per_rank;
  return cap > INT32_MAX ? -1 : cap;
}

int ep_ll_dispatch_ex(const ep_problem_t* p, int32_t max_tokens_per_rank, const ep_ll_args_t* a,
                      void* stream) {
  int rc = validate_payload(p);
  if (rc != EP_OK) return rc;
  if (!a) return EP_ERR_INVALID_ARG;
  const int N = p->num_tokens, K = p->num_topk, E = p->num_experts, R = p->num_ranks;
  const int M = max_tokens_per_rank, H = p->hidden;
  if (ep_ll_capacity(p, M) < 0) return EP_ERR_INVALID_ARG;
  const int T = N / R;
  const bool prequant = a->x_scales != nullptr;
  if ((int64_t)T * K > kAssignTile) return EP_ERR_INVALID_ARG;
  if (!a->recv_count || !a->flags) return EP_ERR_INVALID_ARG;
  if (prequant && !p->use_fp8) return EP_ERR_INVALID_ARG;
  if (N > 0 && (!a->topk_idx || !a->x || !a->slot_of || !a->recv_x)) return EP_ERR_INVALID_ARG;
  if (p->use_fp8 && N > 0 && !a->recv_scales) return EP_ERR_INVALID_ARG;
  if (a->recv_topk_weights && N > 0 && !a->topk_weights) return EP_ERR_INVALID_ARG;
  rc = check_device();
  if (rc != EP_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  if (N == 0) {
    ll_empty_kernel<<<1, kThreads, 0, st>>>(a->recv_count, a->flags, E, R);
    return check_launch("ll_empty");
  }
  const int Q = (T + kLLWaves - 1) / kLLWaves;
  const int grid = R * Q;
  const size_t lds = sizeof(unsigned long long) * kLLWaves * (size_t)E;
  const int mode = prequant ? 2 : (p->use_fp8 ? 1 : 0);
  EP_LOG("ll dispatch N=%d H=%d K=%d E=%d R=%d M=%d mode=%d stats=%d: blocks=%d", N, H, K, E, R,
         M, mode, a->cumulative_recv_stats != nullptr, grid);
#define EP_LL(MD, NV) launch_ll<MD, NV>(grid, lds, st, p, a, T, M, Q)
  if (mode == 0) {
    const int q = (H / 8 + 63) / 64;
    if (q <= 1) EP_LL(0, 1);
    else if (q <= 2) EP_LL(0, 2);
    else if (q <= 4) EP_LL(0, 4);
    else if (q <= 7) EP_LL(0, 7);
    else if (q <= 8) EP_LL(0, 8);
    else if (q <= 14) EP_LL(0, 14);
    else EP_LL(0, 16);
  } else if (mode == 1) {
    const int q = (H + 1023) / 1024;
    if (q <= 1) EP_LL(1, 1);
    else if (q <= 2) EP_LL(1, 2);
    else if (q <= 4) EP_LL(1, 4);
    else if (q <= 7) EP_LL(1, 7);
    else EP_LL(1, 8);
  } else {
    const int q = (H / 16 + 63) / 64;
    if (q <= 1) EP_LL(2, 1);
    else if (q <= 2) EP_LL(2, 2);
    else if (q <= 4) EP_LL(2, 4);
    else if (q <= 7) EP_LL(2, 7);
    else if (q <= 8) EP_LL(2, 8);
    else EP_LL(2, 16);
  }
#undef EP_LL
  return check_launch("ll_dispatch");
}

int ep_ll_dispatch(const ep_problem_t* p, int32_t max_tokens_per_rank, const void* topk_idx,
                   const void* x, const float* topk_weights, int32_t* recv_count,
                   int32_t* slot_of, int32_t* flags, void* recv_x, float* recv_scales,
                   int32_t* recv_src_idx, float* recv_topk_weights, void* stream) {
  ep_ll_args_t a{};
  a.topk_idx = topk_idx;
  a.x = x;
  a.topk_weights = topk_weights;
  a.recv_count = recv_count;
  a.slot_of = slot_of;
  a.flags = flags;
  a.recv_x = recv_x;
  a.recv_scales = recv_scales;
  a.recv_src_idx = recv_src_idx;
  a.recv_topk_weights = recv_topk_weights;
  return ep_ll_dispatch_ex(p, max_tokens_per_rank, &a, stream);
}

int ep_layout_error(const void* workspace, int32_t* flags, void* stream) {
  if (!workspace || !flags) return EP_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  int32_t v = 0;
  if (hipMemcpyAsync(&v, workspace, sizeof v, hipMemcpyDeviceToHost, st) != hipSuccess)
    return EP_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return EP_ERR_HIP;
  *flags = v;
  return EP_OK;
}

const char* ep_status_str(int status) {
  switch (status) {
    case EP_OK: return "ok";
    case EP_ERR_INVALID_ARG: return "invalid argument";
    case EP_ERR_CAPACITY: return "receive capacity below N*K + E*(A-1)";
    case EP_ERR_HIP: return "HIP error";
    case EP_ERR_UNSUPPORTED: return "device is not gfx950";
    case EP_ERR_SCRATCH:
      return "layout workspace larger than the static scratch of ep_get_layout_noalloc";
    default: return "unknown status";
  }
}

}  // extern "C"
