// Jagged-batch scheduler and host-checkable helpers.
//
// The attention's work is one item per (user b, head h, query tile qt); the
// causal cost of an item is qt + 1 key tiles.  Ragged batches skip all padding
// ("Actions Speak Louder than Words" §3.4: fully ragged attention), so the
// only imbalance left is the length spread; the scheduler lists the items in
// longest-processing-time order (cost descending, then b, then h ascending) so
// the hardware dispatcher, which hands out workgroups in index order, starts
// the expensive tiles first.
#include "hstu_internal.h"

namespace hstu {
namespace {

constexpr int kSchedThreads = 1024;
constexpr int kMaxTilesSched = 1024;

__device__ __forceinline__ int n_tiles_of(const int32_t* offsets, int b, int block_rows,
                                          int max_tiles) {
  const int n = offsets[b + 1] - offsets[b];
  const int t = n <= 0 ? 0 : (n + block_rows - 1) / block_rows;
  return t < max_tiles ? t : max_tiles;
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(const int32_t* __restrict__ offsets,
                                                               int B, int H, int block_rows,
                                                               int max_tiles, int32_t* count_out,
                                                               WorkItem* __restrict__ work) {
  __shared__ int hist[kMaxTilesSched + 2];
  __shared__ int start[kMaxTilesSched + 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i <= max_tiles + 1; i += kSchedThreads) hist[i] = 0;
  __syncthreads();
  for (int b = tid; b < B; b += kSchedThreads)
    atomicAdd(&hist[n_tiles_of(offsets, b, block_rows, max_tiles)], 1);
  __syncthreads();
  if (tid == 0) {
    // users with at least c tiles, accumulated from the longest class down;
    // start[c] = first list index of the cost-c class.
    int ge = 0, pos = 0;
    for (int c = max_tiles; c >= 1; --c) {
      ge += hist[c];
      start[c] = pos;
      pos += ge * H;
    }
    *count_out = pos;
  }
  __syncthreads();
  const int n_waves = kSchedThreads / 64;
  for (int c = max_tiles - wave; c >= 1; c -= n_waves) {
    int count = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
      const int b = b0 + lane;
      const bool pred = b < B && n_tiles_of(offsets, b, block_rows, max_tiles) >= c;
      const uint64_t mask = __ballot(pred);
      const int rank = count + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
      if (pred) {
        WorkItem* dst = work + start[c] + (int64_t)rank * H;
        const int32_t t0 = offsets[b], nb = offsets[b + 1] - t0;
        for (int h = 0; h < H; ++h) dst[h] = WorkItem{b, h, c - 1, nb, (int64_t)t0, 0};
      }
      count += __popcll(mask);
    }
  }
}

__global__ __launch_bounds__(1024) void validate_offsets_kernel(int B, const int32_t* __restrict__ offsets,
                                                                int64_t T, int max_seqlen,
                                                                int32_t* flags_out) {
  __shared__ int flags;
  if (threadIdx.x == 0) flags = 0;
  __syncthreads();
  int f = 0;
  if (threadIdx.x == 0) {
    if (offsets[0] != 0) f |= 1;
    if ((int64_t)offsets[B] != T) f |= 4;
  }
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const int n = offsets[b + 1] - offsets[b];
    if (n < 0) f |= 2;
    if (n > max_seqlen) f |= 8;
  }
  if (f) atomicOr(&flags, f);
  __syncthreads();
  if (threadIdx.x == 0) *flags_out = flags;
}

__global__ void debug_buckets_kernel(int B, const int32_t* __restrict__ offsets,
                                     const int64_t* __restrict__ ts, int P, int NT, int64_t R,
                                     const int64_t* __restrict__ ti, const int64_t* __restrict__ tj,
                                     int32_t* pb, int32_t* tb) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  const int64_t a = ti[r], c = tj[r];
  // user owning token a: last b with offsets[b] <= a
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)offsets[mid] <= a) lo = mid; else hi = mid - 1;
  }
  const int64_t base = offsets[lo];
  pb[r] = pos_bucket((int32_t)((a - base) - (c - base)), P - 1);
  tb[r] = time_bucket(ts[a] - ts[c], NT - 1);
}

}  // namespace

hipError_t launch_schedule(const int32_t* offsets, int32_t B, int32_t H, int32_t block_rows,
                           int32_t max_tiles, int32_t* work_count, WorkItem* work,
                           hipStream_t stream) {
  if (max_tiles > kMaxTilesSched) return hipErrorInvalidValue;
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, offsets, B, H,
                     block_rows, max_tiles, work_count, work);
  return hipGetLastError();
}

hipError_t launch_validate_offsets(int32_t B, const int32_t* offsets, int64_t T,
                                   int32_t max_seqlen, int32_t* flags, hipStream_t stream) {
  hipLaunchKernelGGL(validate_offsets_kernel, dim3(1), dim3(1024), 0, stream, B, offsets, T,
                     max_seqlen, flags);
  return hipGetLastError();
}

hipError_t launch_debug_buckets(int32_t B, const int32_t* offsets, const int64_t* ts, int32_t P,
                                int32_t NT, int64_t R, const int64_t* ti, const int64_t* tj,
                                int32_t* pb, int32_t* tb, hipStream_t stream) {
  if (R <= 0) return hipSuccess;
  const int64_t blocks = (R + 255) / 256;
  hipLaunchKernelGGL(debug_buckets_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, B,
                     offsets, ts, P, NT, R, ti, tj, pb, tb);
  return hipGetLastError();
}

}  // namespace hstu
