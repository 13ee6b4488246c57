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

constexpr int kSchedThreads = 256;
constexpr int kMaxTilesSched = 1024;
constexpr int kSchedUsersLds = 4096;  // offsets held in LDS up to this many users; users are
                                      // ranked in chunks of this many
constexpr int kSchedMaxBlocks = 64;

// Workgroups take the cost classes c = max_tiles - blockIdx.x, stepping by the grid size.  Each
// first builds the whole class table itself (cheap: one pass over the users): the offsets go to
// LDS once (batches of up to kSchedUsersLds users; larger ones are read from global memory),
// each user's tile count is histogrammed with LDS atomics, and one wave turns the histogram into
// the first list index of every class (two suffix sums over the classes, 64 classes per step).
// Per class, ballots over the users in index order list those with at least c tiles (their rank
// is their position in the list), and then consecutive threads write consecutive 32-byte
// entries of the class's contiguous range of the work list, so the stores coalesce.
__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(const int32_t* __restrict__ offsets,
                                                               int B, int H, int block_rows,
                                                               int max_tiles, int32_t* count_out,
                                                               WorkItem* __restrict__ work) {
  __shared__ int hist[kMaxTilesSched + 2];   // users with exactly c tiles
  __shared__ int start[kMaxTilesSched + 2];  // first list index of the cost-c class
  __shared__ int32_t offs[kSchedUsersLds + 1];
  __shared__ int32_t users[kSchedUsersLds];  // this class's users of the current chunk, by rank
  __shared__ int wcount[kSchedThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int kW = kSchedThreads / 64;
  const bool in_lds = B <= kSchedUsersLds;
  for (int i = tid; i <= max_tiles + 1; i += kSchedThreads) hist[i] = 0;
  if (in_lds)
    for (int i = tid; i <= B; i += kSchedThreads) offs[i] = offsets[i];
  __syncthreads();
  auto off = [&](int b) { return in_lds ? offs[b] : offsets[b]; };
  auto tiles = [&](int b) {
    const int n = off(b + 1) - off(b);
    const int t = n <= 0 ? 0 : (n + block_rows - 1) / block_rows;
    return t < max_tiles ? t : max_tiles;
  };
  for (int b = tid; b < B; b += kSchedThreads) atomicAdd(&hist[tiles(b)], 1);
  __syncthreads();
  if (wave == 0) {
    // classes from max_tiles down, lane l of a step taking class top - l
    int carry_ge = 0, carry_pos = 0;
    for (int top = max_tiles; top >= 1; top -= 64) {
      const int c = top - lane;
      const int x = c >= 1 ? hist[c] : 0;
      int inc = x;  // inclusive prefix over the lanes: users with tiles in [c, top]
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(inc, o, 64);
        if (lane >= o) inc += y;
      }
      const int g = c >= 1 ? carry_ge + inc : 0;  // users with at least c tiles
      int inc2 = g;                                 // then the sum over classes c .. top
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(inc2, o, 64);
        if (lane >= o) inc2 += y;
      }
      if (c >= 1) start[c] = carry_pos + (inc2 - g) * H;  // items of the classes above c
      carry_ge += __shfl(inc, 63, 64);
      carry_pos += __shfl(inc2, 63, 64) * H;
    }
    if (lane == 0 && blockIdx.x == 0) *count_out = carry_pos;
  }
  __syncthreads();
  for (int c = max_tiles - (int)blockIdx.x; c >= 1; c -= (int)gridDim.x) {
    int run = 0;  // users of this class in the chunks before
    for (int u0 = 0; u0 < B; u0 += kSchedUsersLds) {
      const int u1 = min(B, u0 + kSchedUsersLds);
      int cnt = 0;
      for (int g0 = u0; g0 < u1; g0 += kSchedThreads) {
        const int b = g0 + tid;
        const bool pred = b < u1 && tiles(b) >= c;
        const uint64_t mask = __ballot(pred);
        if (lane == 0) wcount[wave] = __popcll(mask);
        __syncthreads();
        int before = cnt;
        for (int w = 0; w < wave; ++w) before += wcount[w];
        if (pred) {
          const int rank = before + (int)__builtin_amdgcn_mbcnt_hi(
                                        (uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
          users[rank] = b;
        }
        for (int w = 0; w < kW; ++w) cnt += wcount[w];
        __syncthreads();
      }
      WorkItem* dst = work + start[c] + (int64_t)run * H;
      for (int i = tid; i < cnt * H; i += kSchedThreads) {
        const int b = users[i / H];
        const int32_t t0 = off(b), nb = off(b + 1) - t0;
        dst[i] = WorkItem{b, i % H, c - 1, nb, (int64_t)t0, 0};
      }
      run += cnt;
      __syncthreads();
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
  const int blocks = max_tiles < 1 ? 1 : max_tiles < kSchedMaxBlocks ? max_tiles : kSchedMaxBlocks;
  hipLaunchKernelGGL(schedule_kernel, dim3(blocks), dim3(kSchedThreads), 0, stream, offsets, B, H,
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
