// Stochastic Length on the device ("Actions Speak Louder than Words" reading notes §3.3).
//
// For user b with n_b events and L = floor(N_c^(alpha/2)): n_b <= L keeps the sequence; n_b > L
// keeps L of its events with probability 1 - N_c^alpha / n_b^2, else the whole sequence.  The
// random draws are inputs: user b is subsampled iff u_user[b] < 1 - N_c^alpha / n_b^2 (float64),
// and the L events kept are those with the smallest key_tok (ties by lower index), in their
// original order.
//
// Three kernels: per user, a radix select of the L-th smallest key (four 8-bit passes over an
// order-preserving integer image of the float keys, histograms in LDS) and an in-order
// compaction of the kept local indices; one workgroup scanning the new lengths into offsets;
// a gather of the kept rows (any row size that is a multiple of 16 bytes), their timestamps
// and their source indices.
#include "hstu_internal.h"

namespace hstu {
namespace {

constexpr int kSThreads = 1024;

// order-preserving map of float bits to unsigned integers
__device__ __forceinline__ uint32_t key_bits(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// exclusive prefix sum over the 1024 threads of a workgroup; returns the total in *total
__device__ __forceinline__ int block_scan(int v, int* wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (tid < 16) {
    int w = wsum[tid];
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int y = __shfl_up(w, d, 64);
      if (tid >= d) w += y;
    }
    wsum[16 + tid] = w;  // inclusive over waves
  }
  __syncthreads();
  const int before = (wave ? wsum[16 + wave - 1] : 0) + x - v;
  *total = wsum[16 + 15];
  __syncthreads();
  return before;
}

struct SlArgs {
  int32_t B, L;
  double c;  // N_c^alpha
  const int32_t* offsets;
  int32_t max_seqlen;
  const float* u_user;
  const float* key_tok;
  int32_t* sel;      // [T] kept local indices of subsampled users, at the user's input offset
  int32_t* new_len;  // [B]
  int32_t* full;     // [B] 1 = kept whole
};

__global__ __launch_bounds__(kSThreads) void sl_select_kernel(SlArgs a) {
  __shared__ int hist[256];
  __shared__ int wsum[32];
  __shared__ int sh_digit, sh_k;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int64_t s = a.offsets[b];
  const int n = min(a.offsets[b + 1] - (int)s, a.max_seqlen);
  const bool sub = n > a.L && (double)a.u_user[b] < 1.0 - a.c / ((double)n * (double)n);
  if (!sub) {
    if (tid == 0) {
      a.new_len[b] = n;
      a.full[b] = 1;
    }
    return;
  }
  const float* keys = a.key_tok + s;
  // radix select of the L-th smallest key image
  uint32_t prefix = 0, mask = 0;
  int k = a.L;  // rank still to find within the current prefix, 1-based
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kSThreads) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kSThreads) {
      const uint32_t u = key_bits(keys[i]);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1);
    }
    __syncthreads();
    // the digit whose bucket holds rank k: inclusive prefix sums over the 256 buckets (four
    // waves of 64, then the waves' totals); exactly one bucket has cum_before < k <= cum
    if (tid < 256) {
      const int hv = hist[tid], lane = tid & 63;
      int x = hv;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
      }
      if (lane == 63) wsum[tid >> 6] = x;
    }
    __syncthreads();
    if (tid < 256) {
      int before_w = 0;
      for (int w = 0; w < (tid >> 6); ++w) before_w += wsum[w];
      const int hv = hist[tid];
      // recompute this lane's inclusive sum within its wave from the bucket values
      int x = hv;
      const int lane = tid & 63;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
      }
      const int cum = before_w + x;
      if (cum - hv < k && k <= cum) {
        sh_digit = tid;
        sh_k = k - (cum - hv);
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sh_digit << shift;
    mask |= 255u << shift;
    k = sh_k;
    __syncthreads();
  }
  // keep u < prefix, and the first k (in index order) of u == prefix
  const uint32_t thr = prefix;
  const int need_ties = k;
  int kept_before = 0, ties_before = 0;
  for (int i0 = 0; i0 < n; i0 += kSThreads) {
    const int i = i0 + tid;
    const uint32_t u = i < n ? key_bits(keys[i]) : 0xffffffffu;
    const int tie = i < n && u == thr;
    int tot;
    const int tie_rank = ties_before + block_scan(tie, wsum, &tot);
    ties_before += tot;
    const int keep = i < n && (u < thr || (tie && tie_rank < need_ties));
    const int rank = kept_before + block_scan(keep, wsum, &tot);
    kept_before += tot;
    if (keep) a.sel[s + rank] = i;
  }
  if (tid == 0) {
    a.new_len[b] = a.L;
    a.full[b] = 0;
  }
}

// out_offsets = exclusive prefix sums of the new lengths (one workgroup)
__global__ __launch_bounds__(kSThreads) void sl_offsets_kernel(int32_t B, const int32_t* new_len,
                                                              int32_t* out_offsets) {
  __shared__ int wsum[32];
  int carry = 0;
  for (int b0 = 0; b0 < B; b0 += kSThreads) {
    const int b = b0 + (int)threadIdx.x;
    const int v = b < B ? new_len[b] : 0;
    int tot;
    const int ex = block_scan(v, wsum, &tot);
    if (b < B) out_offsets[b] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) out_offsets[B] = carry;
}

// output rows 64 y .. 64 y + 63 of user b: source index, timestamp and row copy
__global__ __launch_bounds__(256) void sl_gather_kernel(SlArgs a, const int32_t* out_offsets,
                                                        const uint4* x, int32_t row_chunks,
                                                        const int64_t* ts, int32_t* src_index,
                                                        uint4* x_out, int64_t* ts_out) {
  const int b = blockIdx.x;
  const int r0 = 64 * blockIdx.y;
  const int len = a.new_len[b];
  if (r0 >= len) return;
  const int rows = min(64, len - r0);
  const int64_t s = a.offsets[b], o = out_offsets[b];
  const bool full = a.full[b] != 0;
  __shared__ int64_t src_s[64];
  if ((int)threadIdx.x < rows) {
    const int r = r0 + threadIdx.x;
    const int64_t src = s + (full ? r : a.sel[s + r]);
    src_s[threadIdx.x] = src;
    src_index[o + r] = (int32_t)src;
    if (ts) ts_out[o + r] = ts[src];
  }
  __syncthreads();
  if (!x) return;
  for (int e = threadIdx.x; e < rows * row_chunks; e += 256) {
    const int r = e / row_chunks, c = e - r * row_chunks;
    x_out[(o + r0 + r) * row_chunks + c] = x[src_s[r] * row_chunks + c];
  }
}

}  // namespace

size_t sl_workspace_bytes(int32_t B, int64_t total_tokens) {
  auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
  return al((size_t)total_tokens * 4) + 2 * al((size_t)B * 4);
}

hipError_t launch_stochastic_length(int32_t B, const int32_t* offsets, int32_t max_seqlen,
                                    int64_t total_tokens, int32_t L, double c, const float* u_user,
                                    const float* key_tok, const void* x, int64_t row_bytes,
                                    const int64_t* ts, int32_t* out_offsets, int32_t* src_index,
                                    void* x_out, int64_t* ts_out, void* workspace,
                                    hipStream_t stream) {
  if (B <= 0) return hipSuccess;
  auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
  SlArgs a{};
  a.B = B;
  a.L = L;
  a.c = c;
  a.offsets = offsets;
  a.max_seqlen = max_seqlen;
  a.u_user = u_user;
  a.key_tok = key_tok;
  char* ws = (char*)workspace;
  a.sel = (int32_t*)ws;
  a.new_len = (int32_t*)(ws + al((size_t)total_tokens * 4));
  a.full = (int32_t*)(ws + al((size_t)total_tokens * 4) + al((size_t)B * 4));
  hipLaunchKernelGGL(sl_select_kernel, dim3(B), dim3(kSThreads), 0, stream, a);
  hipLaunchKernelGGL(sl_offsets_kernel, dim3(1), dim3(kSThreads), 0, stream, B, a.new_len, out_offsets);
  if (max_seqlen > 0)
    hipLaunchKernelGGL(sl_gather_kernel, dim3(B, (max_seqlen + 63) / 64), dim3(256), 0, stream, a,
                       out_offsets, (const uint4*)x, (int32_t)(row_bytes / 16), ts, src_index,
                       (uint4*)x_out, ts_out);
  return hipGetLastError();
}

}  // namespace hstu
