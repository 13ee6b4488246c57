// Internal declarations shared by the HIP translation units of libhstu (not installed).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// s_waitcnt bounding only the vector-memory counter (loads and LDS transfers still in flight)
template <int C>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((C & 15) | (7 << 4) | (15 << 8) | ((C >> 4) << 14));
}

// workgroup barrier with no compiler reordering of memory operations across it (the LDS
// transfers it publishes were waited for explicitly)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// destination of a direct global -> LDS transfer (buffer load with the LDS bit)
typedef __attribute__((address_space(3))) void* lds_ptr;

// Lane moves within a row of 16 lanes (DPP): the value of another lane of the same row.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // lane i <- 7 - i within each 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <- 15 - i within each 16 lanes

// ---- wave-wide reductions and SiLU evaluation in base-2 units (attention kernels) ----

__device__ __forceinline__ int64_t shfl_xor_i64(int64_t v, int m) {
  int lo = __shfl_xor((int)(uint32_t)(uint64_t)v, m, 64);
  int hi = __shfl_xor((int)(uint32_t)((uint64_t)v >> 32), m, 64);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo);
}

// min / max over each 32-lane half of the wave.
__device__ __forceinline__ void half_minmax(int64_t& mn, int64_t& mx) {
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) {
    int64_t a = shfl_xor_i64(mn, m), b = shfl_xor_i64(mx, m);
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
}

// Values the whole wave holds in common, moved to scalar registers.
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int uniform_i32(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uniform_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(uint32_t, v)));
}

// w(y) = y - y^2 (P0 + P1 y^2 + P2 y^4) on |y| <= kPolyRange (near-minimax fit of the
// relative error of 1/(1+2^y); the fitting script sits beside the attention kernel).
constexpr float kPolyRange = 2.0f;
constexpr float kP0 = 0.3463683490f, kP1 = -0.0135027335f, kP2 = 0.0004785898f;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

constexpr int64_t kTMax = 0x7fffffffffffffffLL;
constexpr int64_t kTMin = -kTMax - 1;

// Largest half-width D of a 32x32 tile's y range (y = c + delta, |delta| <= D) for which the
// second-order Taylor expansion of w around the tile's constant bias c is used: its remainder
// is at most max|w'''| D^3 / 6 = 0.0521 D^3 <= 8.4e-5 D, below 2^-13 of the tile's largest
// |w| (which is at least 0.96 D for D this small).
constexpr float kTaylorD = 0.04f;

// ALiBi far cut: pairs whose base-2 SiLU argument is provably y >= kAlibiFarY are skipped.  w(y)
// decreases for y > 1 / ln 2, so each skipped weight is below w(64) = 128 / (1 + 2^64) < 7e-18
// (SiLU below 2.5e-18): a user of n keys loses at most 2.5e-18 n max|v| per output, far below
// the fp32 resolution of any output that a key within reach contributes to.
constexpr float kAlibiFarY = 64.0f;
// Below kFarExpY the exact w(y) = y / (0.5 + 0.5 2^y) is used; from it on (y >= 16) the form
// 2 y e, e = 2^-y: its ratio to w is 1 + e, a relative error of at most 2^-16.
constexpr float kFarExpY = 16.0f;

// w(y) = 2y/(1+2^y) and its first two derivatives at c, as the coefficients of the expansion
// in the raw score s (y = c + cq s): w ~ a0 + a1 s + a2 s^2.  No overflow for any finite c:
// s = 1/(1+2^c) and o = 1 - s come from 2^-|c|.
__device__ __forceinline__ void w_taylor_coeffs(float c, float cq, float& a0, float& a1, float& a2) {
  const float e = exp2f(-fabsf(c));
  const float inv = 1.0f / (1.0f + e);
  const float s = c >= 0.f ? e * inv : inv;
  const float o = c >= 0.f ? inv : e * inv;
  const float g = s * o;
  const float w0 = 2.0f * c * s;
  const float w1 = 2.0f * s - 2.0f * kLn2 * c * g;
  const float w2 = -4.0f * kLn2 * g + 2.0f * kLn2 * kLn2 * c * g * (o - s);
  a0 = w0;
  a1 = w1 * cq;
  a2 = 0.5f * w2 * cq * cq;
}

// One unit of attention work: query tile `qt` of user `b`, head `h`.
// The user's first token and length ride along, so that a workgroup's first dependent reads
// (its Q rows, K / V tiles, timestamps) need one round trip to memory, not two.
struct WorkItem {
  int32_t b, h, qt, n;  // n: the user's length
  int64_t tok0, pad;    // tok0: the user's first token
};

struct BiasArgs {
  int32_t kind;  // 0 none, 1 position + time tables, 2 ALiBi
  const int64_t* ts;
  const float* w_pos;
  const float* w_time;
  int32_t num_pos, num_time, pos_stride, time_stride;
  const float* slopes;  // may be null: 2^(-8 (h+1) / H)
};

// Min and max timestamp of a 32-token block.
struct TimeStat {
  int64_t mn, mx;
};

struct AttnArgs {
  const int32_t* offsets;
  const int32_t* work_count;
  const WorkItem* work;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t q_stride, k_stride, v_stride;  // elements between tokens
  int32_t H;
  int32_t o_f32;  // bf16 inputs only: write O as fp32 instead of bf16
  BiasArgs bias;
  const TimeStat* tstat;  // per token: stats of the 32-token block starting there (bf16 path)
  const int32_t* trel;    // per token: timestamp minus its block's minimum (bf16 path)
  const uint32_t* tclass; // per (query block, key block) pair: bias class (bf16 path)
  int32_t tclass_cols;    // entries per query-block row of tclass (= blocks of the longest user)
  int64_t tclass_bytes;
  float alpha, out_scale;
  f32x4* ostats;          // bf16 path, optional (layer mode): per (token, head) offset m,
                          // mean and M2 of the O row stored as m + bf16 deviations
  const float* knorm;     // bf16 path: per (32-key block, head) max squared key norm, rows as tclass
};

// Rows of the tile-class table: user b's query block i sits on row (offsets[b] + 31 b) / 32 + i,
// which never collides with another user's rows; fewer than (T + 31 B) / 32 + 1 rows in all.
__host__ __device__ inline int64_t tclass_row0(int64_t tok0, int64_t b) { return (tok0 + 31 * b) / 32; }

constexpr int kMaxPosBuckets = 1024;
constexpr int kMaxTimeBuckets = 64;

// Time bucket of the relative bias: floor(log2(1 + max(dt, 0))) clipped to nt - 1.
// Exact on integers: floor(log2(u)) of u >= 1 is the index of its highest set bit.
__device__ __forceinline__ int32_t time_bucket(int64_t dt, int32_t nt_minus_1) {
  uint64_t u = dt < 0 ? 1ull : (uint64_t)dt + 1ull;  // dt = INT64_MAX gives 2^63: still >= 1
  int32_t e = 63 - __builtin_clzll(u);
  return e < nt_minus_1 ? e : nt_minus_1;
}

// Position bucket: i - j clipped to [0, P - 1].
__device__ __forceinline__ int32_t pos_bucket(int32_t i_minus_j, int32_t p_minus_1) {
  int32_t d = i_minus_j < 0 ? 0 : i_minus_j;
  return d < p_minus_1 ? d : p_minus_1;
}

// ALiBi slope of head h when none is given: 2^(-8 (h + 1) / H).
__device__ __forceinline__ float default_alibi_slope(int h, int H) {
  return exp2f(-8.0f * (float)(h + 1) / (float)H);
}

// ---- launchers (host side, defined in the .hip files) ----
hipError_t launch_schedule(const int32_t* offsets, int32_t B, int32_t H, int32_t block_rows,
                           int32_t max_tiles, int32_t* work_count, WorkItem* work,
                           hipStream_t stream);
hipError_t launch_time_stats(int32_t B, const int32_t* offsets, const int64_t* ts,
                             int32_t max_seqlen, TimeStat* stats, int32_t* rel,
                             hipStream_t stream);
// dst[c][r] = src[r][c], bf16 [R][C]
hipError_t launch_transpose_bf16(const bf16* src, bf16* dst, int32_t R, int32_t C,
                                 hipStream_t stream);
// key norm bounds; with ts non-null also the timestamp statistics of launch_time_stats
hipError_t launch_key_norm(int32_t B, const int32_t* offsets, int64_t total_tokens,
                           const void* k, int64_t k_stride, int32_t H, int32_t d, float* knorm,
                           const int64_t* ts, TimeStat* stats, int32_t* rel, hipStream_t stream);
hipError_t launch_tile_class(int32_t B, const int32_t* offsets, const TimeStat* stats,
                             int32_t max_blocks, int32_t num_pos, int32_t num_time,
                             uint32_t* tclass, hipStream_t stream);
hipError_t launch_attn_bf16(int d, const AttnArgs& a, int grid, hipStream_t stream);
hipError_t launch_attn_f32(int d, const AttnArgs& a, int grid, hipStream_t stream);
int attn_block_rows_bf16(int d);
int attn_block_rows_f32(int d);

hipError_t launch_f1_gemm_silu(const bf16* x, const bf16* w1, const float* b1, bf16* z, int64_t M,
                               int32_t N, int32_t K, hipStream_t stream,
                               bool silu_bwd = false, const bf16* resid = nullptr,
                               bool plain = false);
hipError_t launch_ln_gate_f2(const bf16* o, const f32x4* ostats, const bf16* u,
                             int64_t u_stride, const float* gamma, const float* beta, float eps,
                             const bf16* w2, const float* b2, const bf16* x, bf16* y, int64_t M,
                             int32_t D, int32_t H, int32_t dv, hipStream_t stream);
// The same, fused with the next layer's f1: zn = SiLU(y w1n^T + b1n) [M, N1n] (D = 512,
// N1n % 512 == 0); zn may be the buffer u lies in (each workgroup reads only its own rows of u
// before it writes them).
hipError_t launch_ln_gate_f2_f1(const bf16* o, const f32x4* ostats, const bf16* u,
                                int64_t u_stride, const float* gamma, const float* beta, float eps,
                                const bf16* w2, const float* b2, const bf16* x, bf16* y,
                                const bf16* w1n, const float* b1n, bf16* zn, int32_t N1n,
                                int64_t M, int32_t D, int32_t H, int32_t dv, hipStream_t stream);
// Gradients of the bf16 d = 64 attention (attention_bwd.hip).
struct BwdArgs {
  const int32_t* offsets;
  const int32_t* work_count;
  const WorkItem* work;
  const bf16 *q, *k, *v, *dout;
  const bf16* dout_lo;  // optional: bf16 remainder of dO (rows as dout), added in the dO V^T product
  int64_t q_stride, k_stride, v_stride, do_stride;  // elements between tokens
  int32_t H;
  BiasArgs bias;
  float alpha, out_scale;
  bf16 *dq, *dk, *dv;         // [T, H, 64] rows with the strides below
  int64_t dq_stride, dk_stride, dv_stride;
  float *dw_pos, *dw_time;    // position + time bias: gradients shaped like the tables
  const TimeStat* tstat;      // position + time bias: per 32-token block min / max time
};
// query rows per work item of the backward kernels (their own work list)
int attn_bwd_block_rows();
hipError_t launch_attn_bwd_bf16(const BwdArgs& a, int grid, int64_t n_pos_grad,
                                int64_t n_time_grad, hipStream_t stream);

// Layer backward around the attention (layer_bwd.hip).
struct LayerBwdLaunch {
  int64_t T;
  int32_t D, HV, N1, residual;
  float eps;
  const bf16 *x, *w1, *w2, *dy, *o, *u;  // u: Z's U columns, row stride u_stride
  const f32x4* ostats;                    // the forward's per (token, head) O statistics
  int32_t dvh;                            // d_v (features per head of O)
  int64_t u_stride;
  const float *b1, *gamma, *beta;
  bf16 *dg, *g, *dO, *dO_lo, *dz, *dx;    // dz: [T][N1] rows with stride dz_stride
  int64_t dz_stride;
  float *dgamma, *dbeta, *dw1, *db1, *dw2, *db2;
};
hipError_t launch_layer_bwd_pre(const LayerBwdLaunch& L, hipStream_t stream);
hipError_t launch_layer_bwd_post(const LayerBwdLaunch& L, hipStream_t stream);
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t stream);

// Stochastic Length (stochastic_length.hip).
size_t sl_workspace_bytes(int32_t B, int64_t total_tokens);
hipError_t launch_stochastic_length(int32_t B, const int32_t* offsets, int32_t max_seqlen,
                                    int64_t total_tokens, int32_t L, double c, const float* u_user,
                                    const float* key_tok, const void* x, int64_t row_bytes,
                                    const int64_t* ts, int32_t* out_offsets, int32_t* src_index,
                                    void* x_out, int64_t* ts_out, void* workspace,
                                    hipStream_t stream);

// Candidate scoring over a cached history (candidates.hip).
struct CandLaunch {
  int32_t B, H, max_hist, max_cand;
  int64_t total_hist, total_cand;
  void* workspace;         // cand_workspace_bytes(B, max_hist, total_hist, total_cand, H) bytes
  const int32_t* hist_offsets;
  const int32_t* cand_offsets;
  const bf16 *q, *kc, *vc, *kh, *vh;
  int64_t q_stride, kc_stride, vc_stride, kh_stride, vh_stride;
  bf16* o;
  BiasArgs bias;           // bias.ts: history timestamps
  const int64_t* cand_ts;  // candidate timestamps
  float alpha, out_scale;
};
hipError_t launch_attn_candidates_bf16(const CandLaunch& c, hipStream_t stream);
size_t cand_workspace_bytes(int32_t B, int32_t max_hist, int64_t total_hist, int64_t total_cand,
                            int32_t H);

hipError_t launch_embed_sum(int64_t T, int32_t dim, const bf16* item, int64_t num_items,
                            const bf16* action, int32_t num_actions, const int32_t* ids,
                            const int32_t* aids, bf16* x, hipStream_t stream);
hipError_t launch_validate_offsets(int32_t B, const int32_t* offsets, int64_t T,
                                   int32_t max_seqlen, int32_t* flags, hipStream_t stream);
hipError_t launch_debug_buckets(int32_t B, const int32_t* offsets, const int64_t* ts, int32_t P,
                                int32_t NT, int64_t R, const int64_t* ti, const int64_t* tj,
                                int32_t* pb, int32_t* tb, hipStream_t stream);

}  // namespace hstu
