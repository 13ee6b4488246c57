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

// Lane moves within a row of 16 lanes (DPP): the value of another lane of the same row.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // lane i <- 7 - i within each 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <- 15 - i within each 16 lanes

// One unit of attention work: query tile `qt` of user `b`, head `h`.
struct WorkItem {
  int32_t b, h, qt, pad;
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
  f32x2* ostats;          // bf16 path, optional: per (token, head) mean and M2 of the O row
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
hipError_t launch_tile_class(int32_t B, const int32_t* offsets, const TimeStat* stats,
                             int32_t max_blocks, int32_t num_pos, int32_t num_time,
                             uint32_t* tclass, hipStream_t stream);
hipError_t launch_attn_bf16(int d, const AttnArgs& a, int grid, hipStream_t stream);
hipError_t launch_attn_f32(int d, const AttnArgs& a, int grid, hipStream_t stream);
int attn_block_rows_bf16(int d);
int attn_block_rows_f32(int d);

hipError_t launch_f1_gemm_silu(const bf16* x, const bf16* w1, const float* b1, bf16* z, int64_t M,
                               int32_t N, int32_t K, hipStream_t stream);
hipError_t launch_ln_gate_f2(const bf16* o, const f32x2* ostats, const bf16* u,
                             int64_t u_stride, const float* gamma, const float* beta, float eps,
                             const bf16* w2, const float* b2, const bf16* x, bf16* y, int64_t M,
                             int32_t D, int32_t H, int32_t dv, hipStream_t stream);
hipError_t launch_embed_sum(int64_t T, int32_t dim, const bf16* item, int64_t num_items,
                            const bf16* action, int32_t num_actions, const int32_t* ids,
                            const int32_t* aids, bf16* x, hipStream_t stream);
hipError_t launch_validate_offsets(int32_t B, const int32_t* offsets, int64_t T,
                                   int32_t max_seqlen, int32_t* flags, hipStream_t stream);
hipError_t launch_debug_buckets(int32_t B, const int32_t* offsets, const int64_t* ts, int32_t P,
                                int32_t NT, int64_t R, const int64_t* ti, const int64_t* tj,
                                int32_t* pb, int32_t* tb, hipStream_t stream);

}  // namespace hstu
