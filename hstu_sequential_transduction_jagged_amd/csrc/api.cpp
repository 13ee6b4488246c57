// C ABI of libhstu: argument checks, workspace carving and kernel launches.
// Every entry point only enqueues work on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/hstu.h"
#include <cmath>

#include "hstu_internal.h"

using namespace hstu;

namespace {

thread_local char g_last_error[512] = "";

hstu_status fail(hstu_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
hstu_status fail(hstu_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

hstu_status check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return HSTU_OK;
  return fail(HSTU_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kHeader = 256;
constexpr int kMinBlockRows = 128;  // smallest query tile of any attention kernel

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// timestamps may be null only for a batch without tokens (total_tokens 0)
hstu_status check_bias(const hstu_bias* bias, int32_t H, BiasArgs* out, int64_t total_tokens) {
  *out = BiasArgs{};
  if (!bias || bias->kind == HSTU_BIAS_NONE) {
    out->kind = 0;
    return HSTU_OK;
  }
  if (bias->kind == HSTU_BIAS_RAB_PT) {
    if ((!bias->timestamps && total_tokens > 0) || !bias->w_pos || !bias->w_time)
      return fail(HSTU_ERR_INVALID_ARG, "rab_pt bias needs timestamps, w_pos and w_time");
    if (bias->num_pos_buckets < 1 || bias->num_pos_buckets > kMaxPosBuckets)
      return fail(HSTU_ERR_UNSUPPORTED, "num_pos_buckets must be in [1, %d]", kMaxPosBuckets);
    if (bias->num_time_buckets < 1 || bias->num_time_buckets > kMaxTimeBuckets)
      return fail(HSTU_ERR_UNSUPPORTED, "num_time_buckets must be in [1, %d]", kMaxTimeBuckets);
    if (bias->pos_head_stride < 0 || bias->time_head_stride < 0)
      return fail(HSTU_ERR_INVALID_ARG, "table head strides must be >= 0");
    if ((bias->pos_head_stride && bias->pos_head_stride < bias->num_pos_buckets) ||
        (bias->time_head_stride && bias->time_head_stride < bias->num_time_buckets))
      return fail(HSTU_ERR_INVALID_ARG, "a nonzero table head stride must cover the table");
    out->kind = 1;
    out->ts = bias->timestamps;
    out->w_pos = bias->w_pos;
    out->w_time = bias->w_time;
    out->num_pos = bias->num_pos_buckets;
    out->num_time = bias->num_time_buckets;
    out->pos_stride = bias->pos_head_stride;
    out->time_stride = bias->time_head_stride;
    return HSTU_OK;
  }
  if (bias->kind == HSTU_BIAS_ALIBI) {
    out->kind = 2;
    out->slopes = bias->alibi_slopes;
    return HSTU_OK;
  }
  (void)H;
  return fail(HSTU_ERR_INVALID_ARG, "unknown bias kind %d", bias->kind);
}

}  // namespace

extern "C" {

const char* hstu_status_string(int32_t status) {
  switch (status) {
    case HSTU_OK: return "ok";
    case HSTU_ERR_INVALID_ARG: return "invalid argument";
    case HSTU_ERR_UNSUPPORTED: return "unsupported shape or option";
    case HSTU_ERR_WORKSPACE: return "workspace too small or misaligned";
    case HSTU_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* hstu_last_error(void) { return g_last_error; }

// Attention workspace: [count | pad to 256] [work list] [TimeStat x T] [int32 x T]
// [tile classes: 8 bytes x max_blocks per row, rows as tclass_row0 assigns them]
static size_t worklist_bytes(int32_t B, int32_t H, int32_t max_seqlen) {
  const int64_t items = (int64_t)B * H * ceil_div(max_seqlen, kMinBlockRows);
  return kHeader + align256((size_t)items * sizeof(WorkItem));
}

static int32_t tclass_cols(int32_t max_seqlen) { return (int32_t)ceil_div(max_seqlen, 32); }

static size_t tclass_bytes(int32_t B, int32_t max_seqlen, int64_t total_tokens) {
  const int64_t rows = (total_tokens + 31 * (int64_t)B) / 32 + 1;
  return (size_t)rows * (size_t)tclass_cols(max_seqlen) * 8;
}

// per (32-key block, head) key norm bounds, block rows numbered as the tile classes
static size_t knorm_bytes(int32_t B, int32_t H, int64_t total_tokens) {
  const int64_t rows = (total_tokens + 31 * (int64_t)B) / 32 + 1;
  return (size_t)rows * (size_t)H * 4;
}

size_t hstu_attn_workspace_bytes(int32_t B, int32_t H, int32_t max_seqlen, int64_t total_tokens) {
  if (B < 0 || H < 0 || max_seqlen < 0 || total_tokens < 0) return 0;
  return worklist_bytes(B, H, max_seqlen) + align256((size_t)total_tokens * sizeof(TimeStat)) +
         align256((size_t)total_tokens * sizeof(int32_t)) +
         align256(tclass_bytes(B, max_seqlen, total_tokens)) +
         align256(knorm_bytes(B, H, total_tokens));
}

// bf16 inputs with an fp32 output run the bf16 kernels; *o_f32 says which output
static int32_t input_dtype(int32_t dt, bool* o_f32) {
  if (o_f32) *o_f32 = dt == HSTU_DTYPE_BF16_OUT_F32;
  return dt == HSTU_DTYPE_BF16_OUT_F32 ? (int32_t)HSTU_DTYPE_BF16 : dt;
}

int32_t hstu_attn_block_rows(int32_t dt, int32_t d) {
  dt = input_dtype(dt, nullptr);
  if (dt == HSTU_DTYPE_BF16) return attn_block_rows_bf16(d);
  if (dt == HSTU_DTYPE_F32) return attn_block_rows_f32(d);
  return 0;
}

static hstu_status attn_check(int32_t dt, int32_t B, int32_t H, int32_t d_qk, int32_t d_v,
                              int32_t max_seqlen, int64_t total_tokens, int* block_rows) {
  if (dt != HSTU_DTYPE_BF16 && dt != HSTU_DTYPE_F32)
    return fail(HSTU_ERR_INVALID_ARG, "unknown dtype %d", dt);
  if (B < 0 || H < 1 || max_seqlen < 0 || total_tokens < 0)
    return fail(HSTU_ERR_INVALID_ARG, "negative size (B=%d H=%d max_seqlen=%d T=%lld)", B, H,
                max_seqlen, (long long)total_tokens);
  if (d_qk != d_v) return fail(HSTU_ERR_UNSUPPORTED, "d_qk != d_v is not supported");
  *block_rows = hstu_attn_block_rows(dt, d_qk);
  if (*block_rows == 0)
    return fail(HSTU_ERR_UNSUPPORTED, "head dim %d unsupported for dtype %d", d_qk, dt);
  if (max_seqlen > 65536) return fail(HSTU_ERR_UNSUPPORTED, "max_seqlen above 65536");
  if (H > 65535) return fail(HSTU_ERR_UNSUPPORTED, "H above 65535");
  return HSTU_OK;
}

static hstu_status workspace_check(const void* workspace, size_t workspace_bytes, int32_t B,
                                   int32_t H, int32_t max_seqlen, int64_t total_tokens) {
  const size_t need = hstu_attn_workspace_bytes(B, H, max_seqlen, total_tokens);
  if (!workspace) return fail(HSTU_ERR_INVALID_ARG, "null workspace");
  if (workspace_bytes < need || ((uintptr_t)workspace & 255u))
    return fail(HSTU_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                workspace_bytes);
  return HSTU_OK;
}

hstu_status hstu_attn_plan(int32_t dt, int32_t B, int32_t H, int32_t d, const int32_t* offsets,
                           int32_t max_seqlen, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  g_last_error[0] = 0;
  dt = input_dtype(dt, nullptr);
  int block_rows = 0;
  hstu_status st = attn_check(dt, B, H, d, d, max_seqlen, 0, &block_rows);
  if (st != HSTU_OK) return st;
  if (B == 0 || max_seqlen == 0) return HSTU_OK;
  if (!offsets) return fail(HSTU_ERR_INVALID_ARG, "null offsets");
  st = workspace_check(workspace, workspace_bytes, B, H, max_seqlen, 0);
  if (st != HSTU_OK) return st;
  const int32_t max_tiles = (int32_t)ceil_div(max_seqlen, block_rows);
  return check_hip(launch_schedule(offsets, B, H, block_rows, max_tiles, (int32_t*)workspace,
                                   (WorkItem*)((char*)workspace + kHeader), stream),
                   "scheduler launch");
}

// the backward kernels' work list: the forward's scheduler at the backward's item height
static hstu_status bwd_plan(int32_t B, int32_t H, const int32_t* offsets, int32_t max_seqlen,
                            void* workspace, int64_t* grid, hipStream_t stream) {
  const int32_t rows = attn_bwd_block_rows();
  const int32_t max_tiles = (int32_t)ceil_div(max_seqlen, rows);
  *grid = (int64_t)B * H * max_tiles;
  if (*grid > 0x7fffffff) return fail(HSTU_ERR_UNSUPPORTED, "too many work items");
  return check_hip(launch_schedule(offsets, B, H, rows, max_tiles, (int32_t*)workspace,
                                   (WorkItem*)((char*)workspace + kHeader), stream),
                   "scheduler launch");
}

// per 32-token block timestamp statistics for the backward kernels (position + time bias only),
// in the attention workspace's statistics region
static hstu_status bwd_time_stats(int32_t B, const int32_t* offsets, int32_t max_seqlen,
                                  int64_t total_tokens, int32_t H, const BiasArgs& ba,
                                  void* workspace, const TimeStat** out, hipStream_t stream) {
  *out = nullptr;
  if (ba.kind != 1) return HSTU_OK;
  TimeStat* tstat = (TimeStat*)((char*)workspace + worklist_bytes(B, H, max_seqlen));
  int32_t* trel = (int32_t*)((char*)tstat + align256((size_t)total_tokens * sizeof(TimeStat)));
  *out = tstat;
  return check_hip(launch_time_stats(B, offsets, ba.ts, max_seqlen, tstat, trel, stream),
                   "time stats launch");
}

// what attn_planned enqueues: the per-batch prepasses the bf16 kernel reads (timestamp
// statistics and tile classes of the position + time bias, key norm bounds), the attention
// kernel, or both
enum AttnPart { kPrepareAndRun = 0, kPrepareOnly = 1, kRunOnly = 2 };

static hstu_status attn_planned(int32_t dt, int32_t B, int32_t H, int32_t d_qk, int32_t d_v,
                                const int32_t* offsets, int32_t max_seqlen, int64_t total_tokens,
                                const void* q, int64_t q_row_stride, const void* k,
                                int64_t k_row_stride, const void* v, int64_t v_row_stride,
                                const hstu_bias* bias, float alpha, float out_scale, void* o,
                                bool o_f32, f32x4* ostats, void* workspace,
                                size_t workspace_bytes, hipStream_t stream,
                                AttnPart part = kPrepareAndRun, bool classes_ready = false) {
  int block_rows = 0;
  hstu_status st = attn_check(dt, B, H, d_qk, d_v, max_seqlen, total_tokens, &block_rows);
  if (st != HSTU_OK) return st;
  BiasArgs ba;
  st = check_bias(bias, H, &ba, total_tokens);
  if (st != HSTU_OK) return st;
  if (B == 0 || total_tokens == 0 || max_seqlen == 0) return HSTU_OK;
  if (!offsets || !q || !k || !v || !o) return fail(HSTU_ERR_INVALID_ARG, "null pointer argument");
  const int64_t rowlen = (int64_t)H * d_qk;
  if (q_row_stride < rowlen || k_row_stride < rowlen || v_row_stride < rowlen)
    return fail(HSTU_ERR_INVALID_ARG, "row stride smaller than H*d");
  const int elem = dt == HSTU_DTYPE_BF16 ? 2 : 4;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (q_row_stride * elem) % 16 || (k_row_stride * elem) % 16 || (v_row_stride * elem) % 16)
    return fail(HSTU_ERR_INVALID_ARG, "q/k/v/o rows must be 16-byte aligned");
  st = workspace_check(workspace, workspace_bytes, B, H, max_seqlen, total_tokens);
  if (st != HSTU_OK) return st;
  if (o_f32 && dt != HSTU_DTYPE_BF16) return fail(HSTU_ERR_INVALID_ARG, "fp32 output needs bf16 inputs");
  // the bf16 kernel addresses one user's K and V rows with 32-bit byte offsets
  const int64_t max_stride = k_row_stride > v_row_stride ? k_row_stride : v_row_stride;
  if (dt == HSTU_DTYPE_BF16 && (int64_t)max_seqlen * max_stride * 2 >= ((int64_t)1 << 31))
    return fail(HSTU_ERR_UNSUPPORTED, "max_seqlen x row stride reaches 2 GiB per user");

  const int32_t max_tiles = (int32_t)ceil_div(max_seqlen, block_rows);
  TimeStat* tstat = (TimeStat*)((char*)workspace + worklist_bytes(B, H, max_seqlen));
  int32_t* trel = (int32_t*)((char*)tstat + align256((size_t)total_tokens * sizeof(TimeStat)));
  uint32_t* tclass = (uint32_t*)((char*)trel + align256((size_t)total_tokens * sizeof(int32_t)));
  float* knorm = (float*)((char*)tclass + align256(tclass_bytes(B, max_seqlen, total_tokens)));
  if (dt == HSTU_DTYPE_BF16 && part != kRunOnly) {
    // key norm bounds, and for the position + time bias the timestamp statistics with them
    const bool rab = ba.kind == 1;
    st = check_hip(launch_key_norm(B, offsets, total_tokens, k, k_row_stride, H, d_qk, knorm,
                                   rab ? ba.ts : nullptr, rab ? tstat : nullptr,
                                   rab ? trel : nullptr, stream),
                   "key norm launch");
    if (st != HSTU_OK) return st;
  }
  if (dt == HSTU_DTYPE_BF16 && ba.kind == 1 && part != kRunOnly && !classes_ready) {
    st = check_hip(launch_tile_class(B, offsets, tstat, tclass_cols(max_seqlen), ba.num_pos,
                                     ba.num_time, tclass, stream),
                   "tile class launch");
    if (st != HSTU_OK) return st;
  }
  if (part == kPrepareOnly) return HSTU_OK;
  AttnArgs a{};
  a.tstat = tstat;
  a.trel = trel;
  a.tclass = tclass;
  a.tclass_cols = tclass_cols(max_seqlen);
  a.tclass_bytes = (int64_t)tclass_bytes(B, max_seqlen, total_tokens);
  a.offsets = offsets;
  a.work_count = (const int32_t*)workspace;
  a.work = (const WorkItem*)((const char*)workspace + kHeader);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.q_stride = q_row_stride;
  a.k_stride = k_row_stride;
  a.v_stride = v_row_stride;
  a.H = H;
  a.o_f32 = o_f32 ? 1 : 0;
  a.bias = ba;
  a.alpha = alpha;
  a.out_scale = out_scale;
  a.ostats = ostats;
  a.knorm = knorm;
  const int64_t grid = (int64_t)B * H * max_tiles;
  if (grid > 0x7fffffff) return fail(HSTU_ERR_UNSUPPORTED, "too many work items");
  hipError_t e = dt == HSTU_DTYPE_BF16 ? launch_attn_bf16(d_qk, a, (int)grid, stream)
                                       : launch_attn_f32(d_qk, a, (int)grid, stream);
  return check_hip(e, "attention launch");
}

hstu_status hstu_attn_fwd_planned(int32_t dt, int32_t B, int32_t H, int32_t d_qk, int32_t d_v,
                                  const int32_t* offsets, int32_t max_seqlen,
                                  int64_t total_tokens, const void* q, int64_t q_row_stride,
                                  const void* k, int64_t k_row_stride, const void* v,
                                  int64_t v_row_stride, const hstu_bias* bias, float alpha,
                                  float out_scale, void* o, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  g_last_error[0] = 0;
  bool of32 = false;
  dt = input_dtype(dt, &of32);
  return attn_planned(dt, B, H, d_qk, d_v, offsets, max_seqlen, total_tokens, q, q_row_stride, k,
                      k_row_stride, v, v_row_stride, bias, alpha, out_scale, o, of32, nullptr,
                      workspace, workspace_bytes, stream);
}

hstu_status hstu_attn_prepare(int32_t dt, int32_t B, int32_t H, int32_t d,
                              const int32_t* offsets, int32_t max_seqlen, int64_t total_tokens,
                              const void* k, int64_t k_row_stride, const hstu_bias* bias,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error[0] = 0;
  dt = input_dtype(dt, nullptr);
  // q, v and o are not read: K stands in for them so that the shared checks pass
  return attn_planned(dt, B, H, d, d, offsets, max_seqlen, total_tokens, k, k_row_stride, k,
                      k_row_stride, k, k_row_stride, bias, 1.0f, 1.0f, (void*)k, false, nullptr,
                      workspace, workspace_bytes, stream, kPrepareOnly);
}

hstu_status hstu_attn_fwd_prepared(int32_t dt, int32_t B, int32_t H, int32_t d_qk, int32_t d_v,
                                   const int32_t* offsets, int32_t max_seqlen,
                                   int64_t total_tokens, const void* q, int64_t q_row_stride,
                                   const void* k, int64_t k_row_stride, const void* v,
                                   int64_t v_row_stride, const hstu_bias* bias, float alpha,
                                   float out_scale, void* o, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  g_last_error[0] = 0;
  bool of32 = false;
  dt = input_dtype(dt, &of32);
  return attn_planned(dt, B, H, d_qk, d_v, offsets, max_seqlen, total_tokens, q, q_row_stride, k,
                      k_row_stride, v, v_row_stride, bias, alpha, out_scale, o, of32, nullptr,
                      workspace, workspace_bytes, stream, kRunOnly);
}

hstu_status hstu_attn_fwd(int32_t dt, int32_t B, int32_t H, int32_t d_qk, int32_t d_v,
                          const int32_t* offsets, int32_t max_seqlen, int64_t total_tokens,
                          const void* q, int64_t q_row_stride, const void* k,
                          int64_t k_row_stride, const void* v, int64_t v_row_stride,
                          const hstu_bias* bias, float alpha, float out_scale, void* o,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error[0] = 0;
  const int32_t dt_call = dt;
  dt = input_dtype(dt, nullptr);
  int block_rows = 0;
  hstu_status st = attn_check(dt, B, H, d_qk, d_v, max_seqlen, total_tokens, &block_rows);
  if (st != HSTU_OK) return st;
  BiasArgs ba;
  st = check_bias(bias, H, &ba, total_tokens);
  if (st != HSTU_OK) return st;
  if (B == 0 || total_tokens == 0 || max_seqlen == 0) return HSTU_OK;
  if (!offsets || !q || !k || !v || !o || !workspace)
    return fail(HSTU_ERR_INVALID_ARG, "null pointer argument");
  // argument checks of the attention half first, so that nothing is enqueued on error
  const int64_t rowlen = (int64_t)H * d_qk;
  if (q_row_stride < rowlen || k_row_stride < rowlen || v_row_stride < rowlen)
    return fail(HSTU_ERR_INVALID_ARG, "row stride smaller than H*d");
  const int elem = dt == HSTU_DTYPE_BF16 ? 2 : 4;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (q_row_stride * elem) % 16 || (k_row_stride * elem) % 16 || (v_row_stride * elem) % 16)
    return fail(HSTU_ERR_INVALID_ARG, "q/k/v/o rows must be 16-byte aligned");
  st = workspace_check(workspace, workspace_bytes, B, H, max_seqlen, total_tokens);
  if (st != HSTU_OK) return st;
  st = hstu_attn_plan(dt, B, H, d_qk, offsets, max_seqlen, workspace, workspace_bytes, stream);
  if (st != HSTU_OK) return st;
  return hstu_attn_fwd_planned(dt_call, B, H, d_qk, d_v, offsets, max_seqlen, total_tokens, q,
                               q_row_stride, k, k_row_stride, v, v_row_stride, bias, alpha,
                               out_scale, o, workspace, workspace_bytes, stream);
}

// ---- a stack of layers, with the f2 / next f1 boundary fused or not ----
size_t hstu_stack_workspace_bytes(int32_t B, int64_t total_tokens, int32_t d_model, int32_t H,
                                  int32_t d_qk, int32_t d_v, int32_t max_seqlen) {
  const size_t lw = hstu_layer_workspace_bytes(B, total_tokens, d_model, H, d_qk, d_v, max_seqlen);
  if (!lw || total_tokens < 0) return 0;
  return align256(lw) + 2 * align256((size_t)total_tokens * d_model * 2);
}

hstu_status hstu_stack_fwd(int32_t dt, int32_t B, int32_t n_layers, int32_t d_model, int32_t H,
                           int32_t d_qk, int32_t d_v, const int32_t* offsets, int32_t max_seqlen,
                           int64_t total_tokens, const void* x, const void* const* w1,
                           const float* const* b1, const float* const* ln_gamma,
                           const float* const* ln_beta, float ln_eps, const void* const* w2,
                           const float* const* b2, const hstu_bias* const* bias, float alpha,
                           int32_t residual, int32_t fuse_boundaries, void* y, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  g_last_error[0] = 0;
  if (n_layers < 1) return fail(HSTU_ERR_INVALID_ARG, "n_layers must be >= 1");
  if (!w1 || !b1 || !ln_gamma || !ln_beta || !w2 || !b2 || !bias)
    return fail(HSTU_ERR_INVALID_ARG, "null per-layer argument array");
  if (dt != HSTU_DTYPE_BF16) return fail(HSTU_ERR_UNSUPPORTED, "the layer runs in bf16 only");
  if (B < 0 || total_tokens < 0 || d_model < 1 || H < 1 || max_seqlen < 0)
    return fail(HSTU_ERR_INVALID_ARG, "bad sizes");
  if (d_qk != d_v || d_qk != 64) return fail(HSTU_ERR_UNSUPPORTED, "layer needs d_qk = d_v = 64");
  const int32_t N1 = 2 * H * (d_qk + d_v);
  const int32_t HV = H * d_v;
  if (d_model % 128 || N1 % 128 || HV % 64 || HV > 1024)
    return fail(HSTU_ERR_UNSUPPORTED,
                "layer needs d_model %% 128 == 0, 2H(dqk+dv) %% 128 == 0, H dv <= 1024");
  if (fuse_boundaries && (d_model != 512 || N1 % 512))
    return fail(HSTU_ERR_UNSUPPORTED, "the fused boundary needs d_model = 512 and 2H(dqk+dv) %% 512 == 0");
  if (!(ln_eps > 0.f)) return fail(HSTU_ERR_INVALID_ARG, "ln_eps must be > 0");
  for (int l = 0; l < n_layers; ++l) {
    BiasArgs ba;
    const hstu_status st = check_bias(bias[l], H, &ba, total_tokens);
    if (st != HSTU_OK) return st;
    if (!w1[l] || !w2[l]) return fail(HSTU_ERR_INVALID_ARG, "null weight of layer %d", l);
    if (!aligned16(w1[l]) || !aligned16(w2[l]))
      return fail(HSTU_ERR_INVALID_ARG, "weights of layer %d must be 16-byte aligned", l);
  }
  if (B == 0 || total_tokens == 0) return HSTU_OK;
  if (!offsets || !x || !y || !workspace) return fail(HSTU_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(x) || !aligned16(y)) return fail(HSTU_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
  if (x == y) return fail(HSTU_ERR_INVALID_ARG, "y may not alias x");
  const size_t need = hstu_stack_workspace_bytes(B, total_tokens, d_model, H, d_qk, d_v, max_seqlen);
  if (workspace_bytes < need || ((uintptr_t)workspace & 255u))
    return fail(HSTU_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                workspace_bytes);
  const size_t lw = align256(hstu_layer_workspace_bytes(B, total_tokens, d_model, H, d_qk, d_v, max_seqlen));
  const size_t xb = align256((size_t)total_tokens * d_model * 2);
  bf16* mid[2] = {(bf16*)((char*)workspace + lw), (bf16*)((char*)workspace + lw + xb)};
  auto layer_in = [&](int l) -> const bf16* { return l == 0 ? (const bf16*)x : mid[(l - 1) & 1]; };
  auto layer_out = [&](int l) -> bf16* { return l == n_layers - 1 ? (bf16*)y : mid[l & 1]; };
  // The work list depends on the offsets only and the tile classes on the offsets, the
  // timestamps and the bucket counts: both are computed once and reused by every layer whose
  // bias still matches; the key norm bounds (and the timestamp statistics) run per layer.
  size_t zo, oo, so, ao;
  hstu_layer_workspace_offsets(total_tokens, H, d_qk, d_v, &zo, &oo, &so, &ao);
  bf16* z = (bf16*)((char*)workspace + zo);
  bf16* obuf = (bf16*)((char*)workspace + oo);
  f32x4* ostats = (f32x4*)((char*)workspace + so);
  void* aws = (char*)workspace + ao;
  const size_t aws_bytes = align256(hstu_attn_workspace_bytes(B, H, max_seqlen, total_tokens));
  const bf16* U = z;
  const bf16* V = z + HV;
  const bf16* Q = z + 2 * HV;
  const bf16* K = z + 2 * HV + H * d_qk;
  hstu_status st = hstu_attn_plan(HSTU_DTYPE_BF16, B, H, d_qk, offsets, max_seqlen, aws,
                                  aws_bytes, stream);
  if (st != HSTU_OK) return st;
  const int64_t* cls_ts = nullptr;  // the bias the tile classes in the workspace were made for
  int32_t cls_p = -1, cls_nt = -1;
  for (int l = 0; l < n_layers; ++l) {
    if (l == 0 || !fuse_boundaries) {
      st = check_hip(launch_f1_gemm_silu(layer_in(l), (const bf16*)w1[l], b1[l], z, total_tokens,
                                         N1, d_model, stream),
                     "f1 launch");
      if (st != HSTU_OK) return st;
    }
    BiasArgs ba;
    check_bias(bias[l], H, &ba, total_tokens);  // validated above
    const bool ready = ba.kind == 1 && ba.ts == cls_ts && ba.num_pos == cls_p && ba.num_time == cls_nt;
    st = attn_planned(HSTU_DTYPE_BF16, B, H, d_qk, d_v, offsets, max_seqlen, total_tokens, Q, N1,
                      K, N1, V, N1, bias[l], alpha, 1.0f, obuf, false, ostats, aws, aws_bytes,
                      stream, kPrepareAndRun, ready);
    if (st != HSTU_OK) return st;
    if (ba.kind == 1) {
      cls_ts = ba.ts;
      cls_p = ba.num_pos;
      cls_nt = ba.num_time;
    }
    const bf16* res = residual ? layer_in(l) : nullptr;
    if (fuse_boundaries && l + 1 < n_layers)
      st = check_hip(launch_ln_gate_f2_f1(obuf, ostats, U, N1, ln_gamma[l], ln_beta[l], ln_eps,
                                          (const bf16*)w2[l], b2[l], res, layer_out(l),
                                          (const bf16*)w1[l + 1], b1[l + 1], z, N1, total_tokens,
                                          d_model, H, d_v, stream),
                     "fused f2 / f1 launch");
    else
      st = check_hip(launch_ln_gate_f2(obuf, ostats, U, N1, ln_gamma[l], ln_beta[l], ln_eps,
                                       (const bf16*)w2[l], b2[l], res, layer_out(l), total_tokens,
                                       d_model, H, d_v, stream),
                     "f2 launch");
    if (st != HSTU_OK) return st;
  }
  return HSTU_OK;
}

// ---- the attention forward without allocation ----
// Its workspace is a file-scope device array; each device holds its own copy, whose device
// address hipGetSymbolAddress gives once per device (the array's name is only a host-side
// stand-in).  Every call on a device shares that device's copy.
namespace {
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
__device__ __attribute__((aligned(256))) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;
}  // namespace

hstu_status hstu_attn_fwd_noalloc(int32_t dt, int32_t B, int32_t H, int32_t d_qk, int32_t d_v,
                                  const int32_t* offsets, int32_t max_seqlen,
                                  int64_t total_tokens, const void* q, int64_t q_row_stride,
                                  const void* k, int64_t k_row_stride, const void* v,
                                  int64_t v_row_stride, const hstu_bias* bias, float alpha,
                                  float out_scale, void* o, hipStream_t stream) {
  g_last_error[0] = 0;
  const size_t need = hstu_attn_workspace_bytes(B, H, max_seqlen, total_tokens);
  if (need > kNoAllocScratchBytes)
    return fail(HSTU_ERR_UNSUPPORTED,
                "this batch needs %zu bytes of attention workspace; the no-allocation entry point "
                "has %zu (use hstu_attn_fwd with a workspace)",
                need, kNoAllocScratchBytes);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return check_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(HSTU_ERR_UNSUPPORTED, "device %d above %d", dev, kMaxDevices);
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return check_hip(e, "hipGetSymbolAddress(scratch)");
      g_scratch_ptr[dev] = p;
    }
    ws = g_scratch_ptr[dev];
  }
  return hstu_attn_fwd(dt, B, H, d_qk, d_v, offsets, max_seqlen, total_tokens, q, q_row_stride, k,
                       k_row_stride, v, v_row_stride, bias, alpha, out_scale, o, ws,
                       kNoAllocScratchBytes, stream);
}

hstu_status hstu_attn_bwd(int32_t dt, int32_t B, int32_t H, int32_t d_qk, int32_t d_v,
                          const int32_t* offsets, int32_t max_seqlen, int64_t total_tokens,
                          const void* q, int64_t q_row_stride, const void* k,
                          int64_t k_row_stride, const void* v, int64_t v_row_stride,
                          const void* d_o, int64_t do_row_stride, const hstu_bias* bias,
                          float alpha, float out_scale, void* dq, void* dk, void* dv,
                          float* dw_pos, float* dw_time, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  g_last_error[0] = 0;
  if (dt != HSTU_DTYPE_BF16) return fail(HSTU_ERR_UNSUPPORTED, "the backward pass runs in bf16 only");
  if (d_qk != 64 || d_v != 64) return fail(HSTU_ERR_UNSUPPORTED, "the backward pass needs d = 64");
  int block_rows = 0;
  hstu_status st = attn_check(dt, B, H, d_qk, d_v, max_seqlen, total_tokens, &block_rows);
  if (st != HSTU_OK) return st;
  BiasArgs ba;
  st = check_bias(bias, H, &ba, total_tokens);
  if (st != HSTU_OK) return st;
  if (ba.kind == 1 && (!dw_pos || !dw_time))
    return fail(HSTU_ERR_INVALID_ARG, "rab_pt bias needs dw_pos and dw_time");
  if (B == 0 || total_tokens == 0 || max_seqlen == 0) {
    // no pairs: the table gradients are sums over nothing
    if (ba.kind == 1) {
      const int64_t np = ba.pos_stride ? (int64_t)H * ba.pos_stride : ba.num_pos;
      const int64_t nt = ba.time_stride ? (int64_t)H * ba.time_stride : ba.num_time;
      st = check_hip(launch_zero_f32(dw_pos, np, stream), "zero");
      if (st == HSTU_OK) st = check_hip(launch_zero_f32(dw_time, nt, stream), "zero");
    }
    return st;
  }
  if (!offsets || !q || !k || !v || !d_o || !dq || !dk || !dv || !workspace)
    return fail(HSTU_ERR_INVALID_ARG, "null pointer argument");
  const int64_t rowlen = (int64_t)H * d_qk;
  if (q_row_stride < rowlen || k_row_stride < rowlen || v_row_stride < rowlen ||
      do_row_stride < rowlen)
    return fail(HSTU_ERR_INVALID_ARG, "row stride smaller than H*d");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(d_o) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || q_row_stride % 8 || k_row_stride % 8 ||
      v_row_stride % 8 || do_row_stride % 8)
    return fail(HSTU_ERR_INVALID_ARG, "rows must be 16-byte aligned");
  st = workspace_check(workspace, workspace_bytes, B, H, max_seqlen, total_tokens);
  if (st != HSTU_OK) return st;
  int64_t max_stride = k_row_stride > v_row_stride ? k_row_stride : v_row_stride;
  if (q_row_stride > max_stride) max_stride = q_row_stride;
  if (do_row_stride > max_stride) max_stride = do_row_stride;
  if ((int64_t)(max_seqlen + 64) * max_stride * 2 >= ((int64_t)1 << 31))
    return fail(HSTU_ERR_UNSUPPORTED, "max_seqlen x row stride reaches 2 GiB per user");
  int64_t grid = 0;
  st = bwd_plan(B, H, offsets, max_seqlen, workspace, &grid, stream);
  if (st != HSTU_OK) return st;
  BwdArgs a{};
  a.offsets = offsets;
  a.work_count = (const int32_t*)workspace;
  a.work = (const WorkItem*)((const char*)workspace + kHeader);
  a.q = (const bf16*)q; a.k = (const bf16*)k; a.v = (const bf16*)v; a.dout = (const bf16*)d_o;
  a.q_stride = q_row_stride; a.k_stride = k_row_stride; a.v_stride = v_row_stride;
  a.do_stride = do_row_stride;
  a.H = H;
  a.bias = ba;
  a.alpha = alpha;
  a.out_scale = out_scale;
  a.dq = (bf16*)dq; a.dk = (bf16*)dk; a.dv = (bf16*)dv;
  a.dq_stride = a.dk_stride = a.dv_stride = (int64_t)H * 64;
  a.dw_pos = dw_pos; a.dw_time = dw_time;
  st = bwd_time_stats(B, offsets, max_seqlen, total_tokens, H, ba, workspace, &a.tstat, stream);
  if (st != HSTU_OK) return st;
  const int64_t n_pos = ba.kind == 1 ? (ba.pos_stride ? (int64_t)H * ba.pos_stride : ba.num_pos) : 0;
  const int64_t n_time = ba.kind == 1 ? (ba.time_stride ? (int64_t)H * ba.time_stride : ba.num_time) : 0;
  return check_hip(launch_attn_bwd_bf16(a, (int)grid, n_pos, n_time, stream), "backward launch");
}

// layer workspace: Z | O | per (token, head) O statistics (4 fp32) | attention workspace
void hstu_layer_workspace_offsets(int64_t total_tokens, int32_t H, int32_t d_qk, int32_t d_v,
                                  size_t* z_offset, size_t* o_offset, size_t* stats_offset,
                                  size_t* attn_offset) {
  const int64_t N1 = 2LL * H * (d_qk + d_v);
  const size_t z_bytes = align256((size_t)(total_tokens * N1 * 2));
  const size_t o_bytes = align256((size_t)(total_tokens * H * d_v * 2));
  const size_t s_bytes = align256((size_t)(total_tokens * H * 16));
  if (z_offset) *z_offset = 0;
  if (o_offset) *o_offset = z_bytes;
  if (stats_offset) *stats_offset = z_bytes + o_bytes;
  if (attn_offset) *attn_offset = z_bytes + o_bytes + s_bytes;
}

size_t hstu_layer_workspace_bytes(int32_t B, int64_t total_tokens, int32_t d_model, int32_t H,
                                  int32_t d_qk, int32_t d_v, int32_t max_seqlen) {
  if (B < 0 || total_tokens < 0 || d_model < 1 || H < 1 || d_qk < 1 || d_v < 1) return 0;
  size_t attn_off = 0;
  hstu_layer_workspace_offsets(total_tokens, H, d_qk, d_v, nullptr, nullptr, nullptr, &attn_off);
  return attn_off + align256(hstu_attn_workspace_bytes(B, H, max_seqlen, total_tokens));
}

hstu_status hstu_layer_fwd(int32_t dt, int32_t B, int32_t d_model, int32_t H, int32_t d_qk,
                           int32_t d_v, const int32_t* offsets, int32_t max_seqlen,
                           int64_t total_tokens, const void* x, const void* w1, const float* b1,
                           const float* ln_gamma, const float* ln_beta, float ln_eps,
                           const void* w2, const float* b2, const hstu_bias* bias, float alpha,
                           int32_t residual, void* y, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  g_last_error[0] = 0;
  if (dt != HSTU_DTYPE_BF16) return fail(HSTU_ERR_UNSUPPORTED, "the layer runs in bf16 only");
  if (B < 0 || total_tokens < 0 || d_model < 1 || H < 1 || max_seqlen < 0)
    return fail(HSTU_ERR_INVALID_ARG, "bad sizes");
  if (d_qk != d_v || d_qk != 64) return fail(HSTU_ERR_UNSUPPORTED, "layer needs d_qk = d_v = 64");
  const int32_t N1 = 2 * H * (d_qk + d_v);
  const int32_t HV = H * d_v;
  if (d_model % 128 || N1 % 128 || HV % 64 || HV > 1024)
    return fail(HSTU_ERR_UNSUPPORTED,
                "layer needs d_model %% 128 == 0, 2H(dqk+dv) %% 128 == 0, H dv <= 1024");
  if (!(ln_eps > 0.f)) return fail(HSTU_ERR_INVALID_ARG, "ln_eps must be > 0");
  BiasArgs ba;
  hstu_status st = check_bias(bias, H, &ba, total_tokens);
  if (st != HSTU_OK) return st;
  if (B == 0 || total_tokens == 0) return HSTU_OK;
  if (!offsets || !x || !w1 || !w2 || !y || !workspace)
    return fail(HSTU_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(x) || !aligned16(w1) || !aligned16(w2) || !aligned16(y))
    return fail(HSTU_ERR_INVALID_ARG, "x, w1, w2 and y must be 16-byte aligned");
  if (x == y) return fail(HSTU_ERR_INVALID_ARG, "y may not alias x");
  const size_t need = hstu_layer_workspace_bytes(B, total_tokens, d_model, H, d_qk, d_v, max_seqlen);
  if (workspace_bytes < need || ((uintptr_t)workspace & 255u))
    return fail(HSTU_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                workspace_bytes);
  size_t zo, oo, so, ao;
  hstu_layer_workspace_offsets(total_tokens, H, d_qk, d_v, &zo, &oo, &so, &ao);
  bf16* z = (bf16*)((char*)workspace + zo);
  bf16* obuf = (bf16*)((char*)workspace + oo);
  f32x4* ostats = (f32x4*)((char*)workspace + so);  // per (token, head) offset, mean, M2 of O
  void* aws = (char*)workspace + ao;
  const size_t aws_bytes = align256(hstu_attn_workspace_bytes(B, H, max_seqlen, total_tokens));

  st = check_hip(launch_f1_gemm_silu((const bf16*)x, (const bf16*)w1, b1, z, total_tokens, N1,
                                     d_model, stream),
                 "f1 launch");
  if (st != HSTU_OK) return st;
  // Split: U | V | Q | K column blocks of Z
  const bf16* U = z;
  const bf16* V = z + HV;
  const bf16* Q = z + 2 * HV;
  const bf16* K = z + 2 * HV + H * d_qk;
  st = hstu_attn_plan(HSTU_DTYPE_BF16, B, H, d_qk, offsets, max_seqlen, aws, aws_bytes, stream);
  if (st != HSTU_OK) return st;
  st = attn_planned(HSTU_DTYPE_BF16, B, H, d_qk, d_v, offsets, max_seqlen, total_tokens, Q, N1, K,
                    N1, V, N1, bias, alpha, 1.0f, obuf, false, ostats, aws, aws_bytes, stream);
  if (st != HSTU_OK) return st;
  return check_hip(launch_ln_gate_f2(obuf, ostats, U, N1, ln_gamma, ln_beta, ln_eps,
                                     (const bf16*)w2, b2, residual ? (const bf16*)x : nullptr,
                                     (bf16*)y, total_tokens, d_model, H, d_v, stream),
                   "f2 launch");
}

size_t hstu_attn_candidates_workspace_bytes(int32_t B, int32_t H, int32_t max_hist,
                                            int64_t total_hist, int64_t total_cand) {
  if (B < 0 || H < 0 || max_hist < 0 || total_hist < 0 || total_cand < 0) return 0;
  return cand_workspace_bytes(B, max_hist, total_hist, total_cand, H);
}

hstu_status hstu_attn_candidates_fwd(int32_t dt, int32_t B, int32_t H, int32_t d_qk, int32_t d_v,
                                     const int32_t* hist_offsets, int32_t max_hist,
                                     int64_t total_hist, const int32_t* cand_offsets,
                                     int32_t max_cand, int64_t total_cand, const void* q_cand,
                                     int64_t q_stride,
                                     const void* k_cand, int64_t k_cand_stride,
                                     const void* v_cand, int64_t v_cand_stride,
                                     const void* k_hist, int64_t k_hist_stride,
                                     const void* v_hist, int64_t v_hist_stride,
                                     const hstu_bias* bias, const int64_t* cand_timestamps,
                                     float alpha, float out_scale, void* o, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  g_last_error[0] = 0;
  if (dt != HSTU_DTYPE_BF16) return fail(HSTU_ERR_UNSUPPORTED, "candidate scoring runs in bf16 only");
  if (d_qk != 64 || d_v != 64) return fail(HSTU_ERR_UNSUPPORTED, "candidate scoring needs d = 64");
  if (B < 0 || H < 1 || max_hist < 0 || total_hist < 0 || max_cand < 0 || total_cand < 0)
    return fail(HSTU_ERR_INVALID_ARG, "bad sizes");
  BiasArgs ba;
  hstu_status st = check_bias(bias, H, &ba, total_hist + total_cand);
  if (st != HSTU_OK) return st;
  if (B == 0 || total_cand == 0 || max_cand == 0) return HSTU_OK;
  if (!hist_offsets || !cand_offsets || !q_cand || !k_cand || !v_cand || !o)
    return fail(HSTU_ERR_INVALID_ARG, "null pointer argument");
  if (max_hist > 0 && (!k_hist || !v_hist)) return fail(HSTU_ERR_INVALID_ARG, "null history K / V");
  if (ba.kind == 1 && !cand_timestamps)
    return fail(HSTU_ERR_INVALID_ARG, "rab_pt bias needs candidate timestamps");
  const int64_t rowlen = (int64_t)H * 64;
  if (q_stride < rowlen || k_cand_stride < rowlen || v_cand_stride < rowlen ||
      (max_hist > 0 && (k_hist_stride < rowlen || v_hist_stride < rowlen)))
    return fail(HSTU_ERR_INVALID_ARG, "row stride smaller than H*d");
  if (!aligned16(q_cand) || !aligned16(k_cand) || !aligned16(v_cand) || !aligned16(o) ||
      (max_hist > 0 && (!aligned16(k_hist) || !aligned16(v_hist))) || q_stride % 8 ||
      k_cand_stride % 8 || v_cand_stride % 8 || k_hist_stride % 8 || v_hist_stride % 8)
    return fail(HSTU_ERR_INVALID_ARG, "rows must be 16-byte aligned");
  // the kernel addresses one user's history rows with 32-bit byte offsets
  const int64_t hs = k_hist_stride > v_hist_stride ? k_hist_stride : v_hist_stride;
  if ((int64_t)(max_hist + 64) * hs * 2 >= ((int64_t)1 << 31))
    return fail(HSTU_ERR_UNSUPPORTED, "max_hist x row stride reaches 2 GiB per user");
  const size_t need = cand_workspace_bytes(B, max_hist, total_hist, total_cand, H);
  if ((!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)))
    return fail(HSTU_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                workspace_bytes);
  CandLaunch c{};
  c.B = B; c.H = H; c.max_hist = max_hist; c.max_cand = max_cand;
  c.total_hist = total_hist;
  c.total_cand = total_cand;
  c.workspace = workspace;
  c.hist_offsets = hist_offsets; c.cand_offsets = cand_offsets;
  c.q = (const bf16*)q_cand; c.kc = (const bf16*)k_cand; c.vc = (const bf16*)v_cand;
  c.kh = (const bf16*)k_hist; c.vh = (const bf16*)v_hist;
  c.q_stride = q_stride; c.kc_stride = k_cand_stride; c.vc_stride = v_cand_stride;
  c.kh_stride = k_hist_stride; c.vh_stride = v_hist_stride;
  c.o = (bf16*)o; c.bias = ba; c.cand_ts = cand_timestamps;
  c.alpha = alpha; c.out_scale = out_scale;
  return check_hip(launch_attn_candidates_bf16(c, stream), "candidate attention launch");
}

size_t hstu_layer_bwd_workspace_bytes(int32_t B, int64_t total_tokens, int32_t H, int32_t d_qk,
                                      int32_t d_v, int32_t max_seqlen) {
  if (B < 0 || total_tokens < 0 || H < 1 || d_qk < 1 || d_v < 1) return 0;
  const int64_t N1 = 2LL * H * (d_qk + d_v), HV = (int64_t)H * d_v;
  return 4 * align256((size_t)(total_tokens * HV * 2)) + align256((size_t)(total_tokens * N1 * 2)) +
         align256(hstu_attn_workspace_bytes(B, H, max_seqlen, total_tokens));
}

hstu_status hstu_layer_bwd(int32_t dt, int32_t B, int32_t d_model, int32_t H, int32_t d_qk,
                           int32_t d_v, const int32_t* offsets, int32_t max_seqlen,
                           int64_t total_tokens, const void* x, const void* w1, const float* b1,
                           const float* ln_gamma, const float* ln_beta, float ln_eps,
                           const void* w2, const hstu_bias* bias, float alpha, int32_t residual,
                           const void* fwd_workspace, const void* dy, void* dx, float* dw1,
                           float* db1, float* dgamma, float* dbeta, float* dw2, float* db2,
                           float* dw_pos, float* dw_time, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  g_last_error[0] = 0;
  if (dt != HSTU_DTYPE_BF16) return fail(HSTU_ERR_UNSUPPORTED, "the layer backward runs in bf16 only");
  if (d_qk != 64 || d_v != 64) return fail(HSTU_ERR_UNSUPPORTED, "the layer backward needs d = 64");
  if (B < 0 || H < 1 || d_model < 32 || d_model % 32 || max_seqlen < 0 || total_tokens < 0)
    return fail(HSTU_ERR_INVALID_ARG, "bad sizes (d_model must be a positive multiple of 32)");
  if ((int64_t)H * d_v > 2048) return fail(HSTU_ERR_UNSUPPORTED, "H * d_v above 2048");
  if (!(ln_eps > 0.f)) return fail(HSTU_ERR_INVALID_ARG, "ln_eps must be > 0");
  BiasArgs ba;
  hstu_status st = check_bias(bias, H, &ba, total_tokens);
  if (st != HSTU_OK) return st;
  if (ba.kind == 1 && (!dw_pos || !dw_time))
    return fail(HSTU_ERR_INVALID_ARG, "rab_pt bias needs dw_pos and dw_time");
  if (!dw1 || !db1 || !dgamma || !dbeta || !dw2 || !db2)
    return fail(HSTU_ERR_INVALID_ARG, "null weight-gradient pointer");
  const int64_t N1 = 2LL * H * (d_qk + d_v), HV = (int64_t)H * d_v, HQ = (int64_t)H * d_qk;
  // weight gradients are zeroed first (so an empty batch leaves zeros)
  st = check_hip(launch_zero_f32(dw1, N1 * d_model, stream), "zero");
  if (st == HSTU_OK) st = check_hip(launch_zero_f32(db1, N1, stream), "zero");
  if (st == HSTU_OK) st = check_hip(launch_zero_f32(dgamma, HV, stream), "zero");
  if (st == HSTU_OK) st = check_hip(launch_zero_f32(dbeta, HV, stream), "zero");
  if (st == HSTU_OK) st = check_hip(launch_zero_f32(dw2, d_model * HV, stream), "zero");
  if (st == HSTU_OK) st = check_hip(launch_zero_f32(db2, d_model, stream), "zero");
  if (st != HSTU_OK) return st;
  if (ba.kind == 1) {
    const int64_t np = ba.pos_stride ? (int64_t)H * ba.pos_stride : ba.num_pos;
    const int64_t nt = ba.time_stride ? (int64_t)H * ba.time_stride : ba.num_time;
    st = check_hip(launch_zero_f32(dw_pos, np, stream), "zero");
    if (st == HSTU_OK) st = check_hip(launch_zero_f32(dw_time, nt, stream), "zero");
    if (st != HSTU_OK) return st;
  }
  if (B == 0 || total_tokens == 0 || max_seqlen == 0) return HSTU_OK;
  if (!offsets || !x || !w1 || !ln_gamma || !ln_beta || !w2 || !fwd_workspace || !dy || !dx ||
      !workspace)
    return fail(HSTU_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(x) || !aligned16(w1) || !aligned16(w2) || !aligned16(dy) || !aligned16(dx) ||
      ((uintptr_t)fwd_workspace & 255u))
    return fail(HSTU_ERR_INVALID_ARG, "tensors must be 16-byte aligned (workspaces 256)");
  const size_t need = hstu_layer_bwd_workspace_bytes(B, total_tokens, H, d_qk, d_v, max_seqlen);
  if (workspace_bytes < need || ((uintptr_t)workspace & 255u))
    return fail(HSTU_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                workspace_bytes);
  if ((int64_t)(max_seqlen + 64) * N1 * 2 >= ((int64_t)1 << 31))
    return fail(HSTU_ERR_UNSUPPORTED, "max_seqlen x row stride reaches 2 GiB per user");
  size_t z_off = 0, o_off = 0, s_off = 0;
  hstu_layer_workspace_offsets(total_tokens, H, d_qk, d_v, &z_off, &o_off, &s_off, nullptr);
  const bf16* Z = (const bf16*)((const char*)fwd_workspace + z_off);
  const bf16* O = (const bf16*)((const char*)fwd_workspace + o_off);
  const f32x4* ostats = (const f32x4*)((const char*)fwd_workspace + s_off);
  char* ws = (char*)workspace;
  const size_t hvb = align256((size_t)(total_tokens * HV * 2));
  bf16* dG = (bf16*)ws;
  bf16* G = (bf16*)(ws + hvb);
  bf16* dO = (bf16*)(ws + 2 * hvb);
  bf16* dO_lo = (bf16*)(ws + 3 * hvb);
  bf16* dZ = (bf16*)(ws + 4 * hvb);
  void* attn_ws = ws + 4 * hvb + align256((size_t)(total_tokens * N1 * 2));
  const size_t attn_bytes = hstu_attn_workspace_bytes(B, H, max_seqlen, total_tokens);

  LayerBwdLaunch L{};
  L.T = total_tokens; L.D = d_model; L.HV = (int32_t)HV; L.N1 = (int32_t)N1;
  L.residual = residual ? 1 : 0; L.eps = ln_eps;
  L.x = (const bf16*)x; L.w1 = (const bf16*)w1; L.w2 = (const bf16*)w2; L.dy = (const bf16*)dy;
  L.o = O; L.ostats = ostats; L.dvh = d_v; L.u = Z; L.u_stride = N1;
  L.b1 = b1; L.gamma = ln_gamma; L.beta = ln_beta;
  L.dg = dG; L.g = G; L.dO = dO; L.dO_lo = dO_lo; L.dz = dZ; L.dx = (bf16*)dx; L.dz_stride = N1;
  L.dgamma = dgamma; L.dbeta = dbeta; L.dw1 = dw1; L.db1 = db1; L.dw2 = dw2; L.db2 = db2;
  st = check_hip(launch_layer_bwd_pre(L, stream), "layer backward (LN, f2) launch");
  if (st != HSTU_OK) return st;
  // attention gradients straight into dZ's V | Q | K columns
  int block_rows = 0;
  st = attn_check(dt, B, H, d_qk, d_v, max_seqlen, total_tokens, &block_rows);
  if (st != HSTU_OK) return st;
  int64_t grid = 0;
  st = bwd_plan(B, H, offsets, max_seqlen, attn_ws, &grid, stream);
  if (st != HSTU_OK) return st;
  BwdArgs a{};
  a.offsets = offsets;
  a.work_count = (const int32_t*)attn_ws;
  a.work = (const WorkItem*)((const char*)attn_ws + kHeader);
  a.v = Z + HV; a.q = Z + 2 * HV; a.k = Z + 2 * HV + HQ; a.dout = dO; a.dout_lo = dO_lo;
  a.q_stride = a.k_stride = a.v_stride = N1;
  a.do_stride = HV;
  a.H = H;
  a.bias = ba;
  a.alpha = alpha;
  a.out_scale = 1.0f;
  a.dv = dZ + HV; a.dq = dZ + 2 * HV; a.dk = dZ + 2 * HV + HQ;
  a.dq_stride = a.dk_stride = a.dv_stride = N1;
  a.dw_pos = dw_pos; a.dw_time = dw_time;
  st = bwd_time_stats(B, offsets, max_seqlen, total_tokens, H, ba, attn_ws, &a.tstat, stream);
  if (st != HSTU_OK) return st;
  const int64_t n_pos = ba.kind == 1 ? (ba.pos_stride ? (int64_t)H * ba.pos_stride : ba.num_pos) : 0;
  const int64_t n_time = ba.kind == 1 ? (ba.time_stride ? (int64_t)H * ba.time_stride : ba.num_time) : 0;
  st = check_hip(launch_attn_bwd_bf16(a, (int)grid, n_pos, n_time, stream), "attention backward launch");
  if (st != HSTU_OK) return st;
  return check_hip(launch_layer_bwd_post(L, stream), "layer backward (f1) launch");
}

size_t hstu_stochastic_length_workspace_bytes(int32_t B, int64_t total_tokens) {
  if (B < 0 || total_tokens < 0) return 0;
  return sl_workspace_bytes(B, total_tokens);
}

hstu_status hstu_stochastic_length(int32_t B, const int32_t* offsets, int32_t max_seqlen,
                                   int64_t total_tokens, int32_t N_c, double alpha,
                                   const float* u_user, const float* key_tok, const void* x,
                                   int64_t row_bytes, const int64_t* ts, int32_t* out_offsets,
                                   int32_t* src_index, void* x_out, int64_t* ts_out,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error[0] = 0;
  if (B < 0 || max_seqlen < 0 || total_tokens < 0 || N_c < 1)
    return fail(HSTU_ERR_INVALID_ARG, "bad sizes");
  if (!(alpha > 0.0 && alpha <= 2.0)) return fail(HSTU_ERR_INVALID_ARG, "alpha must be in (0, 2]");
  if (B == 0) return HSTU_OK;
  if (!offsets || !u_user || !out_offsets || !workspace)
    return fail(HSTU_ERR_INVALID_ARG, "null pointer argument");
  if (total_tokens > 0 && (!key_tok || !src_index))
    return fail(HSTU_ERR_INVALID_ARG, "null pointer argument");
  if (x && (!x_out || row_bytes <= 0 || row_bytes % 16 || !aligned16(x) || !aligned16(x_out)))
    return fail(HSTU_ERR_INVALID_ARG, "rows must be 16-byte multiples, 16-byte aligned");
  if (ts && !ts_out) return fail(HSTU_ERR_INVALID_ARG, "ts_out missing");
  const size_t need = sl_workspace_bytes(B, total_tokens);
  if (workspace_bytes < need || ((uintptr_t)workspace & 255u))
    return fail(HSTU_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                workspace_bytes);
  // the target length N_c^(alpha/2) (integer part) and N_c^alpha, in double on the host
  const int32_t L = (int32_t)floor(pow((double)N_c, alpha / 2.0));
  const double c = pow((double)N_c, alpha);
  return check_hip(launch_stochastic_length(B, offsets, max_seqlen, total_tokens, L, c, u_user,
                                            key_tok, x, row_bytes, ts, out_offsets, src_index,
                                            x_out, ts_out, workspace, stream),
                   "stochastic length launch");
}

hstu_status hstu_embed_sum_fwd(int64_t total_tokens, int32_t dim, const void* item_table,
                               int64_t num_items, const void* action_table, int32_t num_actions,
                               const int32_t* item_ids, const int32_t* action_ids, void* x,
                               hipStream_t stream) {
  g_last_error[0] = 0;
  if (total_tokens < 0 || dim < 1 || num_items < 0 || num_actions < 0)
    return fail(HSTU_ERR_INVALID_ARG, "bad sizes");
  if (dim % 8) return fail(HSTU_ERR_UNSUPPORTED, "dim must be a multiple of 8");
  if (total_tokens == 0) return HSTU_OK;
  if (!item_table || !action_table || !item_ids || !action_ids || !x)
    return fail(HSTU_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(item_table) || !aligned16(action_table) || !aligned16(x))
    return fail(HSTU_ERR_INVALID_ARG, "tables and x must be 16-byte aligned");
  return check_hip(launch_embed_sum(total_tokens, dim, (const bf16*)item_table, num_items,
                                    (const bf16*)action_table, num_actions, item_ids, action_ids,
                                    (bf16*)x, stream),
                   "embed launch");
}

hstu_status hstu_validate_offsets(int32_t B, const int32_t* offsets, int64_t total_tokens,
                                  int32_t max_seqlen, int32_t* flags_out, hipStream_t stream) {
  g_last_error[0] = 0;
  if (B < 0) return fail(HSTU_ERR_INVALID_ARG, "B < 0");
  if (!offsets || !flags_out) return fail(HSTU_ERR_INVALID_ARG, "null pointer argument");
  return check_hip(launch_validate_offsets(B, offsets, total_tokens, max_seqlen, flags_out, stream),
                   "validate launch");
}

hstu_status hstu_debug_buckets(int32_t B, const int32_t* offsets, const int64_t* timestamps,
                               int32_t num_pos_buckets, int32_t num_time_buckets, int64_t R,
                               const int64_t* token_i, const int64_t* token_j,
                               int32_t* pos_bucket_out, int32_t* time_bucket_out,
                               hipStream_t stream) {
  g_last_error[0] = 0;
  if (B < 1 || R < 0 || num_pos_buckets < 1 || num_time_buckets < 1 || num_time_buckets > 64)
    return fail(HSTU_ERR_INVALID_ARG, "bad sizes");
  if (R == 0) return HSTU_OK;
  if (!offsets || !timestamps || !token_i || !token_j || !pos_bucket_out || !time_bucket_out)
    return fail(HSTU_ERR_INVALID_ARG, "null pointer argument");
  return check_hip(launch_debug_buckets(B, offsets, timestamps, num_pos_buckets, num_time_buckets,
                                        R, token_i, token_j, pos_bucket_out, time_bucket_out,
                                        stream),
                   "debug launch");
}

}  // extern "C"
