// Jagged causal pointwise aggregated attention for gfx950.
//
// Computes, per user b, head h and local row i,
//     O[i] = out_scale * sum_{j <= i} SiLU(alpha <q_i, k_j> + rab_h(i, j)) v_j
// ("Actions Speak Louder than Words" reading notes §3.1 eq. (2) and §3.2: SiLU
// applied element-wise, no softmax; causal mask including the diagonal as in
// the toy layer of "4.4 推荐模型的 Scaling").
//
// Formulation used on the matrix cores.  Scores are produced transposed,
// S^T = K Q^T, so that the accumulator of a 32x32 MFMA tile holds one query
// per lane and 16 keys per lane in registers; that register set is exactly the
// B operand of the next MFMA, O^T += V^T P^T, so the SiLU weights never leave
// registers.  The key order inside a 16-key PV step is a fixed permutation of
// the accumulator's row order; the V^T operand is read in that order from the
// row-major V tile with transposing LDS reads (bf16 path).
//
// SiLU is evaluated in base-2 units: with y = -log2(e) x,
//     SiLU(x) = x / (1 + e^-x) = -(ln 2 / 2) * w(y),   w(y) = 2 y / (1 + 2^y),
// and the matrix cores accumulate w; -(ln 2 / 2) out_scale is applied once per
// output.  y = -log2(e) alpha s + bias_y costs one fma per score (folding the
// scale into Q instead would round the scaled Q to bf16 and double the output
// error).  w is computed either exactly, w = y / (0.5 + 0.5 * 2^y) (exp2 and
// reciprocal), or -- when a per-tile bound shows |y| <= 2 for every score of
// the tile -- by the odd polynomial w = y - y^2 P(y^2) (three fmas, no
// transcendental; relative error of 1/(1+2^y) below 7.5e-5, far under the bf16
// rounding of w).  The bound is |y| <= |alpha log2 e| max|q| max|k| + max|bias_y|
// with max-norms of the tile's query and key rows (Cauchy-Schwarz).
//
// Bias: rab_h(i, j) = w_pos[min(i-j, P-1)] + w_time[min(floor(log2(1+max(t_i-t_j,0))), NT-1)]
// (tables per head or shared), or ALiBi -slope_h (i - j) (GenRank article, part
// (2)).  Tables sit in LDS; for a 32x32 tile whose position bucket is saturated
// and whose time-delta range falls in one bucket (decided exactly from the
// tile's timestamp minima and maxima) the bias is one scalar, otherwise it is
// gathered per element.  The n x n bias is never materialised.
#include "hstu_internal.h"

namespace hstu {
namespace {

// Key (0..31) of a 32x32 accumulator's register r in lane half hf: rows
// 8*(r/4) + 4*hf + r%4 of the MFMA output layout.
__device__ __forceinline__ int acc_key(int r, int hf) { return 8 * (r >> 2) + 4 * hf + (r & 3); }

// Cross-lane moves inside a row of 16 lanes (DPP, no LDS round trip).

// Max over the 64 lanes of a wave, as a wave-uniform value.
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  auto at = [&](int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l)); };
  return fmaxf(fmaxf(at(0), at(16)), fmaxf(at(32), at(48)));
}

// ============================================================================================
// Timestamp statistics: for every 32-token block of a user (blocks start at the user's first
// token), the min and max timestamp, stored at the block's first token; and for every token
// its offset from its block's minimum as int32 (saturated; only read where the block spans
// at most 2^30).  One workgroup per (user, 256-token chunk).
// ============================================================================================
__global__ __launch_bounds__(256) void time_stats_kernel(const int32_t* __restrict__ offsets,
                                                        const int64_t* __restrict__ ts,
                                                        TimeStat* __restrict__ stats,
                                                        int32_t* __restrict__ rel) {
  const int b = blockIdx.x;
  const int64_t s = offsets[b];
  const int n = offsets[b + 1] - offsets[b];
  const int lane = threadIdx.x & 63, l32 = lane & 31;
  const int j = 256 * (int)blockIdx.y + (int)threadIdx.x;
  if (256 * (int)blockIdx.y >= n) return;
  {
    const bool valid = j < n;
    const int64_t t = valid ? ts[s + j] : 0;
    int64_t mn = valid ? t : kTMax, mx = valid ? t : kTMin;
    half_minmax(mn, mx);
    if (valid) {
      const int64_t d = t - mn;
      rel[s + j] = d > 0x7fffffffLL ? 0x7fffffff : (int32_t)d;
      if (l32 == 0) stats[s + j] = TimeStat{mn, mx};
    }
  }
}

// ============================================================================================
// Bias class of every (32-query block, 32-key block) pair of a user with key block <= query
// block, for the position + time bias (independent of the head: timestamps are per token):
//   info = mode | tlo << 4 | thi << 12, and dq = (query block min time) - (key block min time)
// with tlo / thi the smallest / largest time bucket any pair of the two blocks can have (from
// the blocks' min / max times, exactly), and
//   mode 1: position bucket saturated (i - j >= P - 1 for the whole tile), one time bucket;
//   mode 2: position saturated, time buckets tlo and tlo + 1, 32-bit offsets suffice;
//   mode 3: position varies, one time bucket;
//   mode 4: anything else on 32-bit time offsets; mode 5: anything else.
// 32-bit offsets suffice when the key block spans at most 2^30, the query block too, and the
// query times lie within 2^30 of the key block's minimum.  One workgroup per (user, query
// block), one thread per key block.
// ============================================================================================
__global__ __launch_bounds__(256) void tile_class_kernel(const int32_t* __restrict__ offsets,
                                                        const TimeStat* __restrict__ stats,
                                                        int max_blocks, int P, int NT,
                                                        uint32_t* __restrict__ tclass) {
  const int b = blockIdx.x, i = blockIdx.y;
  const int64_t tok0 = offsets[b];
  const int n = offsets[b + 1] - offsets[b];
  if (32 * i >= n) return;
  const TimeStat q = stats[tok0 + 32 * i];
  uint32_t* row = tclass + 2 * ((tclass_row0(tok0, b) + i) * (int64_t)max_blocks);
  for (int j = threadIdx.x; j <= i; j += 256) {
    const TimeStat k = stats[tok0 + 32 * j];
    const bool pconst = 32 * (i - j) - 31 >= P - 1;
    const int tlo = time_bucket(q.mn - k.mx, NT - 1);
    const int thi = time_bucket(q.mx - k.mn, NT - 1);
    const int64_t lim = 1LL << 30;
    const bool fits32 = (k.mx - k.mn) <= lim && (q.mx - q.mn) <= lim && (q.mx - k.mn) <= lim &&
                        (q.mn - k.mn) >= -lim;
    const int mode = pconst ? (tlo == thi ? 1 : (thi == tlo + 1 && fits32) ? 2 : fits32 ? 4 : 5)
                            : (tlo == thi ? 3 : fits32 ? 4 : 5);
    row[2 * j] = (uint32_t)mode | ((uint32_t)tlo << 4) | ((uint32_t)thi << 12);
    row[2 * j + 1] = fits32 ? (uint32_t)(int32_t)(q.mn - k.mn) : 0u;
  }
}

// ============================================================================================
// Key norm bounds: for every 32-key block of a user (blocks start at the user's first token)
// and head h, the largest squared norm of the block's key rows, in fp32 from the bf16 keys,
// at row tclass_row0(tok0, b) + block.  One workgroup of four waves per row: the row's user is
// found by a 64-way search over the offsets (one round trip to memory per factor of 64 users;
// rows between users exit at once); wave w takes heads w, w + 4, ... two at a time, with the
// loads of both heads in flight together: lane l sums the squares of half l % 2 of token l / 2's
// head row (d = 32 or 64 columns), the lane pair adds its halves and the wave's maximum is the
// bound.  No LDS, no barriers.  With timestamps, wave 3 also writes the block's timestamp
// statistics exactly as time_stats_kernel does (one launch fewer for the position + time bias).
// ============================================================================================
constexpr int kNormWaves = 4;

template <int D>
__global__ __launch_bounds__(64 * kNormWaves) void key_norm_kernel(const int32_t* __restrict__ offsets,
                                                       int32_t B, const bf16* __restrict__ k,
                                                       int64_t k_stride, int32_t H,
                                                       float* __restrict__ knorm,
                                                       const int64_t* __restrict__ ts,
                                                       TimeStat* __restrict__ stats,
                                                       int32_t* __restrict__ rel) {
  const int64_t r = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the last user whose first row is at or before r (first rows never decrease with b; user 0's
  // is 0): each step probes 64 users evenly spaced over the remaining range
  int lo = 0, len = B;
  while (len > 1) {
    const int step = (len + 63) / 64;
    const int i = lo + lane * step;
    const bool ok = lane * step < len && tclass_row0(offsets[i], i) <= r;
    const int cnt = (int)__popcll(__ballot(ok));  // >= 1: lane 0 probes lo
    lo += (cnt - 1) * step;
    len = min(step, len - (cnt - 1) * step);
  }
  const int b = __builtin_amdgcn_readfirstlane(lo);
  const int64_t tok0 = offsets[b];
  const int n = offsets[b + 1] - offsets[b];
  const int64_t blk64 = r - tclass_row0(tok0, b);
  if (blk64 < 0 || 32 * blk64 >= n) return;
  const int blk = (int)blk64;
  const int tok = 32 * blk + (lane >> 1);
  const bool valid = tok < n;
  const bf16* row = k + (tok0 + min(tok, n - 1)) * k_stride + (D / 2) * (lane & 1);
  float* dst = knorm + r * H;
  for (int h = wave; h < H; h += 2 * kNormWaves) {
    // heads h and h2 (= h when there is no second head: its result is not stored)
    const int h2 = h + kNormWaves < H ? h + kNormWaves : h;
    bf16x8 kv[2][D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      kv[0][c] = *(const bf16x8*)(row + (int64_t)h * D + 8 * c);
      kv[1][c] = *(const bf16x8*)(row + (int64_t)h2 * D + 8 * c);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < D / 16; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 pr = {kv[u][c][2 * e], kv[u][c][2 * e + 1]};
          acc = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, acc, false);
        }
      if (!valid) acc = 0.f;
      acc += __shfl_xor(acc, 1, 64);
      const float m = wave_max_dpp(acc);
      if (lane == 0 && (u == 0 || h2 != h)) dst[u == 0 ? h : h2] = m;
    }
  }
  if (ts && wave == kNormWaves - 1) {
    const int j = 32 * blk + (lane & 31);
    const bool ok = j < n;
    const int64_t t = ok ? ts[tok0 + j] : 0;
    int64_t mn = ok ? t : kTMax, mx = ok ? t : kTMin;
    half_minmax(mn, mx);
    if (ok && lane < 32) {
      const int64_t d = t - mn;
      rel[tok0 + j] = d > 0x7fffffffLL ? 0x7fffffff : (int32_t)d;
      if (lane == 0) stats[tok0 + j] = TimeStat{mn, mx};
    }
  }
}

// ============================================================================================
// bf16, d = 32 or 64: 4 waves x 32 queries = 128 query rows per work item, 64 keys per LDS
// stage (two stages filled by direct global -> LDS transfers, one barrier per tile), four
// workgroups per CU, so that each SIMD holds one wave of each of four workgroups and a
// workgroup waiting at its barrier leaves the SIMD to the other three.  One instantiation per
// bias kind (0 none, 1 position + time tables, 2 ALiBi), output type and head dim; with d = 32
// the stages keep their 128-byte rows
// and only the first four chunks of each row are fetched and read (two k-steps of the score
// product, one 32-column block of the output).
// ============================================================================================
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQW = 32;
constexpr int kBR = kWaves * kQW;
constexpr int kKB = 64;
constexpr int kD = 64;

// K and V rows of 64 bf16 (128 bytes, eight 16-byte chunks) are stored unpadded with chunk c of
// row r at position c ^ swz(r), swz(r) = ((r >> 1) & 1) << 2 | ((r >> 2) & 3).  Three access
// patterns then meet the 64 banks without conflicts: the K operand reads (16 lanes, one chunk of
// 16 consecutive rows: even and odd rows take the two 64-byte halves and swz is a bijection on
// each), the transposing V reads (32 lanes, chunks 0..3 or 4..7 of 4 consecutive rows: rows r
// and r + 2 differ in bit 2 of swz) and the transfers, which write whole rows.
__device__ __forceinline__ int swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
struct __attribute__((aligned(16))) Stage {
  __attribute__((aligned(16))) bf16 k[kKB * kD];   // row = key, swizzled chunks
  __attribute__((aligned(16))) bf16 v[kKB * kD];
  __attribute__((aligned(16))) int32_t krel[64];   // key time minus its 32-key block's minimum
  __attribute__((aligned(16))) uint32_t cls[64];   // tile class entries (block, half, word)
  __attribute__((aligned(16))) float kn[64];       // [0], [1]: max squared key norm of the halves
  __attribute__((aligned(16))) float dummy[64];    // target of the transfers that carry nothing
};
struct __attribute__((aligned(16))) SmemBf16 {
  __attribute__((aligned(16))) float tay[kMaxTimeBuckets][4];  // per time bucket: c, a0, a1, a2
  float wposx[kMaxPosBuckets + 96];  // -log2(e) * w_pos[h][clamp(i - j, 0, P - 1)] at i - j + 32
  float wtime[kMaxTimeBuckets]; // -log2(e) * w_time[h]
  float wtime_lz[32];           // wtime[min(31 - lz, NT - 1)]: time bias by leading zeros of dt + 1
  int32_t need[kWaves];         // ALiBi: the lowest 32-key block each wave still needs
};

template <int KIND, bool OUT_F32, int D>
__global__ __launch_bounds__(kThreads, 4) void attn_bf16_kernel(AttnArgs a) {
  static_assert(D == 32 || D == 64, "head dim");
  constexpr int NKS = D / 16;  // 16-wide k-steps of the score product
  constexpr int NDB = D / 32;  // 32-column blocks of the output
  __shared__ SmemBf16 sm;
  __shared__ Stage st0, st1;
  const int item = blockIdx.x;
  if (item >= *a.work_count) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31, hf = lane >> 5;
  const WorkItem wi = a.work[item];
  const int b = wi.b, h = wi.h, H = a.H;
  const int64_t tok0 = wi.tok0;
  const int n = wi.n;
  const int q0 = wi.qt * kBR;
  if (q0 >= n) return;
  const int q_end = min(q0 + kBR, n);
  const int n_tiles = (q_end + kKB - 1) / kKB;
  const int qw0 = q0 + wave * kQW;                // first query row of this wave
  const int wq_last = min(qw0 + kQW, q_end) - 1;  // < qw0 when the wave has no rows

  const bf16* __restrict__ qp = (const bf16*)a.q;
  const bf16* __restrict__ kp = (const bf16*)a.k;
  const bf16* __restrict__ vp = (const bf16*)a.v;
  const int64_t* __restrict__ ts = a.bias.ts;
  const TimeStat* __restrict__ tstat = a.tstat;
  const float cq = -a.alpha * kLog2e;
  const int Pm1 = a.bias.num_pos - 1, NTm1 = a.bias.num_time - 1;

  // ---- staging: direct global -> LDS transfers into two stages ----
  // Wave w's K and V transfers fill key rows 16 w .. 16 w + 15 of a stage, two instructions
  // each: lane p of instruction u writes row 16 w + 8 u + p / 8 at chunk position p % 8, i.e.
  // global chunk (p % 8) ^ swz(row).  Rows at or
  // past q_end read as zeros (buffer bounds).  One 4-byte transfer per wave: wave 0 the keys'
  // time offsets, wave 1 the class entries (both position + time bias only), wave 2 the two
  // halves' key norm bounds, the others nothing (out of range).
  const uint32_t kstride_b = (uint32_t)a.k_stride * 2u, vstride_b = (uint32_t)a.v_stride * 2u;
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(kp + tok0 * a.k_stride + (int64_t)h * D), (short)0,
      (int)((uint32_t)(q_end - 1) * kstride_b + 2u * D), 0x00020000);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(vp + tok0 * a.v_stride + (int64_t)h * D), (short)0,
      (int)((uint32_t)(q_end - 1) * vstride_b + 2u * D), 0x00020000);
  uint32_t kvo[2], vvo[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = 16 * wave + 8 * u + (lane >> 3);
    const uint32_t ch = 16u * (uint32_t)((lane & 7) ^ swz(r));
    kvo[u] = (uint32_t)r * kstride_b + ch;
    vvo[u] = (uint32_t)r * vstride_b + ch;
    if (D == 32 && ch >= 64u) kvo[u] = vvo[u] = 0x80000000u;
  }
  const int64_t crow = tclass_row0(tok0, b) + q0 / 32;
  const int64_t cbase = crow * a.tclass_cols * 8;  // bytes
  const int64_t krow0 = tclass_row0(tok0, b);  // the user's first 32-key block row
  const int nkb = (q_end + 31) / 32;            // key blocks this item reads
  const __amdgpu_buffer_rsrc_t rrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(wave == 2 ? (const void*)(a.knorm + krow0 * H + h)
              : KIND != 1 || wave > 2 ? nullptr
              : wave == 0 ? (const void*)(a.trel + tok0)
                          : (const void*)((const char*)a.tclass + cbase)),
      (short)0,
      wave == 2 ? (nkb - 1) * H * 4 + 4
      : KIND != 1 || wave > 2 ? 0
      : wave == 0 ? q_end * 4 : (int)min(a.tclass_bytes - cbase, (int64_t)0x7fffffff),
      0x00020000);
  // lanes whose entries no wave reads (class entries of rows past the item's four query blocks,
  // key norms past the tile's two blocks) fetch nothing: their offsets lie outside every buffer
  const uint32_t roff = wave == 0 ? 4u * lane
                      : wave == 2 ? (lane < 2 ? 4u * (uint32_t)H * (uint32_t)lane : 0x80000000u)
                      : lane < 4 * kWaves ? 8u * (uint32_t)a.tclass_cols * (uint32_t)(lane >> 2) + 4u * (lane & 3)
                                          : 0x80000000u;
  // tiles are visited in steps k = 0, 1, ..., n_loop - 1: upwards from the first key tile, or,
  // with ALiBi, downwards from the diagonal (so that the far tiles, whose weights the bias
  // drives below any fp32 resolution, come last and can be cut off; see kAlibiFarY)
  int n_loop = n_tiles;
  auto tix = [&](int k) { return KIND == 2 ? n_tiles - 1 - k : k; };
  auto dma = [&](Stage& stg, int k) __attribute__((always_inline)) {
    const bool real = k < n_loop;
    const int t = tix(real ? k : 0);
    const uint32_t j0 = (uint32_t)(t * kKB);
    const uint32_t ksoff = __builtin_amdgcn_readfirstlane(real ? j0 * kstride_b : 0x7fffffffu);
    const uint32_t vsoff = __builtin_amdgcn_readfirstlane(real ? j0 * vstride_b : 0x7fffffffu);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc, (lds_ptr)(stg.k + 1024 * wave), 16, kvo[0], ksoff, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc, (lds_ptr)(stg.k + 1024 * wave + 512), 16, kvo[1], ksoff, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrsrc, (lds_ptr)(stg.v + 1024 * wave), 16, vvo[0], vsoff, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrsrc, (lds_ptr)(stg.v + 1024 * wave + 512), 16, vvo[1], vsoff, 0, 0);
    const uint32_t msoff = __builtin_amdgcn_readfirstlane(
        !real ? 0x7fffffffu
        : wave == 2 ? (j0 / 32u) * 4u * (uint32_t)H
        : (KIND == 1 && wave < 2) ? (wave == 0 ? 4u * j0 : j0 / 4u) : 0x7fffffffu);
    void* dst = wave == 0 ? (void*)stg.krel : wave == 1 ? (void*)stg.cls
              : wave == 2 ? (void*)stg.kn : (void*)stg.dummy;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rrsrc, (lds_ptr)dst, 4, roff, msoff, 0, 0);
  };
  // the first tile's transfers go out before the item's register loads, so that their
  // latencies overlap
  dma(st0, 0);

  // ---- Q fragments (B operand of S^T = K Q^T), unscaled ----
  bf16x8 qop[NKS];
  const int row = qw0 + l32;
  const bool qvalid = row <= wq_last;
  {
    // unconditional loads from a row clamped into the item (a load under a branch would make
    // the compiler wait for every transfer in flight), zeroed for rows past it
    const bf16* src = qp + (tok0 + min(row, q_end - 1)) * a.q_stride + (int64_t)h * D + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 raw = *(const u32x4*)(src + 16 * ks);
      if (!qvalid) raw = u32x4{0u, 0u, 0u, 0u};
      qop[ks] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  // |alpha log2 e| times the max norm of the wave's query rows: with a tile's max key norm,
  // a bound on |y - bias| over the tile (Cauchy-Schwarz)
  float qbound;
  {
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2 pr = {qop[ks][2 * e], qop[ks][2 * e + 1]};
        ss = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, ss, false);
      }
    }
    ss += __shfl_xor(ss, 32, 64);  // the two lane halves hold the two halves of a row
    qbound = uniform_f32(fabsf(cq) * 1.0001f * sqrtf(wave_max(ss)));  // margin for rounding
  }

  // ---- bias set-up ----
  float slope_y = 0.f, ta0 = 0.f, ta1 = 0.f, ta2 = 0.f, tabmax = 0.f;
  int32_t tq_rel = 0;  // query time minus the wave's block minimum (32-bit paths)
  if (KIND == 1) {
    // every global read of the set-up goes out before the first of them is used (one memory
    // round trip instead of one per table and loop step); the tables' largest magnitude is
    // taken from LDS after the first barrier
    const float* wp = a.bias.w_pos + (int64_t)h * a.bias.pos_stride;
    const float* wt = a.bias.w_time + (int64_t)h * a.bias.time_stride;
    const int nposx = a.bias.num_pos + 96;
    constexpr int kPX = (kMaxPosBuckets + 96 + kThreads - 1) / kThreads;
    float px[kPX];
    // (indices clamped into the tables and the item: unconditional loads)
#pragma unroll
    for (int u = 0; u < kPX; ++u) px[u] = wp[min(max(tid + kThreads * u - 32, 0), Pm1)];
    const bool tb = tid < a.bias.num_time;
    const float wt_t = wt[min(tid, NTm1)];
    const float wp_sat = wp[Pm1];
    const float wt_lz = wt[min(max(31 - tid, 0), NTm1)];
    const int64_t tmin = tstat[tok0 + min(qw0, q_end - 1)].mn;
    const int64_t tqv = ts[tok0 + min(row, q_end - 1)];
#pragma unroll
    for (int u = 0; u < kPX; ++u) {
      const int i = tid + kThreads * u;
      if (i < nposx) sm.wposx[i] = -kLog2e * px[u];
    }
    if (tb) {
      // per time bucket: the bias of a tile with saturated position bucket, and its Taylor
      // coefficients
      const float c = -kLog2e * (wp_sat + wt_t);
      float x0, x1, x2;
      w_taylor_coeffs(c, cq, x0, x1, x2);
      *(f32x4*)(&sm.tay[tid][0]) = f32x4{c, x0, x1, x2};
      sm.wtime[tid] = -kLog2e * wt_t;
    }
    if (tid < 32) sm.wtime_lz[tid] = -kLog2e * wt_lz;
    if (qvalid) {
      const int64_t d = tqv - tmin;
      tq_rel = d > 0x7fffffffLL ? 0x7fffffff : (int32_t)d;
    }
  } else if (KIND == 0) {
    w_taylor_coeffs(0.f, cq, ta0, ta1, ta2);
  } else {
    slope_y = kLog2e * (a.bias.slopes ? a.bias.slopes[h] : default_alibi_slope(h, H));
  }
  // register r of a 32x32 accumulator holds key acc_key(r, hf) = kc(r) + 4 hf for query l32
  const int lv = l32 - 4 * hf;
  // transposing V reads: this lane's source row (key) and column (d) within a 16-key group
  const int vtr_row0 = 4 * hf + ((lane & 15) >> 2);
  const int vtr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const float neg_slope_y = -slope_y, alibi_lane = slope_y * (float)lv;
  if (KIND == 2) {
    // The far cut.  With y = slope_y (i - j) - log2(e) alpha s and |log2(e) alpha s| <= D_w =
    // qbound max|k| (max over the user's key blocks up to the item's last row), every pair of
    // this wave at distance i - j >= L_w = (kAlibiFarY + D_w) / slope_y has y >= kAlibiFarY.
    // The wave's lowest needed 32-key block is the first whose nearest pair is closer than L_w.
    int need = 0x7fffffff;  // a wave without rows needs nothing
    if (qw0 <= wq_last) {
      need = 0;
      if (slope_y > 0.f) {
        float km = 0.f;
        const int nkb = (q_end + 31) / 32;
        const int64_t krow0 = tclass_row0(tok0, b);
        for (int jb = lane; jb < nkb; jb += 64) km = fmaxf(km, a.knorm[(krow0 + jb) * H + h]);
        const float dw = qbound * sqrtf(wave_max(km)) * 1.0001f;
        const float lf = (kAlibiFarY + dw) / slope_y;
        if (lf < (float)(qw0 - 31)) {
          // blocks jb with qw0 - (32 jb + 31) >= L_w are cut: jb <= (qw0 - 31 - L_w) / 32
          const int lcut = (int)ceilf(lf * 1.0001f) + 1;
          const int jcut = qw0 - 31 - lcut;
          need = jcut >= 0 ? jcut / 32 + 1 : 0;
        }
      }
    }
    if (lane == 0) sm.need[wave] = uniform_i32(need);
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;

  // byte offsets of this lane's operand reads within a stage.  The K read of k-step ks takes
  // chunk 2 ks + hf of row l32 (+ 32 hk), at position (2 ks + hf) ^ swz(l32): kbase ^ (32 ks).
  // The V reads take chunk 4 db + vtr_col / 8 of row vtr_row0 + 8 e (+ 16 m + 32 hk): vbase[e]
  // ^ (64 db).  (The XORs touch bits 5 and 6 only, which the row offsets leave zero.)
  uint32_t kbase, vbase[2];
  {
    const int sk = swz(l32);
    kbase = (uint32_t)(l32 * 128 + 32 * (sk >> 1) + 16 * (hf ^ (sk & 1)));
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = vtr_row0 + 8 * e, sv = swz(r);
      vbase[e] = (uint32_t)(r * 128 + 64 * (sv >> 2) + 16 * ((vtr_col >> 3) ^ (sv & 3)) + 2 * (vtr_col & 7));
    }
  }

  enum { kExact = 0, kPoly = 1, kTaylor = 2, kFar = 3 };
  auto compute = [&](const Stage& stg, int t) __attribute__((always_inline)) {
    const int j0 = t * kKB;
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
      const int j0h = j0 + 32 * hk;
      if (j0h > wq_last || wq_last < qw0) continue;  // past the diagonal, or the wave has no rows
      const float kn2 = uniform_f32(stg.kn[hk]);
      if (KIND == 2) {
        // far tile: y >= slope_y (qw0 - j0h - 31) - qbound |k| >= kAlibiFarY for every pair
        const float room = slope_y * (float)(qw0 - j0h - 31) - kAlibiFarY;
        if (room > 0.f && room * room >= 1.0002f * qbound * qbound * kn2) continue;
      }
      // K operands of this 32-key step (V operands are read after the SiLU)
      bf16x8 kop[NKS], vop[NDB][2];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        kop[ks] = *(const bf16x8*)((const char*)stg.k + 32 * hk * 128 + (kbase ^ (32u * ks)));
      const bool diag = (j0h + 31) > qw0;
      // i - j of register r = dlt + lv - kc(r): a lane term, a tile term and a constant
      const int dlt = qw0 - j0h;
      auto kc = [](int r) { return 8 * (r >> 2) + (r & 3); };
      // dlt capped where every position bucket of the tile saturates: then i - j + 32 indexes
      // the extended position table within its P + 96 entries
      const int dltc = min(dlt, Pm1 + 33);

      // ---- this tile's bias mode and SiLU evaluation ----
      int mode, path, thi = 0, dq = 0;
      float c0 = 0.f, c1 = 0.f, A0 = ta0, A1 = ta1, A2 = ta2;
      if (KIND == 0) {
        mode = diag ? 3 : 1;
        const float D2 = qbound * qbound * kn2;
        path = D2 <= kTaylorD * kTaylorD ? kTaylor : D2 <= kPolyRange * kPolyRange ? kPoly : kExact;
      } else if (KIND == 1) {
        const u32x2 e = *(const u32x2*)(&stg.cls[4 * wave + 2 * hk]);
        const uint32_t info = __builtin_amdgcn_readfirstlane(e[0]);
        dq = (int32_t)__builtin_amdgcn_readfirstlane(e[1]);
        mode = info & 15;
        const int tlo = (info >> 4) & 255;
        thi = info >> 12;
        const f32x4 lo = *(const f32x4*)(&sm.tay[tlo][0]);
        c0 = uniform_f32(mode == 3 ? sm.wtime[tlo] : lo[0]);
        c1 = uniform_f32(sm.tay[thi][0]);
        A0 = uniform_f32(lo[1]);
        A1 = uniform_f32(lo[2]);
        A2 = uniform_f32(lo[3]);
        // |y - bias| <= D = qbound * knorm; Taylor iff the bias is one value and D <= kTaylorD,
        // polynomial iff D + max|bias| <= kPolyRange
        const float cabs = mode == 1 ? fabsf(c0) : mode == 2 ? fmaxf(fabsf(c0), fabsf(c1)) : tabmax;
        const float D2 = qbound * qbound * kn2;
        const float room = kPolyRange - cabs;
        path = (mode == 1 && D2 <= kTaylorD * kTaylorD) ? kTaylor
             : (room >= 0.f && D2 <= room * room) ? kPoly : kExact;
      } else {
        mode = 3;
        // |bias| <= |slope_y| (i - j) <= |slope_y| (qw0 + 31 - j0h) over the tile (any sign of slope)
        const float room = kPolyRange - fabsf(slope_y) * (float)max(qw0 + 31 - j0h, 0);
        path = (room >= 0.f && qbound * qbound * kn2 <= room * room) ? kPoly : kExact;
        // far from the diagonal with a positive slope: y >= slope_y (qw0 - j0h - 31) - D >= 16,
        // where with e = 2^-y the exact w = 2 y e / (1 + e) is 2 y e to a relative 2^-16
        const float fy = slope_y * (float)(qw0 - j0h - 31) - kFarExpY;
        if (fy > 0.f && fy * fy >= 1.0002f * qbound * qbound * kn2) path = kFar;
      }

      // S^T tile: rows = keys, columns = this wave's queries
      f32x16 sacc = {};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qop[ks], sacc, 0, 0, 0);

      // y = -log2(e) (alpha s + bias); w(y) = 2 y / (1 + 2^y) = -(2 / ln 2) SiLU(alpha s + bias)
      auto w_exact = [&](float y) {
        return y * __builtin_amdgcn_rcpf(__builtin_fmaf(__builtin_amdgcn_exp2f(y), 0.5f, 0.5f));
      };
      auto w_poly = [&](float y) {
        const float u = y * y;
        return __builtin_fmaf(-u, __builtin_fmaf(__builtin_fmaf(kP2, u, kP1), u, kP0), y);
      };
      f32x16 w;
      if (path == kTaylor && (mode == 1 || KIND == 0)) {
        // the common case: constant bias, small |delta|
#pragma unroll
        for (int r = 0; r < 16; ++r) w[r] = __builtin_fmaf(__builtin_fmaf(A2, sacc[r], A1), sacc[r], A0);
      } else if (mode == 1 || KIND == 0) {
        if (path == kPoly) {
#pragma unroll
          for (int r = 0; r < 16; ++r) w[r] = w_poly(__builtin_fmaf(sacc[r], cq, c0));
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) w[r] = w_exact(__builtin_fmaf(sacc[r], cq, c0));
        }
      } else if (KIND == 2) {
        // ALiBi: the bias is slope_y (i - j) = base - slope_y kc(r) per register, computed in place
        const float base = alibi_lane + slope_y * (float)dlt;
        if (path == kFar) {
          // far from the diagonal, in z = 1 - y: 2^z = 2 e and w = 2 y e = (1 - z) 2^z, so
          // w = fma(-z, 2^z, 2^z)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float z = __builtin_fmaf(sacc[r], -cq, __builtin_fmaf(slope_y, (float)kc(r), 1.0f - base));
            const float e2 = __builtin_amdgcn_exp2f(z);
            w[r] = __builtin_fmaf(-z, e2, e2);
          }
        } else if (path == kPoly) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            w[r] = w_poly(__builtin_fmaf(sacc[r], cq, __builtin_fmaf(neg_slope_y, (float)kc(r), base)));
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            w[r] = w_exact(__builtin_fmaf(sacc[r], cq, __builtin_fmaf(neg_slope_y, (float)kc(r), base)));
        }
      } else {
        // per-element bias (y units), four registers at a time
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 c4;
          if (mode == 2) {
            // two time buckets: dt >= 2^thi - 1  <=>  rel_j <= (t_i - kmin) - (2^thi - 1)
            const int lim = tq_rel + dq - ((1 << thi) - 1);
            const i32x4 rel4 = *(const i32x4*)(&stg.krel[32 * hk + 8 * g + 4 * hf]);
#pragma unroll
            for (int i = 0; i < 4; ++i) c4[i] = rel4[i] <= lim ? c1 : c0;
          } else if (mode == 3) {
#pragma unroll
            for (int i = 0; i < 4; ++i) c4[i] = sm.wposx[lv + (dltc - kc(4 * g + i)) + 32] + c0;
          } else if (mode == 4) {
            const int ti1 = tq_rel + dq + 1;
            const i32x4 rel4 = *(const i32x4*)(&stg.krel[32 * hk + 8 * g + 4 * hf]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int u = max(ti1 - rel4[i], 1);  // max(dt, 0) + 1
              c4[i] = sm.wposx[lv + (dltc - kc(4 * g + i)) + 32] + sm.wtime_lz[__builtin_clz((uint32_t)u)];
            }
          } else {
            // timestamps spread beyond 2^30 within the tile (rare): exact 64-bit deltas from
            // global memory
            const int64_t tq = ts[tok0 + min(row, n - 1)];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 4 * g + i;
              const int64_t tk = ts[tok0 + min(j0h + kc(r) + 4 * hf, n - 1)];
              c4[i] = sm.wposx[pos_bucket(lv + (dlt - kc(r)), Pm1) + 32] + sm.wtime[time_bucket(tq - tk, NTm1)];
            }
          }
          if (path == kPoly) {
#pragma unroll
            for (int i = 0; i < 4; ++i) w[4 * g + i] = w_poly(__builtin_fmaf(sacc[4 * g + i], cq, c4[i]));
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) w[4 * g + i] = w_exact(__builtin_fmaf(sacc[4 * g + i], cq, c4[i]));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (diag) {
#pragma unroll
        for (int r = 0; r < 16; ++r) w[r] = lv >= kc(r) - dlt ? w[r] : 0.f;
      }
      bf16x8 pop[2];
      {
        f32x8 a0, a1;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          a0[r] = w[r];
          a1[r] = w[r + 8];
        }
        pop[0] = __builtin_convertvector(a0, bf16x8);
        pop[1] = __builtin_convertvector(a1, bf16x8);
      }
      // V^T operands straight from the row-major V tile with transposing LDS reads: in each
      // 16-lane group, source lane j points at keys (row j / 4) and d (4 (j % 4) .. +3); lane i
      // of the group then holds d = i for 4 consecutive keys.  Two reads give the 8 keys of
      // k-slots 8 hf .. 8 hf + 7, in the key order of the Pt registers: 4 hf + {0..3} and
      // 8 + 4 hf + {0..3} within the 16-key group m.
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          bf16x4 half0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4*)((const char*)stg.v + (32 * hk + 16 * m) * 128 + (vbase[0] ^ (64u * db))));
          bf16x4 half1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4*)((const char*)stg.v + (32 * hk + 16 * m) * 128 + (vbase[1] ^ (64u * db))));
          vop[db][m] = bf16x8{half0[0], half0[1], half0[2], half0[3], half1[0], half1[1], half1[2], half1[3]};
        }
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[db][m], pop[m], oacc[db], 0, 0, 0);
    }
  };
  // tile t sits in stage t % 2; the transfers of tile t + 1 go into the stage of tile t - 1
  // (its readers all passed the last barrier) while t is multiplied, then this wave's
  // transfers are waited for and the barrier publishes them to all
  wait_vm<0>();
  lds_barrier();
  if (KIND == 1) {
    // log2(e) (max |w_pos| + max |w_time|), from the LDS tables (-log2(e) w each)
    float mp = 0.f, mt = 0.f;
    for (int i = lane; i < a.bias.num_pos; i += 64) mp = fmaxf(mp, fabsf(sm.wposx[i + 32]));
    for (int i = lane; i < a.bias.num_time; i += 64) mt = fmaxf(mt, fabsf(sm.wtime[i]));
    tabmax = uniform_f32(wave_max(mp) + wave_max(mt));
  }
  if (KIND == 2) {
    // the workgroup stops below the lowest block any wave needs (64-key tile = two blocks)
    int nb = sm.need[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) nb = min(nb, sm.need[w]);
    const int t_low = min(nb / 2, n_tiles);
    n_loop = uniform_i32(n_tiles - t_low);
  }
  auto one = [&](const Stage& c, Stage& nx, int k) __attribute__((always_inline)) {
    dma(nx, k + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(c, tix(k));
    wait_vm<0>();
    lds_barrier();
  };
  for (int k = 0; k < n_loop; k += 2) {
    one(st0, st1, k);
    if (k + 1 >= n_loop) break;
    one(st1, st0, k + 1);
  }
  // the transfers past the last tile land before the kernel ends
  wait_vm<0>();


  // ---- epilogue: O^T accumulators -> O rows, scaled by -(ln 2 / 2) out_scale ----
  const float osc = -0.5f * kLn2 * a.out_scale;
  f32x4 ov[NDB][4];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[db][g][e] = oacc[db][4 * g + e] * osc;
  const int64_t obase = ((tok0 + row) * H + h) * D;
  if (a.ostats && !OUT_F32) {
    // layer mode: each head row is stored as its fp32 mean m plus bf16 deviations from m, so
    // the rounding error scales with the row's spread, not its magnitude (a LayerNorm over the
    // heads divides by that spread); the statistics entry holds m, the mean of the
    // represented values m + dev and their sum of squared deviations (lanes l and l + 32 hold
    // the two halves)
    float sum = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) sum += ov[db][g][e];
    sum += __shfl_xor(sum, 32, 64);
    const float m = sum * (1.0f / D);
    bf16x4 dv[NDB][4];
    float ds = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        dv[db][g] = __builtin_convertvector(ov[db][g] - m, bf16x4);
        const f32x4 back = __builtin_convertvector(dv[db][g], f32x4);
        ov[db][g] = back;
        ds += back[0] + back[1] + back[2] + back[3];
      }
    ds += __shfl_xor(ds, 32, 64);
    const float md = ds * (1.0f / D);
    float q = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) q += (ov[db][g][e] - md) * (ov[db][g][e] - md);
    q += __shfl_xor(q, 32, 64);
    if (qvalid) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(bf16x4*)((bf16*)a.o + obase + 32 * db + 8 * g + 4 * hf) = dv[db][g];
      if (hf == 0) a.ostats[(tok0 + row) * H + h] = f32x4{m, m + md, q, 0.f};
    }
  } else if (qvalid) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hf;
        if (OUT_F32)
          *(f32x4*)((float*)a.o + obase + d0) = ov[db][g];
        else
          *(bf16x4*)((bf16*)a.o + obase + d0) = __builtin_convertvector(ov[db][g], bf16x4);
      }
  }
}

// ============================================================================================
// fp32, d in {32, 64}: 4 waves x 32 queries = 128 query rows per work item, 32 keys per stage,
// v_mfma_f32_32x32x2_f32 for both products.
// ============================================================================================
constexpr int kBRf = 128;
constexpr int kKBf = 32;

template <int D>
struct SmemF32 {
  float k[2][kKBf][D + 1];
  float vt[2][D][kKBf + 1];
  int64_t tk[2][kKBf];
  int64_t tkst[2][2];
  float wpos[kMaxPosBuckets];
  float wtime[kMaxTimeBuckets];
};

template <int D>
__global__ __launch_bounds__(256, 2) void attn_f32_kernel(AttnArgs a) {
  __shared__ SmemF32<D> sm;
  constexpr int NDB = D / 32;       // 32-row blocks of O^T
  constexpr int NC = D / 4;         // 16-byte chunks per row
  constexpr int NLD = (kKBf * NC) / 256;  // chunks per thread per tile
  const int item = blockIdx.x;
  if (item >= *a.work_count) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const WorkItem wi = a.work[item];
  const int h = wi.h, H = a.H;
  const int64_t tok0 = wi.tok0;
  const int n = wi.n;
  const int q0 = wi.qt * kBRf;
  if (q0 >= n) return;
  const int q_end = min(q0 + kBRf, n);
  const int n_tiles = (q_end + kKBf - 1) / kKBf;
  const int qw0 = q0 + wave * 32;
  const int wq_last = min(qw0 + 32, q_end) - 1;

  const float* __restrict__ qp = (const float*)a.q;
  const float* __restrict__ kp = (const float*)a.k;
  const float* __restrict__ vp = (const float*)a.v;
  const int kind = a.bias.kind;
  const int64_t* __restrict__ ts = a.bias.ts;
  if (kind == 1) {
    for (int i = tid; i < a.bias.num_pos; i += 256)
      sm.wpos[i] = -kLog2e * a.bias.w_pos[(int64_t)h * a.bias.pos_stride + i];
    for (int i = tid; i < a.bias.num_time; i += 256)
      sm.wtime[i] = -kLog2e * a.bias.w_time[(int64_t)h * a.bias.time_stride + i];
  }
  const int Pm1 = a.bias.num_pos - 1, NTm1 = a.bias.num_time - 1;
  float slope_y = 0.f;
  if (kind == 2) slope_y = kLog2e * (a.bias.slopes ? a.bias.slopes[h] : default_alibi_slope(h, H));

  const float cq = -a.alpha * kLog2e;
  float qop[D / 2];
  const int row_q = qw0 + l32;
  const bool qvalid = row_q <= wq_last;
#pragma unroll
  for (int ks = 0; ks < D / 2; ++ks)
    qop[ks] = qvalid ? qp[(tok0 + row_q) * a.q_stride + (int64_t)h * D + 2 * ks + hf] * cq : 0.f;
  int64_t tq = 0, tqmin = kTMax, tqmax = kTMin;
  if (kind == 1 && qvalid) {
    tq = ts[tok0 + row_q];
    tqmin = tq;
    tqmax = tq;
  }
  if (kind == 1) half_minmax(tqmin, tqmax);

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;

  f32x4 kreg[NLD], vreg[NLD];
  int64_t treg = kTMax;
  auto gload = [&](int t) {
    const int j0 = t * kKBf;
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int c = tid + 256 * u, row = c / NC, chunk = c % NC;
      const int key = j0 + row;
      kreg[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      vreg[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (key < q_end) {
        kreg[u] = *(const f32x4*)(kp + (tok0 + key) * a.k_stride + (int64_t)h * D + 4 * chunk);
        vreg[u] = *(const f32x4*)(vp + (tok0 + key) * a.v_stride + (int64_t)h * D + 4 * chunk);
      }
    }
    if (kind == 1 && tid < kKBf) {
      const int key = j0 + tid;
      treg = key < q_end ? ts[tok0 + key] : kTMax;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int c = tid + 256 * u, row = c / NC, chunk = c % NC;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sm.k[buf][row][4 * chunk + e] = kreg[u][e];
        sm.vt[buf][4 * chunk + e][row] = vreg[u][e];
      }
    }
    if (kind == 1 && tid < 64) {
      if (tid < kKBf) sm.tk[buf][tid] = treg;
      int64_t mn = treg, mx = treg == kTMax ? kTMin : treg;
      half_minmax(mn, mx);
      if (lane == 0) {
        sm.tkst[buf][0] = mn;
        sm.tkst[buf][1] = mx;
      }
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) gload(t + 1);
    const int j0 = t * kKBf;
    if (j0 <= wq_last && qw0 <= wq_last) {  // before the diagonal, and the wave has rows
      const int base = qw0 - j0 + l32;
      f32x16 c;
      if (kind == 1) {
        const bool pconst = (qw0 - (j0 + 31)) >= Pm1;
        const int tb_lo = time_bucket(tqmin - sm.tkst[buf][1], NTm1);
        const int tb_hi = time_bucket(tqmax - sm.tkst[buf][0], NTm1);
        if (pconst && tb_lo == tb_hi) {
          const float cb = sm.wpos[Pm1] + sm.wtime[tb_lo];
#pragma unroll
          for (int r = 0; r < 16; ++r) c[r] = cb;
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kr = acc_key(r, hf);
            c[r] = sm.wpos[pos_bucket(base - kr, Pm1)] + sm.wtime[time_bucket(tq - sm.tk[buf][kr], NTm1)];
          }
        }
      } else if (kind == 2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) c[r] = slope_y * (float)(base - acc_key(r, hf));
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) c[r] = 0.f;
      }
      f32x16 s = c;
#pragma unroll
      for (int ks = 0; ks < D / 2; ++ks)
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(sm.k[buf][l32][2 * ks + hf], qop[ks], s, 0, 0, 0);
      const bool diag = (j0 + 31) > qw0;
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float y = s[r];
        const float e = __builtin_amdgcn_exp2f(y);
        float av = y * __builtin_amdgcn_rcpf(1.0f + e);
        if (diag && (base - acc_key(r, hf)) < 0) av = 0.f;
        p[r] = av;
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int m = 0; m < 16; ++m)
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(sm.vt[buf][32 * db + l32][acc_key(m, hf)], p[m], oacc[db], 0, 0, 0);
    }
    if (t + 1 < n_tiles) lstore(buf ^ 1);
    __syncthreads();
  }

  if (qvalid) {
    const float osc = -kLn2 * a.out_scale;
    float* dst = (float*)a.o + ((tok0 + row_q) * H + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v4 = {oacc[db][4 * g] * osc, oacc[db][4 * g + 1] * osc, oacc[db][4 * g + 2] * osc,
                    oacc[db][4 * g + 3] * osc};
        *(f32x4*)(dst + 32 * db + 8 * g + 4 * hf) = v4;
      }
  }
}

}  // namespace

int attn_block_rows_bf16(int d) { return (d == 32 || d == 64) ? kBR : 0; }
int attn_block_rows_f32(int d) { return (d == 32 || d == 64) ? kBRf : 0; }

hipError_t launch_time_stats(int32_t B, const int32_t* offsets, const int64_t* ts,
                             int32_t max_seqlen, TimeStat* stats, int32_t* rel,
                             hipStream_t stream) {
  if (B <= 0 || max_seqlen <= 0) return hipSuccess;
  hipLaunchKernelGGL(time_stats_kernel, dim3(B, (max_seqlen + 255) / 256), dim3(256), 0, stream,
                     offsets, ts, stats, rel);
  return hipGetLastError();
}

hipError_t launch_key_norm(int32_t B, const int32_t* offsets, int64_t total_tokens,
                           const void* k, int64_t k_stride, int32_t H, int32_t d, float* knorm,
                           const int64_t* ts, TimeStat* stats, int32_t* rel, hipStream_t stream) {
  if (B <= 0 || total_tokens <= 0) return hipSuccess;
  const int64_t rows = (total_tokens + 31 * (int64_t)B) / 32 + 1;
  if (rows > 0x7fffffff) return hipErrorInvalidValue;
  if (d == 64)
    hipLaunchKernelGGL(key_norm_kernel<64>, dim3((unsigned)rows), dim3(64 * kNormWaves), 0, stream, offsets,
                       B, (const bf16*)k, k_stride, H, knorm, ts, stats, rel);
  else if (d == 32)
    hipLaunchKernelGGL(key_norm_kernel<32>, dim3((unsigned)rows), dim3(64 * kNormWaves), 0, stream, offsets,
                       B, (const bf16*)k, k_stride, H, knorm, ts, stats, rel);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_tile_class(int32_t B, const int32_t* offsets, const TimeStat* stats,
                             int32_t max_blocks, int32_t num_pos, int32_t num_time,
                             uint32_t* tclass, hipStream_t stream) {
  if (B <= 0 || max_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(tile_class_kernel, dim3(B, max_blocks), dim3(256), 0, stream, offsets, stats,
                     max_blocks, num_pos, num_time, tclass);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(int d, const AttnArgs& a, int grid, hipStream_t stream) {
  if (d != 32 && d != 64) return hipErrorInvalidValue;
  if (a.ostats && d != 64) return hipErrorInvalidValue;  // the layer's O layout is for d = 64
  if (grid <= 0) return hipSuccess;
  const dim3 g(grid), blk(kThreads);
#define HSTU_ATTN_BF16(K, F)                                                                  \
  if (d == 64) hipLaunchKernelGGL((attn_bf16_kernel<K, F, 64>), g, blk, 0, stream, a);        \
  else hipLaunchKernelGGL((attn_bf16_kernel<K, F, 32>), g, blk, 0, stream, a);                \
  break;
  switch (a.bias.kind * 2 + (a.o_f32 ? 1 : 0)) {
    case 0: HSTU_ATTN_BF16(0, false)
    case 1: HSTU_ATTN_BF16(0, true)
    case 2: HSTU_ATTN_BF16(1, false)
    case 3: HSTU_ATTN_BF16(1, true)
    case 4: HSTU_ATTN_BF16(2, false)
    case 5: HSTU_ATTN_BF16(2, true)
    default: return hipErrorInvalidValue;
  }
#undef HSTU_ATTN_BF16
  return hipGetLastError();
}

hipError_t launch_attn_f32(int d, const AttnArgs& a, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (d == 32) hipLaunchKernelGGL(attn_f32_kernel<32>, dim3(grid), dim3(256), 0, stream, a);
  else if (d == 64) hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(grid), dim3(256), 0, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace hstu
