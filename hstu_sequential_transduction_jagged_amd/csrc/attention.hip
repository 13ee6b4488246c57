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
// B operand of the next MFMA, O^T += V^T P^T, so the probabilities never leave
// registers.  The key order inside a 16-key PV step is a fixed permutation of
// the accumulator's row order, and V^T is stored in LDS in that permuted order.
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

// MFMA k slot of key k16 (0..15) within a 16-key PV step (inverse of the
// accumulator row order restricted to registers 8m..8m+7).
__device__ __forceinline__ int pv_slot(int k16) {
  int g = k16 >> 3, w = k16 & 7;
  return 8 * (w >> 2) + 4 * g + (w & 3);
}

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
__device__ __forceinline__ float uniform_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(uint32_t, v)));
}

// w(y) = y - y^2 (P0 + P1 y^2 + P2 y^4) on |y| <= kPolyRange (near-minimax fit of the
// relative error of 1/(1+2^y); the fitting script sits beside this file).
constexpr float kPolyRange = 2.0f;
constexpr float kP0 = 0.3463683490f, kP1 = -0.0135027335f, kP2 = 0.0004785898f;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

constexpr int64_t kTMax = 0x7fffffffffffffffLL;
constexpr int64_t kTMin = -kTMax - 1;

// ============================================================================================
// Timestamp statistics: for every 32-token block of a user (blocks start at the user's first
// token), the min and max timestamp, stored at the block's first token; and for every token
// its offset from its block's minimum as int32 (saturated; only read where the block spans
// at most 2^30).  One workgroup per user.
// ============================================================================================
__global__ __launch_bounds__(256) void time_stats_kernel(const int32_t* __restrict__ offsets,
                                                        const int64_t* __restrict__ ts,
                                                        TimeStat* __restrict__ stats,
                                                        int32_t* __restrict__ rel) {
  const int b = blockIdx.x;
  const int64_t s = offsets[b];
  const int n = offsets[b + 1] - offsets[b];
  const int lane = threadIdx.x & 63, l32 = lane & 31;
  for (int j = threadIdx.x; j < ((n + 63) & ~63); j += 256) {
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
// bf16, d = 64: 4 waves x 64 queries = 256 query rows per work item, 64 keys per LDS stage.
// ============================================================================================
constexpr int kWaves = 4;
constexpr int kQW = 64;
constexpr int kBR = kWaves * kQW;
constexpr int kKB = 64;
constexpr int kD = 64;

struct __attribute__((aligned(16))) SmemBf16 {
  __attribute__((aligned(16))) bf16 k[2][kKB * kD];   // row = key, 8 chunks of 16 B, chunk c stored at c ^ ((row / 2) & 7)
  __attribute__((aligned(16))) bf16 vt[2][kD * kKB];  // row = d, 64 keys in PV slot order, chunk c at c ^ ((d + d/8) & 7)
  __attribute__((aligned(16))) int32_t krel[2][kKB];  // key timestamp minus its 32-key block's minimum (0 past the end)
  float knorm2[2][kWaves];      // per wave: max squared norm of the key rows it staged
  float wpos[kMaxPosBuckets];   // -log2(e) * w_pos[h]
  float wtime[kMaxTimeBuckets]; // -log2(e) * w_time[h]
  float wtime_lz[32];           // wtime[min(31 - lz, NT - 1)]: time bias by leading zeros of dt + 1
  float cbuf[kWaves][16][64];   // per-wave bias staging of the 64-bit timestamp path
};

// LDS has 64 four-byte banks and serves 16 lanes of a 16-byte read per cycle: 16 lanes
// reading the same chunk of 16 consecutive 128-byte rows hit distinct banks when the chunk
// is XOR-ed with (row / 2) & 7 (row parity selects the bank half).
__device__ __forceinline__ int k_off(int row, int chunk) { return row * kD + ((chunk ^ ((row >> 1) & 7)) << 3); }
__device__ __forceinline__ int vt_off(int d, int chunk) { return d * kKB + ((chunk ^ ((d + (d >> 3)) & 7)) << 3); }

template <bool OUT_F32>
__global__ __launch_bounds__(256, 2) void attn_bf16_d64_kernel(AttnArgs a) {
  __shared__ SmemBf16 sm;
  const int item = blockIdx.x;
  if (item >= *a.work_count) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31, hf = lane >> 5;
  const WorkItem wi = a.work[item];
  const int b = wi.b, h = wi.h, H = a.H;
  const int64_t tok0 = a.offsets[b];
  const int n = a.offsets[b + 1] - a.offsets[b];
  const int q0 = wi.qt * kBR;
  if (q0 >= n) return;
  const int q_end = min(q0 + kBR, n);
  const int n_tiles = (q_end + kKB - 1) / kKB;
  const int qw0 = q0 + wave * kQW;
  const int wq_last = min(qw0 + kQW, q_end) - 1;  // < qw0 when the wave has no rows

  const bf16* __restrict__ qp = (const bf16*)a.q;
  const bf16* __restrict__ kp = (const bf16*)a.k;
  const bf16* __restrict__ vp = (const bf16*)a.v;
  const int kind = a.bias.kind;
  const int64_t* __restrict__ ts = a.bias.ts;
  const TimeStat* __restrict__ tstat = a.tstat;

  if (kind == 1) {
    for (int i = tid; i < a.bias.num_pos; i += 256)
      sm.wpos[i] = -kLog2e * a.bias.w_pos[(int64_t)h * a.bias.pos_stride + i];
    for (int i = tid; i < a.bias.num_time; i += 256)
      sm.wtime[i] = -kLog2e * a.bias.w_time[(int64_t)h * a.bias.time_stride + i];
    if (tid < 32) {
      const int tb = min(31 - tid, a.bias.num_time - 1);
      sm.wtime_lz[tid] = -kLog2e * a.bias.w_time[(int64_t)h * a.bias.time_stride + tb];
    }
  }
  const int Pm1 = a.bias.num_pos - 1, NTm1 = a.bias.num_time - 1;
  float slope_y = 0.f;
  if (kind == 2) slope_y = kLog2e * (a.bias.slopes ? a.bias.slopes[h] : default_alibi_slope(h, H));

  // ---- Q fragments (B operand of S^T = K Q^T), unscaled; query timestamps ----
  const float cq = -a.alpha * kLog2e;
  bf16x8 qop[2][4];
  int64_t tq[2];
  int64_t tqmin[2] = {0, 0}, tqmax[2] = {0, 0};
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qb0 = qw0 + 32 * qb;
    const int row = qb0 + l32;
    const bool valid = row <= wq_last;
    const bf16* src = qp + (tok0 + row) * a.q_stride + (int64_t)h * kD + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (valid) raw = *(const u32x4*)(src + 16 * ks);
      qop[qb][ks] = __builtin_bit_cast(bf16x8, raw);
    }
    tq[qb] = 0;
    if (kind == 1 && qb0 <= wq_last) {
      const TimeStat st = tstat[tok0 + qb0];
      tqmin[qb] = st.mn;
      tqmax[qb] = st.mx;
      tq[qb] = valid ? ts[tok0 + row] : st.mn;
    }
  }

  // max norm of the query rows of each 32-row block (bound of the polynomial SiLU path)
  float qnorm[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2 pr = {qop[qb][ks][2 * e], qop[qb][ks][2 * e + 1]};
        ss = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, ss, false);
      }
    }
    ss += __shfl_xor(ss, 32, 64);  // the two lane halves hold the two halves of a row
    qnorm[qb] = uniform_f32(sqrtf(wave_max(ss)));
  }
  // largest |bias| the tables can produce (y units)
  float tabmax = 0.f;
  if (kind == 1) {
    float mp = 0.f, mt = 0.f;
    for (int i = lane; i < a.bias.num_pos; i += 64)
      mp = fmaxf(mp, fabsf(a.bias.w_pos[(int64_t)h * a.bias.pos_stride + i]));
    for (int i = lane; i < a.bias.num_time; i += 64)
      mt = fmaxf(mt, fabsf(a.bias.w_time[(int64_t)h * a.bias.time_stride + i]));
    tabmax = uniform_f32(kLog2e * (wave_max(mp) + wave_max(mt)));
  }
  const float acq = fabsf(cq) * 1.0001f;  // rounding margin of the bound

  f32x16 oacc[2][2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][qb][r] = 0.f;

  // ---- staging: global -> registers -> LDS ----
  const int krow0 = tid >> 3, kchunk = tid & 7;       // K rows krow0 and krow0 + 32
  const int vpair = tid >> 3, vch = tid & 7;          // V keys 2 vpair, 2 vpair + 1; d chunk vch
  const bf16* kbase = kp + (tok0 + krow0) * a.k_stride + (int64_t)h * kD + 8 * kchunk;
  const bf16* vbase = vp + (tok0 + 2 * vpair) * a.v_stride + (int64_t)h * kD + 8 * vch;
  // V^T store: element e of the chunk (d = 8 vch + e) goes to row d at key slot vpos; the
  // swizzled 16-byte chunk index of row d is (vpos / 8) ^ ((e + vch) & 7)
  const int vpos = 16 * ((2 * vpair) >> 4) + pv_slot((2 * vpair) & 15);
  uint32_t vsw = 0;  // 8 nibbles: swizzled chunk for e = 0..7
#pragma unroll
  for (int e = 0; e < 8; ++e) vsw |= (uint32_t)(((vpos >> 3) ^ ((e + vch) & 7)) & 7) << (4 * e);
  const int vdst0 = 8 * vch * kKB + (vpos & 7);
  u32x4 kreg[2], vreg[2];
  i32x4 rreg = {0, 0, 0, 0};
  auto gload = [&](int t) {
    const int j0 = t * kKB;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int key = j0 + krow0 + 32 * u;
      kreg[u] = u32x4{0u, 0u, 0u, 0u};
      if (key < q_end) kreg[u] = *(const u32x4*)(kbase + (int64_t)(j0 + 32 * u) * a.k_stride);
      const int vkey = j0 + 2 * vpair + u;
      vreg[u] = u32x4{0u, 0u, 0u, 0u};
      if (vkey < q_end) vreg[u] = *(const u32x4*)(vbase + (int64_t)(j0 + u) * a.v_stride);
    }
    if (kind == 1 && tid < kKB / 4) {
      const int key = j0 + 4 * tid;
      rreg = i32x4{0, 0, 0, 0};
      if (key + 3 < q_end) {
        rreg = *(const i32x4*)(a.trel + tok0 + key);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (key + e < q_end) rreg[e] = a.trel[tok0 + key + e];
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      *(u32x4*)(&sm.k[buf][k_off(krow0 + 32 * u, kchunk)]) = kreg[u];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // element e of both key rows: low (e even) or high (e odd) half of word e / 2
      const uint32_t wa = vreg[0][e >> 1], wb = vreg[1][e >> 1];
      const uint32_t pk = __builtin_amdgcn_perm(wb, wa, (e & 1) ? 0x07060302u : 0x05040100u);
      const int chunk = (vsw >> (4 * e)) & 7;
      *(uint32_t*)(&sm.vt[buf][vdst0 + e * kKB + (chunk << 3)]) = pk;
    }
    if (kind == 1 && tid < kKB / 4) *(i32x4*)(&sm.krel[buf][4 * tid]) = rreg;
    // max squared norm of the staged key rows: 8 threads hold the 8 chunks of a row
    float ss[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bf16x8 kv = __builtin_bit_cast(bf16x8, kreg[u]);
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2 pr = {kv[2 * e], kv[2 * e + 1]};
        acc = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, acc, false);
      }
      acc += __shfl_xor(acc, 1, 64);
      acc += __shfl_xor(acc, 2, 64);
      acc += __shfl_xor(acc, 4, 64);
      ss[u] = acc;
    }
    float mx = fmaxf(ss[0], ss[1]);
    mx = fmaxf(mx, __shfl_xor(mx, 8, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (lane == 0) sm.knorm2[buf][wave] = mx;
  };

  gload(0);
  lstore(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) gload(t + 1);
    const int j0 = t * kKB;
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
      const int j0h = j0 + 32 * hk;
      if (j0h > wq_last) continue;
      // K operands of this 32-key step (V operands are read after the SiLU)
      bf16x8 kop[4], vop[2][2];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kop[ks] = *(const bf16x8*)(&sm.k[buf][k_off(32 * hk + l32, hf + 2 * ks)]);

      // ---- classification of the two 32x32 sub-tiles, all in scalar registers ----
      // mode 0: inactive, 1: scalar bias, 2: two time buckets (one compare per element),
      // 3: per-element bias (gather on 32-bit time offsets, ALiBi, or none with the mask),
      // 4: per-element gather on 64-bit times
      int mode[2], thi2[2];
      float cb[2], chi[2];
      bool diag[2], poly[2];
      float kn2 = fmaxf(fmaxf(sm.knorm2[buf][0], sm.knorm2[buf][1]),
                        fmaxf(sm.knorm2[buf][2], sm.knorm2[buf][3]));
      const float knorm = uniform_f32(sqrtf(kn2));
      int64_t kmn = 0, kmx = 0;
      if (kind == 1) {
        const TimeStat ks = tstat[tok0 + j0h];
        kmn = ks.mn;
        kmx = ks.mx;
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int qb0 = qw0 + 32 * qb;
        const bool act = (qb0 <= wq_last) && (j0h <= min(qb0 + 31, wq_last));
        const bool dg = (j0h + 31) > qb0;
        int md = 3, th = 0;
        float c0 = 0.f, c1 = 0.f;
        if (kind == 0) {
          md = dg ? 3 : 1;
        } else if (kind == 1) {
          const bool pconst = (qb0 - (j0h + 31)) >= Pm1;  // implies !dg
          const int tlo = time_bucket(tqmin[qb] - kmx, NTm1);
          const int thi = time_bucket(tqmax[qb] - kmn, NTm1);
          const int64_t lim30 = 1LL << 30;
          const bool fits32 = (kmx - kmn) <= lim30 && (tqmax[qb] - kmn) <= lim30 &&
                              (tqmin[qb] - kmn) >= -lim30;
          c0 = sm.wpos[Pm1] + sm.wtime[tlo];
          c1 = sm.wpos[Pm1] + sm.wtime[thi];
          th = thi;
          md = (pconst && tlo == thi) ? 1 : (pconst && thi == tlo + 1 && fits32) ? 2 : fits32 ? 3 : 4;
        }
        mode[qb] = act ? md : 0;
        thi2[qb] = th;
        diag[qb] = dg;
        cb[qb] = uniform_f32(c0);
        chi[qb] = uniform_f32(c1);
        // largest |bias_y| in the sub-tile, then the bound on |y|
        float cabs = 0.f;
        if (kind == 1) cabs = md == 1 ? fabsf(cb[qb]) : md == 2 ? fmaxf(fabsf(cb[qb]), fabsf(chi[qb])) : tabmax;
        if (kind == 2) cabs = fabsf(slope_y) * (float)max(qb0 + 31 - j0h, 0);
        poly[qb] = acq * qnorm[qb] * knorm + cabs <= kPolyRange;
      }

      auto qk = [&](int qb) {
        f32x16 sacc = {};
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[0], qop[qb][0], sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[1], qop[qb][1], sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[2], qop[qb][2], sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[3], qop[qb][3], sacc, 0, 0, 0);
        return sacc;
      };
      // y = -log2(e) (alpha s + bias); w(y) = 2 y / (1 + 2^y) = -(2 / ln 2) SiLU(alpha s + bias)
      auto w_exact = [&](float y) {
        return y * __builtin_amdgcn_rcpf(__builtin_fmaf(__builtin_amdgcn_exp2f(y), 0.5f, 0.5f));
      };
      auto w_poly = [&](float y) {
        const float u = y * y;
        return __builtin_fmaf(-u, __builtin_fmaf(__builtin_fmaf(kP2, u, kP1), u, kP0), y);
      };
      auto silu_scalar = [&](const f32x16& sacc, float c, bool pl, bf16x8& p0, bf16x8& p1) {
        f32x8 a0, a1;
        if (pl) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float av = w_poly(__builtin_fmaf(sacc[r], cq, c));
            if (r < 8) a0[r] = av; else a1[r - 8] = av;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float av = w_exact(__builtin_fmaf(sacc[r], cq, c));
            if (r < 8) a0[r] = av; else a1[r - 8] = av;
          }
        }
        p0 = __builtin_convertvector(a0, bf16x8);
        p1 = __builtin_convertvector(a1, bf16x8);
      };
      auto silu_vector = [&](const f32x16& sacc, const f32x16& c, bool mask, bool pl, int base,
                             bf16x8& p0, bf16x8& p1) {
        f32x8 a0, a1;
        if (pl) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float av = w_poly(__builtin_fmaf(sacc[r], cq, c[r]));
            if (r < 8) a0[r] = av; else a1[r - 8] = av;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float av = w_exact(__builtin_fmaf(sacc[r], cq, c[r]));
            if (r < 8) a0[r] = av; else a1[r - 8] = av;
          }
        }
        if (mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool keep = (base - acc_key(r, hf)) >= 0;
            if (r < 8) a0[r] = keep ? a0[r] : 0.f; else a1[r - 8] = keep ? a1[r - 8] : 0.f;
          }
        }
        p0 = __builtin_convertvector(a0, bf16x8);
        p1 = __builtin_convertvector(a1, bf16x8);
      };
      // per-element bias (y units) of sub-tile qb
      auto bias_vector = [&](int qb, int m, int base) {
        f32x16 c;
        if (kind == 2) {
#pragma unroll
          for (int r = 0; r < 16; ++r) c[r] = slope_y * (float)(base - acc_key(r, hf));
        } else if (kind == 0) {
#pragma unroll
          for (int r = 0; r < 16; ++r) c[r] = 0.f;
        } else if (m == 2 || m == 3) {
          i32x4 rel4[4];
#pragma unroll
          for (int g = 0; g < 4; ++g) rel4[g] = *(const i32x4*)(&sm.krel[buf][32 * hk + 8 * g + 4 * hf]);
          if (m == 2) {
            // two time buckets: dt >= 2^thi - 1  <=>  rel_j <= (t_i - kmin) - (2^thi - 1)
            const int64_t lim64 = (tq[qb] - kmn) - ((1LL << thi2[qb]) - 1);
            const int lim = lim64 < -1 ? -1 : (lim64 > 0x7fffffffLL ? 0x7fffffff : (int)lim64);
#pragma unroll
            for (int r = 0; r < 16; ++r) c[r] = rel4[r >> 2][r & 3] <= lim ? chi[qb] : cb[qb];
          } else {
            const int ti1 = (int)(tq[qb] - kmn) + 1;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int u = max(ti1 - rel4[r >> 2][r & 3], 1);  // max(dt, 0) + 1
              const int pb = min(max(base - acc_key(r, hf), 0), Pm1);
              c[r] = sm.wpos[pb] + sm.wtime_lz[__builtin_clz((uint32_t)u)];
            }
          }
        } else {
          // timestamps spread beyond 2^30 within the sub-tile: exact 64-bit deltas, one
          // element at a time through LDS to keep register use flat
#pragma unroll 1
          for (int r = 0; r < 16; ++r) {
            const int kr = acc_key(r, hf);
            const int key = min(j0h + kr, n - 1);
            sm.cbuf[wave][r][lane] = sm.wpos[pos_bucket(base - kr, Pm1)] +
                                     sm.wtime[time_bucket(tq[qb] - ts[tok0 + key], NTm1)];
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) c[r] = sm.cbuf[wave][r][lane];
        }
        return c;
      };

      bf16x8 pop[2][2] = {{bf16x8{}, bf16x8{}}, {bf16x8{}, bf16x8{}}};
      if (mode[0] == 1 && mode[1] == 1) {
        const f32x16 s0 = qk(0);
        const f32x16 s1 = qk(1);
        silu_scalar(s0, cb[0], poly[0], pop[0][0], pop[0][1]);
        silu_scalar(s1, cb[1], poly[1], pop[1][0], pop[1][1]);
      } else {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          if (mode[qb] == 0) continue;
          const int qb0 = qw0 + 32 * qb;
          if (mode[qb] == 1) {
            const f32x16 sacc = qk(qb);
            silu_scalar(sacc, cb[qb], poly[qb], pop[qb][0], pop[qb][1]);
          } else {
            // bias first, then the scores: fewer registers live at once
            const int base = qb0 - j0h + l32;  // i - j = base - acc_key(r, hf)
            const f32x16 c = bias_vector(qb, mode[qb], base);
            const f32x16 sacc = qk(qb);
            silu_vector(sacc, c, diag[qb], poly[qb], base, pop[qb][0], pop[qb][1]);
          }
        }
      }
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int m = 0; m < 2; ++m)
          vop[db][m] = *(const bf16x8*)(&sm.vt[buf][vt_off(32 * db + l32, 4 * hk + 2 * m + hf)]);
      // an inactive sub-tile has P = 0 and adds nothing; issuing its MFMAs anyway keeps the
      // accumulators out of branches (they are rare: diagonal and tail steps only)
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            oacc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[db][m], pop[qb][m], oacc[db][qb], 0, 0, 0);
    }
    if (t + 1 < n_tiles) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O^T accumulators -> O rows, scaled by -(ln 2 / 2) out_scale ----
  const float osc = -0.5f * kLn2 * a.out_scale;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qw0 + 32 * qb + l32;
    if (row > wq_last) continue;
    const int64_t base = ((tok0 + row) * H + h) * kD;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v4 = {oacc[db][qb][4 * g] * osc, oacc[db][qb][4 * g + 1] * osc,
                    oacc[db][qb][4 * g + 2] * osc, oacc[db][qb][4 * g + 3] * osc};
        const int d0 = 32 * db + 8 * g + 4 * hf;
        if (OUT_F32)
          *(f32x4*)((float*)a.o + base + d0) = v4;
        else
          *(bf16x4*)((bf16*)a.o + base + d0) = __builtin_convertvector(v4, bf16x4);
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
  const int b = wi.b, h = wi.h, H = a.H;
  const int64_t tok0 = a.offsets[b];
  const int n = a.offsets[b + 1] - a.offsets[b];
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
    if (j0 <= wq_last) {
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

int attn_block_rows_bf16(int d) { return d == 64 ? kBR : 0; }
int attn_block_rows_f32(int d) { return (d == 32 || d == 64) ? kBRf : 0; }

hipError_t launch_time_stats(int32_t B, const int32_t* offsets, const int64_t* ts, TimeStat* stats,
                             int32_t* rel, hipStream_t stream) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(time_stats_kernel, dim3(B), dim3(256), 0, stream, offsets, ts, stats, rel);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(int d, const AttnArgs& a, int grid, hipStream_t stream) {
  if (d != 64) return hipErrorInvalidValue;
  if (grid <= 0) return hipSuccess;
  if (a.o_f32)
    hipLaunchKernelGGL(attn_bf16_d64_kernel<true>, dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_bf16_d64_kernel<false>, dim3(grid), dim3(256), 0, stream, a);
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
