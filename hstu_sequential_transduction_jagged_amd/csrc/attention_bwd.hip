// Gradients of the jagged causal pointwise attention ("Actions Speak Louder than Words" reading
// notes §3.1 eq. (2), §3.2) for bf16, d_qk = d_v = 64:
//
//   x_ij = alpha <q_i, k_j> + rab(i, j),  a_ij = SiLU(x_ij),  O_i = out_scale sum_{j <= i} a_ij v_j
//   dV_j = out_scale sum_{i >= j} a_ij dO_i
//   g_ij = <dO_i, v_j> SiLU'(x_ij),  SiLU'(x) = s (1 + x (1 - s)),  s = 1 / (1 + e^-x)
//   dQ_i = alpha out_scale sum_{j <= i} g_ij k_j,   dK_j = alpha out_scale sum_{i >= j} g_ij q_i
//   dw_pos[h][pos bucket] += out_scale g_ij,  dw_time[h][time bucket] += out_scale g_ij
//
// Two kernels over the forward's cost-sorted work list of (user, head, 256-row tile) items:
//   - attn_bwd_dq_kernel, query-major like the forward: per wave 32 query rows; per 32-key step
//     S^T = K Q^T and dA^T = V dO^T on v_mfma_f32_32x32x16_bf16 (lane = query, registers = keys),
//     the weights g in registers become the B operand of dQ^T += K^T G^T, K^T read from the
//     row-major K tile with transposing LDS reads (as V^T in the forward);
//   - attn_bwd_dkv_kernel, key-major: per wave 32 key rows held in registers; per 32-query step
//     S = Q K^T and dA = dO V^T (lane = key, registers = queries), then dV^T += dO^T P and
//     dK^T += Q^T G with dO^T and Q^T read from the row-major query tiles with transposing LDS
//     reads; the table gradients are summed per workgroup in LDS and added to the tables with
//     one global atomic per entry touched (so their summation order varies between runs).
// Per 32x32 tile with one bias value (no bias, or saturated position bucket and one time
// bucket, decided exactly from the tile's extreme times) and |alpha s| <= kTaylorD, SiLU and
// SiLU' come from second-order expansions in the raw score (four fmas per score); elsewhere they
// are evaluated exactly (exp2 and reciprocal) with the bias of every element from LDS tables.
#include "hstu_internal.h"

namespace hstu {
namespace {

constexpr int kBWaves = 4;
constexpr int kBThreads = 64 * kBWaves;
constexpr int kBRows = 32 * kBWaves;  // rows of a work item (the forward's tile height)
constexpr int kBTile = 64;            // keys (dq kernel) or queries (dkv kernel) per LDS tile
constexpr int kBD = 64;
constexpr int kBRow = 72;             // dq kernel: padded LDS row (bf16, 144 bytes)

// accumulator register r of a 32x32 MFMA tile holds row 8 (r / 4) + 4 hf + r % 4
__device__ __forceinline__ int accrow(int r) { return 8 * (r >> 2) + (r & 3); }

struct __attribute__((aligned(16))) BwdTables {
  float wpos[kMaxPosBuckets];    // w_pos[h]
  float wtime[kMaxTimeBuckets];  // w_time[h]
  float gpos[kMaxPosBuckets];    // dkv kernel: this workgroup's position-table gradient
  float gtime[kMaxTimeBuckets];  // dkv kernel: this workgroup's time-table gradient
  // per time bucket, for tiles whose position bucket saturates: the bias c and the Taylor
  // coefficients of SiLU and SiLU' in the raw score (see silu_taylor)
  __attribute__((aligned(16))) float tay[kMaxTimeBuckets][8];
};
// dq kernel: the tables and a double-buffered K / V tile with its rows' timestamps
struct __attribute__((aligned(16))) SmemBwd : BwdTables {
  __attribute__((aligned(16))) bf16 x[2][kBTile * kBRow];  // K rows
  __attribute__((aligned(16))) bf16 y[2][kBTile * kBRow];  // V rows
  __attribute__((aligned(16))) int64_t t[2][kBTile];       // the tile rows' timestamps
  __attribute__((aligned(16))) int64_t tmm[2][2][2];  // per 32-row half of a tile: min, max time
};

// dK/dV kernel ring stage: a 64-row tile of Q and of dO (128-byte rows, 16-byte chunk c of row
// r at position c ^ bswz(r): the operand reads, the transposing reads and the transfers meet the
// 64 banks without conflicts), the rows' timestamps and the two 32-row halves' min / max times.
// A 4-byte transfer fills 256 bytes, hence the sizes of tmm and dummy.
struct __attribute__((aligned(16))) BStage {
  __attribute__((aligned(16))) bf16 x[kBTile * kBD];
  __attribute__((aligned(16))) bf16 y[kBTile * kBD];
  __attribute__((aligned(16))) bf16 z[kBTile * kBD];  // dkv kernel: dO's bf16 remainder, if given
  __attribute__((aligned(16))) int64_t t[kBTile];
  __attribute__((aligned(16))) int64_t tmm[32];     // [0..3]: min, max of half 0, then half 1
  __attribute__((aligned(16))) uint32_t dummy[64];  // target of the transfers that carry nothing
};
__device__ __forceinline__ int bswz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

// Second-order expansions in the raw score s around the bias c (x = c + alpha s):
//   SiLU(x)  ~ A0 + A1 s + A2 s^2,   SiLU'(x) ~ B0 + B1 s + B2 s^2
// with SiLU' = sg + c p, SiLU^(2) = 2 p + c p (1 - 2 sg), SiLU^(3) = 3 p (1 - 2 sg)
// + c (p (1 - 2 sg)^2 - 2 p^2), sg = 1 / (1 + e^-c), p = sg (1 - sg); sg and 1 - sg from
// e^-|c| (no overflow).  Used when |alpha s| <= kTaylorD over the tile: the remainders are at
// most max|SiLU^(3)| kTaylorD^3 / 6 <= 3.3e-6 and max|SiLU^(4)| kTaylorD^3 / 6 <= 5.4e-6
// (max|SiLU^(3)| = 0.31, max|SiLU^(4)| = 0.5), relative to the value at most ~1e-4 (the linear
// term is exact where SiLU vanishes).
__device__ __forceinline__ void silu_taylor(float c, float al, float* o) {
  const float e = exp2f(-kLog2e * fabsf(c));
  const float inv = 1.0f / (1.0f + e);
  const float sg = c >= 0.f ? inv : e * inv;
  const float om = c >= 0.f ? e * inv : inv;  // 1 - sg
  const float p = sg * om, d = om - sg;
  const float f0 = c * sg, f1 = sg + c * p, f2 = 2.0f * p + c * p * d;
  const float f3 = 3.0f * p * d + c * (p * d * d - 2.0f * p * p);
  o[0] = c;
  o[1] = f0;
  o[2] = al * f1;
  o[3] = 0.5f * al * al * f2;
  o[4] = f1;
  o[5] = al * f2;
  o[6] = 0.5f * al * al * f3;
  o[7] = 0.f;
}

// max over the wave of |x[r]|, as a wave-uniform value
__device__ __forceinline__ float wave_max_abs16(const f32x16& x) {
  float m = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(x[r]));
  m = fmaxf(m, dpp<kDppXor1>(m));
  m = fmaxf(m, dpp<kDppXor2>(m));
  m = fmaxf(m, dpp<kDppHalfMirror>(m));
  m = fmaxf(m, dpp<kDppMirror>(m));
  auto at = [&](int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m), l)); };
  return fmaxf(fmaxf(at(0), at(16)), fmaxf(at(32), at(48)));
}

// sum over the 64 lanes of a wave, as a wave-uniform value
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  auto at = [&](int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l)); };
  return (at(0) + at(16)) + (at(32) + at(48));
}

// s = 1 / (1 + e^-x) and SiLU'(x) = s (1 + x (1 - s)); a = x s
__device__ __forceinline__ void silu_and_grad(float x, float& a, float& d1) {
  const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * x));
  a = x * s;
  d1 = s * __builtin_fmaf(x, 1.0f - s, 1.0f);
}

typedef long long i64x2 __attribute__((ext_vector_type(2)));

// bias of pair (i, j) of head h (natural units), from the LDS tables
template <int KIND>
__device__ __forceinline__ float pair_bias(const BwdTables& sm, int di, int64_t dt, int Pm1,
                                           int NTm1, float slope) {
  if (KIND == 1) return sm.wpos[max(min(di, Pm1), 0)] + sm.wtime[time_bucket(dt, NTm1)];
  if (KIND == 2) return -slope * (float)di;
  return 0.f;
}

// stage one 64-row tile of two row-major [T, H, 64] bf16 tensors (rows r0 .. r0 + 63 of user
// base tok0, head h; rows at or past `end` read as zeros) and the rows' timestamps
struct TileStager {
  __amdgpu_buffer_rsrc_t xr, yr, tr;
  uint32_t xs, ys, xoff, yoff;
  u32x4 xreg[2], yreg[2];
  uint32_t tlo = 0, thi = 0;
  __device__ void load(int r0, bool with_t, int lane) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      xreg[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, xoff + 32u * u * xs, (uint32_t)r0 * xs, 0));
      yreg[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(yr, yoff + 32u * u * ys, (uint32_t)r0 * ys, 0));
    }
    if (with_t) {
      const u32x2 tt = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(tr, 8u * (uint32_t)lane, 8u * (uint32_t)r0, 0));
      tlo = tt[0];
      thi = tt[1];
    }
  }
};

template <int KIND>
__global__ __launch_bounds__(kBThreads, 2) void attn_bwd_dq_kernel(BwdArgs a) {
  __shared__ SmemBwd sm;
  const int item = blockIdx.x;
  if (item >= *a.work_count) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const WorkItem wi = a.work[item];
  const int h = wi.h, H = a.H;
  const int64_t tok0 = wi.tok0;
  const int n = wi.n;
  const int q0 = wi.qt * kBRows;
  if (q0 >= n) return;
  const int q_end = min(q0 + kBRows, n);
  const int n_tiles = (q_end + kBTile - 1) / kBTile;
  const int qw0 = q0 + wave * 32;
  const int wq_last = min(qw0 + 32, q_end) - 1;
  const int row = qw0 + l32;
  const bool qvalid = row <= wq_last;
  const int Pm1 = a.bias.num_pos - 1, NTm1 = a.bias.num_time - 1;

  // query and upstream-gradient rows of this lane (B operands; d = 16 ks + 8 hf .. + 7)
  bf16x8 qop[4], dop[4];
  {
    const bf16* qs = a.q + (tok0 + row) * a.q_stride + (int64_t)h * kBD + 8 * hf;
    const bf16* ds = a.dout + (tok0 + row) * a.do_stride + (int64_t)h * kBD + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 rq = {0u, 0u, 0u, 0u}, rd = {0u, 0u, 0u, 0u};
      if (qvalid) {
        rq = *(const u32x4*)(qs + 16 * ks);
        rd = *(const u32x4*)(ds + 16 * ks);
      }
      qop[ks] = __builtin_bit_cast(bf16x8, rq);
      dop[ks] = __builtin_bit_cast(bf16x8, rd);
    }
  }
  const int64_t tq = KIND == 1 && qvalid ? a.bias.ts[tok0 + row] : 0;
  int64_t tq_min = 0, tq_max = 0;
  if (KIND == 1) {
    int64_t mn = qvalid ? tq : kTMax, mx = qvalid ? tq : kTMin;
    half_minmax(mn, mx);
    tq_min = uniform_i64(mn);
    tq_max = uniform_i64(mx);
  }
  float slope = 0.f;
  float k0c[8];
  if (KIND == 1) {
    for (int i = tid; i < a.bias.num_pos; i += kBThreads) sm.wpos[i] = a.bias.w_pos[(int64_t)h * a.bias.pos_stride + i];
    if (tid < a.bias.num_time) {
      const float wt = a.bias.w_time[(int64_t)h * a.bias.time_stride + tid];
      sm.wtime[tid] = wt;
      silu_taylor(a.bias.w_pos[(int64_t)h * a.bias.pos_stride + Pm1] + wt, a.alpha, &sm.tay[tid][0]);
    }
  } else if (KIND == 2) {
    slope = a.bias.slopes ? a.bias.slopes[h] : default_alibi_slope(h, H);
  } else {
    silu_taylor(0.f, a.alpha, k0c);
  }

  // staging: thread t moves 16-byte chunk t % 8 of row t / 8 of K and V
  const int srow = tid >> 3, sch = tid & 7;
  TileStager stg;
  stg.xs = (uint32_t)a.k_stride * 2u;
  stg.ys = (uint32_t)a.v_stride * 2u;
  stg.xr = __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + tok0 * a.k_stride + (int64_t)h * kBD), (short)0,
                                             (int)((uint32_t)(q_end - 1) * stg.xs + 2u * kBD), 0x00020000);
  stg.yr = __builtin_amdgcn_make_buffer_rsrc((void*)(a.v + tok0 * a.v_stride + (int64_t)h * kBD), (short)0,
                                             (int)((uint32_t)(q_end - 1) * stg.ys + 2u * kBD), 0x00020000);
  stg.tr = __builtin_amdgcn_make_buffer_rsrc((void*)(KIND == 1 ? a.bias.ts + tok0 : nullptr), (short)0,
                                             KIND == 1 ? 8 * q_end : 0, 0x00020000);
  stg.xoff = (uint32_t)srow * stg.xs + 16u * sch;
  stg.yoff = (uint32_t)srow * stg.ys + 16u * sch;
  auto lstore = [&](int buf, int r0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      *(u32x4*)(&sm.x[buf][(srow + 32 * u) * kBRow + 8 * sch]) = stg.xreg[u];
      *(u32x4*)(&sm.y[buf][(srow + 32 * u) * kBRow + 8 * sch]) = stg.yreg[u];
    }
    if (KIND == 1 && wave == 0) {
      const int64_t tt = (int64_t)(((uint64_t)stg.thi << 32) | stg.tlo);
      sm.t[buf][lane] = tt;
      // the extremes of each 32-key half's times (keys at or past q_end excluded)
      const bool ok = r0 + lane < q_end;
      int64_t mn = ok ? tt : kTMax, mx = ok ? tt : kTMin;
      half_minmax(mn, mx);
      if (l32 == 0) *(i64x2*)(&sm.tmm[buf][hf][0]) = i64x2{mn, mx};
    }
  };
  stg.load(0, KIND == 1 && wave == 0, lane);
  lstore(0, 0);
  __syncthreads();

  // transposing K reads: lane i of each 16-lane group reads keys 4 hf + (i % 16) / 4 (+ the
  // group's offset) at d 16 ((lane / 16) % 2) + 4 (lane % 4) .. + 3 (+ 32 db)
  const int tr_row0 = 4 * hf + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  f32x16 acc[2] = {};
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < n_tiles;
    if (more) stg.load((t + 1) * kBTile, KIND == 1 && wave == 0, lane);
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
      const int j0h = t * kBTile + 32 * hk;
      if (j0h > wq_last || wq_last < qw0) continue;  // past the diagonal, or the wave has no rows
      bf16x8 kop[4], vop[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        kop[ks] = *(const bf16x8*)(&sm.x[buf][(32 * hk + l32) * kBRow + 16 * ks + 8 * hf]);
        vop[ks] = *(const bf16x8*)(&sm.y[buf][(32 * hk + l32) * kBRow + 16 * ks + 8 * hf]);
      }
      f32x16 s = {}, da = {};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qop[ks], s, 0, 0, 0);
        da = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[ks], dop[ks], da, 0, 0, 0);
      }
      // one bias value over the tile (no bias, or saturated position and one time bucket)
      // and a small score range: SiLU' from its expansion around the bias
      bool taylor = false;
      float B0 = 0.f, B1 = 0.f, B2 = 0.f;
      if (KIND != 2) {
        const float D = fabsf(a.alpha) * 1.0001f * uniform_f32(wave_max_abs16(s));
        if (D <= kTaylorD) {
          if (KIND == 0) {
            taylor = true;
            B0 = k0c[4];
            B1 = k0c[5];
            B2 = k0c[6];
          } else {
            const i64x2 mm = *(const i64x2*)(&sm.tmm[buf][hk][0]);
            const int64_t kmin = uniform_i64(mm[0]), kmax = uniform_i64(mm[1]);
            const int tlo = time_bucket(tq_min - kmax, NTm1), thi = time_bucket(tq_max - kmin, NTm1);
            if (qw0 - (j0h + 31) >= Pm1 && tlo == thi) {
              taylor = true;
              const f32x4 bc = *(const f32x4*)(&sm.tay[tlo][4]);
              B0 = uniform_f32(bc[0]);
              B1 = uniform_f32(bc[1]);
              B2 = uniform_f32(bc[2]);
            }
          }
        }
      }
      f32x16 g;
      if (taylor) {
        // keys past the query rows only where the tile crosses the diagonal; keys past n and
        // rows past the item have zero K / V / dO rows, so their g is 0 already
        const bool diag = j0h + 31 > qw0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float d1 = __builtin_fmaf(__builtin_fmaf(B2, s[r], B1), s[r], B0);
          const int j = j0h + accrow(r) + 4 * hf;
          g[r] = (!diag || j <= row) ? da[r] * d1 : 0.f;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jl = 32 * hk + accrow(r) + 4 * hf;  // key within the tile
          const int j = t * kBTile + jl;
          const int64_t dt = KIND == 1 ? tq - sm.t[buf][jl] : 0;
          const float x = __builtin_fmaf(a.alpha, s[r], pair_bias<KIND>(sm, row - j, dt, Pm1, NTm1, slope));
          float aa, d1;
          silu_and_grad(x, aa, d1);
          g[r] = (j <= row && qvalid) ? da[r] * d1 : 0.f;
        }
      }
      bf16x8 gop[2];
      {
        f32x8 g0, g1;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          g0[r] = g[r];
          g1[r] = g[r + 8];
        }
        gop[0] = __builtin_convertvector(g0, bf16x8);
        gop[1] = __builtin_convertvector(g1, bf16x8);
      }
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const bf16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4*)(&sm.x[buf][(tr_row0 + 32 * hk + 16 * mm) * kBRow + 32 * db + tr_col]));
          const bf16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4*)(&sm.x[buf][(tr_row0 + 32 * hk + 16 * mm + 8) * kBRow + 32 * db + tr_col]));
          const bf16x8 ktop = bf16x8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ktop, gop[mm], acc[db], 0, 0, 0);
        }
    }
    if (more) lstore(buf ^ 1, (t + 1) * kBTile);
    __syncthreads();
  }

  // dQ rows: accumulator register 4 g + e holds d = 32 db + 8 g + 4 hf + e of this lane's row
  if (qvalid) {
    const float sc = a.alpha * a.out_scale;
    bf16* op = a.dq + (tok0 + row) * a.dq_stride + (int64_t)h * kBD + 4 * hf;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = acc[db][4 * g + e] * sc;
        *(bf16x4*)(op + 32 * db + 8 * g) = __builtin_convertvector(v4, bf16x4);
      }
  }
}

template <int KIND>
__global__ __launch_bounds__(kBThreads, 2) void attn_bwd_dkv_kernel(BwdArgs a) {
  __shared__ BwdTables sm;
  const int item = blockIdx.x;
  if (item >= *a.work_count) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const WorkItem wi = a.work[item];
  const int h = wi.h, H = a.H;
  const int64_t tok0 = wi.tok0;
  const int n = wi.n;
  // the work list orders items by q_tile; this kernel takes key tile (tiles - 1 - q_tile),
  // whose cost (the query tiles at or after it) is the same q_tile + 1
  const int tiles = (n + kBRows - 1) / kBRows;
  if (wi.qt >= tiles) return;
  const int k0 = (tiles - 1 - wi.qt) * kBRows;
  const int k_end = min(k0 + kBRows, n);
  const int kw0 = k0 + wave * 32;
  const int wk_last = min(kw0 + 32, k_end) - 1;
  const int key = kw0 + l32;
  const bool kvalid = key <= wk_last;
  const int Pm1 = a.bias.num_pos - 1, NTm1 = a.bias.num_time - 1;

  // key and value rows of this lane (B operands; d = 16 ks + 8 hf .. + 7)
  bf16x8 kop[4], vop[4];
  {
    const bf16* ks_ = a.k + (tok0 + key) * a.k_stride + (int64_t)h * kBD + 8 * hf;
    const bf16* vs_ = a.v + (tok0 + key) * a.v_stride + (int64_t)h * kBD + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 rk = {0u, 0u, 0u, 0u}, rv = {0u, 0u, 0u, 0u};
      if (kvalid) {
        rk = *(const u32x4*)(ks_ + 16 * ks);
        rv = *(const u32x4*)(vs_ + 16 * ks);
      }
      kop[ks] = __builtin_bit_cast(bf16x8, rk);
      vop[ks] = __builtin_bit_cast(bf16x8, rv);
    }
  }
  const int64_t tk = KIND == 1 && kvalid ? a.bias.ts[tok0 + key] : 0;
  // the extremes of this wave's key times (both lane halves hold the same keys)
  int64_t tk_min = 0, tk_max = 0;
  if (KIND == 1) {
    int64_t mn = kvalid ? tk : kTMax, mx = kvalid ? tk : kTMin;
    half_minmax(mn, mx);
    tk_min = uniform_i64(mn);
    tk_max = uniform_i64(mx);
  }
  float slope = 0.f;
  float k0c[8];
  if (KIND == 1) {
    for (int i = tid; i < a.bias.num_pos; i += kBThreads) {
      sm.wpos[i] = a.bias.w_pos[(int64_t)h * a.bias.pos_stride + i];
      sm.gpos[i] = 0.f;
    }
    if (tid < a.bias.num_time) {
      const float wt = a.bias.w_time[(int64_t)h * a.bias.time_stride + tid];
      sm.wtime[tid] = wt;
      sm.gtime[tid] = 0.f;
      silu_taylor(a.bias.w_pos[(int64_t)h * a.bias.pos_stride + Pm1] + wt, a.alpha, &sm.tay[tid][0]);
    }
  } else if (KIND == 2) {
    slope = a.bias.slopes ? a.bias.slopes[h] : default_alibi_slope(h, H);
  } else {
    silu_taylor(0.f, a.alpha, k0c);
  }

  // query tiles from the one holding row k0 to the user's last row, through a ring of four
  // stages filled by direct global -> LDS transfers: wave w's Q and dO transfers fill rows
  // 8 w .. 8 w + 7 (lane p: row 8 w + p / 8 at chunk position p % 8, global chunk
  // (p % 8) ^ bswz(row)); rows at or past n read as zeros.  One 4-byte transfer per wave: waves
  // 0, 1 the rows' timestamps (32 each), wave 2 the halves' TimeStat entries, the others
  // nothing.  Tiles go in pairs, one barrier per pair.
  const int t0 = k0 / kBTile, t_end = (n + kBTile - 1) / kBTile;
  __shared__ BStage st0, st1;
  const uint32_t xs = (uint32_t)a.q_stride * 2u, ys = (uint32_t)a.do_stride * 2u;
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.q + tok0 * a.q_stride + (int64_t)h * kBD), (short)0, (int)((uint32_t)(n - 1) * xs + 2u * kBD), 0x00020000);
  const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.dout + tok0 * a.do_stride + (int64_t)h * kBD), (short)0, (int)((uint32_t)(n - 1) * ys + 2u * kBD), 0x00020000);
  // dO's remainder (same rows and stride as dO), when the caller keeps dO to about 16 bits
  const bool lo = a.dout_lo != nullptr;
  const __amdgpu_buffer_rsrc_t zr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(lo ? a.dout_lo + tok0 * a.do_stride + (int64_t)h * kBD : nullptr), (short)0,
      lo ? (int)((uint32_t)(n - 1) * ys + 2u * kBD) : 0, 0x00020000);
  uint32_t xo[2], yo[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = 16 * wave + 8 * u + (lane >> 3);
    const uint32_t ch = 16u * (uint32_t)((lane & 7) ^ bswz(r));
    xo[u] = (uint32_t)r * xs + ch;
    yo[u] = (uint32_t)r * ys + ch;
  }
  const __amdgpu_buffer_rsrc_t mr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(KIND != 1 || wave > 2 ? nullptr : wave < 2 ? (const void*)(a.bias.ts + tok0) : (const void*)(a.tstat + tok0)),
      (short)0, KIND != 1 || wave > 2 ? 0 : wave < 2 ? 8 * n : 16 * n, 0x00020000);
  // waves 0, 1: dword lane of the tile's 256-byte half wave; wave 2: dword lane % 4 of the
  // TimeStat at the first token of half lane / 4
  const uint32_t mo = wave < 2 ? 256u * (uint32_t)wave + 4u * lane : 512u * (uint32_t)(lane >> 2) + 4u * (lane & 3);
  auto dma = [&](BStage& stg, int t) __attribute__((always_inline)) {
    const bool real = t < t_end;
    const uint32_t r0 = (uint32_t)(t * kBTile);
    const uint32_t xsoff = __builtin_amdgcn_readfirstlane(real ? r0 * xs : 0x7fffffffu);
    const uint32_t ysoff = __builtin_amdgcn_readfirstlane(real ? r0 * ys : 0x7fffffffu);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr)(stg.x + 1024 * wave + 512 * u), 16, xo[u], xsoff, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(yr, (lds_ptr)(stg.y + 1024 * wave + 512 * u), 16, yo[u], ysoff, 0, 0);
      if (lo) __builtin_amdgcn_raw_ptr_buffer_load_lds(zr, (lds_ptr)(stg.z + 1024 * wave + 512 * u), 16, yo[u], ysoff, 0, 0);
    }
    const uint32_t msoff = __builtin_amdgcn_readfirstlane(
        (real && KIND == 1 && wave < 3) ? (wave < 2 ? 8u * r0 : 16u * r0) : 0x7fffffffu);
    void* dst = wave < 2 ? (void*)(stg.t + 32 * wave) : wave == 2 ? (void*)stg.tmm : (void*)stg.dummy;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(mr, (lds_ptr)dst, 4, mo, msoff, 0, 0);
  };
  dma(st0, t0);

  // byte offsets of this lane's reads within a stage: the operand read of k-step ks at
  // kbase ^ (32 ks) (row l32 + 32 hq), the transposing reads of column block db at
  // vbase[e] ^ (64 db) (row tr_row0 + 8 e + 16 mm + 32 hq)
  const int tr_row0 = 4 * hf + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  uint32_t kbase, vbase[2];
  {
    const int sk = bswz(l32);
    kbase = (uint32_t)(l32 * 128 + 32 * (sk >> 1) + 16 * (hf ^ (sk & 1)));
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = tr_row0 + 8 * e, sv = bswz(r);
      vbase[e] = (uint32_t)(r * 128 + 64 * (sv >> 2) + 16 * ((tr_col >> 3) ^ (sv & 3)) + 2 * (tr_col & 7));
    }
  }
  f32x16 dvacc[2] = {}, dkacc[2] = {};
  // running per-lane sum of the scores of saturated one-bucket tiles whose time bucket is run_b
  // (wave-uniform; their position bucket is P - 1): added to the tables when the bucket changes
  // and after the last tile, instead of one wave sum and LDS add per tile
  float run_g = 0.f;
  int run_b = -1;
  auto flush = [&]() __attribute__((always_inline)) {
    if (run_b >= 0) {
      const float tot = wave_sum(run_g);
      if (lane == 0) {
        atomicAdd(&sm.gpos[Pm1], tot);
        atomicAdd(&sm.gtime[run_b], tot);
      }
      run_g = 0.f;
      run_b = -1;
    }
  };
  auto compute = [&](const BStage& stg, int t) __attribute__((always_inline)) {
#pragma unroll
    for (int hq = 0; hq < 2; ++hq) {
      const int i0h = t * kBTile + 32 * hq;  // first query of this step
      if (i0h + 31 < kw0 || i0h >= n || kw0 > wk_last) continue;  // uniform: no pair i >= j
      bf16x8 qa[4], da_[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        qa[ks] = *(const bf16x8*)((const char*)stg.x + 32 * hq * 128 + (kbase ^ (32u * ks)));
        da_[ks] = *(const bf16x8*)((const char*)stg.y + 32 * hq * 128 + (kbase ^ (32u * ks)));
      }
      f32x16 s = {}, dd = {};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ks], kop[ks], s, 0, 0, 0);
        dd = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da_[ks], vop[ks], dd, 0, 0, 0);
      }
      if (lo) {
        // dA from dO's remainder too: dA and the table gradients see dO to about 16 bits
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 dl = *(const bf16x8*)((const char*)stg.z + 32 * hq * 128 + (kbase ^ (32u * ks)));
          dd = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dl, vop[ks], dd, 0, 0, 0);
        }
      }
      // the tile's bias class: one position bucket when i - j >= P - 1 for every pair, one or
      // two time buckets when the extreme times say so (exactly)
      int tlo = 0, thi = 0;
      bool sat = true;
      if (KIND == 1) {
        const i64x2 qmm = *(const i64x2*)(&stg.tmm[2 * hq]);
        const int64_t qmin = uniform_i64(qmm[0]), qmax = uniform_i64(qmm[1]);
        tlo = time_bucket(qmin - tk_max, NTm1);
        thi = time_bucket(qmax - tk_min, NTm1);
        sat = i0h - (kw0 + 31) >= Pm1;
      }
      bool taylor = false;
      float A0 = 0.f, A1 = 0.f, A2 = 0.f, B0 = 0.f, B1 = 0.f, B2 = 0.f;
      if (KIND != 2 && sat && tlo == thi) {
        const float D = fabsf(a.alpha) * 1.0001f * uniform_f32(wave_max_abs16(s));
        if (D <= kTaylorD) {
          taylor = true;
          if (KIND == 0) {
            A0 = k0c[1]; A1 = k0c[2]; A2 = k0c[3]; B0 = k0c[4]; B1 = k0c[5]; B2 = k0c[6];
          } else {
            const f32x4 ac = *(const f32x4*)(&sm.tay[tlo][0]);
            const f32x4 bc = *(const f32x4*)(&sm.tay[tlo][4]);
            A0 = uniform_f32(ac[1]); A1 = uniform_f32(ac[2]); A2 = uniform_f32(ac[3]);
            B0 = uniform_f32(bc[0]); B1 = uniform_f32(bc[1]); B2 = uniform_f32(bc[2]);
          }
        }
      }
      // register r: query i = i0h + accrow(r) + 4 hf of this lane's key
      f32x16 p, g;
      if (taylor) {
        // queries before the key only where the tile crosses the diagonal; rows past n and keys
        // past the item have zero Q / dO / K / V rows (their g is 0, their P meets zero dO)
        const bool diag = i0h < kw0 + 31;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float aa = __builtin_fmaf(__builtin_fmaf(A2, s[r], A1), s[r], A0);
          const float d1 = __builtin_fmaf(__builtin_fmaf(B2, s[r], B1), s[r], B0);
          const bool ok = !diag || i0h + accrow(r) + 4 * hf >= key;
          p[r] = ok ? aa : 0.f;
          g[r] = ok ? dd[r] * d1 : 0.f;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int il = 32 * hq + accrow(r) + 4 * hf;
          const int i = t * kBTile + il;
          const int64_t dt = KIND == 1 ? stg.t[il] - tk : 0;
          const float x = __builtin_fmaf(a.alpha, s[r], pair_bias<KIND>(sm, i - key, dt, Pm1, NTm1, slope));
          float aa, d1;
          silu_and_grad(x, aa, d1);
          const bool ok = i >= key && i < n && kvalid;
          p[r] = ok ? aa : 0.f;
          g[r] = ok ? dd[r] * d1 : 0.f;
        }
      }
      if (KIND == 1 && sat && thi == tlo) {
        if (tlo != run_b) {
          flush();
          run_b = tlo;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) run_g += g[r];
      } else if (KIND == 1) {
        // table gradients of this tile: tile sums for one position bucket and one or two time
        // buckets, else one LDS add per score
        float gs = 0.f, ghi = 0.f;
        const int64_t tlim = tk + (((int64_t)1 << thi) - 1);  // dt >= 2^thi - 1
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          gs += g[r];
          if (thi == tlo + 1) ghi += stg.t[32 * hq + accrow(r) + 4 * hf] >= tlim ? g[r] : 0.f;
        }
        if (sat || thi <= tlo + 1) {
          const float tot = wave_sum(gs);
          const float hi = thi == tlo + 1 ? wave_sum(ghi) : 0.f;
          if (lane == 0) {
            if (sat) atomicAdd(&sm.gpos[Pm1], tot);
            if (thi == tlo) {
              atomicAdd(&sm.gtime[tlo], tot);
            } else if (thi == tlo + 1) {
              atomicAdd(&sm.gtime[tlo], tot - hi);
              atomicAdd(&sm.gtime[thi], hi);
            }
          }
        }
        if (!sat) {
          // position buckets of an unsaturated tile: sums along the tile's diagonals.  Score
          // (query qo = accrow(r) + 4 hf, key l32) lies on diagonal qo - l32, i.e. i - j =
          // i0h - kw0 + qo - l32.  For register r, lane (m, hf) takes the score of key
          // (qo - m) mod 32 of its half: diagonal m when qo >= m, m - 32 otherwise; the two
          // halves' sums are added and each of lanes 0..31 adds its two diagonals to the table
          // (scores outside the causal range have g = 0).
          // (in two groups of eight shuffles, each issued before any of them is used)
          float dpos = 0.f, dneg = 0.f;
#pragma unroll
          for (int h8 = 0; h8 < 2; ++h8) {
            float v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const int r = 8 * h8 + q;
              const int src = ((accrow(r) + 4 * hf - l32) & 31) + 32 * hf;
              // (__shfl: a __builtin_bit_cast of an ext-vector element, g[r], to feed the raw
              // ds_bpermute builtin is folded to element 0 by hipcc 7.2)
              v[q] = __shfl(g[r], src, 64);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const int r = 8 * h8 + q;
              if (accrow(r) + 4 * hf >= l32) dpos += v[q];
              else dneg += v[q];
            }
          }
          dpos += __shfl_xor(dpos, 32, 64);
          dneg += __shfl_xor(dneg, 32, 64);
          if (hf == 0) {
            const int dp = i0h - kw0 + l32;  // i - j of diagonal l32; l32 - 32 is dp - 32
            if (dp >= 0) atomicAdd(&sm.gpos[min(dp, Pm1)], dpos);
            if (dp >= 32) atomicAdd(&sm.gpos[min(dp - 32, Pm1)], dneg);
          }
        }
        if (thi > tlo + 1) {
          // three or more time buckets: per bucket b in [tlo, thi], a wave sum of the scores in
          // b and one LDS add (per-score adds would put up to 64 lanes on one address).  Every
          // score's bucket lies in [tlo, thi] (the bucket is monotone in dt); scores outside the
          // causal range have g = 0, whatever bucket they are counted in.
          uint32_t pk[4] = {0u, 0u, 0u, 0u};  // bucket - tlo of register r in byte r % 4 of pk[r / 4]
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int il = 32 * hq + accrow(r) + 4 * hf;
            const uint32_t k = (uint32_t)(time_bucket(stg.t[il] - tk, NTm1) - tlo) & 255u;
            pk[r >> 2] |= k << (8 * (r & 3));
          }
          for (int b = 0; b <= thi - tlo; ++b) {
            float v = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r)
              v += ((pk[r >> 2] >> (8 * (r & 3))) & 255u) == (uint32_t)b ? g[r] : 0.f;
            const float tot = wave_sum(v);
            if (lane == 0) atomicAdd(&sm.gtime[tlo + b], tot);
          }
        }
      }
      bf16x8 pop[2], gop[2];
      {
        f32x8 p0, p1, g0, g1;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          p0[r] = p[r];
          p1[r] = p[r + 8];
          g0[r] = g[r];
          g1[r] = g[r + 8];
        }
        pop[0] = __builtin_convertvector(p0, bf16x8);
        pop[1] = __builtin_convertvector(p1, bf16x8);
        gop[0] = __builtin_convertvector(g0, bf16x8);
        gop[1] = __builtin_convertvector(g1, bf16x8);
      }
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const int rb = (32 * hq + 16 * mm) * 128;
          const bf16x4 d0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4*)((const char*)stg.y + rb + (vbase[0] ^ (64u * db))));
          const bf16x4 d1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4*)((const char*)stg.y + rb + (vbase[1] ^ (64u * db))));
          const bf16x4 e0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4*)((const char*)stg.x + rb + (vbase[0] ^ (64u * db))));
          const bf16x4 e1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4*)((const char*)stg.x + rb + (vbase[1] ^ (64u * db))));
          const bf16x8 dot = bf16x8{d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
          const bf16x8 qt = bf16x8{e0[0], e0[1], e0[2], e0[3], e1[0], e1[1], e1[2], e1[3]};
          dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dot, pop[mm], dvacc[db], 0, 0, 0);
          dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt, gop[mm], dkacc[db], 0, 0, 0);
        }
    }
  };
  wait_vm<0>();
  lds_barrier();
  auto one = [&](const BStage& c, BStage& nx, int t) __attribute__((always_inline)) {
    dma(nx, t + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(c, t);
    wait_vm<0>();
    lds_barrier();
  };
  for (int t = t0; t < t_end; t += 2) {
    one(st0, st1, t);
    if (t + 1 >= t_end) break;
    one(st1, st0, t + 1);
  }

  // dK and dV rows: accumulator register 4 g + e holds d = 32 db + 8 g + 4 hf + e of this
  // lane's key
  if (kvalid) {
    const float sv = a.out_scale, sk = a.alpha * a.out_scale;
    bf16* kp = a.dk + (tok0 + key) * a.dk_stride + (int64_t)h * kBD + 4 * hf;
    bf16* vp = a.dv + (tok0 + key) * a.dv_stride + (int64_t)h * kBD + 4 * hf;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 k4, v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          k4[e] = dkacc[db][4 * g + e] * sk;
          v4[e] = dvacc[db][4 * g + e] * sv;
        }
        *(bf16x4*)(kp + 32 * db + 8 * g) = __builtin_convertvector(k4, bf16x4);
        *(bf16x4*)(vp + 32 * db + 8 * g) = __builtin_convertvector(v4, bf16x4);
      }
  }
  // table gradients: this workgroup's sums, once per touched entry
  if (KIND == 1) {
    flush();
    lds_barrier();
    for (int i = tid; i < a.bias.num_pos; i += kBThreads) {
      const float v = sm.gpos[i];
      if (v != 0.f) atomicAdd(&a.dw_pos[(int64_t)h * a.bias.pos_stride + i], v * a.out_scale);
    }
    if (tid < a.bias.num_time) {
      const float v = sm.gtime[tid];
      if (v != 0.f) atomicAdd(&a.dw_time[(int64_t)h * a.bias.time_stride + tid], v * a.out_scale);
    }
  }
}

// zero fill of the table gradients (a kernel, not a memset: callers may capture the stream)
__global__ void zero_f32_kernel(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

}  // namespace

int attn_bwd_block_rows() { return kBRows; }

hipError_t launch_attn_bwd_bf16(const BwdArgs& a, int grid, int64_t n_pos_grad, int64_t n_time_grad,
                                hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (a.bias.kind == 1) {
    if (n_pos_grad > 0)
      hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((n_pos_grad + 255) / 256)), dim3(256), 0, stream, a.dw_pos, n_pos_grad);
    if (n_time_grad > 0)
      hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((n_time_grad + 255) / 256)), dim3(256), 0, stream, a.dw_time, n_time_grad);
  }
  const dim3 g((unsigned)grid), blk(kBThreads);
  if (a.bias.kind == 1) {
    hipLaunchKernelGGL(attn_bwd_dq_kernel<1>, g, blk, 0, stream, a);
    hipLaunchKernelGGL(attn_bwd_dkv_kernel<1>, g, blk, 0, stream, a);
  } else if (a.bias.kind == 2) {
    hipLaunchKernelGGL(attn_bwd_dq_kernel<2>, g, blk, 0, stream, a);
    hipLaunchKernelGGL(attn_bwd_dkv_kernel<2>, g, blk, 0, stream, a);
  } else {
    hipLaunchKernelGGL(attn_bwd_dq_kernel<0>, g, blk, 0, stream, a);
    hipLaunchKernelGGL(attn_bwd_dkv_kernel<0>, g, blk, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace hstu
