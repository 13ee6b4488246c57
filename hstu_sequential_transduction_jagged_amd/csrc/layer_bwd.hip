// Gradients of one HSTU layer ("Actions Speak Louder than Words" reading notes §3.1 eqs. (1)-(3))
// apart from the attention (attention_bwd.hip), for bf16 storage with fp32 accumulation:
//
//   eq. (3)  Y = G W2^T + b2 (+ X), G = LN(O) * U:
//            dG = dY W2, dW2 = dY^T G, db2 = sum_t dY,
//            dU = dG * LN(O), d(LN) = dG * U, dgamma = sum_t d(LN) * xhat, dbeta = sum_t d(LN),
//            dO = rstd (dxhat - mean(dxhat) - xhat mean(dxhat * xhat)), dxhat = d(LN) * gamma
//   eq. (1)  Z = SiLU(Zpre), Zpre = X W1^T + b1:
//            dZpre = dZ * SiLU'(Zpre) (Zpre recomputed), dX = dZpre W1 (+ dY),
//            dW1 = dZpre^T X, db1 = sum_t dZpre
//
// One GEMM kernel serves all products: C[m][n] = sum_k A(m, k) B(n, k) where either operand is
// stored k-contiguous ([rows][K]) or row-contiguous ([K][rows]); 128 x 128 workgroup tiles,
// 4 waves of 64 x 64 on v_mfma_f32_32x32x16_bf16, 32-deep slices staged through LDS with
// bounded buffer loads one slice ahead.  Row-contiguous operands are read with transposing LDS
// reads (ds_read_b64_tr_b16), whose k order within a 16-deep step is 4 hf + {0..3},
// 8 + 4 hf + {0..3}; k-contiguous operands are read in that same order (two 8-byte reads), so
// the two operands always agree.  Epilogues: bf16 store (optional fp32 column bias and bf16
// residual) and fp32 atomic add (split-k weight gradients).  The recomputed X W1^T + b1 with
// the SiLU backward dZpre = dZ * SiLU'(.) written over dZ runs on the forward's f1 kernel.
#include "hstu_internal.h"

namespace hstu {
namespace {

constexpr int kGB = 128;   // rows of A and of B per workgroup tile
constexpr int kGK = 32;    // slice depth
constexpr int kGPadK = 40;   // LDS row of a k-contiguous tile (bf16): 32 + 8
constexpr int kGPadM = 136;  // LDS row of a row-contiguous tile (bf16): 128 + 8

struct GemmArgs {
  const bf16* a;
  const bf16* b;
  int64_t lda, ldb;
  int32_t M, N, K, k_split;  // k_split: depth per grid.z slice (multiple of 32)
  // epilogues
  bf16* c;             // EPI 0: bf16 out [M][ldc]
  float* cf;           // EPI 1: fp32 [M][ldc] (added to)
  int64_t ldc;
  const float* bias;   // EPI 0: fp32 [N] or null
  const bf16* resid;   // EPI 0: bf16 [M][ldr] added, or null
  int64_t ldr;
};

template <int TA, int TB, int EPI>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int AE = TA ? kGK * kGPadM : kGB * kGPadK;  // elements of an A tile
  constexpr int BE = TB ? kGK * kGPadM : kGB * kGPadK;
  __shared__ __attribute__((aligned(16))) bf16 sa[2][AE];
  __shared__ __attribute__((aligned(16))) bf16 sb[2][BE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.x * kGB, n0 = blockIdx.y * kGB;
  const int kb = blockIdx.z * g.k_split;
  const int ke = min(g.K, kb + g.k_split);
  if (kb >= ke) return;
  const int nslices = (ke - kb + kGK - 1) / kGK;

  // buffer descriptors: rows past M / N, and (row-contiguous operands) k rows past this
  // split's end, read as zeros
  auto rsrc = [](const bf16* p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0,
                                             (int)min(bytes, (int64_t)0x7fffffff), 0x00020000);
  };
  __amdgpu_buffer_rsrc_t ar, br;
  if (TA) ar = rsrc(g.a + (int64_t)kb * g.lda, (int64_t)(ke - kb) * g.lda * 2);
  else ar = rsrc(g.a + (int64_t)m0 * g.lda, (int64_t)max(min(kGB, g.M - m0), 0) * g.lda * 2);
  if (TB) br = rsrc(g.b + (int64_t)kb * g.ldb, (int64_t)(ke - kb) * g.ldb * 2);
  else br = rsrc(g.b + (int64_t)n0 * g.ldb, (int64_t)max(min(kGB, g.N - n0), 0) * g.ldb * 2);

  // staging: 512 chunks of 16 bytes per tile, two per thread
  u32x4 ra[2], rb[2];
  auto gload = [&](int s) {
    const int k0 = s * kGK;  // relative to kb
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = tid + 256 * u;
      uint32_t aoff, boff;
      if (TA) aoff = (uint32_t)((int64_t)(k0 + (c >> 4)) * g.lda * 2 + 2 * (m0 + 8 * (c & 15)));
      else aoff = (uint32_t)((int64_t)(c >> 2) * g.lda * 2 + 2 * (kb + k0 + 8 * (c & 3)));
      if (TB) boff = (uint32_t)((int64_t)(k0 + (c >> 4)) * g.ldb * 2 + 2 * (n0 + 8 * (c & 15)));
      else boff = (uint32_t)((int64_t)(c >> 2) * g.ldb * 2 + 2 * (kb + k0 + 8 * (c & 3)));
      ra[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ar, aoff, 0, 0));
      rb[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(br, boff, 0, 0));
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = tid + 256 * u;
      if (TA) *(u32x4*)(&sa[buf][(c >> 4) * kGPadM + 8 * (c & 15)]) = ra[u];
      else *(u32x4*)(&sa[buf][(c >> 2) * kGPadK + 8 * (c & 3)]) = ra[u];
      if (TB) *(u32x4*)(&sb[buf][(c >> 4) * kGPadM + 8 * (c & 15)]) = rb[u];
      else *(u32x4*)(&sb[buf][(c >> 2) * kGPadK + 8 * (c & 3)]) = rb[u];
    }
  };
  const int tr_row0 = 4 * hf + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  // operand of rows r0 .. r0 + 31 (tile-relative), 16-deep step ks, in the shared k order
  auto operand = [&](const bf16* t, bool trans, int r0, int ks) {
    bf16x4 h0, h1;
    if (trans) {
      h0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4*)(t + (tr_row0 + 16 * ks) * kGPadM + r0 + tr_col));
      h1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4*)(t + (tr_row0 + 16 * ks + 8) * kGPadM + r0 + tr_col));
    } else {
      h0 = *(const bf16x4*)(t + (r0 + l32) * kGPadK + 16 * ks + 4 * hf);
      h1 = *(const bf16x4*)(t + (r0 + l32) * kGPadK + 16 * ks + 8 + 4 * hf);
    }
    return bf16x8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
  };

  f32x16 acc[2][2] = {};
  gload(0);
  lstore(0);
  __syncthreads();
  for (int s = 0; s < nslices; ++s) {
    const int buf = s & 1;
    const bool more = s + 1 < nslices;
    if (more) gload(s + 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) av[i] = operand(sa[buf], TA, 64 * wm + 32 * i, ks);
#pragma unroll
      for (int j = 0; j < 2; ++j) bv[j] = operand(sb[buf], TB, 64 * wn + 32 * j, ks);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
  }

  // acc[i][j] register r: row m = m0 + 64 wm + 32 i + 8 (r / 4) + 4 hf + r % 4, column
  // n = n0 + 64 wn + 32 j + l32
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + 64 * wn + 32 * j + l32;
    if (n >= g.N) continue;
    const float bn = (EPI != 1 && g.bias) ? g.bias[n] : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (m >= g.M) continue;
        const float v = acc[i][j][r];
        if (EPI == 0) {
          float o = v + bn;
          if (g.resid) o += (float)g.resid[(int64_t)m * g.ldr + n];
          g.c[(int64_t)m * g.ldc + n] = (bf16)o;
        } else {
          atomicAdd(&g.cf[(int64_t)m * g.ldc + n], v);
        }
      }
  }
}

// LayerNorm and gate backward, one wave per token (grid-stride): from dG, O and U of the row,
// dU (into dZ's U columns), G = LN(O) * U (for dW2), dO, and per-column sums of d(LN) * xhat
// and d(LN) added to dgamma / dbeta once per wave.  Lane l holds columns 8 (l + 64 c) .. + 7.
constexpr int kMaxHV = 2048;

template <int NC>
__global__ __launch_bounds__(256) void ln_gate_bwd_kernel(
    int64_t T, int32_t HV, float eps, const bf16* __restrict__ dG, const bf16* __restrict__ O,
    const f32x4* __restrict__ ostats, int32_t dvh, const bf16* __restrict__ U, int64_t u_stride,
    const float* __restrict__ gamma, const float* __restrict__ beta, bf16* __restrict__ dU,
    int64_t du_stride, bf16* __restrict__ G, bf16* __restrict__ dO, bf16* __restrict__ dOlo,
    float* __restrict__ dgamma, float* __restrict__ dbeta) {
  __shared__ float red_g[kMaxHV], red_b[kMaxHV];
  for (int i = threadIdx.x; i < HV; i += 256) red_g[i] = red_b[i] = 0.f;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  const int nch = HV / 8;
  float gsum[NC][8] = {}, bsum[NC][8] = {};
  float gm[NC][8], bt[NC][8];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = lane + 64 * c;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      gm[c][e] = ch < nch ? gamma[8 * ch + e] : 0.f;
      bt[c][e] = ch < nch ? beta[8 * ch + e] : 0.f;
    }
  }
  const float inv = 1.0f / (float)HV;
  const int H = HV / dvh;
  for (int64_t t = wave; t < T; t += nwaves) {
    float o[NC][8], dg[NC][8], u[NC][8];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int ch = lane + 64 * c;
      bf16x8 ov = {}, gv = {}, uv = {};
      float moff = 0.f;  // the head's offset: O stores the deviations from it
      if (ch < nch) {
        ov = *(const bf16x8*)(O + t * HV + 8 * ch);
        gv = *(const bf16x8*)(dG + t * HV + 8 * ch);
        uv = *(const bf16x8*)(U + t * u_stride + 8 * ch);
        moff = ostats[t * H + (8 * ch) / dvh][0];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[c][e] = (float)ov[e] + moff;
        dg[c][e] = (float)gv[e];
        u[c][e] = (float)uv[e];
      }
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) s += o[c][e];
    for (int m = 1; m < 64; m <<= 1) s += __shfl_xor(s, m, 64);
    const float mean = s * inv;
    float v = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const bool ok = lane + 64 * c < nch;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = ok ? o[c][e] - mean : 0.f;
        v += d * d;
      }
    }
    for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
    const float rstd = 1.0f / sqrtf(v * inv + eps);
    float s1 = 0.f, s2 = 0.f;
    float xh[NC][8], dxh[NC][8];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int ch = lane + 64 * c;
      bf16x8 duv, gv8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xh[c][e] = (o[c][e] - mean) * rstd;
        const float ln = xh[c][e] * gm[c][e] + bt[c][e];
        duv[e] = (bf16)(dg[c][e] * ln);
        gv8[e] = (bf16)(ln * u[c][e]);
        const float dln = dg[c][e] * u[c][e];
        gsum[c][e] += dln * xh[c][e];
        bsum[c][e] += dln;
        dxh[c][e] = dln * gm[c][e];
        s1 += dxh[c][e];
        s2 += dxh[c][e] * xh[c][e];
      }
      if (ch < nch) {
        *(bf16x8*)(dU + t * du_stride + 8 * ch) = duv;
        *(bf16x8*)(G + t * HV + 8 * ch) = gv8;
      }
    }
    for (int m = 1; m < 64; m <<= 1) {
      s1 += __shfl_xor(s1, m, 64);
      s2 += __shfl_xor(s2, m, 64);
    }
    s1 *= inv;
    s2 *= inv;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int ch = lane + 64 * c;
      // dO in bf16, and (for the attention's dO V^T product) the bf16 rounding of what that
      // leaves, so hi + lo carries dO to about 16 bits
      bf16x8 dov, dol;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float full = rstd * (dxh[c][e] - s1 - xh[c][e] * s2);
        dov[e] = (bf16)full;
        dol[e] = (bf16)(full - (float)dov[e]);
      }
      if (ch < nch) {
        *(bf16x8*)(dO + t * HV + 8 * ch) = dov;
        if (dOlo) *(bf16x8*)(dOlo + t * HV + 8 * ch) = dol;
      }
    }
  }
  // the workgroup's four waves into LDS, then one global add per column
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = lane + 64 * c;
    if (ch < nch)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        atomicAdd(&red_g[8 * ch + e], gsum[c][e]);
        atomicAdd(&red_b[8 * ch + e], bsum[c][e]);
      }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < HV; i += 256) {
    atomicAdd(&dgamma[i], red_g[i]);
    atomicAdd(&dbeta[i], red_b[i]);
  }
}

// column sums of a bf16 [T][N] matrix (row stride ld, N % 8 == 0, 16-byte aligned rows) added
// to out[N]: a workgroup takes 256 columns of rows_per rows; thread t reads the 16-byte chunk
// t % 32 (8 columns) of rows t / 32, t / 32 + 8, ..., and the 8 row groups are added in LDS
__global__ __launch_bounds__(256) void colsum_kernel(const bf16* __restrict__ x, int64_t ld,
                                                     int64_t T, int32_t N, int64_t rows_per,
                                                     float* __restrict__ out) {
  __shared__ float part[8][257];
  const int tid = threadIdx.x, c = tid & 31, rg = tid >> 5;
  const int n0 = blockIdx.x * 256 + 8 * c;
  const int64_t t0 = (int64_t)blockIdx.y * rows_per, t1 = min(T, t0 + rows_per);
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (n0 < N) {
#pragma unroll 4
    for (int64_t t = t0 + rg; t < t1; t += 8) {
      const bf16x8 v = *(const bf16x8*)(x + t * ld + n0);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += (float)v[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rg][8 * c + e] = s[e];
  __syncthreads();
  const int n = blockIdx.x * 256 + tid;
  if (n < N) {
    float v = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) v += part[g][tid];
    atomicAdd(&out[n], v);
  }
}

__global__ void zero_f32_kernel2(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

template <int TA, int TB, int EPI>
hipError_t gemm(const GemmArgs& g, int splits, hipStream_t stream) {
  const dim3 grid((unsigned)((g.M + kGB - 1) / kGB), (unsigned)((g.N + kGB - 1) / kGB),
                  (unsigned)splits);
  hipLaunchKernelGGL((gemm_bf16_kernel<TA, TB, EPI>), grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_f32_kernel2, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_layer_bwd_pre(const LayerBwdLaunch& L, hipStream_t stream) {
  const int64_t T = L.T;
  const int HV = L.HV, D = L.D;
  hipError_t e;
  // dG = dY W2 (W2 is [D][HV]: row-contiguous in HV for the k = d reduction)
  GemmArgs g{};
  g.a = L.dy; g.lda = D;
  g.b = L.w2; g.ldb = HV;
  g.M = (int)T; g.N = HV; g.K = D; g.k_split = D;
  g.c = L.dg; g.ldc = HV;
  if ((e = gemm<0, 1, 0>(g, 1, stream)) != hipSuccess) return e;
  // LayerNorm and gate backward
  const int nc = (HV / 8 + 63) / 64;
  const int64_t want = (T + 3) / 4;
  const unsigned blocks = (unsigned)(want < 1 ? 1 : want > 1024 ? 1024 : want);
  if (nc == 1)
    hipLaunchKernelGGL(ln_gate_bwd_kernel<1>, dim3(blocks), dim3(256), 0, stream, T, HV, L.eps, L.dg, L.o,
                       L.ostats, L.dvh, L.u, L.u_stride, L.gamma, L.beta, L.dz, L.dz_stride, L.g, L.dO,
                       L.dO_lo, L.dgamma, L.dbeta);
  else if (nc == 2)
    hipLaunchKernelGGL(ln_gate_bwd_kernel<2>, dim3(blocks), dim3(256), 0, stream, T, HV, L.eps, L.dg, L.o,
                       L.ostats, L.dvh, L.u, L.u_stride, L.gamma, L.beta, L.dz, L.dz_stride, L.g, L.dO,
                       L.dO_lo, L.dgamma, L.dbeta);
  else
    hipLaunchKernelGGL(ln_gate_bwd_kernel<4>, dim3(blocks), dim3(256), 0, stream, T, HV, L.eps, L.dg, L.o,
                       L.ostats, L.dvh, L.u, L.u_stride, L.gamma, L.beta, L.dz, L.dz_stride, L.g, L.dO,
                       L.dO_lo, L.dgamma, L.dbeta);
  return hipGetLastError();
}

hipError_t launch_layer_bwd_post(const LayerBwdLaunch& L, hipStream_t stream) {
  const int64_t T = L.T;
  const int HV = L.HV, D = L.D, N1 = L.N1;
  hipError_t e;
  // dZpre = dZ * SiLU'(X W1^T + b1), over dZ: the forward's f1 GEMM with a SiLU-backward
  // epilogue (dZ's rows are N1 wide)
  if (L.dz_stride != N1) return hipErrorInvalidValue;
  if ((e = launch_f1_gemm_silu(L.x, L.w1, L.b1, L.dz, T, N1, D, stream, true)) != hipSuccess) return e;
  // dX = dZpre W1 (+ dY): on the f1 kernel with W1^T as its weight operand when the dG buffer
  // (free once the LayerNorm backward has run) holds W1^T, else on the generic kernel
  GemmArgs g{};
  if ((int64_t)D * N1 <= T * HV) {
    bf16* w1t = (bf16*)L.dg;  // [D][N1]
    if ((e = launch_transpose_bf16(L.w1, w1t, N1, D, stream)) != hipSuccess) return e;
    if ((e = launch_f1_gemm_silu(L.dz, w1t, nullptr, L.dx, T, D, N1, stream, false,
                                 L.residual ? L.dy : nullptr, true)) != hipSuccess)
      return e;
  } else {
    g.a = L.dz; g.lda = L.dz_stride;
    g.b = L.w1; g.ldb = D;
    g.M = (int)T; g.N = D; g.K = N1; g.k_split = N1;
    g.c = L.dx; g.ldc = D;
    g.resid = L.residual ? L.dy : nullptr; g.ldr = D;
    if ((e = gemm<0, 1, 0>(g, 1, stream)) != hipSuccess) return e;
  }
  // weight gradients, split over tokens into slices of `kt` rows: about 1 024 workgroups per
  // product (two per CU, twice over), so that the fp32 atomic adds of the partial tiles stay few
  auto token_split = [&](int32_t m, int32_t n, int* splits) {
    const int64_t tiles = (int64_t)((m + kGB - 1) / kGB) * ((n + kGB - 1) / kGB);
    const int64_t want = tiles >= 1024 ? 1 : 1024 / tiles;
    int64_t kt = ((T + want - 1) / want + 31) / 32 * 32;
    if (kt < 256) kt = 256;
    *splits = (int)((T + kt - 1) / kt);
    return kt;
  };
  int splits = 0;
  // dW1 = dZpre^T X  ([N1][D]; both operands row-contiguous in the k = t reduction)
  g = GemmArgs{};
  g.a = L.dz; g.lda = L.dz_stride;
  g.b = L.x; g.ldb = D;
  g.M = N1; g.N = D; g.K = (int)T; g.k_split = (int)token_split(N1, D, &splits);
  g.cf = L.dw1; g.ldc = D;
  if ((e = gemm<1, 1, 1>(g, splits, stream)) != hipSuccess) return e;
  // dW2 = dY^T G  ([D][HV])
  g = GemmArgs{};
  g.a = L.dy; g.lda = D;
  g.b = L.g; g.ldb = HV;
  g.M = D; g.N = HV; g.K = (int)T; g.k_split = (int)token_split(D, HV, &splits);
  g.cf = L.dw2; g.ldc = HV;
  if ((e = gemm<1, 1, 1>(g, splits, stream)) != hipSuccess) return e;
  // bias gradients
  const int64_t rows_per = 512;
  hipLaunchKernelGGL(colsum_kernel, dim3((unsigned)((N1 + 255) / 256), (unsigned)((T + rows_per - 1) / rows_per)), dim3(256), 0, stream, L.dz, L.dz_stride, T, N1, rows_per, L.db1);
  hipLaunchKernelGGL(colsum_kernel, dim3((unsigned)((D + 255) / 256), (unsigned)((T + rows_per - 1) / rows_per)), dim3(256), 0, stream, L.dy, (int64_t)D, T, D, rows_per, L.db2);
  return hipGetLastError();
}

}  // namespace hstu
