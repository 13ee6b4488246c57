// Pointwise parts of the HSTU layer on bf16 MFMA.
//
//  f1:  Z = SiLU(X W1^T + b1), written as bf16 [T, 2H(dqk+dv)] whose column
//       blocks are U | V | Q | K ("Actions Speak Louder than Words" §3.1 eq. (1),
//       and the chunk order of the toy layer in "4.4 推荐模型的 Scaling").  The
//       split is free: the attention reads Q, K, V as strided views of Z.
//  f2:  Y = (LayerNorm(O) * U) W2^T + b2 (+ X), eq. (3); LayerNorm over the H dv
//       features of a token with biased variance.  The LayerNorm statistics,
//       the affine map and the U gate are applied while the GEMM's operand tile
//       is staged into LDS, so the gated activations never go to HBM (the
//       pages fuse LayerNorm and the output MLP into one operator, §3.5).
//
// Both are computed transposed, C^T = W A^T, so each lane of a 32x32 MFMA
// output holds one token row and four consecutive output features per
// register group: epilogue stores are 8-byte row segments.
#include "hstu_internal.h"

namespace hstu {
namespace {

constexpr int kBN = 128;  // output features per workgroup (rows of C^T)
constexpr int kBM = 128;  // tokens per workgroup (columns of C^T)
constexpr int kBK = 64;

struct GemmArgs {
  const bf16* W;       // [N][K]
  int32_t N, K;
  int64_t M;
  const bf16* X;       // mode 0: [M][K]
  const float* O;      // mode 1: attention output [M][K], fp32
  const bf16* U;       // mode 1: gate, row stride u_stride
  int64_t u_stride;
  const float* gamma;  // mode 1: [K] or null
  const float* beta;   // mode 1: [K] or null
  float eps;
  const float* bias;   // [N] or null
  const bf16* R;       // mode 1: residual [M][N] or null
  bf16* Y;             // [M][N]
};

struct SmemGemm {
  bf16 w[2][kBN * kBK];
  bf16 x[2][kBM * kBK];
  float mean[kBM];
  float rstd[kBM];
  float gamma[1024];
  float beta[1024];
};

// 64-bank LDS: 16 lanes reading one chunk of 16 consecutive 128-byte rows are conflict-free
// when the chunk is XOR-ed with (row / 2) & 7.
__device__ __forceinline__ int t_off(int row, int chunk) { return row * kBK + ((chunk ^ ((row >> 1) & 7)) << 3); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

template <int MODE>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  __shared__ SmemGemm sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int wn = wave & 1, wm = wave >> 1;
  const int n0 = blockIdx.x * kBN;
  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int K = g.K, N = g.N;
  const int64_t M = g.M;

  if (MODE == 1) {
    for (int i = tid; i < K; i += 256) {
      sm.gamma[i] = g.gamma ? g.gamma[i] : 1.0f;
      sm.beta[i] = g.beta ? g.beta[i] : 0.0f;
    }
    // LayerNorm statistics of the workgroup's token rows: each lane keeps up to
    // four 4-element chunks of a row in registers; mean first, then the biased
    // variance around it.
    for (int rr = 0; rr < 32; ++rr) {
      const int row = wave * 32 + rr;
      const int64_t m = m0 + row;
      f32x4 vals[4];
      float s = 0.f;
#pragma unroll
      for (int ci = 0; ci < 4; ++ci) {
        const int c = lane + 64 * ci;
        vals[ci] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (m < M && c < K / 4) {
          vals[ci] = *(const f32x4*)(g.O + m * K + 4 * c);
#pragma unroll
          for (int e = 0; e < 4; ++e) s += vals[ci][e];
        }
      }
      const float mean = wave_sum(s) / (float)K;
      float q = 0.f;
#pragma unroll
      for (int ci = 0; ci < 4; ++ci) {
        const int c = lane + 64 * ci;
        if (m < M && c < K / 4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) q += (vals[ci][e] - mean) * (vals[ci][e] - mean);
        }
      }
      const float var = wave_sum(q) / (float)K;
      if (lane == 0) {
        sm.mean[row] = mean;
        sm.rstd[row] = 1.0f / sqrtf(var + g.eps);
      }
    }
    __syncthreads();
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4 wreg[4], xreg[4], ureg[4];
  f32x4 oreg[4][2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + 256 * u, row = c >> 3, chunk = c & 7;
      wreg[u] = *(const u32x4*)(g.W + (int64_t)(n0 + row) * K + k0 + 8 * chunk);
      const int64_t m = m0 + row;
      if (MODE == 0) {
        xreg[u] = u32x4{0u, 0u, 0u, 0u};
        if (m < M) xreg[u] = *(const u32x4*)(g.X + m * K + k0 + 8 * chunk);
      } else {
        ureg[u] = u32x4{0u, 0u, 0u, 0u};
        oreg[u][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        oreg[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (m < M) {
          oreg[u][0] = *(const f32x4*)(g.O + m * K + k0 + 8 * chunk);
          oreg[u][1] = *(const f32x4*)(g.O + m * K + k0 + 8 * chunk + 4);
          ureg[u] = *(const u32x4*)(g.U + m * g.u_stride + k0 + 8 * chunk);
        }
      }
    }
  };
  auto lstore = [&](int buf, int k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + 256 * u, row = c >> 3, chunk = c & 7;
      *(u32x4*)(&sm.w[buf][t_off(row, chunk)]) = wreg[u];
      if (MODE == 0) {
        *(u32x4*)(&sm.x[buf][t_off(row, chunk)]) = xreg[u];
      } else {
        const bf16x8 u8 = __builtin_bit_cast(bf16x8, ureg[u]);
        const float mean = sm.mean[row], rstd = sm.rstd[row];
        f32x8 gv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int col = k0 + 8 * chunk + e;
          const float ov = oreg[u][e >> 2][e & 3];
          gv[e] = ((ov - mean) * rstd * sm.gamma[col] + sm.beta[col]) * (float)u8[e];
        }
        *(bf16x8*)(&sm.x[buf][t_off(row, chunk)]) = __builtin_convertvector(gv, bf16x8);
      }
    }
  };

  const int n_k = K / kBK;
  gload(0);
  lstore(0, 0);
  __syncthreads();
  for (int kt = 0; kt < n_k; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_k) gload((kt + 1) * kBK);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 aop[2], bop[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        aop[i] = *(const bf16x8*)(&sm.w[buf][t_off(64 * wn + 32 * i + l32, 2 * ks + hf)]);
        bop[i] = *(const bf16x8*)(&sm.x[buf][t_off(64 * wm + 32 * i + l32, 2 * ks + hf)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[i], bop[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < n_k) lstore(buf ^ 1, (kt + 1) * kBK);
    __syncthreads();
  }

  // epilogue: acc[i][j] register r -> feature n0 + 64 wn + 32 i + 8 (r/4) + 4 hf + r%4,
  // token m0 + 64 wm + 32 j + l32
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t m = m0 + 64 * wm + 32 * j + l32;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int n = n0 + 64 * wn + 32 * i + 8 * grp + 4 * hf;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * grp + e] + (g.bias ? g.bias[n + e] : 0.f);
        if (MODE == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[e] = v[e] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * v[e]));
        } else if (g.R) {
          const bf16x4 r4 = *(const bf16x4*)(g.R + m * N + n);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += (float)r4[e];
        }
        *(bf16x4*)(g.Y + m * N + n) = __builtin_convertvector(v, bf16x4);
      }
  }
}

__global__ void embed_sum_kernel(int64_t T, int dim, const bf16* __restrict__ item,
                                 int64_t num_items, const bf16* __restrict__ action,
                                 int num_actions, const int32_t* __restrict__ ids,
                                 const int32_t* __restrict__ aids, bf16* __restrict__ x) {
  const int chunks = dim / 8;
  const int64_t total = T * chunks;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = idx / chunks;
    const int c = (int)(idx - t * chunks);
    const int64_t it = ids[t];
    const int at = aids[t];
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (it >= 0 && it < num_items) a = *(const u32x4*)(item + it * dim + 8 * c);
    if (at >= 0 && at < num_actions) b = *(const u32x4*)(action + (int64_t)at * dim + 8 * c);
    const f32x8 s = __builtin_convertvector(__builtin_bit_cast(bf16x8, a), f32x8) +
                    __builtin_convertvector(__builtin_bit_cast(bf16x8, b), f32x8);
    *(bf16x8*)(x + t * dim + 8 * c) = __builtin_convertvector(s, bf16x8);
  }
}

}  // namespace

hipError_t launch_f1_gemm_silu(const bf16* x, const bf16* w1, const float* b1, bf16* z, int64_t M,
                               int32_t N, int32_t K, hipStream_t stream) {
  if (N % kBN || K % kBK) return hipErrorInvalidValue;
  if (M <= 0) return hipSuccess;
  GemmArgs g{};
  g.W = w1; g.N = N; g.K = K; g.M = M; g.X = x; g.bias = b1; g.Y = z;
  dim3 grid(N / kBN, (unsigned)((M + kBM - 1) / kBM));
  hipLaunchKernelGGL(gemm_kernel<0>, grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_ln_gate_f2(const float* o, const bf16* u, int64_t u_stride, const float* gamma,
                             const float* beta, float eps, const bf16* w2, const float* b2,
                             const bf16* x, bf16* y, int64_t M, int32_t D, int32_t HV,
                             hipStream_t stream) {
  if (D % kBN || HV % kBK || HV > 1024) return hipErrorInvalidValue;
  if (M <= 0) return hipSuccess;
  GemmArgs g{};
  g.W = w2; g.N = D; g.K = HV; g.M = M; g.O = o; g.U = u; g.u_stride = u_stride;
  g.gamma = gamma; g.beta = beta; g.eps = eps; g.bias = b2; g.R = x; g.Y = y;
  dim3 grid(D / kBN, (unsigned)((M + kBM - 1) / kBM));
  hipLaunchKernelGGL(gemm_kernel<1>, grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_embed_sum(int64_t T, int32_t dim, const bf16* item, int64_t num_items,
                            const bf16* action, int32_t num_actions, const int32_t* ids,
                            const int32_t* aids, bf16* x, hipStream_t stream) {
  if (dim % 8) return hipErrorInvalidValue;
  if (T <= 0) return hipSuccess;
  const int64_t total = T * (dim / 8);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(embed_sum_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, T, dim, item,
                     num_items, action, num_actions, ids, aids, x);
  return hipGetLastError();
}

}  // namespace hstu
