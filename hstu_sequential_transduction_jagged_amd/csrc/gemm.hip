// Pointwise parts of the HSTU layer on bf16 MFMA.
//
//  f1:  Z = SiLU(X W1^T + b1), written as bf16 [T, 2H(dqk+dv)] whose column
//       blocks are U | V | Q | K ("Actions Speak Louder than Words" §3.1 eq. (1),
//       and the chunk order of the toy layer in "4.4 推荐模型的 Scaling").  The
//       split is free: the attention reads Q, K, V as strided views of Z.
//  f2:  Y = (LayerNorm(O) * U) W2^T + b2 (+ X), eq. (3); LayerNorm over the H dv
//       features of a token with biased variance.  One workgroup owns 64 tokens
//       and every output feature: it reads each token's O and U row once,
//       normalises and gates it in registers and keeps the bf16 result in LDS as
//       the GEMM operand, so the gated activations never go to HBM (the pages
//       fuse LayerNorm and the output MLP into one operator, §3.5).
//
// Both GEMMs are computed transposed, C^T = W A^T, so each lane of a 32x32 MFMA
// output holds one token row and four consecutive output features per register
// group: epilogue stores are 8-byte row segments.
#include "hstu_internal.h"

namespace hstu {
namespace {

// ---------------------------------------------------------------------------------------------
// f1: 128 output features x 256 tokens per workgroup, four waves of 64 features x 128 tokens.
// K is staged 32 deep through two LDS buffers from two register sets, so each slice's global
// loads are issued two slices before their LDS write.  The bf16 results leave through LDS as
// whole 256-byte row segments.

constexpr int kF1Feat = 128;
constexpr int kF1Tok = 256;
constexpr int kF1K = 32;
constexpr int kF1Threads = 256;
constexpr int kF1WElems = kF1Feat * kF1K;  // one W slice
constexpr int kF1XElems = kF1Tok * kF1K;   // one X slice

struct F1Args {
  const bf16* X;       // [M][K]
  const bf16* W;       // [N][K]
  const float* bias;   // [N] or null
  bf16* Y;             // [M][N]
  int64_t M;
  int32_t N, K, tiles;
};

// 64-byte LDS rows of four 16-byte chunks; chunk c of row r sits in slot c ^ ((r >> 2) & 3), so
// 16 lanes that read one chunk of 16 consecutive rows, or write the four chunks of four
// consecutive rows, touch 16 distinct 16-byte bank groups.
__device__ __forceinline__ int f1_off(int row, int chunk) {
  return row * kF1K + ((chunk ^ ((row >> 2) & 3)) << 3);
}

__global__ __launch_bounds__(kF1Threads, 2) void f1_kernel(F1Args g) {
  // two stages of (W slice, X slice); reused by the epilogue as a 128-token x 128-feature tile
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * (kF1WElems + kF1XElems)];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int wf = wave & 1, wt = wave >> 1;

  // Workgroups are dealt to the eight XCDs in turn; XCD x takes the x-th eighth of the tiles in
  // order, so the feature blocks of one token block run on one XCD and share its L2 copy of X.
  const int per = gridDim.x >> 3;
  const int s = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (s >= g.tiles) return;
  const int nfb = g.N / kF1Feat;
  const int tb = s / nfb;
  const int n0 = (s - tb * nfb) * kF1Feat;
  const int64_t m0 = (int64_t)tb * kF1Tok;
  const int K = g.K, N = g.N;
  const int64_t M = g.M;
  const uint32_t kb = 2u * (uint32_t)K;  // bytes per row
  const int64_t rows = M - m0 < kF1Tok ? M - m0 : kF1Tok;

  // Rows are addressed in the vector offset, which the descriptor bounds: token rows at or past
  // M read as zeros.
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.W + (int64_t)n0 * K), (short)0, (int)(kF1Feat * kb), 0x00020000);
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.X + m0 * K), (short)0, (int)(rows * kb), 0x00020000);
  // thread t stages chunk t % 4 of rows t / 4 + 64 u (same swizzle for every u)
  const int srow = tid >> 2, sch = tid & 3;
  const uint32_t voff = (uint32_t)srow * kb + 16u * sch;
  const int lofs = f1_off(srow, sch);
  auto sw = [&](int buf) { return smem + buf * (kF1WElems + kF1XElems); };
  auto sx = [&](int buf) { return smem + buf * (kF1WElems + kF1XElems) + kF1WElems; };

  u32x4 wr[2][2], xr[2][4];
  const int nk = K / kF1K;  // even
  // slices past the end reload the last one: the loads stay unconditional, so the wait counts
  // are exact
  auto gload = [&](int set, int kt) {
    const uint32_t k0 = 2u * (uint32_t)(kt < nk ? kt : nk - 1) * kF1K;
#pragma unroll
    for (int u = 0; u < 2; ++u)
      wr[set][u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 wrs, voff + 64u * u * kb, k0, 0));
#pragma unroll
    for (int u = 0; u < 4; ++u)
      xr[set][u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 xrs, voff + 64u * u * kb, k0, 0));
  };
  auto lstore = [&](int set, int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u) *(u32x4*)(sw(buf) + lofs + 64 * u * kF1K) = wr[set][u];
#pragma unroll
    for (int u = 0; u < 4; ++u) *(u32x4*)(sx(buf) + lofs + 64 * u * kF1K) = xr[set][u];
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 a[2], b[4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *(const bf16x8*)(sw(buf) + f1_off(64 * wf + 32 * i + l32, 2 * ks + hf));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *(const bf16x8*)(sx(buf) + f1_off(128 * wt + 32 * j + l32, 2 * ks + hf));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  // slice kt lives in register set kt % 2 and LDS buffer kt % 2
  gload(0, 0);
  gload(1, 1);
  lstore(0, 0);
  __syncthreads();
  // (scheduling barriers pin the loads ahead of the slice's MFMAs)
  for (int kt = 0; kt < nk; kt += 2) {
    gload(0, kt + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute(0);
    lstore(1, 1);
    __syncthreads();
    gload(1, kt + 3);
    __builtin_amdgcn_sched_barrier(0);
    compute(1);
    lstore(0, 0);
    __syncthreads();
  }
  // the last two gloads were the repeated last slice and are unused; the final lstore wrote
  // buffer 0 after every read of it

  // epilogue: acc[i][j] register r -> feature n0 + 64 wf + 32 i + 8 (r / 4) + 4 hf + r % 4,
  // token m0 + 128 wt + 32 j + l32.  Two passes of 128 tokens (j = 2p, 2p + 1) through an LDS
  // tile of 256-byte rows: 8-byte piece (granule q, half hf) of local row lr sits at granule
  // q ^ (lr & 15), half hf ^ ((lr >> 4) & 1), so each 32-lane half of a write touches 32
  // distinct 8-byte bank pairs and each 16-lane row read 16 distinct granules.
  float bv[2][4][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int grp = 0; grp < 4; ++grp)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        bv[i][grp][e] = g.bias ? g.bias[n0 + 64 * wf + 32 * i + 8 * grp + 4 * hf + e] : 0.f;
  u32x2* tile = (u32x2*)smem;  // [128 rows][32 halves of 8 bytes]
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = 2 * p + jj;
      const int lr = 64 * wt + 32 * jj + l32;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = acc[i][j][4 * grp + e] + bv[i][grp][e];
            v[e] = x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * x));
          }
          const int q = 8 * wf + 4 * i + grp;
          tile[lr * 32 + 2 * (q ^ (lr & 15)) + (hf ^ ((lr >> 4) & 1))] =
              __builtin_bit_cast(u32x2, __builtin_convertvector(v, bf16x4));
        }
    }
    __syncthreads();
    // 128 rows x 16 granules; thread t takes granule t % 16 of rows t / 16 + 16 k
    const int q = tid & 15;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int lr = (tid >> 4) + 16 * k;
      const int64_t m = m0 + 128 * (lr >> 6) + 32 * (2 * p + ((lr >> 5) & 1)) + (lr & 31);
      const u32x4 c = *(const u32x4*)(tile + lr * 32 + 2 * (q ^ (lr & 15)));
      const u32x4 o = ((lr >> 4) & 1) ? u32x4{c[2], c[3], c[0], c[1]} : c;
      if (m < M) *(u32x4*)(g.Y + m * N + n0 + 8 * q) = o;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------
// f2: 64 tokens per workgroup, all output features.  Phase 1 (LayerNorm statistics, affine map,
// U gate) writes the bf16 operand A [64 tokens][HV] to LDS; phase 2 runs C^T = W2 A^T with each
// of the four waves owning a quarter of a 512-feature chunk.  W2 fragments come straight from
// global memory (every W2 element is used by one wave of the workgroup, so LDS staging would not
// be reused) through a ring of four k-steps, out of a copy of W2 in fragment order: one MFMA
// operand is 1 KiB of contiguous bytes, eight whole cache lines per load.

constexpr int kF2Tok = 64;
constexpr int kF2Threads = 256;

struct F2Args {
  const float* O;      // attention output [M][HV], fp32
  const bf16* U;       // gate, row stride u_stride
  int64_t u_stride;
  const float* gamma;  // [HV] or null
  const float* beta;   // [HV] or null
  float eps;
  const bf16* Wp;      // W2 [N][HV] in fragment order (pack_frag_kernel)
  const float* bias;   // [N] or null
  const bf16* R;       // residual [M][N] or null
  bf16* Y;             // [M][N]
  int64_t M;
  int32_t N, HV;
};

// Sum over the 64 lanes of a wave, as a wave-uniform value.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  auto at = [&](int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
  };
  return (at(0) + at(16)) + (at(32) + at(48));
}

// One 128 NI-feature chunk of the output: wave w computes features nb + 32 NI w .. + 32 NI - 1
// for all 64 tokens.  The LDS operand rows are HV + 8 elements apart: (HV / 8 + 1) is odd, so
// 16 consecutive rows at one column fall in 16 distinct 16-byte bank groups.
template <int NI>
__device__ __forceinline__ void f2_chunk(const F2Args& g, const bf16* sa, int nb, int64_t m0,
                                         int lane, int wave) {
  const int l32 = lane & 31, hf = lane >> 5;
  const int HV = g.HV, rs8 = HV / 8 + 1, N = g.N;
  const int fw = nb + 32 * NI * wave;
  // fragment (row block fw / 32 + i, k-step ks) of the packed W2, through a buffer descriptor
  // over this wave's row blocks (fetches past the last k-step read zeros or unused fragments)
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.Wp + (int64_t)fw * HV), (short)0, (int)(32 * NI * HV * 2), 0x00020000);
  const uint32_t voff = 16u * (uint32_t)lane;
  const int nks = HV / 16;  // a multiple of 4
  auto wload = [&](int i, int ks) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                          wrs, voff, (uint32_t)(i * nks + ks) * 1024u, 0));
  };
  f32x16 acc[NI][2];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  bf16x8 wring[4][NI];
#pragma unroll
  for (int p = 0; p < 3; ++p)
#pragma unroll
    for (int i = 0; i < NI; ++i) wring[p][i] = wload(i, p);
  for (int ks0 = 0; ks0 < nks; ks0 += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ks = ks0 + u;
      // unconditional, so the wait counts stay exact: the last three steps fetch fragments
      // past the end of K (the next row, or zeros past the descriptor), never used
#pragma unroll
      for (int i = 0; i < NI; ++i) wring[(u + 3) & 3][i] = wload(i, ks + 3);
      bf16x8 b[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = ((const bf16x8*)sa)[(32 * j + l32) * rs8 + 2 * ks + hf];
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wring[u][i], b[j], acc[i][j], 0, 0, 0);
      // keep each step's fetches three steps ahead of their use
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // acc[i][j] register r -> feature fw + 32 i + 8 (r / 4) + 4 hf + r % 4, token m0 + 32 j + l32
  float bv[NI][4][4];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int grp = 0; grp < 4; ++grp)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        bv[i][grp][e] = g.bias ? g.bias[fw + 32 * i + 8 * grp + 4 * hf + e] : 0.f;
  // y may not alias the residual: all of a token block's residual loads are issued before its
  // stores (rows past M read zeros through the descriptor and are not stored)
  const bf16* __restrict__ R = g.R;
  bf16* __restrict__ Y = g.Y;
  const int64_t nrow = g.M - m0 < kF2Tok ? g.M - m0 : kF2Tok;
  const __amdgpu_buffer_rsrc_t rrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(R ? R + m0 * N : nullptr), (short)0, R ? (int)(nrow * N * 2) : 0, 0x00020000);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int tl = 32 * j + l32;  // token within the block
    u32x2 r4[NI][4];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp)
        r4[i][grp] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                                   rrs, (uint32_t)(tl * N + fw + 4 * hf) * 2u,
                                                   (uint32_t)(32 * i + 8 * grp) * 2u, 0));
    if (tl >= nrow) continue;
    bf16* yrow = Y + (m0 + tl) * N + fw + 4 * hf;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const bf16x4 rb = __builtin_bit_cast(bf16x4, r4[i][grp]);
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * grp + e] + bv[i][grp][e] + (float)rb[e];
        *(bf16x4*)(yrow + 32 * i + 8 * grp) = __builtin_convertvector(v, bf16x4);
      }
  }
}

// QN: 8-feature chunks of a row per lane (HV <= 512 QN).
template <int QN>
__global__ __launch_bounds__(kF2Threads, 2) void f2_kernel(F2Args g) {
  __shared__ bf16 sa[kF2Tok * (512 * QN + 8)];
  // the wave index is uniform: W2 descriptors built from it stay in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int HV = g.HV, nch = HV >> 3;
  const int64_t m0 = (int64_t)blockIdx.x * kF2Tok;
  const int64_t M = g.M;

  // ---- phase 1: wave w normalises and gates token rows 16 w .. 16 w + 15, RB rows at a time;
  // lane l handles the 8-feature chunks l + 64 q of each row.
  constexpr int RB = 4 / QN;
  f32x8 gam[QN], bet[QN];
#pragma unroll
  for (int q = 0; q < QN; ++q) {
    const int c = min(lane + 64 * q, nch - 1);  // lanes past the last chunk repeat it, unused
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      gam[q][e] = g.gamma ? g.gamma[8 * c + e] : 1.0f;
      bet[q][e] = g.beta ? g.beta[8 * c + e] : 0.0f;
    }
  }
  // O and U rows through buffer descriptors bounded at the workgroup's last token: rows past M
  // and lanes past the row's last chunk (offset 2^31) read as zeros, without branches.
  const int64_t nrow = M - m0 < kF2Tok ? M - m0 : kF2Tok;
  const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.O + m0 * HV), (short)0, (int)(nrow * HV * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t urs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.U + m0 * g.u_stride), (short)0, (int)(nrow * g.u_stride * 2), 0x00020000);
  uint32_t vo[QN], vu[QN];
#pragma unroll
  for (int q = 0; q < QN; ++q) {
    const int c = lane + 64 * q;
    vo[q] = c < nch ? 32u * c : 0x80000000u;
    vu[q] = c < nch ? 16u * c : 0x80000000u;
  }
  f32x4 ov[2][RB][QN][2];
  u32x4 uv[2][RB][QN];
  auto load = [&](int slot, int r0) {
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const uint32_t row = 16 * wave + r0 + rr;
#pragma unroll
      for (int q = 0; q < QN; ++q) {
        ov[slot][rr][q][0] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(ors, vo[q], row * HV * 4u, 0));
        ov[slot][rr][q][1] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(ors, vo[q] + 16u, row * HV * 4u, 0));
        uv[slot][rr][q] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(urs, vu[q], row * (uint32_t)g.u_stride * 2u, 0));
      }
    }
  };
  const float inv_hv = 1.0f / (float)HV;
  load(0, 0);
#pragma unroll
  for (int bi = 0; bi < 16 / RB; ++bi) {
    const int slot = bi & 1;
    if (bi + 1 < 16 / RB) load(slot ^ 1, (bi + 1) * RB);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < QN; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) s += ov[slot][rr][q][e >> 2][e & 3];
      const float mean = wave_sum_dpp(s) * inv_hv;
      float d = 0.f;
#pragma unroll
      for (int q = 0; q < QN; ++q) {
        const bool in = lane + 64 * q < nch;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float t = in ? ov[slot][rr][q][e >> 2][e & 3] - mean : 0.f;
          d += t * t;
        }
      }
      const float rstd = 1.0f / sqrtf(wave_sum_dpp(d) * inv_hv + g.eps);
      const int row = 16 * wave + bi * RB + rr;
      // lanes past the row's last chunk write the row's padding chunk, which is never read
#pragma unroll
      for (int q = 0; q < QN; ++q) {
        const int c = lane + 64 * q;
        const bf16x8 u8 = __builtin_bit_cast(bf16x8, uv[slot][rr][q]);
        f32x8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          y[e] = ((ov[slot][rr][q][e >> 2][e & 3] - mean) * rstd * gam[q][e] + bet[q][e]) *
                 (float)u8[e];
        ((bf16x8*)sa)[row * (nch + 1) + (c < nch ? c : nch)] = __builtin_convertvector(y, bf16x8);
      }
    }
  }
  __syncthreads();

  // ---- phase 2
  for (int nb = 0; nb < g.N; nb += 512) {
    const int rem = g.N - nb;
    if (rem >= 512) f2_chunk<4>(g, sa, nb, m0, lane, wave);
    else if (rem == 384) f2_chunk<3>(g, sa, nb, m0, lane, wave);
    else if (rem == 256) f2_chunk<2>(g, sa, nb, m0, lane, wave);
    else f2_chunk<1>(g, sa, nb, m0, lane, wave);
  }
}

// W [N][K] (N % 32 == 0, K % 16 == 0) rewritten in MFMA operand order: fragment (nb, ks), at
// index nb K / 16 + ks, is 64 lanes x 8 bf16 where lane l + 32 h holds row 32 nb + l, columns
// 16 ks + 8 h .. + 7 (the A operand of v_mfma_f32_32x32x16_bf16 for rows 32 nb .. + 31).
__global__ void pack_frag_kernel(const bf16* __restrict__ w, bf16* __restrict__ out, int N, int K) {
  const int64_t total = (int64_t)N * K / 8;  // 16-byte pieces
  const int kst = K / 16;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t frag = idx >> 6;
    const int ln = (int)(idx & 63);
    const int64_t nb = frag / kst;
    const int ks = (int)(frag - nb * kst);
    const int64_t row = 32 * nb + (ln & 31);
    ((u32x4*)out)[idx] = *(const u32x4*)(w + row * K + 16 * ks + 8 * (ln >> 5));
  }
}

// ---------------------------------------------------------------------------------------------

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
  if (N % kF1Feat || K % (2 * kF1K) || K <= 0) return hipErrorInvalidValue;
  if ((int64_t)kF1Tok * 2 * K > 0x7fffffff || (int64_t)kF1Feat * 2 * K > 0x7fffffff)
    return hipErrorInvalidValue;
  if (M <= 0) return hipSuccess;
  const int64_t tiles = (int64_t)(N / kF1Feat) * ((M + kF1Tok - 1) / kF1Tok);
  if (tiles > 0x7ffffff0) return hipErrorInvalidValue;
  F1Args g{};
  g.X = x; g.W = w1; g.bias = b1; g.Y = z; g.M = M; g.N = N; g.K = K; g.tiles = (int32_t)tiles;
  const unsigned grid = (unsigned)((tiles + 7) / 8 * 8);
  hipLaunchKernelGGL(f1_kernel, dim3(grid), dim3(kF1Threads), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_ln_gate_f2(const float* o, const bf16* u, int64_t u_stride, const float* gamma,
                             const float* beta, float eps, const bf16* w2, const float* b2,
                             const bf16* x, bf16* y, int64_t M, int32_t D, int32_t HV,
                             bf16* w2_packed, hipStream_t stream) {
  if (D % 128 || D <= 0 || HV % 64 || HV <= 0 || HV > 1024 || u_stride % 8 || u_stride < HV ||
      u_stride > (1 << 24))
    return hipErrorInvalidValue;
  if (M <= 0) return hipSuccess;
  {
    const int64_t pieces = (int64_t)D * HV / 8;
    hipLaunchKernelGGL(pack_frag_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0,
                       stream, w2, w2_packed, D, HV);
  }
  F2Args g{};
  g.O = o; g.U = u; g.u_stride = u_stride; g.gamma = gamma; g.beta = beta; g.eps = eps;
  g.Wp = w2_packed; g.bias = b2; g.R = x; g.Y = y; g.M = M; g.N = D; g.HV = HV;
  const dim3 grid((unsigned)((M + kF2Tok - 1) / kF2Tok));
  if (HV <= 512)
    hipLaunchKernelGGL(f2_kernel<1>, grid, dim3(kF2Threads), 0, stream, g);
  else
    hipLaunchKernelGGL(f2_kernel<2>, grid, dim3(kF2Threads), 0, stream, g);
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
