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
// f1: 128 output features x 256 tokens per workgroup, four waves of 64 features x 128 tokens,
// three workgroups per CU (167 registers, 48 KiB of LDS each), so that one workgroup's
// SiLU epilogue overlaps the others' MFMA loops.  K is staged 32 deep through two LDS stages
// filled by direct global-to-LDS transfers one slice ahead (no staging registers).  The bf16
// results leave through LDS as whole 256-byte row segments.

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
  const bf16* R;       // EPI 2: [M][N] added before the rounding, or null
  int64_t M;
  int32_t N, K, tiles;
};

// 64-byte LDS rows of four 16-byte chunks; chunk c of row r sits in slot c ^ ((r >> 2) & 3), so
// 16 lanes that read one chunk of 16 consecutive rows touch 16 distinct 16-byte bank groups.
__device__ __forceinline__ int f1_off(int row, int chunk) {
  return row * kF1K + ((chunk ^ ((row >> 2) & 3)) << 3);
}


// NK: K / 32 when known at compile time (the slice loop is then straight-line code, which keeps
// the compiler's own waits on the transfers exact), 0 for any K.  EPI 0: Y = SiLU(acc); EPI 1
// (the layer's backward): Y holds dZ on entry and dZ * SiLU'(acc) on exit, acc = X W^T + b, with
// SiLU'(z) = s (1 + z (1 - s)), s = 1 / (1 + e^-z), the product in fp32 and rounded once;
// EPI 2: Y = acc (+ R), rounded once (the layer backward's dX = dZpre W1 + dY).
template <int NK, int EPI>
__global__ __launch_bounds__(kF1Threads, 3) void f1_kernel(F1Args g) {
  // stage arrays of their own: the compiler then knows which stage a transfer writes
  __shared__ __attribute__((aligned(16))) bf16 sW0[kF1WElems], sW1[kF1WElems];
  __shared__ __attribute__((aligned(16))) bf16 sX0[kF1XElems], sX1[kF1XElems];
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
  // A transfer instruction fills 1 KiB of a stage: lane p writes 16-byte granule 64 v + p, which
  // is row 16 v + p / 4, slot p % 4, so the lane fetches chunk (p % 4) ^ ((row >> 2) & 3) of
  // that row.  Wave w issues instructions v = w + 4 u (W: u < 2, X: u < 4).
  uint32_t wvo[2], xvo[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = 16 * (wave + 4 * u) + (lane >> 2);
    const uint32_t off = (uint32_t)row * kb + 16u * (uint32_t)((lane & 3) ^ ((row >> 2) & 3));
    if (u < 2) wvo[u] = off;
    xvo[u] = off;
  }
  const int nk = NK ? NK : K / kF1K;
  auto dma = [&](bf16* sw, bf16* sx, int kt) {
    // the slice past the end repeats the last one into a stage no one reads again
    const uint32_t k0 = 2u * (uint32_t)(kt < nk ? kt : nk - 1) * kF1K;
#pragma unroll
    for (int u = 0; u < 2; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_ptr)(sw + (wave + 4 * u) * 512), 16,
                                               wvo[u], k0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_ptr)(sx + (wave + 4 * u) * 512), 16,
                                               xvo[u], k0, 0, 0);
  };

  // acc[i][j] register r -> feature n0 + 64 wf + 32 i + 8 (r / 4) + 4 hf + r % 4, token
  // m0 + 128 wt + 32 j + l32; the accumulators start at the bias (a null bias reads zeros)
  const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.bias, (short)0, g.bias ? 4 * N : 0, 0x00020000);
  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const f32x4 b4 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
          brs, 4u * (uint32_t)(n0 + 64 * wf + 4 * hf), 4u * (32 * i + 8 * grp), 0));
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][4 * grp + e] = b4[e];
    }

  auto compute = [&](const bf16* sw, const bf16* sx) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 a[2], b[4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *(const bf16x8*)(sw + f1_off(64 * wf + 32 * i + l32, 2 * ks + hf));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *(const bf16x8*)(sx + f1_off(128 * wt + 32 * j + l32, 2 * ks + hf));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };
  // slice kt lives in stage kt % 2; at slice kt the transfer of slice kt + 1 is issued into the
  // other stage (whose readers all passed the last barrier), then slice kt is multiplied, then
  // the transfer is waited for
  auto step = [&](bf16* cw, bf16* cx, bf16* fw, bf16* fx, int kt) {
    dma(fw, fx, kt + 1);
    __builtin_amdgcn_sched_barrier(0);  // issued ahead of the slice's MFMAs
    compute(cw, cx);
    wait_vm<0>();
    lds_barrier();
  };
  dma(sW0, sX0, 0);
  wait_vm<0>();
  lds_barrier();
#pragma unroll
  for (int kt = 0; kt < (NK ? NK : nk); kt += 2) {
    step(sW0, sX0, sW1, sX1, kt);
    if (kt + 1 < nk) step(sW1, sX1, sW0, sX0, kt + 1);
  }
  wait_vm<0>();  // the repeated transfers past the end land before the stages are reused
  lds_barrier();

  // epilogue: SiLU of acc[i][j] (bias included).  Two passes of 128 tokens (j = 2 p, 2 p + 1) through an LDS
  // tile of 256-byte rows (rows 0..63 in sX0, 64..127 in sX1; local row 64 wt + 32 (j - 2 p) +
  // l32): 8-byte piece (granule q, half hf) of row r sits at granule q ^ (r & 15), half
  // hf ^ ((r >> 4) & 1), so each 32-lane half of a write touches 32 distinct 8-byte bank pairs
  // and each 16-lane row read 16 distinct granules.
  // output rows past M fall outside the descriptor and are dropped
  const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.Y + m0 * N), (short)0, (int)min(rows * N * 2, (int64_t)0x7fffffff), 0x00020000);
  u32x2* wtile = (u32x2*)(wt ? sX1 : sX0);  // [64 rows][32 halves of 8 bytes]
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int r = 32 * jj + l32;  // row within this wave's array
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          f32x4 v;
          if (EPI == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x = acc[i][2 * p + jj][4 * grp + e];
              v[e] = x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * x));
            }
          } else {
            // this lane's token 128 wt + 32 j + l32 and features 64 wf + 32 i + 8 grp + 4 hf .. + 3
            const int64_t tok = 128 * wt + 32 * (2 * p + jj) + l32;
            const bf16* src = EPI == 1 ? g.Y : g.R;
            f32x4 dz = {0.f, 0.f, 0.f, 0.f};
            if (tok < rows && src)
              dz = __builtin_convertvector(
                  *(const bf16x4*)(src + (m0 + tok) * N + n0 + 64 * wf + 32 * i + 8 * grp + 4 * hf), f32x4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x = acc[i][2 * p + jj][4 * grp + e];
              if (EPI == 1) {
                const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * x));
                v[e] = dz[e] * (sg * __builtin_fmaf(x, 1.0f - sg, 1.0f));
              } else {
                v[e] = x + dz[e];
              }
            }
          }
          const int q = 8 * wf + 4 * i + grp;
          wtile[r * 32 + 2 * (q ^ (r & 15)) + (hf ^ ((r >> 4) & 1))] =
              __builtin_bit_cast(u32x2, __builtin_convertvector(v, bf16x4));
        }
    }
    __syncthreads();
    // 128 rows x 16 granules; thread t takes granule t % 16 of rows t / 16 + 16 k
    const int q = tid & 15;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = (tid >> 4) + 16 * k;
      const int rl = r & 63;
      const int tok = 128 * (r >> 6) + 32 * (2 * p + (rl >> 5)) + (rl & 31);  // within the tile
      const u32x2* rtile = (const u32x2*)(r < 64 ? sX0 : sX1);
      const u32x4 c = *(const u32x4*)(rtile + rl * 32 + 2 * (q ^ (rl & 15)));
      const u32x4 o = ((rl >> 4) & 1) ? u32x4{c[2], c[3], c[0], c[1]} : c;
      __builtin_amdgcn_raw_buffer_store_b128(o, yrs, (uint32_t)(tok * N + n0 + 8 * q) * 2u, 0, 0);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------
// f2: 64 tokens x (up to) 512 output features per workgroup, four waves of 128 features x 64
// tokens, wider models in 512-feature chunks.  K (= H dv) is staged 32 deep through two LDS
// buffers, from two register sets one slice ahead: the W2 slice (512 rows x 32) and the gated
// operand slice (64 tokens x 32), which the staging threads compute from O and U on the way,
// ((o - mean) rstd gamma + beta) u, so the gated activations never go to HBM.  The token's
// LayerNorm statistics come from the attention's per-head (mean, M2) pairs (Chan et al.'s
// pairwise combination).  The outputs leave through LDS as whole rows, the residual added there.

constexpr int kF2Tok = 64;
constexpr int kF2K = 32;
constexpr int kF2Threads = 256;
constexpr int kF2MaxHeads = 16;  // heads whose statistics f2 combines (H d_v <= 1024, d_v >= 64)

struct F2Args {
  const bf16* O;        // attention output [M][HV]
  const f32x4* ostats;  // [M][H]: offset m, mean and M2 of each head's d_v values of O
                        // (O holds the bf16 deviations from m)
  const bf16* U;        // gate, row stride u_stride
  int64_t u_stride;
  const float* gamma;   // [HV] or null
  const float* beta;    // [HV] or null
  float eps;
  const bf16* W;        // [N][HV]
  const float* bias;    // [N] or null
  const bf16* R;        // residual [M][N] or null
  bf16* Y;              // [M][N]
  int64_t M;
  int32_t N, HV, H, dv;
  int32_t n_begin, n_end;  // output features of this launch, in chunks of 128 NI
  // fused boundary (FUSE): the next layer's f1, Zn = SiLU(Y W1n^T + b1n) [M][N1n], from the Y
  // tile kept in LDS
  const bf16* W1n;      // [N1n][N]
  const float* b1n;     // [N1n] or null
  bf16* Zn;
  int32_t N1n;
};

// Fused boundary: the Y tile (64 tokens x 512 features, bf16) kept in LDS for the next layer's
// f1.  16-byte chunk c of row r at c ^ (r & 15), so 16 lanes that read one chunk of 16
// consecutive rows (1 KiB apart) touch 16 distinct bank groups.
__device__ __forceinline__ int y_off(int row, int chunk) { return row * 512 + ((chunk ^ (row & 15)) << 3); }

// NI: 32-feature blocks per wave (chunk = 128 NI features)
//
// FUSE (the single operator between two attentions of a layer stack, NI = 4, N = 512): after Y
// is stored, the workgroup also keeps its bf16 Y tile in LDS and computes the next layer's
// Zn = SiLU(Y W1n^T + b1n) for its 64 tokens in 512-feature chunks, streaming W1n through the
// same staging buffers.  The products run in f1's order (bias first, then 16-deep k-steps in
// increasing k) and f1's SiLU expression, so Zn is bit-identical to f1 on the stored Y.
template <int NI, bool FUSE>
__global__ __launch_bounds__(kF2Threads, 2) void f2_kernel(F2Args g) {
  constexpr int CH = 128 * NI;                  // features per chunk
  constexpr int WEL = CH * kF2K, AEL = kF2Tok * kF2K;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * (WEL + AEL)];
  __shared__ __attribute__((aligned(16))) bf16 sY[FUSE ? kF2Tok * 512 : 8];
  // gamma and beta of every feature (1 and 0 when absent), staged once: the slices read them
  // from LDS instead of waiting on a memory round trip each
  __shared__ __attribute__((aligned(16))) float sgb[2 * kF2MaxHeads * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int HV = g.HV, N = g.N;
  const int64_t M = g.M;
  const int64_t m0 = (int64_t)blockIdx.x * kF2Tok;
  const uint32_t kb = 2u * (uint32_t)HV;  // bytes per O / W2 row
  const int64_t nrow = M - m0 < kF2Tok ? M - m0 : kF2Tok;

  // staging roles: chunk sch of W2 rows srow + 64 u and of operand row srow (= token)
  const int srow = tid >> 2, sch = tid & 3;
  const int lofs = f1_off(srow, sch);  // rows srow + 64 u share the swizzle

  // LayerNorm statistics of token srow: mean = mean of the head means; M2 = sum of the head M2
  // plus dv x the squared deviations of the head means (rows past M give zeros)
  float mean, rstd;
  {
    const int64_t t = m0 + srow;
    const int H = g.H;
    const f32x4* st = g.ostats + (t < M ? t : 0) * H;
    // all heads' entries in one round of loads (at most kF2MaxHeads), then combined
    float hm[kF2MaxHeads], h2[kF2MaxHeads];
#pragma unroll
    for (int hh = 0; hh < kF2MaxHeads; ++hh) {
      const f32x4 v = hh < H ? st[hh] : f32x4{0.f, 0.f, 0.f, 0.f};
      hm[hh] = v[1];
      h2[hh] = v[2];
    }
    float hq = 0.f, sm = 0.f;
#pragma unroll
    for (int hh = 0; hh < kF2MaxHeads; ++hh) {
      sm += hm[hh];
      hq += h2[hh];
    }
    mean = sm / (float)H;
    float dev = 0.f;
#pragma unroll
    for (int hh = 0; hh < kF2MaxHeads; ++hh)
      if (hh < H) dev += (hm[hh] - mean) * (hm[hh] - mean);
    rstd = 1.0f / sqrtf((hq + (float)g.dv * dev) / (float)HV + g.eps);
  }
  // each head's offset m (O stores value - m), read per slice: slice kt lies in head kt kF2K / dv
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.ostats + m0 * g.H), (short)0, (int)(nrow * g.H * 16), 0x00020000);
  // O and U rows through descriptors bounded at the block's last token (zeros past M)
  const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.O + m0 * HV), (short)0, (int)(nrow * kb), 0x00020000);
  const __amdgpu_buffer_rsrc_t urs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.U + m0 * g.u_stride), (short)0, (int)(nrow * g.u_stride * 2), 0x00020000);
  const uint32_t voff_o = (uint32_t)srow * kb + 16u * sch;
  const uint32_t voff_u = (uint32_t)srow * (uint32_t)g.u_stride * 2u + 16u * sch;
  for (int i = tid; i < HV; i += kF2Threads) {
    sgb[2 * i] = g.gamma ? g.gamma[i] : 1.0f;
    sgb[2 * i + 1] = g.beta ? g.beta[i] : 0.0f;
  }
  __syncthreads();
  const __amdgpu_buffer_rsrc_t biasrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.bias, (short)0, g.bias ? 4 * N : 0, 0x00020000);

  auto sw = [&](int buf) { return smem + buf * (WEL + AEL); };
  auto sa = [&](int buf) { return smem + buf * (WEL + AEL) + WEL; };

  for (int n0 = g.n_begin; n0 < g.n_end; n0 += CH) {
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(g.W + (int64_t)n0 * HV), (short)0, (int)(CH * kb), 0x00020000);
    const int nk = HV / kF2K;
    u32x4 wr[2 * NI], orr, urr;
    float moff = 0.f;
    auto gload = [&](int kt) {
      moff = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
          srs, 16u * (uint32_t)(srow * g.H + (kt * kF2K) / g.dv), 0, 0));
      const uint32_t k0 = 2u * (uint32_t)kt * kF2K;
#pragma unroll
      for (int u = 0; u < 2 * NI; ++u)
        wr[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              wrs, voff_o + 64u * u * kb, k0, 0));
      orr = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ors, voff_o, k0, 0));
      urr = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(urs, voff_u, k0, 0));
    };
    // gamma / beta of the slice's 8 k-values of this thread, as (gamma, beta) pairs from LDS
    auto lstore = [&](int buf, int kt) {
      const f32x4* gb = (const f32x4*)(sgb + 2 * (kt * kF2K + 8 * sch));
      f32x4 gbv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) gbv[q] = gb[q];
#pragma unroll
      for (int u = 0; u < 2 * NI; ++u) *(u32x4*)(sw(buf) + lofs + 64 * u * kF2K) = wr[u];
      const bf16x8 o8 = __builtin_bit_cast(bf16x8, orr);
      const bf16x8 u8 = __builtin_bit_cast(bf16x8, urr);
      const float shift = moff - mean;
      f32x8 y;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gm = gbv[e >> 1][2 * (e & 1)], bt = gbv[e >> 1][2 * (e & 1) + 1];
        y[e] = (((float)o8[e] + shift) * rstd * gm + bt) * (float)u8[e];
      }
      *(bf16x8*)(sa(buf) + lofs) = __builtin_convertvector(y, bf16x8);
    };

    // acc[i][j] register r -> feature n0 + 32 NI wave + 32 i + 8 (r / 4) + 4 hf + r % 4, token
    // 32 j + l32; the accumulators start at the bias
    f32x16 acc[NI][2];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const f32x4 b4 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
            biasrs, 4u * (uint32_t)(n0 + 32 * NI * wave + 4 * hf), 4u * (32 * i + 8 * grp), 0));
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][4 * grp + e] = b4[e];
      }
    auto compute = [&](int buf) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 a[NI], b[2];
#pragma unroll
        for (int i = 0; i < NI; ++i)
          a[i] = *(const bf16x8*)(sw(buf) + f1_off(32 * NI * wave + 32 * i + l32, 2 * ks + hf));
#pragma unroll
        for (int j = 0; j < 2; ++j) b[j] = *(const bf16x8*)(sa(buf) + f1_off(32 * j + l32, 2 * ks + hf));
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
    };
    // slice kt in LDS buffer kt % 2; slice kt + 1's loads are in flight during slice kt
    gload(0);
    lstore(0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) gload(kt + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(buf);
      if (kt + 1 < nk) lstore(buf ^ 1, kt + 1);
      __syncthreads();
    }

    // epilogue through LDS in two passes of 64 NI features (waves 2 p, 2 p + 1), as an fp32 tile
    // of 64 token rows: granule (4 features) q of row lr sits at q ^ (lr & 15).  The residual is
    // added to the fp32 sum, so each output is rounded once.
    const bf16* __restrict__ R = g.R;
    bf16* __restrict__ Y = g.Y;
    const __amdgpu_buffer_rsrc_t rrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(R ? R + m0 * N : nullptr), (short)0, R ? (int)(nrow * N * 2) : 0, 0x00020000);
    // output rows past M fall outside the descriptor and are dropped
    const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Y + m0 * N), (short)0, (int)(nrow * N * 2), 0x00020000);
    f32x4* tile = (f32x4*)smem;        // [64 rows][16 NI granules]
    constexpr int GPR = 16 * NI;       // granules per row
    constexpr int NPC = 64 * 8 * NI / kF2Threads;  // 8-output pieces per thread and pass
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if ((wave >> 1) == p) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int lr = 32 * j + l32;
#pragma unroll
          for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
              const int q = 8 * NI * (wave & 1) + 8 * i + 2 * grp + hf;
              tile[lr * GPR + (q ^ (lr & 15))] =
                  f32x4{acc[i][j][4 * grp], acc[i][j][4 * grp + 1], acc[i][j][4 * grp + 2],
                        acc[i][j][4 * grp + 3]};
            }
        }
      }
      __syncthreads();
      // piece c = t + 256 k: row c / (8 NI), features 8 (c % (8 NI)) .. + 7 of the pass
      const int fp = n0 + 64 * NI * p;
      u32x4 rv[NPC];
#pragma unroll
      for (int k = 0; k < NPC; ++k) {
        const int c = tid + kF2Threads * k, lr = c / (8 * NI), pc = c % (8 * NI);
        rv[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rrs, (uint32_t)(lr * N + fp + 8 * pc) * 2u, 0, 0));
      }
#pragma unroll
      for (int k = 0; k < NPC; ++k) {
        const int c = tid + kF2Threads * k, lr = c / (8 * NI), pc = c % (8 * NI);
        const f32x4 a0 = tile[lr * GPR + ((2 * pc) ^ (lr & 15))];
        const f32x4 a1 = tile[lr * GPR + ((2 * pc + 1) ^ (lr & 15))];
        const f32x8 r8 = __builtin_convertvector(__builtin_bit_cast(bf16x8, rv[k]), f32x8);
        f32x8 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = a0[e] + r8[e];
          v[e + 4] = a1[e] + r8[e + 4];
        }
        const u32x4 y8 = __builtin_bit_cast(u32x4, __builtin_convertvector(v, bf16x8));
        __builtin_amdgcn_raw_buffer_store_b128(y8, yrs, (uint32_t)(lr * N + fp + 8 * pc) * 2u, 0, 0);
        if (FUSE) *(u32x4*)(sY + y_off(lr, (fp >> 3) + pc)) = y8;
      }
      __syncthreads();  // the tile is the next pass's / chunk's staging area
    }
  }

  if (FUSE) {
    // ---- the next layer's f1 on the Y tile: K = 512 in 32-deep slices, W1n through the
    // staging buffers (rows srow + 64 u, chunk sch), 512 output features per chunk ----
    constexpr int K1 = 512;
    const uint32_t kb1 = 2u * K1;
    const int N1 = g.N1n;
    const __amdgpu_buffer_rsrc_t b1rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)g.b1n, (short)0, g.b1n ? 4 * N1 : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(g.Zn + m0 * N1), (short)0, (int)min(nrow * N1 * 2, (int64_t)0x7fffffff), 0x00020000);
    auto sw1 = [&](int buf) { return smem + buf * (WEL + AEL); };
    for (int n1 = 0; n1 < N1; n1 += CH) {
      const __amdgpu_buffer_rsrc_t w1rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(g.W1n + (int64_t)n1 * K1), (short)0, (int)(CH * kb1), 0x00020000);
      u32x4 wr[2 * NI];
      auto gload1 = [&](int kt) {
        const uint32_t k0 = 2u * (uint32_t)kt * kF2K;
#pragma unroll
        for (int u = 0; u < 2 * NI; ++u)
          wr[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                w1rs, (uint32_t)srow * kb1 + 16u * sch + 64u * u * kb1, k0, 0));
      };
      auto lstore1 = [&](int buf) {
#pragma unroll
        for (int u = 0; u < 2 * NI; ++u) *(u32x4*)(sw1(buf) + lofs + 64 * u * kF2K) = wr[u];
      };
      // acc[i][j] register r -> feature n1 + 32 NI wave + 32 i + 8 (r / 4) + 4 hf + r % 4, token
      // 32 j + l32; the accumulators start at the bias
      f32x16 acc[NI][2];
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const f32x4 b4 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
              b1rs, 4u * (uint32_t)(n1 + 32 * NI * wave + 4 * hf), 4u * (32 * i + 8 * grp), 0));
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][4 * grp + e] = b4[e];
        }
      auto compute1 = [&](int buf, int kt) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8 a[NI], b[2];
#pragma unroll
          for (int i = 0; i < NI; ++i)
            a[i] = *(const bf16x8*)(sw1(buf) + f1_off(32 * NI * wave + 32 * i + l32, 2 * ks + hf));
#pragma unroll
          for (int j = 0; j < 2; ++j) b[j] = *(const bf16x8*)(sY + y_off(32 * j + l32, 4 * kt + 2 * ks + hf));
#pragma unroll
          for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
      };
      constexpr int nk1 = K1 / kF2K;
      gload1(0);
      lstore1(0);
      __syncthreads();
      for (int kt = 0; kt < nk1; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk1) gload1(kt + 1);
        __builtin_amdgcn_sched_barrier(0);
        compute1(buf, kt);
        if (kt + 1 < nk1) lstore1(buf ^ 1);
        __syncthreads();
      }
      // epilogue: SiLU, rounded once, through the fp32 tile as in the f2 part
      f32x4* tile = (f32x4*)smem;
      constexpr int GPR = 16 * NI;
      constexpr int NPC = 64 * 8 * NI / kF2Threads;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        if ((wave >> 1) == p) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int lr = 32 * j + l32;
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
              for (int grp = 0; grp < 4; ++grp) {
                const int q = 8 * NI * (wave & 1) + 8 * i + 2 * grp + hf;
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const float x = acc[i][j][4 * grp + e];
                  v[e] = x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * x));
                }
                tile[lr * GPR + (q ^ (lr & 15))] = v;
              }
          }
        }
        __syncthreads();
        const int fp = n1 + 64 * NI * p;
#pragma unroll
        for (int k = 0; k < NPC; ++k) {
          const int c = tid + kF2Threads * k, lr = c / (8 * NI), pc = c % (8 * NI);
          const f32x4 a0 = tile[lr * GPR + ((2 * pc) ^ (lr & 15))];
          const f32x4 a1 = tile[lr * GPR + ((2 * pc + 1) ^ (lr & 15))];
          const f32x8 v = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(u32x4, __builtin_convertvector(v, bf16x8)), zrs,
              (uint32_t)(lr * N1 + fp + 8 * pc) * 2u, 0, 0);
        }
        __syncthreads();
      }
    }
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
                               int32_t N, int32_t K, hipStream_t stream, bool silu_bwd,
                               const bf16* resid, bool plain) {
  if (N % kF1Feat || K % kF1K || K <= 0) return hipErrorInvalidValue;
  if ((int64_t)kF1Tok * N * 2 > 0x7fffffff) return hipErrorInvalidValue;
  if ((int64_t)kF1Tok * 2 * K > 0x7fffffff || (int64_t)kF1Feat * 2 * K > 0x7fffffff)
    return hipErrorInvalidValue;
  if (M <= 0) return hipSuccess;
  const int64_t tiles = (int64_t)(N / kF1Feat) * ((M + kF1Tok - 1) / kF1Tok);
  if (tiles > 0x7ffffff0) return hipErrorInvalidValue;
  F1Args g{};
  g.X = x; g.W = w1; g.bias = b1; g.Y = z; g.R = resid; g.M = M; g.N = N; g.K = K;
  g.tiles = (int32_t)tiles;
  const unsigned grid = (unsigned)((tiles + 7) / 8 * 8);
  if (plain) {
    hipLaunchKernelGGL((f1_kernel<0, 2>), dim3(grid), dim3(kF1Threads), 0, stream, g);
  } else if (silu_bwd) {
    if (K == 512) hipLaunchKernelGGL((f1_kernel<16, 1>), dim3(grid), dim3(kF1Threads), 0, stream, g);
    else if (K == 256) hipLaunchKernelGGL((f1_kernel<8, 1>), dim3(grid), dim3(kF1Threads), 0, stream, g);
    else hipLaunchKernelGGL((f1_kernel<0, 1>), dim3(grid), dim3(kF1Threads), 0, stream, g);
  } else {
    if (K == 512) hipLaunchKernelGGL((f1_kernel<16, 0>), dim3(grid), dim3(kF1Threads), 0, stream, g);
    else if (K == 256) hipLaunchKernelGGL((f1_kernel<8, 0>), dim3(grid), dim3(kF1Threads), 0, stream, g);
    else hipLaunchKernelGGL((f1_kernel<0, 0>), dim3(grid), dim3(kF1Threads), 0, stream, g);
  }
  return hipGetLastError();
}

// dst[c][r] = src[r][c] for a bf16 [R][C] matrix (both dense), through 32 x 32 LDS tiles
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16* __restrict__ src,
                                                             bf16* __restrict__ dst, int32_t R,
                                                             int32_t C) {
  __shared__ bf16 t[32][33];
  const int c0 = 32 * blockIdx.x, r0 = 32 * blockIdx.y;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int k = ty; k < 32; k += 8)
    if (r0 + k < R && c0 + tx < C) t[k][tx] = src[(int64_t)(r0 + k) * C + c0 + tx];
  __syncthreads();
  for (int k = ty; k < 32; k += 8)
    if (c0 + k < C && r0 + tx < R) dst[(int64_t)(c0 + k) * R + r0 + tx] = t[tx][k];
}

hipError_t launch_transpose_bf16(const bf16* src, bf16* dst, int32_t R, int32_t C,
                                 hipStream_t stream) {
  if (R <= 0 || C <= 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3((C + 31) / 32, (R + 31) / 32), dim3(256), 0,
                     stream, src, dst, R, C);
  return hipGetLastError();
}

hipError_t launch_ln_gate_f2(const bf16* o, const f32x4* ostats, const bf16* u,
                             int64_t u_stride, const float* gamma, const float* beta, float eps,
                             const bf16* w2, const float* b2, const bf16* x, bf16* y, int64_t M,
                             int32_t D, int32_t H, int32_t dv, hipStream_t stream) {
  const int32_t HV = H * dv;
  if (D % 128 || D <= 0 || HV % (2 * kF2K) || HV <= 0 || u_stride % 8 || u_stride < HV || H > kF2MaxHeads)
    return hipErrorInvalidValue;
  if ((int64_t)kF2Tok * 2 * u_stride > 0x7fffffff || (int64_t)512 * 2 * HV > 0x7fffffff)
    return hipErrorInvalidValue;
  if (M <= 0) return hipSuccess;
  F2Args g{};
  g.O = o; g.ostats = ostats; g.U = u; g.u_stride = u_stride; g.gamma = gamma; g.beta = beta;
  g.eps = eps; g.W = w2; g.bias = b2; g.R = x; g.Y = y; g.M = M; g.N = D; g.HV = HV; g.H = H;
  g.dv = dv;
  const dim3 grid((unsigned)((M + kF2Tok - 1) / kF2Tok));
  // chunks of 512 features, then one launch for a narrower remainder
  const int32_t full = D / 512 * 512;
  if (full > 0) {
    g.n_begin = 0; g.n_end = full;
    hipLaunchKernelGGL((f2_kernel<4, false>), grid, dim3(kF2Threads), 0, stream, g);
  }
  if (D > full) {
    g.n_begin = full; g.n_end = D;
    switch ((D - full) / 128) {
      case 1: hipLaunchKernelGGL((f2_kernel<1, false>), grid, dim3(kF2Threads), 0, stream, g); break;
      case 2: hipLaunchKernelGGL((f2_kernel<2, false>), grid, dim3(kF2Threads), 0, stream, g); break;
      default: hipLaunchKernelGGL((f2_kernel<3, false>), grid, dim3(kF2Threads), 0, stream, g); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_ln_gate_f2_f1(const bf16* o, const f32x4* ostats, const bf16* u,
                                int64_t u_stride, const float* gamma, const float* beta, float eps,
                                const bf16* w2, const float* b2, const bf16* x, bf16* y,
                                const bf16* w1n, const float* b1n, bf16* zn, int32_t N1n,
                                int64_t M, int32_t D, int32_t H, int32_t dv, hipStream_t stream) {
  const int32_t HV = H * dv;
  if (D != 512 || HV % (2 * kF2K) || HV <= 0 || u_stride % 8 || u_stride < HV || H > kF2MaxHeads ||
      N1n <= 0 || N1n % 512)
    return hipErrorInvalidValue;
  if ((int64_t)kF2Tok * 2 * u_stride > 0x7fffffff || (int64_t)512 * 2 * HV > 0x7fffffff)
    return hipErrorInvalidValue;
  if (M <= 0) return hipSuccess;
  F2Args g{};
  g.O = o; g.ostats = ostats; g.U = u; g.u_stride = u_stride; g.gamma = gamma; g.beta = beta;
  g.eps = eps; g.W = w2; g.bias = b2; g.R = x; g.Y = y; g.M = M; g.N = D; g.HV = HV; g.H = H;
  g.dv = dv; g.n_begin = 0; g.n_end = D;
  g.W1n = w1n; g.b1n = b1n; g.Zn = zn; g.N1n = N1n;
  hipLaunchKernelGGL((f2_kernel<4, true>), dim3((unsigned)((M + kF2Tok - 1) / kF2Tok)),
                     dim3(kF2Threads), 0, stream, g);
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
