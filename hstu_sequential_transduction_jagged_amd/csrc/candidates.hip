// Candidate scoring over a cached user history (M-FALCON, "Actions Speak Louder than Words"
// reading notes §3.6; candidates of one request share one position, GenRank article part (2)).
//
// For user b with n_b history tokens (positions 0 .. n_b - 1) and candidates c (each at
// position n_b, the position right after the history), head h:
//
//   O[c] = out_scale * ( sum_{j < n_b} SiLU(alpha <q_c, k_j> + bias(n_b - j, t_c - t_j)) v_j
//                        + SiLU(alpha <q_c, k_c> + bias(0, 0)) v_c )
//
// i.e. every candidate sees the whole history and itself but no other candidate: the row that
// eq. (2) gives a candidate appended alone after the history, computed for many candidates at
// once.  The history's K and V are inputs (the cache), so a caller scores candidates in
// micro-batches by calling once per batch with the same history.
//
// bf16, d_qk = d_v = 64.  Work item = (user, head, chunk of 1024 history keys, 128 candidates):
// 4 waves x 32 candidate rows.  A history longer than one chunk is split over several items
// whose fp32 sums a second kernel adds in chunk order (deterministic).  Workgroups are
// persistent: each walks a fixed sequence of items and skips the empty ones (chunks past a
// user's history, candidate tiles past its candidates), so the grid carries no idle
// workgroups.  Key tiles of 64 are moved global -> LDS directly (buffer loads with the LDS
// bit) through a ring of 4 stages, in pairs of tiles with one barrier per pair.  Per tile
// S^T = K Q^T on v_mfma_f32_32x32x16_bf16, the SiLU weights stay in registers as the B operand
// of O^T += V^T P^T, V^T is read with transposing LDS reads; the self term is the
// accumulator's starting value.
#include <algorithm>

#include "hstu_internal.h"

namespace hstu {
namespace {

constexpr int kCWaves = 4;
constexpr int kCThreads = 64 * kCWaves;
constexpr int kCRows = 32 * kCWaves;  // candidates per work item
constexpr int kCKB = 64;              // history keys per tile
constexpr int kCD = 64;
constexpr int kCChunk = 1024;         // history keys per work item
constexpr int kCWgPerCu = 2;

struct CandArgs {
  const int32_t* hist_offsets;  // [B + 1]
  const int32_t* cand_offsets;  // [B + 1]
  const bf16* q;                // candidate queries, row stride q_stride
  const bf16* kc;               // candidate keys
  const bf16* vc;               // candidate values
  const bf16* kh;               // history keys
  const bf16* vh;               // history values
  int64_t q_stride, kc_stride, vc_stride, kh_stride, vh_stride;
  bf16* o;                      // [total candidates, H, 64]
  float* partial;               // [max_chunks, total candidates, H, 64] (split histories)
  const TimeStat* stats;        // per 32-key block of the history: min / max timestamp
  const int32_t* unit_list;     // valid units (b H + h) * max_chunks + chunk, count at [-1]
  const int64_t* th;            // history timestamps (position + time bias)
  const int64_t* tc;            // candidate timestamps
  BiasArgs bias;
  int64_t total_cand;
  int32_t B, H, cand_tiles, max_hist, max_chunks, units, items;
  float alpha, out_scale;
};

// One ring stage: a 64-key tile of K and V (row = key, 64 bf16, unpadded), the keys'
// timestamps and the two 32-key halves' timestamp extremes.  The 16-byte chunk c of row r sits
// at chunk position c ^ cswz_r(r), cswz_r(r) = ((r >> 1) & 1) << 2 | ((r >> 2) & 3), which
// serves all three access patterns without bank conflicts on the 64 banks: the K operand reads
// (16 lanes read one chunk of 16 consecutive rows: even and odd rows take the two 64-byte
// halves and cswz_r is a bijection on each), the transposing V reads (32 lanes read chunks
// 0..3 or 4..7 of 4 consecutive rows: rows r and r + 2 differ in bit 2 of cswz_r) and the
// transfers (whole rows).  (A plain c ^ (r % 8) leaves the transposing reads conflicted.)
struct __attribute__((aligned(16))) CandStage {
  __attribute__((aligned(16))) bf16 k[kCKB * kCD];
  __attribute__((aligned(16))) bf16 v[kCKB * kCD];
  __attribute__((aligned(16))) int64_t kt[kCKB];
  __attribute__((aligned(16))) uint32_t st[128];  // dwords 0..7: TimeStat of halves 0, 1
};

__device__ __forceinline__ int cswz_r(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
// element offset of (row, 16-byte chunk) in a swizzled tile
__device__ __forceinline__ int cswz(int row, int chunk) { return row * kCD + ((chunk ^ cswz_r(row)) << 3); }

typedef long long i64x2 __attribute__((ext_vector_type(2)));

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

// KIND: 0 no bias, 1 position + time tables, 2 ALiBi.
//
// Per 32x32 tile (one wave's candidates x 32 keys) the wave picks how to evaluate the weights
// w(y) = 2y / (1 + 2^y), y = -log2(e) (alpha s + bias), once the scores s are known (D below
// is |alpha log2(e)| max|s| over the tile):
//   - one bias value for the whole tile (no bias; or the position bucket saturated at P - 1
//     for every key and one time bucket for every (candidate, key) pair, decided exactly from
//     the extreme timestamps): the bias and the Taylor coefficients of w around it come from
//     a per-time-bucket table, and w = a0 + a1 s + a2 s^2 when D is small enough, else the
//     polynomial or the exact w with that one bias;
//   - two time buckets with saturated position: one compare per element picks the bias;
//   - otherwise the bias of every element (position table + time table gathered by bucket,
//     or the ALiBi term).
// The polynomial w is used when D plus the largest |bias| of the tile stays within its range.
// Keys at or past n are staged as zero rows of K and V, so their weights (finite, as every
// bias value is) multiply zeros and need no mask.
template <int KIND>
__global__ __launch_bounds__(kCThreads, kCWgPerCu) void attn_cand_bf16_kernel(CandArgs a) {
  // stages as arrays of their own: the compiler then knows which stage a transfer writes
  __shared__ CandStage st0, st1, st2, st3;
  __shared__ __attribute__((aligned(16))) float tay[kMaxTimeBuckets][4];  // c, a0, a1, a2
  __shared__ float wpos_s[kMaxPosBuckets];     // -log2(e) * w_pos[h]
  __shared__ float wtime_s[kMaxTimeBuckets];   // -log2(e) * w_time[h]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int H = a.H;
  constexpr float kL2e = kLog2e;
  const float cq = -a.alpha * kL2e;
  const int Pm1 = a.bias.num_pos - 1, NTm1 = a.bias.num_time - 1;
  // transfers per wave and tile: K and V 2 each, plus (position + time bias) the timestamps
  // (waves 0, 1), the halves' extremes (wave 2) and one out of range (wave 3)
  constexpr int kDma = KIND == 1 ? 5 : 4;
  const uint32_t kstride_b = (uint32_t)a.kh_stride * 2u, vstride_b = (uint32_t)a.vh_stride * 2u;
  // lane offsets of the K / V transfers: instruction u of wave w fills rows 8 (w + 4 u) ..
  // + 7; lane p writes row 8 (w + 4 u) + p / 8 at chunk position p % 8, i.e. global chunk
  // (p % 8) ^ cswz_r(row)
  uint32_t kvo[2], vvo[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t row = 8u * (uint32_t)(wave + 4 * u) + (uint32_t)(lane >> 3);
    const uint32_t ch = 16u * (uint32_t)((lane & 7) ^ cswz_r((int)row));
    kvo[u] = row * kstride_b + ch;
    vvo[u] = row * vstride_b + ch;
  }
  // 4-byte transfers: waves 0, 1 the timestamps of keys 32 w .. 32 w + 31 (lane p: key
  // 32 w + p / 2, word p % 2); wave 2 the two halves' TimeStat (lanes 0..7); wave 3 none
  const uint32_t mvo = wave < 2 ? 256u * (uint32_t)wave + 4u * (uint32_t)lane
                     : (wave == 2 && lane < 8) ? 512u * (uint32_t)(lane >> 2) + 4u * (uint32_t)(lane & 3)
                     : 0x80000000u;

  enum { kExact = 0, kPoly = 1, kTaylor = 2 };
  auto w_exact = [&](float y) {
    return y * __builtin_amdgcn_rcpf(__builtin_fmaf(__builtin_amdgcn_exp2f(y), 0.5f, 0.5f));
  };
  auto w_poly = [&](float y) {
    const float u = y * y;
    return __builtin_fmaf(-u, __builtin_fmaf(__builtin_fmaf(kP2, u, kP1), u, kP0), y);
  };
  // transposing V reads: lane i of each 16-lane group reads keys 4 hf + (i % 16) / 4 (+ the
  // group's offset) at d 16 ((lane / 16) % 2) + 4 (lane % 4) .. + 3 (+ 32 db)
  const int vtr_row0 = 4 * hf + ((lane & 15) >> 2);
  const int vtr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // items: the list holds the valid units (user, head, chunk); unit k goes to XCD k % 8
  // (workgroups are dealt round-robin over the 8 XCDs and the grid is a multiple of 8), and
  // the workgroups of an XCD walk its units' candidate tiles in turn, so the tiles reading
  // one chunk of K / V share that XCD's L2 and every workgroup gets a similar number of
  // similar items
  const int n_units = a.unit_list[-1];
  const int x = blockIdx.x & 7, per_x = gridDim.x >> 3;
  const int x_units = n_units > x ? (n_units - x + 7) >> 3 : 0;
  for (int r = blockIdx.x >> 3; r < x_units * a.cand_tiles; r += per_x) {
    const int ct = r % a.cand_tiles;
    const int code = a.unit_list[8 * (r / a.cand_tiles) + x];
    const int bh = code / a.max_chunks, chunk = code - bh * a.max_chunks;
    const int b = bh / H, h = bh - b * H;
    const int64_t hb = a.hist_offsets[b], cb = a.cand_offsets[b];
    // history length = the candidates' position; lengths past max_hist / max_cand break the
    // calling contract and are cut there so that every access stays inside the rows addressed
    const int n = min(a.hist_offsets[b + 1] - (int)hb, a.max_hist);
    const int m = min(a.cand_offsets[b + 1] - (int)cb, a.cand_tiles * kCRows);
    const int n_chunks = max((n + kCChunk - 1) / kCChunk, 1);
    if (ct * kCRows >= m || chunk >= n_chunks) continue;
    const int jb = chunk * kCChunk;       // first key of this chunk
    const int je = min(n, jb + kCChunk);  // one past its last key
    const int n_tiles = (je - jb + kCKB - 1) / kCKB;
    const int crow = ct * kCRows + 32 * wave + l32;  // this lane's candidate
    const bool cvalid = crow < m;
    const int64_t ctok = cb + min(crow, m - 1);

    // ---- register loads of the item, issued before the tile transfers so that the wait
    // below leaves only transfers outstanding ----
    bf16x8 qop[4], kself[4];
    bf16x4 vself[8];
    {
      const bf16* qs = a.q + ctok * a.q_stride + (int64_t)h * kCD + 8 * hf;
      const bf16* ks = a.kc + ctok * a.kc_stride + (int64_t)h * kCD + 8 * hf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qop[i] = *(const bf16x8*)(qs + 16 * i);
        kself[i] = *(const bf16x8*)(ks + 16 * i);
      }
      // v_c in the accumulator's order: group g of oacc[db] holds d = 32 db + 8 g + 4 hf ..
      const bf16* vs = a.vc + ctok * a.vc_stride + (int64_t)h * kCD + 4 * hf;
#pragma unroll
      for (int i = 0; i < 8; ++i) vself[i] = *(const bf16x4*)(vs + 8 * i);
    }
    int64_t tq = 0;
    float wtv = 0.f, wpv[4] = {0.f, 0.f, 0.f, 0.f}, wp_last = 0.f, wp_first = 0.f, wt_first = 0.f;
    float slope = 0.f;
    if (KIND == 2) slope = a.bias.slopes ? a.bias.slopes[h] : default_alibi_slope(h, H);
    if (KIND == 1) {
      tq = a.tc[ctok];
      const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.bias.w_pos + (int64_t)h * a.bias.pos_stride), (short)0, 4 * a.bias.num_pos, 0x00020000);
      const __amdgpu_buffer_rsrc_t trs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.bias.w_time + (int64_t)h * a.bias.time_stride), (short)0, 4 * a.bias.num_time, 0x00020000);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        wpv[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(prs, 4u * (uint32_t)(tid + kCThreads * i), 0, 0));
      wtv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(trs, 4u * (uint32_t)tid, 0, 0));
      // the entries of bucket P - 1 and of the self term's buckets (0, 0)
      wp_last = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(prs, 4u * (uint32_t)Pm1, 0, 0));
      wp_first = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(prs, 0u, 0, 0));
      wt_first = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(trs, 0u, 0, 0));
    }

    // ---- tile transfers ----
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.kh + hb * a.kh_stride + (int64_t)h * kCD), (short)0,
        n > 0 ? (int)((uint32_t)(n - 1) * kstride_b + 2u * kCD) : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.vh + hb * a.vh_stride + (int64_t)h * kCD), (short)0,
        n > 0 ? (int)((uint32_t)(n - 1) * vstride_b + 2u * kCD) : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
        KIND == 1 ? (wave < 2 ? (void*)(a.th + hb) : (void*)(a.stats + hb)) : nullptr, (short)0,
        KIND == 1 ? (wave < 2 ? 8 * n : 16 * n) : 0, 0x00020000);
    // tile t into a stage (tiles past the last read out of range: zeros, no memory traffic)
    auto dma = [&](CandStage& stg, int t) __attribute__((always_inline)) {
      const bool real = t < n_tiles;
      const uint32_t j0 = (uint32_t)(jb + t * kCKB);
      // (wave-uniform; readfirstlane keeps the offsets in scalar registers)
      const uint32_t ksoff = __builtin_amdgcn_readfirstlane(real ? j0 * kstride_b : 0x7fffffffu);
      const uint32_t vsoff = __builtin_amdgcn_readfirstlane(real ? j0 * vstride_b : 0x7fffffffu);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr)(stg.k + 512 * (wave + 4 * u)), 16,
                                                 kvo[u], ksoff, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr)(stg.v + 512 * (wave + 4 * u)), 16,
                                                 vvo[u], vsoff, 0, 0);
      }
      if (KIND == 1) {
        const uint32_t msoff = __builtin_amdgcn_readfirstlane(real ? j0 * (wave < 2 ? 8u : 16u) : 0x7fffffffu);
        void* dst = wave < 2 ? (void*)(stg.kt + 32 * wave) : (void*)(stg.st + 64 * (wave - 2));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(mrs, (lds_ptr)dst, 4, mvo, msoff, 0, 0);
      }
    };
    dma(st0, 0);
    dma(st1, 1);

    // ---- per-item constants: the register loads have landed once at most the 2 tiles'
    // transfers are outstanding ----
    wait_vm<2 * kDma>();
    int64_t tq_min = 0, tq_max = 0;
    float ta0 = 0.f, ta1 = 0.f, ta2 = 0.f, slope_y = 0.f, cself = 0.f;
    if (KIND == 1) {
      int64_t mn = tq, mx = tq;
      half_minmax(mn, mx);
      tq_min = uniform_i64(mn);
      tq_max = uniform_i64(mx);
      if (tid < a.bias.num_time) {
        const float c = -kL2e * (wp_last + wtv);
        float x0, x1, x2;
        w_taylor_coeffs(c, cq, x0, x1, x2);
        *(f32x4*)(&tay[tid][0]) = f32x4{c, x0, x1, x2};
        wtime_s[tid] = -kL2e * wtv;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tid + kCThreads * i < a.bias.num_pos) wpos_s[tid + kCThreads * i] = -kL2e * wpv[i];
      cself = -kL2e * (wp_first + wt_first);
    } else if (KIND == 0) {
      w_taylor_coeffs(0.f, cq, ta0, ta1, ta2);
    } else {
      slope_y = kL2e * slope;
    }

    // ---- accumulator start: the self term (first chunk only), in fp32 ----
    f32x16 oacc[2];
    {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = __builtin_fmaf((float)qop[i][e], (float)kself[i][e], ss);
      ss += __shfl_xor(ss, 32, 64);
      const float wy = chunk == 0 ? w_exact(__builtin_fmaf(ss, cq, cself)) : 0.f;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) oacc[db][4 * g + e] = wy * (float)vself[4 * db + g][e];
    }

    // one 64-key tile from a stage
    auto compute = [&](const CandStage& stg, int t) __attribute__((always_inline)) {
#pragma unroll
      for (int hk = 0; hk < 2; ++hk) {
        const int j0h = jb + t * kCKB + 32 * hk;  // first key of this half
        if (j0h >= je) break;                      // uniform
        bf16x8 kop[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kop[ks] = *(const bf16x8*)(stg.k + cswz(32 * hk + l32, 2 * ks + hf));
        f32x16 sacc = {};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qop[ks], sacc, 0, 0, 0);
        // |y - bias| <= D over the tile (margin for the rounding of the bound)
        const float D = fabsf(cq) * 1.0001f * uniform_f32(wave_max_abs16(sacc));

        int mode = 3, path = kExact;  // mode 1: one bias; 2: two time buckets; 3: per element
        float c0 = 0.f, c1 = 0.f, A0 = ta0, A1 = ta1, A2 = ta2;
        int64_t tlim = 0;
        if (KIND == 0) {
          mode = 1;
          path = D <= kTaylorD ? kTaylor : D <= kPolyRange ? kPoly : kExact;
        } else if (KIND == 1) {
          const u32x4 e = *(const u32x4*)(&stg.st[4 * hk]);
          const int64_t kmin = uniform_i64((int64_t)(((uint64_t)e[1] << 32) | e[0]));
          const int64_t kmax = uniform_i64((int64_t)(((uint64_t)e[3] << 32) | e[2]));
          const int tlo = time_bucket(tq_min - kmax, NTm1), thi = time_bucket(tq_max - kmin, NTm1);
          const bool sat = n - min(j0h + 31, n - 1) >= Pm1;  // every key's position bucket is P - 1
          if (sat && thi <= tlo + 1) {
            const f32x4 lo = *(const f32x4*)(&tay[tlo][0]);
            c0 = uniform_f32(lo[0]);
            A0 = uniform_f32(lo[1]);
            A1 = uniform_f32(lo[2]);
            A2 = uniform_f32(lo[3]);
            float cabs = fabsf(c0);
            if (thi == tlo) {
              mode = 1;
            } else {
              // dt >= 2^thi - 1  <=>  t_k <= t_q - (2^thi - 1): the larger bucket's bias
              mode = 2;
              c1 = uniform_f32(tay[thi][0]);
              cabs = fmaxf(cabs, fabsf(c1));
              tlim = tq - (((int64_t)1 << thi) - 1);
            }
            path = (mode == 1 && D <= kTaylorD) ? kTaylor : D + cabs <= kPolyRange ? kPoly : kExact;
          }
        }

        // accumulator register 4 g + e holds key j0h + 8 g + 4 hf + e
        f32x16 w;
        if (mode == 1 && path == kTaylor) {
#pragma unroll
          for (int i = 0; i < 16; ++i) w[i] = __builtin_fmaf(__builtin_fmaf(A2, sacc[i], A1), sacc[i], A0);
        } else if (mode == 1) {
          if (path == kPoly) {
#pragma unroll
            for (int i = 0; i < 16; ++i) w[i] = w_poly(__builtin_fmaf(sacc[i], cq, c0));
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) w[i] = w_exact(__builtin_fmaf(sacc[i], cq, c0));
          }
        } else {
          f32x16 cb;
          const int dn = n - j0h - 4 * hf;  // n - j of register 0
          bool per_key = false;
          if (KIND == 1 && mode == 3) {
            // When every key of the half has one time bucket for all of the wave's candidates
            // (decided exactly from the candidates' extreme times; always so for candidates of
            // one request time) the bias depends on the key only: lane l computes it for key
            // j0h + l % 32 and the registers take theirs by lane shuffles.  Keys at or past n
            // meet zero V rows, whatever their bias.
            const int64_t tkl = stg.kt[32 * hk + l32];
            const int blo = time_bucket(tq_min - tkl, NTm1);
            const bool same = blo == time_bucket(tq_max - tkl, NTm1) || j0h + l32 >= n;
            per_key = __builtin_amdgcn_ballot_w64(!same) == 0;
            if (per_key) {
              const float bk = wpos_s[max(min(n - j0h - l32, Pm1), 0)] + wtime_s[blo];
#pragma unroll
              for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int e = 0; e < 4; ++e) cb[4 * g + e] = __shfl(bk, 8 * g + 4 * hf + e, 64);
            }
          }
#pragma unroll
          for (int g = 0; g < 4 && !per_key; ++g) {
            const int jl = 32 * hk + 8 * g + 4 * hf;
            if (KIND == 2) {
              const float base = slope_y * (float)(dn - 8 * g);
#pragma unroll
              for (int e = 0; e < 4; ++e) cb[4 * g + e] = __builtin_fmaf(-slope_y, (float)e, base);
            } else {
              const i64x2 t01 = *(const i64x2*)(&stg.kt[jl]);
              const i64x2 t23 = *(const i64x2*)(&stg.kt[jl + 2]);
              const int64_t kt4[4] = {t01[0], t01[1], t23[0], t23[1]};
              if (mode == 2) {
#pragma unroll
                for (int e = 0; e < 4; ++e) cb[4 * g + e] = kt4[e] <= tlim ? c1 : c0;
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  cb[4 * g + e] = wpos_s[max(min(dn - 8 * g - e, Pm1), 0)] + wtime_s[time_bucket(tq - kt4[e], NTm1)];
              }
            }
          }
          if (mode == 3) path = D + uniform_f32(wave_max_abs16(cb)) <= kPolyRange ? kPoly : kExact;
          if (path == kPoly) {
#pragma unroll
            for (int i = 0; i < 16; ++i) w[i] = w_poly(__builtin_fmaf(sacc[i], cq, cb[i]));
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) w[i] = w_exact(__builtin_fmaf(sacc[i], cq, cb[i]));
          }
        }
        bf16x8 pop[2];
        {
          f32x8 a0, a1;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            a0[i] = w[i];
            a1[i] = w[i + 8];
          }
          pop[0] = __builtin_convertvector(a0, bf16x8);
          pop[1] = __builtin_convertvector(a1, bf16x8);
        }
        bf16x8 vop[2][2];
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int mm = 0; mm < 2; ++mm) {
            const int r0 = 32 * hk + 16 * mm + vtr_row0, col = 32 * db + vtr_col;
            bf16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4*)(stg.v + cswz(r0, col >> 3) + (col & 7)));
            bf16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4*)(stg.v + cswz(r0 + 8, col >> 3) + (col & 7)));
            vop[db][mm] = bf16x8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
          }
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
          for (int db = 0; db < 2; ++db)
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[db][mm], pop[mm], oacc[db], 0, 0, 0);
      }
    };

    // tiles are taken in pairs, one barrier per pair: tiles t, t + 1 sit in stages t % 4,
    // (t + 1) % 4; the transfers of tiles t + 2, t + 3 go into the stages of tiles t - 2, t - 1
    // (their readers all passed the last barrier) while t and t + 1 are multiplied, then this
    // wave's transfers are waited for and the barrier publishes them to all
    wait_vm<0>();
    lds_barrier();
    auto pair = [&](const CandStage& c0, const CandStage& c1, CandStage& n0, CandStage& n1, int t) __attribute__((always_inline)) {
      dma(n0, t + 2);
      dma(n1, t + 3);
      __builtin_amdgcn_sched_barrier(0);
      compute(c0, t);
      if (t + 1 < n_tiles) compute(c1, t + 1);
      wait_vm<0>();
      lds_barrier();
    };
    for (int t = 0; t < n_tiles; t += 4) {
      pair(st0, st1, st2, st3, t);
      if (t + 2 >= n_tiles) break;
      pair(st2, st3, st0, st1, t + 2);
    }
    // the transfers past the last tile land before the stages are reused
    wait_vm<0>();

    // ---- epilogue: a split history leaves its chunk's sum in fp32 for the reduction ----
    if (n_chunks > 1) {
      if (cvalid) {
        float* pp = a.partial + (((int64_t)chunk * a.total_cand + ctok) * H + h) * kCD + 4 * hf;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = oacc[db][4 * g + e];
            *(f32x4*)(pp + 32 * db + 8 * g) = v4;
          }
      }
    } else if (cvalid) {
      // otherwise the O rows of the candidates, scaled by -(ln 2 / 2) out_scale
      const float osc = -0.5f * kLn2 * a.out_scale;
      bf16* op = a.o + (ctok * H + h) * kCD + 4 * hf;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = oacc[db][4 * g + e] * osc;
          *(bf16x4*)(op + 32 * db + 8 * g) = __builtin_convertvector(v4, bf16x4);
        }
    }
    // every wave is done with the stages and tables before the next item refills them
    lds_barrier();
  }
}

// List of the valid units (user b, head h, chunk) for the scoring kernel: a user with
// candidates has H ceil(n_b / 1024) of them (at least H).  One workgroup: counts per user,
// an exclusive scan over the users in blocks of 1024, then each user writes its entries
// ((b H + h) max_chunks + chunk, chunk-major within the user).  The count goes to list[-1].
__global__ __launch_bounds__(1024) void cand_units_kernel(CandArgs a, int32_t* list) {
  __shared__ int32_t part[1024];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int b0 = 0; b0 < a.B; b0 += 1024) {
    const int b = b0 + tid;
    int cnt = 0;
    if (b < a.B) {
      const int n = min(a.hist_offsets[b + 1] - a.hist_offsets[b], a.max_hist);
      const int m = a.cand_offsets[b + 1] - a.cand_offsets[b];
      cnt = m > 0 ? a.H * max((n + kCChunk - 1) / kCChunk, 1) : 0;
    }
    part[tid] = cnt;
    __syncthreads();
    // Hillis-Steele inclusive scan
    for (int d = 1; d < 1024; d <<= 1) {
      const int v = tid >= d ? part[tid - d] : 0;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    const int base = carry_s + part[tid] - cnt;
    for (int i = 0; i < cnt; ++i) {
      const int chunk = i / a.H, h = i - chunk * a.H;
      list[base + i] = (b * a.H + h) * a.max_chunks + chunk;
    }
    __syncthreads();
    if (tid == 1023) carry_s += part[1023];
    __syncthreads();
  }
  if (tid == 0) list[-1] = carry_s;
}

// O rows of candidates whose user's history was split: the chunks' fp32 sums added in chunk
// order, scaled by -(ln 2 / 2) out_scale, rounded once.  Work item (user, 128-candidate tile,
// head); thread t adds features 4 (t % 16) .. + 3 of candidate rows t / 16, t / 16 + 16, ...
__global__ __launch_bounds__(256) void attn_cand_reduce_kernel(CandArgs a) {
  const int b = blockIdx.x / a.cand_tiles, ct = blockIdx.x - b * a.cand_tiles;
  const int h = blockIdx.y;
  const int64_t cb = a.cand_offsets[b];
  const int n = min(a.hist_offsets[b + 1] - a.hist_offsets[b], a.max_hist);
  const int m = min(a.cand_offsets[b + 1] - (int)cb, a.cand_tiles * kCRows);
  const int n_chunks = (n + kCChunk - 1) / kCChunk;
  if (n_chunks <= 1 || ct * kCRows >= m) return;
  const int rows = min(kCRows, m - ct * kCRows);
  const int64_t cstride = a.total_cand * a.H * kCD;
  const float osc = -0.5f * kLn2 * a.out_scale;
  const int f = 4 * (threadIdx.x & 15);
  for (int r = threadIdx.x >> 4; r < rows; r += 16) {
    const int64_t off = ((cb + (int64_t)ct * kCRows + r) * a.H + h) * kCD + f;
    f32x4 acc = *(const f32x4*)(a.partial + off);
    for (int c = 1; c < n_chunks; ++c) acc += *(const f32x4*)(a.partial + c * cstride + off);
    *(bf16x4*)(a.o + off) = __builtin_convertvector(acc * osc, bf16x4);
  }
}

size_t align256c(size_t x) { return (x + 255) & ~(size_t)255; }

int g_cus[64];  // compute units per device (0 = not yet queried)

}  // namespace

// Workspace: [fp32 partial sums of split histories][TimeStat per history token][int32 per
// history token][unit list: 256-byte header whose last int32 is the count, then B H
// max_chunks int32].
size_t cand_workspace_bytes(int32_t B, int32_t max_hist, int64_t total_hist, int64_t total_cand,
                            int32_t H) {
  if (B < 0 || max_hist < 0 || total_hist < 0 || total_cand < 0 || H < 0) return 0;
  const int64_t chunks = max_hist > kCChunk ? (max_hist + kCChunk - 1) / kCChunk : 0;
  const int64_t max_chunks = chunks ? chunks : 1;
  return align256c((size_t)(chunks * total_cand * H * kCD) * sizeof(float)) +
         align256c((size_t)total_hist * sizeof(TimeStat)) +
         align256c((size_t)total_hist * sizeof(int32_t)) + 256 +
         align256c((size_t)((int64_t)B * H * max_chunks) * sizeof(int32_t));
}

hipError_t launch_attn_candidates_bf16(const CandLaunch& c, hipStream_t stream) {
  if (c.B <= 0 || c.max_cand <= 0) return hipSuccess;
  CandArgs a{};
  a.hist_offsets = c.hist_offsets;
  a.cand_offsets = c.cand_offsets;
  a.q = c.q; a.kc = c.kc; a.vc = c.vc; a.kh = c.kh; a.vh = c.vh;
  a.q_stride = c.q_stride; a.kc_stride = c.kc_stride; a.vc_stride = c.vc_stride;
  a.kh_stride = c.kh_stride; a.vh_stride = c.vh_stride;
  a.o = c.o; a.th = c.bias.ts; a.tc = c.cand_ts; a.bias = c.bias;
  a.total_cand = c.total_cand;
  a.B = c.B;
  a.H = c.H;
  a.max_hist = c.max_hist;
  a.cand_tiles = (c.max_cand + kCRows - 1) / kCRows;
  a.max_chunks = c.max_hist > kCChunk ? (c.max_hist + kCChunk - 1) / kCChunk : 1;
  a.alpha = c.alpha; a.out_scale = c.out_scale;
  const int64_t chunks = c.max_hist > kCChunk ? a.max_chunks : 0;
  char* ws = (char*)c.workspace;
  a.partial = (float*)ws;
  ws += align256c((size_t)(chunks * c.total_cand * c.H * kCD) * sizeof(float));
  TimeStat* stats = (TimeStat*)ws;
  ws += align256c((size_t)c.total_hist * sizeof(TimeStat));
  int32_t* rel = (int32_t*)ws;
  ws += align256c((size_t)c.total_hist * sizeof(int32_t));
  int32_t* list = (int32_t*)(ws + 256);
  a.stats = stats;
  a.unit_list = list;
  const int64_t units = (int64_t)c.B * c.H * a.max_chunks;
  const int64_t items = (units + 7) / 8 * 8 * a.cand_tiles;
  if (items > 0x7fffffff) return hipErrorInvalidValue;
  a.units = (int32_t)units;
  a.items = (int32_t)items;
  hipLaunchKernelGGL(cand_units_kernel, dim3(1), dim3(1024), 0, stream, a, list);
  hipError_t e0 = hipGetLastError();
  if (e0 != hipSuccess) return e0;
  if (a.bias.kind == 1 && c.max_hist > 0) {
    hipError_t e = launch_time_stats(c.B, c.hist_offsets, c.bias.ts, c.max_hist, stats, rel, stream);
    if (e != hipSuccess) return e;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!g_cus[dev]) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    g_cus[dev] = cus > 0 ? cus : 1;
  }
  const int64_t grid = std::max<int64_t>(std::min<int64_t>(items, (int64_t)g_cus[dev] * kCWgPerCu) / 8 * 8, 8);
  const dim3 g((unsigned)grid), blk(kCThreads);
  if (a.bias.kind == 1)
    hipLaunchKernelGGL(attn_cand_bf16_kernel<1>, g, blk, 0, stream, a);
  else if (a.bias.kind == 2)
    hipLaunchKernelGGL(attn_cand_bf16_kernel<2>, g, blk, 0, stream, a);
  else
    hipLaunchKernelGGL(attn_cand_bf16_kernel<0>, g, blk, 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.max_chunks == 1) return e;
  hipLaunchKernelGGL(attn_cand_reduce_kernel, dim3((unsigned)(c.B * a.cand_tiles), (unsigned)c.H),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hstu
