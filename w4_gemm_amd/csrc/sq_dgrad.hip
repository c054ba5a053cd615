// Input gradient of the W4 layer straight from the payload (SquareQ README,
// "SquareQ v3 - W4": the format formula; where the page's backward rebuilds a
// dense bf16 weight first, this contracts the packed codes directly):
//
//   dx = dy @ W_hat = (dy @ D) H + (dy @ up) @ down^T,      D = dequant(R)
//
// H is its own inverse, so (dy @ up) @ down^T = ((dy @ up) @ (H down)^T) H and
// one accumulator
//
//   C[m][k] = 2^(11-E_m) * ( sum_n dy16[m][n] * fp16(q[n][k] s[n][k/G])
//                            + sum_r t[m][r] * (H down)[k][r] )
//
// carries both terms; a single rotation of each 256-column block of C and the
// row factor 2^(E_m-11) finish it.  Six launches on the caller's stream:
//   1. k_dg_transpose: up [N][r] -> upT [r][N].
//   2. the row statistics: per 16 rows and one slice of N, the partial row
//      absmax of dy and the partial t = dy @ up on bf16 MFMA (one read of
//      dy): the forward's statistics kernel when N is a multiple of 256,
//      else k_dg_stats.
//   3. k_dg_scale: E_m = ceil(log2 max|dy_m|); dy16 = fp16(dy * 2^(11-E_m))
//      (|dy16| <= 2^11); t summed over the slices in a fixed order, times
//      2^(11-E_m), split into bf16 hi + lo; the row factor 2^(E_m-11).
//   4. k_dg_hdown: H down per 256-row block of down, split into bf16 hi + lo.
//   5. k_dgrad_gemm: C on fp16 MFMA, contracting over the N output features;
//      the rank-r term is three bf16 MFMA passes (hi*hi, lo*hi, hi*lo) into
//      the same accumulators; C is stored as fp32.
//   6. k_dg_finish: dx = (C S) * 2^(E_m-11) / 16 per 256-column block, S the
//      Sylvester matrix, stored as fp32 or bf16.
// N must be a multiple of 64 (one contraction stage).
#include "sq_device.hpp"
#include "sq_kernels.h"

#include <algorithm>

namespace sq {

namespace {

typedef _Float16 dg_half2 __attribute__((ext_vector_type(2)));
typedef unsigned short dg_u16x2 __attribute__((ext_vector_type(2)));
constexpr int DG_WAVES = 4;   // waves of the small kernels

// ---------------------------------------------------------------- 1. transpose
__global__ void __launch_bounds__(256) k_dg_transpose(const uint16_t* __restrict__ up,
                                                       uint16_t* __restrict__ upT, int64_t n,
                                                       int rank) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // index into upT
  if (i >= n * rank) return;
  const int64_t r = i / n, nn = i - r * n;
  upT[i] = up[nn * rank + r];
}

// ---------------------------------------------------------------- 2. statistics
// Grid (ceil(m/16), slices); slice q covers the 32-column steps [q*sps,
// q*sps + sps) of N; the four waves take every fourth unit of eight steps,
// then every fourth of the steps left over.  MFMA step:
// lane (c, g) holds columns 32 st + 8g .. +7 of row c of dy and of row
// 16 rt + c of upT.  Writes amax_part[q][row] (bf16 magnitude bits) and
// t_part[q][row][r] (fp32) for the rows below m.
template <int RANK>
__global__ void __launch_bounds__(64 * DG_WAVES) k_dg_stats(
    const uint16_t* __restrict__ dy, const uint16_t* __restrict__ upT, int64_t m, int64_t n,
    int sps, uint32_t* __restrict__ amax_part, float* __restrict__ t_part) {
  constexpr int RT = RANK / 16;
  __shared__ float red_t[DG_WAVES][16][64];
  __shared__ uint32_t red_max[DG_WAVES][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int64_t lrow = min(row0 + c, m - 1);   // rows past m read the last row
  const int64_t q = blockIdx.y, s_end = min(n >> 5, (q + 1) * sps);

  f32x4 acc[RT > 0 ? RT : 1] = {};
  dg_u16x2 amax2 = {0, 0};
  auto step = [&](const u32x4& xv, int64_t col) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      amax2 = __builtin_elementwise_max(amax2, __builtin_bit_cast(dg_u16x2, xv[e] & 0x7FFF7FFFu));
    const bf16x8 af = __builtin_bit_cast(bf16x8, xv);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const bf16x8 bfr = *reinterpret_cast<const bf16x8*>(upT + (int64_t)(16 * rt + c) * n + col);
      acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr, acc[rt], 0, 0, 0);
    }
  };
  // whole units of eight steps (256 columns: eight 16-byte loads per lane in
  // flight, four 64-byte runs of each row per instruction), then the rest
  const int64_t s0 = q * sps, units = (s_end - s0) >> 3;
  for (int64_t u = wave; u < units; u += DG_WAVES) {
    const int64_t col0 = (s0 + 8 * u) * 32 + 8 * g;
    u32x4 xv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xv[j] = *reinterpret_cast<const u32x4*>(dy + lrow * n + col0 + 32 * j);
#pragma unroll
    for (int j = 0; j < 8; ++j) step(xv[j], col0 + 32 * j);
  }
  for (int64_t st = s0 + 8 * units + wave; st < s_end; st += DG_WAVES) {
    const int64_t col = st * 32 + 8 * g;
    step(*reinterpret_cast<const u32x4*>(dy + lrow * n + col), col);
  }
  // acc[rt][i] = partial t[row0 + 4g + i][16 rt + c]
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red_t[wave][4 * g + i][16 * rt + c] = acc[rt][i];
  red_max[wave][lane] = max((uint32_t)amax2[0], (uint32_t)amax2[1]);
  __syncthreads();
  if constexpr (RANK > 0) {
    for (int i = tid; i < 16 * RANK; i += 64 * DG_WAVES) {
      const int rr = i / RANK, r = i - rr * RANK;
      if (row0 + rr >= m) continue;
      float t = 0.0f;
#pragma unroll
      for (int w = 0; w < DG_WAVES; ++w) t += red_t[w][rr][r];
      t_part[(q * m + row0 + rr) * RANK + r] = t;
    }
  }
  if (tid < 16 && row0 + tid < m) {
    uint32_t mx = 0;
#pragma unroll
    for (int w = 0; w < DG_WAVES; ++w)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) mx = max(mx, red_max[w][tid + 16 * gg]);
    amax_part[q * m + row0 + tid] = mx;
  }
}

// ---------------------------------------------------------------- 3. scale
// Grid (ceil(m/16), ceil(n/256)): 16 rows x 256 columns of dy per workgroup,
// sixteen columns per thread.
__global__ void __launch_bounds__(256) k_dg_scale(
    const uint16_t* __restrict__ dy, int64_t m, int64_t n, int rank, int slices,
    const uint32_t* __restrict__ amax_part, const float* __restrict__ t_part,
    uint16_t* __restrict__ dy16, uint16_t* __restrict__ thi, uint16_t* __restrict__ tlo,
    float* __restrict__ rowscale) {
  __shared__ int s_exp[16];
  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  if (tid < 16) {
    const int64_t row = min(row0 + tid, m - 1);
    s_exp[tid] = row_exponent(slice_max(amax_part + row, m, slices));
  }
  __syncthreads();
  {
    // t: slices summed in a fixed order; the strip's 16 x rank outputs are
    // shared out over the column blocks
    const int outs = 16 * rank;
    const int per = (outs + (int)gridDim.y - 1) / (int)gridDim.y;
    const int i0 = (int)blockIdx.y * per, i1 = min(outs, i0 + per);
    for (int i = i0 + tid; i < i1; i += 256) {
      const int rr = i / rank, r = i - rr * rank;
      const int64_t row = row0 + rr;
      if (row >= m) continue;
      float t = slice_sum(t_part + row * rank + r, m * rank, slices);
      t *= ldexpf(1.0f, 11 - s_exp[rr]);
      const uint16_t hb = f32_to_bf16(t);
      thi[row * rank + r] = hb;
      tlo[row * rank + r] = f32_to_bf16(t - bf16_to_f32(hb));
    }
    if (blockIdx.y == 0 && tid < 16 && row0 + tid < m)
      rowscale[row0 + tid] = ldexpf(1.0f, s_exp[tid] - 11);
  }
  const int rr = tid >> 4;
  const int64_t row = row0 + rr, col = (int64_t)blockIdx.y * 256 + 16 * (tid & 15);
  if (row >= m || col >= n) return;   // n is a multiple of 64: col < n covers all 16
  const float f = ldexpf(1.0f, 11 - s_exp[rr]);   // exact
  const u32x4* src = reinterpret_cast<const u32x4*>(dy + row * n + col);
  u32x4* dst = reinterpret_cast<u32x4*>(dy16 + row * n + col);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const u32x4 w = src[h];
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const _Float16 lo = (_Float16)(bf16_to_f32(w[e] & 0xFFFFu) * f);
      const _Float16 hi = (_Float16)(bf16_to_f32(w[e] >> 16) * f);
      o[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
             ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    dst[h] = o;
  }
}

// ---------------------------------------------------------------- 4. H down
// One wave per 256-row block of down [k][rank] and 16 of its columns, in the
// wave layout of the rotation kernels with the roles of rows and columns
// swapped: lane (c, g) holds column 16 cs + c at block rows 64g .. 64g+63;
// the 256-point butterflies run in registers and lane swaps, then times
// 1/16, split into bf16 hi + lo.
__global__ void __launch_bounds__(64) k_dg_hdown(const uint16_t* __restrict__ down, int rank,
                                                  uint16_t* __restrict__ hd_hi,
                                                  uint16_t* __restrict__ hd_lo) {
  const int lane = threadIdx.x, c = lane & 15, g = lane >> 4;
  const int64_t b = blockIdx.x;
  const int col = 16 * (int)blockIdx.y + c;
  const uint16_t* src = down + (b * 256 + 64 * g) * rank + col;
  float v[64];
#pragma unroll
  for (int j = 0; j < 64; ++j) v[j] = bf16_to_f32(src[j * rank]);
  fwht_inreg64(v);
  fwht_cross64_swap(v);
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    const int64_t o = (b * 256 + swap_col(g, j)) * rank + col;
    const float x = v[j] * 0.0625f;
    const uint16_t hb = f32_to_bf16(x);
    hd_hi[o] = hb;
    hd_lo[o] = f32_to_bf16(x - bf16_to_f32(hb));
  }
}

// ---------------------------------------------------------------- 5. contraction
// BM x 256 output tile (rows of dy x columns of K, one Hadamard block wide)
// per workgroup of eight waves, BM = 256 or 224; wave (wm, wn) owns rows
// (BM/2) wm .. +BM/2-1 and columns 64 wn .. +63 as (BM/32) x 4 MFMA tiles.
// One stage contracts 64 output features n in two 16x16x32 steps.
//
// A = dy16 streams global -> LDS with direct 16-byte buffer loads: 64 n per
// row (128 bytes), chunk c of row r at slot c ^ a_swz(r); loader rows at or
// past BM fetch nothing.
// B: the contraction runs over n, across the packed rows, so the codes are
// transposed on their way into LDS.  Thread (wave w, lane l) loads the 16-bit
// code word l (4 nibbles: columns 4l .. 4l+3 of the tile) of rows 8w .. 8w+7
// of the stage and stores the eight words as one 16-byte chunk: word line l
// (128 bytes = 64 rows) holds row chunk c at slot c ^ a_swz(l).  The fp16
// scales go the same way, one per thread, into group lines of 64 rows (the
// chunks of odd lines rotated by four).  Both swizzles keep the fragment
// reads free of bank conflicts.
// In step ks lane (f, g) of wave wn then reads, with one 16-byte load each,
// word 16 wn + f of rows 16g + 8ks .. +7 and the scales of those rows for
// its group (its A fragment holds the same eight n); each 32-bit half-pair (rows 2p, 2p+1) becomes one fp16 pair per
// column j with one mask:
//   (u >> 4j) & 0x000F000F ^ 0x64086408,
// then (1024 + q + 8) - 1032 is exact and * (s_2p, s_2p+1) rounds once.
// MFMA tile j therefore computes output column 64 wn + 4f + j in lane f.
// Pipeline: three LDS buffers; while stage st computes, the direct loads of A
// for stages st+1 and st+2 and the register loads of B for stage st+2 are in
// flight; B is written to LDS after the MFMAs, then one barrier per stage.
constexpr int DG_THREADS = 512;
__shared__ __attribute__((aligned(16))) uint8_t dg_a0[256 * 128];
__shared__ __attribute__((aligned(16))) uint8_t dg_a1[256 * 128];
__shared__ __attribute__((aligned(16))) uint8_t dg_b0[64 * 128];
__shared__ __attribute__((aligned(16))) uint8_t dg_b1[64 * 128];
__shared__ __attribute__((aligned(16))) uint8_t dg_s0[8 * 128];
__shared__ __attribute__((aligned(16))) uint8_t dg_s1[8 * 128];
__shared__ __attribute__((aligned(16))) uint8_t dg_a2[256 * 128];
__shared__ __attribute__((aligned(16))) uint8_t dg_b2[64 * 128];
__shared__ __attribute__((aligned(16))) uint8_t dg_s2[8 * 128];

typedef __attribute__((address_space(3))) void* dg_lds_ptr;

template <int GSHIFT, int BM>
__global__ void __launch_bounds__(DG_THREADS, 1) k_dgrad_gemm(
    const uint16_t* __restrict__ dy16, const uint8_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ thi,
    const uint16_t* __restrict__ tlo, const uint16_t* __restrict__ hd_hi,
    const uint16_t* __restrict__ hd_lo, float* __restrict__ cbuf, int64_t m, int64_t n,
    int64_t k, int rank) {
  static_assert(BM == 256 || BM == 224, "tile rows");
  constexpr int FM = BM / 32, WROWS = BM / 2;
  constexpr int GPT = 256 >> GSHIFT;   // scale groups per tile row
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int fr = lane & 15, g = lane >> 4;
  const int64_t mt = (m + BM - 1) / BM, kt = k / 256;
  int64_t tile_m, tile_k;
  xcd_tile(blockIdx.x, mt * kt, kt, tile_m, tile_k);
  const int64_t m0 = tile_m * BM, k0 = tile_k * 256;
  const int64_t NS = n / 64;
  const int64_t half_k = k >> 1, ngroups = k >> GSHIFT;
  const int64_t a_rows = min((int64_t)BM, m - m0);

  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(dy16 + m0 * n), (short)0, (int)(a_rows * n * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t c_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(codes + k0 / 2), (short)0, (int)(n * half_k - k0 / 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(scales + (k0 >> GSHIFT)), (short)0, (int)((n * ngroups - (k0 >> GSHIFT)) * 2),
      0x00020000);
  // A loader: wave w fills rows 32w .. 32w+31, eight per instruction
  uint32_t a_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 32 * wave + 8 * i + (lane >> 3);
    a_off[i] = r < BM ? (uint32_t)(min((int64_t)r, a_rows - 1) * n * 2) +
                            16 * ((lane & 7) ^ a_swz(r))
                      : 0x80000000u;
  }
  // (stage offsets go through readfirstlane: the compiler then knows they are
  // uniform and emits no per-lane loop around the loads)
  auto issue_a = [&](int64_t st, uint8_t* abuf) {
    const int so = __builtin_amdgcn_readfirstlane((int)(st * 128));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (dg_lds_ptr)(abuf + wave * 4096 + i * 1024),
                                               16, a_off[i], so, 0, 0);
  };
  // B loader: word `lane` of rows 8 wave .. +7; scale (row, group) = (tid /
  // GPT, tid % GPT) for the first 64 GPT threads
  const uint32_t cb_off = (uint32_t)(8 * wave * half_k + 2 * lane);
  const bool s_thread = tid < 64 * GPT;
  const int s_row = tid / GPT, s_grp = tid % GPT;
  const uint32_t sb_off = s_thread ? (uint32_t)(s_row * ngroups * 2 + 2 * s_grp) : 0x80000000u;
  auto load_b = [&](int64_t st, uint32_t (&cw)[8], uint32_t& sv) {
    const int cst = __builtin_amdgcn_readfirstlane((int)(st * 64 * half_k));
    const int sst = __builtin_amdgcn_readfirstlane((int)(st * 64 * ngroups * 2));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      cw[i] = __builtin_amdgcn_raw_buffer_load_b16(c_rsrc, cb_off + (uint32_t)(i * half_k), cst, 0);
    sv = __builtin_amdgcn_raw_buffer_load_b16(s_rsrc, sb_off, sst, 0);
  };
  const uint32_t bw_addr = (uint32_t)(lane * 128 + 16 * (wave ^ a_swz(lane)));
  // (threads without a scale, 64-groups only, write their zero into the
  // unused upper half of the line block: the store stays unconditional)
  const uint32_t sw_addr =
      s_thread ? (uint32_t)(s_grp * 128 + 16 * ((s_row >> 3) ^ (4 * (s_grp & 1))) + 2 * (s_row & 7))
               : (uint32_t)(512 + 2 * (tid - 256));
  auto write_b = [&](const uint32_t (&cw)[8], uint32_t sv, uint8_t* bbuf, uint8_t* sbuf) {
    const u32x4 d = {cw[0] | (cw[1] << 16), cw[2] | (cw[3] << 16), cw[4] | (cw[5] << 16),
                     cw[6] | (cw[7] << 16)};
    *reinterpret_cast<u32x4*>(bbuf + bw_addr) = d;
    // byte copy: the scale lines are read back as 16-byte vectors
    const uint16_t s16 = (uint16_t)sv;
    __builtin_memcpy(sbuf + sw_addr, &s16, 2);
  };

  // fragment addresses (rows WROWS wm + 16 i + fr share the swizzle a_swz(fr))
  const int swa = a_swz(fr);
  uint32_t a_lane[2], b_lane[2], s_lane[2];
  const int bw = 16 * wn + fr;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    // lane group g contracts rows 16g + 8ks .. +7 of the stage (chunk 2g + ks):
    // this lane-to-chunk order reads A with a tenth of the bank conflicts
    // of chunk 4ks + g
    const int chk = 2 * g + ks;
    a_lane[ks] = (WROWS * wm + fr) * 128 + 16 * (chk ^ swa);
    b_lane[ks] = bw * 128 + 16 * (chk ^ a_swz(bw));
    const int sg = (64 * wn + 4 * fr) >> GSHIFT;
    s_lane[ks] = sg * 128 + 16 * (chk ^ (4 * (sg & 1)));
  }

  f32x4 acc[FM][4];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint8_t* abuf, const uint8_t* bbuf, const uint8_t* sbuf) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      half8 af[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const half8*>(abuf + a_lane[ks] + i * 2048);
      const u32x4 cw = *reinterpret_cast<const u32x4*>(bbuf + b_lane[ks]);
      const u32x4 sw = *reinterpret_cast<const u32x4*>(sbuf + s_lane[ks]);
      uint32_t bq[4][4];
      const dg_half2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        // (through a scalar: this compiler's __builtin_bit_cast of a vector
        // element reads element 0 whatever the index)
        const uint32_t s32 = sw[p];
        const dg_half2 sp = __builtin_bit_cast(dg_half2, s32);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dg_half2 h =
              __builtin_bit_cast(dg_half2, ((cw[p] >> (4 * j)) & 0x000F000Fu) ^ 0x64086408u);
          h = (h - off) * sp;
          bq[j][p] = __builtin_bit_cast(uint32_t, h);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const half8 bf = __builtin_bit_cast(half8, (u32x4){bq[j][0], bq[j][1], bq[j][2], bq[j][3]});
#pragma unroll
        for (int i = 0; i < FM; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf, acc[i][j], 0, 0, 0);
      }
    }
  };
  // Barriers are explicit waits + s_barrier: a workgroup fence would also
  // wait for the direct loads still in flight for later stages.
  auto sync = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Stage st computes from buffer st % 3 while the loads of stage st+2 fill
  // buffer (st+2) % 3 (read last in stage st-1): B's register loads first,
  // then A's direct loads, so that the wait before the barrier (everything
  // but the last four loads) leaves A of stage st+2 in flight.  The last two
  // stages reload the final stage into buffers nobody reads again: no branch,
  // so the compiler's wait counting stays exact (after a join it would wait
  // for every load before the first LDS read).
  uint32_t cw[8], sv;
  auto stage = [&](int64_t st, const uint8_t* ca, const uint8_t* cb, const uint8_t* cs,
                   uint8_t* na, uint8_t* nb, uint8_t* ns) {
    const int64_t sp = min(st + 2, NS - 1);
    load_b(sp, cw, sv);
    __builtin_amdgcn_sched_barrier(0);
    issue_a(sp, na);
    compute(ca, cb, cs);
    write_b(cw, sv, nb, ns);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0074);   // vmcnt(4) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  load_b(0, cw, sv);
  issue_a(0, dg_a0);
  write_b(cw, sv, dg_b0, dg_s0);
  load_b(min((int64_t)1, NS - 1), cw, sv);
  issue_a(min((int64_t)1, NS - 1), dg_a1);
  write_b(cw, sv, dg_b1, dg_s1);
  sync();
  for (int64_t st = 0; st < NS; st += 3) {
    stage(st, dg_a0, dg_b0, dg_s0, dg_a2, dg_b2, dg_s2);
    if (st + 1 >= NS) break;
    stage(st + 1, dg_a1, dg_b1, dg_s1, dg_a0, dg_b0, dg_s0);
    if (st + 2 >= NS) break;
    stage(st + 2, dg_a2, dg_b2, dg_s2, dg_a1, dg_b1, dg_s1);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);   // the tail's redundant loads

  // rank-r term: t (times 2^(11-E)) @ (H down)^T, bf16 hi/lo on MFMA
  const int64_t rbase = m0 + WROWS * wm, cbase = k0 + 64 * wn;
  for (int rr = 0; rr < rank; rr += 32) {
    bf16x8 ah[FM], al[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t r = min(rbase + 16 * i + fr, m - 1);
      ah[i] = *reinterpret_cast<const bf16x8*>(thi + r * rank + rr + 8 * g);
      al[i] = *reinterpret_cast<const bf16x8*>(tlo + r * rank + rr + 8 * g);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = cbase + 4 * fr + j;
      const bf16x8 bh = *reinterpret_cast<const bf16x8*>(hd_hi + col * rank + rr + 8 * g);
      const bf16x8 bl = *reinterpret_cast<const bf16x8*>(hd_lo + col * rank + rr + 8 * g);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bh, acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[i], bh, acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bl, acc[i][j], 0, 0, 0);
      }
    }
  }

  // store C: acc[i][j][v] is row WROWS wm + 16 i + 4g + v, column 64 wn + 4f + j;
  // the descriptor ends at row m, so rows of a ragged last tile are dropped
  const __amdgpu_buffer_rsrc_t o_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(cbuf + m0 * k), (short)0, (int)(a_rows * k * 4), 0x00020000);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t r = WROWS * wm + 16 * i + 4 * g + v;
      const uint32_t off = (uint32_t)((r * k + k0 + 64 * wn + 4 * fr) * 4);
      const f32x4 o = {acc[i][0][v], acc[i][1][v], acc[i][2][v], acc[i][3][v]};
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), o_rsrc, off, 0, 0);
    }
}

// ---------------------------------------------------------------- 6. finish
// Grid (ceil(m/16), ceil(k/1024)); wave w of workgroup (i, j) rotates rows
// 16i .. 16i+15 of the 256-column block 4j + w of C in the wave layout, then
// applies 2^(E-11)/16 and stores four runs of 16 columns per lane.
__global__ void __launch_bounds__(64 * DG_WAVES) k_dg_finish(const float* __restrict__ cbuf,
                                                             const float* __restrict__ rowscale,
                                                             void* __restrict__ dx, int64_t m,
                                                             int64_t k, int dx_bf16) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int64_t b = (int64_t)blockIdx.y * DG_WAVES + wave;
  if (b >= (k >> 8)) return;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int64_t lrow = min(row0 + c, m - 1);
  float v[64];
  const f32x4* src = reinterpret_cast<const f32x4*>(cbuf + lrow * k + b * 256 + 64 * g);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const f32x4 q = src[j];
    v[4 * j] = q[0];
    v[4 * j + 1] = q[1];
    v[4 * j + 2] = q[2];
    v[4 * j + 3] = q[3];
  }
  fwht_inreg64(v);
  fwht_cross64_swap(v);
  const int64_t row = row0 + c;
  if (row >= m) return;
  const float f = rowscale[row] * 0.0625f;   // exact: a power of two
#pragma unroll
  for (int run = 0; run < 4; ++run) {
    const int reg0 = 16 * run;   // registers 32a + 16b .. +15
    const int64_t col = b * 256 + swap_col(g, reg0);
    if (dx_bf16) {
      u32x4* dst = reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(dx) + row * k + col);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = pack_bf16x2(v[reg0 + 8 * h + 2 * e] * f, v[reg0 + 8 * h + 2 * e + 1] * f);
        dst[h] = o;
      }
    } else {
      f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(dx) + row * k + col);
#pragma unroll
      for (int h = 0; h < 4; ++h)
        dst[h] = (f32x4){v[reg0 + 4 * h] * f, v[reg0 + 4 * h + 1] * f, v[reg0 + 4 * h + 2] * f,
                         v[reg0 + 4 * h + 3] * f};
    }
  }
}

struct DgBuffers {
  uint16_t *upT, *dy16, *thi, *tlo, *hd_hi, *hd_lo;
  uint32_t* amax;
  float *tpart, *rowscale, *cbuf;
};

DgBuffers carve(const DgradPlan& p, void* ws) {
  uint8_t* b = static_cast<uint8_t*>(ws);
  DgBuffers o;
  o.upT = reinterpret_cast<uint16_t*>(b + p.off_upT);
  o.dy16 = reinterpret_cast<uint16_t*>(b + p.off_dy16);
  o.thi = reinterpret_cast<uint16_t*>(b + p.off_thi);
  o.tlo = reinterpret_cast<uint16_t*>(b + p.off_tlo);
  o.hd_hi = reinterpret_cast<uint16_t*>(b + p.off_hdhi);
  o.hd_lo = reinterpret_cast<uint16_t*>(b + p.off_hdlo);
  o.amax = reinterpret_cast<uint32_t*>(b + p.off_amax);
  o.tpart = reinterpret_cast<float*>(b + p.off_tpart);
  o.rowscale = reinterpret_cast<float*>(b + p.off_rowscale);
  o.cbuf = reinterpret_cast<float*>(b + p.off_c);
  return o;
}

}  // namespace

// Statistics slices: enough workgroups to cover the chip about four times,
// each wave taking at least two 32-column steps.
DgradPlan plan_dgrad(int64_t m, int64_t n, int64_t k, int group, int rank) {
  DgradPlan p{};
  p.m = m; p.n = n; p.k = k; p.group = group; p.rank = rank;
  const int64_t strips = (m + 15) / 16, steps = n / 32;
  int64_t slices = std::max<int64_t>(1, (1024 + strips - 1) / strips);
  slices = std::min<int64_t>(slices, std::max<int64_t>(1, steps / (2 * DG_WAVES)));
  int64_t sps = (steps + slices - 1) / slices;
  if (sps >= 32) sps = (sps + 31) / 32 * 32;   // whole units for all four waves
  p.stats_sps = (int)sps;
  // N a multiple of 256: the shared row-statistics kernel (one 256-column
  // block of N per wave, several 16-row tiles against one read of its upT
  // fragments)
  p.stats_tiles = 0;
  // contraction tile height: the one with the fewest rows x rounds of 256 CUs
  {
    const int64_t kt = k / 256;
    auto cost = [&](int64_t bm) { return ((((m + bm - 1) / bm) * kt + 255) / 256) * bm; };
    p.tile_m = cost(224) < cost(256) ? 224 : 256;
  }
  p.stats_slices = (int)((steps + sps - 1) / sps);
  if (n % 256 == 0) row_stats_plan(m, n, &p.stats_tiles, &p.stats_slices);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  p.off_upT = take((size_t)rank * n * 2);
  p.off_amax = take((size_t)p.stats_slices * m * 4);
  p.off_tpart = take((size_t)p.stats_slices * m * rank * 4);
  p.off_dy16 = take((size_t)m * n * 2);
  p.off_thi = take((size_t)m * rank * 2);
  p.off_tlo = take((size_t)m * rank * 2);
  p.off_rowscale = take((size_t)m * 4);
  p.off_hdhi = take((size_t)k * rank * 2);
  p.off_hdlo = take((size_t)k * rank * 2);
  p.off_c = take((size_t)m * k * 4);
  p.total = off;
  return p;
}

hipError_t launch_dgrad(const DgradPlan& p, const uint16_t* dy, const uint8_t* codes,
                        const uint16_t* scales, const uint16_t* up, const uint16_t* down,
                        void* dx, int dx_bf16, void* workspace, hipStream_t stream) {
  const DgBuffers b = carve(p, workspace);
  hipError_t err;
  const unsigned strips = (unsigned)((p.m + 15) / 16);
  // the shared statistics kernel reads lora_up as stored at ranks 16 and 32;
  // rank 64 and the kernel for N not a multiple of 256 read a transposed copy
  const bool kmajor = p.stats_tiles > 0 && p.rank > 0 && p.rank <= 32;
  if (p.rank > 0 && !kmajor) {
    const int64_t cnt = p.n * p.rank;
    hipLaunchKernelGGL(k_dg_transpose, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, stream,
                       up, b.upT, p.n, p.rank);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const dim3 sgrid(strips, (unsigned)p.stats_slices);
  if (p.stats_tiles > 0) {
    if ((err = launch_row_stats(dy, kmajor ? up : b.upT, kmajor, p.m, p.n, p.rank, p.stats_tiles,
                                p.stats_slices, b.amax, b.tpart, stream)) != hipSuccess)
      return err;
  } else {
    if (p.rank == 0)
      hipLaunchKernelGGL(k_dg_stats<0>, sgrid, dim3(64 * DG_WAVES), 0, stream, dy, b.upT, p.m,
                         p.n, p.stats_sps, b.amax, b.tpart);
    else if (p.rank == 32)
      hipLaunchKernelGGL(k_dg_stats<32>, sgrid, dim3(64 * DG_WAVES), 0, stream, dy, b.upT, p.m,
                         p.n, p.stats_sps, b.amax, b.tpart);
    else
      hipLaunchKernelGGL(k_dg_stats<64>, sgrid, dim3(64 * DG_WAVES), 0, stream, dy, b.upT, p.m,
                         p.n, p.stats_sps, b.amax, b.tpart);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(k_dg_scale, dim3(strips, (unsigned)((p.n + 255) / 256)), dim3(256), 0, stream,
                     dy, p.m, p.n, p.rank, p.stats_slices, b.amax, b.tpart, b.dy16, b.thi, b.tlo,
                     b.rowscale);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (p.rank > 0) {
    hipLaunchKernelGGL(k_dg_hdown, dim3((unsigned)(p.k / 256), (unsigned)(p.rank / 16)), dim3(64),
                       0, stream, down, p.rank, b.hd_hi, b.hd_lo);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const unsigned tiles = (unsigned)(((p.m + p.tile_m - 1) / p.tile_m) * (p.k / 256));
#define SQ_DG(GS, BM)                                                                           \
  hipLaunchKernelGGL((k_dgrad_gemm<GS, BM>), dim3(tiles), dim3(DG_THREADS), 0, stream, b.dy16, \
                     codes, scales, b.thi, b.tlo, b.hd_hi, b.hd_lo, b.cbuf, p.m, p.n, p.k, p.rank)
  if (p.group == 32) {
    if (p.tile_m == 256) SQ_DG(5, 256); else SQ_DG(5, 224);
  } else {
    if (p.tile_m == 256) SQ_DG(6, 256); else SQ_DG(6, 224);
  }
#undef SQ_DG
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(k_dg_finish,
                     dim3(strips, (unsigned)((p.k / 256 + DG_WAVES - 1) / DG_WAVES)),
                     dim3(64 * DG_WAVES), 0, stream, b.cbuf, b.rowscale, dx, p.m, p.k, dx_bf16);
  return hipGetLastError();
}

}  // namespace sq
