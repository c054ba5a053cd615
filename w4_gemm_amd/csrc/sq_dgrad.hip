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
//   2. k_dg_stats: per 16 rows and one slice of N, the partial row absmax of
//      dy and the partial t = dy @ up on bf16 MFMA (one read of dy).
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
// q*sps + sps) of N and the four waves take every fourth one.  MFMA step:
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
#pragma unroll 4
  for (int64_t st = q * sps + wave; st < s_end; st += DG_WAVES) {
    const int64_t col = st * 32 + 8 * g;
    const u32x4 xv = *reinterpret_cast<const u32x4*>(dy + lrow * n + col);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      amax2 = __builtin_elementwise_max(amax2, __builtin_bit_cast(dg_u16x2, xv[e] & 0x7FFF7FFFu));
    const bf16x8 af = __builtin_bit_cast(bf16x8, xv);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const bf16x8 bfr = *reinterpret_cast<const bf16x8*>(upT + (int64_t)(16 * rt + c) * n + col);
      acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr, acc[rt], 0, 0, 0);
    }
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
    uint32_t mx = 0;
    for (int q = 0; q < slices; ++q) mx = max(mx, amax_part[q * m + row]);
    s_exp[tid] = row_exponent(mx);
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
      float t = 0.0f;
      for (int q = 0; q < slices; ++q) t += t_part[(q * m + row) * rank + r];
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
// One workgroup per 256-row block of down [k][RANK]: the block in LDS as
// fp32, eight butterfly stages along the rows, times 1/16, bf16 hi + lo.
template <int RANK>
__global__ void __launch_bounds__(256) k_dg_hdown(const uint16_t* __restrict__ down,
                                                   uint16_t* __restrict__ hd_hi,
                                                   uint16_t* __restrict__ hd_lo) {
  __shared__ float blk[256][RANK + 1];
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * 256 * RANK;
  for (int i = tid; i < 256 * RANK; i += 256) blk[i / RANK][i % RANK] = bf16_to_f32(down[base + i]);
  for (int h = 1; h < 256; h <<= 1) {
    __syncthreads();
    for (int i = tid; i < 128 * RANK; i += 256) {
      const int p = i / RANK, r = i % RANK;
      const int lo = (p / h) * 2 * h + (p % h), hi = lo + h;
      const float a = blk[lo][r], b = blk[hi][r];
      blk[lo][r] = a + b;
      blk[hi][r] = a - b;
    }
  }
  __syncthreads();
  for (int i = tid; i < 256 * RANK; i += 256) {
    const float v = blk[i / RANK][i % RANK] * 0.0625f;
    const uint16_t hb = f32_to_bf16(v);
    hd_hi[base + i] = hb;
    hd_lo[base + i] = f32_to_bf16(v - bf16_to_f32(hb));
  }
}

// ---------------------------------------------------------------- 5. contraction
// 256 x 256 output tile (rows of dy x columns of K, one Hadamard block wide)
// per workgroup of eight waves; wave (wm, wn) owns rows 128 wm .. +127 and
// columns 64 wn .. +63 as 8 x 4 MFMA tiles.  One stage contracts 64 output
// features n in two 16x16x32 steps.
//
// Operands stream global -> LDS with direct 16-byte buffer loads:
//  * A = dy16: 256 rows x 64 n (128 bytes per row), chunk c of row r at slot
//    c ^ a_swz(r);
//  * B = codes: 64 rows n x 256 columns (128 bytes per row), chunk c of row r
//    at slot c ^ 2((r >> 3) & 3), so the four lane groups of a fragment read
//    (rows 8 apart) hit distinct banks;
//  * the fp16 scales of those 64 rows for the tile's groups (16 bytes a row).
// The contraction runs over n, across the packed rows, so a B fragment is
// gathered: in step ks lane (f, g) reads the 16-bit code word (4 nibbles,
// columns 4f .. 4f+3 of its wave's 64) of rows 32 ks + 8g + i, i = 0..7, and
// each pair of rows becomes one fp16 pair per column with one mask:
//   (u >> 4j) & 0x000F000F ^ 0x64086408, u = w_{2p} | w_{2p+1} << 16,
// then (1024 + q + 8) - 1032 is exact and * (s_{2p}, s_{2p+1}) rounds once.
// MFMA tile j therefore computes output column 64 wn + 4f + j in lane f.
// Pipeline: two LDS buffers; stage st+1 loads while stage st computes, one
// barrier per stage.
constexpr int DG_THREADS = 512;
__shared__ __attribute__((aligned(16))) uint8_t dg_a0[256 * 128];
__shared__ __attribute__((aligned(16))) uint8_t dg_a1[256 * 128];
__shared__ __attribute__((aligned(16))) uint8_t dg_b0[64 * 128];
__shared__ __attribute__((aligned(16))) uint8_t dg_b1[64 * 128];
__shared__ __attribute__((aligned(16))) uint8_t dg_s0[64 * 16];
__shared__ __attribute__((aligned(16))) uint8_t dg_s1[64 * 16];

typedef __attribute__((address_space(3))) void* dg_lds_ptr;

template <int GSHIFT>
__global__ void __launch_bounds__(DG_THREADS, 1) k_dgrad_gemm(
    const uint16_t* __restrict__ dy16, const uint8_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ thi,
    const uint16_t* __restrict__ tlo, const uint16_t* __restrict__ hd_hi,
    const uint16_t* __restrict__ hd_lo, float* __restrict__ cbuf, int64_t m, int64_t n,
    int64_t k, int rank) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int fr = lane & 15, g = lane >> 4;
  const int64_t mt = (m + 255) / 256, kt = k / 256;
  int64_t tile_m, tile_k;
  xcd_tile(blockIdx.x, mt * kt, kt, tile_m, tile_k);
  const int64_t m0 = tile_m * 256, k0 = tile_k * 256;
  const int64_t NS = n / 64;
  const int64_t half_k = k >> 1, ngroups = k >> GSHIFT;
  const int64_t a_rows = min((int64_t)256, m - m0);

  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(dy16 + m0 * n), (short)0, (int)(a_rows * n * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t c_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(codes + k0 / 2), (short)0, (int)(n * half_k - k0 / 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(scales + (k0 >> GSHIFT)), (short)0, (int)((n * ngroups - (k0 >> GSHIFT)) * 2),
      0x00020000);
  // loaders: wave w fills A rows 32w .. 32w+31 (eight per instruction) and B
  // rows 8w .. 8w+7; wave 0 also the 64 scale rows (one per lane)
  uint32_t a_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 32 * wave + 8 * i + (lane >> 3);
    a_off[i] = (uint32_t)(min((int64_t)r, a_rows - 1) * n * 2) + 16 * ((lane & 7) ^ a_swz(r));
  }
  const int br = 8 * wave + (lane >> 3);
  const uint32_t b_off = (uint32_t)(br * half_k) + 16 * ((lane & 7) ^ (((br >> 3) & 3) << 1));
  const uint32_t s_off = (uint32_t)(lane * ngroups * 2);
  auto issue = [&](int64_t st, uint8_t* abuf, uint8_t* bbuf, uint8_t* sbuf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (dg_lds_ptr)(abuf + wave * 4096 + i * 1024),
                                               16, a_off[i], (int)(st * 128), 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c_rsrc, (dg_lds_ptr)(bbuf + wave * 1024), 16, b_off,
                                             (int)(st * 64 * half_k), 0, 0);
    if (wave == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, (dg_lds_ptr)sbuf, 16, s_off,
                                               (int)(st * 64 * ngroups * 2), 0, 0);
  };

  // fragment addresses (rows 128 wm + 16 i + fr share the swizzle a_swz(fr))
  const int swa = a_swz(fr);
  uint32_t a_lane[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) a_lane[ks] = (128 * wm + fr) * 128 + 16 * ((4 * ks + g) ^ swa);
  // code word of row 32 ks + 8g + i: chunk 2 wn + f/8 at slot chunk ^ 2g
  const uint32_t b_lane = (uint32_t)(8 * g * 128 + 16 * ((2 * wn + (fr >> 3)) ^ (2 * g)) +
                                     2 * (fr & 7));
  const uint32_t s_lane = (uint32_t)(8 * g * 16 + 2 * ((64 * wn + 4 * fr) >> GSHIFT));

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint8_t* abuf, const uint8_t* bbuf, const uint8_t* sbuf) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      half8 af[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        af[i] = *reinterpret_cast<const half8*>(abuf + a_lane[ks] + i * 2048);
      uint32_t cw[8], sw[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        cw[i] = *reinterpret_cast<const uint16_t*>(bbuf + b_lane + (32 * ks + i) * 128);
        sw[i] = *reinterpret_cast<const uint16_t*>(sbuf + s_lane + (32 * ks + i) * 16);
      }
      uint32_t bw[4][4];
      const dg_half2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t u = cw[2 * p] | (cw[2 * p + 1] << 16);
        const dg_half2 sp = __builtin_bit_cast(dg_half2, sw[2 * p] | (sw[2 * p + 1] << 16));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dg_half2 h = __builtin_bit_cast(dg_half2, ((u >> (4 * j)) & 0x000F000Fu) ^ 0x64086408u);
          h = (h - off) * sp;
          bw[j][p] = __builtin_bit_cast(uint32_t, h);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const half8 bf = __builtin_bit_cast(half8, (u32x4){bw[j][0], bw[j][1], bw[j][2], bw[j][3]});
#pragma unroll
        for (int i = 0; i < 8; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf, acc[i][j], 0, 0, 0);
      }
    }
  };
  auto sync = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(SQ_WAIT_VM0);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  issue(0, dg_a0, dg_b0, dg_s0);
  sync();
  for (int64_t st = 0; st < NS; st += 2) {
    if (st + 1 < NS) issue(st + 1, dg_a1, dg_b1, dg_s1);
    compute(dg_a0, dg_b0, dg_s0);
    sync();
    if (st + 1 >= NS) break;
    if (st + 2 < NS) issue(st + 2, dg_a0, dg_b0, dg_s0);
    compute(dg_a1, dg_b1, dg_s1);
    sync();
  }

  // rank-r term: t (times 2^(11-E)) @ (H down)^T, bf16 hi/lo on MFMA
  const int64_t rbase = m0 + 128 * wm, cbase = k0 + 64 * wn;
  for (int rr = 0; rr < rank; rr += 32) {
    bf16x8 ah[8], al[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
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
      for (int i = 0; i < 8; ++i) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bh, acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[i], bh, acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bl, acc[i][j], 0, 0, 0);
      }
    }
  }

  // store C: acc[i][j][v] is row 128 wm + 16 i + 4g + v, column 64 wn + 4f + j;
  // the descriptor ends at row m, so rows of a ragged last tile are dropped
  const __amdgpu_buffer_rsrc_t o_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(cbuf + m0 * k), (short)0, (int)(a_rows * k * 4), 0x00020000);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t r = 128 * wm + 16 * i + 4 * g + v;
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
  const int64_t sps = (steps + slices - 1) / slices;
  p.stats_sps = (int)sps;
  p.stats_slices = (int)((steps + sps - 1) / sps);
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
  if (p.rank > 0) {
    const int64_t cnt = p.n * p.rank;
    hipLaunchKernelGGL(k_dg_transpose, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, stream,
                       up, b.upT, p.n, p.rank);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const dim3 sgrid(strips, (unsigned)p.stats_slices);
  if (p.rank == 0)
    hipLaunchKernelGGL(k_dg_stats<0>, sgrid, dim3(64 * DG_WAVES), 0, stream, dy, b.upT, p.m, p.n,
                       p.stats_sps, b.amax, b.tpart);
  else if (p.rank == 32)
    hipLaunchKernelGGL(k_dg_stats<32>, sgrid, dim3(64 * DG_WAVES), 0, stream, dy, b.upT, p.m,
                       p.n, p.stats_sps, b.amax, b.tpart);
  else
    hipLaunchKernelGGL(k_dg_stats<64>, sgrid, dim3(64 * DG_WAVES), 0, stream, dy, b.upT, p.m,
                       p.n, p.stats_sps, b.amax, b.tpart);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(k_dg_scale, dim3(strips, (unsigned)((p.n + 255) / 256)), dim3(256), 0, stream,
                     dy, p.m, p.n, p.rank, p.stats_slices, b.amax, b.tpart, b.dy16, b.thi, b.tlo,
                     b.rowscale);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (p.rank == 32)
    hipLaunchKernelGGL(k_dg_hdown<32>, dim3((unsigned)(p.k / 256)), dim3(256), 0, stream, down,
                       b.hd_hi, b.hd_lo);
  else if (p.rank == 64)
    hipLaunchKernelGGL(k_dg_hdown<64>, dim3((unsigned)(p.k / 256)), dim3(256), 0, stream, down,
                       b.hd_hi, b.hd_lo);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const unsigned tiles = (unsigned)(((p.m + 255) / 256) * (p.k / 256));
  if (p.group == 32)
    hipLaunchKernelGGL(k_dgrad_gemm<5>, dim3(tiles), dim3(DG_THREADS), 0, stream, b.dy16, codes,
                       scales, b.thi, b.tlo, b.hd_hi, b.hd_lo, b.cbuf, p.m, p.n, p.k, p.rank);
  else
    hipLaunchKernelGGL(k_dgrad_gemm<6>, dim3(tiles), dim3(DG_THREADS), 0, stream, b.dy16, codes,
                       scales, b.thi, b.tlo, b.hd_hi, b.hd_lo, b.cbuf, p.m, p.n, p.k, p.rank);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(k_dg_finish,
                     dim3(strips, (unsigned)((p.k / 256 + DG_WAVES - 1) / DG_WAVES)),
                     dim3(64 * DG_WAVES), 0, stream, b.cbuf, b.rowscale, dx, p.m, p.k, dx_bf16);
  return hipGetLastError();
}

}  // namespace sq
