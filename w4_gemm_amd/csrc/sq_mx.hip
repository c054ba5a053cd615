// MXFP4 mode (SquareQ README, "SquareQ v3 - W4": the "Residual codecs"
// bullet's FP4 alternative - e2m1 elements with block scales driving native
// FP4 matrix instructions - and the op-level parity line that describes the
// FP4 forward as rotate + block-quant of the activations + FP4 product +
// epilogue).  The page's NVFP4 layout is one vendor's; this is its OCP MX
// counterpart, which gfx950's scaled MFMA takes directly:
//
//   element  E2M1 (+-{0, 0.5, 1, 1.5, 2, 3, 4, 6}), nibble s<<3 | e<<1 | m
//   block    32 consecutive values along K share an E8M0 scale 2^(e-127),
//            e = floor(log2 absmax) - 2 + 127 clamped to [0, 254]
//   rounding nearest, ties to the even mantissa, saturating at 6
//
//   y = dq(Q(x H)) @ dq(Q(R))^T + (x @ down) @ up^T
//   W_hat = up @ down^T + dq(Q(R)) @ H
//
// Kernels:
//   k_mx_quant_weight  residual, 256-point butterflies, MXFP4 of R (builder)
//   k_mx_quant_act     butterflies of x, MXFP4 of x H, and the block's share
//                      of t = x @ down on bf16 MFMA (fixed-order partials)
//   k_mx_tsum          t = sum of the partials in order, split into bf16 hi + lo
//   k_mx_gemm          the FP4 x FP4 product on v_mfma_scale_f32_16x16x128_f8f6f4
//                      plus the rank-r branch, fp32 or bf16 out
// and bf16 W_hat from the strip kernel of the reconstruct (group code 1).
#include <algorithm>

#include "sq_device.hpp"
#include "sq_kernels.h"

namespace sq {

// ---------------------------------------------------------------- codec
// Magnitude nibble of u = |v| / 2^(e-127) (u exact: a power-of-two scaling).
// Each comparison adds one when u passes a midpoint of the E2M1 grid; at a
// midpoint the inclusive or exclusive side picks the even mantissa
// (0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4),
// and everything past 5 saturates to 6.
__device__ __forceinline__ uint32_t e2m1_mag(float u) {
  return (uint32_t)(u > 0.25f) + (uint32_t)(u >= 0.75f) + (uint32_t)(u > 1.25f) +
         (uint32_t)(u >= 1.75f) + (uint32_t)(u > 2.5f) + (uint32_t)(u >= 3.5f) +
         (uint32_t)(u > 5.0f);
}

// E8M0 exponent of a block with fp32 absmax a: floor(log2 a) + 127 is the
// biased fp32 exponent field (0 for zero and subnormal a), minus 2, floored
// at 0.
__device__ __forceinline__ uint32_t mx_exponent(float a) {
  const int ef = (int)((__float_as_uint(a) >> 23) & 0xFFu);
  return (uint32_t)max(ef - 2, 0);
}

// 1 / 2^(e-127) = 2^(127-e) as fp32 bits (e <= 252, so always normal).
__device__ __forceinline__ float mx_inv_scale(uint32_t e) {
  return __uint_as_float((254u - e) << 23);
}

// 32 values v[off .. off+32) -> exponent byte and 16 bytes of nibbles (even
// element low).
__device__ __forceinline__ uint32_t mx_encode32(const float (&v)[64], int off, u32x4& out) {
  float a = 0.0f;
#pragma unroll
  for (int e = 0; e < 32; ++e) a = __builtin_fmaxf(a, __builtin_fabsf(v[off + e]));
  const uint32_t ex = mx_exponent(a);
  const float inv = mx_inv_scale(ex);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = v[off + 8 * w + e];
      const uint32_t mag = e2m1_mag(__builtin_fabsf(x) * inv);
      const uint32_t nib = mag | ((mag != 0u && x < 0.0f) ? 8u : 0u);
      word |= nib << (4 * e);
    }
    out[w] = word;
  }
  return ex;
}

// ---------------------------------------------------------------- weight quantizer
// One wave per 16 rows x one 256-column block (the W4 quantizer's lane
// layout: each lane holds 64 consecutive values of one row, two MX blocks).
__global__ void __launch_bounds__(256) k_mx_quant_weight(
    const float* __restrict__ w, const uint16_t* __restrict__ up, const uint16_t* __restrict__ down,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ exps, int32_t* __restrict__ flags_out,
    int64_t n, int64_t k, int rank) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t nblk = k >> 8;
  const int64_t blk = (int64_t)blockIdx.y * 4 + wave;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  if (blk >= nblk) return;
  const int c = lane & 15, g = lane >> 4;
  const int64_t row = row0 + c;
  const bool live = row < n;
  const int64_t col = blk * 256 + 64 * g;

  float v[64];
  if (live) {
    const f32x4* src = reinterpret_cast<const f32x4*>(w + row * k + col);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const f32x4 x = src[j];
      v[4 * j] = x[0];
      v[4 * j + 1] = x[1];
      v[4 * j + 2] = x[2];
      v[4 * j + 3] = x[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) v[i] = 0.0f;
  }
  lowrank_acc_16x256(v, up, down, row0, n, blk * 256, rank, true, lane);   // E = W - up down^T
  fwht256_wave(v, lane);
  if (!live) return;
  bool finite = true;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    v[i] *= 0.0625f;
    finite &= (v[i] - v[i]) == 0.0f;
  }
  u32x4 o0, o1;
  const uint32_t e0 = mx_encode32(v, 0, o0), e1 = mx_encode32(v, 32, o1);
  u32x4* dst = reinterpret_cast<u32x4*>(codes + row * (k >> 1) + (col >> 1));
  dst[0] = o0;
  dst[1] = o1;
  *reinterpret_cast<uint16_t*>(exps + row * (k >> 5) + (col >> 5)) = (uint16_t)(e0 | (e1 << 8));
  if (!finite) __hip_atomic_fetch_or(flags_out, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- activations
constexpr int MX_PRE_WAVES = 4;

// down [K][r] -> downT [r][K] (the MFMA B operand of x @ down as 16-byte rows).
__global__ void __launch_bounds__(256) k_mx_transpose(const uint16_t* __restrict__ down,
                                                       uint16_t* __restrict__ downT, int64_t k,
                                                       int rank) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= k * rank) return;
  const int64_t r = i / k, kk = i - r * k;
  downT[i] = down[kk * rank + r];
}

// Grid (ceil(m/16), ceil(nblk/4)); wave w of workgroup (i, j) owns rows 16i..
// and block 4j + w.  Writes xq [m][k/2], the exponents and, when rank > 0,
// the workgroup's partial t_part[j][row][r] (its four blocks summed in wave
// order).  Exponents: PERM = false, xs [m][k/32]; PERM = true, the order in
// which the contraction's MFMA lanes use them: for every 128-row group R and
// 128-value stage s a 512-byte record [g][fr][i] holding the exponent of row
// 128R + 16i + fr, block 4s + g (one 8-byte read per lane and stage).
__device__ __forceinline__ int64_t mx_perm_exp_index(int64_t row, int64_t blk32, int64_t k) {
  const int64_t grp = row >> 7, s = blk32 >> 2;
  return (grp * (k >> 7) + s) * 512 + (blk32 & 3) * 128 + (row & 15) * 8 + ((row >> 4) & 7);
}

template <int RANK, bool PERM>
__global__ void __launch_bounds__(64 * MX_PRE_WAVES) k_mx_quant_act(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ downT, uint8_t* __restrict__ xq,
    uint8_t* __restrict__ xs, float* __restrict__ t_part, int64_t m, int64_t k) {
  constexpr int RT = RANK / 16;
  __shared__ float red_t[MX_PRE_WAVES][16][RANK > 0 ? RANK : 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int64_t nblk = k >> 8;
  const int64_t blk = (int64_t)blockIdx.y * MX_PRE_WAVES + wave;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int64_t lrow = min(row0 + c, m - 1);   // rows past m repeat the last row
  const bool have = blk < nblk;

  if (RANK > 0) {
    f32x4 acc[RT > 0 ? RT : 1] = {};
    if (have) {
      // MFMA s contracts columns 32s .. 32s+31 of the block; lane (c, g)
      // holds columns 32s + 8g .. +8 of row c
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int64_t col = blk * 256 + 32 * s + 8 * g;
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(x + lrow * k + col);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const bf16x8 bf = *reinterpret_cast<const bf16x8*>(downT + (int64_t)(16 * rt + c) * k + col);
          acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[rt], 0, 0, 0);
        }
      }
    }
    // acc[rt][i] = partial t[row0 + 4g + i][16 rt + c]
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red_t[wave][4 * g + i][16 * rt + c] = acc[rt][i];
    __syncthreads();
    for (int i = tid; i < 16 * RANK; i += 64 * MX_PRE_WAVES) {
      const int rr = i / RANK, r = i - rr * RANK;
      if (row0 + rr >= m) continue;
      float t = 0.0f;
#pragma unroll
      for (int ww = 0; ww < MX_PRE_WAVES; ++ww) t += red_t[ww][rr][r];
      t_part[((int64_t)blockIdx.y * m + row0 + rr) * RANK + r] = t;
    }
  }
  if (!have) return;

  // the lane's 64 consecutive columns of its row, rotated with the block
  // (rows past m work on the last row and store nothing)
  const int64_t col = blk * 256 + 64 * g;
  float v[64];
  const u32x4* src = reinterpret_cast<const u32x4*>(x + lrow * k + col);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const u32x4 q = src[j];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[8 * j + 2 * e] = bf16_to_f32(q[e] & 0xFFFFu);
      v[8 * j + 2 * e + 1] = bf16_to_f32(q[e] >> 16);
    }
  }
  fwht256_wave(v, lane);
#pragma unroll
  for (int i = 0; i < 64; ++i) v[i] *= 0.0625f;
  u32x4 o0, o1;
  const uint32_t e0 = mx_encode32(v, 0, o0), e1 = mx_encode32(v, 32, o1);
  const int64_t row = row0 + c;
  if (row >= m) return;
  u32x4* dst = reinterpret_cast<u32x4*>(xq + row * (k >> 1) + (col >> 1));
  dst[0] = o0;
  dst[1] = o1;
  if constexpr (PERM) {
    xs[mx_perm_exp_index(row, col >> 5, k)] = (uint8_t)e0;
    xs[mx_perm_exp_index(row, (col >> 5) + 1, k)] = (uint8_t)e1;
  } else {
    *reinterpret_cast<uint16_t*>(xs + row * (k >> 5) + (col >> 5)) = (uint16_t)(e0 | (e1 << 8));
  }
}

// t = sum over the slices in order, split into bf16 hi + lo (t - hi rounded).
__global__ void __launch_bounds__(256) k_mx_tsum(const float* __restrict__ t_part,
                                                  uint16_t* __restrict__ thi,
                                                  uint16_t* __restrict__ tlo, int64_t m, int rank,
                                                  int slices) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= m * rank) return;
  // fixed summation order; the loads of a group of eight are all in flight
  float t = 0.0f;
  int q = 0;
  for (; q + 8 <= slices; q += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = t_part[(int64_t)(q + u) * m * rank + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) t += v[u];
  }
  for (; q < slices; ++q) t += t_part[(int64_t)q * m * rank + i];
  const uint16_t hb = f32_to_bf16(t);
  thi[i] = hb;
  tlo[i] = f32_to_bf16(t - bf16_to_f32(hb));
}

// ---------------------------------------------------------------- FP4 contraction
// 256 x 256 output tile per workgroup, eight waves of 128 x 64 (8 x 4 MFMA
// tiles of 16 x 16).  One stage = 128 K values: 64 bytes of codes per row of
// each operand and one 4-byte word of block exponents per row.  Operands
// stream global -> LDS with direct 16-byte (codes) and 4-byte (exponents)
// buffer loads into three stage buffers, two stages ahead of the MFMAs.
// Code rows are 64 bytes; chunk c of row r sits at slot c ^ ((r >> 1) & 3),
// which puts the eight rows read by each quarter of a fragment load in eight
// different 16-byte bank groups.  MFMA operand of lane (r, g): the 16 bytes of
// K block g of row r, and that block's exponent byte as its scale.
constexpr int MXG_BM = 256, MXG_BN = 256, MXG_THREADS = 512;
constexpr int MXG_CODE_BYTES = 256 * 64;   // one operand's codes for one stage
constexpr int MXG_EXP_BYTES = 256 * 4;     // one operand's exponents for one stage

__shared__ __attribute__((aligned(16))) uint8_t mx_a0[MXG_CODE_BYTES];
__shared__ __attribute__((aligned(16))) uint8_t mx_a1[MXG_CODE_BYTES];
__shared__ __attribute__((aligned(16))) uint8_t mx_a2[MXG_CODE_BYTES];
__shared__ __attribute__((aligned(16))) uint8_t mx_b0[MXG_CODE_BYTES];
__shared__ __attribute__((aligned(16))) uint8_t mx_b1[MXG_CODE_BYTES];
__shared__ __attribute__((aligned(16))) uint8_t mx_b2[MXG_CODE_BYTES];
__shared__ __attribute__((aligned(16))) uint8_t mx_sa0[MXG_EXP_BYTES];
__shared__ __attribute__((aligned(16))) uint8_t mx_sa1[MXG_EXP_BYTES];
__shared__ __attribute__((aligned(16))) uint8_t mx_sa2[MXG_EXP_BYTES];
__shared__ __attribute__((aligned(16))) uint8_t mx_sb0[MXG_EXP_BYTES];
__shared__ __attribute__((aligned(16))) uint8_t mx_sb1[MXG_EXP_BYTES];
__shared__ __attribute__((aligned(16))) uint8_t mx_sb2[MXG_EXP_BYTES];

typedef __attribute__((address_space(3))) void* mx_lds_t;
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// SKIP (grids with a single ragged tile row): a wave leaves out the MFMAs of
// 16-row fragments that lie wholly past row m.
template <bool SKIP>
__global__ void __launch_bounds__(MXG_THREADS, 1) k_mx_gemm(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ ws,
    const uint16_t* __restrict__ thi, const uint16_t* __restrict__ tlo,
    const uint16_t* __restrict__ up, void* __restrict__ y, int64_t m, int64_t n, int64_t k,
    int rank, int y_bf16, int splits, float* __restrict__ partial) {
  constexpr int FM = 8, FN = 4;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int64_t mt = (m + MXG_BM - 1) / MXG_BM, nt = (n + MXG_BN - 1) / MXG_BN;
  // workgroup b: split b / tiles of tile b % tiles
  const uint32_t tiles = (uint32_t)(mt * nt);
  const int split = __builtin_amdgcn_readfirstlane((int)(blockIdx.x / tiles));
  int64_t tile_m, tile_n;
  xcd_tile(blockIdx.x - (uint32_t)split * tiles, tiles, nt, tile_m, tile_n);
  // the tile indices come out of 64-bit divisions done on the vector unit;
  // pin them to scalar registers so that the buffer descriptors built from
  // them stay scalar (a descriptor in vector registers turns every load into
  // a loop over lanes)
  tile_m = __builtin_amdgcn_readfirstlane((int)tile_m);
  tile_n = __builtin_amdgcn_readfirstlane((int)tile_n);
  const int64_t m0 = tile_m * MXG_BM, n0 = tile_n * MXG_BN;
  // this split's stages kb .. kb + KT - 1 (128 K values each)
  const int64_t kall = k >> 7;
  const int64_t kb = __builtin_amdgcn_readfirstlane((int)((int64_t)split * kall / splits));
  const int64_t KT =
      __builtin_amdgcn_readfirstlane((int)(((int64_t)split + 1) * kall / splits)) - kb;
  const int64_t hk = k >> 1, ek = k >> 5;   // code and exponent bytes per row
  const int fr = lane & 15, g = lane >> 4;

  const int64_t a_rows = min((int64_t)MXG_BM, m - m0), b_rows = min((int64_t)MXG_BN, n - n0);
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(xq + m0 * hk), (short)0, (int)(a_rows * hk), 0x00020000);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(wq + n0 * hk), (short)0, (int)(b_rows * hk), 0x00020000);
  // activation exponents in the lane order (see k_mx_quant_act): the tile's
  // two 128-row groups, 512 bytes per group and stage
  const int64_t ks = k >> 7;
  const int64_t a_groups = (m + 127) >> 7;
  const __amdgpu_buffer_rsrc_t sa_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)xs, (short)0, (int)(a_groups * ks * 512), 0x00020000);
  const __amdgpu_buffer_rsrc_t sb_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(ws + n0 * ek), (short)0, (int)(b_rows * ek), 0x00020000);

  // loaders: wave w fills code rows 32w .. 32w+31 of both operands (two
  // instructions of 16 rows each); waves 0-3 each load a 256-byte quarter
  // of the stage's 1 KB of activation exponents (group w/2, half w%2; a
  // group past the last one reads zeros), waves 4-7 the weight exponent
  // words of rows 64(w-4) .. +64 (rows past the matrix edge repeat the last)
  uint32_t c_off_a[2], c_off_b[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 32 * wave + 16 * i + (lane >> 2);
    const uint32_t slot = (uint32_t)((lane & 3) ^ ((r >> 1) & 3));
    c_off_a[i] = (uint32_t)min((int64_t)r, a_rows - 1) * (uint32_t)hk + 16u * slot;
    c_off_b[i] = (uint32_t)min((int64_t)r, b_rows - 1) * (uint32_t)hk + 16u * slot;
  }
  const bool exp_a = wave < 4;
  const uint32_t e_off =
      exp_a ? (uint32_t)((((m0 >> 7) + (wave >> 1)) * ks) * 512 + (wave & 1) * 256 + lane * 4)
            : (uint32_t)min((int64_t)(64 * (wave & 3) + lane), b_rows - 1) * (uint32_t)ek;

  auto issue = [&](int64_t kl, uint8_t* ab, uint8_t* bb, uint8_t* sab, uint8_t* sbb) {
    const int64_t kt = kb + kl;
    const int so = (int)(kt * 64);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (mx_lds_t)(ab + (32 * wave + 16 * i) * 64), 16,
                                               c_off_a[i], so, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (mx_lds_t)(bb + (32 * wave + 16 * i) * 64), 16,
                                               c_off_b[i], so, 0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(exp_a ? sa_rsrc : sb_rsrc,
                                             (mx_lds_t)((exp_a ? sab : sbb) + 256 * (wave & 3)), 4,
                                             e_off, (int)(kt * (exp_a ? 512 : 4)), 0, 0);
  };

  // fragment addresses (rows 16i + fr share the swizzle of fr)
  const uint32_t swz = (uint32_t)(g ^ ((fr >> 1) & 3));
  const uint32_t a_lane = (uint32_t)(128 * wm + fr) * 64 + 16 * swz;
  const uint32_t b_lane = (uint32_t)(64 * wn + fr) * 64 + 16 * swz;
  const uint32_t sa_lane = (uint32_t)(512 * wm + 128 * g + 8 * fr);
  const uint32_t sb_lane = (uint32_t)(64 * wn + fr) * 4 + g;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int64_t mleft = m - (m0 + 128 * wm);   // live rows of the wave's 128
  auto compute = [&](const uint8_t* ab, const uint8_t* bb, const uint8_t* sab, const uint8_t* sbb) {
    i32x8 bf[FN];
    int sbv[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const u32x4 q = *reinterpret_cast<const u32x4*>(bb + b_lane + j * 1024);
      bf[j] = (i32x8){(int)q[0], (int)q[1], (int)q[2], (int)q[3], 0, 0, 0, 0};
      sbv[j] = sbb[sb_lane + j * 64];
    }
    // the eight A exponents of the lane in one read; byte i & 3 of word i / 4
    // is selected by the instruction's scale byte select
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 sa8 = *reinterpret_cast<const u32x2*>(sab + sa_lane);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (SKIP && 16 * i >= mleft) break;
      const u32x4 q = *reinterpret_cast<const u32x4*>(ab + a_lane + i * 1024);
      const i32x8 af = (i32x8){(int)q[0], (int)q[1], (int)q[2], (int)q[3], 0, 0, 0, 0};
      const int sav = (int)sa8[i >> 2];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        switch (i & 3) {
          case 0: acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], acc[i][j], 4, 4, 0, sav, 0, sbv[j]); break;
          case 1: acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], acc[i][j], 4, 4, 1, sav, 0, sbv[j]); break;
          case 2: acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], acc[i][j], 4, 4, 2, sav, 0, sbv[j]); break;
          default: acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], acc[i][j], 4, 4, 3, sav, 0, sbv[j]); break;
        }
      }
    }
  };
  auto sync = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F75);   // vmcnt(5)
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Three buffers in rotation, stage s in buffer s % 3.  Each step waits for
  // its stage (issued two steps earlier; the wait also covers the stage
  // after it, issued one step earlier), meets the other waves at the
  // barrier (after which the buffer of stage s-1 is free), issues stage s+2
  // into it and computes stage s.  Loads past the last stage re-fetch the
  // last one into a buffer that is never read again.
  issue(0, mx_a0, mx_b0, mx_sa0, mx_sb0);
  issue(min((int64_t)1, KT - 1), mx_a1, mx_b1, mx_sa1, mx_sb1);
  for (int64_t kt = 0; kt < KT; kt += 3) {
    sync();
    issue(min(kt + 2, KT - 1), mx_a2, mx_b2, mx_sa2, mx_sb2);
    compute(mx_a0, mx_b0, mx_sa0, mx_sb0);
    if (kt + 1 >= KT) break;
    sync();
    issue(min(kt + 3, KT - 1), mx_a0, mx_b0, mx_sa0, mx_sb0);
    compute(mx_a1, mx_b1, mx_sa1, mx_sb1);
    if (kt + 2 >= KT) break;
    sync();
    issue(min(kt + 4, KT - 1), mx_a1, mx_b1, mx_sa1, mx_sb1);
    compute(mx_a2, mx_b2, mx_sa2, mx_sb2);
  }
  __builtin_amdgcn_s_waitcnt(SQ_WAIT_VM0);   // the re-fetches past the last stage have landed

  const int64_t rbase = m0 + 128 * wm, cbase = n0 + 64 * wn;
  // rank-r branch: (t_hi + t_lo) @ up^T on bf16 MFMA (rank 16: the upper half
  // of the 32-wide step reads zeros); with split-K split 0 adds it and every
  // split stores its fp32 partial sums to partial [splits][m][n]
  if (splits > 1) {
    if (split > 0) rank = 0;
    y = partial + (int64_t)split * m * n;
    y_bf16 = 0;
  }
  for (int rr = 0; rr < rank; rr += 32) {
    const bool rk = rr + 8 * g < rank;
#pragma unroll
    for (int hl = 0; hl < 2; ++hl) {
      const uint16_t* tsrc = hl ? tlo : thi;
      bf16x8 bu[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t c = min(cbase + 16 * j + fr, n - 1);
        bu[j] = rk ? *reinterpret_cast<const bf16x8*>(up + c * rank + rr + 8 * g) : (bf16x8){};
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int64_t r = min(rbase + 16 * i + fr, m - 1);
        const bf16x8 at = rk ? *reinterpret_cast<const bf16x8*>(tsrc + r * rank + rr + 8 * g) : (bf16x8){};
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(at, bu[j], acc[i][j], 0, 0, 0);
      }
    }
  }
  // acc[i][j][v]: row rbase + 16 i + 4 g + v, column cbase + 16 j + fr
  if (y_bf16) {
    // Each wave stages 64 x 64 bf16 (8 KB, 128-byte rows with the chunk
    // swizzle of the W4 kernels) in its own part of the stage buffers, twice,
    // and stores eight whole 128-byte row segments per instruction.
    __syncthreads();   // every wave is done with the stage buffers
    const int wb = wave >> 1;
    uint8_t* st = (wb == 0 ? mx_a0 : wb == 1 ? mx_a1 : wb == 2 ? mx_b0 : mx_b1) + (wave & 1) * 8192;
    const bool full_cols = (cbase + 64 <= n) && ((n & 7) == 0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int lrow = 16 * i + 4 * g + v;
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int col = 16 * j + fr;   // chunk col/8, element col%8
            *reinterpret_cast<uint16_t*>(st + lrow * 128 + 16 * ((col >> 3) ^ a_swz(lrow)) +
                                         2 * (col & 7)) = f32_to_bf16(acc[4 * h + i][j][v]);
          }
        }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int lrow = 8 * it + (lane >> 3), chunk = lane & 7;
        const int64_t r = rbase + 64 * h + lrow, c = cbase + 8 * chunk;
        const u32x4 o = *reinterpret_cast<const u32x4*>(st + lrow * 128 + 16 * (chunk ^ a_swz(lrow)));
        if (r >= m) continue;
        uint16_t* dst = reinterpret_cast<uint16_t*>(y) + r * n + c;
        if (full_cols) {
          *reinterpret_cast<u32x4*>(dst) = o;
        } else {
          const uint16_t* hv = reinterpret_cast<const uint16_t*>(&o);
          for (int e = 0; e < 8 && c + e < n; ++e) dst[e] = hv[e];
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // the reads are done before the next pass writes
      __builtin_amdgcn_wave_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t r = rbase + 16 * i + 4 * g + v;
      if (r >= m) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t c = cbase + 16 * j + fr;
        if (c < n) reinterpret_cast<float*>(y)[r * n + c] = acc[i][j][v];
      }
    }
}

// Split-K sum: y = sum over the splits of partial [splits][m][n], in split
// order.
__global__ void __launch_bounds__(256) k_mx_splitsum(const float* __restrict__ partial,
                                                      void* __restrict__ y, int64_t mn,
                                                      int splits, int y_bf16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= mn) return;
  float s = 0.0f;
  int z = 0;
  for (; z + 8 <= splits; z += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = partial[(int64_t)(z + u) * mn + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; z < splits; ++z) s += partial[(int64_t)z * mn + i];
  if (y_bf16)
    reinterpret_cast<uint16_t*>(y)[i] = f32_to_bf16(s);
  else
    reinterpret_cast<float*>(y)[i] = s;
}

// ---------------------------------------------------------------- host side
static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Split-K factor of the FP4 contraction: one 256 x 256 tile per CU at a time,
// so a grid of fewer than half the chip's 256 CUs splits K into as many
// slices as fill it, each at least 8 stages (1024 K values) long.
static int mx_splits(int64_t m, int64_t n, int64_t k) {
  const int64_t tiles = ((m + MXG_BM - 1) / MXG_BM) * ((n + MXG_BN - 1) / MXG_BN);
  if (tiles >= 128) return 1;
  const int64_t s = std::min<int64_t>(256 / tiles, (k >> 7) / 8);
  return (int)std::max<int64_t>(s, 1);
}

MxPlan plan_mx(int64_t m, int64_t n, int64_t k, int rank) {
  MxPlan p{};
  p.m = m; p.n = n; p.k = k; p.rank = rank;
  p.slices = (int)(((k >> 8) + MX_PRE_WAVES - 1) / MX_PRE_WAVES);
  p.splits = mx_splits(m, n, k);
  size_t off = 0;
  p.off_xq = off;     off = align256(off + (size_t)m * (k >> 1));
  p.off_xs = off;     off = align256(off + (size_t)((m + 127) / 128) * 128 * (k >> 5));
  p.off_downT = off;  off = align256(off + (size_t)k * std::max(rank, 1) * 2);
  p.off_tpart = off;  off = align256(off + (size_t)p.slices * m * std::max(rank, 1) * 4);
  p.off_thi = off;    off = align256(off + (size_t)m * std::max(rank, 1) * 2);
  p.off_tlo = off;    off = align256(off + (size_t)m * std::max(rank, 1) * 2);
  p.off_part = off;   off = align256(off + (p.splits > 1 ? (size_t)p.splits * m * n * 4 : 0));
  p.total = off;
  return p;
}

hipError_t launch_quantize_mx(const float* w, const uint16_t* up, const uint16_t* down,
                              uint8_t* codes, uint8_t* exps, int32_t* flags, int64_t n, int64_t k,
                              int rank, hipStream_t stream) {
  dim3 grid((unsigned)((n + 15) / 16), (unsigned)(((k >> 8) + 3) / 4));
  hipLaunchKernelGGL(k_mx_quant_weight, grid, dim3(256), 0, stream, w, up, down, codes, exps, flags,
                     n, k, rank);
  return hipGetLastError();
}

hipError_t launch_quantize_act_mx(const uint16_t* x, int64_t m, int64_t k, uint8_t* xq, uint8_t* xs,
                                  hipStream_t stream) {
  dim3 grid((unsigned)((m + 15) / 16), (unsigned)(((k >> 8) + MX_PRE_WAVES - 1) / MX_PRE_WAVES));
  hipLaunchKernelGGL((k_mx_quant_act<0, false>), grid, dim3(64 * MX_PRE_WAVES), 0, stream, x,
                     (const uint16_t*)nullptr, xq, xs, (float*)nullptr, m, k);
  return hipGetLastError();
}

hipError_t launch_fwd_mx(const MxPlan& p, const uint16_t* x, const uint8_t* wq, const uint8_t* wsc,
                         const uint16_t* up, const uint16_t* down, void* y, int y_bf16,
                         void* workspace, hipStream_t stream) {
  char* base = static_cast<char*>(workspace);
  uint8_t* xq = reinterpret_cast<uint8_t*>(base + p.off_xq);
  uint8_t* xs = reinterpret_cast<uint8_t*>(base + p.off_xs);
  uint16_t* downT = reinterpret_cast<uint16_t*>(base + p.off_downT);
  float* tpart = reinterpret_cast<float*>(base + p.off_tpart);
  uint16_t* thi = reinterpret_cast<uint16_t*>(base + p.off_thi);
  uint16_t* tlo = reinterpret_cast<uint16_t*>(base + p.off_tlo);
  float* part = reinterpret_cast<float*>(base + p.off_part);
  hipError_t err;
  if (p.rank > 0) {
    const int64_t cnt = p.k * p.rank;
    hipLaunchKernelGGL(k_mx_transpose, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, stream,
                       down, downT, p.k, p.rank);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const dim3 ag((unsigned)((p.m + 15) / 16), (unsigned)p.slices);
#define SQ_MXACT(R)                                                                              \
  hipLaunchKernelGGL((k_mx_quant_act<R, true>), ag, dim3(64 * MX_PRE_WAVES), 0, stream, x,      \
                     (const uint16_t*)downT, xq, xs, tpart, p.m, p.k)
  if (p.rank == 0) SQ_MXACT(0);
  else if (p.rank == 16) SQ_MXACT(16);
  else if (p.rank == 32) SQ_MXACT(32);
  else SQ_MXACT(64);
#undef SQ_MXACT
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (p.rank > 0) {
    const int64_t cnt = p.m * p.rank;
    hipLaunchKernelGGL(k_mx_tsum, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, stream, tpart,
                       thi, tlo, p.m, p.rank, p.slices);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const int64_t tiles = ((p.m + MXG_BM - 1) / MXG_BM) * ((p.n + MXG_BN - 1) / MXG_BN);
  if (p.m < MXG_BM)
    hipLaunchKernelGGL(k_mx_gemm<true>, dim3((unsigned)(tiles * p.splits)), dim3(MXG_THREADS), 0,
                       stream, xq, xs, wq, wsc, thi, tlo, up, y, p.m, p.n, p.k, p.rank, y_bf16,
                       p.splits, part);
  else
    hipLaunchKernelGGL(k_mx_gemm<false>, dim3((unsigned)(tiles * p.splits)), dim3(MXG_THREADS), 0,
                       stream, xq, xs, wq, wsc, thi, tlo, up, y, p.m, p.n, p.k, p.rank, y_bf16,
                       p.splits, part);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (p.splits > 1) {
    const int64_t mn = p.m * p.n;
    hipLaunchKernelGGL(k_mx_splitsum, dim3((unsigned)((mn + 255) / 256)), dim3(256), 0, stream,
                       part, y, mn, p.splits, y_bf16);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

// The reconstruct runs in the strip kernel of the W4 payload (group code 1):
// an exponent row indexes like a row of group-64 fp16 scales.
hipError_t launch_reconstruct_mx(const uint8_t* codes, const uint8_t* exps, const uint16_t* up,
                                 const uint16_t* down, uint16_t* w_hat, int64_t n, int64_t k,
                                 int rank, hipStream_t stream) {
  return launch_reconstruct(codes, reinterpret_cast<const uint16_t*>(exps), up, down, w_hat, n, k,
                            1, rank, stream);
}

}  // namespace sq
