// Builder-side quantizer (SquareQ README, "SquareQ v3 - W4": the "Residual
// codecs" bullet - int4 with group-32/64 scales whose fraction comes from an
// MSE sweep - applied to the rotated residual of the format formula):
//
//   E = W - up @ down^T ;  R = E @ H ;  per group of G values of R with absmax a:
//   s_i = fp16((70+i)/700 * a), q = clamp(rne(r/s_i), -8, 7), err_i = sum (r - q s_i)^2
//   for i = 0..30; the first i with the least error is kept.
//
// One wave per 16 rows x one 256-column block, in the same lane layout as the
// reconstruct kernel: each lane holds 64 consecutive values of one row, i.e.
// two whole g32 groups or one g64 group, so the whole sweep of a group runs
// inside one lane with no cross-lane reduction.
#include "sq_device.hpp"
#include "sq_kernels.h"

namespace sq {

// f_i / 7 = (70 + i) / 700 rounded to fp32 (31 constants).
__constant__ float c_frac7[31] = {
    70.f / 700, 71.f / 700, 72.f / 700, 73.f / 700, 74.f / 700, 75.f / 700, 76.f / 700,
    77.f / 700, 78.f / 700, 79.f / 700, 80.f / 700, 81.f / 700, 82.f / 700, 83.f / 700,
    84.f / 700, 85.f / 700, 86.f / 700, 87.f / 700, 88.f / 700, 89.f / 700, 90.f / 700,
    91.f / 700, 92.f / 700, 93.f / 700, 94.f / 700, 95.f / 700, 96.f / 700, 97.f / 700,
    98.f / 700, 99.f / 700, 100.f / 700};

__device__ __forceinline__ float fp16_round_f32(float v) { return (float)(_Float16)v; }

// Sweep one group of G values held in v[off .. off+G).  Returns the chosen
// scale (an fp16 value, as fp32) and index; writes the codes' nibbles into
// `nib` (one byte per value, two's complement in the low 4 bits).
template <int G>
__device__ __forceinline__ void sweep_group(const float (&v)[64], int off, float& s_out, int& i_out,
                                            int& flags) {
  float a = 0.0f;
  bool finite = true;
#pragma unroll
  for (int e = 0; e < G; ++e) {
    a = __builtin_fmaxf(a, __builtin_fabsf(v[off + e]));
    finite &= (v[off + e] - v[off + e]) == 0.0f;   // false for NaN and +-inf
  }
  if (!finite) flags |= 1;
  // the largest candidate (f = 1.00) bounds all others
  if (__builtin_isinf(fp16_round_f32(a * c_frac7[30]))) flags |= 2;
  float best = __builtin_inff();
  float s_best = 0.0f;
  int i_best = 0;
  for (int i = 0; i < 31; ++i) {
    const float s = fp16_round_f32(a * c_frac7[i]);
    const float inv = s > 0.0f ? 1.0f / s : 0.0f;
    float err = 0.0f;
#pragma unroll
    for (int e = 0; e < G; ++e) {
      const float r = v[off + e];
      const float q = __builtin_amdgcn_fmed3f(__builtin_rintf(r * inv), -8.0f, 7.0f);
      const float d = __builtin_fmaf(-q, s, r);
      err = __builtin_fmaf(d, d, err);
    }
    if (err < best) {   // strict: the first minimum wins
      best = err;
      s_best = s;
      i_best = i;
    }
  }
  s_out = s_best;
  i_out = i_best;
}

__global__ void __launch_bounds__(256) k_quantize(const float* __restrict__ w,
                                                   const uint16_t* __restrict__ up,
                                                   const uint16_t* __restrict__ down,
                                                   uint8_t* __restrict__ codes,
                                                   uint16_t* __restrict__ scales,
                                                   uint8_t* __restrict__ fidx,
                                                   int32_t* __restrict__ flags_out, int64_t n,
                                                   int64_t k, int group, int rank) {
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
      f32x4 x = src[j];   // plain loads stream faster than non-temporal ones on gfx950
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
#pragma unroll
  for (int i = 0; i < 64; ++i) v[i] *= 0.0625f;
  if (!live) return;

  int flags = 0;
  float s0, s1 = 0.0f;
  int i0, i1 = 0;
  if (group == 32) {
    sweep_group<32>(v, 0, s0, i0, flags);
    sweep_group<32>(v, 32, s1, i1, flags);
  } else {
    sweep_group<64>(v, 0, s0, i0, flags);
  }

  // the forward's fp16(q s) stays finite only while 8 s <= 65504
  if (s0 > 8188.0f || s1 > 8188.0f) flags |= 4;

  // codes of the chosen scales, packed two per byte (even column low)
  u32x4 out[2];
  const float inv0 = s0 > 0.0f ? 1.0f / s0 : 0.0f;
  const float inv1 = group == 32 ? (s1 > 0.0f ? 1.0f / s1 : 0.0f) : inv0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float inv = j < 4 ? inv0 : inv1;
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float q = __builtin_amdgcn_fmed3f(__builtin_rintf(v[8 * j + e] * inv), -8.0f, 7.0f);
      word |= ((uint32_t)(int)q & 0xFu) << (4 * e);
    }
    out[j >> 2][j & 3] = word;
  }
  u32x4* dst = reinterpret_cast<u32x4*>(codes + row * (k >> 1) + (col >> 1));
  dst[0] = out[0];
  dst[1] = out[1];
  uint16_t* srow = scales + row * (k / group);
  if (group == 32) {
    const uint32_t two = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)s0) |
                         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)s1) << 16);
    *reinterpret_cast<uint32_t*>(srow + (col >> 5)) = two;
    if (fidx) {
      uint8_t* frow = fidx + row * (k >> 5) + (col >> 5);
      frow[0] = (uint8_t)i0;
      frow[1] = (uint8_t)i1;
    }
  } else {
    srow[col >> 6] = __builtin_bit_cast(uint16_t, (_Float16)s0);
    if (fidx) fidx[row * (k >> 6) + (col >> 6)] = (uint8_t)i0;
  }
  if (flags) __hip_atomic_fetch_or(flags_out, flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_quantize(const float* w, const uint16_t* up, const uint16_t* down,
                           uint8_t* codes, uint16_t* scales, uint8_t* fidx, int32_t* flags,
                           int64_t n, int64_t k, int group, int rank, hipStream_t stream) {
  const int64_t nblk = k >> 8;
  dim3 grid((unsigned)((n + 15) / 16), (unsigned)((nblk + 3) / 4));
  hipLaunchKernelGGL(k_quantize, grid, dim3(256), 0, stream, w, up, down, codes, scales, fidx,
                     flags, n, k, group, rank);
  return hipGetLastError();
}

}  // namespace sq
