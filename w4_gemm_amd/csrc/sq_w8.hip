// Builder-side quantizer of the int8-residual mode (SquareQ README, "v3.1 -
// int8-residual mode": the format formula with an int8 residual; the sweep
// is the W4 mode's "Residual codecs" bullet on the int8 grid with one scale
// per output row):
//
//   E = W - up @ down^T ;  R = E @ H ;  per row of R with absmax a:
//   s_i = fp16((70+i)/12700 * a), q = clamp(rne(r/s_i), -128, 127),
//   err_i = sum over the row of (r - q s_i)^2 for i = 0..30; the first i with
//   the least error is kept.
//
// A row's scale depends on all K values of the row, so the work splits in
// two launches around an fp32 copy of R in the caller's workspace:
//   1. k_q8_rotate: one wave per 16 rows x one 256-column block (the lane
//      layout of the W4 quantizer): residual, butterflies, 1/16, store R and
//      each lane's absmax of its 64 values.
//   2. k_q8_sweep: one workgroup per row.  Every thread takes a strided
//      quarter-row share of R and accumulates the 31 candidates' errors in
//      registers in a single pass; the sums meet in a fixed-order reduction,
//      thread 0 picks the first minimum, and a second pass writes the codes.
#include "sq_device.hpp"
#include "sq_kernels.h"

namespace sq {

// (70 + i) / 12700 rounded to fp32 (31 constants): f_i / 127.
__constant__ float c_frac127[31] = {
    70.f / 12700, 71.f / 12700, 72.f / 12700, 73.f / 12700, 74.f / 12700, 75.f / 12700,
    76.f / 12700, 77.f / 12700, 78.f / 12700, 79.f / 12700, 80.f / 12700, 81.f / 12700,
    82.f / 12700, 83.f / 12700, 84.f / 12700, 85.f / 12700, 86.f / 12700, 87.f / 12700,
    88.f / 12700, 89.f / 12700, 90.f / 12700, 91.f / 12700, 92.f / 12700, 93.f / 12700,
    94.f / 12700, 95.f / 12700, 96.f / 12700, 97.f / 12700, 98.f / 12700, 99.f / 12700,
    100.f / 12700};

// Launch 1: grid (ceil(n/16), ceil(nblk/4)), four waves per workgroup, wave w
// of workgroup (i, j) on rows 16i.. and block 4j + w.  Writes rbuf [n][k] and
// amax [n][k/64] (entry 4 blk + g of a row: the absmax of columns
// 256 blk + 64 g .. +63).
__global__ void __launch_bounds__(256) k_q8_rotate(const float* __restrict__ w,
                                                    const uint16_t* __restrict__ up,
                                                    const uint16_t* __restrict__ down,
                                                    float* __restrict__ rbuf,
                                                    float* __restrict__ amax,
                                                    int32_t* __restrict__ flags_out, int64_t n,
                                                    int64_t k, int rank) {
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
  float a = 0.0f;
  bool finite = true;
  f32x4* dst = reinterpret_cast<f32x4*>(rbuf + row * k + col);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    f32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float r = v[4 * j + e] * 0.0625f;
      finite &= (r - r) == 0.0f;   // false for NaN and +-inf
      a = __builtin_fmaxf(a, __builtin_fabsf(r));
      o[e] = r;
    }
    dst[j] = o;
  }
  amax[row * (k >> 6) + 4 * blk + g] = a;
  if (!finite) __hip_atomic_fetch_or(flags_out, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, d, 64));
  return v;
}

// Launch 2: one workgroup of 256 threads per row.  Thread t owns the 4-value
// chunks t, t + 256, t + 512, ... of the row.
__global__ void __launch_bounds__(256) k_q8_sweep(const float* __restrict__ rbuf,
                                                   const float* __restrict__ amax,
                                                   int8_t* __restrict__ codes,
                                                   uint16_t* __restrict__ scales,
                                                   uint8_t* __restrict__ fidx,
                                                   int32_t* __restrict__ flags_out, int64_t n,
                                                   int64_t k) {
  __shared__ float s_red[4][32];
  __shared__ float s_am[4];
  __shared__ float s_pick;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const float* rrow = rbuf + row * k;
  const int na = (int)(k >> 6);

  float a = 0.0f;
  for (int i = tid; i < na; i += 256) a = __builtin_fmaxf(a, amax[row * na + i]);
  a = wave_max(a);
  if (lane == 0) s_am[wave] = a;
  __syncthreads();
  a = __builtin_fmaxf(__builtin_fmaxf(s_am[0], s_am[1]), __builtin_fmaxf(s_am[2], s_am[3]));

  float sc[31], inv[31], err[31];
#pragma unroll
  for (int i = 0; i < 31; ++i) {
    sc[i] = (float)(_Float16)(a * c_frac127[i]);
    inv[i] = sc[i] > 0.0f ? 1.0f / sc[i] : 0.0f;
    err[i] = 0.0f;
  }
  const int64_t chunks = k >> 2;
  for (int64_t ch = tid; ch < chunks; ch += 256) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(rrow + 4 * ch);
#pragma unroll
    for (int i = 0; i < 31; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float q = __builtin_amdgcn_fmed3f(__builtin_rintf(x[e] * inv[i]), -128.0f, 127.0f);
        const float d = __builtin_fmaf(-q, sc[i], x[e]);
        err[i] = __builtin_fmaf(d, d, err[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 31; ++i) {
    const float e = wave_sum(err[i]);
    if (lane == 0) s_red[wave][i] = e;
  }
  __syncthreads();
  if (tid == 0) {
    float best = __builtin_inff();
    int ib = 0;
    for (int i = 0; i < 31; ++i) {
      const float e = ((s_red[0][i] + s_red[1][i]) + s_red[2][i]) + s_red[3][i];
      if (e < best) {   // strict: the first minimum wins
        best = e;
        ib = i;
      }
    }
    const float s = (float)(_Float16)(a * c_frac127[ib]);
    s_pick = s;
    scales[row] = __builtin_bit_cast(uint16_t, (_Float16)s);
    if (fidx) fidx[row] = (uint8_t)ib;
    if (__builtin_isinf((float)(_Float16)(a * c_frac127[30])))
      __hip_atomic_fetch_or(flags_out, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const float s = s_pick;
  const float iv = s > 0.0f ? 1.0f / s : 0.0f;
  uint32_t* crow = reinterpret_cast<uint32_t*>(codes + row * k);
  for (int64_t ch = tid; ch < chunks; ch += 256) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(rrow + 4 * ch);
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float q = __builtin_amdgcn_fmed3f(__builtin_rintf(x[e] * iv), -128.0f, 127.0f);
      word |= ((uint32_t)(int)q & 0xFFu) << (8 * e);
    }
    crow[ch] = word;
  }
}

size_t quantize_w8_workspace(int64_t n, int64_t k) {
  const size_t r = ((size_t)n * k * 4 + 255) & ~(size_t)255;
  return r + (size_t)n * (k >> 6) * 4;
}

hipError_t launch_quantize_w8(const float* w, const uint16_t* up, const uint16_t* down,
                              int8_t* codes, uint16_t* scales, uint8_t* fidx, int32_t* flags,
                              int64_t n, int64_t k, int rank, void* workspace,
                              hipStream_t stream) {
  float* rbuf = static_cast<float*>(workspace);
  float* amax = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                         (((size_t)n * k * 4 + 255) & ~(size_t)255));
  const int64_t nblk = k >> 8;
  dim3 grid((unsigned)((n + 15) / 16), (unsigned)((nblk + 3) / 4));
  hipLaunchKernelGGL(k_q8_rotate, grid, dim3(256), 0, stream, w, up, down, rbuf, amax, flags, n,
                     k, rank);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_q8_sweep, dim3((unsigned)n), dim3(256), 0, stream, rbuf, amax, codes,
                     scales, fidx, flags, n, k);
  return hipGetLastError();
}

}  // namespace sq
