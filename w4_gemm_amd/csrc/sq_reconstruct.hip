// Backward-side rebuild of the dense bf16 weight from the W4 payload
// (SquareQ README, "SquareQ v3 - W4": the format formula; the backward visit
// rebuilds bf16 from the same payload):
//
//   w_hat[n][k] = bf16_rne( sum_r up[n][r] down[k][r] + ((q * s) @ H)[n][k] )
//
// One wave per 16 rows x one 256-column Hadamard block.  Every lane reads
// 32 bytes of codes (64 consecutive columns of one row), dequantizes to fp32
// with the 1/16 of H folded into the scale (exact: power of two), runs the
// 256-point butterflies (six stages in registers, two across lanes), adds the
// low-rank term from bf16 MFMA (exact products, fp32 sums) and writes
// 128 contiguous bytes of bf16.  HBM-bound: reads 0.5 + 2/group bytes and
// writes 2 bytes per weight element.
#include "sq_device.hpp"
#include "sq_kernels.h"

namespace sq {

// Dequantize 64 codes (32 bytes) into q * s16 where s16 = scale / 16.
// Offset binary: nibble ^ 8 = q + 8, converted by v_cvt_f32_ubyte*, then
// fma(q + 8, s16, -8 s16) = q s16 exactly (both products fit in fp32).
__device__ __forceinline__ void dequant64(float (&v)[64], const u32x4 (&w)[2], float s_lo,
                                          float s_hi) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t word = w[j >> 2][j & 3] ^ 0x88888888u;
    const float s = (j < 4) ? s_lo : s_hi;
    const float off = -8.0f * s;
    const uint32_t ev = word & 0x0F0F0F0Fu;          // codes 0,2,4,6 of the word
    const uint32_t od = (word >> 4) & 0x0F0F0F0Fu;   // codes 1,3,5,7
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      v[8 * j + 2 * b] = __builtin_fmaf((float)((ev >> (8 * b)) & 0xFFu), s, off);
      v[8 * j + 2 * b + 1] = __builtin_fmaf((float)((od >> (8 * b)) & 0xFFu), s, off);
    }
  }
}

// LDS staging rows: 256 bf16 = 32 x 16 bytes, padded by one 16-byte slot so
// that the 16 rows written by one instruction start in different banks.
constexpr int STAGE_ROW_U4 = 33;

__global__ void __launch_bounds__(256) k_reconstruct(const uint8_t* __restrict__ codes,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint16_t* __restrict__ up,
                                                      const uint16_t* __restrict__ down,
                                                      uint16_t* __restrict__ w_hat, int64_t n,
                                                      int64_t k, int group, int rank) {
  __shared__ __attribute__((aligned(16))) uint32_t s_stage[4][16][STAGE_ROW_U4 * 4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t nblk = k >> 8;
  const int64_t blk = (int64_t)blockIdx.y * 4 + wave;     // 4 blocks of one row strip
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  if (blk >= nblk) return;
  const int c = lane & 15, g = lane >> 4;
  const int64_t row = row0 + c;
  const bool live = row < n;
  const int64_t col = blk * 256 + 64 * g;

  // payload: 32 bytes of codes and one or two fp16 scales
  u32x4 w[2] = {};
  float s_lo = 0.0f, s_hi = 0.0f;
  if (live) {
    const u32x4* src = reinterpret_cast<const u32x4*>(codes + row * (k >> 1) + (col >> 1));
    w[0] = __builtin_nontemporal_load(src);
    w[1] = __builtin_nontemporal_load(src + 1);
    const uint16_t* srow = scales + row * (k / group);
    if (group == 32) {
      const uint32_t two = *reinterpret_cast<const uint32_t*>(srow + (col >> 5));
      s_lo = fp16_bits_to_f32(two & 0xFFFFu) * 0.0625f;
      s_hi = fp16_bits_to_f32(two >> 16) * 0.0625f;
    } else {
      s_lo = s_hi = fp16_bits_to_f32(srow[col >> 6]) * 0.0625f;
    }
  }

  float v[64];
  dequant64(v, w, s_lo, s_hi);
  fwht256_wave(v, lane);
  lowrank_acc_16x256(v, up, down, row0, n, blk * 256, rank, false, lane);

  // Stage the wave's 16 x 256 bf16 tile in LDS so that every global store
  // instruction writes two whole 512-byte row segments.
  u32x4* stage = reinterpret_cast<u32x4*>(&s_stage[wave][0][0]);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(v[8 * j + 2 * e], v[8 * j + 2 * e + 1]);
    stage[c * STAGE_ROW_U4 + 8 * g + j] = o;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int rr = 2 * j + (lane >> 5), piece = lane & 31;
    const u32x4 o = stage[rr * STAGE_ROW_U4 + piece];
    if (row0 + rr < n)
      *reinterpret_cast<u32x4*>(w_hat + (row0 + rr) * k + blk * 256 + 8 * piece) = o;
  }
}

hipError_t launch_reconstruct(const uint8_t* codes, const uint16_t* scales, const uint16_t* up,
                              const uint16_t* down, uint16_t* w_hat, int64_t n, int64_t k,
                              int group, int rank, hipStream_t stream) {
  const int64_t nblk = k >> 8;
  dim3 grid((unsigned)((n + 15) / 16), (unsigned)((nblk + 3) / 4));
  hipLaunchKernelGGL(k_reconstruct, grid, dim3(256), 0, stream, codes, scales, up, down, w_hat, n,
                     k, group, rank);
  return hipGetLastError();
}

}  // namespace sq
