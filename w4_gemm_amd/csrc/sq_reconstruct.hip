// Backward-side rebuild of the dense bf16 weight from the W4 payload
// (SquareQ README, "SquareQ v3 - W4": the format formula; the backward visit
// rebuilds bf16 from the same payload):
//
//   w_hat[n][k] = bf16_rne( sum_r up[n][r] down[k][r] + ((q * s) @ H)[n][k] )
//
// One wave owns one 256-column Hadamard block and a run of 16-row strips of
// it.  The block's rank-r slice of `down` (the MFMA A operand of the low-rank
// term) is loaded into registers once and reused for every strip, so the
// factor costs one 16*r-byte read per lane per run instead of per strip.
// Per strip every lane reads 32 bytes of codes (64 consecutive columns of
// one row; the next strip's codes are in flight while this one computes),
// dequantizes to fp32 with the 1/16 of H folded into the scale (exact: a
// power of two), runs the 256-point butterflies (six stages in registers,
// two across lanes), adds the low-rank term from bf16 MFMA (exact products,
// fp32 sums) and writes its row through an LDS transpose so that every store
// instruction covers two whole 512-byte row segments.  HBM-bound: reads
// 0.5 + 2/group bytes and writes 2 bytes per weight element.
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
constexpr int REC_WAVES = 4;

// Payload of one lane for one strip: 32 bytes of codes, two scales / 16.
struct StripIn {
  u32x4 w[2];
  uint32_t s2;   // fp16 bits: low half for columns 0..31 of the chunk, high for 32..63
};

__device__ __forceinline__ void load_strip(StripIn& in, const uint8_t* __restrict__ codes,
                                           const uint16_t* __restrict__ scales, int64_t row,
                                           bool live, int64_t col, int64_t k, int group) {
  if (live) {
    const u32x4* src = reinterpret_cast<const u32x4*>(codes + row * (k >> 1) + (col >> 1));
    in.w[0] = __builtin_nontemporal_load(src);
    in.w[1] = __builtin_nontemporal_load(src + 1);
    const uint16_t* srow = scales + row * (k / group);
    if (group == 32) {
      in.s2 = *reinterpret_cast<const uint32_t*>(srow + (col >> 5));
    } else {
      const uint32_t one = srow[col >> 6];
      in.s2 = one | (one << 16);
    }
  } else {
    in.w[0] = in.w[1] = (u32x4){0u, 0u, 0u, 0u};
    in.s2 = 0u;
  }
}

template <int RANK>
__global__ void __launch_bounds__(64 * REC_WAVES) k_reconstruct(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ up, const uint16_t* __restrict__ down,
    uint16_t* __restrict__ w_hat, int64_t n, int64_t k, int group, int strips) {
  __shared__ __attribute__((aligned(16))) uint32_t s_stage[REC_WAVES][16][STAGE_ROW_U4 * 4];
  constexpr int RC = RANK / 32;   // rank-32 chunks
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t nblk = k >> 8;
  const int64_t wid = (int64_t)blockIdx.x * REC_WAVES + wave;
  const int64_t blk = wid % nblk;
  const int64_t run_row0 = (wid / nblk) * 16 * (int64_t)strips;
  if (run_row0 >= n) return;
  const int c = lane & 15, g = lane >> 4;
  const int64_t col = blk * 256 + 64 * g;

  // A operand of the low-rank MFMA (row rho = c, k = r): the down row of
  // column 64*(c/4) + 4t + c%4 of the block, so that the result lands in the
  // butterfly layout (lane (c, g) holds row c, columns 64g .. 64g+63).
  bf16x8 dfrag[RC > 0 ? RC : 1][16];
#pragma unroll
  for (int q = 0; q < RC; ++q)
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int64_t dcol = blk * 256 + 64 * (c >> 2) + 4 * t + (c & 3);
      dfrag[q][t] = *reinterpret_cast<const bf16x8*>(down + dcol * RANK + 32 * q + 8 * g);
    }

  const int nstrip = (int)min((int64_t)strips, (n - run_row0 + 15) / 16);
  StripIn cur;
  load_strip(cur, codes, scales, run_row0 + c, run_row0 + c < n, col, k, group);
  u32x4* stage = reinterpret_cast<u32x4*>(&s_stage[wave][0][0]);

  for (int s = 0; s < nstrip; ++s) {
    const int64_t row0 = run_row0 + 16 * s;
    const int64_t row = row0 + c;
    const bool live = row < n;
    // up fragment (B operand, k = r, col = output row c) and the next strip's codes
    bf16x8 ufrag[RC > 0 ? RC : 1];
#pragma unroll
    for (int q = 0; q < RC; ++q)
      ufrag[q] = live ? *reinterpret_cast<const bf16x8*>(up + row * RANK + 32 * q + 8 * g)
                      : (bf16x8){};
    StripIn nxt;
    const bool more = s + 1 < nstrip;
    if (more) load_strip(nxt, codes, scales, row + 16, row + 16 < n, col, k, group);

    float v[64];
    dequant64(v, cur.w, fp16_bits_to_f32(cur.s2 & 0xFFFFu) * 0.0625f,
              fp16_bits_to_f32(cur.s2 >> 16) * 0.0625f);
    fwht256_wave(v, lane);
#pragma unroll
    for (int q = 0; q < RC; ++q)
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        f32x4 acc = {v[4 * t], v[4 * t + 1], v[4 * t + 2], v[4 * t + 3]};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dfrag[q][t], ufrag[q], acc, 0, 0, 0);
        v[4 * t] = acc[0];
        v[4 * t + 1] = acc[1];
        v[4 * t + 2] = acc[2];
        v[4 * t + 3] = acc[3];
      }

    // Transpose the 16 x 256 bf16 tile through LDS: lane (c, g) writes its
    // 128 bytes, then each store instruction takes two whole rows.  The
    // wave's reads of the previous strip finished before its writes here
    // (the stores consumed them), so only compiler ordering is needed.
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(v[8 * j + 2 * e], v[8 * j + 2 * e + 1]);
      stage[c * STAGE_ROW_U4 + 8 * g + j] = o;
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int rr = 2 * j + (lane >> 5), piece = lane & 31;
      const u32x4 o = stage[rr * STAGE_ROW_U4 + piece];
      if (row0 + rr < n)
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(w_hat + (row0 + rr) * k +
                                                                 blk * 256 + 8 * piece));
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_wave_barrier();
    if (more) cur = nxt;
  }
}

// Strips per wave: enough waves to cover the chip a few times over, as few
// factor reloads as that allows.
int rec_strips_per_wave(int64_t n, int64_t k) {
  const int64_t strips = (n + 15) / 16, nblk = k >> 8;
  int s = 8;
  while (s > 1 && ((strips + s - 1) / s) * nblk < 4 * 256 * 4) s >>= 1;
  return s;
}

hipError_t launch_reconstruct(const uint8_t* codes, const uint16_t* scales, const uint16_t* up,
                              const uint16_t* down, uint16_t* w_hat, int64_t n, int64_t k,
                              int group, int rank, hipStream_t stream) {
  const int64_t nblk = k >> 8;
  const int s = rec_strips_per_wave(n, k);
  const int64_t runs = ((n + 15) / 16 + s - 1) / s;
  const int64_t waves = runs * nblk;
  dim3 grid((unsigned)((waves + REC_WAVES - 1) / REC_WAVES));
  if (rank == 0)
    hipLaunchKernelGGL(k_reconstruct<0>, grid, dim3(64 * REC_WAVES), 0, stream, codes, scales, up,
                       down, w_hat, n, k, group, s);
  else if (rank == 32)
    hipLaunchKernelGGL(k_reconstruct<32>, grid, dim3(64 * REC_WAVES), 0, stream, codes, scales, up,
                       down, w_hat, n, k, group, s);
  else
    hipLaunchKernelGGL(k_reconstruct<64>, grid, dim3(64 * REC_WAVES), 0, stream, codes, scales, up,
                       down, w_hat, n, k, group, s);
  return hipGetLastError();
}

}  // namespace sq
