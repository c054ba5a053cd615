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
// two across lanes with the lane-swap instructions), adds the low-rank term from bf16 MFMA (exact products,
// fp32 sums) and writes its row through an LDS transpose so that every store
// instruction covers two whole 512-byte row segments.  HBM-bound: reads
// 0.5 + 2/group bytes and writes 2 bytes per weight element.
#include "sq_device.hpp"
#include "sq_kernels.h"

namespace sq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Dequantize and rotate the lane's 64 codes (32 bytes; element e = column
// 64g + e of the block) over the six in-lane column bits, giving
// v[e] = (1/16) * sum_e' S64[e][e'] * q[e'] * s(e') in fp32 with S64 the
// Sylvester matrix and s(e') = s_lo for e' < 32, s_hi otherwise.
//
// The codes are unpacked two per register straight into fp16: nibble
// positions p and p+4 of word j (elements 8j+p and 8j+p+4) land in the two
// halves as fp16(1024 + (q ^ 8)) = 1024 + q + 8, and subtracting 1032 gives
// q exactly.  Five butterfly stages then run on packed fp16 (two elements per
// instruction): every value stays an integer of magnitude at most 16*8, so
// fp16 holds it exactly.  The last stage (column bit 5) joins the two scale
// groups and is done as fp32 y = s_lo * a +- (s_hi * b), with the fp16
// operands converted inside the mixed-precision FMA; s * b is exact in fp32
// (11-bit times 8-bit significands) and each output is rounded once.
__device__ __forceinline__ void dequant_rotate64(float (&v)[64], const u32x4 (&w)[2], float s_lo,
                                                 float s_hi) {
  half2_t h[32];   // h[4j + p] = (element 8j+p, element 8j+p+4)
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t word = w[j >> 2][j & 3];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t bits = ((word >> (4 * p)) & 0x000F000Fu) ^ 0x64086408u;
      h[4 * j + p] = __builtin_bit_cast(half2_t, bits) - (half2_t){(_Float16)1032.0f, (_Float16)1032.0f};
    }
  }
  // column bits 0, 1 (p) and 3, 4 (j bits 0, 1): pairs of registers
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) {
    if (m == 8 * 2) continue;   // j bit 2 = column bit 5: done in fp32 below
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      if (r & m) continue;
      const half2_t a = h[r], b = h[r + m];
      h[r] = a + b;
      h[r + m] = a - b;
    }
  }
  // column bit 2: the two halves of one register
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    const half2_t a = h[r];
    const half2_t sw = __builtin_shufflevector(a, a, 1, 0);
    h[r] = a * (half2_t){(_Float16)1.0f, (_Float16)-1.0f} + sw;
  }
  // column bit 5 (j bit 2) with the scales, into fp32
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int j = r >> 2, p = r & 3;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const float a = (float)h[r][half], b = (float)h[r + 16][half];
      const float t = __builtin_fmaf(b, s_hi, 0.0f);
      const int e = 8 * j + p + 4 * half;
      v[e] = __builtin_fmaf(a, s_lo, t);
      v[e + 32] = __builtin_fmaf(a, s_lo, -t);
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

// `cbase` / `sbase` point at the strip's first row and the block's first
// column (wave-uniform); the lane offsets are 32-bit.
__device__ __forceinline__ void load_strip(StripIn& in, const uint8_t* cbase,
                                           const uint16_t* sbase, bool live, uint32_t coff,
                                           uint32_t soff, int group) {
  if (live) {
    const u32x4* src = reinterpret_cast<const u32x4*>(cbase + coff);
    in.w[0] = __builtin_nontemporal_load(src);
    in.w[1] = __builtin_nontemporal_load(src + 1);
    if (group == 32) {
      in.s2 = *reinterpret_cast<const uint32_t*>(sbase + soff);
    } else {
      const uint32_t one = sbase[soff];
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
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nblk = k >> 8;
  const int64_t wid = (int64_t)blockIdx.x * REC_WAVES + wave;
  const int64_t blk = wid % nblk;
  const int64_t run_row0 = (wid / nblk) * 16 * (int64_t)strips;
  if (run_row0 >= n) return;
  const int c = lane & 15, g = lane >> 4;
  const int64_t spr = k / group;   // scales per row
  // lane offsets within a strip (elements of each array)
  const uint32_t coff = (uint32_t)(c * (k >> 1)) + 32u * g;
  const uint32_t soff = (uint32_t)(c * spr) + (uint32_t)(64 * g / group);
  const uint32_t uoff = (uint32_t)(c * RANK + 8 * g);
  uint32_t stoff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    stoff[j] = (uint32_t)((2 * j + (lane >> 5)) * k) + 8u * (lane & 31);

  // A operand of the low-rank MFMA (row rho = c, k = r) for accumulator
  // registers 4t .. 4t+3: the down row of the column that register 4t + c%4
  // of lane group c/4 holds after the butterflies, so the product lands on
  // the right columns (MFMA output row rho goes to lane group rho/4,
  // register 4t + rho%4).
  bf16x8 dfrag[RC > 0 ? RC : 1][16];
#pragma unroll
  for (int q = 0; q < RC; ++q)
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int64_t dcol = blk * 256 + swap_col(c >> 2, 4 * t + (c & 3));
      dfrag[q][t] = *reinterpret_cast<const bf16x8*>(down + dcol * RANK + 32 * q + 8 * g);
    }

  const int nstrip = (int)min((int64_t)strips, (n - run_row0 + 15) / 16);
  StripIn cur;
  load_strip(cur, codes + run_row0 * (k >> 1) + blk * 128, scales + run_row0 * spr + blk * 256 / group,
             run_row0 + c < n, coff, soff, group);
  u32x4* stage = reinterpret_cast<u32x4*>(&s_stage[wave][0][0]);

  for (int s = 0; s < nstrip; ++s) {
    const int64_t row0 = run_row0 + 16 * s;
    const int64_t row = row0 + c;
    const bool live = row < n;
    // up fragment (B operand, k = r, col = output row c) and the next strip's codes
    bf16x8 ufrag[RC > 0 ? RC : 1];
#pragma unroll
    for (int q = 0; q < RC; ++q)
      ufrag[q] = live ? *reinterpret_cast<const bf16x8*>(up + row0 * RANK + uoff + 32 * q)
                      : (bf16x8){};
    StripIn nxt;
    const bool more = s + 1 < nstrip;
    if (more)
      load_strip(nxt, codes + (row0 + 16) * (k >> 1) + blk * 128,
                 scales + (row0 + 16) * spr + blk * 256 / group, row + 16 < n, coff, soff, group);

    float v[64];
    dequant_rotate64(v, cur.w, fp16_bits_to_f32(cur.s2 & 0xFFFFu) * 0.0625f,
                     fp16_bits_to_f32(cur.s2 >> 16) * 0.0625f);
    fwht_cross64_swap(v);
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
    // 128 bytes (eight runs of 8 columns, placed by swap_col), then each
    // store instruction takes two whole rows.  The wave's reads of the
    // previous strip finished before its writes here (the stores consumed
    // them), so only compiler ordering is needed.
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(v[8 * j + 2 * e], v[8 * j + 2 * e + 1]);
      stage[c * STAGE_ROW_U4 + (swap_col(g, 8 * j) >> 3)] = o;
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int rr = 2 * j + (lane >> 5), piece = lane & 31;
      const u32x4 o = stage[rr * STAGE_ROW_U4 + piece];
      if (row0 + rr < n)
        __builtin_nontemporal_store(
            o, reinterpret_cast<u32x4*>(w_hat + row0 * k + blk * 256 + stoff[j]));
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
