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
//
// The same kernel rebuilds the int8-residual mode (SquareQ README, "v3.1 -
// int8-residual mode"; GROUP = 0 selects it): 64 bytes of codes per lane
// and strip, one scale per row, the butterflies on exact integers in fp32
// and the scale applied once after the last stage.  GROUP = 1 selects the
// MXFP4 payload (E2M1 nibbles with one E8M0 byte per 32 values, whose
// per-row layout indexes like group-64 fp16 scales: one 16-bit word per 64
// values holds the two exponents).
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
//
// MX = true reads E2M1 nibbles instead: a byte-table permute turns the two
// magnitude fields into 2|v| (an integer in {0, 1, 2, 3, 4, 6, 8, 12}) under
// the fp16 exponent of 1024, one packed subtraction leaves the integer, and
// the nibbles' sign bits move into the fp16 sign bits; the scales then carry
// the factor 1/2.
template <bool MX>
__device__ __forceinline__ void dequant_rotate64(float (&v)[64], const u32x4 (&w)[2], float s_lo,
                                                 float s_hi) {
  half2_t h[32];   // h[4j + p] = (element 8j+p, element 8j+p+4)
  constexpr uint32_t TLO = 0x03020100u, THI = 0x0C080604u;   // 2|E2M1| by magnitude
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t word = w[j >> 2][j & 3];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if constexpr (MX) {
        const uint32_t sh = word >> (4 * p);
        // selector bytes 1 and 3 are zero: they pick the table's 0
        const uint32_t mags = __builtin_amdgcn_perm(THI, TLO, sh & 0x00070007u);
        const half2_t a = __builtin_bit_cast(half2_t, mags | 0x64006400u) -
                          (half2_t){(_Float16)1024.0f, (_Float16)1024.0f};
        h[4 * j + p] = __builtin_bit_cast(
            half2_t, __builtin_bit_cast(uint32_t, a) ^ ((sh << 12) & 0x80008000u));
      } else {
        const uint32_t bits = ((word >> (4 * p)) & 0x000F000Fu) ^ 0x64086408u;
        h[4 * j + p] = __builtin_bit_cast(half2_t, bits) - (half2_t){(_Float16)1032.0f, (_Float16)1032.0f};
      }
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

// int8 codes: the lane's 64 bytes (element e = column 64g + e of the block)
// rotated over the six in-lane column bits, unscaled:
// v[e] = sum_e' S64[e][e'] q[e'].  Each byte converts to fp32 as q + 128 (the
// sign bit flipped) in one instruction; the butterflies run on these exact
// integers (every partial sum is below 2^14 in magnitude), and because S64
// sends the constant 128 to column 0 alone (as 64 * 128), one subtraction
// there removes the offset.
__device__ __forceinline__ void dequant_rotate64_w8(float (&v)[64], const u32x4 (&w)[4]) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t word = w[j >> 2][j & 3] ^ 0x80808080u;
#pragma unroll
    for (int b = 0; b < 4; ++b) v[4 * j + b] = (float)((word >> (8 * b)) & 0xFFu);
  }
  fwht_inreg64(v);
  v[0] -= 8192.0f;
}

// LDS staging rows: 256 bf16 = 32 x 16 bytes, padded by one 16-byte slot so
// that the 16 rows written by one instruction start in different banks.
constexpr int STAGE_ROW_U4 = 33;
constexpr int REC_WAVES = 4;

// Payload of one lane for one strip: 32 bytes of int4 codes and two scales,
// or 64 bytes of int8 codes and the row scale.
template <int GROUP>
struct StripIn {
  u32x4 w[GROUP == 0 ? 4 : 2];
  uint32_t s2;   // fp16 bits: low half for columns 0..31 of the chunk, high for 32..63
};

// `cbase` / `sbase` point at the lane's row and the block's first column.
// The loads are unconditional (callers clamp rows past the end to the last
// row and never store those results): loads under divergent branches make
// the compiler wait for every outstanding memory operation, stores included,
// before the next strip.
template <int GROUP>
__device__ __forceinline__ void load_strip(StripIn<GROUP>& in, const uint8_t* cbase,
                                           const uint16_t* sbase, int g) {
  // plain loads: on gfx950 the non-temporal load path streams these
  // 32-byte row pieces markedly slower (63.5 vs 49.5 us at 16384x6144)
  if constexpr (GROUP == 0) {
    const u32x4* src = reinterpret_cast<const u32x4*>(cbase + 64 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) in.w[i] = src[i];
    in.s2 = sbase[0];
    return;
  }
  const u32x4* src = reinterpret_cast<const u32x4*>(cbase + 32 * g);
  in.w[0] = src[0];
  in.w[1] = src[1];
  if (GROUP == 32) {
    in.s2 = *reinterpret_cast<const uint32_t*>(sbase + 2 * g);
  } else if (GROUP == 64) {
    // one scale covers the lane's whole 64-value chunk: both halves
    const uint32_t sv = sbase[g];
    in.s2 = sv | (sv << 16);
  } else {
    in.s2 = sbase[g];   // MX: one 16-bit word holds the chunk's two exponents
  }
}

// Stores the staged 16 x 256 bf16 tile of strip row0: every instruction
// writes two whole 512-byte row segments.  The buffer descriptor ends at the
// last row of the weight, so rows of a ragged last strip are dropped by the
// hardware range check instead of a branch (a branch around the stores
// would make the compiler's wait counting assume the worst).
__device__ __forceinline__ void store_tile(const u32x4* stage, uint16_t* w_hat, int64_t row0,
                                           int64_t n, int64_t k, uint32_t stoff, int lane) {
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(w_hat + row0 * k), (short)0, (int)(min((int64_t)16, n - row0) * k * 2), 0x00020000);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const u32x4 o = stage[(2 * j + (lane >> 5)) * STAGE_ROW_U4 + (lane & 31)];
    __builtin_amdgcn_raw_buffer_store_b128(o, rsrc, stoff + (uint32_t)(4 * j) * (uint32_t)k, 0,
                                           SQ_CPOL_NT);
  }
}

template <int RANK, int GROUP>
__global__ void __launch_bounds__(64 * REC_WAVES) k_reconstruct(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ up, const uint16_t* __restrict__ down,
    uint16_t* __restrict__ w_hat, int64_t n, int64_t k, int strips) {
  constexpr bool W8 = GROUP == 0;
  constexpr bool MX = GROUP == 1;
  constexpr int SG = MX ? 64 : (GROUP > 0 ? GROUP : 1);   // values per 16-bit scale word
  constexpr int RC = (RANK + 31) / 32;   // rank-32 chunks (rank 16: the upper half reads zero)
  // A operands of the low-rank MFMA for the block, in fragment order
  // [chunk][t][lane] so that every read is 64 consecutive 16-byte slots.
  __shared__ u32x4 s_down[RC > 0 ? RC * 16 * 64 : 1];
  // Per-wave output staging: 16 rows x 256 columns of bf16 (32 slots of
  // 16 bytes) plus one pad slot per row.
  __shared__ u32x4 s_stage[REC_WAVES][16 * STAGE_ROW_U4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nblk = k >> 8;
  const int64_t nstr = (n + 15) / 16;
  // Workgroup ids congruent mod 8 run on the same XCD (L2).  Give each XCD a
  // contiguous run of (strip run, block) pairs, so that the neighbouring
  // blocks of a row, whose scales share 128-byte lines, are read through one
  // L2 instead of up to eight.
  const int64_t nwg = (int64_t)gridDim.x, lin = blockIdx.x;
  const int64_t xcd = lin & 7, per = nwg >> 3, rem = nwg & 7;
  const int64_t t = xcd * per + min(xcd, rem) + (lin >> 3);
  const int64_t blk = t % nblk;
  const int64_t first = (t / nblk) * REC_WAVES * strips + wave;
  const int c = lane & 15, g = lane >> 4;

  // Column of MFMA output row rho in accumulator register 4t + rho%4: the
  // butterfly result that lane group rho/4 holds there (swap_col), so the
  // product lands on the right columns.
#pragma unroll
  for (int m = 0; m < RC * 4; ++m) {
    const int f = tid + 64 * REC_WAVES * m;
    const int q = f >> 10, t = (f >> 6) & 15, l = f & 63;
    const int64_t dcol = blk * 256 + swap_col((l & 15) >> 2, 4 * t + (l & 3));
    s_down[f] = 32 * q + 8 * (l >> 4) < RANK
                    ? *reinterpret_cast<const u32x4*>(down + dcol * RANK + 32 * q + 8 * (l >> 4))
                    : (u32x4){0u, 0u, 0u, 0u};
  }
  __syncthreads();
  if (first >= nstr) return;

  const int64_t spr = W8 ? 1 : k / SG;   // scale words per row
  const int64_t cpr = W8 ? k : k >> 1;                        // code bytes per row
  // byte offset of the lane's 16-byte store piece from the strip's first row
  const uint32_t stoff = 2u * ((uint32_t)((lane >> 5) * k) + (uint32_t)(blk * 256) + 8u * (lane & 31));
  const uint8_t* cblk = codes + blk * (W8 ? 256 : 128);
  const uint16_t* sblk = scales + (W8 ? 0 : blk * (256 / SG));
  u32x4* stage = &s_stage[wave][0];
  // the lane's row of strip st, clamped to the last row
  auto lrow = [&](int64_t st) { return min(st * 16 + c, n - 1); };

  // This wave's strips: first, first + REC_WAVES, ... below nstr.
  //
  // Loads and stores share one in-order completion counter, and the
  // compiler treats them as completing out of order, so a wait for a
  // prefetched load also waits for every store issued before it.  Each
  // iteration therefore starts with the wait, then issues the previous
  // strip's stores (from LDS) and the next strip's loads back to back, and
  // only then computes: the next wait is a whole strip of compute later.
  const int cnt = (int)min((int64_t)strips, (nstr - first + REC_WAVES - 1) / REC_WAVES);
  StripIn<GROUP> cur;
  bf16x8 ufrag[RC > 0 ? RC : 1];
  auto load_up = [&](bf16x8 (&uf)[RC > 0 ? RC : 1], int64_t row) {
#pragma unroll
    for (int q = 0; q < RC; ++q)
      uf[q] = 32 * q + 8 * g < RANK
                  ? *reinterpret_cast<const bf16x8*>(up + row * RANK + 32 * q + 8 * g)
                  : (bf16x8){};
  };
  load_strip<GROUP>(cur, cblk + lrow(first) * cpr, sblk + lrow(first) * spr, g);
  load_up(ufrag, lrow(first));

  for (int i = 0; i < cnt; ++i) {
    const int64_t st = first + (int64_t)REC_WAVES * i;
    const int64_t row0 = st * 16;
    __builtin_amdgcn_s_waitcnt(SQ_WAIT_VM0);
    __builtin_amdgcn_sched_barrier(0);
    // consume this strip's payload, then reuse its registers
    const StripIn<GROUP> in = cur;
    bf16x8 uf[RC > 0 ? RC : 1];
#pragma unroll
    for (int q = 0; q < RC; ++q) uf[q] = ufrag[q];
    if (i > 0) store_tile(stage, w_hat, row0 - 16 * REC_WAVES, n, k, stoff, lane);
    if (i + 1 < cnt) {
      const int64_t nst = st + REC_WAVES;
      load_strip<GROUP>(cur, cblk + lrow(nst) * cpr, sblk + lrow(nst) * spr, g);
      load_up(ufrag, lrow(nst));
    }
    __builtin_amdgcn_sched_barrier(0);

    float v[64];
    if constexpr (W8) {
      dequant_rotate64_w8(v, in.w);
      fwht_cross64_swap(v);   // exact: integers of magnitude at most 2^15
      const float s16 = fp16_bits_to_f32(in.s2) * 0.0625f;
#pragma unroll
      for (int e = 0; e < 64; ++e) v[e] *= s16;
    } else if constexpr (MX) {
      // 2^(e-127) x 1/2 x 1/16 = 2^(e-132), flushed to 0 below the fp32 normals
      dequant_rotate64<true>(v, in.w, __uint_as_float((uint32_t)max((int)(in.s2 & 0xFFu) - 5, 0) << 23),
                             __uint_as_float((uint32_t)max((int)((in.s2 >> 8) & 0xFFu) - 5, 0) << 23));
      fwht_cross64_swap(v);
    } else {
      dequant_rotate64<false>(v, in.w, fp16_bits_to_f32(in.s2 & 0xFFFFu) * 0.0625f,
                              fp16_bits_to_f32(in.s2 >> 16) * 0.0625f);
      fwht_cross64_swap(v);
    }
#pragma unroll
    for (int q = 0; q < RC; ++q)
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, s_down[(q * 16 + t) * 64 + lane]);
        f32x4 acc = {v[4 * t], v[4 * t + 1], v[4 * t + 2], v[4 * t + 3]};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, uf[q], acc, 0, 0, 0);
        v[4 * t] = acc[0];
        v[4 * t + 1] = acc[1];
        v[4 * t + 2] = acc[2];
        v[4 * t + 3] = acc[3];
      }

    // Stage the tile in LDS: lane (c, g) writes its eight runs of 8 columns
    // (placed by swap_col).  The next iteration reads it back for the
    // stores; LDS accesses of one wave complete in order.
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(v[8 * j + 2 * e], v[8 * j + 2 * e + 1]);
      stage[c * STAGE_ROW_U4 + (swap_col(g, 8 * j) >> 3)] = o;
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_wave_barrier();
  }
  store_tile(stage, w_hat, (first + (int64_t)REC_WAVES * (cnt - 1)) * 16, n, k, stoff, lane);
}

// Strips per wave: as many as still leave a few workgroups per CU slot, so
// that the block's factor is loaded as few times as that allows.
static int rec_strips_per_wave(int64_t n, int64_t k) {
  const int64_t nstr = (n + 15) / 16, nblk = k >> 8;
  int s = 8;
  while (s > 1 && ((nstr + REC_WAVES * s - 1) / (REC_WAVES * s)) * nblk < 3 * 4 * 256) s >>= 1;
  return s;
}

template <int RANK>
static void launch_rank(dim3 grid, int group, hipStream_t stream, const uint8_t* codes,
                        const uint16_t* scales, const uint16_t* up, const uint16_t* down,
                        uint16_t* w_hat, int64_t n, int64_t k, int s) {
  if (group == 0)
    hipLaunchKernelGGL((k_reconstruct<RANK, 0>), grid, dim3(64 * REC_WAVES), 0, stream, codes,
                       scales, up, down, w_hat, n, k, s);
  else if (group == 1)
    hipLaunchKernelGGL((k_reconstruct<RANK, 1>), grid, dim3(64 * REC_WAVES), 0, stream, codes,
                       scales, up, down, w_hat, n, k, s);
  else if (group == 32)
    hipLaunchKernelGGL((k_reconstruct<RANK, 32>), grid, dim3(64 * REC_WAVES), 0, stream, codes,
                       scales, up, down, w_hat, n, k, s);
  else
    hipLaunchKernelGGL((k_reconstruct<RANK, 64>), grid, dim3(64 * REC_WAVES), 0, stream, codes,
                       scales, up, down, w_hat, n, k, s);
}

hipError_t launch_reconstruct(const uint8_t* codes, const uint16_t* scales, const uint16_t* up,
                              const uint16_t* down, uint16_t* w_hat, int64_t n, int64_t k,
                              int group, int rank, hipStream_t stream) {
  const int64_t nblk = k >> 8, nstr = (n + 15) / 16;
  const int s = rec_strips_per_wave(n, k);
  const int64_t runs = (nstr + REC_WAVES * s - 1) / (REC_WAVES * s);
  dim3 grid((unsigned)(runs * nblk));
  if (rank == 0)
    launch_rank<0>(grid, group, stream, codes, scales, up, down, w_hat, n, k, s);
  else if (rank == 16)
    launch_rank<16>(grid, group, stream, codes, scales, up, down, w_hat, n, k, s);
  else if (rank == 32)
    launch_rank<32>(grid, group, stream, codes, scales, up, down, w_hat, n, k, s);
  else
    launch_rank<64>(grid, group, stream, codes, scales, up, down, w_hat, n, k, s);
  return hipGetLastError();
}

}  // namespace sq
