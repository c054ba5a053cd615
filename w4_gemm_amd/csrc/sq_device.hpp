// Device helpers shared by the libsq kernels (gfx950, wave64).
//
// Lane layout used by the reconstruct, quantize and activation-rotation
// kernels: one wave covers 16 rows x one 256-wide Hadamard block.  Lane l owns
// row (l % 16) and the 64 consecutive columns 64*(l/16) .. 64*(l/16)+63 of the
// block, held in 64 registers.  The Hadamard butterflies over the low six
// column bits are therefore in-register; the two high bits live in lane bits 4
// and 5 and are exchanged across lanes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Cache-policy operand of the gfx950 buffer intrinsics: non-temporal
// (streaming) access.
constexpr int SQ_CPOL_NT = 2;

// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0]+[15:14], expcnt [6:4],
// lgkmcnt [11:8]): wait for all vector memory operations, others untouched.
constexpr int SQ_WAIT_VM0 = 0x0F70;
// wait until at most n vector memory operations are outstanding (n < 64)
constexpr int sq_wait_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
// wait for all LDS (and scalar memory) operations, the rest untouched
constexpr int SQ_WAIT_LGKM0 = 0xC07F;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> one word of two bf16 (lo in the low half), round to nearest
// even, in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float fp16_bits_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// Smallest e with a <= 2^e for the bf16 magnitude bits `mx` (0 for a zero
// row), floored at -100.
__device__ __forceinline__ int row_exponent(uint32_t mx) {
  const float a = bf16_to_f32(mx);
  int e = 0;
  if (a > 0.0f) {
    int ex;
    const float mant = frexpf(a, &ex);   // a = mant * 2^ex, mant in [0.5, 1)
    e = (mant == 0.5f) ? ex - 1 : ex;
  }
  return max(e, -100);
}

// ---------------------------------------------------------------------------
// 8 packed int4 codes -> fp16(q*s) in the K order [0,4,1,5,2,6,3,7].  Code k
// of the 8 is nibble k of the word (two's complement), so nibble pair p sits
// at bits 4p and 16 + 4p.  Pairs 0 and 2 are selected at bits 0..3 with the
// sign bit flipped (q + 8) under the fp16 exponent of 1024, giving 1032 + q;
// pairs 1 and 3 are selected at bits 4..7, giving 1024 + 16 (q + 8), which
// one exact fma maps back to q.  Each product q*s is rounded once.  One
// shift, four 3-input bit ops and eight packed fp16 ops per word.
// ---------------------------------------------------------------------------
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ half8 dequant8_f16(uint32_t w, _Float16 s) {
  const half2_t s2 = {s, s};
  const half2_t b1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t m72 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t w8 = w >> 8;
  const half2_t h0 = __builtin_bit_cast(half2_t, (w & 0x000F000Fu) ^ 0x64086408u);
  const half2_t h1 = __builtin_bit_cast(half2_t, (w & 0x00F000F0u) ^ 0x64806480u);
  const half2_t h2 = __builtin_bit_cast(half2_t, (w8 & 0x000F000Fu) ^ 0x64086408u);
  const half2_t h3 = __builtin_bit_cast(half2_t, (w8 & 0x00F000F0u) ^ 0x64806480u);
  const half2_t q0 = h0 - b1032, q2 = h2 - b1032;
  const half2_t q1 = __builtin_elementwise_fma(h1, sixteenth, m72);
  const half2_t q3 = __builtin_elementwise_fma(h3, sixteenth, m72);
  return __builtin_bit_cast(
      half8, (u32x4){__builtin_bit_cast(uint32_t, q0 * s2), __builtin_bit_cast(uint32_t, q1 * s2),
                     __builtin_bit_cast(uint32_t, q2 * s2), __builtin_bit_cast(uint32_t, q3 * s2)});
}

// 8 int8 codes (w0 holds codes 0..3, w1 codes 4..7, one two's-complement
// byte each) -> fp16 q in the same K order [0,4,1,5,2,6,3,7].  Pair p takes
// byte p of each word into the low byte of a half (one byte permute), the
// xor flips the sign bits and sets the fp16 exponent of 1024 (1024 + q + 128)
// and one packed subtraction leaves q exactly.  Three ops per two codes.
__device__ __forceinline__ half8 dequant8_i8(uint32_t w0, uint32_t w1) {
  const half2_t b1152 = {(_Float16)1152.0f, (_Float16)1152.0f};
  u32x4 o;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    // byte selectors: p and 4 + p pick byte p of w0 and of w1, 0x0C a zero byte
    const uint32_t t = __builtin_amdgcn_perm(w1, w0, 0x0C000C00u | (uint32_t)p | ((4u + p) << 16));
    o[p] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, t ^ 0x64806480u) - b1152);
  }
  return __builtin_bit_cast(half8, o);
}

// ---------------------------------------------------------------------------
// Tiled contractions (forward and input gradient)
// ---------------------------------------------------------------------------
// Map the linear workgroup id to a tile.  Ids congruent mod 8 are dispatched
// to the same XCD, so each XCD gets one contiguous run of tile numbers; within
// the run the numbers walk XCD_GROUP_M tile rows down before stepping one tile
// column across, so the ~32 workgroups resident on an XCD at a time cover a
// 4 x 8 block of tiles and share both operands in its L2 (4 A strips + 8 B
// strips instead of 1 + 32).
constexpr int64_t XCD_GROUP_M = 4;
__device__ __forceinline__ void xcd_tile(int64_t lin, int64_t tiles, int64_t nt, int64_t& tm,
                                         int64_t& tn) {
  const int64_t xcd = lin & 7, idx = lin >> 3;
  const int64_t per = tiles >> 3, rem = tiles & 7;
  const int64_t t = xcd * per + min(xcd, rem) + idx;
  const int64_t mt = tiles / nt;
  const int64_t grp = t / (XCD_GROUP_M * nt), first = grp * XCD_GROUP_M;
  const int64_t gsz = min(XCD_GROUP_M, mt - first);
  const int64_t w = t - grp * XCD_GROUP_M * nt;
  tm = first + w % gsz;
  tn = w / gsz;
}

// Slot of 16-byte chunk c in row r is c ^ a_swz(r): the 16 rows read by one
// fragment load land in distinct bank groups whether the LDS has 32 or 64 banks.
// Maximum over `slices` partial row maxima part[q * stride] (q in order), with
// eight loads in flight at a time: a loop of single loads would wait out one
// memory round trip per slice.
__device__ __forceinline__ uint32_t slice_max(const uint32_t* __restrict__ part, int64_t stride,
                                              int slices) {
  uint32_t mx = 0;
  int q = 0;
  for (; q + 8 <= slices; q += 8) {
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(q + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) mx = max(mx, v[u]);
  }
  for (; q < slices; ++q) mx = max(mx, part[q * stride]);
  return mx;
}

// Sum in slice order of `slices` fp32 partials part[q * stride], eight loads
// in flight at a time.
__device__ __forceinline__ float slice_sum(const float* __restrict__ part, int64_t stride,
                                           int slices) {
  float t = 0.0f;
  int q = 0;
  for (; q + 8 <= slices; q += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(q + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) t += v[u];
  }
  for (; q < slices; ++q) t += part[q * stride];
  return t;
}

__device__ __forceinline__ int a_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// ---------------------------------------------------------------------------
// Hadamard-256 butterflies in the 16-rows x 256-columns wave layout.
// Unnormalized: after both halves every lane holds S @ v for its block slice,
// S the Sylvester matrix (entries +-1); the caller applies the 1/16.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void fwht_inreg64(float (&v)[64]) {
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if ((i & h) == 0) {
        float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

// Column bits 6 and 7 (lane bits 4 and 5).  For a pair (a in the lane with the
// bit clear, b in its partner) the lane with the bit clear needs a+b and the
// other a-b; both are partner + sign*mine with sign = +1 / -1.
__device__ __forceinline__ void fwht_cross64(float (&v)[64], int lane) {
  const float s16 = (lane & 16) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    // bitmask swizzle: and 0x1f, xor 0x10 -> partner lane ^ 16 (within 32)
    float p = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v[i]), 0x401F));
    v[i] = __builtin_fmaf(s16, v[i], p);
  }
  const float s32 = (lane & 32) ? -1.0f : 1.0f;
  const int addr = (lane ^ 32) << 2;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    float p = __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(v[i])));
    v[i] = __builtin_fmaf(s32, v[i], p);
  }
}

// The same two stages with the gfx950 lane-swap instructions, which run on
// the vector ALU instead of the LDS crossbar.  permlane16_swap(x, y)
// exchanges the odd 16-lane rows of x with the even rows of y, so after it the
// lanes of an even row hold (x, partner's x) and those of an odd row
// (partner's y, y): one add and one subtract then finish the butterfly of
// either element.  permlane32_swap does the same for the two 32-lane halves.
// The result is not in the wave layout above: afterwards lane l (g = l/16)
// holds, in register 32a + 16b + r (a, b in {0,1}, r < 16), block column
//   swap_col(g, 32a + 16b + r) = 128b + 64a + 32(g & 1) + 16(g >> 1) + r,
// that is four runs of 16 consecutive columns.
__device__ __forceinline__ int swap_col(int g, int reg) {
  return 128 * ((reg >> 4) & 1) + 64 * (reg >> 5) + 32 * (g & 1) + 16 * (g >> 1) + (reg & 15);
}

__device__ __forceinline__ void fwht_cross64_swap(float (&v)[64]) {
#pragma unroll
  for (int p = 0; p < 32; ++p) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[p]),
                                                    __float_as_uint(v[p + 32]), false, false);
    const float x = __uint_as_float(r[0]), y = __uint_as_float(r[1]);
    v[p] = x + y;
    v[p + 32] = x - y;
  }
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    if (i & 16) continue;
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]),
                                                    __float_as_uint(v[i + 16]), false, false);
    const float x = __uint_as_float(r[0]), y = __uint_as_float(r[1]);
    v[i] = x + y;
    v[i + 16] = x - y;
  }
}

__device__ __forceinline__ void fwht256_wave(float (&v)[64], int lane) {
  fwht_inreg64(v);
  fwht_cross64(v, lane);
}

// Low-rank product for the wave's 16 rows x 256 columns, accumulated into the
// wave layout above:
//   v[4t+i] += sign * sum_r up[row0 + l%16][r] * down[col0 + 64*(l/16) + 4t + i][r]
// on bf16 MFMA (exact products, fp32 sums), with v as the accumulator input.
// The MFMA's row index rho = 4*(l/16)+i of tile t is mapped to column
// 64*(rho/4) + 4t + rho%4, so each lane's 64 consecutive columns line up with
// its registers.  sign = -1 flips the bf16 sign bits of `down` (exact).
// Rows of `up` at or beyond n_rows read as zero; rank is a multiple of 16
// (ranks past `rank` in the last 32-wide step read as zero).
__device__ __forceinline__ void lowrank_acc_16x256(float (&v)[64], const uint16_t* __restrict__ up,
                                                   const uint16_t* __restrict__ down, int64_t row0,
                                                   int64_t n_rows, int64_t col0, int rank,
                                                   bool negate, int lane) {
  const int c = lane & 15, g = lane >> 4;
  const uint32_t flip = negate ? 0x80008000u : 0u;
  for (int rr = 0; rr < rank; rr += 32) {
    const bool rk = rr + 8 * g < rank;   // false only in the upper half of a rank-16 step
    // B operand (k = r, col = output row): lane holds up[row0 + c][rr + 8g .. +8]
    bf16x8 bfrag;
    if (rk && row0 + c < n_rows) {
      bfrag = *reinterpret_cast<const bf16x8*>(up + (row0 + c) * rank + rr + 8 * g);
    } else {
      bfrag = (bf16x8){};
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      // A operand (row rho = c, k = r): down row of column 64*(c/4) + 4t + c%4
      const int64_t col = col0 + 64 * (c >> 2) + 4 * t + (c & 3);
      u32x4 raw = rk ? *reinterpret_cast<const u32x4*>(down + col * rank + rr + 8 * g)
                     : (u32x4){0u, 0u, 0u, 0u};
      raw ^= (u32x4){flip, flip, flip, flip};
      const bf16x8 afrag = __builtin_bit_cast(bf16x8, raw);
      f32x4 acc = {v[4 * t], v[4 * t + 1], v[4 * t + 2], v[4 * t + 3]};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag, bfrag, acc, 0, 0, 0);
      v[4 * t] = acc[0];
      v[4 * t + 1] = acc[1];
      v[4 * t + 2] = acc[2];
      v[4 * t + 3] = acc[3];
    }
  }
}

}  // namespace sq
