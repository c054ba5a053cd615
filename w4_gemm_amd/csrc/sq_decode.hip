// Small-M forward (M <= 16, the decode shapes): the same product as the
// tiled forward (SquareQ README, "SquareQ v3 - W4": x @ W_hat^T =
// (x H) @ dequant(R)^T + (x @ lora_down) @ lora_up^T), in two launches that
// stream the packed payload once:
//
//   1. k_fwd_decode, grid (K slices, ceil(N/256) + 1).  Workgroup (s, j <
//      last) owns weight rows 256j .. 256j+255 and the K slice s.  It loads
//      its slice of x first, then issues the code loads of its first blocks
//      and, while they are in flight, rotates the slice in LDS:
//        E[m][s]  = ceil(log2 max_{k in slice} |x[m][k]|),
//        xs[m][k] = fp16( (x H)[m][k] * 2^(11 - E) / 16 )   (|xs| <= 2^15).
//      The slice is then contracted on fp16 MFMA (one rounding of the exact
//      q*s per weight, fp32 sums) and the partial sums, times 2^(E - 11), go
//      to partial[s][m][n].  The extra column of workgroups (j = last)
//      computes t_s = x[:, slice] @ lora_down[slice, :] on bf16 MFMA (exact
//      products, fp32 sums).
//   2. k_decode_reduce: y[m][n] = sum_s partial_s[m][n] + sum_r t[m][r] up[n][r],
//      t = sum_s t_s, in fp32 with the slices in order.
//
// The rotation is repeated by the ceil(N/256) workgroups of a slice; at
// M <= 16 it is a few hundred vector instructions per wave, done while the
// first codes load.  Rows of the 16-row MFMA tile at or past M read row M-1
// of xs: row i of an MFMA product depends on row i of its first operand
// only, and those rows are never stored.
#include "sq_device.hpp"
#include "sq_kernels.h"

#include <algorithm>

namespace sq {
namespace {

typedef _Float16 dec_half2 __attribute__((ext_vector_type(2)));

constexpr int DEC_MAX_M = 16;
constexpr int DEC_NB_MAX = 4;                    // blocks per K slice at most
constexpr int DEC_KS_MAX = 256 * DEC_NB_MAX;
constexpr int DEC_XS = DEC_KS_MAX + 8;           // halves per LDS activation row (16 B pad)
// Blocks of codes in flight per wave.  One (the next block's loads go out
// once the current block is contracted) measured fastest: with two waves
// per SIMD the other wave covers the wait, and fewer requests in flight
// keep the memory queues short and the waves' progress even (two or three
// blocks ahead left some waves stalled at issue for microseconds).
constexpr int DEC_DEPTH = 1;

// s_waitcnt immediate: lgkmcnt(0), the other counters untouched.
constexpr int DEC_WAIT_LGKM0 = 0xC07F;

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its global loads in flight (a fence would).  The signal
// fences keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(DEC_WAIT_LGKM0);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Value of lane ^ BIT (BIT < 16) by a DPP move (CTRL >= 0: a quad
// permutation or a row rotation by 8) or a bitmask swizzle (CTRL < 0).
template <int CTRL, int BIT>
__device__ __forceinline__ int lane_xor(int v) {
  if constexpr (CTRL >= 0)
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
  else
    return __builtin_amdgcn_ds_swizzle(v, (BIT << 10) | 0x1F);
}
constexpr int DPP_XOR1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int DPP_ROR8 = 0x128;   // row_ror:8 (= lane ^ 8 within 16 lanes)

// One butterfly stage across lane bit log2(BIT) for 16 values per lane: the
// lane with the bit clear keeps a + b, the other a - b (a = the clear lane's).
template <int CTRL, int BIT>
__device__ __forceinline__ void lane_stage16(float (&v)[16], int lane) {
  const float sg = (lane & BIT) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    v[i] = __builtin_fmaf(sg, v[i], __int_as_float(lane_xor<CTRL, BIT>(__float_as_int(v[i]))));
}

// Hadamard-256 butterflies of one block row held as 16 lanes x 16 values
// (lane l % 16 holds block positions 16(l%16) + 0..15), unnormalized.
__device__ __forceinline__ void fwht16_lanes16(float (&v)[16], int lane) {
#pragma unroll
  for (int hb = 1; hb < 16; hb <<= 1)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if ((i & hb) == 0) {
        const float a = v[i], c = v[i + hb];
        v[i] = a + c;
        v[i + hb] = a - c;
      }
  lane_stage16<DPP_XOR1, 1>(v, lane);
  lane_stage16<DPP_XOR2, 2>(v, lane);
  lane_stage16<-1, 4>(v, lane);
  lane_stage16<DPP_ROR8, 8>(v, lane);
}

// v * f as fp16, each 8-value run in the K order [0,4,1,5,2,6,3,7]: words (k, k + 4).
__device__ __forceinline__ void pack_xs(const float (&v)[16], float f, u32x4& o0, u32x4& o1) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const dec_half2 h0 = {(_Float16)(v[p] * f), (_Float16)(v[p + 4] * f)};
    const dec_half2 h1 = {(_Float16)(v[8 + p] * f), (_Float16)(v[12 + p] * f)};
    o0[p] = __builtin_bit_cast(uint32_t, h0);
    o1[p] = __builtin_bit_cast(uint32_t, h1);
  }
}

// ---------------------------------------------------------------- low-rank column
// t_s[m][r] = sum over slice s of x[m][k] down[k][r] on bf16 MFMA, one wave
// per 256-value block: lane (fr, g) supplies x row fr (rows at or past m read
// as zeros) and, gathered with 2-byte loads (lora_down is stored K-major),
// eight consecutive K of column 16rt + fr.  The waves' sums are added in
// block order; rows m..15 of t_s are zeros.
__device__ __forceinline__ void decode_lowrank(const uint16_t* __restrict__ x,
                                               const uint16_t* __restrict__ down,
                                               float* __restrict__ t_slice, float* red_mem,
                                               int64_t m, int64_t k, int rank, int64_t k0, int nb,
                                               int s) {
  float (*red)[DEC_MAX_M][64] = reinterpret_cast<float (*)[DEC_MAX_M][64]>(red_mem);
  const int tid = threadIdx.x, lane = tid & 63, fr = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool active = wave < nb;
  const int64_t kb = k0 + 256 * wave;
  const __amdgpu_buffer_rsrc_t x_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)(m * k * 2), 0x00020000);
  const int rt_n = rank >> 4;   // 0, 2 or 4 rank tiles of 16
  const uint32_t oob = active ? 0u : 0x80000000u;   // an idle wave reads zeros
  const __amdgpu_buffer_rsrc_t d_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)down, (short)0, (int)(k * rank * 2), 0x00020000);
  // operands of the rank-r projection for 4 of the block's 8 K steps: x row
  // fr (rows at or past m come back as zeros) and eight K of column 16rt + fr
  auto load_t = [&](bf16x8 (&a)[4], uint32_t (&dv)[4][4][8], int half) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t kk = kb + 32 * (4 * half + u) + 8 * g;
      a[u] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                            x_rsrc, oob + (uint32_t)((fr * k + kk) * 2), 0, 0));
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        if (rt >= rt_n) break;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          dv[u][rt][e] = __builtin_amdgcn_raw_buffer_load_b16(
              d_rsrc, oob + (uint32_t)(((kk + e) * rank + 16 * rt + fr) * 2), 0, 0);
      }
    }
  };
  f32x4 acc[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) acc[rt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  auto mma_t = [&](const bf16x8 (&a)[4], const uint32_t (&dv)[4][4][8]) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        if (rt >= rt_n) break;
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (dv[u][rt][2 * e] & 0xFFFFu) | (dv[u][rt][2 * e + 1] << 16);
        acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], __builtin_bit_cast(bf16x8, w), acc[rt],
                                                          0, 0, 0);
      }
  };

  bf16x8 ta[4];
  uint32_t td[4][4][8];
  load_t(ta, td, 0);
  mma_t(ta, td);
  load_t(ta, td, 1);
  mma_t(ta, td);
  // acc[rt][i] = t_b[4g + i][16 rt + fr] (zero for rows past m)
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    if (rt >= rt_n) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * g + i][16 * rt + fr] = acc[rt][i];
  }
  lds_barrier();
  for (int i = tid; i < DEC_MAX_M * rank; i += 256) {
    const int row = i / rank, r = i - row * rank;
    float t = red[0][row][r];
    for (int w = 1; w < nb; ++w) t += red[w][row][r];
    t_slice[((int64_t)s * DEC_MAX_M + row) * rank + r] = t;
  }
}


// ---------------------------------------------------------------- contraction
template <int GSHIFT>
__global__ void __launch_bounds__(256) k_fwd_decode(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ down,
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    float* __restrict__ partial, float* __restrict__ t_slice, int64_t m, int64_t n, int64_t k,
    int rank, int kslice, int ntiles) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[DEC_MAX_M * DEC_XS];
  __shared__ uint32_t s_max[DEC_MAX_M];
  const int tid = threadIdx.x, lane = tid & 63, fr = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = blockIdx.x;
  const int64_t k0 = (int64_t)s * kslice;
  const int nb = (int)((std::min<int64_t>(k, k0 + kslice) - k0) >> 8);   // blocks in the slice
  if ((int)blockIdx.y == ntiles) {
    decode_lowrank(x, down, t_slice, reinterpret_cast<float*>(smem), m, k, rank, k0, nb, s);
    return;
  }

  // ---- the slice of x (rows below m, 16-byte chunks) to LDS as raw bf16,
  // with the slice maxima per row.  Loaded, and waited for, before any code
  // load, so these few bytes do not queue behind the payload.
  const __amdgpu_buffer_rsrc_t x_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)(m * k * 2), 0x00020000);
  const int cpr = nb * 32, nchunks = (int)m * cpr;
  constexpr int XJ = DEC_MAX_M * DEC_KS_MAX / 8 / 256;
  {
    u32x4 xv[XJ];
#pragma unroll
    for (int j = 0; j < XJ; ++j) {
      const int i = tid + 256 * j;
      const int r = i / cpr, cc = i - r * cpr;
      const uint32_t off = i < nchunks ? (uint32_t)((r * k + k0 + 8 * cc) * 2) : 0x80000000u;
      xv[j] = __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, off, 0, 0);
    }
    if (tid < DEC_MAX_M) s_max[tid] = 0;
    lds_barrier();   // s_max cleared
#pragma unroll
    for (int j = 0; j < XJ; ++j) {
      const int i = tid + 256 * j;
      if (i >= nchunks) break;
      const int r = i / cpr, cc = i - r * cpr;
      *reinterpret_cast<u32x4*>(smem + r * DEC_XS + 8 * cc) = xv[j];
      uint32_t mx = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        mx = std::max(mx, std::max(xv[j][e] & 0x7FFFu, (xv[j][e] >> 16) & 0x7FFFu));
      if (mx) __hip_atomic_fetch_max(&s_max[r], mx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- codes and scales: lane (fr, g) of wave w reads weight row
  // n0 + 16t + fr, bytes 32g .. 32g+31 of each block's 128-byte line (K
  // values 64g .. 64g+63 of the block), and the scales of those K values.
  // The int8 payload (GSHIFT 0): bytes 64g .. 64g+63 of the block's 256,
  // one scale per weight row, applied with the row exponent at the end.
  constexpr int CW = GSHIFT ? 2 : 4;                  // 16-byte code pieces per block and tile
  constexpr uint32_t BSTR = GSHIFT ? 128u : 256u;     // code bytes of a block's row
  const int64_t n0 = (int64_t)blockIdx.y * 256 + 64 * wave;
  const int64_t rowb = GSHIFT ? (k >> 1) : k, ngroups = GSHIFT ? (k >> GSHIFT) : 1;
  const int64_t w_rows = std::max<int64_t>(0, std::min<int64_t>(64, n - n0));
  const __amdgpu_buffer_rsrc_t c_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(codes + std::min(n0, n) * rowb), (short)0, (int)(w_rows * rowb), 0x00020000);
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(scales + std::min(n0, n) * ngroups), (short)0, (int)(w_rows * ngroups * 2), 0x00020000);
  uint32_t c_off[4], s_off[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if constexpr (GSHIFT == 0)
      c_off[t] = (uint32_t)((16 * t + fr) * rowb + k0) + 64u * g;
    else
      c_off[t] = (uint32_t)((16 * t + fr) * rowb + (k0 >> 1)) + 32u * g;
    if constexpr (GSHIFT == 5)
      s_off[t] = (uint32_t)(((16 * t + fr) * ngroups + (k0 >> 5)) * 2) + 4u * g;
    else if constexpr (GSHIFT == 6)
      s_off[t] = (uint32_t)(((16 * t + fr) * ngroups + (k0 >> 6)) * 2) + 2u * g;
    else
      s_off[t] = 0;
  }
  // block b: CW x 16 bytes of codes and the lane's scales (two fp16 of group
  // size 32 in one word, one of group size 64) per tile; b >= nb reads zeros
  auto load_blk = [&](u32x4 (&cw)[4][CW], uint32_t (&sc)[4], int b) {
    const uint32_t off = b < nb ? 0u : 0x80000000u;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int q = 0; q < CW; ++q)
        cw[t][q] = __builtin_amdgcn_raw_buffer_load_b128(c_rsrc, off + c_off[t] + BSTR * b + 16u * q,
                                                         0, 0);
      if constexpr (GSHIFT == 5)
        sc[t] = __builtin_amdgcn_raw_buffer_load_b32(s_rsrc, off + s_off[t] + 16u * b, 0, 0);
      else if constexpr (GSHIFT == 6)
        sc[t] = __builtin_amdgcn_raw_buffer_load_b16(s_rsrc, off + s_off[t] + 8u * b, 0, 0);
      else
        sc[t] = 0;
    }
  };
  u32x4 cw[DEC_DEPTH][4][CW];
  uint32_t sc[DEC_DEPTH][4];
#pragma unroll
  for (int d = 0; d < DEC_DEPTH; ++d) {
    load_blk(cw[d], sc[d], d);
    __builtin_amdgcn_sched_barrier(0);   // block by block, in order
  }
  lds_barrier();

  // ---- rotation in place, while the first codes are in flight.  Four
  // (row, block) tasks per wave instruction: lane l works on task slot l/16
  // and holds block positions 16(l%16) + 0..15, so index bits 0..3 are in
  // registers and bits 4..7 in lane bits 0..3.
  {
    const int ql = lane >> 4, il = lane & 15;
    const int ntask = (int)m * nb;
    for (int base = 4 * wave; base < ntask; base += 16) {
      const int task = base + ql;
      const bool ok = task < ntask;
      const int tt = ok ? task : base;
      const int r = tt / nb, b = tt - r * nb;
      uint16_t* seg = smem + r * DEC_XS + 256 * b + 16 * il;
      const u32x4 w0 = *reinterpret_cast<const u32x4*>(seg);
      const u32x4 w1 = *reinterpret_cast<const u32x4*>(seg + 8);
      float v[16];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = bf16_to_f32(w0[e] & 0xFFFFu);
        v[2 * e + 1] = bf16_to_f32(w0[e] >> 16);
        v[8 + 2 * e] = bf16_to_f32(w1[e] & 0xFFFFu);
        v[9 + 2 * e] = bf16_to_f32(w1[e] >> 16);
      }
      fwht16_lanes16(v, lane);
      const float f = ldexpf(1.0f, 11 - row_exponent(s_max[r])) * 0.0625f;   // a power of two
      u32x4 o0, o1;
      pack_xs(v, f, o0, o1);
      if (ok) {
        *reinterpret_cast<u32x4*>(seg) = o0;
        *reinterpret_cast<u32x4*>(seg + 8) = o1;
      }
    }
  }
  lds_barrier();

  // ---- contraction: block b, 16-byte piece c, word e: one 16x16x32 MFMA per
  // tile over K values 64g + 32c + 8e + (0..7) of the block
  f32x4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const uint16_t* a_base = smem + std::min<int64_t>(fr, m - 1) * DEC_XS + 64 * g;
#pragma unroll
  for (int b = 0; b < DEC_NB_MAX; ++b) {
    const int d = b % DEC_DEPTH;
    if (b < nb) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        half8 af[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          af[e] = *reinterpret_cast<const half8*>(a_base + 256 * b + 32 * c + 8 * e);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if constexpr (GSHIFT == 0) {
            // K values 64g + 32c + 8e .. +7: bytes 8e' .. 8e'+7 of piece 2c + e/2
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const u32x4& pc = cw[d][t][2 * c + (e >> 1)];
              acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  af[e], dequant8_i8(pc[2 * (e & 1)], pc[2 * (e & 1) + 1]), acc[t], 0, 0, 0);
            }
          } else {
            const uint32_t sbits =
                GSHIFT == 5 ? (c ? sc[d][t] >> 16 : sc[d][t] & 0xFFFFu) : sc[d][t] & 0xFFFFu;
            const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)sbits);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[e], dequant8_f16(cw[d][t][c][e], sv),
                                                              acc[t], 0, 0, 0);
          }
        }
      }
    }
    if (b + DEC_DEPTH < DEC_NB_MAX) load_blk(cw[d], sc[d], b + DEC_DEPTH);
  }

  // ---- partial[s][row][col] = acc * 2^(E - 11) (int8: times the weight
  // row's scale); acc[t][i]: row 4g + i, col n0 + 16t + fr
  float cs[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t c = n0 + 16 * t + fr;
    cs[t] = (GSHIFT == 0 && c < n) ? (float)__builtin_bit_cast(_Float16, scales[c]) : 1.0f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * g + i;
    if (r >= m) continue;
    const float rs = ldexpf(1.0f, row_exponent(s_max[r]) - 11);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t c = n0 + 16 * t + fr;
      if (c < n) partial[((int64_t)s * m + r) * n + c] = GSHIFT == 0 ? (acc[t][i] * cs[t]) * rs
                                                                      : acc[t][i] * rs;
    }
  }
}

// ---------------------------------------------------------------- reduce
// grid (ceil(n/256), m), one output column per thread:
//   y[m][n] = sum_s partial_s[m][n] + sum_r t[m][r] up[n][r],  t = sum_s t_s,
// in fp32, slices in order.  The row's t goes to LDS once per workgroup; its
// loads and the partial loads are all issued before either sum.
__global__ void __launch_bounds__(256) k_decode_reduce(const float* __restrict__ partial,
                                                       const float* __restrict__ t_slice,
                                                       const uint16_t* __restrict__ up,
                                                       void* __restrict__ y, int64_t m, int64_t n,
                                                       int rank, int splits, int y_bf16) {
  __shared__ float s_t[64];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.y;
  const int64_t col = std::min((int64_t)blockIdx.x * 256 + tid, n - 1);
  const int64_t mn = m * n;
  // the column's up row first, so that every load of the thread is in flight together
  u32x4 urow[8];
  const u32x4* usrc = reinterpret_cast<const u32x4*>(up + col * rank);
#pragma unroll
  for (int c = 0; c < 8; ++c)
    if (c < (rank >> 3)) urow[c] = usrc[c];
  float sum = 0.0f, t = 0.0f;
  for (int z0 = 0; z0 < splits; z0 += 16) {
    float pv[16], tv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int z = std::min(z0 + u, splits - 1);
      pv[u] = partial[(int64_t)z * mn + row * n + col];
      tv[u] = tid < rank ? t_slice[((int64_t)z * DEC_MAX_M + row) * rank + tid] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (z0 + u < splits) {
        sum += pv[u];
        t += tv[u];
      }
  }
  if (tid < rank) s_t[tid] = t;
  __syncthreads();
  if ((int64_t)blockIdx.x * 256 + tid >= n) return;
  float lr = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    if (c >= (rank >> 3)) break;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lr = __builtin_fmaf(s_t[8 * c + 2 * e], bf16_to_f32(urow[c][e] & 0xFFFFu), lr);
      lr = __builtin_fmaf(s_t[8 * c + 2 * e + 1], bf16_to_f32(urow[c][e] >> 16), lr);
    }
  }
  const float out = sum + lr;
  if (y_bf16)
    reinterpret_cast<uint16_t*>(y)[row * n + col] = f32_to_bf16(out);
  else
    reinterpret_cast<float*>(y)[row * n + col] = out;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

bool decode_eligible(int64_t m, int64_t n, int64_t k, int rank, bool int8) {
  // 32-bit buffer offsets: 16 rows of x, one wave's 64 weight rows, lora_down
  return m >= 1 && m <= DEC_MAX_M && DEC_MAX_M * k * 2 < ((int64_t)1 << 31) &&
         64 * (int8 ? k : (k >> 1)) < ((int64_t)1 << 31) && k * rank * 2 < ((int64_t)1 << 31) &&
         (rank == 0 || (int8 && rank == 16) || rank == 32 || rank == 64);
}

// K slice: the longest (at most 1024 values) that still gives about 1600
// waves of 64 weight rows (one to two per SIMD): each wave then streams a few
// blocks, and fewer slices mean fewer fp32 partials.
FwdPlan plan_decode(int64_t m, int64_t n, int64_t k, int group, int rank) {
  FwdPlan p{};
  p.m = m; p.n = n; p.k = k; p.group = group; p.rank = rank;
  p.dec = 1;
  const int64_t ntiles = (n + 255) / 256, nblk = k / 256;
  int64_t bps = (nblk * 4 * ntiles + 1599) / 1600;
  bps = std::max<int64_t>(1, std::min<int64_t>(bps, DEC_NB_MAX));
  p.dec_kslice = (int)(bps * 256);
  p.splits = (int)((k + p.dec_kslice - 1) / p.dec_kslice);
  p.tile_m = DEC_MAX_M; p.tile_n = 256;
  size_t off = 0;
  p.off_xh = off;       off = align256(off + (size_t)m * k * 2);   // x, staged by the split calls
  p.off_downT = off;    off = align256(off + (size_t)k * std::max(rank, 1) * 2);   // lora_down, same
  p.off_tpart = off;    off = align256(off + (size_t)p.splits * DEC_MAX_M * std::max(rank, 1) * 4);
  p.off_partial = off;  off = align256(off + (size_t)p.splits * m * n * 4);
  p.total = off;
  return p;
}

// The first of the split calls stages x and lora_down in the workspace; the
// second then reads them there.
hipError_t launch_decode_prep(const FwdPlan& p, const uint16_t* x, const uint16_t* down,
                              void* workspace, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  hipError_t err =
      hipMemcpyAsync(ws + p.off_xh, x, (size_t)p.m * p.k * 2, hipMemcpyDeviceToDevice, stream);
  if (err != hipSuccess || p.rank == 0) return err;
  return hipMemcpyAsync(ws + p.off_downT, down, (size_t)p.k * p.rank * 2, hipMemcpyDeviceToDevice,
                        stream);
}

hipError_t launch_decode_contract(const FwdPlan& p, const uint16_t* x, const uint16_t* down,
                                  const uint8_t* codes, const uint16_t* scales, const uint16_t* up,
                                  void* y, int y_bf16, void* workspace, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  if (!x) x = reinterpret_cast<const uint16_t*>(ws + p.off_xh);
  if (!down) down = reinterpret_cast<const uint16_t*>(ws + p.off_downT);
  float* t_slice = reinterpret_cast<float*>(ws + p.off_tpart);
  float* partial = reinterpret_cast<float*>(ws + p.off_partial);
  const int ntiles = (int)((p.n + 255) / 256);
  const dim3 grid((unsigned)p.splits, (unsigned)(ntiles + (p.rank > 0 ? 1 : 0)));
  if (p.group == 32)
    hipLaunchKernelGGL(k_fwd_decode<5>, grid, dim3(256), 0, stream, x, down, codes, scales, partial,
                       t_slice, p.m, p.n, p.k, p.rank, p.dec_kslice, ntiles);
  else if (p.group == 0)
    hipLaunchKernelGGL(k_fwd_decode<0>, grid, dim3(256), 0, stream, x, down, codes, scales, partial,
                       t_slice, p.m, p.n, p.k, p.rank, p.dec_kslice, ntiles);
  else
    hipLaunchKernelGGL(k_fwd_decode<6>, grid, dim3(256), 0, stream, x, down, codes, scales, partial,
                       t_slice, p.m, p.n, p.k, p.rank, p.dec_kslice, ntiles);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_decode_reduce, dim3((unsigned)((p.n + 255) / 256), (unsigned)p.m), dim3(256),
                     0, stream, partial, t_slice, up, y, p.m, p.n, p.rank, p.splits, y_bf16);
  return hipGetLastError();
}

}  // namespace sq
