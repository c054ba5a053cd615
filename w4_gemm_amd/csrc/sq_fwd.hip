// Fused W4 forward (SquareQ README, "SquareQ v3 - W4": the format formula
// applied to an activation; H symmetric gives x @ W_hat^T = (x H) @ D^T +
// (x @ down) @ up^T with D = dequant(R)):
//
//   y[m][n] = 2^(E_m - 11) * ( sum_k xh16[m][k] * fp16(q[n][k] s[n][k/G])
//                              + sum_r t16[m][r] * up[n][r] )
//
// Launches on the caller's stream:
//   1. k_fwd_stats: per 16 rows and one slice of K, the partial row absmax
//      and the partial t = x @ down on bf16 MFMA (one read of x).  At rank 64
//      a tiny k_transpose_down (down [K][r] -> downT [r][K]) runs first.
//   2. k_fwd_rotate: per 16 rows x one 256-column block, E_m = ceil(log2 A_m)
//      from the slices' maxima and xh = (x H) * 2^(11-E_m) with the 256-point
//      butterflies in registers and lane swaps, rounded to fp16 (|xh| <= 2^15
//      because every entry of x H is at most 16 A_m) and stored through an
//      LDS transpose; the first column group also adds the slices of t in a
//      fixed order and splits t * 2^(11-E_m) into bf16 hi + lo.
//      For K <= 4096 at ranks 0, 16 and 32, k_fwd_prep does 1 and 2 in one
//      launch, one workgroup per 16-row strip.
//   3. k_fwd_gemm_big (M > 64) or k_fwd_skinny: the int4 contraction on fp16 MFMA.  The packed codes stream
//      from HBM as 16-byte loads, become fp16(q*s) in LDS (one rounding of the
//      exact product), and meet the fp16 activations; the rank-r branch is two
//      bf16 MFMA passes (hi and lo) into the same accumulators; the epilogue
//      applies 2^(E_m - 11) and stores fp32 or bf16.  With split-K the partial
//      sums go to the workspace and k_fwd_reduce adds them in a fixed order.
//
// The K order inside every group of 8 is [0,4,1,5,2,6,3,7] in both operands:
// that is the order in which one 32-bit word of packed nibbles unpacks into
// four fp16 pairs with one mask each.
#include "sq_device.hpp"
#include "sq_kernels.h"

#include <algorithm>
#include <type_traits>

namespace sq {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- transpose
__global__ void __launch_bounds__(256) k_transpose_down(const uint16_t* __restrict__ down,
                                                         uint16_t* __restrict__ downT, int64_t k,
                                                         int rank) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // index into downT
  if (i >= k * rank) return;
  const int64_t r = i / k, kk = i - r * k;
  downT[i] = down[kk * rank + r];
}

// ---------------------------------------------------------------- pre-phase
constexpr int PRE_WAVES = 4;
constexpr int PRE_STAGE_U4 = 33;   // LDS staging row: 32 x 16 bytes + one pad slot
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// 64 consecutive bf16 of one row (128 bytes) as 32 words.
__device__ __forceinline__ void load_x64(uint32_t (&xb)[32], const uint16_t* __restrict__ src) {
  const u32x4* p = reinterpret_cast<const u32x4*>(src);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const u32x4 q = p[j];
    xb[4 * j] = q[0];
    xb[4 * j + 1] = q[1];
    xb[4 * j + 2] = q[2];
    xb[4 * j + 3] = q[3];
  }
}

// Pass 1: grid (ceil(m / (16 TILES)), slices); slice q covers the
// 256-column blocks [q*bps, q*bps + bps) and the workgroup's four waves take
// every fourth one, for TILES 16-row tiles of rows each.  A wave loads its
// block's factor fragments (the MFMA B operand) once and contracts every row
// tile against them, so the factor is read once per TILES tiles; the x loads
// of PF tiles are in flight at once (a ring of PF register sets), so a wave
// streams up to PF x 8 KB of x while it contracts.
// KMAJOR: the factor is given as stored, [k][RANK] (lora_down, or lora_up
// for the input gradient): each wave stages its block's 256 rows of it in
// LDS with direct loads, issued ahead of its x loads, and gathers its
// fragments there (the area then holds the wave's reduction scratch).  Else
// it is given transposed, [RANK][k], and the fragments are read from it.
// Writes amax_part[q][row] (bf16 magnitude bits; they order like the values)
// and t_part[q][row][r] (fp32) for the rows below m.
template <int RANK, int TILES, bool KMAJOR>
__global__ void __launch_bounds__(64 * PRE_WAVES) k_fwd_stats(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ fac, int64_t m, int64_t k,
    int bps, uint32_t* __restrict__ amax_part, float* __restrict__ t_part) {
  static_assert(!KMAJOR || (RANK > 0 && RANK <= 32), "staged factor: ranks 16 and 32");
  constexpr int RT = RANK / 16;   // 16-wide rank tiles
  // tiles in flight: the register sets that fit beside the fragments and sums
  constexpr int PF_MAX = RANK > 32 ? 2 : TILES > 4 ? 2 : 4;
  constexpr int PF = TILES < PF_MAX ? TILES : PF_MAX;
  // per wave: its block's factor rows (KMAJOR), or at least its 16 x 64 fp32 sums
  constexpr int WAVE_LDS = KMAJOR ? 256 * RANK * 2 : 16 * 64 * 4;
  static_assert(WAVE_LDS >= 16 * 64 * 4, "the sums fit the staging area");
  __shared__ __attribute__((aligned(16))) uint8_t wave_lds[PRE_WAVES][WAVE_LDS];
  __shared__ uint32_t red_max[PRE_WAVES][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int64_t rbase = (int64_t)blockIdx.x * 16 * TILES;
  const int64_t nblk = k >> 8, q = blockIdx.y;
  const int64_t b_end = min(nblk, (q + 1) * bps);

  f32x4 acc[TILES][RT > 0 ? RT : 1] = {};
  u16x2 amax2[TILES];
#pragma unroll
  for (int tl = 0; tl < TILES; ++tl) amax2[tl] = (u16x2){0, 0};
  for (int64_t b = q * bps + wave; b < b_end; b += PRE_WAVES) {
    // MFMA j contracts columns 32j .. 32j+31 of the block; lane (c, g) holds
    // eight of them, 32j + 8g .. +7, so the four lanes of a row read 64
    // contiguous bytes (of x and of each factor row) per instruction.
    const int64_t col = b * 256 + 8 * g;
    constexpr int NSTAGE = KMAJOR ? 256 * RANK * 2 / 1024 : 0;   // 1 KB direct loads
    if constexpr (KMAJOR) {
      // the block's 256 factor rows (256 * RANK * 2 contiguous bytes) go to
      // this wave's LDS area first; the x loads below are issued behind them
      const __amdgpu_buffer_rsrc_t f_rsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(fac + b * 256 * RANK), (short)0, 256 * RANK * 2, 0x00020000);
#pragma unroll
      for (int i = 0; i < NSTAGE; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            f_rsrc, (__attribute__((address_space(3))) void*)(&wave_lds[wave][0] + i * 1024), 16,
            (uint32_t)(lane * 16 + i * 1024), 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    u32x4 xv[PF][8];
    auto load_tile = [&](u32x4 (&dst)[8], int tl) {
      const int64_t lrow = min(rbase + 16 * tl + c, m - 1);   // rows past m read the last row
#pragma unroll
      for (int j = 0; j < 8; ++j)
        dst[j] = *reinterpret_cast<const u32x4*>(x + lrow * k + col + 32 * j);
    };
#pragma unroll
    for (int tl = 0; tl < PF; ++tl) load_tile(xv[tl], tl);
    bf16x8 bfrag[RT > 0 ? RT : 1][8];
    if constexpr (KMAJOR) {
      // the staged rows have landed once no more than the x loads behind
      // them are outstanding (loads complete in order)
      __builtin_amdgcn_sched_barrier(0);
      constexpr int XL = PF * 8;
      __builtin_amdgcn_s_waitcnt(sq_wait_vm(XL));
      __builtin_amdgcn_sched_barrier(0);
      // element e of fragment (rt, j): factor row 32j + 8g + e, column 16rt + c
      const uint16_t* st = reinterpret_cast<const uint16_t*>(&wave_lds[wave][0]);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          bf16x8 f;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            f[e] = __builtin_bit_cast(__bf16, st[(32 * j + 8 * g + e) * RANK + 16 * rt + c]);
          bfrag[rt][j] = f;
        }
    } else {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          bfrag[rt][j] =
              *reinterpret_cast<const bf16x8*>(fac + (int64_t)(16 * rt + c) * k + col + 32 * j);
    }
#pragma unroll
    for (int tl = 0; tl < TILES; ++tl) {
      const u32x4 (&xt)[8] = xv[tl % PF];
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          amax2[tl] =
              __builtin_elementwise_max(amax2[tl], __builtin_bit_cast(u16x2, xt[j][e] & 0x7FFF7FFFu));
      // t: A = x (row c), B = the factor (r = 16rt + c), both over the same columns
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bf16x8 afrag = __builtin_bit_cast(bf16x8, xt[j]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          acc[tl][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag, bfrag[rt][j], acc[tl][rt], 0, 0, 0);
      }
      // the freed register set takes tile tl + PF
      if (tl + PF < TILES) load_tile(xv[tl % PF], tl + PF);
    }
  }
  // per row tile: acc[tl][rt][i] = partial t[rbase + 16 tl + 4g + i][16 rt + c];
  // wave w's sums go to the start of its own LDS area (after its factor
  // fragments have been read from there)
  auto red_t = [&](int w) { return reinterpret_cast<float(*)[64]>(&wave_lds[w][0]); };
#pragma unroll
  for (int tl = 0; tl < TILES; ++tl) {
    const int64_t row0 = rbase + 16 * tl;
    if (tl > 0) __syncthreads();   // the previous tile's sums have been read
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red_t(wave)[4 * g + i][16 * rt + c] = acc[tl][rt][i];
    red_max[wave][lane] = max((uint32_t)amax2[tl][0], (uint32_t)amax2[tl][1]);
    __syncthreads();
    if constexpr (RANK > 0) {
      for (int i = tid; i < 16 * RANK; i += 64 * PRE_WAVES) {
        const int rr = i / RANK, r = i - rr * RANK;
        if (row0 + rr >= m) continue;
        float t = 0.0f;
#pragma unroll
        for (int w = 0; w < PRE_WAVES; ++w) t += red_t(w)[rr][r];
        t_part[(q * m + row0 + rr) * RANK + r] = t;
      }
    }
    if (tid < 16 && row0 + tid < m) {
      uint32_t mx = 0;
#pragma unroll
      for (int w = 0; w < PRE_WAVES; ++w)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) mx = max(mx, red_max[w][tid + 16 * gg]);
      amax_part[q * m + row0 + tid] = mx;
    }
  }
}

// Hadamard-256 of a 16-row x 256-column block on the matrix cores.  With
// the column index k = 32 kh + kl, Sylvester's matrix factors as
// S256[k][n] = S8[kh][nh] S32[kl][nl] (n = 32 nh + nl), so
//   1. per 32-column chunk kh, two bf16 MFMAs against S32 (entries +-1: the
//      products are exact, the sums fp32) give Y[kh][nl] = sum_kl x[32kh+kl] S32[kl][nl];
//   2. the 8-point transform over kh runs in each lane's registers.
// A operand: lane (c, g) holds xf[kh] = x[row c][32 kh + 8g .. +7], the
// statistics pass's layout.  The S32 columns are ordered so that output
// column c' of half h is nl = fwht_out_col(h, c') = 8 (c' >> 2) + (c' & 3) + 4h:
// a lane then holds both columns of one word of the xh layout (word p of every
// 8-column run holds columns p and p + 4).
// Result: z[h][nh][i] = (S256 x)[row 4g + i][32 nh + fwht_out_col(h, c)].
__device__ __forceinline__ int fwht_out_col(int h, int cc) { return 8 * (cc >> 2) + (cc & 3) + 4 * h; }

__device__ __forceinline__ void s32_fragments(bf16x8 (&s)[2], int lane) {
  const int c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      s[h][e] = (__builtin_popcount((8 * g + e) & fwht_out_col(h, c)) & 1) ? (__bf16)-1.0f : (__bf16)1.0f;
}

__device__ __forceinline__ void fwht256_mfma(const bf16x8 (&xf)[8], const bf16x8 (&s)[2],
                                             f32x4 (&z)[2][8]) {
#pragma unroll
  for (int kh = 0; kh < 8; ++kh)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      z[h][kh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[kh], s[h], (f32x4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
  for (int st = 1; st < 8; st <<= 1)
#pragma unroll
    for (int kh = 0; kh < 8; ++kh) {
      if (kh & st) continue;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = z[h][kh][i], b = z[h][kh + st][i];
          z[h][kh][i] = a + b;
          z[h][kh + st][i] = a - b;
        }
    }
}

// Scale rows 4g + i by f[i], round to fp16 and store the block: the word of
// (z[0], z[1]) goes to byte 64 nh + 4c of the block's 512-byte segment of
// strip row 4g + i, so 16 lanes write 64 contiguous bytes of a row.  `base` is
// the block's byte offset in row 0 of the strip; the descriptor ends at row
// m, so rows of a ragged last strip are dropped by its range check.
__device__ __forceinline__ void store_xh_block(const f32x4 (&z)[2][8], const float (&f)[4],
                                               __amdgpu_buffer_rsrc_t rsrc, uint32_t base,
                                               uint32_t row_bytes, int lane) {
  const int c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int nh = 0; nh < 8; ++nh) {
      const _Float16 lo = (_Float16)(z[0][nh][i] * f[i]);
      const _Float16 hi = (_Float16)(z[1][nh][i] * f[i]);
      const uint32_t w = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                         ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      __builtin_amdgcn_raw_buffer_store_b32(
          w, rsrc, base + (uint32_t)(4 * g + i) * row_bytes + (uint32_t)(64 * nh + 4 * c), 0, 0);
    }
}

// Pass 2: grid (ceil(m/16), ceil(nblk/4)); wave w of workgroup (i, j) owns
// rows 16i.. and the 256-column block 4j + w.
__global__ void __launch_bounds__(64 * PRE_WAVES) k_fwd_rotate(
    const uint16_t* __restrict__ x, int64_t m, int64_t k, int rank, int slices,
    const uint32_t* __restrict__ amax_part, const float* __restrict__ t_part,
    uint16_t* __restrict__ xh, uint16_t* __restrict__ thi, uint16_t* __restrict__ tlo,
    float* __restrict__ rowscale) {
  __shared__ u32x4 s_stage[PRE_WAVES][16 * PRE_STAGE_U4];
  __shared__ int s_exp[16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int64_t nblk = k >> 8;
  // E of the workgroup's rows (rows past m repeat the last row)
  if (tid < 16) {
    const int64_t row = min(row0 + tid, m - 1);
    s_exp[tid] = row_exponent(slice_max(amax_part + row, m, slices));
  }
  __syncthreads();

  {
    // t slices in a fixed order, scaled, split into bf16 hi + lo; the 16 x
    // rank outputs of the strip are shared out over its column groups, and
    // each output's slice loads go out eight at a time
    const int outs = 16 * rank;
    const int per = (outs + (int)gridDim.y - 1) / (int)gridDim.y;
    const int i0 = (int)blockIdx.y * per, i1 = min(outs, i0 + per);
    for (int i = i0 + tid; i < i1; i += 64 * PRE_WAVES) {
      const int rr = i / rank, r = i - rr * rank;
      const int64_t row = row0 + rr;
      if (row >= m) continue;
      float t = slice_sum(t_part + row * rank + r, m * rank, slices);
      t *= ldexpf(1.0f, 11 - s_exp[rr]);
      const uint16_t hb = f32_to_bf16(t);
      thi[row * rank + r] = hb;
      tlo[row * rank + r] = f32_to_bf16(t - bf16_to_f32(hb));
    }
    if (blockIdx.y == 0 && tid < 16 && row0 + tid < m)
      rowscale[row0 + tid] = ldexpf(1.0f, s_exp[tid] - 11);
  }
  const int64_t b = (int64_t)blockIdx.y * PRE_WAVES + wave;
  if (b >= nblk) return;

  const int64_t lrow = min(row0 + c, m - 1);
  const float f = ldexpf(1.0f, 11 - s_exp[c]) * 0.0625f;   // exact: a power of two
  uint32_t xb[32];
  load_x64(xb, x + lrow * k + b * 256 + 64 * g);
  float v[64];
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    v[2 * j] = bf16_to_f32(xb[j] & 0xFFFFu);
    v[2 * j + 1] = bf16_to_f32(xb[j] >> 16);
  }
  fwht_inreg64(v);
  fwht_cross64_swap(v);

  // fp16 in the permuted K order: word p of each 8-column run holds columns
  // p and p + 4; the run of registers 8j.. holds columns swap_col(g, 8j)..
  u32x4* stage = &s_stage[wave][0];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const _Float16 lo = (_Float16)(v[8 * j + p] * f);
      const _Float16 hi = (_Float16)(v[8 * j + p + 4] * f);
      o[p] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
             ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    stage[c * PRE_STAGE_U4 + (swap_col(g, 8 * j) >> 3)] = o;
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_wave_barrier();
  // every store instruction writes two whole 512-byte row segments; the
  // descriptor ends at row m, so rows of a ragged last strip are dropped
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(xh + row0 * k), (short)0, (int)(min((int64_t)16, m - row0) * k * 2), 0x00020000);
  const uint32_t off = 2u * ((uint32_t)((lane >> 5) * k) + (uint32_t)(b * 256) + 8u * (lane & 31));
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const u32x4 o = stage[(2 * j + (lane >> 5)) * PRE_STAGE_U4 + (lane & 31)];
    __builtin_amdgcn_raw_buffer_store_b128(o, rsrc, off + (uint32_t)(4 * j) * (uint32_t)k, 0, 0);
  }
}

// Both passes in one launch, for K <= 256 * PREP_WAVES * NB and ranks 0, 16
// and 32: workgroup i owns rows 16i .. 16i+15 over all of K, and wave w the
// 256-column blocks w, w + PREP_WAVES, ... (at most NB of them), whose x it
// loads once, in the statistics pass's layout.  Per block the wave takes the
// row maxima, t on MFMA against its block's staged lora_down rows, and the
// Hadamard transform (fwht256_mfma) before any row scale is known; the
// maxima and the waves' t sums then meet in LDS, and every wave scales,
// rounds and stores its blocks.  At these sizes the two passes would be two
// short launches, each mostly latency.
constexpr int PREP_WAVES = 8;
constexpr int PREP_MAX_NB = 2;

template <int RANK, int NB>
__global__ void __launch_bounds__(64 * PREP_WAVES) k_fwd_prep(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ down, int64_t m, int64_t k,
    uint16_t* __restrict__ xh, uint16_t* __restrict__ thi, uint16_t* __restrict__ tlo,
    float* __restrict__ rowscale) {
  static_assert(RANK == 0 || RANK == 16 || RANK == 32, "staged factor: ranks 16 and 32");
  static_assert(NB >= 1 && NB <= PREP_MAX_NB, "blocks per wave");
  constexpr int RT = RANK / 16;
  constexpr int FAC_BYTES = 256 * RANK * 2;   // one block's lora_down rows
  constexpr int SUM_BYTES = 16 * (RANK > 0 ? RANK : 1) * 4;
  constexpr int WAVE_LDS = FAC_BYTES > SUM_BYTES ? FAC_BYTES : SUM_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t wave_lds[PREP_WAVES][WAVE_LDS];
  __shared__ uint32_t red_max[PREP_WAVES][64];
  __shared__ int s_exp[16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int64_t lrow = min(row0 + c, m - 1);   // rows past m read the last row
  const int nblk = (int)(k >> 8);
  const int nown = wave < nblk ? min(NB, (nblk - wave + PREP_WAVES - 1) / PREP_WAVES) : 0;

  // lora_down rows 256b .. 256b+255 ([k][RANK] as stored, contiguous) into
  // this wave's LDS area with direct loads
  auto stage_factor = [&](int b) {
    if constexpr (RANK > 0) {
      const __amdgpu_buffer_rsrc_t f_rsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(down + (int64_t)b * 256 * RANK), (short)0, FAC_BYTES, 0x00020000);
#pragma unroll
      for (int i = 0; i < FAC_BYTES / 1024; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            f_rsrc, (__attribute__((address_space(3))) void*)(&wave_lds[wave][0] + i * 1024), 16,
            (uint32_t)(lane * 16 + i * 1024), 0, 0, 0);
    }
  };

  // the first block's factor rows, then every owned block of x (eight
  // 16-byte loads per block: columns 32j + 8g .. +7 of row c)
  bf16x8 xf[NB][8];
  if (nown > 0) stage_factor(wave);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    if (nb < nown) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        xf[nb][j] = *reinterpret_cast<const bf16x8*>(
            x + lrow * k + (int64_t)(wave + PREP_WAVES * nb) * 256 + 32 * j + 8 * g);
    }
  __builtin_amdgcn_sched_barrier(0);

  bf16x8 s32[2];
  s32_fragments(s32, lane);
  f32x4 acc[RT > 0 ? RT : 1] = {};
  f32x4 z[NB][2][8];
  u16x2 amax2 = (u16x2){0, 0};
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if (nb >= nown) break;
    if constexpr (RANK > 0) {
      __builtin_amdgcn_sched_barrier(0);
      if (nb == 0) {
        // the staged rows have landed once no more than the x loads issued
        // behind them are outstanding (loads complete in order)
        if (NB > 1 && nown > 1) __builtin_amdgcn_s_waitcnt(sq_wait_vm(16));
        else __builtin_amdgcn_s_waitcnt(sq_wait_vm(8));
      } else {
        // the previous block's fragments have been read out of the area
        // (lgkmcnt 0) before the next block's rows are loaded into it; every
        // x load was issued first, so the rows have landed at vmcnt 0
        __builtin_amdgcn_s_waitcnt(SQ_WAIT_LGKM0);
        __builtin_amdgcn_sched_barrier(0);
        stage_factor(wave + PREP_WAVES * nb);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(SQ_WAIT_VM0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // B element e of fragment (rt, j): lora_down row 32j + 8g + e, column 16rt + c
      const uint16_t* st = reinterpret_cast<const uint16_t*>(&wave_lds[wave][0]);
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          bf16x8 f;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            f[e] = __builtin_bit_cast(__bf16, st[(32 * j + 8 * g + e) * RANK + 16 * rt + c]);
          acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[nb][j], f, acc[rt], 0, 0, 0);
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const u32x4 w = __builtin_bit_cast(u32x4, xf[nb][j]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        amax2 = __builtin_elementwise_max(amax2, __builtin_bit_cast(u16x2, w[e] & 0x7FFF7FFFu));
    }
    fwht256_mfma(xf[nb], s32, z[nb]);
  }

  // acc[rt][i] = this wave's part of t[row0 + 4g + i][16 rt + c]; the sums go
  // to the start of the wave's own area (its fragments have been read)
  __builtin_amdgcn_s_waitcnt(SQ_WAIT_LGKM0);
  __builtin_amdgcn_sched_barrier(0);
  auto sums = [&](int w) { return reinterpret_cast<float(*)[RANK > 0 ? RANK : 1]>(&wave_lds[w][0]); };
  if constexpr (RANK > 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sums(wave)[4 * g + i][16 * rt + c] = acc[rt][i];
  }
  red_max[wave][lane] = max((uint32_t)amax2[0], (uint32_t)amax2[1]);
  __syncthreads();
  if (tid < 16) {
    uint32_t mx = 0;
#pragma unroll
    for (int w = 0; w < PREP_WAVES; ++w)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) mx = max(mx, red_max[w][tid + 16 * gg]);
    s_exp[tid] = row_exponent(mx);
    if (row0 + tid < m) rowscale[row0 + tid] = ldexpf(1.0f, s_exp[tid] - 11);
  }
  __syncthreads();
  if constexpr (RANK > 0) {
    // t summed over the waves in a fixed order, scaled, split into bf16 hi + lo
    for (int i = tid; i < 16 * RANK; i += 64 * PREP_WAVES) {
      const int rr = i / RANK, r = i - rr * RANK;
      const int64_t row = row0 + rr;
      if (row >= m) continue;
      float t = 0.0f;
#pragma unroll
      for (int w = 0; w < PREP_WAVES; ++w) t += sums(w)[rr][r];
      t *= ldexpf(1.0f, 11 - s_exp[rr]);
      const uint16_t hb = f32_to_bf16(t);
      thi[row * RANK + r] = hb;
      tlo[row * RANK + r] = f32_to_bf16(t - bf16_to_f32(hb));
    }
  }

  float f[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = ldexpf(1.0f, 11 - s_exp[4 * g + i]) * 0.0625f;   // exact
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(xh + row0 * k), (short)0, (int)(min((int64_t)16, m - row0) * k * 2), 0x00020000);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if (nb >= nown) break;
    store_xh_block(z[nb], f, rsrc, (uint32_t)((wave + PREP_WAVES * nb) * 512), (uint32_t)(k * 2), lane);
  }
}

// ---------------------------------------------------------------- contraction
// K advances 64 values per pipeline stage (two 16x16x32 MFMA steps).
constexpr int GBK = 64;

// ---------------------------------------------------------------- large-tile contraction
// BM x 256 output tile per workgroup (BM = 256, 224 or 128), eight waves of
// (BM/2) x 64 ((BM/32) x 4 MFMA tiles each, two waves per SIMD).
//
// Data path: everything streams global -> LDS with direct 16-byte buffer
// loads (no register staging) into tiles of 128-byte rows whose 16-byte chunk
// c of row r sits at slot c ^ a_swz(r) (conflict-free fragment reads):
//  * A, the fp16 rotated activations: one stage = 64 K values per row;
//  * B, the packed codes: one super-stage = 4 stages = 256 K values = one full
//    128-byte line per weight row; plus 16 bytes of fp16 scales per row.
// Each wave dequantizes its own B fragments in registers (16 codes = one
// 8-byte LDS read per lane per column tile and stage).  Within a stage, lane
// group g = lane/16 owns K offsets 16g .. 16g+15: offsets 16g+0..7 feed the
// first MFMA step and 16g+8..15 the second, so both operands read the same
// 8-element chunk.
//
// Schedule (per wave): a stage is two half-steps of 32 MFMAs.  While the MFMAs
// of one half-step run, the wave reads the A fragments of the next half-step
// and dequantizes its B fragments, so LDS reads and VALU work hide under the
// MFMAs.  The single barrier of a stage sits between its half-steps: there,
// the loads of the next stage have landed (issued one stage earlier) and the
// buffer of this stage has been read by every wave, so it is refilled with the
// stage after next.  Rows and columns past the matrix edge load a clamped
// (valid) row; their results are never stored.
constexpr int BIG_BM = 256, BIG_BN = 256, BIG_THREADS = 512;
constexpr int BIG_TILE_BYTES = BIG_BM * 128;   // one A stage or one B super-stage: 32 KB
constexpr int BIG_S_BYTES = (BIG_BN + 64) * 16;  // scales of one super-stage, 16 B per row (+ tail)

// The pipeline buffers are separate LDS objects so that the compiler can tell
// a direct load into one buffer from a fragment read of another.
__shared__ __attribute__((aligned(16))) uint8_t big_a0[BIG_TILE_BYTES];
__shared__ __attribute__((aligned(16))) uint8_t big_a1[BIG_TILE_BYTES];
__shared__ __attribute__((aligned(16))) uint8_t big_b0[BIG_TILE_BYTES];
__shared__ __attribute__((aligned(16))) uint8_t big_b1[BIG_TILE_BYTES];
__shared__ __attribute__((aligned(16))) uint8_t big_s0[BIG_S_BYTES];
__shared__ __attribute__((aligned(16))) uint8_t big_s1[BIG_S_BYTES];

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt immediates (gfx9 encoding: vmcnt in [3:0], expcnt [6:4], lgkmcnt [11:8])
constexpr int WAIT_VM0 = 0x0F70, WAIT_LGKM0 = 0xC07F;

// BM: tile rows, 256, 224 or 128 (the LDS A tile always has 256 rows; loader
// rows past BM fetch nothing).  Split-K: workgroup
// (tile, z) covers stages [z kts, (z+1) kts) (kts a multiple of 4, so every
// split starts on a super-stage) by shifting the three buffer bases; with
// more than one split the fp32 partial sums, without the row scale, go to
// `partial` [splits][m][n] for k_fwd_reduce, and split 0 adds the rank-r
// branch.  plan_fwd picks BM and the split count.  SPLIT = false compiles
// the single-split kernel without any of the split bookkeeping.
//
// GSHIFT = 0 selects the int8-residual payload (SquareQ README, "v3.1 -
// int8-residual mode"): one stage of B is 64 bytes per weight row, so a
// super-stage is two stages (128 K values, the same 128-byte LDS rows) and
// arrives half a super-stage (128 rows, two loads per wave) per stage; a
// lane reads one 16-byte chunk per column tile and stage and dequantizes it
// into the two half-steps' fragments with dequant8_i8.  No scales stream
// with the codes: the row scale multiplies the fp32 sums before the rank-r
// branch is added.
template <int GSHIFT, int BM, bool SPLIT>   // log2 of the group size (0: int8), tile rows, split-K
__global__ void __launch_bounds__(BIG_THREADS, 1) k_fwd_gemm_big(
    const uint16_t* __restrict__ xh, const uint8_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ thi,
    const uint16_t* __restrict__ tlo, const uint16_t* __restrict__ up,
    const float* __restrict__ rowscale, void* __restrict__ y, float* __restrict__ partial,
    int64_t m, int64_t n, int64_t k, int rank, int y_bf16, int kts) {
  static_assert(BM == 256 || BM == 224 || BM == 128, "tile rows");
  constexpr bool W8 = GSHIFT == 0;
  constexpr int FN = 4;           // wave tile (BM/2) x 64
  constexpr int FM = BM / 32;     // 16-row MFMA tiles per wave
  constexpr int WROWS = BM / 2;   // rows per wave
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int64_t mt = (m + BM - 1) / BM, nt = (n + BIG_BN - 1) / BIG_BN;
  int64_t tile_m, tile_n;
  xcd_tile(blockIdx.x, mt * nt, nt, tile_m, tile_n);
  const int64_t m0 = tile_m * BM, n0 = tile_n * BIG_BN;
  const int z = SPLIT ? (int)blockIdx.y : 0;
  const int64_t kt0 = SPLIT ? (int64_t)z * kts : 0;   // first stage of this split
  const int64_t KT = SPLIT ? (int64_t)kts : k / GBK;
  const int64_t NSS = W8 ? KT >> 1 : KT >> 2;   // kts is a multiple of 4
  const int64_t half_k = k >> 1, ngroups = W8 ? 1 : k >> GSHIFT;
  const int64_t cpr = W8 ? k : half_k;          // code bytes per weight row
  constexpr int CPS = W8 ? GBK : GBK / 2;       // code bytes per row and stage

  const int fr = lane & 15, g = lane >> 4;

  // ---- loaders: wave w fills rows 32w .. 32w+31 of each tile, eight rows
  // (8 lanes x 16 bytes) per instruction
  const int64_t a_rows = min((int64_t)BM, m - m0);
  const int64_t b_rows = min((int64_t)BIG_BN, n - n0);
  // bases at this split's first K value (64 kt0 values: 128 bytes of xh,
  // 32 bytes of codes, 64 kt0 / group scales per row)
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(xh + m0 * k + kt0 * GBK), (short)0, (int)(a_rows * k * 2 - kt0 * GBK * 2),
      0x00020000);
  const __amdgpu_buffer_rsrc_t c_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(codes + n0 * cpr + kt0 * CPS), (short)0, (int)(b_rows * cpr - kt0 * CPS),
      0x00020000);
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(scales + n0 * ngroups + ((kt0 * GBK) >> GSHIFT)), (short)0,
      (int)(b_rows * ngroups * 2 - ((kt0 * GBK) >> GSHIFT) * 2), 0x00020000);
  uint32_t a_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 32 * wave + 8 * i + (lane >> 3);
    // loader rows at or past BM are never read: an offset past the
    // descriptor's range makes their loads fetch nothing (no branch)
    a_off[i] = r < BM ? (uint32_t)(min((int64_t)r, a_rows - 1) * k * 2) + 16 * ((lane & 7) ^ a_swz(r))
                      : 0x80000000u;
  }

  auto a_issue = [&](int64_t kt, uint8_t* buf) {
    uint8_t* base = buf + wave * 4096;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_ptr_t)(base + i * 1024), 16,
                                               a_off[i], (int)(kt * GBK * 2), 0, 0);
  };
  // B arrives a quarter super-stage per stage: quarter qq (rows 64 qq .. +64 of
  // the tile, eight per wave) of super-stage ss, plus those rows' scales
  // (lanes 0..7 of each wave; one instruction per wave either way).
  // (per-quarter offsets are recomputed when issued: a few VALU per stage
  // instead of eight live registers; a_swz(r + 64 qq) = a_swz(r))
  const int cq_slot = 16 * ((lane & 7) ^ a_swz(8 * wave + (lane >> 3)));
  const int b_last = (int)b_rows - 1;
  auto bq_issue = [&](int64_t ss, int qq, uint8_t* bbuf, uint8_t* sbuf) {
    const int r = 64 * qq + 8 * wave + (lane >> 3);
    const int sr = 64 * qq + 8 * wave + lane;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        c_rsrc, (lds_ptr_t)(bbuf + (64 * qq + 8 * wave) * 128), 16,
        (uint32_t)min(r, b_last) * (uint32_t)half_k + cq_slot, (int)(ss * 128), 0, 0);
    // scales: lane l writes row 64 qq + 8 wave + l (row r at r * 16); rows
    // beyond this wave's eight get the same bytes another wave writes for
    // them within the same refill window, and rows past 255 land in the
    // buffer's spare tail
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        s_rsrc, (lds_ptr_t)(sbuf + (64 * qq + 8 * wave) * 16), 16,
        (uint32_t)min(sr, b_last) * (uint32_t)(ngroups * 2), (int)(((ss * 256) >> GSHIFT) * 2), 0,
        0);
  };
  auto b_issue = [&](int64_t ss, uint8_t* bbuf, uint8_t* sbuf) {
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) bq_issue(ss, qq, bbuf, sbuf);
  };
  // int8 codes: half hh (rows 128 hh .. +128, sixteen per wave) of super-stage ss
  auto bh_issue = [&](int64_t ss, int hh, uint8_t* bbuf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 128 * hh + 16 * wave + 8 * i + (lane >> 3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          c_rsrc, (lds_ptr_t)(bbuf + (128 * hh + 16 * wave + 8 * i) * 128), 16,
          (uint32_t)min(r, b_last) * (uint32_t)cpr + 16 * ((lane & 7) ^ a_swz(8 * i + (lane >> 3))),
          (int)(ss * 128), 0, 0);
    }
  };

  // Fragment addresses: for rows r = (WROWS wm | 64 wn) + fr + 16 i the
  // swizzle equals a_swz(fr) (WROWS and 16 are multiples of 16), so row
  // steps are immediate offsets.
  const int swa = a_swz(fr);
  uint32_t a_lane[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) a_lane[ks] = (WROWS * wm + fr) * 128 + 16 * ((2 * g + ks) ^ swa);
  const int b_row0 = 64 * wn + fr;
  // scales of row r live at r * 16
  const uint32_t s_lane = b_row0 * 16 + 2 * ((16 * g) >> GSHIFT);

  auto read_a = [&](half8 (&af)[FM], const uint8_t* abase, int ks) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
      af[i] = *reinterpret_cast<const half8*>(abase + a_lane[ks] + i * 2048);
  };
  // B words (both half-steps) and scales of stage s of a super-stage
  auto read_b = [&](u32x2 (&bw)[FN], _Float16 (&bs)[FN], const uint8_t* bbase,
                    const uint8_t* sbase, int s) {
    const uint32_t bl = b_row0 * 128 + 16 * ((2 * s + (g >> 1)) ^ swa) + 8 * (g & 1);
    const uint32_t sl = s_lane + 2 * ((64 * s) >> GSHIFT);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      bw[j] = *reinterpret_cast<const u32x2*>(bbase + bl + j * 2048);
      bs[j] = *reinterpret_cast<const _Float16*>(sbase + sl + j * 256);
    }
  };
  // int8: the lane's 16-byte chunk 4s + g (K offsets 16g .. 16g+15 of stage s)
  auto read_b8 = [&](u32x4 (&bw)[FN], const uint8_t* bbase, int s) {
    const uint32_t bl = b_row0 * 128 + 16 * ((4 * s + g) ^ swa);
#pragma unroll
    for (int j = 0; j < FN; ++j) bw[j] = *reinterpret_cast<const u32x4*>(bbase + bl + j * 2048);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  auto mfma_step = [&](const half8 (&af)[FM], const half8 (&bj)[FN]) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int i = 0; i < FM; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bj[j], acc[i][j], 0, 0, 0);
  };
  auto sync = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(WAIT_VM0);
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue: stages 0 and 1 of A, super-stage 0 and the first quarter of
  // super-stage 1 of B (the loop issues the rest)
  a_issue(0, big_a0);
  a_issue(min((int64_t)1, KT - 1), big_a1);
  if constexpr (W8) {
    bh_issue(0, 0, big_b0);
    bh_issue(0, 1, big_b0);
    bh_issue(min((int64_t)1, NSS - 1), 0, big_b1);
  } else {
    b_issue(0, big_b0, big_s0);
    bq_issue(min((int64_t)1, NSS - 1), 0, big_b1, big_s1);
  }
  sync();
  half8 af0[FM], af1[FM], bj0[FN], bj1[FN];
  uint32_t bw1[FN];
  _Float16 bsc[FN];
  u32x2 bw81[FN];   // int8: the second half-step's two words
  read_a(af0, big_a0, 0);
  if constexpr (W8) {
    u32x4 bw[FN];
    read_b8(bw, big_b0, 0);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      bj0[j] = dequant8_i8(bw[j][0], bw[j][1]);
      bw81[j] = (u32x2){bw[j][2], bw[j][3]};
    }
  } else {
    u32x2 bw[FN];
    read_b(bw, bsc, big_b0, big_s0, 0);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      bj0[j] = dequant8_f16(bw[j][0], bsc[j]);
      bw1[j] = bw[j][1];
    }
  }

  // Instruction interleave (sched_group_barrier masks: 0x008 MFMA, 0x100 LDS
  // read, 0x002 VALU, 0x020 VMEM read): every MFMA is followed by a share of
  // the LDS reads and of the dequantization, so that they issue while the
  // matrix core works instead of in separate phases.
#define SQ_GROUP(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)
#pragma unroll 1
  for (int64_t kt = 0; kt < KT; ++kt) {
    const bool aodd = kt & 1;
    const uint8_t* acur = aodd ? big_a1 : big_a0;
    // half-step 0: MFMAs of (kt, 0); read A of (kt, 1); dequantize B of (kt, 1)
    read_a(af1, acur, 1);
    mfma_step(af0, bj0);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      bj1[j] = W8 ? dequant8_i8(bw81[j][0], bw81[j][1]) : dequant8_f16(bw1[j], bsc[j]);
#pragma unroll
    for (int t = 0; t < FM; ++t) {
      SQ_GROUP(0x008, 1);
      SQ_GROUP(0x100, 1);
      SQ_GROUP(0x008, 1);
      SQ_GROUP(0x002, 4);
      SQ_GROUP(0x008, 1);
      SQ_GROUP(0x002, 4);
      SQ_GROUP(0x008, 1);
    }
    // barrier: stage kt+1 has landed everywhere, buffer of stage kt is free
    sync();
    {
      const int64_t kn = min(kt + 1, KT - 1);
      // refill: A of stage kt+2 into this stage's buffer; quarter (kt+5) % 4 of
      // super-stage (kt+5) / 4 of B (a super-stage ss is complete by the
      // barrier of stage 4 ss - 1, whose second half-step reads it first);
      // int8: half (kt+3) % 2 of super-stage (kt+3) / 2 (complete by the
      // barrier of stage 2 ss - 1)
      a_issue(min(kt + 2, KT - 1), aodd ? big_a1 : big_a0);
      if constexpr (W8) {
        const int64_t ssn = kn >> 1;
        const int64_t ss = (kt + 3) >> 1;
        u32x4 bw[FN];
        bh_issue(min(ss, NSS - 1), (int)((kt + 3) & 1), (ss & 1) ? big_b1 : big_b0);
        // half-step 1: MFMAs of (kt, 1); read A and B of stage kt+1; dequantize (kt+1, 0)
        read_b8(bw, (ssn & 1) ? big_b1 : big_b0, (int)(kn & 1));
        read_a(af0, aodd ? big_a0 : big_a1, 0);
        mfma_step(af1, bj1);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          bj0[j] = dequant8_i8(bw[j][0], bw[j][1]);
          bw81[j] = (u32x2){bw[j][2], bw[j][3]};
        }
      } else {
        const int64_t ssn = kn >> 2;
        const int64_t ss = (kt + 5) >> 2;
        u32x2 bw[FN];
        bq_issue(min(ss, NSS - 1), (int)((kt + 5) & 3), (ss & 1) ? big_b1 : big_b0,
                 (ss & 1) ? big_s1 : big_s0);
        // half-step 1: MFMAs of (kt, 1); read A and B of stage kt+1; dequantize (kt+1, 0)
        read_b(bw, bsc, (ssn & 1) ? big_b1 : big_b0, (ssn & 1) ? big_s1 : big_s0, (int)(kn & 3));
        read_a(af0, aodd ? big_a0 : big_a1, 0);
        mfma_step(af1, bj1);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          bj0[j] = dequant8_f16(bw[j][0], bsc[j]);
          bw1[j] = bw[j][1];
        }
      }
      SQ_GROUP(0x020, 6);
      SQ_GROUP(0x100, W8 ? 4 : 8);
#pragma unroll
      for (int t = 0; t < FM; ++t) {
        SQ_GROUP(0x008, 1);
        SQ_GROUP(0x100, 1);
        SQ_GROUP(0x008, 1);
      }
#pragma unroll
      for (int t = 0; t < FM; ++t) {
        SQ_GROUP(0x008, 1);
        SQ_GROUP(0x002, 4);
        SQ_GROUP(0x008, 1);
        SQ_GROUP(0x002, 4);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#undef SQ_GROUP

  const int64_t rbase = m0 + WROWS * wm, cbase = n0 + 64 * wn;
  if constexpr (W8) {
    // the row scale of output column c multiplies the code sums
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const float sc = fp16_bits_to_f32(scales[min(cbase + 16 * j + fr, n - 1)]);
#pragma unroll
      for (int i = 0; i < FM; ++i) acc[i][j] *= sc;
    }
  }
  // rank-r branch: (t_hi + t_lo) @ up^T on bf16 MFMA into the same accumulators
  // (rank 16: the upper half of the 32-wide step reads zeros)
  for (int rr = 0; rr < (z == 0 ? rank : 0); rr += 32) {   // (z is 0 unless SPLIT)
    const bool rk = rr + 8 * g < rank;
#pragma unroll
    for (int hl = 0; hl < 2; ++hl) {
      const uint16_t* tsrc = hl ? tlo : thi;
      bf16x8 af[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int64_t r = min(rbase + 16 * i + fr, m - 1);
        af[i] = rk ? *reinterpret_cast<const bf16x8*>(tsrc + r * rank + rr + 8 * g) : (bf16x8){};
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t c = min(cbase + 16 * j + fr, n - 1);
        const bf16x8 bj =
            rk ? *reinterpret_cast<const bf16x8*>(up + c * rank + rr + 8 * g) : (bf16x8){};
#pragma unroll
        for (int i = 0; i < FM; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bj, acc[i][j], 0, 0, 0);
      }
    }
  }

  const int lr4 = 4 * g;
  if constexpr (SPLIT) {
    // split-K partial sums (no row scale): k_fwd_reduce finishes them
    float* pz = partial + (int64_t)z * m * n;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t r = rbase + 16 * i + lr4 + v;
        if (r >= m) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int64_t c = cbase + 16 * j + fr;
          if (c < n) pz[r * n + c] = acc[i][j][v];
        }
      }
    }
    return;
  }
  if (y_bf16) {
    // Each wave stages its WROWS x 64 bf16 sub-tile (at most 16 KB, 128-byte
    // rows with the chunk swizzle) in half of a pipeline buffer, then stores
    // eight whole 128-byte row segments per instruction.
    __builtin_amdgcn_s_waitcnt(WAIT_VM0);   // the final (unused) prefetches have landed
    __syncthreads();                        // every wave is done with the pipeline buffers
    const int wb = wave >> 1;
    uint8_t* st = (wb == 0 ? big_a0 : wb == 1 ? big_a1 : wb == 2 ? big_b0 : big_b1) +
                  (wave & 1) * 16384;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int lrow = 16 * i + lr4 + v;
        const float rs = rowscale[min(rbase + lrow, m - 1)];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = 16 * j + fr;   // chunk col/8, element col%8
          *reinterpret_cast<uint16_t*>(st + lrow * 128 + 16 * ((col >> 3) ^ a_swz(lrow)) +
                                       2 * (col & 7)) = f32_to_bf16(acc[i][j][v] * rs);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
    __builtin_amdgcn_wave_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const bool full_cols = (cbase + 64 <= n) && ((n & 7) == 0);
#pragma unroll
    for (int it = 0; it < WROWS / 8; ++it) {
      const int lrow = 8 * it + (lane >> 3), chunk = lane & 7;
      const int64_t r = rbase + lrow, c = cbase + 8 * chunk;
      const u32x4 o = *reinterpret_cast<const u32x4*>(st + lrow * 128 + 16 * (chunk ^ a_swz(lrow)));
      if (r >= m) continue;
      uint16_t* dst = reinterpret_cast<uint16_t*>(y) + r * n + c;
      if (full_cols) {
        *reinterpret_cast<u32x4*>(dst) = o;
      } else {
        const uint16_t* h = reinterpret_cast<const uint16_t*>(&o);
        for (int e = 0; e < 8 && c + e < n; ++e) dst[e] = h[e];
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t r = rbase + 16 * i + lr4 + v;
      if (r >= m) continue;
      const float rs = rowscale[r];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t c = cbase + 16 * j + fr;
        if (c < n) reinterpret_cast<float*>(y)[r * n + c] = acc[i][j][v] * rs;
      }
    }
  }
}

// ---------------------------------------------------------------- small M
// For M <= 64 the contraction is a stream of the payload past a few rows of
// activations.  One wave owns 64 weight rows and one K slice: per 128 K
// values it loads 16 bytes of codes per lane and weight-row tile (the
// next chunk's codes are in flight while this one computes), dequantizes them
// once into MFMA B fragments and reuses those for every 16-row tile of x.
// MFMA step e of a chunk contracts K offsets 32g + 8e .. +7 in lane group g,
// so one lane's 16 code bytes and 64 activation bytes are contiguous; both
// operands keep the permuted order inside each group of 8.  Rows of xh past
// M and weight rows past N come back as zeros from range-checked buffer
// loads.  Split-K partials go to the workspace (fixed-order sum in
// k_fwd_reduce); split 0 also adds the rank-r branch.
//
// GSHIFT = 0 selects the int8-residual payload: 32 bytes of codes per lane,
// weight-row tile and chunk (MFMA step e reads bytes 8e .. 8e+7), no group
// scales, and the row scale applied to the fp32 sums before the rank-r
// branch is added.
constexpr int SK_ROWS = 64;

template <int GSHIFT, int MT>
__global__ void __launch_bounds__(64) k_fwd_skinny(
    const uint16_t* __restrict__ xh, const uint8_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ thi,
    const uint16_t* __restrict__ tlo, const uint16_t* __restrict__ up,
    float* __restrict__ partial, int64_t m, int64_t n, int64_t k, int rank, int kslice) {
  constexpr bool W8 = GSHIFT == 0;
  constexpr int CW = W8 ? 2 : 1;   // 16-byte code loads per weight-row tile and chunk
  const int lane = threadIdx.x, fr = lane & 15, g = lane >> 4;
  // K slice fastest: neighbouring workgroups sweep whole weight rows
  const int64_t n0 = (int64_t)blockIdx.y * SK_ROWS;
  const int ks = blockIdx.x;
  const int64_t k0 = (int64_t)ks * kslice, k1 = min(k, k0 + kslice);
  const int64_t ngroups = W8 ? 1 : k >> GSHIFT;
  const int64_t cpr = W8 ? k : k >> 1;   // code bytes per weight row
  const int64_t b_rows = min((int64_t)SK_ROWS, n - n0);
  const __amdgpu_buffer_rsrc_t c_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(codes + n0 * cpr), (short)0, (int)(b_rows * cpr), 0x00020000);
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(scales + n0 * ngroups), (short)0, (int)(b_rows * ngroups * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t x_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)xh, (short)0, (int)(m * k * 2), 0x00020000);
  // byte offsets at K offset 0
  uint32_t c_off[4], s_off[4], a_off[MT];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    c_off[t] = (uint32_t)((16 * t + fr) * cpr) + (uint32_t)(16 * CW) * g;
    s_off[t] = (uint32_t)((16 * t + fr) * ngroups) * 2u;
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) a_off[mt] = (uint32_t)((16 * mt + fr) * k + 32 * g) * 2u;

  // kb < 0 asks for nothing: the offsets land past the descriptors' range,
  // so the loads return zeros without touching memory (no branch, so the
  // compiler's wait counting stays exact)
  auto load_codes = [&](u32x4 (&cw)[4 * CW], uint32_t (&sc)[4], int64_t kb) {
    const uint32_t off = kb < 0 ? 0x80000000u : 0u;
    kb = kb < 0 ? 0 : kb;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (W8) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          cw[2 * t + h] = __builtin_amdgcn_raw_buffer_load_b128(
              c_rsrc, off + c_off[t] + (uint32_t)kb + 16u * h, 0, 0);
        sc[t] = 0;
      } else {
        cw[t] = __builtin_amdgcn_raw_buffer_load_b128(c_rsrc, off + c_off[t] + (uint32_t)(kb >> 1),
                                                      0, 0);
        sc[t] = __builtin_amdgcn_raw_buffer_load_b16(
            s_rsrc, off + s_off[t] + (uint32_t)(((kb + 32 * g) >> GSHIFT) * 2), 0, 0);
      }
    }
  };

  f32x4 acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[mt][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // One chunk: activations first, then the codes of the chunk after next
  // into the registers the previous chunk used (loads complete in order, so
  // waiting for the activations leaves that prefetch in flight); two
  // register sets alternate, so no copy forces an early wait.
  auto chunk = [&](const u32x4 (&cw)[4 * CW], const uint32_t (&sc)[4], u32x4 (&cn)[4 * CW],
                   uint32_t (&sn)[4], int64_t kb, int64_t kpre) {
    half8 af[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        af[mt][e] = __builtin_bit_cast(
            half8, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, a_off[mt] + (uint32_t)((kb + 8 * e) * 2),
                                                         0, 0));
    half8 bf[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)sc[t]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        bf[t][e] = W8 ? dequant8_i8(cw[CW * t + (e >> 1)][2 * (e & 1)],
                                    cw[CW * t + (e >> 1)][2 * (e & 1) + 1])
                      : dequant8_f16(cw[CW * t][e], sv);
    }
    load_codes(cn, sn, kpre);
    __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the MFMAs
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mt][e], bf[t][e], acc[mt][t], 0, 0, 0);
  };
  // the slice is a whole number of 256-value pairs of chunks
  u32x4 cw0[4 * CW], cw1[4 * CW];
  uint32_t sc0[4], sc1[4];
  load_codes(cw0, sc0, k0);
  __builtin_amdgcn_sched_barrier(0);   // chunk 0's codes are issued first
  load_codes(cw1, sc1, k0 + 128);
  for (int64_t kb = k0; kb < k1; kb += 256) {
    const bool more = kb + 256 < k1;
    chunk(cw0, sc0, cw0, sc0, kb, more ? kb + 256 : -1);
    chunk(cw1, sc1, cw1, sc1, kb + 128, more ? kb + 384 : -1);
  }

  if constexpr (W8) {
    // the row scale of output column c multiplies the code sums
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float sc = fp16_bits_to_f32(scales[min(n0 + 16 * t + fr, n - 1)]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt][t] *= sc;
    }
  }
  if (ks == 0) {
    // rank-r branch: (t_hi + t_lo) @ up^T on bf16 MFMA (rank 16: the upper
    // half of the 32-wide step reads zeros)
    for (int rr = 0; rr < rank; rr += 32) {
      const bool rk = rr + 8 * g < rank;
#pragma unroll
      for (int hl = 0; hl < 2; ++hl) {
        const uint16_t* tsrc = hl ? tlo : thi;
        bf16x8 bu[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int64_t c = min(n0 + 16 * t + fr, n - 1);
          bu[t] = rk ? *reinterpret_cast<const bf16x8*>(up + c * rank + rr + 8 * g) : (bf16x8){};
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int64_t r = min((int64_t)(16 * mt + fr), m - 1);
          const bf16x8 at =
              rk ? *reinterpret_cast<const bf16x8*>(tsrc + r * rank + rr + 8 * g) : (bf16x8){};
#pragma unroll
          for (int t = 0; t < 4; ++t)
            acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(at, bu[t], acc[mt][t], 0, 0, 0);
        }
      }
    }
  }
  // acc[mt][t][i]: row 16 mt + 4g + i, column n0 + 16 t + fr
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = 16 * mt + 4 * g + i;
      if (r >= m) continue;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int64_t c = n0 + 16 * t + fr;
        if (c < n) partial[((int64_t)ks * m + r) * n + c] = acc[mt][t][i];
      }
    }
}

// ---------------------------------------------------------------- split-K sum
__global__ void __launch_bounds__(256) k_fwd_reduce(const float* __restrict__ partial,
                                                     const float* __restrict__ rowscale,
                                                     void* __restrict__ y, int64_t m, int64_t n,
                                                     int splits, int y_bf16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= m * n) return;
  // fixed summation order; the loads of a group of eight are all in flight
  float s = 0.0f;
  const int64_t mn = m * n;
  int z = 0;
  for (; z + 8 <= splits; z += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = partial[(int64_t)(z + u) * mn + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; z < splits; ++z) s += partial[(int64_t)z * mn + i];
  s *= rowscale[i / n];
  if (y_bf16)
    reinterpret_cast<uint16_t*>(y)[i] = f32_to_bf16(s);
  else
    reinterpret_cast<float*>(y)[i] = s;
}

// ---------------------------------------------------------------- host side
static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Tile choice: M <= 64 the small-M kernel; else the 256-column-tile kernel
// with the tile height and split-K factor of least estimated time.
FwdPlan plan_fwd(int64_t m, int64_t n, int64_t k, int group, int rank) {
  FwdPlan p{};
  p.m = m; p.n = n; p.k = k; p.group = group; p.rank = rank;
  const int64_t KT = k / GBK;
  p.skinny_mt = 0;
  if (m <= 64) {
    // small M: 16-row tiles rounded up to 1, 2 or 4; split K into slices
    // for about a thousand waves (long slices stream best: each wave keeps
    // one 256-value step of codes in flight) while the fp32 partials stay
    // under ~15 % of the payload bytes
    p.skinny_mt = m <= 16 ? 1 : m <= 32 ? 2 : 4;
    const int64_t ntiles = (n + SK_ROWS - 1) / SK_ROWS;
    const double pay = group ? (double)n * k * (0.5 + 2.0 / group) : (double)n * k;
    int64_t s = (1024 + ntiles - 1) / ntiles;
    s = std::min<int64_t>(s, std::max<int64_t>(1, (int64_t)(0.15 * pay / (4.0 * m * n))));
    s = std::max<int64_t>(1, s);
    const int64_t chunks = k / 256;
    s = std::min<int64_t>(s, chunks);
    const int64_t per = (chunks + s - 1) / s;
    p.skinny_kslice = (int)(per * 256);
    p.splits = (int)((chunks + per - 1) / per);
    p.tile_m = 16 * p.skinny_mt; p.tile_n = SK_ROWS;
  } else {
    // The 256-column-tile kernel with tile height BM in {256, 224, 128} and
    // s K splits (whole super-stages each).  Estimated time: rounds of the
    // 256 CUs (one tile each) times the stages per split times the time of
    // one 64-deep stage of a BM-row tile, 0.71 + 0.00273 BM us (a fit to
    // M = 96 .. 2048 on a 6144 x 16384 weight: a 128-row tile costs three
    // quarters of a 256-row one, not half), 10 % more with the chip full;
    // plus writing and re-reading the fp32 partials (~3.3 TB/s) and the
    // reduce launch when s > 1.
    const int64_t nt_big = (n + BIG_BN - 1) / BIG_BN;
    double best = -1.0;
    for (int bm : {256, 224, 128}) {
      const int64_t tiles = ((m + bm - 1) / bm) * nt_big;
      for (int64_t sp = 1; sp <= 16; sp *= 2) {
        if ((KT / 4) % sp) continue;   // every split a whole number of super-stages
        const int64_t wgs = tiles * sp, rounds = (wgs + 255) / 256;
        double t = rounds * (double)(KT / sp) * (0.71e-6 + 2.73e-9 * bm) *
                   (1.0 + 0.1 * (double)std::min<int64_t>(wgs, 256) / 256.0);
        if (sp > 1) t += 1.5 * 8.0 * sp * (double)m * n / 5e12 + 10e-6;
        if (best < 0.0 || t < best - 1e-9) { best = t; p.tile_m = bm; p.splits = (int)sp; }
      }
    }
    p.tile_n = BIG_BN;
  }
  size_t off = 0;
  p.off_xh = off;        off = align256(off + (size_t)m * k * 2);
  p.off_thi = off;       off = align256(off + (size_t)m * std::max(rank, 1) * 2);
  p.off_tlo = off;       off = align256(off + (size_t)m * std::max(rank, 1) * 2);
  p.off_rowscale = off;  off = align256(off + (size_t)m * 4);
  p.off_downT = off;     off = align256(off + (size_t)k * std::max(rank, 1) * 2);
  // statistics pass: one 256-column block per wave, K slices of four blocks
  p.pre_bps = PRE_WAVES;
  row_stats_plan(m, k, &p.pre_tiles, &p.pre_slices);
  // one launch for both passes while a strip's blocks fit in the registers
  // of one workgroup, and the rank's factor rows in its LDS
  p.pre_fused = 0;
  if ((rank == 0 || rank == 16 || rank == 32) && k / 256 <= PREP_WAVES * PREP_MAX_NB)
    p.pre_fused = k / 256 <= PREP_WAVES ? 1 : 2;
  p.off_amax = off;      off = align256(off + (size_t)p.pre_slices * m * 4);
  p.off_tpart = off;     off = align256(off + (size_t)p.pre_slices * m * std::max(rank, 1) * 4);
  const bool partials = p.splits > 1 || p.skinny_mt > 0;
  p.off_partial = off;   off = align256(off + (partials ? (size_t)p.splits * m * n * 4 : 0));
  p.total = off;
  return p;
}

struct FwdBuffers {
  uint16_t *xh, *thi, *tlo, *downT;
  float *rowscale, *partial;
  uint32_t* amax;
  float* tpart;
};

static FwdBuffers carve(const FwdPlan& p, void* workspace) {
  char* ws = static_cast<char*>(workspace);
  return FwdBuffers{reinterpret_cast<uint16_t*>(ws + p.off_xh),
                    reinterpret_cast<uint16_t*>(ws + p.off_thi),
                    reinterpret_cast<uint16_t*>(ws + p.off_tlo),
                    reinterpret_cast<uint16_t*>(ws + p.off_downT),
                    reinterpret_cast<float*>(ws + p.off_rowscale),
                    reinterpret_cast<float*>(ws + p.off_partial),
                    reinterpret_cast<uint32_t*>(ws + p.off_amax),
                    reinterpret_cast<float*>(ws + p.off_tpart)};
}

// Row tiles per statistics workgroup: the most that still fill the chip in
// one resident round (256 to 512 workgroups: at rank 32 a workgroup's staged
// factor rows take 66 KB of LDS, so two fit per CU), else two.  With more
// workgroups than resident slots, long-running many-tile workgroups leave a
// near-empty second round (4480 x 16384: 560 workgroups of eight tiles
// measured 6 us slower than 2240 of two).
void row_stats_plan(int64_t m, int64_t k, int* tiles, int* slices) {
  const int64_t strips = (m + 15) / 16, nblk = k / 256;
  *slices = (int)((nblk + PRE_WAVES - 1) / PRE_WAVES);
  *tiles = 1;
  for (int t : {8, 4, 2}) {
    const int64_t wgs = ((strips + t - 1) / t) * *slices;
    if (wgs >= 256 && (wgs <= 512 || t == 2)) { *tiles = t; break; }
  }
}

hipError_t launch_row_stats(const uint16_t* a, const uint16_t* fac, bool kmajor, int64_t m,
                            int64_t k, int rank, int tiles, int slices, uint32_t* amax_part,
                            float* t_part, hipStream_t stream) {
  const dim3 sgrid((unsigned)((m + 16 * tiles - 1) / (16 * tiles)), (unsigned)slices);
#define SQ_STATS(R, T, KM)                                                                      \
  hipLaunchKernelGGL((k_fwd_stats<R, T, KM>), sgrid, dim3(64 * PRE_WAVES), 0, stream, a, fac, m, \
                     k, PRE_WAVES, amax_part, t_part)
#define SQ_STATS_T(R, KM)                                                                 \
  if (tiles == 8) SQ_STATS(R, 8, KM); else if (tiles == 4) SQ_STATS(R, 4, KM);            \
  else if (tiles == 2) SQ_STATS(R, 2, KM); else SQ_STATS(R, 1, KM)
  if (rank == 0) { SQ_STATS_T(0, false); }
  else if (rank == 16) { if (kmajor) { SQ_STATS_T(16, true); } else { SQ_STATS_T(16, false); } }
  else if (rank == 32) { if (kmajor) { SQ_STATS_T(32, true); } else { SQ_STATS_T(32, false); } }
  else { SQ_STATS_T(64, false); }
#undef SQ_STATS_T
#undef SQ_STATS
  return hipGetLastError();
}

hipError_t launch_fwd_rotate(const FwdPlan& p, const uint16_t* x, const uint16_t* down,
                             void* workspace, hipStream_t stream) {
  const FwdBuffers b = carve(p, workspace);
  hipError_t err;
  if (p.pre_fused) {
    const dim3 grid((unsigned)((p.m + 15) / 16));
#define SQ_PREP(R, NB)                                                                           \
  hipLaunchKernelGGL((k_fwd_prep<R, NB>), grid, dim3(64 * PREP_WAVES), 0, stream, x, down, p.m, \
                     p.k, b.xh, b.thi, b.tlo, b.rowscale)
#define SQ_PREP_NB(R) if (p.pre_fused == 1) SQ_PREP(R, 1); else SQ_PREP(R, 2)
    if (p.rank == 0) { SQ_PREP_NB(0); }
    else if (p.rank == 16) { SQ_PREP_NB(16); }
    else { SQ_PREP_NB(32); }
#undef SQ_PREP_NB
#undef SQ_PREP
    return hipGetLastError();
  }
  // ranks 16 and 32: the statistics pass reads lora_down as stored; rank 64
  // (whose staged rows would not fit beside the sums) reads a transposed copy
  const bool kmajor = p.rank > 0 && p.rank <= 32;
  if (p.rank > 0 && !kmajor) {
    const int64_t cnt = p.k * p.rank;
    hipLaunchKernelGGL(k_transpose_down, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, stream,
                       down, b.downT, p.k, p.rank);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const unsigned strips = (unsigned)((p.m + 15) / 16);
  if ((err = launch_row_stats(x, kmajor ? down : b.downT, kmajor, p.m, p.k, p.rank, p.pre_tiles,
                              p.pre_slices, b.amax, b.tpart, stream)) != hipSuccess)
    return err;
  hipLaunchKernelGGL(k_fwd_rotate, dim3(strips, (unsigned)((p.k / 256 + PRE_WAVES - 1) / PRE_WAVES)),
                     dim3(64 * PRE_WAVES), 0, stream, x, p.m, p.k, p.rank, p.pre_slices, b.amax,
                     b.tpart, b.xh, b.thi, b.tlo, b.rowscale);
  return hipGetLastError();
}

hipError_t launch_fwd_contract(const FwdPlan& p, const uint8_t* codes, const uint16_t* scales,
                               const uint16_t* up, void* y, int y_bf16, void* workspace,
                               hipStream_t stream) {
  const FwdBuffers b = carve(p, workspace);
  hipError_t err;
  const int64_t tiles = ((p.m + p.tile_m - 1) / p.tile_m) * ((p.n + p.tile_n - 1) / p.tile_n);
  dim3 grid((unsigned)tiles, (unsigned)p.splits);
  if (p.skinny_mt > 0) {
    const dim3 sg((unsigned)p.splits, (unsigned)((p.n + SK_ROWS - 1) / SK_ROWS));
#define SQ_SKINNY(GS, MT)                                                                         \
  hipLaunchKernelGGL((k_fwd_skinny<GS, MT>), sg, dim3(64), 0, stream, b.xh, codes, scales, b.thi, \
                     b.tlo, up, b.partial, p.m, p.n, p.k, p.rank, p.skinny_kslice)
    if (p.group == 0) {
      if (p.skinny_mt == 1) SQ_SKINNY(0, 1); else if (p.skinny_mt == 2) SQ_SKINNY(0, 2); else SQ_SKINNY(0, 4);
    } else if (p.group == 32) {
      if (p.skinny_mt == 1) SQ_SKINNY(5, 1); else if (p.skinny_mt == 2) SQ_SKINNY(5, 2); else SQ_SKINNY(5, 4);
    } else {
      if (p.skinny_mt == 1) SQ_SKINNY(6, 1); else if (p.skinny_mt == 2) SQ_SKINNY(6, 2); else SQ_SKINNY(6, 4);
    }
#undef SQ_SKINNY
  } else {
    const int kts = (int)(p.k / GBK / p.splits);
#define SQ_BIG(GS, BM, SP)                                                                      \
  hipLaunchKernelGGL((k_fwd_gemm_big<GS, BM, SP>), grid, dim3(BIG_THREADS), 0, stream, b.xh,    \
                     codes, scales, b.thi, b.tlo, up, b.rowscale, y, b.partial, p.m, p.n, p.k,   \
                     p.rank, y_bf16, kts)
#define SQ_BIG_BM(GS, SP)                                                                       \
  if (p.tile_m == 224) SQ_BIG(GS, 224, SP); else if (p.tile_m == 256) SQ_BIG(GS, 256, SP);     \
  else SQ_BIG(GS, 128, SP)
    if (p.group == 0) {
      if (p.splits > 1) { SQ_BIG_BM(0, true); } else { SQ_BIG_BM(0, false); }
    } else if (p.group == 32) {
      if (p.splits > 1) { SQ_BIG_BM(5, true); } else { SQ_BIG_BM(5, false); }
    } else {
      if (p.splits > 1) { SQ_BIG_BM(6, true); } else { SQ_BIG_BM(6, false); }
    }
#undef SQ_BIG_BM
#undef SQ_BIG
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (p.splits > 1 || p.skinny_mt > 0) {
    const int64_t cnt = p.m * p.n;
    hipLaunchKernelGGL(k_fwd_reduce, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, stream,
                       b.partial, b.rowscale, y, p.m, p.n, p.splits, y_bf16);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace sq
