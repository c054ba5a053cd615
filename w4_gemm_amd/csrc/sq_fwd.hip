// Fused W4 forward (SquareQ README, "SquareQ v3 - W4": the format formula
// applied to an activation; H symmetric gives x @ W_hat^T = (x H) @ D^T +
// (x @ down) @ up^T with D = dequant(R)):
//
//   y[m][n] = 2^(E_m - 11) * ( sum_k xh16[m][k] * fp16(q[n][k] s[n][k/G])
//                              + sum_r t16[m][r] * up[n][r] )
//
// Three launches on the caller's stream:
//   1. k_transpose_down: down [K][r] -> downT [r][K] (tiny; lets the MFMA
//      operands of x @ down be read as 16-byte rows).
//   2. k_fwd_pre: per 16 rows, (a) t = x @ down on bf16 MFMA and the row
//      absmax A_m; E_m = ceil(log2 A_m); (b) xh = (x H) * 2^(11-E_m) with the
//      256-point butterflies in registers/lanes, rounded to fp16 (|xh| <= 2^15
//      because every entry of x H is at most 16 A_m), and t * 2^(11-E_m) split
//      into bf16 hi + lo.
//   3. k_fwd_gemm: the int4 contraction on fp16 MFMA.  The packed codes stream
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
constexpr int PRE_WAVES = 8;

__device__ __forceinline__ void load_x64(uint32_t (&xb)[32], const uint16_t* __restrict__ x,
                                         int64_t row, bool live, int64_t k, int64_t col) {
  if (live) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + row * k + col);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 q = src[j];
      xb[4 * j] = q[0];
      xb[4 * j + 1] = q[1];
      xb[4 * j + 2] = q[2];
      xb[4 * j + 3] = q[3];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j) xb[j] = 0;
  }
}

__global__ void __launch_bounds__(512) k_fwd_pre(const uint16_t* __restrict__ x,
                                                  const uint16_t* __restrict__ downT, int64_t m,
                                                  int64_t k, int rank,
                                                  uint16_t* __restrict__ xh,
                                                  uint16_t* __restrict__ thi,
                                                  uint16_t* __restrict__ tlo,
                                                  float* __restrict__ rowscale) {
  __shared__ float red_t[PRE_WAVES][16][64];
  __shared__ uint32_t red_max[PRE_WAVES][64];
  __shared__ float row_f[16];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int64_t row = row0 + c;
  const bool live = row < m;
  const int64_t nblk = k >> 8;

  // pass 1: t partial sums and |x| max (bf16 magnitudes compare as integers)
  f32x4 acc[4] = {};
  uint32_t amax = 0;
  for (int64_t b = wave; b < nblk; b += PRE_WAVES) {
    const int64_t col = b * 256 + 64 * g;
    uint32_t xb[32];
    load_x64(xb, x, row, live, k, col);
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      amax = max(amax, xb[j] & 0x7FFFu);
      amax = max(amax, (xb[j] >> 16) & 0x7FFFu);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 araw = {xb[4 * j], xb[4 * j + 1], xb[4 * j + 2], xb[4 * j + 3]};
      bf16x8 afrag = __builtin_bit_cast(bf16x8, araw);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        if (16 * rt < rank) {
          bf16x8 bfrag = *reinterpret_cast<const bf16x8*>(downT + (int64_t)(16 * rt + c) * k +
                                                          col + 8 * j);
          acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag, bfrag, acc[rt], 0, 0, 0);
        }
      }
    }
  }
  // acc[rt][i] = partial t[row0 + 4g + i][16 rt + c]
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
    if (16 * rt < rank)
#pragma unroll
      for (int i = 0; i < 4; ++i) red_t[wave][4 * g + i][16 * rt + c] = acc[rt][i];
  red_max[wave][lane] = amax;
  __syncthreads();
  if (threadIdx.x < 16) {
    const int rr = threadIdx.x;
    uint32_t mx = 0;
    for (int w = 0; w < PRE_WAVES; ++w)
      for (int gg = 0; gg < 4; ++gg) mx = max(mx, red_max[w][rr + 16 * gg]);
    const float a = bf16_to_f32(mx);
    int e = 0;
    if (a > 0.0f) {
      int ex;
      const float mant = frexpf(a, &ex);   // a = mant * 2^ex, mant in [0.5, 1)
      e = (mant == 0.5f) ? ex - 1 : ex;    // smallest e with a <= 2^e
    }
    e = max(e, -100);
    row_f[rr] = ldexpf(1.0f, 11 - e);
    if (row0 + rr < m) rowscale[row0 + rr] = ldexpf(1.0f, e - 11);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * rank; i += 512) {
    const int rr = i / rank, r = i - rr * rank;
    if (row0 + rr >= m) continue;
    float t = 0.0f;
    for (int w = 0; w < PRE_WAVES; ++w) t += red_t[w][rr][r];
    t *= row_f[rr];
    const uint16_t hb = f32_to_bf16(t);
    const uint16_t lb = f32_to_bf16(t - bf16_to_f32(hb));
    thi[(row0 + rr) * rank + r] = hb;
    tlo[(row0 + rr) * rank + r] = lb;
  }

  // pass 2: rotation, row scaling, fp16, permuted store
  const float f = row_f[c] * 0.0625f;
  for (int64_t b = wave; b < nblk; b += PRE_WAVES) {
    const int64_t col = b * 256 + 64 * g;
    uint32_t xb[32];
    load_x64(xb, x, row, live, k, col);
    float v[64];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      v[2 * j] = bf16_to_f32(xb[j] & 0xFFFFu);
      v[2 * j + 1] = bf16_to_f32(xb[j] >> 16);
    }
    fwht256_wave(v, lane);
    if (live) {
      u32x4 out[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const _Float16 lo = (_Float16)(v[8 * j + p] * f);
          const _Float16 hi = (_Float16)(v[8 * j + p + 4] * f);
          out[j][p] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
      }
      u32x4* dst = reinterpret_cast<u32x4*>(xh + row * k + col);
#pragma unroll
      for (int j = 0; j < 8; ++j) dst[j] = out[j];
    }
  }
}

// ---------------------------------------------------------------- main contraction
constexpr int GBM = 128, GBN = 128, GBK = 64, LDS_STRIDE = GBK + 8;   // halves per LDS row

// 32 packed codes (one 16-byte load) -> 16 fp16 pairs of q*s, in the permuted
// K order: pair p of word j holds codes (8j+p, 8j+p+4).
__device__ __forceinline__ void dequant32_f16(uint32_t (&out)[16], const u32x4& w, _Float16 s) {
  const half2v sv = {s, s};
  const half2v off = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t word = w[j] ^ 0x88888888u;   // nibble ^ 8 = q + 8
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t bits = ((word >> (4 * p)) & 0x000F000Fu) | 0x64006400u;   // 1024 + q + 8
      half2v h = __builtin_bit_cast(half2v, bits);
      h = (h - off) * sv;
      out[4 * j + p] = __builtin_bit_cast(uint32_t, h);
    }
  }
}

__global__ void __launch_bounds__(256) k_fwd_gemm(
    const uint16_t* __restrict__ xh, const uint8_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ thi,
    const uint16_t* __restrict__ tlo, const uint16_t* __restrict__ up,
    const float* __restrict__ rowscale, void* __restrict__ y, float* __restrict__ partial,
    int64_t m, int64_t n, int64_t k, int group, int rank, int splits, int y_bf16) {
  __shared__ __attribute__((aligned(16))) _Float16 As[2][GBM][LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[2][GBN][LDS_STRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * GBM;
  const int64_t n0 = (int64_t)blockIdx.x * GBN;
  const int z = blockIdx.z;
  const int64_t KT = k / GBK;
  const int64_t per = (KT + splits - 1) / splits;
  const int64_t kt0 = min((int64_t)z * per, KT), kt1 = min(kt0 + per, KT);

  // loader roles: row lr, half lh
  const int lr = tid >> 1, lh = tid & 1;
  const int64_t a_row = m0 + lr, b_row = n0 + lr;
  const bool a_live = a_row < m, b_live = b_row < n;
  const int64_t ngroups = k / group;

  u32x4 a_reg[4];
  u32x4 b_reg;
  _Float16 s_reg;
  auto gload = [&](int64_t kt) {
    const int64_t kk = kt * GBK + 32 * lh;
    if (a_live) {
      const u32x4* src = reinterpret_cast<const u32x4*>(xh + a_row * k + kk);
#pragma unroll
      for (int j = 0; j < 4; ++j) a_reg[j] = src[j];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) a_reg[j] = (u32x4){0, 0, 0, 0};
    }
    if (b_live) {
      b_reg = *reinterpret_cast<const u32x4*>(codes + b_row * (k >> 1) + (kk >> 1));
      s_reg = __builtin_bit_cast(_Float16, scales[b_row * ngroups + kk / group]);
    } else {
      b_reg = (u32x4){0, 0, 0, 0};
      s_reg = (_Float16)0.0f;
    }
  };
  auto lstore = [&](int buf) {
    u32x4* ad = reinterpret_cast<u32x4*>(&As[buf][lr][32 * lh]);
#pragma unroll
    for (int j = 0; j < 4; ++j) ad[j] = a_reg[j];
    uint32_t bq[16];
    dequant32_f16(bq, b_reg, s_reg);
    u32x4* bd = reinterpret_cast<u32x4*>(&Bs[buf][lr][32 * lh]);
#pragma unroll
    for (int j = 0; j < 4; ++j) bd[j] = (u32x4){bq[4 * j], bq[4 * j + 1], bq[4 * j + 2], bq[4 * j + 3]};
  };

  f32x4 acc[4][4] = {};
  if (kt0 < kt1) {
    gload(kt0);
    lstore(0);
    __syncthreads();
    for (int64_t kt = kt0; kt < kt1; ++kt) {
      const int buf = (int)((kt - kt0) & 1);
      const bool more = kt + 1 < kt1;
      if (more) gload(kt + 1);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        half8 af[4], bfr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          af[i] = *reinterpret_cast<const half8*>(&As[buf][wm * 64 + 16 * i + (lane & 15)]
                                                     [32 * ks + 8 * (lane >> 4)]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bfr[j] = *reinterpret_cast<const half8*>(&Bs[buf][wn * 64 + 16 * j + (lane & 15)]
                                                      [32 * ks + 8 * (lane >> 4)]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (more) lstore(buf ^ 1);
      __syncthreads();
    }
  }

  // rank-r branch: (t_hi + t_lo) @ up^T on bf16 MFMA, added once (split 0)
  if (z == 0) {
    for (int rr = 0; rr < rank; rr += 32) {
#pragma unroll
      for (int hl = 0; hl < 2; ++hl) {
        const uint16_t* tsrc = hl ? tlo : thi;
        bf16x8 af[4], bfr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t r = m0 + wm * 64 + 16 * i + (lane & 15);
          af[i] = r < m ? *reinterpret_cast<const bf16x8*>(tsrc + r * rank + rr + 8 * (lane >> 4))
                        : (bf16x8){};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t cc = n0 + wn * 64 + 16 * j + (lane & 15);
          bfr[j] = cc < n ? *reinterpret_cast<const bf16x8*>(up + cc * rank + rr + 8 * (lane >> 4))
                          : (bf16x8){};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    }
  }

  // epilogue: lane holds rows 4*(lane/16)+v of each 16x16 tile, column lane%16
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t r = m0 + wm * 64 + 16 * i + 4 * (lane >> 4) + v;
      if (r >= m) continue;
      const float rs = rowscale[r];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t cc = n0 + wn * 64 + 16 * j + (lane & 15);
        if (cc >= n) continue;
        if (splits > 1) {
          partial[((int64_t)z * m + r) * n + cc] = acc[i][j][v];
        } else if (y_bf16) {
          reinterpret_cast<uint16_t*>(y)[r * n + cc] = f32_to_bf16(acc[i][j][v] * rs);
        } else {
          reinterpret_cast<float*>(y)[r * n + cc] = acc[i][j][v] * rs;
        }
      }
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
  float s = 0.0f;
  for (int z = 0; z < splits; ++z) s += partial[(int64_t)z * m * n + i];   // fixed order
  s *= rowscale[i / n];
  if (y_bf16)
    reinterpret_cast<uint16_t*>(y)[i] = f32_to_bf16(s);
  else
    reinterpret_cast<float*>(y)[i] = s;
}

// ---------------------------------------------------------------- host side
static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

FwdPlan plan_fwd(int64_t m, int64_t n, int64_t k, int group, int rank) {
  FwdPlan p{};
  p.m = m; p.n = n; p.k = k; p.group = group; p.rank = rank;
  p.tile_m = GBM; p.tile_n = GBN;
  const int64_t tiles = ((m + GBM - 1) / GBM) * ((n + GBN - 1) / GBN);
  const int64_t KT = k / GBK;
  // enough workgroups to cover the 256 compute units about twice, but keep
  // at least 8 K-steps per split
  int64_t s = (512 + tiles - 1) / tiles;
  s = std::min<int64_t>(s, std::max<int64_t>(1, KT / 8));
  s = std::max<int64_t>(s, 1);
  p.splits = (int)s;
  size_t off = 0;
  p.off_xh = off;        off = align256(off + (size_t)m * k * 2);
  p.off_thi = off;       off = align256(off + (size_t)m * std::max(rank, 1) * 2);
  p.off_tlo = off;       off = align256(off + (size_t)m * std::max(rank, 1) * 2);
  p.off_rowscale = off;  off = align256(off + (size_t)m * 4);
  p.off_downT = off;     off = align256(off + (size_t)k * std::max(rank, 1) * 2);
  p.off_partial = off;   off = align256(off + (p.splits > 1 ? (size_t)p.splits * m * n * 4 : 0));
  p.total = off;
  return p;
}

struct FwdBuffers {
  uint16_t *xh, *thi, *tlo, *downT;
  float *rowscale, *partial;
};

static FwdBuffers carve(const FwdPlan& p, void* workspace) {
  char* ws = static_cast<char*>(workspace);
  return FwdBuffers{reinterpret_cast<uint16_t*>(ws + p.off_xh),
                    reinterpret_cast<uint16_t*>(ws + p.off_thi),
                    reinterpret_cast<uint16_t*>(ws + p.off_tlo),
                    reinterpret_cast<uint16_t*>(ws + p.off_downT),
                    reinterpret_cast<float*>(ws + p.off_rowscale),
                    reinterpret_cast<float*>(ws + p.off_partial)};
}

hipError_t launch_fwd_rotate(const FwdPlan& p, const uint16_t* x, const uint16_t* down,
                             void* workspace, hipStream_t stream) {
  const FwdBuffers b = carve(p, workspace);
  hipError_t err;
  if (p.rank > 0) {
    const int64_t cnt = p.k * p.rank;
    hipLaunchKernelGGL(k_transpose_down, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, stream,
                       down, b.downT, p.k, p.rank);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(k_fwd_pre, dim3((unsigned)((p.m + 15) / 16)), dim3(512), 0, stream, x,
                     b.downT, p.m, p.k, p.rank, b.xh, b.thi, b.tlo, b.rowscale);
  return hipGetLastError();
}

hipError_t launch_fwd_contract(const FwdPlan& p, const uint8_t* codes, const uint16_t* scales,
                               const uint16_t* up, void* y, int y_bf16, void* workspace,
                               hipStream_t stream) {
  const FwdBuffers b = carve(p, workspace);
  hipError_t err;
  dim3 grid((unsigned)((p.n + GBN - 1) / GBN), (unsigned)((p.m + GBM - 1) / GBM),
            (unsigned)p.splits);
  hipLaunchKernelGGL(k_fwd_gemm, grid, dim3(256), 0, stream, b.xh, codes, scales, b.thi, b.tlo, up,
                     b.rowscale, y, b.partial, p.m, p.n, p.k, p.group, p.rank, p.splits, y_bf16);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (p.splits > 1) {
    const int64_t cnt = p.m * p.n;
    hipLaunchKernelGGL(k_fwd_reduce, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, stream,
                       b.partial, b.rowscale, y, p.m, p.n, p.splits, y_bf16);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace sq
