// Host-side launchers of the libsq kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sq {

hipError_t launch_reconstruct(const uint8_t* codes, const uint16_t* scales, const uint16_t* up,
                              const uint16_t* down, uint16_t* w_hat, int64_t n, int64_t k,
                              int group, int rank, hipStream_t stream);

hipError_t launch_quantize(const float* w, const uint16_t* up, const uint16_t* down,
                           uint8_t* codes, uint16_t* scales, uint8_t* fidx, int32_t* flags,
                           int64_t n, int64_t k, int group, int rank, hipStream_t stream);

// int8-residual mode quantizer (two launches around an fp32 copy of the
// rotated residual in the workspace).  The reconstruct is launch_reconstruct
// with group 0.
size_t quantize_w8_workspace(int64_t n, int64_t k);
hipError_t launch_quantize_w8(const float* w, const uint16_t* up, const uint16_t* down,
                              int8_t* codes, uint16_t* scales, uint8_t* fidx, int32_t* flags,
                              int64_t n, int64_t k, int rank, void* workspace,
                              hipStream_t stream);

// MXFP4 mode: E2M1 codes [rows][K/2] (even k in the low nibble) with E8M0
// block-32 exponents [rows][K/32].
struct MxPlan {
  int64_t m, n, k;
  int rank;
  int slices;   // workgroups along K of the activation pass (4 blocks each)
  int splits;   // split-K factor of the FP4 contraction
  size_t off_xq, off_xs, off_downT, off_tpart, off_thi, off_tlo, off_part, total;
};
MxPlan plan_mx(int64_t m, int64_t n, int64_t k, int rank);
hipError_t launch_quantize_mx(const float* w, const uint16_t* up, const uint16_t* down,
                              uint8_t* codes, uint8_t* exps, int32_t* flags, int64_t n, int64_t k,
                              int rank, hipStream_t stream);
hipError_t launch_quantize_act_mx(const uint16_t* x, int64_t m, int64_t k, uint8_t* xq, uint8_t* xs,
                                  hipStream_t stream);
hipError_t launch_fwd_mx(const MxPlan& p, const uint16_t* x, const uint8_t* wq, const uint8_t* wsc,
                         const uint16_t* up, const uint16_t* down, void* y, int y_bf16,
                         void* workspace, hipStream_t stream);
hipError_t launch_reconstruct_mx(const uint8_t* codes, const uint8_t* exps, const uint16_t* up,
                                 const uint16_t* down, uint16_t* w_hat, int64_t n, int64_t k,
                                 int rank, hipStream_t stream);

// Forward: workspace layout and launch.
struct FwdPlan {
  int64_t m, n, k;
  int group, rank;
  int splits;          // split-K factor of the main contraction
  int tile_m, tile_n;  // output tile of the main contraction
  int skinny_mt;       // > 0: the small-M kernel with this many 16-row tiles
  int skinny_kslice;   // its K slice (a multiple of 256)
  int pre_bps, pre_slices;  // 256-column blocks per K slice of the statistics pass, slices
  int pre_tiles;            // 16-row tiles per statistics workgroup (1, 2, 4 or 8)
  int pre_fused;            // > 0: both pre-phase passes in one launch, this many blocks per wave
  int dec;             // 1: the small-M decode path (rotation inside the contraction)
  int dec_kslice;      // its K slice (a multiple of 256, at most 1024)
  size_t off_xh, off_thi, off_tlo, off_rowscale, off_downT, off_amax, off_tpart, off_partial, total;
};
FwdPlan plan_fwd(int64_t m, int64_t n, int64_t k, int group, int rank);

// Small-M decode path (M <= 16): eligibility, plan and launches.  The whole
// product runs in launch_decode_contract; in the split-call form the first
// half stages x and lora_down in the workspace (launch_decode_prep) and the
// second passes x = down = null to read them there.
bool decode_eligible(int64_t m, int64_t n, int64_t k, int rank, bool int8 = false);
FwdPlan plan_decode(int64_t m, int64_t n, int64_t k, int group, int rank);
hipError_t launch_decode_prep(const FwdPlan& plan, const uint16_t* x, const uint16_t* down,
                              void* workspace, hipStream_t stream);
hipError_t launch_decode_contract(const FwdPlan& plan, const uint16_t* x, const uint16_t* down,
                                  const uint8_t* codes, const uint16_t* scales, const uint16_t* up,
                                  void* y, int y_bf16, void* workspace, hipStream_t stream);

// Row statistics of a bf16 matrix a [m][k] (k a multiple of 256) against a
// bf16 factor: per K slice of four 256-column blocks, the row absmax bits
// amax_part[q][row] and the partial products
// t_part[q][row][r] = sum_{k in slice q} a[row][k] fac[k][r] (fp32, fixed
// order).  The factor is [k][rank] when kmajor (ranks 16 and 32 only), else
// transposed, [rank][k].  rank is 0, 16, 32 or 64; tiles (1, 2, 4 or 8)
// 16-row tiles per workgroup.  row_stats_plan picks the tiles and the slice
// count.
void row_stats_plan(int64_t m, int64_t k, int* tiles, int* slices);
hipError_t launch_row_stats(const uint16_t* a, const uint16_t* fac, bool kmajor, int64_t m,
                            int64_t k, int rank, int tiles, int slices, uint32_t* amax_part,
                            float* t_part, hipStream_t stream);
hipError_t launch_fwd_rotate(const FwdPlan& plan, const uint16_t* x, const uint16_t* down,
                             void* workspace, hipStream_t stream);
hipError_t launch_fwd_contract(const FwdPlan& plan, const uint8_t* codes, const uint16_t* scales,
                               const uint16_t* up, void* y, int y_bf16, void* workspace,
                               hipStream_t stream);

// Input gradient: workspace layout and launch.
struct DgradPlan {
  int64_t m, n, k;
  int group, rank;
  int stats_sps, stats_slices;   // 32-column steps of N per statistics slice, slices
  int stats_tiles;               // > 0: the shared row-statistics kernel (N % 256 == 0), its tiles
  int tile_m;                    // rows of the contraction tile (256 or 224)
  size_t off_upT, off_amax, off_tpart, off_dy16, off_thi, off_tlo, off_rowscale, off_hdhi,
      off_hdlo, off_c, total;
};
DgradPlan plan_dgrad(int64_t m, int64_t n, int64_t k, int group, int rank);

hipError_t launch_dgrad(const DgradPlan& plan, const uint16_t* dy, const uint8_t* codes,
                        const uint16_t* scales, const uint16_t* up, const uint16_t* down,
                        void* dx, int dx_bf16, void* workspace, hipStream_t stream);

}  // namespace sq
