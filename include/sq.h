/* sq.h - C ABI of libsq, the MI355X (gfx950) W4 quantized-frozen-base linear layer.
 *
 * The layer is the SquareQ v3 W4 format (SquareQ README, section "SquareQ v3 -
 * W4 (Hadamard-256 + low-rank + int4 / NVFP4)", the format formula and its
 * "Rotation", "Residual codecs" and "Low-rank branch" bullets):
 *
 *     W_hat = lora_up @ lora_down^T + dequant(R) @ H
 *
 * H is the block-diagonal normalized Hadamard-256 rotation along the input
 * dimension K (Sylvester order, entries +-1/16, symmetric and its own inverse),
 * R holds int4 codes with one fp16 scale per group of 32 or 64 consecutive
 * values along K, and lora_up / lora_down are the bf16 rank-r factors of an
 * SVD of the weight.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates no device memory and keeps no state besides a per-device
 *     architecture check.  Calls are reentrant.
 *   - Arguments are validated synchronously on the host; on any error nothing
 *     is launched and the status says why.  Kernel work is enqueued on
 *     `stream` (a hipStream_t; NULL means the null stream) and is asynchronous:
 *     the library never synchronizes.
 *   - There is exactly one device code path per call and no host fallback: a
 *     device that is not gfx950 gets SQ_E_ARCH.
 *   - All tensors are dense and row-major; every pointer must be 16-byte
 *     aligned (SQ_E_ALIGN).
 */
#ifndef SQ_H
#define SQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SQ_ABI_VERSION 1

typedef enum {
  SQ_OK = 0,
  SQ_E_NULL = 1,      /* a required pointer is NULL                               */
  SQ_E_SHAPE = 2,     /* K % 256 != 0, K < 256, N < 1 or M < 0; the input         */
                      /* gradient also needs N % 64 == 0                          */
  SQ_E_GROUP = 3,     /* group is not 32 or 64                                    */
  SQ_E_RANK = 4,      /* rank is not 0, 32 or 64 (the int8 and MXFP4 modes also  */
                      /* take 16); see the note on ranks below                    */
  SQ_E_ALIGN = 5,     /* a pointer is not 16-byte aligned                         */
  SQ_E_WORKSPACE = 6, /* workspace smaller than the matching *_workspace_bytes()  */
  SQ_E_DTYPE = 7,     /* output dtype is not SQ_F32 or SQ_BF16                    */
  SQ_E_ARCH = 8,      /* the current device is not gfx950                         */
  SQ_E_HIP = 9        /* a HIP runtime call or kernel launch failed               */
} sq_status_t;

typedef enum { SQ_F32 = 0, SQ_BF16 = 1 } sq_dtype_t;

/* Bits OR-ed into *dev_flags by the quantizer (read them after a sync). */
enum {
  SQ_FLAG_NONFINITE = 1,      /* a weight value, or the residual, is NaN or +-inf      */
  SQ_FLAG_SCALE_OVERFLOW = 2, /* absmax/7 of some group (int8 mode: absmax/127 of some */
                              /* row) overflows fp16                                   */
  SQ_FLAG_FP16_RANGE = 4      /* W4 only: some chosen scale exceeds 8188, so the       */
                              /* payload is outside the forward's domain (below)       */
};

/* Ranks.  The page's low-rank branch is rank 32.  The W4 entry points take
 * rank 0, 32 or 64: their kernels walk the factors in 32-wide steps and the
 * input gradient reads whole steps, so rank 16 is refused with SQ_E_RANK
 * rather than read past the factors.  The int8 and MXFP4 modes also take 16
 * (the page's v3.1 split rank).
 *
 * Domain of the W4 forward and input gradient.  Their contraction runs on
 * fp16 MFMA with the weight operand fp16(q * s), q in [-8, 7]; it is finite
 * for every payload whose scales all satisfy 8 * |s| <= 65504, that is
 * |s| <= 8188 (the largest fp16 value below 2^13).  A payload with a larger
 * scale is outside the domain: the products overflow fp16 and y (or dx) holds
 * +-inf or NaN where such a group contributes.  sq_quantize_weight never
 * emits such a payload silently: it sets SQ_FLAG_FP16_RANGE.  Scales in the
 * fp16 subnormal range are inside the domain (q * s is then exact or rounded
 * once, like any other product).  The reconstruct works in fp32 and has no
 * such limit. */

/* The W4 payload of one linear layer with N output and K input features.
 *   codes     uint8  [n][k/2]  byte b of a row = (q[2b] & 0xF) | (q[2b+1] & 0xF) << 4,
 *                              q in [-8, 7] two's complement (even k in the low nibble)
 *   scales    fp16   [n][k/group]  IEEE binary16 bit patterns
 *   lora_up   bf16   [n][rank]     (may be NULL iff rank == 0)
 *   lora_down bf16   [k][rank]     (may be NULL iff rank == 0)
 * Scale g of row n covers q[n][g*group .. g*group+group-1]; those values are
 * coordinates after the rotation, so dequant(R)[n][k] = q[n][k] * s[n][k/group]. */
typedef struct {
  int64_t n, k;
  int32_t group, rank;
  uint8_t *codes;
  uint16_t *scales;
  uint16_t *lora_up;
  uint16_t *lora_down;
} sq_w4_t;

/* Builder side (the format formula read right to left, the "Residual codecs"
 * bullet): quantize the fp32 weight w [n][k].
 *   E = w - lora_up @ lora_down^T           (fp32; the factors are read from p)
 *   R = E @ H                                (block Hadamard-256 along k)
 *   for every group of `group` values of R with absmax a and every
 *   i = 0..30: s_i = fp16(round((70+i)/100 * a / 7)),
 *   q = clamp(round_half_even(r / s_i), -8, 7) (q = 0 when s_i == 0),
 *   err_i = sum (r - q s_i)^2; the first i with the least err wins.
 * Writes p->codes, p->scales and, when fidx != NULL, fidx[n][k/group] = i
 * (uint8).  Non-finite inputs and fp16 scale overflow set bits in *dev_flags
 * (device int32, required; the library only ORs bits into it, so clear it
 * first); outputs are then unspecified but written in bounds.  A chosen scale
 * above 8188 sets SQ_FLAG_FP16_RANGE: the payload is then exact as a format
 * (reconstruct handles it) but outside the forward's domain. */
sq_status_t sq_quantize_weight(const float *w, const sq_w4_t *p, uint8_t *fidx,
                               int32_t *dev_flags, void *stream);

/* Forward (the format formula applied to x; H is symmetric so
 * x @ (dequant(R) @ H)^T = (x @ H) @ dequant(R)^T):
 *   y[m][n] = sum_k (x @ H)[m][k] * q[n][k] * s[n][k/group]
 *           + sum_r (x @ lora_down)[m][r] * lora_up[n][r]
 * x is bf16 [m][k]; y is fp32 or bf16 [m][n] (bf16 = round-to-nearest-even of
 * the fp32 result).  The contraction runs on fp16 MFMA: each row of x @ H is
 * scaled by a power of two that keeps it inside fp16 range and rounded to
 * fp16, the weight operand is fp16(q * s); accumulation is fp32.
 * `workspace` is device scratch of at least sq_linear_fwd_workspace_bytes(m, p)
 * bytes, owned by the caller and not read before it is written.  m == 0 is a
 * no-op that returns SQ_OK. */
size_t sq_linear_fwd_workspace_bytes(int64_t m, const sq_w4_t *p);
sq_status_t sq_linear_fwd(const uint16_t *x, int64_t m, const sq_w4_t *p, void *y,
                          sq_dtype_t y_dtype, void *workspace, size_t workspace_bytes,
                          void *stream);

/* The same forward in its two halves; sq_linear_fwd is exactly
 * sq_linear_fwd_rotate followed by sq_linear_fwd_contract on one stream.
 *   rotate:   reads x, p->lora_down; writes into `workspace` the fp16 rotated
 *             activations, the row powers of two and the rank-r projection
 *             x @ lora_down.
 *   contract: reads that workspace and the payload; writes y.
 * For m <= 16 the rotation and the projection run inside the contraction
 * (the whole call streams the payload once from its first cycle): there
 * rotate only copies x and p->lora_down into the workspace, and contract
 * does the rest from those copies.
 * Both take the same m, p and workspace; contract must follow a rotate of the
 * same x on the same workspace (stream order suffices). */
sq_status_t sq_linear_fwd_rotate(const uint16_t *x, int64_t m, const sq_w4_t *p, void *workspace,
                                 size_t workspace_bytes, void *stream);
sq_status_t sq_linear_fwd_contract(int64_t m, const sq_w4_t *p, void *y, sq_dtype_t y_dtype,
                                   void *workspace, size_t workspace_bytes, void *stream);

/* The forward without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  It computes exactly what sq_linear_fwd computes
 * (same kernels, bit-identical y) with its scratch in a library-owned static
 * device array of SQ_FWD_STATIC_SCRATCH_BYTES (64 MiB), one per device, held
 * by each device the library runs on until the process ends.  It allocates
 * nothing itself; its first call on a device looks up that device's copy of
 * the array.  A call whose sq_linear_fwd_workspace_bytes(m, p) exceeds the
 * array returns SQ_E_WORKSPACE and launches nothing (every m <= 16 forward
 * fits, and so does 4480 x 16384 x 6144).  All calls on one device share the
 * array: calls ordered on one stream are fine, calls that overlap in time on
 * one device (different streams, no ordering) race and give undefined y.
 * Nothing in the array needs to be zero: each call writes what it reads. */
#define SQ_FWD_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
sq_status_t sq_linear_fwd_static(const uint16_t *x, int64_t m, const sq_w4_t *p, void *y,
                                 sq_dtype_t y_dtype, void *stream);

/* Backward side: rebuild the dense bf16 weight from the same payload
 *   w_hat[n][k] = bf16_round_nearest_even( lora_up @ lora_down^T + dequant(R) @ H )
 * with every intermediate in fp32 and one rounding at the end. */
sq_status_t sq_reconstruct_bf16(const sq_w4_t *p, uint16_t *w_hat, void *stream);

/* Input gradient (the format formula transposed: dx = dy @ W_hat; where the
 * page's backward first rebuilds the dense bf16 weight, this contracts the
 * packed codes directly, and H H = I moves the rotation to the end):
 *   dx = (dy @ dequant(R)) @ H + (dy @ lora_up) @ lora_down^T, that is
 *   dx[m][k] = sum_j ( sum_n dy[m][n] q[n][j] s[n][j/group] ) H[j][k]
 *            + sum_r (dy @ lora_up)[m][r] lora_down[k][r].
 * dy is bf16 [m][n]; dx is fp32 or bf16 [m][k] (bf16 = round-to-nearest-even
 * of the fp32 result).  N must be a multiple of 64.  The int4 contraction runs
 * on fp16 MFMA with the same operand treatment as the forward: each row of dy
 * is scaled by a power of two and rounded to fp16, the weight operand is
 * fp16(q * s), accumulation is fp32; the rank-r term is carried as bf16 hi +
 * lo parts.  `workspace` is device scratch of at least
 * sq_linear_dgrad_workspace_bytes(m, p) bytes (0 for unsupported shapes),
 * owned by the caller and not read before it is written.  m == 0 is a no-op
 * that returns SQ_OK. */
size_t sq_linear_dgrad_workspace_bytes(int64_t m, const sq_w4_t *p);
sq_status_t sq_linear_dgrad(const uint16_t *dy, int64_t m, const sq_w4_t *p, void *dx,
                            sq_dtype_t dx_dtype, void *workspace, size_t workspace_bytes,
                            void *stream);

/* ------------------------------------------------------------------------
 * int8-residual mode (SquareQ README, section "v3.1 - int8-residual mode": the
 * same format formula with an int8 residual left by a rank-16 split).  The
 * page names the mode without its details; this library reads it as the W4
 * sweep on the int8 grid with one scale per output row:
 *   W_hat = lora_up @ lora_down^T + dequant(R) @ H,  dequant(R)[n][k] = q[n][k] * s[n]
 * The payload of one layer:
 *   codes     int8   [n][k]     q in [-128, 127], coordinates after the rotation
 *   scales    fp16   [n]        one scale per output row (IEEE binary16 bits)
 *   lora_up   bf16   [n][rank]  rank 0, 16, 32 or 64 (16 is the page's)
 *   lora_down bf16   [k][rank]
 * `reserved` must be 0.  Shapes, alignment, streams and errors follow the W4
 * conventions above. */
typedef struct {
  int64_t n, k;
  int32_t rank, reserved;
  int8_t *codes;
  uint16_t *scales;
  uint16_t *lora_up;
  uint16_t *lora_down;
} sq_w8_t;

/* Builder side of the int8 mode: quantize the fp32 weight w [n][k].
 *   E = w - lora_up @ lora_down^T ;  R = E @ H
 *   per row with absmax a and for i = 0..30: s_i = fp16(round((70+i)/100 * a / 127)),
 *   q = clamp(round_half_even(r / s_i), -128, 127) (q = 0 when s_i == 0),
 *   err_i = sum over the row of (r - q s_i)^2; the first i with the least err wins.
 * Writes p->codes, p->scales and, when fidx != NULL, fidx[n] = i (uint8).
 * `workspace` (device, caller-owned, at least
 * sq_quantize_weight_w8_workspace_bytes(p) bytes) holds the rotated residual
 * in fp32 between the rotation and the sweep.  dev_flags as for
 * sq_quantize_weight. */
size_t sq_quantize_weight_w8_workspace_bytes(const sq_w8_t *p);
sq_status_t sq_quantize_weight_w8(const float *w, const sq_w8_t *p, uint8_t *fidx,
                                  int32_t *dev_flags, void *workspace, size_t workspace_bytes,
                                  void *stream);

/* Rebuild the dense bf16 weight of an int8-mode payload:
 *   w_hat[n][k] = bf16_round_nearest_even( lora_up @ lora_down^T + (q * s[n]) @ H )
 * with the rotation summed exactly on integers, one fp32 rounding for the
 * scale, the rank-r term added in fp32 and one rounding at the end. */
sq_status_t sq_reconstruct_bf16_w8(const sq_w8_t *p, uint16_t *w_hat, void *stream);

/* Forward of an int8-mode payload:
 *   y[m][n] = s[n] * sum_k (x @ H)[m][k] q[n][k] + sum_r (x @ lora_down)[m][r] lora_up[n][r]
 * x bf16 [m][k], y fp32 or bf16 [m][n].  The contraction runs on fp16 MFMA
 * with the activations treated as in sq_linear_fwd (a power of two per row,
 * rounded to fp16) and the codes exact in fp16; the row scale multiplies the
 * fp32 sum.  `workspace` is caller-owned device scratch of at least
 * sq_linear_fwd_w8_workspace_bytes(m, p) bytes; m == 0 is a no-op. */
size_t sq_linear_fwd_w8_workspace_bytes(int64_t m, const sq_w8_t *p);
sq_status_t sq_linear_fwd_w8(const uint16_t *x, int64_t m, const sq_w8_t *p, void *y,
                             sq_dtype_t y_dtype, void *workspace, size_t workspace_bytes,
                             void *stream);

/* ------------------------------------------------------------------------
 * MXFP4 mode (SquareQ README, "SquareQ v3 - W4", the "Residual codecs"
 * bullet's FP4 alternative for native FP4 matrix instructions, and the
 * op-level parity line that describes the FP4 forward as rotate +
 * block-quant of the activations + FP4 product + epilogue).  The page's
 * NVFP4 layout targets one vendor's instructions; this library uses the OCP
 * MX counterpart that gfx950's scaled MFMA takes:
 *   element  FP4 E2M1, magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, nibble
 *            s<<3 | e<<1 | m; a value that rounds to magnitude 0 is nibble 0
 *   block    32 consecutive values along K share an E8M0 byte e (scale
 *            2^(e-127)), e = floor(log2 absmax) - 2 + 127 clamped to [0, 254]
 *            (0 for an all-zero block)
 *   rounding v / 2^(e-127) to the nearest E2M1 value, ties to the even
 *            mantissa, magnitudes above 6 saturate to 6
 * The payload of one layer:
 *   codes     uint8 [n][k/2]   two nibbles per byte, even k in the low nibble,
 *                              coordinates after the rotation
 *   exps      uint8 [n][k/32]  E8M0 block exponents
 *   lora_up   bf16  [n][rank], lora_down bf16 [k][rank]  (rank 0, 16, 32, 64)
 * `reserved` must be 0.  Shapes, alignment, streams and errors follow the W4
 * conventions above. */
typedef struct {
  int64_t n, k;
  int32_t rank, reserved;
  uint8_t *codes;
  uint8_t *exps;
  uint16_t *lora_up;
  uint16_t *lora_down;
} sq_mx4_t;

/* Builder side: codes/exps = MXFP4 of R = (w - lora_up @ lora_down^T) @ H,
 * w fp32 [n][k].  Non-finite values of R set SQ_FLAG_NONFINITE in *dev_flags
 * (outputs are then unspecified but written in bounds). */
sq_status_t sq_quantize_weight_mx4(const float *w, const sq_mx4_t *p, int32_t *dev_flags,
                                   void *stream);

/* Activation half of the forward: xq [m][k/2] / xs [m][k/32] = MXFP4 of
 * x @ H, x bf16 [m][k] (device buffers owned by the caller). */
sq_status_t sq_quantize_act_mx4(const uint16_t *x, int64_t m, int64_t k, uint8_t *xq,
                                uint8_t *xs, void *stream);

/* w_hat[n][k] = bf16_round_nearest_even( lora_up @ lora_down^T + dq(codes, exps) @ H ),
 * the rotation summed in fp32 (exact before the block scales), one rounding
 * at the end. */
sq_status_t sq_reconstruct_bf16_mx4(const sq_mx4_t *p, uint16_t *w_hat, void *stream);

/* Forward: y[m][n] = sum_k dq(Q(x @ H))[m][k] dq(codes, exps)[n][k]
 *                  + sum_r (x @ lora_down)[m][r] lora_up[n][r]
 * with Q the MXFP4 quantization above (the activations are quantized inside
 * the call, as sq_quantize_act_mx4 does), the FP4 product on
 * v_mfma_scale_f32_16x16x128_f8f6f4 with fp32 accumulation, and the rank-r
 * term from the unquantized x (fp32, carried as bf16 hi + lo).  y fp32 or
 * bf16 (RNE of the fp32 result).  `workspace`: caller-owned device scratch
 * of at least sq_linear_fwd_mx4_workspace_bytes(m, p) bytes; m == 0 is a
 * no-op. */
size_t sq_linear_fwd_mx4_workspace_bytes(int64_t m, const sq_mx4_t *p);
sq_status_t sq_linear_fwd_mx4(const uint16_t *x, int64_t m, const sq_mx4_t *p, void *y,
                              sq_dtype_t y_dtype, void *workspace, size_t workspace_bytes,
                              void *stream);

/* Static description of a status code; never NULL. */
const char *sq_status_str(sq_status_t status);
int sq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SQ_H */
