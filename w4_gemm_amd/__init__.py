"""MI355X-native SquareQ v3 W4 linear layer: libsq (HIP, gfx950) + a thin binding.

Entry points (C ABI in include/sq.h, same names here):
  sq_quantize_weight   builder side: rotate + MSE fraction sweep + int4 pack
  sq_linear_fwd        fused forward  y = H256(x) dequant(R)^T + (x down) up^T
  sq_linear_fwd_static the same forward with a library-owned static scratch (no workspace)
  sq_reconstruct_bf16  backward side: bf16 W_hat from the same payload
  sq_linear_dgrad      input gradient dx = dy W_hat straight from the payload
  *_w8                 the same for the int8-residual mode (int8 codes, one scale per row)
  *_mx4                the MXFP4 mode (E2M1 codes, E8M0 block-32 exponents; the forward
                       quantizes the rotated activations too and runs on FP4 MFMA)
The rank-32 SVD split that feeds the quantizer is a host step (svd_init).
"""
from .api import (W4Payload, dgrad_workspace_bytes, empty_payload, fwd_workspace_bytes,
                  linear_dgrad, linear_fwd, linear_fwd_contract, linear_fwd_rotate, linear_fwd_static,
                  quantize_weight, reconstruct_bf16, W8Payload, empty_payload_w8,
                  quantize_weight_w8, reconstruct_bf16_w8, fwd_w8_workspace_bytes, linear_fwd_w8,
                  MX4Payload, empty_payload_mx4, quantize_weight_mx4, quantize_act_mx4,
                  reconstruct_bf16_mx4, fwd_mx4_workspace_bytes, linear_fwd_mx4)
from ._lib import SqError, abi_version
from .svd_init import svd_init

__all__ = ["W4Payload", "empty_payload", "fwd_workspace_bytes", "linear_fwd", "linear_fwd_rotate",
           "linear_fwd_static",
           "linear_fwd_contract", "quantize_weight", "linear_dgrad", "dgrad_workspace_bytes",
           "reconstruct_bf16", "SqError", "abi_version", "svd_init", "W8Payload",
           "empty_payload_w8", "quantize_weight_w8", "reconstruct_bf16_w8",
           "fwd_w8_workspace_bytes", "linear_fwd_w8", "MX4Payload", "empty_payload_mx4",
           "quantize_weight_mx4", "quantize_act_mx4", "reconstruct_bf16_mx4",
           "fwd_mx4_workspace_bytes", "linear_fwd_mx4"]
