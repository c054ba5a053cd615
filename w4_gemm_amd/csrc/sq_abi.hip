// C ABI of libsq: argument validation, device check and kernel launches.
// Every entry point validates synchronously and launches nothing on error;
// work is enqueued on the caller's stream and never synchronized here.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/sq.h"
#include "sq_kernels.h"

namespace {

constexpr int kMaxDevices = 64;
int g_arch_ok[kMaxDevices];   // 0 unknown, 1 gfx950, -1 other
std::mutex g_arch_mu;

sq_status_t check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SQ_E_HIP;
  std::lock_guard<std::mutex> lock(g_arch_mu);
  if (g_arch_ok[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SQ_E_HIP;
    g_arch_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  return g_arch_ok[dev] == 1 ? SQ_OK : SQ_E_ARCH;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

sq_status_t check_payload(const sq_w4_t* p, bool need_codes) {
  if (!p) return SQ_E_NULL;
  if (p->k < 256 || p->k % 256 != 0 || p->n < 1) return SQ_E_SHAPE;
  if (p->group != 32 && p->group != 64) return SQ_E_GROUP;
  if (p->rank != 0 && p->rank != 32 && p->rank != 64) return SQ_E_RANK;
  if (!p->codes || !p->scales) return SQ_E_NULL;
  if (p->rank > 0 && (!p->lora_up || !p->lora_down)) return SQ_E_NULL;
  if (!aligned16(p->codes) || !aligned16(p->scales)) return SQ_E_ALIGN;
  if (p->rank > 0 && (!aligned16(p->lora_up) || !aligned16(p->lora_down))) return SQ_E_ALIGN;
  (void)need_codes;
  return SQ_OK;
}

sq_status_t check_payload_w8(const sq_w8_t* p) {
  if (!p) return SQ_E_NULL;
  if (p->k < 256 || p->k % 256 != 0 || p->n < 1) return SQ_E_SHAPE;
  if ((p->rank != 0 && p->rank != 16 && p->rank != 32 && p->rank != 64) || p->reserved != 0)
    return SQ_E_RANK;
  if (!p->codes || !p->scales) return SQ_E_NULL;
  if (p->rank > 0 && (!p->lora_up || !p->lora_down)) return SQ_E_NULL;
  if (!aligned16(p->codes) || !aligned16(p->scales)) return SQ_E_ALIGN;
  if (p->rank > 0 && (!aligned16(p->lora_up) || !aligned16(p->lora_down))) return SQ_E_ALIGN;
  return SQ_OK;
}

sq_status_t check_payload_mx(const sq_mx4_t* p) {
  if (!p) return SQ_E_NULL;
  if (p->k < 256 || p->k % 256 != 0 || p->n < 1) return SQ_E_SHAPE;
  if ((p->rank != 0 && p->rank != 16 && p->rank != 32 && p->rank != 64) || p->reserved != 0)
    return SQ_E_RANK;
  if (!p->codes || !p->exps) return SQ_E_NULL;
  if (p->rank > 0 && (!p->lora_up || !p->lora_down)) return SQ_E_NULL;
  if (!aligned16(p->codes) || !aligned16(p->exps)) return SQ_E_ALIGN;
  if (p->rank > 0 && (!aligned16(p->lora_up) || !aligned16(p->lora_down))) return SQ_E_ALIGN;
  return SQ_OK;
}

sq_status_t from_hip(hipError_t e) { return e == hipSuccess ? SQ_OK : SQ_E_HIP; }

// Scratch of the allocation-free forward: one copy per device, part of the
// code object's zero-initialised data, held until the process ends.  In host
// code its name is a host-side stand-in; the device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) uint8_t scratch[SQ_FWD_STATIC_SCRATCH_BYTES];
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

sq_status_t scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SQ_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SQ_E_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SQ_OK;
}

}  // namespace

extern "C" {

int sq_abi_version(void) { return SQ_ABI_VERSION; }

const char* sq_status_str(sq_status_t s) {
  switch (s) {
    case SQ_OK: return "ok";
    case SQ_E_NULL: return "a required pointer is NULL";
    case SQ_E_SHAPE:
      return "bad shape: need K % 256 == 0, K >= 256, N >= 1, M >= 0 (input gradient: N % 64 == 0)";
    case SQ_E_GROUP: return "group must be 32 or 64";
    case SQ_E_RANK: return "rank must be 0, 32 or 64 (int8 mode: 0, 16, 32 or 64; reserved 0)";
    case SQ_E_ALIGN: return "every pointer must be 16-byte aligned";
    case SQ_E_WORKSPACE: return "workspace smaller than the entry point's *_workspace_bytes()";
    case SQ_E_DTYPE: return "output dtype must be SQ_F32 or SQ_BF16";
    case SQ_E_ARCH: return "the current device is not gfx950 (MI355X)";
    case SQ_E_HIP: return "a HIP runtime call or kernel launch failed";
  }
  return "unknown status";
}

sq_status_t sq_quantize_weight(const float* w, const sq_w4_t* p, uint8_t* fidx,
                               int32_t* dev_flags, void* stream) {
  sq_status_t st = check_payload(p, true);
  if (st != SQ_OK) return st;
  if (!w || !dev_flags) return SQ_E_NULL;
  if (!aligned16(w) || (fidx && !aligned16(fidx)) || !aligned16(dev_flags)) return SQ_E_ALIGN;
  if ((st = check_device()) != SQ_OK) return st;
  return from_hip(sq::launch_quantize(w, p->lora_up, p->lora_down, p->codes, p->scales, fidx,
                                      dev_flags, p->n, p->k, p->group, p->rank,
                                      static_cast<hipStream_t>(stream)));
}

static sq::FwdPlan make_fwd_plan(int64_t m, const sq_w4_t* p) {
  if (sq::decode_eligible(m, p->n, p->k, p->rank))
    return sq::plan_decode(m, p->n, p->k, p->group, p->rank);
  return sq::plan_fwd(m, p->n, p->k, p->group, p->rank);
}

size_t sq_linear_fwd_workspace_bytes(int64_t m, const sq_w4_t* p) {
  if (!p || m <= 0 || p->k < 256 || p->k % 256 || p->n < 1) return 0;
  return make_fwd_plan(m, p).total;
}

static sq_status_t check_fwd(int64_t m, const sq_w4_t* p, void* workspace, size_t ws_bytes,
                             sq::FwdPlan* plan) {
  sq_status_t st = check_payload(p, true);
  if (st != SQ_OK) return st;
  if (m < 0) return SQ_E_SHAPE;
  if (m == 0) return SQ_OK;
  if (!workspace) return SQ_E_NULL;
  if (!aligned16(workspace)) return SQ_E_ALIGN;
  *plan = make_fwd_plan(m, p);
  if (ws_bytes < plan->total) return SQ_E_WORKSPACE;
  return SQ_OK;
}

sq_status_t sq_linear_fwd_rotate(const uint16_t* x, int64_t m, const sq_w4_t* p, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  sq::FwdPlan plan{};
  sq_status_t st = check_fwd(m, p, workspace, workspace_bytes, &plan);
  if (st != SQ_OK || m == 0) return st;
  if (!x) return SQ_E_NULL;
  if (!aligned16(x)) return SQ_E_ALIGN;
  if ((st = check_device()) != SQ_OK) return st;
  if (plan.dec)
    return from_hip(sq::launch_decode_prep(plan, x, p->lora_down, workspace,
                                           static_cast<hipStream_t>(stream)));
  return from_hip(sq::launch_fwd_rotate(plan, x, p->lora_down, workspace,
                                        static_cast<hipStream_t>(stream)));
}

sq_status_t sq_linear_fwd_contract(int64_t m, const sq_w4_t* p, void* y, sq_dtype_t y_dtype,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  sq::FwdPlan plan{};
  if (y_dtype != SQ_F32 && y_dtype != SQ_BF16) return SQ_E_DTYPE;
  sq_status_t st = check_fwd(m, p, workspace, workspace_bytes, &plan);
  if (st != SQ_OK || m == 0) return st;
  if (!y) return SQ_E_NULL;
  if (!aligned16(y)) return SQ_E_ALIGN;
  if ((st = check_device()) != SQ_OK) return st;
  if (plan.dec)
    return from_hip(sq::launch_decode_contract(plan, nullptr, nullptr, p->codes, p->scales,
                                               p->lora_up, y, y_dtype == SQ_BF16, workspace,
                                               static_cast<hipStream_t>(stream)));
  return from_hip(sq::launch_fwd_contract(plan, p->codes, p->scales, p->lora_up, y,
                                          y_dtype == SQ_BF16, workspace,
                                          static_cast<hipStream_t>(stream)));
}

sq_status_t sq_linear_fwd(const uint16_t* x, int64_t m, const sq_w4_t* p, void* y,
                          sq_dtype_t y_dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (y_dtype != SQ_F32 && y_dtype != SQ_BF16) return SQ_E_DTYPE;
  sq::FwdPlan plan{};
  sq_status_t st = check_fwd(m, p, workspace, workspace_bytes, &plan);
  if (st != SQ_OK || m == 0) return st;
  if (!x || !y) return SQ_E_NULL;
  if (!aligned16(x) || !aligned16(y)) return SQ_E_ALIGN;
  if ((st = check_device()) != SQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (plan.dec)
    return from_hip(sq::launch_decode_contract(plan, x, p->lora_down, p->codes, p->scales,
                                               p->lora_up, y, y_dtype == SQ_BF16, workspace, s));
  if ((st = from_hip(sq::launch_fwd_rotate(plan, x, p->lora_down, workspace, s))) != SQ_OK)
    return st;
  return from_hip(sq::launch_fwd_contract(plan, p->codes, p->scales, p->lora_up, y,
                                          y_dtype == SQ_BF16, workspace, s));
}

sq_status_t sq_linear_fwd_static(const uint16_t* x, int64_t m, const sq_w4_t* p, void* y,
                                 sq_dtype_t y_dtype, void* stream) {
  if (y_dtype != SQ_F32 && y_dtype != SQ_BF16) return SQ_E_DTYPE;
  sq_status_t st = check_payload(p, true);
  if (st != SQ_OK) return st;
  if (m < 0) return SQ_E_SHAPE;
  if (m == 0) return SQ_OK;
  if (!x || !y) return SQ_E_NULL;
  if (!aligned16(x) || !aligned16(y)) return SQ_E_ALIGN;
  const sq::FwdPlan plan = make_fwd_plan(m, p);
  if (plan.total > SQ_FWD_STATIC_SCRATCH_BYTES) return SQ_E_WORKSPACE;
  if ((st = check_device()) != SQ_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != SQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (plan.dec)
    return from_hip(sq::launch_decode_contract(plan, x, p->lora_down, p->codes, p->scales,
                                               p->lora_up, y, y_dtype == SQ_BF16, ws, s));
  if ((st = from_hip(sq::launch_fwd_rotate(plan, x, p->lora_down, ws, s))) != SQ_OK) return st;
  return from_hip(sq::launch_fwd_contract(plan, p->codes, p->scales, p->lora_up, y,
                                          y_dtype == SQ_BF16, ws, s));
}

size_t sq_linear_dgrad_workspace_bytes(int64_t m, const sq_w4_t* p) {
  if (!p || m <= 0 || p->k < 256 || p->k % 256 || p->n < 64 || p->n % 64) return 0;
  if (p->rank != 0 && p->rank != 32 && p->rank != 64) return 0;
  return sq::plan_dgrad(m, p->n, p->k, p->group, p->rank).total;
}

sq_status_t sq_linear_dgrad(const uint16_t* dy, int64_t m, const sq_w4_t* p, void* dx,
                            sq_dtype_t dx_dtype, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (dx_dtype != SQ_F32 && dx_dtype != SQ_BF16) return SQ_E_DTYPE;
  sq_status_t st = check_payload(p, true);
  if (st != SQ_OK) return st;
  if (m < 0 || p->n % 64 != 0) return SQ_E_SHAPE;
  if (m == 0) return SQ_OK;
  if (!dy || !dx || !workspace) return SQ_E_NULL;
  if (!aligned16(dy) || !aligned16(dx) || !aligned16(workspace)) return SQ_E_ALIGN;
  const sq::DgradPlan plan = sq::plan_dgrad(m, p->n, p->k, p->group, p->rank);
  if (workspace_bytes < plan.total) return SQ_E_WORKSPACE;
  if ((st = check_device()) != SQ_OK) return st;
  return from_hip(sq::launch_dgrad(plan, dy, p->codes, p->scales, p->lora_up, p->lora_down, dx,
                                   dx_dtype == SQ_BF16, workspace,
                                   static_cast<hipStream_t>(stream)));
}

sq_status_t sq_reconstruct_bf16(const sq_w4_t* p, uint16_t* w_hat, void* stream) {
  sq_status_t st = check_payload(p, true);
  if (st != SQ_OK) return st;
  if (!w_hat) return SQ_E_NULL;
  if (!aligned16(w_hat)) return SQ_E_ALIGN;
  if ((st = check_device()) != SQ_OK) return st;
  return from_hip(sq::launch_reconstruct(p->codes, p->scales, p->lora_up, p->lora_down, w_hat,
                                         p->n, p->k, p->group, p->rank,
                                         static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- int8-residual mode
size_t sq_quantize_weight_w8_workspace_bytes(const sq_w8_t* p) {
  if (!p || p->k < 256 || p->k % 256 || p->n < 1) return 0;
  return sq::quantize_w8_workspace(p->n, p->k);
}

sq_status_t sq_quantize_weight_w8(const float* w, const sq_w8_t* p, uint8_t* fidx,
                                  int32_t* dev_flags, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  sq_status_t st = check_payload_w8(p);
  if (st != SQ_OK) return st;
  if (!w || !dev_flags || !workspace) return SQ_E_NULL;
  if (!aligned16(w) || (fidx && !aligned16(fidx)) || !aligned16(dev_flags) ||
      !aligned16(workspace))
    return SQ_E_ALIGN;
  if (workspace_bytes < sq::quantize_w8_workspace(p->n, p->k)) return SQ_E_WORKSPACE;
  if ((st = check_device()) != SQ_OK) return st;
  return from_hip(sq::launch_quantize_w8(w, p->lora_up, p->lora_down, p->codes, p->scales, fidx,
                                         dev_flags, p->n, p->k, p->rank, workspace,
                                         static_cast<hipStream_t>(stream)));
}

sq_status_t sq_reconstruct_bf16_w8(const sq_w8_t* p, uint16_t* w_hat, void* stream) {
  sq_status_t st = check_payload_w8(p);
  if (st != SQ_OK) return st;
  if (!w_hat) return SQ_E_NULL;
  if (!aligned16(w_hat)) return SQ_E_ALIGN;
  if ((st = check_device()) != SQ_OK) return st;
  return from_hip(sq::launch_reconstruct(reinterpret_cast<const uint8_t*>(p->codes), p->scales,
                                         p->lora_up, p->lora_down, w_hat, p->n, p->k, 0, p->rank,
                                         static_cast<hipStream_t>(stream)));
}

// group 0 selects the int8 payload in the forward kernels
static sq::FwdPlan make_fwd_plan_w8(int64_t m, const sq_w8_t* p) {
  if (sq::decode_eligible(m, p->n, p->k, p->rank, true))
    return sq::plan_decode(m, p->n, p->k, 0, p->rank);
  return sq::plan_fwd(m, p->n, p->k, 0, p->rank);
}

size_t sq_linear_fwd_w8_workspace_bytes(int64_t m, const sq_w8_t* p) {
  if (!p || m <= 0 || p->k < 256 || p->k % 256 || p->n < 1) return 0;
  return make_fwd_plan_w8(m, p).total;
}

sq_status_t sq_linear_fwd_w8(const uint16_t* x, int64_t m, const sq_w8_t* p, void* y,
                             sq_dtype_t y_dtype, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (y_dtype != SQ_F32 && y_dtype != SQ_BF16) return SQ_E_DTYPE;
  sq_status_t st = check_payload_w8(p);
  if (st != SQ_OK) return st;
  if (m < 0) return SQ_E_SHAPE;
  if (m == 0) return SQ_OK;
  if (!x || !y || !workspace) return SQ_E_NULL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(workspace)) return SQ_E_ALIGN;
  const sq::FwdPlan plan = make_fwd_plan_w8(m, p);
  if (workspace_bytes < plan.total) return SQ_E_WORKSPACE;
  if ((st = check_device()) != SQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (plan.dec)
    return from_hip(sq::launch_decode_contract(
        plan, x, p->lora_down, reinterpret_cast<const uint8_t*>(p->codes), p->scales, p->lora_up,
        y, y_dtype == SQ_BF16, workspace, s));
  if ((st = from_hip(sq::launch_fwd_rotate(plan, x, p->lora_down, workspace, s))) != SQ_OK)
    return st;
  return from_hip(sq::launch_fwd_contract(plan, reinterpret_cast<const uint8_t*>(p->codes),
                                          p->scales, p->lora_up, y, y_dtype == SQ_BF16, workspace,
                                          s));
}

// ---------------------------------------------------------------- MXFP4 mode
sq_status_t sq_quantize_weight_mx4(const float* w, const sq_mx4_t* p, int32_t* dev_flags,
                                   void* stream) {
  sq_status_t st = check_payload_mx(p);
  if (st != SQ_OK) return st;
  if (!w || !dev_flags) return SQ_E_NULL;
  if (!aligned16(w) || !aligned16(dev_flags)) return SQ_E_ALIGN;
  if ((st = check_device()) != SQ_OK) return st;
  return from_hip(sq::launch_quantize_mx(w, p->lora_up, p->lora_down, p->codes, p->exps, dev_flags,
                                         p->n, p->k, p->rank, static_cast<hipStream_t>(stream)));
}

sq_status_t sq_quantize_act_mx4(const uint16_t* x, int64_t m, int64_t k, uint8_t* xq, uint8_t* xs,
                                void* stream) {
  if (m < 0 || k < 256 || k % 256 != 0) return SQ_E_SHAPE;
  if (m == 0) return SQ_OK;
  if (!x || !xq || !xs) return SQ_E_NULL;
  if (!aligned16(x) || !aligned16(xq) || !aligned16(xs)) return SQ_E_ALIGN;
  sq_status_t st = check_device();
  if (st != SQ_OK) return st;
  return from_hip(sq::launch_quantize_act_mx(x, m, k, xq, xs, static_cast<hipStream_t>(stream)));
}

sq_status_t sq_reconstruct_bf16_mx4(const sq_mx4_t* p, uint16_t* w_hat, void* stream) {
  sq_status_t st = check_payload_mx(p);
  if (st != SQ_OK) return st;
  if (!w_hat) return SQ_E_NULL;
  if (!aligned16(w_hat)) return SQ_E_ALIGN;
  if ((st = check_device()) != SQ_OK) return st;
  return from_hip(sq::launch_reconstruct_mx(p->codes, p->exps, p->lora_up, p->lora_down, w_hat,
                                            p->n, p->k, p->rank,
                                            static_cast<hipStream_t>(stream)));
}

size_t sq_linear_fwd_mx4_workspace_bytes(int64_t m, const sq_mx4_t* p) {
  if (!p || m <= 0 || p->k < 256 || p->k % 256 || p->n < 1) return 0;
  return sq::plan_mx(m, p->n, p->k, p->rank).total;
}

sq_status_t sq_linear_fwd_mx4(const uint16_t* x, int64_t m, const sq_mx4_t* p, void* y,
                              sq_dtype_t y_dtype, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (y_dtype != SQ_F32 && y_dtype != SQ_BF16) return SQ_E_DTYPE;
  sq_status_t st = check_payload_mx(p);
  if (st != SQ_OK) return st;
  if (m < 0) return SQ_E_SHAPE;
  if (m == 0) return SQ_OK;
  if (!x || !y || !workspace) return SQ_E_NULL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(workspace)) return SQ_E_ALIGN;
  const sq::MxPlan plan = sq::plan_mx(m, p->n, p->k, p->rank);
  if (workspace_bytes < plan.total) return SQ_E_WORKSPACE;
  if ((st = check_device()) != SQ_OK) return st;
  return from_hip(sq::launch_fwd_mx(plan, x, p->codes, p->exps, p->lora_up, p->lora_down, y,
                                    y_dtype == SQ_BF16, workspace,
                                    static_cast<hipStream_t>(stream)));
}

}  // extern "C"
