// Host-side declarations shared between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "qpn_plan.hpp"

namespace qpn {

// Allow `fn` dynamic LDS up to `bytes` on the current device. The attribute
// belongs to the device, so it is set once per kernel and device: `done` (one
// per kernel) records devices 0..63; any other device sets it on every call.
// A failed call is not recorded and is tried again next time.
inline hipError_t allow_dynamic_lds(const void* fn, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t(1) << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  const hipError_t set = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (set == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return set;
}


// y: fp16 output (or int32 indices for the argmax epilogue); val: the
// argmax epilogue's fp32 max logits (may be null).
hipError_t launch_gemm(int fmt, const GemmPlan& plan, const void* x, const void* packed,
                       const float* row_scales, float tensor_scale, void* y, float* val, void* workspace,
                       int m, int64_t n, int64_t k, hipStream_t stream);

// A weight as the launchers take it.
struct WeightRef {
  int fmt;
  const void* packed;
  const float* row_scales;
  float tensor_scale;
  int64_t n, k;
};

// The MLP of plan p: h = SwiGLU(x W_up^T) (fp16 [m][up.n / 2]) and
// y = h W_dn^T (fp16 [m][dn.n]); one launch when the plan allows it and its
// grid fits on the device at once, else the two GEMMs (unless p asks for one
// launch: then hipErrorCooperativeLaunchTooLarge, nothing enqueued).
// *launches (may be null) gets the number of launches enqueued.
hipError_t launch_mlp(const MlpPlan& p, const WeightRef& up, const WeightRef& dn, const void* x, void* h, void* y,
                      void* workspace, int m, hipStream_t stream, int* launches);

hipError_t launch_pack_nvfp4(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                             void* packed, int32_t* bad, hipStream_t stream);
hipError_t launch_pack_fp8(const uint8_t* codes, int64_t n, int64_t k, void* packed,
                           int32_t* bad, hipStream_t stream);
hipError_t launch_unpack_nvfp4(const void* packed, int64_t n, int64_t k, uint8_t* codes,
                               uint8_t* scales, hipStream_t stream);
hipError_t launch_unpack_fp8(const void* packed, int64_t n, int64_t k, uint8_t* codes,
                             hipStream_t stream);
hipError_t launch_absmax(const float* x, int64_t count, float* out, hipStream_t stream);
hipError_t launch_quantize_nvfp4(const float* w, int64_t n, int64_t k, float tensor_scale,
                                 uint8_t* codes, uint8_t* scales, hipStream_t stream);
hipError_t launch_quantize_fp8(const float* w, int64_t n, int64_t k, uint8_t* codes,
                               float* row_scales, hipStream_t stream);
hipError_t launch_fp8_absmax(const uint8_t* codes, const float* row_scales, int64_t n, int64_t k, float* out,
                             hipStream_t stream);
hipError_t launch_requantize_fp8_nvfp4(const uint8_t* f8, const float* row_scales, int64_t n, int64_t k,
                                       float tensor_scale, uint8_t* codes, uint8_t* scales, hipStream_t stream);
hipError_t launch_read_ceiling(const void* buf, size_t bytes, uint32_t* sink, int grid, int loads,
                               hipStream_t stream);
int read_ceiling_default_grid();

}  // namespace qpn
