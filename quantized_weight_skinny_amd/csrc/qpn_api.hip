// C ABI of libqpn.so (declared in include/qpn.h): the argument checks of
// qpn_checks.cpp on the host, then kernel launches on the caller's stream.
// Every check runs before the first HIP call, so a rejected call touches
// neither the device nor the stream.
#include "../../include/qpn.h"

#include <mutex>

#include "qpn_checks.hpp"
#include "qpn_device.hpp"
#include "qpn_internal.hpp"

namespace {

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

qpn_status from_hip(hipError_t e) { return e == hipSuccess ? QPN_OK : QPN_ERR_HIP; }

// Pack's validation: the counter is cleared, the pack kernels add the invalid
// codes they meet, and the count is read back after the stream has drained,
// so the call reports them itself (QPN_ERR_BAD_CODE) and a GEMM is never
// handed a weight with them.
template <typename Launch>
qpn_status pack_checked(int32_t* bad_codes_dev, hipStream_t s, Launch launch) {
  if (hipMemsetAsync(bad_codes_dev, 0, sizeof(int32_t), s) != hipSuccess) return QPN_ERR_HIP;
  if (launch() != hipSuccess) return QPN_ERR_HIP;
  int32_t bad = 0;
  if (hipMemcpyAsync(&bad, bad_codes_dev, sizeof bad, hipMemcpyDeviceToHost, s) != hipSuccess) return QPN_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return QPN_ERR_HIP;
  return bad ? QPN_ERR_BAD_CODE : QPN_OK;
}

// One GEMM call with launch override o: y_dev is the fp16 output (fp32 for
// the F32 epilogue; for the argmax epilogue the int32 indices, with the fp32
// values in val_dev).
qpn_status gemm_call(const void* x_dev, const qpn_weight* w, void* y_dev, float* val_dev, int32_t m,
                     void* workspace_dev, size_t workspace_bytes, const qpn::LaunchOverride& o, void* stream) {
  qpn::GemmPlan p;
  bool run = false;
  const qpn_status st = qpn::check_gemm(x_dev, w, y_dev, val_dev, m, workspace_dev, workspace_bytes, o, &p, &run);
  if (st != QPN_OK || !run) return st;
  return from_hip(qpn::launch_gemm(w->format, p, x_dev, w->packed, w->row_scales, w->tensor_scale, y_dev, val_dev,
                                   workspace_dev, m, w->n, w->k, as_stream(stream)));
}

// The no-allocation variant's scratch: one array per GPU the library runs on,
// holding the split-K arrival counters (zero at load; every call leaves them
// zero) and the fp32 partial sums. In host code `scratch` only names the
// symbol: its device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is handed on.
static __device__ __align__(256) unsigned char scratch[QPN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

qpn_status scratch_for_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QPN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return QPN_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return QPN_OK;
}

}  // namespace

extern "C" {

qpn_status qpn_pack_nvfp4(const uint8_t* codes_dev, const uint8_t* block_scales_dev, int64_t n,
                          int64_t k, void* packed_dev, size_t packed_bytes, int32_t* bad_codes_dev,
                          void* stream) {
  bool run = false;
  const qpn_status st =
      qpn::check_pack_nvfp4(codes_dev, block_scales_dev, n, k, packed_dev, packed_bytes, bad_codes_dev, &run);
  if (st != QPN_OK || !run) return st;
  const hipStream_t s = as_stream(stream);
  return pack_checked(bad_codes_dev, s, [&] {
    return qpn::launch_pack_nvfp4(codes_dev, block_scales_dev, n, k, packed_dev, bad_codes_dev, s);
  });
}

qpn_status qpn_pack_fp8(const uint8_t* codes_dev, int64_t n, int64_t k, void* packed_dev,
                        size_t packed_bytes, int32_t* bad_codes_dev, void* stream) {
  bool run = false;
  const qpn_status st = qpn::check_pack_fp8(codes_dev, n, k, packed_dev, packed_bytes, bad_codes_dev, &run);
  if (st != QPN_OK || !run) return st;
  const hipStream_t s = as_stream(stream);
  return pack_checked(bad_codes_dev, s,
                      [&] { return qpn::launch_pack_fp8(codes_dev, n, k, packed_dev, bad_codes_dev, s); });
}

qpn_status qpn_unpack_nvfp4(const void* packed_dev, size_t packed_bytes, int64_t n, int64_t k,
                            uint8_t* codes_dev, uint8_t* block_scales_dev, void* stream) {
  bool run = false;
  const qpn_status st =
      qpn::check_unpack_nvfp4(packed_dev, packed_bytes, n, k, codes_dev, block_scales_dev, &run);
  if (st != QPN_OK || !run) return st;
  return from_hip(qpn::launch_unpack_nvfp4(packed_dev, n, k, codes_dev, block_scales_dev, as_stream(stream)));
}

qpn_status qpn_unpack_fp8(const void* packed_dev, size_t packed_bytes, int64_t n, int64_t k,
                          uint8_t* codes_dev, void* stream) {
  bool run = false;
  const qpn_status st = qpn::check_unpack_fp8(packed_dev, packed_bytes, n, k, codes_dev, &run);
  if (st != QPN_OK || !run) return st;
  return from_hip(qpn::launch_unpack_fp8(packed_dev, n, k, codes_dev, as_stream(stream)));
}

qpn_status qpn_absmax_f32(const float* x_dev, int64_t count, float* out_dev, void* stream) {
  bool run = false;
  const qpn_status st = qpn::check_absmax_f32(x_dev, count, out_dev, &run);
  if (st != QPN_OK || !run) return st;
  return from_hip(qpn::launch_absmax(x_dev, count, out_dev, as_stream(stream)));
}

qpn_status qpn_quantize_nvfp4(const float* w_dev, int64_t n, int64_t k, float tensor_scale,
                              uint8_t* codes_dev, uint8_t* block_scales_dev, void* stream) {
  bool run = false;
  const qpn_status st = qpn::check_quantize_nvfp4(w_dev, n, k, tensor_scale, codes_dev, block_scales_dev, &run);
  if (st != QPN_OK || !run) return st;
  return from_hip(qpn::launch_quantize_nvfp4(w_dev, n, k, tensor_scale, codes_dev, block_scales_dev,
                                             as_stream(stream)));
}

qpn_status qpn_quantize_fp8(const float* w_dev, int64_t n, int64_t k, uint8_t* codes_dev,
                            float* row_scales_dev, void* stream) {
  bool run = false;
  const qpn_status st = qpn::check_quantize_fp8(w_dev, n, k, codes_dev, row_scales_dev, &run);
  if (st != QPN_OK || !run) return st;
  return from_hip(qpn::launch_quantize_fp8(w_dev, n, k, codes_dev, row_scales_dev, as_stream(stream)));
}

qpn_status qpn_fp8_absmax(const uint8_t* codes_dev, const float* row_scales_dev, int64_t n, int64_t k,
                          float* out_dev, void* stream) {
  bool run = false;
  const qpn_status st = qpn::check_fp8_absmax(codes_dev, row_scales_dev, n, k, out_dev, &run);
  if (st != QPN_OK || !run) return st;
  return from_hip(qpn::launch_fp8_absmax(codes_dev, row_scales_dev, n, k, out_dev, as_stream(stream)));
}

qpn_status qpn_requantize_fp8_nvfp4(const uint8_t* fp8_codes_dev, const float* row_scales_dev, int64_t n,
                                    int64_t k, float tensor_scale, uint8_t* codes_dev, uint8_t* block_scales_dev,
                                    void* stream) {
  bool run = false;
  const qpn_status st = qpn::check_requantize_fp8_nvfp4(fp8_codes_dev, row_scales_dev, n, k, tensor_scale,
                                                        codes_dev, block_scales_dev, &run);
  if (st != QPN_OK || !run) return st;
  return from_hip(qpn::launch_requantize_fp8_nvfp4(fp8_codes_dev, row_scales_dev, n, k, tensor_scale, codes_dev,
                                                   block_scales_dev, as_stream(stream)));
}

qpn_status qpn_gemm_tuned(const void* x_dev, const qpn_weight* w, void* y_dev, int32_t m,
                          void* workspace_dev, size_t workspace_bytes, const qpn_launch* launch,
                          void* stream) {
  qpn::LaunchOverride o;
  if (!qpn::to_override(launch, &o)) return QPN_ERR_INVALID_ARG;
  if (o.epilogue == QPN_EPILOGUE_ARGMAX) return QPN_ERR_INVALID_ARG;  // two outputs: qpn_gemm_argmax
  return gemm_call(x_dev, w, y_dev, nullptr, m, workspace_dev, workspace_bytes, o, stream);
}

qpn_status qpn_gemm_argmax(const void* x_dev, const qpn_weight* w, int32_t* idx_dev, float* val_dev, int32_t m,
                           void* workspace_dev, size_t workspace_bytes, const qpn_launch* launch, void* stream) {
  qpn::LaunchOverride o;
  if (!qpn::to_override(launch, &o)) return QPN_ERR_INVALID_ARG;
  if (o.epilogue != QPN_EPILOGUE_NONE && o.epilogue != QPN_EPILOGUE_ARGMAX) return QPN_ERR_INVALID_ARG;
  o.epilogue = QPN_EPILOGUE_ARGMAX;
  return gemm_call(x_dev, w, idx_dev, val_dev, m, workspace_dev, workspace_bytes, o, stream);
}

qpn_status qpn_gemm(const void* x_dev, const qpn_weight* w, void* y_dev, int32_t m,
                    void* workspace_dev, size_t workspace_bytes, void* stream) {
  return qpn_gemm_tuned(x_dev, w, y_dev, m, workspace_dev, workspace_bytes, nullptr, stream);
}

qpn_status qpn_gemm_noalloc(const void* x_dev, const qpn_weight* w, void* y_dev, int32_t m, void* stream) {
  const qpn_status st = qpn::check_weight(w);
  if (st != QPN_OK) return st;
  if (m < 0 || m > QPN_MAX_M) return QPN_ERR_INVALID_ARG;
  if (m == 0 || w->n == 0) return QPN_OK;
  qpn::GemmPlan p;
  if (!qpn::plan_gemm(w->format, w->n, w->k, m, qpn::LaunchOverride{}, &p)) return QPN_ERR_UNSUPPORTED;
  if (p.workspace_bytes > QPN_NOALLOC_SCRATCH_BYTES) return QPN_ERR_BUFFER_TOO_SMALL;
  void* ws = nullptr;
  if (p.workspace_bytes) {
    const qpn_status s2 = scratch_for_current_device(&ws);
    if (s2 != QPN_OK) return s2;
  }
  return gemm_call(x_dev, w, y_dev, nullptr, m, ws, p.workspace_bytes ? QPN_NOALLOC_SCRATCH_BYTES : 0,
                   qpn::LaunchOverride{}, stream);
}

qpn_status qpn_mlp(const void* x_dev, const qpn_weight* gate_up, const qpn_weight* down, void* h_dev, void* y_dev,
                   int32_t m, void* workspace_dev, size_t workspace_bytes, const qpn_mlp_launch* launch,
                   int32_t* launches, void* stream) {
  qpn::MlpOverride o;
  if (!qpn::to_mlp_override(launch, &o)) return QPN_ERR_INVALID_ARG;
  qpn::MlpPlan p;
  bool run = false;
  const qpn_status st =
      qpn::check_mlp(x_dev, gate_up, down, h_dev, y_dev, m, workspace_dev, workspace_bytes, o, &p, &run);
  if (launches) *launches = 0;
  if (st != QPN_OK || !run) return st;
  const qpn::WeightRef up{gate_up->format, gate_up->packed, gate_up->row_scales, gate_up->tensor_scale, gate_up->n,
                          gate_up->k};
  const qpn::WeightRef dn{down->format, down->packed, down->row_scales, down->tensor_scale, down->n, down->k};
  int n = 0;
  const hipError_t e = qpn::launch_mlp(p, up, dn, x_dev, h_dev, y_dev, workspace_dev, m, as_stream(stream), &n);
  if (launches) *launches = n;
  if (e == hipErrorCooperativeLaunchTooLarge) return QPN_ERR_UNSUPPORTED;
  return from_hip(e);
}

qpn_status qpn_gemm_swiglu(const void* x_dev, const qpn_weight* w, void* h_dev, int32_t m,
                           void* workspace_dev, size_t workspace_bytes, void* stream) {
  qpn_launch l{};
  l.epilogue = QPN_EPILOGUE_SWIGLU;
  return qpn_gemm_tuned(x_dev, w, h_dev, m, workspace_dev, workspace_bytes, &l, stream);
}

qpn_status qpn_gemm_f32(const void* x_dev, const qpn_weight* w, float* y_dev, int32_t m,
                        void* workspace_dev, size_t workspace_bytes, void* stream) {
  qpn_launch l{};
  l.epilogue = QPN_EPILOGUE_F32;
  return qpn_gemm_tuned(x_dev, w, y_dev, m, workspace_dev, workspace_bytes, &l, stream);
}

int32_t qpn_read_ceiling_grid(void) { return qpn::read_ceiling_default_grid(); }

qpn_status qpn_read_ceiling(const void* buf_dev, size_t bytes, uint32_t* sink_dev, int32_t grid, int32_t loads,
                            void* stream) {
  bool run = false;
  const qpn_status st = qpn::check_read_ceiling(buf_dev, bytes, sink_dev, grid, loads, &run);
  if (st != QPN_OK || !run) return st;
  const int g = grid ? grid : qpn::read_ceiling_default_grid();
  return from_hip(qpn::launch_read_ceiling(buf_dev, bytes, sink_dev, g, loads ? loads : 4, as_stream(stream)));
}

}  // extern "C"
