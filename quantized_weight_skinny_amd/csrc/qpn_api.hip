// C ABI of libqpn.so (declared in include/qpn.h): argument checks on the host,
// then kernel launches on the caller's stream. Every check runs before the
// first HIP call, so a rejected call touches neither the device nor the
// stream.
#include "../../include/qpn.h"

#include <math.h>

#include <mutex>

#include "qpn_device.hpp"
#include "qpn_internal.hpp"

using qpn::ceil_div;

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

qpn_status from_hip(hipError_t e) { return e == hipSuccess ? QPN_OK : QPN_ERR_HIP; }

bool shape_ok(int64_t n, int64_t k) {
  // n * k / 2 must stay addressable and the kernel indexes rows with int.
  return n >= 0 && k >= 0 && k % 16 == 0 && n <= (int64_t(1) << 31) - 16 &&
         k <= (int64_t(1) << 30);
}

qpn_status check_weight(const qpn_weight* w) {
  if (!w || w->reserved != 0) return QPN_ERR_INVALID_ARG;
  if (w->format != QPN_FMT_NVFP4 && w->format != QPN_FMT_FP8_E4M3) return QPN_ERR_INVALID_ARG;
  if (!shape_ok(w->n, w->k)) return QPN_ERR_INVALID_ARG;
  return QPN_OK;
}

}  // namespace

extern "C" {

const char* qpn_status_string(qpn_status s) {
  switch (s) {
    case QPN_OK: return "ok";
    case QPN_ERR_INVALID_ARG: return "invalid argument";
    case QPN_ERR_UNSUPPORTED: return "unsupported";
    case QPN_ERR_BAD_CODE: return "invalid code";
    case QPN_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case QPN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

size_t qpn_packed_bytes(int32_t format, int64_t n, int64_t k) {
  if (!shape_ok(n, k)) return 0;
  const int64_t units = ceil_div(n, qpn::kTileN) * ceil_div(k, qpn::kUnitK);
  if (format == QPN_FMT_NVFP4) return static_cast<size_t>(units) * qpn::kNvUnitBytes;
  if (format == QPN_FMT_FP8_E4M3) return static_cast<size_t>(units) * qpn::kF8UnitBytes;
  return 0;
}

}  // extern "C"

namespace {

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

}  // namespace

extern "C" {

qpn_status qpn_pack_nvfp4(const uint8_t* codes_dev, const uint8_t* block_scales_dev, int64_t n,
                          int64_t k, void* packed_dev, size_t packed_bytes, int32_t* bad_codes_dev,
                          void* stream) {
  if (!shape_ok(n, k)) return QPN_ERR_INVALID_ARG;
  const size_t need = qpn_packed_bytes(QPN_FMT_NVFP4, n, k);
  if (need == 0) return QPN_OK;
  if (!codes_dev || !block_scales_dev || !packed_dev || !aligned(packed_dev, 16))
    return QPN_ERR_INVALID_ARG;
  if (!bad_codes_dev || !aligned(bad_codes_dev, 4)) return QPN_ERR_INVALID_ARG;
  if (packed_bytes < need) return QPN_ERR_BUFFER_TOO_SMALL;
  const hipStream_t s = as_stream(stream);
  return pack_checked(bad_codes_dev, s, [&] {
    return qpn::launch_pack_nvfp4(codes_dev, block_scales_dev, n, k, packed_dev, bad_codes_dev, s);
  });
}

qpn_status qpn_pack_fp8(const uint8_t* codes_dev, int64_t n, int64_t k, void* packed_dev,
                        size_t packed_bytes, int32_t* bad_codes_dev, void* stream) {
  if (!shape_ok(n, k)) return QPN_ERR_INVALID_ARG;
  const size_t need = qpn_packed_bytes(QPN_FMT_FP8_E4M3, n, k);
  if (need == 0) return QPN_OK;
  if (!codes_dev || !packed_dev || !aligned(packed_dev, 16)) return QPN_ERR_INVALID_ARG;
  if (!bad_codes_dev || !aligned(bad_codes_dev, 4)) return QPN_ERR_INVALID_ARG;
  if (packed_bytes < need) return QPN_ERR_BUFFER_TOO_SMALL;
  const hipStream_t s = as_stream(stream);
  return pack_checked(bad_codes_dev, s,
                      [&] { return qpn::launch_pack_fp8(codes_dev, n, k, packed_dev, bad_codes_dev, s); });
}

qpn_status qpn_unpack_nvfp4(const void* packed_dev, size_t packed_bytes, int64_t n, int64_t k,
                            uint8_t* codes_dev, uint8_t* block_scales_dev, void* stream) {
  if (!shape_ok(n, k)) return QPN_ERR_INVALID_ARG;
  const size_t need = qpn_packed_bytes(QPN_FMT_NVFP4, n, k);
  if (need == 0) return QPN_OK;
  if (!packed_dev || !codes_dev || !block_scales_dev || !aligned(packed_dev, 16))
    return QPN_ERR_INVALID_ARG;
  if (packed_bytes < need) return QPN_ERR_BUFFER_TOO_SMALL;
  return from_hip(qpn::launch_unpack_nvfp4(packed_dev, n, k, codes_dev, block_scales_dev,
                                           as_stream(stream)));
}

qpn_status qpn_unpack_fp8(const void* packed_dev, size_t packed_bytes, int64_t n, int64_t k,
                          uint8_t* codes_dev, void* stream) {
  if (!shape_ok(n, k)) return QPN_ERR_INVALID_ARG;
  const size_t need = qpn_packed_bytes(QPN_FMT_FP8_E4M3, n, k);
  if (need == 0) return QPN_OK;
  if (!packed_dev || !codes_dev || !aligned(packed_dev, 16)) return QPN_ERR_INVALID_ARG;
  if (packed_bytes < need) return QPN_ERR_BUFFER_TOO_SMALL;
  return from_hip(qpn::launch_unpack_fp8(packed_dev, n, k, codes_dev, as_stream(stream)));
}

qpn_status qpn_absmax_f32(const float* x_dev, int64_t count, float* out_dev, void* stream) {
  if (count < 0 || !out_dev || !aligned(out_dev, 4)) return QPN_ERR_INVALID_ARG;
  if (count > 0 && (!x_dev || !aligned(x_dev, 4))) return QPN_ERR_INVALID_ARG;
  return from_hip(qpn::launch_absmax(x_dev, count, out_dev, as_stream(stream)));
}

float qpn_nvfp4_tensor_scale(float amax) {
  const float s = amax / 2688.0f;
  return s == 0.0f ? 1.0f : s;
}

qpn_status qpn_quantize_nvfp4(const float* w_dev, int64_t n, int64_t k, float tensor_scale,
                              uint8_t* codes_dev, uint8_t* block_scales_dev, void* stream) {
  if (!shape_ok(n, k) || !isfinite(tensor_scale) || !(tensor_scale > 0.0f)) return QPN_ERR_INVALID_ARG;
  if (n == 0 || k == 0) return QPN_OK;
  if (!w_dev || !codes_dev || !block_scales_dev || !aligned(w_dev, 4)) return QPN_ERR_INVALID_ARG;
  return from_hip(qpn::launch_quantize_nvfp4(w_dev, n, k, tensor_scale, codes_dev, block_scales_dev,
                                             as_stream(stream)));
}

qpn_status qpn_quantize_fp8(const float* w_dev, int64_t n, int64_t k, uint8_t* codes_dev,
                            float* row_scales_dev, void* stream) {
  if (!shape_ok(n, k)) return QPN_ERR_INVALID_ARG;
  if (n == 0) return QPN_OK;
  if (!row_scales_dev || !aligned(row_scales_dev, 4)) return QPN_ERR_INVALID_ARG;
  if (k > 0 && (!w_dev || !codes_dev || !aligned(w_dev, 4))) return QPN_ERR_INVALID_ARG;
  return from_hip(qpn::launch_quantize_fp8(w_dev, n, k, codes_dev, row_scales_dev, as_stream(stream)));
}

qpn_status qpn_fp8_absmax(const uint8_t* codes_dev, const float* row_scales_dev, int64_t n, int64_t k,
                          float* out_dev, void* stream) {
  if (!shape_ok(n, k) || !out_dev || !aligned(out_dev, 4)) return QPN_ERR_INVALID_ARG;
  if (n > 0 && k > 0 && (!codes_dev || !row_scales_dev || !aligned(row_scales_dev, 4)))
    return QPN_ERR_INVALID_ARG;
  return from_hip(qpn::launch_fp8_absmax(codes_dev, row_scales_dev, n, k, out_dev, as_stream(stream)));
}

qpn_status qpn_requantize_fp8_nvfp4(const uint8_t* fp8_codes_dev, const float* row_scales_dev, int64_t n,
                                    int64_t k, float tensor_scale, uint8_t* codes_dev, uint8_t* block_scales_dev,
                                    void* stream) {
  if (!shape_ok(n, k) || !isfinite(tensor_scale) || !(tensor_scale > 0.f)) return QPN_ERR_INVALID_ARG;
  if (n == 0 || k == 0) return QPN_OK;
  if (!fp8_codes_dev || !row_scales_dev || !codes_dev || !block_scales_dev || !aligned(row_scales_dev, 4))
    return QPN_ERR_INVALID_ARG;
  return from_hip(qpn::launch_requantize_fp8_nvfp4(fp8_codes_dev, row_scales_dev, n, k, tensor_scale, codes_dev,
                                                   block_scales_dev, as_stream(stream)));
}

namespace {

bool to_override(const qpn_launch* l, qpn::LaunchOverride* o) {
  if (!l) return true;
  if ((l->valu_dot != 0 && l->valu_dot != 1) || l->whole_groups < 0) return false;
  if (l->block_columns < 0 || l->block_columns > 2) return false;
  if (l->x_stage != QPN_X_STAGE_AUTO && l->x_stage != QPN_X_STAGE_FULL && l->x_stage != QPN_X_STAGE_RING)
    return false;
  if (l->split_k < 0 || l->waves_per_group < 0 || l->depth < 0 || l->k_slices < 0) return false;
  if (l->epilogue != QPN_EPILOGUE_NONE && l->epilogue != QPN_EPILOGUE_SWIGLU && l->epilogue != QPN_EPILOGUE_ARGMAX &&
      l->epilogue != QPN_EPILOGUE_F32)
    return false;
  o->split = l->split_k;
  o->waves = l->waves_per_group;
  o->depth = l->depth;
  o->k_slices = l->k_slices;
  o->epilogue = l->epilogue;
  o->x_stage = l->x_stage;
  o->whole_groups = l->whole_groups;
  o->valu_dot = l->valu_dot;
  o->block_cols = l->block_columns;
  return true;
}

}  // namespace

size_t qpn_workspace_bytes_tuned(const qpn_weight* w, int32_t m, const qpn_launch* launch) {
  if (check_weight(w) != QPN_OK || m < 0 || m > QPN_MAX_M) return 0;
  if (m == 0 || w->n == 0) return 0;
  qpn::LaunchOverride o;
  if (!to_override(launch, &o)) return 0;
  qpn::GemmPlan p;
  if (!qpn::plan_gemm(w->format, w->n, w->k, m, o, &p)) return 0;
  return p.workspace_bytes;
}

size_t qpn_workspace_bytes(const qpn_weight* w, int32_t m) { return qpn_workspace_bytes_tuned(w, m, nullptr); }

qpn_status qpn_gemm_plan(const qpn_weight* w, int32_t m, const qpn_launch* launch, qpn_launch* resolved) {
  const qpn_status st = check_weight(w);
  if (st != QPN_OK) return st;
  if (!resolved || m < 1 || m > QPN_MAX_M || w->n == 0) return QPN_ERR_INVALID_ARG;
  qpn::LaunchOverride o;
  if (!to_override(launch, &o)) return QPN_ERR_INVALID_ARG;
  qpn::GemmPlan p;
  if (!qpn::plan_gemm(w->format, w->n, w->k, m, o, &p)) return QPN_ERR_UNSUPPORTED;
  *resolved = qpn_launch{};
  resolved->split_k = p.split;
  resolved->waves_per_group = p.waves;
  resolved->depth = p.depth;
  resolved->k_slices = p.k_slices;
  resolved->epilogue = p.epilogue;
  resolved->x_stage = p.x_stage;
  resolved->whole_groups = p.whole_groups;
  resolved->valu_dot = p.dot_rows ? 1 : 0;
  resolved->block_columns = p.block_cols ? 1 : 2;
  return QPN_OK;
}

}  // extern "C"

namespace {

// One GEMM call with launch override o: y_dev is the fp16 output (fp32 for
// the F32 epilogue; for the argmax epilogue the int32 indices, with the fp32
// values in val_dev).
qpn_status gemm_call(const void* x_dev, const qpn_weight* w, void* y_dev, float* val_dev, int32_t m,
                     void* workspace_dev, size_t workspace_bytes, const qpn::LaunchOverride& o, void* stream) {
  const qpn_status st = check_weight(w);
  if (st != QPN_OK) return st;
  if (m < 0 || m > QPN_MAX_M) return QPN_ERR_INVALID_ARG;
  if (o.waves != 0 && o.waves != 4 && o.waves != 8) return QPN_ERR_INVALID_ARG;
  if (o.depth != 0 && o.depth != 2 && o.depth != 3 && o.depth != 4 && o.depth != 6 && o.depth != 8)
    return QPN_ERR_INVALID_ARG;
  if (o.k_slices != 0 && o.k_slices != 1 && o.k_slices != 2 && o.k_slices != 4 && o.k_slices != 8)
    return QPN_ERR_INVALID_ARG;
  if (o.epilogue == QPN_EPILOGUE_SWIGLU && w->n % 32) return QPN_ERR_INVALID_ARG;
  if (m == 0 || w->n == 0) return QPN_OK;
  const size_t out_align = o.epilogue == QPN_EPILOGUE_ARGMAX || o.epilogue == QPN_EPILOGUE_F32 ? 4 : 2;
  if (!y_dev || !aligned(y_dev, out_align)) return QPN_ERR_INVALID_ARG;
  if (val_dev && !aligned(val_dev, 4)) return QPN_ERR_INVALID_ARG;
  if (w->k > 0) {
    if (!x_dev || !aligned(x_dev, 16)) return QPN_ERR_INVALID_ARG;
    if (!w->packed || !aligned(w->packed, 16)) return QPN_ERR_INVALID_ARG;
  }
  if (w->format == QPN_FMT_NVFP4 && !isfinite(w->tensor_scale)) return QPN_ERR_INVALID_ARG;
  if (w->format == QPN_FMT_FP8_E4M3 && (!w->row_scales || !aligned(w->row_scales, 4)))
    return QPN_ERR_INVALID_ARG;
  qpn::GemmPlan p;
  if (!qpn::plan_gemm(w->format, w->n, w->k, m, o, &p)) return QPN_ERR_UNSUPPORTED;
  if (p.workspace_bytes) {
    if (!workspace_dev || !aligned(workspace_dev, 16)) return QPN_ERR_INVALID_ARG;
    if (workspace_bytes < p.workspace_bytes) return QPN_ERR_BUFFER_TOO_SMALL;
  }
  return from_hip(qpn::launch_gemm(w->format, p, x_dev, w->packed, w->row_scales, w->tensor_scale,
                                   y_dev, val_dev, workspace_dev, m, w->n, w->k, as_stream(stream)));
}

}  // namespace

extern "C" {

qpn_status qpn_gemm_tuned(const void* x_dev, const qpn_weight* w, void* y_dev, int32_t m,
                          void* workspace_dev, size_t workspace_bytes, const qpn_launch* launch,
                          void* stream) {
  qpn::LaunchOverride o;
  if (!to_override(launch, &o)) return QPN_ERR_INVALID_ARG;
  if (o.epilogue == QPN_EPILOGUE_ARGMAX) return QPN_ERR_INVALID_ARG;  // two outputs: qpn_gemm_argmax
  return gemm_call(x_dev, w, y_dev, nullptr, m, workspace_dev, workspace_bytes, o, stream);
}

qpn_status qpn_gemm_argmax(const void* x_dev, const qpn_weight* w, int32_t* idx_dev, float* val_dev, int32_t m,
                           void* workspace_dev, size_t workspace_bytes, const qpn_launch* launch, void* stream) {
  qpn::LaunchOverride o;
  if (!to_override(launch, &o)) return QPN_ERR_INVALID_ARG;
  if (o.epilogue != QPN_EPILOGUE_NONE && o.epilogue != QPN_EPILOGUE_ARGMAX) return QPN_ERR_INVALID_ARG;
  o.epilogue = QPN_EPILOGUE_ARGMAX;
  return gemm_call(x_dev, w, idx_dev, val_dev, m, workspace_dev, workspace_bytes, o, stream);
}

qpn_status qpn_gemm(const void* x_dev, const qpn_weight* w, void* y_dev, int32_t m,
                    void* workspace_dev, size_t workspace_bytes, void* stream) {
  return qpn_gemm_tuned(x_dev, w, y_dev, m, workspace_dev, workspace_bytes, nullptr, stream);
}

}  // extern "C"

namespace {

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

qpn_status qpn_gemm_noalloc(const void* x_dev, const qpn_weight* w, void* y_dev, int32_t m, void* stream) {
  const qpn_status st = check_weight(w);
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
  if (!buf_dev || !sink_dev || !aligned(buf_dev, 16) || bytes % 16 || grid < 0) return QPN_ERR_INVALID_ARG;
  if (loads != 0 && loads != 2 && loads != 4 && loads != 8) return QPN_ERR_INVALID_ARG;
  if (bytes == 0) return QPN_OK;
  const int g = grid ? grid : qpn::read_ceiling_default_grid();
  return from_hip(qpn::launch_read_ceiling(buf_dev, bytes, sink_dev, g, loads ? loads : 4, as_stream(stream)));
}

}  // extern "C"
