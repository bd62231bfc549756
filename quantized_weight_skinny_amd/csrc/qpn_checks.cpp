// Host-side argument checks (declared in qpn_checks.hpp) and the entry points
// of include/qpn.h that need no device: status strings, sizes and launch plans.
#include "qpn_checks.hpp"

#include <math.h>

namespace qpn {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

qpn_status check_weight(const qpn_weight* w) {
  if (!w || w->reserved != 0) return QPN_ERR_INVALID_ARG;
  if (w->format != QPN_FMT_NVFP4 && w->format != QPN_FMT_FP8_E4M3) return QPN_ERR_INVALID_ARG;
  if (!shape_ok(w->n, w->k)) return QPN_ERR_INVALID_ARG;
  return QPN_OK;
}

bool to_override(const qpn_launch* l, LaunchOverride* o) {
  *o = LaunchOverride{};
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

qpn_status check_pack_nvfp4(const uint8_t* codes, const uint8_t* block_scales, int64_t n, int64_t k,
                            const void* packed, size_t packed_bytes, const int32_t* bad_codes, bool* run) {
  *run = false;
  if (!shape_ok(n, k)) return QPN_ERR_INVALID_ARG;
  const size_t need = qpn::packed_bytes(kFmtNvfp4, n, k);
  if (need == 0) return QPN_OK;
  if (!codes || !block_scales || !packed || !aligned(packed, 16)) return QPN_ERR_INVALID_ARG;
  if (!bad_codes || !aligned(bad_codes, 4)) return QPN_ERR_INVALID_ARG;
  if (packed_bytes < need) return QPN_ERR_BUFFER_TOO_SMALL;
  *run = true;
  return QPN_OK;
}

qpn_status check_pack_fp8(const uint8_t* codes, int64_t n, int64_t k, const void* packed, size_t packed_bytes,
                          const int32_t* bad_codes, bool* run) {
  *run = false;
  if (!shape_ok(n, k)) return QPN_ERR_INVALID_ARG;
  const size_t need = qpn::packed_bytes(kFmtFp8, n, k);
  if (need == 0) return QPN_OK;
  if (!codes || !packed || !aligned(packed, 16)) return QPN_ERR_INVALID_ARG;
  if (!bad_codes || !aligned(bad_codes, 4)) return QPN_ERR_INVALID_ARG;
  if (packed_bytes < need) return QPN_ERR_BUFFER_TOO_SMALL;
  *run = true;
  return QPN_OK;
}

qpn_status check_unpack_nvfp4(const void* packed, size_t packed_bytes, int64_t n, int64_t k, const uint8_t* codes,
                              const uint8_t* block_scales, bool* run) {
  *run = false;
  if (!shape_ok(n, k)) return QPN_ERR_INVALID_ARG;
  const size_t need = qpn::packed_bytes(kFmtNvfp4, n, k);
  if (need == 0) return QPN_OK;
  if (!packed || !codes || !block_scales || !aligned(packed, 16)) return QPN_ERR_INVALID_ARG;
  if (packed_bytes < need) return QPN_ERR_BUFFER_TOO_SMALL;
  *run = true;
  return QPN_OK;
}

qpn_status check_unpack_fp8(const void* packed, size_t packed_bytes, int64_t n, int64_t k, const uint8_t* codes,
                            bool* run) {
  *run = false;
  if (!shape_ok(n, k)) return QPN_ERR_INVALID_ARG;
  const size_t need = qpn::packed_bytes(kFmtFp8, n, k);
  if (need == 0) return QPN_OK;
  if (!packed || !codes || !aligned(packed, 16)) return QPN_ERR_INVALID_ARG;
  if (packed_bytes < need) return QPN_ERR_BUFFER_TOO_SMALL;
  *run = true;
  return QPN_OK;
}

qpn_status check_absmax_f32(const float* x, int64_t count, const float* out, bool* run) {
  *run = false;
  if (count < 0 || !out || !aligned(out, 4)) return QPN_ERR_INVALID_ARG;
  if (count > 0 && (!x || !aligned(x, 4))) return QPN_ERR_INVALID_ARG;
  *run = true;  // an empty input still writes 0
  return QPN_OK;
}

qpn_status check_quantize_nvfp4(const float* w, int64_t n, int64_t k, float tensor_scale, const uint8_t* codes,
                                const uint8_t* block_scales, bool* run) {
  *run = false;
  if (!shape_ok(n, k) || !isfinite(tensor_scale) || !(tensor_scale > 0.0f)) return QPN_ERR_INVALID_ARG;
  if (n == 0 || k == 0) return QPN_OK;
  if (!w || !codes || !block_scales || !aligned(w, 4)) return QPN_ERR_INVALID_ARG;
  *run = true;
  return QPN_OK;
}

qpn_status check_quantize_fp8(const float* w, int64_t n, int64_t k, const uint8_t* codes, const float* row_scales,
                              bool* run) {
  *run = false;
  if (!shape_ok(n, k)) return QPN_ERR_INVALID_ARG;
  if (n == 0) return QPN_OK;
  if (!row_scales || !aligned(row_scales, 4)) return QPN_ERR_INVALID_ARG;
  if (k > 0 && (!w || !codes || !aligned(w, 4))) return QPN_ERR_INVALID_ARG;
  *run = true;  // k == 0 still writes the row scales
  return QPN_OK;
}

qpn_status check_fp8_absmax(const uint8_t* codes, const float* row_scales, int64_t n, int64_t k, const float* out,
                            bool* run) {
  *run = false;
  if (!shape_ok(n, k) || !out || !aligned(out, 4)) return QPN_ERR_INVALID_ARG;
  if (n > 0 && k > 0 && (!codes || !row_scales || !aligned(row_scales, 4))) return QPN_ERR_INVALID_ARG;
  *run = true;  // an empty weight still writes 0
  return QPN_OK;
}

qpn_status check_requantize_fp8_nvfp4(const uint8_t* fp8_codes, const float* row_scales, int64_t n, int64_t k,
                                      float tensor_scale, const uint8_t* codes, const uint8_t* block_scales,
                                      bool* run) {
  *run = false;
  if (!shape_ok(n, k) || !isfinite(tensor_scale) || !(tensor_scale > 0.f)) return QPN_ERR_INVALID_ARG;
  if (n == 0 || k == 0) return QPN_OK;
  if (!fp8_codes || !row_scales || !codes || !block_scales || !aligned(row_scales, 4)) return QPN_ERR_INVALID_ARG;
  *run = true;
  return QPN_OK;
}

qpn_status check_read_ceiling(const void* buf, size_t bytes, const uint32_t* sink, int32_t grid, int32_t loads,
                              bool* run) {
  *run = false;
  if (!buf || !sink || !aligned(buf, 16) || bytes % 16 || grid < 0) return QPN_ERR_INVALID_ARG;
  if (loads != 0 && loads != 2 && loads != 4 && loads != 8) return QPN_ERR_INVALID_ARG;
  *run = bytes != 0;
  return QPN_OK;
}

qpn_status check_gemm(const void* x, const qpn_weight* w, const void* y, const float* val, int32_t m,
                      const void* workspace, size_t workspace_bytes, const LaunchOverride& o, GemmPlan* plan,
                      bool* run) {
  *run = false;
  const qpn_status st = check_weight(w);
  if (st != QPN_OK) return st;
  if (m < 0 || m > QPN_MAX_M) return QPN_ERR_INVALID_ARG;
  if (o.waves != 0 && o.waves != 4 && o.waves != 8 && o.waves != kUnevenWaves) return QPN_ERR_INVALID_ARG;
  if (o.depth != 0 && o.depth != 2 && o.depth != 3 && o.depth != 4 && o.depth != 6 && o.depth != 8)
    return QPN_ERR_INVALID_ARG;
  if (o.k_slices != 0 && o.k_slices != 1 && o.k_slices != 2 && o.k_slices != 4 && o.k_slices != 8)
    return QPN_ERR_INVALID_ARG;
  if (o.epilogue == QPN_EPILOGUE_SWIGLU && w->n % 32) return QPN_ERR_INVALID_ARG;
  if (m == 0 || w->n == 0) return QPN_OK;
  const uintptr_t out_align = o.epilogue == QPN_EPILOGUE_ARGMAX || o.epilogue == QPN_EPILOGUE_F32 ? 4 : 2;
  if (!y || !aligned(y, out_align)) return QPN_ERR_INVALID_ARG;
  if (val && !aligned(val, 4)) return QPN_ERR_INVALID_ARG;
  if (w->k > 0) {
    if (!x || !aligned(x, 16)) return QPN_ERR_INVALID_ARG;
    if (!w->packed || !aligned(w->packed, 16)) return QPN_ERR_INVALID_ARG;
  }
  if (w->format == QPN_FMT_NVFP4 && !isfinite(w->tensor_scale)) return QPN_ERR_INVALID_ARG;
  if (w->format == QPN_FMT_FP8_E4M3 && (!w->row_scales || !aligned(w->row_scales, 4))) return QPN_ERR_INVALID_ARG;
  if (!plan_gemm(w->format, w->n, w->k, m, o, plan)) return QPN_ERR_UNSUPPORTED;
  if (plan->workspace_bytes) {
    if (!workspace || !aligned(workspace, 16)) return QPN_ERR_INVALID_ARG;
    if (workspace_bytes < plan->workspace_bytes) return QPN_ERR_BUFFER_TOO_SMALL;
  }
  *run = true;
  return QPN_OK;
}

bool to_mlp_override(const qpn_mlp_launch* l, MlpOverride* o) {
  *o = MlpOverride{};
  if (!l) return true;
  if (l->reserved != 0 || l->fused < 0 || l->fused > 2 || l->stream_after < -1) return false;
  if (l->down_depth != 0 && l->down_depth != 2 && l->down_depth != 3 && l->down_depth != 4 && l->down_depth != 6 &&
      l->down_depth != 8)
    return false;
  o->fused = l->fused;
  o->down_depth = l->down_depth;
  o->stream_after = l->stream_after;
  return true;
}

qpn_status check_mlp(const void* x, const qpn_weight* up, const qpn_weight* down, const void* h, const void* y,
                     int32_t m, const void* workspace, size_t workspace_bytes, const MlpOverride& o, MlpPlan* plan,
                     bool* run) {
  *run = false;
  qpn_status st = check_weight(up);
  if (st != QPN_OK) return st;
  st = check_weight(down);
  if (st != QPN_OK) return st;
  if (m < 0 || m > QPN_MAX_M) return QPN_ERR_INVALID_ARG;
  if (up->n % 32 || down->k != up->n / 2) return QPN_ERR_INVALID_ARG;
  if (m == 0 || up->n == 0 || down->n == 0) return QPN_OK;
  if (!h || !aligned(h, 16) || !y || !aligned(y, 2)) return QPN_ERR_INVALID_ARG;
  if (up->k > 0 && (!x || !aligned(x, 16))) return QPN_ERR_INVALID_ARG;
  const qpn_weight* const both[2] = {up, down};
  for (const qpn_weight* w : both) {
    if (w->k > 0 && (!w->packed || !aligned(w->packed, 16))) return QPN_ERR_INVALID_ARG;
    if (w->format == QPN_FMT_NVFP4 && !isfinite(w->tensor_scale)) return QPN_ERR_INVALID_ARG;
    if (w->format == QPN_FMT_FP8_E4M3 && (!w->row_scales || !aligned(w->row_scales, 4))) return QPN_ERR_INVALID_ARG;
  }
  if (!plan_mlp(up->format, up->n, up->k, down->format, down->n, down->k, m, o, plan)) return QPN_ERR_UNSUPPORTED;
  if (!workspace || !aligned(workspace, 16)) return QPN_ERR_INVALID_ARG;
  if (workspace_bytes < plan->workspace_bytes) return QPN_ERR_BUFFER_TOO_SMALL;
  *run = true;
  return QPN_OK;
}

}  // namespace qpn

extern "C" {

size_t qpn_mlp_workspace_bytes(const qpn_weight* gate_up, const qpn_weight* down, int32_t m,
                               const qpn_mlp_launch* launch) {
  if (qpn::check_weight(gate_up) != QPN_OK || qpn::check_weight(down) != QPN_OK || m < 1 || m > QPN_MAX_M)
    return 0;
  if (gate_up->n % 32 || down->k != gate_up->n / 2 || gate_up->n == 0 || down->n == 0) return 0;
  qpn::MlpOverride o;
  if (!qpn::to_mlp_override(launch, &o)) return 0;
  qpn::MlpPlan p;
  if (!qpn::plan_mlp(gate_up->format, gate_up->n, gate_up->k, down->format, down->n, down->k, m, o, &p)) return 0;
  return p.workspace_bytes;
}


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

size_t qpn_packed_bytes(int32_t format, int64_t n, int64_t k) { return qpn::packed_bytes(format, n, k); }

float qpn_nvfp4_tensor_scale(float amax) {
  const float s = amax / 2688.0f;
  return s == 0.0f ? 1.0f : s;
}

size_t qpn_workspace_bytes_tuned(const qpn_weight* w, int32_t m, const qpn_launch* launch) {
  if (qpn::check_weight(w) != QPN_OK || m < 0 || m > QPN_MAX_M) return 0;
  if (m == 0 || w->n == 0) return 0;
  qpn::LaunchOverride o;
  if (!qpn::to_override(launch, &o)) return 0;
  qpn::GemmPlan p;
  if (!qpn::plan_gemm(w->format, w->n, w->k, m, o, &p)) return 0;
  return p.workspace_bytes;
}

size_t qpn_workspace_bytes(const qpn_weight* w, int32_t m) { return qpn_workspace_bytes_tuned(w, m, nullptr); }

qpn_status qpn_gemm_plan(const qpn_weight* w, int32_t m, const qpn_launch* launch, qpn_launch* resolved) {
  const qpn_status st = qpn::check_weight(w);
  if (st != QPN_OK) return st;
  if (!resolved || m < 1 || m > QPN_MAX_M || w->n == 0) return QPN_ERR_INVALID_ARG;
  qpn::LaunchOverride o;
  if (!qpn::to_override(launch, &o)) return QPN_ERR_INVALID_ARG;
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
