// Host-side argument checks of the C ABI declared in include/qpn.h. Plain C++
// with no HIP types, so that the checks also build with the host compiler
// alone (the sanitizer test builds them with g++ -fsanitize=address,undefined
// and drives them with arbitrary arguments; pointers are only compared and
// tested for alignment, never dereferenced).
//
// Each check_* returns the status the entry point reports when the check
// fails (QPN_OK when it passes) and sets *run to whether a passing call has
// work to launch: an empty problem passes with *run == false.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/qpn.h"
#include "qpn_plan.hpp"

namespace qpn {

bool aligned(const void* p, uintptr_t a);

qpn_status check_weight(const qpn_weight* w);

// The caller's launch request as a planner override (false: a field is out of
// its documented range). A null request is the automatic launch.
bool to_override(const qpn_launch* l, LaunchOverride* o);

qpn_status check_pack_nvfp4(const uint8_t* codes, const uint8_t* block_scales, int64_t n, int64_t k,
                            const void* packed, size_t packed_bytes, const int32_t* bad_codes, bool* run);
qpn_status check_pack_fp8(const uint8_t* codes, int64_t n, int64_t k, const void* packed, size_t packed_bytes,
                          const int32_t* bad_codes, bool* run);
qpn_status check_unpack_nvfp4(const void* packed, size_t packed_bytes, int64_t n, int64_t k, const uint8_t* codes,
                              const uint8_t* block_scales, bool* run);
qpn_status check_unpack_fp8(const void* packed, size_t packed_bytes, int64_t n, int64_t k, const uint8_t* codes,
                            bool* run);
qpn_status check_absmax_f32(const float* x, int64_t count, const float* out, bool* run);
qpn_status check_quantize_nvfp4(const float* w, int64_t n, int64_t k, float tensor_scale, const uint8_t* codes,
                                const uint8_t* block_scales, bool* run);
qpn_status check_quantize_fp8(const float* w, int64_t n, int64_t k, const uint8_t* codes, const float* row_scales,
                              bool* run);
qpn_status check_fp8_absmax(const uint8_t* codes, const float* row_scales, int64_t n, int64_t k, const float* out,
                            bool* run);
qpn_status check_requantize_fp8_nvfp4(const uint8_t* fp8_codes, const float* row_scales, int64_t n, int64_t k,
                                      float tensor_scale, const uint8_t* codes, const uint8_t* block_scales,
                                      bool* run);
qpn_status check_read_ceiling(const void* buf, size_t bytes, const uint32_t* sink, int32_t grid, int32_t loads,
                              bool* run);

// One GEMM call with planner override o (y is the fp16 output, fp32 for the
// F32 epilogue, the int32 indices for the argmax epilogue with the fp32
// values in val). On success with *run, *plan holds the launch.
qpn_status check_gemm(const void* x, const qpn_weight* w, const void* y, const float* val, int32_t m,
                      const void* workspace, size_t workspace_bytes, const LaunchOverride& o, GemmPlan* plan,
                      bool* run);

// The fused MLP call: plan (*plan) and checks as for qpn_mlp.
bool to_mlp_override(const qpn_mlp_launch* l, MlpOverride* o);
qpn_status check_mlp(const void* x, const qpn_weight* up, const qpn_weight* down, const void* h, const void* y,
                     int32_t m, const void* workspace, size_t workspace_bytes, const MlpOverride& o, MlpPlan* plan,
                     bool* run);

}  // namespace qpn
