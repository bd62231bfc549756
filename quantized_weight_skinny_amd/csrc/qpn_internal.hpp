// Host-side declarations shared between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qpn {

// Launch plan of one GEMM call: the K range is cut into `split` pieces of
// `units_per_split` 256-element units (except for the first `whole_groups`
// groups of n-tiles, which take all of K in one workgroup); each workgroup of
// `waves` wavefronts handles `waves / k_slices` n-tiles of one piece. split > 1
// writes fp32 partial sums to the workspace; the last workgroup of a group to
// finish adds them in piece order.
struct LaunchOverride {
  int split = 0, waves = 0, depth = 0, k_slices = 0;  // 0 = automatic
  int epilogue = 0;  // 0: y[M, N]; 1: SwiGLU (h[M, N/2]); 2: greedy argmax per row
  int x_stage = 0;   // 0 automatic; kStageFull; kStageRing
  int whole_groups = 0;  // with split > 1: leading n-tile groups kept whole (not split)
  int valu_dot = 0;      // 1: the VALU packed-dot path instead of the MFMA
  int block_cols = 0;    // one activation row, NVFP4: 0 automatic (on), 1 on, 2 off
};

constexpr int kStageFull = 1;  // the workgroup's whole K range of x staged before the stream
constexpr int kStageRing = 2;  // a three-unit ring per K slice, refilled alongside the stream

struct GemmPlan {
  int split;
  int waves;
  int k_slices;    // wavefronts of a workgroup that split one n-tile's K range
  int dot_rows;    // 0: MFMA; 1, 2 or 4: the VALU packed-dot path for up to that many rows
  int block_cols;  // 1: MFMA output columns carry K-blocks (one activation row, NVFP4, full stage)
  int depth;       // units of the weight stream each wavefront keeps in flight
  int epilogue;    // 0 y[M, N]; 1 h[M, N/2] = silu(y[:, :N/2]) * y[:, N/2:]; 2 argmax of each row
  int x_stage;     // kStageFull or kStageRing
  int whole_groups;  // split > 1: the first whole_groups groups of n-tiles take all of K
  int units_per_split;
  int lds_stride;  // halves per staged activation row (full stage)
  size_t lds_bytes;
  // Workspace: one split-K arrival counter per n-tile (padded to 256 bytes),
  // a control block (the argmax epilogue's 64 x 16 key slots, 8 KiB), then
  // fp32 partials [split][m][n] from partials_offset (split > 1). 0 bytes
  // when neither split-K nor the argmax epilogue needs it.
  size_t control_offset;
  size_t partials_offset;
  size_t workspace_bytes;
};

bool plan_gemm(int fmt, int64_t n, int64_t k, int m, const LaunchOverride& o, GemmPlan* plan);

// y: fp16 output (or int32 indices for the argmax epilogue); val: the
// argmax epilogue's fp32 max logits (may be null).
hipError_t launch_gemm(int fmt, const GemmPlan& plan, const void* x, const void* packed,
                       const float* row_scales, float tensor_scale, void* y, float* val, void* workspace,
                       int m, int64_t n, int64_t k, hipStream_t stream);

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
