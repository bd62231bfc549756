// Skinny GEMM y[M, N] = x[M, K] * dequant(W)^T for M <= 16 fp16 rows and
// NVFP4 / FP8 weights streamed from HBM in the packed layout of qpn_device.hpp.
//
// [P3] "What I actually built" (https://reddlx.com/feed/productivity-ai-news,
// post "Four Tesla V100s from 2017 matched my RTX 5090 on single-request
// Qwen 3.8 decode"): weights stay compressed while read from HBM and each
// fragment is turned into the fp16 operand format of the matrix unit, with no
// dequantize-to-fp16 pass. On gfx950 the fragment is one dword of 8 E2M1
// codes (or two dwords of 8 E4M3 codes), converted with
// v_cvt_scalef32_pk_f16_fp{4,8}, multiplied by its fp16 block scale and fed
// as the A operand of v_mfma_f32_16x16x32_f16. The activation rows ride in
// the B operand (columns 0..M-1 of the 16-wide tile; the others repeat row
// M-1 and are never stored, since MFMA columns do not mix), so one
// instruction serves any M <= 16 and the verify rows of a speculative
// round cost no extra weight traffic (the 8-row tile of the post's Volta
// design becomes the 16-row MFMA tile here).
//
// Work split: each wavefront owns one 16-row n-tile and a contiguous range of
// 256-element K units. A workgroup holds neighbouring n-tiles of the same K
// range (cut into K slices, one per wavefront of a tile) and stages x into
// LDS, read back as one 16-byte ds_read_b128 per lane per MFMA: either the
// whole range before the weight stream starts, or a ring of three units per
// slice refilled alongside the stream (a much smaller stage, so that large M
// keeps its occupancy and needs no K split). Loads of DEPTH units are kept in
// flight per wavefront. When K is cut into several ranges the fp32 partial
// tiles go to a workspace and the last workgroup of each group of n-tiles to
// finish adds them in range order, which keeps the result deterministic and
// needs no second kernel. The epilogue scales the sums and rounds them once
// to fp16 (or keeps them fp32), or fuses SwiGLU or a greedy argmax.
#include "qpn_gemm_body.hpp"

namespace qpn {
namespace {

template <int FMT, int WAVES, int DEPTH, int EPI, int XP, int DOT>
__global__ __launch_bounds__(WAVES * 64) void gemm_kernel(
    const _Float16* x, const uint8_t* packed, const float* __restrict__ row_scales, float tensor_scale,
    void* __restrict__ y, float* __restrict__ ws, int* __restrict__ counters, ArgmaxOut amax, int M, int N, int K,
    int NT, int KU, int ups, int stride, int KS, int groups, int whole, int split) {
  gemm_body<FMT, WAVES, DEPTH, EPI, XP, DOT, 0>(x, packed, row_scales, tensor_scale, y, ws, counters, amax, M, N, K,
                                               NT, KU, ups, stride, KS, groups, whole, split,
                                               static_cast<int>(blockIdx.x), FuseCtl{});
}

// After the argmax GEMM on the same stream: thread (m, sub) reads and clears
// key slot (sub, m) (device-scope loads and stores: the slots were written by
// device-scope atomics from every XCD); the largest key of each row gives
// its index and value.
__global__ __launch_bounds__(kArgmaxSubs* kMaxM) void argmax_decode_kernel(unsigned long long* keys, int M,
                                                                          int* idx, float* val) {
  __shared__ unsigned long long best[kMaxM];
  const int t = threadIdx.x;
  if (t < M) best[t] = 0;
  __syncthreads();
  const int m = t / kArgmaxSubs, sub = t % kArgmaxSubs;
  if (m < M) {
    unsigned long long* slot = keys + sub * kMaxM + m;
    const unsigned long long k = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(slot, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_max(&best[m], k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __syncthreads();
  if (t < M) {
    int n;
    float v;
    argmax_decode(best[t], &n, &v);
    idx[t] = n;
    if (val) val[t] = v;
  }
}

template <int FMT, int WAVES, int DEPTH, int EPI, int XP, int DOT = 0>
hipError_t launch_kernel(const GemmPlan& p, const void* x, const void* packed, const float* row_scales,
                      float tensor_scale, void* y, float* val, void* workspace, int m, int64_t n, int64_t k,
                      hipStream_t stream) {
  const int NT = static_cast<int>(ceil_div(n, kTileN));
  const int KU = static_cast<int>(ceil_div(k, kUnitK));
  const int groups = static_cast<int>(ceil_div(NT, WAVES / p.k_slices));
  // groups that take all of K (the uneven grid: its workgroups, all of them)
  const int whole = WAVES == kUnevenWaves || p.split > 1 ? p.whole_groups : groups;
  const unsigned grid = static_cast<unsigned>(whole + (groups - whole) * (p.split > 1 ? p.split : 0));
  if (WAVES == kUnevenWaves && (p.k_slices != 1 || p.split != 1 || whole < 1 || whole > NT ||
                                ceil_div(NT, whole) > kUnevenWaves))
    return hipErrorInvalidValue;
  // Dynamic LDS above the 64 KiB default must be allowed per kernel and device.
  static std::atomic<uint64_t> lds_allowed{0};
  const hipError_t attr = allow_dynamic_lds(
      reinterpret_cast<const void*>(&gemm_kernel<FMT, WAVES, DEPTH, EPI, XP, DOT>), static_cast<int>(kLdsBudget),
      lds_allowed);
  if (attr != hipSuccess) return attr;
  char* wsb = static_cast<char*>(workspace);
  int* counters = p.split > 1 ? reinterpret_cast<int*>(wsb) : nullptr;
  float* ws = p.split > 1 ? reinterpret_cast<float*>(wsb + p.partials_offset) : nullptr;
  ArgmaxOut amax{nullptr, nullptr, nullptr};
  if (EPI == kEpiArgmax) {
    amax.keys = reinterpret_cast<unsigned long long*>(wsb + p.control_offset);
    amax.idx = static_cast<int*>(y);
    amax.val = val;
  }
  hipLaunchKernelGGL((gemm_kernel<FMT, WAVES, DEPTH, EPI, XP, DOT>), dim3(grid), dim3(WAVES * 64), p.lds_bytes, stream,
                     static_cast<const _Float16*>(x), static_cast<const uint8_t*>(packed), row_scales,
                     tensor_scale, y, ws, counters, amax, m, static_cast<int>(n),
                     static_cast<int>(k), NT, KU, p.units_per_split, p.lds_stride, p.k_slices, groups, whole,
                     p.split);
  if constexpr (EPI == kEpiArgmax) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(argmax_decode_kernel, dim3(1), dim3(kArgmaxSubs * kMaxM), 0, stream, amax.keys, m,
                       amax.idx, amax.val);
  }
  return hipGetLastError();
}

template <int FMT, int WAVES, int DEPTH, int EPI>
hipError_t launch_cfg_e(const GemmPlan& p, const void* x, const void* packed, const float* row_scales,
                        float tensor_scale, void* y, float* val, void* workspace, int m, int64_t n, int64_t k,
                        hipStream_t stream) {
  if constexpr (EPI == kEpiNone && DEPTH <= 4) {
    // The packed-dot path (full stage, plain epilogue, depths 2..4).
    if (p.dot_rows && p.x_stage == kStageFull) {
      switch (p.dot_rows) {
        case 1:
          return launch_kernel<FMT, WAVES, DEPTH, EPI, 0, 1>(p, x, packed, row_scales, tensor_scale, y, val,
                                                             workspace, m, n, k, stream);
        case 2:
          return launch_kernel<FMT, WAVES, DEPTH, EPI, 0, 2>(p, x, packed, row_scales, tensor_scale, y, val,
                                                             workspace, m, n, k, stream);
        case 4:
          return launch_kernel<FMT, WAVES, DEPTH, EPI, 0, 4>(p, x, packed, row_scales, tensor_scale, y, val,
                                                             workspace, m, n, k, stream);
        default:
          return hipErrorInvalidValue;
      }
    }
  }
  if (p.dot_rows) return hipErrorInvalidValue;
  if (p.block_cols) {
    if constexpr (FMT == kFmtNvfp4)
      return launch_kernel<FMT, WAVES, DEPTH, EPI, 0, kDotBlockCols>(p, x, packed, row_scales, tensor_scale, y, val,
                                                                     workspace, m, n, k, stream);
    return hipErrorInvalidValue;
  }
  if (p.x_stage == kStageFull)
    return launch_kernel<FMT, WAVES, DEPTH, EPI, 0>(p, x, packed, row_scales, tensor_scale, y, val, workspace, m,
                                                    n, k, stream);
  // The ring stage is built for depths 2..4 (the planner allows no other).
  if constexpr (DEPTH <= 4) {
    switch (ring_pieces(WAVES, p.k_slices, m)) {
      case 1:
        return launch_kernel<FMT, WAVES, DEPTH, EPI, 1>(p, x, packed, row_scales, tensor_scale, y, val, workspace,
                                                        m, n, k, stream);
      case 2:
        return launch_kernel<FMT, WAVES, DEPTH, EPI, 2>(p, x, packed, row_scales, tensor_scale, y, val, workspace,
                                                        m, n, k, stream);
      default:
        break;
    }
  }
  return hipErrorInvalidValue;
}

template <int FMT, int WAVES, int DEPTH>
hipError_t launch_cfg(const GemmPlan& p, const void* x, const void* packed, const float* row_scales,
                      float tensor_scale, void* y, float* val, void* workspace, int m, int64_t n, int64_t k,
                      hipStream_t stream) {
  switch (p.epilogue) {
    case kEpiSwiglu:
      return launch_cfg_e<FMT, WAVES, DEPTH, kEpiSwiglu>(p, x, packed, row_scales, tensor_scale, y, val,
                                                          workspace, m, n, k, stream);
    case kEpiArgmax:
      return launch_cfg_e<FMT, WAVES, DEPTH, kEpiArgmax>(p, x, packed, row_scales, tensor_scale, y, val,
                                                          workspace, m, n, k, stream);
    case kEpiF32:
      return launch_cfg_e<FMT, WAVES, DEPTH, kEpiF32>(p, x, packed, row_scales, tensor_scale, y, val,
                                                       workspace, m, n, k, stream);
    default:
      return launch_cfg_e<FMT, WAVES, DEPTH, kEpiNone>(p, x, packed, row_scales, tensor_scale, y, val,
                                                        workspace, m, n, k, stream);
  }
}

template <int FMT, int WAVES>
hipError_t launch_depth(const GemmPlan& p, const void* x, const void* packed, const float* row_scales,
                        float tensor_scale, void* y, float* val, void* workspace, int m, int64_t n, int64_t k,
                        hipStream_t stream) {
  switch (p.depth) {
    case 2: return launch_cfg<FMT, WAVES, 2>(p, x, packed, row_scales, tensor_scale, y, val, workspace, m, n, k, stream);
    case 3: return launch_cfg<FMT, WAVES, 3>(p, x, packed, row_scales, tensor_scale, y, val, workspace, m, n, k, stream);
    case 6: return launch_cfg<FMT, WAVES, 6>(p, x, packed, row_scales, tensor_scale, y, val, workspace, m, n, k, stream);
    case 8: return launch_cfg<FMT, WAVES, 8>(p, x, packed, row_scales, tensor_scale, y, val, workspace, m, n, k, stream);
    default: return launch_cfg<FMT, WAVES, 4>(p, x, packed, row_scales, tensor_scale, y, val, workspace, m, n, k, stream);
  }
}

// The uneven-group grid (NVFP4, fp16 or fp32 y, MFMA, depths 2 and 3).
template <int EPI>
hipError_t launch_uneven_e(const GemmPlan& p, const void* x, const void* packed, float tensor_scale, void* y,
                           int m, int64_t n, int64_t k, hipStream_t stream) {
  constexpr int W = kUnevenWaves;
  const bool ring = p.x_stage == kStageRing;
  if (ring && ring_pieces(W, 1, m) != 1) return hipErrorInvalidValue;
  switch (p.depth) {
    case 2:
      return ring ? launch_kernel<kFmtNvfp4, W, 2, EPI, 1>(p, x, packed, nullptr, tensor_scale, y, nullptr, nullptr,
                                                           m, n, k, stream)
                  : launch_kernel<kFmtNvfp4, W, 2, EPI, 0>(p, x, packed, nullptr, tensor_scale, y, nullptr, nullptr,
                                                           m, n, k, stream);
    case 3:
      return ring ? launch_kernel<kFmtNvfp4, W, 3, EPI, 1>(p, x, packed, nullptr, tensor_scale, y, nullptr, nullptr,
                                                           m, n, k, stream)
                  : launch_kernel<kFmtNvfp4, W, 3, EPI, 0>(p, x, packed, nullptr, tensor_scale, y, nullptr, nullptr,
                                                           m, n, k, stream);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_uneven(const GemmPlan& p, const void* x, const void* packed, float tensor_scale, void* y, int m,
                         int64_t n, int64_t k, hipStream_t stream) {
  if (p.dot_rows || p.block_cols) return hipErrorInvalidValue;
  if (p.epilogue == kEpiNone) return launch_uneven_e<kEpiNone>(p, x, packed, tensor_scale, y, m, n, k, stream);
  if (p.epilogue == kEpiF32) return launch_uneven_e<kEpiF32>(p, x, packed, tensor_scale, y, m, n, k, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(int fmt, const GemmPlan& p, const void* x, const void* packed,
                       const float* row_scales, float tensor_scale, void* y, float* val, void* workspace,
                       int m, int64_t n, int64_t k, hipStream_t stream) {
  if (p.waves == kUnevenWaves)
    return fmt == kFmtNvfp4 ? launch_uneven(p, x, packed, tensor_scale, y, m, n, k, stream) : hipErrorInvalidValue;
  if (fmt == kFmtNvfp4) {
    return p.waves == 8 ? launch_depth<kFmtNvfp4, 8>(p, x, packed, row_scales, tensor_scale, y, val,
                                                      workspace, m, n, k, stream)
                        : launch_depth<kFmtNvfp4, 4>(p, x, packed, row_scales, tensor_scale, y, val,
                                                      workspace, m, n, k, stream);
  }
  return p.waves == 8 ? launch_depth<kFmtFp8, 8>(p, x, packed, row_scales, tensor_scale, y, val,
                                                  workspace, m, n, k, stream)
                      : launch_depth<kFmtFp8, 4>(p, x, packed, row_scales, tensor_scale, y, val,
                                                  workspace, m, n, k, stream);
}

}  // namespace qpn
