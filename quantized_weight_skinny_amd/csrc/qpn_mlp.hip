// The MLP of a decoder layer in one launch: h = SwiGLU(x W_gu^T) and
// y = h W_dn^T, both weights NVFP4 in the packed layout (qpn_mlp with
// launch->fused = 1; its automatic form is the two GEMM launches).
//
// Two GEMM launches leave the chip part idle twice: at the end of gate_up,
// whose last workgroups finish several microseconds after the first, and at
// the start of down, which stages h before its stream gets going. Here the
// gate_up workgroups (producers) come first in the grid and the down
// workgroups (consumers) after them. A consumer's weights do not depend on h,
// so it issues its first units as soon as ctl.stream_after producers have
// finished, which puts the idle end of gate_up to work, and stages h (with
// device-coherent loads) only once every producer has counted itself in after
// its h stores (device-scope, written through to the level all XCDs share)
// were acknowledged. The producers whose arrival completes a stage raise a
// flag in each consumer's own line, which only that consumer polls. This is
// the dependency of the two GEMMs, with no extra pass over memory: the fusion
// of the SwiGLU epilogue between gate_up and down that the pages' layer
// structure implies ([P3] "What I actually built": the dense layer's gate_up
// and down projections).
//
// Measured on the 27B shapes (gate_up 34816 x 5120, down 5120 x 17408) it is
// level with the two launches (one row: 30.2 against 30.15 us; two rows:
// 30.66 against 30.97): the signal from the last producer takes 2.5-3 us to
// reach the consumers (its h stores acknowledged, its arrival returned, the
// flags raised and polled), about what the second launch and down's own
// start cost, and down's work after it (staging h, then 17 units per
// wavefront on 160 CUs) is no shorter for having its first units in flight.
// Polling one shared counter instead of per-consumer lines made the launch
// 50% slower; 32 counter replicas polled by a few consumers each were slower
// than the lines (31.9 us).
//
// Progress: the launcher requires that every workgroup of the grid be
// resident at once (the occupancy of this kernel times the CUs), so the
// producers never wait for a slot that a waiting consumer holds, whatever the
// dispatch order; the waits are bounded besides (fuse_wait). The last
// producer resets the arrival counter and each consumer its own flags, so
// the control block is zero again for the next call.
#include "qpn_gemm_body.hpp"

#include <mutex>

namespace qpn {
namespace {

// One half of the launch: the arguments of gemm_body.
struct HalfArgs {
  const _Float16* x;
  const uint8_t* packed;
  const float* row_scales;
  float tensor_scale;
  void* y;
  float* ws;
  int* counters;
  int M, N, K, NT, KU, ups, stride, KS, groups, whole, split;
};

static_assert(kFuseFlagInts * sizeof(int) == kMlpFlagLineBytes, "one flag line per consumer");

// Raise flag `which` (0 stream, 1 go) in every consumer's line.
__device__ __forceinline__ void fuse_raise(const FuseCtl& ctl, int which) {
  for (int c = threadIdx.x; c < ctl.consumers; c += kMlpWaves * 64)
    __hip_atomic_store(ctl.flags + static_cast<size_t>(c) * kFuseFlagInts + which, 1, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__shared__ int fuse_arrival;

template <int FMT, int DA, int XPA, int DB>
__global__ __launch_bounds__(kMlpWaves * 64) void mlp_kernel(HalfArgs a, HalfArgs b, FuseCtl ctl) {
  if (static_cast<int>(blockIdx.x) < ctl.producers) {
    gemm_body<FMT, kMlpWaves, DA, kEpiSwiglu, XPA, 0, 1>(
        a.x, a.packed, a.row_scales, a.tensor_scale, a.y, a.ws, a.counters, ArgmaxOut{}, a.M, a.N, a.K, a.NT, a.KU,
        a.ups, a.stride, a.KS, a.groups, a.whole, a.split, static_cast<int>(blockIdx.x), ctl);
    // Count this producer in once every h store of the workgroup (and any
    // split-K partial) has been acknowledged at the device-coherent level;
    // the arrival that completes a stage raises its flag for every consumer.
    // (Each earlier producer's stores were acknowledged before its own
    // arrival, which came before this one's.) The last producer also resets
    // the counter: every producer has counted itself in.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
      fuse_arrival = __hip_atomic_fetch_add(ctl.produced, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
    __syncthreads();
    const int arrived = fuse_arrival;
    if (arrived == ctl.stream_after) fuse_raise(ctl, 0);
    if (arrived == ctl.producers) {
      fuse_raise(ctl, 1);
      if (threadIdx.x == 0) __hip_atomic_store(ctl.produced, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
    gemm_body<FMT, kMlpWaves, DB, kEpiNone, 0, 0, 2>(
        b.x, b.packed, b.row_scales, b.tensor_scale, b.y, b.ws, b.counters, ArgmaxOut{}, b.M, b.N, b.K, b.NT, b.KU,
        b.ups, b.stride, b.KS, b.groups, b.whole, b.split, static_cast<int>(blockIdx.x) - ctl.producers, ctl);
  }
}

HalfArgs half_args(const GemmPlan& p, const WeightRef& w, const void* x, void* y, char* ws, int m) {
  HalfArgs h;
  h.x = static_cast<const _Float16*>(x);
  h.packed = static_cast<const uint8_t*>(w.packed);
  h.row_scales = w.row_scales;
  h.tensor_scale = w.tensor_scale;
  h.y = y;
  h.ws = p.split > 1 ? reinterpret_cast<float*>(ws + p.partials_offset) : nullptr;
  h.counters = p.split > 1 ? reinterpret_cast<int*>(ws) : nullptr;
  h.M = m;
  h.N = static_cast<int>(w.n);
  h.K = static_cast<int>(w.k);
  h.NT = static_cast<int>(ceil_div(w.n, kTileN));
  h.KU = static_cast<int>(ceil_div(w.k, kUnitK));
  h.ups = p.units_per_split;
  h.stride = p.lds_stride;
  h.KS = p.k_slices;
  h.groups = static_cast<int>(ceil_div(h.NT, p.waves / p.k_slices));
  h.whole = p.split > 1 ? p.whole_groups : h.groups;
  h.split = p.split;
  return h;
}

// CUs of the current device (cached per device).
int device_cus() {
  static std::mutex mu;
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (!cus[dev] && hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus[dev] = 0;
  return cus[dev];
}

// One launch of the fused kernel, or hipErrorCooperativeLaunchTooLarge
// (nothing enqueued) when its grid cannot be resident all at once.
template <int DA, int XPA, int DB>
hipError_t launch_fused(const MlpPlan& p, const HalfArgs& a, const HalfArgs& b, const FuseCtl& ctl,
                        hipStream_t stream) {
  const void* fn = reinterpret_cast<const void*>(&mlp_kernel<kFmtNvfp4, DA, XPA, DB>);
  static std::atomic<uint64_t> lds_allowed{0};
  const hipError_t attr = allow_dynamic_lds(fn, static_cast<int>(kLdsBudget), lds_allowed);
  if (attr != hipSuccess) return attr;
  int per_cu = 0;
  const hipError_t occ =
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kMlpWaves * 64, p.lds_bytes);
  if (occ != hipSuccess) return occ;
  const int64_t grid = static_cast<int64_t>(ctl.producers) + ctl.consumers;
  if (static_cast<int64_t>(per_cu) * device_cus() < grid) return hipErrorCooperativeLaunchTooLarge;
  hipLaunchKernelGGL((mlp_kernel<kFmtNvfp4, DA, XPA, DB>), dim3(static_cast<unsigned>(grid)), dim3(kMlpWaves * 64),
                     p.lds_bytes, stream, a, b, ctl);
  return hipGetLastError();
}

template <int DA, int XPA>
hipError_t launch_fused_db(const MlpPlan& p, const HalfArgs& a, const HalfArgs& b, const FuseCtl& ctl,
                           hipStream_t stream) {
  switch (p.down_fused.depth) {
    case 2: return launch_fused<DA, XPA, 2>(p, a, b, ctl, stream);
    case 3: return launch_fused<DA, XPA, 3>(p, a, b, ctl, stream);
    case 4: return launch_fused<DA, XPA, 4>(p, a, b, ctl, stream);
    case 6: return launch_fused<DA, XPA, 6>(p, a, b, ctl, stream);
    case 8: return launch_fused<DA, XPA, 8>(p, a, b, ctl, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fused_any(const MlpPlan& p, const HalfArgs& a, const HalfArgs& b, const FuseCtl& ctl,
                            hipStream_t stream) {
  const bool ring = p.up_fused.x_stage != kStageFull;
  if (p.up_fused.depth == 2)
    return ring ? launch_fused_db<2, 1>(p, a, b, ctl, stream) : launch_fused_db<2, 0>(p, a, b, ctl, stream);
  if (p.up_fused.depth == 3)
    return ring ? launch_fused_db<3, 1>(p, a, b, ctl, stream) : launch_fused_db<3, 0>(p, a, b, ctl, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_mlp(const MlpPlan& p, const WeightRef& up, const WeightRef& dn, const void* x, void* h, void* y,
                      void* workspace, int m, hipStream_t stream, int* launches) {
  char* wsb = static_cast<char*>(workspace);
  if (p.fusable && p.producers > 0 && p.consumers > 0) {
    FuseCtl ctl;
    ctl.produced = reinterpret_cast<int*>(wsb + p.counter_offset);
    ctl.status = ctl.produced + 2;
    ctl.flags = reinterpret_cast<int*>(wsb + p.flags_offset);
    ctl.producers = p.producers;
    ctl.consumers = p.consumers;
    ctl.stream_after = p.stream_after;
    const HalfArgs a = half_args(p.up_fused, up, x, h, wsb, m);
    const HalfArgs b = half_args(p.down_fused, dn, h, y, wsb + p.down_ws_offset, m);
    const hipError_t e = launch_fused_any(p, a, b, ctl, stream);
    if (e == hipSuccess) {
      if (launches) *launches = 1;
      return e;
    }
    if (e != hipErrorCooperativeLaunchTooLarge || p.fused_requested) return e;
  }
  if (p.fused_requested) return hipErrorCooperativeLaunchTooLarge;
  hipError_t e = launch_gemm(up.fmt, p.up, x, up.packed, up.row_scales, up.tensor_scale, h, nullptr, wsb, m, up.n,
                             up.k, stream);
  if (e != hipSuccess) return e;
  e = launch_gemm(dn.fmt, p.down, h, dn.packed, dn.row_scales, dn.tensor_scale, y, nullptr, wsb + p.down_ws_offset,
                  m, dn.n, dn.k, stream);
  if (e == hipSuccess && launches) *launches = 2;
  return e;
}

}  // namespace qpn
