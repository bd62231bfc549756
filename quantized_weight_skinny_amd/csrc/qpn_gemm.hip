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
// the B operand (columns 0..M-1 of the 16-wide tile; the rest are zero), so
// one instruction serves any M <= 16 and the verify rows of a speculative
// round cost no extra weight traffic (the 8-row tile of the post's Volta
// design becomes the 16-row MFMA tile here).
//
// Work split: each wavefront owns one 16-row n-tile and a contiguous range of
// 256-element K units. A workgroup holds `WAVES` neighbouring n-tiles of the
// same K range and first stages x[:, range] into LDS (one 16-byte
// ds_read_b128 per lane per MFMA later). Loads of DEPTH units are kept in
// flight per wavefront. When K is cut into several ranges the fp32 partial
// tiles go to a workspace and the last workgroup of each group of n-tiles to
// finish adds them in range order, which keeps the result deterministic and
// needs no second kernel.
#include "qpn_device.hpp"
#include "qpn_internal.hpp"

namespace qpn {
namespace {

constexpr size_t kLdsBudget = 64 * 1024;
constexpr int kTargetWaves = 2048;  // about 8 wavefronts per CU on 256 CUs
constexpr int kRowPad = 8;          // fp16 pad per staged row (bank spread)

__device__ __forceinline__ h8 x_fragment(const _Float16* p) { return *reinterpret_cast<const h8*>(p); }

__device__ __forceinline__ void unit_mfma(const Unit<kFmtNvfp4>& w, const _Float16* xrow, f4& acc) {
  const h2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.sc, 1.0f, false);
  const h2 s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.sc, 1.0f, true);
  const h2 sc[4] = {h2{s01.x, s01.x}, h2{s01.y, s01.y}, h2{s23.x, s23.x}, h2{s23.y, s23.y}};
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t d = word(t < 4 ? w.c0 : w.c1, t & 3);
    const h8 a = decode_fp4x8(d, sc[t >> 1]);
    const h8 b = x_fragment(xrow + t * 8);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
  }
}

__device__ __forceinline__ void unit_mfma(const Unit<kFmtFp8>& w, const _Float16* xrow, f4& acc) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const u4& v = w.q[t >> 1];
    const int i = (t & 1) * 2;
    const h8 a = decode_fp8x8(word(v, i), word(v, i + 1));
    const h8 b = x_fragment(xrow + t * 8);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
  }
}

template <int FMT, int WAVES, int DEPTH>
__global__ __launch_bounds__(WAVES * 64) void gemm_kernel(
    const _Float16* __restrict__ x, const uint8_t* __restrict__ packed,
    const float* __restrict__ row_scales, float tensor_scale, _Float16* __restrict__ y,
    float* __restrict__ ws, int* __restrict__ counters, int M, int N, int K, int NT, int KU, int ups,
    int stride) {
  extern __shared__ __align__(16) _Float16 xs[];
  __shared__ int last_group;
  constexpr int kBytes = Unit<FMT>::kBytes;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = gridDim.y;
  const int s = blockIdx.y;
  const int u0 = s * ups;
  const int nu = min(KU - u0, ups);
  const int nt = blockIdx.x * WAVES + wave;
  const bool active = nt < NT;
  const uint32_t unit_stride = static_cast<uint32_t>(NT) * kBytes;
  const Stream stream(packed + unit_offset(active ? nt : 0, u0, NT, kBytes),
                      active && nu > 0 ? static_cast<uint32_t>(nu - 1) * unit_stride + kBytes : 0u,
                      unit_stride);

  // Issue the first DEPTH units unit by unit, in the order the loop will
  // consume them, so that the wait before each unit counts only its own loads.
  Unit<FMT> buf[DEPTH];
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) {
    if (i < nu) load_unit(buf[i], stream, i, lane);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Stage this K range of every activation row in LDS, zero past K.
  const int chunks = nu * (kUnitK / 8);
  const int kbase = u0 * kUnitK;
  for (int idx = tid; idx < M * chunks; idx += WAVES * 64) {
    const int m = idx / chunks;
    const int c = idx - m * chunks;
    const int kk = kbase + c * 8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (kk < K) v = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(m) * K + kk);
    *reinterpret_cast<uint4*>(xs + m * stride + c * 8) = v;
  }
  __syncthreads();
  // Settle every load issued so far (the first units and the staging reads):
  // the loop below then starts from a known queue of in-flight loads and
  // each unit waits only for its own.
  __builtin_amdgcn_s_waitcnt(0);

  // B-operand column m of the MFMA is activation row m. Lanes of columns
  // m >= M read row M-1 (an LDS broadcast); their output columns are never
  // stored, and MFMA output columns do not mix, so they need no zeroing.
  const int mcol = lane & 15;
  const int g = lane >> 4;
  const _Float16* xrow = xs + min(mcol, M - 1) * stride + g * 64;
  f4 acc = {0.f, 0.f, 0.f, 0.f};

  if (active) {
    // Each slot of buf is consumed and then refilled in place, so the loop
    // carries no register copies and keeps DEPTH-1 units in flight while it
    // computes. The steady-state loop has no conditional loads; the last
    // (< 2*DEPTH) units run as straight-line code.
    int u = 0;
    for (; u + 2 * DEPTH <= nu; u += DEPTH) {
#pragma unroll
      for (int i = 0; i < DEPTH; ++i) {
        unit_mfma(buf[i], xrow + (u + i) * kUnitK, acc);
        load_unit(buf[i], stream, u + DEPTH + i, lane);
        // keep the scheduler from sinking the refill below the next units' math
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) {
      if (u + i < nu) {
        unit_mfma(buf[i], xrow + (u + i) * kUnitK, acc);
        if (u + DEPTH + i < nu) load_unit(buf[i], stream, u + DEPTH + i, lane);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int i = 0; i < DEPTH; ++i)
      if (u + DEPTH + i < nu) unit_mfma(buf[i], xrow + (u + DEPTH + i) * kUnitK, acc);
  }

  // Lane (m = lane % 16, g = lane / 16) holds rows n = 4g + r of column m.
  const int n0 = nt * kTileN + g * 4;
  if (S == 1) {
    if (active && mcol < M) {
      _Float16* dst = y + static_cast<size_t>(mcol) * N;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = n0 + r;
        if (n < N) {
          const float scale = FMT == kFmtNvfp4 ? tensor_scale : row_scales[n];
          dst[n] = static_cast<_Float16>(acc[r] * scale);
        }
      }
    }
    return;
  }

  // K was split over gridDim.y workgroups per group of n-tiles: publish this
  // range's fp32 partials, then the last workgroup of the group to arrive
  // adds all ranges in range order (the same order whichever arrives last, so
  // the result is deterministic) and resets the group's counter for the next
  // call. No workgroup ever waits for another.
  if (active && mcol < M) {
    float* dst = ws + (static_cast<size_t>(s) * M + mcol) * N;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n0 + r < N) dst[n0 + r] = acc[r];
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) last_group = atomicAdd(counters + blockIdx.x, 1) == S - 1;
  __syncthreads();
  if (!last_group) return;
  __threadfence();
  const int rows = WAVES * kTileN;
  const int nbase = blockIdx.x * rows;
  for (int idx = tid; idx < M * rows; idx += WAVES * 64) {
    const int m = idx / rows;
    const int n = nbase + (idx - m * rows);
    if (n >= N) continue;
    const float* src = ws + static_cast<size_t>(m) * N + n;
    float sum = 0.f;
    for (int r = 0; r < S; ++r) sum += src[static_cast<size_t>(r) * M * N];
    const float scale = FMT == kFmtNvfp4 ? tensor_scale : row_scales[n];
    y[static_cast<size_t>(m) * N + n] = static_cast<_Float16>(sum * scale);
  }
  if (tid == 0) atomicExch(counters + blockIdx.x, 0);
}

template <int FMT, int WAVES, int DEPTH>
hipError_t launch_cfg(const GemmPlan& p, const void* x, const void* packed, const float* row_scales,
                      float tensor_scale, void* y, void* workspace, int m, int64_t n, int64_t k,
                      hipStream_t stream) {
  const int NT = static_cast<int>(ceil_div(n, kTileN));
  const int KU = static_cast<int>(ceil_div(k, kUnitK));
  const unsigned groups = static_cast<unsigned>(ceil_div(NT, WAVES));
  int* counters = p.split > 1 ? static_cast<int*>(workspace) : nullptr;
  float* ws = p.split > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + p.partials_offset)
                          : nullptr;
  hipLaunchKernelGGL((gemm_kernel<FMT, WAVES, DEPTH>), dim3(groups, static_cast<unsigned>(p.split)),
                     dim3(WAVES * 64), p.lds_bytes, stream, static_cast<const _Float16*>(x),
                     static_cast<const uint8_t*>(packed), row_scales, tensor_scale,
                     static_cast<_Float16*>(y), ws, counters, m, static_cast<int>(n),
                     static_cast<int>(k), NT, KU, p.units_per_split, p.lds_stride);
  return hipGetLastError();
}

template <int FMT, int WAVES>
hipError_t launch_depth(const GemmPlan& p, const void* x, const void* packed, const float* row_scales,
                        float tensor_scale, void* y, void* workspace, int m, int64_t n, int64_t k,
                        hipStream_t stream) {
  switch (p.depth) {
    case 2: return launch_cfg<FMT, WAVES, 2>(p, x, packed, row_scales, tensor_scale, y, workspace, m, n, k, stream);
    case 3: return launch_cfg<FMT, WAVES, 3>(p, x, packed, row_scales, tensor_scale, y, workspace, m, n, k, stream);
    case 6: return launch_cfg<FMT, WAVES, 6>(p, x, packed, row_scales, tensor_scale, y, workspace, m, n, k, stream);
    case 8: return launch_cfg<FMT, WAVES, 8>(p, x, packed, row_scales, tensor_scale, y, workspace, m, n, k, stream);
    default: return launch_cfg<FMT, WAVES, 4>(p, x, packed, row_scales, tensor_scale, y, workspace, m, n, k, stream);
  }
}

}  // namespace

bool plan_gemm(int fmt, int64_t n, int64_t k, int m, int split_override, int waves_override,
               int depth_override, GemmPlan* p) {
  if (fmt != kFmtNvfp4 && fmt != kFmtFp8) return false;
  if (m < 1 || m > kMaxM || n < 1 || k < 0) return false;
  const int waves = waves_override ? waves_override : 4;
  if (waves != 4 && waves != 8) return false;
  const int depth = depth_override ? depth_override : (fmt == kFmtNvfp4 ? 4 : 2);
  if (depth != 2 && depth != 3 && depth != 4 && depth != 6 && depth != 8) return false;
  const int64_t NT = ceil_div(n, kTileN);
  const int64_t KU = ceil_div(k, kUnitK);
  const int64_t unit_bytes = fmt == kFmtNvfp4 ? kNvUnitBytes : kF8UnitBytes;
  // unit offsets inside one wavefront's stream are 32-bit
  if (NT * KU * unit_bytes >= (int64_t(1) << 31)) return false;
  const int64_t max_ups = (static_cast<int64_t>(kLdsBudget) / (2 * m) - kRowPad) / kUnitK;
  int64_t split;
  if (split_override > 0) {
    split = split_override;
  } else {
    const int64_t s_lds = KU ? ceil_div(KU, max_ups) : 1;
    const int64_t s_occ = ceil_div(kTargetWaves, NT);
    split = s_lds > s_occ ? s_lds : s_occ;
  }
  if (split > KU) split = KU ? KU : 1;
  if (split < 1) split = 1;
  int64_t ups = KU ? ceil_div(KU, split) : 0;
  if (KU) split = ceil_div(KU, ups);
  if (ups > max_ups) return false;
  p->split = static_cast<int>(split);
  p->waves = waves;
  p->depth = depth;
  p->units_per_split = static_cast<int>(ups);
  p->lds_stride = static_cast<int>(ups * kUnitK + kRowPad);
  p->lds_bytes = static_cast<size_t>(m) * p->lds_stride * sizeof(_Float16);
  if (split > 1) {
    // Counters first, sized for the smallest workgroup (4 n-tiles), so that
    // their place does not depend on m, split or workgroup size and a
    // workspace can be shared by calls with different row counts.
    const size_t counters = static_cast<size_t>(ceil_div(NT, 4)) * sizeof(int);
    p->partials_offset = (counters + 255) & ~size_t(255);
    p->workspace_bytes = p->partials_offset + static_cast<size_t>(split) * m * n * sizeof(float);
  } else {
    p->partials_offset = 0;
    p->workspace_bytes = 0;
  }
  return true;
}

hipError_t launch_gemm(int fmt, const GemmPlan& p, const void* x, const void* packed,
                       const float* row_scales, float tensor_scale, void* y, void* workspace,
                       int m, int64_t n, int64_t k, hipStream_t stream) {
  if (fmt == kFmtNvfp4) {
    return p.waves == 8 ? launch_depth<kFmtNvfp4, 8>(p, x, packed, row_scales, tensor_scale, y,
                                                      workspace, m, n, k, stream)
                        : launch_depth<kFmtNvfp4, 4>(p, x, packed, row_scales, tensor_scale, y,
                                                      workspace, m, n, k, stream);
  }
  return p.waves == 8 ? launch_depth<kFmtFp8, 8>(p, x, packed, row_scales, tensor_scale, y,
                                                  workspace, m, n, k, stream)
                      : launch_depth<kFmtFp8, 4>(p, x, packed, row_scales, tensor_scale, y,
                                                  workspace, m, n, k, stream);
}

}  // namespace qpn
