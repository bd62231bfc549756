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
// tiles go to a workspace and splitk_reduce adds them in range order, which
// keeps the result deterministic.
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
    float* __restrict__ ws, int M, int N, int K, int NT, int KU, int ups, int stride) {
  extern __shared__ __align__(16) _Float16 xs[];
  constexpr int kBytes = Unit<FMT>::kBytes;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = blockIdx.y;
  const int u0 = s * ups;
  const int nu = min(KU - u0, ups);
  const int nt = blockIdx.x * WAVES + wave;
  const bool active = nt < NT;
  const Stream stream(packed + (static_cast<size_t>(nt) * KU + u0) * kBytes,
                      active ? static_cast<uint32_t>(nu) * kBytes : 0u);

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
  if (!active) return;
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

  // Lane (m = lane % 16, g = lane / 16) holds rows n = 4g + r of column m.
  if (mcol < M) {
    const int n0 = nt * kTileN + g * 4;
    if (gridDim.y == 1) {
      _Float16* dst = y + static_cast<size_t>(mcol) * N;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = n0 + r;
        if (n < N) {
          const float scale = FMT == kFmtNvfp4 ? tensor_scale : row_scales[n];
          dst[n] = static_cast<_Float16>(acc[r] * scale);
        }
      }
    } else {
      float* dst = ws + (static_cast<size_t>(s) * M + mcol) * N;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n0 + r < N) dst[n0 + r] = acc[r];
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void splitk_reduce(const float* __restrict__ ws,
                                                     const float* __restrict__ row_scales,
                                                     float tensor_scale, _Float16* __restrict__ y,
                                                     int M, int N, int S) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t total = static_cast<int64_t>(M) * N;
  if (idx >= total) return;
  const int n = static_cast<int>(idx % N);
  float acc = 0.f;
  for (int s = 0; s < S; ++s) acc += ws[s * total + idx];
  const float scale = FMT == kFmtNvfp4 ? tensor_scale : row_scales[n];
  y[idx] = static_cast<_Float16>(acc * scale);
}

template <int FMT, int WAVES>
hipError_t launch_fmt(const GemmPlan& p, const void* x, const void* packed, const float* row_scales,
                      float tensor_scale, void* y, void* workspace, int m, int64_t n, int64_t k,
                      hipStream_t stream) {
  constexpr int DEPTH = FMT == kFmtNvfp4 ? 4 : 2;
  const int NT = static_cast<int>(ceil_div(n, kTileN));
  const int KU = static_cast<int>(ceil_div(k, kUnitK));
  dim3 grid(static_cast<unsigned>(ceil_div(NT, WAVES)), static_cast<unsigned>(p.split));
  hipLaunchKernelGGL((gemm_kernel<FMT, WAVES, DEPTH>), grid, dim3(WAVES * 64), p.lds_bytes, stream,
                     static_cast<const _Float16*>(x), static_cast<const uint8_t*>(packed), row_scales,
                     tensor_scale, static_cast<_Float16*>(y), static_cast<float*>(workspace), m,
                     static_cast<int>(n), static_cast<int>(k), NT, KU, p.units_per_split,
                     p.lds_stride);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.split == 1) return e;
  const int64_t total = static_cast<int64_t>(m) * n;
  hipLaunchKernelGGL((splitk_reduce<FMT>), dim3(static_cast<unsigned>(ceil_div(total, 256))),
                     dim3(256), 0, stream, static_cast<const float*>(workspace), row_scales,
                     tensor_scale, static_cast<_Float16*>(y), m, static_cast<int>(n), p.split);
  return hipGetLastError();
}

}  // namespace

bool plan_gemm(int fmt, int64_t n, int64_t k, int m, int split_override, int waves_override,
               GemmPlan* p) {
  if (fmt != kFmtNvfp4 && fmt != kFmtFp8) return false;
  if (m < 1 || m > kMaxM || n < 1 || k < 0) return false;
  const int waves = waves_override ? waves_override : 4;
  if (waves != 4 && waves != 8) return false;
  const int64_t NT = ceil_div(n, kTileN);
  const int64_t KU = ceil_div(k, kUnitK);
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
  p->units_per_split = static_cast<int>(ups);
  p->lds_stride = static_cast<int>(ups * kUnitK + kRowPad);
  p->lds_bytes = static_cast<size_t>(m) * p->lds_stride * sizeof(_Float16);
  p->workspace_bytes = split > 1 ? static_cast<size_t>(split) * m * n * sizeof(float) : 0;
  return true;
}

hipError_t launch_gemm(int fmt, const GemmPlan& p, const void* x, const void* packed,
                       const float* row_scales, float tensor_scale, void* y, void* workspace,
                       int m, int64_t n, int64_t k, hipStream_t stream) {
  if (fmt == kFmtNvfp4) {
    return p.waves == 8 ? launch_fmt<kFmtNvfp4, 8>(p, x, packed, row_scales, tensor_scale, y,
                                                    workspace, m, n, k, stream)
                        : launch_fmt<kFmtNvfp4, 4>(p, x, packed, row_scales, tensor_scale, y,
                                                    workspace, m, n, k, stream);
  }
  return p.waves == 8 ? launch_fmt<kFmtFp8, 8>(p, x, packed, row_scales, tensor_scale, y,
                                                workspace, m, n, k, stream)
                      : launch_fmt<kFmtFp8, 4>(p, x, packed, row_scales, tensor_scale, y, workspace,
                                                m, n, k, stream);
}

}  // namespace qpn
