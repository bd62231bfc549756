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
// Launch-shape heuristic, from a sweep of split x waves x depth on MI355X
// over the 27B shapes (N-tiles 320..9496, K units 20..68, M 1..8): the best
// split puts about 960 wavefronts (n-tiles x K ranges) on the chip, a
// stream depth of 3 units is within noise of the best everywhere, and
// 8-wave workgroups only pay off on very wide matrices.
constexpr int kTargetWaves = 960;
constexpr int kWideTiles = 4096;
constexpr int kRowPad = 8;          // fp16 pad per staged row (bank spread)

typedef __attribute__((address_space(3))) void* lds_ptr;

// Direct-to-LDS load of 16 bytes per lane: lane i's bytes land at LDS byte
// address lds_base + 16 * i (lds_base is wave-uniform and goes through M0).
// Written as inline assembly so that the compiler's wait-count bookkeeping
// does not see an LDS write in flight: left to itself it makes every later
// LDS read wait for all outstanding loads, the weight stream included. The
// caller waits for these loads explicitly before the workgroup barrier.
// (Untracked older loads can only make the compiler's own waits stricter,
// since the counter retires loads in issue order.)
__device__ __forceinline__ void lds_dma16(const void* src, _Float16* lds_dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)(lds_dst))));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(base)
               : "memory", "m0");
}

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
    const _Float16* __restrict__ x, const uint8_t* packed,
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

  // Stage this K range of every activation row in LDS with direct-to-LDS
  // loads: one global_load_lds_dwordx4 moves 64 lanes x 16 B (two units of
  // one row) without passing through registers, so all of them can be in
  // flight at once. Chunks past K (the zero-padded tail of the last unit)
  // are written as zeros first, so that 0 * x stays finite; lanes past the
  // row's staged length are masked off.
  const int row_chunks = nu * (kUnitK / 8);
  const int kbase = u0 * kUnitK;
  const int live_chunks = min(row_chunks, max(0, (K - kbase) / 8));
  if (live_chunks < row_chunks) {
    const int tail = row_chunks - live_chunks;
    for (int idx = tid; idx < M * tail; idx += WAVES * 64) {
      const int m = idx / tail;
      *reinterpret_cast<uint4*>(xs + m * stride + (live_chunks + idx - m * tail) * 8) =
          make_uint4(0u, 0u, 0u, 0u);
    }
  }
  const int windows = (live_chunks + 63) / 64;
  for (int wi = wave; wi < M * windows; wi += WAVES) {
    const int m = wi / windows;
    const int c0 = (wi - m * windows) * 64;
    if (c0 + lane < live_chunks)
      lds_dma16(x + static_cast<size_t>(m) * K + kbase + (c0 + lane) * 8, xs + m * stride + c0 * 8);
  }

  // Then issue the first DEPTH units of the weight stream unit by unit, in
  // the order the loop will consume them. (`packed` is deliberately not
  // __restrict__: with it the compiler may treat the weights as immutable and
  // sink these loads past the barrier below, which would both delay the
  // stream and break the staging wait.) Loads are never conditional: a
  // unit past the wavefront's range lies past the stream's byte range, so
  // the buffer load returns zeros without touching memory. This keeps the
  // compiler's view of in-flight loads exact at every point.
  Unit<FMT> buf[DEPTH];
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) {
    load_unit(buf[i], stream, i, lane);
    asm volatile("" ::: "memory");  // keep the units' loads in this order
  }
  // Wait for the staging loads only (they were issued before the weight
  // loads, and the counter retires loads in order) and for the zero stores,
  // then meet at a bare barrier: the weight loads stay in flight across it.
  // (A full __syncthreads would also wait for them.)
  __builtin_amdgcn_s_waitcnt(vmcnt_only(Unit<FMT>::kLoads * DEPTH));
  __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // B-operand column m of the MFMA is activation row m. Lanes of columns
  // m >= M read row M-1 (an LDS broadcast); their output columns are never
  // stored, and MFMA output columns do not mix, so they need no zeroing.
  const int mcol = lane & 15;
  const int g = lane >> 4;
  const _Float16* xrow = xs + min(mcol, M - 1) * stride + g * 64;
  f4 acc = {0.f, 0.f, 0.f, 0.f};

  if (active) {
    // Each slot of buf is consumed and then refilled in place (unit u + DEPTH
    // goes where unit u was), so the loop carries no register copies and
    // keeps DEPTH-1 units in flight while it computes. Refills past the end
    // of the range read zeros and cost no memory traffic.
    for (int base = 0; base < nu; base += DEPTH) {
#pragma unroll
      for (int i = 0; i < DEPTH; ++i) {
        if (base + i < nu) unit_mfma(buf[i], xrow + (base + i) * kUnitK, acc);
        load_unit(buf[i], stream, base + DEPTH + i, lane);
        // keep the scheduler from sinking the refill below the next units' math
        __builtin_amdgcn_sched_barrier(0);
      }
    }
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
  //
  // Partials and counters are accessed only through relaxed device-scope
  // atomics, which on gfx950 are plain loads and stores that bypass the
  // per-XCD L2 to the device-coherent level (sc1), so no cache-wide
  // writeback or invalidate is needed. Ordering comes from completion: each
  // thread waits for its partial stores to be acknowledged before the
  // workgroup barrier that precedes the counter increment, and the last
  // workgroup issues its loads only after the increment has returned.
  if (active && mcol < M) {
    float* dst = ws + (static_cast<size_t>(s) * M + mcol) * N;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n0 + r < N) __hip_atomic_store(dst + n0 + r, acc[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    last_group = __hip_atomic_fetch_add(counters + blockIdx.x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 S - 1;
  __syncthreads();
  if (!last_group) return;
  const int rows = WAVES * kTileN;
  const int nbase = blockIdx.x * rows;
  for (int idx = tid; idx < M * rows; idx += WAVES * 64) {
    const int m = idx / rows;
    const int n = nbase + (idx - m * rows);
    if (n >= N) continue;
    const float* src = ws + static_cast<size_t>(m) * N + n;
    float sum = 0.f;
    for (int r = 0; r < S; ++r)
      sum += __hip_atomic_load(src + static_cast<size_t>(r) * M * N, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float scale = FMT == kFmtNvfp4 ? tensor_scale : row_scales[n];
    y[static_cast<size_t>(m) * N + n] = static_cast<_Float16>(sum * scale);
  }
  if (tid == 0) __hip_atomic_store(counters + blockIdx.x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  const int64_t NT = ceil_div(n, kTileN);
  const int waves = waves_override ? waves_override : (NT >= kWideTiles ? 8 : 4);
  if (waves != 4 && waves != 8) return false;
  const int depth = depth_override ? depth_override : 3;
  if (depth != 2 && depth != 3 && depth != 4 && depth != 6 && depth != 8) return false;
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
    const int64_t s_occ = (kTargetWaves + NT / 2) / NT;  // nearest
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
