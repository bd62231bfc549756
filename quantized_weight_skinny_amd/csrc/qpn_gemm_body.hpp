// Device code of the skinny GEMM (see qpn_gemm.hip for the method): the
// staging and decode helpers and the GEMM body of one workgroup, shared by
// the GEMM launches (qpn_gemm.hip) and the fused MLP launch (qpn_mlp.hip).
// Everything here has internal linkage; each source that includes it gets its
// own copy.
#pragma once

#include "qpn_device.hpp"
#include "qpn_internal.hpp"

namespace qpn {
namespace {
typedef __attribute__((address_space(3))) void* lds_ptr;

// Direct-to-LDS load of 16 bytes per lane: lane i's bytes land at LDS byte
// address lds_base + 16 * i (lds_base is wave-uniform and goes through M0).
// Written as inline assembly so that the compiler's wait-count bookkeeping
// does not see an LDS write in flight: left to itself it makes every later
// LDS read wait for all outstanding loads, the weight stream included. The
// caller waits for these loads explicitly before the workgroup barrier.
// (Untracked older loads can only make the compiler's own waits stricter,
// since the counter retires loads in issue order.) M0 is a reserved register
// to the compiler, which ignores it in a clobber list: this is safe only
// because nothing else in these kernels uses M0 (no LDS-DMA builtins, message
// sends or indirect register indexing); the generated code holds no M0 write
// other than this one, which a build test checks on the assembly. The clobber
// stays as documentation; its warning is silenced here and nowhere else.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* src, _Float16* lds_dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)(lds_dst))));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(base)
               : "memory", "m0");
}
// The same with the device-coherent cache policy (sc1): the load is served
// from the level all XCDs share, for activations that another workgroup of
// the same launch wrote with device-scope stores.
__device__ __forceinline__ void lds_dma16_coherent(const void* src, _Float16* lds_dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)(lds_dst))));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off sc1" ::"v"(src), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ h8 x_fragment(const _Float16* p) { return *reinterpret_cast<const h8*>(p); }

// LDS pointers kept as such (a select between two of them as generic pointers
// would become flat loads, which also wait on the vector-memory counter).
typedef const __attribute__((address_space(3))) _Float16* lds_half_ptr;
__device__ __forceinline__ lds_half_ptr to_lds(const _Float16* p) { return (lds_half_ptr)(p); }
__device__ __forceinline__ h8 x_fragment(lds_half_ptr p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) h8*>(p);
}

// silu(g) = g / (1 + e^-g) in fp32 (e^-g overflows to +inf for g < -88,
// giving -0, the limit).
__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// Greedy-argmax key of logit v at index n: the float's bits mapped to an
// unsigned order (negative values flipped, positive ones above them) in the
// high word and ~n in the low word, so the largest key is the largest logit
// and, among equal logits, the smallest index. 0 means "nothing yet" (below
// every real key, since -inf maps to 0x007FFFFF).
__device__ __forceinline__ unsigned long long argmax_key(float v, int n) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<unsigned long long>(ord) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(n));
}

__device__ __forceinline__ void argmax_decode(unsigned long long key, int* n, float* v) {
  const uint32_t ord = static_cast<uint32_t>(key >> 32);
  *n = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key));
  *v = __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

// Sum over the S K ranges of one output's fp32 partials (stride apart), in
// range order. The partials are fetched kFixupBatch at a time, all loads of a
// batch in flight together: one memory round trip per batch, not per range.
__device__ __forceinline__ float range_sum(const float* src, size_t stride, int S) {
  float sum = 0.f;
  for (int r0 = 0; r0 < S; r0 += kFixupBatch) {
    float part[kFixupBatch];
#pragma unroll
    for (int j = 0; j < kFixupBatch; ++j)
      part[j] = r0 + j < S ? __hip_atomic_load(src + (r0 + j) * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                           : 0.f;
#pragma unroll
    for (int j = 0; j < kFixupBatch; ++j)
      if (r0 + j < S) sum += part[j];
  }
  return sum;
}

// The eight MFMA steps of a unit alternate between two accumulators, which
// halves the chain of dependent matrix instructions per wavefront; the two
// are added once at the end (a fixed order, so results stay reproducible).
__device__ __forceinline__ void unit_mfma(const Unit<kFmtNvfp4>& w, const _Float16* xrow, f4 (&acc)[2]) {
  const h2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.sc, 1.0f, false);
  const h2 s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.sc, 1.0f, true);
  const h2 sc[4] = {h2{s01.x, s01.x}, h2{s01.y, s01.y}, h2{s23.x, s23.x}, h2{s23.y, s23.y}};
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t d = word(t < 4 ? w.c0 : w.c1, t & 3);
    const h8 a = decode_fp4x8(d, sc[t >> 1]);
    const h8 b = x_fragment(xrow + t * 8);
    acc[t & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[t & 1], 0, 0, 0);
  }
}

// Block columns (one activation row, NVFP4): the MFMA's 16 output columns
// carry the unit's 16 K-blocks instead of 16 activation rows. The B operand
// is block-diagonal: at step t, lane (j = lane % 16, g = lane / 16) holds the
// 8 activations of its K group g only if j is the block those 8 elements
// belong to (j == 4g + t/2), and zeros otherwise, so output column j
// accumulates the unit's block j alone: P[r][j] = sum over block j of
// E2M1(w[r][k]) * x[k]. Each block scale then multiplies one fp32 block sum
// per row, 4 per lane and unit, instead of every decoded weight pair (the
// decode is only the fp4 -> fp16 conversion). bp[p] is the lane's x pointer
// for steps 2p, 2p+1: its own x where j - 4g == p, else a zero region that
// the same offsets keep inside. Output lane (j, g) needs the block scales
// S[4g + i][j], i = 0..3, which the packed layout holds in lane
// (4g + i) + 16 * (j / 4), byte j % 4 (sbase is that lane's byte address for
// i = 0; ssel picks byte j % 4 of two dwords into the low two bytes).
__device__ __forceinline__ void unit_block_cols(const Unit<kFmtNvfp4>& w, const lds_half_ptr (&bp)[4], int off,
                                                int sbase, uint32_t ssel, f4& acc) {
  const uint32_t d0 = __builtin_amdgcn_ds_bpermute(sbase, static_cast<int>(w.sc));
  const uint32_t d1 = __builtin_amdgcn_ds_bpermute(sbase + 4, static_cast<int>(w.sc));
  const uint32_t d2 = __builtin_amdgcn_ds_bpermute(sbase + 8, static_cast<int>(w.sc));
  const uint32_t d3 = __builtin_amdgcn_ds_bpermute(sbase + 12, static_cast<int>(w.sc));
  const uint32_t s4 = __builtin_amdgcn_perm(d1, d0, ssel) | (__builtin_amdgcn_perm(d3, d2, ssel) << 16);
  const f2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(s4, 1.0f, false);
  const f2 s23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(s4, 1.0f, true);
  f4 d[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t c = word(t < 4 ? w.c0 : w.c1, t & 3);
    const h8 a = cat(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 0), __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 1),
                     __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 2), __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 3));
    const h8 b = x_fragment(bp[t >> 1] + off + t * 8);
    d[t & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, d[t & 1], 0, 0, 0);
  }
  acc[0] = fmaf(s01.x, d[0][0], fmaf(s01.x, d[1][0], acc[0]));
  acc[1] = fmaf(s01.y, d[0][1], fmaf(s01.y, d[1][1], acc[1]));
  acc[2] = fmaf(s23.x, d[0][2], fmaf(s23.x, d[1][2], acc[2]));
  acc[3] = fmaf(s23.y, d[0][3], fmaf(s23.y, d[1][3], acc[3]));
}

__device__ __forceinline__ void unit_mfma(const Unit<kFmtFp8>& w, const _Float16* xrow, f4 (&acc)[2]) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const u4& v = w.q[t >> 1];
    const int i = (t & 1) * 2;
    const h8 a = decode_fp8x8(word(v, i), word(v, i + 1));
    const h8 b = x_fragment(xrow + t * 8);
    acc[t & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[t & 1], 0, 0, 0);
  }
}

// The VALU packed-dot alternative to the MFMA (a launch option, measured
// against it): lane (r = lane % 16, g = lane / 16) holds the 64 weights of
// row r in K group g, as fp16 pairs straight from the converts, and adds R
// activation rows' dot products with v_dot2c_f32_f16 (two products and the
// fp32 accumulator per instruction, R per weight pair). The NVFP4 block
// scale multiplies each 16-element block's partial sum once, in fp32. xr[m]
// is row m's staged x at the lane's K group; `off` the unit's offset in it.
__device__ __forceinline__ float dot8(const h8& a, const h8& b, float c) {
  c = __builtin_amdgcn_fdot2(h2{a[0], a[1]}, h2{b[0], b[1]}, c, false);
  c = __builtin_amdgcn_fdot2(h2{a[2], a[3]}, h2{b[2], b[3]}, c, false);
  c = __builtin_amdgcn_fdot2(h2{a[4], a[5]}, h2{b[4], b[5]}, c, false);
  return __builtin_amdgcn_fdot2(h2{a[6], a[7]}, h2{b[6], b[7]}, c, false);
}

template <int R>
__device__ __forceinline__ void unit_dot(const Unit<kFmtNvfp4>& w, const _Float16* const (&xr)[R], int off,
                                         float (&acc)[R]) {
  const h2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.sc, 1.0f, false);
  const h2 s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.sc, 1.0f, true);
  const float bs[4] = {static_cast<float>(s01.x), static_cast<float>(s01.y), static_cast<float>(s23.x),
                       static_cast<float>(s23.y)};
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    float part[R];
#pragma unroll
    for (int m = 0; m < R; ++m) part[m] = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t = 2 * blk + tt;
      const uint32_t d = word(t < 4 ? w.c0 : w.c1, t & 3);
      const h8 a = cat(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0),
                       __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1),
                       __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2),
                       __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3));
#pragma unroll
      for (int m = 0; m < R; ++m) part[m] = dot8(a, x_fragment(xr[m] + off + t * 8), part[m]);
    }
#pragma unroll
    for (int m = 0; m < R; ++m) acc[m] = fmaf(bs[blk], part[m], acc[m]);
  }
}

template <int R>
__device__ __forceinline__ void unit_dot(const Unit<kFmtFp8>& w, const _Float16* const (&xr)[R], int off,
                                         float (&acc)[R]) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const u4& v = w.q[t >> 1];
    const int i = (t & 1) * 2;
    const h8 a = decode_fp8x8(word(v, i), word(v, i + 1));
#pragma unroll
    for (int m = 0; m < R; ++m) acc[m] = dot8(a, x_fragment(xr[m] + off + t * 8), acc[m]);
  }
}

// Outputs of the greedy-argmax epilogue and its workspace.
struct ArgmaxOut {
  unsigned long long* keys;  // [kArgmaxSubs][kMaxM] key slots (zero between calls)
  int* idx;                  // [M] int32 argmax
  float* val;                // [M] fp32 max logit, or null
};

// One output element: rounded once to fp16, or with kEpiF32 the scaled fp32
// accumulator as it is.
template <int EPI>
__device__ __forceinline__ void put_out(void* y, size_t i, float v) {
  if constexpr (EPI == kEpiF32)
    static_cast<float*>(y)[i] = v;
  else
    static_cast<_Float16*>(y)[i] = static_cast<_Float16>(v);
}

// Control of a fused launch in which the workgroups of a second GEMM (the
// consumer) read activations that the workgroups of a first one (the
// producer) write in the same launch. Each consumer polls flags of its own,
// one 128-byte line per consumer (so no line is polled by more than one
// workgroup: a line that all of them polled would queue their reads at one
// memory channel and slow every stream that crosses it); producers count
// themselves in, and the one whose arrival completes a stage raises that
// stage's flag in every consumer's line.
constexpr int kFuseFlagInts = 32;  // ints per consumer line: [0] stream, [1] go
struct FuseCtl {
  int* produced;      // producer workgroups finished (zero between calls)
  int* flags;         // consumer c's line at flags + c * kFuseFlagInts (zero between calls)
  int* status;        // set to 1 when a wait ran out of its bound (never cleared by the kernel)
  int producers;      // producer workgroups in the launch
  int consumers;      // consumer workgroups in the launch
  int stream_after;   // producers finished before the consumers issue their first weight units (0: at once)
};

// A consumer's bounded wait for a flag of its line to be raised: one lane
// polls it (device-coherent loads, a short sleep between them), then the
// workgroup meets at a bare barrier (weight loads already issued stay in
// flight). A wait that runs past kFuseSpinLimit polls gives up and flags
// ctl.status, so a launch always ends: its results are then undefined.
constexpr int kFuseSpinLimit = 1 << 22;
__device__ __forceinline__ void fuse_wait(const FuseCtl& ctl, const int* flag) {
  if (threadIdx.x == 0) {
    int spins = 0;
    while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
      __builtin_amdgcn_s_sleep(4);
      if (++spins == kFuseSpinLimit) {
        __hip_atomic_store(ctl.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Four consecutive fp32 partial sums with one 16-byte store under the
// device-coherent cache policy (sc1, the policy of a relaxed device-scope
// atomic store): as four 4-byte stores, each one costs a write of its own
// memory sector, four times the bytes. The caller waits for the store
// (s_waitcnt) before it publishes the partials.
__device__ __forceinline__ void store4_coherent(float* p, const f4& v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}

// One output pair of SwiGLU values, 4 consecutive fp16 (8 bytes, aligned):
// with COHERENT a device-scope store (written through to the level all XCDs
// share), for a consumer in the same launch.
template <bool COHERENT>
__device__ __forceinline__ void put_h4(_Float16* dst, const float (&v)[4]) {
  union {
    _Float16 h[4];
    unsigned long long u;
  } b;
#pragma unroll
  for (int r = 0; r < 4; ++r) b.h[r] = static_cast<_Float16>(v[r]);
  if constexpr (COHERENT)
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(dst), b.u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *reinterpret_cast<unsigned long long*>(dst) = b.u;
}

template <bool COHERENT>
__device__ __forceinline__ void put_h1(_Float16* dst, float v) {
  if constexpr (COHERENT) {
    const _Float16 h = static_cast<_Float16>(v);
    __hip_atomic_store(reinterpret_cast<unsigned short*>(dst), __builtin_bit_cast(unsigned short, h),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    *dst = static_cast<_Float16>(v);
  }
}

// The GEMM of one workgroup, `block` being its index in the GEMM's grid.
// XP = 0: full stage; XP > 0: ring stage with XP x pieces per thread.
// DOT = 0: MFMA; DOT > 0: the VALU packed-dot path for up to DOT rows (full
// stage and the plain epilogue only).
// FUSE = 0: a launch of its own. FUSE = 1: the producer of a fused launch
// (the SwiGLU epilogue; h is written with device-scope stores). FUSE = 2: the
// consumer (full stage, plain epilogue; `block` is its index among the
// consumers): it issues its first DEPTH weight units once ctl.stream_after
// producers have finished, waits for all of them, and only then stages its
// activations, with device-coherent loads.
template <int FMT, int WAVES, int DEPTH, int EPI, int XP, int DOT, int FUSE>
__device__ __forceinline__ void gemm_body(
    const _Float16* x, const uint8_t* packed,
    const float* __restrict__ row_scales, float tensor_scale, void* __restrict__ y,
    float* __restrict__ ws, int* __restrict__ counters, ArgmaxOut amax, int M, int N, int K, int NT, int KU,
    int ups, int stride, int KS, int groups, int whole, int split, int block, const FuseCtl& ctl) {
  static_assert(FUSE == 0 || (FUSE == 1 && EPI == kEpiSwiglu && DOT == 0) ||
                    (FUSE == 2 && EPI == kEpiNone && XP == 0 && DOT == 0),
                "fused launch: a SwiGLU producer and a full-stage consumer");
  // The uneven-group grid (one K slice, no K split, fp16 or fp32 y):
  // `whole` is its workgroup count G, and workgroup b takes the NT / G or
  // NT / G + 1 consecutive n-tiles from b * (NT / G) + min(b, NT % G), the
  // larger count going to the first NT % G workgroups. Each CU then streams
  // the same number of tiles to within one, with no split-K tail.
  constexpr bool uneven = WAVES == kUnevenWaves;
  static_assert(!uneven || ((EPI == kEpiNone || EPI == kEpiF32) && DOT == 0 && FUSE == 0),
                "uneven grid: fp16 or fp32 y, MFMA");
  constexpr bool coherent_h = FUSE == 1;
  // The epilogue is a template parameter, so the plain kernels carry none of
  // the others: kEpiSwiglu writes h[M, N/2] = silu(y[:, :N/2]) * y[:, N/2:],
  // kEpiArgmax writes each row's largest logit and its index, kEpiF32 writes
  // y in fp32.
  constexpr bool swiglu = EPI == kEpiSwiglu;
  constexpr bool argmax = EPI == kEpiArgmax;
  extern __shared__ __align__(16) _Float16 xs[];
  __shared__ int last_group;
  __shared__ unsigned long long best[kMaxM];
  constexpr int kBytes = Unit<FMT>::kBytes;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroups [0, whole) each take one group of n-tiles over the whole K;
  // each of the other groups has its K cut into `split` ranges of `ups`
  // units, one workgroup per range, range-major (all first ranges, then all
  // second ranges ...).
  int grp, s, S;
  int tile0 = 0, tiles = 0;  // the uneven grid's n-tiles of this workgroup
  if (uneven) {
    const int tmin = NT / whole, extra = NT - tmin * whole;
    tile0 = block * tmin + min(block, extra);
    tiles = tmin + (block < extra ? 1 : 0);
    grp = block;
    s = 0;
    S = 1;
  } else if (block < whole) {
    grp = block;
    s = 0;
    S = 1;
  } else {
    const int r = block - whole;
    const int tail = groups - whole;
    s = r / tail;
    grp = whole + (r - s * tail);
    S = split;
  }
  const int u0 = S == 1 ? 0 : s * ups;
  const int nu = S == 1 ? KU : min(KU - u0, ups);
  // The workgroup's WAVES wavefronts cover TN n-tiles x KS slices of its K
  // range: wavefront (tn, ks) streams n-tile tn over the ks-th slice.
  const int TN = WAVES / KS;
  const int tn = wave % TN;
  const int ks = wave / TN;
  const int sub = (nu + KS - 1) / KS;
  const int wu0 = min(ks * sub, nu);
  const int wnu = min(sub, nu - wu0);
  // With the SwiGLU epilogue the workgroup pairs gate and up n-tiles: its
  // first TN/2 wavefront columns take gate tiles (rows below N/2), the
  // others the up tiles holding the same rows + N/2.
  const int half_tn = TN / 2;
  const int NTh = NT / 2;
  const int pair = grp * half_tn + (tn < half_tn ? tn : tn - half_tn);
  const int nt = uneven ? tile0 + tn : swiglu ? (tn < half_tn ? pair : NTh + pair) : grp * TN + tn;
  const bool active = uneven ? tn < tiles && nt < NT : swiglu ? pair < NTh : nt < NT;
  const uint32_t unit_stride = static_cast<uint32_t>(NT) * kBytes;
  // The weight stream is set up where the first weight units are issued:
  // after the activation loads, behind a scheduling barrier, so that its
  // address arithmetic (some 30-65 instructions) sits between the two.
  // Measured on the 27B shapes, the ring launches at 8 rows run 2-5% faster
  // than with the weight loads issued right behind the activation loads, and
  // the full stage 2% faster than with the set-up ahead of both. The likely
  // reason: the activation requests of all the CU's wavefronts then reach the
  // memory pipeline ahead of the weight requests, so the stage's first
  // barrier does not wait behind those.
  auto weight_stream = [&]() {
    return Stream(packed + unit_offset(active ? nt : 0, u0 + wu0, NT, kBytes),
                  active && wnu > 0 ? static_cast<uint32_t>(wnu - 1) * unit_stride + kBytes : 0u, unit_stride);
  };

  // B-operand column m of the MFMA is activation row m. Lanes of columns
  // m >= M read row M-1 (an LDS broadcast); their output columns are never
  // stored, and MFMA output columns do not mix, so they need no zeroing.
  const int mcol = lane & 15;
  const int g = lane >> 4;
  f4 acc2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  static_assert(DOT <= 0 || (XP == 0 && EPI == kEpiNone), "packed-dot path: full stage, plain epilogue");
  static_assert(DOT != kDotBlockCols || (XP == 0 && FMT == kFmtNvfp4), "block columns: NVFP4, full stage");
  constexpr int kDotRows = DOT > 0 ? DOT : 1;
  float dacc[kDotRows];
#pragma unroll
  for (int m = 0; m < kDotRows; ++m) dacc[m] = 0.f;
  // Loads of the weight stream are never conditional: a unit past the
  // wavefront's range lies past the stream's byte range, so the buffer load
  // returns zeros without touching memory. This keeps the compiler's view of
  // in-flight loads exact at every point. (`packed` is deliberately not
  // __restrict__: with it the compiler may treat the weights as immutable
  // and move their loads across the staging barriers, which would both delay
  // the stream and break the staging waits.)
  Unit<FMT> buf[DEPTH];
  Stream stream;

  if constexpr (XP == 0) {
    // Full stage: this K range of every activation row goes to LDS before
    // the stream starts, with direct-to-LDS loads: one
    // global_load_lds_dwordx4 moves 64 lanes x 16 B (two units of one row)
    // without passing through registers, so all of them can be in flight at
    // once. Chunks past K (the zero-padded tail of the last unit) are
    // written as zeros first, so that 0 * x stays finite; lanes past the
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
    if constexpr (DOT == kDotBlockCols) {
      // the zero region the block-column B operand reads where a lane holds no block
      constexpr int kZeroChunks = (DEPTH * kUnitK + 64) / 8;
      for (int idx = tid; idx < kZeroChunks; idx += WAVES * 64)
        *reinterpret_cast<uint4*>(xs + M * stride + idx * 8) = make_uint4(0u, 0u, 0u, 0u);
    }
    const int windows = (live_chunks + 63) / 64;
    if constexpr (FUSE == 2) {
      // Consumer of a fused launch: its weights do not depend on the
      // producers, so the first DEPTH units go out once ctl.stream_after
      // producers have finished (while the producers' last workgroups still
      // run); the activations are staged only once all of them have, with
      // device-coherent loads. Both flags of the line are then cleared for
      // the next call: no producer writes them again in this launch (the
      // stream flag was seen raised before the go flag was awaited).
      stream = weight_stream();
      const int* line = ctl.flags + static_cast<size_t>(block) * kFuseFlagInts;
      if (ctl.stream_after > 0) fuse_wait(ctl, line);
#pragma unroll
      for (int i = 0; i < DEPTH; ++i) {
        load_unit(buf[i], stream, i, lane);
        asm volatile("" ::: "memory");
      }
      fuse_wait(ctl, line + 1);
      if (tid == 0) {
        __hip_atomic_store(const_cast<int*>(line), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(const_cast<int*>(line) + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      for (int wi = wave; wi < M * windows; wi += WAVES) {
        const int m = wi / windows;
        const int c0 = (wi - m * windows) * 64;
        if (c0 + lane < live_chunks)
          lds_dma16_coherent(x + static_cast<size_t>(m) * K + kbase + (c0 + lane) * 8, xs + m * stride + c0 * 8);
      }
      __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
      __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    } else {
      for (int wi = wave; wi < M * windows; wi += WAVES) {
        const int m = wi / windows;
        const int c0 = (wi - m * windows) * 64;
        if (c0 + lane < live_chunks)
          lds_dma16(x + static_cast<size_t>(m) * K + kbase + (c0 + lane) * 8, xs + m * stride + c0 * 8);
      }
      __builtin_amdgcn_sched_barrier(0);
      stream = weight_stream();

      // Then issue the first DEPTH units of the weight stream unit by unit, in
      // the order the loop will consume them.
#pragma unroll
      for (int i = 0; i < DEPTH; ++i) {
        load_unit(buf[i], stream, i, lane);
        asm volatile("" ::: "memory");  // keep the units' loads in this order
      }
      // Wait for the staging loads only (they were issued before the weight
      // loads, and the counter retires loads in order) and for the zero
      // stores, then meet at a bare barrier: the weight loads stay in flight
      // across it. (A full __syncthreads would also wait for them.)
      __builtin_amdgcn_s_waitcnt(vmcnt_only(Unit<FMT>::kLoads * DEPTH));
      __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }

    const _Float16* xrow = xs + min(mcol, M - 1) * stride + g * 64 + wu0 * kUnitK;
    const _Float16* xr[kDotRows];
#pragma unroll
    for (int m = 0; m < kDotRows; ++m) xr[m] = xs + min(m, M - 1) * stride + g * 64 + wu0 * kUnitK;
    if constexpr (DOT == kDotBlockCols) {
      if (active) {
        // Block columns (M = 1): lane (j, g) reads x for steps 2p, 2p+1 where
        // j - 4g == p, and the zero region otherwise; only the x pointers
        // advance with the stream, so every offset of an iteration stays
        // inside the zero region.
        const int j = lane & 15;
        lds_half_ptr bp[4];
        int inc[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const bool mine = j - 4 * g == p;
          bp[p] = mine ? to_lds(xs + g * 64 + wu0 * kUnitK) : to_lds(xs + M * stride);
          inc[p] = mine ? DEPTH * kUnitK : 0;
        }
        const int sbase = (4 * g + 16 * (j >> 2)) * 4;
        const uint32_t ssel = static_cast<uint32_t>(j & 3) | (static_cast<uint32_t>(4 + (j & 3)) << 8) | 0x0C0C0000u;
        f4 sacc = {0.f, 0.f, 0.f, 0.f};
        for (int base = 0; base < wnu; base += DEPTH) {
#pragma unroll
          for (int i = 0; i < DEPTH; ++i) {
            if (base + i < wnu) {
              if constexpr (FMT == kFmtNvfp4) unit_block_cols(buf[i], bp, i * kUnitK, sbase, ssel, sacc);
            }
            load_unit(buf[i], stream, base + DEPTH + i, lane);
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int p = 0; p < 4; ++p) bp[p] += inc[p];
        }
        acc2[0] = sacc;
      }
    } else if (active) {
      // Each slot of buf is consumed and then refilled in place (unit u +
      // DEPTH goes where unit u was), so the loop carries no register copies
      // and keeps DEPTH-1 units in flight while it computes.
      for (int base = 0; base < wnu; base += DEPTH) {
#pragma unroll
        for (int i = 0; i < DEPTH; ++i) {
          if (base + i < wnu) {
            if constexpr (DOT > 0)
              unit_dot<kDotRows>(buf[i], xr, (base + i) * kUnitK, dacc);
            else
              unit_mfma(buf[i], xrow + (base + i) * kUnitK, acc2);
          }
          load_unit(buf[i], stream, base + DEPTH + i, lane);
          // keep the scheduler from sinking the refill below the next units' math
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  } else {
    // Ring stage: each K slice keeps the activations of three units in LDS
    // (slot c % 3 holds unit c of the slice, all M rows), and the workgroup
    // refills one slot per unit of the stream. The x pieces (8 halves of one
    // row) of a unit are loaded into registers DEPTH + 1 units ahead,
    // alongside the weights, and written to LDS one unit ahead; a barrier
    // per unit publishes the slot. Three slots suffice: the slot written at
    // step j was last read at step j - 2, which every wavefront has finished
    // once it has passed the barrier of step j - 1. The stage is
    // 3 * KS * M * 528 bytes whatever K is, so long K ranges need no split.
    const int slot_halves = M * kRingRow;
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<_Float16*>(x), 0, static_cast<uint32_t>(M) * K * 2, Stream::kRsrcWord3);
    // Piece p of a step: slice p / (32 M), row (p / 32) % M, 8 halves at q * 8
    // of the unit (q = p % 32). Lane tid loads pieces tid + i * WAVES * 64.
    const int pieces = KS * M * 32;
    uint32_t src0[XP];
    int dst0[XP], lim[XP], k0[XP];
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int p = tid + i * WAVES * 64;
      const int q = p & 31, r = p >> 5;
      const int m = r % M, slice = r / M;
      const int su0 = min(slice * sub, nu);
      lim[i] = p < pieces ? min(sub, nu - su0) : 0;  // units of the piece's slice
      k0[i] = (u0 + su0) * kUnitK + q * 8;
      src0[i] = (static_cast<uint32_t>(m) * K + k0[i]) * 2;
      dst0[i] = p < pieces ? (slice * kRingSlots * M + m) * kRingRow + q * 8 : -1;
    }
    // Pieces past the slice's units or past K load as zeros (out of the
    // buffer's range), so the zero-padded tail of the last unit meets 0.
    auto load_x = [&](u4 (&r)[XP], int c) {
#pragma unroll
      for (int i = 0; i < XP; ++i) {
        const bool live = c < lim[i] && k0[i] + c * kUnitK < K;
        r[i] = __builtin_amdgcn_raw_buffer_load_b128(xrs, live ? src0[i] + c * (kUnitK * 2) : 0x80000000u, 0, 0);
      }
    };
    auto store_x = [&](const u4 (&r)[XP], int c) {
#pragma unroll
      for (int i = 0; i < XP; ++i)
        if (dst0[i] >= 0) *reinterpret_cast<u4*>(xs + dst0[i] + (c % kRingSlots) * slot_halves) = r[i];
    };
    // LDS stores done, then a bare barrier: the loads stay in flight.
    auto publish = [&]() {
      __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    // Unit c's pieces live in xr[c % DEPTH] from their load to their store.
    u4 xr[DEPTH][XP];
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) load_x(xr[i], i);
    __builtin_amdgcn_sched_barrier(0);
    stream = weight_stream();
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) {
      load_unit(buf[i], stream, i, lane);
      asm volatile("" ::: "memory");
    }
    store_x(xr[0], 0);
    load_x(xr[0], DEPTH);
    publish();
    const _Float16* xrow = xs + ks * kRingSlots * slot_halves + min(mcol, M - 1) * kRingRow + g * 64;
    // Every wavefront runs the same steps (sub, rounded up to DEPTH), so
    // the barriers match; a wavefront past its own units only stages.
    for (int base = 0; base < sub; base += DEPTH) {
#pragma unroll
      for (int i = 0; i < DEPTH; ++i) {
        const int j = base + i;
        store_x(xr[(i + 1) % DEPTH], j + 1);
        load_x(xr[(i + 1) % DEPTH], j + 1 + DEPTH);
        publish();
        if (active && j < wnu) unit_mfma(buf[i], xrow + (j % kRingSlots) * slot_halves, acc2);
        load_unit(buf[i], stream, j + DEPTH, lane);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  f4 acc = acc2[0] + acc2[1];
  if constexpr (DOT == kDotBlockCols) {
    // Add the 16 block columns of each row (lanes of one K group, j = lane %
    // 16): every lane of the group ends with its rows' sums, so lane (0, g)
    // holds rows 4g .. 4g + 3 of activation row 0, the MFMA output layout the
    // rest of the kernel uses.
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) acc[r] += __shfl_xor(acc[r], o);
  }
  if constexpr (DOT > 0) {
    // Packed-dot path: add the four K groups' sums of each row (lanes 16
    // apart), then move them to the MFMA's output layout, where lane
    // (m, g) holds rows 4g .. 4g + 3 of column m, so the rest is shared.
#pragma unroll
    for (int m = 0; m < kDotRows; ++m) {
      dacc[m] += __shfl_xor(dacc[m], 16);
      dacc[m] += __shfl_xor(dacc[m], 32);
    }
#pragma unroll
    for (int m = 0; m < kDotRows; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = __shfl(dacc[m], g * 4 + r);
        if (mcol == m) acc[r] = v;
      }
  }

  // The KS slices of each n-tile are added through LDS, in slice order, into
  // the slice-0 wavefront. The staged activations are dead by now, so their
  // LDS (sized for this by the launcher) holds the partial tiles.
  if (KS > 1) {
    f4* red = reinterpret_cast<f4*>(xs);
    __syncthreads();
    red[wave * 64 + lane] = acc;
    __syncthreads();
    if (ks == 0) {
      for (int j = 1; j < KS; ++j) acc += red[(j * TN + tn) * 64 + lane];
    }
  }
  const bool owner = active && ks == 0;

  // Lane (m = lane % 16, g = lane / 16) holds rows n = 4g + r of column m.
  const int n0 = nt * kTileN + g * 4;
  const int Nh = N / 2;
  if (S == 1 && swiglu) {
    // The up wavefronts hand their scaled tiles to the gate wavefronts
    // through LDS (the activation stage is dead), which write
    // h = silu(gate) * up, rounded once to fp16.
    f4* xch = reinterpret_cast<f4*>(xs);
    __syncthreads();
    if (ks == 0 && tn >= half_tn) {
      f4 u = acc;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        u[r] *= FMT == kFmtNvfp4 ? tensor_scale : (n0 + r < N ? row_scales[n0 + r] : 0.f);
      xch[(tn - half_tn) * 64 + lane] = u;
    }
    __syncthreads();
    // N/2 is a multiple of 16 and n0 of 4: the lane's 4 rows are all inside
    // h or all past it, and their 8 bytes are aligned.
    if (owner && tn < half_tn && mcol < M && n0 < Nh) {
      const f4 u = xch[tn * 64 + lane];
      float hv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gv = acc[r] * (FMT == kFmtNvfp4 ? tensor_scale : row_scales[n0 + r]);
        hv[r] = silu(gv) * u[r];
      }
      put_h4<coherent_h>(static_cast<_Float16*>(y) + static_cast<size_t>(mcol) * Nh + n0, hv);
    }
    return;
  }
  // Greedy argmax: every row's best key over this group's logits (LDS
  // atomics, order-free), folded into the group's key slot with a
  // device-scope atomic max that nothing waits for. Max is order-free, so
  // the slots hold the same keys whatever order the groups run in;
  // argmax_decode_kernel, launched next on the stream, reads and clears them.
  auto argmax_finish = [&]() {
    __syncthreads();
    if (tid < M)
      __hip_atomic_fetch_max(amax.keys + (grp % kArgmaxSubs) * kMaxM + tid, best[tid], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  };
  if (argmax) {
    if (tid < M) best[tid] = 0;
    __syncthreads();
  }
  if (S == 1 && argmax) {
    if (owner && mcol < M) {
      unsigned long long k = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = n0 + r;
        if (n < N) {
          const unsigned long long kr =
              argmax_key(acc[r] * (FMT == kFmtNvfp4 ? tensor_scale : row_scales[n]), n);
          k = kr > k ? kr : k;
        }
      }
      __hip_atomic_fetch_max(&best[mcol], k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    argmax_finish();
    return;
  }
  if (S == 1) {
    if (owner && mcol < M) {
      const size_t row = static_cast<size_t>(mcol) * N;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = n0 + r;
        if (n < N) {
          const float scale = FMT == kFmtNvfp4 ? tensor_scale : row_scales[n];
          put_out<EPI>(y, row + n, acc[r] * scale);
        }
      }
    }
    return;
  }

  // K was split over S workgroups for this group of n-tiles: publish this
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
  if (owner && mcol < M) {
    float* dst = ws + (static_cast<size_t>(s) * M + mcol) * N;
    if (N % 4 == 0 && n0 + 3 < N) {
      store4_coherent(dst + n0, acc);  // 16-byte aligned: N % 4 == 0 and n0 % 4 == 0
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n0 + r < N) __hip_atomic_store(dst + n0 + r, acc[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    last_group = __hip_atomic_fetch_add(counters + grp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
  __syncthreads();
  if (!last_group) return;
  // Rows of the group: all TN tiles' rows, or (SwiGLU) the gate rows of its
  // TN/2 gate tiles, each combined with its up row N/2 further on.
  const int rows = (swiglu ? half_tn : TN) * kTileN;
  const int nbase = grp * rows;
  const int nend = swiglu ? Nh : N;
  const size_t range_stride = static_cast<size_t>(M) * N;
  for (int idx = tid; idx < M * rows; idx += WAVES * 64) {
    const int m = idx / rows;
    const int n = nbase + (idx - m * rows);
    if (n >= nend) continue;
    const float* src = ws + static_cast<size_t>(m) * N + n;
    const float sum = range_sum(src, range_stride, S) * (FMT == kFmtNvfp4 ? tensor_scale : row_scales[n]);
    if (swiglu) {
      const float u = range_sum(src + Nh, range_stride, S) *
                      (FMT == kFmtNvfp4 ? tensor_scale : row_scales[n + Nh]);
      put_h1<coherent_h>(static_cast<_Float16*>(y) + static_cast<size_t>(m) * Nh + n, silu(sum) * u);
    } else if (argmax) {
      __hip_atomic_fetch_max(&best[m], argmax_key(sum, n), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
      put_out<EPI>(y, static_cast<size_t>(m) * N + n, sum);
    }
  }
  if (tid == 0) __hip_atomic_store(counters + grp, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (argmax) argmax_finish();
}

}  // namespace
}  // namespace qpn
