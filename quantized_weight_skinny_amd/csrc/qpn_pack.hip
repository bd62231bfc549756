// Offline kernels around the GEMM: canonical <-> packed layout, the
// synthetic-weight quantizers, absmax and the read-only bandwidth probe.
//
// The packed layout is described in qpn_device.hpp. Every pack kernel writes
// each byte of the packed buffer exactly once (padding included), so the
// buffer needs no clearing first.
#include "qpn_device.hpp"
#include "qpn_internal.hpp"

namespace qpn {
namespace {

constexpr int kBlock = 256;

__device__ __forceinline__ uint4 load16_bytes(const uint8_t* src, int nbytes) {
  // nbytes in {0, 8, 16}; 16-byte vector loads when aligned, bytes otherwise.
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (nbytes == 16 && (reinterpret_cast<uintptr_t>(src) & 15u) == 0) return *reinterpret_cast<const uint4*>(src);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  for (int i = 0; i < nbytes; ++i) w[i >> 2] |= static_cast<uint32_t>(src[i]) << (8 * (i & 3));
  v.x = w[0]; v.y = w[1]; v.z = w[2]; v.w = w[3];
  return v;
}

__device__ __forceinline__ void store16_bytes(uint8_t* dst, uint4 v, int nbytes) {
  if (nbytes == 16 && (reinterpret_cast<uintptr_t>(dst) & 15u) == 0) {
    *reinterpret_cast<uint4*>(dst) = v;
    return;
  }
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  for (int i = 0; i < nbytes; ++i) dst[i] = static_cast<uint8_t>(w[i >> 2] >> (8 * (i & 3)));
}

__device__ __forceinline__ int count_nan_e4m3(uint32_t w, int nbytes) {
  int bad = 0;
  for (int i = 0; i < nbytes; ++i) bad += ((w >> (8 * i)) & 0x7Fu) == 0x7Fu;
  return bad;
}

// NVFP4 block scales are positive E4M3 values: a NaN code or any code with
// the sign bit set (including -0) is invalid.
__device__ __forceinline__ int count_bad_block_scales(uint32_t w, int nbytes) {
  int bad = 0;
  for (int i = 0; i < nbytes; ++i) {
    const uint32_t b = (w >> (8 * i)) & 0xFFu;
    bad += b >= 0x80u || b == 0x7Fu;
  }
  return bad;
}

// One thread per 32-code chunk (16 bytes) of a padded row.
__global__ __launch_bounds__(kBlock) void pack_nvfp4_codes(const uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ packed, int64_t N,
                                                           int64_t K, int64_t NT, int64_t KU, int64_t total) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (idx >= total) return;
  const int64_t n = idx / (KU * 8);
  const int64_t c = idx - n * (KU * 8);
  const int64_t k0 = c * 32;
  const int64_t u = c >> 3, g = (c >> 1) & 3, h = c & 1;
  const int64_t nt = n >> 4, r = n & 15;
  uint8_t* dst = packed + unit_offset(nt, u, NT, kNvUnitBytes) + h * 1024 + (g * 16 + r) * 16;
  int nbytes = 0;
  if (n < N && k0 < K) nbytes = static_cast<int>((K - k0) / 2 < 16 ? (K - k0) / 2 : 16);
  const uint4 v = load16_bytes(codes + n * (K / 2) + k0 / 2, nbytes);
  *reinterpret_cast<uint4*>(dst) = v;
}

// One thread per group of 4 block scales (64 elements) of a padded row.
__global__ __launch_bounds__(kBlock) void pack_nvfp4_scales(const uint8_t* __restrict__ scales,
                                                            uint8_t* __restrict__ packed, int64_t N,
                                                            int64_t K, int64_t NT, int64_t KU, int64_t total,
                                                            int32_t* __restrict__ bad) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (idx >= total) return;
  const int64_t n = idx / (KU * 4);
  const int64_t q = idx - n * (KU * 4);
  const int64_t u = q >> 2, g = q & 3;
  const int64_t nt = n >> 4, r = n & 15;
  const int64_t nblk = K / 16;
  uint32_t w = 0u;
  int nvalid = 0;
  if (n < N) {
    for (int i = 0; i < 4; ++i) {
      const int64_t b = q * 4 + i;
      if (b < nblk) {
        w |= static_cast<uint32_t>(scales[n * nblk + b]) << (8 * i);
        nvalid = i + 1;
      }
    }
  }
  *reinterpret_cast<uint32_t*>(packed + unit_offset(nt, u, NT, kNvUnitBytes) + 2048 + (g * 16 + r) * 4) = w;
  if (bad) {
    const int nb = count_bad_block_scales(w, nvalid);
    if (nb) atomicAdd(bad, nb);
  }
}

// One thread per 16-code chunk of a padded row.
__global__ __launch_bounds__(kBlock) void pack_fp8_codes(const uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ packed, int64_t N,
                                                         int64_t K, int64_t NT, int64_t KU, int64_t total,
                                                         int32_t* __restrict__ bad) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (idx >= total) return;
  const int64_t n = idx / (KU * 16);
  const int64_t c = idx - n * (KU * 16);
  const int64_t k0 = c * 16;
  const int64_t u = c >> 4, g = (c >> 2) & 3, q = c & 3;
  const int64_t nt = n >> 4, r = n & 15;
  uint8_t* dst = packed + unit_offset(nt, u, NT, kF8UnitBytes) + q * 1024 + (g * 16 + r) * 16;
  const int nbytes = (n < N && k0 < K) ? 16 : 0;
  const uint4 v = load16_bytes(codes + n * K + k0, nbytes);
  *reinterpret_cast<uint4*>(dst) = v;
  if (bad && nbytes) {
    const int nb = count_nan_e4m3(v.x, 4) + count_nan_e4m3(v.y, 4) + count_nan_e4m3(v.z, 4) +
                   count_nan_e4m3(v.w, 4);
    if (nb) atomicAdd(bad, nb);
  }
}

// One thread per 32-code chunk of a row (total = n * KU * 8, so every row
// index is below n).
__global__ __launch_bounds__(kBlock) void unpack_nvfp4_kernel(const uint8_t* __restrict__ packed,
                                                              uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales, int64_t K,
                                                              int64_t NT, int64_t KU, int64_t total) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (idx >= total) return;
  const int64_t n = idx / (KU * 8);
  const int64_t c = idx - n * (KU * 8);
  const int64_t k0 = c * 32;
  if (k0 >= K) return;
  const int64_t u = c >> 3, g = (c >> 1) & 3, h = c & 1;
  const int64_t nt = n >> 4, r = n & 15;
  const uint8_t* unit = packed + unit_offset(nt, u, NT, kNvUnitBytes);
  const uint4 v = *reinterpret_cast<const uint4*>(unit + h * 1024 + (g * 16 + r) * 16);
  const int nbytes = static_cast<int>((K - k0) / 2 < 16 ? (K - k0) / 2 : 16);
  store16_bytes(codes + n * (K / 2) + k0 / 2, v, nbytes);
  if (h == 0) {  // the chunk at the start of each 64-element group also copies its scales
    const uint32_t w = *reinterpret_cast<const uint32_t*>(unit + 2048 + (g * 16 + r) * 4);
    const int64_t nblk = K / 16;
    for (int i = 0; i < 4; ++i) {
      const int64_t b = (k0 / 64) * 4 + i;
      if (b < nblk) scales[n * nblk + b] = static_cast<uint8_t>(w >> (8 * i));
    }
  }
}

// One thread per 16-code chunk of a row (total = n * KU * 16).
__global__ __launch_bounds__(kBlock) void unpack_fp8_kernel(const uint8_t* __restrict__ packed,
                                                            uint8_t* __restrict__ codes, int64_t K,
                                                            int64_t NT, int64_t KU, int64_t total) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (idx >= total) return;
  const int64_t n = idx / (KU * 16);
  const int64_t c = idx - n * (KU * 16);
  const int64_t k0 = c * 16;
  if (k0 >= K) return;
  const int64_t u = c >> 4, g = (c >> 2) & 3, q = c & 3;
  const int64_t nt = n >> 4, r = n & 15;
  const uint4 v = *reinterpret_cast<const uint4*>(packed + unit_offset(nt, u, NT, kF8UnitBytes) + q * 1024 +
                                                  (g * 16 + r) * 16);
  store16_bytes(codes + n * K + k0, v, 16);
}

__global__ void absmax_init(uint32_t* out) { out[0] = 0u; }

// max |x| as the maximum of the sign-cleared fp32 bit patterns: for finite
// values and infinities the unsigned order of those patterns is the numeric
// order, and every NaN pattern lies above +inf, so a NaN anywhere wins.
__global__ __launch_bounds__(kBlock) void absmax_kernel(const float* __restrict__ x, int64_t count,
                                                        uint32_t* __restrict__ out) {
  uint32_t m = 0u;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < count; i += stride) {
    const uint32_t b = __float_as_uint(x[i]) & 0x7FFFFFFFu;
    m = b > m ? b : m;
  }
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off, 64));
    m = o > m ? o : m;
  }
  if ((threadIdx.x & 63) == 0 && m) atomicMax(out, m);
}

// The NVFP4 recipe for one 16-element block: its E4M3 scale (returned) and
// 16 E2M1 codes, element i in nibble i of lo:hi.
__device__ __forceinline__ uint32_t nvfp4_block(const float (&v)[16], float s_t, uint32_t& lo, uint32_t& hi) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t sc = encode_e4m3((amax / 6.0f) / s_t);
  const float d = decode_e4m3(sc) * s_t;
  lo = 0u;
  hi = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t c = d == 0.f ? ((__float_as_uint(v[i]) >> 28) & 0x8u) : encode_e2m1(v[i] / d);
    if (i < 8) lo |= c << (4 * i);
    else hi |= c << (4 * (i - 8));
  }
  return sc;
}

__device__ __forceinline__ void store_nvfp4_block(uint8_t* codes, uint8_t* scales, int64_t K, int64_t n,
                                                  int64_t b, int64_t idx, uint32_t lo, uint32_t hi,
                                                  uint32_t sc) {
  uint8_t* dst = codes + n * (K / 2) + b * 8;
  if ((reinterpret_cast<uintptr_t>(dst) & 7u) == 0) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
  } else {
    for (int i = 0; i < 4; ++i) dst[i] = static_cast<uint8_t>(lo >> (8 * i));
    for (int i = 0; i < 4; ++i) dst[4 + i] = static_cast<uint8_t>(hi >> (8 * i));
  }
  scales[idx] = static_cast<uint8_t>(sc);
}

// One thread per 16-element block of a row.
__global__ __launch_bounds__(kBlock) void quantize_nvfp4_kernel(const float* __restrict__ w,
                                                                int64_t N, int64_t K, float s_t,
                                                                uint8_t* __restrict__ codes,
                                                                uint8_t* __restrict__ scales) {
  const int64_t nblk = K / 16;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (idx >= N * nblk) return;
  const int64_t n = idx / nblk, b = idx - n * nblk;
  const float* src = w + n * K + b * 16;
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = src[i];
  uint32_t lo, hi;
  const uint32_t sc = nvfp4_block(v, s_t, lo, hi);
  store_nvfp4_block(codes, scales, K, n, b, idx, lo, hi, sc);
}

// FP8 -> NVFP4 ([P3] "v1.0 got us here...": the first version converted the
// checkpoint's FP8 regions to NVFP4). Each FP8 value is first the fp32 it
// stands for, E4M3 value times the row scale (one rounding), then the block
// is quantized as above.
__global__ __launch_bounds__(kBlock) void requantize_fp8_nvfp4_kernel(const uint8_t* __restrict__ f8,
                                                                      const float* __restrict__ row_scales,
                                                                      int64_t N, int64_t K, float s_t,
                                                                      uint8_t* __restrict__ codes,
                                                                      uint8_t* __restrict__ scales) {
  const int64_t nblk = K / 16;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (idx >= N * nblk) return;
  const int64_t n = idx / nblk, b = idx - n * nblk;
  const uint8_t* src = f8 + n * K + b * 16;
  const float s_n = row_scales[n];
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = decode_e4m3(src[i]) * s_n;
  uint32_t lo, hi;
  const uint32_t sc = nvfp4_block(v, s_t, lo, hi);
  store_nvfp4_block(codes, scales, K, n, b, idx, lo, hi, sc);
}

// max |E4M3(c) * s_n| over an FP8 weight: per row the largest code
// magnitude (the E4M3 order is the order of its magnitude bits), decoded and
// scaled, as fp32 bits for the integer max. One workgroup per row.
__global__ __launch_bounds__(kBlock) void fp8_absmax_kernel(const uint8_t* __restrict__ f8,
                                                            const float* __restrict__ row_scales, int64_t K,
                                                            uint32_t* __restrict__ out) {
  const int64_t n = blockIdx.x;
  const uint8_t* src = f8 + n * K;
  uint32_t m = 0u;
  for (int64_t i = threadIdx.x; i < K; i += kBlock) {
    const uint32_t c = src[i] & 0x7Fu;
    m = c > m ? c : m;
  }
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off, 64));
    m = o > m ? o : m;
  }
  if ((threadIdx.x & 63) == 0 && m) {
    const uint32_t b = __float_as_uint(fabsf(decode_e4m3(m) * row_scales[n]));
    if (b) atomicMax(out, b);
  }
}

// One workgroup per row: row absmax, then the codes.
__global__ __launch_bounds__(kBlock) void quantize_fp8_kernel(const float* __restrict__ w, int64_t K,
                                                              uint8_t* __restrict__ codes,
                                                              float* __restrict__ row_scales) {
  __shared__ float red[kBlock / 64];
  const int64_t n = blockIdx.x;
  const float* src = w + n * K;
  float amax = 0.f;
  for (int64_t i = threadIdx.x; i < K; i += kBlock) amax = fmaxf(amax, fabsf(src[i]));
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float s = amax / 448.0f;
  if (s == 0.f) s = 1.0f;
  if (threadIdx.x == 0) row_scales[n] = s;
  uint8_t* dst = codes + n * K;
  for (int64_t i = threadIdx.x; i < K; i += kBlock) dst[i] = static_cast<uint8_t>(encode_e4m3(src[i] / s));
}

// Read-only stream: U 16-byte loads in flight per thread (grid-stride),
// XOR-folded so the loads stay live; one word per wavefront is written.
template <int U>
__global__ __launch_bounds__(kBlock) void read_ceiling_kernel(const u4* __restrict__ buf,
                                                              int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u4 v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) v[j] = __builtin_nontemporal_load(buf + i + j * stride);
#pragma unroll
    for (int j = 0; j < U; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; i < n16; i += stride) {
    const u4 a = __builtin_nontemporal_load(buf + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), off, 64));
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6)] = acc;
}

unsigned blocks_for(int64_t total) { return static_cast<unsigned>(ceil_div(total, kBlock)); }

}  // namespace

hipError_t launch_pack_nvfp4(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                             void* packed, int32_t* bad, hipStream_t stream) {
  const int64_t NT = ceil_div(n, kTileN), KU = ceil_div(k, kUnitK);
  if (NT == 0 || KU == 0) return hipSuccess;
  const int64_t rows = NT * kTileN;
  const int64_t t1 = rows * KU * 8;
  hipLaunchKernelGGL(pack_nvfp4_codes, dim3(blocks_for(t1)), dim3(kBlock), 0, stream, codes,
                     static_cast<uint8_t*>(packed), n, k, NT, KU, t1);
  const int64_t t2 = rows * KU * 4;
  hipLaunchKernelGGL(pack_nvfp4_scales, dim3(blocks_for(t2)), dim3(kBlock), 0, stream, scales,
                     static_cast<uint8_t*>(packed), n, k, NT, KU, t2, bad);
  return hipGetLastError();
}

hipError_t launch_pack_fp8(const uint8_t* codes, int64_t n, int64_t k, void* packed, int32_t* bad,
                           hipStream_t stream) {
  const int64_t NT = ceil_div(n, kTileN), KU = ceil_div(k, kUnitK);
  if (NT == 0 || KU == 0) return hipSuccess;
  const int64_t t = NT * kTileN * KU * 16;
  hipLaunchKernelGGL(pack_fp8_codes, dim3(blocks_for(t)), dim3(kBlock), 0, stream, codes,
                     static_cast<uint8_t*>(packed), n, k, NT, KU, t, bad);
  return hipGetLastError();
}

hipError_t launch_unpack_nvfp4(const void* packed, int64_t n, int64_t k, uint8_t* codes,
                               uint8_t* scales, hipStream_t stream) {
  const int64_t NT = ceil_div(n, kTileN), KU = ceil_div(k, kUnitK);
  if (n == 0 || KU == 0) return hipSuccess;
  const int64_t t = n * KU * 8;
  hipLaunchKernelGGL(unpack_nvfp4_kernel, dim3(blocks_for(t)), dim3(kBlock), 0, stream,
                     static_cast<const uint8_t*>(packed), codes, scales, k, NT, KU, t);
  return hipGetLastError();
}

hipError_t launch_unpack_fp8(const void* packed, int64_t n, int64_t k, uint8_t* codes,
                             hipStream_t stream) {
  const int64_t NT = ceil_div(n, kTileN), KU = ceil_div(k, kUnitK);
  if (n == 0 || KU == 0) return hipSuccess;
  const int64_t t = n * KU * 16;
  hipLaunchKernelGGL(unpack_fp8_kernel, dim3(blocks_for(t)), dim3(kBlock), 0, stream,
                     static_cast<const uint8_t*>(packed), codes, k, NT, KU, t);
  return hipGetLastError();
}

hipError_t launch_absmax(const float* x, int64_t count, float* out, hipStream_t stream) {
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
  hipLaunchKernelGGL(absmax_init, dim3(1), dim3(1), 0, stream, o);
  if (count > 0) {
    int64_t blocks = ceil_div(count, kBlock * 16);
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(absmax_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, stream, x,
                       count, o);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_nvfp4(const float* w, int64_t n, int64_t k, float tensor_scale,
                                 uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t t = n * (k / 16);
  if (t == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_nvfp4_kernel, dim3(blocks_for(t)), dim3(kBlock), 0, stream, w, n, k,
                     tensor_scale, codes, scales);
  return hipGetLastError();
}

hipError_t launch_fp8_absmax(const uint8_t* codes, const float* row_scales, int64_t n, int64_t k, float* out,
                             hipStream_t stream) {
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
  hipLaunchKernelGGL(absmax_init, dim3(1), dim3(1), 0, stream, o);
  if (n > 0 && k > 0)
    hipLaunchKernelGGL(fp8_absmax_kernel, dim3(static_cast<unsigned>(n)), dim3(kBlock), 0, stream, codes,
                       row_scales, k, o);
  return hipGetLastError();
}

hipError_t launch_requantize_fp8_nvfp4(const uint8_t* f8, const float* row_scales, int64_t n, int64_t k,
                                       float tensor_scale, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t t = n * (k / 16);
  if (t == 0) return hipSuccess;
  hipLaunchKernelGGL(requantize_fp8_nvfp4_kernel, dim3(blocks_for(t)), dim3(kBlock), 0, stream, f8, row_scales,
                     n, k, tensor_scale, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const float* w, int64_t n, int64_t k, uint8_t* codes,
                               float* row_scales, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_fp8_kernel, dim3(static_cast<unsigned>(n)), dim3(kBlock), 0, stream, w,
                     k, codes, row_scales);
  return hipGetLastError();
}

int read_ceiling_default_grid() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      cus = v;
  }
  return cus * 8;
}

hipError_t launch_read_ceiling(const void* buf, size_t bytes, uint32_t* sink, int grid, int loads,
                               hipStream_t stream) {
  const u4* b = static_cast<const u4*>(buf);
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  const dim3 g(static_cast<unsigned>(grid)), t(kBlock);
  switch (loads) {
    case 2: hipLaunchKernelGGL(read_ceiling_kernel<2>, g, t, 0, stream, b, n16, sink); break;
    case 8: hipLaunchKernelGGL(read_ceiling_kernel<8>, g, t, 0, stream, b, n16, sink); break;
    default: hipLaunchKernelGGL(read_ceiling_kernel<4>, g, t, 0, stream, b, n16, sink); break;
  }
  return hipGetLastError();
}

}  // namespace qpn
