// Device-side building blocks shared by the libqpn kernels: the packed weight
// layout, fp4/fp8 -> fp16 decode and fp32 -> E2M1/E4M3 encoders.
//
// Packed layout (opaque to callers; produced by the pack kernels).
// W[N, K] is cut into n-tiles of 16 rows and units of 256 elements along K,
// padded with zero weights. Tile-unit (nt, u) lives at byte
// ((u * NT) + nt) * UNIT_BYTES, NT = ceil(N / 16): units are stored K-major,
// so the wavefronts that stream neighbouring n-tiles in step read one
// contiguous window of HBM at a time rather than thousands of scattered
// ones. Lane l of a 64-wide
// wavefront owns row r = l % 16 of the tile and the 64-element slice
// k = u*256 + g*64 + [0, 64) with g = l / 16. Its bytes come as 16-byte
// vectors at stride 1024, so one global_load_dwordx4 per vector brings
// 1 KB of the stream to the wavefront, fully coalesced:
//   NVFP4 (2304 B): vectors h = 0,1 at h*1024 + l*16 hold the 32 E2M1 codes
//          of k = ... + h*32 + [0, 32) (canonical nibble order); the four
//          E4M3 block scales of the lane's 64 elements are the 4 bytes at
//          2048 + l*4.
//   FP8 (4096 B):  vectors q = 0..3 at q*1024 + l*16 hold the 16 E4M3 codes
//          of k = ... + q*16 + [0, 16).
// In both formats step t = 0..7 of a unit covers k = u*256 + g*64 + t*8 + e,
// e = 0..7: exactly the 8 fp16 values lane l feeds one 16x16x32 MFMA, so the
// same activation fragment layout serves both formats.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qpn_plan.hpp"

namespace qpn {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));


// s_waitcnt immediate that waits until at most n vector memory operations
// are outstanding and leaves the other counters alone (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// ... and the same for the LDS / scalar-memory counter (vmcnt left at 63).
constexpr int lgkmcnt_only(int n) { return 15 | (3 << 14) | (7 << 4) | ((n & 15) << 8); }

template <int FMT>
struct Unit;

template <>
struct Unit<kFmtNvfp4> {
  static constexpr int kBytes = kNvUnitBytes;
  static constexpr int kLoads = 3;  // vector memory instructions per unit
  u4 c0, c1;
  uint32_t sc;
};

template <>
struct Unit<kFmtFp8> {
  static constexpr int kBytes = kF8UnitBytes;
  static constexpr int kLoads = 4;
  u4 q[4];
};

// Byte offset of tile-unit (nt, u) in a packed buffer with NT n-tiles.
__host__ __device__ constexpr int64_t unit_offset(int64_t nt, int64_t u, int64_t NT, int64_t unit_bytes) {
  return (u * NT + nt) * unit_bytes;
}

// One wavefront's units of one n-tile, read with raw buffer loads: the 64-bit
// base, the byte range and the unit stride sit in scalar registers, per-lane
// offsets are 32-bit, and a load past `bytes` returns zeros instead of
// faulting.
struct Stream {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t stride;  // bytes from one unit of the tile to the next
  Stream() = default;  // set up later, with the constructor below
  __device__ __forceinline__ Stream(const uint8_t* base, uint32_t bytes, uint32_t unit_stride)
      : rsrc(__builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, bytes, kRsrcWord3)),
        stride(unit_stride) {}
  static constexpr int kRsrcWord3 = 0x00020000;
  static constexpr int kStreaming = 2;  // nt: the weights are read once
};

// Streaming loads of unit `u` (counted from the stream's first unit).
__device__ __forceinline__ void load_unit(Unit<kFmtNvfp4>& r, const Stream& s, int u, int lane) {
  const int base = u * s.stride;
  r.c0 = __builtin_amdgcn_raw_buffer_load_b128(s.rsrc, lane * 16, base, Stream::kStreaming);
  r.c1 = __builtin_amdgcn_raw_buffer_load_b128(s.rsrc, lane * 16 + 1024, base, Stream::kStreaming);
  r.sc = __builtin_amdgcn_raw_buffer_load_b32(s.rsrc, lane * 4 + 2048, base, Stream::kStreaming);
}

__device__ __forceinline__ void load_unit(Unit<kFmtFp8>& r, const Stream& s, int u, int lane) {
  const int base = u * s.stride;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    r.q[q] = __builtin_amdgcn_raw_buffer_load_b128(s.rsrc, lane * 16 + q * 1024, base, Stream::kStreaming);
}

__device__ __forceinline__ uint32_t word(const u4& v, int i) { return v[i]; }

__device__ __forceinline__ h8 cat(h2 a, h2 b, h2 c, h2 d) {
  return h8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Eight E2M1 codes (one dword, element e in nibble e) times one block scale,
// as the fp16 A-fragment of one MFMA step. E2M1 * E4M3 has at most 6
// significant bits and lies in [2^-10, 2688], so every product is exact fp16.
__device__ __forceinline__ h8 decode_fp4x8(uint32_t codes, h2 scale) {
  h2 a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * scale;
  h2 a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * scale;
  h2 a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * scale;
  h2 a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * scale;
  return cat(a0, a1, a2, a3);
}

// Eight E4M3 codes (two dwords, element e in byte e) as fp16; exact, since
// every E4M3 value is an fp16 value.
__device__ __forceinline__ h8 decode_fp8x8(uint32_t lo, uint32_t hi) {
  h2 a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  h2 a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  h2 a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  h2 a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return cat(a0, a1, a2, a3);
}

// fp32 -> E4M3FN code: nearest, ties to even, saturating at 448, sign copied.
// Works on the fp32 bit pattern: below 2^-6 the code is the integer
// round-to-even of |v| * 2^9 (0..8, 8 being the smallest normal); above, the
// 23-bit mantissa is rounded to 3 bits with the carry running into the
// exponent, and the exponent is rebiased from 127 to 7.
__device__ __forceinline__ uint32_t encode_e4m3(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {
    code = static_cast<uint32_t>(rintf(a * 512.0f));
  } else {
    const uint32_t b = __float_as_uint(a);
    const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  }
  return sign | code;
}

// E4M3FN code -> fp32 value (exact), from the bit fields.
__device__ __forceinline__ float decode_e4m3(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20))
                      : static_cast<float>(m) * 0.001953125f;
  return (c & 0x80u) ? -mag : mag;
}

// fp32 -> E2M1 code: nearest, ties to even, saturating at 6, sign copied.
// The magnitude code counts the midpoints of {0,.5,1,1.5,2,3,4,6} that |v|
// passes; at a midpoint the comparison is strict when the lower neighbour has
// an even code (0.25, 1.25, 2.5, 5) and inclusive when the upper one does.
__device__ __forceinline__ uint32_t encode_e2m1(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 28) & 0x8u;
  const float a = fabsf(v);
  const uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) +
                     (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return sign | c;
}

}  // namespace qpn
