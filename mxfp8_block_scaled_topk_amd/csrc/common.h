// Internal helpers shared by the HIP kernels and the host entry points.
// Device side: bf16 and MX (e4m3 payload + e8m0 scale) conversions done in
// registers.  Host side: thread-local error reporting and launch checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <initializer_list>

#include "../../include/mxmoe.h"

namespace mxmoe {

// ---------------------------------------------------------------------------
// host
// ---------------------------------------------------------------------------

// Records a printf-style message for mx_last_error() and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Maps a pending launch error to MX_ERR_HIP (with the kernel's name).
int check_launch(const char* what);

// Number of compute units of the current device (cached per device).
int num_cus();

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Expert-weight formats of the grouped GEMMs: e4m3 rows [E, N, Kd]; MXFP4
// (packed e2m1) rows [E, N, Kd/2]; e4m3 in the tile-packed layout that
// mx_pack_weights writes.
constexpr int kWfE4m3 = 0, kWfE2m1 = 1, kWfPacked = 2;

// Largest value any size argument may take (MX_ERR_UNSUPPORTED above it).
// With every dimension at most 2^31 - 1, the host's products of two sizes
// stay far inside int64_t, so no size arithmetic can overflow.
constexpr int64_t kMaxDim = ((int64_t)1 << 31) - 1;

// True when every value lies in [0, kMaxDim].
inline bool dims_in_range(std::initializer_list<int64_t> dims) {
  for (int64_t d : dims)
    if (d < 0 || d > kMaxDim) return false;
  return true;
}

constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// device: number formats
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even float32 -> bf16 bit pattern (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// e8m0 scale byte of a block from its largest magnitude (amax >= 0, finite):
// s = floor(log2 amax) - 8 clamped to [-127, 127], byte = s + 127.  For a
// normal amax the biased exponent field is floor(log2 amax) + 127, so the
// byte is that field minus 8; a zero or subnormal amax gives byte 0.
__device__ __forceinline__ uint32_t e8m0_from_amax(float amax) {
  int field = static_cast<int>(__float_as_uint(amax) >> 23);
  return static_cast<uint32_t>(field > 8 ? field - 8 : 0);
}

// 2^-s for scale byte b (s = b - 127) as a float: biased exponent 254 - b,
// which stays in [8, 254] for every byte the quantiser emits.
__device__ __forceinline__ float e8m0_inverse(uint32_t b) {
  return __uint_as_float((254u - b) << 23);
}

// Four values already divided by the block scale -> four e4m3 bytes packed
// little-endian.  The hardware convert rounds to nearest even and keeps the
// sign of zero, but returns NaN above the largest finite value instead of
// saturating, so inputs are clamped to +-448 first.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  c = fminf(fmaxf(c, -448.0f), 448.0f);
  d = fminf(fmaxf(d, -448.0f), 448.0f);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}

// MX-quantise one 32-element block held in registers.
// Returns the scale byte; writes 32 payload bytes into q[0..7].
__device__ __forceinline__ uint32_t mx_block32(const float (&v)[32], uint32_t (&q)[8]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  uint32_t sb = e8m0_from_amax(amax);
  float inv = e8m0_inverse(sb);
#pragma unroll
  for (int w = 0; w < 8; ++w)
    q[w] = e4m3x4(v[4 * w] * inv, v[4 * w + 1] * inv, v[4 * w + 2] * inv, v[4 * w + 3] * inv);
  return sb;
}

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active) by DPP
// data movement, no LDS: shifts by 1, 2, 4 and 8 lanes inside each row of 16
// lanes (a lane whose source falls outside its row adds 0), then lane 15's
// running total added to row 1 and lane 47's to row 3 (row_bcast:15 under
// row mask 0b1010), then lane 31's to rows 2 and 3 (row_bcast:31 under row
// mask 0b1100).
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return x;
}

// Eight bf16 values packed in a uint4 -> floats.
__device__ __forceinline__ void unpack_bf16x8(const uint4& u, float* f) {
  f[0] = __uint_as_float(u.x << 16); f[1] = __uint_as_float(u.x & 0xFFFF0000u);
  f[2] = __uint_as_float(u.y << 16); f[3] = __uint_as_float(u.y & 0xFFFF0000u);
  f[4] = __uint_as_float(u.z << 16); f[5] = __uint_as_float(u.z & 0xFFFF0000u);
  f[6] = __uint_as_float(u.w << 16); f[7] = __uint_as_float(u.w & 0xFFFF0000u);
}

}  // namespace mxmoe
