// q4lin_device.h -- device-side building blocks shared by the q4lin kernels
// (gfx950 only).  Internal header: not part of the C ABI.
//
// Number formats (Q4_G64_FP16, "linear-benchmark.md" section 4 table; the
// value of a code q is (q - 8) * scale):
//   * a code dword holds 8 nibbles, k0..k7 from the least significant nibble
//     up (even k in the low nibble of each byte);
//   * the kernels pair nibble s with nibble s+4 of a dword, so one dword turns
//     into the four pairs (k0,k4) (k1,k5) (k2,k6) (k3,k7).  Activations are
//     staged in the same pair order, which leaves every dot product unchanged.
//   * weights enter the arithmetic as exact float16 values q - 8; activations
//     as float16 copies of the bf16 inputs scaled by a per-token power of two
//     2^-e (exact for every value within 2^38 of the token's largest
//     magnitude), undone in FP32 at the end.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace q4lin {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));


// float16 pair (q - 8) for the nibble pair (s, s+4): 0x6400 | q is 1024 + q
// exactly (fp16 quantum in [1024, 2048) is 1); subtracting 1032 is exact too.
__device__ __forceinline__ uint32_t f16_pair_q_minus_8(uint32_t w, int s) {
  uint32_t m = ((w >> s) & 0x000F000Fu) | 0x64006400u;
  f16x2_t v = __builtin_bit_cast(f16x2_t, m);
  const f16x2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
  v = v - off;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// binary32 -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// One output of the Q4 op formed again from its definition: per 64-group
// the exact sum of (q - 8) x in binary64 (each product exact), times the
// group's fp16 scale, summed over the groups in binary64 (plus the LinearAdd
// residual), rounded to bf16.  The matrix-core routes call it, one thread per
// output, for the rare outputs whose binary32 arithmetic came out non-finite
// (terms near the top of the binary32 range that cancel, or a binary32 sum
// that overflows although the exact sum does not); an output whose exact
// value overflows bf16 comes out as the same infinity again.
__device__ __attribute__((noinline)) inline uint16_t exact_q4_output(const uint16_t* __restrict__ x,
                                                                     const uint8_t* __restrict__ codes,
                                                                     const uint16_t* __restrict__ scales,
                                                                     const uint16_t* res, int N, int K, int n,
                                                                     int t) {
  const int G = K >> 6;
  const uint8_t* cr = codes + (size_t)n * (size_t)(K >> 1);
  const uint16_t* xr = x + (size_t)t * (size_t)K;
  double acc = 0.0;
  for (int g = 0; g < G; ++g) {
    double p = 0.0;
    for (int j = 0; j < 32; ++j) {
      const uint32_t b = cr[32 * g + j];
      p += (double)((int)(b & 15u) - 8) * (double)bf16_bits_to_f32(xr[64 * g + 2 * j]);
      p += (double)((int)(b >> 4) - 8) * (double)bf16_bits_to_f32(xr[64 * g + 2 * j + 1]);
    }
    acc += (double)f16_bits_to_f32(scales[(size_t)n * (size_t)G + g]) * p;
  }
  if (res != nullptr) acc += (double)bf16_bits_to_f32(res[(size_t)t * (size_t)N + n]);
  return f32_to_bf16_rne((float)acc);
}

// Lane sums of a binary64 value without LDS round trips.  Each step adds
// the value of a partner lane from the other half of the group being merged
// (a pairing that is its own inverse), so every lane of the group ends with
// the same bits (a + b == b + a).  DPP moves inside a row of 16 lanes
// (quad_perm [1,0,3,2] and [2,3,0,1], then the mirror of each half-row and
// of the row), the gfx950 lane swaps across rows (v_permlane16_swap: rows 0
// and 1, 2 and 3; v_permlane32_swap: the two halves of the wave).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// sum over each aligned group of 8 lanes
__device__ __forceinline__ double sum8_lanes(double v) {
  v += dpp_f64<0xB1>(v);   // quad_perm [1,0,3,2]: lane pairs
  v += dpp_f64<0x4E>(v);   // quad_perm [2,3,0,1]: the quads
  v += dpp_f64<0x141>(v);  // row_half_mirror: the other quad of the eight
  return v;
}
// sum over all 64 lanes (every lane active)
__device__ __forceinline__ double sum64_lanes(double v) {
  v = sum8_lanes(v);
  v += dpp_f64<0x140>(v);  // row_mirror: the other eight of the row
  {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const auto l = __builtin_amdgcn_permlane16_swap((uint32_t)b, (uint32_t)b, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
    v = __builtin_bit_cast(double, ((uint64_t)h[0] << 32) | l[0]) +
        __builtin_bit_cast(double, ((uint64_t)h[1] << 32) | l[1]);
  }
  {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const auto l = __builtin_amdgcn_permlane32_swap((uint32_t)b, (uint32_t)b, false, false);
    const auto h = __builtin_amdgcn_permlane32_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
    v = __builtin_bit_cast(double, ((uint64_t)h[0] << 32) | l[0]) +
        __builtin_bit_cast(double, ((uint64_t)h[1] << 32) | l[1]);
  }
  return v;
}

template <int V>
using Slot = std::integral_constant<int, V>;

// Calls f(Slot<0>{}) ... f(Slot<N-1>{}) (compile-time unrolled loop).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(Slot<I>{});
    static_for<N, I + 1>(f);
  }
}

}  // namespace q4lin
