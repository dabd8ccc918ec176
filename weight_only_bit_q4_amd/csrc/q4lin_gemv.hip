// q4lin_gemv.hip -- the few-token route (T = 1..4): vector-ALU dot products.
//
// The pages' prior art for T = 1 is a row-split GEMV ("q4-linear.md", notes
// under the result table: T = 1 uses a dedicated single-token GEMV); this is an
// MI355X design of the same step, not a translation.
//
// Work mapping.  A workgroup of 256 threads (4 wave64s) owns 16 consecutive
// rows; every wave owns 4 rows and gives each row a quarter-wave of 16 lanes.
// A row's codes are cut into 16-byte chunks (32 weights, half a 64-group);
// lane j of a quarter takes chunks j, j+16, j+32, ...  Each lane issues a
// whole batch of chunk loads before touching the activations, so the weight
// stream is in flight early (the op is HBM-bound at few tokens).
//
// Arithmetic.  Nibbles become exact float16 values q - 8 (f16_pair_q_minus_8)
// and meet the activations in v_dot2_f32_f16 with FP32 accumulation; each
// chunk's sum is multiplied by its group's FP16 scale in FP32.  The
// activations are float16 copies of the bf16 inputs scaled by 2^-e[t], with
// e[t] chosen from the token's largest magnitude so that every bf16 value
// within 2^38 of it converts exactly; the workgroup stages all T tokens in
// LDS anyway, so it finds the maximum there, and the epilogue multiplies by
// 2^e[t] (exact).
//
// Reduction: 16 lanes per row through cross-lane shuffles, then one lane per
// row rounds to bf16 and stores.
#include "q4lin_device.h"
#include "q4lin_kernels.h"

namespace q4lin {

namespace {

constexpr int kGemvThreads = 256;
constexpr int kRowsPerBlock = 16;
constexpr int kBatch = 10;  // chunks per lane issued together

// float16 dot product with FP32 accumulation: a.lo*b.lo + a.hi*b.hi + c.
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}

template <int T>
__global__ void __launch_bounds__(kGemvThreads)
gemv_kernel(const u32x4_t* __restrict__ x, const uint8_t* __restrict__ codes,
            const uint16_t* __restrict__ scales, uint16_t* __restrict__ y,
            int N, int K) {
  extern __shared__ u32x4_t lds_x[];  // T*K/8 blocks of 8 values (bf16, then fp16 in pair order)
  __shared__ uint32_t lds_max[kGemvThreads / 64][T];
  __shared__ int lds_exp[T];
  const int C = K >> 5;  // 32-weight chunks per row
  const int G = K >> 6;  // groups per row
  const int nb = K >> 3; // 8-value blocks per token

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int j = lane & 15;
  const int row = blockIdx.x * kRowsPerBlock + (tid >> 4);  // wave*4 + quarter
  const bool row_ok = row < N;
  const u32x4_t* wrow = reinterpret_cast<const u32x4_t*>(codes + (size_t)row * (K >> 1));
  const uint16_t* srow = scales + (size_t)row * G;
  const u32x4_t kZeroCodes = {0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};

  // First batch of weight loads goes out before the activation staging.
  u32x4_t w[kBatch];
  uint16_t sc[kBatch];
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    const int p = j + 16 * i;
    const bool ok = row_ok && p < C;
    w[i] = ok ? __builtin_nontemporal_load(wrow + p) : kZeroCodes;
    sc[i] = ok ? srow[p >> 1] : (uint16_t)0;
  }

  // Stage the bf16 activations in LDS and find each token's largest magnitude.
  uint32_t mx[T];
#pragma unroll
  for (int t = 0; t < T; ++t) mx[t] = 0;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    for (int b = tid; b < nb; b += kGemvThreads) {
      const u32x4_t v = x[(size_t)t * nb + b];
      lds_x[t * nb + b] = v;
      uint32_t m = max(max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu), max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu));
      m = max(m, max(max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu), max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu)));
      mx[t] = max(mx[t], m);
    }
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    uint32_t m = mx[t];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    if (lane == 0) lds_max[tid >> 6][t] = m;
  }
  __syncthreads();
  if (tid < T) {
    uint32_t m = max(max(lds_max[0][tid], lds_max[1][tid]), max(lds_max[2][tid], lds_max[3][tid]));
    if (m >= 0x7F80u) m = 0x7F7Fu;  // Inf/NaN inputs are outside the contract
    int lg = 0;
    if (m >= 0x80u)
      lg = (int)(m >> 7) - 127;
    else if (m != 0u)
      lg = (31 - __builtin_clz(m)) - 133;
    lds_exp[tid] = (m == 0u) ? 0 : lg - 14;  // max * 2^-e lands in [2^14, 2^15)
  }
  __syncthreads();
  // Convert in place (each thread rewrites only the blocks it staged).
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int e = lds_exp[t];
    for (int b = tid; b < nb; b += kGemvThreads) {
      const u32x4_t v = lds_x[t * nb + b];
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
      uint32_t h[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        h[2 * q] = __builtin_bit_cast(uint16_t, (_Float16)__builtin_ldexpf(bf16_bits_to_f32(wv[q] & 0xFFFFu), -e));
        h[2 * q + 1] = __builtin_bit_cast(uint16_t, (_Float16)__builtin_ldexpf(bf16_bits_to_f32(wv[q] >> 16), -e));
      }
      lds_x[t * nb + b] = u32x4_t{h[0] | (h[4] << 16), h[1] | (h[5] << 16), h[2] | (h[6] << 16),
                                  h[3] | (h[7] << 16)};
    }
  }
  __syncthreads();

  float acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = 0.0f;

  for (int base = 0; base < C; base += 16 * kBatch) {
    // Prefetch the next batch while this one is consumed.
    u32x4_t wn[kBatch];
    uint16_t scn[kBatch];
    const int nbase = base + 16 * kBatch;
    const bool more = nbase < C;
    if (more) {
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int p = nbase + j + 16 * i;
        const bool ok = row_ok && p < C;
        wn[i] = ok ? __builtin_nontemporal_load(wrow + p) : kZeroCodes;
        scn[i] = ok ? srow[p >> 1] : (uint16_t)0;
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int p = base + j + 16 * i;
      if (p < C) {
        uint32_t pr[16];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t wd = w[i][d];
          pr[4 * d + 0] = f16_pair_q_minus_8(wd, 0);
          pr[4 * d + 1] = f16_pair_q_minus_8(wd, 4);
          pr[4 * d + 2] = f16_pair_q_minus_8(wd, 8);
          pr[4 * d + 3] = f16_pair_q_minus_8(wd, 12);
        }
        const float s = f16_bits_to_f32(sc[i]);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const u32x4_t* xs = lds_x + t * nb + 4 * p;
          float c = 0.0f;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const u32x4_t xv = xs[d];
            c = dot2_f16(pr[4 * d + 0], xv.x, c);
            c = dot2_f16(pr[4 * d + 1], xv.y, c);
            c = dot2_f16(pr[4 * d + 2], xv.z, c);
            c = dot2_f16(pr[4 * d + 3], xv.w, c);
          }
          acc[t] = __builtin_fmaf(s, c, acc[t]);
        }
      }
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        w[i] = wn[i];
        sc[i] = scn[i];
      }
    }
  }

  // Sum the 16 lanes of each row.
#pragma unroll
  for (int t = 0; t < T; ++t) {
    float v = acc[t];
    v += __shfl_xor(v, 8, 16);
    v += __shfl_xor(v, 4, 16);
    v += __shfl_xor(v, 2, 16);
    v += __shfl_xor(v, 1, 16);
    acc[t] = v;
  }
  if (row_ok && j == 0) {
#pragma unroll
    for (int t = 0; t < T; ++t)
      y[(size_t)t * N + row] = f32_to_bf16_rne(__builtin_ldexpf(acc[t], lds_exp[t]));
  }
}

template <int T>
hipError_t launch_t(const GemvArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.n + kRowsPerBlock - 1) / kRowsPerBlock));
  const size_t lds = gemv_lds_bytes(a.k, T);
  auto kern = gemv_kernel<T>;
  const u32x4_t* x = static_cast<const u32x4_t*>(a.x);
  const uint8_t* codes = static_cast<const uint8_t*>(a.codes);
  const uint16_t* scales = static_cast<const uint16_t*>(a.scales);
  uint16_t* y = static_cast<uint16_t*>(a.y);
  int n = (int)a.n, k = (int)a.k;
  void* args[] = {&x, &codes, &scales, &y, &n, &k};
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, dim3(kGemvThreads), args, lds, stream);
}

}  // namespace

size_t gemv_lds_bytes(int64_t k, int64_t t) { return (size_t)(t * k * 2); }

hipError_t launch_gemv(const GemvArgs& a, hipStream_t stream) {
  switch (a.t) {
    case 1: return launch_t<1>(a, stream);
    case 2: return launch_t<2>(a, stream);
    case 3: return launch_t<3>(a, stream);
    case 4: return launch_t<4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace q4lin
