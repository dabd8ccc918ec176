// q4lin_gemv.hip -- the few-token route (T = 1..4): vector-ALU dot products.
//
// The pages' prior art for T = 1 is a row-split GEMV ("q4-linear.md", notes
// under the result table: T = 1 uses a dedicated single-token GEMV); this is an
// MI355X design of the same step, not a translation.
//
// Work mapping.  A workgroup of 4 waves owns 16 consecutive rows (two octets
// of 8 rows); wave w owns the w-th quarter of every row's 32-weight chunks.
// Inside a wave, lane l serves row (octet*8 + l/8) and chunk positions
// l%8, l%8 + 8, ... of the quarter, so every load instruction reads 8 rows x
// 128 contiguous bytes.  All of a batch's loads are issued before any wait.
//
// Why a quarter per wave.  At one token the activations (cold or not) reach
// a wave late: the weight stream floods the memory system, and a barrier
// across the workgroup would tie every wave to the slowest one.  Each wave
// therefore stages only its own quarter of the activations, finds its own
// power-of-two exponent there, and never waits for another wave until the
// final four-way sum.
//
// Arithmetic.
//   * Activations become float16 copies of the bf16 values times 2^-e (e from
//     the quarter's largest magnitude, so every value within 2^34 of it
//     converts exactly); odd-k activations are further divided by 16.
//   * Codes become float16 operands without any add: masking a code dword
//     with 0x000F000F leaves the fp16 pair (q_k * 2^-24, q_k+4 * 2^-24) --
//     subnormal, exact -- and masking with 0x00F000F0 leaves 16 * q * 2^-24 for
//     the odd k, which the /16 above cancels.  Five VALU operations turn 8
//     codes into 4 operand pairs.
//   * v_dot2_f32_f16 sums q * x (FP32).  The code offset enters as
//     sum_k (q_k - 8) x_k = sum q x - sum 8 x: the second sum per chunk comes
//     from the very same dot2 chain run on the operand pairs of an all-8 code
//     dword, so a chunk of eight-codes contributes P - S = 0 exactly, and
//     the difference is taken per chunk (acc += s * (P - S)) while both chunk
//     sums are still small, so it is exact whenever they are.
//   * Each quarter's result carries 2^-(e + 24); the four quarters are combined
//     in binary64 and the sum is rounded to bf16 once.
#include "q4lin_device.h"
#include "q4lin_kernels.h"

namespace q4lin {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 16;      // rows per workgroup (two octets)
constexpr int kBatch = 5;      // chunk positions per lane per octet per batch

__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}

// largest |x| over 8 bf16 values, as bf16 magnitude bits (monotone in the value)
__device__ __forceinline__ uint32_t max_mag8(u32x4_t v) {
  uint32_t m = max(max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu), max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu));
  return max(m, max(max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu), max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu)));
}

// e such that (largest magnitude) * 2^-e lies in [2^14, 2^15); 0 for all-zero input.
__device__ __forceinline__ int exponent_for(uint32_t m) {
  if (m >= 0x7F80u) m = 0x7F7Fu;  // Inf/NaN inputs are outside the contract
  if (m == 0u) return 0;
  const int lg = (m >= 0x80u) ? (int)(m >> 7) - 127 : (31 - __builtin_clz(m)) - 133;
  return lg - 14;
}

// 8 bf16 values -> 8 float16 values in pair order (k0,k4)(k1,k5)(k2,k6)(k3,k7),
// scaled by 2^-e, odd k scaled by 2^-(e+4).
__device__ __forceinline__ u32x4_t to_f16_pairs(u32x4_t v, int e) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t h[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    h[2 * q] = __builtin_bit_cast(uint16_t, (_Float16)__builtin_ldexpf(bf16_bits_to_f32(w[q] & 0xFFFFu), -e));
    h[2 * q + 1] = __builtin_bit_cast(uint16_t, (_Float16)__builtin_ldexpf(bf16_bits_to_f32(w[q] >> 16), -e - 4));
  }
  return u32x4_t{h[0] | (h[4] << 16), h[1] | (h[5] << 16), h[2] | (h[6] << 16), h[3] | (h[7] << 16)};
}

// dot2 chain of one 32-weight chunk against its activation pairs (4 planes)
__device__ __forceinline__ float chunk_dot(u32x4_t w, const u32x4_t* xs, int plane) {
  float c = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t wd = w[d];
    const uint32_t w8 = wd >> 8;
    const u32x4_t xq = xs[d * plane];
    c = dot2_f16(wd & 0x000F000Fu, xq.x, c);
    c = dot2_f16(wd & 0x00F000F0u, xq.y, c);
    c = dot2_f16(w8 & 0x000F000Fu, xq.z, c);
    c = dot2_f16(w8 & 0x00F000F0u, xq.w, c);
  }
  return c;
}

// ONE: every wave's quarter fits one batch (at most 8 * kBatch chunks); the
// batch loop and its prefetch registers then vanish at compile time.
template <int T, bool ONE>
__global__ void __launch_bounds__(kThreads)
gemv_kernel(const u32x4_t* __restrict__ x, const uint8_t* __restrict__ codes,
            const uint16_t* __restrict__ scales, uint16_t* y,
            int N, int K, int cq, const uint16_t* res, int f32) {
  // Dynamic LDS per wave: activations [T][4 planes][cq] (16 B each), then the
  // all-8 sums [T][cq] (4 B each).  cq = ceil(C / 4) chunk slots per wave.
  extern __shared__ u32x4_t lds[];
  __shared__ float lds_part[kWaves][kRows][T];
  __shared__ int lds_e[kWaves][T];
  const int C = K >> 5;
  const int G = K >> 6;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r8 = lane >> 3, c8 = lane & 7;
  const int row0 = blockIdx.x * kRows;
  const int cw0 = (wave * C) >> 2;
  const int cw = (((wave + 1) * C) >> 2) - cw0;   // chunks of this wave's quarter
  u32x4_t* xq = lds + (size_t)wave * (T * 4 * cq + T * cq / 4 + 1);
  float* s8 = reinterpret_cast<float*>(xq + T * 4 * cq);

  // 1. activations of the quarter (4 blocks of 8 values per chunk), all tokens
  // Every load below reads a clamped, always-valid address and is masked only
  // after all loads are in flight: a select right behind a load would make the
  // compiler wait for that load before issuing the next one.
  const int nb = 4 * cw;
  const int blast = max(nb - 1, 0);
  u32x4_t xv[T][3];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int q = 0; q < 3; ++q)
      xv[t][q] = x[(size_t)t * (K >> 3) + 4 * cw0 + min(lane + 64 * q, blast)];
  // larger quarters stage the rest of the activations in extra passes below
  __builtin_amdgcn_sched_barrier(0);

  // 2. first batch of codes (and their scales)
  const u32x4_t kEights = {0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
  u32x4_t w[2][kBatch];
  uint16_t sc[2][kBatch];
  // Codes and scales of chunk positions i0..i0+kBatch-1 (per octet).  Rows past
  // N and positions past the quarter read a valid clamped address; their scale
  // is zeroed afterwards (mask_batch), so they add exactly 0.
  const int plast = max(cw - 1, 0);
  auto load_batch = [&](int i0, u32x4_t (&wd)[2][kBatch], uint16_t (&sd)[2][kBatch]) {
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      const int row = min(row0 + 8 * o + r8, N - 1);
      const u32x4_t* wp = reinterpret_cast<const u32x4_t*>(codes + (size_t)row * (K >> 1));
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int p = min(c8 + 8 * (i0 + i), plast);
        wd[o][i] = __builtin_nontemporal_load(wp + cw0 + p);
        sd[o][i] = scales[(size_t)row * G + ((cw0 + p) >> 1)];
      }
    }
  };
  auto mask_batch = [&](int i0, uint16_t (&sd)[2][kBatch]) {
#pragma unroll
    for (int o = 0; o < 2; ++o)
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        if (row0 + 8 * o + r8 >= N || c8 + 8 * (i0 + i) >= cw) sd[o][i] = 0;
  };
  load_batch(0, w, sc);
  __builtin_amdgcn_sched_barrier(0);
  mask_batch(0, sc);
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int q = 0; q < 3; ++q)
      if (lane + 64 * q >= nb) xv[t][q] = u32x4_t{0u, 0u, 0u, 0u};

  // 3. per-token exponent of the quarter; float16 activations into LDS
  int e[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    uint32_t m = 0;
#pragma unroll
    for (int q = 0; q < 3; ++q) m = max(m, max_mag8(xv[t][q]));
    if (!ONE)
      for (int b = lane + 192; b < nb; b += 64) m = max(m, max_mag8(x[(size_t)t * (K >> 3) + 4 * cw0 + b]));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    e[t] = exponent_for(m);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int b = lane + 64 * q;
      if (b < nb) xq[(t * 4 + (b & 3)) * cq + (b >> 2)] = to_f16_pairs(xv[t][q], e[t]);
    }
    if (!ONE)
      for (int b = lane + 192; b < nb; b += 64)
        xq[(t * 4 + (b & 3)) * cq + (b >> 2)] = to_f16_pairs(x[(size_t)t * (K >> 3) + 4 * cw0 + b], e[t]);
  }
  // An empty quarter (K = 64 has two chunks for four waves) still runs step 5
  // at the clamped position 0 with zero scales; give that position finite
  // zeros, since 0 times a stale NaN left in LDS would still be NaN.
  if (cw == 0) {
    if (lane < 4 * T) xq[lane * cq] = u32x4_t{0u, 0u, 0u, 0u};
    if (lane < T) s8[lane * cq] = 0.0f;
  }
  // 4. all-8 chunk sums, same dot2 chain as the rows use
  const u32x4_t k8 = kEights;
#pragma unroll
  for (int t = 0; t < T; ++t)
    for (int p = lane; p < cw; p += 64) s8[t * cq + p] = chunk_dot(k8, xq + t * 4 * cq + p, cq);

  // 5. chunks, batch by batch with the next batch in flight
  float acc[2][T];
#pragma unroll
  for (int o = 0; o < 2; ++o)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[o][t] = 0.0f;
  const int nbatch = ONE ? 1 : (cw + 8 * kBatch - 1) / (8 * kBatch);
  for (int bi = 0; bi < nbatch; ++bi) {
    u32x4_t wn[2][kBatch];
    uint16_t scn[2][kBatch];
    const bool more = !ONE && bi + 1 < nbatch;
    if (more) {
      load_batch((bi + 1) * kBatch, wn, scn);
      __builtin_amdgcn_sched_barrier(0);
      mask_batch((bi + 1) * kBatch, scn);
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
#pragma unroll
      for (int o = 0; o < 2; ++o) {
        const int p = min(c8 + 8 * (bi * kBatch + i), plast);
        {
          const float s = f16_bits_to_f32(sc[o][i]);
#pragma unroll
          for (int t = 0; t < T; ++t) {
            const float c = chunk_dot(w[o][i], xq + t * 4 * cq + p, cq);
            acc[o][t] = __builtin_fmaf(s, c - s8[t * cq + p], acc[o][t]);
          }
        }
      }
    }
    if (more) {
#pragma unroll
      for (int o = 0; o < 2; ++o)
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          w[o][i] = wn[o][i];
          sc[o][i] = scn[o][i];
        }
    }
  }

  // 6. sum the 8 lanes of each row, then the four quarters
#pragma unroll
  for (int o = 0; o < 2; ++o)
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float v = acc[o][t];
      v += __shfl_xor(v, 4, 8);
      v += __shfl_xor(v, 2, 8);
      v += __shfl_xor(v, 1, 8);
      if (c8 == 0) lds_part[wave][8 * o + r8][t] = v;
    }
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < T; ++t) lds_e[wave][t] = e[t];
  }
  __syncthreads();
  // Partials carry factors 2^-(e_w + 24) with a different e_w per quarter; the
  // four-term combine runs in binary64, whose range holds every scaled partial
  // (no overflow to mixed-sign infinities, no flush of small quarters).
  if (tid < kRows * T) {
    const int r = tid % kRows, t = tid / kRows;
    const int row = row0 + r;
    if (row < N) {
      double v = 0.0;
#pragma unroll
      for (int q = 0; q < kWaves; ++q) v += __builtin_ldexp((double)lds_part[q][r][t], lds_e[q][t] + 24);
      if (res != nullptr) v += (double)bf16_bits_to_f32(res[(size_t)t * N + row]);  // LinearAdd
      if (f32) reinterpret_cast<float*>(y)[(size_t)t * N + row] = (float)v;  // LinearSwiGLU sums
      else y[(size_t)t * N + row] = f32_to_bf16_rne((float)v);
    }
  }
}

template <int T>
hipError_t launch_t(const GemvArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.n + kRows - 1) / kRows));
  const int cq = (int)gemv_chunks_per_wave(a.k);
  const size_t lds = gemv_lds_bytes(a.k, T);
  const bool one = ((a.k / 32 + 3) / 4) <= 8 * kBatch;
  auto kern = one ? gemv_kernel<T, true> : gemv_kernel<T, false>;
  const u32x4_t* x = static_cast<const u32x4_t*>(a.x);
  const uint8_t* codes = static_cast<const uint8_t*>(a.codes);
  const uint16_t* scales = static_cast<const uint16_t*>(a.scales);
  uint16_t* y = static_cast<uint16_t*>(a.y);
  int n = (int)a.n, k = (int)a.k;
  const uint16_t* res = static_cast<const uint16_t*>(a.res);
  int f32 = a.f32 ? 1 : 0;
  void* args[] = {&x, &codes, &scales, &y, &n, &k, (void*)&cq, &res, &f32};
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, dim3(kThreads), args, lds, stream);
}

}  // namespace

int64_t gemv_chunks_per_wave(int64_t k) {
  const int64_t c = k / 32;
  int64_t q = (c + 3) / 4;
  return (q + 3) / 4 * 4;  // keep every wave's LDS region 64-byte aligned
}

size_t gemv_lds_bytes(int64_t k, int64_t t) {
  const int64_t cq = gemv_chunks_per_wave(k);
  return (size_t)kWaves * (size_t)(t * 4 * cq + t * cq / 4 + 1) * 16;
}

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
