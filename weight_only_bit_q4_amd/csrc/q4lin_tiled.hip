// q4lin_tiled.hip -- the many-token route: LDS-tiled matrix-core GEMM.
//
// The pages' prior art for large T is a tiled BF16-input, FP32-accumulate
// MMA with 32x32 to 64x128 output tiles ("q4-linear.md", notes under the
// result table).  This is an MI355X design of the same step.
//
// Operands.  The 64-group scale must be applied to exact group sums
// (rounding (q-8)*scale to a 16-bit float loses bits the tolerance needs), so
// every group's partial product P = sum_k (q-8) x is formed by the matrix
// cores from exact operands and then scaled in FP32: acc += scale * P.
//   * Weights: a nibble becomes the float16 value q - 8 with two packed
//     16-bit operations per pair (f16_pair_q_minus_8); float16 holds every
//     integer in [-8, 7] exactly.
//   * Activations: bf16 values are not all float16 values, so a short
//     preparation pass multiplies every token by a power of two 2^-e[t]
//     chosen from the token's largest magnitude; then every bf16 value within
//     2^38 of that maximum converts to float16 exactly.  The pass writes the
//     float16 activations in the order the matrix-core operand loads want and
//     stores e[t]; the epilogue multiplies by 2^e[t] (exact).
//   * v_mfma_f32_32x32x16_f16 with A = activations (32 tokens x 16 k) and
//     B = weights (16 k x 32 rows): every lane's 16 accumulators then share
//     one weight row, so one scale per lane per group suffices.
//
// Tiling.  A workgroup owns BN = 32*NS rows and BT = 32*TS*WT tokens; its WT
// waves split the tokens and share the rows.  Per 64-group the workgroup
// dequantizes its BN x 64 weight tile once into LDS (double-buffered, one
// barrier per group) and every wave reads the B operands from there; each
// wave streams its own activation operands straight from global memory.
#include "q4lin_device.h"
#include "q4lin_kernels.h"

namespace q4lin {

namespace {

constexpr int kPrepThreads = 256;
constexpr int kRowBytes = 144;  // one dequantized row-group in LDS: 128 B + 16 B pad

// Activation tile order: for token block tb (32 tokens) and group g a block of
// 2048 halves laid out [m 0..3][h 0..1][i 0..31][slot 0..7]; slot order is the
// pair order of k = 64g + 32h + 8m + 0..7 and i the token within the block.
// Returns the index in 16-byte units.
__device__ __forceinline__ size_t x16_index(int tb, int g, int G, int m, int h, int i) {
  return ((size_t)tb * G + g) * 256 + (size_t)((m * 2 + h) * 32 + i);
}

__global__ void __launch_bounds__(kPrepThreads)
prep_x_kernel(const u32x4_t* __restrict__ x, int K, int T, u32x4_t* __restrict__ x16,
              int* __restrict__ texp) {
  __shared__ uint32_t red[kPrepThreads / 64];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int G = K >> 6;
  const int nblk = K >> 3;
  const int tb = t >> 5, i = t & 31;
  if (t >= T) {  // padding token
    for (int b = tid; b < nblk; b += kPrepThreads) {
      const int g = b >> 3, kb = b & 7;
      x16[x16_index(tb, g, G, kb & 3, kb >> 2, i)] = u32x4_t{0u, 0u, 0u, 0u};
    }
    if (tid == 0) texp[t] = 0;
    return;
  }
  const u32x4_t* xt = x + (size_t)t * nblk;
  uint32_t m = 0;
  for (int b = tid; b < nblk; b += kPrepThreads) {
    const u32x4_t v = xt[b];
    m = max(m, max(max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu), max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu)));
    m = max(m, max(max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu), max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu)));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = max(max(red[0], red[1]), max(red[2], red[3]));
  if (m >= 0x7F80u) m = 0x7F7Fu;  // Inf/NaN inputs are outside the contract
  // floor(log2(max)) from the bf16 bits, then e so that max * 2^-e is in [2^14, 2^15).
  int lg = 0;
  if (m >= 0x80u)
    lg = (int)(m >> 7) - 127;
  else if (m != 0u)
    lg = (31 - __builtin_clz(m)) - 133;
  const int e = (m == 0u) ? 0 : lg - 14;
  if (tid == 0) texp[t] = e;
  for (int b = tid; b < nblk; b += kPrepThreads) {
    const u32x4_t v = xt[b];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t h16[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float lo = __builtin_ldexpf(bf16_bits_to_f32(w[q] & 0xFFFFu), -e);
      const float hi = __builtin_ldexpf(bf16_bits_to_f32(w[q] >> 16), -e);
      h16[2 * q] = __builtin_bit_cast(uint16_t, (_Float16)lo);
      h16[2 * q + 1] = __builtin_bit_cast(uint16_t, (_Float16)hi);
    }
    // pair order x0,x4 | x1,x5 | x2,x6 | x3,x7
    u32x4_t o;
    o.x = h16[0] | (h16[4] << 16);
    o.y = h16[1] | (h16[5] << 16);
    o.z = h16[2] | (h16[6] << 16);
    o.w = h16[3] | (h16[7] << 16);
    const int g = b >> 3, kb = b & 7;
    x16[x16_index(tb, g, G, kb & 3, kb >> 2, i)] = o;
  }
}

template <int NS, int TS, int WT>
__global__ void __launch_bounds__(64 * WT)
tiled_kernel(const u32x4_t* __restrict__ x16, const int* __restrict__ texp,
             const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
             uint16_t* __restrict__ y, int N, int K, int T, int Tpad) {
  constexpr int BN = NS * 32;
  constexpr int NTH = 64 * WT;
  constexpr int TASKS = 2 * BN;                     // (row, half-group) pieces of 16 code bytes
  constexpr int TPT = (TASKS + NTH - 1) / NTH;
  __shared__ __attribute__((aligned(16))) uint8_t lds_w[2][BN * kRowBytes];
  __shared__ float lds_s[2][BN];

  const int G = K >> 6;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, lh = lane >> 5;
  const int n0 = blockIdx.x * BN;
  const int t0w = (blockIdx.y * WT + wave) * TS * 32;  // first token of this wave

  u32x4_t cw[TPT];
  uint16_t csc[TPT];
  auto load_codes = [&](int g) {
#pragma unroll
    for (int q = 0; q < TPT; ++q) {
      const int task = tid + q * NTH;
      const int r = task >> 1, hh = task & 1;
      const int row = n0 + r;
      const bool ok = task < TASKS && row < N;
      cw[q] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
                       codes + (size_t)row * (K >> 1) + (size_t)g * 32 + hh * 16))
                 : u32x4_t{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
      csc[q] = (ok && hh == 0) ? scales[(size_t)row * G + g] : (uint16_t)0;
    }
  };
  auto store_dq = [&](int buf) {
#pragma unroll
    for (int q = 0; q < TPT; ++q) {
      const int task = tid + q * NTH;
      if (task < TASKS) {
        const int r = task >> 1, hh = task & 1;
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(&lds_w[buf][r * kRowBytes + hh * 64]);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t wd = cw[q][d];
          dst[d] = u32x4_t{f16_pair_q_minus_8(wd, 0), f16_pair_q_minus_8(wd, 4),
                           f16_pair_q_minus_8(wd, 8), f16_pair_q_minus_8(wd, 12)};
        }
        if (hh == 0) lds_s[buf][r] = f16_bits_to_f32(csc[q]);
      }
    }
  };

  f16x8_t a[TS][4];
  auto load_x = [&](int g, f16x8_t (&dst)[TS][4]) {
#pragma unroll
    for (int ts = 0; ts < TS; ++ts) {
      const int tb = (t0w >> 5) + ts;
      const bool ok = tb * 32 < Tpad;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const u32x4_t v = ok ? x16[x16_index(tb, g, G, m, lh, li)] : u32x4_t{0u, 0u, 0u, 0u};
        dst[ts][m] = __builtin_bit_cast(f16x8_t, v);
      }
    }
  };

  f32x16_t acc[TS][NS];
#pragma unroll
  for (int ts = 0; ts < TS; ++ts)
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[ts][ns][r] = 0.0f;

  load_codes(0);
  load_x(0, a);
  store_dq(0);
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    const bool more = g + 1 < G;
    f16x8_t an[TS][4];
    if (more) {
      load_codes(g + 1);
      load_x(g + 1, an);
    }
    f16x8_t b[NS][4];
    float s[NS];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      const uint8_t* rowp = &lds_w[buf][(ns * 32 + li) * kRowBytes + lh * 64];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        b[ns][m] = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const u32x4_t*>(rowp + m * 16));
      s[ns] = lds_s[buf][ns * 32 + li];
    }
#pragma unroll
    for (int ts = 0; ts < TS; ++ts) {
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        f32x16_t p = {};
#pragma unroll
        for (int m = 0; m < 4; ++m)
          p = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[ts][m], b[ns][m], p, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[ts][ns][r] = __builtin_fmaf(s[ns], p[r], acc[ts][ns][r]);
      }
    }
    if (more) {
      store_dq(buf ^ 1);
#pragma unroll
      for (int ts = 0; ts < TS; ++ts)
#pragma unroll
        for (int m = 0; m < 4; ++m) a[ts][m] = an[ts][m];
    }
    __syncthreads();
  }

  // Epilogue: lane (li, lh) holds row n = n0 + 32 ns + li and tokens
  // t = t0w + 32 ts + 8 (r / 4) + 4 lh + r % 4.
#pragma unroll
  for (int ts = 0; ts < TS; ++ts) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = t0w + ts * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
      if (t < T) {
        const int e = texp[t];
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          const int n = n0 + ns * 32 + li;
          if (n < N) y[(size_t)t * N + n] = f32_to_bf16_rne(__builtin_ldexpf(acc[ts][ns][r], e));
        }
      }
    }
  }
}

template <int NS, int TS, int WT>
hipError_t launch_cfg(const TiledArgs& a, const u32x4_t* x16, const int* texp, int tpad,
                      hipStream_t stream) {
  constexpr int BN = NS * 32;
  constexpr int BT = TS * WT * 32;
  const dim3 grid((unsigned)((a.n + BN - 1) / BN), (unsigned)((a.t + BT - 1) / BT));
  auto kern = tiled_kernel<NS, TS, WT>;
  const uint8_t* codes = static_cast<const uint8_t*>(a.codes);
  const uint16_t* scales = static_cast<const uint16_t*>(a.scales);
  uint16_t* y = static_cast<uint16_t*>(a.y);
  int n = (int)a.n, k = (int)a.k, t = (int)a.t;
  void* args[] = {&x16, &texp, &codes, &scales, &y, &n, &k, &t, &tpad};
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, dim3(64 * WT), args, 0, stream);
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

int64_t tiled_tpad(int64_t t) { return (t + 31) / 32 * 32; }

size_t tiled_workspace_bytes(int64_t k, int64_t t) {
  const int64_t tp = tiled_tpad(t);
  return align256((size_t)(tp * k * 2)) + align256((size_t)(tp * 4));
}

TiledConfig tiled_pick_config(int64_t n, int64_t k, int64_t t) {
  (void)n;
  (void)k;
  if (t > 128) return TiledConfig{3, 2, 4};
  if (t > 32) return TiledConfig{1, 1, 2};
  return TiledConfig{1, 1, 1};
}

hipError_t launch_tiled(const TiledArgs& a, hipStream_t stream) {
  const int64_t tp = tiled_tpad(a.t);
  u32x4_t* x16 = static_cast<u32x4_t*>(a.workspace);
  int* texp = reinterpret_cast<int*>(static_cast<uint8_t*>(a.workspace) + align256((size_t)(tp * a.k * 2)));
  {
    const u32x4_t* x = static_cast<const u32x4_t*>(a.x);
    int k = (int)a.k, t = (int)a.t;
    void* args[] = {&x, &k, &t, &x16, &texp};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(prep_x_kernel), dim3((unsigned)tp),
                                   dim3(kPrepThreads), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  const int tpad = (int)tp;
  const TiledConfig c = a.cfg;
  if (c.ns == 3 && c.ts == 2 && c.wt == 4) return launch_cfg<3, 2, 4>(a, x16, texp, tpad, stream);
  if (c.ns == 1 && c.ts == 1 && c.wt == 2) return launch_cfg<1, 1, 2>(a, x16, texp, tpad, stream);
  if (c.ns == 1 && c.ts == 1 && c.wt == 1) return launch_cfg<1, 1, 1>(a, x16, texp, tpad, stream);
  return hipErrorInvalidValue;
}

}  // namespace q4lin
