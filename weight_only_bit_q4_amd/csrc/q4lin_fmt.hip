// q4lin_fmt.hip -- the other weight formats of the pure Linear on the few-token
// route: Q5G64_F16S, Q6G64_F16S, W8G32_F16S, NVFP4 (A16) and BF16_CTRL.
//
// The pages list these formats beside Q4G64_F16S for the same A16 Linear and
// give their storage ("linear-benchmark.md", section 0 and the weight-format
// table of section 4: 42 and 50 bytes per 64 weights for Q5/Q6, 34 bytes per
// 32 for W8, 9 bytes per 16 for NVFP4, 2 N K bytes for BF16_CTRL).  Packing
// (the plainest one matching those byte counts):
//   Q5  low plane [N][K/2] (even k in the low nibble), high plane [N][K/8]
//       (bit i of byte b: k = 8b + i), fp16 scales [N][K/64];
//       weight (q - 16) s with q = low | high << 4;
//   Q6  low plane as Q5, high plane [N][K/4] (bits 2i..2i+1 of byte b:
//       k = 4b + i), fp16 scales [N][K/64]; weight (q - 32) s;
//   W8  one two's-complement byte per weight [N][K], fp16 scales [N][K/32];
//       weight c s;
//   NVFP4  E2M1 nibbles [N][K/2] (even k low), E4M3 scale bytes [N][K/16];
//       weight E2M1(code) E4M3(scale);
//   BF16_CTRL  the bf16 weights [N][K].
//
// Work mapping.  One workgroup of eight waves per block of BN <= 16 CT rows;
// the waves split K into eight contiguous runs of "units" (one scale group
// of Q5/Q6/W8, 64 weights of NVFP4, 32 of BF16), so every weight byte is
// read once for all T <= 32 tokens.  Lane l serves row 16 ct + l % 16 and
// the (l / 16)-th quarter of each unit: its loads are 8 (16 for BF16)
// contiguous code bytes per row and unit, plus the matching high bits, and
// 16 or 32 contiguous bytes of activations per token.  Longer T runs the
// kernel once per 32 tokens.
//
// Arithmetic (v_mfma_f32_16x16x32_bf16, A = activations, B = weights, every
// instruction reduces over one unit):
//   * Q5/Q6: two three-input bitwise operations per pair of weights build
//     the exact bf16 value 128 + q (q < 128 has unit spacing there), in the
//     pair order (k0,k4) (k1,k5) (k2,k6) (k3,k7) of a code dword; the
//     activations are permuted into the same order.  The products of a
//     constant all-(offset) operand run through the same instruction
//     sequence, so P - C = sum (q - offset) x, exactly 0 for a unit of
//     offset codes; the unit's scale is applied in FP32.
//   * W8: the byte u = c + 128 is split into nibbles: 128 + lo and
//     256 + 16 hi are exact bf16 values, and their two products with the
//     same activations sum to (384 + u) x; the constant operand of c = 0
//     gives the matching correction.
//   * NVFP4: E2M1 times E4M3 has at most 6 significant bits and lies in
//     [2^-10, 2688], so each weight is formed exactly as bf16 (hardware FP4
//     conversion with a unit scale, an FP32 product with the decoded E4M3
//     scale, a conversion that is exact) and fed straight to the matrix
//     cores.
//   * BF16_CTRL: the weights as they are.
//   * The eight wave partials are summed in binary64 and rounded to bf16
//     once; an output that comes out non-finite (binary32 partials that left
//     the range) is formed again exactly by its thread.
#include "q4lin_device.h"
#include "q4lin_kernels.h"

namespace q4lin {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kUnroll = 2;  // units per pipeline step (the next step's loads fly during this one's products)

// weights per unit (a lane holds a quarter of a row's unit: 8 code bytes,
// 16 for BF16_CTRL)
template <int F>
struct Unit {
  static constexpr int K = (F == FMT_W8 || F == FMT_BF16) ? 32 : 64;
};

// (a & m) | c and (a & m) ^ c in one instruction each (gfx950 three-input
// bitwise operation; truth tables 0xEA and 0x6A for inputs a, m, c)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, m, c, 0xEA);
}
__device__ __forceinline__ uint32_t and_xor(uint32_t a, uint32_t m, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, m, c, 0x6A);
}

// 8 consecutive bf16 activations (x0..x7 as 4 dwords) -> order x0 x4 x1 x5 x2 x6 x3 x7
__device__ __forceinline__ bf16x8_t pair_order(u32x4_t v) {
  u32x4_t r;
  r.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
  r.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
  r.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
  r.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
  return __builtin_bit_cast(bf16x8_t, r);
}

// Q5: code dword w (nibbles of k0..k7) and high byte h (bit s: k_s) -> the
// eight exact bf16 values 128 + q in pair order
__device__ __forceinline__ bf16x8_t q5_operand(uint32_t w, uint32_t h) {
  const uint32_t hs = ((h & 0x0Fu) | ((h & 0xF0u) << 12)) << 4;  // h_s at bit 4 + s, h_{s+4} at bit 20 + s
  u32x4_t r;
  r.x = and_or(hs, 0x00100010u, and_or(w, 0x000F000Fu, 0x43004300u));
  r.y = and_or(hs >> 1, 0x00100010u, and_or(w >> 4, 0x000F000Fu, 0x43004300u));
  r.z = and_or(hs >> 2, 0x00100010u, and_or(w >> 8, 0x000F000Fu, 0x43004300u));
  r.w = and_or(hs >> 3, 0x00100010u, and_or(w >> 12, 0x000F000Fu, 0x43004300u));
  return __builtin_bit_cast(bf16x8_t, r);
}

// Q6: code dword w and high half-word h (bits 2s..2s+1: k_s) -> 128 + q in pair order
__device__ __forceinline__ bf16x8_t q6_operand(uint32_t w, uint32_t h) {
  const uint32_t hs = ((h & 0xFFu) | ((h & 0xFF00u) << 8)) << 4;  // pair s at bits 4 + 2s, pair s+4 at 20 + 2s
  u32x4_t r;
  r.x = and_or(hs, 0x00300030u, and_or(w, 0x000F000Fu, 0x43004300u));
  r.y = and_or(hs >> 2, 0x00300030u, and_or(w >> 4, 0x000F000Fu, 0x43004300u));
  r.z = and_or(hs >> 4, 0x00300030u, and_or(w >> 8, 0x000F000Fu, 0x43004300u));
  r.w = and_or(hs >> 6, 0x00300030u, and_or(w >> 12, 0x000F000Fu, 0x43004300u));
  return __builtin_bit_cast(bf16x8_t, r);
}

// W8: 8 code bytes (two dwords, k0..k7) -> the low operand (128 + lo) and
// the high operand (256 + 16 hi_u), hi_u = high nibble of u = c + 128, both
// in natural order (k0,k1) (k2,k3) ...
__device__ __forceinline__ void w8_operands(uint32_t w0, uint32_t w1, bf16x8_t& lo, bf16x8_t& hi) {
  const uint32_t t[4] = {__builtin_amdgcn_perm(w0, w0, 0x0C010C00u), __builtin_amdgcn_perm(w0, w0, 0x0C030C02u),
                         __builtin_amdgcn_perm(w1, w1, 0x0C010C00u), __builtin_amdgcn_perm(w1, w1, 0x0C030C02u)};
  u32x4_t l, h;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    l[i] = and_or(t[i], 0x000F000Fu, 0x43004300u);
    // 0x4380 | hi_u << 3 with hi_u = (byte >> 4) ^ 8: the byte's top nibble
    // at bits 3..6, its top bit flipped by the exclusive or
    h[i] = and_xor(t[i] >> 1, 0x00780078u, 0x43C043C0u);
  }
  lo = __builtin_bit_cast(bf16x8_t, l);
  hi = __builtin_bit_cast(bf16x8_t, h);
}

// E4M3 (bias 7, subnormals) -> binary32, by its fields
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 0xFu, m = b & 7u;
  const float mag = e != 0u ? __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return (b & 0x80u) ? -mag : mag;
}

// NVFP4: code dword w (E2M1 nibbles of k0..k7, even k low) times scale s ->
// the eight exact bf16 weights in natural order
__device__ __forceinline__ uint32_t nvfp4_pair(f32x2_t v, float s) {
  return (uint32_t)f32_to_bf16_rne(v.x * s) | ((uint32_t)f32_to_bf16_rne(v.y * s) << 16);
}
__device__ __forceinline__ bf16x8_t nvfp4_operand(uint32_t w, float s) {
  u32x4_t r;
  r.x = nvfp4_pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0), s);
  r.y = nvfp4_pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1), s);
  r.z = nvfp4_pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2), s);
  r.w = nvfp4_pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3), s);
  return __builtin_bit_cast(bf16x8_t, r);
}

// Weight W[n][k] of format F in binary64, exact (the plain definition, for
// the repair below).
template <int F>
__device__ double weight_exact(const uint8_t* __restrict__ lo, const uint8_t* __restrict__ hi,
                               const uint8_t* __restrict__ sc, int K, int n, int k) {
  const size_t r = (size_t)n;
  if constexpr (F == FMT_BF16) {
    return (double)bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(lo)[r * K + k]);
  } else if constexpr (F == FMT_W8) {
    const int c = (int)(int8_t)lo[r * K + k];
    return (double)c * (double)f16_bits_to_f32(reinterpret_cast<const uint16_t*>(sc)[r * (K / 32) + k / 32]);
  } else {
    const uint32_t b = lo[r * (K / 2) + k / 2];
    const int nib = (int)((k & 1) ? (b >> 4) : (b & 15u));
    if constexpr (F == FMT_NVFP4) {
      const int e = (nib >> 1) & 3, m = nib & 1;
      double v = e == 0 ? 0.5 * m : __builtin_ldexp(1.0 + 0.5 * m, e - 1);
      if (nib & 8) v = -v;
      return v * (double)e4m3_to_f32(sc[r * (K / 16) + k / 16]);
    } else {
      const double s = (double)f16_bits_to_f32(reinterpret_cast<const uint16_t*>(sc)[r * (K / 64) + k / 64]);
      if constexpr (F == FMT_Q5) {
        const int q = nib | ((int)((hi[r * (K / 8) + k / 8] >> (k & 7)) & 1u) << 4);
        return (double)(q - 16) * s;
      } else {
        const int q = nib | ((int)((hi[r * (K / 4) + k / 4] >> (2 * (k & 3))) & 3u) << 4);
        return (double)(q - 32) * s;
      }
    }
  }
}

// An output whose binary32 partial sums left the range (activations near
// the top of the bf16 range make the products of the offset codes overflow
// although the exact sum may not) is formed again from the inputs: the sum
// over k in binary64 of exact products, rounded once.  Finite outputs never
// come here.
template <int F>
__device__ __attribute__((noinline)) uint16_t exact_output(const uint16_t* __restrict__ x,
                                                           const uint8_t* __restrict__ lo,
                                                           const uint8_t* __restrict__ hi,
                                                           const uint8_t* __restrict__ sc, int K, int n, int t) {
  double acc = 0.0;
  for (int k = 0; k < K; ++k)
    acc += weight_exact<F>(lo, hi, sc, K, n, k) * (double)bf16_bits_to_f32(x[(size_t)t * K + k]);
  return f32_to_bf16_rne((float)acc);
}

// One lane's loads for one unit: code bytes (and high bits, scale) of CT
// rows, activations of TT tokens.
template <int F, int CT, int TT>
struct Loads {
  u32x4_t c[CT];      // code bytes (.x .y for 8-byte formats)
  uint32_t h[CT];     // high bits (Q5: 16, Q6: 32) or the E4M3 scale byte (NVFP4)
  uint16_t s[CT];     // fp16 scale (Q5, Q6, W8)
  u32x4_t a[TT][2];   // activations: [tt][16-byte half]
};

template <int F, int CT, int TT>
__global__ void __launch_bounds__(kThreads, 1)
fmt_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ lo, const uint8_t* __restrict__ hi,
           const uint8_t* __restrict__ sc, uint16_t* __restrict__ y, int N, int K, int T, int BN) {
  using U = Unit<F>;
  constexpr bool NIB = (F == FMT_Q5 || F == FMT_Q6);     // nibble codes with an offset
  constexpr bool SCALED = (F == FMT_Q5 || F == FMT_Q6 || F == FMT_W8);
  constexpr int XH = U::K == 64 ? 2 : 1;                 // 16-byte activation pieces per unit and token
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const int n0 = blockIdx.x * BN;
  const int rows = min(BN, N - n0);
  const int units = K / U::K;
  const int ub = (int)(((int64_t)units * wave) / kWaves), ue = (int)(((int64_t)units * (wave + 1)) / kWaves);

  // per column tile: this lane's row (rows past the block repeat the last
  // one; their sums are never stored)
  const uint8_t* lo_row[CT];
  const uint8_t* hi_row[CT];
  const uint8_t* sc_row[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const size_t r = (size_t)(n0 + min(16 * ct + li, rows - 1));
    if constexpr (F == FMT_BF16) lo_row[ct] = lo + r * (size_t)K * 2 + (size_t)lq * 16;
    else if constexpr (F == FMT_W8) lo_row[ct] = lo + r * (size_t)K + (size_t)lq * 8;
    else lo_row[ct] = lo + r * (size_t)(K / 2) + (size_t)lq * 8;
    if constexpr (F == FMT_Q5) hi_row[ct] = hi + r * (size_t)(K / 8) + (size_t)lq * 2;
    else if constexpr (F == FMT_Q6) hi_row[ct] = hi + r * (size_t)(K / 4) + (size_t)lq * 4;
    else hi_row[ct] = nullptr;
    if constexpr (F == FMT_NVFP4) sc_row[ct] = sc + r * (size_t)(K / 16) + (size_t)lq;
    else if constexpr (F == FMT_W8) sc_row[ct] = sc + r * (size_t)(K / 32) * 2;
    else if constexpr (SCALED) sc_row[ct] = sc + r * (size_t)(K / 64) * 2;
    else sc_row[ct] = nullptr;
  }
  const uint16_t* x_row[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) x_row[tt] = x + (size_t)min(16 * tt + li, T - 1) * (size_t)K + lq * (8 * XH);

  auto load = [&](int u, Loads<F, CT, TT>& L) __device__ {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      if constexpr (F == FMT_BF16) {
        L.c[ct] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(lo_row[ct] + (size_t)u * 64));
      } else {
        const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(lo_row[ct] + (size_t)u * 32));
        L.c[ct] = u32x4_t{v.x, v.y, 0u, 0u};
      }
      if constexpr (F == FMT_Q5) L.h[ct] = *reinterpret_cast<const uint16_t*>(hi_row[ct] + (size_t)u * 8);
      if constexpr (F == FMT_Q6) L.h[ct] = *reinterpret_cast<const uint32_t*>(hi_row[ct] + (size_t)u * 16);
      if constexpr (F == FMT_NVFP4) L.h[ct] = sc_row[ct][(size_t)u * 4];
      if constexpr (SCALED) L.s[ct] = reinterpret_cast<const uint16_t*>(sc_row[ct])[u];
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int p = 0; p < XH; ++p)
        L.a[tt][p] = *reinterpret_cast<const u32x4_t*>(x_row[tt] + (size_t)u * U::K + 8 * p);
  };

  // constant operands of the offset codes (q = 16 for Q5, 32 for Q6; c = 0 for W8)
  const uint32_t kc = F == FMT_Q5 ? 0x43104310u : F == FMT_Q6 ? 0x43204320u : 0x43004300u;
  const bf16x8_t bconst = __builtin_bit_cast(bf16x8_t, u32x4_t{kc, kc, kc, kc});
  const bf16x8_t bconst_hi = __builtin_bit_cast(bf16x8_t, u32x4_t{0x43C043C0u, 0x43C043C0u, 0x43C043C0u, 0x43C043C0u});
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

  f32x4_t acc[CT][TT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[ct][tt] = zero4;

  // the products of one unit
  auto unit_products = [&](const Loads<F, CT, TT>& L) __device__ {
    if constexpr (NIB) {
      bf16x8_t av[TT][2];
      f32x4_t cr[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        av[tt][0] = pair_order(L.a[tt][0]);
        av[tt][1] = pair_order(L.a[tt][1]);
        cr[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tt][0], bconst, zero4, 0, 0, 0);
        cr[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tt][1], bconst, cr[tt], 0, 0, 0);
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        bf16x8_t b0, b1;
        if constexpr (F == FMT_Q5) {
          b0 = q5_operand(L.c[ct].x, L.h[ct] & 0xFFu);
          b1 = q5_operand(L.c[ct].y, L.h[ct] >> 8);
        } else {
          b0 = q6_operand(L.c[ct].x, L.h[ct] & 0xFFFFu);
          b1 = q6_operand(L.c[ct].y, L.h[ct] >> 16);
        }
        const float s = f16_bits_to_f32(L.s[ct]);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          f32x4_t p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tt][0], b0, zero4, 0, 0, 0);
          p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tt][1], b1, p, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[ct][tt][r] = __builtin_fmaf(s, p[r] - cr[tt][r], acc[ct][tt][r]);
        }
      }
    } else if constexpr (F == FMT_W8) {
      bf16x8_t av[TT];
      f32x4_t cr[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        av[tt] = __builtin_bit_cast(bf16x8_t, L.a[tt][0]);
        cr[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tt], bconst, zero4, 0, 0, 0);
        cr[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tt], bconst_hi, cr[tt], 0, 0, 0);
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        bf16x8_t bl, bh;
        w8_operands(L.c[ct].x, L.c[ct].y, bl, bh);
        const float s = f16_bits_to_f32(L.s[ct]);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          f32x4_t p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tt], bl, zero4, 0, 0, 0);
          p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tt], bh, p, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[ct][tt][r] = __builtin_fmaf(s, p[r] - cr[tt][r], acc[ct][tt][r]);
        }
      }
    } else if constexpr (F == FMT_NVFP4) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const float s = e4m3_to_f32(L.h[ct]);
        const bf16x8_t b0 = nvfp4_operand(L.c[ct].x, s), b1 = nvfp4_operand(L.c[ct].y, s);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          acc[ct][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, L.a[tt][0]), b0,
                                                                acc[ct][tt], 0, 0, 0);
          acc[ct][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, L.a[tt][1]), b1,
                                                                acc[ct][tt], 0, 0, 0);
        }
      }
    } else {  // BF16_CTRL
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          acc[ct][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, L.a[tt][0]),
                                                                __builtin_bit_cast(bf16x8_t, L.c[ct]), acc[ct][tt],
                                                                0, 0, 0);
    }
  };

  // the wave's units, kUnroll per step, the next step's loads in flight
  // during this step's products (indexes past the run repeat its last unit,
  // so every load stays inside the planes; those units are skipped)
  if (ub < ue) {
    Loads<F, CT, TT> cur[kUnroll], nxt[kUnroll];
#pragma unroll
    for (int v = 0; v < kUnroll; ++v) load(min(ub + v, ue - 1), cur[v]);
    for (int u = ub; u < ue; u += kUnroll) {
#pragma unroll
      for (int v = 0; v < kUnroll; ++v) load(min(u + kUnroll + v, ue - 1), nxt[v]);
#pragma unroll
      for (int v = 0; v < kUnroll; ++v)
        if (u + v < ue) unit_products(cur[v]);
#pragma unroll
      for (int v = 0; v < kUnroll; ++v) cur[v] = nxt[v];
    }
  }

  // eight-way sum in binary64: red[wave][t < 32][col < BN] binary32 partials
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int col = 16 * ct + li;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tt + 4 * lq + r;
        if (col < BN && t < T) red[(wave * 32 + t) * BN + col] = acc[ct][tt][r];
      }
  }
  __syncthreads();
  for (int i = tid; i < T * rows; i += kThreads) {
    const int t = i / rows, col = i - t * rows;
    double v = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += (double)red[(w * 32 + t) * BN + col];
    uint16_t h = f32_to_bf16_rne((float)v);
    if ((h & 0x7F80u) == 0x7F80u) h = exact_output<F>(x, lo, hi, sc, K, n0 + col, t);  // rare
    y[(size_t)t * N + n0 + col] = h;
  }
}

template <int F, int CT, int TT>
hipError_t launch_one(const FmtArgs& a, const FmtPlan& p, const uint16_t* x, uint16_t* y, int t, hipStream_t s) {
  auto kern = fmt_kernel<F, CT, TT>;
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(kern));
  if (e != hipSuccess) return e;
  kern<<<dim3((unsigned)p.blocks), dim3(kThreads), p.lds_bytes, s>>>(
      x, static_cast<const uint8_t*>(a.lo), static_cast<const uint8_t*>(a.hi), static_cast<const uint8_t*>(a.sc), y,
      (int)a.n, (int)a.k, t, p.bn);
  return hipGetLastError();
}

template <int F>
hipError_t launch_fmt_t(const FmtArgs& a, const FmtPlan& p, hipStream_t s) {
  // 32 tokens per launch (a weight read per launch)
  for (int64_t t0 = 0; t0 < a.t; t0 += 32) {
    const int t = (int)(a.t - t0 < 32 ? a.t - t0 : 32);
    const uint16_t* x = static_cast<const uint16_t*>(a.x) + t0 * a.k;
    uint16_t* y = static_cast<uint16_t*>(a.y) + t0 * a.n;
    hipError_t e;
    const int tt = t > 16 ? 2 : 1;
    if (tt == 1) {
      switch (p.ct) {
        case 1: e = launch_one<F, 1, 1>(a, p, x, y, t, s); break;
        case 2: e = launch_one<F, 2, 1>(a, p, x, y, t, s); break;
        case 3: e = launch_one<F, 3, 1>(a, p, x, y, t, s); break;
        default: e = launch_one<F, 4, 1>(a, p, x, y, t, s); break;
      }
    } else {
      switch (p.ct) {
        case 1: e = launch_one<F, 1, 2>(a, p, x, y, t, s); break;
        case 2: e = launch_one<F, 2, 2>(a, p, x, y, t, s); break;
        case 3: e = launch_one<F, 3, 2>(a, p, x, y, t, s); break;
        default: e = launch_one<F, 4, 2>(a, p, x, y, t, s); break;
      }
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

bool fmt_plan(int fmt, int64_t n, int64_t k, int64_t t, FmtPlan* p) {
  if (fmt < FMT_Q5 || fmt > FMT_BF16 || n < 1 || t < 1 || k < 64 || (k % 64) != 0) return false;
  // per-row offsets are 64-bit; the kernel's int arithmetic needs N, K, T below 2^31
  if (n >= (int64_t(1) << 31) || k >= (int64_t(1) << 30) || t >= (int64_t(1) << 31)) return false;
  int64_t bn = (n + 255) / 256;  // about one workgroup per CU
  if (bn > 64) bn = 64;          // at most four 16-row column tiles per wave
  const int64_t ct = (bn + 15) / 16;
  p->bn = (int)bn;
  p->ct = (int)ct;
  p->blocks = (int)((n + bn - 1) / bn);
  p->lds_bytes = (size_t)kWaves * 32 * (size_t)bn * 4;
  return true;
}

hipError_t launch_fmt(const FmtArgs& a, hipStream_t stream) {
  FmtPlan p;
  if (!fmt_plan(a.fmt, a.n, a.k, a.t, &p)) return hipErrorInvalidValue;
  switch (a.fmt) {
    case FMT_Q5: return launch_fmt_t<FMT_Q5>(a, p, stream);
    case FMT_Q6: return launch_fmt_t<FMT_Q6>(a, p, stream);
    case FMT_W8: return launch_fmt_t<FMT_W8>(a, p, stream);
    case FMT_NVFP4: return launch_fmt_t<FMT_NVFP4>(a, p, stream);
    case FMT_BF16: return launch_fmt_t<FMT_BF16>(a, p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace q4lin
