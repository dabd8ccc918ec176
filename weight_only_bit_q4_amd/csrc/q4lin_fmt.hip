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
// the waves split K into eight contiguous runs of pairs of "units" (a unit
// is one scale group of Q5/Q6/W8, 64 weights of NVFP4, 32 of BF16), so
// every weight byte is read once for all T <= 32 tokens.  Lane l serves row
// 16 ct + l % 16.  Its code loads are 16 contiguous bytes per row and pair:
// quarter q = l / 16 reads half q % 2 of unit q / 2 (BF16: quarter q of
// each unit), with the matching high bits; lanes l and l + 32 then swap
// half of them, so every matrix-core instruction still reduces within one
// unit.  The block's scales are copied into LDS once.  Activations: 16 or
// 32 contiguous bytes per token and unit.  Longer T runs the kernel once
// per 32 tokens.
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
//     scale, whose upper half is already the bf16 value) and fed straight
//     to the matrix cores.
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
constexpr int kTableBytes = 88 * 1024;   // LDS for the block's scales (with the 64 KiB sum area: 152 KiB)
constexpr int kLdsBytes = 160 * 1024;    // LDS of one workgroup
constexpr uint32_t kNowhere = 0x80000000u;  // a buffer offset past every range: reads zeros, no access

// Buffer loads: offsets at or past the resource's byte count return zeros
// without a memory access, so loads past a wave's run need no branch (and
// the wait counts stay fixed).
using rsrc_t = __amdgpu_buffer_rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16-byte direct-to-LDS buffer load: each lane sends 16 bytes from base +
// voffset to lds_base + 16 * lane (lds_base wave-uniform)
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voffset, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, voffset, 0,
                                           0, 0);
}

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4
// and lgkmcnt 11:8 left at "no wait")
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt holds 0..63");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (((N >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4)); }

// A unit is one scale group (Q5, Q6, W8), 64 weights (NVFP4) or 32 (BF16):
// weights, code bytes per row, scale bytes per row
template <int F>
struct Unit {
  static constexpr int K = (F == FMT_W8 || F == FMT_BF16) ? 32 : 64;
  static constexpr int CB = F == FMT_BF16 ? 64 : 32;
  static constexpr int SB = F == FMT_NVFP4 ? 4 : F == FMT_BF16 ? 0 : 2;
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

// Q4: code dword w (nibbles of k0..k7) -> the eight exact bf16 values
// 128 + q in pair order
__device__ __forceinline__ bf16x8_t q4_operand(uint32_t w) {
  u32x4_t r;
  r.x = and_or(w, 0x000F000Fu, 0x43004300u);
  r.y = and_or(w >> 4, 0x000F000Fu, 0x43004300u);
  r.z = and_or(w >> 8, 0x000F000Fu, 0x43004300u);
  r.w = and_or(w >> 12, 0x000F000Fu, 0x43004300u);
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
// the eight exact bf16 weights in natural order.  E2M1 has at most 2
// significant bits and E4M3 at most 4, so the binary32 product is exact
// and fits bf16: its upper half is the weight, no rounding.
__device__ __forceinline__ uint32_t nvfp4_pair(f32x2_t v, float s) {
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, v.y * s), __builtin_bit_cast(uint32_t, v.x * s),
                               0x07060302u);
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
      if constexpr (F == FMT_Q4) {
        return (double)(nib - 8) * s;
      } else if constexpr (F == FMT_Q5) {
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
// over k in binary64 of exact products (plus the residual), rounded once.
// Finite outputs never come here.
template <int F>
__device__ __attribute__((noinline)) uint16_t exact_output(const uint16_t* __restrict__ x,
                                                           const uint8_t* __restrict__ lo,
                                                           const uint8_t* __restrict__ hi,
                                                           const uint8_t* __restrict__ sc,
                                                           const uint16_t* __restrict__ res, int N, int K, int n,
                                                           int t) {
  double acc = 0.0;
  for (int k = 0; k < K; ++k)
    acc += weight_exact<F>(lo, hi, sc, K, n, k) * (double)bf16_bits_to_f32(x[(size_t)t * K + k]);
  if (res != nullptr) acc += (double)bf16_bits_to_f32(res[(size_t)t * N + n]);
  return f32_to_bf16_rne((float)acc);
}

// One lane's loads for one pair of units: 16 code bytes per row (two loads
// of 16 for BF16_CTRL), the high bits that go with them, and the
// activations of both units for TT token tiles.
template <int F, int CT, int TT>
struct Loads {
  static constexpr int NC = F == FMT_BF16 ? 2 : 1;       // 16-byte code loads per row
  static constexpr int NH = F == FMT_Q6 ? 2 : 1;         // high-bit dwords per row
  static constexpr int XH = Unit<F>::K == 64 ? 2 : 1;    // 16-byte activation pieces per unit and token
  u32x4_t c[CT][NC];
  uint32_t h[CT][NH];
  u32x4_t a[2][TT][XH];
};

template <int F, int CT, int TT, int WT>
__global__ void __launch_bounds__(kThreads, 1)
fmt_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ lo, const uint8_t* __restrict__ hi,
           const uint8_t* __restrict__ sc, uint16_t* __restrict__ y, const uint16_t* __restrict__ res, int f32out,
           int N, int K, int T, int BN) {
  using U = Unit<F>;
  using L_t = Loads<F, CT, TT>;
  constexpr int XH = L_t::XH;
  constexpr bool NIB = (F == FMT_Q4 || F == FMT_Q5 || F == FMT_Q6);  // nibble codes with an offset
  constexpr int WK = kWaves / WT;  // waves per token range: each takes a K run
  constexpr int BT = 32 * WT;      // tokens per launch
  constexpr bool PAIRED = F != FMT_BF16;                 // one 16-byte load spans a pair of units
  constexpr int NB = 2;                                  // pairs in flight (register sets)
  // Above 16 tokens the activations go through a ring in LDS: each wave
  // copies its pairs' activations with direct-to-LDS loads in memory order
  // (consecutive lanes read consecutive 16-byte pieces of a token, so the
  // loads coalesce) and reads them back in matrix-core operand order.
  constexpr bool XL = TT == 2;
  constexpr int TTK = 16 * TT;                // tokens per wave
  constexpr int PPT = U::K * 2 / 16;          // 16-byte pieces per token and unit
  constexpr int SLOT = 2 * TTK * PPT * 16;    // one pair's activations [unit][token][piece]
  constexpr int NI = 2 * TTK * PPT / 64;      // direct-to-LDS loads per pair
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wk = wave % WK, wt = wave / WK;  // K run, 32-token range
  const int li = lane & 15, lq = lane >> 4;
  // the quarter of each unit this lane multiplies: after the exchange of
  // the paired loads, quarter lq holds code bytes 8 xq .. 8 xq + 7 of a unit
  const int xq = PAIRED ? (((lq & 1) << 1) | (lq >> 1)) : lq;
  const int n0 = blockIdx.x * BN;
  const int rows = min(BN, N - n0);
  const int units = K / U::K;
  const int pairs = (units + 1) >> 1;
  const int pb = (int)(((int64_t)pairs * wk) / WK), pe = (int)(((int64_t)pairs * (wk + 1)) / WK);
  const int ts = units * U::SB;  // bytes of one row's scales
  // LDS: [activation rings of the 8 waves (XL)] or [partials], then the
  // scale table; the partials of the final sum reuse the start
  uint8_t* tab = lds + (XL ? (size_t)kWaves * 2 * SLOT : (size_t)kWaves * 32 * BN * 4);

  // Byte offsets of this lane's loads, per column tile (rows past the
  // block repeat the last one; their sums are never stored), relative to
  // buffers over the block's rows of each plane.
  const int row_bytes = units * U::CB;
  constexpr int HB = F == FMT_Q5 ? 8 : F == FMT_Q6 ? 16 : 0;  // high-plane bytes per unit and row
  const rsrc_t rlo = make_rsrc(lo + (size_t)n0 * row_bytes, (uint32_t)(rows * row_bytes));
  const rsrc_t rhi = make_rsrc(HB ? hi + (size_t)n0 * units * HB : lo, (uint32_t)(rows * units * HB));
  const rsrc_t rx = make_rsrc(x, (uint32_t)((size_t)T * K * 2));
  uint32_t lo_off[CT], hi_off[CT];
  int tab_row[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int rl = min(16 * ct + li, rows - 1);
    // paired formats: quarter lq reads half lq % 2 of the pair's unit lq / 2
    if constexpr (F == FMT_BF16) lo_off[ct] = (uint32_t)(rl * row_bytes + lq * 16);
    else lo_off[ct] = (uint32_t)(rl * row_bytes + (lq >> 1) * U::CB + (lq & 1) * 16);
    hi_off[ct] = (uint32_t)(rl * units * HB + (lq >> 1) * HB + (lq & 1) * (HB / 2));
    tab_row[ct] = rl * ts;
  }
  uint32_t x_off[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
    x_off[tt] = (uint32_t)(min(32 * wt + 16 * tt + li, T - 1) * K * 2 + xq * 16 * XH);

  // The ring: slot p % 2 holds pair p's activations, piece (v, tl, pc) at
  // position (v TTK + tl) PPT + (pc ^ (tl % PPT)) (the XOR spreads the
  // operand reads of 16 tokens over the banks).  Load j of a pair moves
  // positions 64 j .. 64 j + 63, lane l the one at 64 j + l.
  uint8_t* const ring = lds + (size_t)wave * 2 * SLOT;
  uint32_t xdma[XL ? NI : 1];
  if constexpr (XL) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int q = j * 64 + lane;
      const int v = q / (TTK * PPT), tl = (q / PPT) % TTK, pc = (q % PPT) ^ (tl % PPT);
      xdma[j] = (uint32_t)(min(32 * wt + tl, T - 1) * K * 2 + v * U::K * 2 + pc * 16);
    }
  }
  // a pair past the wave's run reads nothing (zeros land in the slot)
  auto issue_x = [&](int p) __device__ {
    if constexpr (XL) {
      uint8_t* slot = ring + (p & 1) * SLOT;
      const uint32_t base = (uint32_t)(2 * p * U::K * 2);
#pragma unroll
      for (int j = 0; j < NI; ++j) dma16(rx, p < pe ? xdma[j] + base : kNowhere, slot + j * 1024);
    }
  };
  // pair p's operands: lane (li, lq) takes pieces XH xq .. XH xq + XH - 1 of
  // token 16 tt + li in each unit
  auto read_x = [&](int p, u32x4_t (&A)[2][TT][XH]) __device__ {
    const uint8_t* slot = ring + (p & 1) * SLOT;
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int h = 0; h < XH; ++h) {
          const int tl = 16 * tt + li;
          A[v][tt][h] = *reinterpret_cast<const u32x4_t*>(
              slot + ((v * TTK + tl) * PPT + ((XH * xq + h) ^ (tl % PPT))) * 16);
        }
  };

  // Pair p covers units 2p and 2p + 1.  A pair past the wave's run reads
  // nothing; the second unit of the last pair of an odd count reads the
  // next row's bytes or nothing, and its products are skipped.
  auto load = [&](int p, L_t& L) __device__ {
    const bool live = p < pe;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      if constexpr (F == FMT_BF16) {
#pragma unroll
        for (int v = 0; v < 2; ++v)
          L.c[ct][v] = __builtin_amdgcn_raw_buffer_load_b128(
              rlo, live ? lo_off[ct] + (uint32_t)((2 * p + v) * U::CB) : kNowhere, 0, 2);
      } else {
        L.c[ct][0] = __builtin_amdgcn_raw_buffer_load_b128(rlo, live ? lo_off[ct] + (uint32_t)(2 * p * U::CB) : kNowhere,
                                                           0, 2);
      }
      const uint32_t ho = live ? hi_off[ct] + (uint32_t)(2 * p * HB) : kNowhere;
      if constexpr (F == FMT_Q5) L.h[ct][0] = __builtin_amdgcn_raw_buffer_load_b32(rhi, ho, 0, 0);
      if constexpr (F == FMT_Q6) {
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rhi, ho, 0, 0);
        L.h[ct][0] = v.x;
        L.h[ct][1] = v.y;
      }
    }
    if constexpr (!XL) {
#pragma unroll
      for (int v = 0; v < 2; ++v)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int p2 = 0; p2 < XH; ++p2)
            L.a[v][tt][p2] = __builtin_amdgcn_raw_buffer_load_b128(
                rx, live ? x_off[tt] + (uint32_t)(((2 * p + v) * U::K + 8 * p2) * 2) : kNowhere, 0, 0);
    }
  };

  // The block's scales go to LDS once (their rows are contiguous in the
  // plane): eight 2-byte elements per thread and batch.
  const int elems = rows * ts / 2;
  const rsrc_t rsc = make_rsrc(U::SB ? sc + (size_t)n0 * ts : lo, (uint32_t)(rows * ts));
  uint16_t* sdst = reinterpret_cast<uint16_t*>(tab);
  auto stage_load = [&](int i0, uint16_t (&v)[8]) __device__ {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + j * kThreads + tid;
      v[j] = __builtin_amdgcn_raw_buffer_load_b16(rsc, i < elems ? (uint32_t)(2 * i) : kNowhere, 0, 0);
    }
  };
  auto stage_store = [&](int i0, const uint16_t (&v)[8]) __device__ {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + j * kThreads + tid;
      if (i < elems) sdst[i] = v[j];
    }
  };

  // constant operands of the offset codes (q = 8 for Q4, 16 for Q5, 32 for Q6; c = 0 for W8)
  const uint32_t kc = F == FMT_Q4   ? 0x43084308u
                      : F == FMT_Q5 ? 0x43104310u
                      : F == FMT_Q6 ? 0x43204320u
                                    : 0x43004300u;
  const bf16x8_t bconst = __builtin_bit_cast(bf16x8_t, u32x4_t{kc, kc, kc, kc});
  const bf16x8_t bconst_hi = __builtin_bit_cast(bf16x8_t, u32x4_t{0x43C043C0u, 0x43C043C0u, 0x43C043C0u, 0x43C043C0u});
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  const int hsh = (lane >> 5) << 4;  // Q5: the half of a high dword that belongs to this lane

  f32x4_t acc[CT][TT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[ct][tt] = zero4;

  // the products of unit u: a = its activations, c = this lane's 8 code
  // bytes per row (two dwords), h = their high bits
  auto unit_products = [&](int u, const u32x4_t (&a)[TT][XH], const u32x2_t (&c)[CT], const uint32_t (&h)[CT])
      __device__ {
    if constexpr (NIB) {
      bf16x8_t av[TT][2];
      f32x4_t cr[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        av[tt][0] = pair_order(a[tt][0]);
        av[tt][1] = pair_order(a[tt][1]);
        cr[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tt][0], bconst, zero4, 0, 0, 0);
        cr[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tt][1], bconst, cr[tt], 0, 0, 0);
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        bf16x8_t b0, b1;
        if constexpr (F == FMT_Q4) {
          b0 = q4_operand(c[ct].x);
          b1 = q4_operand(c[ct].y);
        } else if constexpr (F == FMT_Q5) {
          b0 = q5_operand(c[ct].x, h[ct]);
          b1 = q5_operand(c[ct].y, h[ct] >> 8);
        } else {
          b0 = q6_operand(c[ct].x, h[ct]);
          b1 = q6_operand(c[ct].y, h[ct] >> 16);
        }
        const float s = f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(tab + tab_row[ct] + 2 * u));
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
        av[tt] = __builtin_bit_cast(bf16x8_t, a[tt][0]);
        cr[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tt], bconst, zero4, 0, 0, 0);
        cr[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tt], bconst_hi, cr[tt], 0, 0, 0);
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        bf16x8_t bl, bh;
        w8_operands(c[ct].x, c[ct].y, bl, bh);
        const float s = f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(tab + tab_row[ct] + 2 * u));
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          f32x4_t p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tt], bl, zero4, 0, 0, 0);
          p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tt], bh, p, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[ct][tt][r] = __builtin_fmaf(s, p[r] - cr[tt][r], acc[ct][tt][r]);
        }
      }
    } else {  // NVFP4: the lane's 16 weights are one E4M3 scale group
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const float s = e4m3_to_f32(tab[tab_row[ct] + 4 * u + xq]);
        const bf16x8_t b0 = nvfp4_operand(c[ct].x, s), b1 = nvfp4_operand(c[ct].y, s);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          acc[ct][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[tt][0]), b0,
                                                                acc[ct][tt], 0, 0, 0);
          acc[ct][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[tt][1]), b1,
                                                                acc[ct][tt], 0, 0, 0);
        }
      }
    }
  };

  // the products of pair p (its second unit is skipped past the row's end)
  auto pair_products = [&](int p, const L_t& L, const u32x4_t (&A)[2][TT][XH]) __device__ {
    const bool second = 2 * p + 1 < units;
    if constexpr (F == FMT_BF16) {
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        if (v == 1 && !second) break;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int tt = 0; tt < TT; ++tt)
            acc[ct][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, A[v][tt][0]),
                                                                  __builtin_bit_cast(bf16x8_t, L.c[ct][v]),
                                                                  acc[ct][tt], 0, 0, 0);
      }
    } else {
      // Lanes l and l + 32 (quarters q and q + 2) exchange half of their
      // 16 bytes: afterwards every lane holds 8 code bytes of each unit,
      // bytes 8 xq .. 8 xq + 7 (and their high bits).
      u32x2_t ca[CT], cb[CT];
      uint32_t ha[CT], hb[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const auto sx = __builtin_amdgcn_permlane32_swap(L.c[ct][0].x, L.c[ct][0].z, false, false);
        const auto sy = __builtin_amdgcn_permlane32_swap(L.c[ct][0].y, L.c[ct][0].w, false, false);
        ca[ct] = u32x2_t{sx[0], sy[0]};
        cb[ct] = u32x2_t{sx[1], sy[1]};
        ha[ct] = hb[ct] = 0u;
        if constexpr (F == FMT_Q5) {
          // both lanes get both dwords: [0] the lower lane's, [1] the upper lane's
          const auto hs = __builtin_amdgcn_permlane32_swap(L.h[ct][0], L.h[ct][0], false, false);
          ha[ct] = hs[0] >> hsh;
          hb[ct] = hs[1] >> hsh;
        }
        if constexpr (F == FMT_Q6) {
          const auto hs = __builtin_amdgcn_permlane32_swap(L.h[ct][0], L.h[ct][1], false, false);
          ha[ct] = hs[0];
          hb[ct] = hs[1];
        }
      }
      unit_products(2 * p, A[0], ca, ha);
      if (second) unit_products(2 * p + 1, A[1], cb, hb);
    }
  };

  // Scales of the block (first batch) in flight with the first two pairs'
  // loads; two register sets (and ring slots) take turns, so while one
  // pair's products run the next pair's loads are in flight.  (A table
  // larger than one batch is copied first, on its own.)
  L_t b[NB];
  uint16_t sv[8];
  const bool one_batch = elems <= 8 * kThreads;
  if constexpr (U::SB > 0) {
    if (!one_batch) {
      for (int i0 = 0; i0 < elems; i0 += 8 * kThreads) {
        stage_load(i0, sv);
        stage_store(i0, sv);
      }
    }
    stage_load(0, sv);  // a repeat of the first batch when already copied
  }
  // per pair, in this order: its activations to LDS (XL), then its codes
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    issue_x(pb + i);
    __builtin_amdgcn_sched_barrier(0);
    load(pb + i, b[i]);
  }
  if constexpr (U::SB > 0) stage_store(0, sv);
  // the table's writes are visible after this; the loads stay in flight
  // (a fence here would also wait for the copies into the rings)
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  // loads per pair: LC code-plane loads after NI activation loads
  constexpr int LC = CT * (Loads<F, CT, TT>::NC + ((F == FMT_Q5 || F == FMT_Q6) ? 1 : 0));
  // (Every load is issued outside the branches, so the compiler's count of
  // the loads in flight stays exact.)
  for (int p = pb; p < pe; p += NB) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      u32x4_t A[2][TT][XH];
      if constexpr (XL) {
        // pair p + i's activations have landed once only the loads issued
        // after them (its codes, the next pair's activations and codes) may
        // be outstanding
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<2 * LC + NI>();
        read_x(p + i, A);
        wait_lgkm0();
        __builtin_amdgcn_sched_barrier(0);
        issue_x(p + i + NB);  // into the slot just read
        __builtin_amdgcn_sched_barrier(0);
      } else {
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
          for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int h = 0; h < XH; ++h) A[v][tt][h] = b[i].a[v][tt][h];
      }
      if (i == 0 || p + i < pe) pair_products(p + i, b[i], A);
      load(p + i + NB, b[i]);
    }
  }
  if constexpr (XL) {
    wait_vm<0>();  // every copy into the rings has landed before they are reused
    __syncthreads();
  }

  // sum over the WK runs in binary64: red[wk][t < BT][col < BN] binary32 partials
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int col = 16 * ct + li;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 32 * wt + 16 * tt + 4 * lq + r;
        if (col < BN && t < T) red[(wk * BT + t) * BN + col] = acc[ct][tt][r];
      }
  }
  __syncthreads();
  for (int i = tid; i < T * rows; i += kThreads) {
    const int t = i / rows, col = i - t * rows;
    double v = 0.0;
#pragma unroll
    for (int w = 0; w < WK; ++w) v += (double)red[(w * BT + t) * BN + col];
    const size_t o = (size_t)t * N + n0 + col;
    if (f32out) {
      reinterpret_cast<float*>(y)[o] = (float)v;  // binary32 sums (the gate and up of LinearSwiGLU)
      continue;
    }
    if (res != nullptr) v += (double)bf16_bits_to_f32(res[o]);  // LinearAdd
    uint16_t h = f32_to_bf16_rne((float)v);
    if ((h & 0x7F80u) == 0x7F80u) h = exact_output<F>(x, lo, hi, sc, res, N, K, n0 + col, t);  // rare
    y[o] = h;
  }
}

template <int F, int CT, int TT, int WT>
hipError_t launch_one(const FmtArgs& a, const FmtPlan& p, const uint16_t* x, uint16_t* y, const uint16_t* res,
                      int t, hipStream_t s) {
  auto kern = fmt_kernel<F, CT, TT, WT>;
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(kern));
  if (e != hipSuccess) return e;
  kern<<<dim3((unsigned)p.blocks), dim3(kThreads), p.lds_bytes, s>>>(
      x, static_cast<const uint8_t*>(a.lo), static_cast<const uint8_t*>(a.hi), static_cast<const uint8_t*>(a.sc), y,
      res, a.f32 ? 1 : 0, (int)a.n, (int)a.k, t, p.bn);
  return hipGetLastError();
}

template <int F, int TT, int WT>
hipError_t launch_ct(const FmtArgs& a, const FmtPlan& p, const uint16_t* x, uint16_t* y, const uint16_t* res, int t,
                     hipStream_t s) {
  switch (p.ct) {
    case 1: return launch_one<F, 1, TT, WT>(a, p, x, y, res, t, s);
    case 2: return launch_one<F, 2, TT, WT>(a, p, x, y, res, t, s);
    case 3: return launch_one<F, 3, TT, WT>(a, p, x, y, res, t, s);
    default: return launch_one<F, 4, TT, WT>(a, p, x, y, res, t, s);
  }
}

template <int F>
hipError_t launch_fmt_t(const FmtArgs& a, const FmtPlan& p, hipStream_t s) {
  // up to 128 tokens per launch (a weight read per launch): 32 per token
  // range of waves, 16 per tile
  const size_t osz = a.f32 ? 4 : 2;
  for (int64_t t0 = 0; t0 < a.t; t0 += 128) {
    const int t = (int)(a.t - t0 < 128 ? a.t - t0 : 128);
    const uint16_t* x = static_cast<const uint16_t*>(a.x) + t0 * a.k;
    uint16_t* y = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(a.y) + (size_t)t0 * a.n * osz);
    const uint16_t* res = a.res ? static_cast<const uint16_t*>(a.res) + t0 * a.n : nullptr;
    hipError_t e;
    if (t <= 16) e = launch_ct<F, 1, 1>(a, p, x, y, res, t, s);
    else if (t <= 32) e = launch_ct<F, 2, 1>(a, p, x, y, res, t, s);
    else if (t <= 64) e = launch_ct<F, 2, 2>(a, p, x, y, res, t, s);
    else e = launch_ct<F, 2, 4>(a, p, x, y, res, t, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

bool fmt_plan(int fmt, int64_t n, int64_t k, int64_t t, FmtPlan* p) {
  if (fmt < FMT_Q4 || fmt > FMT_BF16 || n < 1 || t < 1 || k < 64 || (k % 64) != 0) return false;
  // per-row offsets are 64-bit; the kernel's int arithmetic needs N, K, T below 2^31
  if (n >= (int64_t(1) << 31) || k >= (int64_t(1) << 30) || t >= (int64_t(1) << 31)) return false;
  // bytes of one row's scales in the LDS table
  const int64_t ts = fmt == FMT_BF16 ? 0 : fmt == FMT_W8 || fmt == FMT_NVFP4 ? k / 16 : k / 32;
  // launches of more than 16 tokens keep the waves' activation rings in LDS
  // (two slots of 2 units x 32 tokens per wave)
  const int64_t ppt = (fmt == FMT_W8 || fmt == FMT_BF16) ? 4 : 8;
  const int64_t ring = t > 16 ? (int64_t)kWaves * 2 * (2 * 32 * ppt * 16) : 0;
  const int64_t table_cap = ring + kTableBytes <= kLdsBytes ? kTableBytes : kLdsBytes - ring;
  int64_t bn = (n + 255) / 256;  // about one workgroup per CU
  if (bn > 64) bn = 64;          // at most four 16-row column tiles per wave
  if (ts > 0 && bn * ts > table_cap) bn = table_cap / ts;
  if (bn < 1) return false;
  const int64_t ct = (bn + 15) / 16;
  p->bn = (int)bn;
  p->ct = (int)ct;
  p->blocks = (int)((n + bn - 1) / bn);
  // binary32 partials [8 waves][32 tokens][bn] (the same for every split of
  // the waves into token ranges; they reuse the rings), then the scale table
  const int64_t red = (int64_t)kWaves * 32 * bn * 4;
  p->lds_bytes = (size_t)((red > ring ? red : ring) + (bn * ts + 15) / 16 * 16);
  return true;
}

hipError_t launch_fmt(const FmtArgs& a, hipStream_t stream) {
  FmtPlan p;
  if (!fmt_plan(a.fmt, a.n, a.k, a.t, &p)) return hipErrorInvalidValue;
  switch (a.fmt) {
    case FMT_Q4: return launch_fmt_t<FMT_Q4>(a, p, stream);
    case FMT_Q5: return launch_fmt_t<FMT_Q5>(a, p, stream);
    case FMT_Q6: return launch_fmt_t<FMT_Q6>(a, p, stream);
    case FMT_W8: return launch_fmt_t<FMT_W8>(a, p, stream);
    case FMT_NVFP4: return launch_fmt_t<FMT_NVFP4>(a, p, stream);
    case FMT_BF16: return launch_fmt_t<FMT_BF16>(a, p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace q4lin
