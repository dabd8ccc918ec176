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
// every weight byte is read once per launch.  Lane l serves row
// 16 ct + l % 16.  Its code loads are 16 contiguous bytes per row and pair:
// quarter q = l / 16 reads half q % 2 of unit q / 2 (BF16: quarter q of
// each unit), with the matching high bits; lanes l and l + 32 then swap
// half of them, so every matrix-core instruction still reduces within one
// unit.  The block's scales are copied into LDS once.
//   * Up to 16 tokens (fmt_kernel): the activations of a pair go straight
//     to registers with its codes (16 or 32 contiguous bytes per token and
//     unit).
//   * 17 to 128 tokens (fmt_tok_kernel, up to 64 with 3 or 4 column tiles):
//     every wave takes all the launch's tokens for its run, so each code
//     operand is built once for all of them; the activations pass through a
//     per-wave ring in LDS (direct copies in memory order, read back in
//     operand order); a wave's codes are loaded several pairs at a time.
//   Longer T runs the kernel once per 128 (64) tokens.
//
// Arithmetic (v_mfma_f32_16x16x32_bf16, A = activations, B = weights, every
// instruction reduces over one unit):
//   * Q4: one three-input bitwise operation per pair of weights builds the
//     exact bf16 value 128 + q (q < 128 has unit spacing there); up to 16
//     tokens in the pair order of a code dword as below, from 17 tokens in
//     the activations' own order (k0,k1) (k2,k3) ... (one byte permute per
//     pair), so the activation pieces need no permute; the correction is as
//     for Q5/Q6 with offset 8;
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
constexpr int kRingWave = 16 * 1024;      // LDS of one wave's activation ring (17 to 128 tokens)

// Buffer loads: offsets at or past the resource's byte count return zeros
// without a memory access, so loads past a wave's run need no branch (and
// the wait counts stay fixed).
using rsrc_t = __amdgpu_buffer_rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16-byte direct-to-LDS buffer load: each lane sends 16 bytes from base +
// voffset + soffset to lds_base + 16 * lane (soffset and lds_base
// wave-uniform)
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voffset, uint32_t soffset, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, voffset,
                                           soffset, 0, 0);
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

// Q4: code dword w (nibbles of k0..k7) -> the eight exact bf16 values
// 128 + q in natural order (k0,k1) (k2,k3) (k4,k5) (k6,k7): byte b of w
// gives its low nibble to the pair's low half and, through w >> 4, its high
// nibble to the high half
__device__ __forceinline__ bf16x8_t q4_natural(uint32_t w) {
  const uint32_t u = w >> 4;
  u32x4_t r;
  r.x = and_or(__builtin_amdgcn_perm(u, w, 0x04040000u), 0x000F000Fu, 0x43004300u);
  r.y = and_or(__builtin_amdgcn_perm(u, w, 0x05050101u), 0x000F000Fu, 0x43004300u);
  r.z = and_or(__builtin_amdgcn_perm(u, w, 0x06060202u), 0x000F000Fu, 0x43004300u);
  r.w = and_or(__builtin_amdgcn_perm(u, w, 0x07070303u), 0x000F000Fu, 0x43004300u);
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

// Per-format load shape: 16-byte code loads per row and pair, high-bit
// dwords per row, 16-byte activation pieces per unit and token, high-plane
// bytes per unit and row, loads per column tile and pair.
template <int F>
struct Fmt {
  static constexpr int NC = F == FMT_BF16 ? 2 : 1;
  static constexpr int NH = F == FMT_Q6 ? 2 : 1;
  static constexpr int XH = Unit<F>::K == 64 ? 2 : 1;
  static constexpr int HB = F == FMT_Q5 ? 8 : F == FMT_Q6 ? 16 : 0;
  static constexpr int LPT = NC + ((F == FMT_Q5 || F == FMT_Q6) ? 1 : 0);
  static constexpr bool NIB = F == FMT_Q4 || F == FMT_Q5 || F == FMT_Q6;  // nibble codes with an offset
  static constexpr bool PAIRED = F != FMT_BF16;                            // one 16-byte load spans two units
};

// The codes of one pair of units for CT column tiles (and their high bits)
template <int F, int CT>
struct PairCodes {
  u32x4_t c[CT][Fmt<F>::NC];
  uint32_t h[CT][Fmt<F>::NH];
};

// Byte offsets of this lane's code loads per column tile (rows past the
// block repeat the last one; their sums are never stored), relative to
// buffers over the block's rows of each plane, and the lane's row in the
// scale table.  A tile's pair of units is 64 bytes of each of its 16 rows
// (paired formats: piece q is half q % 2 of unit q / 2; BF16_CTRL: piece q
// of each unit); lane (li, lq) multiplies piece lq of row li.  Direct: it
// loads that piece itself (a quarter-wave reads 16 rows).  COAL: lane l
// loads piece l % 4 of row l / 4 (a quarter-wave reads four rows, about
// three times faster through the address unit) and a lane exchange hands
// the pieces over.  GLU: the first CT / 2 tiles are the gate weight's rows,
// the others the same rows of the up weight, whose scales follow the
// gate's in the table.
template <int F, int CT, bool GLU = false, bool COAL = false>
__device__ __forceinline__ void lane_offsets(int rows, int units, int ts, int li, int lq, uint32_t (&lo_off)[CT],
                                             uint32_t (&hi_off)[CT], int (&tab_row)[CT]) {
  constexpr int HB = Fmt<F>::HB;
  constexpr int CTH = GLU ? CT / 2 : CT;  // column tiles per weight
  const int row_bytes = units * Unit<F>::CB;
  const int lane = 16 * lq + li;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int pl = ct / CTH;
    const int rl = min(16 * (ct - pl * CTH) + li, rows - 1);
    const int rc = COAL ? min(16 * (ct - pl * CTH) + (lane >> 2), rows - 1) : rl;  // the row this lane loads
    const int qc = COAL ? (lane & 3) : lq;                                          // and its piece
    if constexpr (F == FMT_BF16) lo_off[ct] = (uint32_t)(rc * row_bytes + qc * 16);
    else lo_off[ct] = (uint32_t)(rc * row_bytes + (qc >> 1) * Unit<F>::CB + (qc & 1) * 16);
    hi_off[ct] = (uint32_t)(rl * units * HB + (lq >> 1) * HB + (lq & 1) * (HB / 2));
    tab_row[ct] = (pl * rows + rl) * ts;
  }
}

// A lane exchange: every lane takes the 16 bytes lane src4 / 4 holds
__device__ __forceinline__ u32x4_t lane_piece(u32x4_t v, int src4) {
  return u32x4_t{(uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)v.x),
                 (uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)v.y),
                 (uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)v.z),
                 (uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)v.w)};
}

// The code loads of pair p: the pair's offset is the wave-uniform buffer
// offset; a pair past the wave's run reads through the empty resource rnull
// (nothing, zeros).  GLU: the last CT / 2 tiles read the up weight (rlo2).
template <int F, int CT, bool GLU = false>
__device__ __forceinline__ void load_codes(rsrc_t rlo, rsrc_t rlo2, rsrc_t rhi, rsrc_t rnull,
                                           const uint32_t (&lo_off)[CT], const uint32_t (&hi_off)[CT], int p,
                                           bool live, PairCodes<F, CT>& L) {
  static_assert(!GLU || Fmt<F>::HB == 0, "the gated pair has no high planes");
  constexpr int CB = Unit<F>::CB, HB = Fmt<F>::HB;
  const rsrc_t ra = live ? rlo : rnull, rb = live ? rlo2 : rnull, rh = live ? rhi : rnull;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const rsrc_t rl = (GLU && ct >= CT / 2) ? rb : ra;
#pragma unroll
    for (int v = 0; v < Fmt<F>::NC; ++v)
      L.c[ct][v] = __builtin_amdgcn_raw_buffer_load_b128(rl, lo_off[ct], (uint32_t)((2 * p + v) * CB), 2);
    if constexpr (F == FMT_Q5) L.h[ct][0] = __builtin_amdgcn_raw_buffer_load_b32(rh, hi_off[ct], (uint32_t)(2 * p * HB), 0);
    if constexpr (F == FMT_Q6) {
      const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rh, hi_off[ct], (uint32_t)(2 * p * HB), 0);
      L.h[ct][0] = v.x;
      L.h[ct][1] = v.y;
    }
  }
}

// Lanes l and l + 32 (quarters q and q + 2) exchange half of their 16 code
// bytes: afterwards every lane holds 8 code bytes of each unit of the pair,
// bytes 8 xq .. 8 xq + 7, and their high bits (ca, ha: the first unit).
template <int F, int CT>
__device__ __forceinline__ void split_pair(const PairCodes<F, CT>& L, int hsh, u32x2_t (&ca)[CT], u32x2_t (&cb)[CT],
                                           uint32_t (&ha)[CT], uint32_t (&hb)[CT]) {
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
}

// The products of unit u of a paired format for TT token tiles: a = its
// activations (XH 16-byte pieces per tile), c = this lane's 8 code bytes per
// row (two dwords), h = their high bits.  NAT: the Q4 operands are built in
// the activations' own order (k0,k1) (k2,k3) ..., so the activation pieces
// go to the matrix cores as loaded; otherwise the code order (k0,k4) (k1,k5)
// ... and the activations are permuted to it.
template <int F, int CT, int TT, bool NAT>
__device__ __forceinline__ void unit_products(int u, const u32x4_t (&a)[TT][Fmt<F>::XH], const u32x2_t (&c)[CT],
                                              const uint32_t (&h)[CT], const uint8_t* tab, const int (&tab_row)[CT],
                                              int xq, f32x4_t (&acc)[CT][TT]) {
  // constant operands of the offset codes (q = 8 for Q4, 16 for Q5, 32 for Q6; c = 0 for W8)
  constexpr uint32_t kc = F == FMT_Q4 ? 0x43084308u : F == FMT_Q5 ? 0x43104310u : F == FMT_Q6 ? 0x43204320u
                                                                                              : 0x43004300u;
  const bf16x8_t bconst = __builtin_bit_cast(bf16x8_t, u32x4_t{kc, kc, kc, kc});
  const bf16x8_t bconst_hi = __builtin_bit_cast(bf16x8_t, u32x4_t{0x43C043C0u, 0x43C043C0u, 0x43C043C0u, 0x43C043C0u});
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  if constexpr (Fmt<F>::NIB) {
    bf16x8_t av[TT][2];
    f32x4_t cr[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      if constexpr (NAT) {
        av[tt][0] = __builtin_bit_cast(bf16x8_t, a[tt][0]);
        av[tt][1] = __builtin_bit_cast(bf16x8_t, a[tt][1]);
      } else {
        av[tt][0] = pair_order(a[tt][0]);
        av[tt][1] = pair_order(a[tt][1]);
      }
      cr[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tt][0], bconst, zero4, 0, 0, 0);
      cr[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tt][1], bconst, cr[tt], 0, 0, 0);
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      bf16x8_t b0, b1;
      if constexpr (F == FMT_Q4 && NAT) {
        b0 = q4_natural(c[ct].x);
        b1 = q4_natural(c[ct].y);
      } else if constexpr (F == FMT_Q4) {
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
}

// BF16_CTRL: one unit (32 weights) of bf16 weights, c = this lane's 16 bytes per row
template <int CT, int TT>
__device__ __forceinline__ void bf16_unit(const u32x4_t (&a)[TT][1], const u32x4_t (&c)[CT],
                                          f32x4_t (&acc)[CT][TT]) {
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
      acc[ct][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[tt][0]),
                                                            __builtin_bit_cast(bf16x8_t, c[ct]), acc[ct][tt], 0, 0, 0);
}

// Each wave copies the scale bytes of its own units [u0, u1) of the block's
// rows into the LDS table ([row][unit], ts bytes a row, the plane's own
// layout).  No other wave reads them, so the copy needs no workgroup
// barrier: a wave starts on its units as soon as its own loads are in.
// 2-byte elements, eight per lane and batch.
struct WaveTable {
  int ts, boff, ner, ne;  // row bytes, byte offset of u0 in a row, elements per row, elements
  __device__ WaveTable(int rows, int ts_, int u0, int u1, int sb)
      : ts(ts_), boff(u0 * sb), ner((u1 - u0) * sb / 2), ne(rows * ((u1 - u0) * sb / 2)) {}
  // byte offsets (in the plane's rows from the block's first and in the
  // table alike) of batch e0's elements; past the end: kNowhere
  __device__ __forceinline__ void offsets(int e0, int lane, uint32_t (&o)[8]) const {
    // one division per lane; each next element (64 further) steps the row
    // by q and the column by m (carrying into the row)
    const int d = ner > 0 ? ner : 1;
    const int q = 64 / d, m = 64 - q * d;
    int e = e0 + lane, r = e / d, c = e - r * d;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      o[j] = e < ne ? (uint32_t)(r * ts + boff + 2 * c) : kNowhere;
      e += 64;
      r += q;
      c += m;
      if (c >= d) {
        c -= d;
        ++r;
      }
    }
  }
  __device__ __forceinline__ void load(rsrc_t rsc, const uint32_t (&o)[8], uint16_t (&v)[8]) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_amdgcn_raw_buffer_load_b16(rsc, o[j], 0, 0);
  }
  __device__ __forceinline__ void store(uint8_t* tab, const uint32_t (&o)[8], const uint16_t (&v)[8]) const {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (o[j] != kNowhere) *reinterpret_cast<uint16_t*>(tab + o[j]) = v[j];
  }
  // every batch after the first, copied at once (long rows only)
  __device__ __forceinline__ void copy_rest(rsrc_t rsc, uint8_t* tab, int lane) const {
    for (int e0 = 8 * 64; e0 < ne; e0 += 8 * 64) {
      uint32_t o[8];
      uint16_t v[8];
      offsets(e0, lane, o);
      load(rsc, o, v);
      store(tab, o, v);
    }
  }
};

// Row stride of the final sum's partials: BN rounded up to 4 mod 16 floats,
// so the four token quads (4 lq rows apart) of a write land 16 banks apart
__host__ __device__ constexpr int red_stride(int bn) { return (bn + 11) / 16 * 16 + 4; }
// Columns of the partials: the block's rows, or for the gated pair both
// weights' rows, the second from BN rounded up to a multiple of 4
__host__ __device__ constexpr int red_cols(int bn, bool glu) { return glu ? 2 * ((bn + 3) & ~3) : bn; }

// The sum over the eight waves' K runs in binary64: red[w][t < 16 TT][col]
// binary32 partials, rows red_stride() floats apart (lane (li, lq) of wave w
// holds row 16 ct + li, tokens 16 tt + 4 lq + r), then one output per
// thread and step (up to 1024 outputs) or four adjacent ones (16-byte
// partial reads; more outputs), each rounded once; an output that comes out
// non-finite is formed again exactly.  GLU: the up weight's rows are columns BNP.. (BN rounded up to a
// multiple of 4), and the output is bf16(silu(G) U) of the two sums.
template <int F, int CT, int TT, bool GLU = false>
__device__ __forceinline__ void final_sum(const f32x4_t (&acc)[CT][TT], uint8_t* lds, int wave, int li, int lq,
                                          int tid, const uint16_t* __restrict__ x, const uint8_t* __restrict__ lo,
                                          const uint8_t* __restrict__ hi, const uint8_t* __restrict__ sc,
                                          uint16_t* __restrict__ y, const uint16_t* __restrict__ res, int f32out,
                                          int N, int K, int T, int BN, int n0, int rows) {
  constexpr int BT = 16 * TT;
  constexpr int CTH = GLU ? CT / 2 : CT;
  const int BNP = GLU ? (BN + 3) & ~3 : BN;
  const int RS = red_stride(red_cols(BN, GLU));
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int pl = ct / CTH, c = 16 * (ct - pl * CTH) + li, col = pl * BNP + c;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tt + 4 * lq + r;
        if (c < BN && t < T) red[(wave * BT + t) * RS + col] = acc[ct][tt][r];
      }
  }
  __syncthreads();
  // one output from its sums (the gate and up sums for GLU)
  auto finish = [&](double v, double u, size_t o, int t, int col) __device__ -> uint16_t {
    if constexpr (GLU) {
      // each sum rounded to binary32 as where the two sums are stored
      // between passes (+0 maps a -0 sum to +0, as a sum of zero products
      // starts at +0), the gate in binary64, one rounding of the product
      const double g = (double)(float)v + 0.0, uv = (double)(float)u + 0.0;
      const double silu = g / (1.0 + exp(-g));
      return f32_to_bf16_rne((float)(silu * uv));
    } else {
      if (res != nullptr) v += (double)bf16_bits_to_f32(res[o]);  // LinearAdd
      uint16_t h = f32_to_bf16_rne((float)v);
      if ((h & 0x7F80u) == 0x7F80u) h = exact_output<F>(x, lo, hi, sc, res, N, K, n0 + col, t);  // rare
      return h;
    }
  };
  if (T * rows <= 2 * kThreads) {
    // up to two outputs per thread: one per step (the shortest chains)
    for (int i = tid; i < T * rows; i += kThreads) {
      const int t = i / rows, col = i - t * rows;
      double v = 0.0, u = 0.0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        v += (double)red[(w * BT + t) * RS + col];
        if constexpr (GLU) u += (double)red[(w * BT + t) * RS + BNP + col];
      }
      const size_t o = (size_t)t * N + n0 + col;
      if (!GLU && f32out) {
        reinterpret_cast<float*>(y)[o] = (float)v;  // binary32 sums (the gate and up of LinearSwiGLU)
        continue;
      }
      y[o] = finish(v, u, o, t, col);
    }
    return;
  }
  // more: four adjacent outputs of one token per step (16-byte partial
  // reads; columns rows .. 4 G4 - 1 of a row lie within its stride and
  // their sums are never used)
  const int G4 = (rows + 3) >> 2;
  for (int i = tid; i < T * G4; i += kThreads) {
    const int t = i / G4, c0 = 4 * (i - t * G4);
    const int nv = min(4, rows - c0);
    double v[4] = {0.0, 0.0, 0.0, 0.0}, u[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const f32x4_t p = *reinterpret_cast<const f32x4_t*>(red + (w * BT + t) * RS + c0);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] += (double)p[j];
      if constexpr (GLU) {
        const f32x4_t q = *reinterpret_cast<const f32x4_t*>(red + (w * BT + t) * RS + BNP + c0);
#pragma unroll
        for (int j = 0; j < 4; ++j) u[j] += (double)q[j];
      }
    }
    const size_t o = (size_t)t * N + n0 + c0;
    if (!GLU && f32out) {
      // binary32 sums (the gate and up of LinearSwiGLU)
      float* yf = reinterpret_cast<float*>(y) + o;
      if (nv == 4 && (reinterpret_cast<uintptr_t>(yf) & 15) == 0) {
        *reinterpret_cast<f32x4_t*>(yf) = f32x4_t{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (j < nv) yf[j] = (float)v[j];
      }
      continue;
    }
    uint16_t h[4] = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < nv) h[j] = finish(v[j], u[j], o + j, t, c0 + j);
    uint16_t* yo = y + o;
    if (nv == 4 && (reinterpret_cast<uintptr_t>(yo) & 7) == 0) {
      *reinterpret_cast<u32x2_t*>(yo) = u32x2_t{(uint32_t)h[0] | ((uint32_t)h[1] << 16),
                                                (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j < nv) yo[j] = h[j];
    }
  }
}

// Compile-time step numbers: nested_steps<0, M>(n, fn) runs fn(IC<0>),
// then fn(IC<1>) inside a branch taken when 1 < n, and so on up to M - 1,
// so that the code of step s is reached only through steps 0 .. s - 1.
template <int V>
struct IC {
  static constexpr int value = V;
};
template <int I, int M, class Fn>
__device__ __forceinline__ void nested_steps(int n, Fn& fn) {
  fn(IC<I>{});
  if constexpr (I + 1 < M) {
    if (I + 1 < n) nested_steps<I + 1, M>(n, fn);
  }
}

// A launch's second weight.  LinearPair (the kernels' GLU false, n > 0):
// workgroups from row block `first` on take its rows and write y (no
// residual).  LinearSwiGLU (GLU true): every workgroup takes the same rows
// of the gate (the first weight) and of this up weight.
struct Plane2 {
  const uint8_t* lo;
  const uint8_t* hi;
  const uint8_t* sc;
  uint16_t* y;
  int n;
  int first;
};

// ---------------------------------------------------------------------------
// Up to 16 tokens: the eight waves split the block's pairs of units; each
// pair's codes and activations go straight to registers, two register sets
// taking turns (the next pair's loads in flight during a pair's products).
// ---------------------------------------------------------------------------
template <int F, int CT, bool GLU>
__global__ void __launch_bounds__(kThreads, 1)
fmt_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ lo, const uint8_t* __restrict__ hi,
           const uint8_t* __restrict__ sc, uint16_t* __restrict__ y, const uint16_t* __restrict__ res, int f32out,
           int N, int K, int T, int BN, Plane2 p2) {
  using U = Unit<F>;
  constexpr int XH = Fmt<F>::XH, HB = Fmt<F>::HB;
  constexpr int NB = 2;  // pairs in flight (register sets)
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  // the quarter of each unit this lane multiplies: after the exchange of
  // the paired loads, quarter lq holds code bytes 8 xq .. 8 xq + 7 of a unit
  const int xq = Fmt<F>::PAIRED ? (((lq & 1) << 1) | (lq >> 1)) : lq;
  int bid = blockIdx.x;
  if (!GLU && p2.n > 0 && bid >= p2.first) {  // LinearPair: the second weight's row blocks
    lo = p2.lo;
    hi = p2.hi;
    sc = p2.sc;
    y = p2.y;
    N = p2.n;
    res = nullptr;
    bid -= p2.first;
  }
  const int n0 = bid * BN;
  const int rows = min(BN, N - n0);
  const int units = K / U::K;
  const int pairs = (units + 1) >> 1;
  const int pb = (int)(((int64_t)pairs * wave) / kWaves), pe = (int)(((int64_t)pairs * (wave + 1)) / kWaves);
  const int ts = units * U::SB;  // bytes of one row's scales
  // LDS: the partials of the final sum, then the scale table
  uint8_t* tab = lds + (size_t)kWaves * 16 * red_stride(red_cols(BN, GLU)) * 4;

  const rsrc_t rlo = make_rsrc(lo + (size_t)n0 * units * U::CB, (uint32_t)(rows * units * U::CB));
  const rsrc_t rlo2 = GLU ? make_rsrc(p2.lo + (size_t)n0 * units * U::CB, (uint32_t)(rows * units * U::CB)) : rlo;
  const rsrc_t rhi = make_rsrc(HB ? hi + (size_t)n0 * units * HB : lo, (uint32_t)(rows * units * HB));
  const rsrc_t rx = make_rsrc(x, (uint32_t)((size_t)T * K * 2));
  const rsrc_t rnull = make_rsrc(x, 0u);  // every access out of range
  uint32_t lo_off[CT], hi_off[CT];
  int tab_row[CT];
  lane_offsets<F, CT, GLU>(rows, units, ts, li, lq, lo_off, hi_off, tab_row);
  // Activations: lane (li, lq) multiplies pieces XH xq .. XH xq + XH - 1 of
  // token li in each unit.  From five tokens on lane l loads those of token
  // l / 4 and quarter l % 4, so that a quarter-wave reads four token rows
  // (sixteen rows of 16 bytes each take the address unit about three times
  // as long), and a lane exchange then hands every lane its own pieces; up
  // to four tokens a quarter-wave reads at most four rows anyway (tokens
  // past T repeat the last) and each lane loads its own pieces.
  const bool xchg = T > 4;
  const uint32_t x_off = xchg ? (uint32_t)(min(lane >> 2, T - 1) * K * 2 + (lane & 3) * 16 * XH)
                              : (uint32_t)(min(li, T - 1) * K * 2 + xq * 16 * XH);
  const int xsrc4 = (4 * li + xq) * 4;  // the lane holding this lane's pieces (byte address)

  struct Loads {
    PairCodes<F, CT> c;
    u32x4_t a[2][1][XH];
  };
  auto load = [&](int p, Loads& L) __device__ {
    const bool live = p < pe;
    load_codes<F, CT, GLU>(rlo, rlo2, rhi, rnull, lo_off, hi_off, p, live, L.c);
    const rsrc_t r = live ? rx : rnull;
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int p2 = 0; p2 < XH; ++p2)
        L.a[v][0][p2] = __builtin_amdgcn_raw_buffer_load_b128(r, x_off, (uint32_t)(((2 * p + v) * U::K + 8 * p2) * 2), 0);
  };

  const rsrc_t rsc = make_rsrc(U::SB ? sc + (size_t)n0 * ts : lo, (uint32_t)(rows * ts));
  const rsrc_t rsc2 = GLU ? make_rsrc(p2.sc + (size_t)n0 * ts, (uint32_t)(rows * ts)) : rsc;
  uint8_t* const tab2 = tab + rows * ts;  // GLU: the up weight's scales
  const WaveTable wt(rows, ts, 2 * pb, min(2 * pe, units), U::SB);
  const int hsh = (lane >> 5) << 4;  // Q5: the half of a high dword that belongs to this lane

  f32x4_t acc[CT][1];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) acc[ct][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // the products of pair p (its second unit is skipped past the row's end)
  auto pair_products = [&](int p, const Loads& L) __device__ {
    const bool second = 2 * p + 1 < units;
    u32x4_t A[2][1][XH];
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int h = 0; h < XH; ++h) A[v][0][h] = xchg ? lane_piece(L.a[v][0][h], xsrc4) : L.a[v][0][h];
    if constexpr (F == FMT_BF16) {
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        if (v == 1 && !second) break;
        u32x4_t cv[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) cv[ct] = L.c.c[ct][v];
        bf16_unit<CT, 1>(A[v], cv, acc);
      }
    } else {
      u32x2_t ca[CT], cb[CT];
      uint32_t ha[CT], hb[CT];
      split_pair<F, CT>(L.c, hsh, ca, cb, ha, hb);
      unit_products<F, CT, 1, false>(2 * p, A[0], ca, ha, tab, tab_row, xq, acc);
      if (second) unit_products<F, CT, 1, false>(2 * p + 1, A[1], cb, hb, tab, tab_row, xq, acc);
    }
  };

  // The wave's scales (first batch) in flight with the first two pairs'
  // loads.  (Batches past the first are copied before, on their own.)
  Loads b[NB];
  uint32_t so[8];
  uint16_t sv[8], sv2[8];
  if constexpr (U::SB > 0) {
    wt.copy_rest(rsc, tab, lane);
    if constexpr (GLU) wt.copy_rest(rsc2, tab2, lane);
    wt.offsets(0, lane, so);
    wt.load(rsc, so, sv);
    if constexpr (GLU) wt.load(rsc2, so, sv2);
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) load(pb + i, b[i]);
  if constexpr (U::SB > 0) {
    wt.store(tab, so, sv);
    if constexpr (GLU) wt.store(tab2, so, sv2);
  }
  // (a wave reads only the table entries it wrote itself: no barrier)
  wait_lgkm0();
  // (Every load is issued outside the branches, so the compiler's count of
  // the loads in flight stays exact.)
  for (int p = pb; p < pe; p += NB) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (i == 0 || p + i < pe) pair_products(p + i, b[i]);
      load(p + i + NB, b[i]);
    }
  }
  // (the partials area lies before the scale table: no wait for its readers)
  final_sum<F, CT, 1, GLU>(acc, lds, wave, li, lq, tid, x, lo, hi, sc, y, res, f32out, N, K, T, BN, n0, rows);
}

// ---------------------------------------------------------------------------
// 17 to 128 tokens: every wave takes all 16 TT tokens of the launch for its
// run of pairs, so each code operand is built once for all of them.  The
// activations go through a ring of NS unit slots per wave in LDS (direct
// copies in memory order, read back in operand order).  A wave loads the
// codes of a chunk of up to six pairs at once (four or two for Q5/Q6),
// right after the copies of the chunk's first NS units: a unit's copies
// complete in issue order with the codes, so the wait for a unit's
// activations has a fixed count and the codes have the chunk's first units
// to arrive.
// ---------------------------------------------------------------------------
template <int F, int TT>
struct TokShape {
  static constexpr int PPT = Unit<F>::K * 2 / 16;   // 16-byte pieces per token and unit
  static constexpr int TTK = 16 * TT;               // tokens per launch
  static constexpr int SLOT = TTK * PPT * 16;       // one unit's activations [token][piece]
  static constexpr int NS = SLOT * 4 <= kRingWave ? 4 : SLOT * 2 <= kRingWave ? 2 : 1;  // slots per wave
  static constexpr int NI = TTK * PPT / 64;         // direct-to-LDS loads per unit and lane
  static constexpr int RING = kWaves * NS * SLOT;   // all waves' rings
};
// code pairs held in registers at once (fewer with the high bits of Q5/Q6
// and beside the accumulators of eight token tiles)
template <int F, int CT, int TT>
constexpr int tok_pairs() {
  constexpr int m = (F == FMT_Q5 || F == FMT_Q6) ? (CT <= 2 ? 4 : 2) : (CT <= 2 ? 6 : 4);
  return TT >= 8 ? m - 2 : m;
}

template <int F, int CT, int TT, bool GLU>
__global__ void __launch_bounds__(kThreads, 1)
fmt_tok_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ lo, const uint8_t* __restrict__ hi,
               const uint8_t* __restrict__ sc, uint16_t* __restrict__ y, const uint16_t* __restrict__ res,
               int f32out, int N, int K, int T, int BN, int TS, Plane2 p2) {
  using U = Unit<F>;
  using S = TokShape<F, TT>;
  constexpr int XH = Fmt<F>::XH, HB = Fmt<F>::HB;
  constexpr int PPT = S::PPT, NS = S::NS, NI = S::NI, SLOT = S::SLOT;
  constexpr int MP = tok_pairs<F, CT, TT>();
  constexpr int LC = CT * Fmt<F>::LPT;  // code-plane loads per pair
  constexpr bool NAT = F == FMT_Q4;
  static_assert((2 * MP) % NS == 0, "a chunk of pairs keeps the ring's slot order");
  static_assert((NS - 1) * NI + MP * LC <= 63, "the load counter holds 63");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const int xq = Fmt<F>::PAIRED ? (((lq & 1) << 1) | (lq >> 1)) : lq;
  // Workgroup -> (row block, token range of 16 TT tokens).  With TS ranges
  // the TS workgroups of a row block have the same number mod 8, so they run
  // on one XCD (workgroups are dealt to the eight XCDs in turn) and its
  // codes come from HBM once.
  int rb = blockIdx.x, tr = 0;
  if (TS > 1) {
    const int g = blockIdx.x >> 3;
    tr = g % TS;
    rb = (g / TS) * 8 + (blockIdx.x & 7);
  }
  if (!GLU && p2.n > 0 && rb >= p2.first) {  // LinearPair: the second weight's row blocks
    lo = p2.lo;
    hi = p2.hi;
    sc = p2.sc;
    y = p2.y;
    N = p2.n;
    res = nullptr;
    rb -= p2.first;
  }
  const int n0 = rb * BN, t0 = tr * 16 * TT;
  if (n0 >= N || t0 >= T) return;  // (the grid's last row of eight)
  x += (size_t)t0 * K;
  if (res != nullptr) res += (size_t)t0 * N;
  y = f32out ? reinterpret_cast<uint16_t*>(reinterpret_cast<float*>(y) + (size_t)t0 * N) : y + (size_t)t0 * N;
  T = min(16 * TT, T - t0);
  const int rows = min(BN, N - n0);
  const int units = K / U::K;
  const int pairs = (units + 1) >> 1;
  const int pb = (int)(((int64_t)pairs * wave) / kWaves), pe = (int)(((int64_t)pairs * (wave + 1)) / kWaves);
  const int ue = min(2 * pe, units);  // past this wave's last unit
  const int ts = units * U::SB;
  // LDS: the rings, then the scale table; the final sum's partials reuse
  // the start once both are no longer read
  uint8_t* const ring = lds + (size_t)wave * NS * SLOT;
  uint8_t* tab = lds + S::RING;

  const rsrc_t rlo = make_rsrc(lo + (size_t)n0 * units * U::CB, (uint32_t)(rows * units * U::CB));
  const rsrc_t rlo2 = GLU ? make_rsrc(p2.lo + (size_t)n0 * units * U::CB, (uint32_t)(rows * units * U::CB)) : rlo;
  const rsrc_t rhi = make_rsrc(HB ? hi + (size_t)n0 * units * HB : lo, (uint32_t)(rows * units * HB));
  const rsrc_t rx = make_rsrc(x, (uint32_t)((size_t)T * K * 2));
  const rsrc_t rnull = make_rsrc(x, 0u);  // every access out of range
  uint32_t lo_off[CT], hi_off[CT];
  int tab_row[CT];
  lane_offsets<F, CT, GLU, true>(rows, units, ts, li, lq, lo_off, hi_off, tab_row);
  const int csrc4 = (4 * li + lq) * 4;  // the lane that loaded this lane's code pieces (byte address)

  // A slot holds one unit's activations, piece (tl, pc) of token tl at
  // position tl PPT + (pc ^ swz(tl)), swz(tl) = (tl / (16 / PPT)) % PPT: the
  // sixteen lanes of an operand read (16 consecutive tokens, one piece
  // each) then meet every 16-byte bank group of a 256-byte LDS row once.
  // Copy j of a unit moves positions 64 j .. 64 j + 63, lane l the one at
  // 64 j + l: 16 contiguous bytes of memory per lane, consecutive lanes on
  // consecutive pieces.  Tokens past T repeat the last one (their sums are
  // never stored).
  auto swz = [](int tl) { return (tl / (16 / PPT)) % PPT; };
  uint32_t xdma[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int q = j * 64 + lane;
    const int tl = q / PPT, pc = (q % PPT) ^ swz(tl);
    xdma[j] = (uint32_t)(min(tl, T - 1) * K * 2 + pc * 16);
  }
  // the unit's offset is the wave-uniform buffer offset; a unit past the
  // run reads through rnull (nothing lands but zeros)
  auto issue_x = [&](int u, int slot) __device__ {
    uint8_t* dst = ring + slot * SLOT;
    const rsrc_t r = u < ue ? rx : rnull;
#pragma unroll
    for (int j = 0; j < NI; ++j) dma16(r, xdma[j], (uint32_t)(u * U::K * 2), dst + j * 1024);
  };
  // unit operands: lane (li, lq) takes pieces XH xq .. XH xq + XH - 1 of
  // token 16 tt + li (swz(16 tt + li) = swz(li), so only the slot and the
  // token tile move the address, by constants)
  const uint8_t* xrd[XH];
#pragma unroll
  for (int h = 0; h < XH; ++h) xrd[h] = ring + (li * PPT + ((XH * xq + h) ^ swz(li))) * 16;
  auto read_x = [&](int slot, u32x4_t (&A)[TT][XH]) __device__ {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int h = 0; h < XH; ++h)
        A[tt][h] = *reinterpret_cast<const u32x4_t*>(xrd[h] + slot * SLOT + tt * (16 * PPT * 16));
  };

  const rsrc_t rsc = make_rsrc(U::SB ? sc + (size_t)n0 * ts : lo, (uint32_t)(rows * ts));
  const rsrc_t rsc2 = GLU ? make_rsrc(p2.sc + (size_t)n0 * ts, (uint32_t)(rows * ts)) : rsc;
  uint8_t* const tab2 = tab + rows * ts;  // GLU: the up weight's scales
  const WaveTable wt(rows, ts, 2 * pb, ue, U::SB);
  const int hsh = (lane >> 5) << 4;

  f32x4_t acc[CT][TT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[ct][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Prologue: the scales' first batch, the first NS units' activations, then
  // the first chunk's codes.
  PairCodes<F, CT> cc[MP];
  int pchunk = pb;  // the chunk's first pair
  uint32_t so[8];
  uint16_t sv[8], sv2[8];
  if constexpr (U::SB > 0) {
    wt.copy_rest(rsc, tab, lane);
    if constexpr (GLU) wt.copy_rest(rsc2, tab2, lane);
    wt.offsets(0, lane, so);
    wt.load(rsc, so, sv);
    if constexpr (GLU) wt.load(rsc2, so, sv2);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < NS; ++s) issue_x(2 * pb + s, s);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < MP; ++i)
    load_codes<F, CT, GLU>(rlo, rlo2, rhi, rnull, lo_off, hi_off, pb + i, pb + i < pe, cc[i]);
  if constexpr (U::SB > 0) {
    wt.store(tab, so, sv);
    if constexpr (GLU) wt.store(tab2, so, sv2);
  }
  // (a wave reads only the table entries it wrote itself: no barrier; the
  // loads stay in flight)
  wait_lgkm0();

  // Chunks of MP pairs.  Unit j of a chunk reads slot j % NS.  Before it,
  // the loads issued after its activations are: for j < NS the later
  // slots' copies and the chunk's codes (issued after the copies of the
  // chunk's first NS units), else the NS - 1 copies issued after it.  The
  // pairs of a chunk run nested (pair i + 1 inside pair i's branch), so
  // pairs past the run issue nothing and every path to a pair has issued
  // the same loads before it: these counts and the compiler's own stay
  // exact.  The next chunk's codes are loaded only when it exists.
  auto pair_step = [&](auto ic) __device__ {
    constexpr int i = decltype(ic)::value;
    const int p0 = pchunk;
    {
      u32x2_t ca[CT], cb[CT];
      uint32_t ha[CT], hb[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int v = 0; v < Fmt<F>::NC; ++v) cc[i].c[ct][v] = lane_piece(cc[i].c[ct][v], csrc4);
      if constexpr (Fmt<F>::PAIRED) split_pair<F, CT>(cc[i], hsh, ca, cb, ha, hb);
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const int j = 2 * i + v, u = 2 * p0 + j;
        u32x4_t A[TT][XH];
        __builtin_amdgcn_sched_barrier(0);
        if (j < NS) wait_vm<(NS - 1) * NI + MP * LC>();
        else wait_vm<(NS - 1) * NI>();
        read_x(j % NS, A);
        wait_lgkm0();
        __builtin_amdgcn_sched_barrier(0);
        issue_x(u + NS, j % NS);  // into the slot just read
        __builtin_amdgcn_sched_barrier(0);
        if (u < ue) {
          if constexpr (F == FMT_BF16) {
            u32x4_t cv[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) cv[ct] = cc[i].c[ct][v];
            bf16_unit<CT, TT>(A, cv, acc);
          } else {
            unit_products<F, CT, TT, NAT>(u, A, v ? cb : ca, v ? hb : ha, tab, tab_row, xq, acc);
          }
        }
      }
    }
  };
  for (pchunk = pb; pchunk < pe; pchunk += MP) {
    nested_steps<0, MP>(pe - pchunk, pair_step);
    // the next chunk's codes, after the copies of its first NS units (as in
    // the prologue; pairs past the run read nothing)
    __builtin_amdgcn_sched_barrier(0);
    if (pchunk + MP < pe) {
#pragma unroll
      for (int i = 0; i < MP; ++i)
        load_codes<F, CT, GLU>(rlo, rlo2, rhi, rnull, lo_off, hi_off, pchunk + MP + i, pchunk + MP + i < pe, cc[i]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_vm<0>();  // every copy into the rings has landed before the space is reused
  __syncthreads();
  final_sum<F, CT, TT, GLU>(acc, lds, wave, li, lq, tid, x, lo, hi, sc, y, res, f32out, N, K, T, BN, n0, rows);
}

// ---------------------------------------------------------------------------
// BF16_CTRL at one token (K <= 8192): the dense control needs no operand
// work, so it runs as a plain streaming GEMV.  Each wave takes whole rows,
// two at a time (grid-stride over the rows); lane l multiplies pieces
// l, l + 64, ... (8 weights, 16 bytes each) with the same pieces of X, which
// it loads once.  v_dot2_f32_bf16 chains per lane (the bf16 products are
// exact in FP32), the 64 lane partials summed in binary64, one rounding; a
// non-finite result is formed again exactly.
// ---------------------------------------------------------------------------
constexpr int kGemvWaves = 4;
template <int CH>
__global__ void __launch_bounds__(64 * kGemvWaves)
bf16_gemv_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ w, uint16_t* __restrict__ y,
                 const uint16_t* __restrict__ res, int f32out, int N, int K) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kGemvWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = gridDim.x * kGemvWaves;
  const uint32_t row_bytes = (uint32_t)K * 2;
  // pieces past the row read through the resource's end: zeros, no access
  const rsrc_t rx = make_rsrc(x, row_bytes);
  u32x4_t xp[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) xp[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)((lane + 64 * i) * 16), 0, 0);
  // (each dword goes through a scalar: a bit cast of a vector element takes
  // the vector's first bytes)
  auto dot2 = [](uint32_t wv, uint32_t xv, float c) __device__ {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wv), __builtin_bit_cast(bf16x2_t, xv), c, false);
  };
  auto dot = [&](const u32x4_t (&a)[CH]) __device__ {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const uint32_t w0 = a[i].x, w1 = a[i].y, w2 = a[i].z, w3 = a[i].w;
      const uint32_t x0 = xp[i].x, x1 = xp[i].y, x2 = xp[i].z, x3 = xp[i].w;
      s = dot2(w0, x0, s);
      s = dot2(w1, x1, s);
      s = dot2(w2, x2, s);
      s = dot2(w3, x3, s);
    }
    return sum64_lanes((double)s);
  };
  auto finish = [&](int n, double v) __device__ {
    if (f32out) {
      reinterpret_cast<float*>(y)[n] = (float)v;
      return;
    }
    if (res != nullptr) v += (double)bf16_bits_to_f32(res[n]);  // LinearAdd
    uint16_t h = f32_to_bf16_rne((float)v);
    if ((h & 0x7F80u) == 0x7F80u) h = exact_output<FMT_BF16>(x, w, nullptr, nullptr, res, N, K, n, 0);  // rare
    y[n] = h;
  };
  for (int r = gw; r < N; r += 2 * nw) {
    const int r2 = min(r + nw, N - 1);  // (past the rows: the last row again, not stored)
    const rsrc_t ra = make_rsrc(w + (size_t)r * row_bytes, row_bytes);
    const rsrc_t rb = make_rsrc(w + (size_t)r2 * row_bytes, row_bytes);
    u32x4_t a[CH], b[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) a[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, (uint32_t)((lane + 64 * i) * 16), 0, 2);
#pragma unroll
    for (int i = 0; i < CH; ++i) b[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, (uint32_t)((lane + 64 * i) * 16), 0, 2);
    // every load of both rows in flight before the first product (left to
    // itself the scheduler moves each load down to its use, one or two
    // loads in flight at a time)
    __builtin_amdgcn_sched_barrier(0);
    const double va = dot(a), vb = dot(b);
    if (lane == 0) {
      finish(r, va);
      if (r + nw < N) finish(r + nw, vb);
    }
  }
}

// ---------------------------------------------------------------------------
// Q5, Q6, W8 and NVFP4 at one token (K <= 8192): the same streaming GEMV.
// A piece is 16 bytes of the code plane (32 weights; W8: 16) with its high
// bits and scale; lane l takes pieces l, l + 64, ... of each of the wave's
// two rows.  The exact bf16 operands of the matrix-core kernels go through
// v_dot2_f32_bf16 chains (Q5/Q6 in pair order, with the activations
// permuted once per wave); the products of the all-offset codes run through
// the same chain on the same activations (once per wave), so P - C is
// exactly 0 for a piece of offset codes; the scale is applied in FP32 per
// piece; binary64 lane sum, one rounding, exact repair when non-finite.
// ---------------------------------------------------------------------------
template <int F>
struct GemvPiece {
  static constexpr int KW = F == FMT_W8 ? 16 : 32;   // weights per piece
  static constexpr int XV = KW / 8;                  // 16-byte activation vectors per piece
  static constexpr int HB = F == FMT_Q5 ? 4 : F == FMT_Q6 ? 8 : 0;  // high-plane bytes per piece
};
__device__ __forceinline__ float dot2_bf(uint32_t w, uint32_t x, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, x), c, false);
}
// The sum over a piece (code dwords c, high bits hbits, NVFP4 scales s0 and
// s1 of its two sixteens) of operand . activation, in one fixed chain order
// for the code operands and the constant ones alike
template <int F>
__device__ __forceinline__ float piece_chain(u32x4_t c, uint64_t hbits, float s0, float s1,
                                             const u32x4_t (&xa)[GemvPiece<F>::XV], bool constant) {
  float d = 0.0f;
  if constexpr (F == FMT_Q5 || F == FMT_Q6) {
    constexpr uint32_t kc = F == FMT_Q5 ? 0x43104310u : 0x43204320u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // code dword j: weights 8 j .. 8 j + 7 of the piece
      u32x4_t b = u32x4_t{kc, kc, kc, kc};
      if (!constant) {
        const uint32_t cw = c[j];
        b = F == FMT_Q5 ? __builtin_bit_cast(u32x4_t, q5_operand(cw, (uint32_t)(hbits >> (8 * j)) & 0xFFu))
                        : __builtin_bit_cast(u32x4_t, q6_operand(cw, (uint32_t)(hbits >> (16 * j)) & 0xFFFFu));
      }
      const uint32_t b0 = b.x, b1 = b.y, b2 = b.z, b3 = b.w;
      const uint32_t x0 = xa[j].x, x1 = xa[j].y, x2 = xa[j].z, x3 = xa[j].w;
      d = dot2_bf(b0, x0, d);
      d = dot2_bf(b1, x1, d);
      d = dot2_bf(b2, x2, d);
      d = dot2_bf(b3, x3, d);
    }
  } else if constexpr (F == FMT_W8) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // weights 8 h .. 8 h + 7 of the piece
      u32x4_t lo4, hi4;
      if (constant) {
        lo4 = u32x4_t{0x43004300u, 0x43004300u, 0x43004300u, 0x43004300u};
        hi4 = u32x4_t{0x43C043C0u, 0x43C043C0u, 0x43C043C0u, 0x43C043C0u};
      } else {
        bf16x8_t lo8, hi8;
        const uint32_t c0 = c[2 * h], c1 = c[2 * h + 1];
        w8_operands(c0, c1, lo8, hi8);
        lo4 = __builtin_bit_cast(u32x4_t, lo8);
        hi4 = __builtin_bit_cast(u32x4_t, hi8);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t l = lo4[i], hh = hi4[i], xx = xa[h][i];
        d = dot2_bf(l, xx, d);
        d = dot2_bf(hh, xx, d);
      }
    }
  } else {  // NVFP4: exact weights, the E4M3 scale of each 16 inside
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t cw = c[j];
      const u32x4_t b = __builtin_bit_cast(u32x4_t, nvfp4_operand(cw, j < 2 ? s0 : s1));
      const uint32_t b0 = b.x, b1 = b.y, b2 = b.z, b3 = b.w;
      const uint32_t x0 = xa[j].x, x1 = xa[j].y, x2 = xa[j].z, x3 = xa[j].w;
      d = dot2_bf(b0, x0, d);
      d = dot2_bf(b1, x1, d);
      d = dot2_bf(b2, x2, d);
      d = dot2_bf(b3, x3, d);
    }
  }
  return d;
}

template <int F, int CH>
__global__ void __launch_bounds__(64 * kGemvWaves)
fmt_gemv_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ lo, const uint8_t* __restrict__ hi,
                const uint8_t* __restrict__ sc, uint16_t* __restrict__ y, const uint16_t* __restrict__ res,
                int f32out, int N, int K) {
  using P = GemvPiece<F>;
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kGemvWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = gridDim.x * kGemvWaves;
  const uint32_t row_lo = F == FMT_W8 ? (uint32_t)K : (uint32_t)K / 2;
  const uint32_t row_hi = (uint32_t)(K / P::KW) * P::HB;
  const uint32_t row_sc = F == FMT_NVFP4 ? (uint32_t)K / 16 : F == FMT_W8 ? (uint32_t)K / 16 : (uint32_t)K / 32;
  // the activations of this lane's pieces (permuted to pair order for
  // Q5/Q6), and their correction chains; pieces past the row read zeros
  const rsrc_t rx = make_rsrc(x, (uint32_t)K * 2);
  u32x4_t xa[CH][P::XV];
  float corr[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i)
#pragma unroll
    for (int v = 0; v < P::XV; ++v)
      xa[i][v] = __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)(((lane + 64 * i) * P::KW + 8 * v) * 2), 0, 0);
  struct Row {
    u32x4_t c[CH];
    uint64_t h[CH];
    uint32_t sv[CH];
  };
  auto load_row = [&](int r, Row& w) __device__ {
    const rsrc_t rl = make_rsrc(lo + (size_t)r * row_lo, row_lo);
    const rsrc_t rh = make_rsrc(P::HB ? hi + (size_t)r * row_hi : lo, row_hi);
    const rsrc_t rs = make_rsrc(sc + (size_t)r * row_sc, row_sc);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const uint32_t p = (uint32_t)(lane + 64 * i);
      w.c[i] = __builtin_amdgcn_raw_buffer_load_b128(rl, p * 16, 0, 2);
      if constexpr (F == FMT_Q5) {
        w.h[i] = __builtin_amdgcn_raw_buffer_load_b32(rh, p * 4, 0, 0);
      } else if constexpr (F == FMT_Q6) {
        const u32x2_t hv = __builtin_amdgcn_raw_buffer_load_b64(rh, p * 8, 0, 0);
        w.h[i] = (uint64_t)hv.x | ((uint64_t)hv.y << 32);
      } else {
        w.h[i] = 0;
      }
      // the piece's scale bytes: Q5/Q6 and W8 one fp16 per two pieces, NVFP4 two E4M3 bytes per piece
      w.sv[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, F == FMT_NVFP4 ? p * 2 : (p >> 1) * 2, 0, 0);
    }
  };
  auto row_sum = [&](const Row& w) __device__ {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if constexpr (F == FMT_NVFP4) {
        acc += piece_chain<F>(w.c[i], 0, e4m3_to_f32(w.sv[i] & 0xFFu), e4m3_to_f32(w.sv[i] >> 8), xa[i], false);
      } else {
        const float d = piece_chain<F>(w.c[i], w.h[i], 0.f, 0.f, xa[i], false);
        acc = __builtin_fmaf(f16_bits_to_f32(w.sv[i]), d - corr[i], acc);
      }
    }
    return sum64_lanes((double)acc);
  };
  auto finish = [&](int n, double v) __device__ {
    if (f32out) {
      reinterpret_cast<float*>(y)[n] = (float)v;
      return;
    }
    if (res != nullptr) v += (double)bf16_bits_to_f32(res[n]);  // LinearAdd
    uint16_t hv = f32_to_bf16_rne((float)v);
    if ((hv & 0x7F80u) == 0x7F80u) hv = exact_output<F>(x, lo, hi, sc, res, N, K, n, 0);  // rare
    y[n] = hv;
  };
  // The grid gives every wave its two rows gw and gw + nw (2 nw >= N).  All
  // their loads go out before anything waits (left to itself the scheduler
  // moves each load down to its use); the activations' permutation and
  // correction chains run while the rows are in flight.
  const int r = gw;
  if (r >= N) return;
  Row wa, wb;
  load_row(r, wa);
  load_row(min(r + nw, N - 1), wb);  // (past the rows: the last row again, not stored)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    if constexpr (F == FMT_Q5 || F == FMT_Q6) {
#pragma unroll
      for (int v = 0; v < P::XV; ++v) xa[i][v] = __builtin_bit_cast(u32x4_t, pair_order(xa[i][v]));
    }
    corr[i] = F == FMT_NVFP4 ? 0.0f : piece_chain<F>(u32x4_t{0u, 0u, 0u, 0u}, 0, 0.f, 0.f, xa[i], true);
  }
  const double va = row_sum(wa), vb = row_sum(wb);
  if (lane == 0) {
    finish(r, va);
    if (r + nw < N) finish(r + nw, vb);
  }
}

template <int F, int CH>
hipError_t launch_fmt_gemv_ch(const FmtArgs& a, hipStream_t s) {
  const int64_t blocks = (a.n + 2 * kGemvWaves - 1) / (2 * kGemvWaves);  // two rows per wave
  fmt_gemv_kernel<F, CH><<<dim3((unsigned)blocks), dim3(64 * kGemvWaves), 0, s>>>(
      static_cast<const uint16_t*>(a.x), static_cast<const uint8_t*>(a.lo), static_cast<const uint8_t*>(a.hi),
      static_cast<const uint8_t*>(a.sc), static_cast<uint16_t*>(a.y), static_cast<const uint16_t*>(a.res),
      a.f32 ? 1 : 0, (int)a.n, (int)a.k);
  return hipGetLastError();
}
template <int F>
hipError_t launch_fmt_gemv(const FmtArgs& a, hipStream_t s) {
  const int64_t need = (a.k / GemvPiece<F>::KW + 63) / 64;  // pieces per lane
  if (need <= 1) return launch_fmt_gemv_ch<F, 1>(a, s);
  if (need <= 2) return launch_fmt_gemv_ch<F, 2>(a, s);
  if (need <= 3) return launch_fmt_gemv_ch<F, 3>(a, s);
  if (need <= 4) return launch_fmt_gemv_ch<F, 4>(a, s);
  if constexpr (F == FMT_W8) {  // (W8 alone has more than 4: 16 weights a piece)
    if (need <= 5) return launch_fmt_gemv_ch<F, 5>(a, s);
    if (need <= 6) return launch_fmt_gemv_ch<F, 6>(a, s);
    return launch_fmt_gemv_ch<F, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int CH>
hipError_t launch_bf16_gemv_ch(const FmtArgs& a, hipStream_t s) {
  const int64_t blocks = (a.n + 2 * kGemvWaves - 1) / (2 * kGemvWaves);  // two rows per wave
  bf16_gemv_kernel<CH><<<dim3((unsigned)blocks), dim3(64 * kGemvWaves), 0, s>>>(
      static_cast<const uint16_t*>(a.x), static_cast<const uint8_t*>(a.lo), static_cast<uint16_t*>(a.y),
      static_cast<const uint16_t*>(a.res), a.f32 ? 1 : 0, (int)a.n, (int)a.k);
  return hipGetLastError();
}
// pieces per lane: the smallest of these that covers K / 512
hipError_t launch_bf16_gemv(const FmtArgs& a, hipStream_t s) {
  const int64_t need = (a.k / 8 + 63) / 64;
  if (need <= 2) return launch_bf16_gemv_ch<2>(a, s);
  if (need <= 4) return launch_bf16_gemv_ch<4>(a, s);
  if (need <= 6) return launch_bf16_gemv_ch<6>(a, s);
  if (need <= 8) return launch_bf16_gemv_ch<8>(a, s);
  if (need <= 10) return launch_bf16_gemv_ch<10>(a, s);
  if (need <= 12) return launch_bf16_gemv_ch<12>(a, s);
  return launch_bf16_gemv_ch<16>(a, s);
}

// LDS of a launch: the few-token kernel's partials and scale table, or the
// many-token kernel's rings and table (the partials reuse them).  w: the
// weights whose rows a workgroup takes (2 for the gated pair).
size_t fmt_lds(int ppt, int tt, int64_t bn, int64_t ts, int w) {
  const int64_t table = (w * bn * ts + 15) / 16 * 16;
  const int64_t red = (int64_t)kWaves * 16 * tt * red_stride(red_cols((int)bn, w == 2)) * 4;
  if (tt == 1) return (size_t)(red + table);
  const int64_t slot = 16 * tt * ppt * 16;
  const int64_t ns = slot * 4 <= kRingWave ? 4 : slot * 2 <= kRingWave ? 2 : 1;
  const int64_t ring = kWaves * ns * slot;
  return (size_t)(ring + table > red ? ring + table : red);
}

// token tiles per many-token launch: 2, 3, 4, 6 or 8 (at most 4 with 3 or 4
// column tiles, for the registers)
int tok_tiles(int64_t t, int ct) {
  const int cap = ct <= 2 ? 8 : 4;
  const int need = (int)((t + 15) / 16);
  static const int kTiles[] = {2, 3, 4, 6, 8};
  for (int v : kTiles)
    if (v >= need && v <= cap) return v;
  return cap;
}

// Column tiles of a workgroup of bn rows (per weight for the gated pair)
int fmt_col_tiles(int64_t bn, bool glu) { return (int)((glu ? 2 : 1) * ((bn + 15) / 16)); }

// One launch's shape on 17 or more tokens: row blocks of bn rows (ct column
// tiles), ts token ranges of 16 tt tokens each.  Above 64 tokens (when the
// rows allow) a row block twice as tall serves half the tokens: every
// workgroup still does the same work, but the activation bytes it copies
// (its tokens' whole rows) halve (6144 x 5120: T = 65..128 24.4-30.2 us
// against 24.8-32.9); below that the taller block's extra code loads cost
// more than the copies saved (T = 33..64 21-22 against 17-20.5 us).  The
// rows of both weights count: a pair's second weight adds row blocks from
// `first` on.  The gated pair's workgroups take bn rows of each weight and
// keep one token range (3072 x 5120 each: T = 72 24.3 against 26.8 us,
// T = 100 29.8 / 30.9, T = 128 32.0 / 31.5: its taller block has four
// column tiles for 2 x 24 rows).
struct TokLaunch {
  int64_t bn;
  int ct, ts, tt;
  int64_t first;  // row blocks of the first weight
  int64_t grid;
};
TokLaunch tok_launch(const FmtArgs& a, int64_t t, int64_t bn1, int64_t ts_bytes, int64_t table_cap) {
  const int64_t rows = a.glu ? 2 * a.n : a.n + a.n2;
  TokLaunch L;
  L.ts = 1;
  L.bn = bn1;
  if (!a.glu && t > 64 && (rows + 255) / 256 <= 32) {
    const int64_t bn2 = (2 * rows + 255) / 256;
    if (bn2 * ts_bytes <= table_cap) {
      L.ts = 2;
      L.bn = bn2;
    }
  }
  L.ct = fmt_col_tiles(L.bn, a.glu);
  L.tt = tok_tiles((t + L.ts - 1) / L.ts, L.ct);
  L.first = (a.n + L.bn - 1) / L.bn;
  const int64_t nrb = a.glu ? L.first : L.first + (a.n2 + L.bn - 1) / L.bn;
  L.grid = L.ts == 1 ? nrb : (nrb + 7) / 8 * 8 * L.ts;
  return L;
}

// One launch's pointers: the token range's activations, outputs, residual
// and second weight
struct Chunk {
  const uint16_t* x;
  uint16_t* y;
  const uint16_t* res;
  Plane2 p2;
  int t;
};

template <int F, int CT, int TT, bool GLU>
hipError_t launch_tok(const FmtArgs& a, const TokLaunch& L, const Chunk& c, hipStream_t s) {
  auto kern = fmt_tok_kernel<F, CT, TT, GLU>;
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(kern));
  if (e != hipSuccess) return e;
  const size_t lds = fmt_lds(TokShape<F, TT>::PPT, TT, L.bn, (a.k / Unit<F>::K) * Unit<F>::SB, GLU ? 2 : 1);
  Plane2 p2 = c.p2;
  p2.first = (int)L.first;
  kern<<<dim3((unsigned)L.grid), dim3(kThreads), lds, s>>>(
      c.x, static_cast<const uint8_t*>(a.lo), static_cast<const uint8_t*>(a.hi), static_cast<const uint8_t*>(a.sc),
      c.y, c.res, a.f32 ? 1 : 0, (int)a.n, (int)a.k, c.t, (int)L.bn, L.ts, p2);
  return hipGetLastError();
}

template <int F, int CT, bool GLU>
hipError_t launch_tok_ct(const FmtArgs& a, const TokLaunch& L, const Chunk& c, hipStream_t s) {
  switch (L.tt) {
    case 2: return launch_tok<F, CT, 2, GLU>(a, L, c, s);
    case 3: return launch_tok<F, CT, 3, GLU>(a, L, c, s);
    case 4: return launch_tok<F, CT, 4, GLU>(a, L, c, s);
    default:
      if constexpr (CT <= 2) {
        if (L.tt == 6) return launch_tok<F, CT, 6, GLU>(a, L, c, s);
        return launch_tok<F, CT, 8, GLU>(a, L, c, s);
      }
      return hipErrorInvalidValue;
  }
}

template <int F, int CT, bool GLU>
hipError_t launch_few(const FmtArgs& a, const FmtPlan& p, const Chunk& c, hipStream_t s) {
  auto kern = fmt_kernel<F, CT, GLU>;
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(kern));
  if (e != hipSuccess) return e;
  const size_t lds = fmt_lds(0, 1, p.bn, (a.k / Unit<F>::K) * Unit<F>::SB, GLU ? 2 : 1);
  Plane2 p2 = c.p2;
  p2.first = (int)((a.n + p.bn - 1) / p.bn);
  kern<<<dim3((unsigned)p.blocks), dim3(kThreads), lds, s>>>(
      c.x, static_cast<const uint8_t*>(a.lo), static_cast<const uint8_t*>(a.hi), static_cast<const uint8_t*>(a.sc),
      c.y, c.res, a.f32 ? 1 : 0, (int)a.n, (int)a.k, c.t, p.bn, p2);
  return hipGetLastError();
}

template <int F, bool GLU>
hipError_t launch_chunk(const FmtArgs& a, const FmtPlan& p, const Chunk& c, int64_t tsb, int64_t table_cap,
                        hipStream_t s) {
  if (c.t <= 16) {
    if constexpr (GLU) {  // 2 or 4 column tiles: 16 or 32 rows of each weight
      return p.ct == 2 ? launch_few<F, 2, true>(a, p, c, s) : launch_few<F, 4, true>(a, p, c, s);
    } else {
      switch (p.ct) {
        case 1: return launch_few<F, 1, false>(a, p, c, s);
        case 2: return launch_few<F, 2, false>(a, p, c, s);
        case 3: return launch_few<F, 3, false>(a, p, c, s);
        default: return launch_few<F, 4, false>(a, p, c, s);
      }
    }
  }
  const TokLaunch L = tok_launch(a, c.t, p.bn, tsb, table_cap);
  if constexpr (GLU) {
    return L.ct == 2 ? launch_tok_ct<F, 2, true>(a, L, c, s) : launch_tok_ct<F, 4, true>(a, L, c, s);
  } else {
    switch (L.ct) {
      case 1: return launch_tok_ct<F, 1, false>(a, L, c, s);
      case 2: return launch_tok_ct<F, 2, false>(a, L, c, s);
      case 3: return launch_tok_ct<F, 3, false>(a, L, c, s);
      default: return launch_tok_ct<F, 4, false>(a, L, c, s);
    }
  }
}

template <int F>
hipError_t launch_fmt_t(const FmtArgs& a, const FmtPlan& p, hipStream_t s) {
  // one weight pass per launch of up to 128 tokens (64 with 3 or 4 column
  // tiles and one token range)
  const size_t osz = a.f32 ? 4 : 2;
  const int64_t tsb = (a.k / Unit<F>::K) * Unit<F>::SB;
  const int64_t table_cap = kLdsBytes - (int64_t)kWaves * kRingWave;
  int64_t per = 128;
  if (a.t > 16) {
    const TokLaunch L = tok_launch(a, a.t > 128 ? 128 : a.t, p.bn, tsb, table_cap);
    per = (int64_t)L.ts * 16 * (L.ct <= 2 ? 8 : 4);
  }
  for (int64_t t0 = 0; t0 < a.t; t0 += per) {
    Chunk c;
    c.t = (int)(a.t - t0 < per ? a.t - t0 : per);
    c.x = static_cast<const uint16_t*>(a.x) + t0 * a.k;
    c.y = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(a.y) + (size_t)t0 * a.n * osz);
    c.res = a.res ? static_cast<const uint16_t*>(a.res) + t0 * a.n : nullptr;
    c.p2 = Plane2{static_cast<const uint8_t*>(a.lo2), static_cast<const uint8_t*>(a.hi2),
                  static_cast<const uint8_t*>(a.sc2),
                  a.y2 && !a.glu ? static_cast<uint16_t*>(a.y2) + t0 * a.n2 : nullptr, (int)a.n2, 0};
    hipError_t e;
    if constexpr (F == FMT_Q4) {
      e = a.glu ? launch_chunk<F, true>(a, p, c, tsb, table_cap, s) : launch_chunk<F, false>(a, p, c, tsb, table_cap, s);
    } else {
      e = launch_chunk<F, false>(a, p, c, tsb, table_cap, s);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

bool fmt_plan(int fmt, int64_t n, int64_t k, int64_t t, FmtPlan* p, bool glu) {
  if (fmt < FMT_Q4 || fmt > FMT_BF16 || n < 1 || t < 1 || k < 64 || (k % 64) != 0) return false;
  if (glu && fmt != FMT_Q4) return false;
  // per-row offsets are 64-bit; the kernel's int arithmetic needs N, K, T below 2^31
  if (n >= (int64_t(1) << 31) || k >= (int64_t(1) << 30) || t >= (int64_t(1) << 31)) return false;
  // bytes of one row's scales in the LDS table
  const int64_t ts = fmt == FMT_BF16 ? 0 : fmt == FMT_W8 || fmt == FMT_NVFP4 ? k / 16 : k / 32;
  // launches of more than 16 tokens keep the waves' activation rings in LDS
  // (at most kRingWave bytes per wave)
  const int64_t ring = t > 16 ? (int64_t)kWaves * kRingWave : 0;
  const int64_t table_cap = ring + kTableBytes <= kLdsBytes ? kTableBytes : kLdsBytes - ring;
  const int w = glu ? 2 : 1;
  int64_t bn = (n + 255) / 256;  // about one workgroup per CU (the gated pair: 2 bn rows per workgroup)
  if (bn > 64 / w) bn = 64 / w;  // at most four 16-row column tiles per wave
  if (ts > 0 && w * bn * ts > table_cap) bn = table_cap / (w * ts);
  if (bn < 1) return false;
  const int ct = fmt_col_tiles(bn, glu);
  p->bn = (int)bn;
  p->ct = ct;
  p->blocks = (int)((n + bn - 1) / bn);
  // the largest launch's LDS (the partials of 16 tokens per tile)
  const int ppt = (fmt == FMT_W8 || fmt == FMT_BF16) ? 4 : 8;
  const int tt = t <= 16 ? 1 : tok_tiles(t > 128 ? 128 : t, ct);
  p->lds_bytes = fmt_lds(ppt, tt, bn, ts, w);
  return p->lds_bytes <= (size_t)kLdsBytes;
}

hipError_t launch_fmt(const FmtArgs& a, hipStream_t stream) {
  FmtPlan p;
  const bool two = !a.glu && a.n2 > 0;
  if (!fmt_plan(a.fmt, two ? a.n + a.n2 : a.n, a.k, a.t, &p, a.glu)) return hipErrorInvalidValue;
  if (two) p.blocks = (int)((a.n + p.bn - 1) / p.bn + (a.n2 + p.bn - 1) / p.bn);
  if (a.glu && a.fmt != FMT_Q4) return hipErrorInvalidValue;
  if (a.t == 1 && !two && a.k <= 8192) {  // one token: the streaming GEMVs
    switch (a.fmt) {
      case FMT_BF16: return launch_bf16_gemv(a, stream);
      case FMT_Q5: return launch_fmt_gemv<FMT_Q5>(a, stream);
      case FMT_Q6: return launch_fmt_gemv<FMT_Q6>(a, stream);
      case FMT_W8: return launch_fmt_gemv<FMT_W8>(a, stream);
      case FMT_NVFP4: return launch_fmt_gemv<FMT_NVFP4>(a, stream);
      default: break;
    }
  }
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
