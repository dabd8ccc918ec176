// q4lin_decode.hip -- the single-token route (T = 1): vector-ALU dot products,
// one weight stream per CU.
//
// The pages' prior art for T = 1 is a dedicated single-token GEMV
// ("q4-linear.md", notes under the result table); this is an MI355X design of
// that step.
//
// Work mapping.  A workgroup of eight waves owns BN consecutive rows (about
// N / (256 c) with c workgroups per CU) and the whole of K; wave w owns the
// w-th eighth of the 64-groups.  Inside a wave the slice of every row is cut
// into S slots of PL consecutive 16-byte pieces; lane l serves slot l % S of
// rows l / S, l / S + R, ... (R = 64 / S row groups).  So a lane keeps one
// fixed piece of the activations in registers for all its rows, each load
// instruction reads R rows x 16 PL S contiguous bytes, and every load of a
// lane (activations, then its scales, then its codes row by row) is issued
// before the first wait; each row is then processed as soon as its own codes
// have arrived.
//
// Arithmetic (as in the pages' "decode, FP32 accumulate" reading of the op):
//   * The bf16 activations are used as they are, permuted into the pair
//     order (k0,k4) (k1,k5) (k2,k6) (k3,k7) of a code dword's nibbles.
//   * A code pair becomes the exact bf16 pair (128 + q, 128 + q') with one
//     (a & m) | c (bf16 has unit spacing on [128, 256)); v_dot2_f32_bf16 sums
//     (128 + q) x (products exact in FP32).  The offset enters as
//     sum (q - 8) x = sum (128 + q) x - sum 136 x, the second sum from the
//     very same dot chain run on an all-8 code dword, so a piece of
//     eight-codes contributes exactly 0.  Each piece's difference is scaled
//     by its group's scale in FP32.
//   * Activations near the bf16 maximum can overflow those FP32 sums; a wave
//     that sees a non-finite partial redoes its rows on float16 copies of
//     the activations scaled by 2^-e (e from the slice's largest magnitude,
//     every value within 2^34 of it exact; odd k further /16, cancelled by
//     reading 16 q 2^-24 subnormals from the codes with one AND), and its
//     partials carry 2^-(e + 24).
//   * The eight waves' partials are combined in binary64 and rounded to bf16
//     once.
#include "q4lin_device.h"
#include "q4lin_kernels.h"

namespace q4lin {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
template <int MAXR>
constexpr int kRegion = 64 * MAXR * 4 + 16;  // bytes of one wave's LDS scratch region

// s_waitcnt immediate for gfx9: vmcnt in bits 3:0 and 15:14, expcnt 6:4 (7 =
// no wait), lgkmcnt 11:8 (15 = no wait).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }

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

// 8 bf16 values -> float16 pairs (k0,k4) (k1,k5) (k2,k6) (k3,k7), times 2^-e,
// odd k times 2^-(e+4).
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

// 8 bf16 values (k0..k7 in memory order) -> the pairs (k0,k4) (k1,k5)
// (k2,k6) (k3,k7), the order in which a code dword's nibbles pair up below
__device__ __forceinline__ u32x4_t bf16_pairs(u32x4_t v) {
  return u32x4_t{__builtin_amdgcn_perm(v.z, v.x, 0x05040100u), __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                 __builtin_amdgcn_perm(v.w, v.y, 0x05040100u), __builtin_amdgcn_perm(v.w, v.y, 0x07060302u)};
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// (a & m) | c in one instruction (gfx950 three-input bitwise operation)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, m, c, 0xEA);
}

// bf16 dot2 chain of one 16-byte code piece (32 weights) against its
// activations in pair order: the nibbles become the exact bf16 values 128 + q
// (bf16 has unit spacing on [128, 256)), so the chain sums (128 + q) x; the
// same chain over all-eight codes sums 136 x, and the difference is
// sum (q - 8) x, exactly 0 for a piece of eight-codes.
__device__ __forceinline__ float piece_dot_bf16(u32x4_t w, const u32x4_t (&xb)[4]) {
  float c = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t wd = w[d];
    c = dot2_bf16(and_or(wd, 0x000F000Fu, 0x43004300u), xb[d].x, c);
    c = dot2_bf16(and_or(wd >> 4, 0x000F000Fu, 0x43004300u), xb[d].y, c);
    c = dot2_bf16(and_or(wd >> 8, 0x000F000Fu, 0x43004300u), xb[d].z, c);
    c = dot2_bf16(and_or(wd >> 12, 0x000F000Fu, 0x43004300u), xb[d].w, c);
  }
  return c;
}

// float16 dot2 chain of one 16-byte code piece (32 weights) against its
// activations (the overflow path)
__device__ __forceinline__ float piece_dot(u32x4_t w, const u32x4_t (&xf)[4]) {
  float c = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t wd = w[d];
    const uint32_t w8 = wd >> 8;
    c = dot2_f16(wd & 0x000F000Fu, xf[d].x, c);
    c = dot2_f16(wd & 0x00F000F0u, xf[d].y, c);
    c = dot2_f16(w8 & 0x000F000Fu, xf[d].z, c);
    c = dot2_f16(w8 & 0x00F000F0u, xf[d].w, c);
  }
  return c;
}

// (128 + q) bf16 pairs of one 16-byte code piece, in the order of
// piece_dot_bf16's chain, for reuse against several tokens
__device__ __forceinline__ void piece_codes_bf16(u32x4_t w, uint32_t (&c)[16]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t wd = w[d];
    c[4 * d + 0] = and_or(wd, 0x000F000Fu, 0x43004300u);
    c[4 * d + 1] = and_or(wd >> 4, 0x000F000Fu, 0x43004300u);
    c[4 * d + 2] = and_or(wd >> 8, 0x000F000Fu, 0x43004300u);
    c[4 * d + 3] = and_or(wd >> 12, 0x000F000Fu, 0x43004300u);
  }
}

// the chain of piece_dot_bf16 on pre-converted codes (same order, same sum)
__device__ __forceinline__ float piece_dot_pre(const uint32_t (&c)[16], const u32x4_t (&xb)[4]) {
  float a = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    a = dot2_bf16(c[4 * d + 0], xb[d].x, a);
    a = dot2_bf16(c[4 * d + 1], xb[d].y, a);
    a = dot2_bf16(c[4 * d + 2], xb[d].z, a);
    a = dot2_bf16(c[4 * d + 3], xb[d].w, a);
  }
  return a;
}

// PL: consecutive 16-byte pieces per lane and row; MAXR: rows per lane, at
// most; NT: tokens (1..4).  With several tokens every lane keeps each token's
// piece of X, converts each code piece once and runs one dot chain per token
// (vector-ALU work grows with NT, the weight stream does not: a few tokens
// cost little more than one).
// WV: waves per workgroup (8, or 12 for long rows); GLU: LinearSwiGLU in one
// pass (each workgroup takes the same rows of the gate and the up weight).
template <int PL, int MAXR, int NT, int WV, bool GLU>
__global__ void __launch_bounds__(64 * WV)
decode_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
              uint16_t* y, int N, int K, int BN, const uint16_t* res, SecondPlane p2) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int G = K >> 6;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int bid = blockIdx.x;
  constexpr bool glu = GLU;
  if (!glu && p2.n > 0 && bid >= p2.first) {  // LinearPair: the second weight
    codes = p2.codes;
    scales = p2.scales;
    y = p2.y;
    N = p2.n;
    res = nullptr;  // a pair carries no residual
    bid -= p2.first;
  }
  // LinearSwiGLU: the block's rows are hrows gate rows from n0, then the
  // same rows of the up weight
  const int n0 = glu ? bid * (BN >> 1) : bid * BN;
  const int hrows = glu ? min(BN >> 1, N - n0) : 0;
  const int rows = glu ? 2 * hrows : min(BN, N - n0);
  // local row lr of the block (clamped to its rows): the planes it reads and
  // its row there
  auto plane_row = [&](int lr, const uint8_t*& cp, const uint16_t*& sp) __device__ {
    lr = min(lr, rows - 1);
    if (glu && lr >= hrows) {
      cp = p2.codes;
      sp = p2.scales;
      return n0 + lr - hrows;
    }
    cp = codes;
    sp = scales;
    return n0 + lr;
  };

  // wave slice, slots and row groups (all wave-uniform but the lane's own)
  const int gl = (G * wave) / WV, gh = (G * (wave + 1)) / WV;
  const int ng = gh - gl;
  const int P = 2 * ng;                          // pieces per row in the slice
  const int S = max((P + PL - 1) / PL, 1);       // slots per row
  const int R = 64 / S;                          // row groups per wave (>= 1)
  const int grp_raw = lane / S;
  // idle lanes (past R row groups) repeat the last group's addresses (no
  // extra memory traffic); their sums are never read
  const int grp = min(grp_raw, R - 1);
  const int slot = lane - grp_raw * S;
  const int pc0 = slot * PL;

  // LDS: per wave and token a scratch of 64 x MAXR floats (regions 16 bytes
  // more than that apart, so that the eight threads of a row, which read the
  // eight regions at the same offset, hit different banks), then the waves'
  // per-token exponents.
  int* wexp = reinterpret_cast<int*>(lds + WV * NT * kRegion<MAXR>);

  // 1. the lane's activations (first: waiting for them waits for nothing else)
  u32x4_t xv[NT][PL][4];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const u32x4_t* xp =
          reinterpret_cast<const u32x4_t*>(x + (size_t)t * K + 64 * gl + 32 * min(pc0 + i, max(P - 1, 0)));
#pragma unroll
      for (int d = 0; d < 4; ++d) xv[t][i][d] = xp[d];
    }
  // 2. codes of the lane's rows, in row order (the rows are waited for one by
  //    one below; values of rows past the block and pieces past the slice are
  //    never used)
  u32x4_t w[MAXR][PL];
#pragma unroll
  for (int j = 0; j < MAXR; ++j) {
    const uint8_t* cp;
    const uint16_t* sp;
    const int row = plane_row(grp + R * j, cp, sp);
    const uint8_t* rp = cp + (size_t)row * (size_t)(K >> 1) + (size_t)gl * 32;
#pragma unroll
    for (int i = 0; i < PL; ++i)
      w[j][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(rp + 16 * min(pc0 + i, max(P - 1, 0))));
    __builtin_amdgcn_sched_barrier(0);
  }
  // 3. the scales of the lane's pieces, last: they are needed only after
  //    every row's dot products (clamped rows and pieces stay valid)
  uint16_t sbits[MAXR][PL];
#pragma unroll
  for (int j = 0; j < MAXR; ++j) {
    const uint8_t* cp;
    const uint16_t* sp;
    const int row = plane_row(grp + R * j, cp, sp);
    const uint16_t* sr = sp + (size_t)row * (size_t)G + gl;
#pragma unroll
    for (int i = 0; i < PL; ++i) sbits[j][i] = sr[min(pc0 + i, max(P - 1, 0)) >> 1];
  }
  __builtin_amdgcn_sched_barrier(0);

  // 4. activation pairs in the order of the code pairs, and the correction
  //    sums of the all-eight codes through the very same dot chain
  u32x4_t xb[NT][PL][4];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < PL; ++i)
#pragma unroll
      for (int d = 0; d < 4; ++d) xb[t][i][d] = bf16_pairs(xv[t][i][d]);
  const u32x4_t k8 = {0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
  float c8[NT][PL];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < PL; ++i) c8[t][i] = piece_dot_bf16(k8, xb[t][i]);

  // 5. the pieces' sums (q - 8) x, row by row in the order the codes arrive:
  //    row j waits only for its own loads (the younger code loads of later
  //    rows and the scale loads may still be in flight)
  float dp[MAXR][NT][PL];
  static_for<MAXR>([&](auto jj) {
    constexpr int j = decltype(jj)::value;
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((MAXR - 1 - j) * PL + MAXR * PL));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      if constexpr (NT == 1) {
        dp[j][0][i] = piece_dot_bf16(w[j][i], xb[0][i]) - c8[0][i];  // converts as it goes (fewer registers)
      } else {
        uint32_t c[16];
        piece_codes_bf16(w[j][i], c);
#pragma unroll
        for (int t = 0; t < NT; ++t) dp[j][t][i] = piece_dot_pre(c, xb[t][i]) - c8[t][i];
      }
    }
  });
  // 6. scales
  float sc[MAXR][PL];
#pragma unroll
  for (int j = 0; j < MAXR; ++j)
#pragma unroll
    for (int i = 0; i < PL; ++i) sc[j][i] = pc0 + i < P ? f16_bits_to_f32(sbits[j][i]) : 0.0f;
  float acc[NT][MAXR];
  bool bad = false;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < MAXR; ++j) {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        bad |= !__builtin_isfinite(dp[j][t][i]);
        a = __builtin_fmaf(sc[j][i], dp[j][t][i], a);
      }
      acc[t][j] = a;
      bad |= !__builtin_isfinite(a);
    }

  // 7. activations near the bf16 maximum can overflow these FP32 sums: then
  //    the wave redoes its rows on float16 copies of X scaled by 2^-e (e per
  //    token from its slice's largest magnitude, so the sums stay in range)
  //    and its partials carry 2^-(e+24)
  int ew[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) ew[t] = 0;
  if (__builtin_amdgcn_ballot_w64(bad) != 0) {
    // (rare; twelve waves read the activations and codes again, so that
    // their registers need not live through the products above)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (WV != 8) {
#pragma unroll
        for (int i = 0; i < PL; ++i) {
          const u32x4_t* xp =
              reinterpret_cast<const u32x4_t*>(x + (size_t)t * K + 64 * gl + 32 * min(pc0 + i, max(P - 1, 0)));
#pragma unroll
          for (int d = 0; d < 4; ++d) xv[t][i][d] = xp[d];
        }
      }
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < PL; ++i)
#pragma unroll
        for (int d = 0; d < 4; ++d) m = max(m, max_mag8(xv[t][i][d]));
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
      const int e = exponent_for(m);
      u32x4_t xf[PL][4];
#pragma unroll
      for (int i = 0; i < PL; ++i)
#pragma unroll
        for (int d = 0; d < 4; ++d) xf[i][d] = to_f16_pairs(xv[t][i][d], e);
      float s8[PL];
#pragma unroll
      for (int i = 0; i < PL; ++i) s8[i] = piece_dot(k8, xf[i]);
#pragma unroll
      for (int j = 0; j < MAXR; ++j) {
        const uint8_t* cp;
        const uint16_t* sp;
        const int row = plane_row(grp + R * j, cp, sp);
        const uint8_t* rp = cp + (size_t)row * (size_t)(K >> 1) + (size_t)gl * 32;
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < PL; ++i) {
          u32x4_t wj;
          if constexpr (WV != 8) wj = *reinterpret_cast<const u32x4_t*>(rp + 16 * min(pc0 + i, max(P - 1, 0)));
          else wj = w[j][i];
          a = __builtin_fmaf(sc[j][i], piece_dot(wj, xf[i]) - s8[i], a);
        }
        acc[t][j] = a;
      }
      ew[t] = e + 24;
    }
  }
  // waves without groups contribute zero
  if (ng <= 0)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < MAXR; ++j) acc[t][j] = 0.0f;

  // 8. sums: every lane's partials and every wave's exponents into LDS; then
  //    eight threads per (row, token) each add one wave's S slots, scale by
  //    that wave's 2^ew in binary64, and combine the eight by shuffles; the
  //    first of them rounds to bf16 once and stores
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float* scratch = reinterpret_cast<float*>(lds + (wave * NT + t) * kRegion<MAXR>);
#pragma unroll
    for (int j = 0; j < MAXR; ++j) scratch[j * 64 + lane] = acc[t][j];
  }
  if (lane == 0)
#pragma unroll
    for (int t = 0; t < NT; ++t) wexp[wave * NT + t] = ew[t];
  __syncthreads();
  // (twelve waves: each thread leaves its wave's sum in LDS and one thread
  // per (row, token) adds the twelve in wave order)
  double* dsum = reinterpret_cast<double*>(lds + (((size_t)WV * NT * kRegion<MAXR> + (size_t)WV * NT * 4 + 7) & ~(size_t)7));
  // (LinearSwiGLU: the (row, token) sums in binary64, after the wave sums)
  double* dres = dsum + (WV == 8 ? 0 : (size_t)NT * BN * WV);
  for (int idx = tid; idx < NT * rows * WV; idx += 64 * WV) {
    const int wv = idx % WV, rt = idx / WV;
    const int t = NT == 1 ? 0 : rt / rows, r = rt - t * rows;
    const int glw = (G * wv) / WV, ngw = (G * (wv + 1)) / WV - glw;
    const int Sw = max((2 * ngw + PL - 1) / PL, 1), Rw = 64 / Sw;
    const int g = r % Rw, j = r / Rw;
    const float* sp = reinterpret_cast<const float*>(lds + (wv * NT + t) * kRegion<MAXR>) + j * 64 + g * Sw;
    float v0 = 0.0f, v1 = 0.0f, v2 = 0.0f, v3 = 0.0f;
    if ((Sw & 3) == 0 && Sw <= 32) {
      // all reads in flight together (at most 8 clamped 16-byte pieces)
      const int n4 = Sw >> 2;
      f32x4_t t4[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) t4[u] = reinterpret_cast<const f32x4_t*>(sp)[min(u, n4 - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (u < n4) {
          v0 += t4[u].x;
          v1 += t4[u].y;
          v2 += t4[u].z;
          v3 += t4[u].w;
        }
    } else {
      int sl = 0;
      for (; sl + 4 <= Sw; sl += 4) {
        v0 += sp[sl];
        v1 += sp[sl + 1];
        v2 += sp[sl + 2];
        v3 += sp[sl + 3];
      }
      for (; sl < Sw; ++sl) v0 += sp[sl];
    }
    double v = __builtin_ldexp((double)((v0 + v1) + (v2 + v3)), wexp[wv * NT + t]);
    if constexpr (WV == 8) {
      // the eight threads of a (row, token) are eight consecutive lanes of one wave
      v = sum8_lanes(v);
      if (wv == 0) {
        if (glu) {
          dres[t * rows + r] = v;
        } else {
          if (res != nullptr) v += (double)bf16_bits_to_f32(res[(size_t)t * N + n0 + r]);  // LinearAdd
          if (p2.f32) reinterpret_cast<float*>(y)[(size_t)t * N + n0 + r] = (float)v;  // LinearSwiGLU sums
          else y[(size_t)t * N + n0 + r] = f32_to_bf16_rne((float)v);
        }
      }
    } else {
      dsum[idx] = v;
    }
  }
  if constexpr (WV != 8) {
    __syncthreads();
    for (int rt = tid; rt < NT * rows; rt += 64 * WV) {
      const int t = NT == 1 ? 0 : rt / rows, r = rt - t * rows;
      double v = 0.0;
#pragma unroll
      for (int wv = 0; wv < WV; ++wv) v += dsum[rt * WV + wv];
      if (glu) {
        dres[t * rows + r] = v;
        continue;
      }
      if (res != nullptr) v += (double)bf16_bits_to_f32(res[(size_t)t * N + n0 + r]);  // LinearAdd
      if (p2.f32) reinterpret_cast<float*>(y)[(size_t)t * N + n0 + r] = (float)v;  // LinearSwiGLU sums
      else y[(size_t)t * N + n0 + r] = f32_to_bf16_rne((float)v);
    }
  }
  if (glu) {
    // y = bf16(silu(G) U): each sum rounded to binary32 first (the sums a
    // LinearSwiGLU leaves between passes), the gate in binary64, one
    // rounding of the product
    __syncthreads();
    for (int i = tid; i < NT * hrows; i += 64 * WV) {
      const int t = NT == 1 ? 0 : i / hrows, r = i - t * hrows;
      // (+0 maps a -0 sum to +0, as a sum of zero products starts at +0)
      const double g = (double)(float)dres[t * rows + r] + 0.0;
      const double u = (double)(float)dres[t * rows + hrows + r] + 0.0;
      const double silu = g / (1.0 + exp(-g));
      y[(size_t)t * N + n0 + r] = f32_to_bf16_rne((float)(silu * u));
    }
  }
}

// LDS bytes: per wave and token the scratch region, the waves' exponents,
// and for twelve waves the per-wave sums of the bn rows (binary64)
size_t decode_lds(int maxr, int nt, int wv, int64_t bn) {
  const size_t base = (size_t)wv * (size_t)nt * (size_t)(64 * maxr * 4 + 16) + (size_t)wv * (size_t)nt * 4;
  const size_t sums = (size_t)nt * (size_t)bn * 8;  // LinearSwiGLU's (row, token) sums
  return ((base + 7) & ~(size_t)7) + (wv == 8 ? 0 : (size_t)nt * (size_t)bn * (size_t)wv * 8) + sums;
}

template <int PL, int MAXR, int NT, int WV = 8>
hipError_t launch_pm(const DecodePlan& p, const GemvArgs& a, hipStream_t stream) {
  auto kern = a.glu ? decode_kernel<PL, MAXR, NT, WV, WV == 8> : decode_kernel<PL, MAXR, NT, WV, false>;
  const size_t lds = decode_lds(MAXR, NT, WV, p.bn);
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(kern));
  if (e != hipSuccess) return e;
  // (LinearSwiGLU: bn / 2 rows of each weight per workgroup)
  const int blocks1 = a.glu ? (int)((a.n + p.bn / 2 - 1) / (p.bn / 2)) : (int)((a.n + p.bn - 1) / p.bn);
  const int blocks2 = a.glu ? 0 : (int)((a.n2 + p.bn - 1) / p.bn);
  kern<<<dim3((unsigned)(blocks1 + blocks2)), dim3(64 * WV), lds, stream>>>(
      static_cast<const uint16_t*>(a.x), static_cast<const uint8_t*>(a.codes), static_cast<const uint16_t*>(a.scales),
      static_cast<uint16_t*>(a.y), (int)a.n, (int)a.k, p.bn, static_cast<const uint16_t*>(a.res),
      second_plane(a, blocks1));
  return hipGetLastError();
}

// instantiated (pieces per lane, rows per lane) shapes
// Lane shapes (PL, MAXR) in order of preference: the fewest registers first
// (PL 1, MAXR 8 leaves room for two workgroups per CU), then more pieces per
// lane, then more rows per lane.
constexpr int kShapes[][2] = {{1, 8}, {2, 8}, {4, 4}, {1, 16}};

}  // namespace

// One lane shape (pl pieces per lane, at most maxr rows per lane) for wv
// waves: the fewest workgroups per CU (up to cmax) whose blocks it covers.
static bool plan_shape(int64_t n, int64_t G, int64_t t, int wv, int64_t pl, int64_t maxr, int64_t cmax,
                       DecodePlan* p) {
  const int64_t pmax = 2 * ((G + wv - 1) / wv);
  const int64_t pmin = 2 * (G / wv);
  const int64_t s = (pmax + pl - 1) / pl;
  if (s > 64) return false;
  // every wave, also one with the smaller slice, must cover bn rows
  const int64_t smin = pmin > 0 ? (pmin + pl - 1) / pl : 1;
  const int64_t rmin = 64 / (s > smin ? s : smin);
  for (int64_t c = 1; c <= cmax; ++c) {  // workgroups per CU
    const int64_t bn = (n + 256 * c - 1) / (256 * c);
    if ((bn + rmin - 1) / rmin > maxr) continue;
    // fewer than half the lanes busy: leave the shape to the other route
    if (2 * rmin * s < 64 && bn > rmin) continue;
    // c workgroups of this size must fit one CU's 160 KB of LDS
    if (decode_lds((int)maxr, (int)t, wv, bn) * (size_t)c > 160 * 1024) continue;
    p->bn = (int)bn;
    p->pl = (int)pl;
    p->maxr = (int)maxr;
    p->waves = wv;
    p->blocks = (int)((n + bn - 1) / bn);
    return true;
  }
  return false;
}

// For each shape in turn, the fewest workgroups per CU (1..6, so blocks of
// about N / (256 c) rows) whose rows the shape covers.  Measured on
// 6144/14336/34816 x 5120 and 5120 x 17408: more, smaller blocks beat
// more rows per lane.  Two to four tokens take the first shape only (their
// activations and sums need the registers the other shapes use for codes).
constexpr int kMaxDecodeTokens = 4;
bool decode_plan(int64_t n, int64_t k, int64_t t, DecodePlan* p) {
  if (t < 1 || t > kMaxDecodeTokens || n < 1 || k < 64) return false;
  if (n * (k / 2) >= (int64_t(1) << 31)) return false;  // 32-bit buffer offsets
  const int64_t G = k / 64;
  bool found = false;
  for (const auto& sh : kShapes) {
    const int64_t pl = sh[0], maxr = sh[1];
    if (t > 1 && !(pl == 1 && maxr == 8)) continue;
    if (plan_shape(n, G, t, kWaves, pl, maxr, t > 1 ? 1 : 6, p)) {
      found = true;
      break;
    }
  }
  // A long row (K > 16384) needs two pieces per lane with eight waves; twelve
  // waves keep one piece per lane, twenty rows each (3 waves per SIMD, one
  // workgroup per CU).
  if (t == 1 && (!found || p->pl > 1)) {
    DecodePlan q;
    if (plan_shape(n, G, t, 12, 1, 20, 1, &q)) {
      *p = q;
      return true;
    }
  }
  return found;
}

bool decode_glu_ok(int64_t n, int64_t k, int64_t t) {
  DecodePlan p;
  return decode_plan(2 * n, k, t, &p) && p.waves == 8;
}

hipError_t launch_decode(const GemvArgs& a, hipStream_t stream) {
  DecodePlan p;
  if (!decode_plan(a.n + a.n2, a.k, a.t, &p)) return hipErrorInvalidValue;
  if (a.glu) {
    // the plan for both weights' rows, an even count per workgroup (the same
    // rows of each weight); odd counts give up a row
    if (a.n2 != a.n || p.waves != 8) return hipErrorInvalidValue;
    p.bn = p.bn >= 2 ? p.bn & ~1 : 2;
  }
  // Two weights: each ends in its own partial workgroup, which can push the
  // grid one past a round of the CUs (6144 + 1024 rows: 220 + 37 of 28 rows
  // against 256).  Plan for a few more rows (bn grows by one) until the two
  // grids together fit what the plan sized for one.
  for (int64_t extra = p.bn, i = 0; a.n2 > 0 && !a.glu && i < 4; extra += p.bn, ++i) {
    const int64_t b = (a.n + p.bn - 1) / p.bn + (a.n2 + p.bn - 1) / p.bn;
    DecodePlan q;
    if (b <= p.blocks || !decode_plan(a.n + a.n2 + extra, a.k, a.t, &q)) break;
    if (q.pl != p.pl || q.maxr != p.maxr || q.waves != p.waves) break;  // keep the kernel shape
    p = q;
  }
  if (p.waves == 8 && p.pl == 1 && p.maxr == 8) {
    switch (a.t) {
      case 1: return launch_pm<1, 8, 1>(p, a, stream);
      case 2: return launch_pm<1, 8, 2>(p, a, stream);
      case 3: return launch_pm<1, 8, 3>(p, a, stream);
      case 4: return launch_pm<1, 8, 4>(p, a, stream);
    }
  }
  if (a.t != 1) return hipErrorInvalidValue;
  if (p.waves == 12) return p.pl == 1 && p.maxr == 20 ? launch_pm<1, 20, 1, 12>(p, a, stream) : hipErrorInvalidValue;
  if (p.pl == 1 && p.maxr == 16) return launch_pm<1, 16, 1>(p, a, stream);
  if (p.pl == 2 && p.maxr == 8) return launch_pm<2, 8, 1>(p, a, stream);
  if (p.pl == 4 && p.maxr == 4) return launch_pm<4, 4, 1>(p, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace q4lin
