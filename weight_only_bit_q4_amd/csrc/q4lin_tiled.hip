// q4lin_tiled.hip -- the many-token route: LDS-tiled matrix-core GEMM.
//
// The pages' prior art for large T is a tiled BF16-input, FP32-accumulate
// MMA with 32x32 to 64x128 output tiles ("q4-linear.md", notes under the
// result table).  This is an MI355X design of the same step.
//
// Operands.  The matrix cores take float16 on both sides and accumulate in
// FP32 across all groups (v_mfma_f32_32x32x16_f16, A = activations, 32 tokens
// x 16 k; B = weights, 16 k x 32 rows).
//   * Weights are dequantized with their scale, as the pages' large-T path
//     feeds its MMA 16-bit dequantized weights: (q - 8) * s' rounded once to
//     float16 (11 significant bits, three more than bfloat16), with
//     s' = s * 2^c[n] and c[n] a per-row power of two that puts the row's
//     largest scale in [2^11, 2^12) (so nothing overflows float16 and small
//     scales keep full precision).  A code dword gives four float16 pairs:
//     v_bitop3 builds 1024 + q exactly, a packed subtraction of 1032 leaves
//     q - 8, a packed multiply applies s'.
//   * Activations: a preparation pass multiplies each token by a power of two
//     2^-e[t] chosen from its largest magnitude (so every bf16 value within
//     2^34 of it converts to float16 exactly) and writes them in the order the
//     matrix-core operand reads want.
//   * The epilogue multiplies by 2^(e[t] - c[n]) and rounds to bf16.
//
// Data movement.  A workgroup owns BN rows x BT tokens (and, when K is split,
// one share of the 64-groups).  Codes move in pairs of groups, 64 contiguous
// bytes of every row per 16-byte direct-to-LDS load, into an LDS ring of
// pair slots, with the pair's scales; activations go from L2 straight into
// each wave's matrix-core operand registers (AGPRs), a ring of register sets
// several groups ahead.  Each thread dequantizes its own share of a group's
// code dwords, with the scale of their row (loaded by another thread), into a
// padded, double-buffered weight tile; one barrier per group publishes the
// tile and the ring slots to all waves.  Waits are explicit s_waitcnt
// vmcnt(n) with n the count of younger loads still allowed in flight; the
// compiler's own fences would wait for all.
#include <type_traits>

#include "q4lin_device.h"
#include "q4lin_kernels.h"

namespace q4lin {

namespace {


// ---------------------------------------------------------------------------
// activation preparation
// ---------------------------------------------------------------------------
// Tile order: for token block tb (32 tokens) and group g, 4 KB laid out
// [m 0..3][h 0..1][i 0..31][8 values]; the 8 values are k = 64g + 32h + 8m +
// (0,4,1,5,2,6,3,7) (pair order), i the token inside the block.

__device__ __forceinline__ uint32_t max_mag8(u32x4_t v) {
  uint32_t m = max(max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu), max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu));
  return max(m, max(max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu), max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu)));
}

// 8 bf16 values -> float16 in pair order, times 2^-e.
__device__ __forceinline__ u32x4_t to_f16_pairs(u32x4_t v, int e) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t h[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    h[2 * q] = __builtin_bit_cast(uint16_t, (_Float16)__builtin_ldexpf(bf16_bits_to_f32(w[q] & 0xFFFFu), -e));
    h[2 * q + 1] = __builtin_bit_cast(uint16_t, (_Float16)__builtin_ldexpf(bf16_bits_to_f32(w[q] >> 16), -e));
  }
  return u32x4_t{h[0] | (h[4] << 16), h[1] | (h[5] << 16), h[2] | (h[6] << 16), h[3] | (h[7] << 16)};
}

// Per-row exponent c[n]: the row's largest scale magnitude times 2^c lies in
// [2^11, 2^12), clamped to c in [-4, 15] (so 2^c is a normal float16 and
// every scaled weight (q - 8) s 2^c stays below 2^15 in magnitude; the
// smallest float16 scale 2^-24 still scales to a normal 2^-9).  0 for a row
// of zero scales.  Eight lanes per row, 128 rows per workgroup.
constexpr int kRowLanes = 8;
__device__ __forceinline__ uint32_t max_mag_f16x8(u32x4_t v) {
  const uint32_t a = max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu), b = max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu);
  const uint32_t c = max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu), d = max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu);
  return max(max(a, b), max(c, d));
}
// Lane l of a row reads the row's 16-byte pieces l, l+8, ... when the rows
// are 16-byte aligned (G a multiple of 8), else its scales l, l+8, ...; four
// loads in flight per round (one round for rows of up to 32 pieces, K up to
// 16384); the eight lanes then combine their maxima.
__device__ void row_exponents(const uint16_t* __restrict__ scales, int N, int G, int r0, int* __restrict__ rexp) {
  const int r = r0 + (int)threadIdx.x / kRowLanes, sub = (int)threadIdx.x % kRowLanes;
  uint32_t m = 0;
  if (r < N) {
    const uint16_t* s = scales + (int64_t)r * G;
    if ((G & 7) == 0 && (reinterpret_cast<uintptr_t>(scales) & 15) == 0) {
      const int nv = G >> 3;
      const u32x4_t* s4 = reinterpret_cast<const u32x4_t*>(s);
      for (int c0 = sub; c0 < nv; c0 += 4 * kRowLanes) {
        u32x4_t v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = s4[min(c0 + i * kRowLanes, nv - 1)];
#pragma unroll
        for (int i = 0; i < 4; ++i) m = max(m, max_mag_f16x8(v[i]));
      }
    } else {
      for (int c0 = sub; c0 < G; c0 += 4 * kRowLanes) {
        uint32_t v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = s[min(c0 + i * kRowLanes, G - 1)] & 0x7FFFu;
#pragma unroll
        for (int i = 0; i < 4; ++i) m = max(m, v[i]);
      }
    }
  }
  m = max(m, (uint32_t)__shfl_xor((int)m, 1));
  m = max(m, (uint32_t)__shfl_xor((int)m, 2));
  m = max(m, (uint32_t)__shfl_xor((int)m, 4));
  if (r >= N || sub != 0) return;
  if (m >= 0x7C00u) m = 0x7BFFu;  // Inf/NaN scales are outside the contract
  int c = 0;
  if (m != 0u) {
    const int lg = (m >= 0x400u) ? (int)(m >> 10) - 15 : (31 - __builtin_clz(m)) - 24;  // floor(log2 |s|)
    c = min(max(11 - lg, -4), 15);
  }
  rexp[r] = c;
}

// Per-token exponent e[t] from the token's largest magnitude m (bf16 bits
// without sign): m * 2^-e lies in [2^14, 2^15), so every bf16 value within
// 2^34 of it converts to float16 exactly; 0 for an all-zero token.
__device__ __forceinline__ int token_exponent(uint32_t m) {
  if (m >= 0x7F80u) m = 0x7F7Fu;  // Inf/NaN inputs are outside the contract
  if (m == 0u) return 0;
  return ((m >= 0x80u) ? (int)(m >> 7) - 127 : (31 - __builtin_clz(m)) - 133) - 14;
}

// Piece p (values k = 8p .. 8p+7, in pair order) of token t into the tile
// order described above.
__device__ __forceinline__ void store_piece(u32x4_t* __restrict__ x16, int G, int t, int p, u32x4_t v) {
  const int g = p >> 3, kb = p & 7;
  x16[((size_t)(t >> 5) * G + g) * 256 + ((kb & 3) * 2 + (kb >> 2)) * 32 + (t & 31)] = v;
}

// Activation preparation, one pass: a workgroup of eight waves takes TOK
// consecutive tokens of the padded token range (2 for short prompts, so that
// the few tokens still spread over many CUs; 4 for long ones), wave w the
// w-th eighth of their 16-byte pieces; lane l serves token l % TOK and
// pieces l / TOK + (64 / TOK) j of the wave's share.  So every load
// instruction reads runs of 64 * 16 / TOK bytes of TOK token rows and every
// store writes whole 16 TOK-byte runs of the tile order (TOK consecutive
// tokens of a 32-token block).  The token's largest magnitude is combined
// over the lanes and then, through LDS, over the waves; the values wait in
// registers (up to MAXJ pieces per lane; longer rows are read a second time,
// from L2).  Padding tokens write zeros.  The blocks past the token blocks
// compute the row exponents.
constexpr int kPrepThreads = 512;
constexpr int kRowsPerBlock = kPrepThreads / kRowLanes;
constexpr int prep_tokens(int64_t t) { return t <= 128 ? 2 : 4; }
template <int MAXJ, int TOK>
__global__ void __launch_bounds__(kPrepThreads)
prep_act_kernel(const u32x4_t* __restrict__ x, int K, int T, int Tpad, int* __restrict__ texp,
                u32x4_t* __restrict__ x16, const uint16_t* __restrict__ scales, int N, int* __restrict__ rexp,
                int tok_blocks, int row_blocks1, const uint16_t* __restrict__ scales2, int N2,
                int* __restrict__ rexp2) {
  if ((int)blockIdx.x >= tok_blocks) {
    // the row exponents of the weight (and of a second weight after it)
    const int rb = (int)blockIdx.x - tok_blocks;
    if (rb < row_blocks1) row_exponents(scales, N, K >> 6, rb * kRowsPerBlock, rexp);
    else row_exponents(scales2, N2, K >> 6, (rb - row_blocks1) * kRowsPerBlock, rexp2);
    return;
  }
  constexpr int SUBS = 64 / TOK;                         // lanes per token in a wave
  __shared__ uint32_t wmax[kPrepThreads / 64][TOK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int itok = lane % TOK, sub = lane / TOK;
  const int t = blockIdx.x * TOK + itok;                // < Tpad (a multiple of 32)
  const bool real = t < T;
  const int nb = K >> 3, G = K >> 6;
  constexpr int NWV = kPrepThreads / 64;
  const int pw = (nb + NWV - 1) / NWV;                  // pieces per wave
  const int pb = wave * pw, pe = min(pb + pw, nb);
  const int nj = (pw + SUBS - 1) / SUBS;                // pieces per lane
  const u32x4_t* xt = x + (size_t)min(t, T - 1) * nb;  // padding tokens read a valid row
  uint32_t m = 0;
  u32x4_t v[MAXJ];
  if (nj <= MAXJ) {
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) v[j] = xt[min(pb + sub + SUBS * j, nb - 1)];
#pragma unroll
    for (int j = 0; j < MAXJ; ++j)
      if (pb + sub + SUBS * j < pe) m = max(m, max_mag8(v[j]));
  } else {
    for (int b0 = pb; b0 < pe; b0 += SUBS * MAXJ) {
#pragma unroll
      for (int j = 0; j < MAXJ; ++j) v[j] = xt[min(b0 + sub + SUBS * j, nb - 1)];
#pragma unroll
      for (int j = 0; j < MAXJ; ++j)
        if (b0 + sub + SUBS * j < pe) m = max(m, max_mag8(v[j]));
    }
  }
  // lanes of one token: l % TOK equal
#pragma unroll
  for (int o = TOK; o < 64; o <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  if (sub == 0) wmax[wave][itok] = m;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kPrepThreads / 64; ++w) m = max(m, wmax[w][itok]);
  const int e = real ? token_exponent(m) : 0;
  if (nj <= MAXJ) {
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      const int p = pb + sub + SUBS * j;
      if (p < pe) store_piece(x16, G, t, p, real ? to_f16_pairs(v[j], e) : u32x4_t{0u, 0u, 0u, 0u});
    }
  } else {
    for (int b0 = pb; b0 < pe; b0 += SUBS * MAXJ) {
#pragma unroll
      for (int j = 0; j < MAXJ; ++j) v[j] = xt[min(b0 + sub + SUBS * j, nb - 1)];
#pragma unroll
      for (int j = 0; j < MAXJ; ++j) {
        const int p = b0 + sub + SUBS * j;
        if (p < pe) store_piece(x16, G, t, p, real ? to_f16_pairs(v[j], e) : u32x4_t{0u, 0u, 0u, 0u});
      }
    }
  }
  if (wave == 0 && sub == 0) texp[t] = e;
}

// bit i of the result: bf16 value i of the 8 in v is Inf or NaN
__device__ __forceinline__ uint32_t nonfinite8(u32x4_t v) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m |= ((v[i] & 0x7F80u) == 0x7F80u ? 1u : 0u) << (2 * i);
    m |= ((v[i] & 0x7F800000u) == 0x7F800000u ? 1u : 0u) << (2 * i + 1);
  }
  return m;
}

// ---------------------------------------------------------------------------
// the tiled kernel
// ---------------------------------------------------------------------------
// (a & m) | c in one instruction (gfx950 three-input bitwise operation, truth
// table 0xEA), as a builtin so that the compiler sees it when it spaces the
// instructions around matrix-core operand reads.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, m, c, 0xEA);
}

// Weights (q - 8) * s' as float16 pairs in the order (k0,k4) (k1,k5) (k2,k6)
// (k3,k7) of a code dword: v_bitop3 builds 1024 + q exactly (fp16 spacing 1 on
// [1024, 2048)), a packed subtraction of 1032 leaves q - 8 exactly, and a packed
// multiply by the pair sp = (s', s') rounds (q - 8) * s' once to float16.
__device__ __forceinline__ u32x4_t dequant_dword(uint32_t w, uint32_t sp) {
  const f16x2_t o1 = {(_Float16)1032.0f, (_Float16)1032.0f};
  const f16x2_t s2 = __builtin_bit_cast(f16x2_t, sp);
  u32x4_t r;
  r.x = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2_t, and_or(w, 0x000F000Fu, 0x64006400u)) - o1) * s2);
  r.y = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2_t, and_or(w >> 4, 0x000F000Fu, 0x64006400u)) - o1) * s2);
  r.z = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2_t, and_or(w >> 8, 0x000F000Fu, 0x64006400u)) - o1) * s2);
  r.w = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2_t, and_or(w >> 12, 0x000F000Fu, 0x64006400u)) - o1) * s2);
  return r;
}

// Direct-to-LDS buffer loads: every lane of the wave sends BYTES bytes from
// base + voffset + soffset (voffset per lane, soffset wave-uniform) to
// lds_base + lane * BYTES (lds_base wave-uniform).  Reads at or past the
// resource's byte count return zeros.
using rsrc_t = __amdgpu_buffer_rsrc_t;

// raw (unformatted, stride 0) buffer over [base, base + bytes)
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void dma4(rsrc_t r, uint32_t voffset, uint32_t soffset, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 4, voffset,
                                           soffset, 0, 0);
}

__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voffset, uint32_t soffset, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, voffset,
                                           soffset, 0, 0);
}

// s_waitcnt encoding for gfx9: vmcnt in bits 3:0 and 15:14, expcnt 6:4 (7 =
// no wait), lgkmcnt 11:8 (15 = no wait).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }

template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
}

// s_waitcnt lgkmcnt(0) as a builtin, which the compiler's own counter
// tracking sees (an inline-asm wait is opaque to it, and it would then add
// waits of its own that count only the loads it knows).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4)); }

// 16-byte LDS read of a weight fragment into VGPRs, for the matrix cores'
// B operand: a wave's next-group fragments arrive there while its current
// ones (the other register set) are in use.  (The accumulators live in
// AGPRs, which the matrix cores read and write without the VGPR file, so the
// dequantization's VALU work has the VGPRs to itself.)  The compiler does not
// track this load: the caller waits (s_waitcnt lgkmcnt) before the registers
// are read.  The destination is also an input ("+v"), so it stays the
// register set's own: the compiler may not place it over an operand of a
// matrix-core instruction issued just before, which could still be reading
// it when the load returns.
template <int OFF>
__device__ __forceinline__ void lds_read_vgpr(f16x8_t& v, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "+v"(v) : "v"(addr), "i"(OFF));
}

// A dequantized weight tile holds 144 bytes per row: the row's 64 float16
// values (eight 16-byte pieces) and 16 bytes of padding, which spreads the
// matrix-core operand reads (32 rows, one piece each) over distinct banks.
constexpr int kRowBytes = 144;

// 16-byte buffer load into accumulation registers (AGPRs): the activation
// fragments go straight from memory (L2) to the registers the matrix cores
// read.  The compiler does not track this load either: the caller waits
// (s_waitcnt vmcnt) before the registers are read.  The destination is also
// an input ("+a"), for the reason given above.
template <int OFF>
// (The resource and the offset are wave-uniform; readfirstlane states it, so
// that they stay in scalar registers wherever the compiler's uniformity
// analysis loses track.)
__device__ __forceinline__ void buf_read_agpr(f16x8_t& v, u32x4_t rsrc, uint32_t voff, uint32_t soff) {
  const u32x4_t r = {(uint32_t)__builtin_amdgcn_readfirstlane((int)rsrc.x), (uint32_t)__builtin_amdgcn_readfirstlane((int)rsrc.y),
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)rsrc.z), (uint32_t)__builtin_amdgcn_readfirstlane((int)rsrc.w)};
  const uint32_t so = (uint32_t)__builtin_amdgcn_readfirstlane((int)soff);
  asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen offset:%4" : "+a"(v) : "v"(voff), "s"(r), "s"(so), "i"(OFF));
}

// Buffer resource for the raw (stride 0) byte range [base, base + bytes),
// built in scalar registers for the inline loads above.
__device__ __forceinline__ u32x4_t make_rsrc_sgpr(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return u32x4_t{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)) & 0xFFFFu,
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), 0x00020000u};
}

// Ring geometry.  Codes stream in pairs of groups (64 contiguous bytes of
// every row, moved by 16-byte direct-to-LDS loads) through an LDS ring of NP
// pair slots: even step s loads the pair of groups s+DC and s+DC+1 (a
// group's codes are dequantized two groups before its products), and slot
// reuse needs DC <= 2 NP.  The scales travel with their pair, one dword per
// thread and group.  Each wave's activation fragments stream through a ring
// of DA register sets, loaded DACT = DA-1 groups ahead, every step.  Before
// step s the batch of step s-4, which carries group s's activations, must have
// landed (and with it every older load, among them the codes of groups s+2
// and s+3, issued DC - 2 >= DACT groups ahead); the batches of steps
// s-3 .. s-1 may still be in flight.  (Measured: loading the codes the whole
// ring ahead, DC = 2 NP, gains nothing.)  The step code is unrolled over P
// steps, a multiple of every ring period (2 NP groups for the pair slots, DA
// for the register sets, 2 for the weight tiles), so that every slot, tile
// and register set a step touches is fixed by its position in the block:
// LDS addresses are immediates and no step computes an index.
constexpr int NP = 5;
constexpr int DC = 6;
constexpr int DA = 5;
constexpr int DACT = DA - 1;
constexpr int P = 10;
static_assert(DC <= 2 * NP && DC % 2 == 0 && DACT == 4 && DC - 2 >= DACT, "ring geometry");
static_assert(P % DA == 0 && P % (2 * NP) == 0, "the unrolled steps must cover every ring period");

template <int NS, int TS, int WN, int WT>
struct TiledShape {
  static constexpr int NT = 64 * WN * WT;                 // threads
  static constexpr int BN = 32 * NS * WN;                 // rows per workgroup
  static constexpr int BT = 32 * TS * WT;                 // tokens per workgroup
  static constexpr int CD = (BN * 8 + NT - 1) / NT;      // code dwords per thread per group (dequantization)
  static constexpr int CDF = BN * 8 / NT;                 // of which every thread has the first CDF
  static constexpr int AI = TS * 4;                       // 16-byte activation loads per lane per group
  static constexpr int CQ = (BN * 4 + NT - 1) / NT;       // 16-byte code loads per thread per pair
  static constexpr int CP = CQ;                           // loads per thread per pair
  static constexpr int CODE_B = CQ * NT * 16;             // one pair slot ([row][64 bytes], then slack)
  static constexpr int SQ = (BN * 3 + NT - 1) / NT;       // 16-byte loads per thread per scale strip
  static constexpr int STRIP_B = SQ * NT * 16;            // one scale strip ([row][48 bytes], then slack)
  static constexpr int W_B = BN * kRowBytes;              // one dequantized weight tile
  static constexpr int OFF_S = NP * CODE_B;
  static constexpr int OFF_W = OFF_S + 2 * STRIP_B;
  static constexpr int LDS_B = (OFF_W + 2 * W_B > BT * BN * 2) ? OFF_W + 2 * W_B : BT * BN * 2;
  // a partial last dword round covers whole waves (64 lanes, 8 rows each)
  static_assert(BN * 8 % 64 == 0, "code tiles must split into whole waves");
  static_assert(LDS_B <= 160 * 1024, "LDS budget");
  static_assert(3 * AI + 2 * CP + SQ <= 63, "the load counter holds 63");
};

// ADD: the LinearAdd form (a residual joins the results); the plain form
// carries none of its code.  GLU: the gated LinearSwiGLU tile (rows 0 ..
// BN/2 - 1 of a tile are rows n0 .. of the gate, rows BN/2 .. the same rows
// of the up weight, p2's planes; the epilogue forms bf16(silu(G) U)).
template <int NS, int TS, int WN, int WT, bool ADD, bool GLU = false>
__global__ void __launch_bounds__(64 * WN * WT)
tiled_kernel(const u32x4_t* __restrict__ x16, const int* __restrict__ texp, const int* __restrict__ rexp,
             const uint16_t* __restrict__ xraw, const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
             uint16_t* y, float* __restrict__ part, int N, int K, int T, int Tpad, int tiles_n,
             int tiles_t, int KS, const uint16_t* res, TiledPlane2 p2) {
  using Sh = TiledShape<NS, TS, WN, WT>;
  constexpr int NT = Sh::NT, BN = Sh::BN, BT = Sh::BT, CD = Sh::CD, CQ = Sh::CQ, CP = Sh::CP, AI = Sh::AI, SQ = Sh::SQ;
  constexpr int NW = WN * WT;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int G = K >> 6;
  // K split: the workgroup's share is the Gs groups from g0 (all of K when KS
  // is 1); inside the kernel groups are counted from g0
  // two weights: the workgroups from p2.first on serve the second
  int wgi = (int)blockIdx.x;
  if (!GLU && p2.n > 0 && wgi >= p2.first) {
    codes = p2.codes;
    scales = p2.scales;
    y = p2.y;
    part = p2.part;
    rexp = p2.rexp;
    N = p2.n;
    tiles_n = p2.tiles_n;
    wgi -= p2.first;
  }
  const int nblk = tiles_n * tiles_t;
  const int ks = wgi / nblk, bidx = wgi - ks * nblk;
  const int g0 = (int)(((int64_t)G * ks) / KS);
  const int Gs = (int)(((int64_t)G * (ks + 1)) / KS) - g0;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int li = lane & 31, lh = lane >> 5;
  const int wn = wave % WN, wt = wave / WN;

  // XCD-aware tile order.  Workgroups are dealt round-robin to the 8 XCDs,
  // each with its own L2.  Where the tile grid allows, the grid is cut into a
  // 4 x 2 (rows x tokens) block per XCD, so that each XCD's L2 fetches a
  // quarter of W and half of the activations (W would otherwise be fetched by
  // every XCD); else each XCD takes a contiguous run of tiles.  Inside an XCD
  // the row tile varies fastest, so that workgroups close in time share an
  // activation tile.
  int tile_t, tile_n;
  {
    const int xcd = bidx & 7, idx = bidx >> 3;
    if ((tiles_n & 3) == 0 && (tiles_t & 1) == 0) {
      const int bn = tiles_n >> 2, bt = tiles_t >> 1;
      const int lt = idx / bn;
      tile_t = (xcd >> 2) * bt + lt;
      tile_n = (xcd & 3) * bn + (idx - lt * bn);
    } else {
      const int lin = (nblk & 7) == 0 ? xcd * (nblk >> 3) + idx : bidx;
      tile_t = lin / tiles_n;
      tile_n = lin - tile_t * tiles_n;
    }
  }
  // GLU: BH rows of each weight per tile; tile row r < BH is row n0 + r of
  // the gate, r >= BH row n0 + r - BH of the up weight
  constexpr int BH = GLU ? BN / 2 : BN;
  auto prow = [](int r) { return GLU && r >= BH ? r - BH : r; };
  const int n0 = tile_n * BH;
  const int tb0 = tile_t * (BT / 32);                 // first 32-token block
  const int tb_last = Tpad / 32 - 1;

  // --- per-thread load offsets (32-bit, relative to per-group uniform offsets
  // into buffers that start at the tile) ---------------------------------------
  // Code load i of a pair: piece j = (i*NW + wave)*64 + lane, row j/4 of the
  // tile, 16-byte quarter j%4 of the row's 64 bytes; it lands at byte 16 j
  // of the pair slot, so the slot holds [row][64 bytes].  Pieces past the
  // tile (when 4 BN is not a multiple of NT) repeat the last one into the
  // slot's slack; rows past N repeat row N-1 (their outputs are dropped).
  // (GLU: load i of a wave reads 16 rows, 16 (i NW + wave) .. + 15, all of
  // one weight since BH is a multiple of 16; the up weight's from rc2)
  const uint8_t* codes_tile = codes + (size_t)n0 * (K >> 1);
  const uint32_t tile_code_bytes = (uint32_t)min((int64_t)(N - n0) * (K >> 1), (int64_t)0x7FFFFFFF);
  const rsrc_t rc = make_rsrc(codes_tile, tile_code_bytes);
  const rsrc_t rc2 = GLU ? make_rsrc(p2.codes + (size_t)n0 * (K >> 1), tile_code_bytes) : rc;
  static_assert(BH % 16 == 0, "a code load's 16 rows belong to one weight");
  uint32_t coff[CQ];
#pragma unroll
  for (int i = 0; i < CQ; ++i) {
    const int j = min((i * NW + wave) * 64 + lane, 4 * BN - 1);
    coff[i] = (uint32_t)(min(prow(j >> 2), N - 1 - n0) * (K >> 1) + (j & 3) * 16);
  }
  // Scales move in strips of P groups (one strip per block of unrolled
  // steps): strip b holds, for every row of the tile, the 48 bytes (three
  // aligned 16-byte pieces) that cover the row's 2 P bytes of scales of
  // groups g0 + P b .. g0 + P b + P - 1, as [row][48 bytes]; one 16-byte
  // direct-to-LDS load per piece, so a strip costs about one memory request
  // per row instead of one per row and group.  Piece p = i NT + tid of a
  // strip is piece p % 3 of row p / 3 and lands at byte 16 p.  The buffer
  // runs from the 16-byte boundary below the scale plane to the one above
  // its end (an aligned 16-byte piece never leaves the page of its bytes, so
  // the pieces that hold the first and the last scale are read whole; a
  // piece cut by the buffer's end would read as zeros); pieces past it read
  // zeros (they belong to groups past the last row's end, which nothing
  // reads).  With o the byte offset of the row's
  // scale of group g0 + P b, its scale of group g0 + P b + j sits at byte
  // 48 r + (o & 15) + 2 j of the strip.
  static_assert(2 * P + 14 <= 48, "a row's strip must fit three pieces");
  // GLU: each weight's rows take whole 1-KiB chunks of a strip (chunk c =
  // i NW + wave: the gate's rows in chunks 0 .. SCH - 1, the up weight's from
  // chunk SCH, its row r' at byte 1024 SCH + 48 r'), so that every load
  // reads one weight's scale plane.
  constexpr int SCH = (3 * BH + 63) / 64;  // chunks of one weight's rows (GLU)
  static_assert(!GLU || 2 * SCH <= SQ * NW, "both weights' strip chunks fit the strip");
  auto strip_rs = [&](const uint16_t* sc, int n) __device__ {
    const uintptr_t pl = reinterpret_cast<uintptr_t>(sc), base = pl & ~(uintptr_t)15;
    return make_rsrc(reinterpret_cast<const void*>(base),
                     (uint32_t)min(((int64_t)(pl - base) + (int64_t)n * ((int64_t)G * 2) + 15) & ~(int64_t)15,
                                   (int64_t)0x7FFFFFF0));
  };
  const uintptr_t s_plane = reinterpret_cast<uintptr_t>(scales);
  const uintptr_t s_base = s_plane & ~(uintptr_t)15;
  const rsrc_t rs = strip_rs(scales, N);
  const uintptr_t s_plane2 = GLU ? reinterpret_cast<uintptr_t>(p2.scales) : s_plane;
  const uintptr_t s_base2 = s_plane2 & ~(uintptr_t)15;
  const rsrc_t rs2 = GLU ? strip_rs(p2.scales, N) : rs;
  uint32_t so_p[SQ];  // strip 0 offset o of the row of piece i, plus 16 (p % 3)
#pragma unroll
  for (int i = 0; i < SQ; ++i) {
    if constexpr (GLU) {
      const int c = i * NW + wave;
      const bool up = c >= SCH;
      const int p = min((up ? c - SCH : c) * 64 + lane, 3 * BH - 1);
      const int r = min(p / 3, N - 1 - n0);
      so_p[i] = (uint32_t)(up ? s_plane2 - s_base2 : s_plane - s_base) + (uint32_t)((n0 + r) * G + g0) * 2u +
                (uint32_t)(p % 3) * 16u;
    } else {
      const int p = min(i * NT + tid, 3 * BN - 1);
      const int r = min(p / 3, N - 1 - n0);
      so_p[i] = (uint32_t)(s_plane - s_base) + (uint32_t)((n0 + r) * G + g0) * 2u + (uint32_t)(p % 3) * 16u;
    }
  }
  // Code dword c of this thread belongs to tile row (c * NT + tid) / 8;
  // s_r48[c] = 48 r and s_o[c] the strip 0 offset o of that row.  s_mul[c] is
  // the float16 pair (2^c[row], 2^c[row]), made from c[row] after the
  // prologue's wait (a use before it would stall the prologue's loads behind
  // the exponent loads).
  uint32_t s_r48[CD], s_o[CD], s_mul[CD];
  int rx_c[CD];
#pragma unroll
  for (int c = 0; c < CD; ++c) {
    const int r = min((c * NT + tid) >> 3, BN - 1);
    const bool up = GLU && r >= BH;
    const int rr = min(prow(r), N - 1 - n0);
    s_o[c] = (uint32_t)(up ? s_plane2 - s_base2 : s_plane - s_base) + (uint32_t)((n0 + rr) * G + g0) * 2u;
    s_r48[c] = up ? (uint32_t)(1024 * SCH + 48 * (r - BH)) : (uint32_t)r * 48u;
    rx_c[c] = up ? p2.rexp[n0 + rr] : rexp[n0 + rr];
  }
  // The epilogue's exponents, also loaded now: c[n] of the lane's rows and
  // e[t] of its tokens (16 per 32-token block: t = tl + 8 (r / 4) + r % 4,
  // tl a multiple of 4, as four 16-byte loads).  Not needed with a K split.
  int ce[NS];
  int4 ev[TS][4];
  if (part == nullptr) {
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) ce[ns] = rexp[min(n0 + (wn * NS + ns) * 32 + li, N - 1)];
#pragma unroll
    for (int ts = 0; ts < TS; ++ts) {
      const int tl = 32 * tb0 + (wt * TS + ts) * 32 + 4 * lh;
#pragma unroll
      for (int q = 0; q < 4; ++q) ev[ts][q] = *reinterpret_cast<const int4*>(texp + min(tl + 8 * q, Tpad - 4));
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // Activation fragment (ts, m) of lane (li, lh): 16 bytes of token block
  // tb0 + wt*TS + ts, group g, at ((m*2 + lh)*32 + li)*16 of its 4 KB block.
  const uint8_t* x16_tile = reinterpret_cast<const uint8_t*>(x16) + (size_t)tb0 * G * 4096;
  const u32x4_t rx = make_rsrc_sgpr(x16_tile, (uint32_t)min((int64_t)(tb_last + 1 - tb0) * G * 4096, (int64_t)0x7FFFFFFF));
  uint32_t aoff[TS];
#pragma unroll
  for (int ts = 0; ts < TS; ++ts)
    aoff[ts] = (uint32_t)(min(wt * TS + ts, tb_last - tb0) * G * 4096 + (lh * 32 + li) * 16);

  // --- the matrix-core operand registers --------------------------------------
  // Activations: DA sets, set g % DA holds group g.  Weights: two sets, set
  // g & 1 holds group g.  All in AGPRs, filled by untracked loads.
  f16x8_t act[DA][TS][4];
  f16x8_t wgt[2][NS][4];

  // --- one batch: a code pair and its scales into their slots, and
  // this wave's activation fragments of group ga into set A (indexes clamped
  // to the last group, so every batch has the same number of loads) --------
  // Load v of a batch: v < CQ a 16-byte code piece of pair q (groups 2q,
  // 2q+1), v = CQ, CQ+1 the scale dwords of the two groups, then the TS * 4
  // activation fragments of group ga.  Pair and group indexes are clamped to
  // the last ones, so every batch of a kind has the same number of loads.
  // Slots are compile-time: pair p sits in slot p % NP, and QS below is a
  // pair index whose remainder equals the real pair's (the real index may
  // be clamped to the last pair: such a load lands in the slot of a pair
  // past the end, which nothing reads).
  auto code_slot = [&](auto qs) __device__ { return lds + (decltype(qs)::value % NP) * Sh::CODE_B; };
  auto issue_one = [&](int q, auto qs, int ga, f16x8_t (&a)[TS][4], auto vi) __device__ {
    constexpr int v = decltype(vi)::value;
    if constexpr (v < CQ) {
      dma16((GLU && (v * NW + wave) * 16 >= BH) ? rc2 : rc, coff[v], (uint32_t)(g0 + 2 * q) * 32,
            code_slot(qs) + (v * NW + wave) * 1024);
    } else {
      constexpr int i = v - CQ, ts = i / 4, m = i % 4;
      buf_read_agpr<m * 1024>(a[ts][m], rx, aoff[ts], (uint32_t)(g0 + ga) * 4096);
    }
  };
  // scale strip b (of the workgroup's share) into strip buffer b & 1: piece
  // k of a row starts at the 16-byte boundary below the row's first scale
  // of the strip, plus 16 k
  auto issue_strip = [&](int b) __device__ {
    uint8_t* dst = lds + Sh::OFF_S + (b & 1) * Sh::STRIP_B;
#pragma unroll
    for (int i = 0; i < SQ; ++i) {
      // (o + 16 k) & ~15 = (o & ~15) + 16 k, with o the row's strip offset
      dma16((GLU && i * NW + wave >= SCH) ? rs2 : rs, (so_p[i] + (uint32_t)b * (2u * P)) & ~15u, 0u,
            dst + (i * NW + wave) * 1024);
    }
  };
  const int qlast = (Gs - 1) >> 1;
  auto issue_codes = [&](auto qs) __device__ {
    const int q = min((int)decltype(qs)::value, qlast);
    static_for<CP>([&](auto v) { issue_one(q, qs, 0, act[0], v); });
  };
  auto issue_act = [&](int ga, f16x8_t (&a)[TS][4]) __device__ {
    ga = min(ga, Gs - 1);
    static_for<TS * 4>([&](auto i) { issue_one(0, Slot<0>{}, ga, a, Slot<CP + decltype(i)::value>{}); });
  };

  // --- dequantization of group g into weight tile b, in two halves: the LDS
  // reads of this thread's own code dwords and scale dword (dq_load), and the
  // conversion and LDS writes (dq_store) -------------------------------------
  const int dq_off = (tid >> 3) * kRowBytes + (tid & 7) * 16;   // + c*(NT/8)*kRowBytes
  struct DqRegs {
    uint32_t w[CD];
    uint32_t sw[CD];
  };
  // code dword c of this thread: row (c*NT + tid)/8, dword tid%8 of the
  // group's 32 bytes in the row's 64-byte pair (pair slot of QS, group
  // parity PAR); its scale: group P b + J of the share, from strip b
  auto dq_load = [&](auto qs, auto par, int b, auto jj, DqRegs& d) __device__ {
    const uint8_t* cs = code_slot(qs) + (tid >> 3) * 64 + decltype(par)::value * 32 + (tid & 7) * 4;
    const uint8_t* ss = lds + Sh::OFF_S + (b & 1) * Sh::STRIP_B + 2 * decltype(jj)::value;
#pragma unroll
    for (int c = 0; c < CD; ++c) {
      if (c < Sh::CDF || c * NT + tid < BN * 8) {
        d.w[c] = *reinterpret_cast<const uint32_t*>(cs + c * (NT / 8) * 64);
        d.sw[c] = *reinterpret_cast<const uint16_t*>(ss + s_r48[c] + ((s_o[c] + (uint32_t)b * (2u * P)) & 15u));
      }
    }
  };
  // A group (of parity ODD) into weight tile B with the scales s' = s 2^c[row]
  // (exact unless s lies 2^25 or more below the row's largest scale).  Tiles
  // of groups past the end hold whatever the clamped loads brought; no
  // matrix-core instruction reads them.
  auto dq_store_one = [&](auto b, const DqRegs& d, auto odd, int c) __device__ {
    if (c >= Sh::CDF && c * NT + tid >= BN * 8) return;  // past the tile (wave-uniform)
    uint8_t* wb = lds + Sh::OFF_W + decltype(b)::value * Sh::W_B + dq_off;
    (void)odd;
    const f16x2_t s2 = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(d.sw[c], d.sw[c], 0x01000100u));
    const uint32_t sp = __builtin_bit_cast(uint32_t, s2 * __builtin_bit_cast(f16x2_t, s_mul[c]));
    *reinterpret_cast<u32x4_t*>(wb + c * (NT / 8) * kRowBytes) = dequant_dword(d.w[c], sp);
  };
  auto dq_store = [&](auto b, const DqRegs& d, auto odd) __device__ {
#pragma unroll
    for (int c = 0; c < CD; ++c) dq_store_one(b, d, odd, c);
  };

  // --- weight fragments of the group in tile TB --------------------------------
  const int b_row = wn * NS * 32 + li;                                  // + ns*32
  const uint32_t wrd = (uint32_t)reinterpret_cast<uintptr_t>(lds) + (uint32_t)(Sh::OFF_W + b_row * kRowBytes + lh * 64);
  auto read_wgt_one = [&](auto tb, f16x8_t (&b)[NS][4], auto ii) __device__ {
    constexpr int ns = decltype(ii)::value / 4, m = decltype(ii)::value % 4;
    lds_read_vgpr<decltype(tb)::value * Sh::W_B + ns * 32 * kRowBytes + m * 16>(b[ns][m], wrd);
  };
  auto read_wgt = [&](auto tb, f16x8_t (&b)[NS][4]) __device__ {
    static_for<NS * 4>([&](auto i) { read_wgt_one(tb, b, i); });
  };

  f32x16_t acc[TS][NS];
#pragma unroll
  for (int ts = 0; ts < TS; ++ts)
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[ts][ns][r] = 0.0f;

  // Before the barrier of step s: this thread's batch of step s-4 has landed
  // (the three younger batches may still be in flight: 3 activation loads
  // sets and one (s even) or two (s odd) code pairs), and its LDS reads and
  // writes (also the untracked weight reads) are done.
  // (STRIP: a scale strip was issued after batch s-4, so SQ more loads may
  // be in flight)
  auto sync = [&](auto odd, auto strip) __device__ {
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<3 * AI + (decltype(odd)::value ? 2 : 1) * CP + (decltype(strip)::value ? SQ : 0)>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Step g (SL = g % P, so g has the parity of SL).  The memory and VALU
  // work is spread between the matrix-core instructions, so that one wave
  // per SIMD keeps the matrix core, the load path, the LDS and the VALU busy
  // at once:
  //   * after the barrier, read the code and scale dwords of group g+2;
  //   * k-slice 0 of group g's products (no LDS data needed), with a quarter
  //     of the batch's loads (g even: the code pair of groups g+DC, g+DC+1;
  //     activations of g+DACT) between its instructions;
  //   * wait for the dword reads;
  //   * k-slices 1-3, each led by a share of the batch's other loads and a
  //     third of group g+1's weight reads (untracked loads, issued after the
  //     wait so that no wait of the compiler counts them), interleaved with
  //     the dequantization of a third of this thread's dwords of group g+2.
  // (Issued in one burst, the loads of four waves stall their issue behind
  // the load path for longer than a k-slice takes.)
  // Near the last group the reads and the dequantization of groups past the
  // end touch stale LDS (unused) and the loads repeat the last group, so the
  // step is one basic block.
  constexpr int NM = TS * NS;               // matrix-core instructions per k-slice
  auto mfma_one = [&](int m, int j, auto slot) __device__ {
    constexpr int SL = decltype(slot)::value;
    const int ts = j / NS, ns = j % NS;
    acc[ts][ns] = __builtin_amdgcn_mfma_f32_32x32x16_f16(act[SL % DA][ts][m], wgt[SL & 1][ns][m], acc[ts][ns], 0, 0, 0);
  };
  auto step = [&](int g, auto slot, int blk) __device__ {
    constexpr int SL = decltype(slot)::value;
    constexpr bool EVEN = (SL & 1) == 0;
    constexpr int V0 = EVEN ? 0 : CP;          // first load of this step's batch
    constexpr int NV = CP + AI - V0;           // loads in this step's batch
    // g = gb + SL with gb a multiple of P: the pair of group g+2 sits in
    // slot ((SL + 2) >> 1) % NP, the pair this step loads in slot
    // ((SL + DC) >> 1) % NP, and g, g+2 have the parity of SL
    constexpr int QD = (SL + 2) >> 1, QL = (SL + DC) >> 1;
    // the scale strip of block blk is issued at the end of its step 8
    static_assert(P == 10, "strip issue and waits assume blocks of 10 steps");
    sync(std::integral_constant<bool, !EVEN>{}, std::integral_constant<bool, SL == 9 || SL <= 2>{});
    DqRegs d;
    dq_load(Slot<QD>{}, std::integral_constant<int, SL & 1>{}, blk + (SL + 2) / P, Slot<(SL + 2) % P>{}, d);
    const int q = min((g + DC) >> 1, qlast), ga = min(g + DACT, Gs - 1);
    __builtin_amdgcn_sched_barrier(0);
    // the batch's loads: a quarter in k-slice 0 (one or two after each
    // matrix-core instruction), a quarter at the head of each other k-slice
    constexpr int NV0 = NV / 4;
    static_for<NM>([&](auto jj) {
      constexpr int j = decltype(jj)::value;
      mfma_one(0, j, slot);
      static_for<(j + 1) * NV0 / NM - j * NV0 / NM>([&](auto u) {
        issue_one(q, Slot<QL>{}, ga, act[(SL + DACT) % DA], Slot<V0 + j * NV0 / NM + decltype(u)::value>{});
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    wait_lgkm0();
    __builtin_amdgcn_sched_barrier(0);
    static_for<3>([&](auto ss) {
      constexpr int sl = decltype(ss)::value;
      constexpr int r0 = sl * NS * 4 / 3, r1 = (sl + 1) * NS * 4 / 3;
      constexpr int u0 = NV0 + sl * (NV - NV0) / 3, u1 = NV0 + (sl + 1) * (NV - NV0) / 3;
      static_for<u1 - u0>([&](auto u) {
        issue_one(q, Slot<QL>{}, ga, act[(SL + DACT) % DA], Slot<V0 + u0 + decltype(u)::value>{});
      });
      static_for<r1 - r0>([&](auto u) {
        read_wgt_one(Slot<(SL + 1) & 1>{}, wgt[(SL + 1) & 1], Slot<r0 + decltype(u)::value>{});
      });
      __builtin_amdgcn_sched_barrier(0);
      constexpr int c0 = sl * CD / 3, c1 = (sl + 1) * CD / 3;
#pragma unroll
      for (int j = 0; j < NM; ++j) mfma_one(sl + 1, j, slot);
#pragma unroll
      for (int c = c0; c < c1; ++c) dq_store_one(Slot<SL & 1>{}, d, std::integral_constant<bool, (SL & 1) != 0>{}, c);
      // one matrix-core instruction, then a share of the VALU work
      constexpr int kValu = ((c1 - c0) * 18 + NM - 1) / NM;
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);   // VALU
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    // Step 8 of block blk comes after the barrier that ends the last read of
    // strip blk (its group P blk + 9 was read at step 7): strip blk + 2 into
    // the same buffer, ten steps before its first read.  (Past the last
    // strip this reads unused scales or zeros.)
    if constexpr (SL == 8) issue_strip(blk + 2);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Prologue: scale strips 0 and 1, code pairs 0..DC/2-1 (groups 0..DC-1;
  // step 0 loads the next) and activations of groups 0..DACT-1 in flight,
  // then all landed; groups 0 and 1 dequantized; group 0's weights read.
  issue_strip(0);
  issue_strip(1);
  static_for<DC / 2>([&](auto i) { issue_codes(i); });
  static_for<DACT>([&](auto i) { issue_act(decltype(i)::value, act[decltype(i)::value]); });
  // A thread dequantizes its own code dwords but reads row scales that other
  // waves loaded: a barrier after the waits publishes them, and a second one
  // (which also publishes the weight tiles) orders every read of pair slot 0
  // before step 0 loads pair NP into it.
  __builtin_amdgcn_sched_barrier(0);
  wait_vm<0>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < CD; ++c) {
    const uint32_t h = (uint32_t)(rx_c[c] + 15) << 10;
    s_mul[c] = h | (h << 16);
  }
  {
    DqRegs d;
    dq_load(Slot<0>{}, std::integral_constant<int, 0>{}, 0, Slot<0>{}, d);
    dq_store(Slot<0>{}, d, std::false_type{});
    dq_load(Slot<0>{}, std::integral_constant<int, 1>{}, 0, Slot<1>{}, d);
    dq_store(Slot<1>{}, d, std::true_type{});
  }
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  read_wgt(Slot<0>{}, wgt[0]);
  // Steps run in blocks of P (the ring indexes repeat with period P): whole
  // blocks without a test, then the last partial block, which stops after
  // the last group.
  int gb = 0, blk = 0;
  for (; gb + P <= Gs; gb += P, ++blk) static_for<P>([&](auto sl) { step(gb + decltype(sl)::value, sl, blk); });
  if (gb < Gs) {
    static_for<P>([&](auto sl) {
      constexpr int SL = decltype(sl)::value;
      if (SL == 0 || gb + SL < Gs) step(gb + SL, sl, blk);
    });
  }
  // no load may still write this workgroup's LDS or registers after this
  wait_vm<0>();
  wait_lgkm0();

  // Epilogue: lane (li, lh) holds row n = n0 + 32 (wn*NS + ns) + li and tokens
  // t = 32 (tb0 + wt*TS + ts) + 8 (r / 4) + 4 lh + r % 4.  The bf16 results
  // go through LDS ([token][row] order), so that the stores to y are whole
  // 16-byte pieces of token rows.
  static_assert(BT * BN * 2 <= Sh::LDS_B, "output tile must fit the LDS");
  if (part != nullptr) {
    // K split: this split's raw FP32 sums (they carry 2^(c[n] - e[t])) into
    // its slice of the partials, [split][token][row]; a second kernel adds
    // the splits and finishes the outputs
    float* pk = part + (size_t)ks * (size_t)Tpad * (size_t)N;
#pragma unroll
    for (int ts = 0; ts < TS; ++ts)
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        const int n = n0 + (wn * NS + ns) * 32 + li;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = 32 * tb0 + (wt * TS + ts) * 32 + 4 * lh + 8 * (r >> 2) + (r & 3);
          if (t < T && n < N) pk[(size_t)t * N + n] = acc[ts][ns][r];
        }
      }
    return;
  }
  if constexpr (GLU) {
    // LinearSwiGLU: the tile's raw FP32 sums ([token][row]: the gate's rows,
    // then the up weight's) and the exponents go through LDS; each output
    // then takes its two sums as the two-pass form does: scaled by
    // 2^(e[t] - c[n]) in binary64 (+0 maps a -0 sum to +0), the gate
    // silu(g) = g / (1 + e^-g) in binary64, one rounding of the product.
    static_assert(BT * BN * 4 + (BT + BN) * 4 <= 160 * 1024, "the gated tile's sums fit the LDS");
    __syncthreads();
    float* ft = reinterpret_cast<float*>(lds);
    int* el = reinterpret_cast<int*>(lds + BT * BN * 4);
    int* cl = el + BT;
#pragma unroll
    for (int ts = 0; ts < TS; ++ts) {
      const int tl = (wt * TS + ts) * 32 + 4 * lh;
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int ns = 0; ns < NS; ++ns)
          ft[(tl + 8 * (r >> 2) + (r & 3)) * BN + (wn * NS + ns) * 32 + li] = acc[ts][ns][r];
    }
    for (int i = tid; i < BT; i += NT) el[i] = texp[min(32 * tb0 + i, Tpad - 1)];
    for (int i = tid; i < BN; i += NT) cl[i] = (i >= BH ? p2.rexp : rexp)[min(n0 + prow(i), N - 1)];
    __syncthreads();
    // Eight adjacent rows of one token per thread and step: 16-byte LDS
    // reads of their sums and exponents and one 16-byte store where the rows
    // allow (one LDS read and one 2-byte store per output took about 6 us
    // more than the pair's epilogue at 3072 rows of each weight, T = 1024).
    const int tg0 = 32 * tb0;
    constexpr int G8 = BH / 8;
    static_assert(BH % 8 == 0 && BT % 4 == 0, "16-byte groups of rows and exponents");
    const bool vec = (N & 7) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0;
    for (int gi = tid; gi < BT * G8; gi += NT) {
      const int tl = gi / G8, r0 = (gi - tl * G8) * 8;
      if (tg0 + tl >= T || n0 + r0 >= N) continue;
      const f32x4_t* fg = reinterpret_cast<const f32x4_t*>(ft + tl * BN + r0);
      const f32x4_t* fu = reinterpret_cast<const f32x4_t*>(ft + tl * BN + BH + r0);
      const int4* cg = reinterpret_cast<const int4*>(cl + r0);
      const int4* cu = reinterpret_cast<const int4*>(cl + BH + r0);
      const f32x4_t g4[2] = {fg[0], fg[1]}, u4[2] = {fu[0], fu[1]};
      const int4 cg4[2] = {cg[0], cg[1]}, cu4[2] = {cu[0], cu[1]};
      const int e = el[tl];
      uint16_t h[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int cgj = j & 2 ? (j & 1 ? cg4[j >> 2].w : cg4[j >> 2].z) : (j & 1 ? cg4[j >> 2].y : cg4[j >> 2].x);
        const int cuj = j & 2 ? (j & 1 ? cu4[j >> 2].w : cu4[j >> 2].z) : (j & 1 ? cu4[j >> 2].y : cu4[j >> 2].x);
        const float gj = g4[j >> 2][j & 3], uj = u4[j >> 2][j & 3];
        const double gv = __builtin_ldexp((double)gj, e - cgj) + 0.0;
        const double uv = __builtin_ldexp((double)uj, e - cuj) + 0.0;
        const double silu = gv / (1.0 + exp(-gv));
        h[j] = f32_to_bf16_rne((float)(silu * uv));
      }
      uint16_t* yo = y + (size_t)(tg0 + tl) * N + n0 + r0;
      if (vec && n0 + r0 + 8 <= N) {
        *reinterpret_cast<u32x4_t*>(yo) =
            u32x4_t{(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16),
                    (uint32_t)h[4] | ((uint32_t)h[5] << 16), (uint32_t)h[6] | ((uint32_t)h[7] << 16)};
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (n0 + r0 + j < N) yo[j] = h[j];
      }
    }
    return;
  }
  // LinearAdd: the tile's residual values, all loaded before the first use
  // (one round trip: the loads are unconditional, at clamped indices, so no
  // branch separates them), so each joins its FP32 result before the one
  // rounding.  Values of padding tokens and rows are never stored.
  uint16_t rr[TS][NS][16];
  if constexpr (ADD) {
#pragma unroll
    for (int ts = 0; ts < TS; ++ts)
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = min(32 * tb0 + (wt * TS + ts) * 32 + 4 * lh + 8 * (r >> 2) + (r & 3), T - 1);
          const int n = min(n0 + (wn * NS + ns) * 32 + li, N - 1);
          rr[ts][ns][r] = res[(size_t)t * N + n];
        }
  }
  __syncthreads();
  uint16_t* otile = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
  for (int ts = 0; ts < TS; ++ts) {
    const int tl = (wt * TS + ts) * 32 + 4 * lh;
    int e[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      e[4 * q + 0] = ev[ts][q].x;
      e[4 * q + 1] = ev[ts][q].y;
      e[4 * q + 2] = ev[ts][q].z;
      e[4 * q + 3] = ev[ts][q].w;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        float v = __builtin_ldexpf(acc[ts][ns][r], e[r] - ce[ns]);
        if constexpr (ADD) v += bf16_bits_to_f32(rr[ts][ns][r]);
        otile[(tl + 8 * (r >> 2) + (r & 3)) * BN + (wn * NS + ns) * 32 + li] = f32_to_bf16_rne(v);
      }
  }
  __syncthreads();
  const int t0 = 32 * tb0;
  if ((reinterpret_cast<uintptr_t>(y) & 15) == 0 && (N & 7) == 0 && n0 + BN <= N) {
    constexpr int CPR = BN / 8;  // 16-byte pieces per token row of the tile
    for (int c = tid; c < BT * CPR; c += NT) {
      const int tl = c / CPR, cn = c - tl * CPR;
      if (t0 + tl < T) {
        u32x4_t v = *reinterpret_cast<const u32x4_t*>(otile + tl * BN + cn * 8);
        uint32_t bad = nonfinite8(v);
        while (bad != 0u) {  // rare: recompute exactly (exact_q4_output)
          const int i = __builtin_ctz(bad);
          bad &= bad - 1u;
          const uint32_t h = exact_q4_output(xraw, codes, scales, ADD ? res : nullptr, N, K, n0 + cn * 8 + i, t0 + tl);
          v[i >> 1] = (i & 1) ? ((v[i >> 1] & 0xFFFFu) | (h << 16)) : ((v[i >> 1] & 0xFFFF0000u) | h);
        }
        *reinterpret_cast<u32x4_t*>(y + (size_t)(t0 + tl) * N + n0 + cn * 8) = v;
      }
    }
  } else {
    for (int c = tid; c < BT * BN; c += NT) {
      const int tl = c / BN, nl = c - tl * BN;
      if (t0 + tl < T && n0 + nl < N) {
        uint16_t v = otile[c];
        if ((v & 0x7F80u) == 0x7F80u) v = exact_q4_output(xraw, codes, scales, ADD ? res : nullptr, N, K, n0 + nl, t0 + tl);
        y[(size_t)(t0 + tl) * N + n0 + nl] = v;
      }
    }
  }
}

// The K-split outputs: y[t][n] = bf16(2^(e[t] - c[n]) * sum over splits of
// the partials), the splits added in order.  A thread takes four consecutive
// outputs (16-byte partial loads, all issued before the sums) when N is a
// multiple of 4, else one.
constexpr int kMaxSplits = 8;
__device__ __forceinline__ uint16_t reduce_out(float v, int e, const uint16_t* res, size_t i,
                                               const uint16_t* __restrict__ xraw, const uint8_t* __restrict__ codes,
                                               const uint16_t* __restrict__ scales, int N, int K, int n, int t) {
  v = __builtin_ldexpf(v, e);
  if (res != nullptr) v += bf16_bits_to_f32(res[i]);  // LinearAdd
  uint16_t h = f32_to_bf16_rne(v);
  if ((h & 0x7F80u) == 0x7F80u) h = exact_q4_output(xraw, codes, scales, res, N, K, n, t);  // rare
  return h;
}
__global__ void __launch_bounds__(256)
tiled_reduce_kernel(const float* __restrict__ part, const int* __restrict__ texp, const int* __restrict__ rexp,
                    uint16_t* y, int N, int Tpad, int KS, const uint16_t* res, const uint16_t* __restrict__ xraw,
                    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales, int K) {
  const int t = blockIdx.y;
  const size_t stride = (size_t)Tpad * N;
  if ((N & 3) == 0) {
    const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (n >= N) return;
    const size_t i = (size_t)t * N + n;
    f32x4_t p[kMaxSplits];
#pragma unroll
    for (int k = 0; k < kMaxSplits; ++k)
      p[k] = k < KS ? *reinterpret_cast<const f32x4_t*>(part + k * stride + i) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    const u32x4_t ce = *reinterpret_cast<const u32x4_t*>(rexp + n);
    const int et = texp[t];
    uint16_t h[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v = 0.0f;
#pragma unroll
      for (int k = 0; k < kMaxSplits; ++k)
        if (k < KS) v += p[k][j];
      h[j] = reduce_out(v, et - (int)ce[j], res, i + j, xraw, codes, scales, N, K, n + j, t);
    }
    uint16_t* yo = y + i;
    if ((reinterpret_cast<uintptr_t>(yo) & 7) == 0) {
      *reinterpret_cast<u32x2_t*>(yo) = u32x2_t{(uint32_t)h[0] | ((uint32_t)h[1] << 16),
                                                (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) yo[j] = h[j];
    }
    return;
  }
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const size_t i = (size_t)t * N + n;
  float p[kMaxSplits];
#pragma unroll
  for (int k = 0; k < kMaxSplits; ++k) p[k] = k < KS ? part[k * stride + i] : 0.0f;
  float v = 0.0f;
#pragma unroll
  for (int k = 0; k < kMaxSplits; ++k)
    if (k < KS) v += p[k];
  y[i] = reduce_out(v, texp[t] - rexp[n], res, i, xraw, codes, scales, N, K, n, t);
}

// grid of the split sums for n outputs per token
inline dim3 reduce_grid(int64_t n, int64_t t) {
  const int64_t per_block = (n % 4 == 0) ? 1024 : 256;
  return dim3((unsigned)((n + per_block - 1) / per_block), (unsigned)t);
}

// The weight's tiles (and a second weight's after them); the K-split sums
// of each weight, if any, added by a pass per weight.
struct Plane2Host {
  const void* codes = nullptr;
  const void* scales = nullptr;
  void* y = nullptr;
  float* part = nullptr;
  const int* rexp = nullptr;
  int64_t n = 0;
};
template <int NS, int TS, int WN, int WT>
hipError_t launch_cfg(const TiledArgs& a, const u32x4_t* x16, const int* texp, const int* rexp, float* part,
                      int tpad, hipStream_t stream, const Plane2Host& h2 = Plane2Host{}) {
  using Sh = TiledShape<NS, TS, WN, WT>;
  const int tiles_n = (int)((a.n + Sh::BN - 1) / Sh::BN);
  const int tiles_t = (int)((a.t + Sh::BT - 1) / Sh::BT);
  auto kern = a.res != nullptr ? tiled_kernel<NS, TS, WN, WT, true> : tiled_kernel<NS, TS, WN, WT, false>;
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(kern));
  if (e != hipSuccess) return e;
  const int ks = a.cfg.ks;
  if (ks < 1 || ks > kMaxSplits) return hipErrorInvalidValue;
  const bool keep_part = ks > 1 || a.f32;
  TiledPlane2 p2;
  int blocks = tiles_n * tiles_t * ks;
  if (h2.n > 0) {
    p2.codes = static_cast<const uint8_t*>(h2.codes);
    p2.scales = static_cast<const uint16_t*>(h2.scales);
    p2.y = static_cast<uint16_t*>(h2.y);
    p2.part = keep_part ? h2.part : nullptr;
    p2.rexp = h2.rexp;
    p2.n = (int)h2.n;
    p2.tiles_n = (int)((h2.n + Sh::BN - 1) / Sh::BN);
    p2.first = blocks;
    blocks += p2.tiles_n * tiles_t * ks;
  }
  kern<<<dim3((unsigned)blocks), dim3(Sh::NT), Sh::LDS_B, stream>>>(
      x16, texp, rexp, static_cast<const uint16_t*>(a.x), static_cast<const uint8_t*>(a.codes),
      static_cast<const uint16_t*>(a.scales),
      static_cast<uint16_t*>(a.y), keep_part ? part : nullptr, (int)a.n, (int)a.k, (int)a.t, tpad, tiles_n, tiles_t, ks,
      static_cast<const uint16_t*>(a.res), p2);
  e = hipGetLastError();
  if (e != hipSuccess || ks == 1 || a.f32) return e;
  tiled_reduce_kernel<<<reduce_grid(a.n, a.t), dim3(256), 0, stream>>>(
      part, texp, rexp, static_cast<uint16_t*>(a.y), (int)a.n, tpad, ks, static_cast<const uint16_t*>(a.res),
      static_cast<const uint16_t*>(a.x), static_cast<const uint8_t*>(a.codes), static_cast<const uint16_t*>(a.scales),
      (int)a.k);
  e = hipGetLastError();
  if (e != hipSuccess || h2.n == 0) return e;
  tiled_reduce_kernel<<<reduce_grid(h2.n, a.t), dim3(256), 0, stream>>>(
      h2.part, texp, h2.rexp, static_cast<uint16_t*>(h2.y), (int)h2.n, tpad, ks, nullptr,
      static_cast<const uint16_t*>(a.x), static_cast<const uint8_t*>(h2.codes), static_cast<const uint16_t*>(h2.scales),
      (int)a.k);
  return hipGetLastError();
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

int64_t tiled_tpad(int64_t t) { return (t + 31) / 32 * 32; }

bool tiled_shape_ok(int64_t n, int64_t k, int64_t t) {
  const int64_t lim = (int64_t(1) << 31) - 256;
  return tiled_tpad(t) * k * 2 < lim && n * (k / 64) * 2 < lim;
}

// K split factor for a grid of `tiles` workgroup tiles: about `target`
// workgroups in all, at most 8 splits, every split at least 10 groups.
static int pick_ks(int64_t tiles, int64_t target, int64_t k, int64_t t) {
  int64_t ks = target / tiles;
  if (ks > 8) ks = 8;
  if (ks > (k / 64) / 10) ks = (k / 64) / 10;
  if (ks < 1 || t > 4096) ks = 1;
  return (int)ks;
}

TiledConfig tiled_pick_config(int64_t n, int64_t k, int64_t t) {
  if (t <= 32) return TiledConfig{1, 1, 1, 1, 1};
  if (n >= 96 && t > 128 && ((n + 95) / 96) * ((t + 255) / 256) >= 192) return TiledConfig{3, 2, 1, 4, 1};
  if (n >= 192 && t > 128) {
    // 96 x 256 tiles with K split over about 256 workgroups where the tiles
    // alone do not fill the CUs (6144 x 5120: T = 512 53.8 against 60.1 us
    // with 192 x 128 tiles, T = 160 34.4 against 39.2)
    const int64_t tiles = ((n + 95) / 96) * ((t + 255) / 256);
    return TiledConfig{3, 2, 1, 4, pick_ks(tiles, 256, k, t)};
  }
  if (n >= 192) {
    // 192-row tiles (every 32-row tile would read all the activations again),
    // 64 or 128 tokens; with fewer tiles than CUs, K is split (one
    // workgroup per CU: these tiles use most of a CU's registers)
    const bool narrow_t = t <= 64;
    const int64_t tiles = ((n + 191) / 192) * ((t + (narrow_t ? 63 : 127)) / (narrow_t ? 64 : 128));
    const int ks = tiles >= 192 ? 1 : pick_ks(tiles, 256, k, t);
    return narrow_t ? TiledConfig{3, 1, 2, 2, ks} : TiledConfig{3, 2, 2, 2, ks};
  }
  // few rows: 32 x 128 tiles, about three workgroups per CU
  return TiledConfig{1, 1, 1, 4, pick_ks(((n + 31) / 32) * ((t + 127) / 128), 768, k, t)};
}

// Workspace: float16 activations in tile order, then the token exponents,
// then the row exponents, then (K split only) the FP32 partial sums
// [split][Tpad][N].
size_t tiled_workspace_bytes(int64_t n, int64_t k, int64_t t) {
  const int64_t tp = tiled_tpad(t);
  const TiledConfig c = tiled_pick_config(n, k, t);
  const size_t part = c.ks > 1 ? align256((size_t)c.ks * (size_t)tp * (size_t)n * 4) : 0;
  return align256((size_t)(tp * k * 2)) + align256((size_t)(tp * 4)) + align256((size_t)(n * 4)) + part;
}

namespace {

// The activation preparation: X into float16 tiles with the token exponents,
// and the row exponents of the weight (and of a second weight).
hipError_t launch_prep(const TiledArgs& a, u32x4_t* x16, int* texp, int* rexp, const void* scales2, int64_t n2,
                       int* rexp2, hipStream_t stream) {
  const int64_t tp = tiled_tpad(a.t);
  const u32x4_t* x = static_cast<const u32x4_t*>(a.x);
  int k = (int)a.k, t = (int)a.t, n = (int)a.n, tpad = (int)tp;
  const int tok = prep_tokens(a.t);
  const int tok_blocks = (int)(tp / tok);
  const int row_blocks = (int)((a.n + kRowsPerBlock - 1) / kRowsPerBlock);
  const int row_blocks2 = (int)((n2 + kRowsPerBlock - 1) / kRowsPerBlock);
  const int nwv = kPrepThreads / 64;
  const int nj = (int)(((a.k / 8 + nwv - 1) / nwv + 64 / tok - 1) / (64 / tok));  // pieces per lane
  const dim3 grid((unsigned)(tok_blocks + row_blocks + row_blocks2)), block(kPrepThreads);
  const uint16_t* sc = static_cast<const uint16_t*>(a.scales);
  const uint16_t* sc2 = static_cast<const uint16_t*>(scales2);
  const int n2i = (int)n2;
  // longer rows (nj > 10) take the chunked two-pass form of the kernel
  const int mj = nj <= 2 ? 2 : nj <= 5 ? 5 : 10;
  auto launch = [&](auto kern) {
    kern<<<grid, block, 0, stream>>>(x, k, t, tpad, texp, x16, sc, n, rexp, tok_blocks, row_blocks, sc2, n2i, rexp2);
  };
  if (tok == 2) {
    if (mj == 2) launch(prep_act_kernel<2, 2>);
    else if (mj == 5) launch(prep_act_kernel<5, 2>);
    else launch(prep_act_kernel<10, 2>);
  } else {
    if (mj == 2) launch(prep_act_kernel<2, 4>);
    else if (mj == 5) launch(prep_act_kernel<5, 4>);
    else launch(prep_act_kernel<10, 4>);
  }
  return hipGetLastError();
}

hipError_t launch_shape(const TiledArgs& a, const u32x4_t* x16, const int* texp, const int* rexp, float* part,
                        int tpad, hipStream_t stream, const Plane2Host& h2) {
  const TiledConfig c = a.cfg;
  if (c.ns == 3 && c.ts == 2 && c.wn == 2 && c.wt == 2) return launch_cfg<3, 2, 2, 2>(a, x16, texp, rexp, part, tpad, stream, h2);
  if (c.ns == 3 && c.ts == 1 && c.wn == 2 && c.wt == 2) return launch_cfg<3, 1, 2, 2>(a, x16, texp, rexp, part, tpad, stream, h2);
  if (c.ns == 3 && c.ts == 2 && c.wn == 1 && c.wt == 4) return launch_cfg<3, 2, 1, 4>(a, x16, texp, rexp, part, tpad, stream, h2);
  if (c.ns == 1 && c.ts == 1 && c.wn == 1 && c.wt == 4) return launch_cfg<1, 1, 1, 4>(a, x16, texp, rexp, part, tpad, stream, h2);
  if (c.ns == 1 && c.ts == 1 && c.wn == 1 && c.wt == 1) return launch_cfg<1, 1, 1, 1>(a, x16, texp, rexp, part, tpad, stream, h2);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_tiled(const TiledArgs& a, hipStream_t stream) {
  const int64_t tp = tiled_tpad(a.t);
  u32x4_t* x16 = static_cast<u32x4_t*>(a.workspace);
  int* texp = reinterpret_cast<int*>(static_cast<uint8_t*>(a.workspace) + align256((size_t)(tp * a.k * 2)));
  int* rexp = reinterpret_cast<int*>(reinterpret_cast<uint8_t*>(texp) + align256((size_t)(tp * 4)));
  float* part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(rexp) + align256((size_t)(a.n * 4)));
  hipError_t e = launch_prep(a, x16, texp, rexp, nullptr, 0, nullptr, stream);
  if (e != hipSuccess) return e;
  return launch_shape(a, x16, texp, rexp, part, (int)tp, stream, Plane2Host{});
}

// Pair workspace: activations, token exponents, row exponents of each
// weight, then (K split or binary32 sums) each weight's partials
// [split][Tpad][N].
size_t tiled_pair_workspace_bytes(int64_t n1, int64_t n2, int64_t k, int64_t t, bool f32) {
  const int64_t tp = tiled_tpad(t);
  const TiledConfig c = tiled_pick_config(n1 + n2, k, t);
  const bool keep = c.ks > 1 || f32;
  return align256((size_t)(tp * k * 2)) + align256((size_t)(tp * 4)) + align256((size_t)(n1 * 4)) +
         align256((size_t)(n2 * 4)) + (keep ? align256((size_t)c.ks * (size_t)tp * (size_t)n1 * 4) : 0) +
         (keep ? align256((size_t)c.ks * (size_t)tp * (size_t)n2 * 4) : 0);
}

hipError_t launch_tiled_pair(const TiledPairArgs& p, SumSource* src1, SumSource* src2, hipStream_t stream) {
  const TiledArgs& a = p.a;
  const int64_t tp = tiled_tpad(a.t);
  uint8_t* w = static_cast<uint8_t*>(a.workspace);
  u32x4_t* x16 = reinterpret_cast<u32x4_t*>(w);
  w += align256((size_t)(tp * a.k * 2));
  int* texp = reinterpret_cast<int*>(w);
  w += align256((size_t)(tp * 4));
  int* rexp1 = reinterpret_cast<int*>(w);
  w += align256((size_t)(a.n * 4));
  int* rexp2 = reinterpret_cast<int*>(w);
  w += align256((size_t)(p.n2 * 4));
  const bool keep = a.cfg.ks > 1 || a.f32;
  float* part1 = reinterpret_cast<float*>(w);
  w += keep ? align256((size_t)a.cfg.ks * (size_t)tp * (size_t)a.n * 4) : 0;
  float* part2 = reinterpret_cast<float*>(w);
  hipError_t e = launch_prep(a, x16, texp, rexp1, p.scales2, p.n2, rexp2, stream);
  if (e != hipSuccess) return e;
  Plane2Host h2;
  h2.codes = p.codes2;
  h2.scales = p.scales2;
  h2.y = p.y2;
  h2.part = part2;
  h2.rexp = rexp2;
  h2.n = p.n2;
  if (src1 != nullptr) *src1 = SumSource{part1, texp, rexp1, a.cfg.ks, (size_t)tp * (size_t)a.n};
  if (src2 != nullptr) *src2 = SumSource{part2, texp, rexp2, a.cfg.ks, (size_t)tp * (size_t)p.n2};
  return launch_shape(a, x16, texp, rexp1, part1, (int)tp, stream, h2);
}

// LinearSwiGLU in one tiled launch after the activation preparation: every
// 96-row tile takes 48 rows of the gate and the same 48 rows of the up
// weight and forms bf16(silu(G) U) in its epilogue from the same binary32
// sums, scaled and combined as the two-pass form does (no partials, no
// combine pass).  Only where the 2N-row problem takes the 96 x 256 tiles
// without a K split.
bool tiled_glu_ok(int64_t n, int64_t k, int64_t t) {
  const TiledConfig c = tiled_pick_config(2 * n, k, t);
  return c.ns == 3 && c.ts == 2 && c.wn == 1 && c.wt == 4 && c.ks == 1 && tiled_shape_ok(n, k, t);
}

// Workspace: the activations, the token exponents, each weight's row exponents.
size_t tiled_glu_workspace_bytes(int64_t n, int64_t k, int64_t t) {
  const int64_t tp = tiled_tpad(t);
  return align256((size_t)(tp * k * 2)) + align256((size_t)(tp * 4)) + 2 * align256((size_t)(n * 4));
}

hipError_t launch_tiled_glu(const TiledArgs& a, const void* codes_up, const void* scales_up, hipStream_t stream) {
  using Sh = TiledShape<3, 2, 1, 4>;
  constexpr int BH = Sh::BN / 2;
  constexpr size_t kGluLds = (size_t)Sh::BT * Sh::BN * 4 + (size_t)(Sh::BT + Sh::BN) * 4;
  const int64_t tp = tiled_tpad(a.t);
  uint8_t* w = static_cast<uint8_t*>(a.workspace);
  u32x4_t* x16 = reinterpret_cast<u32x4_t*>(w);
  w += align256((size_t)(tp * a.k * 2));
  int* texp = reinterpret_cast<int*>(w);
  w += align256((size_t)(tp * 4));
  int* rexp_g = reinterpret_cast<int*>(w);
  w += align256((size_t)(a.n * 4));
  int* rexp_u = reinterpret_cast<int*>(w);
  hipError_t e = launch_prep(a, x16, texp, rexp_g, scales_up, a.n, rexp_u, stream);
  if (e != hipSuccess) return e;
  auto kern = tiled_kernel<3, 2, 1, 4, false, true>;
  e = allow_full_lds(reinterpret_cast<const void*>(kern));
  if (e != hipSuccess) return e;
  const int tiles_n = (int)((a.n + BH - 1) / BH);
  const int tiles_t = (int)((a.t + Sh::BT - 1) / Sh::BT);
  TiledPlane2 p2;
  p2.codes = static_cast<const uint8_t*>(codes_up);
  p2.scales = static_cast<const uint16_t*>(scales_up);
  p2.rexp = rexp_u;
  p2.n = (int)a.n;
  const size_t lds = (size_t)Sh::LDS_B > kGluLds ? (size_t)Sh::LDS_B : kGluLds;
  kern<<<dim3((unsigned)(tiles_n * tiles_t)), dim3(Sh::NT), lds, stream>>>(
      x16, texp, rexp_g, static_cast<const uint16_t*>(a.x), static_cast<const uint8_t*>(a.codes),
      static_cast<const uint16_t*>(a.scales), static_cast<uint16_t*>(a.y), nullptr, (int)a.n, (int)a.k, (int)a.t,
      (int)tp, tiles_n, tiles_t, 1, nullptr, p2);
  return hipGetLastError();
}

}  // namespace q4lin
