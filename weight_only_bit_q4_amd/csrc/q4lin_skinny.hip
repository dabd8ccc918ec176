// q4lin_skinny.hip -- the small-T route: W streamed once, matrix cores over
// all tokens, K split across the waves of a workgroup.
//
// The pages' prior art for T = 2..24 splits K so that a weight tile is read
// once for several token columns ("q4-linear.md", notes under the result
// table); this is an MI355X design of that step, extended to T <= 32.
//
// Work mapping.  One workgroup per block of BN consecutive rows (BN about
// N / 256, so the grid is one workgroup per CU) covers the whole of K; its
// eight waves split the 64-groups of K into eight contiguous slices.  A wave
// therefore reads every code byte of its slice exactly once and each
// activation of its slice once, and no wave ever waits for another until the
// final eight-way sum.  Rows of a block are contiguous in memory, so the wave
// loads its slice in row-major 16-byte pieces (runs of 128 bytes per row, the
// access pattern the memory system serves best), parks them in a private LDS
// region, and reads them back in matrix-core operand order.
//
// Arithmetic (v_mfma_f32_16x16x32_bf16, A = activations, B = weights).
//   * Weights: one (a & m) | c (v_bitop3) turns nibbles s and s+16 of a code dword into the
//     bf16 pair (128 + q, 128 + q') exactly (bf16 has unit spacing on
//     [128, 256)); four such operations give the 8 operand values of one
//     dword in the order k0 k4 k1 k5 k2 k6 k3 k7.
//   * Activations go to the matrix cores as they are (bf16), each 16-byte
//     run permuted into that same order with v_perm_b32.
//   * P' = sum (128 + q) x and the correction C = sum 136 x come from the same
//     matrix-core instruction sequence (C uses a constant all-136 operand), so
//     P' - C = sum (q - 8) x, and a group of eight-codes gives exactly 0.  The
//     group's scale is applied in FP32: acc += s * (P' - C).
//   * Each lane's four accumulators share one weight row (one scale).
//   * If a wave's sums leave the FP32 range (activations near the bf16
//     maximum), the wave recomputes its slice with every token scaled by a
//     power of two found from the token's largest magnitude, and undoes it in
//     binary64 in the final sum.
//   * The eight wave partials are summed in binary64 and rounded to bf16 once.
//
// Operand placement.  A 64-byte piece pair of a row (two 64-groups) arrives
// as four 16-byte pieces on lanes q = 0..3 of the row's column; two
// v_permlane32_swap_b32 give every lane one dword of each group, so each
// matrix-core instruction reduces over a single group:
//   instruction "a" takes dword {2,6,0,4}[q] of the group, "b" {3,7,1,5}[q].
#include "q4lin_device.h"
#include "q4lin_kernels.h"

namespace q4lin {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kStepGroups = 4;  // 64-groups per pipeline step (128 bytes of each row)

// Direct-to-LDS buffer loads: every lane sends 16 bytes from base + voffset +
// soffset to lds_base + 16 * lane (lds_base wave-uniform); offsets at or past
// the resource's byte count read zeros without a memory access.
using rsrc_t = __amdgpu_buffer_rsrc_t;

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

// s_waitcnt immediate for gfx9: vmcnt in bits 3:0 and 15:14, expcnt 6:4 (7 =
// no wait), lgkmcnt 11:8 (15 = no wait).
// steps in flight: three while the ring fits the LDS comfortably
constexpr int ring_depth(int ct) { return ct <= 2 ? 3 : 2; }

constexpr int vmcnt_imm(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }

// (a & m) | c in one instruction: gfx950's three-input bitwise operation with
// truth table 0xEA.  A builtin rather than inline assembly, so the compiler
// knows the instruction when it spaces matrix-core operand reads after
// vector-ALU writes.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, m, c, 0xEA);
}

// (128 + q) bf16 operand values of one code dword, order k0 k4 k1 k5 k2 k6 k3 k7
__device__ __forceinline__ bf16x8_t bf16_codes(uint32_t w) {
  u32x4_t r;
  r.x = and_or(w, 0x000F000Fu, 0x43004300u);
  r.y = and_or(w >> 4, 0x000F000Fu, 0x43004300u);
  r.z = and_or(w >> 8, 0x000F000Fu, 0x43004300u);
  r.w = and_or(w >> 12, 0x000F000Fu, 0x43004300u);
  return __builtin_bit_cast(bf16x8_t, r);
}

// 8 consecutive bf16 activations (x0..x7 as 4 dwords) -> order x0 x4 x1 x5 x2 x6 x3 x7
__device__ __forceinline__ bf16x8_t act_order(u32x4_t v) {
  u32x4_t r;
  r.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
  r.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
  r.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
  r.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
  return __builtin_bit_cast(bf16x8_t, r);
}

// 8 bf16 values times 2^-e (exact unless a value falls below the bf16 normal
// range, where it rounds; such values are far below the tolerance).
__device__ __forceinline__ u32x4_t scale_bf16x8(u32x4_t v, int e) {
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __builtin_ldexpf(bf16_bits_to_f32(v[i] & 0xFFFFu), -e);
    const float hi = __builtin_ldexpf(bf16_bits_to_f32(v[i] >> 16), -e);
    r[i] = (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
  }
  return r;
}

__device__ __forceinline__ uint32_t max_mag8(u32x4_t v) {
  uint32_t m = max(max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu), max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu));
  return max(m, max(max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu), max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu)));
}

// dword of a 64-group used by lane quarter q in instruction a / b
__device__ __forceinline__ int dword_a(int q) { return (q & 1) * 4 + ((q >> 1) ? 0 : 2); }
__device__ __forceinline__ int dword_b(int q) { return dword_a(q) + 1; }

// CT: 16-row column tiles, TT: 16-token tiles, NL: direct-to-LDS code loads
// per lane per step (8 rows each), DEPTH: steps in flight
template <int CT, int TT, int NL, int DEPTH>
__global__ void __launch_bounds__(kThreads, 1)
skinny_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes,
              const uint16_t* __restrict__ scales, uint16_t* y,
              int N, int K, int T, int BN, int off_codes, int off_red, const uint16_t* res, SecondPlane p2) {
  constexpr int BNP = 16 * CT;  // matrix-core columns (rows of W) per workgroup
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  // LDS: the block's scales (fp16 [BNP][G] from byte s_delta), then the
  // waves' code rings; the final sums reuse the rings.
  const int G = K >> 6;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  int bid = blockIdx.x;
  if (p2.n > 0 && bid >= p2.first) {  // LinearPair: the second weight
    codes = p2.codes;
    scales = p2.scales;
    y = p2.y;
    N = p2.n;
    res = nullptr;  // a pair carries no residual
    bid -= p2.first;
  }
  const int n0 = bid * BN;
  const int rows = min(BN, N - n0);  // real rows of this block (>= 1)

  // --- this wave's slice of K, in steps of four 64-groups -------------------
  // A step is 128 bytes of every row of the block: eight 16-byte pieces per
  // row, fetched by NL direct-to-LDS loads per lane (each instruction reads 8
  // rows x 128 contiguous bytes), so the block's rows stream as long runs.
  // Steps land in a ring of DEPTH slots of the wave's LDS region, DEPTH steps
  // ahead, and are read back in matrix-core operand order.  Piece pc of row r
  // sits in 16-byte slot 8 r + (pc ^ ((r >> 1) & 7)) of its step, which makes
  // the operand reads (16 rows, one piece each) free of bank conflicts.
  const int gl = (G * wave) / kWaves, gh = (G * (wave + 1)) / kWaves;
  const int ng = gh - gl;
  const int nsteps = (ng + kStepGroups - 1) / kStepGroups;
  constexpr int STEP_B = NL * 1024;  // LDS bytes per ring slot
  // the wave's LDS area: the code ring, then its own copy of the scales of
  // its slice (SW dwords per row, enough for the slice at any alignment)
  const int SW = (2 * ((G + kWaves - 1) / kWaves) + 3) / 4 + 1;
  const int wave_b = DEPTH * STEP_B + ((BNP * SW * 4 + 255) & ~255);  // whole 64-lane copies
  uint8_t* cw = lds + off_codes + wave * wave_b;
  uint8_t* sw = cw + DEPTH * STEP_B;
  // Buffer over the whole code plane: slots past the block's rows use an
  // offset beyond it and read zeros without touching memory; pieces of
  // groups past the slice read a neighbour's codes (their scale is 0).
  const rsrc_t rc = make_rsrc(codes, (uint32_t)((size_t)N * (size_t)(K >> 1)));
  uint32_t voff[NL];
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int sl = lane + 64 * j;
    const int r = sl >> 3, pc = (sl & 7) ^ ((r >> 1) & 7);
    voff[j] = (r < BN && n0 + r < N) ? (uint32_t)(n0 + r) * (uint32_t)(K >> 1) + (uint32_t)pc * 16u : 0x80000000u;
  }
  // Steps past the slice are still issued (every step issues the same loads,
  // so the waits below are fixed counts) but read nothing: their offset lies
  // beyond the buffer.
  auto issue = [&](int st) __device__ {
    uint8_t* dst = cw + (st % DEPTH) * STEP_B;
    const uint32_t so = st < nsteps ? (uint32_t)(gl + st * kStepGroups) * 32u : 0x80000000u;
#pragma unroll
    for (int j = 0; j < NL; ++j) dma16(rc, voff[j], so, dst + j * 1024);
  };

  // activation operand rows of this lane: token li + 16 tt
  const int da = dword_a(lq), db = dword_b(lq);
  const uint32_t k136 = 0x43084308u;  // bf16 136.0 pair
  const bf16x8_t b136 = __builtin_bit_cast(bf16x8_t, u32x4_t{k136, k136, k136, k136});

  // reads of the wave's code pieces in operand order: tile ct, lane (li, lq)
  // reads piece 4 p + lq of row 16 ct + li (rows past the block read row 0;
  // their scales are 0)
  int rd_row[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int r = 16 * ct + li < BN ? 16 * ct + li : 0;
    rd_row[ct] = r;
  }
  // scale of (row 16 ct + li, group g) at s_row[ct] + 2 g (rows past the
  // block hold other rows' scales or zeros; they are never stored)
  const uint8_t* s_row[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int r = 16 * ct + li;
    const uint32_t b = (uint32_t)(n0 + r) * (uint32_t)G * 2u + (uint32_t)gl * 2u;
    s_row[ct] = sw + 4 * SW * r + (b & 3u) - 2 * gl;
  }
  auto rd_addr = [&](int st, int ct, int p) __device__ {
    const int r = rd_row[ct];
    return cw + (st % DEPTH) * STEP_B + 16 * (8 * r + ((4 * p + lq) ^ ((r >> 1) & 7)));
  };

  f32x4_t acc[CT][TT];
  int ex[TT];  // per-token exponent of the activation operands (A layout)

  // activation pieces of one pair of groups: [group 0/1][instr a/b][tt].
  // Operand rows of tokens past T repeat token T-1: their product rows are
  // never stored, and the loads stay unconditional.
  auto load_x = [&](int g0, u32x4_t (&xv)[2][2][TT]) __device__ {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const int t = min(li + 16 * tt, T - 1);
        const int g = min(g0 + h, gh - 1);
        const uint16_t* xr = x + (size_t)t * K + 64 * g;
        xv[h][0][tt] = *reinterpret_cast<const u32x4_t*>(xr + 8 * da);
        xv[h][1][tt] = *reinterpret_cast<const u32x4_t*>(xr + 8 * db);
      }
  };

  // products of one pair of groups (g0, g0 + 1), code pieces cp (one 16-byte
  // piece per lane and column tile)
  auto pair_products = [&](int g0, u32x4_t (&cp)[CT], bool scaled, const u32x4_t (&xa)[2][2][TT]) __device__ {
    // regroup: v[2], v[3] hold group g0 and v[0], v[1] group g0 + 1 on every lane
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      auto s02 = __builtin_amdgcn_permlane32_swap(cp[ct].z, cp[ct].x, false, false);
      auto s13 = __builtin_amdgcn_permlane32_swap(cp[ct].w, cp[ct].y, false, false);
      cp[ct] = u32x4_t{s02[1], s13[1], s02[0], s13[0]};
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int g = g0 + h;
      bf16x8_t av[2][TT];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          av[m][tt] = act_order(scaled ? scale_bf16x8(xa[h][m][tt], ex[tt]) : xa[h][m][tt]);
      // corrections C = sum 136 x per token (same instruction sequence)
      f32x4_t cr[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        cr[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[0][tt], b136, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        cr[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[1][tt], b136, cr[tt], 0, 0, 0);
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const uint32_t wa = h == 0 ? cp[ct].z : cp[ct].x;
        const uint32_t wb = h == 0 ? cp[ct].w : cp[ct].y;
        const bf16x8_t ba = bf16_codes(wa), bb = bf16_codes(wb);
        const float sc = g < gh ? f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(s_row[ct] + 2 * g)) : 0.0f;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          f32x4_t pr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[0][tt], ba, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          pr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[1][tt], bb, pr, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[ct][tt][r] = __builtin_fmaf(sc, pr[r] - cr[tt][r], acc[ct][tt][r]);
        }
      }
    }
  };

  // activations of the two pairs of a step
  auto load_xs = [&](int st, u32x4_t (&xv)[2][2][2][TT]) __device__ {
#pragma unroll
    for (int p = 0; p < 2; ++p) load_x(gl + st * kStepGroups + 2 * p, xv[p]);
  };

  // Step st issues the activations of step st + 1 (8 TT loads) and the codes
  // of step st + DEPTH (NL loads; past the slice they read nothing).  So when step st starts, the loads younger
  // than its codes that may still be in flight are the codes of the DEPTH - 1
  // later steps and the activations of step st (older activations have been
  // used, hence have landed): waiting until no more than NL (DEPTH - 1) +
  // 8 TT loads are outstanding means its codes have landed.
  // last: the slice's final step, which prefetches nothing.
  auto step = [&](int st, bool scaled, bool last, const u32x4_t (&xcur)[2][2][2][TT],
                  u32x4_t (&xnext)[2][2][2][TT]) __device__ {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(NL * (DEPTH - 1) + 8 * TT));
    __builtin_amdgcn_sched_barrier(0);
    u32x4_t cp[kStepGroups / 2][CT];
#pragma unroll
    for (int p = 0; p < kStepGroups / 2; ++p)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) cp[p][ct] = *reinterpret_cast<const u32x4_t*>(rd_addr(st, ct, p));
    // the slot is free once the reads are back; refill it with step st + DEPTH
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (!last) {
      load_xs(st + 1, xnext);
      issue(st + DEPTH);
    }
    __builtin_amdgcn_sched_barrier(0);
    const int gs = gl + st * kStepGroups;
#pragma unroll
    for (int p = 0; p < kStepGroups / 2; ++p)
      if (gs + 2 * p < gh) pair_products(gs + 2 * p, cp[p], scaled, xcur[p]);
  };

  // The slice's first DEPTH code steps and first activations (issued
  // before anything waits).
  // Step 0's codes must be issued before step 0's activations (its wait
  // counts the activations among the younger loads), so the scheduler may
  // not move them across.
  auto prologue = [&](u32x4_t (&xs)[2][2][2][TT]) __device__ {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) issue(d);
    __builtin_amdgcn_sched_barrier(0);
    load_xs(0, xs);
    __builtin_amdgcn_sched_barrier(0);
  };

  // One pass over the slice, prologue already issued.  scaled: activations
  // times 2^-ex[tt].
  auto run = [&](bool scaled, u32x4_t (&xs0)[2][2][2][TT]) __device__ {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) acc[ct][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (ng <= 0) return;
    u32x4_t xs1[2][2][2][TT];
    // steps in pairs (the two activation buffers alternate), the last one or
    // two peeled so that nothing past the slice is fetched
    int st = 0;
    for (; st + 2 < nsteps; st += 2) {
      step(st, scaled, false, xs0, xs1);
      step(st + 1, scaled, false, xs1, xs0);
    }
    if (st + 2 == nsteps) {
      step(st, scaled, false, xs0, xs1);
      step(st + 1, scaled, true, xs1, xs0);
    } else {
      step(st, scaled, true, xs0, xs1);
    }
    // the trailing code copies (past the slice: zeros, no memory traffic)
    // must land before the LDS is used otherwise
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_sched_barrier(0);
  };

  // --- the scales of the wave's slice, then its first steps ------------------
  // Each wave copies the dwords holding its slice's scales for the block's
  // BNP rows (rows past N read zeros) into its own LDS area.  These copies are
  // issued first, so step 0's wait covers them: no barrier, and no wave waits
  // for another's memory traffic.
  u32x4_t xs0[2][2][2][TT];
  if (ng > 0) {
    // the byte count rounded up to whole dwords: the copy moves aligned
    // dwords, and the one holding the last scale must not read as zero (an
    // aligned dword never leaves the page of its first byte)
    const rsrc_t rs = make_rsrc(scales, (uint32_t)(((size_t)N * (size_t)G * 2 + 3) & ~(size_t)3));
    const int nd = BNP * SW;
    __builtin_amdgcn_sched_barrier(0);
    for (int i = 0; 64 * i < nd; ++i) {
      const int d = min(64 * i + lane, nd - 1);
      const int r = d / SW, j = d - r * SW;
      const uint32_t b = ((uint32_t)(n0 + r) * (uint32_t)G * 2u + (uint32_t)gl * 2u) & ~3u;
      dma4(rs, b + 4u * (uint32_t)j, 0u, sw + 256 * i);
    }
    __builtin_amdgcn_sched_barrier(0);
    prologue(xs0);
  }

#pragma unroll
  for (int tt = 0; tt < TT; ++tt) ex[tt] = 0;
  run(false, xs0);

  // Sums beyond the FP32 range: recompute this wave's slice with scaled tokens.
  // (Only entries that are stored count: padding rows and tokens may hold
  // anything.)
  bool bad = false;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (16 * ct + li < rows && 16 * tt + 4 * lq + r < T) bad |= !(__builtin_fabsf(acc[ct][tt][r]) <= 3.0e38f);
  const bool rerun = __builtin_amdgcn_ballot_w64(bad) != 0;
  if (rerun) {
    // exponent per token over this wave's slice: largest magnitude in [1, 2)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int t = li + 16 * tt;
      uint32_t m = 0;
      if (t < T)
        for (int k8 = 64 * gl / 8 + lq; k8 < 64 * gh / 8; k8 += 4)
          m = max(m, max_mag8(*reinterpret_cast<const u32x4_t*>(x + (size_t)t * K + 8 * k8)));
      m = max(m, (uint32_t)__shfl_xor((int)m, 16));
      m = max(m, (uint32_t)__shfl_xor((int)m, 32));
      if (m >= 0x7F80u) m = 0x7F7Fu;  // Inf/NaN inputs are outside the contract
      ex[tt] = m >= 0x80u ? (int)(m >> 7) - 127 : 0;
    }
    if (ng > 0) prologue(xs0);
    run(true, xs0);
  }

  // --- eight-way sum in binary64 ----------------------------------------------
  // red: [wave][t < T][col < BN] binary64 (the partial times 2^ex of its token)
  __syncthreads();
  double* red = reinterpret_cast<double*>(lds + off_red);
  int* ex_lds = reinterpret_cast<int*>(red + kWaves * T * BN) + wave * 16 * TT;
  if (lq == 0) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) ex_lds[li + 16 * tt] = ex[tt];
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's exponents are written
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int col = 16 * ct + li;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tt + 4 * lq + r;
        if (col < BN && t < T)
          red[(wave * T + t) * BN + col] = __builtin_ldexp((double)acc[ct][tt][r], ex_lds[t]);
      }
  }
  __syncthreads();
  for (int i = tid; i < T * rows; i += kThreads) {
    const int t = i / rows, col = i - t * rows;
    double v = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += red[(w * T + t) * BN + col];
    if (res != nullptr) v += (double)bf16_bits_to_f32(res[(size_t)t * N + n0 + col]);  // LinearAdd
    if (p2.f32) reinterpret_cast<float*>(y)[(size_t)t * N + n0 + col] = (float)v;  // LinearSwiGLU sums
    else y[(size_t)t * N + n0 + col] = f32_to_bf16_rne((float)v);
  }
}

template <int CT, int TT>
hipError_t launch_ct(const SkinnyPlan& p, const GemvArgs& a, hipStream_t stream) {
  auto kern = skinny_kernel<CT, TT, 2 * CT, ring_depth(CT)>;
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(kern));
  if (e != hipSuccess) return e;
  const int blocks1 = (int)((a.n + p.bn - 1) / p.bn), blocks2 = (int)((a.n2 + p.bn - 1) / p.bn);
  kern<<<dim3((unsigned)(blocks1 + blocks2)), dim3(kThreads), p.lds_bytes, stream>>>(
      static_cast<const uint16_t*>(a.x), static_cast<const uint8_t*>(a.codes),
      static_cast<const uint16_t*>(a.scales), static_cast<uint16_t*>(a.y), (int)a.n, (int)a.k, (int)a.t,
      p.bn, p.off_codes, p.off_red, static_cast<const uint16_t*>(a.res), second_plane(a, blocks1));
  return hipGetLastError();
}


}  // namespace

bool skinny_plan(int64_t n, int64_t k, int64_t t, SkinnyPlan* p) {
  if (t < 1 || t > 32 || n < 1 || k < 64) return false;
  if (n * (k / 2) >= (int64_t(1) << 31)) return false;  // 32-bit code offsets
  const int64_t G = k / 64;
  int64_t bn = (n + 255) / 256;
  if (bn < 8) bn = 8;
  if (bn > n) bn = n;
  const int64_t ct = (bn + 15) / 16;
  const int64_t tt = t > 16 ? 2 : 1;
  if (ct * tt > 4) return false;  // accumulators and operands must fit the registers
  const int64_t sw = (2 * ((G + kWaves - 1) / kWaves) + 3) / 4 + 1;  // scale dwords per row and wave
  const size_t wave_b = (size_t)ring_depth((int)ct) * (size_t)(2 * ct) * 1024 + (size_t)((16 * ct * sw * 4 + 255) & ~255);
  const size_t codes_b = (size_t)kWaves * wave_b;
  const size_t sc = 0;
  const size_t red_b = (size_t)kWaves * (size_t)t * (size_t)bn * 8 + (size_t)kWaves * 16 * 2 * 4;
  const size_t lds = sc + (codes_b > red_b ? codes_b : red_b);
  if (lds > 160 * 1024) return false;
  p->bn = (int)bn;
  p->ct = (int)ct;
  p->tt = (int)tt;
  p->blocks = (int)((n + bn - 1) / bn);
  p->off_codes = (int)sc;
  p->off_red = (int)sc;
  p->lds_bytes = lds;
  return true;
}

hipError_t launch_skinny(const GemvArgs& a, hipStream_t stream) {
  SkinnyPlan p;
  if (!skinny_plan(a.n + a.n2, a.k, a.t, &p)) return hipErrorInvalidValue;
  if (p.tt == 1) {
    switch (p.ct) {
      case 1: return launch_ct<1, 1>(p, a, stream);
      case 2: return launch_ct<2, 1>(p, a, stream);
      case 3: return launch_ct<3, 1>(p, a, stream);
      case 4: return launch_ct<4, 1>(p, a, stream);
    }
  } else {
    switch (p.ct) {
      case 1: return launch_ct<1, 2>(p, a, stream);
      case 2: return launch_ct<2, 2>(p, a, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace q4lin
