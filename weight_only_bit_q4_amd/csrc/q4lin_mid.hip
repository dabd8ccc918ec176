// q4lin_mid.hip -- the medium-T route: T = 17..128 tokens on one weight
// stream, matrix cores on exact codes, no activation-preparation pass.
//
// The pages' prior art between the K-split "capacity" kernels and the large
// tiles is a 32x32 / 32x64 tiled MMA for T = 25..192 ("q4-linear.md", notes
// under the result table).  This is an MI355X design of that step.
//
// Work mapping.  The weight is cut into row blocks of BN rows and K into S
// slices, about one workgroup per CU in all; workgroup (row block, slice)
// reads its BN x K/S codes exactly once and its K/S slice of every token's
// activations once.  Its eight waves form a WR x WT grid over BN rows x BT
// tokens (BT >= T): wave (wr, wt) owns 16 CT rows x 16 TT tokens for all of
// the slice.  Partial sums of the S slices go to the workspace in binary32
// and a second kernel adds them in slice order (S = 1 writes y directly).
//
// Data movement.  The first CW waves load all of the block's codes for the
// slice into LDS at once (pairs of 64-groups: 64 contiguous bytes of every
// row per pair, 16-byte direct-to-LDS loads, in pair order); the other waves
// stream the activations, one 64-group of every token (128 contiguous bytes
// per token) per step through a ring of DX + 1 slots, DX groups ahead, after
// loading the block's scales into an LDS table.  The two kinds of loads are
// issued by different waves, so a code wave waits only for the pair a step
// needs and an activation wave for one fixed count per step (a wave's loads
// complete in order).  One barrier per 64-group step
// publishes both rings.  LDS slots are XOR-swizzled in 16-byte pieces so the
// matrix-core operand reads (16 rows or 16 tokens at 64 / 128-byte strides)
// spread over the banks.
//
// Arithmetic (v_mfma_f32_16x16x32_bf16, A = activations, B = weights; every
// instruction reduces over half a group):
//   * one three-input bitwise operation per pair of codes gives the exact
//     bf16 pair (128 + q, 128 + q') in the order (k0,k4) (k1,k5) (k2,k6)
//     (k3,k7) of a code dword; the activation fragment is permuted into the
//     same order;
//   * the sums P = sum (128 + q) x and C = sum 136 x come from the same
//     instruction sequence (C on a constant operand), so P - C = sum (q-8) x
//     exactly for a group of eight-codes (0); the group's scale is applied in
//     binary32: acc += s (P - C);
//   * outputs whose binary32 arithmetic leaves the range (activations near
//     the bf16 maximum) are formed again exactly by their thread.
#include "q4lin_device.h"
#include "q4lin_kernels.h"

namespace q4lin {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
using rsrc_t = __amdgpu_buffer_rsrc_t;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxSliceGroups = 32;
constexpr int kMaxSplits = 8;
constexpr size_t kLdsLimit = 160 * 1024;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16-byte direct-to-LDS buffer load: each active lane sends 16 bytes from
// base + voffset to lds_base + 16 * lane (lds_base wave-uniform); offsets at
// or past the resource's byte count read zeros
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voffset, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, voffset, 0,
                                           0, 0);
}

// s_waitcnt for gfx9: vmcnt in bits 3:0 and 15:14, expcnt 6:4 (7 = no wait),
// lgkmcnt 11:8 (15 = no wait)
constexpr int vmcnt_imm(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
}
// wait until at most about n loads are outstanding (n rounded down to a
// multiple of 8: s_waitcnt takes an immediate, and waiting for a few more
// loads than needed is only slower)
__device__ __forceinline__ void wait_vm_atmost(int n) {
  switch (min(n, 63) >> 3) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<8>(); break;
    case 2: wait_vm<16>(); break;
    case 3: wait_vm<24>(); break;
    case 4: wait_vm<32>(); break;
    case 5: wait_vm<40>(); break;
    case 6: wait_vm<48>(); break;
    default: wait_vm<56>(); break;
  }
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4)); }

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, m, c, 0xEA);
}

// (128 + q) bf16 values of one code dword, order k0 k4 k1 k5 k2 k6 k3 k7
__device__ __forceinline__ bf16x8_t bf16_codes(uint32_t w) {
  u32x4_t r;
  r.x = and_or(w, 0x000F000Fu, 0x43004300u);
  r.y = and_or(w >> 4, 0x000F000Fu, 0x43004300u);
  r.z = and_or(w >> 8, 0x000F000Fu, 0x43004300u);
  r.w = and_or(w >> 12, 0x000F000Fu, 0x43004300u);
  return __builtin_bit_cast(bf16x8_t, r);
}

// 8 consecutive bf16 activations -> order x0 x4 x1 x5 x2 x6 x3 x7
__device__ __forceinline__ bf16x8_t pair_order(u32x4_t v) {
  u32x4_t r;
  r.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
  r.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
  r.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
  r.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
  return __builtin_bit_cast(bf16x8_t, r);
}

// piece swizzles: code piece pc (0..3) of row r; activation piece pc (0..7) of token t
__device__ __forceinline__ int cswz(int r) { return (r >> 1) & 3; }
__device__ __forceinline__ int xswz(int t) { return t & 7; }

// CT x TT: 16-row x 16-token tiles per wave; WR x WT: the waves' grid; CW:
// code-loading waves (the other 8 - CW load the activations); DX: activation
// groups loaded ahead (a ring of DX + 1 slots).
template <int CT, int TT, int WR, int WT, int CW, int DX>
struct MidShape {
  static constexpr int BN = 16 * CT * WR;                 // rows per workgroup
  static constexpr int BT = 16 * TT * WT;                 // tokens per workgroup (>= T)
  static constexpr int LC = 64 * CW, LX = 64 * (kWaves - CW);  // loader lanes of each kind
  static constexpr int PAIR_B = BN * 64;                  // one code pair [row][64 bytes]
  static constexpr int CI = BN * 4 / LC;                  // loads per code wave per pair
  static constexpr int XG_B = BT * 128;                   // one activation slot [token][128 bytes]
  static constexpr int XI = BT * 8 / LX;                  // loads per activation wave per group
  static constexpr int SV = (BN * kMaxSliceGroups + LX - 1) / LX;  // scale loads per lane, at most
  static_assert(WR * WT == kWaves, "eight waves");
  static_assert(BN * 4 % LC == 0 && BT * 8 % LX == 0, "slots split into whole loads");
  static_assert((DX - 1) * XI <= 63 && DX * XI <= 63, "the load counter holds 63");
  // LDS: every code pair of the slice, then the activation ring, then the
  // scale table [BN][GSP] fp16
  __host__ __device__ static size_t off_x(int npairs) { return (size_t)npairs * PAIR_B; }
  __host__ __device__ static size_t off_s(int npairs) { return off_x(npairs) + (size_t)(DX + 1) * XG_B; }
  __host__ __device__ static size_t lds_bytes(int npairs, int gsp) { return off_s(npairs) + (size_t)BN * gsp * 2; }
};

template <int CT, int TT, int WR, int WT, int CW, int DX>
__global__ void __launch_bounds__(kThreads, 1)
mid_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
           uint16_t* y, float* __restrict__ part, int N, int K, int T, int S, int GSP, int nrb,
           const uint16_t* res, int f32out) {
  using Sh = MidShape<CT, TT, WR, WT, CW, DX>;
  constexpr int BN = Sh::BN, CI = Sh::CI, XI = Sh::XI, LC = Sh::LC, LX = Sh::LX;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const int G = K >> 6;
  // workgroup: row block rb, K slice ks (slices adjacent in the grid share
  // their row block's codes' DRAM pages; rows vary slowest)
  const int ks = blockIdx.x % S, rb = blockIdx.x / S;
  (void)nrb;
  const int n0 = rb * BN;
  const int g0 = (int)(((int64_t)G * ks) / S), gs = (int)(((int64_t)G * (ks + 1)) / S) - g0;
  const int npairs = (gs + 1) >> 1;
  const int last_row = N - 1 - n0;  // rows past it repeat it (never stored)

  const bool code_wave = wave < CW;
  const int lw = code_wave ? wave : wave - CW;  // index among the loader waves of its kind
  uint8_t* const xring = lds + Sh::off_x(npairs);
  uint16_t* const stab = reinterpret_cast<uint16_t*>(lds + Sh::off_s(npairs));

  // --- loads -----------------------------------------------------------------
  const rsrc_t rc = make_rsrc(codes, (uint32_t)((size_t)N * (size_t)(K >> 1)));
  const rsrc_t rx = make_rsrc(x, (uint32_t)((size_t)T * (size_t)K * 2));
  // code wave: load i of pair p moves piece s = i LC + 64 lw + lane of the
  // pair's [row][4 pieces]; piece (r, pc ^ cswz(r)) holds piece pc of row r
  uint32_t coff[CI];
#pragma unroll
  for (int i = 0; i < CI; ++i) {
    const int s = i * LC + lw * 64 + lane;
    const int r = s >> 2, pc = (s & 3) ^ cswz(r);
    coff[i] = (uint32_t)(n0 + min(r, last_row)) * (uint32_t)(K >> 1) + (uint32_t)g0 * 32u + (uint32_t)pc * 16u;
  }
  auto issue_pair = [&](int p) __device__ {
    uint8_t* slot = lds + p * Sh::PAIR_B;
#pragma unroll
    for (int i = 0; i < CI; ++i) dma16(rc, coff[i] + (uint32_t)p * 64u, slot + (i * LC + lw * 64) * 16);
  };
  // activation wave: load i of group g moves piece s = i LX + 64 lw + lane
  // of the slot's [token][8 pieces]; piece (t, pc ^ xswz(t)) holds piece pc
  // of token t
  uint32_t xoff[XI];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int s = i * LX + lw * 64 + lane;
    const int t = s >> 3, pc = (s & 7) ^ xswz(t);
    xoff[i] = (uint32_t)min(t, T - 1) * (uint32_t)K * 2u + (uint32_t)g0 * 128u + (uint32_t)pc * 16u;
  }
  auto issue_x = [&](int g) __device__ {
    const int gc = min(g, gs - 1);  // past the slice: the last group again, into a free slot
    uint8_t* slot = xring + (g % (DX + 1)) * Sh::XG_B;
#pragma unroll
    for (int i = 0; i < XI; ++i) dma16(rx, xoff[i] + (uint32_t)gc * 128u, slot + (i * LX + lw * 64) * 16);
  };

  // prologue: the code waves issue every pair of the slice at once (in
  // order, so pair p has landed when at most (npairs - 1 - p) CI of their
  // loads are outstanding); the activation waves load the block's scales
  // (all in flight), issue groups 0..DX-1, wait for the scales and write them
  // to the LDS table [row][GSP]
  if (code_wave) {
    for (int p = 0; p < npairs; ++p) issue_pair(p);
  } else {
    uint16_t sv[Sh::SV];
#pragma unroll
    for (int j = 0; j < Sh::SV; ++j) {
      const int idx = min(j * LX + lw * 64 + lane, BN * gs - 1);
      const int r = idx / gs, gg = idx - r * gs;
      sv[j] = scales[(size_t)(n0 + min(r, last_row)) * (size_t)G + g0 + gg];
    }
    for (int g = 0; g < DX; ++g) issue_x(g);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<DX * XI>();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < Sh::SV; ++j) {
      const int idx = j * LX + lw * 64 + lane;
      if (idx < BN * gs) {
        const int r = idx / gs, gg = idx - r * gs;
        stab[r * GSP + gg] = sv[j];
      }
    }
  }

  // --- the products --------------------------------------------------------------
  const int wr = wave % WR, wt = wave / WR;
  const uint32_t k136 = 0x43084308u;  // bf16 136.0 pair
  const bf16x8_t b136 = __builtin_bit_cast(bf16x8_t, u32x4_t{k136, k136, k136, k136});
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4_t acc[CT][TT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[ct][tt] = zero4;
  // operand addresses inside a slot: code row r = 16 (wr CT + ct) + li reads 8
  // bytes at byte 8 (lq & 1) of piece 2 (g & 1) + (lq >> 1); token t = 16 (wt
  // TT + tt) + li reads pieces 2 lq and 2 lq + 1
  int crow[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) crow[ct] = 16 * (wr * CT + ct) + li;

  for (int g = 0; g < gs; ++g) {
    __builtin_amdgcn_sched_barrier(0);
    if (code_wave) {
      if ((g & 1) == 0) wait_vm_atmost((npairs - 1 - (g >> 1)) * CI);
    } else {
      wait_vm<(DX - 1) * XI>();
    }
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // refill the activation slot read at the previous step
    if (!code_wave) issue_x(g + DX);
    __builtin_amdgcn_sched_barrier(0);

    const uint8_t* cslot = lds + (g >> 1) * Sh::PAIR_B;
    const uint8_t* xslot = xring + (g % (DX + 1)) * Sh::XG_B;
    bf16x8_t a[TT][2];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int t = 16 * (wt * TT + tt) + li;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        a[tt][h] = pair_order(*reinterpret_cast<const u32x4_t*>(xslot + (t * 8 + ((2 * lq + h) ^ xswz(t))) * 16));
    }
    u32x2_t cw[CT];
    float sc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int r = crow[ct];
      const int pc = 2 * (g & 1) + (lq >> 1);
      cw[ct] = *reinterpret_cast<const u32x2_t*>(cslot + (r * 4 + (pc ^ cswz(r))) * 16 + (lq & 1) * 8);
      sc[ct] = f16_bits_to_f32(stab[r * GSP + g]);
    }
    f32x4_t cr[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      cr[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[tt][0], b136, zero4, 0, 0, 0);
      cr[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[tt][1], b136, cr[tt], 0, 0, 0);
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const bf16x8_t b0 = bf16_codes(cw[ct].x), b1 = bf16_codes(cw[ct].y);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        f32x4_t p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[tt][0], b0, zero4, 0, 0, 0);
        p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[tt][1], b1, p, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[ct][tt][r] = __builtin_fmaf(sc[ct], p[r] - cr[tt][r], acc[ct][tt][r]);
      }
    }
  }
  // no load may still write this workgroup's LDS after this
  wait_vm<0>();

  // --- results: lane (li, lq) holds row n0 + 16 (wr CT + ct) + li, tokens
  // 16 (wt TT + tt) + 4 lq + r ------------------------------------------------
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int n = n0 + crow[ct];
    if (n >= N) continue;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * (wt * TT + tt) + 4 * lq + r;
        if (t >= T) continue;
        const size_t i = (size_t)t * (size_t)N + (size_t)n;
        if (S > 1) {
          part[(size_t)ks * (size_t)T * (size_t)N + i] = acc[ct][tt][r];
        } else if (f32out) {
          reinterpret_cast<float*>(y)[i] = acc[ct][tt][r];
        } else {
          float v = acc[ct][tt][r];
          if (res != nullptr) v += bf16_bits_to_f32(res[i]);  // LinearAdd
          uint16_t h = f32_to_bf16_rne(v);
          if ((h & 0x7F80u) == 0x7F80u) h = exact_q4_output(x, codes, scales, res, N, K, n, t);  // rare
          y[i] = h;
        }
      }
  }
}

// The split sums: y[t][n] = bf16(sum over the S slices of the partials, in
// slice order, in binary64), or the binary32 sum for LinearSwiGLU.  A thread
// takes four consecutive outputs (16-byte partial loads) when N % 4 == 0,
// else one.
constexpr int kReduceOut = 4;
__device__ __forceinline__ void reduce_one(double v, size_t i, uint16_t* y, int N, const uint16_t* res,
                                           const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes,
                                           const uint16_t* __restrict__ scales, int K, int f32out, int n, int t) {
  if (f32out) {
    reinterpret_cast<float*>(y)[i] = (float)v;
    return;
  }
  if (res != nullptr) v += (double)bf16_bits_to_f32(res[i]);  // LinearAdd
  uint16_t h = f32_to_bf16_rne((float)v);
  if ((h & 0x7F80u) == 0x7F80u) h = exact_q4_output(x, codes, scales, res, N, K, n, t);  // rare
  y[i] = h;
}
__global__ void __launch_bounds__(256)
mid_reduce_kernel(const float* __restrict__ part, uint16_t* y, int N, int T, int S, const uint16_t* res,
                  const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes,
                  const uint16_t* __restrict__ scales, int K, int f32out) {
  const int t = blockIdx.y;
  const size_t stride = (size_t)T * N;
  if ((N & 3) == 0) {
    const int n = (blockIdx.x * 256 + threadIdx.x) * kReduceOut;
    if (n >= N) return;
    const size_t i = (size_t)t * N + n;
    f32x4_t p[kMaxSplits];
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s)
      p[s] = s < S ? *reinterpret_cast<const f32x4_t*>(part + s * stride + i) : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kReduceOut; ++j) {
      double v = 0.0;
#pragma unroll
      for (int s = 0; s < kMaxSplits; ++s)
        if (s < S) v += (double)p[s][j];
      reduce_one(v, i + j, y, N, res, x, codes, scales, K, f32out, n + j, t);
    }
  } else {
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    const size_t i = (size_t)t * N + n;
    double v = 0.0;
    for (int s = 0; s < S; ++s) v += (double)part[s * stride + i];
    reduce_one(v, i, y, N, res, x, codes, scales, K, f32out, n, t);
  }
}

template <int CT, int TT, int WR, int WT, int CW, int DX>
hipError_t launch_shape(const GemvArgs& a, const MidPlan& p, float* part, hipStream_t stream) {
  auto kern = mid_kernel<CT, TT, WR, WT, CW, DX>;
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(kern));
  if (e != hipSuccess) return e;
  kern<<<dim3((unsigned)(p.row_blocks * p.splits)), dim3(kThreads), p.lds_bytes, stream>>>(
      static_cast<const uint16_t*>(a.x), static_cast<const uint8_t*>(a.codes), static_cast<const uint16_t*>(a.scales),
      static_cast<uint16_t*>(a.y), part, (int)a.n, (int)a.k, (int)a.t, p.splits, p.gsp, p.row_blocks,
      static_cast<const uint16_t*>(a.res), a.f32 ? 1 : 0);
  e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const int64_t per_block = (a.n % 4 == 0) ? 256 * kReduceOut : 256;
  mid_reduce_kernel<<<dim3((unsigned)((a.n + per_block - 1) / per_block), (unsigned)a.t), dim3(256), 0, stream>>>(
      part, static_cast<uint16_t*>(a.y), (int)a.n, (int)a.t, p.splits, static_cast<const uint16_t*>(a.res),
      static_cast<const uint16_t*>(a.x), static_cast<const uint8_t*>(a.codes),
      static_cast<const uint16_t*>(a.scales), (int)a.k, a.f32 ? 1 : 0);
  return hipGetLastError();
}

// the three shapes (CT, TT, WR, WT, CW, DX)
#define MID_SHAPE0 2, 1, 4, 2, 4, 8
#define MID_SHAPE1 3, 1, 2, 4, 6, 8
#define MID_SHAPE2 3, 2, 2, 4, 6, 4

size_t shape_lds(int shape, int npairs, int gsp) {
  if (shape == 0) return MidShape<MID_SHAPE0>::lds_bytes(npairs, gsp);
  if (shape == 1) return MidShape<MID_SHAPE1>::lds_bytes(npairs, gsp);
  return MidShape<MID_SHAPE2>::lds_bytes(npairs, gsp);
}

}  // namespace

// Shapes by token count: 17..32 tokens 128 rows x 32 tokens (4 x 2 waves of
// 32 x 16), 33..64 tokens 96 x 64 (2 x 4 waves of 48 x 16), 65..128 tokens
// 96 x 128 (2 x 4 waves of 48 x 32).  Splits: about 256 workgroups in all,
// every slice 2..32 groups.
bool mid_plan(int64_t n, int64_t k, int64_t t, MidPlan* p) {
  if (t < 17 || t > 128 || n < 1 || k < 128) return false;
  if (n * (k / 2) >= (int64_t(1) << 31) || t * k * 2 >= (int64_t(1) << 31)) return false;
  const int64_t G = k / 64;
  int shape, bn;
  if (t <= 32) {
    shape = 0;
    bn = 128;
  } else if (t <= 64) {
    shape = 1;
    bn = 96;
  } else {
    shape = 2;
    bn = 96;
  }
  const int64_t rbs = (n + bn - 1) / bn;
  int64_t s = (256 + rbs / 2) / rbs;
  if (s < 1) s = 1;
  if (s > kMaxSplits) s = kMaxSplits;
  while (s > 1 && G / s < 2) --s;
  // every code pair of a slice sits in LDS at once: more slices if it does not fit
  for (;; ++s) {
    if (s > kMaxSplits) return false;
    const int64_t gmax = (G + s - 1) / s;
    if (gmax > kMaxSliceGroups) continue;
    const int64_t gsp = (gmax + 1) & ~int64_t(1);
    const size_t lds = shape_lds(shape, (int)(gsp / 2), (int)gsp);
    if (lds > kLdsLimit) continue;
    p->shape = shape;
    p->bn = bn;
    p->row_blocks = (int)rbs;
    p->splits = (int)s;
    p->gsp = (int)gsp;
    p->lds_bytes = lds;
    return true;
  }
}

size_t mid_workspace_bytes(int64_t n, int64_t k, int64_t t) {
  MidPlan p;
  if (!mid_plan(n, k, t, &p) || p.splits == 1) return 0;
  return (size_t)p.splits * (size_t)t * (size_t)n * 4;
}

hipError_t launch_mid(const GemvArgs& a, void* workspace, hipStream_t stream) {
  MidPlan p;
  if (!mid_plan(a.n, a.k, a.t, &p)) return hipErrorInvalidValue;
  float* part = static_cast<float*>(workspace);
  if (p.shape == 0) return launch_shape<MID_SHAPE0>(a, p, part, stream);
  if (p.shape == 1) return launch_shape<MID_SHAPE1>(a, p, part, stream);
  return launch_shape<MID_SHAPE2>(a, p, part, stream);
}

}  // namespace q4lin
