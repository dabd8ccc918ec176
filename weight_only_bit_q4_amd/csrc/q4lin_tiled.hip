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
//   * Weights: a code dword gives four float16 pairs with two VALU operations
//     each.  Masking with 0x000F000F and OR-ing 0x6400 builds 1024 + q for the
//     nibbles at bits 0-3 of each half; masking with 0x00F000F0 builds
//     1024 + 16 q for the nibbles at bits 4-7.  One packed subtraction
//     (1032 resp. 1152) leaves q - 8 resp. 16 (q - 8), both exact in float16.
//   * Activations: a preparation pass multiplies each token by a power of two
//     2^-e[t] chosen from its largest magnitude (so every bf16 value within
//     2^34 of it converts to float16 exactly), divides the odd-k values by a
//     further 16 (cancelling the 16 above), and writes them in the order the
//     matrix-core operand reads want.  The epilogue multiplies by 2^e[t].
//   * v_mfma_f32_32x32x16_f16 with A = activations (32 tokens x 16 k) and
//     B = weights (16 k x 32 rows): every lane's 16 accumulators share one
//     weight row, so one scale per lane per group suffices.
//
// Data movement.  A workgroup owns BN rows x BT tokens.  Per 64-group it
// needs BN x 32 code bytes, BN scales and BT x 64 activations; these stream
// into an S-stage LDS ring with gfx950 direct-to-LDS loads
// (global_load_lds_dwordx4 / _dword), issued S-2 groups ahead, so the HBM
// latency of the codes and the L2 latency of the activations are covered.
// Each thread dequantizes exactly the code pieces it loaded itself (its own
// load counter is enough), into a padded, double-buffered weight tile; one
// barrier per group publishes that tile and the ring stage to all waves.
// Waits are explicit s_waitcnt vmcnt(n) with n the count of younger stages
// still allowed in flight; the compiler's own fences would wait for all.
#include "q4lin_device.h"
#include "q4lin_kernels.h"

namespace q4lin {

namespace {


// ---------------------------------------------------------------------------
// activation preparation: one wave per token
// ---------------------------------------------------------------------------
constexpr int kPrepWaves = 4;
constexpr int kPrepRegBlocks = 12;  // 8-value blocks per lane kept in registers

// Tile order: for token block tb (32 tokens) and group g, 4 KB laid out
// [m 0..3][h 0..1][i 0..31][8 values]; the 8 values are k = 64g + 32h + 8m +
// (0,4,1,5,2,6,3,7) (pair order), i the token inside the block.  Index in
// 16-byte units.
__device__ __forceinline__ size_t x16_index(int tb, int g, int G, int m, int h, int i) {
  return ((size_t)tb * G + g) * 256 + (size_t)((m * 2 + h) * 32 + i);
}

__device__ __forceinline__ uint32_t max_mag8(u32x4_t v) {
  uint32_t m = max(max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu), max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu));
  return max(m, max(max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu), max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu)));
}

// 8 bf16 values -> float16 in pair order, times 2^-e (odd k: 2^-(e+4)).
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

__global__ void __launch_bounds__(64 * kPrepWaves)
prep_x_kernel(const u32x4_t* __restrict__ x, int K, int T, int Tpad, u32x4_t* __restrict__ x16,
              int* __restrict__ texp) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kPrepWaves + (threadIdx.x >> 6);
  if (t >= Tpad) return;
  const int G = K >> 6;
  const int nb = K >> 3;
  const int tb = t >> 5, i = t & 31;
  if (t >= T) {  // padding token: zeros, exponent 0
    for (int b = lane; b < nb; b += 64) {
      const int g = b >> 3, kb = b & 7;
      x16[x16_index(tb, g, G, kb & 3, kb >> 2, i)] = u32x4_t{0u, 0u, 0u, 0u};
    }
    if (lane == 0) texp[t] = 0;
    return;
  }
  const u32x4_t* xt = x + (size_t)t * nb;
  u32x4_t v[kPrepRegBlocks];
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < kPrepRegBlocks; ++j) {
    const int b = lane + 64 * j;
    v[j] = b < nb ? xt[b] : u32x4_t{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int j = 0; j < kPrepRegBlocks; ++j) m = max(m, max_mag8(v[j]));
  for (int b = lane + 64 * kPrepRegBlocks; b < nb; b += 64) m = max(m, max_mag8(xt[b]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  if (m >= 0x7F80u) m = 0x7F7Fu;  // Inf/NaN inputs are outside the contract
  int e = 0;
  if (m != 0u) e = ((m >= 0x80u) ? (int)(m >> 7) - 127 : (31 - __builtin_clz(m)) - 133) - 14;
  if (lane == 0) texp[t] = e;
#pragma unroll
  for (int j = 0; j < kPrepRegBlocks; ++j) {
    const int b = lane + 64 * j;
    if (b < nb) {
      const int g = b >> 3, kb = b & 7;
      x16[x16_index(tb, g, G, kb & 3, kb >> 2, i)] = to_f16_pairs(v[j], e);
    }
  }
  for (int b = lane + 64 * kPrepRegBlocks; b < nb; b += 64) {
    const int g = b >> 3, kb = b & 7;
    x16[x16_index(tb, g, G, kb & 3, kb >> 2, i)] = to_f16_pairs(xt[b], e);
  }
}

// ---------------------------------------------------------------------------
// the tiled kernel
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
  return r;
}

// q - 8 (bits 0-3) and 16 (q - 8) (bits 4-7) as float16 pairs
__device__ __forceinline__ u32x4_t dequant_dword(uint32_t w) {
  const f16x2_t o1 = {(_Float16)1032.0f, (_Float16)1032.0f};
  const f16x2_t o16 = {(_Float16)1152.0f, (_Float16)1152.0f};
  const uint32_t w8 = w >> 8;
  u32x4_t r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, and_or(w, 0x000F000Fu, 0x64006400u)) - o1);
  r.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, and_or(w, 0x00F000F0u, 0x64006400u)) - o16);
  r.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, and_or(w8, 0x000F000Fu, 0x64006400u)) - o1);
  r.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, and_or(w8, 0x00F000F0u, 0x64006400u)) - o16);
  return r;
}

// Direct-to-LDS loads: every lane of the wave sends `bytes` bytes from its own
// global address to lds_base + lane * bytes (lds_base is wave-uniform).
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, lds_base, 4, 0, 0);
}

// s_waitcnt encoding for gfx9: vmcnt in bits 3:0 and 15:14, expcnt 6:4 (7 =
// no wait), lgkmcnt 11:8 (15 = no wait).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }

template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
}

// Byte offset of 16-byte piece `pi` (0..7) of row r in a dequantized weight
// tile: 128 bytes per row, pieces permuted per row so that the matrix-core
// operand reads (32 rows, one piece each) and the dequantizer's writes hit
// distinct LDS banks.
__device__ __forceinline__ int wpiece(int r, int pi) { return r * 128 + ((pi ^ ((r ^ (r >> 3)) & 7)) << 4); }

// Ring geometry: the activation ring has DX slots and is filled DX groups
// ahead; the code/scale ring has DX slots and is filled DX+1 groups ahead
// (a group's codes are dequantized two groups before its products).
constexpr int DX = 4;
constexpr int DC = DX + 1;

template <int NS, int TS, int WN, int WT>
struct TiledShape {
  static constexpr int NT = 64 * WN * WT;                 // threads
  static constexpr int BN = 32 * NS * WN;                 // rows per workgroup
  static constexpr int BT = 32 * TS * WT;                 // tokens per workgroup
  static constexpr int CI = (2 * BN + NT - 1) / NT;       // code (and scale) loads per thread per batch
  static constexpr int XI = BT * 8 / NT;                  // activation loads per thread per batch
  static constexpr int L = 2 * CI + XI;                   // loads per thread per batch
  static constexpr int CODE_B = CI * NT * 16;             // one code slot
  static constexpr int SCALE_B = CI * NT * 4;             // one scale slot
  static constexpr int X_B = BT * 128;                    // one activation slot
  static constexpr int W_B = BN * 128;                    // one dequantized weight tile
  static constexpr int OFF_C = DX * X_B;
  static constexpr int OFF_S = OFF_C + DX * CODE_B;
  static constexpr int OFF_W = OFF_S + DX * SCALE_B;
  static constexpr int OFF_SB = OFF_W + 2 * W_B;
  static constexpr int LDS_B = OFF_SB + 2 * BN * 4;
  static_assert(BT * 8 % NT == 0, "activation tile must split evenly over the threads");
  static_assert(LDS_B <= 160 * 1024, "LDS budget");
};

template <int NS, int TS, int WN, int WT>
__global__ void __launch_bounds__(64 * WN * WT)
tiled_kernel(const u32x4_t* __restrict__ x16, const int* __restrict__ texp,
             const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
             uint16_t* __restrict__ y, int N, int K, int T, int Tpad, int tiles_n, int tiles_t) {
  using Sh = TiledShape<NS, TS, WN, WT>;
  constexpr int NT = Sh::NT, BN = Sh::BN, BT = Sh::BT, CI = Sh::CI, XI = Sh::XI, L = Sh::L;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float* sbuf = reinterpret_cast<float*>(lds + Sh::OFF_SB);       // 2 x BN scales

  const int G = K >> 6;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, lh = lane >> 5;
  const int wn = wave % WN, wt = wave / WN;

  // XCD-aware tile order: workgroups are dealt round-robin to the 8 XCDs, so
  // give each XCD a contiguous run of tiles (same token tile, neighbouring row
  // tiles) and let its L2 keep that activation tile.
  const int nblk = tiles_n * tiles_t;
  int lin = blockIdx.x;
  if ((nblk & 7) == 0) lin = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int tile_t = lin / tiles_n, tile_n = lin - tile_t * tiles_n;
  const int n0 = tile_n * BN;
  const int tb0 = tile_t * (BT / 32);                 // first 32-token block
  const int tb_last = Tpad / 32 - 1;

  // --- loads: codes and scales of group gc, activations of group gx --------
  // Every thread issues exactly L loads per call; indexes are clamped to valid
  // data, so the batches near the end simply repeat the last group.
  auto issue = [&](int gc, int gx, bool with_x) __device__ {
    gc = min(gc, G - 1);
    gx = min(gx, G - 1);
    uint8_t* cs = lds + Sh::OFF_C + (gc % DX) * Sh::CODE_B;
    uint8_t* ss = lds + Sh::OFF_S + (gc % DX) * Sh::SCALE_B;
    uint8_t* xs = lds + (gx % DX) * Sh::X_B;
#pragma unroll
    for (int c = 0; c < CI; ++c) {
      const int task = (c * NT + tid) % (2 * BN);     // tasks past 2*BN repeat valid ones
      const int row = min(n0 + (task >> 1), N - 1);
      dma16(codes + (size_t)row * (K >> 1) + (size_t)gc * 32 + (task & 1) * 16, cs + c * NT * 16 + wave * 1024);
    }
#pragma unroll
    for (int c = 0; c < CI; ++c) {
      const int task = (c * NT + tid) % (2 * BN);
      const int row = min(n0 + (task >> 1), N - 1);
      // The scale's naturally aligned dword: it never leaves the scale's own
      // page, and the other half is ignored.
      const uintptr_t sa = reinterpret_cast<uintptr_t>(scales + (size_t)row * G + gc) & ~(uintptr_t)3;
      dma4(reinterpret_cast<const void*>(sa), ss + c * NT * 4 + wave * 256);
    }
    if (!with_x) return;
#pragma unroll
    for (int j = 0; j < XI; ++j) {
      const int off = (j * NT + tid) * 16;             // byte offset inside the BT x 128 B slot
      const int tb = min(tb0 + (off >> 12), tb_last);  // 4 KB per 32-token block
      const uint8_t* src = reinterpret_cast<const uint8_t*>(x16) + (((size_t)tb * G + gx) << 12) + (off & 4095);
      dma16(src, xs + j * NT * 16 + wave * 1024);
    }
  };

  // --- dequantize this thread's own code pieces of group g into tile b -----
  auto dequant = [&](int g, int b) __device__ {
    const uint8_t* cs = lds + Sh::OFF_C + (g % DX) * Sh::CODE_B;
    const uint8_t* ss = lds + Sh::OFF_S + (g % DX) * Sh::SCALE_B;
    uint8_t* wb = lds + Sh::OFF_W + b * Sh::W_B;
#pragma unroll
    for (int c = 0; c < CI; ++c) {
      const int task = c * NT + tid;
      if (task < 2 * BN) {
        const int r = task >> 1, hh = task & 1;
        const u32x4_t cw = *reinterpret_cast<const u32x4_t*>(cs + c * NT * 16 + tid * 16);
#pragma unroll
        for (int d = 0; d < 4; ++d)
          *reinterpret_cast<u32x4_t*>(wb + wpiece(r, hh * 4 + d)) = dequant_dword(cw[d]);
        if (hh == 0) {
          const uint32_t sw = *reinterpret_cast<const uint32_t*>(ss + c * NT * 4 + tid * 4);
          const int row = min(n0 + r, N - 1);
          const bool hi = (reinterpret_cast<uintptr_t>(scales + (size_t)row * G + g) & 2) != 0;
          sbuf[b * BN + r] = f16_bits_to_f32((uint16_t)(hi ? (sw >> 16) : (sw & 0xFFFFu)));
        }
      }
    }
  };

  // --- matrix-core operands of group g (activation slot, weight tile g & 1) -
  auto read_a = [&](int g, f16x8_t (&a)[TS][4]) __device__ {
    const uint8_t* xs = lds + (g % DX) * Sh::X_B;
#pragma unroll
    for (int ts = 0; ts < TS; ++ts)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        a[ts][m] = *reinterpret_cast<const f16x8_t*>(xs + ((wt * TS + ts) << 12) + (((m * 2 + lh) * 32 + li) << 4));
  };
  auto read_b = [&](int g, int ns, f16x8_t (&b)[4], float& sc) __device__ {
    const uint8_t* wb = lds + Sh::OFF_W + (g & 1) * Sh::W_B;
    const int r = (wn * NS + ns) * 32 + li;
#pragma unroll
    for (int m = 0; m < 4; ++m) b[m] = *reinterpret_cast<const f16x8_t*>(wb + wpiece(r, lh * 4 + m));
    sc = sbuf[(g & 1) * BN + r];
  };

  f32x16_t acc[TS][NS];
#pragma unroll
  for (int ts = 0; ts < TS; ++ts)
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[ts][ns][r] = 0.0f;
  // Operands of the group in flight: activation and weight fragments are
  // each refilled with the next group's as soon as the last product that
  // reads them has been issued.
  f16x8_t aop[TS][4];
  f16x8_t bop[NS][4];
  float sc[NS], sn[NS];

  // Step g: wait for the batch that carried group g+1's activations and group
  // g+2's codes (issued three steps earlier), publish with a barrier, issue
  // the next batch, run group g's products, refill the operands with group
  // g+1's, and dequantize group g+2 in between.
  auto step = [&](int g) __device__ {
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<(DX - 2) * L>();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(g + DC, g + DX, true);
    __builtin_amdgcn_sched_barrier(0);
    const bool more = g + 1 < G;
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      f32x16_t p[TS];
#pragma unroll
      for (int ts = 0; ts < TS; ++ts) {
        p[ts] = f32x16_t{};
#pragma unroll
        for (int m = 0; m < 4; ++m)
          p[ts] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[ts][m], bop[ns][m], p[ts], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (more) {
        read_b(g + 1, ns, bop[ns], sn[ns]);
        if (ns == NS - 1) read_a(g + 1, aop);
      }
      if (ns == 0 && g + 2 < G) dequant(g + 2, g & 1);
#pragma unroll
      for (int ts = 0; ts < TS; ++ts)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[ts][ns][r] = __builtin_fmaf(sc[ns], p[ts][r], acc[ts][ns][r]);
    }
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) sc[ns] = sn[ns];
  };

  // Prologue: groups 0..DX-1 loaded, groups 0 and 1 dequantized, then the
  // codes of group DX (whose slot group 0 used) in flight, and group 0's
  // operands read.  Step 2 waits for those codes behind two full batches.
  for (int j = 0; j < DX; ++j) issue(j, j, true);
  __builtin_amdgcn_sched_barrier(0);
  wait_vm<0>();
  __builtin_amdgcn_sched_barrier(0);
  dequant(0, 0);
  if (G > 1) dequant(1, 1);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  issue(DX, 0, false);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  read_a(0, aop);
#pragma unroll
  for (int ns = 0; ns < NS; ++ns) read_b(0, ns, bop[ns], sc[ns]);
  for (int g = 0; g < G; ++g) step(g);

  // Epilogue: lane (li, lh) holds row n = n0 + 32 (wn*NS + ns) + li and tokens
  // t = 32 (tb0 + wt*TS + ts) + 8 (r / 4) + 4 lh + r % 4.
  // The exponents are loaded up front (texp has Tpad entries), so that the
  // loads overlap instead of each waiting behind the previous store.
#pragma unroll
  for (int ts = 0; ts < TS; ++ts) {
    const int tbase = 32 * (tb0 + wt * TS + ts) + 4 * lh;
    int e[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = texp[min(tbase + 8 * (r >> 2) + (r & 3), Tpad - 1)];
    // Scale every value before the first (masked) store: the empty asm pins
    // the results here, so the stores below wait for no load.
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        acc[ts][ns][r] = __builtin_ldexpf(acc[ts][ns][r], e[r]);
        asm volatile("" : "+v"(acc[ts][ns][r]));
      }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = tbase + 8 * (r >> 2) + (r & 3);
      if (t < T) {
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          const int n = n0 + 32 * (wn * NS + ns) + li;
          if (n < N) y[(size_t)t * N + n] = f32_to_bf16_rne(acc[ts][ns][r]);
        }
      }
    }
  }
}

template <int NS, int TS, int WN, int WT>
hipError_t launch_cfg(const TiledArgs& a, const u32x4_t* x16, const int* texp, int tpad, hipStream_t stream) {
  using Sh = TiledShape<NS, TS, WN, WT>;
  const int tiles_n = (int)((a.n + Sh::BN - 1) / Sh::BN);
  const int tiles_t = (int)((a.t + Sh::BT - 1) / Sh::BT);
  auto kern = tiled_kernel<NS, TS, WN, WT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, Sh::LDS_B);
  if (e != hipSuccess) return e;
  kern<<<dim3((unsigned)(tiles_n * tiles_t)), dim3(Sh::NT), Sh::LDS_B, stream>>>(
      x16, texp, static_cast<const uint8_t*>(a.codes), static_cast<const uint16_t*>(a.scales),
      static_cast<uint16_t*>(a.y), (int)a.n, (int)a.k, (int)a.t, tpad, tiles_n, tiles_t);
  return hipGetLastError();
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

int64_t tiled_tpad(int64_t t) { return (t + 31) / 32 * 32; }

size_t tiled_workspace_bytes(int64_t k, int64_t t) {
  const int64_t tp = tiled_tpad(t);
  return align256((size_t)(tp * k * 2)) + align256((size_t)(tp * 4));
}

TiledConfig tiled_pick_config(int64_t n, int64_t k, int64_t t) {
  (void)k;
  // 192 x 128 tiles where they fill the chip, else narrower token tiles
  if (t > 96 && (n / 192) * ((t + 127) / 128) >= 192) return TiledConfig{3, 1, 2, 4};
  if (t > 32) return TiledConfig{1, 1, 1, 4};
  return TiledConfig{1, 1, 1, 1};
}

hipError_t launch_tiled(const TiledArgs& a, hipStream_t stream) {
  const int64_t tp = tiled_tpad(a.t);
  u32x4_t* x16 = static_cast<u32x4_t*>(a.workspace);
  int* texp = reinterpret_cast<int*>(static_cast<uint8_t*>(a.workspace) + align256((size_t)(tp * a.k * 2)));
  {
    const u32x4_t* x = static_cast<const u32x4_t*>(a.x);
    int k = (int)a.k, t = (int)a.t, tpad = (int)tp;
    void* args[] = {&x, &k, &t, &tpad, &x16, &texp};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(prep_x_kernel),
                                   dim3((unsigned)((tp + kPrepWaves - 1) / kPrepWaves)), dim3(64 * kPrepWaves),
                                   args, 0, stream);
    if (e != hipSuccess) return e;
  }
  const int tpad = (int)tp;
  const TiledConfig c = a.cfg;
  if (c.ns == 3 && c.ts == 1 && c.wn == 2 && c.wt == 4) return launch_cfg<3, 1, 2, 4>(a, x16, texp, tpad, stream);
  if (c.ns == 1 && c.ts == 1 && c.wn == 1 && c.wt == 4) return launch_cfg<1, 1, 1, 4>(a, x16, texp, tpad, stream);
  if (c.ns == 1 && c.ts == 1 && c.wn == 1 && c.wt == 1) return launch_cfg<1, 1, 1, 1>(a, x16, texp, tpad, stream);
  return hipErrorInvalidValue;
}

}  // namespace q4lin
