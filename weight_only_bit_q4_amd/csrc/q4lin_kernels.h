// q4lin_kernels.h -- host-side launchers of the q4lin kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q4lin {

// Lets `kern` take up to the whole 160 KiB of a gfx950 CU's LDS as dynamic
// LDS.  Only the first call per (kernel, device) reaches the runtime; later
// calls return the recorded result (thread-safe).
hipError_t allow_full_lds(const void* kern);

struct GemvArgs {
  const void* x;
  const void* codes;
  const void* scales;
  void* y;
  int64_t n, k, t;
  const void* res = nullptr;  // LinearAdd residual, bf16 [T][N] like y (nullptr: plain Linear)
  // LinearPair: a second weight (n2 rows, same K) and its output; n2 == 0: none
  const void* codes2 = nullptr;
  const void* scales2 = nullptr;
  void* y2 = nullptr;
  int64_t n2 = 0;
  bool f32 = false;  // outputs as binary32 [T][N] (LinearSwiGLU's gate and up sums), not bf16
  // LinearSwiGLU in one pass (single-token route): codes/scales are the gate,
  // codes2/scales2 the up weight (n2 == n); every workgroup takes the same
  // rows of both and stores bf16(silu(G) * U) into y
  bool glu = false;
};

// The second plane of a LinearPair as the kernels see it: the workgroups from
// `first` on serve it (their block index counted from there).
struct SecondPlane {
  const uint8_t* codes;
  const uint16_t* scales;
  uint16_t* y;
  int n;      // rows (0: no second plane)
  int first;  // its first workgroup
  int f32;    // every output stored as binary32 [T][N] instead of bf16
  int glu;    // LinearSwiGLU: a workgroup's rows are H gate rows, then the same H up rows
};
inline SecondPlane second_plane(const GemvArgs& a, int first) {
  return SecondPlane{static_cast<const uint8_t*>(a.codes2), static_cast<const uint16_t*>(a.scales2),
                     static_cast<uint16_t*>(a.y2), (int)a.n2, first, a.f32 ? 1 : 0, a.glu ? 1 : 0};
}

// Few-token route.  Each of the 4 waves of a workgroup owns a quarter of the
// 32-weight chunks of every row; gemv_chunks_per_wave is that quarter's
// capacity (rounded up), gemv_lds_bytes the dynamic LDS the kernel needs:
// float16 activations plus one all-8 chunk sum per (token, chunk).
int64_t gemv_chunks_per_wave(int64_t k);
size_t gemv_lds_bytes(int64_t k, int64_t t);
hipError_t launch_gemv(const GemvArgs& a, hipStream_t stream);

// Single-token route: a workgroup of eight waves per block of bn rows, K
// split over the waves, activations in registers, no workspace.
struct DecodePlan {
  int bn;      // rows per workgroup
  int pl;      // consecutive 16-byte pieces per lane and row
  int maxr;    // rows per lane, at most
  int blocks;  // workgroups
  int waves;   // waves per workgroup (8, or 12 for long rows)
};
bool decode_plan(int64_t n, int64_t k, int64_t t, DecodePlan* p);
// whether LinearSwiGLU of n rows per weight runs in one pass on this route
bool decode_glu_ok(int64_t n, int64_t k, int64_t t);
hipError_t launch_decode(const GemvArgs& a, hipStream_t stream);

// Small-T route: one workgroup of eight waves per block of bn rows, K split
// over the waves, no workspace.  skinny_plan() says whether the route takes
// (n, k, t) and with which block shape; launch_skinny() uses the same plan.
struct SkinnyPlan {
  int bn;      // rows per workgroup
  int ct;      // 16-row matrix-core column tiles per wave (bn <= 16 * ct)
  int tt;      // 16-token tiles (t <= 16 * tt)
  int blocks;  // workgroups
  int off_codes, off_red;  // LDS byte offsets of the code staging / final sums
  size_t lds_bytes;
};
bool skinny_plan(int64_t n, int64_t k, int64_t t, SkinnyPlan* p);
hipError_t launch_skinny(const GemvArgs& a, hipStream_t stream);

// Tiled matrix-core route.  Workspace layout (256-byte aligned pieces):
//   x16   fp16 activations scaled by 2^-e[t], tile order (see q4lin_tiled.hip),
//         tpad * k * 2 bytes with tpad = t rounded up to 32;
//   texp  int32 e[t], tpad * 4 bytes.
struct TiledConfig {
  int ns;  // 32-row subtiles per wave
  int ts;  // 32-token subtiles per wave
  int wn;  // waves along the rows
  int wt;  // waves along the tokens
  int ks;  // K split into this many workgroup shares (1: none)
};

struct TiledArgs {
  const void* x;
  const void* codes;
  const void* scales;
  void* y;
  int64_t n, k, t;
  void* workspace;
  TiledConfig cfg;
  const void* res = nullptr;  // LinearAdd residual, bf16 [T][N] like y (nullptr: plain Linear)
  bool f32 = false;  // the raw FP32 sums go to the partials for a later pass (LinearSwiGLU)
};

// A binary32 source of sums for the LinearSwiGLU combine: element (t, n) is
// 2^(texp[t] - rexp[n]) * (sum over ks slices of part[s * stride + t*N + n]),
// the exponents omitted when texp is null.
struct SumSource {
  const float* part;
  const int* texp;
  const int* rexp;
  int ks;
  size_t stride;
};

// The second weight of a LinearPair / LinearSwiGLU on the many-token route,
// as the tiled kernel sees it: the workgroups from `first` on serve it.
struct TiledPlane2 {
  const uint8_t* codes = nullptr;
  const uint16_t* scales = nullptr;
  uint16_t* y = nullptr;
  float* part = nullptr;     // its partial sums (K split or binary32 sums)
  const int* rexp = nullptr;  // its row exponents
  int n = 0;                 // rows (0: no second weight)
  int tiles_n = 0;           // its row tiles
  int first = 0;             // its first workgroup
};

// Two weights over one X on the many-token route: one activation
// preparation (it also takes both weights' row exponents) and one launch
// whose workgroups cover both weights' tiles (the second's after the
// first's); the K-split sums, if any, are added per weight.  Workspace: the
// activations once, then each weight's row exponents and partials.
struct TiledPairArgs {
  TiledArgs a;  // x, the first weight, y, n, k, t, workspace, cfg (for n + n2 rows), f32
  const void* codes2;
  const void* scales2;
  void* y2;
  int64_t n2;
};
size_t tiled_pair_workspace_bytes(int64_t n1, int64_t n2, int64_t k, int64_t t, bool f32);
// src1/src2 (binary32 sums only) receive where each weight's sums are
hipError_t launch_tiled_pair(const TiledPairArgs& p, SumSource* src1, SumSource* src2, hipStream_t stream);
// LinearSwiGLU in one tiled launch (after the activation preparation):
// tiles of 48 gate rows and the same 48 up rows, bf16(silu(G) U) formed in
// the epilogue.  a: x, the gate's planes, y, n, k, t, workspace; where
// tiled_glu_ok (the 2N-row problem on 96 x 256 tiles without a K split).
bool tiled_glu_ok(int64_t n, int64_t k, int64_t t);
size_t tiled_glu_workspace_bytes(int64_t n, int64_t k, int64_t t);
hipError_t launch_tiled_glu(const TiledArgs& a, const void* codes_up, const void* scales_up, hipStream_t stream);

int64_t tiled_tpad(int64_t t);
// Whether the tiled kernels can address (n, k, t): their buffer offsets are
// 32-bit, so the float16 activation copy (tpad * k * 2 bytes) and the scale
// plane (n * k / 32 bytes) must each stay below 2 GiB.
bool tiled_shape_ok(int64_t n, int64_t k, int64_t t);
size_t tiled_workspace_bytes(int64_t n, int64_t k, int64_t t);
TiledConfig tiled_pick_config(int64_t n, int64_t k, int64_t t);
hipError_t launch_tiled(const TiledArgs& a, hipStream_t stream);
// y[t][n] = bf16(silu(G) * U), G and U from the two sources ([T][N] each).
hipError_t launch_swiglu_combine(const SumSource& g, const SumSource& u, void* y, int64_t n, int64_t t,
                                 hipStream_t stream);


// The other weight formats (few-token route, any T in runs of 32 tokens).
// Format numbers as in the public header's Q4LIN_FMT_* values.
enum { FMT_Q4 = 0, FMT_Q5 = 1, FMT_Q6 = 2, FMT_W8 = 3, FMT_NVFP4 = 4, FMT_BF16 = 5 };
struct FmtArgs {
  int fmt;
  const void* x;
  const void* lo;  // code plane (BF16_CTRL: the weights)
  const void* hi;  // high plane (Q5, Q6), else unused
  const void* sc;  // scale plane (fp16, or E4M3 bytes for NVFP4; unused for BF16_CTRL)
  void* y;
  int64_t n, k, t;
  const void* res = nullptr;  // LinearAdd residual, bf16 [T][N] (nullptr: plain Linear)
  bool f32 = false;           // outputs as binary32 [T][N] (LinearSwiGLU's sums), not bf16
  // A second weight of the same format and K over the same X in the same
  // launch.  LinearPair (glu false): n2 rows of its own, output y2 (bf16
  // [T][n2], no residual).  LinearSwiGLU (glu true, Q4 only): the up weight
  // of the gate's N rows (lo/sc: the gate); y = bf16(silu(G) U), y2 unused.
  const void* lo2 = nullptr;
  const void* hi2 = nullptr;
  const void* sc2 = nullptr;
  void* y2 = nullptr;
  int64_t n2 = 0;
  bool glu = false;
};
struct FmtPlan {
  int bn;      // rows per workgroup
  int ct;      // 16-row column tiles per wave
  int blocks;  // workgroups
  size_t lds_bytes;
};
// glu: rows per workgroup of each of the gate and up weights (N rows each)
bool fmt_plan(int fmt, int64_t n, int64_t k, int64_t t, FmtPlan* p, bool glu = false);
hipError_t launch_fmt(const FmtArgs& a, hipStream_t stream);

}  // namespace q4lin
