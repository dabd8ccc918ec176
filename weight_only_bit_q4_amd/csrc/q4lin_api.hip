// q4lin_api.hip -- the C ABI: argument validation, route choice, launch.
//
// The contract follows the pages' public Linear call
// linear(x, w, out, policy, workspace, stream) ("linear-benchmark.md",
// section 0): the caller owns every buffer, the workspace size comes from a
// capacity query answered before any timed call (same page, section 1.1),
// and shapes the op does not support are rejected by the op itself (same
// page, section 1.1, on numeric N/K points).  Only the A16 policy exists, so
// there is no policy argument.
#include <stdint.h>

#include <mutex>
#include <utility>
#include <vector>

#include "../../include/q4lin.h"
#include "q4lin_kernels.h"

namespace q4lin {

hipError_t allow_full_lds(const void* kern) {
  static std::mutex mu;
  static std::vector<std::pair<const void*, int>> done;  // (kernel, device) pairs already raised
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& d : done)
    if (d.first == kern && d.second == dev) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e == hipSuccess) done.emplace_back(kern, dev);
  return e;
}

}  // namespace q4lin

namespace {

constexpr int64_t kMaxN = int64_t(1) << 24;
constexpr int64_t kMaxT = int64_t(1) << 21;
constexpr int64_t kMaxK = int64_t(1) << 20;
constexpr int64_t kMaxBytes = int64_t(1) << 40;
constexpr size_t kGemvLdsLimit = 64 * 1024;
// The medium-T route takes T from kMidFirstT to kMidLastT: the weight
// formats' kernel on the Q4 codes, every wave on all the tokens of its run
// (one weight pass, no workspace).
constexpr int64_t kMidFirstT = 33;
constexpr int64_t kMidLastT = 128;

// whether the medium-T route takes (n, k, t)
bool mid_ok(int64_t n, int64_t k, int64_t t) {
  q4lin::FmtPlan fp;
  return t >= kMidFirstT && t <= kMidLastT && q4lin::fmt_plan(q4lin::FMT_Q4, n, k, t, &fp);
}

// The small-T route's single weight from kSmallFmtFirstT tokens on runs the
// few-token kernel of the weight formats on the Q4 codes (6144 x 5120:
// T = 5 9.9 against 11.2 us, T = 17 13.7 / 16.2, T = 32 15.2 / 20.4 on the
// small-T kernel, which keeps two weights in one launch: LinearPair and
// LinearSwiGLU).
constexpr int64_t kSmallFmtFirstT = 5;
bool small_uses_fmt(int64_t n, int64_t k, int64_t t) {
  q4lin::FmtPlan fp;
  return t >= kSmallFmtFirstT && q4lin::fmt_plan(q4lin::FMT_Q4, n, k, t, &fp);
}
static_assert(q4lin::FMT_Q5 == Q4LIN_FMT_Q5G64_F16S && q4lin::FMT_Q6 == Q4LIN_FMT_Q6G64_F16S &&
                  q4lin::FMT_W8 == Q4LIN_FMT_W8G32_F16S && q4lin::FMT_NVFP4 == Q4LIN_FMT_NVFP4 &&
                  q4lin::FMT_BF16 == Q4LIN_FMT_BF16,
              "the kernels' format numbers are the header's");

bool shape_ok(int64_t n, int64_t k, int64_t t) {
  if (n < 0 || t < 0 || k < 64 || (k % 64) != 0) return false;
  if (n > kMaxN || t > kMaxT || k > kMaxK) return false;
  if (n * (k / 2) >= kMaxBytes || t * k * 2 >= kMaxBytes || t * n * 2 >= kMaxBytes) return false;
  return true;
}

int pick_route(int64_t n, int64_t k, int64_t t) {
  if (n == 0 || t == 0) return Q4LIN_ROUTE_NONE;
  q4lin::DecodePlan dp;
  q4lin::SkinnyPlan sp;
  if (q4lin::decode_plan(n, k, t, &dp)) {
    // The single-token route streams best with one 16-byte piece per lane
    // and row; where a wave's slice is longer than 64 pieces (K > 16384) the
    // small-T route beats its wider lane shapes (5120 x 17408: 19.8 against
    // 23.3 us)
    if (dp.pl == 1 || !q4lin::skinny_plan(n, k, t, &sp)) return Q4LIN_ROUTE_DECODE;
    return Q4LIN_ROUTE_SKINNY;
  }
  if (t == 1 && q4lin::gemv_lds_bytes(k, t) <= kGemvLdsLimit) return Q4LIN_ROUTE_GEMV;
  if (q4lin::skinny_plan(n, k, t, &sp)) return Q4LIN_ROUTE_SKINNY;
  if (t <= 4 && q4lin::gemv_lds_bytes(k, t) <= kGemvLdsLimit) return Q4LIN_ROUTE_GEMV;
  if (mid_ok(n, k, t)) return Q4LIN_ROUTE_MID;
  return Q4LIN_ROUTE_TILED;
}

size_t route_workspace(int route, int64_t n, int64_t k, int64_t t) {
  if (route == Q4LIN_ROUTE_TILED) return q4lin::tiled_workspace_bytes(n, k, t);
  return 0;
}

// The small-T and medium-T routes run the Q4 weight through the weight
// formats' kernel (up to 128 tokens per weight read).
q4lin::FmtArgs q4_fmt_args(const q4lin::GemvArgs& g) {
  q4lin::FmtArgs a{q4lin::FMT_Q4, g.x, g.codes, nullptr, g.scales, g.y, g.n, g.k, g.t};
  a.res = g.res;
  a.f32 = g.f32;
  return a;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Host-side checks of the op's arguments other than the workspace: the
// status, and in *route the route for a valid non-empty product.
int check_linear(const void* x, const void* codes, const void* scales, const void* res, const void* y,
                 int64_t n, int64_t k, int64_t t, int* route) {
  *route = Q4LIN_ROUTE_NONE;
  if (!shape_ok(n, k, t)) return Q4LIN_E_SHAPE;
  const int r = pick_route(n, k, t);
  if (r == Q4LIN_ROUTE_NONE) return Q4LIN_OK;
  if (r == Q4LIN_ROUTE_TILED && !q4lin::tiled_shape_ok(n, k, t)) return Q4LIN_E_SHAPE;
  if (!x || !codes || !scales || !y) return Q4LIN_E_NULL;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 2) || !aligned(y, 2) || !aligned(res, 2))
    return Q4LIN_E_ALIGN;
  *route = r;
  return Q4LIN_OK;
}

// Two weights over one X take the many-token route together when the route
// for their rows is that one (shared activation preparation, one launch).
bool pair_on_tiled(int route, int64_t n1, int64_t n2, int64_t k, int64_t t) {
  return route == Q4LIN_ROUTE_TILED && q4lin::tiled_shape_ok(n1, k, t) && q4lin::tiled_shape_ok(n2, k, t);
}

// ... and one launch of the weight formats' kernel where the route for their
// rows runs a single weight there (the small-T route from kSmallFmtFirstT
// tokens, the medium-T route): the second weight's rows are further row
// blocks of the same launch.
bool pair_on_fmt(int route, int64_t n1, int64_t n2, int64_t k, int64_t t) {
  return (route == Q4LIN_ROUTE_SKINNY && small_uses_fmt(n1 + n2, k, t)) || route == Q4LIN_ROUTE_MID;
}

// The op, with an optional residual (LinearAdd when res is not null).
int run_linear(const void* x, const void* codes, const void* scales, const void* res, void* y,
               int64_t n, int64_t k, int64_t t, void* workspace, size_t workspace_bytes, void* stream) {
  int route = Q4LIN_ROUTE_NONE;
  const int st = check_linear(x, codes, scales, res, y, n, k, t, &route);
  if (st != Q4LIN_OK || route == Q4LIN_ROUTE_NONE) return st;
  const size_t need = route_workspace(route, n, k, t);
  if (need > 0) {
    if (workspace_bytes < need) return Q4LIN_E_WORKSPACE;
    if (!workspace) return Q4LIN_E_NULL;
    if (!aligned(workspace, 256)) return Q4LIN_E_ALIGN;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  const q4lin::GemvArgs ga{x, codes, scales, y, n, k, t, res};
  if (route == Q4LIN_ROUTE_GEMV) {
    e = q4lin::launch_gemv(ga, s);
  } else if (route == Q4LIN_ROUTE_DECODE) {
    e = q4lin::launch_decode(ga, s);
  } else if (route == Q4LIN_ROUTE_SKINNY) {
    e = small_uses_fmt(n, k, t) ? q4lin::launch_fmt(q4_fmt_args(ga), s) : q4lin::launch_skinny(ga, s);
  } else if (route == Q4LIN_ROUTE_MID) {
    e = q4lin::launch_fmt(q4_fmt_args(ga), s);
  } else {
    q4lin::TiledArgs a{x, codes, scales, y, n, k, t, workspace, q4lin::tiled_pick_config(n, k, t), res};
    e = q4lin::launch_tiled(a, s);
  }
  return e == hipSuccess ? Q4LIN_OK : Q4LIN_E_LAUNCH;
}

size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

// LinearSwiGLU's plan: how the gate and up sums are made, and the workspace.
//   FUSED: both weights in one launch of the one-to-four-token or small-T
//          route (chosen for 2N rows), binary32 sums into the workspace;
//   SPLIT: one launch per weight on the route chosen for N rows;
//   TILED: the many-token route per weight, its raw sums left in the
//          partials of a workspace half each.
//   MID:   the medium-T route per weight, binary32 sums in each half;
//   GLU:   the single-token route, each workgroup on the same rows of both
//          weights, the gate applied in its final sum (no workspace);
//   FMT:   the same on the weight formats' kernel, kSmallFmtFirstT to
//          kMidLastT tokens (no workspace);
//   TGLU:  the many-token route in one tiled launch whose tiles take the
//          same rows of both weights (96 x 256 tiles for 2N rows, no K
//          split), the gate applied in the epilogue (workspace: the
//          activation preparation only).
enum { SW_FUSED = 1, SW_SPLIT = 2, SW_TILED = 3, SW_MID = 4, SW_GLU = 5, SW_FMT = 6, SW_TGLU = 7 };
struct SwigluPlan {
  int mode;
  int route;
  size_t half;   // bytes of each weight's half of the workspace (TILED: unused)
  size_t total;  // workspace bytes
};

bool swiglu_plan(int64_t n, int64_t k, int64_t t, SwigluPlan* p) {
  if (!shape_ok(n, k, t) || !shape_ok(2 * n, k, t) || !shape_ok(n, k, 2 * t)) return false;
  const int r2 = pick_route(2 * n, k, t);
  if (r2 == Q4LIN_ROUTE_DECODE && q4lin::decode_glu_ok(n, k, t)) {
    *p = SwigluPlan{SW_GLU, r2, 0, 0};
    return true;
  }
  q4lin::FmtPlan fp;
  if (t >= kSmallFmtFirstT && t <= kMidLastT && (r2 == Q4LIN_ROUTE_SKINNY || r2 == Q4LIN_ROUTE_MID) &&
      q4lin::fmt_plan(q4lin::FMT_Q4, n, k, t, &fp, true)) {
    *p = SwigluPlan{SW_FMT, r2, 0, 0};
    return true;
  }
  if (r2 == Q4LIN_ROUTE_DECODE || r2 == Q4LIN_ROUTE_SKINNY) {
    *p = SwigluPlan{SW_FUSED, r2, al256((size_t)(n * t * 4)), 2 * al256((size_t)(n * t * 4))};
    return true;
  }
  const int r1 = pick_route(n, k, t);
  if (r1 == Q4LIN_ROUTE_TILED && !q4lin::tiled_shape_ok(n, k, t)) return false;
  if (r1 == Q4LIN_ROUTE_TILED && q4lin::tiled_glu_ok(n, k, t)) {
    *p = SwigluPlan{SW_TGLU, r1, 0, q4lin::tiled_glu_workspace_bytes(n, k, t)};
    return true;
  }
  if (r1 == Q4LIN_ROUTE_TILED) {
    *p = SwigluPlan{SW_TILED, r1, 0, q4lin::tiled_pair_workspace_bytes(n, n, k, t, true)};
  } else if (r1 == Q4LIN_ROUTE_MID) {
    const size_t half = al256((size_t)(n * t * 4));
    *p = SwigluPlan{SW_MID, r1, half, 2 * half};
  } else {
    *p = SwigluPlan{SW_SPLIT, r1, al256((size_t)(n * t * 4)), 2 * al256((size_t)(n * t * 4))};
  }
  return true;
}

hipError_t launch_sums(int route, const q4lin::GemvArgs& a, hipStream_t s) {
  if (route == Q4LIN_ROUTE_DECODE) return q4lin::launch_decode(a, s);
  if (route == Q4LIN_ROUTE_SKINNY) return q4lin::launch_skinny(a, s);
  return q4lin::launch_gemv(a, s);
}

// ---------------------------------------------------------------------------
// The no-allocation variant's scratch: a static device array (each GPU the
// library runs on holds its own copy until the process ends).  Host code
// never uses the array's name as an address: the device address is fetched
// once per device with hipGetSymbolAddress and kept in scratch_dev.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices];  // device address of `scratch` per device, null until first needed

// The current device's address of the scratch array (looked up on the first
// call on that device, with that device current).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return Q4LIN_E_LAUNCH;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return Q4LIN_E_LAUNCH;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return Q4LIN_OK;
}

}  // namespace

extern "C" {

int64_t q4lin_noalloc_scratch_bytes(void) { return (int64_t)kScratchBytes; }

int64_t q4lin_fmt_weight_bytes(int fmt, int64_t n, int64_t k) {
  if (n < 0 || k < 64 || (k % 64) != 0 || n > kMaxN || k > kMaxK) return -Q4LIN_E_SHAPE;
  switch (fmt) {
    case Q4LIN_FMT_Q4G64_F16S: return n * (k / 64) * 34;
    case Q4LIN_FMT_Q5G64_F16S: return n * (k / 64) * 42;
    case Q4LIN_FMT_Q6G64_F16S: return n * (k / 64) * 50;
    case Q4LIN_FMT_W8G32_F16S: return n * (k / 32) * 34;
    case Q4LIN_FMT_NVFP4: return n * (k / 16) * 9;
    case Q4LIN_FMT_BF16: return 2 * n * k;
    default: return -Q4LIN_E_FORMAT;
  }
}

int64_t q4lin_fmt_workspace_bytes(int fmt, int64_t n, int64_t k, int64_t t) {
  if (fmt == Q4LIN_FMT_Q4G64_F16S) return q4lin_workspace_bytes(n, k, t);
  if (fmt < Q4LIN_FMT_Q5G64_F16S || fmt > Q4LIN_FMT_BF16) return -Q4LIN_E_FORMAT;
  if (!shape_ok(n, k, t) || 2 * n * k >= kMaxBytes) return -Q4LIN_E_SHAPE;
  return 0;
}

int q4lin_linear_fmt(int fmt, const void* x, const void* w, const void* w_hi, const void* scales, void* y,
                     int64_t n, int64_t k, int64_t t, void* workspace, size_t workspace_bytes, void* stream) {
  if (fmt == Q4LIN_FMT_Q4G64_F16S)
    return q4lin_linear(x, w, scales, y, n, k, t, workspace, workspace_bytes, stream);
  if (fmt < Q4LIN_FMT_Q5G64_F16S || fmt > Q4LIN_FMT_BF16) return Q4LIN_E_FORMAT;
  if (!shape_ok(n, k, t) || 2 * n * k >= kMaxBytes) return Q4LIN_E_SHAPE;
  if (n == 0 || t == 0) return Q4LIN_OK;
  const bool has_hi = fmt == Q4LIN_FMT_Q5G64_F16S || fmt == Q4LIN_FMT_Q6G64_F16S;
  const bool has_sc = fmt != Q4LIN_FMT_BF16;
  if (!x || !w || !y || (has_hi && !w_hi) || (has_sc && !scales)) return Q4LIN_E_NULL;
  const uintptr_t hi_align = fmt == Q4LIN_FMT_Q5G64_F16S ? 4 : 8;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 2) || (has_hi && !aligned(w_hi, hi_align)) ||
      (has_sc && !aligned(scales, 2)))
    return Q4LIN_E_ALIGN;
  q4lin::FmtPlan plan;
  if (!q4lin::fmt_plan(fmt, n, k, t, &plan)) return Q4LIN_E_SHAPE;
  (void)workspace;
  (void)workspace_bytes;
  const q4lin::FmtArgs a{fmt, x, w, w_hi, scales, y, n, k, t};
  const hipError_t e = q4lin::launch_fmt(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? Q4LIN_OK : Q4LIN_E_LAUNCH;
}

int q4lin_linear_noalloc(const void* x, const void* codes, const void* scales, void* y,
                         int64_t n, int64_t k, int64_t t, void* stream) {
  int route = Q4LIN_ROUTE_NONE;
  const int st = check_linear(x, codes, scales, nullptr, y, n, k, t, &route);
  if (st != Q4LIN_OK || route == Q4LIN_ROUTE_NONE) return st;
  const size_t need = route_workspace(route, n, k, t);
  if (need > kScratchBytes) return Q4LIN_E_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    const int sa = scratch_address(&ws);
    if (sa != Q4LIN_OK) return sa;
  }
  return run_linear(x, codes, scales, nullptr, y, n, k, t, ws, need, stream);
}

int64_t q4lin_swiglu_workspace_bytes(int64_t n, int64_t k, int64_t t) {
  SwigluPlan p;
  if (!swiglu_plan(n, k, t, &p)) return -Q4LIN_E_SHAPE;
  if (n == 0 || t == 0) return 0;
  return (int64_t)p.total;
}

int q4lin_linear_swiglu(const void* x, const void* codes_gate, const void* scales_gate, const void* codes_up,
                        const void* scales_up, void* y, int64_t n, int64_t k, int64_t t,
                        void* workspace, size_t workspace_bytes, void* stream) {
  SwigluPlan p;
  if (!swiglu_plan(n, k, t, &p)) return Q4LIN_E_SHAPE;
  if (n == 0 || t == 0) return Q4LIN_OK;
  if (!x || !codes_gate || !scales_gate || !codes_up || !scales_up || !y) return Q4LIN_E_NULL;
  if (!aligned(x, 16) || !aligned(codes_gate, 16) || !aligned(scales_gate, 2) || !aligned(codes_up, 16) ||
      !aligned(scales_up, 2) || !aligned(y, 2))
    return Q4LIN_E_ALIGN;
  if (workspace_bytes < p.total) return Q4LIN_E_WORKSPACE;
  if (p.total > 0) {
    if (!workspace) return Q4LIN_E_NULL;
    if (!aligned(workspace, 256)) return Q4LIN_E_ALIGN;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* w0 = static_cast<uint8_t*>(workspace);
  uint8_t* w1 = w0 + p.half;
  q4lin::SumSource sg{reinterpret_cast<const float*>(w0), nullptr, nullptr, 1, 0};
  q4lin::SumSource su{reinterpret_cast<const float*>(w1), nullptr, nullptr, 1, 0};
  hipError_t e = hipSuccess;
  if (p.mode == SW_GLU) {
    // one pass: every workgroup takes the same rows of both weights and
    // stores bf16(silu(G) U) itself
    q4lin::GemvArgs a{x, codes_gate, scales_gate, y, n, k, t};
    a.codes2 = codes_up;
    a.scales2 = scales_up;
    a.n2 = n;
    a.glu = true;
    e = q4lin::launch_decode(a, s);
    return e == hipSuccess ? Q4LIN_OK : Q4LIN_E_LAUNCH;
  }
  if (p.mode == SW_FMT) {
    q4lin::FmtArgs a{q4lin::FMT_Q4, x, codes_gate, nullptr, scales_gate, y, n, k, t};
    a.lo2 = codes_up;
    a.sc2 = scales_up;
    a.n2 = n;
    a.glu = true;
    e = q4lin::launch_fmt(a, s);
    return e == hipSuccess ? Q4LIN_OK : Q4LIN_E_LAUNCH;
  }
  if (p.mode == SW_TGLU) {
    // one activation preparation and one tiled launch whose tiles take the
    // same rows of both weights and store bf16(silu(G) U) themselves
    const q4lin::TiledArgs a{x, codes_gate, scales_gate, y, n, k, t, workspace, q4lin::tiled_pick_config(2 * n, k, t)};
    e = q4lin::launch_tiled_glu(a, codes_up, scales_up, s);
    return e == hipSuccess ? Q4LIN_OK : Q4LIN_E_LAUNCH;
  }
  if (p.mode == SW_FUSED) {
    q4lin::GemvArgs a{x, codes_gate, scales_gate, w0, n, k, t};
    a.codes2 = codes_up;
    a.scales2 = scales_up;
    a.y2 = w1;
    a.n2 = n;
    a.f32 = true;
    e = launch_sums(p.route, a, s);
  } else if (p.mode == SW_SPLIT) {
    q4lin::GemvArgs a{x, codes_gate, scales_gate, w0, n, k, t};
    a.f32 = true;
    e = launch_sums(p.route, a, s);
    if (e == hipSuccess) {
      q4lin::GemvArgs b{x, codes_up, scales_up, w1, n, k, t};
      b.f32 = true;
      e = launch_sums(p.route, b, s);
    }
  } else if (p.mode == SW_MID) {
    q4lin::GemvArgs a{x, codes_gate, scales_gate, w0, n, k, t};
    a.f32 = true;
    e = q4lin::launch_fmt(q4_fmt_args(a), s);
    if (e == hipSuccess) {
      q4lin::GemvArgs b{x, codes_up, scales_up, w1, n, k, t};
      b.f32 = true;
      e = q4lin::launch_fmt(q4_fmt_args(b), s);
    }
  } else {
    // both weights' tiles in one launch after one activation preparation;
    // their raw binary32 sums stay in the workspace for the combine
    q4lin::TiledArgs a{x, codes_gate, scales_gate, y, n, k, t, w0, q4lin::tiled_pick_config(2 * n, k, t)};
    a.f32 = true;
    const q4lin::TiledPairArgs pa{a, codes_up, scales_up, y, n};
    e = q4lin::launch_tiled_pair(pa, &sg, &su, s);
  }
  if (e == hipSuccess) e = q4lin::launch_swiglu_combine(sg, su, y, n, t, s);
  return e == hipSuccess ? Q4LIN_OK : Q4LIN_E_LAUNCH;
}


int64_t q4lin_workspace_bytes(int64_t n, int64_t k, int64_t t) {
  if (!shape_ok(n, k, t)) return -Q4LIN_E_SHAPE;
  const int route = pick_route(n, k, t);
  if (route == Q4LIN_ROUTE_TILED && !q4lin::tiled_shape_ok(n, k, t)) return -Q4LIN_E_SHAPE;
  return (int64_t)route_workspace(route, n, k, t);
}

int q4lin_route(int64_t n, int64_t k, int64_t t) {
  if (!shape_ok(n, k, t)) return -Q4LIN_E_SHAPE;
  return pick_route(n, k, t);
}

int q4lin_linear(const void* x, const void* codes, const void* scales, void* y,
                 int64_t n, int64_t k, int64_t t,
                 void* workspace, size_t workspace_bytes, void* stream) {
  return run_linear(x, codes, scales, nullptr, y, n, k, t, workspace, workspace_bytes, stream);
}

int q4lin_linear_pair(const void* x, const void* codes1, const void* scales1, void* y1, int64_t n1,
                      const void* codes2, const void* scales2, void* y2, int64_t n2, int64_t k, int64_t t,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!shape_ok(n1, k, t) || !shape_ok(n2, k, t) || !shape_ok(n1 + n2, k, t)) return Q4LIN_E_SHAPE;
  if (n1 == 0 || n2 == 0 || t == 0) {  // one plane or none: the plain op
    return n2 == 0 ? run_linear(x, codes1, scales1, nullptr, y1, n1, k, t, workspace, workspace_bytes, stream)
                   : run_linear(x, codes2, scales2, nullptr, y2, n2, k, t, workspace, workspace_bytes, stream);
  }
  const int route = pick_route(n1 + n2, k, t);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (pair_on_tiled(route, n1, n2, k, t)) {
    // the many-token route: one activation preparation, one launch for both
    // weights' tiles
    if (!x || !codes1 || !scales1 || !y1 || !codes2 || !scales2 || !y2) return Q4LIN_E_NULL;
    if (!aligned(x, 16) || !aligned(codes1, 16) || !aligned(scales1, 2) || !aligned(y1, 2) ||
        !aligned(codes2, 16) || !aligned(scales2, 2) || !aligned(y2, 2))
      return Q4LIN_E_ALIGN;
    const size_t need = q4lin::tiled_pair_workspace_bytes(n1, n2, k, t, false);
    if (workspace_bytes < need) return Q4LIN_E_WORKSPACE;
    if (!workspace) return Q4LIN_E_NULL;
    if (!aligned(workspace, 256)) return Q4LIN_E_ALIGN;
    q4lin::TiledPairArgs pa{q4lin::TiledArgs{x, codes1, scales1, y1, n1, k, t, workspace,
                                              q4lin::tiled_pick_config(n1 + n2, k, t)},
                            codes2, scales2, y2, n2};
    const hipError_t e = q4lin::launch_tiled_pair(pa, nullptr, nullptr, s);
    return e == hipSuccess ? Q4LIN_OK : Q4LIN_E_LAUNCH;
  }
  if (pair_on_fmt(route, n1, n2, k, t)) {
    if (!x || !codes1 || !scales1 || !y1 || !codes2 || !scales2 || !y2) return Q4LIN_E_NULL;
    if (!aligned(x, 16) || !aligned(codes1, 16) || !aligned(scales1, 2) || !aligned(y1, 2) ||
        !aligned(codes2, 16) || !aligned(scales2, 2) || !aligned(y2, 2))
      return Q4LIN_E_ALIGN;
    q4lin::FmtArgs a{q4lin::FMT_Q4, x, codes1, nullptr, scales1, y1, n1, k, t};
    a.lo2 = codes2;
    a.sc2 = scales2;
    a.y2 = y2;
    a.n2 = n2;
    const hipError_t e = q4lin::launch_fmt(a, s);
    return e == hipSuccess ? Q4LIN_OK : Q4LIN_E_LAUNCH;
  }
  if (route != Q4LIN_ROUTE_DECODE && route != Q4LIN_ROUTE_SKINNY) {
    // the wide-K routes: one launch sequence per weight
    const int s1 = run_linear(x, codes1, scales1, nullptr, y1, n1, k, t, workspace, workspace_bytes, stream);
    if (s1 != Q4LIN_OK) return s1;
    return run_linear(x, codes2, scales2, nullptr, y2, n2, k, t, workspace, workspace_bytes, stream);
  }
  if (!x || !codes1 || !scales1 || !y1 || !codes2 || !scales2 || !y2) return Q4LIN_E_NULL;
  if (!aligned(x, 16) || !aligned(codes1, 16) || !aligned(scales1, 2) || !aligned(y1, 2) ||
      !aligned(codes2, 16) || !aligned(scales2, 2) || !aligned(y2, 2))
    return Q4LIN_E_ALIGN;
  q4lin::GemvArgs ga{x, codes1, scales1, y1, n1, k, t};
  ga.codes2 = codes2;
  ga.scales2 = scales2;
  ga.y2 = y2;
  ga.n2 = n2;
  const hipError_t e = route == Q4LIN_ROUTE_DECODE ? q4lin::launch_decode(ga, s) : q4lin::launch_skinny(ga, s);
  return e == hipSuccess ? Q4LIN_OK : Q4LIN_E_LAUNCH;
}

int64_t q4lin_pair_workspace_bytes(int64_t n1, int64_t n2, int64_t k, int64_t t) {
  if (!shape_ok(n1, k, t) || !shape_ok(n2, k, t) || !shape_ok(n1 + n2, k, t)) return -Q4LIN_E_SHAPE;
  const int route = pick_route(n1 + n2, k, t);
  if (n1 > 0 && n2 > 0 && (route == Q4LIN_ROUTE_DECODE || route == Q4LIN_ROUTE_SKINNY || route == Q4LIN_ROUTE_MID))
    return 0;
  if (n1 > 0 && n2 > 0 && t > 0 && pair_on_tiled(route, n1, n2, k, t))
    return (int64_t)q4lin::tiled_pair_workspace_bytes(n1, n2, k, t, false);
  const size_t w1 = route_workspace(pick_route(n1, k, t), n1, k, t);
  const size_t w2 = route_workspace(pick_route(n2, k, t), n2, k, t);
  return (int64_t)(w1 > w2 ? w1 : w2);
}

int q4lin_linear_add(const void* x, const void* codes, const void* scales, const void* residual, void* y,
                     int64_t n, int64_t k, int64_t t,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (shape_ok(n, k, t) && n > 0 && t > 0 && !residual) return Q4LIN_E_NULL;
  return run_linear(x, codes, scales, residual, y, n, k, t, workspace, workspace_bytes, stream);
}

const char* q4lin_status_string(int status) {
  switch (status) {
    case Q4LIN_OK: return "ok";
    case Q4LIN_E_NULL: return "a required pointer is NULL";
    case Q4LIN_E_SHAPE: return "shape outside the contract (K a positive multiple of 64, sizes within limits)";
    case Q4LIN_E_ALIGN: return "pointer misaligned (x, codes: 16 B; scales, y, residual: 2 B; workspace: 256 B)";
    case Q4LIN_E_WORKSPACE: return "workspace smaller than q4lin_workspace_bytes()";
    case Q4LIN_E_LAUNCH: return "kernel launch failed";
    case Q4LIN_E_FORMAT: return "unknown weight format";
    default: return "unknown status";
  }
}

int q4lin_version(void) { return 220; }

}  // extern "C"
