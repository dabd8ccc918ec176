// q4lin_swiglu.hip -- the LinearSwiGLU combine: Y = bf16(silu(G) * U).
//
// The pages name LinearSwiGLU among the fused Linear variants ("q4-linear.md"
// and "linear-benchmark.md") without defining it; the reading taken here is
// the gated linear unit with the SiLU gate, silu(g) = g / (1 + e^-g), applied
// to the unrounded sums G = Wg x X and U = Wu x X, and one rounding at the
// end.  The matrix routes leave G and U as binary32 sums in the workspace
// (bf16 never touches them); this pass reads both, forms the gate in
// binary64 and rounds the product once to bf16 through binary32, as every
// route's final store does.  Elementwise and HBM-bound: 8 bytes read (16
// with two K-split slices) and 2 written per output.
#include "q4lin_device.h"
#include "q4lin_kernels.h"

namespace q4lin {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ double source_value(const SumSource& s, size_t i, int t, int n) {
  float v = 0.0f;
  for (int k = 0; k < s.ks; ++k) v += s.part[(size_t)k * s.stride + i];  // slices in order
  double d = (double)v;
  if (s.texp != nullptr) d = __builtin_ldexp(d, s.texp[t] - s.rexp[n]);
  // A sum of products that are all zero is +0 by definition (the sum starts
  // at +0); another summation order may give -0 there.  Adding +0 maps -0 to
  // +0 and leaves every other value as it is.
  return d + 0.0;
}

__global__ void __launch_bounds__(kThreads)
swiglu_combine_kernel(SumSource g, SumSource u, uint16_t* __restrict__ y, int N, int64_t total) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kThreads) {
    const int t = (int)(i / N), n = (int)(i - (int64_t)t * N);
    const double gv = source_value(g, (size_t)i, t, n);
    const double uv = source_value(u, (size_t)i, t, n);
    const double silu = gv / (1.0 + exp(-gv));
    y[i] = f32_to_bf16_rne((float)(silu * uv));
  }
}

}  // namespace

hipError_t launch_swiglu_combine(const SumSource& g, const SumSource& u, void* y, int64_t n, int64_t t,
                                 hipStream_t stream) {
  const int64_t total = n * t;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 8192) blocks = 8192;  // grid-stride beyond 2M outputs
  swiglu_combine_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(g, u, static_cast<uint16_t*>(y),
                                                                              (int)n, total);
  return hipGetLastError();
}

}  // namespace q4lin
