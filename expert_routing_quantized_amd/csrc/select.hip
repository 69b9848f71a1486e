// Exact top-k selection kernel: one block of kSelectThreads threads per
// token runs select_block (the algorithm and its bound are described in
// select_block.h).

#include "select_block.h"

namespace moe {

template <int ACT>
__global__ __launch_bounds__(kSelectThreads) void select_kernel(SelectArgs a) {
  const int t = blockIdx.x;
  select_block<ACT>(a, t, a.idx + size_t(t) * a.k, a.gates + size_t(t) * a.k);
}

SelectArgs make_select_args(const Layer& L, const void* x, const void* z, bool z32, const float* gmax,
                            const double* xnorm, int32_t* idx, float* gates, const RouterBound& rb) {
  SelectArgs a;
  a.R = L.router_eh;
  a.bias = L.d.router_bias;
  a.x = x;
  a.z = z;
  a.z32 = z32 ? 1 : 0;
  a.gmax = gmax;
  a.xnorm = xnorm;
  a.H = L.d.hidden;
  a.E = L.d.n_experts;
  a.k = L.d.top_k;
  a.idx = idx;
  a.gates = gates;
  a.dev_flag = L.dev_flag;
  auto gamma = [](int n, double u) { return n * u / (1.0 - n * u); };
  a.bt_unit = (gamma(rb.d32, 0x1p-23) + gamma(rb.d64, 0x1p-52)) * 1.01 * L.norm_max;
  // absolute term: every binary32 operation may also lose up to 2^-126 to
  // underflow (products flushed to zero included: one per element of x)
  a.bt_abs = (rb.d32 + L.d.hidden) * 0x1p-125 + rb.d64 * 0x1p-1021;
  a.rel = 0x1p-52;
  if (z32) {
    // stored in binary32: one more rounding, |fl32(v) - v| <= 2^-24 |v|
    // (|v| <= |fl32(v)| (1 + 2^-23)), or 2^-126 where it underflows
    a.rel = (0x1p-24 + 0x1p-52) * (1.0 + 0x1p-20);
    a.bt_abs += 0x1p-125;
  }
  a.force_exact = (L.d.flags & MOE_LAYER_FORCE_EXACT_REFINE) ? 1 : 0;
  return a;
}

hipError_t launch_select_impl(const Layer& L, const void* x, int T, const void* z, bool z32,
                              const float* gmax, const double* xnorm, int32_t* idx,
                              float* gates, const RouterBound& rb, hipStream_t s) {
  const SelectArgs a = make_select_args(L, x, z, z32, gmax, xnorm, idx, gates, rb);
  if (L.d.act_dtype == MOE_BF16)
    hipLaunchKernelGGL(select_kernel<MOE_BF16>, dim3(T), dim3(kSelectThreads), 0, s, a);
  else
    hipLaunchKernelGGL(select_kernel<MOE_F32>, dim3(T), dim3(kSelectThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
