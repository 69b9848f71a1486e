// Layer-creation kernels: expert-major copy of an [H][E] router and the
// per-expert router row norms that bound the router's rounding error.
#include "moe_internal.h"

namespace moe {

template <typename Tv>
__global__ void transpose_kernel(const Tv* __restrict__ src, Tv* __restrict__ dst, int H, int E) {
  __shared__ Tv tile[32][33];
  const int e0 = blockIdx.x * 32, h0 = blockIdx.y * 32;
  for (int r = threadIdx.y; r < 32; r += blockDim.y) {
    const int h = h0 + r, e = e0 + threadIdx.x;
    if (h < H && e < E) tile[r][threadIdx.x] = src[size_t(h) * E + e];
  }
  __syncthreads();
  for (int r = threadIdx.y; r < 32; r += blockDim.y) {
    const int e = e0 + r, h = h0 + threadIdx.x;
    if (h < H && e < E) dst[size_t(e) * H + h] = tile[threadIdx.x][r];
  }
}

hipError_t launch_transpose_router(const Layer& L, void* dst, hipStream_t s) {
  const int H = L.d.hidden, E = L.d.n_experts;
  dim3 grid((E + 31) / 32, (H + 31) / 32), block(32, 8);
  if (L.d.act_dtype == MOE_BF16)
    hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, block, 0, s,
                       reinterpret_cast<const uint16_t*>(L.d.router_w), reinterpret_cast<uint16_t*>(dst), H, E);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, block, 0, s,
                       reinterpret_cast<const float*>(L.d.router_w), reinterpret_cast<float*>(dst), H, E);
  return hipGetLastError();
}

__global__ void zero_f32_kernel(float* p) { *p = 0.f; }

// One wave per expert row: f64 sum of squares (exact squares), norm rounded
// up to fp32; the maximum goes to norms[E] via an integer max on the bits
// (non-negative floats order like their bit patterns).
template <int ACT>
__global__ __launch_bounds__(256) void norms_kernel(const void* R, int H, int E, float* norms) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  double s = 0.0;
  for (int c = lane; c < H / 8; c += 64) {
    Chunk<ACT> ch;
    ch.load(R, size_t(e) * H + c * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double v = ch.get(i);
      s += v * v;
    }
  }
  s = wave_sum_d(s) * (1.0 + 1e-12);
  if (lane == 0) {
    float n = (float)sqrt(s);
    n = nextafterf(n, INFINITY);
    norms[e] = n;
    atomicMax(reinterpret_cast<unsigned int*>(norms + E), __float_as_uint(n));
  }
}

hipError_t launch_router_norms(const Layer& L, hipStream_t s) {
  const int H = L.d.hidden, E = L.d.n_experts;
  hipLaunchKernelGGL(zero_f32_kernel, dim3(1), dim3(1), 0, s, L.norms + E);
  if (L.d.act_dtype == MOE_BF16)
    hipLaunchKernelGGL(norms_kernel<MOE_BF16>, dim3((E + 3) / 4), dim3(256), 0, s, L.router_eh, H, E, L.norms);
  else
    hipLaunchKernelGGL(norms_kernel<MOE_F32>, dim3((E + 3) / 4), dim3(256), 0, s, L.router_eh, H, E, L.norms);
  return hipGetLastError();
}

}  // namespace moe

namespace moe {

// ------------------------------------------------------------ hot region
// dst slot s <- src expert ids[s]: `bytes` bytes each, copied in units of U
// (the host picks the widest unit that the pointers' alignment and `bytes`
// allow).  Grid: (units / 256 rounded up, n).
template <typename U>
__global__ __launch_bounds__(256) void gather_experts_kernel(const U* __restrict__ src, U* __restrict__ dst,
                                                             size_t units, const int32_t* __restrict__ ids) {
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= units) return;
  const int slot = blockIdx.y;
  dst[size_t(slot) * units + i] = src[size_t(ids[slot]) * units + i];
}

hipError_t launch_gather_experts(const void* src, void* dst, size_t bytes, const int32_t* ids, int n,
                                 hipStream_t s) {
  if (n <= 0 || bytes == 0) return hipSuccess;
  const uintptr_t al = reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst) | uintptr_t(bytes);
  auto go = [&](auto unit) {
    using U = decltype(unit);
    const size_t units = bytes / sizeof(U);
    hipLaunchKernelGGL(gather_experts_kernel<U>, dim3(unsigned((units + 255) / 256), unsigned(n)), dim3(256), 0, s,
                       reinterpret_cast<const U*>(src), reinterpret_cast<U*>(dst), units, ids);
  };
  if (al % 16 == 0) go(uint4{});
  else if (al % 4 == 0) go(uint32_t{});
  else if (al % 2 == 0) go(uint16_t{});
  else go(uint8_t{});
  return hipGetLastError();
}

// counts[e] += 1 for every valid index among idx[0, n) (the frequency
// record from which a caller picks the hot set).
__global__ __launch_bounds__(256) void expert_counts_kernel(const int32_t* __restrict__ idx, int n, int E,
                                                            uint32_t* __restrict__ counts) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int e = idx[i];
  if (e >= 0 && e < E) atomicAdd(&counts[e], 1u);
}

hipError_t launch_expert_counts(const int32_t* idx, int n, int E, uint32_t* counts, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(expert_counts_kernel, dim3((n + 255) / 256), dim3(256), 0, s, idx, n, E, counts);
  return hipGetLastError();
}

}  // namespace moe
