// Router GEMV for a few tokens: z[t][e] = fl(sum_h x[t][h] R[e][h] + b[e]).
//
// The pages' routing kernel scores all 24,576 experts of the pool for each
// token (pyshine source tour, Understanding the Architecture, paragraph on
// the three residency tiers and the routing kernel); at batch
// 1 this is a GEMV that only streams the router once, and the hexlives
// dispatch reports that matrix units lose on exactly this shape, so the
// product runs on the vector ALUs.
//
// Layout: the router is read expert-major, row e = the H weights of expert
// e (4 KB for H = 2048 in bf16).  One wave owns one row: chunk c of 8
// elements (16 B in bf16) goes to lane c % 64, so each of the wave's loads
// is 1 KB contiguous, and all of the row's loads are issued at once
// (non-temporal: the router is streamed once per token).  For one token x
// is staged once per block in LDS (its loads issued before the row's) and
// each lane takes the same chunks of it.  Blocks of 4 waves, one block per 4
// experts: a measured sweep of launch shapes on gfx950 put this shape at
// the streaming-read ceiling (about 6.5 TB/s), ahead of fewer, longer-lived
// waves and of larger blocks.  Each block also writes the maximum of its 4
// logits (per token), and block 0 writes ||x||^2, so the selection kernel
// reads 1/4 of the logits' bytes to find its candidates.
//
// Rounding model (used by the selection kernel to bound |z_hat - z|), the
// same for every expert, so identical rows give identical logits: each lane
// accumulates its products in binary32 chains of 8 (one chain per 16-byte
// chunk: fmaf on exact bf16 x bf16 products, or, for several tokens, four
// bf16 dot2 instructions counted as two roundings each), converts each chain
// sum to binary64 (exact), and everything after that -- the chains of the
// lane, the 6-level DPP tree across the wave, the bias -- is binary64:
//   |z_hat - z| <= gamma(d32, 2^-23) sum|p| + gamma(d64, 2^-52) sum|p| + ...
// with d32 = 7 (fmaf) or 8 (dot2) and d64 = log2(CPL) + 7.  Converting once
// per chain instead of once per product keeps the conversion (a slow
// instruction) off the bandwidth-bound path.
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int ACT, int CPL, int NT>
__global__ __launch_bounds__(kRouterWaves * 64) __attribute__((amdgpu_waves_per_eu(NT == 1 ? 8 : 1)))
void router_kernel(
    const void* __restrict__ R, const void* __restrict__ x, const float* __restrict__ bias,
    int H, int E, int T, double* __restrict__ z, float* __restrict__ gmax,
    double* __restrict__ xnorm, int* __restrict__ dev_flag) {
  __shared__ double zl[NT][kRouterWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int e = min(blockIdx.x * kRouterWaves + wave, E - 1);   // waves past E redo E-1, unused
  const bool live = blockIdx.x * kRouterWaves + wave < E;
  const int nch = H >> 3;
  const int t0 = blockIdx.y * NT;
  const int nt = min(NT, T - t0);
  const int G4 = (E + kRouterWaves - 1) / kRouterWaves;

  // One token: the block's threads first load x (16 bytes each) for the
  // block's LDS copy, so each wave reads x from LDS instead of all of it
  // through its own loads (as many bytes as its router row); then every
  // wave's row chunks (longest latency).  Chunk indices past the row are
  // clamped to its last chunk and masked afterwards, so every load is
  // issued unconditionally (no branch between loads).
  constexpr int kXPer = (NT == 1) ? ((ACT == MOE_F32 ? 2 : 1) * CPL + 3) / 4 : 1;   // x pieces per thread
  const int n16 = (ACT == MOE_F32 ? 2 : 1) * nch;                                       // 16-byte pieces of x
  uint4 xq[kXPer];
  if constexpr (NT == 1) {
    const uint4* x16 = reinterpret_cast<const uint4*>(x) + size_t(t0) * n16;
#pragma unroll
    for (int u = 0; u < kXPer; ++u) xq[u] = x16[min((int)threadIdx.x + kRouterWaves * 64 * u, n16 - 1)];
  }
  Chunk<ACT> r[CPL];
#pragma unroll
  for (int s = 0; s < CPL; ++s) {
    const int c = min(s * 64 + lane, nch - 1);
    r[s].load_stream(R, size_t(e) * H + c * 8);
  }
  constexpr bool kPacked = (ACT == MOE_BF16) && (NT > 1);
  if constexpr (kPacked) {
    const float b = (bias != nullptr) ? bias[e] : 0.f;
#pragma unroll
    for (int s = 0; s < CPL; ++s)
      if (s * 64 + lane >= nch) r[s].zero();
    uint4 xp[NT][CPL];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int s = 0; s < CPL; ++s) {
        const int c = min(s * 64 + lane, nch - 1);
        const int tt = min(t, nt - 1);
        xp[t][s] = *reinterpret_cast<const uint4*>(
            reinterpret_cast<const uint16_t*>(x) + size_t(t0 + tt) * H + c * 8);
      }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int s = 0; s < CPL; ++s)
        if (s * 64 + lane >= nch || t >= nt) xp[t][s] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      double acc[CPL];
#pragma unroll
      for (int s = 0; s < CPL; ++s) {
        const uint32_t xw[4] = {xp[t][s].x, xp[t][s].y, xp[t][s].z, xp[t][s].w};
        const uint32_t rw[4] = {r[s].v.x, r[s].v.y, r[s].v.z, r[s].v.w};
        float c = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xw[q]),
                                              __builtin_bit_cast(bf16x2_t, rw[q]), c, false);
        acc[s] = (double)c;
      }
#pragma unroll
      for (int w = 1; w < CPL; w <<= 1)
#pragma unroll
        for (int s = 0; s + w < CPL; s += 2 * w) acc[s] += acc[s + w];
      const double v = wave_sum_f64(acc[0]) + (double)b;
      if (lane == t && t < nt && live) z[size_t(t0 + t) * E + e] = v;
      if (lane == 0) zl[t][wave] = live ? v : -INFINITY;
    }
    if (blockIdx.x == 0) {      // ||x_t||^2 of this block's tokens (binary64 sums of exact squares)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t % kRouterWaves != wave || t >= nt) continue;   // wave-uniform
        double q = 0.0;
#pragma unroll
        for (int s2 = 0; s2 < CPL; ++s2) {
          const uint32_t xw[4] = {xp[t][s2].x, xp[t][s2].y, xp[t][s2].z, xp[t][s2].w};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const double xv = (i & 1) ? bf16_hi(xw[i >> 1]) : bf16_lo(xw[i >> 1]);
            q = fma(xv, xv, q);
          }
        }
        q = wave_sum_f64(q);
        if (lane == 0) xnorm[t0 + t] = q;
      }
    }
  } else {
    // one token: binary32 chains of 8 exact products, then binary64.  x
    // (before the row) and the bias (right behind it) are loaded with no
    // branch or wait in between (a bias load under a null-pointer branch
    // made every wave wait for its row before it even asked for x, so the
    // layer passes zeros instead of null); chunks past the row end (clamped
    // loads) are masked by selects on both operands, so they add exact zeros.
    static_assert(NT == 1, "unpacked path handles one token per block row");
    extern __shared__ uint4 sx[];                      // x of the token, n16 pieces + a spare
    const float b = bias[e];                           // never null on this path (zeros without a bias)
    // unconditional stores (pieces past x go to a spare slot that is never
    // read): a store under a branch let the compiler sink the x load behind
    // the row loads
#pragma unroll
    for (int u = 0; u < kXPer; ++u) {
      const int c = threadIdx.x + kRouterWaves * 64 * u;
      sx[c < n16 ? c : n16] = xq[u];
    }
    __syncthreads();
    Chunk<ACT> xc[CPL];
#pragma unroll
    for (int s = 0; s < CPL; ++s) {
      const int c = min(s * 64 + lane, nch - 1);
      if constexpr (ACT == MOE_F32) {
        const uint4 p0 = sx[2 * c], p1 = sx[2 * c + 1];
        xc[s].a = make_float4(__uint_as_float(p0.x), __uint_as_float(p0.y), __uint_as_float(p0.z), __uint_as_float(p0.w));
        xc[s].b = make_float4(__uint_as_float(p1.x), __uint_as_float(p1.y), __uint_as_float(p1.z), __uint_as_float(p1.w));
      } else {
        xc[s].v = sx[c];
      }
    }
    auto xf_get = [](const Chunk<ACT>& c, int i, bool in) { return in ? c.get(i) : 0.f; };
    // chunks past the row end: both operands zeroed by word selects
    auto masked = [](Chunk<ACT> c, bool in) {
      if constexpr (ACT == MOE_BF16) {
        c.v = make_uint4(in ? c.v.x : 0u, in ? c.v.y : 0u, in ? c.v.z : 0u, in ? c.v.w : 0u);
      } else {
        c.a = make_float4(in ? c.a.x : 0.f, in ? c.a.y : 0.f, in ? c.a.z : 0.f, in ? c.a.w : 0.f);
        c.b = make_float4(in ? c.b.x : 0.f, in ? c.b.y : 0.f, in ? c.b.z : 0.f, in ? c.b.w : 0.f);
      }
      return c;
    };
    double acc[CPL];
#pragma unroll
    for (int s = 0; s < CPL; ++s) {
      const bool in = s * 64 + lane < nch;
      const Chunk<ACT> xm = masked(xc[s], in), rm = masked(r[s], in);
      float c = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) c = fmaf(xm.get(i), rm.get(i), c);
      acc[s] = (double)c;
    }
#pragma unroll
    for (int w = 1; w < CPL; w <<= 1)
#pragma unroll
      for (int s = 0; s + w < CPL; s += 2 * w) acc[s] += acc[s + w];
    const double v = wave_sum_f64(acc[0]) + (double)b;
    if (lane == 0 && live) z[size_t(t0) * E + e] = v;
    if (lane == 0) zl[0][wave] = live ? v : -INFINITY;
    if (blockIdx.x == 0 && wave == 0) {   // ||x||^2: exact squares summed in binary64 (no underflow)
      double q = 0.0;
#pragma unroll
      for (int s = 0; s < CPL; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const double xs = xf_get(xc[s], i, s * 64 + lane < nch);
          q = fma(xs, xs, q);
        }
      q = wave_sum_f64(q);
      if (lane == 0) xnorm[t0] = q;
    }
  }
  // maximum of the block's logits per token, rounded up to binary32 (an
  // upper bound: the selection scans a group whenever it might hold a
  // candidate); NaN counts as -inf and raises the non-finite flag.
  __syncthreads();
  if (threadIdx.x < nt) {
    const int t = threadIdx.x;
    double m = -INFINITY;
    bool bad = false;
    for (int w = 0; w < kRouterWaves; ++w) {
      const double v = zl[t][w];
      const bool lw = blockIdx.x * kRouterWaves + w < E;
      if (lw && !isfinite(v)) bad = true;
      if (!isnan(v)) m = fmax(m, v);
    }
    if (bad) atomicOr(dev_flag, kDevNonFinite);
    gmax[size_t(t0 + t) * G4 + blockIdx.x] = isnan(m) ? -INFINITY : f64_to_f32_up(m);
  }
}

template <int ACT, int NT>
static hipError_t launch_cpl(const Layer& L, const void* x, int T, double* z, float* gmax,
                             double* xnorm, hipStream_t s) {
  const int H = L.d.hidden, E = L.d.n_experts;
  const int cpl = (H / 8 + 63) / 64;
  dim3 grid((E + kRouterWaves - 1) / kRouterWaves, 1);
#define MOE_ROUTER_CASE(C)                                                                    \
  if (cpl <= C) {                                                                             \
    constexpr int NTX = (ACT == MOE_BF16 && NT > 1) ? ((NT * C > 32) ? 32 / C : NT) : 1;    \
    grid.y = (T + NTX - 1) / NTX;                                                             \
    const size_t lds = (NTX == 1) ? (size_t(H / 8) * (ACT == MOE_F32 ? 2 : 1) + 1) * 16 : 0;  \
    hipLaunchKernelGGL((router_kernel<ACT, C, NTX>), grid, dim3(kRouterWaves * 64), lds, s,   \
                       L.router_eh, x, router_bias_or_zero(L), H, E, T, z, gmax, xnorm, L.dev_flag); \
    return hipGetLastError();                                                                 \
  }
  MOE_ROUTER_CASE(1)
  MOE_ROUTER_CASE(2)
  MOE_ROUTER_CASE(4)
  MOE_ROUTER_CASE(8)
  MOE_ROUTER_CASE(16)
#undef MOE_ROUTER_CASE
  return hipErrorInvalidValue;
}

// Error model of the kernel chosen for (act dtype, T): see the header comment.
RouterBound router_bound(const Layer& L, int T) {
  const int cpl = (L.d.hidden / 8 + 63) / 64;
  int lg = 0;
  while ((1 << lg) < cpl) ++lg;
  RouterBound b;
  if (router_uses_big_tiles(L, T)) {   // see mfma.hip
    b.d32 = 17 * (L.d.hidden / 16);
    b.d64 = 1;
    return b;
  }
  if (router_uses_mfma(L, T)) {
    b.d32 = 136;
    b.d64 = (L.d.hidden + 127) / 128 + 1;
    return b;
  }
  if (router_uses_skinny(L, T)) {
    b.d32 = 33;
    b.d64 = (L.d.hidden + 127) / 128 + 4;
    return b;
  }
  const bool dot2 = (L.d.act_dtype == MOE_BF16 && T > 1);
  b.d32 = dot2 ? 8 : 7;
  b.d64 = lg + 7;
  return b;
}

hipError_t launch_router(const Layer& L, const void* x, int T, double* z, float* gmax,
                         double* xnorm, hipStream_t s) {
  if (router_uses_skinny(L, T)) return launch_router_skinny(L, x, T, z, gmax, xnorm, s);
  if (L.d.act_dtype == MOE_F32) return launch_cpl<MOE_F32, 1>(L, x, T, z, gmax, xnorm, s);
  if (T == 1) return launch_cpl<MOE_BF16, 1>(L, x, T, z, gmax, xnorm, s);
  return launch_cpl<MOE_BF16, 8>(L, x, T, z, gmax, xnorm, s);
}

}  // namespace moe
