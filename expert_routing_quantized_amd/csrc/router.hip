// Router GEMV for a few tokens: z[t][e] = fl(sum_h x[t][h] R[e][h] + b[e]).
//
// The pages' routing kernel scores all 24,576 experts of the pool for each
// token (pyshine source tour, "Three tiers, one residency table"); at batch
// 1 this is a GEMV that only streams the router once, and the hexlives
// dispatch reports that matrix units lose on exactly this shape, so the
// product runs on the vector ALUs.
//
// Layout: the router is read expert-major, row e = the H weights of expert
// e (4 KB for H = 2048 in bf16).  A wave owns one row at a time: chunk c of
// 8 elements (16 B in bf16) goes to lane c % 64, so each of the wave's loads
// is 1 KB contiguous.  Each lane keeps the same chunks of x in registers.
//
// Rounding model (used by the selection kernel to bound |z_hat - z|): a lane
// accumulates its 8*CPL products in a fixed order with one fp32 rounding per
// product (fmaf on exact bf16 x bf16 products, or the bf16 dot2 instruction
// counted as two roundings per pair), then a 6-level butterfly, then the
// bias: depth 8*CPL + 7 for every expert, independent of e, so identical
// rows give identical logits.
//
// Each block owns kRouterEPB = 64 consecutive experts and also writes the
// k-th largest of its 64 logits per token (a lower bound on the token's
// k-th largest logit, used to pre-filter candidates).
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int ACT, int CPL, int NT>
__global__ __launch_bounds__(512) void router_kernel(
    const void* __restrict__ R, const void* __restrict__ x, const float* __restrict__ bias,
    int H, int E, int T, int k, float* __restrict__ z, float* __restrict__ tau, int ntau) {
  constexpr int kWaves = 8;
  constexpr int kPerWave = kRouterEPB / kWaves;   // 8 experts per wave
  constexpr int kUnroll = (ACT == MOE_BF16) ? 4 : 2;
  __shared__ float zl[NT][kRouterEPB];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nch = H >> 3;
  const int t0 = blockIdx.y * NT;
  const int nt = min(NT, T - t0);

  // x chunks of this lane: floats for one token, packed bf16 pairs for several.
  constexpr bool kPacked = (ACT == MOE_BF16) && (NT > 1);
  float xf[kPacked ? 1 : CPL][kPacked ? 1 : 8];
  uint4 xp[kPacked ? NT : 1][kPacked ? CPL : 1];
  if constexpr (kPacked) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int s = 0; s < CPL; ++s) {
        const int c = s * 64 + lane;
        xp[t][s] = make_uint4(0, 0, 0, 0);
        if (c < nch && t < nt)
          xp[t][s] = *reinterpret_cast<const uint4*>(
              reinterpret_cast<const uint16_t*>(x) + size_t(t0 + t) * H + c * 8);
      }
  } else {
#pragma unroll
    for (int s = 0; s < CPL; ++s) {
      const int c = s * 64 + lane;
      Chunk<ACT> ch;
      if (c < nch) {
        ch.load(x, size_t(t0) * H + c * 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) xf[s][i] = ch.get(i);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) xf[s][i] = 0.f;
      }
    }
  }

  const int e_base = blockIdx.x * kRouterEPB + wave * kPerWave;
  for (int i0 = 0; i0 < kPerWave; i0 += kUnroll) {
    Chunk<ACT> r[kUnroll][CPL];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int e = e_base + i0 + u;
#pragma unroll
      for (int s = 0; s < CPL; ++s) {
        const int c = s * 64 + lane;
        if (e < E && c < nch) {
          r[u][s].load(R, size_t(e) * H + c * 8);
        } else {
          if constexpr (ACT == MOE_BF16) r[u][s].v = make_uint4(0, 0, 0, 0);
          else { r[u][s].a = make_float4(0, 0, 0, 0); r[u][s].b = r[u][s].a; }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int e = e_base + i0 + u;
      const int le = wave * kPerWave + i0 + u;
      const float b = (bias != nullptr && e < E) ? bias[e] : 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float acc = 0.f;
        if constexpr (kPacked) {
#pragma unroll
          for (int s = 0; s < CPL; ++s) {
            const uint32_t xw[4] = {xp[t][s].x, xp[t][s].y, xp[t][s].z, xp[t][s].w};
            const uint32_t rw[4] = {r[u][s].v.x, r[u][s].v.y, r[u][s].v.z, r[u][s].v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xw[q]),
                                                    __builtin_bit_cast(bf16x2_t, rw[q]), acc,
                                                    false);
          }
        } else {
#pragma unroll
          for (int s = 0; s < CPL; ++s)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc = fmaf(xf[s][i], r[u][s].get(i), acc);
        }
        const float v = wave_sum(acc) + b;
        if (lane == t) {
          if (e < E && t < nt) z[size_t(t0 + t) * E + e] = v;
          zl[t][le] = (e < E) ? v : -INFINITY;
        }
      }
    }
  }
  __syncthreads();

  // k-th largest of this block's logits, per token (NaN ranks lowest).
  for (int t = 0; t < nt; ++t) {
    if (threadIdx.x < kRouterEPB) {
      const int j = threadIdx.x;
      const float v = zl[t][j];
      const uint32_t kv = f32_key(v);
      int rank = 0;
      for (int m = 0; m < kRouterEPB; ++m) {
        const uint32_t km = f32_key(zl[t][m]);
        rank += (km > kv) || (km == kv && m < j);
      }
      if (rank == k - 1) tau[size_t(t0 + t) * ntau + blockIdx.x] = isnan(v) ? -INFINITY : v;
    }
    if (k > kRouterEPB && threadIdx.x == 0) tau[size_t(t0 + t) * ntau + blockIdx.x] = -INFINITY;
  }
}

int router_ntau(const Layer& L) { return (L.d.n_experts + kRouterEPB - 1) / kRouterEPB; }

template <int ACT, int NT>
static hipError_t launch_cpl(const Layer& L, const void* x, int T, float* z, float* tau,
                             hipStream_t s) {
  const int H = L.d.hidden, E = L.d.n_experts;
  const int nch = H / 8;
  const int cpl = (nch + 63) / 64;
  const int nb = router_ntau(L);
  dim3 grid(nb, (T + NT - 1) / NT);
#define MOE_ROUTER_CASE(C)                                                                  \
  if (cpl <= C) {                                                                           \
    constexpr int NTX = (ACT == MOE_BF16 && NT > 1) ? ((NT * C > 32) ? 32 / C : NT) : NT; \
    grid.y = (T + NTX - 1) / NTX;                                                           \
    hipLaunchKernelGGL((router_kernel<ACT, C, NTX>), grid, dim3(512), 0, s, L.router_eh, x, \
                       L.d.router_bias, H, E, T, L.d.top_k, z, tau, nb);                    \
    return hipGetLastError();                                                               \
  }
  MOE_ROUTER_CASE(1)
  MOE_ROUTER_CASE(2)
  MOE_ROUTER_CASE(4)
  MOE_ROUTER_CASE(8)
  MOE_ROUTER_CASE(16)
#undef MOE_ROUTER_CASE
  return hipErrorInvalidValue;
}

// Rounding depth of one logit for the kernel chosen for (H, T): see header.
int router_depth(const Layer& L, int T) {
  (void)T;
  const int cpl = (L.d.hidden / 8 + 63) / 64;
  return 8 * cpl + 7;
}

hipError_t launch_router(const Layer& L, const void* x, int T, float* z, float* tau,
                         hipStream_t s) {
  if (L.d.act_dtype == MOE_F32) return launch_cpl<MOE_F32, 1>(L, x, T, z, tau, s);
  if (T == 1) return launch_cpl<MOE_BF16, 1>(L, x, T, z, tau, s);
  return launch_cpl<MOE_BF16, 8>(L, x, T, z, tau, s);
}

}  // namespace moe
