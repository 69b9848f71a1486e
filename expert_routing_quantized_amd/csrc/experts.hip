// Expert GEMVs of one token: h_j = silu(G_e x) * (U_e x) for the k selected
// experts, then out = sum_j g_j D_e h_j.
//
// The pages compute the cached experts with a hand-written GEMV that is
// "already bandwidth-bound"; their tensor-core variant was slower on every
// real shape because a single token fills one row of a 16-row tile (hexlives
// dispatch).  So these are vector-ALU GEMVs: every weight byte is loaded
// once with 16-byte loads, the 4-bit codes are expanded in registers and the
// fp16 block scale is applied to each 32-element partial in fp32 (exact
// dequantisation, nothing rounded to 16 bits).  The router weight is applied
// only in the down/combine kernel (pyshine source tour, "The expert handoff
// is a verified contract").
//
// gate/up: one wave per pair of intermediate rows (gate row i and up row i
// of the same expert), so silu(a)*u is formed in registers; for 4-bit rows
// lane l owns quant block l (32 elements = 16 B of codes + one scale).
// down:    8 lanes per output row; h of all k experts is staged in LDS
// (padded every 32 floats); each lane accumulates g_j times its partial over
// the experts in order j = 0..k-1 and the 8 lanes are summed at the end.
#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + expf(-a)); }

// sum_i nibble_i * xv_i over one 32-element block; codes in 4 dwords.
__device__ __forceinline__ float q4_block_dot(const uint4 w, const float* xv) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float acc = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t lo = ws[q] & 0x0f0f0f0fu;
    const uint32_t hi = (ws[q] >> 4) & 0x0f0f0f0fu;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      acc = fmaf((float)((lo >> (8 * b)) & 0xffu), xv[8 * q + 2 * b], acc);
      acc = fmaf((float)((hi >> (8 * b)) & 0xffu), xv[8 * q + 2 * b + 1], acc);
    }
  }
  return acc;
}

struct DecodeArgs {
  const void* x;
  const int32_t* idx;
  const float* gates;
  const void *wg, *wu, *wd;
  const uint16_t *sg, *su, *sd;
  float* h;          // [k][I]
  float* out;        // [H]
  int H, I, E, k;
  int* dev_flag;
};

// ------------------------------------------------------------ gate/up, 4-bit
// MB = quant blocks per lane (H / 32 / 64 rounded up).
template <int ACT, int MB>
__global__ __launch_bounds__(256) void gateup_q4_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = blockIdx.y;
  const int e = a.idx[j];
  const bool valid = (e >= 0 && e < a.E);
  const int nblk = a.H >> 5;
  float xv[MB][32];
  float xs[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int b = m * 64 + lane;
    xs[m] = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      Chunk<ACT> ch;
      if (b < nblk) {
        ch.load(a.x, b * 32 + c * 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) xv[m][c * 8 + i] = ch.get(i);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) xv[m][c * 8 + i] = 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) xs[m] += xv[m][i];
  }
  constexpr int kRowsPerWave = 2;
  const int i0 = (blockIdx.x * 4 + wave) * kRowsPerWave;
  const size_t rowb = size_t(a.H) / 2;
  uint4 wg[kRowsPerWave][MB], wu[kRowsPerWave][MB];
  float dg[kRowsPerWave][MB], du[kRowsPerWave][MB];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const int i = i0 + r;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int b = m * 64 + lane;
      if (valid && i < a.I && b < nblk) {
        const size_t row = size_t(e) * a.I + i;
        wg[r][m] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.wg) + row * rowb + b * 16);
        wu[r][m] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.wu) + row * rowb + b * 16);
        dg[r][m] = f16_to_f32(a.sg[row * nblk + b]);
        du[r][m] = f16_to_f32(a.su[row * nblk + b]);
      } else {
        wg[r][m] = wu[r][m] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
        dg[r][m] = du[r][m] = 0.f;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    float pa = 0.f, pu = 0.f;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      pa = fmaf(dg[r][m], q4_block_dot(wg[r][m], xv[m]) - 8.f * xs[m], pa);
      pu = fmaf(du[r][m], q4_block_dot(wu[r][m], xv[m]) - 8.f * xs[m], pu);
    }
    const float av = wave_sum(pa), uv = wave_sum(pu);
    const int i = i0 + r;
    if (lane == 0 && i < a.I) a.h[size_t(j) * a.I + i] = valid ? silu_f(av) * uv : NAN;
  }
}

// ------------------------------------------------------------ gate/up, dense
template <int ACT, int WD, int CPL>
__global__ __launch_bounds__(256) void gateup_dense_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = blockIdx.y;
  const int e = a.idx[j];
  const bool valid = (e >= 0 && e < a.E);
  const int nch = a.H >> 3;
  float xv[CPL][8];
#pragma unroll
  for (int s = 0; s < CPL; ++s) {
    const int c = s * 64 + lane;
    Chunk<ACT> ch;
    if (c < nch) {
      ch.load(a.x, c * 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[s][i] = ch.get(i);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[s][i] = 0.f;
    }
  }
  constexpr int kRowsPerWave = 2;
  const int i0 = (blockIdx.x * 4 + wave) * kRowsPerWave;
  Chunk<WD> wg[kRowsPerWave][CPL], wu[kRowsPerWave][CPL];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const int i = i0 + r;
#pragma unroll
    for (int s = 0; s < CPL; ++s) {
      const int c = s * 64 + lane;
      if (valid && i < a.I && c < nch) {
        const size_t row = size_t(e) * a.I + i;
        wg[r][s].load(a.wg, row * a.H + c * 8);
        wu[r][s].load(a.wu, row * a.H + c * 8);
      } else {
        if constexpr (WD == MOE_BF16) { wg[r][s].v = wu[r][s].v = make_uint4(0, 0, 0, 0); }
        else { wg[r][s].a = wg[r][s].b = wu[r][s].a = wu[r][s].b = make_float4(0, 0, 0, 0); }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    float pa = 0.f, pu = 0.f;
#pragma unroll
    for (int s = 0; s < CPL; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pa = fmaf(wg[r][s].get(i), xv[s][i], pa);
        pu = fmaf(wu[r][s].get(i), xv[s][i], pu);
      }
    const float av = wave_sum(pa), uv = wave_sum(pu);
    const int i = i0 + r;
    if (lane == 0 && i < a.I) a.h[size_t(j) * a.I + i] = valid ? silu_f(av) * uv : NAN;
  }
}

// ------------------------------------------------------------ down + combine

template <int WD>
__global__ __launch_bounds__(256) void down_combine_kernel(DecodeArgs a) {
  extern __shared__ float sh[];          // [k][hpad(I)] then hsum [k][I/32]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane & 7, grp = lane >> 3;
  const int I = a.I, k = a.k;
  const int ipad = hpad(I);
  const int nblk = I >> 5;
  float* hs = sh + k * ipad;
  __shared__ int s_bad;
  if (threadIdx.x == 0) {
    int bad = 0;
    for (int j = 0; j < k; ++j) {
      const int e = a.idx[j];
      if (e < 0 || e >= a.E) bad |= kDevBadIndex;
      for (int jj = 0; jj < j; ++jj)
        if (a.idx[jj] == e) bad |= kDevDupIndex;
    }
    s_bad = bad;
    if (bad && blockIdx.x == 0) atomicOr(a.dev_flag, bad);
  }
  for (int q = threadIdx.x; q < k * I; q += blockDim.x) {
    const int j = q / I, i = q - j * I;
    sh[j * ipad + hpad(i)] = a.h[q];
  }
  __syncthreads();
  for (int q = threadIdx.x; q < k * nblk; q += blockDim.x) {
    const int j = q / nblk, b = q - j * nblk;
    float s = 0.f;
    for (int i = 0; i < 32; ++i) s += sh[j * ipad + hpad(b * 32 + i)];
    hs[q] = s;
  }
  __syncthreads();

  const int o = (blockIdx.x * 4 + wave) * 8 + grp;
  float acc = 0.f;
  if (o < a.H && !s_bad) {
    for (int j = 0; j < k; ++j) {
      const int e = a.idx[j];
      const float gj = a.gates[j];
      const size_t row = size_t(e) * a.H + o;
      const float* hj = sh + j * ipad;
      float p = 0.f;
      if constexpr (WD == MOE_Q4B32) {
        for (int b = g; b < nblk; b += 8) {
          const uint4 w = *reinterpret_cast<const uint4*>(
              reinterpret_cast<const uint8_t*>(a.wd) + row * (I / 2) + b * 16);
          const float d = f16_to_f32(a.sd[row * nblk + b]);
          float hv[32];
#pragma unroll
          for (int i = 0; i < 32; ++i) hv[i] = hj[hpad(b * 32) + i];
          p = fmaf(d, q4_block_dot(w, hv) - 8.f * hs[j * nblk + b], p);
        }
      } else {
        for (int c = g; c < (I >> 3); c += 8) {
          Chunk<WD> w;
          w.load(a.wd, row * I + c * 8);
          const float* hv = hj + hpad(c * 8);
#pragma unroll
          for (int i = 0; i < 8; ++i) p = fmaf(w.get(i), hv[i], p);
        }
      }
      acc = fmaf(gj, p, acc);
    }
  }
  acc = group_sum(acc, 8);
  if (g == 0 && o < a.H) a.out[o] = s_bad ? NAN : acc;
}

hipError_t launch_decode_experts(const Layer& L, const void* x, const int32_t* idx,
                                 const float* gates, float* out, float* h, hipStream_t s) {
  DecodeArgs a;
  a.x = x;
  a.idx = idx;
  a.gates = gates;
  a.wg = L.d.w_gate;
  a.wu = L.d.w_up;
  a.wd = L.d.w_down;
  a.sg = L.d.s_gate;
  a.su = L.d.s_up;
  a.sd = L.d.s_down;
  a.h = h;
  a.out = out;
  a.H = L.d.hidden;
  a.I = L.d.inter;
  a.E = L.d.n_experts;
  a.k = L.d.top_k;
  a.dev_flag = L.dev_flag;
  const int act = L.d.act_dtype, wd = L.d.expert_dtype;
  dim3 g1((a.I + 7) / 8, a.k);
  if (wd == MOE_Q4B32) {
    const int mb = (a.H / 32 + 63) / 64;
#define MOE_GU_Q4(M)                                                                    \
  if (mb <= M) {                                                                        \
    if (act == MOE_BF16)                                                                \
      hipLaunchKernelGGL((gateup_q4_kernel<MOE_BF16, M>), g1, dim3(256), 0, s, a);      \
    else                                                                                \
      hipLaunchKernelGGL((gateup_q4_kernel<MOE_F32, M>), g1, dim3(256), 0, s, a);       \
  } else
    MOE_GU_Q4(1) MOE_GU_Q4(2) MOE_GU_Q4(4) return hipErrorInvalidValue;
#undef MOE_GU_Q4
  } else {
    const int cpl = (a.H / 8 + 63) / 64;
#define MOE_GU_D(C)                                                                          \
  if (cpl <= C) {                                                                            \
    if (act == MOE_BF16 && wd == MOE_BF16)                                                   \
      hipLaunchKernelGGL((gateup_dense_kernel<MOE_BF16, MOE_BF16, C>), g1, dim3(256), 0, s, a); \
    else if (act == MOE_F32 && wd == MOE_BF16)                                               \
      hipLaunchKernelGGL((gateup_dense_kernel<MOE_F32, MOE_BF16, C>), g1, dim3(256), 0, s, a);  \
    else                                                                                     \
      hipLaunchKernelGGL((gateup_dense_kernel<MOE_F32, MOE_F32, C>), g1, dim3(256), 0, s, a);   \
  } else
    MOE_GU_D(1) MOE_GU_D(2) MOE_GU_D(4) MOE_GU_D(8) MOE_GU_D(16) return hipErrorInvalidValue;
#undef MOE_GU_D
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t lds = sizeof(float) * (size_t(a.k) * hpad(a.I) + size_t(a.k) * (a.I / 32 + 1));
  dim3 g2((a.H + 31) / 32);
  if (wd == MOE_Q4B32)
    hipLaunchKernelGGL(down_combine_kernel<MOE_Q4B32>, g2, dim3(256), lds, s, a);
  else if (wd == MOE_BF16)
    hipLaunchKernelGGL(down_combine_kernel<MOE_BF16>, g2, dim3(256), lds, s, a);
  else
    hipLaunchKernelGGL(down_combine_kernel<MOE_F32>, g2, dim3(256), lds, s, a);
  return hipGetLastError();
}

}  // namespace moe
