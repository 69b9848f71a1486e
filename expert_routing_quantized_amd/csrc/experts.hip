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
    Chunk<ACT> ch[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) ch[c].load(a.x, min(b, nblk - 1) * 32 + c * 8);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[m][c * 8 + i] = (b < nblk) ? ch[c].get(i) : 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) xs[m] += xv[m][i];
  }
  constexpr int kRowsPerWave = 2;
  const int i0 = (blockIdx.x * 4 + wave) * kRowsPerWave;
  const size_t rowb = size_t(a.H) / 2;
  uint4 wg[kRowsPerWave][MB], wu[kRowsPerWave][MB];
  float dg[kRowsPerWave][MB], du[kRowsPerWave][MB];
  // clamped indices: every load issues unconditionally; out-of-range lanes
  // get scale 0 below (their codes are then irrelevant)
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const int i = min(i0 + r, a.I - 1);
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int b = min(m * 64 + lane, nblk - 1);
      const size_t row = size_t(valid ? e : 0) * a.I + i;
      wg[r][m] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.wg) + row * rowb + b * 16);
      wu[r][m] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.wu) + row * rowb + b * 16);
      dg[r][m] = f16_to_f32(a.sg[row * nblk + b]);
      du[r][m] = f16_to_f32(a.su[row * nblk + b]);
    }
  }
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
    for (int m = 0; m < MB; ++m)
      if (!(i0 + r < a.I && m * 64 + lane < nblk)) dg[r][m] = du[r][m] = 0.f;
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
  {
    Chunk<ACT> ch[CPL];
#pragma unroll
    for (int s = 0; s < CPL; ++s) ch[s].load(a.x, min(s * 64 + lane, nch - 1) * 8);
#pragma unroll
    for (int s = 0; s < CPL; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[s][i] = (s * 64 + lane < nch) ? ch[s].get(i) : 0.f;
  }
  constexpr int kRowsPerWave = 2;
  const int i0 = (blockIdx.x * 4 + wave) * kRowsPerWave;
  Chunk<WD> wg[kRowsPerWave][CPL], wu[kRowsPerWave][CPL];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const size_t row = size_t(valid ? e : 0) * a.I + min(i0 + r, a.I - 1);
#pragma unroll
    for (int s = 0; s < CPL; ++s) {
      const int c = min(s * 64 + lane, nch - 1);
      wg[r][s].load(a.wg, row * a.H + c * 8);
      wu[r][s].load(a.wu, row * a.H + c * 8);
    }
  }
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
    for (int s = 0; s < CPL; ++s)
      if (!(i0 + r < a.I && s * 64 + lane < nch)) {
        wg[r][s].zero();
        wu[r][s].zero();
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

// One block per 8 output rows; wave w of the block handles the selected
// experts j = w, w + W, ... (W = min(k, 16) waves), 8 lanes per output row,
// lane g of a row covering quant blocks (or 8-element chunks) g, g + 8, ...
// of I.  The expert's h slice comes straight from L2 into registers, so the
// weights, the scales and h are all in flight together.  Each wave's
// g_j-weighted partials go through LDS and are summed over the waves in a
// fixed order (deterministic, no float atomics).
template <int WD>
__global__ __launch_bounds__(1024) void down_combine_kernel(DecodeArgs a) {
  __shared__ float part[kMaxK][8];
  __shared__ int s_bad;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int g = lane & 7, grp = lane >> 3;
  const int I = a.I, k = a.k;
  const int o = blockIdx.x * 8 + grp;
  const int oc = min(o, a.H - 1);
  constexpr int kElems = (WD == MOE_Q4B32) ? 32 : 8;
  const int nsl = I / kElems;
  const int nblk = I >> 5;
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  if (threadIdx.x < k) {        // one thread per selected expert checks its index
    const int j = threadIdx.x, e = a.idx[j];
    int bad = (e < 0 || e >= a.E) ? kDevBadIndex : 0;
    for (int jj = 0; jj < j; ++jj)
      if (a.idx[jj] == e) bad |= kDevDupIndex;
    if (bad) {
      atomicOr(&s_bad, bad);
      if (blockIdx.x == 0) atomicOr(a.dev_flag, bad);
    }
  }

  float acc = 0.f;
  for (int j = wave; j < k; j += nw) {
    int e = a.idx[j];
    e = (e >= 0 && e < a.E) ? e : 0;                   // addresses stay in range
    const float gj = a.gates[j];
    const size_t row = size_t(e) * a.H + oc;
    const float* hj = a.h + size_t(j) * I;
    for (int sl = g; sl < nsl; sl += 8) {
      float hv[kElems];
#pragma unroll
      for (int i = 0; i < kElems; i += 4) {
        const float4 v4 = *reinterpret_cast<const float4*>(hj + sl * kElems + i);
        hv[i] = v4.x; hv[i + 1] = v4.y; hv[i + 2] = v4.z; hv[i + 3] = v4.w;
      }
      if constexpr (WD == MOE_Q4B32) {
        const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.wd) + row * (I / 2) + sl * 16);
        const float d = f16_to_f32(a.sd[row * nblk + sl]);
        float hs = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) hs += hv[i];
        acc = fmaf(gj, d * (q4_block_dot(w, hv) - 8.f * hs), acc);
      } else {
        Chunk<WD> w;
        w.load(a.wd, row * I + sl * 8);
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) p = fmaf(w.get(i), hv[i], p);
        acc = fmaf(gj, p, acc);
      }
    }
  }
  acc = group8_sum(acc);
  if (g == 0) part[wave][grp] = acc;
  __syncthreads();
  if (threadIdx.x < 8 && blockIdx.x * 8 + (int)threadIdx.x < a.H) {
    float s = 0.f;
    for (int w = 0; w < nw; ++w) s += part[w][threadIdx.x];
    a.out[blockIdx.x * 8 + threadIdx.x] = s_bad ? NAN : s;
  }
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
  const int nw = a.k < 16 ? a.k : 16;
  dim3 g2((a.H + 7) / 8);
  if (wd == MOE_Q4B32)
    hipLaunchKernelGGL(down_combine_kernel<MOE_Q4B32>, g2, dim3(64 * nw), 0, s, a);
  else if (wd == MOE_BF16)
    hipLaunchKernelGGL(down_combine_kernel<MOE_BF16>, g2, dim3(64 * nw), 0, s, a);
  else
    hipLaunchKernelGGL(down_combine_kernel<MOE_F32>, g2, dim3(64 * nw), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
