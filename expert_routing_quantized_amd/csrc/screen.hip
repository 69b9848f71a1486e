// The router's int8 first pass for one token (batch-1 decode).
//
// The pages' routing kernel scores every expert of the 24,576 for each token
// (pyshine source tour, Understanding the Architecture, paragraph on the
// residency tiers and the routing kernel), and at batch 1 that pass is a
// GEMV whose speed is set by the bytes it streams (hexlives dispatch,
// paragraph on the archived tensor-core benchmark).  The screen streams an
// int8 copy of the router -- half of the bf16 router's bytes -- and bounds
// how far each of its values can be from the exact logit, so that the
// selection (select_screen.h) recomputes only the few experts the bound
// cannot rule out.
//
// Layer preparation (once, at layer creation), one wave per expert row:
//   s_e = fl32(max_h |R_eh| / 127),  q_eh = clamp(rint(R_eh / s_e), -127, 127)
//   (0 for an all-zero row), and the 2-norms of the residual eps_e = R_e - s_e q_e
//   and of s_e q_e, both evaluated exactly in binary64 and rounded up.
//
// Per token: x is written in a 15-bit fixed point common to the token,
//   x_h = 2^-m (128 hi_h + lo_h) + delta_h,   hi_h in [-64, 64], lo_h in [0, 127],
// with m chosen from max_h |x_h| (|x_h 2^m| < 2^13) and rint rounding, so
// |delta_h| <= 2^-(m+1).  Then
//   v_e = fl32( s_e 2^-m (128 HI_e + LO_e) + b_e ),  HI_e = sum_h q_eh hi_h,  LO_e = sum_h q_eh lo_h,
// where HI and LO are exact int32 sums of v_dot4_i32_i8 products (4 int8
// products per instruction), and
//   z_e - (s_e 2^-m (128 HI_e + LO_e) + b_e) = sum_h eps_eh x_h + sum_h s_e q_eh delta_h,
// bounded by ||eps_e|| ||x|| + ||s_e q_e|| ||delta|| (Cauchy-Schwarz).  The
// kernel also writes ||x||^2 and ||delta||^2 (binary64 sums of exact squares,
// block 0) and the maximum of every 4 consecutive values (the selection's
// group maxima).
//
// Layout: the int8 router is expert-major [E][H]; one wave owns RPW rows, lane
// l takes 16-byte chunks l, l + 64, ... of each row (1 KB per wave load, all
// of a row's loads issued before any arithmetic, non-temporal: streamed once
// per token).  Each block recomputes the token's digit planes in LDS (x is
// 4 KB, read from L2) while its row loads are in flight.
#include "select_screen.h"

namespace moe {

constexpr int kScreenWaves = 4;

// ------------------------------------------------------------------ prep
// One wave per expert; consts[0] = max ||eps_e||, consts[1] = max ||s_e q_e||,
// consts[2] = max |b_e| (bit-pattern maxima of non-negative floats).
__global__ __launch_bounds__(256) void screen_prep_kernel(const uint16_t* __restrict__ R, const float* __restrict__ bias,
                                                          int H, int E, int8_t* __restrict__ q8,
                                                          float* __restrict__ sc8, float2* __restrict__ eb8,
                                                          float* __restrict__ consts) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;                                  // wave-uniform
  const int nch = H / 8;
  const uint16_t* row = R + size_t(e) * H;
  float amax = 0.f;
  for (int c = lane; c < nch; c += 64) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + c * 8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[j])), fabsf(bf16_hi(w[j]))));
  }
  amax = wave_max(amax);
  const float s = amax / 127.0f;
  const double sd = (double)s;
  double en2 = 0.0, rq2 = 0.0;
  for (int c = lane; c < nch; c += 64) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + c * 8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double r = (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]);
      double q = (s > 0.f) ? rint(r / sd) : 0.0;
      q = fmin(127.0, fmax(-127.0, q));
      const double rq = sd * q;                      // exact: 24-bit scale times a 7-bit integer
      const double eps = r - rq;                     // exact in binary64 (see the header)
      en2 = fma(eps, eps, en2);
      rq2 = fma(rq, rq, rq2);
      packed[i >> 2] |= (uint32_t(int(q)) & 0xffu) << (8 * (i & 3));
    }
    *reinterpret_cast<uint2*>(q8 + size_t(e) * H + c * 8) = make_uint2(packed[0], packed[1]);
  }
  en2 = wave_sum_d(en2) * (1.0 + 1e-12);
  rq2 = wave_sum_d(rq2) * (1.0 + 1e-12);
  if (lane == 0) {
    const float en = nextafterf((float)sqrt(en2), INFINITY);
    const float rq = nextafterf((float)sqrt(rq2), INFINITY);
    sc8[e] = s;
    eb8[e] = make_float2(en, rq);
    atomicMax(reinterpret_cast<unsigned int*>(consts + 0), __float_as_uint(en));
    atomicMax(reinterpret_cast<unsigned int*>(consts + 1), __float_as_uint(rq));
    const float ab = fabsf(bias[e]);
    if (ab == ab) atomicMax(reinterpret_cast<unsigned int*>(consts + 2), __float_as_uint(ab));
  }
}

__global__ void zero3_kernel(float* p) {
  if (threadIdx.x < 3) p[threadIdx.x] = 0.f;
}

hipError_t launch_screen_prep(const Layer& L, float* consts, hipStream_t s) {
  const int H = L.d.hidden, E = L.d.n_experts;
  hipLaunchKernelGGL(zero3_kernel, dim3(1), dim3(64), 0, s, consts);
  hipLaunchKernelGGL(screen_prep_kernel, dim3((E + 3) / 4), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t*>(L.router_eh), router_bias_or_zero(L), H, E, L.q8,
                     L.sc8, L.eb8, consts);
  return hipGetLastError();
}

// ------------------------------------------------------------------ screen
// Integer sum over the 64 lanes (every lane gets it).
__device__ __forceinline__ int wave_sum_i32(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);
  return __builtin_amdgcn_readlane(v, 63);
}

// Unsigned maximum over the 64 lanes (every lane gets it).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

struct ScreenArgs {
  const int8_t* q8;       // [E][H]
  const float* sc8;       // [E]
  const float* bias;      // [E], never null
  const uint16_t* x;      // [T][H] bf16
  int H, E, T;
  float* z8;              // [T][E]
  float* g8;              // [T][ceil(E/4)]
  double* xq;             // [T][2]: ||x||^2, ||delta||^2
  int* dev_flag;
  // the list (batch 1; hint null: none)
  const uint16_t* R;      // [E][H] bf16 router
  const float2* eb8;      // [E] residual norms, rounded up
  double u8, babs8;       // the bound's relative and absolute terms
  double rqmax;           // max_e ||s_e q_e|| (rounded up)
  const HintWords* hint;  // the call's hint, null: no list
  const HintWords* hsrc;  // never null: hint, or a readable stand-in (read unconditionally)
  unsigned int* lcount;   // the list's counter (in the hint)
  unsigned char* cnt8;    // [waves]
  ulonglong2* list;       // [kListSlots]: (e, logit bits)
};

// One wave owns RPW consecutive rows (RPW a multiple of 4: whole groups of 4
// experts), WPB waves per block; CH = 16-byte chunks per lane of an int8 row
// (H <= 1024 CH).  Every wave works alone -- no LDS, no barrier: lane l
// loads the hidden-state elements of its own row chunks l, l + 64, ...
// (together the wave holds all of x), takes the maximum with a DPP
// reduction, and writes those elements' digits straight into registers.
template <int NB, int WPB, int CH, int RB = 2, int NBUF = 2>
__global__ __launch_bounds__(WPB * 64) void screen_kernel(ScreenArgs a) {
  constexpr int RPW = RB * NB;                       // rows per wave
  static_assert((WPB * RPW) % 4 == 0, "a block holds whole groups of 4 experts");
  __shared__ float s_v[WPB * RPW];                   // the block's values (NaN, past E: -inf)
  __shared__ float s_vf[WPB * RPW], s_eb[WPB * RPW];  // values and ||eps_e|| (for the list)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, E = a.E, t = blockIdx.y;
  const int e0 = (blockIdx.x * WPB + wave) * RPW;
  // (waves past E compute clamped rows and discard them: every wave reaches the barrier)
  const int nch = H >> 4;                            // 16-byte chunks of an int8 row
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  // 1. the lane's x first (loads complete in order, so its digits are
  //    worked out while the rows stream), then the rows, their scales and biases
  uint4 xr[CH][2];                                   // bf16 x of chunk s: elements 16 c .. 16 c + 15
#pragma unroll
  for (int s = 0; s < CH; ++s) {
    const int c = min(s * 64 + lane, nch - 1);
    const uint4* xp = reinterpret_cast<const uint4*>(a.x + size_t(t) * H) + 2 * c;
    xr[s][0] = xp[0];
    xr[s][1] = xp[1];
  }
  // the hint (read whether or not it is used: a load under a branch would
  // wait for every load before it)
  const float ring_v = a.hsrc->ring[lane & (kHintRing - 1)];
  // rows in batches of RB, NBUF batches in flight: batch b + NBUF is issued
  // into the buffer batch b frees (registers for NBUF RB rows whatever NB
  // is, so one wave per row group of RPW rows stays resident; issuing every
  // batch up front measured slower)
  u32x4 r[NBUF][RB][CH];
  auto issue = [&](int bt, int buf) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int e = min(e0 + bt * RB + i, E - 1);
#pragma unroll
      for (int s = 0; s < CH; ++s)
        r[buf][i][s] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(a.q8 + size_t(e) * H) + min(s * 64 + lane, nch - 1));
    }
  };
#pragma unroll
  for (int bt = 0; bt < NBUF; ++bt) issue(bt, bt);
  // scale, bias and ||eps_e|| (the list's bound) of the wave's rows: lane l
  // holds row e0 + l's (the rows' values are evaluated together at the end)
  static_assert(RPW <= 64, "one lane per row of the wave");
  const int el = min(e0 + min(lane, RPW - 1), E - 1);
  const float my_sc = a.sc8[el], my_b = a.bias[el], my_eb = a.eb8[el].x;
  const bool listing = a.hint != nullptr && t == 0;  // uniform
  // 2. max |x| over the wave (= all of x) on the magnitude bits: a non-finite
  //    element has magnitude bits >= 0x7f80
  uint32_t mb = 0u;
#pragma unroll
  for (int s = 0; s < CH; ++s) {
    if (s * 64 + lane >= nch) continue;
    const uint32_t w[8] = {xr[s][0].x, xr[s][0].y, xr[s][0].z, xr[s][0].w,
                           xr[s][1].x, xr[s][1].y, xr[s][1].z, xr[s][1].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) mb = max(mb, max(w[j] & 0x7fffu, (w[j] >> 16) & 0x7fffu));
  }
  mb = wave_max_u32(mb);
  const bool xbad = mb >= 0x7f80u;
  const float mx = __uint_as_float(mb << 16);
  int m = 0;
  if (mx > 0.f && !xbad) {
    int ex;
    frexpf(mx, &ex);                                 // mx = f 2^ex, f in [0.5, 1)
    m = 13 - ex;                                     // |x 2^m| < 2^13
  }
  // x 2^m in binary32, exact: two power-of-two factors, neither over- nor underflowing
  const int m1 = m > 100 ? 100 : (m < -100 ? -100 : m);
  const float sc1 = ldexpf(1.f, m1), sc2 = ldexpf(1.f, m - m1);
  // 3. block 0's first wave sums ||x||^2 and ||delta||^2 exactly in
  //    binary64; then the digits of the lane's chunks (zero past the row, so
  //    the clamped row loads add nothing)
  const double isc = ldexp(1.0, -m);
  if (blockIdx.x == 0 && wave == 0) {                // wave-uniform
    double sx2 = 0.0, sd2 = 0.0;
#pragma unroll
    for (int s = 0; s < CH; ++s) {
      if (s * 64 + lane >= nch) continue;
      const uint32_t w[8] = {xr[s][0].x, xr[s][0].y, xr[s][0].z, xr[s][0].w,
                             xr[s][1].x, xr[s][1].y, xr[s][1].z, xr[s][1].w};
#pragma unroll
      for (int el = 0; el < 16; ++el) {
        const float v = (el & 1) ? bf16_hi(w[el >> 1]) : bf16_lo(w[el >> 1]);
        const double d = (double)v - (double)rintf((v * sc1) * sc2) * isc;   // exact
        sx2 = fma((double)v, (double)v, sx2);
        sd2 = fma(d, d, sd2);
      }
    }
    sx2 = wave_sum_f64(sx2);
    sd2 = wave_sum_f64(sd2);
    if (lane == 0) {
      a.xq[2 * t] = xbad ? NAN : sx2;
      a.xq[2 * t + 1] = xbad ? NAN : sd2;
      if (xbad) atomicOr(a.dev_flag, kDevNonFinite);
    }
  }
  int dh[CH][4], dl[CH][4];
#pragma unroll
  for (int s = 0; s < CH; ++s) {
    const bool in = s * 64 + lane < nch;
    const uint32_t w[8] = {xr[s][0].x, xr[s][0].y, xr[s][0].z, xr[s][0].w,
                           xr[s][1].x, xr[s][1].y, xr[s][1].z, xr[s][1].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t hw = 0u, lw = 0u;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int el = 4 * q + b;                    // element of the chunk
        const uint32_t word = w[el >> 1];
        const float v = (el & 1) ? bf16_hi(word) : bf16_lo(word);
        const int Xi = (int)rintf((v * sc1) * sc2);  // |Xi| <= 2^13
        hw |= (uint32_t(Xi >> 7) & 0xffu) << (8 * b);          // floor(Xi / 128), in [-64, 64]
        lw |= uint32_t(Xi & 127) << (8 * b);                   // in [0, 127]
      }
      dh[s][q] = (in && !xbad) ? (int)hw : 0;
      dl[s][q] = (in && !xbad) ? (int)lw : 0;
    }
  }
  // the list's theta and upper bounds on ||x|| and ||delta||, worked out
  // while the rows stream.  With X the digits' integers (x 2^m = X + d,
  // |d_h| <= 1/2): ||x|| 2^m <= ||X|| + sqrt(H) / 2 and ||delta|| 2^m <=
  // sqrt(H) / 2, where ||X||^2 = 2^14 sum hi^2 + 2^8 sum hi lo + sum lo^2
  // (three exact integer dot products of the digits).  Binary32 with a
  // (1 + 2^-20) margin per result: a handful of roundings each.
  // (wave 0 of each block only: the block's list decisions are its job)
  float theta = INFINITY, xnu = 0.f, dnu = 0.f;
  if (listing && wave == 0) {
    theta = xbad ? INFINITY : hint_threshold_lanes(ring_v);
    int shh = 0, shl = 0, sll = 0;
#pragma unroll
    for (int s = 0; s < CH; ++s)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        shh = __builtin_amdgcn_sdot4(dh[s][q], dh[s][q], shh, false);
        shl = __builtin_amdgcn_sdot4(dh[s][q], dl[s][q], shl, false);
        sll = __builtin_amdgcn_sdot4(dl[s][q], dl[s][q], sll, false);
      }
    shh = wave_sum_i32(shh);
    shl = wave_sum_i32(shl);
    sll = wave_sum_i32(sll);
    // exact in 64-bit integers (the middle term can be negative), one rounding to binary32
    const long long X2i = 16384ll * shh + 256ll * shl + (long long)sll;
    const float X2 = (float)X2i * (1.f + 0x1p-20f);
    const float iscf = ldexpf(1.f, -m);              // 2^-m (m <= 150: normal or subnormal, exact)
    const float hd = 0.5f * sqrtf((float)H) * (1.f + 0x1p-20f);
    xnu = ((sqrtf(X2) * (1.f + 0x1p-20f) + hd) * (1.f + 0x1p-20f)) * iscf * (1.f + 0x1p-20f) + 0x1p-149f;
    dnu = hd * iscf * (1.f + 0x1p-20f) + 0x1p-149f;
  }

  // 4. exact integer dot products per row (lane ri keeps row ri's sums),
  //    then one binary64 evaluation of every row of the wave at once, the
  //    values (and, for the list, whether v + B reaches theta)
  int dacc = 0, hacc = 0, lacc = 0;
#pragma unroll
  for (int bt = 0; bt < NB; ++bt) {
    const int buf = bt % NBUF;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      int HI = 0, LO = 0;
#pragma unroll
      for (int s = 0; s < CH; ++s) {
        const unsigned w[4] = {r[buf][i][s].x, r[buf][i][s].y, r[buf][i][s].z, r[buf][i][s].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          HI = __builtin_amdgcn_sdot4((int)w[q], dh[s][q], HI, false);
          LO = __builtin_amdgcn_sdot4((int)w[q], dl[s][q], LO, false);
        }
      }
      const int ri = bt * RB + i;
      if constexpr (CH <= 2) {
        // H <= 2048: sum_h |q_eh X_h| <= 2048 * 127 * 2^13 < 2^31, so 128 HI + LO
        // and every partial sum of it are exact in int32: one wave sum
        const int D = wave_sum_i32(128 * HI + LO);
        dacc = (lane == ri) ? D : dacc;
      } else {
        const int HS = wave_sum_i32(HI), LS = wave_sum_i32(LO);
        hacc = (lane == ri) ? HS : hacc;
        lacc = (lane == ri) ? LS : lacc;
      }
    }
    if (bt + NBUF < NB) {
      __builtin_amdgcn_sched_barrier(0);             // keep the next loads after this batch (registers)
      issue(bt + NBUF, buf);
    }
  }
  {
    const int ri = lane, e = e0 + ri;
    const double D = (CH <= 2) ? (double)dacc : 128.0 * (double)hacc + (double)lacc;   // exact
    const double v = (double)my_sc * D * isc + (double)my_b;
    const float vf = xbad ? NAN : (float)v;
    if (ri < RPW) {
      s_v[wave * RPW + ri] = (e < E && !isnan(vf)) ? vf : -INFINITY;
      s_vf[wave * RPW + ri] = (e < E) ? vf : NAN;
      s_eb[wave * RPW + ri] = my_eb;
      if (e < E) a.z8[size_t(t) * E + e] = vf;
    }
    if (__ballot(ri < RPW && e < E && !xbad && !isfinite(vf)) != 0ull && lane == 0) atomicOr(a.dev_flag, kDevNonFinite);
  }
  // the maxima of every 4 consecutive experts of the block (NaN: -inf)
  __syncthreads();
  {
    const int G = (E + 3) / 4;
    const int g = blockIdx.x * (WPB * RPW / 4) + tid;
    if (tid < WPB * RPW / 4 && g < G)
      a.g8[size_t(t) * G + g] = fmaxf(fmaxf(s_v[4 * tid], s_v[4 * tid + 1]), fmaxf(s_v[4 * tid + 2], s_v[4 * tid + 3]));
  }
  // the list, by wave 0 of the block: lane l decides for the block's row l
  // whether its upper end v + B reaches theta (binary32, rounded up: every
  // term of B is positive, so (1 + 2^-20) covers its few roundings and
  // 2^-147 those in the subnormal range; the 2^-22 |U| + 2^-149 slack covers
  // the rounding of U and of the slack's own sum), then recomputes the
  // listed rows' logits from the bf16 rows as the selection would
  // (8-element chunks, dot2 chains) and appends them: one atomic add takes
  // the block's slots, in flight while the rows load
  if (!listing || wave != 0) return;
  constexpr int BR = WPB * RPW;                      // rows of the block (<= 64)
  static_assert(BR <= 64, "one lane per row of the block");
  const int eb0 = blockIdx.x * BR;
  unsigned long long listed = 0ull;
  {
    const float rqmax = (float)a.rqmax * (1.f + 0x1p-20f), u8f = (float)a.u8 * (1.f + 0x1p-20f);
    const float babs8f = (float)a.babs8 * (1.f + 0x1p-20f) + 0x1p-149f;
    const float vf = (lane < BR) ? s_vf[lane] : NAN;    // NaN past E
    const float eb = (lane < BR) ? s_eb[lane] : 0.f;
    const float B = fmaf(xnu, eb, fmaf(dnu, rqmax, fmaf(u8f, fabsf(vf), babs8f))) * (1.f + 0x1p-20f) + 0x1p-147f;
    const float U = vf + B;
    listed = __ballot(lane < BR && isfinite(vf) && U + fabsf(U) * 0x1p-22f + 0x1p-149f >= theta);
  }
  if (listed != 0ull) {
    constexpr int CPLR = 2 * CH;
    const int n8 = H >> 3;
    unsigned slot = 0u;
    if (lane == 0) slot = atomicAdd(a.lcount, (unsigned)__popcll(listed));
    uint4 xc[CPLR];
#pragma unroll
    for (int s = 0; s < CPLR; ++s)
      xc[s] = *reinterpret_cast<const uint4*>(a.x + size_t(t) * H + min(s * 64 + lane, n8 - 1) * 8);
    for (unsigned long long m = listed; m != 0ull; m &= m - 1ull) {   // one row at a time (registers)
      const int e = eb0 + __builtin_ctzll(m);
      uint4 rr[CPLR];
#pragma unroll
      for (int s = 0; s < CPLR; ++s)
        rr[s] = *reinterpret_cast<const uint4*>(a.R + size_t(e) * H + min(s * 64 + lane, n8 - 1) * 8);
      const double z = dot2_logit<CPLR>(xc, rr, n8, a.bias[e], lane);
      if (lane == 0 && slot < (unsigned)kListSlots)    // a full list: the selection falls back
        a.list[slot] = make_ulonglong2((unsigned long long)e, (unsigned long long)__double_as_longlong(z));
      ++slot;
    }
  }
  if (lane == 0) a.cnt8[blockIdx.x] = (unsigned char)__popcll(listed);
}

// Launch shape of the screen: 6 rows per wave, one row per batch, two
// batches in flight, 4 waves per block (1024 blocks at E = 24,576, all
// resident at once).  Measured in a sweep of shapes (screen alone, graph of
// launches over six router copies): 10.8-11.0 us per launch against 11.7
// for two-row batches and 12.1 with every batch issued up front; one batch
// in flight 13.5, 4 or 8 rows per wave 11.6-11.8.
constexpr int kScreenBatches = 6;
constexpr int kScreenRowsPerBatch = 1;
constexpr int kScreenBuffers = 2;
constexpr int kScreenRowsPerWave = kScreenRowsPerBatch * kScreenBatches;
constexpr int kScreenWavesPerBlock = 4;

static int screen_blocks(int E) {
  return (E + kScreenWavesPerBlock * kScreenRowsPerWave - 1) / (kScreenWavesPerBlock * kScreenRowsPerWave);
}

template <int CH>
static hipError_t launch_screen_shape(const ScreenArgs& sa, hipStream_t s) {
  hipLaunchKernelGGL((screen_kernel<kScreenBatches, kScreenWavesPerBlock, CH, kScreenRowsPerBatch, kScreenBuffers>),
                     dim3(screen_blocks(sa.E), sa.T),
                     dim3(kScreenWavesPerBlock * 64), 0, s, sa);
  return hipGetLastError();
}

hipError_t launch_screen(const Layer& L, const void* x, int T, float* z8, float* g8, double* xq,
                         const ScreenList* list, hipStream_t s) {
  ScreenArgs a{};
  a.q8 = L.q8;
  a.sc8 = L.sc8;
  a.bias = router_bias_or_zero(L);
  a.x = reinterpret_cast<const uint16_t*>(x);
  a.H = L.d.hidden;
  a.E = L.d.n_experts;
  a.T = T;
  a.z8 = z8;
  a.g8 = g8;
  a.xq = xq;
  a.dev_flag = L.dev_flag;
  a.eb8 = L.eb8;
  a.hsrc = reinterpret_cast<const HintWords*>(L.screen_consts);   // 256 bytes, read and ignored
  if (list != nullptr && T == 1) {
    a.R = reinterpret_cast<const uint16_t*>(L.router_eh);
    const ScreenSelectArgs b = make_screen_select_args(L, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
    a.u8 = b.u8;
    a.babs8 = b.babs8;
    a.rqmax = b.rqmax;
    a.hint = list->hint;
    a.hsrc = list->hint;
    a.lcount = &list->hint->list_count;
    a.cnt8 = list->cnt8;
    a.list = list->list;
  }
  const int ch = (a.H / 16 + 63) / 64;
  if (ch <= 2) return launch_screen_shape<2>(a, s);
  if (ch <= 4) return launch_screen_shape<4>(a, s);
  if (ch <= 8) return launch_screen_shape<8>(a, s);
  return hipErrorInvalidValue;
}

// Blocks of the screen kernel (one count byte each in the list).
int screen_waves(const Layer& L) { return screen_blocks(L.d.n_experts); }

void set_screen_list(ScreenSelectArgs& b, const Layer& L, const ScreenList* list, bool advance) {
  b.hint = list->hint;
  b.cnt8 = list->cnt8;
  b.list = list->list;
  b.nw = screen_waves(L);
  b.advance = advance ? 1 : 0;
}

ScreenSelectArgs make_screen_select_args(const Layer& L, const void* x, const float* z8, const float* g8,
                                         const double* xq, int32_t* idx, float* gates) {
  ScreenSelectArgs b{};
  RouterBound rb = router_bound(L, 1);
  rb.d32 = 8;                     // the recomputed logits' chains of four v_dot2_f32_bf16
  b.sel = make_select_args(L, x, nullptr, false, nullptr, xq, idx, gates, rb);
  b.sel.bias = router_bias_or_zero(L);
  b.z8 = z8;
  b.g8 = g8;
  b.eb8 = L.eb8;
  b.enmax = L.screen_enmax;
  b.rqmax = L.screen_rqmax;
  // binary64 product and sum, then the binary32 store: (2^-24 + 2^-52) |v| (1 + 2^-23)
  // + 2^-53 max |b| (+ underflow of either format)
  b.u8 = 0x1p-23;
  b.babs8 = 0x1p-52 * L.screen_bmax + 0x1p-140;
  return b;
}

// Per-expert bound B_e of the screen values (the selection computes the same
// figure; this copy is for inspection and tests), rounded up to binary32.
__global__ __launch_bounds__(256) void screen_bound_kernel(const float* __restrict__ z8, const double* __restrict__ xq,
                                                           const float2* __restrict__ eb8, int E, int T, double u8,
                                                           double babs8, float* __restrict__ bound) {
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= size_t(T) * E) return;
  const int t = int(i / E), e = int(i - size_t(t) * E);
  const double xn = sqrt(xq[2 * t]) * (1.0 + 1e-3), dn = sqrt(xq[2 * t + 1]) * (1.0 + 1e-3);
  const float2 eb = eb8[e];
  const double B = xn * (double)eb.x + dn * (double)eb.y + u8 * fabs((double)z8[i]) + babs8;
  float bf = (float)B;
  if ((double)bf < B) bf = nextafterf(bf, INFINITY);
  bound[i] = bf;
}

hipError_t launch_screen_bounds(const Layer& L, int T, const float* z8, const double* xq, float* bound,
                                hipStream_t s) {
  const ScreenSelectArgs b = make_screen_select_args(L, nullptr, z8, nullptr, xq, nullptr, nullptr);
  const size_t n = size_t(T) * L.d.n_experts;
  hipLaunchKernelGGL(screen_bound_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, z8, xq, L.eb8,
                     L.d.n_experts, T, b.u8, b.babs8, bound);
  return hipGetLastError();
}

// ------------------------------------------------------------------ select
template <int ACT, int CPL>
__global__ __launch_bounds__(kSelectThreads) void select_screen_kernel(ScreenSelectArgs b) {
  const int t = blockIdx.x;
  select_screen_block<ACT, CPL>(b, t, b.sel.idx + size_t(t) * b.sel.k, b.sel.gates + size_t(t) * b.sel.k);
}

hipError_t launch_select_screen(const Layer& L, const void* x, int T, const float* z8, const float* g8,
                                const double* xq, const ScreenList* list, int32_t* idx, float* gates,
                                hipStream_t s) {
  if (list == nullptr || T != 1) return hipErrorInvalidValue;     // batch 1, with the list
  ScreenSelectArgs b = make_screen_select_args(L, x, z8, g8, xq, idx, gates);
  set_screen_list(b, L, list, true);   // this kernel ends the call
  const int cpl = (L.d.hidden / 8 + 63) / 64;
#define MOE_SEL_SCREEN(C)                                                                             \
  if (cpl <= C) {                                                                                     \
    hipLaunchKernelGGL((select_screen_kernel<MOE_BF16, C>), dim3(T), dim3(kSelectThreads), 0, s, b);  \
    return hipGetLastError();                                                                         \
  }
  MOE_SEL_SCREEN(1)
  MOE_SEL_SCREEN(2)
  MOE_SEL_SCREEN(4)
  MOE_SEL_SCREEN(8)
  MOE_SEL_SCREEN(16)
#undef MOE_SEL_SCREEN
  return hipErrorInvalidValue;
}

}  // namespace moe
