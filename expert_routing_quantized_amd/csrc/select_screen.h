// Exact top-k selection from the router's int8 first pass (batch-1 decode).
//
// The router pass that every decode token pays for reads the whole router;
// at E = 24,576 and H = 2048 that is 100.7 MB of bf16, 92 % of the token's
// bytes.  The screen (screen.hip) reads an int8 copy of the router instead
// (half the bytes) and gives, for every expert e, an approximate logit v_e
// with a rigorous bound
//   |v_e - z_e| <= B_e = ||x|| ||eps_e|| + ||delta|| ||Rq_e|| + u8 |v_e| + babs8,
// where eps_e = R_e - s_e q_e is the expert's quantisation residual, delta the
// hidden state's rounding to the screen's 15-bit fixed point and Rq_e = s_e q_e
// (Cauchy-Schwarz on the two residual products; the screen's integer dot
// products are exact, u8 and babs8 cover its final binary64 / binary32
// roundings).  With the synthetic weights B_e is about 0.28, so about 50
// experts per token cannot be ruled out; they are recomputed from the bf16
// router rows with the batch-1 router's arithmetic (chains of 8 binary32
// products, binary64 after that: the same logits that kernel produces, bound
// about 4e-5), and the certified selection of select_block.h finishes on
// those.  Nothing is approximate in the result: experts outside the
// recomputed set have exact logits strictly below the k-th largest.
//
// Steps (one block of kSelectThreads threads per token):
//  1. tau0 from the screen's maxima of 4 consecutive values (as in
//     select_block: a value k of 64 disjoint set maxima reach) and from it
//     L0, a lower bound on the k-th largest exact logit; groups that may hold
//     an expert with v + B >= L0 are listed;
//  2. their experts' values and per-expert bounds are loaded; tau = the k-th
//     largest lower end v - B_e (all experts with v - B_e >= L0 are listed);
//     the recompute set C is every expert with v + B_e >= tau;
//  3. C's logits are recomputed from the bf16 rows and select_tail certifies
//     the order (exact refinement where intervals overlap).
// More than kScreenMaxCand experts in C (ties of thousands of experts, or a
// screen bound too wide to separate anything) go to select_tail's scan over
// all E screen values with the exact refinement instead.
#pragma once

#include "select_block.h"

namespace moe {

constexpr int kScreenMaxCand = 256;   // experts recomputed from the bf16 rows at most

struct ScreenSelectArgs {
  SelectArgs sel;          // router rows, bias, x, idx/gates, the recomputed logits' bound;
                           // sel.xnorm -> [T][2]: ||x_t||^2, ||delta_t||^2
  const float* z8;         // [T][E] screen values v (binary32, nearest)
  const float* g8;         // [T][ceil(E/4)] their maxima over 4 consecutive experts
  const float2* eb8;       // [E]: (||eps_e|| rounded up, ||Rq_e|| rounded up)
  double enmax, rqmax;     // maxima of the two norms over the experts
  double u8, babs8;        // relative and absolute terms of the screen bound
};

typedef __bf16 sel_bf16x2_t __attribute__((ext_vector_type(2)));

// Logit of one router row recomputed from bf16 (one wave; every lane returns
// it): lane l takes 8-element chunks l, l + 64, ...; per chunk four
// v_dot2_f32_bf16 in a binary32 chain (exact products, at most two roundings
// per instruction: 8 binary32 roundings), then binary64 for the lane's chunks,
// the fixed DPP tree over the wave and the bias -- the error model of the
// several-token router kernel, d32 = 8, d64 = log2(CPL) + 7.
template <int CPL>
__device__ __forceinline__ double dot2_logit(const uint4 (&xc)[CPL], const uint4 (&r)[CPL], int nch, float b,
                                             int lane) {
  double acc[CPL];
#pragma unroll
  for (int s = 0; s < CPL; ++s) {
    const bool in = s * 64 + lane < nch;
    const uint32_t xw[4] = {xc[s].x, xc[s].y, xc[s].z, xc[s].w};
    const uint32_t rw[4] = {in ? r[s].x : 0u, in ? r[s].y : 0u, in ? r[s].z : 0u, in ? r[s].w : 0u};
    float c = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(sel_bf16x2_t, xw[q]),
                                          __builtin_bit_cast(sel_bf16x2_t, rw[q]), c, false);
    acc[s] = (double)c;
  }
#pragma unroll
  for (int w = 1; w < CPL; w <<= 1)
#pragma unroll
    for (int s = 0; s + w < CPL; s += 2 * w) acc[s] += acc[s + w];
  return wave_sum_f64(acc[0]) + (double)b;
}

// Recomputes the logits of the n experts S.c_id[0..n) into S.s_val / S.s_id:
// wave w takes experts w, w + 8, ..., up to kRecomputeRows rows in flight.
constexpr int kRecomputeRows = 8;
template <int CPL>
__device__ __forceinline__ void recompute_logits(const SelectArgs& a, int t, int n, SelectLds& S) {
  constexpr int RB = kRecomputeRows;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nch = a.H >> 3;
  const uint16_t* xb = reinterpret_cast<const uint16_t*>(a.x) + size_t(t) * a.H;
  for (int i0 = wave; i0 < n; i0 += RB * kWavesSel) {
    uint4 xc[CPL];
    uint4 r[RB][CPL];
    int ev[RB];
    float bv[RB];
#pragma unroll
    for (int s = 0; s < CPL; ++s) xc[s] = *reinterpret_cast<const uint4*>(xb + min(s * 64 + lane, nch - 1) * 8);
#pragma unroll
    for (int u = 0; u < RB; ++u) ev[u] = S.c_id[min(i0 + u * kWavesSel, n - 1)];
#pragma unroll
    for (int u = 0; u < RB; ++u)
#pragma unroll
      for (int s = 0; s < CPL; ++s)
        r[u][s] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.R) + size_t(ev[u]) * a.H +
                                                  min(s * 64 + lane, nch - 1) * 8);
#pragma unroll
    for (int u = 0; u < RB; ++u) bv[u] = a.bias[ev[u]];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int i = i0 + u * kWavesSel;
      if (i >= n) break;                                 // wave-uniform
      const double v = dot2_logit<CPL>(xc, r[u], nch, bv[u], lane);
      if (lane == 0) {
        S.s_val[i] = v;
        S.s_id[i] = ev[u];
      }
    }
  }
}

// The selection of token t from the screen (every thread of the block calls
// it); idx and gates go to oi[k] and og[k].  CPL = 8-element chunks per lane
// of a router row, as in the batch-1 router kernel.
template <int ACT, int CPL>
__device__ __forceinline__ void select_screen_block(const ScreenSelectArgs& b, int t, int32_t* oi, float* og) {
  constexpr int GPT = 12;                          // group maxima per thread (E <= 24,576 in one pass)
  constexpr int GPASS = kSelectThreads * GPT;
  const SelectArgs& a = b.sel;
  __shared__ SelectLds S;
  MOE_SELECT_LDS_NAMES(S);
  __shared__ float s_bnd[kSelectMaxCand];          // screen bound of each listed survivor
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, k = a.k;
  const int G = (E + 3) / 4;
  const float* gr = b.g8 + size_t(t) * G;
  const float* zs = b.z8 + size_t(t) * E;
  const int npass = (G + GPASS - 1) / GPASS;
  if (tid == 0) {
    s_cnt = 0;
    c_cnt = 0;
    s_ntop = 0;
    s_done = 0;
    s_ng = 0;
    s_nref = 0;
    s_tau = -INFINITY;
    s_th0 = -INFINITY;
    s_thf = -INFINITY;
  }
  float gv[GPT];
  auto load_pass = [&](int ps) {
#pragma unroll
    for (int i = 0; i < GPT; ++i) gv[i] = gr[min(ps * GPASS + i * kSelectThreads + tid, G - 1)];
#pragma unroll
    for (int i = 0; i < GPT; ++i)
      if (ps * GPASS + i * kSelectThreads + tid >= G) gv[i] = -INFINITY;
  };
  load_pass(0);
  const double xn2 = a.xnorm[2 * t], dn2 = a.xnorm[2 * t + 1];
  if (!(isfinite(xn2) && isfinite(dn2))) {         // non-finite hidden state: no routing
    if (tid < k) {
      oi[tid] = -1;
      og[tid] = NAN;
    }
    if (tid == 0) atomicOr(a.dev_flag, kDevNonFinite);
    return;
  }
  // binary64 sums of exact squares; the factor covers their rounding and the roots
  const double xn = sqrt(xn2) * (1.0 + 1e-3), dn = sqrt(dn2) * (1.0 + 1e-3);
  const double Btg = xn * b.enmax + dn * b.rqmax + b.babs8;   // screen bound without the relative term
  const double u8 = b.u8;
  auto lower8 = [&](double tv) -> double {
    if (isinf(tv)) return tv < 0 ? -INFINITY : tv;
    const double B = Btg + u8 * fabs(tv);
    const double L = tv - B;
    return L - 1e-15 * (fabs(tv) + B + 1.0);
  };

  // 1. tau0 and the listing threshold, as in select_block
  float tm = -INFINITY;
  for (int ps = 0; ps < npass; ++ps) {
    if (ps > 0) load_pass(ps);
#pragma unroll
    for (int i = 0; i < GPT; ++i) tm = fmaxf(tm, gv[i]);
  }
  if (npass > 1) load_pass(0);
  s_tmax[tid] = tm;
  __syncthreads();
  if (wave == 0 && G >= k) {
    float lm = -INFINITY;
    for (int w = 0; w < kWavesSel; ++w) lm = fmaxf(lm, s_tmax[w * 64 + lane]);
    double tau0 = -INFINITY;
    const bool fin = lm > -INFINITY && lm < INFINITY;
    if (__popcll(__ballot(fin)) >= k && __ballot(lm == INFINITY) == 0ull) {
      float hi = wave_max(fin ? lm : -INFINITY);
      float lo = -wave_max(fin ? -lm : -INFINITY);
#pragma unroll
      for (int it = 0; it < kTauSteps; ++it) {
        const float mid = lo + 0.5f * (hi - lo);
        if (__popcll(__ballot(lm >= mid)) >= k) lo = mid;
        else hi = mid;
      }
      tau0 = (double)lo;              // the screen values are binary32: k of them reach lo exactly
    } else {
      const uint32_t key = f32_key(lm);
      uint32_t K = 0;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = K | (1u << bit);
        if (__popcll(__ballot(key >= cand)) >= k) K = cand;
      }
      if (K != 0) tau0 = (double)key_f32(K);
    }
    const double th = cand_threshold(lower8(tau0), Btg, u8);
    float thf = (float)th;
    if ((double)thf > th) thf = nextafterf(thf, -INFINITY);
    if (lane == 0) {
      s_tau = lower8(tau0);             // L0
      s_th0 = th;
      s_thf = thf;
    }
  }
  __syncthreads();
  const double L0 = s_tau;
  const double th0 = s_th0;
  const float thf = s_thf;
  for (int ps = 0; ps < npass; ++ps) {
    if (ps > 0) load_pass(ps);
    unsigned long long msk[GPT];
    int tot = 0;
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
      const int g = ps * GPASS + i * kSelectThreads + tid;
      msk[i] = __ballot(g < G && gv[i] >= thf);
      tot += __popcll(msk[i]);
    }
    if (tot != 0) {
      int base = 0;
      if (lane == 0) base = atomicAdd(&s_ng, tot);
      base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
      for (int i = 0; i < GPT; ++i) {
        if ((msk[i] >> lane) & 1ull) {
          const int p = base + lanes_below(msk[i]);
          if (p < kSelectMaxCand) s_glist[p] = ps * GPASS + i * kSelectThreads + tid;
        }
        base += __popcll(msk[i]);
      }
    }
  }
  __syncthreads();

  // 2. the listed experts' values and bounds; survivors keep v + B_e >= L0
  auto bnd8 = [&](double v, float2 eb) -> double {
    return xn * (double)eb.x + dn * (double)eb.y + u8 * fabs(v) + b.babs8;
  };
  const int ng = min(s_ng, kSelectMaxCand);
  for (int i0 = 0; i0 < 4 * ng; i0 += kSelectThreads) {
    const int i = i0 + tid;
    const int e = (i < 4 * ng) ? s_glist[i >> 2] * 4 + (i & 3) : E;
    const int ec = min(e, E - 1);
    const double v = (double)zs[ec];
    const float2 eb = b.eb8[ec];
    const double B = bnd8(v, eb);
    const bool pred = e < E && isfinite(v) && v + B >= L0;
    const unsigned long long m = __ballot(pred);
    if (m) {
      const int leader = __ffsll((long long)m) - 1;
      int base = 0;
      if (lane == leader) base = atomicAdd(&s_cnt, __popcll(m));
      base = __shfl(base, leader);
      const int p = base + __popcll(m & ((1ull << lane) - 1ull));
      if (pred && p < kSelectMaxCand) {
        s_val[p] = v;
        s_id[p] = e;
        s_bnd[p] = (float)B;          // only for tau below: rounding to binary32 is absorbed there
      }
    }
  }
  __syncthreads();
  const int n1 = (s_ng > kSelectMaxCand) ? kSelectMaxCand + 1 : s_cnt;
  auto zr = [&](int e) -> double { return (double)zs[e]; };
  const double Btr = a.bt_unit * xn + a.bt_abs;   // bound of the recomputed logits
  int nc = kSelectMaxCand + 1;                     // degenerate unless the recompute set is small
  if (n1 <= kSelectMaxCand) {
    // tau: a value that at least k lower ends v - B reach, by a bisection in
    // value space in wave 0 (within 2^-24 of the lower ends' range of the
    // k-th largest); C = the survivors whose upper end v + B reaches it.  The
    // binary32 bounds are widened by one part in 2^20 to cover their rounding.
    if (wave == 0) {
      constexpr int kPer = kSelectMaxCand / 64;
      auto lo_end = [&](int i) { return s_val[i] - (double)s_bnd[i] * (1.0 + 0x1p-20); };
      double lmin = INFINITY, lmax = -INFINITY;
      for (int c = 0; c < kPer && 64 * c < n1; ++c) {
        const int i = 64 * c + lane;
        if (i < n1) {
          lmin = fmin(lmin, lo_end(i));
          lmax = fmax(lmax, lo_end(i));
        }
      }
      lmin = -wave_max_f64(-lmin);
      lmax = wave_max_f64(lmax);
      double lo = lmin, hi = lmax;
      if (n1 >= k && isfinite(lo) && isfinite(hi)) {
        for (int it = 0; it < 24; ++it) {          // invariant: at least k lower ends >= lo
          const double mid = lo + 0.5 * (hi - lo);
          int cnt = 0;
          for (int c = 0; c < kPer && 64 * c < n1; ++c) {
            const int i = 64 * c + lane;
            cnt += __popcll(__ballot(i < n1 && lo_end(i) >= mid));
          }
          if (cnt >= k) lo = mid;
          else hi = mid;
        }
      } else {
        lo = -INFINITY;
      }
      int base = 0;
      for (int c = 0; c < kPer && 64 * c < n1; ++c) {
        const int i = 64 * c + lane;
        const bool in = i < n1 && s_val[i] + (double)s_bnd[i] * (1.0 + 0x1p-20) >= lo;
        const unsigned long long m = __ballot(in);
        if (in) c_id[base + lanes_below(m)] = s_id[i];
        base += __popcll(m);
      }
      if (lane == 0) c_cnt = base;
    }
    __syncthreads();
    if (c_cnt <= kScreenMaxCand) nc = c_cnt;
  }
  __syncthreads();
  if (tid == 0) {                 // select_tail starts from an empty exact-path list
    c_cnt = 0;
    s_tau = -INFINITY;
  }
  // 3. recompute C from the bf16 rows (when it is small), then certify;
  //    otherwise scan every screen value with exact refinement
  if (nc <= kScreenMaxCand) recompute_logits<CPL>(a, t, nc, S);
  __syncthreads();
  select_tail<ACT>(a, t, nc, S, Btr, a.rel, zr, Btg, u8, oi, og);
}

}  // namespace moe
