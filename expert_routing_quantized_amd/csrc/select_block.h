// Exact top-k selection and softmax gates, one workgroup per token.
//
// In the pages the router picks ten experts for every token (pyshine source
// tour, Understanding the Architecture), and the verify window must reproduce
// greedy decoding exactly (same section, paragraph on speculative decoding);
// here the selected experts must equal those of the exact logits
// (each rounded once to binary64, ties to the lower expert index).  The
// router kernel's logits z_hat obey |z_hat - z| <= B(z_hat) with
//   B(v) = Bt + 2^-52 |v|,
//   Bt = (gamma(d32, 2^-23) + gamma(d64, 2^-52)) ||x||_2 max_e ||R_e||_2 (1.01) + tiny
// (Cauchy-Schwarz on the classical summation bounds of the router's binary32
// chains and binary64 tail; see router.hip).
//
// Fast path: from the router's maxima of every 4 consecutive logits, any
// value that k of 64 maxima over disjoint sets of experts reach is a lower
// bound tau0 on the k-th largest z_hat, since k distinct experts reach it;
// a 12-step bisection in value space finds one within 2^-12 of the range of
// the 64 maxima (the k-th largest itself is not needed).  Only
// the groups of 4 whose maximum reaches the candidate threshold are read
// (about a dozen of 6,144), their candidates are compacted with a wave
// ballot and ranked by one wave, and if
// no two of the k+1 leading intervals [z_hat - B, z_hat + B] overlap, their
// order is the exact order: idx and the gates (from the binary64 logits) are
// written without recomputing anything.
//
// Exact path (overlapping intervals: exact or near-exact ties; more than 64
// survivors; binary32-accumulated logits): tau = k-th largest z_hat gives
// L = tau - B(tau), a lower bound on the k-th largest exact logit; experts
// with z_hat + B(z_hat) < L have k experts strictly above them, and the rest
// are recomputed exactly:
//  * double-double accumulation of the exact f64 products (TwoSum chains,
//    Ogita-Rump-Oishi "Sum2" style), error <= 1.1 (n_l + 16)^2 2^-106
//    (sum|p| + |b|), n_l = products per lane;
//  * if that interval does not decide the binary64 rounding of z, an exact
//    fixed-point sum in 16-bit digits (integer atomics in LDS) gives the
//    correctly rounded value.
// Every global load of a phase is issued before any is consumed: this kernel
// is latency-bound.
#pragma once

#include <float.h>

#include "moe_internal.h"

namespace moe {

constexpr int kWavesSel = kSelectThreads / 64;
static_assert(kWavesSel * 8 >= 64, "the 64-survivor rank gives each wave 8 survivors");
constexpr int kBins = 48;
constexpr int kQBase = -352;   // lowest binary exponent of an fp32 x fp32 product lsb, rounded down

struct SelectArgs {
  const void* R;          // expert-major router [E][H]
  const float* bias;
  const void* x;          // [T][H]
  const void* z;          // [T][E] router logits: binary64, or binary32 when z32
  int z32;
  const float* gmax;      // [T][ceil(E/4)] maxima of 4 consecutive logits (rounded up)
  const double* xnorm;    // [T] ||x_t||^2
  int H, E, k;
  int32_t* idx;           // [T][k]
  float* gates;           // [T][k]
  int* dev_flag;
  double bt_unit;         // gamma(d, u) * 1.01 * max_e ||R_e||
  double bt_abs;          // absolute (flush-to-zero) term
  double rel;             // u: relative term of the bound (final rounding)
  int force_exact;
};

// ---------------------------------------------------------------- reductions
static __device__ double block_sum_d(double v, double* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_sum_d(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  double r = 0.0;
  for (int i = 0; i < kWavesSel; ++i) r += red[i];
  __syncthreads();
  return r;
}
static __device__ float block_max_f(float v, double* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = -INFINITY;
  for (int i = 0; i < kWavesSel; ++i) r = fmaxf(r, (float)red[i]);
  __syncthreads();
  return r;
}
static __device__ int block_sum_i(int v, double* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
  __syncthreads();
  if (lane == 0) red[w] = (double)v;
  __syncthreads();
  int r = 0;
  for (int i = 0; i < kWavesSel; ++i) r += (int)red[i];
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------- exact sums
__device__ __forceinline__ void bins_add(long long* bins, double p, int* bad) {
  if (p == 0.0) return;
  const unsigned long long bits = (unsigned long long)__double_as_longlong(p);
  const int ex = int((bits >> 52) & 0x7ff);
  unsigned long long m = bits & ((1ull << 52) - 1);
  int q;
  if (ex == 0) {
    q = -1074;
  } else {
    m |= 1ull << 52;
    q = ex - 1075;
  }
  const int pos = q - kQBase;
  if (pos < 0 || (pos >> 4) + 4 >= kBins) {
    *bad = 1;
    return;
  }
  const int bin = pos >> 4, sh = pos & 15;
  const bool neg = (bits >> 63) != 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const long long dig = (long long)((m >> (16 * i)) & 0xffffull) << sh;
    if (dig) atomicAdd(reinterpret_cast<unsigned long long*>(&bins[bin + i]),
                       (unsigned long long)(neg ? -dig : dig));
  }
}

// Correctly rounded binary64 of the integer accumulator (lane 0 only).
static __device__ double bins_round(const long long* bins) {
  uint32_t dig[kBins];
  long long carry = 0;
  for (int i = 0; i < kBins; ++i) {
    const long long v = bins[i] + carry;
    dig[i] = uint32_t(v & 0xffff);
    carry = v >> 16;   // arithmetic: floor division
  }
  const bool neg = carry < 0;
  if (neg) {   // magnitude = two's complement of the digit string
    uint32_t borrow = 1;
    for (int i = 0; i < kBins; ++i) {
      const uint32_t d = ((~dig[i]) & 0xffffu) + borrow;
      dig[i] = d & 0xffffu;
      borrow = d >> 16;
    }
  }
  int top = -1;
  for (int i = kBins - 1; i >= 0; --i)
    if (dig[i]) { top = i; break; }
  if (top < 0) return 0.0;
  const int lz = __clz(dig[top]) - 16;          // leading zeros inside the 16-bit digit
  unsigned long long W = dig[top];
  int have = 16 - lz;
  int i = top - 1;
  while (have + 16 <= 64 && i >= 0) {
    W = (W << 16) | dig[i];
    have += 16;
    --i;
  }
  uint32_t sticky = 0;
  const int need = 64 - have;
  if (i >= 0) {
    if (need > 0) {
      W = (W << need) | (dig[i] >> (16 - need));
      sticky |= dig[i] & ((1u << (16 - need)) - 1u);
    } else {
      sticky |= dig[i];
    }
    --i;
  } else {
    W <<= need;
  }
  for (; i >= 0; --i) sticky |= dig[i];
  unsigned long long mant = W >> 11;
  const unsigned long long rem = W & 0x7ffull;
  int topexp = 16 * top + (15 - lz) + kQBase;   // weight of the leading bit
  if (rem > 0x400ull || (rem == 0x400ull && (sticky != 0 || (mant & 1ull)))) {
    ++mant;
    if (mant == (1ull << 53)) {
      mant >>= 1;
      ++topexp;
    }
  }
  const double v = ldexp((double)mant, topexp - 52);
  return neg ? -v : v;
}

// Correctly rounded logit of expert e for token t by exact fixed-point
// accumulation (one wave; every lane returns it).  The rare fallback of
// refine_logit, kept out of line so the kernels' hot code stays compact.
template <int ACT>
__device__ __attribute__((noinline)) double exact_logit_bins(const void* R, const void* x, const float* bias, int H,
                                                             int t, int e, long long* bins, int lane,
                                                             int* dev_flag) {
  const int nch = H >> 3;
  const double b = bias ? (double)bias[e] : 0.0;
  for (int i = lane; i < kBins; i += 64) bins[i] = 0;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  int bad = 0;
  for (int ch = lane; ch < nch; ch += 64) {
    Chunk<ACT> xc, rc;
    xc.load(x, size_t(t) * H + ch * 8);
    rc.load(R, size_t(e) * H + ch * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) bins_add(bins, (double)xc.get(i) * (double)rc.get(i), &bad);
  }
  if (lane == 0) bins_add(bins, b, &bad);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  double v = 0.0;
  if (lane == 0) v = bins_round(bins);
  if (bad) atomicOr(dev_flag, kDevInternal);
  __builtin_amdgcn_wave_barrier();
  return __shfl(v, 0);
}

// Exact logit of expert e for token t, computed by one wave (all lanes
// return the same value).  Inlined, so the kernel's argument block is never
// copied to private memory and its pointers keep their global address space.
template <int ACT>
__device__ __forceinline__ double refine_logit(const SelectArgs& a, int t, int e, long long* bins, int lane) {
  const int nch = a.H >> 3;
  const double b = a.bias ? (double)a.bias[e] : 0.0;
  // Four independent TwoSum chains per lane (one per chunk slot) for
  // instruction-level parallelism, merged error-free below.
  double sc[4] = {0.0, 0.0, 0.0, 0.0}, cc[4] = {0.0, 0.0, 0.0, 0.0}, asum = 0.0;
  // up to 4 chunks per lane per batch, all loads issued before the sums
  for (int base = 0; base < nch; base += 256) {
    Chunk<ACT> xc[4], rc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ch = min(base + u * 64 + lane, nch - 1);   // clamped: loads issue unconditionally
      xc[u].load(a.x, size_t(t) * a.H + ch * 8);
      rc[u].load(a.R, size_t(e) * a.H + ch * 8);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (base + u * 64 + lane >= nch) continue;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double p = (double)xc[u].get(i) * (double)rc[u].get(i);
        double ss, ee;
        two_sum(sc[u], p, ss, ee);
        sc[u] = ss;
        cc[u] += ee;
        asum += fabs(p);
      }
    }
  }
  double s, c;
  {
    double s01, e01, s23, e23, ee;
    two_sum(sc[0], sc[1], s01, e01);
    two_sum(sc[2], sc[3], s23, e23);
    two_sum(s01, s23, s, ee);
    c = ((cc[0] + cc[1]) + e01) + ((cc[2] + cc[3]) + e23) + ee;
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const double s2 = __shfl_xor(s, m), c2 = __shfl_xor(c, m), a2 = __shfl_xor(asum, m);
    double ss, ee;
    two_sum(s, s2, ss, ee);
    s = ss;
    c = (c + c2) + ee;
    asum = asum + a2;
  }
  {
    double ss, ee;
    two_sum(s, b, ss, ee);
    s = ss;
    c += ee;
    asum += fabs(b);
  }
  double r, d;
  two_sum(s, c, r, d);
  const double nl = 8.0 * double((nch + 63) / 64);
  const double eps = 1.1 * (nl + 16.0) * (nl + 16.0) * 0x1p-106 * asum;
  const double up = nextafter(r, INFINITY) - r;
  const double dn = r - nextafter(r, -INFINITY);
  const bool ok = !a.force_exact && isfinite(r) && (d + eps < 0.5 * up) && (d - eps > -0.5 * dn);
  if (ok) return r;
  if (lane == 0) atomicAdd(refine_counter(a.dev_flag), 1ull);   // statistics (moe_layer_stats)
  return exact_logit_bins<ACT>(a.R, a.x, a.bias, a.H, t, e, bins, lane, a.dev_flag);
}

// ---------------------------------------------------------------- kernel
constexpr int kTauSteps = 12;   // bisection steps for tau0
constexpr int kFastMax = 256;   // survivors the ranking fast path takes

__device__ __forceinline__ int lanes_below(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
}

// Smallest value th such that every v >= th can satisfy v + Bt + u |v| >= L
// (rounded down: the test is conservative).
static __device__ double cand_threshold(double L, double Bt, double u) {
  if (isinf(L)) return L;
  const double D = L - Bt;
  double th = (D >= 0) ? D / (1.0 + u) : D / (1.0 - u);
  return th - (1e-12 * fabs(th) + 1e-300);
}

__device__ __forceinline__ unsigned long long f64_key(double d) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(d);
  if (isnan(d)) return 0ull;
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}
__device__ __forceinline__ double key_f64(unsigned long long k) {
  const unsigned long long u = (k >> 63) ? (k & 0x7fffffffffffffffull) : ~k;
  return __longlong_as_double((long long)u);
}

// LDS of one block's selection.
struct SelectLds {
  double s_val[kSelectMaxCand];   // survivors' values (then reused by the re-ranking)
  int s_id[kSelectMaxCand];       // survivors' experts
  int c_id[kSelectMaxCand];
  double c_z[kSelectMaxCand];
  int s_glist[kSelectMaxCand];    // listed groups
  float s_tmax[kSelectThreads];
  int top_e[kMaxK], new_e[kMaxK];
  double top_z[kMaxK], new_z[kMaxK], s_w[kMaxK];
  long long bins[kWavesSel][kBins];
  double red[kWavesSel];
  int s_cnt, c_cnt, s_ntop, s_done, s_ng, s_nref;
  int s_ref[64];                  // ranks refined by the cluster pass
  int s_rankp[kWavesSel][kFastMax];   // fast path: each wave's part of each survivor's rank
  double x_z[64];                 // their exact logits, by rank
  double s_tau, s_th0;
  double s_kth;                   // approximate logit of the k-th expert chosen (when all k are)
  int s_red3[3][kWavesSel];       // per-wave partial sums
  int s_nf;                       // survivors the fast path keeps (-1: none, go exact)
  float s_thf;                    // s_th0 in binary32, rounded down
};

// Names of the SelectLds fields inside a selection function.
#define MOE_SELECT_LDS_NAMES(S)                                                        \
  double* s_val = S.s_val;                                                           \
  int* s_id = S.s_id;                                                                \
  int* c_id = S.c_id;                                                                \
  double* c_z = S.c_z;                                                               \
  int* s_glist = S.s_glist;                                                          \
  float* s_tmax = S.s_tmax;                                                          \
  int *top_e = S.top_e, *new_e = S.new_e;                                            \
  double *top_z = S.top_z, *new_z = S.new_z, *s_w = S.s_w;                           \
  auto& bins = S.bins;                                                               \
  double* red = S.red;                                                               \
  int &s_cnt = S.s_cnt, &c_cnt = S.c_cnt, &s_ntop = S.s_ntop, &s_done = S.s_done;    \
  int &s_ng = S.s_ng, &s_nref = S.s_nref;                                            \
  int* s_ref = S.s_ref;                                                              \
  double* x_z = S.x_z;                                                               \
  double &s_tau = S.s_tau, &s_th0 = S.s_th0;                                         \
  float& s_thf = S.s_thf;                                                            \
  (void)s_val; (void)s_id; (void)c_id; (void)c_z; (void)s_glist; (void)s_tmax;       \
  (void)top_e; (void)new_e; (void)top_z; (void)new_z; (void)s_w; (void)bins;         \
  (void)red; (void)s_ref; (void)x_z

// The end of a selection, shared by the full-router and the screened paths.
// On entry S.s_val / S.s_id hold n survivors (n = kSelectMaxCand + 1: too
// many to hold) whose values v obey |v - z| <= Btv + uv |v|, and every
// expert outside them has an exact logit below the k-th largest.  zr(e) is
// an approximate logit of every expert with |zr(e) - z| <= Btz + uz |zr(e)|,
// read only when the survivors did not fit.  Certifies the order (refining
// exactly where intervals overlap) and writes idx and gates to oi / og.
//
// The result depends on the input alone, not on which survivors were
// passed: the order is the exact order (ties by index), and the gates are
// the softmax of the k chosen experts' approximate logits v (the values the
// survivors carry; zt(S) writes them to S.new_z[0..k) for S.top_e[0..k)
// when the exact path chose), in that order.  S.s_kth gets the k-th one.
// The rest of select_tail when the fast path has not certified the order:
// the cluster pass's refinements and re-rank, then the exact path.  (Out of
// line it measured slower: the lambdas' captures then live in scratch.)
template <int ACT, class ZR, class ZT>
__device__ __forceinline__ void select_tail_slow(const SelectArgs& a, int t, int n, int nf, SelectLds& S,
                                                           double Btv, double uv, ZR zr, double Btz, double uz,
                                                           ZT zt, int32_t* oi, float* og) {
  MOE_SELECT_LDS_NAMES(S);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = a.E, k = a.k;
  n = __builtin_amdgcn_readfirstlane(n);           // block-uniform: scalar loop bounds
  const double Bt = Btv, u = uv;
  auto bound = [&](double v) -> double { return Bt + u * fabs(v); };
  auto lower_b = [](double tv, double B0, double uu) -> double {   // tv - B(tv), rounded down
    if (isinf(tv)) return tv < 0 ? -INFINITY : tv;
    const double B = B0 + uu * fabs(tv);
    const double L = tv - B;
    return L - 1e-15 * (fabs(tv) + B + 1.0);
  };
  auto lower = [&](double tv) -> double { return lower_b(tv, Bt, u); };
  // gates of the k ranked experts from their approximate logits zv[0..k) (lanes < k of one wave)
  auto write_gates = [&](const double* zv, const int* ev) {
    // (the sum over the k weights in the fixed order of wave_sum_f64's tree)
    const double w = (lane < k) ? exp(zv[min(lane, k - 1)] - zv[0]) : 0.0;
    const double sum = wave_sum_f64(w);
    if (lane < k) {
      oi[lane] = ev[lane];
      og[lane] = (float)(w / sum);
    }
    if (lane == 0) {
      S.s_kth = zv[k - 1];
      s_done = 1;
    }
  };

  if (nf >= 0 && s_nref > 0) {
    for (int i = wave; i < s_nref; i += kWavesSel) {
      const double zz = refine_logit<ACT>(a, t, c_id[s_ref[i]], bins[wave], lane);
      if (lane == 0) x_z[s_ref[i]] = zz;
    }
    __syncthreads();
    if (wave == 0) {
      // re-rank with the exact logits where known (interval of width 0)
      bool ex = false;
      for (int i = 0; i < s_nref; ++i) ex = ex || (s_ref[i] == lane);
      const double va = (lane < n) ? c_z[lane] : -INFINITY;    // approximate logit (gates)
      const double v = (lane < n) ? (ex ? x_z[lane] : va) : -INFINITY;
      const double bw = (lane < n && !ex) ? bound(va) : 0.0;
      const int e = (lane < n) ? c_id[lane] : 0x7fffffff;
      int rank = 0;
      for (int j = 0; j < n; ++j) {
        const double vj = readlane_f64(v, j);
        const int ej = __builtin_amdgcn_readlane(e, j);
        rank += int((vj > v) | ((vj == v) & (ej < e)));
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      if (lane < n) {          // reuse the first slots of the candidate lists
        s_val[rank] = v;
        x_z[rank] = bw;
        s_id[rank] = e;
        if (rank < k) {
          new_z[rank] = va;
          new_e[rank] = e;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // adjacent ranks r < k: disjoint intervals, or both exact (their
      // order is then the exact order, ties by index)
      const int npair = min(k, n - 1);
      bool bad = false;
      if (lane < npair) {
        const double hv = s_val[lane], hb = x_z[lane], lv = s_val[lane + 1], lb = x_z[lane + 1];
        bad = !((hv - hb > lv + lb) || (hb == 0.0 && lb == 0.0));
      }
      if (__ballot(bad) == 0ull) write_gates(new_z, new_e);
    }
    __syncthreads();
    if (s_done) return;
  }

  // 5b. exact path.
  auto process = [&](int nc) {
    for (int i = wave; i < nc; i += kWavesSel) {
      const double zz = refine_logit<ACT>(a, t, c_id[i], bins[wave], lane);
      if (lane == 0) c_z[i] = zz;
    }
    __syncthreads();
    const int ntop = s_ntop;
    const int nu = ntop + nc;
    for (int q = tid; q < nu; q += kSelectThreads) {
      const int eu = (q < ntop) ? top_e[q] : c_id[q - ntop];
      const double zu = (q < ntop) ? top_z[q] : c_z[q - ntop];
      int rank = 0;
      for (int w = 0; w < nu; ++w) {
        const int ew = (w < ntop) ? top_e[w] : c_id[w - ntop];
        const double zw = (w < ntop) ? top_z[w] : c_z[w - ntop];
        rank += int((zw > zu) | ((zw == zu) & (ew < eu)));
      }
      if (rank < k) {
        new_e[rank] = eu;
        new_z[rank] = zu;
      }
    }
    __syncthreads();
    const int nn = min(k, nu);
    if (tid < nn) {
      top_e[tid] = new_e[tid];
      top_z[tid] = new_z[tid];
    }
    if (tid == 0) {
      s_ntop = nn;
      c_cnt = 0;
    }
    __syncthreads();
  };

  // the candidates near the k-th largest value, refined exactly: the
  // survivors in one range, or (degenerate: more survivors than LDS holds)
  // every expert, range by range, from the approximate logits zr
  const bool degenerate = n > kSelectMaxCand;
  double th;
  if (!degenerate) {
    // tau = k-th largest z_hat among the survivors, then the band around it
    for (int i = tid; i < n; i += kSelectThreads) {
      const double v = s_val[i];
      int gt = 0, ge = 0;
      for (int j = 0; j < n; ++j) {
        gt += s_val[j] > v;
        ge += s_val[j] >= v;
      }
      if (gt < k && k <= ge) s_tau = v;
    }
    __syncthreads();
    th = cand_threshold(lower(s_tau), Bt, u);
  } else {
    // bisection on the monotone 64-bit key for tau
    unsigned long long K = 0;
    for (int bit = 63; bit >= 0; --bit) {
      const unsigned long long cand = K | (1ull << bit);
      int cnt = 0;
      for (int e = tid; e < E; e += kSelectThreads) cnt += (f64_key(zr(e)) >= cand);
      cnt = block_sum_i(cnt, red);
      if (cnt >= k) K = cand;
    }
    const double tau = (K == 0) ? -INFINITY : key_f64(K);
    th = cand_threshold(lower_b(tau, Btz, uz), Btz, uz);
  }
  const int span = degenerate ? E : n;
  for (int r0 = 0; r0 < span; r0 += kSelectMaxCand) {
    const int r1 = min(span, r0 + kSelectMaxCand);
    for (int i = r0 + tid; i < r1; i += kSelectThreads) {
      if (degenerate) {
        const double v = zr(i);
        if (isfinite(v) && v >= th) c_id[atomicAdd(&c_cnt, 1)] = i;
      } else if (s_val[i] >= th) {
        c_id[atomicAdd(&c_cnt, 1)] = s_id[i];
      }
    }
    __syncthreads();
    process(c_cnt);
  }

  // 6. outputs: the k experts in exact order; gates = softmax over their
  //    approximate logits (zt), or over the exact ones when one of those is
  //    not finite.
  const int nt = s_ntop;
  if (nt == k) {
    zt(S);                       // S.new_z[0..k) for S.top_e[0..k) (every thread calls it)
    __syncthreads();
    if (wave == 0) {
      const bool fin = __ballot(lane < k && !isfinite(new_z[lane])) == 0ull;
      write_gates(fin ? new_z : top_z, top_e);
    }
  } else if (tid < k) {
    oi[tid] = (tid < nt) ? top_e[tid] : -1;
    og[tid] = NAN;
  }
  if (tid == 0 && nt < k) atomicOr(a.dev_flag, kDevNonFinite);
}

template <int ACT, class ZR, class ZT>
__device__ __forceinline__ void select_tail(const SelectArgs& a, int t, int n, SelectLds& S, double Btv,
                                            double uv, ZR zr, double Btz, double uz, ZT zt, int32_t* oi,
                                            float* og) {
  MOE_SELECT_LDS_NAMES(S);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = a.E, k = a.k;
  n = __builtin_amdgcn_readfirstlane(n);           // block-uniform: scalar loop bounds
  const double Bt = Btv, u = uv;
  auto bound = [&](double v) -> double { return Bt + u * fabs(v); };
  auto lower_b = [](double tv, double B0, double uu) -> double {   // tv - B(tv), rounded down
    if (isinf(tv)) return tv < 0 ? -INFINITY : tv;
    const double B = B0 + uu * fabs(tv);
    const double L = tv - B;
    return L - 1e-15 * (fabs(tv) + B + 1.0);
  };
  auto lower = [&](double tv) -> double { return lower_b(tv, Bt, u); };
  // gates of the k ranked experts from their approximate logits zv[0..k) (lanes < k of one wave)
  auto write_gates = [&](const double* zv, const int* ev) {
    // (the sum over the k weights in the fixed order of wave_sum_f64's tree)
    const double w = (lane < k) ? exp(zv[min(lane, k - 1)] - zv[0]) : 0.0;
    const double sum = wave_sum_f64(w);
    if (lane < k) {
      oi[lane] = ev[lane];
      og[lane] = (float)(w / sum);
    }
    if (lane == 0) {
      S.s_kth = zv[k - 1];
      s_done = 1;
    }
  };

  // 5a. fast path: the survivors' ranks by v (each wave counts, for every
  //     survivor, the larger ones among its share of the others), then one
  //     wave certifies the order.  Past 64 survivors, ranks 64 and on are
  //     dropped when they lie strictly below rank k-1's interval (none of
  //     them can then be among the k).
  constexpr int Q = kFastMax / 64;
  const bool fast = n <= kFastMax && !a.force_exact;     // block-uniform
  if (fast) {
    double v[Q];
    int e[Q], part[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int i = lane + 64 * q;
      v[q] = (i < n) ? s_val[i] : -INFINITY;
      e[q] = (i < n) ? s_id[i] : 0x7fffffff;
      part[q] = 0;
    }
    if (n <= 64) {
      // wave w compares every survivor (one per lane) with survivors 8 w ..
      // 8 w + 7, read from LDS at one address per instruction (broadcast)
      double vj[8];
      int ej[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {                    // unconditional loads (no branch between them)
        const int j = min(wave * 8 + u, n - 1);
        vj[u] = s_val[j];
        ej[u] = s_id[j];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        part[0] += int((wave * 8 + u < n) & ((vj[u] > v[0]) | ((vj[u] == v[0]) & (ej[u] < e[0]))));
    } else {
    const int J = (n + kWavesSel - 1) / kWavesSel;
    const int j0 = wave * J, j1 = min(n, j0 + J);
    const int nq = (n + 63) >> 6;                      // lane groups in use
#pragma unroll
    for (int qj = 0; qj < Q; ++qj) {
      const int lo = max(j0, 64 * qj), hi = min(j1, 64 * qj + 64);   // wave-uniform
      for (int j = lo; j < hi; ++j) {
        const double vj = readlane_f64(v[qj], j - 64 * qj);
        const int ej = __builtin_amdgcn_readlane(e[qj], j - 64 * qj);
#pragma unroll
        for (int q = 0; q < Q; ++q)      // (bitwise operators: no branches)
          if (q < nq) part[q] += int((vj > v[q]) | ((vj == v[q]) & (ej < e[q])));
      }
    }
    }
    // per-wave partial ranks (no initialisation, no atomics), summed by wave 0
#pragma unroll
    for (int q = 0; q < Q; ++q)
      if (q == 0 || lane + 64 * q < n) S.s_rankp[wave][lane + 64 * q] = part[q];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int i = lane + 64 * q;
        if (i < n) {
          int rank = 0;
#pragma unroll
          for (int w = 0; w < kWavesSel; ++w) rank += S.s_rankp[w][i];
          c_z[rank] = v[q];
          c_id[rank] = e[q];
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      int m = n;
      if (n > 64) {
        const double zk = c_z[k - 1], z64 = c_z[64];
        m = (z64 + bound(z64) < lower(zk)) ? 64 : -1;
        if (m == 64) {          // the kept ranks become the survivors (for the exact path too)
          s_val[lane] = c_z[lane];
          s_id[lane] = c_id[lane];
        }
      }
      if (lane == 0) S.s_nf = m;
    }
    __syncthreads();
  }
  const int nf = fast ? __builtin_amdgcn_readfirstlane(S.s_nf) : -1;   // block-uniform
  if (nf > 0) n = nf;
  if (nf >= 0 && wave == 0) {
    // ranks r and r+1 must not overlap for r < k (order of the k, and the cut)
    const int npair = min(k, n - 1);
    bool bad = false;
    if (lane < npair) {
      const double hi = c_z[lane], lo = c_z[lane + 1];
      bad = !(hi - bound(hi) > lo + bound(lo));
    }
    const unsigned long long bm = __ballot(bad);
    const bool certified = (n >= k) && (bm == 0ull);
    if (certified) {
      write_gates(c_z, c_id);
    } else if (n >= k) {
      // cluster pass: the ranks of every overlapping pair, and, when the
      // cut (k-1, k) overlaps, every later rank whose interval reaches the
      // lower end of rank k's, are refined to their exact logits
      bool mark = lane < n && ((((bm >> lane) & 1ull) != 0) || (lane > 0 && ((bm >> (lane - 1)) & 1ull) != 0));
      if (((bm >> (k - 1)) & 1ull) != 0 && lane > k && lane < n) {
        const double zk = c_z[k];
        if (c_z[lane] + bound(c_z[lane]) >= zk - bound(zk)) mark = true;
      }
      const unsigned long long mm = __ballot(mark);
      if (mark) s_ref[__popcll(mm & ((1ull << lane) - 1ull))] = lane;
      if (lane == 0) s_nref = (__popcll(mm) <= 2 * kWavesSel) ? __popcll(mm) : 0;
    }
  }
  __syncthreads();
  if (s_done) return;
  select_tail_slow<ACT>(a, t, n, nf, S, Btv, uv, zr, Btz, uz, zt, oi, og);
}


// The selection of token t by one block of kSelectThreads threads (every
// thread must call it); idx and gates go to oi[k] and og[k], global or LDS.
template <int ACT>
__device__ __forceinline__ void select_block(const SelectArgs& a, int t, int32_t* oi, float* og) {
  constexpr int GPT = 12;                          // group maxima per thread (E <= 24,576 in one pass)
  constexpr int GPASS = kSelectThreads * GPT;      // groups per pass
  __shared__ SelectLds S;
  MOE_SELECT_LDS_NAMES(S);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, k = a.k;
  const int G = (E + 3) / 4;                       // groups of 4 consecutive experts
  // logit e of this token (binary64 or binary32 storage)
  auto zr = [&](int e) -> double {
    const size_t i = size_t(t) * E + e;
    return a.z32 ? (double)static_cast<const float*>(a.z)[i] : static_cast<const double*>(a.z)[i];
  };
  const float* gr = a.gmax + size_t(t) * G;
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

  // 1. loads: the group maxima (rounded-up binary32 maxima of 4 logits) and ||x||^2.
  float gv[GPT];
  auto load_pass = [&](int ps) {
#pragma unroll
    for (int i = 0; i < GPT; ++i) gv[i] = gr[min(ps * GPASS + i * kSelectThreads + tid, G - 1)];
#pragma unroll
    for (int i = 0; i < GPT; ++i)
      if (ps * GPASS + i * kSelectThreads + tid >= G) gv[i] = -INFINITY;
  };
  load_pass(0);
  // ||x||^2 is a binary64 sum of exact squares (no underflow for any bf16 or
  // fp32 input); the factor covers its rounding and the square root
  const double xn = sqrt(a.xnorm[t]) * (1.0 + 1e-3);
  const double Bt = a.bt_unit * xn + a.bt_abs;
  const double u = a.rel;

  auto bound = [&](double v) -> double { return Bt + u * fabs(v); };
  auto lower = [&](double tv) -> double {   // L(tau) = tau - B(tau), rounded down
    if (isinf(tv)) return tv < 0 ? -INFINITY : tv;
    const double B = bound(tv);
    const double L = tv - B;
    return L - 1e-15 * (fabs(tv) + B + 1.0);
  };

  // 2. tau0, a lower bound on the k-th largest z_hat: each thread's maximum
  //    over its groups, then in wave 0 the maximum over 8 threads per lane
  //    (64 disjoint sets of experts), a value lo that k of those 64 reach,
  //    one binary32 ulp down (the maxima were rounded up): k distinct experts
  //    lie above it.  Wave 0 also turns it into the candidate threshold.
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
    for (int w = 0; w < kWavesSel; ++w) lm = fmaxf(lm, s_tmax[w * 64 + lane]);   // never NaN
    double tau0 = -INFINITY;
    const bool fin = lm > -INFINITY && lm < INFINITY;
    if (__popcll(__ballot(fin)) >= k && __ballot(lm == INFINITY) == 0ull) {
      // bisection in value space; invariant: at least k lane values >= lo
      float hi = wave_max(fin ? lm : -INFINITY);
      float lo = -wave_max(fin ? -lm : -INFINITY);
#pragma unroll
      for (int it = 0; it < kTauSteps; ++it) {
        const float mid = lo + 0.5f * (hi - lo);
        if (__popcll(__ballot(lm >= mid)) >= k) lo = mid;
        else hi = mid;
      }
      tau0 = (double)nextafterf(lo, -INFINITY);
    } else {
      // infinite maxima or fewer than k finite ones: the k-th largest by a
      // bisection on the monotone key (largest K with #{key >= K} >= k)
      const uint32_t key = f32_key(lm);
      uint32_t K = 0;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = K | (1u << bit);
        if (__popcll(__ballot(key >= cand)) >= k) K = cand;
      }
      if (K != 0) tau0 = (double)nextafterf(key_f32(K), -INFINITY);
    }
    const double th = cand_threshold(lower(tau0), Bt, u);
    float thf = (float)th;
    if ((double)thf > th) thf = nextafterf(thf, -INFINITY);
    if (lane == 0) {
      s_th0 = th;
      s_thf = thf;
    }
  }
  __syncthreads();

  // 3. groups whose maximum reaches the threshold (compared in binary32
  //    against th0 rounded down: a superset), listed with one LDS atomic per
  //    wave; then their experts with z_hat >= th0, compacted the same way.
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
    if (tot != 0) {                                    // wave-uniform
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
  const int ng = min(s_ng, kSelectMaxCand);
  for (int i0 = 0; i0 < 4 * ng; i0 += kSelectThreads) {   // 4 experts per listed group
    const int i = i0 + tid;
    const int e = (i < 4 * ng) ? s_glist[i >> 2] * 4 + (i & 3) : E;
    const double v = zr(min(e, E - 1));
    const bool pred = e < E && isfinite(v) && v >= th0;
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
      }
    }
  }
  __syncthreads();
  const int n = (s_ng > kSelectMaxCand) ? kSelectMaxCand + 1 : s_cnt;

  auto zt = [&](SelectLds& S2) {   // the chosen experts' logits as the router gave them
    if (tid < k) S2.new_z[tid] = zr(S2.top_e[tid]);
  };
  select_tail<ACT>(a, t, n, S, Bt, u, zr, Bt, u, zt, oi, og);
}

// SelectArgs of a layer for one call (host).
SelectArgs make_select_args(const Layer& L, const void* x, const void* z, bool z32, const float* gmax,
                            const double* xnorm, int32_t* idx, float* gates, const RouterBound& rb);

}  // namespace moe
