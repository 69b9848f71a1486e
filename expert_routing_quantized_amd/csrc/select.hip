// Exact top-k selection and softmax gates, one workgroup per token.
//
// The pages' router "names ten experts per token" (pyshine source tour) and
// drafts are verified "bit-for-bit identical to greedy" ("Guess, then
// check"); here the selected experts must equal those of the exact logits
// (each rounded once to binary64, ties to the lower expert index).  The
// router kernel's fp32 logits z_hat obey |z_hat - z| <= B(z_hat) with
//   B(v) = Bt + 2^-23 |v|,   Bt = gamma'(d) ||x||_2 max_e ||R_e||_2 (1.01)
// (Cauchy-Schwarz on the classical depth-d summation bound, gamma'(n) =
// n 2^-23 / (1 - n 2^-23) which also covers truncating hardware, plus a
// flush-to-zero term).  With tau the k-th largest z_hat, L = tau - B(tau) is
// a lower bound on the k-th largest exact logit, so any expert with
// z_hat + B(z_hat) < L has k experts strictly above it.  The remaining
// candidates (k plus the few inside the band) are recomputed exactly:
//  * double-double accumulation of the exact f64 products (TwoSum chains,
//    Ogita-Rump-Oishi "Sum2" style); its error |s + c - z| is bounded by
//    1.1 (n_l + 16)^2 2^-106 (sum|p| + |b|), n_l = products per lane;
//  * if that interval does not decide the binary64 rounding of z (a value
//    within the bound of a rounding midpoint), an exact fixed-point sum in
//    16-bit digits (integer atomics in LDS) gives the correctly rounded value.
// The pre-filter uses the router blocks' own k-th largest values (a lower
// bound on tau), so the scan keeps only a few dozen survivors whose ranks
// give tau exactly; a bisection over the fp32 keys covers the degenerate
// case of more survivors than fit in LDS (e.g. all logits equal).
#include "moe_internal.h"

namespace moe {

constexpr int kWavesSel = kSelectThreads / 64;
constexpr int kBins = 48;
constexpr int kQBase = -352;   // lowest binary exponent of an fp32 x fp32 product lsb, rounded down

struct SelectArgs {
  const void* R;          // expert-major router [E][H]
  const float* bias;
  const void* x;          // [T][H]
  const float* z;         // [T][E]
  const float* tau;       // [T][ntau]
  int ntau, H, E, k;
  int32_t* idx;           // [T][k]
  float* gates;           // [T][k]
  int* dev_flag;
  double bt_unit;         // gamma'(d) * 1.01 * max_e ||R_e||
  double bt_abs;          // absolute (flush-to-zero) term
  int force_exact;
};

// ---------------------------------------------------------------- reductions
__device__ double block_sum_d(double v, double* red) {
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
__device__ float block_max_f(float v, double* red) {
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
__device__ int block_sum_i(int v, double* red) {
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
__device__ double bins_round(const long long* bins) {
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

// Exact logit of expert e for token t, computed by one wave (all lanes
// return the same value).
template <int ACT>
__device__ double refine_logit(const SelectArgs& a, int t, int e, long long* bins, int lane) {
  const int nch = a.H >> 3;
  const double b = a.bias ? (double)a.bias[e] : 0.0;
  double s = 0.0, c = 0.0, asum = 0.0;
  for (int ch = lane; ch < nch; ch += 64) {
    Chunk<ACT> xc, rc;
    xc.load(a.x, size_t(t) * a.H + ch * 8);
    rc.load(a.R, size_t(e) * a.H + ch * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double p = (double)xc.get(i) * (double)rc.get(i);
      double ss, ee;
      two_sum(s, p, ss, ee);
      s = ss;
      c += ee;
      asum += fabs(p);
    }
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

  // slow path: exact fixed-point accumulation
  for (int i = lane; i < kBins; i += 64) bins[i] = 0;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  int bad = 0;
  for (int ch = lane; ch < nch; ch += 64) {
    Chunk<ACT> xc, rc;
    xc.load(a.x, size_t(t) * a.H + ch * 8);
    rc.load(a.R, size_t(e) * a.H + ch * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) bins_add(bins, (double)xc.get(i) * (double)rc.get(i), &bad);
  }
  if (lane == 0) bins_add(bins, b, &bad);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  double v = 0.0;
  if (lane == 0) v = bins_round(bins);
  if (bad) atomicOr(a.dev_flag, kDevInternal);
  __builtin_amdgcn_wave_barrier();
  return __shfl(v, 0);
}

// ---------------------------------------------------------------- kernel
template <int ACT>
__global__ __launch_bounds__(kSelectThreads) void select_kernel(SelectArgs a) {
  __shared__ float s_val[kSelectMaxCand];
  __shared__ int s_id[kSelectMaxCand];
  __shared__ int c_id[kSelectMaxCand];
  __shared__ double c_z[kSelectMaxCand];
  __shared__ int top_e[kMaxK], new_e[kMaxK];
  __shared__ double top_z[kMaxK], new_z[kMaxK];
  __shared__ long long bins[kWavesSel][kBins];
  __shared__ double red[kWavesSel];
  __shared__ int s_cnt, c_cnt, s_ntop, s_nonfinite;
  __shared__ float s_tau;

  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, k = a.k;
  const float* zr = a.z + size_t(t) * E;

  if (tid == 0) {
    s_cnt = 0;
    c_cnt = 0;
    s_ntop = 0;
    s_nonfinite = 0;
    s_tau = -INFINITY;
  }

  // 1. ||x_t||_2 in f64 (squares of fp32 values are exact in f64).
  double sq = 0.0;
  for (int h = tid; h < a.H; h += kSelectThreads) {
    const float v = (ACT == MOE_BF16)
                        ? bf16_to_f32(reinterpret_cast<const uint16_t*>(a.x)[size_t(t) * a.H + h])
                        : reinterpret_cast<const float*>(a.x)[size_t(t) * a.H + h];
    sq += (double)v * (double)v;
  }
  const double xn = sqrt(block_sum_d(sq, red)) * (1.0 + 1e-12);
  const double Bt = a.bt_unit * xn + a.bt_abs;

  // 2. tau0: largest per-block k-th value (a lower bound on tau).
  float tmax = -INFINITY;
  for (int i = tid; i < a.ntau; i += kSelectThreads) {
    const float v = a.tau[size_t(t) * a.ntau + i];
    if (!isnan(v)) tmax = fmaxf(tmax, v);
  }
  const float tau0 = block_max_f(tmax, red);

  auto lower = [&](double tv) -> double {   // L(tau) = tau - B(tau), rounded down
    if (isinf(tv)) return -INFINITY;
    const double B = Bt + 0x1p-23 * fabs(tv);
    const double L = tv - B;
    return L - 1e-15 * (fabs(tv) + B + 1.0);
  };
  auto is_cand = [&](float v, double L) -> bool {
    if (!isfinite(v)) return false;
    const double dv = (double)v;
    return dv + (Bt + 0x1p-23 * fabs(dv)) >= L;
  };

  // 3. survivors of the pre-filter.
  const double L0 = lower((double)tau0);
  for (int e = tid; e < E; e += kSelectThreads) {
    const float v = zr[e];
    if (!isfinite(v)) s_nonfinite = 1;
    if (is_cand(v, L0)) {
      const int p = atomicAdd(&s_cnt, 1);
      if (p < kSelectMaxCand) {
        s_val[p] = v;
        s_id[p] = e;
      }
    }
  }
  __syncthreads();
  const int n = s_cnt;

  // 4. tau = k-th largest z_hat.
  if (n <= kSelectMaxCand) {
    for (int i = tid; i < n; i += kSelectThreads) {
      const float v = s_val[i];
      int gt = 0, ge = 0;
      for (int j = 0; j < n; ++j) {
        gt += s_val[j] > v;
        ge += s_val[j] >= v;
      }
      if (gt < k && k <= ge) s_tau = v;
    }
    __syncthreads();
  } else {
    // bisection on the monotone key: largest K with #{key >= K} >= k
    uint32_t K = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = K | (1u << bit);
      int cnt = 0;
      for (int e = tid; e < E; e += kSelectThreads) cnt += (f32_key(zr[e]) >= cand);
      cnt = block_sum_i(cnt, red);
      if (cnt >= k) K = cand;
    }
    if (tid == 0) s_tau = (K == 0) ? -INFINITY : key_f32(K);
    __syncthreads();
  }
  const double L = lower((double)s_tau);

  // 5./6. candidates -> exact logits -> running top-k.
  auto process = [&](int nc) {
    for (int i = wave; i < nc; i += kWavesSel) {
      const double zz = refine_logit<ACT>(a, t, c_id[i], bins[wave], lane);
      if (lane == 0) c_z[i] = zz;
    }
    __syncthreads();
    const int ntop = s_ntop;
    const int nu = ntop + nc;
    for (int u = tid; u < nu; u += kSelectThreads) {
      const int eu = (u < ntop) ? top_e[u] : c_id[u - ntop];
      const double zu = (u < ntop) ? top_z[u] : c_z[u - ntop];
      int rank = 0;
      for (int w = 0; w < nu; ++w) {
        const int ew = (w < ntop) ? top_e[w] : c_id[w - ntop];
        const double zw = (w < ntop) ? top_z[w] : c_z[w - ntop];
        rank += (zw > zu) || (zw == zu && ew < eu);
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

  if (n <= kSelectMaxCand) {
    for (int i = tid; i < n; i += kSelectThreads)
      if (is_cand(s_val[i], L)) c_id[atomicAdd(&c_cnt, 1)] = s_id[i];
    __syncthreads();
    process(c_cnt);
  } else {
    for (int r0 = 0; r0 < E; r0 += kSelectMaxCand) {
      const int r1 = min(E, r0 + kSelectMaxCand);
      for (int e = r0 + tid; e < r1; e += kSelectThreads)
        if (is_cand(zr[e], L)) c_id[atomicAdd(&c_cnt, 1)] = e;
      __syncthreads();
      process(c_cnt);
    }
  }

  // 7. outputs.
  if (tid == 0) {
    const int nt = s_ntop;
    int32_t* oi = a.idx + size_t(t) * k;
    float* og = a.gates + size_t(t) * k;
    if (s_nonfinite || nt < k) atomicOr(a.dev_flag, kDevNonFinite);
    if (nt < k) {
      for (int j = 0; j < k; ++j) {
        oi[j] = (j < nt) ? top_e[j] : -1;
        og[j] = NAN;
      }
    } else {
      const double m = top_z[0];
      double w[kMaxK];
      double sum = 0.0;
      for (int j = 0; j < k; ++j) {
        w[j] = exp(top_z[j] - m);
        sum += w[j];
      }
      for (int j = 0; j < k; ++j) {
        oi[j] = top_e[j];
        og[j] = (float)(w[j] / sum);
      }
    }
  }
}

hipError_t launch_select_impl(const Layer& L, const void* x, int T, const float* z,
                              const float* tau, int ntau, int32_t* idx, float* gates,
                              double bt_unit, double bt_abs, hipStream_t s) {
  SelectArgs a;
  a.R = L.router_eh;
  a.bias = L.d.router_bias;
  a.x = x;
  a.z = z;
  a.tau = tau;
  a.ntau = ntau;
  a.H = L.d.hidden;
  a.E = L.d.n_experts;
  a.k = L.d.top_k;
  a.idx = idx;
  a.gates = gates;
  a.dev_flag = L.dev_flag;
  a.bt_unit = bt_unit;
  a.bt_abs = bt_abs;
  a.force_exact = (L.d.flags & MOE_LAYER_FORCE_EXACT_REFINE) ? 1 : 0;
  if (L.d.act_dtype == MOE_BF16)
    hipLaunchKernelGGL(select_kernel<MOE_BF16>, dim3(T), dim3(kSelectThreads), 0, s, a);
  else
    hipLaunchKernelGGL(select_kernel<MOE_F32>, dim3(T), dim3(kSelectThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
