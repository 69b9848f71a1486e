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

// ---------------------------------------------------------------- the list
// At batch 1 the screen can also do the recompute itself, for the experts
// whose upper end v + B reaches a threshold theta taken from recent tokens
// (their k-th largest logit: consecutive tokens' values spread little, so
// the k experts of the next token nearly always lie above it).  Each such
// expert's logit is recomputed by the screen block that owns its row and
// appended to a list in the workspace: each block that lists rows takes
// consecutive slots with one atomic add on the list's counter, and every
// block also writes how many rows it listed.  The selection then reads
// about 6 KB instead of the screen values, and accepts the list only when
// it can prove it complete:
//  - the counter equals the sum of the blocks' counts and fits the list: the
//    counter started this call at 0, so slots [0, counter) were all written
//    by this call, and no listed row was dropped;
//  - at least k entries have a lower end z - B >= theta, so the k-th
//    largest exact logit is >= theta, above every expert left out (those
//    have z <= v + B < theta).
// Otherwise it selects from the screen values as before; either way the
// result is the same (select_tail's output depends on the input alone).
// The workspace carries the state from call to call: the list's counter,
// which the last kernel of each call sets back to 0 (a counter that did not
// start at 0 -- a workspace's first use -- only makes that call take the
// slower path), a call counter, and the ring of recent k-th logits, into
// which the last kernel moves the call's k-th logit.
constexpr int kHintRing = 16;
constexpr int kListSlots = 256;           // table size (a power of 2, <= kFastMax)

struct HintWords {                        // 128 bytes of the workspace
  unsigned long long epoch;               // calls so far (from any start value)
  float kth;                              // this call's k-th logit (NaN: none)
  unsigned int listed_calls;              // calls whose selection took the list (statistics)
  unsigned int list_count;                // entries appended to the list in this call
  unsigned int win_count[8];              // verify windows: entries appended to token t's list
  float pad[3];
  float ring[kHintRing];                  // k-th logits of recent calls
};
static_assert(sizeof(HintWords) <= 256, "the screen reads a 256-byte stand-in in place of a hint");

// theta from the ring: its minimum less a quarter of its range (+inf, i.e.
// no list, while the ring holds a value that is not finite).  0.25 (mx - mn)
// is exact, so the result does not depend on contraction into an fma.
__device__ __forceinline__ float hint_threshold(const HintWords* h) {
  float mn = INFINITY, mx = -INFINITY;
  bool ok = true;
#pragma unroll
  for (int j = 0; j < kHintRing; ++j) {
    const float r = h->ring[j];
    ok = ok && isfinite(r);
    mn = fminf(mn, r);
    mx = fmaxf(mx, r);
  }
  const float th = mn - 0.25f * (mx - mn);
  return (ok && isfinite(th)) ? th : INFINITY;
}

// hint_threshold for one wave: lane l holds ring[l % 16]; minimum and
// maximum are exact in any order, so every lane gets the same value as
// hint_threshold.
__device__ __forceinline__ float hint_threshold_lanes(float r) {   // r = ring[lane % 16]
  const bool ok = __ballot(!isfinite(r)) == 0ull;
  const float rr = ok ? r : 0.f;
  const float mx = wave_max(rr), mn = -wave_max(-rr);
  const float th = mn - 0.25f * (mx - mn);
  return (ok && isfinite(th)) ? th : INFINITY;
}

// End of a call, by one wave of the call's last kernel: the k-th logit into
// the ring (every slot while the ring is not all finite), then the next
// counter value.  hint_read issues the loads where the kernel starts and
// hint_write only stores, so the wave never waits on them.
struct HintRead {
  unsigned long long epoch;
  float kth;
  float ring;              // ring[lane % 16]
};
__device__ __forceinline__ HintRead hint_read(const HintWords* h, int lane) {
  HintRead r;
  r.epoch = h->epoch;
  r.kth = h->kth;
  r.ring = h->ring[lane & (kHintRing - 1)];
  return r;
}
__device__ __forceinline__ void hint_write(HintWords* h, const HintRead& r, int lane) {   // all 64 lanes
  const bool ok = __ballot(!isfinite(r.ring)) == 0ull;
  if (isfinite(r.kth) && lane < kHintRing && (!ok || int(r.epoch % kHintRing) == lane)) h->ring[lane] = r.kth;
  if (lane == 0) {
    h->kth = NAN;
    h->list_count = 0u;
    h->epoch = r.epoch + 1;
  }
}

struct ScreenSelectArgs {
  SelectArgs sel;          // router rows, bias, x, idx/gates, the recomputed logits' bound;
                           // sel.xnorm -> [T][2]: ||x_t||^2, ||delta_t||^2
  const float* z8;         // [T][E] screen values v (binary32, nearest)
  const float* g8;         // [T][ceil(E/4)] their maxima over 4 consecutive experts
  const float2* eb8;       // [E]: (||eps_e|| rounded up, ||Rq_e|| rounded up)
  double enmax, rqmax;     // maxima of the two norms over the experts
  double u8, babs8;        // relative and absolute terms of the screen bound
  HintWords* hint;         // with the list (else null): the call's state
  const unsigned char* cnt8;   // [nw] rows each screen block listed (windows: [T][cstride])
  const ulonglong2* list;  // [kListSlots] (e, logit bits) (windows: [T][kListSlots])
  int nw;                  // screen blocks (windows: screen waves)
  int advance;             // this kernel ends the call: advance the hint (block 0)
  unsigned int* wcount;    // verify windows: token t's counter is wcount[t] (else null: batch 1)
  int cstride;             // verify windows: bytes of counts per token (a multiple of 16)
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
__device__ __forceinline__ void select_screen_core(const ScreenSelectArgs& b, int t, SelectLds& S, int32_t* oi,
                                                   float* og) {
  constexpr int GPT = 12;                          // group maxima per thread (E <= 24,576 in one pass)
  constexpr int GPASS = kSelectThreads * GPT;
  const SelectArgs& a = b.sel;
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
    S.s_kth = NAN;
  }
  // every load of the list path first (one round trip): ||x||^2 and
  // ||delta||^2, the hint, this thread's table slot and count words
  const double xn2 = a.xnorm[2 * t], dn2 = a.xnorm[2 * t + 1];
  // (a verify window keeps one list, counter and row of counts per token)
  const bool win = b.wcount != nullptr;
  const ulonglong2* tlist = win ? b.list + size_t(t) * kListSlots : b.list;
  const unsigned char* tcnt8 = win ? b.cnt8 + size_t(t) * b.cstride : b.cnt8;
  const float ring_v = b.hint->ring[lane & (kHintRing - 1)];
  const unsigned list_n = win ? b.wcount[t] : b.hint->list_count;
  const ulonglong2 ent = tlist[min(tid, kListSlots - 1)];
  const int nw16 = (b.nw + 15) >> 4;               // 16-byte words of counts
  constexpr int kCw = 2;                           // words per thread loaded up front (E <= 65,536)
  uint4 cwv[kCw];
#pragma unroll
  for (int u = 0; u < kCw; ++u) cwv[u] = reinterpret_cast<const uint4*>(tcnt8)[min(tid + u * kSelectThreads, nw16 - 1)];
  // (a non-finite hidden state is handled once these loads have all been
  // used: an early return here would let the compiler sink them past its wait)
  // binary64 sums of exact squares; the factor covers their rounding and the roots
  const double xn = sqrt(xn2) * (1.0 + 1e-3), dn = sqrt(dn2) * (1.0 + 1e-3);
  const double Btg = xn * b.enmax + dn * b.rqmax + b.babs8;   // screen bound without the relative term
  const double u8 = b.u8;
  const double Btr = a.bt_unit * xn + a.bt_abs;   // bound of the recomputed logits
  auto zr = [&](int e) -> double { return (double)zs[e]; };
  auto zt = [&](SelectLds& S2) {   // the chosen experts' logits recomputed from the bf16 rows
    if (tid < k) S2.c_id[tid] = S2.top_e[tid];
    __syncthreads();
    recompute_logits<CPL>(a, t, k, S2);
    __syncthreads();
    if (tid < k) S2.new_z[tid] = S2.s_val[tid];
  };

  // 0. the screen's table, when it can be proved complete
  {
    const float theta = hint_threshold_lanes(ring_v);
    int csum = 0;
#pragma unroll
    for (int u = 0; u < kCw; ++u) {
      const int w = tid + u * kSelectThreads;
      const int nb = (w < nw16) ? b.nw - 16 * w : 0;   // bytes of this word that are counts
      const uint32_t cw[4] = {cwv[u].x, cwv[u].y, cwv[u].z, cwv[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int valid = min(max(nb - 4 * j, 0), 4);
        const uint32_t m = (valid >= 4) ? 0xffffffffu : ((1u << (8 * valid)) - 1u);
        csum = (int)__builtin_amdgcn_udot4(cw[j] & m, 0x01010101u, (uint32_t)csum, false);
      }
    }
    for (int w = tid + kCw * kSelectThreads; w < nw16; w += kSelectThreads) {   // E > 65,536 only
      const uint4 c = reinterpret_cast<const uint4*>(tcnt8)[w];
      const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
      const int nb = b.nw - 16 * w;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int valid = min(max(nb - 4 * j, 0), 4);
        const uint32_t m = (valid >= 4) ? 0xffffffffu : ((1u << (8 * valid)) - 1u);
        csum = (int)__builtin_amdgcn_udot4(cw[j] & m, 0x01010101u, (uint32_t)csum, false);
      }
    }
    const bool match = tid < kListSlots && (unsigned)tid < list_n;
    const int e = int(ent.x & 0xffffffffull);
    const bool bad = match && (ent.x >= (unsigned long long)E);
    const double zv = __longlong_as_double((long long)ent.y);
    const double Bz = Btr + a.rel * fabs(zv);      // the recomputed logit's lower end, rounded down
    const bool low_ok = match && !bad && (zv - Bz) - 1e-15 * (fabs(zv) + Bz + 1.0) >= (double)theta;
    __syncthreads();                               // s_cnt cleared
    const unsigned long long mm = __ballot(match && !bad);
    if (mm) {
      int base = 0;
      if (lane == 0) base = atomicAdd(&s_cnt, __popcll(mm));
      base = __builtin_amdgcn_readfirstlane(base);
      if (match && !bad) {
        const int p = base + lanes_below(mm);
        s_val[p] = zv;
        s_id[p] = e;
      }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) csum += __shfl_xor(csum, m);
    const int nl = __popcll(__ballot(low_ok)), nb = __popcll(__ballot(bad));
    if (lane == 0) {
      S.s_red3[0][wave] = csum;
      S.s_red3[1][wave] = nl;
      S.s_red3[2][wave] = nb;
    }
    __syncthreads();                               // the appends and the per-wave sums
    int tc = 0, tl = 0, tb = 0;
#pragma unroll
    for (int w = 0; w < kWavesSel; ++w) {
      tc += S.s_red3[0][w];
      tl += S.s_red3[1][w];
      tb += S.s_red3[2][w];
    }
    const int found = s_cnt;                       // = min(list_n, kListSlots) when no entry is bad
    if (!(isfinite(xn2) && isfinite(dn2))) {       // non-finite hidden state: no routing
      if (tid < k) {
        oi[tid] = -1;
        og[tid] = NAN;
      }
      if (tid == 0) atomicOr(a.dev_flag, kDevNonFinite);
      return;
    }
    if (theta < INFINITY && tb == 0 && (int)list_n == tc && list_n <= (unsigned)kListSlots && tl >= k) {
      if (tid == 0 && blockIdx.x == 0) atomicAdd(&b.hint->listed_calls, 1u);
      select_tail<ACT>(a, t, found, S, Btr, a.rel, zr, Btg, u8, zt, oi, og);
      return;
    }
    __syncthreads();
    if (tid == 0) s_cnt = 0;
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
  select_tail<ACT>(a, t, nc, S, Btr, a.rel, zr, Btg, u8, zt, oi, og);
}

// The selection of token t from the screen; with the list, block 0 records
// the call's k-th logit (and, when this kernel ends the call, advances the
// hint).
template <int ACT, int CPL>
__device__ __forceinline__ void select_screen_block(const ScreenSelectArgs& b, int t, int32_t* oi, float* og) {
  __shared__ SelectLds S;
  const bool ends = b.advance && blockIdx.x == 0 && threadIdx.x < 64;   // wave-uniform
  HintRead hr{};
  if (ends) hr = hint_read(b.hint, threadIdx.x);
  select_screen_core<ACT, CPL>(b, t, S, oi, og);
  __syncthreads();
  // a verify window's selection kernel has one block per token, and only it
  // reads the token's counter: back to 0 for the next call (every thread
  // has read it before the barrier above)
  if (b.wcount != nullptr && threadIdx.x == 0) b.wcount[t] = 0u;
  if (ends) {
    hr.kth = (float)S.s_kth;
    hint_write(b.hint, hr, threadIdx.x);
  } else if (threadIdx.x == 0 && blockIdx.x == 0) {
    b.hint->kth = (float)S.s_kth;
  }
}

}  // namespace moe
