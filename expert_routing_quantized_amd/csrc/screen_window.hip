// The router's int8 first pass for verify windows (2 <= T <= 8 tokens).
//
// A verify window scores a few drafted tokens against the whole router in one
// call (pyshine source tour, Understanding the Architecture, the paragraph on
// guessing and then checking drafted tokens); its router pass is the same
// stream as at batch 1, read once for all T tokens.  The screen's arithmetic
// (screen.hip) is unchanged -- int8 router rows, the hidden state as two
// int8 digit planes of a 15-bit fixed point per token, exact int32 sums,
// v = fl32(s_e 2^-m (128 HI + LO) + b_e), bounded by B_e -- but with T tokens
// the integer sums form a dense product [16 planes] x [H] x [E] and run on the
// matrix cores: v_mfma_i32_16x16x64_i8 with the 2 T digit planes as the
// 16-row operand and 16 experts' rows as the 16-column operand.  Products
// and sums are exact integers, so the values equal the batch-1 screen's bit
// for bit, whatever the order of accumulation.
//
// The int8 router is stored a second time in the operands' lane order (q8w):
// group G of 16 experts and slab s of 64 hidden positions fill one 1 KB
// block at (G NS + s) 1024, lane L's 16 bytes at 16 L holding expert
// 16 G + (L & 15) at positions 64 s + 16 (L >> 4) + [0, 16) -- the lane and
// byte to reduction-index map of the operands is the same for both, so only
// the row/column lanes matter.  A wave streams a contiguous run of its
// group's blocks (group-major order: 0.2-0.8 us faster than slab-major,
// where all waves ask for neighbouring blocks at once), and its block
// builds the digit planes in LDS in the same order while they arrive.
//
// After the product, lane L holds the exact sums of planes 4 (L >> 4) + r
// (r = 0..3: hi and lo of tokens 2 (L >> 4) and 2 (L >> 4) + 1) for expert
// 16 G + (L & 15), so every value comes out without a cross-lane reduction.
// Per token the kernel also writes the maxima of 4 consecutive values and,
// with a list, recomputes the logits of the experts whose upper end reaches
// the ring's threshold (as at batch 1) into that token's list.
#include "select_screen.h"

namespace moe {

constexpr int kWinWaves = 4;       // groups of 16 experts per block
constexpr int kWinSplit = 2;       // waves per group (each streams a part of the slabs)
// Slabs each wave keeps in flight (a ring; the next slab's load is issued as
// each product is taken).  Measured on the 24,576-expert router, screen
// alone, T = 2 / 5 / 8: 4 slabs 11.5 / 13.0 / 15.2 us, 2 slabs 12.4 / 14.4 /
// 16.5, 8 slabs 12.3 / 12.8 / 15.6, all 16 slabs of the wave 12.1 / 14.0 /
// 16.5; one wave per group with all 32 slabs in flight 11.6 / 13.2 / 15.2.
constexpr int kWinSlabsInFlight = 4;
constexpr int kWinMaxH = 2048;     // 32 slabs of 64: the whole group in flight in 128 VGPRs

bool screen_window_fits(const moe_layer_desc& d) {
  return d.hidden <= kWinMaxH && d.max_tokens >= 2 && !(d.flags & MOE_LAYER_WINDOW_SCREEN_OFF);
}

static int win_slabs(int H) { return H <= 512 ? 8 : (H <= 1024 ? 16 : 32); }
static int win_groups(int E) { return (E + 15) / 16; }

size_t screen_window_bytes(const moe_layer_desc& d) {
  return size_t(win_groups(d.n_experts)) * win_slabs(d.hidden) * 1024;
}

int screen_window_waves(const Layer& L) { return win_groups(L.d.n_experts); }
int screen_window_cstride(const Layer& L) { return (win_groups(L.d.n_experts) + 15) / 16 * 16; }

// ------------------------------------------------------------------ layout
// One thread per 16-byte operand chunk (zero past E and past H: H is a
// multiple of 32, so a chunk lies wholly inside or outside the row).
__global__ __launch_bounds__(256) void screen_swizzle_kernel(const int8_t* __restrict__ q8, int H, int E, int ngroups,
                                                             size_t nchunks, int8_t* __restrict__ q8w) {
  const size_t c = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (c >= nchunks) return;
  const int L = int(c & 63);
  const size_t sg = c >> 6;                          // block G NS + s
  const int NS = int(nchunks / 64 / size_t(ngroups));
  const int G = int(sg / size_t(NS));
  const int s = int(sg % size_t(NS));
  const int e = 16 * G + (L & 15);
  const int h0 = 64 * s + 16 * (L >> 4);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (e < E && h0 < H) v = *reinterpret_cast<const uint4*>(q8 + size_t(e) * H + h0);
  reinterpret_cast<uint4*>(q8w)[c] = v;
}

hipError_t launch_screen_window_prep(const Layer& L, hipStream_t s) {
  const int NS = win_slabs(L.d.hidden);
  const size_t n = size_t(win_groups(L.d.n_experts)) * NS * 64;
  hipLaunchKernelGGL(screen_swizzle_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, L.q8, L.d.hidden,
                     L.d.n_experts, win_groups(L.d.n_experts), n, L.q8w);
  return hipGetLastError();
}

// ------------------------------------------------------------------ screen
__device__ __forceinline__ uint32_t win_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

struct WinScreenArgs {
  const int8_t* q8w;      // operand-order int8 router
  const float* sc8;       // [E]
  const float* bias;      // [E], never null
  const float2* eb8;      // [E]
  const uint16_t* x;      // [T][H] bf16
  const uint16_t* R;      // [E][H] bf16 router (the listed rows' recompute)
  int H, E, T, ngroups;
  float* z8;              // [T][E]
  float* g8;              // [T][ceil(E/4)]
  double* xq;             // [T][2]: ||x||^2, ||delta||^2
  int* dev_flag;
  double u8, babs8, rqmax;   // the bound's terms, as at batch 1
  const HintWords* hsrc;  // never null: the call's hint, or a readable stand-in
  int listing;            // lists wanted (then hsrc is the hint)
  unsigned int* wcount;   // [kWinMaxT] the lists' counters (in the hint)
  unsigned char* wcnt;    // [T][cstride]
  ulonglong2* wlist;      // [T][kListSlots]
  int cstride;
};

// Block: kWinWaves groups of 16 experts, each split over kWinSplit waves by
// slab range (wave w: group w % kWinWaves, slabs of part w / kWinWaves), so
// each wave streams NS / kWinSplit blocks and the block's digit work is
// spread over kWinWaves * kWinSplit waves; the parts' integer sums are added
// in LDS (exactly) by the first part's waves, which finish the group.
template <int NS, int CPL, int NBUF>
__global__ __launch_bounds__(kWinWaves * kWinSplit * 64, 4) void screen_window_kernel(WinScreenArgs a) {
  kernarg_lines<sizeof(WinScreenArgs)>();
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  constexpr int NT = kWinWaves * kWinSplit * 64;     // threads
  constexpr int NWV = kWinWaves * kWinSplit;         // waves
  constexpr int NSP = NS / kWinSplit;                // slabs per wave
  constexpr int EPT = (NS * 64 / NT) < 2 ? 2 : NS * 64 / NT;   // elements of a padded row per thread (per token)
  static_assert((EPT == 2 || EPT == 4) && NT * EPT >= NS * 64, "2 or 4 elements per thread cover the row");
  __shared__ __attribute__((aligned(16))) unsigned char s_dig[NS * 1024];   // digit planes, operand order
  __shared__ __attribute__((aligned(16))) uint16_t s_x[kWinMaxT][NT * EPT];  // the tokens' x (zero past H, T)
  __shared__ i32x4 s_acc[kWinSplit - 1][kWinWaves][64];                     // the other parts' sums
  __shared__ uint32_t s_mb[NWV][kWinMaxT];
  __shared__ int s_m[kWinMaxT];                                             // per token: m, or INT_MIN if bad
  __shared__ double s_red[NWV][kWinMaxT][3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = wave % kWinWaves, part = wave / kWinWaves;
  const int H = a.H, E = a.E, T = a.T;
  const int Gw = blockIdx.x * kWinWaves + q;         // this wave's group of 16 experts
  const int G = min(Gw, a.ngroups - 1);              // (waves past the last group compute it and discard it)
  // 1. the tokens' x first (EPT elements c * EPT .. of every token, zero
  //    past H and past T; every load unconditional, at clamped addresses):
  //    loads complete in order, so the digits are worked out while the
  //    slabs stream; then the wave's slabs, all in flight
  const int c = tid;                                 // element group of the padded row
  const bool cin = c * EPT < H;                      // H is a multiple of 32
  typedef uint32_t xw_t __attribute__((ext_vector_type(EPT / 2)));
  xw_t xr[kWinMaxT];
#pragma unroll
  for (int t = 0; t < kWinMaxT; ++t)
    xr[t] = *reinterpret_cast<const xw_t*>(a.x + size_t(min(t, T - 1)) * H + min(c * EPT, H - EPT));
  constexpr int NB = NBUF < NSP ? NBUF : NSP;      // slabs in flight per wave
  const i32x4* qsrc = reinterpret_cast<const i32x4*>(a.q8w) + (size_t(G) * NS + part * NSP) * 64 + lane;
  const size_t qstride = 64;
  i32x4 bq[NB];
#pragma unroll
  for (int s = 0; s < NB; ++s) bq[s] = __builtin_nontemporal_load(qsrc + s * qstride);
  const int jl = lane & 15, gl = lane >> 4;          // expert column, plane quad
  const int e = 16 * G + jl, ec = min(e, E - 1);
  const float my_sc = a.sc8[ec], my_b = a.bias[ec], my_eb = a.eb8[ec].x;
  const float ring_v = a.hsrc->ring[lane & (kHintRing - 1)];   // read whether or not it is used
  // max |x_t| on the magnitude bits (a non-finite element has bits >= 0x7f80);
  // x into LDS (its registers are free from here on)
#pragma unroll
  for (int t = 0; t < kWinMaxT; ++t) {
    uint32_t mb = 0u;
    xw_t xv;
#pragma unroll
    for (int w = 0; w < EPT / 2; ++w) {
      xv[w] = (t < T && cin) ? xr[t][w] : 0u;
      mb = max(mb, max(xv[w] & 0x7fffu, (xv[w] >> 16) & 0x7fffu));
    }
    *reinterpret_cast<xw_t*>(&s_x[t][c * EPT]) = xv;
    mb = win_max_u32(mb);
    if (lane == 0) s_mb[wave][t] = mb;
  }
  __syncthreads();
  // 2. per token: the fixed point's exponent m (|x 2^m| < 2^13, as at batch
  //    1), digits into LDS in operand order (plane 2t: hi, 2t + 1: lo), the
  //    exact sum of X^2, and in block 0 the binary64 sums of x^2 and
  //    delta^2.  The planes of tokens past T are left as they are: their
  //    sums are never used.
  const int h0 = c * EPT;
  const int doff = (h0 >> 6) * 1024 + 16 * 16 * ((h0 & 63) >> 4) + (h0 & 15);
#pragma unroll
  for (int t = 0; t < kWinMaxT; ++t) {
    if (t >= T) continue;                              // uniform
    uint32_t mb = s_mb[0][t];
#pragma unroll
    for (int w = 1; w < NWV; ++w) mb = max(mb, s_mb[w][t]);
    const bool bad = mb >= 0x7f80u;
    const float mx = __uint_as_float(mb << 16);
    int m = 0;
    if (mx > 0.f && !bad) {
      int ex;
      frexpf(mx, &ex);
      m = 13 - ex;
    }
    if (tid == 0) s_m[t] = bad ? INT_MIN : m;
    const int m1 = m > 100 ? 100 : (m < -100 ? -100 : m);
    const float sc1 = ldexpf(1.f, m1), sc2 = ldexpf(1.f, m - m1);
    const double isc = ldexp(1.0, -m);
    const xw_t xv = *reinterpret_cast<const xw_t*>(&s_x[t][c * EPT]);
    double pxx = 0.0, pdd = 0.0;
    int x2 = 0;
    uint32_t hw = 0u, lw = 0u;
#pragma unroll
    for (int el = 0; el < EPT; ++el) {
      const uint32_t word = xv[el >> 1];
      const float v = bad ? 0.f : ((el & 1) ? bf16_hi(word) : bf16_lo(word));
      const int Xi = (int)rintf((v * sc1) * sc2);             // |Xi| <= 2^13
      hw |= (uint32_t(Xi >> 7) & 0xffu) << (8 * el);
      lw |= uint32_t(Xi & 127) << (8 * el);
      x2 += Xi * Xi;                                          // <= 4 * 2^26: exact
      if (blockIdx.x == 0) {                                  // uniform
        const double d = (double)v - (double)Xi * isc;        // exact
        pxx = fma((double)v, (double)v, pxx);
        pdd = fma(d, d, pdd);
      }
    }
    if (c * EPT < NS * 64) {
      if constexpr (EPT == 4) {
        *reinterpret_cast<uint32_t*>(s_dig + doff + 16 * (2 * t)) = hw;
        *reinterpret_cast<uint32_t*>(s_dig + doff + 16 * (2 * t + 1)) = lw;
      } else {
        *reinterpret_cast<uint16_t*>(s_dig + doff + 16 * (2 * t)) = (uint16_t)hw;
        *reinterpret_cast<uint16_t*>(s_dig + doff + 16 * (2 * t + 1)) = (uint16_t)lw;
      }
    }
    const double sx = wave_sum_f64((double)x2);        // exact: integers below 2^53
    double sxx = 0.0, sdd = 0.0;
    if (blockIdx.x == 0) {                             // uniform
      sxx = wave_sum_f64(pxx);
      sdd = wave_sum_f64(pdd);
    }
    if (lane == 0) {
      s_red[wave][t][0] = sx;
      s_red[wave][t][1] = sxx;
      s_red[wave][t][2] = sdd;
    }
  }
  __syncthreads();
  if (blockIdx.x == 0 && tid < T) {
    double sxx = 0.0, sdd = 0.0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      sxx += s_red[w][tid][1];
      sdd += s_red[w][tid][2];
    }
    const bool xb = s_m[tid] == INT_MIN;
    a.xq[2 * tid] = xb ? NAN : sxx;
    a.xq[2 * tid + 1] = xb ? NAN : sdd;
    if (xb) atomicOr(a.dev_flag, kDevNonFinite);
  }
  // 3. the product: 16 planes by 16 experts over the wave's slabs; the
  //    other parts hand their sums to the first part's wave of the group
  i32x4 acc = {0, 0, 0, 0};
#pragma unroll
  for (int s = 0; s < NSP; ++s) {
    const i32x4 av = *reinterpret_cast<const i32x4*>(s_dig + (part * NSP + s) * 1024 + 16 * lane);
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bq[s % NB], acc, 0, 0, 0);
    if (s + NB < NSP) {
      __builtin_amdgcn_sched_barrier(0);             // the next slab's load after this product
      bq[s % NB] = __builtin_nontemporal_load(qsrc + (s + NB) * qstride);
    }
  }
  if (part > 0) s_acc[part - 1][q][lane] = acc;
  __syncthreads();
  if (part > 0) return;                              // uniform per wave
#pragma unroll
  for (int p = 0; p < kWinSplit - 1; ++p) acc += s_acc[p][q][lane];   // exact int32 sums
  // 4. values of tokens 2 gl and 2 gl + 1 for expert e, their maxima of 4,
  //    and whether the list takes them
  const int G4 = (E + 3) / 4;
  const float theta = a.listing ? hint_threshold_lanes(ring_v) : INFINITY;
  const float rqmaxf = (float)a.rqmax * (1.f + 0x1p-20f), u8f = (float)a.u8 * (1.f + 0x1p-20f);
  const float babs8f = (float)a.babs8 * (1.f + 0x1p-20f) + 0x1p-149f;
  const float hd = 0.5f * sqrtf((float)H) * (1.f + 0x1p-20f);
  bool lst[2];
  bool nonfin = false;
#pragma unroll
  for (int r2 = 0; r2 < 2; ++r2) {
    const int t = 2 * gl + r2;                       // lane-dependent
    const int mraw = (t < T) ? s_m[t] : 0;
    const bool xb = mraw == INT_MIN;
    const int m = xb ? 0 : mraw;
    double x2 = 0.0;
    if (t < T) {
#pragma unroll
      for (int w = 0; w < NWV; ++w) x2 += s_red[w][t][0];
    }
    const double D = 128.0 * (double)acc[2 * r2] + (double)acc[2 * r2 + 1];   // exact
    const double v = (double)my_sc * D * ldexp(1.0, -m) + (double)my_b;
    const float vf = xb ? NAN : (float)v;
    const bool in = t < T && e < E;
    if (in) a.z8[size_t(t) * E + e] = vf;
    nonfin = nonfin || (in && !xb && !isfinite(vf));
    float gm = (in && !isnan(vf)) ? vf : -INFINITY;
    gm = fmaxf(gm, MOE_DPP_F32(gm, 0xB1, 0xf));      // quads of lanes: 4 consecutive experts
    gm = fmaxf(gm, MOE_DPP_F32(gm, 0x4E, 0xf));
    if (in && (jl & 3) == 0) a.g8[size_t(t) * G4 + (e >> 2)] = gm;
    // the upper end v + B against theta, in binary32 rounded up (as at batch 1)
    const float X2 = (float)x2 * (1.f + 0x1p-20f);
    const float iscf = ldexpf(1.f, -m);
    const float xnu = ((sqrtf(X2) * (1.f + 0x1p-20f) + hd) * (1.f + 0x1p-20f)) * iscf * (1.f + 0x1p-20f) + 0x1p-149f;
    const float dnu = hd * iscf * (1.f + 0x1p-20f) + 0x1p-149f;
    const float B = fmaf(xnu, my_eb, fmaf(dnu, rqmaxf, fmaf(u8f, fabsf(vf), babs8f))) * (1.f + 0x1p-20f) + 0x1p-147f;
    const float U = vf + B;
    lst[r2] = in && isfinite(vf) && U + fabsf(U) * 0x1p-22f + 0x1p-149f >= theta;
  }
  if (__ballot(nonfin) != 0ull && lane == 0) atomicOr(a.dev_flag, kDevNonFinite);
  if (!a.listing || Gw >= a.ngroups) return;          // uniform
  // 5. the lists: per token, the wave's count and (one atomic add) its slots;
  //    each listed expert's row is read once and dotted with every token
  //    that lists it
  const int n8 = H >> 3;
  const unsigned long long m0 = __ballot(lst[0]), m1 = __ballot(lst[1]);
  uint32_t tm[kWinMaxT];
  uint32_t any = 0u;
#pragma unroll
  for (int t = 0; t < kWinMaxT; ++t) {
    tm[t] = (t < T) ? uint32_t((((t & 1) ? m1 : m0) >> (16 * (t >> 1))) & 0xffffull) : 0u;
    any |= tm[t];
  }
  if (lane < T) {
    uint32_t mine = 0u;
#pragma unroll
    for (int t = 0; t < kWinMaxT; ++t) mine = (t == lane) ? tm[t] : mine;
    a.wcnt[size_t(lane) * a.cstride + Gw] = (unsigned char)__popc(mine);
  }
  if (any == 0u) return;
  // (the slots come back while the first row loads: lane t holds token t's first slot)
  unsigned mine = 0u;
  {
    uint32_t cnt = 0u;
#pragma unroll
    for (int t = 0; t < kWinMaxT; ++t) cnt = (t == lane) ? tm[t] : cnt;
    if (lane < T && cnt != 0u) mine = atomicAdd(&a.wcount[lane], (unsigned)__popc(cnt));
  }
  unsigned used[kWinMaxT];
#pragma unroll
  for (int t = 0; t < kWinMaxT; ++t) used[t] = 0u;
  for (uint32_t mj = any; mj != 0u; mj &= mj - 1u) {   // one row at a time (registers)
    const int j = __builtin_ctz(mj);
    const int er = 16 * G + j;
    uint4 rr[CPL];
#pragma unroll
    for (int s = 0; s < CPL; ++s)
      rr[s] = *reinterpret_cast<const uint4*>(a.R + size_t(er) * H + min(s * 64 + lane, n8 - 1) * 8);
    const float br = a.bias[er];
#pragma unroll
    for (int t = 0; t < kWinMaxT; ++t) {
      if (!((tm[t] >> j) & 1u)) continue;            // uniform
      uint4 xc[CPL];
#pragma unroll
      for (int s = 0; s < CPL; ++s)
        xc[s] = *reinterpret_cast<const uint4*>(a.x + size_t(t) * H + min(s * 64 + lane, n8 - 1) * 8);
      const double z = dot2_logit<CPL>(xc, rr, n8, br, lane);
      const unsigned slot = (unsigned)__builtin_amdgcn_readlane((int)mine, t) + used[t];
      if (lane == 0 && slot < (unsigned)kListSlots)      // a full list: the selection falls back
        a.wlist[size_t(t) * kListSlots + slot] =
            make_ulonglong2((unsigned long long)er, (unsigned long long)__double_as_longlong(z));
      ++used[t];
    }
  }
}

hipError_t launch_screen_window(const Layer& L, const void* x, int T, float* z8, float* g8, double* xq,
                                const WinList* list, hipStream_t s) {
  if (!L.screen_win || T < 2 || T > kWinMaxT) return hipErrorInvalidValue;
  WinScreenArgs a{};
  a.q8w = L.q8w;
  a.sc8 = L.sc8;
  a.bias = router_bias_or_zero(L);
  a.eb8 = L.eb8;
  a.x = reinterpret_cast<const uint16_t*>(x);
  a.R = reinterpret_cast<const uint16_t*>(L.router_eh);
  a.H = L.d.hidden;
  a.E = L.d.n_experts;
  a.T = T;
  a.ngroups = win_groups(a.E);
  a.z8 = z8;
  a.g8 = g8;
  a.xq = xq;
  a.dev_flag = L.dev_flag;
  const ScreenSelectArgs b = make_screen_select_args(L, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
  a.u8 = b.u8;
  a.babs8 = b.babs8;
  a.rqmax = b.rqmax;
  a.hsrc = reinterpret_cast<const HintWords*>(L.screen_consts);   // 256 bytes, read and ignored
  if (list != nullptr) {
    a.hsrc = list->hint;
    a.listing = 1;
    a.wcount = list->hint->win_count;
    a.wcnt = list->wcnt;
    a.wlist = list->wlist;
    a.cstride = screen_window_cstride(L);
  }
  const dim3 grid((a.ngroups + kWinWaves - 1) / kWinWaves);
  constexpr int NT = kWinWaves * kWinSplit * 64;
  switch (win_slabs(a.H)) {
    case 8: hipLaunchKernelGGL((screen_window_kernel<8, 1, kWinSlabsInFlight>), grid, dim3(NT), 0, s, a); break;
    case 16: hipLaunchKernelGGL((screen_window_kernel<16, 2, kWinSlabsInFlight>), grid, dim3(NT), 0, s, a); break;
    default:   // H = 2048: windows of 4-6 tokens keep twice the slabs in flight (0.4-0.7 us faster there,
               // slower at 8 tokens, no change at 2-3)
      if (a.T >= 4 && a.T <= 6)
        hipLaunchKernelGGL((screen_window_kernel<32, 4, 2 * kWinSlabsInFlight>), grid, dim3(NT), 0, s, a);
      else
        hipLaunchKernelGGL((screen_window_kernel<32, 4, kWinSlabsInFlight>), grid, dim3(NT), 0, s, a);
      break;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ select
template <int ACT, int CPL>
__global__ __launch_bounds__(kSelectThreads) void select_screen_window_kernel(ScreenSelectArgs b) {
  kernarg_lines<sizeof(ScreenSelectArgs)>();
  const int t = blockIdx.x;
  select_screen_block<ACT, CPL>(b, t, b.sel.idx + size_t(t) * b.sel.k, b.sel.gates + size_t(t) * b.sel.k);
}

hipError_t launch_select_screen_window(const Layer& L, const void* x, int T, const float* z8, const float* g8,
                                       const double* xq, const WinList* list, int32_t* idx, float* gates,
                                       hipStream_t s) {
  if (list == nullptr || T < 2 || T > kWinMaxT) return hipErrorInvalidValue;
  ScreenSelectArgs b = make_screen_select_args(L, x, z8, g8, xq, idx, gates);
  b.hint = list->hint;
  b.cnt8 = list->wcnt;
  b.list = list->wlist;
  b.nw = screen_window_waves(L);
  b.advance = 1;                      // block 0 advances the ring; block t clears its counter
  b.wcount = list->hint->win_count;
  b.cstride = screen_window_cstride(L);
  const int cpl = (L.d.hidden / 8 + 63) / 64;
  if (cpl <= 1) hipLaunchKernelGGL((select_screen_window_kernel<MOE_BF16, 1>), dim3(T), dim3(kSelectThreads), 0, s, b);
  else if (cpl <= 2) hipLaunchKernelGGL((select_screen_window_kernel<MOE_BF16, 2>), dim3(T), dim3(kSelectThreads), 0, s, b);
  else hipLaunchKernelGGL((select_screen_window_kernel<MOE_BF16, 4>), dim3(T), dim3(kSelectThreads), 0, s, b);
  return hipGetLastError();
}

}  // namespace moe
