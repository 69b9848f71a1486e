// Expert GEMVs of one token: h_j = silu(G_e x) * (U_e x) for the k selected
// experts, then out = sum_j g_j D_e h_j.
//
// The pages compute the cached experts with a hand-written GEMV whose speed
// is set by memory bandwidth; their tensor-core variant lost on every real
// shape because a single token fills one row of a 16-row tile (hexlives
// dispatch, paragraph on the archived tensor-core benchmark).  So these are vector-ALU GEMVs: every weight byte is loaded
// once with 16-byte loads, the 4-bit codes are expanded in registers and the
// fp16 block scale is applied to each 32-element partial in fp32 (exact
// dequantisation, nothing rounded to 16 bits).  The router weight is applied
// only in the down/combine kernel (pyshine source tour, Understanding the
// Architecture, paragraph on the expert hand-off).
//
// The same kernels serve a few tokens at once (verify windows): with T
// tokens there are P = T k token-expert pairs.  Short windows compute every
// pair on its own (INDEP); longer ones let the block that holds the first
// pair naming an expert compute every pair of that expert, so the expert's
// weights are read once per call and no sort is needed.
//
// gate/up: one wave per pair of intermediate rows (gate row i and up row i
// of the same expert), so silu(a)*u is formed in registers; for 4-bit rows
// lane l owns quant block l (32 elements = 16 B of codes + one scale).
// down:    8 lanes per output row, one wave per distinct expert, per-pair
// partials in LDS, each token summed over its pairs in selection order.
#include "moe_internal.h"
#include "select_block.h"
#include "select_screen.h"

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

// One lane's part of a 4-bit down row times h: quant block (codes w, scale d)
// against the 32 values of h at hq.
__device__ __forceinline__ float down_lane_partial_q4(const uint4 w, float d, const float* hq) {
  float hv[32];
#pragma unroll
  for (int i = 0; i < 32; i += 4) {
    const float4 v4 = *reinterpret_cast<const float4*>(hq + i);
    hv[i] = v4.x; hv[i + 1] = v4.y; hv[i + 2] = v4.z; hv[i + 3] = v4.w;
  }
  float hs = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) hs += hv[i];
  return d * (q4_block_dot(w, hv) - 8.f * hs);
}

struct PairArgs {
  const void* x;     // [T][H]
  const int32_t* idx;
  const float* gates;
  const void *wg, *wu, *wd;
  const uint16_t *sg, *su, *sd;
  float* h;          // [P][I]
  float* out;        // [T][H]
  int H, I, E, k, T, P;
  int* dev_flag;
  HintWords* hint;   // batch-1 screen list: the down kernel advances it (block 0), else null
  const ExpertTiers* tiers;   // the layer's hot-expert region (device memory), else null
};

// Where expert e's weights are read: the hot region's copy when the layer
// has one that holds e (e then becomes its slot there), else the pool.  With
// no region this is a uniform branch and no load.
struct PoolView {
  const void *wg, *wu, *wd;
  const uint16_t *sg, *su, *sd;
};
__device__ __forceinline__ PoolView pool_view(const PairArgs& a, int& e) {
  PoolView v{a.wg, a.wu, a.wd, a.sg, a.su, a.sd};
  if (a.tiers != nullptr) {
    const ExpertTiers* t = a.tiers;
    const int slot = t->loc[e];
    if (slot >= 0) {
      v = PoolView{t->wg, t->wu, t->wd, t->sg, t->su, t->sd};
      e = slot;
    }
  }
  return v;
}

// Expert of pair p if pair p is the first pair naming it (else -1): the
// block that owns the first occurrence computes every pair of that expert,
// so each selected expert's weights are read once per call.  All threads
// of the block take part; the matching pairs (in any order: each pair's
// result depends on its own token only) are appended to s_match.
__device__ __forceinline__ int claim_pairs(const PairArgs& a, int p, int* s_match, int* s_n) {
  const int e = a.idx[p];
  const bool valid = e >= 0 && e < a.E;
  if (threadIdx.x == 0) *s_n = 0;
  __syncthreads();
  bool earlier = false;
  for (int q = threadIdx.x; q < a.P; q += blockDim.x) {
    if (a.idx[q] == e && valid) {
      if (q < p) earlier = true;
      else s_match[atomicAdd(s_n, 1)] = q;
    }
  }
  if (__syncthreads_or(earlier) || !valid) return -1;
  return e;
}

// ------------------------------------------------------------ gate/up, 4-bit
// MB = quant blocks per lane (H / 32 / 64 rounded up).
// Independent pairs stage the token's x once per block in LDS (each quant
// block's 16-byte chunks padded by one chunk, so a wave's reads of one
// chunk column hit distinct banks), instead of every wave reading the whole
// row from L2: at batch 1 the x reads were more bytes than the weights.
template <int ACT>
struct XStage {
  static constexpr int kChunks = (ACT == MOE_BF16) ? 4 : 8;   // 16-byte chunks per quant block
  static constexpr int kPitch = kChunks + 1;
};

template <int ACT, int MB, bool INDEP, int RPW = 2>   // RPW: intermediate rows per wave
__global__ __launch_bounds__(256) void gateup_q4_kernel(PairArgs a) {
  __shared__ int s_match[kMaxPairs];
  __shared__ int s_n;
  __shared__ uint4 sx[INDEP ? (kMaxH / 32) * XStage<ACT>::kPitch : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int e;
  bool valid = true;
  if constexpr (INDEP) {           // independent pairs: every pair is its own group
    e = a.idx[blockIdx.y];
    valid = e >= 0 && e < a.E;
    e = valid ? e : 0;             // addresses stay in range; h becomes NaN
  } else {
    e = claim_pairs(a, blockIdx.y, s_match, &s_n);
    if (e < 0) return;
  }
  const int nblk = a.H >> 5;
  constexpr int kRowsPerWave = RPW;
  const int i0 = (blockIdx.x * 4 + wave) * kRowsPerWave;
  const size_t rowb = size_t(a.H) / 2;
  const PoolView pv = pool_view(a, e);
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
      const size_t row = size_t(e) * a.I + i;
      wg[r][m] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(pv.wg) + row * rowb + b * 16);
      wu[r][m] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(pv.wu) + row * rowb + b * 16);
      dg[r][m] = f16_to_f32(pv.sg[row * nblk + b]);
      du[r][m] = f16_to_f32(pv.su[row * nblk + b]);
    }
  }
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
    for (int m = 0; m < MB; ++m)
      if (!(i0 + r < a.I && m * 64 + lane < nblk)) dg[r][m] = du[r][m] = 0.f;
  if constexpr (INDEP) {           // x of the pair's token into LDS, while the weights load
    constexpr int CK = XStage<ACT>::kChunks, PK = XStage<ACT>::kPitch;
    const int nc = nblk * CK;
    const uint4* xs = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(a.x) +
                                                     size_t(blockIdx.y / a.k) * a.H * (ACT == MOE_BF16 ? 2 : 4));
    constexpr int NU = (64 * MB * CK + 255) / 256;   // chunks per thread (nblk <= 64 MB)
    uint4 xr[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int c = threadIdx.x + 256 * u;
      xr[u] = xs[min(c, nc - 1)];
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int c = threadIdx.x + 256 * u;
      if (c < nc) sx[(c / CK) * PK + c % CK] = xr[u];
    }
    __syncthreads();
  }
  const int n = INDEP ? 1 : s_n;
  for (int mi = 0; mi < n; ++mi) {
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        opaque_reg(wg[r][m]);
        opaque_reg(wu[r][m]);
      }
    const int q = INDEP ? (int)blockIdx.y : s_match[mi];
    const size_t xoff = size_t(q / a.k) * a.H;
    float xv[MB][32];
    float xs[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int b = m * 64 + lane;
      xs[m] = 0.f;
      Chunk<ACT> ch[4];
      if constexpr (INDEP) {
        constexpr int PK = XStage<ACT>::kPitch;
        const uint4* sb = sx + min(b, nblk - 1) * PK;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if constexpr (ACT == MOE_BF16) {
            ch[c].v = sb[c];
          } else {
            const uint4 p0 = sb[2 * c], p1 = sb[2 * c + 1];
            ch[c].a = make_float4(__uint_as_float(p0.x), __uint_as_float(p0.y), __uint_as_float(p0.z), __uint_as_float(p0.w));
            ch[c].b = make_float4(__uint_as_float(p1.x), __uint_as_float(p1.y), __uint_as_float(p1.z), __uint_as_float(p1.w));
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) ch[c].load(a.x, xoff + min(b, nblk - 1) * 32 + c * 8);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) xv[m][c * 8 + i] = (b < nblk) ? ch[c].get(i) : 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) xs[m] += xv[m][i];
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
      if (lane == 0 && i < a.I) a.h[size_t(q) * a.I + i] = valid ? silu_f(av) * uv : NAN;
    }
  }
}

// ------------------------------------------------------ decode: select + gate/up
// Decode and short verify windows (T <= 8 tokens) with 4-bit experts: the
// selection and the gate/up projections in one launch.  Block b serves pair
// p = b / bpp (token t = p / k, rank j = p % k): it runs the certified
// selection of token t on its own (select_block: the order depends only on
// the logits and the expert indices, so every block of the token reaches
// the same one) and then computes kDecodeRowsPerBlock intermediate rows of
// the token's rank-j expert, with the same per-row arithmetic as
// gateup_q4_kernel.  There is then no launch gap and no dependent index
// load between the selection and the weight stream; the redundant
// selections read the group maxima from L2.  The first block of each token
// publishes its idx and gates for the down projection.
constexpr int kDecodeRowsPerWave = 2;
constexpr int kDecodeRowsPerBlock = kDecodeRowsPerWave * (kSelectThreads / 64);

// SCREEN: the selection runs on the router's int8 screen (select_screen_block,
// T = 1; CPLR = 8-element chunks per lane of a router row), else on the
// full router logits (select_block).
template <int ACT, int CPLR, bool SCREEN>
__device__ __forceinline__ void select_policy(const ScreenSelectArgs& sb, int t, int32_t* oi, float* og) {
  if constexpr (SCREEN) select_screen_block<ACT, CPLR>(sb, t, oi, og);
  else select_block<ACT>(sb.sel, t, oi, og);
}

template <int ACT, int MB, int CPLR, bool SCREEN>
__global__ __launch_bounds__(kSelectThreads) void select_gateup_q4_kernel(ScreenSelectArgs sb, PairArgs a) {
  kernarg_lines<sizeof(ScreenSelectArgs) + sizeof(PairArgs)>();
  const SelectArgs& sa = sb.sel;
  constexpr int RPW = kDecodeRowsPerWave;
  constexpr int CK = XStage<ACT>::kChunks, PK = XStage<ACT>::kPitch;
  __shared__ uint4 sx[(kMaxH / 32) * PK];
  __shared__ int32_t s_idx[kMaxK];
  __shared__ float s_gate[kMaxK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nblk = a.H >> 5;
  const int bpp = (a.I + kDecodeRowsPerBlock - 1) / kDecodeRowsPerBlock;   // blocks per pair
  const int p = blockIdx.x / bpp, t = p / a.k, j = p - t * a.k;
  // the token's x: loaded first, stored to LDS once the selection is done
  // (a store here would wait for the load before the selection's own loads)
  const int nc = nblk * CK;
  constexpr int NU = (64 * MB * CK + kSelectThreads - 1) / kSelectThreads;
  uint4 xr[NU];
  {
    const uint4* xs = reinterpret_cast<const uint4*>(a.x) + size_t(t) * nc;
#pragma unroll
    for (int u = 0; u < NU; ++u) xr[u] = xs[min(tid + kSelectThreads * u, nc - 1)];
  }
  select_policy<ACT, CPLR, SCREEN>(sb, t, s_idx, s_gate);
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int c = tid + kSelectThreads * u;
    if (c < nc) sx[(c / CK) * PK + c % CK] = xr[u];
  }
  __syncthreads();
  if (j == 0 && blockIdx.x == p * bpp && tid < a.k) {   // first block of the token
    sa.idx[size_t(t) * a.k + tid] = s_idx[tid];
    sa.gates[size_t(t) * a.k + tid] = s_gate[tid];
  }
  const int i0 = (blockIdx.x - p * bpp) * kDecodeRowsPerBlock + wave * RPW;
  int e = s_idx[j];
  const bool valid = e >= 0 && e < a.E;
  e = valid ? e : 0;                                   // addresses stay in range; h becomes NaN
  const size_t rowb = size_t(a.H) / 2;
  uint4 wg[RPW][MB], wu[RPW][MB];
  float dg[RPW][MB], du[RPW][MB];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int i = min(i0 + r, a.I - 1);
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int b = min(m * 64 + lane, nblk - 1);
      const size_t row = size_t(e) * a.I + i;
      wg[r][m] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.wg) + row * rowb + b * 16);
      wu[r][m] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.wu) + row * rowb + b * 16);
      dg[r][m] = f16_to_f32(a.sg[row * nblk + b]);
      du[r][m] = f16_to_f32(a.su[row * nblk + b]);
    }
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int m = 0; m < MB; ++m)
      if (!(i0 + r < a.I && m * 64 + lane < nblk)) dg[r][m] = du[r][m] = 0.f;
  float xv[MB][32];
  float xsum[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int b = m * 64 + lane;
    xsum[m] = 0.f;
    Chunk<ACT> ch[4];
    const uint4* sb = sx + min(b, nblk - 1) * PK;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if constexpr (ACT == MOE_BF16) {
        ch[c].v = sb[c];
      } else {
        const uint4 p0 = sb[2 * c], p1 = sb[2 * c + 1];
        ch[c].a = make_float4(__uint_as_float(p0.x), __uint_as_float(p0.y), __uint_as_float(p0.z), __uint_as_float(p0.w));
        ch[c].b = make_float4(__uint_as_float(p1.x), __uint_as_float(p1.y), __uint_as_float(p1.z), __uint_as_float(p1.w));
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[m][c * 8 + i] = (b < nblk) ? ch[c].get(i) : 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) xsum[m] += xv[m][i];
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    float pa = 0.f, pu = 0.f;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      pa = fmaf(dg[r][m], q4_block_dot(wg[r][m], xv[m]) - 8.f * xsum[m], pa);
      pu = fmaf(du[r][m], q4_block_dot(wu[r][m], xv[m]) - 8.f * xsum[m], pu);
    }
    const float av = wave_sum(pa), uv = wave_sum(pu);
    const int i = i0 + r;
    if (lane == 0 && i < a.I) a.h[size_t(p) * a.I + i] = valid ? silu_f(av) * uv : NAN;
  }
}

// ------------------------------------------------------------ gate/up, dense
template <int ACT, int WD, int CPL, bool INDEP>
__global__ __launch_bounds__(256) void gateup_dense_kernel(PairArgs a) {
  __shared__ int s_match[kMaxPairs];
  __shared__ int s_n;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int e;
  bool valid = true;
  if constexpr (INDEP) {
    e = a.idx[blockIdx.y];
    valid = e >= 0 && e < a.E;
    e = valid ? e : 0;
  } else {
    e = claim_pairs(a, blockIdx.y, s_match, &s_n);
    if (e < 0) return;
  }
  const int nch = a.H >> 3;
  constexpr int kRowsPerWave = 2;
  const int i0 = (blockIdx.x * 4 + wave) * kRowsPerWave;
  const PoolView pv = pool_view(a, e);
  Chunk<WD> wg[kRowsPerWave][CPL], wu[kRowsPerWave][CPL];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const size_t row = size_t(e) * a.I + min(i0 + r, a.I - 1);
#pragma unroll
    for (int s = 0; s < CPL; ++s) {
      const int c = min(s * 64 + lane, nch - 1);
      wg[r][s].load(pv.wg, row * a.H + c * 8);
      wu[r][s].load(pv.wu, row * a.H + c * 8);
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
  const int n = INDEP ? 1 : s_n;
  for (int mi = 0; mi < n; ++mi) {
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
      for (int s = 0; s < CPL; ++s) {
        wg[r][s].opaque();
        wu[r][s].opaque();
      }
    const int q = INDEP ? (int)blockIdx.y : s_match[mi];
    const size_t xoff = size_t(q / a.k) * a.H;
    float xv[CPL][8];
    {
      Chunk<ACT> ch[CPL];
#pragma unroll
      for (int s = 0; s < CPL; ++s) ch[s].load(a.x, xoff + min(s * 64 + lane, nch - 1) * 8);
#pragma unroll
      for (int s = 0; s < CPL; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) xv[s][i] = (s * 64 + lane < nch) ? ch[s].get(i) : 0.f;
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
      if (lane == 0 && i < a.I) a.h[size_t(q) * a.I + i] = valid ? silu_f(av) * uv : NAN;
    }
  }
}

// Batch-1 decode with bf16 or fp32 experts: the selection fused with the
// dense gate/up rows, as select_gateup_q4_kernel does for 4-bit experts.
// Block b serves pair p = b / bpp and kDecodeRowsPerBlock rows of its expert
// with gateup_dense_kernel's per-row arithmetic (outputs bitwise equal); the
// lane's x chunks are loaded before the selection starts.
template <int ACT, int WD, int CPL, bool SCREEN>
__global__ __launch_bounds__(kSelectThreads) void select_gateup_dense_kernel(ScreenSelectArgs sb, PairArgs a) {
  kernarg_lines<sizeof(ScreenSelectArgs) + sizeof(PairArgs)>();
  const SelectArgs& sa = sb.sel;
  constexpr int RPW = kDecodeRowsPerWave;
  __shared__ int32_t s_idx[kMaxK];
  __shared__ float s_gate[kMaxK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = a.H >> 3;
  const int bpp = (a.I + kDecodeRowsPerBlock - 1) / kDecodeRowsPerBlock;   // blocks per pair
  const int p = blockIdx.x / bpp, t = p / a.k, j = p - t * a.k;
  Chunk<ACT> xc[CPL];
#pragma unroll
  for (int s = 0; s < CPL; ++s) xc[s].load(a.x, size_t(t) * a.H + min(s * 64 + lane, nch - 1) * 8);
  select_policy<ACT, CPL, SCREEN>(sb, t, s_idx, s_gate);
  __syncthreads();
  if (j == 0 && blockIdx.x == p * bpp && tid < a.k) {   // first block of the token
    sa.idx[size_t(t) * a.k + tid] = s_idx[tid];
    sa.gates[size_t(t) * a.k + tid] = s_gate[tid];
  }
  const int i0 = (blockIdx.x - p * bpp) * kDecodeRowsPerBlock + wave * RPW;
  int e = s_idx[j];
  const bool valid = e >= 0 && e < a.E;
  e = valid ? e : 0;                                   // addresses stay in range; h becomes NaN
  Chunk<WD> wg[RPW][CPL], wu[RPW][CPL];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const size_t row = size_t(e) * a.I + min(i0 + r, a.I - 1);
#pragma unroll
    for (int s = 0; s < CPL; ++s) {
      const int c = min(s * 64 + lane, nch - 1);
      wg[r][s].load(a.wg, row * a.H + c * 8);
      wu[r][s].load(a.wu, row * a.H + c * 8);
    }
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int s = 0; s < CPL; ++s)
      if (!(i0 + r < a.I && s * 64 + lane < nch)) {
        wg[r][s].zero();
        wu[r][s].zero();
      }
  float xv[CPL][8];
#pragma unroll
  for (int s = 0; s < CPL; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) xv[s][i] = (s * 64 + lane < nch) ? xc[s].get(i) : 0.f;
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
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
    if (lane == 0 && i < a.I) a.h[size_t(p) * a.I + i] = valid ? silu_f(av) * uv : NAN;
  }
}

// ------------------------------------------------------------ down + combine

// Independent pairs: block (x, t) computes 8 output rows of token t; wave w
// handles the token's selected experts j = w, w + W, ... (W = min(k, 16)),
// 8 lanes per output row, lane g covering quant blocks (or 8-element chunks)
// g, g + 8, ... of I.  The expert's h slice comes straight from L2 into
// registers, so the weights, the scales and h are all in flight together.
// Each (row, expert) partial y_j is summed over its 8 lanes, and each output
// row is sum_j g_j y_j in selection order (fmaf chain), the arithmetic of
// the window kernel.
template <int WD>
__global__ __launch_bounds__(1024) void down_combine_single_kernel(PairArgs a) {
  kernarg_lines<sizeof(PairArgs)>();
  __shared__ float part[kMaxK][8];
  __shared__ float s_g[kMaxK];
  __shared__ int s_bad;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int g = lane & 7, grp = lane >> 3;
  const int I = a.I, k = a.k, t = blockIdx.y;
  const int o = blockIdx.x * 8 + grp;
  const int oc = min(o, a.H - 1);
  constexpr int kElems = (WD == MOE_Q4B32) ? 32 : 8;
  const int nsl = I / kElems;
  const int nblk = I >> 5;
  const int32_t* ti = a.idx + size_t(t) * k;
  if (threadIdx.x == 0) s_bad = 0;
  // every wave holds the token's k indices, one per lane (k <= 32), and
  // checks its own experts with a ballot (no dependent loads before the
  // weight loads); the gates come with them (the combine after the barrier
  // would otherwise wait for one more round trip).  Both loads issue
  // unconditionally and first: a load under a branch makes the wave wait
  // at the join for every load before it.
  const int v0 = ti[min(lane, k - 1)];
  const float g0 = a.gates[size_t(t) * k + min(lane, k - 1)];
  const int vi = (lane < k) ? v0 : -1;
  // the wave that ends the call reads the hint after them (its wait at the
  // join then comes with theirs)
  const bool ends = a.hint != nullptr && blockIdx.x == 0 && t == 0 && wave == 0;
  HintRead hr{};
  if (ends) hr = hint_read(a.hint, lane);
  if (wave == 0) s_g[min(lane, k - 1)] = g0;         // lanes past k store gate k - 1 again
  __syncthreads();
  for (int j = wave; j < k; j += nw) {
    int e = __shfl(vi, j);
    const bool inval = e < 0 || e >= a.E;
    const bool dup = __ballot(lane < j && vi == e) != 0ull;
    if (lane == 0 && (inval || dup)) {
      const int bad = inval ? kDevBadIndex : kDevDupIndex;
      atomicOr(&s_bad, bad);
      if (blockIdx.x == 0) atomicOr(a.dev_flag, bad);
    }
    e = inval ? 0 : e;                                 // addresses stay in range
    const PoolView pv = pool_view(a, e);
    const size_t row = size_t(e) * a.H + oc;
    const float* hj = a.h + (size_t(t) * k + j) * I;
    float y = 0.f;
    for (int sl = g; sl < nsl; sl += 8) {
      if constexpr (WD == MOE_Q4B32) {
        const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(pv.wd) + row * (I / 2) + sl * 16);
        const float d = f16_to_f32(pv.sd[row * nblk + sl]);
        y += down_lane_partial_q4(w, d, hj + sl * 32);
      } else {
        float hv[8];
        const float4 h0 = *reinterpret_cast<const float4*>(hj + sl * 8);
        const float4 h1 = *reinterpret_cast<const float4*>(hj + sl * 8 + 4);
        hv[0] = h0.x; hv[1] = h0.y; hv[2] = h0.z; hv[3] = h0.w;
        hv[4] = h1.x; hv[5] = h1.y; hv[6] = h1.z; hv[7] = h1.w;
        Chunk<WD> w;
        w.load(pv.wd, row * I + sl * 8);
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) p = fmaf(w.get(i), hv[i], p);
        y += p;
      }
    }
    y = group8_sum(y);
    if (g == 0) part[j][grp] = y;
  }
  __syncthreads();
  if (threadIdx.x < 8 && blockIdx.x * 8 + (int)threadIdx.x < a.H) {
    float s = 0.f;
    for (int j = 0; j < k; ++j) s = fmaf(s_g[j], part[j][threadIdx.x], s);
    a.out[size_t(t) * a.H + blockIdx.x * 8 + threadIdx.x] = s_bad ? NAN : s;
  }
  if (ends) hint_write(a.hint, hr, lane);
}

// Short windows (2 <= T <= 8 tokens, P = T k pairs): one block per 8 output
// rows handles every pair of the window, so each block pays one chain of
// dependent loads instead of one per token.  h of all pairs is staged in
// LDS (every load issued before any is stored), wave w takes pairs w,
// w + 16, ... and issues the weight loads of all of them before computing
// any; per-pair partials meet in LDS and each token's output is summed over
// its pairs in selection order.  Needs P <= 128 and I <= 256 (one quant
// block per lane of an 8-lane row group), so h takes at most 128 KB of LDS
// and UG float4 per thread stage it (P I / 4 <= 64 kWindowWaves UG).
constexpr int kWindowWaves = 16;
constexpr int kPairHLdsBytes = 64 * 1024;
constexpr int kWindowHLdsBytes = 128 * 1024;

bool down_window_fits(const PairArgs& a) {
  return a.T >= 2 && a.P <= kWindowWaves * 8 && a.I <= 8 * 32 && a.I % 32 == 0 &&
         size_t(a.P) * a.I * 4 <= kWindowHLdsBytes;
}

template <int UG>
__global__ __launch_bounds__(64 * kWindowWaves) void down_combine_window_q4_kernel(PairArgs a) {
  extern __shared__ __attribute__((aligned(16))) float sh_h[];   // [P][I]
  __shared__ float part[kMaxPairs][8];
  __shared__ float s_g[kMaxPairs];
  __shared__ int s_bad[kMaxPairs];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane & 7, grp = lane >> 3;
  const int I = a.I, k = a.k, P = a.P;
  const int o = blockIdx.x * 8 + grp;
  const int oc = min(o, a.H - 1);
  const int nsl = I >> 5, nblk = I >> 5;
  const bool ends = a.hint != nullptr && blockIdx.x == 0 && wave == 0;   // this wave ends the call
  HintRead hr{};
  if (ends) hr = hint_read(a.hint, lane);
  const float gq = (tid < P) ? a.gates[tid] : 0.f;  // the gates, read now (P <= 128 threads)
  // 1. h of every pair: all loads in flight (P I / 4 <= 64 kWindowWaves UG)
  const int n4 = P * I / 4;
  float4 hv4[UG];
#pragma unroll
  for (int i = 0; i < UG; ++i) {
    const int c = tid + i * 64 * kWindowWaves;
    hv4[i] = (c < n4) ? reinterpret_cast<const float4*>(a.h)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // 2. this wave's pairs: index, then code bytes and scale of its rows
  int vi[UG];
#pragma unroll
  for (int u = 0; u < UG; ++u) {
    const int p = min(wave + kWindowWaves * u, P - 1);
    const int t = p / k;
    vi[u] = (lane < k) ? a.idx[size_t(t) * k + lane] : -1;   // the token's k indices
  }
  uint4 w[UG];
  float d[UG];
  int badu[UG];
#pragma unroll
  for (int u = 0; u < UG; ++u) {
    const int p = min(wave + kWindowWaves * u, P - 1);
    const int j = p % k;
    int e = __shfl(vi[u], j);
    const bool inval = e < 0 || e >= a.E;
    const bool dup = __ballot(lane < j && vi[u] == e) != 0ull;
    badu[u] = inval ? kDevBadIndex : (dup ? kDevDupIndex : 0);
    e = inval ? 0 : e;                                 // addresses stay in range
    const PoolView pv = pool_view(a, e);
    const size_t row = size_t(e) * a.H + oc;
    const int sl = min(g, nsl - 1);
    w[u] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(pv.wd) + row * (I / 2) + sl * 16);
    d[u] = f16_to_f32(pv.sd[row * nblk + sl]);
  }
  // 3. h into LDS, flags cleared
#pragma unroll
  for (int i = 0; i < UG; ++i) {
    const int c = tid + i * 64 * kWindowWaves;
    if (c < n4) reinterpret_cast<float4*>(sh_h)[c] = hv4[i];
  }
  if (tid < P) s_g[tid] = gq;
  if (tid < a.T) s_bad[tid] = 0;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < UG; ++u) {
    const int p = wave + kWindowWaves * u;
    if (p < P && lane == 0 && badu[u]) {
      atomicOr(&s_bad[p / k], badu[u]);
      if (blockIdx.x == 0) atomicOr(a.dev_flag, badu[u]);
    }
  }
  // 4. per-pair partials
#pragma unroll
  for (int u = 0; u < UG; ++u) {
    const int p = wave + kWindowWaves * u;
    if (p >= P) break;                                 // wave-uniform
    float acc = 0.f;
    if (g < nsl) {
      const float* hq = sh_h + size_t(p) * I + g * 32;
      float hv[32];
#pragma unroll
      for (int i = 0; i < 32; i += 4) {
        const float4 v4 = *reinterpret_cast<const float4*>(hq + i);
        hv[i] = v4.x; hv[i + 1] = v4.y; hv[i + 2] = v4.z; hv[i + 3] = v4.w;
      }
      float hs = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) hs += hv[i];
      acc = d[u] * (q4_block_dot(w[u], hv) - 8.f * hs);
    }
    acc = group8_sum(acc);
    if (g == 0) part[p][grp] = acc;
  }
  __syncthreads();
  // 5. each token: its pairs in selection order, weighted by the gates
  for (int c = tid; c < a.T * 8; c += 64 * kWindowWaves) {
    const int t = c >> 3, r = c & 7;
    if (blockIdx.x * 8 + r >= a.H) continue;
    float s = 0.f;
    for (int j = 0; j < k; ++j) s = fmaf(s_g[t * k + j], part[t * k + j][r], s);
    a.out[size_t(t) * a.H + blockIdx.x * 8 + r] = s_bad[t] ? NAN : s;
  }
  if (ends) hint_write(a.hint, hr, lane);
}

// The window kernels take up to kWindowHLdsBytes of dynamic LDS; allow it
// once per process (the attribute belongs to the function, on every device).
hipError_t window_lds_attributes() {
  static const hipError_t err = [] {
    const void* fns[] = {reinterpret_cast<const void*>(&down_combine_window_q4_kernel<1>),
                         reinterpret_cast<const void*>(&down_combine_window_q4_kernel<2>),
                         reinterpret_cast<const void*>(&down_combine_window_q4_kernel<4>),
                         reinterpret_cast<const void*>(&down_combine_window_q4_kernel<8>)};
    for (const void* f : fns) {
      const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               kWindowHLdsBytes);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }();
  return err;
}

// One block per 8 output rows of all T tokens.  The block first copies h
// of every pair into LDS (when it fits; those loads do not depend on the
// indices, so they overlap the index loads), lists the pairs, marks tokens
// with a bad or repeated index and gives each distinct expert to one wave
// (8 lanes per output row, lane g of a row covering quant blocks, or
// 8-element chunks, g, g + 8, ... of I).  A wave loads the rows of up to UG
// of its experts before computing any, applies each expert to the h of every
// pair naming it, and the per-pair partials meet in LDS; each token's output
// is summed over its pairs in selection order (fixed order, no float
// atomics).
template <int WD, int SPL>
__global__ __launch_bounds__(1024) void down_combine_kernel(PairArgs a) {
  extern __shared__ __attribute__((aligned(16))) float sh_h[];   // [P][I] if it fits
  __shared__ float part[kMaxPairs][8];
  __shared__ int s_idx[kMaxPairs];
  __shared__ int s_uniq[kMaxPairs];
  __shared__ int s_bad[kMaxPairs];
  __shared__ int s_next[kMaxPairs];     // next pair naming the same expert, or -1
  __shared__ float s_g[kMaxPairs];
  __shared__ int s_nu;
  constexpr int UG = SPL == 1 ? 4 : (SPL <= 4 ? 2 : 1);   // experts prefetched per wave
  constexpr int kElems = (WD == MOE_Q4B32) ? 32 : 8;
  using WChunk = Chunk<WD == MOE_Q4B32 ? MOE_BF16 : WD>;   // q4: 16 B of codes
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int g = lane & 7, grp = lane >> 3;
  const int I = a.I, k = a.k, P = a.P;
  const int o = blockIdx.x * 8 + grp;
  const int oc = min(o, a.H - 1);
  const int nsl = I / kElems;
  const int nblk = I >> 5;
  const bool hl = size_t(P) * I * 4 <= kPairHLdsBytes;
  if (hl) {
    const float4* src = reinterpret_cast<const float4*>(a.h);
    float4* dst = reinterpret_cast<float4*>(sh_h);
    for (int c = threadIdx.x; c < P * I / 4; c += blockDim.x) dst[c] = src[c];
  }
  if (threadIdx.x == 0) s_nu = 0;
  for (int q = threadIdx.x; q < P; q += blockDim.x) {
    s_idx[q] = a.idx[q];
    s_g[q] = a.gates[q];                  // read now: the combine after the barriers needs them
  }
  for (int t = threadIdx.x; t < a.T; t += blockDim.x) s_bad[t] = 0;
  __syncthreads();
  for (int q = threadIdx.x; q < P; q += blockDim.x) {
    const int e = s_idx[q], t = q / k;
    const bool valid = e >= 0 && e < a.E;
    int bad = valid ? 0 : kDevBadIndex;
    bool first = valid;
    for (int qq = 0; qq < q && valid; ++qq) {
      if (s_idx[qq] == e) {
        first = false;
        if (qq / k == t) bad |= kDevDupIndex;
      }
    }
    if (bad) {
      atomicOr(&s_bad[t], bad);
      if (blockIdx.x == 0) atomicOr(a.dev_flag, bad);
    }
    if (first) s_uniq[atomicAdd(&s_nu, 1)] = q;
    int nx = -1;
    for (int qq = q + 1; qq < P && valid; ++qq)
      if (s_idx[qq] == e) {
        nx = qq;
        break;
      }
    s_next[q] = nx;
  }
  __syncthreads();
  const float* hbase = hl ? sh_h : a.h;
  const int nu = s_nu;
  for (int u0 = wave; u0 < nu; u0 += UG * nw) {
    WChunk w[UG][SPL];
    float d[UG][SPL];
    int eu[UG], qu[UG];
#pragma unroll
    for (int ug = 0; ug < UG; ++ug) {
      const int u = min(u0 + ug * nw, nu - 1);            // clamped: loads stay in range
      qu[ug] = s_uniq[u];
      eu[ug] = s_idx[qu[ug]];
      int ev = eu[ug];
      const PoolView pv = pool_view(a, ev);
      const size_t row = size_t(ev) * a.H + oc;
#pragma unroll
      for (int sp = 0; sp < SPL; ++sp) {
        const int sl = min(g + 8 * sp, nsl - 1);
        if constexpr (WD == MOE_Q4B32) {
          w[ug][sp].v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(pv.wd) + row * (I / 2) + sl * 16);
          d[ug][sp] = f16_to_f32(pv.sd[row * nblk + sl]);
        } else {
          w[ug][sp].load(pv.wd, row * I + sl * 8);
          d[ug][sp] = 1.f;
        }
      }
    }
#pragma unroll
    for (int ug = 0; ug < UG; ++ug) {
      if (u0 + ug * nw >= nu) break;                      // wave-uniform
      for (int q = qu[ug]; q >= 0; q = s_next[q]) {
        const float* hq = hbase + size_t(q) * I;
        float acc = 0.f;
#pragma unroll
        for (int sp = 0; sp < SPL; ++sp) {
          const int sl = g + 8 * sp;
          if (sl >= nsl) continue;
          float hv[kElems];
#pragma unroll
          for (int i = 0; i < kElems; i += 4) {
            const float4 v4 = *reinterpret_cast<const float4*>(hq + sl * kElems + i);
            hv[i] = v4.x; hv[i + 1] = v4.y; hv[i + 2] = v4.z; hv[i + 3] = v4.w;
          }
          if constexpr (WD == MOE_Q4B32) {
            float hs = 0.f;
#pragma unroll
            for (int i = 0; i < 32; ++i) hs += hv[i];
            acc = fmaf(d[ug][sp], q4_block_dot(w[ug][sp].v, hv) - 8.f * hs, acc);
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) acc = fmaf(w[ug][sp].get(i), hv[i], acc);
          }
        }
        acc = group8_sum(acc);
        if (g == 0) part[q][grp] = acc;
      }
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < a.T * 8; c += blockDim.x) {
    const int t = c >> 3, r = c & 7;
    if (blockIdx.x * 8 + r >= a.H) continue;
    float s = 0.f;
    for (int j = 0; j < k; ++j) s = fmaf(s_g[t * k + j], part[t * k + j][r], s);
    a.out[size_t(t) * a.H + blockIdx.x * 8 + r] = s_bad[t] ? NAN : s;
  }
}

template <bool INDEP>
static hipError_t launch_pairs(const PairArgs& a, int act, int wd, hipStream_t s);

bool pair_path_fits(const Layer& L, int T) { return T >= 1 && T * L.d.top_k <= kMaxPairs; }

// Up to this many tokens every (token, expert) pair is computed on its own
// (an expert named by two tokens is read twice, mostly from cache): in short
// windows nearly all pairs name distinct experts, and skipping the
// per-block deduplication takes it off the path from the indices to the
// weight loads.  Longer windows deduplicate so that shared experts are read
// once per call.
constexpr int kIndependentMaxT = 8;

static PairArgs pair_args(const Layer& L, const void* x, int T, const int32_t* idx,
                          const float* gates, float* out, float* h) {
  PairArgs a;
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
  a.T = T;
  a.P = T * a.k;
  a.dev_flag = L.dev_flag;
  a.hint = nullptr;
  a.tiers = L.tiers;
  return a;
}

hipError_t launch_pair_experts(const Layer& L, const void* x, int T, const int32_t* idx,
                               const float* gates, float* out, float* h, hipStream_t s) {
  const PairArgs a = pair_args(L, x, T, idx, gates, out, h);
  if (a.P > kMaxPairs) return hipErrorInvalidValue;
  if (T <= kIndependentMaxT) return launch_pairs<true>(a, L.d.act_dtype, L.d.expert_dtype, s);
  return launch_pairs<false>(a, L.d.act_dtype, L.d.expert_dtype, s);
}

// Down + combine of independent pairs (T <= kIndependentMaxT): the window
// kernel when h of every pair fits in LDS (4-bit experts), else one block row
// per token.
template <int K>
static hipError_t launch_down_indep(const PairArgs& a, hipStream_t s) {
  const dim3 g2((a.H + 7) / 8);
  if (K == MOE_Q4B32 && down_window_fits(a)) {
    const int ug = (a.P + kWindowWaves - 1) / kWindowWaves;
    const dim3 bw(64 * kWindowWaves);
    const size_t lh = size_t(a.P) * a.I * 4;
    if (hipError_t ea = window_lds_attributes(); ea != hipSuccess) return ea;
    if (ug <= 1) hipLaunchKernelGGL(down_combine_window_q4_kernel<1>, g2, bw, lh, s, a);
    else if (ug <= 2) hipLaunchKernelGGL(down_combine_window_q4_kernel<2>, g2, bw, lh, s, a);
    else if (ug <= 4) hipLaunchKernelGGL(down_combine_window_q4_kernel<4>, g2, bw, lh, s, a);
    else hipLaunchKernelGGL(down_combine_window_q4_kernel<8>, g2, bw, lh, s, a);
  } else {
    const int nw = a.P < 16 ? a.P : 16;
    hipLaunchKernelGGL(down_combine_single_kernel<K>, dim3(g2.x, a.T), dim3(64 * nw), 0, s, a);
  }
  return hipGetLastError();
}

template <bool INDEP>
static hipError_t launch_pairs(const PairArgs& a, int act, int wd, hipStream_t s) {
  dim3 g1((a.I + 7) / 8, a.P);
  if (wd == MOE_Q4B32) {
    const int mb = (a.H / 32 + 63) / 64;
    // batch 1: one row of gate and up per wave (more waves in flight for
    // the latency-bound loads); measured slower for windows of several
    // tokens, which keep two rows per wave
    const bool rows1 = INDEP && a.T == 1;
    const dim3 g4((a.I + 3) / 4, a.P);
#define MOE_GU_Q4(M)                                                                    \
  if (mb <= M) {                                                                        \
    if (rows1 && act == MOE_BF16)                                                       \
      hipLaunchKernelGGL((gateup_q4_kernel<MOE_BF16, M, INDEP, 1>), g4, dim3(256), 0, s, a);   \
    else if (rows1)                                                                     \
      hipLaunchKernelGGL((gateup_q4_kernel<MOE_F32, M, INDEP, 1>), g4, dim3(256), 0, s, a);    \
    else if (act == MOE_BF16)                                                           \
      hipLaunchKernelGGL((gateup_q4_kernel<MOE_BF16, M, INDEP>), g1, dim3(256), 0, s, a);      \
    else                                                                                \
      hipLaunchKernelGGL((gateup_q4_kernel<MOE_F32, M, INDEP>), g1, dim3(256), 0, s, a);       \
  } else
    MOE_GU_Q4(1) MOE_GU_Q4(2) MOE_GU_Q4(4) return hipErrorInvalidValue;
#undef MOE_GU_Q4
  } else {
    const int cpl = (a.H / 8 + 63) / 64;
#define MOE_GU_D(C)                                                                          \
  if (cpl <= C) {                                                                            \
    if (act == MOE_BF16 && wd == MOE_BF16)                                                   \
      hipLaunchKernelGGL((gateup_dense_kernel<MOE_BF16, MOE_BF16, C, INDEP>), g1, dim3(256), 0, s, a); \
    else if (act == MOE_F32 && wd == MOE_BF16)                                               \
      hipLaunchKernelGGL((gateup_dense_kernel<MOE_F32, MOE_BF16, C, INDEP>), g1, dim3(256), 0, s, a);  \
    else                                                                                     \
      hipLaunchKernelGGL((gateup_dense_kernel<MOE_F32, MOE_F32, C, INDEP>), g1, dim3(256), 0, s, a);   \
  } else
    MOE_GU_D(1) MOE_GU_D(2) MOE_GU_D(4) MOE_GU_D(8) MOE_GU_D(16) return hipErrorInvalidValue;
#undef MOE_GU_D
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int nw = a.P < 16 ? a.P : 16;
  dim3 g2((a.H + 7) / 8);
  const size_t lds = (size_t(a.P) * a.I * 4 <= kPairHLdsBytes) ? size_t(a.P) * a.I * 4 : 0;
  const int nsl = a.I / (wd == MOE_Q4B32 ? 32 : 8);
  const int spl = (nsl + 7) / 8;
#define MOE_DOWN_SPL(K, S) \
  if (spl <= S) hipLaunchKernelGGL((down_combine_kernel<K, S>), g2, dim3(64 * nw), lds, s, a); else
#define MOE_DOWN(K)                                                                                    \
  if constexpr (INDEP) {                                                                              \
    if (hipError_t ed = launch_down_indep<K>(a, s); ed != hipSuccess) return ed;                      \
  } else {                                                                                             \
    MOE_DOWN_SPL(K, 1) MOE_DOWN_SPL(K, 2) MOE_DOWN_SPL(K, 4) MOE_DOWN_SPL(K, 8) MOE_DOWN_SPL(K, 16)    \
    MOE_DOWN_SPL(K, 32) MOE_DOWN_SPL(K, 64) return hipErrorInvalidValue;                               \
  }
  if (wd == MOE_Q4B32) {
    MOE_DOWN(MOE_Q4B32)
  } else if (wd == MOE_BF16) {
    MOE_DOWN(MOE_BF16)
  } else {
    MOE_DOWN(MOE_F32)
  }
#undef MOE_DOWN
#undef MOE_DOWN_SPL
  return hipGetLastError();
}

// The kernel serves windows of up to kIndependentMaxT tokens, but it is
// dispatched at T = 1 only: at T = 5 the per-block selections (and the
// exact refinements they run in every block of a token) cost more than the
// launch gap they save (49.2 against 45.9 us per window).
constexpr int kFusedMaxT = 1;

bool decode_fused_fits(const Layer& L, int T) {
  const bool q4 = L.d.expert_dtype == MOE_Q4B32;
  const bool rows_fit = q4 ? (L.d.hidden / 32 + 63) / 64 <= 4 : (L.d.hidden / 8 + 63) / 64 <= 4;
  return L.d.top_k <= kMaxK && rows_fit && T >= 1 && T <= kFusedMaxT && T <= kIndependentMaxT &&
         T * L.d.top_k <= kMaxPairs;
}

// The fused selection + gate/up kernels (q4 or dense experts), then down +
// combine as its own launch.  `sb.sel` alone is used unless SCREEN.
template <bool SCREEN>
static hipError_t launch_select_gateup(const Layer& L, const ScreenSelectArgs& sb, const PairArgs& a,
                                       hipStream_t s) {
  const dim3 g1(a.P * ((a.I + kDecodeRowsPerBlock - 1) / kDecodeRowsPerBlock));
  const int act = L.d.act_dtype, wd = L.d.expert_dtype;
  if (wd != MOE_Q4B32) {
    const int cpl = (a.H / 8 + 63) / 64;
#define MOE_DEC_D(C)                                                                                          \
    if (cpl <= C) {                                                                                           \
      if (act == MOE_BF16 && wd == MOE_BF16)                                                                  \
        hipLaunchKernelGGL((select_gateup_dense_kernel<MOE_BF16, MOE_BF16, C, SCREEN>), g1, dim3(kSelectThreads), 0, s, sb, a); \
      else if constexpr (!SCREEN) {                                                                           \
        if (act == MOE_F32 && wd == MOE_BF16)                                                                 \
          hipLaunchKernelGGL((select_gateup_dense_kernel<MOE_F32, MOE_BF16, C, false>), g1, dim3(kSelectThreads), 0, s, sb, a); \
        else                                                                                                  \
          hipLaunchKernelGGL((select_gateup_dense_kernel<MOE_F32, MOE_F32, C, false>), g1, dim3(kSelectThreads), 0, s, sb, a);  \
      } else return hipErrorInvalidValue;                                                                     \
    } else
    MOE_DEC_D(1) MOE_DEC_D(2) MOE_DEC_D(4) return hipErrorInvalidValue;
#undef MOE_DEC_D
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return wd == MOE_BF16 ? launch_down_indep<MOE_BF16>(a, s) : launch_down_indep<MOE_F32>(a, s);
  }
  const int mb = (a.H / 32 + 63) / 64;
  const int cplr = (a.H / 8 + 63) / 64;
#define MOE_DEC_Q4(M, C)                                                                                    \
  if (mb <= M && cplr <= C) {                                                                               \
    if (act == MOE_BF16)                                                                                    \
      hipLaunchKernelGGL((select_gateup_q4_kernel<MOE_BF16, M, C, SCREEN>), g1, dim3(kSelectThreads), 0, s, sb, a); \
    else if constexpr (!SCREEN)                                                                             \
      hipLaunchKernelGGL((select_gateup_q4_kernel<MOE_F32, M, C, false>), g1, dim3(kSelectThreads), 0, s, sb, a);  \
    else return hipErrorInvalidValue;                                                                       \
  } else
  MOE_DEC_Q4(1, 4) MOE_DEC_Q4(2, 8) MOE_DEC_Q4(4, 16) return hipErrorInvalidValue;
#undef MOE_DEC_Q4
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_down_indep<MOE_Q4B32>(a, s);
}

hipError_t launch_decode_fused(const Layer& L, const void* x, int T, const double* z, const float* gmax,
                               const double* xnorm, const RouterBound& rb, int32_t* idx, float* gates,
                               float* out, float* h, hipStream_t s) {
  if (!decode_fused_fits(L, T)) return hipErrorInvalidValue;
  ScreenSelectArgs sb{};
  sb.sel = make_select_args(L, x, z, false, gmax, xnorm, idx, gates, rb);
  const PairArgs a = pair_args(L, x, T, idx, gates, out, h);
  return launch_select_gateup<false>(L, sb, a, s);
}

hipError_t launch_decode_screen(const Layer& L, const void* x, const float* z8, const float* g8, const double* xq,
                                const ScreenList* list, int32_t* idx, float* gates, float* out, float* h,
                                hipStream_t s) {
  if (list == nullptr) return hipErrorInvalidValue;
  ScreenSelectArgs sb = make_screen_select_args(L, x, z8, g8, xq, idx, gates);
  PairArgs a = pair_args(L, x, 1, idx, gates, out, h);
  set_screen_list(sb, L, list, false);
  a.hint = list->hint;              // the down kernel ends the call
  return launch_select_gateup<true>(L, sb, a, s);
}

}  // namespace moe
