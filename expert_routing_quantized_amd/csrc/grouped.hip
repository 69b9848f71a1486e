// Grouped expert path for T > 1 tokens (verify windows and prefill chunks:
// pyshine source tour, Understanding the Architecture, the paragraphs on
// speculative decoding and on chunked prompt reading).  The T*k token-expert pairs are sorted by expert so that each
// active expert's weights are streamed once for all of its tokens:
//
//   counts[e]  = #pairs routed to e            (integer atomics)
//   offsets    = exclusive scan of counts; active = experts with counts > 0
//   pos[p]     = offsets[e_p] + rank of p inside e's segment
//   ptok[pos]  = token of the pair stored at that segment position
//   Hm[pos][:] = silu(G_e x_t) * (U_e x_t)       (fp32)
//   Y[pos][:]  = D_e Hm[pos]                      (fp32)
//   out[t]     = sum_j g[t][j] Y[pos[t k + j]]    (j in order: deterministic)
//
// The order of pairs inside a segment comes from atomics, but no result
// depends on it: every row of Hm and Y is computed from its own token only.
// The vector-ALU kernels below keep one weight row slice in registers and
// loop over the segment's tokens, which suits the small groups of verify
// windows (about 1.1 tokens per active expert at T = 5).
#include <limits.h>

#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ float silu_g(float a) { return a / (1.0f + expf(-a)); }

__device__ __forceinline__ float q4_dot32(const uint4 w, const float* xv) {
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

__global__ void fill_i32_kernel(int* p, int v, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = v;
}

__global__ void hist_kernel(GroupArgs a) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= a.P) return;
  const int e = a.idx[p];
  if (e < 0 || e >= a.E) {
    atomicOr(a.dev_flag, kDevBadIndex);
    a.slot[p] = -1;
    return;
  }
  const int t = p / a.k, j = p - t * a.k;
  for (int jj = 0; jj < j; ++jj)
    if (a.idx[t * a.k + jj] == e) atomicOr(a.dev_flag, kDevDupIndex);
  a.slot[p] = atomicAdd(&a.counts[e], 1);
}

// Exclusive prefix sum over a 1024-thread block (16 waves); *total gets the sum.
__device__ int block_excl_scan_1024(int v, int* s_w, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_w[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < 16; ++i) {
    const int sw = s_w[i];
    base += (i < w) ? sw : 0;
    tot += sw;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// Single-workgroup exclusive scan of counts and compaction of the active
// experts: thread i owns experts [i C, i C + C) with C = ceil(E / 1024),
// loads their counts once, and three block-wide prefix sums (pairs, active
// experts, 32-row tiles) give every thread its starting offsets; the
// offsets, the active list and the tile list are then written from
// registers in expert order.
// Up to kScanLdsPer experts per thread (E <= 24,576) the counts pass
// through LDS with coalesced global reads and writes: each thread's range
// sits at an odd pitch, so the threads of a wave reading the same position
// of their ranges hit distinct banks.
constexpr int kScanMaxPer = 32;           // E <= 32768 in registers, larger E loops
constexpr int kScanLdsPer = 24;
__global__ __launch_bounds__(1024) void scan_kernel(GroupArgs a) {
  __shared__ int s_w[16];
  __shared__ int s_c[1024 * (kScanLdsPer + 1)];
  const int tid = threadIdx.x;
  const int per = (a.E + 1023) / 1024;
  const int e0 = min(tid * per, a.E), e1 = min(e0 + per, a.E);
  const bool lds = per <= kScanLdsPer;
  const int pitch = per | 1;
  const unsigned long long magic = ((1ull << 32) + per - 1) / per;   // j / per = (j magic) >> 32 for j < 2^20
  auto spos = [&](int j) {
    const int q = int((unsigned long long)j * magic >> 32);
    return q * pitch + (j - q * per);
  };
  if (lds) {
    // every count load issued before the first store (a load-store loop
    // waited one L2 round trip per count)
    int ld[kScanLdsPer];
#pragma unroll
    for (int i = 0; i < kScanLdsPer; ++i) ld[i] = a.counts[min(tid + 1024 * i, a.E - 1)];
#pragma unroll
    for (int i = 0; i < kScanLdsPer; ++i)
      if (tid + 1024 * i < a.E) s_c[spos(tid + 1024 * i)] = ld[i];
    __syncthreads();
  }
  int c[kScanMaxPer];
  int sum = 0, act = 0, til = 0, big = 0;
  auto count = [&](int ce) {
    sum += ce;
    act += (ce > 0 && ce <= a.small_max);
    til += (ce > a.small_max && ce <= kTileRows) ? 1 : 0;
    big += (ce > a.small_max && ce > kTileRows) ? (ce + kBigTileRows - 1) / kBigTileRows : 0;
  };
  if (lds) {
#pragma unroll
    for (int i = 0; i < kScanLdsPer; ++i) c[i] = (e0 + i < e1) ? s_c[tid * pitch + i] : 0;
#pragma unroll
    for (int i = 0; i < kScanLdsPer; ++i) count(c[i]);
  } else if (per <= kScanMaxPer) {
#pragma unroll
    for (int i = 0; i < kScanMaxPer; ++i) c[i] = (e0 + i < e1) ? a.counts[e0 + i] : 0;
#pragma unroll
    for (int i = 0; i < kScanMaxPer; ++i) count(c[i]);
  } else {
    for (int e = e0; e < e1; ++e) count(a.counts[e]);
  }
  int tot_sum, tot_act, tot_til, tot_big;
  int run = block_excl_scan_1024(sum, s_w, &tot_sum);
  int arun = block_excl_scan_1024(act, s_w, &tot_act);
  int trun = block_excl_scan_1024(til, s_w, &tot_til);
  int brun = block_excl_scan_1024(big, s_w, &tot_big);
  auto emit = [&](int e, int ce) {
    if (lds)
      s_c[tid * pitch + (e - e0)] = run;          // written back below, coalesced
    else
      a.offsets[e] = run;
    if (ce > 0 && ce <= a.small_max) {
      a.active[1 + arun++] = e;
    } else if (ce > a.small_max && ce <= kTileRows) {
      a.tiles[1 + 2 * trun] = e;
      a.tiles[2 + 2 * trun] = 0;
      ++trun;
    } else if (ce > a.small_max) {
      for (int r0 = 0; r0 < ce; r0 += kBigTileRows) {
        a.tiles_big[1 + 2 * brun] = e;
        a.tiles_big[2 + 2 * brun] = r0;
        ++brun;
      }
    }
    run += ce;
  };
  if (lds) {
#pragma unroll
    for (int i = 0; i < kScanLdsPer; ++i)
      if (e0 + i < e1) emit(e0 + i, c[i]);
    __syncthreads();
    for (int j = tid; j < a.E; j += 1024) a.offsets[j] = s_c[spos(j)];
  } else if (per <= kScanMaxPer) {
#pragma unroll
    for (int i = 0; i < kScanMaxPer; ++i)
      if (e0 + i < e1) emit(e0 + i, c[i]);
  } else {
    for (int e = e0; e < e1; ++e) emit(e, a.counts[e]);
  }
  if (tid == 0) {
    a.offsets[a.E] = tot_sum;
    a.active[0] = tot_act;
    a.tiles[0] = tot_til;
    a.tiles_big[0] = tot_big;
  }
}

// Grouping of at most 1024 pairs in one workgroup (verify windows and small
// batches): the pairs are ranked by (expert, pair index) directly, so nothing
// proportional to E is touched (no histogram clear, no scan over E).  Writes
// the same outputs as hist + scan + scatter: pos, ptok, active list, tile
// list, and counts / offsets of the active experts (the only entries read).
__global__ __launch_bounds__(1024) void group_small_kernel(GroupArgs a) {
  __shared__ int s_e[1024];
  __shared__ int s_sorted[1024];
  __shared__ int s_w[16];
  const int p = threadIdx.x;
  const int P = a.P;
  int e = INT_MAX;                       // invalid pairs sort after every expert
  if (p < P) {
    const int v = a.idx[p];
    if (v < 0 || v >= a.E) {
      atomicOr(a.dev_flag, kDevBadIndex);
    } else {
      e = v;
      const int t = p / a.k, j = p - t * a.k;
      for (int jj = 0; jj < j; ++jj)
        if (a.idx[t * a.k + jj] == v) atomicOr(a.dev_flag, kDevDupIndex);
    }
  }
  s_e[p] = e;
  const int nv = __syncthreads_count(p < P && e != INT_MAX);
  int r = -1;
  if (p < P && e != INT_MAX) {
    r = 0;
    for (int q = 0; q < P; ++q) {
      const int eq = s_e[q];
      r += (eq < e) || (eq == e && q < p);
    }
    a.ptok[r] = p / a.k;
    s_sorted[r] = e;
  }
  if (p < P) a.pos[p] = r;
  __syncthreads();
  // thread r < nv looks at sorted position r; segment starts own their expert
  const bool start = p < nv && (p == 0 || s_sorted[p - 1] != s_sorted[p]);
  int cnt = 0;
  if (start) {
    const int es = s_sorted[p];
    cnt = 1;
    while (p + cnt < nv && s_sorted[p + cnt] == es) ++cnt;
  }
  const bool listed = start && cnt <= a.small_max;
  const int nt = (start && !listed && cnt <= kTileRows) ? 1 : 0;
  const int nb = (start && !listed && cnt > kTileRows) ? (cnt + kBigTileRows - 1) / kBigTileRows : 0;
  int nact, ntiles, nbig;
  const int ai = block_excl_scan_1024(listed ? 1 : 0, s_w, &nact);
  const int ti = block_excl_scan_1024(nt, s_w, &ntiles);
  const int bi = block_excl_scan_1024(nb, s_w, &nbig);
  if (start) {
    const int es = s_sorted[p];
    if (listed) a.active[1 + ai] = es;
    a.counts[es] = cnt;
    a.offsets[es] = p;
    if (nt) {
      a.tiles[1 + 2 * ti] = es;
      a.tiles[2 + 2 * ti] = 0;
    }
    for (int i = 0; i < nb; ++i) {
      a.tiles_big[1 + 2 * (bi + i)] = es;
      a.tiles_big[2 + 2 * (bi + i)] = i * kBigTileRows;
    }
  }
  if (p == 0) {
    a.active[0] = nact;
    a.tiles[0] = ntiles;
    a.tiles_big[0] = nbig;
  }
}

__global__ void scatter_kernel(GroupArgs a) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= a.P) return;
  const int s = a.slot[p];
  if (s < 0) {
    a.pos[p] = -1;
    return;
  }
  const int q = a.offsets[a.idx[p]] + s;
  a.pos[p] = q;
  a.ptok[q] = p / a.k;
}

// --------------------------------------------------------------- gate/up
// One wave per pair of intermediate rows of one active expert; the weights
// stay in registers while the wave walks the expert's tokens.
template <int ACT, int WD, int SL>
__global__ __launch_bounds__(256) void grouped_gateup_kernel(GroupArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nact = a.active[0];
  constexpr int kRows = 2;
  const int i0 = (blockIdx.x * 4 + wave) * kRows;
  // slot layout: q4 -> SL quant blocks of 32 per lane; dense -> SL chunks of 8 per lane
  constexpr int kElems = (WD == MOE_Q4B32) ? 32 : 8;
  const int nsl = a.H / kElems;
  for (int ai = blockIdx.y; ai < nact; ai += gridDim.y) {
    const int e = a.active[1 + ai];
    const int n = a.counts[e];
    const int seg = a.offsets[e];
    uint4 wq[2][kRows][SL];
    float dq[2][kRows][SL];
    Chunk<WD == MOE_Q4B32 ? MOE_BF16 : WD> wdn[2][kRows][(WD == MOE_Q4B32) ? 1 : SL];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int i = i0 + r;
      const size_t row = size_t(e) * a.I + i;
#pragma unroll
      for (int s = 0; s < SL; ++s) {
        const int c = s * 64 + lane;
        const bool ok = (i < a.I) && (c < nsl);
        if constexpr (WD == MOE_Q4B32) {
          if (ok) {
            wq[0][r][s] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.wg) + row * (a.H / 2) + c * 16);
            wq[1][r][s] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.wu) + row * (a.H / 2) + c * 16);
            dq[0][r][s] = f16_to_f32(a.sg[row * nsl + c]);
            dq[1][r][s] = f16_to_f32(a.su[row * nsl + c]);
          } else {
            wq[0][r][s] = wq[1][r][s] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
            dq[0][r][s] = dq[1][r][s] = 0.f;
          }
        } else {
          if (ok) {
            wdn[0][r][s].load(a.wg, row * a.H + c * 8);
            wdn[1][r][s].load(a.wu, row * a.H + c * 8);
          } else {
            if constexpr (WD == MOE_BF16) { wdn[0][r][s].v = wdn[1][r][s].v = make_uint4(0, 0, 0, 0); }
            else { wdn[0][r][s].a = wdn[0][r][s].b = wdn[1][r][s].a = wdn[1][r][s].b = make_float4(0, 0, 0, 0); }
          }
        }
      }
    }
    for (int q = 0; q < n; ++q) {
      const int t = a.ptok[seg + q];
      float pa[kRows] = {}, pu[kRows] = {};
#pragma unroll
      for (int s = 0; s < SL; ++s) {
        const int c = s * 64 + lane;
        if (c >= nsl) continue;
        float xv[kElems];
#pragma unroll
        for (int cc = 0; cc < kElems / 8; ++cc) {
          Chunk<ACT> ch;
          ch.load(a.x, size_t(t) * a.H + c * kElems + cc * 8);
#pragma unroll
          for (int i = 0; i < 8; ++i) xv[cc * 8 + i] = ch.get(i);
        }
        if constexpr (WD == MOE_Q4B32) {
          float xs = 0.f;
#pragma unroll
          for (int i = 0; i < 32; ++i) xs += xv[i];
#pragma unroll
          for (int r = 0; r < kRows; ++r) {
            pa[r] = fmaf(dq[0][r][s], q4_dot32(wq[0][r][s], xv) - 8.f * xs, pa[r]);
            pu[r] = fmaf(dq[1][r][s], q4_dot32(wq[1][r][s], xv) - 8.f * xs, pu[r]);
          }
        } else {
#pragma unroll
          for (int r = 0; r < kRows; ++r)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              pa[r] = fmaf(wdn[0][r][s].get(i), xv[i], pa[r]);
              pu[r] = fmaf(wdn[1][r][s].get(i), xv[i], pu[r]);
            }
        }
      }
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const float av = wave_sum(pa[r]), uv = wave_sum(pu[r]);
        const int i = i0 + r;
        if (lane == 0 && i < a.I) a.hm[size_t(seg + q) * a.I + i] = silu_g(av) * uv;
      }
    }
  }
}

// --------------------------------------------------------------- down
// 8 lanes per output row; 8 rows per wave; weights in registers, tokens looped.
template <int WD, int SL>
__global__ __launch_bounds__(256) void grouped_down_kernel(GroupArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane & 7, grp = lane >> 3;
  const int nact = a.active[0];
  const int o = (blockIdx.x * 4 + wave) * 8 + grp;
  constexpr int kElems = (WD == MOE_Q4B32) ? 32 : 8;
  const int nsl = a.I / kElems;
  for (int ai = blockIdx.y; ai < nact; ai += gridDim.y) {
    const int e = a.active[1 + ai];
    const int n = a.counts[e];
    const int seg = a.offsets[e];
    const size_t row = size_t(e) * a.H + o;
    uint4 wq[SL];
    float dq[SL];
    Chunk<WD == MOE_Q4B32 ? MOE_BF16 : WD> wdn[(WD == MOE_Q4B32) ? 1 : SL];
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const int c = s * 8 + g;
      const bool ok = (o < a.H) && (c < nsl);
      if constexpr (WD == MOE_Q4B32) {
        if (ok) {
          wq[s] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.wd) + row * (a.I / 2) + c * 16);
          dq[s] = f16_to_f32(a.sd[row * nsl + c]);
        } else {
          wq[s] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
          dq[s] = 0.f;
        }
      } else {
        if (ok) {
          wdn[s].load(a.wd, row * a.I + c * 8);
        } else {
          if constexpr (WD == MOE_BF16) wdn[s].v = make_uint4(0, 0, 0, 0);
          else { wdn[s].a = wdn[s].b = make_float4(0, 0, 0, 0); }
        }
      }
    }
    for (int q = 0; q < n; ++q) {
      const float* hr = a.hm + size_t(seg + q) * a.I;
      float p = 0.f;
#pragma unroll
      for (int s = 0; s < SL; ++s) {
        const int c = s * 8 + g;
        if (c >= nsl) continue;
        float hv[kElems];
#pragma unroll
        for (int i = 0; i < kElems; i += 4) {
          const float4 v4 = *reinterpret_cast<const float4*>(hr + c * kElems + i);
          hv[i] = v4.x; hv[i + 1] = v4.y; hv[i + 2] = v4.z; hv[i + 3] = v4.w;
        }
        if constexpr (WD == MOE_Q4B32) {
          float hs = 0.f;
#pragma unroll
          for (int i = 0; i < 32; ++i) hs += hv[i];
          p = fmaf(dq[s], q4_dot32(wq[s], hv) - 8.f * hs, p);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) p = fmaf(wdn[s].get(i), hv[i], p);
        }
      }
      p = group8_sum(p);
      if (g == 0 && o < a.H) a.y[size_t(seg + q) * a.H + o] = p;
    }
  }
}

// --------------------------------------------------------------- combine
// One block per (1024 outputs, token): the token's k positions and gates go
// to LDS once (with the bad / repeated index check), then each thread sums
// its 4 outputs over the pairs in selection order.
__global__ __launch_bounds__(256) void combine_kernel(GroupArgs a) {
  __shared__ int s_pos[kMaxK];
  __shared__ float s_g[kMaxK];
  __shared__ int s_bad;
  const int t = blockIdx.y;
  const int k = a.k, lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {          // wave 0: the token's k pairs, one per lane (k <= 32)
    const bool live = lane < k;
    const int p = t * k + lane;
    const int e = live ? a.idx[p] : -1;
    const int q = live ? a.pos[p] : 0;
    const float g = live ? a.gates[p] : 0.f;
    bool bad = live && q < 0;
    for (int jj = 0; jj < k; ++jj) {   // a repeated index of the token (shuffles, no loads)
      const int ej = __shfl(e, jj);
      bad |= live && jj < lane && ej == e;
    }
    if (live) {
      s_pos[lane] = q < 0 ? 0 : q;
      s_g[lane] = g;
    }
    const bool any_bad = __ballot(bad) != 0ull;
    if (lane == 0) s_bad = any_bad ? 1 : 0;
  }
  __syncthreads();
  const int o = 4 * (blockIdx.x * blockDim.x + threadIdx.x);   // 4 consecutive outputs (H % 8 == 0)
  if (o >= a.H) return;
  // the k rows' 16-byte pieces in flight together (groups of 8), each output
  // summed in j order
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < k; j0 += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = (j0 + u < k) ? *reinterpret_cast<const float4*>(a.y + size_t(s_pos[j0 + u]) * a.H + o)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (j0 + u < k) {
        const float g = s_g[j0 + u];
        acc.x = fmaf(g, v[u].x, acc.x);
        acc.y = fmaf(g, v[u].y, acc.y);
        acc.z = fmaf(g, v[u].z, acc.z);
        acc.w = fmaf(g, v[u].w, acc.w);
      }
  }
  if (s_bad) acc = make_float4(NAN, NAN, NAN, NAN);
  float* dst = a.out + size_t(t) * a.H + o;
  if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {   // the caller's out need not be 16-byte aligned
    *reinterpret_cast<float4*>(dst) = acc;
  } else {
    dst[0] = acc.x;
    dst[1] = acc.y;
    dst[2] = acc.z;
    dst[3] = acc.w;
  }
}

hipError_t launch_grouped_experts(const Layer& L, const void* x, int T, const int32_t* idx,
                                  const float* gates, float* out, char* ws, const Workspace& W,
                                  hipStream_t s) {
  GroupArgs a;
  a.x = x;
  a.idx = idx;
  a.gates = gates;
  a.wg = L.d.w_gate;
  a.wu = L.d.w_up;
  a.wd = L.d.w_down;
  a.sg = L.d.s_gate;
  a.su = L.d.s_up;
  a.sd = L.d.s_down;
  a.T = T;
  a.H = L.d.hidden;
  a.I = L.d.inter;
  a.E = L.d.n_experts;
  a.k = L.d.top_k;
  a.P = T * a.k;
  a.counts = reinterpret_cast<int*>(ws + W.counts);
  a.offsets = reinterpret_cast<int*>(ws + W.offsets);
  a.slot = reinterpret_cast<int*>(ws + W.slot);
  a.pos = reinterpret_cast<int*>(ws + W.pos);
  a.ptok = reinterpret_cast<int*>(ws + W.ptok);
  a.active = reinterpret_cast<int*>(ws + W.active);
  a.tiles = reinterpret_cast<int*>(ws + W.tiles);
  a.tiles_big = reinterpret_cast<int*>(ws + W.tiles_big);
  a.hm = reinterpret_cast<float*>(ws + W.hm);
  a.y = reinterpret_cast<float*>(ws + W.y);
  a.out = out;
  a.dev_flag = L.dev_flag;
  // bf16 batches on MFMA: experts with few pairs still go to the vector-ALU
  // kernels, whose row-contiguous weight loads stream faster than the
  // tiles' transposed ones; the others get 32-row MFMA tiles
  a.small_max = grouped_uses_mfma(L, T) ? kMfmaSmallMax : INT_MAX;

  if (a.P <= 1024) {
    hipLaunchKernelGGL(group_small_kernel, dim3(1), dim3(1024), 0, s, a);
  } else {
    hipLaunchKernelGGL(fill_i32_kernel, dim3(min(1024, (a.E + 255) / 256)), dim3(256), 0, s, a.counts, 0, a.E);
    hipLaunchKernelGGL(hist_kernel, dim3((a.P + 255) / 256), dim3(256), 0, s, a);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, a);
    hipLaunchKernelGGL(scatter_kernel, dim3((a.P + 255) / 256), dim3(256), 0, s, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  const bool mfma = grouped_uses_mfma(L, T);
  if (!mfma || a.small_max > 0) {      // experts on the vector-ALU list
    const int maxact = min(a.P, a.E);
    const int gy = min(maxact, 4096);
    const int act = L.d.act_dtype, wd = L.d.expert_dtype;
    dim3 g1((a.I + 7) / 8, gy);
    if (wd == MOE_Q4B32) {
      const int sl = (a.H / 32 + 63) / 64;
#define MOE_GG_Q4(S)                                                                           \
    if (sl <= S) {                                                                               \
      if (act == MOE_BF16)                                                                       \
        hipLaunchKernelGGL((grouped_gateup_kernel<MOE_BF16, MOE_Q4B32, S>), g1, dim3(256), 0, s, a); \
      else                                                                                       \
        hipLaunchKernelGGL((grouped_gateup_kernel<MOE_F32, MOE_Q4B32, S>), g1, dim3(256), 0, s, a);  \
    } else
      MOE_GG_Q4(1) MOE_GG_Q4(2) MOE_GG_Q4(4) return hipErrorInvalidValue;
#undef MOE_GG_Q4
    } else {
      const int sl = (a.H / 8 + 63) / 64;
#define MOE_GG_D(S)                                                                                 \
    if (sl <= S) {                                                                                    \
      if (act == MOE_BF16 && wd == MOE_BF16)                                                          \
        hipLaunchKernelGGL((grouped_gateup_kernel<MOE_BF16, MOE_BF16, S>), g1, dim3(256), 0, s, a);   \
      else if (act == MOE_F32 && wd == MOE_BF16)                                                      \
        hipLaunchKernelGGL((grouped_gateup_kernel<MOE_F32, MOE_BF16, S>), g1, dim3(256), 0, s, a);    \
      else                                                                                            \
        hipLaunchKernelGGL((grouped_gateup_kernel<MOE_F32, MOE_F32, S>), g1, dim3(256), 0, s, a);     \
    } else
      MOE_GG_D(1) MOE_GG_D(2) MOE_GG_D(4) MOE_GG_D(8) MOE_GG_D(16) return hipErrorInvalidValue;
#undef MOE_GG_D
    }
    err = hipGetLastError();
    if (err != hipSuccess) return err;

    dim3 g2((a.H + 31) / 32, gy);
    if (wd == MOE_Q4B32) {
      const int sl = (a.I / 32 + 7) / 8;
#define MOE_GD_Q4(S) \
    if (sl <= S) hipLaunchKernelGGL((grouped_down_kernel<MOE_Q4B32, S>), g2, dim3(256), 0, s, a); else
      MOE_GD_Q4(1) MOE_GD_Q4(2) MOE_GD_Q4(4) MOE_GD_Q4(8) MOE_GD_Q4(16) return hipErrorInvalidValue;
#undef MOE_GD_Q4
    } else {
      const int sl = (a.I / 8 + 7) / 8;
#define MOE_GD_D(S)                                                                      \
    if (sl <= S) {                                                                         \
      if (wd == MOE_BF16) hipLaunchKernelGGL((grouped_down_kernel<MOE_BF16, S>), g2, dim3(256), 0, s, a); \
      else hipLaunchKernelGGL((grouped_down_kernel<MOE_F32, S>), g2, dim3(256), 0, s, a);  \
    } else
      MOE_GD_D(1) MOE_GD_D(2) MOE_GD_D(4) MOE_GD_D(8) MOE_GD_D(16) MOE_GD_D(32) MOE_GD_D(64) return hipErrorInvalidValue;
#undef MOE_GD_D
    }
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (mfma) {
    err = launch_grouped_mfma(a, s);
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(combine_kernel, dim3((a.H + 1023) / 1024, T), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
