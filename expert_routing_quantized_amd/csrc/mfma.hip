// Router logits of a prefill chunk or large verify batch as a bf16 MFMA GEMM:
// z[t][e] = sum_h x[t][h] R[e][h] + b[e] for T tokens at once.
//
// At batch 1 the router is a GEMV and matrix units waste their tile (the
// hexlives dispatch's archived tensor-core experiment); with T = 2048 tokens
// it is a dense 2048 x 2048 x 24,576 contraction (206 GFLOP), the one place
// on the path where MFMA is the bound.  Both operands are K-contiguous (x
// rows, router rows).  Each 512-thread block computes a 128-token x
// 128-expert tile with v_mfma_f32_32x32x16_bf16 (8 waves of 32 x 64),
// staging 64-wide K slices of both operands through LDS with 128-byte row
// pieces, two slices prefetched into registers ahead of the one being
// multiplied.  Tiles are ordered for the 8 XCDs: blocks are dealt to XCDs
// round-robin, so XCD j gets a contiguous range of expert tiles and walks
// all token tiles of one expert tile before the next, which keeps that
// router tile in its own L2 while every token tile reuses it.
//
// Rounding model for the certified selection: the fp32 MFMA accumulators are
// added into binary64 accumulators after every 128 of K (8 instructions of
// K = 16, each counted as at most 17 binary32 roundings, truncation
// included), and the remaining sums and the bias are binary64: d32 = 136,
// d64 = H/128 + 1.  The epilogue writes the binary64 logits, the maximum of
// every 4 consecutive experts (rounded up to binary32) and ||x_t||^2 -- the
// same outputs as the vector-ALU router, so the same selection kernel runs.
#include "moe_internal.h"

#include <type_traits>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBK = 32;                    // K granularity the MFMA paths require
constexpr int kRM = 128, kRN = 128;        // router GEMM block tile (tokens x experts)
constexpr int kRK = 64, kRKP = kRK + 8;    // K slice and its LDS row pitch (elements)
constexpr int kRThreads = 512;
constexpr int kRChunks = (kRM + kRN) * (kRK / 8) / kRThreads;   // 16-byte loads per thread per slice

__global__ __launch_bounds__(kRThreads) void router_gemm_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ R, const float* __restrict__ bias,
    int T, int H, int E, int nm, int nn, int nper, double* __restrict__ z, float* __restrict__ gmax,
    double* __restrict__ xnorm, int* __restrict__ dev_flag) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][kRM][kRKP];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][kRN][kRKP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int xcd = blockIdx.x % 8, loc = blockIdx.x / 8;
  const int nb = xcd * nper + loc / nm, mb = loc % nm;
  if (nb >= nn) return;                                  // whole block
  const int m0 = mb * kRM, n0 = nb * kRN;
  const int wm = (wave & 3) * 32, wn = (wave >> 2) * 64;

  // chunk c = tid + 512 i: staging row c / 8 (x rows, then router rows), 16-byte piece c % 8
  const uint16_t* src[kRChunks];
  int drow[kRChunks], dcol[kRChunks];
  bool isb[kRChunks];
#pragma unroll
  for (int i = 0; i < kRChunks; ++i) {
    const int c = tid + i * kRThreads;
    const int r = c >> 3;
    dcol[i] = (c & 7) * 8;
    isb[i] = r >= kRM;
    drow[i] = isb[i] ? r - kRM : r;
    src[i] = isb[i] ? R + size_t(min(n0 + drow[i], E - 1)) * H : X + size_t(min(m0 + drow[i], T - 1)) * H;
  }
  const int nk = (H + kRK - 1) / kRK;
  auto load = [&](int kt, uint4 (&v)[kRChunks]) {
#pragma unroll
    for (int i = 0; i < kRChunks; ++i) {
      const int k = kt * kRK + dcol[i];
      const uint4 w = *reinterpret_cast<const uint4*>(src[i] + min(k, H - 8));
      v[i] = (k < H) ? w : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto stage = [&](int buf, const uint4 (&v)[kRChunks]) {
#pragma unroll
    for (int i = 0; i < kRChunks; ++i) {
      uint16_t* d = isb[i] ? &sb[buf][drow[i]][dcol[i]] : &sa[buf][drow[i]][dcol[i]];
      *reinterpret_cast<uint4*>(d) = v[i];
    }
  };
  f32x16_t acc[2];
  double accd[2][16];
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc[n][i] = 0.f;
      accd[n][i] = 0.0;
    }
  auto compute = [&](int kt, int buf) {
#pragma unroll
    for (int kk = 0; kk < kRK; kk += 16) {
      const int kc = kk + 8 * (lane >> 5);
      const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(&sa[buf][wm + (lane & 31)][kc]);
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(&sb[buf][wn + 32 * n + (lane & 31)][kc]);
        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[n], 0, 0, 0);
      }
    }
    if ((kt & 1) == 1 || kt + 1 == nk) {                 // every 128 of K
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          accd[n][i] += (double)acc[n][i];
          acc[n][i] = 0.f;
        }
    }
  };
  uint4 v0[kRChunks], v1[kRChunks];
  load(0, v0);
  load(min(1, nk - 1), v1);
  float bpre[2];                                         // bias, loaded before the K loop (never null)
#pragma unroll
  for (int n = 0; n < 2; ++n) bpre[n] = bias[min(n0 + wn + 32 * n + (lane & 31), E - 1)];
  for (int kt = 0; kt < nk; kt += 2) {
    stage(0, v0);
    __syncthreads();
    load(min(kt + 2, nk - 1), v0);
    compute(kt, 0);
    if (kt + 1 < nk) {
      stage(1, v1);
      __syncthreads();
      load(min(kt + 3, nk - 1), v1);
      compute(kt + 1, 1);
    }
  }

  // epilogue: lane holds rows 8*(i/4) + 4*(lane/32) + i%4 of column lane%32
  bool bad = false;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int e = n0 + wn + 32 * n + (lane & 31);
    const double b = (e < E) ? (double)bpre[n] : 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = m0 + wm + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      const double v = accd[n][i] + b;
      if (e < E && t < T) {
        z[size_t(t) * E + e] = v;
        if (!isfinite(v)) bad = true;
      }
      // maximum over the 4 consecutive experts of lanes 4q..4q+3, taken on
      // the values rounded up to binary32 (rounding up is monotone, so this
      // is the rounded-up maximum)
      float m = (e < E && !isnan(v)) ? f64_to_f32_up(v) : -INFINITY;
      m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                       __builtin_bit_cast(int, -INFINITY), __builtin_bit_cast(int, m), 0xB1, 0xf, 0xf, false)));
      m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                       __builtin_bit_cast(int, -INFINITY), __builtin_bit_cast(int, m), 0x4E, 0xf, 0xf, false)));
      if ((lane & 3) == 0 && t < T && e < E) gmax[size_t(t) * ((E + 3) / 4) + (e >> 2)] = m;
    }
  }
  if (bad) atomicOr(dev_flag, kDevNonFinite);

  if (nb == 0) {          // ||x_t||^2 for this block's tokens, 16 per wave
    for (int r = 0; r < kRM / 8; ++r) {
      const int t = m0 + wave * (kRM / 8) + r;
      if (t >= T) break;
      double q = 0.0;   // exact squares summed in binary64 (no underflow)
      for (int c = lane; c < H / 8; c += 64) {
        const uint4 v = *reinterpret_cast<const uint4*>(X + size_t(t) * H + c * 8);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const double lo = bf16_lo(w[j]), hi = bf16_hi(w[j]);
          q = fma(lo, lo, q);
          q = fma(hi, hi, q);
        }
      }
      q = wave_sum_f64(q);
      if (lane == 0) xnorm[t] = q;
    }
  }
}

// ---------------------------------------------------------------------------
// Large batches (T >= 512, H >= 128): 256-token x 256-expert tiles, 4 waves
// of 128 x 128 (256 fp32 accumulators per lane, one wave per SIMD), 32-wide
// K slices.  Operands go from memory straight into LDS with the direct
// 16-byte LDS loads (no register staging, no LDS store instructions), into a
// ring of 4 slices (128 KB): slice k + 3 is requested while slice k is
// multiplied.  Each wave's half-step interleaves its 16 MFMAs with the 8
// operand reads for the next half-step and the 8 slice loads, so the LDS
// and memory requests of the 4 waves are spread over the MFMA time instead
// of arriving in one burst after every barrier (that burst alone cost 15 %
// of the loop).  The LDS rows (64 bytes) hold their four 16-byte pieces in
// an XOR order that keeps every group of 8 or 16 consecutive lanes of an
// operand read on distinct banks.  Tiles are dealt to the 8 XCDs as in the
// small kernel.  The 256 accumulators per lane leave no room for binary64
// partial sums: each logit is accumulated in the MFMA's fp32 accumulator
// over all of H and converted once.  Rounding model: H/16 instructions of
// K = 16, each counted as at most 17 binary32 roundings (d32 = 17 H / 16),
// then the binary64 bias addition (d64 = 1).  The wider bound only moves
// more near-ties into the selection's exact refinement.  The group maxima
// go through LDS so they leave as 16-byte row pieces.
constexpr int kGM = 256, kGN = 256, kGK = 32, kGStages = 4;
constexpr int kGThreads = 256;
constexpr int kGOpBytes = kGM * kGK * 2;                 // one operand of one slice: 16 KB
constexpr int kGStage = 2 * kGOpBytes;
constexpr int kGLds = kGStages * kGStage;                // 128 KB of dynamic LDS
constexpr int kBigT = 512;                               // smallest batch that takes the big tiles
constexpr int kBigMinH = 4 * kGK;                        // the K loop keeps 3 slices in flight

// XOR order of the four 16-byte pieces of LDS row r (bits 1..4 of r)
__device__ __forceinline__ int gpiece(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// Direct load of 16 bytes per lane from sbase + voff into LDS at m0 + 16 lane.
// The compiler cannot see the memory instruction inside the asm, so the asm
// supplies the wait states its operands may need: 5 when a vector
// instruction (v_readlane, v_readfirstlane, as in register-spill restores)
// has just written the base SGPRs or M0, which also covers the one that M0
// needs after a scalar write.
__device__ __forceinline__ void dma16(uint32_t voff, const void* sbase, uint32_t lds_addr) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds_addr)
               : "memory");
}

// K loop of one 256 x 256 tile on 4 waves of 128 x 128 (see above).  The
// operands are rows of two row sets: A row r is 16 bytes per lane at
// xa + voa[j] (rows 16 (4 w + j) + lane / 4 of wave w), B likewise from xb +
// vob[j]; the base pointers are wave-uniform and advance 32 elements per
// slice.  A wave multiplies A rows wm .. wm + 127 with the B rows brow(b) ..
// brow(b) + 31, b = 0..3.  On return every LDS read and slice load of the
// block is complete and the ring may be reused.
template <typename BRow>
__device__ __forceinline__ void big_tile_kloop(uint8_t* glds, int wave, int lane, int nk,
                                               const uint16_t* xa, const uint16_t* xb,
                                               const uint32_t (&voa)[4], const uint32_t (&vob)[4],
                                               int wm, BRow brow, f32x16_t (&acc)[4][4]) {
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)glds;
  // operand reads: row (lane & 31) of a 32-row group, logical piece 2 s + (lane >> 5)
  const int pc = (lane >> 5) ^ gpiece(lane & 31);
  const uint32_t lb0 = (lane & 31) * 64 + pc * 16, lb1 = (lane & 31) * 64 + (pc ^ 2) * 16;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;
  bf16x8_t f0a[4], f0b[4], f1a[4], f1b[4];
  auto issue = [&](int kt, int stage) {
    const uint32_t base = lds0 + stage * kGStage + wave * 4096;
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(voa[j], xa + kt * kGK, base + j * 1024);
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(vob[j], xb + kt * kGK, base + kGOpBytes + j * 1024);
  };
  // one half-step: 16 MFMAs on (fa, fb), b-major (the operand read last is
  // used last), interleaved with the 8 operand reads of the other register
  // set and, when asked, the 8 loads of slice dk
  auto half = [&](const bf16x8_t (&fa)[4], const bf16x8_t (&fb)[4], auto rd, int rstage, uint32_t lb,
                  bf16x8_t (&ga)[4], bf16x8_t (&gb)[4], auto dm, int dk, int dstage) {
    const uint8_t* p = glds + rstage * kGStage + lb;
    const uint32_t dbase = lds0 + dstage * kGStage + wave * 4096;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      if constexpr (decltype(dm)::value) {
        if (g < 4) dma16(voa[g], xa + dk * kGK, dbase + g * 1024);
        else dma16(vob[g - 4], xb + dk * kGK, dbase + kGOpBytes + (g - 4) * 1024);
      }
      if constexpr (decltype(rd)::value) {
        if (g < 4) ga[g] = *reinterpret_cast<const bf16x8_t*>(p + (wm + 32 * g) * 64);
        else gb[g - 4] = *reinterpret_cast<const bf16x8_t*>(p + kGOpBytes + brow(g - 4) * 64);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int idx = 2 * g + q, b = idx >> 2, a = idx & 3;
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using On = std::integral_constant<bool, true>;
  using Off = std::integral_constant<bool, false>;
  // K loop: at the barrier of slice k every wave's loads of slice k + 1 have
  // landed (vmcnt counts this wave's loads in order; slice k + 2 may still be
  // in flight) and every wave has finished reading slice k - 1, whose ring
  // slot then takes slice k + 3.
  issue(0, 0);
  issue(1, 1);
  issue(2, 2);
  asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int a = 0; a < 4; ++a) f0a[a] = *reinterpret_cast<const bf16x8_t*>(glds + lb0 + (wm + 32 * a) * 64);
#pragma unroll
  for (int b = 0; b < 4; ++b) f0b[b] = *reinterpret_cast<const bf16x8_t*>(glds + kGOpBytes + lb0 + brow(b) * 64);
  int k = 0;
  for (; k + 3 < nk; ++k) {
    const int S = k & 3;
    half(f0a, f0b, On{}, S, lb1, f1a, f1b, Off{}, 0, 0);
    asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
    half(f1a, f1b, On{}, (S + 1) & 3, lb0, f0a, f0b, On{}, k + 3, (S + 3) & 3);
  }
  // the last three slices: nothing more to load
  half(f0a, f0b, On{}, k & 3, lb1, f1a, f1b, Off{}, 0, 0);
  asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
  half(f1a, f1b, On{}, (k + 1) & 3, lb0, f0a, f0b, Off{}, 0, 0);
  ++k;
  half(f0a, f0b, On{}, k & 3, lb1, f1a, f1b, Off{}, 0, 0);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  half(f1a, f1b, On{}, (k + 1) & 3, lb0, f0a, f0b, Off{}, 0, 0);
  ++k;
  half(f0a, f0b, On{}, k & 3, lb1, f1a, f1b, Off{}, 0, 0);
  half(f1a, f1b, Off{}, 0, lb0, f0a, f0b, Off{}, 0, 0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // the ring is free from here on
}

template <typename ZT>   // logits stored in binary64, or in binary32 for the selection (one more rounding)
__global__ __launch_bounds__(kGThreads, 1) void router_gemm_big_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ R, const float* __restrict__ bias,
    int T, int H, int E, int nm, int nn, int nper, ZT* __restrict__ z, float* __restrict__ gmax,
    double* __restrict__ xnorm, int* __restrict__ dev_flag) {
  extern __shared__ __attribute__((aligned(16))) uint8_t glds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int xcd = blockIdx.x % 8, loc = blockIdx.x / 8;
  const int nb = xcd * nper + loc / nm, mb = loc % nm;
  if (nb >= nn) return;                                  // whole block
  const int m0 = mb * kGM, n0 = nb * kGN;
  const int wm = (wave & 1) * 128, wn = (wave >> 1) * 128;
  // slice loads: wave w, instruction j moves rows 16 (4 w + j) .. +15 of an
  // operand; lane l lands in LDS slot l (row l / 4, stored piece l % 4).
  // Rows past T or E repeat the last row (never stored).
  uint32_t voa[4], vob[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 16 * (4 * wave + j) + (lane >> 2);
    const int c = (lane & 3) ^ gpiece(r);
    voa[j] = uint32_t((min(m0 + r, T - 1) - m0) * H + c * 8) * 2;
    vob[j] = uint32_t((min(n0 + r, E - 1) - n0) * H + c * 8) * 2;
  }
  const uint16_t* xa = X + size_t(m0) * H;
  const uint16_t* xb = R + size_t(n0) * H;
  float bpre[4];                                         // bias, loaded before the K loop (never null)
#pragma unroll
  for (int b = 0; b < 4; ++b) bpre[b] = bias[min(n0 + wn + 32 * b + (lane & 31), E - 1)];
  f32x16_t acc[4][4];
  big_tile_kloop(glds, wave, lane, H / kGK, xa, xb, voa, vob, wm, [&](int b) { return wn + 32 * b; }, acc);

  // epilogue: lane holds rows 8*(i/4) + 4*(lane/32) + i%4 of column lane%32
  // of each 32x32 accumulator; interior tiles skip every bounds check
  const bool full = m0 + kGM <= T && n0 + kGN <= E && (E % 16) == 0;   // block-uniform
  const size_t G4 = size_t(E + 3) / 4;
  float* sg = reinterpret_cast<float*>(glds);             // group maxima [256 tokens][64 groups]
  bool bad = false;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int el = wn + 32 * b + (lane & 31), e = n0 + el;
    const double bs = (double)bpre[b];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int tl = wm + 32 * a + 4 * (lane >> 5);
      double v[16];
      float f[16], d[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        v[i] = (double)acc[a][b][i] + bs;
        f[i] = isnan(v[i]) ? -INFINITY : f64_to_f32_up(v[i]);
      }
      // maximum over the 4 consecutive experts of lanes 4q..4q+3 (rounded up
      // values: rounding up is monotone, so this is the rounded-up maximum;
      // lanes past E hold a copy of expert E - 1)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        d[i] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, f[i]), 0xB1, 0xf, 0xf, false));
#pragma unroll
      for (int i = 0; i < 16; ++i) f[i] = d[i] > f[i] ? d[i] : f[i];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        d[i] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, f[i]), 0x4E, 0xf, 0xf, false));
#pragma unroll
      for (int i = 0; i < 16; ++i) f[i] = d[i] > f[i] ? d[i] : f[i];
      ZT* zb = z + size_t(m0 + tl) * E + min(e, E - 1);
      if (full) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          zb[size_t(8 * (i >> 2) + (i & 3)) * E] = (ZT)v[i];
          bad |= !isfinite(v[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 8 * (i >> 2) + (i & 3);
          if (e < E && m0 + tl + r < T) {
            zb[size_t(r) * E] = (ZT)v[i];
            bad |= !isfinite(v[i]);
          }
        }
      }
      if ((lane & 3) == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sg[(tl + 8 * (i >> 2) + (i & 3)) * 64 + (el >> 2)] = f[i];
      }
    }
  }
  if (bad) atomicOr(dev_flag, kDevNonFinite);
  __syncthreads();
  if (full) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int q = tid + kGThreads * u, tok = q >> 4, g4 = q & 15;
      *reinterpret_cast<float4*>(gmax + size_t(m0 + tok) * G4 + n0 / 4 + g4 * 4) =
          *reinterpret_cast<const float4*>(&sg[tok * 64 + g4 * 4]);
    }
  } else {
    for (int q = tid; q < kGM * 64; q += kGThreads) {
      const int tok = q >> 6, g = q & 63;
      if (m0 + tok < T && size_t(n0 / 4 + g) < G4) gmax[size_t(m0 + tok) * G4 + n0 / 4 + g] = sg[q];
    }
  }
  // ||x_t||^2 of this token tile: 64 groups of 4 tokens (one per wave), dealt
  // to the tile's first expert tiles (all groups to tile 0 when nn = 1)
  for (int g = nb; g < kGM / 4; g += nn) {
    const int t = m0 + g * 4 + wave;
    if (t >= T) break;
    double q = 0.0;   // exact squares summed in binary64 (no underflow)
    for (int c = lane; c < H / 8; c += 64) {
      const uint4 xv = *reinterpret_cast<const uint4*>(X + size_t(t) * H + c * 8);
      const uint32_t w[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const double lo = bf16_lo(w[j]), hi = bf16_hi(w[j]);
        q = fma(lo, lo, q);
        q = fma(hi, hi, q);
      }
    }
    q = wave_sum_f64(q);
    if (lane == 0) xnorm[t] = q;
  }
}

bool router_uses_mfma(const Layer& L, int T) {
  return L.d.act_dtype == MOE_BF16 && T >= 16 && (L.d.hidden % kBK) == 0;
}

bool router_uses_big_tiles(const Layer& L, int T) {
  return router_uses_mfma(L, T) && T >= kBigT && L.d.hidden >= kBigMinH;
}

bool router_logits_f32(const Layer& L, int T) { return router_uses_big_tiles(L, T); }

// The big-tile kernels take kGLds bytes of dynamic LDS; allow it once per
// process (the attribute belongs to the function, on every device).
static hipError_t big_lds_attributes() {
  static const hipError_t err = [] {
    const void* fns[] = {reinterpret_cast<const void*>(&router_gemm_big_kernel<float>),
                         reinterpret_cast<const void*>(&router_gemm_big_kernel<double>)};
    for (const void* f : fns) {
      const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kGLds);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }();
  return err;
}

hipError_t launch_router_gemm(const Layer& L, const void* x, int T, void* z, bool z32, float* gmax,
                              double* xnorm, hipStream_t s) {
  const int H = L.d.hidden, E = L.d.n_experts;
  const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
  const uint16_t* rb = reinterpret_cast<const uint16_t*>(L.router_eh);
  if (router_uses_big_tiles(L, T)) {
    if (hipError_t ea = big_lds_attributes(); ea != hipSuccess) return ea;
    const int nm = (T + kGM - 1) / kGM, nn = (E + kGN - 1) / kGN, nper = (nn + 7) / 8;
    if (z32)
      hipLaunchKernelGGL(router_gemm_big_kernel<float>, dim3(8 * nper * nm), dim3(kGThreads), kGLds, s, xb, rb,
                         router_bias_or_zero(L), T, H, E, nm, nn, nper, static_cast<float*>(z), gmax,
                         xnorm, L.dev_flag);
    else
      hipLaunchKernelGGL(router_gemm_big_kernel<double>, dim3(8 * nper * nm), dim3(kGThreads), kGLds, s, xb, rb,
                         router_bias_or_zero(L), T, H, E, nm, nn, nper, static_cast<double*>(z), gmax,
                         xnorm, L.dev_flag);
    return hipGetLastError();
  }
  if (z32) return hipErrorInvalidValue;                  // binary32 logits only from the big tiles
  const int nm = (T + kRM - 1) / kRM, nn = (E + kRN - 1) / kRN;
  const int nper = (nn + 7) / 8;                         // expert tiles per XCD
  hipLaunchKernelGGL(router_gemm_kernel, dim3(8 * nper * nm), dim3(kRThreads), 0, s, xb, rb,
                     router_bias_or_zero(L), T, H, E, nm, nn, nper, static_cast<double*>(z), gmax, xnorm,
                     L.dev_flag);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router for a few tokens (2 <= T < 16: verify windows).  The contraction is
// still a stream of the whole router, so the goal is the streaming-read
// ceiling, not matrix throughput; MFMA only replaces the per-token wave
// reductions that a vector-ALU GEMV needs for each (token, expert) pair.
// Block = 16 experts x all T tokens (padded to 16) with v_mfma_f32_16x16x32_bf16;
// the 4 waves split H into quarters.  The MFMA operand layout wants 16
// different expert rows in every load instruction (64 B per row), which
// streams poorly; for the common hidden sizes the kernel instead loads each
// row quarter with 512-byte-contiguous instructions (all of them issued up
// front) and transposes it through a per-wave LDS buffer in two phases, the
// second phase's data arriving while the first is multiplied.
// Each MFMA's fp32 result (a sum of 32 exact products) is added into binary64
// at once, and the 4 quarters, then the bias, are added in binary64:
// d32 = 33, d64 = ceil(H / 128) + 4.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int kSkQ = 16;     // MFMAs (of K = 32) per wave per batch

__device__ __forceinline__ void skinny_epilogue(double (*red)[16][17], const uint16_t* X,
                                                float bias_v, int T, int H, int E, int n0,
                                                double* z, float* gmax, double* xnorm, int* dev_flag);
// Bias of expert e (clamped: lanes past E are never stored), loaded at the
// start of the kernel; the pointer is never null (the layer passes zeros),
// because a load under a null-pointer test in the epilogue cost every block
// one more memory round trip at its end.
__device__ __forceinline__ float skinny_bias(const float* bias, int e, int E) {
  return bias[min(e, E - 1)];
}

bool router_uses_skinny(const Layer& L, int T) {
  return L.d.act_dtype == MOE_BF16 && T >= 2 && T < 16 && (L.d.hidden % 32) == 0;
}

__global__ __launch_bounds__(256) void router_skinny_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ R, const float* __restrict__ bias,
    int T, int H, int E, double* __restrict__ z, float* __restrict__ gmax,
    double* __restrict__ xnorm, int* __restrict__ dev_flag) {
  __shared__ double red[4][16][17];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16;
  const int nq = H / 32;
  const int qpw = (nq + 3) / 4;
  const int q0 = wave * qpw, q1 = min(nq, q0 + qpw);
  const int tr = lane & 15;
  // operand layout of 16x16x32: lane l holds row / column l % 16 and the 8
  // consecutive K elements starting at 8 * (l / 16)
  const uint16_t* pb = R + size_t(min(n0 + tr, E - 1)) * H + 8 * (lane >> 4);
  const uint16_t* pa = X + size_t(min(tr, T - 1)) * H + 8 * (lane >> 4);
  const float bias_v = skinny_bias(bias, n0 + (tid & 15), E);
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int qb = q0; qb < q1; qb += kSkQ) {
    uint4 b[kSkQ], xa[kSkQ];
#pragma unroll
    for (int i = 0; i < kSkQ; ++i) b[i] = load_nt(pb + 32 * min(qb + i, q1 - 1));
#pragma unroll
    for (int i = 0; i < kSkQ; ++i) xa[i] = *reinterpret_cast<const uint4*>(pa + 32 * min(qb + i, q1 - 1));
#pragma unroll
    for (int i = 0; i < kSkQ; ++i) {
      if (qb + i < q1) {                                   // wave-uniform
        f32x4_t d = {0.f, 0.f, 0.f, 0.f};                   // rows past T: token T-1 again, never stored
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xa[i]),
                                                     __builtin_bit_cast(bf16x8_t, b[i]), d, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += (double)d[r];
      }
    }
  }
  // D layout: lane l holds expert column l % 16, token rows 4 * (l / 16) + r
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][4 * (lane >> 4) + r][lane & 15] = acc[r];
  __syncthreads();
  skinny_epilogue(red, X, bias_v, T, H, E, n0, z, gmax, xnorm, dev_flag);
}

// The shared epilogue of both few-token kernels: sum the 4 quarters in
// order, add the bias, write logits and 4-expert maxima, flag non-finite
// logits; block 0 also writes ||x_t||^2.
__device__ __forceinline__ void skinny_epilogue(double (*red)[16][17], const uint16_t* X,
                                                float bias_v, int T, int H, int E, int n0,
                                                double* z, float* gmax, double* xnorm, int* dev_flag) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = tid >> 4, el = tid & 15, e = n0 + el;
  double v = ((red[0][t][el] + red[1][t][el]) + red[2][t][el]) + red[3][t][el];
  v += (double)bias_v;
  const bool live = e < E && t < T;
  if (live) z[size_t(t) * E + e] = v;
  if (live && !isfinite(v)) atomicOr(dev_flag, kDevNonFinite);
  double m = (e < E && !isnan(v)) ? v : -INFINITY;
  m = fmax(m, dpp_f64<0xB1, 0xf>(m, -INFINITY));
  m = fmax(m, dpp_f64<0x4E, 0xf>(m, -INFINITY));
  if ((el & 3) == 0 && live) gmax[size_t(t) * ((E + 3) / 4) + (e >> 2)] = f64_to_f32_up(m);
  if (blockIdx.x == 0) {
    for (int tt = wave; tt < T; tt += 4) {
      double q = 0.0;   // exact squares summed in binary64 (no underflow)
      for (int c = lane; c < H / 8; c += 64) {
        const uint4 xv = *reinterpret_cast<const uint4*>(X + size_t(tt) * H + c * 8);
        const uint32_t w[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const double lo = bf16_lo(w[j]), hi = bf16_hi(w[j]);
          q = fma(lo, lo, q);
          q = fma(hi, hi, q);
        }
      }
      q = wave_sum_f64(q);
      if (lane == 0) xnorm[tt] = q;
    }
  }
}

template <int HH>
__global__ __launch_bounds__(256) void router_skinny_lds_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ R, const float* __restrict__ bias,
    int T, int E, double* __restrict__ z, float* __restrict__ gmax,
    double* __restrict__ xnorm, int* __restrict__ dev_flag) {
  constexpr int NP = 2;                     // phases per row quarter
  constexpr int PE = (HH / 4) / NP;         // elements per row per phase
  constexpr int LPR = PE / 8;               // lanes per row in one load instruction
  constexpr int RPI = 64 / LPR;             // rows per load instruction
  constexpr int NI = 16 / RPI;              // load instructions per phase
  constexpr int QP = PE / 32;               // MFMAs per phase
  static_assert(LPR <= 64 && 64 % LPR == 0 && QP >= 1, "unsupported hidden size");
  __shared__ __attribute__((aligned(16))) uint16_t sr[4][16][PE + 8];
  __shared__ double red[4][16][17];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16;
  const int tr = lane & 15, g = lane >> 4;
  const int kw = wave * (HH / 4);
  uint4 b[NP][NI];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int i = 0; i < NI; ++i)
      b[p][i] = load_nt(R + size_t(min(n0 + i * RPI + lane / LPR, E - 1)) * HH + kw + p * PE + 8 * (lane % LPR));
  const float bias_v = skinny_bias(bias, n0 + (tid & 15), E);
  const uint16_t* pa = X + size_t(min(tr, T - 1)) * HH + kw;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    uint4 xa[QP];
#pragma unroll
    for (int q = 0; q < QP; ++q)   // rows past T repeat token T-1; their outputs are never stored
      xa[q] = *reinterpret_cast<const uint4*>(pa + p * PE + 32 * q + 8 * g);
    // the wave's LDS buffer is reused by the next phase (wave-level syncs
    // order the lanes' accesses; no workgroup barrier is needed)
#pragma unroll
    for (int i = 0; i < NI; ++i)
      *reinterpret_cast<uint4*>(&sr[wave][i * RPI + lane / LPR][8 * (lane % LPR)]) = b[p][i];
    wave_lds_sync();                                      // other lanes' writes before the reads
#pragma unroll
    for (int q = 0; q < QP; ++q) {
      const uint4 bv = *reinterpret_cast<const uint4*>(&sr[wave][tr][32 * q + 8 * g]);
      f32x4_t d = {0.f, 0.f, 0.f, 0.f};
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xa[q]),
                                                   __builtin_bit_cast(bf16x8_t, bv), d, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] += (double)d[r];
    }
    wave_lds_sync();                                      // all reads before the next phase's writes
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][4 * g + r][tr] = acc[r];
  __syncthreads();
  skinny_epilogue(red, X, bias_v, T, HH, E, n0, z, gmax, xnorm, dev_flag);
}

hipError_t launch_router_skinny(const Layer& L, const void* x, int T, double* z, float* gmax,
                                double* xnorm, hipStream_t s) {
  const int H = L.d.hidden, E = L.d.n_experts;
  const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
  const uint16_t* rb = reinterpret_cast<const uint16_t*>(L.router_eh);
  const dim3 grid((E + 15) / 16);
#define MOE_SKINNY_LDS(HV)                                                                        \
  if (H == HV) {                                                                                  \
    hipLaunchKernelGGL(router_skinny_lds_kernel<HV>, grid, dim3(256), 0, s, xb, rb, router_bias_or_zero(L), \
                       T, E, z, gmax, xnorm, L.dev_flag);                                         \
    return hipGetLastError();                                                                     \
  }
  MOE_SKINNY_LDS(512)
  MOE_SKINNY_LDS(1024)
  MOE_SKINNY_LDS(2048)
  MOE_SKINNY_LDS(4096)
#undef MOE_SKINNY_LDS
  hipLaunchKernelGGL(router_skinny_kernel, grid, dim3(256), 0, s, xb, rb, router_bias_or_zero(L), T, H, E, z,
                     gmax, xnorm, L.dev_flag);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grouped bf16 experts on MFMA (prefill chunks, large verify batches).  The
// token-expert pairs are sorted by expert and cut into tiles of 32 rows of
// one expert's segment; each tile is one MFMA M-tile.  Most experts of a
// 2048-token chunk receive 1-3 tokens, so most tiles are nearly empty and
// the kernels are bound by the expert-weight stream, which every tile reads
// once; the few experts with hundreds of tokens are where MFMA throughput
// matters.  So the weights are streamed the way that reads HBM best: each
// wave loads its own 32 weight rows in 128-byte row pieces (8 lanes per
// row), two K slices ahead of the slice being multiplied, and transposes
// them into the MFMA operand layout through LDS.
//
// gate/up: block = (64 intermediate channels, tile); waves 0-1 own 32 gate
//   channels each, waves 2-3 the matching up channels; the tile's gathered
//   token rows are staged through LDS (rows past the segment are zeros);
//   epilogue h = silu(a) * u in fp32, the up results passing through LDS.
// down: block = (128 output rows, tile); the tile's 32 rows of h (fp32) are
//   split into bf16 hi + lo parts in LDS (h = hi + lo to 2^-16 relative) and
//   multiplied by the same bf16 weights twice, so the down projection keeps
//   fp32-level accuracy.
constexpr int kGC = 64;              // gate (and up) channels per gate/up block
constexpr int kDR = 128;             // output rows per down block
constexpr int kKS = 64;              // K elements per slice
constexpr int kKP = kKS + 8;         // LDS row pitch (elements) of a slice

bool grouped_uses_mfma(const Layer& L, int T) {
  return L.d.expert_dtype == MOE_BF16 && L.d.act_dtype == MOE_BF16 && T >= 16 &&
         (L.d.hidden % 32) == 0 && (L.d.inter % 32) == 0 && L.d.inter <= 256;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne_dev(float f) {
  const uint32_t u = __float_as_uint(f);
  return uint16_t((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// 16 bytes at row + k (k a multiple of 8); zeros where k >= K (the address
// is clamped so the load stays inside the row).
__device__ __forceinline__ uint4 load_row_chunk(const uint16_t* row, int k, int K, bool live) {
  const uint4 v = load_nt(row + min(k, K - 8));
  return (live && k < K) ? v : make_uint4(0u, 0u, 0u, 0u);
}

// MT = 32-row sub-tiles per tile: 1 for the 32-row list, 2 for the 64-row
// list of experts with more than 32 tokens (their weights then stream once
// per 64 tokens instead of once per 32).
template <int MT>
__global__ __launch_bounds__(256) void gateup_mfma_kernel(GroupArgs a) {
  constexpr int TR = kTileRows * MT;                     // tile rows
  constexpr int XC = TR * (kKS / 8) / 256;               // x chunks per thread per slice
  __shared__ __attribute__((aligned(16))) uint16_t sw[2][2 * kGC][kKP];
  __shared__ __attribute__((aligned(16))) uint16_t sx[2][TR][kKP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, I = a.I;
  const uint16_t* W = reinterpret_cast<const uint16_t*>(wave < 2 ? a.wg : a.wu);
  const uint16_t* X = reinterpret_cast<const uint16_t*>(a.x);
  const int lr = lane >> 3, lc = lane & 7;               // weight loads: row lr + 8 i, chunk lc
  const int xc = tid & 7;                                // x loads: tile rows (tid >> 3) + 32 j, chunk xc
  const int nks = (H + kKS - 1) / kKS;
  const int* tl = (MT == 1) ? a.tiles : a.tiles_big;   // MT > 1: the big-tile list
  const int ntiles = tl[0];
  // work item w = (tile, channel block), tile-major.  Blocks are dealt to the
  // 8 XCDs round-robin, so XCD j takes a contiguous run of work items: a
  // tile's channel blocks (same token rows) and an expert's consecutive tiles
  // (same weights) then meet in one L2.
  const int nwork = ntiles * gridDim.x;
  const int lin = blockIdx.x + gridDim.x * blockIdx.y, nblk = gridDim.x * gridDim.y;
  const int per_xcd = (nwork + 7) / 8;
  for (int it = lin / 8; it < per_xcd; it += nblk / 8) {
    const int w = (lin & 7) * per_xcd + it;
    if (w >= nwork) break;                               // block-uniform
    const int ti = w / gridDim.x;
    const int ch0 = (w - ti * gridDim.x) * kGC;
    const int wc = ch0 + 32 * (wave & 1);                // first channel of this wave
    const int e = tl[1 + 2 * ti], r0 = tl[2 + 2 * ti];
    const int n = a.counts[e], seg = a.offsets[e];
    const int nrow = min(TR, n - r0);
    const uint16_t* px[XC];
    bool xlive[XC];
#pragma unroll
    for (int j = 0; j < XC; ++j) {
      const int xr = (tid >> 3) + 32 * j;
      xlive[j] = xr < nrow;
      px[j] = X + size_t(a.ptok[seg + r0 + min(xr, nrow - 1)]) * H;
    }
    const uint16_t* pw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pw[i] = W + (size_t(e) * I + min(wc + lr + 8 * i, I - 1)) * H;
    uint4 wA[4], wB[4], xA[XC], xB[XC];
#pragma unroll
    for (int i = 0; i < 4; ++i) wA[i] = load_row_chunk(pw[i], 8 * lc, H, true);
#pragma unroll
    for (int j = 0; j < XC; ++j) xA[j] = load_row_chunk(px[j], 8 * xc, H, xlive[j]);
#pragma unroll
    for (int i = 0; i < 4; ++i) wB[i] = load_row_chunk(pw[i], kKS + 8 * lc, H, true);
#pragma unroll
    for (int j = 0; j < XC; ++j) xB[j] = load_row_chunk(px[j], kKS + 8 * xc, H, xlive[j]);
    f32x16_t acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][i] = 0.f;
    // one K slice: stage it, refill its registers two slices ahead, multiply
    // (sub-tiles past the segment are skipped: a block-uniform test)
#define MOE_GU_SLICE(KT, WR, XR, BUF)                                                          \
    {                                                                                          \
      _Pragma("unroll") for (int i = 0; i < 4; ++i)                                            \
        *reinterpret_cast<uint4*>(&sw[BUF][32 * wave + lr + 8 * i][8 * lc]) = WR[i];           \
      _Pragma("unroll") for (int j = 0; j < XC; ++j)                                           \
        *reinterpret_cast<uint4*>(&sx[BUF][(tid >> 3) + 32 * j][8 * xc]) = XR[j];              \
      __syncthreads();                                                                         \
      const int kn = ((KT) + 2) * kKS;                                                         \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) WR[i] = load_row_chunk(pw[i], kn + 8 * lc, H, true); \
      _Pragma("unroll") for (int j = 0; j < XC; ++j) XR[j] = load_row_chunk(px[j], kn + 8 * xc, H, xlive[j]); \
      _Pragma("unroll") for (int q = 0; q < kKS / 16; ++q) {                                   \
        const int kk = 16 * q + 8 * (lane >> 5);                                               \
        const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(&sw[BUF][32 * wave + (lane & 31)][kk]); \
        _Pragma("unroll") for (int m = 0; m < MT; ++m) {                                       \
          if (m == 0 || 32 * m < nrow) {                                                       \
            const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(&sx[BUF][32 * m + (lane & 31)][kk]); \
            acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[m], 0, 0, 0);         \
          }                                                                                    \
        }                                                                                      \
      }                                                                                        \
    }
    for (int kt = 0; kt < nks; kt += 2) {
      MOE_GU_SLICE(kt, wA, xA, 0)
      if (kt + 1 < nks) MOE_GU_SLICE(kt + 1, wB, xB, 1)
    }
#undef MOE_GU_SLICE
    // epilogue: D rows 8 (i / 4) + 4 (lane / 32) + i % 4 (tokens), column lane % 32 (channel)
    float* su = reinterpret_cast<float*>(&sw[0][0][0]);   // [32][kGC + 1] up results of one sub-tile
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m > 0 && 32 * m >= nrow) break;                 // block-uniform
      __syncthreads();
      if (wave >= 2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          su[r * (kGC + 1) + 32 * (wave - 2) + (lane & 31)] = acc[m][i];
        }
      }
      __syncthreads();
      if (wave < 2) {
        const int ch = wc + (lane & 31);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 32 * m + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          if (r < nrow && ch < I) {
            const float g = acc[m][i], u = su[(r - 32 * m) * (kGC + 1) + 32 * wave + (lane & 31)];
            a.hm[size_t(seg + r0 + r) * I + ch] = g / (1.0f + expf(-g)) * u;
          }
        }
      }
    }
    __syncthreads();   // LDS reuse by the next tile
  }
}

template <int NS>   // K slices of 64 (I <= 64 NS); 32-row tiles
__global__ __launch_bounds__(256) void down_mfma_kernel(GroupArgs a) {
  constexpr int KP = NS * kKS + 8;
  __shared__ __attribute__((aligned(16))) uint16_t shi[kTileRows][KP];
  __shared__ __attribute__((aligned(16))) uint16_t slo[kTileRows][KP];
  __shared__ __attribute__((aligned(16))) uint16_t sw[4][32][kKP];   // wave-private slices
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, I = a.I;
  const int ow = blockIdx.x * kDR + 32 * wave;           // first output row of this wave
  const int lr = lane >> 3, lc = lane & 7;
  const uint16_t* WD = reinterpret_cast<const uint16_t*>(a.wd);
  const int* tl = a.tiles;                               // the 32-row tile list
  const int ntiles = tl[0];
  for (int ti = blockIdx.y; ti < ntiles; ti += gridDim.y) {
    const int e = tl[1 + 2 * ti], r0 = tl[2 + 2 * ti];
    const int n = a.counts[e], seg = a.offsets[e];
    const int nrow = min(kTileRows, n - r0);
    // the wave's 32 weight rows, all of K, in flight at once (read once per tile)
    uint4 w[NS][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint16_t* row = WD + (size_t(e) * H + min(ow + lr + 8 * i, H - 1)) * I;
#pragma unroll
      for (int sl = 0; sl < NS; ++sl) w[sl][i] = load_row_chunk(row, sl * kKS + 8 * lc, I, true);
    }
    {
      // h rows of the tile -> bf16 hi/lo (rows past the segment and columns past I: zeros)
      for (int q = tid; q < kTileRows * (NS * kKS / 4); q += 256) {
        const int r = q / (NS * kKS / 4), c = (q - r * (NS * kKS / 4)) * 4;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (r < nrow && c < I) v = *reinterpret_cast<const float4*>(a.hm + size_t(seg + r0 + r) * I + c);
        const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint16_t hi = f32_to_bf16_rne_dev(vv[j]);
          const float rem = vv[j] - __uint_as_float(uint32_t(hi) << 16);
          shi[r][c + j] = hi;
          slo[r][c + j] = f32_to_bf16_rne_dev(rem);
        }
      }
      __syncthreads();
      f32x16_t acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int sl = 0; sl < NS; ++sl) {
        // the wave's private slice buffer, reused by every slice (wave-level
        // syncs order the lanes' accesses; no workgroup barrier is needed)
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&sw[wave][lr + 8 * i][8 * lc]) = w[sl][i];
        wave_lds_sync();                                  // other lanes' writes before the reads
#pragma unroll
        for (int q = 0; q < kKS / 16; ++q) {
          const int kk = 16 * q + 8 * (lane >> 5);
          const bf16x8_t ah = *reinterpret_cast<const bf16x8_t*>(&shi[lane & 31][sl * kKS + kk]);
          const bf16x8_t al = *reinterpret_cast<const bf16x8_t*>(&slo[lane & 31][sl * kKS + kk]);
          const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(&sw[wave][lane & 31][kk]);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bv, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bv, acc, 0, 0, 0);
        }
        wave_lds_sync();                                  // all reads before the next slice's writes
      }
      const int o = ow + (lane & 31);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        if (r < nrow && o < H) a.y[size_t(seg + r0 + r) * H + o] = acc[i];
      }
    }
    __syncthreads();   // h staging reuse by the next tile
  }
}

// ---------------------------------------------------------------------------
// Down projection of the big tiles (experts with more than 32 tokens) as a
// small GEMM: block = (128 output rows, tile of TM tokens); per K slice of
// 32 the tile's h (fp32) is split into bf16 hi + lo in LDS and both parts
// meet the same bf16 weight slice, staged once in LDS for all waves (the
// 32-row kernel gives each wave its own weight rows, which would repeat
// them per 32-row part of a larger tile).  Both operands are K-contiguous; LDS rows hold 32 K
// elements (64 B) with 16-byte chunk c of row r at chunk c ^ ((r >> 1) & 3),
// so the staging writes and the operand reads of a wave hit distinct banks.
// The accumulation order (K ascending in steps of 16, hi then lo, fp32) is
// the one of the 32-row kernel.
constexpr int kHotBK = 32;

__device__ __forceinline__ int hot_pos(int row, int chunk) {
  return row * kHotBK + ((chunk ^ ((row >> 1) & 3)) << 3);
}

template <int TM>   // tokens per tile: waves (token half, output half) hold TM/2 x 64
__global__ __launch_bounds__(256, 2) void down_tile_kernel(GroupArgs a) {
  constexpr int MB = TM / 64;                      // 32-row blocks per wave
  constexpr int HR = TM / 64;                      // h rows per staging thread
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][(2 * TM + 128) * kHotBK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, I = a.I;
  const int* tl = a.tiles_big;
  const int o0 = blockIdx.x * 128;
  const uint16_t* WD = reinterpret_cast<const uint16_t*>(a.wd);
  const int sr = tid >> 2, sc = tid & 3;           // staging: chunk sc of rows sr + 64 i
  const int wm = (wave & 1) * (TM / 2), wn = (wave >> 1) * 64;
  const int rl = lane & 31, hk = lane >> 5;
  const int nk = I / kHotBK;
  const int ntiles = tl[0];
  for (int ti = blockIdx.y; ti < ntiles; ti += gridDim.y) {
    const int e = tl[1 + 2 * ti], r0 = tl[2 + 2 * ti];
    const int n = a.counts[e], seg = a.offsets[e];
    const int nrow = min(TM, n - r0);
    const float* hsrc[HR];
    const uint16_t* wsrc[2];
#pragma unroll
    for (int i = 0; i < HR; ++i)              // rows past the tile repeat its last row
      hsrc[i] = a.hm + size_t(seg + r0 + min(sr + 64 * i, nrow - 1)) * I + sc * 8;
#pragma unroll
    for (int i = 0; i < 2; ++i) wsrc[i] = WD + (size_t(e) * H + min(o0 + sr + 64 * i, H - 1)) * I + sc * 8;
    f32x16_t acc[MB][2];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[m][b][i] = 0.f;
    float4 hf[HR][2];
    uint4 wv[2];
    auto gload = [&](int kt) {
      const int ko = kt * kHotBK;
#pragma unroll
      for (int i = 0; i < HR; ++i) {
        hf[i][0] = *reinterpret_cast<const float4*>(hsrc[i] + ko);
        hf[i][1] = *reinterpret_cast<const float4*>(hsrc[i] + ko + 4);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) wv[i] = load_nt(wsrc[i] + ko);
    };
    auto lstore = [&](int buf) {
#pragma unroll
      for (int i = 0; i < HR; ++i) {
        const float v[8] = {hf[i][0].x, hf[i][0].y, hf[i][0].z, hf[i][0].w,
                            hf[i][1].x, hf[i][1].y, hf[i][1].z, hf[i][1].w};
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint16_t h0 = f32_to_bf16_rne_dev(v[2 * j]), h1 = f32_to_bf16_rne_dev(v[2 * j + 1]);
          const uint16_t l0 = f32_to_bf16_rne_dev(v[2 * j] - __uint_as_float(uint32_t(h0) << 16));
          const uint16_t l1 = f32_to_bf16_rne_dev(v[2 * j + 1] - __uint_as_float(uint32_t(h1) << 16));
          hi[j] = uint32_t(h0) | (uint32_t(h1) << 16);
          lo[j] = uint32_t(l0) | (uint32_t(l1) << 16);
        }
        const int r = sr + 64 * i;
        *reinterpret_cast<uint4*>(&lds[buf][hot_pos(r, sc)]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        *reinterpret_cast<uint4*>(&lds[buf][hot_pos(TM + r, sc)]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) *reinterpret_cast<uint4*>(&lds[buf][hot_pos(2 * TM + sr + 64 * i, sc)]) = wv[i];
    };
    __syncthreads();                               // LDS reuse by the previous tile
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      gload(min(kt + 1, nk - 1));
#pragma unroll
      for (int q = 0; q < kHotBK / 16; ++q) {
        const int ck = 2 * q + hk;
        bf16x8_t ah[MB], al[MB], bv[2];
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          ah[m] = *reinterpret_cast<const bf16x8_t*>(&lds[buf][hot_pos(wm + 32 * m + rl, ck)]);
          al[m] = *reinterpret_cast<const bf16x8_t*>(&lds[buf][hot_pos(TM + wm + 32 * m + rl, ck)]);
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) bv[b] = *reinterpret_cast<const bf16x8_t*>(&lds[buf][hot_pos(2 * TM + wn + 32 * b + rl, ck)]);
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            acc[m][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[m], bv[b], acc[m][b], 0, 0, 0);
            acc[m][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[m], bv[b], acc[m][b], 0, 0, 0);
          }
      }
      if (kt + 1 < nk) lstore(buf ^ 1);
      __syncthreads();
    }
    // D rows 8 (i / 4) + 4 (lane / 32) + i % 4 (tokens), column lane % 32 (output row)
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int o = o0 + wn + 32 * b + rl;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = wm + 32 * m + 8 * (i >> 2) + 4 * hk + (i & 3);
          if (r < nrow && o < H) a.y[size_t(seg + r0 + r) * H + o] = acc[m][b][i];
        }
      }
  }
}

// The 32-row tiles first (most experts: bound by the weight stream), then
// the 64-row tiles of the hot experts (gate/up as 2 sub-tiles, down as a
// small GEMM).
hipError_t launch_grouped_mfma(const GroupArgs& a, hipStream_t s) {
  constexpr int MB = kBigTileRows / kTileRows;
  const int gy = 2048, gyb = 256;
  const int ns = (a.I + kKS - 1) / kKS;
  if (ns > 4) return hipErrorInvalidValue;
  const dim3 g1((a.I + kGC - 1) / kGC, gy), g1b((a.I + kGC - 1) / kGC, gyb);
  const dim3 g2((a.H + kDR - 1) / kDR, gy);
  hipLaunchKernelGGL(gateup_mfma_kernel<1>, g1, dim3(256), 0, s, a);
  hipLaunchKernelGGL(gateup_mfma_kernel<MB>, g1b, dim3(256), 0, s, a);
  if (ns == 1) hipLaunchKernelGGL((down_mfma_kernel<1>), g2, dim3(256), 0, s, a);
  else if (ns == 2) hipLaunchKernelGGL((down_mfma_kernel<2>), g2, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((down_mfma_kernel<4>), g2, dim3(256), 0, s, a);
  hipLaunchKernelGGL(down_tile_kernel<kBigTileRows>, dim3((a.H + 127) / 128, gyb), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
