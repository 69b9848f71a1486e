// Internal declarations of libmoe: layer object, workspace layout, device
// helpers shared by the kernels, and the launchers each kernel file exports.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <vector>

#include "../../include/moe.h"

namespace moe {

// ------------------------------------------------------------------ limits
constexpr int kMaxK = 32;
constexpr int kMaxPairs = 256;  // token-expert pairs of the few-token expert path
constexpr int kMaxH = 8192;
constexpr int kMaxI = 4096;
constexpr int kRouterWaves = 4;      // router block = 4 waves, one expert row per wave
constexpr int kSelectThreads = 512;
constexpr int kSelectMaxCand = 1024;  // candidates held in LDS at once

// device fault bits (moe_device_error)
constexpr int kDevBadIndex = 1;
constexpr int kDevDupIndex = 2;
constexpr int kDevNonFinite = 4;
constexpr int kDevInternal = 8;

// Fetch every 64-byte line of a kernel's arguments (the first BYTES bytes)
// at once: the compiler reads the arguments with scalar loads as it needs
// them, and each line it reaches first misses the scalar cache in turn, a
// round trip per line on the kernel's critical path (0.3 us of a 344-byte
// argument block, measured on the batch-1 decode chain).  Scalar loads of
// one dword per line, waited for in the same statement; offsets stay below
// BYTES.
template <int BYTES>
__device__ __forceinline__ void kernarg_lines() {
  constexpr int L = (BYTES + 63) / 64;
  static_assert(L >= 1 && L <= 6, "at most six lines");
  constexpr int o1 = (L > 1 ? 1 : 0) * 64, o2 = (L > 2 ? 2 : 0) * 64, o3 = (L > 3 ? 3 : 0) * 64;
  constexpr int o4 = (L > 4 ? 4 : 0) * 64, o5 = (L > 5 ? 5 : 0) * 64;
  const char* ka = (const char*)__builtin_amdgcn_kernarg_segment_ptr();   // (constant address space)
  unsigned d0, d1, d2, d3, d4, d5;
  asm volatile(
      "s_load_dword %0, %6, 0\n"
      "s_load_dword %1, %6, %7\n"
      "s_load_dword %2, %6, %8\n"
      "s_load_dword %3, %6, %9\n"
      "s_load_dword %4, %6, %10\n"
      "s_load_dword %5, %6, %11\n"
      "s_waitcnt lgkmcnt(0)"
      : "=s"(d0), "=s"(d1), "=s"(d2), "=s"(d3), "=s"(d4), "=s"(d5)
      : "s"(ka), "i"(o1), "i"(o2), "i"(o3), "i"(o4), "i"(o5)
      : "memory");
}

// ------------------------------------------------------------------ layer
// The hot-expert region (moe_layer_set_hot_experts): compact copies of
// chosen experts' weights in the pool's own per-expert layout, slot s
// holding expert ids[s], and where each expert is read from.  Device memory.
struct ExpertTiers {
  const int32_t* loc;       // [E]: slot of e in the region, or -1 (read from the pool)
  const void *wg, *wu, *wd; // [n][I][H], [n][I][H], [n][H][I] in the pool's element format
  const uint16_t *sg, *su, *sd;   // 4-bit scales per slot (else null)
};

struct Layer {
  moe_layer_desc d;         // caller's description (pointers to caller weights)
  const void* router_eh;    // expert-major router actually read by the kernels
  void* router_copy;        // owned copy when the caller's layout is [H][E]
  float* norms;             // owned: [E] router row 2-norms (rounded up), then [1] max
  int* dev_flag;            // owned: sticky device fault word, then the refinement counter
  float* zero_bias;         // owned: [E] zeros when the caller gives no bias, else null
  double norm_max;          // host copy of max_e ||R_e||_2 (rounded up)
  int device;
  void* scratch;            // device address of this GPU's library scratch (moe_grouped_forward_noalloc)
  // the router's int8 first pass (batch-1 routing), when `screen`:
  bool screen;
  int8_t* q8;               // owned: [E][H] int8 router
  float* sc8;               // owned: [E] scales
  float2* eb8;              // owned: [E] (||eps_e||, ||s_e q_e||), rounded up
  float* screen_consts;     // owned: device maxima of the two norms and of |b|
  double screen_enmax, screen_rqmax, screen_bmax;   // host copies
  // the verify windows' screen (2 <= T <= kWinMaxT), when `screen_win`:
  bool screen_win;
  int8_t* q8w;              // owned: the int8 router in MFMA operand order (screen_window.hip)
  // the hot-expert region, when n_hot > 0 (the few-token path reads through it)
  int n_hot;
  void* hot_buf;            // owned: loc table, the ExpertTiers record and the copies
  const ExpertTiers* tiers; // inside hot_buf (null without a region or host tier)
  std::vector<int32_t>* hot_ids;   // owned: the region's experts (null: none)
  struct HostTier* host;    // owned: the host tier (host_tier.hip), null without one
};

// Verify windows of up to this many tokens route through the int8 screen
// (one 16-row MFMA operand holds two digit planes of each token).
constexpr int kWinMaxT = 8;

// The layer's device words: the sticky fault bits (int), then at byte 8 the
// count of exact refinements (unsigned long long, statistics).
constexpr size_t kDevWordsBytes = 16;
__host__ __device__ inline unsigned long long* refine_counter(int* dev_flag) {
  return reinterpret_cast<unsigned long long*>(reinterpret_cast<char*>(dev_flag) + 8);
}

// Layers with at least this many experts (bf16 activations, H a multiple of
// 32) screen the batch-1 router pass unless MOE_LAYER_SCREEN_OFF: the int8
// stream is half the bf16 router's bytes; with fewer experts the router is
// short enough that the extra kernel work does not pay.
constexpr int kScreenMinExperts = 4096;

// The router bias as the GEMV and few-token router kernels read it: never
// null (zeros when the caller gives none), so their loads need no branch.
inline const float* router_bias_or_zero(const Layer& L) {
  return L.d.router_bias != nullptr ? L.d.router_bias : L.zero_bias;
}

// Byte offsets of the per-call scratch regions inside the caller's workspace.
struct Workspace {
  size_t z;         // f64 [T][E] approximate logits
  size_t gmax;      // f32 [T][ceil(E/4)] maxima of 4 consecutive logits (rounded up)
  size_t xnorm;     // f64 [T] squared norms of the hidden states ([T][2] with the screen's ||delta||^2)
  size_t idx;       // int32 [T][k] routing (when the caller passes none)
  size_t gates;     // fp32 [T][k]
  size_t h;         // fp32 [k][I] decode intermediate
  size_t counts;    // int32 [E] pairs per expert
  size_t offsets;   // int32 [E + 1] exclusive scan of counts
  size_t slot;      // int32 [P] rank of a pair inside its expert's segment
  size_t pos;       // int32 [P] segment position of pair p
  size_t ptok;      // int32 [P] token of the pair at a segment position
  size_t active;    // int32 [E + 1] active experts (count first)
  size_t tiles;     // int32 [1 + 2 * max tiles]: count, then (expert, first row) per 32-row tile
  size_t tiles_big; // int32, same layout: kBigTileRows-row tiles of experts with more than 32 pairs
  size_t hm;        // fp32 [P][I] grouped intermediate
  size_t y;         // fp32 [P][H] grouped expert outputs
  size_t hint;      // batch-1 screen list: HintWords (128 B; state carried from call to call)
  size_t cnt8;      // u8 [screen blocks] rows each block of the screen listed
  size_t list;      // 16 B [kListSlots] the listed experts' recomputed logits
  size_t wcnt;      // verify windows on the screen: u8 [T][cstride] entries each screen wave listed
  size_t wlist;     // 16 B [T][kListSlots] the windows' per-token lists
  size_t total;
};

Workspace workspace_layout(const Layer& L, int T);

// ------------------------------------------------------------------ helpers
__host__ __device__ __forceinline__ int hpad(int i) { return i + ((i >> 5) << 2); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ float f16_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// DPP lane exchanges (within 16-lane rows, plus row broadcasts).
#define MOE_DPP_F32(v, ctrl, rmask) \
  __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, (v)), (ctrl), (rmask), 0xf, false))

// Sum over the 64 lanes of a wave, returned to every lane.  Fixed tree for
// every call: pairs inside quads, then quads, then 8-lane halves of a row
// (each lane of a row then holds the row sum), then row 0 into row 1 and
// row 2 into row 3 (row_bcast15), then rows 0-1 into rows 2-3 (row_bcast31);
// lane 63 holds (r2 + r3) + (r0 + r1) and is broadcast.  Depth 6.
__device__ __forceinline__ float wave_sum(float v) {
  v += MOE_DPP_F32(v, 0xB1, 0xf);     // quad_perm [1,0,3,2]
  v += MOE_DPP_F32(v, 0x4E, 0xf);     // quad_perm [2,3,0,1]
  v += MOE_DPP_F32(v, 0x141, 0xf);    // row_half_mirror
  v += MOE_DPP_F32(v, 0x140, 0xf);    // row_mirror
  v += MOE_DPP_F32(v, 0x142, 0xa);    // row_bcast:15 into rows 1 and 3
  v += MOE_DPP_F32(v, 0x143, 0xc);    // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
// Maximum over the 64 lanes (NaN-free inputs), returned to every lane.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, MOE_DPP_F32(v, 0xB1, 0xf));
  v = fmaxf(v, MOE_DPP_F32(v, 0x4E, 0xf));
  v = fmaxf(v, MOE_DPP_F32(v, 0x141, 0xf));
  v = fmaxf(v, MOE_DPP_F32(v, 0x140, 0xf));
  const float b15 = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      __builtin_bit_cast(int, -INFINITY), __builtin_bit_cast(int, v), 0x142, 0xa, 0xf, false));
  v = fmaxf(v, b15);
  const float b31 = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      __builtin_bit_cast(int, -INFINITY), __builtin_bit_cast(int, v), 0x143, 0xc, 0xf, false));
  v = fmaxf(v, b31);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
// Sum over aligned groups of 8 lanes; every lane of a group gets its sum.
__device__ __forceinline__ float group8_sum(float v) {
  v += MOE_DPP_F32(v, 0xB1, 0xf);
  v += MOE_DPP_F32(v, 0x4E, 0xf);
  v += MOE_DPP_F32(v, 0x141, 0xf);
  return v;
}
// 64-bit lane exchanges as two 32-bit DPP moves.
// Lanes of rows outside RMASK receive `old`.
template <int CTRL, int RMASK>
__device__ __forceinline__ double dpp_f64(double v, double old = 0.0) {
  const long long b = __double_as_longlong(v), o = __double_as_longlong(old);
  const int lo = __builtin_amdgcn_update_dpp(int(o & 0xffffffff), int(b & 0xffffffff), CTRL, RMASK, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(int(o >> 32), int(b >> 32), CTRL, RMASK, 0xf, false);
  return __longlong_as_double((long long)(unsigned)lo | ((long long)hi << 32));
}
#define MOE_DPP_F64(v, ctrl, rmask) dpp_f64<(ctrl), (rmask)>(v)
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane(int(b & 0xffffffff), lane);
  const int hi = __builtin_amdgcn_readlane(int(b >> 32), lane);
  return __longlong_as_double((long long)(unsigned)lo | ((long long)hi << 32));
}
// f64 sum over the 64 lanes with the same fixed tree as wave_sum (depth 6).
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += MOE_DPP_F64(v, 0xB1, 0xf);
  v += MOE_DPP_F64(v, 0x4E, 0xf);
  v += MOE_DPP_F64(v, 0x141, 0xf);
  v += MOE_DPP_F64(v, 0x140, 0xf);
  v += MOE_DPP_F64(v, 0x142, 0xa);
  v += MOE_DPP_F64(v, 0x143, 0xc);
  return readlane_f64(v, 63);
}
// f64 maximum over each 16-lane row (every lane of a row gets its row max).
__device__ __forceinline__ double row_max_f64(double v) {
  v = fmax(v, MOE_DPP_F64(v, 0xB1, 0xf));
  v = fmax(v, MOE_DPP_F64(v, 0x4E, 0xf));
  v = fmax(v, MOE_DPP_F64(v, 0x141, 0xf));
  v = fmax(v, MOE_DPP_F64(v, 0x140, 0xf));
  return v;
}
// f64 maximum over the 64 lanes (NaN-free inputs), returned to every lane.
__device__ __forceinline__ double wave_max_f64(double v) {
  v = row_max_f64(v);
  v = fmax(v, dpp_f64<0x142, 0xa>(v, -INFINITY));
  v = fmax(v, dpp_f64<0x143, 0xc>(v, -INFINITY));
  return readlane_f64(v, 63);
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

// Monotone map of fp32 onto uint32 (larger float -> larger key); NaN -> 0.
__device__ __forceinline__ uint32_t f32_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (isnan(f)) return 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_f32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// Knuth's TwoSum: s + e == a + b exactly (no overflow).  Written so that
// contraction cannot change it (no products).
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal (streamed data that is read once).
__device__ __forceinline__ uint4 load_nt(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Router chunk decoding: 8 consecutive elements of an act-dtype row.
// Upper bound of a binary64 value in binary32, without branches: the nearest
// binary32 value, moved one ulp up when it fell below v (a value below the
// binary32 normal range that rounded to zero gets FLT_MIN, an upper bound
// even where denormal results are flushed).  Not for NaN inputs.
__device__ __forceinline__ float f64_to_f32_up(double v) {
  const float f = (float)v;
  const uint32_t u = __float_as_uint(f);
  const uint32_t up = (u & 0x80000000u) ? (u == 0x80000000u ? 0x00800000u : u - 1u)
                                        : (u == 0u ? 0x00800000u : u + 1u);
  return ((double)f < v) ? __uint_as_float(up) : f;
}

// Orders LDS writes and reads of different lanes of one wave: a wave-wide
// barrier between release and acquire fences, so the compiler keeps every
// LDS access on its side of it (cross-lane data exchange through LDS is a
// race in the language model without one).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Register barrier: tells the compiler the value may change here, so work
// derived from loop-invariant weights (e.g. expanding 4-bit codes to floats)
// stays inside the loop instead of being hoisted into extra registers.
__device__ __forceinline__ void opaque_reg(uint4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}
__device__ __forceinline__ void opaque_reg(float4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

template <int ACT>
struct Chunk;
template <>
struct Chunk<MOE_BF16> {
  uint4 v;
  __device__ __forceinline__ void load(const void* base, size_t elem) {
    v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + elem);
  }
  __device__ __forceinline__ void load_stream(const void* base, size_t elem) {
    v = load_nt(reinterpret_cast<const uint16_t*>(base) + elem);
  }
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void opaque() { opaque_reg(v); }
  __device__ __forceinline__ float get(int i) const {
    uint32_t w = (i < 2) ? v.x : (i < 4) ? v.y : (i < 6) ? v.z : v.w;
    return (i & 1) ? bf16_hi(w) : bf16_lo(w);
  }
};
template <>
struct Chunk<MOE_F32> {
  float4 a, b;
  __device__ __forceinline__ void load(const void* base, size_t elem) {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem);
    a = p[0];
    b = p[1];
  }
  __device__ __forceinline__ void load_stream(const void* base, size_t elem) {
    const float* p = reinterpret_cast<const float*>(base) + elem;
    const uint4 u = load_nt(p), w = load_nt(p + 4);
    a = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
    b = make_float4(__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z), __uint_as_float(w.w));
  }
  __device__ __forceinline__ void opaque() {
    opaque_reg(a);
    opaque_reg(b);
  }
  __device__ __forceinline__ void zero() {
    a = make_float4(0, 0, 0, 0);
    b = a;
  }
  __device__ __forceinline__ float get(int i) const {
    switch (i) {
      case 0: return a.x; case 1: return a.y; case 2: return a.z; case 3: return a.w;
      case 4: return b.x; case 5: return b.y; case 6: return b.z; default: return b.w;
    }
  }
};

// Arguments of the grouped-path kernels (grouped.hip, mfma.hip).
struct GroupArgs {
  const void* x;            // [T][H]
  const int32_t* idx;       // [T][k]
  const float* gates;       // [T][k]
  const void *wg, *wu, *wd;
  const uint16_t *sg, *su, *sd;
  int T, H, I, E, k, P;
  int* counts;              // [E]
  int* offsets;             // [E+1]
  int* slot;                // [P]
  int* pos;                 // [P]
  int* ptok;                // [P]
  int small_max;            // experts with 1..small_max pairs: vector-ALU list, more: MFMA tiles
  int* active;              // [E+1]: [0] = number of listed experts (those with 1..small_max pairs)
  int* tiles;               // [0] = number of 32-row tiles (experts with small_max < n <= 32), then (expert, first row)
  int* tiles_big;           // same for kBigTileRows-row tiles of experts with n > 32
  float* hm;                // [P][I]
  float* y;                 // [P][H]
  float* out;               // [T][H]
  int* dev_flag;
};
constexpr int kTileRows = 32;
constexpr int kBigTileRows = 64;
constexpr int kMfmaSmallMax = 0;   // bf16 MFMA path: experts with at most this many pairs run on the vector ALUs

// ------------------------------------------------------------------ launchers
// router.hip: approximate logits z[t][e] (binary64) for tokens [0, T), the
// maximum of every 4 consecutive logits gmax[t][e/4] (binary32, rounded up)
// and ||x_t||^2 (binary64).
hipError_t launch_router(const Layer& L, const void* x, int T, double* z, float* gmax,
                         double* xnorm, hipStream_t s);
// Error model of one router logit:
//   |z_hat - z| <= (gamma(d32, 2^-23) + gamma(d64, 2^-52)) ||x|| ||R_e||
//                  + d32 2^-125 + d64 2^-1021 + 2^-52 |z_hat|,
// gamma(n, u) = n u / (1 - n u) (the u's are twice the unit roundoffs, which
// also covers truncating hardware).
struct RouterBound {
  int d32;
  int d64;
};
RouterBound router_bound(const Layer& L, int T);
// mfma.hip: the router as a bf16 MFMA GEMM for T >= 16 tokens (same outputs).
bool router_uses_mfma(const Layer& L, int T);
bool router_uses_big_tiles(const Layer& L, int T);   // fp32 accumulation over all of H
// Binary32 logits (the big-tile GEMM's fp32 sums plus the bias, rounded once
// more) when the route path calls it with z32; binary64 otherwise.
bool router_logits_f32(const Layer& L, int T);
hipError_t launch_router_gemm(const Layer& L, const void* x, int T, void* z, bool z32, float* gmax,
                              double* xnorm, hipStream_t s);
// mfma.hip: the router for 2 <= T < 16 bf16 tokens on 16x16x32 MFMA tiles.
bool router_uses_skinny(const Layer& L, int T);
hipError_t launch_router_skinny(const Layer& L, const void* x, int T, double* z, float* gmax,
                                double* xnorm, hipStream_t s);
// mfma.hip: grouped bf16 experts on MFMA (used when grouped_uses_mfma).
bool grouped_uses_mfma(const Layer& L, int T);
hipError_t launch_grouped_mfma(const GroupArgs& a, hipStream_t s);
// select.hip: exact top-k + gates per token from z; bt_unit/bt_abs give
// the router's error bound Bt = bt_unit * ||x||_2 + bt_abs.
hipError_t launch_select_impl(const Layer& L, const void* x, int T, const void* z, bool z32,
                              const float* gmax, const double* xnorm, int32_t* idx,
                              float* gates, const RouterBound& rb, hipStream_t s);
// experts.hip: expert GEMVs + combine for T tokens with T k <= kMaxPairs
// (batch-1 decode and verify windows); h is [T k][I] fp32 workspace.
bool pair_path_fits(const Layer& L, int T);
hipError_t launch_pair_experts(const Layer& L, const void* x, int T, const int32_t* idx,
                               const float* gates, float* out, float* h, hipStream_t s);
// experts.hip: T <= 8 routed tokens with 4-bit experts after the router:
// selection fused with gate/up (idx, gates written), then down + combine;
// h is [T k][I] fp32 workspace.
bool decode_fused_fits(const Layer& L, int T);

// ---- host helpers shared by the entry points (moe_api.hip) and the decoder
constexpr int kMaxDecoderLayers = 64;
moe_status api_fail(moe_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status api_ok();
const moe_layer_desc& layer_desc(const moe_layer* layer);
int layer_device(const moe_layer* layer);
long long host_clock_us();
hipError_t launch_decode_fused(const Layer& L, const void* x, int T, const double* z, const float* gmax,
                            const double* xnorm, const RouterBound& rb, int32_t* idx, float* gates,
                            float* out, float* h, hipStream_t s);
// grouped.hip: index sort, grouped experts, weighted un-permute.
hipError_t launch_grouped_experts(const Layer& L, const void* x, int T, const int32_t* idx,
                                  const float* gates, float* out, char* ws,
                                  const Workspace& W, hipStream_t s);
// screen.hip: the router's int8 first pass (batch-1 routing).  prep builds
// q8 / sc8 / eb8 and the maxima (consts[3]); screen writes the values z8
// [T][E], their maxima of 4 g8 and ||x||^2, ||delta||^2 into xq [T][2], and,
// with a list at T = 1, the listed experts' recomputed logits.
struct HintWords;
struct ScreenList {            // workspace regions of the batch-1 list
  HintWords* hint;
  unsigned char* cnt8;
  ulonglong2* list;
};
hipError_t launch_screen_prep(const Layer& L, float* consts, hipStream_t s);
hipError_t launch_screen(const Layer& L, const void* x, int T, float* z8, float* g8, double* xq,
                         const ScreenList* list, hipStream_t s);
int screen_waves(const Layer& L);
struct ScreenSelectArgs;
ScreenSelectArgs make_screen_select_args(const Layer& L, const void* x, const float* z8, const float* g8,
                                         const double* xq, int32_t* idx, float* gates);
void set_screen_list(ScreenSelectArgs& b, const Layer& L, const ScreenList* list, bool advance);
hipError_t launch_select_screen(const Layer& L, const void* x, int T, const float* z8, const float* g8,
                                const double* xq, const ScreenList* list, int32_t* idx, float* gates,
                                hipStream_t s);
// the screen values' error bounds B_e of tokens [0, T) (inspection)
hipError_t launch_screen_bounds(const Layer& L, int T, const float* z8, const double* xq, float* bound,
                                hipStream_t s);
// screen_window.hip: the screen for verify windows (2 <= T <= kWinMaxT) on
// MFMA, with one list per token (lists null: values only).
struct WinList {               // workspace regions of the windows' lists
  HintWords* hint;
  unsigned char* wcnt;
  ulonglong2* wlist;
};
bool screen_window_fits(const moe_layer_desc& d);
size_t screen_window_bytes(const moe_layer_desc& d);
int screen_window_waves(const Layer& L);
int screen_window_cstride(const Layer& L);
hipError_t launch_screen_window_prep(const Layer& L, hipStream_t s);
hipError_t launch_screen_window(const Layer& L, const void* x, int T, float* z8, float* g8, double* xq,
                                const WinList* list, hipStream_t s);
hipError_t launch_select_screen_window(const Layer& L, const void* x, int T, const float* z8, const float* g8,
                                       const double* xq, const WinList* list, int32_t* idx, float* gates,
                                       hipStream_t s);
// experts.hip: batch-1 decode after the screen: selection + gate/up, then
// down + combine (which ends the call: it advances the list's hint).
hipError_t launch_decode_screen(const Layer& L, const void* x, const float* z8, const float* g8, const double* xq,
                                const ScreenList* list, int32_t* idx, float* gates, float* out, float* h,
                                hipStream_t s);
// prep.hip: the hot region's copies (rows of `bytes` bytes of src for each
// listed expert, into consecutive slots of dst) and per-expert counts.
hipError_t launch_gather_experts(const void* src, void* dst, size_t bytes, const int32_t* ids, int n,
                                 hipStream_t s);
hipError_t launch_expert_counts(const int32_t* idx, int n, int E, uint32_t* counts, hipStream_t s);
// host_tier.hip: experts computed on the host's cores (moe_layer_set_host_experts).
struct HostTier;
hipError_t host_tier_create(const Layer& L, const int32_t* ids, int n, int n_threads, hipStream_t s,
                            HostTier** out);
void host_tier_destroy(HostTier* h);
const std::vector<int32_t>& host_tier_ids(const HostTier* h);
int host_tier_tmax(const HostTier* h);
hipError_t host_tier_fork(HostTier* h, const void* x, int T, const int32_t* idx, const float* gates,
                          hipStream_t s);
hipError_t host_tier_join(HostTier* h, int T, float* out, hipStream_t s);
void cpu_experts(const moe_layer_desc& d, const void* x, int T, const int32_t* idx, const float* gates, float* out,
                 int n_threads);
// prep.hip: layer creation helpers.
hipError_t launch_transpose_router(const Layer& L, void* dst, hipStream_t s);
hipError_t launch_router_norms(const Layer& L, hipStream_t s);

}  // namespace moe
