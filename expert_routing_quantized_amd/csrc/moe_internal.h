// Internal declarations of libmoe: layer object, workspace layout, device
// helpers shared by the kernels, and the launchers each kernel file exports.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ------------------------------------------------------------------ limits
constexpr int kMaxK = 32;
constexpr int kMaxH = 8192;
constexpr int kMaxI = 4096;
constexpr int kRouterEPB = 64;      // experts per router block (one k-th-value per block)
constexpr int kSelectThreads = 1024;
constexpr int kSelectMaxCand = 2048;  // candidates held in LDS at once

// device fault bits (moe_device_error)
constexpr int kDevBadIndex = 1;
constexpr int kDevDupIndex = 2;
constexpr int kDevNonFinite = 4;
constexpr int kDevInternal = 8;

// ------------------------------------------------------------------ layer
struct Layer {
  moe_layer_desc d;         // caller's description (pointers to caller weights)
  const void* router_eh;    // expert-major router actually read by the kernels
  void* router_copy;        // owned copy when the caller's layout is [H][E]
  float* norms;             // owned: [E] router row 2-norms (rounded up), then [1] max
  int* dev_flag;            // owned: sticky device fault word
  double norm_max;          // host copy of max_e ||R_e||_2 (rounded up)
  int device;
};

// Byte offsets of the per-call scratch regions inside the caller's workspace.
struct Workspace {
  size_t z;         // fp32 [T][E] approximate logits
  size_t tau;       // fp32 [T][ntau] per-block k-th largest approximate logit
  size_t idx;       // int32 [T][k] routing (when the caller passes none)
  size_t gates;     // fp32 [T][k]
  size_t h;         // fp32 [k][I] decode intermediate
  size_t counts;    // int32 [E] pairs per expert
  size_t offsets;   // int32 [E + 1] exclusive scan of counts
  size_t slot;      // int32 [P] rank of a pair inside its expert's segment
  size_t pos;       // int32 [P] segment position of pair p
  size_t ptok;      // int32 [P] token of the pair at a segment position
  size_t active;    // int32 [E + 1] active experts (count first)
  size_t hm;        // fp32 [P][I] grouped intermediate (or bf16 hi/lo pairs)
  size_t y;         // fp32 [P][H] grouped expert outputs
  size_t total;
  int ntau;
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

// Butterfly sum over the 64 lanes of a wave: every lane ends with the same
// bits (each level adds the partner's value; fp addition commutes).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int m = 1; m < width; m <<= 1) v += __shfl_xor(v, m);
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

// Router chunk decoding: 8 consecutive elements of an act-dtype row.
template <int ACT>
struct Chunk;
template <>
struct Chunk<MOE_BF16> {
  uint4 v;
  __device__ __forceinline__ void load(const void* base, size_t elem) {
    v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + elem);
  }
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
  __device__ __forceinline__ float get(int i) const {
    switch (i) {
      case 0: return a.x; case 1: return a.y; case 2: return a.z; case 3: return a.w;
      case 4: return b.x; case 5: return b.y; case 6: return b.z; default: return b.w;
    }
  }
};

// ------------------------------------------------------------------ launchers
// router.hip: approximate fp32 logits z[t][e] for tokens [0, T) and per-block
// k-th largest value tau[t][b]; returns the number of blocks (tau columns).
int router_ntau(const Layer& L);
hipError_t launch_router(const Layer& L, const void* x, int T, float* z, float* tau,
                         hipStream_t s);
// Rounding depth of one router logit of launch_router (see router.hip).
int router_depth(const Layer& L, int T);
// select.hip: exact top-k + gates per token from z/tau; bt_unit/bt_abs give
// the router's error bound Bt = bt_unit * ||x||_2 + bt_abs.
hipError_t launch_select_impl(const Layer& L, const void* x, int T, const float* z,
                              const float* tau, int ntau, int32_t* idx, float* gates,
                              double bt_unit, double bt_abs, hipStream_t s);
// experts.hip: single-token expert GEMVs and combine.
hipError_t launch_decode_experts(const Layer& L, const void* x, const int32_t* idx,
                                 const float* gates, float* out, float* h, hipStream_t s);
// grouped.hip: index sort, grouped experts, weighted un-permute.
hipError_t launch_grouped_experts(const Layer& L, const void* x, int T, const int32_t* idx,
                                  const float* gates, float* out, char* ws,
                                  const Workspace& W, hipStream_t s);
// prep.hip: layer creation helpers.
hipError_t launch_transpose_router(const Layer& L, void* dst, hipStream_t s);
hipError_t launch_router_norms(const Layer& L, hipStream_t s);

}  // namespace moe
