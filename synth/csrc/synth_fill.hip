// On-device fill of synthetic layer inputs (the generator of synth/__init__.py,
// implemented a second time for HBM-sized pools).  Holds no step of the MoE
// method: it draws numbers and encodes them into the layer's storage formats.
//
//   word(i)  = SplitMix64 output function of (key + (i + 1) * GAMMA)
//   S        = sum of the word's four 16-bit fields - 131070
//   value    = fp32(S) * scale   (one IEEE fp32 multiply; scale passed as fp32 bits)
//   bf16     = round-to-nearest-even of the fp32 bits
//   4-bit    = blocks of 32 along a row: d = fp16_rne(amax / 7) (f64 quotient),
//              q = clamp(rint(w / d), -7, 7) (0 when d == 0), nibble q + 8,
//              low nibble = even element.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float value_f32(uint64_t key, uint64_t i, float scale) {
  const uint64_t r = mix64(key + (i + 1ull) * kGamma);
  const int s = int(r & 0xffff) + int((r >> 16) & 0xffff) + int((r >> 32) & 0xffff) +
                int(r >> 48) - 131070;
  return __fmul_rn((float)s, scale);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return uint16_t((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// binary64 -> binary16, round to nearest even, directly from the double's bits.
__device__ uint16_t f64_to_f16_rne(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint16_t sign = uint16_t((b >> 48) & 0x8000u);
  const int e = int((b >> 52) & 0x7ff);
  const uint64_t m = b & ((1ull << 52) - 1);
  if (e == 0x7ff) return sign | 0x7c00u | (m ? 0x200u : 0u);
  if (e == 0) return sign;                       // f64 subnormals are far below fp16's range
  const uint64_t M = m | (1ull << 52);
  const int ue = e - 1023;
  if (ue > 15) return sign | 0x7c00u;
  int shift;
  bool normal = ue >= -14;
  shift = normal ? 42 : 28 - ue;                 // keep 11 bits, or units of 2^-24
  if (shift > 63) return sign;
  uint64_t mant = M >> shift;
  const uint64_t rem = M & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (mant & 1ull))) ++mant;
  if (normal) {
    const uint32_t h = (uint32_t(ue + 14) << 10) + uint32_t(mant);   // carry rolls into exponent
    if (h >= 0x7c00u) return sign | 0x7c00u;
    return sign | uint16_t(h);
  }
  return sign | uint16_t(mant);
}

__global__ void fill_kernel(void* dst, int bf16, uint64_t key, uint64_t base, float scale, int64_t n) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float v = value_f32(key, base + uint64_t(i), scale);
    if (bf16)
      reinterpret_cast<uint16_t*>(dst)[i] = f32_to_bf16_rne(v);
    else
      reinterpret_cast<float*>(dst)[i] = v;
  }
}

// One thread per 32-element block of a [rows][K] bf16 matrix, rows starting at row_base.
__global__ void fill_q4_kernel(uint8_t* q, uint16_t* scales, uint64_t key, uint64_t row_base,
                               int64_t rows, int K, float scale) {
  const int nb = K / 32;
  const int64_t total = rows * nb;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t blk = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; blk < total; blk += stride) {
    const int64_t r = blk / nb;
    const int b = int(blk - r * nb);
    const uint64_t i0 = (row_base + uint64_t(r)) * uint64_t(K) + uint64_t(b) * 32;
    float w[32];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint16_t h = f32_to_bf16_rne(value_f32(key, i0 + i, scale));
      w[i] = __uint_as_float(uint32_t(h) << 16);
      amax = fmaxf(amax, fabsf(w[i]));
    }
    const uint16_t dbits = f64_to_f16_rne((double)amax / 7.0);
    const double d = (double)__builtin_bit_cast(_Float16, dbits);
    uint32_t words[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      double qq = 0.0;
      if (d != 0.0) qq = rint((double)w[i] / d);
      qq = fmin(7.0, fmax(-7.0, qq));
      const uint32_t nib = uint32_t(int(qq) + 8);
      words[i >> 3] |= nib << (4 * (i & 7));
    }
    *reinterpret_cast<uint4*>(q + r * (K / 2) + b * 16) = make_uint4(words[0], words[1], words[2], words[3]);
    scales[r * nb + b] = dbits;
  }
}

int grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return int(g);
}

}  // namespace

extern "C" {

// Fill n elements (fp32 or bf16) with counters base .. base + n - 1 of stream `key`.
int synth_fill_values(void* dst, int bf16, uint64_t key, uint64_t base, uint32_t scale_bits,
                      int64_t n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(fill_kernel, dim3(grid_for(n)), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     dst, bf16, key, base, __builtin_bit_cast(float, scale_bits), n);
  return int(hipGetLastError());
}

// Fill `rows` 4-bit rows of length K (codes [rows][K/2], scales [rows][K/32]).
int synth_fill_q4(uint8_t* q, uint16_t* scales, uint64_t key, uint64_t row_base, int64_t rows,
                  int32_t K, uint32_t scale_bits, void* stream) {
  if (rows <= 0) return 0;
  if (K % 32) return -1;
  hipLaunchKernelGGL(fill_q4_kernel, dim3(grid_for(rows * (K / 32))), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), q, scales, key, row_base, rows, K,
                     __builtin_bit_cast(float, scale_bits));
  return int(hipGetLastError());
}

}  // extern "C"
