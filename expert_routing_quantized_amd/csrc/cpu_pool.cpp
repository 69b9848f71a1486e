// The host tier's pool: expert SwiGLU GEMVs on the host's cores.
//
// The pages compute the experts the GPU does not hold on CPU threads with
// wide vector instructions over weights in host RAM (pyshine source tour,
// Understanding the Architecture, the paragraph on three tiers and one
// residency table).  Each dot product runs in binary32 over 16 (or 8)
// independent lanes summed at the end; the row loops are built for AVX-512,
// AVX2 and baseline x86-64, and the loader picks the widest the host
// supports.
#include "cpu_pool.h"

#include <immintrin.h>
#include <math.h>
#include <string.h>

#include <algorithm>

namespace moe {

// ------------------------------------------------------------ arithmetic
static inline float half_to_float(uint16_t h) {
  const uint32_t s = uint32_t(h >> 15) << 31, ex = (h >> 10) & 0x1f, m = h & 0x3ff;
  if (ex == 0) {                                   // zero or subnormal: m 2^-24
    const float v = ldexpf((float)m, -24);
    return s ? -v : v;
  }
  uint32_t bits;
  if (ex == 31) bits = s | 0x7f800000u | (m << 13);
  else bits = s | ((ex + 112) << 23) | (m << 13);
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

static inline float bf16_to_float(uint16_t b) {
  const uint32_t bits = uint32_t(b) << 16;
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

// The activation a row multiplies, split for 4-bit rows: block b's even
// elements (the low nibbles) at ev[16 b ..], odd ones at od[16 b ..], and
// the block sum at bs[b], so a block's 32 products are two 16-wide multiply-
// adds with no shuffle and the -8 offset is one term per block.
struct SplitVec {
  std::vector<float> ev, od, bs;
  void set(const float* v, int K) {
    const int nb = K / 32;
    ev.resize(size_t(nb) * 16);
    od.resize(size_t(nb) * 16);
    bs.resize(size_t(nb));
    for (int b = 0; b < nb; ++b) {
      float s = 0.f;
      for (int i = 0; i < 16; ++i) {
        ev[16 * b + i] = v[32 * b + 2 * i];
        od[16 * b + i] = v[32 * b + 2 * i + 1];
        s += v[32 * b + 2 * i] + v[32 * b + 2 * i + 1];
      }
      bs[b] = s;
    }
  }
};

// One 4-bit row (K elements: K/2 code bytes, K/32 fp16 scales):
// sum_b d_b (sum_i q_i v_i - 8 sum_i v_i), the codes' products kept in 16
// binary32 lanes across the blocks (each lane's chain runs over the row) and
// the lanes summed at the end.  Three builds of the same arithmetic: AVX-512
// (one 16-lane register per block), AVX2 (two 8-lane halves) and plain C++;
// the lanes are summed in the same fixed order by all three.
static float lanes_sum16(const float* acc) {
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += acc[i];
  return s;
}

__attribute__((target("avx512f")))
static float dot_q4_avx512(const uint8_t* codes, const uint16_t* scales, const SplitVec& v, int K) {
  const int nb = K / 32;
  __m512 acc = _mm512_setzero_ps();
  const __m512i m15 = _mm512_set1_epi32(15);
  float corr = 0.f;
  for (int b = 0; b < nb; ++b) {
    const float d = half_to_float(scales[b]);
    const __m512i ci = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(codes + 16 * b)));
    const __m512 lo = _mm512_cvtepi32_ps(_mm512_and_si512(ci, m15));
    const __m512 hi = _mm512_cvtepi32_ps(_mm512_srli_epi32(ci, 4));
    const __m512 t = _mm512_fmadd_ps(hi, _mm512_loadu_ps(v.od.data() + 16 * b),
                                     _mm512_mul_ps(lo, _mm512_loadu_ps(v.ev.data() + 16 * b)));
    acc = _mm512_fmadd_ps(_mm512_set1_ps(d), t, acc);
    corr += d * v.bs[b];
  }
  alignas(64) float l[16];
  _mm512_store_ps(l, acc);
  return lanes_sum16(l) - 8.f * corr;
}

__attribute__((target("avx2,fma")))
static float dot_q4_avx2(const uint8_t* codes, const uint16_t* scales, const SplitVec& v, int K) {
  const int nb = K / 32;
  __m256 acc0 = _mm256_setzero_ps(), acc1 = _mm256_setzero_ps();
  const __m256i m15 = _mm256_set1_epi32(15);
  float corr = 0.f;
  for (int b = 0; b < nb; ++b) {
    const float d = half_to_float(scales[b]);
    const __m128i c = _mm_loadu_si128(reinterpret_cast<const __m128i*>(codes + 16 * b));
    const __m256i c0 = _mm256_cvtepu8_epi32(c), c1 = _mm256_cvtepu8_epi32(_mm_srli_si128(c, 8));
    const float* e = v.ev.data() + 16 * b;
    const float* o = v.od.data() + 16 * b;
    const __m256 t0 = _mm256_fmadd_ps(_mm256_cvtepi32_ps(_mm256_srli_epi32(c0, 4)), _mm256_loadu_ps(o),
                                      _mm256_mul_ps(_mm256_cvtepi32_ps(_mm256_and_si256(c0, m15)), _mm256_loadu_ps(e)));
    const __m256 t1 = _mm256_fmadd_ps(_mm256_cvtepi32_ps(_mm256_srli_epi32(c1, 4)), _mm256_loadu_ps(o + 8),
                                      _mm256_mul_ps(_mm256_cvtepi32_ps(_mm256_and_si256(c1, m15)), _mm256_loadu_ps(e + 8)));
    const __m256 dv = _mm256_set1_ps(d);
    acc0 = _mm256_fmadd_ps(dv, t0, acc0);
    acc1 = _mm256_fmadd_ps(dv, t1, acc1);
    corr += d * v.bs[b];
  }
  alignas(32) float l[16];
  _mm256_store_ps(l, acc0);
  _mm256_store_ps(l + 8, acc1);
  return lanes_sum16(l) - 8.f * corr;
}

static float dot_q4_plain(const uint8_t* codes, const uint16_t* scales, const SplitVec& v, int K) {
  const int nb = K / 32;
  float acc[16] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float corr = 0.f;
  for (int b = 0; b < nb; ++b) {
    const float d = half_to_float(scales[b]);
    const uint8_t* c = codes + 16 * b;
    const float* e = v.ev.data() + 16 * b;
    const float* o = v.od.data() + 16 * b;
    for (int i = 0; i < 16; ++i) acc[i] = fmaf(d, fmaf(float(c[i] >> 4), o[i], float(c[i] & 15) * e[i]), acc[i]);
    corr += d * v.bs[b];
  }
  return lanes_sum16(acc) - 8.f * corr;
}

static int isa_level() {
  static const int level = [] {
    __builtin_cpu_init();
    if (__builtin_cpu_supports("avx512f")) return 2;
    if (__builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma")) return 1;
    return 0;
  }();
  return level;
}

static float dot_q4(const uint8_t* codes, const uint16_t* scales, const SplitVec& v, int K) {
  switch (isa_level()) {
    case 2: return dot_q4_avx512(codes, scales, v, K);
    case 1: return dot_q4_avx2(codes, scales, v, K);
    default: return dot_q4_plain(codes, scales, v, K);
  }
}

// Dense rows: 16 binary32 lanes across the row, summed at the end.
__attribute__((target_clones("avx512f", "avx2", "default")))
static float dot_bf16(const uint16_t* w, const float* x, int K) {
  float acc[16] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < K; j += 16)
    for (int i = 0; i < 16; ++i) acc[i] += bf16_to_float(w[j + i]) * x[j + i];
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += acc[i];
  return s;
}

__attribute__((target_clones("avx512f", "avx2", "default")))
static float dot_f32(const float* w, const float* x, int K) {
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < K; j += 8)
    for (int i = 0; i < 8; ++i) acc[i] += w[j + i] * x[j + i];
  float s = 0.f;
  for (int i = 0; i < 8; ++i) s += acc[i];
  return s;
}

// row `row` of a matrix with K columns in the experts' format, against v
static float row_dot(const HostExperts& w, const void* base, const uint16_t* scales, size_t row, int K,
                     const float* v, const SplitVec& sv) {
  if (w.expert_dtype == 2)
    return dot_q4(static_cast<const uint8_t*>(base) + row * (K / 2), scales + row * (K / 32), sv, K);
  if (w.expert_dtype == 1) return dot_bf16(static_cast<const uint16_t*>(base) + row * K, v, K);
  return dot_f32(static_cast<const float*>(base) + row * K, v, K);
}

void x_to_float(const void* x, int act, size_t n, float* dst) {
  if (act == 1)
    for (size_t i = 0; i < n; ++i) dst[i] = bf16_to_float(static_cast<const uint16_t*>(x)[i]);
  else
    memcpy(dst, x, n * sizeof(float));
}

// ------------------------------------------------------------ thread pool
CpuPool::CpuPool(int n_workers) {
  for (int i = 0; i < n_workers; ++i) th_.emplace_back([this] { work(); });
}

CpuPool::~CpuPool() {
  {
    std::lock_guard<std::mutex> g(m_);
    stop_ = true;
  }
  cv_.notify_all();
  for (auto& t : th_) t.join();
}

void CpuPool::run(int n, const std::function<void(int)>& f) {
  if (n <= 0) return;
  {
    std::lock_guard<std::mutex> g(m_);
    job_ = &f;
    njobs_ = n;
    next_.store(0);
    left_ = n;
    ++gen_;
  }
  cv_.notify_all();
  drain();
  std::unique_lock<std::mutex> l(m_);
  done_.wait(l, [this] { return left_ == 0; });
  job_ = nullptr;
}

void CpuPool::drain() {
  for (;;) {
    const int i = next_.fetch_add(1);
    if (i >= njobs_) return;
    (*job_)(i);
    std::lock_guard<std::mutex> g(m_);
    if (--left_ == 0) done_.notify_all();
  }
}

void CpuPool::work() {
  uint64_t seen = 0;
  for (;;) {
    {
      std::unique_lock<std::mutex> l(m_);
      cv_.wait(l, [&] { return stop_ || (gen_ != seen && job_ != nullptr); });
      if (stop_) return;
      seen = gen_;
    }
    drain();
  }
}

// ------------------------------------------------------------ forward
void pool_forward(CpuPool* pool, const HostExperts& w, const float* x, int T, int k, const int32_t* idx,
                  const float* gates, const std::function<int(int)>& slot_of, float* out) {
  const int H = w.H, I = w.I;
  struct Pair {
    int t, slot;
    float g;
  };
  std::vector<Pair> pairs;
  std::vector<std::vector<int>> by_token(T);
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      const int s = slot_of(idx[size_t(t) * k + j]);
      if (s < 0) continue;
      by_token[t].push_back(int(pairs.size()));
      pairs.push_back({t, s, gates[size_t(t) * k + j]});
    }
  std::fill(out, out + size_t(T) * H, 0.f);
  if (pairs.empty()) return;
  const bool q4 = w.expert_dtype == 2;
  std::vector<SplitVec> xs(q4 ? T : 0);
  for (int t = 0; t < T && q4; ++t) xs[t].set(x + size_t(t) * H, H);
  const SplitVec none;
  std::vector<float> h(pairs.size() * size_t(I));
  std::vector<SplitVec> hs(q4 ? pairs.size() : 0);
  constexpr int kRows = 32;
  const int rchunks = (I + kRows - 1) / kRows;
  auto gateup = [&](int job) {
    const int pi = job / rchunks;
    const Pair& p = pairs[pi];
    const int i0 = (job % rchunks) * kRows, i1 = std::min(I, i0 + kRows);
    const float* xt = x + size_t(p.t) * H;
    const SplitVec& sv = q4 ? xs[p.t] : none;
    for (int i = i0; i < i1; ++i) {
      const size_t row = size_t(p.slot) * I + i;
      const float a = row_dot(w, w.wg, w.sg, row, H, xt, sv), u = row_dot(w, w.wu, w.su, row, H, xt, sv);
      h[size_t(pi) * I + i] = a / (1.f + expf(-a)) * u;
    }
  };
  const int n1 = int(pairs.size()) * rchunks;
  if (pool) pool->run(n1, gateup);
  else for (int j = 0; j < n1; ++j) gateup(j);
  for (size_t pi = 0; pi < hs.size(); ++pi) hs[pi].set(h.data() + pi * I, I);
  constexpr int kOut = 64;
  const int ochunks = (H + kOut - 1) / kOut;
  auto down = [&](int job) {
    const int t = job / ochunks, o0 = (job % ochunks) * kOut, o1 = std::min(H, o0 + kOut);
    for (int o = o0; o < o1; ++o) {
      float s = 0.f;
      for (int pi : by_token[t]) {
        const Pair& p = pairs[pi];
        s += p.g * row_dot(w, w.wd, w.sd, size_t(p.slot) * H + o, I, h.data() + size_t(pi) * I, q4 ? hs[pi] : none);
      }
      out[size_t(t) * H + o] = s;
    }
  };
  if (pool) pool->run(T * ochunks, down);
  else for (int j = 0; j < T * ochunks; ++j) down(j);
}

}  // namespace moe
