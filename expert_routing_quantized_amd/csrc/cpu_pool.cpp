// The host tier's pool: expert SwiGLU GEMVs on the host's cores.
//
// The pages compute the experts the GPU does not hold on CPU threads with
// wide vector instructions over weights in host RAM (pyshine source tour,
// Understanding the Architecture, the paragraph on three tiers and one
// residency table).  Each dot product is one binary32 chain per row (4-bit
// rows: per 32-element block d_b * sum (q - 8) x); the row loops are built
// for AVX-512, AVX2 and baseline x86-64, and the loader picks the widest the
// host supports.
#include "cpu_pool.h"

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

// One 4-bit row (K elements: K/2 code bytes, K/32 fp16 scales) against x.
__attribute__((target_clones("avx512f", "avx2", "default")))
static float dot_q4(const uint8_t* codes, const uint16_t* scales, const float* x, int K) {
  float acc = 0.f;
  for (int b = 0; b < K / 32; ++b) {
    const uint8_t* c = codes + 16 * b;
    const float* xb = x + 32 * b;
    float lo[16], hi[16];
    for (int i = 0; i < 16; ++i) {
      lo[i] = float(int(c[i] & 15) - 8) * xb[2 * i];
      hi[i] = float(int(c[i] >> 4) - 8) * xb[2 * i + 1];
    }
    float s = 0.f;
    for (int i = 0; i < 16; ++i) s += lo[i] + hi[i];
    acc += half_to_float(scales[b]) * s;
  }
  return acc;
}

__attribute__((target_clones("avx512f", "avx2", "default")))
static float dot_bf16(const uint16_t* w, const float* x, int K) {
  float acc = 0.f;
  for (int i = 0; i < K; ++i) acc += bf16_to_float(w[i]) * x[i];
  return acc;
}

__attribute__((target_clones("avx512f", "avx2", "default")))
static float dot_f32(const float* w, const float* x, int K) {
  float acc = 0.f;
  for (int i = 0; i < K; ++i) acc += w[i] * x[i];
  return acc;
}

static float row_dot(const HostExperts& w, const void* base, const uint16_t* scales, size_t row, int K,
                     const float* x) {
  if (w.expert_dtype == 2)
    return dot_q4(static_cast<const uint8_t*>(base) + row * (K / 2), scales + row * (K / 32), x, K);
  if (w.expert_dtype == 1) return dot_bf16(static_cast<const uint16_t*>(base) + row * K, x, K);
  return dot_f32(static_cast<const float*>(base) + row * K, x, K);
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
  std::vector<float> h(pairs.size() * size_t(I));
  constexpr int kRows = 32;
  const int rchunks = (I + kRows - 1) / kRows;
  auto gateup = [&](int job) {
    const int pi = job / rchunks;
    const Pair& p = pairs[pi];
    const int i0 = (job % rchunks) * kRows, i1 = std::min(I, i0 + kRows);
    const float* xt = x + size_t(p.t) * H;
    for (int i = i0; i < i1; ++i) {
      const size_t row = size_t(p.slot) * I + i;
      const float a = row_dot(w, w.wg, w.sg, row, H, xt), u = row_dot(w, w.wu, w.su, row, H, xt);
      h[size_t(pi) * I + i] = a / (1.f + expf(-a)) * u;
    }
  };
  const int n1 = int(pairs.size()) * rchunks;
  if (pool) pool->run(n1, gateup);
  else for (int j = 0; j < n1; ++j) gateup(j);
  constexpr int kOut = 64;
  const int ochunks = (H + kOut - 1) / kOut;
  auto down = [&](int job) {
    const int t = job / ochunks, o0 = (job % ochunks) * kOut, o1 = std::min(H, o0 + kOut);
    for (int o = o0; o < o1; ++o) {
      float s = 0.f;
      for (int pi : by_token[t]) {
        const Pair& p = pairs[pi];
        s += p.g * row_dot(w, w.wd, w.sd, size_t(p.slot) * H + o, I, h.data() + size_t(pi) * I);
      }
      out[size_t(t) * H + o] = s;
    }
  };
  if (pool) pool->run(T * ochunks, down);
  else for (int j = 0; j < T * ochunks; ++j) down(j);
}

}  // namespace moe
