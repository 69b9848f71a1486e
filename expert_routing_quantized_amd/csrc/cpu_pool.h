// The host tier's pool: expert SwiGLU GEMVs on the host's cores (plain C++;
// cpu_pool.cpp is compiled for the host only).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

namespace moe {

// The weights of experts in the pool's layout (host memory): slot s of each
// array holds one expert.  dtype: 0 fp32, 1 bf16, 2 4-bit blocks (the
// moe_dtype values).
struct HostExperts {
  int H, I, expert_dtype;
  const void *wg, *wu, *wd;
  const uint16_t *sg, *su, *sd;
};

// A fixed set of worker threads; run(n, f) calls f(0) ... f(n - 1) on them
// and on the calling thread and returns when all are done.
class CpuPool {
 public:
  explicit CpuPool(int n_workers);
  ~CpuPool();
  void run(int n, const std::function<void(int)>& f);

 private:
  void drain();
  void work();
  std::vector<std::thread> th_;
  std::mutex m_;
  std::condition_variable cv_, done_;
  const std::function<void(int)>* job_ = nullptr;
  int njobs_ = 0, left_ = 0;
  std::atomic<int> next_{0};
  uint64_t gen_ = 0;
  bool stop_ = false;
};

// x of T tokens ([T][H], act dtype 0 fp32 / 1 bf16) to binary32.
void x_to_float(const void* x, int act, size_t n, float* dst);

// out[T][H] = for each token the sum over its pairs j < k (in order) that
// slot_of maps to a slot (>= 0) of gates[t][j] * y(slot), y = D (silu(G x) *
// (U x)) in binary32.  pool may be null (the calling thread alone).
void pool_forward(CpuPool* pool, const HostExperts& w, const float* x, int T, int k, const int32_t* idx,
                  const float* gates, const std::function<int(int)>& slot_of, float* out);

}  // namespace moe
