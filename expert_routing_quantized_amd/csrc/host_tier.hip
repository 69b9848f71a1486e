// The host tier: experts computed by the host's cores.
//
// The pages run the experts that the GPU does not hold on CPU threads,
// reading 4-bit weights from host RAM with wide vector instructions while
// the GPU computes the resident ones, and add the two parts at the combine
// (pyshine source tour, Understanding the Architecture, the paragraphs on
// three tiers and one residency table and on the CPU pool behind a
// doorbell).  Here an expert of the host tier is read by the GPU kernels as
// an all-zero expert of the layer's region (its part is then exactly 0 in
// their sums), and on a second stream the call's indices, gates and hidden
// states go to pinned memory, a host node runs the pool over the host
// tier's pairs, and the pool's output comes back and is added to the GPU's
// after both are done.  The host copies are made from the device pool when
// the tier is set.
//
// The pool's arithmetic (also exported on its own as moe_cpu_experts):
// a = G_e x, u = U_e x row by row in binary32 (4-bit rows: per 32-element
// block d_b * sum (q - 8) x), h = silu(a) u, then per output row the sum
// over the token's host pairs in selection order of g_j (D_e h_j).
#include <algorithm>
#include <thread>
#include <vector>

#include "cpu_pool.h"
#include "moe_internal.h"

namespace moe {

// ------------------------------------------------------------ the tier
struct HostTier;
struct HostCall {          // a host node's argument: the tier and the call's T
  HostTier* tier;
  int T;
};

struct HostTier {
  int n = 0, E = 0, H = 0, I = 0, k = 0, act = 0, tmax = 0;
  std::vector<int32_t> ids;
  std::vector<int32_t> slot;        // [E]: slot in the host copies, or -1
  HostExperts w{};
  void* copies = nullptr;           // pinned: the experts' weights
  int32_t* s_idx = nullptr;         // pinned staging [tmax k]
  float* s_gates = nullptr;         // pinned [tmax k]
  void* s_x = nullptr;              // pinned [tmax H] act dtype
  float* s_out = nullptr;           // pinned [tmax H]
  float* d_out = nullptr;           // device [tmax H]
  std::vector<float> xf;            // [tmax H] x in binary32
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  CpuPool* pool = nullptr;
  std::vector<HostCall> calls;      // one per T in [1, tmax]
};

static void host_node(void* arg) {
  HostCall* c = static_cast<HostCall*>(arg);
  HostTier& h = *c->tier;
  x_to_float(h.s_x, h.act, size_t(c->T) * h.H, h.xf.data());
  pool_forward(h.pool, h.w, h.xf.data(), c->T, h.k, h.s_idx, h.s_gates,
               [&](int e) { return (e >= 0 && e < h.E) ? h.slot[e] : -1; }, h.s_out);
}

__global__ __launch_bounds__(256) void add_f32_kernel(float* __restrict__ out, const float* __restrict__ add, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] += add[i];
}

void host_tier_destroy(HostTier* h) {
  if (!h) return;
  if (h->side) (void)hipStreamSynchronize(h->side);
  delete h->pool;
  if (h->copies) (void)hipHostFree(h->copies);
  if (h->s_idx) (void)hipHostFree(h->s_idx);
  if (h->s_gates) (void)hipHostFree(h->s_gates);
  if (h->s_x) (void)hipHostFree(h->s_x);
  if (h->s_out) (void)hipHostFree(h->s_out);
  if (h->d_out) (void)hipFree(h->d_out);
  if (h->fork) (void)hipEventDestroy(h->fork);
  if (h->join) (void)hipEventDestroy(h->join);
  if (h->side) (void)hipStreamDestroy(h->side);
  delete h;
}

const std::vector<int32_t>& host_tier_ids(const HostTier* h) { return h->ids; }

hipError_t host_tier_create(const Layer& L, const int32_t* ids, int n, int n_threads, hipStream_t s,
                            HostTier** out) {
  *out = nullptr;
  HostTier* h = new HostTier();
  const moe_layer_desc& d = L.d;
  h->n = n;
  h->E = d.n_experts;
  h->H = d.hidden;
  h->I = d.inter;
  h->k = d.top_k;
  h->act = d.act_dtype;
  h->tmax = std::max(1, std::min(d.max_tokens, kMaxPairs / d.top_k));
  h->ids.assign(ids, ids + n);
  h->slot.assign(size_t(h->E), -1);
  for (int i = 0; i < n; ++i) h->slot[ids[i]] = i;
  const size_t H = d.hidden, I = d.inter, N = size_t(n);
  const bool q4 = d.expert_dtype == MOE_Q4B32;
  const size_t elt = d.expert_dtype == MOE_F32 ? 4 : 2;
  const size_t gu = q4 ? I * H / 2 : I * H * elt, dn = q4 ? H * I / 2 : H * I * elt;
  const size_t sgu = q4 ? I * (H / 32) * 2 : 0, sdn = q4 ? H * (I / 32) * 2 : 0;
  const size_t per = 2 * gu + dn + 2 * sgu + sdn;
  const size_t ab = d.act_dtype == MOE_BF16 ? 2 : 4;
  hipError_t e;
  auto bail = [&](hipError_t err) {
    host_tier_destroy(h);
    return err;
  };
  if ((e = hipHostMalloc(&h->copies, std::max<size_t>(N * per, 16), hipHostMallocDefault)) != hipSuccess) return bail(e);
  if ((e = hipHostMalloc(reinterpret_cast<void**>(&h->s_idx), size_t(kMaxPairs) * 4, hipHostMallocDefault)) != hipSuccess ||
      (e = hipHostMalloc(reinterpret_cast<void**>(&h->s_gates), size_t(kMaxPairs) * 4, hipHostMallocDefault)) != hipSuccess ||
      (e = hipHostMalloc(&h->s_x, size_t(h->tmax) * H * ab, hipHostMallocDefault)) != hipSuccess ||
      (e = hipHostMalloc(reinterpret_cast<void**>(&h->s_out), size_t(h->tmax) * H * 4, hipHostMallocDefault)) != hipSuccess ||
      (e = hipMalloc(reinterpret_cast<void**>(&h->d_out), size_t(h->tmax) * H * 4)) != hipSuccess ||
      (e = hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking)) != hipSuccess ||
      (e = hipEventCreateWithFlags(&h->fork, hipEventDisableTiming)) != hipSuccess ||
      (e = hipEventCreateWithFlags(&h->join, hipEventDisableTiming)) != hipSuccess)
    return bail(e);
  char* c = static_cast<char*>(h->copies);
  h->w.H = d.hidden;
  h->w.I = d.inter;
  h->w.expert_dtype = d.expert_dtype;
  h->w.wg = c;
  h->w.wu = c + N * gu;
  h->w.wd = c + 2 * N * gu;
  char* sc = c + 2 * N * gu + N * dn;
  h->w.sg = q4 ? reinterpret_cast<const uint16_t*>(sc) : nullptr;
  h->w.su = q4 ? reinterpret_cast<const uint16_t*>(sc + N * sgu) : nullptr;
  h->w.sd = q4 ? reinterpret_cast<const uint16_t*>(sc + 2 * N * sgu) : nullptr;
  // the host copies, expert by expert, from the device pool
  for (int i = 0; i < n && e == hipSuccess; ++i) {
    const size_t ex = size_t(ids[i]);
    struct { const void* src; size_t bytes; const void* dst; } parts[6] = {
        {d.w_gate, gu, h->w.wg}, {d.w_up, gu, h->w.wu}, {d.w_down, dn, h->w.wd},
        {d.s_gate, sgu, h->w.sg}, {d.s_up, sgu, h->w.su}, {d.s_down, sdn, h->w.sd}};
    for (const auto& p : parts) {
      if (p.bytes == 0) continue;
      e = hipMemcpyAsync(const_cast<char*>(static_cast<const char*>(p.dst)) + i * p.bytes,
                         static_cast<const char*>(p.src) + ex * p.bytes, p.bytes, hipMemcpyDeviceToHost, s);
      if (e != hipSuccess) break;
    }
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return bail(e);
  h->xf.resize(size_t(h->tmax) * H);
  const unsigned hw = std::max(1u, std::thread::hardware_concurrency());
  const int nt = n_threads > 0 ? n_threads : int(std::min(16u, hw));
  h->pool = nt > 1 ? new CpuPool(nt - 1) : nullptr;   // the host node's thread works too
  h->calls.resize(size_t(h->tmax) + 1);
  for (int t = 0; t <= h->tmax; ++t) h->calls[t] = HostCall{h, t};
  *out = h;
  return hipSuccess;
}

// Before the GPU's expert kernels: the side stream takes the call's
// indices, gates and hidden states to pinned memory and runs the pool.
hipError_t host_tier_fork(HostTier* h, const void* x, int T, const int32_t* idx, const float* gates,
                          hipStream_t s) {
  if (T < 1 || T > h->tmax) return hipErrorInvalidValue;
  const size_t P = size_t(T) * h->k, ab = h->act == MOE_BF16 ? 2 : 4;
  hipError_t e;
  if ((e = hipEventRecord(h->fork, s)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(h->side, h->fork, 0)) != hipSuccess) return e;
  if ((e = hipMemcpyAsync(h->s_idx, idx, P * 4, hipMemcpyDeviceToHost, h->side)) != hipSuccess) return e;
  if ((e = hipMemcpyAsync(h->s_gates, gates, P * 4, hipMemcpyDeviceToHost, h->side)) != hipSuccess) return e;
  if ((e = hipMemcpyAsync(h->s_x, x, size_t(T) * h->H * ab, hipMemcpyDeviceToHost, h->side)) != hipSuccess) return e;
  if ((e = hipLaunchHostFunc(h->side, host_node, &h->calls[T])) != hipSuccess) return e;
  if ((e = hipMemcpyAsync(h->d_out, h->s_out, size_t(T) * h->H * 4, hipMemcpyHostToDevice, h->side)) != hipSuccess)
    return e;
  return hipEventRecord(h->join, h->side);
}

// After them: wait for the pool's part and add it.
hipError_t host_tier_join(HostTier* h, int T, float* out, hipStream_t s) {
  hipError_t e = hipStreamWaitEvent(s, h->join, 0);
  if (e != hipSuccess) return e;
  const int n = T * h->H;
  hipLaunchKernelGGL(add_f32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, out, h->d_out, n);
  return hipGetLastError();
}

int host_tier_tmax(const HostTier* h) { return h->tmax; }

// moe_cpu_experts: the pool's arithmetic on caller host arrays.
void cpu_experts(const moe_layer_desc& d, const void* x, int T, const int32_t* idx, const float* gates, float* out,
                 int n_threads) {
  HostExperts w{d.hidden, d.inter, d.expert_dtype, d.w_gate, d.w_up, d.w_down, d.s_gate, d.s_up, d.s_down};
  std::vector<float> xf(size_t(T) * d.hidden);
  x_to_float(x, d.act_dtype, xf.size(), xf.data());
  CpuPool* pool = n_threads > 1 ? new CpuPool(n_threads - 1) : nullptr;
  const int E = d.n_experts;
  pool_forward(pool, w, xf.data(), T, d.top_k, idx, gates, [&](int e) { return (e >= 0 && e < E) ? e : -1; }, out);
  delete pool;
}

}  // namespace moe
