// Batch-1 decode through a stack of layers, one captured HIP graph per layer.
//
// The pages' engine composes a token from one captured graph per layer: a
// graph bakes in its arguments, so the per-token values reach it through
// fixed-address device buffers, and the host decides when each layer's
// graph runs, told by a doorbell from the device (pyshine source tour,
// paragraph on the driver that composes one token).  Here every expert is
// resident in HBM, so the doorbell has no miss pool to wake; it is the
// host's view of how far the device has got, and the host can wait on it
// before launching the next layer.
//
// Layer l's graph: moe_grouped_forward (T = 1, routed inside) on fixed
// buffers -- input slot x_l (bf16 [H]), its own workspace, idx_l, gates_l,
// out_l (fp32 [H]) -- then the layer epilogue (one block): the residual
// stream x_{l+1} = bf16(x_l + out_l) (fp32 sum, rounded to nearest even)
// into the next slot, and the doorbell: once every store of the layer is
// in memory, the step number goes to the layer's host-pinned word.  The
// last layer's epilogue also advances the device step counter.
#include <stdarg.h>
#include <stdio.h>

#include <vector>

#include "moe_internal.h"

namespace {

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);   // NaN stays NaN (quiet)
  return uint16_t((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

constexpr int kEpilogueThreads = 1024;

// x_next = bf16(x + out), then the doorbell (`last`: advance the step counter).
__global__ __launch_bounds__(kEpilogueThreads) void layer_epilogue_kernel(const uint16_t* x, const float* out,
                                                                           uint16_t* x_next, int H,
                                                                           unsigned long long* step,
                                                                           unsigned long long* bell, int last) {
  for (int h = threadIdx.x; h < H; h += kEpilogueThreads) {
    const float v = __uint_as_float(uint32_t(x[h]) << 16) + out[h];
    x_next[h] = f32_to_bf16_rne(v);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned long long s = *step + 1ull;
    __threadfence_system();                                    // the block's stores first
    __hip_atomic_store(bell, s, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    if (last) __hip_atomic_store(step, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

struct moe_decoder {
  int n = 0;
  int H = 0, k = 0;
  int device = 0;
  char* dmem = nullptr;                     // owned device memory: every fixed buffer
  unsigned long long* bells = nullptr;      // owned host-pinned doorbells [n]
  unsigned long long steps = 0;             // steps launched (host count)
  std::vector<uint16_t*> x;                 // [n + 1] input slots, then the result slot
  std::vector<float*> out;
  std::vector<int32_t*> idx;
  std::vector<float*> gates;
  std::vector<hipGraphExec_t> exec;
  std::vector<hipGraph_t> graph;
  hipGraph_t token_graph = nullptr;         // every layer's graph as a child node, in order
  hipGraphExec_t token_exec = nullptr;
};

namespace {

constexpr long long kDoorbellSpinUs = 2000000;   // 2 s: a bounded wait

moe_status destroy_all(moe_decoder* d) {
  if (d->token_exec) (void)hipGraphExecDestroy(d->token_exec);
  if (d->token_graph) (void)hipGraphDestroy(d->token_graph);
  for (auto e : d->exec)
    if (e) (void)hipGraphExecDestroy(e);
  for (auto g : d->graph)
    if (g) (void)hipGraphDestroy(g);
  if (d->dmem) (void)hipFree(d->dmem);
  if (d->bells) (void)hipHostFree(d->bells);
  delete d;
  return MOE_OK;
}

size_t round256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

extern "C" {

moe_status moe_decoder_create(const moe_layer* const* layers, int32_t n_layers, void* stream, moe_decoder** out) {
  if (!out) return moe::api_fail(MOE_E_NULL, "out is NULL");
  *out = nullptr;
  if (!layers) return moe::api_fail(MOE_E_NULL, "layers is NULL");
  if (n_layers < 1 || n_layers > moe::kMaxDecoderLayers)
    return moe::api_fail(MOE_E_RANGE, "n_layers=%d outside [1, %d]", n_layers, moe::kMaxDecoderLayers);
  const moe_layer_desc* d0 = nullptr;
  for (int l = 0; l < n_layers; ++l) {
    if (!layers[l]) return moe::api_fail(MOE_E_NULL, "layers[%d] is NULL", l);
    const moe_layer_desc& d = moe::layer_desc(layers[l]);
    if (d.act_dtype != MOE_BF16) return moe::api_fail(MOE_E_DTYPE, "layer %d: the decoder needs bf16 activations", l);
    if (d.max_tokens < 1) return moe::api_fail(MOE_E_RANGE, "layer %d: max_tokens < 1", l);
    if (d0 && d.hidden != d0->hidden)
      return moe::api_fail(MOE_E_GEOMETRY, "layer %d: hidden %d differs from layer 0's %d", l, d.hidden, d0->hidden);
    if (moe::layer_device(layers[l]) != moe::layer_device(layers[0]))
      return moe::api_fail(MOE_E_RANGE, "layer %d is on another device", l);
    if (!d0) d0 = &d;
  }
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return moe::api_fail(MOE_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (cur != moe::layer_device(layers[0]))
    return moe::api_fail(MOE_E_RANGE, "the current device is not the layers' device");
  moe_decoder* dec = new moe_decoder;
  dec->n = n_layers;
  dec->H = d0->hidden;
  dec->device = cur;
  const int H = dec->H;
  // one allocation: step counter, the n + 1 input slots, then per layer out, idx, gates and workspace
  std::vector<size_t> ws_bytes(n_layers);
  size_t total = 256;
  total += size_t(n_layers + 1) * round256(size_t(H) * 2);
  for (int l = 0; l < n_layers; ++l) {
    if (moe_status st = moe_workspace_bytes(layers[l], 1, &ws_bytes[l])) {
      destroy_all(dec);
      return st;
    }
    const int k = moe::layer_desc(layers[l]).top_k;
    total += round256(size_t(H) * 4) + 2 * round256(size_t(k) * 4) + round256(ws_bytes[l]);
  }
  if ((e = hipMalloc(&dec->dmem, total)) != hipSuccess) {
    destroy_all(dec);
    return moe::api_fail(MOE_E_HIP, "hipMalloc(%zu): %s", total, hipGetErrorString(e));
  }
  if ((e = hipMemset(dec->dmem, 0, total)) != hipSuccess ||
      (e = hipHostMalloc(reinterpret_cast<void**>(&dec->bells), size_t(n_layers) * 8,
                         hipHostMallocMapped | hipHostMallocCoherent)) != hipSuccess) {
    destroy_all(dec);
    return moe::api_fail(MOE_E_HIP, "decoder buffers: %s", hipGetErrorString(e));
  }
  for (int l = 0; l < n_layers; ++l) dec->bells[l] = 0ull;
  unsigned long long* dbells = nullptr;      // the device's address of the doorbells
  if ((e = hipHostGetDevicePointer(reinterpret_cast<void**>(&dbells), dec->bells, 0)) != hipSuccess) {
    destroy_all(dec);
    return moe::api_fail(MOE_E_HIP, "hipHostGetDevicePointer: %s", hipGetErrorString(e));
  }
  char* p = dec->dmem;
  auto* step = reinterpret_cast<unsigned long long*>(p);
  p += 256;
  for (int l = 0; l <= n_layers; ++l) {
    dec->x.push_back(reinterpret_cast<uint16_t*>(p));
    p += round256(size_t(H) * 2);
  }
  std::vector<char*> ws(n_layers);
  for (int l = 0; l < n_layers; ++l) {
    const int k = moe::layer_desc(layers[l]).top_k;
    dec->out.push_back(reinterpret_cast<float*>(p));
    p += round256(size_t(H) * 4);
    dec->idx.push_back(reinterpret_cast<int32_t*>(p));
    p += round256(size_t(k) * 4);
    dec->gates.push_back(reinterpret_cast<float*>(p));
    p += round256(size_t(k) * 4);
    ws[l] = p;
    p += round256(ws_bytes[l]);
  }
  // capture one graph per layer on a private stream (default priority)
  hipStream_t cs = nullptr;
  if ((e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking)) != hipSuccess) {
    destroy_all(dec);
    return moe::api_fail(MOE_E_HIP, "hipStreamCreate: %s", hipGetErrorString(e));
  }
  // the caller's stream's earlier work (the workspace clear above is synchronous)
  hipStream_t us = reinterpret_cast<hipStream_t>(stream);
  if ((e = hipStreamSynchronize(us)) != hipSuccess) {
    (void)hipStreamDestroy(cs);
    destroy_all(dec);
    return moe::api_fail(MOE_E_HIP, "hipStreamSynchronize: %s", hipGetErrorString(e));
  }
  moe_status st = MOE_OK;
  for (int l = 0; l < n_layers && st == MOE_OK; ++l) {
    hipGraph_t g = nullptr;
    if ((e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal)) != hipSuccess) {
      st = moe::api_fail(MOE_E_HIP, "hipStreamBeginCapture: %s", hipGetErrorString(e));
      break;
    }
    st = moe_grouped_forward(layers[l], dec->x[l], 1, dec->idx[l], dec->gates[l], MOE_ROUTE_INTERNAL, dec->out[l],
                             ws[l], ws_bytes[l], cs);
    if (st == MOE_OK) {
      hipLaunchKernelGGL(layer_epilogue_kernel, dim3(1), dim3(kEpilogueThreads), 0, cs, dec->x[l], dec->out[l],
                         dec->x[l + 1], H, step, dbells + l, l == n_layers - 1 ? 1 : 0);
      if ((e = hipGetLastError()) != hipSuccess) st = moe::api_fail(MOE_E_HIP, "epilogue launch: %s", hipGetErrorString(e));
    }
    const hipError_t ee = hipStreamEndCapture(cs, &g);
    if (st == MOE_OK && ee != hipSuccess) st = moe::api_fail(MOE_E_HIP, "hipStreamEndCapture: %s", hipGetErrorString(ee));
    dec->graph.push_back(g);
    if (st != MOE_OK) break;
    hipGraphExec_t x = nullptr;
    if ((e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0)) != hipSuccess) {
      st = moe::api_fail(MOE_E_HIP, "hipGraphInstantiate: %s", hipGetErrorString(e));
      break;
    }
    dec->exec.push_back(x);
  }
  (void)hipStreamDestroy(cs);
  // the whole token as one graph (one launch per token when the host does
  // not wait between layers): the layers' graphs as child nodes in a chain
  if (st == MOE_OK && (e = hipGraphCreate(&dec->token_graph, 0)) != hipSuccess)
    st = moe::api_fail(MOE_E_HIP, "hipGraphCreate: %s", hipGetErrorString(e));
  hipGraphNode_t prev = nullptr;
  for (int l = 0; l < n_layers && st == MOE_OK; ++l) {
    hipGraphNode_t node = nullptr;
    if ((e = hipGraphAddChildGraphNode(&node, dec->token_graph, prev ? &prev : nullptr, prev ? 1 : 0,
                                       dec->graph[l])) != hipSuccess)
      st = moe::api_fail(MOE_E_HIP, "hipGraphAddChildGraphNode: %s", hipGetErrorString(e));
    prev = node;
  }
  if (st == MOE_OK && (e = hipGraphInstantiate(&dec->token_exec, dec->token_graph, nullptr, nullptr, 0)) != hipSuccess)
    st = moe::api_fail(MOE_E_HIP, "hipGraphInstantiate(token): %s", hipGetErrorString(e));
  if (st != MOE_OK) {
    destroy_all(dec);
    return st;
  }
  dec->k = moe::layer_desc(layers[0]).top_k;
  *out = dec;
  return moe::api_ok();
}

moe_status moe_decoder_destroy(moe_decoder* d) {
  if (!d) return moe::api_ok();
  (void)hipDeviceSynchronize();            // no graph of the decoder may still run
  destroy_all(d);
  return moe::api_ok();
}

moe_status moe_decoder_buffers(const moe_decoder* d, int32_t layer, void** x, float** out, int32_t** idx,
                               float** gates) {
  if (!d) return moe::api_fail(MOE_E_NULL, "decoder is NULL");
  if (layer < 0 || layer > d->n) return moe::api_fail(MOE_E_RANGE, "layer %d outside [0, %d]", layer, d->n);
  if (x) *x = d->x[layer];
  const bool has = layer < d->n;             // layer n: only the result slot
  if (out) *out = has ? d->out[layer] : nullptr;
  if (idx) *idx = has ? d->idx[layer] : nullptr;
  if (gates) *gates = has ? d->gates[layer] : nullptr;
  return moe::api_ok();
}

moe_status moe_decoder_step(moe_decoder* d, void* stream, int32_t wait_doorbell) {
  if (!d) return moe::api_fail(MOE_E_NULL, "decoder is NULL");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const unsigned long long want = d->steps + 1ull;
  if (!wait_doorbell) {                      // one launch: the token graph
    const hipError_t e = hipGraphLaunch(d->token_exec, s);
    if (e != hipSuccess) return moe::api_fail(MOE_E_HIP, "hipGraphLaunch(token): %s", hipGetErrorString(e));
    d->steps = want;
    return moe::api_ok();
  }
  for (int l = 0; l < d->n; ++l) {
    hipError_t e = hipGraphLaunch(d->exec[l], s);
    if (e != hipSuccess) return moe::api_fail(MOE_E_HIP, "hipGraphLaunch(layer %d): %s", l, hipGetErrorString(e));
    if (l + 1 < d->n) {                      // the host launches layer l + 1 once layer l has rung
      const long long t0 = moe::host_clock_us();
      while (__atomic_load_n(d->bells + l, __ATOMIC_ACQUIRE) < want) {
        if (moe::host_clock_us() - t0 > kDoorbellSpinUs) {
          d->steps = want;                   // the launched layers still ring
          return moe::api_fail(MOE_E_HIP, "layer %d's doorbell did not ring within %lld us", l, kDoorbellSpinUs);
        }
      }
    }
  }
  d->steps = want;
  return moe::api_ok();
}

moe_status moe_decoder_doorbell(const moe_decoder* d, int32_t layer, uint64_t* step) {
  if (!d) return moe::api_fail(MOE_E_NULL, "decoder is NULL");
  if (!step) return moe::api_fail(MOE_E_NULL, "step is NULL");
  if (layer < 0 || layer >= d->n) return moe::api_fail(MOE_E_RANGE, "layer %d outside [0, %d)", layer, d->n);
  *step = __atomic_load_n(d->bells + layer, __ATOMIC_ACQUIRE);
  return moe::api_ok();
}

}  // extern "C"
