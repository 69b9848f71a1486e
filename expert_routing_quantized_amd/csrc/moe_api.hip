// C ABI of libmoe: argument validation, layer lifetime, workspace layout and
// the launch sequence of each entry point.  Every check that the host can
// make runs before anything is enqueued (a wrong expert geometry is refused
// rather than mis-indexed: pyshine source tour, "The expert handoff is a
// verified contract").
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>

#include "moe_internal.h"

using moe::Layer;
using moe::Workspace;

struct moe_layer {
  Layer L;
};

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status ok() {
  g_last_error.clear();
  return MOE_OK;
}

moe_status hip_fail(hipError_t e, const char* where) {
  return fail(MOE_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t act_bytes(int dt) { return dt == MOE_BF16 ? 2 : 4; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

moe_status validate_desc(const moe_layer_desc* d) {
  if (!d) return fail(MOE_E_NULL, "desc is NULL");
  const int H = d->hidden, E = d->n_experts, k = d->top_k, I = d->inter;
  if (d->act_dtype != MOE_F32 && d->act_dtype != MOE_BF16)
    return fail(MOE_E_DTYPE, "act_dtype %d unsupported (MOE_F32 or MOE_BF16)", d->act_dtype);
  if (d->expert_dtype != MOE_F32 && d->expert_dtype != MOE_BF16 && d->expert_dtype != MOE_Q4B32)
    return fail(MOE_E_DTYPE, "expert_dtype %d unsupported", d->expert_dtype);
  if (d->expert_dtype == MOE_F32 && d->act_dtype != MOE_F32)
    return fail(MOE_E_DTYPE, "fp32 experts need fp32 activations");
  if (d->router_layout != MOE_ROUTER_HE && d->router_layout != MOE_ROUTER_EH)
    return fail(MOE_E_DTYPE, "router_layout %d unsupported", d->router_layout);
  if (d->flags & ~MOE_LAYER_FORCE_EXACT_REFINE) return fail(MOE_E_RANGE, "unknown desc.flags bits 0x%x", d->flags);
  const int mult = (d->expert_dtype == MOE_Q4B32) ? 32 : 8;
  if (H < 8 || H > moe::kMaxH || H % mult)
    return fail(MOE_E_GEOMETRY, "hidden=%d must be a multiple of %d in [8, %d]", H, mult, moe::kMaxH);
  if (I < 8 || I > moe::kMaxI || I % mult)
    return fail(MOE_E_GEOMETRY, "inter=%d must be a multiple of %d in [8, %d]", I, mult, moe::kMaxI);
  if (E < 1 || E > (1 << 20)) return fail(MOE_E_GEOMETRY, "n_experts=%d outside [1, 2^20]", E);
  if (k < 1 || k > E || k > moe::kMaxK)
    return fail(MOE_E_GEOMETRY, "top_k=%d outside [1, min(E=%d, %d)]", k, E, moe::kMaxK);
  if (d->max_tokens < 1 || d->max_tokens > 65536)
    return fail(MOE_E_GEOMETRY, "max_tokens=%d outside [1, 65536]", d->max_tokens);
  if (!d->router_w || !d->w_gate || !d->w_up || !d->w_down)
    return fail(MOE_E_NULL, "router_w, w_gate, w_up and w_down are required");
  const bool q4 = d->expert_dtype == MOE_Q4B32;
  if (q4 && (!d->s_gate || !d->s_up || !d->s_down))
    return fail(MOE_E_NULL, "4-bit experts need s_gate, s_up and s_down");
  if (!q4 && (d->s_gate || d->s_up || d->s_down))
    return fail(MOE_E_DTYPE, "scales given for experts that are not 4-bit");
  if (!aligned(d->router_w, 16) || !aligned(d->w_gate, 16) || !aligned(d->w_up, 16) ||
      !aligned(d->w_down, 16))
    return fail(MOE_E_ALIGN, "router and expert weights must be 16-byte aligned");
  if (d->router_bias && !aligned(d->router_bias, 4)) return fail(MOE_E_ALIGN, "router_bias must be 4-byte aligned");
  if (q4 && (!aligned(d->s_gate, 2) || !aligned(d->s_up, 2) || !aligned(d->s_down, 2)))
    return fail(MOE_E_ALIGN, "scales must be 2-byte aligned");
  return MOE_OK;
}

moe_status check_layer(const moe_layer* l) {
  if (!l) return fail(MOE_E_NULL, "layer is NULL");
  return MOE_OK;
}

moe_status check_ws(const Layer& L, int T, const void* ws, size_t ws_bytes, Workspace* W) {
  *W = moe::workspace_layout(L, T);
  if (!ws) return fail(MOE_E_WORKSPACE, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(MOE_E_ALIGN, "workspace must be 256-byte aligned");
  if (ws_bytes < W->total)
    return fail(MOE_E_WORKSPACE, "workspace of %zu bytes < %zu needed for T=%d", ws_bytes, W->total, T);
  return MOE_OK;
}

moe_status route_impl(const Layer& L, const void* x, int T, int32_t* idx, float* gates,
                      char* ws, const Workspace& W, hipStream_t s) {
  // the selection reads binary32 logits from the big-tile GEMM (half the bytes to write)
  void* z = ws + W.z;
  float* gmax = reinterpret_cast<float*>(ws + W.gmax);
  double* xnorm = reinterpret_cast<double*>(ws + W.xnorm);
  const bool z32 = moe::router_uses_mfma(L, T) && moe::router_logits_f32(L, T);
  hipError_t e = moe::router_uses_mfma(L, T)
                     ? moe::launch_router_gemm(L, x, T, z, z32, gmax, xnorm, s)
                     : moe::launch_router(L, x, T, static_cast<double*>(z), gmax, xnorm, s);
  if (e != hipSuccess) return hip_fail(e, "router launch");
  e = moe::launch_select_impl(L, x, T, z, z32, gmax, xnorm, idx, gates, moe::router_bound(L, T), s);
  if (e != hipSuccess) return hip_fail(e, "select launch");
  return MOE_OK;
}

}  // namespace

namespace moe {

Workspace workspace_layout(const Layer& L, int T) {
  Workspace W{};
  const size_t E = L.d.n_experts, k = L.d.top_k, I = L.d.inter, H = L.d.hidden;
  const size_t Tz = T < 1 ? 1 : size_t(T);
  const size_t P = Tz * k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = round_up(off + bytes, 256);
    return o;
  };
  W.z = take(Tz * E * 8);
  W.gmax = take(Tz * ((E + 3) / 4) * 4);
  W.xnorm = take(Tz * 8);
  W.idx = take(P * 4);
  W.gates = take(P * 4);
  W.h = take(k * I * 4);
  if (Tz > 1) {
    W.counts = take(E * 4);
    W.offsets = take((E + 1) * 4);
    W.slot = take(P * 4);
    W.pos = take(P * 4);
    W.ptok = take(P * 4);
    W.active = take((E + 1) * 4);
    W.tiles = take((1 + 2 * ((P + moe::kTileRows - 1) / moe::kTileRows + std::min(P, E))) * 4);
    W.tiles_big = take((1 + 2 * ((P + moe::kBigTileRows - 1) / moe::kBigTileRows + std::min(P, E))) * 4);
    W.hm = take(P * I * 4);
    W.y = take(P * H * 4);
  }
  W.total = off;
  return W;
}

}  // namespace moe

extern "C" {

int32_t moe_abi_version(void) { return 1; }

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_E_NULL: return "MOE_E_NULL: a required pointer is NULL";
    case MOE_E_GEOMETRY: return "MOE_E_GEOMETRY: shapes inconsistent or unsupported";
    case MOE_E_DTYPE: return "MOE_E_DTYPE: unsupported dtype or combination";
    case MOE_E_ALIGN: return "MOE_E_ALIGN: pointer misaligned";
    case MOE_E_WORKSPACE: return "MOE_E_WORKSPACE: workspace missing or too small";
    case MOE_E_RANGE: return "MOE_E_RANGE: argument out of range";
    case MOE_E_HIP: return "MOE_E_HIP: HIP runtime error";
    case MOE_E_DEVICE_FLAG: return "MOE_E_DEVICE_FLAG: device-side fault recorded";
  }
  return "unknown moe_status";
}

const char* moe_last_error_message(void) { return g_last_error.c_str(); }

// Frees what a layer owns (fields still null are skipped).
static void release_layer(Layer& L) {
  if (L.router_copy) (void)hipFree(L.router_copy);
  if (L.norms) (void)hipFree(L.norms);
  if (L.dev_flag) (void)hipFree(L.dev_flag);
  if (L.zero_bias) (void)hipFree(L.zero_bias);
}

moe_status moe_layer_create(const moe_layer_desc* desc, void* stream, moe_layer** out) {
  if (!out) return fail(MOE_E_NULL, "out is NULL");
  *out = nullptr;
  moe_status st = validate_desc(desc);
  if (st != MOE_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  moe_layer* l = new moe_layer();
  Layer& L = l->L;
  L.d = *desc;
  hipError_t e = hipGetDevice(&L.device);
  const size_t E = desc->n_experts, H = desc->hidden;
  auto cleanup = [&](moe_status code) {
    release_layer(L);
    delete l;
    return code;
  };
  if (e != hipSuccess) return cleanup(hip_fail(e, "hipGetDevice"));
  if ((e = hipMalloc(&L.norms, (E + 1) * sizeof(float))) != hipSuccess)
    return cleanup(hip_fail(e, "hipMalloc(norms)"));
  if ((e = hipMalloc(&L.dev_flag, sizeof(int))) != hipSuccess)
    return cleanup(hip_fail(e, "hipMalloc(flag)"));
  if ((e = hipMemsetAsync(L.dev_flag, 0, sizeof(int), s)) != hipSuccess)
    return cleanup(hip_fail(e, "hipMemsetAsync(flag)"));
  if (!desc->router_bias) {
    if ((e = hipMalloc(&L.zero_bias, E * sizeof(float))) != hipSuccess)
      return cleanup(hip_fail(e, "hipMalloc(zero bias)"));
    if ((e = hipMemsetAsync(L.zero_bias, 0, E * sizeof(float), s)) != hipSuccess)
      return cleanup(hip_fail(e, "hipMemsetAsync(zero bias)"));
  }
  if (desc->router_layout == MOE_ROUTER_HE) {
    if ((e = hipMalloc(&L.router_copy, E * H * act_bytes(desc->act_dtype))) != hipSuccess)
      return cleanup(hip_fail(e, "hipMalloc(router copy)"));
    if ((e = moe::launch_transpose_router(L, L.router_copy, s)) != hipSuccess)
      return cleanup(hip_fail(e, "router transpose"));
    L.router_eh = L.router_copy;
  } else {
    L.router_eh = desc->router_w;
  }
  if ((e = moe::launch_router_norms(L, s)) != hipSuccess) return cleanup(hip_fail(e, "router norms"));
  float nmax = 0.f;
  if ((e = hipMemcpyAsync(&nmax, L.norms + E, sizeof(float), hipMemcpyDeviceToHost, s)) != hipSuccess)
    return cleanup(hip_fail(e, "norm readback"));
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return cleanup(hip_fail(e, "hipStreamSynchronize"));
  if (!(nmax >= 0.f) || isinf(nmax)) return cleanup(fail(MOE_E_RANGE, "router weights are not finite"));
  L.norm_max = nmax;
  *out = l;
  return ok();
}

moe_status moe_layer_destroy(moe_layer* layer) {
  if (!layer) return ok();
  release_layer(layer->L);
  delete layer;
  return ok();
}

moe_status moe_workspace_bytes(const moe_layer* layer, int32_t T, size_t* bytes) {
  if (moe_status st = check_layer(layer)) return st;
  if (!bytes) return fail(MOE_E_NULL, "bytes is NULL");
  if (T < 0 || T > layer->L.d.max_tokens)
    return fail(MOE_E_RANGE, "T=%d outside [0, max_tokens=%d]", T, layer->L.d.max_tokens);
  *bytes = moe::workspace_layout(layer->L, T).total;
  return ok();
}

moe_status moe_route(const moe_layer* layer, const void* x, int32_t T, int32_t* idx, float* gates,
                     void* ws, size_t ws_bytes, void* stream) {
  if (moe_status st = check_layer(layer)) return st;
  const Layer& L = layer->L;
  if (T < 0 || T > L.d.max_tokens) return fail(MOE_E_RANGE, "T=%d outside [0, max_tokens=%d]", T, L.d.max_tokens);
  if (T == 0) return ok();
  if (!x || !idx || !gates) return fail(MOE_E_NULL, "x, idx and gates are required");
  if (!aligned(x, 16)) return fail(MOE_E_ALIGN, "x must be 16-byte aligned");
  if (!aligned(idx, 4) || !aligned(gates, 4)) return fail(MOE_E_ALIGN, "idx/gates must be 4-byte aligned");
  Workspace W;
  if (moe_status st = check_ws(L, T, ws, ws_bytes, &W)) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (moe_status st = route_impl(L, x, T, idx, gates, static_cast<char*>(ws), W, s)) return st;
  return ok();
}

moe_status moe_router_logits(const moe_layer* layer, const void* x, int32_t T, double* z, void* ws,
                             size_t ws_bytes, void* stream) {
  if (moe_status st = check_layer(layer)) return st;
  const Layer& L = layer->L;
  if (T < 0 || T > L.d.max_tokens) return fail(MOE_E_RANGE, "T=%d outside [0, max_tokens=%d]", T, L.d.max_tokens);
  if (T == 0) return ok();
  if (!x || !z) return fail(MOE_E_NULL, "x and z are required");
  if (!aligned(x, 16)) return fail(MOE_E_ALIGN, "x must be 16-byte aligned");
  if (!aligned(z, 8)) return fail(MOE_E_ALIGN, "z must be 8-byte aligned");
  Workspace W;
  if (moe_status st = check_ws(L, T, ws, ws_bytes, &W)) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  float* gm = reinterpret_cast<float*>(w + W.gmax);
  double* xn = reinterpret_cast<double*>(w + W.xnorm);
  hipError_t e = moe::router_uses_mfma(L, T) ? moe::launch_router_gemm(L, x, T, z, false, gm, xn, s)
                                             : moe::launch_router(L, x, T, z, gm, xn, s);
  if (e != hipSuccess) return hip_fail(e, "router launch");
  return ok();
}

moe_status moe_expert_decode(const moe_layer* layer, const void* x, const int32_t* idx,
                             const float* gates, float* out, void* ws, size_t ws_bytes,
                             void* stream) {
  if (moe_status st = check_layer(layer)) return st;
  const Layer& L = layer->L;
  if (!x || !idx || !gates || !out) return fail(MOE_E_NULL, "x, idx, gates and out are required");
  if (!aligned(x, 16)) return fail(MOE_E_ALIGN, "x must be 16-byte aligned");
  if (!aligned(idx, 4) || !aligned(gates, 4) || !aligned(out, 4))
    return fail(MOE_E_ALIGN, "idx/gates/out must be 4-byte aligned");
  Workspace W;
  if (moe_status st = check_ws(L, 1, ws, ws_bytes, &W)) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float* h = reinterpret_cast<float*>(static_cast<char*>(ws) + W.h);
  hipError_t e = moe::launch_pair_experts(L, x, 1, idx, gates, out, h, s);
  if (e != hipSuccess) return hip_fail(e, "expert decode launch");
  return ok();
}

moe_status moe_grouped_forward(const moe_layer* layer, const void* x, int32_t T, int32_t* idx,
                               float* gates, uint32_t flags, float* out, void* ws,
                               size_t ws_bytes, void* stream) {
  if (moe_status st = check_layer(layer)) return st;
  const Layer& L = layer->L;
  if (flags != MOE_ROUTE_INTERNAL && flags != MOE_ROUTE_GIVEN)
    return fail(MOE_E_RANGE, "flags=0x%x must be MOE_ROUTE_INTERNAL or MOE_ROUTE_GIVEN", flags);
  if (T < 0 || T > L.d.max_tokens) return fail(MOE_E_RANGE, "T=%d outside [0, max_tokens=%d]", T, L.d.max_tokens);
  if (T == 0) return ok();
  if (!x || !out) return fail(MOE_E_NULL, "x and out are required");
  if (flags == MOE_ROUTE_GIVEN && (!idx || !gates))
    return fail(MOE_E_NULL, "MOE_ROUTE_GIVEN needs idx and gates");
  if ((idx == nullptr) != (gates == nullptr))
    return fail(MOE_E_NULL, "idx and gates must both be given or both be NULL");
  if (!aligned(x, 16)) return fail(MOE_E_ALIGN, "x must be 16-byte aligned");
  if (!aligned(out, 4) || (idx && (!aligned(idx, 4) || !aligned(gates, 4))))
    return fail(MOE_E_ALIGN, "idx/gates/out must be 4-byte aligned");
  Workspace W;
  if (moe_status st = check_ws(L, T, ws, ws_bytes, &W)) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  int32_t* ri = idx ? idx : reinterpret_cast<int32_t*>(w + W.idx);
  float* rg = gates ? gates : reinterpret_cast<float*>(w + W.gates);
  if (flags == MOE_ROUTE_INTERNAL && !moe::router_uses_mfma(L, T) && moe::decode_fused_fits(L, T)) {
    // batch-1 decode: router, then the selection fused with gate/up, then
    // down + combine
    double* z = reinterpret_cast<double*>(w + W.z);
    float* gmax = reinterpret_cast<float*>(w + W.gmax);
    double* xnorm = reinterpret_cast<double*>(w + W.xnorm);
    hipError_t e = moe::launch_router(L, x, T, z, gmax, xnorm, s);
    if (e != hipSuccess) return hip_fail(e, "router launch");
    e = moe::launch_decode_fused(L, x, T, z, gmax, xnorm, moe::router_bound(L, T), ri, rg, out,
                              reinterpret_cast<float*>(w + (T == 1 ? W.h : W.hm)), s);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return ok();
  }
  if (flags == MOE_ROUTE_INTERNAL) {
    if (moe_status st = route_impl(L, x, T, ri, rg, w, W, s)) return st;
  }
  hipError_t e;
  if (T == 1)
    e = moe::launch_pair_experts(L, x, 1, ri, rg, out, reinterpret_cast<float*>(w + W.h), s);
  else if (!moe::grouped_uses_mfma(L, T) && moe::pair_path_fits(L, T))
    e = moe::launch_pair_experts(L, x, T, ri, rg, out, reinterpret_cast<float*>(w + W.hm), s);
  else
    e = moe::launch_grouped_experts(L, x, T, ri, rg, out, w, W, s);
  if (e != hipSuccess) return hip_fail(e, "expert launch");
  return ok();
}

moe_status moe_device_error(const moe_layer* layer, void* stream, int32_t* code) {
  if (moe_status st = check_layer(layer)) return st;
  if (!code) return fail(MOE_E_NULL, "code is NULL");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int v = 0;
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemcpy(&v, layer->L.dev_flag, sizeof(int), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemset(layer->L.dev_flag, 0, sizeof(int));
  if (e != hipSuccess) return hip_fail(e, "moe_device_error");
  *code = v;
  if (v) return fail(MOE_E_DEVICE_FLAG, "device fault bits 0x%x", v);
  return ok();
}

}  // extern "C"
