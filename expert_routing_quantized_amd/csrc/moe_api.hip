// C ABI of libmoe: argument validation, layer lifetime, workspace layout and
// the launch sequence of each entry point.  Every check that the host can
// make runs before anything is enqueued (a wrong expert geometry is refused
// rather than mis-indexed: pyshine source tour, Understanding the
// Architecture, paragraph on the expert hand-off).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <chrono>
#include <mutex>
#include <string>
#include <vector>

#include "select_screen.h"

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
  const uint32_t known =
      MOE_LAYER_FORCE_EXACT_REFINE | MOE_LAYER_SCREEN_ON | MOE_LAYER_SCREEN_OFF | MOE_LAYER_WINDOW_SCREEN_OFF;
  if (d->flags & ~known) return fail(MOE_E_RANGE, "unknown desc.flags bits 0x%x", d->flags);
  if ((d->flags & MOE_LAYER_SCREEN_ON) && (d->flags & MOE_LAYER_SCREEN_OFF))
    return fail(MOE_E_RANGE, "MOE_LAYER_SCREEN_ON and MOE_LAYER_SCREEN_OFF together");
  if ((d->flags & MOE_LAYER_SCREEN_ON) && (d->act_dtype != MOE_BF16 || d->hidden % 32))
    return fail(MOE_E_DTYPE, "the router screen needs bf16 activations and hidden %% 32 == 0");
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

moe::ScreenList screen_list(char* ws, const Workspace& W) {
  moe::ScreenList l;
  l.hint = reinterpret_cast<moe::HintWords*>(ws + W.hint);
  l.cnt8 = reinterpret_cast<unsigned char*>(ws + W.cnt8);
  l.list = reinterpret_cast<ulonglong2*>(ws + W.list);
  return l;
}

moe::WinList win_list(char* ws, const Workspace& W) {
  moe::WinList l;
  l.hint = reinterpret_cast<moe::HintWords*>(ws + W.hint);
  l.wcnt = reinterpret_cast<unsigned char*>(ws + W.wcnt);
  l.wlist = reinterpret_cast<ulonglong2*>(ws + W.wlist);
  return l;
}

bool window_on_screen(const Layer& L, int T) { return L.screen_win && T >= 2 && T <= moe::kWinMaxT; }

moe_status route_impl(const Layer& L, const void* x, int T, int32_t* idx, float* gates,
                      char* ws, const Workspace& W, hipStream_t s) {
  if (window_on_screen(L, T)) {   // verify windows: the int8 screen on MFMA, one list per token
    float* z8 = reinterpret_cast<float*>(ws + W.z);
    float* g8 = reinterpret_cast<float*>(ws + W.gmax);
    double* xq = reinterpret_cast<double*>(ws + W.xnorm);
    const moe::WinList list = win_list(ws, W);
    hipError_t e = moe::launch_screen_window(L, x, T, z8, g8, xq, &list, s);
    if (e != hipSuccess) return hip_fail(e, "window screen launch");
    e = moe::launch_select_screen_window(L, x, T, z8, g8, xq, &list, idx, gates, s);
    if (e != hipSuccess) return hip_fail(e, "window select launch");
    return MOE_OK;
  }
  if (T == 1 && L.screen) {     // the int8 first pass, then the selection recomputes its candidates
    float* z8 = reinterpret_cast<float*>(ws + W.z);
    float* g8 = reinterpret_cast<float*>(ws + W.gmax);
    double* xq = reinterpret_cast<double*>(ws + W.xnorm);
    const moe::ScreenList list = screen_list(ws, W);
    hipError_t e = moe::launch_screen(L, x, 1, z8, g8, xq, &list, s);
    if (e != hipSuccess) return hip_fail(e, "screen launch");
    e = moe::launch_select_screen(L, x, 1, z8, g8, xq, &list, idx, gates, s);
    if (e != hipSuccess) return hip_fail(e, "select launch");
    return MOE_OK;
  }
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

// ---------------------------------------------------------------- scratch
// Device scratch of moe_grouped_forward_noalloc, for callers that cannot
// allocate.  Each GPU holds its own copy until the process ends; in host
// code the array's name is only a stand-in, so the device address of each
// GPU's copy is looked up once, with that GPU current, and used everywhere
// host code needs the memory.
constexpr size_t kScratchBytes = size_t(8) << 20;
constexpr int kScratchMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kScratchMaxDevices];

// Device address of `scratch` on device `dev` (the current device).
hipError_t scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kScratchMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// Shared by moe_grouped_forward and moe_grouped_forward_noalloc: checks of
// everything but the workspace, then the launch sequence.
moe_status grouped_check(const Layer& L, const void* x, int32_t T, const int32_t* idx, const float* gates,
                         uint32_t flags, const float* out) {
  if (flags != MOE_ROUTE_INTERNAL && flags != MOE_ROUTE_GIVEN)
    return fail(MOE_E_RANGE, "flags=0x%x must be MOE_ROUTE_INTERNAL or MOE_ROUTE_GIVEN", flags);
  if (T < 0 || T > L.d.max_tokens) return fail(MOE_E_RANGE, "T=%d outside [0, max_tokens=%d]", T, L.d.max_tokens);
  if (L.host && T > moe::host_tier_tmax(L.host))
    return fail(MOE_E_RANGE, "T=%d: a layer with host-tier experts serves calls of at most %d tokens", T,
                moe::host_tier_tmax(L.host));
  if (T == 0) return MOE_OK;
  if (!x || !out) return fail(MOE_E_NULL, "x and out are required");
  if (flags == MOE_ROUTE_GIVEN && (!idx || !gates))
    return fail(MOE_E_NULL, "MOE_ROUTE_GIVEN needs idx and gates");
  if ((idx == nullptr) != (gates == nullptr))
    return fail(MOE_E_NULL, "idx and gates must both be given or both be NULL");
  if (!aligned(x, 16)) return fail(MOE_E_ALIGN, "x must be 16-byte aligned");
  if (!aligned(out, 4) || (idx && (!aligned(idx, 4) || !aligned(gates, 4))))
    return fail(MOE_E_ALIGN, "idx/gates/out must be 4-byte aligned");
  return MOE_OK;
}

moe_status grouped_impl(const Layer& L, const void* x, int32_t T, int32_t* idx, float* gates,
                        uint32_t flags, float* out, char* w, const Workspace& W, hipStream_t s) {
  int32_t* ri = idx ? idx : reinterpret_cast<int32_t*>(w + W.idx);
  float* rg = gates ? gates : reinterpret_cast<float*>(w + W.gates);
  if (flags == MOE_ROUTE_INTERNAL && T == 1 && L.screen && L.tiers == nullptr) {
    // batch-1 decode on the screen: the int8 first pass (with the list),
    // the selection fused with gate/up, then down + combine
    float* z8 = reinterpret_cast<float*>(w + W.z);
    float* g8 = reinterpret_cast<float*>(w + W.gmax);
    double* xq = reinterpret_cast<double*>(w + W.xnorm);
    const moe::ScreenList list = screen_list(w, W);
    hipError_t e = moe::launch_screen(L, x, 1, z8, g8, xq, &list, s);
    if (e != hipSuccess) return hip_fail(e, "screen launch");
    e = moe::launch_decode_screen(L, x, z8, g8, xq, &list, ri, rg, out, reinterpret_cast<float*>(w + W.h), s);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return MOE_OK;
  }
  if (flags == MOE_ROUTE_INTERNAL && !moe::router_uses_mfma(L, T) && moe::decode_fused_fits(L, T) && L.tiers == nullptr) {
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
    return MOE_OK;
  }
  if (flags == MOE_ROUTE_INTERNAL) {
    if (moe_status st = route_impl(L, x, T, ri, rg, w, W, s)) return st;
  }
  hipError_t e;
  if (L.host) {                  // the host tier's part on a second stream, beside the GPU's
    if ((e = moe::host_tier_fork(L.host, x, T, ri, rg, s)) != hipSuccess) return hip_fail(e, "host tier");
    e = moe::launch_pair_experts(L, x, T, ri, rg, out, reinterpret_cast<float*>(w + (T == 1 ? W.h : W.hm)), s);
    if (e != hipSuccess) return hip_fail(e, "expert launch");
    if ((e = moe::host_tier_join(L.host, T, out, s)) != hipSuccess) return hip_fail(e, "host tier");
    return MOE_OK;
  }
  if (T == 1)
    e = moe::launch_pair_experts(L, x, 1, ri, rg, out, reinterpret_cast<float*>(w + W.h), s);
  else if (!moe::grouped_uses_mfma(L, T) && moe::pair_path_fits(L, T))
    e = moe::launch_pair_experts(L, x, T, ri, rg, out, reinterpret_cast<float*>(w + W.hm), s);
  else
    e = moe::launch_grouped_experts(L, x, T, ri, rg, out, w, W, s);
  if (e != hipSuccess) return hip_fail(e, "expert launch");
  return MOE_OK;
}

}  // namespace

namespace moe {

moe_status api_fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status api_ok() { return ok(); }

const moe_layer_desc& layer_desc(const moe_layer* layer) { return layer->L.d; }

int layer_device(const moe_layer* layer) { return layer->L.device; }

long long host_clock_us() {
  return std::chrono::duration_cast<std::chrono::microseconds>(std::chrono::steady_clock::now().time_since_epoch())
      .count();
}

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
  if (L.screen) {      // first, at the same place for every T (the hint outlives the call)
    W.hint = take(sizeof(moe::HintWords));
    W.cnt8 = take(size_t(moe::screen_waves(L)) + 16);
    W.list = take(size_t(moe::kListSlots) * 16);
  }
  if (L.screen_win && T >= 2 && T <= moe::kWinMaxT) {
    W.wcnt = take(Tz * size_t(moe::screen_window_cstride(L)));
    W.wlist = take(Tz * size_t(moe::kListSlots) * 16);
  }
  W.z = take(Tz * E * 8);
  W.gmax = take(Tz * ((E + 3) / 4) * 4);
  W.xnorm = take(Tz * 16);
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
  if (L.q8) (void)hipFree(L.q8);
  if (L.sc8) (void)hipFree(L.sc8);
  if (L.eb8) (void)hipFree(L.eb8);
  if (L.screen_consts) (void)hipFree(L.screen_consts);
  if (L.q8w) (void)hipFree(L.q8w);
  if (L.hot_buf) (void)hipFree(L.hot_buf);
  delete L.hot_ids;
  moe::host_tier_destroy(L.host);
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
  if ((e = scratch_address(L.device, &L.scratch)) != hipSuccess)
    return cleanup(hip_fail(e, "hipGetSymbolAddress(scratch)"));
  if ((e = hipMalloc(&L.norms, (E + 1) * sizeof(float))) != hipSuccess)
    return cleanup(hip_fail(e, "hipMalloc(norms)"));
  // the sticky fault word, then (8-byte aligned) the count of exact refinements
  if ((e = hipMalloc(&L.dev_flag, moe::kDevWordsBytes)) != hipSuccess)
    return cleanup(hip_fail(e, "hipMalloc(flag)"));
  if ((e = hipMemsetAsync(L.dev_flag, 0, moe::kDevWordsBytes, s)) != hipSuccess)
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
  // the int8 first pass of the batch-1 router (layer-owned: E H bytes + 12 E)
  L.screen = desc->act_dtype == MOE_BF16 && H % 32 == 0 && !(desc->flags & MOE_LAYER_SCREEN_OFF) &&
             (E >= size_t(moe::kScreenMinExperts) || (desc->flags & MOE_LAYER_SCREEN_ON));
  float sconst[3] = {0.f, 0.f, 0.f};
  if (L.screen) {
    if ((e = hipMalloc(&L.q8, E * H)) != hipSuccess) return cleanup(hip_fail(e, "hipMalloc(screen router)"));
    if ((e = hipMalloc(&L.sc8, E * sizeof(float))) != hipSuccess) return cleanup(hip_fail(e, "hipMalloc(screen scales)"));
    if ((e = hipMalloc(&L.eb8, E * sizeof(float2))) != hipSuccess) return cleanup(hip_fail(e, "hipMalloc(screen norms)"));
    // 256 bytes: the three maxima, and a stand-in the screen reads in place of a hint
    if ((e = hipMalloc(&L.screen_consts, 256)) != hipSuccess)
      return cleanup(hip_fail(e, "hipMalloc(screen maxima)"));
    if ((e = moe::launch_screen_prep(L, L.screen_consts, s)) != hipSuccess) return cleanup(hip_fail(e, "screen prep"));
    if ((e = hipMemcpyAsync(sconst, L.screen_consts, sizeof(sconst), hipMemcpyDeviceToHost, s)) != hipSuccess)
      return cleanup(hip_fail(e, "screen maxima readback"));
    // verify windows' screen: the same int8 router in MFMA operand order
    if (moe::screen_window_fits(*desc)) {
      if ((e = hipMalloc(&L.q8w, moe::screen_window_bytes(*desc))) != hipSuccess)
        return cleanup(hip_fail(e, "hipMalloc(window screen router)"));
      if ((e = moe::launch_screen_window_prep(L, s)) != hipSuccess) return cleanup(hip_fail(e, "window screen prep"));
      L.screen_win = true;
    }
  }
  float nmax = 0.f;
  if ((e = hipMemcpyAsync(&nmax, L.norms + E, sizeof(float), hipMemcpyDeviceToHost, s)) != hipSuccess)
    return cleanup(hip_fail(e, "norm readback"));
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return cleanup(hip_fail(e, "hipStreamSynchronize"));
  if (!(nmax >= 0.f) || isinf(nmax)) return cleanup(fail(MOE_E_RANGE, "router weights are not finite"));
  L.norm_max = nmax;
  L.screen_enmax = sconst[0];
  L.screen_rqmax = sconst[1];
  L.screen_bmax = sconst[2];
  if (L.screen) {
    if (!(isfinite(sconst[0]) && isfinite(sconst[1]) && isfinite(sconst[2])))
      return cleanup(fail(MOE_E_RANGE, "router weights or bias are not finite"));
  }
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

moe_status moe_router_screen(const moe_layer* layer, const void* x, int32_t T, float* v, float* bound,
                             void* ws, size_t ws_bytes, void* stream) {
  if (moe_status st = check_layer(layer)) return st;
  const Layer& L = layer->L;
  if (!L.screen) return fail(MOE_E_DTYPE, "this layer has no router screen (bf16 activations, hidden %% 32 == 0, "
                                         "E >= %d or MOE_LAYER_SCREEN_ON)", moe::kScreenMinExperts);
  if (T < 0 || T > L.d.max_tokens) return fail(MOE_E_RANGE, "T=%d outside [0, max_tokens=%d]", T, L.d.max_tokens);
  if (T == 0) return ok();
  if (!x || !v) return fail(MOE_E_NULL, "x and v are required");
  if (!aligned(x, 16)) return fail(MOE_E_ALIGN, "x must be 16-byte aligned");
  if (!aligned(v, 4) || (bound && !aligned(bound, 4))) return fail(MOE_E_ALIGN, "v and bound must be 4-byte aligned");
  Workspace W;
  if (moe_status st = check_ws(L, T, ws, ws_bytes, &W)) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  float* g8 = reinterpret_cast<float*>(w + W.gmax);
  double* xq = reinterpret_cast<double*>(w + W.xnorm);
  hipError_t e = window_on_screen(L, T) ? moe::launch_screen_window(L, x, T, v, g8, xq, nullptr, s)
                                         : moe::launch_screen(L, x, T, v, g8, xq, nullptr, s);
  if (e == hipSuccess && bound) e = moe::launch_screen_bounds(L, T, v, xq, bound, s);
  if (e != hipSuccess) return hip_fail(e, "screen launch");
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
  hipError_t e;
  if (L.host && (e = moe::host_tier_fork(L.host, x, 1, idx, gates, s)) != hipSuccess) return hip_fail(e, "host tier");
  e = moe::launch_pair_experts(L, x, 1, idx, gates, out, h, s);
  if (e != hipSuccess) return hip_fail(e, "expert decode launch");
  if (L.host && (e = moe::host_tier_join(L.host, 1, out, s)) != hipSuccess) return hip_fail(e, "host tier");
  return ok();
}

moe_status moe_grouped_forward(const moe_layer* layer, const void* x, int32_t T, int32_t* idx,
                               float* gates, uint32_t flags, float* out, void* ws,
                               size_t ws_bytes, void* stream) {
  if (moe_status st = check_layer(layer)) return st;
  const Layer& L = layer->L;
  if (moe_status st = grouped_check(L, x, T, idx, gates, flags, out)) return st;
  if (T == 0) return ok();
  Workspace W;
  if (moe_status st = check_ws(L, T, ws, ws_bytes, &W)) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (moe_status st = grouped_impl(L, x, T, idx, gates, flags, out, static_cast<char*>(ws), W, s)) return st;
  return ok();
}

moe_status moe_grouped_forward_noalloc(const moe_layer* layer, const void* x, int32_t T, int32_t* idx,
                                       float* gates, uint32_t flags, float* out, void* stream) {
  if (moe_status st = check_layer(layer)) return st;
  const Layer& L = layer->L;
  if (moe_status st = grouped_check(L, x, T, idx, gates, flags, out)) return st;
  if (T == 0) return ok();
  const Workspace W = moe::workspace_layout(L, T);
  if (W.total > kScratchBytes)
    return fail(MOE_E_WORKSPACE, "T=%d needs %zu bytes of scratch, more than the %zu bytes of the "
                "library's device scratch (use moe_grouped_forward with a workspace)", T, W.total, kScratchBytes);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != L.device)
    return fail(MOE_E_RANGE, "current device %d is not the layer's device %d", dev, L.device);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (moe_status st = grouped_impl(L, x, T, idx, gates, flags, out, static_cast<char*>(L.scratch), W, s))
    return st;
  return ok();
}

}  // extern "C"

namespace {

// The tier table from the region's experts (L.hot_ids) and the host tier's:
// slot i of the region holds hot_ids[i]; with a host tier one more slot of
// zeros, which every host-tier expert points at (the GPU's part of such an
// expert is then exactly 0).  Synchronises `s`.
moe_status rebuild_tiers(Layer& L, hipStream_t s) {
  const int E = L.d.n_experts;
  hipError_t e = hipStreamSynchronize(s);            // earlier calls may still read the old table
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  if (L.hot_buf) (void)hipFree(L.hot_buf);
  L.hot_buf = nullptr;
  L.tiers = nullptr;
  L.n_hot = 0;
  const std::vector<int32_t> none;
  const std::vector<int32_t>& hot = L.hot_ids ? *L.hot_ids : none;
  const std::vector<int32_t>& cold = L.host ? moe::host_tier_ids(L.host) : none;
  const int n = int(hot.size());
  const int nslots = n + (cold.empty() ? 0 : 1);
  if (nslots == 0) return MOE_OK;
  std::vector<int32_t> loc(size_t(E), -1);
  for (int i = 0; i < n; ++i) loc[hot[i]] = i;
  for (int c : cold) loc[c] = n;
  // per-expert bytes of each array, in the pool's own layout
  const size_t H = L.d.hidden, I = L.d.inter, N = size_t(nslots);
  const bool q4 = L.d.expert_dtype == MOE_Q4B32;
  const size_t elt = L.d.expert_dtype == MOE_F32 ? 4 : 2;
  const size_t gu = q4 ? I * H / 2 : I * H * elt, dn = q4 ? H * I / 2 : H * I * elt;
  const size_t sgu = q4 ? I * (H / 32) * 2 : 0, sdn = q4 ? H * (I / 32) * 2 : 0;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = round_up(off + bytes, 256);
    return o;
  };
  const size_t o_rec = take(sizeof(moe::ExpertTiers)), o_loc = take(size_t(E) * 4), o_ids = take(N * 4);
  const size_t o_wg = take(N * gu), o_wu = take(N * gu), o_wd = take(N * dn);
  const size_t o_sg = take(N * sgu), o_su = take(N * sgu), o_sd = take(N * sdn);
  char* buf = nullptr;
  if ((e = hipMalloc(reinterpret_cast<void**>(&buf), off)) != hipSuccess) return hip_fail(e, "hipMalloc(hot region)");
  moe::ExpertTiers rec{};
  rec.loc = reinterpret_cast<const int32_t*>(buf + o_loc);
  rec.wg = buf + o_wg;
  rec.wu = buf + o_wu;
  rec.wd = buf + o_wd;
  rec.sg = q4 ? reinterpret_cast<const uint16_t*>(buf + o_sg) : nullptr;
  rec.su = q4 ? reinterpret_cast<const uint16_t*>(buf + o_su) : nullptr;
  rec.sd = q4 ? reinterpret_cast<const uint16_t*>(buf + o_sd) : nullptr;
  const int32_t* dids = reinterpret_cast<const int32_t*>(buf + o_ids);
  const size_t sizes[6] = {gu, gu, dn, sgu, sgu, sdn};
  const size_t offs[6] = {o_wg, o_wu, o_wd, o_sg, o_su, o_sd};
  const void* srcs[6] = {L.d.w_gate, L.d.w_up, L.d.w_down, L.d.s_gate, L.d.s_up, L.d.s_down};
  e = hipMemcpyAsync(buf + o_loc, loc.data(), size_t(E) * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess && n > 0) e = hipMemcpyAsync(buf + o_ids, hot.data(), size_t(n) * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(buf + o_rec, &rec, sizeof(rec), hipMemcpyHostToDevice, s);
  for (int a = 0; a < 6 && e == hipSuccess; ++a) {
    if (sizes[a] == 0) continue;
    e = moe::launch_gather_experts(srcs[a], buf + offs[a], sizes[a], dids, n, s);
    if (e == hipSuccess && nslots > n) e = hipMemsetAsync(buf + offs[a] + size_t(n) * sizes[a], 0, sizes[a], s);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    (void)hipStreamSynchronize(s);
    (void)hipFree(buf);
    return hip_fail(e, "hot region copies");
  }
  L.hot_buf = buf;
  L.tiers = reinterpret_cast<const moe::ExpertTiers*>(buf + o_rec);
  L.n_hot = n;
  return MOE_OK;
}

// ids distinct, in [0, E) and, when `other` is given, not in it.
moe_status check_ids(const Layer& L, const int32_t* ids, int n, const std::vector<int32_t>* other,
                     const char* other_name) {
  const int E = L.d.n_experts;
  if (n < 0 || n > E) return fail(MOE_E_RANGE, "n=%d outside [0, n_experts=%d]", n, E);
  if (n > 0 && !ids) return fail(MOE_E_NULL, "ids is NULL");
  std::vector<int32_t> seen(size_t(E), -1);
  if (other)
    for (int e : *other) seen[e] = -2;
  for (int i = 0; i < n; ++i) {
    const int e = ids[i];
    if (e < 0 || e >= E) return fail(MOE_E_RANGE, "ids[%d]=%d outside [0, %d)", i, e, E);
    if (seen[e] == -2) return fail(MOE_E_RANGE, "ids[%d]=%d is in the %s", i, e, other_name);
    if (seen[e] >= 0) return fail(MOE_E_RANGE, "ids[%d]=%d repeats ids[%d]", i, e, seen[e]);
    seen[e] = i;
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layer_set_hot_experts(moe_layer* layer, const int32_t* ids, int32_t n, void* stream) {
  if (moe_status st = check_layer(layer)) return st;
  Layer& L = layer->L;
  const std::vector<int32_t>* host = L.host ? &moe::host_tier_ids(L.host) : nullptr;
  if (moe_status st = check_ids(L, ids, n, host, "host tier")) return st;
  delete L.hot_ids;
  L.hot_ids = n > 0 ? new std::vector<int32_t>(ids, ids + n) : nullptr;
  if (moe_status st = rebuild_tiers(L, reinterpret_cast<hipStream_t>(stream))) return st;
  return ok();
}

moe_status moe_layer_set_host_experts(moe_layer* layer, const int32_t* ids, int32_t n, int32_t n_threads,
                                      void* stream) {
  if (moe_status st = check_layer(layer)) return st;
  Layer& L = layer->L;
  if (moe_status st = check_ids(L, ids, n, L.hot_ids, "hot region")) return st;
  if (n_threads < 0 || n_threads > 1024) return fail(MOE_E_RANGE, "n_threads=%d outside [0, 1024]", n_threads);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  moe::host_tier_destroy(L.host);
  L.host = nullptr;
  if (n > 0 && (e = moe::host_tier_create(L, ids, n, n_threads, s, &L.host)) != hipSuccess)
    return hip_fail(e, "host tier");
  if (moe_status st = rebuild_tiers(L, s)) return st;
  return ok();
}

moe_status moe_cpu_experts(const moe_layer_desc* desc, const void* x, int32_t T, const int32_t* idx,
                           const float* gates, float* out, int32_t n_threads) {
  if (!desc) return fail(MOE_E_NULL, "desc is NULL");
  const moe_layer_desc& d = *desc;
  if (d.act_dtype != MOE_F32 && d.act_dtype != MOE_BF16)
    return fail(MOE_E_DTYPE, "act_dtype %d unsupported (MOE_F32 or MOE_BF16)", d.act_dtype);
  if (d.expert_dtype != MOE_F32 && d.expert_dtype != MOE_BF16 && d.expert_dtype != MOE_Q4B32)
    return fail(MOE_E_DTYPE, "expert_dtype %d unsupported", d.expert_dtype);
  const int mult = (d.expert_dtype == MOE_Q4B32) ? 32 : 8;
  if (d.hidden < 8 || d.hidden > moe::kMaxH || d.hidden % mult || d.inter < 8 || d.inter > moe::kMaxI ||
      d.inter % mult || d.n_experts < 1 || d.top_k < 1 || d.top_k > moe::kMaxK)
    return fail(MOE_E_GEOMETRY, "hidden=%d inter=%d n_experts=%d top_k=%d unsupported", d.hidden, d.inter,
                d.n_experts, d.top_k);
  if (!d.w_gate || !d.w_up || !d.w_down) return fail(MOE_E_NULL, "w_gate, w_up and w_down are required");
  const bool q4 = d.expert_dtype == MOE_Q4B32;
  if (q4 && (!d.s_gate || !d.s_up || !d.s_down)) return fail(MOE_E_NULL, "4-bit experts need s_gate, s_up and s_down");
  if (T < 0) return fail(MOE_E_RANGE, "T=%d is negative", T);
  if (T == 0) return ok();
  if (!x || !idx || !gates || !out) return fail(MOE_E_NULL, "x, idx, gates and out are required");
  if (n_threads < 0 || n_threads > 1024) return fail(MOE_E_RANGE, "n_threads=%d outside [0, 1024]", n_threads);
  moe::cpu_experts(d, x, T, idx, gates, out, n_threads == 0 ? 1 : n_threads);
  return ok();
}

moe_status moe_expert_counts(const moe_layer* layer, const int32_t* idx, int32_t n, uint32_t* counts,
                             void* stream) {
  if (moe_status st = check_layer(layer)) return st;
  if (n < 0) return fail(MOE_E_RANGE, "n=%d is negative", n);
  if (n == 0) return ok();
  if (!idx || !counts) return fail(MOE_E_NULL, "idx and counts are required");
  if (!aligned(idx, 4) || !aligned(counts, 4)) return fail(MOE_E_ALIGN, "idx and counts must be 4-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = moe::launch_expert_counts(idx, n, layer->L.d.n_experts, counts, s);
  if (e != hipSuccess) return hip_fail(e, "expert counts launch");
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

moe_status moe_layer_stats(const moe_layer* layer, void* stream, uint64_t* exact_refinements) {
  if (moe_status st = check_layer(layer)) return st;
  if (!exact_refinements) return fail(MOE_E_NULL, "exact_refinements is NULL");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  unsigned long long v = 0;
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemcpy(&v, moe::refine_counter(layer->L.dev_flag), sizeof(v), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "moe_layer_stats");
  *exact_refinements = v;
  return ok();
}

}  // extern "C"
