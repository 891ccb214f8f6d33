// C-ABI host library: argument validation, workspace carving and the launch
// sequence of the layer. Every entry point validates before enqueuing
// anything, never throws across the ABI and never synchronises the stream.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "lcmoe.h"
#include "kernels.h"

// Workspace of lcmoe_forward_noalloc: one fixed array in the library's code
// object, so each device that runs the library holds its own copy until the
// process ends. Host code never passes this name to a kernel (on the host it
// is a stand-in, not a device address): the device address of each copy
// comes from hipGetSymbolAddress, looked up once per device.
constexpr size_t kNoallocScratchBytes = LCMOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

using namespace lcmoe;

constexpr size_t kAlign = 256;

// Device addresses of `scratch`, per device id, filled on each device's
// first no-allocation call with that device current.
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

lcmoe_status noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return LCMOE_ERR_HIP;
  }
  if (dev >= kMaxDevices) return LCMOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return LCMOE_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LCMOE_OK;
}

struct Layout {
  int ks = 1, kchunk = 0, ntile = 0;
  long long smax = 0;
  size_t zpart = 0, masks = 0, tilecnt = 0, tileoff = 0, offsets = 0, mt_prefix = 0,
         meta = 0, routing_end = 0, perm = 0, row_of_slot = 0, permute_end = 0, H = 0, Y = 0,
         xq = 0, xs = 0, hq = 0, hs = 0, total = 0;
};

inline long long n_experts(const lcmoe_shape& s) { return (long long)s.n_ffn + s.n_zero; }

lcmoe_status check_shape(const lcmoe_shape* s) {
  if (s == nullptr) return LCMOE_ERR_INVALID_ARG;
  if (s->n_ffn < 1 || s->n_zero < 0 || s->top_k < 1 || s->d_model < 1 || s->d_expert < 1)
    return LCMOE_ERR_INVALID_ARG;
  if (s->top_k > n_experts(*s)) return LCMOE_ERR_INVALID_ARG;
  if (s->w_dtype != LCMOE_W_BF16 && s->w_dtype != LCMOE_W_FP8_E4M3_B128 &&
      s->w_dtype != LCMOE_W_FP8_E4M3_B128_A8)
    return LCMOE_ERR_INVALID_ARG;
  if (s->top_k > 64 || n_experts(*s) > 2048) return LCMOE_ERR_UNSUPPORTED;
  if (s->d_model % 32 != 0 || s->d_expert % 32 != 0) return LCMOE_ERR_UNSUPPORTED;
  // One expert's gate/up matrix is addressed with 32-bit byte offsets.
  const long long wbytes = s->w_dtype == LCMOE_W_BF16 ? 2 : 1;
  if (2ll * s->d_expert * s->d_model * wbytes >= (1ll << 32)) return LCMOE_ERR_UNSUPPORTED;
  if (s->w_dtype != LCMOE_W_BF16 &&
      (s->d_model % 128 != 0 || s->d_expert % 128 != 0 || s->d_model > 16384 ||
       s->d_expert > 16384))
    return LCMOE_ERR_UNSUPPORTED;
  return LCMOE_OK;
}

// Router split-K factor: enough blocks (about two per CU) to cover the chip
// at small T; each split keeps at least 4 k-stages of 32.
void router_splits(int T, int E, int d, int& ks, int& kchunk) {
  const long long base = (long long)((T + 255) / 256) * ((E + 127) / 128);
  const int nstages = d / 32;
  int k = (int)std::min<long long>(32, std::max<long long>(1, 512 / std::max<long long>(base, 1)));
  k = std::min(k, std::max(1, nstages / 4));
  const int st_per = (nstages + k - 1) / k;
  kchunk = st_per * 32;
  ks = (d + kchunk - 1) / kchunk;
}

Layout make_layout(const lcmoe_shape& s, int T) {
  Layout L;
  const long long E = n_experts(s), N = s.n_ffn, K = s.top_k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + kAlign - 1) / kAlign * kAlign;
    return o;
  };
  router_splits(T, (int)E, s.d_model, L.ks, L.kchunk);
  L.ntile = (T + 63) / 64;
  L.zpart = take((size_t)L.ks * T * E * 4);
  L.masks = take((size_t)L.ntile * E * 8);
  L.tilecnt = take((size_t)L.ntile * E * 4);
  L.tileoff = take((size_t)L.ntile * E * 4);
  L.offsets = take((size_t)(N + 1) * 4);
  L.mt_prefix = take((size_t)(N + 1) * 4);
  L.meta = take(64);
  L.routing_end = off;
  L.perm = take((size_t)T * K * 4);
  L.row_of_slot = take((size_t)T * K * 4);
  L.permute_end = off;
  L.smax = (long long)T * std::min(K, N);
  L.H = take((size_t)L.smax * s.d_expert * 2);
  L.Y = take((size_t)L.smax * s.d_model * 2);
  if (s.w_dtype == LCMOE_W_FP8_E4M3_B128_A8) {
    // fp8 activations: codes and per-row scales of x and of H.
    L.xq = take((size_t)T * s.d_model);
    L.xs = take((size_t)T * 4);
    L.hq = take((size_t)L.smax * s.d_expert);
    L.hs = take((size_t)L.smax * 4);
  }
  L.total = off;
  return L;
}

// Backward workspace: the routing and permutation regions of the forward
// layout, then the backward's own buffers (S = T * min(K, N) slot rows).
struct BwdLayout {
  Layout f;
  size_t idx = 0, gate = 0, counts = 0, logits = 0, tprefix = 0, bprefix = 0, bmeta = 0, Xs = 0,
         dYs = 0, Q = 0, dU = 0, Hg = 0, dgp = 0, dXs = 0, dg = 0, dzp = 0, dzt = 0, wsp = 0,
         rg = 0, dxr = 0, total = 0;
  int nslices = 0;  // 128-column blocks of the gate/up pass (dg partials per row: 4 per block)
  int Ep = 0;  // experts padded to a multiple of 64 (router-gradient planes)
};

BwdLayout make_bwd_layout(const lcmoe_shape& s, int T) {
  BwdLayout B;
  B.f = make_layout(s, T);
  const long long E = n_experts(s), K = s.top_k, N = s.n_ffn, d = s.d_model, I = s.d_expert;
  const long long S = B.f.smax;
  size_t off = B.f.permute_end;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + kAlign - 1) / kAlign * kAlign;
    return o;
  };
  B.idx = take((size_t)T * K * 4);
  B.gate = take((size_t)T * K * 4);
  B.counts = take((size_t)E * 4);
  B.logits = take((size_t)T * E * 4);
  B.tprefix = take((size_t)(N + 1) * 4);
  B.bprefix = take((size_t)(N + 1) * 4);
  B.bmeta = take(16);
  B.Xs = take((size_t)S * d * 2);
  B.dYs = take((size_t)S * d * 2);
  B.Q = take((size_t)S * I * 4);
  B.dU = take((size_t)S * 2 * I * 2);
  B.Hg = take((size_t)S * I * 2);
  B.nslices = (int)((I + kBigColsGateUp - 1) / kBigColsGateUp);
  B.dgp = take((size_t)S * 4 * B.nslices * 4);
  B.dXs = take((size_t)S * d * 4);
  B.dg = take((size_t)T * K * 4);
  B.Ep = (int)((E + 63) / 64 * 64);
  B.dzp = take((size_t)T * 6 * B.Ep * 2);
  B.dzt = take((size_t)3 * T * B.Ep * 2);
  B.wsp = take((size_t)6 * B.Ep * d * 2);
  B.rg = take(64);
  B.dxr = take((size_t)T * d * 4);
  B.total = off;
  return B;
}

// The backward's second stream, per device id: the weight-gradient GEMMs
// (write-bound) run on it beside the data-gradient GEMM (read-bound) on the
// caller's stream, forked and joined with events. Default priority. Created
// on a device's first backward call with that device current; g_aux_mu is
// held from the fork to the join of each call, so calls from several host
// threads never interleave their use of the events.
struct AuxStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_aux_mu;
AuxStream g_aux[kMaxDevices];

lcmoe_status aux_stream(AuxStream** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return LCMOE_ERR_HIP;
  }
  if (dev >= kMaxDevices) return LCMOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_aux_mu);
  AuxStream& a = g_aux[dev];
  if (a.s == nullptr) {
    hipStream_t s = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&j, hipEventDisableTiming) != hipSuccess) {
      if (j != nullptr) (void)hipEventDestroy(j);
      if (f != nullptr) (void)hipEventDestroy(f);
      if (s != nullptr) (void)hipStreamDestroy(s);
      (void)hipGetLastError();
      return LCMOE_ERR_HIP;
    }
    a.s = s;
    a.fork = f;
    a.join = j;
  }
  *out = &a;
  return LCMOE_OK;
}

// Share of the CUs (in eighths) the weight-gradient GEMMs run on while the
// data-gradient GEMM runs beside them (measured at the LongCat prefill batch:
// 4/8 and 8/8 slower, 5/8 and 6/8 within 1%).
constexpr int kBwdWgradEighths = 6;

// Largest layout over every T <= tmax, so a workspace sized for tmax serves
// any smaller call and the size is non-decreasing in tmax. Every region
// grows with T except the router's split-K partials, whose split factor
// depends on T only through ceil(T / 256) and falls as T grows: within each
// run of 256 token counts the layout grows with T, so its largest value is
// at the run's last T. Once the split factor is 1 it stays 1 and the layout
// only grows.
template <typename F>
size_t max_total_upto(const lcmoe_shape& s, int tmax, F total) {
  size_t best = total(tmax);
  const int E = (int)n_experts(s);
  for (long long t = 256; t < tmax; t += 256) {
    best = std::max(best, total((int)t));
    int ks = 1, kchunk = 0;
    router_splits((int)t, E, s.d_model, ks, kchunk);
    if (ks == 1) break;
  }
  return best;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Carve the workspace: returns the aligned base or nullptr if too small.
char* ws_base(void* ws, size_t ws_bytes, size_t need) {
  if (ws == nullptr) return nullptr;
  const uintptr_t b = ((uintptr_t)ws + kAlign - 1) & ~(uintptr_t)(kAlign - 1);
  const size_t pad = b - (uintptr_t)ws;
  if (ws_bytes < pad || ws_bytes - pad < need) return nullptr;
  return reinterpret_cast<char*>(b);
}

// Status of the launches just enqueued (the sticky error is cleared before
// the first launch of every entry point, see clear_hip_error).
lcmoe_status hip_status() {
  return hipGetLastError() == hipSuccess ? LCMOE_OK : LCMOE_ERR_HIP;
}
void clear_hip_error() { (void)hipGetLastError(); }

// Record stage boundary `i` on the stream when the caller asked for it.
void mark(hipEvent_t* ev, int i, hipStream_t st) {
  if (ev != nullptr) (void)hipEventRecord(ev[i], st);
}

template <typename T>
T* at(char* base, size_t off) {
  return reinterpret_cast<T*>(base + off);
}

// Routing sequence shared by route and forward: router GEMM, top-K + gates,
// histogram / scan / schedule (+ optional scatter).
void enqueue_routing(const lcmoe_shape& s, int T, const Layout& L, char* base,
                     const void* x, const float* wr, const float* bias, int32_t* idx,
                     float* gate, int32_t* counts, float* logits_out, int32_t* offsets,
                     int32_t* perm, int32_t* row_of_slot, hipStream_t st) {
  const int E = (int)n_experts(s);
  float* zpart = at<float>(base, L.zpart);
  launch_router(static_cast<const uint16_t*>(x), wr, zpart, T, E, s.d_model, L.ks, L.kchunk, st);
  launch_topk(zpart, L.ks, bias, T, E, s.top_k, idx, gate, logits_out, st);
  launch_permute(idx, T, s.top_k, E, s.n_ffn, L.ntile, at<unsigned long long>(base, L.masks),
                 at<int>(base, L.tilecnt), at<int>(base, L.tileoff), counts, offsets,
                 at<int>(base, L.mt_prefix), at<int>(base, L.meta),
                 perm, row_of_slot, st);
}

}  // namespace

extern "C" {

size_t lcmoe_workspace_bytes(const lcmoe_shape* shape, int32_t max_tokens) {
  if (check_shape(shape) != LCMOE_OK || max_tokens < 0) return 0;
  if ((long long)max_tokens * shape->top_k >= (1ll << 31)) return 0;
  const lcmoe_shape s = *shape;
  return max_total_upto(s, max_tokens, [&](int t) { return make_layout(s, t).total; }) + kAlign;
}

lcmoe_status lcmoe_route(const lcmoe_shape* shape, int32_t T, const void* x_bf16,
                         const float* w_router, const float* bias, int32_t* topk_idx,
                         float* topk_gate, int32_t* counts, float* logits_out, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  lcmoe_status st = check_shape(shape);
  if (st != LCMOE_OK) return st;
  if (T < 0 || counts == nullptr) return LCMOE_ERR_INVALID_ARG;
  if (T > 0 && (x_bf16 == nullptr || w_router == nullptr || bias == nullptr ||
                topk_idx == nullptr || topk_gate == nullptr))
    return LCMOE_ERR_INVALID_ARG;
  if ((long long)T * shape->top_k >= (1ll << 31)) return LCMOE_ERR_UNSUPPORTED;
  const int E = (int)n_experts(*shape);
  if (T == 0) {
    clear_hip_error();
    launch_zero_fill(counts, (size_t)E * 4, stream);
    return hip_status();
  }
  if (!aligned16(x_bf16) || !aligned16(w_router)) return LCMOE_ERR_UNSUPPORTED;
  const Layout L = make_layout(*shape, T);
  char* base = ws_base(ws, ws_bytes, L.routing_end);
  if (base == nullptr) return LCMOE_ERR_WORKSPACE;
  clear_hip_error();
  enqueue_routing(*shape, T, L, base, x_bf16, w_router, bias, topk_idx, topk_gate, counts,
                  logits_out, at<int>(base, L.offsets), nullptr, nullptr, stream);
  return hip_status();
}

lcmoe_status lcmoe_permute(const lcmoe_shape* shape, int32_t T, const int32_t* topk_idx,
                           int32_t* counts, int32_t* offsets, int32_t* perm,
                           int32_t* row_of_slot, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  lcmoe_status st = check_shape(shape);
  if (st != LCMOE_OK) return st;
  if (T < 0 || counts == nullptr || offsets == nullptr) return LCMOE_ERR_INVALID_ARG;
  if (T > 0 && (topk_idx == nullptr || perm == nullptr || row_of_slot == nullptr))
    return LCMOE_ERR_INVALID_ARG;
  if ((long long)T * shape->top_k >= (1ll << 31)) return LCMOE_ERR_UNSUPPORTED;
  const int E = (int)n_experts(*shape);
  if (T == 0) {
    clear_hip_error();
    launch_zero_fill(counts, (size_t)E * 4, stream);
    launch_zero_fill(offsets, (size_t)(shape->n_ffn + 1) * 4, stream);
    return hip_status();
  }
  const Layout L = make_layout(*shape, T);
  char* base = ws_base(ws, ws_bytes, L.routing_end);
  if (base == nullptr) return LCMOE_ERR_WORKSPACE;
  clear_hip_error();
  launch_permute(topk_idx, T, shape->top_k, E, shape->n_ffn, L.ntile,
                 at<unsigned long long>(base, L.masks), at<int>(base, L.tilecnt),
                 at<int>(base, L.tileoff), counts, offsets,
                 at<int>(base, L.mt_prefix), at<int>(base, L.meta), perm, row_of_slot, stream);
  return hip_status();
}

namespace {

// Argument checks of the forward entry points (everything but the
// workspace), before any HIP call.
lcmoe_status check_forward_args(const lcmoe_shape* shape, int32_t T, const void* x_bf16,
                                const float* w_router, const float* bias, const void* w13,
                                const float* w13_scale, const void* w2, const float* w2_scale,
                                const void* y_bf16, const int32_t* topk_idx,
                                const float* topk_gate, const int32_t* counts) {
  lcmoe_status st = check_shape(shape);
  if (st != LCMOE_OK) return st;
  const bool fp8 = shape->w_dtype != LCMOE_W_BF16;  // fp8 weights
  if (T < 0 || counts == nullptr) return LCMOE_ERR_INVALID_ARG;
  if (T > 0 && (x_bf16 == nullptr || w_router == nullptr || bias == nullptr || w13 == nullptr ||
                w2 == nullptr || y_bf16 == nullptr || topk_idx == nullptr ||
                topk_gate == nullptr))
    return LCMOE_ERR_INVALID_ARG;
  if (T > 0 && fp8 && (w13_scale == nullptr || w2_scale == nullptr)) return LCMOE_ERR_INVALID_ARG;
  if ((long long)T * shape->top_k >= (1ll << 31)) return LCMOE_ERR_UNSUPPORTED;
  // x rows are gathered with 32-bit byte offsets.
  if ((long long)T * shape->d_model * 2 >= (1ll << 32)) return LCMOE_ERR_UNSUPPORTED;
  if (T > 0 && (!aligned16(x_bf16) || !aligned16(w_router) || !aligned16(w13) ||
                !aligned16(w2) || !aligned16(y_bf16)))
    return LCMOE_ERR_UNSUPPORTED;
  return LCMOE_OK;
}

// Caller buffers that receive the fp8 activation path's intermediates in
// place of the workspace regions (lcmoe_forward_inspect).
struct A8Out {
  uint8_t* xq = nullptr;
  float* xs = nullptr;
  uint16_t* h = nullptr;
  uint8_t* hq = nullptr;
  float* hs = nullptr;
};

// The forward; usave (bf16 weights only, may be null) receives the gate/up
// pre-activations of every FFN slot row; a8o (fp8 activations only, may be
// null) redirects the activation codes, scales and the pre-quantization H.
lcmoe_status forward_impl(const lcmoe_shape* shape, int32_t T, const void* x_bf16,
                          const float* w_router, const float* bias, const void* w13,
                          const float* w13_scale, const void* w2, const float* w2_scale,
                          void* y_bf16, int32_t* topk_idx, float* topk_gate, int32_t* counts,
                          void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t* stage_events,
                          float* usave, const A8Out* a8o = nullptr) {
  lcmoe_status st = check_forward_args(shape, T, x_bf16, w_router, bias, w13, w13_scale, w2,
                                       w2_scale, y_bf16, topk_idx, topk_gate, counts);
  if (st != LCMOE_OK) return st;
  const bool fp8 = shape->w_dtype != LCMOE_W_BF16;             // fp8 weights
  const bool a8 = shape->w_dtype == LCMOE_W_FP8_E4M3_B128_A8;  // and fp8 activations
  if (T == 0) {
    clear_hip_error();
    launch_zero_fill(counts, (size_t)n_experts(*shape) * 4, stream);
    return hip_status();
  }
  const Layout L = make_layout(*shape, T);
  char* base = ws_base(ws, ws_bytes, L.total);
  if (base == nullptr) return LCMOE_ERR_WORKSPACE;
  clear_hip_error();

  int* offsets = at<int>(base, L.offsets);
  int* perm = at<int>(base, L.perm);
  int* row_of_slot = at<int>(base, L.row_of_slot);
  const int E = (int)n_experts(*shape);
  hipEvent_t* ev = stage_events;
  // fp8 activations: codes and scales of x and of H, and H before its
  // quantization (the workspace, or the caller's buffers when inspected)
  uint8_t* xq = a8 ? at<uint8_t>(base, L.xq) : nullptr;
  float* xs = a8 ? at<float>(base, L.xs) : nullptr;
  uint8_t* hq = a8 ? at<uint8_t>(base, L.hq) : nullptr;
  float* hs = a8 ? at<float>(base, L.hs) : nullptr;
  uint16_t* H = at<uint16_t>(base, L.H);
  uint16_t* Hpre = H;  // quantized in place unless inspected
  if (a8o != nullptr) {
    xq = a8o->xq;
    xs = a8o->xs;
    hq = a8o->hq;
    hs = a8o->hs;
    Hpre = a8o->h;
  }
  mark(ev, 0, stream);
  {
    float* zpart = at<float>(base, L.zpart);
    launch_router(static_cast<const uint16_t*>(x_bf16), w_router, zpart, T, E, shape->d_model,
                  L.ks, L.kchunk, stream);
    mark(ev, 1, stream);
    launch_topk(zpart, L.ks, bias, T, E, shape->top_k, topk_idx, topk_gate, nullptr, stream);
    mark(ev, 2, stream);
    launch_permute(topk_idx, T, shape->top_k, E, shape->n_ffn, L.ntile,
                   at<unsigned long long>(base, L.masks), at<int>(base, L.tilecnt),
                   at<int>(base, L.tileoff), counts, offsets, at<int>(base, L.mt_prefix),
                   at<int>(base, L.meta), perm, row_of_slot, stream);
    if (a8)  // fp8 activations: quantize x per row (timed with the permutation stage)
      launch_quant_rows(static_cast<const uint16_t*>(x_bf16), T, nullptr, shape->d_model, xq, xs,
                        std::min(2048, (T + 3) / 4), stream);
    mark(ev, 3, stream);
  }

  const int N = shape->n_ffn, d = shape->d_model, I = shape->d_expert;
  uint16_t* Y = at<uint16_t>(base, L.Y);

  // Grid bound from what the host knows (no device->host sync): at most
  // S/320 + min(N, S) M-tiles (each touched expert adds at most one partial
  // tile to its share of S/320).
  const long long smax = L.smax;
  const long long n_tiles_ub =
      (smax + kBigTileRows - 1) / kBigTileRows + std::min<long long>(N, smax);
  auto grid_of = [&](int nsl) {
    const long long g = std::max<long long>(8, (n_tiles_ub * nsl + 7) / 8 * 8);
    return (int)std::min<long long>(g, (1ll << 30));
  };

  GemmArgs a{};
  a.offsets = offsets;
  a.counts = counts;
  a.mt_prefix = at<int>(base, L.mt_prefix);
  a.meta = at<int>(base, L.meta);
  a.perm = perm;
  a.topk = shape->top_k;
  a.n_ffn = N;

  // gate/up: H = silu(X W1^T) * (X W3^T)
  a.w = w13;
  a.wscale = w13_scale;
  a.src = static_cast<const uint16_t*>(x_bf16);
  a.src8 = xq;
  a.ascale = xs;
  a.out = Hpre;
  a.usave = usave;
  a.kdim = d;
  a.n_out = I;
  a.rows_total = 2 * I;
  a.nslices = (I + kBigColsGateUp - 1) / kBigColsGateUp;
  if (a8) launch_gemm_big_a8(a, true, grid_of(a.nslices), stream);
  else launch_gemm_big(a, true, fp8, grid_of(a.nslices), stream);
  mark(ev, 4, stream);
  if (a8)  // quantize the S rows of H (S read on the device; timed with the down stage)
    launch_quant_rows(Hpre, 0, at<int>(base, L.meta) + 2, I, hq, hs,
                      (int)std::min<long long>(2048, (smax + 3) / 4), stream);

  // down: Y = H W2^T
  a.usave = nullptr;
  a.w = w2;
  a.wscale = w2_scale;
  a.src = H;
  a.src8 = hq;
  a.ascale = hs;
  a.out = Y;
  a.kdim = I;
  a.n_out = d;
  a.rows_total = d;
  a.nslices = (d + kBigColsDown - 1) / kBigColsDown;
  if (a8) launch_gemm_big_a8(a, false, grid_of(a.nslices), stream);
  else launch_gemm_big(a, false, fp8, grid_of(a.nslices), stream);
  mark(ev, 5, stream);

  launch_combine(static_cast<const uint16_t*>(x_bf16), Y, topk_idx, topk_gate, row_of_slot, T,
                 d, shape->top_k, static_cast<uint16_t*>(y_bf16), stream);
  mark(ev, 6, stream);
  return hip_status();
}

}  // namespace

lcmoe_status lcmoe_forward_staged(const lcmoe_shape* shape, int32_t T, const void* x_bf16,
                                  const float* w_router, const float* bias, const void* w13,
                                  const float* w13_scale, const void* w2, const float* w2_scale,
                                  void* y_bf16, int32_t* topk_idx, float* topk_gate,
                                  int32_t* counts, void* ws, size_t ws_bytes,
                                  hipStream_t stream, hipEvent_t* stage_events) {
  return forward_impl(shape, T, x_bf16, w_router, bias, w13, w13_scale, w2, w2_scale, y_bf16,
                      topk_idx, topk_gate, counts, ws, ws_bytes, stream, stage_events, nullptr);
}

lcmoe_status lcmoe_forward_train(const lcmoe_shape* shape, int32_t T, const void* x_bf16,
                                 const float* w_router, const float* bias, const void* w13,
                                 const void* w2, void* y_bf16, int32_t* topk_idx,
                                 float* topk_gate, int32_t* counts, void* u_save, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  lcmoe_status st = check_shape(shape);
  if (st != LCMOE_OK) return st;
  if (shape->w_dtype != LCMOE_W_BF16) return LCMOE_ERR_UNSUPPORTED;
  if (T > 0 && u_save == nullptr) return LCMOE_ERR_INVALID_ARG;
  if (T > 0 && !aligned16(u_save)) return LCMOE_ERR_UNSUPPORTED;
  return forward_impl(shape, T, x_bf16, w_router, bias, w13, nullptr, w2, nullptr, y_bf16,
                      topk_idx, topk_gate, counts, ws, ws_bytes, stream, nullptr,
                      static_cast<float*>(u_save));
}

lcmoe_status lcmoe_forward(const lcmoe_shape* shape, int32_t T, const void* x_bf16,
                           const float* w_router, const float* bias, const void* w13,
                           const float* w13_scale, const void* w2, const float* w2_scale,
                           void* y_bf16, int32_t* topk_idx, float* topk_gate, int32_t* counts,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  return lcmoe_forward_staged(shape, T, x_bf16, w_router, bias, w13, w13_scale, w2, w2_scale,
                              y_bf16, topk_idx, topk_gate, counts, ws, ws_bytes, stream, nullptr);
}

lcmoe_status lcmoe_forward_inspect(const lcmoe_shape* shape, int32_t T, const void* x_bf16,
                                   const float* w_router, const float* bias, const void* w13,
                                   const float* w13_scale, const void* w2, const float* w2_scale,
                                   void* y_bf16, int32_t* topk_idx, float* topk_gate,
                                   int32_t* counts, void* xq, float* xs, void* h, void* hq,
                                   float* hs, void* ws, size_t ws_bytes, hipStream_t stream) {
  lcmoe_status st = check_shape(shape);
  if (st != LCMOE_OK) return st;
  if (shape->w_dtype != LCMOE_W_FP8_E4M3_B128_A8) return LCMOE_ERR_UNSUPPORTED;
  if (T > 0 && (xq == nullptr || xs == nullptr || h == nullptr || hq == nullptr || hs == nullptr))
    return LCMOE_ERR_INVALID_ARG;
  if (T > 0 && (!aligned16(xq) || !aligned16(xs) || !aligned16(h) || !aligned16(hq) ||
                !aligned16(hs)))
    return LCMOE_ERR_UNSUPPORTED;
  A8Out o;
  o.xq = static_cast<uint8_t*>(xq);
  o.xs = xs;
  o.h = static_cast<uint16_t*>(h);
  o.hq = static_cast<uint8_t*>(hq);
  o.hs = hs;
  return forward_impl(shape, T, x_bf16, w_router, bias, w13, w13_scale, w2, w2_scale, y_bf16,
                      topk_idx, topk_gate, counts, ws, ws_bytes, stream, nullptr, nullptr, &o);
}

lcmoe_status lcmoe_forward_noalloc(const lcmoe_shape* shape, int32_t T, const void* x_bf16,
                                   const float* w_router, const float* bias, const void* w13,
                                   const float* w13_scale, const void* w2, const float* w2_scale,
                                   void* y_bf16, int32_t* topk_idx, float* topk_gate,
                                   int32_t* counts, hipStream_t stream) {
  lcmoe_status st = check_forward_args(shape, T, x_bf16, w_router, bias, w13, w13_scale, w2,
                                       w2_scale, y_bf16, topk_idx, topk_gate, counts);
  if (st != LCMOE_OK) return st;
  if (T > 0 && make_layout(*shape, T).total > kNoallocScratchBytes) return LCMOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (T > 0) {
    st = noalloc_scratch(&ws);
    if (st != LCMOE_OK) return st;
  }
  return forward_impl(shape, T, x_bf16, w_router, bias, w13, w13_scale, w2, w2_scale, y_bf16,
                      topk_idx, topk_gate, counts, ws, ws != nullptr ? kNoallocScratchBytes : 0,
                      stream, nullptr, nullptr);
}

size_t lcmoe_backward_workspace_bytes(const lcmoe_shape* shape, int32_t max_tokens) {
  if (check_shape(shape) != LCMOE_OK || max_tokens < 0 || shape->w_dtype != LCMOE_W_BF16) return 0;
  if ((long long)max_tokens * shape->top_k >= (1ll << 31)) return 0;
  const lcmoe_shape s = *shape;
  return max_total_upto(s, max_tokens, [&](int t) { return make_bwd_layout(s, t).total; }) +
         kAlign;
}

namespace {

// The backward; usaved (may be null) holds the forward's gate/up
// pre-activations, which then replace the recomputation of u.
lcmoe_status backward_impl(const lcmoe_shape* shape, int32_t T, const void* x_bf16,
                           const float* w_router, const float* bias, const void* w13,
                           const void* w2, const void* dy_bf16, float* dx, float* dw_router,
                           void* dw13, void* dw2, void* ws, size_t ws_bytes, hipStream_t stream,
                           hipEvent_t* ev, const float* usaved) {
  lcmoe_status st = check_shape(shape);
  if (st != LCMOE_OK) return st;
  if (shape->w_dtype != LCMOE_W_BF16) return LCMOE_ERR_UNSUPPORTED;
  if (T < 0 || dw_router == nullptr || dw13 == nullptr || dw2 == nullptr)
    return LCMOE_ERR_INVALID_ARG;
  if (T > 0 && (x_bf16 == nullptr || w_router == nullptr || bias == nullptr || w13 == nullptr ||
                w2 == nullptr || dy_bf16 == nullptr || dx == nullptr))
    return LCMOE_ERR_INVALID_ARG;
  if ((long long)T * shape->top_k >= (1ll << 31)) return LCMOE_ERR_UNSUPPORTED;
  const int N = shape->n_ffn, d = shape->d_model, I = shape->d_expert, K = shape->top_k;
  const int E = (int)n_experts(*shape);
  // the grouped GEMMs address one expert's slot rows (up to T of them), and
  // the router-gradient planes of T tokens, with 32-bit byte offsets
  const long long Ep = (E + 63) / 64 * 64;
  if ((long long)T * std::max<long long>(std::max(d, 2 * I), 6 * Ep) * 2 >= (1ll << 32))
    return LCMOE_ERR_UNSUPPORTED;
  if (T == 0) {  // no tokens: every gradient is zero
    clear_hip_error();
    launch_zero_fill(dw_router, (size_t)E * d * 4, stream);
    launch_zero_fill(dw13, (size_t)N * 2 * I * d * 2, stream);
    launch_zero_fill(dw2, (size_t)N * d * I * 2, stream);
    return hip_status();
  }
  if (!aligned16(x_bf16) || !aligned16(w_router) || !aligned16(w13) || !aligned16(w2) ||
      !aligned16(dy_bf16) || !aligned16(dx) || !aligned16(dw_router) || !aligned16(dw13) ||
      !aligned16(dw2))
    return LCMOE_ERR_UNSUPPORTED;
  const BwdLayout B = make_bwd_layout(*shape, T);
  const Layout& L = B.f;
  char* base = ws_base(ws, ws_bytes, B.total);
  if (base == nullptr) return LCMOE_ERR_WORKSPACE;
  AuxStream* aux = nullptr;  // stage events time the stages in order, on one stream
  if (ev == nullptr) {
    lcmoe_status sa = aux_stream(&aux);
    if (sa != LCMOE_OK) return sa;
  }
  clear_hip_error();

  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  const uint16_t* dy = static_cast<const uint16_t*>(dy_bf16);
  int* idx = at<int>(base, B.idx);
  float* gate = at<float>(base, B.gate);
  int* counts = at<int>(base, B.counts);
  float* logits = at<float>(base, B.logits);
  int* offsets = at<int>(base, L.offsets);
  int* perm = at<int>(base, L.perm);
  int* row_of_slot = at<int>(base, L.row_of_slot);
  int* tprefix = at<int>(base, B.tprefix);
  uint16_t* Xs = at<uint16_t>(base, B.Xs);
  uint16_t* dYs = at<uint16_t>(base, B.dYs);
  float* Q = at<float>(base, B.Q);
  uint16_t* dU = at<uint16_t>(base, B.dU);
  uint16_t* Hg = at<uint16_t>(base, B.Hg);
  float* dXs = at<float>(base, B.dXs);
  float* dg = at<float>(base, B.dg);
  uint16_t* dzp = at<uint16_t>(base, B.dzp);
  uint16_t* dzt = at<uint16_t>(base, B.dzt);
  float* dxr = at<float>(base, B.dxr);
  const int* s_dev = at<int>(base, L.meta) + 2;  // FFN slot count

  // 1. routing as in the forward (same kernels, so the same selection), with
  //    the fp32 logits kept for the softmax backward; the permutation; the
  //    x and dy rows of every FFN slot gathered into slot order
  mark(ev, 0, stream);
  launch_router(x, w_router, at<float>(base, L.zpart), T, E, d, L.ks, L.kchunk, stream);
  launch_topk(at<float>(base, L.zpart), L.ks, bias, T, E, K, idx, gate, logits, stream);
  launch_permute(idx, T, K, E, N, L.ntile, at<unsigned long long>(base, L.masks),
                 at<int>(base, L.tilecnt), at<int>(base, L.tileoff), counts, offsets,
                 at<int>(base, L.mt_prefix), at<int>(base, L.meta),
                 perm, row_of_slot, stream);
  launch_tile_prefix(counts, N, kBwdTileM, tprefix, nullptr, stream);
  int* bmeta = at<int>(base, B.bmeta);
  launch_tile_prefix(counts, N, kBigTileRows, at<int>(base, B.bprefix), bmeta + 1, stream);
  const long long smax = L.smax;
  const int row_grid = (int)std::min<long long>(4096, (smax + 3) / 4);
  launch_gather_rows(x, dy, perm, s_dev, K, d, Xs, dYs, row_grid, stream);
  mark(ev, 1, stream);

  BwdGemmArgs g{};
  g.counts = counts;
  g.offsets = offsets;
  g.tile_prefix = tprefix;
  g.n_ffn = N;

  // 2. Q = dY_e W2_e (W2 read k-major), per FFN slot row
  g.a = dYs; g.a_ld = d;
  g.b = static_cast<const uint16_t*>(w2); g.b_ld = I; g.b_estride = (long long)d * I;
  g.c = Q; g.c_ld = I; g.N = I; g.K = d;
  launch_bwd_dgrad(g, kBwdQ, bwd_dgrad_grid(smax, N, I), stream);
  mark(ev, 2, stream);

  // 3. u = W13_e x per FFN slot row on the forward's large-M gate/up GEMM
  //    (every expert with slots, M-tiles of up to kBigTileRows rows), with the
  //    SiLU backward in its epilogue: g h, dU and the partials of dg = <Q, h>;
  //    or, with the forward's saved u, the SiLU backward alone
  if (usaved != nullptr) {
    launch_bwd_silu_saved(usaved, Q, perm, gate, s_dev, I, dU, Hg, dg, row_grid, stream);
  } else {
    GemmArgs ga{};
    ga.w = w13;
    ga.src = x;
    ga.perm = perm;
    ga.offsets = offsets;
    ga.counts = counts;
    ga.mt_prefix = at<int>(base, B.bprefix);
    ga.meta = bmeta;
    ga.out = Hg;
    ga.kdim = d;
    ga.n_out = I;
    ga.rows_total = 2 * I;
    ga.topk = K;
    ga.n_ffn = N;
    ga.nslices = B.nslices;
    ga.bq = Q;
    ga.bgate = gate;
    ga.bdu = dU;
    ga.bdgp = at<float>(base, B.dgp);
    const long long tiles_ub = smax / kBigTileRows + std::min<long long>(N, smax);
    const long long grid = std::max<long long>(8, (tiles_ub * B.nslices + 7) / 8 * 8);
    launch_gemm_big_bwd_u(ga, (int)std::min<long long>(grid, 1ll << 30), stream);
  }
  mark(ev, 3, stream);

  // 4. dg of the FFN slots (sum of the partials) and of the zero slots;
  //    router dz
  if (usaved == nullptr)
    launch_bwd_dg_reduce(at<float>(base, B.dgp), 4 * B.nslices, perm, s_dev, dg,
                         (int)std::min<long long>(4096, (smax + 255) / 256), stream);
  launch_bwd_zero_dg(x, dy, idx, T, d, K, N, dg, stream);
  launch_bwd_router_dz(logits, idx, gate, dg, T, E, B.Ep, K, dzp, dzt, stream);
  mark(ev, 4, stream);

  // 5.-9. dX per slot row = dU_e W13_e (W13 read k-major); dW2_e[c][j] = sum
  // over the expert's slots of dy[t][c] (g h)[s][j]; dW13_e[r][c] = sum over
  // the expert's slots of dU[s][r] x[t][c]; the router gradients dW_r = dz^T x
  // and dx_r = dz W_r (bf16 MFMA on exact planes of dz and W_r, fp32
  // accumulation); dx. The weight gradients depend on nothing after step 4
  // and nothing after them depends on them, so without stage events they go
  // to the second stream on part of the CUs (HBM writes) while dX and the
  // router gradients run on the caller's stream (HBM reads).
  auto dx_rows = [&](hipStream_t s) {
    BwdGemmArgs h = g;
    h.a = dU; h.a_ld = 2 * I;
    h.b = static_cast<const uint16_t*>(w13); h.b_ld = d; h.b_estride = (long long)2 * I * d;
    h.c = dXs; h.c_ld = d; h.N = d; h.K = 2 * I;
    launch_bwd_dgrad(h, kBwdDx, bwd_dgrad_grid(smax, N, d), s);
  };
  auto wgrad = [&](BwdOp op, hipStream_t s, int max_blocks) {
    BwdGemmArgs h = g;
    if (op == kBwdDw2) {
      h.a = dYs; h.a_ld = d;
      h.b = Hg; h.b_ld = I; h.b_estride = 0;
      h.c = dw2; h.c_ld = I; h.M = d; h.m_store = d; h.N = I;
    } else {
      h.a = dU; h.a_ld = 2 * I;
      h.b = Xs; h.b_ld = d; h.b_estride = 0;
      h.c = dw13; h.c_ld = d; h.M = 2 * I; h.m_store = 2 * I; h.N = d;
    }
    launch_bwd_wgrad(h, op, bwd_wgrad_grid(N, h.M, h.N, max_blocks), s);
  };
  auto router = [&](hipStream_t s) {
    launch_router_grads(dzp, dzt, x, w_router, T, E, B.Ep, d, at<uint16_t>(base, B.wsp),
                        at<int>(base, B.rg), dw_router, dxr, s);
  };
  auto dx_final = [&](hipStream_t s) {
    launch_bwd_dx(dXs, dy, dxr, row_of_slot, gate, T, d, K, dx, s);
  };
  if (aux == nullptr) {
    dx_rows(stream);
    mark(ev, 5, stream);
    wgrad(kBwdDw2, stream, 0);
    mark(ev, 6, stream);
    wgrad(kBwdDw13, stream, 0);
    mark(ev, 7, stream);
    router(stream);
    mark(ev, 8, stream);
    dx_final(stream);
    mark(ev, 9, stream);
    return hip_status();
  }
  std::lock_guard<std::mutex> lock(g_aux_mu);
  if (hipEventRecord(aux->fork, stream) != hipSuccess ||
      hipStreamWaitEvent(aux->s, aux->fork, 0) != hipSuccess)
    return LCMOE_ERR_HIP;
  const int share = std::max(8, bwd_device_cus() * kBwdWgradEighths / 8 / 8 * 8);
  wgrad(kBwdDw2, aux->s, share);
  wgrad(kBwdDw13, aux->s, share);
  if (hipEventRecord(aux->join, aux->s) != hipSuccess) return LCMOE_ERR_HIP;
  dx_rows(stream);
  router(stream);
  dx_final(stream);
  if (hipStreamWaitEvent(stream, aux->join, 0) != hipSuccess) return LCMOE_ERR_HIP;
  return hip_status();
}

}  // namespace

lcmoe_status lcmoe_backward_staged(const lcmoe_shape* shape, int32_t T, const void* x_bf16,
                                   const float* w_router, const float* bias, const void* w13,
                                   const void* w2, const void* dy_bf16, float* dx,
                                   float* dw_router, void* dw13, void* dw2, void* ws,
                                   size_t ws_bytes, hipStream_t stream, hipEvent_t* ev) {
  return backward_impl(shape, T, x_bf16, w_router, bias, w13, w2, dy_bf16, dx, dw_router, dw13,
                       dw2, ws, ws_bytes, stream, ev, nullptr);
}

lcmoe_status lcmoe_backward(const lcmoe_shape* shape, int32_t T, const void* x_bf16,
                            const float* w_router, const float* bias, const void* w13,
                            const void* w2, const void* dy_bf16, float* dx, float* dw_router,
                            void* dw13, void* dw2, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  return backward_impl(shape, T, x_bf16, w_router, bias, w13, w2, dy_bf16, dx, dw_router, dw13,
                       dw2, ws, ws_bytes, stream, nullptr, nullptr);
}

lcmoe_status lcmoe_backward_saved(const lcmoe_shape* shape, int32_t T, const void* x_bf16,
                                  const float* w_router, const float* bias, const void* w13,
                                  const void* w2, const void* dy_bf16, const void* u_saved,
                                  float* dx, float* dw_router, void* dw13, void* dw2, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  if (T > 0 && u_saved == nullptr) return LCMOE_ERR_INVALID_ARG;
  if (T > 0 && !aligned16(u_saved)) return LCMOE_ERR_UNSUPPORTED;
  return backward_impl(shape, T, x_bf16, w_router, bias, w13, w2, dy_bf16, dx, dw_router, dw13,
                       dw2, ws, ws_bytes, stream, nullptr,
                       static_cast<const float*>(u_saved));
}

lcmoe_status lcmoe_bias_update(const lcmoe_shape* shape, int32_t t_all, const int32_t* counts,
                               double mu, double k_e, float* bias, hipStream_t stream) {
  lcmoe_status st = check_shape(shape);
  if (st != LCMOE_OK) return st;
  if (t_all <= 0 || counts == nullptr || bias == nullptr || !std::isfinite(mu) ||
      !std::isfinite(k_e))
    return LCMOE_ERR_INVALID_ARG;
  clear_hip_error();
  launch_bias_update(counts, shape->n_ffn, shape->top_k, t_all, mu, k_e, bias, stream);
  return hip_status();
}

size_t lcmoe_router_stats_workspace_bytes(const lcmoe_shape* shape, int32_t n_groups) {
  if (check_shape(shape) != LCMOE_OK || n_groups < 1 || shape->n_ffn % n_groups != 0) return 0;
  return (size_t)kStatsBlocks * (size_t)(n_groups + 2) * sizeof(double) + kAlign;
}

lcmoe_status lcmoe_router_stats(const lcmoe_shape* shape, int32_t T, const void* x_bf16,
                                const float* logits, const int32_t* counts, int32_t n_groups,
                                double k_e, double alpha, double lambda, double* stats,
                                void* ws, size_t ws_bytes, hipStream_t stream) {
  lcmoe_status st = check_shape(shape);
  if (st != LCMOE_OK) return st;
  if (T < 0 || stats == nullptr || counts == nullptr || n_groups < 1 ||
      shape->n_ffn % n_groups != 0 || !std::isfinite(k_e) || !(k_e > 0.0) ||
      k_e > (double)shape->top_k || !std::isfinite(alpha) || !std::isfinite(lambda))
    return LCMOE_ERR_INVALID_ARG;
  if (T > 0 && (x_bf16 == nullptr || logits == nullptr)) return LCMOE_ERR_INVALID_ARG;
  if (T > 0 && (!aligned16(x_bf16) || !aligned16(logits))) return LCMOE_ERR_UNSUPPORTED;
  const size_t need = (size_t)kStatsBlocks * (size_t)(n_groups + 2) * sizeof(double);
  char* base = ws_base(ws, ws_bytes, need);
  if (base == nullptr) return LCMOE_ERR_WORKSPACE;
  clear_hip_error();
  launch_router_stats(logits, static_cast<const uint16_t*>(x_bf16), T, (int)n_experts(*shape),
                      shape->d_model, shape->n_ffn, n_groups, shape->top_k, counts, k_e, alpha,
                      lambda, reinterpret_cast<double*>(base), stats, stream);
  return hip_status();
}

const char* lcmoe_status_str(lcmoe_status status) {
  switch (status) {
    case LCMOE_OK: return "LCMOE_OK";
    case LCMOE_ERR_INVALID_ARG: return "LCMOE_ERR_INVALID_ARG";
    case LCMOE_ERR_UNSUPPORTED: return "LCMOE_ERR_UNSUPPORTED";
    case LCMOE_ERR_WORKSPACE: return "LCMOE_ERR_WORKSPACE";
    case LCMOE_ERR_HIP: return "LCMOE_ERR_HIP";
  }
  return "LCMOE_ERR_UNKNOWN";
}

}  // extern "C"
