// qmoe_api.hip -- the extern "C" entry points declared in include/qmoe.h:
// argument validation, workspace sizing, and dispatch to the launchers.
// Nothing here allocates, frees or synchronises (qmoe_workspace_status
// excepted, which reads one word back).
#include <cmath>
#include <cstring>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "qmoe.h"
#include "qmoe_common.h"

// Workspace of qmoe_moe_decode_noalloc: a fixed device array, one copy per
// GPU (each device holds it until the process ends).  Host code never uses
// this name as an address: the device address comes from
// hipGetSymbolAddress, per device (see scratch_for_device).
constexpr size_t kScratchBytes = (size_t)512 << 10;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace qmoe {
qmoe_status launch_gemv4(const qmoe_qtensor& W, const uint16_t* x, float* y, void* stream);
size_t tiled4_size(int rows, int cols);
size_t sample_ws_bytes(int V, int K);
bool sample_supported(int V, int K);
qmoe_status launch_sample(const float* logits, int V, float temperature, int K, float top_p,
                          float u, int32_t* token, int32_t* ranked, uint8_t* ws, void* stream);
bool attn_supported(int D, int G);
size_t attn_ws_bytes(int Hq, int Hkv, int D, int S);
size_t attn_ctl_bytes(int Hkv);
qmoe_status launch_attn(const float* q, const float* k, const float* v, int Hq, int Hkv, int D,
                        int S, bool circular, int pos, float rope_base, float scale, uint16_t* kc,
                        uint16_t* vc, uint16_t* out, void* ws, void* stream);
bool gemv_tiled4_supported(int cols);
qmoe_status launch_gemv_tiled4(const uint8_t* T, int rows, int cols, const uint16_t* x, float* y,
                               int rbw, void* stream);
qmoe_status launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int T, int H,
                           uint16_t* out, void* stream);
qmoe_status launch_router(const qmoe_qtensor& Wr, const float* lbias, const uint16_t* x, int T,
                          int K, int32_t* idx, float* w, float* logits, uint8_t* ws, void* stream);
qmoe_status launch_moe_step(const qmoe_moe_layer& L, const uint16_t* x, const int32_t* idx_in,
                            const float* w_in, const int32_t* slot, const uint16_t* residual,
                            uint16_t* out, int32_t* idx_out, float* w_out, uint8_t* ws, int mode,
                            void* stream, void* ev_start = nullptr, void* ev_stop = nullptr,
                            int heal = 0);
qmoe_status launch_prefill(const qmoe_moe_layer& L, const uint16_t* X, int T, const int32_t* idx,
                           const float* w, const uint16_t* residual, uint16_t* out, uint8_t* ws,
                           void* stream);
size_t prefill_ws_bytes(const qmoe_moe_layer& L, int T);
void prefill_dispatch_offsets(const qmoe_moe_layer& L, int T, size_t* counts, size_t* offsets,
                              size_t* perm);
bool moe_step_supported(const qmoe_moe_layer& L);
qmoe_status launch_moe_stack(const qmoe_moe_layer& L, const void* table, int n_layers,
                             const uint16_t* x, uint16_t* out, uint16_t* lout, int32_t* idx_out,
                             float* w_out, uint8_t* ws, uint16_t* xb, void* stream);

static bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static qmoe_status check_q(const qmoe_qtensor* t, int bits) {
  if (!t || !t->q || !t->scales || !t->biases) return QMOE_ERR_NULL_ARG;
  if (t->bits != bits || t->group != 64) return QMOE_ERR_UNSUPPORTED;
  if (t->rows <= 0 || t->cols <= 0 || t->cols % 64) return QMOE_ERR_BAD_SHAPE;
  if (!al16(t->q) || (t->expert_stride_bytes & 15) || t->expert_stride_bytes < 0)
    return QMOE_ERR_ALIGN;
  if (!al16(t->scales) || !al16(t->biases)) return QMOE_ERR_ALIGN;
  return QMOE_OK;
}

static qmoe_status check_layer(const qmoe_moe_layer* L) {
  if (!L) return QMOE_ERR_NULL_ARG;
  const int H = L->hidden, E = L->n_experts, K = L->top_k, I = L->inter, Is = L->shared_inter;
  if (H <= 0 || E <= 0 || K <= 0 || I <= 0 || Is <= 0) return QMOE_ERR_BAD_SHAPE;
  if (H % 64 || I % 64 || Is % 64) return QMOE_ERR_BAD_SHAPE;
  if (K > E) return QMOE_ERR_BAD_SHAPE;
  if (K > QMOE_MAX_TOP_K || E > QMOE_MAX_EXPERTS || H > QMOE_MAX_HIDDEN) return QMOE_ERR_UNSUPPORTED;
  // staged fp32 activations of the down projections must fit one block's LDS
  if ((size_t)(K * I + Is) * 4 > 96 * 1024) return QMOE_ERR_UNSUPPORTED;
  qmoe_status s;
  if ((s = check_q(&L->router, 8)) != QMOE_OK) return s;
  const qmoe_qtensor* m4[6] = {&L->gate, &L->up, &L->down, &L->sh_gate, &L->sh_up, &L->sh_down};
  for (int i = 0; i < 6; ++i)
    if ((s = check_q(m4[i], 4)) != QMOE_OK) return s;
  if (L->router.rows != E || L->router.cols != H) return QMOE_ERR_BAD_SHAPE;
  if (L->gate.rows != I || L->gate.cols != H || L->up.rows != I || L->up.cols != H)
    return QMOE_ERR_BAD_SHAPE;
  if (L->down.rows != H || L->down.cols != I) return QMOE_ERR_BAD_SHAPE;
  if (L->sh_gate.rows != Is || L->sh_gate.cols != H || L->sh_up.rows != Is || L->sh_up.cols != H)
    return QMOE_ERR_BAD_SHAPE;
  if (L->sh_down.rows != H || L->sh_down.cols != Is) return QMOE_ERR_BAD_SHAPE;
  if (L->rms_gamma && !al16(L->rms_gamma)) return QMOE_ERR_ALIGN;
  return QMOE_OK;
}

static size_t ws_bytes_layer(const qmoe_moe_layer* L, int T) {
  WsLayout wl = ws_layout(L->n_experts, L->top_k, L->inter, L->shared_inter, T);
  size_t d = wl.total;
  size_t p = wl.pf + prefill_ws_bytes(*L, T);
  return p > d ? p : d;
}

// Stack workspace: the one-token layer workspace, then the two layer-input
// buffers.
static size_t stack_xb_offset(const qmoe_moe_layer* L) { return align256(ws_bytes_layer(L, 1)); }
static size_t stack_ws_bytes(const qmoe_moe_layer* L) {
  return stack_xb_offset(L) + align256((size_t)2 * L->hidden * 2);
}

static bool same_shape(const qmoe_moe_layer& a, const qmoe_moe_layer& b) {
  return a.hidden == b.hidden && a.n_experts == b.n_experts && a.top_k == b.top_k &&
         a.inter == b.inter && a.shared_inter == b.shared_inter && a.rms_eps == b.rms_eps;
}

// Zero n16 16-byte words (a kernel, not hipMemsetAsync, so that the fill
// can sit in a captured graph).
__global__ void k_zero16(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

// The current device's address of `scratch`, looked up once per device
// (with that device current) and kept; the first call on a device also
// enqueues the zero fill a workspace needs before its first use, on the
// caller's stream, ahead of that call's kernels.
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static uint8_t* g_scratch[kMaxDevices];

static qmoe_status scratch_for_device(hipStream_t st, uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return QMOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return QMOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QMOE_ERR_HIP;
    hipLaunchKernelGGL(k_zero16, dim3(256), dim3(256), 0, st, static_cast<uint4*>(p),
                       kScratchBytes / 16);
    if (hipGetLastError() != hipSuccess) return QMOE_ERR_HIP;
    g_scratch[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch[dev];
  return QMOE_OK;
}
}  // namespace qmoe

using namespace qmoe;

extern "C" {

const char* qmoe_status_string(qmoe_status s) {
  switch (s) {
    case QMOE_OK: return "ok";
    case QMOE_ERR_NULL_ARG: return "a required pointer is NULL";
    case QMOE_ERR_BAD_SHAPE: return "inconsistent or out-of-range sizes";
    case QMOE_ERR_UNSUPPORTED: return "bits, group or size not supported by these kernels";
    case QMOE_ERR_WORKSPACE: return "workspace missing or too small";
    case QMOE_ERR_ALIGN: return "pointer or stride not aligned (16 bytes for codes and activations)";
    case QMOE_ERR_HIP: return "HIP runtime call failed";
    case QMOE_ERR_DEVICE: return "a device-side wait gave up; outputs of that call are undefined";
  }
  return "unknown status";
}

size_t qmoe_workspace_bytes(const qmoe_moe_layer* L, int32_t T) {
  if (check_layer(L) != QMOE_OK || T < 1 || T > QMOE_MAX_TOKENS) return 0;
  return ws_bytes_layer(L, T);
}

size_t qmoe_router_workspace_bytes(int32_t n_experts, int32_t T) {
  if (n_experts < 1 || n_experts > QMOE_MAX_EXPERTS || T < 1 || T > QMOE_MAX_TOKENS) return 0;
  return ws_layout(n_experts, QMOE_MAX_TOP_K, 0, 0, T).total;
}

qmoe_status qmoe_gemv_affine4(const qmoe_qtensor* W, const uint16_t* x, float* y, void* stream) {
  if (!W || !x || !y) return QMOE_ERR_NULL_ARG;
  qmoe_status s = check_q(W, 4);
  if (s != QMOE_OK) return s;
  if (W->cols > QMOE_MAX_HIDDEN) return QMOE_ERR_UNSUPPORTED;
  if (!al16(x)) return QMOE_ERR_ALIGN;
  return launch_gemv4(*W, x, y, stream);
}

size_t qmoe_sample_workspace_bytes(int32_t V, int32_t top_k) {
  if (V < 1 || top_k < 1) return 0;
  return sample_ws_bytes(V, top_k);
}

qmoe_status qmoe_sample(const float* logits, int32_t V, float temperature, int32_t top_k,
                        float top_p, float u, int32_t* token, int32_t* ranked, void* ws,
                        size_t ws_bytes, void* stream) {
  if (!logits || !token || !ws) return QMOE_ERR_NULL_ARG;
  if (V < 1 || top_k < 1 || top_k > V) return QMOE_ERR_BAD_SHAPE;
  if (!(temperature >= 0.f) || !(top_p > 0.f && top_p <= 1.f) || !(u >= 0.f && u < 1.f))
    return QMOE_ERR_BAD_SHAPE;
  if (!sample_supported(V, top_k)) return QMOE_ERR_UNSUPPORTED;
  if (ws_bytes < sample_ws_bytes(V, top_k)) return QMOE_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % 8 || reinterpret_cast<uintptr_t>(logits) % 4)
    return QMOE_ERR_ALIGN;
  return launch_sample(logits, V, temperature, top_k, top_p, u, token, ranked,
                       static_cast<uint8_t*>(ws), stream);
}

static bool attn_shape_ok(const qmoe_attn_shape* s) {
  return s->n_heads >= 1 && s->n_kv_heads >= 1 && s->n_heads % s->n_kv_heads == 0 &&
         s->head_dim >= 2 && s->slots >= 1 && (s->circular == 0 || s->circular == 1) &&
         s->rope_base > 1.f && std::isfinite(s->rope_base) && std::isfinite(s->scale);
}

size_t qmoe_attn_workspace_bytes(const qmoe_attn_shape* s) {
  if (!s || !attn_shape_ok(s)) return 0;
  return attn_ws_bytes(s->n_heads, s->n_kv_heads, s->head_dim, s->slots);
}

qmoe_status qmoe_attn_decode(const qmoe_attn_shape* s, const float* q, const float* k,
                             const float* v, int32_t pos, uint16_t* k_cache, uint16_t* v_cache,
                             uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  if (!s || !q || !k || !v || !k_cache || !v_cache || !out || !ws) return QMOE_ERR_NULL_ARG;
  if (!attn_shape_ok(s) || pos < 0 || (!s->circular && pos >= s->slots))
    return QMOE_ERR_BAD_SHAPE;
  if (!attn_supported(s->head_dim, s->n_heads / s->n_kv_heads)) return QMOE_ERR_UNSUPPORTED;
  if ((int64_t)s->n_kv_heads * s->slots * s->head_dim > ((int64_t)1 << 40)) return QMOE_ERR_UNSUPPORTED;
  if (ws_bytes < attn_ws_bytes(s->n_heads, s->n_kv_heads, s->head_dim, s->slots))
    return QMOE_ERR_WORKSPACE;
  const uintptr_t al = reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache) |
                       reinterpret_cast<uintptr_t>(ws);
  if (al % 16 || reinterpret_cast<uintptr_t>(q) % 4 || reinterpret_cast<uintptr_t>(k) % 4 ||
      reinterpret_cast<uintptr_t>(v) % 4 || reinterpret_cast<uintptr_t>(out) % 2)
    return QMOE_ERR_ALIGN;
  return launch_attn(q, k, v, s->n_heads, s->n_kv_heads, s->head_dim, s->slots, s->circular != 0,
                     pos, s->rope_base, s->scale, k_cache, v_cache, out, ws, stream);
}

qmoe_status qmoe_attn_workspace_status(void* ws, size_t ws_bytes, int32_t n_kv_heads,
                                       int32_t* device_code, void* stream) {
  if (!ws || !device_code) return QMOE_ERR_NULL_ARG;
  if (n_kv_heads < 1) return QMOE_ERR_BAD_SHAPE;
  if (ws_bytes < attn_ctl_bytes(n_kv_heads)) return QMOE_ERR_WORKSPACE;
  uint32_t v = 0;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(&v, ws, 4, hipMemcpyDeviceToHost, st) != hipSuccess) return QMOE_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return QMOE_ERR_HIP;
  *device_code = (int32_t)v;
  if (v != 0) {
    // a merge gave up: partial words of the unfinished call may remain;
    // the whole workspace starts afresh
    if (hipMemsetAsync(ws, 0, ws_bytes, st) != hipSuccess) return QMOE_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return QMOE_ERR_HIP;
    return QMOE_ERR_DEVICE;
  }
  return QMOE_OK;
}

size_t qmoe_tiled4_bytes(int32_t rows, int32_t cols) {
  if (rows < 1 || cols < 64 || cols % 64) return 0;
  return tiled4_size(rows, cols);
}

// Host-side gather into the tiled order (see include/qmoe.h); rows past
// `rows` stay zero.
qmoe_status qmoe_repack_tiled4(const uint8_t* q, const uint16_t* scales, const uint16_t* biases,
                               int32_t rows, int32_t cols, void* out, size_t out_bytes) {
  if (!q || !scales || !biases || !out) return QMOE_ERR_NULL_ARG;
  const size_t need = qmoe_tiled4_bytes(rows, cols);
  if (need == 0) return QMOE_ERR_BAD_SHAPE;
  if (out_bytes < need) return QMOE_ERR_WORKSPACE;
  const int64_t CH = cols / 32, G = cols / 64, RB = (rows + 7) / 8;
  uint8_t* o = static_cast<uint8_t*>(out);
  std::memset(o, 0, need);
  for (int64_t rb = 0; rb < RB; ++rb)
    for (int64_t c = 0; c < CH; ++c)
      for (int64_t r = 0; r < 8; ++r) {
        const int64_t row = rb * 8 + r;
        if (row < rows) std::memcpy(o + ((rb * CH + c) * 8 + r) * 16, q + (row * CH + c) * 16, 16);
      }
  uint32_t* pairs = reinterpret_cast<uint32_t*>(o + RB * CH * 8 * 16);
  for (int64_t rb = 0; rb < RB; ++rb)
    for (int64_t r = 0; r < 8; ++r) {
      const int64_t row = rb * 8 + r;
      if (row >= rows) continue;
      for (int64_t g = 0; g < G; ++g)
        pairs[(rb * 8 + r) * G + g] =
            (uint32_t)scales[row * G + g] | ((uint32_t)biases[row * G + g] << 16);
    }
  return QMOE_OK;
}

qmoe_status qmoe_gemv_tiled4(const void* tiled, int32_t rows, int32_t cols, const uint16_t* x,
                             float* y, int32_t row_blocks_per_wave, void* stream) {
  if (!tiled || !x || !y) return QMOE_ERR_NULL_ARG;
  if (qmoe_tiled4_bytes(rows, cols) == 0) return QMOE_ERR_BAD_SHAPE;
  if (row_blocks_per_wave < 0 || row_blocks_per_wave > 2) return QMOE_ERR_BAD_SHAPE;
  if (!gemv_tiled4_supported(cols)) return QMOE_ERR_UNSUPPORTED;
  if (!al16(tiled) || !al16(x)) return QMOE_ERR_ALIGN;
  return launch_gemv_tiled4(static_cast<const uint8_t*>(tiled), rows, cols, x, y,
                            row_blocks_per_wave, stream);
}

qmoe_status qmoe_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int32_t T, int32_t H,
                         uint16_t* out, void* stream) {
  if (!x || !gamma || !out) return QMOE_ERR_NULL_ARG;
  if (T < 1 || H < 64 || H % 64 || H > QMOE_MAX_HIDDEN) return QMOE_ERR_BAD_SHAPE;
  if (!al16(x) || !al16(gamma) || !al16(out)) return QMOE_ERR_ALIGN;
  return launch_rmsnorm(x, gamma, eps, T, H, out, stream);
}

qmoe_status qmoe_router_topk(const qmoe_qtensor* Wr, const float* logit_bias, const uint16_t* x,
                             int32_t T, int32_t top_k, int32_t* idx, float* w, float* logits,
                             void* ws, size_t ws_bytes, void* stream) {
  if (!Wr || !x || !idx || !w) return QMOE_ERR_NULL_ARG;
  qmoe_status s = check_q(Wr, 8);
  if (s != QMOE_OK) return s;
  if (T < 1 || T > QMOE_MAX_TOKENS || top_k < 1 || top_k > Wr->rows) return QMOE_ERR_BAD_SHAPE;
  if (top_k > QMOE_MAX_TOP_K || Wr->rows > QMOE_MAX_EXPERTS || Wr->cols > QMOE_MAX_HIDDEN)
    return QMOE_ERR_UNSUPPORTED;
  if (!al16(x)) return QMOE_ERR_ALIGN;
  if (!ws) return QMOE_ERR_WORKSPACE;
  if (ws_bytes < qmoe_router_workspace_bytes(Wr->rows, T)) return QMOE_ERR_WORKSPACE;
  return launch_router(*Wr, logit_bias, x, T, top_k, idx, w, logits, static_cast<uint8_t*>(ws),
                       stream);
}

qmoe_status qmoe_expert_ffn(const qmoe_moe_layer* L, const uint16_t* h, const int32_t* idx,
                            const float* w, const int32_t* expert_slot, const uint16_t* residual,
                            uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  qmoe_status s = check_layer(L);
  if (s != QMOE_OK) return s;
  if (!h || !idx || !w || !out) return QMOE_ERR_NULL_ARG;
  if (!al16(h) || (residual && (reinterpret_cast<uintptr_t>(residual) & 1u))) return QMOE_ERR_ALIGN;
  if (!ws) return QMOE_ERR_WORKSPACE;
  if (ws_bytes < ws_bytes_layer(L, 1)) return QMOE_ERR_WORKSPACE;
  return launch_moe_step(*L, h, idx, w, expert_slot, residual, out, nullptr, nullptr,
                         static_cast<uint8_t*>(ws), 0, stream);
}

qmoe_status qmoe_expert_ffn_shared(const qmoe_moe_layer* L, const uint16_t* h, void* ws,
                                   size_t ws_bytes, void* stream) {
  qmoe_status s = check_layer(L);
  if (s != QMOE_OK) return s;
  if (!h) return QMOE_ERR_NULL_ARG;
  if (!al16(h)) return QMOE_ERR_ALIGN;
  if (!ws || ws_bytes < ws_bytes_layer(L, 1)) return QMOE_ERR_WORKSPACE;
  return launch_moe_step(*L, h, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                         static_cast<uint8_t*>(ws), kStepShared, stream);
}

qmoe_status qmoe_expert_ffn_routed(const qmoe_moe_layer* L, const uint16_t* h, const int32_t* idx,
                                   const float* w, const int32_t* expert_slot,
                                   const uint16_t* residual, uint16_t* out, void* ws,
                                   size_t ws_bytes, void* stream) {
  qmoe_status s = check_layer(L);
  if (s != QMOE_OK) return s;
  if (!h || !idx || !w || !out) return QMOE_ERR_NULL_ARG;
  if (!al16(h) || (residual && (reinterpret_cast<uintptr_t>(residual) & 1u))) return QMOE_ERR_ALIGN;
  if (!ws || ws_bytes < ws_bytes_layer(L, 1)) return QMOE_ERR_WORKSPACE;
  return launch_moe_step(*L, h, idx, w, expert_slot, residual, out, nullptr, nullptr,
                         static_cast<uint8_t*>(ws), kStepRouted, stream);
}

qmoe_status qmoe_moe_decode(const qmoe_moe_layer* L, const uint16_t* x, const int32_t* expert_slot,
                            int32_t residual, uint16_t* out, int32_t* idx_out, float* w_out,
                            void* ws, size_t ws_bytes, void* stream) {
  qmoe_status s = check_layer(L);
  if (s != QMOE_OK) return s;
  if (!x || !out) return QMOE_ERR_NULL_ARG;
  if (!al16(x)) return QMOE_ERR_ALIGN;
  if (!ws) return QMOE_ERR_WORKSPACE;
  if (ws_bytes < ws_bytes_layer(L, 1)) return QMOE_ERR_WORKSPACE;
  return launch_moe_step(*L, x, nullptr, nullptr, expert_slot, residual ? x : nullptr, out,
                         idx_out, w_out, static_cast<uint8_t*>(ws), 0, stream);
}

qmoe_status qmoe_moe_decode_noalloc(const qmoe_moe_layer* L, const uint16_t* x,
                                    const int32_t* expert_slot, int32_t residual, uint16_t* out,
                                    int32_t* idx_out, float* w_out, void* stream) {
  qmoe_status s = check_layer(L);
  if (s != QMOE_OK) return s;
  if (!x || !out) return QMOE_ERR_NULL_ARG;
  if (!al16(x)) return QMOE_ERR_ALIGN;
  if (ws_bytes_layer(L, 1) > kScratchBytes) return QMOE_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint8_t* ws = nullptr;
  if ((s = scratch_for_device(st, &ws)) != QMOE_OK) return s;
  return launch_moe_step(*L, x, nullptr, nullptr, expert_slot, residual ? x : nullptr, out,
                         idx_out, w_out, ws, 0, stream, nullptr, nullptr, /*heal=*/1);
}

qmoe_status qmoe_prefill_grouped(const qmoe_moe_layer* L, const uint16_t* X, int32_t T,
                                 const int32_t* idx, const float* w, const uint16_t* residual,
                                 uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  qmoe_status s = check_layer(L);
  if (s != QMOE_OK) return s;
  if (!X || !idx || !w || !out) return QMOE_ERR_NULL_ARG;
  if (T < 1 || T > QMOE_MAX_TOKENS) return QMOE_ERR_BAD_SHAPE;
  if (!al16(X) || !al16(out) || (residual && !al16(residual))) return QMOE_ERR_ALIGN;
  if (!ws) return QMOE_ERR_WORKSPACE;
  if (ws_bytes < ws_bytes_layer(L, T)) return QMOE_ERR_WORKSPACE;
  return launch_prefill(*L, X, T, idx, w, residual, out, static_cast<uint8_t*>(ws), stream);
}

qmoe_status qmoe_prefill_dispatch_offsets(const qmoe_moe_layer* L, int32_t T,
                                          size_t* counts, size_t* offsets, size_t* perm) {
  qmoe_status s = check_layer(L);
  if (s != QMOE_OK) return s;
  if (!counts || !offsets || !perm) return QMOE_ERR_NULL_ARG;
  if (T < 1 || T > QMOE_MAX_TOKENS) return QMOE_ERR_BAD_SHAPE;
  prefill_dispatch_offsets(*L, T, counts, offsets, perm);
  return QMOE_OK;
}

qmoe_status qmoe_workspace_status(void* ws, size_t ws_bytes, int32_t* device_code, void* stream) {
  if (!ws || !device_code) return QMOE_ERR_NULL_ARG;
  if (ws_bytes < kCtlBytes) return QMOE_ERR_WORKSPACE;
  uint32_t v = 0;
  uint8_t* word = static_cast<uint8_t*>(ws) + (size_t)ctl::kError * 4;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(&v, word, 4, hipMemcpyDeviceToHost, st) != hipSuccess) return QMOE_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return QMOE_ERR_HIP;
  *device_code = (int32_t)v;
  if (v != 0) {
    // a wait gave up: flags, tags and counters may hold values of the
    // unfinished call; start the control area afresh
    if (hipMemsetAsync(ws, 0, kCtlBytes, st) != hipSuccess) return QMOE_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return QMOE_ERR_HIP;
    return QMOE_ERR_DEVICE;
  }
  return QMOE_OK;
}

qmoe_status qmoe_workspace_tag_counter(void* ws, size_t ws_bytes, uint32_t* value, void* stream) {
  if (!ws || !value) return QMOE_ERR_NULL_ARG;
  if (ws_bytes < kCtlBytes) return QMOE_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint32_t v[ctl::kGenRep];
  for (int r = 0; r < ctl::kGenRep; ++r)
    if (hipMemcpyAsync(&v[r], static_cast<uint8_t*>(ws) + ctl::kGenBase + ctl::kGenStride * r, 4,
                       hipMemcpyDeviceToHost, st) != hipSuccess)
      return QMOE_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return QMOE_ERR_HIP;
  for (int r = 1; r < ctl::kGenRep; ++r)
    if (v[r] != v[0]) return QMOE_ERR_DEVICE;
  *value = v[0];
  return QMOE_OK;
}

qmoe_status qmoe_workspace_raise_tag_counter(void* ws, size_t ws_bytes, uint32_t value,
                                             void* stream) {
  if (!ws) return QMOE_ERR_NULL_ARG;
  if (ws_bytes < kCtlBytes) return QMOE_ERR_WORKSPACE;
  uint32_t cur = 0;
  qmoe_status s = qmoe_workspace_tag_counter(ws, ws_bytes, &cur, stream);
  if (s != QMOE_OK) return s;
  if (value < cur || value >= ctl::kGenLimit) return QMOE_ERR_BAD_SHAPE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  for (int r = 0; r < ctl::kGenRep; ++r)
    if (hipMemcpyAsync(static_cast<uint8_t*>(ws) + ctl::kGenBase + ctl::kGenStride * r, &value, 4,
                       hipMemcpyHostToDevice, st) != hipSuccess)
      return QMOE_ERR_HIP;
  return hipStreamSynchronize(st) == hipSuccess ? QMOE_OK : QMOE_ERR_HIP;
}

qmoe_status qmoe_moe_decode_timed(const qmoe_moe_layer* L, const uint16_t* x,
                                  const int32_t* expert_slot, int32_t residual, uint16_t* out,
                                  int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes,
                                  void* stream, void* ev_start, void* ev_stop) {
  qmoe_status s = check_layer(L);
  if (s != QMOE_OK) return s;
  if (!x || !out) return QMOE_ERR_NULL_ARG;
  if (!al16(x)) return QMOE_ERR_ALIGN;
  if (!ws || ws_bytes < ws_bytes_layer(L, 1)) return QMOE_ERR_WORKSPACE;
  return launch_moe_step(*L, x, nullptr, nullptr, expert_slot, residual ? x : nullptr, out,
                         idx_out, w_out, static_cast<uint8_t*>(ws), 0, stream, ev_start, ev_stop);
}

/* Test-only variant: runs the step as separate launches per role instead of
 * one launch with in-kernel waits (same kernels, same arithmetic). */
qmoe_status qmoe_moe_decode_phased(const qmoe_moe_layer* L, const uint16_t* x,
                                   const int32_t* expert_slot, int32_t residual, uint16_t* out,
                                   int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes,
                                   void* stream) {
  qmoe_status s = check_layer(L);
  if (s != QMOE_OK) return s;
  if (!x || !out) return QMOE_ERR_NULL_ARG;
  if (!al16(x)) return QMOE_ERR_ALIGN;
  if (!ws || ws_bytes < ws_bytes_layer(L, 1)) return QMOE_ERR_WORKSPACE;
  return launch_moe_step(*L, x, nullptr, nullptr, expert_slot, residual ? x : nullptr, out,
                         idx_out, w_out, static_cast<uint8_t*>(ws), 1, stream);
}

size_t qmoe_stack_table_bytes(int32_t n_layers) {
  if (n_layers < 1 || n_layers > QMOE_MAX_LAYERS) return 0;
  return sizeof(StackLayerDev) * (size_t)n_layers;
}

qmoe_status qmoe_stack_table_init(const qmoe_moe_layer* layers, int32_t n_layers, void* table,
                                  size_t table_bytes, void* stream) {
  if (!layers || !table) return QMOE_ERR_NULL_ARG;
  if (n_layers < 1 || n_layers > QMOE_MAX_LAYERS) return QMOE_ERR_BAD_SHAPE;
  if (!al16(table)) return QMOE_ERR_ALIGN;
  if (table_bytes < qmoe_stack_table_bytes(n_layers)) return QMOE_ERR_WORKSPACE;
  StackLayerDev* host = new StackLayerDev[n_layers];
  for (int l = 0; l < n_layers; ++l) {
    const qmoe_moe_layer& L = layers[l];
    qmoe_status s = check_layer(&L);
    if (s == QMOE_OK && !same_shape(L, layers[0])) s = QMOE_ERR_BAD_SHAPE;
    if (s != QMOE_OK) {
      delete[] host;
      return s;
    }
    StackLayerDev& d = host[l];
    d.router = devq(L.router); d.gate = devq(L.gate); d.up = devq(L.up); d.down = devq(L.down);
    d.shg = devq(L.sh_gate); d.shu = devq(L.sh_up); d.shd = devq(L.sh_down);
    d.gamma = L.rms_gamma;
    d.lbias = L.logit_bias;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  qmoe_status r = QMOE_OK;
  if (hipMemcpyAsync(table, host, sizeof(StackLayerDev) * n_layers, hipMemcpyHostToDevice, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    r = QMOE_ERR_HIP;
  delete[] host;
  return r;
}

size_t qmoe_stack_workspace_bytes(const qmoe_moe_layer* L) {
  if (check_layer(L) != QMOE_OK) return 0;
  return stack_ws_bytes(L);
}

qmoe_status qmoe_stack_decode(const qmoe_moe_layer* L, const void* table, int32_t n_layers,
                              const uint16_t* x, uint16_t* out, uint16_t* layer_out,
                              int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes,
                              void* stream) {
  qmoe_status s = check_layer(L);
  if (s != QMOE_OK) return s;
  if (!table || !x || !out) return QMOE_ERR_NULL_ARG;
  if (n_layers < 1 || n_layers > QMOE_MAX_LAYERS) return QMOE_ERR_BAD_SHAPE;
  if (!al16(table) || !al16(x) || !al16(out) || (layer_out && !al16(layer_out)))
    return QMOE_ERR_ALIGN;
  if (x == out) return QMOE_ERR_BAD_SHAPE;
  if (!ws || ws_bytes < stack_ws_bytes(L)) return QMOE_ERR_WORKSPACE;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  return launch_moe_stack(*L, table, n_layers, x, out, layer_out, idx_out, w_out, w8,
                          reinterpret_cast<uint16_t*>(w8 + stack_xb_offset(L)), stream);
}

}  // extern "C"
