// qmoe_router.hip -- the 8-bit affine router for up to 128 tokens at once
// (the prefill chunk) on the matrix cores, with the softmax top-k
// (devtrends.cc "Come eseguire un modello da 26 miliardi…", section "Qual è
// il trucco principale dell'architettura": a router picks 8 experts per
// token; remio.ai "TurboFieldfare esegue Mac Gemma 4 26B in 2 GB…", section
// "L'affermazione dei 2 GB…": 8-bit affine router weights).
//
//   logit[t][e] = sum_g ( s[e][g] * D_g[t][e] + b[e][g] * X_g[t] )  (+ bias[e])
//   D_g[t][e]  = sum_{c in group g} q[e][c] x[t][c],   X_g[t] = sum_{c in g} x[t][c]
//
// Codes 0..255 and the bf16 inputs are exact bf16 operands, so every
// product is exact: D_g comes from two v_mfma_f32_16x16x32_bf16 per group of
// 64 columns (fp32 accumulation), X_g from the same instruction with a ones
// operand, and the per-group scale and bias are applied in fp32 on the
// vector units.  A block owns a tile of 8 tokens x 16 experts (the MFMA's
// 16 A rows hold the 8 tokens twice); its 8 waves split the groups, and
// their partial tiles are summed in a fixed order.  The last block of a
// token tile (a counter) runs the top-k of its tokens, one per wave.
#include <hip/hip_runtime.h>

#include "qmoe_common.h"
#include "qmoe_topk.h"

namespace qmoe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float rt_f4_t __attribute__((ext_vector_type(4)));

constexpr int kRtTile = 16;                // experts per tile (MFMA rows and columns)
constexpr int kRtTokTile = 8;              // tokens per tile: one per wave in the top-k
constexpr int kRtWaves = 8;                // waves per block: the groups split 8 ways
constexpr int kRtThreads = kRtWaves * 64;
constexpr int kRtGP = 6;                   // groups per wave per pass (loads issued at once)

// Eight codes (the bytes of w0 then w1) as bf16; integers 0..255 are exact.
__device__ __forceinline__ bf16x8_t codes8_bf16(uint32_t w0, uint32_t w1) {
  bf16x8_t o;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w = i < 4 ? w0 : w1;
    const float f = (float)((w >> (8 * (i & 3))) & 0xffu);
    o[i] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(f) >> 16));
  }
  return o;
}

// grid (ceil(E/16), ceil(T/8)), kRtThreads threads.  NV = ceil(E/64) value
// slots per lane in the top-k.
template <int NV>
__global__ __launch_bounds__(kRtThreads) void k_router_mma(DevQ Wr, const float* lbias,
                                                           const uint16_t* x, int T, int E, int H,
                                                           int K, int32_t* idx, float* w,
                                                           float* logits_out, float* logits_ws,
                                                           uint32_t* ctlw) {
  __shared__ float part[kRtWaves][kRtTile * kRtTile];
  __shared__ uint64_t xch[kRtWaves][2 * QMOE_MAX_TOP_K];
  __shared__ int32_t idx_sh[kRtWaves][QMOE_MAX_TOP_K];
  __shared__ float w_sh[kRtWaves][QMOE_MAX_TOP_K];
  __shared__ uint32_t last;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, j = lane >> 4;
  const int e0 = blockIdx.x * kRtTile, t0 = blockIdx.y * kRtTokTile;
  const int G = H / 64;
  const int g0 = wave * G / kRtWaves, g1 = (wave + 1) * G / kRtWaves;
  // this lane's A row (token) and B column (expert); past the end: a valid
  // row whose results are not stored
  const int ta = min(t0 + (n & (kRtTokTile - 1)), T - 1), eb = min(e0 + n, E - 1);
  const uint16_t* xr = x + (size_t)ta * H;
  const uint8_t* qr = Wr.q + (size_t)eb * H;
  const QMOE_GLOBAL uint16_t* sr = gptr(Wr.s + (size_t)eb * G);
  const QMOE_GLOBAL uint16_t* br = gptr(Wr.b + (size_t)eb * G);
  bf16x8_t ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = __builtin_bit_cast(__bf16, (uint16_t)0x3F80);
  rt_f4_t acc = {0.f, 0.f, 0.f, 0.f};
  // the logit bias of the expert this thread sums below, read ahead of the
  // weights so that it is not a round trip after the reduction
  float lb = 0.f;
  if (lbias && threadIdx.x < kRtTile * kRtTile)
    lb = gptr(lbias)[min(e0 + (int)threadIdx.x % kRtTile, E - 1)];
  // MFMA k slots 8j..8j+7 of the first instruction hold columns 16j..16j+7
  // of the group, those of the second 16j+8..16j+15 (any assignment of
  // columns to slots gives the same exact products)
  for (int gb = g0; gb < g1; gb += kRtGP) {
    uint4 xa[kRtGP], xb[kRtGP], qv[kRtGP];
    uint32_t sb[kRtGP];
#pragma unroll
    for (int i = 0; i < kRtGP; ++i) {
      const int c = 64 * min(gb + i, g1 - 1) + 16 * j;
      xa[i] = ld_g16(xr + c, 0);
      xb[i] = ld_g16(xr + c + 8, 0);
      qv[i] = ld_g16(qr + c, 0);
      const int g = min(gb + i, g1 - 1);
      sb[i] = (uint32_t)sr[g] | ((uint32_t)br[g] << 16);
    }
#pragma unroll
    for (int i = 0; i < kRtGP; ++i) {
      if (gb + i < g1) {
        const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, xa[i]);
        const bf16x8_t a2 = __builtin_bit_cast(bf16x8_t, xb[i]);
        rt_f4_t d = {0.f, 0.f, 0.f, 0.f}, xs = {0.f, 0.f, 0.f, 0.f};
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, codes8_bf16(qv[i].x, qv[i].y), d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2, codes8_bf16(qv[i].z, qv[i].w), d, 0, 0, 0);
        xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, ones, xs, 0, 0, 0);
        xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2, ones, xs, 0, 0, 0);
        const float s = half_to_f32(sb[i] & 0xffffu), b = half_to_f32(sb[i] >> 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[r] = fmaf(s, d[r], acc[r]);
          acc[r] = fmaf(b, xs[r], acc[r]);
        }
      }
    }
  }
  // lane holds tokens t0 + 4j + r, expert e0 + n; sum the waves in order
#pragma unroll
  for (int r = 0; r < 4; ++r) part[wave][(4 * j + r) * kRtTile + n] = acc[r];
  __syncthreads();
  if (threadIdx.x < kRtTile * kRtTile) {
    const int m = threadIdx.x / kRtTile, c = threadIdx.x % kRtTile;
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < kRtWaves; ++q) v += part[q][threadIdx.x];
    const int t = t0 + m, e = e0 + c;
    if (m < kRtTokTile && t < T && e < E) {
      if (lbias) v += lb;
      st_dev(logits_ws + (size_t)t * E + e, v);
      if (logits_out) logits_out[(size_t)t * E + e] = v;
    }
  }
  // the last block of this token tile runs the top-k of its tokens
  wait_vm();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t* cnt = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(ctlw) + ctl::kCntBase +
                                                64 * (ctl::kCntRouterTile + blockIdx.y));
    const uint32_t prev = add_dev(cnt, 1u);
    last = prev == gridDim.x - 1;
    if (prev == gridDim.x - 1) st_dev(cnt, 0u);
  }
  __syncthreads();
  if (!last) return;
  static_assert(kRtTokTile == kRtWaves, "one token per wave");
  for (int t = t0 + wave; t < min(T, t0 + kRtTokTile); t += kRtWaves) {
    float v[NV];
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int e = lane + 64 * m;
      v[m] = ld_dev(logits_ws + (size_t)t * E + min(e, E - 1));
    }
    wave_topk_radix<NV>(v, E, K, idx_sh[wave], w_sh[wave], idx + (size_t)t * K, w + (size_t)t * K,
                        xch[wave]);
  }
}

template <int NV>
static void launch_router_nv(const qmoe_qtensor& Wr, const float* lbias, const uint16_t* x, int T,
                             int K, int32_t* idx, float* w, float* logits, float* lw, uint32_t* c,
                             hipStream_t st) {
  const int E = Wr.rows, H = Wr.cols;
  dim3 grid(cdiv(E, kRtTile), cdiv(T, kRtTokTile));
  hipLaunchKernelGGL(k_router_mma<NV>, grid, dim3(kRtThreads), 0, st, devq(Wr), lbias, x, T, E, H,
                     K, idx, w, logits, lw, c);
}

qmoe_status launch_router(const qmoe_qtensor& Wr, const float* lbias, const uint16_t* x, int T,
                          int K, int32_t* idx, float* w, float* logits, uint8_t* ws,
                          void* stream) {
  const int E = Wr.rows;
  WsLayout wl = ws_layout(E, K, 0, 0, T);
  float* lw = reinterpret_cast<float*>(ws + wl.logits);
  uint32_t* c = reinterpret_cast<uint32_t*>(ws + wl.ctl);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (E <= 64)
    launch_router_nv<1>(Wr, lbias, x, T, K, idx, w, logits, lw, c, st);
  else if (E <= 128)
    launch_router_nv<2>(Wr, lbias, x, T, K, idx, w, logits, lw, c, st);
  else if (E <= 256)
    launch_router_nv<4>(Wr, lbias, x, T, K, idx, w, logits, lw, c, st);
  else
    launch_router_nv<8>(Wr, lbias, x, T, K, idx, w, logits, lw, c, st);
  return hipGetLastError() == hipSuccess ? QMOE_OK : QMOE_ERR_HIP;
}

}  // namespace qmoe
