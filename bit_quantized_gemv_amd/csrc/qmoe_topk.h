// qmoe_topk.h -- top-k of the router logits and the softmax over the kept
// ones, for one wave (devtrends.cc "Come eseguire un modello da 26 miliardi…",
// section "Qual è il trucco principale dell'architettura": the router keeps
// 8 experts per token; remio.ai "TurboFieldfare esegue Mac Gemma 4 26B in
// 2 GB…", section "L'affermazione dei 2 GB…").  Order: descending logit,
// equal logits by lower expert index; weights p_j = exp(l_j - l_max) /
// sum_j p_j, the sum taken in rank order.
#pragma once
#include "qmoe_common.h"

namespace qmoe {

// Order value of a logit: an unsigned integer that increases with the
// fp32 value (-0 counts as +0), and back.
__device__ __forceinline__ uint32_t topk_ord(float f) {
  const uint32_t b = __float_as_uint(f + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float topk_value(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// One wave: top-k of E logits held as v[m] = logit[lane + 64 m] and the
// softmax over the kept ones, with a short dependency chain (no rounds of
// argmax):
//   1. T = the k-th largest order value, bit by bit from the top: keep a
//      bit when at least k order values are >= the prefix with it (one
//      ballot count per value slot and bit);
//   2. the k selected are the values above T and, in index order, the
//      first k - #(above T) of those equal to T (ballot prefix counts);
//   3. they are gathered into k slots of `xch` (LDS, 2k words of 8 bytes)
//      as (order value, complemented index) keys, and lane j < k ranks
//      slot j against the k keys;
//   4. lane j takes rank j for the softmax.
// stamps (trace builds; else null): s_memrealtime after the select, the
// gather and the ranking, in stamps[0..3).
template <int NV>
__device__ void wave_topk_radix(const float (&v)[NV], int E, int K, int32_t* idx_s, float* w_s,
                                int32_t* idx2, float* w2, uint64_t* xch, int tid = threadIdx.x,
                                uint64_t* stamps = nullptr) {
  const int lane = tid & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  uint32_t o[NV];
#pragma unroll
  for (int m = 0; m < NV; ++m) o[m] = lane + 64 * m < E ? topk_ord(v[m]) : 0u;  // 0: no expert
  uint32_t T = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = T | (1u << b);
    uint32_t n = 0;
#pragma unroll
    for (int m = 0; m < NV; ++m) n += (uint32_t)__popcll(__ballot(o[m] >= c));
    if (n >= (uint32_t)K) T = c;
  }
  if (stamps && lane == 0) stamps[0] = __builtin_amdgcn_s_memrealtime();
  uint32_t above = 0;
#pragma unroll
  for (int m = 0; m < NV; ++m) above += (uint32_t)__popcll(__ballot(o[m] > T));
  const uint32_t need = (uint32_t)K - above;
  uint32_t ties = 0, base = 0;
#pragma unroll
  for (int m = 0; m < NV; ++m) {
    const uint64_t tie = __ballot(o[m] == T);
    const bool take =
        o[m] > T || (o[m] == T && ties + (uint32_t)__popcll(tie & below) < need);
    ties += (uint32_t)__popcll(tie);
    const uint64_t sel = __ballot(take);
    if (take)
      xch[base + (uint32_t)__popcll(sel & below)] =
          ((uint64_t)o[m] << 32) | (uint32_t)~(lane + 64 * m);
    base += (uint32_t)__popcll(sel);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if (stamps && lane == 0) stamps[1] = __builtin_amdgcn_s_memrealtime();
  if (lane < K) {
    const uint64_t kj = xch[lane];
    uint32_t r = 0;
    for (int j = 0; j < K; ++j) r += xch[j] > kj ? 1u : 0u;
    xch[K + r] = kj;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if (stamps && lane == 0) stamps[2] = __builtin_amdgcn_s_memrealtime();
  float p = 0.f;
  int e = 0;
  if (lane < K) {
    const uint64_t kr = xch[K + lane];
    e = (int)~(uint32_t)kr;
    p = expf(topk_value((uint32_t)(kr >> 32)) - topk_value((uint32_t)(xch[K] >> 32)));
  }
  float sum = 0.f;
  for (int j = 0; j < K; ++j)
    sum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p), j));
  if (lane < K) {
    const float wj = p / sum;
    idx_s[lane] = e;
    w_s[lane] = wj;
    if (idx2) idx2[lane] = e;
    if (w2) w2[lane] = wj;
  }
}

}  // namespace qmoe
