// qmoe_sample.hip -- the token choice after the last layer: the top-K of
// the vocabulary's logits, their softmax at a temperature, the top-P cut and
// one draw (elsolitario.org, TurboFieldfare article, section "Cómo empezar":
// temperature 0.2, top-K 64 and top-P 0.95 by default, temperature 0 for a
// deterministic choice; iitog.ru "TurboFieldfare: движок с открытым
// кодом…", technical paragraph: sampling is one of the engine's kernels).
//
// Order: descending logit, equal logits by lower token id.  Temperature 0
// takes rank 0.  Otherwise p_j = exp((l_j - l_0) / T) over the K kept
// ranks; rank j stays while the mass of the ranks before it is below
// top_p of the total; the draw u in [0, 1) takes the first kept rank whose
// cumulative mass exceeds u times the kept mass.  Sums in rank order, fp32.
//
// Two launches:
//   local  block b takes 1024 logits (4096 past 262,144 logits): each wave
//          the top-K of its quarter, then wave 0 the top-K of the waves' 4K;
//          the block's K keys go to the workspace in rank order
//   final  one block of 16 waves: a bound at or below the K-th largest key
//          from the blocks' leading keys, the keys at or above it (a few
//          hundred for smooth logits) compacted into LDS, their top-K in
//          rank order, then the softmax, the cut and the draw
// A key is (order value of the logit) << 32 | ~id: one unsigned order for
// "larger logit, then lower id", unique per token; missing entries get keys
// of order 0 (below every real key), each a different one, so every key of
// a selection is unique.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmoe.h"
#include "qmoe_common.h"
#include "qmoe_topk.h"

namespace qmoe {

constexpr int kSmpBlock = 256;               // local: 4 waves
constexpr int kSmpPerWave = 1024;            // keys per wave (16 per lane)
constexpr int kSmpPerBlock = 4 * kSmpPerWave;
constexpr int kSmpFinalWaves = 16;           // final: 1024 threads
constexpr int kSmpMaxBlocks = kSmpFinalWaves * kSmpPerWave / 64;  // K <= 64 keys per block

__device__ __forceinline__ uint64_t smp_key(float l, uint32_t id) {
  return ((uint64_t)topk_ord(l) << 32) | (uint32_t)~id;
}
// Key of a missing entry number u: order value 0 (below every logit), and
// distinct for distinct u (u < 2^30), so that all keys of a selection are
// unique.  Numbering: token ids past V; 2^21 + position for padding.
__device__ __forceinline__ uint64_t smp_pad(uint32_t u) { return (uint64_t)(uint32_t)~u; }
constexpr uint32_t kPadBase = 1u << 21;

// One wave: the K (<= 64) largest of the NV * 64 keys k[m] (lane + 64 m),
// written to out[0..K) in descending order.  The keys are unique.
//   1. T, bit by bit from the top: keep a bit when at least K keys are >=
//      the prefix with it; when exactly K are, those are the K largest and
//      the search ends (real keys part after a few dozen bits at most);
//   2. the K taken are the keys above T and, in position order, the first
//      K - #(above T) of those equal to T, gathered into xch[0..K);
//   3. lane j < K ranks slot j against the others (equal keys by slot).
template <int NV>
__device__ void wave_topk_keys(const uint64_t (&k)[NV], int K, uint64_t* xch, uint64_t* out,
                               int lane) {
  uint64_t T = 0;
  for (int b = 63; b >= 0; --b) {
    const uint64_t c = T | (1ull << b);
    uint32_t n = 0;
#pragma unroll
    for (int m = 0; m < NV; ++m) n += (uint32_t)__popcll(__ballot(k[m] >= c));
    if (n >= (uint32_t)K) {
      T = c;
      if (n == (uint32_t)K) break;
    }
  }
  const uint64_t below = (1ull << lane) - 1ull;
  uint32_t above = 0;
#pragma unroll
  for (int m = 0; m < NV; ++m) above += (uint32_t)__popcll(__ballot(k[m] > T));
  const uint32_t need = (uint32_t)K - above;
  uint32_t ties = 0, base = 0;
#pragma unroll
  for (int m = 0; m < NV; ++m) {
    const uint64_t tie = __ballot(k[m] == T);
    const bool take = k[m] > T || (k[m] == T && ties + (uint32_t)__popcll(tie & below) < need);
    ties += (uint32_t)__popcll(tie);
    const uint64_t sel = __ballot(take);
    if (take) xch[base + (uint32_t)__popcll(sel & below)] = k[m];
    base += (uint32_t)__popcll(sel);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  {
    // rank = keys greater (unique keys); every lane reads all 64 slots with
    // no branch between the reads (past K: stale keys, masked)
    const uint64_t kj = xch[lane];
    uint32_t r = 0;
#pragma unroll 16
    for (int i = 0; i < 64; ++i) r += (uint32_t)(xch[i] > kj) & (uint32_t)(i < K);
    if (lane < K) out[r] = kj;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

template <int NV>
__global__ __launch_bounds__(kSmpBlock) void k_sample_local(const float* logits, int V, int K,
                                                            uint64_t* cand) {
  __shared__ uint64_t xch[4][64];
  __shared__ uint64_t wtop[4 * 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t base = ((int64_t)blockIdx.x * 4 + wave) * 64 * NV;
  uint64_t k[NV];
#pragma unroll
  for (int m = 0; m < NV; ++m) {
    const int64_t i = base + lane + 64 * m;
    k[m] = i < V ? smp_key(logits[i], (uint32_t)i) : smp_pad((uint32_t)i);
  }
  // ranks >= K stay missing (distinct per block, wave and lane)
  wtop[wave * 64 + lane] = smp_pad(kPadBase + (blockIdx.x * 4 + wave) * 64 + lane);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  wave_topk_keys<NV>(k, K, xch[wave], wtop + wave * 64, lane);
  __syncthreads();
  if (wave == 0) {
    uint64_t k2[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) k2[m] = wtop[m * 64 + lane];
    wave_topk_keys<4>(k2, K, xch[0], cand + (int64_t)blockIdx.x * K, lane);
  }
}

// The top-K of n keys read through load(i) (i < n <= 16 * 64 * NV0), in
// rank order into top[0..K), by every thread of the 16-wave block: each
// wave the top-K of its share, waves 0..3 the top-K of four waves' each,
// wave 0 the top-K of theirs.  Missing entries get pad keys numbered from
// pad0 (16384 + 2048 numbers).
template <int NV0, typename Load>
__device__ void block_topk(Load load, int n, int K, uint32_t pad0, uint64_t (*xch)[64],
                           uint64_t* wtop, uint64_t* top) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint64_t k[NV0];
#pragma unroll
  for (int m = 0; m < NV0; ++m) {
    const int i = (wave * NV0 + m) * 64 + lane;
    k[m] = i < n ? load(i) : smp_pad(pad0 + (uint32_t)i);
  }
  wtop[wave * 64 + lane] = smp_pad(pad0 + 16384u + wave * 64 + lane);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  wave_topk_keys<NV0>(k, K, xch[wave], wtop + wave * 64, lane);
  __syncthreads();
  uint64_t k2[4];
  if (wave < 4) {
#pragma unroll
    for (int m = 0; m < 4; ++m) k2[m] = wtop[(4 * wave + m) * 64 + lane];
  }
  __syncthreads();
  if (wave < 4) {
    wtop[wave * 64 + lane] = smp_pad(pad0 + 16384u + 1024u + wave * 64 + lane);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    wave_topk_keys<4>(k2, K, xch[wave], wtop + wave * 64, lane);
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int m = 0; m < 4; ++m) k2[m] = wtop[m * 64 + lane];
    wave_topk_keys<4>(k2, K, xch[0], top, lane);
  }
  __syncthreads();
}

// Final block (16 waves) over the nb blocks' K keys each (nb <= 256, each
// block's keys in rank order):
//   1. a bound M at or below the K-th largest key: with nb >= K, the K-th
//      largest of the blocks' first keys (K blocks each hold a key >= it);
//      else the smallest of the blocks' j-th keys, j = ceil(K / nb) (every
//      block holds j keys >= it);
//   2. the keys >= M (at least K of them) compacted into LDS;
//   3. their top-K: one wave when they fit in 256, else the tree.  There
//      are at most K * K = 4096: with nb >= K only the K blocks whose first
//      key is >= M hold keys >= M; else there are nb * K < K * K keys;
// then the softmax, the top-P cut and the draw on wave 0.
constexpr int kSmpSurvCap = 4096;
__global__ __launch_bounds__(kSmpFinalWaves * 64) void k_sample_final(
    const uint64_t* cand, int nb, int K, float temperature, float top_p, float u, int32_t* token,
    int32_t* ranked) {
  __shared__ uint64_t xch[kSmpFinalWaves][64];
  __shared__ uint64_t wtop[kSmpFinalWaves * 64];
  __shared__ uint64_t top[64];
  __shared__ uint64_t surv[kSmpSurvCap];
  __shared__ uint64_t bound;
  __shared__ uint32_t nsurv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // pad numbers past the local blocks' (at most 256 * 256 of them)
  constexpr uint32_t kPadFinal = kPadBase + 256u * 256u;
  const int n = nb * K;
  if (threadIdx.x == 0) nsurv = 0;
  // every key this thread filters in 2., loaded before the bound's search
  constexpr int kPer = kSmpMaxBlocks * 64 / (kSmpFinalWaves * 64);  // nb * K <= 256 * 64
  uint64_t x[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int i = r * kSmpFinalWaves * 64 + (int)threadIdx.x;
    x[r] = i < n ? cand[i] : 0ull;
  }
  // 1. the bound
  if (nb >= K) {
    if (wave == 0) {
      uint64_t k[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int b = lane + 64 * m;
        k[m] = b < nb ? cand[(int64_t)b * K] : smp_pad(kPadFinal + (uint32_t)b);
      }
      wave_topk_keys<4>(k, K, xch[0], top, lane);
      if (lane == 0) bound = top[K - 1];
    }
  } else if (wave == 0) {
    const int j = (K + nb - 1) / nb;
    uint64_t mn = ~0ull;
    for (int b = lane; b < nb; b += 64) {
      const uint64_t x = cand[(int64_t)b * K + j - 1];
      mn = x < mn ? x : mn;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const uint64_t y = __shfl_xor(mn, o);
      mn = y < mn ? y : mn;
    }
    if (lane == 0) bound = mn;
  }
  __syncthreads();
  // 2. the keys >= bound, one LDS count per wave and pass
  const uint64_t M = bound;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int i = r * kSmpFinalWaves * 64 + (int)threadIdx.x;
    const bool keep = i < n && x[r] >= M;
    const uint64_t bal = __ballot(keep);
    if (bal == 0) continue;  // wave-uniform
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&nsurv, (uint32_t)__popcll(bal));
    base = __shfl(base, 0);
    const uint32_t p = base + (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
    if (keep) surv[p] = x[r];  // p < K * K <= kSmpSurvCap (see 3.)
  }
  __syncthreads();
  // 3. their top-K
  const int S = (int)nsurv;
  if (S <= 256) {
    if (wave == 0) {
      uint64_t k[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int i = lane + 64 * m;
        k[m] = i < S ? surv[i] : smp_pad(kPadFinal + 20000u + (uint32_t)i);
      }
      wave_topk_keys<4>(k, K, xch[0], top, lane);
    }
    __syncthreads();
  } else {
    block_topk<4>([&](int i) { return surv[i]; }, S, K, kPadFinal + 20000u, xch, wtop, top);
  }
  if (wave != 0) return;
  // lane r holds rank r
  const uint64_t key = lane < K ? top[lane] : 0ull;
  const int32_t id = (int32_t)~(uint32_t)key;
  if (ranked && lane < K) ranked[lane] = id;
  int r = 0;
  if (temperature > 0.f) {
    const float l0 = topk_value((uint32_t)(top[0] >> 32));
    const float p = lane < K ? expf((topk_value((uint32_t)(key >> 32)) - l0) / temperature) : 0.f;
    // exclusive and inclusive sums in rank order
    float c = 0.f, ex = 0.f, inc = 0.f;
    for (int j = 0; j < K; ++j) {
      const float pj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p), j));
      if (lane == j) ex = c;
      c += pj;
      if (lane == j) inc = c;
    }
    const bool kept = lane < K && (lane == 0 || ex < top_p * c);
    const int m = (int)__popcll(__ballot(kept));
    const float km = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, inc), m - 1));
    const float target = u * km;
    const uint64_t hit = __ballot(lane < m && inc > target);
    r = hit ? (int)__builtin_ctzll(hit) : m - 1;
  }
  const int32_t tok = __builtin_amdgcn_readlane(id, r);
  if (lane == 0) *token = tok;
}

// Logits per phase-one block: 1024 (4 per lane) up to 262,144 logits (256
// blocks), 4096 (16 per lane) past that, so that at most 256 blocks feed
// the final block.
static int sample_per_block(int V) { return V <= 256 * 1024 ? 1024 : kSmpPerBlock; }

size_t sample_ws_bytes(int V, int K) {
  return (size_t)cdiv(V, sample_per_block(V)) * (size_t)K * sizeof(uint64_t);
}

bool sample_supported(int V, int K) {
  return V >= 1 && K >= 1 && K <= 64 && K <= V && cdiv(V, kSmpPerBlock) <= kSmpMaxBlocks;
}

qmoe_status launch_sample(const float* logits, int V, float temperature, int K, float top_p,
                          float u, int32_t* token, int32_t* ranked, uint8_t* ws, void* stream) {
  const int per = sample_per_block(V);
  const int nb = cdiv(V, per);
  uint64_t* cand = reinterpret_cast<uint64_t*>(ws);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (per == 1024)
    hipLaunchKernelGGL(k_sample_local<4>, dim3(nb), dim3(kSmpBlock), 0, st, logits, V, K, cand);
  else
    hipLaunchKernelGGL(k_sample_local<16>, dim3(nb), dim3(kSmpBlock), 0, st, logits, V, K, cand);
  hipLaunchKernelGGL(k_sample_final, dim3(1), dim3(kSmpFinalWaves * 64), 0, st, cand, nb, K,
                     temperature, top_p, u, token, ranked);
  return hipGetLastError() == hipSuccess ? QMOE_OK : QMOE_ERR_HIP;
}

}  // namespace qmoe
