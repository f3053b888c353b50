// qmoe_attn.hip -- decode attention over an FP16 key/value cache, with RoPE
// (iitog.ru "TurboFieldfare: движок с открытым кодом…", technical paragraph:
// the engine's own attention and RoPE kernels, an FP16 KV cache, 25
// sliding-window layers in a bounded circular store and 5 full-attention
// layers in a linear one; remio.ai "TurboFieldfare esegue Mac Gemma 4 26B in
// 2 GB…", section "Mac Gemma 4 26B entra nello spazio disponibile…": a
// 4,096-token cache).
//
// One call handles the token at time pos:
//   q' = RoPE(q), k' = RoPE(k): planes (i, i + D/2), angle pos * base^(-2i/D),
//   rotated in fp64; cache slot pos mod S receives fp16(k') and fp16(v);
//   query head h attends with key/value head h / (Hq / Hkv):
//   out_h = sum_t softmax_t(scale * <q'_h, K_t>) V_t over the window, as bf16.
// Slots attended: 0 .. min(pos + 1, S) - 1.  In a circular store the current
// token's slot held time pos - S, which has just left the window, so every
// other slot holds a token of the window; in a linear store (pos < S) the
// slots past pos are not read.  The current token is never read back from
// memory: split 0 of each key/value head takes its key and value from this
// call's inputs.
//
// Cache layout: [Hkv][S][D] fp16, so one key/value head's tokens are one
// contiguous run.
//
// Split launch, block (split, g): 32 * NP slots of key/value head g, four
// waves of 8 * NP slots each.
//   keys    lane (p = lane / 8, j = lane % 8) holds the 16-byte chunks j,
//           j + 8, ... of the key row of slot 8 * pass + p (8 lanes read 128
//           contiguous bytes); the dot with q' (LDS, 8 distinct addresses
//           per read) is summed over the 8 lanes of the slot
//   values  lane l holds dims 4 (l % (D/4)) .. + 3 of one value row (one
//           row per wave instruction at D = 256, two at D = 128); the row's
//           probability is read from the lane that holds its score
// Every key and value load of a wave is issued before the first use.  The
// block merges its waves (and, in split 0, the current token) into a
// (max, sum, unnormalised output) per head.  With one split it writes the
// output itself; else every split publishes its partial as 64-bit words
// tagged with this call's epoch, and 8 more blocks per key/value head,
// after the split blocks in the grid, merge 64 outputs each as the words
// arrive (one launch per call).  The epochs are workspace words, one per
// merging block; a workspace starts zero-filled.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "qmoe.h"
#include "qmoe_common.h"

namespace qmoe {

constexpr int kAttnWaves = 4;
constexpr int kAttnCUs = 256;  // the split count aims at two blocks per CU or more
constexpr int kAttnErr = 0;         // workspace word: nonzero when a merge wait gave up
constexpr int kAttnEpoch = 16;      // workspace words from here: [Hkv][kAttnMergers] epochs
constexpr int kAttnMergers = 8;     // merging blocks per key/value head (64 outputs each)
constexpr int kAttnSpinLimit = 1 << 20;
// control words (error, epochs), then the partials
size_t attn_ctl_bytes(int Hkv) {
  return ((size_t)(kAttnEpoch + Hkv * kAttnMergers) * 4 + 255) / 256 * 256;
}

// fp64 -> fp16 with one rounding (to nearest, ties to even): round to fp32
// toward zero with the last bit set when inexact ("round to odd"), then to
// fp16; fp32 carries more than two bits beyond fp16's, so the second
// rounding sees the same tie/non-tie decision as the exact value.
__device__ __forceinline__ uint16_t f64_to_f16_bits(double d) {
  float f = (float)d;
  if ((double)f != d) {
    uint32_t u = __float_as_uint(f);
    if (fabs((double)f) > fabs(d)) u -= 1u;  // back toward zero, same sign
    f = __uint_as_float(u | 1u);
  }
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// 8 bytes at p (global memory, non-temporal: the cache is read once per call).
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 ldg8(const uint16_t* p) {
  u32x2_t v = __builtin_nontemporal_load(gptr(reinterpret_cast<const u32x2_t*>(p)));
  return make_uint2(v.x, v.y);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

struct AttnArgs {
  const float* q;      // [Hq][D]
  const float* k;      // [Hkv][D]
  const float* v;      // [Hkv][D]
  uint16_t* kc;        // [Hkv][S][D] fp16
  uint16_t* vc;        // [Hkv][S][D] fp16
  uint16_t* out;       // [Hq][D] bf16
  uint32_t* ctl;       // workspace words: error, epoch
  uint64_t* part;      // [Hkv][nsplit][G][D + 2] tagged words: output, max, sum
  int Hq, S, pos, n_iter, cur, nsplit;
  float scale;
  double log2_base;
};

// Merging block m of key/value head g (launched after the head's split
// blocks, so it never waits for a block that is not yet running): outputs
// 64 m .. 64 m + 63 of the head's group (head t / D, dim t % D).  Thread
// (j = tid / 64, o = tid % 64) takes splits j, j + 4, ...: every word it
// needs, 8 splits per round trip, with the tags checked in plain arithmetic
// (any stale word: load the batch again), so the wait for a late split and
// the read of its words are the same loads; the four split groups meet in
// LDS.  The epoch word (g, m) is this block's
// own: it reads it first and writes the next value last; every merging
// block of every call that splits steps its word once, so the words of a
// head stay equal to the one the split blocks read, (g, 0).
template <int D, int G>
__device__ void attn_merge(const AttnArgs& a, int g, int m) {
  constexpr int kOut = 64, kGrp = kAttnWaves, kB = 8;
  __shared__ float gm[kGrp][kOut], gl[kGrp][kOut], go[kGrp][kOut];
  uint32_t* ep = a.ctl + kAttnEpoch + g * kAttnMergers + m;
  const uint32_t epoch = ld_dev(ep);
  const uint32_t tag = epoch + 1u == 0u ? 1u : epoch + 1u;
  const int j = threadIdx.x / kOut, o = threadIdx.x % kOut, t = m * kOut + o;
  const bool mine = m * kOut < G * D;
  const uint64_t* gp = a.part + (int64_t)g * a.nsplit * G * (D + 2);
  bool failed = false;
  if (mine) {
    // the words, merged online over this thread's splits; each batch
    // polls its own words until all carry this call's tag
    const int tt = t < G * D ? t : 0;
    const int row = (tt / D) * (D + 2), d = tt % D;
    float M = -INFINITY, on = 0.f, ln = 0.f;
    for (int c0 = j; c0 < a.nsplit; c0 += kGrp * kB) {
      float ms[kB], ls[kB], os[kB];
      for (int spin = 0;; ++spin) {
        uint32_t bad = 0;
#pragma unroll
        for (int b = 0; b < kB; ++b) {
          const int sp = c0 + b * kGrp;
          const bool in = sp < a.nsplit;
          const uint64_t* w = gp + (int64_t)(in ? sp : 0) * G * (D + 2) + row;
          const uint64_t wm = ld_dev(w + D), wl = ld_dev(w + D + 1), wo = ld_dev(w + d);
          ms[b] = in ? __uint_as_float((uint32_t)wm) : -INFINITY;
          ls[b] = __uint_as_float((uint32_t)wl);
          os[b] = __uint_as_float((uint32_t)wo);
          const uint32_t x = ((uint32_t)(wm >> 32) ^ tag) | ((uint32_t)(wl >> 32) ^ tag) |
                             ((uint32_t)(wo >> 32) ^ tag);
          bad |= in ? x : 0u;
        }
        if (bad == 0 || failed) break;
        if (spin >= kAttnSpinLimit) {
          failed = true;
          break;
        }
        __builtin_amdgcn_s_sleep(4);
      }
      float Mb = M;
#pragma unroll
      for (int b = 0; b < kB; ++b) Mb = fmaxf(Mb, ms[b]);
      if (Mb == -INFINITY) continue;
      const float r = M == -INFINITY ? 0.f : expf(M - Mb);
      on *= r;
      ln *= r;
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        if (ms[b] == -INFINITY) continue;
        const float f = expf(ms[b] - Mb);
        on = fmaf(f, os[b], on);
        ln = fmaf(f, ls[b], ln);
      }
      M = Mb;
    }
    gm[j][o] = M;
    gl[j][o] = ln;
    go[j][o] = on;
  }
  const bool any_failed = __syncthreads_or(failed);
  if (mine && j == 0 && t < G * D) {
    float Mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < kGrp; ++i) Mt = fmaxf(Mt, gm[i][o]);
    float on = 0.f, ln = 0.f;
#pragma unroll
    for (int i = 0; i < kGrp; ++i) {
      if (gm[i][o] == -INFINITY) continue;
      const float f = expf(gm[i][o] - Mt);
      on = fmaf(f, go[i][o], on);
      ln = fmaf(f, gl[i][o], ln);
    }
    a.out[(int64_t)(g * G) * D + t] = f32_to_bf16(on / ln);
  }
  if (threadIdx.x == 0) {
    if (any_failed) st_dev(a.ctl + kAttnErr, 1u);
    st_dev(ep, tag);
  }
}

template <int D, int G, int NP>
__global__ __launch_bounds__(kAttnWaves * 64) void k_attn_split(AttnArgs a) {
  constexpr int NCH = D / 64;    // 16-byte key chunks per lane and slot
  constexpr int VL = D / 4;      // lanes per value row (8 bytes each)
  constexpr int VR = 64 / VL;    // value rows per wave instruction
  constexpr int SPW = 8 * NP;    // slots per wave
  constexpr int NV = SPW / VR;   // value loads per lane
  constexpr int HALF = D / 2;
  __shared__ float qs[G][D];
  __shared__ float kcur[D], vcur[D];
  __shared__ float ow[kAttnWaves][G][D];
  __shared__ float mw[kAttnWaves][G], lw[kAttnWaves][G];
  __shared__ float scur[G];

  const int g = blockIdx.y, split = blockIdx.x;
  if (split >= a.nsplit) {
    attn_merge<D, G>(a, g, split - a.nsplit);
    return;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int s0 = (split * kAttnWaves + wave) * SPW;  // this wave's first slot
  const int64_t head = (int64_t)g * a.S;

  // 0. this thread's RoPE items (query planes of the group's heads, then,
  //    in split 0, the current key's) and value element, loaded before the
  //    cache rows so that waiting for them does not wait for the rows
  static_assert((G + 1) * HALF <= 2 * kAttnWaves * 64, "two RoPE items per thread");
  const int nrot = (G + (split == 0 ? 1 : 0)) * HALF;
  float rx[2][2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int t0 = threadIdx.x + r * kAttnWaves * 64;
    const int t = t0 < nrot ? t0 : 0;
    const int h = t / HALF, i = t - h * HALF;
    const float* x = h < G ? a.q + (int64_t)(g * G + h) * D : a.k + (int64_t)g * D;
    rx[r][0] = x[i];
    rx[r][1] = x[i + HALF];
  }
  const float vin = a.v[(int64_t)g * D + (threadIdx.x < D ? threadIdx.x : 0)];
  const uint32_t epoch = ld_dev(a.ctl + kAttnEpoch + g * kAttnMergers);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  // 1. every key and value load of the wave, before anything waits.  The
  //    loads are unconditional (a slot outside the range reads slot 0
  //    instead), so that no branch splits them; such a slot's score is
  //    masked and its value row zeroed.
  const int pk = lane >> 3, jk = lane & 7;
  uint4 kr[NP][NCH];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int slot = s0 + 8 * p + pk;
    const uint16_t* row = a.kc + (head + (slot < a.n_iter ? slot : 0)) * D;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      kr[p][c] = ldg16(reinterpret_cast<const uint8_t*>(row + 8 * (8 * c + jk)));
  }
  const int vrow = lane / VL, vcol = lane % VL;
  uint2 vr[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int slot = s0 + VR * i + vrow;
    vr[i] = ldg8(a.vc + (head + (slot < a.n_iter ? slot : 0)) * D + 4 * vcol);
  }

  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  // 2. RoPE of this group's queries (and, in split 0, of the current key),
  //    in fp64 while the loads are in flight
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int t = threadIdx.x + r * kAttnWaves * 64;
    if (t >= nrot) break;
    const int h = t / HALF, i = t - h * HALF;
    const double ang = (double)a.pos * exp2(-(2.0 * i / D) * a.log2_base);
    double sn, cs;
    sincos(ang, &sn, &cs);
    const double x0 = rx[r][0], x1 = rx[r][1];
    if (h < G) {
      qs[h][i] = (float)(x0 * cs - x1 * sn);
      qs[h][i + HALF] = (float)(x1 * cs + x0 * sn);
    } else {
      const uint16_t r0 = f64_to_f16_bits(x0 * cs - x1 * sn);
      const uint16_t r1 = f64_to_f16_bits(x1 * cs + x0 * sn);
      uint16_t* dst = a.kc + (head + a.cur) * D;
      dst[i] = r0;
      dst[i + HALF] = r1;
      kcur[i] = half_to_f32(r0);
      kcur[i + HALF] = half_to_f32(r1);
    }
  }
  if (split == 0 && threadIdx.x < D) {
    const uint16_t b = f64_to_f16_bits((double)vin);
    a.vc[(head + a.cur) * D + threadIdx.x] = b;
    vcur[threadIdx.x] = half_to_f32(b);
  }
  __syncthreads();
  if (split == 0 && wave < G) {
    float s = 0.f;
    for (int d = lane; d < D; d += 64) s = fmaf(qs[wave][d], kcur[d], s);
    s = wave_sum(s);
    if (lane == 0) scur[wave] = s * a.scale;
  }

  // 3. scores of the wave's slots
  float sc[NP][G];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const uint32_t w[4] = {kr[p][c].x, kr[p][c].y, kr[p][c].z, kr[p][c].w};
      float kf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[2 * e] = half_to_f32(w[e] & 0xffffu);
        kf[2 * e + 1] = half_to_f32(w[e] >> 16);
      }
      const int d0 = 8 * (8 * c + jk);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float4 qa = *reinterpret_cast<const float4*>(&qs[h][d0]);
        const float4 qb = *reinterpret_cast<const float4*>(&qs[h][d0 + 4]);
        float s = acc[h];
        s = fmaf(qa.x, kf[0], s);
        s = fmaf(qa.y, kf[1], s);
        s = fmaf(qa.z, kf[2], s);
        s = fmaf(qa.w, kf[3], s);
        s = fmaf(qb.x, kf[4], s);
        s = fmaf(qb.y, kf[5], s);
        s = fmaf(qb.z, kf[6], s);
        s = fmaf(qb.w, kf[7], s);
        acc[h] = s;
      }
    }
    const int slot = s0 + 8 * p + pk;
    const bool ok = slot < a.n_iter && slot != a.cur;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float s = acc[h];
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s += __shfl_xor(s, 4);
      sc[p][h] = ok ? s * a.scale : -INFINITY;
    }
  }

  // 4. the wave's max and probabilities (a lane with no valid slot: 0)
  float m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = sc[0][h];
#pragma unroll
    for (int p = 1; p < NP; ++p) mx = fmaxf(mx, sc[p][h]);
    m[h] = wave_max(mx);
    float sum = 0.f;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      sc[p][h] = sc[p][h] == -INFINITY ? 0.f : expf(sc[p][h] - m[h]);
      sum += sc[p][h];
    }
    l[h] = wave_sum(jk == 0 ? sum : 0.f);
  }

  // 5. probabilities times values
  float o[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) o[h][e] = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int slot = s0 + VR * i + vrow;
    const bool ok = slot < a.n_iter && slot != a.cur;
    const uint32_t vx = ok ? vr[i].x : 0u, vy = ok ? vr[i].y : 0u;
    float vf[4] = {half_to_f32(vx & 0xffffu), half_to_f32(vx >> 16), half_to_f32(vy & 0xffffu),
                   half_to_f32(vy >> 16)};
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float pr;
      if (VR == 1) {
        const int si = i;  // slot index in the wave: pass si / 8, lane 8 (si % 8)
        pr = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                            __builtin_bit_cast(int, sc[si / 8][h]), 8 * (si % 8)));
      } else {
        const int sa = VR * i, sb = VR * i + 1;
        const float pa = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc[sa / 8][h]), 8 * (sa % 8)));
        const float pb = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc[sb / 8][h]), 8 * (sb % 8)));
        pr = vrow ? pb : pa;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) o[h][e] = fmaf(pr, vf[e], o[h][e]);
    }
  }
  if (VR == 2) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[h][e] += __shfl_xor(o[h][e], 32);
  }
  if (lane < VL) {
#pragma unroll
    for (int h = 0; h < G; ++h)
      *reinterpret_cast<float4*>(&ow[wave][h][4 * vcol]) = make_float4(o[h][0], o[h][1], o[h][2], o[h][3]);
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mw[wave][h] = m[h];
      lw[wave][h] = l[h];
    }
  }
  __syncthreads();

  // 6. merge the waves (and the current token in split 0) into this
  //    split's (max, sum, unnormalised output) per head
  const uint32_t tag = epoch + 1u == 0u ? 1u : epoch + 1u;
  uint64_t* pp = a.part + ((int64_t)g * a.nsplit + split) * G * (D + 2);
  for (int t = threadIdx.x; t < G * D; t += kAttnWaves * 64) {
    const int h = t / D, d = t - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, mw[w][h]);
    if (split == 0) M = fmaxf(M, scur[h]);
    float on = 0.f, ln = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        if (mw[w][h] == -INFINITY) continue;
        const float f = expf(mw[w][h] - M);
        on = fmaf(f, ow[w][h][d], on);
        ln = fmaf(f, lw[w][h], ln);
      }
      if (split == 0) {
        const float f = expf(scur[h] - M);
        on = fmaf(f, vcur[d], on);
        ln += f;
      }
    }
    if (a.nsplit == 1) {
      a.out[(int64_t)(g * G + h) * D + d] = f32_to_bf16(on / ln);
    } else {
      // publish: every word carries this call's tag, so the merging blocks
      // need no flag and no wait for these stores to complete
      const uint64_t hi = (uint64_t)tag << 32;
      st_dev(pp + h * (D + 2) + d, (uint64_t)__float_as_uint(on) | hi);
      if (d == 0) {
        st_dev(pp + h * (D + 2) + D, (uint64_t)__float_as_uint(M) | hi);
        st_dev(pp + h * (D + 2) + D + 1, (uint64_t)__float_as_uint(ln) | hi);
      }
    }
  }
}

// Slots per wave pass group: the largest NP in {4, 2, 1} that still gives
// two split blocks per CU (measured: a 4,096-slot cache runs faster in 512
// blocks of 64 slots than in 256 of 128); 1 when none does.
static int attn_np(int n_iter, int Hkv) {
  for (int np = 4; np > 1; np /= 2)
    if ((int64_t)cdiv(n_iter, 32 * np) * Hkv >= 2 * kAttnCUs) return np;
  return 1;
}

bool attn_supported(int D, int G) {
  return (D == 128 && (G == 1 || G == 2 || G == 4)) || (D == 256 && (G == 1 || G == 2));
}

size_t attn_ws_bytes(int Hq, int Hkv, int D, int S) {
  return attn_ctl_bytes(Hkv) +
         (size_t)cdiv(S, 32) * (size_t)Hq * (size_t)(D + 2) * sizeof(uint64_t);
}

template <int D, int G>
static void launch_split(const AttnArgs& a, int np, int Hkv, hipStream_t st) {
  static_assert(G * D <= kAttnMergers * 64, "merging blocks cover the group's outputs");
  const dim3 grid(a.nsplit + (a.nsplit > 1 ? kAttnMergers : 0), Hkv), block(kAttnWaves * 64);
  if (np == 4)
    hipLaunchKernelGGL((k_attn_split<D, G, 4>), grid, block, 0, st, a);
  else if (np == 2)
    hipLaunchKernelGGL((k_attn_split<D, G, 2>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((k_attn_split<D, G, 1>), grid, block, 0, st, a);
}

qmoe_status launch_attn(const float* q, const float* k, const float* v, int Hq, int Hkv, int D,
                        int S, bool circular, int pos, float rope_base, float scale, uint16_t* kc,
                        uint16_t* vc, uint16_t* out, void* ws, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.kc = kc;
  a.vc = vc;
  a.out = out;
  a.ctl = reinterpret_cast<uint32_t*>(ws);
  a.part = reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(ws) + attn_ctl_bytes(Hkv));
  a.Hq = Hq;
  a.S = S;
  a.pos = pos;
  a.n_iter = pos + 1 < S ? pos + 1 : S;
  a.cur = circular ? pos % S : pos;
  const int np = attn_np(a.n_iter, Hkv);
  a.nsplit = cdiv(a.n_iter, 32 * np);
  a.scale = scale;
  a.log2_base = log2((double)rope_base);
  const int G = Hq / Hkv;
  if (D == 256) {
    if (G == 1) launch_split<256, 1>(a, np, Hkv, st);
    else launch_split<256, 2>(a, np, Hkv, st);
  } else {
    if (G == 1) launch_split<128, 1>(a, np, Hkv, st);
    else if (G == 2) launch_split<128, 2>(a, np, Hkv, st);
    else launch_split<128, 4>(a, np, Hkv, st);
  }
  return hipGetLastError() == hipSuccess ? QMOE_OK : QMOE_ERR_HIP;
}

}  // namespace qmoe
