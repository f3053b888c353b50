// qmoe_prefill.hip -- chunked prefill of up to 128 tokens on the matrix
// cores: the (token, rank) pairs of the chunk are grouped by expert so that
// one loaded copy of each expert serves all of its rows (devtrends.cc
// "Come eseguire un modello da 26 miliardi…", section "Prestazioni nel mondo
// reale"; remio.ai "TurboFieldfare esegue Mac Gemma 4 26B in 2 GB…", section
// "L'affermazione dei 2 GB…"; iitog.ru, technical paragraph).
//
// Launches (one stream):
//   dispatch  counts/offsets of the pairs per expert and their stable order
//             (expert, then token, then rank), from wave ballots
//   prep      X (bf16) -> fp16, each 8 columns in the order the weights are
//             unpacked in: (x0,x2,x4,x6,x1,x3,x5,x7)
//   gemm gu   per (expert, 64 output rows): A = gelu(X_e Wg^T) * (X_e Wu^T)
//             for the expert's rows; the shared expert over all T rows
//   gemm down per (expert, 64 output rows): Y_e = A_e Wd^T; shared likewise
//   combine   out[t] = bf16(Y_s[t] + sum_j w[t][j] Y[pos(t,j)] (+ residual))
//
// The GEMMs use v_mfma_f32_16x16x32_f16 with fp32 accumulation.  Weights are
// dequantized to fp16 in registers (codes through the fp8 conversion, then
// s*q + b with a packed fp16 FMA), so a K-slice may mix quantization groups
// and no per-group rescale of the accumulators is needed.  Activations and
// weights are fp16 (relative rounding 2^-11); inputs must be finite and below
// the fp16 range (65504) in magnitude.
#include "qmoe_common.h"

namespace qmoe {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int kPfRows = 64;   // weight rows (output features) per block
constexpr int kPfMaxM = 64;   // A rows (an expert's tokens) per pass of a block
constexpr int kPfMSub = kPfMaxM / 16;
constexpr int kPfMChunks = 2; // row chunks of one expert handled by separate blocks

struct PfLayout {
  size_t counts, offsets, perm, pos, xh, act, act_sh, y, y_sh, total;
};

__host__ __device__ inline PfLayout pf_layout(int E, int K, int I, int Is, int H, int T) {
  PfLayout L;
  size_t o = 0;
  L.counts = o; o += align256((size_t)E * 4);
  L.offsets = o; o += align256((size_t)(E + 1) * 4);
  L.perm = o; o += align256((size_t)T * K * 4);
  L.pos = o; o += align256((size_t)T * K * 4);
  L.xh = o; o += align256((size_t)T * H * 2);
  L.act = o; o += align256((size_t)T * K * I * 2);
  L.act_sh = o; o += align256((size_t)T * Is * 2);
  L.y = o; o += align256((size_t)T * K * H * 4);
  L.y_sh = o; o += align256((size_t)T * H * 4);
  L.total = o;
  return L;
}

size_t prefill_ws_bytes(const qmoe_moe_layer& L, int T) {
  return pf_layout(L.n_experts, L.top_k, L.inter, L.shared_inter, L.hidden, T).total;
}

// ============================================================== dispatch
// One block of 1024 threads, thread p = flat pair index t*K + j (n <= 1024).
// rank of p among the pairs of its expert = pairs of the same expert in
// earlier waves (per-wave counts, prefix over waves) + earlier lanes of its
// wave with the same expert (ballot match on the bits of the expert id).
__global__ __launch_bounds__(1024) void k_pf_dispatch(const int32_t* idx, int n, int E,
                                                      int32_t* counts, int32_t* offsets,
                                                      int32_t* perm, int32_t* pos_of) {
  __shared__ int32_t cnt[16][QMOE_MAX_EXPERTS];  // per-wave counts, then prefixes
  __shared__ int32_t off[QMOE_MAX_EXPERTS + 1];
  const int p = threadIdx.x, wave = p >> 6, lane = p & 63;
  for (int i = p; i < 16 * QMOE_MAX_EXPERTS; i += 1024) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const bool act = p < n;
  int e = act ? min(max(idx[p], 0), E - 1) : 0;
  uint64_t mask = __ballot(act);
  for (int b = 0; (1 << b) < E; ++b) {
    uint64_t bal = __ballot((e >> b) & 1);
    mask &= ((e >> b) & 1) ? bal : ~bal;
  }
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  const int rank = __popcll(mask & below);
  if (act && rank == 0) cnt[wave][e] = __popcll(mask);
  __syncthreads();
  // per expert: exclusive prefix over the 16 waves, total count
  for (int x = p; x < E; x += 1024) {
    int s = 0;
    for (int w = 0; w < 16; ++w) {
      int c = cnt[w][x];
      cnt[w][x] = s;
      s += c;
    }
    off[x + 1] = s;
    counts[x] = s;
  }
  if (p == 0) off[0] = 0;
  __syncthreads();
  // inclusive scan of off[1..E] (Hillis-Steele over up to 512 entries)
  for (int d = 1; d < E; d <<= 1) {
    int v = 0;
    if (p >= d && p < E) v = off[p + 1 - d];
    __syncthreads();
    if (p >= d && p < E) off[p + 1] += v;
    __syncthreads();
  }
  for (int x = p; x <= E; x += 1024) offsets[x] = off[x];
  if (act) {
    int pos = off[e] + cnt[wave][e] + rank;
    perm[pos] = p;
    pos_of[p] = pos;
  }
}

// ================================================================== prep
// X bf16 [T][H] -> fp16, columns of each 8 reordered (0,2,4,6,1,3,5,7).
__global__ __launch_bounds__(kBlock) void k_pf_prep(const uint16_t* X, int n8, _Float16* xh) {
  const int v = blockIdx.x * kBlock + threadIdx.x;
  if (v >= n8) return;
  uint4 r = reinterpret_cast<const uint4*>(X)[v];
  uint32_t w[4] = {r.x, r.y, r.z, r.w};
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(w[i] & 0xffffu);
    f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
  h8_t o;
  const int order[8] = {0, 2, 4, 6, 1, 3, 5, 7};
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (_Float16)f[order[i]];
  reinterpret_cast<h8_t*>(xh)[v] = o;
}

// ================================================================= GEMMs
// One block: 64 weight rows (wave w: rows n0 + 16w + l%16) of NM matrices
// against up to 128 rows of A (an expert's tokens), K in steps of 128
// codes.  Per step the block stages its A rows (fp16, prepared layout) in
// LDS once for all four waves, while every lane holds the next two steps
// of its weights in registers: lane (n = l%16, j = l/16) holds codes
// [128kb + 32j, +32) of its row as 4 words; word t feeds MFMA t (K slots
// 8j..8j+7), dequantized to fp16 in the order (q0,q2,q4,q6,q1,q3,q5,q7).
__device__ __forceinline__ h8_t dequant_word(uint32_t v, h2_t s2, h2_t b2) {
  const uint32_t lo = v & 0x0F0F0F0Fu, hi = (v >> 4) & 0x0F0F0F0Fu;
  h2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, false);  // q0, q2
  h2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, true);   // q4, q6
  h2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, false);  // q1, q3
  h2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, true);   // q5, q7
  // one rounding each (an explicit fused multiply-add, the same in every
  // instantiation)
  p0 = __builtin_elementwise_fma(p0, s2, b2);
  p1 = __builtin_elementwise_fma(p1, s2, b2);
  p2 = __builtin_elementwise_fma(p2, s2, b2);
  p3 = __builtin_elementwise_fma(p3, s2, b2);
  h8_t o;
  o[0] = p0.x; o[1] = p0.y; o[2] = p1.x; o[3] = p1.y;
  o[4] = p2.x; o[5] = p2.y; o[6] = p3.x; o[7] = p3.y;
  return o;
}

struct PfArgs {
  int T, K, E, H, I, Is;
  DevQ gate, up, down, shg, shu, shd;
  const int32_t* slot;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* perm;
  const _Float16* xh;   // [T][H] prepared input
  _Float16* act;        // [T*K][I] routed activations (sorted order, prepared layout)
  _Float16* act_sh;     // [T][Is]
  float* y;             // [T*K][H] routed outputs (sorted order)
  float* y_sh;          // [T][H]
};

constexpr int kPfAStride = 136;  // fp16 per staged A row: 128 + 8 (conflict-free reads)

typedef unsigned int u4v_t __attribute__((ext_vector_type(4)));

struct PfShared {
  _Float16 a[2][kPfMaxM * kPfAStride];  // A rows of two K-steps (double buffer)
  int32_t rows[kPfMaxM];  // element offset of each A row from the A base
};

template <int NM>
struct PfW {
  u4v_t q[NM];
  uint32_t sb[NM];
};

// Weights of step kb (clamped to a valid address past the end).
template <int NM>
__device__ __forceinline__ void pf_load_w(PfW<NM>& B, const DevQ (&W)[NM], int n_row, int K,
                                          int kb) {
  const int j = (threadIdx.x & 63) >> 4;
  const int c = min(128 * kb + 32 * j, K - 32);
  const int G = K / 64;
#pragma unroll
  for (int k = 0; k < NM; ++k) {
    // cached loads: a step reads half of each 128-byte line, the next step
    // the other half
    B.q[k] = *reinterpret_cast<const u4v_t*>(W[k].q + (int64_t)n_row * (K / 2) + c / 2);
    B.sb[k] = (uint32_t)W[k].s[(int64_t)n_row * G + c / 64] |
              ((uint32_t)W[k].b[(int64_t)n_row * G + c / 64] << 16);
  }
}

// A rows of step kb: thread (r0 = tid/16, seg = tid%16) loads 16 bytes of
// rows r0 + 16i, i < NMS.  Rows past Mc re-read row Mc-1 (zeroed at store).
template <int NMS>
struct PfA {
  u4v_t v[NMS];
};
template <int NMS>
__device__ __forceinline__ void pf_load_a(PfA<NMS>& A, const _Float16* abase, const PfShared& sh,
                                          int Mc, int K, int kb) {
  const int seg = threadIdx.x & 15, r0 = threadIdx.x >> 4;
  const int col = min(128 * kb + 8 * seg, K - 8);
#pragma unroll
  for (int i = 0; i < NMS; ++i)
    A.v[i] = *reinterpret_cast<const u4v_t*>(abase + sh.rows[min(r0 + 16 * i, Mc - 1)] + col);
}
template <int NMS>
__device__ __forceinline__ void pf_store_a(const PfA<NMS>& A, _Float16* buf, int Mc, int K, int kb) {
  const int seg = threadIdx.x & 15, r0 = threadIdx.x >> 4;
  const bool colok = 128 * kb + 8 * seg < K;
#pragma unroll
  for (int i = 0; i < NMS; ++i) {
    const int m = r0 + 16 * i;
    const u4v_t z = {0u, 0u, 0u, 0u};
    *reinterpret_cast<u4v_t*>(buf + m * kPfAStride + 8 * seg) = (colok && m < Mc) ? A.v[i] : z;
  }
}

template <int NM, int NMS>
__device__ __forceinline__ void pf_mma(const PfW<NM>& B, int K, int kb, const _Float16* buf,
                                       f4_t (&acc)[NMS][NM]) {
  const int lane = threadIdx.x & 63, m = lane & 15, j = lane >> 4;
  const bool kok = 128 * kb + 32 * j < K;
  h8_t Bf[NM][4];
#pragma unroll
  for (int k = 0; k < NM; ++k) {
    _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)(B.sb[k] & 0xffffu));
    _Float16 bv = __builtin_bit_cast(_Float16, (uint16_t)(B.sb[k] >> 16));
    if (!kok) sv = bv = (_Float16)0.f;
    const h2_t s2 = {sv, sv}, b2 = {bv, bv};
    const u4v_t z = {0u, 0u, 0u, 0u};
    const u4v_t q = kok ? B.q[k] : z;
    Bf[k][0] = dequant_word(q.x, s2, b2);
    Bf[k][1] = dequant_word(q.y, s2, b2);
    Bf[k][2] = dequant_word(q.z, s2, b2);
    Bf[k][3] = dequant_word(q.w, s2, b2);
  }
#pragma unroll
  for (int ms = 0; ms < NMS; ++ms) {
    const h8_t* ap = reinterpret_cast<const h8_t*>(buf + (ms * 16 + m) * kPfAStride + 32 * j);
    const h8_t A0 = ap[0], A1 = ap[1], A2 = ap[2], A3 = ap[3];
#pragma unroll
    for (int k = 0; k < NM; ++k) {
      acc[ms][k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, Bf[k][0], acc[ms][k], 0, 0, 0);
      acc[ms][k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, Bf[k][1], acc[ms][k], 0, 0, 0);
      acc[ms][k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A2, Bf[k][2], acc[ms][k], 0, 0, 0);
      acc[ms][k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A3, Bf[k][3], acc[ms][k], 0, 0, 0);
    }
    // keep each subtile's fragment reads next to its MFMAs (bounded registers)
    __builtin_amdgcn_sched_barrier(0);
  }
}

// C = A W^T over one pass of Mc <= 64 A rows (sh.rows[0..Mc) set), K
// columns; acc[ms][k]: lane l holds rows 16ms + 4(l/16) + r, column l%16.
// Weights run two steps ahead in registers; A rows are loaded two steps
// ahead into registers (two alternating sets) and stored to the LDS buffer
// of the next step (two alternating buffers, one barrier per step).
template <int NM, int NMS>
__device__ __forceinline__ void pf_pass(const DevQ (&W)[NM], int n_row, int K, int Mc,
                                        const _Float16* abase, PfShared& sh,
                                        f4_t (&acc)[NMS][NM]) {
#pragma unroll
  for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
    for (int k = 0; k < NM; ++k) acc[ms][k] = f4_t{0.f, 0.f, 0.f, 0.f};
  const int nkb = (K + 127) / 128;
  PfW<NM> B0, B1;
  PfA<NMS> Aa, Ab;
  pf_load_w<NM>(B0, W, n_row, K, 0);
  pf_load_a<NMS>(Aa, abase, sh, Mc, K, 0);
  pf_load_w<NM>(B1, W, n_row, K, 1);
  pf_load_a<NMS>(Ab, abase, sh, Mc, K, min(1, nkb - 1));
  pf_store_a<NMS>(Aa, sh.a[0], Mc, K, 0);
  __syncthreads();
  for (int kb = 0; kb < nkb; kb += 2) {
    // step kb: buffer 0 holds A(kb); Ab holds A(kb + 1)
    pf_load_a<NMS>(Aa, abase, sh, Mc, K, min(kb + 2, nkb - 1));
    pf_mma<NM, NMS>(B0, K, kb, sh.a[0], acc);
    pf_load_w<NM>(B0, W, n_row, K, kb + 2);
    if (kb + 1 >= nkb) break;
    pf_store_a<NMS>(Ab, sh.a[1], Mc, K, kb + 1);
    __syncthreads();
    // step kb + 1: buffer 1 holds A(kb + 1); Aa holds A(kb + 2)
    pf_load_a<NMS>(Ab, abase, sh, Mc, K, min(kb + 3, nkb - 1));
    pf_mma<NM, NMS>(B1, K, kb + 1, sh.a[1], acc);
    pf_load_w<NM>(B1, W, n_row, K, kb + 3);
    if (kb + 2 >= nkb) break;
    pf_store_a<NMS>(Aa, sh.a[0], Mc, K, kb + 2);
    __syncthreads();
  }
  __syncthreads();  // the LDS is free for the next pass
}

// Column position of output feature n inside its group of 8 in the prepared
// layout (0,2,4,6,1,3,5,7).
__device__ __forceinline__ int prep_col(int n) {
  const int v = n & 7;
  return (n & ~7) | ((v & 1) ? 4 + (v >> 1) : (v >> 1));
}

template <int NMS>
__device__ __forceinline__ void pf_gu_store(const f4_t (&acc)[NMS][2], _Float16* out, int ld, int base, int Mc,
                            int n) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = ms * 16 + 4 * (lane >> 4) + r;
      if (m < Mc) {
        float v = gelu_tanh(acc[ms][0][r]) * acc[ms][1][r];
        // the product is rounded to fp32, then to fp16, in every copy of
        // this code (the backend would otherwise fuse the multiply with the
        // conversion in some copies only: other bits, other signs of zero)
        asm volatile("" : "+v"(v));
        out[(size_t)(base + m) * ld + prep_col(n)] = (_Float16)v;
      }
    }
}
template <int NMS>
__device__ __forceinline__ void pf_down_store(const f4_t (&acc)[NMS][1], float* out, int ld, int base, int Mc,
                              int n) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = ms * 16 + 4 * (lane >> 4) + r;
      if (m < Mc) out[(size_t)(base + m) * ld + n] = acc[ms][0][r];
    }
}

// gate/up: grid (tiles of 64 rows over max(I, Is), E + 1, kPfMChunks);
// y = 0: the shared expert (largest, started first), y = e + 1: expert e;
// z: which 64-row chunks of the expert's rows (z, z + gridDim.z, ...), so
// that the chunks of the shared and the busiest experts run side by side.
__global__ __launch_bounds__(kBlock, 2) void k_pf_gu(PfArgs a) {
  __shared__ PfShared sh;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool shared = blockIdx.y == 0;
  const int e = blockIdx.y - 1;
  const int N = shared ? a.Is : a.I;
  const int n0 = blockIdx.x * kPfRows;
  if (n0 >= N) return;
  const int M = shared ? a.T : a.counts[e];
  const int base = shared ? 0 : a.offsets[e];
  DevQ W[2];
  if (shared) {
    W[0] = a.shg;
    W[1] = a.shu;
  } else {
    int s = a.slot ? a.slot[e] : e;
    W[0] = devq_at(a.gate, s);
    W[1] = devq_at(a.up, s);
  }
  const int n = n0 + 16 * wave + (lane & 15);  // N is a multiple of 64
  _Float16* out = shared ? a.act_sh : a.act;
  const int ld = shared ? a.Is : a.I;
  for (int mc = blockIdx.z * kPfMaxM; mc < M; mc += gridDim.z * kPfMaxM) {
    const int Mc = min(M - mc, kPfMaxM);
    __syncthreads();
    for (int m = threadIdx.x; m < Mc; m += kBlock) {
      int t = shared ? mc + m : a.perm[base + mc + m] / a.K;
      sh.rows[m] = t * a.H;
    }
    __syncthreads();
    if (Mc <= 16) {
      f4_t acc[1][2];
      pf_pass<2, 1>(W, n, a.H, Mc, a.xh, sh, acc);
      pf_gu_store<1>(acc, out, ld, base + mc, Mc, n);
    } else if (Mc <= 32) {
      f4_t acc[2][2];
      pf_pass<2, 2>(W, n, a.H, Mc, a.xh, sh, acc);
      pf_gu_store<2>(acc, out, ld, base + mc, Mc, n);
    } else {
      f4_t acc[4][2];
      pf_pass<2, 4>(W, n, a.H, Mc, a.xh, sh, acc);
      pf_gu_store<4>(acc, out, ld, base + mc, Mc, n);
    }
  }
}

// down: grid (tiles of 64 rows over H, E + 1, kPfMChunks); y and z as for
// gate/up.
__global__ __launch_bounds__(kBlock, 3) void k_pf_down(PfArgs a) {
  __shared__ PfShared sh;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool shared = blockIdx.y == 0;
  const int e = blockIdx.y - 1;
  const int n0 = blockIdx.x * kPfRows;
  const int M = shared ? a.T : a.counts[e];
  const int base = shared ? 0 : a.offsets[e];
  const int Kd = shared ? a.Is : a.I;
  const _Float16* src = shared ? a.act_sh : a.act;
  DevQ W[1];
  if (shared) {
    W[0] = a.shd;
  } else {
    int s = a.slot ? a.slot[e] : e;
    W[0] = devq_at(a.down, s);
  }
  const int n = n0 + 16 * wave + (lane & 15);  // H is a multiple of 64
  float* out = shared ? a.y_sh : a.y;
  for (int mc = blockIdx.z * kPfMaxM; mc < M; mc += gridDim.z * kPfMaxM) {
    const int Mc = min(M - mc, kPfMaxM);
    __syncthreads();
    for (int m = threadIdx.x; m < Mc; m += kBlock) sh.rows[m] = (base + mc + m) * Kd;
    __syncthreads();
    if (Mc <= 16) {
      f4_t acc[1][1];
      pf_pass<1, 1>(W, n, Kd, Mc, src, sh, acc);
      pf_down_store<1>(acc, out, a.H, base + mc, Mc, n);
    } else if (Mc <= 32) {
      f4_t acc[2][1];
      pf_pass<1, 2>(W, n, Kd, Mc, src, sh, acc);
      pf_down_store<2>(acc, out, a.H, base + mc, Mc, n);
    } else {
      f4_t acc[4][1];
      pf_pass<1, 4>(W, n, Kd, Mc, src, sh, acc);
      pf_down_store<4>(acc, out, a.H, base + mc, Mc, n);
    }
  }
}

// ================================================================ combine
// out[t][h] = bf16(y_sh[t][h] + sum_j w[t][j] * y[pos(t,j)][h] (+ res)),
// ranks j in order.  grid (T, H/(8*kBlock) rounded up); 8 columns/thread.
__global__ __launch_bounds__(kBlock) void k_pf_combine(int K, int H, const float* w,
                                                       const int32_t* pos_of, const float* y,
                                                       const float* y_sh, const uint16_t* res,
                                                       uint16_t* out) {
  const int t = blockIdx.y;
  const int h = (blockIdx.x * kBlock + threadIdx.x) * 8;
  if (h >= H) return;
  float acc[8];
  const float4* ys = reinterpret_cast<const float4*>(y_sh + (size_t)t * H + h);
  float4 a0 = ys[0], a1 = ys[1];
  acc[0] = a0.x; acc[1] = a0.y; acc[2] = a0.z; acc[3] = a0.w;
  acc[4] = a1.x; acc[5] = a1.y; acc[6] = a1.z; acc[7] = a1.w;
  for (int j = 0; j < K; ++j) {
    const float wj = w[t * K + j];
    const float4* yr = reinterpret_cast<const float4*>(y + (size_t)pos_of[t * K + j] * H + h);
    float4 b0 = yr[0], b1 = yr[1];
    acc[0] = fmaf(wj, b0.x, acc[0]); acc[1] = fmaf(wj, b0.y, acc[1]);
    acc[2] = fmaf(wj, b0.z, acc[2]); acc[3] = fmaf(wj, b0.w, acc[3]);
    acc[4] = fmaf(wj, b1.x, acc[4]); acc[5] = fmaf(wj, b1.y, acc[5]);
    acc[6] = fmaf(wj, b1.z, acc[6]); acc[7] = fmaf(wj, b1.w, acc[7]);
  }
  uint32_t o[4];
  if (res) {
    uint4 rr = *reinterpret_cast<const uint4*>(res + (size_t)t * H + h);
    uint32_t rw[4] = {rr.x, rr.y, rr.z, rr.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16_to_f32(rw[i] & 0xffffu);
      acc[2 * i + 1] += bf16_to_f32(rw[i] >> 16);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = (uint32_t)f32_to_bf16(acc[2 * i]) | ((uint32_t)f32_to_bf16(acc[2 * i + 1]) << 16);
  *reinterpret_cast<uint4*>(out + (size_t)t * H + h) = make_uint4(o[0], o[1], o[2], o[3]);
}

// ========================================================== host launcher
static hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

qmoe_status launch_prefill(const qmoe_moe_layer& L, const uint16_t* X, int T, const int32_t* idx,
                           const float* w, const uint16_t* residual, uint16_t* out, uint8_t* ws,
                           void* stream) {
  const int E = L.n_experts, K = L.top_k, H = L.hidden, I = L.inter, Is = L.shared_inter;
  if (T * K > 1024 || I % 64 || Is % 64) return QMOE_ERR_UNSUPPORTED;
  WsLayout wl = ws_layout(E, K, I, Is, T);
  uint8_t* pf = ws + wl.pf;
  PfLayout pl = pf_layout(E, K, I, Is, H, T);
  PfArgs a;
  a.T = T; a.K = K; a.E = E; a.H = H; a.I = I; a.Is = Is;
  a.gate = devq(L.gate); a.up = devq(L.up); a.down = devq(L.down);
  a.shg = devq(L.sh_gate); a.shu = devq(L.sh_up); a.shd = devq(L.sh_down);
  a.slot = nullptr;
  a.counts = reinterpret_cast<int32_t*>(pf + pl.counts);
  a.offsets = reinterpret_cast<int32_t*>(pf + pl.offsets);
  a.perm = reinterpret_cast<int32_t*>(pf + pl.perm);
  a.xh = reinterpret_cast<_Float16*>(pf + pl.xh);
  a.act = reinterpret_cast<_Float16*>(pf + pl.act);
  a.act_sh = reinterpret_cast<_Float16*>(pf + pl.act_sh);
  a.y = reinterpret_cast<float*>(pf + pl.y);
  a.y_sh = reinterpret_cast<float*>(pf + pl.y_sh);
  int32_t* pos_of = reinterpret_cast<int32_t*>(pf + pl.pos);
  hipLaunchKernelGGL(k_pf_dispatch, dim3(1), dim3(1024), 0, S(stream), idx, T * K, E,
                     const_cast<int32_t*>(a.counts), const_cast<int32_t*>(a.offsets),
                     const_cast<int32_t*>(a.perm), pos_of);
  const int n8 = T * H / 8;
  hipLaunchKernelGGL(k_pf_prep, dim3((n8 + kBlock - 1) / kBlock), dim3(kBlock), 0, S(stream), X, n8,
                     const_cast<_Float16*>(a.xh));
  const int ngu = ((I > Is ? I : Is) + kPfRows - 1) / kPfRows;
  hipLaunchKernelGGL(k_pf_gu, dim3(ngu, E + 1, kPfMChunks), dim3(kBlock), 0, S(stream), a);
  hipLaunchKernelGGL(k_pf_down, dim3(H / kPfRows, E + 1, kPfMChunks), dim3(kBlock), 0, S(stream), a);
  hipLaunchKernelGGL(k_pf_combine, dim3((H / 8 + kBlock - 1) / kBlock, T), dim3(kBlock), 0,
                     S(stream), K, H, w, pos_of, a.y, a.y_sh, residual, out);
  return hipGetLastError() == hipSuccess ? QMOE_OK : QMOE_ERR_HIP;
}

// Byte offsets, inside a workspace, of the dispatch arrays written by the
// last prefill call on it.
void prefill_dispatch_offsets(const qmoe_moe_layer& L, int T, size_t* counts, size_t* offsets,
                              size_t* perm) {
  WsLayout wl = ws_layout(L.n_experts, L.top_k, L.inter, L.shared_inter, T);
  PfLayout pl = pf_layout(L.n_experts, L.top_k, L.inter, L.shared_inter, L.hidden, T);
  *counts = wl.pf + pl.counts;
  *offsets = wl.pf + pl.offsets;
  *perm = wl.pf + pl.perm;
}

}  // namespace qmoe
