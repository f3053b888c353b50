// qmoe_prefill.hip -- chunked prefill of up to 128 tokens on the matrix
// cores: the (token, rank) pairs of the chunk are grouped by expert so that
// one loaded copy of each expert serves all of its rows (devtrends.cc
// "Come eseguire un modello da 26 miliardi…", section "Prestazioni nel mondo
// reale"; remio.ai "TurboFieldfare esegue Mac Gemma 4 26B in 2 GB…", section
// "L'affermazione dei 2 GB…"; iitog.ru, technical paragraph).
//
// Launches (one stream):
//   dispatch  counts/offsets of the pairs per expert and their stable order
//             (expert, then token, then rank), from wave ballots; the work
//             list of the GEMMs: items of at most 64 rows of one expert
//             (the shared expert's first, then the experts' by decreasing
//             row count)
//   prep      X (bf16) -> fp16, each 8 columns in the order the weights are
//             unpacked in: (x0,x2,x4,x6,x1,x3,x5,x7), rows padded with zeros
//             to a multiple of 128 columns
//   gemm gu   per (item, 64 output rows): A = gelu(X_e Wg^T) * (X_e Wu^T)
//             for the item's rows
//   gemm down per (item, 64 output rows): Y_e = A_e Wd^T
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

// A operands (the fp16 input and the activations) are stored with rows
// padded to a multiple of 128 columns, the padding zero, so that every
// K-step of 128 columns reads whole rows and needs no masking.
__host__ __device__ constexpr int pad128(int n) { return (n + 127) & ~127; }

struct PfLayout {
  size_t counts, offsets, perm, pos, items, xh, act, act_sh, y, y_sh, total;
};

// Work items of the GEMMs: chunks of at most kPfMaxM A rows of one expert
// (or of the shared expert).  An upper bound on their number, from the
// shapes alone: the shared expert's chunks, plus per expert with rows one
// partial chunk, plus the full chunks of all pairs.
__host__ __device__ inline int pf_max_items(int E, int K, int T) {
  const int n = T * K;
  return (T + kPfMaxM - 1) / kPfMaxM + (E < n ? E : n) + n / kPfMaxM;
}

__host__ __device__ inline PfLayout pf_layout(int E, int K, int I, int Is, int H, int T) {
  PfLayout L;
  size_t o = 0;
  L.counts = o; o += align256((size_t)E * 4);
  L.offsets = o; o += align256((size_t)(E + 1) * 4);
  L.perm = o; o += align256((size_t)T * K * 4);
  L.pos = o; o += align256((size_t)T * K * 4);
  L.items = o; o += align256((size_t)(1 + 3 * pf_max_items(E, K, T)) * 4);
  L.xh = o; o += align256((size_t)T * pad128(H) * 2);
  L.act = o; o += align256((size_t)T * K * pad128(I) * 2);
  L.act_sh = o; o += align256((size_t)T * pad128(Is) * 2);
  L.y = o; o += align256((size_t)T * K * H * 4);
  L.y_sh = o; o += align256((size_t)T * H * 4);
  L.total = o;
  return L;
}

size_t prefill_ws_bytes(const qmoe_moe_layer& L, int T) {
  return pf_layout(L.n_experts, L.top_k, L.inter, L.shared_inter, L.hidden, T).total;
}

// ================================================================== prep
// X bf16 [T][H] -> fp16 [T][pad128(H)], columns of each 8 reordered
// (0,2,4,6,1,3,5,7), the padding zero.  Word v: 8 columns.
__device__ __forceinline__ void pf_prep_word(const uint16_t* X, int T, int H, _Float16* xh, int v) {
  const int H8 = H / 8, P8 = pad128(H) / 8;
  const int t = v / P8, c8 = v - t * P8;
  h8_t o;
  if (c8 < H8) {
    uint4 r = reinterpret_cast<const uint4*>(X)[t * H8 + c8];
    uint32_t w[4] = {r.x, r.y, r.z, r.w};
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_to_f32(w[i] & 0xffffu);
      f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
    const int order[8] = {0, 2, 4, 6, 1, 3, 5, 7};
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (_Float16)f[order[i]];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (_Float16)0.f;
  }
  reinterpret_cast<h8_t*>(xh)[v] = o;
}

// ============================================================== dispatch
// Block 0 (1024 threads): thread p = flat pair index t*K + j (n <= 1024).
// rank of p among the pairs of its expert = pairs of the same expert in
// earlier waves (per-wave counts, prefix over waves) + earlier lanes of its
// wave with the same expert (ballot match on the bits of the expert id).
//
// It also writes the GEMMs' work list, items = [n_items | n_pairs << 16,
// (e, row0, M)...]:
// first the shared expert's chunks of kPfMaxM token rows (e = -1, row0 =
// first token), then the experts' chunks of kPfMaxM pair rows (row0 = first
// sorted pair), experts in order of decreasing row count (ties: lower id
// first), so that the longest blocks start first.
// Blocks 1.. of the same launch prepare the A rows (independent work: the
// chunk saves a launch).
__global__ __launch_bounds__(1024) void k_pf_dispatch(const int32_t* idx, int n, int T, int E,
                                                      int32_t* counts, int32_t* offsets,
                                                      int32_t* perm, int32_t* pos_of,
                                                      int32_t* items, const uint16_t* X, int H,
                                                      _Float16* xh) {
  if (blockIdx.x > 0) {
    const int v = (blockIdx.x - 1) * 1024 + threadIdx.x;
    if (v < T * (pad128(H) / 8)) pf_prep_word(X, T, H, xh, v);
    return;
  }
  __shared__ int32_t cnt[16][QMOE_MAX_EXPERTS];  // per-wave counts, then prefixes
  __shared__ int32_t off[QMOE_MAX_EXPERTS + 1];
  __shared__ int32_t tot[QMOE_MAX_EXPERTS];      // rows per expert
  __shared__ int32_t ist[QMOE_MAX_EXPERTS + 1];  // chunks per rank, then first item per rank
  __shared__ int32_t npair;                       // experts with two chunks
  __shared__ int32_t rk[QMOE_MAX_EXPERTS];        // rank of each expert
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
    tot[x] = s;
    counts[x] = s;
  }
  if (p == 0) off[0] = 0;
  __syncthreads();
  // experts by decreasing count: the rank of expert x, summed over `per`
  // threads (each counts the experts y = part, part + per, ... that come
  // before x), and its chunks at that rank
  if (p == 0) npair = 0;
  __syncthreads();
  {
    const int per = E <= 128 ? 8 : (E <= 256 ? 4 : 2);
    const int x = p / per, part = p - x * per;
    int r = 0;
    if (x < E) {
      const int cx = tot[x];
      for (int y = part; y < E; y += per) {
        const int cy = tot[y];
        r += (cy > cx) || (cy == cx && y < x);
      }
    }
    for (int o = 1; o < per; o <<= 1) r += __shfl_xor(r, o);
    if (x < E && part == 0) {
      rk[x] = r;
      ist[r + 1] = (tot[x] + kPfMaxM - 1) / kPfMaxM;
      if (tot[x] > kPfMaxM) atomicAdd(&npair, 1);
    }
  }
  if (p == 0) ist[0] = 0;
  __syncthreads();
  // inclusive scans of off[1..E] (wave 0) and ist[1..E] (wave 1): each lane
  // sums a run of up to 8 consecutive entries, the runs' sums are scanned
  // across the wave by shuffles, and each lane adds its prefix back
  if (wave < 2) {
    int32_t* arr = (wave == 0 ? off : ist) + 1;
    const int run = (E + 63) / 64;
    const int j0 = lane * run;
    int loc[8];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      loc[i] = (i < run && j0 + i < E) ? arr[j0 + i] : 0;
      sum += loc[i];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    int acc = incl - sum;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc += loc[i];
      if (i < run && j0 + i < E) arr[j0 + i] = acc;
    }
  }
  __syncthreads();
  for (int x = p; x <= E; x += 1024) offsets[x] = off[x];
  if (act) {
    int pos = off[e] + cnt[wave][e] + rank;
    perm[pos] = p;
    pos_of[p] = pos;
  }
  // the work list
  const int nsh = (T + kPfMaxM - 1) / kPfMaxM;
  if (p < nsh) {
    items[1 + 3 * p] = -1;
    items[2 + 3 * p] = p * kPfMaxM;
    items[3 + 3 * p] = min(T - p * kPfMaxM, kPfMaxM);
  }
  if (p < E) {
    const int cx = tot[p];
    for (int c = 0; c * kPfMaxM < cx; ++c) {
      const int it = nsh + ist[rk[p]] + c;
      items[1 + 3 * it] = p;
      items[2 + 3 * it] = off[p] + c * kPfMaxM;
      items[3 + 3 * it] = min(cx - c * kPfMaxM, kPfMaxM);
    }
  }
  // the item count, and in bits 16.. the experts with two chunks (they
  // lead the experts' items: the GEMMs pair their chunks' tiles)
  if (p == 0) items[0] = (nsh + ist[E]) | (npair << 16);
}

// ================================================================= GEMMs
// One block: 64 weight rows (wave w: rows n0 + 16w + l%16) of NM matrices
// against up to 64 rows of A (an item: one expert's tokens), K in steps of
// 128 codes.  Per step the block stages its A rows (fp16, prepared layout)
// in LDS once for all four waves; lane (n = l%16, j = l/16) of a wave loads
// codes [128kb + 32j, +32) of its weight row straight into registers as 4
// words (the four lanes j of a row read 64 contiguous bytes, and the two
// steps of a pair the row's whole 128-byte line); word t feeds MFMA t (K
// slots 8j..8j+7), dequantized to fp16 in the order (q0,q2,q4,q6,q1,q3,q5,q7).
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
  const int32_t* perm;   // sorted pair -> flat pair index t*K + j
  const int32_t* items;  // [n_items | n_pairs << 16, (e, row0, M) ...] (the dispatch's work list)
  const _Float16* xh;   // [T][pad128(H)] prepared input
  _Float16* act;        // [T*K][pad128(I)] routed activations (sorted order, prepared layout)
  _Float16* act_sh;     // [T][pad128(Is)]
  float* y;             // [T*K][H] routed outputs (sorted order)
  float* y_sh;          // [T][H]
};

constexpr int kPfAStride = 136;  // fp16 per staged A row: 128 + 8 (conflict-free reads)

typedef unsigned int u4v_t __attribute__((ext_vector_type(4)));

constexpr int kPfWaves = kBlock / 64;

// LDS of a block: the A rows of two K-steps (double buffer), the A row
// offsets, and with SB, per wave and matrix the scales and biases of the
// wave's 16 rows over all K/64 groups: [16][G] scales, then [16][G] biases,
// filled once per pass (whole 64-lane writes of 16 bytes: 1536 halves for
// G <= 48).
constexpr int kPfSbMaxG = 48;
constexpr int kPfSbHalves = 1536;
template <int NM, bool SB>
struct PfShared {
  _Float16 a[2][kPfMaxM * kPfAStride];
  int32_t rows[kPfMaxM];  // element offset of each A row from the A base
  uint16_t sb[kPfWaves][NM][SB ? kPfSbHalves : 1];
};

// Codes of one pair of K-steps (2p, 2p + 1) for this lane, in the layout
// the MFMAs take: v[k][h] = codes [128 (2p + h) + 32 j, +32) of row n of
// matrix k (16 bytes).  Past the end of a row the last chunk is re-read:
// finite values whose products meet zero A columns.
template <int NM>
struct PfWG {
  u4v_t v[NM][2];
};
struct PfGOff {
  uint32_t row;   // byte offset of the lane's row
  uint32_t j16;   // 16 j: the lane's bytes within a step
  uint32_t qmax;  // last 16-byte chunk of a row: K/2 - 16
};
__device__ __forceinline__ PfGOff pf_goff(int n_wave0, int K) {
  const int lane = threadIdx.x & 63;
  PfGOff o;
  o.row = (uint32_t)(n_wave0 + (lane & 15)) * (uint32_t)(K / 2);
  o.j16 = 16u * (uint32_t)(lane >> 4);
  o.qmax = (uint32_t)(K / 2 - 16);
  return o;
}
template <int NM>
__device__ __forceinline__ void pf_load_wg(PfWG<NM>& G, const DevQ (&W)[NM], const PfGOff& o,
                                           int p) {
  const uint32_t o0 = min(128u * (uint32_t)p + o.j16, o.qmax);
  const uint32_t o1 = min(128u * (uint32_t)p + 64u + o.j16, o.qmax);
#pragma unroll
  for (int k = 0; k < NM; ++k) {
    G.v[k][0] = *reinterpret_cast<const u4v_t*>(W[k].q + (o.row + o0));
    G.v[k][1] = *reinterpret_cast<const u4v_t*>(W[k].q + (o.row + o1));
  }
}

// Scale and bias of the group of a lane's codes in step kb, as loaded
// (combined only where they are used, so that no instruction needs a load
// right after issuing it).  Lane (n = l%16, j = l/16) takes codes
// [128 kb + 32 j, +32) of row n in step kb.
template <int NM>
struct PfSB {
  uint32_t s[NM], b[NM];  // fp16 bits, zero-extended
};
struct PfSOff {
  uint32_t srow;  // element offset of the row's scales and biases
  uint32_t j16;   // 16 j: the lane's bytes within a step
  uint32_t qmax;  // K/2 - 16
};
__device__ __forceinline__ PfSOff pf_soff(int n_row, int K) {
  PfSOff o;
  o.srow = (uint32_t)n_row * (uint32_t)(K / 64);
  o.j16 = 16u * (uint32_t)((threadIdx.x & 63) >> 4);
  o.qmax = (uint32_t)(K / 2 - 16);
  return o;
}
template <int NM>
__device__ __forceinline__ void pf_load_sb(PfSB<NM>& B, const DevQ (&W)[NM], const PfSOff& o,
                                           int kb) {
  const uint32_t so = o.srow + (min(64u * (uint32_t)kb + o.j16, o.qmax) >> 5);
#pragma unroll
  for (int k = 0; k < NM; ++k) {
    B.s[k] = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(W[k].s) + 2u * so);
    B.b[k] = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(W[k].b) + 2u * so);
  }
}

// A rows of step kb: thread (r0 = tid/16, seg = tid%16) loads 16 bytes of
// rows r0 + 16i, i < NMS.  Rows past Mc re-read row Mc - 1: they only feed
// output rows that are not stored.
template <int NMS>
struct PfA {
  u4v_t v[NMS];
};
// Byte offsets (from the A base) of this thread's A rows, read from
// sh.rows once per pass.
template <int NMS, int NM, bool SB>
__device__ __forceinline__ void pf_rows(uint32_t (&roff)[NMS], const PfShared<NM, SB>& sh, int Mc) {
  const int r0 = threadIdx.x >> 4;
#pragma unroll
  for (int i = 0; i < NMS; ++i) roff[i] = 2u * (uint32_t)sh.rows[min(r0 + 16 * i, Mc - 1)];
}
template <int NMS>
__device__ __forceinline__ void pf_load_a(PfA<NMS>& A, const _Float16* abase,
                                          const uint32_t (&roff)[NMS], int kb) {
  const int seg = threadIdx.x & 15;
  const uint32_t col = 2u * (uint32_t)(128 * kb + 8 * seg);
  const uint8_t* ab = reinterpret_cast<const uint8_t*>(abase);
#pragma unroll
  for (int i = 0; i < NMS; ++i) A.v[i] = *reinterpret_cast<const u4v_t*>(ab + (roff[i] + col));
}
template <int NMS>
__device__ __forceinline__ void pf_store_a(const PfA<NMS>& A, _Float16* buf) {
  const int seg = threadIdx.x & 15, r0 = threadIdx.x >> 4;
  _Float16* dst = buf + r0 * kPfAStride + 8 * seg;
#pragma unroll
  for (int i = 0; i < NMS; ++i) *reinterpret_cast<u4v_t*>(dst + 16 * i * kPfAStride) = A.v[i];
}

// MFMAs of one K-step kb: the lane's codes (16 bytes of row n = l%16 per
// matrix, half h of the pair in C), dequantized with
// the group's scale and bias (from the wave's LDS table with SB, else as
// loaded into B), against the staged A rows.
template <int NM, int NMS, bool SB>
__device__ __forceinline__ void pf_mma(const PfWG<NM>& C, int h, const PfSB<NM>& B,
                                       const uint16_t (*tb)[SB ? kPfSbHalves : 1], int kb, int K,
                                       const _Float16* buf, f4_t (&acc)[NMS][NM]) {
  const int lane = threadIdx.x & 63, m = lane & 15, j = lane >> 4;
  const int G = K / 64, g = min(64 * kb + 16 * j, K / 2 - 16) >> 5;
  h8_t Bf[NM][4];
#pragma unroll
  for (int k = 0; k < NM; ++k) {
    const u4v_t q = C.v[k][h];
    const _Float16 sv = __builtin_bit_cast(_Float16, SB ? tb[k][m * G + g] : (uint16_t)B.s[k]);
    const _Float16 bv =
        __builtin_bit_cast(_Float16, SB ? tb[k][16 * G + m * G + g] : (uint16_t)B.b[k]);
    const h2_t s2 = {sv, sv}, b2 = {bv, bv};
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

// Depth of the pipeline: pairs of K-steps whose codes are held in registers
// (kPfPD), and A row sets loaded ahead for up to 32 rows and for more.
// 2 kPfPD must be a multiple of both.  (Deeper settings, 3 or 4 pairs and
// 4 or 8 A sets, measured no faster on the 128-token chunk.)
constexpr int kPfPD = 2;
constexpr int kPfADSmall = 4;
constexpr int kPfADBig = 2;

// C = A W^T over one pass of Mc <= 64 A rows (sh.rows[0..Mc) set: element
// offsets of rows of pad128(K) columns, the padding zero), K columns, for
// the wave's 16 weight rows from n_wave0 on; acc[ms][k]: lane l holds rows
// 16ms + 4(l/16) + r, column n_wave0 + l%16.
//
// Pipeline, per iteration SPI = 2 PD K-steps:
//  - codes: pair i of the iteration in register set G[i], which takes pair
//    i + PD once both of its steps are done;
//  - scales and biases (without SB): per step, NSS steps ahead (NSS sets);
//  - A rows: in AD register sets, loaded AD + 1 steps ahead and stored, AD
//    steps after their loads were issued, to the LDS buffer of the next
//    step (two alternating buffers, one barrier per step).
// Loads and stores are unconditional (past the last step they re-read the
// last one), so every wait for a load in flight waits for that load only;
// the last iteration stops after step nkb - 1 (a uniform branch).  Loads
// complete in issue order, so a code load is complete at the latest when
// the A load issued after it is needed: AD steps bound the codes' lead too.
// rows(): writes sh.rows[0..Mc) and ends with a block barrier; it runs
// after the first weight loads are issued, so its reads overlap them.
template <int NM, int NMS, bool SB, typename Rows>
__device__ __forceinline__ void pf_pass(const DevQ (&W)[NM], int n_wave0, int K, int Mc,
                                        const _Float16* abase, PfShared<NM, SB>& sh,
                                        f4_t (&acc)[NMS][NM], Rows rows) {
  constexpr int PD = kPfPD;
  constexpr int SPI = 2 * PD;
  constexpr int AD = NMS <= 2 ? kPfADSmall : kPfADBig;
  static_assert(SPI % AD == 0, "A sets must divide the steps of an iteration");
  constexpr int NSS = SPI % 4 == 0 ? 4 : (SPI % 3 == 0 ? 3 : 2);
#pragma unroll
  for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
    for (int k = 0; k < NM; ++k) acc[ms][k] = f4_t{0.f, 0.f, 0.f, 0.f};
  const int nkb = (K + 127) / 128;
  const int wave = threadIdx.x >> 6;
  const PfGOff go = pf_goff(n_wave0, K);
  const PfSOff so = pf_soff(n_wave0 + ((threadIdx.x & 63) & 15), K);
  PfWG<NM> G[PD];
  PfSB<NM> S[NSS];  // without SB: scales and biases, NSS steps ahead
  PfA<NMS> R[AD];   // R[(s + 1) % AD] holds A(s + 1) when step s begins
  if constexpr (SB) {
    // the table: 16-byte units of the wave's rows' scales, then biases,
    // straight into LDS (no registers); issued first, so the waits below
    // for later loads cover them (loads complete in issue order)
    const int lane = threadIdx.x & 63, G = K / 64, nu = 4 * G;
#pragma unroll
    for (int k = 0; k < NM; ++k)
      for (int i = 0; i < cdiv(nu, 64); ++i) {
        const int u = min(64 * i + lane, nu - 1);
        const uint8_t* src =
            u < 2 * G ? reinterpret_cast<const uint8_t*>(W[k].s) + (size_t)n_wave0 * G * 2 + 16 * u
                      : reinterpret_cast<const uint8_t*>(W[k].b) + (size_t)n_wave0 * G * 2 +
                            16 * (u - 2 * G);
        __builtin_amdgcn_global_load_lds(
            (const QMOE_GLOBAL void*)src,
            (__attribute__((address_space(3))) void*)(&sh.sb[wave][k][512 * i]), 16, 0, 0);
      }
  }
  // prologue: the loads of a virtual iteration before the first, in the
  // loop's own order (per step t the A set it refills, then its scales;
  // after each pair's second step that pair's codes), so that at the loop
  // head the waits counted along both incoming paths agree: codes of pairs
  // 0..PD-1 (pair 0 first of all, before rows()), scales and biases of
  // steps 0..NSS-1, A(1)..A(AD); A(0) goes to LDS buffer 0.
  pf_load_wg<NM>(G[0], W, go, 0);
  rows();
  uint32_t roff[NMS];
  pf_rows<NMS, NM, SB>(roff, sh, Mc);
  PfA<NMS> A0;
  pf_load_a<NMS>(A0, abase, roff, 0);
#pragma unroll
  for (int t = 0; t < SPI; ++t) {
    const int ia = t + 1 + AD - SPI;
    if (ia >= 1) pf_load_a<NMS>(R[(t + 1) % AD], abase, roff, min(ia, nkb - 1));
    if constexpr (!SB)
      if (t >= SPI - NSS) pf_load_sb<NM>(S[t % NSS], W, so, t - (SPI - NSS));
    if ((t & 1) && (t >> 1) > 0) pf_load_wg<NM>(G[t >> 1], W, go, t >> 1);
  }
  pf_store_a<NMS>(A0, sh.a[0]);
  __syncthreads();
  // one step s = kb + t: A(s + 1) to the other buffer, A(s + 1 + AD) into
  // the set just freed, the MFMAs on A(s), scales and biases of s + NSS
  auto step = [&](int kb, int t, PfSB<NM>& Sx, const PfWG<NM>& C) {
    PfA<NMS>& X = R[(t + 1) % AD];
    pf_store_a<NMS>(X, sh.a[(t + 1) & 1]);
    pf_load_a<NMS>(X, abase, roff, min(kb + t + 1 + AD, nkb - 1));
    pf_mma<NM, NMS, SB>(C, t & 1, Sx, sh.sb[wave], kb + t, K, sh.a[t & 1], acc);
    if constexpr (!SB) pf_load_sb<NM>(Sx, W, so, kb + t + NSS);
    __syncthreads();
  };
  for (int kb = 0; kb < nkb; kb += SPI) {
#pragma unroll
    for (int t = 0; t < SPI; ++t) {
      if (t > 0 && kb + t >= nkb) break;
      step(kb, t, S[t % NSS], G[t >> 1]);
      if (t & 1) pf_load_wg<NM>(G[t >> 1], W, go, (kb >> 1) + (t >> 1) + PD);
    }
  }
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

// Work unit of block b: (item, tile of 64 weight rows).  The shared items
// (the first nsh) have tsh tiles each and come first; the experts' items
// have tr tiles each.  Returns false past the last item.
//
// Sibling items stream the same weights: the two chunks of the shared
// expert (T > 64), and those of each expert with more than kPfMaxM rows
// (they lead the experts' items, which come in decreasing row count; the
// dispatch puts their number in bits 16.. of the list's first word).  Their
// equal tiles get blocks 8 apart: the same XCD, dispatched together, so
// that the second read of a tile's weights can hit that XCD's L2.  A pair's
// 2 nt units go in groups of up to 8 tiles, the first chunk's then the
// second's.
struct PfUnit {
  int e, row0, M, n0;
};
__device__ __forceinline__ void pf_pair_unit(int u, int nt, int& chunk, int& tile) {
  const int g = u / 16, r = u - 16 * g;
  const int w = min(8, nt - 8 * g);  // tiles in this group
  chunk = r >= w ? 1 : 0;
  tile = 8 * g + (r >= w ? r - w : r);
}
__device__ __forceinline__ bool pf_unit(const int32_t* items, int T, int E, int K, int tsh, int tr,
                                        PfUnit& u) {
  const int b = blockIdx.x;
  const int nsh = (T + kPfMaxM - 1) / kPfMaxM;
  // it_p / tile_p: the unit as part of a sibling pair of experts' items,
  // it_q / tile_q: as a plain one (which applies is known once the list's
  // first word is in; both items' words are read with it)
  int it_p, tile_p, it_q, tile_q;
  bool routed = false;
  int b2 = 0;
  if (b < nsh * tsh) {
    if (nsh == 2) {
      pf_pair_unit(b, tsh, it_q, tile_q);
    } else {
      it_q = b / tsh;
      tile_q = b - it_q * tsh;
    }
    it_p = it_q;
    tile_p = tile_q;
  } else {
    routed = true;
    b2 = b - nsh * tsh;
    it_q = nsh + b2 / tr;
    tile_q = b2 - (it_q - nsh) * tr;
    const int pr = b2 / (2 * tr);
    int c;
    pf_pair_unit(b2 - pr * 2 * tr, tr, c, tile_p);
    it_p = min(nsh + 2 * pr + c, pf_max_items(E, K, T) - 1);
  }
  // one round trip: the items' words are read together with the list's
  // first word (the list has room for every item the grid can name)
  // (the empty asm uses all of them before the compares: the compiler would
  // otherwise read the items' words only after them, a second round trip)
  const int w0 = items[0];
  const int ep = items[1 + 3 * it_p], rp = items[2 + 3 * it_p], Mp = items[3 + 3 * it_p];
  const int eq = items[1 + 3 * it_q], rq = items[2 + 3 * it_q], Mq = items[3 + 3 * it_q];
  asm volatile("" ::"s"(w0), "s"(ep), "s"(rp), "s"(Mp), "s"(eq), "s"(rq), "s"(Mq));
  const int n = w0 & 0xffff, npair = w0 >> 16;
  const bool pair = routed && b2 < 2 * npair * tr;
  const int it = pair ? it_p : it_q;
  u.e = pair ? ep : eq;
  u.row0 = pair ? rp : rq;
  u.M = pair ? Mp : Mq;
  u.n0 = (pair ? tile_p : tile_q) * kPfRows;
  return it < n;
}

// gate/up: one block per unit (1-D grid); a unit of the shared expert
// covers token rows [row0, row0 + M) of X, one of expert e the sorted pair
// rows [row0, row0 + M).
template <bool SB>
__global__ __launch_bounds__(kBlock, 2) void k_pf_gu(PfArgs a) {
  __shared__ PfShared<2, SB> sh;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  PfUnit u;
  if (!pf_unit(a.items, a.T, a.E, a.K, a.Is / kPfRows, a.I / kPfRows, u)) return;
  const bool shared = u.e < 0;
  DevQ W[2];
  if (shared) {
    W[0] = a.shg;
    W[1] = a.shu;
  } else {
    int s = a.slot ? a.slot[u.e] : u.e;
    W[0] = devq_at(a.gate, s);
    W[1] = devq_at(a.up, s);
  }
  const int n = u.n0 + 16 * wave + (lane & 15);  // N is a multiple of 64
  _Float16* out = shared ? a.act_sh : a.act;
  const int N = shared ? a.Is : a.I, ld = pad128(N);
  const int Mc = u.M;
  // the last tile also zeroes the padding columns of its rows
  if (u.n0 + kPfRows == N) {
    const int np = ld - N;
    for (int i = threadIdx.x; i < Mc * np; i += kBlock) {
      const int m = i / np;
      out[(size_t)(u.row0 + m) * ld + N + (i - m * np)] = (_Float16)0.f;
    }
  }
  auto rows = [&] {
    for (int m = threadIdx.x; m < Mc; m += kBlock) {
      int t = shared ? u.row0 + m : a.perm[u.row0 + m] / a.K;
      sh.rows[m] = t * pad128(a.H);
    }
    __syncthreads();
  };
  if (Mc <= 16) {
    f4_t acc[1][2];
    pf_pass<2, 1, SB>(W, n - (lane & 15), a.H, Mc, a.xh, sh, acc, rows);
    pf_gu_store<1>(acc, out, ld, u.row0, Mc, n);
  } else if (Mc <= 32) {
    f4_t acc[2][2];
    pf_pass<2, 2, SB>(W, n - (lane & 15), a.H, Mc, a.xh, sh, acc, rows);
    pf_gu_store<2>(acc, out, ld, u.row0, Mc, n);
  } else {
    f4_t acc[4][2];
    pf_pass<2, 4, SB>(W, n - (lane & 15), a.H, Mc, a.xh, sh, acc, rows);
    pf_gu_store<4>(acc, out, ld, u.row0, Mc, n);
  }
}

// down: one block per unit (1-D grid), H / 64 tiles per item.
template <bool SB>
__global__ __launch_bounds__(kBlock, 3) void k_pf_down(PfArgs a) {
  __shared__ PfShared<1, SB> sh;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  PfUnit u;
  if (!pf_unit(a.items, a.T, a.E, a.K, a.H / kPfRows, a.H / kPfRows, u)) return;
  const bool shared = u.e < 0;
  const int Kd = shared ? a.Is : a.I;
  const _Float16* src = shared ? a.act_sh : a.act;
  DevQ W[1];
  if (shared) {
    W[0] = a.shd;
  } else {
    int s = a.slot ? a.slot[u.e] : u.e;
    W[0] = devq_at(a.down, s);
  }
  const int n = u.n0 + 16 * wave + (lane & 15);  // H is a multiple of 64
  float* out = shared ? a.y_sh : a.y;
  const int Mc = u.M;
  auto rows = [&] {
    for (int m = threadIdx.x; m < Mc; m += kBlock) sh.rows[m] = (u.row0 + m) * pad128(Kd);
    __syncthreads();
  };
  if (Mc <= 16) {
    f4_t acc[1][1];
    pf_pass<1, 1, SB>(W, n - (lane & 15), Kd, Mc, src, sh, acc, rows);
    pf_down_store<1>(acc, out, a.H, u.row0, Mc, n);
  } else if (Mc <= 32) {
    f4_t acc[2][1];
    pf_pass<1, 2, SB>(W, n - (lane & 15), Kd, Mc, src, sh, acc, rows);
    pf_down_store<2>(acc, out, a.H, u.row0, Mc, n);
  } else {
    f4_t acc[4][1];
    pf_pass<1, 4, SB>(W, n - (lane & 15), Kd, Mc, src, sh, acc, rows);
    pf_down_store<4>(acc, out, a.H, u.row0, Mc, n);
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
  int32_t* counts = reinterpret_cast<int32_t*>(pf + pl.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(pf + pl.offsets);
  a.perm = reinterpret_cast<int32_t*>(pf + pl.perm);
  a.xh = reinterpret_cast<_Float16*>(pf + pl.xh);
  a.act = reinterpret_cast<_Float16*>(pf + pl.act);
  a.act_sh = reinterpret_cast<_Float16*>(pf + pl.act_sh);
  a.y = reinterpret_cast<float*>(pf + pl.y);
  a.y_sh = reinterpret_cast<float*>(pf + pl.y_sh);
  int32_t* pos_of = reinterpret_cast<int32_t*>(pf + pl.pos);
  a.items = reinterpret_cast<int32_t*>(pf + pl.items);
  const int n8 = T * (pad128(H) / 8);
  hipLaunchKernelGGL(k_pf_dispatch, dim3(1 + (n8 + 1023) / 1024), dim3(1024), 0, S(stream), idx,
                     T * K, T, E, counts, offsets, const_cast<int32_t*>(a.perm), pos_of,
                     const_cast<int32_t*>(a.items), X, H, const_cast<_Float16*>(a.xh));
  // 1-D grids over the work units; blocks past the last item return at once
  const int nsh = (T + kPfMaxM - 1) / kPfMaxM;
  const int nr = pf_max_items(E, K, T) - nsh;
  const int gu_blocks = nsh * (Is / kPfRows) + nr * (I / kPfRows);
  const int dn_blocks = (nsh + nr) * (H / kPfRows);
  // scales and biases from an LDS table where a row's groups fit it
  if (H / 64 <= kPfSbMaxG)
    hipLaunchKernelGGL(k_pf_gu<true>, dim3(gu_blocks), dim3(kBlock), 0, S(stream), a);
  else
    hipLaunchKernelGGL(k_pf_gu<false>, dim3(gu_blocks), dim3(kBlock), 0, S(stream), a);
  if ((I > Is ? I : Is) / 64 <= kPfSbMaxG)
    hipLaunchKernelGGL(k_pf_down<true>, dim3(dn_blocks), dim3(kBlock), 0, S(stream), a);
  else
    hipLaunchKernelGGL(k_pf_down<false>, dim3(dn_blocks), dim3(kBlock), 0, S(stream), a);
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
