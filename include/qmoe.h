/*
 * qmoe.h -- C ABI of the MI355X (gfx950) quantized Mixture-of-Experts FFN
 * step: 8-bit affine router with softmax top-k, 4-bit affine (MLX-style,
 * group 64) expert GEMVs for the routed and the shared expert, router-
 * weighted combine, and the chunked-prefill variant.
 *
 * What the step computes is described in words on these pages:
 *  - devtrends.cc, "Come eseguire un modello da 26 miliardi di parametri in
 *    due gigabyte di memoria su un Mac normale", section "Qual è il trucco
 *    principale dell'architettura" (a router per layer selects 8 experts;
 *    16-slot LFU expert cache; the shared branch is computed while missing
 *    experts are read) and section "Prestazioni nel mondo reale" (128-token
 *    prefill chunks so one loaded expert serves a group of rows);
 *  - remio.ai, "TurboFieldfare esegue Mac Gemma 4 26B in 2 GB, ma la velocità
 *    dell'SSD diventa il compromesso", section "L'affermazione dei 2 GB
 *    trasforma la larghezza di banda dell'SSD nel nuovo vincolo" (4-bit MLX
 *    affine weights, 8-bit router, shared and routed branches combined, 30
 *    layers, prefill chunks of up to 128 tokens);
 *  - iitog.ru, "TurboFieldfare: движок с открытым кодом запускает Gemma 4 26B
 *    на Mac с 8 ГБ памяти", technical paragraph (quantized GEMV, MoE routing
 *    and normalisation kernels);
 *  - elsolitario.org, TurboFieldfare article, section "Detalles técnicos y
 *    rendimiento" (MLX affine 4-bit, group size 64; router at 8 bits).
 *
 * Conventions shared by every entry point
 *  - Tensor pointers are DEVICE pointers owned by the caller.  Structs are
 *    host memory and are read only during the call.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *    default stream).  No entry point allocates, frees or synchronises,
 *    except qmoe_workspace_status(), which reads back one word.
 *  - Scratch memory comes from the caller through `ws`/`ws_bytes`, sized by
 *    qmoe_workspace_bytes().  A workspace must be zero-filled once before its
 *    first use; every call leaves it ready for the next one.  One workspace
 *    serves one call at a time (calls sharing a workspace must be ordered on
 *    one stream).
 *  - Arguments are validated before anything is launched; on error nothing
 *    is launched and a qmoe_status other than QMOE_OK is returned.  Device-
 *    side faults surface at the caller's next synchronisation.  NaN/Inf
 *    inputs give undefined (but finite-time) results.
 *  - Numbers: bf16 and fp16 values travel as their uint16_t bit patterns.
 *    Arithmetic is fp32 with fp32 accumulation; each layer output is rounded
 *    to bf16 (round to nearest even) once, after the residual add.
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QMOE_OK = 0,
  QMOE_ERR_NULL_ARG = 1,    /* a required pointer is NULL */
  QMOE_ERR_BAD_SHAPE = 2,   /* inconsistent or out-of-range sizes */
  QMOE_ERR_UNSUPPORTED = 3, /* bits/group/size outside what the kernels do */
  QMOE_ERR_WORKSPACE = 4,   /* ws NULL or smaller than qmoe_workspace_bytes */
  QMOE_ERR_ALIGN = 5,       /* a pointer or stride is not 16-byte aligned */
  QMOE_ERR_HIP = 6,         /* a HIP runtime call failed */
  QMOE_ERR_DEVICE = 7       /* the device reported a failed wait (status read) */
} qmoe_status;

/* One affine-quantized matrix W[rows][cols] (MLX-style, group 64):
 *   W[r][c] = scale[r][c/64] * q[r][c] + bias[r][c/64]
 * q: uint32 words, codes packed least-significant-bits first along the
 *    column axis (8 codes per word for bits=4, 4 for bits=8), rows
 *    contiguous: [rows][cols*bits/32].  16-byte aligned.
 * scales, biases: fp16 bit patterns, [rows][cols/64].
 * expert_stride_bytes: for stacked experts, expert e's q/scales/biases are
 *    at the given pointers plus e*expert_stride_bytes (all three advance by
 *    the same stride, which suits one contiguous blob per expert); 0 for a
 *    single matrix.  Multiple of 16. */
typedef struct {
  const uint32_t* q;
  const uint16_t* scales;
  const uint16_t* biases;
  int32_t rows, cols, bits, group;
  int64_t expert_stride_bytes;
} qmoe_qtensor;

/* One MoE layer.  router: bits=8, [n_experts x hidden].  gate/up: bits=4,
 * [inter x hidden] per expert; down: bits=4, [hidden x inter] per expert
 * (stacked through expert_stride_bytes).  sh_gate/sh_up: [shared_inter x
 * hidden]; sh_down: [hidden x shared_inter].
 * rms_gamma: bf16 [hidden] RMSNorm weight applied before the router and the
 * experts (NULL: the experts see the input as is); rms_eps its epsilon.
 * logit_bias: fp32 [n_experts] added to the router logits (NULL: none). */
typedef struct {
  int32_t hidden, n_experts, top_k, inter, shared_inter;
  qmoe_qtensor router;
  qmoe_qtensor gate, up, down;
  qmoe_qtensor sh_gate, sh_up, sh_down;
  const uint16_t* rms_gamma;
  float rms_eps;
  const float* logit_bias;
} qmoe_moe_layer;

/* Limits of the kernels (checked; larger sizes give QMOE_ERR_UNSUPPORTED). */
#define QMOE_MAX_TOP_K 8
#define QMOE_MAX_EXPERTS 512
#define QMOE_MAX_HIDDEN 16384
#define QMOE_MAX_TOKENS 128
#define QMOE_MAX_LAYERS 128

/* y[r] = sum_c W[r][c] x[c] for a 4-bit affine matrix (the quantized GEMV).
 * Defined by: elsolitario.org, TurboFieldfare article, section "Detalles
 * técnicos y rendimiento" (MLX affine 4-bit weights, group size 64);
 * iitog.ru, "TurboFieldfare: движок с открытым кодом…", technical paragraph
 * (a quantized-GEMV kernel).
 * W: bits=4, group=64, expert_stride_bytes ignored.  x: bf16 [cols].
 * y: fp32 [rows].  Returns QMOE_ERR_UNSUPPORTED for bits != 4. */
qmoe_status qmoe_gemv_affine4(const qmoe_qtensor* W, const uint16_t* x, float* y,
                              void* stream);

/* Offline repack of a 4-bit affine matrix into the GPU-tiled layout, and the
 * GEMV on it (devtrends.cc "Come eseguire un modello da 26 miliardi…",
 * section "Senza dipendenze da llama.cpp e MLX": a Repack step converts the
 * downloaded weights once into the engine's own layout; remio.ai
 * "TurboFieldfare esegue Mac Gemma 4 26B in 2 GB…", section "Mac Gemma 4
 * 26B entra nello spazio disponibile…").  Same numbers, different order:
 *   codes  [RB][CH][8][16 B]  row-block rb (8 rows), chunk c (32 codes):
 *                             the MLX row's code bytes 16c..16c+16
 *   pairs  [RB][8][G] uint32  scale | bias << 16 (fp16 bits), group g
 * RB = ceil(rows / 8), CH = cols / 32, G = cols / 64; rows past `rows` are
 * zero.  One wave load of a row-block is then one contiguous 1 KiB.
 * qmoe_tiled4_bytes: size of the repacked matrix (0 for invalid shapes:
 *   rows < 1, cols < 64 or not a multiple of 64).
 * qmoe_repack_tiled4: HOST memory in and out (an offline step, no GPU):
 *   q [rows][cols/2] codes (low nibble first), scales and biases fp16
 *   [rows][cols/64]; out: out_bytes >= qmoe_tiled4_bytes(rows, cols).
 *   The caller copies `out` to the device.
 * qmoe_gemv_tiled4: y[r] = sum_c W[r][c] x[c] from the repacked matrix on
 *   the device (16-byte aligned), x bf16 [cols] (16-byte aligned), y fp32
 *   [rows]; the same bits as qmoe_gemv_affine4 on the source matrix.
 *   cols must be 2816 or 704 (the compiled widths; else
 *   QMOE_ERR_UNSUPPORTED).  row_blocks_per_wave: 1 or 2 (rows per wave
 *   8 or 16, one row-block after the other), 0 for the library's choice
 *   (1). */
/* The token choice after the last layer (elsolitario.org, TurboFieldfare
 * article, section "Cómo empezar": temperature 0.2, top-K 64, top-P 0.95 by
 * default, temperature 0 for a deterministic choice; iitog.ru
 * "TurboFieldfare: движок с открытым кодом…", technical paragraph: a
 * sampling kernel).  Keep the top_k largest logits (equal logits: lower
 * token id first), in descending order.  temperature 0: token = rank 0.
 * Otherwise p_j = exp((l_j - l_0) / temperature) over the kept ranks; rank j
 * stays while the mass of the ranks before it is below top_p of the total;
 * the draw u in [0, 1) (the caller's uniform variate) takes the first kept
 * rank whose cumulative mass exceeds u times the kept mass (sums in rank
 * order, fp32).
 * logits: fp32 [V] on the device (finite).  token: int32 [1] on the device.
 * ranked: int32 [top_k] on the device (the kept-set candidates in rank
 * order) or NULL.  1 <= V <= 1,048,576; 1 <= top_k <= min(64, V);
 * 0 < top_p <= 1; temperature >= 0; 0 <= u < 1; else QMOE_ERR_BAD_SHAPE
 * (QMOE_ERR_UNSUPPORTED for V or top_k past the limits).
 * ws: at least qmoe_sample_workspace_bytes(V, top_k) bytes. */
size_t qmoe_sample_workspace_bytes(int32_t V, int32_t top_k);
qmoe_status qmoe_sample(const float* logits, int32_t V, float temperature, int32_t top_k,
                        float top_p, float u, int32_t* token, int32_t* ranked, void* ws,
                        size_t ws_bytes, void* stream);

size_t qmoe_tiled4_bytes(int32_t rows, int32_t cols);
qmoe_status qmoe_repack_tiled4(const uint8_t* q, const uint16_t* scales, const uint16_t* biases,
                               int32_t rows, int32_t cols, void* out, size_t out_bytes);
qmoe_status qmoe_gemv_tiled4(const void* tiled, int32_t rows, int32_t cols, const uint16_t* x,
                             float* y, int32_t row_blocks_per_wave, void* stream);

/* Router of T tokens (devtrends.cc "Come eseguire un modello da 26 miliardi…",
 * section "Qual è il trucco principale dell'architettura": a router per
 * layer selects 8 experts; remio.ai "TurboFieldfare esegue Mac Gemma 4 26B
 * in 2 GB…", section "L'affermazione dei 2 GB…": the router is 8-bit affine):
 * logits[t][e] = sum_c Wr[e][c] x[t][c] (+ bias[e]);
 * keep the top_k largest (ties: lower expert index first), ordered by
 * descending logit; w[t][j] = softmax over the kept logits (equal to a full
 * softmax renormalised over the kept experts).
 * Wr: bits=8 [E x H].  x: bf16 [T][H].  idx: int32 [T][top_k].
 * w: fp32 [T][top_k].  logits: fp32 [T][E] or NULL.  1 <= T <= 128,
 * 1 <= top_k <= min(8, E).  ws: at least qmoe_router_workspace_bytes(E, T). */
qmoe_status qmoe_router_topk(const qmoe_qtensor* Wr, const float* logit_bias,
                             const uint16_t* x, int32_t T, int32_t top_k,
                             int32_t* idx, float* w, float* logits, void* ws,
                             size_t ws_bytes, void* stream);

/* FFN of one token given its routing (remio.ai "TurboFieldfare esegue Mac
 * Gemma 4 26B in 2 GB…", sections "Mac Gemma 4 26B entra nello spazio
 * disponibile…" (eight routed experts and one shared expert) and
 * "L'affermazione dei 2 GB…" (the shared and routed branches are combined)):
 * for M in {shared, idx[0..k)}
 *   a_M = gelu_tanh(W_gate,M h) * (W_up,M h);   y_M = W_down,M a_M
 *   out = bf16( y_shared + sum_j w[j] y_idx[j]  (+ residual) )
 * h: bf16 [H] (the expert input, already normalised if the model norms).
 * idx: int32 [top_k] device; w: fp32 [top_k] device.
 * expert_slot: int32 [n_experts] device map expert -> position in the
 *   stacked routed tensors, or NULL for the identity.
 * residual: bf16 [H] or NULL.  out: bf16 [H]. */
qmoe_status qmoe_expert_ffn(const qmoe_moe_layer* L, const uint16_t* h,
                            const int32_t* idx, const float* w,
                            const int32_t* expert_slot, const uint16_t* residual,
                            uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/* One whole decode step of one layer for one token, in a single launch
 * (remio.ai "TurboFieldfare esegue Mac Gemma 4 26B in 2 GB…", section
 * "L'affermazione dei 2 GB…": router, experts and combine, per layer and
 * token):
 *   h = L->rms_gamma ? bf16(rmsnorm(x) * gamma) : x
 *   routing = top-k softmax of the router on h (+ logit_bias)
 *   out = bf16( FFN combine as in qmoe_expert_ffn  (+ x if residual) )
 * x: bf16 [H].  idx_out/w_out: optional copies of the routing (device,
 * [top_k]).  expert_slot as in qmoe_expert_ffn. */
qmoe_status qmoe_moe_decode(const qmoe_moe_layer* L, const uint16_t* x,
                            const int32_t* expert_slot, int32_t residual,
                            uint16_t* out, int32_t* idx_out, float* w_out,
                            void* ws, size_t ws_bytes, void* stream);

/* The same step as qmoe_moe_decode, run as three ordered launches (router;
 * shared and routed gate/up; down and combine) instead of one launch whose
 * blocks wait on each other.  Same kernels and arithmetic, so the results
 * are bitwise equal; kept for diagnosis and for comparing launch overheads. */
qmoe_status qmoe_moe_decode_phased(const qmoe_moe_layer* L, const uint16_t* x,
                                   const int32_t* expert_slot, int32_t residual,
                                   uint16_t* out, int32_t* idx_out, float* w_out,
                                   void* ws, size_t ws_bytes, void* stream);

/* qmoe_moe_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same step and kernels, bitwise the same results, with the
 * workspace in a fixed 512 KiB device array of the library, one per GPU (held
 * until the process ends; the first call on a GPU looks it up and zero-fills
 * it on `stream`).  Nothing is allocated or freed.  Layers whose workspace
 * (qmoe_workspace_bytes(L, 1)) exceeds 512 KiB get QMOE_ERR_WORKSPACE.  Every
 * call on a GPU uses that GPU's one array, which keeps the last call's
 * state: calls that overlap on one GPU race, so order them (one stream, or
 * events between streams).  No caller can read this array's error word: a
 * failed in-kernel wait (which valid inputs do not cause) leaves that call's
 * outputs undefined, and the call's last block restores the array for the
 * next call. */
qmoe_status qmoe_moe_decode_noalloc(const qmoe_moe_layer* L, const uint16_t* x,
                                    const int32_t* expert_slot, int32_t residual,
                                    uint16_t* out, int32_t* idx_out, float* w_out,
                                    void* stream);

/* qmoe_moe_decode with kernel timing: ev_start and ev_stop (hipEvent_t, or
 * NULL) are recorded by the launch itself at the start and at the end of
 * the step's kernel, so hipEventElapsedTime gives the kernel's duration
 * without the gaps around it.  Otherwise identical to qmoe_moe_decode. */
qmoe_status qmoe_moe_decode_timed(const qmoe_moe_layer* L, const uint16_t* x,
                                  const int32_t* expert_slot, int32_t residual,
                                  uint16_t* out, int32_t* idx_out, float* w_out,
                                  void* ws, size_t ws_bytes, void* stream,
                                  void* ev_start, void* ev_stop);

/* Chunked prefill of T <= 128 tokens that share one loaded copy of each
 * expert (devtrends.cc "Come eseguire un modello da 26 miliardi…", section
 * "Prestazioni nel mondo reale": 128-token chunks, one loaded expert serves
 * a group of rows; remio.ai, section "L'affermazione dei 2 GB…": chunks of
 * up to 128 tokens): the (token, rank) pairs are grouped by expert (stable: expert,
 * then token, then rank) and every expert runs one grouped dequantizing
 * GEMM over its rows on the matrix cores; the shared expert runs as a dense
 * GEMM over all T rows; then
 *   out[t] = bf16( y_shared[t] + sum_j w[t][j] y_idx[t][j][t]  (+ residual[t]) )
 * X: bf16 [T][H] (expert input).  idx/w: [T][top_k] device (from
 * qmoe_router_topk); idx values must lie in [0, n_experts) (others are
 * clamped into that range); an expert may repeat within a token.
 * residual: bf16 [T][H] or NULL.  out: bf16 [T][H].
 * The matrix cores take fp16 operands: X and the gate/up activations are
 * rounded to fp16 and each weight s*q + b is rounded to fp16 once (fp32
 * accumulation), so |X| and the activations must stay below 65504. */
qmoe_status qmoe_prefill_grouped(const qmoe_moe_layer* L, const uint16_t* X,
                                 int32_t T, const int32_t* idx, const float* w,
                                 const uint16_t* residual, uint16_t* out,
                                 void* ws, size_t ws_bytes, void* stream);

/* Inspection hook for tests: byte offsets inside the workspace of the
 * dispatch arrays that the last qmoe_prefill_grouped call on it wrote for
 * T tokens: counts int32[n_experts], offsets int32[n_experts + 1] (exclusive
 * prefix of counts), perm int32[T*top_k] (flat pair index t*top_k + j, in
 * the order expert, then t, then j). */
qmoe_status qmoe_prefill_dispatch_offsets(const qmoe_moe_layer* L, int32_t T,
                                          size_t* counts, size_t* offsets,
                                          size_t* perm);

/* out[t][i] = bf16( x[t][i] * gamma[i] / sqrt(mean_i x[t][i]^2 + eps) ).
 * x, out: bf16 [T][H]; gamma: bf16 [H]. */
qmoe_status qmoe_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps,
                         int32_t T, int32_t H, uint16_t* out, void* stream);

/* Workspace sizes in bytes (0 when the layer description is invalid). */
size_t qmoe_workspace_bytes(const qmoe_moe_layer* L, int32_t T);
size_t qmoe_router_workspace_bytes(int32_t n_experts, int32_t T);

/* Reads (synchronising `stream`) and clears the device error word of a
 * workspace.  *device_code receives 0 when every in-kernel wait completed,
 * nonzero when one gave up (the outputs of that call are then undefined).
 * In that case the whole control area (flags, tags, counters) is zeroed as
 * well, so the workspace is ready again.
 * Returns QMOE_OK, QMOE_ERR_DEVICE when the word was nonzero, or an error. */
qmoe_status qmoe_workspace_status(void* ws, size_t ws_bytes, int32_t* device_code,
                                  void* stream);

/* The workspace's tag counter.  Cross-block hand-offs inside a decode call
 * match flag and tag words against values above every value already in
 * the workspace: a one-layer call (qmoe_moe_decode, _timed, _phased,
 * qmoe_expert_ffn, the split FFN calls) uses counter + 1, a stack call of n
 * layers counter + 1 .. counter + n, and one block of the call raises the
 * counter by that many once every block of the call has read it.  So no
 * word left by an earlier call, of any shape or mode, matches a later
 * call's, whatever else ran in between.  A zero-filled workspace starts at
 * 0; near the top of the 32-bit range the last block zeroes every flag and
 * tag and restarts the counter at 0.
 * qmoe_workspace_tag_counter reads it (synchronising `stream`; all replicas
 * must agree, else QMOE_ERR_DEVICE).  qmoe_workspace_raise_tag_counter sets
 * it to `value` (test hook; only raising is allowed, and only below the
 * restart threshold 0xFFFFFF00, else QMOE_ERR_BAD_SHAPE). */
qmoe_status qmoe_workspace_tag_counter(void* ws, size_t ws_bytes, uint32_t* value, void* stream);
qmoe_status qmoe_workspace_raise_tag_counter(void* ws, size_t ws_bytes, uint32_t value,
                                             void* stream);

const char* qmoe_status_string(qmoe_status s);

/* ---------------------------------------------------------------------
 * Decode through a stack of layers in one launch (remio.ai "TurboFieldfare
 * esegue Mac Gemma 4 26B in 2 GB…", section "L'affermazione dei 2 GB
 * trasforma la larghezza di banda dell'SSD nel nuovo vincolo": the step
 * repeats in each of the model's 30 layers for every generated token).
 * Layer l maps x_l to x_{l+1} exactly as qmoe_moe_decode with residual = 1
 * (RMSNorm with the layer's rms_gamma, router top-k, shared and routed
 * FFN, combine, residual add, one bf16 rounding); the results are bitwise
 * those of n_layers ordered qmoe_moe_decode calls.  Weights are resident
 * (no expert -> slot map).
 * ------------------------------------------------------------------- */

/* Bytes of the device layer table for n_layers layers (0 when n_layers is
 * outside [1, QMOE_MAX_LAYERS]). */
size_t qmoe_stack_table_bytes(int32_t n_layers);

/* Writes the device form of layers[0..n_layers) (host array) into `table`
 * (device memory, caller-owned, 16-byte aligned, table_bytes >=
 * qmoe_stack_table_bytes(n_layers)).  Every layer must be valid and have the
 * sizes and rms_eps of layers[0].  Set-up, not the hot path: the copy is
 * enqueued on `stream` and the call waits for it.  The table holds the
 * layers' device pointers, so it stays valid while their weights do. */
qmoe_status qmoe_stack_table_init(const qmoe_moe_layer* layers, int32_t n_layers,
                                  void* table, size_t table_bytes, void* stream);

/* Workspace of qmoe_stack_decode for layers of this shape (0 if invalid):
 * the one-layer workspace plus two bf16 [hidden] buffers for the layer
 * inputs. */
size_t qmoe_stack_workspace_bytes(const qmoe_moe_layer* shape);

/* x_0 = x; x_{l+1} = layer l applied to x_l; out = x_{n_layers}.
 * shape: any layer of the stack (sizes, rms_eps; its pointers are not
 * used).  table: from qmoe_stack_table_init with at least n_layers layers
 * of that shape (not checked: the table is device memory).
 * x, out: bf16 [H], 16-byte aligned (out must not alias x).
 * layer_out: bf16 [n_layers][H] or NULL; receives every x_{l+1}.
 * idx_out/w_out: int32/fp32 [n_layers][top_k] or NULL; every layer's routing.
 * One cooperative launch: QMOE_ERR_UNSUPPORTED when the device cannot hold
 * all of its blocks at once.  Waits inside the launch are bounded as in
 * qmoe_moe_decode (see qmoe_workspace_status). */
qmoe_status qmoe_stack_decode(const qmoe_moe_layer* shape, const void* table,
                              int32_t n_layers, const uint16_t* x, uint16_t* out,
                              uint16_t* layer_out, int32_t* idx_out, float* w_out,
                              void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------
 * Split FFN: the shared expert's gate/up first, the rest after the routed
 * experts' weights are in place, so that host -> device copies of missing
 * experts (on another stream) overlap the shared expert (devtrends.cc,
 * section "Qual è il trucco principale dell'architettura").  Run on one
 * stream and one workspace, in this order, the pair computes exactly what
 * qmoe_expert_ffn computes (bitwise).
 * ------------------------------------------------------------------- */
qmoe_status qmoe_expert_ffn_shared(const qmoe_moe_layer* L, const uint16_t* h,
                                   void* ws, size_t ws_bytes, void* stream);
qmoe_status qmoe_expert_ffn_routed(const qmoe_moe_layer* L, const uint16_t* h,
                                   const int32_t* idx, const float* w,
                                   const int32_t* expert_slot,
                                   const uint16_t* residual, uint16_t* out,
                                   void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------
 * Host-resident expert pool (devtrends.cc, section "Qual è il trucco
 * principale dell'architettura": 16 slots per layer, least frequently
 * used; remio.ai "TurboFieldfare esegue Mac Gemma 4 26B in 2 GB…", section
 * "Mac Gemma 4 26B entra nello spazio disponibile…").
 *
 * Every routed expert blob of every layer sits in pinned host memory
 * (host_blobs[layer * experts + e], blob_bytes each, allocated with
 * hipHostMalloc by the caller).  Each layer has a device arena of `slots`
 * blobs (dev_slot_arena[layer], caller-owned); the layer's gate/up/down
 * qmoe_qtensors point into it with expert_stride_bytes = blob_bytes, and
 * the FFN kernels find an expert through the expert -> slot map that
 * qmoe_pool_acquire writes.
 *
 * Replacement, per layer (one acquire is one step): every needed expert's
 * use count is incremented and its last use set to the step; needed experts
 * in a slot are hits; misses, in rank order, take the lowest free slot, or
 * evict the resident expert not needed in this step with the smallest
 * (use count, last use, id).  Counts are never reset.
 * ------------------------------------------------------------------- */
typedef struct qmoe_pool qmoe_pool;
typedef struct {
  int64_t hits, misses;       /* cumulative over every acquire */
  int64_t h2d_bytes;          /* cumulative host -> device bytes */
  int32_t last_hits, last_misses;
} qmoe_pool_stats;

/* host_blobs and dev_slot_arena may both be NULL: a planning-only pool
 * (bookkeeping without copies, usable without a GPU; see qmoe_pool_plan).
 * dev_slot_arena without host_blobs: a file-backed pool (filled only by
 * qmoe_pool_acquire_file).
 * Allocates host memory only (bookkeeping and two pinned expert -> slot
 * staging maps per layer). */
qmoe_status qmoe_pool_create(int32_t layers, int32_t experts, int32_t slots,
                             size_t blob_bytes, const void* const* host_blobs,
                             void* const* dev_slot_arena, qmoe_pool** out);

/* One replacement step of `layer` for the needed experts host_idx[0..k)
 * (distinct, host memory), without copies.  slot_out/hit_out/victim_out
 * ([k], host, each may be NULL): the slot of each needed expert, 1 for a
 * hit, and the expert evicted to make room (-1: none). */
qmoe_status qmoe_pool_plan(qmoe_pool* pool, int32_t layer, const int32_t* host_idx,
                           int32_t k, int32_t* slot_out, int32_t* hit_out,
                           int32_t* victim_out);

/* One replacement step (as qmoe_pool_plan), then on copy_stream: the
 * missing blobs host -> device into their slots, the layer's expert -> slot
 * map into dev_expert_slot (int32 [experts], device), and `ready` (a
 * hipEvent_t, or NULL) recorded after them.  The compute stream must wait
 * for `ready` before the routed part of the layer.  Slots are overwritten:
 * work that read this layer's slots must be complete (or ordered before
 * copy_stream).  st (or NULL) receives the cumulative statistics. */
qmoe_status qmoe_pool_acquire(qmoe_pool* pool, int32_t layer, const int32_t* host_idx,
                              int32_t k, int32_t* dev_expert_slot, void* copy_stream,
                              void* ready, qmoe_pool_stats* st);
qmoe_status qmoe_pool_stats_get(const qmoe_pool* pool, qmoe_pool_stats* st);
void qmoe_pool_destroy(qmoe_pool* pool);

/* File-backed expert tier (devtrends.cc "Come eseguire un modello da 26
 * miliardi…", section "Qual è il trucco principale dell'architettura": the
 * CPU compares the router's choice with the cache and issues bounded
 * parallel reads for the missing experts while the shared expert computes;
 * remio.ai "TurboFieldfare esegue Mac Gemma 4 26B in 2 GB…", section
 * "L'affermazione dei 2 GB trasforma la larghezza di banda dell'SSD nel
 * nuovo vincolo": storage bandwidth becomes the constraint).
 *
 * The file is expert-major: the blob of (layer, e) (blob_bytes, the same
 * bytes as a host blob of the pool) at byte offset (layer * experts + e) *
 * stride, stride >= blob_bytes and a multiple of 4096.  `threads` worker
 * threads (1..64) pread whole strides into pinned staging buffers (two sets
 * of max_misses strides, 1 <= max_misses <= 8, used in turn); with direct
 * != 0 the file is opened O_DIRECT and one stride is read at once to check
 * that the file system takes it (QMOE_ERR_UNSUPPORTED if not).
 * Errors: QMOE_ERR_BAD_SHAPE for a missing or short file or bad sizes,
 * QMOE_ERR_ALIGN for a stride not a multiple of 4096.
 *
 * qmoe_pool_acquire_file: as qmoe_pool_acquire for a pool created with
 * dev_slot_arena and host_blobs == NULL (a file-backed pool): one LFU step,
 * then the missing blobs are read from the file (the call returns after the
 * reads; QMOE_ERR_HIP if a read failed) and copied host -> device on
 * copy_stream, then the map and `ready`.  k <= max_misses.  Calls on one
 * tier must not overlap. */
typedef struct qmoe_file_tier qmoe_file_tier;
typedef struct {
  int64_t reads, read_bytes; /* cumulative blobs and bytes read (whole strides) */
  int64_t read_ns;           /* wall time spent in the reads (all workers busy or done) */
  int32_t last_errno;        /* errno of the last failed read (-1: end of file), else 0 */
} qmoe_file_tier_stats;
qmoe_status qmoe_file_tier_open(const char* path, int32_t layers, int32_t experts,
                                size_t blob_bytes, size_t stride, int32_t threads,
                                int32_t max_misses, int32_t direct, qmoe_file_tier** out);
qmoe_status qmoe_pool_acquire_file(qmoe_pool* pool, qmoe_file_tier* tier, int32_t layer,
                                   const int32_t* host_idx, int32_t k, int32_t* dev_expert_slot,
                                   void* copy_stream, void* ready, qmoe_pool_stats* st);
qmoe_status qmoe_file_tier_stats_get(const qmoe_file_tier* tier, qmoe_file_tier_stats* st);
void qmoe_file_tier_close(qmoe_file_tier* tier);

/* Decode attention over an FP16 key/value cache, with RoPE (iitog.ru
 * "TurboFieldfare: движок с открытым кодом…", technical paragraph: attention
 * and RoPE kernels, an FP16 KV cache, 25 sliding-window layers in a bounded
 * circular store and 5 full-attention layers in a linear one; remio.ai
 * "TurboFieldfare esegue Mac Gemma 4 26B in 2 GB…", section "Mac Gemma 4 26B
 * entra nello spazio disponibile…": a 4,096-token cache).  Head shapes are
 * not on the pages: they are arguments.
 *
 * One call is the token at time pos (0-based):
 *   q' = RoPE(q), k' = RoPE(k): element i and element i + D/2 (i < D/2)
 *     rotated by the angle pos * rope_base^(-2i/D) in the positive sense
 *     (x_i cos - x_{i+D/2} sin, x_{i+D/2} cos + x_i sin), computed in fp64;
 *   slot = pos mod S (circular) or pos (linear) receives fp16(k') in
 *     k_cache and fp16(v) in v_cache (round to nearest even);
 *   query head h attends with key/value head h / (Hq / Hkv) over the tokens
 *     in the cache: times pos - S + 1 .. pos (circular; 0 .. pos while pos
 *     < S) or 0 .. pos (linear): score_t = scale * <q'_h, K_t> (fp32),
 *     out_h = sum_t softmax(score)_t V_t, written as bf16.
 * q: fp32 [Hq][D]; k, v: fp32 [Hkv][D] (the projections of this token);
 * k_cache, v_cache: fp16 [Hkv][S][D], owned by the caller, 16-byte aligned;
 *   slots that hold no token of the window are neither read nor written;
 * out: bf16 [Hq][D].  All on the device.
 * Supported: head_dim 128 with Hq / Hkv in {1, 2, 4}, head_dim 256 with
 * Hq / Hkv in {1, 2} (else QMOE_ERR_UNSUPPORTED); Hkv divides Hq; S >= 1;
 * pos >= 0, and pos < S for a linear cache (else QMOE_ERR_BAD_SHAPE);
 * rope_base > 1.  ws: at least qmoe_attn_workspace_bytes(shape) bytes, 16-
 * byte aligned: control words (an error word, one epoch per key/value head)
 * and the partial results of the splits of the cache, tagged with the
 * epoch.  The workspace must be zero-filled before its first call; one fill
 * serves every later call, of any shape.  Calls that share a cache or a
 * workspace run in stream order.
 * qmoe_attn_workspace_status: reads the error word (in *device_code),
 * nonzero when an in-kernel wait for another block's partial gave up (the
 * output of that call is not valid); then the whole workspace is zeroed
 * and QMOE_ERR_DEVICE returned.  Synchronises the stream. */
typedef struct {
  int32_t n_heads;     /* Hq: query heads */
  int32_t n_kv_heads;  /* Hkv: key/value heads, divides Hq */
  int32_t head_dim;    /* D */
  int32_t slots;       /* S: cache capacity in tokens */
  int32_t circular;    /* 1: sliding window of S tokens; 0: linear, pos < S */
  float rope_base;     /* RoPE frequency base */
  float scale;         /* score scale (e.g. 1 / sqrt(D)) */
} qmoe_attn_shape;
size_t qmoe_attn_workspace_bytes(const qmoe_attn_shape* shape);
qmoe_status qmoe_attn_decode(const qmoe_attn_shape* shape, const float* q, const float* k,
                             const float* v, int32_t pos, uint16_t* k_cache, uint16_t* v_cache,
                             uint16_t* out, void* ws, size_t ws_bytes, void* stream);
qmoe_status qmoe_attn_workspace_status(void* ws, size_t ws_bytes, int32_t n_kv_heads,
                                       int32_t* device_code, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* QMOE_H */
