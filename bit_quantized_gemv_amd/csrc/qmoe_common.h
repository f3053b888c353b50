// qmoe_common.h -- device helpers and internal layouts of the gfx950 kernels.
//
// Storage format read by every kernel (MLX-style affine quantization, group
// 64; remio.ai "TurboFieldfare esegue Mac Gemma 4 26B in 2 GB…", section
// "L'affermazione dei 2 GB trasforma la larghezza di banda dell'SSD nel
// nuovo vincolo"; elsolitario.org, "Detalles técnicos y rendimiento"):
// codes packed LSB-first along the input axis into uint32 words, one fp16
// scale and one fp16 bias per row and per 64 inputs, W = scale * q + bias.
//
// Work is cut into 16-byte "chunks": one chunk holds 32 four-bit codes (half
// a group) or 16 eight-bit codes (a quarter group).  A wave works on a
// "row-block" of 8 rows: lane l owns row (l & 7) and chunk slot (l >> 3), so
// one load instruction reads 8 consecutive chunks (128 contiguous bytes) of
// each of 8 rows, and every lane keeps a single running sum for its row.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmoe.h"

namespace qmoe {

constexpr int kWave = 64;
constexpr int kBlock = 256;          // threads per block for every kernel here
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kRowsPerUnit = 8;      // rows of one row-block (lane & 7)
constexpr int kSlots = 8;            // chunk slots per step (lane >> 3)

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// ----------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_to_f32(uint32_t v) {
  return __uint_as_float(v << 16);
}

// fp32 -> bf16, round to nearest, ties to even.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float half_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// ------------------------------------------------------------ dequant dots
// A byte holding a code q in 0..15, read as an OCP e4m3 number, is exactly
// q * 2^-9 (codes 0..7 are its subnormals, 8..15 its first binade), so the
// gfx950 fp8 conversions turn masked nibbles into exact numbers:
//   lo = w & 0x0F0F0F0F holds codes (q0, q2, q4, q6) of word w,
//   hi = (w >> 4) & 0x0F0F0F0F holds (q1, q3, q5, q7).
// Activations are stored in the matching order.

// Four-bit codes against bf16 activations on the dot2 unit.  The converted
// pairs are (q0,q2) (q4,q6) (q1,q3) (q5,q7) in exact bf16 (scale 2^9); the
// activation pairs of the word are stored as (x0,x2) (x4,x6) (x1,x3) (x5,x7).
__device__ __forceinline__ float dot_word4_bf16(uint32_t v, uint4 xp, float acc) {
  const uint32_t lo = v & 0x0F0F0F0Fu, hi = (v >> 4) & 0x0F0F0F0Fu;
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, false),
                                        __builtin_bit_cast(bf16x2_t, xp.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, true),
                                        __builtin_bit_cast(bf16x2_t, xp.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, false),
                                        __builtin_bit_cast(bf16x2_t, xp.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, true),
                                        __builtin_bit_cast(bf16x2_t, xp.w), acc, false);
  return acc;
}

// Four-bit codes against fp32 activations: the fp8 conversion yields
// q * 2^-9 in fp32 (exact); the caller folds 2^9 into the scale.  The
// activations of word v are stored as (a0,a2,a4,a6) and (a1,a3,a5,a7).
__device__ __forceinline__ void dot_word4_f32(uint32_t v, float4 ae, float4 ao, float& acc0,
                                              float& acc1) {
  const uint32_t lo = v & 0x0F0F0F0Fu, hi = (v >> 4) & 0x0F0F0F0Fu;
  f32x2_t p0 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);  // q0, q2
  f32x2_t p1 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);   // q4, q6
  f32x2_t p2 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);  // q1, q3
  f32x2_t p3 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);   // q5, q7
  acc0 = fmaf(p0.x, ae.x, acc0);
  acc1 = fmaf(p0.y, ae.y, acc1);
  acc0 = fmaf(p1.x, ae.z, acc0);
  acc1 = fmaf(p1.y, ae.w, acc1);
  acc0 = fmaf(p2.x, ao.x, acc0);
  acc1 = fmaf(p2.y, ao.y, acc1);
  acc0 = fmaf(p3.x, ao.z, acc0);
  acc1 = fmaf(p3.y, ao.w, acc1);
}

// Eight-bit codes (4 per word, in column order) against fp32 activations.
__device__ __forceinline__ float dot_word8_f32(uint32_t v, float4 x, float acc) {
  acc = fmaf((float)(v & 0xffu), x.x, acc);
  acc = fmaf((float)((v >> 8) & 0xffu), x.y, acc);
  acc = fmaf((float)((v >> 16) & 0xffu), x.z, acc);
  acc = fmaf((float)(v >> 24), x.w, acc);
  return acc;
}

// Sum over the 8 lanes of a wave that share (lane & 7); every lane gets the
// same bits (the butterfly adds the same operands in the same order).
__device__ __forceinline__ float rowblock_sum(float v) {
  v += __shfl_xor(v, 8);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float gelu_tanh(float z) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  const float k1 = 0.044715f;
  return 0.5f * z * (1.0f + tanhf(k0 * fmaf(k1 * z * z, z, z)));
}

// Loads through these pointers are global-memory loads.  Pointers that the
// compiler cannot trace to a kernel argument (read from a table in device
// memory) would otherwise become flat loads, which also count as LDS
// operations: every wait for an LDS result or barrier would then wait for
// all weight loads in flight.
#define QMOE_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ const QMOE_GLOBAL T* gptr(const T* p) {
  return (const QMOE_GLOBAL T*)p;
}

// Weights are read once per step: non-temporal loads, so that they do not
// displace the kernel's code and the small exchanged data from the caches.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldg16(const uint8_t* p) {
  u32x4_t v = __builtin_nontemporal_load(gptr(reinterpret_cast<const u32x4_t*>(p)));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 16 bytes at p + 16 i through the cache (a global-memory load).
__device__ __forceinline__ uint4 ld_g16(const void* p, int64_t i) {
  u32x4_t v = gptr(reinterpret_cast<const u32x4_t*>(p))[i];
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Packed (scale | bias << 16) fp16 pair at element offset `off`.
__device__ __forceinline__ uint32_t ld_sb(const uint16_t* s, const uint16_t* b, int64_t off) {
  return (uint32_t)__builtin_nontemporal_load(gptr(s + off)) |
         ((uint32_t)__builtin_nontemporal_load(gptr(b + off)) << 16);
}

// ----------------------------------------- device-coherent data exchange
// Values handed from one block to another inside a launch are written and
// read with agent-scope relaxed atomics, which gfx950 performs with the
// device-coherence bit (sc1): they bypass the non-coherent per-XCD L2
// copies.  A producer publishes by waiting for its stores to complete
// (vmcnt 0) before its flag store; a consumer reads data only after it has
// seen the flag.  No cache writeback/invalidate fences are issued.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_dev(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte device-coherent load (buffer load with the sc1 bit) of
// base[byte_off .. byte_off+16); `base` must be wave-uniform, reads past
// `nbytes` return zeros.
__device__ __forceinline__ float4 ld_dev16(const float* base, uint32_t nbytes, uint32_t byte_off) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, (int)nbytes, 0x00020000);
  v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 16 /* sc1 */);
  return __builtin_bit_cast(float4, v);
}
// Wait until every vector memory operation of this wave has completed.
__device__ __forceinline__ void wait_vm() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ------------------------------------------------------- device matrices
struct DevQ {
  const uint8_t* q;
  const uint16_t* s;
  const uint16_t* b;
  int64_t stride;  // bytes between experts (0: single)
};

__host__ __device__ inline DevQ devq(const qmoe_qtensor& t) {
  DevQ d;
  d.q = reinterpret_cast<const uint8_t*>(t.q);
  d.s = t.scales;
  d.b = t.biases;
  d.stride = t.expert_stride_bytes;
  return d;
}

__device__ __forceinline__ DevQ devq_at(DevQ d, int64_t slot) {
  DevQ r;
  r.q = d.q + slot * d.stride;
  r.s = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(d.s) + slot * d.stride);
  r.b = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(d.b) + slot * d.stride);
  r.stride = 0;
  return r;
}

// ----------------------------------------------------------- workspace
// Control area.  Small values that many blocks poll (the router's logits
// and the per-group flags) are published in kRep replicas kRepStride bytes
// apart, so that pollers spread over memory channels instead of all
// hitting one line; consumer block b reads replica b % kRep.
namespace ctl {
constexpr int kError = 0;             // word: nonzero when an in-kernel wait gave up
// Tag counter G of the workspace, in kGenRep replicas kGenStride bytes
// apart (block b reads replica b % kGenRep).  A call whose flags and tags
// are matched against the values v = G+1 .. G+n (one per layer) raises G by
// n once every block of the call has read it, so every value a call waits
// for is larger than any flag or tag already in the workspace.  A zero-
// filled workspace starts at G = 0 (flags and tags 0).  Near the top of the
// 32-bit range the control area is cleared instead and G restarts at 0.
constexpr int kGenBase = 64;
constexpr int kGenRep = 8;
constexpr int kGenStride = 64;
constexpr uint32_t kGenLimit = 0xFFFFFF00u;
constexpr int kRep = 4;              // fewer stores per producer; more readers per replica
                                      // (decode step: 4 beat 1, 2, 8 and 16)
constexpr int kRepStride = 4352;      // bytes between replicas (4 KiB + 256)
constexpr int kTagBase = 4096;        // byte offset of the tagged-logit replicas
constexpr int kFlagBase = kTagBase + kRep * kRepStride;   // per-block flag replicas:
                                      // words [0, nS) shared gate/up blocks, then
                                      // [nS + k*perG + i) routed expert k block i
constexpr int kMaxFlags = kRepStride / 4;
constexpr int kCntBase = kFlagBase + kRep * kRepStride;   // counters, 64 B apart
constexpr int kCntRouterTile = 0;     // [16] standalone router: per token tile
constexpr int kCntStack = 16;         // layer stack: output blocks done with the last layer
constexpr int kCntDone = 17;          // [kGenRep] one-layer call: its last role's blocks done,
                                      // per group (block index % kGenRep)
constexpr int kCntDoneTop = kCntDone + kGenRep;  // groups done
constexpr int kNCnt = kCntDoneTop + 1;
constexpr int kBytes = kCntBase + kNCnt * 64;
}  // namespace ctl
constexpr size_t kCtlBytes = (size_t)ctl::kBytes;

// Device form of one layer of a decode stack (the pointers of
// qmoe_moe_layer that change from layer to layer).
struct StackLayerDev {
  DevQ router, gate, up, down, shg, shu, shd;
  const uint16_t* gamma;
  const float* lbias;
};

// Launch modes of the decode step.
constexpr int kStepFused = 0, kStepPhased = 1, kStepShared = 2, kStepRouted = 3;

__host__ __device__ inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

struct WsLayout {
  size_t ctl, logits, idx, w, act, act_stride, pf, total;
};

// Decode/FFN/router workspace for T tokens.  The gate/up activations of a
// decode step (shared [Is] then routed [K][I], fp32) are published in
// ctl::kRep replicas act_stride bytes apart.  Prefill extras start at `pf`.
__host__ __device__ inline WsLayout ws_layout(int E, int K, int I, int Is, int T) {
  WsLayout L;
  size_t o = 0;
  L.ctl = o; o += align256(kCtlBytes);
  L.logits = o; o += align256((size_t)T * E * 4);
  L.idx = o; o += align256((size_t)T * K * 4);
  L.w = o; o += align256((size_t)T * K * 4);
  L.act_stride = align256(((size_t)Is + (size_t)K * I) * 4) + 256;
  L.act = o; o += L.act_stride * ctl::kRep;
  L.pf = o;
  L.total = o;
  return L;
}

}  // namespace qmoe
