// qmoe_decode.hip -- decode-path kernels for gfx950: the 4-bit GEMV, the
// 8-bit router with softmax top-k, RMSNorm, and the MoE FFN step (shared +
// routed gate/up with GELU, down projections, router-weighted combine,
// residual) in one launch.
//
// The step (remio.ai "TurboFieldfare esegue Mac Gemma 4 26B in 2 GB…",
// section "L'affermazione dei 2 GB trasforma la larghezza di banda dell'SSD
// nel nuovo vincolo"; devtrends.cc "Come eseguire un modello da 26 miliardi…",
// section "Qual è il trucco principale dell'architettura"): per layer a router
// picks 8 experts for the token, the always-on shared expert runs alongside,
// and the two branches are combined.
//
// Decode is bound by HBM bandwidth (about 3.5 flop per weight byte), so the
// kernels are vector-memory GEMVs: 16-byte loads of packed codes that read
// 128 contiguous bytes per row per instruction, dequantization in registers,
// activations staged once per block in LDS, wave shuffles for row sums.  No
// matrix cores here.
//
// One decode step is one launch whose blocks take "roles", ordered so that a
// block only ever waits for blocks with smaller indices:
//   R  router: 8 experts per block; publishes its logits
//   S  shared-expert gate/up (+GELU): 4 row-blocks of 8 rows per block
//   G  routed-expert gate/up (+GELU): needs the routing
//   D  8 output rows per block: shared down rows as soon as S is done, then
//      each routed expert's down rows as soon as that expert's G blocks are
//      done; weighted combine, residual, bf16 output
// Every block that needs the routing computes the top-k itself from the
// published logits (no extra hop).  Workgroups are dispatched in index
// order, so a waiting block's producers have all been dispatched and never
// wait on it: every wait ends.  Each wait is also bounded in time and then
// reports a device error instead of hanging.
//
// Hand-offs: every producer block raises its own flag word to the call's
// tag, a value of the workspace's tag counter that no earlier call has
// used (the counter advances once every block of a call has read it);
// exchanged values travel as device-coherent stores/loads; small values
// that many blocks poll (router logits, flags, gate/up activations) are
// written in a few replicas so that pollers spread over memory channels.
// No cache fences; the only atomics are the counts that advance the tag
// counter (every block's registration in a fused one-layer call, the last
// role's completion counts otherwise).
//
// Every weight and scale load is unconditional (out-of-range chunks re-read
// a valid address and only the arithmetic is predicated) and, for the model
// shapes, every trip count is a compile-time constant: the compiler then
// waits for each load just before its first use, so the math of the first
// chunks overlaps the transfer of the last ones.
#include <hip/hip_ext.h>
#include <string.h>

#include "qmoe_common.h"
#include "qmoe_topk.h"

namespace qmoe {

constexpr int kSP = 11;          // gate/up steps per pass (runtime shapes)
constexpr int kMaxXW = 2;        // activation words per thread kept in registers
constexpr int kSR = 8;           // router steps per wave per pass (runtime shapes)
constexpr uint64_t kWaitTicks = 20000000ull;  // 0.2 s of the 100 MHz clock
// Blocks whose first weight loads are not on the critical path hold them
// back this long (100 MHz ticks), so the router's loads reach the memory
// queues first.
constexpr uint64_t kHoldTicks = 0;

// LDS "sys" words at the start of every block's LDS
constexpr int kSysOk = 1, kSysDone = 2, kSysIdx = 8, kSysW = 16, kSysRed = 32;
constexpr int kSysSlot = 24;  // stacked position of each routed expert
constexpr int kSysTkIdx = 96, kSysTkW = 160;  // per-wave top-k of the standalone router
constexpr int kSysXch = 96;    // top-k exchange slots (2k 64-bit words) of the step roles
constexpr int kSysWait = 184;  // stack kernel: 64-bit length of the last wait for a layer input
constexpr int kSysTrace = 128; // trace builds: kNStamp 64-bit phase timestamps
constexpr int kNStamp = 16;
constexpr int kSysBytes = 768;

// Trace builds (-DQMOE_TRACE) record per-block phase timestamps of the step
// kernel: s_memrealtime values (the 100 MHz constant clock, the same on every
// CU) kept in the block's LDS while it works, so that a stamp adds no memory
// operation, and written out when the block ends to
// qmoe_trace_buf[((G % slots) * blocks + block) * kNStamp + i] (G: the
// call's tag counter).  Stamp i is taken by lane 0 of the wave that reaches
// the phase named in the role that uses it (thread 0 takes every stamp);
// unused stamps stay 0.
#ifdef QMOE_TRACE
__device__ uint64_t* qmoe_trace_buf;
__device__ int qmoe_trace_slots;
#define QMOE_STAMP(sys, i)                                                              \
  do {                                                                                  \
    if (threadIdx.x == 0)                                                               \
      reinterpret_cast<uint64_t*>((sys) + kSysTrace)[i] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define QMOE_STAMP(sys, i) \
  do {                     \
  } while (0)
#endif
// Stamps: 0 block start; 1 first weight loads issued; 2 input staged (S,
// G) / logits computed (R) / routing known (D); 3 routing known (G) /
// logits published (R) / shared flags seen (D); 4 computed (S, G) / input
// staged (R) / shared staged (D); 5 published (S, G) / routed flags seen
// (D); 6 routed staged (D); 7 combined (D); 8 output stored (D); 9 block
// end; 10 routing seen (G, D: the poll that saw every tag returned); 11
// top-k done (G, D); 12-14 top-k select, gather, rank done (G, D).

__host__ __device__ inline size_t al16(size_t n) { return (n + 15) & ~(size_t)15; }

// ----------------------------------------------------------- arguments
struct DecodeArgs {
  int H, E, K, I, Is;
  DevQ router, gate, up, down, shg, shu, shd;
  const uint16_t* x;        // bf16 [H]: layer input (or expert input h)
  const uint16_t* gamma;    // bf16 [H] RMSNorm weight, or null
  float eps;
  const float* lbias;       // fp32 [E] or null
  const int32_t* idx_in;    // given routing or null (router runs)
  const float* w_in;
  const int32_t* slot;      // expert -> stacked position, or null
  const uint16_t* residual; // bf16 [H] or null
  uint16_t* out;
  int32_t* idx_out;         // optional copies of the routing
  float* w_out;
  uint8_t* ws;
  WsLayout wl;
  int nR, nS, nG, nD;       // role sizes in blocks
  int perG;                 // G blocks per expert
  int role0;                // role index of blockIdx.x == 0
  int nowait;               // 1: producers ran in earlier launches (no waits)
  int s_done;               // 1: the S blocks ran in an earlier launch
  int dwait;                // stack: output blocks of the previous layer to wait for
  uint32_t dtag;            // stack: their flag value
  int cnt;                  // role whose blocks count the call done: kCntNone/S/D
  uint32_t ntags;           // tag values the call uses (advance of the tag counter)
  int heal;                 // 1: a failed wait is cleared by the call's last block (no
                            // caller can read the error word of this workspace)
  int early;                // 1: the first shared block advances the tag counter once
                            // every block has registered (see early_advance)
};
constexpr int kCntNone = 0, kCntS = 1, kCntD = 2;

__device__ __forceinline__ uint32_t* ctl_of(const DecodeArgs& a) {
  return reinterpret_cast<uint32_t*>(a.ws + a.wl.ctl);
}
// Replica `r` of a published area at byte offset `base` of the control area.
__device__ __forceinline__ uint8_t* rep_of(const DecodeArgs& a, int base, int r) {
  return a.ws + a.wl.ctl + base + (size_t)r * ctl::kRepStride;
}
__device__ __forceinline__ float* logits_of(const DecodeArgs& a) {
  return reinterpret_cast<float*>(a.ws + a.wl.logits);
}
// Replica r of the activations: shared [Is], then routed [K][I].
__device__ __forceinline__ float* act_of(const DecodeArgs& a, int r) {
  return reinterpret_cast<float*>(a.ws + a.wl.act + (size_t)r * a.wl.act_stride);
}

// --------------------------------------------------------------- waits
// The workspace's tag counter G (see ctl::kGenBase): a one-layer call
// matches its flags and tags against G + 1, a stack call layer l's against
// G + 1 + l.  Every value ever written to a flag or tag of the workspace
// is <= G, so stale words never match.  Read device-coherently from this
// block's replica.
__device__ __forceinline__ uint32_t load_gen(const uint8_t* ws, size_t ctl_off) {
  return ld_dev(reinterpret_cast<const uint32_t*>(ws + ctl_off + ctl::kGenBase +
                                                  ctl::kGenStride * (blockIdx.x % ctl::kGenRep)));
}

// Zero every flag and tag replica and restart the tag counter (the counter
// is about to leave its range).  Only the last block of a call runs this,
// when no block of the call reads the control area any more.
__device__ void ctl_restart(uint8_t* ws, size_t ctl_off, int E, int tid = threadIdx.x) {
  uint8_t* c = ws + ctl_off;
  for (int r = 0; r < ctl::kRep; ++r) {
    uint64_t* tg = reinterpret_cast<uint64_t*>(c + ctl::kTagBase + (size_t)r * ctl::kRepStride);
    uint32_t* fl = reinterpret_cast<uint32_t*>(c + ctl::kFlagBase + (size_t)r * ctl::kRepStride);
    for (int i = tid; i < E; i += kBlock) st_dev(tg + i, (uint64_t)0);
    for (int i = tid; i < ctl::kMaxFlags; i += kBlock) st_dev(fl + i, 0u);
  }
  wait_vm();
  __syncthreads();
  if (tid < ctl::kGenRep)
    st_dev(reinterpret_cast<uint32_t*>(c + ctl::kGenBase + ctl::kGenStride * tid), 0u);
}

// The call's tags are used up: G += n in every replica, or a restart when G
// would leave its range.  Whole block, by its last block only.
__device__ void gen_advance(uint8_t* ws, size_t ctl_off, int E, uint32_t gen, uint32_t n,
                            int tid = threadIdx.x) {
  if (gen + n >= ctl::kGenLimit) {
    ctl_restart(ws, ctl_off, E, tid);
    return;
  }
  if (tid < ctl::kGenRep)
    st_dev(reinterpret_cast<uint32_t*>(ws + ctl_off + ctl::kGenBase + ctl::kGenStride * tid),
           gen + n);
}

// Block i of the n blocks of the role whose completion ends a one-layer
// call (every block of the call has read the tag counter when all of them
// are done, whether their waits completed or not): count it; the last one
// advances the counter by the call's tags.  Counters per group of blocks
// (i % kGenRep), then one for the groups, so that few atomics meet on one
// address.  After a failed wait the counter stays (qmoe_workspace_status
// restarts the control area), or with `heal` the last block restarts it and
// clears the error word itself.  Whole block.
__device__ void call_done(const DecodeArgs& a, int i, int n, uint32_t gen, uint32_t* sys,
                          int tid = threadIdx.x) {
  if (tid == 0) {
    uint8_t* c = a.ws + a.wl.ctl + ctl::kCntBase;
    const int g = i % ctl::kGenRep;
    const uint32_t ng = (uint32_t)((n - g + ctl::kGenRep - 1) / ctl::kGenRep);
    const uint32_t ngroups = (uint32_t)min(n, ctl::kGenRep);
    uint32_t* cg = reinterpret_cast<uint32_t*>(c + 64 * (ctl::kCntDone + g));
    uint32_t last = 0;
    if (add_dev(cg, 1u) == ng - 1) {
      st_dev(cg, 0u);
      uint32_t* top = reinterpret_cast<uint32_t*>(c + 64 * ctl::kCntDoneTop);
      if (add_dev(top, 1u) == ngroups - 1) {
        st_dev(top, 0u);
        last = 1;
      }
    }
    sys[kSysDone] = last;
  }
  __syncthreads();
  if (!sys[kSysDone]) return;
  uint32_t* err = reinterpret_cast<uint32_t*>(a.ws + a.wl.ctl) + ctl::kError;
  if (ld_dev(err) == 0) {
    gen_advance(a.ws, a.wl.ctl, a.E, gen, a.ntags, tid);
  } else if (a.heal) {
    ctl_restart(a.ws, a.wl.ctl, a.E, tid);
    if (tid == 0) st_dev(err, 0u);
  }
}

constexpr int kPollSleep = 1;  // s_sleep units (64 cycles) between polls: a poll is a round trip
                               // already (decode step: 0, 1, 2, 6 units gave 19.79, 19.81,
                               // 19.85, 20.02 us)

// Early advance of the tag counter (a one-layer call with every role in one
// launch and shared blocks): each block, once it has used the call's tag
// (so that its read of the counter is complete), adds 1 to the done count
// of its group (block index % kGenRep), without waiting for the atomic; the
// first shared block, after its own publication, waits until the groups'
// counts add up to the launch's blocks, zeroes them and advances the
// counter.  Every block has read the counter by then, so the advance is the
// same one the output blocks' completion count would make at the end, but
// it is off the call's critical path: the output blocks end right after
// their stores.  Near the top of the counter's range the restart must wait
// until no block reads the control area any more: such a call counts at the
// end as the other modes do.
__device__ __forceinline__ bool early_on(const DecodeArgs& a, uint32_t gen) {
  return a.early && gen + a.ntags < ctl::kGenLimit;
}
__device__ __forceinline__ void call_register(const DecodeArgs& a, uint32_t epoch,
                                              int tid = threadIdx.x) {
  if (tid == 0) {
    uint32_t one = 1u;
    asm volatile("" : "+v"(one) : "v"(epoch));  // issued after the tag's load returned
    uint32_t* c = reinterpret_cast<uint32_t*>(a.ws + a.wl.ctl + ctl::kCntBase +
                                              64 * (ctl::kCntDone + blockIdx.x % ctl::kGenRep));
    (void)__hip_atomic_fetch_add(c, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}
// The first shared block, whole block: wait (bounded) for every block's
// registration, then zero the counts and raise the counter by the call's
// tags.  A wait that gives up sets the error word (code 5) and leaves the
// counter (qmoe_workspace_status restarts the control area).
__device__ void early_advance(const DecodeArgs& a, uint32_t gen, int tid = threadIdx.x) {
  if (tid == 0) {
    uint8_t* c = a.ws + a.wl.ctl;
    uint32_t* cnt = reinterpret_cast<uint32_t*>(c + ctl::kCntBase + 64 * ctl::kCntDone);
    uint32_t* err = reinterpret_cast<uint32_t*>(c) + ctl::kError;
    const uint32_t total = gridDim.x;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    bool ok = true;
    for (int it = 0;; ++it) {
      uint32_t v[ctl::kGenRep], n = 0;  // every load issued before the sum
#pragma unroll
      for (int g = 0; g < ctl::kGenRep; ++g) v[g] = ld_dev(cnt + 16 * g);
#pragma unroll
      for (int g = 0; g < ctl::kGenRep; ++g) n += v[g];
      if (n == total) break;
      if ((it & 15) == 15) {
        if (ld_dev(err) != 0 || __builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
          if (ld_dev(err) == 0) st_dev(err, 5u);
          ok = false;
          break;
        }
      }
      __builtin_amdgcn_s_sleep(kPollSleep);
    }
    if (ok) {
#pragma unroll
      for (int g = 0; g < ctl::kGenRep; ++g) {
        st_dev(cnt + 16 * g, 0u);
        st_dev(reinterpret_cast<uint32_t*>(c + ctl::kGenBase + ctl::kGenStride * g),
               gen + a.ntags);
      }
    }
  }
}

// One full wave: wait until flags[0..n) all equal `epoch`.  Every poll reads
// all n flags at once (a few loads per lane), so the wait ends one round
// trip after the last flag is raised.
__device__ bool wave_wait_flags(const uint32_t* flags, int n, uint32_t epoch, uint32_t* ctlw,
                                uint32_t code, int tid = threadIdx.x) {
  const int lane = tid & 63;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  // a polling wave issues ahead of the bulk weight loads of its CU
  __builtin_amdgcn_s_setprio(2);
  for (int it = 0;; ++it) {
    {
      uint32_t bad = 0;  // every load issued before the first compare
      for (int i = lane; i < n; i += 64) bad |= ld_dev(flags + i) ^ epoch;
      if (__all(bad == 0)) {
        __builtin_amdgcn_s_setprio(0);
        return true;
      }
    }
    if ((it & 15) == 15) {
      if (ld_dev(ctlw + ctl::kError) != 0) return false;
      if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
        if (lane == 0) st_dev(ctlw + ctl::kError, code);
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(kPollSleep);
  }
}

// Spin until `ticks` of the constant clock have passed since `t0`.
__device__ __forceinline__ void hold_until(uint64_t t0, uint64_t ticks) {
  while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) __builtin_amdgcn_s_sleep(1);
}

// Whole block: wave `pw` waits, the others meet it at a barrier.
__device__ bool block_wait_flags(const uint32_t* flags, int n, uint32_t epoch, uint32_t* ctlw,
                                 uint32_t code, uint32_t* sys, int pw = 0, int tid = threadIdx.x) {
  if ((int)(tid >> 6) == pw) {
    bool ok = wave_wait_flags(flags, n, epoch, ctlw, code, tid);
    if ((tid & 63) == 0) sys[kSysOk] = ok ? 1u : 0u;
  }
  __syncthreads();
  bool ok = sys[kSysOk] != 0;
  __syncthreads();
  return ok;
}

// This block's device stores are complete: raise its flag (word `flag` of
// every flag replica).
__device__ void block_publish(const DecodeArgs& a, int flag, uint32_t epoch, int tid = threadIdx.x) {
  wait_vm();
  __syncthreads();
  if (tid < ctl::kRep)
    st_dev(reinterpret_cast<uint32_t*>(rep_of(a, ctl::kFlagBase, tid)) + flag, epoch);
}

// Stack layers: the whole block waits until every output block of the
// previous layer has published (its rows of this layer's input are then
// readable device-coherently).  Wave `pw` polls, but only after three
// quarters of its previous wait for a layer input have passed: the flags
// cannot rise much sooner, and the polls of several hundred waiting blocks
// would otherwise load the memory system while the output blocks stage
// their activations.
__device__ bool wait_prev_layer(const DecodeArgs& a, uint32_t* sys, int pw, int tid = threadIdx.x) {
  if (!a.dwait) return true;
  const uint32_t* flags =
      reinterpret_cast<const uint32_t*>(rep_of(a, ctl::kFlagBase, blockIdx.x % ctl::kRep)) +
      a.nS + a.nG;
  if ((int)(tid >> 6) == pw) {
    uint64_t* last = reinterpret_cast<uint64_t*>(sys + kSysWait);
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    hold_until(t0, *last / 4 * 3);
    bool ok = wave_wait_flags(flags, a.dwait, a.dtag, ctl_of(a), 4, tid);
    if ((tid & 63) == 0) {
      *last = __builtin_amdgcn_s_memrealtime() - t0;
      sys[kSysOk] = ok ? 1u : 0u;
    }
  }
  __syncthreads();
  bool ok = sys[kSysOk] != 0;
  __syncthreads();
  return ok;
}

// Values made opaque to the compiler where they are used inside the layer
// loop of the stack kernel, so that address arithmetic derived from them is
// recomputed per layer instead of being hoisted out of the loop and held in
// registers across it.
__device__ __forceinline__ void opaque_s(int& v) { asm volatile("" : "+s"(v)); }
__device__ __forceinline__ void opaque_v(int& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  opaque_v(t);
  return t;
}

struct NoPre {
  __device__ void operator()() const {}
};

// ------------------------------------------------------------ reductions
// Block-wide sum of one float per thread (fixed order; same bits everywhere).
__device__ float block_sum(float v, float* red, int tid = threadIdx.x) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  int wave = tid >> 6;
  __syncthreads();
  if ((tid & 63) == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < kWavesPerBlock; ++i) s += red[i];
  return s;
}

// ============================================================== routing
// One wave: wait until all E tagged logits of one replica carry `epoch`
// (each is (epoch << 32) | fp32 bits, written with one 64-bit store), then
// top-k on them.  Every poll reads all of them.  In a launch that follows
// its producers, no waiting.
template <int NV>
__device__ bool wave_routing(const DecodeArgs& a, uint32_t epoch, int32_t* idx_s, float* w_s,
                             bool write_out, uint64_t* xch, uint32_t* sys, int tid = threadIdx.x) {
  (void)sys;
  const int lane = tid & 63;
  const uint64_t* tag = reinterpret_cast<const uint64_t*>(
      rep_of(a, ctl::kTagBase, blockIdx.x % ctl::kRep));
  uint32_t* ctlw = ctl_of(a);
  float v[NV];
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  __builtin_amdgcn_s_setprio(2);  // issue ahead of the CU's bulk weight loads
  for (int it = 0;; ++it) {
    bool ok = true;
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int e = lane + 64 * m;
      const uint64_t t = ld_dev(tag + min(e, a.E - 1));
      v[m] = __uint_as_float((uint32_t)t);
      ok = ok && (a.nowait || (uint32_t)(t >> 32) == epoch);
    }
    if (__all(ok)) break;
    if ((it & 15) == 15) {
      if (ld_dev(ctlw + ctl::kError) != 0) return false;
      if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
        if (lane == 0) st_dev(ctlw + ctl::kError, 1u);
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(kPollSleep);
  }
  QMOE_STAMP(sys, 10);
  // the selection runs at the polling priority: it is on every consumer's
  // critical path
#ifdef QMOE_TRACE
  uint64_t* tstamps = tid == 0 ? reinterpret_cast<uint64_t*>(sys + kSysTrace) + 12 : nullptr;
#else
  uint64_t* tstamps = nullptr;
#endif
  wave_topk_radix<NV>(v, a.E, a.K, idx_s, w_s, write_out ? a.idx_out : nullptr,
                      write_out ? a.w_out : nullptr, xch, tid, tstamps);
  __builtin_amdgcn_s_setprio(0);
  return true;
}

// Routing for a consumer block: from the caller's arrays, or from the
// router blocks' published logits.  Leaves idx/w in sys LDS, and each
// routed expert's stacked position (through the expert -> slot map, if
// any) in sys[kSysSlot + j], so that no consumer waits on that lookup.
template <int NV>
__device__ bool block_routing(const DecodeArgs& a, uint32_t epoch, uint32_t* sys, bool write_out,
                              int tid = threadIdx.x) {
  int32_t* idx_s = reinterpret_cast<int32_t*>(sys + kSysIdx);
  float* w_s = reinterpret_cast<float*>(sys + kSysW);
  int32_t* slot_s = reinterpret_cast<int32_t*>(sys + kSysSlot);
  if (a.idx_in) {
    if (tid < a.K) {
      const int e = gptr(a.idx_in)[tid];
      idx_s[tid] = e;
      w_s[tid] = gptr(a.w_in)[tid];
      slot_s[tid] = a.slot ? gptr(a.slot)[e] : e;
    }
    __syncthreads();
    return true;
  }
  if (tid < 64) {
    bool ok = wave_routing<NV>(a, epoch, idx_s, w_s, write_out,
                               reinterpret_cast<uint64_t*>(sys + kSysXch), sys, tid);
    QMOE_STAMP(sys, 11);
    if (ok && tid < a.K) {
      const int e = idx_s[tid];
      slot_s[tid] = a.slot ? gptr(a.slot)[e] : e;
    }
    if (tid == 0) sys[kSysOk] = ok ? 1u : 0u;
  }
  __syncthreads();
  bool ok = sys[kSysOk] != 0;
  __syncthreads();
  return ok;
}

// -------------------------------------------------------------- staging
// Eight bf16 values (one uint4) of the expert input: x as is, or
// bf16(x * inv * gamma).
__device__ __forceinline__ uint4 norm_word(uint4 r, const uint16_t* gamma, float inv, int v) {
  if (!gamma) return r;
  uint4 g = ld_g16(gamma, v);
  uint32_t xr[4] = {r.x, r.y, r.z, r.w}, gr[4] = {g.x, g.y, g.z, g.w}, o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo = bf16_to_f32(xr[i] & 0xffffu) * inv * bf16_to_f32(gr[i] & 0xffffu);
    float hi = bf16_to_f32(xr[i] >> 16) * inv * bf16_to_f32(gr[i] >> 16);
    o[i] = (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// The activation words of this thread, loaded first so that nothing issued
// later has to complete before they can be staged.
struct XRegs {
  uint4 w[kMaxXW];
};
__device__ __forceinline__ void x_load(XRegs& X, const uint16_t* x, int H, int tid = threadIdx.x) {
  const int Wn = H / 8;
#pragma unroll
  for (int i = 0; i < kMaxXW; ++i) X.w[i] = ld_g16(x, min(tid + i * kBlock, Wn - 1));
}

// The same words read device-coherently: the layer input of a stack layer
// was written by other blocks of the launch.
__device__ __forceinline__ void x_load_dev(XRegs& X, const uint16_t* x, int H, int tid = threadIdx.x) {
  const float* xf = reinterpret_cast<const float*>(x);
  const int Wn = H / 8;
#pragma unroll
  for (int i = 0; i < kMaxXW; ++i) {
    const uint32_t v = (uint32_t)min(tid + i * kBlock, Wn - 1);
    X.w[i] = __builtin_bit_cast(uint4, ld_dev16(xf, (uint32_t)H * 2, v * 16));
  }
}

__device__ float x_inv_rms(const XRegs& X, const uint16_t* x, int H, float eps, float* red, int tid = threadIdx.x) {
  float ss = 0.f;
  const int Wn = H / 8;
  for (int i = 0; i * kBlock < Wn; ++i) {
    int v = tid + i * kBlock;
    if (v >= Wn) break;
    uint4 w;
    if (i < kMaxXW) {
      w = X.w[0];
#pragma unroll
      for (int k = 1; k < kMaxXW; ++k)
        if (i == k) w = X.w[k];
    } else {
      w = ld_g16(x, v);
    }
    uint32_t r[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float lo = bf16_to_f32(r[k] & 0xffffu), hi = bf16_to_f32(r[k] >> 16);
      ss = fmaf(lo, lo, ss);
      ss = fmaf(hi, hi, ss);
    }
  }
  ss = block_sum(ss, red, tid);
  return 1.0f / sqrtf(ss / (float)H + eps);
}

// Word v's eight bf16 values -> the dot2 pair layout xs[j*CH + c] (v = 4c+j)
// and chunk sums xh[c].
__device__ __forceinline__ void put_pairs(uint4 r, int v, bool ok, int CH, uint4* xs, float* xh) {
  uint4 pr;
  pr.x = (r.x & 0xffffu) | (r.y << 16);          // x0, x2
  pr.y = (r.z & 0xffffu) | (r.w << 16);          // x4, x6
  pr.z = (r.x >> 16) | (r.y & 0xffff0000u);      // x1, x3
  pr.w = (r.z >> 16) | (r.w & 0xffff0000u);      // x5, x7
  float s = ((bf16_to_f32(r.x & 0xffffu) + bf16_to_f32(r.x >> 16)) +
             (bf16_to_f32(r.y & 0xffffu) + bf16_to_f32(r.y >> 16))) +
            ((bf16_to_f32(r.z & 0xffffu) + bf16_to_f32(r.z >> 16)) +
             (bf16_to_f32(r.w & 0xffffu) + bf16_to_f32(r.w >> 16)));
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  if (ok) {
    int c = v >> 2, j = v & 3;
    xs[j * CH + c] = pr;
    if (j == 0) xh[c] = s;
  }
}

// Word v's values -> router layout xr[j*CH8 + c] (fp32, column order), sums.
__device__ __forceinline__ void put_f32(uint4 r, int v, bool ok, int CH8, float4* xr, float* xh) {
  float4 f0 = make_float4(bf16_to_f32(r.x & 0xffffu), bf16_to_f32(r.x >> 16),
                          bf16_to_f32(r.y & 0xffffu), bf16_to_f32(r.y >> 16));
  float4 f1 = make_float4(bf16_to_f32(r.z & 0xffffu), bf16_to_f32(r.z >> 16),
                          bf16_to_f32(r.w & 0xffffu), bf16_to_f32(r.w >> 16));
  float s = ((f0.x + f0.y) + (f0.z + f0.w)) + ((f1.x + f1.y) + (f1.z + f1.w));
  s += __shfl_xor(s, 1);
  if (ok) {
    int c = v >> 1, j = (v & 1) * 2;
    xr[j * CH8 + c] = f0;
    xr[(j + 1) * CH8 + c] = f1;
    if ((v & 1) == 0) xh[c] = s;
  }
}

// Stage the expert input h into LDS (pairs layout or router layout).  The
// words held in X are used; words beyond kMaxXW per thread are loaded here.
template <bool PAIRS>
__device__ void x_stage(const XRegs& X, const uint16_t* x, const uint16_t* gamma, float inv, int H,
                        void* dst, float* xh, int tid = threadIdx.x) {
  const int Wn = H / 8;
#pragma unroll
  for (int i = 0; i < kMaxXW; ++i) {
    if (i * kBlock < Wn) {
      int v = tid + i * kBlock;
      bool ok = v < Wn;
      uint4 r = ok ? norm_word(X.w[i], gamma, inv, v) : make_uint4(0, 0, 0, 0);
      if (PAIRS)
        put_pairs(r, v, ok, H / 32, reinterpret_cast<uint4*>(dst), xh);
      else
        put_f32(r, v, ok, H / 16, reinterpret_cast<float4*>(dst), xh);
    }
  }
  for (int i = kMaxXW; i * kBlock < Wn; ++i) {
    int v = tid + i * kBlock;
    bool ok = v < Wn;
    uint4 r = ok ? norm_word(ld_g16(x, v), gamma, inv, v) : make_uint4(0, 0, 0, 0);
    if (PAIRS)
      put_pairs(r, v, ok, H / 32, reinterpret_cast<uint4*>(dst), xh);
    else
      put_f32(r, v, ok, H / 16, reinterpret_cast<float4*>(dst), xh);
  }
}

// ------------------------------------------------- 4-bit row-block GEMV
// NM matrices with the same shape and the same input (gate and up) share
// the staged activations.  Each wave owns a row-block of 8 rows; its
// scale/bias pairs go through a wave-private LDS table sbl[k][8][G] of
// (s | b << 16), filled with one 16-byte load of s and one of b per lane.
// SP: steps per pass (8 chunks per step); CHC: chunks per row when known at
// compile time (0: runtime, passes of SP steps).
template <int NM, int SP>
struct Rows4 {
  uint4 w[NM][SP];
  uint4 sv[NM], bv[NM];
};

// Scale units (8 fp16 each) of the row-block; the load is unconditional,
// lanes past the row-block's units re-read its last one.
template <int NM, int SP>
__device__ __forceinline__ void rows4_load_sb(Rows4<NM, SP>& R, const DevQ (&m)[NM], int row0,
                                              int rows, int G, int tid = threadIdx.x) {
  const int lane = tid & 63;
  const int64_t total = (int64_t)rows * G / 8;          // whole units in the array
  const int64_t first = (int64_t)min(row0, rows - 1) * G / 8;
  const int64_t u = min(first + min(lane, G - 1), total - 1);
#pragma unroll
  for (int k = 0; k < NM; ++k) {
    R.sv[k] = ld_g16(m[k].s, u);
    R.bv[k] = ld_g16(m[k].b, u);
  }
}

__device__ __forceinline__ void put_sb8(uint4 sv, uint4 bv, uint32_t* dst) {
  uint4 lo, hi;
  lo.x = (sv.x & 0xffffu) | (bv.x << 16);
  lo.y = (sv.x >> 16) | (bv.x & 0xffff0000u);
  lo.z = (sv.y & 0xffffu) | (bv.y << 16);
  lo.w = (sv.y >> 16) | (bv.y & 0xffff0000u);
  hi.x = (sv.z & 0xffffu) | (bv.z << 16);
  hi.y = (sv.z >> 16) | (bv.z & 0xffff0000u);
  hi.z = (sv.w & 0xffffu) | (bv.w << 16);
  hi.w = (sv.w >> 16) | (bv.w & 0xffff0000u);
  reinterpret_cast<uint4*>(dst)[0] = lo;
  reinterpret_cast<uint4*>(dst)[1] = hi;
}

// Fill the table.  The fast path covers row-blocks of 8 whole rows with
// G <= 64 (one unit per lane); otherwise pairs are copied one by one.
template <int NM, int SP>
__device__ __forceinline__ void rows4_put_sb(const Rows4<NM, SP>& R, const DevQ (&m)[NM], int row0,
                                             int rows, int G, uint32_t* sbl, int tid = threadIdx.x) {
  const int lane = tid & 63;
  const int nr = max(0, min(kRowsPerUnit, rows - row0));
  const bool fast = nr == kRowsPerUnit && G <= 64;
#pragma unroll
  for (int k = 0; k < NM; ++k) {
    uint32_t* t = sbl + k * kRowsPerUnit * G;
    if (fast) {
      if (lane < G) put_sb8(R.sv[k], R.bv[k], t + 8 * lane);
    } else {
      const QMOE_GLOBAL uint16_t* s = gptr(m[k].s + (int64_t)row0 * G);
      const QMOE_GLOBAL uint16_t* b = gptr(m[k].b + (int64_t)row0 * G);
      for (int h = lane; h < nr * G; h += 64) t[h] = (uint32_t)s[h] | ((uint32_t)b[h] << 16);
    }
  }
}

template <int NM, int SP>
__device__ __forceinline__ void rows4_load(Rows4<NM, SP>& R, const DevQ (&m)[NM], int row,
                                           int CH, int c0, int CW, int step0, int p) {
#pragma unroll
  for (int i = 0; i < SP; ++i) {
    int c = c0 + min((step0 + i) * kSlots + p, CW - 1);
    int64_t o = ((int64_t)row * CH + c) * 16;
#pragma unroll
    for (int k = 0; k < NM; ++k) R.w[k][i] = ldg16(m[k].q + o);
  }
}

template <int NM, int SP>
__device__ __forceinline__ void rows4_compute(const Rows4<NM, SP>& R, const uint4* xs,
                                              const float* xh, const uint32_t* sbl, int r, int G,
                                              int CH, int c0, int CW, int step0, int p,
                                              float (&acc)[NM]) {
#pragma unroll
  for (int i = 0; i < SP; ++i) {
    int cl = (step0 + i) * kSlots + p;
    if (cl < CW) {
      int c = c0 + cl;
      uint4 x0 = xs[c], x1 = xs[CH + c], x2 = xs[2 * CH + c], x3 = xs[3 * CH + c];
      float X = xh[c];
#pragma unroll
      for (int k = 0; k < NM; ++k) {
        uint32_t sb = sbl[(k * kRowsPerUnit + r) * G + (c >> 1)];
        float d = 0.f;
        d = dot_word4_bf16(R.w[k][i].x, x0, d);
        d = dot_word4_bf16(R.w[k][i].y, x1, d);
        d = dot_word4_bf16(R.w[k][i].z, x2, d);
        d = dot_word4_bf16(R.w[k][i].w, x3, d);
        acc[k] = fmaf(half_to_f32(sb & 0xffffu), d, acc[k]);
        acc[k] = fmaf(half_to_f32(sb >> 16), X, acc[k]);
      }
    }
  }
}

// One wave: rows [row0, row0+8) of NM matrices of `rows` rows and H columns,
// chunks [c0, c0+CW) of each row (CWC: CW when known at compile time).
// `stage` runs between the first pass's loads and its math and must end
// with a block barrier.  sbl: this wave's LDS table (NM*8*G words).
template <int NM, int CWC, typename StageFn>
__device__ __forceinline__ void rows4_run(const DevQ (&m)[NM], int row0, int rows, int H, int c0,
                                          int CW_rt, const uint4* xs, const float* xh,
                                          uint32_t* sbl, StageFn stage, float (&acc)[NM], int tid = threadIdx.x) {
  constexpr int SP = CWC ? cdiv(CWC, kSlots) : kSP;
  const int CW = CWC ? CWC : CW_rt;
  const int CH = H / 32, G = CH / 2, nsteps = cdiv(CW, kSlots);
  const int lane = tid & 63, r = lane & 7, p = lane >> 3;
  const int row = min(row0 + r, rows - 1);
  Rows4<NM, SP> R;
#pragma unroll
  for (int k = 0; k < NM; ++k) acc[k] = 0.f;
  rows4_load_sb<NM, SP>(R, m, row0, rows, G, tid);
  rows4_load<NM, SP>(R, m, row, CH, c0, CW, 0, p);
  rows4_put_sb<NM, SP>(R, m, row0, rows, G, sbl, tid);
  stage();
  rows4_compute<NM, SP>(R, xs, xh, sbl, r, G, CH, c0, CW, 0, p, acc);
  if (!CWC) {
    for (int s0 = SP; s0 < nsteps; s0 += SP) {
      rows4_load<NM, SP>(R, m, row, CH, c0, CW, s0, p);
      rows4_compute<NM, SP>(R, xs, xh, sbl, r, G, CH, c0, CW, s0, p, acc);
    }
  }
#pragma unroll
  for (int k = 0; k < NM; ++k) acc[k] = rowblock_sum(acc[k]);
}

// LDS carve-ups (bytes).  Gate/up: sys | xs pairs (H*2) | xh (H/32 floats)
// | per-wave scale tables (4 waves x 16 rows x H/64 words).
__host__ __device__ inline size_t gu_xh_off(int H) { return kSysBytes + (size_t)H * 2; }
__host__ __device__ inline size_t gu_sb_off(int H) { return al16(gu_xh_off(H) + (size_t)(H / 32) * 4); }
// (room for two row-blocks: the step's gate/up waves hold 16 rows)
__host__ __device__ inline size_t gu_sb_words(int H) { return (size_t)2 * kRowsPerUnit * (H / 64); }
__host__ __device__ inline size_t gu_lds(int H) {
  return gu_sb_off(H) + (size_t)kWavesPerBlock * gu_sb_words(H) * 4;
}
__host__ __device__ inline size_t router_lds(int H) {
  return kSysBytes + (size_t)H * 4 + (size_t)(H / 16) * 4;
}
// Down: sys | a_s (Is floats) | a_k (K x I floats) | chunk sums of a_s
// (Is/32) | chunk sums of a_k (K x I/32): every activation of the step.
__host__ __device__ inline size_t down_ah_off(int I, int Is, int K) {
  return kSysBytes + ((size_t)Is + (size_t)K * I) * 4;
}
__host__ __device__ inline size_t down_lds(int I, int Is, int K) {
  return down_ah_off(I, Is, K) + ((size_t)Is + (size_t)K * I) / 32 * 4;
}

// ======================================================= qmoe_gemv_affine4
template <int CHC>
__global__ __launch_bounds__(kBlock) void k_gemv4(DevQ W, int rows, int cols, const uint16_t* x,
                                                  float* y) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint4* xs = reinterpret_cast<uint4*>(smem + kSysBytes);
  float* xh = reinterpret_cast<float*>(smem + gu_xh_off(cols));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t* sbl = reinterpret_cast<uint32_t*>(smem + gu_sb_off(cols)) + wave * gu_sb_words(cols);
  const int row0 = (blockIdx.x * kWavesPerBlock + wave) * kRowsPerUnit;
  XRegs X;
  x_load(X, x, cols);
  DevQ m[1] = {W};
  float acc[1];
  rows4_run<1, CHC>(m, row0, rows, cols, 0, cols / 32, xs, xh, sbl,
                    [&] {
                      x_stage<true>(X, x, nullptr, 1.f, cols, xs, xh);
                      __syncthreads();
                    },
                    acc);
  if ((lane >> 3) == 0 && row0 + (lane & 7) < rows) y[row0 + (lane & 7)] = acc[0];
}

// =================================================== tiled 4-bit layout
// The same affine 4-bit matrix repacked offline (qmoe_repack_tiled4) so
// that every wave load of a row-block is one contiguous 1 KiB segment:
//   codes  [RB][CH][8][16 B]  row-block rb, chunk c (32 codes), row r of
//                             the block: the MLX row's bytes 16c..16c+16
//   pairs  [RB][8][G] u32     (scale | bias << 16), fp16 bits, group g
// RB = ceil(rows / 8), CH = cols / 32, G = cols / 64; rows past `rows` are
// zero.  Step i of a row-block is chunks 8i..8i+8 of its 8 rows: lane
// (r = lane & 7, p = lane >> 3) reads tile bytes 16 lane of that 1 KiB.
// The pairs of a row-block are the kernel's LDS table as stored.
__host__ __device__ inline size_t tiled4_code_bytes(int rows, int cols) {
  return (size_t)cdiv(rows, kRowsPerUnit) * (cols / 32) * kRowsPerUnit * 16;
}
__host__ __device__ inline size_t tiled4_bytes(int rows, int cols) {
  return tiled4_code_bytes(rows, cols) +
         (size_t)cdiv(rows, kRowsPerUnit) * kRowsPerUnit * (cols / 64) * 4;
}

// One wave: RBW consecutive row-blocks, one after the other (one register
// set: the next row-block's loads are issued when the previous one's math
// is done).  Per row-block the pairs go straight from memory into the
// wave's LDS table (global_load_lds: 16 bytes per lane at table + 16 lane,
// no registers; the table area holds whole 64-lane writes, later lanes
// repeat the last unit), then the codes are issued; waiting for all but
// the SP code loads waits for the pairs (loads complete in issue order).
// x is staged once per block, after the first row-block's loads.  The math
// is the MLX-layout GEMV's (same operations in the same order, same bits).
// RBW = 2 gives half the blocks for the same rows: one x staging for more
// rows, and a grid that fits the resident slots in fewer rounds.
template <int CHC>
__host__ __device__ constexpr int gemv4t_table_units() { return 64 * cdiv(CHC, 64); }
__host__ __device__ inline size_t gemv4t_lds(int cols) {
  return gu_sb_off(cols) + (size_t)kWavesPerBlock * 64 * cdiv(cols / 32, 64) * 16;
}
template <int CHC, int RBW>
__global__ __launch_bounds__(kBlock, RBW == 2 ? 4 : 1) void k_gemv4t(const uint8_t* T, int rows,
                                                                     int cols, const uint16_t* x,
                                                                     float* y) {
  constexpr int CH = CHC, G = CHC / 2, SP = cdiv(CHC, kSlots);
  constexpr int NU = cdiv(2 * G, 64);  // 16-byte units of pairs per lane and row-block
  constexpr int kWaitPairs = (SP & 15) | (7 << 4) | (15 << 8) | ((SP >> 4) << 14);
  extern __shared__ __align__(16) uint8_t smem[];
  uint4* xs = reinterpret_cast<uint4*>(smem + kSysBytes);
  float* xh = reinterpret_cast<float*>(smem + gu_xh_off(cols));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 7, p = lane >> 3;
  uint32_t* sbl = reinterpret_cast<uint32_t*>(smem + gu_sb_off(cols)) +
                  wave * gemv4t_table_units<CHC>() * 4;
  const int RB = cdiv(rows, kRowsPerUnit);
  const int rb0 = (blockIdx.x * kWavesPerBlock + wave) * RBW;
  const uint4* pairs = reinterpret_cast<const uint4*>(T + tiled4_code_bytes(rows, cols));
  Rows4<1, SP> R;
  auto load = [&](int j) {
    const int rb = min(rb0 + j, RB - 1);
#pragma unroll
    for (int u = 0; u < NU; ++u)
      __builtin_amdgcn_global_load_lds(
          (const QMOE_GLOBAL void*)(pairs + (int64_t)rb * 2 * G + min(lane + 64 * u, 2 * G - 1)),
          (__attribute__((address_space(3))) void*)(sbl + 256 * u), 16, 0, 0);
    const uint8_t* tile = T + (size_t)rb * CH * kRowsPerUnit * 16;
#pragma unroll
    for (int i = 0; i < SP; ++i) {
      const int c = min(i * kSlots + p, CH - 1);
      R.w[0][i] = ldg16(tile + ((size_t)c * kRowsPerUnit + r) * 16);
    }
  };
  auto math = [&](int j) {
    float acc[1] = {0.f};
    rows4_compute<1, SP>(R, xs, xh, sbl, r, G, CH, 0, CH, 0, p, acc);
    acc[0] = rowblock_sum(acc[0]);
    const int row = (rb0 + j) * kRowsPerUnit + r;
    if (p == 0 && rb0 + j < RB && row < rows) y[row] = acc[0];
  };
  {
    XRegs X;
    x_load(X, x, cols);
    load(0);
    __builtin_amdgcn_s_waitcnt(kWaitPairs);  // x and the pairs
    x_stage<true>(X, x, nullptr, 1.f, cols, xs, xh);
    __syncthreads();
    math(0);
  }
#pragma unroll 1
  for (int j = 1; j < RBW; ++j) {
    // the table is this wave's own: every lane's reads of the previous one
    // are done before the new pairs land
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    load(j);
    __builtin_amdgcn_s_waitcnt(kWaitPairs);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    math(j);
  }
}

// ============================================================= RMSNorm
__global__ __launch_bounds__(kBlock) void k_rmsnorm(const uint16_t* x, const uint16_t* gamma,
                                                    float eps, int H, uint16_t* out) {
  __shared__ float red[kWavesPerBlock];
  const uint16_t* xt = x + (size_t)blockIdx.x * H;
  const uint4* x4 = reinterpret_cast<const uint4*>(xt);
  float ss = 0.f;
  for (int v = threadIdx.x; v < H / 8; v += kBlock) {
    uint4 r = x4[v];
    uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float lo = bf16_to_f32(w[k] & 0xffffu), hi = bf16_to_f32(w[k] >> 16);
      ss = fmaf(lo, lo, ss);
      ss = fmaf(hi, hi, ss);
    }
  }
  ss = block_sum(ss, red);
  float inv = 1.0f / sqrtf(ss / (float)H + eps);
  uint4* o4 = reinterpret_cast<uint4*>(out + (size_t)blockIdx.x * H);
  for (int v = threadIdx.x; v < H / 8; v += kBlock) o4[v] = norm_word(x4[v], gamma, inv, v);
}

// ============================================================== router
// Logits of rows [row0, row0+8) of the 8-bit router for one staged token;
// wave w takes steps w, w+4, ...  SR steps per wave per pass.
template <int SR>
struct RRegs {
  uint4 w[SR];
  uint32_t sb[SR];
};
template <int SR>
__device__ __forceinline__ void router_load(RRegs<SR>& R, const DevQ& Wr, int row0, int E, int H,
                                            int s0, int tid = threadIdx.x) {
  const int wave = tid >> 6, lane = tid & 63, r = lane & 7, p = lane >> 3;
  const int CH8 = H / 16, G = H / 64, row = min(row0 + r, E - 1);
#pragma unroll
  for (int i = 0; i < SR; ++i) {
    int c = min((s0 + wave + i * kWavesPerBlock) * kSlots + p, CH8 - 1);
    R.w[i] = ldg16(Wr.q + ((int64_t)row * CH8 + c) * 16);
    R.sb[i] = ld_sb(Wr.s, Wr.b, (int64_t)row * G + (c >> 2));
  }
}
template <int SR>
__device__ __forceinline__ float router_compute(const RRegs<SR>& R, int H, int s0,
                                                const float4* xr, const float* xh, float acc, int tid = threadIdx.x) {
  const int wave = tid >> 6, lane = tid & 63, p = lane >> 3;
  const int CH8 = H / 16;
#pragma unroll
  for (int i = 0; i < SR; ++i) {
    int c = (s0 + wave + i * kWavesPerBlock) * kSlots + p;
    if (c < CH8) {
      float d = 0.f;
      d = dot_word8_f32(R.w[i].x, xr[c], d);
      d = dot_word8_f32(R.w[i].y, xr[CH8 + c], d);
      d = dot_word8_f32(R.w[i].z, xr[2 * CH8 + c], d);
      d = dot_word8_f32(R.w[i].w, xr[3 * CH8 + c], d);
      acc = fmaf(half_to_f32(R.sb[i] & 0xffffu), d, acc);
      acc = fmaf(half_to_f32(R.sb[i] >> 16), xh[c], acc);
    }
  }
  return acc;
}
// Sum the 4 waves' row partials: returns the logit in threads 0..7.
__device__ float router_finish(float acc, float* red, int tid = threadIdx.x) {
  const int wave = tid >> 6, lane = tid & 63;
  acc = rowblock_sum(acc);
  if ((lane >> 3) == 0) red[wave * 8 + (lane & 7)] = acc;
  __syncthreads();
  float s = 0.f;
  if (tid < 8)
    for (int w = 0; w < kWavesPerBlock; ++w) s += red[w * 8 + tid];
  __syncthreads();
  return s;
}

// One token's logits for rows [row0, row0+8) (threads 0..7 hold them).
// H8C: H/16 when known at compile time (0: runtime).  XDEV: the input is
// read device-coherently after the first weight loads are issued and
// `pre` (a whole-block wait) has returned.
template <int H8C, bool XDEV = false, typename Pre = NoPre>
__device__ float router_token(const DevQ& Wr, int row0, int E, int H_rt, const uint16_t* x,
                              const uint16_t* gamma, float eps, float4* xr, float* xh, float* red,
                              Pre pre = Pre(), int tid = threadIdx.x) {
  constexpr int SR = H8C ? cdiv(cdiv(H8C, kSlots), kWavesPerBlock) : kSR;
  const int H = H8C ? H8C * 16 : H_rt;
  const int nsteps = cdiv(H / 16, kSlots);
  XRegs X;
  if constexpr (!XDEV) x_load(X, x, H, tid);
  float acc = 0.f;
  {
    RRegs<SR> R;
    router_load<SR>(R, Wr, row0, E, H, 0, tid);
    uint32_t* sys = reinterpret_cast<uint32_t*>(red) - kSysRed;
    (void)sys;
    QMOE_STAMP(sys, 1);
    if constexpr (XDEV) {
      pre();
      x_load_dev(X, x, H, tid);
    }
    float inv = gamma ? x_inv_rms(X, x, H, eps, red, tid) : 1.f;
    x_stage<false>(X, x, gamma, inv, H, xr, xh, tid);
    __syncthreads();
    QMOE_STAMP(sys, 4);
    acc = router_compute<SR>(R, H, 0, xr, xh, acc, tid);
  }
  if (!H8C) {
    for (int s0 = SR * kWavesPerBlock; s0 < nsteps; s0 += SR * kWavesPerBlock) {
      RRegs<SR> R;
      router_load<SR>(R, Wr, row0, E, H, s0, tid);
      acc = router_compute<SR>(R, H, s0, xr, xh, acc, tid);
    }
  }
  return router_finish(acc, red, tid);
}

// ========================================================= MoE FFN step
constexpr int kSysLg = 64;  // sys words: the router block's 8 logits

// STK: a stack layer (router weights issued, then the wait for the layer
// input).  Returns false when a wait gave up.
template <int HC, bool STK>
__device__ bool role_router(const DecodeArgs& a, int b, uint8_t* smem, uint32_t epoch) {
  // the router is on every other block's critical path: its waves issue first
  __builtin_amdgcn_s_setprio(3);
  uint32_t* sys = reinterpret_cast<uint32_t*>(smem);
  int tid = threadIdx.x;
  if constexpr (STK) opaque_v(tid);
  const int H = HC ? HC : a.H;
  float4* xr = reinterpret_cast<float4*>(smem + kSysBytes);
  float* xh = reinterpret_cast<float*>(smem + kSysBytes + (size_t)H * 4);
  float* red = reinterpret_cast<float*>(sys + kSysRed);
  const int row0 = b * kRowsPerUnit;
  bool ok = true;
  float s;
  if constexpr (STK) {
    s = router_token<HC / 16, true>(a.router, row0, a.E, H, a.x, a.gamma, a.eps, xr, xh, red,
                                    [&] {
                                      ok = wait_prev_layer(a, sys, 0, tid);
                                      __builtin_amdgcn_s_setprio(3);
                                    },
                                    tid);
    if (!ok) return false;
  } else {
    s = router_token<HC / 16>(a.router, row0, a.E, H, a.x, a.gamma, a.eps, xr, xh, red);
  }
  QMOE_STAMP(sys, 2);
  if (tid < 8) {
    int e = min(row0 + tid, a.E - 1);
    if (a.lbias) s += gptr(a.lbias)[e];
    reinterpret_cast<float*>(sys + kSysLg)[tid] = s;
  }
  __syncthreads();
  // publish (epoch, logit) pairs in every replica: one 64-bit store each
  const int j = tid & 7, rep = tid >> 3;
  if (rep < ctl::kRep && row0 + j < a.E) {
    uint64_t v = ((uint64_t)epoch << 32) | __float_as_uint(reinterpret_cast<float*>(sys + kSysLg)[j]);
    st_dev(reinterpret_cast<uint64_t*>(rep_of(a, ctl::kTagBase, rep)) + row0 + j, v);
  }
  QMOE_STAMP(sys, 3);
  return true;
}

// Gate/up of 16 rows (two row-blocks of 8): wave w computes matrix (w & 1:
// gate, up) over column half (w >> 1) for both row-blocks, whose loads are
// all issued before any math; the block sums the halves and applies the
// GELU gating.  expert_rank < 0: shared expert.
constexpr int kGuRows = 2 * kRowsPerUnit;

// The same matrix seen from 8 rows further down.
__device__ __forceinline__ DevQ rows_below(DevQ m, int H) {
  const int G = H / 64;
  m.q += (int64_t)kRowsPerUnit * (H / 2);
  m.s += (int64_t)kRowsPerUnit * G;
  m.b += (int64_t)kRowsPerUnit * G;
  return m;
}

// STK: a stack layer; the layer input is read device-coherently after the
// wait for the previous layer (the shared expert's weights are issued
// before it).  Returns false when a wait gave up.
template <int HC, int NV, bool STK>
__device__ bool role_gate_up(const DecodeArgs& a, int expert_rank, int rb, int rows,
                             uint8_t* smem, uint32_t epoch, uint64_t t_start) {
  uint32_t* sys = reinterpret_cast<uint32_t*>(smem);
  int tid = threadIdx.x;
  if constexpr (STK) opaque_v(tid);
  const int H = HC ? HC : a.H;
  uint4* xs = reinterpret_cast<uint4*>(smem + kSysBytes);
  float* xh = reinterpret_cast<float*>(smem + gu_xh_off(H));
  float* red = reinterpret_cast<float*>(sys + kSysRed);
  const int wave = tid >> 6, lane = tid & 63;
  const int mi = wave & 1, half = wave >> 1;
  uint32_t* sbl = reinterpret_cast<uint32_t*>(smem + gu_sb_off(H)) + wave * gu_sb_words(H);
  const int row0 = rb * kGuRows;  // rows is a multiple of 16: both row-blocks are whole
  const int CWh = H / 64;  // chunks per column half
  XRegs X;
  if constexpr (!STK) x_load(X, a.x, H, tid);
  DevQ m[2];
  size_t dst;  // element offset inside an activation replica
  float acc[2];
  if (expert_rank < 0) {
    hold_until(t_start, kHoldTicks);
    m[0] = mi ? a.shu : a.shg;
    m[1] = rows_below(m[0], H);
    dst = 0;
    bool ok = true;
    rows4_run<2, HC / 64>(m, row0, rows, H, half * CWh, CWh, xs, xh, sbl,
                          [&] {
                            QMOE_STAMP(sys, 1);
                            if constexpr (STK) {
                              ok = wait_prev_layer(a, sys, 0, tid);
                              x_load_dev(X, a.x, H, tid);
                            }
                            float inv = a.gamma ? x_inv_rms(X, a.x, H, a.eps, red, tid) : 1.f;
                            x_stage<true>(X, a.x, a.gamma, inv, H, xs, xh, tid);
                            __syncthreads();
                            QMOE_STAMP(sys, 2);
                          },
                          acc, tid);
    if (!ok) return false;
  } else {
    if constexpr (STK) {
      if (!wait_prev_layer(a, sys, 0, tid)) return false;
      x_load_dev(X, a.x, H, tid);
    }
    // stage h while the router finishes, then resolve the expert
    float inv = a.gamma ? x_inv_rms(X, a.x, H, a.eps, red, tid) : 1.f;
    x_stage<true>(X, a.x, a.gamma, inv, H, xs, xh, tid);
    __syncthreads();
    QMOE_STAMP(sys, 2);
    if (!block_routing<NV>(a, epoch, sys, false, tid)) return false;
    QMOE_STAMP(sys, 3);
    const int s = reinterpret_cast<int32_t*>(sys + kSysSlot)[expert_rank];
    m[0] = devq_at(mi ? a.up : a.gate, s);
    m[1] = rows_below(m[0], H);
    dst = (size_t)a.Is + (size_t)expert_rank * a.I;
    // (the registration after the weight loads, which it would otherwise
    // hold back when the memory pipeline is full)
    rows4_run<2, HC / 64>(m, row0, rows, H, half * CWh, CWh, xs, xh, sbl,
                          [&] {
                            QMOE_STAMP(sys, 1);
                            if (!STK && early_on(a, epoch - 1u)) call_register(a, epoch, tid);
                          },
                          acc, tid);
  }
  QMOE_STAMP(sys, 4);
  if ((lane >> 3) == 0) {
    red[(wave * 2 + 0) * 8 + (lane & 7)] = acc[0];
    red[(wave * 2 + 1) * 8 + (lane & 7)] = acc[1];
  }
  __syncthreads();
  // a = gelu(g) * u for the 16 rows, stored in every activation replica
  const int t = tid & 15, rep = tid >> 4;
  if (rep < ctl::kRep) {
    const int k = t >> 3, rr = t & 7;
    float g = red[((0 * 2 + k) * 8) + rr] + red[((2 * 2 + k) * 8) + rr];
    float u = red[((1 * 2 + k) * 8) + rr] + red[((3 * 2 + k) * 8) + rr];
    st_dev(act_of(a, rep) + dst + row0 + t, gelu_tanh(g) * u);
  }
  return true;
}

// Activations [off, off + n) of a replica (fp32) -> LDS in one pass: each
// thread issues all its 16-byte device-coherent loads before it uses any,
// so a pass costs one round trip.  The run is a sequence of segments of
// `seg` values (the shared activations, or one expert's): per segment
// (CH = seg/32 chunks), word v = 4c + j (8 values) goes to the even/odd
// layout as[(2j+e)*CH + c] and ah[c] is the sum of chunk c.  The caller
// passes the run's value and chunk-sum bases; tid is threadIdx.x.
constexpr int kStageUnroll = 4;  // words (8 floats) per thread per pass
__device__ __forceinline__ void stage_run(const float* act, int off, int n, int seg, float4* as,
                                          float* ah, int tid) {
  const int Wn = n / 8, Wseg = seg / 8, CH = seg / 32;
  const uint32_t nbytes = (uint32_t)(off + n) * 4;
  for (int v0 = 0; v0 < Wn; v0 += kStageUnroll * kBlock) {
    float4 lo[kStageUnroll], hi[kStageUnroll];
#pragma unroll
    for (int u = 0; u < kStageUnroll; ++u) {
      const uint32_t v = (uint32_t)(v0 + u * kBlock + tid);
      lo[u] = ld_dev16(act, nbytes, (uint32_t)off * 4 + v * 32);  // past the end: zeros
      hi[u] = ld_dev16(act, nbytes, (uint32_t)off * 4 + v * 32 + 16);
    }
#pragma unroll
    for (int u = 0; u < kStageUnroll; ++u) {
      const int v = v0 + u * kBlock + tid;
      float s = ((lo[u].x + lo[u].y) + (lo[u].z + lo[u].w)) +
                ((hi[u].x + hi[u].y) + (hi[u].z + hi[u].w));
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      if (v < Wn) {
        const int k = v / Wseg, vl = v - k * Wseg;
        float4* a4 = as + (size_t)k * seg / 4;
        const int c = vl >> 2, j = vl & 3;
        a4[(2 * j) * CH + c] = make_float4(lo[u].x, lo[u].z, hi[u].x, hi[u].z);
        a4[(2 * j + 1) * CH + c] = make_float4(lo[u].y, lo[u].w, hi[u].y, hi[u].w);
        if (j == 0) ah[k * CH + c] = s;
      }
    }
  }
}

// One down task of a lane: chunk c (32 inputs) of the 8 rows [row0, row0+8)
// of a 4-bit matrix.  The lane reads the chunk's staged activations once
// and applies them to all 8 rows.
struct DTask {
  uint4 w[kRowsPerUnit];
  uint32_t sb[kRowsPerUnit];
};

__device__ __forceinline__ void dtask_load(DTask& T, const DevQ& W, int row0, int CH, int c) {
  const int G = CH / 2;
#pragma unroll
  for (int r = 0; r < kRowsPerUnit; ++r) {
    T.w[r] = ldg16(W.q + ((int64_t)(row0 + r) * CH + c) * 16);
    T.sb[r] = ld_sb(W.s, W.b, (int64_t)(row0 + r) * G + (c >> 1));
  }
}

// acc[r] += wgt * (s * sum(q a) + b * sum(a)) over the chunk, for the 8 rows.
__device__ __forceinline__ void dtask_acc(const DTask& T, const float4* as, const float* ah, int CH,
                                          int c, float wgt, float (&acc)[kRowsPerUnit]) {
  float4 x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = as[i * CH + c];
  const float hs = ah[c];
#pragma unroll
  for (int r = 0; r < kRowsPerUnit; ++r) {
    float a0 = 0.f, a1 = 0.f;
    dot_word4_f32(T.w[r].x, x[0], x[1], a0, a1);
    dot_word4_f32(T.w[r].y, x[2], x[3], a0, a1);
    dot_word4_f32(T.w[r].z, x[4], x[5], a0, a1);
    dot_word4_f32(T.w[r].w, x[6], x[7], a0, a1);
    // the fp8 conversion gave q * 2^-9: fold 2^9 into the scale
    float v = fmaf(512.0f * half_to_f32(T.sb[r] & 0xffffu), a0 + a1,
                   half_to_f32(T.sb[r] >> 16) * hs);
    acc[r] = fmaf(wgt, v, acc[r]);
  }
}

// Sum acc[0..8) of every lane of the block, per row; threads 0..7 return
// rows 0..7 (fixed order: a reduce-scatter over the wave, then the waves
// in turn).
__device__ float rows8_block_sum(float (&acc)[kRowsPerUnit], float* red, int tid = threadIdx.x) {
  const int lane = tid & 63, wave = tid >> 6;
  float v4[4], v2[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool hi = lane & 32;
    float send = hi ? acc[i] : acc[4 + i];
    float keep = hi ? acc[4 + i] : acc[i];
    v4[i] = keep + __shfl_xor(send, 32);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const bool hi = lane & 16;
    float send = hi ? v4[i] : v4[2 + i];
    float keep = hi ? v4[2 + i] : v4[i];
    v2[i] = keep + __shfl_xor(send, 16);
  }
  float v;
  {
    const bool hi = lane & 8;
    float send = hi ? v2[0] : v2[1];
    float keep = hi ? v2[1] : v2[0];
    v = keep + __shfl_xor(send, 8);
  }
  // lane l now holds row (l >> 3) & 7 over 8 of the lanes; finish the wave
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 1);
  __syncthreads();
  if ((lane & 7) == 0) red[wave * 8 + (lane >> 3)] = v;
  __syncthreads();
  float s = 0.f;
  if (tid < kRowsPerUnit)
    for (int w = 0; w < kWavesPerBlock; ++w) s += red[w * 8 + tid];
  return s;
}

// Down projections + combine for output rows [8b, 8b+8).  The block's 256
// lanes own chunk tasks of all 8 rows: task t < K*CHk is routed (expert
// rank k = t / CHk, chunk c), the next CHs tasks are the shared chunks.
// Order: shared-down weights -> routing -> at once the routed-down weights
// (they stream while the gate/up blocks work) -> shared activations once
// the shared gate/up blocks are done, shared part -> one wait for the
// gate/up blocks of all experts, their activations in one pass, routed part
// -> combine.  Under the load of the weight streams a dependent memory
// access takes microseconds, so the routing is fetched before the stream
// starts, the waits are polled by the last wave (its tasks are shared ones,
// loaded early) and every staging is one round trip.  IC/ISC: expert and
// shared intermediate sizes when known (0: runtime).
// STK: a stack layer.  The residual is the block's own output rows of the
// previous layer, kept in `held` (threads 0..7; a.residual for the first
// layer); the output goes device-coherently to a.out (the next layer's
// input) and, if given, to `lout`.  Returns false when a wait gave up.
template <int IC, int ISC, int NV, bool STK>
__device__ bool role_down(const DecodeArgs& a, int b, uint8_t* smem, uint32_t epoch,
                          uint64_t t_start, uint32_t& held, uint16_t* lout) {
  uint32_t* sys = reinterpret_cast<uint32_t*>(smem);
  const int K = a.K;
  const int I = IC ? IC : a.I, Is = ISC ? ISC : a.Is;
  const int CHk = I / 32, CHs = Is / 32;
  // tasks per lane: one pass with all loads issued at once when the shapes
  // are known and fit; otherwise pass by pass
  constexpr bool kOnePass = IC && ISC && QMOE_MAX_TOP_K * (IC / 32) + ISC / 32 <= kBlock;
  float4* as_sh = reinterpret_cast<float4*>(smem + kSysBytes);
  float* ah_sh = reinterpret_cast<float*>(smem + down_ah_off(I, Is, K));
  const float4* ask = as_sh + Is / 4;
  const float* ahk = ah_sh + Is / 32;
  constexpr int kPollWave = kWavesPerBlock - 1;
  float* red = reinterpret_cast<float*>(sys + kSysRed);
  uint32_t* ctlw = ctl_of(a);
  const uint32_t* flags =
      reinterpret_cast<const uint32_t*>(rep_of(a, ctl::kFlagBase, blockIdx.x % ctl::kRep));
  const int row0 = b * kRowsPerUnit;  // H is a multiple of 64: all 8 rows exist
  const int nrt = K * CHk, ntask = nrt + CHs;
  int t = threadIdx.x;
  if constexpr (STK) opaque_v(t);
  const bool routed = t < nrt;
  float acc[kRowsPerUnit];
#pragma unroll
  for (int r = 0; r < kRowsPerUnit; ++r) acc[r] = 0.f;
  DTask T;

  // 1. shared-down weights
  hold_until(t_start, kHoldTicks);
  if (kOnePass && !routed) dtask_load(T, a.shd, row0, CHs, min(t - nrt, CHs - 1));
  QMOE_STAMP(sys, 1);
  // 2. routing, then at once the routed-down weights
  if (!block_routing<NV>(a, epoch, sys, false, t)) return false;
  QMOE_STAMP(sys, 2);
  const int32_t* slot_s = reinterpret_cast<const int32_t*>(sys + kSysSlot);
  const float* w_s = reinterpret_cast<const float*>(sys + kSysW);
  if (kOnePass && routed) {
    const int k = t / CHk, c = t - k * CHk;
    dtask_load(T, devq_at(a.down, slot_s[k]), row0, CHk, c);
  }
  // (the registration and block 0's copy of the routing for the caller
  // after the routed-down loads, which they would otherwise hold back when
  // the memory pipeline is full)
  if (!STK && early_on(a, epoch - 1u)) call_register(a, epoch, t);
  if (b == 0 && t < K) {
    if (a.idx_out) a.idx_out[t] = reinterpret_cast<const int32_t*>(sys + kSysIdx)[t];
    if (a.w_out) a.w_out[t] = w_s[t];
  }
  if constexpr (kOnePass) {
    // 3-4. two passes through one copy of the wait / staging / accumulate
    //    code: pass 0 takes the shared activations once the S blocks are
    //    published, pass 1 the routed ones once the G blocks of all K
    //    experts are (one wait, one staging pass).  Each lane's one task
    //    falls in one of the passes.  The routed pass, on the critical
    //    path, runs instructions the shared pass has already fetched.
#pragma clang loop unroll(disable)
    for (int p = 0; p < 2; ++p) {
      if (!a.nowait && !(p == 0 && a.s_done) &&
          !block_wait_flags(flags + (p ? a.nS : 0), p ? K * a.perG : a.nS, epoch, ctlw, 2 + p, sys,
                            kPollWave, t))
        return false;
      QMOE_STAMP(sys, 3 + 2 * p);
      const int off = p ? Is : 0;
      stage_run(act_of(a, blockIdx.x % ctl::kRep), off, p ? K * I : Is, p ? I : Is,
                as_sh + off / 4, ah_sh + off / 32, t);
      __syncthreads();
      QMOE_STAMP(sys, 4 + 2 * p);
      // the weights as if reloaded per pass: their decoded forms are not
      // hoisted out of the loop and held in registers across both passes
#pragma unroll
      for (int r = 0; r < kRowsPerUnit; ++r)
        asm volatile("" : "+v"(T.w[r].x), "+v"(T.w[r].y), "+v"(T.w[r].z), "+v"(T.w[r].w),
                     "+v"(T.sb[r]));
      if (p ? routed : (!routed && t < ntask)) {
        const int k = routed ? t / CHk : 0;
        const int base = routed ? Is + k * I : 0;  // first activation of the task's segment
        dtask_acc(T, as_sh + base / 4, ah_sh + base / 32, routed ? CHk : CHs,
                  routed ? t - k * CHk : t - nrt, routed ? w_s[k] : 1.0f, acc);
      }
    }
  } else {
    // 3. shared activations once the S blocks are published, shared part
    if (!a.nowait && !a.s_done &&
        !block_wait_flags(flags, a.nS, epoch, ctlw, 2, sys, kPollWave, t))
      return false;
    stage_run(act_of(a, blockIdx.x % ctl::kRep), 0, Is, Is, as_sh, ah_sh, t);
    __syncthreads();
    for (int c = t; c < CHs; c += kBlock) {
      DTask U;
      dtask_load(U, a.shd, row0, CHs, c);
      dtask_acc(U, as_sh, ah_sh, CHs, c, 1.0f, acc);
    }
    // 4. one wait for the G blocks of all K experts, their activations in
    //    one pass, routed part
    if (!a.nowait &&
        !block_wait_flags(flags + a.nS, K * a.perG, epoch, ctlw, 3, sys, kPollWave, t))
      return false;
    stage_run(act_of(a, blockIdx.x % ctl::kRep), Is, K * I, I, as_sh + Is / 4, ah_sh + Is / 32, t);
    __syncthreads();
    for (int u = t; u < nrt; u += kBlock) {
      const int k = u / CHk, c = u - k * CHk;
      DTask U;
      dtask_load(U, devq_at(a.down, slot_s[k]), row0, CHk, c);
      dtask_acc(U, ask + (size_t)k * I / 4, ahk + k * CHk, CHk, c, w_s[k], acc);
    }
  }
  // 5. combine: rows over the block, residual, bf16
  float s = rows8_block_sum(acc, red, t);
  QMOE_STAMP(sys, 7);
  if constexpr (STK) {
    uint32_t o = 0;
    if (t < kRowsPerUnit) {
      const int rr = row0 + t;
      s += bf16_to_f32(a.residual ? (uint32_t)gptr(a.residual)[rr] : held);
      o = f32_to_bf16(s);
      held = o;
      if (lout) lout[rr] = (uint16_t)o;
    }
    // rows in pairs: one 32-bit device-coherent store per two rows
    const uint32_t nb = (uint32_t)__shfl_down((int)o, 1);
    if (t < kRowsPerUnit && !(t & 1))
      st_dev(reinterpret_cast<uint32_t*>(a.out + row0 + t), o | (nb << 16));
  } else {
    if (threadIdx.x < kRowsPerUnit) {
      const int rr = row0 + threadIdx.x;
      if (a.residual) s += bf16_to_f32(gptr(a.residual)[rr]);
      a.out[rr] = f32_to_bf16(s);
    }
  }
  QMOE_STAMP(sys, 8);
  return true;
}

// EC: number of experts when known at compile time (0: up to 512).
#ifdef QMOE_TRACE
__device__ void trace_flush(uint32_t* sys, uint32_t gen) {
  __syncthreads();
  if (qmoe_trace_buf && threadIdx.x < kNStamp) {
    const size_t slot = gen % (uint32_t)qmoe_trace_slots;
    qmoe_trace_buf[(slot * gridDim.x + blockIdx.x) * kNStamp + threadIdx.x] =
        reinterpret_cast<uint64_t*>(sys + kSysTrace)[threadIdx.x];
  }
}
#endif

template <int HC, int IC, int ISC, int EC>
// (trace builds: bounded to the VGPRs of four waves per SIMD, which the
// plain build meets by itself, so that every block is resident at once in
// both and the timeline measures the same schedule)
#ifdef QMOE_TRACE
__global__ __launch_bounds__(kBlock, 4) void k_moe_step(DecodeArgs a) {
#else
__global__ __launch_bounds__(kBlock) void k_moe_step(DecodeArgs a) {
#endif
  constexpr int NV = EC ? cdiv(EC, 64) : QMOE_MAX_EXPERTS / 64;
  extern __shared__ __align__(16) uint8_t smem[];
  uint32_t* sys = reinterpret_cast<uint32_t*>(smem);
  const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
#ifdef QMOE_TRACE
  if (threadIdx.x < kNStamp) reinterpret_cast<uint64_t*>(sys + kSysTrace)[threadIdx.x] = 0;
  QMOE_STAMP(sys, 0);
#endif
  const uint32_t gen = load_gen(a.ws, a.wl.ctl);
  const uint32_t epoch = gen + 1;
  const int rb = a.role0 + blockIdx.x;
  const bool early = early_on(a, gen);
  if (rb < a.nR) {
    role_router<HC, false>(a, rb, smem, epoch);
    if (early) call_register(a, epoch);
  } else if (rb < a.nR + a.nS) {
    const int s = rb - a.nR;
    // (a block whose wait gave up publishes all the same, so that its
    // consumers end at once; the error word marks the call as failed)
    const bool ok = role_gate_up<HC, NV, false>(a, -1, s, ISC ? ISC : a.Is, smem, epoch, t_start);
    block_publish(a, s, epoch);
    QMOE_STAMP(sys, 5);
    (void)ok;
    if (early) {
      call_register(a, epoch);
      if (s == 0) early_advance(a, gen);
    }
    if (a.cnt == kCntS) call_done(a, s, a.nS, gen, sys);
  } else if (rb < a.nR + a.nS + a.nG) {
    const int gb = rb - a.nR - a.nS;
    role_gate_up<HC, NV, false>(a, gb / a.perG, gb % a.perG, IC ? IC : a.I, smem, epoch, t_start);
    block_publish(a, a.nS + gb, epoch);
    QMOE_STAMP(sys, 5);
  } else {
    uint32_t held = 0;
    const int d = rb - a.nR - a.nS - a.nG;
    role_down<IC, ISC, NV, false>(a, d, smem, epoch, t_start, held, nullptr);
    if (a.cnt == kCntD && !early) call_done(a, d, a.nD, gen, sys);
  }
#ifdef QMOE_TRACE
  QMOE_STAMP(sys, 9);
  trace_flush(sys, gen);
#endif
}

// ============================================================ layer stack
// One decode token through L layers in one launch (a cooperative launch:
// every block is resident, which the waits on later blocks need).  Each
// block keeps its role for all layers, so its code stays in the
// instruction cache, and before waiting for a layer's input it issues the
// loads that do not depend on it (router and shared-expert weights; the
// output blocks' shared-down weights).  Layer l's input is the caller's x
// (l = 0) or the previous layer's output, ping-ponged through two buffers
// of the workspace; the router, shared and routed gate/up blocks wait for
// every output block of the previous layer, which also guarantees that
// nothing still reads the buffers, activations or tags they overwrite.
// The last layer's output goes to `out`; the last output block to finish
// (a counter) clears every flag and tag, so the next call starts from zero.
// Layer l's arguments: the table's pointers, the layer's input and output
// buffers, the tags.
__device__ __forceinline__ void stack_layer_args(DecodeArgs& a, const DecodeArgs& a0,
                                                 const StackLayerDev* tab, int l, int L,
                                                 uint16_t* xb, int H, uint32_t tag0) {
  a = a0;
  const StackLayerDev& T = tab[l];
  a.router = T.router; a.gate = T.gate; a.up = T.up; a.down = T.down;
  a.shg = T.shg; a.shu = T.shu; a.shd = T.shd;
  a.gamma = T.gamma; a.lbias = T.lbias;
  a.x = l ? xb + (size_t)((l - 1) & 1) * H : a0.x;
  a.out = l == L - 1 ? a0.out : xb + (size_t)(l & 1) * H;
  a.residual = l ? nullptr : a0.x;
  a.idx_out = a0.idx_out ? a0.idx_out + (size_t)l * a0.K : nullptr;
  a.w_out = a0.w_out ? a0.w_out + (size_t)l * a0.K : nullptr;
  a.dwait = l ? a0.nD : 0;
  a.dtag = tag0 + (uint32_t)l - 1u;
}

template <int HC, int IC, int ISC, int EC>
// (the table is read-only for the whole launch: __restrict__ lets its
// fields be read with scalar loads through the constant cache)
__global__ __launch_bounds__(kBlock, 4) void k_moe_stack(DecodeArgs a0,
                                                         const StackLayerDev* __restrict__ tab,
                                                         int L, uint16_t* xb, uint16_t* lout) {
  constexpr int NV = EC ? cdiv(EC, 64) : QMOE_MAX_EXPERTS / 64;
  extern __shared__ __align__(16) uint8_t smem[];
  uint32_t* sys = reinterpret_cast<uint32_t*>(smem);
  const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
  const int rb = blockIdx.x;
  const int H = HC ? HC : a0.H;
  const int nRSG = a0.nR + a0.nS + a0.nG;
  // layer l's flags and tags carry G + 1 + l
  const uint32_t gen = load_gen(a0.ws, a0.wl.ctl);
  const uint32_t tag0 = gen + 1;
  if (threadIdx.x == 0) *reinterpret_cast<uint64_t*>(sys + kSysWait) = 0;
  DecodeArgs a;
  // every role runs its own loop over the layers
  if (rb < a0.nR) {
    for (int l = 0; l < L; ++l) {
      stack_layer_args(a, a0, tab, l, L, xb, H, tag0);
      __syncthreads();  // the previous layer's LDS contents are consumed
      int b = rb;
      opaque_s(b);
      if (!role_router<HC, true>(a, b, smem, tag0 + (uint32_t)l)) return;
    }
    return;
  }
  if (rb < a0.nR + a0.nS) {
    const int sb = rb - a0.nR;
    for (int l = 0; l < L; ++l) {
      stack_layer_args(a, a0, tab, l, L, xb, H, tag0);
      __syncthreads();
      int b = sb;
      opaque_s(b);
      if (!role_gate_up<HC, NV, true>(a, -1, b, ISC ? ISC : a.Is, smem, tag0 + (uint32_t)l,
                                      t_start))
        return;
      block_publish(a, sb, tag0 + (uint32_t)l, opaque_tid());
    }
    return;
  }
  if (rb < nRSG) {
    const int gb = rb - a0.nR - a0.nS;
    for (int l = 0; l < L; ++l) {
      stack_layer_args(a, a0, tab, l, L, xb, H, tag0);
      __syncthreads();
      int b = gb;
      opaque_s(b);
      if (!role_gate_up<HC, NV, true>(a, b / a.perG, b % a.perG, IC ? IC : a.I, smem,
                                      tag0 + (uint32_t)l, t_start))
        return;
      block_publish(a, a.nS + gb, tag0 + (uint32_t)l, opaque_tid());
    }
    return;
  }
  const int d = rb - nRSG;
  uint32_t held = 0;
  for (int l = 0; l < L; ++l) {
    stack_layer_args(a, a0, tab, l, L, xb, H, tag0);
    __syncthreads();
    int b = d;
    opaque_s(b);
    if (!role_down<IC, ISC, NV, true>(a, b, smem, tag0 + (uint32_t)l, t_start, held,
                                      lout ? lout + (size_t)l * H : nullptr))
      return;
    // the last layer's outputs have no reader inside the launch
    if (l < L - 1) block_publish(a, a.nS + a.nG + d, tag0 + (uint32_t)l, opaque_tid());
  }
  // output blocks: count the finished ones; the last advances the tag
  // counter past this call's layers
  wait_vm();
  __syncthreads();
  uint32_t* cnt = reinterpret_cast<uint32_t*>(a0.ws + a0.wl.ctl + ctl::kCntBase +
                                              64 * ctl::kCntStack);
  if (threadIdx.x == 0) {
    const uint32_t prev = add_dev(cnt, 1u);
    sys[kSysOk] = prev == (uint32_t)a0.nD - 1;
  }
  __syncthreads();
  if (!sys[kSysOk]) return;
  if (threadIdx.x == 0) st_dev(cnt, 0u);
  gen_advance(a0.ws, a0.wl.ctl, a0.E, gen, (uint32_t)L);
}

// ======================================================== host launchers
static hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

#ifdef QMOE_TRACE
}  // namespace qmoe
// Trace builds only: where the step kernel writes its phase stamps (device
// buffer of slots * blocks * 16 uint64; NULL turns tracing off).
extern "C" qmoe_status qmoe_trace_set(void* buf, int32_t slots) {
  if (slots < 1) return QMOE_ERR_BAD_SHAPE;
  if (hipMemcpyToSymbol(HIP_SYMBOL(qmoe::qmoe_trace_buf), &buf, sizeof(buf)) != hipSuccess ||
      hipMemcpyToSymbol(HIP_SYMBOL(qmoe::qmoe_trace_slots), &slots, sizeof(slots)) != hipSuccess)
    return QMOE_ERR_HIP;
  return QMOE_OK;
}
namespace qmoe {
#endif

qmoe_status launch_gemv4(const qmoe_qtensor& W, const uint16_t* x, float* y, void* stream) {
  const int units = cdiv(W.rows, kRowsPerUnit);
  const int blocks = cdiv(units, kWavesPerBlock);
  const size_t lds = gu_lds(W.cols);
  const DevQ d = devq(W);
  switch (W.cols / 32) {
    case 88: hipLaunchKernelGGL(k_gemv4<88>, dim3(blocks), dim3(kBlock), lds, S(stream), d, W.rows, W.cols, x, y); break;
    case 66: hipLaunchKernelGGL(k_gemv4<66>, dim3(blocks), dim3(kBlock), lds, S(stream), d, W.rows, W.cols, x, y); break;
    case 22: hipLaunchKernelGGL(k_gemv4<22>, dim3(blocks), dim3(kBlock), lds, S(stream), d, W.rows, W.cols, x, y); break;
    case 16: hipLaunchKernelGGL(k_gemv4<16>, dim3(blocks), dim3(kBlock), lds, S(stream), d, W.rows, W.cols, x, y); break;
    default: hipLaunchKernelGGL(k_gemv4<0>, dim3(blocks), dim3(kBlock), lds, S(stream), d, W.rows, W.cols, x, y); break;
  }
  return hipGetLastError() == hipSuccess ? QMOE_OK : QMOE_ERR_HIP;
}

size_t tiled4_size(int rows, int cols) { return tiled4_bytes(rows, cols); }

// Compiled widths: 2816 (the layer's hidden size) and 704 (its expert
// width); rbw: row-blocks per wave (1 or 2).
bool gemv_tiled4_supported(int cols) { return cols == 2816 || cols == 704; }

qmoe_status launch_gemv_tiled4(const uint8_t* T, int rows, int cols, const uint16_t* x, float* y,
                               int rbw, void* stream) {
  const int RB = cdiv(rows, kRowsPerUnit);
  const size_t lds = gemv4t_lds(cols);
  // measured on MI355X, one row-block per wave: width 2816 at 65,536 rows
  // 18.0 us (0.72 of HBM peak), width 704 at 262,144 rows 17.7 us (0.74);
  // two per wave 18.5 and 17.9 us
  if (rbw == 0) rbw = 1;
  const dim3 grid(cdiv(RB, kWavesPerBlock * rbw));
  if (cols == 2816) {
    if (rbw == 2) hipLaunchKernelGGL((k_gemv4t<88, 2>), grid, dim3(kBlock), lds, S(stream), T, rows, cols, x, y);
    else hipLaunchKernelGGL((k_gemv4t<88, 1>), grid, dim3(kBlock), lds, S(stream), T, rows, cols, x, y);
  } else {
    if (rbw == 2) hipLaunchKernelGGL((k_gemv4t<22, 2>), grid, dim3(kBlock), lds, S(stream), T, rows, cols, x, y);
    else hipLaunchKernelGGL((k_gemv4t<22, 1>), grid, dim3(kBlock), lds, S(stream), T, rows, cols, x, y);
  }
  return hipGetLastError() == hipSuccess ? QMOE_OK : QMOE_ERR_HIP;
}

qmoe_status launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int T, int H,
                           uint16_t* out, void* stream) {
  hipLaunchKernelGGL(k_rmsnorm, dim3(T), dim3(kBlock), 0, S(stream), x, gamma, eps, H, out);
  return hipGetLastError() == hipSuccess ? QMOE_OK : QMOE_ERR_HIP;
}


// Dynamic LDS of the step and stack kernels: the largest role.
static size_t step_lds(int H, int E, int I, int Is, int K) {
  (void)E;
  size_t lds = gu_lds(H);
  if (router_lds(H) > lds) lds = router_lds(H);
  if (down_lds(I, Is, K) > lds) lds = down_lds(I, Is, K);
  return lds;
}

bool moe_step_supported(const qmoe_moe_layer& L) {
  const int nR = cdiv(L.n_experts, kRowsPerUnit);
  const int perG = L.inter / kGuRows;
  const int nS = L.shared_inter / kGuRows;
  return L.hidden / 8 <= kMaxXW * kBlock && nR <= 64 &&
         step_lds(L.hidden, L.n_experts, L.inter, L.shared_inter, L.top_k) <= 65536 &&
         L.n_experts * 8 <= ctl::kRepStride && nS + L.top_k * perG <= ctl::kMaxFlags;
}

// ev0/ev1: optional hipEvent_t recorded by the dispatch itself at the
// kernel's start and end (hipExtLaunchKernelGGL), for exact kernel timing.
template <int HC, int IC, int ISC, int EC>
static void launch_step_kernel(const DecodeArgs& a, int blocks, size_t lds, void* stream,
                               hipEvent_t ev0, hipEvent_t ev1) {
  if (ev0 || ev1)
    hipExtLaunchKernelGGL((k_moe_step<HC, IC, ISC, EC>), dim3(blocks), dim3(kBlock), lds,
                          S(stream), ev0, ev1, 0, a);
  else
    hipLaunchKernelGGL((k_moe_step<HC, IC, ISC, EC>), dim3(blocks), dim3(kBlock), lds, S(stream), a);
}

static void launch_step(const DecodeArgs& a, int blocks, size_t lds, void* stream,
                        hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr) {
  if (a.H == 2816 && a.I == 704 && a.Is == 2112 && a.E == 128)
    launch_step_kernel<2816, 704, 2112, 128>(a, blocks, lds, stream, ev0, ev1);
  else if (a.H == 512 && a.I == 256 && a.Is == 512 && a.E == 32)
    launch_step_kernel<512, 256, 512, 32>(a, blocks, lds, stream, ev0, ev1);
  else
    launch_step_kernel<0, 0, 0, 0>(a, blocks, lds, stream, ev0, ev1);
}

// mode: kStepFused = one launch with in-kernel waits; kStepPhased = three
// ordered launches; kStepShared = the shared gate/up blocks only;
// kStepRouted = routed gate/up, down and combine after a kStepShared launch
// on the same workspace and stream (the last two need a given routing).
// ev_start/ev_stop (hipEvent_t or null): recorded at the start of the first
// and the end of the last kernel of the step.
qmoe_status launch_moe_step(const qmoe_moe_layer& L, const uint16_t* x, const int32_t* idx_in,
                            const float* w_in, const int32_t* slot, const uint16_t* residual,
                            uint16_t* out, int32_t* idx_out, float* w_out, uint8_t* ws, int mode,
                            void* stream, void* ev_start, void* ev_stop, int heal) {
  const int phased = mode == kStepPhased;
  if (!moe_step_supported(L)) return QMOE_ERR_UNSUPPORTED;
  hipEvent_t e0 = reinterpret_cast<hipEvent_t>(ev_start);
  hipEvent_t e1 = reinterpret_cast<hipEvent_t>(ev_stop);
  DecodeArgs a;
  a.H = L.hidden; a.E = L.n_experts; a.K = L.top_k; a.I = L.inter; a.Is = L.shared_inter;
  a.router = devq(L.router); a.gate = devq(L.gate); a.up = devq(L.up); a.down = devq(L.down);
  a.shg = devq(L.sh_gate); a.shu = devq(L.sh_up); a.shd = devq(L.sh_down);
  a.x = x;
  // with a given routing (or for the shared blocks alone) x is the expert
  // input h itself: no router, no normalisation
  const bool given = idx_in || mode == kStepShared;
  a.gamma = given ? nullptr : L.rms_gamma;
  a.eps = L.rms_eps;
  a.lbias = L.logit_bias;
  a.idx_in = idx_in; a.w_in = w_in; a.slot = slot; a.residual = residual;
  a.out = out; a.idx_out = idx_out; a.w_out = w_out;
  a.ws = ws;
  a.wl = ws_layout(a.E, a.K, a.I, a.Is, 1);
  a.nR = given ? 0 : cdiv(a.E, kRowsPerUnit);
  a.nS = a.Is / kGuRows;
  a.perG = a.I / kGuRows;
  a.nG = a.K * a.perG;
  a.nD = a.H / kRowsPerUnit;
  const size_t lds = step_lds(a.H, a.E, a.I, a.Is, a.K);
  a.nowait = phased;
  a.s_done = 0;
  a.dwait = 0;
  a.dtag = 0;
  // one tag per call; the workspace's tag counter advances once every block
  // of the call has read it (early_advance in a fused call, else the
  // completion count of the call's last role)
  a.ntags = 1;
  a.cnt = kCntD;
  a.heal = heal;
  a.early = 0;
  if (mode == kStepShared || mode == kStepRouted) {
    if (mode == kStepRouted && !idx_in) return QMOE_ERR_NULL_ARG;
    if (mode == kStepShared) {
      a.cnt = kCntS;
      a.role0 = a.nR;
      launch_step(a, a.nS, lds, stream, e0, e1);
    } else {
      a.s_done = 1;
      a.role0 = a.nR + a.nS;
      launch_step(a, a.nG + a.nD, lds, stream, e0, e1);
    }
    return hipGetLastError() == hipSuccess ? QMOE_OK : QMOE_ERR_HIP;
  }
  if (!phased) {
    a.role0 = 0;
    a.early = !heal && a.nS > 0;
    launch_step(a, a.nR + a.nS + a.nG + a.nD, lds, stream, e0, e1);
    return hipGetLastError() == hipSuccess ? QMOE_OK : QMOE_ERR_HIP;
  }
  // router; shared + routed gate/up; down (waits are then satisfied on
  // entry).  The three launches share the call's tag; the last advances it.
  a.cnt = kCntNone;
  if (a.nR) {
    a.role0 = 0;
    launch_step(a, a.nR, lds, stream, e0, nullptr);
    e0 = nullptr;
  }
  a.role0 = a.nR;
  launch_step(a, a.nS + a.nG, lds, stream, e0, nullptr);
  a.cnt = kCntD;
  a.role0 = a.nR + a.nS + a.nG;
  launch_step(a, a.nD, lds, stream, nullptr, e1);
  return hipGetLastError() == hipSuccess ? QMOE_OK : QMOE_ERR_HIP;
}

template <int HC, int IC, int ISC, int EC>
static hipError_t launch_stack_kernel(DecodeArgs a, const StackLayerDev* tab, int L,
                                      uint16_t* xb, uint16_t* lout, int blocks, size_t lds,
                                      void* stream) {
  void* args[] = {&a, &tab, &L, &xb, &lout};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&k_moe_stack<HC, IC, ISC, EC>),
                                    dim3(blocks), dim3(kBlock), args, (unsigned)lds, S(stream));
}

// n_layers layers of shape L (weights from the device table) for one token.
// xb: two bf16 [H] buffers inside the workspace.
qmoe_status launch_moe_stack(const qmoe_moe_layer& L, const void* table, int n_layers,
                             const uint16_t* x, uint16_t* out, uint16_t* lout, int32_t* idx_out,
                             float* w_out, uint8_t* ws, uint16_t* xb, void* stream) {
  if (!moe_step_supported(L)) return QMOE_ERR_UNSUPPORTED;
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.H = L.hidden; a.E = L.n_experts; a.K = L.top_k; a.I = L.inter; a.Is = L.shared_inter;
  a.eps = L.rms_eps;
  a.x = x; a.out = out; a.idx_out = idx_out; a.w_out = w_out;
  a.ws = ws;
  a.wl = ws_layout(a.E, a.K, a.I, a.Is, 1);
  a.nR = cdiv(a.E, kRowsPerUnit);
  a.nS = a.Is / kGuRows;
  a.perG = a.I / kGuRows;
  a.nG = a.K * a.perG;
  a.nD = a.H / kRowsPerUnit;
  if (a.nS + a.nG + a.nD > ctl::kMaxFlags) return QMOE_ERR_UNSUPPORTED;
  const size_t lds = step_lds(a.H, a.E, a.I, a.Is, a.K);
  const int blocks = a.nR + a.nS + a.nG + a.nD;
  const StackLayerDev* tab = static_cast<const StackLayerDev*>(table);
  hipError_t e;
  if (a.H == 2816 && a.I == 704 && a.Is == 2112 && a.E == 128)
    e = launch_stack_kernel<2816, 704, 2112, 128>(a, tab, n_layers, xb, lout, blocks, lds, stream);
  else if (a.H == 512 && a.I == 256 && a.Is == 512 && a.E == 32)
    e = launch_stack_kernel<512, 256, 512, 32>(a, tab, n_layers, xb, lout, blocks, lds, stream);
  else
    e = launch_stack_kernel<0, 0, 0, 0>(a, tab, n_layers, xb, lout, blocks, lds, stream);
  if (e == hipErrorCooperativeLaunchTooLarge) {
    (void)hipGetLastError();
    return QMOE_ERR_UNSUPPORTED;
  }
  return e == hipSuccess ? QMOE_OK : QMOE_ERR_HIP;
}

}  // namespace qmoe
