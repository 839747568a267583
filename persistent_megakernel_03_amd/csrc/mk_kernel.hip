// The persistent decode megakernel for gfx950 (CDNA4), and the weight re-layout kernels.
//
// One workgroup of 512 threads (8 wave64s) runs on each CU, and all of them must be resident at once
// (the LDS allows one per CU, the grid is the CU count; multi-step launches are cooperative, so the
// runtime guarantees it; a single step uses a plain launch on a device running nothing else, and a
// wait that can never be met ends at the watchdog). Each workgroup walks its own task queue, built
// ahead of time, once per step of the launch (the AOT mode of "MPK: A Compiler and Runtime for
// Mega-Kernelizing Tensor Programs", analogy 3), or, in the run-time mode, takes tasks from one
// device-wide ready queue. For each task it:
//   - issues the loads that do not depend on this step (weights, cached K/V rows),
//   - polls for its inputs: epoch-tagged activation words, each carrying the step that wrote it,
//   - runs the tile and its epilogue, and stores its outputs tagged with the step's epoch.
// This is the worker loop of the Mirage Persistent Kernel ("LLMs in einen MegaKernel kompilieren",
// "Worker" and "Ereignisbasierte Ausführung"), with the pages' separate scheduler SMs folded into the
// workers: every CU keeps streaming weights, and an event is the set of tags its consumer polls.
// Only the LM head's partial maxima travel under flags (the argmax waits for them).
//
// Memory model. Data that one CU writes and another CU reads in the same step goes through
// agent-scope atomic loads and stores (the sc1 cache policy), coherent across the XCDs' separate L2
// caches. A tagged word is one 64-bit single-copy-atomic store (value | epoch << 32), so a consumer
// that sees this step's epoch sees this step's value, whatever the order in which words land. For the
// flags, a producer's waves wait for their stores to complete (s_waitcnt vmcnt(0)) before one lane
// stores the flag, and the consumer issues its data loads only after the flags. Weights and the K/V
// rows of earlier steps are immutable within a step and are read with plain nontemporal loads.
#include <hip/hip_runtime.h>
#include <cstdlib>
#include <mutex>
#include <stdint.h>

#include "mk_graph.h"

namespace mk {

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int NT = 512;     // threads per workgroup
constexpr int NW = NT / 64; // waves per workgroup
constexpr int NSLOT = 16;   // 1 KB weight units in flight per wave (16 KB), one register slot each
// s_getreg operand for the hardware register holding the wave's XCD id (register 20 on gfx940-family
// parts, bits 3..0): id | offset << 6 | (size - 1) << 11
constexpr int kHwRegXccId = 20 | (0 << 6) | ((4 - 1) << 11);

// ----------------------------------------------------------------------------- helpers
__device__ __forceinline__ float ldc(const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ uint32_t ldc(const uint32_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ uint64_t ldc(const uint64_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void stc(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void stc(uint32_t* p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void stc(uint64_t* p, uint64_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// fp32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Wait until this wave's vector memory operations (loads, stores, LDS DMA) have completed. Issued
// through the builtin (s_waitcnt with vmcnt 0 and the other counters at their maximum: 0x0F70 on
// gfx9-family encodings) rather than inline assembly, so that the compiler's own wait insertion
// knows the counter is drained afterwards; otherwise it treats LDS DMA as possibly pending and
// guards later LDS accesses with full waits.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier that orders LDS only. __syncthreads() also carries a workgroup release fence,
// which waits for every outstanding global load (vmcnt(0)) and would stall the weight prefetch
// in flight across task boundaries. Global memory is ordered explicitly in this kernel: a wave
// waits for its own stores (wait_stores) before any flag is published, and cross-CU data is read
// with agent-scope loads issued after the flags were observed.
__device__ __forceinline__ void bar() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// DPP moves within a row of 16 lanes: swap pairs, swap pairs of pairs, mirror within 8, mirror within 16.
// Applied in turn, each adds a lane's partner from another group, so LPP consecutive lanes end with the
// sum over all of them (LPP = 8 uses the first three).
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// The two values of a lane pair {l, l ^ OFF}, in the same order on both lanes: (lower lane's,
// upper lane's). Distances 16 and 32 swap rows or halves of the wave in one VALU instruction.
template <int OFF>
__device__ __forceinline__ void lane_pair(float v, float& lo, float& hi) {
  if constexpr (OFF == 16 || OFF == 32) {
    const uint32_t b = __float_as_uint(v);
    const auto r = OFF == 16 ? __builtin_amdgcn_permlane16_swap(b, b, false, false)
                             : __builtin_amdgcn_permlane32_swap(b, b, false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
  } else {
    const float o = __shfl_xor(v, OFF);
    const bool upper = (threadIdx.x & OFF) != 0;
    lo = upper ? o : v;
    hi = upper ? v : o;
  }
}

// Sum over aligned groups of n lanes (n a power of two up to 64), the same bits on every lane of a
// group: four DPP steps within rows of 16 lanes, then row and half-wave swaps.
__device__ __forceinline__ float lanes_sum(float v, int n) {
  if (n >= 2) v = dpp_add<0xB1>(v);
  if (n >= 4) v = dpp_add<0x4E>(v);
  if (n >= 8) v = dpp_add<0x141>(v);
  if (n >= 16) v = dpp_add<0x140>(v);
  if (n >= 32) {
    float a, b;
    lane_pair<16>(v, a, b);
    v = a + b;
  }
  if (n >= 64) {
    float a, b;
    lane_pair<32>(v, a, b);
    v = a + b;
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) { return lanes_sum(v, 64); }
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// Small control block at the start of LDS.
struct Ctl {
  GemvGeom geoms[G_COUNT];  // copied once per launch
  int32_t ctx[16];          // context lengths of the first 16 sequences, read once per launch
  float red[NW * 8];
  // attention work of this step: blocks per (sequence, KV head) segment of sequence s (0 when the
  // sequence is inactive), and the first block of sequence s's segments in the layer's block order
  int32_t anb[16], aoff[17];
  int32_t ate;  // attention tasks that get blocks this step (the rest are empty)
  uint32_t aborted;
  uint64_t kred[NW];
  uint64_t t_ready;         // trace: when the running task's inputs were all present
  uint64_t t_streamed;      // trace: when its own streaming ended
  int32_t jtask;            // dynamic scheduling: the task taken from the ready queue (< 0: none)
  int32_t jpush, jc0, jn;   // the consumer range this task's completion released, and its queue slots
};

__device__ __forceinline__ float block_sum(float v, Ctl* ctl) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  bar();
  if (l == 0) ctl->red[w] = v;
  bar();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) s += ctl->red[i];
  return s;
}

__device__ void raise_error(const KernelParams& p, uint32_t code, uint32_t a, uint32_t b) {
  uint32_t expected = 0;
  if (__hip_atomic_compare_exchange_strong(&p.err[E_CODE], &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT)) {
    stc(&p.err[E_INFO0], a);
    stc(&p.err[E_INFO1], b);
  }
}

// ----------------------------------------------------------------------------- tagged activations
// Values that one CU hands to another within a step travel as 64-bit words: the fp32 bits (or a
// packed bf16 pair) in the low half and the step epoch in the high half, written by one
// single-copy-atomic store. A consumer polls the words it needs until each carries the current
// epoch. The data is thus its own ready signal: a producer neither waits for its stores to complete
// nor sets a flag afterwards, and a consumer needs no second round trip to fetch the data after
// seeing a flag. With cross-XCD round trips near a microsecond and every layer crossing five
// dependency boundaries, those two round trips are most of a boundary's cost. Each buffer holds one
// layer, so every word is written exactly once per step and the epoch alone names its version.
__device__ __forceinline__ void st_tag(uint64_t* p, uint32_t bits, uint32_t ep) { stc(p, ((uint64_t)ep << 32) | bits); }
__device__ __forceinline__ void st_tagf(uint64_t* p, float v, uint32_t ep) { st_tag(p, __float_as_uint(v), ep); }

__device__ __forceinline__ uint64_t* xt_at(const KernelParams& p, int l, int which, int s) {
  return p.xt + (((size_t)l * 2 + which) * p.max_seqs + s) * p.d;
}
__device__ __forceinline__ uint64_t* qt_at(const KernelParams& p, int l, int s) {
  return p.qt + ((size_t)l * p.max_seqs + s) * p.hq * p.dh;
}
__device__ __forceinline__ uint64_t* ot_at(const KernelParams& p, int l, int s) {
  return p.ot + ((size_t)l * p.max_seqs + s) * p.hq * p.dh;
}
__device__ __forceinline__ uint64_t* ht_at(const KernelParams& p, int l, int s) {
  return p.ht + ((size_t)l * p.max_seqs + s) * p.f;
}
__device__ __forceinline__ uint64_t* kvt_at(const KernelParams& p, int l, int s, int kv, int grp) {
  return p.kvt + ((((size_t)l * p.max_seqs + s) * 2 + kv) * p.hk + grp) * (p.dh / 2);
}

// Coherent 64-bit load through a buffer resource. The lane's byte offset sits in one VGPR and the
// word's offset in an SGPR, so polling K words per lane costs no per-word address registers. The
// volatile bit keeps the compiler from hoisting re-loads out of a poll loop; such loads also bypass
// the caches that are not coherent across XCDs.
typedef unsigned v2u __attribute__((ext_vector_type(2)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tag_rsrc(const uint64_t* base) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ uint64_t ld_tag(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const v2u v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, (int)((1u << 31) | 16u));
  return ((uint64_t)v.y << 32) | v.x;
}
__device__ __forceinline__ uint32_t first_words(int n) { return n >= 32 ? ~0u : n <= 0 ? 0u : (1u << n) - 1u; }

// Every 8th pass of a poll: whether the kernel is aborting, or the wait has outlived the watchdog
// (then the timeout is raised, naming `what`, and the kernel aborts). The abort flag is a load of its
// own that would double the time of every pass if read on each; an abort only drains the grid after
// an error, so the few extra passes it takes to notice cost nothing that matters.
__device__ __forceinline__ bool poll_give_up(const KernelParams& p, uint32_t ep, uint32_t pass, uint64_t t0, uint32_t what) {
  if ((pass & 7u) != 0u) return false;
  if (ldc(&p.err[E_ABORT])) return true;
  if (__builtin_amdgcn_s_memrealtime() - t0 > p.watchdog_ticks) {
    if ((threadIdx.x & 63) == 0) {
      raise_error(p, ERR_TIMEOUT, what, ep);
      stc(&p.err[E_ABORT], 1u);
    }
    return true;
  }
  return false;
}

// Polls this thread's tagged words k (bit k of `pending`, k < K); word k sits at byte base + voff(k)
// + soff(k), soff uniform across the wave. sink(k, bits) receives a word's low half once the word
// carries the step's epoch `ep`. Each pass issues the loads of all words still stale before checking any;
// passes follow each other with no sleep between them (a pass is a memory round trip already, and a
// sleep measured 8-10 us per token slower on the 8B decode). A wave
// stops when all its lanes are done, when the kernel is aborting, or when the watchdog expires (which
// raises the timeout, naming `what`, and aborts the kernel).
template <int K, typename Voff, typename Soff, typename Sink>
__device__ __forceinline__ void poll_tagged(const KernelParams& p, uint32_t ep, const uint64_t* base, Voff voff, Soff soff,
                                            uint32_t pending, uint32_t what, Sink sink) {
  const __amdgpu_buffer_rsrc_t r = tag_rsrc(base);
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (uint32_t pass = 1;; ++pass) {
    uint64_t w[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
      if ((pending >> k) & 1u) w[k] = ld_tag(r, voff(k), soff(k));
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (((pending >> k) & 1u) && (uint32_t)(w[k] >> 32) == ep) {
        sink(k, (uint32_t)w[k]);
        pending &= ~(1u << k);
      }
    }
    if (!__any(pending != 0u)) break;
    if (poll_give_up(p, ep, pass, t0, what)) break;
  }
}

// Finishes a poll whose first loads are already in w (bit k of `pending`: word k issued, not yet
// seen current): checks the words, and re-issues reload(k) for those still stale, reusing w, with the
// same abort and watchdog rules as poll_tagged.
template <int K, typename Reload, typename Sink>
__device__ __forceinline__ void poll_finish(const KernelParams& p, uint32_t ep, uint64_t (&w)[K], uint32_t pending,
                                            uint32_t what, Reload reload, Sink sink) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (uint32_t pass = 1;; ++pass) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (((pending >> k) & 1u) && (uint32_t)(w[k] >> 32) == ep) {
        sink(k, (uint32_t)w[k]);
        pending &= ~(1u << k);
      }
    }
    if (!__any(pending != 0u)) break;
    if (poll_give_up(p, ep, pass, t0, what)) break;
#pragma unroll
    for (int k = 0; k < K; ++k)
      if ((pending >> k) & 1u) w[k] = reload(k);
  }
}

// The watchdog's names for a wait on the next step's token and for a wait on a slot of the ready queue
// (event indices name the other waits).
constexpr uint32_t kWhatToken = 0xFFFFFFFEu;
constexpr uint32_t kWhatQueue = 0xFFFFFFFDu;

// A whole vector src[0, n): wave w polls the contiguous words [w * chunk, (w + 1) * chunk), chunk =
// n / 8 rounded up to 64, lane l taking words l, l + 64, ..., so each load is one coalesced 512-byte
// row and the word offsets fit the instruction's immediate (with one SGPR per 4 KB).
__device__ __forceinline__ int poll_chunk(int n) { return ((n + NW * 64 - 1) / (NW * 64)) * 64; }
__device__ __forceinline__ int poll_index(int n, int k) {
  return (int)(threadIdx.x >> 6) * poll_chunk(n) + (int)(threadIdx.x & 63) + 64 * k;
}
template <int K, typename Sink>
__device__ __forceinline__ void poll_vector(const KernelParams& p, uint32_t ep, const uint64_t* src, int n, uint32_t what,
                                            Sink sink) {
  const int i0 = poll_index(n, 0);
  const int cnt = min(poll_chunk(n) / 64, (n - i0 + 63) / 64);
  poll_tagged<K>(p, ep, src, [&](int k) { return i0 * 8 + (k & 7) * 512; }, [](int k) { return (k >> 3) * 4096; },
                 first_words(cnt), what, sink);
}

// ----------------------------------------------------------------------------- events
// Wave 0 polls every producer flag of the event until all hold >= the step's epoch. A watchdog on the
// 100 MHz real-time counter turns a wait that never ends into an error and a kernel-wide abort.
__device__ __forceinline__ void wait_event(const KernelParams& p, uint32_t ep, const TaskDesc& t, Ctl* ctl) {
  if (threadIdx.x < 64) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    const int lane = threadIdx.x;
    uint32_t ab = 0;
    while (true) {
      bool ok = true;
      for (int i = lane; i < t.wait_nslots; i += 64) ok = ok && (ldc(&p.flags[t.wait_slot0 + i]) >= ep);
      if (__all(ok)) break;
      ab = ldc(&p.err[E_ABORT]);
      if (ab) break;
      if (__builtin_amdgcn_s_memrealtime() - t0 > p.watchdog_ticks) {
        if (lane == 0) {
          raise_error(p, ERR_TIMEOUT, (uint32_t)t.wait_ev, ep);
          stc(&p.err[E_ABORT], 1u);
        }
        ab = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (lane == 0) ctl->aborted = ab;
  }
  bar();
}

// Publishing a finished task: every wave waits for its own stores, the workgroup meets at a
// barrier, and then one lane per slot stores the epoch. `my_sig` is this thread's slot (loaded
// when the task started, so no load sits on the publish path), or -1. Only wave 0 holds slots
// (a task has at most 64).
__device__ __forceinline__ void publish(const KernelParams& p, uint32_t ep, int my_sig) {
  if (my_sig >= 0) stc(&p.flags[my_sig], ep);
}

// ----------------------------------------------------------------------------- GEMV tile
// ys[r] = sum_k W[row0 + r][k] * xs[k] for the task's rows. Row groups are split evenly over
// the 8 waves. Each wave streams its contiguous run of 1 KB units with nontemporal dwordx4
// loads, NSLOT units in flight. The xs entries past K are zero, and so are the padded weights.
// The GEMV input vector sits in LDS as two planes: plane A holds elements 8p..8p+3 of every
// 16-byte weight piece p at A[4p..4p+3], plane B holds 8p+4..8p+7 at B[4p..4p+3]. Lanes that
// read consecutive pieces then read consecutive 16-byte words of each plane, free of bank
// conflicts (a plain [K] layout puts lanes 32 bytes apart: an 8-way conflict).
__device__ __forceinline__ int xs_index(int i, int npieces) {
  const int p = i >> 3, e = i & 7;
  return (e < 4) ? (p << 2) + e : (npieces << 2) + (p << 2) + (e - 4);
}

__device__ __forceinline__ void unit_fma_v(const v4u w, const v4f a, const v4f b, float& acc0, float& acc1) {
  acc0 = fmaf(bf_lo(w.x), a.x, acc0);
  acc1 = fmaf(bf_hi(w.x), a.y, acc1);
  acc0 = fmaf(bf_lo(w.y), a.z, acc0);
  acc1 = fmaf(bf_hi(w.y), a.w, acc1);
  acc0 = fmaf(bf_lo(w.z), b.x, acc0);
  acc1 = fmaf(bf_hi(w.z), b.y, acc1);
  acc0 = fmaf(bf_lo(w.w), b.z, acc0);
  acc1 = fmaf(bf_hi(w.w), b.w, acc1);
}
__device__ __forceinline__ void unit_fma(const v4u w, const float* xa, const float* xb, float& acc0, float& acc1) {
  unit_fma_v(w, *(const v4f*)xa, *(const v4f*)xb, acc0, acc1);
}

// FP8 weights: the lane's 16 bytes are the E4M3 codes of two pieces, the piece of bf16-layout unit
// 2u (bytes 0..7, elements 0..7) and of unit 2u + 1 (bytes 8..15); the conversion to fp32 is exact.
typedef float v2f __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void unit_fma8_v(const v4u w, const v4f a0, const v4f b0, const v4f a1, const v4f b1,
                                            float& acc0, float& acc1) {
  v2f c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
  acc0 = fmaf(c.x, a0.x, acc0);
  acc1 = fmaf(c.y, a0.y, acc1);
  c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
  acc0 = fmaf(c.x, a0.z, acc0);
  acc1 = fmaf(c.y, a0.w, acc1);
  c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
  acc0 = fmaf(c.x, b0.x, acc0);
  acc1 = fmaf(c.y, b0.y, acc1);
  c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
  acc0 = fmaf(c.x, b0.z, acc0);
  acc1 = fmaf(c.y, b0.w, acc1);
  c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.z, false);
  acc0 = fmaf(c.x, a1.x, acc0);
  acc1 = fmaf(c.y, a1.y, acc1);
  c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.z, true);
  acc0 = fmaf(c.x, a1.z, acc0);
  acc1 = fmaf(c.y, a1.w, acc1);
  c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.w, false);
  acc0 = fmaf(c.x, b1.x, acc0);
  acc1 = fmaf(c.y, b1.y, acc1);
  c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.w, true);
  acc0 = fmaf(c.x, b1.z, acc0);
  acc1 = fmaf(c.y, b1.w, acc1);
}
__device__ __forceinline__ void unit_fma8(const v4u w, const float* xa0, const float* xb0, const float* xa1,
                                          const float* xb1, float& acc0, float& acc1) {
  unit_fma8_v(w, *(const v4f*)xa0, *(const v4f*)xb0, *(const v4f*)xa1, *(const v4f*)xb1, acc0, acc1);
}

// Register pipeline of one wave's weight stream: NSLOT slots of one unit each. A task's first
// NSLOT units are loaded before the task polls for its inputs: weights do not depend on
// activations, so the HBM stream keeps running across the dependency wait. The registers flow
// straight from the loads into the GEMV without copies (a copy would have to wait for the loads
// to land).
struct WPipe {
  v4u R[NSLOT];
};

struct WaveRun {
  const v4u* src;  // this lane's first 16-byte piece of the wave's run of units
  int nunits, g0;  // units in the run; first row group
};

template <bool FP8>
__device__ __forceinline__ WaveRun wave_run(const KernelParams& p, const TaskDesc& t, const GemvGeom& gm) {
  // The wave index is made explicitly wave-uniform so that unit counts and loop bounds live in
  // scalar registers and loads need no per-lane branches.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rows = t.row1 - t.row0;
  const int ngroups = (rows + gm.rg - 1) / gm.rg;
  const int gA = ngroups * wave / NW, gB = ngroups * (wave + 1) / NW;
  WaveRun r;
  r.g0 = gA;
  const int su = FP8 ? gm.S >> 1 : gm.S;  // units per row group
  r.nunits = (gB - gA) * su;
  r.src = (const v4u*)(p.wpacked + t.wofs) + (size_t)gA * su * 64 + (threadIdx.x & 63);
  return r;
}

// Within a round the loads are unconditional (units past the run re-read its last unit and are never
// consumed), so the in-order wait counter is exact: a slot is waited for only when consumed. A round
// whose refills would all lie past the run is written without loads (a branch on the wave-uniform
// unit count around a whole round keeps the counts exact): such refills cost no bytes worth having,
// but they sit in the in-order queue ahead of the next task's first loads and input poll.
__device__ __forceinline__ v4u load_unit(const WaveRun& w, int i) {
  return __builtin_nontemporal_load(w.src + (size_t)(uint32_t)min(i, w.nunits - 1) * 64);  // i >= 0, nunits >= 1
}

__device__ __forceinline__ bool is_gemv(int type) {
  return type == T_QKV || type == T_OPROJ || type == T_GATEUP || type == T_DOWN || type == T_LMHEAD;
}

__device__ __forceinline__ WaveRun dummy_run(const KernelParams& p) {
  WaveRun w;
  w.src = (const v4u*)p.wpacked + (threadIdx.x & 63);
  w.nunits = 1;
  w.g0 = 0;
  return w;
}

// The LDS stage of each wave: kStageUnits units that follow its first NSLOT register units.
__shared__ v4u g_stage[NW][kStageUnits][64];

// Issues the DMA of units NSLOT .. NSLOT + kStageUnits - 1 of the wave's run into its stage (only
// units the run has). Each lane's 16 bytes land at lane * 16 of the unit's 1 KB slot, at the LDS
// address in M0. The DMA is written as inline assembly and issued before any other load of the task:
// the compiler then neither sees a DMA in flight (with one, it drains the whole counter before any
// LDS access it cannot prove separate) nor miscounts the waits of later loads, all of which are
// younger. Its completion is waited for explicitly where the stage is read. No register receives
// data, so nothing is left to be overwritten in flight; M0 (the LDS address) is restored after issue.
__device__ __forceinline__ void stage_units(const WaveRun& w) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int j = 0; j < kStageUnits; ++j)
    if (NSLOT + j < w.nunits) {
      const uint32_t dst = (uint32_t)(size_t)(__attribute__((address_space(3))) void*)&g_stage[wave][j][0];
      uint32_t keep;  // M0 is the compiler's: it is saved and restored around the DMA
      asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt\n\t"
                   "s_nop 4\n\ts_mov_b32 m0, %0"
                   : "=&s"(keep)
                   : "v"(w.src + (size_t)(NSLOT + j) * 64), "s"(dst)
                   : "memory");
    }
}

// gemv_tile for rows of 4096 inputs (512 pieces: 64 lanes per row, 8 units per row). Each lane then
// meets the same 8 pieces in every row it streams, so it holds their 64 inputs in registers for the
// whole tile instead of reading them from LDS per unit. The position of a unit in its row is known at
// compile time in every slot: the run starts at a row, the first round holds units 0..NSLOT-1 and the
// stage the next kStageUnits, and every later round starts NSLOT + kStageUnits + NSLOT r, which is 2
// mod 8 (FP8: unit i covers bf16-layout units 2i and 2i + 1). The arithmetic, and its order, are those
// of the general tile below.
template <bool FP8, bool S2>
__device__ __forceinline__ void gemv_tile_r512(const KernelParams& p, const TaskDesc& t, const GemvGeom gm, const float* xs,
                                               float* ys, WPipe& wp, bool restage, const WaveRun next, const float* ysc) {
  static_assert(NSLOT % 8 == 0, "unit positions in the row are fixed per slot");
  // units held before the register rounds: the first round, the stage and (S2) the second stage
  constexpr int PRE = NSLOT + kStageUnits + (S2 ? kStage2Units : 0);
  const WaveRun w = wave_run<FP8>(p, t, gm);
  const int nunits = w.nunits;
  if (nunits <= 0) return;
  // the lane index made opaque per call: its input addresses are computed here, not held in
  // registers through every other task
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rows = t.row1 - t.row0;
  v4f xa[8], xb[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    xa[u] = *(const v4f*)(xs + (u * 64 + lane) * 4);
    xb[u] = *(const v4f*)(xs + 512 * 4 + (u * 64 + lane) * 4);
  }
  int g = w.g0;
  float acc0 = 0.f, acc1 = 0.f;
  // unit of bf16-layout position ug (0..7) in its row; the row ends with position 7
  auto unit = [&](const v4u& wv, const int ug) {
    if constexpr (FP8) {
      unit_fma8_v(wv, xa[ug], xb[ug], xa[ug + 1], xb[ug + 1], acc0, acc1);
    } else {
      unit_fma_v(wv, xa[ug], xb[ug], acc0, acc1);
    }
    if (ug + (FP8 ? 2 : 1) == 8) {
      const float acc = lanes_sum(acc0 + acc1, 64);
      if (lane == 0 && g < rows) ys[g] = FP8 ? acc * ysc[g] : acc;
      acc0 = 0.f;
      acc1 = 0.f;
      ++g;
    }
  };
  constexpr int US = FP8 ? 2 : 1;  // bf16-layout units per unit
  const bool more = nunits > PRE;  // wave-uniform: the run goes on past the prefetched units
  if (more) {
#pragma unroll
    for (int j = 0; j < NSLOT; ++j) {
      if (j < nunits) unit(wp.R[j], (US * j) & 7);
      wp.R[j] = load_unit(w, j + PRE);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int j = 0; j < NSLOT; ++j)
      if (j < nunits) unit(wp.R[j], (US * j) & 7);
  }
  if (nunits > NSLOT) {
    // both stages' DMA went out before this round's refills, the youngest NSLOT loads (with no
    // refills, everything outstanding)
    if (more) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NSLOT) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // staged units, each read one unit ahead of its use (the reads are issued before the row-end
    // stores of the unit before, so they overlap its arithmetic)
    const v4u* st2 = (const v4u*)((const char*)xs + p.stage2_off) + wave * kStage2Units * 64 + lane;
    constexpr int NST = kStageUnits + kStage2Units;
    auto staged_at = [&](int j) { return j < kStageUnits ? g_stage[wave][j][lane] : st2[(j - kStageUnits) * 64]; };
    v4u cur = staged_at(0);
#pragma unroll
    for (int j = 0; j < NST; ++j) {
      const v4u nxt = staged_at(j + 1 < NST ? j + 1 : j);
      if (NSLOT + j < nunits) unit(cur, (US * (NSLOT + j)) & 7);
      cur = nxt;
    }
  }
  if (restage) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    stage_units(next);
  }
  // rounds whose refills still reach into the run, then the last round with no refills
  int i0 = PRE;
  for (; i0 + NSLOT < nunits; i0 += NSLOT) {
#pragma unroll
    for (int j = 0; j < NSLOT; ++j) {
      unit(wp.R[j], (US * (PRE + j)) & 7);
      wp.R[j] = load_unit(w, i0 + j + NSLOT);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (i0 < nunits) {
#pragma unroll
    for (int j = 0; j < NSLOT; ++j)
      if (i0 + j < nunits) unit(wp.R[j], (US * (PRE + j)) & 7);
  }
}

// One sequence, rows of 4096 inputs: the DMA of the wave's units NSLOT + kStageUnits .. + kStage2Units - 1
// (those the run has) into its part of the second stage, at byte offset stage2_off of the working set
// `ws`. Issued after the task's register units, so the polls before it do not wait for it.
__device__ __forceinline__ void stage2_units(const WaveRun& w, const float* ws, int stage2_off) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int j = 0; j < kStage2Units; ++j)
    if (NSLOT + kStageUnits + j < w.nunits) {
      const uint32_t dst = (uint32_t)(size_t)(__attribute__((address_space(3))) void*)((const char*)ws + stage2_off) +
                           (uint32_t)((wave * kStage2Units + j) * 1024);
      uint32_t keep;
      asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt\n\t"
                   "s_nop 4\n\ts_mov_b32 m0, %0"
                   : "=&s"(keep)
                   : "v"(w.src + (size_t)(NSLOT + kStageUnits + j) * 64), "s"(dst)
                   : "memory");
    }
}

// restage: once this task has read its own staged units, the stage receives those of run `next`.
// FP8: each unit covers two bf16-layout units of the row group, and a finished row is scaled by its
// row's 2^e (ysc, in LDS).
template <bool FP8>
__device__ __forceinline__ void gemv_tile(const KernelParams& p, const TaskDesc& t, const GemvGeom gm, const float* xs, float* ys,
                          WPipe& wp, bool restage, const WaveRun next, const float* ysc) {
  if (gm.lpr == 64 && gm.S == 8 && p.stage2_off > 0) {
    gemv_tile_r512<FP8, true>(p, t, gm, xs, ys, wp, restage, next, ysc);
    return;
  }
  const WaveRun w = wave_run<FP8>(p, t, gm);
  const int nunits = w.nunits;
  if (nunits <= 0) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rows = t.row1 - t.row0;
  const int S = gm.S, lpr = gm.lpr;
  const int sub = lane & (lpr - 1), rin = lane / lpr;
  const float* xa = xs + sub * 4;
  const float* xb = xs + S * lpr * 4 + sub * 4;
  int g = w.g0, ug = 0;
  float acc0 = 0.f, acc1 = 0.f;

  auto unit = [&](const v4u& wv) {
    if constexpr (FP8) {
      unit_fma8(wv, xa + ug * lpr * 4, xb + ug * lpr * 4, xa + (ug + 1) * lpr * 4, xb + (ug + 1) * lpr * 4, acc0, acc1);
      ug += 2;
    } else {
      unit_fma(wv, xa + ug * lpr * 4, xb + ug * lpr * 4, acc0, acc1);
      ++ug;
    }
    if (ug == S) {
      const float acc = lanes_sum(acc0 + acc1, lpr);
      const int r = g * gm.rg + rin;
      if (sub == 0 && r < rows) ys[r] = FP8 ? acc * ysc[r] : acc;
      acc0 = 0.f;
      acc1 = 0.f;
      ug = 0;
      ++g;
    }
  };
  // Units in run order: 0 .. NSLOT - 1 from the registers, the next kStageUnits from the LDS stage,
  // then the rest through the registers again. Slot j holds unit i0 + j of its round and is refilled
  // with the unit NSLOT further on as soon as it has been consumed (the first round's refills skip
  // the staged units), so NSLOT - 1 loads stay in flight while a unit is processed. Refills past the
  // run re-read its last unit; the last round, whose refills would all lie past it, has none. A
  // scheduling barrier after each slot keeps each refill
  // after its slot's use. The compiler still waits for most of a round's loads at the round's start
  // (the first fill is not kept in slot order), so about one round of loads is in flight per wave;
  // measured on the 8B decode, this streams slightly faster than a strict slot-by-slot pipeline
  // with 16 loads always in flight: the HBM stream is already saturated.
#pragma unroll
  for (int j = 0; j < NSLOT; ++j) {
    if (j < nunits) unit(wp.R[j]);
    wp.R[j] = load_unit(w, j + NSLOT + kStageUnits);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (nunits > NSLOT) {
    // The stage's DMA was issued before every other load of the task, the first round's NSLOT refills
    // are the youngest, and the counter completes in order: once at most NSLOT loads are outstanding,
    // it has landed. (The compiler does not know of the DMA, so the wait is explicit.)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NSLOT) : "memory");
#pragma unroll
    for (int j = 0; j < kStageUnits; ++j)
      if (NSLOT + j < nunits) unit(g_stage[wave][j][lane]);
  }
  if (restage) {  // the stage's reads have returned before the DMA may overwrite it
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    stage_units(next);
  }
  // rounds whose refills still reach into the run, then the last round with no refills
  int i0 = NSLOT + kStageUnits;
  for (; i0 + NSLOT < nunits; i0 += NSLOT) {
#pragma unroll
    for (int j = 0; j < NSLOT; ++j) {
      unit(wp.R[j]);
      wp.R[j] = load_unit(w, i0 + j + NSLOT);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (i0 < nunits) {
#pragma unroll
    for (int j = 0; j < NSLOT; ++j)
      if (i0 + j < nunits) unit(wp.R[j]);
  }
}

__device__ __forceinline__ int token_of(const KernelParams& p, int s) {
  int tok = p.tokens_in[s];
  if (tok < 0 || tok >= p.vocab) {
    if (threadIdx.x == 0) raise_error(p, ERR_TOKEN, (uint32_t)s, (uint32_t)tok);
    tok = 0;
  }
  return tok;
}

// Position of sequence s's current token, or -1 (error latched) when the cache cannot hold it.
__device__ __forceinline__ int checked_pos(const KernelParams& p, const Ctl* ctl, int s) {
  const int pos = ctl->ctx[s];
  if (pos < 0 || pos >= p.max_pos) {
    if (threadIdx.x == 0) raise_error(p, ERR_CTX, (uint32_t)s, (uint32_t)pos);
    return -1;
  }
  return pos;
}

__device__ __forceinline__ const uint16_t* layer_norm_gain(const KernelParams& p, int l, int which) {
  return p.norms + ((size_t)l * 2 + which) * p.d;
}

// ----------------------------------------------------------------------------- QKV
// Per 4-row set of the packed QKV rows: what the epilogue needs besides the GEMV results. Loaded
// before the GEMV so that these loads' latency hides under the weight stream.
struct QkvSet {
  float2 cs0, cs1;  // rotary cos/sin of the set's two pairs (q and k heads)
  float b0, b1, b2, b3;
  int blk;          // KV block of the current position (k and v heads)
};

__device__ __forceinline__ QkvSet qkv_set_consts(const KernelParams& p, int l, int r, int pos, int s) {
  const int G = p.hq / p.hk, dh = p.dh, Rg = (G + 2) * dh;
  const int grp = r / Rg, within = r % Rg, slot = within / dh, jh = within % dh, i0 = jh >> 1;
  QkvSet c;
  c.cs0 = make_float2(1.f, 0.f);
  c.cs1 = make_float2(1.f, 0.f);
  c.b0 = c.b1 = c.b2 = c.b3 = 0.f;
  c.blk = 0;
  (void)grp;
  if (p.bias) {
    const uint16_t* b = p.bias + (size_t)l * (p.hq + 2 * p.hk) * dh + r;
    c.b0 = bf2f(b[0]); c.b1 = bf2f(b[1]); c.b2 = bf2f(b[2]); c.b3 = bf2f(b[3]);
  }
  if (slot <= G) {
    c.cs0 = ((const float2*)p.rope)[(size_t)pos * (dh / 2) + i0];
    c.cs1 = ((const float2*)p.rope)[(size_t)pos * (dh / 2) + i0 + 1];
  }
  if (slot >= G) c.blk = p.page_table[(size_t)s * p.max_blocks + pos / 16];
  return c;
}

// The epilogue of one 4-row set of packed QKV rows (r = its first row) for sequence s: bias, the
// rotation of q and k, then the stores. The rotated query goes to the tagged query buffer; the key or
// value pairs, rounded to bf16, go to the tagged current-row buffer and to the cache at position pos.
// An out-of-range position (pos < 0) skips the append; a bad block is reported and skipped.
__device__ __forceinline__ void qkv_store_set(const KernelParams& p, int l, int s, int r, float y0, float y1, float y2,
                                              float y3, const QkvSet& c, int pos, uint16_t* const* pools, uint32_t ep) {
  const int G = p.hq / p.hk, dh = p.dh, Rg = (G + 2) * dh;
  const int grp = r / Rg, within = r % Rg, slot = within / dh, jh = within % dh;
  const int i0 = jh >> 1;  // even dim index; the set holds dims i0, i0 + dh/2, i0 + 1, i0 + 1 + dh/2
  y0 += c.b0;
  y1 += c.b1;
  y2 += c.b2;
  y3 += c.b3;
  if (slot <= G) {  // rotate q and k: pair (i0, i0 + dh/2) and pair (i0 + 1, i0 + 1 + dh/2)
    const float a0 = y0 * c.cs0.x - y1 * c.cs0.y, b0 = y1 * c.cs0.x + y0 * c.cs0.y;
    const float a1 = y2 * c.cs1.x - y3 * c.cs1.y, b1 = y3 * c.cs1.x + y2 * c.cs1.y;
    y0 = a0; y1 = b0; y2 = a1; y3 = b1;
  }
  if (slot < G) {
    uint64_t* q = qt_at(p, l, s) + (size_t)(grp * G + slot) * dh;
    st_tagf(&q[i0], y0, ep);
    st_tagf(&q[i0 + dh / 2], y1, ep);
    st_tagf(&q[i0 + 1], y2, ep);
    st_tagf(&q[i0 + 1 + dh / 2], y3, ep);
  } else {
    // the rounded key/value pairs go to the cache and, tagged, to this step's attention
    const uint32_t w0 = f2bf(y0) | (f2bf(y2) << 16), w1 = f2bf(y1) | (f2bf(y3) << 16);
    uint64_t* kv = kvt_at(p, l, s, slot == G ? 0 : 1, grp);
    st_tag(&kv[i0 >> 1], w0, ep);
    st_tag(&kv[(i0 + dh / 2) >> 1], w1, ep);
    const int blk = c.blk;
    if (blk < 0 || blk >= p.num_blocks) {
      raise_error(p, ERR_PAGE, (uint32_t)s, (uint32_t)blk);
      return;
    }
    if (pos < 0) return;
    uint16_t* pool = pools[(slot == G ? 0 : p.n_layers) + l];
    uint32_t* row = (uint32_t*)(pool + (((size_t)blk * p.hk + grp) * 16 + (pos & 15)) * dh);
    stc(&row[i0 >> 1], w0);
    stc(&row[(i0 + dh / 2) >> 1], w1);
  }
}

// ----------------------------------------------------------------------------- attention
// Grouped-query decode attention over the paged cache, split across CUs as flash-decoding.
//
// Work split. A layer's attention is a set of segments, one per (sequence s, KV head g): the cache
// blocks 0 .. nb_s - 1 of s, the last one holding the current position. The segments are laid end to
// end (sequence-major, then KV head) and this concatenation of blocks is cut into T equal ranges, one
// per attention task, at run time from the context lengths. Every task thus streams about the same
// number of key and value bytes whatever the mix of context lengths in the batch. The G query heads
// that share a KV head read each key and value row once ("LLM高速化勉強会資料", slide 28).
//
// Within a task's part of a segment, each wave streams its own groups of positions (64 lanes = PPW
// positions x DH/8 lanes, 8 dimensions per lane) through a register pipeline of keys and values, issued
// before the task polls for its queries: cached rows do not depend on this step ("MPK: A Compiler and
// Runtime for Mega-Kernelizing Tensor Programs", analogy 4). Each lane group keeps its own
// online-softmax state per head: running max, running sum, and the unnormalised output of its 8
// dimensions, rescaled when the max grows by more than 8 ("LLM高速化勉強会資料", slide 13;
// the online softmax of "Hạt nhân là gì và tại sao mọi người lại viết hạt nhân mới"). No barrier runs
// inside the stream. The lane groups of a wave, then the waves of the workgroup (in wave order), are
// merged by log-sum-exp. The current position's key and value come from this step's tagged words.
//
// A segment held whole by one task ends there as o = sum / l. A segment cut between tasks: each task
// but the last writes its partial (m, l, unnormalised o) as tagged words; the last (the one holding
// the segment's final block) polls them and merges them in task order.
template <int DH, int GMAX>
struct AttnShape {
  static constexpr int LPP = DH / 8;         // lanes per position
  static constexpr int PPW = 64 / LPP;       // positions per wave-wide load
  static constexpr int EPT = (GMAX * DH + NT - 1) / NT;  // output elements (head, dim) per thread
};

// First block of attention task i's range: T tasks cut W blocks evenly. (The first blocks are
// tabulated in LDS once per launch, alo[i] for i = 0..T; tasks past the T used this step start at W.)
__device__ __forceinline__ int attn_lo_of(int W, int T, int i) { return (int)((uint32_t)W * (uint32_t)i / (uint32_t)T); }
// With a cost per segment start PB > 0: T tasks cut the layer's cost evenly, where each block costs 1
// and each segment start after the first PB more (a cut that lands inside a start's cost falls on the
// segment's first block). Segment j (s, g) covers blocks aoff[s] + g nb .. + nb, nb = anb[s], and costs
// [S_j + PB j, S_j+1 + PB j) plus the PB before the next start.
__device__ int attn_lo_cost(const Ctl* ctl, int hk, int W, int T, int i, int PB) {
  if (PB == 0 || W == 0) return attn_lo_of(W, T, i);
  int nseg = 0;
  for (int s = 0; s < 16; ++s) nseg += ctl->anb[s] > 0 ? hk : 0;
  const int64_t t = ((int64_t)W + (int64_t)PB * (nseg - 1)) * i / T;
  int j = 0;
  for (int s = 0; s < 16; ++s) {
    const int nb = ctl->anb[s];
    if (nb == 0) continue;
    for (int g = 0; g < hk; ++g, ++j) {
      const int64_t s0 = ctl->aoff[s] + (int64_t)g * nb, s1 = s0 + nb;
      if (t < s1 + (int64_t)PB * (j + 1)) return (int)min(s1, max(s0, t - (int64_t)PB * j));
    }
  }
  return W;
}
// The task whose range holds block x: the last i < T with alo[i] <= x. With an even cut of W blocks
// this has a closed form; with a cut by cost, a search of alo (in LDS, non-decreasing).
__device__ __forceinline__ int attn_task_of(int W, int T, int x) {
  return min(T - 1, (int)(((uint32_t)(x + 1) * (uint32_t)T - 1u) / (uint32_t)W));
}
__device__ __forceinline__ int attn_task_of(const int32_t* alo, int T, int x) {
  int lo = 0, hi = T - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (alo[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Scores of one position for every head: s_h = q_h . k, this lane's 8 dimensions summed over the
// position's lanes. The heads' reductions are interleaved so that each DPP move reads a value written
// several instructions earlier.
template <int DH, int GMAX>
__device__ __forceinline__ void attn_scores(const v4u kv, bool valid, int G, const float (&qr)[GMAX][8], float (&a)[GMAX]) {
  const float kf[8] = {bf_lo(kv.x), bf_hi(kv.x), bf_lo(kv.y), bf_hi(kv.y), bf_lo(kv.z), bf_hi(kv.z), bf_lo(kv.w), bf_hi(kv.w)};
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    a[h] = 0.f;
    if (h < G) {
#pragma unroll
      for (int e = 0; e < 8; ++e) a[h] = fmaf(qr[h][e], kf[e], a[h]);
    }
  }
#pragma unroll
  for (int h = 0; h < GMAX; ++h) a[h] = dpp_add<0xB1>(a[h]);
#pragma unroll
  for (int h = 0; h < GMAX; ++h) a[h] = dpp_add<0x4E>(a[h]);
#pragma unroll
  for (int h = 0; h < GMAX; ++h) a[h] = dpp_add<0x141>(a[h]);
  if (DH == 128) {
#pragma unroll
    for (int h = 0; h < GMAX; ++h) a[h] = dpp_add<0x140>(a[h]);
  }
#pragma unroll
  for (int h = 0; h < GMAX; ++h) a[h] = valid ? a[h] : -INFINITY;
}

// Raises each head's running max to cover mx, rescaling the running sum and output.
template <int GMAX>
__device__ __forceinline__ void attn_rescale(int G, const float (&mx)[GMAX], float (&mr)[GMAX], float (&lr)[GMAX],
                                             float (&orr)[GMAX][8]) {
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    if (h >= G) break;
    const float mn = fmaxf(mr[h], mx[h]), al = __expf(mr[h] - mn);
    lr[h] *= al;
#pragma unroll
    for (int e = 0; e < 8; ++e) orr[h][e] *= al;
    mr[h] = mn;
  }
}

// Adds one position's values with weights exp(s_h - m_h).
template <int GMAX>
__device__ __forceinline__ void attn_accum(const v4u vv, int G, const float (&a)[GMAX], const float (&mr)[GMAX],
                                           float (&lr)[GMAX], float (&orr)[GMAX][8]) {
  const float vf[8] = {bf_lo(vv.x), bf_hi(vv.x), bf_lo(vv.y), bf_hi(vv.y), bf_lo(vv.z), bf_hi(vv.z), bf_lo(vv.w), bf_hi(vv.w)};
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    if (h >= G) break;
    const float pe = __expf(a[h] - mr[h]);
    lr[h] += pe;
#pragma unroll
    for (int e = 0; e < 8; ++e) orr[h][e] = fmaf(pe, vf[e], orr[h][e]);
  }
}

// Attention over positions [c0, c1) of segment (s, grp), c1 <= pos + 1 (pos = the current position).
// Returns, per output element (head, dim) of this thread, the merged (max, sum, unnormalised output).
// Log-sum-exp merge of the wave's lane groups (LPP lanes hold one position group's state): every
// lane ends with the merge over the 64 / LPP groups, the same bits on every lane.
template <int OFF, int GMAX>
__device__ __forceinline__ void attn_merge_level(int G, float (&mr)[GMAX], float (&lr)[GMAX], float (&orr)[GMAX][8]) {
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    if (h >= G) break;
    float ma, mb, la, lb;
    lane_pair<OFF>(mr[h], ma, mb);
    lane_pair<OFF>(lr[h], la, lb);
    const float mx = fmaxf(ma, mb), ea = __expf(ma - mx), eb = __expf(mb - mx);
    lr[h] = fmaf(la, ea, lb * eb);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float oa, ob;
      lane_pair<OFF>(orr[h][e], oa, ob);
      orr[h][e] = fmaf(oa, ea, ob * eb);
    }
    mr[h] = mx;
  }
}
template <int LPP, int GMAX>
__device__ __forceinline__ void attn_lane_merge(int G, float (&mr)[GMAX], float (&lr)[GMAX], float (&orr)[GMAX][8]) {
  if constexpr (LPP <= 8) attn_merge_level<8, GMAX>(G, mr, lr, orr);
  if constexpr (LPP <= 16) attn_merge_level<16, GMAX>(G, mr, lr, orr);
  attn_merge_level<32, GMAX>(G, mr, lr, orr);
}

template <int DH, int GMAX, int ANS, bool PF>
__device__ __forceinline__ void attn_part(const KernelParams& p, uint32_t ep, const TaskDesc& t, float* lds, Ctl* ctl,
                                          uint16_t* const* pools, int s, int grp, int pos, int c0, int c1,
                                          float (&Mo)[AttnShape<DH, GMAX>::EPT], float (&Lo)[AttnShape<DH, GMAX>::EPT],
                                          float (&Ao)[AttnShape<DH, GMAX>::EPT]) {
  using AS = AttnShape<DH, GMAX>;
  constexpr int LPP = AS::LPP, PPW = AS::PPW, EPT = AS::EPT;
  // the thread index made opaque per call: per-lane offsets are then computed here rather than hoisted
  // out of the task loop and held in registers through every other task
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int G = p.hq / p.hk, h0 = grp * G, l = t.layer, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pg = lane / LPP, c = lane % LPP;
  float* qs = lds;  // [G][2][DH/2] scaled queries: dims 8c..8c+3 at 4c, 8c+4..8c+7 at DH/2 + 4c
  uint32_t* kvc = (uint32_t*)(qs + GMAX * DH);  // the current position's key (DH/2 words) then value row
  float* wbuf = (float*)(kvc + DH);          // [NW][G][DH + 2]: each wave's merged (m, l, o)
  const uint32_t what = (uint32_t)t.wait_ev;
  const bool cur = pos >= 0 && c1 == pos + 1;  // the part ends with the current position
  // Chunked prefill (PF, p.prefill): row r of the step is position cs + r of one sequence, so the
  // positions cs .. pos were all written in this step. They come from those rows' tagged key and value
  // words (xn of them, from x0), not from the cache, whose entries this step's rows may still be
  // writing; the cache supplies [c0, ce) below cs.
  int x0 = c1, xn = 0;
  if constexpr (PF) {
    if (p.prefill && pos >= 0) {
      const int cs = __builtin_amdgcn_readfirstlane(ctl->ctx[0]);
      x0 = max(c0, cs);
      xn = max(0, c1 - x0);
    }
  }
  const int ce = min(cur ? pos : c1, x0);    // cached positions [c0, ce)
  const int ngr = ce > c0 ? (ce - c0 + PPW - 1) / PPW : 0;
  const int nw = ngr > wave ? (ngr - wave + NW - 1) / NW : 0;  // this wave's groups: wave + NW k
  // Cache rows: this lane's 8 dims of group k's position (clamped to the last cached position), with
  // nontemporal loads (each row is read once per step). Page entries are clamped into the pool here
  // and checked once per part after the stream.
  const uint16_t* kpool = pools[l];
  const uint16_t* vpool = pools[p.n_layers + l];
  const int32_t* ptab = p.page_table + (size_t)s * p.max_blocks;
  // The page entries of the wave's groups pbase .. pbase + 63 sit one per lane (lane i: group pbase + i),
  // loaded a window at a time; a group's entry is then a lane read, not a memory load inside the stream
  // (a load there would make the in-order wait drain every key and value load in flight).
  int pbase = 0, pent = 0;
  // Every cached block of the part holds the first position of some group, so checking the entries as
  // they are loaded covers the part; a bad entry is reported and clamped into the pool.
  auto load_pages = [&](int base) {
    pbase = base;
    const int k = min(base + lane, max(nw - 1, 0));
    const int raw = nw > 0 ? ptab[(c0 + (wave + NW * k) * PPW) >> 4] : 0;
    if (raw < 0 || raw >= p.num_blocks) raise_error(p, ERR_PAGE, (uint32_t)s, (uint32_t)raw);
    pent = min(max(raw, 0), p.num_blocks - 1);
  };
  load_pages(0);
  auto row_load = [&](const uint16_t* pool, int k) {
    size_t off = (size_t)c * 8;  // no cached rows: a dummy row, block 0
    if (nw > 0) {
      const int kk = min(k, nw - 1);
      const int p0g = c0 + (wave + NW * kk) * PPW;
      const int b = __builtin_amdgcn_readlane(pent, kk - pbase);
      off = (((size_t)b * p.hk + grp) * 16 + (min(p0g + pg, ce - 1) & 15)) * DH + c * 8;
    }
    return __builtin_nontemporal_load((const v4u*)(pool + off));
  };
  v4u RK[ANS], RV[ANS];
#pragma unroll
  for (int j = 0; j < ANS; ++j) {
    RK[j] = row_load(kpool, j);
    RV[j] = row_load(vpool, j);
  }
  // the group's queries (a vector poll) and, when the part ends with the current position, its key
  // and value rows (words KQ and KQ + 1 of the first DH/2 threads), in one poll
  auto q_slot = [&](int i) -> float& {
    const int h = i / DH, d = i % DH, e = d & 7;
    return qs[h * DH + (e < 4 ? 0 : DH / 2) + (d >> 3) * 4 + (e & 3)];
  };
  {
    constexpr int KQ = (GMAX * DH + NW * 64 - 1) / (NW * 64);
    const uint64_t* qsrc = qt_at(p, l, s) + (size_t)h0 * DH;
    const float qscale = 1.0f / sqrtf((float)DH);  // the scores' 1 / sqrt(dh), folded into the queries
    const int nq = G * DH, iq = (tid >> 6) * poll_chunk(nq) + (tid & 63);  // poll_index, from the opaque tid
    const int dk = (int)((const char*)kvt_at(p, l, s, 0, grp) - (const char*)qsrc);  // bytes, > 0
    const int dv = dk + p.hk * (DH / 2) * 8;
    uint32_t pend = first_words(min(poll_chunk(nq) / 64, (nq - iq + 63) / 64));
    if (cur && xn == 0 && tid < DH / 2) pend |= 3u << KQ;
    poll_tagged<KQ + 2>(
        p, ep, qsrc, [&](int k) { return k < KQ ? iq * 8 + k * 512 : tid * 8; },
        [&](int k) { return k < KQ ? 0 : k == KQ ? dk : dv; }, pend, what, [&](int k, uint32_t b) {
          if (k < KQ) q_slot(iq + 64 * k) = __uint_as_float(b) * qscale;
          else kvc[(k - KQ) * (DH / 2) + tid] = b;
        });
    if constexpr (PF) {
      if (xn > 0) {
        // the rows' key and value words, [xn][DH] after the merge buffers: word i of the block is row
        // i / DH, its key (first DH / 2) or value (last DH / 2) pair i % DH
        constexpr int KX = (16 * DH + NT - 1) / NT;
        uint32_t* kvx = (uint32_t*)(wbuf + NW * GMAX * (DH + 2));
        const int rx0 = x0 - __builtin_amdgcn_readfirstlane(ctl->ctx[0]);
        uint32_t px = 0;
#pragma unroll
        for (int j = 0; j < KX; ++j)
          if (tid + NT * j < xn * DH) px |= 1u << j;
        poll_tagged<KX>(
            p, ep, qsrc,
            [&](int j) {
              const int i = tid + NT * j, r = min(i / DH, xn - 1), w = i % DH;
              return (int)((const char*)(kvt_at(p, l, rx0 + r, w < DH / 2 ? 0 : 1, grp) + (w % (DH / 2))) -
                           (const char*)qsrc);
            },
            [](int) { return 0; }, px, what, [&](int j, uint32_t b) { kvx[tid + NT * j] = b; });
      }
    }
  }
  bar();
  if (p.trace && tid == 0) ctl->t_ready = __builtin_amdgcn_s_memrealtime();
  float mr[GMAX], lr[GMAX], orr[GMAX][8];
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    mr[h] = -1e30f;  // finite: a fully masked position then adds exp(-inf) = 0
    lr[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) orr[h][e] = 0.f;
  }
  // this lane's 8 dimensions of each head's scaled query
  float qr[GMAX][8];
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    const v4f qa = *(const v4f*)(qs + min(h, G - 1) * DH + c * 4);
    const v4f qb = *(const v4f*)(qs + min(h, G - 1) * DH + DH / 2 + c * 4);
    qr[h][0] = qa.x; qr[h][1] = qa.y; qr[h][2] = qa.z; qr[h][3] = qa.w;
    qr[h][4] = qb.x; qr[h][5] = qb.y; qr[h][6] = qb.z; qr[h][7] = qb.w;
  }
  // Slot j holds group k0 + j; it is refilled with group k0 + j + ANS once consumed. Slots past the
  // wave's groups weigh 0. The running max moves only when a score passes
  // it by more than 8: until then exp(s - m) stays below e^8, far inside fp32, and the sums need no
  // rescaling (the result is the same ratio).
  for (int k0 = 0; k0 < nw; k0 += ANS) {
    if (k0 + 2 * ANS > pbase + 64) load_pages(k0);  // this round's refills need groups up to k0 + 2 ANS - 1
#pragma unroll
    for (int j = 0; j < ANS; ++j) {
      if (k0 + j >= nw) break;  // wave-uniform: the slots past the wave's groups hold nothing
      const int pp = c0 + (wave + NW * (k0 + j)) * PPW + pg;
      float sc[GMAX];
      attn_scores<DH, GMAX>(RK[j], pp < ce, G, qr, sc);
      bool up = false;
#pragma unroll
      for (int h = 0; h < GMAX; ++h)
        if (h < G) up = up || sc[h] > mr[h] + 8.f;
      if (__builtin_expect(__any(up), 0)) attn_rescale<GMAX>(G, sc, mr, lr, orr);
      attn_accum<GMAX>(RV[j], G, sc, mr, lr, orr);
      if (k0 + j + ANS < nw) {  // no loads past the wave's groups: nothing is left in flight
        RK[j] = row_load(kpool, k0 + j + ANS);
        RV[j] = row_load(vpool, k0 + j + ANS);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if constexpr (PF) {
    // the positions written in this step: the chunk's rows x0 .. x0 + xn - 1 (chunked prefill), or the
    // current position; one per round on wave 0, lane c's 8 dims are words 4c..4c+3 of each row
    const uint32_t* xb = xn > 0 ? (const uint32_t*)(wbuf + NW * GMAX * (DH + 2)) : kvc;
    const int xr = xn > 0 ? xn : (cur ? 1 : 0);
    if (wave == 0) {
      for (int b = 0; b < xr; ++b) {
        const v4u kq = *(const v4u*)(xb + b * DH + 4 * c), vq = *(const v4u*)(xb + b * DH + DH / 2 + 4 * c);
        float sq[GMAX];
        attn_scores<DH, GMAX>(kq, pg == 0, G, qr, sq);
        attn_rescale<GMAX>(G, sq, mr, lr, orr);
        attn_accum<GMAX>(vq, G, sq, mr, lr, orr);
      }
    }
  } else if (cur && wave == 0) {  // the current position: lane c's 8 dims are words 4c..4c+3 of each row
    const v4u kq = *(const v4u*)(kvc + 4 * c), vq = *(const v4u*)(kvc + DH / 2 + 4 * c);
    float sq[GMAX];
    attn_scores<DH, GMAX>(kq, pg == 0, G, qr, sq);
    attn_rescale<GMAX>(G, sq, mr, lr, orr);
    attn_accum<GMAX>(vq, G, sq, mr, lr, orr);
  }
  // merge the wave's lane groups, then the waves
  attn_lane_merge<LPP, GMAX>(G, mr, lr, orr);
  if (pg == 0) {
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      if (h >= G) break;
      float* wb = wbuf + (wave * G + h) * (DH + 2);
      if (c == 0) {
        wb[0] = mr[h];
        wb[1] = lr[h];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) wb[2 + c * 8 + e] = orr[h][e];
    }
  }
  bar();
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int i = min(tid + e * NT, G * DH - 1), h = i / DH, dd = i % DH;
    float M = -1e30f;
    for (int w = 0; w < NW; ++w) M = fmaxf(M, wbuf[(w * G + h) * (DH + 2)]);
    float L = 0.f, A = 0.f;
    for (int w = 0; w < NW; ++w) {
      const float* wb = wbuf + (w * G + h) * (DH + 2);
      const float f = __expf(wb[0] - M);
      L = fmaf(wb[1], f, L);
      A = fmaf(wb[2 + dd], f, A);
    }
    Mo[e] = M;
    Lo[e] = L;
    Ao[e] = A;
  }
}

template <int DH, int GMAX, int ANS, bool COST>
__device__ __forceinline__ void task_attn(const KernelParams& p, uint32_t ep, const TaskDesc& t, float* lds, Ctl* ctl,
                                          uint16_t* const* pools, const int32_t* alo) {
  using AS = AttnShape<DH, GMAX>;
  constexpr int EPT = AS::EPT;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int T = p.attn_tasks, ti = t.a2, W = __builtin_amdgcn_readfirstlane(ctl->aoff[16]);
  const int G = p.hq / p.hk, l = t.layer;
  const uint32_t what = (uint32_t)t.wait_ev;
  const int lo = __builtin_amdgcn_readfirstlane(alo[ti]), hi = __builtin_amdgcn_readfirstlane(alo[ti + 1]);
  // this task's partial slots: [2][G][DH + 2] words (m, l, unnormalised o)
  auto part_base = [&](int task, int slot) { return p.pt + (((size_t)l * T + task) * 2 + slot) * G * (DH + 2); };
  auto seg_start = [&](int x) {  // first block of the segment holding block x
    int s = 0;
    while (s < 15 && ctl->aoff[s + 1] <= x) ++s;
    return __builtin_amdgcn_readfirstlane(ctl->aoff[s] + (x - ctl->aoff[s]) / ctl->anb[s] * ctl->anb[s]);
  };
  auto seg_end = [&](int x) {  // one past the last block of the segment holding block x
    int s = 0;
    while (s < 15 && ctl->aoff[s + 1] <= x) ++s;
    return seg_start(x) + __builtin_amdgcn_readfirstlane(ctl->anb[s]);
  };
  // When the task's last segment goes on past it, that partial is computed and written first: partials
  // never wait on merges, so a merge waits at most for its writers' streaming, never for a chain of
  // other merges. The rest of the range follows in block order, or, with a cut by cost (where a task
  // may hold several whole segments), the segments that lie whole in the range first and last the
  // piece that ends a segment begun by earlier tasks: its merge polls their partials, which by then
  // have had the longest to land.
  const int b_last = hi > lo ? max(lo, seg_start(hi - 1)) : hi;
  int s_last = 0;
  while (hi > lo && s_last < 15 && ctl->aoff[s_last + 1] <= hi - 1) ++s_last;
  const bool last_partial = hi > lo && seg_start(hi - 1) + __builtin_amdgcn_readfirstlane(ctl->anb[s_last]) > hi;
  const int p_end = last_partial ? b_last : hi;  // the partial is [b_last, hi)
  const int lead_end = hi > lo && seg_start(lo) < lo ? min(hi, seg_end(lo)) : lo;  // the merge piece: [lo, lead_end)
  const bool lead = lead_end > lo && p_end > lo;  // (with b_last == lo the whole range is the partial)
  int phase = last_partial ? 0 : lead_end < p_end ? 1 : 2;
  for (int k = 0, x = COST ? (phase == 0 ? b_last : phase == 1 ? lead_end : lo) : (last_partial ? b_last : lo); x < hi; ++k) {
    // the segment holding block x (values read from LDS are made explicitly wave-uniform, so that the
    // page-table reads that depend on them are scalar loads)
    int s = 0;
    while (s < 15 && ctl->aoff[s + 1] <= x) ++s;
    s = __builtin_amdgcn_readfirstlane(s);
    const int nb = __builtin_amdgcn_readfirstlane(ctl->anb[s]), a0 = __builtin_amdgcn_readfirstlane(ctl->aoff[s]);
    const int grp = (x - a0) / nb, B = a0 + grp * nb, E = B + nb;
    const int xe = min(hi, E);
    int pos = __builtin_amdgcn_readfirstlane(ctl->ctx[s]);
    const bool ok = pos >= 0 && pos < p.max_pos;
    if (!ok && tid == 0 && x == B) raise_error(p, ERR_CTX, (uint32_t)s, (uint32_t)pos);
    const int c0 = ok ? 16 * (x - B) : 0, c1 = ok ? min(16 * (xe - B), pos + 1) : 0;
    if (!ok) pos = -1;
    float M[EPT], L[EPT], A[EPT];
    attn_part<DH, GMAX, ANS, COST>(p, ep, t, lds, ctl, pools, s, grp, pos, c0, c1, M, L, A);
    if (p.trace && tid == 0) ctl->t_streamed = __builtin_amdgcn_s_memrealtime();
    if (xe < E) {  // the segment goes on in later tasks: this task's partial
      uint64_t* pb = part_base(ti, x == lo ? 0 : 1);
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int i = tid + e * NT;
        if (i < G * DH) {
          const int h = i / DH, dd = i % DH;
          if (dd == 0) {
            st_tagf(&pb[h * (DH + 2)], M[e], ep);
            st_tagf(&pb[h * (DH + 2) + 1], L[e], ep);
          }
          st_tagf(&pb[h * (DH + 2) + 2 + dd], A[e], ep);
        }
      }
    } else {
      // This task holds the segment's last block: merge the earlier tasks' partials in task order,
      // then its own, R tasks per poll round (3 words per task and element: m, l, o[dim]).
      const int first = COST ? __builtin_amdgcn_readfirstlane(attn_task_of(alo, __builtin_amdgcn_readfirstlane(ctl->ate), B))
                             : attn_task_of(W, __builtin_amdgcn_readfirstlane(ctl->ate), B);
      float Mm[EPT], Lm[EPT], Am[EPT];
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        Mm[e] = -1e30f;
        Lm[e] = 0.f;
        Am[e] = 0.f;
      }
      constexpr int R = 8 / EPT;
      int hb[EPT], ob[EPT];  // byte offsets of the element's head row: m at +0, l at +8, o[dim] at +(2 + dim) 8
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int i = min(tid + e * NT, G * DH - 1);
        hb[e] = (i / DH) * (DH + 2) * 8;
        ob[e] = hb[e] + (2 + i % DH) * 8;
      }
      // the first contributing task holds the segment as its last part (slot 1) when it starts before it
      const int slot_first = __builtin_amdgcn_readfirstlane(alo[first]) < B ? 1 : 0;
      const int task_words = 2 * G * (DH + 2);
      for (int j0 = first; j0 < ti; j0 += R) {
        uint32_t live = 0;  // bit r: task j0 + r contributes (tasks with empty ranges wrote nothing)
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int j = j0 + r;
          if (j < ti && alo[min(j, T - 1)] < alo[min(j, T - 1) + 1]) live |= 1u << r;
        }
        live = __builtin_amdgcn_readfirstlane(live);
        uint32_t pend = 0;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int e = 0; e < EPT; ++e)
            if (((live >> r) & 1u) && tid + e * NT < G * DH) pend |= 7u << ((e * R + r) * 3);
        float mv[EPT][R], lv[EPT][R], ov[EPT][R];
        poll_tagged<3 * R * EPT>(
            p, ep, part_base(0, 0),
            [&](int k) {
              const int e = k / (3 * R), c3 = k % 3;
              return c3 == 2 ? ob[e] : hb[e] + c3 * 8;
            },
            [&](int k) {
              const int j = j0 + (k / 3) % R;
              return ((j - first) * task_words + (first * task_words + (j == first ? slot_first : 0) * G * (DH + 2))) * 8;
            },
            pend, what,
            [&](int k, uint32_t b) {
              const int e = k / (3 * R), r = (k / 3) % R, c3 = k % 3;
              const float f = __uint_as_float(b);
              if (c3 == 0) mv[e][r] = f;
              else if (c3 == 1) lv[e][r] = f;
              else ov[e][r] = f;
            });
#pragma unroll
        for (int e = 0; e < EPT; ++e)
#pragma unroll
          for (int r = 0; r < R; ++r) {
            if (!((live >> r) & 1u) || tid + e * NT >= G * DH) continue;
            const float mn = fmaxf(Mm[e], mv[e][r]);
            const float a = __expf(Mm[e] - mn), b = __expf(mv[e][r] - mn);
            Lm[e] = Lm[e] * a + lv[e][r] * b;
            Am[e] = Am[e] * a + ov[e][r] * b;
            Mm[e] = mn;
          }
      }
      uint64_t* od = ot_at(p, l, s) + (size_t)grp * G * DH;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int i = tid + e * NT;
        if (i >= G * DH) continue;
        const float mn = fmaxf(Mm[e], M[e]);
        const float a = __expf(Mm[e] - mn), b = __expf(M[e] - mn);
        const float Lt = Lm[e] * a + L[e] * b, At = Am[e] * a + A[e] * b;
        st_tagf(&od[i], ok ? At / Lt : 0.f, ep);
      }
    }
    bar();  // the next part reuses the LDS staging
    if constexpr (COST) {
      if (phase == 1 && xe < p_end) {
        x = xe;  // the next whole segment
      } else if (phase == 0 && lead_end < p_end) {
        phase = 1;
        x = lead_end;
      } else if (phase <= 1 && lead) {
        phase = 2;
        x = lo;
      } else {
        break;
      }
    } else {
      // after the leading partial, go back to the start of the range; stop before the partial's blocks
      if (last_partial && k == 0) {
        if (b_last == lo) break;
        x = lo;
      } else {
        x = xe;
        if (last_partial && x >= b_last) break;
      }
    }
  }
}

// ----------------------------------------------------------------------------- argmax keys
// Order-preserving key: larger float -> larger key; on equal values the lower index wins. A NaN of
// either sign takes the top key (above +inf), so the argmax task sees it and reports it.
constexpr uint32_t kNanKey = 0xFFFFFFFFu;
__device__ __forceinline__ uint64_t argmax_key(float v, int idx) {
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  if (v != v) u = kNanKey;
  return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}

__device__ __forceinline__ uint64_t block_max_u64(uint64_t k, Ctl* ctl) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = __shfl_xor(k, off);
    k = o > k ? o : k;
  }
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  bar();
  if (l == 0) ctl->kred[w] = k;
  bar();
  uint64_t m = 0;
  for (int i = 0; i < NW; ++i) m = ctl->kred[i] > m ? ctl->kred[i] : m;
  return m;
}

// ----------------------------------------------------------------------------- GEMV tasks
// Every GEMV task runs one code path: stage the input vector into LDS (polled tagged words, or the
// token's embedding row), RMS-normalise it where the operator starts with a norm, stream the weight
// tile against it, then apply the operator's epilogue:
//   QKV      x (after the previous layer) -> RMSNorm -> rows of q, k, v -> bias, RoPE, KV append
//   O-proj   attention output -> x after O = x + W o
//   gate/up  x after O -> RMSNorm -> interleaved gate/up rows -> SwiGLU
//   down     SwiGLU output -> x after down = x + W h
//   LM head  final x -> RMSNorm -> logits and the tile's argmax key
// One shared path keeps the instruction footprint small. The kernel's code is larger than the
// instruction cache, and code that a CU runs once per layer is otherwise fetched anew each time.
// ep: the step's epoch; step: the step's index within this launch. nxt: the CU's next task in this
// launch, or null. staged: on entry, whether this wave's stage (bit 0) and second stage (bit 1) already
// hold this task's units (staged by the previous task); on return, whether they hold the next task's.
template <bool FP8>
__device__ __forceinline__ void gemv_task(const KernelParams& p, uint32_t ep, int step, const TaskDesc& t, float* lds,
                                          Ctl* ctl, WPipe& wp, uint16_t* const* pools, const TaskDesc* nxt,
                                          int& staged) {
  const int type = t.type, l = t.layer, s = 0;
  // the thread index made opaque per task: per-thread offsets are computed here rather than hoisted
  // out of the task loop and held in registers through every other task
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const uint32_t what = (uint32_t)t.wait_ev;
  const GemvGeom gm = ctl->geoms[t.geom];
  const int padded = gm.S * gm.lpr * 8, np = padded >> 3;
  float* xs = lds;
  float* ys = lds + padded;
  const bool norm = type == T_QKV || type == T_GATEUP || type == T_LMHEAD;
  const bool resid = type == T_OPROJ || type == T_DOWN;
  const int n = type == T_OPROJ ? p.hq * p.dh : type == T_DOWN ? p.f : p.d;
  const uint64_t* src = type == T_QKV      ? xt_at(p, l > 0 ? l - 1 : 0, 1, s)
                        : type == T_GATEUP ? xt_at(p, l, 0, s)
                        : type == T_LMHEAD ? xt_at(p, p.n_layers - 1, 1, s)
                        : type == T_OPROJ  ? ot_at(p, l, s)
                                           : ht_at(p, l, s);
  const bool in_embed = type == T_QKV && l == 0;     // the first QKV reads the embedding row
  const bool res_embed = type == T_OPROJ && l == 0;  // the first O-proj adds to it
  // After a launch's first step the token is the tagged word the previous step's argmax published; its
  // first load goes out with the input poll, ahead of the weights.
  const bool tok_tagged = (in_embed || res_embed) && step > 0;

  // Everything the task loads before its GEMV is issued ahead of the weight stream: the wait counter
  // of vector memory completes in order, so a load issued after the stream's first NSLOT units per
  // wave could not be used before they had all arrived. In order: the first pass of the input poll,
  // the RMSNorm gains, the residual words; then the weight units; then the QKV epilogue constants,
  // which are needed only after the GEMV.
  // Input words: thread t polls words i0 + 64k (see poll_vector), landing at xs_index(i0) + 32k.
  // The LDS stage's DMA goes out first, ahead of every other load of the task (see stage_units).
  // An O-projection task runs while HBM is nearly idle (its weights arrived during attention) and is
  // followed on its CU by a gate/up task: it fills the stage with that task's units, at once when
  // its own units fit the registers, else as soon as it has read its own staged units. When its own
  // units also leave the second stage unused, it fills that one too, at once, while attention runs.
  WaveRun wrun = wave_run<FP8>(p, t, gm);
  if (wrun.nunits <= 0) wrun = dummy_run(p);
  if (!(staged & 1)) stage_units(wrun);
  const bool second_stage = p.stage2_off > 0 && gm.lpr == 64 && gm.S == 8;
  const bool own_stage2 = second_stage && !(staged & 2);  // this task issues its second stage's DMA
  const bool restage_next = type == T_OPROJ && nxt != nullptr && is_gemv(nxt->type);
  WaveRun wnext = wrun;
  int staged_next = 0;
  if (restage_next) {
    const GemvGeom& gn = ctl->geoms[nxt->geom];
    wnext = wave_run<FP8>(p, *nxt, gn);
    if (wnext.nunits <= 0) wnext = dummy_run(p);
    if (wrun.nunits <= NSLOT) stage_units(wnext);
    staged_next = 1;
    if (p.stage2_off > 0 && gn.lpr == 64 && gn.S == 8 && (!second_stage || wrun.nunits <= NSLOT + kStageUnits)) {
      stage2_units(wnext, xs, p.stage2_off);
      staged_next |= 2;
    }
  }
  staged = staged_next;
  const __amdgpu_buffer_rsrc_t rin = tag_rsrc(src);
  const int i0 = poll_index(n, 0);
  uint32_t pending = in_embed ? 0u : first_words(min(poll_chunk(n) / 64, (n - i0 + 63) / 64));
  uint64_t w1[32];
#pragma unroll
  for (int k = 0; k < 32; ++k)
    if ((pending >> k) & 1u) w1[k] = ld_tag(rin, i0 * 8 + (k & 7) * 512, (k >> 3) * 4096);
  uint64_t tw[1] = {0};
  if (tok_tagged) tw[0] = ld_tag(tag_rsrc(p.tokt), s * 8, 0);
  // Gains: thread t scales elements [8t, 8t + 8) and [4096 + 8t, 4096 + 8t + 8) (n <= 8192).
  const uint16_t* gain = type == T_QKV      ? layer_norm_gain(p, l, 0)
                         : type == T_GATEUP ? layer_norm_gain(p, l, 1)
                                            : p.norms + (size_t)p.n_layers * 2 * p.d;
  v4u gq[2];
  if (norm) {
#pragma unroll
    for (int c = 0; c < 2; ++c) gq[c] = *(const v4u*)(gain + min(8 * tid + 4096 * c, n - 8));
  }
  // O-proj and down: the residual words, clamped to the task's last row. They were written a stage
  // before the input vector, so they are nearly always current once it is; a stale one is polled
  // again below.
  const uint64_t* rsrc = type == T_OPROJ ? xt_at(p, l > 0 ? l - 1 : 0, 1, s) : xt_at(p, l, 0, s);
  const int nrows = t.row1 - t.row0;
  uint64_t rw[4] = {0, 0, 0, 0};
  if (resid && !res_embed) {
    const __amdgpu_buffer_rsrc_t rr = tag_rsrc(rsrc + t.row0);
#pragma unroll
    for (int k = 0; k < 4; ++k) rw[k] = ld_tag(rr, min(tid + k * NT, nrows - 1) * 8, 0);
  }
  // FP8 weights: the scales 2^e of the task's rows (thread t: rows t and t + 512)
  float scv[2] = {1.f, 1.f};
  if constexpr (FP8) {
#pragma unroll
    for (int k = 0; k < 2; ++k)
      if (tid + k * NT < nrows) scv[k] = p.wscale[t.a1 + tid + k * NT];
  }
  // the wave's first NSLOT / 2 weight units (the rest go out after the input's second poll pass)
#pragma unroll
  for (int j = 0; j < NSLOT / 2; ++j) wp.R[j] = load_unit(wrun, j);
  // QKV: the rotary, bias and page-table constants of the thread's 4-row set. An out-of-range
  // position is reported and the row is not appended, but q, k and v are still written (at
  // position 0's rotation) so that no consumer waits for them.
  const int nsets = nrows >> 2;
  int pos = 0;
  QkvSet pre;
  if (type == T_QKV) {
    pos = checked_pos(p, ctl, s);
    if (tid < nsets) pre = qkv_set_consts(p, l, t.row0 + 4 * tid, pos < 0 ? 0 : pos, s);
  }
  const uint16_t* erow = nullptr;
  if (in_embed || res_embed) {
    int tok;
    if (tok_tagged) {
      uint32_t b = 0;
      poll_finish<1>(p, ep, tw, 1u, kWhatToken, [&](int) { return ld_tag(tag_rsrc(p.tokt), s * 8, 0); },
                     [&](int, uint32_t v) { b = v; });
      tok = (int)min(b, (uint32_t)(p.vocab - 1));
    } else {
      tok = token_of(p, s);
    }
    erow = p.embed + (size_t)tok * p.d;
  }

  // the input vector, two-plane layout in LDS, zero past n
  float* xd = xs + xs_index(i0, np);
  if (in_embed) {
#pragma unroll
    for (int j = NSLOT / 2; j < NSLOT; ++j) wp.R[j] = load_unit(wrun, j);
    if (own_stage2) stage2_units(wrun, xs, p.stage2_off);
    // one 16-byte piece (8 values) per thread and load, into both planes (n is a multiple of 8 and the
    // row starts 16-byte aligned)
    for (int pc = tid; 8 * pc < n; pc += NT) {
      const v4u e = *(const v4u*)(erow + 8 * pc);
      const v4f a = {bf_lo(e.x), bf_hi(e.x), bf_lo(e.y), bf_hi(e.y)};
      const v4f b = {bf_lo(e.z), bf_hi(e.z), bf_lo(e.w), bf_hi(e.w)};
      *(v4f*)(xs + 4 * pc) = a;
      *(v4f*)(xs + 4 * np + 4 * pc) = b;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      if (((pending >> k) & 1u) && (uint32_t)(w1[k] >> 32) == ep) {
        xd[32 * k] = __uint_as_float((uint32_t)w1[k]);
        pending &= ~(1u << k);
      }
    }
    if (__any(pending != 0u)) {
      // the second pass goes out ahead of the second half of the prefetch, so it waits only behind the first
#pragma unroll
      for (int k = 0; k < 32; ++k)
        if ((pending >> k) & 1u) w1[k] = ld_tag(rin, i0 * 8 + (k & 7) * 512, (k >> 3) * 4096);
#pragma unroll
      for (int j = NSLOT / 2; j < NSLOT; ++j) wp.R[j] = load_unit(wrun, j);
      if (own_stage2) stage2_units(wrun, xs, p.stage2_off);
      poll_finish<32>(p, ep, w1, pending, what, [&](int k) { return ld_tag(rin, i0 * 8 + (k & 7) * 512, (k >> 3) * 4096); },
                      [&](int k, uint32_t b) { xd[32 * k] = __uint_as_float(b); });
    } else {
#pragma unroll
      for (int j = NSLOT / 2; j < NSLOT; ++j) wp.R[j] = load_unit(wrun, j);
      if (own_stage2) stage2_units(wrun, xs, p.stage2_off);
    }
  }
  for (int i = n + tid; i < padded; i += NT) xs[xs_index(i, np)] = 0.f;
  float* ysc = ys + ((nrows + 63) & ~63);
  if constexpr (FP8) {
#pragma unroll
    for (int k = 0; k < 2; ++k)
      if (tid + k * NT < nrows) ysc[tid + k * NT] = scv[k];
  }
  bar();
  if (norm) {  // the sum of squares runs over the staged values in a fixed order
    float ss = 0.f;
    for (int i = tid; i < n; i += NT) {
      const float v = xs[xs_index(i, np)];
      ss += v * v;
    }
    ss = block_sum(ss, ctl);
    const float r = 1.0f / sqrtf(ss / (float)n + p.eps);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int pc = tid + 512 * c;  // piece: elements 8 pc .. 8 pc + 7
      if (8 * pc < n) {
        v4f* pa = (v4f*)(xs + 4 * pc);
        v4f* pb = (v4f*)(xs + 4 * np + 4 * pc);
        v4f a = *pa, b = *pb;
        const v4u g = gq[c];
        a.x = a.x * r * bf_lo(g.x); a.y = a.y * r * bf_hi(g.x); a.z = a.z * r * bf_lo(g.y); a.w = a.w * r * bf_hi(g.y);
        b.x = b.x * r * bf_lo(g.z); b.y = b.y * r * bf_hi(g.z); b.z = b.z * r * bf_lo(g.w); b.w = b.w * r * bf_hi(g.w);
        *pa = a;
        *pb = b;
      }
    }
    bar();
  }
  float res[4] = {0.f, 0.f, 0.f, 0.f};
  if (resid) {
    uint32_t stale = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = tid + k * NT;
      if (r < nrows) {
        if (res_embed) res[k] = bf2f(erow[t.row0 + r]);
        else if ((uint32_t)(rw[k] >> 32) == ep) res[k] = __uint_as_float((uint32_t)rw[k]);
        else stale |= 1u << k;
      }
    }
    if (__any(stale != 0u))
      poll_tagged<4>(p, ep, rsrc + t.row0, [&](int k) { return (tid + k * NT) * 8; }, [](int) { return 0; }, stale, what,
                     [&](int k, uint32_t b) { res[k] = __uint_as_float(b); });
  }
  if (p.trace && tid == 0) ctl->t_ready = __builtin_amdgcn_s_memrealtime();

  gemv_tile<FP8>(p, t, gm, xs, ys, wp, restage_next && wrun.nunits > NSLOT, wnext, ysc);
  bar();
  if (p.trace && tid == 0) ctl->t_streamed = __builtin_amdgcn_s_memrealtime();

  if (type == T_QKV) {
    for (int m = tid; m < nsets; m += NT) {
      const int r = t.row0 + 4 * m;
      const QkvSet c = (m == tid) ? pre : qkv_set_consts(p, l, r, pos < 0 ? 0 : pos, s);
      qkv_store_set(p, l, s, r, ys[4 * m], ys[4 * m + 1], ys[4 * m + 2], ys[4 * m + 3], c, pos, pools, ep);
    }
  } else if (resid) {
    uint64_t* dst = xt_at(p, l, type == T_OPROJ ? 0 : 1, s);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = t.row0 + tid + k * NT;
      if (r < t.row1) st_tagf(&dst[r], res[k] + ys[r - t.row0], ep);
    }
  } else if (type == T_GATEUP) {
    const int npairs = nrows >> 1;
    uint64_t* hd = ht_at(p, l, s) + (t.row0 >> 1);
    for (int m = tid; m < npairs; m += NT) {
      const float a = ys[2 * m], b = ys[2 * m + 1];
      const float silu = a / (1.0f + expf(-a));
      st_tagf(&hd[m], silu * b, ep);
    }
  } else {  // LM head
    uint64_t best = 0;
    for (int r = t.row0 + tid; r < t.row1; r += NT) {
      const float v = ys[r - t.row0];
      p.logits[(size_t)s * p.vocab + r] = v;
      const uint64_t k = argmax_key(v, r);
      best = k > best ? k : best;
    }
    best = block_max_u64(best, ctl);
    if (tid == 0) stc(&p.amax[(size_t)s * p.n_lm_parts + t.a0], best);
  }
}

// ----------------------------------------------------------------------------- batched GEMM tiles
// With several sequences each GEMV becomes a skinny GEMM, Y[rows][seqs] = W[rows][K] X[seqs][K]^T,
// 16 sequences wide, and runs on v_mfma_f32_16x16x32_bf16. A packed weight unit is the 16x32 row
// operand as it comes from memory; the inputs form the 32x16 column operand. Each fp32 input is split
// into a bf16 high part and a bf16 remainder and every unit takes two MFMAs, so the products carry
// about 16 significant bits of each input and accumulate in fp32.
//
// A task covers a tile of rows and a range of 32-column units. Its input columns are staged in LDS as
// MFMA fragments (unit u, lane l: 8 columns of sequence l % 16, high parts then remainders), one block
// of at most 32 units at a time (16 when a task streams several blocks). Each wave streams an even
// share of the block's (row group, unit) items; a 16x16 accumulator runs along a row group's units and
// goes to LDS at the group's end. Groups that straddle two waves are summed in wave order afterwards,
// so the result does not depend on timing. When a tile's columns are split over kS tasks, each writes
// its partial sums as tagged words; each then sums the kS partials (in split order) of its share of
// the tile's row quads and applies the epilogue to that share. RMSNorm enters as a per-sequence scale
// of the sums, W (g * x) / rms(x), with the sums of squares exchanged along with the partials.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v4f mfma_bf16(const v4u a, const v4u b, const v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Token and position of sequence s; any thread may report a bad one (the first report is kept). After a
// launch's first step the token is the tagged word the previous step's argmax published.
__device__ __forceinline__ int token_any(const KernelParams& p, uint32_t ep, int step, int s) {
  if (step > 0) {
    uint32_t b = 0;
    poll_tagged<1>(p, ep, p.tokt, [&](int) { return s * 8; }, [](int) { return 0; }, 1u, kWhatToken,
                   [&](int, uint32_t v) { b = v; });
    return (int)min(b, (uint32_t)(p.vocab - 1));
  }
  int tok = p.tokens_in[s];
  if (tok < 0 || tok >= p.vocab) {
    raise_error(p, ERR_TOKEN, (uint32_t)s, (uint32_t)tok);
    tok = 0;
  }
  return tok;
}
__device__ __forceinline__ int pos_any(const KernelParams& p, const Ctl* ctl, int s) {
  const int pos = ctl->ctx[s];
  if (pos < 0 || pos >= p.max_pos) {
    raise_error(p, ERR_CTX, (uint32_t)s, (uint32_t)pos);
    return -1;
  }
  return pos;
}

__device__ __forceinline__ void gemv_task_b(const KernelParams& p, uint32_t ep, int step, const TaskDesc& t, float* lds,
                                            Ctl* ctl, uint16_t* const* pools) {
  WPipe wp;  // task-local: no weight loads are carried into the next task
  // The thread index made opaque per task: per-lane offsets are computed here rather than hoisted out of
  // the task loop and held in registers through every other task.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int type = t.type, l = t.layer, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t what = (uint32_t)t.wait_ev;
  const int nact = min(p.n_active, p.max_seqs);
  const int rows = t.row1 - t.row0, R = (rows + 15) >> 4, Q = (rows + 3) >> 2;
  const int kb0 = t.a2 & 0xFFFF, nu = t.a2 >> 16, js = t.a3 & 0xFF, kS = t.a3 >> 8;
  const bool multi = nu > 32;  // one column split streaming several 16-unit blocks
  const int ub = multi ? 16 : nu, nb = multi ? nu >> 4 : 1;
  const bool norm = type == T_QKV || type == T_GATEUP || type == T_LMHEAD;
  const bool resid = type == T_OPROJ || type == T_DOWN;
  const int K = type == T_OPROJ ? p.hq * p.dh : type == T_DOWN ? p.f : p.d;
  // sequence s's input vector is src + s * K (one buffer per layer)
  const uint64_t* src = type == T_QKV      ? xt_at(p, l > 0 ? l - 1 : 0, 1, 0)
                        : type == T_GATEUP ? xt_at(p, l, 0, 0)
                        : type == T_LMHEAD ? xt_at(p, p.n_layers - 1, 1, 0)
                        : type == T_OPROJ  ? ot_at(p, l, 0)
                                           : ht_at(p, l, 0);
  const bool in_embed = type == T_QKV && l == 0;
  const uint16_t* gain = type == T_QKV      ? layer_norm_gain(p, l, 0)
                         : type == T_GATEUP ? layer_norm_gain(p, l, 1)
                                            : p.norms + (size_t)p.n_layers * 2 * p.d;

  uint32_t* afrag = (uint32_t*)lds;  // [unit][64 lanes][4 dwords high | 4 dwords low]: 2 KB per unit, 64 KB
  float* T = lds + 16384;            // [R][64 lanes][4]: the tile's sums, one 16x16 MFMA tile per row group
  float* E = T + R * 256;            // [NW][2][64][4]: each wave's partial first and last row groups
  float* ssl = E + NW * 2 * 256;     // [16] sums of squares of this task's columns, per sequence
  float* rsq = ssl + 16;             // [16] per-sequence scale of the sums (1 / rms, or 1)
  unsigned long long* kseq = (unsigned long long*)(rsq + 16);  // [16] LM head: best argmax key per sequence
  if (tid < 16) kseq[tid] = 0ull;

  // Input staging. Thread (wave w, lane) holds sequences 2w and 2w + 1, columns 64 c + lane of the
  // block (c < 16): each load is a coalesced 512-byte row of one sequence's tagged words. The loads are
  // unconditional, so all of them issue together; only the words of active sequences inside K are
  // polled. The buffer range check covers the lane offset, not the uniform one, so a sequence past the
  // configured ones reads the last configured sequence's row instead, and columns past the task's
  // (or past K) read at most one 1024-column block past a row: for tagged words inside the scratch
  // buffer, for gains and embedding rows inside the weights buffer (whose layout ends with a pad of
  // that size). Such values are never used: with K a multiple of 32, every column a task stages lies
  // inside K.
  const int ln = lane;
  const int s0 = 2 * wave;
  float ss[2] = {0.f, 0.f};
  uint64_t xw[32];  // the words in flight; once current, their low halves are the inputs
  uint32_t gq[16];
  uint32_t xpend = 0, xvalid = 0;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, p.max_seqs * K * 8, 0x00020000);
  const __amdgpu_buffer_rsrc_t rgain = __builtin_amdgcn_make_buffer_rsrc((void*)gain, (short)0, K * 2, 0x00020000);
  auto x_word = [&](int b, int kw) {
    const int c0 = 32 * (kb0 + b * ub), c = kw & 15, sq = min(s0 + (kw >> 4), p.max_seqs - 1);
    return ld_tag(rx, ln * 8 + (c & 7) * 512, (sq * K + c0) * 8 + (c >> 3) * 4096);
  };
  auto x_issue = [&](int b) {
    const int c0 = 32 * (kb0 + b * ub), ncol = 32 * min(ub, nu - b * ub);
    xvalid = 0;
#pragma unroll
    for (int kw = 0; kw < 32; ++kw) {
      const int h = kw >> 4, c = kw & 15;
      if (s0 + h < nact && 64 * c + ln < ncol && c0 + 64 * c + ln < K) xvalid |= 1u << kw;
    }
    if (in_embed) {  // the first layer's input: the tokens' embedding rows, as current words
      xpend = 0;
      for (int h = 0; h < 2; ++h) {
        const int tk = s0 + h < nact ? token_any(p, ep, step, s0 + h) : 0;
        const __amdgpu_buffer_rsrc_t re =
            __builtin_amdgcn_make_buffer_rsrc((void*)(p.embed + (size_t)tk * p.d), (short)0, p.d * 2, 0x00020000);
#pragma unroll
        for (int c = 0; c < 16; ++c)
          xw[16 * h + c] = (uint64_t)__builtin_amdgcn_raw_buffer_load_b16(re, ln * 2, (c0 + 64 * c) * 2, 0) << 16;
      }
    } else {
      xpend = xvalid;
#pragma unroll
      for (int kw = 0; kw < 32; ++kw) xw[kw] = x_word(b, kw);
    }
    if (norm) {
#pragma unroll
      for (int c = 0; c < 16; ++c) gq[c] = __builtin_amdgcn_raw_buffer_load_b16(rgain, ln * 2, (c0 + 64 * c) * 2, 0);
    }
  };
  auto x_finish = [&](int b) {
    const int ncol = 32 * min(ub, nu - b * ub);
    poll_finish<32>(p, ep, xw, xpend, what, [&](int kw) { return x_word(b, kw); }, [](int, uint32_t) {});
    // Fragments: sequence s, column col -> unit col / 32, lane s + 16 ((col % 32) / 8), element col % 8.
    // Lane pairs swap halves so each lane stores one dword: the even lane two high parts, the odd lane
    // two remainders. With col = 64 c + lane, word kw lands at dword 1024 c + 8 h past the lane's base.
    uint32_t* al = afrag + (multi ? (b & 1) * 8192 : 0) +
                   ((ln >> 5) * 64 + s0 + 16 * ((ln & 31) >> 3)) * 8 + (ln & 1) * 4 + ((ln & 7) >> 1);
#pragma unroll
    for (int kw = 0; kw < 32; ++kw) {
      const int h = kw >> 4, c = kw & 15;
      const float x = ((xvalid >> kw) & 1u) ? __uint_as_float((uint32_t)xw[kw]) : 0.f;
      ss[h] = fmaf(x, x, ss[h]);
      const float v = norm ? x * bf2f((uint16_t)gq[c]) : x;
      const uint32_t hi = f2bf(v), lo = f2bf(v - bf2f((uint16_t)hi));
      const uint32_t other = (uint32_t)__shfl_xor((int)((ln & 1) ? hi : lo), 1);
      const uint32_t word = (ln & 1) ? (other | (lo << 16)) : (hi | (other << 16));
      if (64 * c + ln < ncol) al[1024 * c + 8 * h] = word;
    }
  };

  // This wave's items of each block: (row group, unit) pairs [ia, ib) in that order. Several blocks:
  // whole row groups per wave, so that a round of NSLOT units is one group's block.
  int ia, ib;
  if (multi) {
    ia = 16 * (R * wave / NW);
    ib = 16 * (R * (wave + 1) / NW);
  } else {
    ia = R * nu * wave / NW;
    ib = R * nu * (wave + 1) / NW;
  }
  const int cnt = ib - ia, rpb = (cnt + NSLOT - 1) / NSLOT, nrounds = nb * rpb;
  const v4u* wbase = (const v4u*)(p.wpacked + t.wofs) + lane;
  auto round_base = [&](int r) -> int {  // packed unit of slot 0 of round r
    if (!multi) return ia + NSLOT * r;
    const int b = r / rpb, rr = r - b * rpb;
    return (ia / 16 + rr) * nu + 16 * b;
  };
  const int last_unit = max(0, multi ? (ib / 16) * nu - 1 : ib - 1);
  auto load_w = [&](int a) { return __builtin_nontemporal_load(wbase + (size_t)min(a, last_unit) * 64); };

  x_issue(0);
  {  // the wave's first NSLOT weight units stream while the inputs arrive
    const int a0 = cnt > 0 ? round_base(0) : 0;
#pragma unroll
    for (int j = 0; j < NSLOT; ++j) wp.R[j] = load_w(a0 + j);
  }
  x_finish(0);
  bar();
  if (p.trace && tid == 0) ctl->t_ready = __builtin_amdgcn_s_memrealtime();

  auto flush = [&](int g, int b, v4f v) {
    v4f* dst;
    if (multi) {
      dst = (v4f*)T + g * 64 + lane;
      if (b > 0) v += *dst;
    } else {
      const bool whole = g * ub >= ia && (g + 1) * ub <= ib;
      dst = whole ? (v4f*)T + g * 64 + lane : (v4f*)E + (wave * 2 + (g == ia / ub ? 0 : 1)) * 64 + lane;
    }
    *dst = v;
  };
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < nb; ++b) {
    if (b > 0) {
      x_issue(b);
      x_finish(b);
      bar();
    }
    const uint32_t* ab = afrag + (multi ? (b & 1) * 8192 : 0);
    int g = ia / ub, u = ia % ub;
    v4f cur = zero;
    auto item = [&](int rr, int j) {
      if (NSLOT * rr + j < cnt) {
        const v4u* a = (const v4u*)(ab + (u * 64 + lane) * 8);
        const v4u ahi = a[0], alo = a[1];
        cur = mfma_bf16(wp.R[j], ahi, cur);
        cur = mfma_bf16(wp.R[j], alo, cur);
        if (++u == ub) {
          flush(g, b, cur);
          cur = zero;
          u = 0;
          ++g;
        }
      }
    };
    for (int rr = 0; rr < rpb; ++rr) {
      const int r = b * rpb + rr;
      if (r + 1 < nrounds) {
        const int nbase = round_base(r + 1);
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) {
          item(rr, j);
          wp.R[j] = load_w(nbase + j);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        // the stream's last round: no refills (they would sit in the in-order queue ahead of the
        // exchange's polls)
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) item(rr, j);
      }
    }
    if (u != 0 && cnt > 0) flush(g, b, cur);  // the wave's items end inside a row group
  }
  {
    const float sa = wave_sum(ss[0]), sb = wave_sum(ss[1]);
    if (lane == 0) {
      ssl[s0] = sa;
      ssl[s0 + 1] = sb;
    }
  }
  bar();
  if (p.trace && tid == 0) ctl->t_streamed = __builtin_amdgcn_s_memrealtime();
  if (!multi) {  // row groups shared by two waves: their partials, in wave order
    const int per = R * nu;
    for (int e = tid; e < R * 256; e += NT) {
      const int g = e >> 8;
      float acc = 0.f;
      bool edge = false;
      for (int w = 0; w < NW; ++w) {
        const int a = per * w / NW, z = per * (w + 1) / NW;
        if (a == z || a >= (g + 1) * nu || z <= g * nu) continue;
        if (a <= g * nu && z >= (g + 1) * nu) break;  // one wave holds the whole group
        acc += E[(w * 2 + (g == a / nu ? 0 : 1)) * 256 + (e & 255)];
        edge = true;
      }
      if (edge) T[e] = acc;
    }
    bar();
  }

  // This task's share of the tile: row quads [qa, qb) (all of them without a column split). The sums
  // of quad q for sequence s sit at word ((q / 4) * 64 + s + 16 (q % 4)) * 4 of a tile: rows 4q .. 4q+3.
  const int qa = Q * js / kS, qb = Q * (js + 1) / kS;
  const int npairs = (qb - qa) * nact;
  if (kS > 1) {
    uint64_t* bp = p.bpt + t.a1;
    const int SW = R * 256 + 64;  // words of one split's block: the tile, then the sums of squares
    for (int e = tid; e < R * 256; e += NT) {
      const int le = (e >> 2) & 63, q = 4 * (e >> 8) + (le >> 4);  // lane and quad of word e
      if ((le & 15) < nact && (q < qa || q >= qb)) st_tagf(&bp[(size_t)js * SW + e], T[e], ep);
    }
    if (norm && tid < nact) st_tagf(&bp[(size_t)js * SW + R * 256 + tid], ssl[tid], ep);
    // tpp threads per (quad, sequence) pair, each summing the splits congruent to it, in order
    int tpp = 1;
    while (2 * tpp <= kS && npairs * 2 * tpp <= NT) tpp *= 2;
    const int sub = tid % tpp;
    float* scr = (float*)afrag;  // the fragments are no longer needed
    for (int pb = 0; pb < npairs; pb += NT / tpp) {
      const int pair = pb + tid / tpp;
      const bool act = pair < npairs;
      const int q = qa + (act ? pair / nact : 0), s = act ? pair % nact : 0;
      const int eo = ((q >> 2) * 64 + s + 16 * (q & 3)) * 4;
      float y0 = 0.f, y1 = 0.f, y2 = 0.f, y3 = 0.f, sq = 0.f;
      for (int jb = sub; jb < kS; jb += 6 * tpp) {  // up to 6 splits per poll round
        uint32_t pend = 0;
#pragma unroll
        for (int i = 0; i < 6; ++i) {
          const int jj = jb + i * tpp;
          if (act && jj < kS && jj != js) pend |= (norm ? 0x1Fu : 0xFu) << (5 * i);
        }
        float v[30];
        poll_tagged<30>(
            p, ep, bp,
            [&](int k) {
              const int i = k / 5, c = k % 5;
              return ((jb + i * tpp) * SW + (c < 4 ? eo + c : R * 256 + s)) * 8;
            },
            [](int) { return 0; }, pend, what, [&](int k, uint32_t bits) { v[k] = __uint_as_float(bits); });
#pragma unroll
        for (int i = 0; i < 6; ++i) {
          const int jj = jb + i * tpp;
          if (!act || jj >= kS) continue;
          if (jj == js) {
            y0 += T[eo];
            y1 += T[eo + 1];
            y2 += T[eo + 2];
            y3 += T[eo + 3];
            sq += ssl[s];
          } else {
            y0 += v[5 * i];
            y1 += v[5 * i + 1];
            y2 += v[5 * i + 2];
            y3 += v[5 * i + 3];
            if (norm) sq += v[5 * i + 4];
          }
        }
      }
      scr[tid * 5 + 0] = y0;
      scr[tid * 5 + 1] = y1;
      scr[tid * 5 + 2] = y2;
      scr[tid * 5 + 3] = y3;
      scr[tid * 5 + 4] = sq;
      bar();
      if (act && sub == 0) {
        float z[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < tpp; ++k)
#pragma unroll
          for (int c = 0; c < 5; ++c) z[c] += scr[(tid + k) * 5 + c];
        T[eo] = z[0];
        T[eo + 1] = z[1];
        T[eo + 2] = z[2];
        T[eo + 3] = z[3];
        if (q == qa) rsq[s] = norm ? 1.0f / sqrtf(z[4] / (float)K + p.eps) : 1.f;
      }
      bar();
    }
  } else {
    if (tid < 16) rsq[tid] = norm ? 1.0f / sqrtf(ssl[tid] / (float)K + p.eps) : 1.f;
    bar();
  }

  // the epilogue of each (quad, sequence) of the share
  for (int pr = tid; pr < npairs; pr += NT) {
    const int q = qa + pr / nact, s = pr % nact;
    const int eo = ((q >> 2) * 64 + s + 16 * (q & 3)) * 4;
    const float sc = rsq[s];
    const float y[4] = {T[eo] * sc, T[eo + 1] * sc, T[eo + 2] * sc, T[eo + 3] * sc};
    const int r0 = t.row0 + 4 * q, nr = min(4, t.row1 - r0);
    if (type == T_QKV) {
      const int pos = pos_any(p, ctl, s);
      const QkvSet c = qkv_set_consts(p, l, r0, pos < 0 ? 0 : pos, s);
      qkv_store_set(p, l, s, r0, y[0], y[1], y[2], y[3], c, pos, pools, ep);
    } else if (resid) {
      float xo[4] = {0.f, 0.f, 0.f, 0.f};
      if (type == T_OPROJ && l == 0) {
        const uint16_t* er = p.embed + (size_t)token_any(p, ep, step, s) * p.d;
        for (int r = 0; r < nr; ++r) xo[r] = bf2f(er[r0 + r]);
      } else {
        const uint64_t* rb = type == T_OPROJ ? xt_at(p, l - 1, 1, 0) : xt_at(p, l, 0, 0);
        poll_tagged<4>(p, ep, rb, [&](int k) { return (s * p.d + r0 + k) * 8; }, [](int) { return 0; }, first_words(nr), what,
                       [&](int k, uint32_t bits) { xo[k] = __uint_as_float(bits); });
      }
      uint64_t* dst = xt_at(p, l, type == T_OPROJ ? 0 : 1, s) + r0;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (r < nr) st_tagf(&dst[r], xo[r] + y[r], ep);
    } else if (type == T_GATEUP) {
      uint64_t* hd = ht_at(p, l, s) + (r0 >> 1);
      st_tagf(&hd[0], y[0] / (1.0f + expf(-y[0])) * y[1], ep);
      if (nr > 2) st_tagf(&hd[1], y[2] / (1.0f + expf(-y[2])) * y[3], ep);
    } else {  // LM head
      unsigned long long best = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (r < nr) {
          p.logits[(size_t)s * p.vocab + r0 + r] = y[r];
          const unsigned long long k = argmax_key(y[r], r0 + r);
          best = k > best ? k : best;
        }
      atomicMax(&kseq[s], best);
    }
  }
  if (type == T_LMHEAD) {
    bar();
    if (tid < nact) stc(&p.amax[(size_t)tid * p.n_lm_parts + t.a0], (uint64_t)kseq[tid]);
  }
}

// The step's token of sequence s: the largest of the LM tiles' keys. It goes to the caller's output
// row of this step and, tagged with the next step's epoch, to the next step's embedding lookups; the
// sequence's context length becomes this step's position + 1.
__device__ __forceinline__ void task_argmax(const KernelParams& p, uint32_t ep, int step, const TaskDesc& t, Ctl* ctl) {
  const int s = t.a0;
  uint64_t best = 0;
  for (int i = threadIdx.x; i < p.n_lm_parts; i += NT) {
    const uint64_t k = ldc(&p.amax[(size_t)s * p.n_lm_parts + i]);
    best = k > best ? k : best;
  }
  best = block_max_u64(best, ctl);
  if (threadIdx.x == 0 && s < p.n_active) {
    const int32_t tok = (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
    if ((uint32_t)(best >> 32) == kNanKey) raise_error(p, ERR_NAN, (uint32_t)s, (uint32_t)tok);
    p.tokens_out[(size_t)step * p.n_active + s] = tok;
    p.ctx_lens[s] = ctl->ctx[s] + 1;
    st_tag(&p.tokt[s], (uint32_t)tok, ep + 1);
  }
}

// ----------------------------------------------------------------------------- the megakernel
// One instantiation per (head dim, query heads per KV head rounded up to 2, 4 or 8): the
// attention tile keeps GMAX x 8 query values and accumulators per lane in registers, and a
// kernel's register budget is set by its largest path.
// JIT: dynamic scheduling. Instead of walking its own queue, a workgroup takes the next slot of one
// device-wide ready queue and runs the task that lands there. A task's completion counts toward the
// one event it signals; the completion that finishes the event appends the event's consumer tasks
// (contiguous in the global order) to the queue. The tasks that wait on nothing fill its first slots.
// Slots are taken in order and a task waits only on tasks appended before it (attention merges on the
// layer's earlier attention tasks), all of which some workgroup has already taken: every wait ends.
// The kernel's parameters as a task reads them: scalar loads from the kernel-argument segment (the
// kernel's one explicit argument sits at its offset 0), through a pointer made opaque so that the loads
// happen when a task starts and cannot be hoisted out of the task loop. Held in scalar registers across
// the whole persistent loop instead, they overflowed the scalar file, and the spills into vector-register
// lanes made up about a sixth of the one-sequence kernel's code (76 KB before, 65 KB after).
__device__ __forceinline__ const KernelParams& task_params() {
  auto q = (const __attribute__((address_space(4))) KernelParams*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(q));
  return *(const KernelParams*)q;
}

template <int DH, int GMAX, bool BATCHED, bool FP8, bool JIT>
__global__ __launch_bounds__(NT, 1) void mk_megakernel(KernelParams launch_params) {
  const KernelParams& p = launch_params;  // set-up; each task reads task_params()
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  static_assert(sizeof(Ctl) <= 1024, "control block fits its 1 KB");
  Ctl* ctl = (Ctl*)lds_raw;
  // LDS: control block | per-layer K/V pool pointers | this CU's queue | working set
  uint16_t** pools = (uint16_t**)(lds_raw + 1024);
  const size_t pools_bytes = ((size_t)2 * p.n_layers * sizeof(void*) + 255) & ~size_t(255);
  TaskDesc* tq = (TaskDesc*)(lds_raw + 1024 + pools_bytes);
  // the attention tasks' first blocks for this step (W * i / T, i = 0..T), then the working set
  int32_t* alo = (int32_t*)((unsigned char*)tq + (((size_t)p.max_queue * sizeof(TaskDesc) + 255) & ~size_t(255)));
  float* lds = (float*)((unsigned char*)alo + (((size_t)(p.attn_tasks + 1) * 4 + 255) & ~size_t(255)));
  const int cu = blockIdx.x;
  // This launch runs the tasks of global order [task_lo, task_hi) (the whole step, or one dependency
  // stage in a stage-sliced launch): the contiguous part of this CU's queue inside that range.
  int q0 = p.queue_off[cu], q1 = p.queue_off[cu + 1];
  while (q0 < q1 && p.queue_idx[q0] < p.task_lo) ++q0;
  while (q1 > q0 && p.queue_idx[q1 - 1] >= p.task_hi) --q1;
  if constexpr (JIT) q0 = q1 = 0;  // no static queue: the loop below runs until the ready queue is done
  if (threadIdx.x < G_COUNT * (int)(sizeof(GemvGeom) / 4))
    ((int32_t*)ctl->geoms)[threadIdx.x] = ((const int32_t*)p.geoms)[threadIdx.x];
  for (int i = threadIdx.x; i < p.n_layers; i += NT) {
    pools[i] = p.kpool[i];
    pools[p.n_layers + i] = p.vpool[i];
  }
  // Stage the queue's descriptors in LDS: a task switch then costs an LDS read instead of two
  // dependent scalar loads from memory on the path between one task's publish and the next wait.
  for (int i = threadIdx.x; i < (q1 - q0) * 16; i += NT) {
    const int k = i >> 4, w = i & 15;
    ((int32_t*)&tq[k])[w] = ((const int32_t*)&p.tasks[p.queue_idx[q0 + k]])[w];
  }
  if constexpr (JIT) q1 = 0x7FFFFFFF;
  WPipe wp;
  int staged = 0;  // this wave's LDS stages hold the next GEMV task's units (bit 0: the stage, bit 1: the second)
  // Steps run one after another, each with its own epoch. Every task of a step is an ancestor of the
  // step's argmax, which every task of the next step follows, so a buffer rewritten in the next step has
  // no reader left in this one. One loop walks (step, task): a nested step loop keeps more values live
  // across the whole launch and costs registers.
  for (int step = 0, qi = q0; qi < q1;) {
    const KernelParams& p = task_params();
    const uint32_t ep = p.epoch + (uint32_t)step;
    if (qi == q0) {
      // Context lengths: read at launch, then one more per step for the running sequences (the argmax
      // task stores the same values). They change only between steps, after every reader.
      if (threadIdx.x < 16) {
        const int s = threadIdx.x;
        const bool act = s < min(p.n_active, p.max_seqs);
        const int pos = step == 0 ? (s < p.max_seqs ? p.ctx_lens[s] : 0) : ctl->ctx[s] + (act ? 1 : 0);
        ctl->ctx[s] = pos;
        // an active sequence attends to blocks 0 .. pos / 16 (one block when its position is out of
        // range: the task holding it reports the error and writes zeros)
        ctl->anb[s] = act ? ((pos >= 0 && pos < p.max_pos) ? (pos >> 4) + 1 : 1) : 0;
      }
      bar();
      if (threadIdx.x < 17) {  // first block of sequence s's segments: hk segments per earlier sequence
        int o = 0;
        for (int s = 0; s < (int)threadIdx.x; ++s) o += ctl->anb[s];
        ctl->aoff[threadIdx.x] = o * p.hk;
      }
      bar();
      {
        const int W = ctl->aoff[16], te = min(p.attn_tasks, max(1, (W + p.attn_min_blocks - 1) / p.attn_min_blocks));
        if constexpr (BATCHED) {  // several sequences: a cut by cost, each segment start counting kAttnPieceBlocks blocks
          for (int i = threadIdx.x; i <= p.attn_tasks; i += NT) alo[i] = attn_lo_cost(ctl, p.hk, W, te, min(i, te), kAttnPieceBlocks);
        } else {
          for (int i = threadIdx.x; i <= p.attn_tasks; i += NT) alo[i] = attn_lo_of(W, te, min(i, te));
        }
        if (threadIdx.x == 0) ctl->ate = te;
      }
      bar();
    }
    int tix = 0;  // JIT: the task's index in the global order
    if constexpr (JIT) {
      if (threadIdx.x == 0) {
        int32_t* work = p.jit_work;
        const int slot = __hip_atomic_fetch_add(&work[0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int v = -1;  // -1: every task is taken; -2: the kernel is aborting
        if (slot < p.task_hi) {
          const uint32_t* qs = (const uint32_t*)(work + 2 + p.n_events + slot);
          const uint64_t w0 = __builtin_amdgcn_s_memrealtime();
          for (uint32_t pass = 1;; ++pass) {
            v = (int)ldc(qs);
            if (v >= 0) break;
            if ((pass & 7u) == 0u) {
              if (ldc(&p.err[E_ABORT])) { v = -2; break; }
              if (__builtin_amdgcn_s_memrealtime() - w0 > p.watchdog_ticks) {
                raise_error(p, ERR_TIMEOUT, kWhatQueue, ep);
                stc(&p.err[E_ABORT], 1u);
                v = -2;
                break;
              }
            }
            __builtin_amdgcn_s_sleep(1);
          }
        }
        ctl->jtask = v;
      }
      bar();
      tix = __builtin_amdgcn_readfirstlane(ctl->jtask);
      if (tix < 0) break;
    }
    const TaskDesc t = JIT ? p.tasks[tix] : tq[qi - q0];
    // Only the LM head's partial maxima travel under flags (the argmax task waits for them); every
    // other input is a tagged activation that its consumer polls for inside the task.
    const int my_sig = (t.type == T_LMHEAD && (int)threadIdx.x < t.sig_n) ? p.sig_slots[t.sig_off + threadIdx.x] : -1;
    uint64_t t_queue = 0;
    if (p.trace && threadIdx.x == 0) {
      t_queue = __builtin_amdgcn_s_memrealtime();
      ctl->t_ready = t_queue;
      ctl->t_streamed = t_queue;
    }
    // Each task starts its own input streams before it polls for its inputs (they do not depend on
    // them): an attention task its first keys and values, a GEMV its first weight units.
    if (t.type == T_ATTN) {
      // position groups in flight per wave: more for batches (long streams), fewer for one sequence
      // and for many heads per KV head (register budget: one sequence with 8 heads per KV head spills
      // about 40 registers at 4 groups, 6 at 2)
      task_attn<DH, GMAX, (GMAX > 4 && !BATCHED) ? 2 : (GMAX > 4 || !BATCHED) ? 4 : 8, BATCHED>(p, ep, t, lds, ctl, pools, alo);
      staged = 0;
    } else if (t.type == T_ARGMAX) {
      staged = 0;
      if (t.wait_ev >= 0) wait_event(p, ep, t, ctl);
      if (p.trace && threadIdx.x == 0) ctl->t_ready = __builtin_amdgcn_s_memrealtime();
      if (t.wait_ev < 0 || !ctl->aborted) task_argmax(p, ep, step, t, ctl);
    } else if constexpr (BATCHED) {
      gemv_task_b(p, ep, step, t, lds, ctl, pools);
    } else {
      gemv_task<FP8>(p, ep, step, t, lds, ctl, wp, pools, (!JIT && qi + 1 < q1) ? &tq[qi + 1 - q0] : nullptr, staged);
    }
    // The LM head's stores must be complete before its flags go out; other tasks' consumers check
    // the tags themselves.
    if (t.type == T_LMHEAD) wait_stores();
    bar();
    publish(p, ep, my_sig);
    if (p.trace && threadIdx.x == 0) {
      TraceRec r;
      r.t_queue = t_queue;
      r.t_ready = ctl->t_ready;
      r.t_streamed = ctl->t_streamed;
      r.t_done = __builtin_amdgcn_s_memrealtime();
      r.cu = (uint16_t)cu;
      r.type = (uint8_t)t.type;
      r.layer = (uint8_t)t.layer;
      r.epoch = ep;
      r.xcc = __builtin_amdgcn_s_getreg(kHwRegXccId) & 0xFu;  // the XCD this CU sits on
      r.step = (uint32_t)step;
      p.trace[JIT ? tix : p.queue_idx[qi]] = r;
    }
    if constexpr (JIT) {
      // (after the trace record, so that a consumer never starts before its producer's recorded end)
      // count this completion toward its event; the one that finishes the event appends the event's
      // consumers to the ready queue (one slot range, written by the whole workgroup)
      if (threadIdx.x == 0) {
        int push = -1, c0 = 0, n = 0;
        const int e = p.jit_tab[tix];
        if (e >= 0) {
          __threadfence();
          const int32_t* evt = p.jit_tab + p.task_hi;  // [3][E]: producers, first consumer, end
          const int old = __hip_atomic_fetch_add(&p.jit_work[2 + e], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (old + 1 == evt[e]) {
            c0 = evt[p.n_events + e];
            n = evt[2 * p.n_events + e] - c0;
            if (n > 0) push = __hip_atomic_fetch_add(&p.jit_work[1], n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        ctl->jpush = push;
        ctl->jc0 = c0;
        ctl->jn = n;
      }
      bar();
      const int push = ctl->jpush;
      if (push >= 0) {
        uint32_t* q = (uint32_t*)(p.jit_work + 2 + p.n_events);
        for (int i = threadIdx.x; i < ctl->jn; i += NT) stc(&q[push + i], (uint32_t)(ctl->jc0 + i));
      }
    }
    if (++qi == q1 && ++step < p.n_steps) qi = q0;  // the next step walks the queue again
  }
}

// ----------------------------------------------------------------------------- weight re-layout
// One 64-thread block per 1 KB unit of a stage's tiles. Tasks [task0, task0 + ntasks) of the
// stage are contiguous in the task array with contiguous tiles.
// RepackArgs and RepackKind are declared in mk_graph.h.
// The natural-layout source row of packed row pr of a stage: QKV rows grouped per KV head and
// pair-interleaved within a head, gate/up rows alternating, other stages in order.
__device__ __forceinline__ const uint16_t* repack_src_row(const RepackArgs& a, int pr) {
  if (a.kind == RK_QKV) {
    const int Rg = (a.G + 2) * a.dh, grp = pr / Rg, within = pr % Rg, slot = within / a.dh, jh = within % a.dh;
    const int dim = (jh & 1) ? (jh >> 1) + a.dh / 2 : (jh >> 1);
    if (slot < a.G) return a.w0 + ((size_t)(grp * a.G + slot) * a.dh + dim) * a.gm.K;
    if (slot == a.G) return a.w1 + ((size_t)grp * a.dh + dim) * a.gm.K;
    return a.w2 + ((size_t)grp * a.dh + dim) * a.gm.K;
  }
  if (a.kind == RK_GU) return ((pr & 1) ? a.w1 : a.w0) + (size_t)(pr >> 1) * a.gm.K;
  return a.w0 + (size_t)pr * a.gm.K;
}

extern "C" __global__ __launch_bounds__(64) void mk_repack(RepackArgs a) {
  const int64_t unit = blockIdx.x;
  const int64_t byte = a.tasks[a.task0].wofs + unit * 1024;
  int lo = a.task0, hi = a.task0 + a.ntasks - 1;
  while (lo < hi) {  // last task whose tile starts at or before `byte`
    const int mid = (lo + hi + 1) >> 1;
    if (a.tasks[mid].wofs <= byte) lo = mid; else hi = mid - 1;
  }
  const TaskDesc t = a.tasks[lo];
  const int64_t u = (byte - t.wofs) / 1024;
  // one sequence: groups of S units; batched: groups of the task's own units, from its first column unit
  const int gs = a.gm.mfma ? (t.a2 >> 16) : a.gm.S, uoff = a.gm.mfma ? (t.a2 & 0xFFFF) : 0;
  const int gi = (int)(u / gs), ui = (int)(u % gs) + uoff;
  const int lane = threadIdx.x;
  const int rl = gi * a.gm.rg + (a.gm.mfma ? lane % 16 : lane / a.gm.lpr);
  const int piece = ui * a.gm.lpr + (a.gm.mfma ? lane / 16 : (lane & (a.gm.lpr - 1)));
  v4u v = {0u, 0u, 0u, 0u};
  if (rl < t.row1 - t.row0 && piece < a.gm.P) {
    const int pr = t.row0 + rl;
    const uint16_t* srow;
    if (a.kind == RK_QKV) {
      const int Rg = (a.G + 2) * a.dh, grp = pr / Rg, within = pr % Rg, slot = within / a.dh, jh = within % a.dh;
      const int dim = (jh & 1) ? (jh >> 1) + a.dh / 2 : (jh >> 1);
      if (slot < a.G) srow = a.w0 + ((size_t)(grp * a.G + slot) * a.dh + dim) * a.gm.K;
      else if (slot == a.G) srow = a.w1 + ((size_t)grp * a.dh + dim) * a.gm.K;
      else srow = a.w2 + ((size_t)grp * a.dh + dim) * a.gm.K;
    } else if (a.kind == RK_GU) {
      srow = ((pr & 1) ? a.w1 : a.w0) + (size_t)(pr >> 1) * a.gm.K;
    } else {
      srow = a.w0 + (size_t)pr * a.gm.K;
    }
    v = *(const v4u*)(srow + (size_t)piece * 8);
  }
  *((v4u*)(a.out + byte) + lane) = v;
}

// QKV bias in packed row order: one thread per packed row.
// ---- FP8 weights (OCP E4M3 codes, one power-of-two scale per packed row)
// The row's scale 2^e: e is the smallest integer with max |w| <= 448 * 2^e (448 = 0.875 * 2^9, the
// largest E4M3 value), clamped to [-100, 100]; 0 for a zero row. One wave per packed row.
extern "C" __global__ __launch_bounds__(64) void mk_row_scales(RepackArgs a, int nrows) {
  const int pr = blockIdx.x;
  if (pr >= nrows) return;
  const uint16_t* src = repack_src_row(a, pr);
  float m = 0.f;
  for (int k = threadIdx.x; k < a.gm.K; k += 64) m = fmaxf(m, fabsf(bf2f(src[k])));
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (threadIdx.x == 0) {
    int e = 0;
    if (m > 0.f) {
      int ex;
      const float fr = frexpf(m, &ex);  // m = fr 2^ex, fr in [0.5, 1)
      e = min(100, max(-100, ex - 9 + (fr > 0.875f ? 1 : 0)));
    }
    a.scales[a.scale0 + pr] = ldexpf(1.0f, e);
  }
}

// The E4M3 code nearest to v (|v| <= 448), ties to an even mantissa. In the normal range (exponents
// -6..8) the fp32 mantissa is rounded to 3 bits, to nearest even; below 2^-6 to the nearest multiple
// of 2^-9 (the subnormal step), where 8 steps carry into the smallest normal code.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t u = __float_as_uint(v), sign = (u >> 31) << 7, a = u & 0x7FFFFFFFu;
  const int E = (int)(a >> 23) - 127;
  uint32_t code;
  if (E < -6) {
    code = (uint32_t)rintf(__uint_as_float(a) * 512.0f);
  } else {
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    code = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
  }
  return sign | code;
}

// One 1 KB unit per block: lane (row rl, sub) packs the 16 codes of its row's pieces of bf16-layout
// units 2u and 2u + 1, each weight scaled by its row's 2^-e first (exact).
extern "C" __global__ __launch_bounds__(64) void mk_repack_fp8(RepackArgs a) {
  const int64_t unit = blockIdx.x;
  const int64_t byte = a.tasks[a.task0].wofs + unit * 1024;
  int lo = a.task0, hi = a.task0 + a.ntasks - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.tasks[mid].wofs <= byte) lo = mid; else hi = mid - 1;
  }
  const TaskDesc t = a.tasks[lo];
  const int64_t u = (byte - t.wofs) / 1024;
  const int su = a.gm.S / 2;
  const int gi = (int)(u / su), ui = (int)(u % su);
  const int lane = threadIdx.x;
  const int rl = gi * a.gm.rg + lane / a.gm.lpr, sub = lane & (a.gm.lpr - 1);
  uint32_t wd[4] = {0u, 0u, 0u, 0u};
  if (rl < t.row1 - t.row0) {
    const int pr = t.row0 + rl;
    const uint16_t* src = repack_src_row(a, pr);
    const float inv = 1.0f / a.scales[a.scale0 + pr];  // 2^-e, exact
    for (int h = 0; h < 2; ++h) {
      const int piece = (2 * ui + h) * a.gm.lpr + sub;
      if (piece >= a.gm.P) continue;
      for (int e = 0; e < 8; ++e) wd[2 * h + e / 4] |= e4m3_rne(bf2f(src[(size_t)piece * 8 + e]) * inv) << (8 * (e % 4));
    }
  }
  v4u v;
  v.x = wd[0]; v.y = wd[1]; v.z = wd[2]; v.w = wd[3];
  *((v4u*)(a.out + byte) + lane) = v;
}

extern "C" __global__ __launch_bounds__(256) void mk_repack_bias(const uint16_t* bq, const uint16_t* bk,
                                                                  const uint16_t* bv, int G, int dh, int nrows,
                                                                  uint16_t* out) {
  const int pr = blockIdx.x * 256 + threadIdx.x;
  if (pr >= nrows) return;
  const int Rg = (G + 2) * dh, grp = pr / Rg, within = pr % Rg, slot = within / dh, jh = within % dh;
  const int dim = (jh & 1) ? (jh >> 1) + dh / 2 : (jh >> 1);
  uint16_t v;
  if (slot < G) v = bq[(grp * G + slot) * dh + dim];
  else if (slot == G) v = bk[grp * dh + dim];
  else v = bv[grp * dh + dim];
  out[pr] = v;
}

// ----------------------------------------------------------------------------- host-side launchers
template <bool B, bool F, bool J>
static const void* megakernel_for_t(int dh, int g) {
  if (dh == 128)
    return g <= 2 ? (const void*)mk_megakernel<128, 2, B, F, J> : g <= 4 ? (const void*)mk_megakernel<128, 4, B, F, J>
                                                                         : (const void*)mk_megakernel<128, 8, B, F, J>;
  return g <= 2 ? (const void*)mk_megakernel<64, 2, B, F, J> : g <= 4 ? (const void*)mk_megakernel<64, 4, B, F, J>
                                                                       : (const void*)mk_megakernel<64, 8, B, F, J>;
}
// One sequence: GEMV tiles on the vector units, over bf16 or FP8 weights, from static queues or (bf16)
// the ready queue. Several: the batched instantiation (MFMA tiles, bf16 weights).
static const void* megakernel_for(int dh, int hq, int hk, bool batched, bool fp8, bool jit) {
  if (batched) return megakernel_for_t<true, false, false>(dh, hq / hk);
  if (jit) return megakernel_for_t<false, false, true>(dh, hq / hk);
  return fp8 ? megakernel_for_t<false, true, false>(dh, hq / hk) : megakernel_for_t<false, false, false>(dh, hq / hk);
}

hipError_t launch_megakernel(const KernelParams& p, int grid, size_t lds_bytes, hipStream_t stream, bool coop) {
  KernelParams copy = p;
  void* args[] = {(void*)&copy};
  // The grid is one workgroup per CU and the LDS allows one per CU, so on a device running nothing
  // else every workgroup is resident at once, which the task queues need. A launch of several steps is
  // cooperative: the runtime then guarantees co-residency, for about 18 us per dispatch on MI355X,
  // which the steps share. A single step uses a plain launch by default; where other work may hold
  // CUs, MK_COOPERATIVE_LAUNCH=1 makes it cooperative too. (Without it, waits that cannot be met end at
  // the watchdog with an error, not in a hang.)
  static const bool coop_env = std::getenv("MK_COOPERATIVE_LAUNCH") != nullptr;
  if (coop || coop_env)
    return hipLaunchCooperativeKernel(megakernel_for(p.dh, p.hq, p.hk, p.max_seqs > 1, p.fp8_weights != 0, p.jit_tab != nullptr), dim3(grid), dim3(NT), args,
                                      (unsigned)lds_bytes, stream);
  return hipLaunchKernel(megakernel_for(p.dh, p.hq, p.hk, p.max_seqs > 1, p.fp8_weights != 0, p.jit_tab != nullptr), dim3(grid), dim3(NT), args,
                         (unsigned)lds_bytes, stream);
}

hipError_t megakernel_occupancy(int* blocks_per_cu, size_t lds_bytes, int dh, int hq, int hk, bool batched, bool fp8) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, megakernel_for(dh, hq, hk, batched, fp8, false), NT, lds_bytes);
}

// ----------------------------------------------------------------------------- static scratch
// The working memory of the entry point that allocates nothing (mk_decode_step_static): the step's copy
// of the task graph and rotary table, the event flags, the tagged activations, the partial results and
// the argmax keys live in this array instead of the caller's scratch buffer. Every GPU the library runs
// on holds its own copy until the process ends. In host code the name is a stand-in, not a device
// address: host code uses only the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

// The device address of `scratch` on `device`, resolved once per device with that device current.
hipError_t static_scratch_address(int device, void** out) {
  static std::mutex mu;
  static void* addr[64] = {};
  if (device < 0 || device >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device) return hipErrorInvalidDevice;  // the caller makes `device` current first
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    addr[device] = ptr;
  }
  *out = addr[device];
  return hipSuccess;
}

// Zeroes [p, p + bytes) (16-byte aligned, a multiple of 16) with plain stores: a fill kernel rather than
// hipMemsetAsync, so that the clearing can sit in a captured graph.
extern "C" __global__ __launch_bounds__(256) void mk_fill_zero(v4u* p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) p[i] = v4u{0u, 0u, 0u, 0u};
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  if (((uintptr_t)p & 15) || (bytes & 15)) return hipErrorInvalidValue;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t blocks = (n16 + 255) / 256;
  hipLaunchKernelGGL(mk_fill_zero, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, stream, (v4u*)p, n16);
  return hipGetLastError();
}

hipError_t launch_repack(const RepackArgs& a, int64_t units, hipStream_t stream) {
  if (units <= 0) return hipSuccess;
  hipLaunchKernelGGL(mk_repack, dim3((unsigned)units), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_row_scales(const RepackArgs& a, int nrows, hipStream_t stream) {
  hipLaunchKernelGGL(mk_row_scales, dim3((unsigned)nrows), dim3(64), 0, stream, a, nrows);
  return hipGetLastError();
}

hipError_t launch_repack_fp8(const RepackArgs& a, int64_t units, hipStream_t stream) {
  hipLaunchKernelGGL(mk_repack_fp8, dim3((unsigned)units), dim3(64), 0, stream, a);
  return hipGetLastError();
}

// Dynamic scheduling, before each launch: queue head 0, tail n0 (the opening tasks in slots 0..n0-1),
// event counts 0, the other slots empty (-1). A kernel, not a memset, so the launch may be captured.
extern "C" __global__ __launch_bounds__(256) void mk_jit_reset(int32_t* w, int n_events, int n_tasks, int n0) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= 2 + n_events + n_tasks) return;
  int v = 0;
  if (i == 1) v = n0;
  else if (i >= 2 + n_events) v = (i - 2 - n_events) < n0 ? (i - 2 - n_events) : -1;
  w[i] = v;
}

hipError_t launch_jit_reset(int32_t* w, int n_events, int n_tasks, int n0, hipStream_t stream) {
  const int n = 2 + n_events + n_tasks;
  hipLaunchKernelGGL(mk_jit_reset, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, w, n_events, n_tasks, n0);
  return hipGetLastError();
}

hipError_t launch_repack_bias(const uint16_t* bq, const uint16_t* bk, const uint16_t* bv, int G, int dh, int nrows,
                              uint16_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(mk_repack_bias, dim3((nrows + 255) / 256), dim3(256), 0, stream, bq, bk, bv, G, dh, nrows, out);
  return hipGetLastError();
}

}  // namespace mk
