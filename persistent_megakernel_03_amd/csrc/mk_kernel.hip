// The persistent decode megakernel for gfx950 (CDNA4), and the weight re-layout kernel.
//
// One workgroup of 512 threads (8 wave64s) runs on each CU, launched cooperatively, so all
// are co-resident. Each workgroup walks its own task queue. For each task it:
//   - waits for its input event,
//   - runs the tile,
//   - publishes its epoch number into its flag slots.
// This is the worker loop of the Mirage Persistent Kernel ("LLMs in einen MegaKernel
// kompilieren", "Worker" and "Ereignisbasierte Ausführung"). The pages' separate scheduler
// SMs are folded into the workers. The queues are built ahead of time (the AOT launch of
// "MPK: A Compiler and Runtime for Mega-Kernelizing Tensor Programs", analogy 3). So the
// scheduler's job reduces to one wave polling the event's flags. Every CU keeps streaming
// weights; giving up CUs to scheduling would cost a share of the HBM stream.
//
// Memory model. Data that one CU writes and another CU reads in the same step goes through
// agent-scope atomic loads and stores (the sc1 cache policy). These are coherent across the
// XCDs' separate L2 caches. Ordering uses one rule: a producer's waves wait for their
// stores to complete (s_waitcnt vmcnt(0)) before one lane stores the flag. A consumer
// polls the flags with agent-scope loads, and only after that issues its data loads.
// Weights and the KV rows of earlier steps are immutable within a step. They are read with
// plain nontemporal loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_graph.h"

namespace mk {

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int NT = 512;     // threads per workgroup
constexpr int NW = NT / 64; // waves per workgroup
constexpr int UB = 8;       // 1 KB units per load batch per wave (two batches in flight)

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

__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// Small control block at the start of LDS.
struct Ctl {
  float red[NW * 8];
  float m_run[16], l_run[16], scale[16];
  uint32_t flag;
  uint32_t aborted;
  uint64_t kred[NW];
};

__device__ __forceinline__ float block_sum(float v, Ctl* ctl) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) ctl->red[w] = v;
  __syncthreads();
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

// ----------------------------------------------------------------------------- events
// Wave 0 polls every producer flag of the event until all hold >= epoch. A watchdog on the
// 100 MHz real-time counter turns a wait that never ends into an error and a kernel-wide abort.
__device__ void wait_event(const KernelParams& p, int ev, Ctl* ctl) {
  if (threadIdx.x < 64) {
    const EventDesc e = p.events[ev];
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    const int lane = threadIdx.x;
    uint32_t ab = 0;
    while (true) {
      bool ok = true;
      for (int i = lane; i < e.nslots; i += 64) ok = ok && (ldc(&p.flags[e.slot0 + i]) >= p.epoch);
      if (__all(ok)) break;
      ab = ldc(&p.err[E_ABORT]);
      if (ab) break;
      if (__builtin_amdgcn_s_memrealtime() - t0 > p.watchdog_ticks) {
        if (lane == 0) {
          raise_error(p, ERR_TIMEOUT, (uint32_t)ev, p.epoch);
          stc(&p.err[E_ABORT], 1u);
        }
        ab = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (lane == 0) ctl->aborted = ab;
  }
  __syncthreads();
}

// Every wave waits for its own stores, then one lane per slot publishes the epoch.
__device__ void signal_slots(const KernelParams& p, const TaskDesc& t) {
  wait_stores();
  __syncthreads();
  if ((int)threadIdx.x < t.sig_n) stc(&p.flags[p.sig_slots[t.sig_off + threadIdx.x]], p.epoch);
}

// ----------------------------------------------------------------------------- GEMV tile
// ys[r] = sum_k W[row0 + r][k] * xs[k] for the task's rows. Row groups are split evenly over
// the 8 waves. Each wave streams its contiguous run of 1 KB units with nontemporal dwordx4
// loads, two batches of UB units in flight. The xs entries past K are zero, and so are the
// padded weights.
__device__ __forceinline__ void unit_fma(const v4u w, const float* xp, float& acc) {
  const v4f a = *(const v4f*)xp;
  const v4f b = *(const v4f*)(xp + 4);
  acc = fmaf(bf_lo(w.x), a.x, acc);
  acc = fmaf(bf_hi(w.x), a.y, acc);
  acc = fmaf(bf_lo(w.y), a.z, acc);
  acc = fmaf(bf_hi(w.y), a.w, acc);
  acc = fmaf(bf_lo(w.z), b.x, acc);
  acc = fmaf(bf_hi(w.z), b.y, acc);
  acc = fmaf(bf_lo(w.w), b.z, acc);
  acc = fmaf(bf_hi(w.w), b.w, acc);
}

__device__ void gemv_tile(const KernelParams& p, const TaskDesc& t, const GemvGeom gm, const float* xs, float* ys) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rows = t.row1 - t.row0;
  const int ngroups = (rows + gm.rg - 1) / gm.rg;
  const int gA = ngroups * wave / NW, gB = ngroups * (wave + 1) / NW;
  const int S = gm.S, lpr = gm.lpr;
  const int nunits = (gB - gA) * S;
  const int sub = lane & (lpr - 1), rin = lane / lpr;
  const v4u* src = (const v4u*)(p.wpacked + t.wofs) + (size_t)gA * S * 64 + lane;
  int g = gA, ug = 0;
  float acc = 0.f;
  v4u A[UB], B[UB];

  auto load = [&](v4u(&R)[UB], int i0) {
#pragma unroll
    for (int j = 0; j < UB; ++j)
      if (i0 + j < nunits) R[j] = __builtin_nontemporal_load(src + (size_t)(i0 + j) * 64);
  };
  auto consume = [&](v4u(&R)[UB], int i0) {
#pragma unroll
    for (int j = 0; j < UB; ++j) {
      if (i0 + j < nunits) {
        unit_fma(R[j], xs + (ug * lpr + sub) * 8, acc);
        if (++ug == S) {
          for (int off = lpr >> 1; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
          const int r = g * gm.rg + rin;
          if (sub == 0 && r < rows) ys[r] = acc;
          acc = 0.f;
          ug = 0;
          ++g;
        }
      }
    }
  };
  load(A, 0);
  for (int i0 = 0; i0 < nunits; i0 += 2 * UB) {
    load(B, i0 + UB);
    consume(A, i0);
    load(A, i0 + 2 * UB);
    consume(B, i0 + UB);
  }
}

// xs[0, K) = RMSNorm(src) * gain; xs[K, padded) = 0. src is the residual stream (fp32, coherent
// loads) or, for the first layer, the token's embedding row (bf16).
__device__ void rmsnorm_to_lds(const KernelParams& p, const float* xsrc, const uint16_t* esrc, const uint16_t* gain,
                               int d, int padded, float* xs, Ctl* ctl) {
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += NT) {
    const float v = esrc ? bf2f(esrc[i]) : ldc(&xsrc[i]);
    xs[i] = v;
    ss += v * v;
  }
  for (int i = d + threadIdx.x; i < padded; i += NT) xs[i] = 0.f;
  ss = block_sum(ss, ctl);
  const float r = 1.0f / sqrtf(ss / (float)d + p.eps);
  for (int i = threadIdx.x; i < d; i += NT) xs[i] = xs[i] * r * bf2f(gain[i]);
  __syncthreads();
}

__device__ void load_vec_to_lds(const float* src, int n, int padded, float* xs) {
  for (int i = threadIdx.x; i < n; i += NT) xs[i] = ldc(&src[i]);
  for (int i = n + threadIdx.x; i < padded; i += NT) xs[i] = 0.f;
  __syncthreads();
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
__device__ __forceinline__ int checked_pos(const KernelParams& p, int s) {
  const int pos = p.ctx_lens[s];
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
__device__ void task_qkv(const KernelParams& p, const TaskDesc& t, float* lds, Ctl* ctl) {
  const GemvGeom gm = p.geoms[G_QKV];
  const int padded = gm.S * gm.lpr * 8;
  float* xs = lds;
  float* ys = lds + padded;
  const int s = 0;
  const int l = t.layer;
  const uint16_t* esrc = nullptr;
  if (l == 0) esrc = p.embed + (size_t)token_of(p, s) * p.d;
  rmsnorm_to_lds(p, p.x + (size_t)s * p.d, esrc, layer_norm_gain(p, l, 0), p.d, padded, xs, ctl);
  gemv_tile(p, t, gm, xs, ys);
  __syncthreads();
  const int G = p.hq / p.hk, dh = p.dh, Rg = (G + 2) * dh;
  const int pos = checked_pos(p, s);
  const int nsets = pos < 0 ? 0 : (t.row1 - t.row0) >> 2;
  for (int m = threadIdx.x; m < nsets; m += NT) {
    const int r = t.row0 + 4 * m;
    const int grp = r / Rg, within = r % Rg, slot = within / dh, jh = within % dh;
    const int i0 = jh >> 1;  // even dim index; the set holds dims i0, i0 + dh/2, i0 + 1, i0 + 1 + dh/2
    float y0 = ys[4 * m], y1 = ys[4 * m + 1], y2 = ys[4 * m + 2], y3 = ys[4 * m + 3];
    if (p.bias) {
      const uint16_t* b = p.bias + (size_t)l * (p.hq + 2 * p.hk) * dh + r;
      y0 += bf2f(b[0]); y1 += bf2f(b[1]); y2 += bf2f(b[2]); y3 += bf2f(b[3]);
    }
    if (slot <= G) {  // rotate q and k: pair (i0, i0 + dh/2) and pair (i0 + 1, i0 + 1 + dh/2)
      const float2 cs0 = ((const float2*)p.rope)[(size_t)pos * (dh / 2) + i0];
      const float2 cs1 = ((const float2*)p.rope)[(size_t)pos * (dh / 2) + i0 + 1];
      const float a0 = y0 * cs0.x - y1 * cs0.y, b0 = y1 * cs0.x + y0 * cs0.y;
      const float a1 = y2 * cs1.x - y3 * cs1.y, b1 = y3 * cs1.x + y2 * cs1.y;
      y0 = a0; y1 = b0; y2 = a1; y3 = b1;
    }
    if (slot < G) {
      float* q = p.q + (size_t)s * p.hq * dh + (size_t)(grp * G + slot) * dh;
      stc(&q[i0], y0);
      stc(&q[i0 + dh / 2], y1);
      stc(&q[i0 + 1], y2);
      stc(&q[i0 + 1 + dh / 2], y3);
    } else {
      const int blk = p.page_table[(size_t)s * p.max_blocks + pos / 16];
      if (blk < 0 || blk >= p.num_blocks) {
        raise_error(p, ERR_PAGE, (uint32_t)s, (uint32_t)blk);
        continue;
      }
      uint16_t* pool = (slot == G ? p.kpool : p.vpool)[l];
      uint32_t* row = (uint32_t*)(pool + (((size_t)blk * p.hk + grp) * 16 + (pos & 15)) * dh);
      stc(&row[i0 >> 1], f2bf(y0) | (f2bf(y2) << 16));
      stc(&row[(i0 + dh / 2) >> 1], f2bf(y1) | (f2bf(y3) << 16));
    }
  }
  signal_slots(p, t);
}

// ----------------------------------------------------------------------------- attention
// One split of grouped-query attention for (seq, kv head): its range of cache blocks.
// The G query heads that share the KV head read each key and value row once. Online
// softmax runs over chunks of up to 512 positions. The running max and sum rescale the
// output ([SL] slide 13 and the kernel page's online-softmax passage). The partial
// (m, l, unnormalised o) goes to `part`. The split that finishes last merges all partials
// by log-sum-exp and publishes the group's slot.
template <int DH, int GMAX>
__device__ void task_attn(const KernelParams& p, const TaskDesc& t, float* lds, Ctl* ctl) {
  constexpr int LPP = DH / 8;       // lanes per position (8 dims each)
  constexpr int PPW = 64 / LPP;     // positions per wave per step
  constexpr int CH = 512;           // positions per chunk
  const int s = t.a0, grp = t.a1, j = t.a2;
  const int G = p.hq / p.hk, h0 = grp * G;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, pg = lane / LPP, c = lane % LPP;
  const int cpos = s < p.n_active ? checked_pos(p, s) : -1;
  const bool active = cpos >= 0;
  float* scores = lds;                  // [G][CH]
  float* obuf = lds + G * CH;           // [NW][G][DH]
  const int splits = p.splits;
  float* part = p.part + ((size_t)s * p.hq) * splits * (DH + 2);

  int p0 = 0, p1 = 0, pos = 0;
  if (active) {
    pos = cpos;
    const int n = pos + 1, nb = (n + 15) >> 4, pps = (nb + splits - 1) / splits;
    p0 = min(n, j * pps * 16);
    p1 = min(n, (j + 1) * pps * 16);
  }
  const uint16_t* kpool = p.kpool[t.layer];
  const uint16_t* vpool = p.vpool[t.layer];
  const int32_t* ptab = p.page_table + (size_t)s * p.max_blocks;
  const float scale = 1.0f / sqrtf((float)DH);

  float qr[GMAX][8];  // this lane's 8 dims of each query head of the group
#pragma unroll
  for (int h = 0; h < GMAX; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) qr[h][e] = (h < G && active) ? ldc(&p.q[(size_t)s * p.hq * DH + (size_t)(h0 + h) * DH + c * 8 + e]) : 0.f;
  float oacc[GMAX][8];
#pragma unroll
  for (int h = 0; h < GMAX; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) oacc[h][e] = 0.f;
  if (threadIdx.x < 16) {
    ctl->m_run[threadIdx.x] = -INFINITY;
    ctl->l_run[threadIdx.x] = 0.f;
  }
  __syncthreads();

  auto row_ptr = [&](const uint16_t* pool, int pp) -> const uint16_t* {
    int blk = ptab[pp >> 4];
    if (blk < 0 || blk >= p.num_blocks) {
      raise_error(p, ERR_PAGE, (uint32_t)s, (uint32_t)blk);
      blk = 0;
    }
    return pool + (((size_t)blk * p.hk + grp) * 16 + (pp & 15)) * DH + c * 8;
  };
  auto load_row = [&](const uint16_t* pool, int pp) -> v4u {
    const uint16_t* rp = row_ptr(pool, pp);
    if (pp == pos) {  // written by another CU in this step: coherent loads
      const uint32_t* r32 = (const uint32_t*)rp;
      v4u v;
      v.x = ldc(&r32[0]); v.y = ldc(&r32[1]); v.z = ldc(&r32[2]); v.w = ldc(&r32[3]);
      return v;
    }
    return __builtin_nontemporal_load((const v4u*)rp);
  };

  for (int cs = p0; cs < p1; cs += CH) {
    const int ce = min(p1, cs + CH);
    // scores = q . k * scale
    for (int base = cs + wave * PPW; base < ce; base += NW * PPW) {
      const int pp = base + pg;
      const bool valid = pp < ce;
      v4u kv = {0u, 0u, 0u, 0u};
      if (valid) kv = load_row(kpool, pp);
      float kf[8] = {bf_lo(kv.x), bf_hi(kv.x), bf_lo(kv.y), bf_hi(kv.y), bf_lo(kv.z), bf_hi(kv.z), bf_lo(kv.w), bf_hi(kv.w)};
#pragma unroll
      for (int h = 0; h < GMAX; ++h) {
        if (h >= G) break;
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaf(qr[h][e], kf[e], a);
#pragma unroll
        for (int off = LPP >> 1; off >= 1; off >>= 1) a += __shfl_xor(a, off);
        if (c == 0 && valid) scores[h * CH + (pp - cs)] = a * scale;
      }
    }
    __syncthreads();
    // chunk max and running-max update, one wave per head
    const int nch = ce - cs;
    for (int h = wave; h < G; h += NW) {
      float mx = -INFINITY;
      for (int i = lane; i < nch; i += 64) mx = fmaxf(mx, scores[h * CH + i]);
      mx = wave_max(mx);
      const float m_old = ctl->m_run[h];
      const float m_new = fmaxf(m_old, mx);
      float sum = 0.f;
      for (int i = lane; i < nch; i += 64) {
        const float e = expf(scores[h * CH + i] - m_new);
        scores[h * CH + i] = e;
        sum += e;
      }
      sum = wave_sum(sum);
      if (lane == 0) {
        const float sc = (m_old == -INFINITY) ? 0.f : expf(m_old - m_new);
        ctl->scale[h] = sc;
        ctl->l_run[h] = ctl->l_run[h] * sc + sum;
        ctl->m_run[h] = m_new;
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      if (h >= G) break;
      const float sc = ctl->scale[h];
#pragma unroll
      for (int e = 0; e < 8; ++e) oacc[h][e] *= sc;
    }
    // o += p * v
    for (int base = cs + wave * PPW; base < ce; base += NW * PPW) {
      const int pp = base + pg;
      if (pp < ce) {
        const v4u vv = load_row(vpool, pp);
        const float vf[8] = {bf_lo(vv.x), bf_hi(vv.x), bf_lo(vv.y), bf_hi(vv.y), bf_lo(vv.z), bf_hi(vv.z), bf_lo(vv.w), bf_hi(vv.w)};
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
          if (h >= G) break;
          const float pw = scores[h * CH + (pp - cs)];
#pragma unroll
          for (int e = 0; e < 8; ++e) oacc[h][e] = fmaf(pw, vf[e], oacc[h][e]);
        }
      }
    }
    __syncthreads();
  }
  // reduce o over the position groups of each wave, then over waves
#pragma unroll
  for (int h = 0; h < GMAX; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = oacc[h][e];
      for (int off = LPP; off < 64; off <<= 1) v += __shfl_xor(v, off);
      oacc[h][e] = v;
    }
  if (pg == 0)
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      if (h >= G) break;
#pragma unroll
      for (int e = 0; e < 8; ++e) obuf[(wave * G + h) * DH + c * 8 + e] = oacc[h][e];
    }
  __syncthreads();
  if (active) {
    for (int i = threadIdx.x; i < G * DH; i += NT) {
      const int h = i / DH, dd = i % DH;
      float v = 0.f;
      for (int w = 0; w < NW; ++w) v += obuf[(w * G + h) * DH + dd];
      stc(&part[((size_t)(h0 + h) * splits + j) * (DH + 2) + 2 + dd], v);
    }
    if (threadIdx.x < G) {
      stc(&part[((size_t)(h0 + threadIdx.x) * splits + j) * (DH + 2) + 0], ctl->m_run[threadIdx.x]);
      stc(&part[((size_t)(h0 + threadIdx.x) * splits + j) * (DH + 2) + 1], ctl->l_run[threadIdx.x]);
    }
  }
  // arrive; the last split of the group merges
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&p.counters[t.a3], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ctl->flag = (old + 1 == p.epoch * (uint32_t)splits) ? 1u : 0u;
  }
  __syncthreads();
  if (!ctl->flag) return;
  if (active) {
    for (int i = threadIdx.x; i < G * DH; i += NT) {
      const int h = i / DH, dd = i % DH;
      const float* ph = part + (size_t)(h0 + h) * splits * (DH + 2);
      float M = -INFINITY;
      for (int k = 0; k < splits; ++k) M = fmaxf(M, ldc(&ph[k * (DH + 2)]));
      float Lsum = 0.f, acc = 0.f;
      for (int k = 0; k < splits; ++k) {
        const float mk = ldc(&ph[k * (DH + 2)]);
        if (mk == -INFINITY) continue;
        const float w = expf(mk - M);
        Lsum += ldc(&ph[k * (DH + 2) + 1]) * w;
        acc += ldc(&ph[k * (DH + 2) + 2 + dd]) * w;
      }
      stc(&p.o[(size_t)s * p.hq * DH + (size_t)(h0 + h) * DH + dd], acc / Lsum);
    }
  }
  signal_slots(p, t);
}

// ----------------------------------------------------------------------------- O / down projection
__device__ void task_residual_gemv(const KernelParams& p, const TaskDesc& t, float* lds, Ctl* ctl, int geom,
                                   const float* in, int n_in) {
  const GemvGeom gm = p.geoms[geom];
  const int padded = gm.S * gm.lpr * 8;
  float* xs = lds;
  float* ys = lds + padded;
  const int s = 0;
  load_vec_to_lds(in + (size_t)s * n_in, n_in, padded, xs);
  gemv_tile(p, t, gm, xs, ys);
  __syncthreads();
  const bool from_embed = (t.type == T_OPROJ && t.layer == 0);
  const uint16_t* erow = from_embed ? p.embed + (size_t)token_of(p, s) * p.d : nullptr;
  for (int r = t.row0 + threadIdx.x; r < t.row1; r += NT) {
    const float resid = from_embed ? bf2f(erow[r]) : ldc(&p.x[(size_t)s * p.d + r]);
    stc(&p.x[(size_t)s * p.d + r], resid + ys[r - t.row0]);
  }
  signal_slots(p, t);
}

// ----------------------------------------------------------------------------- gate/up + SwiGLU
__device__ void task_gateup(const KernelParams& p, const TaskDesc& t, float* lds, Ctl* ctl) {
  const GemvGeom gm = p.geoms[G_GU];
  const int padded = gm.S * gm.lpr * 8;
  float* xs = lds;
  float* ys = lds + padded;
  const int s = 0;
  rmsnorm_to_lds(p, p.x + (size_t)s * p.d, nullptr, layer_norm_gain(p, t.layer, 1), p.d, padded, xs, ctl);
  gemv_tile(p, t, gm, xs, ys);
  __syncthreads();
  const int npairs = (t.row1 - t.row0) >> 1;
  for (int m = threadIdx.x; m < npairs; m += NT) {
    const float a = ys[2 * m], b = ys[2 * m + 1];
    const float silu = a / (1.0f + expf(-a));
    stc(&p.h[(size_t)s * p.f + (t.row0 >> 1) + m], silu * b);
  }
  signal_slots(p, t);
}

// ----------------------------------------------------------------------------- LM head + argmax
// Order-preserving key: larger float -> larger key; on equal values the lower index wins.
__device__ __forceinline__ uint64_t argmax_key(float v, int idx) {
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}

__device__ uint64_t block_max_u64(uint64_t k, Ctl* ctl) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = __shfl_xor(k, off);
    k = o > k ? o : k;
  }
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) ctl->kred[w] = k;
  __syncthreads();
  uint64_t m = 0;
  for (int i = 0; i < NW; ++i) m = ctl->kred[i] > m ? ctl->kred[i] : m;
  return m;
}

__device__ void task_lmhead(const KernelParams& p, const TaskDesc& t, float* lds, Ctl* ctl) {
  const GemvGeom gm = p.geoms[G_LM];
  const int padded = gm.S * gm.lpr * 8;
  float* xs = lds;
  float* ys = lds + padded;
  const int s = 0;
  rmsnorm_to_lds(p, p.x + (size_t)s * p.d, nullptr, p.norms + (size_t)p.n_layers * 2 * p.d, p.d, padded, xs, ctl);
  gemv_tile(p, t, gm, xs, ys);
  __syncthreads();
  uint64_t best = 0;
  for (int r = t.row0 + threadIdx.x; r < t.row1; r += NT) {
    const float v = ys[r - t.row0];
    p.logits[(size_t)s * p.vocab + r] = v;
    const uint64_t k = argmax_key(v, r);
    best = k > best ? k : best;
  }
  best = block_max_u64(best, ctl);
  if (threadIdx.x == 0) stc(&p.amax[(size_t)s * p.n_lm_parts + t.a0], best);
  signal_slots(p, t);
}

__device__ void task_argmax(const KernelParams& p, const TaskDesc& t, Ctl* ctl) {
  const int s = t.a0;
  uint64_t best = 0;
  for (int i = threadIdx.x; i < p.n_lm_parts; i += NT) {
    const uint64_t k = ldc(&p.amax[(size_t)s * p.n_lm_parts + i]);
    best = k > best ? k : best;
  }
  best = block_max_u64(best, ctl);
  if (threadIdx.x == 0 && s < p.n_active) {
    p.tokens_out[s] = (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
    p.ctx_lens[s] = p.ctx_lens[s] + 1;
  }
}

// ----------------------------------------------------------------------------- the megakernel
extern "C" __global__ __launch_bounds__(NT, 1) void mk_megakernel(KernelParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  Ctl* ctl = (Ctl*)lds_raw;
  float* lds = (float*)(lds_raw + ((sizeof(Ctl) + 255) & ~size_t(255)));
  const int cu = blockIdx.x;
  const int q0 = p.queue_off[cu], q1 = p.queue_off[cu + 1];
  for (int qi = q0; qi < q1; ++qi) {
    const TaskDesc t = p.tasks[p.queue_idx[qi]];
    if (t.wait_ev >= 0) {
      wait_event(p, t.wait_ev, ctl);
      if (ctl->aborted) {  // drain: publish without computing so no other CU waits forever
        signal_slots(p, t);
        continue;
      }
    }
    switch (t.type) {
      case T_QKV: task_qkv(p, t, lds, ctl); break;
      case T_ATTN:
        if (p.dh == 128) task_attn<128, 8>(p, t, lds, ctl);
        else task_attn<64, 8>(p, t, lds, ctl);
        break;
      case T_OPROJ: task_residual_gemv(p, t, lds, ctl, G_O, p.o, p.hq * p.dh); break;
      case T_GATEUP: task_gateup(p, t, lds, ctl); break;
      case T_DOWN: task_residual_gemv(p, t, lds, ctl, G_D, p.h, p.f); break;
      case T_LMHEAD: task_lmhead(p, t, lds, ctl); break;
      case T_ARGMAX: task_argmax(p, t, ctl); break;
      default: break;
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------- weight re-layout
// One 64-thread block per 1 KB unit of a stage's tiles. Tasks [task0, task0 + ntasks) of the
// stage are contiguous in the task array with contiguous tiles.
// RepackArgs and RepackKind are declared in mk_graph.h.
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
  const int gi = (int)(u / a.gm.S), ui = (int)(u % a.gm.S);
  const int lane = threadIdx.x;
  const int rl = gi * a.gm.rg + lane / a.gm.lpr;
  const int piece = ui * a.gm.lpr + (lane & (a.gm.lpr - 1));
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
hipError_t launch_megakernel(const KernelParams& p, int grid, size_t lds_bytes, hipStream_t stream) {
  KernelParams copy = p;
  void* args[] = {(void*)&copy};
  return hipLaunchCooperativeKernel((const void*)mk_megakernel, dim3(grid), dim3(NT), args, (unsigned)lds_bytes, stream);
}

hipError_t megakernel_occupancy(int* blocks_per_cu, size_t lds_bytes) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, (const void*)mk_megakernel, NT, lds_bytes);
}

hipError_t launch_repack(const RepackArgs& a, int64_t units, hipStream_t stream) {
  if (units <= 0) return hipSuccess;
  hipLaunchKernelGGL(mk_repack, dim3((unsigned)units), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_repack_bias(const uint16_t* bq, const uint16_t* bk, const uint16_t* bv, int G, int dh, int nrows,
                              uint16_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(mk_repack_bias, dim3((nrows + 255) / 256), dim3(256), 0, stream, bq, bk, bv, G, dh, nrows, out);
  return hipGetLastError();
}

}  // namespace mk
