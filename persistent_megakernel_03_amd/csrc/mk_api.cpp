// Host runtime behind the C ABI declared in include/mk.h.
//
// It owns only host structures: the config and the task graph. All device memory
// belongs to the caller and is bound once. A decode step is one launch of the
// megakernel; the host does no synchronisation and no per-token
// bookkeeping beyond incrementing the step epoch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_host.h"

namespace mk {
hipError_t launch_megakernel(const KernelParams& p, int grid, size_t lds_bytes, hipStream_t stream);
hipError_t megakernel_occupancy(int* blocks_per_cu, size_t lds_bytes, int dh, int hq, int hk, bool batched);
hipError_t launch_repack(const RepackArgs& a, int64_t units, hipStream_t stream);
hipError_t launch_repack_bias(const uint16_t* bq, const uint16_t* bk, const uint16_t* bv, int G, int dh, int nrows,
                              uint16_t* out, hipStream_t stream);
}  // namespace mk

using namespace mk;

struct mk_ctx {
  HostGraph g;
  int device = -1;  // -1: host-only context
  bool bound = false, loaded = false;
  uint8_t* d_weights = nullptr;
  uint8_t* d_scratch = nullptr;
  std::vector<void*> kpools, vpools;
  int32_t* d_page_table = nullptr;
  int32_t* d_ctx_lens = nullptr;
  float* d_logits = nullptr;
  uint32_t epoch = 0;
  uint32_t watchdog_ticks = 200000000u;  // 2 s at 100 MHz
  TraceRec* d_trace = nullptr;
};

namespace {
thread_local std::string g_err;

mk_status fail(mk_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

#define HIPCHK(x)                                                                          \
  do {                                                                                     \
    hipError_t e_ = (x);                                                                   \
    if (e_ != hipSuccess) return fail(MK_ERR_HIP, std::string(#x) + ": " + hipGetErrorString(e_)); \
  } while (0)

// Makes the context's device current for the duration of a call, then restores the caller's.
struct DeviceGuard {
  int old = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (dev < 0) return;
    if (hipGetDevice(&old) != hipSuccess) old = -1;
    ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    if (old >= 0) (void)hipSetDevice(old);
  }
};

mk_status build(const mk_model_config* cfg, int n_cus, mk_ctx** out) {
  if (!cfg || !out) return fail(MK_ERR_INVALID_ARG, "null argument");
  *out = nullptr;
  mk_ctx* c = new mk_ctx();
  const std::string why = build_graph(*cfg, n_cus, c->g);
  if (!why.empty()) {
    delete c;
    return fail(MK_ERR_SHAPE, why);
  }
  if (const char* w = std::getenv("MK_WATCHDOG_US")) {  // wait budget in microseconds (100 ticks each)
    const long us = std::atol(w);
    if (us > 0 && us < 40000000L) c->watchdog_ticks = (uint32_t)(us * 100L);
  }
  *out = c;
  return MK_OK;
}

void rope_table(const mk_model_config& c, int max_pos, std::vector<float>& out) {
  const int half = c.head_dim / 2;
  out.resize((size_t)max_pos * half * 2);
  for (int p = 0; p < max_pos; ++p)
    for (int i = 0; i < half; ++i) {
      const double a = (double)p * std::pow((double)c.rope_theta, -2.0 * i / c.head_dim);
      out[((size_t)p * half + i) * 2 + 0] = (float)std::cos(a);
      out[((size_t)p * half + i) * 2 + 1] = (float)std::sin(a);
    }
}

mk_status read_error_word(mk_ctx* c, hipStream_t st) {
  uint32_t e[4] = {0, 0, 0, 0};
  HIPCHK(hipStreamSynchronize(st));
  HIPCHK(hipMemcpy(e, c->d_scratch + c->g.sl.err, sizeof(e), hipMemcpyDeviceToHost));
  if (e[E_CODE] == ERR_NONE) return MK_OK;
  // clear the word; after a timeout the flags are inconsistent, so reset them too
  HIPCHK(hipMemset(c->d_scratch + c->g.sl.err, 0, E_COUNT * 4));
  std::string what;
  mk_status s = MK_ERR_DEVICE_FAULT;
  if (e[E_CODE] == ERR_TOKEN) what = "token id out of range (seq " + std::to_string(e[1]) + ", token " + std::to_string((int32_t)e[2]) + ")";
  else if (e[E_CODE] == ERR_PAGE) what = "page table entry out of range (seq " + std::to_string(e[1]) + ", block " + std::to_string((int32_t)e[2]) + ")";
  else if (e[E_CODE] == ERR_CTX) what = "context length outside the cache (seq " + std::to_string(e[1]) + ", length " + std::to_string((int32_t)e[2]) + ")";
  else {
    what = "device wait exceeded the watchdog (event " + std::to_string(e[1]) + ", epoch " + std::to_string(e[2]) + ")";
    s = MK_ERR_DEVICE_TIMEOUT;
  }
  if (e[E_ABORT] || s == MK_ERR_DEVICE_TIMEOUT) {
    HIPCHK(hipMemset(c->d_scratch + c->g.sl.flags, 0, (size_t)c->g.n_flag_slots * 4));
    // epochs restart at 1, so tags of the aborted steps must not survive
    HIPCHK(hipMemset(c->d_scratch + c->g.sl.tagged_begin, 0, (size_t)(c->g.sl.tagged_end - c->g.sl.tagged_begin)));
    HIPCHK(hipDeviceSynchronize());
    c->epoch = 0;
  }
  return fail(s, what);
}

KernelParams make_params(mk_ctx* c) {
  const HostGraph& g = c->g;
  const mk_model_config& m = g.cfg;
  uint8_t* S = c->d_scratch;
  KernelParams p{};
  p.tasks = (const TaskDesc*)(S + g.sl.tasks);
  p.queue_off = (const int32_t*)(S + g.sl.queue_off);
  p.queue_idx = (const int32_t*)(S + g.sl.queue_idx);
  p.events = (const EventDesc*)(S + g.sl.events);
  p.sig_slots = (const int32_t*)(S + g.sl.sig_slots);
  p.geoms = (const GemvGeom*)(S + g.sl.geoms);
  p.rope = (const float*)(S + g.sl.rope);
  p.flags = (uint32_t*)(S + g.sl.flags);
  p.err = (uint32_t*)(S + g.sl.err);
  p.wpacked = c->d_weights;
  p.embed = (const uint16_t*)(c->d_weights + g.wl.embed);
  p.norms = (const uint16_t*)(c->d_weights + g.wl.norms);
  p.bias = m.qkv_bias ? (const uint16_t*)(c->d_weights + g.wl.bias) : nullptr;
  p.kpool = (uint16_t* const*)(S + g.sl.pools);
  p.vpool = (uint16_t* const*)(S + g.sl.pools + (size_t)m.n_layers * 8);
  p.page_table = c->d_page_table;
  p.ctx_lens = c->d_ctx_lens;
  p.xt = (uint64_t*)(S + g.sl.xt);
  p.qt = (uint64_t*)(S + g.sl.qt);
  p.kvt = (uint64_t*)(S + g.sl.kvt);
  p.ot = (uint64_t*)(S + g.sl.ot);
  p.ht = (uint64_t*)(S + g.sl.ht);
  p.pt = (uint64_t*)(S + g.sl.pt);
  p.bpt = (uint64_t*)(S + g.sl.bpt);
  p.logits = c->d_logits;
  p.amax = (uint64_t*)(S + g.sl.amax);
  p.n_layers = m.n_layers;
  p.d = m.d_model;
  p.hq = m.n_q_heads;
  p.hk = m.n_kv_heads;
  p.dh = m.head_dim;
  p.f = m.d_ffn;
  p.vocab = m.vocab;
  p.eps = m.rms_eps;
  p.max_seqs = m.max_seqs;
  p.max_blocks = m.max_blocks_per_seq;
  p.num_blocks = m.num_blocks;
  p.block_size = m.block_size;
  p.splits = g.splits;
  p.n_lm_parts = g.n_lm_parts;
  p.max_pos = g.max_pos;
  p.watchdog_ticks = c->watchdog_ticks;
  p.max_queue = g.max_queue;
  p.attn_tasks = g.attn_tasks;
  p.attn_min_blocks = g.cfg.attn_min_blocks > 0 ? g.cfg.attn_min_blocks : kAttnMinBlocks;
  p.trace = c->d_trace;
  return p;
}

// One decode step: one launch over the whole task graph, or (staged) one launch per dependency
// stage, in order, each running only that stage's tasks with the same kernel and step epoch.
mk_status launch_step(mk_ctx* c, const int32_t* tin, int n_active, int32_t* tout, hipStream_t st, bool staged = false) {
  KernelParams p = make_params(c);
  p.tokens_in = tin;
  p.tokens_out = tout;
  p.n_active = n_active;
  p.epoch = ++c->epoch;
  if (!staged) {
    p.task_lo = 0;
    p.task_hi = (int32_t)c->g.tasks.size();
    HIPCHK(launch_megakernel(p, c->g.n_cus, (size_t)c->g.lds_bytes, st));
    return MK_OK;
  }
  const auto& t = c->g.tasks;
  for (size_t a = 0; a < t.size();) {
    size_t b = a + 1;
    while (b < t.size() && t[b].type == t[a].type && t[b].layer == t[a].layer) ++b;
    p.task_lo = (int32_t)a;
    p.task_hi = (int32_t)b;
    HIPCHK(launch_megakernel(p, c->g.n_cus, (size_t)c->g.lds_bytes, st));
    a = b;
  }
  return MK_OK;
}
}  // namespace

extern "C" {

mk_status mk_create(const mk_model_config* cfg, int device, mk_ctx** out) {
  if (!cfg || !out) return fail(MK_ERR_INVALID_ARG, "null argument");
  int ndev = 0;
  HIPCHK(hipGetDeviceCount(&ndev));
  if (device < 0 || device >= ndev) return fail(MK_ERR_INVALID_ARG, "no such device");
  hipDeviceProp_t prop;
  HIPCHK(hipGetDeviceProperties(&prop, device));
  int coop = 0;
  HIPCHK(hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, device));
  if (!coop) return fail(MK_ERR_UNSUPPORTED, "device does not support cooperative launch");
  mk_status s = build(cfg, prop.multiProcessorCount, out);
  if (s != MK_OK) return s;
  (*out)->device = device;
  DeviceGuard dg(device);
  int blocks = 0;
  if (megakernel_occupancy(&blocks, (size_t)(*out)->g.lds_bytes, cfg->head_dim, cfg->n_q_heads, cfg->n_kv_heads,
                           cfg->max_seqs > 1) !=
          hipSuccess ||
      blocks < 1) {
    mk_destroy(*out);
    *out = nullptr;
    return fail(MK_ERR_UNSUPPORTED, "one workgroup per CU does not fit (LDS or registers)");
  }
  return MK_OK;
}

mk_status mk_create_host(const mk_model_config* cfg, int n_cus, mk_ctx** out) { return build(cfg, n_cus, out); }

mk_status mk_workspace_size(const mk_ctx* c, size_t* wb, size_t* kvb, size_t* sb) {
  if (!c) return fail(MK_ERR_INVALID_ARG, "null context");
  const mk_model_config& m = c->g.cfg;
  if (wb) *wb = (size_t)c->g.wl.total;
  if (kvb) *kvb = (size_t)m.num_blocks * m.n_kv_heads * m.block_size * m.head_dim * 2;
  if (sb) *sb = (size_t)c->g.sl.total;
  return MK_OK;
}

mk_status mk_bind_memory(mk_ctx* c, void* d_weights, void* const* d_k_pools, void* const* d_v_pools, void* d_scratch,
                         int32_t* d_page_table, int32_t* d_ctx_lens, float* d_logits) {
  if (!c) return fail(MK_ERR_INVALID_ARG, "null context");
  if (c->device < 0) return fail(MK_ERR_STATE, "host-only context");
  if (!d_weights || !d_k_pools || !d_v_pools || !d_scratch || !d_page_table || !d_ctx_lens || !d_logits)
    return fail(MK_ERR_INVALID_ARG, "null pointer");
  const int L = c->g.cfg.n_layers;
  for (int l = 0; l < L; ++l)
    if (!d_k_pools[l] || !d_v_pools[l]) return fail(MK_ERR_INVALID_ARG, "null KV pool pointer");
  auto misaligned = [](const void* p) { return ((uintptr_t)p & 255) != 0; };
  if (misaligned(d_weights) || misaligned(d_scratch)) return fail(MK_ERR_INVALID_ARG, "buffers must be 256-byte aligned");
  DeviceGuard dg(c->device);
  if (!dg.ok) return fail(MK_ERR_HIP, "hipSetDevice failed");
  const HostGraph& g = c->g;
  c->d_weights = (uint8_t*)d_weights;
  c->d_scratch = (uint8_t*)d_scratch;
  c->kpools.assign(d_k_pools, d_k_pools + L);
  c->vpools.assign(d_v_pools, d_v_pools + L);
  c->d_page_table = d_page_table;
  c->d_ctx_lens = d_ctx_lens;
  c->d_logits = d_logits;
  uint8_t* S = c->d_scratch;
  auto up = [&](int64_t off, const void* src, size_t n) { return hipMemcpy(S + off, src, n, hipMemcpyHostToDevice); };
  HIPCHK(up(g.sl.tasks, g.tasks.data(), g.tasks.size() * sizeof(TaskDesc)));
  HIPCHK(up(g.sl.queue_off, g.queue_off.data(), g.queue_off.size() * 4));
  HIPCHK(up(g.sl.queue_idx, g.queue_idx.data(), g.queue_idx.size() * 4));
  HIPCHK(up(g.sl.events, g.events.data(), g.events.size() * sizeof(EventDesc)));
  if (!g.sig_slots.empty()) HIPCHK(up(g.sl.sig_slots, g.sig_slots.data(), g.sig_slots.size() * 4));
  HIPCHK(up(g.sl.geoms, g.geoms, sizeof(g.geoms)));
  std::vector<float> rope;
  rope_table(g.cfg, g.max_pos, rope);
  HIPCHK(up(g.sl.rope, rope.data(), rope.size() * 4));
  std::vector<void*> pools(c->kpools);
  pools.insert(pools.end(), c->vpools.begin(), c->vpools.end());
  HIPCHK(up(g.sl.pools, pools.data(), pools.size() * 8));
  HIPCHK(hipMemset(S + g.sl.flags, 0, (size_t)g.n_flag_slots * 4));
  HIPCHK(hipMemset(S + g.sl.err, 0, E_COUNT * 4));
  HIPCHK(hipMemset(S + g.sl.tagged_begin, 0, (size_t)(g.sl.tagged_end - g.sl.tagged_begin)));
  HIPCHK(hipDeviceSynchronize());
  c->epoch = 0;
  c->bound = true;
  c->loaded = false;
  return MK_OK;
}

mk_status mk_load_weights(mk_ctx* c, const mk_tensor* ts, int n, void* stream) {
  if (!c || (!ts && n > 0) || n < 0) return fail(MK_ERR_INVALID_ARG, "null argument");
  if (!c->bound) return fail(MK_ERR_STATE, "bind memory before loading weights");
  const HostGraph& g = c->g;
  const mk_model_config& m = g.cfg;
  const int L = m.n_layers, d = m.d_model, hq = m.n_q_heads, hk = m.n_kv_heads, dh = m.head_dim, f = m.d_ffn,
            V = m.vocab;
  std::map<std::string, int64_t> want;
  want["embed"] = (int64_t)V * d;
  want["final_norm"] = d;
  if (!m.tied_embeddings) want["lm_head"] = (int64_t)V * d;
  for (int l = 0; l < L; ++l) {
    const std::string p = "layers." + std::to_string(l) + ".";
    want[p + "attn_norm"] = d;
    want[p + "wq"] = (int64_t)hq * dh * d;
    want[p + "wk"] = (int64_t)hk * dh * d;
    want[p + "wv"] = (int64_t)hk * dh * d;
    if (m.qkv_bias) {
      want[p + "bq"] = (int64_t)hq * dh;
      want[p + "bk"] = (int64_t)hk * dh;
      want[p + "bv"] = (int64_t)hk * dh;
    }
    want[p + "wo"] = (int64_t)d * hq * dh;
    want[p + "ffn_norm"] = d;
    want[p + "wg"] = (int64_t)f * d;
    want[p + "wu"] = (int64_t)f * d;
    want[p + "wd"] = (int64_t)d * f;
  }
  std::map<std::string, const uint16_t*> have;
  for (int i = 0; i < n; ++i) {
    if (!ts[i].name || !ts[i].ptr) return fail(MK_ERR_INVALID_ARG, "tensor with null name or pointer");
    auto it = want.find(ts[i].name);
    if (it == want.end()) return fail(MK_ERR_INVALID_ARG, std::string("unknown tensor ") + ts[i].name);
    if (have.count(ts[i].name)) return fail(MK_ERR_INVALID_ARG, std::string("duplicate tensor ") + ts[i].name);
    if (ts[i].numel != it->second)
      return fail(MK_ERR_SHAPE, std::string("tensor ") + ts[i].name + " has " + std::to_string(ts[i].numel) +
                                    " elements, expected " + std::to_string(it->second));
    if (((uintptr_t)ts[i].ptr & 15) != 0) return fail(MK_ERR_INVALID_ARG, std::string("tensor ") + ts[i].name + " is not 16-byte aligned");
    have[ts[i].name] = (const uint16_t*)ts[i].ptr;
  }
  for (auto& w : want)
    if (!have.count(w.first)) return fail(MK_ERR_INVALID_ARG, "missing tensor " + w.first);
  DeviceGuard dg(c->device);
  hipStream_t st = (hipStream_t)stream;
  const TaskDesc* dtasks = (const TaskDesc*)(c->d_scratch + g.sl.tasks);
  // re-lay out each GEMV stage (its tasks are contiguous in the task array)
  const int nt = (int)g.tasks.size();
  for (int t0 = 0; t0 < nt;) {
    const TaskDesc& a = g.tasks[t0];
    int t1 = t0 + 1;
    while (t1 < nt && g.tasks[t1].type == a.type && g.tasks[t1].layer == a.layer) ++t1;
    if (a.type == T_ATTN || a.type == T_ARGMAX) {
      t0 = t1;
      continue;
    }
    RepackArgs r{};
    r.tasks = dtasks;
    r.task0 = t0;
    r.ntasks = t1 - t0;
    r.gm = g.geoms[a.geom];
    r.G = hq / hk;
    r.dh = dh;
    r.out = c->d_weights;
    const std::string p = "layers." + std::to_string(a.layer) + ".";
    switch (a.type) {
      case T_QKV: r.kind = RK_QKV; r.w0 = have[p + "wq"]; r.w1 = have[p + "wk"]; r.w2 = have[p + "wv"]; break;
      case T_OPROJ: r.kind = RK_PLAIN; r.w0 = have[p + "wo"]; break;
      case T_GATEUP: r.kind = RK_GU; r.w0 = have[p + "wg"]; r.w1 = have[p + "wu"]; break;
      case T_DOWN: r.kind = RK_PLAIN; r.w0 = have[p + "wd"]; break;
      case T_LMHEAD: r.kind = RK_PLAIN; r.w0 = m.tied_embeddings ? have["embed"] : have["lm_head"]; break;
      default: break;
    }
    const TaskDesc& last = g.tasks[t1 - 1];
    const int64_t bytes = last.wofs + task_tile_bytes(r.gm, last) - a.wofs;
    HIPCHK(launch_repack(r, bytes / 1024, st));
    t0 = t1;
  }
  HIPCHK(hipMemcpyAsync(c->d_weights + g.wl.embed, have["embed"], (size_t)V * d * 2, hipMemcpyDeviceToDevice, st));
  uint8_t* norms = c->d_weights + g.wl.norms;
  for (int l = 0; l < L; ++l) {
    const std::string p = "layers." + std::to_string(l) + ".";
    HIPCHK(hipMemcpyAsync(norms + (size_t)(2 * l) * d * 2, have[p + "attn_norm"], (size_t)d * 2, hipMemcpyDeviceToDevice, st));
    HIPCHK(hipMemcpyAsync(norms + (size_t)(2 * l + 1) * d * 2, have[p + "ffn_norm"], (size_t)d * 2, hipMemcpyDeviceToDevice, st));
    if (m.qkv_bias)
      HIPCHK(launch_repack_bias(have[p + "bq"], have[p + "bk"], have[p + "bv"], hq / hk, dh, qkv_rows(m),
                                (uint16_t*)(c->d_weights + g.wl.bias) + (size_t)l * qkv_rows(m), st));
  }
  HIPCHK(hipMemcpyAsync(norms + (size_t)(2 * L) * d * 2, have["final_norm"], (size_t)d * 2, hipMemcpyDeviceToDevice, st));
  c->loaded = true;
  return MK_OK;
}

mk_status mk_decode_step(mk_ctx* c, const int32_t* d_tokens_in, int n_seqs, int32_t* d_tokens_out, void* stream) {
  if (!c || !d_tokens_in || !d_tokens_out) return fail(MK_ERR_INVALID_ARG, "null argument");
  if (!c->bound || !c->loaded) return fail(MK_ERR_STATE, "bind memory and load weights before decoding");
  if (n_seqs < 1 || n_seqs > c->g.cfg.max_seqs) return fail(MK_ERR_INVALID_ARG, "n_seqs out of range");
  DeviceGuard dg(c->device);
  return launch_step(c, d_tokens_in, n_seqs, d_tokens_out, (hipStream_t)stream);
}

mk_status mk_decode_step_staged(mk_ctx* c, const int32_t* d_tokens_in, int n_seqs, int32_t* d_tokens_out, void* stream) {
  if (!c || !d_tokens_in || !d_tokens_out) return fail(MK_ERR_INVALID_ARG, "null argument");
  if (!c->bound || !c->loaded) return fail(MK_ERR_STATE, "bind memory and load weights before decoding");
  if (n_seqs < 1 || n_seqs > c->g.cfg.max_seqs) return fail(MK_ERR_INVALID_ARG, "n_seqs out of range");
  DeviceGuard dg(c->device);
  return launch_step(c, d_tokens_in, n_seqs, d_tokens_out, (hipStream_t)stream, true);
}

mk_status mk_prefill(mk_ctx* c, int seq, const int32_t* h_tokens, int n_tokens, int32_t* d_token_out, void* stream) {
  if (!c || (!h_tokens && n_tokens > 0) || n_tokens < 0) return fail(MK_ERR_INVALID_ARG, "null argument");
  if (!c->bound || !c->loaded) return fail(MK_ERR_STATE, "bind memory and load weights before prefill");
  if (c->g.cfg.max_seqs != 1 || seq != 0) return fail(MK_ERR_UNSUPPORTED, "prefill runs batch-1 contexts, sequence 0");
  if (n_tokens == 0) return MK_OK;
  if (n_tokens > c->g.max_pos) return fail(MK_ERR_INVALID_ARG, "prompt longer than the cache");
  for (int i = 0; i < n_tokens; ++i)
    if (h_tokens[i] < 0 || h_tokens[i] >= c->g.cfg.vocab) return fail(MK_ERR_INVALID_ARG, "prompt token out of range");
  DeviceGuard dg(c->device);
  hipStream_t st = (hipStream_t)stream;
  int32_t* tokbuf = (int32_t*)(c->d_scratch + c->g.sl.tokbuf);
  int32_t* tokout = (int32_t*)(c->d_scratch + c->g.sl.tokout);
  HIPCHK(hipMemcpyAsync(tokbuf, h_tokens, (size_t)n_tokens * 4, hipMemcpyHostToDevice, st));
  HIPCHK(hipStreamSynchronize(st));  // the host array may be released when this call returns
  for (int i = 0; i < n_tokens; ++i) {
    int32_t* out = (i == n_tokens - 1 && d_token_out) ? d_token_out : tokout;
    mk_status s = launch_step(c, tokbuf + i, 1, out, st);
    if (s != MK_OK) return s;
  }
  return MK_OK;
}

mk_status mk_read_logits(mk_ctx* c, int seq, float* h_dst, size_t n, void* stream) {
  if (!c || !h_dst) return fail(MK_ERR_INVALID_ARG, "null argument");
  if (!c->bound) return fail(MK_ERR_STATE, "memory not bound");
  if (seq < 0 || seq >= c->g.cfg.max_seqs || n > (size_t)c->g.cfg.vocab) return fail(MK_ERR_INVALID_ARG, "seq or n out of range");
  DeviceGuard dg(c->device);
  hipStream_t st = (hipStream_t)stream;
  HIPCHK(hipMemcpyAsync(h_dst, c->d_logits + (size_t)seq * c->g.cfg.vocab, n * 4, hipMemcpyDeviceToHost, st));
  return read_error_word(c, st);
}

mk_status mk_sync_check(mk_ctx* c, void* stream) {
  if (!c) return fail(MK_ERR_INVALID_ARG, "null context");
  if (!c->bound) return fail(MK_ERR_STATE, "memory not bound");
  DeviceGuard dg(c->device);
  return read_error_word(c, (hipStream_t)stream);
}

mk_status mk_set_trace(mk_ctx* c, void* d_buf, size_t bytes) {
  if (!c) return fail(MK_ERR_INVALID_ARG, "null context");
  if (!d_buf) {
    c->d_trace = nullptr;
    return MK_OK;
  }
  if (bytes < c->g.tasks.size() * sizeof(TraceRec)) return fail(MK_ERR_INVALID_ARG, "trace buffer too small");
  if (((uintptr_t)d_buf & 7) != 0) return fail(MK_ERR_INVALID_ARG, "trace buffer must be 8-byte aligned");
  c->d_trace = (TraceRec*)d_buf;
  return MK_OK;
}

mk_status mk_graph_stats(const mk_ctx* c, mk_graph_info* out) {
  if (!c || !out) return fail(MK_ERR_INVALID_ARG, "null argument");
  const HostGraph& g = c->g;
  out->n_tasks = (int64_t)g.tasks.size();
  out->n_events = (int64_t)g.events.size();
  out->n_flag_slots = g.n_flag_slots;
  out->n_attn_groups = g.n_attn_groups;
  int64_t mq = 0;
  for (int i = 0; i < g.n_cus; ++i) mq = std::max<int64_t>(mq, g.queue_off[i + 1] - g.queue_off[i]);
  out->max_queue_len = mq;
  out->weight_bytes = g.wl.packed_bytes;
  out->lds_bytes = g.lds_bytes;
  out->hash = graph_hash(g);
  int64_t stages = 0;
  for (size_t a = 0; a < g.tasks.size(); ++a)
    if (a == 0 || g.tasks[a].type != g.tasks[a - 1].type || g.tasks[a].layer != g.tasks[a - 1].layer) ++stages;
  out->n_stages = stages;
  return MK_OK;
}

mk_status mk_graph_validate(const mk_ctx* c) {
  if (!c) return fail(MK_ERR_INVALID_ARG, "null context");
  const std::string why = validate_graph(c->g);
  return why.empty() ? MK_OK : fail(MK_ERR_SHAPE, why);
}

mk_status mk_graph_simulate(const mk_ctx* c, uint64_t seed, int n_steps) {
  if (!c || n_steps < 0) return fail(MK_ERR_INVALID_ARG, "bad argument");
  const std::string why = simulate_graph(c->g, seed, n_steps);
  return why.empty() ? MK_OK : fail(MK_ERR_SHAPE, why);
}

void mk_destroy(mk_ctx* c) { delete c; }

const char* mk_status_str(mk_status s) {
  switch (s) {
    case MK_OK: return "MK_OK";
    case MK_ERR_INVALID_ARG: return "MK_ERR_INVALID_ARG";
    case MK_ERR_SHAPE: return "MK_ERR_SHAPE";
    case MK_ERR_STATE: return "MK_ERR_STATE";
    case MK_ERR_HIP: return "MK_ERR_HIP";
    case MK_ERR_DEVICE_TIMEOUT: return "MK_ERR_DEVICE_TIMEOUT";
    case MK_ERR_DEVICE_FAULT: return "MK_ERR_DEVICE_FAULT";
    case MK_ERR_UNSUPPORTED: return "MK_ERR_UNSUPPORTED";
    default: return "unknown status";
  }
}

const char* mk_last_error(void) { return g_err.c_str(); }

}  // extern "C"
