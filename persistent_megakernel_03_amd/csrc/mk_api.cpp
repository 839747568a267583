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
#include <memory>
#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_host.h"

namespace mk {
hipError_t launch_megakernel(const KernelParams& p, int grid, size_t lds_bytes, hipStream_t stream, bool coop);
hipError_t megakernel_occupancy(int* blocks_per_cu, size_t lds_bytes, int dh, int hq, int hk, bool batched, bool fp8);
hipError_t launch_repack(const RepackArgs& a, int64_t units, hipStream_t stream);
hipError_t launch_row_scales(const RepackArgs& a, int nrows, hipStream_t stream);
hipError_t launch_repack_fp8(const RepackArgs& a, int64_t units, hipStream_t stream);
hipError_t launch_jit_reset(int32_t* w, int n_events, int n_tasks, int n0, hipStream_t stream);
hipError_t launch_repack_bias(const uint16_t* bq, const uint16_t* bk, const uint16_t* bv, int G, int dh, int nrows,
                              uint16_t* out, hipStream_t stream);
hipError_t static_scratch_address(int device, void** out);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);
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
  uint8_t* d_static = nullptr;     // this device's static scratch array (mk_decode_step_static)
  std::vector<float> rope_host;    // the rotary table and the per-layer pool pointers, as uploaded at bind
  std::vector<void*> pool_table;
  // One-sequence contexts with prefill_rows > 1: the batched graph the prompt runs through, with its
  // re-laid-out weights and its working memory at these offsets in the bound weights and scratch buffers.
  std::unique_ptr<HostGraph> pg;
  int64_t pg_w = 0, pg_s = 0;
  uint32_t pg_epoch = 0;
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

int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

mk_status build(const mk_model_config* cfg, int n_cus, mk_ctx** out) {
  if (!cfg || !out) return fail(MK_ERR_INVALID_ARG, "null argument");
  *out = nullptr;
  mk_ctx* c = new mk_ctx();
  const std::string why = build_graph(*cfg, n_cus, c->g);
  if (!why.empty()) {
    delete c;
    return fail(MK_ERR_SHAPE, why);
  }
  if (cfg->max_seqs == 1 && cfg->prefill_rows > 1) {
    mk_model_config pc = *cfg;
    pc.max_seqs = cfg->prefill_rows;
    pc.prefill_rows = 0;
    c->pg.reset(new HostGraph());
    const std::string pwhy = build_graph(pc, n_cus, *c->pg);
    if (!pwhy.empty()) {
      delete c;
      return fail(MK_ERR_SHAPE, "prefill graph: " + pwhy);
    }
    c->pg_w = align256(c->g.wl.total);
    c->pg_s = align256(c->g.sl.total);
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

// Clears a graph's event flags and tagged buffers (synchronous memsets, outside any step).
hipError_t clear_working(const HostGraph& g, uint8_t* S) {
  hipError_t e = hipMemset(S + g.sl.flags, 0, (size_t)g.n_flag_slots * 4);
  if (e != hipSuccess) return e;
  return hipMemset(S + g.sl.tagged_begin, 0, (size_t)(g.sl.tagged_end - g.sl.tagged_begin));
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
  else if (e[E_CODE] == ERR_NAN) what = "NaN among the logits (seq " + std::to_string(e[1]) + ", first at index " + std::to_string((int32_t)e[2]) + ")";
  else {
    const std::string ev = e[1] == 0xFFFFFFFEu ? std::string("the next step's token") : "event " + std::to_string(e[1]);
    what = "device wait exceeded the watchdog (" + ev + ", epoch " + std::to_string(e[2]) + ")";
    s = MK_ERR_DEVICE_TIMEOUT;
  }
  if (e[E_ABORT] || s == MK_ERR_DEVICE_TIMEOUT) {
    HIPCHK(clear_working(c->g, c->d_scratch));  // epochs restart at 1: no tag of the aborted steps survives
    c->epoch = 0;
    if (c->pg) {
      HIPCHK(clear_working(*c->pg, c->d_scratch + c->pg_s));
      c->pg_epoch = 0;
    }
    HIPCHK(hipDeviceSynchronize());
  }
  return fail(s, what);
}

// Kernel arguments of graph g. Its read-only tables (task graph, rotary table, pool pointers) come from
// its region R of the bound scratch buffer, the working memory a step writes (flags, tagged activations,
// partials, argmax keys) from the region at W (R itself, or the static array), its re-laid-out weights
// from Wt. Errors always go to the context's own error word.
KernelParams make_params(mk_ctx* c, const HostGraph& g, uint8_t* R, uint8_t* W, uint8_t* Wt) {
  const mk_model_config& m = g.cfg;
  KernelParams p{};
  p.tasks = (const TaskDesc*)(R + g.sl.tasks);
  p.queue_off = (const int32_t*)(R + g.sl.queue_off);
  p.queue_idx = (const int32_t*)(R + g.sl.queue_idx);
  p.events = (const EventDesc*)(R + g.sl.events);
  p.sig_slots = (const int32_t*)(R + g.sl.sig_slots);
  p.geoms = (const GemvGeom*)(R + g.sl.geoms);
  p.rope = (const float*)(R + g.sl.rope);
  p.err = (uint32_t*)(c->d_scratch + c->g.sl.err);
  uint8_t* S = W;
  p.flags = (uint32_t*)(S + g.sl.flags);
  p.wpacked = Wt;
  p.embed = (const uint16_t*)(Wt + g.wl.embed);
  p.norms = (const uint16_t*)(Wt + g.wl.norms);
  p.bias = m.qkv_bias ? (const uint16_t*)(Wt + g.wl.bias) : nullptr;
  p.kpool = (uint16_t* const*)(R + g.sl.pools);
  p.vpool = (uint16_t* const*)(R + g.sl.pools + (size_t)m.n_layers * 8);
  p.page_table = c->d_page_table;
  p.ctx_lens = c->d_ctx_lens;
  p.xt = (uint64_t*)(S + g.sl.xt);
  p.qt = (uint64_t*)(S + g.sl.qt);
  p.kvt = (uint64_t*)(S + g.sl.kvt);
  p.ot = (uint64_t*)(S + g.sl.ot);
  p.ht = (uint64_t*)(S + g.sl.ht);
  p.pt = (uint64_t*)(S + g.sl.pt);
  p.bpt = (uint64_t*)(S + g.sl.bpt);
  p.tokt = (uint64_t*)(S + g.sl.tokt);
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
  p.trace = &g == &c->g ? c->d_trace : nullptr;
  p.fp8_weights = m.weight_format == MK_WEIGHTS_FP8_E4M3 ? 1 : 0;
  p.stage2_off = (int32_t)g.stage2_off;
  p.wscale = p.fp8_weights ? (const float*)(Wt + g.wl.scales) : nullptr;
  return p;
}

KernelParams make_params(mk_ctx* c, uint8_t* W) { return make_params(c, c->g, c->d_scratch, W, c->d_weights); }

// Epochs grow by one per step. Long before the 32-bit tags could wrap (a tag of epoch 0 or 1 would pass
// the checks of a restarted count), the flags and tagged buffers are cleared and epochs restart at 1.
constexpr uint32_t kEpochLimit = 0x40000000u;
// Steps one mk_decode_n launch may run (each step's tokens go to its own row of the output array).
constexpr int kMaxStepsPerLaunch = 1 << 16;

mk_status reserve_epochs(const HostGraph& g, uint8_t* S, uint32_t& epoch, int n_steps, hipStream_t st) {
  if (epoch + (uint32_t)n_steps + 1u < kEpochLimit) return MK_OK;
  HIPCHK(hipStreamSynchronize(st));
  HIPCHK(clear_working(g, S));
  HIPCHK(hipDeviceSynchronize());
  epoch = 0;
  return MK_OK;
}

// Decode steps: one launch over the whole task graph for n_steps steps (each feeding its tokens to the
// next; cooperative when n_steps > 1), or (staged, one step) one launch per dependency stage, in order,
// each running only that stage's tasks with the same kernel and step epoch.
mk_status launch_step(mk_ctx* c, const int32_t* tin, int n_active, int32_t* tout, hipStream_t st, bool staged = false,
                      int n_steps = 1) {
  if (mk_status s = reserve_epochs(c->g, c->d_scratch, c->epoch, n_steps, st)) return s;
  KernelParams p = make_params(c, c->d_scratch);
  p.tokens_in = tin;
  p.tokens_out = tout;
  p.n_active = n_active;
  p.n_steps = n_steps;
  p.epoch = c->epoch + 1;
  c->epoch += (uint32_t)n_steps;
  if (!staged) {
    p.task_lo = 0;
    p.task_hi = (int32_t)c->g.tasks.size();
    HIPCHK(launch_megakernel(p, c->g.n_cus, (size_t)c->g.lds_bytes, st, n_steps > 1));
    return MK_OK;
  }
  const auto& t = c->g.tasks;
  for (size_t a = 0; a < t.size();) {
    size_t b = a + 1;
    while (b < t.size() && t[b].type == t[a].type && t[b].layer == t[a].layer) ++b;
    p.task_lo = (int32_t)a;
    p.task_hi = (int32_t)b;
    HIPCHK(launch_megakernel(p, c->g.n_cus, (size_t)c->g.lds_bytes, st, false));
    a = b;
  }
  return MK_OK;
}
// Re-lays out the weights for graph g (its task table at R on the device) into the weights region Wt:
// every GEMV stage's tiles in the graph's order, then the embedding, norm gains and bias copies.
mk_status load_graph_weights(const HostGraph& g, uint8_t* R, uint8_t* Wt,
                             const std::map<std::string, const uint16_t*>& have, hipStream_t st) {
  const mk_model_config& m = g.cfg;
  const int L = m.n_layers, d = m.d_model, hq = m.n_q_heads, hk = m.n_kv_heads, V = m.vocab, dh = m.head_dim;
  const TaskDesc* dtasks = (const TaskDesc*)(R + g.sl.tasks);
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
    r.out = Wt;
    const std::string p = "layers." + std::to_string(a.layer) + ".";
    switch (a.type) {
      case T_QKV: r.kind = RK_QKV; r.w0 = have.at(p + "wq"); r.w1 = have.at(p + "wk"); r.w2 = have.at(p + "wv"); break;
      case T_OPROJ: r.kind = RK_PLAIN; r.w0 = have.at(p + "wo"); break;
      case T_GATEUP: r.kind = RK_GU; r.w0 = have.at(p + "wg"); r.w1 = have.at(p + "wu"); break;
      case T_DOWN: r.kind = RK_PLAIN; r.w0 = have.at(p + "wd"); break;
      case T_LMHEAD: r.kind = RK_PLAIN; r.w0 = m.tied_embeddings ? have.at("embed") : have.at("lm_head"); break;
      default: break;
    }
    const TaskDesc& last = g.tasks[t1 - 1];
    const int64_t bytes = last.wofs + task_tile_bytes(r.gm, last) - a.wofs;
    if (r.gm.fp8) {  // the rows' scales first, then the codes (the stage's first task starts at row 0)
      r.scales = (float*)(Wt + g.wl.scales);
      r.scale0 = a.a1;
      HIPCHK(launch_row_scales(r, last.row1, st));
      HIPCHK(launch_repack_fp8(r, bytes / 1024, st));
    } else {
      HIPCHK(launch_repack(r, bytes / 1024, st));
    }
    t0 = t1;
  }
  HIPCHK(hipMemcpyAsync(Wt + g.wl.embed, have.at("embed"), (size_t)V * d * 2, hipMemcpyDeviceToDevice, st));
  uint8_t* norms = Wt + g.wl.norms;
  for (int l = 0; l < L; ++l) {
    const std::string p = "layers." + std::to_string(l) + ".";
    HIPCHK(hipMemcpyAsync(norms + (size_t)(2 * l) * d * 2, have.at(p + "attn_norm"), (size_t)d * 2, hipMemcpyDeviceToDevice, st));
    HIPCHK(hipMemcpyAsync(norms + (size_t)(2 * l + 1) * d * 2, have.at(p + "ffn_norm"), (size_t)d * 2, hipMemcpyDeviceToDevice, st));
    if (m.qkv_bias)
      HIPCHK(launch_repack_bias(have.at(p + "bq"), have.at(p + "bk"), have.at(p + "bv"), hq / hk, dh, qkv_rows(m),
                                (uint16_t*)(Wt + g.wl.bias) + (size_t)l * qkv_rows(m), st));
  }
  HIPCHK(hipMemcpyAsync(norms + (size_t)(2 * L) * d * 2, have.at("final_norm"), (size_t)d * 2, hipMemcpyDeviceToDevice, st));
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
                           cfg->max_seqs > 1, cfg->weight_format == MK_WEIGHTS_FP8_E4M3) !=
          hipSuccess ||
      blocks < 1) {
    mk_destroy(*out);
    *out = nullptr;
    return fail(MK_ERR_UNSUPPORTED, "one workgroup per CU does not fit (LDS or registers)");
  }
  if ((*out)->pg && (megakernel_occupancy(&blocks, (size_t)(*out)->pg->lds_bytes, cfg->head_dim, cfg->n_q_heads,
                                          cfg->n_kv_heads, true, false) != hipSuccess ||
                     blocks < 1)) {
    mk_destroy(*out);
    *out = nullptr;
    return fail(MK_ERR_UNSUPPORTED, "prefill graph: one workgroup per CU does not fit (LDS or registers)");
  }
  // this device's copy of the static scratch array, resolved once per device at set-up
  void* st = nullptr;
  const hipError_t e = static_scratch_address(device, &st);
  if (e != hipSuccess) {
    mk_destroy(*out);
    *out = nullptr;
    return fail(MK_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
  }
  (*out)->d_static = (uint8_t*)st;
  return MK_OK;
}

mk_status mk_create_host(const mk_model_config* cfg, int n_cus, mk_ctx** out) { return build(cfg, n_cus, out); }

mk_status mk_workspace_size(const mk_ctx* c, size_t* wb, size_t* kvb, size_t* sb) {
  if (!c) return fail(MK_ERR_INVALID_ARG, "null context");
  const mk_model_config& m = c->g.cfg;
  if (wb) *wb = (size_t)(c->pg ? c->pg_w + c->pg->wl.total : c->g.wl.total);
  if (kvb) *kvb = (size_t)m.num_blocks * m.n_kv_heads * m.block_size * m.head_dim * 2;
  if (sb) *sb = (size_t)(c->pg ? c->pg_s + c->pg->sl.total : c->g.sl.total);
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
  rope_table(g.cfg, g.max_pos, c->rope_host);
  c->pool_table = c->kpools;
  c->pool_table.insert(c->pool_table.end(), c->vpools.begin(), c->vpools.end());
  // each graph's read-only tables into its region of the scratch buffer (the prefill graph has the same
  // positions and pools, so the same rotary table and pool pointers)
  auto upload = [&](const HostGraph& h, uint8_t* S) -> hipError_t {
    auto up = [&](int64_t off, const void* src, size_t n) { return hipMemcpy(S + off, src, n, hipMemcpyHostToDevice); };
    hipError_t e;
    if ((e = up(h.sl.tasks, h.tasks.data(), h.tasks.size() * sizeof(TaskDesc))) != hipSuccess) return e;
    if ((e = up(h.sl.queue_off, h.queue_off.data(), h.queue_off.size() * 4)) != hipSuccess) return e;
    if ((e = up(h.sl.queue_idx, h.queue_idx.data(), h.queue_idx.size() * 4)) != hipSuccess) return e;
    if ((e = up(h.sl.events, h.events.data(), h.events.size() * sizeof(EventDesc))) != hipSuccess) return e;
    if (!h.sig_slots.empty() && (e = up(h.sl.sig_slots, h.sig_slots.data(), h.sig_slots.size() * 4)) != hipSuccess)
      return e;
    if ((e = up(h.sl.geoms, h.geoms, sizeof(h.geoms))) != hipSuccess) return e;
    if ((e = up(h.sl.rope, c->rope_host.data(), c->rope_host.size() * 4)) != hipSuccess) return e;
    if ((e = up(h.sl.pools, c->pool_table.data(), c->pool_table.size() * 8)) != hipSuccess) return e;
    {  // dynamic scheduling tables: task -> event, then per event producers, first and end consumer
      std::vector<int32_t> jt(h.jit_task_ev);
      jt.insert(jt.end(), h.jit_ev_n.begin(), h.jit_ev_n.end());
      jt.insert(jt.end(), h.jit_ev_c0.begin(), h.jit_ev_c0.end());
      jt.insert(jt.end(), h.jit_ev_c1.begin(), h.jit_ev_c1.end());
      if (!jt.empty() && (e = up(h.sl.jit_tab, jt.data(), jt.size() * 4)) != hipSuccess) return e;
    }
    if ((e = hipMemset(S + h.sl.err, 0, E_COUNT * 4)) != hipSuccess) return e;
    return clear_working(h, S);
  };
  HIPCHK(upload(g, c->d_scratch));
  if (c->pg) HIPCHK(upload(*c->pg, c->d_scratch + c->pg_s));
  HIPCHK(hipDeviceSynchronize());
  c->epoch = 0;
  c->pg_epoch = 0;
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
  if (mk_status e = load_graph_weights(g, c->d_scratch, c->d_weights, have, st)) return e;
  if (c->pg)
    if (mk_status e = load_graph_weights(*c->pg, c->d_scratch + c->pg_s, c->d_weights + c->pg_w, have, st)) return e;
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

mk_status mk_decode_n(mk_ctx* c, const int32_t* d_tokens_in, int n_seqs, int n_steps, int32_t* d_tokens_out,
                      void* stream) {
  if (!c || !d_tokens_in || !d_tokens_out) return fail(MK_ERR_INVALID_ARG, "null argument");
  if (!c->bound || !c->loaded) return fail(MK_ERR_STATE, "bind memory and load weights before decoding");
  if (n_seqs < 1 || n_seqs > c->g.cfg.max_seqs) return fail(MK_ERR_INVALID_ARG, "n_seqs out of range");
  if (n_steps < 1 || n_steps > kMaxStepsPerLaunch) return fail(MK_ERR_INVALID_ARG, "n_steps out of range");
  DeviceGuard dg(c->device);
  return launch_step(c, d_tokens_in, n_seqs, d_tokens_out, (hipStream_t)stream, false, n_steps);
}

mk_status mk_decode_step_static(mk_ctx* c, const int32_t* d_tokens_in, int n_seqs, int32_t* d_tokens_out, void* stream) {
  if (!c || !d_tokens_in || !d_tokens_out) return fail(MK_ERR_INVALID_ARG, "null argument");
  if (!c->bound || !c->loaded) return fail(MK_ERR_STATE, "bind memory and load weights before decoding");
  if (n_seqs < 1 || n_seqs > c->g.cfg.max_seqs) return fail(MK_ERR_INVALID_ARG, "n_seqs out of range");
  const HostGraph& g = c->g;
  if ((size_t)g.sl.total > kStaticScratchBytes)
    return fail(MK_ERR_SHAPE, "this graph's working memory (" + std::to_string(g.sl.total) +
                                  " bytes) exceeds the static scratch array (" + std::to_string(kStaticScratchBytes) + " bytes)");
  if (!c->d_static) return fail(MK_ERR_STATE, "no static scratch on this device");
  DeviceGuard dg(c->device);
  hipStream_t st = (hipStream_t)stream;
  uint8_t* S = c->d_static;
  // The array keeps whatever the last call on this device left in it: the flags and the tagged buffers
  // are cleared (a fill kernel on the stream), so the step starts from epoch 1. The argmax keys and the
  // partial results are written before they are read within the step.
  HIPCHK(launch_fill_zero(S + g.sl.flags, ((size_t)g.n_flag_slots * 4 + 255) & ~(size_t)255, st));
  HIPCHK(launch_fill_zero(S + g.sl.tagged_begin, (size_t)(g.sl.tagged_end - g.sl.tagged_begin), st));
  KernelParams p = make_params(c, S);
  p.tokens_in = d_tokens_in;
  p.tokens_out = d_tokens_out;
  p.n_active = n_seqs;
  p.n_steps = 1;
  p.epoch = 1;
  p.task_lo = 0;
  p.task_hi = (int32_t)g.tasks.size();
  HIPCHK(launch_megakernel(p, g.n_cus, (size_t)g.lds_bytes, st, false));
  return MK_OK;
}

mk_status mk_decode_step_dynamic(mk_ctx* c, const int32_t* d_tokens_in, int n_seqs, int32_t* d_tokens_out, void* stream) {
  if (!c || !d_tokens_in || !d_tokens_out) return fail(MK_ERR_INVALID_ARG, "null argument");
  if (!c->bound || !c->loaded) return fail(MK_ERR_STATE, "bind memory and load weights before decoding");
  if (n_seqs != 1) return fail(MK_ERR_INVALID_ARG, "n_seqs must be 1");
  const HostGraph& g = c->g;
  if (!g.jit_ok || g.cfg.weight_format != MK_WEIGHTS_BF16)
    return fail(MK_ERR_UNSUPPORTED, "dynamic scheduling runs one-sequence contexts with bf16 weights");
  DeviceGuard dg(c->device);
  hipStream_t st = (hipStream_t)stream;
  if (mk_status s = reserve_epochs(g, c->d_scratch, c->epoch, 1, st)) return s;
  KernelParams p = make_params(c, c->d_scratch);
  p.tokens_in = d_tokens_in;
  p.tokens_out = d_tokens_out;
  p.n_active = 1;
  p.n_steps = 1;
  p.epoch = ++c->epoch;
  p.task_lo = 0;
  p.task_hi = (int32_t)g.tasks.size();
  p.jit_tab = (const int32_t*)(c->d_scratch + g.sl.jit_tab);
  p.jit_work = (int32_t*)(c->d_scratch + g.sl.jit_work);
  p.n_events = (int32_t)g.events.size();
  HIPCHK(launch_jit_reset(p.jit_work, p.n_events, p.task_hi, g.jit_n0, st));
  HIPCHK(launch_megakernel(p, g.n_cus, (size_t)g.lds_bytes, st, false));
  return MK_OK;
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
  const mk_model_config& m = c->g.cfg;
  if (seq < 0 || seq >= m.max_seqs) return fail(MK_ERR_INVALID_ARG, "seq out of range");
  if (n_tokens == 0) return MK_OK;
  if (n_tokens > c->g.max_pos) return fail(MK_ERR_INVALID_ARG, "prompt longer than the cache");
  for (int i = 0; i < n_tokens; ++i)
    if (h_tokens[i] < 0 || h_tokens[i] >= m.vocab) return fail(MK_ERR_INVALID_ARG, "prompt token out of range");
  DeviceGuard dg(c->device);
  hipStream_t st = (hipStream_t)stream;
  if (m.max_seqs == 1 && !c->pg) {  // one decode step per prompt token
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
  // Chunked: steps of the batched graph whose R rows are R consecutive positions of sequence seq. Every
  // row reads seq's page table row (copied R times) and its own context length, so row i appends its
  // key and value at position p0 + i and attends to positions 0 .. p0 + i; the QKV stage (every row's
  // append) completes before any attention task starts, so the earlier rows' entries are in the cache.
  const bool own = !c->pg;
  const HostGraph& g = own ? c->g : *c->pg;
  uint8_t* S = own ? c->d_scratch : c->d_scratch + c->pg_s;
  uint8_t* Wt = own ? c->d_weights : c->d_weights + c->pg_w;
  uint32_t& epoch = own ? c->epoch : c->pg_epoch;
  const int R = g.cfg.max_seqs, MB = m.max_blocks_per_seq, V = m.vocab;
  int32_t p0 = 0;
  HIPCHK(hipStreamSynchronize(st));
  HIPCHK(hipMemcpy(&p0, c->d_ctx_lens + seq, 4, hipMemcpyDeviceToHost));
  if (p0 < 0 || (int64_t)p0 + n_tokens > g.max_pos)
    return fail(MK_ERR_INVALID_ARG, "the prompt runs past the sequence's cache (length " + std::to_string(p0) + ")");
  const int n_chunks = (n_tokens + R - 1) / R;
  if ((int64_t)n_chunks * 16 * 4 > (int64_t)(g.max_pos / R + 2) * 16 * 4) return fail(MK_ERR_SHAPE, "prefill chunk table too small");
  std::vector<int32_t> lens((size_t)n_chunks * 16, 0);
  for (int k = 0; k < n_chunks; ++k)
    for (int i = 0; i < R && k * R + i < n_tokens; ++i) lens[(size_t)k * 16 + i] = p0 + k * R + i;
  int32_t* tokbuf = (int32_t*)(S + g.sl.tokbuf);
  int32_t* ptab = (int32_t*)(S + g.sl.pf_ptab);
  int32_t* ctxs = (int32_t*)(S + g.sl.pf_ctx);
  float* logits = (float*)(S + g.sl.pf_logits);
  int32_t* toks = (int32_t*)(S + g.sl.pf_tok);
  HIPCHK(hipMemcpyAsync(tokbuf, h_tokens, (size_t)n_tokens * 4, hipMemcpyHostToDevice, st));
  HIPCHK(hipMemcpyAsync(ctxs, lens.data(), lens.size() * 4, hipMemcpyHostToDevice, st));
  for (int r = 0; r < R; ++r)
    HIPCHK(hipMemcpyAsync(ptab + (size_t)r * MB, c->d_page_table + (size_t)seq * MB, (size_t)MB * 4,
                          hipMemcpyDeviceToDevice, st));
  HIPCHK(hipStreamSynchronize(st));  // the host arrays may be released when this call returns
  if (mk_status s = reserve_epochs(g, S, epoch, n_chunks, st)) return s;
  for (int k = 0; k < n_chunks; ++k) {
    KernelParams p = make_params(c, g, S, S, Wt);
    p.page_table = ptab;
    p.ctx_lens = ctxs + (size_t)k * 16;
    p.logits = logits;
    p.tokens_in = tokbuf + (size_t)k * R;
    p.tokens_out = toks;
    p.n_active = std::min(R, n_tokens - k * R);
    p.prefill = 1;
    p.n_steps = 1;
    p.epoch = ++epoch;
    p.task_lo = 0;
    p.task_hi = (int32_t)g.tasks.size();
    HIPCHK(launch_megakernel(p, g.n_cus, (size_t)g.lds_bytes, st, false));
  }
  const int last = (n_tokens - 1) % R;
  HIPCHK(hipMemcpyAsync(c->d_logits + (size_t)seq * V, logits + (size_t)last * V, (size_t)V * 4, hipMemcpyDeviceToDevice, st));
  if (d_token_out) HIPCHK(hipMemcpyAsync(d_token_out, toks + last, 4, hipMemcpyDeviceToDevice, st));
  if (mk_status s = read_error_word(c, st)) return s;  // synchronises the stream
  const int32_t len = p0 + n_tokens;
  HIPCHK(hipMemcpy(c->d_ctx_lens + seq, &len, 4, hipMemcpyHostToDevice));
  return MK_OK;
}

mk_status mk_read_fp8_weights(mk_ctx* c, const char* name, uint8_t* h_codes, int32_t* h_exps, void* stream) {
  if (!c || !name || !h_codes || !h_exps) return fail(MK_ERR_INVALID_ARG, "null argument");
  if (!c->bound || !c->loaded) return fail(MK_ERR_STATE, "bind memory and load weights first");
  const HostGraph& g = c->g;
  const mk_model_config& m = g.cfg;
  if (m.weight_format != MK_WEIGHTS_FP8_E4M3) return fail(MK_ERR_STATE, "the context's weights are not FP8");
  // which stage holds the matrix, and which of its packed rows are the matrix's
  const std::string nm = name;
  int type = -1, layer = m.n_layers, which = 0;
  if (nm == "lm_head" || (nm == "embed" && m.tied_embeddings)) {
    type = T_LMHEAD;
  } else if (nm.rfind("layers.", 0) == 0) {
    const size_t dot = nm.find('.', 7);
    if (dot == std::string::npos) return fail(MK_ERR_INVALID_ARG, "unknown tensor " + nm);
    layer = std::atoi(nm.substr(7, dot - 7).c_str());
    const std::string t = nm.substr(dot + 1);
    if (t == "wq") { type = T_QKV; which = 0; }
    else if (t == "wk") { type = T_QKV; which = 1; }
    else if (t == "wv") { type = T_QKV; which = 2; }
    else if (t == "wo") type = T_OPROJ;
    else if (t == "wg") { type = T_GATEUP; which = 0; }
    else if (t == "wu") { type = T_GATEUP; which = 1; }
    else if (t == "wd") type = T_DOWN;
    if (layer < 0 || layer >= m.n_layers) type = -1;
  }
  if (type < 0) return fail(MK_ERR_INVALID_ARG, "not an FP8 matrix: " + nm);
  size_t t0 = 0;
  while (t0 < g.tasks.size() && !(g.tasks[t0].type == type && g.tasks[t0].layer == layer)) ++t0;
  size_t t1 = t0;
  while (t1 < g.tasks.size() && g.tasks[t1].type == type && g.tasks[t1].layer == layer) ++t1;
  if (t0 == t1) return fail(MK_ERR_STATE, "no such stage");
  const GemvGeom& q = g.geoms[g.tasks[t0].geom];
  const int64_t b0 = g.tasks[t0].wofs, b1 = g.tasks[t1 - 1].wofs + task_tile_bytes(q, g.tasks[t1 - 1]);
  const int nrows = g.tasks[t1 - 1].row1;
  std::vector<uint8_t> tiles((size_t)(b1 - b0));
  std::vector<float> sc((size_t)nrows);
  DeviceGuard dg(c->device);
  hipStream_t st = (hipStream_t)stream;
  HIPCHK(hipMemcpyAsync(tiles.data(), c->d_weights + b0, tiles.size(), hipMemcpyDeviceToHost, st));
  HIPCHK(hipMemcpyAsync(sc.data(), c->d_weights + g.wl.scales + (size_t)g.tasks[t0].a1 * 4, sc.size() * 4,
                        hipMemcpyDeviceToHost, st));
  HIPCHK(hipStreamSynchronize(st));
  const int G = m.n_q_heads / m.n_kv_heads, dh = m.head_dim, K = q.K, su = q.S / 2;
  // packed row -> (sub-matrix, its row), the mapping the re-layout applies
  auto source = [&](int pr, int* sub) {
    if (type == T_QKV) {
      const int Rg = (G + 2) * dh, grp = pr / Rg, within = pr % Rg, slot = within / dh, jh = within % dh;
      const int dim = (jh & 1) ? (jh >> 1) + dh / 2 : (jh >> 1);
      if (slot < G) { *sub = 0; return (grp * G + slot) * dh + dim; }
      *sub = slot == G ? 1 : 2;
      return grp * dh + dim;
    }
    if (type == T_GATEUP) { *sub = pr & 1; return pr >> 1; }
    *sub = 0;
    return pr;
  };
  for (size_t ti = t0; ti < t1; ++ti) {
    const TaskDesc& t = g.tasks[ti];
    const int64_t units = task_tile_bytes(q, t) / 1024;
    for (int64_t u = 0; u < units; ++u) {
      const int gi = (int)(u / su), ui = (int)(u % su);
      for (int lane = 0; lane < 64; ++lane) {
        const int rl = gi * q.rg + lane / q.lpr;
        if (rl >= t.row1 - t.row0) continue;
        const int pr = t.row0 + rl;
        int sub = 0;
        const int row = source(pr, &sub);
        if (sub != which) continue;
        int ex = 0;
        (void)std::frexp(sc[(size_t)pr], &ex);  // the scale is 2^(ex - 1)
        h_exps[row] = ex - 1;
        for (int h = 0; h < 2; ++h) {
          const int piece = (2 * ui + h) * q.lpr + (lane & (q.lpr - 1));
          if (piece >= q.P) continue;
          const uint8_t* src = tiles.data() + (t.wofs - b0) + u * 1024 + lane * 16 + h * 8;
          std::memcpy(h_codes + (size_t)row * K + (size_t)piece * 8, src, 8);
        }
      }
    }
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
  out->attn_tasks = g.attn_tasks;
  out->n_cus = g.n_cus;
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

mk_status mk_graph_corrupt(mk_ctx* c, int kind) {
  if (!c) return fail(MK_ERR_INVALID_ARG, "null context");
  if (c->device >= 0) return fail(MK_ERR_STATE, "only host-only contexts may be corrupted");
  const std::string why = corrupt_graph(c->g, kind);
  return why.empty() ? MK_OK : fail(MK_ERR_INVALID_ARG, why);
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
