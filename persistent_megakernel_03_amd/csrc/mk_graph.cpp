// Host-side task-graph builder, validator and interleaving simulator.
//
// The builder refines the decode step's operators into per-CU tasks over the
// data units that really depend on each other ("LLMs in einen MegaKernel
// kompilieren", "Part 1. Compiler": one task per SM, events as sync points,
// a fine-grained task graph; "MPK: A Compiler and Runtime for
// Mega-Kernelizing Tensor Programs", analogy 2, the SM-level graph).
//
// The decode graph is fixed, so the builder emits it directly, ahead of time.
// Every CU's queue follows one global topological order. All workgroups are
// co-resident, so this order makes the graph deadlock-free. Each task runs on
// one CU. The tasks of one operator stage are spread evenly, one per CU, so
// every CU streams an equal share of each weight matrix.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <numeric>
#include <string>

#include "mk_host.h"

namespace mk {

static int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

GemvGeom choose_geom(int K) {
  GemvGeom g{};
  g.K = K;
  g.P = K / 8;
  int lpr = 0;
  for (int c : {64, 32, 16})
    if (g.P % c == 0) { lpr = c; break; }
  if (!lpr)
    for (int c : {64, 32, 16, 8, 4, 2, 1}) {
      const int64_t padded = (int64_t)(g.P + c - 1) / c * c;
      if ((padded - g.P) * 16 <= g.P) { lpr = c; break; }
    }
  g.lpr = lpr;
  g.rg = 64 / lpr;
  g.S = (g.P + lpr - 1) / lpr;
  return g;
}

GemvGeom choose_geom_batched(int K) {
  GemvGeom g{};
  g.K = K;
  g.P = K / 8;
  g.lpr = 4;
  g.rg = 16;
  g.S = (K + 511) / 512 * 16;
  g.mfma = 1;
  return g;
}

namespace {

struct Range { int r0, r1; };

// Rows [0, N) in units of A rows, split as evenly as possible over n CUs.
std::vector<Range> distribute(int N, int A, int n) {
  std::vector<Range> out(n);
  const int64_t units = (N + A - 1) / A;
  for (int c = 0; c < n; ++c) {
    const int64_t u0 = units * c / n, u1 = units * (c + 1) / n;
    out[c].r0 = (int)std::min<int64_t>(N, u0 * A);
    out[c].r1 = (int)std::min<int64_t>(N, u1 * A);
  }
  return out;
}

// Rows [0, N) in units of A rows over n CUs in proportion to weights w (all positive): CU c gets the
// units between the rounded cumulative shares of CUs < c and <= c.
std::vector<Range> distribute_weighted(int N, int A, const std::vector<double>& w) {
  const int n = (int)w.size();
  std::vector<Range> out(n);
  const int64_t units = (N + A - 1) / A;
  double tot = 0.0;
  for (double x : w) tot += x;
  double acc = 0.0;
  int64_t u0 = 0;
  for (int c = 0; c < n; ++c) {
    acc += w[c];
    const int64_t u1 = c == n - 1 ? units : std::min<int64_t>(units, (int64_t)std::llround(units * acc / tot));
    out[c].r0 = (int)std::min<int64_t>(N, u0 * A);
    out[c].r1 = (int)std::min<int64_t>(N, std::max(u0, u1) * A);
    u0 = std::max(u0, u1);
  }
  return out;
}

// Column split of a batched GEMV stage: kS splits of nu units (32 columns each) per row tile.
struct KSplit {
  int kS, nu, tiles;
};
constexpr int kMaxTileGroups = 48;  // 16-row groups of one batched tile: their partial sums stay in LDS

// Per-CU bytes of a batched stage for each candidate split count, and the cheapest. A CU streams its
// weight tile (rows x its columns) and reads its columns of every sequence's input as tagged 64-bit
// words from the coherent level (16 sequences x 8 B per column). Splitting the columns cuts that
// input traffic kS-fold but adds an exchange: each split writes its partial sums of the tile and
// reads back kS partials of its own share, plus one more cross-CU round trip (charged as 40 KB).
// With one split and more than 32 units, the task streams its columns in blocks of 16 units.
KSplit choose_ksplit(int N, int K, int n_cus, int max_split) {
  const int nu_tot = (K + 31) / 32;
  const int64_t units16 = (N + 15) / 16;
  KSplit best{0, 0, 0};
  int64_t best_cost = INT64_MAX;
  for (int kS = 1; kS <= std::min({nu_tot, n_cus, max_split}); ++kS) {
    int nu = (nu_tot + kS - 1) / kS;
    if ((nu_tot + nu - 1) / nu != kS) continue;  // the last split would be empty
    if (kS > 1 && nu > 32) continue;               // a split's columns fit one LDS block
    if (nu > 32) nu = (int)align_up(nu, 16);
    // one split: as many row tiles as CUs, or more (several per CU) when tiles would outgrow the LDS;
    // with a column split, one task per CU and stage (its splits wait for each other)
    const int64_t tiles = kS == 1 ? std::max<int64_t>(n_cus, (units16 + kMaxTileGroups - 1) / kMaxTileGroups) : n_cus / kS;
    const int64_t R = (units16 + tiles - 1) / tiles;
    if (R > kMaxTileGroups) continue;
    if (kS > 1) {  // every split must own rows: each non-empty tile needs at least kS row quads
      int min_q = INT_MAX;
      for (const Range& r : distribute(N, 16, (int)tiles))
        if (r.r1 > r.r0) min_q = std::min(min_q, (r.r1 - r.r0 + 3) / 4);
      if (min_q < kS) continue;
    }
    const int64_t per_cu = (tiles + n_cus - 1) / n_cus;  // tasks per CU and stage
    const int64_t cost = per_cu * (R * nu * 1024 + (int64_t)4096 * nu) + (kS > 1 ? 4096 * R + 40000 : 0);
    if (cost < best_cost) {
      best_cost = cost;
      best = KSplit{kS, nu, (int)tiles};
    }
  }
  return best;
}

struct Builder {
  HostGraph& g;
  const mk_model_config& c;
  std::vector<int32_t> task_cu;
  std::vector<std::vector<std::pair<int, int>>> task_sig;  // (event, producer index) per task
  std::vector<int> ev_producers;                            // producer count per event
  int64_t packed = 0;

  Builder(HostGraph& g_, const mk_model_config& c_) : g(g_), c(c_) {}

  int new_event(int nprod) {
    ev_producers.push_back(nprod);
    return (int)ev_producers.size() - 1;
  }
  int add_task(const TaskDesc& t, int cu) {
    g.tasks.push_back(t);
    g.acc.emplace_back();
    g.comb_acc.emplace_back();
    g.task_group.push_back(-1);
    g.task_comb.push_back(0);
    task_cu.push_back(cu);
    task_sig.emplace_back();
    return (int)g.tasks.size() - 1;
  }
  void acc(int t, int buf, int64_t lo, int64_t hi, int w) {
    if (hi > lo) g.acc[t].push_back(Access{buf, lo, hi, w});
  }
  void cacc(int t, int buf, int64_t lo, int64_t hi, int w) {
    if (hi > lo) g.comb_acc[t].push_back(Access{buf, lo, hi, w});
  }
  int64_t tile_bytes(int geom, int rows) const {
    const GemvGeom& q = g.geoms[geom];
    return (int64_t)((rows + q.rg - 1) / q.rg) * (q.fp8 ? q.S / 2 : q.S) * 1024;
  }
  int64_t scale_rows = 0;  // FP8 weights: packed GEMV rows so far, the row-scale array's length
  // A GEMV stage: one task per CU with a non-empty row range, over the CUs not marked in `skip`.
  std::vector<int> gemv_stage(int type, int layer, int geom, int N, int A, int wait_ev,
                              const std::vector<char>* skip = nullptr, const std::vector<double>* weight = nullptr) {
    std::vector<int> ids, cus;
    for (int cu = 0; cu < g.n_cus; ++cu)
      if (!skip || !(*skip)[cu]) cus.push_back(cu);
    std::vector<double> w;
    for (int cu : cus) w.push_back(weight ? (*weight)[cu] : 1.0);
    auto rs = weight ? distribute_weighted(N, A, w) : distribute(N, A, (int)cus.size());
    for (size_t k = 0; k < cus.size(); ++k) {
      const int cu = cus[k];
      if (rs[k].r1 <= rs[k].r0) continue;
      TaskDesc t{};
      t.type = type;
      t.layer = layer;
      t.wait_ev = wait_ev;
      t.row0 = rs[k].r0;
      t.row1 = rs[k].r1;
      t.geom = geom;
      t.wofs = packed;
      if (g.geoms[geom].fp8) t.a1 = (int32_t)(scale_rows + t.row0);
      packed += tile_bytes(geom, t.row1 - t.row0);
      ids.push_back(add_task(t, cu));
    }
    if (g.geoms[geom].fp8) scale_rows += N;
    return ids;
  }
};

int lcm_i(int a, int b) { return a / std::gcd(a, b) * b; }

}  // namespace

std::string build_graph(const mk_model_config& c, int n_cus, HostGraph& g) {
  g = HostGraph{};
  if (n_cus < 1 || n_cus > 4096) return "n_cus out of range";
  if (c.n_layers < 1 || c.d_model < 8 || c.n_q_heads < 1 || c.n_kv_heads < 1 || c.head_dim < 4 || c.d_ffn < 8 ||
      c.vocab < 2)
    return "non-positive model dimension";
  if (c.n_q_heads % c.n_kv_heads) return "n_q_heads must be a multiple of n_kv_heads";
    if (c.d_model % 8 || c.d_ffn % 8 || (c.n_q_heads * c.head_dim) % 8) return "GEMV inner dims must be multiples of 8";
  if (c.n_q_heads / c.n_kv_heads > 8) return "at most 8 query heads per KV head";
  if (c.head_dim != 64 && c.head_dim != 128) return "head_dim must be 64 or 128";
  // a workgroup polls each tagged activation vector with at most 16 (d, hq*dh) or 32 (d_ffn) words per thread
  if (c.d_model > 8192 || c.n_q_heads * c.head_dim > 8192 || c.d_ffn > 16384) return "model too wide for the activation polls";
  if (c.block_size != 16) return "block_size must be 16";
  if (c.max_seqs < 1 || c.max_seqs > 16) return "max_seqs must be 1..16 (one 16-row MFMA tile of sequences)";
  // batched tiles stage the normalised inputs 32 columns at a time; every staged column of a normalised
  // input must be a real one
  if (c.max_seqs > 1 && c.d_model % 32) return "batched decode needs d_model to be a multiple of 32";
  if (c.max_blocks_per_seq < 1 || c.num_blocks < 1) return "empty KV cache";
  if (!(c.rms_eps >= 0.f) || !(c.rope_theta > 0.f)) return "bad rms_eps or rope_theta";
  if (c.attn_splits < 0 || c.attn_splits > 64) return "attn_splits out of range";
  if (c.attn_min_blocks < 0 || c.attn_min_blocks > (1 << 20)) return "attn_min_blocks out of range";
  if (c.prefill_rows < 0 || c.prefill_rows > 16) return "prefill_rows must be 0..16";
  if (c.max_seqs > 1 && c.prefill_rows != 0)
    return "prefill_rows applies to one-sequence contexts (a batched context prefills through its own rows)";
  if (c.prefill_rows > 1 && c.d_model % 32) return "chunked prefill needs d_model to be a multiple of 32";
  if (c.weight_format != MK_WEIGHTS_BF16 && c.weight_format != MK_WEIGHTS_FP8_E4M3) return "unknown weight_format";
  if (c.weight_format == MK_WEIGHTS_FP8_E4M3 && (c.max_seqs != 1 || c.prefill_rows > 1))
    return "FP8 weights run one-sequence contexts without prefill_rows";
  g.cfg = c;
  g.n_cus = n_cus;
  g.max_pos = c.max_blocks_per_seq * c.block_size;
  const int L = c.n_layers, d = c.d_model, hq = c.n_q_heads, hk = c.n_kv_heads, dh = c.head_dim, f = c.d_ffn,
            V = c.vocab, S = c.max_seqs, G = hq / hk;
  const int qd = hq * dh, Nqkv = qkv_rows(c), Rg = (G + 2) * dh;
  if (c.attn_splits > 0) {
    g.splits = c.attn_splits;
  } else if (S == 1) {
    // one sequence: with a short cache attention is a latency hop between two stages, and eight tasks
    // per KV head (the step's blocks cut evenly over them) measured fastest on the 8B decode across
    // contexts from 60 to 400 positions; more tasks take CUs away from the O projection. A long cache
    // makes attention the largest stream of the layer, so the tasks grow with it, to 32 per KV head
    // from 2,048 blocks (32K positions) on.
    g.splits = std::max(1, std::min(c.max_blocks_per_seq, std::clamp(c.max_blocks_per_seq / 64, 8, 32)));
  } else {
    // about one staged chunk of positions per split (8 waves x 64/(dh/8) positions x 4 slots)
    const int chunk_blocks = 8 * (64 / (dh / 8)) * 4 / 16;
    int sp = (c.max_blocks_per_seq + chunk_blocks - 1) / chunk_blocks;
    sp = std::min(sp, 32);
    sp = std::min(sp, std::max(1, 2 * n_cus / (S * hk)));
    g.splits = std::max(1, sp);
  }
  // one sequence: row-per-lanes GEMV tiles; several: 16-row MFMA tiles (the GEMV becomes a skinny GEMM)
  auto geom = S > 1 ? choose_geom_batched : choose_geom;
  g.geoms[G_QKV] = geom(d);
  g.geoms[G_O] = geom(qd);
  g.geoms[G_GU] = geom(d);
  g.geoms[G_D] = geom(f);
  g.geoms[G_LM] = geom(d);
  if (c.weight_format == MK_WEIGHTS_FP8_E4M3)
    for (int i = 0; i < G_COUNT; ++i) {
      // An FP8 unit carries two bf16-layout units of a row group, so a group needs an even count: an
      // odd one is doubled by halving the lanes per row (twice the rows per group), then padded.
      GemvGeom& q = g.geoms[i];
      q.fp8 = 1;
      if ((q.S & 1) && q.lpr > 1) {
        q.lpr /= 2;
        q.rg = 64 / q.lpr;
        q.S = (q.P + q.lpr - 1) / q.lpr;
      }
      q.S += q.S & 1;
    }

  g.sym_size[S_X] = (int64_t)S * d;
  g.sym_size[S_Q] = (int64_t)S * qd;
  g.sym_size[S_KVCUR] = (int64_t)L * S * hk * 2 * dh;
  g.sym_size[S_PART] = (int64_t)L * 2 * S * hk * g.splits;
  g.sym_size[S_O] = (int64_t)S * qd;
  g.sym_size[S_H] = (int64_t)S * f;
  g.sym_size[S_LOGITS] = (int64_t)S * V;
  g.sym_size[S_CTX] = S;
  g.sym_size[S_TOKOUT] = S;

  Builder b(g, c);
  // Batched stages also split the columns over CUs. MK_BATCHED_MAX_KSPLIT caps the number of column
  // splits (1 = row tiles only, whose columns then stream in 512-column blocks).
  int max_ksplit = 1 << 20;
  if (const char* e = std::getenv("MK_BATCHED_MAX_KSPLIT")) max_ksplit = std::max(1, std::atoi(e));
  int64_t bpt_words = 0;
  int64_t bpart_slots = 0;
  std::string err;

  // Reads of columns [c0, c1) of every sequence's GEMV input.
  auto in_acc = [&](int t, int type, int l, int64_t c0, int64_t c1) {
    for (int s = 0; s < S; ++s) {
      if (type == T_QKV) {
        if (l > 0) b.acc(t, S_X, (int64_t)s * d + c0, (int64_t)s * d + c1, 0);
      } else if (type == T_OPROJ) {
        b.acc(t, S_O, (int64_t)s * qd + c0, (int64_t)s * qd + c1, 0);
      } else if (type == T_DOWN) {
        b.acc(t, S_H, (int64_t)s * f + c0, (int64_t)s * f + c1, 0);
      } else {
        b.acc(t, S_X, (int64_t)s * d + c0, (int64_t)s * d + c1, 0);
      }
    }
  };
  // Output rows [r0, r1) of every sequence, with the residual rows and context lengths the epilogue
  // reads, in the task's first phase or (comb) its second.
  auto out_acc = [&](int t, int type, int l, int r0, int r1, bool comb) {
    auto A = [&](int buf, int64_t lo, int64_t hi, int w) {
      if (comb) b.cacc(t, buf, lo, hi, w);
      else b.acc(t, buf, lo, hi, w);
    };
    for (int s = 0; s < S; ++s) {
      if (type == T_QKV) {
        A(S_CTX, s, s + 1, 0);
        // packed rows -> written q / k / v elements (pairs [a/2, b/2) and their + dh/2 partners)
        for (int r = r0; r < r1;) {
          const int grp = r / Rg, within = r % Rg, slot = within / dh;
          const int hs = grp * Rg + slot * dh;  // packed start of this head
          const int e = std::min(r1, hs + dh);
          const int p0 = (r - hs) / 2, p1 = (e - hs) / 2;
          if (slot < G) {
            const int64_t base = (int64_t)s * qd + (int64_t)(grp * G + slot) * dh;
            A(S_Q, base + p0, base + p1, 1);
            A(S_Q, base + p0 + dh / 2, base + p1 + dh / 2, 1);
          } else {
            const int64_t base = (((int64_t)l * S + s) * hk + grp) * 2 * dh + (slot == G ? 0 : dh);
            A(S_KVCUR, base + p0, base + p1, 1);
            A(S_KVCUR, base + p0 + dh / 2, base + p1 + dh / 2, 1);
          }
          r = e;
        }
      } else if (type == T_OPROJ || type == T_DOWN) {
        if (type == T_DOWN || l > 0) A(S_X, (int64_t)s * d + r0, (int64_t)s * d + r1, 0);
        A(S_X, (int64_t)s * d + r0, (int64_t)s * d + r1, 1);
      } else if (type == T_GATEUP) {
        A(S_H, (int64_t)s * f + r0 / 2, (int64_t)s * f + r1 / 2, 1);
      } else {
        A(S_LOGITS, (int64_t)s * V + r0, (int64_t)s * V + r1, 1);
      }
    }
  };
  struct StageTask {
    int id, r0, r1;  // task and the output rows it writes
    bool comb;       // written in its second phase
  };
  // One GEMV stage. One sequence: one task per CU with a row tile. Several: row tiles of 16-row
  // groups, each split by columns over kS CUs; each split then sums the kS partials of its share of
  // the tile's rows (a quarter-row-group granularity) and applies the epilogue to it.
  auto stage = [&](int type, int l, int geom, int N, int K, int align, int wait_ev,
                   const std::vector<char>* skip, const std::vector<double>* weight = nullptr) -> std::vector<StageTask> {
    std::vector<StageTask> out;
    if (S == 1) {
      for (int id : b.gemv_stage(type, l, geom, N, align, wait_ev, skip, weight)) {
        in_acc(id, type, l, 0, K);
        out.push_back({id, g.tasks[id].row0, g.tasks[id].row1, false});
      }
      return out;
    }
    const KSplit ks = choose_ksplit(N, K, n_cus, max_ksplit);
    if (!ks.kS) {
      err = "no column split of a batched GEMV stage fits the LDS";
      return out;
    }
    const int nu_tot = (K + 31) / 32, tiles = ks.tiles;
    const auto rs = distribute(N, 16, tiles);
    for (int k = 0; k < tiles; ++k) {
      if (rs[k].r1 <= rs[k].r0) continue;
      const int rows = rs[k].r1 - rs[k].r0, R = (rows + 15) / 16, Q = (rows + 3) / 4;
      if (Q < ks.kS) {
        err = "a batched tile has fewer row quads than column splits";
        return out;
      }
      g.max_tile_groups = std::max(g.max_tile_groups, R);
      int grp = -1;
      const int64_t pofs = bpt_words, slot0 = bpart_slots;
      if (ks.kS > 1) {
        bpt_words += (int64_t)ks.kS * (R * 256 + 64);
        bpart_slots += ks.kS;
        grp = (int)g.group_size.size();
        g.group_size.push_back(ks.kS);
        g.group_ordered.push_back(0);
      }
      for (int j = 0; j < ks.kS; ++j) {
        TaskDesc t{};
        t.type = type;
        t.layer = l;
        t.wait_ev = wait_ev;
        t.row0 = rs[k].r0;
        t.row1 = rs[k].r1;
        t.geom = geom;
        t.wofs = b.packed;
        const int kb0 = j * ks.nu, nuj = ks.kS == 1 ? ks.nu : std::min(ks.nu, nu_tot - kb0);
        t.a1 = (int32_t)pofs;
        t.a2 = kb0 | (nuj << 16);
        t.a3 = j | (ks.kS << 8);
        b.packed += (int64_t)R * nuj * 1024;
        const int id = b.add_task(t, (k * ks.kS + j) % n_cus);
        g.task_group[id] = grp;
        g.task_comb[id] = ks.kS > 1;
        in_acc(id, type, l, 32LL * kb0, std::min<int64_t>(K, 32LL * (kb0 + nuj)));
        if (ks.kS > 1) {
          b.acc(id, S_BPART, slot0 + j, slot0 + j + 1, 1);
          b.cacc(id, S_BPART, slot0, slot0 + ks.kS, 0);
        }
        const int r0 = rs[k].r0 + 4 * (Q * j / ks.kS), r1 = std::min(rs[k].r1, rs[k].r0 + 4 * (Q * (j + 1) / ks.kS));
        out.push_back({id, r0, r1, ks.kS > 1});
      }
    }
    return out;
  };

  int ev_x = -1;  // event "residual stream ready for this layer" (none before layer 0)
  int max_task_rows = 0;
  // Each layer's T attention tasks, one per CU, spread over the CUs (the same CUs in every layer).
  // When they are few, those CUs get no QKV and no O-projection task: an attention task then starts
  // as soon as its CU has finished the previous layer's down projection, and its first cache rows
  // arrive while the other CUs stream the QKV weights; the others hold their O tiles in registers
  // through attention.
  const int T = std::min(S * hk * g.splits, n_cus);  // the cut is balanced: one task per CU suffices
  std::vector<char> attn_cu(n_cus, 0);
  // at most one task per CU: spread; more: round-major (CU c runs tasks c, c + n_cus, ...), so that
  // a merging task never waits on a task that is queued behind another merge
  auto attn_cu_of = [&](int i) { return T <= n_cus ? (int)((int64_t)i * n_cus / T) : i % n_cus; };
  for (int i = 0; i < T; ++i) attn_cu[attn_cu_of(i)] = 1;
  const bool few_attn = (int)std::count(attn_cu.begin(), attn_cu.end(), 1) * 4 <= n_cus;
  const std::vector<char>* skip_attn = few_attn ? &attn_cu : nullptr;
  for (int l = 0; l < L; ++l) {
    // ---- QKV: RMSNorm + GEMV + bias + RoPE + KV append
    auto qkv = stage(T_QKV, l, G_QKV, Nqkv, d, lcm_i(4, g.geoms[G_QKV].rg), ev_x, skip_attn);
    if (!err.empty()) return err;
    const int ev_qkv = b.new_event((int)qkv.size());
    for (size_t i = 0; i < qkv.size(); ++i) {
      const StageTask& st = qkv[i];
      b.task_sig[st.id].push_back({ev_qkv, (int)i});
      max_task_rows = std::max(max_task_rows, g.tasks[st.id].row1 - g.tasks[st.id].row0);
      out_acc(st.id, T_QKV, l, st.r0, st.r1, st.comb);
    }
    // ---- attention: T tasks cut the layer's (sequence, KV head) segments of cache blocks evenly at run
    // time; the task holding a segment's last block merges the others' partials of it. In the symbolic
    // model the layer's tasks form one group: each may merge any segment, and the last one stands for
    // the writers of the attention output.
    g.attn_tasks = T;
    // the device cuts the step's blocks with 32-bit products (blocks x tasks)
    if ((int64_t)S * hk * c.max_blocks_per_seq * T >= ((int64_t)1 << 32)) return "too many KV blocks x attention tasks";
    const int ev_att = b.new_event(T);
    {
      const int agrp = (int)g.group_size.size();
      g.group_size.push_back(T);
      g.group_ordered.push_back(1);
      for (int i = 0; i < T; ++i) {
        TaskDesc t{};
        t.type = T_ATTN;
        t.layer = l;
        t.wait_ev = ev_qkv;
        t.a2 = i;
        t.a3 = l * T + i;
        const int id = b.add_task(t, attn_cu_of(i));
        g.task_group[id] = agrp;
        g.task_comb[id] = 1;
        b.task_sig[id].push_back({ev_att, i});
        b.acc(id, S_Q, 0, (int64_t)S * qd, 0);
        b.acc(id, S_KVCUR, (int64_t)l * S * hk * 2 * dh, (int64_t)(l + 1) * S * hk * 2 * dh, 0);
        b.acc(id, S_CTX, 0, S, 0);
        b.acc(id, S_PART, ((int64_t)l * T + i) * 2, ((int64_t)l * T + i + 1) * 2, 1);
        b.cacc(id, S_PART, (int64_t)l * T * 2, ((int64_t)l * T + i + 1) * 2, 0);  // its own and earlier tasks'
        if (i == T - 1) b.cacc(id, S_O, 0, (int64_t)S * qd, 1);
      }
      g.n_attn_groups = (l + 1) * S * hk;
    }
    // ---- O projection + residual
    auto op = stage(T_OPROJ, l, G_O, d, qd, g.geoms[G_O].rg, ev_att, skip_attn);
    if (!err.empty()) return err;
    const int ev_o = b.new_event((int)op.size());
    for (size_t i = 0; i < op.size(); ++i) {
      max_task_rows = std::max(max_task_rows, g.tasks[op[i].id].row1 - g.tasks[op[i].id].row0);
      b.task_sig[op[i].id].push_back({ev_o, (int)i});
      out_acc(op[i].id, T_OPROJ, l, op[i].r0, op[i].r1, op[i].comb);
    }
    // ---- RMSNorm + gate/up + SwiGLU
    // One sequence: the CUs that ran attention (and no QKV or O projection) start gate/up early, and CUs on
    // odd XCDs (workgroup i runs on XCD i % 8) stream it measurably slower; their row shares are
    // weighted so that the stage ends together (weights measured on the 8B decode).
    std::vector<double> gu_w(n_cus, 1.0);
    if (S == 1 && few_attn)
      for (int cu = 0; cu < n_cus; ++cu) gu_w[cu] = 1.0 + (attn_cu[cu] ? 0.10 : 0.0) - ((cu & 1) ? 0.02 : 0.0);
    auto gu = stage(T_GATEUP, l, G_GU, 2 * f, d, lcm_i(2, g.geoms[G_GU].rg), ev_o, nullptr, S == 1 && few_attn ? &gu_w : nullptr);
    if (!err.empty()) return err;
    const int ev_gu = b.new_event((int)gu.size());
    for (size_t i = 0; i < gu.size(); ++i) {
      max_task_rows = std::max(max_task_rows, g.tasks[gu[i].id].row1 - g.tasks[gu[i].id].row0);
      b.task_sig[gu[i].id].push_back({ev_gu, (int)i});
      out_acc(gu[i].id, T_GATEUP, l, gu[i].r0, gu[i].r1, gu[i].comb);
    }
    // ---- down projection + residual
    auto dn = stage(T_DOWN, l, G_D, d, f, g.geoms[G_D].rg, ev_gu, nullptr);
    if (!err.empty()) return err;
    ev_x = b.new_event((int)dn.size());
    for (size_t i = 0; i < dn.size(); ++i) {
      max_task_rows = std::max(max_task_rows, g.tasks[dn[i].id].row1 - g.tasks[dn[i].id].row0);
      b.task_sig[dn[i].id].push_back({ev_x, (int)i});
      out_acc(dn[i].id, T_DOWN, l, dn[i].r0, dn[i].r1, dn[i].comb);
    }
  }
  // ---- final RMSNorm + LM head + partial argmax (one part per task)
  // the LM head streams about 7% slower on odd XCDs: their CUs take proportionally fewer rows
  std::vector<double> lm_w(n_cus, 1.0);
  for (int cu = 0; cu < n_cus; ++cu) lm_w[cu] = (cu & 1) ? 0.965 : 1.035;
  auto lm = stage(T_LMHEAD, L, G_LM, V, d, g.geoms[G_LM].rg, ev_x, nullptr, S == 1 ? &lm_w : nullptr);
  if (!err.empty()) return err;
  g.n_lm_parts = (int)lm.size();
  g.sym_size[S_AMAX] = (int64_t)S * g.n_lm_parts;
  const int ev_lm = b.new_event((int)lm.size());
  for (size_t i = 0; i < lm.size(); ++i) {
    const int t = lm[i].id;
    g.tasks[t].a0 = (int)i;
    max_task_rows = std::max(max_task_rows, g.tasks[t].row1 - g.tasks[t].row0);
    b.task_sig[t].push_back({ev_lm, (int)i});
    out_acc(t, T_LMHEAD, L, lm[i].r0, lm[i].r1, lm[i].comb);
    for (int s = 0; s < S; ++s) {
      const int64_t e = (int64_t)s * g.n_lm_parts + (int64_t)i;
      if (lm[i].comb) b.cacc(t, S_AMAX, e, e + 1, 1);
      else b.acc(t, S_AMAX, e, e + 1, 1);
    }
  }
  // ---- argmax per sequence
  for (int s = 0; s < S; ++s) {
    TaskDesc t{};
    t.type = T_ARGMAX;
    t.layer = L;
    t.wait_ev = ev_lm;
    t.a0 = s;
    const int id = b.add_task(t, (int)((int64_t)s * n_cus / S));
    b.acc(id, S_AMAX, (int64_t)s * g.n_lm_parts, (int64_t)(s + 1) * g.n_lm_parts, 0);
    b.acc(id, S_CTX, s, s + 1, 0);
    b.acc(id, S_CTX, s, s + 1, 1);
    b.acc(id, S_TOKOUT, s, s + 1, 1);
  }
  g.sym_size[S_BPART] = bpart_slots;

  // ---- events -> contiguous flag slots; task signal lists -> absolute slots
  g.events.resize(b.ev_producers.size());
  int32_t slot = 0;
  for (size_t e = 0; e < g.events.size(); ++e) {
    g.events[e].slot0 = slot;
    g.events[e].nslots = b.ev_producers[e];
    slot += b.ev_producers[e];
  }
  g.n_flag_slots = slot;
  for (size_t t = 0; t < g.tasks.size(); ++t) {
    if (g.tasks[t].wait_ev >= 0) {
      g.tasks[t].wait_slot0 = g.events[g.tasks[t].wait_ev].slot0;
      g.tasks[t].wait_nslots = g.events[g.tasks[t].wait_ev].nslots;
    }
    g.tasks[t].sig_off = (int32_t)g.sig_slots.size();
    g.tasks[t].sig_n = (int32_t)b.task_sig[t].size();
    for (auto& s : b.task_sig[t]) g.sig_slots.push_back(g.events[s.first].slot0 + s.second);
  }
  // ---- dynamic scheduling tables: a task's completion counts toward the one event it signals; the
  // event's consumers (the tasks that wait on it) are contiguous in the global order, and the tasks
  // that wait on nothing open the step
  {
    const int T = (int)g.tasks.size(), E = (int)g.events.size();
    g.jit_task_ev.assign(T, -1);
    g.jit_ev_n.assign(E, 0);
    g.jit_ev_c0.assign(E, -1);
    g.jit_ev_c1.assign(E, -1);
    bool ok = S == 1;
    for (int t = 0; t < T; ++t) {
      if (b.task_sig[t].size() > 1) ok = false;
      if (!b.task_sig[t].empty()) g.jit_task_ev[t] = b.task_sig[t][0].first;
      const int e = g.tasks[t].wait_ev;
      if (e < 0) {
        if (t != g.jit_n0) ok = false;  // the opening tasks form a prefix
        g.jit_n0 = t + 1;
        continue;
      }
      if (g.jit_ev_c0[e] < 0) g.jit_ev_c0[e] = t;
      else if (g.jit_ev_c1[e] != t) ok = false;  // consumers must be contiguous
      g.jit_ev_c1[e] = t + 1;
    }
    for (int e = 0; e < E; ++e) {
      g.jit_ev_n[e] = b.ev_producers[e];
      if (g.jit_ev_c0[e] < 0) g.jit_ev_c0[e] = g.jit_ev_c1[e] = 0;
    }
    g.jit_ok = ok;
  }
  // the O and down tasks keep their residual rows in registers: at most 4 per thread of 512
  for (const TaskDesc& td : g.tasks)
    if (S == 1 && (td.type == T_OPROJ || td.type == T_DOWN) && td.row1 - td.row0 > 4 * 512) return "residual task too tall";
  // ---- per-CU queues in global order
  g.queue_off.assign(n_cus + 1, 0);
  for (int32_t cu : b.task_cu) g.queue_off[cu + 1]++;
  for (int i = 0; i < n_cus; ++i) g.queue_off[i + 1] += g.queue_off[i];
  g.queue_idx.assign(g.tasks.size(), 0);
  {
    std::vector<int32_t> fill(g.queue_off.begin(), g.queue_off.end() - 1);
    for (size_t t = 0; t < g.tasks.size(); ++t) g.queue_idx[fill[b.task_cu[t]]++] = (int32_t)t;
  }

  // ---- weights buffer layout
  g.wl.packed_bytes = align_up(b.packed, 256);
  g.wl.embed = g.wl.packed_bytes;
  g.wl.norms = align_up(g.wl.embed + (int64_t)V * d * 2, 256);
  g.wl.bias = align_up(g.wl.norms + (int64_t)(2 * L + 1) * d * 2, 256);
  // a tail pad: batched tasks load gains and embedding columns a block at a time and may read up to one
  // 1024-column block (2 KB) past a row's end (the values are not used)
  g.wl.scales = align_up(g.wl.bias + (c.qkv_bias ? (int64_t)L * Nqkv * 2 : 0), 256);
  g.wl.n_scale_rows = b.scale_rows;
  g.wl.total = align_up(g.wl.scales + b.scale_rows * 4, 256) + 2048;

  // ---- scratch layout
  int64_t o = 0;
  auto take = [&](int64_t bytes) { const int64_t at = o; o = align_up(o + std::max<int64_t>(bytes, 4), 256); return at; };
  g.sl.tasks = take((int64_t)g.tasks.size() * sizeof(TaskDesc));
  g.sl.queue_off = take((int64_t)g.queue_off.size() * 4);
  g.sl.queue_idx = take((int64_t)g.queue_idx.size() * 4);
  g.sl.events = take((int64_t)g.events.size() * sizeof(EventDesc));
  g.sl.sig_slots = take((int64_t)g.sig_slots.size() * 4);
  g.sl.geoms = take((int64_t)G_COUNT * sizeof(GemvGeom));
  g.sl.rope = take((int64_t)g.max_pos * (dh / 2) * 8);
  g.sl.flags = take((int64_t)g.n_flag_slots * 4);
  g.sl.err = take((int64_t)E_COUNT * 4);
  g.sl.tagged_begin = o;
  g.sl.xt = take((int64_t)L * 2 * S * d * 8);
  g.sl.qt = take((int64_t)L * S * qd * 8);
  g.sl.kvt = take((int64_t)L * S * 2 * hk * (dh / 2) * 8);
  g.sl.ot = take((int64_t)L * S * qd * 8);
  g.sl.ht = take((int64_t)L * S * f * 8);
  g.sl.pt = take((int64_t)L * g.attn_tasks * 2 * G * (dh + 2) * 8);
  g.sl.bpt = take(bpt_words * 8);
  g.sl.tokt = take((int64_t)S * 8);
  g.sl.tagged_end = o;
  g.sl.amax = take((int64_t)S * g.n_lm_parts * 8);
  g.sl.tokbuf = take((int64_t)std::max(g.max_pos, 64) * 4);
  g.sl.tokout = take(64 * 4);
  g.sl.pools = take((int64_t)2 * L * 8);
  g.sl.jit_tab = take(((int64_t)g.tasks.size() + 3 * (int64_t)g.events.size()) * 4);
  g.sl.jit_work = take((2 + (int64_t)g.events.size() + (int64_t)g.tasks.size()) * 4);
  if (S > 1) {  // chunked prefill: the rows of a step are consecutive positions of one sequence
    g.sl.pf_ptab = take((int64_t)S * c.max_blocks_per_seq * 4);
    g.sl.pf_ctx = take((int64_t)(g.max_pos / S + 2) * 16 * 4);
    g.sl.pf_logits = take((int64_t)S * V * 4);
    g.sl.pf_tok = take(64 * 4);
  }
  g.sl.total = o;

  // ---- LDS: padded GEMV input vector + per-row results, or the attention working set
  int64_t xs = 0;
  for (int i = 0; i < G_COUNT; ++i) xs = std::max<int64_t>(xs, (int64_t)g.geoms[i].S * g.geoms[i].lpr * 8);
  int64_t gemv_lds = xs * 4 + (int64_t)align_up(max_task_rows, 64) * 4 * S + 1024;
  if (c.weight_format == MK_WEIGHTS_FP8_E4M3) {
    // a task's row scales are loaded two rows per thread
    if (max_task_rows > 2 * 512) return "FP8 weights: a GEMV task of more than 1024 rows";
    gemv_lds += (int64_t)align_up(max_task_rows, 64) * 4;  // the row scales beside the results
  }
  if (S > 1)  // batched: the input columns as MFMA fragments (32 units x 64 lanes x 32 B), the tile's
              // partial sums (1 KB per 16-row group), two edge tiles per wave, per-sequence scalars
    gemv_lds = 32 * 64 * 32 + (int64_t)g.max_tile_groups * 1024 + 8 * 2 * 1024 + 256;
  // attention: the staged queries (G rounded up to 2, 4 or 8 heads), the current key and value rows,
  // each wave's merged (m, l, o) per head
  const int gmax = G <= 2 ? 2 : G <= 4 ? 4 : 8;
  // (batched graphs: each wave's buffer sized for gmax heads, then a chunked prefill's 16 key/value rows)
  const int64_t attn_lds = (int64_t)gmax * dh * 4 + (int64_t)dh * 4 +
                           (S > 1 ? (int64_t)8 * gmax * (dh + 2) * 4 + (int64_t)16 * dh * 4 : (int64_t)8 * G * (dh + 2) * 4);
  int max_q = 0;
  for (int cu = 0; cu < n_cus; ++cu) max_q = std::max(max_q, g.queue_off[cu + 1] - g.queue_off[cu]);
  g.max_queue = max_q;
  // control block + pool pointers + this CU's task descriptors + the attention tasks' first blocks
  const int64_t fixed_lds = 1024 + align_up((int64_t)2 * L * 8, 256) + align_up((int64_t)max_q * (int64_t)sizeof(TaskDesc), 256) +
                            align_up((int64_t)(g.attn_tasks + 1) * 4, 256);
  // One sequence: the second weight stage of the tasks with rows of 4096 inputs, after their input
  // vector, results and row scales, when the LDS has room for it.
  g.stage2_off = 0;
  bool rows512 = false;
  for (int i = 0; i < G_COUNT; ++i) rows512 = rows512 || (!g.geoms[i].mfma && g.geoms[i].lpr == 64 && g.geoms[i].S == 8);
  if (S == 1 && rows512) {
    const int planes = c.weight_format == MK_WEIGHTS_FP8_E4M3 ? 2 : 1;  // results (and FP8 row scales)
    const int64_t off = align_up(4096 * 4 + planes * (int64_t)align_up(max_task_rows, 64) * 4, 1024);
    const int64_t need = off + (int64_t)8 * kStage2Units * 1024;
    if (fixed_lds + align_up(std::max({gemv_lds, attn_lds, need}), 256) + kStageBytes <= 160 * 1024) {
      gemv_lds = std::max(gemv_lds, need);
      g.stage2_off = off;
    }
  }
  // ... + the larger of the GEMV and attention working sets
  g.lds_bytes = fixed_lds + align_up(std::max(gemv_lds, attn_lds), 256);
  if (g.lds_bytes + (S == 1 ? kStageBytes : 0) > 160 * 1024) return "working set exceeds 160 KB of LDS";
  return "";
}

// ----------------------------------------------------------------------------- validation
std::string validate_graph(const HostGraph& g) {
  const int nt = (int)g.tasks.size();
  // every task in exactly one queue, queues in increasing global order
  std::vector<int> seen(nt, 0);
  for (int cu = 0; cu < g.n_cus; ++cu) {
    int prev = -1;
    for (int i = g.queue_off[cu]; i < g.queue_off[cu + 1]; ++i) {
      const int t = g.queue_idx[i];
      if (t < 0 || t >= nt) return "queue index out of range";
      if (t <= prev) return "queue not in global order on CU " + std::to_string(cu);
      prev = t;
      seen[t]++;
    }
  }
  for (int t = 0; t < nt; ++t)
    if (seen[t] != 1) return "task " + std::to_string(t) + " is not in exactly one queue";
  // slot writers: each slot has one writer task, or one (seq, kv head) group of attention splits
  std::vector<int> writer(g.n_flag_slots, -1);
  for (int t = 0; t < nt; ++t) {
    const TaskDesc& td = g.tasks[t];
    for (int i = 0; i < td.sig_n; ++i) {
      const int s = g.sig_slots[td.sig_off + i];
      if (s < 0 || s >= g.n_flag_slots) return "signal slot out of range";
      const int key = td.type == T_ATTN ? -2 - td.a3 : t;   // all splits of one group share their slot
      if (writer[s] != -1 && writer[s] != key) return "flag slot " + std::to_string(s) + " has two writers";
      writer[s] = key;
    }
  }
  for (int s = 0; s < g.n_flag_slots; ++s)
    if (writer[s] == -1) return "flag slot " + std::to_string(s) + " has no writer";
  // every producer of a task's event comes before the task in global order
  std::vector<int> last_writer_task(g.n_flag_slots, -1);
  for (int t = 0; t < nt; ++t)
    for (int i = 0; i < g.tasks[t].sig_n; ++i) {
      const int s = g.sig_slots[g.tasks[t].sig_off + i];
      last_writer_task[s] = std::max(last_writer_task[s], t);
    }
  for (int t = 0; t < nt; ++t) {
    const int e = g.tasks[t].wait_ev;
    if (e < -1 || e >= (int)g.events.size()) return "wait event out of range";
    if (e < 0) continue;
    const EventDesc& ev = g.events[e];
    if (ev.nslots <= 0) return "event with no producers";
    if (g.tasks[t].wait_slot0 != ev.slot0 || g.tasks[t].wait_nslots != ev.nslots) return "task's copy of its event differs";
    for (int s = ev.slot0; s < ev.slot0 + ev.nslots; ++s)
      if (last_writer_task[s] >= t) return "task " + std::to_string(t) + " waits on a later producer";
  }
  // every output row of a GEMV stage is written exactly once (once per column split when the stage's
  // tiles are split by columns): the row ranges of the tasks with one split index tile [0, N)
  for (int t0 = 0; t0 < nt;) {
    int t1 = t0 + 1;
    while (t1 < nt && g.tasks[t1].type == g.tasks[t0].type && g.tasks[t1].layer == g.tasks[t0].layer) ++t1;
    const TaskDesc& a = g.tasks[t0];
    if (a.type != T_ATTN && a.type != T_ARGMAX) {
      const mk_model_config& c = g.cfg;
      const int N = a.type == T_QKV ? qkv_rows(c) : a.type == T_GATEUP ? 2 * c.d_ffn : a.type == T_LMHEAD ? c.vocab : c.d_model;
      const int kS = g.geoms[a.geom].mfma ? std::max(1, a.a3 >> 8) : 1;
      for (int j = 0; j < kS; ++j) {
        std::vector<std::pair<int, int>> rs;
        for (int t = t0; t < t1; ++t)
          if (!g.geoms[a.geom].mfma || (g.tasks[t].a3 & 0xFF) == j) rs.push_back({g.tasks[t].row0, g.tasks[t].row1});
        std::sort(rs.begin(), rs.end());
        int at = 0;
        for (auto& r : rs) {
          if (r.first != at)
            return "stage of type " + std::to_string(a.type) + " (layer " + std::to_string(a.layer) + ") " +
                   (r.first < at ? "writes rows " + std::to_string(r.first) + ".." + std::to_string(at) + " twice"
                                 : "leaves rows " + std::to_string(at) + ".." + std::to_string(r.first) + " unwritten");
          at = r.second;
        }
        if (at != N) return "stage of type " + std::to_string(a.type) + " (layer " + std::to_string(a.layer) + ") does not end at row " + std::to_string(N);
      }
    }
    t0 = t1;
  }
  // GEMV tiles: contiguous in stage order and in range
  int64_t end = 0;
  for (int t = 0; t < nt; ++t) {
    const TaskDesc& td = g.tasks[t];
    if (td.type == T_ATTN || td.type == T_ARGMAX) continue;
    const GemvGeom& q = g.geoms[td.geom];
    if (td.row1 <= td.row0) return "empty GEMV task";
    if (td.wofs != end) return "GEMV tiles not contiguous in stage order";
    if (q.mfma) {  // a batched split: its columns lie inside K, and a several-block task has whole blocks
      const int kb0 = td.a2 & 0xFFFF, nu = td.a2 >> 16, kS = td.a3 >> 8;
      if (nu < 1 || 32 * kb0 >= q.K || (kS > 1 && nu > 32) || (nu > 32 && nu % 16)) return "bad batched column split";
      if ((td.row1 - td.row0 + 15) / 16 > g.max_tile_groups) return "batched tile taller than its LDS";
    }
    end += task_tile_bytes(q, td);
    if (td.type == T_QKV && (td.row0 % 4 || td.row1 % 4)) return "QKV task not aligned to RoPE pair sets";
    if (td.type == T_GATEUP && (td.row0 % 2 || td.row1 % 2)) return "gate/up task splits a pair";
  }
  if (end > g.wl.packed_bytes) return "tiles exceed the packed weights";
  if (g.lds_bytes + (g.cfg.max_seqs == 1 ? kStageBytes : 0) > 160 * 1024) return "LDS over budget";
  return "";
}

// ----------------------------------------------------------------------------- simulation
namespace {
uint64_t sm_next(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ULL);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}
}  // namespace

// The dynamic schedule of one step (what mk_decode_step_dynamic runs): tasks leave a FIFO ready queue
// (filled first with the opening tasks) onto at most n_cus workgroups and finish in a random order;
// a finished task counts toward its event, and the event's last producer appends the event's consumers.
// A task of an ordered group (attention) finishes only after the group's earlier members. Checks that
// every task runs exactly once, that no task starts before every earlier-positioned writer of an
// element it reads has finished (partials excepted: they are polled), and that the queue never stalls.
static std::string simulate_dynamic(const HostGraph& g, uint64_t seed) {
  const int nt = (int)g.tasks.size(), ne = (int)g.events.size();
  if (!g.jit_ok) return "";
  std::vector<std::vector<std::vector<int>>> writers(S_COUNT);
  for (int b = 0; b < S_COUNT; ++b) writers[b].resize(g.sym_size[b]);
  for (int t = 0; t < nt; ++t)
    for (const auto* as : {&g.acc[t], &g.comb_acc[t]})
      for (const Access& a : *as)
        if (a.write)
          for (int64_t e = a.lo; e < a.hi; ++e) writers[a.buf][e].push_back(t);
  std::vector<int> queue, cnt(ne, 0), done(nt, 0), started(nt, 0), running;
  for (int t = 0; t < g.jit_n0; ++t) queue.push_back(t);
  size_t head = 0;
  uint64_t rng = seed * 0x9E3779B97F4A7C15ULL + 1;
  auto rnd = [&]() { rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17; return rng; };
  int finished = 0;
  while (finished < nt) {
    while ((int)running.size() < g.n_cus && head < queue.size()) {
      const int t = queue[head++];
      if (t < 0 || t >= nt || started[t]++) return "dynamic schedule: task " + std::to_string(t) + " queued twice";
      for (const auto* as : {&g.acc[t], &g.comb_acc[t]})
        for (const Access& a : *as) {
          if (a.write || a.buf == S_PART || a.buf == S_BPART) continue;
          for (int64_t e = a.lo; e < a.hi; ++e)
            for (int w : writers[a.buf][e])
              if (w < t && !done[w])
                return "dynamic schedule: task " + std::to_string(t) + " started before its producer " + std::to_string(w);
        }
      running.push_back(t);
    }
    std::vector<int> can;
    for (size_t i = 0; i < running.size(); ++i) {
      const int t = running[i], gi = g.task_group[t];
      bool ok = true;
      if (gi >= 0 && g.group_ordered[gi])
        for (int m = 0; m < t && ok; ++m)
          if (g.task_group[m] == gi && !done[m]) ok = false;
      if (ok) can.push_back((int)i);
    }
    if (can.empty()) return "dynamic schedule stalls with " + std::to_string(running.size()) + " tasks running";
    const int i = can[rnd() % can.size()], t = running[i];
    running.erase(running.begin() + i);
    done[t] = 1;
    ++finished;
    const int e = g.jit_task_ev[t];
    if (e >= 0 && ++cnt[e] == g.jit_ev_n[e])
      for (int c = g.jit_ev_c0[e]; c < g.jit_ev_c1[e]; ++c) queue.push_back(c);
  }
  if ((int)queue.size() != nt) return "dynamic schedule: " + std::to_string(queue.size()) + " tasks queued of " + std::to_string(nt);
  return "";
}

std::string simulate_graph(const HostGraph& g, uint64_t seed, int n_steps) {
  if (n_steps > 0) {
    const std::string d = simulate_dynamic(g, seed);
    if (!d.empty()) return d;
  }
  const int nt = (int)g.tasks.size();
  const int ng = (int)g.group_size.size();
  // Static writer/reader lists per element; a task's second-phase accesses count at its position.
  std::vector<std::vector<std::vector<int>>> writers(S_COUNT), readers(S_COUNT);
  for (int b = 0; b < S_COUNT; ++b) {
    writers[b].resize(g.sym_size[b]);
    readers[b].resize(g.sym_size[b]);
  }
  auto add = [&](const Access& a, int pos) {
    if (a.lo < 0 || a.hi > g.sym_size[a.buf]) return false;
    for (int64_t e = a.lo; e < a.hi; ++e) (a.write ? writers : readers)[a.buf][e].push_back(pos);
    return true;
  };
  for (int t = 0; t < nt; ++t) {
    for (const Access& a : g.acc[t])
      if (!add(a, t)) return "access out of symbolic range";
    if (g.task_comb[t])
      for (const Access& a : g.comb_acc[t])
        if (!add(a, t)) return "second-phase access out of symbolic range";
  }
  for (int b = 0; b < S_COUNT; ++b)
    for (auto& v : writers[b]) {
      std::sort(v.begin(), v.end());
      v.erase(std::unique(v.begin(), v.end()), v.end());
    }
  // Dynamic state.
  std::vector<std::vector<int64_t>> ver(S_COUNT);  // step * nt + writer position, or -1
  for (int b = 0; b < S_COUNT; ++b) ver[b].assign(g.sym_size[b], -1);
  std::vector<uint32_t> flags(g.n_flag_slots, 0);
  uint64_t rng = seed;
  for (int step = 0; step < n_steps; ++step) {
    const uint32_t epoch = (uint32_t)step + 1;
    std::vector<char> ended(nt, 0), phase(nt, 0);  // phase 1: first phase running, 2: waiting for its group
    std::vector<int> group_done(ng, 0);            // tasks of the group past their first phase
    // members of ordered groups, in global order
    std::vector<std::vector<int>> members(ng);
    for (int t = 0; t < nt; ++t)
      if (g.task_group[t] >= 0 && g.group_ordered[g.task_group[t]]) members[g.task_group[t]].push_back(t);
    auto group_ready = [&](int t) {
      const int gi = g.task_group[t];
      if (!g.group_ordered[gi]) return group_done[gi] >= g.group_size[gi];
      for (int m : members[gi]) {
        if (m > t) break;
        if (phase[m] < 2 && !ended[m]) return false;
      }
      return true;
    };
    std::vector<int> qpos(g.n_cus), running(g.n_cus, -1);
    for (int cu = 0; cu < g.n_cus; ++cu) qpos[cu] = g.queue_off[cu];
    // Expected version of element e for a reader at global position pos: the last writer before
    // pos in this step (at or before pos in a second phase, which runs after the task's own first
    // phase). A batched tile's partials are read from every split of its group, earlier or later in
    // the global order: they must all be this step's.
    auto expected = [&](int b, int64_t e, int pos, bool inclusive) -> int64_t {
      const auto& w = writers[b][e];
      if (b == S_BPART || b == S_PART) return w.size() == 1 ? (int64_t)step * nt + w[0] : -2;
      auto it = inclusive ? std::upper_bound(w.begin(), w.end(), pos) : std::lower_bound(w.begin(), w.end(), pos);
      if (it != w.begin()) return (int64_t)step * nt + *(it - 1);
      if (!w.empty() && step > 0) return (int64_t)(step - 1) * nt + w.back();
      return ver[b][e] == -1 ? -1 : ver[b][e];  // written outside the graph (initial state)
    };
    auto check_reads = [&](const std::vector<Access>& as, int pos, bool inclusive, std::string& err) {
      for (const Access& a : as) {
        if (a.write) continue;
        for (int64_t e = a.lo; e < a.hi; ++e)
          if (ver[a.buf][e] != expected(a.buf, e, pos, inclusive)) {
            err = "task " + std::to_string(pos) + " read buffer " + std::to_string(a.buf) + " element " +
                  std::to_string(e) + " before its producer finished";
            return false;
          }
      }
      return true;
    };
    auto apply_writes = [&](const std::vector<Access>& as, int pos, std::string& err) {
      for (const Access& a : as) {
        if (!a.write) continue;
        for (int64_t e = a.lo; e < a.hi; ++e) {
          const auto& w = writers[a.buf][e];
          auto it = std::lower_bound(w.begin(), w.end(), pos);
          const int prev = it != w.begin() ? *(it - 1) : -1;
          // (a group's partials are written once per step and read only within it)
          for (int r : readers[a.buf][e])
            if (a.buf != S_BPART && a.buf != S_PART && r > prev && r < pos && !ended[r]) {
              err = "task " + std::to_string(pos) + " overwrote buffer " + std::to_string(a.buf) + " element " +
                    std::to_string(e) + " while task " + std::to_string(r) + " still needed it";
              return false;
            }
          ver[a.buf][e] = (int64_t)step * nt + pos;
        }
      }
      return true;
    };
    auto ready = [&](int t) {
      const int e = g.tasks[t].wait_ev;
      if (e < 0) return true;
      for (int s = g.events[e].slot0; s < g.events[e].slot0 + g.events[e].nslots; ++s)
        if (flags[s] < epoch) return false;
      return true;
    };
    auto finish = [&](int t) {  // a group's tasks without a second phase leave publishing to those with one
      ended[t] = 1;
      if (g.task_group[t] >= 0 && !g.task_comb[t]) return;
      const TaskDesc& td = g.tasks[t];
      for (int i = 0; i < td.sig_n; ++i) flags[g.sig_slots[td.sig_off + i]] = epoch;
    };
    int done = 0;
    std::vector<int> cand;
    while (done < nt) {
      cand.clear();
      for (int cu = 0; cu < g.n_cus; ++cu) {
        if (running[cu] >= 0) {
          const int t = running[cu];
          // a second phase waits until every task of its group has finished its first phase
          if (phase[t] == 2 && !group_ready(t)) continue;
          cand.push_back(cu);
        } else if (qpos[cu] < g.queue_off[cu + 1] && ready(g.queue_idx[qpos[cu]])) {
          cand.push_back(cu);
        }
      }
      if (cand.empty()) return "deadlock at step " + std::to_string(step) + " after " + std::to_string(done) + " tasks";
      const int cu = cand[sm_next(rng) % cand.size()];
      std::string err;
      if (running[cu] < 0) {
        const int t = g.queue_idx[qpos[cu]++];
        if (!check_reads(g.acc[t], t, false, err)) return err;
        phase[t] = 1;
        running[cu] = t;
      } else if (phase[running[cu]] == 1) {
        const int t = running[cu];
        if (!apply_writes(g.acc[t], t, err)) return err;
        if (g.task_group[t] >= 0) ++group_done[g.task_group[t]];
        if (g.task_comb[t]) {
          phase[t] = 2;
        } else {
          running[cu] = -1;
          finish(t);
          ++done;
        }
      } else {
        const int t = running[cu];
        running[cu] = -1;
        // an attention merge reads its own split's partial, written in its first phase
        if (!check_reads(g.comb_acc[t], t, g.tasks[t].type == T_ATTN, err)) return err;
        if (!apply_writes(g.comb_acc[t], t, err)) return err;
        finish(t);
        ++done;
      }
    }
  }
  return "";
}

// ----------------------------------------------------------------------------- test hook
// Breaks a built graph in one named way, so that tests can show the validator and the simulator
// reject it. Host graphs only; never used on a graph a kernel runs.
std::string corrupt_graph(HostGraph& g, int kind) {
  const int nt = (int)g.tasks.size();
  auto first_of = [&](int type, int layer) {
    for (int t = 0; t < nt; ++t)
      if (g.tasks[t].type == type && g.tasks[t].layer == layer) return t;
    return -1;
  };
  switch (kind) {
    case 1: {  // two tasks of one CU's queue swapped: the queue leaves the global order
      for (int cu = 0; cu < g.n_cus; ++cu)
        if (g.queue_off[cu + 1] - g.queue_off[cu] >= 2) {
          std::swap(g.queue_idx[g.queue_off[cu]], g.queue_idx[g.queue_off[cu] + 1]);
          return "";
        }
      return "no queue holds two tasks";
    }
    case 2: {  // a task waits on an event whose producers come after it (a dependency cycle)
      const int t = first_of(T_QKV, 0), p = first_of(T_DOWN, 0);
      if (t < 0 || p < 0 || g.tasks[p].sig_n < 1) return "no QKV or down task";
      const int slot = g.sig_slots[g.tasks[p].sig_off];
      for (size_t e = 0; e < g.events.size(); ++e)
        if (g.events[e].slot0 <= slot && slot < g.events[e].slot0 + g.events[e].nslots) {
          g.tasks[t].wait_ev = (int32_t)e;
          g.tasks[t].wait_slot0 = g.events[e].slot0;
          g.tasks[t].wait_nslots = g.events[e].nslots;
          return "";
        }
      return "no event";
    }
    case 3: {  // a flag slot with two writers: a second GEMV task publishes into the first one's slot
      const int t = first_of(T_OPROJ, 0);
      if (t < 0 || t + 1 >= nt || g.tasks[t + 1].type != T_OPROJ) return "no two O tasks";
      g.sig_slots[g.tasks[t + 1].sig_off] = g.sig_slots[g.tasks[t].sig_off];
      return "";
    }
    case 4: {  // a producer that never publishes: its slot has no writer
      const int t = first_of(T_GATEUP, 0);
      if (t < 0) return "no gate/up task";
      g.tasks[t].sig_n = 0;
      return "";
    }
    case 5: {  // two tiles of one stage overlap: rows written twice
      const int t = first_of(T_DOWN, 0);
      if (t < 0 || t + 1 >= nt || g.tasks[t + 1].type != T_DOWN) return "no two down tasks";
      g.tasks[t].row1 += 1;
      return "";
    }
    case 6: {  // a consumer that does not wait: an attention task's input wait removed
      const int t = first_of(T_ATTN, 0);
      if (t < 0) return "no attention task";
      g.tasks[t].wait_ev = -1;
      g.tasks[t].wait_slot0 = 0;
      g.tasks[t].wait_nslots = 0;
      return "";
    }
    case 7: {  // rows left unwritten: a stage's last tile ends early
      int t = first_of(T_LMHEAD, g.cfg.n_layers);
      if (t < 0) return "no LM-head task";
      while (t + 1 < nt && g.tasks[t + 1].type == T_LMHEAD) ++t;
      g.tasks[t].row1 -= 1;
      return "";
    }
    case 8: {  // run-time scheduling: an event's consumer range loses its last task (never queued)
      for (size_t e = 0; e < g.jit_ev_c0.size(); ++e)
        if (g.jit_ok && g.jit_ev_c1[e] - g.jit_ev_c0[e] >= 2) {
          g.jit_ev_c1[e] -= 1;
          return "";
        }
      return "no run-time scheduling tables";
    }
    case 9: {  // run-time scheduling: an event expects one producer more than signal it (never complete)
      for (size_t e = 0; e < g.jit_ev_n.size(); ++e)
        if (g.jit_ok && g.jit_ev_c1[e] > g.jit_ev_c0[e]) {
          g.jit_ev_n[e] += 1;
          return "";
        }
      return "no run-time scheduling tables";
    }
    default:
      return "unknown corruption kind";
  }
}

uint64_t graph_hash(const HostGraph& g) {
  uint64_t h = 0xcbf29ce484222325ULL;
  auto mix = [&](const void* p, size_t n) {
    const unsigned char* c = (const unsigned char*)p;
    for (size_t i = 0; i < n; ++i) {
      h ^= c[i];
      h *= 0x100000001b3ULL;
    }
  };
  mix(g.tasks.data(), g.tasks.size() * sizeof(TaskDesc));
  mix(g.queue_off.data(), g.queue_off.size() * 4);
  mix(g.queue_idx.data(), g.queue_idx.size() * 4);
  mix(g.events.data(), g.events.size() * sizeof(EventDesc));
  mix(g.sig_slots.data(), g.sig_slots.size() * 4);
  mix(g.geoms, sizeof(g.geoms));
  return h;
}

}  // namespace mk
