// Host-side graph object: the builder's output plus the symbolic read/write sets
// the validator and the simulator check. Not visible to device code.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_graph.h"

namespace mk {

// Symbolic buffers for the validator/simulator (element granularity).
// S_BPART has one element per column split of a batched GEMV tile (the split's whole partial block).
enum SymBuf : int32_t { S_X, S_Q, S_KVCUR, S_PART, S_O, S_H, S_LOGITS, S_AMAX, S_CTX, S_TOKOUT, S_BPART, S_COUNT };

struct Access {
  int32_t buf;
  int64_t lo, hi;  // element range [lo, hi)
  int32_t write;   // 0 = read, 1 = write
};

struct HostGraph {
  mk_model_config cfg{};
  int n_cus = 0;
  int splits = 1;
  int max_pos = 0;
  int n_attn_groups = 0;  // (layer, sequence, KV head) segments of attention
  int attn_tasks = 0;     // attention tasks per layer  // (layer, sequence, KV head) groups whose attention splits are merged
  int n_lm_parts = 0;
  int max_queue = 0;
  int64_t lds_bytes = 0;
  int64_t stage2_off = 0;  // see KernelParams::stage2_off
  GemvGeom geoms[G_COUNT]{};
  std::vector<TaskDesc> tasks;               // global topological order
  std::vector<std::vector<Access>> acc;      // per task
  std::vector<std::vector<Access>> comb_acc; // accesses of a task's second phase (below)
  // Split groups: the attention splits of one (layer, sequence, KV head), or the column splits of
  // one batched GEMV tile. A task with a second phase (task_comb) runs it only after every task of
  // its group has finished its first phase: the last attention split merges the group's partials;
  // every split of a batched tile sums the group's partials for its share of the rows.
  std::vector<int32_t> task_group;           // per task: group index or -1
  std::vector<char> task_comb;               // per task: has a second phase
  std::vector<int32_t> group_size;           // per group
  // per group: 1 = a member's second phase waits only for the members before it in the global order
  // (attention merges read earlier tasks' partials); 0 = for all members (batched column splits)
  std::vector<char> group_ordered;
  int max_tile_groups = 0;                   // batched: most 16-row groups in one tile
  std::vector<int32_t> queue_off, queue_idx;
  std::vector<EventDesc> events;
  std::vector<int32_t> sig_slots;
  int32_t n_flag_slots = 0;
  WeightLayout wl{};
  ScratchLayout sl{};
  int64_t sym_size[S_COUNT]{};
  // Dynamic scheduling (one-sequence graphs): per task, the event its completion counts toward (-1:
  // none); per event, its producer count and its consumer tasks [c0, c1), contiguous in the global
  // order; the tasks ready when a step starts are [0, jit_n0).
  std::vector<int32_t> jit_task_ev, jit_ev_n, jit_ev_c0, jit_ev_c1;
  int32_t jit_n0 = 0;
  bool jit_ok = false;
};

// Builds the graph; returns an empty string on success, else the reason.
std::string build_graph(const mk_model_config& cfg, int n_cus, HostGraph& g);
std::string validate_graph(const HostGraph& g);
std::string simulate_graph(const HostGraph& g, uint64_t seed, int n_steps);
uint64_t graph_hash(const HostGraph& g);
// Test hook: breaks the graph in one of the ways mk_graph_corrupt names; "" on success.
std::string corrupt_graph(HostGraph& g, int kind);
GemvGeom choose_geom(int K);
GemvGeom choose_geom_batched(int K);

// Bytes of a GEMV task's packed tile.
inline int64_t task_tile_bytes(const GemvGeom& q, const TaskDesc& t) {
  if (q.mfma) return (int64_t)((t.row1 - t.row0 + 15) / 16) * (t.a2 >> 16) * 1024;
  return (int64_t)((t.row1 - t.row0 + q.rg - 1) / q.rg) * (q.fp8 ? q.S / 2 : q.S) * 1024;
}

// Packed-row bookkeeping shared with the weight re-layout.
// QKV rows are grouped per KV head g: the G query heads of g, then k head g, then v head g.
// Within a head, rows are pair-interleaved: packed 2i -> dim i, packed 2i+1 -> dim i + dh/2.
// gate/up rows alternate: packed 2f = gate row f, 2f + 1 = up row f.
inline int qkv_rows(const mk_model_config& c) { return (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim; }

}  // namespace mk
