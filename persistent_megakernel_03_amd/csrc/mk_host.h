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
enum SymBuf : int32_t { S_X, S_Q, S_KVCUR, S_PART, S_O, S_H, S_LOGITS, S_AMAX, S_CTX, S_TOKOUT, S_COUNT };

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
  int n_attn_groups = 0;  // (layer, sequence, KV head) groups whose attention splits are merged
  int n_lm_parts = 0;
  int max_queue = 0;
  int64_t lds_bytes = 0;
  GemvGeom geoms[G_COUNT]{};
  std::vector<TaskDesc> tasks;               // global topological order
  std::vector<std::vector<Access>> acc;      // per task
  std::vector<std::vector<Access>> comb_acc; // ATTN tasks: accesses of the merge the last split performs
  std::vector<int32_t> queue_off, queue_idx;
  std::vector<EventDesc> events;
  std::vector<int32_t> sig_slots;
  int32_t n_flag_slots = 0;
  WeightLayout wl{};
  ScratchLayout sl{};
  int64_t sym_size[S_COUNT]{};
};

// Builds the graph; returns an empty string on success, else the reason.
std::string build_graph(const mk_model_config& cfg, int n_cus, HostGraph& g);
std::string validate_graph(const HostGraph& g);
std::string simulate_graph(const HostGraph& g, uint64_t seed, int n_steps);
uint64_t graph_hash(const HostGraph& g);
GemvGeom choose_geom(int K);

// Packed-row bookkeeping shared with the weight re-layout.
// QKV rows are grouped per KV head g: the G query heads of g, then k head g, then v head g.
// Within a head, rows are pair-interleaved: packed 2i -> dim i, packed 2i+1 -> dim i + dh/2.
// gate/up rows alternate: packed 2f = gate row f, 2f + 1 = up row f.
inline int qkv_rows(const mk_model_config& c) { return (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim; }

}  // namespace mk
