// Task-graph data structures shared by the host builder (mk_graph.cpp), the host
// runtime (mk_api.cpp) and the megakernel (mk_kernel.hip).
//
// The decode step is split into tasks, each run by one workgroup (one CU). A
// task waits on at most one event and, when done, publishes its epoch number
// into one or more flag slots. An event is a contiguous range of flag slots,
// one per producer task. It is satisfied for step `epoch` once every slot
// holds a value >= epoch. So no counter is ever reset, and a slot has
// exactly one writer. This follows the pages' events with counters and
// thresholds ("LLMs in einen MegaKernel kompilieren", "Ereignisbasierte
// Ausführung"). A count of producers becomes a set of per-producer flags, so
// that no two CUs contend for one atomic.
#pragma once
#include <stdint.h>

namespace mk {

enum TaskType : int32_t {
  T_QKV = 1,     // RMSNorm + QKV GEMV (+bias) + RoPE + KV append
  T_ATTN = 2,    // one split of paged GQA attention; the last split of a (seq, kv head) also merges
  T_OPROJ = 3,   // O projection + residual
  T_GATEUP = 4,  // RMSNorm + gate/up GEMV + SiLU(gate) * up
  T_DOWN = 5,    // down projection + residual
  T_LMHEAD = 6,  // final RMSNorm + LM head GEMV + partial argmax
  T_ARGMAX = 7,  // argmax over the LM-head partials, token out, context length + 1
};

// One sequence: 1 KB weight units per wave that a GEMV task stages in LDS (by DMA) on top of the
// units it holds in registers, all issued before the task waits for its input. The stage is a
// static LDS array of 8 waves x kStageUnits KB beside the dynamic working set.
constexpr int kStageUnits = 10;

// Attention: by default the layer's cache blocks are cut over at most one task per kAttnMinBlocks
// blocks. With 1, every attention task gets blocks once there are as many blocks as tasks: on
// MI355X the extra merges cost less than fewer, longer tasks.
constexpr int kAttnMinBlocks = 1;
// Several sequences: the blocks are cut by cost instead, each block costing 1 and each segment start
// (a new (sequence, KV head) piece for a task to begin) kAttnPieceBlocks more. On MI355X a piece costs
// a query poll that waits behind its first row loads, the wave merges and a partial write: with 16
// sequences of mixed lengths, about 24 blocks' streaming.
constexpr int kAttnPieceBlocks = 24;
constexpr int kStageBytes = 8 * kStageUnits * 1024;
// One sequence, rows of 4096 inputs: a second stage of kStage2Units units per wave in the dynamic
// working set, which such tasks use only in part (their input vector is 16 KB). With it a wave holds
// 32 units (four rows) before its input arrives, all of a QKV task's share on 192 CUs.
constexpr int kStage2Units = 6;
// Size of the static device array that holds a step's working memory for the entry point that
// allocates nothing (mk_decode_step_static); larger graphs are refused there.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;

// Geometry of one GEMV operand in the packed (streaming) layout. A row of K bf16 values is
// P = K/8 pieces of 16 bytes. A "unit" is 1 KB: 64 lanes x 16 B.
//  mfma == 0 (one sequence): rows go in groups of rg = 64/lpr rows; a group is S units. In unit u
//    of a group, lane l holds piece u*lpr + l%lpr of row l/lpr.
//  mfma == 1 (batched): rows go in groups of 16; unit u of a group covers columns [32u, 32u + 32)
//    and lane l holds piece 4u + l/16 of row l%16: the row operand of one 16x16x32 bf16 MFMA.
//    A task streams only the units of its own column range (see TaskDesc); S is the number of
//    units that cover K.
// Pieces past P are zero.
struct GemvGeom {
  int32_t K, P, lpr, rg, S;
  int32_t mfma;
  // FP8 weights: a 1 KB unit holds 16 codes per lane, the lane's pieces of two consecutive bf16-layout
  // units (S is then even: a row group streams S / 2 units)
  int32_t fp8;
  int32_t pad;
};
enum GeomIndex : int32_t { G_QKV = 0, G_O = 1, G_GU = 2, G_D = 3, G_LM = 4, G_COUNT = 5 };

struct TaskDesc {       // 64 bytes; read with scalar loads
  int32_t type;
  int32_t layer;
  int32_t wait_ev;      // event index, or -1
  int32_t sig_off;      // this task's flag slots: sig_slots[sig_off .. sig_off + sig_n)
  int32_t sig_n;
  int32_t row0, row1;   // GEMV: packed output rows [row0, row1)
  int32_t geom;         // GEMV: GeomIndex
  int64_t wofs;         // GEMV: byte offset of the tile in the packed weights
  // ATTN: a2 = task index within its layer, a3 = a unique id | ARGMAX: a0 = seq | LMHEAD: a0 = part.
  // Batched GEMV (several sequences): the tile's rows are split over kS tasks by columns.
  //   a1 = word offset of the tile's partial sums in KernelParams::bpt (kS > 1),
  //   a2 = first column unit | units << 16 (units of 32 columns),
  //   a3 = split index | kS << 8.
  // One-sequence GEMV with FP8 weights: a1 = index of the task's first row in the row-scale array.
  int32_t a0, a1, a2, a3;
  int32_t wait_slot0, wait_nslots;  // the wait event's flag slots (copied from events[wait_ev])
};
static_assert(sizeof(TaskDesc) == 64, "TaskDesc is 64 bytes");

struct EventDesc {
  int32_t slot0, nslots;
};

// Byte offsets of the regions inside the caller's scratch buffer.
struct ScratchLayout {
  int64_t tasks, queue_off, queue_idx, events, sig_slots, geoms, rope;
  int64_t flags, err;
  // tagged activations (64-bit words: value bits | step epoch << 32), one buffer per layer
  int64_t xt, qt, kvt, ot, ht, pt;
  int64_t tokt;                      // [max_seqs]: the token each sequence feeds into the next step
  int64_t bpt;                       // batched GEMV: per-tile partial sums of each column split
  int64_t tagged_begin, tagged_end;  // byte range holding all tagged buffers
  int64_t amax, tokbuf, tokout, pools;
  // batched graphs, chunked prefill: the rows' page table (copies of one sequence's row), their context
  // lengths (16 per chunk), the rows' logits and tokens
  int64_t pf_ptab = -1, pf_ctx = -1, pf_logits = -1, pf_tok = -1;
  // dynamic scheduling: the read-only tables (task -> event [T], event -> producers, first and end
  // consumer [3][E]) and the working memory a launch resets (ready-queue head and tail, per-event
  // counts [E], the queue of task indices [T])
  int64_t jit_tab = -1, jit_work = -1;
  int64_t total;
};

// Byte offsets inside the caller's weights buffer (after the packed tiles).
struct WeightLayout {
  int64_t packed_bytes;  // tiles of every GEMV stage
  int64_t embed;         // natural [V, d] copy for the embedding gather
  int64_t norms;         // [L][2][d] (attn, ffn) then final [d]
  int64_t bias;          // packed-QKV-order bias [L][Nqkv] (when qkv_bias)
  int64_t scales;        // FP8 weights: fp32 scale 2^e of every packed GEMV row, stage after stage
  int64_t n_scale_rows;
  int64_t total;
};

// Device error word layout (uint32 slots in scratch).
enum ErrSlot : int32_t { E_CODE = 0, E_INFO0 = 1, E_INFO1 = 2, E_ABORT = 3, E_COUNT = 16 };
enum ErrCode : uint32_t { ERR_NONE = 0, ERR_TOKEN = 1, ERR_PAGE = 2, ERR_TIMEOUT = 3, ERR_CTX = 4, ERR_NAN = 5 };

// One task's timestamps (s_memrealtime, 100 MHz), written when tracing is on.
struct TraceRec {
  uint64_t t_queue;   // the CU reached the task in its queue
  uint64_t t_ready;   // its inputs were all present
  uint64_t t_streamed;  // its own streaming ended: GEMV before the epilogue, attention before the partials
  uint64_t t_done;    // its outputs were published
  uint16_t cu;        // the workgroup (queue) index
  uint8_t type;       // TaskType
  uint8_t layer;      // layer index (n_layers for the LM head and argmax), mod 256
  uint32_t epoch;
  uint32_t xcc;       // the XCD the workgroup ran on (hardware register)
  uint32_t step;      // the step's index within its launch
};
static_assert(sizeof(TraceRec) == 48, "TraceRec is 48 bytes");

// Everything the megakernel reads, passed by value.
struct KernelParams {
  const TaskDesc* tasks;
  const int32_t* queue_off;   // [n_cus + 1]
  const int32_t* queue_idx;
  const EventDesc* events;
  const int32_t* sig_slots;
  const GemvGeom* geoms;
  const float* rope;          // [max_pos][dh/2][2] (cos, sin)
  uint32_t* flags;
  uint32_t* err;
  const uint8_t* wpacked;     // packed tiles
  const uint16_t* embed;      // natural embedding [V, d]
  const uint16_t* norms;      // [L][2][d] + final [d]
  const uint16_t* bias;       // packed QKV bias or nullptr
  uint16_t* const* kpool;     // [L] device array of per-layer K pool pointers
  uint16_t* const* vpool;
  const int32_t* page_table;  // [max_seqs][max_blocks]
  int32_t* ctx_lens;          // [max_seqs]
  // Activations handed from CU to CU within a step, as tagged 64-bit words (value bits in the low
  // half, the step epoch in the high half), one buffer per layer so every word is written once per step.
  uint64_t* xt;               // [L][2][max_seqs][d] residual stream after O-proj (0) and after down-proj (1)
  uint64_t* qt;               // [L][max_seqs][hq*dh] rotated queries
  uint64_t* kvt;              // [L][max_seqs][2][hk][dh/2] the current position's key and value (bf16 pairs)
  uint64_t* ot;               // [L][max_seqs][hq*dh] attention output
  uint64_t* ht;               // [L][max_seqs][f] SwiGLU output
  uint64_t* pt;               // [L][attention task][2][G][dh + 2] attention partials (m, l, unnormalised o)
  uint64_t* bpt;              // batched GEMV tiles: [split][16-row group][64 lanes][4] partial sums + 64 words
                              // (sums of squares per sequence), one block per tile (see TaskDesc)
  float* logits;              // [max_seqs][V]
  uint64_t* amax;             // [max_seqs][n_lm_parts] packed argmax keys
  const int32_t* tokens_in;   // [max_seqs]: the first step's tokens
  int32_t* tokens_out;        // [n_steps][n_active]: each step's greedy tokens
  uint64_t* tokt;             // [max_seqs] tagged: the token each sequence feeds into the next step
  int32_t n_layers, d, hq, hk, dh, f, vocab;
  float eps;
  int32_t max_seqs, n_active, max_blocks, num_blocks, block_size, splits, n_lm_parts, max_pos;
  uint32_t epoch;             // the first step's epoch; step i runs with epoch + i
  int32_t n_steps;            // steps this launch runs, each feeding its tokens to the next
  uint32_t watchdog_ticks;    // s_memrealtime ticks (100 MHz) a wait may spin before the kernel aborts
  int32_t max_queue;          // longest per-CU queue (its descriptors are staged in LDS)
  int32_t attn_tasks;         // attention tasks per layer (they cut the layer's KV blocks evenly)
  int32_t task_lo, task_hi;   // this launch runs the tasks [task_lo, task_hi) of the global order
  int32_t attn_min_blocks;    // cache blocks per attention task at least (fewer tasks get blocks)
  int32_t prefill;            // batched graphs: 1 = the rows are consecutive positions of one sequence
  int32_t fp8_weights;        // 1: GEMV tiles hold E4M3 codes, row r's products scale by wscale[r]
  int32_t stage2_off;         // one sequence: byte offset of the second weight stage in the working set, or 0
  const int32_t* jit_tab;     // dynamic scheduling tables (see ScratchLayout::jit_tab), or nullptr
  int32_t* jit_work;          // dynamic scheduling working memory
  int32_t n_events;
  const float* wscale;        // FP8 weights: 2^e of every packed GEMV row (TaskDesc::a1 indexes it)
  TraceRec* trace;            // per-task timestamps of the last step, or nullptr
};

// Arguments of the weight re-layout kernel: one stage's tasks [task0, task0 + ntasks), whose
// tiles are contiguous in the packed buffer.
enum RepackKind : int32_t { RK_PLAIN = 0, RK_QKV = 1, RK_GU = 2 };
struct RepackArgs {
  const TaskDesc* tasks;  // device copy of the task array
  int32_t task0, ntasks;
  GemvGeom gm;
  int32_t kind;
  const uint16_t* w0;     // plain: W; QKV: wq; gate/up: wg
  const uint16_t* w1;     // QKV: wk; gate/up: wu
  const uint16_t* w2;     // QKV: wv
  int32_t G, dh;
  uint8_t* out;           // packed weights base
  float* scales;          // FP8 weights: the row-scale array, and the index of the stage's first row in it
  int32_t scale0;
};

}  // namespace mk
