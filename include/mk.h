/*
 * mk.h — C ABI of a persistent decode megakernel for AMD MI355X (gfx950).
 *
 * The library runs the per-token decode step of a Llama-style decoder (RMSNorm,
 * QKV projection, rotary embedding with KV-cache append, grouped-query
 * attention, output projection, SwiGLU FFN, LM head and argmax) as ONE
 * persistent kernel. The kernel's work is a fine-grained task graph.
 *   - A host-side builder splits every operator into per-CU tiles.
 *   - Tiles are joined by events: arrays of per-producer epoch flags.
 *   - Each workgroup walks its own task queue: it waits on a task's event,
 *     runs the tile and publishes its flag.
 * This is the design of the Mirage Persistent Kernel ("LLMs in einen
 * MegaKernel kompilieren": "Part 1. Compiler", "Part 2. Laufzeit", "Worker",
 * "Ereignisbasierte Ausführung"; "MPK: A Compiler and Runtime for
 * Mega-Kernelizing Tensor Programs", analogies 1–3), re-made for one MI355X.
 *
 * Conventions
 *   - Every function returns mk_status: 0 = MK_OK, < 0 = error. No C++
 *     exception crosses this boundary. mk_last_error() returns the calling
 *     thread's last message.
 *   - The caller allocates ALL device memory (e.g. with PyTorch). The
 *     library borrows the pointers bound by mk_bind_memory for the life of
 *     the context and never frees them. It owns only host structures.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   - Device-side errors are latched in a device error word: a token id,
 *     page index or context length out of range, or a wait that exceeds
 *     the watchdog (MK_WATCHDOG_US, default 2 s, read at mk_create). The
 *     next synchronising call (mk_read_logits, mk_sync_check) reports them
 *     and clears the word. After a watchdog expiry it also resets the
 *     event flags, so the context can decode again.
 *   - Weights are bf16. All activations are fp32. K/V caches are bf16.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mk_status;
#define MK_OK 0
#define MK_ERR_INVALID_ARG (-1)     /* a NULL pointer, a negative size, an unknown tensor name */
#define MK_ERR_SHAPE (-2)           /* a config or tensor shape the library cannot run */
#define MK_ERR_STATE (-3)           /* call out of order (e.g. decode before weights are loaded) */
#define MK_ERR_HIP (-4)             /* a HIP runtime call failed; mk_last_error() names it */
#define MK_ERR_DEVICE_TIMEOUT (-5)  /* a device-side wait exceeded the watchdog; results are invalid */
#define MK_ERR_DEVICE_FAULT (-6)    /* the device saw a token id, page index or context length out of range, or a NaN logit */
#define MK_ERR_UNSUPPORTED (-7)     /* a valid request this build does not implement */

typedef struct mk_ctx mk_ctx; /* opaque, owned by the library */

/* Model and cache shape.
 *   - All weights are bf16 PyTorch tensors in [out, in] row-major layout.
 *   - tied_embeddings: the LM head reuses the embedding matrix.
 *   - qkv_bias: q, k and v projections have a bias.
 *   - max_seqs: the largest batch a decode step may carry (1..16).
 *   - block_size: KV positions per cache block. Must be 16.
 *   - max_blocks_per_seq: columns of the page table.
 *   - num_blocks: blocks in each layer's K pool and in each layer's V pool.
 *   - attn_splits: KV splits per (sequence, KV head). 0 = chosen from
 *     max_blocks_per_seq. The layer's attention tasks are at most
 *     max_seqs * n_kv_heads * attn_splits (and at most one per compute unit).
 *   - attn_min_blocks: each step cuts its cache blocks over at most
 *     ceil(blocks / attn_min_blocks) of those tasks (fewer tasks, fewer
 *     merges); 0 = 1, every task gets blocks once there are enough.
 *     With max_seqs > 1 the cut is by cost: each (sequence, KV head)
 *     segment start counts as 24 blocks more, so a task that begins
 *     several segments gets fewer blocks (possibly none).
 *   - prefill_rows: one-sequence contexts only (0 when max_seqs > 1). 0 or 1:
 *     mk_prefill runs the prompt one decode step per token. 2..16: the
 *     context also holds the batched (matrix-core) task graph for that many
 *     rows, and mk_prefill runs the prompt through it that many positions per
 *     step; its weights and working memory are counted by mk_workspace_size
 *     (about twice the weight bytes). Needs d_model to be a multiple of 32.
 *   - weight_format: MK_WEIGHTS_BF16 (0), or MK_WEIGHTS_FP8_E4M3 (1): weight-
 *     only quantisation of every GEMV matrix ("LLM高速化勉強会資料", slide 33:
 *     fewer bits per weight, fewer bytes per step; slide 34: products
 *     accumulate in a wider format). mk_load_weights quantises the bf16
 *     tensors on the device: each output row is one block with a power-of-two
 *     scale 2^e, e the smallest integer with max |w| <= 448 * 2^e (clamped to
 *     [-100, 100], 0 for a zero row), and each weight becomes the OCP E4M3
 *     code nearest to w * 2^-e (ties to an even mantissa). The step then
 *     computes with decode(code) * 2^e, exactly, accumulating in fp32. The
 *     embedding table, norm gains and biases stay bf16. One-sequence contexts
 *     without prefill_rows only. */
typedef struct {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, d_ffn, vocab;
  float rms_eps, rope_theta;
  int32_t tied_embeddings, qkv_bias;
  int32_t max_seqs, block_size, max_blocks_per_seq, num_blocks;
  int32_t attn_splits;
  int32_t attn_min_blocks;
  int32_t prefill_rows;
  int32_t weight_format;
} mk_model_config;
#define MK_WEIGHTS_BF16 0
#define MK_WEIGHTS_FP8_E4M3 1

/* One weight tensor for mk_load_weights.
 *   - name: "embed", "final_norm", "lm_head", or "layers.<l>.<t>" with t in
 *     attn_norm, wq, wk, wv, bq, bk, bv, wo, ffn_norm, wg, wu, wd.
 *   - ptr: device pointer to the bf16 values in [out, in] row-major order.
 *   - numel: number of elements. It must match the config. */
typedef struct {
  const char* name;
  const void* ptr;
  int64_t numel;
} mk_tensor;

/* Validate `cfg` and build the task graph (host only, deterministic).
 * `device` is the HIP device ordinal. The graph is sized for that device's
 * compute-unit count. *out receives the new context.
 * The builder refines every operator into per-CU tasks joined by events ("LLMs
 * in einen MegaKernel kompilieren", "Part 1. Compiler"; "MPK: A Compiler and
 * Runtime for Mega-Kernelizing Tensor Programs", analogy 2).
 * Errors: MK_ERR_INVALID_ARG, MK_ERR_SHAPE, MK_ERR_HIP, MK_ERR_UNSUPPORTED
 * (the device lacks cooperative launch, or one workgroup per CU does not fit). */
mk_status mk_create(const mk_model_config* cfg, int device, mk_ctx** out);

/* Like mk_create, but builds the graph for `n_cus` compute units without
 * touching a GPU. Such a context serves only mk_workspace_size and the graph
 * inspection calls below. Any call that needs a device returns MK_ERR_STATE. */
mk_status mk_create_host(const mk_model_config* cfg, int n_cus, mk_ctx** out);

/* Bytes the caller must allocate before mk_bind_memory. The KV pools are the
 * block-managed cache of "LLM高速化勉強会資料", slide 17 (PagedAttention); a
 * pool's size follows the deck's KV-cache size formula (slide 10).
 *   - weights_bytes: one device buffer for the re-laid-out weights.
 *   - kv_pool_bytes: bytes of EACH per-layer K pool and EACH per-layer V
 *     pool, laid out [num_blocks, n_kv_heads, block_size, head_dim] bf16.
 *   - scratch_bytes: one device buffer for activations, partial results,
 *     event flags, the task graph and the rotary table.
 * Alignment: every buffer must be 256-byte aligned. */
mk_status mk_workspace_size(const mk_ctx* ctx, size_t* weights_bytes, size_t* kv_pool_bytes, size_t* scratch_bytes);

/* Bind caller-owned device memory. All pointers are device pointers. The KV
 * cache keeps every earlier position's keys and values for reuse ("Crear desde
 * cero un motor de inferencia para LLM usando C++ y CUDA", section 1.1), in
 * 16-position blocks named by a page table ("LLM高速化勉強会資料", slide 17).
 *   - d_k_pools, d_v_pools: HOST arrays of n_layers device pointers.
 *   - d_page_table: [max_seqs, max_blocks_per_seq] int32. Logical position
 *     p of sequence s is stored in block d_page_table[s][p / 16] at offset
 *     p % 16. The table is shared by all layers.
 *   - d_ctx_lens: [max_seqs] int32, the number of positions already cached
 *     per sequence. A decode step reads it and increments it for every
 *     sequence it runs.
 *   - d_logits: [max_seqs, vocab] fp32. Each step writes it.
 * Uploads the graph and the rotary table into scratch (synchronous) and
 * resets the event flags. The caller fills the page table and the context
 * lengths. */
mk_status mk_bind_memory(mk_ctx* ctx, void* d_weights, void* const* d_k_pools, void* const* d_v_pools,
                         void* d_scratch, int32_t* d_page_table, int32_t* d_ctx_lens, float* d_logits);

/* Copy the model weights into the bound weights buffer, re-laid out into
 * the per-tile streaming order (loading a model means filling its blocks with
 * stored weights: "Crear desde cero un motor de inferencia para LLM usando C++
 * y CUDA", section 1). Runs kernels on `stream`. The source
 * tensors may be freed once the stream has passed this call. Every tensor
 * the config needs must be present.
 * Errors: MK_ERR_INVALID_ARG (unknown or duplicate name), MK_ERR_SHAPE
 * (wrong numel), MK_ERR_STATE (memory not bound). */
mk_status mk_load_weights(mk_ctx* ctx, const mk_tensor* ts, int n, void* stream);

/* One decode step for sequences 0..n_seqs-1: one new token per sequence
 * against its KV cache ("Crear desde cero un motor de inferencia para LLM
 * usando C++ y CUDA", section 1.1, the decode phase).
 * d_tokens_in and d_tokens_out are [n_seqs] int32 device arrays (they may be
 * the same array).
 *   - Sequence s takes token d_tokens_in[s] at position d_ctx_lens[s].
 *   - Its key and value are appended at that position.
 *   - It attends to positions 0..d_ctx_lens[s].
 *   - It writes its logits and greedy token (argmax, lowest index on ties).
 *   - d_ctx_lens[s] is incremented.
 * Asynchronous: one kernel launch on `stream` (one workgroup per compute
 * unit, all resident at once on a device running nothing else; with the
 * environment variable MK_COOPERATIVE_LAUNCH set, a cooperative launch that
 * the runtime guarantees co-resident), with no host synchronisation. n_seqs
 * must be at most max_seqs. */
mk_status mk_decode_step(mk_ctx* ctx, const int32_t* d_tokens_in, int n_seqs, int32_t* d_tokens_out, void* stream);

/* n_steps greedy decode steps in ONE kernel launch: the megakernel stays
 * resident and each step's argmax feeds the next step's embedding lookup on
 * the device, so no launch separates the tokens ("LLMs in einen MegaKernel
 * kompilieren", "Überblick und Vorteile des MegaKernel-Ansatzes": no repeated
 * kernel launches; "MPK: A Compiler and Runtime for Mega-Kernelizing Tensor
 * Programs", analogy 1).
 *   - d_tokens_in: [n_seqs] int32, the first step's tokens (device memory).
 *   - d_tokens_out: [n_steps, n_seqs] int32 device array; row i receives
 *     step i's greedy tokens. It must not overlap d_tokens_in.
 *   - Step i of sequence s runs at position d_ctx_lens[s] + i; afterwards
 *     d_ctx_lens[s] has grown by n_steps.
 *   - d_logits holds the LAST step's logits.
 * The results are those of n_steps calls of mk_decode_step, each fed the
 * previous call's tokens (same graph, same arithmetic, bit for bit).
 * The launch is cooperative, so the runtime guarantees that every workgroup is
 * resident. Asynchronous. Errors: MK_ERR_INVALID_ARG (n_steps < 1 or above
 * 65536, n_seqs out of range, NULL arrays), MK_ERR_STATE. A position past the
 * cache is reported by the next synchronising call, like mk_decode_step's. */
mk_status mk_decode_n(mk_ctx* ctx, const int32_t* d_tokens_in, int n_seqs, int n_steps, int32_t* d_tokens_out,
                      void* stream);

/* mk_decode_step for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same step, but the working memory it writes (event flags, tagged
 * activations, attention and column-split partials, argmax keys) lives in the
 * library's static device array of 64 MiB per GPU instead of the bound scratch
 * buffer. It allocates nothing and copies nothing from the host: it clears
 * that array's flags and tagged buffers with a fill kernel on `stream`, then
 * launches the step. The read-only task graph, rotary table and pool pointers
 * come from the bound scratch buffer (uploaded by mk_bind_memory), and device
 * errors are latched in the context's own error word, reported by the next
 * synchronising call as for mk_decode_step.
 *   - Arguments, results and context-length update: as mk_decode_step.
 *   - Every call on one GPU shares that GPU's array; calls whose launches
 *     overlap on one GPU (two streams, two threads) race and must not be made.
 *   - The array keeps the last call's contents; each call clears what must
 *     start at zero, so calls from different contexts may alternate.
 * Errors: as mk_decode_step, plus MK_ERR_SHAPE when the graph's scratch
 * layout (mk_workspace_size's scratch_bytes) exceeds 64 MiB. */
mk_status mk_decode_step_static(mk_ctx* ctx, const int32_t* d_tokens_in, int n_seqs, int32_t* d_tokens_out,
                                void* stream);

/* The same decode step as mk_decode_step with the tasks scheduled at run time
 * instead of ahead of time (the just-in-time mode of "MPK: A Compiler and
 * Runtime for Mega-Kernelizing Tensor Programs", analogy 3; the event-driven
 * runtime of "LLMs in einen MegaKernel kompilieren", "Part 2. Runtime"). No
 * workgroup owns a queue: each takes the next slot of one device-wide ready
 * queue and runs the task that lands there. A task's completion counts toward
 * the event it signals; the completion that finishes an event appends the
 * tasks that wait on it. The tasks and their arithmetic are those of
 * mk_decode_step, so tokens and logits are identical; only which CU runs a
 * task, and when, differ.
 *   - One-sequence contexts with bf16 weights; n_seqs must be 1.
 *   - Arguments and errors: as mk_decode_step, plus MK_ERR_UNSUPPORTED for
 *     other contexts. A wait on an empty queue slot is watched like every
 *     other wait. Asynchronous. */
mk_status mk_decode_step_dynamic(mk_ctx* ctx, const int32_t* d_tokens_in, int n_seqs, int32_t* d_tokens_out,
                                 void* stream);

/* The same decode step as mk_decode_step, launched as one kernel dispatch per dependency stage
 * (QKV, attention, O projection, gate/up and down of each layer, then the LM head and the argmax):
 * the same kernel, task graph and arithmetic, so the results are identical. Each dispatch runs only
 * its stage's tasks, so a stage starts only after the previous one has fully drained. This is the
 * operator-by-operator execution the persistent kernel replaces ("LLMs in einen MegaKernel
 * kompilieren", "Part 1. Compiler": one kernel per operator in conventional designs); it exists to measure
 * the pass-to-pass gaps that the single launch removes. Asynchronous, same arguments and errors as
 * mk_decode_step; mk_graph_info.n_stages dispatches per step. */
mk_status mk_decode_step_staged(mk_ctx* ctx, const int32_t* d_tokens_in, int n_seqs, int32_t* d_tokens_out,
                                void* stream);

/* Prefill: build sequence `seq`'s KV cache from the prompt (the prefill phase
 * of "LLM高速化勉強会資料", slide 9; "Crear desde cero un motor de inferencia
 * para LLM usando C++ y CUDA", section 1.1), appending the n_tokens host tokens
 * h_tokens at the sequence's current length (d_ctx_lens[seq]).
 *   - Batched contexts (max_seqs > 1), and one-sequence contexts with
 *     prefill_rows > 1: chunked prefill (slide 43 of the deck, "Chunked
 *     Prefill"; several prompt tokens at once for a shorter time to the first
 *     token, "Crear desde cero ...", section 4). Each step of the batched
 *     graph carries R = max_seqs (or prefill_rows) consecutive positions as
 *     its rows: the GEMVs become R-row matrix-core tiles that read the weights
 *     once for all R positions, and row i attends only to the positions up to
 *     its own (causal masking; the masked part is never visited, "Hạt nhân là
 *     gì"). The other sequences' caches, lengths and logits are untouched.
 *     The call synchronises the stream and reports any device error.
 *   - One-sequence contexts with prefill_rows 0 or 1: one decode step per
 *     prompt token, asynchronous like mk_decode_step.
 * Afterwards d_ctx_lens[seq] has grown by n_tokens, the logits row of `seq`
 * holds the last prompt token's logits and, when d_token_out is not NULL, it
 * receives the greedy token after the prompt.
 * Errors: MK_ERR_INVALID_ARG (seq out of range, a token outside [0, vocab),
 * the prompt running past the sequence's cache); device errors as for
 * mk_sync_check. */
mk_status mk_prefill(mk_ctx* ctx, int seq, const int32_t* h_tokens, int n_tokens, int32_t* d_token_out,
                     void* stream);

/* The FP8 codes a context with weight_format MK_WEIGHTS_FP8_E4M3 streams for
 * one matrix, read back from its tiles into natural layout (inspection, for
 * checking the quantiser; the format is described at weight_format).
 *   - name: "layers.<l>.wq" (wk, wv, wo, wg, wu, wd), or "lm_head" ("embed"
 *     for a tied head).
 *   - h_codes: host, [out_rows, in] uint8 E4M3 codes; h_exps: host,
 *     [out_rows] int32, each row's scale exponent e (scale 2^e).
 * Synchronises `stream`. Errors: MK_ERR_INVALID_ARG (unknown name),
 * MK_ERR_STATE (weights not loaded, or not FP8). */
mk_status mk_read_fp8_weights(mk_ctx* ctx, const char* name, uint8_t* h_codes, int32_t* h_exps, void* stream);

/* Copy the last step's logits of sequence `seq` (n <= vocab floats) to host
 * memory. (No passage: the boundary's own, for parity checks.) Synchronises
 * `stream`. Returns the device error word if one is set. */
mk_status mk_read_logits(mk_ctx* ctx, int seq, float* h_dst, size_t n, void* stream);

/* Synchronise `stream` and report the device error word (MK_OK if clear). The
 * pages give no error model; this is the boundary's own. */
mk_status mk_sync_check(mk_ctx* ctx, void* stream);

/* Task tracing: the per-task timing behind the pages' 1-2 us between tasks
 * ("LLMs in einen MegaKernel kompilieren", "Ereignisbasierte Ausführung").
 * With a device buffer of at least n_tasks * 48 bytes (n_tasks from
 * mk_graph_stats), every later step writes one record per task, indexed by the
 * task's position in the global order. A record is {uint64 t_queue, t_ready,
 * t_streamed, t_done; uint16 cu; uint8 type; uint8 layer; uint32 epoch;
 * uint32 xcc; uint32 step}:
 *   - the times (100 MHz device real-time counter) when the CU reached the
 *     task, when its inputs were all present, when its own streaming ended (a
 *     GEMV's weights, before the epilogue; attention's cache rows and its
 *     in-task merge, before partials are written or merged) and when it
 *     published its outputs;
 *   - the workgroup (queue) index; the task type (1 QKV, 2 attention, 3 O
 *     projection, 4 gate/up, 5 down, 6 LM head, 7 argmax); its layer (n_layers
 *     for the LM head and argmax, mod 256); the step's epoch; the XCD the
 *     workgroup ran on (read from the hardware); the step's index in its launch.
 * Each step overwrites the records. d_buf == NULL turns tracing off. The
 * buffer stays the caller's.
 * Errors: MK_ERR_INVALID_ARG (too small or not 8-byte aligned). */
mk_status mk_set_trace(mk_ctx* ctx, void* d_buf, size_t bytes);

/* Graph inspection (host only, no GPU needed). The pages' compiler emits the
 * task graph ahead of time ("MPK: A Compiler and Runtime for Mega-Kernelizing
 * Tensor Programs", analogy 3); these calls check what the builder emitted.
 *   - mk_graph_stats: counts of tasks, events, flag slots and per-CU queue
 *     length (max), and the graph's 64-bit FNV-1a hash over its serialised
 *     form.
 *   - mk_graph_validate: checks the graph. Each event's producer count
 *     matches its slots. Each queue follows one global topological order.
 *     Every consumer comes after all its producers. Returns MK_OK or
 *     MK_ERR_SHAPE with a message.
 *   - mk_graph_simulate: runs the graph on the host. The per-CU queues
 *     advance in an order drawn from `seed`, against symbolic buffers.
 *     Returns MK_OK if every task ran with its inputs complete and no buffer
 *     was overwritten while a pending reader needed it. */
typedef struct {
  int64_t n_tasks, n_events, n_flag_slots, n_attn_groups, max_queue_len;
  int64_t weight_bytes, lds_bytes;
  uint64_t hash;
  int64_t n_stages; /* dependency stages: the dispatches of mk_decode_step_staged */
  int64_t attn_tasks; /* attention tasks per layer */
  int64_t n_cus;      /* compute units (queues) the graph was built for */
} mk_graph_info;
mk_status mk_graph_stats(const mk_ctx* ctx, mk_graph_info* out);
mk_status mk_graph_validate(const mk_ctx* ctx);
mk_status mk_graph_simulate(const mk_ctx* ctx, uint64_t seed, int n_steps);

/* Test hook, host-only contexts (mk_create_host) only: breaks the built graph in
 * one way, so that tests can show mk_graph_validate and mk_graph_simulate reject
 * it. kind: 1 two tasks of a queue swapped (queue out of the global order);
 * 2 a task waits on a later producer (a cycle); 3 a flag slot with two writers;
 * 4 a producer that never publishes (a slot with no writer); 5 two tiles of a
 * stage overlapping (rows written twice); 6 a consumer with its wait removed;
 * 7 a stage's last tile ending early (rows never written), 8 an event of the
 * run-time scheduling tables losing its last consumer (never queued), 9 an
 * event expecting one producer more than signal it (never complete); the last
 * two are caught by mk_graph_simulate's run of the ready queue.
 * Errors: MK_ERR_STATE (a device context), MK_ERR_INVALID_ARG (unknown kind, or
 * the graph has no task of the kind's type). */
mk_status mk_graph_corrupt(mk_ctx* ctx, int kind);

/* Release host structures. Device memory stays with the caller. (No passage:
 * the boundary's own.) */
void mk_destroy(mk_ctx* ctx);

const char* mk_status_str(mk_status s);
const char* mk_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
