/* mk.h -- C ABI of the MI355X decode megakernel library (libmk.so).
 *
 * One decode step of a decoder-only transformer is lowered once, on the host, into a
 * static, topologically ordered array of 64-byte task descriptors plus a flat CSR
 * array of dependency edges ("Mega kernel initial", 1y33.com: sections on the
 * lowering, the task descriptor and the edge array).  mk_decode_step then runs the
 * whole step as ONE persistent kernel launch: one workgroup per compute unit pulls
 * tasks in emission order and starts each one as soon as its own producers have
 * finished, tracked by per-task readiness counters in device memory -- no grid-wide
 * barrier ("Megakernels", runhoid.com: "Megakernel iceberg", layer 6, and "Hoid's
 * approach to megakernels").
 *
 * Conventions for every entry point:
 *   - Return value: 0 on success, a negative MK_ERR_* code on failure.  Nothing throws
 *     across the ABI.  mk_last_error() returns a thread-local message for the last
 *     failing call on the calling thread.
 *   - "device pointer" = memory from hipMalloc (or a PyTorch CUDA/HIP tensor) on the
 *     current device; "host pointer" = ordinary process memory.
 *   - Streams are hipStream_t passed as void* (NULL = the null stream).
 *   - The caller owns every buffer it passes (weights, KV caches, scratch, tokens,
 *     positions, logits).  The library never frees caller memory.  The library owns
 *     the graph object, its host copies of tasks and edges, and its small device
 *     allocations (descriptor blob, buffer table, readiness counters, control block),
 *     all released by mk_destroy.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MK_ABI_VERSION 1u

/* ---- error codes ---------------------------------------------------------------- */
#define MK_OK 0
#define MK_ERR_ABI (-1)        /* abi_version or struct_size mismatch                  */
#define MK_ERR_INVALID (-2)    /* a configuration value or argument is out of range    */
#define MK_ERR_ALIGN (-3)      /* a device pointer is not 16-byte aligned              */
#define MK_ERR_HIP (-4)        /* a HIP runtime call failed (message has the reason)  */
#define MK_ERR_NOMEM (-5)      /* host or device allocation failed                    */
#define MK_ERR_DEVICE (-6)     /* the device status word reports a failure (mk_status) */

/* Device status word (mk_status): 0 = ok; otherwise the top 4 bits hold the kind and
 * the low 28 bits the index of the task that raised it. */
#define MK_STATUS_TIMEOUT 0x10000000u      /* a dependency wait exceeded its bound      */
#define MK_STATUS_BAD_POSITION 0x20000000u /* positions[b] outside [0, kv_len[b])       */
#define MK_STATUS_BAD_TOKEN 0x30000000u    /* tokens[b] outside [0, vocab)              */
#define MK_STATUS_KIND_MASK 0xF0000000u

/* ---- task descriptor ("Mega kernel initial", descriptor section) ------------------
 * 64-byte POD, identical on host and device; buffers are referenced by uint16 index
 * into the buffer table, never by pointer.  Field offsets: 0,2,4,6,8,12,16,20,26,28,
 * 32,36,40,44.  Per-op meaning of m/n/k/kv_len/reserved (reserved = per-op scalars):
 *   GEMV (2):    m = batch rows, n = output columns of the whole matmul, k = inner dim;
 *                reserved = {col_begin, col_count, I (SILU_MUL: up rows start) or 0};
 *                in_buf = {x, W, gamma (RMS_NORM_INPUT) | residual (ADD_RESIDUAL) | none}
 *   ATTENTION_APPEND (7): m = batch, n = head_dim, k = KV head g, kv_len = capacity;
 *                reserved = {b, first q head, q heads per group, kcache buf, vcache buf}
 *   ATTENTION_PARTIAL (8): m = chunks of sequence b, n = head_dim, k = g,
 *                kv_len = chunk size; reserved = {b, first q head, heads, chunk c,
 *                first partial slot of (b, g)}; in_buf = {q_rot, kcache, vcache}
 *   ATTENTION_COMBINE (9): as PARTIAL with reserved[3] = 0; in_buf = {partials}
 *   MEMCPY (1):  embedding gather, m = batch, n = hidden; in_buf = {tokens, E}
 *   RMSNORM (3): row b = reserved[0] of out = rmsnorm(x [+ residual]) * gamma; m =
 *                batch, n = hidden; in_buf = {x, gamma, residual | none}; flags
 *                FUSED_RESIDUAL: the sum x + residual is also written to buffer
 *                reserved[1]
 *   SAMPLE (6):  row b = reserved[0]: out (the tokens buffer)[b] = argmax of row b of
 *                in_buf[0] (the logits; lowest index on ties), positions (buffer
 *                reserved[1])[b] += 1; m = batch, n = vocab
 *   NOP (0):     join node; only the dependency fields are set.
 * remaining_deps is the in-degree (constant; run-time readiness uses separate
 * counters).  step is always 0.  config_id selects the body variant: GEMV 0 fp32,
 * 1 bf16 vector, 2 bf16 MFMA; APPEND/PARTIAL cache dtype (0 f32, 1 bf16); MEMCPY
 * embedding dtype. */
typedef struct mk_task {
  uint16_t op_id;
  uint16_t config_id;
  uint16_t step;
  uint16_t flags;
  int32_t remaining_deps;
  int32_t num_dependents;
  uint32_t dependents_offset;
  uint16_t in_buf[3];
  uint16_t out_buf;
  int32_t m;
  int32_t n;
  int32_t k;
  int32_t kv_len;
  uint32_t reserved[5];
} mk_task_t;

/* OpId values and flag bits as listed on the page (OpId table; flags paragraph). */
enum {
  MK_OP_NOP = 0, MK_OP_MEMCPY = 1, MK_OP_GEMV = 2, MK_OP_RMSNORM = 3, MK_OP_ATTENTION = 4,
  MK_OP_MLP = 5, MK_OP_SAMPLE = 6, MK_OP_ATTENTION_APPEND = 7, MK_OP_ATTENTION_PARTIAL = 8,
  MK_OP_ATTENTION_COMBINE = 9
};
enum { MK_FLAG_SILU_MUL = 1, MK_FLAG_ADD_RESIDUAL = 2, MK_FLAG_RMS_NORM_INPUT = 4 };
enum { MK_FLAG_FUSED_RESIDUAL = 2 }; /* the same bit on an RMSNORM descriptor */

enum { MK_DTYPE_F32 = 0, MK_DTYPE_BF16 = 1 };
enum { MK_GEMV_F32 = 0, MK_GEMV_BF16 = 1, MK_GEMV_BF16_MFMA = 2 };

/* ---- model configuration -----------------------------------------------------------
 * Decoder: per layer qkv = W_qkv * rmsnorm(x, attn_norm); RoPE-append; GQA attention
 * over the cache; h = x + W_o * att; x' = h + W_down * (silu(gate) * up) with
 * [gate; up] = W_gate_up * rmsnorm(h, mlp_norm); logits = W_lm * rmsnorm(x, final_norm)
 * ("Mega kernel initial", graph API section).  Weights are row-major [out, in].
 * kv_len[b] (host pointer, batch entries, read during the call only) is the attended
 * length planned for sequence b including the new token; it fixes that sequence's
 * number of KV chunks.  At run time sequence b attends to slots [0, positions[b]], so
 * positions[b] + 1 <= kv_len[b] <= kv_capacity. */
typedef struct mk_model_cfg {
  uint32_t abi_version; /* MK_ABI_VERSION */
  uint32_t struct_size; /* sizeof(mk_model_cfg) */
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, intermediate, vocab, batch;
  float rms_eps, rope_theta;
  int32_t weight_dtype, kv_dtype; /* MK_DTYPE_* */
  int32_t gemv_tiles;             /* column tiles per matmul (T) */
  int32_t kv_chunk;               /* keys per ATTENTION_PARTIAL task */
  int32_t join_nodes;             /* 1: insert NOP join tasks for shared parent sets */
  int32_t gemv_config;            /* MK_GEMV_* */
  int32_t kv_capacity;            /* cache slots per (layer, sequence, KV head) */
  int32_t options;                /* MK_LOWER_* bits (0: fused step, logits only) */
  const int32_t* kv_len;          /* host pointer, [batch] */
} mk_model_cfg;

/* Lowering options ("Mega kernel initial": the graph-API section writes the decoder
 * with its fusions given by hand and names a pass that finds them automatically as
 * future work; the OpId table lists RMSNORM and SAMPLE).  The lowering first writes
 * the step as a list of ops with no fusion -- every RMSNorm its own op, each residual
 * add carried by the next RMSNorm (FUSED_RESIDUAL) -- then runs that pass, which
 * folds each residual add into the matmul producing the summand (ADD_RESIDUAL) and
 * each RMSNorm read only by matmuls into them (RMS_NORM_INPUT); the result is the
 * hand-fused decoder.
 *   MK_LOWER_UNFUSED: skip the pass.  Every RMSNorm runs as RMSNORM tasks (one per
 *     batch row) and the graph has 4 n_layers + 1 more activation buffers (BufIdx
 *     order: after the logits, per layer the normed attention input, the o-projection
 *     output, the normed MLP input, the down-projection output; then the normed
 *     lm_head input).
 *   MK_LOWER_SAMPLE: one SAMPLE task per batch row after the lm_head, so a step
 *     writes each row's greedy token (argmax, lowest index on ties) into tokens_dev
 *     and advances positions_dev: one launch runs a whole greedy step. */
#define MK_LOWER_UNFUSED 1
#define MK_LOWER_SAMPLE 2
/*   MK_LOWER_PACKED_WEIGHTS: the five matrices of every layer and the lm_head (W_qkv,
 *     W_o, W_gate_up, W_down, W_lm; not the embedding) are passed in the 16-row tile
 *     layout that mk_pack_matrix writes.  Needs gemv_config MK_GEMV_BF16_MFMA (the
 *     matrix-core tiles read that layout one contiguous kilobyte per wave and k-step);
 *     MK_ERR_INVALID otherwise.  The descriptors are the same as without the bit: the
 *     layout is a property of the weight buffers, and the results are bitwise those of
 *     the row-major weights. */
#define MK_LOWER_PACKED_WEIGHTS 4

/* Weights in canonical order (buffer-table section of the page: append-only, one
 * index per tensor): [0] embedding [vocab, hidden]; per layer l at 1 + 6 l:
 * attn_norm [hidden], W_qkv [(Hq + 2 Hkv) hd, hidden], W_o [hidden, Hq hd],
 * mlp_norm [hidden], W_gate_up [2 I, hidden], W_down [hidden, I]; then final_norm
 * [hidden] and W_lm [vocab, hidden].  count = 3 + 6 n_layers.  Device pointers in
 * weight_dtype, each 16-byte aligned. */
typedef struct mk_weights {
  uint32_t count;
  void* const* dev_ptrs; /* host array of device pointers */
} mk_weights;

typedef struct mk_graph mk_graph;     /* lowered + uploaded graph (device-side state) */
typedef struct mk_lowered mk_lowered; /* host-only lowering result */

/* Sizes of the lowered graph and of the scratch block the caller must provide.
 * Host only; touches no GPU. */
typedef struct mk_plan_info {
  uint32_t n_tasks;
  uint32_t n_edges;
  uint32_t n_buffers;
  uint32_t n_levels;         /* 1 + max level (level = 1 + max parent level) */
  uint64_t scratch_bytes;    /* activation scratch for one step */
  uint64_t kv_layer_bytes;   /* bytes of one layer's K (or V) cache slab */
} mk_plan_info;

/* Validate `cfg` and size the lowered graph: task, edge, buffer and level counts, and
 * the activation scratch the caller allocates ("Mega kernel initial": the lowering
 * section fans each op out into tiles, and the buffer-table section allocates each
 * op's output on demand; here every output gets its own span of one scratch block).
 * Host only; touches no GPU.  Errors: MK_ERR_ABI, MK_ERR_INVALID. */
int mk_plan(const mk_model_cfg* cfg, mk_plan_info* out);

/* Host-only lowering (no GPU calls; "Mega kernel initial": the lowering section --
 * fan-out into column tiles, parents tracked per column range, flattened to an edge
 * array -- and the descriptor section): the descriptor array and CSR edge array that
 * mk_build_graph would upload.  Arrays stay owned by the mk_lowered object.  Errors:
 * MK_ERR_ABI, MK_ERR_INVALID, MK_ERR_NOMEM. */
int mk_lower(const mk_model_cfg* cfg, mk_lowered** out);
int mk_lowered_tasks(const mk_lowered* g, const mk_task_t** tasks, uint32_t* n);
int mk_lowered_edges(const mk_lowered* g, const uint32_t** edges, uint32_t* n);
/* Byte offset and size of activation buffer `buf_index` inside the scratch block
 * (error for buffers that are not scratch). */
int mk_lowered_scratch_span(const mk_lowered* g, uint32_t buf_index, uint64_t* offset, uint64_t* bytes);
/* The static schedule mk_build_graph would compute for a grid of `workers`
 * workgroups (see mk_set_schedule and mk_graph_schedule for the layout).  Arrays are
 * owned by the mk_lowered object and replaced by the next call. */
int mk_lowered_schedule(mk_lowered* g, uint32_t workers, const uint32_t** order,
                        const uint32_t** offsets, double* est_us);
/* Level-synchronous lists (the order MK_SCHED_LEVELS runs): the non-NOP task indices
 * grouped by level of the task DAG (one more than the highest level among a task's
 * parents, NOP joins included in that count), ascending within a level, levels that
 * hold only NOP joins dropped.  Level i is tasks[offsets[i] .. offsets[i + 1]), i <
 * n_levels.  Arrays are library-owned, valid until the next call or mk_lowered_free. */
int mk_lowered_levels(mk_lowered* g, const uint32_t** tasks, const uint32_t** offsets, uint32_t* n_levels);
void mk_lowered_free(mk_lowered* g);

/* Lower, then upload descriptors + edges (one blob behind a 64-byte header) and the
 * buffer table to the device, on `stream` ("Mega kernel initial": the lowering, edge
 * and upload sections; the buffer table holds indices, the pointers live in a table
 * of their own).  `scratch_dev` (device pointer, at least mk_plan().scratch_bytes,
 * 256-byte aligned) holds the step's activations; NULL builds a graph that only
 * mk_decode_step_noalloc can run.  The weights must stay valid for the graph's
 * lifetime.  Synchronises `stream` before returning.  Errors: MK_ERR_ABI,
 * MK_ERR_INVALID (configuration or weights), MK_ERR_ALIGN, MK_ERR_NOMEM, MK_ERR_HIP;
 * *out is NULL on failure. */
int mk_build_graph(const mk_model_cfg* cfg, const mk_weights* weights, void* scratch_dev,
                   void* stream, mk_graph** out);

/* Write the 16-row tile layout of one bf16 matrix, for graphs lowered with
 * MK_LOWER_PACKED_WEIGHTS (a one-time conversion when the weights are loaded; not part
 * of the pages' method: the matrix-core tile reads it with whole-kilobyte loads).
 * src: device pointer, row-major [rows, cols] bf16; dst: device pointer to
 * rows * cols * 2 bytes, not overlapping src.  Both 16-byte aligned, rows % 16 == 0,
 * cols % 32 == 0.  Layout: for row block r (rows 16 r .. 16 r + 15) and k-step j
 * (cols 32 j .. 32 j + 31) a 1024-byte tile at byte (r * cols / 32 + j) * 1024 holds,
 * for lane l = 0..63, the 8 values src[16 r + l % 16][32 j + 8 (l / 16) + e], e = 0..7,
 * at byte 16 l + 2 e.  A block of 16 rows keeps its place (the same 32 cols bytes as
 * row-major).  Enqueued on `stream` (asynchronous; no allocation).  Errors:
 * MK_ERR_INVALID (sizes, NULL, overlap), MK_ERR_ALIGN, MK_ERR_HIP. */
int mk_pack_matrix(const void* src_dev, void* dst_dev, int32_t rows, int32_t cols, void* stream);

/* Host copies of what mk_build_graph uploaded (library-owned, valid until mk_destroy). */
int mk_graph_tasks(const mk_graph* g, const mk_task_t** tasks, uint32_t* n);
int mk_graph_edges(const mk_graph* g, const uint32_t** edges, uint32_t* n);

/* One decode step as ONE persistent-kernel launch ("Megakernels", runhoid.com: "Hoid's
 * approach to megakernels" -- one kernel that interprets the task list, each block
 * waiting only on its own producers -- and iceberg layer 6), enqueued on `stream` (no
 * host synchronisation).  Device pointers: tokens_dev int32[batch]; positions_dev
 * int32[batch]; kcache_dev / vcache_dev [n_layers][batch][n_kv_heads][kv_capacity]
 * [head_dim] in kv_dtype (slot positions[b] of every layer is overwritten with the new
 * token's rotated k and its v); logits_dev float32[batch][vocab].  The step reads the
 * cache slots [0, positions[b]].  Out-of-range positions set the device status
 * (mk_status) and leave the outputs of the affected sequence undefined.  Errors:
 * MK_ERR_INVALID (NULL graph or pointer, graph built without scratch), MK_ERR_ALIGN
 * (buffers not 16-byte aligned; tokens and positions 4), MK_ERR_HIP (launch). */
int mk_decode_step(mk_graph* g, void* stream, const int32_t* tokens_dev, const int32_t* positions_dev,
                   void* kcache_dev, void* vcache_dev, float* logits_dev);

/* For callers that cannot allocate device memory at step time (code under HIP-graph
 * capture, tight serving loops, harnesses that forbid allocation): mk_decode_step with
 * the step's activations in a static array of the library instead of the caller's
 * scratch block.  Same kernels, same descriptors, same arguments and results as
 * mk_decode_step.  It calls no hipMalloc, hipFree or other allocating routine.
 *   - The array is a file-scope device array of 64 MiB (MK_STATIC_SCRATCH_BYTES); each
 *     device the library runs on holds its own copy until the process ends.  A graph
 *     whose mk_plan scratch_bytes exceed it is rejected with MK_ERR_INVALID.
 *   - Its address on a device is taken once, when a graph is built on that device.
 *   - Every call on one device shares that device's array: calls that overlap on one
 *     device (several streams, or several graphs, without stream order between them)
 *     race and give undefined results.  Each step writes every activation it reads,
 *     so nothing has to be cleared between calls.
 *   - A graph built with scratch_dev = NULL can run only through this call.
 * Errors: as mk_decode_step, plus MK_ERR_INVALID for a graph beyond the limit. */
#define MK_STATIC_SCRATCH_BYTES (64ull << 20)
int mk_decode_step_noalloc(mk_graph* g, void* stream, const int32_t* tokens_dev, const int32_t* positions_dev,
                           void* kcache_dev, void* vcache_dev, float* logits_dev);

/* The same step with the same task bodies and descriptors, one kernel launch per op
 * (stream order instead of readiness counters): the per-op-launch baseline the pages
 * measure against ("Megakernels", runhoid.com, Introduction: the launch gaps and tails
 * of one kernel per op).  Same errors as mk_decode_step. */
int mk_decode_step_per_op(mk_graph* g, void* stream, const int32_t* tokens_dev,
                          const int32_t* positions_dev, void* kcache_dev, void* vcache_dev,
                          float* logits_dev);

/* Greedy SAMPLE ("Mega kernel initial", 1y33.com, the op table: SAMPLE), enqueued on
 * `stream` (no host synchronisation): for each batch row b, tokens_dev[b] = the lowest
 * index holding the largest value of logits_dev row b ([batch, vocab] fp32; NaN never
 * wins, a row with no comparable value gives 0), and positions_dev[b] += 1, ready
 * for the next step.  One workgroup per row; batch and vocab are the graph's.  Runs as
 * its own small kernel after the step rather than as tasks of the graph.  While the
 * graph's device status word holds a failure (see mk_status) it writes nothing: tokens
 * and positions keep their values.  Errors: MK_ERR_INVALID, MK_ERR_ALIGN, MK_ERR_HIP. */
int mk_sample_greedy(mk_graph* g, void* stream, const float* logits_dev, int32_t* tokens_dev,
                     int32_t* positions_dev);

/* n_steps greedy decode steps with no host round trip, so step i + 1 embeds step i's
 * tokens at the next positions and appends to the same caches.  For a graph built with
 * MK_LOWER_SAMPLE each step is ONE launch (its SAMPLE tasks pick the tokens and advance
 * the positions); otherwise each step is mk_decode_step on these buffers followed by
 * mk_sample_greedy.  When tokens_out_dev is non-NULL
 * (device, n_steps * batch int32), step i's tokens are also written to
 * tokens_out_dev[i * batch + b].  Positions must stay below each sequence's kv_len
 * (the graph's chunk fan-out); a step past it sets MK_STATUS_BAD_POSITION, which
 * mk_status reports.  From a failed step on, the later steps run no task and their
 * SAMPLE writes no token and advances no position.  Same errors as mk_decode_step. */
int mk_decode_greedy(mk_graph* g, void* stream, int n_steps, int32_t* tokens_dev, int32_t* positions_dev,
                     void* kcache_dev, void* vcache_dev, float* logits_dev, int32_t* tokens_out_dev);

/* Context for the per-op baseline ("Megakernel iceberg" page, the CUDA-graphs layer:
 * graph replay removes the host's per-launch cost but keeps one kernel boundary per
 * op).  mk_capture_per_op_graph records the launches of mk_decode_step_per_op for
 * the given step buffers into a HIP graph owned by `g` (replacing any earlier one),
 * captured on a stream of the library's own; the buffers are baked into the graph and
 * must stay valid while it is replayed.  mk_launch_per_op_graph enqueues one replay
 * on `stream` (one whole step, same results as mk_decode_step_per_op).  Errors:
 * MK_ERR_INVALID (bad arguments, or no graph captured yet), MK_ERR_HIP. */
int mk_capture_per_op_graph(mk_graph* g, const int32_t* tokens_dev, const int32_t* positions_dev,
                            void* kcache_dev, void* vcache_dev, float* logits_dev);
int mk_launch_per_op_graph(mk_graph* g, void* stream);

/* Synchronises `g`'s last stream and reads the device status word (see
 * MK_STATUS_*).  A non-zero status is cleared and the graph's scheduler state is
 * reset, so the next step runs normally.  Returns MK_ERR_DEVICE if it was non-zero. */
int mk_status(mk_graph* g, uint32_t* device_status);

/* Bound on one dependency wait, in ticks of the 100 MHz constant clock
 * (default 200,000,000 = 2 s).  A wait that exceeds it sets MK_STATUS_TIMEOUT and
 * the kernel drains instead of hanging. */
int mk_set_wait_limit(mk_graph* g, uint64_t ticks);

/* Trace mode: when `trace_dev` is non-NULL (device pointer, n_tasks * 8 uint64), the
 * next mk_decode_step calls record per task {XCC_ID << 32 | HW_ID register, start
 * time, ready time (dependency wait over), body end time, release end time, mark 0,
 * mark 1, mark 2}, times in ticks of the constant 100 MHz clock.  Marks are points
 * inside a body (0 where a body sets none): GEMV -- every wave past the input
 * staging, last row reduced, the control wave done staging the input;
 * ATTENTION_PARTIAL -- chunk folded, partials merged; ATTENTION_COMBINE -- weights
 * computed.  NOP joins run no body and record nothing.  NULL turns it off.  The
 * pointer must stay valid while steps that use it run. */
int mk_set_trace(mk_graph* g, uint64_t* trace_dev);

/* Number of workgroups the persistent kernel is launched with (one per CU). */
int mk_graph_grid(const mk_graph* g, uint32_t* workgroups);

/* Name of the kernel specialisation the graph runs (library-owned string; "" for a
 * NULL graph). */
const char* mk_graph_kernel_name(const mk_graph* g);

/* How the persistent kernel's workgroups find their next task.
 *
 * MK_SCHED_STATIC (default): each workgroup walks its own list of task indices,
 * computed once by mk_build_graph.  This follows the host-side grouping of task
 * indices ahead of time in "Mega kernel initial" (1y33.com, the level section: task
 * indices grouped, plus the offsets where each group starts), except that the groups
 * are per workgroup, not per level, and no grid barrier separates them.  The lists
 * come from simulating list scheduling in emission order with a byte-count cost
 * model, which hands each workgroup one tile of every wide matmul and so removes
 * the wave-quantisation tail of "Megakernels" (runhoid.com, Fig. 2).  Each list is in
 * increasing task order.
 * MK_SCHED_DYNAMIC: each workgroup claims the next task index from a device-wide
 * ticket counter ("Megakernels", runhoid.com, Fig. 5 b: a queue the SMs pop from).
 *
 * MK_SCHED_LEVELS: the level-synchronous variant of "Mega kernel initial" (1y33.com,
 * the level section): the non-NOP tasks grouped by their level in the DAG, each level
 * run round robin by the workgroups of one cooperative kernel, with a grid barrier
 * between levels and no readiness counters.  An ablation of what the counters buy.
 *
 * In the counter modes NOP joins are never run as tasks: their children poll the
 * join's own counter.  Takes effect from the next mk_decode_step; results are bitwise
 * identical in all modes. */
#define MK_SCHED_STATIC 0
#define MK_SCHED_DYNAMIC 1
#define MK_SCHED_LEVELS 2
int mk_set_schedule(mk_graph* g, int mode);

/* The static schedule: `order` holds the non-NOP task indices grouped by workgroup,
 * workgroup w's list is order[offsets[w] .. offsets[w + 1]), `workers` = grid size;
 * `est_us` (may be NULL) receives the cost model's simulated step time.  Arrays are
 * library-owned, valid until mk_destroy. */
int mk_graph_schedule(const mk_graph* g, const uint32_t** order, const uint32_t** offsets,
                      uint32_t* workers, double* est_us);

void mk_destroy(mk_graph* g);
const char* mk_last_error(void);
uint32_t mk_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
