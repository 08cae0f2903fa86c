// Host runtime of the decode megakernel: uploads a lowered graph (descriptor blob,
// buffer table, readiness counters), picks the kernel specialisation for the model's
// shape, and launches a step -- as ONE persistent kernel (mk_decode_step) or as one
// launch per op of the same task bodies (mk_decode_step_per_op, the baseline).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "device_common.h"
#include "internal.h"

namespace mk {

struct KernelSet {
  const void* persistent;
  const void* per_op;
  const void* levels;
};

// Specialisations compiled from kern_spec.hip, one object each.
#define MK_SPEC(name, wbf16, kvbf16, bm, kba, kbd) KernelSet ks_##name();
#include "specs.def"
#undef MK_SPEC

struct SpecEntry {
  const char* name;
  bool wbf16, kvbf16;
  int bm, kba, kbd;
  KernelSet (*get)();
};

static const SpecEntry kSpecs[] = {
#define MK_SPEC(name, wbf16, kvbf16, bm, kba, kbd) {#name, wbf16, kvbf16, bm, kba, kbd, &ks_##name},
#include "specs.def"
#undef MK_SPEC
};

// kblocks of one weight row: 64 lanes x 16 bytes per kblock.
static int kblocks(int K, bool bf16) { return (K * (bf16 ? 2 : 4) / 16 + 63) / 64; }

// The specialisation whose compile-time row shapes match the model, else the generic
// one of the same dtypes and batch block.
static const SpecEntry* select_spec(const mk_model_cfg& c) {
  const bool wb = c.weight_dtype == MK_DTYPE_BF16, kb = c.kv_dtype == MK_DTYPE_BF16;
  const int bm = c.gemv_config == MK_GEMV_BF16_MFMA ? (c.batch <= 8 ? 16 : 32) : (c.batch == 1 ? 1 : 8);
  const int ka = kblocks(c.hidden, wb), kd = kblocks(c.intermediate, wb);
  const SpecEntry* generic = nullptr;
  for (const SpecEntry& s : kSpecs) {
    if (s.wbf16 != wb || s.kvbf16 != kb || s.bm != bm) continue;
    if (s.kba == ka && s.kbd == kd) return &s;
    if (s.kba == 0 && s.kbd == 0) generic = &s;
  }
  return generic;
}

// Greedy SAMPLE ("Mega kernel initial", the op table's SAMPLE: argmax over the
// vocabulary), one workgroup per batch row: tokens[b] = the lowest index holding the
// row's largest logit (NaN never wins; a row with no comparable value gives 0), also
// written to out[b] when out is non-null, and positions[b] += 1 for the next step.
// After a failed step (non-zero status word) the logits are not trusted: tokens,
// out and positions are left as they are.
constexpr int kSampleThreads = 256;
__global__ __launch_bounds__(kSampleThreads) void sample_greedy_kernel(const float* logits, int vocab,
                                                                        int32_t* tokens, int32_t* positions,
                                                                        int32_t* out, const Ctrl* ctrl) {
  const int b = blockIdx.x;
  const float* row = logits + (size_t)b * vocab;
  float best = -INFINITY;
  int bi = INT32_MAX;
  for (int v = threadIdx.x; v < vocab; v += kSampleThreads) {
    const float x = row[v];
    if (x > best || (x == best && v < bi)) {
      best = x;
      bi = v;
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    const float ob = __shfl_xor(best, off);
    const int oi = __shfl_xor(bi, off);
    if (ob > best || (ob == best && oi < bi)) {
      best = ob;
      bi = oi;
    }
  }
  __shared__ float sb[kSampleThreads / 64];
  __shared__ int si[kSampleThreads / 64];
  if ((threadIdx.x & 63) == 0) {
    sb[threadIdx.x >> 6] = best;
    si[threadIdx.x >> 6] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t status =
        __hip_atomic_load((const MK_GLOBAL uint32_t*)&ctrl->status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (status != 0) return;
    for (int w = 1; w < kSampleThreads / 64; ++w)
      if (sb[w] > best || (sb[w] == best && si[w] < bi)) {
        best = sb[w];
        bi = si[w];
      }
    const int32_t tok = bi == INT32_MAX ? 0 : bi;
    tokens[b] = tok;
    if (out) out[b] = tok;
    positions[b] += 1;
  }
}

// 16-row tile layout of a bf16 matrix (mk_pack_matrix): one thread per 16-byte piece of
// the output, which is written in order; piece p is lane l = p % 64 of tile p / 64, the
// tile of row block r and k-step j being number r * (cols / 32) + j.
__global__ __launch_bounds__(256) void pack_matrix_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                          uint64_t pieces, uint32_t cols) {
  const uint64_t steps = cols / 32;
  for (uint64_t p = (uint64_t)blockIdx.x * 256 + threadIdx.x; p < pieces; p += (uint64_t)gridDim.x * 256) {
    const uint64_t tile = p >> 6, l = p & 63;
    const uint64_t r = tile / steps, j = tile - r * steps;
    const uint64_t row = 16 * r + (l & 15), col = 32 * j + 8 * (l >> 4);
    dst[p] = src[(row * cols + col) / 8];
  }
}

// Activation scratch of mk_decode_step_noalloc, for callers that cannot allocate: a
// file-scope device array, one copy per device, held until the process ends.  In host
// code `scratch` is a host-side stand-in for the symbol, not a device address: the
// address comes from hipGetSymbolAddress, taken once per device (with that device
// current) when a graph is built there, and kept in scratch_dev[].
constexpr uint64_t kStaticScratchBytes = uint64_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices];

__global__ void reset_kernel(uint32_t* arrivals, uint32_t n, Ctrl* ctrl) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    arrivals[(size_t)i * kArrivalStride] = 0;
  if (blockIdx.x == 0 && threadIdx.x < sizeof(Ctrl) / 4) ((uint32_t*)ctrl)[threadIdx.x] = 0;
}

}  // namespace mk

struct mk_graph {
  mk::Lowered low;
  const mk::SpecEntry* spec = nullptr;
  mk::KernelSet kernels{};
  int device = -1;
  uint32_t grid = 0;
  char* d_blob = nullptr;
  mk_task_t* d_tasks = nullptr;
  uint32_t* d_edges = nullptr;       // as lowered
  uint32_t* d_eslot = nullptr;       // per edge: the arrival counter it increments
  uint32_t* d_join = nullptr;        // per task: its NOP join's first shard counter, or 0xFFFFFFFF
  uint32_t* d_jcnt = nullptr;        // per join shard: parents counting on it
  uint32_t n_counters = 0;           // tasks + joins x kJoinShards
  uint32_t* d_order = nullptr;       // static schedule lists
  uint32_t* d_order_off = nullptr;   // [grid + 1]
  uint32_t* d_lvl = nullptr;         // level-synchronous lists: non-NOP tasks by level
  uint32_t* d_lvl_off = nullptr;     // [n_lvls + 1]
  uint32_t n_lvls = 0;               // non-empty levels
  uint32_t barrier_base = 0;         // Ctrl::barrier before the next level-synchronous step
  float* d_rope = nullptr;           // [kv_capacity][head_dim / 2] (cos, sin) pairs
  mk::Schedule sched;
  int sched_mode = MK_SCHED_STATIC;
  uint64_t* d_table = nullptr;
  void* scratch = nullptr;           // caller's activation workspace (may be null: mk_decode_step_noalloc only)
  uint32_t* d_arrivals = nullptr;
  mk::Ctrl* d_ctrl = nullptr;
  uint64_t* d_trace = nullptr;
  uint32_t epoch = 0;
  uint32_t ticket_base = 0;
  uint64_t wait_limit = 200000000ull;
  hipGraph_t per_op_graph = nullptr;        // captured per-op launches (baseline context)
  hipGraphExec_t per_op_exec = nullptr;
  bool needs_reset = false;
  hipStream_t last_stream = nullptr;
};

namespace {

// Records "what: HIP's message" without allocating (entry points that must not
// allocate report HIP failures through it too).
int hip_fail(hipError_t e, const char* what) {
  char buf[320];
  std::snprintf(buf, sizeof(buf), "%s: %s", what, hipGetErrorString(e));
  return mk::set_error(MK_ERR_HIP, buf);
}

#define HIP_TRY(call)                                  \
  do {                                                 \
    hipError_t e_ = (call);                            \
    if (e_ != hipSuccess) return hip_fail(e_, #call);  \
  } while (0)

bool misaligned(const void* p, uintptr_t a) { return ((uintptr_t)p) & (a - 1); }

void free_graph(mk_graph* g) {
  if (!g) return;
  if (g->d_blob) (void)hipFree(g->d_blob);
  if (g->d_table) (void)hipFree(g->d_table);
  if (g->d_arrivals) (void)hipFree(g->d_arrivals);
  if (g->d_ctrl) (void)hipFree(g->d_ctrl);
  delete g;
}

mk::LaunchArgs make_args(const mk_graph* g, const int32_t* tokens, const int32_t* positions, void* kcache,
                         void* vcache, float* logits) {
  mk::LaunchArgs a;
  std::memset(&a, 0, sizeof(a));
  a.tasks = g->d_tasks;
  a.edges = g->d_edges;
  a.eslot = g->d_eslot;
  a.join = g->d_join;
  a.jcnt = g->d_jcnt;
  if (g->sched_mode == MK_SCHED_STATIC) {
    a.order = g->d_order;
    a.order_off = g->d_order_off;
  }
  a.table = g->d_table;
  a.rope = g->d_rope;
  a.arrivals = g->d_arrivals;
  a.ctrl = g->d_ctrl;
  a.trace = g->d_trace;
  a.rt[mk::TAG_ABS] = 0;
  a.rt[mk::TAG_KCACHE] = (uint64_t)(uintptr_t)kcache;
  a.rt[mk::TAG_VCACHE] = (uint64_t)(uintptr_t)vcache;
  a.rt[mk::TAG_TOKENS] = (uint64_t)(uintptr_t)tokens;
  a.rt[mk::TAG_POSITIONS] = (uint64_t)(uintptr_t)positions;
  a.rt[mk::TAG_LOGITS] = (uint64_t)(uintptr_t)logits;
  a.rt[mk::TAG_SCRATCH] = (uint64_t)(uintptr_t)g->scratch;
  a.n_tasks = (uint32_t)g->low.tasks.size();
  a.wait_limit = g->wait_limit;
  a.lvl = g->d_lvl;
  a.lvl_off = g->d_lvl_off;
  a.n_levels = g->n_lvls;
  a.barrier_base = g->barrier_base;
  const mk_model_cfg& c = g->low.cfg;
  a.rms_eps = c.rms_eps;
  a.rope_theta = c.rope_theta;
  a.hidden = c.hidden;
  a.n_q_heads = c.n_q_heads;
  a.n_kv_heads = c.n_kv_heads;
  a.head_dim = c.head_dim;
  a.batch = c.batch;
  a.intermediate = c.intermediate;
  a.vocab = c.vocab;
  a.kv_capacity = c.kv_capacity;
  a.wpacked = (c.options & MK_LOWER_PACKED_WEIGHTS) ? 1u : 0u;
  return a;
}

int check_step_args(mk_graph* g, const int32_t* tokens, const int32_t* positions, void* kcache, void* vcache,
                    float* logits) {
  if (!g) return mk::set_error(MK_ERR_INVALID, "graph is NULL");
  if (!tokens || !positions || !kcache || !vcache || !logits)
    return mk::set_error(MK_ERR_INVALID, "NULL device pointer");
  if (misaligned(kcache, 16) || misaligned(vcache, 16) || misaligned(logits, 16) || misaligned(tokens, 4) ||
      misaligned(positions, 4))
    return mk::set_error(MK_ERR_ALIGN, "kcache/vcache/logits must be 16-byte aligned");
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev != g->device) return mk::set_error(MK_ERR_INVALID, "current device differs from the graph's device");
  return MK_OK;
}

// The caller's activation workspace, which every step entry point except
// mk_decode_step_noalloc needs.
int check_workspace(const mk_graph* g) {
  if (!g->scratch)
    return mk::set_error(MK_ERR_INVALID, "graph built without a scratch block: only mk_decode_step_noalloc can run it");
  return MK_OK;
}

int reset_state(mk_graph* g, hipStream_t s) {
  const uint32_t n = g->n_counters;
  const uint32_t blocks = (n + 255) / 256 > 0 ? (n + 255) / 256 : 1;
  hipLaunchKernelGGL(mk::reset_kernel, dim3(blocks < 1024 ? blocks : 1024), dim3(256), 0, s, g->d_arrivals, n,
                     g->d_ctrl);
  HIP_TRY(hipGetLastError());
  g->epoch = 0;
  g->ticket_base = 0;
  g->barrier_base = 0;
  g->needs_reset = false;
  return MK_OK;
}

// Device address of the static scratch array on device dev (the current device):
// taken once with hipGetSymbolAddress, then read from the per-device table.
int static_scratch(int dev, void** out) {
  if (dev < 0 || dev >= mk::kMaxDevices) return mk::set_error(MK_ERR_INVALID, "device index beyond the static scratch table");
  std::lock_guard<std::mutex> lock(mk::scratch_mu);
  if (!mk::scratch_dev[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(mk::scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return mk::set_error(MK_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    mk::scratch_dev[dev] = p;
  }
  *out = mk::scratch_dev[dev];
  return MK_OK;
}

// Enqueue one step of g with launch arguments a (per-step buffers resolved): the
// persistent kernel, or the level-synchronous one.  Allocates nothing.
int launch_step(mk_graph* g, hipStream_t s, mk::LaunchArgs& a) {
  int rc;
  if (g->needs_reset && (rc = reset_state(g, s)) != MK_OK) return rc;
  a.epoch = g->epoch + 1;
  a.ticket_base = g->ticket_base;
  a.barrier_base = g->barrier_base;
  void* params[] = {&a};
  if (g->sched_mode == MK_SCHED_LEVELS) {
    // Counters untouched (the epoch stays): only the barrier counter advances.
    hipError_t e = hipLaunchCooperativeKernel(g->kernels.levels, dim3(g->grid), dim3(mk::kThreads), params, 0, s);
    if (e != hipSuccess) return hip_fail(e, "hipLaunchCooperativeKernel(levels)");
    g->barrier_base += g->n_lvls * g->grid;
    g->last_stream = s;
    return MK_OK;
  }
  // Cooperative launch: the runtime refuses the launch (instead of letting the
  // spinning workgroups deadlock) if the whole grid cannot be resident at once.
  hipError_t e = hipLaunchCooperativeKernel(g->kernels.persistent, dim3(g->grid), dim3(mk::kThreads), params, 0, s);
  if (e != hipSuccess) return hip_fail(e, "hipLaunchCooperativeKernel(interpreter)");
  g->epoch += 1;
  // Dynamic mode: every ticket is claimed once and every workgroup makes one failing
  // claim; static mode leaves the counter alone.
  if (g->sched_mode == MK_SCHED_DYNAMIC) g->ticket_base += (uint32_t)g->low.tasks.size() + g->grid;
  g->last_stream = s;
  return MK_OK;
}

}  // namespace

extern "C" {

int mk_build_graph(const mk_model_cfg* cfg, const mk_weights* weights, void* scratch_dev, void* stream,
                   mk_graph** out) {
  if (!out) return mk::set_error(MK_ERR_INVALID, "out is NULL");
  *out = nullptr;
  mk_graph* g = new (std::nothrow) mk_graph();
  if (!g) return mk::set_error(MK_ERR_NOMEM, "out of host memory");
  int rc;
  try {
    rc = mk::lower(cfg, g->low);
  } catch (const std::bad_alloc&) {
    rc = mk::set_error(MK_ERR_NOMEM, "out of host memory while lowering");
  }
  if (rc) {
    free_graph(g);
    return rc;
  }
  const mk::Lowered& L = g->low;
  const mk::BufIdx& bi = L.bi;
  const int nl = L.cfg.n_layers;
  auto fail = [&](int code) {
    free_graph(g);
    return code;
  };
  if (!weights || weights->count != 3u + 6u * nl || !weights->dev_ptrs)
    return fail(mk::set_error(MK_ERR_INVALID, "weights: expected 3 + 6 * n_layers device pointers"));
  for (uint32_t i = 0; i < weights->count; ++i) {
    if (!weights->dev_ptrs[i]) return fail(mk::set_error(MK_ERR_INVALID, "weights: NULL pointer"));
    if (misaligned(weights->dev_ptrs[i], 16))
      return fail(mk::set_error(MK_ERR_ALIGN, "weights: pointer not 16-byte aligned"));
  }
  if (misaligned(scratch_dev, 256)) return fail(mk::set_error(MK_ERR_ALIGN, "scratch_dev not 256-byte aligned"));
  g->scratch = scratch_dev;
  g->spec = mk::select_spec(L.cfg);
  if (!g->spec) return fail(mk::set_error(MK_ERR_INVALID, "no kernel specialisation for these dtypes"));
  g->kernels = g->spec->get();
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipGetDevice(&g->device);
  if (e != hipSuccess) return fail(hip_fail(e, "hipGetDevice"));
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, g->device);
  if (e != hipSuccess) return fail(hip_fail(e, "hipGetDeviceProperties"));
  {
    // Set-up of mk_decode_step_noalloc on this device: the static scratch array's
    // address, taken here with the device current so that the step itself calls
    // nothing but launches.
    void* unused = nullptr;
    if ((rc = static_scratch(g->device, &unused)) != MK_OK) return fail(rc);
  }
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, g->kernels.persistent, mk::kThreads, 0);
  if (e != hipSuccess) return fail(hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor"));
  if (per_cu < 1) return fail(mk::set_error(MK_ERR_INVALID, "interpreter kernel cannot be resident"));
  g->grid = (uint32_t)prop.multiProcessorCount;  // one workgroup per CU

  // Buffer table: absolute pointers for weights, tagged offsets for the per-step
  // buffers (tokens, positions, caches, logits) and for the activations in the
  // scratch block, resolved from the launch arguments.
  std::vector<uint64_t> table(bi.count(), 0);
  auto W = [&](uint32_t i) { return (uint64_t)(uintptr_t)weights->dev_ptrs[i]; };
  table[bi.tokens()] = (uint64_t)mk::TAG_TOKENS << mk::kTagShift;
  table[bi.positions()] = (uint64_t)mk::TAG_POSITIONS << mk::kTagShift;
  table[bi.embedding()] = W(0);
  for (int l = 0; l < nl; ++l) {
    table[bi.layer(l, mk::W_ATTN_NORM)] = W(1 + 6 * l + 0);
    table[bi.layer(l, mk::W_QKV)] = W(1 + 6 * l + 1);
    table[bi.layer(l, mk::W_O)] = W(1 + 6 * l + 2);
    table[bi.layer(l, mk::W_MLP_NORM)] = W(1 + 6 * l + 3);
    table[bi.layer(l, mk::W_GATE_UP)] = W(1 + 6 * l + 4);
    table[bi.layer(l, mk::W_DOWN)] = W(1 + 6 * l + 5);
    table[bi.layer(l, mk::KCACHE)] = ((uint64_t)mk::TAG_KCACHE << mk::kTagShift) | (uint64_t)l * L.kv_layer_bytes;
    table[bi.layer(l, mk::VCACHE)] = ((uint64_t)mk::TAG_VCACHE << mk::kTagShift) | (uint64_t)l * L.kv_layer_bytes;
  }
  table[bi.final_norm()] = W(1 + 6 * nl);
  table[bi.w_lm()] = W(2 + 6 * nl);
  for (uint32_t i = 0; i < bi.count(); ++i)
    if (L.scratch_off[i] != UINT64_MAX) table[i] = ((uint64_t)mk::TAG_SCRATCH << mk::kTagShift) | L.scratch_off[i];
  table[bi.logits()] = (uint64_t)mk::TAG_LOGITS << mk::kTagShift;

  // Static schedule over one workgroup per CU.
  try {
    mk::build_schedule(L, g->grid, g->sched);
  } catch (const std::bad_alloc&) {
    return fail(mk::set_error(MK_ERR_NOMEM, "out of host memory while scheduling"));
  }
  const mk::Schedule& S = g->sched;

  // One blob: 64-byte header, task array, edge array as lowered, the counter each edge
  // increments, each task's NOP join (a task has at most one: the lowering emits one
  // join per op) as the first of the join's shard counters, the parents per shard, the
  // static lists and their offsets.  Counters: one per task, then kJoinShards per join;
  // parent p of a join counts on the join's shard p % kJoinShards.
  const size_t nt = L.tasks.size(), ne = L.edges.size(), no = S.order.size();
  constexpr uint32_t JS = mk::kJoinShards;
  std::vector<uint32_t> jord(nt, 0xFFFFFFFFu);
  uint32_t nj = 0;
  for (size_t n = 0; n < nt; ++n)
    if (L.tasks[n].op_id == MK_OP_NOP) jord[n] = nj++;
  std::vector<uint32_t> join(nt, 0xFFFFFFFFu), eslot(ne), jcnt((size_t)nj * JS, 0u);
  for (size_t p = 0; p < nt; ++p) {
    const mk_task_t& d = L.tasks[p];
    for (int32_t i = 0; i < d.num_dependents; ++i) {
      const size_t k = (size_t)d.dependents_offset + i;
      const uint32_t c = L.edges[k];
      if (jord[c] == 0xFFFFFFFFu) {
        eslot[k] = c;
      } else {
        eslot[k] = (uint32_t)nt + jord[c] * JS + (uint32_t)(p % JS);
        ++jcnt[(size_t)jord[c] * JS + p % JS];
      }
    }
    if (d.op_id != MK_OP_NOP) continue;
    for (int32_t i = 0; i < d.num_dependents; ++i) {
      const uint32_t c = L.edges[(size_t)d.dependents_offset + i];
      if (join[c] != 0xFFFFFFFFu) return fail(mk::set_error(MK_ERR_INVALID, "a task with two join parents"));
      join[c] = (uint32_t)nt + jord[p] * JS;
    }
  }
  g->n_counters = (uint32_t)nt + nj * JS;
  const size_t off_tasks = sizeof(mk::BlobHeader);
  const size_t off_edges = off_tasks + nt * sizeof(mk_task_t);
  const size_t off_eslot = off_edges + ne * 4;
  const size_t off_join = off_eslot + ne * 4;
  const size_t off_jcnt = off_join + nt * 4;
  const size_t off_order = off_jcnt + jcnt.size() * 4;
  const size_t off_order_off = off_order + no * 4;
  // RoPE coefficients of every cache slot: the angle pos * theta^(-2i/hd) and its
  // cosine and sine in binary64, rounded to binary32.  They depend on the position
  // only, so APPEND reads them (a static input) before its dependency wait instead of
  // evaluating binary64 transcendentals on the critical path.
  const size_t half = (size_t)L.cfg.head_dim / 2, cap = (size_t)L.cfg.kv_capacity;
  const size_t off_rope = (off_order_off + S.offsets.size() * 4 + 15) & ~(size_t)15;
  mk::Levels levels;
  mk::build_levels(L, levels);
  const std::vector<uint32_t>& lvl = levels.tasks;
  const std::vector<uint32_t>& lvl_off = levels.offsets;
  const size_t off_lvl = off_rope + cap * half * 8;
  const size_t off_lvl_off = off_lvl + lvl.size() * 4;
  const size_t blob_bytes = off_lvl_off + lvl_off.size() * 4;
  std::vector<char> blob(blob_bytes);
  {
    float* rope = (float*)(blob.data() + off_rope);
    for (size_t i = 0; i < half; ++i) {
      const double inv = std::pow((double)L.cfg.rope_theta, -2.0 * (double)i / (double)L.cfg.head_dim);
      for (size_t pos = 0; pos < cap; ++pos) {
        const double ang = (double)pos * inv;
        rope[(pos * half + i) * 2] = (float)std::cos(ang);
        rope[(pos * half + i) * 2 + 1] = (float)std::sin(ang);
      }
    }
  }
  std::memcpy(blob.data(), &L.header, sizeof(mk::BlobHeader));
  std::memcpy(blob.data() + off_tasks, L.tasks.data(), nt * sizeof(mk_task_t));
  if (ne) std::memcpy(blob.data() + off_edges, L.edges.data(), ne * 4);
  if (ne) std::memcpy(blob.data() + off_eslot, eslot.data(), ne * 4);
  if (nt) std::memcpy(blob.data() + off_join, join.data(), nt * 4);
  if (!jcnt.empty()) std::memcpy(blob.data() + off_jcnt, jcnt.data(), jcnt.size() * 4);
  if (no) std::memcpy(blob.data() + off_order, S.order.data(), no * 4);
  std::memcpy(blob.data() + off_order_off, S.offsets.data(), S.offsets.size() * 4);
  if (!lvl.empty()) std::memcpy(blob.data() + off_lvl, lvl.data(), lvl.size() * 4);
  std::memcpy(blob.data() + off_lvl_off, lvl_off.data(), lvl_off.size() * 4);
  if ((e = hipMalloc(&g->d_blob, blob_bytes)) != hipSuccess) return fail(hip_fail(e, "hipMalloc(blob)"));
  if ((e = hipMalloc(&g->d_table, table.size() * 8)) != hipSuccess) return fail(hip_fail(e, "hipMalloc(table)"));
  if ((e = hipMalloc(&g->d_arrivals, (g->n_counters ? g->n_counters : 1) * 4 * (size_t)mk::kArrivalStride)) !=
      hipSuccess)
    return fail(hip_fail(e, "hipMalloc(arrivals)"));
  if ((e = hipMalloc(&g->d_ctrl, sizeof(mk::Ctrl))) != hipSuccess) return fail(hip_fail(e, "hipMalloc(ctrl)"));
  g->d_tasks = (mk_task_t*)(g->d_blob + off_tasks);
  g->d_edges = (uint32_t*)(g->d_blob + off_edges);
  g->d_eslot = (uint32_t*)(g->d_blob + off_eslot);
  g->d_join = (uint32_t*)(g->d_blob + off_join);
  g->d_jcnt = (uint32_t*)(g->d_blob + off_jcnt);
  g->d_order = (uint32_t*)(g->d_blob + off_order);
  g->d_order_off = (uint32_t*)(g->d_blob + off_order_off);
  g->d_rope = (float*)(g->d_blob + off_rope);
  g->d_lvl = (uint32_t*)(g->d_blob + off_lvl);
  g->d_lvl_off = (uint32_t*)(g->d_blob + off_lvl_off);
  g->n_lvls = (uint32_t)(lvl_off.size() - 1);
  if ((e = hipMemcpyAsync(g->d_blob, blob.data(), blob_bytes, hipMemcpyHostToDevice, s)) != hipSuccess)
    return fail(hip_fail(e, "hipMemcpyAsync(blob)"));
  if ((e = hipMemcpyAsync(g->d_table, table.data(), table.size() * 8, hipMemcpyHostToDevice, s)) != hipSuccess)
    return fail(hip_fail(e, "hipMemcpyAsync(table)"));
  if ((rc = reset_state(g, s)) != MK_OK) return fail(rc);
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return fail(hip_fail(e, "hipStreamSynchronize"));
  g->last_stream = s;
  *out = g;
  return MK_OK;
}

int mk_graph_tasks(const mk_graph* g, const mk_task_t** tasks, uint32_t* n) {
  if (!g || !tasks || !n) return mk::set_error(MK_ERR_INVALID, "NULL argument");
  *tasks = g->low.tasks.data();
  *n = (uint32_t)g->low.tasks.size();
  return MK_OK;
}

int mk_graph_edges(const mk_graph* g, const uint32_t** edges, uint32_t* n) {
  if (!g || !edges || !n) return mk::set_error(MK_ERR_INVALID, "NULL argument");
  *edges = g->low.edges.data();
  *n = (uint32_t)g->low.edges.size();
  return MK_OK;
}

int mk_graph_grid(const mk_graph* g, uint32_t* workgroups) {
  if (!g || !workgroups) return mk::set_error(MK_ERR_INVALID, "NULL argument");
  *workgroups = g->grid;
  return MK_OK;
}

const char* mk_graph_kernel_name(const mk_graph* g) { return g && g->spec ? g->spec->name : ""; }

int mk_set_schedule(mk_graph* g, int mode) {
  if (!g || (mode != MK_SCHED_STATIC && mode != MK_SCHED_DYNAMIC && mode != MK_SCHED_LEVELS))
    return mk::set_error(MK_ERR_INVALID, "graph is NULL or unknown schedule mode");
  g->sched_mode = mode;
  return MK_OK;
}

int mk_graph_schedule(const mk_graph* g, const uint32_t** order, const uint32_t** offsets, uint32_t* workers,
                      double* est_us) {
  if (!g || !order || !offsets || !workers) return mk::set_error(MK_ERR_INVALID, "NULL argument");
  *order = g->sched.order.data();
  *offsets = g->sched.offsets.data();
  *workers = g->grid;
  if (est_us) *est_us = g->sched.est_us;
  return MK_OK;
}

int mk_set_wait_limit(mk_graph* g, uint64_t ticks) {
  if (!g || ticks == 0) return mk::set_error(MK_ERR_INVALID, "graph is NULL or limit is 0");
  g->wait_limit = ticks;
  return MK_OK;
}

int mk_set_trace(mk_graph* g, uint64_t* trace_dev) {
  if (!g) return mk::set_error(MK_ERR_INVALID, "graph is NULL");
  if (misaligned(trace_dev, 8)) return mk::set_error(MK_ERR_ALIGN, "trace buffer not 8-byte aligned");
  g->d_trace = trace_dev;
  return MK_OK;
}

int mk_decode_step(mk_graph* g, void* stream, const int32_t* tokens_dev, const int32_t* positions_dev,
                   void* kcache_dev, void* vcache_dev, float* logits_dev) {
  int rc = check_step_args(g, tokens_dev, positions_dev, kcache_dev, vcache_dev, logits_dev);
  if (rc || (rc = check_workspace(g))) return rc;
  mk::LaunchArgs a = make_args(g, tokens_dev, positions_dev, kcache_dev, vcache_dev, logits_dev);
  return launch_step(g, (hipStream_t)stream, a);
}

int mk_decode_step_noalloc(mk_graph* g, void* stream, const int32_t* tokens_dev, const int32_t* positions_dev,
                           void* kcache_dev, void* vcache_dev, float* logits_dev) {
  int rc = check_step_args(g, tokens_dev, positions_dev, kcache_dev, vcache_dev, logits_dev);
  if (rc) return rc;
  if (g->low.scratch_total > mk::kStaticScratchBytes)
    return mk::set_error(MK_ERR_INVALID,
                         "the step's activations exceed the 64 MiB static scratch array (mk_plan scratch_bytes)");
  void* p = nullptr;
  if ((rc = static_scratch(g->device, &p)) != MK_OK) return rc;
  mk::LaunchArgs a = make_args(g, tokens_dev, positions_dev, kcache_dev, vcache_dev, logits_dev);
  a.rt[mk::TAG_SCRATCH] = (uint64_t)(uintptr_t)p;
  return launch_step(g, (hipStream_t)stream, a);
}

int mk_decode_step_per_op(mk_graph* g, void* stream, const int32_t* tokens_dev, const int32_t* positions_dev,
                          void* kcache_dev, void* vcache_dev, float* logits_dev) {
  int rc = check_step_args(g, tokens_dev, positions_dev, kcache_dev, vcache_dev, logits_dev);
  if (rc || (rc = check_workspace(g))) return rc;
  hipStream_t s = (hipStream_t)stream;
  mk::LaunchArgs a = make_args(g, tokens_dev, positions_dev, kcache_dev, vcache_dev, logits_dev);
  a.trace = nullptr;
  for (const mk::OpRange& op : g->low.ops) {
    a.first_task = op.first;
    void* params[] = {&a};
    HIP_TRY(hipLaunchKernel(g->kernels.per_op, dim3(op.count), dim3(mk::kThreads), params, 0, s));
  }
  g->last_stream = s;
  return MK_OK;
}

int mk_sample_greedy(mk_graph* g, void* stream, const float* logits_dev, int32_t* tokens_dev,
                     int32_t* positions_dev) {
  if (!g || !logits_dev || !tokens_dev || !positions_dev) return mk::set_error(MK_ERR_INVALID, "NULL argument");
  if (misaligned(logits_dev, 4) || misaligned(tokens_dev, 4) || misaligned(positions_dev, 4))
    return mk::set_error(MK_ERR_ALIGN, "logits/tokens/positions must be 4-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const mk_model_cfg& c = g->low.cfg;
  hipLaunchKernelGGL(mk::sample_greedy_kernel, dim3(c.batch), dim3(mk::kSampleThreads), 0, s, logits_dev, c.vocab,
                     tokens_dev, positions_dev, (int32_t*)nullptr, g->d_ctrl);
  HIP_TRY(hipGetLastError());
  g->last_stream = s;
  return MK_OK;
}

int mk_pack_matrix(const void* src_dev, void* dst_dev, int32_t rows, int32_t cols, void* stream) {
  if (!src_dev || !dst_dev) return mk::set_error(MK_ERR_INVALID, "mk_pack_matrix: NULL pointer");
  if (rows < 16 || cols < 32 || rows % 16 || cols % 32)
    return mk::set_error(MK_ERR_INVALID, "mk_pack_matrix: rows must be a positive multiple of 16, cols of 32");
  if (misaligned(src_dev, 16) || misaligned(dst_dev, 16))
    return mk::set_error(MK_ERR_ALIGN, "mk_pack_matrix: src and dst must be 16-byte aligned");
  const uint64_t bytes = (uint64_t)rows * (uint64_t)cols * 2u;
  const uintptr_t s0 = (uintptr_t)src_dev, d0 = (uintptr_t)dst_dev;
  if (s0 < d0 + bytes && d0 < s0 + bytes) return mk::set_error(MK_ERR_INVALID, "mk_pack_matrix: src and dst overlap");
  const uint64_t pieces = bytes / 16;
  const uint64_t blocks = (pieces + 255) / 256;
  hipLaunchKernelGGL(mk::pack_matrix_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0,
                     (hipStream_t)stream, (const uint4*)src_dev, (uint4*)dst_dev, pieces, (uint32_t)cols);
  HIP_TRY(hipGetLastError());
  return MK_OK;
}

int mk_decode_greedy(mk_graph* g, void* stream, int n_steps, int32_t* tokens_dev, int32_t* positions_dev,
                     void* kcache_dev, void* vcache_dev, float* logits_dev, int32_t* tokens_out_dev) {
  if (!g) return mk::set_error(MK_ERR_INVALID, "graph is NULL");
  if (n_steps < 0) return mk::set_error(MK_ERR_INVALID, "n_steps < 0");
  if (misaligned(tokens_out_dev, 4)) return mk::set_error(MK_ERR_ALIGN, "tokens_out must be 4-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const int batch = g->low.cfg.batch;
  if (g->low.cfg.options & MK_LOWER_SAMPLE) {
    // SAMPLE tasks end the graph: one launch per token.
    int rc = check_step_args(g, tokens_dev, positions_dev, kcache_dev, vcache_dev, logits_dev);
    if (rc || (rc = check_workspace(g))) return rc;
    for (int i = 0; i < n_steps; ++i) {
      mk::LaunchArgs a = make_args(g, tokens_dev, positions_dev, kcache_dev, vcache_dev, logits_dev);
      a.tokens_out = tokens_out_dev ? tokens_out_dev + (size_t)i * batch : nullptr;
      if ((rc = launch_step(g, s, a)) != MK_OK) return rc;
    }
    return MK_OK;
  }
  for (int i = 0; i < n_steps; ++i) {
    int rc = mk_decode_step(g, stream, tokens_dev, positions_dev, kcache_dev, vcache_dev, logits_dev);
    if (rc) return rc;
    hipLaunchKernelGGL(mk::sample_greedy_kernel, dim3(batch), dim3(mk::kSampleThreads), 0, s, logits_dev,
                       g->low.cfg.vocab, tokens_dev, positions_dev,
                       tokens_out_dev ? tokens_out_dev + (size_t)i * batch : (int32_t*)nullptr, g->d_ctrl);
    HIP_TRY(hipGetLastError());
  }
  return MK_OK;
}

namespace {

void drop_per_op_graph(mk_graph* g) {
  if (g->per_op_exec) (void)hipGraphExecDestroy(g->per_op_exec);
  if (g->per_op_graph) (void)hipGraphDestroy(g->per_op_graph);
  g->per_op_exec = nullptr;
  g->per_op_graph = nullptr;
}

}  // namespace

int mk_capture_per_op_graph(mk_graph* g, const int32_t* tokens_dev, const int32_t* positions_dev,
                            void* kcache_dev, void* vcache_dev, float* logits_dev) {
  int rc = check_step_args(g, tokens_dev, positions_dev, kcache_dev, vcache_dev, logits_dev);
  if (rc || (rc = check_workspace(g))) return rc;
  drop_per_op_graph(g);
  hipStream_t cs = nullptr;
  HIP_TRY(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
  hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e == hipSuccess) {
    mk::LaunchArgs a = make_args(g, tokens_dev, positions_dev, kcache_dev, vcache_dev, logits_dev);
    a.trace = nullptr;
    for (const mk::OpRange& op : g->low.ops) {
      a.first_task = op.first;
      void* params[] = {&a};
      e = hipLaunchKernel(g->kernels.per_op, dim3(op.count), dim3(mk::kThreads), params, 0, cs);
      if (e != hipSuccess) break;
    }
    hipGraph_t graph = nullptr;
    const hipError_t e2 = hipStreamEndCapture(cs, &graph);  // ends the capture on every path
    if (e == hipSuccess) e = e2;
    if (e == hipSuccess) e = hipGraphInstantiate(&g->per_op_exec, graph, nullptr, nullptr, 0);
    if (e == hipSuccess) g->per_op_graph = graph;
    else if (graph) (void)hipGraphDestroy(graph);
  }
  (void)hipStreamDestroy(cs);
  if (e != hipSuccess) {
    g->per_op_exec = nullptr;
    return hip_fail(e, "capturing the per-op launches");
  }
  return MK_OK;
}

int mk_launch_per_op_graph(mk_graph* g, void* stream) {
  if (!g) return mk::set_error(MK_ERR_INVALID, "NULL graph");
  if (!g->per_op_exec) return mk::set_error(MK_ERR_INVALID, "no per-op graph captured");
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(hipGraphLaunch(g->per_op_exec, s));
  g->last_stream = s;
  return MK_OK;
}

int mk_status(mk_graph* g, uint32_t* device_status) {
  if (!g || !device_status) return mk::set_error(MK_ERR_INVALID, "NULL argument");
  HIP_TRY(hipStreamSynchronize(g->last_stream));
  uint32_t st = 0;
  HIP_TRY(hipMemcpy(&st, &g->d_ctrl->status, 4, hipMemcpyDeviceToHost));
  *device_status = st;
  if (st != 0) {
    g->needs_reset = true;
    char buf[96];
    std::snprintf(buf, sizeof(buf), "device status 0x%08x (kind 0x%x, task %u)", st, st >> 28, st & 0x0FFFFFFFu);
    return mk::set_error(MK_ERR_DEVICE, buf);
  }
  return MK_OK;
}

void mk_destroy(mk_graph* g) {
  if (!g) return;
  drop_per_op_graph(g);
  if (g->last_stream) (void)hipStreamSynchronize(g->last_stream);
  free_graph(g);
}

}  // extern "C"
