// Device-side shared pieces of the interpreter: launch arguments, buffer-table
// resolution, explicit global-memory accessors, bf16 conversion, wavefront
// reductions, and the readiness protocol (wait on a task's own counter, then count
// one arrival on each dependent's, with device-scope accesses for the shared data).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mk.h"

namespace mk {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));  // an MFMA bf16 operand

constexpr int kThreads = 512;  // 8 wave64s per workgroup, one workgroup per CU
constexpr int kWaves = kThreads / 64;
// LDS: x staging, GEMV partial sums, attention merge.  Most of the CU's 160 KB, so
// the persistent kernel gets exactly one workgroup per CU (co-residency of the whole
// grid).
constexpr int kSmemBytes = 148 * 1024;
constexpr int kRedFloats = 1024;  // reduction scratch

// Arrival counters sit one per 128-byte line, so the atomics of a join's fan-out (one
// wave incrementing up to 256 children) and the children's polls never share a line.
constexpr uint32_t kArrivalStride = 32;
// A NOP join's arrivals are spread over this many counters (parent task index modulo
// the count picks one), each on its own line: a join with 256 parents then takes 32
// increments per word instead of 256 on one, and its children poll all of them.
constexpr uint32_t kJoinShards = 8;
// Word 3 of a raw (stride 0, untyped) buffer resource on gfx950, and the cache-policy
// operand of a buffer load that streams (non-temporal).
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kCachePolicyNT = 2;
// Cache-policy operand of a device-scope (sc1) load.
constexpr int kCachePolicySC1 = 16;

// Buffer-table entry tags (top byte): 0 = absolute device pointer; otherwise an
// offset into a base passed at launch: the per-step buffers, and the activation
// scratch block (the caller's workspace, or the library's static array).
enum : uint32_t {
  TAG_ABS = 0, TAG_KCACHE = 1, TAG_VCACHE = 2, TAG_TOKENS = 3, TAG_POSITIONS = 4, TAG_LOGITS = 5, TAG_SCRATCH = 6
};
constexpr uint64_t kTagShift = 56;
constexpr uint64_t kOffMask = (uint64_t(1) << kTagShift) - 1;

struct Ctrl {
  uint32_t head;     // ticket counter (monotone across steps)
  uint32_t status;   // sticky device status word
  uint32_t barrier;  // level-synchronous mode: grid-barrier arrivals (monotone across steps)
  uint32_t pad[61];
};

struct Smem {
  float xs[kSmemBytes / 4];       // staged activations / attention merge
  float red[kRedFloats];          // reductions
  alignas(16) mk_task_t desc[3];  // current, next and next-but-one descriptors (rotating)
  uint64_t t_ready;               // trace: when the dependency wait ended
  uint64_t t_mark[3];             // trace: optional points inside a task body
  uint32_t ticket[3];
  uint32_t flag;
  uint32_t stop;  // set when a task raised an error status: end after the current task
};

struct LaunchArgs {
  const mk_task_t* tasks;
  const uint32_t* edges;      // dependents array (CSR, as lowered)
  const uint32_t* eslot;      // per edge: the arrival counter it increments (a join's shard)
  const uint32_t* join;       // per task: first counter of its NOP join's shards, or 0xFFFFFFFF
  const uint32_t* jcnt;       // per join shard (counter index - n_tasks): parents counting on it
  const uint32_t* order;      // static schedule: task lists grouped by workgroup
  const uint32_t* order_off;  // [grid + 1]; null = dynamic tickets
  const uint64_t* table;
  const float* rope;   // [kv_capacity][head_dim / 2] (cos, sin): RoPE coefficients per cache slot
  uint32_t* arrivals;  // one counter per kArrivalStride words
  Ctrl* ctrl;
  uint64_t* trace;
  int32_t* tokens_out;  // SAMPLE tasks also write their token here when non-null ([batch])
  uint32_t wpacked;     // 1: the matrices are in the 16-row tile layout of mk_pack_matrix
  uint64_t rt[8];  // per-step bases indexed by tag
  uint32_t n_tasks;
  uint32_t epoch;
  uint32_t ticket_base;
  uint32_t first_task;  // per-op launches: first task of the op
  uint64_t wait_limit;  // ticks of the 100 MHz clock
  const uint32_t* lvl;       // level-synchronous mode: non-NOP task indices grouped by level
  const uint32_t* lvl_off;   // [n_levels + 1]
  uint32_t n_levels;         // non-empty levels
  uint32_t barrier_base;     // Ctrl::barrier at the start of this step
  float rms_eps, rope_theta;
  int32_t hidden, n_q_heads, n_kv_heads, head_dim, batch, intermediate, vocab, kv_capacity;
};

// Every buffer lives in device global memory.  Pointers come out of the buffer table
// as generic pointers; these accessors cast them to the global address space so the
// compiler emits global_load/global_store (counted by vmcnt only) instead of flat
// accesses (which also count against lgkmcnt and force full waits).
#define MK_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ T ldg(const void* p, size_t i) {
  return ((const MK_GLOBAL T*)p)[i];
}
template <typename T>
__device__ __forceinline__ T ldg_nt(const void* p, size_t i) {
  return __builtin_nontemporal_load(((const MK_GLOBAL T*)p) + i);
}
template <typename T>
__device__ __forceinline__ void stg(void* p, size_t i, T v) {
  ((MK_GLOBAL T*)p)[i] = v;
}

// Device-scope accesses, for the data one task writes and another task reads within
// the same step (activations, attention partials, the new token's cache row).
//
// The MI355X has one L2 per XCD and the L2s are not kept coherent with each other.
// The fence-based protocol (a release fence before the counter increment, an acquire
// fence after the counter wait) costs a whole-L2 writeback (buffer_wbl2) on every
// release and a whole-L2 invalidate (buffer_inv) on every acquire, and the writebacks
// of the workgroups of one XCD serialise: under a wide matmul's 256 simultaneous
// releases one release took 5-20 us.  Instead, every access to in-step shared data is
// an agent-scope relaxed atomic, which the compiler emits as a global load/store with
// the device-scope cache-policy bit (sc1): the store is written through to the
// device's coherence point before it is acknowledged, and the load is served from
// there.  Ordering then needs no cache maintenance: the producer waits for its stores
// to be acknowledged (s_waitcnt vmcnt(0)) before its counter increments, and the
// consumer issues its loads only after it has observed its counter.  Plain
// (CU-scope) loads are kept for data no task of the step writes: weights, norm
// gammas, the embedding, tokens, positions and the cache rows of earlier steps
// (kernel boundaries make those coherent).
template <typename T>
__device__ __forceinline__ T ld_dev(const void* p, size_t i) {
  static_assert(sizeof(T) == 2 || sizeof(T) == 4 || sizeof(T) == 8, "scalar device-scope load");
  return __hip_atomic_load((const MK_GLOBAL T*)p + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st_dev(void* p, size_t i, T v) {
  static_assert(sizeof(T) == 2 || sizeof(T) == 4 || sizeof(T) == 8, "scalar device-scope store");
  __hip_atomic_store((MK_GLOBAL T*)p + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes at p + 16 * i4, as two 8-byte device-scope loads.
__device__ __forceinline__ u32x4 ld_dev_u4(const void* p, size_t i4) {
  const uint64_t lo = ld_dev<uint64_t>(p, 2 * i4), hi = ld_dev<uint64_t>(p, 2 * i4 + 1);
  u32x4 r;
  r.x = (uint32_t)lo;
  r.y = (uint32_t)(lo >> 32);
  r.z = (uint32_t)hi;
  r.w = (uint32_t)(hi >> 32);
  return r;
}
__device__ __forceinline__ f32x4 ld_dev_f4(const void* p, size_t i4) {
  const u32x4 u = ld_dev_u4(p, i4);
  f32x4 r;
  r.x = __uint_as_float(u.x);
  r.y = __uint_as_float(u.y);
  r.z = __uint_as_float(u.z);
  r.w = __uint_as_float(u.w);
  return r;
}

// Wave index as a wave-uniform (scalar) value, so branches on it stay scalar.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// The buffer table is written by the host before the launch and only read here: a
// scalar load through the constant address space (counted by lgkmcnt, so it never
// makes a wave wait behind its own outstanding vector loads).
__device__ __forceinline__ char* resolve(const LaunchArgs& a, uint32_t idx) {
  const uint64_t e = ((const __attribute__((address_space(4))) uint64_t*)a.table)[idx];
  const uint32_t tag = (uint32_t)(e >> kTagShift);
  // Compare chain instead of indexing a.rt with a run-time tag (an indexed kernel
  // argument would be copied to private memory).
  uint64_t base = 0;
  base = tag == TAG_KCACHE ? a.rt[TAG_KCACHE] : base;
  base = tag == TAG_VCACHE ? a.rt[TAG_VCACHE] : base;
  base = tag == TAG_TOKENS ? a.rt[TAG_TOKENS] : base;
  base = tag == TAG_POSITIONS ? a.rt[TAG_POSITIONS] : base;
  base = tag == TAG_LOGITS ? a.rt[TAG_LOGITS] : base;
  base = tag == TAG_SCRATCH ? a.rt[TAG_SCRATCH] : base;
  return (char*)(base + (e & kOffMask));
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// The value held by lane (this lane ^ OFF), OFF a power of two below 64, without an
// LDS round trip where gfx950 has a VALU form: DPP quad_perm for 1 and 2, DPP
// row_ror:8 for 8, v_permlane16_swap / v_permlane32_swap for 16 and 32 (each swap
// hands back both halves; the lane keeps its partner's); ds_swizzle (xor mode)
// for 4.
template <int OFF>
__device__ __forceinline__ float lane_xor(float v) {
  const uint32_t u = __float_as_uint(v);
  if constexpr (OFF == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, (int)u, 0xB1, 0xF, 0xF, false));
  else if constexpr (OFF == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, (int)u, 0x4E, 0xF, 0xF, false));
  else if constexpr (OFF == 4) return __int_as_float(__builtin_amdgcn_ds_swizzle((int)u, (4 << 10) | 0x1F));
  else if constexpr (OFF == 8) return __int_as_float(__builtin_amdgcn_update_dpp(0, (int)u, 0x128, 0xF, 0xF, false));
  else if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
  } else {
    static_assert(OFF == 32, "lane_xor offset");
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
  v += lane_xor<32>(v);
  v += lane_xor<16>(v);
  v += lane_xor<8>(v);
  v += lane_xor<4>(v);
  v += lane_xor<2>(v);
  v += lane_xor<1>(v);
  return v;
}

// Wavefront sum with DPP moves only (no LDS): row_shr 1/2/4/8 leaves each 16-lane
// row's sum in its lane 15, row_bcast15 and row_bcast31 fold the four rows into lane
// 63.  Only lane 63 holds the total.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
  const int s = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, true);
  return v + __int_as_float(s);
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = dpp_add<0x111, 0xF>(v);  // row_shr:1
  v = dpp_add<0x112, 0xF>(v);  // row_shr:2
  v = dpp_add<0x114, 0xF>(v);  // row_shr:4
  v = dpp_add<0x118, 0xF>(v);  // row_shr:8
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Sum across aligned groups of `width` lanes (a wave-uniform power of two <= 64),
// leaving the group's total in every lane of the group.  Up to 16 lanes this is a
// butterfly of DPP moves (VALU only, no LDS round trip): quad_perm [1,0,3,2] and
// [2,3,0,1] sum each quad, row_half_mirror pairs the two quads of each 8 lanes,
// row_mirror the two halves of each 16.  Wider groups finish with xor shuffles.
template <int CTRL>
__device__ __forceinline__ float dpp_swap_add(float v) {
  const int s = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false);
  return v + __int_as_float(s);
}
template <int W>
__device__ __forceinline__ float group_allsum(float v) {
  static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "group width");
  if constexpr (W >= 2) v = dpp_swap_add<0xB1>(v);
  if constexpr (W >= 4) v = dpp_swap_add<0x4E>(v);
  if constexpr (W >= 8) v = dpp_swap_add<0x141>(v);
  if constexpr (W >= 16) v = dpp_swap_add<0x140>(v);
  if constexpr (W >= 32) v += lane_xor<16>(v);
  if constexpr (W >= 64) v += lane_xor<32>(v);
  return v;
}
__device__ __forceinline__ float group_allsum(float v, int width) {
  if (width >= 2) v = dpp_swap_add<0xB1>(v);   // quad_perm [1,0,3,2]
  if (width >= 4) v = dpp_swap_add<0x4E>(v);   // quad_perm [2,3,0,1]
  if (width >= 8) v = dpp_swap_add<0x141>(v);  // row_half_mirror
  if (width >= 16) v = dpp_swap_add<0x140>(v); // row_mirror
  if (width >= 32) v += __shfl_xor(v, 16, 64);
  if (width >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

__device__ __forceinline__ uint64_t clock100() { return wall_clock64(); }

// Trace mode: thread 0 records a point inside a task body (trace words 5..7).
__device__ __forceinline__ void trace_mark(const LaunchArgs& a, Smem& sm, int i) {
  if (a.trace != nullptr && threadIdx.x == 0) sm.t_mark[i] = clock100();
}

__device__ __forceinline__ void raise_status(const LaunchArgs& a, uint32_t code) {
  uint32_t expected = 0u;
  __hip_atomic_compare_exchange_strong((MK_GLOBAL uint32_t*)&a.ctrl->status, &expected, code, __ATOMIC_RELAXED,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t read_status(const LaunchArgs& a) {
  return __hip_atomic_load((MK_GLOBAL uint32_t*)&a.ctrl->status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll one readiness counter until it reaches target (wrapping 32-bit comparison),
// bounded by the wait limit and abandoned if another workgroup raised an error.
// Thread 0 only; returns 0 if the step was abandoned.  A device-scope load is a
// round trip to memory, so the loop's period is what a waiting task adds to its
// producers' release: every iteration reads the counter alone, and only every 16th
// also reads the clock and the status word.
__device__ __forceinline__ uint32_t poll_counter(const LaunchArgs& a, uint32_t t, const uint32_t* counter,
                                                 uint32_t target) {
  MK_GLOBAL uint32_t* cnt = (MK_GLOBAL uint32_t*)counter;
  uint32_t v = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((int32_t)(v - target) >= 0) return 1;
  const uint64_t t0 = clock100();
  for (uint32_t it = 1;; ++it) {
    __builtin_amdgcn_s_sleep(1);
    v = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((int32_t)(v - target) >= 0) return 1;
    if ((it & 15u) == 0u) {
      if (clock100() - t0 > a.wait_limit) {
        raise_status(a, MK_STATUS_TIMEOUT | t);
        return 0;
      }
      if (read_status(a) != 0) return 0;
    }
  }
}

// Poll until every shard of a NOP join has its parents of this step: shard s of the
// join whose counters start at `base` expects epoch * jcnt[base - n_tasks + s].  The
// shards are read together each round.  One thread; 0 if the step was abandoned.
__device__ __forceinline__ uint32_t poll_join(const LaunchArgs& a, uint32_t t, uint32_t base) {
  uint32_t target[kJoinShards];
#pragma unroll
  for (uint32_t s = 0; s < kJoinShards; ++s) target[s] = a.epoch * ldg<uint32_t>(a.jcnt, base - a.n_tasks + s);
  const uint64_t t0 = clock100();
  for (uint32_t it = 1;; ++it) {
    uint32_t v[kJoinShards];
#pragma unroll
    for (uint32_t s = 0; s < kJoinShards; ++s)
      v[s] = __hip_atomic_load((MK_GLOBAL uint32_t*)(a.arrivals + (size_t)(base + s) * kArrivalStride),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool ok = true;
#pragma unroll
    for (uint32_t s = 0; s < kJoinShards; ++s) ok &= (int32_t)(v[s] - target[s]) >= 0;
    if (ok) return 1;
    __builtin_amdgcn_s_sleep(1);
    if ((it & 15u) == 0u) {
      if (clock100() - t0 > a.wait_limit) {
        raise_status(a, MK_STATUS_TIMEOUT | t);
        return 0;
      }
      if (read_status(a) != 0) return 0;
    }
  }
}

// Poll until all of this step's parents of task t have arrived.  A task whose parents
// include a NOP join (at most one: one join per op) waits for the join's shards (the
// join's parents count on them directly, nobody fires the join) and for its own
// counter to reach epoch * (indeg - 1); any other task waits for epoch * indeg on its
// own counter.  One thread; returns 0 if the step was abandoned (timeout, or another
// workgroup raised an error).
__device__ __forceinline__ uint32_t poll_deps(const LaunchArgs& a, uint32_t t, int32_t indeg) {
  if (indeg == 0) return 1;
  const uint32_t j = ldg<uint32_t>(a.join, t);
  uint32_t ok = 1, own = (uint32_t)indeg;
  if (j != 0xFFFFFFFFu) {
    ok = poll_join(a, t, j);
    own -= 1;
  }
  if (ok && own > 0) ok = poll_counter(a, t, a.arrivals + (size_t)t * kArrivalStride, a.epoch * own);
  return ok;
}

// Wait until all of this step's parents of task t have arrived (thread 0 polls).  The
// producers' data was written at device scope and acknowledged before their
// increments, and every wave reads it with device-scope loads issued after the
// closing barrier, so no cache invalidate is needed.  Bounded: on timeout (or if
// another workgroup raised an error) the step is abandoned.  Returns false if the
// step was abandoned.  Called by all threads.
__device__ __forceinline__ bool dep_wait(const LaunchArgs& a, uint32_t t, int32_t indeg, Smem& sm) {
  if (indeg == 0) {
    if (threadIdx.x == 0) sm.t_ready = clock100();
    return true;
  }
  if (threadIdx.x == 0) {
    sm.flag = poll_deps(a, t, indeg);
    sm.t_ready = clock100();
  }
  __syncthreads();
  return sm.flag != 0;
}

// Count one arrival on each of the n dependents listed at edges[off]: on the
// dependent's own counter, or for a NOP join on the join shard this parent feeds
// (eslot holds the counter of every edge).  Wave 0 only; the caller has waited for its
// own data stores to be acknowledged.
__device__ __forceinline__ void signal_dependents(const LaunchArgs& a, uint32_t off, uint32_t n) {
  for (uint32_t i = lane_id(); i < n; i += 64) {
    const uint32_t c = ldg<uint32_t>(a.eslot, off + i);
    __hip_atomic_fetch_add((MK_GLOBAL uint32_t*)a.arrivals + (size_t)c * kArrivalStride, 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Wait until every device-scope store of the workgroup is acknowledged (written
// through to the device coherence point), then count one arrival on every
// dependent.  The asm's memory clobber and the barrier keep the compiler from moving
// any store past the increments.  Called by all threads after the task body.
__device__ __forceinline__ void release_dependents(const LaunchArgs& a, const mk_task_t& d) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (wave_id() == 0) signal_dependents(a, d.dependents_offset, (uint32_t)d.num_dependents);
}

}  // namespace mk
