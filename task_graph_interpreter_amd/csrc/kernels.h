// The persistent interpreter kernel and the per-op-launch baseline kernel, both
// specialised at compile time for one model shape (Spec): weight and cache dtypes,
// batch block, and the kblock counts (16-byte-per-lane row blocks) of the two GEMV
// inner dimensions a decoder uses (hidden and intermediate).  Each specialisation is
// compiled in its own translation unit (kern_*.hip); any shape without one runs the
// generic specialisation, whose GEMV streams one kblock at a time.
//
// Scheduling ("Megakernels", runhoid.com: "Megakernel iceberg" layer 6 and "Hoid's
// approach to megakernels"): one workgroup per CU, all co-resident; each pulls the
// next ticket of a device-wide counter, so tasks start in the lowering's topological
// emission order ("Mega kernel initial", edge section); a task waits only for its own
// readiness counter, and on completion increments the counter of every dependent
// (the page's old queue path decremented remaining_deps; here the counters count
// arrivals and never need resetting: task t is ready in step e once
// arrivals[t] >= e * remaining_deps[t]).  Deadlock freedom: tickets are taken in
// topological order and every workgroup is resident, so the lowest claimed but
// unfinished task always has all of its parents finished.
#pragma once

#include "tasks.h"

namespace mk {

template <bool WBF16_, bool KVBF16_, int BM_, int KBA_, int KBD_>
struct Spec {
  static constexpr bool WBF16 = WBF16_;    // weights bf16 (else fp32)
  static constexpr bool KVBF16 = KVBF16_;  // KV cache bf16 (else fp32)
  static constexpr int BM = BM_;           // batch rows per GEMV pass (1 or 8); MFMA tiles: 16 (batch <= 8), 32
  static constexpr int KBA = KBA_;         // kblocks of K = hidden (0: generic)
  static constexpr int KBD = KBD_;         // kblocks of K = intermediate (0: generic)
};

// A row of KB kblocks -> (kblocks per segment, segments, rows in flight): 8 to 16
// loads of 16 bytes in flight per lane (a two-row ring for 8-kblock rows holds a whole
// 16-row tile of a 4096-wide matrix).  Other row lengths take the generic path.
constexpr bool kb_compiled(int KB) { return KB == 1 || KB == 2 || KB == 4 || KB == 8 || KB == 16 || KB == 28; }

template <int BM, bool BF16, int KB>
__device__ __forceinline__ void gemv_kb(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm) {
  if constexpr (KB == 1) gemv_run<BM, BF16, 1, 1, 8>(a, d, t, sm);
  else if constexpr (KB == 2) gemv_run<BM, BF16, 2, 1, 4>(a, d, t, sm);
  else if constexpr (KB == 4) gemv_run<BM, BF16, 4, 1, 2>(a, d, t, sm);
  else if constexpr (KB == 8) gemv_run<BM, BF16, 8, 1, 2>(a, d, t, sm);
  else if constexpr (KB == 16) gemv_run<BM, BF16, 8, 2, 1>(a, d, t, sm);
  else if constexpr (KB == 28 && BM == 1) gemv_run<BM, BF16, 14, 2, 1>(a, d, t, sm);
  else if constexpr (KB == 28) gemv_run<BM, BF16, 7, 4, 1>(a, d, t, sm);
  else gemv_run<BM, BF16, 0, 1, 1>(a, d, t, sm);
}

template <class S>
__device__ __forceinline__ void gemv_spec(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm) {
  if constexpr (S::BM == 32) {  // batched tiles on the matrix cores (every GEMV of the graph)
    gemv_mfma(a, d, t, sm);
    return;
  } else if constexpr (S::BM == 16) {  // small-batch tiles on the matrix cores (batch <= 8)
    gemv_mfma_small(a, d, t, sm);
    return;
  }
  constexpr int VEC = S::WBF16 ? 8 : 4;
  const int kb = (d.k / VEC + 63) >> 6;
  if (S::KBA > 0 && kb == S::KBA) gemv_kb<S::BM, S::WBF16, S::KBA>(a, d, t, sm);
  else if (S::KBD > 0 && S::KBD != S::KBA && kb == S::KBD) gemv_kb<S::BM, S::WBF16, S::KBD>(a, d, t, sm);
  else gemv_run<S::BM, S::WBF16, 0, 1, 1>(a, d, t, sm);
}

// Run task t.
template <class S>
__device__ __forceinline__ void run_task_spec(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm) {
  switch (d.op_id) {
    case MK_OP_GEMV: gemv_spec<S>(a, d, t, sm); break;
    case MK_OP_ATTENTION_APPEND: task_append(a, d, t, sm); break;
    case MK_OP_ATTENTION_PARTIAL: task_partial_kv<S::KVBF16, S::BM == 32, (S::BM > 1 ? 2 : 1)>(a, d, t, sm); break;
    case MK_OP_ATTENTION_COMBINE: task_combine(a, d, t, sm); break;
    case MK_OP_MEMCPY: task_memcpy(a, d, t, sm); break;
    case MK_OP_RMSNORM: task_rmsnorm(a, d, t, sm); break;
    case MK_OP_SAMPLE: task_sample(a, d, t, sm); break;
    default: break;  // NOP joins never run as tasks: their children poll their counter
  }
}

__device__ __forceinline__ uint32_t claim_ticket(const LaunchArgs& a) {
  return __hip_atomic_fetch_add((MK_GLOBAL uint32_t*)&a.ctrl->head, 1u, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT) - a.ticket_base;
}

// Thread 0 stages descriptor t (64 bytes) into LDS slot `slot`.
__device__ __forceinline__ void stage_desc(const LaunchArgs& a, uint32_t t, Smem& sm, int slot) {
  u32x4* dst = (u32x4*)&sm.desc[slot];
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = ldg<u32x4>(a.tasks, (size_t)t * 4 + i);
}

// Every thread reads the staged descriptor as wave-uniform (scalar) values.
__device__ __forceinline__ mk_task_t read_desc(const Smem& sm, int slot) {
  uint32_t w[16];
  const uint32_t* p = (const uint32_t*)&sm.desc[slot];
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i] = __builtin_amdgcn_readfirstlane(p[i]);
  mk_task_t d;
  __builtin_memcpy(&d, w, sizeof(d));
  return d;
}

// The next task of this workgroup: the next entry of its static list, or (dynamic
// mode) the next ticket of the device-wide counter.  NOP joins are skipped: their
// children poll the join's counter.  Thread 0 only.
__device__ __forceinline__ uint32_t next_task(const LaunchArgs& a, uint32_t& pos, uint32_t end) {
  if (a.order_off) return pos < end ? ldg<uint32_t>(a.order, pos++) : 0xFFFFFFFFu;
  for (;;) {
    const uint32_t t = claim_ticket(a);
    if (t >= a.n_tasks) return 0xFFFFFFFFu;
    if (ldg<uint16_t>(a.tasks, (size_t)t * 32) != MK_OP_NOP) return t;
  }
}

// The persistent interpreter.  Tasks are fetched two ahead: while task i runs, the
// descriptors of tasks i and i + 1 are in LDS and the id of task i + 2 is being
// fetched (the claim's round trip, or the list read, overlaps the current task); the
// descriptor of task i + 2 is copied into its LDS slot right after task i's release.
// Descriptors and ids rotate through three LDS slots, which is safe because every
// iteration ends in a workgroup barrier and slot i + 2 is written only at the end of
// iteration i.  In dynamic mode each workgroup makes exactly one failing claim
// per step, so the ticket counter advances by n_tasks + grid per step and never needs
// a reset; a workgroup holding two claimed tasks runs them in claim order, so the
// lowest unfinished task is always running.  Trace mode (a.trace != null) records
// timestamps.
template <class S>
__global__ __launch_bounds__(kThreads, 1) void interpreter_kernel(LaunchArgs a) {
  __shared__ Smem sm;
  const bool trace = a.trace != nullptr;
  uint32_t pos = 0, end = 0;  // static list cursor (thread 0)
  if (threadIdx.x == 0) {
    if (a.order_off) {
      pos = ldg<uint32_t>(a.order_off, blockIdx.x);
      end = ldg<uint32_t>(a.order_off, blockIdx.x + 1);
    }
    uint32_t t0 = next_task(a, pos, end);
    if (read_status(a) != 0) t0 = 0xFFFFFFFFu;
    const uint32_t t1 = t0 < a.n_tasks ? next_task(a, pos, end) : 0xFFFFFFFFu;
    sm.ticket[0] = t0;
    sm.ticket[1] = t1;
    sm.stop = 0;
    if (t0 < a.n_tasks) stage_desc(a, t0, sm, 0);
    if (t1 < a.n_tasks) stage_desc(a, t1, sm, 1);
  }
  __syncthreads();
  for (int s = 0;; s = s == 2 ? 0 : s + 1) {
    const int s1 = s == 2 ? 0 : s + 1, s2 = s1 == 2 ? 0 : s1 + 1;
    const uint32_t t = __builtin_amdgcn_readfirstlane(sm.ticket[s]);
    if (t >= a.n_tasks || __builtin_amdgcn_readfirstlane(sm.stop) != 0) break;
    const mk_task_t d = read_desc(sm, s);
    const uint32_t tn = __builtin_amdgcn_readfirstlane(sm.ticket[s1]);
    uint64_t t_claim = 0;
    uint32_t nn = 0xFFFFFFFFu, status = 0;
    if (threadIdx.x == 0) {
      if (trace) {
        t_claim = clock100();
        sm.t_mark[0] = sm.t_mark[1] = sm.t_mark[2] = 0;
      }
      if (tn < a.n_tasks) nn = next_task(a, pos, end);
      // Read while the task runs: a read issued after the task body would hold up the
      // release, which waits for all of the workgroup's outstanding memory operations.
      status = read_status(a);
    }
    run_task_spec<S>(a, d, t, sm);
    uint64_t t_end = 0;
    if (threadIdx.x == 0) {
      if (trace) t_end = clock100();
      if (status != 0) sm.stop = 1;
      sm.ticket[s2] = nn;
    }
    release_dependents(a, d);
    // Descriptor i + 2 is copied into its slot after the release (a load issued before
    // it would hold the release up): lanes 0..3 of wave 0 each copy 16 bytes with a
    // global-to-LDS load.  The next iteration's release waits for it and meets at a
    // barrier, so the slot is complete before it is read two iterations on.
    if (wave_id() == 0) {
      const uint32_t ln = lane_id();
      const uint32_t t2 = sm.ticket[s2];
      if (ln < 4 && t2 < a.n_tasks)
        __builtin_amdgcn_global_load_lds((const MK_GLOBAL void*)((const MK_GLOBAL u32x4*)a.tasks + (size_t)t2 * 4 + ln),
                                         (__attribute__((address_space(3))) void*)&sm.desc[s2], 16, 0, 0);
    }
    if (trace && threadIdx.x == 0) {
      const uint64_t t_rel = clock100();
      const uint32_t hw = __builtin_amdgcn_s_getreg((4) | (0 << 6) | (31 << 11));   // HW_ID
      const uint32_t xcc = __builtin_amdgcn_s_getreg((20) | (0 << 6) | (31 << 11));  // XCC_ID
      stg<uint64_t>(a.trace, 8ull * t + 0, ((uint64_t)xcc << 32) | hw);
      stg<uint64_t>(a.trace, 8ull * t + 1, t_claim);
      stg<uint64_t>(a.trace, 8ull * t + 2, sm.t_ready);
      stg<uint64_t>(a.trace, 8ull * t + 3, t_end);
      stg<uint64_t>(a.trace, 8ull * t + 4, t_rel);
      for (int i = 0; i < 3; ++i) stg<uint64_t>(a.trace, 8ull * t + 5 + i, sm.t_mark[i]);
    }
  }
  // A stop after an error can leave the last descriptor copy in flight.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// One launch per op: blockIdx.x = task within the op; stream order replaces the
// readiness counters.
template <class S>
__global__ __launch_bounds__(kThreads, 1) void per_op_kernel(LaunchArgs a) {
  __shared__ Smem sm;
  const uint32_t t = a.first_task + blockIdx.x;
  if (threadIdx.x == 0) stage_desc(a, t, sm, 0);
  __syncthreads();
  mk_task_t d = read_desc(sm, 0);
  d.remaining_deps = 0;
  run_task_spec<S>(a, d, t, sm);
}

// Level-synchronous variant ("Mega kernel initial", 1y33.com, the level section: the
// host groups task indices by level and a grid barrier separates the levels), with the
// same task bodies.  Every workgroup runs its round-robin share of a level, then all
// meet at a device-wide barrier before the next level.  No readiness counters: every
// parent of a task sits in an earlier level.  The barrier counts arrivals on one
// monotone counter in the control block (target barrier_base + (level + 1) * grid, so
// it needs no reset) after each workgroup's stores are acknowledged, and polls it with
// the bounded wait of a dependency (a timeout reports task index 0x0FFFFFFF).
template <class S>
__global__ __launch_bounds__(kThreads, 1) void level_kernel(LaunchArgs a) {
  __shared__ Smem sm;
  const uint32_t G = gridDim.x;
  // A step after a failed one (sticky status word, cleared by mk_status) runs
  // nothing; a workgroup that leaves here never arrives at a barrier, and the
  // others' barrier polls give up on the same status word.
  if (threadIdx.x == 0) sm.flag = read_status(a) == 0;
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(sm.flag) == 0) return;
  for (uint32_t lv = 0; lv < a.n_levels; ++lv) {
    const uint32_t b = ldg<uint32_t>(a.lvl_off, lv), e = ldg<uint32_t>(a.lvl_off, lv + 1);
    for (uint32_t i = b + blockIdx.x; i < e; i += G) {
      const uint32_t t = ldg<uint32_t>(a.lvl, i);
      if (threadIdx.x == 0) stage_desc(a, t, sm, 0);
      __syncthreads();
      mk_task_t d = read_desc(sm, 0);
      d.remaining_deps = 0;
      run_task_spec<S>(a, d, t, sm);
      // Every wave's loads (LDS copies included) have landed and every wave is done
      // with the LDS before the next descriptor is staged.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this workgroup's stores acknowledged
    __syncthreads();
    if (threadIdx.x == 0) {
      MK_GLOBAL uint32_t* bar = (MK_GLOBAL uint32_t*)&a.ctrl->barrier;
      __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sm.flag = poll_counter(a, 0x0FFFFFFFu, (const uint32_t*)&a.ctrl->barrier, a.barrier_base + (lv + 1) * G);
    }
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(sm.flag) == 0) break;  // step abandoned
  }
}

struct KernelSet {
  const void* persistent;
  const void* per_op;
  const void* levels;
};

template <class S>
KernelSet kernel_set() {
  return KernelSet{(const void*)interpreter_kernel<S>, (const void*)per_op_kernel<S>, (const void*)level_kernel<S>};
}

}  // namespace mk
