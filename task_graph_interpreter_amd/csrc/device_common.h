// Device-side shared pieces of the interpreter: launch arguments, buffer-table
// resolution, explicit global-memory accessors, bf16 conversion, wavefront
// reductions, and the readiness protocol (acquire-wait on a task's own counter,
// release-increment of each dependent's).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mk.h"

namespace mk {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;  // 8 wave64s per workgroup, one workgroup per CU
constexpr int kWaves = kThreads / 64;
// LDS: x staging / attention merge.  Above half of the CU's 160 KB, so the persistent
// kernel gets exactly one workgroup per CU (co-residency of the whole grid).
constexpr int kSmemBytes = 128 * 1024;
constexpr int kRedFloats = 1024;  // reduction scratch

// Buffer-table entry tags (top byte): 0 = absolute device pointer; otherwise an
// offset into a per-step base passed at launch.
enum : uint32_t { TAG_ABS = 0, TAG_KCACHE = 1, TAG_VCACHE = 2, TAG_TOKENS = 3, TAG_POSITIONS = 4, TAG_LOGITS = 5 };
constexpr uint64_t kTagShift = 56;
constexpr uint64_t kOffMask = (uint64_t(1) << kTagShift) - 1;

struct Ctrl {
  uint32_t head;    // ticket counter (monotone across steps)
  uint32_t status;  // sticky device status word
  uint32_t pad[62];
};

struct Smem {
  float xs[kSmemBytes / 4];       // staged activations / attention merge
  float red[kRedFloats];          // reductions
  alignas(16) mk_task_t desc[2];  // current / next descriptor (double-buffered)
  uint64_t t_ready;               // trace: when the dependency wait ended
  uint32_t ticket[2];
  uint32_t flag;
};

struct LaunchArgs {
  const mk_task_t* tasks;
  // Dependents array as uploaded, with bit 31 set on edges whose child is a NOP join
  // (the CSR indices are unchanged; the flag saves a descriptor load per edge).
  const uint32_t* edges;
  const uint32_t* order;      // static schedule: task lists grouped by workgroup
  const uint32_t* order_off;  // [grid + 1]; null = dynamic tickets
  const uint64_t* table;
  uint32_t* arrivals;
  Ctrl* ctrl;
  uint64_t* trace;
  uint64_t rt[8];  // per-step bases indexed by tag
  uint32_t n_tasks;
  uint32_t epoch;
  uint32_t ticket_base;
  uint32_t first_task;  // per-op launches: first task of the op
  uint64_t wait_limit;  // ticks of the 100 MHz clock
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

// Wave index as a wave-uniform (scalar) value, so branches on it stay scalar.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ char* resolve(const LaunchArgs& a, uint32_t idx) {
  const uint64_t e = ldg<uint64_t>(a.table, idx);
  const uint32_t tag = (uint32_t)(e >> kTagShift);
  // Compare chain instead of indexing a.rt with a run-time tag (an indexed kernel
  // argument would be copied to private memory).
  uint64_t base = 0;
  base = tag == TAG_KCACHE ? a.rt[TAG_KCACHE] : base;
  base = tag == TAG_VCACHE ? a.rt[TAG_VCACHE] : base;
  base = tag == TAG_TOKENS ? a.rt[TAG_TOKENS] : base;
  base = tag == TAG_POSITIONS ? a.rt[TAG_POSITIONS] : base;
  base = tag == TAG_LOGITS ? a.rt[TAG_LOGITS] : base;
  return (char*)(base + (e & kOffMask));
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
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

// Sum across groups of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ uint64_t clock100() { return wall_clock64(); }

__device__ __forceinline__ void raise_status(const LaunchArgs& a, uint32_t code) {
  uint32_t expected = 0u;
  __hip_atomic_compare_exchange_strong((MK_GLOBAL uint32_t*)&a.ctrl->status, &expected, code, __ATOMIC_RELAXED,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t read_status(const LaunchArgs& a) {
  return __hip_atomic_load((MK_GLOBAL uint32_t*)&a.ctrl->status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until task t's counter shows all of this step's parents have arrived
// (arrivals[t] - epoch * indeg >= 0 in wrapping 32-bit arithmetic), then acquire at
// agent scope so every wave of the workgroup sees the producers' writes.  Bounded:
// on timeout (or if another workgroup raised an error) the step is abandoned.
// Returns false if the step was abandoned.  Called by all threads.
__device__ __forceinline__ bool dep_wait(const LaunchArgs& a, uint32_t t, int32_t indeg, Smem& sm) {
  if (indeg == 0) {
    if (threadIdx.x == 0) sm.t_ready = clock100();
    return true;
  }
  if (threadIdx.x == 0) {
    MK_GLOBAL uint32_t* cnt = (MK_GLOBAL uint32_t*)a.arrivals + t;
    const uint32_t target = a.epoch * (uint32_t)indeg;
    uint32_t ok = 1;
    uint32_t v = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((int32_t)(v - target) < 0) {
      const uint64_t t0 = clock100();
      for (;;) {
        __builtin_amdgcn_s_sleep(1);
        v = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((int32_t)(v - target) >= 0) break;
        if (clock100() - t0 > a.wait_limit) {
          raise_status(a, MK_STATUS_TIMEOUT | t);
          ok = 0;
          break;
        }
        if (read_status(a) != 0) {
          ok = 0;
          break;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    sm.flag = ok;
    sm.t_ready = clock100();
  }
  __syncthreads();
  return sm.flag != 0;
}

// Count one arrival on each of the n dependents listed at edges[off].  A NOP join is
// never run as a task: the parent whose increment completes its count (the returned
// old value is the last one short of epoch * indeg) fires it on the spot, counting
// one arrival on each of the NOP's own dependents.  NOP joins never feed NOP joins
// (checked when lowering), so this recursion is one level deep.  Wave 0 only; the
// caller has issued the release fence.
__device__ __forceinline__ void signal_dependents(const LaunchArgs& a, uint32_t off, uint32_t n) {
  const int lane = lane_id();
  for (uint32_t i0 = 0; i0 < n; i0 += 64) {
    const uint32_t i = i0 + lane;
    uint32_t fire = 0xFFFFFFFFu;
    if (i < n) {
      const uint32_t e = ldg<uint32_t>(a.edges, off + i);
      const uint32_t c = e & 0x7FFFFFFFu;
      MK_GLOBAL uint32_t* cnt = (MK_GLOBAL uint32_t*)a.arrivals + c;
      if (e >> 31) {
        const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t indeg = ldg<uint32_t>(a.tasks, (size_t)c * 16 + 2);  // remaining_deps
        if (old + 1u == a.epoch * indeg) fire = c;
      } else {
        __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    uint64_t pending = __ballot(fire != 0xFFFFFFFFu);
    while (pending) {
      const int src = __builtin_ctzll(pending);
      pending &= pending - 1;
      const uint32_t c = __builtin_amdgcn_readlane(fire, src);
      // Every other parent's data was released before its increment, which this wave
      // has now observed; order that before the NOP's own releases.
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const uint32_t nd = __builtin_amdgcn_readfirstlane(ldg<uint32_t>(a.tasks, (size_t)c * 16 + 3));
      const uint32_t no = __builtin_amdgcn_readfirstlane(ldg<uint32_t>(a.tasks, (size_t)c * 16 + 4));
      for (uint32_t j = lane; j < nd; j += 64) {
        const uint32_t cc = ldg<uint32_t>(a.edges, no + j) & 0x7FFFFFFFu;
        __hip_atomic_fetch_add((MK_GLOBAL uint32_t*)a.arrivals + cc, 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// Make this workgroup's writes visible at agent scope, then count one arrival on
// every dependent.  Called by all threads after the task body.
__device__ __forceinline__ void release_dependents(const LaunchArgs& a, const mk_task_t& d) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (wave_id() == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    signal_dependents(a, d.dependents_offset, (uint32_t)d.num_dependents);
  }
}

}  // namespace mk
