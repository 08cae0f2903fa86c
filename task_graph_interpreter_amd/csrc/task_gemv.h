// GEMV task body ("Mega kernel initial", lowering section: one task per output-column
// tile; descriptor section: flags SILU_MUL=1, ADD_RESIDUAL=2, RMS_NORM_INPUT=4):
//   y[b, c] = sum_k xin[b, k] W[c, k]  (+ res[b, c] with ADD_RESIDUAL)
//   xin = x (mean(x^2) + eps)^-1/2 gamma with RMS_NORM_INPUT; the scale r_b is applied
//   to the finished dot product, the gamma product while staging x
//   SILU_MUL: y[b, c] = silu(g) u with g from weight row c and u from row I + c.
//
// Streaming layout (HBM-bound; no MFMA: the contraction has M <= 8 rows):
//  * wavefront w owns the tile's outputs w, w + 8, ...; each output is one logical
//    weight row (two with SILU_MUL: gate, then up);
//  * a row is read in "kblocks": 64 lanes x 16 contiguous bytes = 1 KB, coalesced;
//  * one loop iteration consumes RPG whole rows held in a ring of RPG * KBT registers
//    and refills each slot with the same kblock of the row RPG ahead, so RPG * KBT
//    16-byte loads per lane stay in flight.  The loop body is straight-line code:
//    loads are unconditional, so the compiler's wait counts stay exact instead of
//    draining the ring at every branch.  Weights are read with buffer loads; a slot
//    refilled past the wave's last row gets an offset beyond the buffer's range, which
//    the hardware answers with zeros and no memory access (its result is discarded);
//  * the ring's first fill is issued before the dependency wait: weights are static,
//    so the tile's first bytes arrive while its producers are still finishing;
//  * one wave (the control wave) waits for the producers and stages the input rows
//    in LDS (fp32, x * gamma) while the other waves' rings are still landing: a
//    wave's loads complete in issue order, so its poll queues only behind its own
//    ring.  No larger prefetch is issued: requests queued in the workgroup's memory
//    pipeline hold up the poll at the moment the producers finish;
//  * a finished row is reduced across the wavefront with DPP (no LDS traffic) and
//    parked in the register of lane (row % 64); parked results are stored 64 at a
//    time, outside the streaming loop for every shape the workloads use.
#pragma once

#include <type_traits>

#include "device_common.h"

namespace mk {

// Range of the weight buffer resource: every offset of a matrix (< 4 GiB, checked when
// lowering, rows a multiple of 16 bytes) is below it; kPastEnd is not.
constexpr uint32_t kWeightRange = 0xFFFFFFF0u;
constexpr uint32_t kPastEnd = 0xFFFFFFF0u;
// The wave that waits for a tile's producers and stages its input (it streams its own
// rows too).
constexpr int kCtrlWave = kWaves - 1;
// s_waitcnt operand: vector memory counter 0, the others unconstrained.
constexpr int kWaitVmcnt0 = 0x0F70;

struct GemvGeom {
  const char* W;
  __amdgpu_buffer_rsrc_t wr;  // raw buffer over W (stride 0, range kWeightRange)
  int K, KC;      // inner dim, 16-byte chunks per row
  int c0, I;      // first output column, up-row offset (SILU_MUL)
  int nout, NQ;   // outputs of this wave, logical rows of this wave
  int wave;       // wave index (scalar)
  int silu;
};

__device__ __forceinline__ u32x4 gemv_load(const GemvGeom& g, int q, int kb, int lane) {
  const bool past = q >= g.NQ;  // past the wave's last row: out of range, reads nothing
  const int j = g.silu ? (q >> 1) : q;
  const int row = g.c0 + g.wave + kWaves * j + ((g.silu && (q & 1)) ? g.I : 0);
  int chunk = kb * 64 + lane;
  chunk = chunk < g.KC ? chunk : g.KC - 1;  // partial last kblock: masked when consumed
  // 32-bit byte offset into the matrix (every weight matrix is < 4 GiB).
  const uint32_t off = ((uint32_t)row * (uint32_t)g.KC + (uint32_t)chunk) * 16u;
  return __builtin_amdgcn_raw_buffer_load_b128(g.wr, past ? kPastEnd : off, 0, kCachePolicyNT);
}

template <int BM, bool BF16>
__device__ __forceinline__ void gemv_consume(const u32x4 w, const float* xs, int K, int chunk, bool valid, int nb,
                                             float acc[BM]) {
  constexpr int VEC = BF16 ? 8 : 4;
  float wf[8];
  if (BF16) {
    wf[0] = bf16_lo(w.x); wf[1] = bf16_hi(w.x); wf[2] = bf16_lo(w.y); wf[3] = bf16_hi(w.y);
    wf[4] = bf16_lo(w.z); wf[5] = bf16_hi(w.z); wf[6] = bf16_lo(w.w); wf[7] = bf16_hi(w.w);
  } else {
    wf[0] = __uint_as_float(w.x); wf[1] = __uint_as_float(w.y);
    wf[2] = __uint_as_float(w.z); wf[3] = __uint_as_float(w.w);
    wf[4] = wf[5] = wf[6] = wf[7] = 0.f;
  }
  const float m = valid ? 1.f : 0.f;  // a masked chunk contributes 0
  chunk = valid ? chunk : 0;
#pragma unroll
  for (int b = 0; b < BM; ++b) {
    if (b < nb) {
      const f32x4* xb = (const f32x4*)(xs + b * K + chunk * VEC);
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < VEC / 4; ++e) {
        const f32x4 xv = xb[e];
        s = fmaf(wf[4 * e + 0], xv.x, s);
        s = fmaf(wf[4 * e + 1], xv.y, s);
        s = fmaf(wf[4 * e + 2], xv.z, s);
        s = fmaf(wf[4 * e + 3], xv.w, s);
      }
      acc[b] = fmaf(s, m, acc[b]);
    }
  }
}

// Wait for the tile's producers (the control wave polls), then stage its input rows
// 0 .. nb-1 into LDS on every wave: each thread copies its share of the rows with
// device-scope (sc1) global-to-LDS loads and, with RMS_NORM_INPUT, scales the same
// elements by gamma (loaded meanwhile) and sums their squares, so no wave waits for
// another's copies; the waves' partial sums meet in LDS at the closing barrier.
// Returns r_b (1 without the norm) in rs[], or false if the step was abandoned.  The
// control wave's poll queues only behind its own weight ring.
template <int BM, bool GBF16>
__device__ __forceinline__ bool gemv_wait_stage(const LaunchArgs& a, uint32_t t, int32_t indeg, const float* x,
                                                const char* gamma, bool norm, int K, int nb, float eps, Smem& sm,
                                                float rs[BM]) {
  const bool ctrl = wave_id() == kCtrlWave;
  const int lane = lane_id(), w = wave_id();
  if (ctrl && lane == 0) {
    sm.flag = poll_deps(a, t, indeg);
    sm.t_ready = clock100();
  }
  __syncthreads();
  const uint32_t ok = __builtin_amdgcn_readfirstlane(sm.flag);
  float* part = sm.red + kRedFloats - 128;  // [BM][kWaves] partial sums of squares
  if (ok) {
    const int K4 = K >> 2;
    for (int b = 0; b < nb; ++b)
      for (int c = w * 64; c < K4; c += kThreads)
        if (c + lane < K4)
          __builtin_amdgcn_global_load_lds((const MK_GLOBAL void*)((const MK_GLOBAL f32x4*)x + (size_t)b * K4 + c + lane),
                                           (__attribute__((address_space(3))) void*)(sm.xs + (size_t)b * K + 4 * c),
                                           16, 0, kCachePolicySC1);
    // gamma (weight dtype) in raw form: 8 bytes per 4 values in bf16, 16 in fp32; the
    // thread's chunks are k4 = 64 w + lane + 512 j, the ones it copied.
    typedef typename std::conditional<GBF16, u32x2, u32x4>::type graw_t;
    constexpr int GB = 8;
    for (int b = 0; b < nb; ++b) {
      f32x4* xo = (f32x4*)(sm.xs + (size_t)b * K);
      float ss = 0.f;
      for (int c0 = w * 64 + lane; c0 < K4; c0 += kThreads * GB) {
        graw_t gv[GB];
        if (norm) {
#pragma unroll
          for (int u = 0; u < GB; ++u) {
            const int k4 = c0 + u * kThreads;
            gv[u] = ldg<graw_t>(gamma, k4 < K4 ? k4 : 0);
          }
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this thread's LDS copies have landed
        if (norm) {
#pragma unroll
          for (int u = 0; u < GB; ++u) {
            const int k4 = c0 + u * kThreads;
            if (k4 < K4) {
              f32x4 v = xo[k4];
              ss = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss))));
              f32x4 gf;
              if constexpr (GBF16) gf = f32x4{bf16_lo(gv[u].x), bf16_hi(gv[u].x), bf16_lo(gv[u].y), bf16_hi(gv[u].y)};
              else gf = f32x4{__uint_as_float(gv[u].x), __uint_as_float(gv[u].y), __uint_as_float(gv[u].z),
                              __uint_as_float(gv[u].w)};
              xo[k4] = v * gf;
            }
          }
        }
      }
      if (norm) {
        ss = wave_sum(ss);
        if (lane == 0) part[b * kWaves + w] = ss;
      }
    }
  }
  __syncthreads();
  // Trace mode: when the input was staged (mark 2; marks 0 and 1 are thread 0's).
  if (a.trace != nullptr && ctrl && lane == 0) sm.t_mark[2] = clock100();
  // Every wave now waits for its own ring and input copies.  Written as the builtin
  // (not inline asm) so that the compiler's wait-count tracking sees it: otherwise
  // the copies' pending LDS writes would make it put a full wait before every LDS
  // read of the staged input inside the streaming loop, draining the ring each step.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  if (ok == 0) return false;
#pragma unroll
  for (int b = 0; b < BM; ++b) {
    float tot = 0.f;
    if (norm && b < nb) {
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) tot += part[b * kWaves + ww];
    }
    rs[b] = (norm && b < nb) ? 1.0f / sqrtf(tot / (float)K + eps) : 1.f;
  }
  return true;
}

// Store the parked results of logical rows [q_base, q_base + 64) of this wave (lane l
// holds row q_base + l): SiLU*mul pairs gate (even row) with up (odd row) through a
// lane swap; the residual is added at store time.
template <int BM>
__device__ __forceinline__ void gemv_flush(const GemvGeom& g, const float park[BM], int q_base, int nb, bool resid,
                                           const float* res, float* y, int N, int b0) {
  const int lane = lane_id();
  const int q = q_base + lane;
#pragma unroll
  for (int b = 0; b < BM; ++b) {
    if (b < nb) {
      float v = park[b];
      if (g.silu) {
        const float up = __shfl_xor(v, 1, 64);
        v = v / (1.f + __expf(-v)) * up;
      }
      const bool mine = q < g.NQ && (!g.silu || !(q & 1));
      if (mine) {
        const int j = g.silu ? (q >> 1) : q;
        const int c = g.c0 + g.wave + kWaves * j;
        const size_t o = (size_t)(b0 + b) * N + c;
        st_dev<float>(y, o, v + (resid ? ld_dev<float>(res, o) : 0.f));
      }
    }
  }
}

// Geometry of this wave's share of GEMV tile d.
template <bool BF16>
__device__ __forceinline__ GemvGeom gemv_geom(const LaunchArgs& a, const mk_task_t& d, int wave) {
  constexpr int VEC = BF16 ? 8 : 4;
  GemvGeom g;
  g.wave = wave;
  g.W = resolve(a, d.in_buf[1]);
  g.wr = __builtin_amdgcn_make_buffer_rsrc((void*)g.W, (short)0, (int)kWeightRange, kRawBufferWord3);
  g.K = d.k;
  g.KC = d.k / VEC;
  g.c0 = (int)d.reserved[0];
  g.I = (int)d.reserved[2];
  g.silu = (d.flags & MK_FLAG_SILU_MUL) ? 1 : 0;
  const int cnt = (int)d.reserved[1];
  g.nout = cnt > g.wave ? (cnt - g.wave + kWaves - 1) / kWaves : 0;
  g.NQ = g.nout << g.silu;
  return g;
}

// Batch rows staged per pass of a tile with inner dimension K.
template <int BM>
__device__ __forceinline__ int gemv_batch_pass(int K) {
  const int bp = (kSmemBytes / 4) / K;
  return bp < BM ? bp : BM;
}

// A row is SEG segments of KBT kblocks (compile time; KBT = 0: any K, one kblock at a
// time); RPG rows are in flight per wave.  Ring slot (r, kb) cycles through kblock
// s * KBT + kb of row r for s = 0 .. SEG-1, then moves to the row RPG ahead.
template <int BM, bool BF16, int KBT, int SEG, int RPG>
__device__ __forceinline__ void gemv_run(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm) {
  constexpr int KBS = KBT > 0 ? KBT : 1;
  int lane = lane_id();
  // Opaque to the optimiser: the per-lane offsets below are recomputed in each task
  // (a few instructions) instead of being hoisted out of the interpreter loop, where
  // they were spilled and came back as a chain of dependent scratch loads.
  asm volatile("" : "+v"(lane));
  const GemvGeom g = gemv_geom<BF16>(a, d, wave_id());
  const int KB = KBT > 0 ? KBT : (g.KC + 63) >> 6;
  const int N = d.n, B = d.m;
  const float* x = (const float*)resolve(a, d.in_buf[0]);
  const char* aux = d.in_buf[2] != 0xFFFF ? resolve(a, d.in_buf[2]) : nullptr;
  float* y = (float*)resolve(a, d.out_buf);
  const bool norm = d.flags & MK_FLAG_RMS_NORM_INPUT;
  const bool resid = d.flags & MK_FLAG_ADD_RESIDUAL;
  const int bp = gemv_batch_pass<BM>(g.K);

  for (int b0 = 0; b0 < B; b0 += bp) {
    const int nb = (B - b0) < bp ? (B - b0) : bp;
    // The register ring's first rows are loaded before the dependency wait (weights are
    // static).  Nothing larger is issued ahead: a bulk prefetch queued in the same
    // memory pipeline delays the control wave's poll by microseconds at the moment the
    // producers finish, which costs more than the prefetch saves.
    u32x4 buf[RPG][KBS];
    if (KBT > 0 && g.NQ > 0) {
#pragma unroll
      for (int r = 0; r < RPG; ++r)
#pragma unroll
        for (int kb = 0; kb < KBS; ++kb) buf[r][kb] = gemv_load(g, r, kb, lane);
    }
    float rs[BM];
    // One call site for every batch pass (later passes have no producers to wait
    // for): staging code duplicated on two paths into the streaming loop made the
    // compiler's wait counts there drain the whole ring at every row.
    if (!gemv_wait_stage<BM, BF16>(a, t, b0 == 0 ? d.remaining_deps : 0, x + (size_t)b0 * g.K, aux, norm, g.K, nb,
                                   a.rms_eps, sm, rs))
      return;
    if (b0 == 0) trace_mark(a, sm, 0);
    float park[BM];
#pragma unroll
    for (int b = 0; b < BM; ++b) park[b] = 0.f;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // nothing pending into LDS (ring already landed)
    // Short compiled rings: the last ring iteration refills nothing.  Its next-row
    // refills would all fall past the wave's last row, and such loads still in flight
    // at the end of the stream complete behind the workgroup's other loads and hold up
    // the flush (1B: 0.792 -> 0.787 ms).  The same peel of the 8-kblock ring pushed the
    // 8B kernel into spills, so longer rings keep the single loop.
    if constexpr (KBT > 0 && SEG == 1 && KBS <= 4) {
      auto iteration = [&](int it, auto refill_c) __attribute__((always_inline)) {
        constexpr bool REFILL = decltype(refill_c)::value;
        const int q0 = it * RPG;
#pragma unroll
        for (int r = 0; r < RPG; ++r) {
          float acc[BM];
#pragma unroll
          for (int b = 0; b < BM; ++b) acc[b] = 0.f;
#pragma unroll
          for (int kb = 0; kb < KBS; ++kb) {
            const int chunk = kb * 64 + lane;
            gemv_consume<BM, BF16>(buf[r][kb], sm.xs, g.K, chunk, chunk < g.KC, nb, acc);
            if (REFILL) buf[r][kb] = gemv_load(g, q0 + RPG + r, kb, lane);
          }
          const int q = q0 + r;
#pragma unroll
          for (int b = 0; b < BM; ++b) {
            if (b < nb) {
              const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_sum_dpp(acc[b])), 63));
              park[b] = (lane == (q & 63)) ? v * rs[b] : park[b];
            }
          }
          if ((q & 63) == 63 && q + 1 < g.NQ)  // more than 64 rows per wave: flush now
            gemv_flush<BM>(g, park, q - 63, nb, resid, (const float*)aux, y, N, b0);
        }
      };
      if (g.NQ > 0) {
        const int iters_ring = (g.NQ + RPG - 1) / RPG;
        for (int it = 0; it + 1 < iters_ring; ++it) iteration(it, std::true_type{});
        iteration(iters_ring - 1, std::false_type{});
      }
    } else {
      if (g.NQ > 0) {
        const int iters_ring = (g.NQ + RPG - 1) / RPG;
        for (int it = 0; it < iters_ring; ++it) {
          const int q0 = it * RPG;
          // Short rows: the compiler may keep the staged input in registers across rows.
          // Long rows: an opaque offset keeps the LDS reads inside the loop instead of
          // pinning 8 registers per kblock.
          int xoff = 0;
          if (KBS * SEG > 8) asm volatile("" : "+v"(xoff));
          const float* xsr = sm.xs + xoff;
  #pragma unroll
          for (int r = 0; r < RPG; ++r) {
            float acc[BM];
  #pragma unroll
            for (int b = 0; b < BM; ++b) acc[b] = 0.f;
            if (KBT > 0) {
  #pragma unroll
              for (int s = 0; s < SEG; ++s) {
  #pragma unroll
                for (int kb = 0; kb < KBS; ++kb) {
                  const int chunk = (s * KBS + kb) * 64 + lane;
                  gemv_consume<BM, BF16>(buf[r][kb], xsr, g.K, chunk, chunk < g.KC, nb, acc);
                  if (s + 1 < SEG) buf[r][kb] = gemv_load(g, q0 + r, (s + 1) * KBS + kb, lane);
                  else buf[r][kb] = gemv_load(g, q0 + RPG + r, kb, lane);
                }
              }
            } else {
              for (int kb = 0; kb < KB; ++kb) {
                const int chunk = kb * 64 + lane;
                const u32x4 w = gemv_load(g, q0 + r, kb, lane);
                gemv_consume<BM, BF16>(w, sm.xs, g.K, chunk, chunk < g.KC, nb, acc);
              }
            }
            const int q = q0 + r;
  #pragma unroll
            for (int b = 0; b < BM; ++b) {
              if (b < nb) {
                const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_sum_dpp(acc[b])), 63));
                park[b] = (lane == (q & 63)) ? v * rs[b] : park[b];
              }
            }
            if ((q & 63) == 63 && q + 1 < g.NQ)  // more than 64 rows per wave: flush now
              gemv_flush<BM>(g, park, q - 63, nb, resid, (const float*)aux, y, N, b0);
          }
        }
      }
    }
    if (g.NQ > 0) {
      if (b0 == 0) trace_mark(a, sm, 1);
      gemv_flush<BM>(g, park, ((g.NQ - 1) >> 6) << 6, nb, resid, (const float*)aux, y, N, b0);
    }
    if (b0 + bp < B) __syncthreads();  // LDS reused by the next batch block
  }
}

}  // namespace mk
