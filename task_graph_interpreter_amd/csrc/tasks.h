// Task bodies of the interpreter (one device function per OpId of the page's OpId
// table that a Llama-style layer uses, plus MEMCPY and the NOP join), shared by the
// persistent kernel and by the per-op-launch baseline (dispatch: kernels.h).  Each
// body: resolve its buffers, prefetch static inputs, wait for its own producers
// (dep_wait), compute, return; the caller releases the dependents.
#pragma once

#include <climits>

#include "device_common.h"
#include "task_attn.h"
#include "task_gemv.h"
#include "task_gemv_mfma.h"
#include "task_gemv_mfma_small.h"

namespace mk {

// ---------------------------------------------------------------------------------
// MEMCPY: embedding gather x0[b, :] = E[tokens[b], :] widened to fp32 (utility OpId
// of the page's table, used here for the embedding lookup).
// ---------------------------------------------------------------------------------
__device__ __forceinline__ void task_memcpy(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm) {
  const int B = d.m, H = d.n;
  const int32_t* tokens = (const int32_t*)resolve(a, d.in_buf[0]);
  const char* E = resolve(a, d.in_buf[1]);
  float* x0 = (float*)resolve(a, d.out_buf);
  if (!dep_wait(a, t, d.remaining_deps, sm)) return;
  for (int b = 0; b < B; ++b) {
    int tok = ldg<int32_t>(tokens, b);
    if (tok < 0 || tok >= a.vocab) {
      if (threadIdx.x == 0) raise_status(a, MK_STATUS_BAD_TOKEN | t);
      tok = 0;
    }
    for (int k = threadIdx.x; k < H; k += kThreads) {
      float v;
      if (d.config_id == MK_DTYPE_BF16) v = __uint_as_float((uint32_t)ldg<uint16_t>(E, (size_t)tok * H + k) << 16);
      else v = ldg<float>(E, (size_t)tok * H + k);
      st_dev<float>(x0, (size_t)b * H + k, v);
    }
  }
}

// ---------------------------------------------------------------------------------
// RMSNORM (OpId 3 of the page's OpId table; FUSED_RESIDUAL from its flags paragraph),
// for graphs lowered without epilogue fusion: row b = reserved[0] of
//   v = x[b] (+ residual[b] with FUSED_RESIDUAL, the sum also stored to buffer
//   reserved[1]);  out[b] = v (mean(v^2) + eps)^-1/2 gamma.
// The row is staged in LDS while its sum of squares is taken.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ void task_rmsnorm(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm) {
  const int b = (int)d.reserved[0], H = d.n;
  const bool res = d.flags & MK_FLAG_FUSED_RESIDUAL;
  const float* x = (const float*)resolve(a, d.in_buf[0]);
  const char* gamma = resolve(a, d.in_buf[1]);
  const float* r = res ? (const float*)resolve(a, d.in_buf[2]) : nullptr;
  float* y = (float*)resolve(a, d.out_buf);
  float* sum = res ? (float*)resolve(a, d.reserved[1]) : nullptr;
  if (!dep_wait(a, t, d.remaining_deps, sm)) return;
  const size_t row = (size_t)b * H;
  float ss = 0.f;
  for (int k = threadIdx.x; k < H; k += kThreads) {
    float v = ld_dev<float>(x, row + k);
    if (res) {
      v += ld_dev<float>(r, row + k);
      st_dev<float>(sum, row + k, v);
    }
    sm.xs[k] = v;
    ss = fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  if (lane_id() == 0) sm.red[wave_id()] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int i = 0; i < kWaves; ++i) tot += sm.red[i];
  const float rinv = 1.0f / sqrtf(tot / (float)H + a.rms_eps);
  for (int k = threadIdx.x; k < H; k += kThreads) {
    const float g = d.config_id == MK_DTYPE_BF16 ? __uint_as_float((uint32_t)ldg<uint16_t>(gamma, k) << 16)
                                                 : ldg<float>(gamma, k);
    st_dev<float>(y, row + k, sm.xs[k] * rinv * g);
  }
}

// ---------------------------------------------------------------------------------
// SAMPLE (OpId 6 of the page's OpId table: greedy argmax at the end of a decode step):
// row b = reserved[0] of the logits (in_buf[0], [batch, vocab] fp32) -> out (the
// tokens buffer)[b] = the lowest index of the row's largest value (NaN never wins; a
// row with no comparable value gives 0), and positions (buffer reserved[1])[b] += 1,
// so the next launch embeds this token at the next position; also tokens_out[b] when
// the launch passes one.  Nothing is written if the step has failed.  The logits are
// this step's data: every thread reads 16-byte pieces of the row with device-scope
// buffer loads, 16 per round trip, then the workgroup reduces (value, index) pairs.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ void task_sample(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm) {
  const int b = (int)d.reserved[0], V = d.n;
  const float* logits = (const float*)resolve(a, d.in_buf[0]) + (size_t)b * V;
  int32_t* tokens = (int32_t*)resolve(a, d.out_buf);
  int32_t* positions = (int32_t*)resolve(a, d.reserved[1]);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)logits, (short)0, (int)((uint32_t)V * 4u), kRawBufferWord3);
  if (!dep_wait(a, t, d.remaining_deps, sm)) return;
  constexpr int U = 16;
  const int V4 = (V + 3) >> 2;
  float best = -INFINITY;
  int bi = INT32_MAX;
  for (int base = 0; base < V4; base += kThreads * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i4 = base + u * kThreads + (int)threadIdx.x;
      // past the row: out of range, reads nothing (and is skipped below)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, i4 < V4 ? (uint32_t)i4 * 16u : 0xFFFFFFF0u, 0,
                                                   kCachePolicySC1);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i0 = 4 * (base + u * kThreads + (int)threadIdx.x);
      const uint32_t e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float xv = __uint_as_float(e[j]);
        const int i = i0 + j;
        if (i < V && (xv > best || (xv == best && i < bi))) {
          best = xv;
          bi = i;
        }
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ob = __shfl_xor(best, off, 64);
    const int oi = __shfl_xor(bi, off, 64);
    if (ob > best || (ob == best && oi < bi)) {
      best = ob;
      bi = oi;
    }
  }
  if (lane_id() == 0) {
    sm.red[wave_id()] = best;
    sm.red[kWaves + wave_id()] = __int_as_float(bi);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kWaves; ++w) {
      const float ob = sm.red[w];
      const int oi = __float_as_int(sm.red[kWaves + w]);
      if (ob > best || (ob == best && oi < bi)) {
        best = ob;
        bi = oi;
      }
    }
    if (read_status(a) == 0) {
      const int32_t tok = bi == INT32_MAX ? 0 : bi;
      st_dev<int32_t>(tokens, b, tok);
      st_dev<int32_t>(positions, b, ldg<int32_t>(positions, b) + 1);
      if (a.tokens_out != nullptr) st_dev<int32_t>(a.tokens_out, b, tok);
    }
  }
}

}  // namespace mk
