// Task bodies of the interpreter (one device function per OpId of the page's OpId
// table that a Llama-style layer uses, plus MEMCPY and the NOP join), shared by the
// persistent kernel and by the per-op-launch baseline (dispatch: kernels.h).  Each
// body: resolve its buffers, prefetch static inputs, wait for its own producers
// (dep_wait), compute, return; the caller releases the dependents.
#pragma once

#include "device_common.h"
#include "task_attn.h"
#include "task_gemv.h"
#include "task_gemv_mfma.h"

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

}  // namespace mk
