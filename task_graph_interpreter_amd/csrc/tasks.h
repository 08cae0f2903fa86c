// Task bodies of the interpreter (one device function per OpId of the page's OpId
// table that a Llama-style layer uses, plus MEMCPY and the NOP join), shared by the
// persistent kernel and by the per-op-launch baseline.  Each body: resolve its
// buffers, wait for its own producers (dep_wait), compute, return; the caller
// releases the dependents.
#pragma once

#include "device_common.h"

namespace mk {

// ---------------------------------------------------------------------------------
// GEMV ("Mega kernel initial", lowering section: one task per output-column tile;
// descriptor section: flags SILU_MUL=1, ADD_RESIDUAL=2, RMS_NORM_INPUT=4).
//   y[b, c] = sum_k xin[b, k] * W[c, k]  (+ res[b, c] with ADD_RESIDUAL)
//   xin = x * (mean(x^2) + eps)^-1/2 * gamma  with RMS_NORM_INPUT
//   SILU_MUL: y[b, c] = silu(g) * u with g from row c and u from row I + c.
// One wavefront per output column: lanes stream the weight row(s) in 16-byte pieces
// against the staged input in LDS and reduce across the wavefront.
// ---------------------------------------------------------------------------------
template <int BM, bool BF16>
__device__ __forceinline__ void gemv_dot(const char* __restrict__ wrow, const float* xs, int K, int nb,
                                         float acc[BM]) {
  constexpr int VEC = BF16 ? 8 : 4;      // elements per 16-byte load
  const int lane = threadIdx.x & 63;
  const int KC = K / VEC;                // 16-byte chunks per row
  const u32x4* w4 = (const u32x4*)wrow;
  constexpr int SU = 8;
  for (int s0 = 0; s0 < KC; s0 += 64 * SU) {
    u32x4 wv[SU];
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      const int j = s0 + lane + 64 * u;
      if (j < KC) wv[u] = __builtin_nontemporal_load(w4 + j);
      else wv[u] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      const int j = s0 + lane + 64 * u;
      if (j >= KC) break;
      float wf[VEC];
      if (BF16) {
        wf[0] = bf16_lo(wv[u].x); wf[1] = bf16_hi(wv[u].x);
        wf[2] = bf16_lo(wv[u].y); wf[3] = bf16_hi(wv[u].y);
        wf[4 % VEC] = bf16_lo(wv[u].z); wf[5 % VEC] = bf16_hi(wv[u].z);
        wf[6 % VEC] = bf16_lo(wv[u].w); wf[7 % VEC] = bf16_hi(wv[u].w);
      } else {
        wf[0] = __uint_as_float(wv[u].x); wf[1] = __uint_as_float(wv[u].y);
        wf[2] = __uint_as_float(wv[u].z); wf[3] = __uint_as_float(wv[u].w);
      }
#pragma unroll
      for (int b = 0; b < BM; ++b) {
        if (b < nb) {
          const float4* xb = (const float4*)(xs + b * K + j * VEC);
          float s = acc[b];
#pragma unroll
          for (int e = 0; e < VEC / 4; ++e) {
            const float4 xv = xb[e];
            s = fmaf(wf[4 * e + 0], xv.x, s);
            s = fmaf(wf[4 * e + 1], xv.y, s);
            s = fmaf(wf[4 * e + 2], xv.z, s);
            s = fmaf(wf[4 * e + 3], xv.w, s);
          }
          acc[b] = s;
        }
      }
    }
  }
}

template <int BM, bool BF16>
__device__ void gemv_outputs(const mk_task_t& d, const char* W, const float* xs, const float* aux, float* y,
                             int b0, int nb) {
  constexpr int ES = BF16 ? 2 : 4;
  const int K = d.k, N = d.n;
  const int c0 = (int)d.reserved[0], cnt = (int)d.reserved[1], I = (int)d.reserved[2];
  const bool silu = d.flags & MK_FLAG_SILU_MUL;
  const bool resid = d.flags & MK_FLAG_ADD_RESIDUAL;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int i = wave; i < cnt; i += kWaves) {
    const int c = c0 + i;
    float acc[BM], accu[BM];
#pragma unroll
    for (int b = 0; b < BM; ++b) acc[b] = accu[b] = 0.f;
    gemv_dot<BM, BF16>(W + (size_t)c * K * ES, xs, K, nb, acc);
    if (silu) gemv_dot<BM, BF16>(W + (size_t)(I + c) * K * ES, xs, K, nb, accu);
#pragma unroll
    for (int b = 0; b < BM; ++b) {
      if (b < nb) {
        float g = wave_sum(acc[b]);
        if (silu) {
          const float u = wave_sum(accu[b]);
          g = g / (1.f + __expf(-g)) * u;
        }
        if (lane == 0) {
          if (resid) g += aux[(size_t)(b0 + b) * N + c];
          y[(size_t)(b0 + b) * N + c] = g;
        }
      }
    }
  }
}

__device__ void task_gemv(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm) {
  const int B = d.m, K = d.k;
  const bool bf16 = d.config_id != MK_GEMV_F32;
  const char* W = resolve(a, d.in_buf[1]);
  const float* x = (const float*)resolve(a, d.in_buf[0]);
  const float* aux = d.in_buf[2] != 0xFFFF ? (const float*)resolve(a, d.in_buf[2]) : nullptr;
  float* y = (float*)resolve(a, d.out_buf);
  const bool norm = d.flags & MK_FLAG_RMS_NORM_INPUT;
  if (!dep_wait(a, t, d.remaining_deps, sm)) return;
  int bp = (kSmemBytes / 4) / K;
  bp = bp < 8 ? bp : 8;
  for (int b0 = 0; b0 < B; b0 += bp) {
    const int nb = (B - b0) < bp ? (B - b0) : bp;
    // Stage (normalised) input rows b0..b0+nb into LDS.
    for (int b = 0; b < nb; ++b) {
      const float* xr = x + (size_t)(b0 + b) * K;
      float* xo = sm.xs + b * K;
      float ss = 0.f;
      for (int k = threadIdx.x; k < K; k += kThreads) {
        const float v = xr[k];
        xo[k] = v;
        ss = fmaf(v, v, ss);
      }
      if (norm) {
        const float tot = block_sum(ss, sm.red);
        const float r = 1.0f / sqrtf(tot / (float)K + a.rms_eps);
        for (int k = threadIdx.x; k < K; k += kThreads) {
          float g;
          if (bf16) g = bf16_lo(((const uint16_t*)aux)[k]);
          else g = ((const float*)aux)[k];
          xo[k] = xo[k] * r * g;
        }
      }
    }
    __syncthreads();
    if (bf16) {
      if (nb == 1) gemv_outputs<1, true>(d, W, sm.xs, aux, y, b0, nb);
      else gemv_outputs<8, true>(d, W, sm.xs, aux, y, b0, nb);
    } else {
      if (nb == 1) gemv_outputs<1, false>(d, W, sm.xs, aux, y, b0, nb);
      else gemv_outputs<8, false>(d, W, sm.xs, aux, y, b0, nb);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------
// MEMCPY: embedding gather x0[b, :] = E[tokens[b], :] widened to fp32 (utility OpId
// of the page's table, used here for the embedding lookup).
// ---------------------------------------------------------------------------------
__device__ void task_memcpy(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm) {
  const int B = d.m, H = d.n;
  const int32_t* tokens = (const int32_t*)resolve(a, d.in_buf[0]);
  const char* E = resolve(a, d.in_buf[1]);
  float* x0 = (float*)resolve(a, d.out_buf);
  if (!dep_wait(a, t, d.remaining_deps, sm)) return;
  for (int b = 0; b < B; ++b) {
    int tok = tokens[b];
    if (tok < 0 || tok >= a.vocab) {
      if (threadIdx.x == 0) raise_status(a, MK_STATUS_BAD_TOKEN | t);
      tok = 0;
    }
    for (int k = threadIdx.x; k < H; k += kThreads) {
      float v;
      if (d.config_id == MK_DTYPE_BF16) v = bf16_lo(((const uint16_t*)E)[(size_t)tok * H + k]);
      else v = ((const float*)E)[(size_t)tok * H + k];
      x0[(size_t)b * H + k] = v;
    }
  }
}

// ---------------------------------------------------------------------------------
// ATTENTION_APPEND ("RoPE-append current k,v" in the page's OpId table): for sequence
// b and KV head g, rotate the group's query heads and k_g (rotate-half RoPE, angle
// pos * theta^(-2i/hd) evaluated in fp64), write rotated q to q_rot and the rotated k
// and v into cache slot positions[b], rounded to the cache dtype.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ void rope_cs(int pos, int i, int hd, float theta, float& c, float& s) {
  const double inv = pow((double)theta, -2.0 * (double)i / (double)hd);
  const double ang = (double)pos * inv;
  double sd, cd;
  sincos(ang, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}

__device__ void task_append(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm) {
  const int b = (int)d.reserved[0], h0 = (int)d.reserved[1], hc = (int)d.reserved[2];
  const int g = d.k, hd = d.n, cap = d.kv_len;
  const int Hq = a.n_q_heads, Hkv = a.n_kv_heads;
  const float* qkv = (const float*)resolve(a, d.in_buf[0]);
  float* qrot = (float*)resolve(a, d.out_buf);
  char* kc = resolve(a, d.reserved[3]);
  char* vc = resolve(a, d.reserved[4]);
  const int32_t* positions = (const int32_t*)a.rt[TAG_POSITIONS];
  if (!dep_wait(a, t, d.remaining_deps, sm)) return;
  const int pos = positions[b];
  if (pos < 0 || pos >= cap) {
    if (threadIdx.x == 0) raise_status(a, MK_STATUS_BAD_POSITION | t);
    return;
  }
  const int half = hd / 2;
  const float* row = qkv + (size_t)b * (Hq + 2 * Hkv) * hd;
  const size_t slot = (((size_t)b * Hkv + g) * cap + pos) * hd;
  // (hc q heads + 1 k head) x half rotation pairs, then hd v elements.
  const int nrot = (hc + 1) * half;
  for (int e = threadIdx.x; e < nrot + hd; e += kThreads) {
    if (e < nrot) {
      const int hh = e / half, i = e % half;
      float c, s;
      rope_cs(pos, i, hd, a.rope_theta, c, s);
      const float* src = hh < hc ? row + (size_t)(h0 + hh) * hd : row + (size_t)(Hq + g) * hd;
      const float x0 = src[i], x1 = src[i + half];
      const float r0 = x0 * c - x1 * s;
      const float r1 = x1 * c + x0 * s;
      if (hh < hc) {
        float* dst = qrot + (size_t)b * Hq * hd + (size_t)(h0 + hh) * hd;
        dst[i] = r0;
        dst[i + half] = r1;
      } else if (d.config_id == MK_DTYPE_BF16) {
        ((uint16_t*)kc)[slot + i] = f32_to_bf16_rne(r0);
        ((uint16_t*)kc)[slot + i + half] = f32_to_bf16_rne(r1);
      } else {
        ((float*)kc)[slot + i] = r0;
        ((float*)kc)[slot + i + half] = r1;
      }
    } else {
      const int i = e - nrot;
      const float v = row[(size_t)(Hq + Hkv + g) * hd + i];
      if (d.config_id == MK_DTYPE_BF16) ((uint16_t*)vc)[slot + i] = f32_to_bf16_rne(v);
      else ((float*)vc)[slot + i] = v;
    }
  }
}

// ---------------------------------------------------------------------------------
// ATTENTION_PARTIAL ("online-softmax over one KV chunk -> (m,l,o) scratch"): keys
// [c*chunk, min((c+1)*chunk, positions[b]+1)) of KV head g, for the group's q heads.
// Scores s_j = q.k_j / sqrt(hd); m = max s; l = sum e^(s-m); o = sum e^(s-m) v_j
// (unnormalised).  Empty chunk -> (-inf, 0, 0).  Slot layout: [heads][hd + 2] with
// o in [0, hd), m at hd, l at hd + 1.
// ---------------------------------------------------------------------------------
template <bool BF16>
__device__ void partial_body(const LaunchArgs& a, const mk_task_t& d, Smem& sm, const float* q, const char* kc,
                             const char* vc, float* out, int lo, int hi) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int VEC = 16 / ES;
  const int hd = d.n, hc = (int)d.reserved[2];
  const int n = hi - lo;
  const int lpk = hd / VEC;           // lanes per key row (16 bytes each)
  const int kpw = 64 / lpk;           // keys per wavefront pass
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kl = lane / lpk, dl = lane % lpk;
  const float scale = 1.0f / sqrtf((float)hd);
  float* qs = sm.xs;                   // [hc][hd]
  float* sc = sm.xs + hc * hd;         // [hc][n] scores, then weights
  for (int e = threadIdx.x; e < hc * hd; e += kThreads) qs[e] = q[e];
  __syncthreads();
  // Scores.
  for (int j0 = wave * kpw; j0 < n; j0 += kWaves * kpw) {
    const int j = j0 + kl;
    const bool ok = j < n;
    float kf[VEC];
    if (ok) {
      const uint4 kv = *(const uint4*)(kc + ((size_t)(lo + j) * hd + dl * VEC) * ES);
      if (BF16) {
        kf[0] = bf16_lo(kv.x); kf[1] = bf16_hi(kv.x); kf[2] = bf16_lo(kv.y); kf[3] = bf16_hi(kv.y);
        kf[4 % VEC] = bf16_lo(kv.z); kf[5 % VEC] = bf16_hi(kv.z); kf[6 % VEC] = bf16_lo(kv.w);
        kf[7 % VEC] = bf16_hi(kv.w);
      } else {
        kf[0] = __uint_as_float(kv.x); kf[1] = __uint_as_float(kv.y);
        kf[2] = __uint_as_float(kv.z); kf[3] = __uint_as_float(kv.w);
      }
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) kf[e] = 0.f;
    }
    for (int h = 0; h < hc; ++h) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) s = fmaf(kf[e], qs[h * hd + dl * VEC + e], s);
      s = group_sum(s, lpk);
      if (ok && dl == 0) sc[h * n + j] = s * scale;
    }
  }
  __syncthreads();
  // Per head: max, exp, sum.  One wavefront per head.
  for (int h = wave; h < hc; h += kWaves) {
    float m = -INFINITY;
    for (int j = lane; j < n; j += 64) m = fmaxf(m, sc[h * n + j]);
    m = wave_max(m);
    float l = 0.f;
    for (int j = lane; j < n; j += 64) {
      const float e = __expf(sc[h * n + j] - m);
      sc[h * n + j] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) {
      out[h * (hd + 2) + hd] = n > 0 ? m : -INFINITY;
      out[h * (hd + 2) + hd + 1] = l;
    }
  }
  __syncthreads();
  // o = sum_j e_j v_j: lane holds VEC dims of one key row; reduce over keys.
  float acc[8][VEC];
  const int HMAX = 8;
  for (int h0 = 0; h0 < hc; h0 += HMAX) {
    const int hn = (hc - h0) < HMAX ? (hc - h0) : HMAX;
#pragma unroll
    for (int h = 0; h < HMAX; ++h)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[h][e] = 0.f;
    for (int j0 = wave * kpw; j0 < n; j0 += kWaves * kpw) {
      const int j = j0 + kl;
      if (j < n) {
        const uint4 vv = *(const uint4*)(vc + ((size_t)(lo + j) * hd + dl * VEC) * ES);
        float vf[VEC];
        if (BF16) {
          vf[0] = bf16_lo(vv.x); vf[1] = bf16_hi(vv.x); vf[2] = bf16_lo(vv.y); vf[3] = bf16_hi(vv.y);
          vf[4 % VEC] = bf16_lo(vv.z); vf[5 % VEC] = bf16_hi(vv.z); vf[6 % VEC] = bf16_lo(vv.w);
          vf[7 % VEC] = bf16_hi(vv.w);
        } else {
          vf[0] = __uint_as_float(vv.x); vf[1] = __uint_as_float(vv.y);
          vf[2] = __uint_as_float(vv.z); vf[3] = __uint_as_float(vv.w);
        }
#pragma unroll
        for (int h = 0; h < HMAX; ++h) {
          if (h < hn) {
            const float p = sc[(h0 + h) * n + j];
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
          }
        }
      }
    }
    // Reduce over the kpw key lanes of the wavefront, then across wavefronts via LDS.
    float* part = sm.red;  // [kWaves][hn][hd] must fit: 8 * 8 * hd <= kRedFloats? use xs tail
    part = sc + hc * n;
    for (int h = 0; h < hn; ++h) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float v = acc[h][e];
        for (int o = lpk; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
        if (kl == 0) part[(wave * hn + h) * hd + dl * VEC + e] = v;
      }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < hn * hd; e += kThreads) {
      const int h = e / hd, dd = e % hd;
      float s = 0.f;
      for (int w = 0; w < kWaves; ++w) s += part[(w * hn + h) * hd + dd];
      out[(h0 + h) * (hd + 2) + dd] = s;
    }
    __syncthreads();
  }
}

__device__ void task_partial(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm) {
  const int b = (int)d.reserved[0], h0 = (int)d.reserved[1], hc = (int)d.reserved[2];
  const int c = (int)d.reserved[3], base = (int)d.reserved[4];
  const int g = d.k, hd = d.n, chunk = d.kv_len, nchunks = d.m;
  const int cap = a.kv_capacity, Hkv = a.n_kv_heads, Hq = a.n_q_heads;
  const float* qrot = (const float*)resolve(a, d.in_buf[0]);
  const char* kc = resolve(a, d.in_buf[1]);
  const char* vc = resolve(a, d.in_buf[2]);
  float* part = (float*)resolve(a, d.out_buf);
  const int32_t* positions = (const int32_t*)a.rt[TAG_POSITIONS];
  if (!dep_wait(a, t, d.remaining_deps, sm)) return;
  const int pos = positions[b];
  if (pos < 0 || pos >= cap || pos >= nchunks * chunk) {
    if (threadIdx.x == 0) raise_status(a, MK_STATUS_BAD_POSITION | t);
    return;
  }
  int hi = (c + 1) * chunk;
  hi = hi < pos + 1 ? hi : pos + 1;
  int lo = c * chunk;
  lo = lo < hi ? lo : hi;
  const int es = d.config_id == MK_DTYPE_BF16 ? 2 : 4;
  const size_t head_off = (((size_t)b * Hkv + g) * cap) * hd * es;
  float* out = part + (size_t)(base + c) * hc * (hd + 2);
  const float* q = qrot + (size_t)b * Hq * hd + (size_t)h0 * hd;
  if (d.config_id == MK_DTYPE_BF16) partial_body<true>(a, d, sm, q, kc + head_off, vc + head_off, out, lo, hi);
  else partial_body<false>(a, d, sm, q, kc + head_off, vc + head_off, out, lo, hi);
}

// ---------------------------------------------------------------------------------
// ATTENTION_COMBINE ("LSE-merge of the partials -> final O"): per head,
// M = max_c m_c, w_c = e^(m_c - M), O = sum_c w_c o_c / sum_c w_c l_c.
// ---------------------------------------------------------------------------------
__device__ void task_combine(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm) {
  const int b = (int)d.reserved[0], h0 = (int)d.reserved[1], hc = (int)d.reserved[2];
  const int base = (int)d.reserved[4], nch = d.m, hd = d.n;
  const float* part = (const float*)resolve(a, d.in_buf[0]);
  float* att = (float*)resolve(a, d.out_buf);
  if (!dep_wait(a, t, d.remaining_deps, sm)) return;
  const int Hq = a.n_q_heads;
  for (int e = threadIdx.x; e < hc * hd; e += kThreads) {
    const int h = e / hd, dd = e % hd;
    float M = -INFINITY;
    for (int c = 0; c < nch; ++c) M = fmaxf(M, part[((size_t)(base + c) * hc + h) * (hd + 2) + hd]);
    float lam = 0.f, o = 0.f;
    for (int c = 0; c < nch; ++c) {
      const float* s = part + ((size_t)(base + c) * hc + h) * (hd + 2);
      const float m = s[hd];
      const float w = m == -INFINITY ? 0.f : __expf(m - M);
      lam = fmaf(w, s[hd + 1], lam);
      o = fmaf(w, s[dd], o);
    }
    att[(size_t)b * Hq * hd + (size_t)(h0 + h) * hd + dd] = o / lam;
  }
}

__device__ __forceinline__ void run_task(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm) {
  switch (d.op_id) {
    case MK_OP_GEMV: task_gemv(a, d, t, sm); break;
    case MK_OP_ATTENTION_APPEND: task_append(a, d, t, sm); break;
    case MK_OP_ATTENTION_PARTIAL: task_partial(a, d, t, sm); break;
    case MK_OP_ATTENTION_COMBINE: task_combine(a, d, t, sm); break;
    case MK_OP_MEMCPY: task_memcpy(a, d, t, sm); break;
    default: dep_wait(a, t, d.remaining_deps, sm); break;  // NOP join
  }
}

}  // namespace mk
