// Attention task bodies: ATTENTION_APPEND, ATTENTION_PARTIAL, ATTENTION_COMBINE
// ("Mega kernel initial", OpId table and lowering section: one partial per (sequence,
// KV-head group, KV chunk) producing (m, l, o), then a log-sum-exp merge -- plain
// flash-decoding).
#pragma once

#include "device_common.h"

namespace mk {

// ---------------------------------------------------------------------------------
// ATTENTION_APPEND (OpId 7 of the OpId table in "Mega kernel initial"): for sequence
// b and KV head g, rotate the group's query heads and k_g (rotate-half RoPE, angle
// pos * theta^(-2i/hd)), write rotated q to q_rot and the rotated k and v into cache
// slot positions[b], rounded to the cache dtype.  The cosine and sine of each angle
// come from a per-slot table the host fills once per graph (binary64, rounded to
// binary32); they depend on the position only, so they are loaded before the wait.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ void task_append(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm) {
  const int b = (int)d.reserved[0], h0 = (int)d.reserved[1], hc = (int)d.reserved[2];
  const int g = d.k, hd = d.n, cap = d.kv_len;
  const int Hq = a.n_q_heads, Hkv = a.n_kv_heads;
  const float* qkv = (const float*)resolve(a, d.in_buf[0]);
  float* qrot = (float*)resolve(a, d.out_buf);
  char* kc = resolve(a, d.reserved[3]);
  char* vc = resolve(a, d.reserved[4]);
  // positions is a per-step input (no producer task): read it before waiting.
  const int pos = ldg<int32_t>((const void*)a.rt[TAG_POSITIONS], b);
  const bool bad = pos < 0 || pos >= cap;
  // Rotation coefficients do not depend on producers either (a bad position reads
  // slot 0 and is reported after the wait).
  const int half = hd / 2;
  const int nrot = (hc + 1) * half;
  const size_t cs_row = (size_t)(bad ? 0 : pos) * half;
  uint64_t cs0 = 0;  // (cos, sin) as two binary32 words
  const int e0 = threadIdx.x;
  if (e0 < nrot) cs0 = ldg<uint64_t>(a.rope, cs_row + e0 % half);
  if (!dep_wait(a, t, d.remaining_deps, sm)) return;
  if (bad) {
    if (threadIdx.x == 0) raise_status(a, MK_STATUS_BAD_POSITION | t);
    return;
  }
  const size_t row = (size_t)b * (Hq + 2 * Hkv) * hd;
  const size_t slot = (((size_t)b * Hkv + g) * cap + pos) * hd;
  const bool bf16 = d.config_id == MK_DTYPE_BF16;
  // (hc q heads + 1 k head) x half rotation pairs, then hd v elements.
  for (int e = threadIdx.x; e < nrot + hd; e += kThreads) {
    if (e < nrot) {
      const int hh = e / half, i = e % half;
      const uint64_t cs = e == e0 ? cs0 : ldg<uint64_t>(a.rope, cs_row + i);
      const float c = __uint_as_float((uint32_t)cs), s = __uint_as_float((uint32_t)(cs >> 32));
      const size_t src = hh < hc ? row + (size_t)(h0 + hh) * hd : row + (size_t)(Hq + g) * hd;
      const float x0 = ld_dev<float>(qkv, src + i), x1 = ld_dev<float>(qkv, src + i + half);
      const float r0 = x0 * c - x1 * s;
      const float r1 = x1 * c + x0 * s;
      if (hh < hc) {
        const size_t dst = (size_t)b * Hq * hd + (size_t)(h0 + hh) * hd;
        st_dev<float>(qrot, dst + i, r0);
        st_dev<float>(qrot, dst + i + half, r1);
      } else if (bf16) {
        st_dev<uint16_t>(kc, slot + i, f32_to_bf16_rne(r0));
        st_dev<uint16_t>(kc, slot + i + half, f32_to_bf16_rne(r1));
      } else {
        st_dev<float>(kc, slot + i, r0);
        st_dev<float>(kc, slot + i + half, r1);
      }
    } else {
      const int i = e - nrot;
      const float v = ld_dev<float>(qkv, row + (size_t)(Hq + Hkv + g) * hd + i);
      if (bf16) st_dev<uint16_t>(vc, slot + i, f32_to_bf16_rne(v));
      else st_dev<float>(vc, slot + i, v);
    }
  }
}

// ---------------------------------------------------------------------------------
// ATTENTION_PARTIAL (OpId 8 of the same table): keys
// [c*chunk, min((c+1)*chunk, positions[b]+1)) of KV head g, for the group's q heads.
//   s_j = q.k_j / sqrt(hd); m = max s; l = sum e^(s-m); o = sum e^(s-m) v_j
// (o unnormalised; an empty chunk gives (-inf, 0, 0)).  Slot layout [heads][hd + 2]:
// o in [0, hd), m at hd, l at hd + 1.
//
// A key row is read by a group of hd*es/16 lanes (16 bytes each); the rows of the
// chunk are spread over the workgroup in rounds, processed in double-buffered
// batches of R rounds.  Rows older than the new token are static, so the first batch
// is loaded before the dependency wait; the new token's row (written by this step's
// APPEND) is read after it and folded in last.  Each lane group keeps a running
// (m, l, o) per head (the dot product is summed across the group with DPP moves);
// the states of all groups are merged with the same log-sum-exp rule in one pass
// through LDS.
// ---------------------------------------------------------------------------------

template <bool BF16>
__device__ __forceinline__ void unpack(const u32x4 v, float f[8]) {
  if (BF16) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  } else {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y); f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w); f[4] = f[5] = f[6] = f[7] = 0.f;
  }
}

// Merge the running (m, l, o) states of the workgroup's lane groups for one pass of
// query heads (log-sum-exp rule) and write the pass's output slots.  State st =
// wave * kpw + (lane / (64 / kpw)) holds o[h][0 .. VEC) at dims (lane % (64 / kpw)) VEC
// and (m[h], l[h]); every lane of a state holds the same m and l.
template <int HM, int VEC>
__device__ __forceinline__ void partial_merge(const LaunchArgs& a, Smem& sm, bool first, int hc, int hd, int kpw,
                                              const float (&m)[HM], const float (&l)[HM], const float (&o)[HM][8],
                                              float* out, size_t out0, int stride) {
  const int lane = lane_id(), wave = wave_id();
  const int lpk = 64 / kpw, kl = lane / lpk, dl = lane % lpk;
  // Merge the running states of every lane group of the workgroup in one LDS pass
  // (log-sum-exp rule): each group writes its (m, l) and its slice of o, one wave per
  // head turns the S = kWaves * kpw maxima into the head's M and per-state weights
  // w_s = e^(m_s - M) (and L = sum_s w_s l_s) with wave reductions, and each thread
  // then sums one output element over the S states.  Layout in the staging area:
  // o as [S][HM][hd], then (m, l) as [S][HM][2], then w as [HM][S].
  const int S = kWaves * kpw;
  float* po = sm.xs;
  float* pml = po + (size_t)S * HM * hd;
  float* pw = pml + (size_t)S * HM * 2;
  if (!first) __syncthreads();  // the previous pass may still read po / pml / pw
  {
    const int st = wave * kpw + kl;
#pragma unroll
    for (int h = 0; h < HM; ++h) {
      if (h < hc) {
        float* dst = po + ((size_t)st * HM + h) * hd + dl * VEC;
        *(f32x4*)dst = f32x4{o[h][0], o[h][1], o[h][2], o[h][3]};
        if (VEC == 8) *(f32x4*)(dst + 4) = f32x4{o[h][4], o[h][5], o[h][6], o[h][7]};
        if (dl == 0) {
          pml[(st * HM + h) * 2] = m[h];
          pml[(st * HM + h) * 2 + 1] = l[h];
        }
      }
    }
  }
  __syncthreads();
  if (wave < hc) {
    const int h = wave;
    float mx = -INFINITY;
    for (int st = lane; st < S; st += 64) mx = fmaxf(mx, pml[(st * HM + h) * 2]);
    mx = fmaxf(mx, lane_xor<32>(mx));
    mx = fmaxf(mx, lane_xor<16>(mx));
    mx = fmaxf(mx, lane_xor<8>(mx));
    mx = fmaxf(mx, lane_xor<4>(mx));
    mx = fmaxf(mx, lane_xor<2>(mx));
    mx = fmaxf(mx, lane_xor<1>(mx));
    float lsum = 0.f;
    for (int st = lane; st < S; st += 64) {
      const float ms = pml[(st * HM + h) * 2];
      const float w = ms == -INFINITY ? 0.f : __expf(ms - mx);  // every state empty: M = -inf, all 0
      pw[h * S + st] = w;
      lsum = fmaf(w, pml[(st * HM + h) * 2 + 1], lsum);
    }
    lsum = wave_sum(lsum);
    if (lane == 0) {
      st_dev<float>(out, out0 + h * stride + hd, mx);
      st_dev<float>(out, out0 + h * stride + hd + 1, lsum);
    }
  }
  __syncthreads();
  trace_mark(a, sm, 1);
  for (int e = threadIdx.x; e < hc * hd; e += kThreads) {
    const int h = e / hd, dd = e % hd;
    const float* wh = pw + h * S;
    const float* oh = po + (size_t)h * hd + dd;
    // Blocks of 8 states: the LDS reads of a block are issued together.
    float acc = 0.f;
    int st = 0;
    for (; st + 8 <= S; st += 8) {
      float ov[8], wv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        ov[u] = oh[(size_t)(st + u) * HM * hd];
        wv[u] = wh[st + u];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc = fmaf(ov[u], wv[u], acc);
    }
    for (; st < S; ++st) acc = fmaf(oh[(size_t)st * HM * hd], wh[st], acc);
    st_dev<float>(out, out0 + h * stride + dd, acc);
  }
}

// The same log-sum-exp merge for the matrix-core pass, whose states come as kpw row
// groups per wave that share the wave's maximum: lane l of wave w holds o[h][0 .. 8)
// of row group l / lpk at dims 8 (l % lpk) (lpk = 64 / kpw lanes per row group), and
// every lane holds the wave's (m[h], l[h]).  Each row group writes its o and lane 0
// the wave's (m, l); after one barrier each thread finishes one output element: the
// head's maximum M over the kWaves waves, one weight e^(m_w - M) per wave, applied
// to the sum of that wave's row groups.
template <int HM>
__device__ __forceinline__ void partial_merge_rg(Smem& sm, bool first, int hc, int hd, int kpw, const float (&m)[HM],
                                                 const float (&l)[HM], const float (&o)[HM][8], float* out,
                                                 size_t out0, int stride) {
  const int lane = lane_id(), wave = wave_id();
  const int lpk = 64 / kpw, kl = lane / lpk, dl = lane % lpk;
  // Staging: o as [kWaves * kpw][HM][hd], then (m, l) as [kWaves][HM][2].
  float* po = sm.xs;
  float* pml = po + (size_t)kWaves * kpw * HM * hd;
  if (!first) __syncthreads();  // the previous pass may still read po / pml
#pragma unroll
  for (int h = 0; h < HM; ++h) {
    if (h < hc) {
      float* dst = po + ((size_t)(wave * kpw + kl) * HM + h) * hd + dl * 8;
      *(f32x4*)dst = f32x4{o[h][0], o[h][1], o[h][2], o[h][3]};
      *(f32x4*)(dst + 4) = f32x4{o[h][4], o[h][5], o[h][6], o[h][7]};
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < HM; ++h) {
      pml[(wave * HM + h) * 2] = m[h];
      pml[(wave * HM + h) * 2 + 1] = l[h];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < hc * hd; e += kThreads) {
    const int h = e / hd, dd = e % hd;
    float ms[kWaves];
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      ms[w] = pml[(w * HM + h) * 2];
      mx = fmaxf(mx, ms[w]);
    }
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = ms[w] == -INFINITY ? 0.f : __expf(ms[w] - mx);  // every state empty: all 0
      float ow = 0.f;
      for (int k = 0; k < kpw; ++k) ow += po[((size_t)(w * kpw + k) * HM + h) * hd + dd];
      acc = fmaf(wt, ow, acc);
      lsum = fmaf(wt, pml[(w * HM + h) * 2 + 1], lsum);
    }
    st_dev<float>(out, out0 + h * stride + dd, acc);
    if (dd == 0) {
      st_dev<float>(out, out0 + h * stride + hd, mx);
      st_dev<float>(out, out0 + h * stride + hd + 1, lsum);
    }
  }
}

// One pass over the chunk for query heads [hg, hg + HM) of the group; the first pass
// (hg == 0) prefetches before waiting on the producers.
template <bool BF16, int HM, int LPK, int R, bool BATCHED>
__device__ __forceinline__ bool partial_pass(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm, int hg) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int VEC = 16 / ES;
  const int b = (int)d.reserved[0], h0 = (int)d.reserved[1], hc_all = (int)d.reserved[2];
  const int c = (int)d.reserved[3], base = (int)d.reserved[4];
  const int g = d.k, hd = d.n, chunk = d.kv_len, nchunks = d.m;
  const int cap = a.kv_capacity, Hkv = a.n_kv_heads, Hq = a.n_q_heads;
  const int hc = (hc_all - hg) < HM ? (hc_all - hg) : HM;
  const float* qrot = (const float*)resolve(a, d.in_buf[0]);
  const int rowq = hd * ES / 16;  // 16-byte pieces per cache row
  const size_t head_off = (((size_t)b * Hkv + g) * cap) * rowq;
  const char* kc = resolve(a, d.in_buf[1]);
  const char* vc = resolve(a, d.in_buf[2]);
  const int stride = hd + 2;
  float* out = (float*)resolve(a, d.out_buf);
  const size_t out0 = ((size_t)(base + c) * hc_all + hg) * stride;
  const int pos = ldg<int32_t>((const void*)a.rt[TAG_POSITIONS], b);
  const bool bad = pos < 0 || pos >= cap || pos >= nchunks * chunk;
  int hi = (c + 1) * chunk;
  hi = hi < pos + 1 ? hi : pos + 1;
  int lo = c * chunk;
  lo = lo < hi ? lo : hi;
  const int n = bad ? 0 : hi - lo;
  const int jnew = pos - lo;  // row of the new token (if inside this chunk)

  const int lane = lane_id(), wave = wave_id();
  const int lpk = LPK > 0 ? LPK : rowq, kpw = 64 / lpk, kpr = kWaves * kpw;
  const int kl = lane / lpk, dl = lane % lpk;
  const int jbase = wave * kpw + kl;  // this lane group's row in round 0
  const int rounds = (n + kpr - 1) / kpr;
  const bool first = hg == 0;
  // K and V of this (sequence, KV head) are read through raw buffer resources over
  // the head's cache rows.  A row past the chunk's end gets an out-of-range offset:
  // the load returns zeros without touching memory and the row is masked when
  // folded, so every load below is unconditional within a wave-uniform branch.
  const uint32_t head_bytes = (uint32_t)cap * (uint32_t)rowq * 16u;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(kc + head_off * 16), (short)0, (int)head_bytes, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(vc + head_off * 16), (short)0, (int)head_bytes, kRawBufferWord3);
  auto row_off = [&](int j) -> uint32_t {
    return j < n ? ((uint32_t)(lo + j) * (uint32_t)rowq + (uint32_t)dl) * 16u : 0xFFFFFFF0u;
  };
  auto ldk = [&](int j) { return __builtin_amdgcn_raw_buffer_load_b128(krs, row_off(j), 0, 0); };
  auto ldv = [&](int j) { return __builtin_amdgcn_raw_buffer_load_b128(vrs, row_off(j), 0, 0); };

  // Rows of earlier steps never change during the step: the first R rounds are
  // loaded before the dependency wait.  The new token's row is loaded too but masked
  // (it is stale until this step's APPEND has run) and folded in after the loop.
  u32x4 kr[R], vr[R];
  if (rounds > 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      kr[r] = ldk(jbase + r * kpr);
      vr[r] = ldv(jbase + r * kpr);
    }
  }
  if (first) {
    if (!dep_wait(a, t, d.remaining_deps, sm)) return false;
    if (bad) {
      if (threadIdx.x == 0) raise_status(a, MK_STATUS_BAD_POSITION | t);
      return false;
    }
  }
  const float scale = 1.0f / sqrtf((float)hd);
  float q[HM][8];
#pragma unroll
  for (int h = 0; h < HM; ++h) {
    if (h < hc) {
      const size_t q4 = ((size_t)b * Hq * hd + (size_t)(h0 + hg + h) * hd + dl * VEC) / 4;
      const f32x4 q0 = ld_dev_f4(qrot, q4);
      q[h][0] = q0.x * scale; q[h][1] = q0.y * scale; q[h][2] = q0.z * scale; q[h][3] = q0.w * scale;
      if (VEC == 8) {
        const f32x4 q1 = ld_dev_f4(qrot, q4 + 1);
        q[h][4] = q1.x * scale; q[h][5] = q1.y * scale; q[h][6] = q1.z * scale; q[h][7] = q1.w * scale;
      } else {
        q[h][4] = q[h][5] = q[h][6] = q[h][7] = 0.f;
      }
    }
  }
  // The new token's row, written by this step's APPEND: wave 0 issues its
  // device-scope loads together with the query's, and its lane group 0 folds the row
  // in after the loop.
  const bool has_new = jnew >= 0 && jnew < n;
  u32x4 knew = {0u, 0u, 0u, 0u}, vnew = {0u, 0u, 0u, 0u};
  if (has_new && wave == 0) {
    const size_t rn = head_off + (size_t)pos * rowq + dl;
    knew = ld_dev_u4(kc, rn);
    vnew = ld_dev_u4(vc, rn);
  }
  float m[HM], l[HM], o[HM][8];
#pragma unroll
  for (int h = 0; h < HM; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  }
  // Score one row against the heads and fold it into the running (m, l, o) of the
  // lanes where `ok` holds (every lane of a group gets the group's full dot product).
  auto fold = [&](const u32x4 kv, const u32x4 vv, bool ok) {
    float kf[8], vf[8];
    unpack<BF16>(kv, kf);
    unpack<BF16>(vv, vf);
#pragma unroll
    for (int h = 0; h < HM; ++h) {
      if (h < hc) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) s = fmaf(kf[e], q[h][e], s);
        if constexpr (LPK > 0) s = group_allsum<LPK>(s);
        else s = group_allsum(s, lpk);
        // Branch-free online-softmax step; a masked lane keeps (m, l, o) unchanged.
        const float mn = ok ? fmaxf(m[h], s) : m[h];
        const float al = (m[h] == mn) ? 1.f : __expf(m[h] - mn);  // m = -inf -> 0
        const float p = ok ? __expf(s - mn) : 0.f;
        l[h] = fmaf(l[h], al, p);
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[h][e] = fmaf(o[h][e], al, p * vf[e]);
        m[h] = mn;
      }
    }
  };
  // The same for a batch of R rows at once (BATCHED): all R scores first, then one
  // running-max update and one rescale of (l, o) per head, then the R weighted rows
  // (one exp per row instead of two, one rescale per batch instead of one per row).
  // Masked rows score -inf and weigh 0.  Used by the long-context kernel, whose chunks
  // run many batches; the batch-1 kernel keeps the per-row step, whose smaller code
  // leaves the register allocation of the GEMV loops in the same kernel alone.
  auto fold_batch = [&](const u32x4 (&kb)[R], const u32x4 (&vb)[R], const bool (&okb)[R]) {
    float sc[R][HM];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float kf[8];
      unpack<BF16>(kb[r], kf);
#pragma unroll
      for (int h = 0; h < HM; ++h) {
        if (h < hc) {
          float sv = 0.f;
#pragma unroll
          for (int e = 0; e < VEC; ++e) sv = fmaf(kf[e], q[h][e], sv);
          if constexpr (LPK > 0) sv = group_allsum<LPK>(sv);
          else sv = group_allsum(sv, lpk);
          sc[r][h] = okb[r] ? sv : -INFINITY;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < HM; ++h) {
      if (h < hc) {
        float mb = m[h];
#pragma unroll
        for (int r = 0; r < R; ++r) mb = fmaxf(mb, sc[r][h]);
        const float al = (m[h] == mb) ? 1.f : __expf(m[h] - mb);  // m = -inf -> 0
        l[h] *= al;
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[h][e] *= al;
        m[h] = mb;
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float vf[8];
      unpack<BF16>(vb[r], vf);
#pragma unroll
      for (int h = 0; h < HM; ++h) {
        if (h < hc) {
          const float p = (sc[r][h] == -INFINITY) ? 0.f : __expf(sc[r][h] - m[h]);
          l[h] += p;
#pragma unroll
          for (int e = 0; e < VEC; ++e) o[h][e] = fmaf(p, vf[e], o[h][e]);
        }
      }
    }
  };
  // Batches of R rounds, double-buffered: the next batch's loads are issued before
  // the current batch is folded.  All loads are unconditional (rows past the chunk,
  // including the last batch's look-ahead, are out of range and read nothing), so the
  // compiler keeps 2R rounds in flight with counted waits.
  const int nbatch = (rounds + R - 1) / R;
  for (int bt = 0; bt < nbatch; ++bt) {
    u32x4 kn[R], vn[R];
    const int jn = jbase + (bt + 1) * R * kpr;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      kn[r] = ldk(jn + r * kpr);
      vn[r] = ldv(jn + r * kpr);
    }
    if constexpr (BATCHED) {
      bool okb[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int j = jbase + (bt * R + r) * kpr;
        okb[r] = j < n && j != jnew;
      }
      fold_batch(kr, vr, okb);
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int j = jbase + (bt * R + r) * kpr;
        fold(kr[r], vr[r], j < n && j != jnew);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      kr[r] = kn[r];
      vr[r] = vn[r];
    }
  }
  if (has_new && wave == 0) fold(knew, vnew, kl == 0);
  trace_mark(a, sm, 0);
  partial_merge<HM, VEC>(a, sm, first, hc, hd, kpw, m, l, o, out, out0, stride);
  return true;
}

// The same ATTENTION_PARTIAL pass with the scores on the matrix cores, for a bf16
// cache with head_dim HD = 64 or 128 (the 16-lane fold above spends most of its
// time in per-row softmax work that every lane of a row group repeats).
//  * The chunk's keys go in blocks of 16, dealt to the waves round robin (block
//    wave + 8 i).  Scores S[key][head] = K[key] . q_head / sqrt(HD) come from
//    v_mfma_f32_16x16x32_bf16 with A = 16 key rows x 32 dims (lane l: key l % 16,
//    dims 8 (l / 16) .. +8 of each 32) and B = the pass's query heads as columns
//    0..3 (columns 4..15 zero); the query is split into bf16 hi and lo parts (q =
//    hi + lo to about 16 bits) and both products accumulate into the same scores.
//  * In the result a lane holds 4 keys of one head (column), so the block maximum,
//    e^(s - m) and the running sum are computed once per (key, head): the maximum
//    over the block and the rescale factor are shared across the wave with lane
//    swaps and lane reads.
//  * p = e^(s - m) goes through a 256-byte slice of LDS private to the wave to the
//    lanes that hold the matching V rows (row groups of HD / 8 lanes, 16 bytes each,
//    as in the pass above), which accumulate o[head][dims] += p v.  Those row
//    groups' o, with the wave's (m, l), are the states partial_merge_rg combines.
//  * The query rows are staged once into LDS after the wait (two waves' global-to-LDS
//    loads), and every wave builds its B operand from there.
//  * A ring of NS blocks of K and V is held in registers, loaded before the
//    dependency wait and refilled in place after each block is folded (no refill
//    past the wave's last block).  The new token's row is masked in the ring (it is
//    stale until APPEND has run); wave 0 reads it with device-scope loads after the
//    wait and folds it first, as a block holding only that row.
template <int HD, int NS>
__device__ __forceinline__ bool partial_pass_mfma(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm,
                                                  int hg) {
  constexpr int HM = 4, VEC = 8;
  constexpr int LPK = HD / 8;       // lanes per V row (16 bytes each)
  constexpr int KPV = 64 / LPK;     // V rows per wave load
  constexpr int KS = HD / 32;       // 32-dim steps of a key row
  constexpr int VJ = 16 / KPV;      // V loads per block of 16 keys
  constexpr int rowq = HD / 8;      // 16-byte pieces per cache row
  const int b = (int)d.reserved[0], h0 = (int)d.reserved[1], hc_all = (int)d.reserved[2];
  const int c = (int)d.reserved[3], base = (int)d.reserved[4];
  const int g = d.k, chunk = d.kv_len, nchunks = d.m;
  const int cap = a.kv_capacity, Hkv = a.n_kv_heads, Hq = a.n_q_heads;
  const int hc = (hc_all - hg) < HM ? (hc_all - hg) : HM;
  const float* qrot = (const float*)resolve(a, d.in_buf[0]);
  const size_t head_off = (((size_t)b * Hkv + g) * cap) * rowq;
  const char* kc = resolve(a, d.in_buf[1]);
  const char* vc = resolve(a, d.in_buf[2]);
  const int stride = HD + 2;
  float* out = (float*)resolve(a, d.out_buf);
  const size_t out0 = ((size_t)(base + c) * hc_all + hg) * stride;
  const int pos = ldg<int32_t>((const void*)a.rt[TAG_POSITIONS], b);
  const bool bad = pos < 0 || pos >= cap || pos >= nchunks * chunk;
  int hi = (c + 1) * chunk;
  hi = hi < pos + 1 ? hi : pos + 1;
  int lo = c * chunk;
  lo = lo < hi ? lo : hi;
  const int n = bad ? 0 : hi - lo;
  const int jnew = pos - lo;  // the new token's key (if inside this chunk)
  const bool first = hg == 0;

  int lane = lane_id();
  asm volatile("" : "+v"(lane));  // per-lane offsets are recomputed per task, not hoisted and spilled
  const int wave = wave_id();
  const int qc = lane & 15, g4 = lane >> 4;       // score layout: head column, key group
  const int kv = lane / LPK, dl = lane % LPK;     // V layout: row in a load, dims dl * 8
  const int nblk = (n + 15) >> 4;
  const int nbw = nblk > wave ? (nblk - wave + kWaves - 1) / kWaves : 0;  // blocks of this wave
  const uint32_t head_bytes = (uint32_t)cap * (uint32_t)rowq * 16u;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(kc + head_off * 16), (short)0, (int)head_bytes, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(vc + head_off * 16), (short)0, (int)head_bytes, kRawBufferWord3);
  // Keys past the chunk get an out-of-range offset: the load reads nothing, returns 0.
  auto koff = [&](int i, int s) -> uint32_t {
    const int key = 16 * (wave + kWaves * i) + qc;
    return key < n ? ((uint32_t)(lo + key) * rowq + 4u * s + (uint32_t)g4) * 16u : 0xFFFFFFF0u;
  };
  auto voff = [&](int i, int j) -> uint32_t {
    const int key = 16 * (wave + kWaves * i) + kv + KPV * j;
    return key < n ? ((uint32_t)(lo + key) * rowq + (uint32_t)dl) * 16u : 0xFFFFFFF0u;
  };
  u32x4 kr[NS][KS], vr[NS][VJ];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int e = 0; e < KS; ++e) kr[s][e] = __builtin_amdgcn_raw_buffer_load_b128(krs, koff(s, e), 0, 0);
#pragma unroll
    for (int j = 0; j < VJ; ++j) vr[s][j] = __builtin_amdgcn_raw_buffer_load_b128(vrs, voff(s, j), 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (first) {
    if (!dep_wait(a, t, d.remaining_deps, sm)) return false;
    if (bad) {
      if (threadIdx.x == 0) raise_status(a, MK_STATUS_BAD_POSITION | t);
      return false;
    }
  }
  // The new token's row (written by this step's APPEND), wave 0 only: K in the
  // score layout (lanes of key 0), V in the row layout (lanes of row 0).
  const bool has_new = jnew >= 0 && jnew < n;
  u32x4 knew[KS], vnew[VJ];
#pragma unroll
  for (int e = 0; e < KS; ++e) knew[e] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < VJ; ++j) vnew[j] = u32x4{0u, 0u, 0u, 0u};
  if (has_new && wave == 0) {
    const size_t rn = head_off + (size_t)pos * rowq;
    if (qc == 0) {
#pragma unroll
      for (int e = 0; e < KS; ++e) knew[e] = ld_dev_u4(kc, rn + 4 * e + g4);
    }
    if (kv == 0) vnew[0] = ld_dev_u4(vc, rn + dl);
  }
  // The pass's rotated query rows (hc x HD fp32, contiguous) are staged once into LDS
  // by waves 1 and 2 with device-scope global-to-LDS loads (every wave needs all of
  // them; eight waves loading the same bytes queue behind one another).
  float* qs = sm.red + 512;  // [hc][HD]; the p slices use sm.red[0 .. 512)
  if (wave == 1 || wave == 2) {
    const int p = (wave - 1) * 64 + lane;  // 16-byte piece
    if (p < hc * HD / 4)
      __builtin_amdgcn_global_load_lds(
          (const MK_GLOBAL void*)((const MK_GLOBAL f32x4*)qrot + ((size_t)b * Hq + h0 + hg) * (HD / 4) + p),
          (__attribute__((address_space(3))) void*)(qs + (wave - 1) * 256), 16, 0, kCachePolicySC1);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the copies have landed
  }
  __syncthreads();
  // B operand: column qc = head qc of the pass (zero past hc and for columns >= HM),
  // dims 32 e + 8 g4 .. +8, scaled by 1/sqrt(HD) and split into bf16 hi and lo.
  const float scale = 1.0f / sqrtf((float)HD);
  bf16x8 qh[KS], ql[KS];
#pragma unroll
  for (int e = 0; e < KS; ++e) {
    float qv[8];
    if (qc < hc) {
      const f32x4* qp = (const f32x4*)(qs + qc * HD + 32 * e + 8 * g4);
      const f32x4 q0 = qp[0], q1 = qp[1];
      qv[0] = q0.x; qv[1] = q0.y; qv[2] = q0.z; qv[3] = q0.w; qv[4] = q1.x; qv[5] = q1.y; qv[6] = q1.z; qv[7] = q1.w;
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) qv[u] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float v = qv[u] * scale;
      const __bf16 h = (__bf16)v;
      qh[e][u] = h;
      ql[e][u] = (__bf16)(v - (float)h);
    }
  }
  float m = -INFINITY, l = 0.f;  // score layout: head qc; l over this lane's keys
  float o[HM][8];
#pragma unroll
  for (int h = 0; h < HM; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  float* pw = sm.red + wave * 64;  // [16 keys][HM] p of the current block
  // Fold one block: keys key0 + 0..15; `only` >= 0 keeps just that key (the new
  // row), else keys < n other than the new token's.
  auto block = [&](const u32x4 (&kb)[KS], const u32x4 (&vb)[VJ], int key0, int only) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < KS; ++e) {
      const bf16x8 ka = __builtin_bit_cast(bf16x8, kb[e]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qh[e], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, ql[e], acc, 0, 0, 0);
    }
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + 4 * g4 + r;
      const bool ok = only >= 0 ? key == only : (key < n && key != jnew);
      sc[r] = ok ? acc[r] : -INFINITY;
    }
    float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    bm = fmaxf(bm, lane_xor<16>(bm));
    bm = fmaxf(bm, lane_xor<32>(bm));
    const float mn = fmaxf(m, bm);
    const float al = (m == mn) ? 1.f : __expf(m - mn);  // m = -inf -> 0
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = sc[r] == -INFINITY ? 0.f : __expf(sc[r] - mn);
    l = fmaf(l, al, (p[0] + p[1]) + (p[2] + p[3]));
    m = mn;
    if (qc < HM) {
#pragma unroll
      for (int r = 0; r < 4; ++r) pw[(4 * g4 + r) * HM + qc] = p[r];
    }
    float alh[HM];
    bool rescale = false;
#pragma unroll
    for (int h = 0; h < HM; ++h) {
      alh[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), h));
      rescale |= alh[h] != 1.f;
    }
    // The p slice is written and read by this wave only: LDS operations of a wave
    // complete in order, the wait keeps the compiler from reordering them.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (rescale) {
#pragma unroll
      for (int h = 0; h < HM; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] *= alh[h];
    }
#pragma unroll
    for (int j = 0; j < VJ; ++j) {
      float vf[8];
      unpack<true>(vb[j], vf);
      const f32x4 pj = *(const f32x4*)(pw + (kv + KPV * j) * HM);
      const float ph[HM] = {pj.x, pj.y, pj.z, pj.w};
#pragma unroll
      for (int h = 0; h < HM; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = fmaf(ph[h], vf[e], o[h][e]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  // The new row first: its registers are then free during the streaming loop (its
  // loads were issued with the query's, which every block waits for anyway).
  if (has_new && wave == 0) block(knew, vnew, jnew, jnew);
  for (int i0 = 0; i0 < nbw; i0 += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int i = i0 + s;
      if (i < nbw) block(kr[s], vr[s], 16 * (wave + kWaves * i), -1);
      __builtin_amdgcn_sched_barrier(0);
      if (i + NS < nbw) {
#pragma unroll
        for (int e = 0; e < KS; ++e) kr[s][e] = __builtin_amdgcn_raw_buffer_load_b128(krs, koff(i + NS, e), 0, 0);
#pragma unroll
        for (int j = 0; j < VJ; ++j) vr[s][j] = __builtin_amdgcn_raw_buffer_load_b128(vrs, voff(i + NS, j), 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  trace_mark(a, sm, 0);
  // The merge's states: the wave's V row groups, which share its m; the wave's l is
  // summed over the score layout's key groups.
  float lt = l + lane_xor<16>(l);
  lt += lane_xor<32>(lt);
  float mh[HM], lh[HM];
#pragma unroll
  for (int h = 0; h < HM; ++h) {
    mh[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), h));
    lh[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lt), h));
  }
  partial_merge_rg<HM>(sm, first, hc, HD, KPV, mh, lh, o, out, out0, stride);
  return true;
}

template <int HD, int NS>
__device__ __forceinline__ void partial_heads_mfma(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm) {
  const int hc = (int)d.reserved[2];
  for (int hg = 0; hg < hc; hg += 4)
    if (!partial_pass_mfma<HD, NS>(a, d, t, sm, hg)) return;
}

template <bool KVBF16, int LPK, int R, bool BATCHED>
__device__ __forceinline__ void partial_heads(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm) {
  const int hc = (int)d.reserved[2];
  for (int hg = 0; hg < hc; hg += 4)
    if (!partial_pass<KVBF16, 4, LPK, R, BATCHED>(a, d, t, sm, hg)) return;
}

// Lanes per cache row (head_dim * element size / 16) as a compile-time constant for
// the common shapes (head_dim 64 and 128), else a run-time value.
// NS > 0: the matrix-core pass with a ring of NS blocks of 16 keys per wave (the
// kernels pass 2 for batches above 1; 1 for batch 1, whose chunks give each wave
// about one block), for a bf16 cache with head_dim 64 or 128; otherwise, and for
// other shapes, the 16-lane fold.
template <bool KVBF16, bool BATCHED, int NS>
__device__ __forceinline__ void task_partial_kv(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm) {
  if constexpr (KVBF16 && NS > 0) {
    if (d.n == 128) return partial_heads_mfma<128, NS>(a, d, t, sm);
    if (d.n == 64) return partial_heads_mfma<64, NS>(a, d, t, sm);
  }
  // R rounds per batch: 2 for chunks of at most two rounds, else 4.
  const int lpk = d.n * (KVBF16 ? 2 : 4) / 16;
  const bool short_chunk = d.kv_len <= 2 * kWaves * (64 / lpk);
  if (lpk == 8) {
    if (short_chunk) partial_heads<KVBF16, 8, 2, BATCHED>(a, d, t, sm);
    else partial_heads<KVBF16, 8, 4, BATCHED>(a, d, t, sm);
  } else if (lpk == 16) {
    if (short_chunk) partial_heads<KVBF16, 16, 2, BATCHED>(a, d, t, sm);
    else partial_heads<KVBF16, 16, 4, BATCHED>(a, d, t, sm);
  } else {
    partial_heads<KVBF16, 0, 4, BATCHED>(a, d, t, sm);
  }
}

// ---------------------------------------------------------------------------------
// ATTENTION_COMBINE (OpId 9 of the same table): per head,
// M = max_c m_c, w_c = e^(m_c - M), O = sum_c w_c o_c / sum_c w_c l_c.
// One output element per thread.  The thread loads its o values and its head's
// (m, l) for a block of chunks at once (one memory round trip per block of 16
// chunks) and folds each block into a running (M, lam, O) with the same log-sum-exp
// rule.  No LDS is used.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ void task_combine(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm) {
  const int b = (int)d.reserved[0], h0 = (int)d.reserved[1], hc = (int)d.reserved[2];
  const int base = (int)d.reserved[4], nch = d.m, hd = d.n;
  const float* part = (const float*)resolve(a, d.in_buf[0]);
  float* att = (float*)resolve(a, d.out_buf);
  if (!dep_wait(a, t, d.remaining_deps, sm)) return;
  const int Hq = a.n_q_heads, stride = hd + 2;
  constexpr int CB = 16;
  for (int e = threadIdx.x; e < hc * hd; e += kThreads) {
    const int h = e / hd, dd = e % hd;
    float M = -INFINITY, lam = 0.f, O = 0.f;
    for (int c0 = 0; c0 < nch; c0 += CB) {
      float mv[CB], lv[CB], ov[CB];
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        const int c = c0 + u < nch ? c0 + u : nch - 1;  // past the last chunk: masked below
        const size_t s0 = ((size_t)(base + c) * hc + h) * stride;
        ov[u] = ld_dev<float>(part, s0 + dd);
        mv[u] = ld_dev<float>(part, s0 + hd);
        lv[u] = ld_dev<float>(part, s0 + hd + 1);
      }
      float Mb = M;
#pragma unroll
      for (int u = 0; u < CB; ++u)
        if (c0 + u < nch) Mb = fmaxf(Mb, mv[u]);
      const float sc = (M == Mb) ? 1.f : __expf(M - Mb);  // M = -inf -> 0
      lam *= sc;
      O *= sc;
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        if (c0 + u < nch) {
          const float w = mv[u] == -INFINITY ? 0.f : __expf(mv[u] - Mb);
          lam = fmaf(w, lv[u], lam);
          O = fmaf(w, ov[u], O);
        }
      }
      M = Mb;
    }
    st_dev<float>(att, (size_t)b * Hq * hd + (size_t)(h0 + h) * hd + dd, O / lam);
  }
}

}  // namespace mk
