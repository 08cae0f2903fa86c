// GEMV task body on the matrix cores for a small batch (B <= 8 rows), descriptor
// config_id MK_GEMV_BF16_MFMA.  Same operation as the streaming GEMV ("Mega kernel
// initial", lowering section: one task per output-column tile; descriptor section:
// flags SILU_MUL, ADD_RESIDUAL, RMS_NORM_INPUT):
//   y[b, c] = r_b * sum_k (x[b, k] gamma_k) W[c, k]   (+ res[b, c]; SiLU pairs)
//
// Why the matrix cores at B = 8: each 16 weight bytes (8 bf16) meet 8 batch rows, 64
// fp32 FMAs; streaming 8 TB/s of weights that way needs about 4 x 10^15 FMA/s...
// per CU about 125 G FMA/s against the 154 G FMA/s a CU's SIMDs issue without packed
// fp32 math, before any conversion or LDS traffic.  One v_mfma_f32_16x16x32_bf16 does
// the 16 x 32 x 16 block in one instruction.
//
// Operand layout (D[16 x 16] += A[16 x 32] B[32 x 16]):
//  * A = 16 weight rows x 32 k: lane l holds row l % 16, k = 8 (l / 16) .. +8, one
//    16-byte load: from the row-major weights, 16 rows x 64 bytes per wave load; from
//    the 16-row tile layout (mk_pack_matrix, MK_LOWER_PACKED_WEIGHTS), one contiguous
//    kilobyte, which streams about a fifth faster from HBM;
//  * B = 32 k x 16 columns: columns 0..7 hold the bf16 "hi" parts of the 8 batch rows'
//    input, columns 8..15 their "lo" parts (u = x gamma = hi + lo, hi = u with the low
//    16 bits cleared, lo = the same of the exact remainder u - hi: the input keeps
//    about 16 significant bits), so ONE product per block and k-step gives W hi and W lo
//    side by side; lane l builds column l % 16 for k = 8 (l / 16) .. +8.  Lanes l and
//    l ^ 8 (hi and lo of one batch row) each load and split 4 of the 8 input values
//    and swap the halves the other needs with one DPP move per bf16 pair -- this
//    operand build is the tile's VALU cost per k-step (about 40 instructions);
//  * D: lane l holds column l % 16 of rows 4 (l / 16) .. +4;  y[b, row] sums columns
//    b and b + 8.
//
// Work split, with no workgroup barrier in the streaming loop: the k-steps of 32 are
// dealt to the 8 waves round robin, and every wave runs all the tile's 16-row blocks
// (in groups of G, SiLU gate/up blocks interleaved so a pair stays in one group) over
// its own steps, with a ring of D k-steps of weight, input and gamma loads in flight
// (the weight ring of the first group is issued before the dependency wait).  The input is
// a whole activation buffer every producer has finished, so after the wait it is read
// with plain, L2-cached loads following one agent-scope acquire: the 32 CUs of an XCD
// share it through their L2.  Per group, the 8 waves' partial products meet once in
// LDS, and the epilogue (r_b, residual, SiLU * up) writes y.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "task_gemv_mfma.h"

namespace mk {


// Byte offset of lane `lane`'s 16 weight bytes of block gb at the wave's k-step s, which
// covers k = 32 (w + 8 s) .. +32 (kPastEnd past the last step: reads nothing).  Either
// weight layout gives the block's base (its first row times 2K bytes: a block of 16 rows
// is 32K contiguous bytes in both) + a per-lane term + s times a per-step stride:
//  * row-major [N, K]: lane l reads row l % 16 at k = 32 (w + 8 s) + 8 (l / 16):
//    lane term 2K (l % 16) + 16 (l / 16) + 64 w, stride 512 bytes;
//  * tile layout (mk_pack_matrix): k-step j of a block is one 1 KB tile at 1024 j, with
//    lane l's 16 bytes at 16 l: lane term 16 l + 1024 w, stride 8192 bytes.  A wave's
//    load is then one contiguous kilobyte instead of 16 half cache lines.
__device__ __forceinline__ uint32_t mfma_small_woff(const MfmaGeom& g, int gb, uint32_t lterm, uint32_t sstride,
                                                    int s, int nst) {
  return s < nst ? (uint32_t)mfma_block_row(g, gb) * g.K * 2u + lterm + (uint32_t)s * sstride : kPastEnd;
}

template <int G, int D>
__device__ __forceinline__ bool mfma_small_group(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm,
                                                 const MfmaGeom& g, int gb0, bool first, const char* aux, float* y,
                                                 __amdgpu_buffer_rsrc_t wrs, __amdgpu_buffer_rsrc_t xrs,
                                                 __amdgpu_buffer_rsrc_t grs, bool need_ss) {
  int lane = lane_id();
  asm volatile("" : "+v"(lane));  // recomputed per task, not hoisted and spilled
  const int w = wave_id();
  const int B = d.m, N = d.n;
  const bool norm = d.flags & MK_FLAG_RMS_NORM_INPUT;
  const bool resid = d.flags & MK_FLAG_ADD_RESIDUAL;
  // Wave w takes the k-steps w, w + 8, w + 16, ... (32 k each): at any time the 8 waves
  // of a workgroup read adjacent pieces of the same weight rows (row-major: 8 x 64
  // bytes per row; tile layout: 8 adjacent kilobyte tiles) instead of 8 far-apart places.
  const int nst = (int)g.K / (32 * kWaves);
  const int k0 = 32 * w;
  const int colj = lane & 15, kq = lane >> 4, bb = colj & 7;
  const uint32_t lterm = a.wpacked ? 16u * (uint32_t)lane + 1024u * (uint32_t)w
                                   : 2u * g.K * (uint32_t)colj + 16u * (uint32_t)kq + 64u * (uint32_t)w;
  const uint32_t sstride = a.wpacked ? 8192u : 512u;
  const bool lo_lane = colj >= 8;
  // Input: this lane's 4 of the 8 values of batch row bb at k = k0 + 256 s + 8 kq (+4 on
  // the lo lanes), one 16-byte load, and the 4 matching gamma values (8 bytes); rows
  // past the batch read nothing (zeros).
  const uint32_t xbase = (uint32_t)bb * g.K * 4u + (uint32_t)(k0 + 8 * kq + (lo_lane ? 4 : 0)) * 4u;
  auto xoff = [&](int s) -> uint32_t { return (s < nst && bb < B) ? xbase + (uint32_t)s * 1024u : kPastEnd; };
  const uint32_t gbase = (uint32_t)(k0 + 8 * kq + (lo_lane ? 4 : 0)) * 2u;
  auto goff = [&](int s) -> uint32_t { return s < nst ? gbase + (uint32_t)s * 512u : kPastEnd; };
  // Without the norm the gamma loads return zeros: OR-ing in bf16 1.0 makes u = x.
  const uint32_t gor = norm ? 0u : 0x3F803F80u;

  // The ring is filled in the order the loop consumes and refills it (each slot's
  // loads kept together by a scheduling barrier): the wait counts the compiler places
  // at the loop head then hold on entry too, instead of draining every load.
  u32x4 wr[D][G];
#pragma unroll
  for (int dd = 0; dd < D; ++dd) {
#pragma unroll
    for (int r = 0; r < G; ++r)
      wr[dd][r] = __builtin_amdgcn_raw_buffer_load_b128(wrs, mfma_small_woff(g, gb0 + r, lterm, sstride, dd, nst), 0,
                                                        kCachePolicyNT);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (first) {
    if (!dep_wait(a, t, d.remaining_deps, sm)) return false;
    // The input is read with plain loads: drop stale L1/L2 lines first.
    if (threadIdx.x == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    __syncthreads();
  }
  u32x4 xr[D];
  u32x2 gr[D];
#pragma unroll
  for (int dd = 0; dd < D; ++dd) {
    xr[dd] = __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff(dd), 0, 0);
    gr[dd] = __builtin_amdgcn_raw_buffer_load_b64(grs, goff(dd), 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  f32x4 acc[G];
#pragma unroll
  for (int r = 0; r < G; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
  // One k-step from ring slot dd (steps s0 + dd; the slot is refilled with s0 + dd + D).
  auto step = [&](int dd, int s0, auto refill_c) __attribute__((always_inline)) {
    constexpr bool REFILL = decltype(refill_c)::value;
    const int sn = s0 + dd + D;
    // u = x gamma for this lane's 4 values (the sum of squares is of x itself).
    float u[4];
    {
      const u32x4 xx = xr[dd];
      const u32x2 gg = gr[dd];
      const float xv[4] = {__uint_as_float(xx.x), __uint_as_float(xx.y), __uint_as_float(xx.z),
                           __uint_as_float(xx.w)};
      const uint32_t g0 = gg.x | gor, g1 = gg.y | gor;
      const float gv[4] = {bf16_lo(g0), bf16_hi(g0), bf16_lo(g1), bf16_hi(g1)};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ss = fmaf(xv[e], xv[e], ss);
        u[e] = xv[e] * gv[e];
      }
    }
    // Every read of the slots' old values is done before they are refilled, so the
    // refills land in the same registers (no copies, whose waits would drain the ring):
    // the products are pinned in registers first.
#pragma unroll
    for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(u[e]));
    __builtin_amdgcn_sched_barrier(0);
    if (REFILL) {
      xr[dd] = __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff(sn), 0, 0);
      gr[dd] = __builtin_amdgcn_raw_buffer_load_b64(grs, goff(sn), 0, 0);
    }
    // hi = u with the low 16 bits cleared, lo = the same of the exact remainder u - hi;
    // v_perm packs the upper halves of two floats into one bf16 pair.  The lane splits
    // its own 4 values and swaps half with its partner (lane ^ 8): a hi lane keeps the
    // hi parts of k .. k+3 and receives those of k+4 .. k+7, a lo lane the reverse.
    uint32_t hw[2], lw[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t a0 = __float_as_uint(u[2 * e]), a1 = __float_as_uint(u[2 * e + 1]);
      hw[e] = __builtin_amdgcn_perm(a1, a0, 0x07060302u);
      const float r0 = u[2 * e] - __uint_as_float(a0 & 0xFFFF0000u);
      const float r1 = u[2 * e + 1] - __uint_as_float(a1 & 0xFFFF0000u);
      lw[e] = __builtin_amdgcn_perm(__float_as_uint(r1), __float_as_uint(r0), 0x07060302u);
    }
    const uint32_t s0w = lo_lane ? hw[0] : lw[0], s1w = lo_lane ? hw[1] : lw[1];
    const uint32_t r0w = __float_as_uint(lane_xor<8>(__uint_as_float(s0w)));
    const uint32_t r1w = __float_as_uint(lane_xor<8>(__uint_as_float(s1w)));
    uint32_t bw[4];
    bw[0] = lo_lane ? r0w : hw[0];
    bw[1] = lo_lane ? r1w : hw[1];
    bw[2] = lo_lane ? lw[0] : r0w;
    bw[3] = lo_lane ? lw[1] : r1w;
    const bf16x8 bop = __builtin_bit_cast(bf16x8, u32x4{bw[0], bw[1], bw[2], bw[3]});
#pragma unroll
    for (int r = 0; r < G; ++r) {
      // The product first, then the refill of the same ring slot: the new load can
      // land in the registers the product has read, so the ring never needs copying.
      acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wr[dd][r]), bop, acc[r], 0, 0, 0);
      if (REFILL)
        wr[dd][r] = __builtin_amdgcn_raw_buffer_load_b128(wrs, mfma_small_woff(g, gb0 + r, lterm, sstride, sn, nst), 0,
                                                          kCachePolicyNT);
    }
    // Keep each step's loads in its own step: the scheduler would otherwise gather
    // them at the end of the unrolled body, where they all drain before the next.
    __builtin_amdgcn_sched_barrier(0);
  };
  // The first D steps run outside the loop: they leave the ring in the order the loop
  // refills it, so the wait counts at the loop head are exact on entry as well.
  // The last D steps refill nothing (their refills would all fall past the last step,
  // and loads still in flight at the end of the stream hold up the epilogue).
  if (nst > D) {
#pragma unroll
    for (int dd = 0; dd < D; ++dd) step(dd, 0, std::true_type{});
    int s0 = D;
    for (; s0 + D < nst; s0 += D) {
#pragma unroll
      for (int dd = 0; dd < D; ++dd) step(dd, s0, std::true_type{});
    }
#pragma unroll
    for (int dd = 0; dd < D; ++dd) step(dd, s0, std::false_type{});
  } else {
#pragma unroll
    for (int dd = 0; dd < D; ++dd) step(dd, 0, std::false_type{});
  }
  // Sum of squares of each batch row over this wave's segment: the hi and lo lanes of
  // the row's column pair in the four k-quarters hold every value once.
  float* part = sm.xs;                       // [kWaves][G][64 lanes] f32x4
  float* row_ss = sm.red + kRedFloats - 128;  // [kWaves][8]
  if (need_ss) {
    ss += lane_xor<8>(ss);  // the hi and lo lanes of a row hold its two halves
    ss += lane_xor<16>(ss);
    ss += lane_xor<32>(ss);
    if (lane < 8) row_ss[w * 8 + lane] = ss;
  }
#pragma unroll
  for (int r = 0; r < G; ++r) *(f32x4*)(part + ((w * G + r) * 64 + lane) * 4) = acc[r];
  __syncthreads();

  // Epilogue: element e = (block or SiLU pair q, row n of the block, batch row b).
  const int per = g.silu ? G / 2 : G;
  const int nel = per * 16 * B;
  for (int e = threadIdx.x; e < nel; e += kThreads) {
    const int q = e / (16 * B), rem = e - q * 16 * B, n = rem / B, b = rem - n * B;
    const int lh = (n >> 2) * 16 + b, ll = lh + 8, tt = n & 3;
    auto sum_block = [&](int r) {
      float s = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float* pr = part + (ww * G + r) * 64 * 4;
        s += pr[lh * 4 + tt] + pr[ll * 4 + tt];
      }
      return s;
    };
    float scale = 1.f;
    if (norm) {
      float tot = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) tot += row_ss[ww * 8 + b];
      scale = 1.0f / sqrtf(tot / (float)g.K + a.rms_eps);
    }
    float v;
    int col;
    if (g.silu) {
      const float gt = sum_block(2 * q) * scale, up = sum_block(2 * q + 1) * scale;
      v = gt / (1.f + __expf(-gt)) * up;
      col = g.c0 + 16 * ((gb0 >> 1) + q) + n;
    } else {
      v = sum_block(q) * scale;
      col = g.c0 + 16 * (gb0 + q) + n;
    }
    const size_t o = (size_t)b * N + col;
    st_dev<float>(y, o, v + (resid ? ld_dev<float>(aux, o) : 0.f));
  }
  __syncthreads();  // the partial-sum area and the row sums are read by every thread
  return true;
}

__device__ __forceinline__ void gemv_mfma_small(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm) {
  MfmaGeom g;
  g.W = resolve(a, d.in_buf[1]);
  g.K = (uint32_t)d.k;
  g.c0 = (int)d.reserved[0];
  g.cols = (int)d.reserved[1];
  g.I = (int)d.reserved[2];
  g.silu = (d.flags & MK_FLAG_SILU_MUL) ? 1 : 0;
  g.nc = 0;
  g.packed = a.wpacked ? 1 : 0;
  const char* x = resolve(a, d.in_buf[0]);
  const char* aux = d.in_buf[2] != 0xFFFF ? resolve(a, d.in_buf[2]) : nullptr;
  float* y = (float*)resolve(a, d.out_buf);
  const bool norm = d.flags & MK_FLAG_RMS_NORM_INPUT;
  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.W, (short)0, (int)kWeightRange, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)((uint32_t)d.m * g.K * 4u), kRawBufferWord3);
  // Without the norm the gamma resource has range 0: its loads (unconditional, so the
  // streaming loop has no branch) read nothing and return zeros, which are not used.
  const __amdgpu_buffer_rsrc_t grs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(norm ? aux : x), (short)0, (int)(norm ? g.K * 2u : 0u), kRawBufferWord3);
  const int R = (g.cols >> 4) << g.silu;  // blocks of 16 weight rows
  bool first = true;
  for (int gb0 = 0; gb0 < R;) {
    const int left = R - gb0;
    bool ok;
    if (left >= 8) {
      ok = mfma_small_group<8, 2>(a, d, t, sm, g, gb0, first, aux, y, wrs, xrs, grs, first);
      gb0 += 8;
    } else if (left >= 4) {
      ok = mfma_small_group<4, 4>(a, d, t, sm, g, gb0, first, aux, y, wrs, xrs, grs, first);
      gb0 += 4;
    } else if (left >= 2) {
      ok = mfma_small_group<2, 8>(a, d, t, sm, g, gb0, first, aux, y, wrs, xrs, grs, first);
      gb0 += 2;
    } else {
      ok = mfma_small_group<1, 8>(a, d, t, sm, g, gb0, first, aux, y, wrs, xrs, grs, first);
      gb0 += 1;
    }
    if (!ok) return;
    first = false;
  }
}

}  // namespace mk
