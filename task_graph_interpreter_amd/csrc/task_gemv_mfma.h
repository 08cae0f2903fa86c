// GEMV task body on the matrix cores, for tiles whose batch makes the product a real
// dense contraction (descriptor config_id MK_GEMV_BF16_MFMA: bf16 weights, column
// tiles aligned to 16).  Same operation as the streaming GEMV ("Mega kernel initial",
// lowering section: one task per output-column tile; descriptor section: flags
// SILU_MUL, ADD_RESIDUAL, RMS_NORM_INPUT):
//   y[b, c] = r_b * sum_k (x[b, k] gamma_k) W[c, k]   (+ res[b, c]; SiLU pairs)
// The matrix cores take bf16 operands.  The weights are bf16 already; the fp32 input
// is split as u = hi + lo with hi = bf16(u) and lo = bf16(u - hi) (u - hi is exact in
// fp32), and W u = W hi + W lo takes two products, so the input keeps ~16 significant
// bits instead of 8 (rounding it to bf16 alone moved 8B-class logits by up to 0.14
// after 32 layers, far outside the parity bound).
//
// Layout (v_mfma_f32_16x16x32_bf16: D[16 x 16] += A[16 x 32] B[32 x 16]):
//  * A = 16 weight rows x 32 k: lane l holds row l % 16, k = 8 (l / 16) .. +8, which
//    is one 16-byte load straight from the row-major weights;
//  * B = 32 k x 16 batch rows of the staged input (hi, then lo), from LDS; four
//    products per A cover 32 batch rows;
//  * D: lane l holds batch row l % 16 of output rows 4 (l / 16) .. +4.
//
// Work split.  The weight rows of the tile are cut into blocks of 16 (SILU_MUL: gate
// and up blocks interleaved, so a pair stays in one group), processed in groups of G
// slots (8 slots for 5..8 blocks, 4 for 3..4, then 2, 1; every group restages the
// whole input, so a tile runs as few groups as it can, and the empty slots of a group
// load zeros without touching memory).  K is cut into chunks of 256.  The workgroup's
// waves specialise, because
// a wave's loads complete in issue order: a wave that loaded both weights and input
// would drain its whole weight ring every time it waited for an input chunk.
//  * Compute waves 0-3: wave w owns k-steps 2w and 2w + 1 (32 k each) of every chunk,
//    for every block of the group.  A ring of 8 / G chunks of weight loads per block
//    is in flight per lane (started before the dependency wait for the first group).
//  * Staging waves 4-7 load input chunks two ahead into registers, scale by gamma,
//    split into bf16 hi and lo (the hardware pair conversion, round to nearest even),
//    and write them to one of three LDS buffers, accumulating x^2 per batch row for the
//    RMS scale; tiles without the norm compile neither the gamma product nor the sums.
//    The staging VALU work is what bounds these tiles.
//  * One workgroup barrier per chunk.  A buffer is rewritten one chunk after the
//    compute waves last read it (the barrier in between orders the two).
// After the last chunk, the four compute waves' partial sums are added in LDS in a
// fixed order, and the epilogue (r_b, residual, SiLU * up) writes y.
//
// The input is a whole activation buffer that every producer has finished (the tile
// reads all K columns).  So after the wait it is read with plain, L2-cached loads
// following one agent-scope acquire: the 32 CUs of an XCD then share it through their
// L2.
#pragma once

#include <type_traits>

#include "device_common.h"

namespace mk {

constexpr int kMfmaKC = 256;                 // k per chunk: 4 compute waves x 2 x 32
constexpr int kMfmaXPitch = kMfmaKC + 8;     // bf16 per staged row (+16 B against bank conflicts)
constexpr int kMfmaXHalf = 32 * kMfmaXPitch; // bf16 per staged chunk part (hi or lo; 32 batch rows)
constexpr int kMfmaXBuf = 2 * kMfmaXHalf;    // bf16 per staged chunk (hi, then lo)
constexpr int kMfmaXBufs = 3;                // staged chunks held in LDS
constexpr int kMfmaComputeWaves = 4;

struct MfmaGeom {
  const char* W;
  uint32_t K;        // inner dim
  int c0, cols, I;   // first output column, tile width, up-row offset (SILU_MUL)
  int silu;
  int nc;            // chunks
  int packed;        // weights in the 16-row tile layout of mk_pack_matrix
};

// First weight row of global block gb (SILU_MUL: even blocks gate, odd blocks up).
__device__ __forceinline__ int mfma_block_row(const MfmaGeom& g, int gb) {
  if (!g.silu) return g.c0 + 16 * gb;
  return g.c0 + 16 * (gb >> 1) + ((gb & 1) ? g.I : 0);
}

// One lane's 16 bytes of A for a block whose first row starts at byte `blk` of the
// matrix, chunk c, k-step s (0..7).  Both layouts give the block's base (first row
// times 2K) + a per-lane term + c and s times per-chunk and per-step strides:
//  * row-major: lane l reads row l % 16 at k = 256 c + 32 s + 8 (l / 16): lane term
//    2K (l % 16) + 16 (l / 16), strides 512 and 64 bytes;
//  * tile layout: the k-step's 1 KB tile of the block sits at 1024 (8 c + s), lane l's
//    bytes at 16 l: lane term 16 l, strides 8192 and 1024 bytes (the same values).
// A raw buffer load with a 32-bit offset (offsets < 4 GiB, checked when lowering):
// no per-load layout branch or 64-bit address arithmetic, so the ring fill issues its
// loads back to back instead of waiting on values the compiler had spilled.
struct MfmaWAddr {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t lterm, cstride, sstride;
};

// The resource's range is the matrix's bytes (rows = the tile's N, or gate and up
// rows with SiLU): a block slot with no block points at the end, so its loads fall
// out of range and read zeros without a memory access.
__device__ __forceinline__ uint32_t mfma_matrix_bytes(const MfmaGeom& g, const mk_task_t& d) {
  const uint32_t rows = g.silu ? 2u * (uint32_t)g.I : (uint32_t)d.n;
  return rows * g.K * 2u;
}

__device__ __forceinline__ MfmaWAddr mfma_waddr(const MfmaGeom& g, int lane, uint32_t range) {
  MfmaWAddr w;
  w.rs = __builtin_amdgcn_make_buffer_rsrc((void*)g.W, (short)0, (int)range, kRawBufferWord3);
  w.lterm = g.packed ? 16u * (uint32_t)lane : 2u * g.K * (uint32_t)(lane & 15) + 16u * (uint32_t)(lane >> 4);
  w.cstride = g.packed ? 8192u : 512u;
  w.sstride = g.packed ? 1024u : 64u;
  return w;
}

__device__ __forceinline__ uint32_t mfma_blk(const MfmaGeom& g, int gb) {
  return (uint32_t)mfma_block_row(g, gb) * g.K * 2u;
}

__device__ __forceinline__ u32x4 mfma_wload(const MfmaWAddr& wa, uint32_t blk, int c, int s) {
  return __builtin_amdgcn_raw_buffer_load_b128(wa.rs, blk + wa.lterm + (uint32_t)c * wa.cstride + (uint32_t)s * wa.sstride,
                                               0, kCachePolicyNT);
}

// Input chunk c of batch rows [b0, b0 + 32), as loaded by one staging thread st
// (0..255): float4 k4 = st % 64 of rows b0 + st / 64 + 4 i, i = 0..7, and the gammas
// of its k4.  Loads are unconditional (rows past the batch re-read the last row and
// are zeroed when staged; without the norm `gamma` points at any readable buffer and
// is ignored), so the wait counts stay exact.  The input is read through a raw buffer
// resource with 32-bit offsets computed here from an opaque row base, so the compiler
// keeps no per-row pointers alive across the chunk loop.
struct XChunk {
  f32x4 v[8];
  u32x2 gm;
};

__device__ __forceinline__ void mfma_xload(__amdgpu_buffer_rsrc_t xr, const char* gamma, uint32_t K, int B, int b0,
                                           int c, int st, XChunk& xr_out) {
  int r0 = b0 + (st >> 6);
  asm volatile("" : "+v"(r0));
  const uint32_t col = (uint32_t)c * kMfmaKC * 4u + (uint32_t)(st & 63) * 16u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int b = r0 + 4 * i;
    const uint32_t row = (uint32_t)(b < B ? b : B - 1);
    const uint32_t off = row * K * 4u + col;
    xr_out.v[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
  }
  xr_out.gm = ldg<u32x2>(gamma, (size_t)c * (kMfmaKC / 4) + (st & 63));
}

// Two floats rounded to bf16 (nearest even) and packed, the first in the low half.
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)a, (__bf16)b});
}

// Writes u = x * gamma into LDS buffer `xb` as bf16 hi and lo parts and, if `count`,
// adds x^2 into ss (pre-gamma; the RMS scale multiplies the finished dot product).
// Without the norm (NORM false) u = x and no sum is kept.  Staging wave w' holds rows
// w' + 4 i; rows past the batch are written as zeros (`full`: none is).
template <bool NORM>
__device__ __forceinline__ void mfma_xstage(const XChunk& xr, bool count, bool full, int B, int b0, int st,
                                            uint16_t* xb, float ss[8]) {
  const float g0 = NORM ? bf16_lo(xr.gm.x) : 1.f, g1 = NORM ? bf16_hi(xr.gm.x) : 1.f;
  const float g2 = NORM ? bf16_lo(xr.gm.y) : 1.f, g3 = NORM ? bf16_hi(xr.gm.y) : 1.f;
  // Row st / 64 + 4 i, element 4 (st % 64): one base address, compile-time offsets.
  uint16_t* base = xb + (st >> 6) * kMfmaXPitch + 4 * (st & 63);
  const int br0 = b0 + (st >> 6);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f32x4 v = xr.v[i];
    if (!full && br0 + 4 * i >= B) v = f32x4{0.f, 0.f, 0.f, 0.f};
    if (NORM) {
      const float q = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, v.w * v.w)));
      ss[i] += count ? q : 0.f;
    }
    const float u0 = NORM ? v.x * g0 : v.x, u1 = NORM ? v.y * g1 : v.y;
    const float u2 = NORM ? v.z * g2 : v.z, u3 = NORM ? v.w * g3 : v.w;
    // Round to nearest even with the hardware pair conversion (v_cvt_pk_bf16_f32).
    const u32x2 hi = {cvt_bf16x2(u0, u1), cvt_bf16x2(u2, u3)};
    const u32x2 lo = {cvt_bf16x2(u0 - bf16_lo(hi.x), u1 - bf16_hi(hi.x)),
                      cvt_bf16x2(u2 - bf16_lo(hi.y), u3 - bf16_hi(hi.y))};
    *(u32x2*)(base + 4 * i * kMfmaXPitch) = hi;
    *(u32x2*)(base + kMfmaXHalf + 4 * i * kMfmaXPitch) = lo;
  }
}

__device__ __forceinline__ f32x4 mfma_step(const u32x4 a, const uint16_t* xb, int h, int s, int lane, f32x4 acc) {
  const int off = (16 * h + (lane & 15)) * kMfmaXPitch + 32 * s + 8 * (lane >> 4);
  const u32x4 bh = *(const u32x4*)(xb + off);
  const u32x4 bl = *(const u32x4*)(xb + kMfmaXHalf + off);
  const bf16x8 av = __builtin_bit_cast(bf16x8, a);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, bh), acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, bl), acc, 0, 0, 0);
}

// One group of G block slots, the first nreal of them blocks [gb0, gb0 + nreal), over
// all K for batch rows [b0, b0 + 32): each group restages the whole input, so a tile
// runs as few groups as possible.  Slots past nreal load through a buffer resource of
// range 0 (zeros, no memory access) and are not written.  Returns false if the step
// was abandoned while waiting.
template <int G>
__device__ __forceinline__ bool mfma_group(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm,
                                           const MfmaGeom& g, int gb0, int nreal, int b0, bool first, const float* x,
                                           const char* aux, float* y, bool need_ss) {
  constexpr int D = 8 / G;           // chunks of weight loads in flight per block (2 k-steps each)
  constexpr int U = D < 2 ? 2 : D;   // chunk loop unroll: ring slot and input register set are static
  int lane = lane_id();
  asm volatile("" : "+v"(lane));  // recomputed per task, not hoisted and spilled
  const int w = wave_id();
  const bool compute = w < kMfmaComputeWaves;
  const int B = d.m, N = d.n;
  const bool norm = d.flags & MK_FLAG_RMS_NORM_INPUT;
  const bool resid = d.flags & MK_FLAG_ADD_RESIDUAL;
  const char* gamma = norm ? aux : (const char*)x;
  uint16_t* xbuf = (uint16_t*)sm.xs;  // [kMfmaXBufs][hi, lo][32][kMfmaXPitch] bf16
  // The input rows as a raw buffer (B x K fp32; B * K * 4 < 4 GiB, checked when lowering).
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)((uint32_t)B * g.K * 4u), kRawBufferWord3);
  const int st = threadIdx.x - kMfmaComputeWaves * 64;  // staging thread index (staging waves)

  float* row_ss = sm.red + kRedFloats - 32;
  float* part = sm.xs;  // [4 compute waves][G][2 halves][64 lanes][4]
  // The two roles run in separate branches from the first load to the hand-off of
  // their results, so the weight ring and accumulators (compute waves) and the staged
  // input registers (staging waves) are never live at the same time and can share
  // registers.  The branch is wave-uniform, and both sides execute the same sequence
  // of barriers: the dependency wait's, one after the first input chunks are staged,
  // one per chunk, and one before the partial sums are written.
  if (compute) {
    const uint32_t range = mfma_matrix_bytes(g, d);
    const MfmaWAddr wad = mfma_waddr(g, lane, range);
    uint32_t blk[G];  // byte offset of each block's first row (wave-uniform); past the end if none
#pragma unroll
    for (int r = 0; r < G; ++r) blk[r] = r < nreal ? mfma_blk(g, gb0 + r) : range;
    u32x4 ring[D][G][2];
#pragma unroll
    for (int dc = 0; dc < D; ++dc)
#pragma unroll
      for (int r = 0; r < G; ++r)
#pragma unroll
        for (int j = 0; j < 2; ++j) ring[dc][r][j] = mfma_wload(wad, dc < g.nc ? blk[r] : range, dc < g.nc ? dc : 0, 2 * w + j);
    if (first) {
      if (!dep_wait(a, t, d.remaining_deps, sm)) return false;
      // The input is read with plain loads: drop stale L1/L2 lines first.
      if (threadIdx.x == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __syncthreads();
    }
    __syncthreads();  // the first input chunks are staged
    f32x4 acc[G][2];
#pragma unroll
    for (int r = 0; r < G; ++r) acc[r][0] = acc[r][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < g.nc; c0 += U) {
#pragma unroll
      for (int dc = 0; dc < U; ++dc) {
        const int c = c0 + dc;
        if (c < g.nc) {
          const uint16_t* xc = xbuf + (c % kMfmaXBufs) * kMfmaXBuf;
          // Refills past the last chunk point past the matrix's range: they read
          // nothing (no repeated loads of the last chunk).
          const bool past = c + D >= g.nc;
          const int cn = past ? 0 : c + D;
#pragma unroll
          for (int r = 0; r < G; ++r) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const u32x4 wa = ring[dc % D][r][j];
              ring[dc % D][r][j] = mfma_wload(wad, past ? range : blk[r], cn, 2 * w + j);
              acc[r][0] = mfma_step(wa, xc, 0, 2 * w + j, lane, acc[r][0]);
              acc[r][1] = mfma_step(wa, xc, 1, 2 * w + j, lane, acc[r][1]);
            }
          }
          __syncthreads();
        }
      }
    }
    __syncthreads();  // every wave is done with the staged input; partial sums reuse it
#pragma unroll
    for (int r = 0; r < G; ++r)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        *(f32x4*)(part + (((w * G + r) * 2 + h) * 64 + lane) * 4) = acc[r][h];
  } else {
    if (first) {
      if (!dep_wait(a, t, d.remaining_deps, sm)) return false;
      __syncthreads();
    }
    const bool full = b0 + 32 <= B;  // every staged row is a batch row
    // The staging loop, with the norm's gamma product and sums of squares compiled in
    // only where the tile has the norm.
    auto stage_all = [&](auto norm_c) __attribute__((always_inline)) {
      constexpr bool NORM = decltype(norm_c)::value;
      float ss[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      XChunk xa, xb2;  // the next two input chunks to stage
      mfma_xload(xrs, gamma, g.K, B, b0, 0, st, xa);
      mfma_xload(xrs, gamma, g.K, B, b0, g.nc > 1 ? 1 : 0, st, xb2);
      mfma_xstage<NORM>(xa, true, full, B, b0, st, xbuf, ss);
      mfma_xload(xrs, gamma, g.K, B, b0, g.nc > 2 ? 2 : g.nc - 1, st, xa);
      mfma_xstage<NORM>(xb2, g.nc > 1, full, B, b0, st, xbuf + kMfmaXBuf, ss);
      mfma_xload(xrs, gamma, g.K, B, b0, g.nc > 3 ? 3 : g.nc - 1, st, xb2);
      __syncthreads();  // the first input chunks are staged
      for (int c0 = 0; c0 < g.nc; c0 += U) {
#pragma unroll
        for (int dc = 0; dc < U; ++dc) {
          const int c = c0 + dc;
          if (c < g.nc) {
            // Stage chunk c + 2 into the buffer chunk c - 1 used (every compute wave
            // finished chunk c - 1 before the previous barrier), then load chunk c + 4
            // into the freed registers.  Chunks past the end re-stage the last one
            // into an idle buffer and are not counted in ss.
            XChunk& xs = (dc & 1) ? xb2 : xa;  // c0 is even
            mfma_xstage<NORM>(xs, c + 2 < g.nc, full, B, b0, st, xbuf + ((c + 2) % kMfmaXBufs) * kMfmaXBuf, ss);
            mfma_xload(xrs, gamma, g.K, B, b0, c + 4 < g.nc ? c + 4 : g.nc - 1, st, xs);
            __syncthreads();
          }
        }
      }
      // Sum of squares of each staged batch row, kept in LDS for every group of this
      // batch block (first group only: later groups restage the same rows).  Staging
      // wave w' holds rows w' + 4 i, each lane one float4 of every chunk.
      if (NORM && need_ss) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float s = wave_sum(ss[i]);
          if (lane == 0) row_ss[(w - kMfmaComputeWaves) + 4 * i] = s;
        }
      }
    };
    if (norm) stage_all(std::true_type{});
    else stage_all(std::false_type{});
    __syncthreads();  // every wave is done with the staged input; partial sums reuse it
  }
  __syncthreads();

  // Epilogue: element e = (pair or block, row 0..15, batch 0..31), real blocks only.
  const int per = g.silu ? nreal / 2 : nreal;
  for (int e = threadIdx.x; e < per * 512; e += kThreads) {
    const int q = e >> 9, rem = e & 511, rho = rem >> 5, bb = rem & 31;
    const int b = b0 + bb;
    if (b >= B) continue;
    const int h = bb >> 4, ln = (rho >> 2) * 16 + (bb & 15), i = rho & 3;
    auto sum_block = [&](int r) {
      float s = 0.f;
      for (int ww = 0; ww < kMfmaComputeWaves; ++ww) s += part[(((ww * G + r) * 2 + h) * 64 + ln) * 4 + i];
      return s;
    };
    const float scale = norm ? 1.0f / sqrtf(row_ss[bb] / (float)g.K + a.rms_eps) : 1.f;
    float v;
    int col;
    if (g.silu) {
      const float gt = sum_block(2 * q) * scale, up = sum_block(2 * q + 1) * scale;
      v = gt / (1.f + __expf(-gt)) * up;
      col = g.c0 + 16 * ((gb0 >> 1) + q) + rho;
    } else {
      v = sum_block(q) * scale;
      col = g.c0 + 16 * (gb0 + q) + rho;
    }
    const size_t o = (size_t)b * N + col;
    st_dev<float>(y, o, v + (resid ? ld_dev<float>(aux, o) : 0.f));
  }
  __syncthreads();  // the partial-sum area is the next group's input buffer
  return true;
}

__device__ __forceinline__ void gemv_mfma(const LaunchArgs& a, const mk_task_t& d, uint32_t t, Smem& sm) {
  MfmaGeom g;
  g.W = resolve(a, d.in_buf[1]);
  g.K = (uint32_t)d.k;
  g.c0 = (int)d.reserved[0];
  g.cols = (int)d.reserved[1];
  g.I = (int)d.reserved[2];
  g.silu = (d.flags & MK_FLAG_SILU_MUL) ? 1 : 0;
  g.nc = d.k / kMfmaKC;
  g.packed = a.wpacked ? 1 : 0;
  const float* x = (const float*)resolve(a, d.in_buf[0]);
  const char* aux = d.in_buf[2] != 0xFFFF ? resolve(a, d.in_buf[2]) : nullptr;
  float* y = (float*)resolve(a, d.out_buf);
  const int R = (g.cols >> 4) << g.silu;  // blocks of 16 weight rows
  bool first = true;
  for (int b0 = 0; b0 < d.m; b0 += 32) {
    bool need_ss = true;
    for (int gb0 = 0; gb0 < R;) {
      const int left = R - gb0;
      bool ok;
      // Groups of 8 slots take 5..8 blocks, of 4 take 3..4 (with SiLU the count is even).
      if (left >= 5) {
        const int nr = left < 8 ? left : 8;
        ok = mfma_group<8>(a, d, t, sm, g, gb0, nr, b0, first, x, aux, y, need_ss);
        gb0 += nr;
      } else if (left >= 3) {
        ok = mfma_group<4>(a, d, t, sm, g, gb0, left, b0, first, x, aux, y, need_ss);
        gb0 += left;
      } else if (left == 2) {
        ok = mfma_group<2>(a, d, t, sm, g, gb0, 2, b0, first, x, aux, y, need_ss);
        gb0 += 2;
      } else {
        ok = mfma_group<1>(a, d, t, sm, g, gb0, 1, b0, first, x, aux, y, need_ss);
        gb0 += 1;
      }
      if (!ok) return;
      first = false;
      need_ss = false;
    }
  }
}

}  // namespace mk
