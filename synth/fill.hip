// Device twin of the seeded generator defined in gen.py (SplitMix64 stream per
// tensor, Irwin-Hall(4) of the four 16-bit fields, v = mean + z*scale in binary64
// without fusion, rounded to binary32 and then to bfloat16 for bf16 tensors).
// Used to fill multi-gigabyte weights and KV caches in place on the GPU; holds no
// arithmetic of the decode method.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define G_INC 0x9E3779B97F4A7C15ULL

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

__device__ __forceinline__ double draw(uint64_t key, uint64_t i, double mean, double scale) {
#pragma clang fp contract(off)
    uint64_t w = mix64(key + (i + 1) * G_INC);
    int64_t s = (int64_t)(w & 0xFFFF) + (int64_t)((w >> 16) & 0xFFFF) +
                (int64_t)((w >> 32) & 0xFFFF) + (int64_t)(w >> 48);
    double t = (double)(s - 131070) * scale;
    return mean + t;
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ void store(void* dst, int dtype, uint64_t j, double v) {
    if (dtype == 0) ((float*)dst)[j] = __double2float_rn(v);
    else ((uint16_t*)dst)[j] = bf16_rne(__double2float_rn(v));
}

__global__ void fill_flat_kernel(void* dst, int dtype, uint64_t n, uint64_t start, uint64_t key,
                                 double mean, double scale) {
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
        store(dst, dtype, j, draw(key, start + j, mean, scale));
}

__global__ void fill_cache_kernel(void* dst, int dtype, uint64_t n_bg, uint64_t n_slots,
                                  uint64_t head_dim, uint64_t pitch, uint64_t key, double mean,
                                  double scale) {
    uint64_t total = n_bg * n_slots * head_dim;
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < total; j += stride) {
        uint64_t d = j % head_dim, r = j / head_dim;
        uint64_t slot = r % n_slots, bg = r / n_slots;
        store(dst, dtype, j, draw(key, (bg * pitch + slot) * head_dim + d, mean, scale));
    }
}

static uint64_t host_mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static unsigned grid_for(uint64_t n) {
    uint64_t g = (n + 255) / 256;
    return (unsigned)(g > 65536 ? 65536 : (g == 0 ? 1 : g));
}

extern "C" int synth_gpu_fill_flat(void* dst, int dtype, uint64_t n, uint64_t start, uint64_t seed,
                                   uint64_t tid, double mean, double scale, void* stream) {
    if (n == 0) return 0;
    uint64_t key = host_mix64(host_mix64(seed + G_INC) + (tid + 1) * G_INC);
    hipLaunchKernelGGL(fill_flat_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, dst,
                       dtype, n, start, key, mean, scale);
    return (int)hipGetLastError();
}

extern "C" int synth_gpu_fill_cache(void* dst, int dtype, uint64_t n_bg, uint64_t n_slots,
                                    uint64_t head_dim, uint64_t pitch, uint64_t seed, uint64_t tid,
                                    double mean, double scale, void* stream) {
    uint64_t total = n_bg * n_slots * head_dim;
    if (total == 0) return 0;
    uint64_t key = host_mix64(host_mix64(seed + G_INC) + (tid + 1) * G_INC);
    hipLaunchKernelGGL(fill_cache_kernel, dim3(grid_for(total)), dim3(256), 0, (hipStream_t)stream,
                       dst, dtype, n_bg, n_slots, head_dim, pitch, key, mean, scale);
    return (int)hipGetLastError();
}

// A plain device copy of n_bytes (a multiple of 16): every byte read once and
// written once.  Profilers run it beside the decode step to calibrate their HBM byte
// counters against a known traffic.
__global__ void copy16_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, uint64_t n) {
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride) dst[j] = src[j];
}

extern "C" int synth_gpu_copy(void* dst, const void* src, uint64_t n_bytes, void* stream) {
    if (n_bytes % 16 != 0) return (int)hipErrorInvalidValue;
    if (n_bytes == 0) return 0;
    hipLaunchKernelGGL(copy16_kernel, dim3(1024), dim3(256), 0, (hipStream_t)stream, (const uint4*)src,
                       (uint4*)dst, n_bytes / 16);
    return (int)hipGetLastError();
}

// A plain streaming read of n 16-byte words: every byte read once, one word per
// workgroup written (the XOR of what it read, so the loads are kept).  The measured
// ceiling of a read-only stream on this part, beside the published peak.  Eight
// independent 16-byte non-temporal loads per thread and iteration (the weight streams'
// access kind) keep enough bytes in flight.
typedef unsigned int read_u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read16_kernel(const read_u32x4* __restrict__ src, uint64_t n, uint32_t* out) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; j + 7 * stride < n; j += 8 * stride) {
        read_u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + j + u * stride);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; j < n; j += stride) {
        const read_u32x4 a = __builtin_nontemporal_load(src + j);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    __shared__ uint32_t red[256];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int i = 0; i < 256; ++i) r ^= red[i];
        out[blockIdx.x] = r;
    }
}

// out: blocks uint32 words (device).  n_bytes a multiple of 16.
extern "C" int synth_gpu_read(const void* src, uint64_t n_bytes, void* out, uint32_t blocks, void* stream) {
    if (n_bytes % 16 != 0 || blocks == 0) return (int)hipErrorInvalidValue;
    if (n_bytes == 0) return 0;
    hipLaunchKernelGGL(read16_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const read_u32x4*)src,
                       n_bytes / 16, (uint32_t*)out);
    return (int)hipGetLastError();
}
