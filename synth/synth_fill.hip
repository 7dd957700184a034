// synth_fill.hip -- device side of the seeded synthetic gradients (the
// definitions are in synth.h; synth.c is the host side and must produce the
// same bits), the streaming compute kernel the overlap measurement runs
// beside the all-reduce, and plain streaming kernels of known bytes (a copy,
// a read, a write) that calibrate the memory counters and give the rate the
// hardware reaches on a plain stream.  None of the all-reduce's arithmetic
// is here.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kG = 0x9E3779B97F4A7C15ull;

__host__ __device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// One IEEE operation per step, in the order synth.c takes them.
__device__ __forceinline__ float value_f32(int dist, uint64_t key, int rank, uint64_t e,
                                           double scale) {
    switch (dist) {
    case 0: {  // uniform [-1, 1)
        int32_t u = (int32_t)(mix64(key + (e + 1) * kG) >> 40);
        return (float)(u - (1 << 23)) * 0x1p-23f;
    }
    case 1: {  // Irwin-Hall approximation of N(0, sigma^2)
        int64_t s = 0;
        for (int j = 0; j < 6; ++j) {
            uint64_t w = mix64(key + (6 * e + (uint64_t)j + 1) * kG);
            s += (int64_t)(w & 0xffffffffull) + (int64_t)(w >> 32);
        }
        int64_t T = 2 * s - 12 * (int64_t)0xffffffffll;
        return __double2float_rn(__dmul_rn((double)T, scale));
    }
    case 2:
        return (float)(rank + 1);
    default:
        return (float)((int)(mix64(key + (e + 1) * kG) >> 57) - 64);
    }
}

__global__ void fill_f32(float *dst, int dist, uint64_t key, int rank, uint64_t first,
                         uint64_t count, double scale) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
        dst[i] = value_f32(dist, key, rank, first + i, scale);
}

__global__ void fill_f16(_Float16 *dst, int dist, uint64_t key, int rank, uint64_t first,
                         uint64_t count, double scale) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
        dst[i] = (_Float16)value_f32(dist, key, rank, first + i, scale);
}

// a = alpha * a + beta over n floats, 16 bytes per lane access: stands in for
// the backward-pass compute the all-reduce overlaps with.
__global__ void stream_compute(float *a, uint64_t n, float alpha, float beta) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const uint64_t nv = n / 4;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    f32x4 *v = reinterpret_cast<f32x4 *>(a);
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nv; i += stride) {
        f32x4 x = v[i];
        v[i] = x * alpha + beta;
    }
    for (uint64_t i = nv * 4 + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += stride)
        a[i] = a[i] * alpha + beta;
}

// Plain streams of known bytes: every workgroup moves tiles of 256 16-byte
// vectors, one per lane (4 KB), with non-temporal accesses (each byte
// touched once); the elements past the last whole tile go one per lane.
// Measured on MI355X over 1.2 GB, one tile per workgroup: a copy 6.43-6.58
// TB/s with one vector per lane against 5.80-5.90 with two (and 5.56 with
// eight), a read 6.95-7.01, a write 6.42-6.79.
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr uint64_t kStreamTile = 256;  // vectors per tile

__global__ __launch_bounds__(256) void stream_copy(const float *src, float *dst, uint64_t n) {
    const f32x4 *s = reinterpret_cast<const f32x4 *>(src);
    f32x4 *d = reinterpret_cast<f32x4 *>(dst);
    const uint64_t tiles = n / 4 / kStreamTile;
    for (uint64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const uint64_t i = t * kStreamTile + threadIdx.x;
        __builtin_nontemporal_store(__builtin_nontemporal_load(s + i), d + i);
    }
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = tiles * kStreamTile * 4 + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
         i < n; i += stride)
        dst[i] = src[i];
}

// Reads n floats; a lane writes its sum to sink[lane] only if it equals a
// value no input here produces (so the loads cannot be dropped).
__global__ __launch_bounds__(256) void stream_read(const float *src, uint64_t n, float *sink) {
    const f32x4 *s = reinterpret_cast<const f32x4 *>(src);
    const uint64_t tiles = n / 4 / kStreamTile;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (uint64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const uint64_t i = t * kStreamTile + threadIdx.x;
        acc += __builtin_nontemporal_load(s + i);
    }
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = tiles * kStreamTile * 4 + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
         i < n; i += stride)
        acc.x += src[i];
    if (acc.x + acc.y + acc.z + acc.w == -0x1.fffffep127f)
        sink[threadIdx.x] = acc.x;
}

__global__ __launch_bounds__(256) void stream_write(float *dst, uint64_t n, float value) {
    f32x4 *d = reinterpret_cast<f32x4 *>(dst);
    const f32x4 v = {value, value, value, value};
    const uint64_t tiles = n / 4 / kStreamTile;
    for (uint64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const uint64_t i = t * kStreamTile + threadIdx.x;
        __builtin_nontemporal_store(v, d + i);
    }
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = tiles * kStreamTile * 4 + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
         i < n; i += stride)
        dst[i] = value;
}

unsigned stream_grid(uint64_t n) {
    const uint64_t tiles = n / 4 / kStreamTile;
    return (unsigned)(tiles < 1 ? 1 : tiles < (1u << 20) ? tiles : (1u << 20));
}

}  // namespace

extern "C" {

// Elements [first, first+count) of rank `rank` into device memory dst
// (dtype 0 = binary32, 1 = binary16).  Returns a hipError_t.
int synth_fill_device(void *dst, int dtype, int dist, uint64_t seed, int rank, uint64_t first,
                      uint64_t count, double sigma, void *stream) {
    if (count == 0)
        return 0;
    if (!dst)
        return (int)hipErrorInvalidValue;
    const uint64_t key = mix64(seed + (uint64_t)(rank + 1) * kG);
    const double scale = sigma * 0x1p-33;
    const uint64_t blocks64 = (count + 255) / 256;
    const unsigned blocks = (unsigned)(blocks64 < 65536 ? blocks64 : 65536);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == 0)
        hipLaunchKernelGGL(fill_f32, dim3(blocks), dim3(256), 0, s, static_cast<float *>(dst),
                           dist, key, rank, first, count, scale);
    else
        hipLaunchKernelGGL(fill_f16, dim3(blocks), dim3(256), 0, s,
                           static_cast<_Float16 *>(dst), dist, key, rank, first, count, scale);
    return (int)hipGetLastError();
}

// In-place a = alpha * a + beta over n floats (a 16-byte aligned).
int synth_stream_compute(void *a, uint64_t n, float alpha, float beta, void *stream) {
    if (n == 0)
        return 0;
    if (!a || ((uintptr_t)a & 15))
        return (int)hipErrorInvalidValue;
    const uint64_t blocks64 = (n / 4 + 255) / 256;
    const unsigned blocks = (unsigned)(blocks64 < 8192 ? (blocks64 ? blocks64 : 1) : 8192);
    hipLaunchKernelGGL(stream_compute, dim3(blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<float *>(a), n, alpha,
                       beta);
    return (int)hipGetLastError();
}

// The plain streams (n floats, pointers 16-byte aligned): dst = src, a read
// of src (sink: 256 floats the kernel writes only in a case that does not
// arise), and dst = value.  Return a hipError_t.
int synth_stream_copy(const void *src, void *dst, uint64_t n, void *stream) {
    if (n == 0)
        return 0;
    if (!src || !dst || (((uintptr_t)src | (uintptr_t)dst) & 15))
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_copy, dim3(stream_grid(n)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const float *>(src),
                       static_cast<float *>(dst), n);
    return (int)hipGetLastError();
}

int synth_stream_read(const void *src, uint64_t n, void *sink, void *stream) {
    if (n == 0)
        return 0;
    if (!src || !sink || ((uintptr_t)src & 15))
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_read, dim3(stream_grid(n)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const float *>(src), n,
                       static_cast<float *>(sink));
    return (int)hipGetLastError();
}

int synth_stream_write(void *dst, uint64_t n, float value, void *stream) {
    if (n == 0)
        return 0;
    if (!dst || ((uintptr_t)dst & 15))
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_write, dim3(stream_grid(n)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<float *>(dst), n, value);
    return (int)hipGetLastError();
}

}  // extern "C"
