// Microbenchmarks of the machine's own limits, measured beside the vendor's
// published peaks: HBM streaming (copy, read-only) and dense MFMA issue rate
// (bf16 16x16x32 and fp32 16x16x4), with the shader clock observed under the
// MFMA load. Built into a library of its own (libgdn_peaks.so); nothing on the
// GDN path calls it.
//
// Every entry point only enqueues one kernel on `stream` and returns 0, or a
// nonzero HIP error code if the launch fails. Buffers are the caller's device
// memory; sizes are in bytes.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Streaming in the decode step's pattern: each 512-thread workgroup moves one
// contiguous 64 KiB block, every thread issuing its eight 16-byte loads (lane
// order: consecutive lanes, consecutive addresses) before any store.
constexpr int kBlockWords = 4096;   // 16-byte words per workgroup (64 KiB)

// dst = src, one block per workgroup, non-temporal.
__global__ __launch_bounds__(512) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst) {
    const int64_t base = (int64_t)blockIdx.x * kBlockWords + threadIdx.x;
    u32x4 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = __builtin_nontemporal_load(&src[base + 512 * j]);
#pragma unroll
    for (int j = 0; j < 8; ++j) __builtin_nontemporal_store(x[j], &dst[base + 512 * j]);
}

// Reads whole blocks; the xor of everything a thread read is stored only if it
// equals a value it practically never takes, so no load can be dropped.
__global__ __launch_bounds__(512) void read_kernel(const u32x4* __restrict__ src, uint32_t* __restrict__ sink) {
    const int64_t base = (int64_t)blockIdx.x * kBlockWords + threadIdx.x;
    u32x4 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = __builtin_nontemporal_load(&src[base + 512 * j]);
    const u32x4 y = ((x[0] ^ x[1]) ^ (x[2] ^ x[3])) ^ ((x[4] ^ x[5]) ^ (x[6] ^ x[7]));
    const uint32_t r = y[0] ^ y[1] ^ y[2] ^ y[3];
    if (r == 0x9E3779B9u) sink[0] = r;
}

// Each wave issues `iters` rounds of 8 independent MFMAs. Lane 0 of every wave
// records the shader-clock ticks and the 100 MHz real-time ticks it spent, so
// the host can take the clock the MFMA pipes actually ran at.
template <bool BF16>
__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* __restrict__ sink, uint64_t* __restrict__ ticks) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float fa = 1e-3f * (float)lane, fb = 1e-3f * (float)(63 - lane);
    const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    if constexpr (BF16) {
        bf16x8 a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = (__bf16)(fa + 1e-4f * (float)i);
            b[i] = (__bf16)(fb - 1e-4f * (float)i);
        }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
        }
    } else {
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa, fb, acc[j], 0, 0, 0);
        }
    }
    const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    f32x4 s = acc[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) s += acc[j];
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
    if (lane == 0) {
        ticks[2 * wave] = c1 - c0;
        ticks[2 * wave + 1] = r1 - r0;
    }
}

int launched(hipError_t e) { return e == hipSuccess ? 0 : (int)e; }

}  // namespace

extern "C" {

// Copies `bytes` (a multiple of 64 KiB) from src to dst (no overlap).
int peaks_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    if (bytes <= 0 || bytes % (16 * kBlockWords) != 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)(bytes / (16 * kBlockWords))), dim3(512), 0, (hipStream_t)stream,
                       (const u32x4*)src, (u32x4*)dst);
    return launched(hipGetLastError());
}

// Reads `bytes` (a multiple of 64 KiB) from src; sink: one uint32 of device memory.
int peaks_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
    if (bytes <= 0 || bytes % (16 * kBlockWords) != 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(read_kernel, dim3((unsigned)(bytes / (16 * kBlockWords))), dim3(512), 0, (hipStream_t)stream,
                       (const u32x4*)src, sink);
    return launched(hipGetLastError());
}

// `blocks` workgroups of 4 waves, each wave 8 x iters MFMAs (bf16: 16x16x32,
// 16,384 flop each; fp32: 16x16x4, 2,048 flop each). sink: blocks x 256 floats;
// ticks: 2 uint64 per wave (shader-clock ticks, 100 MHz real-time ticks).
int peaks_mfma(int bf16, int blocks, int iters, float* sink, uint64_t* ticks, void* stream) {
    if (bf16)
        hipLaunchKernelGGL(mfma_kernel<true>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, sink, ticks);
    else
        hipLaunchKernelGGL(mfma_kernel<false>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, sink, ticks);
    return launched(hipGetLastError());
}

}  // extern "C"
