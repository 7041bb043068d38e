// Measured ceilings of one MI355X (gfx950), for reporting beside the
// published peaks: the bf16 matrix-core rate of a register-fed MFMA loop,
// the rate of a plain streaming read of HBM, and the shader clock.  These are
// measurement kernels for the benchmark, not part of the attention path.
//
//   attn_probe_mfma        every wave runs `iters` rounds of four independent
//                          v_mfma_f32_32x32x16_bf16 chains (32768 FLOP each)
//                          on register operands; 8 waves per workgroup (two
//                          per SIMD); writes one checksum per lane and the
//                          shader-clock / 100 MHz-clock cycles of each wave
//   attn_probe_mfma_random the same rate with operands of the attention
//                          workloads' kind: eight register sets of pseudo-
//                          random bf16 values (spread like N(0,1)), so both
//                          operands change on every MFMA.  The chip's power
//                          limit depends on the operand bits the matrix cores
//                          switch, so this rate and its clock are the
//                          ceiling that random bf16 data can reach
//   attn_probe_stream_read reads `bytes` (a multiple of 16 MiB) once with
//                          16-byte loads written straight to LDS (non-
//                          temporal), as the decode kernel streams its cache;
//                          one checksum word per workgroup
//   attn_probe_clock       one wave that samples the shader clock and the
//                          100 MHz reference clock `ticks` reference ticks
//                          apart (bounded spin), to read the clock while
//                          another kernel runs
//
// All pointers are device pointers owned by the caller; calls only enqueue
// on `stream` and return the hipError_t of the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_probe.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(512) void mfma_kernel(float* out, unsigned long long* cyc, int iters) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    f32x16 acc[4] = {};
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(1e-3f * (float)(lane + i));
        b[i] = (__bf16)(2e-3f * (float)i);
    }
    const unsigned long long t0 = __builtin_readcyclecounter();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
    }
    float s = 0.f;
    for (int k = 0; k < 4; ++k)
        for (int j = 0; j < 16; ++j) s += acc[k][j];
    const unsigned long long t1 = __builtin_readcyclecounter();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    out[(size_t)blockIdx.x * 512 + threadIdx.x] = s;
    if (lane == 0) {
        cyc[((size_t)blockIdx.x * 8 + wave) * 2] = t1 - t0;
        cyc[((size_t)blockIdx.x * 8 + wave) * 2 + 1] = r1 - r0;
    }
}

// Integer hash (xorshift-multiply) of the lane's operand index.
__device__ inline uint32_t hash32(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352dU;
    x ^= x >> 15;
    x *= 0x846ca68bU;
    x ^= x >> 16;
    return x;
}
// A value in (-2.4, 2.4) with a triangular density (sum of two uniforms):
// bf16 bit patterns like those of N(0,1) inputs.
__device__ inline __bf16 spread(uint32_t h) {
    const float u = (float)(h & 0xffffu) * (1.f / 65536.f) + (float)(h >> 16) * (1.f / 65536.f) - 1.f;
    return (__bf16)(2.4f * u);
}

__global__ __launch_bounds__(512) void mfma_random_kernel(float* out, unsigned long long* cyc, int iters) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    f32x16 acc[4] = {};
    bf16x8 a[8], b[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t h = hash32((uint32_t)(blockIdx.x * 4096u + threadIdx.x * 64u + r * 8u + i));
            a[r][i] = spread(h);
            b[r][i] = spread(hash32(h));
        }
    }
    const unsigned long long t0 = __builtin_readcyclecounter();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        // 32 MFMAs: chain k takes A set r and B set r + k, so consecutive
        // MFMAs never repeat an operand
#pragma unroll
        for (int r = 0; r < 8; ++r) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[r], b[(r + k) & 7], acc[k], 0, 0, 0);
        }
    }
    float s = 0.f;
    for (int k = 0; k < 4; ++k)
        for (int j = 0; j < 16; ++j) s += acc[k][j];
    const unsigned long long t1 = __builtin_readcyclecounter();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    out[(size_t)blockIdx.x * 512 + threadIdx.x] = s;
    if (lane == 0) {
        cyc[((size_t)blockIdx.x * 8 + wave) * 2] = t1 - t0;
        cyc[((size_t)blockIdx.x * 8 + wave) * 2 + 1] = r1 - r0;
    }
}

// Each workgroup (4 waves) reads one contiguous 16 MiB / gridDim slice in
// 4 KiB rounds (1 KiB per wave), 4 rounds in flight in a 16 KiB LDS ring.
constexpr int kStreamWaves = 4;
__global__ __launch_bounds__(64 * kStreamWaves) void stream_kernel(const unsigned char* src, size_t per_wg,
                                                                   unsigned* sink) {
    __shared__ __attribute__((aligned(1024))) unsigned char ring[4][kStreamWaves * 1024];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const unsigned char* base = src + (size_t)blockIdx.x * per_wg;
    const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(base), (short)0,
                                                     (int)per_wg, 0x00020000);
    const int rounds = (int)(per_wg / (kStreamWaves * 1024));
    for (int i = 0; i < rounds; ++i) {
        if (i >= 4) __builtin_amdgcn_s_waitcnt((3 & 15) | (7 << 4) | (15 << 8));  // vmcnt(3)
        const uint32_t off = (uint32_t)i * (kStreamWaves * 1024) + wave * 1024 + lane * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)&ring[i & 3][wave * 1024], 16, (int)off, 0, 0, 2);
    }
    __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));  // vmcnt(0)
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned x = 0;
        for (int i = 0; i < 4 * kStreamWaves * 1024; i += 4) x ^= *reinterpret_cast<const unsigned*>(&ring[0][0] + i);
        sink[blockIdx.x] = x;
    }
}

// One wave: shader cycles and reference ticks between two samples taken
// `ticks` reference ticks apart (the spin also stops after 2^26 rounds).
__global__ __launch_bounds__(64) void clock_kernel(unsigned long long* out, int ticks) {
    const unsigned long long t0 = __builtin_readcyclecounter();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    unsigned long long r1 = r0;
    for (int i = 0; i < (1 << 26) && r1 - r0 < (unsigned long long)ticks; ++i) {
        __builtin_amdgcn_s_sleep(2);
        r1 = __builtin_amdgcn_s_memrealtime();
    }
    const unsigned long long t1 = __builtin_readcyclecounter();
    if (threadIdx.x == 0) {
        out[0] = t1 - t0;
        out[1] = r1 - r0;
    }
}

}  // namespace

extern "C" {

int attn_probe_mfma(int n_wg, int iters, float* out, unsigned long long* cycles, void* stream) {
    if (n_wg <= 0 || iters <= 0 || !out || !cycles) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_kernel, dim3(n_wg), dim3(512), 0, static_cast<hipStream_t>(stream), out, cycles,
                       iters);
    return (int)hipGetLastError();
}

int attn_probe_mfma_random(int n_wg, int iters, float* out, unsigned long long* cycles, void* stream) {
    if (n_wg <= 0 || iters <= 0 || !out || !cycles) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_random_kernel, dim3(n_wg), dim3(512), 0, static_cast<hipStream_t>(stream), out,
                       cycles, iters);
    return (int)hipGetLastError();
}

int attn_probe_stream_read(const void* src, size_t bytes, unsigned* sink, int n_wg, void* stream) {
    const size_t per_wg = n_wg > 0 ? bytes / (size_t)n_wg : 0;
    if (!src || !sink || n_wg <= 0 || per_wg == 0 || per_wg % (16 * kStreamWaves * 1024) != 0 ||
        per_wg >= (1ull << 31) || per_wg * (size_t)n_wg != bytes)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_kernel, dim3(n_wg), dim3(64 * kStreamWaves), 0, static_cast<hipStream_t>(stream),
                       static_cast<const unsigned char*>(src), per_wg, sink);
    return (int)hipGetLastError();
}

int attn_probe_clock(unsigned long long* out, int ticks, void* stream) {
    if (!out || ticks <= 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(clock_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), out, ticks);
    return (int)hipGetLastError();
}

}  // extern "C"
