// ceilings.hip -- measured ceilings of the two resources the attention
// kernels are bound by, for the benchmark to print beside the spec-sheet
// peaks (libgqa_ceilings.so; not part of the attention interface):
//
//   int gqa_ceiling_read(const void* src, size_t bytes, uint32_t* sink,
//                        int blocks, void* stream)
//       streams `bytes` (a multiple of 16) of device memory at `src` with
//       16-byte non-temporal loads, the load form the decode kernels use for
//       K/V, each of `blocks` work-groups of 256 threads reading its own
//       contiguous range (as a decode split reads its keys);
//       each thread XOR-folds what it read into sink[thread] (device,
//       blocks * 256 words, so that the loads are not optimised away).
//   int gqa_ceiling_mfma(float* sink, int blocks, int iters, void* stream)
//       each wave of `blocks` work-groups of 256 threads issues iters * 4
//       v_mfma_f32_32x32x16_bf16 (32768 flops each) on four independent
//       accumulators held in registers, operands alternating between two
//       pseudo-random sets; sink[thread] (device, blocks * 256
//       floats) receives a sum of the accumulators.
//
// Both return 0, 2 for invalid sizes or a NULL pointer (checked before any
// launch) or 5 for a launch error; work is enqueued on `stream`.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ src, size_t n,
                                                        uint32_t* __restrict__ sink) {
    // work-group w streams its own contiguous range of ceil(n / groups)
    // 16-byte words, 4 KiB per wave instruction group, four loads in flight
    const size_t per = (n + gridDim.x - 1) / gridDim.x;
    const size_t beg = (size_t)blockIdx.x * per;
    const size_t end = beg + per < n ? beg + per : n;
    size_t i = beg + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * kThreads < end; i += 4 * kThreads) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        const u32x4 b = __builtin_nontemporal_load(src + i + kThreads);
        const u32x4 c = __builtin_nontemporal_load(src + i + 2 * kThreads);
        const u32x4 d = __builtin_nontemporal_load(src + i + 3 * kThreads);
        const u32x4 x = a ^ b ^ c ^ d;
        acc ^= x.x ^ x.y ^ x.z ^ x.w;
    }
    for (; i < end; i += kThreads) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kThreads) void mfma_kernel(float* __restrict__ sink, int iters) {
    const int tid = threadIdx.x;
    // two operand sets of pseudo-random values in [1, 2) with full mantissas,
    // alternated between MFMAs so the operand bits change at every issue (a
    // constant operand pair draws less power and runs at a higher clock than
    // attention's data does)
    bf16x8 a0, a1, b0, b1;
    uint32_t h = 0x9e3779b9u * (uint32_t)(blockIdx.x * kThreads + tid + 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        h ^= h << 13; h ^= h >> 17; h ^= h << 5;
        a0[i] = __builtin_bit_cast(__bf16, (uint16_t)(0x3f80 | (h & 0x7f)));
        a1[i] = __builtin_bit_cast(__bf16, (uint16_t)(0x3f80 | ((h >> 7) & 0x7f)));
        b0[i] = __builtin_bit_cast(__bf16, (uint16_t)(0xbf80 | ((h >> 14) & 0x7f)));
        b1[i] = __builtin_bit_cast(__bf16, (uint16_t)(0x3f80 | ((h >> 21) & 0x7f)));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    sink[(size_t)blockIdx.x * kThreads + tid] = s;
}

}  // namespace

extern "C" {

int gqa_ceiling_read(const void* src, size_t bytes, uint32_t* sink, int blocks, void* stream) {
    if (!src || !sink || blocks < 1 || bytes < 16 || bytes % 16 != 0) return 2;
    (void)hipGetLastError();
    hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                       (const u32x4*)src, bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

int gqa_ceiling_mfma(float* sink, int blocks, int iters, void* stream) {
    if (!sink || blocks < 1 || iters < 1) return 2;
    (void)hipGetLastError();
    hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream, sink,
                       iters);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
