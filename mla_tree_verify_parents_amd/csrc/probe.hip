// Roofline probes (include/ddt_probe.h): a bf16 MFMA loop and streaming
// HBM read / copy kernels, so the achievable rates of the device are
// measured on the same run as the verify kernels.
#include "ddt_probe.h"

#include "common.h"

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kOps = 4;  // operand fragments per lane and operand
constexpr int kAcc = 4;  // independent accumulator chains per wavefront
static_assert(2 * kOps * 64 * 8 == DDT_PROBE_MFMA_OPERANDS, "operand buffer size");
static_assert(kOps * kAcc * 2 * 32 * 32 * 16 == DDT_PROBE_MFMA_FLOP_PER_WAVE_ITER, "flop per iteration");

// Every wavefront runs kAcc independent chains of 32x32x16 bf16 products;
// consecutive products take different operand fragments, so the multiplier
// inputs change from one product to the next as they do in a real kernel.
__global__ __launch_bounds__(DDT_PROBE_THREADS) void mfma_probe(const uint16_t* __restrict__ ops,
                                                                float* __restrict__ sink,
                                                                uint64_t* __restrict__ clk, int iters) {
    const int lane = threadIdx.x & 63;
    bf16x8 a[kOps], b[kOps];
#pragma unroll
    for (int k = 0; k < kOps; ++k) {
        a[k] = *reinterpret_cast<const bf16x8*>(ops + (k * 64 + lane) * 8);
        b[k] = *reinterpret_cast<const bf16x8*>(ops + ((kOps + k) * 64 + lane) * 8);
    }
    floatx16 acc[kAcc];
#pragma unroll
    for (int c = 0; c < kAcc; ++c) acc[c] = floatx16{};
    const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < kOps; ++k)
#pragma unroll
            for (int c = 0; c < kAcc; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[(k + c) % kOps], acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kAcc; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[c][e];
    const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    sink[(size_t)blockIdx.x * DDT_PROBE_THREADS + threadIdx.x] = s;
    if (clk != nullptr && threadIdx.x == 0) {
        clk[2 * (size_t)blockIdx.x] = c1 - c0;
        clk[2 * (size_t)blockIdx.x + 1] = r1 - r0;
    }
}

constexpr int kUnroll = 4;  // independent 16-byte loads in flight per thread

__global__ __launch_bounds__(DDT_PROBE_THREADS) void read_probe(const u32x4* __restrict__ src, size_t n,
                                                                uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * DDT_PROBE_THREADS;
    size_t i = (size_t)blockIdx.x * DDT_PROBE_THREADS + threadIdx.x;
    u32x4 f = {0u, 0u, 0u, 0u};
    for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) f ^= v[u];
    }
    for (; i < n; i += stride) f ^= __builtin_nontemporal_load(src + i);
    sink[(size_t)blockIdx.x * DDT_PROBE_THREADS + threadIdx.x] = f[0] ^ f[1] ^ f[2] ^ f[3];
}

__global__ __launch_bounds__(DDT_PROBE_THREADS) void copy_probe(const u32x4* __restrict__ src,
                                                                u32x4* __restrict__ dst, size_t n) {
    const size_t stride = (size_t)gridDim.x * DDT_PROBE_THREADS;
    size_t i = (size_t)blockIdx.x * DDT_PROBE_THREADS + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
    }
    for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

extern "C" int ddt_probe_mfma_bf16(const void* ops, float* sink, uint64_t* clk, int blocks, int iters,
                                   hipStream_t stream) {
    if (ops == nullptr || sink == nullptr || blocks <= 0 || iters <= 0) return DDT_EINVAL;
    if (!ddt::aligned(ops, 16) || !ddt::aligned(sink, 4) || (clk != nullptr && !ddt::aligned(clk, 8)))
        return DDT_EINVAL;
    hipLaunchKernelGGL(mfma_probe, dim3(blocks), dim3(DDT_PROBE_THREADS), 0, stream,
                       static_cast<const uint16_t*>(ops), sink, clk, iters);
    DDT_CHECK_LAUNCH();
    return DDT_OK;
}

extern "C" int ddt_probe_read(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t stream) {
    if (src == nullptr || sink == nullptr || blocks <= 0 || bytes == 0 || bytes % 16 != 0) return DDT_EINVAL;
    if (!ddt::aligned(src, 16) || !ddt::aligned(sink, 4)) return DDT_EINVAL;
    hipLaunchKernelGGL(read_probe, dim3(blocks), dim3(DDT_PROBE_THREADS), 0, stream,
                       static_cast<const u32x4*>(src), bytes / 16, sink);
    DDT_CHECK_LAUNCH();
    return DDT_OK;
}

extern "C" int ddt_probe_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t stream) {
    if (src == nullptr || dst == nullptr || blocks <= 0 || bytes == 0 || bytes % 16 != 0) return DDT_EINVAL;
    if (!ddt::aligned(src, 16) || !ddt::aligned(dst, 16)) return DDT_EINVAL;
    const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
    if (s < d + bytes && d < s + bytes) return DDT_EINVAL;  // overlapping ranges
    hipLaunchKernelGGL(copy_probe, dim3(blocks), dim3(DDT_PROBE_THREADS), 0, stream,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
    DDT_CHECK_LAUNCH();
    return DDT_OK;
}
