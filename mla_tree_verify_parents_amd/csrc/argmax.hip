// Target argmax over logits rows ("The Architecture of Pragmatic Ambition",
// section "The Decision Architecture": greedy token selection).
//
// An HBM scan: each row is cut into chunks so that the launch has enough
// workgroups to keep every XCD's memory pipes busy; each workgroup streams
// its chunk with 16-byte loads and reduces a 64-bit key that orders values
// first and indices second:
//   key = order(value) << 32 | (0xffffffff - index)
// where order() maps fp32 bits to an unsigned integer with the same order
// as the values (NaN above +inf, -0 equal to +0).  The maximum key is the
// lowest index of the largest value.  With several chunks per row each
// workgroup folds its key into the row's slot of the workspace with a 64-bit
// atomic max and counts itself in; the row's last workgroup writes the index
// and clears the slot, so one launch does the whole reduction and leaves the
// workspace zeroed for the next call.
#include "common.h"

namespace {

constexpr int kArgThreads = 256;
constexpr int64_t kChunkAlign = 2048;  // elements, a multiple of 256 threads x 8 per load

__device__ inline uint32_t order_key(uint32_t u) {
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0xffffffffu;  // NaN: above every number
    if (u == 0x80000000u) u = 0;                              // -0 == +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline uint64_t pack(uint32_t bits, int64_t idx) {
    return ((uint64_t)order_key(bits) << 32) | (uint64_t)(0xffffffffu - (uint32_t)idx);
}

__device__ inline uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <typename T>
__device__ inline uint32_t f32_bits(T v);
template <>
__device__ inline uint32_t f32_bits<float>(float v) { return __float_as_uint(v); }
template <>
__device__ inline uint32_t f32_bits<uint16_t>(uint16_t v) { return (uint32_t)v << 16; }

// Reduce a chunk [c0, c1) of one row.  VEC elements per 16-byte load when
// `vec` holds, scalar loads otherwise.
template <typename T, bool kVec>
__device__ uint64_t scan_chunk(const T* __restrict__ row, int64_t c0, int64_t c1) {
    constexpr int VEC = 16 / sizeof(T);
    uint64_t best = 0;
    const int tid = threadIdx.x;
    if (kVec) {
        typedef uint32_t V4 __attribute__((ext_vector_type(4)));
        const int64_t nvec = (c1 - c0) / VEC;
        const V4* p = reinterpret_cast<const V4*>(row + c0);
        int64_t v = tid;
        // four independent 16-byte loads in flight per thread
        for (; v + 3 * kArgThreads < nvec; v += 4 * kArgThreads) {
            V4 x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) x[u] = __builtin_nontemporal_load(p + v + u * kArgThreads);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const T* e = reinterpret_cast<const T*>(&x[u]);
                const int64_t base = c0 + (v + u * kArgThreads) * VEC;
#pragma unroll
                for (int k = 0; k < VEC; ++k) best = umax64(best, pack(f32_bits<T>(e[k]), base + k));
            }
        }
        for (; v < nvec; v += kArgThreads) {
            V4 x = __builtin_nontemporal_load(p + v);
            const T* e = reinterpret_cast<const T*>(&x);
#pragma unroll
            for (int k = 0; k < VEC; ++k) best = umax64(best, pack(f32_bits<T>(e[k]), c0 + v * VEC + k));
        }
        for (int64_t i = c0 + nvec * VEC + tid; i < c1; i += kArgThreads)
            best = umax64(best, pack(f32_bits<T>(row[i]), i));
    } else {
        for (int64_t i = c0 + tid; i < c1; i += kArgThreads) best = umax64(best, pack(f32_bits<T>(row[i]), i));
    }
    return best;
}

__device__ inline uint64_t block_max(uint64_t v) {
    __shared__ uint64_t red[kArgThreads / ddt::kWave];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = umax64(v, __shfl_xor(v, o, ddt::kWave));
    const int wave = threadIdx.x / ddt::kWave;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kArgThreads / ddt::kWave; ++w) v = umax64(v, red[w]);
    }
    return v;  // valid in thread 0
}

// Per-row merge slot of the workspace (zero between calls).
struct RowSlot {
    unsigned long long key;  // running maximum key of the row
    unsigned int done;       // workgroups of the row that have folded their key in
    unsigned int pad;
};

template <typename T, bool kVec>
__global__ __launch_bounds__(kArgThreads) void argmax_chunks(const T* __restrict__ logits, int64_t V,
                                                             int64_t ld, int nchunk, int64_t chunk,
                                                             int32_t* __restrict__ idx, RowSlot* __restrict__ slots) {
    const int64_t r = blockIdx.x / nchunk;
    const int c = blockIdx.x - (int)(r * nchunk);
    const int64_t c0 = (int64_t)c * chunk;
    const int64_t c1 = c0 + chunk < V ? c0 + chunk : V;
    uint64_t best = scan_chunk<T, kVec>(logits + r * ld, c0, c1);
    best = block_max(best);
    if (threadIdx.x == 0) {
        if (nchunk == 1) {
            idx[r] = (int32_t)(0xffffffffu - (uint32_t)best);
        } else {
            RowSlot* s = slots + r;
            // the max is performed (its old value has come back) before this
            // workgroup counts itself in; no cache-wide fence is needed
            const unsigned long long prev = atomicMax(&s->key, (unsigned long long)best);
            asm volatile("s_waitcnt vmcnt(0)" :: "v"(prev) : "memory");
            if (atomicAdd(&s->done, 1u) == (unsigned)nchunk - 1) {
                // every other workgroup of the row has folded its key in
                const unsigned long long k = atomicMax(&s->key, 0ull);
                idx[r] = (int32_t)(0xffffffffu - (uint32_t)k);
                atomicExch(&s->key, 0ull);
                atomicExch(&s->done, 0u);
            }
        }
    }
}

// Chunks per row: enough rows x chunks to give ~2048 workgroups, chunks of at
// least 8192 elements.
void plan(int64_t rows, int64_t V, int* nchunk, int64_t* chunk) {
    int64_t want = rows >= 2048 ? 1 : (2048 + rows - 1) / rows;
    int64_t maxc = (V + 8191) / 8192;
    int64_t n = want < maxc ? want : maxc;
    if (n < 1) n = 1;
    int64_t ch = (int64_t)ddt::round_up((size_t)((V + n - 1) / n), kChunkAlign);
    *chunk = ch;
    *nchunk = (int)((V + ch - 1) / ch);
}

template <typename T>
int launch(const void* logits, int64_t rows, int64_t V, int64_t ld, int32_t* idx, void* ws,
           hipStream_t stream) {
    int nchunk;
    int64_t chunk;
    plan(rows, V, &nchunk, &chunk);
    const bool vec = ddt::aligned(logits, 16) && ((ld * (int64_t)sizeof(T)) % 16 == 0);
    const dim3 grid((unsigned)(rows * nchunk));
    auto* slots = static_cast<RowSlot*>(ws);
    if (vec)
        hipLaunchKernelGGL((argmax_chunks<T, true>), grid, dim3(kArgThreads), 0, stream,
                           static_cast<const T*>(logits), V, ld, nchunk, chunk, idx, slots);
    else
        hipLaunchKernelGGL((argmax_chunks<T, false>), grid, dim3(kArgThreads), 0, stream,
                           static_cast<const T*>(logits), V, ld, nchunk, chunk, idx, slots);
    DDT_CHECK_LAUNCH();
    return DDT_OK;
}

}  // namespace

extern "C" int ddt_argmax_workspace(int64_t rows, int64_t V, size_t* bytes) {
    if (bytes == nullptr || rows < 0 || V < 1 || V > 0x7fffffff) return DDT_EINVAL;
    int nchunk;
    int64_t chunk;
    plan(rows > 0 ? rows : 1, V, &nchunk, &chunk);
    *bytes = nchunk > 1 ? (size_t)rows * sizeof(RowSlot) : 0;
    return DDT_OK;
}

extern "C" int ddt_argmax(const void* logits, int dtype, int64_t rows, int64_t V, int64_t ld, int32_t* idx,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (rows < 0 || V < 1 || V > 0x7fffffff || ld < V) return DDT_EINVAL;
    if (dtype != DDT_F32 && dtype != DDT_BF16) return DDT_EUNSUPPORTED;
    if (rows == 0) return DDT_OK;
    if (logits == nullptr || idx == nullptr) return DDT_EINVAL;
    if (rows > 0x7fffffff / 64) return DDT_EINVAL;
    size_t need = 0;
    ddt_argmax_workspace(rows, V, &need);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need || !ddt::aligned(workspace, 16)))
        return DDT_EWORKSPACE;
    int nchunk;
    int64_t chunk;
    plan(rows, V, &nchunk, &chunk);
    if (rows * (int64_t)nchunk > 0x7fffffff) return DDT_EINVAL;
    return dtype == DDT_F32 ? launch<float>(logits, rows, V, ld, idx, workspace, stream)
                            : launch<uint16_t>(logits, rows, V, ld, idx, workspace, stream);
}
