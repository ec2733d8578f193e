// Target argmax building blocks ("The Architecture of Pragmatic Ambition",
// section "The Decision Architecture": greedy token selection), shared by
// the stand-alone argmax launch and the argmax workgroups that ride along
// in the attention launch.
//
// Each workgroup reduces a chunk of one row to a 64-bit key that orders
// values first and indices second:
//   key = order(value) << 32 | (0xffffffff - index)
// where order() maps fp32 bits to an unsigned integer with the same order
// as the values (NaN above +inf, -0 equal to +0).  The maximum key is the
// lowest index of the largest value.  A row cut into several chunks merges
// them through its slot in the workspace: a 64-bit atomic max, then a count;
// the row's last workgroup writes the index and clears the slot, so the
// workspace is zero again after every call.
#pragma once

#include "common.h"

namespace ddt {

constexpr int kArgThreads = 256;
constexpr int64_t kChunkAlign = 2048;  // elements, a multiple of 256 threads x 8 per load

__device__ inline uint32_t order_key(uint32_t u) {
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0xffffffffu;  // NaN: above every number
    if (u == 0x80000000u) u = 0;                              // -0 == +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline uint64_t pack_key(uint32_t bits, int64_t idx) {
    return ((uint64_t)order_key(bits) << 32) | (uint64_t)(0xffffffffu - (uint32_t)idx);
}

__device__ inline uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <typename T>
__device__ inline uint32_t f32_bits(T v);
template <>
__device__ inline uint32_t f32_bits<float>(float v) { return __float_as_uint(v); }
template <>
__device__ inline uint32_t f32_bits<uint16_t>(uint16_t v) { return (uint32_t)v << 16; }

// Reduce a chunk [c0, c1) of one row (this thread's share) to its key, the
// exact way: one key per element.  With kVec, VEC elements per 16-byte
// load and UNROLL independent loads in flight per thread.
template <typename T, bool kVec, int UNROLL>
__device__ uint64_t scan_chunk_exact(const T* __restrict__ row, int64_t c0, int64_t c1) {
    constexpr int VEC = 16 / sizeof(T);
    uint64_t best = 0;
    const int tid = threadIdx.x;
    if (kVec) {
        typedef uint32_t V4 __attribute__((ext_vector_type(4)));
        const int64_t nvec = (c1 - c0) / VEC;
        const V4* p = reinterpret_cast<const V4*>(row + c0);
        int64_t v = tid;
        for (; v + (UNROLL - 1) * kArgThreads < nvec; v += UNROLL * kArgThreads) {
            V4 x[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) x[u] = __builtin_nontemporal_load(p + v + u * kArgThreads);
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const T* e = reinterpret_cast<const T*>(&x[u]);
                const int64_t base = c0 + (v + u * kArgThreads) * VEC;
#pragma unroll
                for (int k = 0; k < VEC; ++k) best = umax64(best, pack_key(f32_bits<T>(e[k]), base + k));
            }
        }
        for (; v < nvec; v += kArgThreads) {
            V4 x = __builtin_nontemporal_load(p + v);
            const T* e = reinterpret_cast<const T*>(&x);
#pragma unroll
            for (int k = 0; k < VEC; ++k) best = umax64(best, pack_key(f32_bits<T>(e[k]), c0 + v * VEC + k));
        }
        for (int64_t i = c0 + nvec * VEC + tid; i < c1; i += kArgThreads)
            best = umax64(best, pack_key(f32_bits<T>(row[i]), i));
    } else {
        for (int64_t i = c0 + tid; i < c1; i += kArgThreads) best = umax64(best, pack_key(f32_bits<T>(row[i]), i));
    }
    return best;
}

// max(a, b, c) of floats without the NaN-quieting the compiler adds to
// fmaxf on values it cannot prove canonical (loaded data); NaN-free input.
__device__ inline float fmax3_raw(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

template <typename T>
__device__ inline float widen(T v);
template <>
__device__ inline float widen<float>(float v) { return v; }
template <>
__device__ inline float widen<uint16_t>(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// The same key, found cheaply (the VALU, not memory, limits a scan run by
// one wavefront per SIMD): per batch of UNROLL 16-byte loads the thread
// takes the float maximum (v_max3, half an operation per element) and only
// when it beats the running maximum searches the batch for the first
// element equal to it (ascending index order, so ties keep the lowest index
// and -0 == +0).  A running sum of the elements turns NaN if any element is
// NaN (or infinities of both signs meet); then the thread's share is
// scanned again the exact way, which also orders NaN above every number.
template <typename T, bool kVec, int UNROLL>
__device__ uint64_t scan_chunk(const T* __restrict__ row, int64_t c0, int64_t c1) {
    if (!kVec) return scan_chunk_exact<T, false, 1>(row, c0, c1);
    constexpr int VEC = 16 / sizeof(T);
    typedef uint32_t V4 __attribute__((ext_vector_type(4)));
    const int tid = threadIdx.x;
    const int64_t nvec = (c1 - c0) / VEC;
    const V4* p = reinterpret_cast<const V4*>(row + c0);
    float bv = -INFINITY;
    int64_t bi = -1;
    float probe = 0.f;
    int64_t v = tid;
    for (; v + (UNROLL - 1) * kArgThreads < nvec; v += UNROLL * kArgThreads) {
        V4 x[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) x[u] = __builtin_nontemporal_load(p + v + u * kArgThreads);
        float m = -INFINITY;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const T* e = reinterpret_cast<const T*>(&x[u]);
#pragma unroll
            for (int k = 0; k < VEC; k += 2) {
                const float a = widen<T>(e[k]), b2 = widen<T>(e[k + 1]);
                m = fmax3_raw(m, a, b2);
                probe += a + b2;
            }
        }
        if (m > bv || bi < 0) {  // (the first batch always records, -inf rows included)
            int64_t found = -1;
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const T* e = reinterpret_cast<const T*>(&x[u]);
#pragma unroll
                for (int k = 0; k < VEC; ++k)
                    if (found < 0 && widen<T>(e[k]) == m) found = c0 + (v + u * kArgThreads) * VEC + k;
            }
            bv = m;
            bi = found;
        }
    }
    uint64_t best = bi >= 0 ? pack_key(__float_as_uint(bv), bi) : 0;
    // the rest of the share (fewer than UNROLL loads) and the unaligned tail
    for (; v < nvec; v += kArgThreads) {
        V4 x = __builtin_nontemporal_load(p + v);
        const T* e = reinterpret_cast<const T*>(&x);
#pragma unroll
        for (int k = 0; k < VEC; ++k) best = umax64(best, pack_key(f32_bits<T>(e[k]), c0 + v * VEC + k));
    }
    for (int64_t i = c0 + nvec * VEC + tid; i < c1; i += kArgThreads)
        best = umax64(best, pack_key(f32_bits<T>(row[i]), i));
    if (probe != probe) best = scan_chunk_exact<T, true, 4>(row, c0, c1);  // NaN seen: exact rescan
    return best;
}

// Maximum over the workgroup (kArgThreads threads); valid in thread 0.
__device__ inline uint64_t block_max(uint64_t v) {
    __shared__ uint64_t red[kArgThreads / kWave];
    __syncthreads();  // a previous call's readers are done with red[]
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = umax64(v, __shfl_xor(v, o, kWave));
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kArgThreads / kWave; ++w) v = umax64(v, red[w]);
    }
    return v;
}

// Per-row merge slot of the workspace (zero between calls).
struct RowSlot {
    unsigned long long key;  // running maximum key of the row
    unsigned int done;       // chunks of the row folded in so far
    unsigned int pad;
};

// Thread 0 of the workgroup that reduced chunk c of row r (key `best`, row
// cut into nchunk chunks) records it; the row's last chunk writes idx[r].
__device__ inline void finish_chunk(uint64_t best, int64_t r, int nchunk, int32_t* __restrict__ idx,
                                    RowSlot* __restrict__ slots) {
    if (nchunk == 1) {
        idx[r] = (int32_t)(0xffffffffu - (uint32_t)best);
        return;
    }
    RowSlot* s = slots + r;
    // the max is performed (its old value has come back) before this chunk
    // counts itself in; no cache-wide fence is needed
    const unsigned long long prev = atomicMax(&s->key, (unsigned long long)best);
    asm volatile("s_waitcnt vmcnt(0)" ::"v"(prev) : "memory");
    if (atomicAdd(&s->done, 1u) == (unsigned)nchunk - 1) {
        // every other chunk of the row has folded its key in
        const unsigned long long k = atomicMax(&s->key, 0ull);
        idx[r] = (int32_t)(0xffffffffu - (uint32_t)k);
        atomicExch(&s->key, 0ull);
        atomicExch(&s->done, 0u);
    }
}

// Chunks per row for `wgs` workgroups over `rows` rows: chunks of at least
// 8192 elements, rounded to kChunkAlign.
inline void argmax_plan(int64_t rows, int64_t V, int64_t wgs, int* nchunk, int64_t* chunk) {
    int64_t want = rows >= wgs ? 1 : (wgs + rows - 1) / rows;
    int64_t maxc = (V + 8191) / 8192;
    int64_t n = want < maxc ? want : maxc;
    if (n < 1) n = 1;
    int64_t ch = (int64_t)round_up((size_t)((V + n - 1) / n), kChunkAlign);
    *chunk = ch;
    *nchunk = (int)((V + ch - 1) / ch);
}

}  // namespace ddt
