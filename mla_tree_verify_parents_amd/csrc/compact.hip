// KV compaction after acceptance ("The Architectural Keystone: Writing the
// Model Header ...", section "The Reasoning That Preceded the Header": the
// accepted path's latents, recomputed root included, are gathered into
// contiguous slots and the length advances; section "Mistakes and Iterative
// Refinement": source and destination slots alias).
//
// One workgroup per request.  Destination slot P+j receives source slot
// P+path[j].  The path starts at 0 and increases, so path[j] >= j: a copy
// never reads a row that an earlier copy (smaller j) wrote, and a row that a
// later copy reads lies above every destination written before it.  Copies
// are therefore done in blocks of increasing j, each block loaded whole into
// LDS before any of its rows is stored -- race free with no global scratch.
#include "common.h"

namespace {

constexpr int kCompThreads = 256;
constexpr int kStageBytes = 32768;

template <typename U>
__global__ __launch_bounds__(kCompThreads) void compact_kernel(char* __restrict__ ckv, int64_t ld_ckv,
                                                               char* __restrict__ kpe, int64_t ld_kpe,
                                                               int ckv_units, int kpe_units,
                                                               const int64_t* __restrict__ kv_base,
                                                               int32_t* __restrict__ prefix_len,
                                                               const int32_t* __restrict__ path,
                                                               const int32_t* __restrict__ accept_len,
                                                               int N, int32_t* __restrict__ src_slot,
                                                               int rows_per_block) {
    extern __shared__ uint4 stage_raw[];
    U* stage = reinterpret_cast<U*>(stage_raw);
    __shared__ int s_bad;
    const int b = blockIdx.x;
    const int64_t off = (int64_t)b * N;
    const int k = accept_len[b];
    const int64_t P = prefix_len[b];
    const int64_t base = kv_base[b];
    if (threadIdx.x == 0) s_bad = (k < 0 || k >= N) ? 1 : 0;
    __syncthreads();
    if (s_bad == 0) {
        int bad = 0;
        for (int j = threadIdx.x; j <= k; j += blockDim.x) {
            const int p = path[off + j];
            bad |= (j == 0) ? (p != 0) : (p <= path[off + j - 1] || p >= N);
        }
        if (bad) atomicOr(&s_bad, 1);
    }
    __syncthreads();
    const bool ok = s_bad == 0;
    if (src_slot != nullptr) {
        for (int j = threadIdx.x; j < N; j += blockDim.x)
            src_slot[off + j] = (ok && j <= k) ? (int32_t)(P + path[off + j]) : -1;
    }
    if (!ok) return;

    const int upr = ckv_units + kpe_units;  // U units per cache row
    for (int j0 = 0; j0 <= k; j0 += rows_per_block) {
        const int jn = (k + 1 - j0) < rows_per_block ? (k + 1 - j0) : rows_per_block;
        const int total = jn * upr;
        for (int u = threadIdx.x; u < total; u += blockDim.x) {
            const int j = j0 + u / upr, part = u % upr;
            const int src = path[off + j];
            if (src == j) continue;  // already in place
            const int64_t row = base + P + src;
            stage[u] = part < ckv_units
                           ? reinterpret_cast<const U*>(ckv + row * ld_ckv)[part]
                           : reinterpret_cast<const U*>(kpe + row * ld_kpe)[part - ckv_units];
        }
        __syncthreads();
        for (int u = threadIdx.x; u < total; u += blockDim.x) {
            const int j = j0 + u / upr, part = u % upr;
            if (path[off + j] == j) continue;
            const int64_t row = base + P + j;
            if (part < ckv_units)
                reinterpret_cast<U*>(ckv + row * ld_ckv)[part] = stage[u];
            else
                reinterpret_cast<U*>(kpe + row * ld_kpe)[part - ckv_units] = stage[u];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) prefix_len[b] = (int32_t)(P + k + 1);
}

}  // namespace

extern "C" int ddt_compact_kv(void* ckv, int64_t ld_ckv, void* kpe, int64_t ld_kpe, int dtype, int d_lat,
                              int d_rope, const int64_t* kv_base, int32_t* prefix_len, const int32_t* path,
                              const int32_t* accept_len, int B, int N, int32_t* src_slot, hipStream_t stream) {
    if (B < 0 || N < 1 || N > DDT_MAX_NODES || d_lat < 1 || d_rope < 0) return DDT_EINVAL;
    if (dtype != DDT_F32 && dtype != DDT_BF16) return DDT_EUNSUPPORTED;
    if (B == 0) return DDT_OK;
    if (!ckv || !kv_base || !prefix_len || !path || !accept_len) return DDT_EINVAL;
    if (d_rope > 0 && !kpe) return DDT_EINVAL;
    if (d_rope == 0) kpe = ckv;
    const int es = ddt::elem_bytes(dtype);
    const int64_t lc = ld_ckv * es, lk = ld_kpe * es;
    const int rc = d_lat * es, rk = d_rope * es;
    if (ld_ckv < d_lat || (d_rope > 0 && ld_kpe < d_rope)) return DDT_EINVAL;
    auto fits = [&](int a) {
        return ddt::aligned(ckv, a) && ddt::aligned(kpe, a) && lc % a == 0 && (d_rope == 0 || lk % a == 0) &&
               rc % a == 0 && rk % a == 0;
    };
    const int row_bytes = rc + rk;
    int rows_per_block = kStageBytes / row_bytes;
    if (rows_per_block < 1) return DDT_EUNSUPPORTED;
    if (rows_per_block > N) rows_per_block = N;
    const size_t shm = (size_t)rows_per_block * row_bytes;
    if (fits(16)) {
        hipLaunchKernelGGL(compact_kernel<uint4>, dim3(B), dim3(kCompThreads), shm, stream, (char*)ckv, lc,
                           (char*)kpe, lk, rc / 16, rk / 16, kv_base, prefix_len, path, accept_len, N, src_slot,
                           rows_per_block);
    } else if (fits(4)) {
        hipLaunchKernelGGL(compact_kernel<uint32_t>, dim3(B), dim3(kCompThreads), shm, stream, (char*)ckv, lc,
                           (char*)kpe, lk, rc / 4, rk / 4, kv_base, prefix_len, path, accept_len, N, src_slot,
                           rows_per_block);
    } else {
        return DDT_EINVAL;
    }
    DDT_CHECK_LAUNCH();
    return DDT_OK;
}
