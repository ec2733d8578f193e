// KV compaction after acceptance ("The Architectural Keystone: Writing the
// Model Header ...", section "The Reasoning That Preceded the Header": the
// accepted path's latents, recomputed root included, are gathered into
// contiguous slots and the length advances; section "Mistakes and Iterative
// Refinement": source and destination slots alias).
//
// One workgroup per request.  Destination slot P+j receives source slot
// P+path[j]; the path starts at 0 and increases, so path[j] >= j and the
// block-wise LDS-staged copy of ddt::copy_path_rows (tree_tail.h) is race
// free with no global scratch.  ddt_accept_compact runs acceptance and
// compaction of a request in one workgroup (ddt::accept_compact_body).
// ddt_compact_kv_paged maps slots to pool rows through a block table.
#include "common.h"
#include "tree_tail.h"

namespace {

template <typename U>
__global__ __launch_bounds__(ddt::kCompactThreads) void compact_kernel(
    char* __restrict__ ckv, int64_t ld_ckv, char* __restrict__ kpe, int64_t ld_kpe, int ckv_units, int kpe_units,
    const ddt::SlotMap map, int32_t* __restrict__ prefix_len, const int32_t* __restrict__ path,
    const int32_t* __restrict__ accept_len, int N, int32_t* __restrict__ src_slot, int rows_per_block) {
    extern __shared__ uint4 stage_raw[];
    __shared__ int s_bad;
    const int b = blockIdx.x;
    const int64_t off = (int64_t)b * N;
    const int k = accept_len[b];
    const int64_t P = prefix_len[b];
    if (threadIdx.x == 0) s_bad = (k < 0 || k >= N) ? 1 : 0;
    __syncthreads();
    if (s_bad == 0) {
        int bad = 0;
        for (int j = threadIdx.x; j <= k; j += blockDim.x) {
            const int p = path[off + j];
            bad |= (j == 0) ? (p != 0) : (p <= path[off + j - 1] || p >= N);
            // the path's last slot bounds every slot moved: it must be
            // mappable (P >= 0; paged: inside the request's table row)
            if (j == k) bad |= !map.covers(P, (int64_t)p + 1);
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
    ddt::copy_path_rows<U>(ckv, ld_ckv, kpe, ld_kpe, ckv_units, kpe_units, map, b, P, k, rows_per_block,
                           reinterpret_cast<U*>(stage_raw), [&](int j) { return path[off + j]; });
    if (threadIdx.x == 0) prefix_len[b] = (int32_t)(P + k + 1);
}

// Acceptance and compaction of one request per workgroup.
template <typename U>
__global__ __launch_bounds__(ddt::kCompactThreads) void accept_compact_kernel(const ddt::AcceptCompactArgs a) {
    extern __shared__ uint4 stage_raw[];
    ddt::accept_compact_body<U>(a, blockIdx.x, reinterpret_cast<U*>(stage_raw));
}

// The copy of ddt_compact_kv and ddt_compact_kv_paged after their checks.
int launch_compact(void* ckv, int64_t ld_ckv, void* kpe, int64_t ld_kpe, int dtype, int d_lat, int d_rope,
                   const ddt::SlotMap& map, int32_t* prefix_len, const int32_t* path, const int32_t* accept_len, int B,
                   int N, int32_t* src_slot, hipStream_t stream) {
    if (d_rope == 0) kpe = ckv;
    ddt::CompactLayout lay;
    const int rc = ddt::compact_layout(ckv, ld_ckv, kpe, ld_kpe, dtype, d_lat, d_rope, N, &lay);
    if (rc != DDT_OK) return rc;
    if (lay.vec16)
        hipLaunchKernelGGL(compact_kernel<uint4>, dim3(B), dim3(ddt::kCompactThreads), lay.stage_bytes, stream,
                           (char*)ckv, lay.lc, (char*)kpe, lay.lk, lay.ckv_units, lay.kpe_units, map, prefix_len, path,
                           accept_len, N, src_slot, lay.rows_per_block);
    else
        hipLaunchKernelGGL(compact_kernel<uint32_t>, dim3(B), dim3(ddt::kCompactThreads), lay.stage_bytes, stream,
                           (char*)ckv, lay.lc, (char*)kpe, lay.lk, lay.ckv_units, lay.kpe_units, map, prefix_len, path,
                           accept_len, N, src_slot, lay.rows_per_block);
    DDT_CHECK_LAUNCH();
    return DDT_OK;
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
    return launch_compact(ckv, ld_ckv, kpe, ld_kpe, dtype, d_lat, d_rope, ddt::SlotMap{kv_base, nullptr, 0, 0},
                          prefix_len, path, accept_len, B, N, src_slot, stream);
}

extern "C" int ddt_compact_kv_paged(void* ckv, int64_t ld_ckv, void* kpe, int64_t ld_kpe, int dtype, int d_lat,
                                    int d_rope, const int32_t* block_table, int64_t bt_ld, int page_size,
                                    int32_t* prefix_len, const int32_t* path, const int32_t* accept_len, int B, int N,
                                    int32_t* src_slot, hipStream_t stream) {
    if (B < 0 || N < 1 || N > DDT_MAX_NODES || d_lat < 1 || d_rope < 0) return DDT_EINVAL;
    if (dtype != DDT_F32 && dtype != DDT_BF16) return DDT_EUNSUPPORTED;
    if (page_size < 1 || page_size > (1 << 16) || (page_size & (page_size - 1)) != 0 || bt_ld < 1) return DDT_EINVAL;
    if (B == 0) return DDT_OK;
    if (!ckv || !block_table || !prefix_len || !path || !accept_len) return DDT_EINVAL;
    if (d_rope > 0 && !kpe) return DDT_EINVAL;
    return launch_compact(ckv, ld_ckv, kpe, ld_kpe, dtype, d_lat, d_rope,
                          ddt::SlotMap{nullptr, block_table, bt_ld, __builtin_ctz((unsigned)page_size)}, prefix_len,
                          path, accept_len, B, N, src_slot, stream);
}

// The launch of ddt_accept_compact and ddt_accept_compact_paged after their
// own argument checks (slots mapped by `map`).
int launch_accept_compact(const int32_t* target_ids, const int32_t* draft_ids, const int32_t* parents, int B, int N,
                          int32_t* accept_len, int32_t* path, int32_t* tokens, void* ckv, int64_t ld_ckv, void* kpe,
                          int64_t ld_kpe, int dtype, int d_lat, int d_rope, const ddt::SlotMap& map,
                          const int32_t* prefix_len, int32_t* new_prefix_len, int32_t* src_slot, hipStream_t stream) {
    if (!target_ids || !draft_ids || !parents || !accept_len || !path || !tokens) return DDT_EINVAL;
    if (!ckv || !prefix_len || !new_prefix_len) return DDT_EINVAL;
    if (d_rope > 0 && !kpe) return DDT_EINVAL;
    if (d_rope == 0) kpe = ckv;
    ddt::CompactLayout lay;
    const int rc = ddt::compact_layout(ckv, ld_ckv, kpe, ld_kpe, dtype, d_lat, d_rope, N, &lay);
    if (rc != DDT_OK) return rc;
    ddt::AcceptCompactArgs a{target_ids, draft_ids, parents, N, accept_len, path, tokens, (char*)ckv, (char*)kpe,
                             lay.lc, lay.lk, lay.ckv_units, lay.kpe_units, lay.rows_per_block,
                             map, prefix_len, new_prefix_len, src_slot};
    if (lay.vec16)
        hipLaunchKernelGGL(accept_compact_kernel<uint4>, dim3(B), dim3(ddt::kCompactThreads), lay.stage_bytes,
                           stream, a);
    else
        hipLaunchKernelGGL(accept_compact_kernel<uint32_t>, dim3(B), dim3(ddt::kCompactThreads), lay.stage_bytes,
                           stream, a);
    DDT_CHECK_LAUNCH();
    return DDT_OK;
}

extern "C" int ddt_accept_compact(const int32_t* target_ids, const int32_t* draft_ids, const int32_t* parents,
                                  int B, int N, int32_t* accept_len, int32_t* path, int32_t* tokens, void* ckv,
                                  int64_t ld_ckv, void* kpe, int64_t ld_kpe, int dtype, int d_lat, int d_rope,
                                  const int64_t* kv_base, const int32_t* prefix_len, int32_t* new_prefix_len,
                                  int32_t* src_slot, hipStream_t stream) {
    if (B < 0 || N < 1 || N > DDT_MAX_NODES || d_lat < 1 || d_rope < 0) return DDT_EINVAL;
    if (dtype != DDT_F32 && dtype != DDT_BF16) return DDT_EUNSUPPORTED;
    if (B == 0) return DDT_OK;
    if (!kv_base) return DDT_EINVAL;
    return launch_accept_compact(target_ids, draft_ids, parents, B, N, accept_len, path, tokens, ckv, ld_ckv, kpe,
                                 ld_kpe, dtype, d_lat, d_rope, ddt::SlotMap{kv_base, nullptr, 0, 0}, prefix_len,
                                 new_prefix_len, src_slot, stream);
}

extern "C" int ddt_accept_compact_paged(const int32_t* target_ids, const int32_t* draft_ids, const int32_t* parents,
                                        int B, int N, int32_t* accept_len, int32_t* path, int32_t* tokens, void* ckv,
                                        int64_t ld_ckv, void* kpe, int64_t ld_kpe, int dtype, int d_lat, int d_rope,
                                        const int32_t* block_table, int64_t bt_ld, int page_size,
                                        const int32_t* prefix_len, int32_t* new_prefix_len, int32_t* src_slot,
                                        hipStream_t stream) {
    if (B < 0 || N < 1 || N > DDT_MAX_NODES || d_lat < 1 || d_rope < 0) return DDT_EINVAL;
    if (dtype != DDT_F32 && dtype != DDT_BF16) return DDT_EUNSUPPORTED;
    if (page_size < 1 || page_size > (1 << 16) || (page_size & (page_size - 1)) != 0 || bt_ld < 1) return DDT_EINVAL;
    if (B == 0) return DDT_OK;
    if (!block_table) return DDT_EINVAL;
    return launch_accept_compact(target_ids, draft_ids, parents, B, N, accept_len, path, tokens, ckv, ld_ckv, kpe,
                                 ld_kpe, dtype, d_lat, d_rope,
                                 ddt::SlotMap{nullptr, block_table, bt_ld, __builtin_ctz((unsigned)page_size)},
                                 prefix_len, new_prefix_len, src_slot, stream);
}
