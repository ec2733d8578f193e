// Target argmax over logits rows ("The Architecture of Pragmatic Ambition",
// section "The Decision Architecture": greedy token selection).
//
// An HBM scan: each row is cut into chunks so that the launch has enough
// workgroups to keep every XCD's memory pipes busy; the key encoding and the
// in-workspace merge of a row's chunks are in argmax_scan.h.
#include "argmax_scan.h"

namespace {

using ddt::kArgThreads;

template <typename T, bool kVec>
__global__ __launch_bounds__(kArgThreads) void argmax_chunks(const T* __restrict__ logits, int64_t V,
                                                             int64_t ld, int nchunk, int64_t chunk,
                                                             int32_t* __restrict__ idx,
                                                             ddt::RowSlot* __restrict__ slots) {
    const int64_t r = blockIdx.x / nchunk;
    const int c = blockIdx.x - (int)(r * nchunk);
    const int64_t c0 = (int64_t)c * chunk;
    const int64_t c1 = c0 + chunk < V ? c0 + chunk : V;
    uint64_t best = ddt::scan_chunk<T, kVec, 4>(logits + r * ld, c0, c1);
    best = ddt::block_max(best);
    if (threadIdx.x == 0) ddt::finish_chunk(best, r, nchunk, idx, slots);
}

// Chunks per row: enough rows x chunks to give ~2048 workgroups.
void plan(int64_t rows, int64_t V, int* nchunk, int64_t* chunk) { ddt::argmax_plan(rows, V, 2048, nchunk, chunk); }

template <typename T>
int launch(const void* logits, int64_t rows, int64_t V, int64_t ld, int32_t* idx, void* ws,
           hipStream_t stream) {
    int nchunk;
    int64_t chunk;
    plan(rows, V, &nchunk, &chunk);
    const bool vec = ddt::aligned(logits, 16) && ((ld * (int64_t)sizeof(T)) % 16 == 0);
    const dim3 grid((unsigned)(rows * nchunk));
    auto* slots = static_cast<ddt::RowSlot*>(ws);
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
    *bytes = nchunk > 1 ? (size_t)rows * sizeof(ddt::RowSlot) : 0;
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
