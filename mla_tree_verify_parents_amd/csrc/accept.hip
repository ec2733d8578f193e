// Greedy tree acceptance ("The Architecture of Pragmatic Ambition", section
// "The Knowledge Architecture": walk the verified tree greedily for the
// longest path matching the target's predictions).
//
// One wavefront per request, the tree staged in LDS; the walk itself is
// ddt::greedy_walk (tree_tail.h).
#include "common.h"
#include "tree_tail.h"

namespace {

__global__ __launch_bounds__(ddt::kWave) void accept_kernel(const int32_t* __restrict__ target,
                                                            const int32_t* __restrict__ draft,
                                                            const int32_t* __restrict__ parents, int N,
                                                            int32_t* __restrict__ accept_len,
                                                            int32_t* __restrict__ path,
                                                            int32_t* __restrict__ tokens) {
    __shared__ int32_t spar[DDT_MAX_NODES];
    __shared__ int32_t sdraft[DDT_MAX_NODES];
    __shared__ int32_t spath[DDT_MAX_NODES];
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int64_t off = (int64_t)b * N;
    for (int i = lane; i < N; i += ddt::kWave) {
        spar[i] = parents[off + i];
        sdraft[i] = draft[off + i];
    }
    __syncthreads();
    const int n = ddt::greedy_walk(target, off, spar, sdraft, N, spath, lane);
    __syncthreads();
    ddt::write_accept(target, off, sdraft, spath, n, N, b, lane, accept_len, path, tokens);
}

}  // namespace

extern "C" int ddt_greedy_accept(const int32_t* target_ids, const int32_t* draft_ids, const int32_t* parents,
                                 int B, int N, int32_t* accept_len, int32_t* path, int32_t* tokens,
                                 hipStream_t stream) {
    if (B < 0 || N < 1 || N > DDT_MAX_NODES) return DDT_EINVAL;
    if (B == 0) return DDT_OK;
    if (!target_ids || !draft_ids || !parents || !accept_len || !path || !tokens) return DDT_EINVAL;
    hipLaunchKernelGGL(accept_kernel, dim3(B), dim3(ddt::kWave), 0, stream, target_ids, draft_ids, parents, N,
                       accept_len, path, tokens);
    DDT_CHECK_LAUNCH();
    return DDT_OK;
}
