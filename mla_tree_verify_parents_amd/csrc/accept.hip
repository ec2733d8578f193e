// Greedy tree acceptance ("The Architecture of Pragmatic Ambition", section
// "The Knowledge Architecture": walk the verified tree greedily for the
// longest path matching the target's predictions).
//
// One wavefront per request.  The tree is staged in LDS; each step of the
// walk is a wavefront-wide search for the lowest-numbered child k > c of the
// current node c whose draft token equals the target token after c: 64
// candidate nodes are tested at once and the ballot's lowest set bit is the
// answer.  The current node strictly increases, so the walk ends after at
// most N steps even for a malformed tree.
#include "common.h"

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
    int c = 0, n = 1;
    if (lane == 0) spath[0] = 0;
    for (;;) {
        const int want = target[off + c];
        int next = -1;
        for (int base = c + 1; base < N; base += ddt::kWave) {
            const int k = base + lane;
            const bool hit = k < N && spar[k] == c && sdraft[k] == want;
            const uint64_t m = __ballot(hit);
            if (m != 0) {
                next = base + __builtin_ctzll(m);
                break;
            }
        }
        if (next < 0) break;
        c = next;
        if (lane == 0) spath[n] = c;
        ++n;
    }
    __syncthreads();
    const int bonus = target[off + c];
    for (int j = lane; j < N; j += ddt::kWave) {
        const int p = j < n ? spath[j] : -1;
        path[off + j] = p;
        int tok = -1;
        if (j + 1 < n) tok = sdraft[spath[j + 1]];
        else if (j + 1 == n) tok = bonus;
        tokens[off + j] = tok;
    }
    if (lane == 0) accept_len[b] = n - 1;
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
