// Ancestor mask of a draft tree ("The Architecture of Pragmatic Ambition",
// section "The Decision Architecture": tree verification differs from
// prefill only in the mask; a node sees its own ancestors inside the tree).
//
// One workgroup per request, O(N log 64 + N*W) work for any tree shape (a
// 1024-node chain -- a causal prefill chunk -- costs as little as a bushy
// tree).  The parent array is staged in LDS and checked, then:
//  1. Nodes are cut into blocks of 64 (the mask words).  One wavefront per
//     block finds, for each node i of the block, inblock[i] = the bits of
//     its ancestors-or-self inside the block and up[i] = its first ancestor
//     below the block (or -1), by pointer doubling across the wavefront:
//     lane l holds node 64w + l with the ancestor bits of the path segment
//     from i up to (excluding) its jump target J; a round ORs in the
//     segment of J and takes over J's jump, while J stays in the block.
//     Parents precede their children, so at most 63 in-block ancestors
//     exist and 6 rounds finish every lane.
//  2. Node i's word w is inblock[a] for the first ancestor-or-self a of i
//     inside block w, reached by following up[] (each jump leaves a block),
//     or 0 if the ancestry skips block w.  Depth = popcount of the row - 1.
#include "common.h"

namespace {

constexpr int kMaskThreads = 256;

__global__ __launch_bounds__(kMaskThreads) void mask_kernel(const int32_t* __restrict__ parents, int N,
                                                            int W, uint64_t* __restrict__ mask,
                                                            int32_t* __restrict__ depth,
                                                            int32_t* __restrict__ tree_err) {
    __shared__ int32_t spar[DDT_MAX_NODES];
    __shared__ uint64_t inblock[DDT_MAX_NODES];
    __shared__ int32_t up[DDT_MAX_NODES];
    __shared__ int s_bad;
    const int b = blockIdx.x;
    const int32_t* par = parents + (int64_t)b * N;
    if (threadIdx.x == 0) s_bad = 0;
    __syncthreads();
    int bad = 0;
    for (int i = threadIdx.x; i < N; i += blockDim.x) {
        const int p = par[i];
        spar[i] = p;
        bad |= (i == 0) ? (p != -1) : (p < 0 || p >= i);
    }
    if (bad) atomicOr(&s_bad, 1);
    __syncthreads();
    const bool ok = s_bad == 0;
    if (tree_err != nullptr && threadIdx.x == 0) tree_err[b] = ok ? 0 : 1;

    uint64_t* mrow = mask + (int64_t)b * N * W;
    if (!ok) {  // invalid tree: all-zero mask, depth -1
        for (int idx = threadIdx.x; idx < N * W; idx += blockDim.x) mrow[idx] = 0;
        if (depth != nullptr)
            for (int i = threadIdx.x; i < N; i += blockDim.x) depth[(int64_t)b * N + i] = -1;
        return;
    }

    // 1. per-block ancestor bits and the first ancestor below the block
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int w = wave; w < W; w += kMaskThreads / 64) {
        const int lo = 64 * w, i = lo + lane;
        const bool valid = i < N;
        uint64_t S = valid ? (1ull << lane) : 0ull;
        int J = valid ? spar[i] : -1;
#pragma unroll
        for (int round = 0; round < 6; ++round) {
            const bool inb = J >= lo;
            const int src = inb ? J - lo : lane;
            const uint64_t Ss = __shfl(S, src, 64);
            const int Js = __shfl(J, src, 64);
            if (inb) {
                S |= Ss;
                J = Js;
            }
        }
        if (valid) {
            inblock[i] = S;
            up[i] = J;
        }
    }
    __syncthreads();

    // 2. one node per thread: walk the block-level jumps, highest word first
    for (int i = threadIdx.x; i < N; i += blockDim.x) {
        uint64_t* row = mrow + (int64_t)i * W;
        int a = i, pop = 0;
        for (int w = W - 1; w >= 0; --w) {
            uint64_t bits = 0;
            if (a >= 0 && (a >> 6) == w) {
                bits = inblock[a];
                a = up[a];
            }
            pop += __popcll(bits);
            row[w] = bits;
        }
        if (depth != nullptr) depth[(int64_t)b * N + i] = pop - 1;
    }
}

}  // namespace

extern "C" int ddt_version(void) { return 100; }

extern "C" const char* ddt_status_string(int status) {
    switch (status) {
        case DDT_OK: return "DDT_OK";
        case DDT_EINVAL: return "DDT_EINVAL: invalid argument";
        case DDT_EUNSUPPORTED: return "DDT_EUNSUPPORTED: shape or dtype not built";
        case DDT_EWORKSPACE: return "DDT_EWORKSPACE: workspace missing or too small";
        case DDT_EHIP: return "DDT_EHIP: HIP runtime error";
        default: return "unknown ddt status";
    }
}

extern "C" int ddt_build_mask(const int32_t* parents, int B, int N, uint64_t* mask, int32_t* depth,
                              int32_t* tree_err, hipStream_t stream) {
    if (B < 0 || N < 1 || N > DDT_MAX_NODES) return DDT_EINVAL;
    if (B == 0) return DDT_OK;
    if (parents == nullptr || mask == nullptr) return DDT_EINVAL;
    const int W = (N + 63) / 64;
    hipLaunchKernelGGL(mask_kernel, dim3(B), dim3(kMaskThreads), 0, stream, parents, N, W, mask, depth,
                       tree_err);
    DDT_CHECK_LAUNCH();
    return DDT_OK;
}
