// Ancestor mask of a draft tree ("The Architecture of Pragmatic Ambition",
// section "The Decision Architecture": tree verification differs from
// prefill only in the mask; a node sees its own ancestors inside the tree).
//
// One workgroup per request.  The parent array is staged in LDS and checked;
// every (node, word) pair is then one work item that walks the parent links
// from the node towards the root.  Node numbers strictly decrease along the
// walk, so a walk for word w stops as soon as it drops below 64*w.
#include "common.h"

namespace {

constexpr int kMaskThreads = 256;

__global__ __launch_bounds__(kMaskThreads) void mask_kernel(const int32_t* __restrict__ parents, int N,
                                                            int W, uint64_t* __restrict__ mask,
                                                            int32_t* __restrict__ depth,
                                                            int32_t* __restrict__ tree_err) {
    __shared__ int32_t spar[DDT_MAX_NODES];
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
    for (int idx = threadIdx.x; idx < N * W; idx += blockDim.x) {
        const int i = idx / W, w = idx - (idx / W) * W;
        const int lo = w * 64;
        uint64_t bits = 0;
        if (ok) {
            for (int j = i; j >= lo; j = spar[j])
                if (j < lo + 64) bits |= 1ull << (j - lo);
        }
        mrow[idx] = bits;
    }
    if (depth != nullptr) {
        for (int i = threadIdx.x; i < N; i += blockDim.x) {
            int d = -1;
            if (ok) {
                d = 0;
                for (int j = i; spar[j] >= 0; j = spar[j]) ++d;
            }
            depth[(int64_t)b * N + i] = d;
        }
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
