// Per-head projections around the absorbed attention, gfx950.
//
// What is computed ("The Architecture of Pragmatic Ambition", section "The
// Thinking Process: A Window into Engineering Deliberation": W_UK is
// absorbed into the query, q_lat[h] = q_nope[h] @ W_UK[h]; section "The
// Output Knowledge: What This Message Creates": every projection is
// y = x @ W with W stored [in, out], and the absorbed parameters w_kc, w_vc
// are given directly).  For every row r = t*H + h (token-major, head-minor:
// the query row order of the attention):
//   y[r][n] = sum_k x[r][k] * W[h][k][n]
// The two uses: q_lat = q_nope @ w_kc[h] (K = d_nope, n_out = d_lat) before
// the attention, and o = out_lat @ w_vc[h] (K = d_lat, n_out = d_v) after it.
//
// How (MI355X-first): at K2 shapes a (token, head) row moves 1280 bytes for
// 131 kflop, about 100 flop/B, under the ridge of the chip: the kernel is an
// HBM stream whose products must run on the matrix cores to stay one.
//  * The weights are static, so they are packed once (ddt_proj_pack_weight)
//    into the B-operand order of MFMA 32x32x16 bf16: fragment (h, column
//    tile of 32, k-step of 16) is 64 lanes x 16 bytes, lane l holding
//    W[h][16 ks + 8 (l/32) + e][32 nb + l%32], e = 0..7.  Each B load of a
//    wavefront is then 1 KB contiguous.
//  * A workgroup owns 64 rows of one head (tokens t0..t0+63) and 128 output
//    columns.  The 64 x K input tile goes to LDS once (16-byte loads, rows
//    padded by 16 bytes so the fragment reads of 32 consecutive rows hit
//    distinct bank groups); each of the 4 wavefronts multiplies it by its
//    own 32 columns with two accumulators (rows 0-31 and 32-63).
//  * The fp32 results are rounded to bf16 (round to nearest even) into an
//    LDS tile and written back as 16-byte stores along the output rows.
//  * Logical workgroups run column block fastest, then token tile, then
//    head, each XCD taking a contiguous range (xcd_logical_block): the
//    column blocks of an input tile share its L2 copy, and a head's weights
//    stay in the L2 of the XCDs that run it.
//  * Few rows (a grid of fewer workgroups than CUs, e.g. one verify step's
//    64 tree nodes): the reduction is split instead.  A workgroup owns 64
//    rows x 32 columns of one head; each wavefront takes a quarter of the
//    k-steps with its A fragments loaded straight from the rows (16
//    contiguous bytes per lane), and the four partial tiles are summed
//    through LDS -- 4x (n_out/128 x more) workgroups, a quarter of the
//    dependent MFMA chain each.
#include "common.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 64;    // rows (tokens of one head) per workgroup
constexpr int kCols = 128;   // output columns per workgroup (32 per wavefront)
constexpr int kThreads = 256;
constexpr int kMaxK = 512;

__device__ inline uint16_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

// One thread per packed fragment lane: 16 bytes out, 8 strided reads in.
__global__ __launch_bounds__(256) void proj_pack_kernel(const uint16_t* __restrict__ w, int H, int K, int n_out,
                                                        u32x4* __restrict__ wp) {
    const int64_t total = (int64_t)H * (n_out / 32) * (K / 16) * 64;
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= total) return;
    const int lane = (int)(g & 63);
    int64_t f = g >> 6;
    const int ks = (int)(f % (K / 16));
    f /= K / 16;
    const int nb = (int)(f % (n_out / 32));
    const int h = (int)(f / (n_out / 32));
    const int n = 32 * nb + (lane & 31);
    const int k0 = 16 * ks + 8 * (lane >> 5);
    const uint16_t* src = w + ((int64_t)h * K + k0) * n_out + n;
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = src[(int64_t)e * n_out];
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (uint32_t)v[2 * e] | ((uint32_t)v[2 * e + 1] << 16);
    wp[g] = o;
}

template <int K>
__global__ __launch_bounds__(kThreads) void proj_kernel(const uint16_t* __restrict__ x, int64_t ld_x,
                                                        const bf16x8* __restrict__ wp, int M, int H, int n_out,
                                                        uint16_t* __restrict__ y, int64_t ld_y, int n_tt, int n_cb) {
    static_assert(K % 16 == 0 && K <= kMaxK, "reduction depth: whole k-steps of 16, at most 512");
    constexpr int KS = K / 16;                 // MFMA k-steps
    constexpr int XCH = K / 8;                 // 16-byte chunks per input row
    constexpr int XROW = K * 2 + 16;           // padded LDS row of the input tile (bytes)
    constexpr int YROW = kCols * 2 + 16;       // padded LDS row of the output tile (bytes)
    constexpr int LDS = (kRows * XROW > kRows * YROW) ? kRows * XROW : kRows * YROW;
    __shared__ __attribute__((aligned(16))) unsigned char smem[LDS];

    const int nblocks = H * n_cb * n_tt;
    const int wg = ddt::xcd_logical_block(blockIdx.x, nblocks);
    const int cb = wg % n_cb;                  // the column blocks of one input tile run together
    const int tt = (wg / n_cb) % n_tt;
    const int h = wg / (n_tt * n_cb);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t0 = tt * kRows;

    // the B fragments of the first KP k-steps load before the input tile, so
    // their (L2) latency overlaps the tile's.  The deepest reduction (K =
    // 512: 64 KB of input per workgroup, two workgroups per CU) prefetches
    // every fragment and puts all of a thread's tile loads in flight before
    // its first LDS write: measured 13.3 -> 11.6 us at 512 tokens x 64 heads
    // and 7.3 -> 6.3 us at 2048 x 8.  At K = 128 the same took more
    // registers and fewer workgroups per CU, 3 % slower, so the shallower
    // reductions keep eight fragments ahead and put a thread's tile loads
    // in flight two at a time (12.6 -> 11.4 us at K = 128 against one at a
    // time, with no more registers).
    constexpr bool kBurst = K >= 512;
    const int nb = cb * (kCols / 32) + wave;  // this wavefront's 32-column tile
    const bool has_cols = nb * 32 < n_out;
    const bf16x8* wf = wp + ((int64_t)(h * (n_out / 32) + (has_cols ? nb : 0)) * KS) * 64 + lane;
    constexpr int KP = kBurst ? KS : (KS < 8 ? KS : 8);
    bf16x8 bpre[KP];
#pragma unroll
    for (int ks = 0; ks < KP; ++ks) bpre[ks] = wf[ks * 64];
    // input tile: rows t0..t0+63 of head h, zero past M
    if constexpr (kBurst) {
        constexpr int XU = kRows * XCH / kThreads;  // 16-byte chunks per thread
        static_assert((kRows * XCH) % kThreads == 0, "whole chunks per thread");
        u32x4 xv[XU];
#pragma unroll
        for (int u = 0; u < XU; ++u) {
            const int c = tid + u * kThreads, row = c / XCH, ch = c % XCH;
            const int t = t0 + row;
            xv[u] = u32x4{0u, 0u, 0u, 0u};
            if (t < M) xv[u] = *reinterpret_cast<const u32x4*>(x + ((int64_t)t * H + h) * ld_x + ch * 8);
        }
#pragma unroll
        for (int u = 0; u < XU; ++u) {
            const int c = tid + u * kThreads, row = c / XCH, ch = c % XCH;
            *reinterpret_cast<u32x4*>(smem + row * XROW + ch * 16) = xv[u];
        }
    } else {
        constexpr int XU = kRows * XCH / kThreads;
        constexpr int XB = XU >= 2 ? 2 : 1;  // loads in flight per batch
#pragma unroll
        for (int u0 = 0; u0 < XU; u0 += XB) {
            u32x4 xv[XB];
#pragma unroll
            for (int u = 0; u < XB; ++u) {
                const int c = tid + (u0 + u) * kThreads, row = c / XCH, ch = c % XCH;
                const int t = t0 + row;
                xv[u] = u32x4{0u, 0u, 0u, 0u};
                if (t < M) xv[u] = *reinterpret_cast<const u32x4*>(x + ((int64_t)t * H + h) * ld_x + ch * 8);
            }
#pragma unroll
            for (int u = 0; u < XB; ++u) {
                const int c = tid + (u0 + u) * kThreads, row = c / XCH, ch = c % XCH;
                *reinterpret_cast<u32x4*>(smem + row * XROW + ch * 16) = xv[u];
            }
        }
    }
    __syncthreads();

    floatx16 acc0 = {}, acc1 = {};
    if (has_cols) {
        const unsigned char* a0p = smem + (lane & 31) * XROW + (lane >> 5) * 16;
        const unsigned char* a1p = a0p + 32 * XROW;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 b = ks < KP ? bpre[ks < KP ? ks : 0] : wf[ks * 64];
            const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(a0p + ks * 32);
            const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(a1p + ks * 32);
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b, acc1, 0, 0, 0);
        }
    }
    __syncthreads();  // the input tile is dead; its LDS becomes the output tile

    // C[i][j] of a 32x32 product sits in lane j + 32*((i/4)%2), register
    // 4*(i/8) + i%4; here i = row (token) and j = column
    {
        unsigned char* col = smem + (wave * 32 + (lane & 31)) * 2;
        const int g = lane >> 5;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 8 * (r >> 2) + 4 * g + (r & 3);
            *reinterpret_cast<uint16_t*>(col + i * YROW) = bf16_bits(acc0[r]);
            *reinterpret_cast<uint16_t*>(col + (32 + i) * YROW) = bf16_bits(acc1[r]);
        }
    }
    __syncthreads();

    const int cols = min(kCols, n_out - cb * kCols);  // a multiple of 32
    const int och = cols / 8;
    for (int c = tid; c < kRows * (kCols / 8); c += kThreads) {
        const int row = c / (kCols / 8), ch = c % (kCols / 8);
        const int t = t0 + row;
        if (t >= M || ch >= och) continue;
        *reinterpret_cast<u32x4*>(y + ((int64_t)t * H + h) * ld_y + cb * kCols + ch * 8) =
            *reinterpret_cast<const u32x4*>(smem + row * YROW + ch * 16);
    }
}

template <int K>
__global__ __launch_bounds__(kThreads) void proj_splitk_kernel(const uint16_t* __restrict__ x, int64_t ld_x,
                                                               const bf16x8* __restrict__ wp, int M, int H,
                                                               int n_out, uint16_t* __restrict__ y, int64_t ld_y,
                                                               int n_tt, int n_nb) {
    static_assert(K % 64 == 0 && K <= kMaxK, "reduction depth: four equal shares of whole k-steps");
    constexpr int KS = K / 16, KQ = KS / 4;    // k-steps, and each wavefront's share
    constexpr int PROW = 32 * 4 + 4;           // padded LDS row of a partial tile (bytes: 32 fp32 + 4)
    __shared__ __attribute__((aligned(16))) float part[4][kRows * PROW / 4 + 4];

    const int nblocks = H * n_nb * n_tt;
    const int wg = ddt::xcd_logical_block(blockIdx.x, nblocks);
    const int tt = wg % n_tt;
    const int nb = (wg / n_tt) % n_nb;         // 32-column tile
    const int h = wg / (n_tt * n_nb);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t0 = tt * kRows;

    // A fragment of row group rg, k-step ks: row t0 + 32 rg + lane%32, k = 16 ks + 8 (lane/32) .. +8
    const bf16x8* wf = wp + ((int64_t)(h * (n_out / 32) + nb) * KS) * 64 + lane;
    const int ra = t0 + (lane & 31), rb = ra + 32;
    const uint16_t* xa = x + ((int64_t)ra * H + h) * ld_x + (lane >> 5) * 8;
    const uint16_t* xb = x + ((int64_t)rb * H + h) * ld_x + (lane >> 5) * 8;
    floatx16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int j = 0; j < KQ; ++j) {
        const int ks = wave * KQ + j;
        const bf16x8 b = wf[ks * 64];
        bf16x8 a0 = {}, a1 = {};
        if (ra < M) a0 = *reinterpret_cast<const bf16x8*>(xa + ks * 16);
        if (rb < M) a1 = *reinterpret_cast<const bf16x8*>(xb + ks * 16);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b, acc1, 0, 0, 0);
    }
    // partial tile of this wavefront: C[i][j] in lane j + 32*((i/4)%2), register 4*(i/8) + i%4
    {
        float* pt = part[wave];
        const int g = lane >> 5, j = lane & 31;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 8 * (r >> 2) + 4 * g + (r & 3);
            pt[i * (PROW / 4) + j] = acc0[r];
            pt[(32 + i) * (PROW / 4) + j] = acc1[r];
        }
    }
    __syncthreads();
    // 64 rows x 32 columns: each thread sums 8 consecutive columns of one row
    const int row = tid >> 2, c0 = (tid & 3) * 8;
    const int t = t0 + row;
    if (t < M) {
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int off = row * (PROW / 4) + c0 + 2 * e + k;
                v[k] = (part[0][off] + part[1][off]) + (part[2][off] + part[3][off]);
            }
            o[e] = (uint32_t)bf16_bits(v[0]) | ((uint32_t)bf16_bits(v[1]) << 16);
        }
        *reinterpret_cast<u32x4*>(y + ((int64_t)t * H + h) * ld_y + nb * 32 + c0) = u32x4{o[0], o[1], o[2], o[3]};
    }
}

int num_cus() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

template <int K>
int launch_proj(const uint16_t* x, int64_t ld_x, const bf16x8* wp, int M, int H, int n_out, uint16_t* y,
                int64_t ld_y, hipStream_t s) {
    const int n_tt = (M + kRows - 1) / kRows, n_cb = (n_out + kCols - 1) / kCols;
    const int64_t nblocks = (int64_t)H * n_cb * n_tt;
    if (nblocks > 0x7fffffff) return DDT_EINVAL;
    if (nblocks < num_cus()) {  // too few workgroups to fill the chip: split the reduction
        const int n_nb = n_out / 32;
        hipLaunchKernelGGL(proj_splitk_kernel<K>, dim3((unsigned)((int64_t)H * n_nb * n_tt)), dim3(kThreads), 0, s,
                           x, ld_x, wp, M, H, n_out, y, ld_y, n_tt, n_nb);
        DDT_CHECK_LAUNCH();
        return DDT_OK;
    }
    hipLaunchKernelGGL(proj_kernel<K>, dim3((unsigned)nblocks), dim3(kThreads), 0, s, x, ld_x, wp, M, H, n_out, y,
                       ld_y, n_tt, n_cb);
    DDT_CHECK_LAUNCH();
    return DDT_OK;
}

bool proj_shape_ok(int H, int K, int n_out) {
    return H >= 1 && (K == 64 || K == 128 || K == 256 || K == 512) && n_out >= 32 && n_out % 32 == 0 &&
           n_out <= 4096;
}

}  // namespace

extern "C" int ddt_proj_pack_weight(const void* w, int H, int K, int n_out, int dtype, void* packed,
                                    hipStream_t stream) {
    if (!w || !packed) return DDT_EINVAL;
    if (!proj_shape_ok(H, K, n_out)) return DDT_EINVAL;
    if (dtype != DDT_BF16) return DDT_EUNSUPPORTED;
    if (!ddt::aligned(packed, 16) || !ddt::aligned(w, 2)) return DDT_EINVAL;
    if (w == packed) return DDT_EINVAL;
    const int64_t total = (int64_t)H * (n_out / 32) * (K / 16) * 64;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7fffffff) return DDT_EINVAL;
    hipLaunchKernelGGL(proj_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(w), H, K, n_out, static_cast<u32x4*>(packed));
    DDT_CHECK_LAUNCH();
    return DDT_OK;
}

extern "C" int ddt_head_proj(const void* x, int64_t ld_x, const void* w_packed, int M, int H, int K, int n_out,
                             int dtype, void* y, int64_t ld_y, hipStream_t stream) {
    if (!w_packed || M < 0) return DDT_EINVAL;
    if (!proj_shape_ok(H, K, n_out)) return DDT_EINVAL;
    if (dtype != DDT_BF16) return DDT_EUNSUPPORTED;
    if (ld_x < K || ld_y < n_out || ld_x % 8 != 0 || ld_y % 8 != 0) return DDT_EINVAL;
    if (M == 0) return DDT_OK;  // x and y are not touched (and may be null)
    if (!x || !y) return DDT_EINVAL;
    if (!ddt::aligned(x, 16) || !ddt::aligned(y, 16) || !ddt::aligned(w_packed, 16)) return DDT_EINVAL;
    {   // x and y must not overlap (rows are read into LDS while others are written)
        const int64_t rows = (int64_t)M * H;
        const uintptr_t x0 = (uintptr_t)x, x1 = x0 + (uintptr_t)(((rows - 1) * ld_x + K) * 2);
        const uintptr_t y0 = (uintptr_t)y, y1 = y0 + (uintptr_t)(((rows - 1) * ld_y + n_out) * 2);
        if (x0 < y1 && y0 < x1) return DDT_EINVAL;
    }
    const auto* xs = static_cast<const uint16_t*>(x);
    const auto* wp = static_cast<const bf16x8*>(w_packed);
    auto* ys = static_cast<uint16_t*>(y);
    switch (K) {
        case 64: return launch_proj<64>(xs, ld_x, wp, M, H, n_out, ys, ld_y, stream);
        case 128: return launch_proj<128>(xs, ld_x, wp, M, H, n_out, ys, ld_y, stream);
        case 256: return launch_proj<256>(xs, ld_x, wp, M, H, n_out, ys, ld_y, stream);
        default: return launch_proj<512>(xs, ld_x, wp, M, H, n_out, ys, ld_y, stream);
    }
}
