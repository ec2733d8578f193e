// Tree-verify attention in absorbed MLA form, gfx950.
//
// What is computed ("The Architecture of Pragmatic Ambition", sections
// "The Decision Architecture" and "The Thinking Process"; "The
// Architectural Keystone ...", sections "What the Header Declares" and "The
// Reasoning That Preceded the Header"): every query row (request b, node i,
// head h) attends over the latent cache rows [0, P_b) and over the tree
// nodes it descends from (mask bits), with score
//   s_t = scale * (q_lat . c_kv[t] + q_pe . k_pe[t])
// and value c_kv[t].  All H*N query rows of a request share one latent key
// / value stream (an MQA-shaped problem with a 576-wide key and a 512-wide
// value that is the first 512 columns of the key).
//
// How (MI355X-first):
//  * A workgroup of 4 wavefronts owns 128 query rows (32 per wavefront) of
//    one request and one contiguous split of its key range.  Key tiles of 32
//    latent rows are staged HBM -> registers -> LDS once per workgroup and
//    shared by all 128 rows, double buffered so the next tile's global loads
//    are in flight while the current tile is multiplied.
//  * S^T = K . Q^T on MFMA 32x32x16 bf16 (32x32x2 f32 for fp32 data): the K
//    tile is the A operand (read from LDS), the wavefront's 32 queries are
//    the B operand and stay in registers for the whole split.  With this
//    orientation the scores of one query row land in one lane pair (l,
//    l+32), so the online-softmax max/sum need a single cross-half swap and
//    the running max, sum and rescale factor are per-lane scalars.
//  * O^T += V^T . P^T: the probabilities come straight out of the score
//    accumulators as the B operand; V^T is the A operand, read from a second
//    LDS copy of the tile written transposed during staging.  Keys inside a
//    16-key block are stored in the order the score accumulator hands them
//    out, so every A fragment is one 16-byte LDS read.  The 32x512 fp32
//    output accumulator lives in AGPR/VGPRs, one row per lane pair.
//  * fp32 online softmax in the log2 domain; the output rescale is skipped
//    when no row's running max moved.
//  * The key range of each request is cut into splits so that the launch
//    covers the 256 CUs; splits write normalised partial outputs and a
//    log-sum-exp to the workspace in the MFMA register order (1 KB
//    contiguous per store instruction), and a combine kernel merges them.
//    A request with one split writes its final output directly.
//  * Workgroup ids are remapped so that each XCD runs a contiguous range of
//    work items: the row tiles sharing one key split run on one XCD and
//    reuse its L2.
#include <math.h>

#include "common.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int KT = 32;               // keys per tile
constexpr int NW = 4;                // wavefronts per workgroup
constexpr int ROWS_WG = 32 * NW;     // query rows per workgroup
constexpr int kThreads = 64 * NW;
constexpr int kMinChunk = 256;       // smallest automatic split (keys)
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

template <typename T>
struct Traits;

template <>
struct Traits<uint16_t> {  // bf16 bit patterns
    static constexpr int KPL = 8;  // k elements per lane per MFMA
    using Frag = bf16x8;
    __device__ static floatx16 mfma(Frag a, Frag b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static Frag load(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
    __device__ static Frag zero() { return Frag{}; }
    __device__ static Frag from_f32(const float* v) {
        Frag r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = static_cast<__bf16>(v[e]);
        return r;
    }
};

template <>
struct Traits<float> {
    static constexpr int KPL = 1;
    using Frag = float;
    __device__ static floatx16 mfma(Frag a, Frag b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    __device__ static Frag load(const float* p) { return *p; }
    __device__ static Frag zero() { return 0.f; }
    __device__ static Frag from_f32(const float* v) { return v[0]; }
};

__device__ inline uint16_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

template <typename T>
__device__ inline void store4(T* dst, const float* v);
template <>
__device__ inline void store4<uint16_t>(uint16_t* dst, const float* v) {
    uint2 w;
    w.x = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
    w.y = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
    *reinterpret_cast<uint2*>(dst) = w;
}
template <>
__device__ inline void store4<float>(float* dst, const float* v) {
    *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
}

// Position of tile key `key` (0..31) inside a V^T row.  The score
// accumulator of lane half g holds, at index a = 4i + j, the key 8i + 4g + j;
// the value MFMA consumes indices a in groups of KPL per k-step, lane half g
// reading positions [ks*2*KPL + g*KPL, +KPL).  Storing each key at the
// position its score occupies makes every A fragment one contiguous read.
template <int KPL>
__device__ constexpr int vt_pos(int key) {
    const int i = key >> 3, g = (key >> 2) & 1, j = key & 3;
    const int a = 4 * i + j;
    return (a / KPL) * 2 * KPL + g * KPL + (a % KPL);
}

struct VerifyParams {
    const void* q_lat;
    const void* q_pe;
    const void* ckv;
    const void* kpe;
    const int64_t* kv_base;
    const uint64_t* mask;
    void* out;
    float* lse;
    float* ws_o;    // [slot][NW][NCT][4][64][4] fp32, normalised partial outputs
    float* ws_lse;  // [slot][ROWS_WG] fp32, log2-domain partial log-sum-exp
    int64_t ld_ql, ld_qp, ld_ckv, ld_kpe;
    int B, H, N, W, rows, row_tiles, chunk, total_wg;
    float scale_log2;
    int P[DDT_MAX_BATCH];
    int nsplit[DDT_MAX_BATCH];
    int wg_begin[DDT_MAX_BATCH + 1];
};

template <typename T, int DL, int DR>
struct Shape {
    using Tr = Traits<T>;
    static constexpr int KPL = Tr::KPL;
    static constexpr int DQK = DL + DR;
    static constexpr int KSTEP = 2 * KPL;        // k per MFMA
    static constexpr int NKS = DQK / KSTEP;      // score MFMAs per tile
    static constexpr int NCT = DL / 32;          // 32-column output tiles
    static constexpr int NPS = KT / KSTEP;       // value MFMA k-steps per tile
    static constexpr int VEC = 16 / sizeof(T);   // elements per 16-byte chunk
    static constexpr int KSTR = DQK + VEC;       // K-layout row stride (16-byte pad)
    static constexpr int VSTR = KT + VEC;        // V^T row stride (16-byte pad)
    static constexpr int KBUF = KT * KSTR;
    static constexpr int VBUF = DL * VSTR;
    static constexpr int STAGE = KBUF + VBUF;    // elements per pipeline stage
    static constexpr int NU_C = (KT / 4) * (DL / VEC);  // c_kv staging units (4 keys x 16 B)
    static constexpr int NU_R = KT * (DR / VEC);        // k_pe staging units (1 key x 16 B)
    static constexpr int UC = (NU_C + kThreads - 1) / kThreads;
    static constexpr int UR = (NU_R + kThreads - 1) / kThreads;
    static constexpr int WS_SLOT = NW * 32 * DL;  // floats of partial output per work item
    static_assert(DL % KSTEP == 0 && DR % KSTEP == 0, "head dims must be multiples of the MFMA k");
    static_assert(DL % 32 == 0 && DL % VEC == 0 && DR % VEC == 0, "head dims must tile");
};

template <typename T, int DL, int DR>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void verify_split(
    const VerifyParams p) {
    using S = Shape<T, DL, DR>;
    using Tr = typename S::Tr;
    using Frag = typename Tr::Frag;
    constexpr int KPL = S::KPL, VEC = S::VEC;
    __shared__ __attribute__((aligned(16))) T smem[2 * S::STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;

    // ---- work item: (request, key split, row tile), XCD-contiguous ----
    const int wl = ddt::xcd_logical_block(blockIdx.x, gridDim.x);
    int b = 0;
    {
        int lo = 0, hi = p.B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.wg_begin[mid] <= wl) lo = mid; else hi = mid - 1;
        }
        b = lo;
    }
    const int local = wl - p.wg_begin[b];
    const int split = local / p.row_tiles;
    const int rt = local - split * p.row_tiles;
    const int P = p.P[b];
    const int kbeg = split * p.chunk;
    const int kend = min(kbeg + p.chunk, P + p.N);
    const int ntiles = (kend - kbeg + KT - 1) / KT;
    const int64_t kvb = p.kv_base[b];
    const T* __restrict__ ckv = static_cast<const T*>(p.ckv);
    const T* __restrict__ kpe = static_cast<const T*>(p.kpe);

    const int wrow0 = rt * ROWS_WG + wave * 32;
    const bool wave_active = wrow0 < p.rows;
    const int row = wrow0 + l32;  // this lane's query row within the request
    const bool row_ok = row < p.rows;
    const int node = row_ok ? row / p.H : 0;
    const int64_t qrow = (int64_t)b * p.rows + (row_ok ? row : 0);
    const uint64_t* __restrict__ mrow = p.mask + ((int64_t)b * p.N + node) * p.W;

    // ---- queries: B operand of the score MFMA, resident for the whole split ----
    Frag q[S::NKS];
#pragma unroll
    for (int s = 0; s < S::NKS; ++s) {
        const int d0 = s * S::KSTEP + g * KPL;
        const T* src = d0 < DL ? static_cast<const T*>(p.q_lat) + qrow * p.ld_ql + d0
                               : static_cast<const T*>(p.q_pe) + qrow * p.ld_qp + (d0 - DL);
        q[s] = row_ok ? Tr::load(src) : Tr::zero();
    }

    floatx16 o[S::NCT];
#pragma unroll
    for (int c = 0; c < S::NCT; ++c) o[c] = floatx16{};
    float m_run = -INFINITY, l_run = 0.f;

    // ---- staging: global -> registers -> LDS (K layout + transposed V^T) ----
    uint4 rc[S::UC][4];
    uint4 rr[S::UR];
    auto stage_load = [&](int t0) {
#pragma unroll
        for (int x = 0; x < S::UC; ++x) {
            const int u = tid + x * kThreads;
            const int kg = u % (KT / 4), c = u / (KT / 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = t0 + 4 * kg + j;
                rc[x][j] = (u < S::NU_C && t < kend)
                               ? *reinterpret_cast<const uint4*>(ckv + (kvb + t) * p.ld_ckv + c * VEC)
                               : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int x = 0; x < S::UR; ++x) {
            const int u = tid + x * kThreads;
            const int c = u % (DR / VEC), key = u / (DR / VEC);
            const int t = t0 + key;
            rr[x] = (u < S::NU_R && t < kend)
                        ? *reinterpret_cast<const uint4*>(kpe + (kvb + t) * p.ld_kpe + c * VEC)
                        : make_uint4(0, 0, 0, 0);
        }
    };
    auto stage_store = [&](int buf) {
        T* sK = smem + buf * S::STAGE;
        T* sV = sK + S::KBUF;
#pragma unroll
        for (int x = 0; x < S::UC; ++x) {
            const int u = tid + x * kThreads;
            if (u < S::NU_C) {
                const int kg = u % (KT / 4), c = u / (KT / 4);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<uint4*>(sK + (4 * kg + j) * S::KSTR + c * VEC) = rc[x][j];
                if constexpr (KPL == 8) {
                    // 4 consecutive keys land at 4 consecutive V^T positions: one 8-byte write per column
                    const int pos = vt_pos<KPL>(4 * kg);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        const int sh = (e & 1) * 16;
                        const uint32_t v0 = ((reinterpret_cast<const uint32_t*>(&rc[x][0]))[e >> 1] >> sh) & 0xffffu;
                        const uint32_t v1 = ((reinterpret_cast<const uint32_t*>(&rc[x][1]))[e >> 1] >> sh) & 0xffffu;
                        const uint32_t v2 = ((reinterpret_cast<const uint32_t*>(&rc[x][2]))[e >> 1] >> sh) & 0xffffu;
                        const uint32_t v3 = ((reinterpret_cast<const uint32_t*>(&rc[x][3]))[e >> 1] >> sh) & 0xffffu;
                        *reinterpret_cast<uint2*>(sV + (c * VEC + e) * S::VSTR + pos) =
                            make_uint2(v0 | (v1 << 16), v2 | (v3 << 16));
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const T* vals = reinterpret_cast<const T*>(&rc[x][j]);
                        const int pos = vt_pos<KPL>(4 * kg + j);
#pragma unroll
                        for (int e = 0; e < VEC; ++e) sV[(c * VEC + e) * S::VSTR + pos] = vals[e];
                    }
                }
            }
        }
#pragma unroll
        for (int x = 0; x < S::UR; ++x) {
            const int u = tid + x * kThreads;
            if (u < S::NU_R) {
                const int c = u % (DR / VEC), key = u / (DR / VEC);
                *reinterpret_cast<uint4*>(sK + key * S::KSTR + DL + c * VEC) = rr[x];
            }
        }
    };

    // ---- one key tile: scores, online softmax, value product ----
    auto compute = [&](int buf, int t0) {
        const T* sK = smem + buf * S::STAGE;
        const T* sV = sK + S::KBUF;
        floatx16 s = floatx16{};
#pragma unroll
        for (int ks = 0; ks < S::NKS; ++ks)
            s = Tr::mfma(Tr::load(sK + l32 * S::KSTR + ks * S::KSTEP + g * KPL), q[ks], s);

        float x[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) x[v] = s[v] * p.scale_log2;
        if (t0 + KT > P || t0 + KT > kend) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int t = t0 + (v >> 2) * 8 + g * 4 + (v & 3);
                bool vis = t < kend;
                if (vis && t >= P) {
                    const int j = t - P;
                    vis = (mrow[j >> 6] >> (j & 63)) & 1ull;
                }
                if (!vis) x[v] = -INFINITY;
            }
        }
        float mx = x[0];
#pragma unroll
        for (int v = 1; v < 16; ++v) mx = fmaxf(mx, x[v]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        const float base = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - base);
        float ps[16];
        float rs = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            ps[v] = __builtin_amdgcn_exp2f(x[v] - base);
            rs += ps[v];
        }
        rs += __shfl_xor(rs, 32, 64);
        l_run = l_run * alpha + rs;
        m_run = m_new;
        if (__ballot(alpha != 1.f) != 0) {
#pragma unroll
            for (int c = 0; c < S::NCT; ++c) o[c] *= alpha;
        }
        Frag pb[S::NPS];
#pragma unroll
        for (int ks = 0; ks < S::NPS; ++ks) pb[ks] = Tr::from_f32(ps + ks * KPL);
#pragma unroll
        for (int c = 0; c < S::NCT; ++c) {
#pragma unroll
            for (int ks = 0; ks < S::NPS; ++ks)
                o[c] = Tr::mfma(Tr::load(sV + (c * 32 + l32) * S::VSTR + ks * S::KSTEP + g * KPL), pb[ks], o[c]);
        }
    };

    stage_load(kbeg);
    stage_store(0);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
        const int t0 = kbeg + it * KT;
        const bool more = it + 1 < ntiles;
        if (more) stage_load(t0 + KT);
        if (wave_active) compute(it & 1, t0);
        if (more) stage_store((it + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue ----
    if (!row_ok) return;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const float lse2 = l_run > 0.f ? m_run + __log2f(l_run) : -INFINITY;
    if (p.nsplit[b] == 1) {
        T* dst = static_cast<T*>(p.out) + qrow * DL;
#pragma unroll
        for (int c = 0; c < S::NCT; ++c) {
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = o[c][grp * 4 + e] * inv;
                store4<T>(dst + c * 32 + grp * 8 + g * 4, v);
            }
        }
        if (g == 0) p.lse[qrow] = lse2 * kLn2;
    } else {
        float* ws = p.ws_o + ((size_t)wl * NW + wave) * (S::NCT * 4 * 64 * 4);
#pragma unroll
        for (int c = 0; c < S::NCT; ++c) {
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const float4 v = make_float4(o[c][grp * 4 + 0] * inv, o[c][grp * 4 + 1] * inv,
                                             o[c][grp * 4 + 2] * inv, o[c][grp * 4 + 3] * inv);
                *reinterpret_cast<float4*>(ws + ((c * 4 + grp) * 64 + lane) * 4) = v;
            }
        }
        if (g == 0) p.ws_lse[(size_t)wl * ROWS_WG + wave * 32 + l32] = lse2;
    }
}

// Merge the key splits of every row of multi-split requests:
//   M = max_s lse_s, w_s = 2^(lse_s - M), out = sum_s w_s o_s / sum_s w_s,
//   lse = (M + log2 sum_s w_s) ln 2.
// One workgroup per (request, row tile, wavefront, 32-column tile); thread
// (grp, lane) owns the 4 consecutive outputs the split kernel's lane `lane`
// stored at group `grp`.
template <typename T, int DL>
__global__ __launch_bounds__(256) void verify_combine(const VerifyParams p) {
    constexpr int NCT = DL / 32;
    const int per_b = p.row_tiles * NW * NCT;
    const int b = blockIdx.x / per_b;
    const int ns = p.nsplit[b];
    if (ns <= 1) return;
    int rem = blockIdx.x - b * per_b;
    const int rt = rem / (NW * NCT);
    rem -= rt * (NW * NCT);
    const int wave = rem / NCT, c = rem - (rem / NCT) * NCT;
    const int grp = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 5, l32 = lane & 31;
    const int row = rt * ROWS_WG + wave * 32 + l32;
    if (row >= p.rows) return;
    const int64_t qrow = (int64_t)b * p.rows + row;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) {
        const int slot = p.wg_begin[b] + s * p.row_tiles + rt;
        M = fmaxf(M, p.ws_lse[(size_t)slot * ROWS_WG + wave * 32 + l32]);
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    for (int s = 0; s < ns; ++s) {
        const int slot = p.wg_begin[b] + s * p.row_tiles + rt;
        const float ls = p.ws_lse[(size_t)slot * ROWS_WG + wave * 32 + l32];
        const float w = ls == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ls - M);
        const float4 v = *reinterpret_cast<const float4*>(
            p.ws_o + ((size_t)slot * NW + wave) * (NCT * 4 * 64 * 4) + ((c * 4 + grp) * 64 + lane) * 4);
        acc[0] += w * v.x;
        acc[1] += w * v.y;
        acc[2] += w * v.z;
        acc[3] += w * v.w;
        wsum += w;
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] *= inv;
    store4<T>(static_cast<T*>(p.out) + qrow * DL + c * 32 + grp * 8 + g * 4, acc);
    if (c == 0 && grp == 0 && g == 0) p.lse[qrow] = (M + __log2f(wsum)) * kLn2;
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

struct Plan {
    int row_tiles = 0, chunk = 0, total_wg = 0;
    bool any_split = false;
    size_t ws_bytes = 0, ws_lse_off = 0;
};

int check_desc(const ddt_attn_desc* d, const int32_t* prefix_len_host) {
    if (d == nullptr || prefix_len_host == nullptr) return DDT_EINVAL;
    if (d->B < 1 || d->B > DDT_MAX_BATCH || d->H < 1 || d->N < 1 || d->N > DDT_MAX_NODES) return DDT_EINVAL;
    if (d->kv_chunk < 0) return DDT_EINVAL;
    const bool k2 = d->d_lat == 512 && d->d_rope == 64 && d->dtype == DDT_BF16;
    const bool tiny = d->d_lat == 64 && d->d_rope == 16 && d->dtype == DDT_F32;
    if (!k2 && !tiny) return DDT_EUNSUPPORTED;
    if (d->ld_ql < d->d_lat || d->ld_qp < d->d_rope || d->ld_ckv < d->d_lat || d->ld_kpe < d->d_rope)
        return DDT_EINVAL;
    const int64_t es = ddt::elem_bytes(d->dtype);
    if ((d->ld_ql * es) % 16 || (d->ld_qp * es) % 16 || (d->ld_ckv * es) % 16 || (d->ld_kpe * es) % 16)
        return DDT_EINVAL;
    if ((int64_t)d->H * d->N > (1 << 24)) return DDT_EINVAL;
    for (int b = 0; b < d->B; ++b)
        if (prefix_len_host[b] < 0 || (int64_t)prefix_len_host[b] + d->N > 0x7fffffff - 4096) return DDT_EINVAL;
    return DDT_OK;
}

Plan make_plan(const ddt_attn_desc* d, const int32_t* P, VerifyParams* vp) {
    Plan pl;
    const int rows = d->H * d->N;
    pl.row_tiles = (rows + ROWS_WG - 1) / ROWS_WG;
    if (d->kv_chunk > 0) {
        pl.chunk = (int)ddt::round_up((size_t)d->kv_chunk, KT);
    } else {
        int64_t work = 0;
        for (int b = 0; b < d->B; ++b) work += (int64_t)pl.row_tiles * (P[b] + d->N);
        const int64_t ideal = (work + num_cus() - 1) / num_cus();
        int64_t ch = (int64_t)ddt::round_up((size_t)ideal, KT);
        if (ch < kMinChunk) ch = kMinChunk;
        pl.chunk = (int)ch;
    }
    int64_t total = 0;
    for (int b = 0; b < d->B; ++b) {
        const int64_t T = (int64_t)P[b] + d->N;
        const int ns = (int)((T + pl.chunk - 1) / pl.chunk);
        if (ns > 1) pl.any_split = true;
        if (vp) {
            vp->P[b] = P[b];
            vp->nsplit[b] = ns;
            vp->wg_begin[b] = (int)total;
        }
        total += (int64_t)ns * pl.row_tiles;
    }
    if (total > 0x7fffffff) total = 0x7fffffff;
    pl.total_wg = (int)total;
    if (vp) vp->wg_begin[d->B] = pl.total_wg;
    if (pl.any_split) {
        const size_t o = (size_t)pl.total_wg * NW * 32 * d->d_lat * sizeof(float);
        pl.ws_lse_off = ddt::round_up(o, 256);
        pl.ws_bytes = pl.ws_lse_off + ddt::round_up((size_t)pl.total_wg * ROWS_WG * sizeof(float), 256);
    }
    return pl;
}

template <typename T, int DL, int DR>
int launch(const VerifyParams& vp, const Plan& pl, hipStream_t stream) {
    hipLaunchKernelGGL((verify_split<T, DL, DR>), dim3(pl.total_wg), dim3(kThreads), 0, stream, vp);
    DDT_CHECK_LAUNCH();
    if (pl.any_split) {
        const int nblk = vp.B * pl.row_tiles * NW * (DL / 32);
        hipLaunchKernelGGL((verify_combine<T, DL>), dim3(nblk), dim3(256), 0, stream, vp);
        DDT_CHECK_LAUNCH();
    }
    return DDT_OK;
}

}  // namespace

extern "C" int ddt_verify_workspace(const ddt_attn_desc* d, const int32_t* prefix_len_host, size_t* bytes) {
    if (bytes == nullptr) return DDT_EINVAL;
    const int rc = check_desc(d, prefix_len_host);
    if (rc != DDT_OK) return rc;
    *bytes = make_plan(d, prefix_len_host, nullptr).ws_bytes;
    return DDT_OK;
}

extern "C" int ddt_verify_attn(const ddt_attn_desc* d, const void* q_lat, const void* q_pe, const void* ckv,
                               const void* kpe, const int64_t* kv_base, const int32_t* prefix_len_host,
                               const uint64_t* mask, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    int rc = check_desc(d, prefix_len_host);
    if (rc != DDT_OK) return rc;
    if (!q_lat || !q_pe || !ckv || !kpe || !kv_base || !mask || !out || !lse) return DDT_EINVAL;
    if (!ddt::aligned(q_lat, 16) || !ddt::aligned(q_pe, 16) || !ddt::aligned(ckv, 16) || !ddt::aligned(kpe, 16) ||
        !ddt::aligned(out, 16) || !ddt::aligned(lse, 4))
        return DDT_EINVAL;
    VerifyParams vp{};
    const Plan pl = make_plan(d, prefix_len_host, &vp);
    if (pl.ws_bytes > 0) {
        if (workspace == nullptr || workspace_bytes < pl.ws_bytes || !ddt::aligned(workspace, 256))
            return DDT_EWORKSPACE;
        vp.ws_o = static_cast<float*>(workspace);
        vp.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.ws_lse_off);
    }
    vp.q_lat = q_lat;
    vp.q_pe = q_pe;
    vp.ckv = ckv;
    vp.kpe = kpe;
    vp.kv_base = kv_base;
    vp.mask = mask;
    vp.out = out;
    vp.lse = lse;
    vp.ld_ql = d->ld_ql;
    vp.ld_qp = d->ld_qp;
    vp.ld_ckv = d->ld_ckv;
    vp.ld_kpe = d->ld_kpe;
    vp.B = d->B;
    vp.H = d->H;
    vp.N = d->N;
    vp.W = (d->N + 63) / 64;
    vp.rows = d->H * d->N;
    vp.row_tiles = pl.row_tiles;
    vp.chunk = pl.chunk;
    vp.total_wg = pl.total_wg;
    vp.scale_log2 = d->scale * kLog2e;
    if (d->dtype == DDT_BF16) return launch<uint16_t, 512, 64>(vp, pl, stream);
    return launch<float, 64, 16>(vp, pl, stream);
}
