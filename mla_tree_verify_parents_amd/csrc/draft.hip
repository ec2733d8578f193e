// The step before the verify path: the drafter's per-depth top-k candidates
// and the best-first draft tree built from them ("The Architecture of
// Pragmatic Ambition", section "The Knowledge Architecture": the tree
// builder takes per-depth top-k candidates from a drafter and builds a
// best-first tree; "The Architectural Keystone: Writing the Model Header
// ...", section "The Context: Building an Engine from First Principles":
// the GPU builder replaced a per-request heap on the CPU).
//
// ddt_draft_topk: a row of draft logits is cut into chunks of 16384
// entries, 64 per thread (16 coalesced 16-byte loads, in registers).  A
// chunk workgroup reduces the chunk's (maximum, sum of exp(x - maximum))
// and finds its top K through a threshold: each wavefront takes the K-th
// largest of its 64 threads' maxima, so at least K entries of the chunk
// reach the largest of those four values T, and every entry of the chunk's
// top K is at least T.  The entries >= T (typically K to 2K of them) go to
// an LDS list, and one wavefront takes the top K of the list in K rounds of
// a wavefront maximum over 64-bit keys (order-preserving value bits, then
// the inverted index: the largest key is the largest value at the lowest
// index).  When the list overflows (many equal values) the workgroup falls
// back to K rounds of a workgroup maximum over every entry.  A second
// launch, one workgroup per row, selects the top K among the chunks'
// candidates and merges the (maximum, sum) pairs into the row's
// log-sum-exp.  HBM-bound: 4 bytes per logit.  (Chunks of 4096 entries with
// the K workgroup rounds per chunk measured 91 us at 256 x 163840, the
// rounds dominating.)
//
// ddt_best_first_tree: one wavefront per request.  Each pop is a wavefront
// maximum over packed keys (score, then lower depth, then earlier
// insertion), then the node is written and the first child and the next
// sibling enter the frontier.  Trees of at most 64 nodes keep the frontier
// and the nodes in registers (one per lane); larger trees keep the
// frontier in LDS.  Scores are fp32 sums along the
// path, as the tree's definition fixes them.
#include "argmax_scan.h"
#include "common.h"

namespace {

constexpr int kTopkThreads = 256;
constexpr int kChunkPerThread = 64;                          // entries per thread in a chunk
constexpr int kTopkChunk = kTopkThreads * kChunkPerThread;   // 16384 entries per chunk workgroup
constexpr int kCandCap = 1024;                               // LDS list of a chunk's entries >= T
constexpr int kMaxTopK = 16;
constexpr int kMergePerLane = 16;                            // candidates per lane in the row merge
constexpr int64_t kMaxDraftVocab = 1 << 20;
static_assert(kMaxDraftVocab / kTopkChunk * kMaxTopK <= 64 * kMergePerLane, "the merge holds every candidate");

__device__ inline uint64_t umax(uint64_t a, uint64_t b) { return a > b ? a : b; }

// One step of a wavefront maximum by DPP: every lane takes the larger of its
// value and the value of the lane the DPP control names (lanes with no
// source, or outside row_mask, keep theirs).
template <int kCtrl, int kRowMask>
__device__ inline uint32_t dpp_max_step(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kCtrl, kRowMask, 0xf, false);
    return o > v ? o : v;
}
template <int kCtrl, int kRowMask>
__device__ inline uint64_t dpp_max_step(uint64_t v) {
    const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
    const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, kCtrl, kRowMask, 0xf, false);
    const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, kCtrl, kRowMask, 0xf, false);
    const uint64_t o = ((uint64_t)ohi << 32) | olo;
    return o > v ? o : v;
}

// Wavefront maximum of unsigned keys, returned uniform: prefix maxima inside
// each row of 16 lanes (row_shr 1, 2, 4, 8), then row 0's and row 2's last
// lane into rows 1 and 3 (row_bcast:15), then lane 31 into rows 2 and 3
// (row_bcast:31): lane 63 holds the maximum.
template <typename U>
__device__ inline U wave_max(U v) {
    v = dpp_max_step<0x111, 0xf>(v);
    v = dpp_max_step<0x112, 0xf>(v);
    v = dpp_max_step<0x114, 0xf>(v);
    v = dpp_max_step<0x118, 0xf>(v);
    v = dpp_max_step<0x142, 0xa>(v);
    v = dpp_max_step<0x143, 0xc>(v);
    if constexpr (sizeof(U) == 8) {
        const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 63);
        const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
        return ((uint64_t)hi << 32) | lo;
    } else {
        return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
    }
}

// Workgroup maximum of one 64-bit key per thread, returned to every thread.
__device__ inline uint64_t block_max_all(uint64_t v, uint64_t* red) {
    v = wave_max(v);
    const int wave = threadIdx.x / ddt::kWave;
    __syncthreads();  // the previous round's readers are done with red[]
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    uint64_t m = red[0];
#pragma unroll
    for (int w = 1; w < kTopkThreads / ddt::kWave; ++w) m = umax(m, red[w]);
    return m;
}

// Merge of (maximum, sum of exp(x - maximum)) pairs; a pair with maximum
// -inf holds nothing.
__device__ inline void ms_merge(float& m, float& s, float mo, float so) {
    const float mn = fmaxf(m, mo);
    s = (m == -INFINITY ? 0.f : s * __expf(m - mn)) + (mo == -INFINITY ? 0.f : so * __expf(mo - mn));
    m = mn;
}

// The float whose order key is u (the inverse of ddt::order_key on numbers).
__device__ inline float key_float(uint32_t u) {
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// The K largest of the wavefront's keys (J per lane, 0 = empty, distinct)
// in K rounds of a wavefront maximum; round k's key lands in lane k.
template <int J>
__device__ inline uint64_t wave_top(uint64_t (&key)[J], int K, int lane) {
    uint32_t taken = 0;
    uint64_t res = 0;
    for (int k = 0; k < K; ++k) {
        uint64_t b = 0;
#pragma unroll
        for (int j = 0; j < J; ++j) b = ((taken >> j) & 1u) ? b : umax(b, key[j]);
        const uint64_t mk = wave_max(b);
        if (lane == k) res = mk;
        if (mk != 0 && b == mk) {
#pragma unroll
            for (int j = 0; j < J; ++j)
                if (key[j] == mk) taken |= 1u << j;
        }
    }
    return res;
}

template <int J>
__device__ inline uint64_t list_top(const uint64_t* list, int n, int K, int lane) {
    uint64_t key[J];
#pragma unroll
    for (int j = 0; j < J; ++j) key[j] = j * 64 + lane < n ? list[j * 64 + lane] : 0;
    return wave_top<J>(key, K, lane);
}

// Chunk c of row r: top-K keys and (max, sum exp(x - max)) into the
// workspace.  Entry i of thread t is column c*16384 + ((i/4)*256 + t)*4 +
// i%4 (16-byte loads, consecutive threads on consecutive 16 bytes).  kVec:
// every column of the chunk lies in the row and the row is 16-byte aligned;
// otherwise scalar loads, columns past the row padded with -inf and left
// out.  Workgroup g takes chunk c0 + g % cn of row g / cn.
template <bool kVec>
__global__ __launch_bounds__(kTopkThreads) void topk_chunks(const float* __restrict__ logits, int64_t V, int64_t ld,
                                                           int nchunk, int c0, int cn, int K,
                                                           uint64_t* __restrict__ ws_keys,
                                                           float2* __restrict__ ws_ms) {
    constexpr int NW = kTopkThreads / ddt::kWave;
    __shared__ uint64_t red[NW];
    __shared__ float2 red_ms[NW];
    __shared__ uint32_t red_thr[NW];
    __shared__ uint64_t s_cand[kCandCap];
    __shared__ uint64_t out[kMaxTopK];
    __shared__ int s_n;
    const int64_t r = blockIdx.x / cn;
    const int c = c0 + (int)(blockIdx.x - r * cn);
    const float* row = logits + r * ld;
    const int64_t base = (int64_t)c * kTopkChunk;
    const int lim = V - base < kTopkChunk ? (int)(V - base) : kTopkChunk;  // columns of the chunk in the row
    const uint32_t idx0 = (uint32_t)base;  // (V <= 2^20)
    uint64_t* keys_out = ws_keys + (r * nchunk + c) * K;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid / ddt::kWave;
    if (tid == 0) s_n = 0;
    auto cidx = [&](int i) { return ((i / 4) * kTopkThreads + tid) * 4 + (i % 4); };
    auto valid = [&](int i) { return kVec || cidx(i) < lim; };
    float x[kChunkPerThread];
    if constexpr (kVec) {
        typedef float F4 __attribute__((ext_vector_type(4)));
        const F4* p = reinterpret_cast<const F4*>(row + base) + tid;
#pragma unroll
        for (int q = 0; q < kChunkPerThread / 4; ++q) {
            const F4 v = __builtin_nontemporal_load(p + q * kTopkThreads);
            x[4 * q] = v.x, x[4 * q + 1] = v.y, x[4 * q + 2] = v.z, x[4 * q + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < kChunkPerThread; ++i) x[i] = valid(i) ? row[base + cidx(i)] : -INFINITY;
    }
    // this thread's maximum (NaN ignored) and sum of exp(x - maximum)
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kChunkPerThread; ++i) m = fmaxf(m, x[i]);  // (padding is -inf)
    float sm = 0.f;
#pragma unroll
    for (int i = 0; i < kChunkPerThread; ++i) sm += valid(i) ? __expf(x[i] - m) : 0.f;
    const bool any = valid(0);  // entry 0 is the thread's first column
    // The threshold: this wavefront's K-th largest thread maximum (ties
    // taken together), when at least K of its threads hold columns.  Each
    // such thread holds an entry whose key is at least its maximum's (a NaN
    // entry's key is above every number), so at least K entries reach it.
    {
        const uint32_t u = any ? ddt::order_key(__float_as_uint(m)) : 0u;
        bool live = any;
        int removed = 0;
        uint32_t tw = 0;
        for (int k = 0; k < K && removed < K; ++k) {
            const uint32_t mx = wave_max(live ? u : 0u);
            if (mx == 0) break;
            tw = mx;
            const bool hit = live && u == mx;
            removed += __popcll(__ballot(hit));
            live = live && !hit;
        }
        if (lane == 0) red_thr[wave] = removed >= K ? tw : 0u;
    }
    // the chunk's (max, sum): wavefront, then workgroup (at the end)
    {
        float mw = m, sw = sm;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ms_merge(mw, sw, __shfl_xor(mw, o, ddt::kWave), __shfl_xor(sw, o, ddt::kWave));
        if (lane == 0) red_ms[wave] = make_float2(mw, sw);
    }
    __syncthreads();
    uint32_t T = red_thr[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) T = red_thr[w] > T ? red_thr[w] : T;
    // Every entry whose key is >= T onto the list: for numbers that is
    // x >= key_float(T); NaN keys are above every threshold.  T = 0: every
    // column.
    const float tf = T == 0 ? -INFINITY : key_float(T);
#pragma unroll
    for (int i = 0; i < kChunkPerThread; ++i) {
        if (valid(i) && !(x[i] < tf)) {
            const int at = atomicAdd(&s_n, 1);
            if (at < kCandCap) s_cand[at] = ddt::pack_key(__float_as_uint(x[i]), idx0 + cidx(i));
        }
    }
    __syncthreads();
    const int n = s_n;
    if (n <= kCandCap) {
        if (wave != 0) return;
        const uint64_t res = n <= 64    ? list_top<1>(s_cand, n, K, lane)
                             : n <= 256 ? list_top<4>(s_cand, n, K, lane)
                                        : list_top<kCandCap / 64>(s_cand, n, K, lane);
        if (lane < K) keys_out[lane] = res;
    } else {
        // many equal values: K rounds of a workgroup maximum over every
        // entry (a thread's entries ascend in column, so its first largest
        // key is its best)
        uint64_t taken = 0;
        for (int k = 0; k < K; ++k) {
            uint32_t bk = 0;
            int bi = -1;
#pragma unroll
            for (int i = 0; i < kChunkPerThread; ++i) {
                const uint32_t u = ddt::order_key(__float_as_uint(x[i]));
                if (valid(i) && !((taken >> i) & 1u) && u > bk) bk = u, bi = i;
            }
            const uint64_t b = bi < 0 ? 0 : ((uint64_t)bk << 32) | (0xffffffffu - (idx0 + (uint32_t)cidx(bi)));
            const uint64_t mk = block_max_all(b, red);
            if (tid == 0) out[k] = mk;
            if (mk != 0 && b == mk) taken |= 1ull << bi;
        }
        __syncthreads();
        if (tid < K) keys_out[tid] = out[tid];
    }
    if (tid == 0) {
        float M = red_ms[0].x, S = red_ms[0].y;
#pragma unroll
        for (int w = 1; w < NW; ++w) ms_merge(M, S, red_ms[w].x, red_ms[w].y);
        ws_ms[r * nchunk + c] = make_float2(M, S);
    }
}

// Row r, one wavefront: top K among its chunks' candidates, then the
// log-softmax values (the row's log-sum-exp from the chunks' pairs).
__global__ __launch_bounds__(64) void topk_merge(const float* __restrict__ logits, int64_t ld, int nchunk, int K,
                                                const uint64_t* __restrict__ ws_keys,
                                                const float2* __restrict__ ws_ms, int32_t* __restrict__ ids,
                                                float* __restrict__ logp) {
    const int64_t r = blockIdx.x;
    const int lane = threadIdx.x;
    const int n = nchunk * K;  // at most 64 * kMergePerLane
    float m = -INFINITY, s = 0.f;
    for (int c = lane; c < nchunk; c += ddt::kWave) {
        const float2 p = ws_ms[r * nchunk + c];
        ms_merge(m, s, p.x, p.y);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ms_merge(m, s, __shfl_xor(m, o, ddt::kWave), __shfl_xor(s, o, ddt::kWave));
    const float lse = m + __logf(s);
    const uint64_t* cand = ws_keys + r * n;
    const uint64_t res = n <= 64    ? list_top<1>(cand, n, K, lane)
                         : n <= 256 ? list_top<4>(cand, n, K, lane)
                                    : list_top<kMergePerLane>(cand, n, K, lane);
    if (lane < K) {
        const int32_t id = (int32_t)(0xffffffffu - (uint32_t)res);
        ids[r * K + lane] = id;
        logp[r * K + lane] = logits[r * ld + id] - lse;
    }
}

// ---------------------------------------------------------------- tree ----

constexpr int kTreeMaxDK = 4096;  // D * K candidates per request, staged in LDS

// Frontier key: score (order-preserving bits), then lower depth, then
// earlier insertion: the largest key goes next.
__device__ inline uint64_t frontier_key(float score, int d, int seq) {
    return ((uint64_t)ddt::order_key(__float_as_uint(score)) << 32) | ((uint64_t)(255 - d) << 24) |
           (uint64_t)(0xffffff - seq);
}

__global__ __launch_bounds__(64) void best_first_kernel(const int32_t* __restrict__ ids, const float* __restrict__ lp,
                                                       int D, int K, int budget, const int32_t* __restrict__ roots,
                                                       int32_t* __restrict__ parents, int32_t* __restrict__ tokens,
                                                       int32_t* __restrict__ depth) {
    __shared__ float s_lp[kTreeMaxDK];
    __shared__ int32_t s_id[kTreeMaxDK];
    __shared__ float f_score[DDT_MAX_NODES];
    __shared__ int32_t f_dr[DDT_MAX_NODES];   // depth << 16 | rank
    __shared__ int32_t f_par[DDT_MAX_NODES];
    __shared__ int32_t f_seq[DDT_MAX_NODES];
    __shared__ float n_score[DDT_MAX_NODES];
    const int b = blockIdx.x, lane = threadIdx.x;
    const int DK = D * K;
    for (int i = lane; i < DK; i += 64) {
        s_lp[i] = lp[(int64_t)b * DK + i];
        s_id[i] = ids[(int64_t)b * DK + i];
    }
    const int64_t o = (int64_t)b * (budget + 1);
    int nf = 0, seq = 0;
    if (lane == 0) {
        parents[o] = -1;
        tokens[o] = roots[b];
        depth[o] = 0;
        n_score[0] = 0.f;
    }
    __syncthreads();
    if (budget > 0) {
        if (lane == 0) {
            f_score[0] = 0.f + s_lp[0];
            f_dr[0] = 1 << 16;
            f_par[0] = 0;
            f_seq[0] = 0;
        }
        nf = 1;
        seq = 1;
    }
    for (int n = 1; n <= budget; ++n) {
        __syncthreads();  // (one wavefront: orders the LDS writes of the previous pop)
        // the best frontier entry: each lane scans a stride, then a wavefront maximum
        uint64_t best = 0;
        int at = -1;
        for (int i = lane; i < nf; i += 64) {
            const int dr = f_dr[i];
            const uint64_t k = frontier_key(f_score[i], dr >> 16, f_seq[i]);
            if (k > best) best = k, at = i;
        }
        uint64_t m = best;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) m = umax(m, __shfl_xor(m, off, 64));
        const uint64_t win = __ballot(best == m && at >= 0);
        if (win == 0) break;  // (cannot happen: the host checked that the candidates suffice)
        const int i = __shfl(at, __builtin_ctzll(win), 64);
        // the popped entry, read by every lane before lane 0 rewrites the frontier
        const float sc = f_score[i];
        const int dr = f_dr[i], d = dr >> 16, r = dr & 0xffff, par = f_par[i];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the reads above have completed
        if (lane == 0) {
            const int last = nf - 1;  // the last entry takes the popped one's place
            f_score[i] = f_score[last];
            f_dr[i] = f_dr[last];
            f_par[i] = f_par[last];
            f_seq[i] = f_seq[last];
            int nn = last;
            parents[o + n] = par;
            tokens[o + n] = s_id[(d - 1) * K + r];
            depth[o + n] = d;
            n_score[n] = sc;
            if (d < D) {  // first child
                f_score[nn] = sc + s_lp[d * K];
                f_dr[nn] = (d + 1) << 16;
                f_par[nn] = n;
                f_seq[nn] = seq;
                ++nn;
            }
            if (r + 1 < K) {  // next sibling
                f_score[nn] = n_score[par] + s_lp[(d - 1) * K + r + 1];
                f_dr[nn] = (d << 16) | (r + 1);
                f_par[nn] = par;
                f_seq[nn] = seq + 1;
                ++nn;
            }
        }
        // every lane keeps the same count: one popped, up to two inserted
        nf = nf - 1 + (d < D ? 1 : 0) + (r + 1 < K ? 1 : 0);
        seq += 2;
    }
}

// Trees of at most 64 nodes: the frontier never holds more than 64
// candidates (a pop adds at most one net), so lane l keeps candidate l in
// registers and lane n keeps node n.  A pop is a wavefront maximum over the
// same packed keys, taken in two 32-bit steps (the score word; then, only
// when scores tie, the depth / insertion word of the tied lanes), the
// winner's fields broadcast from its lane; the first child and then the
// next sibling take the lowest free lanes.  With at most 64 candidates per
// request (kRegTables) lane i also holds candidate i's log-probability and
// token, read by v_readlane instead of LDS.  Same arithmetic and order as
// best_first_kernel, so the trees are identical.
template <bool kRegTables>
__global__ __launch_bounds__(64) void best_first_wave_kernel(const int32_t* __restrict__ ids,
                                                            const float* __restrict__ lp, int D, int K, int budget,
                                                            const int32_t* __restrict__ roots,
                                                            int32_t* __restrict__ parents,
                                                            int32_t* __restrict__ tokens,
                                                            int32_t* __restrict__ depth) {
    __shared__ float s_lp[kRegTables ? 1 : kTreeMaxDK];
    __shared__ int32_t s_id[kRegTables ? 1 : kTreeMaxDK];
    const int b = blockIdx.x, lane = threadIdx.x;
    const int DK = D * K;
    float r_lp = 0.f;
    int r_id = 0;
    if constexpr (kRegTables) {
        if (lane < DK) {
            r_lp = lp[(int64_t)b * DK + lane];
            r_id = ids[(int64_t)b * DK + lane];
        }
    } else {
        for (int i = lane; i < DK; i += 64) {
            s_lp[i] = lp[(int64_t)b * DK + i];
            s_id[i] = ids[(int64_t)b * DK + i];
        }
        __syncthreads();
    }
    // candidate i's log-probability and token (i wave-uniform)
    auto cand_lp = [&](int i) {
        if constexpr (kRegTables)
            return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r_lp), i));
        else
            return s_lp[i];
    };
    auto cand_id = [&](int i) {
        if constexpr (kRegTables)
            return __builtin_amdgcn_readlane(r_id, i);
        else
            return s_id[i];
    };
    // this lane's frontier candidate
    bool valid = false;
    float fs = 0.f;
    int fd = 0, fr = 0, fp = 0, fq = 0;
    // this lane's node (node index == lane): the root in lane 0
    int np = -1, nt = 0, nd = 0;
    float ns = 0.f;
    if (lane == 0) nt = roots[b];
    int seq = 0;
    if (budget > 0) {
        const float l0 = cand_lp(0);
        if (lane == 0) {
            valid = true;
            fs = 0.f + l0;
            fd = 1;
        }
        seq = 1;
    }
    for (int n = 1; n <= budget; ++n) {
        // the frontier key, (score word) << 32 | (depth / insertion word)
        const uint32_t hi = valid ? ddt::order_key(__float_as_uint(fs)) : 0u;
        const uint32_t lo = ((uint32_t)(255 - fd) << 24) | (uint32_t)(0xffffff - fq);
        const uint32_t mhi = wave_max(hi);
        uint64_t win = __ballot(valid && hi == mhi);
        if (win == 0) break;  // (cannot happen: the host checked that the candidates suffice)
        if (__popcll(win) > 1) {  // tied scores: the depth / insertion word decides
            const bool tied = valid && hi == mhi;
            const uint32_t mlo = wave_max(tied ? lo : 0u);
            win = __ballot(tied && lo == mlo);
        }
        const int wl = __builtin_ctzll(win);  // (uniform: readlane broadcasts into scalar registers)
        const float sc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fs), wl));
        const int d = __builtin_amdgcn_readlane(fd, wl), r = __builtin_amdgcn_readlane(fr, wl);
        const int par = __builtin_amdgcn_readlane(fp, wl);
        if (lane == wl) valid = false;
        const int tok = cand_id((d - 1) * K + r);
        if (lane == n) {
            np = par;
            nt = tok;
            nd = d;
            ns = sc;
        }
        const float pscore =  // node par (< n) is already recorded
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ns), par));
        if (d < D) {  // first child
            const float lc = cand_lp(d * K);
            const int fl = __builtin_ctzll(~__ballot(valid));
            if (lane == fl) {
                valid = true;
                fs = sc + lc;
                fd = d + 1;
                fr = 0;
                fp = n;
                fq = seq;
            }
        }
        if (r + 1 < K) {  // next sibling
            const float ls = cand_lp((d - 1) * K + r + 1);
            const int fl = __builtin_ctzll(~__ballot(valid));
            if (lane == fl) {
                valid = true;
                fs = pscore + ls;
                fd = d;
                fr = r + 1;
                fp = par;
                fq = seq + 1;
            }
        }
        seq += 2;
    }
    const int64_t o = (int64_t)b * (budget + 1);
    if (lane <= budget) {
        parents[o + lane] = np;
        tokens[o + lane] = nt;
        depth[o + lane] = nd;
    }
}

}  // namespace

extern "C" int ddt_draft_topk_workspace(int64_t rows, int64_t V, int K, size_t* bytes) {
    if (bytes == nullptr || rows < 0 || V < 1 || V > kMaxDraftVocab || K < 1 || K > kMaxTopK || K > V)
        return DDT_EINVAL;
    const int64_t nchunk = (V + kTopkChunk - 1) / kTopkChunk;
    *bytes = (size_t)rows * nchunk * (K * sizeof(uint64_t) + sizeof(float2));
    return DDT_OK;
}

extern "C" int ddt_draft_topk(const float* logits, int64_t rows, int64_t V, int64_t ld, int K, int32_t* ids,
                              float* logp, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    size_t need = 0;
    const int rc = ddt_draft_topk_workspace(rows, V, K, &need);
    if (rc != DDT_OK || ld < V) return DDT_EINVAL;
    if (rows == 0) return DDT_OK;
    if (!logits || !ids || !logp) return DDT_EINVAL;
    const int64_t nchunk = (V + kTopkChunk - 1) / kTopkChunk;
    if (rows * nchunk > 0x7fffffff) return DDT_EINVAL;
    if (workspace == nullptr || workspace_bytes < need || !ddt::aligned(workspace, 16)) return DDT_EWORKSPACE;
    uint64_t* keys = static_cast<uint64_t*>(workspace);
    float2* ms = reinterpret_cast<float2*>(keys + rows * nchunk * K);
    const bool vec = ddt::aligned(logits, 16) && (ld * 4) % 16 == 0;
    const int nfull = vec ? (int)(V / kTopkChunk) : 0;  // chunks taken by 16-byte loads
    if (nfull > 0) {
        hipLaunchKernelGGL(topk_chunks<true>, dim3((unsigned)(rows * nfull)), dim3(kTopkThreads), 0, stream, logits,
                           V, ld, (int)nchunk, 0, nfull, K, keys, ms);
        DDT_CHECK_LAUNCH();
    }
    if (nchunk > nfull) {
        const int nrest = (int)nchunk - nfull;
        hipLaunchKernelGGL(topk_chunks<false>, dim3((unsigned)(rows * nrest)), dim3(kTopkThreads), 0, stream,
                           logits, V, ld, (int)nchunk, nfull, nrest, K, keys, ms);
        DDT_CHECK_LAUNCH();
    }
    hipLaunchKernelGGL(topk_merge, dim3((unsigned)rows), dim3(64), 0, stream, logits, ld, (int)nchunk, K,
                       keys, ms, ids, logp);
    DDT_CHECK_LAUNCH();
    return DDT_OK;
}

extern "C" int ddt_best_first_tree(const int32_t* ids, const float* logp, int B, int D, int K, int budget,
                                   const int32_t* root_tokens, int32_t* parents, int32_t* tokens, int32_t* depth,
                                   hipStream_t stream) {
    if (B < 0 || D < 1 || K < 1 || budget < 0 || budget + 1 > DDT_MAX_NODES || D > 255 || K > 0xffff ||
        (int64_t)D * K > kTreeMaxDK)
        return DDT_EINVAL;
    // enough candidates: sum over d = 1..D of K^d >= budget
    int64_t avail = 0, level = 1;
    for (int d = 1; d <= D && avail < budget; ++d) {
        level = level * K > budget ? budget + 1 : level * K;
        avail += level;
    }
    if (avail < budget) return DDT_EINVAL;
    if (B == 0) return DDT_OK;
    if (!ids || !logp || !root_tokens || !parents || !tokens || !depth) return DDT_EINVAL;
    if (budget + 1 <= 64 && D * K <= 64)  // frontier and candidate tables one per lane
        hipLaunchKernelGGL(best_first_wave_kernel<true>, dim3(B), dim3(64), 0, stream, ids, logp, D, K, budget,
                           root_tokens, parents, tokens, depth);
    else if (budget + 1 <= 64)  // the frontier fits one candidate per lane
        hipLaunchKernelGGL(best_first_wave_kernel<false>, dim3(B), dim3(64), 0, stream, ids, logp, D, K, budget,
                           root_tokens, parents, tokens, depth);
    else
        hipLaunchKernelGGL(best_first_kernel, dim3(B), dim3(64), 0, stream, ids, logp, D, K, budget, root_tokens,
                           parents, tokens, depth);
    DDT_CHECK_LAUNCH();
    return DDT_OK;
}
