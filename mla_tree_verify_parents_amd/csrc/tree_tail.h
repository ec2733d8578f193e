// Device building blocks of the end of a verify step, shared by the
// stand-alone acceptance and compaction kernels and their fused form.
//
// greedy_walk: "The Architecture of Pragmatic Ambition", section "The
// Knowledge Architecture" (walk the verified tree greedily for the longest
// path matching the target's predictions).
// copy_path_rows: "The Architectural Keystone: Writing the Model Header ...",
// section "The Reasoning That Preceded the Header" (the accepted path's
// latents are gathered into contiguous slots) and section "Mistakes and
// Iterative Refinement" (source and destination slots alias).
#pragma once

#include "common.h"

namespace ddt {

// One wavefront walks request b's tree.  spar / sdraft hold the request's
// parents and draft ids in LDS.  From the root, repeatedly move to the
// lowest-numbered child k of the current node c whose draft id equals the
// target id after c: 64 candidate nodes are tested at once and the ballot's
// lowest set bit is the answer.  The current node strictly increases, so
// the walk ends after at most N steps even for a malformed tree.  spath
// receives the path (root first); returns its length (accepted drafts + 1),
// valid in every lane.
__device__ inline int greedy_walk(const int32_t* __restrict__ target, int64_t off, const int32_t* spar,
                                  const int32_t* sdraft, int N, int32_t* spath, int lane) {
    int c = 0, n = 1;
    if (lane == 0) spath[0] = 0;
    for (;;) {
        const int want = target[off + c];
        int next = -1;
        for (int base = c + 1; base < N; base += kWave) {
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
    return n;
}

// The acceptance outputs of one request from its walk (one wavefront):
// path = [0, k1, ...] then -1, tokens = draft ids along the path then the
// bonus token target[last], then -1, accept_len = n - 1.
__device__ inline void write_accept(const int32_t* __restrict__ target, int64_t off, const int32_t* sdraft,
                                    const int32_t* spath, int n, int N, int b, int lane,
                                    int32_t* __restrict__ accept_len, int32_t* __restrict__ path,
                                    int32_t* __restrict__ tokens) {
    const int bonus = target[off + spath[n - 1]];
    for (int j = lane; j < N; j += kWave) {
        const int p = j < n ? spath[j] : -1;
        path[off + j] = p;
        int tok = -1;
        if (j + 1 < n) tok = sdraft[spath[j + 1]];
        else if (j + 1 == n) tok = bonus;
        tokens[off + j] = tok;
    }
    if (lane == 0) accept_len[b] = n - 1;
}

// Where the cache slots of a request live in the pool.  Contiguous: slot t
// of request b is row kv_base[b] + t.  Paged (table non-null): slot t is row
// table[b*ld + (t >> shift)] * 2^shift + (t mod 2^shift), pages of 2^shift
// rows named by a block table.
struct SlotMap {
    const int64_t* kv_base;
    const int32_t* table;
    int64_t ld;
    int shift;
    __device__ int64_t row(int b, int64_t t) const {
        if (table == nullptr) return kv_base[b] + t;
        const int64_t pg = table[(int64_t)b * ld + (t >> shift)];
        return (pg << shift) + (t & ((1ll << shift) - 1));
    }
    // Whether slots [P, P + n) can be mapped: P >= 0 and, paged, every one of
    // them falls inside the request's table row (a stale or oversized length
    // must not reach the next request's table entries or past the table).
    __device__ bool covers(int64_t P, int64_t n) const {
        if (P < 0 || n < 1) return false;
        return table == nullptr || ((P + n - 1) >> shift) < ld;
    }
};

// Cache slot P+j <- cache slot P+path(j), j = 0..k, for a path that
// starts at 0 and increases (so path(j) >= j): copies go in blocks of
// increasing j, each block loaded whole into LDS (stage, rows_per_block
// rows) before any of its rows is stored.  A copy then never reads a row an
// earlier block wrote, and no global scratch is needed.  All threads of the
// workgroup take part; PathAt(j) returns path(j).
template <typename U, typename PathAt>
__device__ inline void copy_path_rows(char* __restrict__ ckv, int64_t ld_ckv, char* __restrict__ kpe,
                                      int64_t ld_kpe, int ckv_units, int kpe_units, const SlotMap& map, int b,
                                      int64_t P, int k, int rows_per_block, U* stage, PathAt path_at) {
    const int upr = ckv_units + kpe_units;  // U units per cache row
    for (int j0 = 0; j0 <= k; j0 += rows_per_block) {
        const int jn = (k + 1 - j0) < rows_per_block ? (k + 1 - j0) : rows_per_block;
        const int total = jn * upr;
        for (int u = threadIdx.x; u < total; u += blockDim.x) {
            const int j = j0 + u / upr, part = u % upr;
            const int src = path_at(j);
            if (src == j) continue;  // already in place
            const int64_t row = map.row(b, P + src);
            stage[u] = part < ckv_units ? reinterpret_cast<const U*>(ckv + row * ld_ckv)[part]
                                        : reinterpret_cast<const U*>(kpe + row * ld_kpe)[part - ckv_units];
        }
        __syncthreads();
        for (int u = threadIdx.x; u < total; u += blockDim.x) {
            const int j = j0 + u / upr, part = u % upr;
            if (path_at(j) == j) continue;
            const int64_t row = map.row(b, P + j);
            if (part < ckv_units)
                reinterpret_cast<U*>(ckv + row * ld_ckv)[part] = stage[u];
            else
                reinterpret_cast<U*>(kpe + row * ld_kpe)[part - ckv_units] = stage[u];
        }
        __syncthreads();
    }
}

// Arguments of acceptance + compaction for every request of a batch (row
// strides in bytes; copy units as in CompactLayout).
struct AcceptCompactArgs {
    const int32_t* target;   // [B*N] target ids (argmax of the target logits)
    const int32_t* draft;    // [B*N] draft ids
    const int32_t* parents;  // [B*N]
    int N;
    int32_t* accept_len;  // [B]
    int32_t* path;        // [B*N]
    int32_t* tokens;      // [B*N]
    char* ckv;
    char* kpe;
    int64_t ld_ckv, ld_kpe;
    int ckv_units, kpe_units, rows_per_block;
    SlotMap map;
    const int32_t* prefix_len;  // [B] committed lengths
    int32_t* new_prefix_len;    // [B] may be prefix_len itself
    int32_t* src_slot;          // [B*N] or null
};

// Acceptance and compaction of request b by one workgroup: wavefront 0
// walks the tree (LDS), all threads then move the accepted rows through
// `stage` (rows_per_block rows).  The walk only moves to higher node
// numbers, so its path is always a valid compaction path.  Every thread
// reads the committed length before thread 0 writes the new one, so
// new_prefix_len may alias prefix_len.
template <typename U>
__device__ void accept_compact_body(const AcceptCompactArgs& a, int b, U* stage) {
    __shared__ int32_t spar[DDT_MAX_NODES];
    __shared__ int32_t sdraft[DDT_MAX_NODES];
    __shared__ int32_t spath[DDT_MAX_NODES];
    __shared__ int s_n;
    const int N = a.N;
    const int64_t off = (int64_t)b * N;
    for (int i = threadIdx.x; i < N; i += blockDim.x) {
        spar[i] = a.parents[off + i];
        sdraft[i] = a.draft[off + i];
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
        const int n = greedy_walk(a.target, off, spar, sdraft, N, spath, threadIdx.x);
        if (threadIdx.x == 0) s_n = n;
    }
    __syncthreads();
    const int n = s_n, k = n - 1;
    if (threadIdx.x < kWave)
        write_accept(a.target, off, sdraft, spath, n, N, b, threadIdx.x, a.accept_len, a.path, a.tokens);
    const int64_t P = a.prefix_len[b];
    // slots P .. P + path[k] must be mappable (a committed length that is
    // negative or, paged, runs past the table row leaves the request's
    // cache and length untouched)
    const bool ok = a.map.covers(P, (int64_t)spath[k] + 1);
    if (a.src_slot != nullptr) {
        for (int j = threadIdx.x; j < N; j += blockDim.x)
            a.src_slot[off + j] = (ok && j <= k) ? (int32_t)(P + spath[j]) : -1;
    }
    if (!ok) {
        if (threadIdx.x == 0) a.new_prefix_len[b] = (int32_t)P;  // (the value every thread read: no race if aliased)
        return;
    }
    copy_path_rows<U>(a.ckv, a.ld_ckv, a.kpe, a.ld_kpe, a.ckv_units, a.kpe_units, a.map, b, P, k, a.rows_per_block,
                      stage, [&](int j) { return spath[j]; });  // (ends with a barrier: every thread has read P)
    if (threadIdx.x == 0) a.new_prefix_len[b] = (int32_t)(P + k + 1);
}

// Copy granularity and LDS staging of a compaction, chosen on the host.
struct CompactLayout {
    int64_t lc, lk;           // row strides in bytes
    int ckv_units, kpe_units;  // units of the copy type per row part
    int rows_per_block;
    size_t stage_bytes;
    bool vec16;                // 16-byte units (else 4-byte)
};

constexpr int kCompactThreads = 256;
constexpr int kCompactStageBytes = 32768;

// Fills `lay` for the given layout; returns DDT_OK, DDT_EINVAL or DDT_EUNSUPPORTED.
inline int compact_layout(const void* ckv, int64_t ld_ckv, const void* kpe, int64_t ld_kpe, int dtype, int d_lat,
                          int d_rope, int N, CompactLayout* lay) {
    const int es = elem_bytes(dtype);
    lay->lc = ld_ckv * es;
    lay->lk = ld_kpe * es;
    const int rc = d_lat * es, rk = d_rope * es;
    if (ld_ckv < d_lat || (d_rope > 0 && ld_kpe < d_rope)) return DDT_EINVAL;
    auto fits = [&](int a) {
        return aligned(ckv, a) && aligned(kpe, a) && lay->lc % a == 0 && (d_rope == 0 || lay->lk % a == 0) &&
               rc % a == 0 && rk % a == 0;
    };
    const int row_bytes = rc + rk;
    int rpb = kCompactStageBytes / row_bytes;
    if (rpb < 1) return DDT_EUNSUPPORTED;
    if (rpb > N) rpb = N;
    lay->rows_per_block = rpb;
    lay->stage_bytes = (size_t)rpb * row_bytes;
    if (fits(16)) {
        lay->vec16 = true;
        lay->ckv_units = rc / 16;
        lay->kpe_units = rk / 16;
    } else if (fits(4)) {
        lay->vec16 = false;
        lay->ckv_units = rc / 4;
        lay->kpe_units = rk / 4;
    } else {
        return DDT_EINVAL;
    }
    return DDT_OK;
}

}  // namespace ddt
