/*
 * oracle.c -- plain, slow, fp64 CPU oracle for DDTree tree-verify MLA.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no source with the HIP library.
 *
 * Every function is the plain definition of one step of the verify step of
 * DDTree speculative decoding for an MLA model, as described on the pages
 *   [P1] "The Architecture of Pragmatic Ambition: Building a Native C++
 *        Inference Engine for Kimi K2.6"
 *   [P2] "The Architectural Keystone: Writing the Model Header for a Native
 *        DDTree Inference Engine"
 * with no blocking, fusion or reordering beyond the definition.  Floating
 * point work is done in double precision on inputs converted exactly from
 * fp32 or bf16.  Loops over independent output rows use OpenMP; each row is
 * computed by one thread, in the order the definition states.
 *
 * Return values: 0 on success, a negative number on an argument error, and
 * a positive number when an internal self-check fails.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F64 2 /* only the per-head projection takes fp64 inputs (to chain oracle results) */

/* Exact widening of one stored element to double. */
static double orc_load(const void* base, int dtype, int64_t idx) {
    if (dtype == ORC_F64) return ((const double*)base)[idx];
    if (dtype == ORC_F32) return (double)((const float*)base)[idx];
    uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int orc_elem_bytes(int dtype) { return dtype == ORC_F32 ? 4 : 2; }

/* Tree validity: node 0 is the root (parent -1); every other node's parent
 * precedes it (parents[i] in [0, i)).  The verify step places node i at
 * cache slot P+i, so nodes are numbered in a topological order ([P2],
 * "The Reasoning That Preceded the Header": root at the next free slot,
 * budget+1 nodes). */
static int orc_tree_valid(const int32_t* par, int N) {
    if (N < 1 || par[0] != -1) return 0;
    for (int i = 1; i < N; ++i)
        if (par[i] < 0 || par[i] >= i) return 0;
    return 1;
}

/*
 * Ancestor mask ([P1] "The Decision Architecture": prefill and verify differ
 * only in the attention mask; tree verify exposes a node's ancestors).
 * mask[b][i][w] bit (j mod 64) of word w = j / 64 is set iff j is i or an
 * ancestor of i, found by walking the parent links from i up to the root.
 * depth[b][i] = number of edges from i to the root.  For an invalid tree the
 * request's mask words are all zero, depth is -1 and tree_err[b] = 1.
 */
int orc_build_mask(const int32_t* parents, int B, int N, uint64_t* mask,
                   int32_t* depth, int32_t* tree_err) {
    if (!parents || !mask || B < 0 || N < 1) return -1;
    int W = (N + 63) / 64;
    for (int b = 0; b < B; ++b) {
        const int32_t* par = parents + (int64_t)b * N;
        uint64_t* mb = mask + (int64_t)b * N * W;
        int ok = orc_tree_valid(par, N);
        if (tree_err) tree_err[b] = ok ? 0 : 1;
        memset(mb, 0, sizeof(uint64_t) * (size_t)N * W);
        for (int i = 0; i < N; ++i) {
            int d = -1;
            if (ok) {
                for (int j = i; j >= 0; j = par[j]) {
                    mb[(int64_t)i * W + j / 64] |= (uint64_t)1 << (j % 64);
                    ++d;
                }
            }
            if (depth) depth[(int64_t)b * N + i] = d;
        }
    }
    return 0;
}

/* j is visible from node i inside the tree iff j is i or an ancestor. */
static int orc_is_ancestor_or_self(const int32_t* par, int i, int j) {
    for (int a = i; a >= 0; a = par[a])
        if (a == j) return 1;
    return 0;
}

/*
 * Tree-verify attention in absorbed MLA form.
 *
 * [P1] "The Thinking Process" / "The Decision Architecture": the no-rope
 * score q_nope . (W_UK c_kv[t]) is computed as q_lat . c_kv[t] with the
 * absorbed query q_lat, so attention runs in the latent space and the value
 * of key t is c_kv[t] itself.  [P2] "What the Header Declares": the cache
 * keeps c_kv and the decoupled rope key k_pe per token.  [P2] "The Reasoning
 * That Preceded the Header": the verify forward processes budget+1 nodes,
 * the root at the next free slot, so node j sits at slot P+j; the whole
 * committed prefix [0, P) is visible, and inside the tree a node sees only
 * itself and its ancestors.
 *
 * For row (b, i, h), V = [0, P_b) u {P_b + j : j in anc*(i)}:
 *   s_t   = scale * (sum_d q_lat[d] c_kv[t][d] + sum_e q_pe[e] k_pe[t][e])
 *   m     = max_t s_t,  w_t = exp(s_t - m),  l = sum_t w_t
 *   out   = sum_t w_t c_kv[t] / l,   lse = m + ln l.
 *
 * Layouts: q rows are [B][N][H]; q_lat of flat row r starts at
 * q_lat + r*ld_ql and q_pe at q_pe + r*ld_qp (elements).  Cache row t of
 * request b is kv_base[b] + t; its c_kv starts at ckv + row*ld_ckv and its
 * k_pe at kpe + row*ld_kpe.  If `rows` is non-null only the listed flat rows
 * r = (b*N + i)*H + h are computed and out/lse/wsum are indexed by list
 * position; otherwise all B*N*H rows.  wsum (nullable) receives
 * sum_t (w_t / l), checked here to be 1 within max(1e-12, 4*T*eps).
 */
int orc_verify_attn(int B, int H, int N, int d_lat, int d_rope, int dtype, double scale,
                    const void* q_lat, int64_t ld_ql, const void* q_pe, int64_t ld_qp,
                    const void* ckv, int64_t ld_ckv, const void* kpe, int64_t ld_kpe,
                    const int64_t* kv_base, const int32_t* prefix_len,
                    const int32_t* parents, const int64_t* rows, int64_t nrows,
                    double* out, double* lse, double* wsum) {
    if (B < 1 || H < 1 || N < 1 || d_lat < 1 || d_rope < 0) return -1;
    if (!q_lat || !ckv || !kv_base || !prefix_len || !parents || !out || !lse) return -1;
    if (d_rope > 0 && (!q_pe || !kpe)) return -1;
    for (int b = 0; b < B; ++b)
        if (!orc_tree_valid(parents + (int64_t)b * N, N) || prefix_len[b] < 0) return -2;
    int64_t total = rows ? nrows : (int64_t)B * N * H;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
    for (int64_t k = 0; k < total; ++k) {
        int64_t r = rows ? rows[k] : k;
        int i = (int)((r / H) % N);
        int b = (int)(r / ((int64_t)H * N));
        if (b < 0 || b >= B) { ++bad; continue; }
        const int32_t* par = parents + (int64_t)b * N;
        int64_t P = prefix_len[b];
        int64_t T = P + N;
        double* s = (double*)malloc(sizeof(double) * (size_t)T);
        char* vis = (char*)malloc((size_t)T);
        if (!s || !vis) { free(s); free(vis); ++bad; continue; }
        /* visibility */
        for (int64_t t = 0; t < P; ++t) vis[t] = 1;
        for (int j = 0; j < N; ++j) vis[P + j] = (char)orc_is_ancestor_or_self(par, i, j);
        /* scores */
        double m = -INFINITY;
        for (int64_t t = 0; t < T; ++t) {
            if (!vis[t]) continue;
            int64_t row = kv_base[b] + t;
            double acc = 0.0;
            for (int d = 0; d < d_lat; ++d)
                acc += orc_load(q_lat, dtype, r * ld_ql + d) * orc_load(ckv, dtype, row * ld_ckv + d);
            for (int e = 0; e < d_rope; ++e)
                acc += orc_load(q_pe, dtype, r * ld_qp + e) * orc_load(kpe, dtype, row * ld_kpe + e);
            s[t] = scale * acc;
            if (s[t] > m) m = s[t];
        }
        /* softmax weights and weighted sum of the latent values */
        double l = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            if (!vis[t]) continue;
            s[t] = exp(s[t] - m);
            l += s[t];
        }
        double* o = out + k * d_lat;
        for (int d = 0; d < d_lat; ++d) o[d] = 0.0;
        double sum_w = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            if (!vis[t]) continue;
            double w = s[t] / l;
            sum_w += w;
            int64_t row = kv_base[b] + t;
            for (int d = 0; d < d_lat; ++d) o[d] += w * orc_load(ckv, dtype, row * ld_ckv + d);
        }
        lse[k] = m + log(l);
        if (wsum) wsum[k] = sum_w;
        /* the weights sum to one up to the rounding of |V| additions */
        double tol = 1e-12 > 4.0 * (double)T * 2.220446049250313e-16 ? 1e-12 : 4.0 * (double)T * 2.220446049250313e-16;
        if (fabs(sum_w - 1.0) > tol) ++bad;
        free(s);
        free(vis);
    }
    return bad ? 1 : 0;
}

/*
 * Target argmax ([P1] "The Decision Architecture": greedy token selection
 * from logits).  idx[r] = first index of the maximum of row r in a
 * left-to-right scan; a NaN counts as larger than every number, so the
 * first NaN wins (the convention of numpy.argmax).  -0 and +0 are equal.
 */
int orc_argmax(const void* logits, int dtype, int64_t rows, int64_t V, int64_t ld, int32_t* idx) {
    if (!logits || !idx || rows < 0 || V < 1 || ld < V) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t best = 0;
        double bv = orc_load(logits, dtype, r * ld);
        if (!isnan(bv)) {
            for (int64_t v = 1; v < V; ++v) {
                double x = orc_load(logits, dtype, r * ld + v);
                if (isnan(x)) { best = v; break; }
                if (x > bv) { bv = x; best = v; }
            }
        }
        idx[r] = (int32_t)best;
    }
    return 0;
}

/*
 * Greedy tree acceptance ([P1] "The Knowledge Architecture": the accept
 * kernel walks the verified tree greedily to find the longest prefix that
 * matches the target's predictions).  t[b][c] is the target's greedy token
 * after node c.  Starting at the root, move to the lowest-numbered child k
 * of the current node whose draft token equals t[c]; stop when no child
 * matches.  path = [0, k1, k2, ...], accept_len = number of accepted draft
 * nodes, tokens = drafts along the path followed by the bonus t[last].
 * Unused entries of path and tokens are -1.  draft_ids[b][0] is not read.
 */
int orc_greedy_accept(const int32_t* t, const int32_t* draft, const int32_t* parents,
                      int B, int N, int32_t* accept_len, int32_t* path, int32_t* tokens) {
    if (!t || !draft || !parents || !accept_len || !path || !tokens || B < 0 || N < 1) return -1;
    for (int b = 0; b < B; ++b) {
        const int32_t* tb = t + (int64_t)b * N;
        const int32_t* db = draft + (int64_t)b * N;
        const int32_t* pb = parents + (int64_t)b * N;
        int32_t* pathb = path + (int64_t)b * N;
        int32_t* tokb = tokens + (int64_t)b * N;
        for (int j = 0; j < N; ++j) pathb[j] = tokb[j] = -1;
        int c = 0, n = 0;
        pathb[n++] = 0;
        for (;;) {
            int next = -1;
            for (int k = 1; k < N; ++k)
                if (pb[k] == c && db[k] == tb[c]) { next = k; break; }
            if (next < 0) break;
            c = next;
            pathb[n++] = c;
        }
        accept_len[b] = n - 1;
        for (int j = 1; j < n; ++j) tokb[j - 1] = db[pathb[j]];
        tokb[n - 1] = tb[c];
    }
    return 0;
}

/*
 * KV compaction ([P2] "The Reasoning That Preceded the Header": after
 * acceptance the accepted path's latents, recomputed root included, are
 * gathered into contiguous cache slots and the length advances; [P2]
 * "Mistakes and Iterative Refinement": source and destination can alias, so
 * the gather reads from a copy taken before any write).
 * For request b with P = prefix_len[b], k = accept_len[b]:
 *   new slot P+j <- old slot P+path[j] for j = 0..k (c_kv and k_pe rows),
 *   prefix_len[b] = P + k + 1,
 *   src_slot[b][j] = P + path[j] for j <= k, else -1 (nullable).
 * Slots from P+k+1 on are left as they were.
 */
int orc_compact_kv(void* ckv, int64_t ld_ckv, void* kpe, int64_t ld_kpe, int dtype, int d_lat, int d_rope,
                   const int64_t* kv_base, int32_t* prefix_len, const int32_t* path,
                   const int32_t* accept_len, int B, int N, int32_t* src_slot) {
    if (!ckv || !kv_base || !prefix_len || !path || !accept_len || B < 0 || N < 1) return -1;
    if (d_rope > 0 && !kpe) return -1;
    int es = orc_elem_bytes(dtype);
    for (int b = 0; b < B; ++b) {
        int k = accept_len[b];
        const int32_t* pb = path + (int64_t)b * N;
        if (k < 0 || k >= N) return -2;
        int64_t P = prefix_len[b];
        char* cbuf = (char*)malloc((size_t)(k + 1) * d_lat * es);
        char* kbuf = (char*)malloc((size_t)(k + 1) * (d_rope > 0 ? d_rope : 1) * es);
        if (!cbuf || !kbuf) { free(cbuf); free(kbuf); return 2; }
        for (int j = 0; j <= k; ++j) {
            int64_t src = kv_base[b] + P + pb[j];
            memcpy(cbuf + (size_t)j * d_lat * es, (char*)ckv + src * ld_ckv * es, (size_t)d_lat * es);
            if (d_rope > 0)
                memcpy(kbuf + (size_t)j * d_rope * es, (char*)kpe + src * ld_kpe * es, (size_t)d_rope * es);
        }
        for (int j = 0; j <= k; ++j) {
            int64_t dst = kv_base[b] + P + j;
            memcpy((char*)ckv + dst * ld_ckv * es, cbuf + (size_t)j * d_lat * es, (size_t)d_lat * es);
            if (d_rope > 0)
                memcpy((char*)kpe + dst * ld_kpe * es, kbuf + (size_t)j * d_rope * es, (size_t)d_rope * es);
        }
        free(cbuf);
        free(kbuf);
        if (src_slot)
            for (int j = 0; j < N; ++j)
                src_slot[(int64_t)b * N + j] = j <= k ? (int32_t)(P + pb[j]) : -1;
        prefix_len[b] = (int32_t)(P + k + 1);
    }
    return 0;
}

/*
 * Per-depth draft candidates ([P1] "The Knowledge Architecture": the tree
 * builder takes the drafter's per-depth top-k candidates).  For each row r
 * of fp32 draft logits (row stride ld): ids[r][0..K) are the K largest
 * entries in order of value (descending), equal values by index
 * (ascending); logp[r][k] = x[ids[r][k]] - lse, the log-softmax over the
 * whole row, lse = m + ln(sum_v exp(x_v - m)) with m the row maximum, in
 * fp64.  Selection k is the largest entry that comes after selection k-1 in
 * that order, found by a left-to-right scan.  Finite logits, 1 <= K <= V.
 */
int orc_draft_topk(const float* logits, int64_t rows, int64_t V, int64_t ld, int K, int32_t* ids,
                   double* logp) {
    if (!logits || !ids || !logp || rows < 0 || V < 1 || ld < V || K < 1 || K > V) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float* x = logits + r * ld;
        double m = x[0];
        for (int64_t v = 1; v < V; ++v)
            if (x[v] > m) m = x[v];
        double s = 0.0;
        for (int64_t v = 0; v < V; ++v) s += exp((double)x[v] - m);
        const double lse = m + log(s);
        int64_t prev = -1;
        for (int k = 0; k < K; ++k) {
            int64_t best = -1;
            for (int64_t v = 0; v < V; ++v) {
                /* only entries after the previous selection in (value desc, index asc) order */
                if (prev >= 0 && !(x[v] < x[prev] || (x[v] == x[prev] && v > prev))) continue;
                if (best < 0 || x[v] > x[best]) best = v;
            }
            ids[r * K + k] = (int32_t)best;
            logp[r * K + k] = (double)x[best] - lse;
            prev = best;
        }
    }
    return 0;
}

/*
 * Best-first draft tree ([P1] "The Knowledge Architecture": a best-first
 * tree from the drafter's per-depth top-k; [P2] "The Context: Building an
 * Engine from First Principles": the GPU builder replaced a per-request
 * heap on the CPU).  Candidates: the token of rank r at depth d (ids[d-1][r],
 * log-probability lp[d-1][r]) under a node at depth d-1.  A node's score is
 * its parent's plus its own lp, an fp32 addition (the root scores 0).  The
 * frontier starts with (depth 1, rank 0) under the root; repeatedly the
 * frontier candidate with the highest score (then the lower depth, then the
 * earlier insertion) becomes the next node, and its first child (depth
 * d+1, rank 0; if d < D) and next sibling (depth d, rank r+1; if r+1 < K)
 * enter the frontier, in that order.  budget+1 nodes result, numbered in
 * that order: parents[i] < i, tokens[0] = root, depth[0] = 0.  Returns -2
 * when the candidates run out first.
 */
int orc_best_first_tree(const int32_t* ids, const float* lp, int D, int K, int budget, int32_t root,
                        int32_t* parents, int32_t* tokens, int32_t* depth) {
    if (!ids || !lp || !parents || !tokens || !depth || D < 0 || K < 0 || budget < 0) return -1;
    int cap = 2 * budget + 2;
    float* fs = (float*)malloc(sizeof(float) * cap);
    int* fd = (int*)malloc(sizeof(int) * cap);
    int* fr = (int*)malloc(sizeof(int) * cap);
    int* fp = (int*)malloc(sizeof(int) * cap);
    long* fq = (long*)malloc(sizeof(long) * cap);
    float* ns = (float*)malloc(sizeof(float) * (budget + 1));
    if (!fs || !fd || !fr || !fp || !fq || !ns) {
        free(fs); free(fd); free(fr); free(fp); free(fq); free(ns);
        return 2;
    }
    int nf = 0;
    long seq = 0;
    parents[0] = -1;
    tokens[0] = root;
    depth[0] = 0;
    ns[0] = 0.0f;
    if (budget > 0 && D > 0 && K > 0) {
        fs[nf] = ns[0] + lp[0]; fd[nf] = 1; fr[nf] = 0; fp[nf] = 0; fq[nf] = seq++; ++nf;
    }
    int n = 1, rc = 0;
    while (n < budget + 1) {
        if (nf == 0) { rc = -2; break; }
        int best = 0;
        for (int i = 1; i < nf; ++i) {
            if (fs[i] > fs[best] || (fs[i] == fs[best] && (fd[i] < fd[best] || (fd[i] == fd[best] && fq[i] < fq[best]))))
                best = i;
        }
        const float sc = fs[best];
        const int d = fd[best], r = fr[best], par = fp[best];
        --nf;  /* remove: the last candidate takes its place */
        fs[best] = fs[nf]; fd[best] = fd[nf]; fr[best] = fr[nf]; fp[best] = fp[nf]; fq[best] = fq[nf];
        parents[n] = par;
        tokens[n] = ids[(d - 1) * K + r];
        depth[n] = d;
        ns[n] = sc;
        if (d < D) {
            fs[nf] = ns[n] + lp[d * K]; fd[nf] = d + 1; fr[nf] = 0; fp[nf] = n; fq[nf] = seq++; ++nf;
        }
        if (r + 1 < K) {
            fs[nf] = ns[par] + lp[(d - 1) * K + r + 1]; fd[nf] = d; fr[nf] = r + 1; fp[nf] = par; fq[nf] = seq++; ++nf;
        }
        ++n;
    }
    free(fs); free(fd); free(fr); free(fp); free(fq); free(ns);
    return rc;
}

/*
 * Per-head projection around the absorbed attention ([P1] "The Thinking
 * Process: A Window into Engineering Deliberation": W_UK is absorbed into
 * the query, q_lat[h] = q_nope[h] @ W_UK[h]; the latent output returns to
 * the head's value space through W_UV[h].  [P1] "The Output Knowledge: What
 * This Message Creates": every projection is y = x @ W with W stored
 * [in, out]).  Rows r = t*H + h, t in [0, M) (token-major, head-minor, the
 * attention's query row order):
 *   y[r][n] = sum_{k=0}^{K-1} x[r][k] * W[h][k][n]
 * x row r starts at x + r*ld_x; W is [H][K][n_out] row-major; y is dense
 * [M*H][n_out].  x and W may be fp32, bf16 or fp64 (dtype codes 0, 1, 2).
 */
int orc_head_proj(int64_t M, int H, int K, int n_out, const void* x, int x_dtype, int64_t ld_x,
                  const void* w, int w_dtype, double* y) {
    if (M < 0 || H < 1 || K < 1 || n_out < 1 || ld_x < K || !x || !w || !y) return -1;
    if (x_dtype < 0 || x_dtype > 2 || w_dtype < 0 || w_dtype > 2) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < M * H; ++r) {
        int h = (int)(r % H);
        for (int n = 0; n < n_out; ++n) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += orc_load(x, x_dtype, r * ld_x + k) *
                       orc_load(w, w_dtype, ((int64_t)h * K + k) * n_out + n);
            y[r * n_out + n] = acc;
        }
    }
    return 0;
}

/* Number of OpenMP threads the oracle runs with (for reporting). */
int orc_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
