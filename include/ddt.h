/*
 * ddt.h -- C ABI of libddt.so: the data-parallel hot path of one DDTree
 * verify step for an MLA model, on one MI355X (gfx950).
 *
 * The step, as described on the pages
 *   "The Architecture of Pragmatic Ambition: Building a Native C++ Inference
 *    Engine for Kimi K2.6" (below: [Ambition]) and
 *   "The Architectural Keystone: Writing the Model Header for a Native
 *    DDTree Inference Engine" (below: [Keystone]),
 * is: parent array -> ancestor mask; tree-verify attention in absorbed MLA
 * form over the committed latent cache plus the tree nodes; target argmax;
 * greedy tree acceptance; compaction of the accepted path's latents.
 *
 * Conventions for every call:
 *  - Pointers are caller-owned DEVICE memory unless the name ends in _host.
 *    Nothing here allocates device memory.  Buffers a call needs beyond its
 *    inputs and outputs are passed in as a caller-owned workspace, sized by
 *    the matching *_workspace query.
 *  - Every call is asynchronous on `stream` (0 = the null stream) and
 *    returns DDT_OK or a negative ddt_status synchronously.  Argument errors
 *    that the host can see (null pointers, sizes out of range, unsupported
 *    shapes or dtypes, misalignment, a workspace that is too small) return
 *    an error before anything is launched.  Errors that depend on device
 *    data (an invalid tree) are reported through device-side flags.
 *  - Calls keep no state between invocations and may be made from several
 *    host threads on different streams.  Calls that write the same buffers
 *    must be ordered by the caller.
 *  - Floating point data is fp32 (DDT_F32) or bf16 (DDT_BF16, stored as
 *    16-bit patterns); accumulation is always fp32.
 */
#ifndef DDT_H
#define DDT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DDT_OK = 0,
    DDT_EINVAL = -1,       /* null pointer, size or stride out of range, misalignment */
    DDT_EUNSUPPORTED = -2, /* shape / dtype combination not built into the library   */
    DDT_EWORKSPACE = -3,   /* workspace missing or smaller than the query returned   */
    DDT_EHIP = -4          /* a HIP runtime call or kernel launch failed              */
} ddt_status;

typedef enum { DDT_F32 = 0, DDT_BF16 = 1 } ddt_dtype;

#define DDT_MAX_NODES 1024 /* budget + 1 */
#define DDT_MAX_BATCH 128  /* requests per verify-attention call */

/* Library version (major*10000 + minor*100 + patch) and a status name. */
int ddt_version(void);
const char* ddt_status_string(int status);

/*
 * Ancestor mask of each request's draft tree.
 *
 * [Ambition], section "The Decision Architecture": prefill, decode and tree
 * verification share one attention and differ only in the mask; in tree
 * verification a node sees the committed prefix and, inside the tree, only
 * its own ancestors.  A node also sees itself (so a chain-shaped tree is
 * causal attention and a one-node tree is plain decode).
 *
 * parents  [B][N] int32: parents[b][0] = -1 (root), parents[b][i] in [0, i).
 * mask     [B][N][W] uint64, W = ceil(N/64): bit (j % 64) of word j / 64 of
 *          row (b, i) is set iff node j is i or an ancestor of i.
 * depth    [B][N] int32 or NULL: edges from node i to the root.
 * tree_err [B] int32 or NULL: 0 for a valid tree, 1 otherwise; an invalid
 *          request gets an all-zero mask and depth -1.
 * 1 <= N <= DDT_MAX_NODES, B >= 0 (B = 0 launches nothing).
 */
int ddt_build_mask(const int32_t* parents, int B, int N, uint64_t* mask, int32_t* depth,
                   int32_t* tree_err, hipStream_t stream);

/*
 * Shape and layout of a tree-verify attention call.
 *
 * Queries: flat row r = (b*N + i)*H + h (node-major, head-minor).  The
 * absorbed no-rope query q_lat (d_lat wide) of row r starts at
 * q_lat + r*ld_ql and its rope part q_pe (d_rope wide) at q_pe + r*ld_qp
 * (elements).  [Ambition], section "The Thinking Process": absorbing W_UK
 * into the query turns q_nope . (W_UK c_kv) into q_lat . c_kv, so the keys
 * and values are the cached latents themselves.
 *
 * Cache: [Keystone], section "What the Header Declares": per token the
 * cache keeps the latent c_kv (d_lat = kv_lora_rank) and the decoupled rope
 * key k_pe (d_rope).  Cache row t of request b is pool row kv_base[b] + t;
 * its c_kv starts at ckv + row*ld_ckv and its k_pe at kpe + row*ld_kpe.  The
 * usual layout interleaves them: kpe = ckv + d_lat, ld_ckv = ld_kpe =
 * d_lat + d_rope.  [Keystone], section "The Reasoning That Preceded the
 * Header": the committed prefix occupies rows [0, P_b) and the N tree nodes
 * (root = last committed token, recomputed) occupy rows P_b .. P_b+N-1, so
 * node j is key P_b + j and a request has T_b = P_b + N keys.
 *
 * scale multiplies the full score q_lat.c_kv + q_pe.k_pe before softmax;
 * it must be positive and finite (DDT_EINVAL otherwise).
 * kv_chunk: keys per split of the key range (rounded up to a multiple of
 * 32); 0 lets the library choose.  Results do not depend on it beyond
 * rounding: the partial outputs of a split request pass through the
 * workspace in fp32 (accumulation stays fp32 from the products to the
 * merged output).
 *
 * Built instances (d_lat, d_rope, dtype): (512, 64, BF16), (64, 16, F32).
 * Alignment: q_lat, q_pe, ckv, kpe 16-byte aligned; every row stride times
 * the element size a multiple of 16 bytes, and below 2 GiB for ckv and kpe.
 *
 * Paged cache (block_table non-NULL).  [Keystone], section "Assumptions
 * Embedded in the Design": one-token pages leave the cache fragmented,
 * which the pages name a real performance problem; larger pages named by a
 * block table keep a request's slots in page-sized runs.  Slot t of
 * request b is then pool row
 *   block_table[b*bt_ld + t / page_size] * page_size + t % page_size
 * (the pool row stride stays ld_ckv / ld_kpe) and kv_base is not read (it
 * may be NULL).  page_size: a power of two in [32, 65536], with a page's
 * bytes (page_size times the row stride of c_kv, and of k_pe) below 4 GiB;
 * bt_ld >= ceil((P_b + N) / page_size) for every request (DDT_EINVAL
 * otherwise).
 * The table entries (device int32, caller-owned) must name pages inside
 * the pool: they are not checked.  Zero-initialised fields (NULL table)
 * give the contiguous layout.  ddt_verify_attn, ddt_verify_attn_argmax and
 * ddt_verify_step (attention, acceptance and compaction) take either; the
 * paged form is built for the bf16 (512, 64) instance (DDT_EUNSUPPORTED
 * otherwise) and has the contiguous form's work plan (any split length).
 *
 * Device-resident lengths (prefix_len_dev non-NULL).  [Keystone], section
 * "The Reasoning That Preceded the Header": the committed length advances
 * on the device every step (by accept_len + 1 <= N).  With prefix_len_dev
 * set, prefix_len_host[b] is only an upper bound: the launch is planned,
 * validated and sized (workspace, block-table width) for the bounds, and
 * the kernels read request b's committed length P_b = min(prefix_len_dev[b],
 * prefix_len_host[b]) (negative values as 0) from device memory when they
 * run, so a caller can enqueue or capture several steps without reading the
 * lengths back.  Results are those for the lengths P_b; key splits past
 * P_b + N contribute nothing; no cache row at or past P_b + N (nor any page
 * past it) is read.  prefix_len_dev must stay unchanged while the call's
 * kernels run (ddt_verify_step updates acc->new_prefix_len in its last
 * launch, after the attention).
 */
typedef struct {
    int B, H, N;
    int d_lat, d_rope;
    int dtype; /* ddt_dtype */
    float scale;
    int kv_chunk;
    int64_t ld_ql, ld_qp;
    int64_t ld_ckv, ld_kpe;
    const int32_t* block_table; /* [B][bt_ld] page numbers, or NULL (contiguous) */
    int64_t bt_ld;
    int page_size;
    const int32_t* prefix_len_dev; /* [B] device committed lengths, or NULL */
} ddt_attn_desc;

/* Workspace bytes ddt_verify_attn needs for this shape and these prefix
 * lengths (host array [B]); may be 0.  The workspace must be 256-byte
 * aligned; it is scratch between the attention's two launches (no zeroing
 * needed), and concurrent calls must not share one. */
int ddt_verify_workspace(const ddt_attn_desc* d, const int32_t* prefix_len_host, size_t* bytes);

/* Work plan of ddt_verify_attn for this shape and these host lengths, on
 * the host (no device work): the split-KV decomposition of the attention
 * below.  Request b's keys [0, P_b + N) are cut into splits of *chunk keys
 * whose partial results the merge combines exactly; a work item is one
 * split of one request for one row tile of 64 query rows, one per
 * attention workgroup.  *n_blocks: attention workgroups the launch starts
 * (work items plus workgroups that only pad the deal to the XCDs);
 * nsplit [B] (may be NULL): splits of each request; *n_items: work items;
 * items [cap][6] int32 (may be NULL): per work item, in workgroup order,
 * (workgroup, request, split, row tile, first key, end key).  Host arrays,
 * caller-owned.  DDT_EINVAL when items is given and cap < *n_items (the
 * counts are still set), or as ddt_verify_workspace.  For schedulers that
 * size launches and for tests of the decomposition. */
int ddt_verify_plan(const ddt_attn_desc* d, const int32_t* prefix_len_host, int* n_blocks, int* chunk,
                    int32_t* nsplit, int32_t* items, int cap, int* n_items);

/*
 * Tree-verify attention, absorbed MLA form.  For every (b, i, h):
 *   visible keys V = [0, P_b) u {P_b + j : mask bit j of row (b, i) set}
 *   s_t  = scale * (q_lat . c_kv[t] + q_pe . k_pe[t])
 *   out  = sum_{t in V} softmax(s)_t c_kv[t]          [B][N][H][d_lat], dtype
 *   lse  = ln sum_{t in V} exp(s_t)                   [B][N][H] fp32
 * out rows are contiguous (row stride d_lat).  prefix_len_host [B] is read
 * on the host during the call (it plans the work split); kv_base [B] int64
 * and mask (from ddt_build_mask) are device arrays.  Keys past T_b are never
 * read; nor are tree keys past a row's own node (nodes are numbered
 * parents-first, so a mask bit j > i is never set by ddt_build_mask, and a
 * caller-built mask must not set one).  Accumulation and softmax are fp32;
 * probabilities enter the value product in the input dtype.  Requires
 * B <= DDT_MAX_BATCH,
 * N <= DDT_MAX_NODES, P_b >= 0.
 */
int ddt_verify_attn(const ddt_attn_desc* d, const void* q_lat, const void* q_pe, const void* ckv,
                    const void* kpe, const int64_t* kv_base, const int32_t* prefix_len_host,
                    const uint64_t* mask, void* out, float* lse, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/*
 * ddt_verify_attn for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, plan, kernels and results as
 * ddt_verify_attn, without the workspace: the split partials go to a
 * device array inside the library, DDT_NOALLOC_SCRATCH_BYTES bytes per
 * device (held by every device the library runs on until the process
 * ends).  A call whose partials need more than that (the figure
 * ddt_verify_workspace returns) fails with DDT_EWORKSPACE before anything
 * is launched; use ddt_verify_attn with a workspace then.  Nothing is
 * allocated and nothing needs clearing (every partial is written before
 * the merge reads it).  All calls on one device share that device's
 * array, so calls that overlap on one device (different streams or host
 * threads without ordering) race: the caller must order them.
 * ddt_verify_noalloc_scratch_bytes() returns DDT_NOALLOC_SCRATCH_BYTES.
 */
#define DDT_NOALLOC_SCRATCH_BYTES (64u << 20)
int ddt_verify_attn_noalloc(const ddt_attn_desc* d, const void* q_lat, const void* q_pe, const void* ckv,
                            const void* kpe, const int64_t* kv_base, const int32_t* prefix_len_host,
                            const uint64_t* mask, void* out, float* lse, hipStream_t stream);
size_t ddt_verify_noalloc_scratch_bytes(void);

/*
 * Target argmax.  [Ambition], section "The Decision Architecture": greedy
 * token selection from logits.  idx[r] = lowest index of the maximum of row
 * r of logits (row r at logits + r*ld, V entries, dtype fp32 or bf16).  -0
 * and +0 compare equal; a NaN counts as larger than every number, so the
 * first NaN wins.  rows >= 0, 1 <= V <= 2^31-1, ld >= V.
 * Workspace: ddt_argmax_workspace bytes (16-byte aligned), which must be
 * zero-filled before the first call; every call leaves it zero-filled
 * again, so it can be reused without clearing.  Concurrent calls must not
 * share one workspace.
 */
int ddt_argmax_workspace(int64_t rows, int64_t V, size_t* bytes);
int ddt_argmax(const void* logits, int dtype, int64_t rows, int64_t V, int64_t ld, int32_t* idx,
               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Per-depth draft candidates.  [Ambition], section "The Knowledge
 * Architecture": the tree builder takes the drafter's per-depth top-k.
 * For each row r of fp32 draft logits (row at logits + r*ld, V entries):
 *   ids[r][0..K)  = the K largest entries, by value (descending), equal
 *                   values by index (ascending)                   int32
 *   logp[r][k]    = logits[r][ids[r][k]] - lse(row), the log-softmax over
 *                   the whole row, computed in fp32 (|error| < 1e-4 at
 *                   V = 163840 against fp64)                     fp32
 * Finite logits; 1 <= K <= 16, K <= V <= 2^20, ld >= V.
 * Workspace: ddt_draft_topk_workspace bytes (16-byte aligned), scratch
 * between its launches (no zeroing needed).
 */
int ddt_draft_topk_workspace(int64_t rows, int64_t V, int K, size_t* bytes);
int ddt_draft_topk(const float* logits, int64_t rows, int64_t V, int64_t ld, int K, int32_t* ids, float* logp,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Best-first draft tree.  [Ambition], section "The Knowledge Architecture"
 * (a best-first tree from the drafter's per-depth top-k); [Keystone],
 * section "The Context: Building an Engine from First Principles" (a GPU
 * builder in place of a per-request heap on the CPU).  Per request b,
 * candidates: the token of rank r at depth d is ids[b][d-1][r] with
 * log-probability logp[b][d-1][r] (ddt_draft_topk's layout with rows
 * b*D + d-1).  A node's score is its parent's plus its own log-probability
 * (an fp32 addition; the root, root_tokens[b], scores 0).  The frontier
 * starts with (depth 1, rank 0) under the root; repeatedly the frontier
 * candidate with the highest score (then the lower depth, then the earlier
 * insertion) becomes the next node, and its first child (depth d+1, rank 0;
 * if d < D) and next sibling (depth d, rank r+1; if r+1 < K) enter the
 * frontier, in that order.  Outputs [B][budget+1] int32, nodes numbered in
 * that order: parents (root -1, parents[i] < i), tokens (root first),
 * depth.  1 <= D <= 255, 1 <= K, D*K <= 4096, 0 <= budget < DDT_MAX_NODES,
 * and the candidates must suffice (sum of K^d over d = 1..D >= budget):
 * otherwise DDT_EINVAL.  One wavefront per request.
 */
int ddt_best_first_tree(const int32_t* ids, const float* logp, int B, int D, int K, int budget,
                        const int32_t* root_tokens, int32_t* parents, int32_t* tokens, int32_t* depth,
                        hipStream_t stream);

/*
 * Tree-verify attention and target argmax in one launch: the results of
 * ddt_verify_attn and of ddt_argmax (same arguments, same outputs, same
 * workspace contracts).  The two are independent; the argmax runs as extra
 * workgroups dispatched after every attention workgroup, so on a small
 * batch it fills the CUs the attention leaves idle instead of following it.
 */
typedef struct {
    const void* logits;     /* [rows][ld], dtype fp32 or bf16                  */
    int dtype;              /* ddt_dtype                                       */
    int64_t rows, V, ld;
    int32_t* idx;           /* [rows] device, lowest index of the row maximum  */
    void* workspace;        /* ddt_argmax_workspace bytes, zero before first use */
    size_t workspace_bytes;
} ddt_argmax_task;
int ddt_verify_attn_argmax(const ddt_attn_desc* d, const void* q_lat, const void* q_pe, const void* ckv,
                           const void* kpe, const int64_t* kv_base, const int32_t* prefix_len_host,
                           const uint64_t* mask, void* out, float* lse, void* workspace, size_t workspace_bytes,
                           const ddt_argmax_task* am, hipStream_t stream);

/*
 * Greedy tree acceptance.  [Ambition], section "The Knowledge
 * Architecture": walk the verified tree greedily for the longest path that
 * matches the target's predictions.  target_ids[b][c] is the target's
 * greedy token after node c.  From the root, repeatedly move to the
 * lowest-numbered child k of the current node c with
 * draft_ids[b][k] == target_ids[b][c]; stop when none matches.
 *   path[b]       = [0, k1, k2, ...] then -1            [B][N] int32
 *   accept_len[b] = number of accepted draft nodes       [B] int32
 *   tokens[b]     = draft ids along the path, then the bonus token
 *                   target_ids[b][last], then -1       [B][N] int32
 * draft_ids[b][0] is not read.  parents as for ddt_build_mask; on an
 * invalid tree the walk still ends (it only moves to higher node numbers).
 */
int ddt_greedy_accept(const int32_t* target_ids, const int32_t* draft_ids, const int32_t* parents,
                      int B, int N, int32_t* accept_len, int32_t* path, int32_t* tokens,
                      hipStream_t stream);

/*
 * KV compaction and length update.  [Keystone], section "The Reasoning That
 * Preceded the Header": after acceptance the accepted path's latents, the
 * recomputed root included, are gathered into contiguous slots and the
 * cache length advances; section "Mistakes and Iterative Refinement":
 * source and destination slots alias, which must not race.
 * For request b with P = prefix_len[b] and k = accept_len[b]:
 *   cache row P+j <- old cache row P+path[b][j], j = 0..k (c_kv and k_pe),
 *   prefix_len[b] <- P + k + 1        (device array, updated in place),
 *   src_slot[b][j] = P + path[b][j] for j <= k, else -1   (NULL allowed).
 * Rows from P+k+1 on are left as they were.  A request whose accept_len is
 * outside [0, N), whose path is not 0 followed by increasing node numbers
 * below N, or whose slots P .. P+path[k] cannot be mapped (P < 0; paged:
 * a slot past the request's table row) is left untouched (src_slot all -1,
 * prefix_len unchanged); these checks run on the device.
 * Layout arguments as in ddt_attn_desc; row strides times the element size
 * and the pointers must be 4-byte aligned.
 */
int ddt_compact_kv(void* ckv, int64_t ld_ckv, void* kpe, int64_t ld_kpe, int dtype, int d_lat,
                   int d_rope, const int64_t* kv_base, int32_t* prefix_len, const int32_t* path,
                   const int32_t* accept_len, int B, int N, int32_t* src_slot, hipStream_t stream);

/*
 * ddt_compact_kv on a paged cache (see ddt_attn_desc): slot t of request b
 * is pool row block_table[b*bt_ld + t/page_size]*page_size + t%page_size.
 * page_size a power of two in [1, 65536], bt_ld >= 1.  A request whose
 * slots P .. P+path[k] run past its table row (bt_ld pages) is left
 * untouched, like an invalid path; the page numbers themselves are device
 * data and must name pages inside the pool (not checked).  Otherwise as
 * ddt_compact_kv.
 */
int ddt_compact_kv_paged(void* ckv, int64_t ld_ckv, void* kpe, int64_t ld_kpe, int dtype, int d_lat, int d_rope,
                         const int32_t* block_table, int64_t bt_ld, int page_size, int32_t* prefix_len,
                         const int32_t* path, const int32_t* accept_len, int B, int N, int32_t* src_slot,
                         hipStream_t stream);

/*
 * Acceptance and compaction in one launch.  [Ambition], section "The
 * Knowledge Architecture"; [Keystone], sections "The Reasoning That
 * Preceded the Header" and "Mistakes and Iterative Refinement".  The same
 * results as ddt_greedy_accept followed by ddt_compact_kv on the path it
 * found: one workgroup per request walks the tree, writes accept_len, path
 * and tokens, then moves the accepted rows.  The committed lengths are read
 * from prefix_len and the advanced ones written to new_prefix_len (device
 * arrays of B; the same array for an in-place update).  Other arguments,
 * layouts and errors as for those two calls (the walk's path is always a
 * valid compaction path; a request whose slots cannot be mapped still gets
 * its acceptance outputs, and new_prefix_len = prefix_len with no rows
 * moved).
 */
int ddt_accept_compact(const int32_t* target_ids, const int32_t* draft_ids, const int32_t* parents, int B, int N,
                       int32_t* accept_len, int32_t* path, int32_t* tokens, void* ckv, int64_t ld_ckv, void* kpe,
                       int64_t ld_kpe, int dtype, int d_lat, int d_rope, const int64_t* kv_base,
                       const int32_t* prefix_len, int32_t* new_prefix_len, int32_t* src_slot, hipStream_t stream);

/*
 * ddt_accept_compact on a paged cache, as ddt_compact_kv_paged addresses it
 * (slot t of request b at pool row block_table[b*bt_ld + t/page_size] *
 * page_size + t%page_size; page_size a power of two in [1, 65536], bt_ld >=
 * 1).  A request whose slots P .. P+path[k] run past its table row gets its
 * acceptance outputs and new_prefix_len = prefix_len, with no rows moved;
 * the page numbers must name pages inside the pool (not checked).
 * Otherwise as ddt_accept_compact.
 */
int ddt_accept_compact_paged(const int32_t* target_ids, const int32_t* draft_ids, const int32_t* parents, int B,
                             int N, int32_t* accept_len, int32_t* path, int32_t* tokens, void* ckv, int64_t ld_ckv,
                             void* kpe, int64_t ld_kpe, int dtype, int d_lat, int d_rope, const int32_t* block_table,
                             int64_t bt_ld, int page_size, const int32_t* prefix_len, int32_t* new_prefix_len,
                             int32_t* src_slot, hipStream_t stream);

/*
 * One verify step after the mask: tree-verify attention, target argmax,
 * greedy acceptance and KV compaction with the length update, in two
 * launches.  [Ambition], sections "The Thinking Process", "The Decision
 * Architecture" and "The Knowledge Architecture"; [Keystone], sections
 * "What the Header Declares" and "The Reasoning That Preceded the Header".
 * Results are those of
 * ddt_verify_attn_argmax followed by ddt_accept_compact with
 * target_ids = am->idx and the attention's cache (ckv, kpe, kv_base, dtype,
 * d_lat, d_rope, strides).  The first launch runs the attention with the
 * argmax on idle CUs; the second runs the split merge with one
 * acceptance + compaction workgroup per request beside it (the compaction
 * writes the cache only after the attention has read it).
 * am->rows must be B*N (one target row per tree node, request-major).
 * acc->prefix_len (device) must hold the same lengths as prefix_len_host,
 * or lengths at most those when d->prefix_len_dev is set (normally
 * d->prefix_len_dev == acc->prefix_len).
 * mask may be NULL when N <= 128: the attention then derives each row's
 * ancestor bits from acc->parents itself (pointer doubling across a
 * wavefront), so the step needs no ddt_build_mask launch; a request whose
 * tree is invalid sees no tree keys, as with ddt_build_mask's all-zero
 * mask.  (Depth and tree_err are then not produced.)  A NULL mask with
 * N > 128 is DDT_EINVAL.  Other errors as for the calls it replaces.
 */
typedef struct {
    const int32_t* draft_ids;   /* [B][N] device                               */
    const int32_t* parents;     /* [B][N] device                               */
    int32_t* accept_len;        /* [B] out                                     */
    int32_t* path;              /* [B][N] out                                  */
    int32_t* tokens;            /* [B][N] out                                  */
    const int32_t* prefix_len;  /* [B] device, committed lengths               */
    int32_t* new_prefix_len;    /* [B] out, advanced lengths (may be prefix_len) */
    int32_t* src_slot;          /* [B][N] out, or NULL                         */
} ddt_accept_task;
int ddt_verify_step(const ddt_attn_desc* d, const void* q_lat, const void* q_pe, void* ckv, void* kpe,
                    const int64_t* kv_base, const int32_t* prefix_len_host, const uint64_t* mask, void* out,
                    float* lse, void* workspace, size_t workspace_bytes, const ddt_argmax_task* am,
                    const ddt_accept_task* acc, hipStream_t stream);

/*
 * Per-head projections around the absorbed attention.  [Ambition], section
 * "The Thinking Process: A Window into Engineering Deliberation": W_UK is
 * absorbed into the query, q_lat[h] = q_nope[h] @ W_UK[h] (and the latent
 * output is brought back to the head's value space by W_UV[h]); section
 * "The Output Knowledge: What This Message Creates": projections are
 * y = x @ W with W stored [in, out], and the absorbed weights w_kc, w_vc
 * are given directly.
 *
 * ddt_proj_pack_weight: w = [H][K][n_out] (row-major, [in, out] per head)
 * -> packed, the same number of bytes (H*K*n_out*2) in the library's
 * operand order (opaque; only ddt_head_proj reads it).  Weights are static:
 * pack once, reuse for every call.  packed must not alias w and must be
 * 16-byte aligned.
 *
 * ddt_head_proj: for every row r = t*H + h, t in [0, M) (token-major,
 * head-minor: the attention's query row order, with t = b*N + i):
 *   y[r][n] = sum_k x[r][k] * W[h][k][n],  n in [0, n_out)
 * x row r starts at x + r*ld_x, y row r at y + r*ld_y (elements); only
 * columns [0, n_out) of y are written, so q_lat can be written straight
 * into the first d_lat columns of the concatenated q_lat|q_pe rows
 * (ld_y = d_lat + d_rope).  Uses: q_lat = ddt_head_proj(q_nope, w_kc)
 * with K = d_nope, n_out = d_lat; o = ddt_head_proj(out_lat, w_vc) with
 * K = d_lat, n_out = d_v.  bf16 in and out (fp32 accumulation, output
 * rounded to nearest even).
 * Supported: dtype DDT_BF16 (else DDT_EUNSUPPORTED); K in {64, 128, 256,
 * 512}; n_out a multiple of 32 in [32, 4096]; ld_x >= K, ld_y >= n_out,
 * both multiples of 8; x, y, w_packed 16-byte aligned; M >= 0 (M = 0 is a
 * no-op, and x, y may then be null); x and y must not overlap.  Otherwise
 * DDT_EINVAL.
 */
int ddt_proj_pack_weight(const void* w, int H, int K, int n_out, int dtype, void* packed, hipStream_t stream);
int ddt_head_proj(const void* x, int64_t ld_x, const void* w_packed, int M, int H, int K, int n_out, int dtype,
                  void* y, int64_t ld_y, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DDT_H */
