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
//  * A workgroup owns one work item = (request, key split, 64 query rows)
//    and specialises its four wavefronts (one per SIMD).  Key tiles of 32
//    latent rows (576 columns) reach LDS by LDS-DMA (buffer_load ... lds,
//    issued as inline asm with hand-built buffer descriptors; rows past the
//    split end fall outside the descriptor and read as zeros) into a ring of
//    four slots, and every tile is shared by all 64 rows.
//  * Score wavefronts (0, 1; 32 rows each, queries resident in AGPRs)
//    compute S^T = K . Q^T on MFMA 32x32x16 bf16 (32x32x2 f32 for fp32
//    data) with the K tile as the A operand, so a query row's scores land
//    in one lane pair and its maximum needs one permlane swap.  They apply
//    the ancestor bits (from the mask, or derived in the kernel from the
//    parents by pointer doubling across the wavefront), take the softmax
//    against a fixed per-row reference (a second pass over the split if a
//    later scaled score exceeds it by more than 64 in log2) and publish
//    bf16 P^T to LDS.
//    The softmax of tile j-1 runs on the VALU under the MFMAs of tile j.
//  * Value wavefronts (2, 3) each own all 64 rows and half of the 512 value
//    columns: O^T += V^T . P^T with V^T read by transposing LDS reads
//    (ds_read_b64_tr_b16), each fragment feeding both row groups; row sums
//    come from an extra MFMA against ones.  They issue the tile loads (and,
//    for long key streams, 4-byte L2 touches of tile j+2) between MFMAs.
//  * Each request's key range is cut into splits (the host picks the chunk
//    that minimises an estimate of the launch's finish time) and work items
//    are dealt to the XCDs so that row tiles of one split share an L2.
//    Split partials (unnormalised, fp32, MFMA register order) with each
//    row's softmax reference and row sum go to the
//    workspace; verify_combine weighs, sums and normalises them.  A request with one split writes its output directly.
//  * Optional co-tasks: target-argmax workgroups on the CUs the attention
//    leaves idle (verify_split), and acceptance + compaction workgroups
//    beside the merge (verify_combine).
//  * Paged caches: a split's page numbers stream through a small ring of
//    LDS windows (filled by LDS-DMA two windows ahead of the tiles), and
//    each tile takes its pool rows from one page (a tile never crosses a
//    page).
#include <math.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "argmax_scan.h"
#include "common.h"
#include "tree_tail.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) short4v lds_short4v;

constexpr int KT = 32;               // keys per tile
constexpr int NW = 4;                // wavefronts per workgroup
constexpr int NGRP = 2;              // row groups of 32 query rows per workgroup
constexpr int ROWS_WG = 32 * NGRP;   // query rows per workgroup
constexpr int kThreads = 64 * NW;
constexpr int NSTAGE = 4;            // LDS ring depth (tiles resident or in flight)
constexpr int kMinChunk = 256;       // smallest automatic split (keys)
constexpr int kRsrcFlags = 0x00020000;  // raw 32-bit buffer descriptor word 3
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kSpan = 64.f;         // log2 headroom of the fixed softmax reference
#ifndef DDT_SCORE_AHEAD
#define DDT_SCORE_AHEAD 3
#endif
#ifndef DDT_VALUE_AHEAD
#define DDT_VALUE_AHEAD 2
#endif
constexpr int kScoreAhead = DDT_SCORE_AHEAD;  // score fragment reads run this many MFMAs ahead
constexpr int kValueAhead = DDT_VALUE_AHEAD;  // value fragments are read this many fragments ahead

// A key tile in LDS is two regions, each row-major with 16-byte chunks:
//   A: c_kv,  KT rows x CA chunks    (CA = d_lat * elem / 16)
//   B: k_pe,  KT rows x CB chunks    (CB = d_rope * elem / 16)
// Chunk c of row r is stored at chunk c ^ sw(r) of that row.  Tiles are
// filled by LDS-DMA (buffer_load ... lds): each 64-lane instruction writes
// 64 consecutive chunks of one region, so every instruction reads from one
// source array through one buffer descriptor.
template <typename T>
struct Traits;

// bf16: MFMA 32x32x16, 8 k-values per lane.  Swizzles over the 16 LDS bank
// groups of 16 bytes: region A rows are 1 KB and swA(r) = 4*(r%4) + (r/4)%4
// keeps both the score reads (16 consecutive rows, one chunk) and the
// transposed value reads (4 consecutive rows x 4 consecutive chunks) free of
// conflicts; region B rows are 128 B and swB(r) = (r/2)%8 does the same for
// the score reads.
template <>
struct Traits<uint16_t> {
    static constexpr int KPL = 8;
    using Frag = bf16x8;
    __device__ static floatx16 mfma(Frag a, Frag b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    // c += a.b with c pinned to AGPRs (the value accumulators take all of
    // them); VALU reads of c need mfma_settle() first, VALU writes of c
    // need it before the next product.
    __device__ static void mfma_acc(Frag a, Frag b, floatx16& c) {
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    }
    __device__ static Frag global_frag(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
    __device__ static Frag from_f32(const float* v) {
        Frag r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = static_cast<__bf16>(v[e]);
        return r;
    }
    __device__ static constexpr int swA(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }
    __device__ static constexpr int swB(int r) { return (r >> 1) & 7; }

    // Per-lane byte offsets inside a ring slot; each fragment address is one
    // of these plus a compile-time immediate.
    struct Lane {
        uint32_t ka[8];     // score A operand, c_kv depth chunk 2ks+g: ka[ks & 7] + 256*(ks >> 3)
        uint32_t kb[4];     // score A operand, k_pe depth chunk 2m+g
        uint32_t v[2][4];   // value A operand: v[hi][c & 3] + 16*CA*16*kk + 256*(c >> 2)
    };
    template <int DL, int DR>
    __device__ static Lane lane_offsets(int lane) {
        constexpr int CA = DL / 8, CB = DR / 8;
        static_assert(CA % 16 == 0 && CB == 8, "bf16 layout: c_kv rows of whole 16-chunk groups, 8-chunk k_pe rows");
        const int g = lane >> 5, l32 = lane & 31, r = l32;
        Lane L;
#pragma unroll
        for (int m = 0; m < 8; ++m) L.ka[m] = (uint32_t)((r * CA + ((2 * m + g) ^ swA(r))) * 16);
#pragma unroll
        for (int m = 0; m < 4; ++m) L.kb[m] = (uint32_t)((KT * CA + r * CB + ((2 * m + g) ^ swB(r))) * 16);
        // Transposed value reads: in each 16-lane group, source lane a + 4k
        // reads row 16kk + 8hi + 4g + k, columns 32c + 16half + 4a .. +3; the
        // hardware hands lane 4a + e the 4 rows (keys) of column
        // 32c + 16half + 4a + e.  swA of that row is 4k + 2hi + g.
        const int grp = lane >> 4, s = lane & 15, a = s & 3, k = s >> 2, half = grp & 1;
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) {
            const int row = 8 * hi + 4 * g + k;
#pragma unroll
            for (int c3 = 0; c3 < 4; ++c3) {
                const int chunk = (4 * c3 + 2 * half + (a >> 1)) ^ (4 * k + 2 * hi + g);
                L.v[hi][c3] = (uint32_t)((row * CA + chunk) * 16 + (a & 1) * 8);
            }
        }
        return L;
    }
    template <int DL, int DR>
    __device__ static Frag k_frag(const char* slot, const Lane& L, int ks) {
        constexpr int NKA = DL / 16;
        const char* p = ks < NKA ? slot + L.ka[ks & 7] + 256 * (ks >> 3) : slot + L.kb[ks - NKA];
        return *reinterpret_cast<const bf16x8*>(p);
    }
    // value A operand, 32 output columns [32c, 32c+32), key k-step kk (keys 16kk .. 16kk+15)
    template <int DL, int DR>
    __device__ static Frag v_frag(const char* slot, const Lane& L, int c, int kk) {
        constexpr int CA = DL / 8;
        const uint32_t imm = 16 * CA * 16 * kk + 256 * (c >> 2);
        const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(slot + L.v[0][c & 3] + imm));
        const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(slot + L.v[1][c & 3] + imm));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
};

// fp32: MFMA 32x32x2, 1 k-value per lane, no swizzle (small shapes only).
template <>
struct Traits<float> {
    static constexpr int KPL = 1;
    using Frag = float;
    __device__ static floatx16 mfma(Frag a, Frag b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    __device__ static void mfma_acc(Frag a, Frag b, floatx16& c) {
        asm volatile("v_mfma_f32_32x32x2_f32 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    }
    __device__ static Frag global_frag(const float* p) { return *p; }
    __device__ static Frag from_f32(const float* v) { return v[0]; }
    __device__ static constexpr int swA(int) { return 0; }
    __device__ static constexpr int swB(int) { return 0; }
    struct Lane {
        uint32_t ka, kb, v;
    };
    template <int DL, int DR>
    __device__ static Lane lane_offsets(int lane) {
        const int g = lane >> 5, l32 = lane & 31;
        return Lane{(uint32_t)((l32 * DL + g) * 4), (uint32_t)((KT * DL + l32 * DR + g) * 4),
                    (uint32_t)((4 * g * DL + l32) * 4)};
    }
    // score A operand: key l32, depth 2ks + g
    template <int DL, int DR>
    __device__ static Frag k_frag(const char* slot, const Lane& L, int ks) {
        constexpr int NKA = DL / 2;
        const char* p = ks < NKA ? slot + L.ka + 8 * ks : slot + L.kb + 8 * (ks - NKA);
        return *reinterpret_cast<const float*>(p);
    }
    // value A operand: column 32c + l32 of the key whose score sits at
    // accumulator index kk of lane half g: key = 8*(kk/4) + 4g + kk%4.
    template <int DL, int DR>
    __device__ static Frag v_frag(const char* slot, const Lane& L, int c, int kk) {
        const int key = 8 * (kk >> 2) + (kk & 3);
        return *reinterpret_cast<const float*>(slot + L.v + (key * DL + 32 * c) * 4);
    }
};

// acc *= a, element by element, without moving the accumulator out of the
// registers it lives in (accumulation registers are not VALU operands).
__device__ inline void scale_acc(floatx16& acc, float a) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        float e = acc[k];
        float t;
        asm volatile(
            "v_accvgpr_read_b32 %1, %0\n\t"
            "v_mul_f32 %1, %2, %1\n\t"
            "v_accvgpr_write_b32 %0, %1"
            : "+a"(e), "=&v"(t)
            : "v"(a));
        acc[k] = e;
    }
}

// 24 wait states: more than any MFMA result needs before a VALU access of
// its registers, and more than any VALU write needs before an MFMA reads it.
__device__ inline void mfma_settle() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// max(a, b, c) without the NaN-quieting the compiler puts in front of
// fmaxf on values it cannot prove canonical (MFMA results).  Inline asm:
// an MFMA result needs mfma_settle() before it gets here.
__device__ inline float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
// The maximum of v over the lane pair (l, l xor 32): v_permlane32_swap
// hands every lane both v[l mod 32] and v[l mod 32 + 32].
__device__ inline float pair_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return max3f(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A raw buffer descriptor (stride 0) over [base, base + bytes): loads past
// the range return zeros.
__device__ inline u32x4 buffer_rsrc(const void* base, int bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
    r[2] = __builtin_amdgcn_readfirstlane((uint32_t)bytes);
    r[3] = (uint32_t)kRsrcFlags;
    return r;
}
__device__ inline uint32_t lds_addr(const void* p) {
    return (uint32_t)reinterpret_cast<uintptr_t>((const lds_void*)p);
}
// LDS-DMA of 16 bytes per lane: lane l's chunk at byte voff of the buffer
// goes to LDS address lds + 16 l (lds: wave-uniform, read from the first
// lane into M0).  Issued as inline asm, so the compiler
// neither orders it against LDS reads of other addresses (its alias
// analysis of LDS-DMA is conservative and would wait for every load) nor
// counts it: the callers wait for it with explicit vmcnt waits before the
// workgroup barrier that publishes the tile.
__device__ inline void dma16(u32x4 rsrc, uint32_t lds, uint32_t voff) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, 0 offen lds"
        :
        : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds))
        : "m0");
}

// LDS-DMA of 4 bytes per lane: lane l's word at byte voff of the buffer
// goes to LDS address lds + 4 l (offsets outside the descriptor's range
// deliver zeros).  Inline asm and uncounted by the compiler, like dma16.
__device__ inline void dma4(u32x4 rsrc, uint32_t lds, uint32_t voff) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %0, %1, 0 offen lds"
        :
        : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds))
        : "m0");
}

// Two LDS-DMAs of 16 bytes per lane under one M0: the second lands 2048
// bytes after the first in LDS, from byte voff1 + 2048 of the buffer (the
// instruction offset moves both addresses).
__device__ inline void dma16x2(u32x4 rsrc, uint32_t lds, uint32_t voff0, uint32_t voff1) {
    asm volatile(
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %2, 0 offen lds\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen offset:2048 lds"
        :
        : "v"(voff0), "v"(voff1), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds))
        : "m0");
}

// Touch 4 bytes per lane at rsrc + voff, delivered into LDS at `lds`
// (64 lanes x 4 bytes of scratch): pulls the lines into L2 with no register
// destination for the compiler to track.  Offsets outside the descriptor's
// range read nothing.
__device__ inline void l2_touch(u32x4 rsrc, uint32_t lds, uint32_t voff) { dma4(rsrc, lds, voff); }

// An opaque (empty) redefinition of a register value.
template <typename V>
__device__ inline void pin_reg(V& v) {
    asm volatile("" : "+v"(v));
}
// The same, defining the value in accumulation registers (MFMA operands can
// be read from there directly).
template <typename V>
__device__ inline void pin_acc(V& v) {
    asm volatile("" : "+a"(v));
}

// A wave-uniform pointer, pinned to scalar registers.
__device__ inline const char* uniform_ptr(const char* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

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
// Four fp32 values with a non-temporal hint: split partials are streamed to
// memory for the merge launch rather than kept in this XCD's L2 (measured
// 1.1 us off the attention launch at the K2-like head share).
__device__ inline void store4_nt_f32(float* dst, const float* v) {
    typedef float F4 __attribute__((ext_vector_type(4)));
    const F4 w = {v[0], v[1], v[2], v[3]};
    __builtin_nontemporal_store(w, reinterpret_cast<F4*>(dst));
}
// four consecutive fp32 values
__device__ inline float4 load4_f32(const float* src) { return *reinterpret_cast<const float4*>(src); }

// Wait until this wavefront's vector-memory loads (the LDS-DMA of later
// tiles, issued as inline asm the compiler does not count) have landed.
__device__ inline void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Ancestor bits (self included) of `node` in a tree of N <= 128 nodes
// whose parents are par[0..N) (the ancestor mask of "The Architecture of
// Pragmatic Ambition", section "The Decision Architecture", for one row),
// as two 64-bit words, by pointer doubling across the wavefront: lane l
// keeps nodes l and l + 64, each with the set of ancestors found so far and
// a jump to the first ancestor not yet in it.  A round ORs in the jump
// target's set and takes over its jump; the set then still holds exactly
// the ancestors below the jump, and the jump at least doubles its distance,
// so log2(depth) + 1 rounds finish.  A tree that is not valid (parents[0]
// != -1 or parents[i] outside [0, i)) gives no bits, like ddt_build_mask's
// all-zero mask.  Every lane of the wavefront must take part.
__device__ inline void tree_ancestors(const int32_t* __restrict__ par, int N, int node, uint64_t& w0,
                                      uint64_t& w1) {
    const int lane = threadIdx.x & 63;
    const int u1 = lane + 64;
    int j0 = lane < N ? par[lane] : -1;
    int j1 = u1 < N ? par[u1] : -1;
    const bool ok = (lane >= N || (lane == 0 ? j0 == -1 : (j0 >= 0 && j0 < lane))) &&
                    (u1 >= N || (j1 >= 0 && j1 < u1));
    w0 = 0;
    w1 = 0;
    if (__ballot(!ok) != 0) return;
    uint64_t a0 = 1ull << lane, a1 = 0;  // node lane: words 0 and 1 of its set
    uint64_t b0 = 0, b1 = 1ull << lane;  // node lane + 64
    if (N <= 64) {
        while (__ballot(j0 >= 0) != 0) {
            const int src = j0 < 0 ? 0 : j0;
            const uint64_t ta = __shfl(a0, src, 64);
            const int tj = __shfl(j0, src, 64);
            if (j0 >= 0) {
                a0 |= ta;
                j0 = tj;
            }
        }
        w0 = __shfl(a0, node, 64);
        return;
    }
    // (a shuffle returns the source lane's own register, so both nodes of
    // the source lane are fetched and the reader picks one)
    while (__ballot(j0 >= 0 || j1 >= 0) != 0) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            int& j = k == 0 ? j0 : j1;
            const int src = (j < 0 ? 0 : j) & 63;
            const bool hi = j >= 64;
            const uint64_t xa0 = __shfl(a0, src, 64), xa1 = __shfl(a1, src, 64);
            const uint64_t xb0 = __shfl(b0, src, 64), xb1 = __shfl(b1, src, 64);
            const int xj0 = __shfl(j0, src, 64), xj1 = __shfl(j1, src, 64);
            if (j >= 0) {
                const uint64_t x0 = hi ? xb0 : xa0, x1 = hi ? xb1 : xa1;
                if (k == 0) {
                    a0 |= x0;
                    a1 |= x1;
                } else {
                    b0 |= x0;
                    b1 |= x1;
                }
                j = hi ? xj1 : xj0;
            }
        }
    }
    const bool hi = node >= 64;
    const uint64_t ya0 = __shfl(a0, node & 63, 64), ya1 = __shfl(a1, node & 63, 64);
    const uint64_t yb0 = __shfl(b0, node & 63, 64), yb1 = __shfl(b1, node & 63, 64);
    w0 = hi ? yb0 : ya0;
    w1 = hi ? yb1 : ya1;
}

struct VerifyParams {
    const void* q_lat;
    const void* q_pe;
    const void* ckv;
    const void* kpe;
    ddt::SlotMap map;           // cache slot -> pool row (contiguous from kv_base, or paged)
    const int32_t* P_dev;       // committed lengths on the device (at most P[]), or null
    const uint64_t* mask;       // ancestor bits from ddt_build_mask, or null:
    const int32_t* parents;     // then each row's bits come from the parents (N <= 128)
    void* out;
    float* lse;
    void* ws_o;     // [slot][row group][DL/32][4][64][4] fp32, unnormalised partial outputs
    float2* ws_ml;  // [slot][ROWS_WG] (softmax reference m, log2 domain; row sum l) of the unnormalised partials
    int64_t ld_ql, ld_qp, ld_ckv, ld_kpe;
    int B, H, N, W, rows, row_tiles, chunk, total_wg;
    float scale_log2;
    int P[DDT_MAX_BATCH];
    int nsplit[DDT_MAX_BATCH];
    int wg_begin[DDT_MAX_BATCH + 1];  // partial-output slot of (b, split 0, row tile 0)
    // dispatch order: groups (b, split) of row tiles, cut into units of up
    // to unit_rows row tiles dealt to the XCDs round robin; whole-chunk
    // splits first (request-major), then each request's shorter last split,
    // longest first
    int full_gbegin[DDT_MAX_BATCH + 1];  // first whole-chunk group of request b
    int part_b[DDT_MAX_BATCH];           // request of the k-th last-split group
    int n_full_groups, n_units, unit_rows, units_per_group;
    int whole_blocks;  // blocks of the units dealt whole (a multiple of 8 units); the rest row by row
    int single_round;  // at most one workgroup per CU: XCD x takes a contiguous range of work items
    int rt_desc;       // deal a split's row tiles last first (large trees: later rows see more keys)
    // target argmax riding along in the same launch (workgroups n_attn ..)
    int n_attn;                 // attention workgroups (the rest are argmax workgroups)
    int am_wgs, am_dtype, am_vec;
    int64_t am_rows, am_V, am_ld, am_E;  // am_E: elements of the flattened rows x V range per workgroup
    const void* am_logits;
    int32_t* am_idx;
    ddt::RowSlot* am_slots;
    // acceptance + compaction riding along in the merge launch (workgroups 0 .. n_accept-1)
    int n_accept, acc_vec16;
    ddt::AcceptCompactArgs acc;
};

// Argmax workgroup `am_id` scans elements [am_id*E, (am_id+1)*E) of the
// rows x V logits taken as one flat range (equal shares for every
// workgroup); a row is split among the workgroups whose shares touch it and
// they merge as in ddt_argmax.  With one wavefront per SIMD, loads alone
// cannot keep enough bytes in flight, so the share streams through the
// workgroup's LDS in stages by LDS-DMA (double buffered: the next stage
// loads while this one is reduced).  One wavefront per SIMD also issues
// VALU work slowly, so the reduction is kept lean: 32-bit offsets within
// the row's segment, per 16-byte chunk the float maximum (v_max3) and an
// unordered-compare NaN flag, and a search for the first index holding
// the maximum only when a thread's maximum improves (first chunk whose
// maximum equals it, then the element inside, re-read from LDS).  A thread
// whose stage holds a NaN also reduces it the exact key way, which orders
// NaN above every number.  Shares start at whole 16-byte chunks (rows of
// a multiple of 16 bytes, V a multiple of the chunk), so a stage's valid
// elements end on a chunk boundary.
template <typename L, int kStageBytes>
__device__ void argmax_stream(const VerifyParams& p, int am_id, char* lds) {
    static_assert(kStageBytes % (16 * kThreads) == 0, "whole DMA instructions and 16-byte chunks per thread");
    constexpr int VEC = 16 / (int)sizeof(L);
    constexpr int kChunks = kStageBytes / 1024 / (kThreads / 64);  // DMA instructions per wavefront per stage
    constexpr int kPerThread = kStageBytes / 16 / kThreads;        // 16-byte chunks a thread reduces per stage
    constexpr int kStageElems = kStageBytes / (int)sizeof(L);
    typedef uint32_t V4 __attribute__((ext_vector_type(4)));
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t V = p.am_V, E = p.am_E, total = p.am_rows * V;
    const int64_t e0 = (int64_t)am_id * E;
    const int64_t e1 = e0 + E < total ? e0 + E : total;
    const uint32_t lds0 = lds_addr(lds);
    for (int64_t r = e0 / V; r * V < e1; ++r) {
        const int64_t c0 = e0 > r * V ? e0 - r * V : 0;
        const int len = (int)((e1 < (r + 1) * V ? e1 - r * V : V) - c0);  // segment [c0, c0 + len) of row r
        const char* seg = static_cast<const char*>(p.am_logits) + (r * p.am_ld + c0) * (int64_t)sizeof(L);
        const int nst = (len + kStageElems - 1) / kStageElems;
        auto issue = [&](int st) {
            const int s0 = st * kStageElems;
            const int n = len - s0 < kStageElems ? len - s0 : kStageElems;
            const u32x4 rs = buffer_rsrc(seg + (int64_t)s0 * (int)sizeof(L), n * (int)sizeof(L));
            const uint32_t buf = lds0 + (uint32_t)((st & 1) * kStageBytes);
#pragma unroll
            for (int i = 0; i < kChunks; ++i) {
                const int j = wave * kChunks + i;
                dma16(rs, buf + (uint32_t)(j * 1024), (uint32_t)(lane * 16 + j * 1024));
            }
        };
        float bv = -INFINITY;
        int bl = -1;  // offset in the segment of the thread's first maximum
        uint64_t bexact = 0;
        issue(0);
        for (int st = 0; st < nst; ++st) {
            if (st + 1 < nst) {
                issue(st + 1);
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kChunks) : "memory");  // stage st landed
            } else {
                wait_vmem_all();
            }
            __syncthreads();  // every wavefront's part of stage st is in LDS
            const int s0 = st * kStageElems;
            const int nch = (len - s0 < kStageElems ? len - s0 : kStageElems) / VEC;  // valid chunks
            const char* buf = lds + (st & 1) * kStageBytes;
            V4 x[kPerThread];
#pragma unroll
            for (int u = 0; u < kPerThread; ++u) x[u] = *reinterpret_cast<const V4*>(buf + (tid + kThreads * u) * 16);
            float mu[kPerThread];
            bool nan = false;
#pragma unroll
            for (int u = 0; u < kPerThread; ++u) {
                const L* e = reinterpret_cast<const L*>(&x[u]);
                float c = ddt::widen<L>(e[0]);
                bool q = false;
#pragma unroll
                for (int k = 1; k < VEC; k += 2) {
                    const float a = ddt::widen<L>(e[k]);
                    const float b2 = k + 1 < VEC ? ddt::widen<L>(e[k + 1]) : a;
                    c = ddt::fmax3_raw(c, a, b2);
                    q |= __builtin_isunordered(a, b2);
                }
                q |= __builtin_isunordered(ddt::widen<L>(e[0]), ddt::widen<L>(e[0]));
                const bool valid = tid + kThreads * u < nch;
                mu[u] = valid ? c : -INFINITY;
                nan |= valid && q;
            }
            float m = mu[0];
#pragma unroll
            for (int u = 1; u < kPerThread; u += 2)
                m = ddt::fmax3_raw(m, mu[u], u + 1 < kPerThread ? mu[u + 1] : mu[u]);
            if (m > bv || bl < 0) {  // (the first stage always searches, -inf rows included)
                int fu = -1;
#pragma unroll
                for (int u = kPerThread - 1; u >= 0; --u)
                    if (mu[u] == m && tid + kThreads * u < nch) fu = u;
                if (fu >= 0) {
                    const V4 y = *reinterpret_cast<const V4*>(buf + (tid + kThreads * fu) * 16);
                    const L* e = reinterpret_cast<const L*>(&y);
                    int fk = VEC - 1;
#pragma unroll
                    for (int k = VEC - 2; k >= 0; --k)
                        if (ddt::widen<L>(e[k]) == m) fk = k;
                    bv = m;
                    bl = s0 + (tid + kThreads * fu) * VEC + fk;
                }
            }
            if (nan) {
#pragma unroll
                for (int u = 0; u < kPerThread; ++u) {
                    const L* e = reinterpret_cast<const L*>(&x[u]);
                    const int o = s0 + (tid + kThreads * u) * VEC;
                    if (tid + kThreads * u < nch) {
#pragma unroll
                        for (int k = 0; k < VEC; ++k)
                            bexact = ddt::umax64(bexact, ddt::pack_key(ddt::f32_bits<L>(e[k]), c0 + o + k));
                    }
                }
            }
            __syncthreads();  // stage st consumed: its buffer takes stage st+2
        }
        uint64_t key = bl >= 0 ? ddt::pack_key(__float_as_uint(bv), c0 + bl) : 0;
        key = ddt::umax64(key, bexact);
        key = ddt::block_max(key);
        const int parts = (int)(((r + 1) * V - 1) / E - (r * V) / E + 1);
        if (threadIdx.x == 0) ddt::finish_chunk(key, r, parts, p.am_idx, p.am_slots);
    }
}
// Rows whose layout does not allow 16-byte loads (unaligned start, row
// stride or length) take the plain exact scan.
template <typename L>
__device__ void argmax_plain(const VerifyParams& p, int am_id) {
    const int64_t V = p.am_V, E = p.am_E, total = p.am_rows * V;
    const int64_t e0 = (int64_t)am_id * E;
    const int64_t e1 = e0 + E < total ? e0 + E : total;
    const L* logits = static_cast<const L*>(p.am_logits);
    for (int64_t r = e0 / V; r * V < e1; ++r) {
        const int64_t c0 = e0 > r * V ? e0 - r * V : 0;
        const int64_t c1 = e1 < (r + 1) * V ? e1 - r * V : V;
        uint64_t key = ddt::scan_chunk_exact<L, false, 1>(logits + r * p.am_ld, c0, c1);
        key = ddt::block_max(key);
        const int parts = (int)(((r + 1) * V - 1) / E - (r * V) / E + 1);
        if (threadIdx.x == 0) ddt::finish_chunk(key, r, parts, p.am_idx, p.am_slots);
    }
}
template <int kStageBytes>
__device__ inline void argmax_role(const VerifyParams& p, int am_id, char* lds) {
    if (p.am_dtype == DDT_F32) {
        if (p.am_vec) argmax_stream<float, kStageBytes>(p, am_id, lds);
        else argmax_plain<float>(p, am_id);
    } else {
        if (p.am_vec) argmax_stream<uint16_t, kStageBytes>(p, am_id, lds);
        else argmax_plain<uint16_t>(p, am_id);
    }
}

template <typename T, int DL, int DR>
struct Shape {
    using Tr = Traits<T>;
    using Frag = typename Tr::Frag;
    static constexpr int KPL = Tr::KPL;
    static constexpr int DQK = DL + DR;
    static constexpr int KSTEP = 2 * KPL;          // k per MFMA
    static constexpr int NKS = DQK / KSTEP;        // score MFMAs per tile
    static constexpr int NCT = DL / 32;            // 32-column output tiles of a value wavefront
    static constexpr int NPS = KT / KSTEP;         // value k-steps per tile
    static constexpr int VEC = 16 / sizeof(T);     // elements per 16-byte chunk
    static constexpr int CA = DL / VEC, CB = DR / VEC;      // chunks per row, regions A / B
    static constexpr int RPI_A = 64 / CA, RPI_B = 64 / CB;  // rows per DMA instruction
    static constexpr int NI_A = KT * CA / 64, NI_B = KT * CB / 64;  // DMA instructions per tile
    static constexpr int NI = NI_A + NI_B;
    static constexpr int NDW = NGRP;               // wavefronts that issue the DMA (the value wavefronts)
    static constexpr int IA = NI_A / NDW, IB = NI_B / NDW;
    static constexpr int DPW = IA + IB;            // DMA instructions per value wavefront per tile
    static constexpr int STAGE_BYTES = NI * 64 * 16;
    static constexpr int RING = NSTAGE * STAGE_BYTES;
    static constexpr int PBUF = NPS * 64 * (int)sizeof(Frag);  // one row group's probabilities of one tile
    static constexpr int LDS_BYTES = RING + 2 * NGRP * PBUF;
    static_assert(DL % KSTEP == 0 && DR % KSTEP == 0, "head dims must be multiples of the MFMA k");
    static_assert(DL % 32 == 0, "value columns come in 32-column tiles");
    static_assert(CA <= 64 && CB <= 64 && 64 % CA == 0 && 64 % CB == 0, "rows must tile DMA instructions");
    static_assert((KT * CA) % 64 == 0 && (KT * CB) % 64 == 0, "regions must be whole instructions");
    static_assert(NI_A % NDW == 0 && NI_B % NDW == 0, "value wavefronts split each region evenly");
    static_assert(DPW <= NCT * NPS, "DMA instructions interleave with the value MFMAs");
    static_assert(LDS_BYTES + ROWS_WG * 4 + 4 <= 160 * 1024, "LDS budget");
};


// One workgroup = one work item (request b, key split, tile of 64 query
// rows).  Wavefronts 0 and 1 are score wavefronts (row groups 0 and 1: S^T,
// mask, softmax, probabilities to LDS); wavefronts 2 and 3 are value
// wavefronts (row groups 0 and 1: O^T += V^T P^T, and the LDS-DMA of the key
// tiles).  Every wavefront takes the same sequence of workgroup barriers:
// per pass, one before phase 0 and one after each of the ntiles + 2 phases.
// In phase j (between barriers j and j+1) the score wavefronts run the
// MFMAs of tile j together with the softmax of tile j-1, and the value
// wavefronts multiply tile j-2 while loading tile j+1 into the ring slot of
// tile j-3.
// Work item of attention block `blk`: request b, key split, row tile rt;
// false for the few blocks that pad the XCD deal.  The hardware deals
// blocks to the 8 XCDs round robin, so block x + 8j runs on XCD x; unit u
// (up to unit_rows row tiles of one key split, which then share that XCD's
// L2) goes to position u / 8 of XCD u % 8 (of XCD 7 - u % 8 at odd
// positions), and units are numbered in the order they should start.  The last n_units % 8 units are dealt row tile
// by row tile instead, so every XCD gets the same number of workgroups
// (give or take one).
__host__ __device__ inline bool work_item(const VerifyParams& p, int blk, int& b, int& split, int& rt) {
    if (p.single_round) {
        // one round: XCD x runs work items [x*n/8, (x+1)*n/8) in (request,
        // split, row tile) order: neighbouring key splits and the row tiles
        // of a split share the XCD (measured 0.9 us faster than the deal
        // below at the K2-like head share)
        const int wl = ddt::xcd_logical_block(blk, p.total_wg);
        if (blk >= p.total_wg) return false;
        int lo = 0, hi = p.B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.wg_begin[mid] <= wl) lo = mid; else hi = mid - 1;
        }
        b = lo;
        const int local = wl - p.wg_begin[b];
        split = local / p.row_tiles;
        rt = local - split * p.row_tiles;
        return true;
    }
    int u, r_in;
    if (blk < p.whole_blocks) {
        // position pos of XCD x: units are dealt in snake order (XCDs 0..7,
        // then 7..0, ...), so with units longest first the XCDs' sums of
        // work even out (a simulation of the dispatch over random ragged
        // batches: 12 % shorter on average than round robin, never longer)
        const int x = blk % ddt::kXcds, j = blk / ddt::kXcds;
        const int pos = j / p.unit_rows;
        r_in = j - pos * p.unit_rows;
        u = pos * ddt::kXcds + ((pos & 1) ? ddt::kXcds - 1 - x : x);
    } else {
        const int item = blk - p.whole_blocks;
        const int du = item / p.unit_rows;
        r_in = item - du * p.unit_rows;
        u = p.whole_blocks / p.unit_rows + du;
    }
    if (u >= p.n_units) return false;
    const int grp = u / p.units_per_group, sg = u - grp * p.units_per_group;
    rt = sg * p.unit_rows + r_in;
    if (rt >= p.row_tiles) return false;
    if (p.rt_desc) rt = p.row_tiles - 1 - rt;
    if (grp < p.n_full_groups) {
        int lo = 0, hi = p.B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.full_gbegin[mid] <= grp) lo = mid; else hi = mid - 1;
        }
        b = lo;
        split = grp - p.full_gbegin[b];
    } else {
        b = p.part_b[grp - p.n_full_groups];
        split = (p.P[b] + p.N) / p.chunk;  // the shorter last split
    }
    return true;
}

// paged cache: a split's page numbers stream through a ring of kPgSlots
// windows of kPgWin consecutive table entries in LDS
constexpr int kPgWin = 64, kPgSlots = 4;

template <typename T, int DL, int DR, bool kArgmax, bool kTouch, bool kPaged, bool kClip>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void verify_split(
    const VerifyParams p) {
    using S = Shape<T, DL, DR>;
    using Tr = typename S::Tr;
    using Frag = typename Tr::Frag;
    constexpr int KPL = S::KPL;
    __shared__ __attribute__((aligned(16))) char smem[S::LDS_BYTES];
    if (kArgmax && (int)blockIdx.x >= p.n_attn) {
        // dispatched after every attention workgroup, so it takes a CU the
        // attention leaves idle
        // stages of at most 64 KB, two of them in this kernel's LDS
        constexpr int kAmStage = S::LDS_BYTES / 2 >= 65536 ? 65536 : (S::LDS_BYTES / 2) / 4096 * 4096;
        argmax_role<kAmStage>(p, (int)blockIdx.x - p.n_attn, smem);
        return;
    }
    __shared__ float s_mref[ROWS_WG];  // per-row softmax reference, for the log-sum-exp
    __shared__ __attribute__((aligned(256))) char s_touch[256];  // landing area of the L2 touches
    __shared__ int s_redo;

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave % NGRP;

    // ---- work item: (request, key split, row tile) ----
    int b = 0, split = 0, rt = 0;
    if (!work_item(p, (int)blockIdx.x, b, split, rt)) return;  // (uniform: the whole workgroup)
    const int wl = p.wg_begin[b] + split * p.row_tiles + rt;   // partial-output slot
    // committed length: the planned one, or the device's (at most the
    // planned bound, which the work items cover)
    const int P = p.P_dev == nullptr ? p.P[b]
                                     : __builtin_amdgcn_readfirstlane(max(0, min(p.P_dev[b], p.P[b])));
    const int kT = P + p.N;  // the request's keys: rows [0, kT) are read, no further
    const int kbeg = split * p.chunk;
    // kClip (large trees, e.g. prefill chunks): nodes are numbered
    // parents-first, so a row of node i sees no tree key past P + i; keys
    // past P + imax + 1 (imax: the last node among this work item's rows)
    // are invisible to every row here and are not read.  At least one key
    // stays, fully masked, so a split past imax is an ordinary work item
    // with an empty partial; so is a split past a device length below the
    // planned one (its key, at or past kT, is neither read nor visible).
    const int kend0 = max(kbeg + 1, min(kbeg + p.chunk, kT));
    const int kend =
        kClip ? __builtin_amdgcn_readfirstlane(
                    max(kbeg + 1, min(kend0, P + (min(p.rows, (rt + 1) * ROWS_WG) - 1) / p.H + 1)))
              : kend0;
    const int ntiles = (kend - kbeg + KT - 1) / KT;
    // rows the tiles read: [kbeg, kread), kread <= kT (an empty split reads none)
    const int kread = max(kbeg, min(kend, kT));
    // paged cache: the split's page numbers, window w (entries [w*kPgWin,
    // (w+1)*kPgWin) from the split's first page) in ring slot w % kPgSlots;
    // the value wavefronts fill and read them (the tile loop reads them in
    // order with its other LDS traffic: a scalar load per tile would make
    // every LDS wait in the loop wait for it too)
    __shared__ __attribute__((aligned(16))) int32_t s_pgwin[kPaged ? kPgWin * kPgSlots : 1];

    const int wrow0 = rt * ROWS_WG + grp * 32;
    const bool active = wrow0 < p.rows;            // the row group has real rows
    const int row = min(wrow0 + l32, p.rows - 1);  // padded rows recompute the last row, never stored
    const int64_t qrow = (int64_t)b * p.rows + row;
    // probabilities of tile j for row group grp: pbuf0 + (j & 1) * NGRP * PBUF
    char* const pbuf0 = smem + S::RING + grp * S::PBUF;

    if (tid == 0) s_redo = 0;  // read only after the first pass's barriers

    if (wave < NGRP) {
        // =========================== score wavefront ===========================
        const int node = row / p.H;
        const uint64_t* __restrict__ mrow = p.mask + ((int64_t)b * p.N + node) * p.W;  // (unused without a mask)
        // queries: B operand of the score MFMA, resident for the whole split
        Frag q[S::NKS];
#pragma unroll
        for (int s = 0; s < S::NKS; ++s) {
            const int d0 = s * S::KSTEP + g * KPL;
            const T* src = d0 < DL ? static_cast<const T*>(p.q_lat) + qrow * p.ld_ql + d0
                                   : static_cast<const T*>(p.q_pe) + qrow * p.ld_qp + (d0 - DL);
            q[s] = Tr::global_frag(src);
        }
        // the first two mask words of this row (trees up to 128 nodes) stay in
        // registers; larger trees fetch words per tile
        uint64_t mreg[2] = {0, 0};
        if (kend > P) {
            if (p.mask != nullptr) {
#pragma unroll
                for (int w = 0; w < 2; ++w)
                    if (w < p.W) mreg[w] = mrow[w];
            } else {
                tree_ancestors(p.parents + (int64_t)b * p.N, p.N, node, mreg[0], mreg[1]);
            }
        }
        // Settle the query and mask loads here, once, behind an opaque
        // definition, so no wait inside the loop is tied to them.
#pragma unroll
        for (int s = 0; s < S::NKS; ++s) pin_acc(q[s]);
#pragma unroll
        for (int w = 0; w < 2; ++w) pin_reg(mreg[w]);

        const typename Tr::Lane LO = Tr::template lane_offsets<DL, DR>(lane);
        float m_ref = -INFINITY;   // per-row softmax reference (log2 domain)
        float m_seen = -INFINITY;  // per-row maximum of the scores seen so far
        bool overflow = false;
        float x[16];               // raw dot products, then probabilities, of the tile in softmax
        float mx = 0.f, nb = 0.f;

        // tiles reaching into the tree part or past the split end need the mask
        auto tile_masked = [&](int tp) {
            const int t0 = kbeg + tp * KT;
            return t0 + KT > P || t0 + KT > kend;
        };
        auto mask_x = [&](int tp) {
            // keys [t0, t0+32) touch at most two mask words
            const int t0 = kbeg + tp * KT;
            const int wlo = (t0 - P > 0 ? t0 - P : 0) >> 6;
            uint64_t mw0, mw1;
            if (wlo == 0) {
                mw0 = mreg[0];
                mw1 = mreg[1];
            } else if (p.mask == nullptr) {  // at most 128 nodes: word 1 is the last
                mw0 = mreg[1];
                mw1 = mreg[1];
            } else {
                mw0 = mrow[wlo < p.W ? wlo : p.W - 1];
                mw1 = mrow[wlo + 1 < p.W ? wlo + 1 : p.W - 1];
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int t = t0 + (v >> 2) * 8 + g * 4 + (v & 3);
                const int jn = t - P;
                // bit (jn mod 64) of the word holding jn, tested with 32-bit operations
                const uint64_t word = (jn >> 6) == wlo ? mw0 : mw1;
                const uint32_t half = (jn & 32) ? (uint32_t)(word >> 32) : (uint32_t)word;
                const uint32_t vis = (uint32_t)(t < kend) & (uint32_t)(t < kT) &
                                     ((uint32_t)(t < P) | ((half >> (jn & 31)) & 1u));
                x[v] = vis ? x[v] : -INFINITY;
            }
        };
        // Step `st` of the softmax of tile tp (raw dot products in acc, or
        // already masked in x when HaveX).  The steps ride on the MFMA stream
        // of the next tile, at most one exponential and two other VALU
        // operations per MFMA, which is what one wavefront hides under a
        // 32x32x16 product.
        // Softmax against a fixed per-row reference m_ref: the max of the
        // first tile in which the row sees any key.  Probabilities
        // 2^(scale*s - m_ref) stay finite unless a later score exceeds m_ref
        // by more than kSpan; then the split is recomputed with the split's
        // maximum as the reference, so no accumulator is ever rescaled.  The
        // row sums are taken by the value wavefronts (an MFMA against ones).
        auto sm_step = [&](int st, const floatx16& acc, auto have_x, int tp) {
            if (st < 8) {
                if constexpr (!decltype(have_x)::value) {
                    x[2 * st] = acc[2 * st];
                    x[2 * st + 1] = acc[2 * st + 1];
                }
                mx = max3f(st == 0 ? x[0] : mx, x[2 * st], x[2 * st + 1]);
            }
            if (st == 8) mx *= p.scale_log2;  // scale > 0
            if (st == 9) mx = pair_max(mx);
            if (st == 10) m_seen = max3f(m_seen, mx, mx);
            if (st == 11 && m_ref == -INFINITY) m_ref = mx;
            if (st == 12) overflow |= mx > m_ref + kSpan;
            if (st == 13) nb = m_ref == -INFINITY ? 0.f : -m_ref;
            if (st >= 14 && st < 30) {
                const int e = st - 14;
                x[e] = __builtin_amdgcn_exp2f(fmaf(x[e], p.scale_log2, nb));
            }
            // publish P^T in the value MFMA's B-operand order
            if (st == 30 || st == 32) {
                char* pw = pbuf0 + (tp & 1) * (NGRP * S::PBUF);
                constexpr int H2 = S::NPS / 2;
                const int j0 = st == 30 ? 0 : H2;
#pragma unroll
                for (int j = j0; j < j0 + H2; ++j)
                    *reinterpret_cast<Frag*>(pw + (j * 64 + lane) * (int)sizeof(Frag)) = Tr::from_f32(x + j * KPL);
            }
        };
        constexpr int NST = 33;  // softmax steps
        static_assert(S::NKS >= NST, "softmax steps ride on the score MFMAs");
        // Phase `it`: scores of tile it into cur (one accumulator chain:
        // back-to-back dependent products issue without stalls; fragment
        // reads run AH MFMAs ahead), with the softmax of tile it-1 (in prv)
        // when WithSm.
        auto qk_phase = [&](floatx16& cur, const floatx16& prv, int it, auto with_sm, auto have_x) {
            const char* slot = smem + (it % NSTAGE) * S::STAGE_BYTES;
            // the softmax reads the previous tile's MFMA results through inline asm
            if constexpr (decltype(with_sm)::value && !decltype(have_x)::value) mfma_settle();
            constexpr int AH = kScoreAhead;
            Frag f[AH + 1];
#pragma unroll
            for (int k = 0; k < AH; ++k) f[k] = Tr::template k_frag<DL, DR>(slot, LO, k);
#pragma unroll
            for (int ks = 0; ks < S::NKS; ++ks) {
                if (ks + AH < S::NKS) f[(ks + AH) % (AH + 1)] = Tr::template k_frag<DL, DR>(slot, LO, ks + AH);
                cur = Tr::mfma(f[ks % (AH + 1)], q[ks], ks == 0 ? floatx16{} : cur);
                if constexpr (decltype(with_sm)::value) {
                    if (ks < NST) sm_step(ks, prv, have_x, it - 1);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        auto run_phase = [&](floatx16& cur, const floatx16& prv, int it) {
            if (tile_masked(it - 1)) {
#pragma unroll
                for (int v = 0; v < 16; ++v) x[v] = prv[v];
                mask_x(it - 1);
                qk_phase(cur, prv, it, std::true_type{}, std::true_type{});
            } else {
                qk_phase(cur, prv, it, std::true_type{}, std::false_type{});
            }
        };
        auto sm_last = [&](const floatx16& acc, int tp) {
            mfma_settle();
#pragma unroll
            for (int v = 0; v < 16; ++v) x[v] = acc[v];
            if (tile_masked(tp)) mask_x(tp);
#pragma unroll
            for (int st = 0; st < NST; ++st) sm_step(st, acc, std::true_type{}, tp);
        };

        floatx16 sA, sB;  // raw dot products of even / odd tiles
        for (int pass = 0;; ++pass) {
            __syncthreads();  // tile 0 resident
            if (active) qk_phase(sA, sB, 0, std::false_type{}, std::false_type{});
            __syncthreads();  // tile 1 resident
            int it = 1;
            for (; it + 1 < ntiles; it += 2) {
                if (active) run_phase(sB, sA, it);
                __syncthreads();  // probabilities of tile it-1 published; tile it+1 resident
                if (active) run_phase(sA, sB, it + 1);
                __syncthreads();
            }
            if (it < ntiles) {
                // one more tile (odd index); the last tile's scores end in sB
                if (active) run_phase(sB, sA, it);
                __syncthreads();
                if (active) sm_last(sB, ntiles - 1);
            } else {
                if (active) sm_last(sA, ntiles - 1);
            }
            __syncthreads();  // probabilities of the last tile published
            if (active && g == 0) s_mref[grp * 32 + l32] = m_ref;
            if (pass == 0 && __ballot(overflow) != 0 && lane == 0) s_redo = 1;
            __syncthreads();  // last value phase done
            if (pass == 1 || s_redo == 0) break;
            m_ref = m_seen;
            overflow = false;
        }
        return;
    }

    // ============================= value wavefront =============================
    // LDS-DMA of tile `tile` into its ring slot.  Each region (A: c_kv, B:
    // k_pe) of a tile is NI_A / NI_B instructions of 64 16-byte chunks;
    // value wavefront grp issues instructions grp, grp + NDW, ...  Rows at or
    // past the split end fall outside the buffer descriptor's range and read
    // as zeros (their probabilities are zero).  A tile index past the split
    // loads an empty range, i.e. zeros, into its slot, which then holds a
    // consumed tile; so every phase issues DPW loads and the loop body has
    // no branches.
    // A tile's 32 rows are consecutive slots from a multiple of 32, so they
    // are consecutive pool rows in a contiguous cache and inside one page
    // (pages of 2^shift >= 32 rows) in a paged one: one row lookup per tile.
    const int64_t kvb = kPaged ? 0 : p.map.kv_base[b];
    const char* ckv_b = uniform_ptr(reinterpret_cast<const char*>(static_cast<const T*>(p.ckv) + kvb * p.ld_ckv));
    const char* kpe_b = uniform_ptr(reinterpret_cast<const char*>(static_cast<const T*>(p.kpe) + kvb * p.ld_kpe));
    const int pshift = kPaged ? p.map.shift : 0;
    const int ppg0 = kPaged ? (kbeg >> pshift) : 0;
    const int npg = kPaged ? ((kend - 1) >> pshift) - ppg0 + 1 : 0;  // pages of the split
    // the split's table entries (entries past them deliver zeros); value
    // wavefront 0 streams them into the window ring by LDS-DMA, landing
    // under the same waits and barriers as the tiles
    u32x4 pg_rsrc = {};
    if constexpr (kPaged)
        pg_rsrc = buffer_rsrc(p.map.table + (int64_t)b * p.map.ld + ppg0, npg * (int)sizeof(int32_t));
    auto pg_fill = [&](int w) {
        if constexpr (kPaged) {
            if (grp == 0)
                dma4(pg_rsrc, lds_addr(s_pgwin) + (uint32_t)((w % kPgSlots) * kPgWin * (int)sizeof(int32_t)),
                     (uint32_t)((w * kPgWin + lane) * (int)sizeof(int32_t)));
        }
    };
    int pg_filled = 0;  // windows [0, pg_filled] are in the ring (or on their way)
    const int ldA = (int)(p.ld_ckv * (int64_t)sizeof(T)), ldB = (int)(p.ld_kpe * (int64_t)sizeof(T));
    const uint32_t pg_bytesA = (uint32_t)ldA << pshift, pg_bytesB = (uint32_t)ldB << pshift;  // (paged)
    // instructions 2k and 2k+1 of a wavefront (same region, 2048 bytes apart
    // in LDS) go out as one pair under one M0: half the M0 writes and their
    // wait states in the value wavefronts' instruction stream (measured 1.7 %
    // faster at 32 ragged requests of 8 heads, neutral at 131072 keys)
    constexpr bool kPairDma = sizeof(T) == 2 && S::IA % 2 == 0 && S::IB % 2 == 0 && S::NDW * 64 * 16 == 2048;
    uint32_t voff[S::DPW];
#pragma unroll
    for (int i = 0; i < S::DPW; ++i) {
        const bool ra = i < S::IA;
        const int jj = grp + S::NDW * (ra ? i : i - S::IA);
        const int r = jj * (ra ? S::RPI_A : S::RPI_B) + lane / (ra ? S::CA : S::CB);
        const int chunk = ra ? (lane % S::CA) ^ Tr::swA(r) : (lane % S::CB) ^ Tr::swB(r);
        voff[i] = (uint32_t)(r * (ra ? ldA : ldB) + chunk * 16);
        if (kPairDma && (i & 1)) voff[i] -= 2048;  // the pair's instruction offset adds it back
        pin_reg(voff[i]);
    }
    // L2 touches of a tile: every 128-byte line of its rows (LA lines of
    // c_kv, then LB of k_pe, per row), 64 lines per instruction, three
    // instructions per value wavefront; wavefront grp's instruction k covers
    // lines grp*64 + 128k ..; lines past the tile read nothing
    constexpr int LA = (DL * (int)sizeof(T) + 127) / 128, LB = (DR * (int)sizeof(T) + 127) / 128;
    constexpr int kTouches = 3;
    static_assert(KT * (LA + LB) <= kTouches * 64 * S::NDW, "three touches per value wavefront cover a tile");
    static_assert((KT * LA) % 64 == 0, "an instruction's lines lie in one region");
    uint32_t toff[kTouches];
#pragma unroll
    for (int k = 0; k < kTouches; ++k) {
        const int i = grp * 64 + lane + 128 * k, j = i - KT * LA;
        toff[k] = i < KT * LA ? (uint32_t)((i / LA) * ldA + (i % LA) * 128)
                              : (j < KT * LB ? (uint32_t)((j / LB) * ldB + (j % LB) * 128) : 0xFFFFFFF0u);
        pin_reg(toff[k]);
    }
    // per-tile descriptors of the two regions (rows [t0, min(t0 + KT, kread)))
    struct TileDma {
        u32x4 ra, rb;    // raw buffer descriptors of the tile's rows in c_kv / k_pe
        uint32_t lds;    // LDS byte address of the tile's ring slot
    };
    // paged: the page holding a tile's rows (a tile past the split: the
    // last tile's page; its descriptor is empty), read from the window ring;
    // the loop reads the next phase's page number at the end of a phase, so
    // no phase starts with a wait on an LDS read before its first load.
    // page_direct reads the table itself (the prologue's tiles).
    auto page_index = [&](int tile) { return ((kbeg + (tile < ntiles ? tile : ntiles - 1) * KT) >> pshift) - ppg0; };
    auto page_of = [&](int tile) -> int32_t {
        if constexpr (kPaged) {
            const int pi = page_index(tile);
            return s_pgwin[(pi / kPgWin) % kPgSlots * kPgWin + pi % kPgWin];
        } else {
            return 0;
        }
    };
    auto page_direct = [&](int tile) -> int32_t {
        if constexpr (kPaged) {
            return p.map.table[(int64_t)b * p.map.ld + ppg0 + page_index(tile)];
        } else {
            return 0;
        }
    };
    auto tile_dma = [&](int tile, int32_t page) {
        const bool real = tile < ntiles;
        const int t0 = kbeg + (real ? tile : 0) * KT;
        int nrows = kread - t0;
        nrows = real ? (nrows > KT ? KT : nrows) : 0;
        TileDma d;
        if constexpr (kPaged) {  // pool row of slot t0: its page's first row + the offset in the page
            // page * (bytes of a page) + (row in the page) * (row bytes): a
            // 32 x 32 -> 64-bit product and a 32-bit one (a page's bytes
            // stay below 4 GiB), fewer scalar instructions per tile than a
            // 64-bit row index times the stride
            const uint32_t pg = (uint32_t)__builtin_amdgcn_readfirstlane(page);
            const uint32_t in_pg = (uint32_t)(t0 & ((1 << pshift) - 1));
            const uint64_t offA = (uint64_t)pg * pg_bytesA + in_pg * (uint32_t)ldA;
            const uint64_t offB = (uint64_t)pg * pg_bytesB + in_pg * (uint32_t)ldB;
            d.ra = buffer_rsrc(ckv_b + offA, nrows * ldA);
            d.rb = buffer_rsrc(kpe_b + offB, nrows * ldB);
        } else {
            d.ra = buffer_rsrc(ckv_b + (int64_t)t0 * ldA, nrows * ldA);
            d.rb = buffer_rsrc(kpe_b + (int64_t)t0 * ldB, nrows * ldB);
        }
        d.lds = lds_addr(smem) + (uint32_t)((tile % NSTAGE) * S::STAGE_BYTES);
        return d;
    };
    auto issue = [&](const TileDma& d, int i) {
        const bool ra = i < S::IA;
        const int jj = grp + S::NDW * (ra ? i : i - S::IA);
        const uint32_t lds = d.lds + (uint32_t)(((ra ? 0 : KT * S::CA) + jj * 64) * 16);
        if constexpr (kPairDma) {
            if ((i & 1) == 0) dma16x2(ra ? d.ra : d.rb, lds, voff[i], voff[i + 1]);
        } else {
            dma16(ra ? d.ra : d.rb, lds, voff[i]);
        }
    };
    auto issue_tile = [&](int tile) {
        const TileDma d = tile_dma(tile, page_direct(tile));
#pragma unroll
        for (int i = 0; i < S::DPW; ++i) issue(d, i);
    };
    // Value wavefront `half` (= grp) owns output columns [half*DL/2,
    // (half+1)*DL/2) of all 64 rows: every V^T fragment read from LDS feeds
    // the products of both row groups.  Row group 0 always has real rows;
    // row group 1 may not (last row tile), and then its products run on
    // stale probabilities and are never stored.
    const int half = grp;
    constexpr int NCH = S::NCT / 2;  // 32-column tiles of this wavefront
    const typename Tr::Lane LO = Tr::template lane_offsets<DL, DR>(lane);
    Frag ones;  // A operand of the row-sum product: every key weighs 1
    {
        float one[KPL];
#pragma unroll
        for (int e = 0; e < KPL; ++e) one[e] = 1.f;
        ones = Tr::from_f32(one);
    }
    floatx16 o[NGRP][NCH];
    floatx16 lsum[NGRP];  // every element: the row's sum of (rounded) probabilities
    for (int pass = 0;; ++pass) {
#pragma unroll
        for (int rb = 0; rb < NGRP; ++rb) {
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                o[rb][c] = floatx16{};
                pin_acc(o[rb][c]);
            }
            lsum[rb] = floatx16{};
        }
        mfma_settle();  // the zeroing writes above precede the first product
        // paged: the first two page windows land with tile 0 (a second pass
        // refills them: later windows took their slots)
        pg_fill(0);
        pg_fill(1);
        pg_filled = 1;
        // (loading the first four tiles at once measured slower at the
        // K2-like head share: the burst delays tile 0)
        issue_tile(0);
        wait_vmem_all();
        __syncthreads();  // tile 0 resident
        issue_tile(1);    // phase 0: scores of tile 0
        wait_vmem_all();
        __syncthreads();  // tile 1 resident
        issue_tile(2);    // phase 1: scores of tile 1, softmax of tile 0
        wait_vmem_all();
        __syncthreads();  // tile 2 resident; probabilities of tile 0 published
        // the descriptors of a tile are made once: a phase touches tile it+2,
        // and the next phase loads it with the same descriptors
        TileDma d_next = tile_dma(3, page_of(3));
        int32_t pg_touch = page_of(4);  // (paged) page of the next touched tile
        for (int it = 2; it <= ntiles + 1; ++it) {
            // phase it: O^T (this wavefront's columns x 64 rows) += V^T . P^T
            // for tile it-2: key step outer, column tile inner, row group
            // innermost (the two products of a fragment are independent);
            // value fragments run AV fragments ahead; the loads of tile it+1
            // (into the slot of tile it-3) ride one per MFMA, then the L2
            // touches of tile it+2, so its load in the next phase finds it in
            // L2 (one phase of lead is shorter than HBM latency under this
            // load: measured 0.4 us of load wait per 1.2 us phase at 131072
            // keys without the touches; touching two or three phases ahead
            // measured 2 % slower).  Without kTouch (key streams that stay in
            // the last-level cache) the touches are not issued at all.
            const int tv = it - 2;
            const char* slot = smem + (tv % NSTAGE) * S::STAGE_BYTES;
            if constexpr (kPaged) {
                // keep the ring two windows ahead of the tile whose page this
                // phase's end reads (it + 3): a window holds >= kPgWin
                // tiles, so one fill per phase keeps up, and the slot it
                // takes held a window no lookup needs any more.  Issued
                // before the tile loads, it has landed by this phase's
                // closing wait.
                const int need = page_index(it + 3) / kPgWin + 2;
                if (pg_filled < need && (pg_filled + 1) * kPgWin < npg) pg_fill(++pg_filled);
            }
            const TileDma d = d_next;
            const TileDma dt = tile_dma(it + 2, pg_touch);  // touched into L2 one phase before its load
            const uint32_t touch_lds = lds_addr(s_touch);
            Frag pb[NGRP][S::NPS];
#pragma unroll
            for (int rb = 0; rb < NGRP; ++rb) {
                const char* pr = smem + S::RING + rb * S::PBUF + (tv & 1) * (NGRP * S::PBUF);
#pragma unroll
                for (int j = 0; j < S::NPS; ++j)
                    pb[rb][j] = *reinterpret_cast<const Frag*>(pr + (j * 64 + lane) * (int)sizeof(Frag));
            }
            constexpr int NQ = NCH * S::NPS;  // fragments per tile
            static_assert(S::DPW + kTouches <= NQ * NGRP, "loads and touches ride on distinct MFMAs");
            constexpr int AV = kValueAhead;
            Frag vf[AV + 1];
#pragma unroll
            for (int q = 0; q < AV; ++q) vf[q] = Tr::template v_frag<DL, DR>(slot, LO, half * NCH + q % NCH, q / NCH);
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                if (q + AV < NQ)
                    vf[(q + AV) % (AV + 1)] =
                        Tr::template v_frag<DL, DR>(slot, LO, half * NCH + (q + AV) % NCH, (q + AV) / NCH);
#pragma unroll
                for (int rb = 0; rb < NGRP; ++rb) {
                    const int m = q * NGRP + rb;
                    Tr::mfma_acc(vf[q % (AV + 1)], pb[rb][q / NCH], o[rb][q % NCH]);
                    if (m < S::DPW) issue(d, m);
                    if (kTouch && m >= S::DPW && m < S::DPW + kTouches) {
                        const int k = m - S::DPW;
                        l2_touch(grp * 64 + 128 * k < KT * LA ? dt.ra : dt.rb, touch_lds, toff[k]);
                    }
                    // row sums ride at the end of each key step
                    if (q % NCH == NCH - 1) lsum[rb] = Tr::mfma(ones, pb[rb][q / NCH], lsum[rb]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            d_next = dt;
            if constexpr (kPaged) pg_touch = page_of(it + 3);
            // tile it+1 landed (loads complete in issue order); this phase's
            // touches may stay in flight
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kTouch ? kTouches : 0) : "memory");
            __syncthreads();  // tile it+1 resident; tile it-2 and probabilities it-2 consumed
        }
        if (pass == 1 || s_redo == 0) break;
    }
    wait_vmem_all();

    // ---- epilogue: normalise and store this wavefront's columns of the 64 rows ----
    // normalise in the accumulator registers, so the loop never keeps a
    // second copy of O ready for this point
    mfma_settle();
#pragma unroll
    for (int rb = 0; rb < NGRP; ++rb) {
        const int r = rt * ROWS_WG + rb * 32 + l32;
        const bool ok = r < p.rows;
        const int64_t qr = (int64_t)b * p.rows + (ok ? r : 0);
        const float l = lsum[rb][0];
        const bool whole = p.nsplit[b] == 1;  // (uniform)
        if (half == rb && g == 0 && ok) {
            const float mr = s_mref[rb * 32 + l32];
            if (whole)
                p.lse[qr] = (l > 0.f ? mr + __log2f(l) : -INFINITY) * kLn2;
            else  // the merge weighs the unnormalised partial by 2^(m - M) and divides by the weighed sums
                p.ws_ml[(size_t)wl * ROWS_WG + rb * 32 + l32] =
                    l > 0.f ? make_float2(mr, l) : make_float2(-INFINITY, 0.f);
        }
        if (whole) {  // final output: normalise in place
            const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
            for (int c = 0; c < NCH; ++c) scale_acc(o[rb][c], inv);
        }
        asm volatile("s_nop 7" ::: "memory");
        if (!ok) continue;
        if (p.nsplit[b] == 1) {
            T* dst = static_cast<T*>(p.out) + qr * DL + half * (DL / 2);
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = o[rb][c][v4 * 4 + e];
                    store4<T>(dst + c * 32 + v4 * 8 + g * 4, v);
                }
            }
        } else {
            // unnormalised fp32 partials (the merge divides): one 64-lane
            // store writes 64 x 4 consecutive elements
            float* ws = static_cast<float*>(p.ws_o) + (size_t)wl * (ROWS_WG * DL) + (size_t)rb * (32 * DL) +
                    (size_t)half * NCH * (4 * 64 * 4);
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = o[rb][c][v4 * 4 + e];
                    store4_nt_f32(ws + ((c * 4 + v4) * 64 + lane) * 4, v);
                }
            }
        }
    }
}

// Merge the key splits of every row of multi-split requests.  Split s left
// its unnormalised output O_s = sum_t 2^(x_t - m_s) c_kv[t] (x: scaled score
// in log2 units, m_s: the split's softmax reference) and its row sum
// l_s = sum_t 2^(x_t - m_s):
//   M = max_s m_s, w_s = 2^(m_s - M),
//   out = sum_s w_s O_s / sum_s w_s l_s,  lse = (M + log2 sum_s w_s l_s) ln 2.
// One workgroup per (request, row tile, wavefront, 32-column tile of that
// wavefront); thread (grp, lane) owns the 4 consecutive outputs that the
// split kernel's lane `lane` stored at group `grp`.
template <typename T, int DL, bool kAccept>
__global__ __launch_bounds__(256) void verify_combine(const VerifyParams p) {
    static_assert(ddt::kCompactThreads == 256, "acceptance workgroups share the merge's block size");
    if (kAccept && (int)blockIdx.x < p.n_accept) {
        // acceptance + compaction of request blockIdx.x: the attention that
        // reads the cache rows it moves has finished (previous launch)
        __shared__ uint4 stage[ddt::kCompactStageBytes / 16];
        if (p.acc_vec16)
            ddt::accept_compact_body<uint4>(p.acc, blockIdx.x, stage);
        else
            ddt::accept_compact_body<uint32_t>(p.acc, blockIdx.x, reinterpret_cast<uint32_t*>(stage));
        return;
    }
    const int bid = kAccept ? (int)blockIdx.x - p.n_accept : (int)blockIdx.x;
    constexpr int NCTW = DL / 64;
    const int per_b = p.row_tiles * NW * NCTW;
    const int b = bid / per_b;
    const int ns = p.nsplit[b];
    if (ns <= 1) return;
    int rem = bid - b * per_b;
    const int rt = rem / (NW * NCTW);
    rem -= rt * (NW * NCTW);
    const int wave = rem / NCTW, c = rem - (rem / NCTW) * NCTW;
    const int grp = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 5, l32 = lane & 31;
    const int prow = (wave >> 1) * 32 + l32;
    const int row = rt * ROWS_WG + prow;
    if (row >= p.rows) return;
    const int64_t qrow = (int64_t)b * p.rows + row;
    // splits in batches with all loads of a batch issued together (the
    // partials sit in L2 / last-level cache: latency, not bandwidth,
    // decides), merged with a running maximum
    auto slot_of = [&](int s) { return p.wg_begin[b] + min(s, ns - 1) * p.row_tiles + rt; };
    float M = -INFINITY;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    // batches of KB splits, KB the smallest of 4, 8, 12, 16, 24, 32 that holds the
    // request's splits (indices past the last split load nothing and weigh 0)
    auto merge = [&](auto kb) {
        constexpr int KB = decltype(kb)::value;
        for (int s0 = 0; s0 < ns; s0 += KB) {
            float2 ml[KB];
            float4 v[KB];
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                ml[k] = make_float2(-INFINITY, 0.f);
                v[k] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (s0 + k < ns) {  // uniform: no load for the padding
                    const int slot = slot_of(s0 + k);
                    ml[k] = p.ws_ml[(size_t)slot * ROWS_WG + prow];
                    v[k] = load4_f32(static_cast<const float*>(p.ws_o) + ((size_t)slot * NW + wave) * (NCTW * 4 * 64 * 4) +
                                    ((c * 4 + grp) * 64 + lane) * 4);
                }
            }
            float mb = M;
#pragma unroll
            for (int k = 0; k < KB; ++k) mb = fmaxf(mb, s0 + k < ns ? ml[k].x : -INFINITY);
            if (mb != M && M != -INFINITY) {  // rescale what earlier batches summed
                const float r = __builtin_amdgcn_exp2f(M - mb);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] *= r;
                wsum *= r;
            }
            M = mb;
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const float w = (s0 + k >= ns || ml[k].x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ml[k].x - M);
                acc[0] += w * v[k].x;
                acc[1] += w * v[k].y;
                acc[2] += w * v[k].z;
                acc[3] += w * v[k].w;
                wsum += w * ml[k].y;
            }
        }
    };
    if (ns <= 4)
        merge(std::integral_constant<int, 4>{});
    else if (ns <= 8)
        merge(std::integral_constant<int, 8>{});
    else if (ns <= 12)
        merge(std::integral_constant<int, 12>{});
    else if (ns <= 16)
        merge(std::integral_constant<int, 16>{});
    else if (ns <= 24)
        merge(std::integral_constant<int, 24>{});
    else
        merge(std::integral_constant<int, 32>{});
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] *= inv;
    store4<T>(static_cast<T*>(p.out) + qrow * DL + (wave & 1) * (DL / 2) + c * 32 + grp * 8 + g * 4, acc);
    if (c == 0 && grp == 0 && g == 0 && (wave & 1) == 0) p.lse[qrow] = (M + __log2f(wsum)) * kLn2;
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
    int n_blocks = 0;  // attention blocks launched (work items plus padding of the XCD deal)
    bool touch = false;  // the instance that touches tiles into L2
    bool any_split = false;
    size_t ws_bytes = 0, ws_ml_off = 0;
};

int check_desc(const ddt_attn_desc* d, const int32_t* prefix_len_host) {
    if (d == nullptr || prefix_len_host == nullptr) return DDT_EINVAL;
    if (d->B < 1 || d->B > DDT_MAX_BATCH || d->H < 1 || d->N < 1 || d->N > DDT_MAX_NODES) return DDT_EINVAL;
    if (d->kv_chunk < 0) return DDT_EINVAL;
    if (!(d->scale > 0.f) || !isfinite(d->scale)) return DDT_EINVAL;  // the softmax takes maxima of unscaled dots
    const bool k2 = d->d_lat == 512 && d->d_rope == 64 && d->dtype == DDT_BF16;
    const bool tiny = d->d_lat == 64 && d->d_rope == 16 && d->dtype == DDT_F32;
    if (!k2 && !tiny) return DDT_EUNSUPPORTED;
    if (d->ld_ql < d->d_lat || d->ld_qp < d->d_rope || d->ld_ckv < d->d_lat || d->ld_kpe < d->d_rope)
        return DDT_EINVAL;
    const int64_t es = ddt::elem_bytes(d->dtype);
    if ((d->ld_ql * es) % 16 || (d->ld_qp * es) % 16 || (d->ld_ckv * es) % 16 || (d->ld_kpe * es) % 16)
        return DDT_EINVAL;
    if (d->ld_ckv * es > INT32_MAX || d->ld_kpe * es > INT32_MAX) return DDT_EINVAL;  // row strides in 32 bits
    if ((int64_t)d->H * d->N > (1 << 24)) return DDT_EINVAL;
    for (int b = 0; b < d->B; ++b)
        if (prefix_len_host[b] < 0 || (int64_t)prefix_len_host[b] + d->N > 0x7fffffff - 4096) return DDT_EINVAL;
    if (d->block_table != nullptr) {  // pages: a power of two of at least one key tile; every slot in the table
        const int ps = d->page_size;
        if (ps < KT || ps > (1 << 16) || (ps & (ps - 1)) != 0 || d->bt_ld < 1) return DDT_EINVAL;
        if (d->ld_ckv * es * ps > UINT32_MAX || d->ld_kpe * es * ps > UINT32_MAX) return DDT_EINVAL;  // page < 4 GiB
        if (d->dtype != DDT_BF16) return DDT_EUNSUPPORTED;
        for (int b = 0; b < d->B; ++b)
            if (((int64_t)prefix_len_host[b] + d->N + ps - 1) / ps > d->bt_ld) return DDT_EINVAL;
    }
    return DDT_OK;
}

// Estimated finish time, in tile phases, of the attention launch when the
// keys are split into chunks of `chunk`: workgroups of a whole chunk start
// first and fill the CUs in rounds; the shorter last splits then go, longest
// first, to the earliest free CUs (loads are kept as (value, count) buckets
// in a heap, so the estimate costs a few heap steps per request, not one per
// workgroup); a merge launch is added when any request is split.
constexpr int64_t kItemOverhead = 10;   // prologue, pipeline fill and epilogue of a workgroup, in tiles
constexpr int64_t kMergeCost = 8;       // the split merge launch, in tiles
constexpr int64_t kPartialRowBytes = 512 * 4;  // fp32 partial output of one row (K2 latent width)

// `T` holds the requests' key counts in descending order.
int64_t plan_cost(const int64_t* T, int B, int row_tiles, int64_t chunk, int cus) {
    int64_t full = 0;
    bool split = false;
    int64_t tails[DDT_MAX_BATCH];
    int nt = 0;
    for (int b = 0; b < B; ++b) {
        full += T[b] / chunk;
        if (T[b] > chunk) split = true;
        if (T[b] % chunk) tails[nt++] = T[b] % chunk;
    }
    std::sort(tails, tails + nt, [](int64_t x, int64_t y) { return x > y; });
    const int64_t cf = (chunk + KT - 1) / KT + kItemOverhead;
    const int64_t items = full * row_tiles;
    const int64_t rounds = items / cus, rem = items % cus;
    // CU loads as (value, count) buckets in a min-heap; a group's workgroups
    // go to the least-loaded CUs
    struct Bucket {
        int64_t v, n;
    };
    constexpr int kMaxBuckets = 4 * DDT_MAX_BATCH + 4;
    Bucket heap[kMaxBuckets];    // (uninitialised: only the first nb are live)
    Bucket loaded[kMaxBuckets];  // buckets a group has just loaded
    int nb = 0;
    const auto later = [](const Bucket& x, const Bucket& y) { return x.v > y.v; };
    auto push = [&](int64_t v, int64_t n) {
        heap[nb++] = Bucket{v, n};
        std::push_heap(heap, heap + nb, later);
    };
    if (cus - rem > 0) push(rounds * cf, cus - rem);
    if (rem > 0) push((rounds + 1) * cf, rem);
    int64_t finish = rem > 0 ? (rounds + 1) * cf : rounds * cf;
    for (int k = 0; k < nt; ++k) {
        const int64_t c = (tails[k] + KT - 1) / KT + kItemOverhead;
        int64_t need = row_tiles;
        int nl = 0;
        while (need > 0) {
            std::pop_heap(heap, heap + nb, later);
            const Bucket low = heap[--nb];
            const int64_t take = low.n < need ? low.n : need;
            need -= take;
            if (take < low.n) push(low.v, low.n - take);
            const int64_t v = low.v + c;
            if (nl > 0 && loaded[nl - 1].v == v)
                loaded[nl - 1].n += take;
            else if (nl < kMaxBuckets / 2)
                loaded[nl++] = Bucket{v, take};
            else
                loaded[nl - 1] = Bucket{v, loaded[nl - 1].n + take};  // (fold: loads only grow)
            finish = v > finish ? v : finish;
            if (nb == 0 && need > 0) {  // more workgroups than CUs: the rest queue behind these
                for (int j = 0; j < nl; ++j) push(loaded[j].v, loaded[j].n);
                nl = 0;
            }
        }
        for (int j = 0; j < nl; ++j) {
            if (nb < kMaxBuckets)
                push(loaded[j].v, loaded[j].n);
            else  // keep the heap bounded: fold into the lowest bucket (an estimate)
                heap[0].n += loaded[j].n;
        }
    }
    // the split partials: in a launch of one round every split work item
    // writes its fp32 partials at once at the end and the merge reads them
    // back right after, all exposed; with several rounds the writes overlap
    // other work items and mostly the merge's read is left (measured at the
    // K2-like head share: 25.9 us at 256 keys per split, 23.9 at 384)
    int64_t part_items = 0;
    for (int b = 0; b < B; ++b)
        if (T[b] > chunk) part_items += (T[b] + chunk - 1) / chunk * row_tiles;
    const int64_t part_mib = part_items * ROWS_WG * kPartialRowBytes >> 20;
    const int64_t items_all = items + (int64_t)nt * row_tiles;
    const int64_t part_cost = items_all <= cus ? part_mib : part_mib / 16;
    return finish + (split ? kMergeCost : 0) + part_cost;
}

// The key chunk with the lowest estimated finish time among chunks that cut
// the longest request into 1 to 32 equal parts, that give the CUs 1 to 16
// rounds of equal work (a spread of each), and the smallest chunk (ties go
// to the larger chunk: fewer partial outputs).
int64_t choose_chunk(const ddt_attn_desc* d, const int32_t* P, int row_tiles, int cus) {
    int64_t T[DDT_MAX_BATCH];
    int64_t tmax = 0, work = 0;
    for (int b = 0; b < d->B; ++b) {
        T[b] = (int64_t)P[b] + d->N;
        tmax = T[b] > tmax ? T[b] : tmax;
        work += T[b] * row_tiles;
    }
    const int64_t top = (int64_t)ddt::round_up((size_t)tmax, KT);
    int64_t best = top, best_cost = plan_cost(T, d->B, row_tiles, top, cus);
    int64_t tried[64];
    int nt = 0;
    auto consider = [&](int64_t c) {
        c = (int64_t)ddt::round_up((size_t)c, KT);
        if (c < kMinChunk) c = kMinChunk;
        if (c > top) c = top;
        for (int i = 0; i < nt; ++i)
            if (tried[i] == c) return;
        if (nt < 64) tried[nt++] = c;
        const int64_t cost = plan_cost(T, d->B, row_tiles, c, cus);
        if (cost < best_cost || (cost == best_cost && c > best)) best = c, best_cost = cost;
    };
    consider(kMinChunk);
    static const int kParts[] = {2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 14, 16, 20, 24, 28, 32};
    for (const int m : kParts) consider((tmax + m - 1) / m);
    static const int kRounds[] = {1, 2, 3, 4, 5, 6, 8, 10, 12, 16};
    for (const int k : kRounds) consider((work + (int64_t)k * cus - 1) / ((int64_t)k * cus));
    return best;
}

constexpr int kUnitRows = 8;  // row tiles of one key split dealt to one XCD together
constexpr int64_t kTouchMinBytes = 192ll << 20;  // key stream size above which tiles are touched into L2

Plan make_plan(const ddt_attn_desc* d, const int32_t* P, VerifyParams* vp) {
    Plan pl;
    const int rows = d->H * d->N;
    pl.row_tiles = (rows + ROWS_WG - 1) / ROWS_WG;
    const int cus = num_cus();
    if (d->kv_chunk > 0)
        pl.chunk = (int)std::min<int64_t>((int64_t)ddt::round_up((size_t)d->kv_chunk, KT), int64_t(1) << 30);
    else
        pl.chunk = (int)choose_chunk(d, P, pl.row_tiles, cus);
    int64_t total = 0;
    int n_full = 0;
    for (int b = 0; b < d->B; ++b) {
        const int64_t T = (int64_t)P[b] + d->N;
        const int ns = (int)((T + pl.chunk - 1) / pl.chunk);
        if (ns > 1) pl.any_split = true;
        if (vp) {
            vp->P[b] = P[b];
            vp->nsplit[b] = ns;
            vp->wg_begin[b] = (int)total;
            vp->full_gbegin[b] = n_full;
        }
        n_full += (int)(T / pl.chunk);
        total += (int64_t)ns * pl.row_tiles;
    }
    if (total > 0x7fffffff) total = 0x7fffffff;
    pl.total_wg = (int)total;
    // last splits shorter than a chunk, longest first
    int order[DDT_MAX_BATCH];
    int n_part = 0;
    for (int b = 0; b < d->B; ++b)
        if (((int64_t)P[b] + d->N) % pl.chunk) order[n_part++] = b;
    std::stable_sort(order, order + n_part, [&](int a, int c) {
        return ((int64_t)P[a] + d->N) % pl.chunk > ((int64_t)P[c] + d->N) % pl.chunk;
    });
    // units of kUnitRows row tiles that share a key split through one XCD's
    // L2, dealt whole while they fill all 8 XCDs equally, the rest row by
    // row (even XCD loads: with one round the idle CUs, which take the
    // argmax riding along, then sit evenly on all XCDs)
    const int unit_rows = pl.row_tiles < kUnitRows ? pl.row_tiles : kUnitRows;
    const int upg = (pl.row_tiles + unit_rows - 1) / unit_rows;
    const int64_t n_units = (int64_t)(n_full + n_part) * upg;
    const int64_t whole = n_units / ddt::kXcds * ddt::kXcds * unit_rows;
    const int64_t rest = (n_units % ddt::kXcds) * unit_rows;
    const int64_t blocks = whole + (rest + ddt::kXcds - 1) / ddt::kXcds * ddt::kXcds;
    pl.n_blocks = pl.total_wg <= cus ? pl.total_wg : (blocks > 0x7fffffff ? 0x7fffffff : (int)blocks);
    // L2 touches pay off once the launch's key stream outgrows the
    // last-level cache (measured: +12 to +16 % at 318 MB to 1.45 GB,
    // neutral at 151 MB, a loss at 5 MB where the keys stay cached)
    int64_t key_bytes = 0;
    for (int b = 0; b < d->B; ++b)
        key_bytes += ((int64_t)P[b] + d->N) * (d->d_lat + d->d_rope) * ddt::elem_bytes(d->dtype);
    pl.touch = key_bytes > kTouchMinBytes;
    if (vp) {
        vp->wg_begin[d->B] = pl.total_wg;
        vp->full_gbegin[d->B] = n_full;
        for (int k = 0; k < n_part; ++k) vp->part_b[k] = order[k];
        vp->n_full_groups = n_full;
        vp->n_units = (int)n_units;
        vp->whole_blocks = (int)whole;
        vp->single_round = pl.total_wg <= cus ? 1 : 0;
        // trees past 128 nodes (prefill chunks, causal): a row tile's keys end
        // at its last node, so later row tiles are longer work items; dealt
        // longest first they pack the CUs tighter (a host simulation of the
        // dispatch: 5 % shorter for an 8192-token prompt in 1024-token chunks)
        vp->rt_desc = d->N > 128 ? 1 : 0;
        vp->unit_rows = unit_rows;
        vp->units_per_group = upg;
    }
    if (pl.any_split) {
        const size_t o = (size_t)pl.total_wg * ROWS_WG * d->d_lat * sizeof(float);
        pl.ws_ml_off = ddt::round_up(o, 256);
        pl.ws_bytes = pl.ws_ml_off + ddt::round_up((size_t)pl.total_wg * ROWS_WG * sizeof(float2), 256);
    }
    return pl;
}

template <typename T, int DL, int DR>
int launch(const VerifyParams& vp, const Plan& pl, int n_argmax, hipStream_t stream) {
    const dim3 grid(pl.n_blocks + n_argmax);
    // trees of more than 128 nodes (prefill chunks) skip keys past each
    // work item's last node; the argmax co-task rides with verify-sized trees
    const bool clip = vp.N > 128 && n_argmax == 0;
    auto split = [&](auto paged) {
        constexpr bool kP = decltype(paged)::value;
        if (n_argmax > 0) {
            if (pl.touch)
                hipLaunchKernelGGL((verify_split<T, DL, DR, true, true, kP, false>), grid, dim3(kThreads), 0, stream,
                                   vp);
            else
                hipLaunchKernelGGL((verify_split<T, DL, DR, true, false, kP, false>), grid, dim3(kThreads), 0, stream,
                                   vp);
        } else if (clip) {
            if (pl.touch)
                hipLaunchKernelGGL((verify_split<T, DL, DR, false, true, kP, true>), grid, dim3(kThreads), 0, stream,
                                   vp);
            else
                hipLaunchKernelGGL((verify_split<T, DL, DR, false, false, kP, true>), grid, dim3(kThreads), 0, stream,
                                   vp);
        } else {
            if (pl.touch)
                hipLaunchKernelGGL((verify_split<T, DL, DR, false, true, kP, false>), grid, dim3(kThreads), 0, stream,
                                   vp);
            else
                hipLaunchKernelGGL((verify_split<T, DL, DR, false, false, kP, false>), grid, dim3(kThreads), 0,
                                   stream, vp);
        }
    };
    if constexpr (std::is_same<T, uint16_t>::value) {  // paged caches: the bf16 instance
        if (vp.map.table != nullptr)
            split(std::true_type{});
        else
            split(std::false_type{});
    } else {
        split(std::false_type{});
    }
    DDT_CHECK_LAUNCH();
    const int nblk = pl.any_split ? vp.B * pl.row_tiles * NW * (DL / 64) : 0;
    if (vp.n_accept > 0) {
        hipLaunchKernelGGL((verify_combine<T, DL, true>), dim3(vp.n_accept + nblk), dim3(256), 0, stream, vp);
        DDT_CHECK_LAUNCH();
    } else if (nblk > 0) {
        hipLaunchKernelGGL((verify_combine<T, DL, false>), dim3(nblk), dim3(256), 0, stream, vp);
        DDT_CHECK_LAUNCH();
    }
    return DDT_OK;
}

// Validates the call and fills the attention part of the launch parameters.
// A null mask takes the ancestor bits from `parents` in the kernel.
int setup_attn(const ddt_attn_desc* d, const void* q_lat, const void* q_pe, const void* ckv, const void* kpe,
               const int64_t* kv_base, const int32_t* prefix_len_host, const uint64_t* mask, const int32_t* parents,
               void* out, float* lse, void* workspace, size_t workspace_bytes, VerifyParams* vp, Plan* pl) {
    int rc = check_desc(d, prefix_len_host);
    if (rc != DDT_OK) return rc;
    if (!q_lat || !q_pe || !ckv || !kpe || !out || !lse) return DDT_EINVAL;
    if (!kv_base && !d->block_table) return DDT_EINVAL;
    if (!mask && !parents) return DDT_EINVAL;
    if (!mask && d->N > 128) return DDT_EINVAL;  // in-kernel ancestor bits cover two words
    if (!ddt::aligned(q_lat, 16) || !ddt::aligned(q_pe, 16) || !ddt::aligned(ckv, 16) || !ddt::aligned(kpe, 16) ||
        !ddt::aligned(out, 16) || !ddt::aligned(lse, 4))
        return DDT_EINVAL;
    *pl = make_plan(d, prefix_len_host, vp);
    if (pl->ws_bytes > 0) {
        if (workspace == nullptr || workspace_bytes < pl->ws_bytes || !ddt::aligned(workspace, 256))
            return DDT_EWORKSPACE;
        vp->ws_o = workspace;
        vp->ws_ml = reinterpret_cast<float2*>(static_cast<char*>(workspace) + pl->ws_ml_off);
    }
    vp->q_lat = q_lat;
    vp->q_pe = q_pe;
    vp->ckv = ckv;
    vp->kpe = kpe;
    vp->map = ddt::SlotMap{kv_base, d->block_table, d->block_table ? d->bt_ld : 0,
                           d->block_table ? __builtin_ctz((unsigned)d->page_size) : 0};
    vp->P_dev = d->prefix_len_dev;
    vp->mask = mask;
    vp->parents = mask ? nullptr : parents;
    vp->out = out;
    vp->lse = lse;
    vp->ld_ql = d->ld_ql;
    vp->ld_qp = d->ld_qp;
    vp->ld_ckv = d->ld_ckv;
    vp->ld_kpe = d->ld_kpe;
    vp->B = d->B;
    vp->H = d->H;
    vp->N = d->N;
    vp->W = (d->N + 63) / 64;
    vp->rows = d->H * d->N;
    vp->row_tiles = pl->row_tiles;
    vp->chunk = pl->chunk;
    vp->total_wg = pl->total_wg;
    vp->n_attn = pl->n_blocks;
    vp->scale_log2 = d->scale * kLog2e;
    return DDT_OK;
}

int run(const ddt_attn_desc* d, const VerifyParams& vp, const Plan& pl, int n_argmax, hipStream_t stream) {
    if (d->dtype == DDT_BF16) return launch<uint16_t, 512, 64>(vp, pl, n_argmax, stream);
    return launch<float, 64, 16>(vp, pl, n_argmax, stream);
}

// Validates the argmax task (as ddt_argmax does) and fills its part of the
// launch parameters; *wgs receives the number of argmax workgroups (0 for
// an empty task).
int setup_argmax(const ddt_argmax_task* am, const Plan& pl, VerifyParams* vp, int* n_wgs) {
    *n_wgs = 0;
    if (am == nullptr) return DDT_EINVAL;
    if (am->rows < 0 || am->V < 1 || am->V > 0x7fffffff || am->ld < am->V) return DDT_EINVAL;
    if (am->dtype != DDT_F32 && am->dtype != DDT_BF16) return DDT_EUNSUPPORTED;
    if (am->rows == 0) return DDT_OK;
    if (am->logits == nullptr || am->idx == nullptr || am->rows > 0x7fffffff / 64) return DDT_EINVAL;
    size_t need = 0;
    ddt_argmax_workspace(am->rows, am->V, &need);
    if (need > 0 && (am->workspace == nullptr || am->workspace_bytes < need || !ddt::aligned(am->workspace, 16)))
        return DDT_EWORKSPACE;
    // one argmax workgroup per CU the attention leaves idle, each taking an
    // equal share of the flattened rows x V range; when the attention takes
    // every CU (several rounds), two workgroups per CU that start as the
    // attention's last workgroups end; rows are shared between workgroups
    // only where the workspace can merge them
    const int cus = num_cus();
    int64_t wgs = pl.total_wg < cus ? cus - pl.total_wg : 2 * (int64_t)cus;
    if (wgs < 1) wgs = 1;
    const int64_t es = ddt::elem_bytes(am->dtype);
    const int64_t vec_elems = 16 / es;
    const int64_t total = am->rows * am->V;
    int64_t E;
    if (need > 0) {
        E = (int64_t)ddt::round_up((size_t)((total + wgs - 1) / wgs), (size_t)ddt::kChunkAlign);
    } else {
        // rows may not be split: whole rows per workgroup
        const int64_t rpw = (am->rows + wgs - 1) / wgs;
        E = rpw * am->V;
    }
    wgs = (total + E - 1) / E;
    vp->am_wgs = (int)wgs;
    vp->am_dtype = am->dtype;
    vp->am_vec = ddt::aligned(am->logits, 16) && (am->ld * es) % 16 == 0 && am->V % vec_elems == 0;
    vp->am_rows = am->rows;
    vp->am_V = am->V;
    vp->am_ld = am->ld;
    vp->am_E = E;
    vp->am_logits = am->logits;
    vp->am_idx = am->idx;
    vp->am_slots = static_cast<ddt::RowSlot*>(am->workspace);
    *n_wgs = (int)wgs;
    return DDT_OK;
}

// Scratch of ddt_verify_attn_noalloc: the split partials in a file-scope
// device array instead of a caller workspace (each device the library runs
// on holds its own copy until the process ends).  Host code never uses the
// array's name as an address: scratch_ptr() asks the runtime for this
// device's copy once and keeps it.
constexpr size_t kNoAllocScratchBytes = (size_t)DDT_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (looked up on the first call on
// that device, with that device current); DDT_OK or DDT_EHIP.
int scratch_ptr(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DDT_EHIP;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        // (two threads may both look it up: the runtime returns the same address)
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return DDT_EHIP;
        }
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
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

extern "C" int ddt_verify_plan(const ddt_attn_desc* d, const int32_t* prefix_len_host, int* n_blocks, int* chunk,
                               int32_t* nsplit, int32_t* items, int cap, int* n_items) {
    if (n_blocks == nullptr || chunk == nullptr || n_items == nullptr) return DDT_EINVAL;
    const int rc = check_desc(d, prefix_len_host);
    if (rc != DDT_OK) return rc;
    VerifyParams vp{};
    const Plan pl = make_plan(d, prefix_len_host, &vp);
    *n_blocks = pl.n_blocks;
    *chunk = pl.chunk;
    if (nsplit != nullptr)
        for (int b = 0; b < d->B; ++b) nsplit[b] = vp.nsplit[b];
    // the fields work_item reads besides the plan's (setup_attn sets them for a launch)
    vp.B = d->B;
    vp.H = d->H;
    vp.N = d->N;
    vp.rows = d->H * d->N;
    vp.row_tiles = pl.row_tiles;
    vp.chunk = pl.chunk;
    vp.total_wg = pl.total_wg;
    int n = 0;
    for (int blk = 0; blk < pl.n_blocks; ++blk) {
        int b, split, rt;
        if (!work_item(vp, blk, b, split, rt)) continue;
        if (items != nullptr && n < cap) {
            const int64_t T = (int64_t)prefix_len_host[b] + d->N, k0 = (int64_t)split * pl.chunk;
            int32_t* it = items + 6 * (int64_t)n;
            it[0] = blk;
            it[1] = b;
            it[2] = split;
            it[3] = rt;
            it[4] = (int32_t)k0;
            it[5] = (int32_t)(k0 + pl.chunk < T ? k0 + pl.chunk : T);
        }
        ++n;
    }
    *n_items = n;
    return items != nullptr && cap < n ? DDT_EINVAL : DDT_OK;
}

extern "C" int ddt_verify_attn(const ddt_attn_desc* d, const void* q_lat, const void* q_pe, const void* ckv,
                               const void* kpe, const int64_t* kv_base, const int32_t* prefix_len_host,
                               const uint64_t* mask, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    VerifyParams vp{};
    Plan pl;
    const int rc = setup_attn(d, q_lat, q_pe, ckv, kpe, kv_base, prefix_len_host, mask, nullptr, out, lse,
                              workspace, workspace_bytes, &vp, &pl);
    if (rc != DDT_OK) return rc;
    return run(d, vp, pl, 0, stream);
}

extern "C" int ddt_verify_attn_noalloc(const ddt_attn_desc* d, const void* q_lat, const void* q_pe, const void* ckv,
                                       const void* kpe, const int64_t* kv_base, const int32_t* prefix_len_host,
                                       const uint64_t* mask, void* out, float* lse, hipStream_t stream) {
    const int rc0 = check_desc(d, prefix_len_host);
    if (rc0 != DDT_OK) return rc0;
    // the same plan as ddt_verify_attn; its partials must fit the scratch
    if (make_plan(d, prefix_len_host, nullptr).ws_bytes > kNoAllocScratchBytes) return DDT_EWORKSPACE;
    void* ws = nullptr;
    const int rs = scratch_ptr(&ws);
    if (rs != DDT_OK) return rs;
    VerifyParams vp{};
    Plan pl;
    const int rc = setup_attn(d, q_lat, q_pe, ckv, kpe, kv_base, prefix_len_host, mask, nullptr, out, lse, ws,
                              kNoAllocScratchBytes, &vp, &pl);
    if (rc != DDT_OK) return rc;
    return run(d, vp, pl, 0, stream);
}

extern "C" size_t ddt_verify_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

extern "C" int ddt_verify_attn_argmax(const ddt_attn_desc* d, const void* q_lat, const void* q_pe, const void* ckv,
                                      const void* kpe, const int64_t* kv_base, const int32_t* prefix_len_host,
                                      const uint64_t* mask, void* out, float* lse, void* workspace,
                                      size_t workspace_bytes, const ddt_argmax_task* am, hipStream_t stream) {
    VerifyParams vp{};
    Plan pl;
    int rc = setup_attn(d, q_lat, q_pe, ckv, kpe, kv_base, prefix_len_host, mask, nullptr, out, lse,
                        workspace, workspace_bytes, &vp, &pl);
    if (rc != DDT_OK) return rc;
    int wgs = 0;
    rc = setup_argmax(am, pl, &vp, &wgs);
    if (rc != DDT_OK) return rc;
    return run(d, vp, pl, wgs, stream);
}

extern "C" int ddt_verify_step(const ddt_attn_desc* d, const void* q_lat, const void* q_pe, void* ckv, void* kpe,
                               const int64_t* kv_base, const int32_t* prefix_len_host, const uint64_t* mask,
                               void* out, float* lse, void* workspace, size_t workspace_bytes,
                               const ddt_argmax_task* am, const ddt_accept_task* acc, hipStream_t stream) {
    if (am == nullptr || acc == nullptr) return DDT_EINVAL;
    VerifyParams vp{};
    Plan pl;
    int rc = setup_attn(d, q_lat, q_pe, ckv, kpe, kv_base, prefix_len_host, mask, acc->parents, out, lse,
                        workspace, workspace_bytes, &vp, &pl);
    if (rc != DDT_OK) return rc;
    if (am->rows != (int64_t)d->B * d->N) return DDT_EINVAL;  // one target row per tree node
    int wgs = 0;
    rc = setup_argmax(am, pl, &vp, &wgs);
    if (rc != DDT_OK) return rc;
    if (!acc->draft_ids || !acc->parents || !acc->accept_len || !acc->path || !acc->tokens || !acc->prefix_len ||
        !acc->new_prefix_len)
        return DDT_EINVAL;
    ddt::CompactLayout lay;
    rc = ddt::compact_layout(ckv, d->ld_ckv, kpe, d->ld_kpe, d->dtype, d->d_lat, d->d_rope, d->N, &lay);
    if (rc != DDT_OK) return rc;
    vp.n_accept = d->B;
    vp.acc_vec16 = lay.vec16 ? 1 : 0;
    vp.acc = ddt::AcceptCompactArgs{am->idx, acc->draft_ids, acc->parents, d->N, acc->accept_len, acc->path,
                                    acc->tokens, static_cast<char*>(ckv), static_cast<char*>(kpe), lay.lc, lay.lk,
                                    lay.ckv_units, lay.kpe_units, lay.rows_per_block, vp.map, acc->prefix_len,
                                    acc->new_prefix_len, acc->src_slot};
    return run(d, vp, pl, wgs, stream);
}
