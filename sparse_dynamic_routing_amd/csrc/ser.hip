// Sparse edge referral (SER), forward and backward, for gfx950.
//
// Forward (ai.info "Graph Machine: Towards Better Pretraining via Edges",
// Key Contributions 3: A' = Sparsify_s1(A1 A2) over the up-to s2*s3 two-hop
// candidates; Methodology: the first leg's indices fetch the second leg's
// indices and weights, then a hard cut to the s1 largest; rit.work article:
// paths to the same address are merged and the heaviest kept).
//
// One lane per path: a team of L = pow2(s2*s3) lanes per unit (b, i, h);
// lane a*s3 + c follows leg-1 slot a to token j and reads leg-2 slot c of
// row j.  The whole row fits one wavefront, so the merge and the top-s1 run
// in registers with cross-lane shuffles:
//   merge  each lane scans the team's lanes in path order (a, c) and sums,
//          in double starting from 0, the path weights (exact fp32*fp32
//          products) whose target equals its own; the lowest such lane owns
//          the target.  This is the order and precision of the definition,
//          so the fp32-rounded weight is bit-exact.
//   rank   an owner's rank is the number of owners with a larger positive
//          weight, or the same weight and a lower index; ranks < s1 write
//          their slot.  A ballot counts the owners; the remaining slots get
//          the padding edge (0, 0.0f).
//
// Backward (ai.info Methodology: gradients reach the kept weights alone): for
// each path whose target is a retained slot t (w_out_t > 0) and whose two
// leg weights are positive, dw1[i,a] += dw_out_t w2[j,c] and
// dw2[j,c] += dw_out_t w1[i,a].  Contributions are added in fp64 with
// atomics into a workspace (dw2 lands in other tokens' rows), then rounded
// once to fp32.  When dw1 and dw2 alias, one workspace receives both.
#include "gm_common.h"
#include "gm_internal.h"
#include "gm_select.h"
#include "gm_wave.h"

namespace gm {
namespace {

struct SerArgs {
    const int32_t* idx1;
    const float* w1;
    const int32_t* idx2;
    const float* w2;
    int32_t* idx_out;
    float* w_out;
    int n, hkv, s1, s2, s3, U;
};

template <int L>
__global__ __launch_bounds__(kBlock) void ser_fwd_kernel(SerArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int sub = lane & (L - 1);
    const int base = lane & ~(L - 1);
    const long long gunit = ((long long)blockIdx.x * kBlock + threadIdx.x) / L;
    if (gunit >= a.U) return;  // whole team leaves together
    const int unit = (int)gunit;
    const int ncand = a.s2 * a.s3;
    const bool valid = sub < ncand;
    int m = -1;
    double cw = 0.0;
    if (valid) {
        const int h = unit % a.hkv;
        const int b = unit / a.hkv / a.n;
        const int la = sub / a.s3;
        const int lc = sub - la * a.s3;
        const int j = a.idx1[(size_t)unit * a.s2 + la];
        const float x = a.w1[(size_t)unit * a.s2 + la];
        const size_t r2 = ((size_t)b * a.n + j) * a.hkv + h;
        m = a.idx2[r2 * a.s3 + lc];
        const float y = a.w2[r2 * a.s3 + lc];
        cw = (double)x * (double)y;  // exact: 24-bit x 24-bit mantissas
    }
    // merge duplicate targets, summing in path order
    double acc = 0.0;
    bool owner = valid;
#pragma unroll
    for (int k = 0; k < L; ++k) {
        const int mk = __shfl(m, base + k, kWave);
        const double ck = __shfl(cw, base + k, kWave);
        if (valid && mk == m) {
            acc += ck;
            if (k < sub) owner = false;
        }
    }
    const float key = (float)acc;
    const bool cand = owner && key > 0.0f;
    // rank among candidates: larger weight first, then lower index
    int rank = 0;
#pragma unroll
    for (int k = 0; k < L; ++k) {
        const float kk = __shfl(key, base + k, kWave);
        const int mk = __shfl(m, base + k, kWave);
        const int ck = __shfl((int)cand, base + k, kWave);
        if (ck && (kk > key || (kk == key && mk < m))) ++rank;
    }
    const size_t ob = (size_t)unit * a.s1;
    if (cand && rank < a.s1) {
        a.idx_out[ob + rank] = m;
        a.w_out[ob + rank] = key;
    }
    const unsigned long long bal = __ballot(cand);
    const unsigned long long mask = (L == 64) ? ~0ull : (((1ull << L) - 1ull) << base);
    const int nd = __popcll(bal & mask);
    for (int p = nd + sub; p < a.s1; p += L) {
        a.idx_out[ob + p] = 0;
        a.w_out[ob + p] = 0.0f;
    }
}

struct SerBwdArgs {
    const int32_t* idx1;
    const float* w1;
    const int32_t* idx2;
    const float* w2;
    const int32_t* idx_out;
    const float* w_out;
    const float* dw_out;
    double* ws1;
    double* ws2;
    int n, hkv, s1, s2, s3, U;
};

template <int L>
__global__ __launch_bounds__(kBlock) void ser_bwd_kernel(SerBwdArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int sub = lane & (L - 1);
    const long long gunit = ((long long)blockIdx.x * kBlock + threadIdx.x) / L;
    if (gunit >= a.U) return;
    const int unit = (int)gunit;
    if (sub >= a.s2 * a.s3) return;   // no cross-lane traffic below
    const int h = unit % a.hkv;
    const int b = unit / a.hkv / a.n;
    const int la = sub / a.s3;
    const int lc = sub - la * a.s3;
    const float x = a.w1[(size_t)unit * a.s2 + la];
    if (!(x > 0.0f)) return;
    const int j = a.idx1[(size_t)unit * a.s2 + la];
    const size_t r2 = ((size_t)b * a.n + j) * a.hkv + h;
    const int m = a.idx2[r2 * a.s3 + lc];
    const float y = a.w2[r2 * a.s3 + lc];
    if (!(y > 0.0f)) return;
    double g = 0.0;
    bool hit = false;
    const size_t ob = (size_t)unit * a.s1;
    for (int t = 0; t < a.s1; ++t) {
        if (a.w_out[ob + t] > 0.0f && a.idx_out[ob + t] == m) {
            g += (double)a.dw_out[ob + t];
            hit = true;
        }
    }
    if (!hit) return;
    unsafeAtomicAdd(a.ws1 + (size_t)unit * a.s2 + la, g * (double)y);
    unsafeAtomicAdd(a.ws2 + r2 * a.s3 + lc, g * (double)x);
}


// ----------------------------------------------------- one lane per unit
// For s2, s3 <= 4 (at most 16 candidates) a lane holds a whole unit: its
// leg-1 row, the leg-2 rows it points to and all candidates live in
// registers (static indices, candidate k = 4a + c), so the merge and the
// ranking need no cross-lane traffic and a wave serves 64 units.  The merge
// scans the candidates in path order (a, c) and adds each path weight to the
// first candidate with the same target, from 0 and in double: the order and
// precision of the definition, hence bit-exact fp32 weights.
struct SerUnitArgs {
    const int32_t* idx1;
    const float* w1;
    const int32_t* idx2;
    const float* w2;
    int32_t* idx_out;
    float* w_out;
    const float* dw_out;   // backward only
    double* ws1;           // backward: dw1 per leg-1 slot (plain stores)
    double* ws2;           // backward: dw2 per leg-2 slot (atomics)
    int n, hkv, s1, s2, s3, U;
    FastDiv fd_hkv, fd_n;
    int vec_out;           // forward: outputs 16-byte aligned, s1 == 4
    int vec_in;            // legs 16-byte aligned, s2 == s3 == 4: one load per row
    uint64_t* paths = nullptr;   // forward: the path map of every unit, or null
};

constexpr int kSmax = 4;
constexpr int kCand = kSmax * kSmax;

// Path map of a unit (s2, s3, s1 <= 4): 4 bits per path k = 4a + c (leg-1
// slot a, leg-2 slot c), the slot of A' whose target the path reaches, or
// kNoSlot when the path has a zero leg weight or its target was not kept.
// With it the backward knows every path's gradient dw'[slot] without
// gathering the leg-2 indices or reading A' again.
constexpr uint32_t kNoSlot = 15;
__device__ __forceinline__ uint64_t path_map(const int (&m)[kCand], const float (&x)[kSmax],
                                             const float (&y)[kCand], const int (&om)[kSmax],
                                             const float (&ow)[kSmax], int s1) {
    uint64_t mp = 0;
#pragma unroll
    for (int k = 0; k < kCand; ++k) {
        uint32_t sl = kNoSlot;
        if (m[k] >= 0 && x[k / kSmax] > 0.0f && y[k] > 0.0f) {
#pragma unroll
            for (int r = 0; r < kSmax; ++r) sl = r < s1 && ow[r] > 0.0f && om[r] == m[k] ? r : sl;
        }
        mp |= (uint64_t)sl << (4 * k);
    }
    return mp;
}

// Token i of unit u (u = (b*n + i)*hkv + h); the row of token j of the same
// (b, h) is u + (j - i) * hkv.
__device__ __forceinline__ int token_of(int u, const SerUnitArgs& a) {
    const int bi = (int)fdiv((uint32_t)u, a.fd_hkv);
    return bi - (int)fdiv((uint32_t)bi, a.fd_n) * a.n;
}

// Load the unit's paths: m[k] target, x[k] leg-1 weight, y[k] leg-2 weight,
// r2[a] leg-2 row; invalid candidates get m = -1.
__device__ __forceinline__ void load_paths(const SerUnitArgs& a, int u, int (&m)[kCand],
                                           float (&x)[kSmax], float (&y)[kCand],
                                           int (&r2)[kSmax]) {
    const int i = token_of(u, a);
    int j[kSmax];
    if (a.vec_in) {
        const int4 ji = *reinterpret_cast<const int4*>(a.idx1 + (size_t)u * 4);
        const float4 xi = *reinterpret_cast<const float4*>(a.w1 + (size_t)u * 4);
        j[0] = ji.x; j[1] = ji.y; j[2] = ji.z; j[3] = ji.w;
        x[0] = xi.x; x[1] = xi.y; x[2] = xi.z; x[3] = xi.w;
#pragma unroll
        for (int aa = 0; aa < kSmax; ++aa) r2[aa] = u + (j[aa] - i) * a.hkv;
#pragma unroll
        for (int aa = 0; aa < kSmax; ++aa) {
            const int4 mi = *reinterpret_cast<const int4*>(a.idx2 + (size_t)r2[aa] * 4);
            const float4 yi = *reinterpret_cast<const float4*>(a.w2 + (size_t)r2[aa] * 4);
            m[aa * 4 + 0] = mi.x; m[aa * 4 + 1] = mi.y; m[aa * 4 + 2] = mi.z; m[aa * 4 + 3] = mi.w;
            y[aa * 4 + 0] = yi.x; y[aa * 4 + 1] = yi.y; y[aa * 4 + 2] = yi.z; y[aa * 4 + 3] = yi.w;
        }
        return;
    }
#pragma unroll
    for (int aa = 0; aa < kSmax; ++aa) {
        j[aa] = 0;
        x[aa] = 0.0f;
        if (aa < a.s2) {
            j[aa] = a.idx1[(size_t)u * a.s2 + aa];
            x[aa] = a.w1[(size_t)u * a.s2 + aa];
        }
        r2[aa] = u + (j[aa] - i) * a.hkv;
    }
#pragma unroll
    for (int aa = 0; aa < kSmax; ++aa) {
#pragma unroll
        for (int c = 0; c < kSmax; ++c) {
            const int k = aa * kSmax + c;
            m[k] = -1;
            y[k] = 0.0f;
            if (aa < a.s2 && c < a.s3) {
                m[k] = a.idx2[(size_t)r2[aa] * a.s3 + c];
                y[k] = a.w2[(size_t)r2[aa] * a.s3 + c];
            }
        }
    }
}

__global__ __launch_bounds__(kBlock) void ser_fwd_unit_kernel(SerUnitArgs a) {
    const int u = xcd_unit(a.U);
    if (u < 0) return;
    int m[kCand];
    float x[kSmax], y[kCand];
    int r2[kSmax];
    load_paths(a, u, m, x, y, r2);
    // merge in path order
    double acc[kCand];
    bool own[kCand];
#pragma unroll
    for (int k = 0; k < kCand; ++k) {
        const double cw = (double)x[k / kSmax] * (double)y[k];
        bool matched = false;
#pragma unroll
        for (int k2 = 0; k2 < k; ++k2) {
            const bool hit = !matched && m[k] >= 0 && m[k2] == m[k];
            acc[k2] = hit ? acc[k2] + cw : acc[k2];
            matched = matched || hit;
        }
        own[k] = m[k] >= 0 && !matched;
        acc[k] = own[k] ? 0.0 + cw : 0.0;
    }
    float key[kCand];
    bool cand[kCand];
    int nd = 0;
#pragma unroll
    for (int k = 0; k < kCand; ++k) {
        key[k] = (float)acc[k];
        cand[k] = own[k] && key[k] > 0.0f;
        nd += cand[k];
    }
    // rank: larger weight first, then lower index
    int om[kSmax];
    float ow[kSmax];
#pragma unroll
    for (int r = 0; r < kSmax; ++r) { om[r] = 0; ow[r] = 0.0f; }
    const size_t ob = (size_t)u * a.s1;
#pragma unroll
    for (int k = 0; k < kCand; ++k) {
        int rank = 0;
#pragma unroll
        for (int k2 = 0; k2 < kCand; ++k2) {
            if (k2 == k) continue;
            rank += cand[k2] && (key[k2] > key[k] || (key[k2] == key[k] && m[k2] < m[k]));
        }
        if (a.s1 <= kSmax) {
#pragma unroll
            for (int r = 0; r < kSmax; ++r) {
                const bool put = cand[k] && rank == r;
                om[r] = put ? m[k] : om[r];
                ow[r] = put ? key[k] : ow[r];
            }
        } else if (cand[k] && rank < a.s1) {
            a.idx_out[ob + rank] = m[k];
            a.w_out[ob + rank] = key[k];
        }
    }
    if (a.s1 <= kSmax) {
        if (a.paths) a.paths[u] = path_map(m, x, y, om, ow, a.s1);
        if (a.vec_out) {
            *reinterpret_cast<int4*>(a.idx_out + ob) = make_int4(om[0], om[1], om[2], om[3]);
            *reinterpret_cast<float4*>(a.w_out + ob) = make_float4(ow[0], ow[1], ow[2], ow[3]);
        } else {
#pragma unroll
            for (int r = 0; r < kSmax; ++r) {
                if (r < a.s1) {
                    a.idx_out[ob + r] = om[r];
                    a.w_out[ob + r] = ow[r];
                }
            }
        }
    } else {
        for (int p = nd; p < a.s1; ++p) {
            a.idx_out[ob + p] = 0;
            a.w_out[ob + p] = 0.0f;
        }
    }
}

// ------------------------- s2 = s3 = 4 legs, s1 = 4 or 2, aligned rows
// Straight-line version of the lane-per-unit forward.  Merge: every path
// weight is added, in path order, to each earlier candidate (the weight when
// the targets match, else 0.0, which leaves these non-negative sums
// unchanged), so the first candidate of each target receives its paths'
// weights in the order and precision of the definition; later duplicates
// are not candidates.  Ranking: a selection network over 64-bit keys
// (weight bits << 32 | ~target; 0 = no candidate) orders larger weights
// first and, among equal weights, lower targets first; positive fp32
// weights compare like their bit patterns.
__device__ __forceinline__ void load_paths_vec(const SerUnitArgs& a, int u, int (&m)[kCand],
                                               float (&x)[kSmax], float (&y)[kCand]) {
    const int i = token_of(u, a);
    const int4 ji = *reinterpret_cast<const int4*>(a.idx1 + (size_t)u * 4);
    const float4 xi = *reinterpret_cast<const float4*>(a.w1 + (size_t)u * 4);
    const int j[4] = {ji.x, ji.y, ji.z, ji.w};
    x[0] = xi.x; x[1] = xi.y; x[2] = xi.z; x[3] = xi.w;
#pragma unroll
    for (int aa = 0; aa < kSmax; ++aa) {
        const int r2 = u + (j[aa] - i) * a.hkv;
        const int4 mi = *reinterpret_cast<const int4*>(a.idx2 + (size_t)r2 * 4);
        const float4 yi = *reinterpret_cast<const float4*>(a.w2 + (size_t)r2 * 4);
        m[aa * 4 + 0] = mi.x; m[aa * 4 + 1] = mi.y; m[aa * 4 + 2] = mi.z; m[aa * 4 + 3] = mi.w;
        y[aa * 4 + 0] = yi.x; y[aa * 4 + 1] = yi.y; y[aa * 4 + 2] = yi.z; y[aa * 4 + 3] = yi.w;
    }
}

// S1: retained slots (4, or 2 for the narrower top-2-of-16 budget).
// MAP: also write the path map (held to 128 registers, four wavefronts per
// SIMD: the map keeps the candidates' targets live through the sorting
// network; without it the kernel needs fewer)
template <int S1, bool MAP>
__global__ __launch_bounds__(kBlock, MAP ? 4 : 1) void ser_fwd_vec_kernel(SerUnitArgs a) {
    static_assert(S1 == 2 || S1 == 4, "vector stores of 2 or 4 slots");
    const int u = xcd_unit(a.U);
    if (u < 0) return;
    int m[kCand];
    float x[kSmax], y[kCand];
    load_paths_vec(a, u, m, x, y);
    // a candidate that repeats an earlier target gets bit 31 of its target
    // set (targets are >= 0): it then matches no later candidate, whose
    // weight goes to the earlier, first candidate of the target instead
    double cw[kCand], acc[kCand];
    uint32_t pos = 0;   // paths of positive weight (both legs > 0), for the path map
#pragma unroll
    for (int k = 0; k < kCand; ++k) {
        cw[k] = (double)x[k / kSmax] * (double)y[k];
        acc[k] = cw[k];
        pos |= (cw[k] > 0.0 ? 1u : 0u) << k;
    }
#pragma unroll
    for (int k = 1; k < kCand; ++k) {
        uint32_t dup = 0;
#pragma unroll
        for (int k2 = 0; k2 < k; ++k2) {
            const bool same = m[k2] == m[k];
            acc[k2] += same ? cw[k] : 0.0;
            dup |= same ? 0x80000000u : 0u;
        }
        m[k] = (int)((uint32_t)m[k] | dup);
    }
    uint64_t key[kCand];
#pragma unroll
    for (int k = 0; k < kCand; ++k) {
        const float wk = (float)acc[k];
        key[k] = m[k] >= 0 && wk > 0.0f
                     ? ((uint64_t)__float_as_uint(wk) << 32) | (uint32_t)~(uint32_t)m[k]
                     : 0ull;
    }
    sort4_desc(key + 0); sort4_desc(key + 4); sort4_desc(key + 8); sort4_desc(key + 12);
    merge_top4(key + 0, key + 4);
    merge_top4(key + 8, key + 12);
    merge_top4(key + 0, key + 8);
    int om[4];
    float ow[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        om[r] = key[r] ? (int)~(uint32_t)key[r] : 0;
        ow[r] = key[r] ? __uint_as_float((uint32_t)(key[r] >> 32)) : 0.0f;
    }
    if constexpr (S1 == 4) {
        *reinterpret_cast<int4*>(a.idx_out + (size_t)u * 4) =
            make_int4(om[0], om[1], om[2], om[3]);
        *reinterpret_cast<float4*>(a.w_out + (size_t)u * 4) =
            make_float4(ow[0], ow[1], ow[2], ow[3]);
    } else {
        *reinterpret_cast<int2*>(a.idx_out + (size_t)u * 2) = make_int2(om[0], om[1]);
        *reinterpret_cast<float2*>(a.w_out + (size_t)u * 2) = make_float2(ow[0], ow[1]);
    }
    if constexpr (MAP) {
        // targets with the duplicate mark (bit 31) cleared
        uint64_t mp = 0;
#pragma unroll
        for (int k = 0; k < kCand; ++k) {
            const int tk = (int)((uint32_t)m[k] & 0x7fffffffu);
            uint32_t sl = kNoSlot;
#pragma unroll
            for (int r = 0; r < S1; ++r) sl = ow[r] > 0.0f && om[r] == tk ? r : sl;
            sl = (pos >> k) & 1u ? sl : kNoSlot;
            mp |= (uint64_t)sl << (4 * k);
        }
        a.paths[u] = mp;
    }
}

// ------------------------------------------- two chained referral steps
// A2 = Sp(A1 A1) with A1 = Sp(A0 A0): the edge matrix raised to the power
// 4 by two referral steps, each mixing the edges the previous step left
// (ai.info Key Contributions 2, the l-th power of the edge matrix, here
// l = 2; Methodology: referral works on the current stored edges).
// Step 2 reads rows of A1 at any earlier token of the pair, rows that other
// workgroups would write, so one launch cannot wait for them without a
// grid-wide barrier.  Instead a lane owns unit i and ranks A1's row i from
// A0, then A1's rows at the S targets of that row (again from A0), and then
// A2's row i from those: S + 1 referrals of A0 and one of A1 per unit, with
// no intermediate tensor in memory (it may still be written, for a later
// backward).  Every row goes through the arithmetic of one referral step
// (path products in double, merged in path order, rounded once, ranked by
// weight then lower index), so A1 and A2 are bitwise those of two separate
// steps.  s1 = s2 = s3 = S, S = 2 or 4, rows S-word aligned.
struct SerChainArgs {
    const int32_t* idx;   // A0
    const float* w;
    int32_t* idx_mid;     // A1, or null
    float* w_mid;
    int32_t* idx_out;     // A2
    float* w_out;
    int hkv, U;
    FastDiv fd_hkv, fd_n;
    int n;
};

template <int S>
__device__ __forceinline__ void load_row(const int32_t* idx, const float* w, int row,
                                         int* m, float* y) {
    if constexpr (S == 4) {
        const int4 mi = *reinterpret_cast<const int4*>(idx + (size_t)row * 4);
        const float4 yi = *reinterpret_cast<const float4*>(w + (size_t)row * 4);
        m[0] = mi.x; m[1] = mi.y; m[2] = mi.z; m[3] = mi.w;
        y[0] = yi.x; y[1] = yi.y; y[2] = yi.z; y[3] = yi.w;
    } else {
        const int2 mi = *reinterpret_cast<const int2*>(idx + (size_t)row * 2);
        const float2 yi = *reinterpret_cast<const float2*>(w + (size_t)row * 2);
        m[0] = mi.x; m[1] = mi.y;
        y[0] = yi.x; y[1] = yi.y;
    }
}

template <int S>
__device__ __forceinline__ void store_row(int32_t* idx, float* w, int row, const int (&m)[S],
                                          const float (&y)[S]) {
    if constexpr (S == 4) {
        *reinterpret_cast<int4*>(idx + (size_t)row * 4) = make_int4(m[0], m[1], m[2], m[3]);
        *reinterpret_cast<float4*>(w + (size_t)row * 4) = make_float4(y[0], y[1], y[2], y[3]);
    } else {
        *reinterpret_cast<int2*>(idx + (size_t)row * 2) = make_int2(m[0], m[1]);
        *reinterpret_cast<float2*>(w + (size_t)row * 2) = make_float2(y[0], y[1]);
    }
}

template <int S, bool MID>
__global__ __launch_bounds__(kBlock) void ser_chain2_kernel(SerChainArgs a) {
    constexpr int C = S * S;
    const int u = xcd_unit(a.U);
    if (u < 0) return;
    const int bi = (int)fdiv((uint32_t)u, a.fd_hkv);
    const int i = bi - (int)fdiv((uint32_t)bi, a.fd_n) * a.n;
    // Rows r = 0 .. S + 1, one at a time: r = 0 is A1's row i, r = 1 .. S
    // A1's rows at the S targets of row i (the second step's leg 2), each
    // referred from A0; r = S + 1 is A2's row i, referred from those.  Rows
    // are parked in this lane's LDS slots.  The merge is written once, in
    // the loop body: ranked side by side (or behind a helper function) the
    // rows' merges hold far more registers than one (a single wavefront
    // per SIMD).
    __shared__ int2 park[(S + 1) * S][kBlock];
#pragma unroll 1
    for (int r = 0; r <= S + 1; ++r) {
        int m[C];
        float x[S], y[C];
        if (r <= S) {
            const int tgt = r == 0 ? i : park[r - 1][threadIdx.x].x;
            const int row = u + (tgt - i) * a.hkv;
            int j[S];
            load_row<S>(a.idx, a.w, row, j, x);
#pragma unroll
            for (int aa = 0; aa < S; ++aa)
                load_row<S>(a.idx, a.w, row + (j[aa] - tgt) * a.hkv, m + aa * S, y + aa * S);
        } else {
#pragma unroll
            for (int c = 0; c < S; ++c) x[c] = __int_as_float(park[c][threadIdx.x].y);
#pragma unroll
            for (int k = 0; k < C; ++k) {
                const int2 e = park[S + k][threadIdx.x];
                m[k] = e.x;
                y[k] = __int_as_float(e.y);
            }
        }
        // merge in path order (ser_fwd_vec_kernel's arithmetic), then rank
        double cw[C], acc[C];
#pragma unroll
        for (int k = 0; k < C; ++k) {
            cw[k] = (double)x[k / S] * (double)y[k];
            acc[k] = cw[k];
        }
#pragma unroll
        for (int k = 1; k < C; ++k) {
            uint32_t dup = 0;
#pragma unroll
            for (int k2 = 0; k2 < k; ++k2) {
                const bool same = m[k2] == m[k];
                acc[k2] += same ? cw[k] : 0.0;
                dup |= same ? 0x80000000u : 0u;
            }
            m[k] = (int)((uint32_t)m[k] | dup);
        }
        uint64_t key[C];
#pragma unroll
        for (int k = 0; k < C; ++k) {
            const float wk = (float)acc[k];
            key[k] = m[k] >= 0 && wk > 0.0f
                         ? ((uint64_t)__float_as_uint(wk) << 32) | (uint32_t)~(uint32_t)m[k]
                         : 0ull;
        }
        if constexpr (S == 4) {
            sort4_desc(key + 0); sort4_desc(key + 4); sort4_desc(key + 8); sort4_desc(key + 12);
            merge_top4(key + 0, key + 4);
            merge_top4(key + 8, key + 12);
            merge_top4(key + 0, key + 8);
        } else {
            sort4_desc(key);
        }
        int om[S];
        float ow[S];
#pragma unroll
        for (int c = 0; c < S; ++c) {
            om[c] = key[c] ? (int)~(uint32_t)key[c] : 0;
            ow[c] = key[c] ? __uint_as_float((uint32_t)(key[c] >> 32)) : 0.0f;
        }
        if (r <= S) {
#pragma unroll
            for (int c = 0; c < S; ++c)
                park[r * S + c][threadIdx.x] = make_int2(om[c], __float_as_int(ow[c]));
        }
        if (MID && r == 0) store_row<S>(a.idx_mid, a.w_mid, u, om, ow);
        if (r == S + 1) store_row<S>(a.idx_out, a.w_out, u, om, ow);
    }
}

__global__ __launch_bounds__(kBlock) void ser_bwd_unit_kernel(SerUnitArgs a) {
    const int u = blockIdx.x * kBlock + threadIdx.x;
    if (u >= a.U) return;
    if (a.paths && a.vec_in) {
        // with the forward's path map (s2 = s3 = 4): the leg-1 row, the map,
        // the leg-2 weights and dw' are enough; the same fp64 terms as below
        const int i = token_of(u, a);
        const int4 j4 = *reinterpret_cast<const int4*>(a.idx1 + (size_t)u * 4);
        const float4 x4 = *reinterpret_cast<const float4*>(a.w1 + (size_t)u * 4);
        const uint64_t mp = a.paths[u];
        const int j[4] = {j4.x, j4.y, j4.z, j4.w};
        const float x[4] = {x4.x, x4.y, x4.z, x4.w};
        float gt[kSmax];
#pragma unroll
        for (int t = 0; t < kSmax; ++t) gt[t] = t < a.s1 ? a.dw_out[(size_t)u * a.s1 + t] : 0.0f;
        float y[kCand];
        int r2[kSmax];
#pragma unroll
        for (int aa = 0; aa < kSmax; ++aa) {
            r2[aa] = u + (j[aa] - i) * a.hkv;
            const float4 yi = *reinterpret_cast<const float4*>(a.w2 + (size_t)r2[aa] * 4);
            y[aa * 4 + 0] = yi.x; y[aa * 4 + 1] = yi.y; y[aa * 4 + 2] = yi.z; y[aa * 4 + 3] = yi.w;
        }
        // the terms in the order of the path below: slot t, then path k
        double d1[kSmax];
#pragma unroll
        for (int aa = 0; aa < kSmax; ++aa) d1[aa] = 0.0;
#pragma unroll
        for (int t = 0; t < kSmax; ++t) {
            const double g = (double)gt[t];
#pragma unroll
            for (int k = 0; k < kCand; ++k) {
                if (((uint32_t)(mp >> (4 * k)) & 0xFu) != (uint32_t)t) continue;
                const int aa = k / kSmax;
                d1[aa] += g * (double)y[k];
                unsafeAtomicAdd(a.ws2 + (size_t)r2[aa] * a.s3 + (k % kSmax), g * (double)x[aa]);
            }
        }
#pragma unroll
        for (int aa = 0; aa < kSmax; ++aa) a.ws1[(size_t)u * a.s2 + aa] = d1[aa];
        return;
    }
    int m[kCand];
    float x[kSmax], y[kCand];
    int r2[kSmax];
    load_paths(a, u, m, x, y, r2);
    const size_t ob = (size_t)u * a.s1;
    double d1[kSmax];
#pragma unroll
    for (int aa = 0; aa < kSmax; ++aa) d1[aa] = 0.0;
    // gradient of each path: sum of dw_out over retained slots with its target
    auto slot = [&](int mt, float wt, float gt_) {
        if (!(wt > 0.0f)) return;
        const double gt = (double)gt_;
#pragma unroll
        for (int k = 0; k < kCand; ++k) {
            const int aa = k / kSmax;
            if (m[k] == mt && x[aa] > 0.0f && y[k] > 0.0f) {
                d1[aa] += gt * (double)y[k];
                unsafeAtomicAdd(a.ws2 + (size_t)r2[aa] * a.s3 + (k % kSmax), gt * (double)x[aa]);
            }
        }
    };
    if (a.vec_out) {
        const int4 mt = *reinterpret_cast<const int4*>(a.idx_out + ob);
        const float4 wt = *reinterpret_cast<const float4*>(a.w_out + ob);
        const float4 gt = *reinterpret_cast<const float4*>(a.dw_out + ob);
        slot(mt.x, wt.x, gt.x);
        slot(mt.y, wt.y, gt.y);
        slot(mt.z, wt.z, gt.z);
        slot(mt.w, wt.w, gt.w);
    } else {
        for (int t = 0; t < a.s1; ++t) slot(a.idx_out[ob + t], a.w_out[ob + t], a.dw_out[ob + t]);
    }
#pragma unroll
    for (int aa = 0; aa < kSmax; ++aa)
        if (aa < a.s2) a.ws1[(size_t)u * a.s2 + aa] = d1[aa];
}


// ------------------------------------------------- pull-style SER backward
// One lane per row r.  dw1 of row r comes from r's own paths (as above);
// dw2 of row r, i.e. the gradient of r's leg-2 slots, is pulled from the
// units whose leg-1 edges point at r, found in the reverse index of leg 1:
// for such an edge (unit i, slot a) with weight x and each leg-2 slot c of r
// with target m_c, the contribution is x * (sum of dw_out over i's retained
// slots with target m_c).  Every row is written once; no atomics.
struct SerPullArgs {
    const int32_t* idx1;
    const float* w1;
    const int32_t* idx2;
    const float* w2;
    const int32_t* idx_out;
    const float* w_out;
    const float* dw_out;
    float* dw1;
    float* dw2;
    const int* beg;
    const int* len;
    const int* list;
    int n, hkv, s1, s2, s3, U, aliased;
    FastDiv fd_hkv, fd_n, fd_s2;
    int vec_in, vec_ap;   // 16-byte rows: legs (s2 == s3 == 4), A' (s1 == 4)
};

// Retained slots of A' row u: target, weight (> 0 means retained), gradient.
__device__ __forceinline__ void load_aprime(const SerPullArgs& a, int u, int (&mt)[kSmax],
                                            float (&wt)[kSmax], float (&gt)[kSmax]) {
    const size_t ob = (size_t)u * a.s1;
    if (a.vec_ap) {
        const int4 m4 = *reinterpret_cast<const int4*>(a.idx_out + ob);
        const float4 w4 = *reinterpret_cast<const float4*>(a.w_out + ob);
        const float4 g4 = *reinterpret_cast<const float4*>(a.dw_out + ob);
        mt[0] = m4.x; mt[1] = m4.y; mt[2] = m4.z; mt[3] = m4.w;
        wt[0] = w4.x; wt[1] = w4.y; wt[2] = w4.z; wt[3] = w4.w;
        gt[0] = g4.x; gt[1] = g4.y; gt[2] = g4.z; gt[3] = g4.w;
        return;
    }
#pragma unroll
    for (int t = 0; t < kSmax; ++t) {
        mt[t] = -1;
        wt[t] = 0.0f;
        gt[t] = 0.0f;
        if (t < a.s1) {
            mt[t] = a.idx_out[ob + t];
            wt[t] = a.w_out[ob + t];
            gt[t] = a.dw_out[ob + t];
        }
    }
}

__device__ __forceinline__ double path_grad(int m, const int (&mt)[kSmax],
                                            const float (&wt)[kSmax], const float (&gt)[kSmax]) {
    double g = 0.0;
#pragma unroll
    for (int t = 0; t < kSmax; ++t)
        if (wt[t] > 0.0f && mt[t] == m) g += (double)gt[t];
    return g;
}

__global__ __launch_bounds__(kBlock) void ser_bwd_pull_kernel(SerPullArgs a) {
    const int u = xcd_unit(a.U);
    if (u < 0) return;
    SerUnitArgs ua{a.idx1, a.w1, a.idx2, a.w2, nullptr, nullptr, nullptr, nullptr, nullptr,
                   a.n, a.hkv, a.s1, a.s2, a.s3, a.U, a.fd_hkv, a.fd_n, 0, a.vec_in};
    int m[kCand];
    float x[kSmax], y[kCand];
    int r2[kSmax];
    load_paths(ua, u, m, x, y, r2);
    int mt[kSmax];
    float wt[kSmax], gt[kSmax];
    load_aprime(a, u, mt, wt, gt);
    double d1[kSmax], d2[kSmax];
#pragma unroll
    for (int aa = 0; aa < kSmax; ++aa) {
        d1[aa] = 0.0;
        d2[aa] = 0.0;
        if (!(x[aa] > 0.0f)) continue;
#pragma unroll
        for (int c = 0; c < kSmax; ++c) {
            const int k = aa * kSmax + c;
            if (m[k] >= 0 && y[k] > 0.0f) d1[aa] += path_grad(m[k], mt, wt, gt) * (double)y[k];
        }
    }
    // this row's own leg-2 slots
    int m2[kSmax];
    float y2[kSmax];
#pragma unroll
    for (int c = 0; c < kSmax; ++c) {
        m2[c] = -1;
        y2[c] = 0.0f;
        if (c < a.s3) {
            m2[c] = a.idx2[(size_t)u * a.s3 + c];
            y2[c] = a.w2[(size_t)u * a.s3 + c];
        }
    }
    // incoming leg-1 edges, four per round trip
    const int bi = (int)fdiv((uint32_t)u, a.fd_hkv);
    const int b = (int)fdiv((uint32_t)bi, a.fd_n);
    const int i = bi - b * a.n;
    const int pair = b * a.hkv + (u - bi * a.hkv);
    const int e_beg = a.beg[pair * a.n + i], e_end = e_beg + a.len[pair * a.n + i];
    for (int e0 = e_beg; e0 < e_end; e0 += 4) {
        int eid[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) eid[q] = e0 + q < e_end ? a.list[e0 + q] : -1;
        float xs[4];
        int mts[4][kSmax];
        float wts[4][kSmax], gts[4][kSmax];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            xs[q] = 0.0f;
            if (eid[q] >= 0) {
                xs[q] = a.w1[eid[q]];
                load_aprime(a, (int)fdiv((uint32_t)eid[q], a.fd_s2), mts[q], wts[q], gts[q]);
            } else {
#pragma unroll
                for (int t = 0; t < kSmax; ++t) { mts[q][t] = -1; wts[q][t] = 0.0f; gts[q][t] = 0.0f; }
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int c = 0; c < kSmax; ++c)
                if (y2[c] > 0.0f) d2[c] += path_grad(m2[c], mts[q], wts[q], gts[q]) * (double)xs[q];
        }
    }
    if (a.aliased) {
#pragma unroll
        for (int k = 0; k < kSmax; ++k)
            if (k < a.s2) a.dw1[(size_t)u * a.s2 + k] = (float)(d1[k] + d2[k]);
    } else {
#pragma unroll
        for (int k = 0; k < kSmax; ++k) {
            if (k < a.s2) a.dw1[(size_t)u * a.s2 + k] = (float)d1[k];
            if (k < a.s3) a.dw2[(size_t)u * a.s3 + k] = (float)d2[k];
        }
    }
}

// -------------- SER backward by source chunks, s2 = s3 = 4, s1 = 4 or 2
// No reverse index.  Pass 1: one 1024-thread workgroup per (pair, chunk c of
// 1024 source tokens), one source per thread.  The thread recomputes the
// gradient of each of its 16 paths from its own rows and adds
// x * (path gradient) into an fp64 LDS accumulator of the path's leg-1
// target row (j <= i, so rows [0, end of the chunk)), with LDS atomics;
// when dw1 and dw2 alias, its own-row part dw1 goes into the same
// accumulator, else it is rounded and written at once.  The workgroup then
// writes its accumulator rows as an fp64 partial.  Pass 2: one thread per
// row sums the partials of the chunks at or above the row's own chunk, in
// chunk order, and rounds once.  The chunks of a pair run on one XCD, so
// the leg-2 rows they gather stay in its L2.
constexpr int kSerThreads = 1024;   // sources per chunk
constexpr int kSerPartRows = 4096;  // rows of one pair in LDS (128 KiB of fp64 x 4)

struct SerPartArgs {
    SerUnitArgs u;
    const int32_t* idx_out;
    const float* w_out;
    const float* dw_out;
    const uint64_t* paths;   // the forward's path map, or null
    float* dw1;
    float* dw2;
    double* part;
    int nch, npairs, aliased;
};

// offset (in rows) of chunk c's partial inside its pair's block, and the
// pair's block size: chunk c covers rows [0, min(n, 1024 (c + 1)))
__host__ __device__ inline long long part_row_off(int n, int c) {
    long long off = 0;
    for (int k = 0; k < c; ++k) off += (k + 1) * kSerThreads < n ? (k + 1) * kSerThreads : n;
    return off;
}

// Source i's contributions, from the gradients pg of its 16 paths: its own
// dw1 (into the accumulator when the legs alias, else stored), and
// dw2[j_a, c] += pg(a, c) w1[i, a] into the accumulator rows j_a.
__device__ __forceinline__ void ser_part_accumulate(const SerPartArgs& a, double* acc, int i,
                                                    int u, const int (&j)[4],
                                                    const float (&x)[kSmax],
                                                    const float (&y)[kCand],
                                                    const double (&pg)[kCand]) {
    // own row: dw1[i, a] = sum_c g(a, c) w2[j_a, c]
    double d1[kSmax];
#pragma unroll
    for (int aa = 0; aa < kSmax; ++aa) {
        d1[aa] = 0.0;
#pragma unroll
        for (int cc = 0; cc < kSmax; ++cc) d1[aa] += pg[aa * kSmax + cc] * (double)y[aa * kSmax + cc];
    }
    if (a.aliased) {
#pragma unroll
        for (int aa = 0; aa < kSmax; ++aa)
            if (d1[aa] != 0.0) atomicAdd(acc + i * 4 + aa, d1[aa]);
    } else {
        *reinterpret_cast<float4*>(a.dw1 + (size_t)u * 4) =
            make_float4((float)d1[0], (float)d1[1], (float)d1[2], (float)d1[3]);
    }
    // leg-2 slots of the target rows: dw2[j_a, c] += g(a, c) w1[i, a]
#pragma unroll
    for (int aa = 0; aa < kSmax; ++aa) {
#pragma unroll
        for (int cc = 0; cc < kSmax; ++cc) {
            const double g = pg[aa * kSmax + cc];
            if (g != 0.0) atomicAdd(acc + j[aa] * 4 + cc, g * (double)x[aa]);
        }
    }
}

template <int S1>
__global__ __launch_bounds__(kSerThreads) void ser_bwd_part_kernel(SerPartArgs a) {
    __shared__ double acc[kSerPartRows * 4];
    const int total = a.npairs * a.nch;
    int lin = (int)blockIdx.x;
    if (total % kXcds == 0)
        lin = ((int)blockIdx.x % kXcds) * (total / kXcds) + (int)blockIdx.x / kXcds;
    const int pair = lin / a.nch, c = lin - (lin / a.nch) * a.nch;
    const int n = a.u.n, hkv = a.u.hkv;
    const int b = pair / hkv, h = pair - (pair / hkv) * hkv;
    const int i0 = c * kSerThreads;
    const int thi = i0 + kSerThreads < n ? i0 + kSerThreads : n;
    for (int e = threadIdx.x; e < thi * 4; e += kSerThreads) acc[e] = 0.0;
    __syncthreads();

    const int i = i0 + (int)threadIdx.x;
    if (i < thi && a.paths) {
        // with the forward's path map: leg-1 row, leg-2 weights, dw' only
        const int u = (b * n + i) * hkv + h;
        const int4 j4 = *reinterpret_cast<const int4*>(a.u.idx1 + (size_t)u * 4);
        const float4 x4 = *reinterpret_cast<const float4*>(a.u.w1 + (size_t)u * 4);
        const uint64_t mp = a.paths[u];
        const int j[4] = {j4.x, j4.y, j4.z, j4.w};
        const float x[4] = {x4.x, x4.y, x4.z, x4.w};
        float y[kCand];
#pragma unroll
        for (int aa = 0; aa < kSmax; ++aa) {
            const float4 yi =
                *reinterpret_cast<const float4*>(a.u.w2 + ((size_t)u + (j[aa] - i) * hkv) * 4);
            y[aa * 4 + 0] = yi.x; y[aa * 4 + 1] = yi.y; y[aa * 4 + 2] = yi.z; y[aa * 4 + 3] = yi.w;
        }
        float gt[kSmax];
        if constexpr (S1 == 4) {
            const float4 g4 = *reinterpret_cast<const float4*>(a.dw_out + (size_t)u * 4);
            gt[0] = g4.x; gt[1] = g4.y; gt[2] = g4.z; gt[3] = g4.w;
        } else {
            const float2 g2 = *reinterpret_cast<const float2*>(a.dw_out + (size_t)u * 2);
            gt[0] = g2.x; gt[1] = g2.y; gt[2] = 0.0f; gt[3] = 0.0f;
        }
        double pg[kCand];
#pragma unroll
        for (int k = 0; k < kCand; ++k) {
            const uint32_t sl = (uint32_t)(mp >> (4 * k)) & 0xFu;
            float g = 0.0f;
#pragma unroll
            for (int t = 0; t < kSmax; ++t) g = sl == (uint32_t)t ? gt[t] : g;
            pg[k] = sl != kNoSlot ? 0.0 + (double)g : 0.0;
        }
        ser_part_accumulate(a, acc, i, u, j, x, y, pg);
    } else if (i < thi) {
        const int u = (b * n + i) * hkv + h;
        int m[kCand];
        float x[kSmax], y[kCand];
        load_paths_vec(a.u, u, m, x, y);
        const int4 j4 = *reinterpret_cast<const int4*>(a.u.idx1 + (size_t)u * 4);
        const int j[4] = {j4.x, j4.y, j4.z, j4.w};
        // retained slots of A' (s1 = 4, or 2 with the rest dead)
        int mt[kSmax];
        float wt[kSmax], gt[kSmax];
        if constexpr (S1 == 4) {
            const int4 m4 = *reinterpret_cast<const int4*>(a.idx_out + (size_t)u * 4);
            const float4 w4 = *reinterpret_cast<const float4*>(a.w_out + (size_t)u * 4);
            const float4 g4 = *reinterpret_cast<const float4*>(a.dw_out + (size_t)u * 4);
            mt[0] = m4.x; mt[1] = m4.y; mt[2] = m4.z; mt[3] = m4.w;
            wt[0] = w4.x; wt[1] = w4.y; wt[2] = w4.z; wt[3] = w4.w;
            gt[0] = g4.x; gt[1] = g4.y; gt[2] = g4.z; gt[3] = g4.w;
        } else {
            const int2 m2 = *reinterpret_cast<const int2*>(a.idx_out + (size_t)u * 2);
            const float2 w2 = *reinterpret_cast<const float2*>(a.w_out + (size_t)u * 2);
            const float2 g2 = *reinterpret_cast<const float2*>(a.dw_out + (size_t)u * 2);
            mt[0] = m2.x; mt[1] = m2.y; mt[2] = -1; mt[3] = -1;
            wt[0] = w2.x; wt[1] = w2.y; wt[2] = 0.0f; wt[3] = 0.0f;
            gt[0] = g2.x; gt[1] = g2.y; gt[2] = 0.0f; gt[3] = 0.0f;
        }
        double pg[kCand];
#pragma unroll
        for (int k = 0; k < kCand; ++k)
            pg[k] = x[k / kSmax] > 0.0f && y[k] > 0.0f ? path_grad(m[k], mt, wt, gt) : 0.0;
        ser_part_accumulate(a, acc, i, u, j, x, y, pg);
    }
    __syncthreads();
    double* dst = a.part + (part_row_off(n, a.nch) * pair + part_row_off(n, c)) * 4;
    for (int e = threadIdx.x; e < thi * 2; e += kSerThreads)
        reinterpret_cast<double2*>(dst)[e] = reinterpret_cast<const double2*>(acc)[e];
}

// one thread per row u = (b n + r) hkv + h: sum of the partials of chunks
// floor(r / 1024) .. nch - 1, in that order
__global__ __launch_bounds__(kBlock) void ser_bwd_part_sum_kernel(SerPartArgs a) {
    const long long U = (long long)a.npairs * a.u.n;
    const long long u = (long long)blockIdx.x * kBlock + threadIdx.x;
    if (u >= U) return;
    const int n = a.u.n, hkv = a.u.hkv;
    const int bi = (int)(u / hkv), h = (int)(u - (long long)bi * hkv);
    const int b = bi / n, r = bi - b * n;
    const int pair = b * hkv + h;
    const long long base = part_row_off(n, a.nch) * pair;
    double d[4] = {0.0, 0.0, 0.0, 0.0};
    for (int c = r / kSerThreads; c < a.nch; ++c) {
        const double* p = a.part + (base + part_row_off(n, c) + r) * 4;
        const double2 lo = *reinterpret_cast<const double2*>(p);
        const double2 hi = *reinterpret_cast<const double2*>(p + 2);
        d[0] += lo.x; d[1] += lo.y; d[2] += hi.x; d[3] += hi.y;
    }
    float* out = a.aliased ? a.dw1 : a.dw2;
    *reinterpret_cast<float4*>(out + u * 4) =
        make_float4((float)d[0], (float)d[1], (float)d[2], (float)d[3]);
}

// dw1 = ws1, dw2 = ws2 rounded to fp32; when they alias, dw = ws1 + ws2.
__global__ __launch_bounds__(kBlock) void ser_bwd_finish_kernel(const double* ws1,
                                                                const double* ws2, float* dw1,
                                                                float* dw2, size_t n1, size_t n2,
                                                                int aliased) {
    const size_t stride = (size_t)gridDim.x * kBlock;
    for (size_t e = (size_t)blockIdx.x * kBlock + threadIdx.x; e < n1; e += stride)
        dw1[e] = aliased ? (float)(ws1[e] + ws2[e]) : (float)ws1[e];
    if (!aliased)
        for (size_t e = (size_t)blockIdx.x * kBlock + threadIdx.x; e < n2; e += stride)
            dw2[e] = (float)ws2[e];
}

__global__ __launch_bounds__(kBlock) void round_f64_kernel(const double* src, float* dst,
                                                           size_t count) {
    for (size_t e = (size_t)blockIdx.x * kBlock + threadIdx.x; e < count;
         e += (size_t)gridDim.x * kBlock)
        dst[e] = (float)src[e];
}

__global__ __launch_bounds__(kBlock) void zero_f32_kernel(float* p, size_t count) {
    // float4 stores when 16-byte aligned, plain stores otherwise
    const size_t n4 = ((uintptr_t)p & 15u) ? 0 : count / 4;
    float4* p4 = reinterpret_cast<float4*>(p);
    const size_t stride = (size_t)gridDim.x * kBlock;
    for (size_t e = (size_t)blockIdx.x * kBlock + threadIdx.x; e < n4; e += stride)
        p4[e] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (size_t e = n4 * 4 + (size_t)blockIdx.x * kBlock + threadIdx.x; e < count; e += stride)
        p[e] = 0.f;
}

__global__ __launch_bounds__(kBlock) void zero_f64_kernel(double* p, size_t count) {
    const size_t stride = (size_t)gridDim.x * kBlock;
    for (size_t e = (size_t)blockIdx.x * kBlock + threadIdx.x; e < count; e += stride)
        p[e] = 0.0;
}

__global__ __launch_bounds__(kBlock) void check_edges_kernel(int n, int hkv, const int32_t* idx,
                                                             const float* w, int s,
                                                             size_t count,
                                                             unsigned long long* counts) {
    unsigned long long bad = 0, live = 0;
    for (size_t e = (size_t)blockIdx.x * kBlock + threadIdx.x; e < count;
         e += (size_t)gridDim.x * kBlock) {
        const size_t unit = e / s;
        const int i = (int)((unit / hkv) % n);
        const int j = idx[e];
        const float wt = w[e];
        if (j < 0 || j > i || !(wt >= 0.0f) || wt == INFINITY) ++bad;
        if (wt > 0.0f) ++live;
    }
    for (int m = 32; m > 0; m >>= 1) {
        bad += __shfl_xor(bad, m, kWave);
        live += __shfl_xor(live, m, kWave);
    }
    if ((threadIdx.x & (kWave - 1)) == 0) {
        if (bad) atomicAdd(counts, bad);
        if (live) atomicAdd(counts + 1, live);
    }
}

unsigned grid_for(size_t work, unsigned cap) {
    size_t blocks = (work + kBlock - 1) / kBlock;
    if (blocks < 1) blocks = 1;
    return (unsigned)(blocks < cap ? blocks : cap);
}

template <int L>
hipError_t run_fwd(const SerArgs& a, hipStream_t st) {
    const long long threads = (long long)a.U * L;
    hipLaunchKernelGGL((ser_fwd_kernel<L>), dim3((unsigned)((threads + kBlock - 1) / kBlock)),
                       dim3(kBlock), 0, st, a);
    return hipGetLastError();
}

template <int L>
hipError_t run_bwd(const SerBwdArgs& a, hipStream_t st) {
    const long long threads = (long long)a.U * L;
    hipLaunchKernelGGL((ser_bwd_kernel<L>), dim3((unsigned)((threads + kBlock - 1) / kBlock)),
                       dim3(kBlock), 0, st, a);
    return hipGetLastError();
}

}  // namespace

void make_seg_plan(SegPlan& sp, int B, int n, int hkv) {
    const long long npairs = (long long)B * hkv;
    int lgS = 0;
    while ((npairs << lgS) % kXcds != 0 && (npairs << lgS) < 64 && (n % (2 << lgS)) == 0)
        ++lgS;
    sp.n = n;
    sp.hkv = hkv;
    sp.lgS = lgS;
    sp.nseg = (int)(npairs << lgS);
    sp.L = n >> lgS;
    sp.fd_L = make_fastdiv((uint32_t)(sp.L > 0 ? sp.L : 1));
    sp.fd_hkv = make_fastdiv((uint32_t)(hkv > 0 ? hkv : 1));
}

bool ser_backward_part_fits(int n) { return n >= 1 && n <= kSerPartRows; }

size_t ser_backward_part_bytes(int B, int n, int hkv) {
    if (!ser_backward_part_fits(n)) return 0;
    const int nch = (n + kSerThreads - 1) / kSerThreads;
    return (size_t)B * hkv * (size_t)part_row_off(n, nch) * 4 * sizeof(double);
}

size_t ser_backward_pull_bytes(long long rows, int s2) {
    return (size_t)rows * (2 + s2) * sizeof(int);
}

int persistent_grid(const void* kernel, int items, int per_wg) {
    static int cus_by_dev[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int cus = cus_by_dev[dev];
    if (!cus) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        cus_by_dev[dev] = cus;
    }
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kBlock, 0) != hipSuccess ||
        per_cu <= 0)
        per_cu = 1;
    long long full = (long long)cus * per_cu;
    full -= full % 8;
    if (full < 8) full = 8;
    long long need = ((long long)items + per_wg - 1) / per_wg;
    need = (need + 7) / 8 * 8;
    return (int)(need < full ? need : full);
}

hipError_t launch_zero_f32(float* p, size_t count, hipStream_t st) {
    if (!count) return hipSuccess;
    hipLaunchKernelGGL(zero_f32_kernel, dim3(grid_for(count / 4 + 1, 8192)), dim3(kBlock), 0, st,
                       p, count);
    return hipGetLastError();
}

hipError_t launch_zero_f64(double* p, size_t count, hipStream_t st) {
    if (!count) return hipSuccess;
    hipLaunchKernelGGL(zero_f64_kernel, dim3(grid_for(count, 8192)), dim3(kBlock), 0, st, p,
                       count);
    return hipGetLastError();
}

hipError_t launch_ser_forward(int B, int n, int hkv, const int32_t* idx1, const float* w1,
                              int s2, const int32_t* idx2, const float* w2, int s3,
                              int32_t* idx_out, float* w_out, int s1, uint64_t* paths,
                              hipStream_t st) {
    if (s2 <= kSmax && s3 <= kSmax) {
        SerUnitArgs u{idx1, w1, idx2, w2, idx_out, w_out, nullptr, nullptr, nullptr,
                      n, hkv, s1, s2, s3, B * n * hkv,
                      make_fastdiv((uint32_t)hkv), make_fastdiv((uint32_t)n),
                      s1 == 4 && (((uintptr_t)idx_out | (uintptr_t)w_out) & 15) == 0,
                      s2 == 4 && s3 == 4 &&
                          (((uintptr_t)idx1 | (uintptr_t)w1 | (uintptr_t)idx2 | (uintptr_t)w2) &
                           15) == 0};
        u.paths = s1 <= kSmax ? paths : nullptr;
        const bool out8 = (((uintptr_t)idx_out | (uintptr_t)w_out) & 7) == 0;
        const dim3 grid(xcd_unit_grid(u.U));
        if (s1 == 4 && u.vec_out && u.vec_in) {
            if (u.paths)
                hipLaunchKernelGGL((ser_fwd_vec_kernel<4, true>), grid, dim3(kBlock), 0, st, u);
            else
                hipLaunchKernelGGL((ser_fwd_vec_kernel<4, false>), grid, dim3(kBlock), 0, st, u);
        } else if (s1 == 2 && out8 && u.vec_in) {
            if (u.paths)
                hipLaunchKernelGGL((ser_fwd_vec_kernel<2, true>), grid, dim3(kBlock), 0, st, u);
            else
                hipLaunchKernelGGL((ser_fwd_vec_kernel<2, false>), grid, dim3(kBlock), 0, st, u);
        }
        else
            hipLaunchKernelGGL(ser_fwd_unit_kernel, dim3(xcd_unit_grid(u.U)), dim3(kBlock), 0, st,
                               u);
        return hipGetLastError();
    }
    SerArgs a{idx1, w1, idx2, w2, idx_out, w_out, n, hkv, s1, s2, s3, B * n * hkv};
    switch (pow2_ceil(s2 * s3)) {
        case 1: return run_fwd<1>(a, st);
        case 2: return run_fwd<2>(a, st);
        case 4: return run_fwd<4>(a, st);
        case 8: return run_fwd<8>(a, st);
        case 16: return run_fwd<16>(a, st);
        case 32: return run_fwd<32>(a, st);
        case 64: return run_fwd<64>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_ser_chain2(int B, int n, int hkv, const int32_t* idx, const float* w, int s,
                             int32_t* idx_mid, float* w_mid, int32_t* idx_out, float* w_out,
                             hipStream_t st) {
    SerChainArgs a{idx, w, idx_mid, w_mid, idx_out, w_out, hkv, B * n * hkv,
                   make_fastdiv((uint32_t)hkv), make_fastdiv((uint32_t)n), n};
    const dim3 grid(xcd_unit_grid(a.U));
    const bool mid = idx_mid != nullptr;
    if (s == 4 && mid)
        hipLaunchKernelGGL((ser_chain2_kernel<4, true>), grid, dim3(kBlock), 0, st, a);
    else if (s == 4)
        hipLaunchKernelGGL((ser_chain2_kernel<4, false>), grid, dim3(kBlock), 0, st, a);
    else if (s == 2 && mid)
        hipLaunchKernelGGL((ser_chain2_kernel<2, true>), grid, dim3(kBlock), 0, st, a);
    else if (s == 2)
        hipLaunchKernelGGL((ser_chain2_kernel<2, false>), grid, dim3(kBlock), 0, st, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_ser_backward(int B, int n, int hkv, const int32_t* idx1, const float* w1,
                               int s2, const int32_t* idx2, const float* w2, int s3,
                               const int32_t* idx_out, const float* w_out, int s1,
                               const float* dw_out, const uint64_t* paths, float* dw1,
                               float* dw2, double* ws1, double* ws2, hipStream_t st) {
    const size_t rows = (size_t)B * n * hkv;
    const bool aliased = dw1 == dw2;
    // the source-chunk path: legs of 4 slots, A' of 4 or 2, vector-aligned rows
    const bool vec4 = (s1 == 4 || s1 == 2) && s2 == 4 && s3 == 4 &&
                      (((uintptr_t)idx1 | (uintptr_t)w1 | (uintptr_t)idx2 | (uintptr_t)w2 |
                        (uintptr_t)dw1 | (uintptr_t)dw2) & 15) == 0 &&
                      (((uintptr_t)idx_out | (uintptr_t)w_out | (uintptr_t)dw_out) &
                       (s1 == 4 ? 15 : 7)) == 0;
    if (vec4 && ser_backward_part_fits(n) && ((uintptr_t)ws1 & 15) == 0) {
        SerPartArgs pa;
        pa.u = SerUnitArgs{idx1, w1, idx2, w2, nullptr, nullptr, nullptr, nullptr, nullptr,
                           n, hkv, s1, s2, s3, (int)rows,
                           make_fastdiv((uint32_t)hkv), make_fastdiv((uint32_t)n), 1, 1};
        pa.idx_out = idx_out; pa.w_out = w_out; pa.dw_out = dw_out;
        pa.paths = paths;
        pa.dw1 = dw1; pa.dw2 = dw2;
        pa.part = ws1;
        pa.nch = (n + kSerThreads - 1) / kSerThreads;
        pa.npairs = B * hkv;
        pa.aliased = aliased;
        if (s1 == 4)
            hipLaunchKernelGGL(ser_bwd_part_kernel<4>, dim3((unsigned)(pa.npairs * pa.nch)),
                               dim3(kSerThreads), 0, st, pa);
        else
            hipLaunchKernelGGL(ser_bwd_part_kernel<2>, dim3((unsigned)(pa.npairs * pa.nch)),
                               dim3(kSerThreads), 0, st, pa);
        hipLaunchKernelGGL(ser_bwd_part_sum_kernel, dim3((unsigned)((rows + kBlock - 1) / kBlock)),
                           dim3(kBlock), 0, st, pa);
        return hipGetLastError();
    }
    // the reverse index of leg 1 pays off only where it is built in one
    // pass per pair (n <= 4096); longer sequences take the fp64-atomic path
    if (s1 <= kSmax && s2 <= kSmax && s3 <= kSmax && edge_index_one_pass(n)) {
        // reverse index of leg 1 in the workspace, then one pass, no atomics
        int* beg = reinterpret_cast<int*>(ws1);
        int* len = beg + rows;
        int* list = len + rows;
        hipError_t e = launch_edge_index(B, n, hkv, idx1, w1, s2, nullptr, beg, len, list, nullptr, st);
        if (e != hipSuccess) return e;
        SerPullArgs pa{idx1, w1, idx2, w2, idx_out, w_out, dw_out, dw1, dw2, beg, len, list,
                       n, hkv, s1, s2, s3, (int)rows, (int)aliased,
                       make_fastdiv((uint32_t)hkv), make_fastdiv((uint32_t)n),
                       make_fastdiv((uint32_t)s2),
                       s2 == 4 && s3 == 4 &&
                           (((uintptr_t)idx1 | (uintptr_t)w1 | (uintptr_t)idx2 | (uintptr_t)w2) &
                            15) == 0,
                       s1 == 4 && (((uintptr_t)idx_out | (uintptr_t)w_out | (uintptr_t)dw_out) &
                                   15) == 0};
        hipLaunchKernelGGL(ser_bwd_pull_kernel, dim3(xcd_unit_grid((int)rows)), dim3(kBlock), 0,
                           st, pa);
        return hipGetLastError();
    }
    if (s2 <= kSmax && s3 <= kSmax) {
        // ws1: dw1 (every slot stored), ws2: dw2 (zeroed, then atomics)
        hipError_t e = launch_zero_f64(ws2, rows * s3, st);
        if (e != hipSuccess) return e;
        SerUnitArgs u{idx1, w1, idx2, w2, const_cast<int32_t*>(idx_out),
                      const_cast<float*>(w_out), dw_out, ws1, ws2,
                      n, hkv, s1, s2, s3, (int)rows,
                      make_fastdiv((uint32_t)hkv), make_fastdiv((uint32_t)n),
                      s1 == 4 && (((uintptr_t)idx_out | (uintptr_t)w_out | (uintptr_t)dw_out) &
                                  15) == 0,
                      s2 == 4 && s3 == 4 &&
                          (((uintptr_t)idx1 | (uintptr_t)w1 | (uintptr_t)idx2 | (uintptr_t)w2) &
                           15) == 0};
        u.paths = const_cast<uint64_t*>(paths);
        hipLaunchKernelGGL(ser_bwd_unit_kernel, dim3((unsigned)((rows + kBlock - 1) / kBlock)),
                           dim3(kBlock), 0, st, u);
        hipLaunchKernelGGL(ser_bwd_finish_kernel, dim3(grid_for(rows * s2, 8192)), dim3(kBlock), 0,
                           st, (const double*)ws1, (const double*)ws2, dw1, dw2, rows * s2,
                           rows * s3, (int)aliased);
        return hipGetLastError();
    }
    hipError_t e = launch_zero_f64(ws1, rows * s2, st);
    if (e == hipSuccess && !aliased) e = launch_zero_f64(ws2, rows * s3, st);
    if (e != hipSuccess) return e;
    SerBwdArgs a{idx1, w1, idx2, w2, idx_out, w_out, dw_out, ws1, aliased ? ws1 : ws2,
                 n, hkv, s1, s2, s3, (int)rows};
    switch (pow2_ceil(s2 * s3)) {
        case 1: e = run_bwd<1>(a, st); break;
        case 2: e = run_bwd<2>(a, st); break;
        case 4: e = run_bwd<4>(a, st); break;
        case 8: e = run_bwd<8>(a, st); break;
        case 16: e = run_bwd<16>(a, st); break;
        case 32: e = run_bwd<32>(a, st); break;
        case 64: e = run_bwd<64>(a, st); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(round_f64_kernel, dim3(grid_for(rows * s2, 8192)), dim3(kBlock), 0, st,
                       (const double*)ws1, dw1, rows * s2);
    if (!aliased)
        hipLaunchKernelGGL(round_f64_kernel, dim3(grid_for(rows * s3, 8192)), dim3(kBlock), 0, st,
                           (const double*)ws2, dw2, rows * s3);
    return hipGetLastError();
}

hipError_t launch_check_edges(int B, int n, int hkv, const int32_t* idx, const float* w, int s,
                              unsigned long long* counts, hipStream_t st) {
    const size_t count = (size_t)B * n * hkv * s;
    if (!count) return hipSuccess;
    hipLaunchKernelGGL(check_edges_kernel, dim3(grid_for(count, 4096)), dim3(kBlock), 0, st, n,
                       hkv, idx, w, s, count, counts);
    return hipGetLastError();
}

}  // namespace gm
