// Refresh edges from a dense attention layer (page "Graph Machine: Towards
// Better Pretraining via Edges", ai.info, Methodology, referral paragraph:
// optional refresh edges bring in the positions that the most recent dense
// attention layer attends to most; Main Findings: refresh helps).  Reading
// (the pages do not define the ranking): per (batch, token i, KV head h) the
// positions j <= i ranked by the group-mean attention probability
//   pbar_j = (1/G) sum_g exp(scale q_g . k_j - lse_g),
// the s largest kept (equal values: the lower position first), weight pbar_j.
//
// The scores are a dense contraction and run on the matrix cores
// (v_mfma_f32_16x16x32_bf16), computed transposed, S^T = K Q^T: the key
// tile is the A operand and the query rows the B operand, so in the result
// lane l holds ONE token (column l%16) and keys 4(l/16)+r, r < 4.  Each lane
// therefore keeps its own token's running state (one max/sum per head, one
// short sorted top list) and the per-token reductions at the end run over
// the four lanes l%16 + 16c (two swaps) instead of over sixteen.
//
// A workgroup of 8 wavefronts takes 128 or 256 consecutive tokens of one
// (batch, KV head): each wavefront RT 16-token tiles for all G query heads,
// with its query rows held as B-fragments in registers (two tiles in the lse
// pass when G * d <= 256 and G <= 2, one in the selection pass, whose top
// lists need the registers).  Key tiles of 64 rows are brought into LDS by
// direct global->LDS loads (no registers in between), double-buffered so
// the next tile's loads are in flight while the current one is used; the
// 16-byte pieces of a row are XOR-swizzled with the row index so that the
// sixteen rows of a fragment load fall on different banks.  The more tokens
// a workgroup covers, the fewer times each key row is fetched (the keys of
// a pair are re-read once per later token tile).  The kernels are held to
// 128 registers (four wavefronts per SIMD): the vector work of one
// wavefront then overlaps the matrix work of another.  Workgroups are
// issued heaviest first (the last token tiles see the most keys),
// consecutive workgroups on different (batch, KV head) pairs so one XCD
// keeps a fixed set of pairs.
//
// Two passes: the first keeps an online max/sum per (token, head) in base 2
// (rescaled only when a term would pass 2^16, a wavefront-uniform branch
// that is rarely taken) and writes lse (skipped when the caller passes the
// dense layer's own lse); the second recomputes the scores, forms pbar and
// keeps, per lane, a sorted top list of its own keys.  After every key tile
// the four lanes of a token find the S-th largest value they hold together
// (two bitonic merges across lanes): a later key at or below it already
// has S positions ahead of it and is dropped without touching a list; the
// rest enter by a branch-free insertion.
#include "gm_common.h"
#include "gm_internal.h"
#include "gm_wave.h"

#include <type_traits>

namespace gm {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRefKeys = 64;     // keys per LDS tile
constexpr int kRefWaves = 8;     // wavefronts per workgroup
constexpr int kRefSmax = 8;      // kept positions per token, at most
constexpr float kLog2e = 1.4426950408889634f;

struct RefreshArgs {
    const bf16_t* q;    // [B][n][hq][d]
    const bf16_t* k;    // [B][n][hkv][d]
    float* lse;         // [B][n][hq], natural log
    int32_t* idx_out;   // [B][n][hkv][s]
    float* w_out;
    int n, hq, hkv, s, ntile, npair;
    float c;            // scale * log2(e)
};

// 2^x by the hardware instruction alone: results below 2^-126 flush to zero,
// which changes no kept position (the largest probability of a token is at
// least 1/n) and no log-sum-exp beyond 2^-126 relative
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float max4(float a, float b, float c, float d) {
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}
constexpr float kSlack = 16.0f;

// The S-th largest value over the four lanes of a token (lanes l%16 + 16c,
// c = grp), each holding S values sorted in descending order.  For two
// sorted lists a and b, max(a_i, b_{S-1-i}) over i is the set of the S
// largest of both (bitonic); sorted by a bitonic merge it pairs again with
// the other pair's set, and the smallest of those S maxima is the answer.
template <int S>
__device__ __forceinline__ float union_kth(const float (&v)[S], int grp) {
    const bool odd16 = (grp & 1) != 0, odd32 = grp >= 2;
    float c[S];
#pragma unroll
    for (int i = 0; i < S; ++i) {
        // a permlane16 swap of (x, y) hands odd rows the even rows' y and
        // even rows the odd rows' x: both hold v_{S-1-i}, the partner's
        float x = v[S - 1 - i], y = v[S - 1 - i];
        swap16(x, y);
        c[i] = fmaxf(v[i], odd16 ? x : y);
    }
#pragma unroll
    for (int k = S / 2; k >= 1; k /= 2)
#pragma unroll
        for (int i = 0; i < S; ++i)
            if ((i & k) == 0) {
                const float hi = fmaxf(c[i], c[i + k]), lo = fminf(c[i], c[i + k]);
                c[i] = hi;
                c[i + k] = lo;
            }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < S; ++i) {
        float x = c[S - 1 - i], y = c[S - 1 - i];
        swap32(x, y);
        const float d = fmaxf(c[i], odd32 ? x : y);
        m = i == 0 ? d : fminf(m, d);
    }
    return m;
}

__device__ __forceinline__ bf16x8_t as_frag(const uint4& u) {
    return __builtin_bit_cast(bf16x8_t, u);
}

// a sorted list of S candidates: larger value first, equal values by the
// lower position; empty entries hold (0, INT_MAX) and lose to any positive
template <int S>
struct TopS {
    float v[S];
    int j[S];
};
__device__ __forceinline__ bool ahead(float va, int ja, float vb, int jb) {
    return va > vb || (va == vb && ja < jb);
}
// insert (v, j) where j exceeds every position already held, without
// branches: ge[e] (entry e stays ahead: larger, or equal and earlier) is
// true below the insertion point and false from it on, so each entry either
// stays, takes the new pair or takes its predecessor; v at or below the last
// entry changes nothing
template <int S>
__device__ __forceinline__ void insert_later(TopS<S>& t, float v, int j) {
    bool ge[S];
#pragma unroll
    for (int e = 0; e < S; ++e) ge[e] = t.v[e] >= v;
#pragma unroll
    for (int e = S - 1; e > 0; --e) {
        const float nv = ge[e - 1] ? (ge[e] ? t.v[e] : v) : t.v[e - 1];
        const int nj = ge[e - 1] ? (ge[e] ? t.j[e] : j) : t.j[e - 1];
        t.v[e] = nv;
        t.j[e] = nj;
    }
    t.v[0] = ge[0] ? t.v[0] : v;
    t.j[0] = ge[0] ? t.j[0] : j;
}
// merge two sorted lists over disjoint positions, keeping the first S
template <int S>
__device__ __forceinline__ TopS<S> merge(const TopS<S>& a, const TopS<S>& b) {
    TopS<S> r;
    int ia = 0, ib = 0;
#pragma unroll
    for (int e = 0; e < S; ++e) {
        // ia + ib == e <= S - 1: both heads are inside their lists
        float va = a.v[0], vb = b.v[0];
        int ja = a.j[0], jb = b.j[0];
#pragma unroll
        for (int x = 1; x < S; ++x) {
            if (x == ia) { va = a.v[x]; ja = a.j[x]; }
            if (x == ib) { vb = b.v[x]; jb = b.j[x]; }
        }
        const bool ta = ahead(va, ja, vb, jb);
        r.v[e] = ta ? va : vb;
        r.j[e] = ta ? ja : jb;
        ia += ta ? 1 : 0;
        ib += ta ? 0 : 1;
    }
    return r;
}

// LDS slot of the 16-byte piece p of key row r in a tile: rows of D / 8
// pieces, the piece index XORed with the row, so the sixteen rows that one
// fragment load reads (same p) sit on sixteen different bank groups
template <int D>
__device__ __forceinline__ int key_slot(int r, int p) {
    constexpr int PPR = D / 8;
    return r * PPR + (p ^ (r & (PPR - 1)));
}

// Direct global->LDS loads of a tile of kRefKeys key rows from position j0
// (rows past n - 1 repeat row n - 1; their scores are masked).  Each
// wavefront instruction fills 64 consecutive 16-byte slots, lane l slot l,
// so every lane fetches the piece that belongs at its slot.
template <int D>
__device__ __forceinline__ void load_key_tile(uint4* buf, const bf16_t* kbase, size_t kstride,
                                              int j0, int n, int wv, int lane) {
    constexpr int PPR = D / 8;
    constexpr int SLOTS = kRefKeys * PPR;
    constexpr int U = SLOTS / (kRefWaves * kWave);   // instructions per wavefront
    static_assert(U >= 1 && U * kRefWaves * kWave == SLOTS, "tile slots must divide evenly");
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int base = (u * kRefWaves + wv) * kWave;   // first slot of the instruction
        const int slot = base + lane;
        const int row = slot / PPR;
        const int piece = (slot % PPR) ^ (row & (PPR - 1));
        const int j = j0 + row < n ? j0 + row : n - 1;
        __builtin_amdgcn_global_load_lds(
            kbase + (size_t)j * kstride + piece * 8,
            (__attribute__((address_space(3))) void*)(buf + base), 16, 0, 0);
    }
}

// 16-token tiles per wavefront: two for the lse pass when the query
// fragments (RT * G * d / 8 registers) leave room; one for the selection
// pass, whose top lists and insertion need the registers
constexpr int ref_rt(int MODE, int D, int G) {
    return (MODE == 0 && G <= 2 && G * D <= 256) || (MODE == 2 && G * D <= 128) ? 2 : 1;
}
constexpr int ref_tokens(int MODE, int D, int G) { return kRefWaves * 16 * ref_rt(MODE, D, G); }

// MODE 0: lse; MODE 1: the top-S refresh edges given lse; MODE 2 (G = 1):
// both in one pass.  With one query head per KV head pbar_j = exp(score_j -
// lse) ranks the keys as their raw scores do, so the lanes keep their top
// lists by score while they form lse, and the kept weights are taken from
// the final lse at the end.  D head dim, G query heads per KV head.
template <int MODE, int D, int G, int S>
__global__ __launch_bounds__(kRefWaves * kWave, 4) void refresh_kernel(RefreshArgs a) {
    constexpr int RT = ref_rt(MODE, D, G);        // 16-token tiles per wavefront
    constexpr int TW = 16 * RT;                   // tokens per wavefront
    constexpr int KS = D / 32;                    // MFMA k-steps over d
    __shared__ __attribute__((aligned(16))) uint4 kt[2][kRefKeys * D / 8];
    const int lane = (int)(threadIdx.x & (kWave - 1));
    // wavefront index, scalar: every per-wavefront bound below is uniform
    const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int pair = (int)blockIdx.x % a.npair;
    const int tile = a.ntile - 1 - (int)blockIdx.x / a.npair;   // heaviest first
    const int b = pair / a.hkv, h = pair - (pair / a.hkv) * a.hkv;
    const int n = a.n;
    const int T0 = tile * (kRefWaves * TW);
    const int t0 = T0 + wv * TW;                  // this wavefront's tokens
    const int col = lane & 15, grp = lane >> 4;

    // query B-fragments: token tile rt, head g, k-step ks; lane l holds
    // q[token t0 + 16 rt + l%16][32 ks + 8(l/16) .. + 8]
    bf16x8_t qf[RT][G][KS];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int tok = t0 + 16 * rt + col;
        const int tc = tok < n ? tok : n - 1;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const bf16_t* qr = a.q + (((size_t)b * n + tc) * a.hq + h * G + g) * D;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[rt][g][ks] = as_frag(*reinterpret_cast<const uint4*>(qr + 32 * ks + 8 * grp));
        }
    }
    static_assert(MODE != 2 || G == 1, "one pass only for one query head per KV head");
    constexpr bool LSE = MODE != 1, SEL = MODE != 0;
    // (values of the lists: pbar in MODE 1, the raw score in MODE 2)
    constexpr float kEmpty = MODE == 2 ? -INFINITY : 0.0f;
    float m2[RT][G], z[RT][G];     // MODE 0, 2: running max / sum, base 2
    float ls2[RT][G];             // MODE 1: the token's lse + log(G), base 2
    TopS<S> top[RT];             // MODE 1, 2: this lane's sorted top list
    float thr[RT];               // MODE 1, 2: the token's S-th value at the last tile
    const float log2g = G == 1 ? 0.0f : G == 2 ? 1.0f : G == 4 ? 2.0f : 3.0f;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int tok = t0 + 16 * rt + col;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            m2[rt][g] = -1e30f;   // finite: x - m2 stays -inf (not NaN) for masked keys
            z[rt][g] = 0.0f;
            ls2[rt][g] = 0.0f;
            if constexpr (MODE == 1)
                if (tok < n)   // log2 of G folded in: the sum of the G terms is the mean
                    ls2[rt][g] = fmaf(a.lse[((size_t)b * n + tok) * a.hq + h * G + g], kLog2e,
                                      log2g);
        }
        thr[rt] = kEmpty;
#pragma unroll
        for (int e = 0; e < S; ++e) { top[rt].v[e] = kEmpty; top[rt].j[e] = 0x7fffffff; }
    }

    // key tiles, double-buffered: filled by direct global->LDS loads (no
    // registers in between), the next tile's loads in flight while the
    // current one is used
    const bf16_t* kbase = a.k + ((size_t)b * n * a.hkv + h) * D;
    const size_t kstride = (size_t)a.hkv * D;
    const int last = T0 + kRefWaves * TW - 1 < n - 1 ? T0 + kRefWaves * TW - 1 : n - 1;
    load_key_tile<D>(kt[0], kbase, kstride, 0, n, wv, lane);
    for (int j0 = 0, buf = 0; j0 <= last; j0 += kRefKeys, buf ^= 1) {
        // this thread's loads of the tile have landed; after the barrier
        // every thread's have, and no wavefront still reads the other buffer
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (j0 + kRefKeys <= last)
            load_key_tile<D>(kt[buf ^ 1], kbase, kstride, j0 + kRefKeys, n, wv, lane);
        if (j0 > t0 + TW - 1) continue;   // every key of the tile is after this wavefront's tokens
        const uint4* cur = kt[buf];
#pragma unroll
        for (int sub = 0; sub < kRefKeys / 16; ++sub) {
            const int jk = j0 + 16 * sub;
            if (jk > t0 + TW - 1) break;
            const int krow = 16 * sub + col;
            const int key0 = jk + 4 * grp;   // this lane's keys key0 + r
            bool liv[RT];                    // token tile rt has a key at or before it here
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) liv[rt] = jk <= t0 + 16 * rt + 15;
            // every score of the sub-tile first (the matrix cores work through
            // the later tiles while the vector units take the earlier ones),
            // k-step outermost so one key fragment is live at a time and the
            // RT * G accumulator chains interleave
            f32x4_t scs[RT][G];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                // key A-fragment: lane l holds k[jk + l%16][32 ks + 8(l/16) .. + 8]
                const bf16x8_t kf = as_frag(cur[key_slot<D>(krow, 4 * ks + grp)]);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    if (liv[rt])
#pragma unroll
                        for (int g = 0; g < G; ++g)
                            scs[rt][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                kf, qf[rt][g][ks], ks == 0 ? f32x4_t{0.0f, 0.0f, 0.0f, 0.0f} : scs[rt][g], 0, 0, 0);
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                if (!liv[rt]) continue;
                const int tok = t0 + 16 * rt + col;
                const f32x4_t* sc = scs[rt];
                // keys past the token only in the diagonal tiles: masks there alone
                auto body = [&](auto masked) {
                    constexpr bool M = decltype(masked)::value;
                    bool live[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) live[r] = !M || key0 + r <= tok;
                    float x[G][4];
#pragma unroll
                    for (int g = 0; g < G; ++g)
#pragma unroll
                        for (int r = 0; r < 4; ++r) x[g][r] = live[r] ? sc[g][r] : -INFINITY;
                    if constexpr (LSE) {
                        float y[G][4];
                        float my = -INFINITY;
#pragma unroll
                        for (int g = 0; g < G; ++g)
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                y[g][r] = fmaf(x[g][r], a.c, -m2[rt][g]);
                                my = fmaxf(my, y[g][r]);
                            }
                        // rescale only when some lane's term would pass
                        // 2^kSlack: rare once a few hundred keys are in
                        if (__builtin_amdgcn_ballot_w64(my > kSlack)) {
#pragma unroll
                            for (int g = 0; g < G; ++g) {
                                const float mn = fmaxf(
                                    m2[rt][g], max4(x[g][0], x[g][1], x[g][2], x[g][3]) * a.c);
                                z[rt][g] *= fexp2(m2[rt][g] - mn);
                                m2[rt][g] = mn;
#pragma unroll
                                for (int r = 0; r < 4; ++r) y[g][r] = fmaf(x[g][r], a.c, -mn);
                            }
                        }
#pragma unroll
                        for (int g = 0; g < G; ++g)
                            z[rt][g] += (fexp2(y[g][0]) + fexp2(y[g][1])) +
                                        (fexp2(y[g][2]) + fexp2(y[g][3]));
                    }
                    if constexpr (SEL) {
                        float pb[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            if constexpr (MODE == 2) {
                                pb[r] = x[0][r];
                            } else {
                                float e = fexp2(fmaf(sc[0][r], a.c, -ls2[rt][0]));
#pragma unroll
                                for (int g = 1; g < G; ++g)
                                    e += fexp2(fmaf(sc[g][r], a.c, -ls2[rt][g]));
                                pb[r] = live[r] ? e : 0.0f;
                            }
                        }
                        // a key enters only past the token's bound and this
                        // lane's last entry; keys in position order, the
                        // insertion run by the lanes that need it
                        float lim = fmaxf(thr[rt], top[rt].v[S - 1]);
                        if (__builtin_amdgcn_ballot_w64(max4(pb[0], pb[1], pb[2], pb[3]) > lim)) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                if (pb[r] > lim) {
                                    insert_later(top[rt], pb[r], key0 + r);
                                    lim = fmaxf(thr[rt], top[rt].v[S - 1]);
                                }
                            }
                        }
                    }
                };
                if (jk + 15 > t0 + 16 * rt)
                    body(std::true_type{});
                else
                    body(std::false_type{});
            }
        }
        if constexpr (SEL) {
            // the token's four lanes each hold S positions, all before the
            // next tile's keys: a later key no larger than the S-th largest
            // value they hold together has S positions ahead of it and is
            // dropped
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) thr[rt] = union_kth<S>(top[rt].v, grp);
        }
    }

    // combine the four lanes of each token (l%16 + 16c) and write
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int tok = t0 + 16 * rt + col;
        float lse2 = 0.0f;   // MODE 2: the token's lse, base 2
        if constexpr (LSE) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float m = m2[rt][g], zz = z[rt][g];
#pragma unroll
                for (int o = 16; o < kWave; o <<= 1) {
                    const float mo = __shfl_xor(m, o, kWave);
                    const float zo = __shfl_xor(zz, o, kWave);
                    const float mn = fmaxf(m, mo);
                    zz = zz * fexp2(m - mn) + zo * fexp2(mo - mn);
                    m = mn;
                }
                lse2 = m + log2f(zz);
                if (grp == 0 && tok < n)
                    a.lse[((size_t)b * n + tok) * a.hq + h * G + g] = lse2 * 0.69314718055994531f;
            }
        }
        if constexpr (SEL) {
            TopS<S> t = top[rt];
#pragma unroll
            for (int o = 16; o < kWave; o <<= 1) {
                TopS<S> p;
#pragma unroll
                for (int e = 0; e < S; ++e) {
                    p.v[e] = __shfl_xor(t.v[e], o, kWave);
                    p.j[e] = __shfl_xor(t.j[e], o, kWave);
                }
                t = merge(t, p);
            }
            if (grp == 0 && tok < n) {
                const size_t ob = (((size_t)b * n + tok) * a.hkv + h) * a.s;
#pragma unroll
                for (int e = 0; e < S; ++e) {
                    if (e < a.s) {
                        // MODE 2: the weight of a kept score from the final lse
                        const float w = MODE == 2 ? (t.j[e] != 0x7fffffff
                                                         ? fexp2(fmaf(t.v[e], a.c, -lse2))
                                                         : 0.0f)
                                                  : t.v[e];
                        const bool ok = w > 0.0f;
                        a.idx_out[ob + e] = ok ? t.j[e] : 0;
                        a.w_out[ob + e] = ok ? w : 0.0f;
                    }
                }
            }
        }
    }
}

template <int MODE, int D, int G>
hipError_t launch_sel(RefreshArgs a, dim3 grid, hipStream_t st) {
    const dim3 block(kRefWaves * kWave);
    if (a.s <= 2)
        hipLaunchKernelGGL((refresh_kernel<MODE, D, G, 2>), grid, block, 0, st, a);
    else if (a.s <= 4)
        hipLaunchKernelGGL((refresh_kernel<MODE, D, G, 4>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((refresh_kernel<MODE, D, G, kRefSmax>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <int D, int G>
hipError_t run_dg(RefreshArgs a, int B, bool lse_given, hipStream_t st) {
    a.npair = B * a.hkv;
    auto grid = [&](int mode) {
        const int tok = mode == 0   ? ref_tokens(0, D, G)
                        : mode == 1 ? ref_tokens(1, D, G)
                                    : ref_tokens(2, D, G);
        a.ntile = (a.n + tok - 1) / tok;
        return dim3((unsigned)(a.npair * a.ntile));
    };
    if constexpr (G == 1) {
        if (!lse_given) {   // one pass: lse and the edges together
            const dim3 g2 = grid(2);
            return launch_sel<2, D, G>(a, g2, st);
        }
    } else if (!lse_given) {
        const dim3 g0 = grid(0);
        hipLaunchKernelGGL((refresh_kernel<0, D, G, 1>), g0, dim3(kRefWaves * kWave), 0, st, a);
    }
    const dim3 g1 = grid(1);
    return launch_sel<1, D, G>(a, g1, st);
}

}  // namespace

bool dense_refresh_supported(int d, int G, int s) {
    const bool dg = (d == 64 && (G == 1 || G == 2 || G == 4 || G == 8)) ||
                    (d == 128 && (G == 1 || G == 2 || G == 4)) ||
                    (d == 256 && (G == 1 || G == 2));
    return dg && s >= 1 && s <= kRefSmax;
}

hipError_t launch_dense_refresh(int B, int n, int hq, int hkv, int d, float scale,
                                const void* q, const void* k, int s, bool lse_given, float* lse,
                                int32_t* idx_out, float* w_out, hipStream_t st) {
    RefreshArgs a;
    a.q = static_cast<const bf16_t*>(q);
    a.k = static_cast<const bf16_t*>(k);
    a.lse = lse; a.idx_out = idx_out; a.w_out = w_out;
    a.n = n; a.hq = hq; a.hkv = hkv; a.s = s;
    a.c = scale * kLog2e;
    const int G = hq / hkv;
    if (d == 64) {
        switch (G) {
            case 1: return run_dg<64, 1>(a, B, lse_given, st);
            case 2: return run_dg<64, 2>(a, B, lse_given, st);
            case 4: return run_dg<64, 4>(a, B, lse_given, st);
            case 8: return run_dg<64, 8>(a, B, lse_given, st);
        }
    } else if (d == 128) {
        switch (G) {
            case 1: return run_dg<128, 1>(a, B, lse_given, st);
            case 2: return run_dg<128, 2>(a, B, lse_given, st);
            case 4: return run_dg<128, 4>(a, B, lse_given, st);
        }
    } else if (d == 256) {
        switch (G) {
            case 1: return run_dg<256, 1>(a, B, lse_given, st);
            case 2: return run_dg<256, 2>(a, B, lse_given, st);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace gm
