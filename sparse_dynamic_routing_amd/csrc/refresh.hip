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
// (batch, KV head): each wavefront RT 16-token tiles (two when G * d <= 256
// and G <= 2, else one) for all G query heads, with its query rows held as
// B-fragments in registers.  Key tiles of 64 rows are staged in LDS (rows
// padded by 16 bytes against bank conflicts), shared by the eight
// wavefronts, the next tile's global loads in flight while the current one
// is used; the more tokens a workgroup covers, the fewer times each key row
// is fetched (the keys of a pair are re-read once per later token tile).
// The kernels are held to 128 registers (four wavefronts per SIMD): the
// vector work of one wavefront then overlaps the matrix work of another,
// which measured worth more than the few spilled registers it costs.
// Workgroups are issued heaviest first (the last token tiles see the most
// keys), consecutive workgroups on different (batch, KV head) pairs so one
// XCD keeps a fixed set of pairs.
//
// Two passes: the first keeps an online max/sum per (token, head) in base 2
// (rescaled only when a maximum passes the reference by a factor 2^16, a wavefront-
// uniform branch that is rarely taken) and writes lse (skipped when the caller
// passes the dense layer's own lse); the second recomputes the scores, forms
// pbar and keeps the top list.  The four lanes of a token share, after
// every 16 keys, the largest of their S-th kept values: a later key at or
// below it already has S positions ahead of it, so it is dropped without
// touching the list.
#include "gm_common.h"
#include "gm_internal.h"
#include "gm_wave.h"

#include <type_traits>

namespace gm {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRefKeys = 64;     // keys per LDS tile
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

// the largest of x over the four rows of the wavefront (lanes l%16 + 16c)
__device__ __forceinline__ float max_over_rows(float x) {
    float a = x, b = x;
    swap16(a, b);
    x = fmaxf(a, b);
    a = x;
    b = x;
    swap32(a, b);
    return fmaxf(a, b);
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
// insert (v, j) where j exceeds every position already held: an equal value
// stays behind, so only a strictly larger one enters
template <int S>
__device__ __forceinline__ void insert_later(TopS<S>& t, float v, int j) {
    if (!(v > t.v[S - 1])) return;
    t.v[S - 1] = v;
    t.j[S - 1] = j;
#pragma unroll
    for (int e = S - 1; e > 0; --e) {
        if (t.v[e] > t.v[e - 1]) {
            const float tv = t.v[e]; t.v[e] = t.v[e - 1]; t.v[e - 1] = tv;
            const int tj = t.j[e]; t.j[e] = t.j[e - 1]; t.j[e - 1] = tj;
        }
    }
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

// 16-token tiles per wavefront: as many as keep the query fragments within
// 128 registers (RT * G * d / 8 of them)
constexpr int ref_rt(int D, int G) { return G <= 2 && G * D <= 256 ? 2 : 1; }
constexpr int kRefWaves = 8;     // wavefronts per workgroup
constexpr int ref_tokens(int D, int G) { return kRefWaves * 16 * ref_rt(D, G); }

// MODE 0: lse; MODE 1: the top-S refresh edges.  D head dim, G query heads
// per KV head.
template <int MODE, int D, int G, int S>
__global__ __launch_bounds__(kRefWaves * kWave, 4) void refresh_kernel(RefreshArgs a) {
    constexpr int RT = ref_rt(D, G);              // 16-token tiles per wavefront
    constexpr int NT = kRefWaves * kWave;         // threads
    constexpr int TW = 16 * RT;                   // tokens per wavefront
    constexpr int KS = D / 32;                    // MFMA k-steps over d
    constexpr int ROWB = D * 2 + 16;              // padded LDS row bytes
    constexpr int PPR = D / 8;                    // 16-byte pieces per key row
    constexpr int U = kRefKeys * PPR / NT;        // pieces per thread per tile
    static_assert(U >= 1 && U * NT == kRefKeys * PPR, "tile pieces must divide evenly");
    __shared__ __attribute__((aligned(16))) unsigned char kt[kRefKeys * ROWB];
    const int lane = (int)(threadIdx.x & (kWave - 1));
    const int wv = (int)threadIdx.x / kWave;
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
    float m2[RT][G], z[RT][G];     // MODE 0: running max / sum, base 2
    float ls2[RT][G];             // MODE 1: the token's lse + log(G), base 2
    const float log2g = G == 1 ? 0.0f : G == 2 ? 1.0f : G == 4 ? 2.0f : 3.0f;
    TopS<S> top[RT];
    float thr[RT];               // MODE 1: drop candidates at or below this
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
#pragma unroll
        for (int e = 0; e < S; ++e) { top[rt].v[e] = 0.0f; top[rt].j[e] = 0x7fffffff; }
        thr[rt] = 0.0f;
    }

    // this thread's pieces of a key tile: piece p = threadIdx + NT u
    const bf16_t* kbase = a.k + ((size_t)b * n * a.hkv + h) * D;
    const size_t kstride = (size_t)a.hkv * D;
    uint4 pf[U];
    auto fetch = [&](int j0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = (int)threadIdx.x + NT * u;
            const int row = p / PPR, piece = p - (p / PPR) * PPR;
            const int j = j0 + row < n ? j0 + row : n - 1;
            pf[u] = *reinterpret_cast<const uint4*>(kbase + (size_t)j * kstride + piece * 8);
        }
    };
    const int last = T0 + kRefWaves * TW - 1 < n - 1 ? T0 + kRefWaves * TW - 1 : n - 1;
    fetch(0);
    for (int j0 = 0; j0 <= last; j0 += kRefKeys) {
        __syncthreads();   // every wavefront is done with the previous tile
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = (int)threadIdx.x + NT * u;
            const int row = p / PPR, piece = p - (p / PPR) * PPR;
            *reinterpret_cast<uint4*>(kt + row * ROWB + piece * 16) = pf[u];
        }
        __syncthreads();
        if (j0 + kRefKeys <= last) fetch(j0 + kRefKeys);   // in flight during this tile
        if (j0 > t0 + TW - 1) continue;   // every key of the tile is after this wavefront's tokens
#pragma unroll
        for (int sub = 0; sub < kRefKeys / 16; ++sub) {
            const int jk = j0 + 16 * sub;
            if (jk > t0 + TW - 1) break;
            // key A-fragments: lane l holds k[jk + l%16][32 ks + 8(l/16) .. + 8]
            bf16x8_t kf[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kf[ks] = as_frag(*reinterpret_cast<const uint4*>(kt + (16 * sub + col) * ROWB +
                                                                 (32 * ks + 8 * grp) * 2));
            const int key0 = jk + 4 * grp;   // this lane's keys key0 + r
            // every score of the sub-tile first: the matrix cores work through
            // the later tiles while the vector units take the earlier ones
            f32x4_t scs[RT][G];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                if (jk > t0 + 16 * rt + 15) continue;   // all keys after all tokens
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qf[rt][g][ks], acc,
                                                                      0, 0, 0);
                    scs[rt][g] = acc;
                }
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                if (jk > t0 + 16 * rt + 15) continue;
                const int tok = t0 + 16 * rt + col;
                const f32x4_t* sc = scs[rt];
                // keys past the token only in the diagonal tiles: masks there alone
                auto body = [&](auto masked) {
                    constexpr bool M = decltype(masked)::value;
                    bool live[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) live[r] = !M || key0 + r <= tok;
                    if constexpr (MODE == 0) {
#pragma unroll
                        for (int g = 0; g < G; ++g) {
                            float x[4];
#pragma unroll
                            for (int r = 0; r < 4; ++r) x[r] = live[r] ? sc[g][r] : -INFINITY;
                            const float mx = max4(x[0], x[1], x[2], x[3]) * a.c;
                            // rescale only when some lane's maximum passes its
                            // reference by kSlack (terms stay below 2^kSlack):
                            // rare once a few hundred keys are in
                            if (__builtin_amdgcn_ballot_w64(mx > m2[rt][g] + kSlack)) {
                                const float mn = fmaxf(m2[rt][g], mx);
                                z[rt][g] *= fexp2(m2[rt][g] - mn);
                                m2[rt][g] = mn;
                            }
                            const float nm = -m2[rt][g];
                            z[rt][g] += (fexp2(fmaf(x[0], a.c, nm)) + fexp2(fmaf(x[1], a.c, nm))) +
                                        (fexp2(fmaf(x[2], a.c, nm)) + fexp2(fmaf(x[3], a.c, nm)));
                        }
                    } else {
                        float pb[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            float x = fexp2(fmaf(sc[0][r], a.c, -ls2[rt][0]));
#pragma unroll
                            for (int g = 1; g < G; ++g) x += fexp2(fmaf(sc[g][r], a.c, -ls2[rt][g]));
                            pb[r] = live[r] ? x : 0.0f;
                        }
                        const float mx = max4(pb[0], pb[1], pb[2], pb[3]);
                        if (mx > thr[rt]) {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                insert_later(top[rt], pb[r] > thr[rt] ? pb[r] : 0.0f, key0 + r);
                        }
                    }
                };
                if (jk + 15 > t0 + 16 * rt)
                    body(std::true_type{});
                else
                    body(std::false_type{});
            }
            if constexpr (MODE == 1) {
                // the token's four lanes each hold S positions, all before this
                // sub-tile's keys: a later key no larger than the largest of
                // their S-th values has S positions ahead of it and is dropped
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) thr[rt] = max_over_rows(top[rt].v[S - 1]);
            }
        }
    }

    // combine the four lanes of each token (l%16 + 16c) and write
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int tok = t0 + 16 * rt + col;
        if constexpr (MODE == 0) {
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
                if (grp == 0 && tok < n)
                    a.lse[((size_t)b * n + tok) * a.hq + h * G + g] =
                        (m + log2f(zz)) * 0.69314718055994531f;
            }
        } else {
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
                        const bool ok = t.v[e] > 0.0f;
                        a.idx_out[ob + e] = ok ? t.j[e] : 0;
                        a.w_out[ob + e] = ok ? t.v[e] : 0.0f;
                    }
                }
            }
        }
    }
}

template <int D, int G>
hipError_t run_dg(RefreshArgs a, int B, bool lse_given, hipStream_t st) {
    constexpr int TOK = ref_tokens(D, G);
    a.ntile = (a.n + TOK - 1) / TOK;
    a.npair = B * a.hkv;
    const dim3 grid((unsigned)(a.npair * a.ntile)), block(kRefWaves * kWave);
    if (!lse_given) hipLaunchKernelGGL((refresh_kernel<0, D, G, 1>), grid, block, 0, st, a);
    if (a.s <= 2)
        hipLaunchKernelGGL((refresh_kernel<1, D, G, 2>), grid, block, 0, st, a);
    else if (a.s <= 4)
        hipLaunchKernelGGL((refresh_kernel<1, D, G, 4>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((refresh_kernel<1, D, G, kRefSmax>), grid, block, 0, st, a);
    return hipGetLastError();
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
