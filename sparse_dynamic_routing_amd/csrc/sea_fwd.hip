// Sparse edge attention, forward, for gfx950.
//
// Computes, per unit (b, token i, KV head h) and per query head of the group
// (ai.info "Graph Machine: Towards Better Pretraining via Edges", Key
// Contributions 3 and Methodology, second job of a sparse layer):
//   l_t = scale * q . k[idx_t] + ln w_t   over the live slots (w_t > 0)
//   o   = sum_t softmax(l)_t v[idx_t]
// in the log2 domain (l * log2 e), which is the same softmax.
//
// Mapping: one team of R * P lanes per unit.  R lanes hold one d-row of K
// or V in 16-byte pieces (one global_load_dwordx4 per lane), P slots are
// loaded side by side, so at d = 128 bf16 and s = 4 one wave64 fetches the
// unit's four K rows in one instruction and its four V rows in another, and
// that single fetch serves all G query heads of the KV group.  Dot products
// reduce over the R lanes of a row; the softmax and the weighted V sum reduce
// over the P slot lanes.  The output is reduce-scattered so every lane
// stores a distinct piece.  No MFMA and no LDS: the work is a gather with a
// few FLOPs per byte (HBM-bound).
#include "gm_common.h"
#include "gm_internal.h"
#include "gm_select.h"
#include "gm_wave.h"

#include <math.h>

namespace gm {

TeamShape sea_team(int d, int elem_bytes, int s) {
    TeamShape t;
    t.R = d * elem_bytes / 16;
    t.log2R = ilog2(t.R);
    int pmax = kWave / t.R;
    t.P = pow2_ceil(s) < pmax ? pow2_ceil(s) : pmax;
    t.team = t.R * t.P;
    t.nchunk = (s + t.P - 1) / t.P;
    return t;
}

namespace {

// The saved statistics of a unit (pair-major row `prow`) are E G + 2 rows
// of s 4-byte words: p / w per query head and slot, in the precision the
// backward computes in (E = 1: fp32 for bf16 inputs; E = 2: fp64 for fp32
// inputs, G s doubles), then the unit's edge indices (int32 bits) and
// weights, a pair-major copy of its edge row for the backward.  A is the
// accumulation type (float for bf16 inputs, double for fp32), so E =
// sizeof(A) / 4.
template <typename A>
__device__ __forceinline__ void store_edge_copy(float* stats, size_t prow, int G, int s, int t,
                                                int j, float wt) {
    constexpr int E = sizeof(A) / 4;
    float* e = stats + (prow * (E * G + 2) + E * G) * s;
    e[t] = __int_as_float(j);
    e[s + t] = wt;
}
template <typename A>
__device__ __forceinline__ void store_pw(float* stats, size_t prow, int G, int s, int g, int t,
                                         A v) {
    if constexpr (sizeof(A) == 4)
        stats[(prow * (G + 2) + g) * s + t] = v;
    else
        reinterpret_cast<double*>(stats)[(prow * (G + 1) + g) * s + t] = v;
}

struct SeaFwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* idx;
    const float* w;
    void* o;
    float* stats;   // [B][hkv][n][E G + 2][s]: p / w per live slot (0 dead), idx, w; or null
    int n, hq, hkv, d, s, U;
    float scale;
    TeamShape ts;
};

template <typename T, int GT>
__global__ __launch_bounds__(kBlock) void sea_fwd_kernel(SeaFwdArgs a) {
    // GT > 0: the group size as a constant; 0: any group size, from the heads
    const int G = GT > 0 ? GT : a.hq / a.hkv;
    using A = typename io<T>::acc;
    constexpr int V = io<T>::V;
    constexpr int LOG2V = ilog2(V);
    const int R = a.ts.R, team = a.ts.team;
    const int lane = threadIdx.x & (kWave - 1);
    const int tl = lane & (team - 1);
    const int r = tl & (R - 1);
    const int sl = tl >> a.ts.log2R;
    const long long gunit = ((long long)blockIdx.x * kBlock + threadIdx.x) / team;
    if (gunit >= a.U) return;  // whole team leaves together
    const int unit = (int)gunit;
    const int h = unit % a.hkv;
    const int bi = unit / a.hkv;          // b * n + i
    const int b = bi / a.n;
    const size_t srow = ((size_t)b * a.hkv + h) * a.n + (bi - b * a.n);   // pair-major row
    const size_t d = (size_t)a.d;
    const T* qp = static_cast<const T*>(a.q) + ((size_t)bi * a.hq + (size_t)h * G) * d + r * V;
    T* op = static_cast<T*>(a.o) + ((size_t)bi * a.hq + (size_t)h * G) * d + r * V;
    const T* kp = static_cast<const T*>(a.k) + r * V;
    const T* vp = static_cast<const T*>(a.v) + r * V;
    const size_t kv0 = (size_t)b * a.n * a.hkv + h;   // K/V row of token j: kv0 + j * hkv
    const int32_t* ip = a.idx + (size_t)unit * a.s;
    const float* wp = a.w + (size_t)unit * a.s;
    const A c = (A)a.scale * (A)1.4426950408889634;  // scale * log2(e)
    const A NEG = -INFINITY;
    // lanes holding a duplicate of another lane's output piece do not store
    const bool storer = (sl >> LOG2V) == 0;

    if (a.ts.nchunk == 1) {
        const int t = sl;
        bool live = false;
        A lw = NEG;
        A kr[V], vr[V];
#pragma unroll
        for (int e = 0; e < V; ++e) { kr[e] = 0; vr[e] = 0; }
        if (t < a.s) {
            const float wt = wp[t];
            if (wt > 0.0f) {
                live = true;
                lw = alog2((A)wt);
                const size_t row = (kv0 + (size_t)ip[t] * a.hkv) * d;
                load16(kp + row, kr);
                load16(vp + row, vr);
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            A qg[V];
            load16(qp + g * d, qg);
            A dot = 0;
#pragma unroll
            for (int e = 0; e < V; ++e) dot += qg[e] * kr[e];
            dot = sum_bits(dot, 1, R);
            const A l = live ? dot * c + lw : NEG;
            const A M = max_bits(l, R, team);
            const A ex = live ? aexp2(l - M) : (A)0;
            const A Z = sum_bits(ex, R, team);
            A ov[V];
#pragma unroll
            for (int e = 0; e < V; ++e) ov[e] = ex * vr[e];
            int len;
            const int off = reduce_scatter(ov, tl, R, team, len);
            const A inv = Z > 0 ? (A)1 / Z : (A)0;
            if (a.stats && r == 0 && t < a.s)
                store_pw<A>(a.stats, srow, G, a.s, g, t, live ? aexp2(dot * c - M) * inv : (A)0);
#pragma unroll
            for (int e = 0; e < V; ++e) ov[e] *= inv;
            if (storer) store_len(op + g * d + off, ov, len);
        }
        if (a.stats && r == 0 && t < a.s)
            store_edge_copy<A>(a.stats, srow, G, a.s, t, ip[t], wp[t]);
        return;
    }

    // s > P: walk the slots in chunks of P with a running max and sum.
    const int P = a.ts.P;
#pragma unroll 1
    for (int g = 0; g < G; ++g) {
        A qg[V];
        load16(qp + g * d, qg);
        A M = NEG, Z = 0;
        A ov[V];
#pragma unroll
        for (int e = 0; e < V; ++e) ov[e] = 0;
#pragma unroll 1
        for (int ch = 0; ch < a.ts.nchunk; ++ch) {
            const int t = ch * P + sl;
            bool live = false;
            A lw = NEG;
            A kr[V], vr[V];
#pragma unroll
            for (int e = 0; e < V; ++e) { kr[e] = 0; vr[e] = 0; }
            if (t < a.s) {
                const float wt = wp[t];
                if (wt > 0.0f) {
                    live = true;
                    lw = alog2((A)wt);
                    const size_t row = (kv0 + (size_t)ip[t] * a.hkv) * d;
                    load16(kp + row, kr);
                    load16(vp + row, vr);
                }
            }
            A dot = 0;
#pragma unroll
            for (int e = 0; e < V; ++e) dot += qg[e] * kr[e];
            dot = sum_bits(dot, 1, R);
            const A l = live ? dot * c + lw : NEG;
            const A Mn = amax(M, max_bits(l, R, team));
            if (Mn == NEG) continue;  // uniform over the team: nothing live yet
            const A alpha = aexp2(M - Mn);
            const A ex = live ? aexp2(l - Mn) : (A)0;
            Z = Z * alpha + sum_bits(ex, R, team);
#pragma unroll
            for (int e = 0; e < V; ++e) ov[e] = ov[e] * alpha + ex * vr[e];
            M = Mn;
        }
        int len;
        const int off = reduce_scatter(ov, tl, R, team, len);
        const A inv = Z > 0 ? (A)1 / Z : (A)0;
#pragma unroll
        for (int e = 0; e < V; ++e) ov[e] *= inv;
        if (storer) store_len(op + g * d + off, ov, len);
        if (a.stats) {
            // p / w of every slot needs the final M and Z: the scores again
#pragma unroll 1
            for (int ch = 0; ch < a.ts.nchunk; ++ch) {
                const int t = ch * P + sl;
                bool live = false;
                A kr[V];
#pragma unroll
                for (int e = 0; e < V; ++e) kr[e] = 0;
                if (t < a.s && wp[t] > 0.0f) {
                    live = true;
                    load16(kp + (kv0 + (size_t)ip[t] * a.hkv) * d, kr);
                }
                A dot = 0;
#pragma unroll
                for (int e = 0; e < V; ++e) dot += qg[e] * kr[e];
                dot = sum_bits(dot, 1, R);
                if (r == 0 && t < a.s) {
                    store_pw<A>(a.stats, srow, G, a.s, g, t,
                                live ? aexp2(dot * c - M) * inv : (A)0);
                    if (g == 0) store_edge_copy<A>(a.stats, srow, G, a.s, t, ip[t], wp[t]);
                }
            }
        }
    }
}


// ----------------------------------------------------------------- fast path
// One d-row (256 bytes: bf16 d=128 or fp32 d=64; the row kernel also takes
// 128- and 512-byte rows) = one 16-lane row of the wave.  Persistent
// XCD-aware loop over units in pair-major order; the next unit's edge slots
// are fetched one unit ahead.
struct SeaFwdFast {
    const char* q;
    const char* k;
    const char* v;
    const int32_t* idx;
    const float* w;
    char* o;
    float* stats;   // [B][hkv][n][G + 2][s]: p / w per live slot (0 dead), idx, w; or null
    int n, hq, hkv, s, U;
    float scale;
    SegPlan sp;
    int vec;   // s == 4 and 16-byte aligned edge rows: one load per row
};

struct UnitPos {
    int unit;      // (b*n + i)*hkv + h
    int bi;        // b*n + i
    int kvrow0;    // K/V row of token 0 of the pair: b*n*hkv + h
    int prow;      // pair-major row: (b*hkv + h)*n + i
};

__device__ __forceinline__ UnitPos unit_pos(const SegPlan& sp, int x, int q) {
    int pair, i;
    sched_item(sp, x, q, pair, i);
    const int n = sp.n, hkv = sp.hkv;
    const int b = (int)fdiv((uint32_t)pair, sp.fd_hkv);
    const int h = pair - b * hkv;
    UnitPos p;
    p.bi = b * n + i;
    p.unit = p.bi * hkv + h;
    p.kvrow0 = b * n * hkv + h;
    p.prow = pair * n + i;
    return p;
}

template <typename T, int G>
hipError_t run(const SeaFwdArgs& a, hipStream_t st) {
    const long long threads = (long long)a.U * a.ts.team;
    const unsigned blocks = (unsigned)((threads + kBlock - 1) / kBlock);
    hipLaunchKernelGGL((sea_fwd_kernel<T, G>), dim3(blocks), dim3(kBlock), 0, st, a);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch_g(const SeaFwdArgs& a, int G, hipStream_t st) {
    switch (G) {
        case 1: return run<T, 1>(a, st);
        case 2: return run<T, 2>(a, st);
        case 4: return run<T, 4>(a, st);
        case 8: return run<T, 8>(a, st);
        case 16: return run<T, 16>(a, st);
        default: return run<T, 0>(a, st);   // other group sizes
    }
}

// One unit per 16-lane row, four units per wavefront.  Lane r of the row
// holds bytes [256k + 16r, 256k + 16r + 16), k < R, of every (256 R)-byte
// d-row the unit touches (its G query rows, and the K and V rows of its S
// edge slots, side by side in registers): R = 1 for bf16 at d = 128 (and
// fp32 at d = 64), R = 2 for bf16 at d = 256 and fp32 at d = 128.  R = 0
// takes 128-byte rows (bf16 d = 64, fp32 d = 32): lane r holds bytes
// [8r, 8r + 8) in the low half of its registers, the high half zero.  The
// only cross-lane step is the 16-lane DPP sum of each score; the softmax
// over the slots and the weighted sum of the V rows are lane-local.  Slots
// t >= s (when s < S) are dead.  Rows never exchange data, so rows of one
// wavefront may leave the item loop at different times.  With s = 4,
// aligned edge rows and bf16 256- or 512-byte d-rows, the edge rows of a
// wavefront's next four units come through the scalar data cache, so the
// wait for them at the top of a unit does not also drain the previous
// unit's vector stores (at 128-byte rows, and with the fp64 accumulators of
// fp32 inputs, the scalar rows' registers cost more than the drain:
// measured slower).
template <typename T, int G, int S, bool VEC, int R>
__global__ __launch_bounds__(kBlock) void sea_fwd_row_kernel(SeaFwdFast a) {
    using A = typename io<T>::acc;
    constexpr int V = io<T>::V;
    constexpr int ROW = R == 0 ? 128 : 256 * R;
    constexpr int NP = R == 0 ? 1 : R;    // register parts per row
    constexpr int LB = R == 0 ? 8 : 16;   // bytes of a part per lane
    constexpr int GC = G < 4 ? G : 4;     // query rows held at once
    const int r = threadIdx.x & 15;
    const A c = (A)a.scale * (A)1.4426950408889634;
    const A NEG = -INFINITY;
    const Sched sc = xcd_sched(a.sp, 16);
    if (sc.q >= sc.end) return;

    constexpr bool SCAL = VEC && S == 4 && R != 0 && std::is_same<T, bf16_t>::value;
    struct Item {
        UnitPos pos;
        int j[S];
        float wt[S];
        float sr[SCAL ? 32 : 1];   // SCAL: the four units' index and weight rows
    };
    // the item's edge slots; past the end the last item is read again (a
    // valid address, so the load needs no branch) and never used
    auto fetch = [&](int u) {
        Item it;
        it.pos = unit_pos(a.sp, sc.x, u < sc.end ? u : sc.end - 1);
        if constexpr (SCAL) {
            // row k of the wavefront holds item ub + k (row 0's item is
            // ub), clamped at the end like the vector path
            typedef const __attribute__((address_space(4))) float cf4;
            const int ub = __builtin_amdgcn_readfirstlane(u);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const UnitPos pk = unit_pos(a.sp, sc.x, ub + k < sc.end ? ub + k : sc.end - 1);
                cf4* ip = (cf4*)(reinterpret_cast<const float*>(a.idx) + (size_t)pk.unit * 4);
                cf4* wp = (cf4*)(a.w + (size_t)pk.unit * 4);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    it.sr[k * 8 + t] = ip[t];
                    it.sr[k * 8 + 4 + t] = wp[t];
                }
            }
            return it;
        } else if constexpr (VEC) {
            const int4 j4 = *reinterpret_cast<const int4*>(a.idx + (size_t)it.pos.unit * 4);
            const float4 w4 = *reinterpret_cast<const float4*>(a.w + (size_t)it.pos.unit * 4);
            it.j[0] = j4.x; it.j[1] = j4.y; it.j[2] = j4.z; it.j[3] = j4.w;
            it.wt[0] = w4.x; it.wt[1] = w4.y; it.wt[2] = w4.z; it.wt[3] = w4.w;
        } else {
            const size_t e0 = (size_t)it.pos.unit * a.s;
#pragma unroll
            for (int t = 0; t < S; ++t) {
                const int tt = t < a.s ? t : a.s - 1;
                it.j[t] = a.idx[e0 + tt];
                const float wv = a.w[e0 + tt];
                it.wt[t] = t < a.s ? wv : 0.0f;
            }
        }
        return it;
    };

    Item cur = fetch(sc.q);
    for (int u = sc.q; u < sc.end; u += sc.step) {
        const Item nxt = fetch(u + sc.step);
        if constexpr (SCAL) {
            // this row's unit: a blend of the four scalar rows under row
            // masks (opaque, so that the blend is not turned into an
            // indexed access through scratch memory)
            const int rw = (threadIdx.x >> 4) & 3;
            uint32_t m0 = rw == 0 ? ~0u : 0u, m1 = rw == 1 ? ~0u : 0u;
            uint32_t m2 = rw == 2 ? ~0u : 0u, m3 = rw == 3 ? ~0u : 0u;
            asm("" : "+v"(m0), "+v"(m1), "+v"(m2), "+v"(m3));
#pragma unroll
            for (int w = 0; w < 32; ++w) asm("" : "+s"(cur.sr[w]));
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const uint32_t v = (__float_as_uint(cur.sr[t]) & m0) |
                                   (__float_as_uint(cur.sr[8 + t]) & m1) |
                                   (__float_as_uint(cur.sr[16 + t]) & m2) |
                                   (__float_as_uint(cur.sr[24 + t]) & m3);
                if (t < 4) cur.j[t] = (int)v; else cur.wt[t - 4] = __uint_as_float(v);
            }
        }
        bool live[S];
        uint4 kr[S][NP], vr[S][NP];
#pragma unroll
        for (int t = 0; t < S; ++t) {
            live[t] = cur.wt[t] > 0.0f;
            const uint32_t off =
                (uint32_t)(cur.pos.kvrow0 + (live[t] ? cur.j[t] : 0) * a.hkv) * ROW + r * LB;
#pragma unroll
            for (int k = 0; k < NP; ++k) {
                if constexpr (R == 0) {
                    const uint2 k2 = *reinterpret_cast<const uint2*>(a.k + off);
                    const uint2 v2 = *reinterpret_cast<const uint2*>(a.v + off);
                    kr[t][k] = make_uint4(k2.x, k2.y, 0u, 0u);
                    vr[t][k] = make_uint4(v2.x, v2.y, 0u, 0u);
                } else {
                    kr[t][k] = *reinterpret_cast<const uint4*>(a.k + off + 256 * k);
                    vr[t][k] = *reinterpret_cast<const uint4*>(a.v + off + 256 * k);
                }
            }
        }
        const uint32_t qoff =
            (uint32_t)(cur.pos.bi * a.hq + (cur.pos.unit - cur.pos.bi * a.hkv) * G) * ROW + r * LB;
        A lw[S];
#pragma unroll
        for (int t = 0; t < S; ++t) lw[t] = live[t] ? fast_log2((A)cur.wt[t]) : NEG;
        // the unit's statistics, p / w per head and slot, then its edge
        // indices and weights, in one store per lane when they fit 16 lanes
        // (fp32 words only: fp64 p / w, E = 2, store per head)
        constexpr int E = sizeof(A) / 4;
        const bool st_one = E == 1 && (G + 2) * a.s <= 16;
        float st_val = 0.0f;
        if (a.stats) {
            // lanes G s .. (G + 2) s - 1: the edge copy (index bits, then weight)
            const int te = r - G * a.s;
            float ev = 0.0f;
#pragma unroll
            for (int t = 0; t < S; ++t) {
                if (t < a.s) {
                    ev = te == t ? __int_as_float(cur.j[t]) : ev;
                    ev = te == a.s + t ? cur.wt[t] : ev;
                }
            }
            if (st_one) {
                st_val = ev;
            } else if (r < a.s) {
                float* e = a.stats + ((size_t)cur.pos.prow * (E * G + 2) + E * G) * a.s;
                float jv = 0.0f, wv = 0.0f;
#pragma unroll
                for (int t = 0; t < S; ++t) {
                    jv = r == t ? __int_as_float(cur.j[t]) : jv;
                    wv = r == t ? cur.wt[t] : wv;
                }
                __builtin_nontemporal_store(jv, e + r);
                __builtin_nontemporal_store(wv, e + a.s + r);
            }
        }
#pragma unroll
        for (int g0 = 0; g0 < G; g0 += GC) {
            uint4 qr[GC][NP];
#pragma unroll
            for (int g = 0; g < GC; ++g)
#pragma unroll
                for (int k = 0; k < NP; ++k)
                    qr[g][k] = R == 0 ? load_nt8(a.q + qoff + (g0 + g) * ROW)
                                      : load_nt16(a.q + qoff + (g0 + g) * ROW + 256 * k);
#pragma unroll
            for (int g = 0; g < GC; ++g) {
                A l[S], sd[S], M = NEG;
#pragma unroll
                for (int t = 0; t < S; ++t) {
                    A dp = dot16<V, A>(qr[g][0], kr[t][0]);
#pragma unroll
                    for (int k = 1; k < NP; ++k) dp += dot16<V, A>(qr[g][k], kr[t][k]);
                    sd[t] = row_sum16(dp) * c;
                    l[t] = live[t] ? sd[t] + lw[t] : NEG;
                    M = l[t] > M ? l[t] : M;
                }
                A p[S], Z = 0;
#pragma unroll
                for (int t = 0; t < S; ++t) {
                    p[t] = live[t] ? fast_exp2(l[t] - M) : (A)0;
                    Z += p[t];
                }
                const A inv = Z > (A)0 ? fast_rcp(Z) : (A)0;
                if (a.stats) {
                    // p / w of slot t (the backward's softmax without q):
                    // when the unit's G * s values fit the 16 lanes, lane
                    // g * s + t keeps it for one store per row after the
                    // heads; otherwise lane t stores it per head
                    const int t0 = st_one ? r - (g0 + g) * a.s : r;
                    A mine = sd[0];
                    bool ml = live[0];
#pragma unroll
                    for (int t = 1; t < S; ++t) {
                        mine = t0 == t ? sd[t] : mine;
                        ml = t0 == t ? live[t] : ml;
                    }
                    const A pv = ml ? fast_exp2(mine - M) * inv : (A)0;
                    if (t0 >= 0 && t0 < a.s) st_val = (float)pv;
                    if (!st_one && t0 >= 0 && t0 < a.s) {
                        if constexpr (E == 1)
                            __builtin_nontemporal_store(
                                st_val,
                                a.stats + ((size_t)cur.pos.prow * (G + 2) + g0 + g) * a.s + t0);
                        else
                            __builtin_nontemporal_store(
                                (double)pv, reinterpret_cast<double*>(a.stats) +
                                                ((size_t)cur.pos.prow * (G + 1) + g0 + g) * a.s + t0);
                    }
                }
#pragma unroll
                for (int k = 0; k < NP; ++k) {
                    A o[V];
#pragma unroll
                    for (int e = 0; e < V; ++e) o[e] = 0;
#pragma unroll
                    for (int t = 0; t < S; ++t) {
                        A vf[V];
                        unpack16<A, V>(vr[t][k], vf);
                        const A pt = p[t] * inv;
#pragma unroll
                        for (int e = 0; e < V; ++e) o[e] += pt * vf[e];
                    }
                    char* op = a.o + qoff + (g0 + g) * ROW + 256 * k;
                    if constexpr (R == 0) {
                        if constexpr (V == 8) {
                            const u32x2_t h = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
                            __builtin_nontemporal_store(h, reinterpret_cast<u32x2_t*>(op));
                        } else {
                            store_f32_nt<2>(op, o);
                        }
                    } else if constexpr (V == 8) {
                        store_u32x4_nt(op, pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                                       pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7]));
                    } else {
                        store_f32_nt<4>(op, o);
                    }
                }
            }
        }
        if (a.stats && st_one && r < (G + 2) * a.s)
            __builtin_nontemporal_store(st_val,
                                        a.stats + (size_t)cur.pos.prow * (G + 2) * a.s + r);
        cur = nxt;
    }
}

template <typename T, int G, int S, bool VEC, int R>
hipError_t run_row(const SeaFwdFast& a, hipStream_t st) {
    const void* fn = reinterpret_cast<const void*>(&sea_fwd_row_kernel<T, G, S, VEC, R>);
    const int nwg = persistent_grid(fn, a.U, kBlock / 16);
    hipLaunchKernelGGL((sea_fwd_row_kernel<T, G, S, VEC, R>), dim3(nwg), dim3(kBlock), 0, st, a);
    return hipGetLastError();
}

template <typename T, int G, int R>
hipError_t fast_p(const SeaFwdFast& a, hipStream_t st) {
    if (a.s <= 1) return run_row<T, G, 1, false, R>(a, st);
    if (a.s <= 2) return run_row<T, G, 2, false, R>(a, st);
    if (a.vec) return run_row<T, G, 4, true, R>(a, st);
    return run_row<T, G, 4, false, R>(a, st);
}

template <typename T, int R>
hipError_t fast_g(const SeaFwdFast& a, int G, hipStream_t st) {
    switch (G) {
        case 1: return fast_p<T, 1, R>(a, st);
        case 2: return fast_p<T, 2, R>(a, st);
        case 4: return fast_p<T, 4, R>(a, st);
        case 8: return fast_p<T, 8, R>(a, st);
        case 16: return fast_p<T, 16, R>(a, st);
        default: return hipErrorInvalidValue;
    }
}


// ------------------------------------------------- fused SER -> SEA forward
// A' = Sparsify_4(A1 A2) and o = SEA(q, k, v, A') in one pass, for bf16,
// d = 128, s1 = s2 = s3 = 4 (the measured layer): one unit per 16-lane row
// as in sea_fwd_row_kernel, and lane k of the row holds the unit's two-hop
// candidate k = 4a + c (leg-1 slot a, leg-2 slot c).  The row merges and
// ranks its 16 candidates with the team code of gm_select.h (DPP row
// rotations; fp64 sums in path order, so A' is bitwise what gm_ser_forward
// writes), writes A', and goes on with the kept slots exactly as the SEA
// row kernel.  The unit's leg-1 row is read two units ahead and its leg-2
// rows one unit ahead, so the three dependent loads of a unit (leg 1, leg 2,
// K/V) overlap other units' work; A' never goes through memory between the
// two stages.
struct SerSeaFwd {
    SeaFwdFast f;          // SEA part; f.idx / f.w unused (A' is in registers)
    const int32_t* idx1;
    const float* w1;
    const int32_t* idx2;
    const float* w2;
    int32_t* idx_out;
    float* w_out;
    uint64_t* paths;       // path map per unit (as gm_ser_forward writes it), or null
};

template <int G>
__global__ __launch_bounds__(kBlock) void ser_sea_fwd_row_kernel(SerSeaFwd a) {
    using A = float;
    constexpr int V = 8, S = 4;
    constexpr int ROW = 256;
    constexpr int GC = G < 4 ? G : 4;     // query rows held at once
    const int r = threadIdx.x & 15;       // d-row piece, and candidate k = 4 aa + cc
    const int aa = r >> 2, cc = r & 3;
    const int rbase = threadIdx.x & (kWave - 1) & ~15;   // first lane of this 16-lane row
    const A c = (A)a.f.scale * (A)1.4426950408889634;
    const A NEG = -INFINITY;
    const int hkv = a.f.hkv;
    const Sched sc = xcd_sched(a.f.sp, 16);
    if (sc.q >= sc.end) return;

    struct Leg1 {
        UnitPos pos;
        int j;       // leg-1 slot aa: target token
        float x;     // and weight
    };
    struct Leg2 {
        UnitPos pos;
        int m;       // candidate aa, cc: target token
        double cw;   // path weight (exact fp32 x fp32 product)
    };
    // past the end the last item is read again (a valid address), never used
    auto fetch1 = [&](int u) {
        Leg1 l;
        l.pos = unit_pos(a.f.sp, sc.x, u < sc.end ? u : sc.end - 1);
        l.j = a.idx1[(size_t)l.pos.unit * S + aa];
        l.x = a.w1[(size_t)l.pos.unit * S + aa];
        return l;
    };
    auto fetch2 = [&](const Leg1& l) {
        Leg2 t;
        t.pos = l.pos;
        const int u2 = l.pos.kvrow0 + l.j * hkv;   // unit (b, j, h)
        t.m = a.idx2[(size_t)u2 * S + cc];
        const float y = a.w2[(size_t)u2 * S + cc];
        t.cw = (double)l.x * (double)y;
        return t;
    };

    Leg1 l1 = fetch1(sc.q + sc.step);
    Leg2 cur = fetch2(fetch1(sc.q));
    for (int u = sc.q; u < sc.end; u += sc.step) {
        const Leg1 l2 = fetch1(u + 2 * sc.step);
        const Leg2 nxt = fetch2(l1);
        // SER: merge and rank the row's 16 candidates
        float key;
        bool cand;
        int rank;
        team16_merge_rank(r, cur.m, cur.cw, true, key, cand, rank);
        const bool kept = cand && rank < S;
        int jt[S];
        float wt[S];
#pragma unroll
        for (int t = 0; t < S; ++t) {
            const uint64_t mk = __ballot(kept && rank == t);
            const uint32_t seg = (uint32_t)(mk >> rbase) & 0xFFFFu;
            const int src = rbase + (seg ? __ffs(seg) - 1 : 0);
            const int mt = __shfl(cur.m, src, kWave);
            const float kt = __shfl(key, src, kWave);
            jt[t] = seg ? mt : 0;
            wt[t] = seg ? kt : 0.0f;
        }
        if (r == 0)
            *reinterpret_cast<int4*>(a.idx_out + (size_t)cur.pos.unit * S) =
                make_int4(jt[0], jt[1], jt[2], jt[3]);
        if (r == 1)
            *reinterpret_cast<float4*>(a.w_out + (size_t)cur.pos.unit * S) =
                make_float4(wt[0], wt[1], wt[2], wt[3]);
        if (a.paths) {
            // path r's slot of A' (15: none), four bits per path, gathered
            // from the row's lanes bit plane by bit plane
            uint32_t sl = 15;
#pragma unroll
            for (int t = 0; t < S; ++t) sl = cur.cw > 0.0 && wt[t] > 0.0f && jt[t] == cur.m ? t : sl;
            uint64_t mp = 0;
#pragma unroll
            for (int bit = 0; bit < 4; ++bit) {
                const uint32_t plane = (uint32_t)(__ballot((sl >> bit) & 1u) >> rbase) & 0xFFFFu;
#pragma unroll
                for (int k = 0; k < 16; ++k) mp |= (uint64_t)((plane >> k) & 1u) << (4 * k + bit);
            }
            if (r == 2) a.paths[cur.pos.unit] = mp;
        }

        // SEA on the kept slots (as sea_fwd_row_kernel, 256-byte rows)
        bool live[S];
        uint4 kr[S], vr[S];
#pragma unroll
        for (int t = 0; t < S; ++t) {
            live[t] = wt[t] > 0.0f;
            const uint32_t off =
                (uint32_t)(cur.pos.kvrow0 + (live[t] ? jt[t] : 0) * hkv) * ROW + r * 16;
            kr[t] = *reinterpret_cast<const uint4*>(a.f.k + off);
            vr[t] = *reinterpret_cast<const uint4*>(a.f.v + off);
        }
        const uint32_t qoff =
            (uint32_t)(cur.pos.bi * a.f.hq + (cur.pos.unit - cur.pos.bi * hkv) * G) * ROW + r * 16;
        A lw[S];
#pragma unroll
        for (int t = 0; t < S; ++t) lw[t] = live[t] ? fast_log2((A)wt[t]) : NEG;
        constexpr bool st_one = (G + 2) * S <= 16;
        float st_val = 0.0f;
        if (a.f.stats) {
            const int te = r - G * S;
            float ev = 0.0f;
#pragma unroll
            for (int t = 0; t < S; ++t) {
                ev = te == t ? __int_as_float(jt[t]) : ev;
                ev = te == S + t ? wt[t] : ev;
            }
            if constexpr (st_one) {
                st_val = ev;
            } else if (r < S) {
                float* e = a.f.stats + ((size_t)cur.pos.prow * (G + 2) + G) * S;
                float jv = 0.0f, wv = 0.0f;
#pragma unroll
                for (int t = 0; t < S; ++t) {
                    jv = r == t ? __int_as_float(jt[t]) : jv;
                    wv = r == t ? wt[t] : wv;
                }
                __builtin_nontemporal_store(jv, e + r);
                __builtin_nontemporal_store(wv, e + S + r);
            }
        }
#pragma unroll
        for (int g0 = 0; g0 < G; g0 += GC) {
            uint4 qr[GC];
#pragma unroll
            for (int g = 0; g < GC; ++g) qr[g] = load_nt16(a.f.q + qoff + (g0 + g) * ROW);
#pragma unroll
            for (int g = 0; g < GC; ++g) {
                A l[S], sd[S], M = NEG;
#pragma unroll
                for (int t = 0; t < S; ++t) {
                    sd[t] = row_sum16(dot16<V, A>(qr[g], kr[t])) * c;
                    l[t] = live[t] ? sd[t] + lw[t] : NEG;
                    M = l[t] > M ? l[t] : M;
                }
                A p[S], Z = 0;
#pragma unroll
                for (int t = 0; t < S; ++t) {
                    p[t] = live[t] ? fast_exp2(l[t] - M) : (A)0;
                    Z += p[t];
                }
                const A inv = Z > (A)0 ? fast_rcp(Z) : (A)0;
                if (a.f.stats) {
                    const int t0 = st_one ? r - (g0 + g) * S : r;
                    A mine = sd[0];
                    bool ml = live[0];
#pragma unroll
                    for (int t = 1; t < S; ++t) {
                        mine = t0 == t ? sd[t] : mine;
                        ml = t0 == t ? live[t] : ml;
                    }
                    if (t0 >= 0 && t0 < S) st_val = ml ? (float)(fast_exp2(mine - M) * inv) : 0.0f;
                    if (!st_one && t0 >= 0 && t0 < S)
                        __builtin_nontemporal_store(
                            st_val, a.f.stats + ((size_t)cur.pos.prow * (G + 2) + g0 + g) * S + t0);
                }
                A o[V];
#pragma unroll
                for (int e = 0; e < V; ++e) o[e] = 0;
#pragma unroll
                for (int t = 0; t < S; ++t) {
                    A vf[V];
                    unpack16<A, V>(vr[t], vf);
                    const A pt = p[t] * inv;
#pragma unroll
                    for (int e = 0; e < V; ++e) o[e] += pt * vf[e];
                }
                store_u32x4_nt(a.f.o + qoff + (g0 + g) * ROW, pack_bf16x2(o[0], o[1]),
                               pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                               pack_bf16x2(o[6], o[7]));
            }
        }
        if (st_one && a.f.stats && r < (G + 2) * S)
            __builtin_nontemporal_store(st_val, a.f.stats + (size_t)cur.pos.prow * (G + 2) * S + r);
        cur = nxt;
        l1 = l2;
    }
}

template <int G>
hipError_t run_ser_sea(const SerSeaFwd& a, hipStream_t st) {
    const void* fn = reinterpret_cast<const void*>(&ser_sea_fwd_row_kernel<G>);
    const int nwg = persistent_grid(fn, a.f.U, kBlock / 16);
    hipLaunchKernelGGL((ser_sea_fwd_row_kernel<G>), dim3(nwg), dim3(kBlock), 0, st, a);
    return hipGetLastError();
}

}  // namespace

bool sea_row_group(int G) { return G == 1 || G == 2 || G == 4 || G == 8 || G == 16; }

bool sea_fast_shape(int B, int n, int hq, int hkv, int d, bool bf16, int s) {
    const long long es = bf16 ? 2 : 4;
    const long long qbytes = (long long)B * n * hq * d * es;
    return d * es == 256 && s <= 4 && qbytes < (1ll << 32);
}

// the forward's row kernel takes 128-, 256- and 512-byte rows: its R, or -1
static int sea_fwd_row_pieces(int B, int n, int hq, int hkv, int d, bool bf16, int s) {
    const long long es = bf16 ? 2 : 4;
    const long long qbytes = (long long)B * n * hq * d * es;
    if (s > 4 || qbytes >= (1ll << 32)) return -1;
    return d * es == 128 ? 0 : d * es == 256 ? 1 : d * es == 512 ? 2 : -1;
}

hipError_t launch_sea_forward(int B, int n, int hq, int hkv, int d, bool bf16, float scale,
                              const void* q, const void* k, const void* v,
                              const int32_t* idx, const float* w, int s, void* o,
                              float* stats, hipStream_t st) {
    SeaFwdArgs a;
    a.q = q; a.k = k; a.v = v; a.idx = idx; a.w = w; a.o = o; a.stats = stats;
    a.n = n; a.hq = hq; a.hkv = hkv; a.d = d; a.s = s;
    a.U = B * n * hkv;
    a.scale = scale;
    a.ts = sea_team(d, bf16 ? 2 : 4, s);
    const int G = hq / hkv;
    if (const int R = sea_fwd_row_pieces(B, n, hq, hkv, d, bf16, s); R >= 0 && sea_row_group(G)) {
        SeaFwdFast f;
        f.q = static_cast<const char*>(q); f.k = static_cast<const char*>(k);
        f.v = static_cast<const char*>(v); f.idx = idx; f.w = w; f.o = static_cast<char*>(o);
        f.stats = stats;
        f.n = n; f.hq = hq; f.hkv = hkv; f.s = s; f.U = a.U; f.scale = scale;
        make_seg_plan(f.sp, B, n, hkv);
        f.vec = s == 4 && (((uintptr_t)idx | (uintptr_t)w) & 15) == 0;
        if (R == 0) return bf16 ? fast_g<bf16_t, 0>(f, G, st) : fast_g<float, 0>(f, G, st);
        if (R == 2) return bf16 ? fast_g<bf16_t, 2>(f, G, st) : fast_g<float, 2>(f, G, st);
        return bf16 ? fast_g<bf16_t, 1>(f, G, st) : fast_g<float, 1>(f, G, st);
    }
    return bf16 ? dispatch_g<bf16_t>(a, G, st) : dispatch_g<float>(a, G, st);
}

}  // namespace gm

namespace gm {

bool ser_sea_fused_shape(int B, int n, int hq, int hkv, int d, bool bf16, int s1, int s2, int s3,
                         const void* idx1, const void* w1, const void* idx2, const void* w2,
                         const void* idx_out, const void* w_out) {
    const int G = hkv > 0 ? hq / hkv : 0;
    return bf16 && d == 128 && s1 == 4 && s2 == 4 && s3 == 4 && sea_row_group(G) &&
           (long long)B * n * hq * d * 2 < (1ll << 32) &&
           (((uintptr_t)idx1 | (uintptr_t)w1 | (uintptr_t)idx2 | (uintptr_t)w2 |
             (uintptr_t)idx_out | (uintptr_t)w_out) & 15) == 0;
}

hipError_t launch_ser_sea_forward(int B, int n, int hq, int hkv, int d, bool bf16, float scale,
                                  const int32_t* idx1, const float* w1, int s2,
                                  const int32_t* idx2, const float* w2, int s3, int s1,
                                  const void* q, const void* k, const void* v,
                                  int32_t* idx_out, float* w_out, void* o, float* stats,
                                  uint64_t* paths, hipStream_t st) {
    if (!ser_sea_fused_shape(B, n, hq, hkv, d, bf16, s1, s2, s3, idx1, w1, idx2, w2, idx_out,
                             w_out)) {
        // other shapes: the two stages one after the other
        const hipError_t e = launch_ser_forward(B, n, hkv, idx1, w1, s2, idx2, w2, s3, idx_out,
                                                w_out, s1, paths, st);
        if (e != hipSuccess) return e;
        return launch_sea_forward(B, n, hq, hkv, d, bf16, scale, q, k, v, idx_out, w_out, s1, o,
                                  stats, st);
    }
    SerSeaFwd a;
    a.f.q = static_cast<const char*>(q); a.f.k = static_cast<const char*>(k);
    a.f.v = static_cast<const char*>(v); a.f.idx = idx_out; a.f.w = w_out;
    a.f.o = static_cast<char*>(o);
    a.f.stats = stats;
    a.f.n = n; a.f.hq = hq; a.f.hkv = hkv; a.f.s = 4; a.f.U = B * n * hkv; a.f.scale = scale;
    make_seg_plan(a.f.sp, B, n, hkv);
    a.f.vec = 1;
    a.idx1 = idx1; a.w1 = w1; a.idx2 = idx2; a.w2 = w2;
    a.idx_out = idx_out; a.w_out = w_out;
    a.paths = paths;
    switch (hq / hkv) {
        case 1: return run_ser_sea<1>(a, st);
        case 2: return run_ser_sea<2>(a, st);
        case 4: return run_ser_sea<4>(a, st);
        case 8: return run_ser_sea<8>(a, st);
        case 16: return run_ser_sea<16>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gm
