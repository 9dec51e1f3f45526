// Sparse edge attention, backward, for gfx950.
//
// Chain rule of the forward with the indices held fixed (rit.work "Graph
// Machine" article: indices get no gradient, learning goes through the soft
// edge weights).  Per unit and query head, over the live slots t:
//   p_t  = softmax(scale q.k_t + ln w_t)      (recomputed, log2 domain)
//   g_t  = dout . v_t,  gbar = sum_t p_t g_t,  dl_t = p_t (g_t - gbar)
//   (g_t - gbar is formed as sum_{u != t} p_u (g_t - g_u), free of the
//   cancellation of the plain difference when p_t is close to 1)
//   dq   = scale sum_t dl_t k_t
//   dk[idx_t] += scale dl_t q,  dv[idx_t] += p_t dout   (over the group's heads)
//   dw_t = sum_heads dl_t / w_t = sum_heads exp2(ls_t - M) / Z (g_t - gbar)
// The last form never divides by w, so it stays finite for tiny weights.
//
// The dk/dv scatter is done as a sort by target instead of float atomics
// (the L2 retires roughly one atomic lane per channel per clock, which made
// 1024 atomic lanes per unit the bottleneck):
//   1. source pass, one team per unit (as the forward): dq and dw in
//      registers; per (slot, head) the pair (scale*dl, p) goes to a
//      coefficient array; the in-degree of each target row is counted.
//   2. exclusive scan of the in-degrees -> row offsets (two small kernels).
//   3. fill: every live edge id (unit * s + slot) is placed in its target
//      row's segment of the reverse edge list.
//   4. target pass, one team per K/V row: walks the row's incoming edges,
//      gathers the source's q and dout rows and sums
//      dk = sum coef.a * q, dv = sum coef.p * dout, then writes the row once
//      (rows without incoming edges get zeros), so no zero-fill is needed.
// Within a segment the edges are put in ascending id order after the fill,
// so each dk/dv row is summed in the same order on every run (bitwise
// deterministic).
#include <type_traits>

#include "gm_common.h"
#include "gm_internal.h"
#include "gm_wave.h"

#include <math.h>

namespace gm {

namespace {

constexpr int kScanPerBlock = 4096;  // counts scanned by one 1024-thread block

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Workspace {
    float2* coef;   // [U * s * G]  (scale * dl, p) per edge and head
    int* cnt;       // [U]  in-degree, then the fill cursor (long sequences)
    int* off;       // [U + 1]  segment offsets (long sequences)
    int* bsum;      // [ceil(U / kScanPerBlock)]
    int* list;      // [U * s]  edge ids grouped by target row
    int* beg;       // [U]  per K/V row in pair-major order: first list slot
    int* len;       // [U]  ... and number of incoming edges
    int* head;      // [U * 4]  per row in pair-major order: its first 4 edge ids, -1 padded
    int* tgt;       // [U * s]  per source row in pair-major order: target of each slot, -1 dead
    int2* stage;    // [U * s]  (edge, target) staging of the partitioned index (n > 4096)
};

struct WsLayout {
    size_t coef, cnt, off, bsum, list, beg, len, head, tgt, stage, total;
};

WsLayout ws_layout(long long U, int s, int G, int n) {
    WsLayout l;
    l.coef = 0;
    l.cnt = l.coef + align256((size_t)U * s * G * sizeof(float2));
    l.off = l.cnt + align256((size_t)U * sizeof(int));
    l.bsum = l.off + align256((size_t)(U + 1) * sizeof(int));
    l.list = l.bsum + align256((size_t)((U + kScanPerBlock - 1) / kScanPerBlock) * sizeof(int));
    // eight spare entries: the target pass reads the next four ids of a row
    // at once, up to seven past the row's end
    l.beg = l.list + align256(((size_t)U * s + 8) * sizeof(int));
    l.len = l.beg + align256((size_t)U * sizeof(int));
    l.head = l.len + align256((size_t)U * sizeof(int));
    l.tgt = l.head + align256((size_t)U * 4 * sizeof(int));
    l.stage = l.tgt + align256((size_t)U * s * sizeof(int));
    const bool partitioned = !edge_index_one_pass(n) && edge_index_supported(n, s);
    l.total = l.stage + (partitioned ? align256((size_t)U * s * sizeof(int2)) : 0);
    return l;
}

struct SeaBwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const int32_t* idx;
    const float* w;
    float* dq;
    float* dk;
    float* dv;
    float* dw;
    Workspace ws;
    int n, hq, hkv, d, s, U;
    float scale;
    TeamShape ts;   // source pass
    TeamShape tt;   // target pass (P = edges walked side by side)
};

// ------------------------------------------------------------ source pass
template <typename T, int GT>
__global__ __launch_bounds__(kBlock) void sea_bwd_src_kernel(SeaBwdArgs a) {
    // GT > 0: the group size as a constant; 0: any group size, from the heads
    const int G = GT > 0 ? GT : a.hq / a.hkv;
    using A = typename io<T>::acc;
    constexpr int V = io<T>::V;
    constexpr int LOG2V = ilog2(V);
    const int R = a.ts.R, team = a.ts.team, P = a.ts.P;
    const int lane = threadIdx.x & (kWave - 1);
    const int tl = lane & (team - 1);
    const int r = tl & (R - 1);
    const int sl = tl >> a.ts.log2R;
    const long long gunit = ((long long)blockIdx.x * kBlock + threadIdx.x) / team;
    if (gunit >= a.U) return;  // whole team leaves together
    const int unit = (int)gunit;
    const int h = unit % a.hkv;
    const int bi = unit / a.hkv;
    const int b = bi / a.n;
    const size_t d = (size_t)a.d;
    const size_t qoff = ((size_t)bi * a.hq + (size_t)h * G) * d + r * V;
    const T* qp = static_cast<const T*>(a.q) + qoff;
    const T* dop = static_cast<const T*>(a.dout) + qoff;
    float* dqp = a.dq + qoff;
    const T* kp = static_cast<const T*>(a.k) + r * V;
    const T* vp = static_cast<const T*>(a.v) + r * V;
    const size_t kv0 = (size_t)b * a.n * a.hkv + h;
    const int32_t* ip = a.idx + (size_t)unit * a.s;
    const float* wp = a.w + (size_t)unit * a.s;
    float2* cp = a.ws.coef + (size_t)unit * a.s * G;
    const A c = (A)a.scale * (A)1.4426950408889634;
    const A sc = (A)a.scale;
    const A NEG = -INFINITY;
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
                const long long row = (long long)(kv0 + (size_t)ip[t] * a.hkv);
                load16(kp + row * d, kr);
                load16(vp + row * d, vr);
                if (r == 0) atomicAdd(a.ws.cnt + row, 1);
            }
        }
        A dws = 0;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            A qg[V], dg[V];
            load16(qp + g * d, qg);
            load16(dop + g * d, dg);
            A sd = 0, gd = 0;
#pragma unroll
            for (int e = 0; e < V; ++e) { sd += qg[e] * kr[e]; gd += dg[e] * vr[e]; }
            sd = sum_bits(sd, 1, R);
            gd = sum_bits(gd, 1, R);
            const A ls = sd * c;
            const A l = live ? ls + lw : NEG;
            const A M = max_bits(l, R, team);
            const A ex = live ? aexp2(l - M) : (A)0;
            const A Z = sum_bits(ex, R, team);
            const A invZ = Z > 0 ? (A)1 / Z : (A)0;
            const A p = ex * invZ;
            // g_t - gbar as the sum over the other slots u of p_u (g_t - g_u)
            // (no cancellation when one slot holds nearly all the mass)
            A cg = 0;
            const int lbase = lane - tl;
#pragma unroll 1
            for (int u = 0; u < P; ++u) {
                const A pu = __shfl(p, lbase + u * R, kWave);
                const A gu = __shfl(gd, lbase + u * R, kWave);
                if (u != t) cg += pu * (gd - gu);
            }
            const A dls = p * cg * sc;
            A dqv[V];
#pragma unroll
            for (int e = 0; e < V; ++e) dqv[e] = dls * kr[e];
            int len;
            const int off = reduce_scatter(dqv, tl, R, team, len);
            if (storer) store_len(dqp + g * d + off, dqv, len);
            if (live && r == 0) cp[t * G + g] = make_float2((float)dls, (float)p);
            if (live) dws += aexp2(ls - M) * invZ * cg;
        }
        if (r == 0 && t < a.s) a.dw[(size_t)unit * a.s + t] = (float)dws;
        return;
    }

    // s > P: per head, pass 1 over the chunks finds the running max M, the
    // sum Z and sum e*g; pass 2 recomputes p and dl.  dw is summed over the
    // heads with atomics (the caller zero-filled it).
#pragma unroll 1
    for (int g = 0; g < G; ++g) {
        A qg[V], dg[V];
        load16(qp + g * d, qg);
        load16(dop + g * d, dg);
        A M = NEG, Z = 0, Sg = 0;
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
            A sd = 0, gd = 0;
#pragma unroll
            for (int e = 0; e < V; ++e) { sd += qg[e] * kr[e]; gd += dg[e] * vr[e]; }
            sd = sum_bits(sd, 1, R);
            gd = sum_bits(gd, 1, R);
            const A l = live ? sd * c + lw : NEG;
            const A Mn = amax(M, max_bits(l, R, team));
            if (Mn == NEG) continue;  // uniform over the team: nothing live yet
            const A alpha = aexp2(M - Mn);
            const A ex = live ? aexp2(l - Mn) : (A)0;
            Z = Z * alpha + sum_bits(ex, R, team);
            Sg = Sg * alpha + sum_bits(ex * gd, R, team);
            M = Mn;
        }
        const A invZ = Z > 0 ? (A)1 / Z : (A)0;
        A dqv[V];
#pragma unroll
        for (int e = 0; e < V; ++e) dqv[e] = 0;
#pragma unroll 1
        for (int ch = 0; ch < a.ts.nchunk; ++ch) {
            const int t = ch * P + sl;
            if (t >= a.s) continue;
            const float wt = wp[t];
            if (!(wt > 0.0f)) continue;
            const A lw = alog2((A)wt);
            const long long row = (long long)(kv0 + (size_t)ip[t] * a.hkv);
            A kr[V], vr[V];
            load16(kp + row * d, kr);
            load16(vp + row * d, vr);
            A sd = 0, gd = 0;
#pragma unroll
            for (int e = 0; e < V; ++e) { sd += qg[e] * kr[e]; gd += dg[e] * vr[e]; }
            // the row lanes of one slot are all here (same t): reduce them
            sd = sum_bits(sd, 1, R);
            gd = sum_bits(gd, 1, R);
            const A ls = sd * c;
            const A p = aexp2(ls + lw - M) * invZ;
            // g_t - gbar from the unnormalised sums: exactly 0 for a single
            // live slot (Z and Sg are then one term each)
            const A cg = (gd * Z - Sg) * invZ;
            const A dls = p * cg * sc;
#pragma unroll
            for (int e = 0; e < V; ++e) dqv[e] += dls * kr[e];
            if (r == 0) {
                cp[t * G + g] = make_float2((float)dls, (float)p);
                unsafeAtomicAdd(a.dw + (size_t)unit * a.s + t,
                                (float)(aexp2(ls - M) * invZ * cg));
                if (g == 0) atomicAdd(a.ws.cnt + row, 1);
            }
        }
        int len;
        const int off = reduce_scatter(dqv, tl, R, team, len);
        if (storer) store_len(dqp + g * d + off, dqv, len);
    }
}

// --------------------------------------------------------------- index build
// Exclusive scan of cnt[0 .. U) into off, 4096 counts per block.
__global__ __launch_bounds__(1024) void scan_local_kernel(const int* cnt, int* off, int* bsum,
                                                          int U) {
    __shared__ int part[1024 / kWave];
    const int base = blockIdx.x * kScanPerBlock + threadIdx.x * 4;
    int v[4], s = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[e] = base + e < U ? cnt[base + e] : 0;
        s += v[e];
    }
    // inclusive scan of the per-thread sums across the wave
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    int inc = s;
    for (int m = 1; m < kWave; m <<= 1) {
        const int o = __shfl_up(inc, m, kWave);
        if (lane >= m) inc += o;
    }
    if (lane == kWave - 1) part[wave] = inc;
    __syncthreads();
    int wbase = 0;
    for (int k = 0; k < wave; ++k) wbase += part[k];
    int run = wbase + inc - s;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (base + e < U) off[base + e] = run;
        run += v[e];
    }
    if (threadIdx.x == 1023) bsum[blockIdx.x] = wbase + inc;
}

// Add the preceding blocks' totals; copy the offsets into the fill cursor.
__global__ __launch_bounds__(1024) void scan_add_kernel(int* off, int* cursor, const int* bsum,
                                                        int U) {
    __shared__ int base_s;
    if (threadIdx.x < kWave) {
        int sum = 0;
        for (int k = threadIdx.x; k < (int)blockIdx.x; k += kWave) sum += bsum[k];
        for (int m = 32; m > 0; m >>= 1) sum += __shfl_xor(sum, m, kWave);
        if (threadIdx.x == 0) base_s = sum;
    }
    __syncthreads();
    const int base = base_s;
    const int first = blockIdx.x * kScanPerBlock;
    for (int e = threadIdx.x; e < kScanPerBlock; e += 1024) {
        const int x = first + e;
        if (x < U) {
            const int o = off[x] + base;
            off[x] = o;
            cursor[x] = o;
        }
    }
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) off[U] = base + bsum[blockIdx.x];
}

// Place every live edge id (unit * s + slot) in its target row's segment.
__global__ __launch_bounds__(kBlock) void edge_fill_kernel(const int32_t* idx, const float* w,
                                                           int n, int hkv, int s, long long E,
                                                           int* cursor, int* list) {
    for (long long e = (long long)blockIdx.x * kBlock + threadIdx.x; e < E;
         e += (long long)gridDim.x * kBlock) {
        if (!(w[e] > 0.0f)) continue;
        const int unit = (int)(e / s);
        const int h = unit % hkv;
        const int b = unit / hkv / n;
        const int row = (b * n + idx[e]) * hkv + h;
        const int pos = atomicAdd(cursor + row, 1);
        list[pos] = (int)e;
    }
}

// The fill's atomics leave each row's segment in an order that varies
// between runs: copy every live edge to its row's start plus the number of
// the segment's edges with a smaller id, so `out` lists each row's edges by
// ascending id (the same on every run).
__global__ __launch_bounds__(kBlock) void edge_order_kernel(const int32_t* idx, const float* w,
                                                            int n, int hkv, int s, long long E,
                                                            const int* off, const int* list,
                                                            int* out) {
    for (long long e = (long long)blockIdx.x * kBlock + threadIdx.x; e < E;
         e += (long long)gridDim.x * kBlock) {
        if (!(w[e] > 0.0f)) continue;
        const int unit = (int)(e / s);
        const int h = unit % hkv;
        const int b = unit / hkv / n;
        const int row = (b * n + idx[e]) * hkv + h;
        const int b0 = off[row], b1 = off[row + 1];
        int rk = 0;
        for (int p = b0; p < b1; ++p) rk += list[p] < (int)e;
        out[b0 + rk] = (int)e;
    }
}

// ------------------------------------------------------------ target pass
// One team of R * P lanes per K/V row (b, j, h): P incoming edges side by
// side, R lanes per 16-byte piece of a d-row, G query heads per edge.
template <typename T, int GT>
__global__ __launch_bounds__(kBlock) void sea_bwd_dst_kernel(SeaBwdArgs a) {
    // GT > 0: the group size as a constant; 0: any group size, from the heads
    const int G = GT > 0 ? GT : a.hq / a.hkv;
    using A = typename io<T>::acc;
    constexpr int V = io<T>::V;
    constexpr int LOG2V = ilog2(V);
    const int R = a.tt.R, team = a.tt.team, P = a.tt.P;
    const int lane = threadIdx.x & (kWave - 1);
    const int tl = lane & (team - 1);
    const int r = tl & (R - 1);
    const int sl = tl >> a.tt.log2R;
    const long long grow = ((long long)blockIdx.x * kBlock + threadIdx.x) / team;
    if (grow >= a.U) return;
    const int row = (int)grow;
    const int h = row % a.hkv;
    const size_t d = (size_t)a.d;
    const int beg = a.ws.off[row], end = a.ws.off[row + 1];
    const T* qb = static_cast<const T*>(a.q) + (size_t)h * G * d + r * V;
    const T* db = static_cast<const T*>(a.dout) + (size_t)h * G * d + r * V;
    A ak[V], av[V];
#pragma unroll
    for (int e = 0; e < V; ++e) { ak[e] = 0; av[e] = 0; }
#pragma unroll 1
    for (int e0 = beg; e0 < end; e0 += P) {
        const int ei = e0 + sl;
        if (ei < end) {
            const int eid = a.ws.list[ei];
            const int unit = eid / a.s;
            const size_t src = (size_t)(unit / a.hkv) * a.hq * d;   // (b*n + i) * hq * d
            const float2* cf = a.ws.coef + (size_t)eid * G;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float2 ap = cf[g];
                A qg[V], dg[V];
                load16(qb + src + g * d, qg);
                load16(db + src + g * d, dg);
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    ak[e] += (A)ap.x * qg[e];
                    av[e] += (A)ap.y * dg[e];
                }
            }
        }
    }
    int len;
    const int off = reduce_scatter(ak, tl, R, team, len);
    reduce_scatter(av, tl, R, team, len);
    if ((sl >> LOG2V) == 0) {
        float* dkp = a.dk + (size_t)row * d + r * V + off;
        float* dvp = a.dv + (size_t)row * d + r * V + off;
        store_len(dkp, ak, len);
        store_len(dvp, av, len);
    }
}



// ----------------------------------------------------------------- fast path
// Same geometry as the forward's fast path: one d-row (256 bytes; the wide
// source kernel and the target row kernel also take 128 and 512) per 16-lane
// row, one unit (source pass) or P incoming edges (target pass) per row,
// XCD-aware schedules in pair-major order.
struct SeaBwdFast {
    const char* q;
    const char* k;
    const char* v;
    const char* dout;
    const float* stats;   // [B][hkv][n][G + 2][s] p / w, idx, w from the forward, or null
    const int32_t* idx;
    const float* w;
    char* dq;
    char* dk;
    char* dv;
    float* dw;
    Workspace ws;
    int n, hq, hkv, s, U;
    float scale;
    FastDiv fd_s, fd_hkv;
    SegPlan sp;
    int global_index;   // 1: in-degrees counted here, offsets from the global scan
    int write_tgt;      // 1: the source pass writes ws.tgt for the single-pass index
    int vec;            // s == 4 and 16-byte aligned edge rows: one load per row
};

struct Pos {
    int unit, bi, kvrow0, prow;   // prow = pair * n + i (pair-major row)
};

// The forward's saved statistics of a unit (pair-major row prow): E G + 2
// rows of s 4-byte words, p / w per head and slot in the accumulation type A
// (E = sizeof(A) / 4: fp32 for bf16 inputs, fp64 for fp32 inputs), then the
// unit's edge indices and weights.
template <typename A>
__device__ __forceinline__ const float* saved_edge_copy(const float* stats, size_t prow, int G,
                                                        int s) {
    constexpr int E = sizeof(A) / 4;
    return stats + (prow * (E * G + 2) + E * G) * s;
}
template <typename A, int S, bool VEC>
__device__ __forceinline__ void load_saved_pw(const float* stats, size_t prow, int G, int s, int g,
                                              A (&st)[S]) {
    if constexpr (sizeof(A) == 4) {
        const float* sp = stats + (prow * (G + 2) + g) * s;
        if constexpr (VEC) {
            const float4 s4 = *reinterpret_cast<const float4*>(sp);
            st[0] = s4.x; st[1] = s4.y; st[2] = s4.z; st[3] = s4.w;
        } else {
#pragma unroll
            for (int t = 0; t < S; ++t) st[t] = sp[t < s ? t : s - 1];
        }
    } else {
        const double* sp = reinterpret_cast<const double*>(stats) + (prow * (G + 1) + g) * s;
        if constexpr (VEC) {
            const double2 lo = *reinterpret_cast<const double2*>(sp);
            const double2 hi = *reinterpret_cast<const double2*>(sp + 2);
            st[0] = lo.x; st[1] = lo.y; st[2] = hi.x; st[3] = hi.y;
        } else {
#pragma unroll
            for (int t = 0; t < S; ++t) st[t] = sp[t < s ? t : s - 1];
        }
    }
}

__device__ __forceinline__ Pos pos_of(const SegPlan& sp, int x, int q) {
    int pair, i;
    sched_item(sp, x, q, pair, i);
    const int b = (int)fdiv((uint32_t)pair, sp.fd_hkv);
    const int h = pair - b * sp.hkv;
    Pos p;
    p.bi = b * sp.n + i;
    p.unit = p.bi * sp.hkv + h;
    p.kvrow0 = b * sp.n * sp.hkv + h;
    p.prow = pair * sp.n + i;
    return p;
}

// g_t - gbar with gbar = sum_u p_u g_u, written as sum over u != t of
// p_u (g_t - g_u): the same value when the p sum to 1, without the
// cancellation of the plain difference when one slot holds nearly all the
// mass (exactly 0 when a single slot is live).  That difference times p / w
// is dw, and p / w is large for small w.
template <int S, typename A>
__device__ __forceinline__ void centered_pairwise(const A (&p)[S], const A (&g)[S], A (&d)[S]) {
#pragma unroll
    for (int t = 0; t < S; ++t) {
        A x = 0;
#pragma unroll
        for (int u = 0; u < S; ++u)
            if (u != t) x += p[u] * (g[t] - g[u]);
        d[t] = x;
    }
}

template <int L, typename A>
__device__ __forceinline__ void store_f32(char* p, const A* x) {
    store_n<L>(reinterpret_cast<float*>(p), x);
}

// 16-lane sum of the product of two rows held as R parts per lane
template <int V, typename A, int R>
__device__ __forceinline__ A row_dot(const uint4 (&x)[R], const uint4 (&y)[R]) {
    if constexpr (R == 1) {
        return row_sum16(dot16<V, A>(x[0], y[0]));
    } else {
        return row_sum16(dot16<V, A>(x[0], y[0]) + dot16<V, A>(x[1], y[1]));
    }
}

// Source pass with one unit per 16-lane row, four units per wavefront: lane
// r holds bytes [16r, 16r + 16) of the unit's G query and upstream-gradient
// rows and of the K and V rows of its S edge slots (registers).  Scores and
// the dout.v products are 16-lane DPP sums; the softmax, dl, dq and dw are
// lane-local.  Lane t < S writes slot t's per-edge coefficients and dw.
// GLOBAL: also count the in-degree of every K/V row (global index path).
// SAVED: the softmax comes from the forward's p / w statistics (p = stat * w),
// so q is not read here and no scores are formed.
// BLK (G = 2, s = 4, segments of a multiple of 4 tokens): the four units of
// a wavefront are consecutive tokens of one pair, so their saved records
// (p / w of both heads, then the edge copy: 16 words each) are one 256-byte
// block.  The edge copies (index and weight words) come one unit ahead
// through the scalar data cache, so the wait for them at the top of a unit
// does not also drain the previous unit's vector stores; the p / w words
// are read with one word per lane and spread over each 16-lane row by row
// broadcasts (two L2 requests per wavefront instead of eight).
template <typename T, int G, int S, bool VEC, bool GLOBAL, bool SAVED, bool BLK>
__global__ __launch_bounds__(kBlock) void sea_bwd_src_row_kernel(SeaBwdFast a) {
    using A = typename io<T>::acc;
    constexpr int V = io<T>::V;
    constexpr int ROW = 256;                          // bytes of an input d-row
    constexpr int FROW = ROW * 4 / (int)sizeof(T);    // bytes of an fp32 gradient row
    constexpr int GC = G < 2 ? G : 2;                 // query heads held at once
    static_assert(!BLK || (SAVED && VEC && G == 2 && S == 4), "16-word records");
    const int r = threadIdx.x & 15;
    const A c = (A)a.scale * (A)1.4426950408889634;
    const A sc = (A)a.scale;
    const A NEG = -INFINITY;
    const Sched sch = xcd_sched(a.sp, 16);
    if (sch.q >= sch.end) return;

    struct Item {
        Pos pos;
        int j[S];
        float wt[S];
        size_t rec;      // BLK: word offset of the wavefront's record block
        float sr[32];    // BLK: the four units' index and weight words (scalar)
    };
    auto fetch = [&](int u) {
        Item it;
        it.pos = pos_of(a.sp, sch.x, u < sch.end ? u : sch.end - 1);
        if constexpr (BLK) {
            // row 0 holds the wavefront's first item; past the end, the
            // last block is read again (never used)
            int ub = __builtin_amdgcn_readfirstlane(u);
            ub = ub < sch.end ? ub : sch.end - 4;
            const Pos p0 = pos_of(a.sp, sch.x, ub);
            it.rec = (size_t)p0.prow * 16;
            typedef const __attribute__((address_space(4))) float cf4;
            cf4* rp = (cf4*)(a.stats + it.rec);
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int w = 0; w < 8; ++w) it.sr[k * 8 + w] = rp[k * 16 + 8 + w];
            return it;
        } else if constexpr (SAVED) {
            // the forward's pair-major copy of the edge row: contiguous for
            // the consecutive tokens of a wavefront, where the interleaved
            // rows of the eight KV heads would bring whole lines to every XCD
            const float* e = saved_edge_copy<A>(a.stats, (size_t)it.pos.prow, G, a.s);
            if constexpr (VEC) {
                const int4 j4 = *reinterpret_cast<const int4*>(e);
                const float4 w4 = *reinterpret_cast<const float4*>(e + 4);
                it.j[0] = j4.x; it.j[1] = j4.y; it.j[2] = j4.z; it.j[3] = j4.w;
                it.wt[0] = w4.x; it.wt[1] = w4.y; it.wt[2] = w4.z; it.wt[3] = w4.w;
            } else {
#pragma unroll
                for (int t = 0; t < S; ++t) {
                    const int tt = t < a.s ? t : a.s - 1;
                    it.j[t] = __float_as_int(e[tt]);
                    const float wv = e[a.s + tt];
                    it.wt[t] = t < a.s ? wv : 0.0f;
                }
            }
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

    Item cur = fetch(sch.q);
    for (int u = sch.q; u < sch.end; u += sch.step) {
        const Item nxt = fetch(u + sch.step);
        float brec = 0.0f;   // BLK: word (lane) of the wavefront's record block
        if constexpr (BLK) {
            const int rw = (threadIdx.x >> 4) & 3;
            // row masks, opaque so that the blend below is not turned into
            // an indexed (scratch) access
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
            brec = a.stats[cur.rec + (threadIdx.x & (kWave - 1))];
        }
        bool live[S];
        int kvrow[S];
        uint4 kr[S], vr[S];
#pragma unroll
        for (int t = 0; t < S; ++t) {
            live[t] = cur.wt[t] > 0.0f;
            kvrow[t] = cur.pos.kvrow0 + (live[t] ? cur.j[t] : 0) * a.hkv;
            const uint32_t off = (uint32_t)kvrow[t] * ROW;
            kr[t] = load_split<V>(a.k + off, r);
            vr[t] = load_split<V>(a.v + off, r);
        }
        const int h = cur.pos.unit - cur.pos.bi * a.hkv;
        const uint32_t qrow = (uint32_t)(cur.pos.bi * a.hq + h * G);
        if constexpr (GLOBAL) {
#pragma unroll
            for (int t = 0; t < S; ++t)
                if (r == t && live[t]) atomicAdd(a.ws.cnt + kvrow[t], 1);
        }
        A lw[S], dws[S];
#pragma unroll
        for (int t = 0; t < S; ++t) {
            lw[t] = live[t] ? fast_log2((A)cur.wt[t]) : NEG;
            dws[t] = 0;
        }
        // coefficients (scale * dl, p) of this lane's slot, one per head
        A my_dl[G], my_p[G];
#pragma unroll
        for (int g0 = 0; g0 < G; g0 += GC) {
            uint4 qr[GC], dr[GC];
            A st[GC][S];
#pragma unroll
            for (int g = 0; g < GC; ++g) {
                if constexpr (BLK) {
                    if (g0 + g == 0) {
                        st[g][0] = row_bcast<0>(brec); st[g][1] = row_bcast<1>(brec);
                        st[g][2] = row_bcast<2>(brec); st[g][3] = row_bcast<3>(brec);
                    } else {
                        st[g][0] = row_bcast<4>(brec); st[g][1] = row_bcast<5>(brec);
                        st[g][2] = row_bcast<6>(brec); st[g][3] = row_bcast<7>(brec);
                    }
                } else if constexpr (SAVED) {
                    load_saved_pw<A, S, VEC>(a.stats, (size_t)cur.pos.prow, G, a.s, g0 + g, st[g]);
                } else {
                    qr[g] = load_split_nt<V>(a.q + (qrow + g0 + g) * ROW, r);
                }
                dr[g] = load_split_nt<V>(a.dout + (qrow + g0 + g) * ROW, r);
            }
#pragma unroll
            for (int g = 0; g < GC; ++g) {
                A gd[S], p[S], pw[S];
                if constexpr (SAVED) {
#pragma unroll
                    for (int t = 0; t < S; ++t) {
                        gd[t] = row_sum16(dot16<V, A>(dr[g], vr[t]));
                        pw[t] = live[t] ? (A)st[g][t] : (A)0;
                        p[t] = pw[t] * (A)cur.wt[t];
                    }
                } else {
                    A ls[S], l[S], M = NEG;
#pragma unroll
                    for (int t = 0; t < S; ++t) {
                        ls[t] = row_sum16(dot16<V, A>(qr[g], kr[t])) * c;
                        gd[t] = row_sum16(dot16<V, A>(dr[g], vr[t]));
                        l[t] = live[t] ? ls[t] + lw[t] : NEG;
                        M = l[t] > M ? l[t] : M;
                    }
                    A ex[S], Z = 0;
#pragma unroll
                    for (int t = 0; t < S; ++t) {
                        ex[t] = live[t] ? fast_exp2(l[t] - M) : (A)0;
                        Z += ex[t];
                    }
                    const A invZ = Z > (A)0 ? fast_rcp(Z) : (A)0;
#pragma unroll
                    for (int t = 0; t < S; ++t) {
                        p[t] = ex[t] * invZ;
                        // dl / w = exp(l - M) / (Z w) = exp(scale * dot - M) / Z
                        pw[t] = live[t] ? fast_exp2(ls[t] - M) * invZ : (A)0;
                    }
                }
                A dg[S], dls[S];
                centered_pairwise<S>(p, gd, dg);
#pragma unroll
                for (int t = 0; t < S; ++t) {
                    dls[t] = p[t] * dg[t] * sc;
                    dws[t] += pw[t] * dg[t];
                }
                A sel_dl = dls[0], sel_p = p[0];
#pragma unroll
                for (int t = 1; t < S; ++t) {
                    sel_dl = r == t ? dls[t] : sel_dl;
                    sel_p = r == t ? p[t] : sel_p;
                }
                my_dl[g0 + g] = sel_dl;
                my_p[g0 + g] = sel_p;
                // dq of this head: sum over the slots of scale * dl * k
                A dq[V];
#pragma unroll
                for (int e = 0; e < V; ++e) dq[e] = 0;
#pragma unroll
                for (int t = 0; t < S; ++t) {
                    A kf[V];
                    unpack16<A, V>(kr[t], kf);
#pragma unroll
                    for (int e = 0; e < V; ++e) dq[e] += dls[t] * kf[e];
                }
                store_split_f32_nt<V>(a.dq + (qrow + g0 + g) * FROW, r, dq);
            }
        }
        // lane t < s: coefficients of slot t (live slots only; the target
        // pass reads live edges only) and its dw
        bool my_live = live[0];
        A my_dw = dws[0];
#pragma unroll
        for (int t = 1; t < S; ++t) {
            my_live = r == t ? live[t] : my_live;
            my_dw = r == t ? dws[t] : my_dw;
        }
        const size_t my_e = (size_t)cur.pos.unit * a.s + r;
        if (r < a.s) {
            if (my_live) {
                float2* cp = a.ws.coef + my_e * G;
#pragma unroll
                for (int g = 0; g < G; ++g) cp[g] = make_float2((float)my_dl[g], (float)my_p[g]);
            }
            a.dw[my_e] = (float)my_dw;
            if (a.write_tgt) {
                int my_j = cur.j[0];
#pragma unroll
                for (int t = 1; t < S; ++t) my_j = r == t ? cur.j[t] : my_j;
                a.ws.tgt[(size_t)cur.pos.prow * a.s + r] = my_live ? my_j : -1;
            }
        }
        cur = nxt;
    }
}

// The source pass for 512-byte rows (R = 2: bf16 d = 256, fp32 d = 128)
// and 128-byte rows (R = 0: bf16 d = 64): as sea_bwd_src_row_kernel, with
// lane r holding the split piece of each of the two 256-byte parts of every
// row it touches, or bytes [8r, 8r + 8) of a 128-byte row in the low half of
// its registers (high half zero).  A separate kernel, so the code of the
// 256-byte kernel stays as it is scheduled best.  Scores and
// the dout.v products are 16-lane DPP sums; the softmax, dl, dq and dw are
// lane-local.  Lane t < S writes slot t's per-edge coefficients and dw.
// GLOBAL: also count the in-degree of every K/V row (global index path).
// SAVED: the softmax comes from the forward's p / w statistics (p = stat * w),
// so q is not read here and no scores are formed.
template <typename T, int G, int S, bool VEC, bool GLOBAL, bool SAVED, int R>
__global__ __launch_bounds__(kBlock) void sea_bwd_src_wide_kernel(SeaBwdFast a) {
    using A = typename io<T>::acc;
    constexpr int V = io<T>::V;
    constexpr int ROW = R == 0 ? 128 : 256 * R;       // bytes of an input d-row
    constexpr int NP = R == 0 ? 1 : R;                // register parts per row
    constexpr int FROW = ROW * 4 / (int)sizeof(T);    // bytes of an fp32 gradient row
    constexpr int FPART = FROW / NP;                  // fp32 bytes of one part
    constexpr int GC = G < 2 ? G : 2;                 // query heads held at once
    const int r = threadIdx.x & 15;
    const A c = (A)a.scale * (A)1.4426950408889634;
    const A sc = (A)a.scale;
    const A NEG = -INFINITY;
    const Sched sch = xcd_sched(a.sp, 16);
    if (sch.q >= sch.end) return;

    struct Item {
        Pos pos;
        int j[S];
        float wt[S];
    };
    auto fetch = [&](int u) {
        Item it;
        it.pos = pos_of(a.sp, sch.x, u < sch.end ? u : sch.end - 1);
        if constexpr (SAVED) {
            // the forward's pair-major copy of the edge row: contiguous for
            // the consecutive tokens of a wavefront, where the interleaved
            // rows of the eight KV heads would bring whole lines to every XCD
            const float* e = saved_edge_copy<A>(a.stats, (size_t)it.pos.prow, G, a.s);
            if constexpr (VEC) {
                const int4 j4 = *reinterpret_cast<const int4*>(e);
                const float4 w4 = *reinterpret_cast<const float4*>(e + 4);
                it.j[0] = j4.x; it.j[1] = j4.y; it.j[2] = j4.z; it.j[3] = j4.w;
                it.wt[0] = w4.x; it.wt[1] = w4.y; it.wt[2] = w4.z; it.wt[3] = w4.w;
            } else {
#pragma unroll
                for (int t = 0; t < S; ++t) {
                    const int tt = t < a.s ? t : a.s - 1;
                    it.j[t] = __float_as_int(e[tt]);
                    const float wv = e[a.s + tt];
                    it.wt[t] = t < a.s ? wv : 0.0f;
                }
            }
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

    Item cur = fetch(sch.q);
    for (int u = sch.q; u < sch.end; u += sch.step) {
        const Item nxt = fetch(u + sch.step);
        bool live[S];
        int kvrow[S];
        uint4 kr[S][NP], vr[S][NP];
#pragma unroll
        for (int t = 0; t < S; ++t) {
            live[t] = cur.wt[t] > 0.0f;
            kvrow[t] = cur.pos.kvrow0 + (live[t] ? cur.j[t] : 0) * a.hkv;
            const uint32_t off = (uint32_t)kvrow[t] * ROW;
#pragma unroll
            for (int k = 0; k < NP; ++k) {
                if constexpr (R == 0) {
                    const uint2 k2 = *reinterpret_cast<const uint2*>(a.k + off + r * 8);
                    const uint2 v2 = *reinterpret_cast<const uint2*>(a.v + off + r * 8);
                    kr[t][k] = make_uint4(k2.x, k2.y, 0u, 0u);
                    vr[t][k] = make_uint4(v2.x, v2.y, 0u, 0u);
                } else {
                    kr[t][k] = load_split<V>(a.k + off + 256 * k, r);
                    vr[t][k] = load_split<V>(a.v + off + 256 * k, r);
                }
            }
        }
        const int h = cur.pos.unit - cur.pos.bi * a.hkv;
        const uint32_t qrow = (uint32_t)(cur.pos.bi * a.hq + h * G);
        if constexpr (GLOBAL) {
#pragma unroll
            for (int t = 0; t < S; ++t)
                if (r == t && live[t]) atomicAdd(a.ws.cnt + kvrow[t], 1);
        }
        A lw[S], dws[S];
#pragma unroll
        for (int t = 0; t < S; ++t) {
            lw[t] = live[t] ? fast_log2((A)cur.wt[t]) : NEG;
            dws[t] = 0;
        }
        // coefficients (scale * dl, p) of this lane's slot, one per head
        A my_dl[G], my_p[G];
#pragma unroll
        for (int g0 = 0; g0 < G; g0 += GC) {
            uint4 qr[GC][NP], dr[GC][NP];
            A st[GC][S];
#pragma unroll
            for (int g = 0; g < GC; ++g) {
                if constexpr (SAVED) {
                    load_saved_pw<A, S, VEC>(a.stats, (size_t)cur.pos.prow, G, a.s, g0 + g, st[g]);
                } else {
#pragma unroll
                    for (int k = 0; k < NP; ++k)
                        qr[g][k] = R == 0 ? load_nt8(a.q + (qrow + g0 + g) * ROW + r * 8)
                                          : load_split_nt<V>(a.q + (qrow + g0 + g) * ROW + 256 * k, r);
                }
#pragma unroll
                for (int k = 0; k < NP; ++k)
                    dr[g][k] = R == 0 ? load_nt8(a.dout + (qrow + g0 + g) * ROW + r * 8)
                                      : load_split_nt<V>(a.dout + (qrow + g0 + g) * ROW + 256 * k, r);
            }
#pragma unroll
            for (int g = 0; g < GC; ++g) {
                A gd[S], p[S], pw[S];
                if constexpr (SAVED) {
#pragma unroll
                    for (int t = 0; t < S; ++t) {
                        gd[t] = row_dot<V, A, NP>(dr[g], vr[t]);
                        pw[t] = live[t] ? (A)st[g][t] : (A)0;
                        p[t] = pw[t] * (A)cur.wt[t];
                    }
                } else {
                    A ls[S], l[S], M = NEG;
#pragma unroll
                    for (int t = 0; t < S; ++t) {
                        ls[t] = row_dot<V, A, NP>(qr[g], kr[t]) * c;
                        gd[t] = row_dot<V, A, NP>(dr[g], vr[t]);
                        l[t] = live[t] ? ls[t] + lw[t] : NEG;
                        M = l[t] > M ? l[t] : M;
                    }
                    A ex[S], Z = 0;
#pragma unroll
                    for (int t = 0; t < S; ++t) {
                        ex[t] = live[t] ? fast_exp2(l[t] - M) : (A)0;
                        Z += ex[t];
                    }
                    const A invZ = Z > (A)0 ? fast_rcp(Z) : (A)0;
#pragma unroll
                    for (int t = 0; t < S; ++t) {
                        p[t] = ex[t] * invZ;
                        // dl / w = exp(l - M) / (Z w) = exp(scale * dot - M) / Z
                        pw[t] = live[t] ? fast_exp2(ls[t] - M) * invZ : (A)0;
                    }
                }
                A dg[S], dls[S];
                centered_pairwise<S>(p, gd, dg);
#pragma unroll
                for (int t = 0; t < S; ++t) {
                    dls[t] = p[t] * dg[t] * sc;
                    dws[t] += pw[t] * dg[t];
                }
                A sel_dl = dls[0], sel_p = p[0];
#pragma unroll
                for (int t = 1; t < S; ++t) {
                    sel_dl = r == t ? dls[t] : sel_dl;
                    sel_p = r == t ? p[t] : sel_p;
                }
                my_dl[g0 + g] = sel_dl;
                my_p[g0 + g] = sel_p;
                // dq of this head: sum over the slots of scale * dl * k
#pragma unroll
                for (int k = 0; k < NP; ++k) {
                    A dq[V];
#pragma unroll
                    for (int e = 0; e < V; ++e) dq[e] = 0;
#pragma unroll
                    for (int t = 0; t < S; ++t) {
                        A kf[V];
                        unpack16<A, V>(kr[t][k], kf);
#pragma unroll
                        for (int e = 0; e < V; ++e) dq[e] += dls[t] * kf[e];
                    }
                    if constexpr (R == 0) {
                        // the low half: elements [V/2 r, V/2 (r + 1)) of the row
                        store_f32_nt<V / 2>(a.dq + (qrow + g0 + g) * FROW + r * (V / 2) * 4, dq);
                    } else {
                        store_split_f32_nt<V>(a.dq + (qrow + g0 + g) * FROW + FPART * k, r, dq);
                    }
                }
            }
        }
        // lane t < s: coefficients of slot t (live slots only; the target
        // pass reads live edges only) and its dw
        bool my_live = live[0];
        A my_dw = dws[0];
#pragma unroll
        for (int t = 1; t < S; ++t) {
            my_live = r == t ? live[t] : my_live;
            my_dw = r == t ? dws[t] : my_dw;
        }
        const size_t my_e = (size_t)cur.pos.unit * a.s + r;
        if (r < a.s) {
            if (my_live) {
                float2* cp = a.ws.coef + my_e * G;
#pragma unroll
                for (int g = 0; g < G; ++g) cp[g] = make_float2((float)my_dl[g], (float)my_p[g]);
            }
            a.dw[my_e] = (float)my_dw;
            if (a.write_tgt) {
                int my_j = cur.j[0];
#pragma unroll
                for (int t = 1; t < S; ++t) my_j = r == t ? cur.j[t] : my_j;
                a.ws.tgt[(size_t)cur.pos.prow * a.s + r] = my_live ? my_j : -1;
            }
        }
        cur = nxt;
    }
}

template <typename T, int G, int P>
__global__ __launch_bounds__(kBlock) void sea_bwd_dst_fast_kernel(SeaBwdFast a) {
    using A = typename io<T>::acc;
    constexpr int V = io<T>::V;
    constexpr int ROW = 256;
    constexpr int FROW = ROW * 4 / (int)sizeof(T);
    constexpr int L = V / P;
    const int lane = threadIdx.x & (kWave - 1);
    const int r = lane & 15;
    const int row = lane >> 4;
    const int slot = row & (P - 1);
    const Sched sch = xcd_sched(a.sp, 16 * P);

    // row header: output row, head, and its segment [beg, end) of the list
    struct Hdr {
        int unit, h, beg, end;
    };
    auto header = [&](int u) {
        Hdr hd{0, 0, 0, 0};
        if (u < sch.end) {
            const Pos pos = pos_of(a.sp, sch.x, u);
            hd.unit = pos.unit;
            hd.h = pos.unit - pos.bi * a.hkv;
            if (a.global_index) {
                hd.beg = a.ws.off[pos.unit];
                hd.end = a.ws.off[pos.unit + 1];
            } else {
                hd.beg = a.ws.beg[pos.prow];
                hd.end = hd.beg + a.ws.len[pos.prow];
            }
        }
        return hd;
    };
    auto edge_at = [&](int ei, int end) { return ei < end ? a.ws.list[ei] : -1; };

    Hdr h0 = header(sch.q);
    Hdr h1 = header(sch.q + sch.step);
    int e0 = edge_at(h0.beg + slot, h0.end);
    for (int u = sch.q; u < sch.end; u += sch.step) {
        const Hdr h2 = header(u + 2 * sch.step);
        const int e1 = edge_at(h1.beg + slot, h1.end);
        A ak[V], av[V];
#pragma unroll
        for (int e = 0; e < V; ++e) { ak[e] = 0; av[e] = 0; }
        int eid = e0;
        for (int e0pos = h0.beg; e0pos < h0.end; e0pos += P) {
            if (e0pos != h0.beg) eid = edge_at(e0pos + slot, h0.end);
            if (eid >= 0) {
                const int src = (int)fdiv((uint32_t)eid, a.fd_s);      // source unit
                const int sbi = (int)fdiv((uint32_t)src, a.fd_hkv);    // its b*n + i
                const uint32_t qrow = (uint32_t)(sbi * a.hq + h0.h * G);
                const float2* cf = a.ws.coef + (size_t)eid * G;
                uint4 qr[G], dr[G];
                float2 co[G];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    qr[g] = *reinterpret_cast<const uint4*>(a.q + (qrow + g) * ROW + r * 16);
                    dr[g] = *reinterpret_cast<const uint4*>(a.dout + (qrow + g) * ROW + r * 16);
                    co[g] = cf[g];
                }
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    A qf[V], df[V];
                    unpack16<A, V>(qr[g], qf);
                    unpack16<A, V>(dr[g], df);
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        ak[e] += (A)co[g].x * qf[e];
                        av[e] += (A)co[g].y * df[e];
                    }
                }
            }
        }
        rows_reduce_scatter<P, V>(ak);
        rows_reduce_scatter<P, V>(av);
        const uint32_t o = (uint32_t)h0.unit * FROW + r * 16 * 4 / (int)sizeof(T) +
                           rs_offset<V, P>(row) * 4;
        store_f32_nt<L>(a.dk + o, ak);
        store_f32_nt<L>(a.dv + o, av);
        h0 = h1;
        h1 = h2;
        e0 = e1;
    }
}

// Target pass, dispatched rather than persistent: the workgroups of XCD x
// take the items of x's list in order, one item per P 16-lane rows, so the
// hardware dispatcher, which starts workgroups in order as others retire,
// keeps each XCD's working window inside about one pair however unevenly
// the in-degrees fall (a persistent grid's teams drift apart and spread the
// window over two pairs, whose gathered rows do not fit one L2).  The row's
// first edge ids come from its head record, loaded together with its
// length, so a team waits on two round trips (ids, then the gathered rows);
// further passes load their ids before waiting on the current gathers.
// one wavefront per workgroup: the finest granularity for the hardware's
// in-order start of workgroups as others retire (measured ~3 us faster per
// pass than four wavefronts per workgroup; eight were slower)
constexpr int kDstBlock = kWave;

template <typename T, int G, int P, int R>
__global__ __launch_bounds__(kDstBlock) void sea_bwd_dst_row_kernel(SeaBwdFast a) {
    using A = typename io<T>::acc;
    constexpr int V = io<T>::V;
    // R 256-byte parts per d-row; R = 0: a 128-byte row, lane r holding
    // bytes [8r, 8r + 8) in the low half of its registers (bf16 only)
    constexpr int ROW = R == 0 ? 128 : 256 * R;
    constexpr int NP = R == 0 ? 1 : R;
    constexpr int FROW = ROW * 4 / (int)sizeof(T);
    constexpr int FPART = FROW / NP;
    static_assert(R > 0 || V / 2 >= P, "a 128-byte row needs V/2 >= P");
    constexpr int L = V / P;
    static_assert(P == 2 || P == 4, "two or four 16-lane rows per target row");
    const int lane = threadIdx.x & (kWave - 1);
    const int r = lane & 15;
    const int row = lane >> 4;
    const int slot = row & (P - 1);
    constexpr int TPW = 4 / P;   // rows per wavefront, one per 16P lanes
    const int x = blockIdx.x % kXcds;
    const int q = ((int)(blockIdx.x / kXcds) * (kDstBlock / kWave) + (int)threadIdx.x / kWave) * TPW +
                  row / P;
    const int nseg_x = x < a.sp.nseg ? (a.sp.nseg - x + kXcds - 1) / kXcds : 0;
    if (q >= nseg_x * a.sp.L) return;
    const Pos pos = pos_of(a.sp, x, q);
    const int h = pos.unit - pos.bi * a.hkv;
    int eid = a.ws.head[(size_t)pos.prow * 4 + slot];
    const int beg = a.ws.beg[pos.prow];
    const int len = a.ws.len[pos.prow];
    if (slot >= len) eid = -1;
    const uint32_t qbase = (uint32_t)h * G;

    A ak[NP][V], av[NP][V];
#pragma unroll
    for (int k = 0; k < NP; ++k)
#pragma unroll
        for (int e = 0; e < V; ++e) { ak[k][e] = 0; av[k][e] = 0; }
    for (int p0 = 0;;) {
        uint4 qr[G][NP], dr[G][NP];
        float2 co[G];
        if (eid >= 0) {
            const int src = (int)fdiv((uint32_t)eid, a.fd_s);      // source unit
            const int sbi = (int)fdiv((uint32_t)src, a.fd_hkv);    // its b*n + i
            const uint32_t qrow = (uint32_t)sbi * a.hq + qbase;
            const float2* cf = a.ws.coef + (size_t)eid * G;
#pragma unroll
            for (int g = 0; g < G; ++g) {
#pragma unroll
                for (int k = 0; k < NP; ++k) {
                    if constexpr (R == 0) {
                        const uint2 q2 = *reinterpret_cast<const uint2*>(a.q + (qrow + g) * ROW + r * 8);
                        const uint2 d2 =
                            *reinterpret_cast<const uint2*>(a.dout + (qrow + g) * ROW + r * 8);
                        qr[g][k] = make_uint4(q2.x, q2.y, 0u, 0u);
                        dr[g][k] = make_uint4(d2.x, d2.y, 0u, 0u);
                    } else {
                        qr[g][k] = *reinterpret_cast<const uint4*>(a.q + (qrow + g) * ROW +
                                                                   256 * k + r * 16);
                        dr[g][k] = *reinterpret_cast<const uint4*>(a.dout + (qrow + g) * ROW +
                                                                   256 * k + r * 16);
                    }
                }
                co[g] = cf[g];
            }
        }
        const int pn = p0 + P;
        const int enext = pn + slot < len ? a.ws.list[beg + pn + slot] : -1;
        if (eid >= 0) {
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int k = 0; k < NP; ++k) {
                    A qf[V], df[V];
                    unpack16<A, V>(qr[g][k], qf);
                    unpack16<A, V>(dr[g][k], df);
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        ak[k][e] += (A)co[g].x * qf[e];
                        av[k][e] += (A)co[g].y * df[e];
                    }
                }
        }
        if (pn >= len) break;
        p0 = pn;
        eid = enext;
    }
    if constexpr (R == 0) {
        // only the low V/2 accumulators hold data
        A hk[V / 2], hv[V / 2];
#pragma unroll
        for (int e = 0; e < V / 2; ++e) { hk[e] = ak[0][e]; hv[e] = av[0][e]; }
        rows_reduce_scatter<P, V / 2>(hk);
        rows_reduce_scatter<P, V / 2>(hv);
        const uint32_t o = (uint32_t)pos.unit * FROW + r * (V / 2) * 4 + rs_offset<V / 2, P>(row) * 4;
        store_f32_nt<V / 2 / P>(a.dk + o, hk);
        store_f32_nt<V / 2 / P>(a.dv + o, hv);
        return;
    }
#pragma unroll
    for (int k = 0; k < NP; ++k) {
        rows_reduce_scatter<P, V>(ak[k]);
        rows_reduce_scatter<P, V>(av[k]);
    }
    const uint32_t o = (uint32_t)pos.unit * FROW + r * 16 * 4 / (int)sizeof(T) +
                       rs_offset<V, P>(row) * 4;
#pragma unroll
    for (int k = 0; k < NP; ++k) {
        store_f32_nt<L>(a.dk + o + FPART * k, ak[k]);
        store_f32_nt<L>(a.dv + o + FPART * k, av[k]);
    }
}

// Target pass with four incoming edges per pass (s = 4): the same work as
// sea_bwd_dst_row_kernel<T, G, 4, R>, with everything that is the same for
// the whole wavefront read through the scalar data cache: the row's head
// record, offset and length, each pass's four coefficient records and the
// next pass's four edge ids.  Only the q/dout rows go through the vector
// memory path, whose outstanding requests per CU bound this pass.
template <typename T, int G, int R>
__global__ __launch_bounds__(kDstBlock) void sea_bwd_dst_row_s_kernel(SeaBwdFast a) {
    using A = typename io<T>::acc;
    constexpr int V = io<T>::V;
    constexpr int P = 4;
    constexpr int ROW = R == 0 ? 128 : 256 * R;
    constexpr int NP = R == 0 ? 1 : R;
    constexpr int FROW = ROW * 4 / (int)sizeof(T);
    constexpr int FPART = FROW / NP;
    static_assert(R > 0 || V / 2 >= P, "a 128-byte row needs V/2 >= P");
    static_assert(G >= 1 && G <= 4, "the coefficient records of four edges fit the scalar registers");
    constexpr int L = V / P;
    constexpr int CW = 2 * G;   // coefficient words per edge
    const int lane = threadIdx.x & (kWave - 1);
    const int r = lane & 15;
    const int row = lane >> 4;   // the edge slot of this 16-lane row
    const int x = blockIdx.x % kXcds;
    const int q = (int)(blockIdx.x / kXcds);   // one target row per wavefront
    const int nseg_x = x < a.sp.nseg ? (a.sp.nseg - x + kXcds - 1) / kXcds : 0;
    if (q >= nseg_x * a.sp.L) return;
    const Pos pos = pos_of(a.sp, x, q);
    const int h = pos.unit - pos.bi * a.hkv;
    const int* hp = a.ws.head + (size_t)pos.prow * 4;
    int e0 = hp[0], e1 = hp[1], e2 = hp[2], e3 = hp[3];   // -1 padded
    asm("" : "+s"(e0), "+s"(e1), "+s"(e2), "+s"(e3));
    const int beg = a.ws.beg[pos.prow];
    const int len = a.ws.len[pos.prow];
    const uint32_t qbase = (uint32_t)h * G;
    const float* coef = reinterpret_cast<const float*>(a.ws.coef);

    A ak[NP][V], av[NP][V];
#pragma unroll
    for (int k = 0; k < NP; ++k)
#pragma unroll
        for (int e = 0; e < V; ++e) { ak[k][e] = 0; av[k][e] = 0; }
    for (int p0 = 0;;) {
        int eid = e0;
        eid = row == 1 ? e1 : eid;
        eid = row == 2 ? e2 : eid;
        eid = row == 3 ? e3 : eid;
        uint4 qr[G][NP], dr[G][NP];
        if (eid >= 0) {
            const int src = (int)fdiv((uint32_t)eid, a.fd_s);      // source unit
            const int sbi = (int)fdiv((uint32_t)src, a.fd_hkv);    // its b*n + i
            const uint32_t qrow = (uint32_t)sbi * a.hq + qbase;
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int k = 0; k < NP; ++k) {
                    if constexpr (R == 0) {
                        const uint2 q2 = *reinterpret_cast<const uint2*>(a.q + (qrow + g) * ROW + r * 8);
                        const uint2 d2 =
                            *reinterpret_cast<const uint2*>(a.dout + (qrow + g) * ROW + r * 8);
                        qr[g][k] = make_uint4(q2.x, q2.y, 0u, 0u);
                        dr[g][k] = make_uint4(d2.x, d2.y, 0u, 0u);
                    } else {
                        qr[g][k] = *reinterpret_cast<const uint4*>(a.q + (qrow + g) * ROW +
                                                                   256 * k + r * 16);
                        dr[g][k] = *reinterpret_cast<const uint4*>(a.dout + (qrow + g) * ROW +
                                                                   256 * k + r * 16);
                    }
                }
        }
        // the four edges' coefficient records (a dead slot reads record 0)
        // and the next pass's ids (the list ends in eight spare entries, so
        // these reads stay inside it), all in one scalar round trip
        float c0[CW], c1[CW], c2[CW], c3[CW];
        const int pn = p0 + P;
        int n0, n1, n2, n3;
        {
            const float* p0c = coef + (size_t)(e0 < 0 ? 0 : e0) * CW;
            const float* p1c = coef + (size_t)(e1 < 0 ? 0 : e1) * CW;
            const float* p2c = coef + (size_t)(e2 < 0 ? 0 : e2) * CW;
            const float* p3c = coef + (size_t)(e3 < 0 ? 0 : e3) * CW;
#pragma unroll
            for (int j = 0; j < CW; ++j) {
                c0[j] = p0c[j]; c1[j] = p1c[j]; c2[j] = p2c[j]; c3[j] = p3c[j];
                // opaque to the optimiser: a select between loaded values
                // would otherwise become branches around the loads
                asm("" : "+s"(c0[j]), "+s"(c1[j]), "+s"(c2[j]), "+s"(c3[j]));
            }
            const int* lp = a.ws.list + beg + pn;
            n0 = lp[0]; n1 = lp[1]; n2 = lp[2]; n3 = lp[3];
            asm("" : "+s"(n0), "+s"(n1), "+s"(n2), "+s"(n3));
            n0 = pn < len ? n0 : -1;
            n1 = pn + 1 < len ? n1 : -1;
            n2 = pn + 2 < len ? n2 : -1;
            n3 = pn + 3 < len ? n3 : -1;
        }
        if (eid >= 0) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float cx = c0[2 * g], cy = c0[2 * g + 1];
                cx = row == 1 ? c1[2 * g] : cx;
                cy = row == 1 ? c1[2 * g + 1] : cy;
                cx = row == 2 ? c2[2 * g] : cx;
                cy = row == 2 ? c2[2 * g + 1] : cy;
                cx = row == 3 ? c3[2 * g] : cx;
                cy = row == 3 ? c3[2 * g + 1] : cy;
#pragma unroll
                for (int k = 0; k < NP; ++k) {
                    A qf[V], df[V];
                    unpack16<A, V>(qr[g][k], qf);
                    unpack16<A, V>(dr[g][k], df);
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        ak[k][e] += (A)cx * qf[e];
                        av[k][e] += (A)cy * df[e];
                    }
                }
            }
        }
        if (pn >= len) break;
        p0 = pn;
        e0 = n0; e1 = n1; e2 = n2; e3 = n3;
    }
    if constexpr (R == 0) {
        A hk[V / 2], hv[V / 2];
#pragma unroll
        for (int e = 0; e < V / 2; ++e) { hk[e] = ak[0][e]; hv[e] = av[0][e]; }
        rows_reduce_scatter<P, V / 2>(hk);
        rows_reduce_scatter<P, V / 2>(hv);
        const uint32_t o = (uint32_t)pos.unit * FROW + r * (V / 2) * 4 + rs_offset<V / 2, P>(row) * 4;
        store_f32_nt<V / 2 / P>(a.dk + o, hk);
        store_f32_nt<V / 2 / P>(a.dv + o, hv);
        return;
    }
#pragma unroll
    for (int k = 0; k < NP; ++k) {
        rows_reduce_scatter<P, V>(ak[k]);
        rows_reduce_scatter<P, V>(av[k]);
    }
    const uint32_t o = (uint32_t)pos.unit * FROW + r * 16 * 4 / (int)sizeof(T) +
                       rs_offset<V, P>(row) * 4;
#pragma unroll
    for (int k = 0; k < NP; ++k) {
        store_f32_nt<L>(a.dk + o + FPART * k, ak[k]);
        store_f32_nt<L>(a.dv + o + FPART * k, av[k]);
    }
}

template <typename T, int G, int PD, int R>
void launch_dst_row(const SeaBwdFast& a, hipStream_t st) {
    const long long per_x = (long long)((a.sp.nseg + kXcds - 1) / kXcds) * a.sp.L;
    const long long rows_per_block = kDstBlock / kWave * (4 / PD);
    const long long blocks = kXcds * ((per_x + rows_per_block - 1) / rows_per_block);
    if constexpr (PD == 4 && G >= 1 && G <= 4) {
        hipLaunchKernelGGL((sea_bwd_dst_row_s_kernel<T, G, R>), dim3((unsigned)blocks),
                           dim3(kDstBlock), 0, st, a);
    } else {
        hipLaunchKernelGGL((sea_bwd_dst_row_kernel<T, G, PD, R>), dim3((unsigned)blocks),
                           dim3(kDstBlock), 0, st, a);
    }
}

void launch_index(const SeaBwdArgs& a, long long E, hipStream_t st) {
    const unsigned sblocks = (unsigned)((a.U + kScanPerBlock - 1) / kScanPerBlock);
    hipLaunchKernelGGL(scan_local_kernel, dim3(sblocks), dim3(1024), 0, st,
                       (const int*)a.ws.cnt, a.ws.off, a.ws.bsum, a.U);
    hipLaunchKernelGGL(scan_add_kernel, dim3(sblocks), dim3(1024), 0, st, a.ws.off, a.ws.cnt,
                       (const int*)a.ws.bsum, a.U);
    long long fb = (E + kBlock - 1) / kBlock;
    if (fb > 16384) fb = 16384;
    hipLaunchKernelGGL(edge_fill_kernel, dim3((unsigned)fb), dim3(kBlock), 0, st, a.idx, a.w, a.n,
                       a.hkv, a.s, E, a.ws.cnt, a.ws.list);
    // the id-ordered list goes to ws.tgt (unused on these paths), which the
    // target passes then read as their list
    hipLaunchKernelGGL(edge_order_kernel, dim3((unsigned)fb), dim3(kBlock), 0, st, a.idx, a.w,
                       a.n, a.hkv, a.s, E, (const int*)a.ws.off, (const int*)a.ws.list,
                       a.ws.tgt);
}

template <typename T, int G>
hipError_t run(const SeaBwdArgs& a, long long E, hipStream_t st) {
    const long long src_threads = (long long)a.U * a.ts.team;
    hipLaunchKernelGGL((sea_bwd_src_kernel<T, G>),
                       dim3((unsigned)((src_threads + kBlock - 1) / kBlock)), dim3(kBlock), 0, st,
                       a);
    launch_index(a, E, st);
    SeaBwdArgs t = a;
    t.ws.list = a.ws.tgt;   // the id-ordered list
    const long long dst_threads = (long long)a.U * a.tt.team;
    hipLaunchKernelGGL((sea_bwd_dst_kernel<T, G>),
                       dim3((unsigned)((dst_threads + kBlock - 1) / kBlock)), dim3(kBlock), 0, st,
                       t);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch_g(const SeaBwdArgs& a, int G, long long E, hipStream_t st) {
    switch (G) {
        case 1: return run<T, 1>(a, E, st);
        case 2: return run<T, 2>(a, E, st);
        case 4: return run<T, 4>(a, E, st);
        case 8: return run<T, 8>(a, E, st);
        case 16: return run<T, 16>(a, E, st);
        default: return run<T, 0>(a, E, st);   // other group sizes
    }
}

template <typename T, int G, int S, bool VEC, bool GLOBAL, bool SAVED, int R>
void launch_src_k(const SeaBwdFast& a, hipStream_t st) {
    if constexpr (R == 1) {
        if constexpr (SAVED && VEC && G == 2 && S == 4 && std::is_same<T, bf16_t>::value) {
            if ((a.sp.L & 3) == 0) {
                const void* fn = reinterpret_cast<const void*>(
                    &sea_bwd_src_row_kernel<T, G, S, VEC, GLOBAL, SAVED, true>);
                hipLaunchKernelGGL((sea_bwd_src_row_kernel<T, G, S, VEC, GLOBAL, SAVED, true>),
                                   dim3(persistent_grid(fn, a.U, kBlock / 16)), dim3(kBlock), 0,
                                   st, a);
                return;
            }
        }
        const void* fn = reinterpret_cast<const void*>(
            &sea_bwd_src_row_kernel<T, G, S, VEC, GLOBAL, SAVED, false>);
        hipLaunchKernelGGL((sea_bwd_src_row_kernel<T, G, S, VEC, GLOBAL, SAVED, false>),
                           dim3(persistent_grid(fn, a.U, kBlock / 16)), dim3(kBlock), 0, st, a);
    } else {
        const void* fn = reinterpret_cast<const void*>(
            &sea_bwd_src_wide_kernel<T, G, S, VEC, GLOBAL, SAVED, R>);
        hipLaunchKernelGGL((sea_bwd_src_wide_kernel<T, G, S, VEC, GLOBAL, SAVED, R>),
                           dim3(persistent_grid(fn, a.U, kBlock / 16)), dim3(kBlock), 0, st, a);
    }
}

template <typename T, int G, int S, bool VEC, bool GLOBAL, int R>
void launch_src(const SeaBwdFast& a, hipStream_t st) {
    // the saved statistics (fp32 p / w for bf16 inputs, fp64 for fp32
    // inputs) replace the recomputed softmax
    if (a.stats) {
        launch_src_k<T, G, S, VEC, GLOBAL, true, R>(a, st);
    } else {
        launch_src_k<T, G, S, VEC, GLOBAL, false, R>(a, st);
    }
}

// 512-byte rows (R = 2): the single-pass or partitioned index only (the
// global-index target kernel takes 256-byte rows)
template <typename T, int G, int S, bool VEC, int PD, int R>
hipError_t run_fast2(const SeaBwdArgs& g, const SeaBwdFast& a, long long E, hipStream_t st) {
    (void)g; (void)E;
    launch_src<T, G, S, VEC, false, R>(a, st);
    const hipError_t e =
        edge_index_one_pass(a.n)
            ? launch_edge_index(a.U / (a.n * a.hkv), a.n, a.hkv, a.idx, a.w, a.s, a.ws.tgt,
                                a.ws.beg, a.ws.len, a.ws.list, a.ws.head, st)
            : launch_edge_index_long(a.U / (a.n * a.hkv), a.n, a.hkv, a.idx, a.w, a.s,
                                     a.ws.tgt, a.ws.beg, a.ws.len, a.ws.list, a.ws.head,
                                     a.ws.cnt, a.ws.off, a.ws.bsum, a.ws.stage, st);
    if (e != hipSuccess) return e;
    launch_dst_row<T, G, PD, R>(a, st);
    return hipGetLastError();
}

template <typename T, int G, int S, bool VEC, int PD, int R>
hipError_t run_fast(const SeaBwdArgs& g, const SeaBwdFast& a, long long E, hipStream_t st) {
    if constexpr (R != 1) return run_fast2<T, G, S, VEC, PD, R>(g, a, E, st);
    if (a.global_index) {
        const hipError_t e = launch_zero_f32(reinterpret_cast<float*>(a.ws.cnt), (size_t)a.U, st);
        if (e != hipSuccess) return e;
        launch_src<T, G, S, VEC, true, 1>(a, st);
        launch_index(g, E, st);
    } else if (!edge_index_one_pass(a.n)) {
        // long sequences: the partitioned index, from the source pass's
        // compact targets
        launch_src<T, G, S, VEC, false, 1>(a, st);
        const hipError_t e = launch_edge_index_long(
            a.U / (a.n * a.hkv), a.n, a.hkv, a.idx, a.w, a.s, a.ws.tgt, a.ws.beg, a.ws.len,
            a.ws.list, a.ws.head, a.ws.cnt, a.ws.off, a.ws.bsum, a.ws.stage, st);
        if (e != hipSuccess) return e;
    } else {
        launch_src<T, G, S, VEC, false, 1>(a, st);
        const hipError_t e = launch_edge_index(a.U / (a.n * a.hkv), a.n, a.hkv, a.idx, a.w, a.s,
                                               a.ws.tgt, a.ws.beg, a.ws.len, a.ws.list,
                                               a.ws.head, st);
        if (e != hipSuccess) return e;
    }
    if (!a.global_index) {
        launch_dst_row<T, G, PD, 1>(a, st);
        return hipGetLastError();
    }
    const int ndst = persistent_grid(reinterpret_cast<const void*>(
                                         &sea_bwd_dst_fast_kernel<T, G, PD>),
                                     a.U, kBlock / (16 * PD));
    SeaBwdFast t = a;
    t.ws.list = a.ws.tgt;   // the id-ordered list
    hipLaunchKernelGGL((sea_bwd_dst_fast_kernel<T, G, PD>), dim3(ndst), dim3(kBlock), 0, st, t);
    return hipGetLastError();
}

template <typename T, int G, int R>
hipError_t fast_p(const SeaBwdArgs& g, const SeaBwdFast& a, long long E, hipStream_t st) {
    if (a.s <= 1) return run_fast<T, G, 1, false, 2, R>(g, a, E, st);
    if (a.s <= 2) return run_fast<T, G, 2, false, 2, R>(g, a, E, st);
    if (a.vec) return run_fast<T, G, 4, true, 4, R>(g, a, E, st);
    return run_fast<T, G, 4, false, 4, R>(g, a, E, st);
}

template <typename T>
hipError_t dispatch_fast(const SeaBwdArgs& g, const SeaBwdFast& a, int G, int R, long long E,
                         hipStream_t st) {
    if constexpr (std::is_same<T, bf16_t>::value) {
        if (R == 0) {
            switch (G) {
                case 1: return fast_p<T, 1, 0>(g, a, E, st);
                case 2: return fast_p<T, 2, 0>(g, a, E, st);
                case 4: return fast_p<T, 4, 0>(g, a, E, st);
                case 8: return fast_p<T, 8, 0>(g, a, E, st);
                case 16: return fast_p<T, 16, 0>(g, a, E, st);
                default: return hipErrorInvalidValue;
            }
        }
    }
    if (R == 2) {
        switch (G) {
            case 1: return fast_p<T, 1, 2>(g, a, E, st);
            case 2: return fast_p<T, 2, 2>(g, a, E, st);
            case 4: return fast_p<T, 4, 2>(g, a, E, st);
            case 8: return fast_p<T, 8, 2>(g, a, E, st);
            default: return hipErrorInvalidValue;
        }
    }
    switch (G) {
        case 1: return fast_p<T, 1, 1>(g, a, E, st);
        case 2: return fast_p<T, 2, 1>(g, a, E, st);
        case 4: return fast_p<T, 4, 1>(g, a, E, st);
        case 8: return fast_p<T, 8, 1>(g, a, E, st);
        case 16: return fast_p<T, 16, 1>(g, a, E, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t sea_backward_workspace_bytes(long long U, int s, int G, int n) {
    return ws_layout(U, s, G, n).total;
}

hipError_t launch_sea_backward(int B, int n, int hq, int hkv, int d, bool bf16, float scale,
                               const void* q, const void* k, const void* v,
                               const int32_t* idx, const float* w, int s, const void* dout,
                               const float* stats, float* dq, float* dk, float* dv, float* dw,
                               void* workspace, hipStream_t st) {
    const int G = hq / hkv;
    SeaBwdArgs a;
    a.q = q; a.k = k; a.v = v; a.dout = dout; a.idx = idx; a.w = w;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dw = dw;
    a.n = n; a.hq = hq; a.hkv = hkv; a.d = d; a.s = s;
    a.U = B * n * hkv;
    a.scale = scale;
    const int es = bf16 ? 2 : 4;
    a.ts = sea_team(d, es, s);
    // target pass: up to 8 incoming edges side by side (rows have ~s on average)
    a.tt = sea_team(d, es, 8);
    const WsLayout l = ws_layout(a.U, s, G, n);
    char* base = static_cast<char*>(workspace);
    a.ws.coef = reinterpret_cast<float2*>(base + l.coef);
    a.ws.cnt = reinterpret_cast<int*>(base + l.cnt);
    a.ws.off = reinterpret_cast<int*>(base + l.off);
    a.ws.bsum = reinterpret_cast<int*>(base + l.bsum);
    a.ws.list = reinterpret_cast<int*>(base + l.list);
    a.ws.beg = reinterpret_cast<int*>(base + l.beg);
    a.ws.len = reinterpret_cast<int*>(base + l.len);
    a.ws.head = reinterpret_cast<int*>(base + l.head);
    a.ws.tgt = reinterpret_cast<int*>(base + l.tgt);
    a.ws.stage = reinterpret_cast<int2*>(base + l.stage);
    const long long E = (long long)a.U * s;
    // row kernels: 256-byte rows with any index; with the single-pass or
    // partitioned index also 512-byte rows (G <= 8) and bf16 128-byte rows
    const bool part = edge_index_supported(n, s);
    const int R = sea_fast_shape(B, n, hq, hkv, d, bf16, s)                          ? 1
                  : sea_fast_shape(B, n, hq, hkv, d / 2, bf16, s) && G <= 8 && part ? 2
                  : bf16 && sea_fast_shape(B, n, hq, hkv, d * 2, bf16, s) && part   ? 0
                                                                                    : -1;
    if (R >= 0 && sea_row_group(G) && (long long)B * n * hq * d * 4 < (1ll << 32)) {
        SeaBwdFast f;
        f.q = static_cast<const char*>(q); f.k = static_cast<const char*>(k);
        f.v = static_cast<const char*>(v); f.dout = static_cast<const char*>(dout);
        f.stats = (s == 4 && ((uintptr_t)stats & 15)) ? nullptr : stats;
        f.idx = idx; f.w = w;
        f.dq = reinterpret_cast<char*>(dq); f.dk = reinterpret_cast<char*>(dk);
        f.dv = reinterpret_cast<char*>(dv); f.dw = dw;
        f.ws = a.ws;
        f.n = n; f.hq = hq; f.hkv = hkv; f.s = s; f.U = a.U; f.scale = scale;
        f.fd_hkv = make_fastdiv((uint32_t)hkv);
        f.fd_s = make_fastdiv((uint32_t)s);
        make_seg_plan(f.sp, B, n, hkv);
        f.global_index = !edge_index_supported(n, s);
        f.write_tgt = !f.global_index;
        f.vec = s == 4 && (((uintptr_t)idx | (uintptr_t)w) & 15) == 0;
        return bf16 ? dispatch_fast<bf16_t>(a, f, G, R, E, st)
                    : dispatch_fast<float>(a, f, G, R, E, st);
    }
    hipError_t e = launch_zero_f32(reinterpret_cast<float*>(a.ws.cnt), (size_t)a.U, st);
    if (e == hipSuccess && a.ts.nchunk > 1) e = launch_zero_f32(dw, (size_t)a.U * s, st);
    if (e != hipSuccess) return e;
    return bf16 ? dispatch_g<bf16_t>(a, G, E, st) : dispatch_g<float>(a, G, E, st);
}

}  // namespace gm
