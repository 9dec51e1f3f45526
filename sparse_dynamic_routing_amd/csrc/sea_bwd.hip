// Sparse edge attention, backward, for gfx950.
//
// Chain rule of the forward with the indices held fixed (rit.work "Graph
// Machine" article: indices get no gradient, learning goes through the soft
// edge weights).  Per unit and query head, over the live slots t:
//   p_t  = softmax(scale q.k_t + ln w_t)      (recomputed, log2 domain)
//   g_t  = dout . v_t,  gbar = sum_t p_t g_t,  dl_t = p_t (g_t - gbar)
//   dq   = scale sum_t dl_t k_t               (reduce-scattered, fp32 store)
//   dk[idx_t] += scale dl_t q,  dv[idx_t] += p_t dout   (summed over the
//                                              group's heads, then scattered)
//   dw_t = sum_heads dl_t / w_t = sum_heads exp2(ls_t - M) / Z (g_t - gbar)
// The last form never divides by w, so it is finite for tiny weights.
//
// Mapping as in the forward: a team of R * P lanes per unit, one 16-byte
// piece of a K/V/q/dout row per lane.  The dk/dv rows of a wave are written
// to LDS and read back transposed, so each global fp32 atomic instruction
// covers 64 consecutive floats of one row (two 128-byte lines) instead of
// 64 scattered lanes.
#include "gm_common.h"
#include "gm_internal.h"

#include <math.h>

namespace gm {
namespace {

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
    int n, hq, hkv, d, s, U, log2d;
    float scale;
    TeamShape ts;
};

// Per-wave staging of dk/dv rows (64 lanes x V floats each) and row targets.
template <int V>
struct Stage {
    float dk[kBlock / kWave][kWave * V];
    float dv[kBlock / kWave][kWave * V];
    int tgt[kBlock / kWave][kWave];
};

// Write this lane's V floats of its slot row to LDS, then scatter the wave's
// rows with contiguous atomics.  Every lane of the block must call this.
template <int V, typename A>
__device__ __forceinline__ void scatter_rows(Stage<V>& sm, const A (&dk)[V], const A (&dv)[V],
                                             long long tgt_row, int R, int log2d, int d,
                                             float* gdk, float* gdv) {
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int e = 0; e < V; ++e) {
        sm.dk[wave][lane * V + e] = (float)dk[e];
        sm.dv[wave][lane * V + e] = (float)dv[e];
    }
    if ((lane & (R - 1)) == 0) sm.tgt[wave][lane / R] = (int)tgt_row;
    __syncthreads();
#pragma unroll
    for (int it = 0; it < V; ++it) {
        const int f = it * kWave + lane;
        const int row = f >> log2d;
        const int col = f & (d - 1);
        const int tr = sm.tgt[wave][row];
        if (tr >= 0) {
            const size_t o = (size_t)tr * d + col;
            unsafeAtomicAdd(gdk + o, sm.dk[wave][f]);
            unsafeAtomicAdd(gdv + o, sm.dv[wave][f]);
        }
    }
    __syncthreads();
}

template <typename T, int G>
__global__ __launch_bounds__(kBlock) void sea_bwd_kernel(SeaBwdArgs a) {
    using A = typename io<T>::acc;
    constexpr int V = io<T>::V;
    constexpr int LOG2V = ilog2(V);
    __shared__ Stage<V> sm;
    const int R = a.ts.R, team = a.ts.team, P = a.ts.P;
    const int lane = threadIdx.x & (kWave - 1);
    const int tl = lane & (team - 1);
    const int r = tl & (R - 1);
    const int sl = tl >> a.ts.log2R;
    const long long gunit = ((long long)blockIdx.x * kBlock + threadIdx.x) / team;
    const bool active = gunit < a.U;   // no early return: the block synchronises
    const int unit = active ? (int)gunit : 0;
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
    const A c = (A)a.scale * (A)1.4426950408889634;
    const A sc = (A)a.scale;
    const A NEG = -INFINITY;
    const bool storer = active && (sl >> LOG2V) == 0;

    if (a.ts.nchunk == 1) {
        const int t = sl;
        bool live = false;
        A lw = NEG;
        long long tgt = -1;
        A kr[V], vr[V];
#pragma unroll
        for (int e = 0; e < V; ++e) { kr[e] = 0; vr[e] = 0; }
        if (active && t < a.s) {
            const float wt = wp[t];
            if (wt > 0.0f) {
                live = true;
                lw = alog2((A)wt);
                tgt = (long long)(kv0 + (size_t)ip[t] * a.hkv);
                load16(kp + tgt * d, kr);
                load16(vp + tgt * d, vr);
            }
        }
        A dka[V], dva[V];
#pragma unroll
        for (int e = 0; e < V; ++e) { dka[e] = 0; dva[e] = 0; }
        A dws = 0;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            A qg[V], dg[V];
            if (active) {
                load16(qp + g * d, qg);
                load16(dop + g * d, dg);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e) { qg[e] = 0; dg[e] = 0; }
            }
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
            const A gbar = sum_bits(p * gd, R, team);
            const A dls = p * (gd - gbar) * sc;
            A dqv[V];
#pragma unroll
            for (int e = 0; e < V; ++e) dqv[e] = dls * kr[e];
            int len;
            const int off = reduce_scatter(dqv, tl, R, team, len);
            if (storer) store_len(dqp + g * d + off, dqv, len);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                dka[e] += dls * qg[e];
                dva[e] += p * dg[e];
            }
            if (live) dws += aexp2(ls - M) * invZ * (gd - gbar);
        }
        if (active && r == 0 && t < a.s) a.dw[(size_t)unit * a.s + t] = (float)dws;
        scatter_rows<V>(sm, dka, dva, tgt, R, a.log2d, a.d, a.dk, a.dv);
        return;
    }

    // s > P: per head, pass 1 over the chunks finds the running max M, the
    // sum Z and sum e*g; pass 2 recomputes p, dl and scatters each chunk.
    // dw is accumulated with atomics here (the caller zero-filled it).
#pragma unroll 1
    for (int g = 0; g < G; ++g) {
        A qg[V], dg[V];
        if (active) {
            load16(qp + g * d, qg);
            load16(dop + g * d, dg);
        } else {
#pragma unroll
            for (int e = 0; e < V; ++e) { qg[e] = 0; dg[e] = 0; }
        }
        A M = NEG, Z = 0, Sg = 0;
#pragma unroll 1
        for (int ch = 0; ch < a.ts.nchunk; ++ch) {
            const int t = ch * P + sl;
            bool live = false;
            A lw = NEG;
            A kr[V], vr[V];
#pragma unroll
            for (int e = 0; e < V; ++e) { kr[e] = 0; vr[e] = 0; }
            if (active && t < a.s) {
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
            if (Mn == NEG) continue;
            const A alpha = aexp2(M - Mn);
            const A ex = live ? aexp2(l - Mn) : (A)0;
            Z = Z * alpha + sum_bits(ex, R, team);
            Sg = Sg * alpha + sum_bits(ex * gd, R, team);
            M = Mn;
        }
        const A invZ = Z > 0 ? (A)1 / Z : (A)0;
        const A gbar = Sg * invZ;
        A dqv[V];
#pragma unroll
        for (int e = 0; e < V; ++e) dqv[e] = 0;
#pragma unroll 1
        for (int ch = 0; ch < a.ts.nchunk; ++ch) {
            const int t = ch * P + sl;
            bool live = false;
            A lw = NEG;
            long long tgt = -1;
            A kr[V], vr[V];
#pragma unroll
            for (int e = 0; e < V; ++e) { kr[e] = 0; vr[e] = 0; }
            if (active && t < a.s) {
                const float wt = wp[t];
                if (wt > 0.0f) {
                    live = true;
                    lw = alog2((A)wt);
                    tgt = (long long)(kv0 + (size_t)ip[t] * a.hkv);
                    load16(kp + tgt * d, kr);
                    load16(vp + tgt * d, vr);
                }
            }
            A sd = 0, gd = 0;
#pragma unroll
            for (int e = 0; e < V; ++e) { sd += qg[e] * kr[e]; gd += dg[e] * vr[e]; }
            sd = sum_bits(sd, 1, R);
            gd = sum_bits(gd, 1, R);
            const A ls = sd * c;
            const A p = live ? aexp2(ls + lw - M) * invZ : (A)0;
            const A dls = p * (gd - gbar) * sc;
            A dka[V], dva[V];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                dqv[e] += dls * kr[e];
                dka[e] = dls * qg[e];
                dva[e] = p * dg[e];
            }
            if (live && r == 0)
                unsafeAtomicAdd(a.dw + (size_t)unit * a.s + t,
                                (float)(aexp2(ls - M) * invZ * (gd - gbar)));
            scatter_rows<V>(sm, dka, dva, tgt, R, a.log2d, a.d, a.dk, a.dv);
        }
        int len;
        const int off = reduce_scatter(dqv, tl, R, team, len);
        if (storer) store_len(dqp + g * d + off, dqv, len);
    }
}

template <typename T, int G>
hipError_t run(const SeaBwdArgs& a, hipStream_t st) {
    const long long threads = (long long)a.U * a.ts.team;
    const unsigned blocks = (unsigned)((threads + kBlock - 1) / kBlock);
    hipLaunchKernelGGL((sea_bwd_kernel<T, G>), dim3(blocks), dim3(kBlock), 0, st, a);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch_g(const SeaBwdArgs& a, int G, hipStream_t st) {
    switch (G) {
        case 1: return run<T, 1>(a, st);
        case 2: return run<T, 2>(a, st);
        case 4: return run<T, 4>(a, st);
        case 8: return run<T, 8>(a, st);
        case 16: return run<T, 16>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_sea_backward(int B, int n, int hq, int hkv, int d, bool bf16, float scale,
                               const void* q, const void* k, const void* v,
                               const int32_t* idx, const float* w, int s, const void* dout,
                               float* dq, float* dk, float* dv, float* dw, hipStream_t st) {
    SeaBwdArgs a;
    a.q = q; a.k = k; a.v = v; a.dout = dout; a.idx = idx; a.w = w;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dw = dw;
    a.n = n; a.hq = hq; a.hkv = hkv; a.d = d; a.s = s;
    a.U = B * n * hkv;
    a.log2d = ilog2(d);
    a.scale = scale;
    a.ts = sea_team(d, bf16 ? 2 : 4, s);
    const size_t nkv = (size_t)B * n * hkv * d;
    hipError_t e = launch_zero_f32(dk, nkv, st);
    if (e == hipSuccess) e = launch_zero_f32(dv, nkv, st);
    if (e == hipSuccess && a.ts.nchunk > 1) e = launch_zero_f32(dw, (size_t)B * n * hkv * s, st);
    if (e != hipSuccess) return e;
    const int G = hq / hkv;
    return bf16 ? dispatch_g<bf16_t>(a, G, st) : dispatch_g<float>(a, G, st);
}

}  // namespace gm
