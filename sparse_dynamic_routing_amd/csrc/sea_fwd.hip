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

struct SeaFwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* idx;
    const float* w;
    void* o;
    int n, hq, hkv, d, s, U;
    float scale;
    TeamShape ts;
};

template <typename T, int G>
__global__ __launch_bounds__(kBlock) void sea_fwd_kernel(SeaFwdArgs a) {
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
#pragma unroll
            for (int e = 0; e < V; ++e) ov[e] *= inv;
            if (storer) store_len(op + g * d + off, ov, len);
        }
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
    }
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
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_sea_forward(int B, int n, int hq, int hkv, int d, bool bf16, float scale,
                              const void* q, const void* k, const void* v,
                              const int32_t* idx, const float* w, int s, void* o,
                              hipStream_t st) {
    SeaFwdArgs a;
    a.q = q; a.k = k; a.v = v; a.idx = idx; a.w = w; a.o = o;
    a.n = n; a.hq = hq; a.hkv = hkv; a.d = d; a.s = s;
    a.U = B * n * hkv;
    a.scale = scale;
    a.ts = sea_team(d, bf16 ? 2 : 4, s);
    const int G = hq / hkv;
    return bf16 ? dispatch_g<bf16_t>(a, G, st) : dispatch_g<float>(a, G, st);
}

}  // namespace gm
