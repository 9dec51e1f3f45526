// Decode step: SER then SEA for the newest token of each sequence, against
// caches of earlier edge rows and K/V rows (inference; page "Graph Machine:
// Towards Better Pretraining via Edges", ai.info, "Why This Matters":
// long-context inference, where KV access is the binding cost).
//
// One 64-lane wavefront per (batch, KV head) unit, one launch per step:
//   lane k < s2*s3 holds candidate path k = (a, c): the token's leg-1 slot a
//   points at row j_a of the edge cache, whose slot c names target m; its
//   weight is w1[a] * w2[j_a][c] in fp64.  The first lane of each target
//   adds the later lanes of the same target in path order (the definition's
//   order and precision, so the weights are bit-identical to the training
//   pass), later ones drop out; each lane's rank among positive keys
//   (weight desc, target asc) comes from one sweep over the lanes (DPP row
//   rotations for up to 16 candidates, v_readlane beyond), and rank r < s1
//   writes output slot r (padding (0, 0) after the last candidate).
//   SEA then reads the kept slots' K/V cache rows in 16-byte pieces (lane l
//   holds piece l of each d-row; the query rows are loaded while SER runs),
//   four slots per step, each score a wavefront sum, with an online softmax
//   per query head.
// Everything is latency: a step reads ~s2*s3 edge entries and 2*s1 K/V rows
// per unit.  For bf16, d = 128 and at most 16 candidates a second kernel
// (decode16_kernel, below) loads every candidate's K/V rows while SER ranks
// them, so the third memory round trip no longer waits for the merge and
// ranking (8.4 -> 6.6 us per step of 8 sequences x 8 KV heads at a
// 4,096-token cache; 5.9 us with the ranking by DPP rotations).
#include "gm_common.h"
#include "gm_internal.h"
#include "gm_select.h"
#include "gm_wave.h"

namespace gm {
namespace {

struct DecodeArgs {
    const int32_t* idx1;    // [B][hkv][s2] the token's leg-1 row
    const float* w1;
    const int32_t* idx2;    // [B][T][hkv][s3] edge cache (leg 2)
    const float* w2;
    const void* q;          // [B][hq][d]
    const void* k;          // [B][T][hkv][d]
    const void* v;
    int32_t* idx_out;       // [B][hkv][s1]
    float* w_out;
    void* o;                // [B][hq][d]
    int B, T, hq, hkv, d, s1, s2, s3;
    float scale;
};

// sum over the wavefront: DPP inside each 16-lane row, then the rows
// combined with the permlane swaps (no LDS round trip)
template <typename A>
__device__ __forceinline__ A wave_sum(A x) {
    x = row_sum16(x);
    A a = x, b = x;
    swap16(a, b);
    x = a + b;
    a = x;
    b = x;
    swap32(a, b);
    return a + b;
}

// value of lane k (k uniform): v_readlane, no LDS round trip
__device__ __forceinline__ int lane_i(int x, int k) { return __builtin_amdgcn_readlane(x, k); }
__device__ __forceinline__ float lane_f(float x, int k) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), k));
}
__device__ __forceinline__ double lane_d(double x, int k) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, k);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), k);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

template <typename T, int G>
__global__ __launch_bounds__(kWave) void decode_kernel(DecodeArgs a) {
    using A = typename io<T>::acc;
    constexpr int V = io<T>::V;            // elements per 16-byte piece
    const int unit = (int)blockIdx.x;       // b * hkv + h
    const int b = unit / a.hkv, h = unit - (unit / a.hkv) * a.hkv;
    const int lane = (int)threadIdx.x;
    const int nc = a.s2 * a.s3;
    const int R = a.d / V;                  // 16-byte pieces per d-row (<= 64)
    const bool piece = lane < R;

    // the token's query rows (independent of SER: in flight meanwhile)
    const T* qb = static_cast<const T*>(a.q) + ((size_t)b * a.hq + (size_t)h * G) * a.d;
    A qf[G][V];
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int e = 0; e < V; ++e) qf[g][e] = 0;
        if (piece) load16(qb + (size_t)g * a.d + lane * V, qf[g]);
    }

    // SER: lane k < s2*s3 holds path k = (a, c)
    int m = -1;
    double cw = 0.0;
    if (lane < nc) {
        const int aa = lane / a.s3, c = lane - (lane / a.s3) * a.s3;
        const int j = a.idx1[(size_t)unit * a.s2 + aa];
        const float x = a.w1[(size_t)unit * a.s2 + aa];
        const size_t r2 = ((size_t)b * a.T + j) * a.hkv + h;
        m = a.idx2[r2 * a.s3 + c];
        cw = (double)x * (double)a.w2[r2 * a.s3 + c];
    }
    float key;
    bool cand;
    int rank = 0;
    if (nc <= 16) {
        // up to 16 candidates: DPP rotations inside the first 16-lane row
        team16_merge_rank(lane & 15, m, cw, lane < nc, key, cand, rank);
    } else {
        // merge: the first lane of a target sums its later lanes in path order
        double acc = cw;
        bool dup = false;
        for (int k2 = 0; k2 < nc; ++k2) {
            const int mk = lane_i(m, k2);
            const double ck = lane_d(cw, k2);
            if (mk == m) {
                if (k2 < lane) dup = true;
                if (k2 > lane) acc += ck;
            }
        }
        key = (float)acc;
        cand = lane < nc && !dup && key > 0.0f;
        // rank among the candidates: larger weight first, then the lower target
        const uint64_t cm = __ballot(cand);
        for (int k2 = 0; k2 < nc; ++k2) {
            if (!((cm >> k2) & 1)) continue;
            const float kk = lane_f(key, k2);
            const int mk = lane_i(m, k2);
            if (kk > key || (kk == key && mk < m)) ++rank;
        }
    }
    const uint64_t cmask = __ballot(cand);
    const size_t ob = (size_t)unit * a.s1;
    if (cand && rank < a.s1) {
        a.idx_out[ob + rank] = m;
        a.w_out[ob + rank] = key;
    }
    const int ncand = __popcll(cmask);
    for (int r = ncand + lane; r < a.s1; r += kWave) {
        a.idx_out[ob + r] = 0;
        a.w_out[ob + r] = 0.0f;
    }
    const int live = ncand < a.s1 ? ncand : a.s1;

    // SEA over the live slots (slot r = the lane of rank r), four slots per
    // step with their K and V pieces loaded together, online softmax per head
    const T* kb = static_cast<const T*>(a.k);
    const T* vb = static_cast<const T*>(a.v);
    const A c = (A)a.scale * (A)1.4426950408889634;   // scale * log2(e)
    A M[G], Z[G], ov[G][V];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        M[g] = -INFINITY;
        Z[g] = 0;
#pragma unroll
        for (int e = 0; e < V; ++e) ov[g][e] = 0;
    }
    for (int r0 = 0; r0 < live; r0 += 4) {
        A kf[4][V], vf[4][V], lw[4];
        bool on[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = r0 + u;
            on[u] = r < live;
#pragma unroll
            for (int e = 0; e < V; ++e) { kf[u][e] = 0; vf[u][e] = 0; }
            lw[u] = 0;
            if (on[u]) {
                const int src = __ffsll(__ballot(cand && rank == r)) - 1;
                const int j = lane_i(m, src);
                lw[u] = alog2((A)lane_f(key, src));
                const size_t kr = (((size_t)b * a.T + j) * a.hkv + h) * a.d + (size_t)lane * V;
                if (piece) {
                    load16(kb + kr, kf[u]);
                    load16(vb + kr, vf[u]);
                }
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (!on[u]) continue;
                A dot = 0;
#pragma unroll
                for (int e = 0; e < V; ++e) dot += qf[g][e] * kf[u][e];
                const A l = wave_sum(dot) * c + lw[u];
                const A Mn = l > M[g] ? l : M[g];
                const A alpha = aexp2(M[g] - Mn);   // 0 on the first slot (M = -inf)
                const A p = aexp2(l - Mn);
                Z[g] = Z[g] * alpha + p;
#pragma unroll
                for (int e = 0; e < V; ++e) ov[g][e] = ov[g][e] * alpha + p * vf[u][e];
                M[g] = Mn;
            }
        }
    }
    T* obase = static_cast<T*>(a.o) + ((size_t)b * a.hq + (size_t)h * G) * a.d;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const A inv = Z[g] > (A)0 ? (A)1 / Z[g] : (A)0;
        A y[V];
#pragma unroll
        for (int e = 0; e < V; ++e) y[e] = ov[g][e] * inv;
        if (piece) store_n<V>(obase + (size_t)g * a.d + lane * V, y);
    }
}

// bf16, d = 128, at most 16 candidate paths: the K/V rows of every
// candidate are loaded while SER merges and ranks them, so the kept slots'
// rows are already in registers when the ranking ends (the K/V round trip
// overlaps the ranking instead of following it).  Lanes form four 16-lane rows; row g holds
// piece r = lane % 16 (16 bytes) of candidates g, g + 4, g + 8, g + 12.
// Scores of all candidates are 16-lane sums; the softmax runs over the kept
// ones (the others get probability 0) and the rows' partial outputs are
// added with the permlane swaps.
template <int G>
__global__ __launch_bounds__(kWave) void decode16_kernel(DecodeArgs a) {
    const int unit = (int)blockIdx.x;       // b * hkv + h
    const int b = unit / a.hkv, h = unit - (unit / a.hkv) * a.hkv;
    const int lane = (int)threadIdx.x;
    const int grp = lane >> 4, r = lane & 15;
    const int nc = a.s2 * a.s3;             // <= 16
    const bf16_t* qb = static_cast<const bf16_t*>(a.q) + ((size_t)b * a.hq + (size_t)h * G) * 128;
    float qf[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) load16(qb + (size_t)g * 128 + r * 8, qf[g]);

    // SER candidates: lane k < nc holds path k = (slot a, slot c)
    int m = -1;
    double cw = 0.0;
    if (lane < nc) {
        const int aa = lane / a.s3, c = lane - (lane / a.s3) * a.s3;
        const int j = a.idx1[(size_t)unit * a.s2 + aa];
        const float x = a.w1[(size_t)unit * a.s2 + aa];
        const size_t r2 = ((size_t)b * a.T + j) * a.hkv + h;
        m = a.idx2[r2 * a.s3 + c];
        cw = (double)x * (double)a.w2[r2 * a.s3 + c];
    }
    // every candidate's K/V rows, before the merge: row grp takes candidates
    // grp + 4i (a clamped row for missing ones, masked below)
    const bf16_t* kb = static_cast<const bf16_t*>(a.k);
    const bf16_t* vb = static_cast<const bf16_t*>(a.v);
    uint4 kr[4], vr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = grp + 4 * i;
        const int mc = __shfl(m, c, kWave);
        // clamped into the cache: a candidate that is never kept (a dead or
        // padding slot) may carry any index
        const int j = c < nc ? (mc < 0 ? 0 : mc < a.T ? mc : a.T - 1) : 0;
        const size_t row = (((size_t)b * a.T + j) * a.hkv + h) * 128 + (size_t)r * 8;
        kr[i] = *reinterpret_cast<const uint4*>(kb + row);
        vr[i] = *reinterpret_cast<const uint4*>(vb + row);
    }
    // merge and rank by DPP rotations inside the first 16-lane row (the
    // candidates' lanes; the other rows sweep their own, unused, lanes):
    // the same sums in the same order as decode_kernel's lane sweeps
    float key;
    bool cand;
    int rank;
    team16_merge_rank(lane & 15, m, cw, lane < nc, key, cand, rank);
    const uint64_t cmask = __ballot(cand);
    const size_t ob = (size_t)unit * a.s1;
    if (cand && rank < a.s1) {
        a.idx_out[ob + rank] = m;
        a.w_out[ob + rank] = key;
    }
    const int ncand = __popcll(cmask);
    for (int rr = ncand + lane; rr < a.s1; rr += kWave) {
        a.idx_out[ob + rr] = 0;
        a.w_out[ob + rr] = 0.0f;
    }

    // SEA over the kept candidates (probability 0 for the rest)
    const float cs = a.scale * 1.4426950408889634f;   // scale * log2(e)
    const bool keep = cand && rank < a.s1;
    const float lwk = keep ? alog2(key) : 0.0f;
    float lg[4][G];
    bool on[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = grp + 4 * i;
        on[i] = __shfl((int)keep, c, kWave) != 0;
        const float lw = __shfl(lwk, c, kWave);
        float kf[8];
        bf16x8_to_f32(kr[i], kf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float dot = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) dot += qf[g][e] * kf[e];
            dot = row_sum16(dot);
            lg[i][g] = on[i] ? dot * cs + lw : -INFINITY;
        }
    }
    bf16_t* obase = static_cast<bf16_t*>(a.o) + ((size_t)b * a.hq + (size_t)h * G) * 128;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float mx = fmaxf(fmaxf(lg[0][g], lg[1][g]), fmaxf(lg[2][g], lg[3][g]));
        {
            float x0 = mx, x1 = mx;
            swap16(x0, x1);
            mx = fmaxf(x0, x1);
            x0 = mx; x1 = mx;
            swap32(x0, x1);
            mx = fmaxf(x0, x1);
        }
        float z = 0.0f, y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float pr = on[i] ? aexp2(lg[i][g] - mx) : 0.0f;
            float vf[8];
            bf16x8_to_f32(vr[i], vf);
            z += pr;
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] += pr * vf[e];
        }
        // z is the same in the 16 lanes of a row: add the four rows
        {
            float x0 = z, x1 = z;
            swap16(x0, x1);
            z = x0 + x1;
            x0 = z; x1 = z;
            swap32(x0, x1);
            z = x0 + x1;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x0 = y[e], x1 = y[e];
            swap16(x0, x1);
            y[e] = x0 + x1;
            x0 = y[e]; x1 = y[e];
            swap32(x0, x1);
            y[e] = x0 + x1;
        }
        const float inv = z > 0.0f ? 1.0f / z : 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] *= inv;
        if (grp == 0) store_n<8>(obase + (size_t)g * 128 + r * 8, y);
    }
}

}  // namespace

hipError_t launch_decode_step(int B, int T, int hq, int hkv, int d, bool bf16, float scale,
                              const int32_t* idx1, const float* w1, int s2,
                              const int32_t* idx2, const float* w2, int s3, int s1,
                              const void* q, const void* k, const void* v, int32_t* idx_out,
                              float* w_out, void* o, hipStream_t st) {
    DecodeArgs a{idx1, w1, idx2, w2, q, k, v, idx_out, w_out, o,
                 B, T, hq, hkv, d, s1, s2, s3, scale};
    const dim3 grid((unsigned)(B * hkv));
    if (bf16 && d == 128 && s2 * s3 <= 16 && (hq / hkv == 1 || hq / hkv == 2 || hq / hkv == 4)) {
        switch (hq / hkv) {
            case 1: hipLaunchKernelGGL((decode16_kernel<1>), grid, dim3(kWave), 0, st, a); break;
            case 2: hipLaunchKernelGGL((decode16_kernel<2>), grid, dim3(kWave), 0, st, a); break;
            default: hipLaunchKernelGGL((decode16_kernel<4>), grid, dim3(kWave), 0, st, a); break;
        }
        return hipGetLastError();
    }
    auto go = [&](auto tag) {
        using T = decltype(tag);
        switch (hq / hkv) {
            case 1: hipLaunchKernelGGL((decode_kernel<T, 1>), grid, dim3(kWave), 0, st, a); break;
            case 2: hipLaunchKernelGGL((decode_kernel<T, 2>), grid, dim3(kWave), 0, st, a); break;
            case 4: hipLaunchKernelGGL((decode_kernel<T, 4>), grid, dim3(kWave), 0, st, a); break;
            case 8: hipLaunchKernelGGL((decode_kernel<T, 8>), grid, dim3(kWave), 0, st, a); break;
            case 16:
                hipLaunchKernelGGL((decode_kernel<T, 16>), grid, dim3(kWave), 0, st, a);
                break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    };
    return bf16 ? go(bf16_t{}) : go(float{});
}

}  // namespace gm
