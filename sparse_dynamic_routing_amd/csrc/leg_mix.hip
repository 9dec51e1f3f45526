// Leg construction: a token's K stored edges mixed into one leg and
// sparsified (page "Graph Machine: Towards Better Pretraining via Edges",
// ai.info, Methodology, referral paragraph: the stored edges are mixed into
// pairs and each leg is sparsified before the legs are composed).  The
// mixing is a reading: leg weight of target m = sum over the stored slots k
// pointing at m of alpha[h][k] * w[k], merged in slot order in fp64, then
// SER's selection (top s by fp32 weight, ties to the lower index, (0, 0)
// padding).
//
// Forward, K = 16 with 16-byte aligned rows and s = 4 or 2: one lane per
// unit, SER's register network (below).  Otherwise a team of
// L = max(16, pow2(K)) lanes per unit, lane k holding
// stored slot k; the first lane of each target sums the later lanes of that
// target in slot order (the definition's order and precision, so the
// weights are bit-identical to the oracle's), and each candidate's rank
// comes from one sweep over the team (DPP row rotations for 16-lane teams,
// shuffles for wider ones).
// Backward: the same teams, each lane matching its slot against the leg's
// retained slots: dw = alpha * dleg (own row, no scatter); dalpha sums
// w * dleg over every unit of a KV head: each workgroup reduces its units
// (one head, 64 tokens) in a fixed order into a partial, and a second
// kernel adds the partials in a fixed order and rounds once (deterministic).
#include "gm_common.h"
#include "gm_internal.h"
#include "gm_select.h"

#include <utility>

namespace gm {
namespace {

constexpr int kLegTokens = 64;   // tokens of one KV head per backward workgroup

struct LegArgs {
    const int32_t* idx;     // [B][n][hkv][K] stored edges
    const float* w;
    const float* alpha;     // [hkv][K]
    int32_t* idx_out;       // [B][n][hkv][s] the leg
    float* w_out;
    const float* dleg;      // backward: [B][n][hkv][s]
    float* dw;              // backward: [B][n][hkv][K]
    float* dalpha;          // backward: [hkv][K]
    double* part;           // backward: [hkv][nchunk][K]
    int n, hkv, K, s, U, BN, nchunk;
};

template <int L>
__global__ __launch_bounds__(kBlock) void leg_mix_fwd_kernel(LegArgs a) {
    const int lane = (int)(threadIdx.x & (kWave - 1));
    const int k = lane & (L - 1);
    const long long gu = ((long long)blockIdx.x * kBlock + threadIdx.x) / L;
    const bool in = gu < a.U;
    const int u = in ? (int)gu : 0;
    const int h = u % a.hkv;
    const int base = lane & ~(L - 1);      // the team's first lane
    int m = -1;
    double cw = 0.0;
    if (in && k < a.K) {
        m = a.idx[(size_t)u * a.K + k];
        cw = (double)a.alpha[(size_t)h * a.K + k] * (double)a.w[(size_t)u * a.K + k];
    }
    double acc = cw;
    bool dup = false;
    float key;
    bool cand;
    int rank = 0;
    if constexpr (L == 16) {
        // 16-lane rows: DPP rotations (every lane of the wave takes part,
        // so no lane leaves before the sweeps)
        team16_merge_rank(k, m, cw, in && k < a.K, key, cand, rank);
    } else {
        for (int k2 = 0; k2 < a.K; ++k2) {
            const int mk = __shfl(m, k2, L);
            const double ck = __shfl(cw, k2, L);
            if (mk == m) {
                if (k2 < k) dup = true;
                if (k2 > k) acc += ck;
            }
        }
        key = (float)acc;
        cand = in && k < a.K && !dup && key > 0.0f;
        for (int k2 = 0; k2 < a.K; ++k2) {
            const float kk = __shfl(key, k2, L);
            const int mk = __shfl(m, k2, L);
            const bool ck = __shfl((int)cand, k2, L) != 0;
            if (ck && (kk > key || (kk == key && mk < m))) ++rank;
        }
    }
    if (!in) return;
    const size_t ob = (size_t)u * a.s;
    if (cand && rank < a.s) {
        a.idx_out[ob + rank] = m;
        a.w_out[ob + rank] = key;
    }
    const uint64_t team = L == kWave ? ~0ull : ((1ull << L) - 1) << base;
    const int ncand = __popcll(__ballot(cand) & team);
    for (int r = ncand + k; r < a.s; r += L) {
        a.idx_out[ob + r] = 0;
        a.w_out[ob + r] = 0.0f;
    }
}

// workgroup (h, chunk): the units (t, h) for the kLegTokens flattened tokens
// t = b * n + i of the chunk; every thread of a team walks them in steps of
// the workgroup's team count and keeps its slot's w * dleg sum in fp64
template <int L>
__global__ __launch_bounds__(kBlock) void leg_mix_bwd_kernel(LegArgs a) {
    constexpr int kTeams = kBlock / L;
    __shared__ double red[kTeams][L];
    const int h = (int)blockIdx.x / a.nchunk, chunk = (int)blockIdx.x % a.nchunk;
    const int team = (int)threadIdx.x / L, k = (int)threadIdx.x & (L - 1);
    const float al = k < a.K ? a.alpha[(size_t)h * a.K + k] : 0.0f;
    double da = 0.0;
    const int t0 = chunk * kLegTokens;
    const int t1 = t0 + kLegTokens < a.BN ? t0 + kLegTokens : a.BN;
    for (int t = t0 + team; t < t1; t += kTeams) {
        const int u = t * a.hkv + h;
        if (k >= a.K) continue;
        const int m = a.idx[(size_t)u * a.K + k];
        const float x = a.w[(size_t)u * a.K + k];
        double g = 0.0;
        if (al > 0.0f && x > 0.0f) {
            const size_t ob = (size_t)u * a.s;
            for (int r = 0; r < a.s; ++r)
                if (a.w_out[ob + r] > 0.0f && a.idx_out[ob + r] == m) g += (double)a.dleg[ob + r];
        }
        a.dw[(size_t)u * a.K + k] = (float)(g * (double)al);
        da += g * (double)x;
    }
    red[team][k] = da;
    __syncthreads();
    if ((int)threadIdx.x < L && (int)threadIdx.x < a.K) {
        double s = 0.0;
        for (int q = 0; q < kTeams; ++q) s += red[q][threadIdx.x];
        a.part[((size_t)h * a.nchunk + chunk) * a.K + threadIdx.x] = s;
    }
}

// dalpha[h][k]: one wavefront per element; lane l adds chunks l, l + 64, ...
// into four running sums in a fixed pattern, then a fixed butterfly over the
// lanes; rounded once
__global__ __launch_bounds__(kBlock) void leg_mix_alpha_kernel(LegArgs a) {
    const int e = (int)((blockIdx.x * kBlock + threadIdx.x) / kWave);
    const int lane = (int)(threadIdx.x & (kWave - 1));
    if (e >= a.hkv * a.K) return;          // whole wavefronts
    const int h = e / a.K, k = e - (e / a.K) * a.K;
    // four independent running sums (loads in flight together), combined in
    // a fixed order
    const double* pr = a.part + (size_t)h * a.nchunk * a.K + k;
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    int c = lane;
    for (; c + 3 * kWave < a.nchunk; c += 4 * kWave) {
        s0 += pr[(size_t)c * a.K];
        s1 += pr[(size_t)(c + kWave) * a.K];
        s2 += pr[(size_t)(c + 2 * kWave) * a.K];
        s3 += pr[(size_t)(c + 3 * kWave) * a.K];
    }
    for (; c < a.nchunk; c += kWave) s0 += pr[(size_t)c * a.K];
    double s = (s0 + s1) + (s2 + s3);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) s += __shfl_xor(s, o, kWave);
    if (lane == 0) a.dalpha[e] = (float)s;
}

// K = 16 stored slots with 16-byte aligned rows: one lane per unit, the
// whole row in registers (four 16-byte loads each of idx, w and the head's
// alpha), merged and ranked as in SER's forward (sorting network of
// gm_select.h); units chunked per XCD as SER's are.  Same arithmetic and
// order as the team kernel, so the same bits.
template <int S>
__global__ __launch_bounds__(kBlock) void leg_mix_vec_kernel(LegArgs a) {
    static_assert(S == 2 || S == 4, "vector stores of 2 or 4 slots");
    const int u = xcd_unit(a.U);
    if (u < 0) return;
    const int h = u % a.hkv;
    int m[16];
    double cw[16];
    const int4* ir = reinterpret_cast<const int4*>(a.idx + (size_t)u * 16);
    const float4* wr = reinterpret_cast<const float4*>(a.w + (size_t)u * 16);
    const float4* ar = reinterpret_cast<const float4*>(a.alpha + (size_t)h * 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int4 i4 = ir[q];
        const float4 w4 = wr[q], a4 = ar[q];
        m[4 * q + 0] = i4.x; m[4 * q + 1] = i4.y; m[4 * q + 2] = i4.z; m[4 * q + 3] = i4.w;
        cw[4 * q + 0] = (double)a4.x * (double)w4.x;
        cw[4 * q + 1] = (double)a4.y * (double)w4.y;
        cw[4 * q + 2] = (double)a4.z * (double)w4.z;
        cw[4 * q + 3] = (double)a4.w * (double)w4.w;
    }
    // the merge and selection of SER's forward, written out here as there
    // (98 registers; the same code as a shared inline function compiled to
    // 256 registers and one wavefront per SIMD): a candidate that repeats an
    // earlier target gets bit 31 of its target set and drops out, its weight
    // added to the target's first candidate in slot order
    double acc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = cw[k];
#pragma unroll
    for (int k = 1; k < 16; ++k) {
        uint32_t dup = 0;
#pragma unroll
        for (int k2 = 0; k2 < k; ++k2) {
            const bool same = m[k2] == m[k];
            acc[k2] += same ? cw[k] : 0.0;
            dup |= same ? 0x80000000u : 0u;
        }
        m[k] = (int)((uint32_t)m[k] | dup);
    }
    uint64_t key[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
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
    if constexpr (S == 4) {
        *reinterpret_cast<int4*>(a.idx_out + (size_t)u * 4) = make_int4(om[0], om[1], om[2], om[3]);
        *reinterpret_cast<float4*>(a.w_out + (size_t)u * 4) =
            make_float4(ow[0], ow[1], ow[2], ow[3]);
    } else {
        *reinterpret_cast<int2*>(a.idx_out + (size_t)u * 2) = make_int2(om[0], om[1]);
        *reinterpret_cast<float2*>(a.w_out + (size_t)u * 2) = make_float2(ow[0], ow[1]);
    }
}

// Backward for the same shapes: one lane per unit (u = workgroup * 256 +
// thread), its stored row, the head's alpha and its leg row in registers.
// g_k = sum of dleg over the retained leg slots with index m_k (fp64, slot
// order); dw_k = g_k * alpha_k; the unit's dalpha terms w_k * g_k go to LDS,
// and threads (h, k) add them over the workgroup's units of head h in unit
// order into the partial of (h, workgroup, k), written for every head (0 if
// the workgroup has none of its units); leg_mix_alpha_kernel then adds the
// partials in workgroup order.  Deterministic.
template <int S>
__global__ __launch_bounds__(kBlock) void leg_mix_bwd_vec_kernel(LegArgs a) {
    __shared__ double red[kBlock][17];   // 16 terms per unit, padded row
    const int u0 = (int)blockIdx.x * kBlock;
    const int u = u0 + (int)threadIdx.x;
    const bool in = u < a.U;
    double c[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) c[k] = 0.0;
    if (in) {
        const int h = u % a.hkv;
        int m[16];
        float x[16], al[16];
        const int4* ir = reinterpret_cast<const int4*>(a.idx + (size_t)u * 16);
        const float4* wr = reinterpret_cast<const float4*>(a.w + (size_t)u * 16);
        const float4* ar = reinterpret_cast<const float4*>(a.alpha + (size_t)h * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int4 i4 = ir[q];
            const float4 w4 = wr[q], a4 = ar[q];
            m[4 * q + 0] = i4.x; m[4 * q + 1] = i4.y; m[4 * q + 2] = i4.z; m[4 * q + 3] = i4.w;
            x[4 * q + 0] = w4.x; x[4 * q + 1] = w4.y; x[4 * q + 2] = w4.z; x[4 * q + 3] = w4.w;
            al[4 * q + 0] = a4.x; al[4 * q + 1] = a4.y; al[4 * q + 2] = a4.z; al[4 * q + 3] = a4.w;
        }
        int om[4];
        float ow[4], og[4];
        if constexpr (S == 4) {
            const int4 i4 = *reinterpret_cast<const int4*>(a.idx_out + (size_t)u * 4);
            const float4 w4 = *reinterpret_cast<const float4*>(a.w_out + (size_t)u * 4);
            const float4 g4 = *reinterpret_cast<const float4*>(a.dleg + (size_t)u * 4);
            om[0] = i4.x; om[1] = i4.y; om[2] = i4.z; om[3] = i4.w;
            ow[0] = w4.x; ow[1] = w4.y; ow[2] = w4.z; ow[3] = w4.w;
            og[0] = g4.x; og[1] = g4.y; og[2] = g4.z; og[3] = g4.w;
        } else {
            const int2 i2 = *reinterpret_cast<const int2*>(a.idx_out + (size_t)u * 2);
            const float2 w2 = *reinterpret_cast<const float2*>(a.w_out + (size_t)u * 2);
            const float2 g2 = *reinterpret_cast<const float2*>(a.dleg + (size_t)u * 2);
            om[0] = i2.x; om[1] = i2.y; om[2] = 0; om[3] = 0;
            ow[0] = w2.x; ow[1] = w2.y; ow[2] = 0.0f; ow[3] = 0.0f;
            og[0] = g2.x; og[1] = g2.y; og[2] = 0.0f; og[3] = 0.0f;
        }
        float dwv[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            double g = 0.0;
#pragma unroll
            for (int t = 0; t < S; ++t) g += ow[t] > 0.0f && om[t] == m[k] ? (double)og[t] : 0.0;
            const bool on = al[k] > 0.0f && x[k] > 0.0f;
            dwv[k] = on ? (float)(g * (double)al[k]) : 0.0f;
            c[k] = on ? g * (double)x[k] : 0.0;
        }
        float4* dr = reinterpret_cast<float4*>(a.dw + (size_t)u * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            dr[q] = make_float4(dwv[4 * q], dwv[4 * q + 1], dwv[4 * q + 2], dwv[4 * q + 3]);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) red[threadIdx.x][k] = c[k];
    __syncthreads();
    // partial of (h, k): units u0 + l with (u0 + l) % hkv == h, in order
    for (int e = (int)threadIdx.x; e < a.hkv * 16; e += kBlock) {
        const int h = e / 16, k = e - (e / 16) * 16;
        int l = h - u0 % a.hkv;
        if (l < 0) l += a.hkv;
        double sum = 0.0;
        for (; l < kBlock; l += a.hkv) sum += red[l][k];
        a.part[((size_t)h * a.nchunk + blockIdx.x) * 16 + k] = sum;
    }
}

template <int L>
void launch_fwd(const LegArgs& a, hipStream_t st) {
    const long long threads = (long long)a.U * L;
    hipLaunchKernelGGL(leg_mix_fwd_kernel<L>, dim3((unsigned)((threads + kBlock - 1) / kBlock)),
                       dim3(kBlock), 0, st, a);
}

template <int L>
void launch_bwd(const LegArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(leg_mix_bwd_kernel<L>, dim3((unsigned)(a.hkv * a.nchunk)), dim3(kBlock),
                       0, st, a);
    const long long lanes = (long long)a.hkv * a.K * kWave;
    hipLaunchKernelGGL(leg_mix_alpha_kernel, dim3((unsigned)((lanes + kBlock - 1) / kBlock)),
                       dim3(kBlock), 0, st, a);
}

// K = 16, s = 4 or 2, every row 16-byte aligned: the lane-per-unit kernels
bool lane_rows(const LegArgs& a, bool fwd) {
    // stored rows, alpha and dw: 16-byte loads / stores; leg rows: s * 4 bytes
    uintptr_t rows = (uintptr_t)a.idx | (uintptr_t)a.w | (uintptr_t)a.alpha;
    uintptr_t legs = (uintptr_t)a.idx_out | (uintptr_t)a.w_out;
    if (!fwd) {
        rows |= (uintptr_t)a.dw;
        legs |= (uintptr_t)a.dleg;
    }
    return a.K == 16 && (a.s == 4 || a.s == 2) && rows % 16 == 0 &&
           legs % (uintptr_t)(a.s * 4) == 0;
}

template <bool FWD>
hipError_t dispatch(const LegArgs& a, hipStream_t st) {
    const bool rows16 = lane_rows(a, FWD);
    if (!FWD && rows16) {
        const dim3 grid((unsigned)((a.U + kBlock - 1) / kBlock));
        if (a.s == 4)
            hipLaunchKernelGGL(leg_mix_bwd_vec_kernel<4>, grid, dim3(kBlock), 0, st, a);
        else
            hipLaunchKernelGGL(leg_mix_bwd_vec_kernel<2>, grid, dim3(kBlock), 0, st, a);
        const long long lanes = (long long)a.hkv * a.K * kWave;
        hipLaunchKernelGGL(leg_mix_alpha_kernel, dim3((unsigned)((lanes + kBlock - 1) / kBlock)),
                           dim3(kBlock), 0, st, a);
        return hipGetLastError();
    }
    if (FWD && rows16) {   // lane per unit
        if (a.s == 4)
            hipLaunchKernelGGL(leg_mix_vec_kernel<4>, dim3(xcd_unit_grid(a.U)), dim3(kBlock), 0,
                               st, a);
        else
            hipLaunchKernelGGL(leg_mix_vec_kernel<2>, dim3(xcd_unit_grid(a.U)), dim3(kBlock), 0,
                               st, a);
        return hipGetLastError();
    }
    if (FWD && a.K <= 16) {   // 16-lane teams: the DPP sweeps
        launch_fwd<16>(a, st);
        return hipGetLastError();
    }
    switch (pow2_ceil(a.K)) {
        case 1: FWD ? launch_fwd<1>(a, st) : launch_bwd<1>(a, st); break;
        case 2: FWD ? launch_fwd<2>(a, st) : launch_bwd<2>(a, st); break;
        case 4: FWD ? launch_fwd<4>(a, st) : launch_bwd<4>(a, st); break;
        case 8: FWD ? launch_fwd<8>(a, st) : launch_bwd<8>(a, st); break;
        case 16: FWD ? launch_fwd<16>(a, st) : launch_bwd<16>(a, st); break;
        case 32: FWD ? launch_fwd<32>(a, st) : launch_bwd<32>(a, st); break;
        case 64: FWD ? launch_fwd<64>(a, st) : launch_bwd<64>(a, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

// fp64 partials of dalpha: [hkv][chunks][K], chunks of 64 tokens of one head
// (team kernels) or, for K = 16, of 256 units (lane-per-unit kernel),
// whichever is more
size_t leg_mix_backward_workspace_bytes(int B, int n, int hkv, int K) {
    long long chunks = ((long long)B * n + kLegTokens - 1) / kLegTokens;
    if (K == 16) {
        const long long wgs = ((long long)B * n * hkv + kBlock - 1) / kBlock;
        if (wgs > chunks) chunks = wgs;
    }
    return (size_t)hkv * (size_t)chunks * (size_t)K * sizeof(double);
}

hipError_t launch_leg_mix_forward(int B, int n, int hkv, const int32_t* idx, const float* w,
                                  int K, const float* alpha, int s, int32_t* idx_out,
                                  float* w_out, hipStream_t st) {
    LegArgs a{};
    a.idx = idx; a.w = w; a.alpha = alpha; a.idx_out = idx_out; a.w_out = w_out;
    a.n = n; a.hkv = hkv; a.K = K; a.s = s; a.U = B * n * hkv; a.BN = B * n;
    return dispatch<true>(a, st);
}

hipError_t launch_leg_mix_backward(int B, int n, int hkv, const int32_t* idx, const float* w,
                                   int K, const float* alpha, const int32_t* idx_out,
                                   const float* w_out, int s, const float* dleg, float* dw,
                                   float* dalpha, double* part, hipStream_t st) {
    LegArgs a{};
    a.idx = idx; a.w = w; a.alpha = alpha; a.idx_out = const_cast<int32_t*>(idx_out);
    a.w_out = const_cast<float*>(w_out); a.dleg = dleg; a.dw = dw; a.dalpha = dalpha;
    a.part = part;
    a.n = n; a.hkv = hkv; a.K = K; a.s = s; a.U = B * n * hkv; a.BN = B * n;
    a.nchunk = lane_rows(a, false) ? (a.U + kBlock - 1) / kBlock
                                   : (a.BN + kLegTokens - 1) / kLegTokens;
    return dispatch<false>(a, st);
}

}  // namespace gm
