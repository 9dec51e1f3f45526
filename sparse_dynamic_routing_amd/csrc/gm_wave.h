// Wave64 building blocks for the gfx950 fast paths.  One d-row of K/V/q
// (256 bytes: bf16 d=128 or fp32 d=64) is spread over one 16-lane row of the
// wavefront (16 bytes per lane).  The forward and the source pass hold one
// unit per row and its edge slots in registers; the target pass puts the
// P <= 4 incoming edges of a unit in consecutive rows.  Sums inside a row
// use DPP (the permute is fused into the add); reductions across rows use
// gfx950's v_permlane16_swap / v_permlane32_swap, so no LDS traffic and no
// lane-address arithmetic are needed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gm_common.h"

namespace gm {

// DPP controls (gfx9 encoding).
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i inside each 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i inside each 16

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Lane L of each 16-lane row, to every lane of that row.
template <int L>
__device__ __forceinline__ float row_bcast(float x) {
    return dpp<0x150 + L>(x);
}

// Sum / max over the 16 lanes of each row; every lane gets the result.
template <typename A>
__device__ __forceinline__ A row_sum16(A x) {
    x += dpp<kDppXor1>(x);
    x += dpp<kDppXor2>(x);
    x += dpp<kDppHalfMirror>(x);
    x += dpp<kDppMirror>(x);
    return x;
}

// Cross-row swaps.  swap16(a, b): odd rows of a trade places with even rows
// of b; swap32(a, b): the upper 32 lanes of a trade with the lower 32 of b.
__device__ __forceinline__ void swap16(float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, a),
                                                    __builtin_bit_cast(uint32_t, b), false, false);
    a = __builtin_bit_cast(float, (uint32_t)r[0]);
    b = __builtin_bit_cast(float, (uint32_t)r[1]);
}
__device__ __forceinline__ void swap32(float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a),
                                                    __builtin_bit_cast(uint32_t, b), false, false);
    a = __builtin_bit_cast(float, (uint32_t)r[0]);
    b = __builtin_bit_cast(float, (uint32_t)r[1]);
}
__device__ __forceinline__ void swap16(double& a, double& b) {
    uint64_t ua = __builtin_bit_cast(uint64_t, a), ub = __builtin_bit_cast(uint64_t, b);
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)ua, (uint32_t)ub, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(ua >> 32), (uint32_t)(ub >> 32),
                                                     false, false);
    a = __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi[0] << 32) | (uint32_t)lo[0]);
    b = __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi[1] << 32) | (uint32_t)lo[1]);
}
__device__ __forceinline__ void swap32(double& a, double& b) {
    uint64_t ua = __builtin_bit_cast(uint64_t, a), ub = __builtin_bit_cast(uint64_t, b);
    const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)ua, (uint32_t)ub, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(ua >> 32), (uint32_t)(ub >> 32),
                                                     false, false);
    a = __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi[0] << 32) | (uint32_t)lo[0]);
    b = __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi[1] << 32) | (uint32_t)lo[1]);
}

// Reduce-scatter a V-vector over the P rows of a team.  Afterwards x[0 .. V/P)
// holds the sums of elements [off, off + V/P) of the vector, with
// off = rs_offset<V, P>(row); V >= P.
template <int P, int V, typename A>
__device__ __forceinline__ void rows_reduce_scatter(A (&x)[V]) {
    if constexpr (P >= 2) {
        constexpr int h = V / 2;
#pragma unroll
        for (int e = 0; e < h; ++e) {
            swap16(x[e], x[e + h]);
            x[e] += x[e + h];
        }
    }
    if constexpr (P >= 4) {
        constexpr int h = V / 4;
#pragma unroll
        for (int e = 0; e < h; ++e) {
            swap32(x[e], x[e + h]);
            x[e] += x[e + h];
        }
    }
}
template <int V, int P>
__device__ __forceinline__ int rs_offset(int row) {
    int off = 0;
    if constexpr (P >= 2) off += (row & 1) * (V / 2);
    if constexpr (P >= 4) off += ((row >> 1) & 1) * (V / 4);
    return off;
}

// Division of 0 <= x < 2^31 by an invariant divisor 1 <= d < 2^31 with a
// multiply-high, add and shift (Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994): with l = ceil(log2 d),
// m = floor(2^32 (2^l - d) / d) + 1, q = (mulhi(m, x) + x) >> l.
struct FastDiv {
    uint32_t d, m, l;
};
inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    f.l = 0;
    while ((1ull << f.l) < d) ++f.l;
    f.m = (uint32_t)((((1ull << 32) * ((1ull << f.l) - d)) / d) + 1);
    return f;
}
__device__ __forceinline__ uint32_t fdiv(uint32_t x, const FastDiv& f) {
    return (__umulhi(f.m, x) + x) >> f.l;
}

// XCD-aware persistent schedule over units (or K/V rows) of B*hkv (batch,
// KV head) pairs of n tokens.  Each pair is cut into S = 2^lgS segments of
// L = n / S tokens (S > 1 only when there are few pairs), and segment k goes
// to XCD k % 8: workgroups are dealt to the 8 XCDs round robin, so XCD x runs
// workgroups x, x+8, ... and takes segments x, x+8, ... in that order.  The
// XCD's teams walk its items side by side, team t taking items t, t+T, ...
// (T teams on the XCD), so at any moment an XCD is inside one or two pairs,
// whose K/V rows stay in its 4 MB L2, while the 8 XCDs work on 8 different
// pairs (different KV heads of a batch), which spreads the accesses of the
// moment over all HBM channels.
constexpr int kXcds = 8;
struct SegPlan {
    int n, hkv, nseg, lgS, L;
    FastDiv fd_L, fd_hkv;
};
struct Sched {
    int q, step, end;   // this team's item positions in its XCD's list
    int x;              // XCD
};
__device__ __forceinline__ Sched xcd_sched(const SegPlan& sp, int team_size) {
    const int x = blockIdx.x % kXcds;
    const int wslot = blockIdx.x / kXcds;
    const int teams_per_wg = kBlock / team_size;
    Sched s;
    s.x = x;
    s.q = wslot * teams_per_wg + (int)threadIdx.x / team_size;
    s.step = (gridDim.x / kXcds) * teams_per_wg;
    const int nseg_x = x < sp.nseg ? (sp.nseg - x + kXcds - 1) / kXcds : 0;
    s.end = nseg_x * sp.L;
    return s;
}
// Item q of XCD x -> (pair, token).
__device__ __forceinline__ void sched_item(const SegPlan& sp, int x, int q, int& pair, int& i) {
    const int m = (int)fdiv((uint32_t)q, sp.fd_L);
    const int k = x + kXcds * m;
    pair = k >> sp.lgS;
    i = (k & ((1 << sp.lgS) - 1)) * sp.L + (q - m * sp.L);
}

// Unpack 8 bf16 (one 16-byte piece) to fp32, and fp32 to a double vector.
__device__ __forceinline__ void bf16x8_to_f32(const uint4& u, float (&x)[8]) {
    x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x);
    x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
    x[4] = bf16_lo(u.z); x[5] = bf16_hi(u.z);
    x[6] = bf16_lo(u.w); x[7] = bf16_hi(u.w);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Dot product of two 16-byte bf16 pieces, accumulated in fp32.
__device__ __forceinline__ float dot_bf16x8(const uint4& a, const uint4& b) {
    float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x),
                                              __builtin_bit_cast(bf16x2_t, b.x), 0.0f, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y),
                                        __builtin_bit_cast(bf16x2_t, b.y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z),
                                        __builtin_bit_cast(bf16x2_t, b.z), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w),
                                        __builtin_bit_cast(bf16x2_t, b.w), s, false);
    return s;
}

// Two fp32 values to packed bf16 (hardware round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// exp2 / log2 / reciprocal: the hardware approximations in fp32 (about 1 ulp),
// the libm functions in fp64.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ double fast_exp2(double x) { return exp2(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ double fast_log2(double x) { return log2(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ double fast_rcp(double x) { return 1.0 / x; }

// One 16-byte piece of a d-row (8 bf16 or 4 fp32) in the accumulation type,
// and the dot product of two pieces.
template <typename A, int V>
__device__ __forceinline__ void unpack16(const uint4& u, A (&x)[V]) {
    if constexpr (V == 8) {
        float f[8];
        bf16x8_to_f32(u, f);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = f[e];
    } else {
        x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y);
        x[2] = __uint_as_float(u.z); x[3] = __uint_as_float(u.w);
    }
}
template <int V, typename A>
__device__ __forceinline__ A dot16(const uint4& a, const uint4& b) {
    if constexpr (V == 8) {
        return dot_bf16x8(a, b);
    } else {
        return (A)__uint_as_float(a.x) * (A)__uint_as_float(b.x) +
               (A)__uint_as_float(a.y) * (A)__uint_as_float(b.y) +
               (A)__uint_as_float(a.z) * (A)__uint_as_float(b.z) +
               (A)__uint_as_float(a.w) * (A)__uint_as_float(b.w);
    }
}

// Split piece of a 256-byte d-row for lane r of a 16-lane row: bytes
// [8r, 8r + 8) and [128 + 8r, 128 + 8r + 8) for bf16 (elements 4r .. 4r+3
// and 64 + 4r .. 64 + 4r + 3), bytes [16r, 16r + 16) for fp32 (elements
// 4r .. 4r+3).  With this mapping the lane's fp32 results for a bf16 row are
// two 16-byte runs at 16r and 256 + 16r of the 512-byte fp32 row, so each
// store instruction of the row covers 256 contiguous bytes.
template <int V>
__device__ __forceinline__ uint4 load_split(const char* row, int r) {
    if constexpr (V == 8) {
        const uint2 lo = *reinterpret_cast<const uint2*>(row + r * 8);
        const uint2 hi = *reinterpret_cast<const uint2*>(row + 128 + r * 8);
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
    } else {
        return *reinterpret_cast<const uint4*>(row + r * 16);
    }
}

// Streaming (non-temporal) 16-byte loads of rows read once, so they do not
// push reused (gathered) rows out of the L2.
typedef uint32_t u32x2_ld_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_ld_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt16(const char* p) {
    const u32x4_ld_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_ld_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
// 8 bytes in the low half of a 16-byte register group, the high half zero
__device__ __forceinline__ uint4 load_nt8(const char* p) {
    const u32x2_ld_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_ld_t*>(p));
    return make_uint4(v.x, v.y, 0u, 0u);
}
template <int V>
__device__ __forceinline__ uint4 load_split_nt(const char* row, int r) {
    if constexpr (V == 8) {
        const u32x2_ld_t lo =
            __builtin_nontemporal_load(reinterpret_cast<const u32x2_ld_t*>(row + r * 8));
        const u32x2_ld_t hi =
            __builtin_nontemporal_load(reinterpret_cast<const u32x2_ld_t*>(row + 128 + r * 8));
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
    } else {
        return load_nt16(row + r * 16);
    }
}

// Streaming (non-temporal) stores of outputs nobody reads soon, so they do
// not push gathered rows out of the L2.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int L, typename A>
__device__ __forceinline__ void store_f32_nt(char* p, const A* x) {
    if constexpr (L == 1) {
        __builtin_nontemporal_store((float)x[0], reinterpret_cast<float*>(p));
    } else if constexpr (L == 2) {
        const f32x2_t v = {(float)x[0], (float)x[1]};
        __builtin_nontemporal_store(v, reinterpret_cast<f32x2_t*>(p));
    } else {
#pragma unroll
        for (int e = 0; e < L; e += 4) {
            const f32x4_t v = {(float)x[e], (float)x[e + 1], (float)x[e + 2], (float)x[e + 3]};
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p + 4 * e));
        }
    }
}

// fp32 results of lane r for a split piece (see load_split), streaming stores.
template <int V, typename A>
__device__ __forceinline__ void store_split_f32_nt(char* frow, int r, const A (&x)[V]) {
    store_f32_nt<4>(frow + r * 16, x);
    if constexpr (V == 8) store_f32_nt<4>(frow + 256 + r * 16, x + 4);
}

__device__ __forceinline__ void store_u32x4_nt(char* p, uint32_t a, uint32_t b, uint32_t c,
                                               uint32_t d) {
    const u32x4_t v = {a, b, c, d};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

}  // namespace gm
