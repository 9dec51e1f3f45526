// Shared device helpers for the gfx950 kernels of the Graph Machine path.
// Wave64 everywhere: a "team" is a power-of-two group of lanes inside one
// wavefront that works on one unit (b, token i, KV head h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gm {

constexpr int kWave = 64;
constexpr int kBlock = 256;  // four waves per workgroup

struct bf16_t { uint16_t bits; };

// Per-dtype layout of one 16-byte vector load: V elements per lane, and the
// accumulation type (fp32 for bf16 inputs, fp64 for fp32 inputs).
template <typename T> struct io;
template <> struct io<bf16_t> { static constexpr int V = 8; using acc = float; };
template <> struct io<float>  { static constexpr int V = 4; using acc = double; };

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

template <typename A>
__device__ __forceinline__ void load16(const bf16_t* p, A (&x)[8]) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x);
    x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
    x[4] = bf16_lo(u.z); x[5] = bf16_hi(u.z);
    x[6] = bf16_lo(u.w); x[7] = bf16_hi(u.w);
}

template <typename A>
__device__ __forceinline__ void load16(const float* p, A (&x)[4]) {
    const float4 f = *reinterpret_cast<const float4*>(p);
    x[0] = f.x; x[1] = f.y; x[2] = f.z; x[3] = f.w;
}

// Store L consecutive accumulator values as dtype T (L in {1, 2, 4, 8}).
template <int L, typename A>
__device__ __forceinline__ void store_n(bf16_t* p, const A* x) {
    if constexpr (L == 1) {
        p->bits = (uint16_t)f32_to_bf16((float)x[0]);
    } else {
        uint32_t w[L / 2];
#pragma unroll
        for (int e = 0; e < L / 2; ++e)
            w[e] = f32_to_bf16((float)x[2 * e]) | (f32_to_bf16((float)x[2 * e + 1]) << 16);
        if constexpr (L == 2) *reinterpret_cast<uint32_t*>(p) = w[0];
        if constexpr (L == 4) *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
        if constexpr (L == 8) *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

template <int L, typename A>
__device__ __forceinline__ void store_n(float* p, const A* x) {
    if constexpr (L == 1) *p = (float)x[0];
    if constexpr (L == 2) *reinterpret_cast<float2*>(p) = make_float2((float)x[0], (float)x[1]);
    if constexpr (L >= 4) {
#pragma unroll
        for (int e = 0; e < L; e += 4)
            *reinterpret_cast<float4*>(p + e) =
                make_float4((float)x[e], (float)x[e + 1], (float)x[e + 2], (float)x[e + 3]);
    }
}

__device__ __forceinline__ float xor_shfl(float x, int m) { return __shfl_xor(x, m, kWave); }
__device__ __forceinline__ double xor_shfl(double x, int m) { return __shfl_xor(x, m, kWave); }

__device__ __forceinline__ float amax(float a, float b) { return fmaxf(a, b); }
__device__ __forceinline__ double amax(double a, double b) { return fmax(a, b); }
__device__ __forceinline__ float aexp2(float x) { return exp2f(x); }
__device__ __forceinline__ double aexp2(double x) { return exp2(x); }
__device__ __forceinline__ float alog2(float x) { return log2f(x); }
__device__ __forceinline__ double alog2(double x) { return log2(x); }

// Sum over the lanes whose team-lane index differs only in bits [lo, hi)
// (masks lo, 2lo, ..., hi/2), leaving the total in every such lane.
template <typename A>
__device__ __forceinline__ A sum_bits(A x, int lo, int hi) {
    for (int m = lo; m < hi; m <<= 1) x += xor_shfl(x, m);
    return x;
}
template <typename A>
__device__ __forceinline__ A max_bits(A x, int lo, int hi) {
    for (int m = lo; m < hi; m <<= 1) x = amax(x, xor_shfl(x, m));
    return x;
}

// Reduce-scatter of a V-vector over the P = hi/lo lanes that differ in bits
// [lo, hi) of the team-lane index tl: afterwards each lane holds
// len = max(1, V/P) summed elements in x[0 .. len), starting at element
// offset `off` of the V-vector (returned).  When V < P the last steps are
// plain all-reduces, so several lanes hold the same element.  The step count
// is a runtime value, but every array index is static (no scratch spills).
template <int K, int V, typename A>
__device__ __forceinline__ void reduce_scatter_step(A (&x)[V], int tl, int lo, int hi, int& off,
                                                    int& len) {
    if constexpr (K < 6) {
        const int m = lo << K;
        if (m < hi) {
            if constexpr ((V >> K) > 1) {
                constexpr int half = V >> (K + 1);
                const bool upper = (tl & m) != 0;
#pragma unroll
                for (int e = 0; e < half; ++e) {
                    const A send = upper ? x[e] : x[e + half];
                    const A keep = upper ? x[e + half] : x[e];
                    x[e] = keep + xor_shfl(send, m);
                }
                if (upper) off += half;
                len = half;
            } else {
                x[0] += xor_shfl(x[0], m);
            }
            reduce_scatter_step<K + 1>(x, tl, lo, hi, off, len);
        }
    }
}

template <int V, typename A>
__device__ __forceinline__ int reduce_scatter(A (&x)[V], int tl, int lo, int hi, int& len) {
    int off = 0;
    len = V;
    reduce_scatter_step<0>(x, tl, lo, hi, off, len);
    return off;
}

// Store x[0 .. len) (len in {1, 2, 4, 8}, at most V) as dtype T.
template <int V, typename T, typename A>
__device__ __forceinline__ void store_len(T* p, const A (&x)[V], int len) {
    if (len >= 8) { if constexpr (V >= 8) store_n<8>(p, x); }
    else if (len == 4) { if constexpr (V >= 4) store_n<4>(p, x); }
    else if (len == 2) store_n<2>(p, x);
    else store_n<1>(p, x);
}

__host__ __device__ constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }

__host__ __device__ inline int pow2_ceil(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

}  // namespace gm
