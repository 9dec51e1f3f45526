// Pieces shared by the kernels that keep the largest of a few weighted
// candidates per unit with one lane per unit (SER's two-hop referral, leg
// construction): the XCD-chunked unit of a lane and a sorting / merging
// network over 64-bit keys (weight bits << 32 | ~index, so that a larger
// weight, then a lower index, is a larger key).
#pragma once

#include "gm_common.h"
#include "gm_wave.h"

namespace gm {

// Unit of this lane when units are split into 8 contiguous chunks, one per
// XCD (workgroups are dealt to XCDs round robin): every chunk holds whole
// batches (or a contiguous part of one), i.e. all KV heads of its tokens, so
// the small edge rows it reads share cache lines and stay in its L2.
// Launch with kXcds * ceil(ceil(U / 8) / kBlock) workgroups; -1: no unit.
__device__ __forceinline__ int xcd_unit(int U) {
    const int chunk = (U + kXcds - 1) / kXcds;
    const int x = blockIdx.x % kXcds;
    const int q = (int)(blockIdx.x / kXcds) * kBlock + (int)threadIdx.x;
    const int u = x * chunk + q;
    return (q < chunk && u < U) ? u : -1;
}
inline unsigned xcd_unit_grid(int U) {
    const int chunk = (U + kXcds - 1) / kXcds;
    return (unsigned)(kXcds * ((chunk + kBlock - 1) / kBlock));
}

// compare-exchange: hi >= lo afterwards
__device__ __forceinline__ void cx(uint64_t& hi, uint64_t& lo) {
    const bool sw = lo > hi;
    const uint64_t t = sw ? lo : hi;
    lo = sw ? hi : lo;
    hi = t;
}
__device__ __forceinline__ void sort4_desc(uint64_t* k) {
    cx(k[0], k[1]); cx(k[2], k[3]);
    cx(k[0], k[2]); cx(k[1], k[3]);
    cx(k[1], k[2]);
}
// top 4 of two descending runs of 4, descending, into a
__device__ __forceinline__ void merge_top4(uint64_t* a, const uint64_t* b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = a[i] > b[3 - i] ? a[i] : b[3 - i];   // bitonic
    cx(a[0], a[2]); cx(a[1], a[3]);
    cx(a[0], a[1]); cx(a[2], a[3]);
}

// The 16 candidates (target m[k], fp64 weight cw[k], k in order) of one
// unit: targets are merged by summing, in candidate order, into their first
// candidate (later ones drop out), the sums rounded to fp32 and the 4
// largest positive ones returned as keys, descending (0 for none).  Each
// candidate's sum is finished before the next one starts, and each group of
// four keys is sorted as soon as it exists, so little state is live at once
// (one fp64 sum, a flag per candidate) and the kernel keeps
// several wavefronts per SIMD.
__device__ __forceinline__ void top4_of_16(const int (&m)[16], const double (&cw)[16],
                                           uint64_t (&key)[16]) {
    bool rep[16];   // candidate k repeats an earlier target
#pragma unroll
    for (int k = 0; k < 16; ++k) rep[k] = false;
#pragma unroll
    for (int k2 = 0; k2 < 16; ++k2) {
        double acc = cw[k2];
#pragma unroll
        for (int k = k2 + 1; k < 16; ++k) {
            const bool same = m[k] == m[k2];
            acc += same ? cw[k] : 0.0;
            rep[k] = rep[k] || same;
        }
        const float wk = (float)acc;
        key[k2] = !rep[k2] && m[k2] >= 0 && wk > 0.0f
                      ? ((uint64_t)__float_as_uint(wk) << 32) | (uint32_t)~(uint32_t)m[k2]
                      : 0ull;
        if ((k2 & 3) == 3) sort4_desc(key + (k2 - 3));
    }
    merge_top4(key + 0, key + 4);
    merge_top4(key + 8, key + 12);
    merge_top4(key + 0, key + 8);
}

}  // namespace gm
