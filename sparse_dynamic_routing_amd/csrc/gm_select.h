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

}  // namespace gm
