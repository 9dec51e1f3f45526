// Pieces shared by the kernels that keep the largest of a few weighted
// candidates per unit with one lane per unit (SER's two-hop referral, leg
// construction, the decode step): the XCD-chunked unit of a lane, a
// sorting / merging network over 64-bit keys (weight bits << 32 | ~index, so
// that a larger weight, then a lower index, is a larger key), and the
// 16-lane team merge and rank by DPP row rotations.
#pragma once

#include "gm_common.h"
#include "gm_wave.h"

#include <utility>

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

// Rotation inside a 16-lane row (DPP row_ror:D): every lane reads one lane
// of its own row, so a team of 16 sweeps its partners without LDS.
template <int D>
__device__ __forceinline__ int ror_i(int x) {
    return __builtin_amdgcn_update_dpp(0, x, 0x120 + D, 0xF, 0xF, false);
}
template <int D>
__device__ __forceinline__ float ror_f(float x) {
    return __int_as_float(ror_i<D>(__float_as_int(x)));
}
template <int D>
__device__ __forceinline__ double ror_d(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)ror_i<D>((int)(uint32_t)u);
    const uint32_t hi = (uint32_t)ror_i<D>((int)(uint32_t)(u >> 32));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

struct Cand {
    int k, m;
    double cw, acc;
    bool dup;
    float key;
    bool cand;
    int rank;
};
// merge step against the partner D lanes away (its slot index read along)
template <int D>
__device__ __forceinline__ void merge_step(Cand& c) {
    const int k2 = ror_i<D>(c.k);
    const int mk = ror_i<D>(c.m);
    const double ck = ror_d<D>(c.cw);
    if (mk == c.m) {
        if (k2 < c.k) c.dup = true;
        else c.acc += ck;
    }
}
template <int D>
__device__ __forceinline__ void rank_step(Cand& c) {
    const float kk = ror_f<D>(c.key);
    const int mk = ror_i<D>(c.m);
    const bool ck = ror_i<D>((int)c.cand) != 0;
    if (ck && (kk > c.key || (kk == c.key && mk < c.m))) ++c.rank;
}
// later slots must be added in increasing slot order: the sweep runs in
// whichever rotation direction visits them that way
template <int... D>
__device__ __forceinline__ void merge_up(Cand& c, std::integer_sequence<int, D...>) {
    (merge_step<D + 1>(c), ...);
}
template <int... D>
__device__ __forceinline__ void merge_down(Cand& c, std::integer_sequence<int, D...>) {
    (merge_step<15 - D>(c), ...);
}
template <int... D>
__device__ __forceinline__ void rank_all(Cand& c, std::integer_sequence<int, D...>) {
    (rank_step<D + 1>(c), ...);
}

// A 16-lane row as a team of 16 candidates, lane k = candidate k (k = lane
// % 16; target m, fp64 weight cw, `valid` false for lanes without one):
// each target's first lane sums the later lanes of that target in candidate
// order (fp64), key = that sum rounded to fp32, cand = a valid first lane
// with key > 0, rank = its place among the row's candidates (larger key
// first, then the lower target).  Every lane of the wavefront takes part.
__device__ __forceinline__ void team16_merge_rank(int k, int m, double cw, bool valid,
                                                  float& key, bool& cand, int& rank) {
    Cand c{k, m, cw, cw, false, 0.0f, false, 0};
    if (ror_i<1>(k) == ((k + 1) & 15))
        merge_up(c, std::make_integer_sequence<int, 15>{});
    else
        merge_down(c, std::make_integer_sequence<int, 15>{});
    c.key = (float)c.acc;
    c.cand = valid && !c.dup && c.key > 0.0f;
    rank_all(c, std::make_integer_sequence<int, 15>{});
    key = c.key;
    cand = c.cand;
    rank = c.rank;
}

}  // namespace gm
