// Reverse (target-sorted) index of an edge tensor, for the pull-style
// backward passes: for every (batch, KV head) pair and target token j, the
// list of live edge ids e = unit * s + slot with idx[e] == j.
//
// Counting sorts in LDS; no per-edge global atomics (device-scope atomics on
// this multi-XCD part are slow, and a returning one per edge bounds the
// build).  n <= 4096: one 1024-thread workgroup per (pair, target half)
// loads the pair's edges once and sorts its half in LDS; the edges come
// either from idx/w (rows of all KV heads interleaved, 16 bytes used per
// 128-byte line) or from a compact per-pair copy of the live targets that
// the SEA backward's source pass writes as it goes (both index builders
// take either source).  Longer sequences:
// a bucket partition, then an LDS sort per bucket (below).  The pair's list
// occupies the fixed range [pair * n * s, (pair + 1) * n * s); beg and len
// are indexed by the pair-major row pair * n + j.  Inside one target's
// segment the edges are in ascending id order (the LDS atomics place them,
// a ranking pass then fixes their order), so the index is the same on every
// run.
#include "gm_common.h"
#include "gm_internal.h"
#include "gm_wave.h"

#include <limits.h>

namespace gm {
namespace {

constexpr int kIndexThreads = 1024;
constexpr int kTok = 4;            // tokens per thread per batch
constexpr int kSlotMax = 4;        // fast loads for s <= 4

struct IndexArgs {
    const int32_t* idx;
    const float* w;
    const int* tgt;   // pair-major live targets (-1 dead) instead of idx/w, or null
    int n, hkv, s, K, npairs, vec;
    int* beg;
    int* len;
    int* list;
    int* head;     // [pair-major row * 4] or null
};

// ------------------------------------------------ fixed order within rows
// The counting sorts place edges with LDS atomics, in an order that varies
// between runs.  sort_runs then puts every row's run of edge ids in
// ascending order (the index, and the order the backward sums a row's edges
// in, are then the same on every run).  Row j's run is
// list[end[j] - len[j], end[j]).  By run length:
//   <= 32    one lane, a sorting network in registers (Batcher's
//            odd-even merge sort of 4, 8, 16 or 32 keys: 5, 19, 63 or 191
//            compare-exchanges);
//   33..256  one wavefront, a bitonic sort of 64, 128 or 256 keys held one,
//            two or four per lane (partners in other lanes through shuffles,
//            in other registers of the same lane beyond 64);
//   longer   each id's rank (the number of smaller ids in the run) counted
//            over the run in memory, the id written to its place in `spill`
//            (global memory of the run's size at the same offsets), then
//            read back.
// Ids are < 2^31 - 1, so INT_MAX pads.  Every thread of the workgroup must
// call it.  Inlined, so that at each call the compiler sees which arrays
// live in LDS and addresses them as such.
constexpr int kNetRun = 32;
constexpr int kWaveRun = 256;

__device__ __forceinline__ void cswap(int& a, int& b) {
    const int lo = a < b ? a : b, hi = a < b ? b : a;
    a = lo;
    b = hi;
}

__device__ __forceinline__ void sort4(int (&r)[32]) {
    cswap(r[0], r[1]); cswap(r[2], r[3]); cswap(r[0], r[2]); cswap(r[1], r[3]);
    cswap(r[1], r[2]);
}

__device__ __forceinline__ void sort8(int (&r)[32]) {
    cswap(r[0], r[1]); cswap(r[2], r[3]); cswap(r[4], r[5]); cswap(r[6], r[7]);
    cswap(r[0], r[2]); cswap(r[1], r[3]); cswap(r[4], r[6]); cswap(r[5], r[7]);
    cswap(r[1], r[2]); cswap(r[5], r[6]);
    cswap(r[0], r[4]); cswap(r[1], r[5]); cswap(r[2], r[6]); cswap(r[3], r[7]);
    cswap(r[2], r[4]); cswap(r[3], r[5]);
    cswap(r[1], r[2]); cswap(r[3], r[4]); cswap(r[5], r[6]);
}

__device__ __forceinline__ void sort16(int (&r)[32]) {
    cswap(r[0], r[1]); cswap(r[2], r[3]); cswap(r[0], r[2]); cswap(r[1], r[3]);
    cswap(r[1], r[2]); cswap(r[4], r[5]); cswap(r[6], r[7]); cswap(r[4], r[6]);
    cswap(r[5], r[7]); cswap(r[5], r[6]); cswap(r[0], r[4]); cswap(r[2], r[6]);
    cswap(r[2], r[4]); cswap(r[1], r[5]); cswap(r[3], r[7]); cswap(r[3], r[5]);
    cswap(r[1], r[2]); cswap(r[3], r[4]); cswap(r[5], r[6]); cswap(r[8], r[9]);
    cswap(r[10], r[11]); cswap(r[8], r[10]); cswap(r[9], r[11]); cswap(r[9], r[10]);
    cswap(r[12], r[13]); cswap(r[14], r[15]); cswap(r[12], r[14]); cswap(r[13], r[15]);
    cswap(r[13], r[14]); cswap(r[8], r[12]); cswap(r[10], r[14]); cswap(r[10], r[12]);
    cswap(r[9], r[13]); cswap(r[11], r[15]); cswap(r[11], r[13]); cswap(r[9], r[10]);
    cswap(r[11], r[12]); cswap(r[13], r[14]); cswap(r[0], r[8]); cswap(r[4], r[12]);
    cswap(r[4], r[8]); cswap(r[2], r[10]); cswap(r[6], r[14]); cswap(r[6], r[10]);
    cswap(r[2], r[4]); cswap(r[6], r[8]); cswap(r[10], r[12]); cswap(r[1], r[9]);
    cswap(r[5], r[13]); cswap(r[5], r[9]); cswap(r[3], r[11]); cswap(r[7], r[15]);
    cswap(r[7], r[11]); cswap(r[3], r[5]); cswap(r[7], r[9]); cswap(r[11], r[13]);
    cswap(r[1], r[2]); cswap(r[3], r[4]); cswap(r[5], r[6]); cswap(r[7], r[8]);
    cswap(r[9], r[10]); cswap(r[11], r[12]); cswap(r[13], r[14]);
}

__device__ __forceinline__ void sort32(int (&r)[32]) {
    cswap(r[0], r[1]); cswap(r[2], r[3]); cswap(r[0], r[2]); cswap(r[1], r[3]);
    cswap(r[1], r[2]); cswap(r[4], r[5]); cswap(r[6], r[7]); cswap(r[4], r[6]);
    cswap(r[5], r[7]); cswap(r[5], r[6]); cswap(r[0], r[4]); cswap(r[2], r[6]);
    cswap(r[2], r[4]); cswap(r[1], r[5]); cswap(r[3], r[7]); cswap(r[3], r[5]);
    cswap(r[1], r[2]); cswap(r[3], r[4]); cswap(r[5], r[6]); cswap(r[8], r[9]);
    cswap(r[10], r[11]); cswap(r[8], r[10]); cswap(r[9], r[11]); cswap(r[9], r[10]);
    cswap(r[12], r[13]); cswap(r[14], r[15]); cswap(r[12], r[14]); cswap(r[13], r[15]);
    cswap(r[13], r[14]); cswap(r[8], r[12]); cswap(r[10], r[14]); cswap(r[10], r[12]);
    cswap(r[9], r[13]); cswap(r[11], r[15]); cswap(r[11], r[13]); cswap(r[9], r[10]);
    cswap(r[11], r[12]); cswap(r[13], r[14]); cswap(r[0], r[8]); cswap(r[4], r[12]);
    cswap(r[4], r[8]); cswap(r[2], r[10]); cswap(r[6], r[14]); cswap(r[6], r[10]);
    cswap(r[2], r[4]); cswap(r[6], r[8]); cswap(r[10], r[12]); cswap(r[1], r[9]);
    cswap(r[5], r[13]); cswap(r[5], r[9]); cswap(r[3], r[11]); cswap(r[7], r[15]);
    cswap(r[7], r[11]); cswap(r[3], r[5]); cswap(r[7], r[9]); cswap(r[11], r[13]);
    cswap(r[1], r[2]); cswap(r[3], r[4]); cswap(r[5], r[6]); cswap(r[7], r[8]);
    cswap(r[9], r[10]); cswap(r[11], r[12]); cswap(r[13], r[14]); cswap(r[16], r[17]);
    cswap(r[18], r[19]); cswap(r[16], r[18]); cswap(r[17], r[19]); cswap(r[17], r[18]);
    cswap(r[20], r[21]); cswap(r[22], r[23]); cswap(r[20], r[22]); cswap(r[21], r[23]);
    cswap(r[21], r[22]); cswap(r[16], r[20]); cswap(r[18], r[22]); cswap(r[18], r[20]);
    cswap(r[17], r[21]); cswap(r[19], r[23]); cswap(r[19], r[21]); cswap(r[17], r[18]);
    cswap(r[19], r[20]); cswap(r[21], r[22]); cswap(r[24], r[25]); cswap(r[26], r[27]);
    cswap(r[24], r[26]); cswap(r[25], r[27]); cswap(r[25], r[26]); cswap(r[28], r[29]);
    cswap(r[30], r[31]); cswap(r[28], r[30]); cswap(r[29], r[31]); cswap(r[29], r[30]);
    cswap(r[24], r[28]); cswap(r[26], r[30]); cswap(r[26], r[28]); cswap(r[25], r[29]);
    cswap(r[27], r[31]); cswap(r[27], r[29]); cswap(r[25], r[26]); cswap(r[27], r[28]);
    cswap(r[29], r[30]); cswap(r[16], r[24]); cswap(r[20], r[28]); cswap(r[20], r[24]);
    cswap(r[18], r[26]); cswap(r[22], r[30]); cswap(r[22], r[26]); cswap(r[18], r[20]);
    cswap(r[22], r[24]); cswap(r[26], r[28]); cswap(r[17], r[25]); cswap(r[21], r[29]);
    cswap(r[21], r[25]); cswap(r[19], r[27]); cswap(r[23], r[31]); cswap(r[23], r[27]);
    cswap(r[19], r[21]); cswap(r[23], r[25]); cswap(r[27], r[29]); cswap(r[17], r[18]);
    cswap(r[19], r[20]); cswap(r[21], r[22]); cswap(r[23], r[24]); cswap(r[25], r[26]);
    cswap(r[27], r[28]); cswap(r[29], r[30]); cswap(r[0], r[16]); cswap(r[8], r[24]);
    cswap(r[8], r[16]); cswap(r[4], r[20]); cswap(r[12], r[28]); cswap(r[12], r[20]);
    cswap(r[4], r[8]); cswap(r[12], r[16]); cswap(r[20], r[24]); cswap(r[2], r[18]);
    cswap(r[10], r[26]); cswap(r[10], r[18]); cswap(r[6], r[22]); cswap(r[14], r[30]);
    cswap(r[14], r[22]); cswap(r[6], r[10]); cswap(r[14], r[18]); cswap(r[22], r[26]);
    cswap(r[2], r[4]); cswap(r[6], r[8]); cswap(r[10], r[12]); cswap(r[14], r[16]);
    cswap(r[18], r[20]); cswap(r[22], r[24]); cswap(r[26], r[28]); cswap(r[1], r[17]);
    cswap(r[9], r[25]); cswap(r[9], r[17]); cswap(r[5], r[21]); cswap(r[13], r[29]);
    cswap(r[13], r[21]); cswap(r[5], r[9]); cswap(r[13], r[17]); cswap(r[21], r[25]);
    cswap(r[3], r[19]); cswap(r[11], r[27]); cswap(r[11], r[19]); cswap(r[7], r[23]);
    cswap(r[15], r[31]); cswap(r[15], r[23]); cswap(r[7], r[11]); cswap(r[15], r[19]);
    cswap(r[23], r[27]); cswap(r[3], r[5]); cswap(r[7], r[9]); cswap(r[11], r[13]);
    cswap(r[15], r[17]); cswap(r[19], r[21]); cswap(r[23], r[25]); cswap(r[27], r[29]);
    cswap(r[1], r[2]); cswap(r[3], r[4]); cswap(r[5], r[6]); cswap(r[7], r[8]);
    cswap(r[9], r[10]); cswap(r[11], r[12]); cswap(r[13], r[14]); cswap(r[15], r[16]);
    cswap(r[17], r[18]); cswap(r[19], r[20]); cswap(r[21], r[22]); cswap(r[23], r[24]);
    cswap(r[25], r[26]); cswap(r[27], r[28]); cswap(r[29], r[30]);
}

// Ascending bitonic sort of C * 64 keys, key c * 64 + lane in v[c].
template <int C>
__device__ __forceinline__ void wave_bitonic(int (&v)[C]) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int k = 2; k <= C * kWave; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            if (j >= kWave) {
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    const int pc = c ^ (j / kWave);
                    if (pc > c) {
                        const bool up = ((c * kWave + lane) & k) == 0;
                        const int lo = v[c] < v[pc] ? v[c] : v[pc];
                        const int hi = v[c] < v[pc] ? v[pc] : v[c];
                        v[c] = up ? lo : hi;
                        v[pc] = up ? hi : lo;
                    }
                }
            } else {
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    const int x = __shfl_xor(v[c], j, kWave);
                    const bool up = ((c * kWave + lane) & k) == 0;
                    const bool lower = (lane & j) == 0;
                    v[c] = (up == lower) ? (v[c] < x ? v[c] : x) : (v[c] < x ? x : v[c]);
                }
            }
        }
    }
}

template <int C>
__device__ __forceinline__ void wave_sort_run(int* run, int L) {
    const int lane = threadIdx.x & (kWave - 1);
    int v[C];
#pragma unroll
    for (int c = 0; c < C; ++c) v[c] = c * kWave + lane < L ? run[c * kWave + lane] : INT_MAX;
    wave_bitonic<C>(v);
#pragma unroll
    for (int c = 0; c < C; ++c)
        if (c * kWave + lane < L) run[c * kWave + lane] = v[c];
}

// Load run[0, L) (L <= N) into r, pad with INT_MAX, sort with the network,
// store back.
template <int N, typename Net>
__device__ __forceinline__ void sort_small(int* run, int L, int (&r)[32], Net net) {
#pragma unroll
    for (int k = 0; k < N; ++k) r[k] = k < L ? run[k] : INT_MAX;
    net(r);
#pragma unroll
    for (int k = 0; k < N; ++k)
        if (k < L) run[k] = r[k];
}

// Rows are first grouped by run length (5..8, 9..16, 17..32, longer) into
// `cls` (stream compaction with one LDS atomic per wavefront and class), so
// that the lanes of a wavefront run one network size without divergence.
// cls needs kClsRows ints: at most E / 5, E / 9, E / 17, E / 33 rows of each
// class for E <= kOneList edges, and at most the 512 rows of a bucket in the
// long-sequence sort, whatever its edge count.
constexpr int kCls0 = 0, kCls1 = kCls0 + 3277, kCls2 = kCls1 + 1821, kCls3 = kCls2 + 964;
constexpr int kClsRows = kCls3 + 512;
__device__ __forceinline__ void sort_runs(int* list, const int* end, const int* len, int nr,
                                          int* cls, int* ncls, int* spill) {
    if (threadIdx.x < 4) ncls[threadIdx.x] = 0;
    __syncthreads();
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave, nwave = blockDim.x / kWave;
    const unsigned long long below = (1ull << lane) - 1ull;
    const int cbase[4] = {kCls0, kCls1, kCls2, kCls3};
    for (int j0 = wave * kWave; j0 < nr; j0 += nwave * kWave) {
        const int j = j0 + lane;
        const int L = j < nr ? len[j] : 0;
        if (L >= 2 && L <= 4) {
            int r[32];
            sort_small<4>(list + (end[j] - L), L, r, sort4);
        }
        const int c = L <= 4 ? -1 : L <= 8 ? 0 : L <= 16 ? 1 : L <= kNetRun ? 2 : 3;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const unsigned long long m = __ballot(c == k);
            if (!m) continue;
            int base = 0;
            if (lane == 0) base = atomicAdd(ncls + k, __popcll(m));
            base = __shfl(base, 0, kWave);
            if (c == k) cls[cbase[k] + base + __popcll(m & below)] = j;
        }
    }
    __syncthreads();
    // one network size per class, a lane per row
    for (int q = threadIdx.x; q < ncls[0]; q += blockDim.x) {
        const int j = cls[kCls0 + q], L = len[j];
        int r[32];
        sort_small<8>(list + (end[j] - L), L, r, sort8);
    }
    for (int q = threadIdx.x; q < ncls[1]; q += blockDim.x) {
        const int j = cls[kCls1 + q], L = len[j];
        int r[32];
        sort_small<16>(list + (end[j] - L), L, r, sort16);
    }
    for (int q = threadIdx.x; q < ncls[2]; q += blockDim.x) {
        const int j = cls[kCls2 + q], L = len[j];
        int r[32];
        sort_small<32>(list + (end[j] - L), L, r, sort32);
    }
    // longer runs: a wavefront each
    const int nh = ncls[3];
    bool spilled = false;
    for (int q = wave; q < nh; q += nwave) {
        const int j = cls[kCls3 + q];
        const int L = len[j];
        const int b0 = end[j] - L;
        int* run = list + b0;
        if (L <= kWave) {
            wave_sort_run<1>(run, L);
        } else if (L <= 2 * kWave) {
            wave_sort_run<2>(run, L);
        } else if (L <= kWaveRun) {
            wave_sort_run<4>(run, L);
        } else {
            spilled = true;
            for (int p = lane; p < L; p += kWave) {
                const int v = run[p];
                int rk = 0;
                for (int u = 0; u < L; ++u) rk += run[u] < v;
                spill[b0 + rk] = v;
            }
        }
    }
    // long runs come back from global memory once every wavefront is done
    if (__syncthreads_or(spilled)) {
        for (int q = wave; q < nh; q += nwave) {
            const int j = cls[kCls3 + q];
            const int L = len[j];
            if (L <= kWaveRun) continue;
            const int b0 = end[j] - L;
            for (int p = lane; p < L; p += kWave) list[b0 + p] = spill[b0 + p];
        }
        __syncthreads();
    }
}

// The head record of rows [0, nr) (their first four edge ids, -1 padded) at
// head[4 * (row0 + j)], from runs lst[beg[j], beg[j] + len[j]).
__device__ __forceinline__ void write_heads(int* head, size_t row0, const int* lst,
                                            const int* beg, const int* len, int nr) {
    for (int j = threadIdx.x; j < nr; j += blockDim.x) {
        const int l = len[j], b0 = beg[j];
        int4 hd;
        hd.x = l > 0 ? lst[b0] : -1;
        hd.y = l > 1 ? lst[b0 + 1] : -1;
        hd.z = l > 2 ? lst[b0 + 2] : -1;
        hd.w = l > 3 ? lst[b0 + 3] : -1;
        reinterpret_cast<int4*>(head)[row0 + j] = hd;
    }
}

// Single-pass variant for n <= kIndexThreads * kTok: each thread holds its
// kTok tokens' edges in registers from one load, the range's list is
// placed in LDS and then copied out with coalesced stores, and beg/len are
// written row-contiguously.  Every load is unconditional (a clamped valid
// address, masked afterwards), so the loads of a thread issue back to back.
constexpr int kOneRows = kIndexThreads * kTok;   // 4096 tokens: targets of a range
constexpr int kOneList = kOneRows * kSlotMax;    // edges of a pair

template <bool VEC>
__global__ __launch_bounds__(kIndexThreads) void edge_index_one_kernel(IndexArgs a) {
    __shared__ int cnt[kOneRows];    // count, then fill cursor (range-relative)
    __shared__ int rlen[kOneRows];
    __shared__ int sorted[kOneList];
    __shared__ int part[kIndexThreads / kWave];
    __shared__ int range_total;
    __shared__ int cls[kClsRows];   // rows grouped by run length for sort_runs
    __shared__ int ncls[4];
    const int total = a.npairs * a.K;
    int lin = (int)blockIdx.x;
    if (total % kXcds == 0)
        lin = ((int)blockIdx.x % kXcds) * (total / kXcds) + (int)blockIdx.x / kXcds;
    const int pair = lin / a.K, kq = lin - (lin / a.K) * a.K;
    const int n = a.n, s = a.s, hkv = a.hkv;
    const int jlo = (int)((long long)kq * n / a.K), jhi = (int)((long long)(kq + 1) * n / a.K);
    const int nr = jhi - jlo;
    const int b = pair / hkv, h = pair - (pair / hkv) * hkv;
    const int lbase = pair * n * s;
    for (int j = threadIdx.x; j < nr; j += kIndexThreads) cnt[j] = 0;
    __syncthreads();

    int tj[kTok * kSlotMax], te[kTok * kSlotMax];
#pragma unroll
    for (int k = 0; k < kTok; ++k) {
        const int iv = k * kIndexThreads + (int)threadIdx.x;
        const bool ok = iv < n;
        const int i = ok ? iv : n - 1;
        const int e0 = ((b * n + i) * hkv + h) * s;
        if (a.tgt) {
            // compact rows: the live targets of this pair, contiguous per token
            const int* tr = a.tgt + (size_t)(pair * n + i) * s;
            if constexpr (VEC) {
                const int4 t4 = *reinterpret_cast<const int4*>(tr);
                tj[k * 4 + 0] = t4.x; tj[k * 4 + 1] = t4.y;
                tj[k * 4 + 2] = t4.z; tj[k * 4 + 3] = t4.w;
            } else {
#pragma unroll
                for (int t = 0; t < kSlotMax; ++t) tj[k * kSlotMax + t] = tr[t < s ? t : s - 1];
            }
#pragma unroll
            for (int t = 0; t < kSlotMax; ++t) {
                const int sl = k * kSlotMax + t;
                te[sl] = ok && t < s && tj[sl] >= 0 ? e0 + t : -1;
            }
        } else if constexpr (VEC) {
            const int4 j4 = *reinterpret_cast<const int4*>(a.idx + e0);
            const float4 w4 = *reinterpret_cast<const float4*>(a.w + e0);
            tj[k * 4 + 0] = j4.x; tj[k * 4 + 1] = j4.y;
            tj[k * 4 + 2] = j4.z; tj[k * 4 + 3] = j4.w;
            te[k * 4 + 0] = ok && w4.x > 0.0f ? e0 + 0 : -1;
            te[k * 4 + 1] = ok && w4.y > 0.0f ? e0 + 1 : -1;
            te[k * 4 + 2] = ok && w4.z > 0.0f ? e0 + 2 : -1;
            te[k * 4 + 3] = ok && w4.w > 0.0f ? e0 + 3 : -1;
        } else {
#pragma unroll
            for (int t = 0; t < kSlotMax; ++t) {
                const int sl = k * kSlotMax + t;
                const int e = e0 + (t < s ? t : s - 1);
                tj[sl] = a.idx[e];
                te[sl] = ok && t < s && a.w[e] > 0.0f ? e : -1;
            }
        }
    }
    int below = 0;
#pragma unroll
    for (int k = 0; k < kTok * kSlotMax; ++k) {
        if (te[k] < 0) continue;
        if (tj[k] < jlo) ++below;
        else if (tj[k] < jhi) atomicAdd(&cnt[tj[k] - jlo], 1);
    }
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    for (int m = 32; m > 0; m >>= 1) below += __shfl_xor(below, m, kWave);
    if (lane == 0) part[wave] = below;
    __syncthreads();
    int below_all = 0;
    for (int k = 0; k < kIndexThreads / kWave; ++k) below_all += part[k];
    __syncthreads();

    // exclusive scan of the counts: each thread scans a contiguous run
    const int run_len = (nr + kIndexThreads - 1) / kIndexThreads;
    const int j0 = threadIdx.x * run_len;
    int run = 0;
    for (int j = j0; j < j0 + run_len && j < nr; ++j) run += cnt[j];
    int inc = run;
    for (int m = 1; m < kWave; m <<= 1) {
        const int o = __shfl_up(inc, m, kWave);
        if (lane >= m) inc += o;
    }
    if (lane == kWave - 1) part[wave] = inc;
    __syncthreads();
    int base = 0;
    for (int k = 0; k < wave; ++k) base += part[k];
    if (threadIdx.x == kIndexThreads - 1) range_total = base + inc;
    base += inc - run;
    for (int j = j0; j < j0 + run_len && j < nr; ++j) {
        const int c = cnt[j];
        rlen[j] = c;
        cnt[j] = base;
        base += c;
    }
    __syncthreads();
    const int gbase = lbase + below_all;   // list slot of the range's first edge
    for (int j = threadIdx.x; j < nr; j += kIndexThreads) {
        a.beg[pair * n + jlo + j] = gbase + cnt[j];
        a.len[pair * n + jlo + j] = rlen[j];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kTok * kSlotMax; ++k)
        if (te[k] >= 0 && tj[k] >= jlo && tj[k] < jhi)
            sorted[atomicAdd(&cnt[tj[k] - jlo], 1)] = te[k];
    __syncthreads();
    // ascending edge ids within every row (long rows spill to their final
    // place in the global list, which the copy below then rewrites)
    sort_runs(sorted, cnt, rlen, nr, cls, ncls, a.list + gbase);
    for (int p = threadIdx.x; p < range_total; p += kIndexThreads) a.list[gbase + p] = sorted[p];
    if (a.head) {
        // cnt[j] is now the end of row j's run in `sorted`
        for (int j = threadIdx.x; j < nr; j += kIndexThreads) {
            const int l = rlen[j], b0 = cnt[j] - l;
            int4 hd;
            hd.x = l > 0 ? sorted[b0] : -1;
            hd.y = l > 1 ? sorted[b0 + 1] : -1;
            hd.z = l > 2 ? sorted[b0 + 2] : -1;
            hd.w = l > 3 ? sorted[b0 + 3] : -1;
            reinterpret_cast<int4*>(a.head)[pair * n + jlo + j] = hd;
        }
    }
}

// ------------------------------------------- index of long sequences
// For n > kOneRows the per-pair workgroups above would each read every
// token of a pair; instead the edges are first partitioned by target bucket
// (kBucket rows) with only workgroup-local atomics, then each bucket is
// sorted in LDS like a short sequence:
//   count:   workgroup (pair, chunk of kOneRows source tokens) counts its
//            live edges per bucket (LDS) into counts[pair][bucket][chunk];
//   scan:    per pair, exclusive offsets in (bucket, chunk) order, so each
//            bucket's edges and, inside it, each chunk's are contiguous;
//   scatter: the count workgroups again, each edge to
//            offset + (LDS cursor of its bucket) in staging, as (edge, target);
//   sort:    workgroup (pair, bucket) counts the bucket's rows in LDS, writes
//            beg/len and places the edges (through LDS when they fit).
// The list of pair p is again [p * n * s, (p + 1) * n * s).
constexpr int kBucket = 512;        // target rows per bucket (far edges crowd the first
                                    // rows: at n = 65536 the first 512 rows of a pair
                                    // collect ~16k edges, about what LDS can stage)
constexpr int kMaxBuckets = 2048;   // n <= 2^20
static_assert(kBucket <= kClsRows - kCls3, "sort_runs' longest class holds a bucket's rows");

struct LongIndexArgs {
    const int32_t* idx;
    const float* w;
    const int* tgt;   // pair-major live targets (-1 dead) instead of idx/w, or null
    int n, hkv, s, npairs, nb, nch, vec;
    int* counts;   // [npairs][nb][nch]
    int* offs;     // [npairs][nb][nch]
    int* tot;      // [npairs]
    int2* stage;   // [npairs * n * s]
    int* beg;
    int* len;
    int* list;
    int* head;     // [pair-major row * 4] or null
};

// targets and edge ids (-1: dead) of the kTok tokens i0 + k * kIndexThreads
// + threadIdx.x of pair (b, h); unconditional loads from clamped addresses
template <bool VEC>
__device__ __forceinline__ void load_tokens(const LongIndexArgs& a, int b, int h, int i0,
                                            int (&tj)[kTok * kSlotMax],
                                            int (&te)[kTok * kSlotMax]) {
    const int n = a.n, s = a.s, hkv = a.hkv;
#pragma unroll
    for (int k = 0; k < kTok; ++k) {
        const int iv = i0 + k * kIndexThreads + (int)threadIdx.x;
        const bool ok = iv < n;
        const int i = ok ? iv : n - 1;
        const int e0 = ((b * n + i) * hkv + h) * s;
        if (a.tgt) {
            // compact rows: the live targets of this pair, contiguous per token
            const int* tr = a.tgt + ((size_t)(b * hkv + h) * n + i) * s;
            if constexpr (VEC) {
                const int4 t4 = *reinterpret_cast<const int4*>(tr);
                tj[k * 4 + 0] = t4.x; tj[k * 4 + 1] = t4.y;
                tj[k * 4 + 2] = t4.z; tj[k * 4 + 3] = t4.w;
            } else {
#pragma unroll
                for (int t = 0; t < kSlotMax; ++t) tj[k * kSlotMax + t] = tr[t < s ? t : s - 1];
            }
#pragma unroll
            for (int t = 0; t < kSlotMax; ++t) {
                const int sl = k * kSlotMax + t;
                te[sl] = ok && t < s && tj[sl] >= 0 ? e0 + t : -1;
            }
        } else if constexpr (VEC) {
            const int4 j4 = *reinterpret_cast<const int4*>(a.idx + e0);
            const float4 w4 = *reinterpret_cast<const float4*>(a.w + e0);
            tj[k * 4 + 0] = j4.x; tj[k * 4 + 1] = j4.y;
            tj[k * 4 + 2] = j4.z; tj[k * 4 + 3] = j4.w;
            te[k * 4 + 0] = ok && w4.x > 0.0f ? e0 + 0 : -1;
            te[k * 4 + 1] = ok && w4.y > 0.0f ? e0 + 1 : -1;
            te[k * 4 + 2] = ok && w4.z > 0.0f ? e0 + 2 : -1;
            te[k * 4 + 3] = ok && w4.w > 0.0f ? e0 + 3 : -1;
        } else {
#pragma unroll
            for (int t = 0; t < kSlotMax; ++t) {
                const int sl = k * kSlotMax + t;
                const int e = e0 + (t < s ? t : s - 1);
                tj[sl] = a.idx[e];
                te[sl] = ok && t < s && a.w[e] > 0.0f ? e : -1;
            }
        }
    }
}

// workgroup x + 8k runs on XCD x: XCD x takes consecutive items
__device__ __forceinline__ int xcd_item(int total) {
    int lin = (int)blockIdx.x;
    if (total % kXcds == 0)
        lin = ((int)blockIdx.x % kXcds) * (total / kXcds) + (int)blockIdx.x / kXcds;
    return lin;
}

template <bool VEC, bool SCATTER>
__global__ __launch_bounds__(kIndexThreads) void long_index_pass_kernel(LongIndexArgs a) {
    __shared__ int hist[kMaxBuckets];
    const int lin = xcd_item(a.npairs * a.nch);
    const int pair = lin / a.nch, c = lin - (lin / a.nch) * a.nch;
    const int b = pair / a.hkv, h = pair - (pair / a.hkv) * a.hkv;
    for (int k = threadIdx.x; k < a.nb; k += kIndexThreads)
        hist[k] = SCATTER ? a.offs[((size_t)pair * a.nb + k) * a.nch + c] : 0;
    __syncthreads();
    int tj[kTok * kSlotMax], te[kTok * kSlotMax];
    load_tokens<VEC>(a, b, h, c * kOneRows, tj, te);
    const size_t sbase = (size_t)pair * a.n * a.s;
#pragma unroll
    for (int k = 0; k < kTok * kSlotMax; ++k) {
        if (te[k] < 0 || (unsigned)tj[k] >= (unsigned)a.n) continue;   // dead (or invalid)
        const int bk = tj[k] / kBucket;
        const int pos = atomicAdd(&hist[bk], 1);
        if constexpr (SCATTER) a.stage[sbase + pos] = make_int2(te[k], tj[k]);
    }
    if constexpr (!SCATTER) {
        __syncthreads();
        for (int k = threadIdx.x; k < a.nb; k += kIndexThreads)
            a.counts[((size_t)pair * a.nb + k) * a.nch + c] = hist[k];
    }
}

// per pair: exclusive scan of counts in (bucket, chunk) order
__global__ __launch_bounds__(kIndexThreads) void long_index_scan_kernel(LongIndexArgs a) {
    __shared__ int part[kIndexThreads / kWave];
    const int pair = blockIdx.x;
    const int N = a.nb * a.nch;
    const int* cnt = a.counts + (size_t)pair * N;
    int* off = a.offs + (size_t)pair * N;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int run_len = (N + kIndexThreads - 1) / kIndexThreads;
    const int j0 = threadIdx.x * run_len;
    int run = 0;
    for (int j = j0; j < j0 + run_len && j < N; ++j) run += cnt[j];
    int inc = run;
    for (int m = 1; m < kWave; m <<= 1) {
        const int o = __shfl_up(inc, m, kWave);
        if (lane >= m) inc += o;
    }
    if (lane == kWave - 1) part[wave] = inc;
    __syncthreads();
    int base = 0;
    for (int k = 0; k < wave; ++k) base += part[k];
    if (threadIdx.x == kIndexThreads - 1) a.tot[pair] = base + inc;
    base += inc - run;
    for (int j = j0; j < j0 + run_len && j < N; ++j) {
        off[j] = base;
        base += cnt[j];
    }
}

// per (pair, bucket): counting sort of the bucket's edges by target row
__global__ __launch_bounds__(kIndexThreads) void long_index_sort_kernel(LongIndexArgs a) {
    __shared__ int cnt[kBucket];
    __shared__ int rlen[kBucket];
    __shared__ int rbeg[kBucket];
    __shared__ int sorted[kOneList];
    __shared__ int part[kIndexThreads / kWave];
    __shared__ int cls[kClsRows];   // rows grouped by run length for sort_runs
    __shared__ int ncls[4];
    const int lin = xcd_item(a.npairs * a.nb);
    const int pair = lin / a.nb, bk = lin - (lin / a.nb) * a.nb;
    const int n = a.n;
    const int jlo = bk * kBucket, jhi = jlo + kBucket < n ? jlo + kBucket : n;
    const int nr = jhi - jlo;
    const int* offp = a.offs + (size_t)pair * a.nb * a.nch;
    const int ebeg = offp[(size_t)bk * a.nch];
    const int eend = bk + 1 < a.nb ? offp[(size_t)(bk + 1) * a.nch] : a.tot[pair];
    const int ne = eend - ebeg;
    const size_t lbase = (size_t)pair * n * a.s;
    const int2* st = a.stage + lbase + ebeg;
    for (int j = threadIdx.x; j < nr; j += kIndexThreads) cnt[j] = 0;
    __syncthreads();
    // kUnroll independent loads per thread before their LDS atomics: the
    // first buckets collect most far edges, so their loops are long
    constexpr int kUnroll = 8;
    for (int p0 = 0; p0 < ne; p0 += kIndexThreads * kUnroll) {
        int row[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int p = p0 + u * kIndexThreads + (int)threadIdx.x;
            row[u] = p < ne ? st[p < ne ? p : 0].y - jlo : -1;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (row[u] >= 0) atomicAdd(&cnt[row[u]], 1);
    }
    __syncthreads();
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int run_len = (nr + kIndexThreads - 1) / kIndexThreads;
    const int j0 = threadIdx.x * run_len;
    int run = 0;
    for (int j = j0; j < j0 + run_len && j < nr; ++j) run += cnt[j];
    int inc = run;
    for (int m = 1; m < kWave; m <<= 1) {
        const int o = __shfl_up(inc, m, kWave);
        if (lane >= m) inc += o;
    }
    if (lane == kWave - 1) part[wave] = inc;
    __syncthreads();
    int base = 0;
    for (int k = 0; k < wave; ++k) base += part[k];
    base += inc - run;
    for (int j = j0; j < j0 + run_len && j < nr; ++j) {
        const int c = cnt[j];
        rlen[j] = c;
        cnt[j] = base;
        base += c;
    }
    __syncthreads();
    const size_t gbase = lbase + ebeg;   // list slot of the bucket's first edge
    for (int j = threadIdx.x; j < nr; j += kIndexThreads) {
        a.beg[(size_t)pair * n + jlo + j] = (int)(gbase + cnt[j]);
        a.len[(size_t)pair * n + jlo + j] = rlen[j];
        rbeg[j] = cnt[j];
    }
    __syncthreads();
    const bool staged = ne <= kOneList;
    // placement in an order the LDS atomics decide (varies between runs)
    for (int p0 = 0; p0 < ne; p0 += kIndexThreads * kUnroll) {
        int2 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int p = p0 + u * kIndexThreads + (int)threadIdx.x;
            v[u] = st[p < ne ? p : 0];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (p0 + u * kIndexThreads + (int)threadIdx.x >= ne) continue;
            const int pos = atomicAdd(&cnt[v[u].y - jlo], 1);
            if (staged) sorted[pos] = v[u].x;
            else a.list[gbase + pos] = v[u].x;
        }
    }
    __syncthreads();
    // ascending edge ids within every row; the staging entries, no longer
    // needed, give long runs outside LDS their spill space
    if (staged) {
        sort_runs(sorted, cnt, rlen, nr, cls, ncls, a.list + gbase);
        for (int p = threadIdx.x; p < ne; p += kIndexThreads) a.list[gbase + p] = sorted[p];
        if (a.head) write_heads(a.head, (size_t)pair * n + jlo, sorted, rbeg, rlen, nr);
    } else {
        sort_runs(a.list + gbase, cnt, rlen, nr, cls, ncls,
                  reinterpret_cast<int*>(a.stage + lbase + ebeg));
        if (a.head) write_heads(a.head, (size_t)pair * n + jlo, a.list + gbase, rbeg, rlen, nr);
    }
}

}  // namespace

bool edge_index_supported(int n, int s) {
    return s <= kSlotMax && (long long)n <= (long long)kBucket * kMaxBuckets;
}

bool edge_index_one_pass(int n) { return n <= kOneRows; }

hipError_t launch_edge_index(int B, int n, int hkv, const int32_t* idx, const float* w, int s,
                             const int* tgt, int* beg, int* len, int* list, int* head,
                             hipStream_t st) {
    if (n > kOneRows || s > kSlotMax) return hipErrorInvalidValue;
    IndexArgs a;
    a.idx = idx; a.w = w; a.tgt = tgt; a.n = n; a.hkv = hkv; a.s = s;
    a.npairs = B * hkv;
    // target ranges per pair: enough workgroups to fill the device's 256
    // compute units when there are few pairs
    a.K = 1;
    while (a.npairs * a.K < 256 && a.K < 8 && n >= 2 * a.K) a.K *= 2;
    a.vec = s == 4 && (tgt ? ((uintptr_t)tgt & 15) == 0
                           : (((uintptr_t)idx | (uintptr_t)w) & 15) == 0);
    a.beg = beg; a.len = len; a.list = list; a.head = head;
    const dim3 grid((unsigned)(a.npairs * a.K));
    if (a.vec)
        hipLaunchKernelGGL(edge_index_one_kernel<true>, grid, dim3(kIndexThreads), 0, st, a);
    else
        hipLaunchKernelGGL(edge_index_one_kernel<false>, grid, dim3(kIndexThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_edge_index_long(int B, int n, int hkv, const int32_t* idx, const float* w,
                                  int s, const int* tgt, int* beg, int* len, int* list,
                                  int* head, int* counts, int* offs, int* tot, int2* stage,
                                  hipStream_t st) {
    LongIndexArgs a;
    a.idx = idx; a.w = w; a.tgt = tgt; a.n = n; a.hkv = hkv; a.s = s;
    a.npairs = B * hkv;
    a.nb = (n + kBucket - 1) / kBucket;
    a.nch = (n + kOneRows - 1) / kOneRows;
    if (a.nb > kMaxBuckets || s > kSlotMax) return hipErrorInvalidValue;
    a.vec = s == 4 && (tgt ? ((uintptr_t)tgt & 15) == 0
                           : (((uintptr_t)idx | (uintptr_t)w) & 15) == 0);
    a.counts = counts;
    a.offs = offs;
    a.tot = tot;
    a.stage = stage;
    a.beg = beg; a.len = len; a.list = list; a.head = head;
    const dim3 gpass((unsigned)(a.npairs * a.nch)), th(kIndexThreads);
    if (a.vec) hipLaunchKernelGGL((long_index_pass_kernel<true, false>), gpass, th, 0, st, a);
    else hipLaunchKernelGGL((long_index_pass_kernel<false, false>), gpass, th, 0, st, a);
    hipLaunchKernelGGL(long_index_scan_kernel, dim3((unsigned)a.npairs), th, 0, st, a);
    if (a.vec) hipLaunchKernelGGL((long_index_pass_kernel<true, true>), gpass, th, 0, st, a);
    else hipLaunchKernelGGL((long_index_pass_kernel<false, true>), gpass, th, 0, st, a);
    hipLaunchKernelGGL(long_index_sort_kernel, dim3((unsigned)(a.npairs * a.nb)), th, 0, st, a);
    return hipGetLastError();
}

}  // namespace gm
