// Gather-ceiling probe (measurement only; not part of the layer path).
//
// How fast can this GPU bring 256-byte rows to 16-lane rows of a wavefront
// (lane r reads bytes [16r, 16r + 16) of its row: the access pattern of the
// SEA kernels' K/V and q/dout gathers), as a function of how many distinct
// rows each XCD draws from (its "set") and how many row loads each 16-lane
// team keeps in flight?  Workgroups are dealt to the 8 XCDs round robin, as
// in the layer kernels; XCD x reads only its own table region and index
// list, so a set of S bytes per XCD competes for that XCD's 4 MB L2 alone.
//
//   int gm_probe_gather(const void* table, long long rows_per_xcd,
//                       const int* idx, long long n_per_xcd, int in_flight,
//                       unsigned* sink, int grid, hipStream_t stream);
//
//   table  [8][rows_per_xcd][256 bytes], device
//   idx    [8][n_per_xcd] row numbers in [0, rows_per_xcd), device
//   sink   [grid * 256] words, device: an xor of everything read, so that
//          no load is dead
//   in_flight in {1, 2, 4}: row loads per team issued before the first is
//          used; the next group's row numbers are read before the current
//          rows are waited on (as the layer kernels do with their edge ids)
//   grid   workgroups of 256 threads, a multiple of 8
// Returns 0, 1 for bad arguments, 2 when the launch fails.
//
// Dispatch-rate probe (same library): how long does the GPU take just to
// start `waves` wavefronts that each store one word per lane, dealt as
// one-wavefront workgroups or as four-wavefront workgroups?  The SEA
// backward's target pass starts one one-wavefront workgroup per target row.
//
//   int gm_probe_dispatch(unsigned* out, long long waves, int waves_per_wg,
//                         hipStream_t stream);
//
//   out    [waves * 64] words, device (every word written once)
//   waves_per_wg in {1, 4}; waves a multiple of waves_per_wg
// Returns 0, 1 for bad arguments, 2 when the launch fails.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kXcds = 8;
constexpr int kBlock = 256;
constexpr int kTeam = 16;

template <int INF>
__global__ __launch_bounds__(kBlock) void gather_probe_kernel(const uint4* __restrict__ table,
                                                              long long rows_per_xcd,
                                                              const int* __restrict__ idx,
                                                              long long n_per_xcd,
                                                              unsigned* __restrict__ sink) {
    const int x = blockIdx.x % kXcds;
    const long long team = (long long)(blockIdx.x / kXcds) * (kBlock / kTeam) + threadIdx.x / kTeam;
    const long long teams = (long long)(gridDim.x / kXcds) * (kBlock / kTeam);
    const int r = threadIdx.x & (kTeam - 1);
    const uint4* tx = table + (size_t)x * (size_t)rows_per_xcd * (256 / 16);
    const int* ix = idx + (size_t)x * (size_t)n_per_xcd;
    const long long last = n_per_xcd - 1;
    uint4 acc = make_uint4(0u, 0u, 0u, 0u);
    long long k = team * INF;
    int id[INF];
#pragma unroll
    for (int f = 0; f < INF; ++f) id[f] = ix[k + f < last ? k + f : last];
    for (; k < n_per_xcd; k += teams * INF) {
        uint4 v[INF];
#pragma unroll
        for (int f = 0; f < INF; ++f) v[f] = tx[(size_t)id[f] * (256 / 16) + r];
        const long long kn = k + teams * INF;
#pragma unroll
        for (int f = 0; f < INF; ++f) id[f] = ix[kn + f < last ? kn + f : last];
#pragma unroll
        for (int f = 0; f < INF; ++f) {
            const uint32_t m = k + f <= last ? ~0u : 0u;   // past the end: read, not counted
            acc.x ^= v[f].x & m; acc.y ^= v[f].y & m; acc.z ^= v[f].z & m; acc.w ^= v[f].w & m;
        }
    }
    sink[(size_t)blockIdx.x * kBlock + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" int gm_probe_gather(const void* table, long long rows_per_xcd, const int* idx,
                               long long n_per_xcd, int in_flight, unsigned* sink, int grid,
                               hipStream_t stream) {
    if (!table || !idx || !sink || rows_per_xcd < 1 || n_per_xcd < 1 || grid < kXcds ||
        grid % kXcds != 0)
        return 1;
    const uint4* t = static_cast<const uint4*>(table);
    switch (in_flight) {
        case 1:
            hipLaunchKernelGGL(gather_probe_kernel<1>, dim3(grid), dim3(kBlock), 0, stream, t,
                               rows_per_xcd, idx, n_per_xcd, sink);
            break;
        case 2:
            hipLaunchKernelGGL(gather_probe_kernel<2>, dim3(grid), dim3(kBlock), 0, stream, t,
                               rows_per_xcd, idx, n_per_xcd, sink);
            break;
        case 4:
            hipLaunchKernelGGL(gather_probe_kernel<4>, dim3(grid), dim3(kBlock), 0, stream, t,
                               rows_per_xcd, idx, n_per_xcd, sink);
            break;
        default:
            return 1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

namespace {

template <int W>
__global__ __launch_bounds__(64 * W) void dispatch_probe_kernel(unsigned* __restrict__ out) {
    out[(size_t)blockIdx.x * (64 * W) + threadIdx.x] = blockIdx.x;
}

}  // namespace

extern "C" int gm_probe_dispatch(unsigned* out, long long waves, int waves_per_wg,
                                 hipStream_t stream) {
    if (!out || waves < 1 || (waves_per_wg != 1 && waves_per_wg != 4) ||
        waves % waves_per_wg != 0 || waves / waves_per_wg > 0x7fffffffLL)
        return 1;
    const unsigned grid = (unsigned)(waves / waves_per_wg);
    if (waves_per_wg == 1)
        hipLaunchKernelGGL(dispatch_probe_kernel<1>, dim3(grid), dim3(64), 0, stream, out);
    else
        hipLaunchKernelGGL(dispatch_probe_kernel<4>, dim3(grid), dim3(256), 0, stream, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
