// C ABI of the Graph Machine sparse-layer path (declared in include/gm.h):
// host-side argument checks, then the kernel launches on the caller's stream.
// Nothing here allocates; every check happens before the first launch.
#include "gm.h"
#include "gm_internal.h"

#include <limits.h>
#include <stdint.h>

#include <mutex>

// Scratch space of gm_sea_backward_noalloc: one copy per GPU, held by the
// loaded code object until the process ends.  Host code never names it
// directly (its name is only a host-side stand-in); it takes the device
// address that hipGetSymbolAddress returns for the call's GPU.
static __device__ __align__(256) unsigned char scratch[GM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// Device address of `scratch` on the GPU that `stream` belongs to (the
// current GPU for the null stream), looked up once per GPU with that GPU
// current.
gm_status scratch_address(hipStream_t stream, void** out) {
    int dev = -1;
    if (stream) {
        if (hipStreamGetDevice(stream, &dev) != hipSuccess) return GM_ERR_HIP;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return GM_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return GM_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return GM_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return GM_ERR_HIP;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return GM_ERR_HIP;
        if (e != hipSuccess || !p) return GM_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GM_OK;
}

using gm::TeamShape;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool pow2_in(int x, int lo, int hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }

// Units and element counts must fit the kernels' index types.
gm_status check_units(int B, int n, int hkv) {
    if (B < 0 || n < 0 || hkv < 0) return GM_ERR_SHAPE;
    if ((long long)B * n * hkv >= (long long)INT_MAX) return GM_ERR_SHAPE;
    return GM_OK;
}

bool empty(int B, int n, int hkv) { return (long long)B * n * hkv == 0; }

gm_status check_edge_ptrs(const int32_t* idx, const float* w) {
    if (!idx || !w) return GM_ERR_NULL;
    if (!aligned(idx, 4) || !aligned(w, 4)) return GM_ERR_ALIGN;
    return GM_OK;
}

gm_status check_sea(int B, int n, int hq, int hkv, int d, gm_dtype dt, int s1) {
    gm_status st = check_units(B, n, hkv);
    if (st != GM_OK) return st;
    if (hq < 0) return GM_ERR_SHAPE;
    if (hkv == 0) return empty(B, n, hkv) ? GM_OK : GM_ERR_SHAPE;
    if (hq % hkv != 0 || hq == 0) return GM_ERR_UNSUPPORTED;
    if (!pow2_in(d, 16, 256)) return GM_ERR_UNSUPPORTED;
    if (dt != GM_F32 && dt != GM_BF16) return GM_ERR_UNSUPPORTED;
    if (s1 < 1 || s1 > 64) return GM_ERR_UNSUPPORTED;
    if ((long long)B * n * hq * d >= (1ll << 46)) return GM_ERR_SHAPE;
    return GM_OK;
}

gm_status check_ser(int B, int n, int hkv, int s1, int s2, int s3) {
    gm_status st = check_units(B, n, hkv);
    if (st != GM_OK) return st;
    if (s1 < 1 || s1 > 64 || s2 < 1 || s3 < 1 || s2 * s3 > 64) return GM_ERR_UNSUPPORTED;
    return GM_OK;
}

gm_status hip_status(hipError_t e) { return e == hipSuccess ? GM_OK : GM_ERR_HIP; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return a && b && x < y + bn && y < x + an;
}

}  // namespace

extern "C" {

int gm_abi_version(void) { return 8; }

const char* gm_status_string(gm_status s) {
    switch (s) {
        case GM_OK: return "ok";
        case GM_ERR_NULL: return "a required pointer is NULL";
        case GM_ERR_SHAPE: return "invalid or overflowing size";
        case GM_ERR_UNSUPPORTED: return "s, d, dtype or head ratio outside the supported set";
        case GM_ERR_WORKSPACE: return "workspace missing or too small";
        case GM_ERR_HIP: return "HIP launch or runtime error";
        case GM_ERR_ALIGN: return "pointer not aligned as required";
        case GM_ERR_ALIAS: return "an output overlaps an input";
        case GM_ERR_TOO_LARGE:
            return "sizes need more scratch than the fixed GM_NOALLOC_SCRATCH_BYTES of the "
                   "allocation-free call (use the call with a workspace)";
        case GM_STATUS_RANGE: break;
    }
    return "unknown status";
}

// The optional path map: produced for s1, s2, s3 <= 4; 8-byte aligned and
// overlapping none of the call's other arrays.
static gm_status check_paths(const uint64_t* paths, int s1, int s2, int s3, size_t rows,
                      const void* const* arrays, const size_t* bytes, int narrays) {
    if (!paths) return GM_OK;
    if (s1 > 4 || s2 > 4 || s3 > 4) return GM_ERR_UNSUPPORTED;
    if (!aligned(paths, 8)) return GM_ERR_ALIGN;
    for (int a = 0; a < narrays; ++a)
        if (arrays[a] && bytes[a] && overlaps(paths, rows * 8, arrays[a], bytes[a]))
            return GM_ERR_ALIAS;
    return GM_OK;
}

gm_status gm_ser_forward(int B, int n, int hkv, const int32_t* idx1, const float* w1, int s2,
                         const int32_t* idx2, const float* w2, int s3, int32_t* idx_out,
                         float* w_out, int s1, uint64_t* paths, hipStream_t stream) {
    gm_status st = check_ser(B, n, hkv, s1, s2, s3);
    if (st != GM_OK) return st;
    if (paths && (s1 > 4 || s2 > 4 || s3 > 4)) return GM_ERR_UNSUPPORTED;
    if (empty(B, n, hkv)) return GM_OK;
    if ((st = check_edge_ptrs(idx1, w1)) != GM_OK) return st;
    if ((st = check_edge_ptrs(idx2, w2)) != GM_OK) return st;
    if ((st = check_edge_ptrs(idx_out, w_out)) != GM_OK) return st;
    const size_t rows = (size_t)B * n * hkv;
    const size_t o4 = rows * s1 * 4;
    if (overlaps(idx_out, o4, idx1, rows * s2 * 4) || overlaps(idx_out, o4, w1, rows * s2 * 4) ||
        overlaps(idx_out, o4, idx2, rows * s3 * 4) || overlaps(idx_out, o4, w2, rows * s3 * 4) ||
        overlaps(w_out, o4, idx1, rows * s2 * 4) || overlaps(w_out, o4, w1, rows * s2 * 4) ||
        overlaps(w_out, o4, idx2, rows * s3 * 4) || overlaps(w_out, o4, w2, rows * s3 * 4) ||
        overlaps(idx_out, o4, w_out, o4))
        return GM_ERR_ALIAS;
    const void* arr[6] = {idx1, w1, idx2, w2, idx_out, w_out};
    const size_t arb[6] = {rows * s2 * 4, rows * s2 * 4, rows * s3 * 4, rows * s3 * 4, o4, o4};
    if ((st = check_paths(paths, s1, s2, s3, rows, arr, arb, 6)) != GM_OK) return st;
    return hip_status(gm::launch_ser_forward(B, n, hkv, idx1, w1, s2, idx2, w2, s3, idx_out,
                                             w_out, s1, paths, stream));
}

gm_status gm_ser_forward_chain2(int B, int n, int hkv, const int32_t* idx, const float* w,
                                int s, int32_t* idx_mid, float* w_mid, int32_t* idx_out,
                                float* w_out, hipStream_t stream) {
    gm_status st = check_ser(B, n, hkv, s, s, s);
    if (st != GM_OK) return st;
    if (s != 2 && s != 4) return GM_ERR_UNSUPPORTED;
    if (empty(B, n, hkv)) return GM_OK;
    if ((st = check_edge_ptrs(idx, w)) != GM_OK) return st;
    if ((st = check_edge_ptrs(idx_out, w_out)) != GM_OK) return st;
    if (!idx_mid != !w_mid) return GM_ERR_NULL;
    const uintptr_t row = (uintptr_t)s * 4;
    if (!aligned(idx, row) || !aligned(w, row) || !aligned(idx_out, row) ||
        !aligned(w_out, row) || (idx_mid && (!aligned(idx_mid, row) || !aligned(w_mid, row))))
        return GM_ERR_ALIGN;
    const size_t bytes = (size_t)B * n * hkv * s * 4;
    const void* ins[2] = {idx, w};
    const void* outs[4] = {idx_out, w_out, idx_mid, w_mid};
    for (int o = 0; o < 4; ++o) {
        for (int i = 0; i < 2; ++i)
            if (overlaps(outs[o], bytes, ins[i], bytes)) return GM_ERR_ALIAS;
        for (int o2 = o + 1; o2 < 4; ++o2)
            if (overlaps(outs[o], bytes, outs[o2], bytes)) return GM_ERR_ALIAS;
    }
    return hip_status(gm::launch_ser_chain2(B, n, hkv, idx, w, s, idx_mid, w_mid, idx_out, w_out,
                                            stream));
}

gm_status gm_sea_forward(int B, int n, int hq, int hkv, int d, gm_dtype dt, float scale,
                         const void* q, const void* k, const void* v, const int32_t* idx,
                         const float* w, int s1, void* o, float* stats, hipStream_t stream) {
    gm_status st = check_sea(B, n, hq, hkv, d, dt, s1);
    if (st != GM_OK) return st;
    if (empty(B, n, hkv)) return GM_OK;
    if (!q || !k || !v || !o) return GM_ERR_NULL;
    if ((st = check_edge_ptrs(idx, w)) != GM_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        (stats && !aligned(stats, 16)))
        return GM_ERR_ALIGN;
    const size_t es = dt == GM_BF16 ? 2 : 4;
    const size_t qb = (size_t)B * n * hq * d * es, kb = (size_t)B * n * hkv * d * es;
    const size_t eb = (size_t)B * n * hkv * s1 * 4;
    // statistics: E G + 2 rows of s1 words per unit (E = 2 for fp32 inputs)
    const size_t sb = (size_t)B * n * ((dt == GM_BF16 ? 1 : 2) * hq + 2 * hkv) * s1 * 4;
    if (overlaps(o, qb, q, qb) || overlaps(o, qb, k, kb) || overlaps(o, qb, v, kb) ||
        overlaps(o, qb, idx, eb) || overlaps(o, qb, w, eb))
        return GM_ERR_ALIAS;
    if (stats && (overlaps(stats, sb, q, qb) || overlaps(stats, sb, k, kb) ||
                  overlaps(stats, sb, v, kb) || overlaps(stats, sb, idx, eb) ||
                  overlaps(stats, sb, w, eb) || overlaps(stats, sb, o, qb)))
        return GM_ERR_ALIAS;
    return hip_status(gm::launch_sea_forward(B, n, hq, hkv, d, dt == GM_BF16, scale, q, k, v,
                                             idx, w, s1, o, stats, stream));
}

gm_status gm_ser_sea_forward(int B, int n, int hq, int hkv, int d, gm_dtype dt, float scale,
                             const int32_t* idx1, const float* w1, int s2, const int32_t* idx2,
                             const float* w2, int s3, int s1, const void* q, const void* k,
                             const void* v, int32_t* idx_out, float* w_out, void* o,
                             float* stats, uint64_t* paths, hipStream_t stream) {
    gm_status st = check_ser(B, n, hkv, s1, s2, s3);
    if (st != GM_OK) return st;
    if ((st = check_sea(B, n, hq, hkv, d, dt, s1)) != GM_OK) return st;
    if (paths && (s1 > 4 || s2 > 4 || s3 > 4)) return GM_ERR_UNSUPPORTED;
    if (empty(B, n, hkv)) return GM_OK;
    if ((st = check_edge_ptrs(idx1, w1)) != GM_OK) return st;
    if ((st = check_edge_ptrs(idx2, w2)) != GM_OK) return st;
    if ((st = check_edge_ptrs(idx_out, w_out)) != GM_OK) return st;
    if (!q || !k || !v || !o) return GM_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        (stats && !aligned(stats, 16)))
        return GM_ERR_ALIGN;
    const size_t es = dt == GM_BF16 ? 2 : 4;
    const size_t rows = (size_t)B * n * hkv;
    const size_t qb = (size_t)B * n * hq * d * es, kb = (size_t)B * n * hkv * d * es;
    const size_t sb = (size_t)B * n * ((dt == GM_BF16 ? 1 : 2) * hq + 2 * hkv) * s1 * 4;
    const void* ins[7] = {idx1, w1, idx2, w2, q, k, v};
    const size_t inb[7] = {rows * s2 * 4, rows * s2 * 4, rows * s3 * 4, rows * s3 * 4, qb, kb, kb};
    const void* outs[4] = {idx_out, w_out, o, stats};
    const size_t outb[4] = {rows * s1 * 4, rows * s1 * 4, qb, stats ? sb : 0};
    for (int a = 0; a < 4; ++a) {
        if (!outb[a]) continue;
        for (int b = 0; b < 7; ++b)
            if (overlaps(outs[a], outb[a], ins[b], inb[b])) return GM_ERR_ALIAS;
        for (int b = a + 1; b < 4; ++b)
            if (outb[b] && overlaps(outs[a], outb[a], outs[b], outb[b])) return GM_ERR_ALIAS;
    }
    const void* arr[11] = {idx1, w1, idx2, w2, q, k, v, idx_out, w_out, o, stats};
    const size_t arb[11] = {inb[0], inb[1], inb[2], inb[3], inb[4], inb[5], inb[6],
                            outb[0], outb[1], outb[2], outb[3]};
    if ((st = check_paths(paths, s1, s2, s3, rows, arr, arb, 11)) != GM_OK) return st;
    return hip_status(gm::launch_ser_sea_forward(B, n, hq, hkv, d, dt == GM_BF16, scale, idx1, w1,
                                                 s2, idx2, w2, s3, s1, q, k, v, idx_out, w_out,
                                                 o, stats, paths, stream));
}

gm_status gm_leg_mix_forward(int B, int n, int hkv, const int32_t* idx, const float* w, int K,
                             const float* alpha, int s, int32_t* idx_out, float* w_out,
                             hipStream_t stream) {
    gm_status st = check_units(B, n, hkv);
    if (st != GM_OK) return st;
    if (K < 1 || K > 64 || s < 1 || s > 64) return GM_ERR_UNSUPPORTED;
    if (empty(B, n, hkv)) return GM_OK;
    if ((st = check_edge_ptrs(idx, w)) != GM_OK) return st;
    if ((st = check_edge_ptrs(idx_out, w_out)) != GM_OK) return st;
    if (!alpha) return GM_ERR_NULL;
    if (!aligned(alpha, 4)) return GM_ERR_ALIGN;
    const size_t rows = (size_t)B * n * hkv;
    const void* ins[3] = {idx, w, alpha};
    const size_t inb[3] = {rows * K * 4, rows * K * 4, (size_t)hkv * K * 4};
    const void* outs[2] = {idx_out, w_out};
    const size_t outb[2] = {rows * s * 4, rows * s * 4};
    for (int a = 0; a < 2; ++a) {
        for (int b = 0; b < 3; ++b)
            if (overlaps(outs[a], outb[a], ins[b], inb[b])) return GM_ERR_ALIAS;
    }
    if (overlaps(idx_out, outb[0], w_out, outb[1])) return GM_ERR_ALIAS;
    return hip_status(
        gm::launch_leg_mix_forward(B, n, hkv, idx, w, K, alpha, s, idx_out, w_out, stream));
}

size_t gm_leg_mix_backward_workspace_bytes(int B, int n, int hkv, int K) {
    if (check_units(B, n, hkv) != GM_OK || K < 1 || K > 64) return 0;
    return gm::leg_mix_backward_workspace_bytes(B, n, hkv, K);
}

gm_status gm_leg_mix_backward(int B, int n, int hkv, const int32_t* idx, const float* w, int K,
                              const float* alpha, const int32_t* idx_out, const float* w_out,
                              int s, const float* dleg, float* dw, float* dalpha, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    gm_status st = check_units(B, n, hkv);
    if (st != GM_OK) return st;
    if (K < 1 || K > 64 || s < 1 || s > 64) return GM_ERR_UNSUPPORTED;
    if (empty(B, n, hkv)) return GM_OK;
    if ((st = check_edge_ptrs(idx, w)) != GM_OK) return st;
    if ((st = check_edge_ptrs(idx_out, w_out)) != GM_OK) return st;
    if (!alpha || !dleg || !dw || !dalpha) return GM_ERR_NULL;
    if (!aligned(alpha, 4) || !aligned(dleg, 4) || !aligned(dw, 4) || !aligned(dalpha, 4))
        return GM_ERR_ALIGN;
    const size_t need = gm_leg_mix_backward_workspace_bytes(B, n, hkv, K);
    if (!workspace || workspace_bytes < need) return GM_ERR_WORKSPACE;
    if (!aligned(workspace, 8)) return GM_ERR_ALIGN;
    const size_t rows = (size_t)B * n * hkv;
    const void* ins[6] = {idx, w, alpha, idx_out, w_out, dleg};
    const size_t inb[6] = {rows * K * 4, rows * K * 4, (size_t)hkv * K * 4, rows * s * 4,
                           rows * s * 4, rows * s * 4};
    const void* outs[3] = {dw, dalpha, workspace};
    const size_t outb[3] = {rows * K * 4, (size_t)hkv * K * 4, need};
    for (int a = 0; a < 3; ++a) {
        for (int b = 0; b < 6; ++b)
            if (overlaps(outs[a], outb[a], ins[b], inb[b])) return GM_ERR_ALIAS;
        for (int b = a + 1; b < 3; ++b)
            if (overlaps(outs[a], outb[a], outs[b], outb[b])) return GM_ERR_ALIAS;
    }
    return hip_status(gm::launch_leg_mix_backward(B, n, hkv, idx, w, K, alpha, idx_out, w_out, s,
                                                  dleg, dw, dalpha,
                                                  static_cast<double*>(workspace), stream));
}

gm_status gm_decode_step(int B, int T, int hq, int hkv, int d, gm_dtype dt, float scale,
                         const int32_t* idx1, const float* w1, int s2, const int32_t* idx2,
                         const float* w2, int s3, int s1, const void* q, const void* k,
                         const void* v, int32_t* idx_out, float* w_out, void* o,
                         hipStream_t stream) {
    gm_status st = check_sea(B, T, hq, hkv, d, dt, s1);
    if (st != GM_OK) return st;
    if ((st = check_ser(B, T, hkv, s1, s2, s3)) != GM_OK) return st;
    // the decode kernel keeps the group's query rows in registers, built for
    // these group sizes
    if (hkv > 0 && !pow2_in(hq / hkv, 1, 16)) return GM_ERR_UNSUPPORTED;
    if ((long long)B * hkv == 0) return GM_OK;
    if (T < 1) return GM_ERR_SHAPE;
    if (!q || !k || !v || !o) return GM_ERR_NULL;
    if ((st = check_edge_ptrs(idx1, w1)) != GM_OK) return st;
    if ((st = check_edge_ptrs(idx2, w2)) != GM_OK) return st;
    if (!idx_out || !w_out) return GM_ERR_NULL;
    if (!aligned(idx_out, 4) || !aligned(w_out, 4)) return GM_ERR_ALIGN;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
        return GM_ERR_ALIGN;
    const size_t es = dt == GM_BF16 ? 2 : 4;
    const size_t units = (size_t)B * hkv;
    const size_t qb = (size_t)B * hq * d * es, kb = (size_t)B * T * hkv * d * es;
    const void* ins[7] = {idx1, w1, idx2, w2, q, k, v};
    const size_t inb[7] = {units * s2 * 4, units * s2 * 4, units * T * s3 * 4,
                           units * T * s3 * 4, qb, kb, kb};
    const void* outs[3] = {idx_out, w_out, o};
    const size_t outb[3] = {units * s1 * 4, units * s1 * 4, qb};
    for (int a = 0; a < 3; ++a) {
        for (int b = 0; b < 7; ++b)
            if (overlaps(outs[a], outb[a], ins[b], inb[b])) return GM_ERR_ALIAS;
        for (int b = a + 1; b < 3; ++b)
            if (overlaps(outs[a], outb[a], outs[b], outb[b])) return GM_ERR_ALIAS;
    }
    return hip_status(gm::launch_decode_step(B, T, hq, hkv, d, dt == GM_BF16, scale, idx1, w1,
                                             s2, idx2, w2, s3, s1, q, k, v, idx_out, w_out, o,
                                             stream));
}

gm_status gm_dense_refresh(int B, int n, int hq, int hkv, int d, gm_dtype dt, float scale,
                           const void* q, const void* k, int s, int lse_given, float* lse,
                           int32_t* idx_out, float* w_out, hipStream_t stream) {
    gm_status st = check_units(B, n, hkv);
    if (st != GM_OK) return st;
    if (hq < 0) return GM_ERR_SHAPE;
    if (hkv == 0) return empty(B, n, hkv) ? GM_OK : GM_ERR_SHAPE;
    if (hq == 0 || hq % hkv != 0) return GM_ERR_UNSUPPORTED;
    if (dt != GM_BF16 || !gm::dense_refresh_supported(d, hq / hkv, s)) return GM_ERR_UNSUPPORTED;
    if (!(scale > 0.0f) || scale > 3.4e38f) return GM_ERR_UNSUPPORTED;   // positive and finite
    if ((long long)B * n * hq * d >= (1ll << 46)) return GM_ERR_SHAPE;
    if (empty(B, n, hkv)) return GM_OK;
    if (!q || !k || !lse) return GM_ERR_NULL;
    if ((st = check_edge_ptrs(idx_out, w_out)) != GM_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(lse, 4)) return GM_ERR_ALIGN;
    const size_t qb = (size_t)B * n * hq * d * 2, kb = (size_t)B * n * hkv * d * 2;
    const size_t lb = (size_t)B * n * hq * 4, eb = (size_t)B * n * hkv * s * 4;
    const void* ins[2] = {q, k};
    const size_t inb[2] = {qb, kb};
    const void* outs[3] = {lse, idx_out, w_out};
    const size_t outb[3] = {lb, eb, eb};
    for (int a = 0; a < 3; ++a) {
        for (int b = 0; b < 2; ++b)
            if (overlaps(outs[a], outb[a], ins[b], inb[b])) return GM_ERR_ALIAS;
        for (int b = a + 1; b < 3; ++b)
            if (overlaps(outs[a], outb[a], outs[b], outb[b])) return GM_ERR_ALIAS;
    }
    return hip_status(gm::launch_dense_refresh(B, n, hq, hkv, d, scale, q, k, s, lse_given != 0,
                                               lse, idx_out, w_out, stream));
}

size_t gm_sea_backward_workspace_bytes(int B, int n, int hq, int hkv, int s1) {
    if (check_units(B, n, hkv) != GM_OK || hkv <= 0 || hq <= 0 || hq % hkv || s1 < 1) return 0;
    return gm::sea_backward_workspace_bytes((long long)B * n * hkv, s1, hq / hkv, n);
}

}  // extern "C"

namespace {

// Every host-side check of gm_sea_backward; `workspace` null: the
// allocation-free call, whose scratch is the library's own (no workspace
// checks).  Returns GM_OK when the call may launch.
gm_status sea_backward_checks(int B, int n, int hq, int hkv, int d, gm_dtype dt,
                              const void* q, const void* k, const void* v, const int32_t* idx,
                              const float* w, int s1, const void* dout, const float* stats,
                              float* dq, float* dk, float* dv, float* dw, const void* workspace,
                              size_t workspace_bytes) {
    if ((long long)B * n * hkv * s1 >= (long long)INT_MAX) return GM_ERR_SHAPE;
    if (!q || !k || !v || !dout || !dq || !dk || !dv || !dw) return GM_ERR_NULL;
    gm_status st;
    if ((st = check_edge_ptrs(idx, w)) != GM_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) ||
        !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(dw, 4) ||
        (stats && !aligned(stats, 16)))
        return GM_ERR_ALIGN;
    const size_t es = dt == GM_BF16 ? 2 : 4;
    const size_t nq = (size_t)B * n * hq * d, nk = (size_t)B * n * hkv * d;
    const size_t ne = (size_t)B * n * hkv * s1;
    // statistics: E G + 2 rows of s1 words per unit (E = 2 for fp32 inputs)
    const size_t ns = (size_t)B * n * ((dt == GM_BF16 ? 1 : 2) * hq + 2 * hkv) * s1;
    const void* ins[7] = {q, k, v, dout, idx, w, stats};
    const size_t inb[7] = {nq * es, nk * es, nk * es, nq * es, ne * 4, ne * 4,
                           stats ? ns * 4 : 0};
    const size_t need = gm_sea_backward_workspace_bytes(B, n, hq, hkv, s1);
    if (workspace) {
        if (workspace_bytes < need) return GM_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return GM_ERR_ALIGN;
    }
    const void* outs[5] = {dq, dk, dv, dw, workspace};
    const size_t outb[5] = {nq * 4, nk * 4, nk * 4, ne * 4, workspace ? need : 0};
    for (int a = 0; a < 5; ++a) {
        for (int b = 0; b < 7; ++b)
            if (inb[b] && outb[a] && overlaps(outs[a], outb[a], ins[b], inb[b]))
                return GM_ERR_ALIAS;
        for (int b = a + 1; b < 5; ++b)
            if (outb[a] && outb[b] && overlaps(outs[a], outb[a], outs[b], outb[b]))
                return GM_ERR_ALIAS;
    }
    return GM_OK;
}

}  // namespace

extern "C" {

gm_status gm_sea_backward(int B, int n, int hq, int hkv, int d, gm_dtype dt, float scale,
                          const void* q, const void* k, const void* v, const int32_t* idx,
                          const float* w, int s1, const void* dout, const float* stats,
                          float* dq, float* dk, float* dv, float* dw, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
    gm_status st = check_sea(B, n, hq, hkv, d, dt, s1);
    if (st != GM_OK) return st;
    if (empty(B, n, hkv)) return GM_OK;
    if (!workspace) return GM_ERR_WORKSPACE;
    if ((st = sea_backward_checks(B, n, hq, hkv, d, dt, q, k, v, idx, w, s1, dout, stats, dq, dk,
                                  dv, dw, workspace, workspace_bytes)) != GM_OK)
        return st;
    return hip_status(gm::launch_sea_backward(B, n, hq, hkv, d, dt == GM_BF16, scale, q, k, v,
                                              idx, w, s1, dout, stats, dq, dk, dv, dw,
                                              workspace, stream));
}

gm_status gm_sea_backward_noalloc(int B, int n, int hq, int hkv, int d, gm_dtype dt, float scale,
                                  const void* q, const void* k, const void* v,
                                  const int32_t* idx, const float* w, int s1, const void* dout,
                                  const float* stats, float* dq, float* dk, float* dv, float* dw,
                                  hipStream_t stream) {
    gm_status st = check_sea(B, n, hq, hkv, d, dt, s1);
    if (st != GM_OK) return st;
    if (empty(B, n, hkv)) return GM_OK;
    if ((st = sea_backward_checks(B, n, hq, hkv, d, dt, q, k, v, idx, w, s1, dout, stats, dq, dk,
                                  dv, dw, nullptr, 0)) != GM_OK)
        return st;
    if (gm_sea_backward_workspace_bytes(B, n, hq, hkv, s1) > GM_NOALLOC_SCRATCH_BYTES)
        return GM_ERR_TOO_LARGE;
    void* ws = nullptr;
    if ((st = scratch_address(stream, &ws)) != GM_OK) return st;
    // the workspace's contents on entry do not matter (the kernels fill
    // what they read): nothing to clear, and no allocation
    return hip_status(gm::launch_sea_backward(B, n, hq, hkv, d, dt == GM_BF16, scale, q, k, v,
                                              idx, w, s1, dout, stats, dq, dk, dv, dw, ws,
                                              stream));
}

size_t gm_ser_backward_workspace_bytes(int B, int n, int hkv, int s2, int s3, int aliased) {
    (void)aliased;
    if (check_units(B, n, hkv) != GM_OK || s2 < 1 || s3 < 1) return 0;
    const size_t rows = (size_t)B * n * hkv;
    const size_t acc = rows * s2 * sizeof(double) + rows * s3 * sizeof(double);
    const size_t pull = gm::ser_backward_pull_bytes((long long)rows, s2);
    size_t need = acc > pull ? acc : pull;
    if (s2 == 4 && s3 == 4) {
        const size_t part = gm::ser_backward_part_bytes(B, n, hkv);
        if (part > need) need = part;
    }
    return need;
}

gm_status gm_ser_backward(int B, int n, int hkv, const int32_t* idx1, const float* w1, int s2,
                          const int32_t* idx2, const float* w2, int s3,
                          const int32_t* idx_out, const float* w_out, int s1,
                          const float* dw_out, const uint64_t* paths, float* dw1, float* dw2,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
    gm_status st = check_ser(B, n, hkv, s1, s2, s3);
    if (st != GM_OK) return st;
    if (paths && (s1 > 4 || s2 > 4 || s3 > 4)) return GM_ERR_UNSUPPORTED;
    if (empty(B, n, hkv)) return GM_OK;
    if ((st = check_edge_ptrs(idx1, w1)) != GM_OK) return st;
    if ((st = check_edge_ptrs(idx2, w2)) != GM_OK) return st;
    if ((st = check_edge_ptrs(idx_out, w_out)) != GM_OK) return st;
    if (!dw_out || !dw1 || !dw2) return GM_ERR_NULL;
    if (!aligned(dw_out, 4) || !aligned(dw1, 4) || !aligned(dw2, 4)) return GM_ERR_ALIGN;
    const bool aliased = dw1 == dw2;
    if (aliased && s2 != s3) return GM_ERR_ALIAS;
    const size_t need = gm_ser_backward_workspace_bytes(B, n, hkv, s2, s3, aliased);
    if (!workspace || workspace_bytes < need) return GM_ERR_WORKSPACE;
    if (!aligned(workspace, 8)) return GM_ERR_ALIGN;
    const size_t rows = (size_t)B * n * hkv;
    const void* ins[7] = {idx1, w1, idx2, w2, idx_out, w_out, dw_out};
    const size_t inb[7] = {rows * s2 * 4, rows * s2 * 4, rows * s3 * 4, rows * s3 * 4,
                           rows * s1 * 4, rows * s1 * 4, rows * s1 * 4};
    const void* outs[3] = {dw1, dw2, workspace};
    const size_t outb[3] = {rows * s2 * 4, rows * s3 * 4, need};
    for (int a = 0; a < 3; ++a) {
        for (int b = 0; b < 7; ++b)
            if (overlaps(outs[a], outb[a], ins[b], inb[b])) return GM_ERR_ALIAS;
        for (int b = a + 1; b < 3; ++b) {
            if (a == 0 && b == 1 && aliased) continue;
            if (overlaps(outs[a], outb[a], outs[b], outb[b])) return GM_ERR_ALIAS;
        }
    }
    const void* arr[10] = {idx1, w1, idx2, w2, idx_out, w_out, dw_out, dw1, dw2, workspace};
    const size_t arb[10] = {inb[0], inb[1], inb[2], inb[3], inb[4], inb[5], inb[6],
                            outb[0], outb[1], outb[2]};
    if ((st = check_paths(paths, s1, s2, s3, rows, arr, arb, 10)) != GM_OK) return st;
    double* ws1 = static_cast<double*>(workspace);
    double* ws2 = ws1 + rows * s2;
    return hip_status(gm::launch_ser_backward(B, n, hkv, idx1, w1, s2, idx2, w2, s3, idx_out,
                                              w_out, s1, dw_out, paths, dw1, dw2, ws1, ws2,
                                              stream));
}

gm_status gm_check_edges(int B, int n, int hkv, const int32_t* idx, const float* w, int s,
                         unsigned long long* counts, hipStream_t stream) {
    gm_status st = check_units(B, n, hkv);
    if (st != GM_OK) return st;
    if (s < 1) return GM_ERR_SHAPE;
    if (empty(B, n, hkv)) return GM_OK;
    if ((st = check_edge_ptrs(idx, w)) != GM_OK) return st;
    if (!counts) return GM_ERR_NULL;
    if (!aligned(counts, 8)) return GM_ERR_ALIGN;
    return hip_status(gm::launch_check_edges(B, n, hkv, idx, w, s, counts, stream));
}

}  // extern "C"
