// Internal launch interface between the C ABI (gm_api.hip) and the kernels.
// Host code only; argument checking has already happened when these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gm_wave.h"

namespace gm {

// Lane team of one unit in the SEA kernels: R lanes hold one d-row (16 bytes
// each), P slots are handled side by side, team = R * P lanes (<= 64), and
// the s slots are walked in nchunk chunks of P.
struct TeamShape {
    int R, P, team, nchunk, log2R;
};
TeamShape sea_team(int d, int elem_bytes, int s);

// paths: optional path map per unit (s2, s3, s1 <= 4), read back by the
// backward's source-chunk kernel; ignored for other shapes.
hipError_t launch_ser_forward(int B, int n, int hkv, const int32_t* idx1, const float* w1,
                              int s2, const int32_t* idx2, const float* w2, int s3,
                              int32_t* idx_out, float* w_out, int s1, uint64_t* paths,
                              hipStream_t st);

// Two chained referral steps in one launch (s1 = s2 = s3 = s, s = 2 or 4,
// rows s-word aligned): A2 = Sp(A1 A1), A1 = Sp(A0 A0); idx_mid / w_mid
// receive A1 when not null.
hipError_t launch_ser_chain2(int B, int n, int hkv, const int32_t* idx, const float* w, int s,
                             int32_t* idx_mid, float* w_mid, int32_t* idx_out, float* w_out,
                             hipStream_t st);

// The 16-lane-row fast kernels apply: one d-row is 256 bytes, s <= 4, and
// activation tensors are addressable with 32-bit byte offsets.
bool sea_fast_shape(int B, int n, int hq, int hkv, int d, bool bf16, int s);
// Group sizes (query heads per KV head) the row kernels are built for; other
// sizes take the general kernels.
bool sea_row_group(int G);

hipError_t launch_sea_forward(int B, int n, int hq, int hkv, int d, bool bf16, float scale,
                              const void* q, const void* k, const void* v,
                              const int32_t* idx, const float* w, int s, void* o,
                              float* stats, hipStream_t st);

// SER then SEA forward in one call: one fused kernel where
// ser_sea_fused_shape holds (bf16, d = 128, s1 = s2 = s3 = 4, 16-byte aligned
// edge rows, a row-kernel group size), else the two launches in sequence.
bool ser_sea_fused_shape(int B, int n, int hq, int hkv, int d, bool bf16, int s1, int s2, int s3,
                         const void* idx1, const void* w1, const void* idx2, const void* w2,
                         const void* idx_out, const void* w_out);
hipError_t launch_ser_sea_forward(int B, int n, int hq, int hkv, int d, bool bf16, float scale,
                                  const int32_t* idx1, const float* w1, int s2,
                                  const int32_t* idx2, const float* w2, int s3, int s1,
                                  const void* q, const void* k, const void* v,
                                  int32_t* idx_out, float* w_out, void* o, float* stats,
                                  uint64_t* paths, hipStream_t st);

// Leg construction (stored edges mixed into a leg), forward and backward.
size_t leg_mix_backward_workspace_bytes(int B, int n, int hkv, int K);
hipError_t launch_leg_mix_forward(int B, int n, int hkv, const int32_t* idx, const float* w,
                                  int K, const float* alpha, int s, int32_t* idx_out,
                                  float* w_out, hipStream_t st);
hipError_t launch_leg_mix_backward(int B, int n, int hkv, const int32_t* idx, const float* w,
                                   int K, const float* alpha, const int32_t* idx_out,
                                   const float* w_out, int s, const float* dleg, float* dw,
                                   float* dalpha, double* part, hipStream_t st);

// One decode step (SER + SEA of one new token per sequence against caches).
hipError_t launch_decode_step(int B, int T, int hq, int hkv, int d, bool bf16, float scale,
                              const int32_t* idx1, const float* w1, int s2,
                              const int32_t* idx2, const float* w2, int s3, int s1,
                              const void* q, const void* k, const void* v, int32_t* idx_out,
                              float* w_out, void* o, hipStream_t st);

// Refresh edges of a dense causal attention layer (bf16 q/k, MFMA scores):
// the top-s positions per (batch, token, KV head) by group-mean probability,
// and the per-head lse (computed first unless lse_given).
bool dense_refresh_supported(int d, int G, int s);
hipError_t launch_dense_refresh(int B, int n, int hq, int hkv, int d, float scale,
                                const void* q, const void* k, int s, bool lse_given, float* lse,
                                int32_t* idx_out, float* w_out, hipStream_t st);

size_t sea_backward_workspace_bytes(long long U, int s, int G, int n);
hipError_t launch_sea_backward(int B, int n, int hq, int hkv, int d, bool bf16, float scale,
                               const void* q, const void* k, const void* v,
                               const int32_t* idx, const float* w, int s, const void* dout,
                               const float* stats, float* dq, float* dk, float* dv, float* dw,
                               void* workspace, hipStream_t st);

hipError_t launch_ser_backward(int B, int n, int hkv, const int32_t* idx1, const float* w1,
                               int s2, const int32_t* idx2, const float* w2, int s3,
                               const int32_t* idx_out, const float* w_out, int s1,
                               const float* dw_out, const uint64_t* paths, float* dw1,
                               float* dw2, double* ws1, double* ws2, hipStream_t st);

// Reverse (target-sorted) index of an edge tensor [B][n][hkv][s], s <= 4:
// beg/len per pair-major row (pair * n + j), list of edge ids; list needs
// B*n*hkv*s entries, beg and len B*n*hkv each.
bool edge_index_supported(int n, int s);
// n small enough for the single-pass index (one load pass per pair)
bool edge_index_one_pass(int n);
// The same index for n > 4096 (s <= 4, n <= 2^20) in four passes without
// per-edge global atomics: counts and offs need B*hkv * ceil(n/512) *
// ceil(n/4096) ints each (at most B*n*hkv), tot B*hkv ints, stage B*n*hkv*s
// int2 entries.  Both write, when head is not null, each row's first four
// list entries (-1 padded) to head[4 * pair-major row].
hipError_t launch_edge_index_long(int B, int n, int hkv, const int32_t* idx, const float* w,
                                  int s, const int* tgt, int* beg, int* len, int* list,
                                  int* head, int* counts, int* offs, int* tot, int2* stage,
                                  hipStream_t st);
// In both, tgt, when not null, holds the live targets per pair-major source
// row (tgt[row * s + t], -1 for a dead slot) and replaces idx and w.
hipError_t launch_edge_index(int B, int n, int hkv, const int32_t* idx, const float* w, int s,
                             const int* tgt, int* beg, int* len, int* list, int* head,
                             hipStream_t st);

// Workspace of the pull-style SER backward (reverse index of leg 1).
size_t ser_backward_pull_bytes(long long rows, int s2);
// fp64 partials of the source-chunk SER backward (s2 = s3 = 4, s1 = 4 or 2,
// n <= 4096)
bool ser_backward_part_fits(int n);
size_t ser_backward_part_bytes(int B, int n, int hkv);

hipError_t launch_check_edges(int B, int n, int hkv, const int32_t* idx, const float* w, int s,
                              unsigned long long* counts, hipStream_t st);

struct SegPlan;
// Segment plan of the XCD-aware schedule for B*hkv pairs of n tokens.
void make_seg_plan(SegPlan& sp, int B, int n, int hkv);

// Workgroups for a persistent XCD-aware kernel: as many as fit on the device
// at once (occupancy x compute units), a multiple of 8 (one share per XCD),
// and no more than the work needs (`items` units, `per_wg` per workgroup and
// pass).  Device properties and occupancy are cached per device / kernel.
int persistent_grid(const void* kernel, int items, int per_wg);

// Zero `count` 4-byte words (or doubles) with a fill kernel (graph-capture safe).
hipError_t launch_zero_f32(float* p, size_t count, hipStream_t st);
hipError_t launch_zero_f64(double* p, size_t count, hipStream_t st);

}  // namespace gm
