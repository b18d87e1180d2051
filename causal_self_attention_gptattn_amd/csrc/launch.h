// Internal host-side launchers shared by the C-ABI file and the kernel files.
// Arguments are assumed validated; each returns the status of its launches.
#pragma once

#include <hip/hip_runtime.h>

namespace gptattn {

// bf16 storage, D in {64, 128}; N = B * H independent head-problems.
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int N, int T, int D, float scale, hipStream_t stream);
// Backward in two launches.  delta: N * T floats, the row term
// sum_d dO O, written by the dq launch and read by the dk/dv launch.
hipError_t launch_bwd_dq_bf16(const void* q, const void* k, const void* v, const void* o,
                              const void* dO, const float* lse, void* dq, float* delta, int N,
                              int T, int D, float scale, hipStream_t stream);
hipError_t launch_bwd_dkdv_bf16(const void* q, const void* k, const void* v, const void* dO,
                                const float* lse, const float* delta, void* dk, void* dv, int N,
                                int T, int D, float scale, hipStream_t stream);

// float32 storage, D in {16, 32, 64}.
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int N, int T, int D, float scale, hipStream_t stream);
hipError_t launch_bwd_dq_f32(const float* q, const float* k, const float* v, const float* o,
                             const float* dO, const float* lse, float* dq, float* delta, int N,
                             int T, int D, float scale, hipStream_t stream);
hipError_t launch_bwd_dkdv_f32(const float* q, const float* k, const float* v, const float* dO,
                               const float* lse, const float* delta, float* dk, float* dv, int N,
                               int T, int D, float scale, hipStream_t stream);

}  // namespace gptattn
