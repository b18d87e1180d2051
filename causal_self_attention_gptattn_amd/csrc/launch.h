// Internal host-side launchers shared by the C-ABI file and the kernel files.
// Arguments are assumed validated; each returns the status of its launches.
#pragma once

#include <hip/hip_runtime.h>

namespace gptattn {

// A [B][H][rows][D] tensor with D contiguous: element (b, h, t, d) is at
// data + b * sb + h * sh + t * st + d (strides in elements).
struct TensorArg {
  const void* data;
  long long sb, sh, st;
};

// Query i of Tq sees key j of Tk when j <= i + off and, with win > 0,
// j > i + off - win.  Plain causal attention: Tq = Tk, off = 0, win = 0.
// dropout > 0 drops attention weights with that probability; the keep mask
// is drawn from Philox4x32-10 keyed by `seed` (see attn_common.h).
struct ProblemArg {
  int B, H, Tq, Tk, D, off, win;
  float scale;
  float dropout;
  unsigned long long seed;
  unsigned int stream;
};

// bf16 storage, D in {64, 128}.  lse: [B][H][Tq] float32, contiguous.
hipError_t launch_fwd_bf16(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                           const TensorArg& o, float* lse, const ProblemArg& p,
                           hipStream_t stream);
// Backward in two launches.  delta: [B][H][Tq] floats, the row term
// sum_d dO O, written by the dq launch and read by the dk/dv launch.
hipError_t launch_bwd_dq_bf16(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                              const TensorArg& o, const TensorArg& dO, const float* lse,
                              const TensorArg& dq, float* delta, const ProblemArg& p,
                              hipStream_t stream);
hipError_t launch_bwd_dkdv_bf16(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                                const TensorArg& dO, const float* lse, const float* delta,
                                const TensorArg& dk, const TensorArg& dv, const ProblemArg& p,
                                hipStream_t stream);

// Head size 64 without dropout: the software-pipelined kernels
// (attn_d64.hip); the bf16 launchers route such problems there themselves.
hipError_t launch_bwd_dkdv_d64(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                               const TensorArg& dO, const float* lse, const float* delta,
                               const TensorArg& dk, const TensorArg& dv, const ProblemArg& p,
                               hipStream_t stream);

// Head size 128 without dropout, dense tensors, more (head, 128-key block)
// items than compute units: the persistent dK/dV kernel (attn_d128.hip).
bool dkdv_d128_applies(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                       const TensorArg& dO, const TensorArg& dk, const TensorArg& dv,
                       const ProblemArg& p, hipStream_t stream);
hipError_t launch_bwd_dkdv_d128(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                                const TensorArg& dO, const float* delta, const TensorArg& dk,
                                const TensorArg& dv, const ProblemArg& p, hipStream_t stream);

// Compute units of the device `stream` runs on (cached per device; 0 if the
// runtime cannot say).
int cu_count(hipStream_t stream);

// A [B][H][T][D] tensor laid out densely (rows of D contiguous elements,
// heads of T rows, batches of H heads).
inline bool dense_bhtd(const TensorArg& t, int H, long long T, int D) {
  return t.st == D && t.sh == T * D && t.sb == (long long)H * T * D;
}

// Short query blocks (Tq <= 4, Tk >= 64, no dropout, bf16): one workgroup per
// head streams the keys (attn_decode.hip).  launch_fwd_bf16 routes such
// problems here itself.
bool decode_applies(const ProblemArg& p);
hipError_t launch_decode_bf16(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                              const TensorArg& o, float* lse, const ProblemArg& p,
                              hipStream_t stream);

// float32 storage, D in {16, 32, 64}; same arguments.
hipError_t launch_fwd_f32(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                          const TensorArg& o, float* lse, const ProblemArg& p,
                          hipStream_t stream);
hipError_t launch_bwd_dq_f32(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                             const TensorArg& o, const TensorArg& dO, const float* lse,
                             const TensorArg& dq, float* delta, const ProblemArg& p,
                             hipStream_t stream);
hipError_t launch_bwd_dkdv_f32(const TensorArg& q, const TensorArg& k, const TensorArg& v,
                               const TensorArg& dO, const float* lse, const float* delta,
                               const TensorArg& dk, const TensorArg& dv, const ProblemArg& p,
                               hipStream_t stream);

}  // namespace gptattn
