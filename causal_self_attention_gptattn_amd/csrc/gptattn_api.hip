// C-ABI entry points of libgptattn: argument validation and dispatch to the
// gfx950 kernels.  See include/gptattn.h for the contract of each call.
// Validation never touches the HIP runtime, so a rejected call enqueues
// nothing and can run on a machine without a GPU.
#include <math.h>
#include <stdint.h>

#include "gptattn.h"
#include "launch.h"

#define GPTATTN_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kVersion = 10000;  // 1.0.0

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) % GPTATTN_ALIGNMENT) == 0; }

// Element count of one [B][H][T][D] tensor and of the [B][H][T] vector; false
// if a dimension is < 1 or a byte size would not fit in 63 bits.
bool sizes(int B, int H, int T, int D, size_t elem, size_t* tensor_bytes, size_t* rows_bytes) {
  if (B < 1 || H < 1 || T < 1 || D < 1) return false;
  const unsigned __int128 rows = (unsigned __int128)B * H * T;
  const unsigned __int128 tb = rows * D * elem;
  if (tb >= ((unsigned __int128)1 << 62)) return false;
  if (rows * 4 >= ((unsigned __int128)1 << 62)) return false;
  // kernels index workgroups with 32-bit ints
  if ((unsigned __int128)B * H * ((T + 63) / 64) >= ((unsigned __int128)1 << 31)) return false;
  *tensor_bytes = (size_t)tb;
  *rows_bytes = (size_t)(rows * 4);
  return true;
}

Range rng(const void* p, size_t n) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + n};
}

bool scale_ok(float s) { return isfinite(s) && s > 0.0f; }

bool bf16_head_ok(int D) { return D == 64 || D == 128; }
bool f32_head_ok(int D) { return D == 16 || D == 32 || D == 64; }

// Outputs must not overlap inputs or each other.  Inputs may alias inputs.
bool outputs_disjoint(const Range* outs, int nout, const Range* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlaps(outs[i], ins[j])) return false;
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(outs[i], outs[j])) return false;
  }
  return true;
}

int check_fwd(const void* q, const void* k, const void* v, const void* o, const float* lse, int B,
              int H, int T, int D, float scale, size_t elem, bool head_ok) {
  size_t tb = 0, rb = 0;
  if (!q || !k || !v || !o || !lse) return GPTATTN_ERROR_INVALID_VALUE;
  if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(o) || !aligned(lse))
    return GPTATTN_ERROR_INVALID_VALUE;
  if (!sizes(B, H, T, D, elem, &tb, &rb)) return GPTATTN_ERROR_INVALID_VALUE;
  if (!scale_ok(scale)) return GPTATTN_ERROR_INVALID_VALUE;
  if (!head_ok) return GPTATTN_ERROR_NOT_SUPPORTED;
  const Range outs[2] = {rng(o, tb), rng(lse, rb)};
  const Range ins[3] = {rng(q, tb), rng(k, tb), rng(v, tb)};
  if (!outputs_disjoint(outs, 2, ins, 3)) return GPTATTN_ERROR_INVALID_VALUE;
  return GPTATTN_SUCCESS;
}

// Generic check for the backward calls: every listed pointer non-null and
// aligned, sizes and scale valid, head size compiled, workspace present and
// large enough, and outputs disjoint from inputs and from each other.
// Tensor pointers cover tb bytes; the lse / workspace ranges cover rb bytes.
struct Buf {
  const void* p;
  bool rows;  // [B][H][T] float32 (lse, workspace) rather than a full tensor
};

int check_bwd(const Buf* ins, int nin, const Buf* outs, int nout, const void* ws,
              size_t ws_bytes, bool ws_is_output, int B, int H, int T, int D, float scale,
              size_t elem, bool head_ok) {
  size_t tb = 0, rb = 0;
  for (int i = 0; i < nin; ++i)
    if (!ins[i].p || !aligned(ins[i].p)) return GPTATTN_ERROR_INVALID_VALUE;
  for (int i = 0; i < nout; ++i)
    if (!outs[i].p || !aligned(outs[i].p)) return GPTATTN_ERROR_INVALID_VALUE;
  if (!sizes(B, H, T, D, elem, &tb, &rb)) return GPTATTN_ERROR_INVALID_VALUE;
  if (!scale_ok(scale)) return GPTATTN_ERROR_INVALID_VALUE;
  if (!head_ok) return GPTATTN_ERROR_NOT_SUPPORTED;
  if (!ws || !aligned(ws) || ws_bytes < rb) return GPTATTN_ERROR_WORKSPACE;
  Range ri[8], ro[8];
  int ni = 0, no = 0;
  for (int i = 0; i < nin; ++i) ri[ni++] = rng(ins[i].p, ins[i].rows ? rb : tb);
  for (int i = 0; i < nout; ++i) ro[no++] = rng(outs[i].p, outs[i].rows ? rb : tb);
  if (ws_is_output) {
    ro[no++] = rng(ws, rb);
  } else {
    ri[ni++] = rng(ws, rb);
  }
  if (!outputs_disjoint(ro, no, ri, ni)) return GPTATTN_ERROR_INVALID_VALUE;
  return GPTATTN_SUCCESS;
}

int launched(hipError_t e) { return e == hipSuccess ? GPTATTN_SUCCESS : GPTATTN_ERROR_LAUNCH; }

}  // namespace

GPTATTN_API int gptattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int T, int D, float scale, void* stream) {
  const int st = check_fwd(q, k, v, o, lse, B, H, T, D, scale, 2, bf16_head_ok(D));
  if (st != GPTATTN_SUCCESS) return st;
  return launched(gptattn::launch_fwd_bf16(q, k, v, o, lse, B * H, T, D, scale,
                                           static_cast<hipStream_t>(stream)));
}

GPTATTN_API int gptattn_bwd(const void* q, const void* k, const void* v, const void* o,
                            const void* dO, const float* lse, void* dq, void* dk, void* dv, int B,
                            int H, int T, int D, float scale, void* workspace,
                            size_t workspace_bytes, void* stream) {
  const Buf ins[6] = {{q, false}, {k, false}, {v, false}, {o, false}, {dO, false}, {lse, true}};
  const Buf outs[3] = {{dq, false}, {dk, false}, {dv, false}};
  const int st = check_bwd(ins, 6, outs, 3, workspace, workspace_bytes, true, B, H, T, D, scale,
                           2, bf16_head_ok(D));
  if (st != GPTATTN_SUCCESS) return st;
  float* delta = static_cast<float*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e =
      gptattn::launch_bwd_dq_bf16(q, k, v, o, dO, lse, dq, delta, B * H, T, D, scale, s);
  if (e != hipSuccess) return GPTATTN_ERROR_LAUNCH;
  return launched(
      gptattn::launch_bwd_dkdv_bf16(q, k, v, dO, lse, delta, dk, dv, B * H, T, D, scale, s));
}

GPTATTN_API int gptattn_bwd_dq(const void* q, const void* k, const void* v, const void* o,
                               const void* dO, const float* lse, void* dq, int B, int H, int T,
                               int D, float scale, void* workspace, size_t workspace_bytes,
                               void* stream) {
  const Buf ins[6] = {{q, false}, {k, false}, {v, false}, {o, false}, {dO, false}, {lse, true}};
  const Buf outs[1] = {{dq, false}};
  const int st = check_bwd(ins, 6, outs, 1, workspace, workspace_bytes, true, B, H, T, D, scale,
                           2, bf16_head_ok(D));
  if (st != GPTATTN_SUCCESS) return st;
  return launched(gptattn::launch_bwd_dq_bf16(q, k, v, o, dO, lse, dq,
                                              static_cast<float*>(workspace), B * H, T, D, scale,
                                              static_cast<hipStream_t>(stream)));
}

GPTATTN_API int gptattn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                                 const float* lse, void* dk, void* dv, int B, int H, int T, int D,
                                 float scale, const void* workspace, size_t workspace_bytes,
                                 void* stream) {
  const Buf ins[5] = {{q, false}, {k, false}, {v, false}, {dO, false}, {lse, true}};
  const Buf outs[2] = {{dk, false}, {dv, false}};
  const int st = check_bwd(ins, 5, outs, 2, workspace, workspace_bytes, false, B, H, T, D, scale,
                           2, bf16_head_ok(D));
  if (st != GPTATTN_SUCCESS) return st;
  return launched(gptattn::launch_bwd_dkdv_bf16(q, k, v, dO, lse,
                                                static_cast<const float*>(workspace), dk, dv,
                                                B * H, T, D, scale,
                                                static_cast<hipStream_t>(stream)));
}

GPTATTN_API int gptattn_fwd_f32(const float* q, const float* k, const float* v, float* o,
                                float* lse, int B, int H, int T, int D, float scale,
                                void* stream) {
  const int st = check_fwd(q, k, v, o, lse, B, H, T, D, scale, 4, f32_head_ok(D));
  if (st != GPTATTN_SUCCESS) return st;
  return launched(gptattn::launch_fwd_f32(q, k, v, o, lse, B * H, T, D, scale,
                                          static_cast<hipStream_t>(stream)));
}

GPTATTN_API int gptattn_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                                const float* dO, const float* lse, float* dq, float* dk,
                                float* dv, int B, int H, int T, int D, float scale,
                                void* workspace, size_t workspace_bytes, void* stream) {
  const Buf ins[6] = {{q, false}, {k, false}, {v, false}, {o, false}, {dO, false}, {lse, true}};
  const Buf outs[3] = {{dq, false}, {dk, false}, {dv, false}};
  const int st = check_bwd(ins, 6, outs, 3, workspace, workspace_bytes, true, B, H, T, D, scale,
                           4, f32_head_ok(D));
  if (st != GPTATTN_SUCCESS) return st;
  float* delta = static_cast<float*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e =
      gptattn::launch_bwd_dq_f32(q, k, v, o, dO, lse, dq, delta, B * H, T, D, scale, s);
  if (e != hipSuccess) return GPTATTN_ERROR_LAUNCH;
  return launched(
      gptattn::launch_bwd_dkdv_f32(q, k, v, dO, lse, delta, dk, dv, B * H, T, D, scale, s));
}

GPTATTN_API int gptattn_bwd_dq_f32(const float* q, const float* k, const float* v,
                                   const float* o, const float* dO, const float* lse, float* dq,
                                   int B, int H, int T, int D, float scale, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  const Buf ins[6] = {{q, false}, {k, false}, {v, false}, {o, false}, {dO, false}, {lse, true}};
  const Buf outs[1] = {{dq, false}};
  const int st = check_bwd(ins, 6, outs, 1, workspace, workspace_bytes, true, B, H, T, D, scale,
                           4, f32_head_ok(D));
  if (st != GPTATTN_SUCCESS) return st;
  return launched(gptattn::launch_bwd_dq_f32(q, k, v, o, dO, lse, dq,
                                             static_cast<float*>(workspace), B * H, T, D, scale,
                                             static_cast<hipStream_t>(stream)));
}

GPTATTN_API int gptattn_bwd_dkdv_f32(const float* q, const float* k, const float* v,
                                     const float* dO, const float* lse, float* dk, float* dv,
                                     int B, int H, int T, int D, float scale,
                                     const void* workspace, size_t workspace_bytes,
                                     void* stream) {
  const Buf ins[5] = {{q, false}, {k, false}, {v, false}, {dO, false}, {lse, true}};
  const Buf outs[2] = {{dk, false}, {dv, false}};
  const int st = check_bwd(ins, 5, outs, 2, workspace, workspace_bytes, false, B, H, T, D, scale,
                           4, f32_head_ok(D));
  if (st != GPTATTN_SUCCESS) return st;
  return launched(gptattn::launch_bwd_dkdv_f32(q, k, v, dO, lse,
                                               static_cast<const float*>(workspace), dk, dv,
                                               B * H, T, D, scale,
                                               static_cast<hipStream_t>(stream)));
}

GPTATTN_API size_t gptattn_bwd_workspace_bytes(int B, int H, int T, int D, int is_f32) {
  size_t tb = 0, rb = 0;
  if (!sizes(B, H, T, D, is_f32 ? 4 : 2, &tb, &rb)) return 0;
  return rb;
}

GPTATTN_API const char* gptattn_status_string(int status) {
  switch (status) {
    case GPTATTN_SUCCESS: return "GPTATTN_SUCCESS: no error";
    case GPTATTN_ERROR_INVALID_VALUE:
      return "GPTATTN_ERROR_INVALID_VALUE: null or misaligned pointer, non-positive size, "
             "scale not finite and positive, or overlapping output buffers";
    case GPTATTN_ERROR_NOT_SUPPORTED:
      return "GPTATTN_ERROR_NOT_SUPPORTED: head size not compiled (bf16: 64, 128; f32: 16, 32, 64)";
    case GPTATTN_ERROR_WORKSPACE:
      return "GPTATTN_ERROR_WORKSPACE: workspace missing, misaligned or too small";
    case GPTATTN_ERROR_LAUNCH: return "GPTATTN_ERROR_LAUNCH: kernel launch failed";
    default: return "GPTATTN: unknown status code";
  }
}

GPTATTN_API int gptattn_version(void) { return kVersion; }
