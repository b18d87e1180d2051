// C-ABI entry points of libgptattn: argument validation and dispatch to the
// gfx950 kernels.  See include/gptattn.h for the contract of each call.
// Validation never touches the HIP runtime, so a rejected call enqueues
// nothing and can run on a machine without a GPU.
#include <math.h>
#include <stdint.h>

#include <mutex>

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

// A launch covers at most B * H * ceil(max(Tq, Tk) / 64) workgroups of at
// most 256 work-items; the dispatch counts work-items in 32 bits.
bool grid_ok(int B, int H, int Tq, int Tk) {
  const long long t = Tq > Tk ? Tq : Tk;
  return (unsigned __int128)B * H * ((t + 63) / 64) < ((unsigned __int128)1 << 24);
}

// Element count of one [B][H][T][D] tensor and of the [B][H][T] vector; false
// if a dimension is < 1 or a byte size would not fit in 63 bits.
bool sizes(int B, int H, int T, int D, size_t elem, size_t* tensor_bytes, size_t* rows_bytes) {
  if (B < 1 || H < 1 || T < 1 || D < 1) return false;
  const unsigned __int128 rows = (unsigned __int128)B * H * T;
  const unsigned __int128 tb = rows * D * elem;
  if (tb >= ((unsigned __int128)1 << 62)) return false;
  if (rows * 4 >= ((unsigned __int128)1 << 62)) return false;
  if (!grid_ok(B, H, T, T)) return false;
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
              size_t elem, bool head_ok, bool has_ws = true) {
  size_t tb = 0, rb = 0;
  for (int i = 0; i < nin; ++i)
    if (!ins[i].p || !aligned(ins[i].p)) return GPTATTN_ERROR_INVALID_VALUE;
  for (int i = 0; i < nout; ++i)
    if (!outs[i].p || !aligned(outs[i].p)) return GPTATTN_ERROR_INVALID_VALUE;
  if (!sizes(B, H, T, D, elem, &tb, &rb)) return GPTATTN_ERROR_INVALID_VALUE;
  if (!scale_ok(scale)) return GPTATTN_ERROR_INVALID_VALUE;
  if (!head_ok) return GPTATTN_ERROR_NOT_SUPPORTED;
  // the workspace holds two [B][H][T] float vectors (see include/gptattn.h)
  const size_t wb = 2 * rb;
  if (has_ws && (!ws || !aligned(ws) || ws_bytes < wb)) return GPTATTN_ERROR_WORKSPACE;
  Range ri[8], ro[8];
  int ni = 0, no = 0;
  for (int i = 0; i < nin; ++i) ri[ni++] = rng(ins[i].p, ins[i].rows ? rb : tb);
  for (int i = 0; i < nout; ++i) ro[no++] = rng(outs[i].p, outs[i].rows ? rb : tb);
  if (!has_ws) {
  } else if (ws_is_output) {
    ro[no++] = rng(ws, wb);
  } else {
    ri[ni++] = rng(ws, wb);
  }
  if (!outputs_disjoint(ro, no, ri, ni)) return GPTATTN_ERROR_INVALID_VALUE;
  return GPTATTN_SUCCESS;
}

int launched(hipError_t e) { return e == hipSuccess ? GPTATTN_SUCCESS : GPTATTN_ERROR_LAUNCH; }

// Dense [B][H][T][D] tensor and the plain causal problem over it.
gptattn::TensorArg dense(const void* p, int H, int T, int D) {
  return gptattn::TensorArg{p, (long long)H * T * D, (long long)T * D, (long long)D};
}
gptattn::ProblemArg causal(int B, int H, int T, int D, float scale) {
  return gptattn::ProblemArg{B, H, T, T, D, 0, 0, scale, 0.0f, 0ull, 0u};
}

// ---------------------------------------------------------------------------
// Validation of the strided (*_ex) calls.
//
// Each view is summarised, in bytes, as a set of contiguous runs: dimensions
// whose stride equals the run length so far are merged into the run (D is
// always contiguous), and the rest only move the run by multiples of
// `period`, the gcd of their strides.  Two such sets are disjoint if their
// byte ranges are, or if, modulo the common period, one set's runs fit in
// the gaps of the other's (how q, k and v interleave in a packed [B][T][3C]
// projection output).  This is a sufficient test: exotic layouts that do
// not overlap may still be refused.
// ---------------------------------------------------------------------------
struct Lattice {
  uintptr_t base;
  unsigned long long span;    // bytes from base to one past the last element
  unsigned long long run;     // length of each contiguous run
  unsigned long long period;  // runs start at base + multiples of this (0: one run)
  bool injective;             // no two elements share an address
};

unsigned long long gcd(unsigned long long a, unsigned long long b) {
  while (b) {
    const unsigned long long t = a % b;
    a = b;
    b = t;
  }
  return a;
}

Lattice contiguous(const void* p, unsigned long long bytes) {
  return Lattice{reinterpret_cast<uintptr_t>(p), bytes, bytes, 0, true};
}

Lattice lattice(const gptattn_tensor& t, int B, int H, int T, int D, size_t elem) {
  struct Dim {
    unsigned long long stride, extent;
  } dims[3] = {{(unsigned long long)t.stride_b * elem, (unsigned long long)B},
               {(unsigned long long)t.stride_h * elem, (unsigned long long)H},
               {(unsigned long long)t.stride_t * elem, (unsigned long long)T}};
  Lattice L{reinterpret_cast<uintptr_t>(t.data), (unsigned long long)D * elem,
            (unsigned long long)D * elem, 0, true};
  Dim live[3];
  int n = 0;
  for (const Dim& d : dims) {
    if (d.extent < 2) continue;
    L.span += d.stride * (d.extent - 1);
    if (d.stride == 0) {
      L.injective = false;  // repeats the same rows; adds no address
      continue;
    }
    live[n++] = d;
  }
  for (int i = 1; i < n; ++i)  // sort by stride (three entries)
    for (int j = i; j > 0 && live[j].stride < live[j - 1].stride; --j) {
      const Dim x = live[j];
      live[j] = live[j - 1];
      live[j - 1] = x;
    }
  int i = 0;
  for (; i < n && live[i].stride == L.run; ++i) L.run *= live[i].extent;
  unsigned long long reach = L.run;  // bytes covered by the dimensions so far
  for (; i < n; ++i) {
    if (live[i].stride < reach) L.injective = false;
    reach += live[i].stride * (live[i].extent - 1);
    L.period = gcd(L.period, live[i].stride);
  }
  return L;
}

bool disjoint(const Lattice& a, const Lattice& b) {
  if (a.base + a.span <= b.base || b.base + b.span <= a.base) return true;
  const unsigned long long g = gcd(a.period, b.period);
  if (g == 0 || a.run > g || b.run > g) return false;
  const long long d = (long long)(b.base - a.base);
  const unsigned long long r = (unsigned long long)(((d % (long long)g) + (long long)g) % (long long)g);
  return r >= a.run && r + b.run <= g;
}

constexpr long long kMaxLen = 1LL << 29;        // Tq, Tk, |offset|, window
constexpr long long kMaxRowStride = 1LL << 23;  // elements between rows

int check_problem(const gptattn_problem* p, size_t* elem, bool* head_ok) {
  if (!p) return GPTATTN_ERROR_INVALID_VALUE;
  if (p->dtype != GPTATTN_DTYPE_BF16 && p->dtype != GPTATTN_DTYPE_F32)
    return GPTATTN_ERROR_INVALID_VALUE;
  if (p->B < 1 || p->H < 1 || p->Tq < 1 || p->Tk < 1 || p->D < 1)
    return GPTATTN_ERROR_INVALID_VALUE;
  if (p->Tq > kMaxLen || p->Tk > kMaxLen || p->causal_offset > kMaxLen ||
      p->causal_offset < -kMaxLen || p->window < 0 || p->window > kMaxLen)
    return GPTATTN_ERROR_INVALID_VALUE;
  if (!grid_ok(p->B, p->H, p->Tq, p->Tk)) return GPTATTN_ERROR_INVALID_VALUE;
  if ((unsigned __int128)p->B * p->H * p->Tq * 4 >= ((unsigned __int128)1 << 62))
    return GPTATTN_ERROR_INVALID_VALUE;
  if (!scale_ok(p->scale)) return GPTATTN_ERROR_INVALID_VALUE;
  if (!(p->dropout >= 0.0f && p->dropout < 1.0f)) return GPTATTN_ERROR_INVALID_VALUE;  // NaN too
  *elem = p->dtype == GPTATTN_DTYPE_F32 ? 4 : 2;
  *head_ok = p->dtype == GPTATTN_DTYPE_F32 ? f32_head_ok(p->D) : bf16_head_ok(p->D);
  return GPTATTN_SUCCESS;
}

// One tensor argument: present, aligned, strides non-negative multiples of
// the 16-byte vector, rows that do not overlap (stride_t >= D), row stride
// within the kernels' 32-bit tile offsets, and the whole view addressable.
bool tensor_ok(const gptattn_tensor* t, int B, int H, int T, int D, size_t elem) {
  if (!t || !t->data || !aligned(t->data)) return false;
  const long long q = GPTATTN_ALIGNMENT / (long long)elem;
  const long long s[3] = {t->stride_b, t->stride_h, t->stride_t};
  for (long long x : s)
    if (x < 0 || x % q != 0) return false;
  if (t->stride_t > kMaxRowStride || (T > 1 && t->stride_t < D)) return false;
  const unsigned __int128 span =
      ((unsigned __int128)t->stride_b * (B - 1) + (unsigned __int128)t->stride_h * (H - 1) +
       (unsigned __int128)t->stride_t * (T - 1) + D) * elem;
  return span < ((unsigned __int128)1 << 62);
}

// Outputs injective and disjoint from every input and from each other.
bool views_ok(const Lattice* outs, int nout, const Lattice* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    if (!outs[i].injective) return false;
    for (int j = 0; j < nin; ++j)
      if (!disjoint(outs[i], ins[j])) return false;
    for (int j = i + 1; j < nout; ++j)
      if (!disjoint(outs[i], outs[j])) return false;
  }
  return true;
}

// The kernels stage rows through range-checked loads that rely on
// stride_t >= D; with a single row its stride is never used, so any value
// passed for it is replaced by D.
gptattn::TensorArg targ(const gptattn_tensor* t, int rows, int D) {
  return gptattn::TensorArg{t->data, t->stride_b, t->stride_h, rows == 1 ? D : t->stride_t};
}
gptattn::ProblemArg parg(const gptattn_problem* p) {
  return gptattn::ProblemArg{p->B,    p->H,     p->Tq,      p->Tk,   p->D,
                             p->causal_offset, p->window, p->scale, p->dropout, p->seed,
                             p->rng_stream};
}

// ---------------------------------------------------------------------------
// Shared bodies.  The dense entry points describe their [B][H][T][D] buffers
// as views and the plain causal problem; the *_ex entry points pass the
// caller's views and problem through.
// ---------------------------------------------------------------------------
using gptattn::ProblemArg;
using gptattn::TensorArg;

hipError_t fwd_any(bool f32, const TensorArg& q, const TensorArg& k, const TensorArg& v,
                   const TensorArg& o, float* lse, const ProblemArg& p, hipStream_t s) {
  return f32 ? gptattn::launch_fwd_f32(q, k, v, o, lse, p, s)
             : gptattn::launch_fwd_bf16(q, k, v, o, lse, p, s);
}
hipError_t dq_any(bool f32, const TensorArg& q, const TensorArg& k, const TensorArg& v,
                  const TensorArg& o, const TensorArg& dO, const float* lse, const TensorArg& dq,
                  float* delta, const ProblemArg& p, hipStream_t s) {
  return f32 ? gptattn::launch_bwd_dq_f32(q, k, v, o, dO, lse, dq, delta, p, s)
             : gptattn::launch_bwd_dq_bf16(q, k, v, o, dO, lse, dq, delta, p, s);
}
hipError_t dkdv_any(bool f32, const TensorArg& q, const TensorArg& k, const TensorArg& v,
                    const TensorArg& dO, const float* lse, const float* delta,
                    const TensorArg& dk, const TensorArg& dv, const ProblemArg& p,
                    hipStream_t s) {
  return f32 ? gptattn::launch_bwd_dkdv_f32(q, k, v, dO, lse, delta, dk, dv, p, s)
             : gptattn::launch_bwd_dkdv_bf16(q, k, v, dO, lse, delta, dk, dv, p, s);
}

int dense_fwd(bool f32, const void* q, const void* k, const void* v, void* o, float* lse, int B,
              int H, int T, int D, float scale, void* stream) {
  const int st = check_fwd(q, k, v, o, lse, B, H, T, D, scale, f32 ? 4 : 2,
                           f32 ? f32_head_ok(D) : bf16_head_ok(D));
  if (st != GPTATTN_SUCCESS) return st;
  return launched(fwd_any(f32, dense(q, H, T, D), dense(k, H, T, D), dense(v, H, T, D),
                          dense(o, H, T, D), lse, causal(B, H, T, D, scale),
                          static_cast<hipStream_t>(stream)));
}

int dense_bwd(bool f32, const void* q, const void* k, const void* v, const void* o,
              const void* dO, const float* lse, void* dq, void* dk, void* dv, int B, int H, int T,
              int D, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  const Buf ins[6] = {{q, false}, {k, false}, {v, false}, {o, false}, {dO, false}, {lse, true}};
  const Buf outs[3] = {{dq, false}, {dk, false}, {dv, false}};
  const int st = check_bwd(ins, 6, outs, 3, workspace, workspace_bytes, true, B, H, T, D, scale,
                           f32 ? 4 : 2, f32 ? f32_head_ok(D) : bf16_head_ok(D));
  if (st != GPTATTN_SUCCESS) return st;
  float* delta = static_cast<float*>(workspace);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const ProblemArg p = causal(B, H, T, D, scale);
  if (dq_any(f32, dense(q, H, T, D), dense(k, H, T, D), dense(v, H, T, D), dense(o, H, T, D),
             dense(dO, H, T, D), lse, dense(dq, H, T, D), delta, p, s) != hipSuccess)
    return GPTATTN_ERROR_LAUNCH;
  return launched(dkdv_any(f32, dense(q, H, T, D), dense(k, H, T, D), dense(v, H, T, D),
                           dense(dO, H, T, D), lse, delta, dense(dk, H, T, D),
                           dense(dv, H, T, D), p, s));
}

int dense_bwd_dq(bool f32, const void* q, const void* k, const void* v, const void* o,
                 const void* dO, const float* lse, void* dq, int B, int H, int T, int D,
                 float scale, void* workspace, size_t workspace_bytes, void* stream) {
  const Buf ins[6] = {{q, false}, {k, false}, {v, false}, {o, false}, {dO, false}, {lse, true}};
  const Buf outs[1] = {{dq, false}};
  const int st = check_bwd(ins, 6, outs, 1, workspace, workspace_bytes, true, B, H, T, D, scale,
                           f32 ? 4 : 2, f32 ? f32_head_ok(D) : bf16_head_ok(D));
  if (st != GPTATTN_SUCCESS) return st;
  return launched(dq_any(f32, dense(q, H, T, D), dense(k, H, T, D), dense(v, H, T, D),
                         dense(o, H, T, D), dense(dO, H, T, D), lse, dense(dq, H, T, D),
                         static_cast<float*>(workspace), causal(B, H, T, D, scale),
                         static_cast<hipStream_t>(stream)));
}

int dense_bwd_dkdv(bool f32, const void* q, const void* k, const void* v, const void* dO,
                   const float* lse, void* dk, void* dv, int B, int H, int T, int D, float scale,
                   const void* workspace, size_t workspace_bytes, void* stream) {
  const Buf ins[5] = {{q, false}, {k, false}, {v, false}, {dO, false}, {lse, true}};
  const Buf outs[2] = {{dk, false}, {dv, false}};
  const int st = check_bwd(ins, 5, outs, 2, workspace, workspace_bytes, false, B, H, T, D, scale,
                           f32 ? 4 : 2, f32 ? f32_head_ok(D) : bf16_head_ok(D));
  if (st != GPTATTN_SUCCESS) return st;
  return launched(dkdv_any(f32, dense(q, H, T, D), dense(k, H, T, D), dense(v, H, T, D),
                           dense(dO, H, T, D), lse, static_cast<const float*>(workspace),
                           dense(dk, H, T, D), dense(dv, H, T, D), causal(B, H, T, D, scale),
                           static_cast<hipStream_t>(stream)));
}

}  // namespace

GPTATTN_API int gptattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int T, int D, float scale, void* stream) {
  return dense_fwd(false, q, k, v, o, lse, B, H, T, D, scale, stream);
}

GPTATTN_API int gptattn_bwd(const void* q, const void* k, const void* v, const void* o,
                            const void* dO, const float* lse, void* dq, void* dk, void* dv, int B,
                            int H, int T, int D, float scale, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return dense_bwd(false, q, k, v, o, dO, lse, dq, dk, dv, B, H, T, D, scale, workspace,
                   workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// Backward pass without a workspace argument and without allocating: the
// per-query values gptattn_bwd keeps in its workspace (two float vectors of
// B*H*T) live in `scratch`, a device array of fixed size.  Each GPU holds its
// own copy; its address is looked up once per device, with that device
// current, and kept in g_scratch (the array's name in host code is only a
// host-side stand-in, never a device address).  Calls on one GPU share that
// GPU's copy, so calls whose executions overlap on one GPU race.  Nothing in
// it needs to start at zero: the dQ launch writes every value the dK/dV
// launch reads.
// ---------------------------------------------------------------------------
namespace {
constexpr long long kNoallocRows = GPTATTN_NOALLOC_MAX_ROWS;
static __device__ __align__(256) float scratch[2 * kNoallocRows];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// This device's copy of the scratch array (nullptr on failure).
void* scratch_on(int dev) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}
}  // namespace

GPTATTN_API int gptattn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                    const void* dO, const float* lse, void* dq, void* dk,
                                    void* dv, int B, int H, int T, int D, float scale,
                                    void* stream) {
  const Buf ins[6] = {{q, false}, {k, false}, {v, false}, {o, false}, {dO, false}, {lse, true}};
  const Buf outs[3] = {{dq, false}, {dk, false}, {dv, false}};
  const int st = check_bwd(ins, 6, outs, 3, nullptr, 0, true, B, H, T, D, scale, 2,
                           bf16_head_ok(D), false);
  if (st != GPTATTN_SUCCESS) return st;
  if ((long long)B * H * T > kNoallocRows) return GPTATTN_ERROR_SCRATCH;
  // the scratch copy of the device the stream belongs to, which must be the
  // current device (the library never changes it)
  const hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = -1, sdev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return GPTATTN_ERROR_LAUNCH;
  if (s && (hipStreamGetDevice(s, &sdev) != hipSuccess || sdev != dev))
    return GPTATTN_ERROR_INVALID_VALUE;
  float* delta = static_cast<float*>(scratch_on(dev));
  if (!delta) return GPTATTN_ERROR_LAUNCH;
  const ProblemArg p = causal(B, H, T, D, scale);
  if (dq_any(false, dense(q, H, T, D), dense(k, H, T, D), dense(v, H, T, D), dense(o, H, T, D),
             dense(dO, H, T, D), lse, dense(dq, H, T, D), delta, p, s) != hipSuccess)
    return GPTATTN_ERROR_LAUNCH;
  return launched(dkdv_any(false, dense(q, H, T, D), dense(k, H, T, D), dense(v, H, T, D),
                           dense(dO, H, T, D), lse, delta, dense(dk, H, T, D),
                           dense(dv, H, T, D), p, s));
}

GPTATTN_API int gptattn_bwd_dq(const void* q, const void* k, const void* v, const void* o,
                               const void* dO, const float* lse, void* dq, int B, int H, int T,
                               int D, float scale, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return dense_bwd_dq(false, q, k, v, o, dO, lse, dq, B, H, T, D, scale, workspace,
                      workspace_bytes, stream);
}

GPTATTN_API int gptattn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                                 const float* lse, void* dk, void* dv, int B, int H, int T, int D,
                                 float scale, const void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return dense_bwd_dkdv(false, q, k, v, dO, lse, dk, dv, B, H, T, D, scale, workspace,
                        workspace_bytes, stream);
}

GPTATTN_API int gptattn_fwd_f32(const float* q, const float* k, const float* v, float* o,
                                float* lse, int B, int H, int T, int D, float scale,
                                void* stream) {
  return dense_fwd(true, q, k, v, o, lse, B, H, T, D, scale, stream);
}

GPTATTN_API int gptattn_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                                const float* dO, const float* lse, float* dq, float* dk,
                                float* dv, int B, int H, int T, int D, float scale,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return dense_bwd(true, q, k, v, o, dO, lse, dq, dk, dv, B, H, T, D, scale, workspace,
                   workspace_bytes, stream);
}

GPTATTN_API int gptattn_bwd_dq_f32(const float* q, const float* k, const float* v,
                                   const float* o, const float* dO, const float* lse, float* dq,
                                   int B, int H, int T, int D, float scale, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return dense_bwd_dq(true, q, k, v, o, dO, lse, dq, B, H, T, D, scale, workspace,
                      workspace_bytes, stream);
}

GPTATTN_API int gptattn_bwd_dkdv_f32(const float* q, const float* k, const float* v,
                                     const float* dO, const float* lse, float* dk, float* dv,
                                     int B, int H, int T, int D, float scale,
                                     const void* workspace, size_t workspace_bytes,
                                     void* stream) {
  return dense_bwd_dkdv(true, q, k, v, dO, lse, dk, dv, B, H, T, D, scale, workspace,
                        workspace_bytes, stream);
}

GPTATTN_API int gptattn_fwd_ex(const gptattn_problem* p, const gptattn_tensor* q,
                               const gptattn_tensor* k, const gptattn_tensor* v,
                               const gptattn_tensor* o, float* lse, void* stream) {
  size_t elem = 0;
  bool head_ok = false;
  int st = check_problem(p, &elem, &head_ok);
  if (st != GPTATTN_SUCCESS) return st;
  if (!tensor_ok(q, p->B, p->H, p->Tq, p->D, elem) || !tensor_ok(k, p->B, p->H, p->Tk, p->D, elem) ||
      !tensor_ok(v, p->B, p->H, p->Tk, p->D, elem) || !tensor_ok(o, p->B, p->H, p->Tq, p->D, elem) ||
      !lse || !aligned(lse))
    return GPTATTN_ERROR_INVALID_VALUE;
  if (!head_ok) return GPTATTN_ERROR_NOT_SUPPORTED;
  const Lattice ins[3] = {lattice(*q, p->B, p->H, p->Tq, p->D, elem),
                          lattice(*k, p->B, p->H, p->Tk, p->D, elem),
                          lattice(*v, p->B, p->H, p->Tk, p->D, elem)};
  const Lattice outs[2] = {lattice(*o, p->B, p->H, p->Tq, p->D, elem),
                           contiguous(lse, (unsigned long long)p->B * p->H * p->Tq * 4)};
  if (!views_ok(outs, 2, ins, 3)) return GPTATTN_ERROR_INVALID_VALUE;
  const int Tq = p->Tq, Tk = p->Tk, D = p->D;
  return launched(fwd_any(elem == 4, targ(q, Tq, D), targ(k, Tk, D), targ(v, Tk, D),
                          targ(o, Tq, D), lse, parg(p), static_cast<hipStream_t>(stream)));
}

GPTATTN_API int gptattn_bwd_ex(const gptattn_problem* p, const gptattn_tensor* q,
                               const gptattn_tensor* k, const gptattn_tensor* v,
                               const gptattn_tensor* o, const gptattn_tensor* dO,
                               const float* lse, const gptattn_tensor* dq,
                               const gptattn_tensor* dk, const gptattn_tensor* dv,
                               void* workspace, size_t workspace_bytes, void* stream) {
  size_t elem = 0;
  bool head_ok = false;
  int st = check_problem(p, &elem, &head_ok);
  if (st != GPTATTN_SUCCESS) return st;
  const int B = p->B, H = p->H, Tq = p->Tq, Tk = p->Tk, D = p->D;
  if (!tensor_ok(q, B, H, Tq, D, elem) || !tensor_ok(k, B, H, Tk, D, elem) ||
      !tensor_ok(v, B, H, Tk, D, elem) || !tensor_ok(o, B, H, Tq, D, elem) ||
      !tensor_ok(dO, B, H, Tq, D, elem) || !tensor_ok(dq, B, H, Tq, D, elem) ||
      !tensor_ok(dk, B, H, Tk, D, elem) || !tensor_ok(dv, B, H, Tk, D, elem) || !lse ||
      !aligned(lse))
    return GPTATTN_ERROR_INVALID_VALUE;
  if (!head_ok) return GPTATTN_ERROR_NOT_SUPPORTED;
  const unsigned long long rb = (unsigned long long)B * H * Tq * 4;
  const Lattice ins[6] = {lattice(*q, B, H, Tq, D, elem), lattice(*k, B, H, Tk, D, elem),
                          lattice(*v, B, H, Tk, D, elem), lattice(*o, B, H, Tq, D, elem),
                          lattice(*dO, B, H, Tq, D, elem), contiguous(lse, rb)};
  const Lattice outs[4] = {lattice(*dq, B, H, Tq, D, elem), lattice(*dk, B, H, Tk, D, elem),
                           lattice(*dv, B, H, Tk, D, elem), contiguous(workspace, 2 * rb)};
  if (!views_ok(outs, 4, ins, 6)) return GPTATTN_ERROR_INVALID_VALUE;
  if (!workspace || !aligned(workspace) || workspace_bytes < 2 * rb)
    return GPTATTN_ERROR_WORKSPACE;
  const bool f32 = elem == 4;
  float* delta = static_cast<float*>(workspace);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const ProblemArg pa = parg(p);
  const TensorArg tq = targ(q, Tq, D), tk = targ(k, Tk, D), tv = targ(v, Tk, D);
  const TensorArg tdo = targ(dO, Tq, D);
  if (dq_any(f32, tq, tk, tv, targ(o, Tq, D), tdo, lse, targ(dq, Tq, D), delta, pa, s) !=
      hipSuccess)
    return GPTATTN_ERROR_LAUNCH;
  return launched(
      dkdv_any(f32, tq, tk, tv, tdo, lse, delta, targ(dk, Tk, D), targ(dv, Tk, D), pa, s));
}

GPTATTN_API size_t gptattn_bwd_ex_workspace_bytes(const gptattn_problem* p) {
  size_t elem = 0;
  bool head_ok = false;
  if (check_problem(p, &elem, &head_ok) != GPTATTN_SUCCESS) return 0;
  return (size_t)p->B * p->H * p->Tq * 8;
}

GPTATTN_API size_t gptattn_bwd_workspace_bytes(int B, int H, int T, int D, int is_f32) {
  size_t tb = 0, rb = 0;
  if (!sizes(B, H, T, D, is_f32 ? 4 : 2, &tb, &rb)) return 0;
  return 2 * rb;
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
    case GPTATTN_ERROR_SCRATCH:
      return "GPTATTN_ERROR_SCRATCH: B*H*T exceeds GPTATTN_NOALLOC_MAX_ROWS, the size of "
             "gptattn_bwd_noalloc's scratch array";
    default: return "GPTATTN: unknown status code";
  }
}

GPTATTN_API int gptattn_version(void) { return kVersion; }
