/*
 * gptattn -- batched multi-head causal scaled dot-product self-attention,
 * forward and backward, for AMD Instinct MI355X (gfx950).
 *
 * What is computed (lecture description "Let's build GPT: from scratch, in
 * code, spelled out", chapters "version 3: adding softmax" and "THE CRUX OF
 * THE VIDEO: version 4: self-attention", note 6 on scaled attention and the
 * corrections at 00:57:00 and 01:20:05; chapter "batched multi-headed
 * self-attention" and exercise EX1 for heads as a batch dimension):
 *
 *   for every batch element b and head h (independent problems):
 *     S[i][j]  = scale * sum_d Q[i][d] K[j][d]      for keys j <= i
 *     P[i][.]  = softmax over the visible keys j <= i (future keys get 0)
 *     O[i][d]  = sum_j P[i][j] V[j][d]
 *     lse[i]   = log(sum_{j<=i} exp(S[i][j]))       natural log
 *
 * The backward pass returns the gradients of a scalar loss L given
 * dO = dL/dO:  dV = P^T dO,  dP = dO V^T,
 *   dS[i][j] = P[i][j] (dP[i][j] - sum_k P[i][k] dP[i][k]),
 *   dQ = scale dS K,  dK = scale dS^T Q.
 *
 * Layout: every tensor is a dense row-major [B][H][T][D] array (D fastest,
 * heads as a batch dimension); lse is [B][H][T] float32.  T may be any
 * positive length.  `scale` is passed explicitly (1/sqrt(D) for standard
 * attention).
 *
 * Precision: the *_bf16 entry points (named without suffix) read and write
 * bfloat16 tensors, multiply on the matrix cores in bf16 with float32
 * accumulation, keep softmax statistics in float32, and round P and dS to
 * bf16 before the products that consume them.  The *_f32 entry points do
 * every step in float32.
 *
 * Ownership and execution: the caller owns every buffer (device memory).
 * The library allocates nothing, frees nothing, never synchronises and never
 * changes the current device (gptattn_bwd_noalloc uses a fixed array of its
 * own, see there); all work is enqueued on `stream`, a
 * hipStream_t passed as void* (NULL = the default stream), and completes
 * asynchronously.  Outputs are fully overwritten, never accumulated.  Inputs
 * are read only.  Outputs may not overlap the inputs or each other.
 *
 * Errors: every entry point returns 0 (GPTATTN_SUCCESS) or a status code.
 * Arguments are validated before any HIP call, so a call that returns
 * INVALID_VALUE, NOT_SUPPORTED, WORKSPACE or SCRATCH has enqueued nothing.
 * GPTATTN_ERROR_LAUNCH reports a failed kernel launch.  Faults inside a
 * kernel surface at the caller's next synchronisation.  Nothing aborts and
 * no C++ exception crosses this interface.
 *
 * Thread safety: stateless and reentrant (except gptattn_bwd_noalloc, whose
 * overlapping calls on one GPU race); concurrent calls on different streams
 * are safe provided their buffers do not overlap.
 */
#ifndef GPTATTN_H
#define GPTATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum gptattn_status {
  GPTATTN_SUCCESS = 0,
  /* null or misaligned pointer, B/H/T/D < 1, scale not finite or <= 0,
     overlapping output buffers, or sizes that overflow 64-bit indexing */
  GPTATTN_ERROR_INVALID_VALUE = 1,
  /* head size D outside the compiled set (bf16: 64, 128; f32: 16, 32, 64) */
  GPTATTN_ERROR_NOT_SUPPORTED = 2,
  /* backward workspace null or smaller than gptattn_bwd_workspace_bytes() */
  GPTATTN_ERROR_WORKSPACE = 3,
  /* a kernel launch failed (hipLaunchKernel returned an error) */
  GPTATTN_ERROR_LAUNCH = 4,
  /* gptattn_bwd_noalloc: B*H*T larger than GPTATTN_NOALLOC_MAX_ROWS */
  GPTATTN_ERROR_SCRATCH = 5
};

/* Required alignment, in bytes, of every tensor pointer. */
#define GPTATTN_ALIGNMENT 16

/*
 * Forward pass, bfloat16 tensors.
 *   q, k, v : [B][H][T][D] bf16, read only.
 *   o       : [B][H][T][D] bf16, written: softmax(scale Q K^T + causal) V.
 *   lse     : [B][H][T] float32, written: natural-log row normaliser of the
 *             scaled, masked scores (kept for the backward pass).
 *   D must be 64 or 128.
 */
int gptattn_fwd(const void* q, const void* k, const void* v, void* o,
                float* lse, int B, int H, int T, int D, float scale,
                void* stream);

/*
 * Backward pass, bfloat16 tensors.
 *   q, k, v, o, dO : [B][H][T][D] bf16, read only (o and lse as written by
 *                    gptattn_fwd for the same q, k, v, scale).
 *   lse            : [B][H][T] float32, read only.
 *   dq, dk, dv     : [B][H][T][D] bf16, written.
 *   workspace      : device scratch of at least
 *                    gptattn_bwd_workspace_bytes(B, H, T, D, 0) bytes; its
 *                    contents on entry are ignored and on return undefined.
 *   D must be 64 or 128.
 * The loss gradient dO is taken as given (dL/dO); the row term
 * sum_k P[i][k] dP[i][k] is formed as sum_d dO[i][d] O[i][d].
 */
int gptattn_bwd(const void* q, const void* k, const void* v, const void* o,
                const void* dO, const float* lse, void* dq, void* dk,
                void* dv, int B, int H, int T, int D, float scale,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass, bfloat16 tensors, without a workspace and without any
 * allocation: for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid it).
 * Arguments and results as for gptattn_bwd, minus the workspace.  The
 * per-query values gptattn_bwd keeps in its workspace go to a scratch array
 * the library holds in device memory: 2 * GPTATTN_NOALLOC_MAX_ROWS float32
 * (8 MiB) on every GPU it runs on, until the process ends.
 *   - B*H*T must not exceed GPTATTN_NOALLOC_MAX_ROWS, else
 *     GPTATTN_ERROR_SCRATCH (checked with the other arguments, before any
 *     HIP call).
 *   - `stream` must belong to the current device (else INVALID_VALUE); the
 *     first call on a device looks up that device's copy of the array.
 *   - Every call on one GPU uses that GPU's one copy: calls whose executions
 *     overlap on one GPU (on different streams, or from threads that do not
 *     order them) race.  The array needs no initial value.
 */
#define GPTATTN_NOALLOC_MAX_ROWS 1048576
int gptattn_bwd_noalloc(const void* q, const void* k, const void* v,
                        const void* o, const void* dO, const float* lse,
                        void* dq, void* dk, void* dv, int B, int H, int T,
                        int D, float scale, void* stream);

/*
 * The backward pass as its two launches, for callers that schedule them
 * separately (for example to overlap dK/dV with other work, or to time
 * each kernel).  gptattn_bwd == gptattn_bwd_dq followed, on the same stream,
 * by gptattn_bwd_dkdv with the same workspace.
 *
 * gptattn_bwd_dq writes dq and stores per-query values in `workspace` (two
 * [B][H][T] float32 vectors; bf16 entry points: minus the row term
 * sum_d dO O, then -lse/scale; float32 entry points: the row term).
 * gptattn_bwd_dkdv reads them from `workspace` (which must hold the values
 * gptattn_bwd_dq stored for the same inputs, on the same stream or after
 * synchronising) and writes dk, dv.  Arguments as for gptattn_bwd.
 */
int gptattn_bwd_dq(const void* q, const void* k, const void* v, const void* o,
                   const void* dO, const float* lse, void* dq, int B, int H,
                   int T, int D, float scale, void* workspace,
                   size_t workspace_bytes, void* stream);
int gptattn_bwd_dkdv(const void* q, const void* k, const void* v,
                     const void* dO, const float* lse, void* dk, void* dv,
                     int B, int H, int T, int D, float scale,
                     const void* workspace, size_t workspace_bytes,
                     void* stream);

/* Forward pass, float32 tensors; same contract, D in {16, 32, 64}. */
int gptattn_fwd_f32(const float* q, const float* k, const float* v,
                    float* o, float* lse, int B, int H, int T, int D,
                    float scale, void* stream);

/* Backward pass, float32 tensors; same contract, D in {16, 32, 64}. */
int gptattn_bwd_f32(const float* q, const float* k, const float* v,
                    const float* o, const float* dO, const float* lse,
                    float* dq, float* dk, float* dv, int B, int H, int T,
                    int D, float scale, void* workspace,
                    size_t workspace_bytes, void* stream);

/* The two backward launches, float32 tensors (see gptattn_bwd_dq). */
int gptattn_bwd_dq_f32(const float* q, const float* k, const float* v,
                       const float* o, const float* dO, const float* lse,
                       float* dq, int B, int H, int T, int D, float scale,
                       void* workspace, size_t workspace_bytes, void* stream);
int gptattn_bwd_dkdv_f32(const float* q, const float* k, const float* v,
                         const float* dO, const float* lse, float* dk,
                         float* dv, int B, int H, int T, int D, float scale,
                         const void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Bytes of device workspace gptattn_bwd / gptattn_bwd_f32 need for the given
 * shape (is_f32 selects the float32 entry point); 0 if the shape is invalid.
 * Holds two float32 vectors of B*H*T per-query values (see gptattn_bwd_dq).
 */
size_t gptattn_bwd_workspace_bytes(int B, int H, int T, int D, int is_f32);

/* ------------------------------------------------------------------------
 * Generalised calls: strided tensors, Tq != Tk, shifted and banded masks.
 *
 * Same operation as above with two generalisations:
 *
 * 1. Strided views.  Heads are a batch dimension reached by a reshape
 *    (lecture chapters "multi-headed self-attention" and "batched
 *    multi-headed self-attention", exercise EX1), so a tensor need not be a
 *    dense [B][H][T][D] array: element (b, h, t, d) is read at
 *        data + b*stride_b + h*stride_h + t*stride_t + d       (elements)
 *    with the D elements of a row contiguous.  This reads q, k and v in
 *    place from one packed projection output [B][T][3][H][D] (stride_b =
 *    T*3*H*D, stride_h = D, stride_t = 3*H*D, k and v at offsets H*D and
 *    2*H*D) and writes o straight into a [B][T][H][D] buffer.  Strides are
 *    non-negative multiples of 16 bytes; rows do not overlap (stride_t >= D
 *    when the view has more than one row; with one row stride_t is
 *    ignored); stride_t is at most 2^23 elements.
 *    An input stride may be 0 (the same keys and values for every head).
 *    Output views must not repeat an element, and outputs must not overlap
 *    each other or an input; overlap is tested on address ranges and, for
 *    interleaved views such as q/k/v of one packed buffer, on their common
 *    period.  A layout the test cannot prove disjoint is refused.
 *
 * 2. Visibility.  Query i (0 <= i < Tq) sees key j (0 <= j < Tk) when
 *        j <= i + causal_offset            (nothing from its future)
 *    and, if window > 0, also
 *        j >  i + causal_offset - window   (only the `window` most recent)
 *    causal_offset = Tk - Tq places Tq new queries after a context of
 *    Tk - Tq positions (Tq = 1: one decoding step).  window > 0 gives the
 *    locally banded causal pattern that GPT-3 alternates with dense layers
 *    (minGPT README, GPT-3 notes).  causal_offset = 0, window = 0,
 *    Tq = Tk is the plain causal case of gptattn_fwd.  A query that sees no
 *    key (possible when causal_offset < 0) gets O = 0 and lse = -inf and
 *    contributes no gradient.
 *
 * 3. Dropout.  With dropout = p > 0 the softmax weights are dropped with
 *    probability p and the kept ones scaled by the inverse of the keep
 *    probability before they weight the values (lecture chapter "scaling up the model! ... adding dropout";
 *    nanoGPT README's --dropout flag); lse stays the softmax's own
 *    normaliser.  The keep mask is not stored: every kernel redraws it from
 *    Philox4x32-10 (Salmon et al., "Parallel Random Numbers: As Easy as 1,
 *    2, 3", SC 2011).  For head-problem n = b*H + h, query i and key j the
 *    generator runs on counter (j / 4, i / 2, n, rng_stream) with key
 *    (seed & 0xffffffff, seed >> 32); the draw is the low 16 bits of output
 *    word j % 4 for even i and its high 16 bits for odd i, and the weight is
 *    kept iff draw >= thr = ceil(p * 2^16).  The keep probability realised
 *    is then (2^16 - thr) / 2^16, and kept weights are scaled by
 *    2^16 / (2^16 - thr), so the dropped-out weights are unbiased.  The
 *    same problem (seed, rng_stream, p) must be passed to the forward and
 *    backward calls.
 *
 * lse is dense: [B][H][Tq] float32; the workspace holds two such vectors.
 * ------------------------------------------------------------------------ */

enum gptattn_dtype {
  GPTATTN_DTYPE_BF16 = 0, /* bfloat16 tensors, matrix cores; D in {64, 128} */
  GPTATTN_DTYPE_F32 = 1   /* float32 tensors, all steps float32; D in {16, 32, 64} */
};

typedef struct gptattn_tensor {
  void* data;         /* device pointer to element (0, 0, 0, 0), 16-byte aligned */
  long long stride_b; /* elements between consecutive batch entries */
  long long stride_h; /* elements between consecutive heads */
  long long stride_t; /* elements between consecutive positions */
} gptattn_tensor;

typedef struct gptattn_problem {
  int B, H;          /* batch size and heads, >= 1 */
  int Tq, Tk;        /* query and key/value lengths, 1 .. 2^29 */
  int D;             /* head size */
  int causal_offset; /* -2^29 .. 2^29 */
  int window;        /* 0 (unbounded) or band width 1 .. 2^29 */
  float scale;       /* finite, > 0; 1/sqrt(D) for standard attention */
  int dtype;         /* enum gptattn_dtype */
  float dropout;     /* attention dropout probability p, 0 <= p < 1 (0: none) */
  unsigned int rng_stream;  /* dropout: fourth counter word (e.g. layer index) */
  unsigned long long seed;  /* dropout: 64-bit generator key */
} gptattn_problem;

/*
 * Forward pass over views.
 *   q : Tq rows; k, v : Tk rows; read only.
 *   o : Tq rows, written.
 *   lse : [B][H][Tq] float32, written.
 * Errors as for gptattn_fwd (dtype outside the enum, or dropout outside
 * [0, 1), is INVALID_VALUE).
 */
int gptattn_fwd_ex(const gptattn_problem* p, const gptattn_tensor* q,
                   const gptattn_tensor* k, const gptattn_tensor* v,
                   const gptattn_tensor* o, float* lse, void* stream);

/*
 * Backward pass over views (the two launches of gptattn_bwd, on `stream`).
 *   q, o, dO : Tq rows; k, v : Tk rows; lse : [B][H][Tq]; read only.
 *   dq : Tq rows; dk, dv : Tk rows; written.
 *   workspace : at least gptattn_bwd_ex_workspace_bytes(p) bytes.
 */
int gptattn_bwd_ex(const gptattn_problem* p, const gptattn_tensor* q,
                   const gptattn_tensor* k, const gptattn_tensor* v,
                   const gptattn_tensor* o, const gptattn_tensor* dO,
                   const float* lse, const gptattn_tensor* dq,
                   const gptattn_tensor* dk, const gptattn_tensor* dv,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for gptattn_bwd_ex (two B*H*Tq float32 vectors); 0 if p is
 * invalid. */
size_t gptattn_bwd_ex_workspace_bytes(const gptattn_problem* p);

/* Static, human-readable text for a status code (never NULL). */
const char* gptattn_status_string(int status);

/* Library version as major * 10000 + minor * 100 + patch. */
int gptattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GPTATTN_H */
