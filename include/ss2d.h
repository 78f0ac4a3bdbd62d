/*
 * ss2d.h -- C ABI of the SS2D library (cross-scan -> selective scan S6 -> cross-merge)
 * for AMD Instinct MI355X (gfx950).
 *
 * The operations are defined on these pages:
 *   [VMamba]  "VMamba: Visual State Space Model" (Chinese translation, blog.csdn.net):
 *             section "2-D selective scan (SS2D) for visual data" and the Fig. 2 caption --
 *             SS2D unfolds the map along four routes (cross-scan), runs one S6 scan per
 *             route, and merges the results back onto the map (cross-merge).
 *   [S6]      "Vision Mamba structure and principle" (freeymw.com), section 1 (the merge
 *             adds the routes) and section 2: `selective_scan_fn`, `SelectiveScanFn`
 *             (forward/backward interface) and `selective_scan_ref` (the semantics).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  * Pointers are DEVICE pointers to dense, contiguous buffers (last index fastest),
 *    owned by the caller.  The library never allocates, frees or synchronises device
 *    memory; scratch space comes in through an explicit workspace argument whose size
 *    is given by the matching *_workspace_bytes query.
 *  * Every call enqueues its kernels on `stream` and returns; SS2D_OK means "enqueued".
 *    Device-side faults surface at the caller's next synchronisation.
 *  * Arguments are validated before anything is launched; on an error nothing is
 *    enqueued and no output is touched.
 *  * I/O tensors use `dtype` (SS2D_DTYPE_F32 or SS2D_DTYPE_BF16).  Parameters A, D,
 *    delta_bias and the gradients dA, dD, ddelta_bias are always fp32.  The scan state
 *    and all accumulation are fp32.
 *  * Sizes of 0 (empty batch, no channels, empty sequence) are valid and do nothing
 *    except write zeros to gradients that are sums over an empty set.
 *  * Apart from the scratch of ss2d_fwd_noalloc (one fixed array per GPU), the library keeps
 *    no global state; calls on different streams may run concurrently as long as their
 *    workspaces do not overlap.
 */
#ifndef SS2D_H_
#define SS2D_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SS2D_ABI_VERSION 8

/* Status codes returned by every entry point. */
enum {
  SS2D_OK = 0,
  SS2D_ERR_INVALID_ARGUMENT = 1, /* null required pointer, negative size, dim % ngroups != 0,
                                    workspace missing or too small, misaligned pointer */
  SS2D_ERR_UNSUPPORTED = 2,      /* dtype not F32/BF16, dstate outside [1, 64] */
  SS2D_ERR_HIP = 3,              /* a kernel launch reported an error */
  SS2D_ERR_TOO_LARGE = 4         /* ss2d_fwd_noalloc: the problem needs more scratch than the
                                    library holds (ss2d_fwd_noalloc_max_workspace_bytes) */
};

/* I/O element types. */
enum { SS2D_DTYPE_F32 = 0, SS2D_DTYPE_BF16 = 1 };

/* Version of this ABI (SS2D_ABI_VERSION of the build). */
int ss2d_abi_version(void);

/* Static, never-freed description of a status code. */
const char* ss2d_status_string(int status);

/* ---------------------------------------------------------------------------------
 * Cross-scan [VMamba, Fig. 2 caption]: unfold a map along the four routes.
 *   x  : (batch, channels, height, width)           dtype
 *   xs : (batch, 4, channels, L), L = height*width   dtype
 * Route k visits pixel (h, w) at step pi_k(h, w):
 *   pi_0 = h*width + w      (row-major)        pi_2 = L-1-pi_0
 *   pi_1 = w*height + h     (column-major)     pi_3 = L-1-pi_1
 * xs[b, k, c, pi_k(h, w)] = x[b, c, h, w]: a bit-exact copy.
 * ------------------------------------------------------------------------------- */
int ss2d_cross_scan(const void* x, void* xs, int64_t batch, int64_t channels, int64_t height,
                    int64_t width, int dtype, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * Cross-merge [S6 page, section 1: the four routes are added and merged back]:
 *   ys : (batch, 4, channels, L)   dtype
 *   y  : (batch, channels, height, width)  dtype
 * y[b, c, h, w] = ((ys0[pi_0] + ys1[pi_1]) + ys2[pi_2]) + ys3[pi_3], summed in fp32 in
 * that order and rounded once to dtype (round to nearest even).
 * ------------------------------------------------------------------------------- */
int ss2d_cross_merge(const void* ys, void* y, int64_t batch, int64_t channels, int64_t height,
                     int64_t width, int dtype, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * Selective scan S6 [S6 page, section 2, `selective_scan_ref`]:
 *   delta_t = softplus(delta_raw_t + delta_bias[d])   (bias/softplus optional)
 *   h_t[n]  = exp(delta_t*A[d, n]) * h_{t-1}[n] + delta_t * B[b, g, n, t] * u_t,  h_{-1} = 0
 *   y_t     = sum_n C[b, g, n, t] * h_t[n] + D[d]*u_t,  out_t = y_t * silu(z_t) (z optional)
 * with channel d reading group g = d / (dim / ngroups).
 * Layouts:  u, delta, z, out : (batch, dim, seqlen)          dtype
 *           A                : (dim, dstate)                  fp32
 *           Bm, Cm           : (batch, ngroups, dstate, seqlen) dtype
 *           Dskip, delta_bias: (dim)                           fp32, may be NULL
 *           last_state       : (batch, dim, dstate)            fp32, may be NULL
 * The workspace (optional for the forward) receives the scan state at every
 * checkpoint (before every 8th step up to 16 states, every 4th up to 32, else every 2nd)
 * so that the backward need not recompute it, and lets the forward split long sequences
 * across wavefronts when there are few rows.
 * ------------------------------------------------------------------------------- */
size_t selective_scan_workspace_bytes(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                      int64_t ngroups);

typedef struct ss_fwd_args {
  const void* u;
  const void* delta;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;      /* may be NULL */
  const void* z;           /* may be NULL */
  const float* delta_bias; /* may be NULL */
  void* out;
  float* last_state;       /* may be NULL */
  void* workspace;         /* may be NULL; else >= selective_scan_workspace_bytes(...) */
  size_t workspace_bytes;
  int64_t batch, dim, dstate, seqlen, ngroups;
  int dtype;
  int delta_softplus;
} ss_fwd_args;

int selective_scan_fwd(const ss_fwd_args* args, hipStream_t stream);

/* Backward of selective_scan_fwd [S6 page, section 2, `SelectiveScanFn.backward`]:
 * given dout = dLoss/dout, writes
 *   du, ddelta, dz : (batch, dim, seqlen)  dtype   (ddelta is w.r.t. the RAW delta,
 *                                                   before bias and softplus)
 *   dBm, dCm       : (batch, ngroups, dstate, seqlen) dtype (fp32 sums, rounded once)
 *   dA             : (dim, dstate) fp32;  dDskip, ddelta_bias : (dim) fp32
 * All outputs are overwritten, never accumulated into.  dz is written iff z != NULL,
 * dDskip iff Dskip != NULL, ddelta_bias iff delta_bias != NULL.
 * The workspace is required (>= selective_scan_workspace_bytes(...)).  If
 * workspace_has_states != 0 it must hold what selective_scan_fwd wrote into it for the
 * same inputs; otherwise the backward recomputes the states itself. */
typedef struct ss_bwd_args {
  const void* u;
  const void* delta;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;
  const void* z;
  const float* delta_bias;
  const void* dout;
  void* du;
  void* ddelta;
  float* dA;
  void* dBm;
  void* dCm;
  float* dDskip;
  void* dz;
  float* ddelta_bias;
  void* workspace;
  size_t workspace_bytes;
  int workspace_has_states;
  int64_t batch, dim, dstate, seqlen, ngroups;
  int dtype;
  int delta_softplus;
} ss_bwd_args;

int selective_scan_bwd(const ss_bwd_args* args, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * One recurrent step from a carried state, for token-by-token inference [S6 page, section 2:
 * the `Mamba` module keeps `ssm_state` -- the last_state of selective_scan_fwd -- and advances
 * it one token at a time in place; the step is one iteration of `selective_scan_ref`'s loop]:
 *   delta = softplus(delta_raw + delta_bias)          (bias/softplus optional)
 *   state[b, d, n] <- exp(delta*A[d, n]) * state[b, d, n] + delta * B[b, g, n] * x[b, d]
 *   out[b, d] = (sum_n C[b, g, n] * state[b, d, n] + D[d] * x[b, d]) * silu(z[b, d])  (z optional)
 * with channel d reading group g = d / (dim / ngroups).
 * Layouts:  state          : (batch, dim, dstate) fp32, read and overwritten (caller-owned)
 *           x, delta, z, out: (batch, dim)          dtype
 *           A              : (dim, dstate) fp32;  Bm, Cm : (batch, ngroups, dstate) dtype
 *           Dskip, delta_bias : (dim) fp32, may be NULL
 * No workspace.  Chaining steps from a zero state gives selective_scan_fwd's outputs and
 * last_state, up to rounding.
 * ------------------------------------------------------------------------------- */
typedef struct ss_step_args {
  float* state;
  const void* x;
  const void* delta;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;      /* may be NULL */
  const void* z;           /* may be NULL */
  const float* delta_bias; /* may be NULL */
  void* out;
  int64_t batch, dim, dstate, ngroups;
  int dtype;
  int delta_softplus;
} ss_step_args;

int selective_scan_step(const ss_step_args* args, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * Fused SS2D forward [VMamba, SS2D section]: equivalent, up to fp32 rounding order, to
 *   cross_merge(selective_scan_fwd(cross_scan(x), delta, A, B, C, D, delta_bias,
 *               softplus, ngroups = 4))  then  * silu(z)  per pixel (z optional)
 * The route outputs stay fp32 until they are summed; the gated sum is rounded once to dtype
 * (the composition would also round each route's output to dtype: where routes cancel, that
 * intermediate rounding alone can exceed one rounding of the result).
 * Layouts:  x, z, out  : (batch, dim, height, width)      dtype   (grid)
 *           delta      : (batch, 4, dim, L)               dtype   (route k in its own order)
 *           Bm, Cm     : (batch, 4, dstate, L)            dtype   (shared by the dim channels
 *                                                                  of route k)
 *           A          : (4, dim, dstate) fp32;  Dskip, delta_bias : (4, dim) fp32 (may be NULL)
 * The gate is applied once per pixel after the merge, which equals gating every route
 * with the cross-scanned z and merging (silu(z) is the same factor on all four).
 * The workspace is required (>= ss2d_workspace_bytes(...)); the same size serves calls with
 * and without the input front.
 * ------------------------------------------------------------------------------- */
/* Workspace of ss2d_fwd / ss2d_bwd with the Δ/B/C producer (dt_rank >= 1): the plain size plus
 * the fp32 projected inputs, their gradients and the weight-gradient partials.  0 if invalid. */
size_t ss2d_proj_workspace_bytes(int64_t batch, int64_t dim, int64_t height, int64_t width, int64_t dstate,
                                 int64_t dt_rank, int dtype);
size_t ss2d_workspace_bytes(int64_t batch, int64_t dim, int64_t height, int64_t width,
                            int64_t dstate, int dtype);

typedef struct ss2d_fwd_args {
  const void* x;
  const void* delta;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;      /* may be NULL */
  const float* delta_bias; /* may be NULL */
  const void* z;           /* may be NULL */
  void* out;
  void* workspace;
  size_t workspace_bytes;
  int64_t batch, dim, height, width, dstate;
  int dtype;
  int delta_softplus;
  int keep_states;         /* nonzero: the workspace also keeps the checkpoint states (and, with
                              a gate, the fp32 pre-gate merged map), so that ss2d_bwd can run
                              with workspace_has_states (a training forward) */
  /* Optional input front [S6 page, section 1: in the VSS block the SS2D input passes through a
   * depthwise convolution and SiLU]: with conv_w != NULL the four routes scan
   *   u = silu(pre),  pre[b,c,h,w] = conv_b[c] + sum_{i,j} conv_w[c,i,j] x[b,c,h+i-r,w+j-r]
   * (r = conv_k / 2, zero outside the map; conv_k odd, 1..7), computed once per pixel and kept
   * in fp32 in the workspace (the routes and the skip term read it without a rounding to the
   * I/O type); the skip term then uses u as well. */
  const float* conv_w;     /* (dim, conv_k, conv_k) fp32, or NULL: no front (u = x) */
  const float* conv_b;     /* (dim) fp32, may be NULL */
  int conv_k;
  /* Optional back half [S6 page, section 1: in the VSS block the SS2D features are
   * layer-normalised, then multiplied by the gate branch]: with layer_norm != 0,
   *   out = LN(M) * silu(z)  (LN(M) without z),  LN(M)[c] = (M[c] - mu) / sqrt(var + ln_eps) * ln_w[c] + ln_b[c]
   * with mu, var (biased) over the dim channels of each pixel of the merged map M (the four
   * routes' sum with its skip term), all in fp32, one rounding at the end. */
  int layer_norm;
  const float* ln_w;       /* (dim) fp32, or NULL: 1 */
  const float* ln_b;       /* (dim) fp32, or NULL: 0 */
  float ln_eps;            /* >= 0 (1e-5 is the usual LayerNorm default) */
  /* Optional Δ/B/C producer [S6 page, section 2: the Mamba module's x_proj and dt_proj, one
   * S6 block per route]: with x_proj_w != NULL, delta, Bm and Cm are not read (pass NULL), and
   * route k's inputs come from its own scanned sequence xs_k (of u: the front's output, or x):
   *   x_dbl = x_proj_w[k] @ xs_k   ((dt_rank + 2 dstate) x L), dt = rows [0, R), B = rows
   *   [R, R + N), C = rows [R + N, R + 2N), delta_raw = dt_proj_w[k] @ dt   (R = dt_rank)
   * in fp32 on the matrix cores; the route scans then run in fp32 (delta_bias is dt_proj's
   * bias).  The workspace must hold ss2d_proj_workspace_bytes(...). */
  const float* x_proj_w;   /* (4, dt_rank + 2 dstate, dim) fp32 */
  const float* dt_proj_w;  /* (4, dim, dt_rank) fp32 */
  int dt_rank;             /* 1..dim */
} ss2d_fwd_args;

int ss2d_fwd(const ss2d_fwd_args* args, hipStream_t stream);

/* Whether ss2d_fwd(args) runs as one kernel per (image, channel) plane instead of the three
 * stages below: 1 for dstate 1, 2 or 4 without the input front, the LayerNorm, the producer
 * and keep_states, when height * width is a multiple of 8, the plane's LDS arrays
 * (16 L' bytes, L' = L rounded up to 16) fit 63 KB and every I/O
 * tensor is 16-byte aligned; 0 otherwise (also for invalid or empty arguments).  The single
 * kernel reads x, delta, B, C and z once and writes only out (the workspace is unused); its
 * result equals the staged one up to the order of the scan's roundings (the single kernel
 * scans each route in parallel segments, the stages step by step).  Enqueues nothing. */
int ss2d_fwd_single_kernel(const ss2d_fwd_args* args);

/* ---------------------------------------------------------------------------------
 * Allocation-free ss2d_fwd, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same forward as
 * ss2d_fwd(args), bit for bit, with its workspace taken from a fixed scratch array that the
 * library holds on each GPU (ss2d_fwd_noalloc_max_workspace_bytes() bytes, 128 MiB, allocated
 * with the library's code object on every GPU it is loaded on and kept until the process ends).
 * `workspace` and `workspace_bytes` are ignored; the caller still passes every input and `out`.
 * Nothing is allocated or freed.  The scratch of the current device is used, so `stream` must
 * belong to the current device.
 *   * Returns SS2D_ERR_TOO_LARGE, with nothing enqueued, when the call needs more than that
 *     (ss2d_workspace_bytes(...) or ss2d_proj_workspace_bytes(...) of its shape; calls that run
 *     as one kernel per plane, see ss2d_fwd_single_kernel, need none), and
 *     SS2D_ERR_INVALID_ARGUMENT for keep_states != 0 (no backward can reach the scratch).
 *   * Every call on one GPU shares that GPU's scratch, which keeps what the last call left
 *     there (no call relies on its contents): calls that may overlap in time on one GPU (on
 *     different streams, or from different threads) race and must be serialised by the caller.
 * ------------------------------------------------------------------------------- */
size_t ss2d_fwd_noalloc_max_workspace_bytes(void);
int ss2d_fwd_noalloc(const ss2d_fwd_args* args, hipStream_t stream);

/* One stage of ss2d_fwd, for callers that time or overlap the stages separately.
 * ss2d_fwd(args) == stage 0, then 1, then 2 on the same workspace (where
 * ss2d_fwd_single_kernel(args) is 1, ss2d_fwd runs its one kernel instead, and the stages give
 * its result up to rounding):
 *   stage 0 (SS2D_STAGE_TRANSPOSE): per-plane transpose of x into the workspace (feeds the
 *                                   column-major routes);
 *   stage 1 (SS2D_STAGE_SCAN):      the four route scans, fp32 route outputs into the workspace;
 *   stage 2 (SS2D_STAGE_MERGE):     cross-merge + skip term + gate into `out`.
 * A stage reads what the earlier stages left in the workspace; any other stage value is
 * SS2D_ERR_INVALID_ARGUMENT. */
enum { SS2D_STAGE_TRANSPOSE = 0, SS2D_STAGE_SCAN = 1, SS2D_STAGE_MERGE = 2 };
int ss2d_fwd_stage(const ss2d_fwd_args* args, int stage, hipStream_t stream);

/* Backward of ss2d_fwd: given dout (batch, dim, height, width), writes
 *   dx, dz     : (batch, dim, height, width)  dtype  (dz iff z != NULL)
 *   ddelta     : (batch, 4, dim, L) dtype (w.r.t. the raw delta);
 *   dBm, dCm   : (batch, 4, dstate, L) dtype;
 *   dA         : (4, dim, dstate) fp32;  dDskip, ddelta_bias : (4, dim) fp32 (iff given)
 * Everything is overwritten.  The workspace (>= ss2d_workspace_bytes(...)) is required.  With
 * workspace_has_states == 0 the forward is recomputed inside it; otherwise it must hold what
 * ss2d_fwd with keep_states wrote for the same inputs (the transposed x, the route outputs, the
 * checkpoint states and, with a gate or the LayerNorm, the fp32 pre-gate merged map), untouched
 * since, and the forward is not run again.  ss2d_bwd itself
 * overwrites the route outputs there (with the routes' input gradients), so a second backward on
 * the same workspace must pass workspace_has_states == 0. */
typedef struct ss2d_bwd_args {
  const void* x;
  const void* delta;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;
  const float* delta_bias;
  const void* z;
  const void* dout;
  void* dx;
  void* ddelta;
  float* dA;
  void* dBm;
  void* dCm;
  float* dDskip;
  float* ddelta_bias;
  void* dz;
  void* workspace;
  size_t workspace_bytes;
  int64_t batch, dim, height, width, dstate;
  int dtype;
  int delta_softplus;
  int workspace_has_states;
  /* the input front, as in ss2d_fwd_args; with conv_w != NULL dx is the gradient w.r.t. the
   * input of the convolution, and dconv_w (dim, conv_k, conv_k) and dconv_b (dim, iff conv_b)
   * receive the filter's gradients (fp32, summed over images and pixels, overwritten) */
  const float* conv_w;
  const float* conv_b;
  int conv_k;
  float* dconv_w;
  float* dconv_b;
  /* the back half, as in ss2d_fwd_args; dln_w, dln_b (dim, fp32, overwritten) receive the
   * LayerNorm parameters' gradients (required iff ln_w, ln_b are given) */
  int layer_norm;
  const float* ln_w;
  const float* ln_b;
  float ln_eps;
  float* dln_w;
  float* dln_b;
  /* the Δ/B/C producer, as in ss2d_fwd_args: then delta, Bm, Cm are not read and ddelta,
   * dBm, dCm not written (may be NULL); dx includes the projections' path, and dx_proj_w
   * (4, dt_rank + 2 dstate, dim) and ddt_proj_w (4, dim, dt_rank) receive the weights'
   * gradients (fp32, summed over images, overwritten) */
  const float* x_proj_w;
  const float* dt_proj_w;
  int dt_rank;
  float* dx_proj_w;
  float* ddt_proj_w;
} ss2d_bwd_args;

int ss2d_bwd(const ss2d_bwd_args* args, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * Bidirectional scan of Vision Mamba [S6 page, section 2: `bimamba_inner_ref` and the
 * `Mamba` module with bimamba_type "v2"; the Vim article]: two selective scans over one
 * sequence, direction 0 in order and direction 1 over the reversed sequence, each with its own
 * parameters, the second output flipped back and added:
 *   y_k = selective_scan_fwd(u_k, delta_k, A_k, B_k, C_k, D_k, delta_bias_k)    (k = 0, 1)
 *   out[b, d, l] = (y_0[b, d, l] + y_1[b, d, L-1-l]) * silu(z[b, d, l])         (z optional)
 * The y_k stay fp32 until they are added; the gated sum is rounded once to dtype.  Gating the
 * sum equals gating each direction with z in its own order (the page's form): silu(z) is the
 * same factor for both terms.  The page's
 * first variant (shared u, delta, B, C, D, delta_bias; separate A) is the case where direction
 * 1's inputs are the flipped copies of direction 0's.
 * Layouts:  u, delta   : (batch, 2, dim, L)    dtype  (direction k in its own scan order)
 *           Bm, Cm     : (batch, 2, dstate, L) dtype  (direction k in its own scan order)
 *           A          : (2, dim, dstate) fp32;  Dskip, delta_bias : (2, dim) fp32 (may be NULL)
 *           z, out     : (batch, dim, L)       dtype  (forward order)
 * The workspace is required (>= vim_bidir_workspace_bytes(...)); sizes as for ss2d_fwd.
 * ------------------------------------------------------------------------------- */
size_t vim_bidir_workspace_bytes(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int dtype);

typedef struct vim_bidir_fwd_args {
  const void* u;
  const void* delta;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;      /* may be NULL */
  const float* delta_bias; /* may be NULL */
  const void* z;           /* may be NULL */
  void* out;
  void* workspace;
  size_t workspace_bytes;
  int64_t batch, dim, seqlen, dstate;
  int dtype;
  int delta_softplus;
  int keep_states;         /* nonzero: the workspace also keeps the direction outputs' checkpoint
                              states, so that vim_bidir_bwd can run with workspace_has_states
                              (a training forward) */
} vim_bidir_fwd_args;

int vim_bidir_fwd(const vim_bidir_fwd_args* args, hipStream_t stream);

/* One stage of vim_bidir_fwd (the same stage codes as ss2d_fwd_stage; there is no transpose):
 *   SS2D_STAGE_SCAN:  the two direction scans, outputs (dtype, each direction's order) into
 *                     the workspace;
 *   SS2D_STAGE_MERGE: flip, add and gate into `out`.
 * SS2D_STAGE_TRANSPOSE does nothing; any other value is SS2D_ERR_INVALID_ARGUMENT. */
int vim_bidir_fwd_stage(const vim_bidir_fwd_args* args, int stage, hipStream_t stream);

/* Backward of vim_bidir_fwd: given dout (batch, dim, L), writes
 *   du, ddelta : (batch, 2, dim, L) dtype (ddelta w.r.t. the raw delta);
 *   dBm, dCm   : (batch, 2, dstate, L) dtype;
 *   dA         : (2, dim, dstate) fp32;  dDskip, ddelta_bias : (2, dim) fp32 (iff given);
 *   dz         : (batch, dim, L) dtype (iff z).
 * Everything is overwritten.  The forward is recomputed inside unless workspace_has_states is
 * nonzero: then `workspace` must be the one a vim_bidir_fwd with keep_states used on the same
 * inputs (its direction outputs and states are read, and the gradients are bit for bit those of
 * the recomputing call).  The gradient reaching each direction, dout * silu(z), is kept in fp32. */
typedef struct vim_bidir_bwd_args {
  const void* u;
  const void* delta;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;
  const float* delta_bias;
  const void* z;
  const void* dout;
  void* du;
  void* ddelta;
  float* dA;
  void* dBm;
  void* dCm;
  float* dDskip;
  float* ddelta_bias;
  void* dz;
  void* workspace;
  size_t workspace_bytes;
  int64_t batch, dim, seqlen, dstate;
  int dtype;
  int delta_softplus;
  int workspace_has_states;
} vim_bidir_bwd_args;

int vim_bidir_bwd(const vim_bidir_bwd_args* args, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SS2D_H_ */
