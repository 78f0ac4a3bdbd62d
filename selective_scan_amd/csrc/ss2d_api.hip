// C ABI entry points (declared in include/ss2d.h): argument validation, workspace layout and
// kernel dispatch.  Nothing here allocates, frees or synchronises.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/ss2d.h"
#include "device_common.h"
#include "internal.h"
#include "plane_fwd.h"

using namespace ss2d;

namespace {

constexpr int64_t kAlign = 256;
inline int64_t align_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int esize(int dtype) { return dtype == SS2D_DTYPE_F32 ? 4 : 2; }
inline bool aligned(const void* p, int64_t a) { return (reinterpret_cast<uintptr_t>(p) % uintptr_t(a)) == 0; }

int status_from(hipError_t e) { return e == hipSuccess ? SS2D_OK : SS2D_ERR_HIP; }

bool dtype_ok(int dtype) { return dtype == SS2D_DTYPE_F32 || dtype == SS2D_DTYPE_BF16; }

// Limit on grid sizes: one-dimensional grids of at most 2^31 - 1 workgroups.
constexpr int64_t kMaxBlocks = (int64_t(1) << 31) - 1;

// ---- selective-scan workspace layout -------------------------------------------------
// Split long sequences across wavefronts only when the rows alone cannot fill the GPU.  The
// forward and the backward plan separately: each targets a whole number of "rounds" of its
// kernel (1024 SIMDs x the wavefronts per SIMD its registers allow), so the last round is not
// a short tail.  Chunks are whole tiles.
constexpr int64_t kSimds = 1024;  // 256 CUs x 4 SIMDs on MI355X

// channels per wavefront (two lanes per channel from 16 states up, in both directions) and
// wavefronts per SIMD the kernels' registers allow, by padded state count
inline int64_t rows_per_wave(int64_t dstate) { return padded_states(dstate) >= 16 ? kWave / 2 : kWave; }

void plan_chunks(int64_t row_waves, int64_t L, int64_t waves_per_simd, bool can_chunk, int64_t* chunk_len,
                 int* n_chunks) {
  const int64_t n_tiles = cdiv(L, kTile);
  const int64_t round = kSimds * waves_per_simd;
  if (!can_chunk || row_waves * 2 >= round || n_tiles <= 1) {
    *chunk_len = (n_tiles > 0 ? n_tiles : 1) * kTile;
    *n_chunks = 1;
    return;
  }
  // the most chunks that still fit in one round (at least two chunks)
  int64_t want = round / row_waves;
  if (want < 2) want = 2;
  if (want > n_tiles) want = n_tiles;
  const int64_t tiles_per_chunk = cdiv(n_tiles, want);
  *chunk_len = tiles_per_chunk * kTile;
  *n_chunks = int(cdiv(L, *chunk_len));
}

struct ScanLayout {
  int64_t rows, n_ckpt, dblocks, per_group;
  int64_t chunk_len, bwd_chunk_len;  // forward / backward chunk plans
  int n_chunks, bwd_n_chunks, ckpt_every;
  int64_t off_ckpt, off_sum, off_lam, off_dB, off_dC, off_dA, off_dD, off_dbias, total;
};

// Wavefronts per SIMD whose whole rounds the forward chunk plan fills.  Below 16 states a
// chunk's first pass costs nearly as much as its output pass, so the plan stops at two.
inline int64_t fwd_plan_waves(int ns, bool bf16) { return ns >= 16 ? fwd_waves_per_simd(ns, bf16) : 2; }

// The chunk plans depend on the element type (through the kernels' occupancy) but the
// workspace size does not: the per-chunk buffers are sized for the larger plan of the two.
ScanLayout scan_layout(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int64_t ngroups, int dtype) {
  ScanLayout l{};
  l.rows = batch * dim;
  l.ckpt_every = ckpt_steps(padded_states(dstate));
  l.n_ckpt = cdiv(seqlen, l.ckpt_every);
  l.per_group = ngroups > 0 ? dim / ngroups : 0;
  l.dblocks = cdiv(l.per_group, rows_per_wave(dstate));  // channel blocks of one wavefront (dB/dC partials)
  const int64_t row_waves = batch * ngroups * l.dblocks;
  const int ns = padded_states(dstate);
  const bool bf16 = dtype == SS2D_DTYPE_BF16;
  plan_chunks(row_waves, seqlen, fwd_plan_waves(ns, bf16), true, &l.chunk_len, &l.n_chunks);
  plan_chunks(row_waves, seqlen, bwd_waves_per_simd(ns), true, &l.bwd_chunk_len, &l.bwd_n_chunks);
  int64_t other_len;
  int other_n;
  plan_chunks(row_waves, seqlen, fwd_plan_waves(ns, !bf16), true, &other_len, &other_n);
  int64_t nc = l.n_chunks > l.bwd_n_chunks ? l.n_chunks : l.bwd_n_chunks;
  if (other_n > nc) nc = other_n;
  int64_t o = 0;
  l.off_ckpt = o;  o += align_up(l.rows * l.n_ckpt * dstate * 4);
  l.off_sum = o;   o += align_up(l.rows * nc * 4);
  l.off_lam = o;   o += align_up(l.rows * nc * dstate * 4);
  l.off_dB = o;    o += align_up(l.dblocks * batch * ngroups * dstate * seqlen * 4);
  l.off_dC = o;    o += align_up(l.dblocks * batch * ngroups * dstate * seqlen * 4);
  l.off_dA = o;    o += align_up(nc * l.rows * dstate * 4);
  l.off_dD = o;    o += align_up(nc * l.rows * 4);
  l.off_dbias = o; o += align_up(nc * l.rows * 4);
  l.total = o;
  return l;
}

// Up to rank 16 the dt_proj product is formed inside the route scans (the raw delta never goes
// through memory); larger ranks materialise delta with a separate product.
static bool fused_dt(int64_t dt_rank) { return dt_rank >= 1 && dt_rank <= 16; }

// ---- SS2D workspace layout -----------------------------------------------------------
struct SS2DLayout {
  int64_t off_xT, off_ys, off_scan, off_merged, off_dM, off_dMT, off_xc, off_cpart, off_lnpart, total;
  // the Δ/B/C producer (dt_rank > 0): fp32 projected inputs, their gradients, weight partials
  // x_dbl and its gradient are (batch, 4, R + 2N, L): rows [0, R) dt, [R, R + N) B, [R + N, R + 2N) C
  int64_t off_pxdbl, off_pdelta, off_pddelta, off_pdxdbl, off_pwx, off_pwdt;
  int64_t proj_splits;  // slices of the weight-gradient products (partials summed afterwards)
  ScanLayout scan;    // chunk plan for the I/O type
  ScanLayout scan32;  // chunk plan of the fp32 scans of the projected path (same offsets)
};

SS2DLayout ss2d_layout(int64_t batch, int64_t dim, int64_t H, int64_t W, int64_t dstate, int dtype,
                       int64_t dt_rank = 0) {
  SS2DLayout l{};
  const int64_t L = H * W;
  int64_t o = 0;
  l.off_xT = o;     o += align_up(batch * dim * L * 4);  // the map's transpose (dtype, or fp32 from the front)
  l.off_ys = o;     o += align_up(batch * 4 * dim * L * 4);  // fp32 route outputs; fp32 du in the backward
  l.scan = scan_layout(batch, 4 * dim, dstate, L, 4, dtype);
  l.off_scan = o;   o += l.scan.total;
  l.off_merged = o; o += align_up(batch * dim * L * 4);
  l.off_dM = o;     o += align_up(batch * dim * L * 4);
  l.off_dMT = o;    o += align_up(batch * dim * L * 4);
  l.off_xc = o;     o += align_up(batch * dim * L * 4);                            // input front output (fp32)
  l.off_cpart = o;  o += align_up(batch * dim * front_tiles(H, W) * (kFrontMaxK * kFrontMaxK + 1) * 4);
  l.off_lnpart = o; o += align_up(ln_part_rows(batch, L) * 2 * dim * 4);  // LayerNorm parameter partials
  l.scan32 = scan_layout(batch, 4 * dim, dstate, L, 4, SS2D_DTYPE_F32);
  if (dt_rank > 0) {
    const int64_t R = dt_rank, N = dstate, Cp = R + 2 * N, S = wgrad_splits(batch, L);
    l.proj_splits = S;
    l.off_pxdbl = o;   o += align_up(batch * 4 * Cp * L * 4);
    l.off_pdelta = o;  o += fused_dt(R) ? 0 : align_up(batch * 4 * dim * L * 4);
    l.off_pddelta = o; o += align_up(batch * 4 * dim * L * 4);
    l.off_pdxdbl = o;  o += align_up(batch * 4 * Cp * L * 4);
    l.off_pwx = o;     o += align_up(S * 4 * Cp * dim * 4);
    l.off_pwdt = o;    o += align_up(S * 4 * dim * R * 4);
  }
  l.total = o;
  return l;
}

inline char* at(void* base, int64_t off) { return static_cast<char*>(base) + off; }

// Common checks of the selective-scan shapes.
int check_scan_shapes(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int64_t ngroups, int dtype) {
  if (!dtype_ok(dtype)) return SS2D_ERR_UNSUPPORTED;
  if (batch < 0 || dim < 0 || seqlen < 0) return SS2D_ERR_INVALID_ARGUMENT;
  if (dstate < 1 || dstate > 64) return SS2D_ERR_UNSUPPORTED;
  if (ngroups < 1 || (dim % ngroups) != 0) return SS2D_ERR_INVALID_ARGUMENT;
  return SS2D_OK;
}

bool elem_aligned(int dtype, std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p && !aligned(p, esize(dtype))) return false;
  return true;
}
bool vec_aligned(int dtype, std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p && !aligned(p, 4 * esize(dtype))) return false;
  return true;
}

}  // namespace

extern "C" {

int ss2d_abi_version(void) { return SS2D_ABI_VERSION; }

const char* ss2d_status_string(int status) {
  switch (status) {
    case SS2D_OK: return "ok";
    case SS2D_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SS2D_ERR_UNSUPPORTED: return "unsupported dtype or state size";
    case SS2D_ERR_HIP: return "HIP launch error";
    case SS2D_ERR_TOO_LARGE: return "problem too large for the allocation-free scratch";
    default: return "unknown status";
  }
}

int ss2d_cross_scan(const void* x, void* xs, int64_t batch, int64_t channels, int64_t height, int64_t width,
                    int dtype, hipStream_t stream) {
  if (!dtype_ok(dtype)) return SS2D_ERR_UNSUPPORTED;
  if (batch < 0 || channels < 0 || height < 0 || width < 0) return SS2D_ERR_INVALID_ARGUMENT;
  const int64_t L = height * width;
  if (batch * channels * L == 0) return SS2D_OK;
  if (!x || !xs || !elem_aligned(dtype, {x, xs})) return SS2D_ERR_INVALID_ARGUMENT;
  if (height > (1 << 30) || width > (1 << 30) || batch * channels * cdiv(height, 32) * cdiv(width, 32) > kMaxBlocks)
    return SS2D_ERR_INVALID_ARGUMENT;
  const int e = esize(dtype);
  ScanOutputs o;
  for (int k = 0; k < 4; ++k) o.out[k] = at(xs, int64_t(k) * channels * L * e);
  o.batch_stride = 4 * channels * L;
  return status_from(launch_route_scatter(x, o, batch, channels, height, width, e, stream));
}

int ss2d_cross_merge(const void* ys, void* y, int64_t batch, int64_t channels, int64_t height, int64_t width,
                     int dtype, hipStream_t stream) {
  if (!dtype_ok(dtype)) return SS2D_ERR_UNSUPPORTED;
  if (batch < 0 || channels < 0 || height < 0 || width < 0) return SS2D_ERR_INVALID_ARGUMENT;
  if (batch * channels * height * width == 0) return SS2D_OK;
  if (!ys || !y || !elem_aligned(dtype, {ys, y})) return SS2D_ERR_INVALID_ARGUMENT;
  if (height > (1 << 30) || width > (1 << 30) || batch * channels * cdiv(height, 32) * cdiv(width, 32) > kMaxBlocks)
    return SS2D_ERR_INVALID_ARGUMENT;
  MergeArgs a{};
  a.routes = ys;
  a.routes_f32 = dtype == SS2D_DTYPE_F32;
  a.y = y;
  a.batch = batch;
  a.C = channels;
  a.H = height;
  a.W = width;
  a.dtype = dtype;
  return status_from(launch_merge(a, stream));
}

size_t selective_scan_workspace_bytes(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                      int64_t ngroups) {
  if (batch < 0 || dim < 0 || dstate < 1 || seqlen < 0 || ngroups < 1) return 0;
  return size_t(scan_layout(batch, dim, dstate, seqlen, ngroups, SS2D_DTYPE_BF16).total);
}

// The generic forward; with a workspace the sequence may be chunked, and with keep_states the
// state before every ckpt_every-th step is kept there for the backward.
static int scan_fwd_impl(const ss_fwd_args* a, bool keep_states, hipStream_t stream, bool out_f32 = false) {
  if (!a) return SS2D_ERR_INVALID_ARGUMENT;
  int st = check_scan_shapes(a->batch, a->dim, a->dstate, a->seqlen, a->ngroups, a->dtype);
  if (st != SS2D_OK) return st;
  const int64_t rows = a->batch * a->dim;
  if (rows == 0 || a->seqlen == 0) {
    if (rows > 0 && a->last_state)
      return status_from(launch_fill_zero(a->last_state, rows * a->dstate, stream));
    return SS2D_OK;
  }
  if (!a->u || !a->delta || !a->A || !a->Bm || !a->Cm || !a->out) return SS2D_ERR_INVALID_ARGUMENT;
  if (!elem_aligned(a->dtype, {a->u, a->delta, a->Bm, a->Cm, a->z, a->out})) return SS2D_ERR_INVALID_ARGUMENT;
  if (!aligned(a->A, 4) || (a->Dskip && !aligned(a->Dskip, 4)) || (a->delta_bias && !aligned(a->delta_bias, 4)) ||
      (a->last_state && !aligned(a->last_state, 16)))
    return SS2D_ERR_INVALID_ARGUMENT;
  const ScanLayout lay = scan_layout(a->batch, a->dim, a->dstate, a->seqlen, a->ngroups, a->dtype);
  if (a->workspace && (a->workspace_bytes < size_t(lay.total) || !aligned(a->workspace, kAlign)))
    return SS2D_ERR_INVALID_ARGUMENT;

  ScanFwdParams p{};
  p.u = a->u;
  p.delta = a->delta;
  p.A = a->A;
  p.Bm = a->Bm;
  p.Cm = a->Cm;
  p.Dskip = a->Dskip;
  p.z = a->z;
  p.delta_bias = a->delta_bias;
  p.out = a->out;
  p.last_state = a->last_state;
  p.batch = a->batch;
  p.dim = a->dim;
  p.L = a->seqlen;
  p.G = a->ngroups;
  p.per_group = lay.per_group;
  p.dblocks = lay.dblocks;
  p.n_ckpt = int(lay.n_ckpt);
  p.ckpt_every = lay.ckpt_every;
  p.N = int(a->dstate);
  p.softplus = a->delta_softplus ? 1 : 0;
  p.ss2d = 0;
  p.dtype = a->dtype;
  p.vec = (a->seqlen % 4 == 0) && vec_aligned(a->dtype, {a->u, a->delta, a->Bm, a->Cm, a->z, a->out});
  p.chunk_len = lay.chunk_len;
  p.n_chunks = lay.n_chunks;
  if (!a->workspace) {  // no scratch for the chunk states: one chunk per row
    p.chunk_len = cdiv(a->seqlen, kTile) * kTile;
    p.n_chunks = 1;
  }
  p.store_states = keep_states && a->workspace != nullptr;
  p.out_f32 = out_f32 ? 1 : 0;
  if (a->batch * a->ngroups * lay.dblocks * 2 * p.n_chunks > kMaxBlocks) return SS2D_ERR_INVALID_ARGUMENT;
  if (a->workspace) {
    p.ckpt = reinterpret_cast<float*>(at(a->workspace, lay.off_ckpt));
    p.chunk_sum = reinterpret_cast<float*>(at(a->workspace, lay.off_sum));
  }
  hipError_t e = hipSuccess;
  if (p.n_chunks > 1) {
    p.pass = 1;
    e = launch_scan_fwd(p, stream);
    if (e == hipSuccess) e = launch_chunk_combine(p, stream);
  }
  p.pass = 0;
  if (e == hipSuccess) e = launch_scan_fwd(p, stream);
  return status_from(e);
}

int selective_scan_fwd(const ss_fwd_args* a, hipStream_t stream) {
  return scan_fwd_impl(a, a && a->workspace != nullptr, stream);
}

int selective_scan_step(const ss_step_args* a, hipStream_t stream) {
  if (!a) return SS2D_ERR_INVALID_ARGUMENT;
  if (!dtype_ok(a->dtype)) return SS2D_ERR_UNSUPPORTED;
  if (a->dstate < 1 || a->dstate > 64) return SS2D_ERR_UNSUPPORTED;
  if (a->batch < 0 || a->dim < 0 || a->ngroups < 1 || a->dim % a->ngroups != 0) return SS2D_ERR_INVALID_ARGUMENT;
  const int64_t rows = a->batch * a->dim;
  if (rows == 0) return SS2D_OK;
  if (cdiv(rows * padded_states(a->dstate), 256) > kMaxBlocks) return SS2D_ERR_INVALID_ARGUMENT;
  if (!a->state || !a->x || !a->delta || !a->A || !a->Bm || !a->Cm || !a->out) return SS2D_ERR_INVALID_ARGUMENT;
  if (!elem_aligned(a->dtype, {a->x, a->delta, a->Bm, a->Cm, a->z, a->out})) return SS2D_ERR_INVALID_ARGUMENT;
  if (!aligned(a->state, 4) || !aligned(a->A, 4) || (a->Dskip && !aligned(a->Dskip, 4)) ||
      (a->delta_bias && !aligned(a->delta_bias, 4)))
    return SS2D_ERR_INVALID_ARGUMENT;
  StepParams p{};
  p.state = a->state;
  p.x = a->x;
  p.delta = a->delta;
  p.A = a->A;
  p.Bm = a->Bm;
  p.Cm = a->Cm;
  p.Dskip = a->Dskip;
  p.z = a->z;
  p.delta_bias = a->delta_bias;
  p.out = a->out;
  p.batch = a->batch;
  p.dim = a->dim;
  p.G = a->ngroups;
  p.N = int(a->dstate);
  p.softplus = a->delta_softplus ? 1 : 0;
  p.dtype = a->dtype;
  return status_from(launch_scan_step(p, stream));
}

size_t ss2d_workspace_bytes(int64_t batch, int64_t dim, int64_t height, int64_t width, int64_t dstate, int dtype) {
  if (batch < 0 || dim < 0 || height < 0 || width < 0 || dstate < 1 || !dtype_ok(dtype)) return 0;
  return size_t(ss2d_layout(batch, dim, height, width, dstate, dtype).total);
}

size_t ss2d_proj_workspace_bytes(int64_t batch, int64_t dim, int64_t height, int64_t width, int64_t dstate,
                                 int64_t dt_rank, int dtype) {
  if (batch < 0 || dim < 0 || height < 0 || width < 0 || dstate < 1 || dstate > 64 || !dtype_ok(dtype) ||
      dt_rank < 1 || dt_rank > (dim > 0 ? dim : 1))
    return 0;
  return size_t(ss2d_layout(batch, dim, height, width, dstate, dtype, dt_rank).total);
}

// Stages of the SS2D forward (all on one workspace).
// The map the four routes scan: x, or its fp32 copy in the workspace (the input front's output,
// or the cast copy the projected path scans).
static const void* scan_input(const void* x, bool in_ws, void* ws, const SS2DLayout& lay) {
  return in_ws ? static_cast<const void*>(at(ws, lay.off_xc)) : x;
}

static float* wsf(void* ws, int64_t off) { return reinterpret_cast<float*>(at(ws, off)); }


// The Δ/B/C producer: for each route k, x_dbl = x_proj_w[k] @ xs_k (rows dt, B, C), then
// delta = dt_proj_w[k] @ dt, all fp32 in route order in the workspace.  xs_k is the fp32 map
// (routes 0, 2) or its transpose (routes 1, 3), read backwards for the reversed routes.
static int ss2d_project(const ss2d_fwd_args* a, const SS2DLayout& lay, hipStream_t stream) {
  const int64_t L = a->height * a->width, D = a->dim, N = a->dstate, R = a->dt_rank, Cp = R + 2 * N;
  void* ws = a->workspace;
  ProjArgs f{};  // x_dbl (Cp x L) = x_proj_w[k] (Cp x D) xs_k (D x L)
  f.w = a->x_proj_w;
  f.w_k = Cp * D;
  f.w_i = D;
  f.w_kk = 1;
  f.x0 = wsf(ws, lay.off_xc);
  f.x1 = wsf(ws, lay.off_xT);
  f.x_b = D * L;
  f.x_r = L;
  f.c = wsf(ws, lay.off_pxdbl);
  f.c_b = 4 * Cp * L;
  f.c_k = Cp * L;
  f.c_r = L;
  f.M = Cp;
  f.K = D;
  f.L = L;
  f.batch = a->batch;
  f.nk = 4;
  f.rev_routes = 1;
  if (D % 4 == 0 && (reinterpret_cast<uintptr_t>(a->x_proj_w) & 15) == 0) {  // routes k and k + 2 from one read of their map
    f.M = 2 * Cp;
    f.nk = 2;
    f.rev_routes = 0;
    f.pair_routes = 1;
  }
  if (launch_proj(f, stream) != hipSuccess) return SS2D_ERR_HIP;
  if (fused_dt(R)) return SS2D_OK;
  ProjArgs g{};  // delta (D x L) = dt_proj_w[k] (D x R) dt (R x L)
  g.w = a->dt_proj_w;
  g.w_k = D * R;
  g.w_i = R;
  g.w_kk = 1;
  g.x0 = g.x1 = wsf(ws, lay.off_pxdbl);
  g.x_b = 4 * Cp * L;
  g.x_k = Cp * L;
  g.x_r = L;
  g.c = wsf(ws, lay.off_pdelta);
  g.c_b = 4 * D * L;
  g.c_k = D * L;
  g.c_r = L;
  g.M = D;
  g.K = R;
  g.L = L;
  g.batch = a->batch;
  g.nk = 4;
  return status_from(launch_proj(g, stream));
}

// Stage 0: the column-major copy of the scanned map (and, with the input front, the map itself).
static int ss2d_transpose_stage(const ss2d_fwd_args* a, const SS2DLayout& lay, hipStream_t stream) {
  if (a->conv_w) {
    FrontArgs f{};
    f.x = a->x;
    f.w = a->conv_w;
    f.bias = a->conv_b;
    f.xc = reinterpret_cast<float*>(at(a->workspace, lay.off_xc));
    f.xcT = reinterpret_cast<float*>(at(a->workspace, lay.off_xT));
    f.batch = a->batch;
    f.C = a->dim;
    f.H = a->height;
    f.W = a->width;
    f.k = a->conv_k;
    f.dtype = a->dtype;
    if (launch_front_fwd(f, stream) != hipSuccess) return SS2D_ERR_HIP;
    return a->x_proj_w ? ss2d_project(a, lay, stream) : SS2D_OK;
  }
  if (a->x_proj_w) {
    if (launch_cast_transpose(a->x, wsf(a->workspace, lay.off_xc), wsf(a->workspace, lay.off_xT), a->batch, a->dim,
                              a->height, a->width, a->dtype, stream) != hipSuccess)
      return SS2D_ERR_HIP;
    return ss2d_project(a, lay, stream);
  }
  return status_from(launch_transpose(a->x, at(a->workspace, lay.off_xT), a->batch, a->dim, a->height, a->width,
                                      esize(a->dtype), stream));
}

// The four route scans with fp32 outputs (route order) into the ys region; when keep_states,
// the state before every ckpt_every-th step of every row is kept for the backward.
static int ss2d_scan_stage(const ss2d_fwd_args* a, const SS2DLayout& lay, bool keep_states, hipStream_t stream) {
  const int64_t L = a->height * a->width;
  ScanFwdParams p{};
  const bool proj = a->x_proj_w != nullptr;  // fp32 scans of the projected inputs
  const ScanLayout& sl = proj ? lay.scan32 : lay.scan;
  p.u = scan_input(a->x, (a->conv_w != nullptr || a->x_proj_w != nullptr), a->workspace, lay);
  p.uT = at(a->workspace, lay.off_xT);
  p.u_f32 = a->conv_w != nullptr && a->dtype != 0 && !proj;
  p.delta = proj ? (fused_dt(a->dt_rank) ? nullptr : wsf(a->workspace, lay.off_pdelta)) : a->delta;
  if (proj && fused_dt(a->dt_rank)) {
    p.dt = wsf(a->workspace, lay.off_pxdbl);
    p.dt_w = a->dt_proj_w;
    p.dt_rank = int(a->dt_rank);
  }
  p.A = a->A;
  p.Bm = proj ? wsf(a->workspace, lay.off_pxdbl) + a->dt_rank * L : a->Bm;
  p.Cm = proj ? wsf(a->workspace, lay.off_pxdbl) + (a->dt_rank + a->dstate) * L : a->Cm;
  p.bc_stride = proj ? (a->dt_rank + 2 * a->dstate) * L : 0;
  p.delta_bias = a->delta_bias;
  p.out = at(a->workspace, lay.off_ys);
  p.batch = a->batch;
  p.dim = 4 * a->dim;
  p.L = L;
  p.G = 4;
  p.per_group = a->dim;
  p.dblocks = sl.dblocks;
  p.n_ckpt = int(sl.n_ckpt);
  p.ckpt_every = sl.ckpt_every;
  p.N = int(a->dstate);
  p.softplus = a->delta_softplus ? 1 : 0;
  p.ss2d = 1;
  p.out_blocked = ss2d_routes_blocked(a->height, a->width) ? 1 : 0;
  p.dtype = proj ? SS2D_DTYPE_F32 : a->dtype;
  p.vec = (L % 4 == 0) && vec_aligned(p.dtype, {p.u, p.delta, p.Bm, p.Cm});
  p.chunk_len = sl.chunk_len;
  p.n_chunks = sl.n_chunks;
  if (a->batch * 4 * sl.dblocks * 2 * p.n_chunks > kMaxBlocks) return SS2D_ERR_INVALID_ARGUMENT;
  p.chunk_sum = reinterpret_cast<float*>(at(a->workspace, lay.off_scan + lay.scan.off_sum));
  if (p.n_chunks > 1 || keep_states) p.ckpt = reinterpret_cast<float*>(at(a->workspace, lay.off_scan + lay.scan.off_ckpt));
  p.store_states = keep_states;
  hipError_t err = hipSuccess;
  if (p.n_chunks > 1) {
    p.pass = 1;
    err = launch_scan_fwd(p, stream);
    if (err == hipSuccess) err = launch_chunk_combine(p, stream);
    if (err != hipSuccess) return SS2D_ERR_HIP;
  }
  p.pass = 0;
  return status_from(launch_scan_fwd(p, stream));
}

static int ss2d_merge_stage(const ss2d_fwd_args* a, const SS2DLayout& lay, hipStream_t stream) {
  MergeArgs m{};
  m.routes = at(a->workspace, lay.off_ys);
  m.routes_f32 = 1;  // the scan stage writes fp32 route outputs
  m.routes_blocked = ss2d_routes_blocked(a->height, a->width) ? 1 : 0;  // in its layout
  m.x = scan_input(a->x, (a->conv_w != nullptr || a->x_proj_w != nullptr), a->workspace, lay);
  m.x_f32 = (a->conv_w != nullptr || a->x_proj_w != nullptr);
  m.Dskip = a->Dskip;
  m.batch = a->batch;
  m.C = a->dim;
  m.H = a->height;
  m.W = a->width;
  m.dtype = a->dtype;
  if (!a->layer_norm) {
    m.z = a->z;
    m.y = a->out;
    // a training forward with a gate keeps the fp32 pre-gate map: the gate's backward reads it
    // instead of the four route outputs
    if (a->keep_states && a->z) m.merged_f32 = reinterpret_cast<float*>(at(a->workspace, lay.off_merged));
    return status_from(launch_merge(m, stream));
  }
  // with the LayerNorm: the fp32 merged map, then the normalisation and the gate per pixel
  float* merged = reinterpret_cast<float*>(at(a->workspace, lay.off_merged));
  m.merged_f32 = merged;
  if (launch_merge(m, stream) != hipSuccess) return SS2D_ERR_HIP;
  LnArgs l{};
  l.M = merged;
  l.w = a->ln_w;
  l.b = a->ln_b;
  l.z = a->z;
  l.out = a->out;
  l.batch = a->batch;
  l.C = a->dim;
  l.L = a->height * a->width;
  l.eps = a->ln_eps;
  l.dtype = a->dtype;
  return status_from(launch_ln_gate_fwd(l, stream));
}

static int check_ss2d(int64_t batch, int64_t dim, int64_t height, int64_t width, int64_t dstate, int dtype) {
  if (!dtype_ok(dtype)) return SS2D_ERR_UNSUPPORTED;
  if (batch < 0 || dim < 0 || height < 0 || width < 0) return SS2D_ERR_INVALID_ARGUMENT;
  if (dstate < 1 || dstate > 64) return SS2D_ERR_UNSUPPORTED;
  if (height > (1 << 30) || width > (1 << 30)) return SS2D_ERR_INVALID_ARGUMENT;
  return SS2D_OK;
}

// The LayerNorm parameters: fp32, 4-byte aligned; eps finite and >= 0.
static int check_ln(int on, const float* w, const float* b, float eps) {
  if (!on) return SS2D_OK;
  if ((w && !aligned(w, 4)) || (b && !aligned(b, 4))) return SS2D_ERR_INVALID_ARGUMENT;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return SS2D_ERR_INVALID_ARGUMENT;
  return SS2D_OK;
}

// The Δ/B/C producer's weights: both or neither, dt_rank in [1, dim], fp32 4-byte aligned.
static int check_proj(const float* wx, const float* wdt, int rank, int64_t dim) {
  if (!wx) return wdt ? SS2D_ERR_INVALID_ARGUMENT : SS2D_OK;
  if (!wdt || rank < 1 || rank > dim || !aligned(wx, 4) || !aligned(wdt, 4)) return SS2D_ERR_INVALID_ARGUMENT;
  return SS2D_OK;
}

// The input front's filter: odd size 1..7, fp32 pointers 4-byte aligned.
static int check_front(const float* w, const float* b, int k) {
  if (!w) return b ? SS2D_ERR_INVALID_ARGUMENT : SS2D_OK;
  if (k < 1 || k > kFrontMaxK || k % 2 == 0) return SS2D_ERR_UNSUPPORTED;
  if (!aligned(w, 4) || (b && !aligned(b, 4))) return SS2D_ERR_INVALID_ARGUMENT;
  return SS2D_OK;
}

// Validation shared by ss2d_fwd and ss2d_fwd_stage.  Returns SS2D_OK with *empty set when there
// is nothing to compute.
static int validate_ss2d_fwd(const ss2d_fwd_args* a, SS2DLayout* lay, bool* empty, bool check_ws = true) {
  *empty = false;
  if (!a) return SS2D_ERR_INVALID_ARGUMENT;
  int st = check_ss2d(a->batch, a->dim, a->height, a->width, a->dstate, a->dtype);
  if (st == SS2D_OK) st = check_front(a->conv_w, a->conv_b, a->conv_k);
  if (st == SS2D_OK) st = check_ln(a->layer_norm, a->ln_w, a->ln_b, a->ln_eps);
  if (st == SS2D_OK && a->dim > 0) st = check_proj(a->x_proj_w, a->dt_proj_w, a->dt_rank, a->dim);
  if (st != SS2D_OK) return st;
  if (a->batch * a->dim * a->height * a->width == 0) {
    *empty = true;
    return SS2D_OK;
  }
  const bool proj = a->x_proj_w != nullptr;  // delta, Bm, Cm come from the producer
  if (!a->x || (!proj && (!a->delta || !a->Bm || !a->Cm)) || !a->A || !a->out || (check_ws && !a->workspace))
    return SS2D_ERR_INVALID_ARGUMENT;
  if (!elem_aligned(a->dtype, {a->x, proj ? nullptr : a->delta, proj ? nullptr : a->Bm, proj ? nullptr : a->Cm, a->z,
                               a->out}))
    return SS2D_ERR_INVALID_ARGUMENT;
  if (!aligned(a->A, 4) || (a->Dskip && !aligned(a->Dskip, 4)) || (a->delta_bias && !aligned(a->delta_bias, 4)))
    return SS2D_ERR_INVALID_ARGUMENT;
  *lay = ss2d_layout(a->batch, a->dim, a->height, a->width, a->dstate, a->dtype, proj ? a->dt_rank : 0);
  if (check_ws && (a->workspace_bytes < size_t(lay->total) || !aligned(a->workspace, kAlign)))
    return SS2D_ERR_INVALID_ARGUMENT;
  if (a->batch * a->dim * cdiv(a->height, 32) * cdiv(a->width, 32) > kMaxBlocks) return SS2D_ERR_INVALID_ARGUMENT;
  return SS2D_OK;
}

// The single-kernel path (small state sizes, plain SS2D: no front, LayerNorm, producer or
// kept states), when its shape and alignment conditions hold.
static bool plane_path(const ss2d_fwd_args* a, PlaneFwdArgs* p) {
  if (a->conv_w || a->x_proj_w || a->layer_norm || a->keep_states) return false;
  p->x = a->x;
  p->delta = a->delta;
  p->Bm = a->Bm;
  p->Cm = a->Cm;
  p->A = a->A;
  p->Dskip = a->Dskip;
  p->delta_bias = a->delta_bias;
  p->z = a->z;
  p->out = a->out;
  p->batch = a->batch;
  p->dim = a->dim;
  p->H = a->height;
  p->W = a->width;
  p->N = int(a->dstate);
  p->dtype = a->dtype;
  p->softplus = a->delta_softplus ? 1 : 0;
  return plane_fwd_supported(*p);
}

int ss2d_fwd_single_kernel(const ss2d_fwd_args* a) {
  SS2DLayout lay;
  bool empty;
  if (validate_ss2d_fwd(a, &lay, &empty) != SS2D_OK || empty) return 0;
  PlaneFwdArgs p{};
  return plane_path(a, &p) ? 1 : 0;
}

int ss2d_fwd(const ss2d_fwd_args* a, hipStream_t stream) {
  SS2DLayout lay;
  bool empty;
  int st = validate_ss2d_fwd(a, &lay, &empty);
  if (st != SS2D_OK || empty) return st;
  PlaneFwdArgs pa{};
  if (plane_path(a, &pa)) return status_from(launch_plane_fwd(pa, stream));
  st = ss2d_transpose_stage(a, lay, stream);
  if (st == SS2D_OK) st = ss2d_scan_stage(a, lay, a->keep_states != 0, stream);
  if (st == SS2D_OK) st = ss2d_merge_stage(a, lay, stream);
  return st;
}

// ---- the allocation-free forward ------------------------------------------------------
// Its scratch: one array per GPU, allocated with the library's code object when the library
// is loaded on that GPU and held until the process ends.  Host code never uses the array's
// name as an address (on the host it is only a stand-in for the device symbol): the device
// address comes from hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = size_t(128) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// The device address of the current device's scratch (looked up on its first use there).
static int scratch_of_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SS2D_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SS2D_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SS2D_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return SS2D_OK;
}

size_t ss2d_fwd_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

int ss2d_fwd_noalloc(const ss2d_fwd_args* a, hipStream_t stream) {
  SS2DLayout lay;
  bool empty;
  int st = validate_ss2d_fwd(a, &lay, &empty, /*check_ws=*/false);
  if (st != SS2D_OK || empty) return st;
  if (a->keep_states) return SS2D_ERR_INVALID_ARGUMENT;  // no backward can reach the scratch
  PlaneFwdArgs pa{};
  if (plane_path(a, &pa)) return status_from(launch_plane_fwd(pa, stream));  // needs no scratch
  if (size_t(lay.total) > kScratchBytes) return SS2D_ERR_TOO_LARGE;
  void* ptr = nullptr;
  st = scratch_of_current_device(&ptr);
  if (st != SS2D_OK) return st;
  ss2d_fwd_args c = *a;
  c.workspace = ptr;
  c.workspace_bytes = kScratchBytes;
  st = ss2d_transpose_stage(&c, lay, stream);
  if (st == SS2D_OK) st = ss2d_scan_stage(&c, lay, false, stream);
  if (st == SS2D_OK) st = ss2d_merge_stage(&c, lay, stream);
  return st;
}

int ss2d_fwd_stage(const ss2d_fwd_args* a, int stage, hipStream_t stream) {
  if (stage < SS2D_STAGE_TRANSPOSE || stage > SS2D_STAGE_MERGE) return SS2D_ERR_INVALID_ARGUMENT;
  SS2DLayout lay;
  bool empty;
  int st = validate_ss2d_fwd(a, &lay, &empty);
  if (st != SS2D_OK || empty) return st;
  if (stage == SS2D_STAGE_TRANSPOSE) return ss2d_transpose_stage(a, lay, stream);
  if (stage == SS2D_STAGE_SCAN) return ss2d_scan_stage(a, lay, a->keep_states != 0, stream);
  return ss2d_merge_stage(a, lay, stream);
}

// The forward scans with no outputs: only the checkpoint states (for a backward without them).
static hipError_t scan_states_only(ScanFwdParams p, hipStream_t stream) {
  p.out = nullptr;
  p.last_state = nullptr;
  p.store_states = 1;
  hipError_t e = hipSuccess;
  if (p.n_chunks > 1) {
    p.pass = 1;
    e = launch_scan_fwd(p, stream);
    if (e == hipSuccess) e = launch_chunk_combine(p, stream);
    if (e != hipSuccess) return e;
  }
  p.pass = 0;
  return launch_scan_fwd(p, stream);
}

// Zero the gradients that are sums over an empty set.
static int zero_param_grads(float* dA, float* dD, float* dbias, int64_t dim, int64_t dstate, hipStream_t stream) {
  hipError_t e = launch_fill_zero(dA, dim * dstate, stream);
  if (e == hipSuccess && dD) e = launch_fill_zero(dD, dim, stream);
  if (e == hipSuccess && dbias) e = launch_fill_zero(dbias, dim, stream);
  return status_from(e);
}

// Adjoint scans + partial-sum reduction, shared by selective_scan_bwd and ss2d_bwd.
static int run_scan_bwd(ScanBwdParams bp, const ScanLayout& lay, void* ws, void* dB, void* dC, float* dA, float* dD,
                        float* dbias, hipStream_t stream) {
  bp.ckpt = reinterpret_cast<const float*>(at(ws, lay.off_ckpt));
  bp.chunk_sum = reinterpret_cast<float*>(at(ws, lay.off_sum));
  bp.lam_carry = reinterpret_cast<float*>(at(ws, lay.off_lam));
  bp.dB_part = reinterpret_cast<float*>(at(ws, lay.off_dB));
  bp.dC_part = reinterpret_cast<float*>(at(ws, lay.off_dC));
  bp.dA_part = reinterpret_cast<float*>(at(ws, lay.off_dA));
  bp.dD_part = reinterpret_cast<float*>(at(ws, lay.off_dD));
  bp.dbias_part = reinterpret_cast<float*>(at(ws, lay.off_dbias));
  bp.chunk_len = lay.bwd_chunk_len;
  bp.n_chunks = lay.bwd_n_chunks;
  bp.n_ckpt = int(lay.n_ckpt);
  hipError_t e = hipSuccess;
  if (bp.n_chunks > 1) {
    bp.pass = 1;
    e = launch_scan_bwd(bp, stream);
    if (e == hipSuccess) e = launch_lambda_combine(bp, stream);
    if (e != hipSuccess) return SS2D_ERR_HIP;
  }
  bp.pass = 0;
  e = launch_scan_bwd(bp, stream);
  if (e != hipSuccess) return SS2D_ERR_HIP;
  BwdReduceArgs r{};
  r.dB_part = bp.dB_part;
  r.dC_part = bp.dC_part;
  r.dA_part = bp.dA_part;
  r.dD_part = bp.dD_part;
  r.dbias_part = bp.dbias_part;
  r.dB = dB;
  r.dC = dC;
  r.dA = dA;
  r.dD = dD;
  r.dbias = dbias;
  r.batch = bp.batch;
  r.dim = bp.dim;
  r.L = bp.L;
  r.G = bp.G;
  r.dblocks = bp.dblocks;
  r.n_chunks = bp.n_chunks;
  r.N = bp.N;
  r.dtype = bp.dtype;
  r.bc_out_stride = bp.bc_stride;
  r.bc_blocked = bp.bc_blocked;
  return status_from(launch_bwd_reduce(r, stream));
}

int selective_scan_bwd(const ss_bwd_args* a, hipStream_t stream) {
  if (!a) return SS2D_ERR_INVALID_ARGUMENT;
  int st = check_scan_shapes(a->batch, a->dim, a->dstate, a->seqlen, a->ngroups, a->dtype);
  if (st != SS2D_OK) return st;
  if ((a->Dskip && !a->dDskip) || (a->delta_bias && !a->ddelta_bias) || (a->z && !a->dz))
    return SS2D_ERR_INVALID_ARGUMENT;
  if (a->dim == 0) return SS2D_OK;
  if (!a->dA) return SS2D_ERR_INVALID_ARGUMENT;
  if (a->batch == 0 || a->seqlen == 0)
    return zero_param_grads(a->dA, a->Dskip ? a->dDskip : nullptr, a->delta_bias ? a->ddelta_bias : nullptr, a->dim,
                            a->dstate, stream);
  if (!a->u || !a->delta || !a->A || !a->Bm || !a->Cm || !a->dout || !a->du || !a->ddelta || !a->dBm || !a->dCm ||
      !a->workspace)
    return SS2D_ERR_INVALID_ARGUMENT;
  if (!elem_aligned(a->dtype, {a->u, a->delta, a->Bm, a->Cm, a->z, a->dout, a->du, a->ddelta, a->dBm, a->dCm, a->dz}))
    return SS2D_ERR_INVALID_ARGUMENT;
  if (!aligned(a->A, 4) || !aligned(a->dA, 4) || (a->Dskip && !aligned(a->Dskip, 4)) ||
      (a->delta_bias && !aligned(a->delta_bias, 4)) || (a->dDskip && !aligned(a->dDskip, 4)) ||
      (a->ddelta_bias && !aligned(a->ddelta_bias, 4)))
    return SS2D_ERR_INVALID_ARGUMENT;
  const ScanLayout lay = scan_layout(a->batch, a->dim, a->dstate, a->seqlen, a->ngroups, a->dtype);
  if (a->workspace_bytes < size_t(lay.total) || !aligned(a->workspace, kAlign)) return SS2D_ERR_INVALID_ARGUMENT;
  if (a->batch * a->ngroups * lay.dblocks * lay.bwd_n_chunks > kMaxBlocks ||
      a->batch * a->ngroups * lay.dblocks * 2 * lay.n_chunks > kMaxBlocks)
    return SS2D_ERR_INVALID_ARGUMENT;
  const bool vec = (a->seqlen % 4 == 0) &&
                   vec_aligned(a->dtype, {a->u, a->delta, a->Bm, a->Cm, a->z, a->dout, a->du, a->ddelta});

  if (!a->workspace_has_states) {
    ScanFwdParams p{};
    p.u = a->u;
    p.delta = a->delta;
    p.A = a->A;
    p.Bm = a->Bm;
    p.Cm = a->Cm;
    p.delta_bias = a->delta_bias;
    p.ckpt = reinterpret_cast<float*>(at(a->workspace, lay.off_ckpt));
    p.chunk_sum = reinterpret_cast<float*>(at(a->workspace, lay.off_sum));
    p.batch = a->batch;
    p.dim = a->dim;
    p.L = a->seqlen;
    p.G = a->ngroups;
    p.per_group = lay.per_group;
    p.dblocks = lay.dblocks;
    p.chunk_len = lay.chunk_len;
    p.n_chunks = lay.n_chunks;
    p.n_ckpt = int(lay.n_ckpt);
    p.ckpt_every = lay.ckpt_every;
    p.N = int(a->dstate);
    p.softplus = a->delta_softplus ? 1 : 0;
    p.dtype = a->dtype;
    p.vec = vec;
    if (scan_states_only(p, stream) != hipSuccess) return SS2D_ERR_HIP;
  }
  ScanBwdParams bp{};
  bp.u = a->u;
  bp.delta = a->delta;
  bp.A = a->A;
  bp.Bm = a->Bm;
  bp.Cm = a->Cm;
  bp.Dskip = a->Dskip;
  bp.z = a->z;
  bp.delta_bias = a->delta_bias;
  bp.dout = a->dout;
  bp.du = a->du;
  bp.ddelta = a->ddelta;
  bp.dz = a->dz;
  bp.batch = a->batch;
  bp.dim = a->dim;
  bp.L = a->seqlen;
  bp.G = a->ngroups;
  bp.per_group = lay.per_group;
  bp.dblocks = lay.dblocks;
  bp.N = int(a->dstate);
  bp.softplus = a->delta_softplus ? 1 : 0;
  bp.ss2d = 0;
  bp.dtype = a->dtype;
  bp.vec = vec;
  return run_scan_bwd(bp, lay, a->workspace, a->dBm, a->dCm, a->dA, a->Dskip ? a->dDskip : nullptr,
                      a->delta_bias ? a->ddelta_bias : nullptr, stream);
}

// The Δ/B/C producer's gradient, given the scans' fp32 gradients of delta, B and C (route order,
// dB and dC already in rows [R, R + 2N) of the x_dbl gradient):
//   d dt = dt_proj_w[k]^T ddelta (rows [0, R));  du_k += x_proj_w[k]^T (d dt; dB; dC) (added to the
//   routes' du before the merge);  dx_proj_w[k] = sum_b (d dt; dB; dC) xs_k^T;
//   ddt_proj_w[k] = sum_b ddelta dt^T  (the weight products as partials of proj_splits slices,
//   then summed over the slices).
static int ss2d_project_bwd(const ss2d_bwd_args* a, const SS2DLayout& lay, hipStream_t stream) {
  const int64_t L = a->height * a->width, D = a->dim, N = a->dstate, R = a->dt_rank, Cp = R + 2 * N;
  const int64_t S = lay.proj_splits;
  void* ws = a->workspace;
  {  // d dt (R x L) = dt_proj_w[k]^T (R x D) ddelta (D x L)
    ProjArgs g{};
    g.w = a->dt_proj_w;
    g.w_k = D * R;
    g.w_i = 1;
    g.w_kk = R;
    g.x0 = g.x1 = wsf(ws, lay.off_pddelta);
    g.x_b = 4 * D * L;
    g.x_k = D * L;
    g.x_r = L;
    g.c = wsf(ws, lay.off_pdxdbl);
    g.c_b = 4 * Cp * L;
    g.c_k = Cp * L;
    g.c_r = L;
    g.M = R;
    g.K = D;
    g.L = L;
    g.batch = a->batch;
    g.nk = 4;
    if (launch_proj(g, stream) != hipSuccess) return SS2D_ERR_HIP;
  }
  {  // du_k (D x L) += x_proj_w[k]^T (D x Cp) dx_dbl (Cp x L), into the routes' du
    ProjArgs g{};
    g.w = a->x_proj_w;
    g.w_k = Cp * D;
    g.w_i = 1;
    g.w_kk = D;
    g.x0 = g.x1 = wsf(ws, lay.off_pdxdbl);
    g.x_b = 4 * Cp * L;
    g.x_k = Cp * L;
    g.x_r = L;
    g.c = wsf(ws, lay.off_ys);
    g.c_b = 4 * D * L;
    g.c_k = D * L;
    g.c_r = L;
    g.M = D;
    g.K = Cp;
    g.L = L;
    g.batch = a->batch;
    g.nk = 4;
    g.accumulate = 1;
    if (launch_proj(g, stream) != hipSuccess) return SS2D_ERR_HIP;
  }
  {  // dx_proj_w[k] (Cp x D) = sum_{b, l} dx_dbl[c, l] xs_k[d, l]; the reversed routes pair step l
     // of dx_dbl with pixel L-1-l of the source map
    WgradArgs g{};
    g.a = wsf(ws, lay.off_pdxdbl);
    g.a_b = 4 * Cp * L;
    g.a_k = Cp * L;
    g.a_r = L;
    g.b0 = wsf(ws, lay.off_xc);
    g.b1 = wsf(ws, lay.off_xT);
    g.b_b = D * L;
    g.b_r = L;
    g.c = wsf(ws, lay.off_pwx);
    g.M = 2 * Cp;  // routes k and k + 2 from one read of their map
    g.N = D;
    g.K = L;
    g.batch = a->batch;
    g.nk = 2;
    g.splits = int(S);
    g.rev_routes = 1;
    g.pair_routes = 1;
    if (launch_wgrad(g, stream) != hipSuccess) return SS2D_ERR_HIP;
  }
  {  // ddt_proj_w[k] (D x R) = sum_{b, l} ddelta[d, l] dt[r, l]
    WgradArgs g{};
    g.a = wsf(ws, lay.off_pddelta);
    g.a_b = 4 * D * L;
    g.a_k = D * L;
    g.a_r = L;
    g.b0 = g.b1 = wsf(ws, lay.off_pxdbl);
    g.b_b = 4 * Cp * L;
    g.b_k = Cp * L;
    g.b_r = L;
    g.c = wsf(ws, lay.off_pwdt);
    g.M = D;
    g.N = R;
    g.K = L;
    g.batch = a->batch;
    g.nk = 4;
    g.splits = int(S);
    if (launch_wgrad(g, stream) != hipSuccess) return SS2D_ERR_HIP;
  }
  if (launch_sum_parts(wsf(ws, lay.off_pwx), a->dx_proj_w, 4 * Cp * D, S, stream) != hipSuccess ||
      launch_sum_parts(wsf(ws, lay.off_pwdt), a->ddt_proj_w, 4 * D * R, S, stream) != hipSuccess)
    return SS2D_ERR_HIP;
  return SS2D_OK;
}

int ss2d_bwd(const ss2d_bwd_args* a, hipStream_t stream) {
  if (!a) return SS2D_ERR_INVALID_ARGUMENT;
  int st = check_ss2d(a->batch, a->dim, a->height, a->width, a->dstate, a->dtype);
  if (st == SS2D_OK) st = check_front(a->conv_w, a->conv_b, a->conv_k);
  if (st == SS2D_OK) st = check_ln(a->layer_norm, a->ln_w, a->ln_b, a->ln_eps);
  if (st == SS2D_OK && a->dim > 0) st = check_proj(a->x_proj_w, a->dt_proj_w, a->dt_rank, a->dim);
  if (st != SS2D_OK) return st;
  const bool lnw = a->layer_norm && a->ln_w, lnb = a->layer_norm && a->ln_b;
  const bool proj = a->x_proj_w != nullptr;
  if ((a->Dskip && !a->dDskip) || (a->delta_bias && !a->ddelta_bias) || (a->z && !a->dz) ||
      (a->conv_w && !a->dconv_w) || (a->conv_b && !a->dconv_b) || (lnw && !a->dln_w) || (lnb && !a->dln_b) ||
      (proj && (!a->dx_proj_w || !a->ddt_proj_w)))
    return SS2D_ERR_INVALID_ARGUMENT;
  if ((a->dconv_w && !aligned(a->dconv_w, 4)) || (a->dconv_b && !aligned(a->dconv_b, 4)) ||
      (a->dln_w && !aligned(a->dln_w, 4)) || (a->dln_b && !aligned(a->dln_b, 4)) ||
      (proj && (!aligned(a->dx_proj_w, 4) || !aligned(a->ddt_proj_w, 4))))
    return SS2D_ERR_INVALID_ARGUMENT;
  if (a->dim == 0) return SS2D_OK;
  if (!a->dA) return SS2D_ERR_INVALID_ARGUMENT;
  if (a->batch * a->height * a->width == 0) {
    st = zero_param_grads(a->dA, a->Dskip ? a->dDskip : nullptr, a->delta_bias ? a->ddelta_bias : nullptr,
                          4 * a->dim, a->dstate, stream);
    if (st == SS2D_OK && a->conv_w)
      st = zero_param_grads(a->dconv_w, a->conv_b ? a->dconv_b : nullptr, nullptr, a->dim,
                            int64_t(a->conv_k) * a->conv_k, stream);
    if (st == SS2D_OK && lnw) st = status_from(launch_fill_zero(a->dln_w, a->dim, stream));
    if (st == SS2D_OK && lnb) st = status_from(launch_fill_zero(a->dln_b, a->dim, stream));
    if (st == SS2D_OK && proj) {
      const int64_t Cp = a->dt_rank + 2 * a->dstate;
      st = status_from(launch_fill_zero(a->dx_proj_w, 4 * Cp * a->dim, stream));
      if (st == SS2D_OK) st = status_from(launch_fill_zero(a->ddt_proj_w, 4 * a->dim * a->dt_rank, stream));
    }
    return st;
  }
  if (!a->x || !a->A || !a->dout || !a->dx || !a->workspace ||
      (!proj && (!a->delta || !a->Bm || !a->Cm || !a->ddelta || !a->dBm || !a->dCm)))
    return SS2D_ERR_INVALID_ARGUMENT;
  if (!elem_aligned(a->dtype, {a->x, a->z, a->dout, a->dx, a->dz}) ||
      (!proj && !elem_aligned(a->dtype, {a->delta, a->Bm, a->Cm, a->ddelta, a->dBm, a->dCm})))
    return SS2D_ERR_INVALID_ARGUMENT;
  if (!aligned(a->A, 4) || !aligned(a->dA, 4) || (a->Dskip && !aligned(a->Dskip, 4)) ||
      (a->delta_bias && !aligned(a->delta_bias, 4)) || (a->dDskip && !aligned(a->dDskip, 4)) ||
      (a->ddelta_bias && !aligned(a->ddelta_bias, 4)))
    return SS2D_ERR_INVALID_ARGUMENT;
  const SS2DLayout lay =
      ss2d_layout(a->batch, a->dim, a->height, a->width, a->dstate, a->dtype, proj ? a->dt_rank : 0);
  if (a->workspace_bytes < size_t(lay.total) || !aligned(a->workspace, kAlign)) return SS2D_ERR_INVALID_ARGUMENT;
  if (a->batch * a->dim * cdiv(a->height, 32) * cdiv(a->width, 32) > kMaxBlocks ||
      a->batch * 4 * lay.scan.dblocks * 2 * (proj ? lay.scan32.n_chunks : lay.scan.n_chunks) > kMaxBlocks ||
      a->batch * 4 * lay.scan.dblocks * lay.scan.bwd_n_chunks > kMaxBlocks)
    return SS2D_ERR_INVALID_ARGUMENT;
  const int64_t L = a->height * a->width;

  // forward again (unless the workspace holds it): transposed x, route outputs, checkpoint states
  if (!a->workspace_has_states) {
    ss2d_fwd_args f{};
    f.x = a->x;
    f.delta = a->delta;
    f.A = a->A;
    f.Bm = a->Bm;
    f.Cm = a->Cm;
    f.Dskip = a->Dskip;
    f.delta_bias = a->delta_bias;
    f.workspace = a->workspace;
    f.workspace_bytes = a->workspace_bytes;
    f.batch = a->batch;
    f.dim = a->dim;
    f.height = a->height;
    f.width = a->width;
    f.dstate = a->dstate;
    f.dtype = a->dtype;
    f.delta_softplus = a->delta_softplus;
    f.conv_w = a->conv_w;
    f.conv_b = a->conv_b;
    f.conv_k = a->conv_k;
    f.x_proj_w = a->x_proj_w;
    f.dt_proj_w = a->dt_proj_w;
    f.dt_rank = a->dt_rank;
    st = ss2d_transpose_stage(&f, lay, stream);
    if (st == SS2D_OK) st = ss2d_scan_stage(&f, lay, true, stream);
    if (st != SS2D_OK) return st;
  }

  const void* u = scan_input(a->x, (a->conv_w != nullptr || a->x_proj_w != nullptr), a->workspace, lay);
  if (a->layer_norm) {
    // the LayerNorm's and the gate's backward need the whole pixel: the fp32 merged map first,
    // then dz, dM (grid order) and the parameter partials per pixel block, then dM transposed
    float* merged = reinterpret_cast<float*>(at(a->workspace, lay.off_merged));
    float* dM = reinterpret_cast<float*>(at(a->workspace, lay.off_dM));
    if (!a->workspace_has_states) {  // (a keep_states forward left the merged map there)
      MergeArgs m{};
      m.routes = at(a->workspace, lay.off_ys);
      m.routes_f32 = 1;
      m.routes_blocked = ss2d_routes_blocked(a->height, a->width) ? 1 : 0;  // as the scan stage wrote them
      m.x = u;
      m.x_f32 = (a->conv_w != nullptr || a->x_proj_w != nullptr);
      m.Dskip = a->Dskip;
      m.merged_f32 = merged;
      m.batch = a->batch;
      m.C = a->dim;
      m.H = a->height;
      m.W = a->width;
      m.dtype = a->dtype;
      if (launch_merge(m, stream) != hipSuccess) return SS2D_ERR_HIP;
    }
    LnArgs l{};
    l.M = merged;
    l.w = a->ln_w;
    l.b = a->ln_b;
    l.z = a->z;
    l.dout = a->dout;
    l.dM = dM;
    l.dz = a->dz;
    l.part = reinterpret_cast<float*>(at(a->workspace, lay.off_lnpart));
    l.dw = a->ln_w ? a->dln_w : nullptr;
    l.db = a->ln_b ? a->dln_b : nullptr;
    l.batch = a->batch;
    l.C = a->dim;
    l.L = L;
    l.eps = a->ln_eps;
    l.dtype = a->dtype;
    if (launch_ln_gate_bwd(l, stream) != hipSuccess || launch_ln_reduce(l, stream) != hipSuccess) return SS2D_ERR_HIP;
    if (launch_transpose(dM, at(a->workspace, lay.off_dMT), a->batch, a->dim, a->height, a->width, 4, stream) !=
        hipSuccess)
      return SS2D_ERR_HIP;
  } else {
    // gate (with the pre-gate merge it needs): dz, and dM = dout * silu(z) in grid and
    // transposed order
    MergeGateArgs gb{};
    gb.routes = reinterpret_cast<const float*>(at(a->workspace, lay.off_ys));
    gb.routes_blocked = ss2d_routes_blocked(a->height, a->width) ? 1 : 0;
    gb.x = u;
    gb.x_f32 = (a->conv_w != nullptr || a->x_proj_w != nullptr);
    gb.Dskip = a->Dskip;
    gb.z = a->z;
    gb.dout = a->dout;
    gb.dz = a->dz;
    gb.dM = reinterpret_cast<float*>(at(a->workspace, lay.off_dM));
    gb.dMT = reinterpret_cast<float*>(at(a->workspace, lay.off_dMT));
    gb.merged = reinterpret_cast<float*>(at(a->workspace, lay.off_merged));
    gb.merged_in = (a->workspace_has_states && a->z) ? 1 : 0;
    gb.batch = a->batch;
    gb.C = a->dim;
    gb.H = a->height;
    gb.W = a->width;
    gb.dtype = a->dtype;
    if (launch_merge_gate_bwd(gb, stream) != hipSuccess) return SS2D_ERR_HIP;
  }

  // adjoint scans of the four routes; du (fp32, route order) reuses the route-output region
  ScanBwdParams bp{};
  void* ws = a->workspace;
  bp.u = u;
  bp.uT = at(ws, lay.off_xT);
  bp.u_f32 = a->conv_w != nullptr && a->dtype != 0 && !proj;
  bp.delta = proj ? (fused_dt(a->dt_rank) ? nullptr : wsf(ws, lay.off_pdelta)) : a->delta;
  if (proj && fused_dt(a->dt_rank)) {
    bp.dt = wsf(ws, lay.off_pxdbl);
    bp.dt_w = a->dt_proj_w;
    bp.dt_rank = int(a->dt_rank);
  }
  bp.A = a->A;
  bp.Bm = proj ? wsf(ws, lay.off_pxdbl) + a->dt_rank * L : a->Bm;
  bp.Cm = proj ? wsf(ws, lay.off_pxdbl) + (a->dt_rank + a->dstate) * L : a->Cm;
  bp.bc_stride = proj ? (a->dt_rank + 2 * a->dstate) * L : 0;
  bp.Dskip = a->Dskip;
  bp.delta_bias = a->delta_bias;
  bp.dout = at(a->workspace, lay.off_dM);
  bp.doutT = at(a->workspace, lay.off_dMT);
  bp.du = at(a->workspace, lay.off_ys);
  bp.ddelta = proj ? wsf(ws, lay.off_pddelta) : a->ddelta;
  bp.batch = a->batch;
  bp.dim = 4 * a->dim;
  bp.L = L;
  bp.G = 4;
  bp.per_group = a->dim;
  bp.dblocks = lay.scan.dblocks;
  bp.N = int(a->dstate);
  bp.softplus = a->delta_softplus ? 1 : 0;
  bp.ss2d = 1;
  bp.dtype = proj ? SS2D_DTYPE_F32 : a->dtype;
  bp.vec = (L % 4 == 0) && vec_aligned(bp.dtype, {u, bp.delta, bp.Bm, bp.Cm, bp.ddelta});
  void* dB_out = proj ? static_cast<void*>(wsf(ws, lay.off_pdxdbl) + a->dt_rank * L) : a->dBm;
  void* dC_out = proj ? static_cast<void*>(wsf(ws, lay.off_pdxdbl) + (a->dt_rank + a->dstate) * L) : a->dCm;
  // whole-line stores of du (read back only by the dx merge below; the producer's backward reads
  // it row by row) and of the dB / dC partial sums (whose reduction stores 4 steps at once)
  const bool blocked = ss2d_routes_blocked(a->height, a->width);
  bp.du_blocked = (blocked && !proj) ? 1 : 0;
  bp.bc_blocked = (blocked && vec_aligned(bp.dtype, {dB_out, dC_out})) ? 1 : 0;
  st = run_scan_bwd(bp, lay.scan, at(ws, lay.off_scan), dB_out, dC_out, a->dA, a->Dskip ? a->dDskip : nullptr,
                    a->delta_bias ? a->ddelta_bias : nullptr, stream);
  if (st != SS2D_OK) return st;
  if (proj) {
    st = ss2d_project_bwd(a, lay, stream);
    if (st != SS2D_OK) return st;
  }

  // dx = cross-merge of the routes' du (with the input front: the gradient w.r.t. its output,
  // in fp32, which the front's backward turns into dx and the filter gradients)
  MergeArgs m{};
  m.routes = at(a->workspace, lay.off_ys);
  m.routes_f32 = 1;
  m.routes_blocked = bp.du_blocked;  // as the adjoint scans wrote du
  m.batch = a->batch;
  m.C = a->dim;
  m.H = a->height;
  m.W = a->width;
  m.dtype = a->dtype;
  if (!a->conv_w) {
    m.y = a->dx;
    return status_from(launch_merge(m, stream));
  }
  float* dxc = reinterpret_cast<float*>(at(a->workspace, lay.off_merged));
  m.merged_f32 = dxc;
  if (launch_merge(m, stream) != hipSuccess) return SS2D_ERR_HIP;
  FrontArgs fr{};
  fr.x = a->x;
  fr.w = a->conv_w;
  fr.bias = a->conv_b;
  fr.dxc = dxc;
  fr.dx = a->dx;
  fr.part = reinterpret_cast<float*>(at(a->workspace, lay.off_cpart));
  fr.dw = a->dconv_w;
  fr.dbias = a->conv_b ? a->dconv_b : nullptr;
  fr.batch = a->batch;
  fr.C = a->dim;
  fr.H = a->height;
  fr.W = a->width;
  fr.k = a->conv_k;
  fr.dtype = a->dtype;
  if (launch_front_bwd(fr, stream) != hipSuccess) return SS2D_ERR_HIP;
  return status_from(launch_front_reduce(fr, stream));
}

// ---- Bidirectional (Vision Mamba) scan --------------------------------------------------
// The two directions are the two groups of one generic scan over rows (b, k*D + d): the
// direction-major layouts of u, delta, B, C, A, D and delta_bias are exactly that scan's
// (batch, 2D, L), (batch, 2, N, L), (2D, N) and (2D) layouts.
struct VimLayout {
  ScanLayout scan;
  int64_t off_scan, off_ys, off_dy, total;
};

static VimLayout vim_layout(int64_t batch, int64_t dim, int64_t L, int64_t dstate, int dtype) {
  VimLayout l{};
  l.scan = scan_layout(batch, 2 * dim, dstate, L, 2, dtype);
  int64_t o = 0;
  l.off_scan = o; o += align_up(l.scan.total);
  l.off_ys = o;   o += align_up(batch * 2 * dim * L * 4);              // fp32 direction outputs, own order
  l.off_dy = o;   o += align_up(batch * 2 * dim * L * 4);              // fp32 gradient reaching them
  l.total = o;
  return l;
}

static int check_vim(int64_t batch, int64_t dim, int64_t L, int64_t dstate, int dtype) {
  if (!dtype_ok(dtype)) return SS2D_ERR_UNSUPPORTED;
  if (batch < 0 || dim < 0 || L < 0) return SS2D_ERR_INVALID_ARGUMENT;
  if (dstate < 1 || dstate > 64) return SS2D_ERR_UNSUPPORTED;
  if (cdiv(batch * dim * L, 256) > kMaxBlocks) return SS2D_ERR_INVALID_ARGUMENT;
  return SS2D_OK;
}

size_t vim_bidir_workspace_bytes(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int dtype) {
  if (check_vim(batch, dim, seqlen, dstate, dtype) != SS2D_OK) return 0;
  return size_t(vim_layout(batch, dim, seqlen, dstate, dtype).total);
}

static int validate_vim_fwd(const vim_bidir_fwd_args* a, VimLayout* lay, bool* empty) {
  *empty = false;
  if (!a) return SS2D_ERR_INVALID_ARGUMENT;
  int st = check_vim(a->batch, a->dim, a->seqlen, a->dstate, a->dtype);
  if (st != SS2D_OK) return st;
  if (a->batch * a->dim * a->seqlen == 0) {
    *empty = true;
    return SS2D_OK;
  }
  if (!a->u || !a->delta || !a->A || !a->Bm || !a->Cm || !a->out || !a->workspace) return SS2D_ERR_INVALID_ARGUMENT;
  if (!elem_aligned(a->dtype, {a->u, a->delta, a->Bm, a->Cm, a->z, a->out})) return SS2D_ERR_INVALID_ARGUMENT;
  if (!aligned(a->A, 4) || (a->Dskip && !aligned(a->Dskip, 4)) || (a->delta_bias && !aligned(a->delta_bias, 4)))
    return SS2D_ERR_INVALID_ARGUMENT;
  *lay = vim_layout(a->batch, a->dim, a->seqlen, a->dstate, a->dtype);
  if (a->workspace_bytes < size_t(lay->total) || !aligned(a->workspace, kAlign)) return SS2D_ERR_INVALID_ARGUMENT;
  return SS2D_OK;
}

// the two direction scans as one generic scan, outputs into the workspace
static ss_fwd_args vim_scan_args(const void* u, const void* delta, const float* A, const void* Bm, const void* Cm,
                                 const float* Dskip, const float* delta_bias, void* ws, const VimLayout& lay,
                                 int64_t batch, int64_t dim, int64_t L, int64_t dstate, int dtype, int softplus) {
  ss_fwd_args f{};
  f.u = u;
  f.delta = delta;
  f.A = A;
  f.Bm = Bm;
  f.Cm = Cm;
  f.Dskip = Dskip;
  f.z = nullptr;
  f.delta_bias = delta_bias;
  f.out = at(ws, lay.off_ys);
  f.workspace = at(ws, lay.off_scan);
  f.workspace_bytes = size_t(lay.scan.total);
  f.batch = batch;
  f.dim = 2 * dim;
  f.dstate = dstate;
  f.seqlen = L;
  f.ngroups = 2;
  f.dtype = dtype;
  f.delta_softplus = softplus;
  return f;
}

static int vim_merge_stage(const vim_bidir_fwd_args* a, const VimLayout& lay, hipStream_t stream) {
  BidirArgs m{};
  m.ys = reinterpret_cast<const float*>(at(a->workspace, lay.off_ys));
  m.z = a->z;
  m.out = a->out;
  m.batch = a->batch;
  m.C = a->dim;
  m.L = a->seqlen;
  m.dtype = a->dtype;
  return status_from(launch_bidir_merge(m, stream));
}

static int vim_scan_stage(const vim_bidir_fwd_args* a, const VimLayout& lay, hipStream_t stream) {
  const ss_fwd_args f = vim_scan_args(a->u, a->delta, a->A, a->Bm, a->Cm, a->Dskip, a->delta_bias, a->workspace, lay,
                                      a->batch, a->dim, a->seqlen, a->dstate, a->dtype, a->delta_softplus);
  return scan_fwd_impl(&f, a->keep_states != 0, stream, true);
}

int vim_bidir_fwd(const vim_bidir_fwd_args* a, hipStream_t stream) {
  VimLayout lay;
  bool empty;
  int st = validate_vim_fwd(a, &lay, &empty);
  if (st != SS2D_OK || empty) return st;
  st = vim_scan_stage(a, lay, stream);
  if (st == SS2D_OK) st = vim_merge_stage(a, lay, stream);
  return st;
}

int vim_bidir_fwd_stage(const vim_bidir_fwd_args* a, int stage, hipStream_t stream) {
  if (stage != SS2D_STAGE_TRANSPOSE && stage != SS2D_STAGE_SCAN && stage != SS2D_STAGE_MERGE)
    return SS2D_ERR_INVALID_ARGUMENT;
  VimLayout lay;
  bool empty;
  int st = validate_vim_fwd(a, &lay, &empty);
  if (st != SS2D_OK || empty || stage == SS2D_STAGE_TRANSPOSE) return st;
  return stage == SS2D_STAGE_SCAN ? vim_scan_stage(a, lay, stream) : vim_merge_stage(a, lay, stream);
}

int vim_bidir_bwd(const vim_bidir_bwd_args* a, hipStream_t stream) {
  if (!a) return SS2D_ERR_INVALID_ARGUMENT;
  int st = check_vim(a->batch, a->dim, a->seqlen, a->dstate, a->dtype);
  if (st != SS2D_OK) return st;
  if ((a->Dskip && !a->dDskip) || (a->delta_bias && !a->ddelta_bias) || (a->z && !a->dz))
    return SS2D_ERR_INVALID_ARGUMENT;
  if (a->dim == 0) return SS2D_OK;
  if (!a->dA) return SS2D_ERR_INVALID_ARGUMENT;
  if (a->batch == 0 || a->seqlen == 0)
    return zero_param_grads(a->dA, a->Dskip ? a->dDskip : nullptr, a->delta_bias ? a->ddelta_bias : nullptr,
                            2 * a->dim, a->dstate, stream);
  if (!a->u || !a->delta || !a->A || !a->Bm || !a->Cm || !a->dout || !a->du || !a->ddelta || !a->dBm || !a->dCm ||
      !a->workspace)
    return SS2D_ERR_INVALID_ARGUMENT;
  if (!elem_aligned(a->dtype, {a->u, a->delta, a->Bm, a->Cm, a->z, a->dout, a->du, a->ddelta, a->dBm, a->dCm, a->dz}))
    return SS2D_ERR_INVALID_ARGUMENT;
  if (!aligned(a->A, 4) || !aligned(a->dA, 4) || (a->Dskip && !aligned(a->Dskip, 4)) ||
      (a->delta_bias && !aligned(a->delta_bias, 4)) || (a->dDskip && !aligned(a->dDskip, 4)) ||
      (a->ddelta_bias && !aligned(a->ddelta_bias, 4)))
    return SS2D_ERR_INVALID_ARGUMENT;
  const VimLayout lay = vim_layout(a->batch, a->dim, a->seqlen, a->dstate, a->dtype);
  if (a->workspace_bytes < size_t(lay.total) || !aligned(a->workspace, kAlign)) return SS2D_ERR_INVALID_ARGUMENT;
  if (a->batch * 2 * lay.scan.dblocks * lay.scan.bwd_n_chunks > kMaxBlocks) return SS2D_ERR_INVALID_ARGUMENT;
  const int64_t L = a->seqlen;

  // forward again, unless a training forward left them: direction outputs and checkpoint states
  if (!a->workspace_has_states) {
    const ss_fwd_args f = vim_scan_args(a->u, a->delta, a->A, a->Bm, a->Cm, a->Dskip, a->delta_bias, a->workspace,
                                        lay, a->batch, a->dim, L, a->dstate, a->dtype, a->delta_softplus);
    st = scan_fwd_impl(&f, true, stream, true);
    if (st != SS2D_OK) return st;
  }

  // gate: dz, and the fp32 gradient reaching each direction in its own order
  BidirArgs g{};
  g.ys = reinterpret_cast<const float*>(at(a->workspace, lay.off_ys));
  g.z = a->z;
  g.dout = a->dout;
  g.dy = reinterpret_cast<float*>(at(a->workspace, lay.off_dy));
  g.dz = a->dz;
  g.batch = a->batch;
  g.C = a->dim;
  g.L = L;
  g.dtype = a->dtype;
  if (launch_bidir_gate_bwd(g, stream) != hipSuccess) return SS2D_ERR_HIP;

  // adjoint scans of the two directions
  ScanBwdParams bp{};
  bp.u = a->u;
  bp.delta = a->delta;
  bp.A = a->A;
  bp.Bm = a->Bm;
  bp.Cm = a->Cm;
  bp.Dskip = a->Dskip;
  bp.delta_bias = a->delta_bias;
  bp.dout = g.dy;
  bp.dout_f32 = 1;
  bp.du = a->du;
  bp.ddelta = a->ddelta;
  bp.batch = a->batch;
  bp.dim = 2 * a->dim;
  bp.L = L;
  bp.G = 2;
  bp.per_group = lay.scan.per_group;
  bp.dblocks = lay.scan.dblocks;
  bp.N = int(a->dstate);
  bp.softplus = a->delta_softplus ? 1 : 0;
  bp.ss2d = 0;
  bp.dtype = a->dtype;
  bp.vec = (L % 4 == 0) && vec_aligned(a->dtype, {a->u, a->delta, a->Bm, a->Cm, a->du, a->ddelta});
  return run_scan_bwd(bp, lay.scan, at(a->workspace, lay.off_scan), a->dBm, a->dCm, a->dA,
                      a->Dskip ? a->dDskip : nullptr, a->delta_bias ? a->ddelta_bias : nullptr, stream);
}

}  // extern "C"
