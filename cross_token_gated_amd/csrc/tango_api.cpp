// tango_api.cpp - the C ABI of include/tango.h: validation, workspace layout,
// launch order and error reporting.  No memory is allocated here; every
// kernel runs on the caller's stream.
#include "../../include/tango.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "kernels.hpp"

// Scratch of wango_decode_step_noalloc: one array per device, in the code
// object, held until the process ends.  On the host, `scratch` names a host
// stand-in, not the device array: its device address comes from
// hipGetSymbolAddress in ensure_init (with the device current), and only that
// address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[TANGO_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace tango;

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return TANGO_OK;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(TANGO_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

int64_t pad_rows(int64_t T) { return (T + kRowPad - 1) / kRowPad * kRowPad; }

size_t elem_size(int dtype) { return dtype == TANGO_BF16 ? 2 : 4; }

// Gate columns per head, and padded: the packed gates (and the WANGO read-out
// n_old) hold head a's column c at a * head_pad + c, the pad columns zero, so
// every kernel that walks one head's columns works on whole 64-column blocks.
// A head width that is already a multiple of 64 is not padded.  Otherwise
// WANGO pads to a multiple of 64 (its scan and band kernels pay for every
// column), TANGO to a multiple of 512 when that adds at most a fifth (the
// aggregation then runs its widest tiles: at 16 heads of 1,780 columns, 2.76 ms
// on 2,048 columns against 3.49 ms on 1,792), else to 64.
// (v and gbar are never padded.)
int head_width(const tango_shape_t* s) { return s->d_gate / s->n_heads; }
int head_pad(const tango_shape_t* s, bool wango) {
  const int fh = head_width(s);
  if (fh % 64 == 0) return fh;
  const int p512 = (fh + 511) / 512 * 512;
  if (!wango && 5 * p512 <= 6 * fh) return p512;
  return (fh + 63) / 64 * 64;
}
int64_t gate_pad(const tango_shape_t* s, bool wango) { return (int64_t)s->n_heads * head_pad(s, wango); }
// Operand parts of the projection and output GEMMs' activation operand.
int op_parts(const tango_shape_t* s) { return s->dtype == TANGO_BF16 && s->operand_parts == 2 ? 2 : 1; }
// Bytes of one element of v: bf16 with one bf16 operand part, else float32.
size_t v_elem(const tango_shape_t* s) { return s->dtype == TANGO_BF16 && op_parts(s) == 1 ? 2 : 4; }

// ---- validation -----------------------------------------------------------

int check_shape(const tango_shape_t* s) {
  if (!s) return fail(TANGO_ERR_NULL, "shape is NULL");
  if (s->dtype != TANGO_F32 && s->dtype != TANGO_BF16)
    return fail(TANGO_ERR_DTYPE, "dtype %d is neither TANGO_F32 (0) nor TANGO_BF16 (1)", s->dtype);
  if (s->io_dtype != TANGO_F32 && s->io_dtype != TANGO_BF16)
    return fail(TANGO_ERR_DTYPE, "io_dtype %d is neither TANGO_F32 (0) nor TANGO_BF16 (1)", s->io_dtype);
  if (s->batch < 1 || s->seq_len < 1 || s->d_model < 1 || s->d_gate < 1 || s->n_heads < 1 ||
      s->head_dim < 1)
    return fail(TANGO_ERR_SHAPE, "sizes must be >= 1 (B=%d T=%d d=%d F=%d H=%d d_h=%d)", s->batch,
                s->seq_len, s->d_model, s->d_gate, s->n_heads, s->head_dim);
  if (s->d_gate % s->n_heads != 0)
    return fail(TANGO_ERR_SHAPE, "d_gate %d is not a multiple of n_heads %d", s->d_gate, s->n_heads);
  if (!(s->rms_eps > 0.f) || !std::isfinite(s->rms_eps))
    return fail(TANGO_ERR_SHAPE, "rms_eps must be finite and > 0");
  if (!(s->rope_base >= 0.f) || !std::isfinite(s->rope_base))
    return fail(TANGO_ERR_SHAPE, "rope_base must be finite and >= 0");
  if (s->operand_parts < 0 || s->operand_parts > 2 || (s->operand_parts == 2 && s->dtype != TANGO_BF16))
    return fail(TANGO_ERR_SHAPE, "operand_parts %d: need 0 or 1, or 2 with dtype TANGO_BF16", s->operand_parts);
  if ((int64_t)s->batch * pad_rows(s->seq_len) > ((int64_t)1 << 26))
    return fail(TANGO_ERR_UNSUPPORTED, "batch * padded seq_len exceeds 2^26 rows");
  if (s->d_model % 128 != 0 || s->d_model > 4096)
    return fail(TANGO_ERR_UNSUPPORTED, "d_model %d: need a multiple of 128, at most 4096", s->d_model);
  if (s->d_gate % 64 != 0 || (s->d_gate / s->n_heads) % 4 != 0)
    return fail(TANGO_ERR_UNSUPPORTED, "d_gate %d: need d_gate a multiple of 64 and d_gate/n_heads of 4",
                s->d_gate);
  if (s->head_dim != 32 && s->head_dim != 64 && s->head_dim != 128)
    return fail(TANGO_ERR_UNSUPPORTED, "head_dim %d: supported are 32, 64 and 128", s->head_dim);
  if ((int64_t)s->n_heads * s->head_dim > 1024)
    return fail(TANGO_ERR_UNSUPPORTED, "n_heads * head_dim exceeds 1024");
  return TANGO_OK;
}

int check_wango(const tango_shape_t* s, int32_t window, int32_t phi_dim, int32_t chunk) {
  if (window < 1) return fail(TANGO_ERR_SHAPE, "window %d < 1", window);
  if (phi_dim != s->head_dim)
    return fail(TANGO_ERR_SHAPE, "phi_dim %d must equal head_dim %d (phi acts elementwise)", phi_dim,
                s->head_dim);
  if (chunk != 64 && chunk != 128)
    return fail(TANGO_ERR_UNSUPPORTED, "chunk %d: supported are 64 and 128", chunk);
  if (window % chunk != 0)
    return fail(TANGO_ERR_UNSUPPORTED, "window %d is not a multiple of chunk %d", window, chunk);
  return TANGO_OK;
}

bool aligned(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Range {
  const void* p;
  size_t n;
  const char* name;
};

bool overlap(const Range& a, const Range& b) {
  if (!a.p || !b.p || !a.n || !b.n) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

// Each output must not overlap any input or other output; out may equal x
// exactly (in place).
int check_ranges(const Range* ins, int nin, const Range* outs, int nout, const void* inplace_x,
                 const void* inplace_out) {
  for (int i = 0; i < nin; ++i)
    if (ins[i].p && !aligned(ins[i].p)) return fail(TANGO_ERR_ALIGN, "%s is not 16-byte aligned", ins[i].name);
  for (int o = 0; o < nout; ++o)
    if (outs[o].p && !aligned(outs[o].p))
      return fail(TANGO_ERR_ALIGN, "%s is not 16-byte aligned", outs[o].name);
  for (int o = 0; o < nout; ++o) {
    for (int i = 0; i < nin; ++i) {
      // the one permitted overlap: out == x exactly (in place)
      if (inplace_out && outs[o].p == inplace_out && ins[i].p == inplace_x && inplace_x == inplace_out &&
          outs[o].n == ins[i].n)
        continue;
      if (overlap(outs[o], ins[i]))
        return fail(TANGO_ERR_ALIAS, "%s overlaps %s", outs[o].name, ins[i].name);
    }
    for (int o2 = o + 1; o2 < nout; ++o2)
      if (overlap(outs[o], outs[o2]))
        return fail(TANGO_ERR_ALIAS, "%s overlaps %s", outs[o].name, outs[o2].name);
  }
  return TANGO_OK;
}

// ---- workspace layout -------------------------------------------------------

struct Layout {
  size_t gp, v, qh, kh, gbar;           // offsets
  size_t xs, rinv;                      // projection input parts, RMSNorm scales
  size_t fq, fk;                        // WANGO features
  size_t part, part_den, counters;      // TANGO split scratch
  size_t states, zstates, seg_state, seg_z;   // WANGO chunk states, segment sums
  size_t total;
  AggPlan agg;
  ScanPlan scan;
};

// Bytes of the WANGO chunk states the scan leaves for the band's read-out
// (ScanArgs::states; with z: ScanArgs::zstates).
size_t wango_states_bytes(const tango_shape_t* s, int32_t chunk, bool z) {
  const int64_t nch = pad_rows(s->seq_len) / chunk;
  const int64_t per = z ? 1 : gate_pad(s, true) / s->n_heads / 16;
  return (size_t)s->batch * s->n_heads * nch * per * (s->head_dim / 32) * 64 * 8 * elem_size(s->dtype);
}

Layout make_layout(const tango_shape_t* s, bool wango, int32_t window, int32_t chunk) {
  Layout L{};
  const size_t es = elem_size(s->dtype);
  const int64_t M = (int64_t)s->batch * pad_rows(s->seq_len);
  const int64_t F = gate_pad(s, wango), HD = (int64_t)s->n_heads * s->head_dim;   // padded gate width
  const int64_t Fv = s->d_gate;                                              // v, gbar: not padded
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L.gp = take(M * F * es);
  L.v = take(M * Fv * v_elem(s));
  L.qh = take(M * HD * es);
  L.kh = take(M * HD * es);
  L.gbar = take(M * Fv * es);
  const bool bf = s->dtype == TANGO_BF16;
  L.xs = take(proj_parts_bytes(M, s->d_model, bf, op_parts(s)));
  L.rinv = take(M * sizeof(float));
  if (!wango) {
    L.agg = tango_agg_plan(s->batch, (int)pad_rows(s->seq_len), (int)F, s->n_heads, s->head_dim, bf);
    const int64_t n = L.agg.n_split_tiles;
    L.part = take((size_t)n * 2 * L.agg.br * L.agg.fs * sizeof(float));
    L.part_den = take((size_t)n * 2 * L.agg.br * sizeof(float));
    L.counters = take((size_t)n * sizeof(int));
  } else {
    (void)window;
    L.scan = wango_scan_plan(s->batch, (int)pad_rows(s->seq_len), (int)F, s->n_heads, chunk);
    L.fq = take(M * HD * es);
    L.fk = take(M * HD * es);
    L.states = take(wango_states_bytes(s, chunk, false));
    L.zstates = take(wango_states_bytes(s, chunk, true));
    const int64_t bh = (int64_t)s->batch * s->n_heads;
    L.seg_state = take((size_t)bh * L.scan.nseg * s->head_dim * (F / s->n_heads) * sizeof(float));
    L.seg_z = take((size_t)bh * L.scan.nseg * s->head_dim * sizeof(float));
  }
  L.total = off;
  return L;
}

// ---- one-time set-up (per device) -----------------------------------------------

std::mutex g_init_mu;
bool g_init_done[64];
void* g_scratch[64];   // device address of `scratch` on each device

int ensure_init() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(TANGO_ERR_HIP, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_init_mu);
  if (g_init_done[dev]) return TANGO_OK;
  if ((e = gemm_kernels_init()) != hipSuccess) return hip_fail(e, "kernel attributes");
  void* ptr = nullptr;
  if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess)
    return hip_fail(e, "hipGetSymbolAddress(scratch)");
  if (!ptr || ((uintptr_t)ptr & 255u) != 0)
    return fail(TANGO_ERR_HIP, "the scratch array of device %d is not 256-byte aligned", dev);
  g_scratch[dev] = ptr;
  g_init_done[dev] = true;
  return TANGO_OK;
}

// The current device's scratch array (after ensure_init), or NULL.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(g_init_mu);
  return g_init_done[dev] ? g_scratch[dev] : nullptr;
}

// ---- argument blocks ------------------------------------------------------------

ProjArgs proj_args(const tango_shape_t* s, const tango_weights_t* w, const void* x, void* gp, void* v,
                   void* qh, void* kh, bool wango) {
  ProjArgs a{};
  a.x = x;
  a.w_g = w->w_g;
  a.w_v = w->w_v;
  a.w_q = w->w_q;
  a.w_k = w->w_k;
  a.gain = w->rms_gain;
  a.theta = w->theta;
  a.gp = gp;
  a.v = v;
  a.qh = qh;
  a.kh = kh;
  a.B = s->batch;
  a.T = s->seq_len;
  a.Tp = (int)pad_rows(s->seq_len);
  a.d = s->d_model;
  a.F = s->d_gate;
  a.Fh = head_width(s);
  a.Fhp = head_pad(s, wango);
  a.Fp = (int)gate_pad(s, wango);
  a.HD = s->n_heads * s->head_dim;
  a.dh = s->head_dim;
  a.rope_base = s->rope_base;
  a.eps = s->rms_eps;
  a.parts = op_parts(s);
  return a;
}

OutArgs out_args(const tango_shape_t* s, const void* w_o, const void* x, const void* gbar, const void* v,
                 void* out) {
  OutArgs a{};
  a.x = x;
  a.w_o = w_o;
  a.gbar = gbar;
  a.v = v;
  a.out = out;
  a.B = s->batch;
  a.T = s->seq_len;
  a.Tp = (int)pad_rows(s->seq_len);
  a.d = s->d_model;
  a.F = s->d_gate;
  a.parts = op_parts(s);
  return a;
}

AggArgs agg_args(const tango_shape_t* s, const float* theta, const float* null_bias, const void* qh,
                 const void* kh, const void* gp, void* gbar, bool wango) {
  AggArgs a{};
  a.qh = qh;
  a.kh = kh;
  a.gp = gp;
  a.gbar = gbar;
  a.theta = theta;
  a.null_bias = null_bias;
  a.B = s->batch;
  a.T = s->seq_len;
  a.Tp = (int)pad_rows(s->seq_len);
  a.F = (int)gate_pad(s, wango);   // the kernels walk the head-padded gate columns
  a.Fo = s->d_gate;         // gbar is not padded
  a.Fho = head_width(s);
  a.H = s->n_heads;
  a.dh = s->head_dim;
  return a;
}

ScanArgs scan_args(const tango_shape_t* s, int32_t window, int32_t chunk, const void* fq,
                   const void* fk, const void* gp, float* n_old, float* z_old, float* seg_state,
                   float* seg_z) {
  ScanArgs a{};
  a.fq = fq;
  a.fk = fk;
  a.gp = gp;
  a.n_old = n_old;
  a.z_old = z_old;
  a.seg_state = seg_state;
  a.seg_z = seg_z;
  a.B = s->batch;
  a.T = s->seq_len;
  a.Tp = (int)pad_rows(s->seq_len);
  a.F = (int)gate_pad(s, true);
  a.H = s->n_heads;
  a.dh = s->head_dim;
  a.window = window;
  a.chunk = chunk;
  return a;
}

int check_weights(const tango_weights_t* w, bool need_all) {
  if (!w) return fail(TANGO_ERR_NULL, "weights is NULL");
  if (need_all && (!w->w_g || !w->w_v || !w->w_q || !w->w_k || !w->w_o))
    return fail(TANGO_ERR_NULL, "a weight matrix pointer is NULL");
  if (!w->theta) return fail(TANGO_ERR_NULL, "theta is NULL");
  return TANGO_OK;
}

template <typename Fn>
int guarded(Fn fn) {
  try {
    return fn();
  } catch (...) {
    return fail(TANGO_ERR_HIP, "unexpected C++ exception inside the library");
  }
}

// Scratch of the projection stage calls: input parts at offset 0, then the
// row scales.
struct ProjScratch {
  size_t rinv, total;
};
ProjScratch proj_scratch(const tango_shape_t* s) {
  const int64_t M = (int64_t)s->batch * pad_rows(s->seq_len);
  ProjScratch p{};
  p.rinv = align256(proj_parts_bytes(M, s->d_model, s->dtype == TANGO_BF16, op_parts(s)));
  p.total = p.rinv + M * sizeof(float);
  return p;
}

// Projection stage (fq, fk non-null: the WANGO features too).
int stage_proj_common(const tango_shape_t* s, const tango_weights_t* weights, const void* x, void* gp,
                      void* v, void* qh, void* kh, void* fq, void* fk, void* ws, size_t ws_bytes,
                      void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if ((rc = check_weights(weights, true))) return rc;
  if (!x || !gp || !v || !qh || !kh || !ws) return fail(TANGO_ERR_NULL, "a buffer pointer is NULL");
  const ProjScratch ps = proj_scratch(s);
  if (ws_bytes < ps.total)
    return fail(TANGO_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes,
                ps.total);
  const bool wango = fq != nullptr;
  const size_t es = elem_size(s->dtype), M = (size_t)s->batch * pad_rows(s->seq_len);
  const size_t d = s->d_model, F = s->d_gate, HD = (size_t)s->n_heads * s->head_dim;
  const Range ins[] = {{x, (size_t)s->batch * s->seq_len * d * elem_size(s->io_dtype), "x"},
                       {weights->w_g, F * d * es, "w_g"},
                       {weights->w_v, F * d * es, "w_v"},
                       {weights->w_q, HD * d * es, "w_q"},
                       {weights->w_k, HD * d * es, "w_k"},
                       {weights->rms_gain, d * es, "rms_gain"},
                       {wango ? weights->theta : nullptr, s->n_heads * sizeof(float), "theta"}};
  const size_t Fp = gate_pad(s, wango);
  const Range outs[] = {{gp, M * Fp * es, "gp"}, {v, M * F * v_elem(s), "v"}, {qh, M * HD * es, "qh"},
                        {kh, M * HD * es, "kh"}, {ws, ps.total, "workspace"},
                        {fq, M * HD * es, "fq"}, {fk, M * HD * es, "fk"}};
  if ((rc = check_ranges(ins, 7, outs, wango ? 7 : 5, nullptr, nullptr))) return rc;
  if ((rc = ensure_init())) return rc;
  hipError_t ez = launch_zero_pad(gp, (int64_t)M, s->n_heads, head_width(s), head_pad(s, wango),
                                  s->dtype == TANGO_BF16, static_cast<hipStream_t>(stream));
  if (ez != hipSuccess) return hip_fail(ez, "pad-column fill");
  ProjArgs pa = proj_args(s, weights, x, gp, v, qh, kh, wango);
  pa.xs = ws;
  pa.rinv = reinterpret_cast<float*>(static_cast<char*>(ws) + ps.rinv);
  pa.fq = fq;
  pa.fk = fk;
  hipError_t e = launch_proj(pa, s->dtype == TANGO_BF16, s->io_dtype == TANGO_BF16,
                             static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "projection kernel");
}

int block_common(const tango_shape_t* s, const tango_weights_t* w, bool wango, int32_t window,
                 int32_t phi_dim, int32_t chunk, const void* x, void* out, void* ws, size_t ws_bytes,
                 void* stream, bool check_only = false) {
  int rc = check_shape(s);
  if (rc) return rc;
  if ((rc = check_weights(w, true))) return rc;
  if (wango && (rc = check_wango(s, window, phi_dim, chunk))) return rc;
  if (!x || !out) return fail(TANGO_ERR_NULL, "x or out is NULL");
  if (!ws) return fail(TANGO_ERR_NULL, "workspace is NULL");
  const Layout L = make_layout(s, wango, window, chunk);
  if (ws_bytes < L.total)
    return fail(TANGO_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes,
                L.total);
  const size_t es = elem_size(s->dtype);
  const size_t d = s->d_model, F = s->d_gate, HD = (size_t)s->n_heads * s->head_dim;
  const size_t xb = (size_t)s->batch * s->seq_len * d * elem_size(s->io_dtype);
  const Range ins[] = {{x, xb, "x"},
                       {w->w_g, F * d * es, "w_g"},
                       {w->w_v, F * d * es, "w_v"},
                       {w->w_q, HD * d * es, "w_q"},
                       {w->w_k, HD * d * es, "w_k"},
                       {w->w_o, d * F * es, "w_o"},
                       {w->rms_gain, d * es, "rms_gain"},
                       {w->theta, s->n_heads * sizeof(float), "theta"},
                       {w->null_bias, s->n_heads * sizeof(float), "null_bias"}};
  const Range outs[] = {{out, xb, "out"}, {ws, L.total, "workspace"}};
  if ((rc = check_ranges(ins, 9, outs, 2, x, out))) return rc;
  if (check_only) return ok();
  if ((rc = ensure_init())) return rc;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf = s->dtype == TANGO_BF16;
  char* base = static_cast<char*>(ws);
  void* gp = base + L.gp;
  void* v = base + L.v;
  void* qh = base + L.qh;
  void* kh = base + L.kh;
  void* gbar = base + L.gbar;
  const bool io_bf = s->io_dtype == TANGO_BF16;
  ProjArgs pa = proj_args(s, w, x, gp, v, qh, kh, wango);
  pa.xs = base + L.xs;
  pa.rinv = reinterpret_cast<float*>(base + L.rinv);
  if (wango) {
    pa.fq = base + L.fq;
    pa.fk = base + L.fk;
  } else if (L.agg.split) {
    pa.zero = reinterpret_cast<int*>(base + L.counters);
    pa.zero_n = L.agg.n_split_tiles;
  }
  hipError_t e = launch_zero_pad(gp, (int64_t)s->batch * pad_rows(s->seq_len), s->n_heads, head_width(s),
                                 head_pad(s, wango), bf, st);
  if (e != hipSuccess) return hip_fail(e, "pad-column fill");
  e = launch_proj(pa, bf, io_bf, st);
  if (e != hipSuccess) return hip_fail(e, "projection kernel");
  AggArgs aa = agg_args(s, w->theta, w->null_bias, qh, kh, gp, gbar, wango);
  if (!wango) {
    aa.part = reinterpret_cast<float*>(base + L.part);
    aa.part_den = reinterpret_cast<float*>(base + L.part_den);
    aa.counters = reinterpret_cast<int*>(base + L.counters);
    e = launch_tango_agg(aa, L.agg, bf, true, st);
    if (e != hipSuccess) return hip_fail(e, "aggregation kernel");
  } else {
    // the scan leaves the chunk states, the band reads them out
    ScanArgs sa = scan_args(s, window, chunk, base + L.fq, base + L.fk, gp, nullptr, nullptr,
                            reinterpret_cast<float*>(base + L.seg_state),
                            reinterpret_cast<float*>(base + L.seg_z));
    sa.states = base + L.states;
    sa.zstates = base + L.zstates;
    e = launch_wango_scan(sa, L.scan, bf, st);
    if (e != hipSuccess) return hip_fail(e, "scan kernels");
    aa.states = base + L.states;
    aa.zstates = base + L.zstates;
    aa.fq = base + L.fq;
    aa.window = window;
    aa.chunk = chunk;
    e = launch_wango_band(aa, bf, st);
    if (e != hipSuccess) return hip_fail(e, "band kernel");
  }
  e = launch_out(out_args(s, w->w_o, x, gbar, v, out), bf, io_bf, st);
  if (e != hipSuccess) return hip_fail(e, "output kernel");
  return ok();
}

}  // namespace

extern "C" {

size_t tango_workspace_size(const tango_shape_t* shape) {
  if (check_shape(shape)) return 0;
  return make_layout(shape, false, 0, 0).total;
}

size_t wango_workspace_size(const tango_shape_t* shape, int32_t window, int32_t phi_dim, int32_t chunk) {
  if (check_shape(shape) || check_wango(shape, window, phi_dim, chunk)) return 0;
  return make_layout(shape, true, window, chunk).total;
}

int tango_block_fwd(const tango_shape_t* shape, const tango_weights_t* weights, const void* x, void* out,
                    void* workspace, size_t workspace_bytes, void* hip_stream) {
  return guarded([&] {
    return block_common(shape, weights, false, 0, 0, 0, x, out, workspace, workspace_bytes, hip_stream);
  });
}

size_t tango_stack_workspace_size(const tango_shape_t* shapes, int32_t n_sets) {
  if (!shapes || n_sets < 1) return 0;
  size_t need = 0;
  for (int32_t k = 0; k < n_sets; ++k) {
    if (check_shape(&shapes[k])) return 0;
    need = std::max(need, make_layout(&shapes[k], false, 0, 0).total);
  }
  return need;
}

int tango_stack_fwd(const tango_shape_t* shapes, const tango_weights_t* sets, int32_t n_sets,
                    const int32_t* schedule, int32_t n_apps, const void* x, void* out, void* workspace,
                    size_t workspace_bytes, void* hip_stream) {
  return guarded([&]() -> int {
    if (!shapes || !sets || !schedule) return fail(TANGO_ERR_NULL, "shapes, sets or schedule is NULL");
    if (n_sets < 1 || n_apps < 1)
      return fail(TANGO_ERR_SHAPE, "n_sets %d and n_apps %d must be >= 1", n_sets, n_apps);
    // everything is checked before the first launch
    size_t need = 0;
    for (int32_t k = 0; k < n_sets; ++k) {
      const tango_shape_t& a = shapes[k];
      int rc = check_shape(&a);
      if (rc) return rc;
      if ((rc = check_weights(&sets[k], true))) return rc;
      const tango_shape_t& z = shapes[0];
      if (a.batch != z.batch || a.seq_len != z.seq_len || a.d_model != z.d_model || a.dtype != z.dtype ||
          a.io_dtype != z.io_dtype)
        return fail(TANGO_ERR_SHAPE, "set %d: batch, seq_len, d_model, dtype and io_dtype must match set 0",
                    k);
      need = std::max(need, make_layout(&a, false, 0, 0).total);
    }
    for (int32_t r = 0; r < n_apps; ++r)
      if (schedule[r] < 0 || schedule[r] >= n_sets)
        return fail(TANGO_ERR_SHAPE, "schedule[%d] = %d is not a set index below %d", r, schedule[r], n_sets);
    if (!x || !out) return fail(TANGO_ERR_NULL, "x or out is NULL");
    if (!workspace) return fail(TANGO_ERR_NULL, "workspace is NULL");
    if (workspace_bytes < need)
      return fail(TANGO_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                  workspace_bytes, need);
    for (int pass = 0; pass < 2; ++pass)   // pass 0 checks every call, pass 1 launches
      for (int32_t r = 0; r < n_apps; ++r) {
        const int32_t k = schedule[r];
        const int rc = block_common(&shapes[k], &sets[k], false, 0, 0, 0, r == 0 ? x : out, out, workspace,
                                    workspace_bytes, hip_stream, pass == 0);
        if (rc) return rc;
      }
    return ok();
  });
}

int wango_block_fwd(const tango_shape_t* shape, const tango_weights_t* weights, int32_t window,
                    int32_t phi_dim, int32_t chunk, const void* x, void* out, void* workspace,
                    size_t workspace_bytes, void* hip_stream) {
  return guarded([&] {
    return block_common(shape, weights, true, window, phi_dim, chunk, x, out, workspace, workspace_bytes,
                        hip_stream);
  });
}

const char* tango_status_string(int status) {
  switch (status) {
    case TANGO_OK: return "TANGO_OK";
    case TANGO_ERR_NULL: return "TANGO_ERR_NULL: a required pointer is NULL";
    case TANGO_ERR_SHAPE: return "TANGO_ERR_SHAPE: inconsistent sizes";
    case TANGO_ERR_DTYPE: return "TANGO_ERR_DTYPE: unknown dtype or io_dtype";
    case TANGO_ERR_ALIGN: return "TANGO_ERR_ALIGN: pointer not 16-byte aligned";
    case TANGO_ERR_UNSUPPORTED: return "TANGO_ERR_UNSUPPORTED: shape not covered by the kernels";
    case TANGO_ERR_WORKSPACE: return "TANGO_ERR_WORKSPACE: workspace too small";
    case TANGO_ERR_ALIAS: return "TANGO_ERR_ALIAS: buffers overlap";
    case TANGO_ERR_HIP: return "TANGO_ERR_HIP: HIP runtime error";
    default: return "unknown tango status";
  }
}

const char* tango_last_error(void) { return g_last_error.c_str(); }

int tango_version(void) { return TANGO_ABI_VERSION; }

size_t tango_proj_workspace_size(const tango_shape_t* shape) {
  if (check_shape(shape)) return 0;
  return proj_scratch(shape).total;
}

int tango_stage_proj(const tango_shape_t* shape, const tango_weights_t* weights, const void* x, void* gp,
                     void* v, void* qh, void* kh, void* workspace, size_t workspace_bytes,
                     void* hip_stream) {
  return guarded([&] {
    return stage_proj_common(shape, weights, x, gp, v, qh, kh, nullptr, nullptr, workspace,
                             workspace_bytes, hip_stream);
  });
}

int tango_stage_aggregate(const tango_shape_t* shape, const float* theta, const float* null_bias,
                          const void* qh, const void* kh, const void* gp, void* gbar, void* workspace,
                          size_t workspace_bytes, void* hip_stream) {
  return guarded([&] {
    int rc = check_shape(shape);
    if (rc) return rc;
    if (!theta || !qh || !kh || !gp || !gbar || !workspace)
      return fail(TANGO_ERR_NULL, "a buffer pointer is NULL");
    const tango_shape_t* s = shape;
    const Layout L = make_layout(s, false, 0, 0);
    if (workspace_bytes < L.total)
      return fail(TANGO_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                  workspace_bytes, L.total);
    const size_t es = elem_size(s->dtype), M = (size_t)s->batch * pad_rows(s->seq_len);
    const size_t F = gate_pad(s, false), HD = (size_t)s->n_heads * s->head_dim;   // head-padded
    const Range ins[] = {{qh, M * HD * es, "qh"}, {kh, M * HD * es, "kh"}, {gp, M * F * es, "gp"},
                         {theta, s->n_heads * sizeof(float), "theta"},
                         {null_bias, s->n_heads * sizeof(float), "null_bias"}};
    const Range outs[] = {{gbar, M * (size_t)s->d_gate * es, "gbar"}, {workspace, L.total, "workspace"}};
    if ((rc = check_ranges(ins, 5, outs, 2, nullptr, nullptr))) return rc;
    if ((rc = ensure_init())) return rc;
    char* base = static_cast<char*>(workspace);
    AggArgs aa = agg_args(s, theta, null_bias, qh, kh, gp, gbar, false);
    aa.part = reinterpret_cast<float*>(base + L.part);
    aa.part_den = reinterpret_cast<float*>(base + L.part_den);
    aa.counters = reinterpret_cast<int*>(base + L.counters);
    hipError_t e = launch_tango_agg(aa, L.agg, s->dtype == TANGO_BF16, false,
                                    static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? ok() : hip_fail(e, "aggregation kernel");
  });
}

// ---- backward of the TANGO aggregation ------------------------------------

int tango_aggregate_fwd_train(const tango_shape_t* shape, const float* theta, const float* null_bias,
                              const void* qh, const void* kh, const void* gp, void* gbar, float* den,
                              void* workspace, size_t workspace_bytes, void* hip_stream) {
  return guarded([&] {
    int rc = check_shape(shape);
    if (rc) return rc;
    if (!theta || !qh || !kh || !gp || !gbar || !den || !workspace)
      return fail(TANGO_ERR_NULL, "a buffer pointer is NULL");
    const tango_shape_t* s = shape;
    const Layout L = make_layout(s, false, 0, 0);
    if (workspace_bytes < L.total)
      return fail(TANGO_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                  workspace_bytes, L.total);
    const size_t es = elem_size(s->dtype), M = (size_t)s->batch * pad_rows(s->seq_len);
    const size_t F = gate_pad(s, false), HD = (size_t)s->n_heads * s->head_dim;
    const Range ins[] = {{qh, M * HD * es, "qh"}, {kh, M * HD * es, "kh"}, {gp, M * F * es, "gp"},
                         {theta, s->n_heads * sizeof(float), "theta"},
                         {null_bias, s->n_heads * sizeof(float), "null_bias"}};
    const Range outs[] = {{gbar, M * (size_t)s->d_gate * es, "gbar"},
                          {den, M * s->n_heads * sizeof(float), "den"},
                          {workspace, L.total, "workspace"}};
    if ((rc = check_ranges(ins, 5, outs, 3, nullptr, nullptr))) return rc;
    if ((rc = ensure_init())) return rc;
    char* base = static_cast<char*>(workspace);
    AggArgs aa = agg_args(s, theta, null_bias, qh, kh, gp, gbar, false);
    aa.part = reinterpret_cast<float*>(base + L.part);
    aa.part_den = reinterpret_cast<float*>(base + L.part_den);
    aa.counters = reinterpret_cast<int*>(base + L.counters);
    aa.den_out = den;
    hipError_t e = launch_tango_agg(aa, L.agg, s->dtype == TANGO_BF16, false,
                                    static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? ok() : hip_fail(e, "aggregation kernel");
  });
}

namespace {

struct BwdLayout {
  size_t u_rm, g_rm, qT, kT, q_rev, k_rev, u_rev_pk, delta, ds_rm, ds_t, part, part_theta;
  size_t agg_part, part_den, counters;   // split scratch of the reversed aggregation (dg)
  size_t total;
  BwdPlan plan;
  AggPlan agg;
};

BwdLayout make_bwd_layout(const tango_shape_t* s) {
  BwdLayout L{};
  const int64_t M = (int64_t)s->batch * pad_rows(s->seq_len);
  const int64_t HD = (int64_t)s->n_heads * s->head_dim, Fp = gate_pad(s, false);
  L.plan = tango_bwd_plan(s->batch, (int)pad_rows(s->seq_len), head_pad(s, false), s->n_heads);
  L.agg = tango_agg_plan(s->batch, (int)pad_rows(s->seq_len), (int)Fp, s->n_heads, s->head_dim, true);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const size_t es = 2;   // bfloat16
  L.u_rm = take((size_t)M * s->n_heads * L.plan.FhC * es);
  L.g_rm = take((size_t)M * s->n_heads * L.plan.FhC * es);
  L.qT = take((size_t)M * HD * es);
  L.kT = take((size_t)M * HD * es);
  L.q_rev = take((size_t)M * HD * es);
  L.k_rev = take((size_t)M * HD * es);
  L.u_rev_pk = take((size_t)M * Fp * es);
  L.delta = take((size_t)M * s->n_heads * sizeof(float));
  const size_t tiles = (size_t)L.plan.items_ds * kBwdTile * kBwdTile * es;
  L.ds_rm = take(tiles);
  L.ds_t = take(tiles);
  L.part = take((size_t)2 * L.plan.nch * M * HD * sizeof(float));
  L.part_theta = take((size_t)L.plan.items_ds * sizeof(float));
  const int64_t n = L.agg.n_split_tiles;
  L.agg_part = take((size_t)n * 2 * L.agg.br * L.agg.fs * sizeof(float));
  L.part_den = take((size_t)n * 2 * L.agg.br * sizeof(float));
  L.counters = take((size_t)n * sizeof(int));
  L.total = off;
  return L;
}

int check_bwd_shape(const tango_shape_t* s) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (s->dtype != TANGO_BF16)
    return fail(TANGO_ERR_UNSUPPORTED, "the aggregation backward is implemented for bfloat16 only");
  return TANGO_OK;
}

}  // namespace

size_t tango_aggregate_bwd_workspace_size(const tango_shape_t* shape) {
  if (!shape || check_bwd_shape(shape) != TANGO_OK) return 0;
  return make_bwd_layout(shape).total;
}

int tango_aggregate_bwd(const tango_shape_t* shape, const float* theta, const float* null_bias,
                        const void* qh, const void* kh, const void* gp, const void* gbar,
                        const float* den, const void* dgbar, float* dq, float* dk, void* dg,
                        float* dtheta, float* dnull, void* workspace, size_t workspace_bytes,
                        void* hip_stream) {
  return guarded([&] {
    int rc = check_bwd_shape(shape);
    if (rc) return rc;
    if (!theta || !qh || !kh || !gp || !gbar || !den || !dgbar || !dq || !dk || !dg || !dtheta ||
        !workspace)
      return fail(TANGO_ERR_NULL, "a buffer pointer is NULL");
    if ((null_bias == nullptr) != (dnull == nullptr))
      return fail(TANGO_ERR_NULL, "null_bias and dnull must both be given or both be NULL");
    const tango_shape_t* s = shape;
    const BwdLayout L = make_bwd_layout(s);
    if (workspace_bytes < L.total)
      return fail(TANGO_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                  workspace_bytes, L.total);
    const size_t M = (size_t)s->batch * pad_rows(s->seq_len);
    const size_t F = s->d_gate, Fp = gate_pad(s, false), HD = (size_t)s->n_heads * s->head_dim;
    const size_t H = s->n_heads;
    const Range ins[] = {{qh, M * HD * 2, "qh"},          {kh, M * HD * 2, "kh"},
                         {gp, M * Fp * 2, "gp"},          {gbar, M * F * 2, "gbar"},
                         {den, M * H * sizeof(float), "den"}, {dgbar, M * F * 2, "dgbar"},
                         {theta, H * sizeof(float), "theta"}, {null_bias, H * sizeof(float), "null_bias"}};
    const Range outs[] = {{dq, M * HD * sizeof(float), "dq"},  {dk, M * HD * sizeof(float), "dk"},
                          {dg, M * F * 2, "dg"},               {dtheta, H * sizeof(float), "dtheta"},
                          {dnull, H * sizeof(float), "dnull"}, {workspace, L.total, "workspace"}};
    if ((rc = check_ranges(ins, 8, outs, 6, nullptr, nullptr))) return rc;
    if ((rc = ensure_init())) return rc;
    const hipStream_t st = static_cast<hipStream_t>(hip_stream);
    char* base = static_cast<char*>(workspace);
    BwdArgs a{};
    a.qh = qh;
    a.kh = kh;
    a.gp = gp;
    a.gbar = gbar;
    a.dgbar = dgbar;
    a.den = den;
    a.theta = theta;
    a.null_bias = null_bias;
    a.u_rm = base + L.u_rm;
    a.g_rm = base + L.g_rm;
    a.qT = base + L.qT;
    a.kT = base + L.kT;
    a.q_rev = base + L.q_rev;
    a.k_rev = base + L.k_rev;
    a.u_rev_pk = base + L.u_rev_pk;
    a.delta = reinterpret_cast<float*>(base + L.delta);
    a.ds_rm = base + L.ds_rm;
    a.ds_t = base + L.ds_t;
    a.part = reinterpret_cast<float*>(base + L.part);
    a.part_theta = reinterpret_cast<float*>(base + L.part_theta);
    a.dq = dq;
    a.dk = dk;
    a.dtheta = dtheta;
    a.dnull = dnull;
    a.B = s->batch;
    a.T = s->seq_len;
    a.Tp = (int)pad_rows(s->seq_len);
    a.H = s->n_heads;
    a.dh = s->head_dim;
    a.F = s->d_gate;
    a.Fh = head_width(s);
    a.Fhp = head_pad(s, false);
    a.Fp = (int)Fp;
    a.FhC = L.plan.FhC;
    if (L.agg.split) {   // the row prep clears the dg aggregation's split counters
      a.zero_ints = reinterpret_cast<int*>(base + L.counters);
      a.n_zero_ints = L.agg.n_split_tiles;
    }
    hipError_t e = launch_tango_bwd_prep(a, L.plan, st);
    if (e != hipSuccess) return hip_fail(e, "backward prep kernels");
    // dg: the aggregation of the time-reversed problem, numerator only
    AggArgs aa = agg_args(s, theta, nullptr, a.k_rev, a.q_rev, a.u_rev_pk, dg, false);
    aa.part = reinterpret_cast<float*>(base + L.agg_part);
    aa.part_den = reinterpret_cast<float*>(base + L.part_den);
    aa.counters = reinterpret_cast<int*>(base + L.counters);
    aa.num_only = 1;
    aa.rev_out = 1;
    if ((e = launch_tango_agg(aa, L.agg, true, true, st)) != hipSuccess)
      return hip_fail(e, "reversed aggregation (dg)");
    if ((e = launch_tango_ds(a, L.plan, st)) != hipSuccess) return hip_fail(e, "ds tile kernel");
    if ((e = launch_tango_dsmm(a, L.plan, st)) != hipSuccess) return hip_fail(e, "dq / dk kernel");
    if ((e = launch_tango_bwd_finish(a, L.plan, st)) != hipSuccess) return hip_fail(e, "backward finish");
    return ok();
  });
}

}  // extern "C"

namespace {

constexpr int32_t kWangoBwdMaxWindow = 7 * kBwdTile + 1;   // near tiles of one product chunk

int check_wango_bwd(const tango_shape_t* s, int32_t window, int32_t chunk) {
  int rc = check_bwd_shape(s);
  if (rc) return rc;
  if ((rc = check_wango(s, window, s->head_dim, chunk))) return rc;
  if (window > kWangoBwdMaxWindow)
    return fail(TANGO_ERR_UNSUPPORTED, "window %d: the WANGO backward covers windows up to %d", window,
                kWangoBwdMaxWindow);
  return TANGO_OK;
}

// Scratch of the WANGO forward-train call: features, then the scan's.
struct WFwdLayout {
  size_t fq, fk, tmp, states, zstates, seg_state, seg_z, total;
  ScanPlan scan;
};
WFwdLayout make_wfwd_layout(const tango_shape_t* s, int32_t chunk) {
  WFwdLayout L{};
  const int64_t M = (int64_t)s->batch * pad_rows(s->seq_len);
  const int64_t F = gate_pad(s, true), HD = (int64_t)s->n_heads * s->head_dim;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L.scan = wango_scan_plan(s->batch, (int)pad_rows(s->seq_len), (int)F, s->n_heads, chunk);
  L.fq = take((size_t)M * HD * 2);
  L.fk = take((size_t)M * HD * 2);
  L.tmp = take((size_t)M * HD * 2);
  L.states = take(wango_states_bytes(s, chunk, false));
  L.zstates = take(wango_states_bytes(s, chunk, true));
  const int64_t bh = (int64_t)s->batch * s->n_heads;
  L.seg_state = take((size_t)bh * L.scan.nseg * s->head_dim * (F / s->n_heads) * sizeof(float));
  L.seg_z = take((size_t)bh * L.scan.nseg * s->head_dim * sizeof(float));
  L.total = off;
  return L;
}

// The WANGO scan + band of one problem into gbar (options set by the caller).
hipError_t wango_scan_band(const tango_shape_t* s, int32_t window, int32_t chunk, const WFwdLayout& L,
                           char* base, const BwdArgs& fa, const void* q, const void* k, const void* gp,
                           AggArgs aa, hipStream_t st, bool features_ready = false) {
  // destination features of q (permuted order), source features of k (packed),
  // unless the caller has written them already
  hipError_t e = hipSuccess;
  if (!features_ready && (e = launch_wango_bwd_features(fa, base + L.fq, base + L.tmp, q, k, base + L.fk, st)) != hipSuccess)
    return e;
  ScanArgs sa = scan_args(s, window, chunk, base + L.fq, base + L.fk, gp, nullptr, nullptr,
                          reinterpret_cast<float*>(base + L.seg_state), reinterpret_cast<float*>(base + L.seg_z));
  sa.states = base + L.states;
  sa.zstates = base + L.zstates;
  if ((e = launch_wango_scan(sa, L.scan, true, st)) != hipSuccess) return e;
  aa.states = base + L.states;
  aa.zstates = base + L.zstates;
  aa.fq = base + L.fq;
  aa.window = window;
  aa.chunk = chunk;
  return launch_wango_band(aa, true, st);
}

struct WBwdLayout {
  WFwdLayout f;   // the reversed problem's forward scratch (dg)
  size_t u_rm, g_rm, qT, kT, pT, aT, p_rm, a_rm, q_rev, k_rev, u_rev_pk, delta;
  size_t ds_rm, ds_t, dp_rm, dp_t, part, part_theta, theta_el, tsum, state, total;
  BwdPlan plan;
};
WBwdLayout make_wbwd_layout(const tango_shape_t* s, int32_t window, int32_t chunk) {
  WBwdLayout L{};
  L.f = make_wfwd_layout(s, chunk);
  const int64_t M = (int64_t)s->batch * pad_rows(s->seq_len);
  const int64_t Fp = gate_pad(s, true), HD = (int64_t)s->n_heads * s->head_dim;
  const int64_t bh = (int64_t)s->batch * s->n_heads;
  L.plan = wango_bwd_plan(s->batch, (int)pad_rows(s->seq_len), head_pad(s, true), s->n_heads, window);
  size_t off = L.f.total;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const size_t es = 2, rows = (size_t)M * s->n_heads * L.plan.FhC * es;
  L.u_rm = take(rows);
  L.g_rm = take(rows);
  L.qT = take((size_t)M * HD * es);
  L.kT = take((size_t)M * HD * es);
  L.pT = take((size_t)M * HD * es);
  L.aT = take((size_t)M * HD * es);
  L.p_rm = take((size_t)M * HD * es);
  L.a_rm = take((size_t)M * HD * es);
  L.q_rev = take((size_t)M * HD * es);
  L.k_rev = take((size_t)M * HD * es);
  L.u_rev_pk = take((size_t)M * Fp * es);
  L.delta = take((size_t)M * s->n_heads * sizeof(float));
  const size_t tiles = (size_t)L.plan.items_ds * kBwdTile * kBwdTile * es;
  L.ds_rm = take(tiles);
  L.ds_t = take(tiles);
  L.dp_rm = take(tiles);
  L.dp_t = take(tiles);
  L.part = take((size_t)6 * M * HD * sizeof(float));
  L.part_theta = take((size_t)L.plan.items_ds * sizeof(float));
  L.theta_el = take((size_t)((M * HD + 255) / 256) * s->n_heads * sizeof(float));
  const size_t st_el = (size_t)bh * L.plan.nt * s->head_dim * L.plan.FhC;
  L.tsum = take(st_el * sizeof(float));
  L.state = take(st_el * es);
  L.total = off;
  return L;
}

BwdArgs bwd_args(const tango_shape_t* s, const float* theta, const float* null_bias, const void* qh,
                 const void* kh, const void* gp, const void* gbar, const float* den, const void* dgbar, bool wango) {
  BwdArgs a{};
  a.qh = qh;
  a.kh = kh;
  a.gp = gp;
  a.gbar = gbar;
  a.dgbar = dgbar;
  a.den = den;
  a.theta = theta;
  a.null_bias = null_bias;
  a.B = s->batch;
  a.T = s->seq_len;
  a.Tp = (int)pad_rows(s->seq_len);
  a.H = s->n_heads;
  a.dh = s->head_dim;
  a.F = s->d_gate;
  a.Fh = head_width(s);
  a.Fhp = head_pad(s, wango);
  a.Fp = (int)gate_pad(s, wango);
  return a;
}

}  // namespace

extern "C" {

size_t wango_aggregate_fwd_train_workspace_size(const tango_shape_t* shape, int32_t window, int32_t chunk) {
  if (!shape || check_wango_bwd(shape, window, chunk) != TANGO_OK) return 0;
  return make_wfwd_layout(shape, chunk).total;
}

int wango_aggregate_fwd_train(const tango_shape_t* shape, int32_t window, int32_t chunk, const float* theta,
                              const float* null_bias, const void* qh, const void* kh, const void* gp, void* gbar,
                              float* den, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return guarded([&] {
    int rc = check_wango_bwd(shape, window, chunk);
    if (rc) return rc;
    if (!theta || !qh || !kh || !gp || !gbar || !den || !workspace)
      return fail(TANGO_ERR_NULL, "a buffer pointer is NULL");
    const tango_shape_t* s = shape;
    const WFwdLayout L = make_wfwd_layout(s, chunk);
    if (workspace_bytes < L.total)
      return fail(TANGO_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                  workspace_bytes, L.total);
    const size_t M = (size_t)s->batch * pad_rows(s->seq_len);
    const size_t F = gate_pad(s, true), HD = (size_t)s->n_heads * s->head_dim;
    const Range ins[] = {{qh, M * HD * 2, "qh"}, {kh, M * HD * 2, "kh"}, {gp, M * F * 2, "gp"},
                         {theta, s->n_heads * sizeof(float), "theta"},
                         {null_bias, s->n_heads * sizeof(float), "null_bias"}};
    const Range outs[] = {{gbar, M * (size_t)s->d_gate * 2, "gbar"},
                          {den, M * s->n_heads * sizeof(float), "den"},
                          {workspace, L.total, "workspace"}};
    if ((rc = check_ranges(ins, 5, outs, 3, nullptr, nullptr))) return rc;
    if ((rc = ensure_init())) return rc;
    const BwdArgs fa = bwd_args(s, theta, null_bias, qh, kh, gp, nullptr, nullptr, nullptr, true);
    AggArgs aa = agg_args(s, theta, null_bias, qh, kh, gp, gbar, true);
    aa.den_out = den;
    hipError_t e = wango_scan_band(s, window, chunk, L, static_cast<char*>(workspace), fa, qh, kh, gp, aa,
                                   static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? ok() : hip_fail(e, "WANGO scan / band kernels");
  });
}

size_t wango_aggregate_bwd_workspace_size(const tango_shape_t* shape, int32_t window, int32_t chunk) {
  if (!shape || check_wango_bwd(shape, window, chunk) != TANGO_OK) return 0;
  return make_wbwd_layout(shape, window, chunk).total;
}

int wango_aggregate_bwd(const tango_shape_t* shape, int32_t window, int32_t chunk, const float* theta,
                        const float* null_bias, const void* qh, const void* kh, const void* gp, const void* gbar,
                        const float* den, const void* dgbar, float* dq, float* dk, void* dg, float* dtheta,
                        float* dnull, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return guarded([&] {
    int rc = check_wango_bwd(shape, window, chunk);
    if (rc) return rc;
    if (!theta || !qh || !kh || !gp || !gbar || !den || !dgbar || !dq || !dk || !dg || !dtheta || !workspace)
      return fail(TANGO_ERR_NULL, "a buffer pointer is NULL");
    if ((null_bias == nullptr) != (dnull == nullptr))
      return fail(TANGO_ERR_NULL, "null_bias and dnull must both be given or both be NULL");
    const tango_shape_t* s = shape;
    const WBwdLayout L = make_wbwd_layout(s, window, chunk);
    if (workspace_bytes < L.total)
      return fail(TANGO_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                  workspace_bytes, L.total);
    const size_t M = (size_t)s->batch * pad_rows(s->seq_len);
    const size_t F = s->d_gate, Fp = gate_pad(s, true), HD = (size_t)s->n_heads * s->head_dim;
    const size_t H = s->n_heads;
    const Range ins[] = {{qh, M * HD * 2, "qh"},          {kh, M * HD * 2, "kh"},
                         {gp, M * Fp * 2, "gp"},          {gbar, M * F * 2, "gbar"},
                         {den, M * H * sizeof(float), "den"}, {dgbar, M * F * 2, "dgbar"},
                         {theta, H * sizeof(float), "theta"}, {null_bias, H * sizeof(float), "null_bias"}};
    const Range outs[] = {{dq, M * HD * sizeof(float), "dq"},  {dk, M * HD * sizeof(float), "dk"},
                          {dg, M * F * 2, "dg"},               {dtheta, H * sizeof(float), "dtheta"},
                          {dnull, H * sizeof(float), "dnull"}, {workspace, L.total, "workspace"}};
    if ((rc = check_ranges(ins, 8, outs, 6, nullptr, nullptr))) return rc;
    if ((rc = ensure_init())) return rc;
    const hipStream_t st = static_cast<hipStream_t>(hip_stream);
    char* base = static_cast<char*>(workspace);
    BwdArgs a = bwd_args(s, theta, null_bias, qh, kh, gp, gbar, den, dgbar, true);
    a.u_rm = base + L.u_rm;
    a.g_rm = base + L.g_rm;
    a.qT = base + L.qT;
    a.kT = base + L.kT;
    a.pT = base + L.pT;
    a.aT = base + L.aT;
    a.p_rm = base + L.p_rm;
    a.a_rm = base + L.a_rm;
    a.q_rev = base + L.q_rev;
    a.k_rev = base + L.k_rev;
    a.u_rev_pk = base + L.u_rev_pk;
    a.delta = reinterpret_cast<float*>(base + L.delta);
    a.ds_rm = base + L.ds_rm;
    a.ds_t = base + L.ds_t;
    a.dp_rm = base + L.dp_rm;
    a.dp_t = base + L.dp_t;
    a.part = reinterpret_cast<float*>(base + L.part);
    a.part_theta = reinterpret_cast<float*>(base + L.part_theta);
    a.dq = dq;
    a.dk = dk;
    a.dtheta = dtheta;
    a.dnull = dnull;
    a.window = window;
    a.nb = L.plan.nb;
    a.FhC = L.plan.FhC;
    hipError_t e = launch_wango_bwd_prep(a, L.plan, base + L.f.fq, base + L.f.fk, st);
    if (e != hipSuccess) return hip_fail(e, bwd_last_step());
    // dg: the whole WANGO aggregation (scan + band) of the time-reversed
    // problem, numerator only (its features come from the prep)
    AggArgs aa = agg_args(s, theta, nullptr, a.k_rev, a.q_rev, a.u_rev_pk, dg, true);
    aa.num_only = 1;
    aa.rev_out = 1;
    if ((e = wango_scan_band(s, window, chunk, L.f, base, a, a.k_rev, a.q_rev, a.u_rev_pk, aa, st, true)) != hipSuccess)
      return hip_fail(e, "reversed scan / band (dg)");
    // window and near older pairs
    if ((e = launch_tango_ds(a, L.plan, st)) != hipSuccess) return hip_fail(e, "ds tile kernel");
    if ((e = launch_tango_dsmm(a, L.plan, st)) != hipSuccess) return hip_fail(e, "tile product kernel");
    // far older pairs: prefix states of a g^T and suffix states of p u^T
    const int64_t MHD = (int64_t)M * HD;
    WStateArgs w{};
    w.tsum = reinterpret_cast<float*>(base + L.tsum);
    w.state = base + L.state;
    w.B = s->batch;
    w.H = s->n_heads;
    w.dh = s->head_dim;
    w.Tp = a.Tp;
    w.FhC = L.plan.FhC;
    w.nt = L.plan.nt;
    w.nb = L.plan.nb;
    w.aT = a.aT;
    w.xrm = a.g_rm;
    w.rows = a.u_rm;
    w.out = a.part + 4 * MHD;
    if ((e = launch_wango_state_sums(w, st)) != hipSuccess || (e = launch_wango_state_scan(w, false, st)) != hipSuccess ||
        (e = launch_wango_state_readout(w, st)) != hipSuccess)
      return hip_fail(e, "prefix states (dp)");
    w.aT = a.pT;
    w.xrm = a.u_rm;
    w.rows = a.g_rm;
    w.out = a.part + 5 * MHD;
    if ((e = launch_wango_state_sums(w, st)) != hipSuccess || (e = launch_wango_state_scan(w, true, st)) != hipSuccess ||
        (e = launch_wango_state_readout(w, st)) != hipSuccess)
      return hip_fail(e, "suffix states (da)");
    if ((e = launch_wango_bwd_finish(a, L.plan, reinterpret_cast<float*>(base + L.theta_el), st)) != hipSuccess)
      return hip_fail(e, "backward finish");
    return ok();
  });
}

int tango_stage_out(const tango_shape_t* shape, const void* w_o, const void* x, const void* gbar,
                    const void* v, void* out, void* hip_stream) {
  return guarded([&] {
    int rc = check_shape(shape);
    if (rc) return rc;
    if (!w_o || !x || !gbar || !v || !out) return fail(TANGO_ERR_NULL, "a buffer pointer is NULL");
    const tango_shape_t* s = shape;
    const size_t es = elem_size(s->dtype), M = (size_t)s->batch * pad_rows(s->seq_len);
    const size_t d = s->d_model, F = s->d_gate;
    const size_t xb = (size_t)s->batch * s->seq_len * d * elem_size(s->io_dtype);
    const Range ins[] = {{w_o, d * F * es, "w_o"}, {x, xb, "x"}, {gbar, M * F * es, "gbar"},
                         {v, M * F * v_elem(s), "v"}};
    const Range outs[] = {{out, xb, "out"}};
    if ((rc = check_ranges(ins, 4, outs, 1, x, out))) return rc;
    if ((rc = ensure_init())) return rc;
    hipError_t e = launch_out(out_args(s, w_o, x, gbar, v, out), s->dtype == TANGO_BF16,
                              s->io_dtype == TANGO_BF16, static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? ok() : hip_fail(e, "output kernel");
  });
}

int wango_stage_proj(const tango_shape_t* shape, const tango_weights_t* weights, const void* x, void* gp,
                     void* v, void* qh, void* kh, void* fq, void* fk, void* workspace,
                     size_t workspace_bytes, void* hip_stream) {
  return guarded([&] {
    if (!fq || !fk) return fail(TANGO_ERR_NULL, "a buffer pointer is NULL");
    return stage_proj_common(shape, weights, x, gp, v, qh, kh, fq, fk, workspace, workspace_bytes,
                             hip_stream);
  });
}

int wango_stage_scan(const tango_shape_t* shape, int32_t window, int32_t chunk, const void* fq,
                     const void* fk, const void* gp, void* n_old, void* z_old, void* workspace,
                     size_t workspace_bytes, void* hip_stream) {
  return guarded([&] {
    int rc = check_shape(shape);
    if (rc) return rc;
    if ((rc = check_wango(shape, window, shape->head_dim, chunk))) return rc;
    if (!fq || !fk || !gp || !n_old || !z_old || !workspace)
      return fail(TANGO_ERR_NULL, "a buffer pointer is NULL");
    const tango_shape_t* s = shape;
    const Layout L = make_layout(s, true, window, chunk);
    if (workspace_bytes < L.total)
      return fail(TANGO_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                  workspace_bytes, L.total);
    const size_t es = elem_size(s->dtype), M = (size_t)s->batch * pad_rows(s->seq_len);
    const size_t F = gate_pad(s, true), HD = (size_t)s->n_heads * s->head_dim;   // head-padded
    const Range ins[] = {{fq, M * HD * es, "fq"}, {fk, M * HD * es, "fk"}, {gp, M * F * es, "gp"}};
    const Range outs[] = {{n_old, M * F * sizeof(float), "n_old"},
                          {z_old, M * s->n_heads * sizeof(float), "z_old"},
                          {workspace, L.total, "workspace"}};
    if ((rc = check_ranges(ins, 3, outs, 3, nullptr, nullptr))) return rc;
    if ((rc = ensure_init())) return rc;
    char* base = static_cast<char*>(workspace);
    ScanArgs sa = scan_args(s, window, chunk, fq, fk, gp, static_cast<float*>(n_old),
                            static_cast<float*>(z_old), reinterpret_cast<float*>(base + L.seg_state),
                            reinterpret_cast<float*>(base + L.seg_z));
    hipError_t e = launch_wango_scan(sa, L.scan, s->dtype == TANGO_BF16, static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? ok() : hip_fail(e, "scan kernels");
  });
}

int wango_stage_band(const tango_shape_t* shape, const float* theta, const float* null_bias, int32_t window,
                     int32_t chunk, const void* qh, const void* kh, const void* gp, const float* n_old,
                     const float* z_old, void* gbar, void* hip_stream) {
  return guarded([&] {
    int rc = check_shape(shape);
    if (rc) return rc;
    if ((rc = check_wango(shape, window, shape->head_dim, chunk))) return rc;
    if (!theta || !qh || !kh || !gp || !n_old || !z_old || !gbar)
      return fail(TANGO_ERR_NULL, "a buffer pointer is NULL");
    const tango_shape_t* s = shape;
    const size_t es = elem_size(s->dtype), M = (size_t)s->batch * pad_rows(s->seq_len);
    const size_t F = gate_pad(s, true), HD = (size_t)s->n_heads * s->head_dim;   // head-padded
    const Range ins[] = {{qh, M * HD * es, "qh"}, {kh, M * HD * es, "kh"}, {gp, M * F * es, "gp"},
                         {n_old, M * F * sizeof(float), "n_old"},
                         {z_old, M * s->n_heads * sizeof(float), "z_old"},
                         {theta, s->n_heads * sizeof(float), "theta"},
                         {null_bias, s->n_heads * sizeof(float), "null_bias"}};
    const Range outs[] = {{gbar, M * (size_t)s->d_gate * es, "gbar"}};
    if ((rc = check_ranges(ins, 7, outs, 1, nullptr, nullptr))) return rc;
    if ((rc = ensure_init())) return rc;
    AggArgs aa = agg_args(s, theta, null_bias, qh, kh, gp, gbar, true);
    aa.n_old = n_old;
    aa.z_old = z_old;
    aa.window = window;
    aa.chunk = chunk;
    hipError_t e = launch_wango_band(aa, s->dtype == TANGO_BF16, static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? ok() : hip_fail(e, "band kernel");
  });
}


// ---- autoregressive decode -----------------------------------------------------

}  // extern "C"

namespace {

struct DecLayout {
  // state
  size_t kc, gc, S, z, state_total;
  // workspace
  size_t xs, rinv, v, q, part, gv, opart, ocount, ws_total;
  int64_t n_ocount;
  int P, nch;
  int64_t Mp;
};

int check_decode(const tango_shape_t* s, bool wango, int32_t window, int32_t phi_dim) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (wango) {
    if (window < 1) return fail(TANGO_ERR_SHAPE, "window %d < 1", window);
    if (phi_dim != s->head_dim)
      return fail(TANGO_ERR_SHAPE, "phi_dim %d must equal head_dim %d (phi acts elementwise)", phi_dim,
                  s->head_dim);
    if (window > kDecMaxWindow)
      return fail(TANGO_ERR_UNSUPPORTED, "window %d: the decode kernels take at most %d", window,
                  kDecMaxWindow);
  }
  if (s->n_heads > 32) return fail(TANGO_ERR_UNSUPPORTED, "n_heads %d: decode takes at most 32", s->n_heads);
  if (head_width(s) % 64 != 0)
    return fail(TANGO_ERR_UNSUPPORTED, "d_gate / n_heads = %d: decode needs a multiple of 64", head_width(s));
  return TANGO_OK;
}

DecLayout make_dec_layout(const tango_shape_t* s, bool wango, int32_t window) {
  DecLayout L{};
  const size_t es = elem_size(s->dtype);
  const int64_t B = s->batch, F = s->d_gate, HD = (int64_t)s->n_heads * s->head_dim;
  L.P = wango ? window + 1 : s->seq_len;
  L.nch = wango ? 0 : (L.P + kDecChunk - 1) / kDecChunk;
  L.Mp = pad_rows(B);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L.kc = take((size_t)B * L.P * HD * es);
  L.gc = take((size_t)B * L.P * F * es);
  if (wango) {
    L.S = take((size_t)B * s->n_heads * s->head_dim * (F / s->n_heads) * sizeof(float));
    L.z = take((size_t)B * 2 * s->n_heads * s->head_dim * sizeof(float));
  }
  L.state_total = off;
  off = 0;
  const bool bf = s->dtype == TANGO_BF16;
  L.xs = take(proj_parts_bytes(L.Mp, s->d_model, bf, decode_parts(bf)));
  L.rinv = take((size_t)L.Mp * sizeof(float));
  L.v = take((size_t)L.Mp * F * es);
  L.q = take((size_t)L.Mp * HD * es);
  if (!wango) L.part = take((size_t)B * L.nch * (F + 64) * sizeof(float));
  L.gv = take((size_t)decode_parts(bf) * L.Mp * F * es);
  L.opart = take((size_t)kOutSplit * L.Mp * s->d_model * sizeof(float));
  L.n_ocount = (int64_t)(s->d_model / 16) * ((B + 15) / 16);   // output tiles (16 tokens or more each)
  L.ocount = take((size_t)L.n_ocount * sizeof(int));
  L.ws_total = off;
  return L;
}

// lib_scratch: the scratch is the library's own array of the current device
// (ws and ws_bytes are ignored; the size is checked against the array), taken
// after every argument has been validated.
int decode_common(const tango_shape_t* s, const tango_weights_t* w, bool wango, int32_t window,
                  int32_t phi_dim, const int32_t* pos, const void* x, void* out, void* state,
                  size_t state_bytes, void* ws, size_t ws_bytes, void* stream, bool lib_scratch = false) {
  int rc = check_decode(s, wango, window, phi_dim);
  if (rc) return rc;
  if ((rc = check_weights(w, true))) return rc;
  if (!pos || !x || !out) return fail(TANGO_ERR_NULL, "pos, x or out is NULL");
  if (!state) return fail(TANGO_ERR_NULL, "state is NULL");
  if (!lib_scratch && !ws) return fail(TANGO_ERR_NULL, "workspace is NULL");
  const DecLayout L = make_dec_layout(s, wango, window);
  if (state_bytes < L.state_total)
    return fail(TANGO_ERR_WORKSPACE, "state of %zu bytes is smaller than the %zu needed", state_bytes,
                L.state_total);
  if (lib_scratch) {
    if (L.ws_total > TANGO_NOALLOC_SCRATCH_BYTES)
      return fail(TANGO_ERR_WORKSPACE,
                  "this decode step needs %zu bytes of scratch; the library's array holds %zu "
                  "(TANGO_NOALLOC_SCRATCH_BYTES): decode fewer sequences per call or pass a workspace",
                  L.ws_total, (size_t)TANGO_NOALLOC_SCRATCH_BYTES);
    ws = nullptr;   // taken below, once the arguments are valid
    ws_bytes = 0;
  } else if (ws_bytes < L.ws_total) {
    return fail(TANGO_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes,
                L.ws_total);
  }
  const size_t es = elem_size(s->dtype);
  const size_t d = s->d_model, F = s->d_gate, HD = (size_t)s->n_heads * s->head_dim;
  const size_t xb = (size_t)s->batch * d * elem_size(s->io_dtype);
  const Range ins[] = {{x, xb, "x"},
                       {pos, (size_t)s->batch * sizeof(int32_t), "pos"},
                       {w->w_g, F * d * es, "w_g"},
                       {w->w_v, F * d * es, "w_v"},
                       {w->w_q, HD * d * es, "w_q"},
                       {w->w_k, HD * d * es, "w_k"},
                       {w->w_o, d * F * es, "w_o"},
                       {w->rms_gain, d * es, "rms_gain"},
                       {w->theta, s->n_heads * sizeof(float), "theta"},
                       {w->null_bias, s->n_heads * sizeof(float), "null_bias"}};
  const Range outs[] = {{out, xb, "out"}, {state, L.state_total, "state"}, {ws, L.ws_total, "workspace"}};
  const int n_outs = lib_scratch ? 2 : 3;   // the library's array cannot alias the caller's buffers
  // pos only needs 4-byte alignment
  for (const Range& r : ins)
    if (r.p && r.p != pos && !aligned(r.p)) return fail(TANGO_ERR_ALIGN, "%s is not 16-byte aligned", r.name);
  if (((uintptr_t)pos & 3u) != 0) return fail(TANGO_ERR_ALIGN, "pos is not 4-byte aligned");
  Range ins16[9];
  int n16 = 0;
  for (const Range& r : ins)
    if (r.p != pos) ins16[n16++] = r;
  if ((rc = check_ranges(ins16, n16, outs, n_outs, x, out))) return rc;
  for (int o = 0; o < n_outs; ++o)
    if (overlap(outs[o], ins[1])) return fail(TANGO_ERR_ALIAS, "%s overlaps pos", outs[o].name);
  if ((rc = ensure_init())) return rc;
  if (lib_scratch) {
    ws = device_scratch();
    if (!ws) return fail(TANGO_ERR_HIP, "no scratch array on the current device");
  }

  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf = s->dtype == TANGO_BF16, io_bf = s->io_dtype == TANGO_BF16;
  char* sb = static_cast<char*>(state);
  char* wb = static_cast<char*>(ws);
  // row prep over the B new tokens taken as one sequence of B rows
  ProjArgs pa{};
  pa.x = x;
  pa.gain = w->rms_gain;
  pa.xs = wb + L.xs;
  pa.rinv = reinterpret_cast<float*>(wb + L.rinv);
  pa.B = 1;
  pa.T = s->batch;
  pa.Tp = (int)L.Mp;
  pa.d = s->d_model;
  pa.eps = s->rms_eps;
  pa.parts = decode_parts(bf);
  pa.zero = reinterpret_cast<int*>(wb + L.ocount);   // the output GEMM's counters
  pa.zero_n = L.n_ocount;
  hipError_t e = launch_prep(pa, bf, io_bf, st);
  if (e != hipSuccess) return hip_fail(e, "row-prep kernel");
  DecArgs a{};
  a.B = s->batch;
  a.Mp = (int)L.Mp;
  a.d = s->d_model;
  a.F = s->d_gate;
  a.H = s->n_heads;
  a.dh = s->head_dim;
  a.HD = (int)HD;
  a.P = L.P;
  a.window = wango ? window : 0;
  a.nch = L.nch;
  a.rope_base = s->rope_base;
  a.pos = pos;
  a.w_g = w->w_g;
  a.w_v = w->w_v;
  a.w_q = w->w_q;
  a.w_k = w->w_k;
  a.w_o = w->w_o;
  a.theta = w->theta;
  a.null_bias = w->null_bias;
  a.kc = sb + L.kc;
  a.gc = sb + L.gc;
  a.S = wango ? reinterpret_cast<float*>(sb + L.S) : nullptr;
  a.z = wango ? reinterpret_cast<float*>(sb + L.z) : nullptr;
  a.xs = wb + L.xs;
  a.rinv = reinterpret_cast<const float*>(wb + L.rinv);
  a.v = wb + L.v;
  a.q = wb + L.q;
  a.part = wango ? nullptr : reinterpret_cast<float*>(wb + L.part);
  a.gv = wb + L.gv;
  a.opart = reinterpret_cast<float*>(wb + L.opart);
  a.ocount = reinterpret_cast<int*>(wb + L.ocount);
  a.x = x;
  a.out = out;
  e = launch_decode(a, bf, io_bf, st);
  return e == hipSuccess ? ok() : hip_fail(e, "decode kernels");
}

}  // namespace

extern "C" {

size_t tango_decode_state_size(const tango_shape_t* shape) {
  if (check_decode(shape, false, 0, 0)) return 0;
  return make_dec_layout(shape, false, 0).state_total;
}

size_t tango_decode_workspace_size(const tango_shape_t* shape) {
  if (check_decode(shape, false, 0, 0)) return 0;
  return make_dec_layout(shape, false, 0).ws_total;
}

size_t wango_decode_state_size(const tango_shape_t* shape, int32_t window, int32_t phi_dim) {
  if (check_decode(shape, true, window, phi_dim)) return 0;
  return make_dec_layout(shape, true, window).state_total;
}

size_t wango_decode_workspace_size(const tango_shape_t* shape, int32_t window, int32_t phi_dim) {
  if (check_decode(shape, true, window, phi_dim)) return 0;
  return make_dec_layout(shape, true, window).ws_total;
}

int tango_decode_step(const tango_shape_t* shape, const tango_weights_t* weights, const int32_t* pos,
                      const void* x, void* out, void* state, size_t state_bytes, void* workspace,
                      size_t workspace_bytes, void* hip_stream) {
  return guarded([&] {
    return decode_common(shape, weights, false, 0, 0, pos, x, out, state, state_bytes, workspace,
                         workspace_bytes, hip_stream);
  });
}

int wango_decode_step(const tango_shape_t* shape, const tango_weights_t* weights, int32_t window,
                      int32_t phi_dim, const int32_t* pos, const void* x, void* out, void* state,
                      size_t state_bytes, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return guarded([&] {
    return decode_common(shape, weights, true, window, phi_dim, pos, x, out, state, state_bytes, workspace,
                         workspace_bytes, hip_stream);
  });
}

int wango_decode_step_noalloc(const tango_shape_t* shape, const tango_weights_t* weights, int32_t window,
                              int32_t phi_dim, const int32_t* pos, const void* x, void* out, void* state,
                              size_t state_bytes, void* hip_stream) {
  return guarded([&] {
    return decode_common(shape, weights, true, window, phi_dim, pos, x, out, state, state_bytes, nullptr, 0,
                         hip_stream, true);
  });
}

}  // extern "C"
