// decode_kernels.hip - one autoregressive decode step of the TANGO / WANGO
// block on gfx950.
//
// "TANGO: Token-Aggregated Nonlinear Gating Operators ...": a decode step gives
// the block output (§2.1 eqs. 2-5 and 3) at the next position p of every
// sequence from a state kept between steps.  TANGO keeps every unit key and
// gate so far (eq. 6 sums over the whole prefix).  WANGO keeps the running sums
// S, z of §2.2 eq. 10 -- the token that leaves the trailing window is added to
// them when the position advances -- and the keys and gates of the last W + 1
// positions, a state that does not grow with the position (§6.1).
//
// One step of one block is four or five launches on the caller's stream:
//   prep  (the forward's row-prep kernel) RMSNorm scale, operand parts of h*gain;
//   dproj the projections of the new tokens as a skinny MFMA GEMM (16 weight
//         rows per wave); SiLU gates and RoPE + unit keys go straight into the
//         state at the token's position, features and unit queries to scratch;
//   TANGO dagg  streams the key/gate cache in chunks of kChunk positions: exp
//               weights e^{tau (s - 1)} (static shift: |s| <= 1), float32
//               partial numerators and denominators per chunk;
//         dcomb adds the chunk partials, divides, forms gbar * v;
//   WANGO dband per (sequence, head, column block): adds the leaving token to S
//               and z, reads phi_q^T S out, adds the window's exp-weighted
//               gates, divides, forms gbar * v;
//   dout  out = x + (gbar * v) W_o^T as a skinny MFMA GEMM, K split over waves.
// The older-prefix terms carry the same e^{-tau} factor as the window weights,
// so the shift cancels in the ratio (as in the forward kernels).
#include "common.hpp"
#include "kernels.hpp"

namespace tango {

namespace {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecTokens = 64;                 // tokens (4 m-tiles of 16) per workgroup
constexpr int kDecMT = kDecTokens / 16;
constexpr int kAggThreadsD = 256;
constexpr int kBandThreads = 256;

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }

__device__ __forceinline__ float tau_of(const float* theta, int h) {
  return __expf(fminf(theta[h], 2.995732273553991f));   // exp(min(theta, log 20))
}

// Slot of position p in the state: the position itself for the TANGO cache, p
// mod (W + 1) for the WANGO ring (a.P = W + 1 there).
__device__ __forceinline__ int64_t state_row(const DecArgs& a, int64_t b, int p) {
  return b * a.P + (a.window > 0 ? p % a.P : p);
}

__device__ __forceinline__ bool pos_ok(const DecArgs& a, int p) {
  return p >= 0 && (a.window > 0 || p < a.P);
}

// ---------------------------------------------------------------------------
// dproj: [g | v | q | k] rows of the new tokens.  Workgroup: 8 waves x 16
// weight rows = 128 rows of the stacked [W_g; W_v; W_q; W_k] against up to 64
// tokens.  A head of q or k (d_h in {32, 64, 128}, starting at a multiple of
// d_h past 2F, which is a multiple of 128) never straddles two workgroups, so
// its norm is reduced through LDS.
// ---------------------------------------------------------------------------
template <typename T, int AS>
__global__ __launch_bounds__(kDecThreads) void dproj_kernel(DecArgs a) {
  __shared__ float nrm[kDecWaves][kDecTokens];
  const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int F = a.F, HD = a.HD, d = a.d;
  const int N = 2 * F + 2 * HD;
  const int n0 = blockIdx.x * (kDecWaves * 16) + wave * 16;
  const int m0 = blockIdx.y * kDecTokens;
  const bool live = n0 < N;
  const int cls = n0 < F ? 0 : n0 < 2 * F ? 1 : n0 < 2 * F + HD ? 2 : 3;
  const int wrow = cls == 0 ? n0 : cls == 1 ? n0 - F : cls == 2 ? n0 - 2 * F : n0 - 2 * F - HD;
  const T* W = static_cast<const T*>(cls == 0 ? a.w_g : cls == 1 ? a.w_v : cls == 2 ? a.w_q : a.w_k);
  const T* xs = static_cast<const T*>(a.xs);

  f32x4 acc[kDecMT];
#pragma unroll
  for (int mt = 0; mt < kDecMT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (live) {
    const T* wr = W + (int64_t)(wrow + li) * d + lg * 8;
    const T* xr = xs + (int64_t)(m0 + li) * d + lg * 8;
#pragma unroll 2
    for (int k0 = 0; k0 < d; k0 += 32) {
      const Frag<T> A = load_frag<T>(wr + k0);
#pragma unroll
      for (int mt = 0; mt < kDecMT; ++mt)
#pragma unroll
        for (int part = 0; part < AS; ++part)
          mma(acc[mt], A, load_frag<T>(xr + ((int64_t)part * a.Mp + mt * 16) * d + k0));
    }
  }

  // epilogue: lane (li, lg) holds rows n0 + 4 lg + r of token m0 + 16 mt + li
  float val[kDecMT][4];
  int pos[kDecMT];
#pragma unroll
  for (int mt = 0; mt < kDecMT; ++mt) {
    const int m = m0 + mt * 16 + li;
    const float rs = a.rinv[m];                     // zero for padding rows
    pos[mt] = m < a.B ? a.pos[m] : -1;
#pragma unroll
    for (int r = 0; r < 4; ++r) val[mt][r] = acc[mt][r] * rs;
  }
  const int col = n0 + 4 * lg;                      // first of this lane's 4 rows
  if (live && cls == 0) {
#pragma unroll
    for (int mt = 0; mt < kDecMT; ++mt) {
      const int m = m0 + mt * 16 + li;
      if (m < a.B && pos_ok(a, pos[mt])) {
        f32x4 g;
#pragma unroll
        for (int r = 0; r < 4; ++r) g[r] = silu_f(val[mt][r]);
        store_quad<T>(static_cast<T*>(a.gc) + state_row(a, m, pos[mt]) * F + col, cvt_quad<T>(g));
      }
    }
  } else if (live && cls == 1) {
#pragma unroll
    for (int mt = 0; mt < kDecMT; ++mt) {
      const int m = m0 + mt * 16 + li;
      if (m < a.B)
        store_quad<T>(static_cast<T*>(a.v) + (int64_t)m * F + col - F,
                      cvt_quad<T>(f32x4{val[mt][0], val[mt][1], val[mt][2], val[mt][3]}));
    }
  }
  // queries and keys: RoPE on the pairs (4 lg, 4 lg + 1), (4 lg + 2, 4 lg + 3),
  // then the squared norm of this wave's 16 rows of the head
  const bool qk = live && cls >= 2;
  const int e0 = qk ? col - (cls == 2 ? 2 * F : 2 * F + HD) : 0;   // column within q or k
  if (qk && a.rope_base > 0.f) {
    const int c0 = (e0 % a.dh) / 2;
    // rotation rate of pairs c0, c0 + 1 in revolutions per position (float64:
    // a float32 angle at large positions would be off by ~1e-3 rad)
    const double f0 = pow((double)a.rope_base, -2.0 * c0 / a.dh) * 0.15915494309189533577;
    const double f1 = pow((double)a.rope_base, -2.0 * (c0 + 1) / a.dh) * 0.15915494309189533577;
#pragma unroll
    for (int mt = 0; mt < kDecMT; ++mt) {
      const double p = (double)max(pos[mt], 0);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const double rev = p * (h2 ? f1 : f0);
        const float fr = (float)(rev - rint(rev));
        const float fs = __builtin_amdgcn_sinf(fr), fc = __builtin_amdgcn_cosf(fr);
        const float u0 = val[mt][2 * h2], u1 = val[mt][2 * h2 + 1];
        val[mt][2 * h2] = u0 * fc - u1 * fs;
        val[mt][2 * h2 + 1] = u0 * fs + u1 * fc;
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < kDecMT; ++mt) {
    float ss = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) ss += val[mt][r] * val[mt][r];
    ss = group_sum(ss);                              // the wave's 16 rows, token li
    if (lg == 0) nrm[wave][mt * 16 + li] = ss;
  }
  __syncthreads();
  if (qk) {
    const int wph = a.dh / 16;                       // waves per head
    const int hw0 = wave - (e0 % a.dh) / 16;         // first wave of this head
#pragma unroll
    for (int mt = 0; mt < kDecMT; ++mt) {
      const int m = m0 + mt * 16 + li;
      float tot = 0.f;
      for (int w2 = 0; w2 < wph; ++w2) tot += nrm[hw0 + w2][mt * 16 + li];
      const float inv = 1.0f / fmaxf(sqrtf(tot), 1e-12f);
      const f32x4 u = {val[mt][0] * inv, val[mt][1] * inv, val[mt][2] * inv, val[mt][3] * inv};
      if (m < a.B) {
        if (cls == 2)
          store_quad<T>(static_cast<T*>(a.q) + (int64_t)m * HD + e0, cvt_quad<T>(u));
        else if (pos_ok(a, pos[mt]))
          store_quad<T>(static_cast<T*>(a.kc) + state_row(a, m, pos[mt]) * HD + e0, cvt_quad<T>(u));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// TANGO dagg: chunk c of sequence b, sources j in [c kChunk, min(c kChunk +
// kChunk, p + 1)).  Partial numerators [F] and denominators [H] in float32,
// row stride F + 64 floats.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kAggThreadsD) void dagg_kernel(DecArgs a) {
  __shared__ float qs[1024];
  __shared__ float pw[kDecChunk * 32];
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.y;
  const int c = blockIdx.x;
  const int p = a.pos[b];
  if (!pos_ok(a, p)) return;
  const int j0 = c * kDecChunk;
  if (j0 > p) return;
  const int nj = min(kDecChunk, p + 1 - j0);
  const int F = a.F, HD = a.HD, H = a.H, dh = a.dh, Fh = F / H;
  const T* kc = static_cast<const T*>(a.kc);
  const T* gc = static_cast<const T*>(a.gc);
  for (int i = tid; i < HD; i += kAggThreadsD) qs[i] = tof<T>(static_cast<const T*>(a.q)[b * HD + i]);
  __syncthreads();
  // exp weights, one (source, head) item per thread and pass
  for (int it = tid; it < kDecChunk * H; it += kAggThreadsD) {
    const int jl = it / H, h = it - (it / H) * H;
    float w = 0.f;
    if (jl < nj) {
      const T* kr = kc + (b * a.P + j0 + jl) * HD + h * dh;
      float s = 0.f;
      for (int e = 0; e < dh; e += 8) {
        const Frag<T> kf = load_frag<T>(kr + e);
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) s += qs[h * dh + e + s8] * tof<T>(kf[s8]);
      }
      w = __builtin_amdgcn_exp2f(tau_of(a.theta, h) * kLog2e * (s - 1.0f));
    }
    pw[jl * H + h] = w;
  }
  __syncthreads();
  float* part = a.part + ((int64_t)b * a.nch + c) * (F + 64);
  for (int f0 = 0; f0 < F; f0 += kAggThreadsD * 8) {
    const int col = f0 + tid * 8;
    if (col < F) {
      const int h = col / Fh;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const T* gr = gc + (b * a.P + j0) * F + col;
#pragma unroll 8
      for (int jl = 0; jl < nj; ++jl) {
        const Frag<T> g = load_frag<T>(gr + (int64_t)jl * F);
        const float w = pw[jl * H + h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += w * tof<T>(g[e]);
      }
      *reinterpret_cast<f32x4*>(part + col) = f32x4{acc[0], acc[1], acc[2], acc[3]};
      *reinterpret_cast<f32x4*>(part + col + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    }
  }
  if (tid < H) {
    float s = 0.f;
    for (int jl = 0; jl < nj; ++jl) s += pw[jl * H + tid];
    part[F + tid] = s;
  }
}

// Split gbar * v (float32) into the AS parts of the output GEMM's operand.
template <typename T, int AS>
__device__ __forceinline__ void store_gv(const DecArgs& a, int64_t m, int col, const float (&gv)[8]) {
  T* dst = static_cast<T*>(a.gv) + m * a.F + col;
  Frag<T> hi;
#pragma unroll
  for (int e = 0; e < 8; ++e) hi[e] = cvt<T>(gv[e]);
  store_frag<T>(dst, hi);
  if constexpr (AS == 2) {
    Frag<T> lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) lo[e] = cvt<T>(gv[e] - tof<T>(hi[e]));
    store_frag<T>(dst + (int64_t)a.Mp * a.F, lo);
  }
}

// gbar (rounded to the storage type, as the forward stores it) times v.
template <typename T>
__device__ __forceinline__ void form_gv(const DecArgs& a, int64_t m, int col, const float (&num)[8], float den,
                                        float (&gv)[8]) {
  const Frag<T> v = load_frag<T>(static_cast<const T*>(a.v) + m * a.F + col);
  const float inv = 1.0f / den;
#pragma unroll
  for (int e = 0; e < 8; ++e) gv[e] = tof<T>(cvt<T>(num[e] * inv)) * tof<T>(v[e]);
}

// ---------------------------------------------------------------------------
// TANGO dcomb: gbar = sum of chunk numerators / (sum of denominators + null).
// ---------------------------------------------------------------------------
template <typename T, int AS>
__global__ __launch_bounds__(256) void dcomb_kernel(DecArgs a) {
  const int64_t b = blockIdx.y;
  const int col = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (col >= a.F) return;
  const int p = a.pos[b];
  float gv[8];
  if (!pos_ok(a, p)) {
#pragma unroll
    for (int e = 0; e < 8; ++e) gv[e] = __builtin_nanf("");
    store_gv<T, AS>(a, b, col, gv);
    return;
  }
  const int h = col / (a.F / a.H);
  const int nc = p / kDecChunk + 1;
  const int64_t stride = a.F + 64;
  const float* part = a.part + b * a.nch * stride;
  float num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
#pragma unroll 4
  for (int c = 0; c < nc; ++c) {
    const f32x4 n0 = *reinterpret_cast<const f32x4*>(part + c * stride + col);
    const f32x4 n1 = *reinterpret_cast<const f32x4*>(part + c * stride + col + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      num[e] += n0[e];
      num[4 + e] += n1[e];
    }
    den += part[c * stride + a.F + h];
  }
  if (a.null_bias) den += (float)(p + 1) * __expf(a.null_bias[h] - tau_of(a.theta, h));
  form_gv<T>(a, b, col, num, den, gv);
  store_gv<T, AS>(a, b, col, gv);
}

// ---------------------------------------------------------------------------
// WANGO dband: workgroup (column block, head, sequence), FB columns of the
// head (FB in {64, 128, 256} dividing F/H).  Threads: CG = FB/8 column groups
// of 8 columns times RG = 256/CG row groups.
// ---------------------------------------------------------------------------
template <typename T, int AS, int FB>
__global__ __launch_bounds__(kBandThreads) void dband_kernel(DecArgs a) {
  constexpr int CG = FB / 8, RG = kBandThreads / CG;
  __shared__ float qs[128], fq[128], fk[128];
  __shared__ float pw[kDecMaxWindow];
  __shared__ float red[RG * FB];
  __shared__ float sred[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cg = tid % CG, rg = tid / CG;
  const int64_t b = blockIdx.z;
  const int h = blockIdx.y, fb = blockIdx.x;
  const int F = a.F, HD = a.HD, H = a.H, dh = a.dh, Fh = F / H, W = a.window;
  const int c8 = fb * FB + cg * 8;                 // first column within the head
  const int col = h * Fh + c8;
  const int p = a.pos[b];
  if (p < 0) {
    if (rg == 0) {
      float gv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) gv[e] = __builtin_nanf("");
      store_gv<T, AS>(a, b, col, gv);
    }
    return;
  }
  const T* kc = static_cast<const T*>(a.kc);
  const T* gc = static_cast<const T*>(a.gc);
  const float tau = tau_of(a.theta, h), stau = sqrtf(tau), isd = 1.0f / sqrtf((float)dh);
  const float escale = __expf(-tau);
  const bool fold = p >= W;                        // token p - W leaves the window
  const int64_t so = fold ? state_row(a, b, p - W) : 0;
  if (tid < dh) {
    const float qv = tof<T>(static_cast<const T*>(a.q)[b * HD + h * dh + tid]);
    qs[tid] = qv;
    fq[tid] = phi_feature(stau * qv, isd);
    fk[tid] = fold ? phi_feature(stau * tof<T>(kc[so * HD + h * dh + tid]), isd) : 0.f;
  }
  __syncthreads();
  // window exp weights, j in [p - nw + 1, p]
  const int nw = min(W, p + 1);
  const int jlo = p - nw + 1;
  for (int t = tid; t < nw; t += kBandThreads) {
    const T* kr = kc + state_row(a, b, jlo + t) * HD + h * dh;
    float s = 0.f;
    for (int e = 0; e < dh; e += 8) {
      const Frag<T> kf = load_frag<T>(kr + e);
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) s += qs[e + s8] * tof<T>(kf[s8]);
    }
    pw[t] = __builtin_amdgcn_exp2f(tau * kLog2e * (s - 1.0f));
  }
  __syncthreads();
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int t = rg; t < nw; t += RG) {
    const Frag<T> g = load_frag<T>(gc + state_row(a, b, jlo + t) * F + col);
    const float w = pw[t];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += w * tof<T>(g[e]);
  }
  if (fold) {
    // S += phi_k g_old^T on this block's columns, then n_old = phi_q^T S
    const Frag<T> go = load_frag<T>(gc + so * F + col);
    float gold[8], nacc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 8; ++e) gold[e] = tof<T>(go[e]);
    const bool fresh = p == W;                     // S held nothing before this step
    float* Sb = a.S + ((b * H + h) * (int64_t)dh) * Fh + c8;
    for (int e = rg; e < dh; e += RG) {
      float* sr = Sb + (int64_t)e * Fh;
      f32x4 s0 = fresh ? f32x4{0.f, 0.f, 0.f, 0.f} : *reinterpret_cast<const f32x4*>(sr);
      f32x4 s1 = fresh ? f32x4{0.f, 0.f, 0.f, 0.f} : *reinterpret_cast<const f32x4*>(sr + 4);
      const float fke = fk[e], fqe = fq[e];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s0[r] += fke * gold[r];
        s1[r] += fke * gold[4 + r];
        nacc[r] += fqe * s0[r];
        nacc[4 + r] += fqe * s1[r];
      }
      *reinterpret_cast<f32x4*>(sr) = s0;
      *reinterpret_cast<f32x4*>(sr + 4) = s1;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += escale * nacc[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg * FB + cg * 8 + e] = acc[e];
  // denominator pieces: window sum (wave 0), phi_q^T z (wave 1)
  if (wave == 0) {
    float s = 0.f;
    for (int t = lane; t < nw; t += 64) s += pw[t];
    s = wave_sum(s);
    if (lane == 0) sred[0] = s;
  } else if (wave == 1) {
    float zq = 0.f;
    if (fold) {
      const bool fresh = p == W;
      const float* zprev = a.z + ((b * 2 + ((p + 1) & 1)) * H + h) * (int64_t)dh;   // after step p - 1
      float* znext = a.z + ((b * 2 + (p & 1)) * H + h) * (int64_t)dh;
      for (int e = lane; e < dh; e += 64) {
        const float zn = (fresh ? 0.f : zprev[e]) + fk[e];
        if (fb == 0) znext[e] = zn;
        zq += fq[e] * zn;
      }
    }
    zq = wave_sum(zq);
    if (lane == 0) sred[1] = zq;
  }
  __syncthreads();
  if (rg == 0) {
    float num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int r2 = 0; r2 < RG; ++r2)
#pragma unroll
      for (int e = 0; e < 8; ++e) num[e] += red[r2 * FB + cg * 8 + e];
    float den = sred[0] + escale * sred[1];
    if (a.null_bias) den += (float)(p + 1) * __expf(a.null_bias[h] - tau);
    float gv[8];
    form_gv<T>(a, b, col, num, den, gv);
    store_gv<T, AS>(a, b, col, gv);
  }
}

// ---------------------------------------------------------------------------
// dout: out = x + (gbar * v) W_o^T.  Workgroup: 16 output columns (rows of
// W_o) x up to 64 tokens; the k-steps of 32 are dealt round robin to the 8
// waves and their accumulators summed through LDS.
// ---------------------------------------------------------------------------
template <typename T, typename IO, int AS>
__global__ __launch_bounds__(kDecThreads) void dout_kernel(DecArgs a) {
  __shared__ f32x4 red[kDecWaves][kDecMT][64];
  const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int F = a.F, d = a.d;
  const int n0 = blockIdx.x * 16;
  const int m0 = blockIdx.y * kDecTokens;
  const T* wr = static_cast<const T*>(a.w_o) + (int64_t)(n0 + li) * F + lg * 8;
  const T* gr = static_cast<const T*>(a.gv) + (int64_t)(m0 + li) * F + lg * 8;
  f32x4 acc[kDecMT];
#pragma unroll
  for (int mt = 0; mt < kDecMT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = wave * 32; k0 < F; k0 += kDecWaves * 32) {
    const Frag<T> A = load_frag<T>(wr + k0);
#pragma unroll
    for (int mt = 0; mt < kDecMT; ++mt)
#pragma unroll
      for (int part = 0; part < AS; ++part)
        mma(acc[mt], A, load_frag<T>(gr + ((int64_t)part * a.Mp + mt * 16) * F + k0));
  }
#pragma unroll
  for (int mt = 0; mt < kDecMT; ++mt) red[wave][mt][lane] = acc[mt];
  __syncthreads();
  if (threadIdx.x < kDecMT * 64) {
    const int mt = threadIdx.x >> 6, l2 = threadIdx.x & 63;
    const int m = m0 + mt * 16 + (l2 & 15);
    if (m < a.B) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w2 = 0; w2 < kDecWaves; ++w2) s += red[w2][mt][l2];
      const int n = n0 + 4 * (l2 >> 4);
      const IO* xr = static_cast<const IO*>(a.x) + (int64_t)m * d + n;
      IO* orow = static_cast<IO*>(a.out) + (int64_t)m * d + n;
      f32x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = tof<IO>(xr[r]) + s[r];
#pragma unroll
      for (int r = 0; r < 4; ++r) orow[r] = cvt<IO>(o[r]);
    }
  }
}

template <typename T, int AS>
hipError_t launch_decode_t(const DecArgs& a, bool io_bf, hipStream_t s) {
  const int N = 2 * a.F + 2 * a.HD;
  const unsigned mg = (unsigned)ceil_div(a.B, kDecTokens);
  hipLaunchKernelGGL((dproj_kernel<T, AS>), dim3((unsigned)ceil_div(N, kDecWaves * 16), mg),
                     dim3(kDecThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.window == 0) {
    hipLaunchKernelGGL((dagg_kernel<T>), dim3((unsigned)a.nch, (unsigned)a.B), dim3(kAggThreadsD), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((dcomb_kernel<T, AS>), dim3((unsigned)ceil_div(a.F, 256 * 8), (unsigned)a.B), dim3(256),
                       0, s, a);
  } else {
    const int Fh = a.F / a.H;
    const dim3 grid3(1, (unsigned)a.H, (unsigned)a.B);
    if (Fh % 256 == 0)
      hipLaunchKernelGGL((dband_kernel<T, AS, 256>), dim3((unsigned)(Fh / 256), grid3.y, grid3.z),
                         dim3(kBandThreads), 0, s, a);
    else if (Fh % 128 == 0)
      hipLaunchKernelGGL((dband_kernel<T, AS, 128>), dim3((unsigned)(Fh / 128), grid3.y, grid3.z),
                         dim3(kBandThreads), 0, s, a);
    else
      hipLaunchKernelGGL((dband_kernel<T, AS, 64>), dim3((unsigned)(Fh / 64), grid3.y, grid3.z),
                         dim3(kBandThreads), 0, s, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const dim3 og((unsigned)(a.d / 16), mg);
  if (io_bf)
    hipLaunchKernelGGL((dout_kernel<T, bf16, AS>), og, dim3(kDecThreads), 0, s, a);
  else
    hipLaunchKernelGGL((dout_kernel<T, float, AS>), og, dim3(kDecThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int decode_parts(bool bf) { return bf ? 2 : 1; }

hipError_t launch_decode(const DecArgs& a, bool bf, bool io_bf, hipStream_t s) {
  return bf ? launch_decode_t<bf16, 2>(a, io_bf, s) : launch_decode_t<float, 1>(a, io_bf, s);
}

}  // namespace tango
