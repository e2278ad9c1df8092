// decode_kernels.hip - one autoregressive decode step of the TANGO / WANGO
// block on gfx950.
//
// "TANGO: Token-Aggregated Nonlinear Gating Operators ...": a decode step gives
// the block output (§2.1 eqs. 2-5 and 3) at the next position p of every
// sequence from a state kept between steps.  TANGO keeps every unit key and
// gate so far (eq. 6 sums over the whole prefix).  WANGO keeps the running sums
// S, z of §2.2 eq. 10 -- when p advances, the key and gate at p - W join S and
// z -- and the keys and gates of the last W + 1 positions, a state whose size
// does not depend on the position (§6.1).
//
// One step of one block is four or five launches on the caller's stream:
//   prep  (the forward's row-prep kernel) RMSNorm scale, operand parts of h*gain;
//   dproj the projections of the new tokens as a skinny MFMA GEMM; SiLU gates
//         and RoPE-rotated keys go straight into the state at the token's
//         position, features and rotated queries to scratch (queries and keys
//         are normalised where they are read);
//   TANGO dagg  streams the key/gate cache in chunks of kChunk positions: exp
//               weights e^{tau (s - 1)} (static shift: |s| <= 1), float32
//               partial numerators and denominators per chunk;
//         dcomb adds the chunk partials, divides, forms gbar * v;
//   WANGO dband per (sequence, head, column block): adds the leaving token to S
//               and z, reads phi_q^T S out, adds the window's exp-weighted
//               gates, divides, forms gbar * v;
//   dout  out = x + (gbar * v) W_o^T as a skinny MFMA GEMM, K split over
//         workgroups and waves.
// The two GEMMs deal their k-steps to the 8 waves of a workgroup so that every
// load is in flight at once, and take as many 16-token tiles as the batch needs.
// The older-prefix terms carry the same e^{-tau} factor as the window weights,
// so the shift cancels in the ratio (as in the forward kernels).
#include "common.hpp"
#include "kernels.hpp"

namespace tango {

namespace {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
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

// acc[mt] += W[16 rows, k] X[16 tokens of tile mt, k]^T over `steps` k-steps of
// 32 starting at k_first, k_stride apart.  wr and xr point at this lane's row
// and first k-slot; the AS operand parts of X are part_stride elements apart.
// The k-steps go in batches of NB whose loads are all issued before the first
// product; a batch past the last step reloads the last step and multiplies it
// by a zeroed A, so there is no branch for the compiler to wait at.
template <typename T, int NT, int MT, int AS, int NB>
__device__ __forceinline__ void skinny_mma(f32x4 (&acc)[NT][MT], const T* wr, int64_t w_row16, const T* xr,
                                           int64_t x_row16, int64_t part_stride, int k_first, int k_stride,
                                           int steps) {
  for (int s0 = 0; s0 < steps; s0 += NB) {
    Frag<T> A[NB][NT], X[NB][MT][AS];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int k0 = k_first + min(s0 + u, steps - 1) * k_stride;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) A[u][nt] = load_frag<T>(wr + nt * w_row16 + k0);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int part = 0; part < AS; ++part) X[u][mt][part] = load_frag<T>(xr + part * part_stride + mt * x_row16 + k0);
    }
    // keep the loads ahead of the products: the scheduler would otherwise pair
    // each load with its product and wait for them one at a time
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const bool live = s0 + u < steps;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const Frag<T> Au = live ? A[u][nt] : Frag<T>{};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int part = 0; part < AS; ++part) mma(acc[nt][mt], Au, X[u][mt][part]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dproj: [g | v | q | k] rows of the new tokens.  Workgroup: 16 rows of the
// stacked [W_g; W_v; W_q; W_k] (NT tiles of 16; the class boundaries F, 2F and
// 2F + HD are multiples of 32, so a 32-row block never straddles two weights)
// against MT tiles of 16 tokens; the k-steps of 32
// are dealt round robin to the 8 waves, each of which has all of its loads in
// flight at once, and the accumulators are summed through LDS.  Queries and
// keys leave with RoPE applied but not normalised (a head's norm would span
// several workgroups): the aggregation kernels normalise them on read.
// ---------------------------------------------------------------------------
template <typename T, int AS, int MT, int NT>
__global__ __launch_bounds__(kDecThreads) void dproj_kernel(DecArgs a) {
  static_assert(NT * MT <= kDecWaves, "one (row tile, token tile) pair per wave in the epilogue");
  __shared__ f32x4 red[kDecWaves][NT * MT][64];
  const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int F = a.F, HD = a.HD, d = a.d;
  const int nb0 = blockIdx.x * NT * 16;             // N = 2F + 2HD is a multiple of 16 NT
  const int m0 = blockIdx.y * MT * 16;
  const int cls = nb0 < F ? 0 : nb0 < 2 * F ? 1 : nb0 < 2 * F + HD ? 2 : 3;
  const int wrow = cls == 0 ? nb0 : cls == 1 ? nb0 - F : cls == 2 ? nb0 - 2 * F : nb0 - 2 * F - HD;
  const T* W = static_cast<const T*>(cls == 0 ? a.w_g : cls == 1 ? a.w_v : cls == 2 ? a.w_q : a.w_k);
  const T* xs = static_cast<const T*>(a.xs);

  f32x4 acc[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nks = d / 32;
  skinny_mma<T, NT, MT, AS, 2>(acc, W + (int64_t)(wrow + li) * d + lg * 8, (int64_t)16 * d,
                               xs + (int64_t)(m0 + li) * d + lg * 8, (int64_t)16 * d, (int64_t)a.Mp * d, wave * 32,
                               kDecWaves * 32, (nks - wave + kDecWaves - 1) / kDecWaves);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[wave][nt * MT + mt][lane] = acc[nt][mt];
  __syncthreads();
  if (threadIdx.x >= NT * MT * 64) return;
  // thread (nt, mt, l2) holds rows n0 + 4 lg2 + r of token m0 + 16 mt + li2
  const int pr = threadIdx.x >> 6, l2 = threadIdx.x & 63, li2 = l2 & 15, lg2 = l2 >> 4;
  const int mt = pr % MT, n0 = nb0 + (pr / MT) * 16;
  const int m = m0 + mt * 16 + li2;
  if (m >= a.B) return;
  f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w2 = 0; w2 < kDecWaves; ++w2) sum += red[w2][pr][l2];
  const float rs = a.rinv[m];
  float val[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) val[r] = sum[r] * rs;
  const int p = a.pos[m];
  const int col = n0 + 4 * lg2;
  if (cls == 0) {
    if (pos_ok(a, p)) {
      f32x4 g;
#pragma unroll
      for (int r = 0; r < 4; ++r) g[r] = silu_f(val[r]);
      store_quad<T>(static_cast<T*>(a.gc) + state_row(a, m, p) * F + col, cvt_quad<T>(g));
    }
    return;
  }
  if (cls == 1) {
    store_quad<T>(static_cast<T*>(a.v) + (int64_t)m * F + col - F, cvt_quad<T>(f32x4{val[0], val[1], val[2], val[3]}));
    return;
  }
  // queries and keys: RoPE on the pairs (4 lg2, 4 lg2 + 1), (4 lg2 + 2, 4 lg2 + 3)
  const int e0 = col - (cls == 2 ? 2 * F : 2 * F + HD);   // column within q or k
  if (a.rope_base > 0.f) {
    const int c0 = (e0 % a.dh) / 2;
    // rotation rate of pair c in revolutions per position (float64: a float32
    // angle at large positions would be off by ~1e-3 rad)
    const double pp = (double)max(p, 0);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const double f = pow((double)a.rope_base, -2.0 * (c0 + h2) / a.dh) * 0.15915494309189533577;
      const double rev = pp * f;
      const float fr = (float)(rev - rint(rev));
      const float fs = __builtin_amdgcn_sinf(fr), fc = __builtin_amdgcn_cosf(fr);
      const float u0 = val[2 * h2], u1 = val[2 * h2 + 1];
      val[2 * h2] = u0 * fc - u1 * fs;
      val[2 * h2 + 1] = u0 * fs + u1 * fc;
    }
  }
  const Quad<T> u = cvt_quad<T>(f32x4{val[0], val[1], val[2], val[3]});
  if (cls == 2)
    store_quad<T>(static_cast<T*>(a.q) + (int64_t)m * HD + e0, u);
  else if (pos_ok(a, p))
    store_quad<T>(static_cast<T*>(a.kc) + state_row(a, m, p) * HD + e0, u);
}

// ---------------------------------------------------------------------------
// TANGO dagg: chunk c of sequence b, sources j in [c kChunk, min(c kChunk +
// kChunk, p + 1)).  Partial numerators [F] and denominators [H] in float32,
// row stride F + 64 floats.
// All workgroups of a step are resident at once, so the kernel takes about
// as long as one workgroup's chain of memory round trips: each key row is
// read by two lanes (half of d_h each) with all of their loads issued
// together, and each thread keeps 16 gate rows in flight.
// ---------------------------------------------------------------------------
template <typename T, int DH>
__global__ __launch_bounds__(kAggThreadsD) void dagg_kernel(DecArgs a) {
  constexpr int HALF = DH / 2, NF = HALF / 8, GB = 16;
  __shared__ float qs[1024];
  __shared__ float pw[kDecChunk * 32];
  __shared__ float qinv[32];
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.y;
  const int c = blockIdx.x;
  const int p = a.pos[b];
  if (!pos_ok(a, p)) return;
  const int j0 = c * kDecChunk;
  if (j0 > p) return;
  const int nj = min(kDecChunk, p + 1 - j0);
  const int F = a.F, HD = a.HD, H = a.H, Fh = F / H;
  const T* kc = static_cast<const T*>(a.kc);
  const T* gc = static_cast<const T*>(a.gc);
  for (int i = tid; i < HD; i += kAggThreadsD) qs[i] = tof<T>(static_cast<const T*>(a.q)[b * HD + i]);
  __syncthreads();
  if (tid < H) {
    float ss = 0.f;
    for (int e = 0; e < DH; ++e) ss += qs[tid * DH + e] * qs[tid * DH + e];
    qinv[tid] = 1.0f / fmaxf(sqrtf(ss), 1e-12f);   // unit query ([TANGO] §2.1)
  }
  __syncthreads();
  // exp weights, one (source, head) item per pair of lanes and pass; s = q.k / |q| |k|
  // (zero weight for sources past the chunk's end)
  const int n_items = kDecChunk * H, part = tid & 1;
  for (int it0 = 0; it0 < n_items; it0 += kAggThreadsD / 2) {
    const int it = it0 + (tid >> 1);
    const int jl = it / H, h = it - (it / H) * H;
    const bool live = it < n_items && jl < nj;
    float s = 0.f, kk = 0.f;
    if (live) {
      const T* kr = kc + (b * a.P + j0 + jl) * HD + h * DH + part * HALF;
      Frag<T> kf[NF];
#pragma unroll
      for (int q = 0; q < NF; ++q) kf[q] = load_frag<T>(kr + q * 8);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < NF; ++q)
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
          const float kv = tof<T>(kf[q][s8]);
          s += qs[h * DH + part * HALF + q * 8 + s8] * kv;
          kk += kv * kv;
        }
    }
    s += __shfl_xor(s, 1, 64);
    kk += __shfl_xor(kk, 1, 64);
    if (part == 0 && it < n_items) {
      float w = 0.f;
      if (live) {
        const float sn = s * qinv[h] / fmaxf(sqrtf(kk), 1e-12f);
        w = __builtin_amdgcn_exp2f(tau_of(a.theta, h) * kLog2e * (sn - 1.0f));
      }
      pw[jl * H + h] = w;
    }
  }
  __syncthreads();
  float* part_out = a.part + ((int64_t)b * a.nch + c) * (F + 64);
  for (int f0 = 0; f0 < F; f0 += kAggThreadsD * 8) {
    const int col = f0 + tid * 8;
    if (col < F) {
      const int h = col / Fh;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const T* gr = gc + (b * a.P + j0) * F + col;
      // all kDecChunk rows in batches of GB loads; rows past the chunk's end
      // re-read its last row and carry weight zero
      for (int jb = 0; jb < kDecChunk; jb += GB) {
        Frag<T> g[GB];
#pragma unroll
        for (int u = 0; u < GB; ++u) g[u] = load_frag<T>(gr + (int64_t)min(jb + u, nj - 1) * F);
        // keep the batch together: left alone, the compiler issues one load per
        // wait to save VGPRs for occupancy, which serialises the round trips
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < GB; ++u) {
          const float w = pw[(jb + u) * H + h];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += w * tof<T>(g[u][e]);
        }
      }
      *reinterpret_cast<f32x4*>(part_out + col) = f32x4{acc[0], acc[1], acc[2], acc[3]};
      *reinterpret_cast<f32x4*>(part_out + col + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    }
  }
  if (tid < H) {
    float s = 0.f;
    for (int jl = 0; jl < nj; ++jl) s += pw[jl * H + tid];
    part_out[F + tid] = s;
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
// Workgroup: 256 columns of one sequence; 32 column groups of 8 x 8 chunk
// groups, summed through LDS.
// ---------------------------------------------------------------------------
constexpr int kCombCols = 256, kCombGroups = 8;
template <typename T, int AS>
__global__ __launch_bounds__(256) void dcomb_kernel(DecArgs a) {
  __shared__ float red[kCombGroups][kCombCols];
  __shared__ float rden[kCombGroups][32];       // per column group: a block may span heads
  const int64_t b = blockIdx.y;
  const int cgp = threadIdx.x & 31, chg = threadIdx.x >> 5;
  const int col = blockIdx.x * kCombCols + cgp * 8;
  const int p = a.pos[b];
  const bool ok = pos_ok(a, p);
  const int h = col / (a.F / a.H);
  const int nc = ok ? p / kDecChunk + 1 : 0;
  const int64_t stride = a.F + 64;
  const float* part = a.part + b * a.nch * stride;
  float num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (col < a.F) {
    // every load of this thread's chunks in flight at once, in batches of 8
    for (int c0 = chg; c0 < nc; c0 += 8 * kCombGroups) {
      f32x4 n0[8], n1[8];
      float dn[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = min(c0 + u * kCombGroups, nc - 1);
        n0[u] = *reinterpret_cast<const f32x4*>(part + c * stride + col);
        n1[u] = *reinterpret_cast<const f32x4*>(part + c * stride + col + 4);
        dn[u] = part[c * stride + a.F + h];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float keep = c0 + u * kCombGroups < nc ? 1.f : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          num[e] += keep * n0[u][e];
          num[4 + e] += keep * n1[u][e];
        }
        den += keep * dn[u];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[chg][cgp * 8 + e] = num[e];
  rden[chg][cgp] = den;
  __syncthreads();
  if (chg == 0 && col < a.F) {
    float gv[8];
    if (!ok) {
#pragma unroll
      for (int e = 0; e < 8; ++e) gv[e] = __builtin_nanf("");
    } else {
      float tot[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, dt = 0.f;
      for (int g2 = 0; g2 < kCombGroups; ++g2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) tot[e] += red[g2][cgp * 8 + e];
        dt += rden[g2][cgp];
      }
      if (a.null_bias) dt += (float)(p + 1) * __expf(a.null_bias[h] - tau_of(a.theta, h));
      form_gv<T>(a, b, col, tot, dt, gv);
    }
    store_gv<T, AS>(a, b, col, gv);
  }
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
  if (wave < 2) {
    // wave 0: the unit query and its features; wave 1: the features of the
    // leaving token's unit key (d_h <= 128: two elements a lane)
    const T* src = wave == 0 ? static_cast<const T*>(a.q) + b * HD + h * dh : kc + so * HD + h * dh;
    const bool on = wave == 0 || fold;
    const float u0 = on && lane < dh ? tof<T>(src[lane]) : 0.f;
    const float u1 = on && lane + 64 < dh ? tof<T>(src[lane + 64]) : 0.f;
    const float inv = 1.0f / fmaxf(sqrtf(wave_sum(u0 * u0 + u1 * u1)), 1e-12f);
    float* feat = wave == 0 ? fq : fk;
    if (lane < dh) {
      if (wave == 0) qs[lane] = u0 * inv;
      feat[lane] = on ? phi_feature(stau * u0 * inv, isd) : 0.f;
    }
    if (lane + 64 < dh) {
      if (wave == 0) qs[lane + 64] = u1 * inv;
      feat[lane + 64] = on ? phi_feature(stau * u1 * inv, isd) : 0.f;
    }
  }
  __syncthreads();
  // window exp weights, j in [p - nw + 1, p]; s = q.k / |k| with the unit query
  const int nw = min(W, p + 1);
  const int jlo = p - nw + 1;
  for (int t = tid; t < nw; t += kBandThreads) {
    const T* kr = kc + state_row(a, b, jlo + t) * HD + h * dh;
    float s = 0.f, kk = 0.f;
    for (int e = 0; e < dh; e += 8) {
      const Frag<T> kf = load_frag<T>(kr + e);
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) {
        const float kv = tof<T>(kf[s8]);
        s += qs[e + s8] * kv;
        kk += kv * kv;
      }
    }
    s /= fmaxf(sqrtf(kk), 1e-12f);
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
// W_o) x MT tiles of 16 tokens x one of kOutSplit quarters of K; its k-steps
// of 32 are dealt round robin to the 8 waves (all loads in flight at once) and
// summed through LDS.  The quarters meet through float32 partials: the last
// workgroup of a tile to finish (an atomic counter, cleared by the row-prep
// kernel of the same step) adds them in a fixed order, so the result does not
// depend on which finished first.  The partials and the counter use
// agent-scope atomic stores and loads (coherent across the XCD L2s).
// ---------------------------------------------------------------------------
template <typename T, typename IO, int AS, int MT>
__global__ __launch_bounds__(kDecThreads) void dout_kernel(DecArgs a) {
  __shared__ f32x4 red[kDecWaves][MT][64];
  __shared__ int last;
  const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int F = a.F, d = a.d;
  const int n0 = blockIdx.x * 16;
  const int m0 = blockIdx.y * MT * 16;
  const int kq = blockIdx.z;
  const int nks = F / 32;
  const int ks0 = kq * nks / kOutSplit, ks1 = (kq + 1) * nks / kOutSplit;
  f32x4 acc[1][MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[0][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  skinny_mma<T, 1, MT, AS, 2>(acc, static_cast<const T*>(a.w_o) + (int64_t)(n0 + li) * F + lg * 8, 0,
                              static_cast<const T*>(a.gv) + (int64_t)(m0 + li) * F + lg * 8, (int64_t)16 * F,
                              (int64_t)a.Mp * F, (ks0 + wave) * 32, kDecWaves * 32,
                              (ks1 - ks0 - wave + kDecWaves - 1) / kDecWaves);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) red[wave][mt][lane] = acc[0][mt];
  __syncthreads();
  const int mt = threadIdx.x >> 6, l2 = threadIdx.x & 63;
  const int m = m0 + mt * 16 + (l2 & 15);
  const int n = n0 + 4 * (l2 >> 4);
  // partial of this quarter: [kOutSplit][Mp][d] float32
  float* opart = a.opart + ((int64_t)kq * a.Mp + m) * d + n;
  if (threadIdx.x < MT * 64) {
    f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w2 = 0; w2 < kDecWaves; ++w2) s4 += red[w2][mt][l2];
#pragma unroll
    for (int r = 0; r < 4; ++r) __hip_atomic_store(opart + r, s4[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(a.ocount + blockIdx.y * gridDim.x + blockIdx.x, 1, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT) == kOutSplit - 1;
  __syncthreads();
  if (!last || threadIdx.x >= MT * 64 || m >= a.B) return;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int q2 = 0; q2 < kOutSplit; ++q2) {
    const float* src = a.opart + ((int64_t)q2 * a.Mp + m) * d + n;
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] += __hip_atomic_load(src + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const IO* xr = static_cast<const IO*>(a.x) + (int64_t)m * d + n;
  IO* orow = static_cast<IO*>(a.out) + (int64_t)m * d + n;
  float o[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) o[r] = tof<IO>(xr[r]) + s[r];
#pragma unroll
  for (int r = 0; r < 4; ++r) orow[r] = cvt<IO>(o[r]);
}

template <typename T, int AS, int MT>
hipError_t launch_decode_mt(const DecArgs& a, bool io_bf, hipStream_t s) {
  const int N = 2 * a.F + 2 * a.HD;
  const unsigned mg = (unsigned)ceil_div(a.B, MT * 16);
  // 32 weight rows per workgroup: half the workgroups (N / 16 would overrun
  // one round of the 256 CUs at the usual widths) and half the re-reads of the
  // tokens' operand parts per weight row.
  hipLaunchKernelGGL((dproj_kernel<T, AS, MT, 2>), dim3((unsigned)(N / 32), mg), dim3(kDecThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.window == 0) {
    const dim3 ga((unsigned)a.nch, (unsigned)a.B);
    switch (a.dh) {
      case 32: hipLaunchKernelGGL((dagg_kernel<T, 32>), ga, dim3(kAggThreadsD), 0, s, a); break;
      case 64: hipLaunchKernelGGL((dagg_kernel<T, 64>), ga, dim3(kAggThreadsD), 0, s, a); break;
      case 128: hipLaunchKernelGGL((dagg_kernel<T, 128>), ga, dim3(kAggThreadsD), 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((dcomb_kernel<T, AS>), dim3((unsigned)ceil_div(a.F, kCombCols), (unsigned)a.B), dim3(256),
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
  const dim3 og((unsigned)(a.d / 16), mg, kOutSplit);
  if (io_bf)
    hipLaunchKernelGGL((dout_kernel<T, bf16, AS, MT>), og, dim3(kDecThreads), 0, s, a);
  else
    hipLaunchKernelGGL((dout_kernel<T, float, AS, MT>), og, dim3(kDecThreads), 0, s, a);
  return hipGetLastError();
}

// Token tiles per workgroup of the two GEMMs: as few as the batch needs.
template <typename T, int AS>
hipError_t launch_decode_t(const DecArgs& a, bool io_bf, hipStream_t s) {
  if (a.B <= 16) return launch_decode_mt<T, AS, 1>(a, io_bf, s);
  if (a.B <= 32) return launch_decode_mt<T, AS, 2>(a, io_bf, s);
  return launch_decode_mt<T, AS, 4>(a, io_bf, s);
}

}  // namespace

int decode_parts(bool bf) { return bf ? 2 : 1; }

hipError_t launch_decode(const DecArgs& a, bool bf, bool io_bf, hipStream_t s) {
  return bf ? launch_decode_t<bf16, 2>(a, io_bf, s) : launch_decode_t<float, 1>(a, io_bf, s);
}

}  // namespace tango
