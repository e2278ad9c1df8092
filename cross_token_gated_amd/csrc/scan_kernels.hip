// scan_kernels.hip - WANGO older-prefix running sums on gfx950.
//
// "TANGO: Token-Aggregated Nonlinear Gating Operators ...", §2.2 eqs. 8-10:
// for destination i and head a, the sources older than the window are
// G_i = {j <= i - W}; their weights factor as phi(sqrt(tau) q_i)^T phi(sqrt(tau) k_j)
// with phi(u) = max(ELU(u) + 1 + 1e-4, 1e-4) / sqrt(d_h), so their numerator and
// denominator are read out of the running sums
//     S = sum_{j in G_i} phi(sqrt(tau) k_j) g_j^T   (d_h x F/H)
//     z = sum_{j in G_i} phi(sqrt(tau) k_j)         (d_h)
// as n_old_i = phi_q_i^T S and z_old_i = phi_q_i^T z.
//
// Positions are processed in chunks of CH (CH divides W).  The sources of
// chunk c are the ones that leave the window for the destinations of chunk
// d = c + W/CH; destination i of chunk d sees source j of chunk c exactly when
// j - cCH <= i - dCH.  So, per chunk,
//     n_old(d)^T = S_{<c}^T phi_Q(d)^T + G_c^T tril(phi_Q(d) phi_K(c)^T)^T
//     S += phi_K(c)^T G_c,   z += column sums of phi_K(c).
// The state S lives in MFMA accumulators (one 16-column slice per wave); its
// accumulator layout is used directly as the A operand of the read-out.
//
// The sequence is cut into segments so that many workgroups run at once:
// pass 1 sums every segment's contribution, pass 2 turns those sums into
// exclusive prefixes, pass 3 replays each segment from its prefix.
#include "common.hpp"
#include "kernels.hpp"

namespace tango {

namespace {

constexpr int kScanThreads = 256;   // 4 waves, 16 gate columns each
constexpr int kFSlice = 64;         // gate columns per workgroup

template <typename T> constexpr int pad_of() { return 16 / (int)sizeof(T); }

template <typename T, int DH, int CH> struct ScanLds {
  static constexpr int PK = DH + pad_of<T>();   // row stride of phiK, phiQ  [CH][PK]
  static constexpr int PT = CH + pad_of<T>();   // row stride of phiK^T [DH][PT] and M [CH][PT]
  static constexpr size_t phik = 0;
  static constexpr size_t phikt = phik + (size_t)CH * PK * sizeof(T);
  static constexpr size_t phiq = phikt + (size_t)DH * PT * sizeof(T);
  static constexpr size_t mdc = phiq + (size_t)CH * PK * sizeof(T);
  static constexpr size_t zs = mdc + (size_t)CH * PT * sizeof(T);
  static constexpr size_t bytes = zs + (size_t)DH * sizeof(float);
};

__device__ __forceinline__ float phi_map(float u, float inv_sqrt_dh) {
  const float elu1 = u > 0.f ? u + 1.0f : __expf(u);   // ELU(u) + 1 with alpha = 1
  return fmaxf(elu1 + 1e-4f, 1e-4f) * inv_sqrt_dh;
}

// phi(sqrt(tau) x) of CH rows of a [rows, H*DH] array into LDS, row-major
// ([CH][PK]) and, if dst_t is given, transposed ([DH][PT]).
template <typename T, int DH, int CH>
__device__ __forceinline__ void fill_phi(const T* __restrict__ src, int64_t row0, int HD, int h,
                                         float st, T* dst, T* dst_t) {
  constexpr int PK = ScanLds<T, DH, CH>::PK, PT = ScanLds<T, DH, CH>::PT;
  const float isd = 1.0f / sqrtf((float)DH);
  for (int it = threadIdx.x; it < CH * DH / 4; it += kScanThreads) {
    const int r = it / (DH / 4), c = (it % (DH / 4)) * 4;
    const Quad<T> v = load_quad<T>(src + (row0 + r) * HD + h * DH + c);
    Quad<T> o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = cvt<T>(phi_map(st * tof<T>(v[e]), isd));
    store_quad<T>(dst + r * PK + c, o);
    if (dst_t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) dst_t[(c + e) * PT + r] = o[e];
    }
  }
}

// S (this wave's DH x 16 slice, DH/16 accumulator blocks) += phiK^T G_c.
template <typename T, int DH, int CH>
__device__ __forceinline__ void state_update(f32x4 (&S)[DH / 16], const T* phikt,
                                             const Frag<T> (&gf)[CH / 32], int li, int lg) {
  constexpr int PT = ScanLds<T, DH, CH>::PT;
#pragma unroll
  for (int eb = 0; eb < DH / 16; ++eb)
#pragma unroll
    for (int ks = 0; ks < CH / 32; ++ks) {
      const T* row = phikt + (eb * 16 + li) * PT + ks * 32;
      const Frag<T> af = join(load_quad<T>(row + lg * 4), load_quad<T>(row + 16 + lg * 4));
      mma(S[eb], af, gf[ks]);
    }
}

template <typename T, int CH>
__device__ __forceinline__ void load_gate_frags(Frag<T> (&gf)[CH / 32], const T* __restrict__ gp,
                                                int64_t row0, int64_t col, int F, int lg) {
#pragma unroll
  for (int ks = 0; ks < CH / 32; ++ks) gf[ks] = load_frag<T>(gp + packed_offset(row0 / 32 + ks, lg, col, F));
}

// Pass 1: per-segment sums of phi_K^T G and of phi_K (all segments but the last).
template <typename T, int DH, int CH>
__global__ __launch_bounds__(kScanThreads) void scan_partial_kernel(ScanArgs a) {
  using Ls = ScanLds<T, DH, CH>;
  extern __shared__ __align__(16) unsigned char smem[];
  T* phikt = reinterpret_cast<T*>(smem + Ls::phikt);
  T* phik = reinterpret_cast<T*>(smem + Ls::phik);
  const int Fh = a.F / a.H, nfs = Fh / kFSlice, nseg = a.nseg;
  int64_t id = blockIdx.x;
  const int seg = (int)(id % (nseg - 1)); id /= (nseg - 1);
  const int fsl = (int)(id % nfs); id /= nfs;
  const int h = (int)(id % a.H);
  const int64_t b = id / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, lg = lane >> 4;
  const int HD = a.H * DH;
  const float st = sqrtf(__expf(fminf(a.theta[h], 2.995732273553991f)));
  const int64_t mseq = b * a.Tp;
  const int64_t col = (int64_t)h * Fh + fsl * kFSlice + wave * 16 + li;
  const T* qk = static_cast<const T*>(a.kh);
  const T* gp = static_cast<const T*>(a.gp);

  f32x4 S[DH / 16];
#pragma unroll
  for (int eb = 0; eb < DH / 16; ++eb) S[eb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float zacc = 0.f;

  const int nchunks = a.Tp / CH;
  const int c0 = seg * a.chunks_per_seg;
  const int c1 = min(nchunks, c0 + a.chunks_per_seg);
  for (int c = c0; c < c1; ++c) {
    fill_phi<T, DH, CH>(qk, mseq + (int64_t)c * CH, HD, h, st, phik, phikt);
    Frag<T> gf[CH / 32];
    load_gate_frags<T, CH>(gf, gp, mseq + (int64_t)c * CH, col, a.F, lg);
    __syncthreads();
    state_update<T, DH, CH>(S, phikt, gf, li, lg);
    if (tid < DH) {
      const T* row = phikt + tid * Ls::PT;
      for (int j = 0; j < CH; ++j) zacc += tof<T>(row[j]);
    }
    __syncthreads();
  }
  float* dst = a.seg_state + (((b * a.H + h) * nseg + seg) * (int64_t)DH) * Fh;
#pragma unroll
  for (int eb = 0; eb < DH / 16; ++eb)
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[(int64_t)(eb * 16 + lg * 4 + r) * Fh + (col - (int64_t)h * Fh)] = S[eb][r];
  if (fsl == 0 && tid < DH) a.seg_z[((b * a.H + h) * nseg + seg) * DH + tid] = zacc;
}

// Pass 2: exclusive prefix over segments, in place.  One thread per state element.
__global__ void scan_prefix_kernel(float* state, float* segz, int64_t per_bh, int nseg, int64_t nbh,
                                   int dh) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = nbh * per_bh;
  if (i < total) {
    const int64_t bh = i / per_bh, e = i % per_bh;
    float* p = state + bh * nseg * per_bh + e;
    float run = 0.f;
    for (int s = 0; s + 1 < nseg; ++s) {   // the last segment has no sum of its own
      const float v = p[(int64_t)s * per_bh];
      p[(int64_t)s * per_bh] = run;
      run += v;
    }
    p[(int64_t)(nseg - 1) * per_bh] = run;
  }
  if (i < nbh * dh) {
    const int64_t bh = i / dh, e = i % dh;
    float* p = segz + bh * nseg * dh + e;
    float run = 0.f;
    for (int s = 0; s + 1 < nseg; ++s) {
      const float v = p[(int64_t)s * dh];
      p[(int64_t)s * dh] = run;
      run += v;
    }
    p[(int64_t)(nseg - 1) * dh] = run;
  }
}

// Pass 3: replay each segment from its prefix and emit n_old, z_old.
template <typename T, int DH, int CH>
__global__ __launch_bounds__(kScanThreads) void scan_main_kernel(ScanArgs a) {
  using Ls = ScanLds<T, DH, CH>;
  constexpr int PK = Ls::PK, PT = Ls::PT, NIB = CH / 16, IBW = NIB / 4;  // IBW: dest blocks per wave
  extern __shared__ __align__(16) unsigned char smem[];
  T* phik = reinterpret_cast<T*>(smem + Ls::phik);
  T* phikt = reinterpret_cast<T*>(smem + Ls::phikt);
  T* phiq = reinterpret_cast<T*>(smem + Ls::phiq);
  T* md = reinterpret_cast<T*>(smem + Ls::mdc);
  float* zs = reinterpret_cast<float*>(smem + Ls::zs);

  const int Fh = a.F / a.H, nfs = Fh / kFSlice, nseg = a.nseg;
  int64_t id = blockIdx.x;
  const int seg = (int)(id % nseg); id /= nseg;
  const int fsl = (int)(id % nfs); id /= nfs;
  const int h = (int)(id % a.H);
  const int64_t b = id / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, lg = lane >> 4;
  const int HD = a.H * DH, F = a.F;
  const float st = sqrtf(__expf(fminf(a.theta[h], 2.995732273553991f)));
  const int64_t mseq = b * a.Tp;
  const int64_t fcol0 = (int64_t)h * Fh + fsl * kFSlice + wave * 16;   // this wave's 16 columns
  const T* qh = static_cast<const T*>(a.qh);
  const T* kh = static_cast<const T*>(a.kh);
  const T* gp = static_cast<const T*>(a.gp);
  const int nchunks = a.Tp / CH, lag = a.window / CH;
  const int c0 = seg * a.chunks_per_seg;
  const int c1 = min(nchunks, c0 + a.chunks_per_seg);

  // state prefix of this segment
  f32x4 S[DH / 16];
  {
    const float* src = a.seg_state + (((b * a.H + h) * nseg + seg) * (int64_t)DH) * Fh;
#pragma unroll
    for (int eb = 0; eb < DH / 16; ++eb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S[eb][r] = seg == 0 ? 0.f : src[(int64_t)(eb * 16 + lg * 4 + r) * Fh + (fcol0 - (int64_t)h * Fh) + li];
  }
  if (tid < DH) zs[tid] = seg == 0 ? 0.f : a.seg_z[((b * a.H + h) * nseg + seg) * DH + tid];

  // destinations with no older source: zeros
  if (seg == 0) {
    const int zc = min(lag, nchunks);
    for (int dchunk = 0; dchunk < zc; ++dchunk) {
#pragma unroll
      for (int ib = 0; ib < NIB; ++ib) {
        const int64_t nblk = ((mseq + (int64_t)dchunk * CH) / 16 + ib) * (F / 16) + fcol0 / 16;
        *reinterpret_cast<f32x4*>(a.n_old + (nblk * 64 + lane) * 4) = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if (fsl == 0)
        for (int r = tid; r < CH; r += kScanThreads) a.z_old[(mseq + (int64_t)dchunk * CH + r) * a.H + h] = 0.f;
    }
  }
  __syncthreads();

  for (int c = c0; c < c1; ++c) {
    const int dchunk = c + lag;
    const bool has_dest = dchunk < nchunks;
    const int64_t srow = mseq + (int64_t)c * CH, drow = mseq + (int64_t)dchunk * CH;
    fill_phi<T, DH, CH>(kh, srow, HD, h, st, phik, phikt);
    if (has_dest) fill_phi<T, DH, CH>(qh, drow, HD, h, st, phiq, nullptr);
    Frag<T> gf[CH / 32];
    load_gate_frags<T, CH>(gf, gp, srow, fcol0 + li, F, lg);
    __syncthreads();

    if (has_dest) {
      // M^T blocks: this wave's two destination blocks against all source blocks;
      // masked, rounded, stored as M[i][j]; row sums kept for z_old.
      float msum[IBW];
#pragma unroll
      for (int ii = 0; ii < IBW; ++ii) {
        msum[ii] = 0.f;
        const int ib = IBW * wave + ii;
        Frag<T> qf[DH / 32];
#pragma unroll
        for (int ks = 0; ks < DH / 32; ++ks) qf[ks] = load_frag<T>(phiq + (ib * 16 + li) * PK + ks * 32 + lg * 8);
#pragma unroll
        for (int jb = 0; jb < NIB; ++jb) {
          f32x4 m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < DH / 32; ++ks) {
            const Frag<T> kf = load_frag<T>(phik + (jb * 16 + li) * PK + ks * 32 + lg * 8);
            mma(m, kf, qf[ks]);
          }
          Quad<T> mq;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int jl = jb * 16 + lg * 4 + r, il = ib * 16 + li;
            mq[r] = cvt<T>(jl <= il ? m[r] : 0.f);
            msum[ii] += tof<T>(mq[r]);
          }
          store_quad<T>(md + (ib * 16 + li) * PT + jb * 16 + lg * 4, mq);
        }
      }
      __syncthreads();
      // z_old = phi_q . z + row sums of M  (written once per (b, h) by slice 0)
      if (fsl == 0) {
#pragma unroll
        for (int ii = 0; ii < IBW; ++ii) {
          const int ib = IBW * wave + ii;
          const int il = ib * 16 + li;
          float dot = 0.f;
          for (int e = lg; e < DH; e += 4) dot += tof<T>(phiq[il * PK + e]) * zs[e];
          const float tot = group_sum(dot) + group_sum(msum[ii]);
          if (lg == 0) a.z_old[(drow + il) * a.H + h] = tot;
        }
      }
      // n_old^T = S^T phi_Q^T + G_c^T M^T for this wave's 16 columns
#pragma unroll
      for (int ib = 0; ib < NIB; ++ib) {
        f32x4 n = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DH / 32; ++ks) {
          const Frag<T> sa = join(cvt_quad<T>(S[2 * ks]), cvt_quad<T>(S[2 * ks + 1]));
          const T* qrow = phiq + (ib * 16 + li) * PK + ks * 32;
          const Frag<T> qb = join(load_quad<T>(qrow + lg * 4), load_quad<T>(qrow + 16 + lg * 4));
          mma(n, sa, qb);
        }
#pragma unroll
        for (int ks = 0; ks < CH / 32; ++ks) {
          const T* mrow = md + (ib * 16 + li) * PT + ks * 32;
          const Frag<T> mb = join(load_quad<T>(mrow + lg * 4), load_quad<T>(mrow + 16 + lg * 4));
          mma(n, gf[ks], mb);
        }
        const int64_t nblk = (drow / 16 + ib) * (F / 16) + fcol0 / 16;
        *reinterpret_cast<f32x4*>(a.n_old + (nblk * 64 + lane) * 4) = n;
      }
    }
    // S += phi_K^T G_c ;  z += column sums of phi_K
    state_update<T, DH, CH>(S, phikt, gf, li, lg);
    __syncthreads();
    if (tid < DH) {
      const T* row = phikt + tid * PT;
      float acc = 0.f;
      for (int j = 0; j < CH; ++j) acc += tof<T>(row[j]);
      zs[tid] += acc;
    }
    __syncthreads();
  }
}

template <typename T, int DH, int CH>
hipError_t launch_scan_t(const ScanArgs& a, hipStream_t s) {
  using Ls = ScanLds<T, DH, CH>;
  const int Fh = a.F / a.H;
  const int64_t groups = (int64_t)a.B * a.H * (Fh / kFSlice);
  if (a.nseg > 1) {
    hipLaunchKernelGGL((scan_partial_kernel<T, DH, CH>), dim3((unsigned)(groups * (a.nseg - 1))),
                       dim3(kScanThreads), Ls::bytes, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t per_bh = (int64_t)DH * Fh, nbh = (int64_t)a.B * a.H;
    const int64_t n = nbh * per_bh;
    hipLaunchKernelGGL(scan_prefix_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s,
                       a.seg_state, a.seg_z, per_bh, a.nseg, nbh, DH);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((scan_main_kernel<T, DH, CH>), dim3((unsigned)(groups * a.nseg)),
                     dim3(kScanThreads), Ls::bytes, s, a);
  return hipGetLastError();
}

template <typename T, int CH>
hipError_t launch_scan_dh(const ScanArgs& a, hipStream_t s) {
  switch (a.dh) {
    case 32: return launch_scan_t<T, 32, CH>(a, s);
    case 64: return launch_scan_t<T, 64, CH>(a, s);
    case 128: return launch_scan_t<T, 128, CH>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int DH, int CH>
hipError_t set_attr_scan() {
  using Ls = ScanLds<T, DH, CH>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&scan_main_kernel<T, DH, CH>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)Ls::bytes);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&scan_partial_kernel<T, DH, CH>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)Ls::bytes);
}

}  // namespace

// Internal chunk: the requested chunk for bf16; 64 for float32 (LDS budget).
static int internal_chunk(int chunk, bool bf) { return bf ? chunk : 64; }

ScanPlan wango_scan_plan(int B, int Tp, int F, int H, int chunk, int window, bool bf) {
  (void)window;
  ScanPlan p;
  const int ch = internal_chunk(chunk, bf);
  const int nchunks = Tp / ch;
  const int64_t groups = (int64_t)B * H * ((F / H) / kFSlice);
  int64_t nseg = ceil_div(512, groups);
  if (nseg < 1) nseg = 1;
  if (nseg > nchunks) nseg = nchunks;
  p.chunks_per_seg = (int)ceil_div(nchunks, nseg);
  p.nseg = (int)ceil_div(nchunks, p.chunks_per_seg);
  p.fs = kFSlice;
  return p;
}

hipError_t launch_wango_scan(const ScanArgs& a, const ScanPlan& p, bool bf, hipStream_t s) {
  ScanArgs aa = a;
  aa.nseg = p.nseg;
  aa.chunks_per_seg = p.chunks_per_seg;
  const int ch = internal_chunk(a.chunk, bf);
  aa.chunk = ch;
  if (bf) return ch == 128 ? launch_scan_dh<bf16, 128>(aa, s) : launch_scan_dh<bf16, 64>(aa, s);
  return launch_scan_dh<float, 64>(aa, s);
}

hipError_t scan_kernels_init() {
  hipError_t e;
#define TANGO_SET(T, DH, CH) \
  if ((e = set_attr_scan<T, DH, CH>()) != hipSuccess) return e;
  TANGO_SET(bf16, 32, 64) TANGO_SET(bf16, 64, 64) TANGO_SET(bf16, 128, 64)
  TANGO_SET(bf16, 32, 128) TANGO_SET(bf16, 64, 128) TANGO_SET(bf16, 128, 128)
  TANGO_SET(float, 32, 64) TANGO_SET(float, 64, 64) TANGO_SET(float, 128, 64)
#undef TANGO_SET
  return hipSuccess;
}

}  // namespace tango
