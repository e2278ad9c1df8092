// scan_kernels.hip - WANGO older-prefix running sums on gfx950.
//
// "TANGO: Token-Aggregated Nonlinear Gating Operators ...", §2.2 eqs. 8-10:
// the sources older than the window of destination i are G_i = {j <= i - W};
// their weights factor as phi(sqrt(tau) q_i)^T phi(sqrt(tau) k_j), so their
// numerator and denominator are read out of running sums
//     S = sum_j phi(sqrt(tau) k_j) g_j^T   (d_h x F/H),   z = sum_j phi(sqrt(tau) k_j).
//
// Positions are taken in chunks of CH (CH divides W).  Source chunk c holds
// the sources that leave the window for destination chunk d = c + W/CH.  This
// kernel emits, for every destination i, the read-out of the state at the
// chunk boundary,
//     n_old_i = phi_q_i^T S_{<cCH},   z_old_i = phi_q_i^T z_{<cCH},
// and the window-band kernel adds the remaining older sources of chunk c
// (cCH <= j <= i - W) as pairwise phi weights next to its exp weights: it
// visits exactly those source positions anyway.
//
// The features phi(sqrt(tau) q) and phi(sqrt(tau) k) come from the projection
// kernel: keys source-packed (the A operand of the state update
// S += phi_K^T G), queries in the permuted feature order (the B operand of the
// read-out n_old^T = S^T phi_Q^T, whose A operand is the state accumulator
// itself).  No LDS is used.  z rides along as the state of a column of ones,
// kept by one wave per (sequence, head).
//
// The sequence is cut into segments so that many workgroups run at once:
// pass 1 sums every segment's contribution, pass 2 turns the sums into
// exclusive prefixes, pass 3 replays each segment from its prefix.
#include "common.hpp"
#include "kernels.hpp"

namespace tango {

namespace {

constexpr int kScanWaves = 4;
constexpr int kScanThreads = 64 * kScanWaves;

template <typename T> __device__ __forceinline__ Frag<T> ones_frag() {
  Frag<T> f;
#pragma unroll
  for (int s = 0; s < 8; ++s) f[s] = cvt<T>(1.0f);
  return f;
}

// Workgroup decode: (b, h, column slice of kScanWaves * 16 * NFB, segment).
struct ScanWg {
  int64_t b;
  int h, fsl, seg;
};
__device__ __forceinline__ ScanWg scan_wg(int64_t id, int nslices, int H, int nsegs) {
  ScanWg w;
  w.seg = (int)(id % nsegs);
  id /= nsegs;
  w.fsl = (int)(id % nslices);
  id /= nslices;
  w.h = (int)(id % H);
  w.b = id / H;
  return w;
}

// A unit of sources in registers: the gate fragments of this wave's columns
// and the key-feature fragments (A operand of S += phi_K^T G).  Loads run one
// unit ahead of the MFMAs; the unit is 64 sources, 32 for d_h = 128 (whose
// key fragments are twice as many registers).
template <int DH> constexpr int unit_len() { return DH >= 128 ? 32 : 64; }
template <typename T, int DH, int NFB> struct UnitRegs {
  static constexpr int U = unit_len<DH>();
  Frag<T> g[U / 32][NFB];
  Frag<T> k[U / 32][DH / 16];
};

template <typename T, int DH, int NFB>
__device__ __forceinline__ void load_unit(UnitRegs<T, DH, NFB>& c, const T* __restrict__ fk,
                                          const T* __restrict__ gp, int64_t row0, int HD, int hcol,
                                          int64_t col, int F, int li, int lg) {
#pragma unroll
  for (int ks = 0; ks < unit_len<DH>() / 32; ++ks) {
    const int64_t blk = row0 / 32 + ks;
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb) c.g[ks][fb] = load_frag<T>(gp + packed_offset(blk, lg, col + fb * 16 + li, F));
#pragma unroll
    for (int eb = 0; eb < DH / 16; ++eb) c.k[ks][eb] = load_frag<T>(fk + packed_offset(blk, lg, hcol + eb * 16 + li, HD));
  }
}

// S (this wave's DH x 16*NFB slice; DH/16 x NFB accumulator blocks) += phi_K^T G
// over one unit, and Sz += phi_K^T 1 when with_z.
template <typename T, int DH, int NFB>
__device__ __forceinline__ void apply_unit(f32x4 (&S)[DH / 16][NFB], f32x4 (&Sz)[DH / 16], bool with_z,
                                           const UnitRegs<T, DH, NFB>& c) {
#pragma unroll
  for (int ks = 0; ks < unit_len<DH>() / 32; ++ks)
#pragma unroll
    for (int eb = 0; eb < DH / 16; ++eb) {
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb) mma(S[eb][fb], c.k[ks][eb], c.g[ks][fb]);
      if (with_z) mma(Sz[eb], c.k[ks][eb], ones_frag<T>());
    }
}

// Pass 1: per-segment sums (all segments but the last).
template <typename T, int DH, int CH, int NFB>
__global__ __launch_bounds__(kScanThreads) void scan_partial_kernel(ScanArgs a) {
  constexpr int FSC = kScanWaves * 16 * NFB;
  const int Fh = a.F / a.H, HD = a.H * DH;
  const ScanWg w = scan_wg(blockIdx.x, Fh / FSC, a.H, a.nseg - 1);
  const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool with_z = w.fsl == 0 && wave == 0;
  const int64_t mseq = w.b * a.Tp;
  const int cf = w.fsl * FSC + wave * 16 * NFB;            // first column within the head
  const int64_t col = (int64_t)w.h * Fh + cf;
  const T* fk = static_cast<const T*>(a.fk);
  const T* gp = static_cast<const T*>(a.gp);

  f32x4 S[DH / 16][NFB], Sz[DH / 16];
#pragma unroll
  for (int eb = 0; eb < DH / 16; ++eb) {
    Sz[eb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb) S[eb][fb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int nchunks = a.Tp / CH;
  const int c0 = w.seg * a.chunks_per_seg, c1 = min(nchunks, c0 + a.chunks_per_seg);
  // two register sets: unit u + 1 loads while unit u is applied
  constexpr int UPC = CH / unit_len<DH>();   // units per chunk
  const int u0 = c0 * UPC, u1 = c1 * UPC;
  UnitRegs<T, DH, NFB> r0, r1;
  auto load = [&](UnitRegs<T, DH, NFB>& r, int u) {
    load_unit<T, DH, NFB>(r, fk, gp, mseq + (int64_t)min(u, u1 - 1) * unit_len<DH>(), HD, w.h * DH, col, a.F, li, lg);
  };
  if (u0 < u1) load(r0, u0);
  for (int u = u0; u < u1; u += 2) {
    load(r1, u + 1);
    apply_unit<T, DH, NFB>(S, Sz, with_z, r0);
    if (u + 1 < u1) {
      load(r0, u + 2);
      apply_unit<T, DH, NFB>(S, Sz, with_z, r1);
    }
  }

  float* dst = a.seg_state + (((w.b * a.H + w.h) * a.nseg + w.seg) * (int64_t)DH) * Fh;
#pragma unroll
  for (int eb = 0; eb < DH / 16; ++eb)
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(int64_t)(eb * 16 + lg * 4 + r) * Fh + cf + fb * 16 + li] = S[eb][fb][r];
  if (with_z && li == 0) {
    float* zd = a.seg_z + ((w.b * a.H + w.h) * a.nseg + w.seg) * DH;
#pragma unroll
    for (int eb = 0; eb < DH / 16; ++eb)
#pragma unroll
      for (int r = 0; r < 4; ++r) zd[eb * 16 + lg * 4 + r] = Sz[eb][r];
  }
}

// Pass 2: exclusive prefix over segments, in place.  One thread per state
// element; the segment values are loaded in independent batches of kBatch so
// that the memory latency is paid once per batch, not once per segment.
constexpr int kBatch = 16;
__device__ __forceinline__ void exclusive_prefix(float* p, int64_t stride, int nseg) {
  float run = 0.f;
  for (int s0 = 0; s0 < nseg - 1; s0 += kBatch) {   // the last segment has no sum of its own
    float v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (s0 + u < nseg - 1) v[u] = p[(int64_t)(s0 + u) * stride];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (s0 + u < nseg - 1) {
        p[(int64_t)(s0 + u) * stride] = run;
        run += v[u];
      }
  }
  p[(int64_t)(nseg - 1) * stride] = run;
}

__global__ void scan_prefix_kernel(float* state, float* segz, int64_t per_bh, int nseg, int64_t nbh,
                                   int dh) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nbh * per_bh) {
    const int64_t bh = i / per_bh, e = i % per_bh;
    exclusive_prefix(state + bh * nseg * per_bh + e, per_bh, nseg);
  }
  if (i < nbh * dh) {
    const int64_t bh = i / dh, e = i % dh;
    exclusive_prefix(segz + bh * nseg * dh + e, dh, nseg);
  }
}

// Pass 3: replay each segment from its prefix and emit n_old, z_old.
template <typename T, int DH, int CH, int NFB>
__global__ __launch_bounds__(kScanThreads) void scan_main_kernel(ScanArgs a) {
  constexpr int FSC = kScanWaves * 16 * NFB, NIB = CH / 16, KE = DH / 32;
  const int Fh = a.F / a.H, HD = a.H * DH, F = a.F;
  const ScanWg w = scan_wg(blockIdx.x, Fh / FSC, a.H, a.nseg);
  const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool with_z = w.fsl == 0 && wave == 0;
  const int64_t mseq = w.b * a.Tp;
  const int cf = w.fsl * FSC + wave * 16 * NFB;
  const int64_t col = (int64_t)w.h * Fh + cf;
  const T* fk = static_cast<const T*>(a.fk);
  const T* fq = static_cast<const T*>(a.fq);
  const T* gp = static_cast<const T*>(a.gp);
  const int nchunks = a.Tp / CH, lag = a.window / CH;
  const int c0 = w.seg * a.chunks_per_seg, c1 = min(nchunks, c0 + a.chunks_per_seg);

  // state prefix of this segment
  f32x4 S[DH / 16][NFB], Sz[DH / 16];
  {
    const float* src = a.seg_state + (((w.b * a.H + w.h) * a.nseg + w.seg) * (int64_t)DH) * Fh;
    const float* zs = a.seg_z + ((w.b * a.H + w.h) * a.nseg + w.seg) * DH;
#pragma unroll
    for (int eb = 0; eb < DH / 16; ++eb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = eb * 16 + lg * 4 + r;
        Sz[eb][r] = (w.seg == 0 || !with_z) ? 0.f : zs[e];
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb) S[eb][fb][r] = w.seg == 0 ? 0.f : src[(int64_t)e * Fh + cf + fb * 16 + li];
      }
  }

  // destinations with no older chunk: zeros
  if (w.seg == 0) {
    for (int dchunk = 0; dchunk < min(lag, nchunks); ++dchunk) {
#pragma unroll
      for (int ib = 0; ib < NIB; ++ib)
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb) {
          const int64_t nblk = ((mseq + (int64_t)dchunk * CH) / 16 + ib) * (F / 16) + col / 16 + fb;
          *reinterpret_cast<f32x4*>(a.n_old + (nblk * 64 + lane) * 4) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      if (with_z && lg == 0)
        for (int ib = 0; ib < NIB; ++ib)
          a.z_old[(mseq + (int64_t)dchunk * CH + ib * 16 + li) * a.H + w.h] = 0.f;
    }
  }

  constexpr int UPC = CH / unit_len<DH>();   // units per chunk
  const int u0 = c0 * UPC, u1 = c1 * UPC;
  UnitRegs<T, DH, NFB> r0, r1;
  auto load = [&](UnitRegs<T, DH, NFB>& r, int u) {
    load_unit<T, DH, NFB>(r, fk, gp, mseq + (int64_t)min(u, u1 - 1) * unit_len<DH>(), HD, w.h * DH, col, F, li, lg);
  };
  // read-out of S_{<cCH} for destination chunk c + lag: n_old^T = S^T phi_Q^T
  auto readout = [&](int c) {
    const int dchunk = c + lag;
    if (dchunk < nchunks) {
      // read-out of S_{<cCH} for destination chunk d: n_old^T = S^T phi_Q^T
      Frag<T> sa[KE][NFB], za[KE];
#pragma unroll
      for (int ke = 0; ke < KE; ++ke) {
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb) sa[ke][fb] = join(cvt_quad<T>(S[2 * ke][fb]), cvt_quad<T>(S[2 * ke + 1][fb]));
        za[ke] = join(cvt_quad<T>(Sz[2 * ke]), cvt_quad<T>(Sz[2 * ke + 1]));
      }
      const int64_t drow = mseq + (int64_t)dchunk * CH;
#pragma unroll
      for (int ib = 0; ib < NIB; ++ib) {
        Frag<T> qb[KE];
#pragma unroll
        for (int ke = 0; ke < KE; ++ke)
          qb[ke] = load_frag<T>(fq + (drow + ib * 16 + li) * HD + w.h * DH + ke * 32 + lg * 8);
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb) {
          f32x4 n = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ke = 0; ke < KE; ++ke) mma(n, sa[ke][fb], qb[ke]);
          const int64_t nblk = (drow / 16 + ib) * (F / 16) + col / 16 + fb;
          *reinterpret_cast<f32x4*>(a.n_old + (nblk * 64 + lane) * 4) = n;
        }
        if (with_z) {
          f32x4 nz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ke = 0; ke < KE; ++ke) mma(nz, za[ke], qb[ke]);
          if (lg == 0) a.z_old[(drow + ib * 16 + li) * a.H + w.h] = nz[0];
        }
      }
    }
  };
  // the read-out for chunk c comes before its first unit is applied
  if (u0 < u1) load(r0, u0);
  for (int u = u0; u < u1; u += 2) {
    load(r1, u + 1);
    if (u % UPC == 0) readout(u / UPC);
    apply_unit<T, DH, NFB>(S, Sz, with_z, r0);
    if (u + 1 < u1) {
      load(r0, u + 2);
      if ((u + 1) % UPC == 0) readout((u + 1) / UPC);
      apply_unit<T, DH, NFB>(S, Sz, with_z, r1);
    }
  }
}

template <typename T, int DH, int CH, int NFB>
hipError_t launch_scan_t(const ScanArgs& a, hipStream_t s) {
  constexpr int FSC = kScanWaves * 16 * NFB;
  const int Fh = a.F / a.H;
  const int64_t groups = (int64_t)a.B * a.H * (Fh / FSC);
  if (a.nseg > 1) {
    hipLaunchKernelGGL((scan_partial_kernel<T, DH, CH, NFB>), dim3((unsigned)(groups * (a.nseg - 1))),
                       dim3(kScanThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t per_bh = (int64_t)DH * Fh, nbh = (int64_t)a.B * a.H;
    hipLaunchKernelGGL(scan_prefix_kernel, dim3((unsigned)ceil_div(nbh * per_bh, 256)), dim3(256), 0, s,
                       a.seg_state, a.seg_z, per_bh, a.nseg, nbh, DH);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((scan_main_kernel<T, DH, CH, NFB>), dim3((unsigned)(groups * a.nseg)),
                     dim3(kScanThreads), 0, s, a);
  return hipGetLastError();
}

template <typename T, int DH, int CH>
hipError_t launch_scan_nfb(const ScanArgs& a, hipStream_t s) {
  if ((a.F / a.H) % (kScanWaves * 32) == 0) return launch_scan_t<T, DH, CH, 2>(a, s);
  return launch_scan_t<T, DH, CH, 1>(a, s);
}

template <typename T, int CH>
hipError_t launch_scan_dh(const ScanArgs& a, hipStream_t s) {
  switch (a.dh) {
    case 32: return launch_scan_nfb<T, 32, CH>(a, s);
    case 64: return launch_scan_nfb<T, 64, CH>(a, s);
    case 128: return launch_scan_nfb<T, 128, CH>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

ScanPlan wango_scan_plan(int B, int Tp, int F, int H, int chunk) {
  ScanPlan p;
  const int nchunks = Tp / chunk;
  p.fs = ((F / H) % (kScanWaves * 32) == 0) ? kScanWaves * 32 : kScanWaves * 16;
  const int64_t groups = (int64_t)B * H * ((F / H) / p.fs);
  int64_t nseg = ceil_div(384, groups);
  if (nseg < 1) nseg = 1;
  if (nseg > nchunks) nseg = nchunks;
  p.chunks_per_seg = (int)ceil_div(nchunks, nseg);
  p.nseg = (int)ceil_div(nchunks, p.chunks_per_seg);
  return p;
}

hipError_t launch_wango_scan(const ScanArgs& a, const ScanPlan& p, bool bf, hipStream_t s) {
  ScanArgs aa = a;
  aa.nseg = p.nseg;
  aa.chunks_per_seg = p.chunks_per_seg;
  if (bf) return a.chunk == 128 ? launch_scan_dh<bf16, 128>(aa, s) : launch_scan_dh<bf16, 64>(aa, s);
  return a.chunk == 128 ? launch_scan_dh<float, 128>(aa, s) : launch_scan_dh<float, 64>(aa, s);
}

}  // namespace tango
