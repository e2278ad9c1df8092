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
// itself).  z rides along as the state of a column of ones, kept by one wave
// per (sequence, head).
//
// The sequence is cut into segments so that many workgroups run at once:
// pass 1 sums every segment's contribution (all but the last segment); pass 2
// adds the sums of the segments before its own to get its starting state, then
// replays its segment and emits the read-outs.  Both passes are bound by the
// latency of their loads, so each wave keeps a ring of register sets of source
// units with all but one in flight, and pass 2 stages the query
// features of the next chunk through LDS while the current chunk runs.  The
// key features of a unit, which all four waves multiply, are loaded once per
// workgroup (a quarter by each wave) and shared through an LDS ring.
#include "common.hpp"
#include "kernels.hpp"

namespace tango {

namespace {

constexpr int kScanWaves = 4;
constexpr int kScanThreads = 64 * kScanWaves;
// Source-unit register sets per wave (ring depth): all but one are in flight.
// The LDS feature ring has as many slots, and at least three: the slot a unit
// is stashed into was last read two units earlier, and only with three or more
// slots does a barrier lie between that read and the write (with two, a wave
// ahead of the others overwrites features another wave is still multiplying).
// (Five or six sets for bf16 measured no faster than four; with the features
// shared through LDS, six or eight in pass 1 and five in pass 2 neither.)
template <typename T, int DH, bool MAIN> constexpr int ring_sets() { return sizeof(T) == 4 ? 3 : 4; }
// Segment sums loaded per batch while the starting state is summed: about 64
// registers of loads in flight.
template <int DH, int NFB> constexpr int prefix_batch() {
  return (DH / 16) * NFB >= 16 ? 1 : 16 / ((DH / 16) * NFB);
}

template <typename T> __device__ __forceinline__ Frag<T> ones_frag() {
  Frag<T> f;
#pragma unroll
  for (int s = 0; s < 8; ++s) f[s] = cvt<T>(1.0f);
  return f;
}

// Workgroup barrier that orders LDS only: global loads stay in flight across it.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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

// A unit of sources: the gate fragments of this wave's columns in registers,
// and the key-feature fragments (A operand of S += phi_K^T G), which every wave
// of the workgroup needs, shared through an LDS ring: each wave loads KW of
// the unit's KF fragments and stashes them one unit ahead.  The unit is 64
// sources, 32 for d_h = 128.
template <int DH> constexpr int unit_len() { return DH >= 128 ? 32 : 64; }
template <int DH> constexpr int unit_kf() { return unit_len<DH>() / 32 * (DH / 16); }   // KF
template <typename T, int DH, int NFB> struct UnitRegs {
  static constexpr int U = unit_len<DH>(), KW = unit_kf<DH>() / kScanWaves;
  static_assert(unit_kf<DH>() % kScanWaves == 0, "feature fragments per wave");
  Frag<T> g[U / 32][NFB];
  Frag<T> kq[KW];   // fragments wave * KW .. wave * KW + KW - 1 of the unit (ks-major)
};
// LDS ring of the units' feature fragments: [NS][KF][64 lanes].
template <typename T, int DH, int NS> using FeatRing = Frag<T>[NS][unit_kf<DH>()][64];

template <typename T, int DH, int NFB>
__device__ __forceinline__ void load_unit(UnitRegs<T, DH, NFB>& c, const T* __restrict__ fk,
                                          const T* __restrict__ gp, int64_t row0, int HD, int hcol,
                                          int64_t col, int F, int li, int lg, int wave) {
  constexpr int KW = UnitRegs<T, DH, NFB>::KW;
#pragma unroll
  for (int ks = 0; ks < unit_len<DH>() / 32; ++ks) {
    const int64_t blk = row0 / 32 + ks;
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb) c.g[ks][fb] = load_frag<T>(gp + packed_offset(blk, lg, col + fb * 16 + li, F));
  }
#pragma unroll
  for (int q = 0; q < KW; ++q) {
    const int fi = wave * KW + q, ks = fi / (DH / 16), eb = fi % (DH / 16);
    c.kq[q] = load_frag<T>(fk + packed_offset(row0 / 32 + ks, lg, hcol + eb * 16 + li, HD));
  }
}

template <typename T, int DH, int NFB, int NS>
__device__ __forceinline__ void stash_unit(FeatRing<T, DH, NS>& ring, int slot, const UnitRegs<T, DH, NFB>& c,
                                           int wave, int lane) {
  constexpr int KW = UnitRegs<T, DH, NFB>::KW;
#pragma unroll
  for (int q = 0; q < KW; ++q) ring[slot][wave * KW + q][lane] = c.kq[q];
}

// S (this wave's DH x 16*NFB slice; DH/16 x NFB accumulator blocks) += phi_K^T G
// over one unit (features from ring slot `slot`), and Sz += phi_K^T 1 when with_z.
template <typename T, int DH, int NFB, int NS>
__device__ __forceinline__ void apply_unit(f32x4 (&S)[DH / 16][NFB], f32x4 (&Sz)[DH / 16], bool with_z,
                                           const UnitRegs<T, DH, NFB>& c, const FeatRing<T, DH, NS>& ring,
                                           int slot, int lane) {
#pragma unroll
  for (int ks = 0; ks < unit_len<DH>() / 32; ++ks) {
    Frag<T> k[DH / 16];
#pragma unroll
    for (int eb = 0; eb < DH / 16; ++eb) k[eb] = ring[slot][ks * (DH / 16) + eb][lane];
#pragma unroll
    for (int eb = 0; eb < DH / 16; ++eb)
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb) mma(S[eb][fb], k[eb], c.g[ks][fb]);
    if (with_z) {
#pragma unroll
      for (int eb = 0; eb < DH / 16; ++eb) mma(Sz[eb], k[eb], ones_frag<T>());
    }
  }
}

// Offset (floats) of a wave's accumulator block (eb, fb) in the segment sums,
// stored in accumulator order: block-contiguous, lane-major, 4 floats a lane.
template <int DH, int NFB>
__device__ __forceinline__ int64_t seg_block(int64_t slice_seg, int wave, int eb, int fb, int lane) {
  constexpr int FSC = kScanWaves * 16 * NFB;
  return slice_seg * (int64_t)(DH * FSC) + (((wave * (DH / 16) + eb) * NFB + fb) * 64 + lane) * 4;
}

// One segment: its source units in order through a ring of NS register sets
// (and NS LDS slots for the features).  Before unit u is applied, the
// features of unit u + 1 (loaded NS - 2 units earlier) go to their slot and an
// LDS-only barrier publishes them; unit u's slot was published one unit ago,
// and a slot is rewritten NS - 2 barriers after it was last read (NS >= 3).  MAIN adds,
// before the first unit of every chunk, the read-out of the state for the
// destination chunk that chunk feeds (through `boundary`).  The caller has
// loaded units u0 .. u0 + NS - 2, stashed unit u0 and synchronised.
template <typename T, int DH, int NFB, int UPC, int NS, typename Boundary>
__device__ __forceinline__ void walk_units(f32x4 (&S)[DH / 16][NFB], f32x4 (&Sz)[DH / 16], bool with_z,
                                           UnitRegs<T, DH, NFB> (&R)[NS], FeatRing<T, DH, NS>& ring, int u0,
                                           int u1, const T* fk, const T* gp, int64_t mseq, int HD, int hcol,
                                           int64_t col, int F, int li, int lg, int wave, Boundary&& boundary) {
  static_assert(NS >= 3, "a barrier must separate a slot's last read from its next write");
  const int lane = lg * 16 + li;
  auto load = [&](UnitRegs<T, DH, NFB>& r, int u) {
    load_unit<T, DH, NFB>(r, fk, gp, mseq + (int64_t)min(u, u1 - 1) * unit_len<DH>(), HD, hcol, col, F, li, lg,
                          wave);
  };
  for (int u = u0; u < u1; u += NS) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      load(R[(j + NS - 1) % NS], u + j + NS - 1);
      // units past the end re-read the last one: stashing them is harmless
      stash_unit<T, DH, NFB, NS>(ring, (j + 1) % NS, R[(j + 1) % NS], wave, lane);
      lds_sync();
      if ((u + j) % UPC == 0 && u + j < u1) boundary((u + j) / UPC);
      if (u + j < u1) apply_unit<T, DH, NFB, NS>(S, Sz, with_z, R[j], ring, j, lane);
    }
  }
}

// Pass 1: per-segment sums (all segments but the last).
template <typename T, int DH, int CH, int NFB>
__global__ __launch_bounds__(kScanThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void scan_partial_kernel(ScanArgs a) {
  constexpr int FSC = kScanWaves * 16 * NFB;
  const int Fh = a.F / a.H, HD = a.H * DH;
  const int nslices = Fh / FSC;
  const ScanWg w = scan_wg(blockIdx.x, nslices, a.H, a.nseg - 1);
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
  constexpr int UPC = CH / unit_len<DH>(), NS = ring_sets<T, DH, false>();
  const int u0 = c0 * UPC, u1 = c1 * UPC;
  __shared__ FeatRing<T, DH, NS> ring;
  UnitRegs<T, DH, NFB> R[NS];
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    load_unit<T, DH, NFB>(R[j], fk, gp, mseq + (int64_t)min(u0 + j, u1 - 1) * unit_len<DH>(), HD, w.h * DH,
                          col, a.F, li, lg, wave);
  stash_unit<T, DH, NFB, NS>(ring, 0, R[0], wave, lane);
  lds_sync();
  walk_units<T, DH, NFB, UPC, NS>(S, Sz, with_z, R, ring, u0, u1, fk, gp, mseq, HD, w.h * DH, col, a.F, li, lg,
                                  wave, [](int) {});

  const int64_t slice_seg = (((w.b * a.H + w.h) * nslices + w.fsl) * (int64_t)a.nseg + w.seg);
#pragma unroll
  for (int eb = 0; eb < DH / 16; ++eb)
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb)
      *reinterpret_cast<f32x4*>(a.seg_state + seg_block<DH, NFB>(slice_seg, wave, eb, fb, lane)) = S[eb][fb];
  if (with_z && li == 0) {
    float* zd = a.seg_z + ((w.b * a.H + w.h) * a.nseg + w.seg) * DH;
#pragma unroll
    for (int eb = 0; eb < DH / 16; ++eb) *reinterpret_cast<f32x4*>(zd + eb * 16 + lg * 4) = Sz[eb];
  }
}

// Pass 2: the segment's starting state (sum of the sums of the segments before
// it), then the replay of its sources with, at every chunk boundary, either
// the read-outs of n_old, z_old (RO) or the state itself in the read-out's
// A-operand layout, for the band kernel to read out (no query features then).
template <typename T, int DH, int CH, int NFB, bool RO>
__global__ __launch_bounds__(kScanThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void scan_main_kernel(ScanArgs a) {
  constexpr int FSC = kScanWaves * 16 * NFB, NIB = CH / 16, KE = DH / 32;
  constexpr int QF = NIB * KE * 64;                 // query fragments per chunk
  constexpr int QPT = QF / kScanThreads;            // ... per thread
  constexpr int NQB = sizeof(T) == 2 ? 2 : 1;       // LDS query buffers
  static_assert(QF % kScanThreads == 0, "query fragments per chunk");
  __shared__ Frag<T> qs[RO ? NQB : 1][RO ? QF : 1];
  const int Fh = a.F / a.H, HD = a.H * DH, F = a.F;
  const int nslices = Fh / FSC;
  const ScanWg w = scan_wg(blockIdx.x, nslices, a.H, a.nseg);
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
  constexpr int UPC = CH / unit_len<DH>(), NS = ring_sets<T, DH, true>();
  const int u0 = c0 * UPC, u1 = c1 * UPC;

  // query features of a destination chunk, fragment order, QPT per thread
  Frag<T> qn[QPT];
  auto load_q = [&](int c) {
    const int64_t drow = mseq + (int64_t)min(c + lag, nchunks - 1) * CH;
#pragma unroll
    for (int q = 0; q < QPT; ++q) {
      const int f = threadIdx.x + q * kScanThreads;
      const int fl = f & 63, ke = (f >> 6) % KE, ib = f / (64 * KE);
      qn[q] = load_frag<T>(fq + (drow + ib * 16 + (fl & 15)) * HD + w.h * DH + ke * 32 + (fl >> 4) * 8);
    }
  };
  if constexpr (RO) load_q(c0);   // first: the ring loads issued after it keep later waits on it precise

  // first source units in flight
  __shared__ FeatRing<T, DH, NS> ring;
  UnitRegs<T, DH, NFB> R[NS];
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    load_unit<T, DH, NFB>(R[j], fk, gp, mseq + (int64_t)min(u0 + j, u1 - 1) * unit_len<DH>(), HD, w.h * DH,
                          col, F, li, lg, wave);
  // starting state: sum of the segment sums before this one
  f32x4 S[DH / 16][NFB], Sz[DH / 16];
#pragma unroll
  for (int eb = 0; eb < DH / 16; ++eb) {
    Sz[eb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb) S[eb][fb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  {
    const int64_t slice0 = ((w.b * a.H + w.h) * nslices + w.fsl) * (int64_t)a.nseg;
    const float* zs = a.seg_z + (w.b * a.H + w.h) * (int64_t)a.nseg * DH;
    // two batches in flight; loads past the last predecessor re-read it and are dropped
    constexpr int PB = prefix_batch<DH, NFB>();
    using Batch = f32x4[PB][DH / 16][NFB];
    auto load_batch = [&](Batch& v, int s0) {
#pragma unroll
      for (int p = 0; p < PB; ++p)
#pragma unroll
        for (int eb = 0; eb < DH / 16; ++eb)
#pragma unroll
          for (int fb = 0; fb < NFB; ++fb)
            v[p][eb][fb] = *reinterpret_cast<const f32x4*>(
                a.seg_state + seg_block<DH, NFB>(slice0 + min(s0 + p, w.seg - 1), wave, eb, fb, lane));
    };
    auto add_batch = [&](const Batch& v, int s0) {
#pragma unroll
      for (int p = 0; p < PB; ++p) {
        const float keep = s0 + p < w.seg ? 1.f : 0.f;
#pragma unroll
        for (int eb = 0; eb < DH / 16; ++eb)
#pragma unroll
          for (int fb = 0; fb < NFB; ++fb) S[eb][fb] += keep * v[p][eb][fb];
      }
    };
    if (w.seg > 0) {
      Batch va, vb;
      load_batch(va, 0);
      for (int s0 = 0; s0 < w.seg; s0 += 2 * PB) {
        load_batch(vb, s0 + PB);
        add_batch(va, s0);
        load_batch(va, s0 + 2 * PB);
        add_batch(vb, s0 + PB);
      }
    }
    if (with_z) {
      constexpr int ZB = 8;
      for (int s0 = 0; s0 < w.seg; s0 += ZB) {
        f32x4 zv[ZB][DH / 16];
#pragma unroll
        for (int p = 0; p < ZB; ++p)
#pragma unroll
          for (int eb = 0; eb < DH / 16; ++eb)
            zv[p][eb] = *reinterpret_cast<const f32x4*>(zs + (int64_t)min(s0 + p, w.seg - 1) * DH + eb * 16 + lg * 4);
#pragma unroll
        for (int p = 0; p < ZB; ++p) {
          const float keep = s0 + p < w.seg ? 1.f : 0.f;
#pragma unroll
          for (int eb = 0; eb < DH / 16; ++eb) Sz[eb] += keep * zv[p][eb];
        }
      }
    }
  }

  // destinations with no older chunk: zeros (the band reads no state for them)
  if (RO && w.seg == 0) {
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

  // chunk c: the state S_{<cCH} of destination chunk c + lag.  RO: stage the
  // chunk's query features, read the state out (n_old^T = S^T phi_Q^T), then
  // fetch the next chunk's features; otherwise store the state's A-operand
  // fragments (the same bf16 parts the read-out multiplies)
  auto boundary = [&](int c) {
    if constexpr (!RO) {
      const int dchunk = c + lag;
      if (dchunk < nchunks) {
        T* st = static_cast<T*>(a.states);
        const int64_t dbase = (w.b * a.H + w.h) * (int64_t)nchunks + dchunk;
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
          for (int ke = 0; ke < KE; ++ke)
            store_frag<T>(st + (((dbase * (Fh / 16) + cf / 16 + fb) * KE + ke) * 64 + lane) * 8,
                          join(cvt_quad<T>(S[2 * ke][fb]), cvt_quad<T>(S[2 * ke + 1][fb])));
        if (with_z) {
          T* zt = static_cast<T*>(a.zstates);
#pragma unroll
          for (int ke = 0; ke < KE; ++ke)
            store_frag<T>(zt + ((dbase * KE + ke) * 64 + lane) * 8,
                          join(cvt_quad<T>(Sz[2 * ke]), cvt_quad<T>(Sz[2 * ke + 1])));
        }
      }
    } else {
      Frag<T>* buf = qs[NQB == 2 ? (c & 1) : 0];
      if constexpr (NQB == 1) lds_sync();   // the previous read-out is done with the buffer
#pragma unroll
      for (int q = 0; q < QPT; ++q) buf[threadIdx.x + q * kScanThreads] = qn[q];
      lds_sync();
      const int dchunk = c + lag;
      if (dchunk < nchunks) {
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
          for (int ke = 0; ke < KE; ++ke) qb[ke] = buf[(ib * KE + ke) * 64 + lane];
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
      if (c + 1 < c1) load_q(c + 1);   // after the stores: waits on it stay precise
    }
  };
  stash_unit<T, DH, NFB, NS>(ring, 0, R[0], wave, lane);
  lds_sync();
  walk_units<T, DH, NFB, UPC, NS>(S, Sz, with_z, R, ring, u0, u1, fk, gp, mseq, HD, w.h * DH, col, F, li, lg, wave,
                                  boundary);
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
  }
  if (a.states)
    hipLaunchKernelGGL((scan_main_kernel<T, DH, CH, NFB, false>), dim3((unsigned)(groups * a.nseg)),
                       dim3(kScanThreads), 0, s, a);
  else
    hipLaunchKernelGGL((scan_main_kernel<T, DH, CH, NFB, true>), dim3((unsigned)(groups * a.nseg)),
                       dim3(kScanThreads), 0, s, a);
  return hipGetLastError();
}

template <typename T, int DH, int CH>
hipError_t launch_scan_nfb(const ScanArgs& a, hipStream_t s) {
  if (a.slice == kScanWaves * 32) return launch_scan_t<T, DH, CH, 2>(a, s);
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
  // Column slices of 128 when there are enough of them, else of 64: more
  // slices need fewer segments, and every segment re-reads the sums of the
  // segments before it.
  const int Fh = F / H;
  const bool wide = Fh % (kScanWaves * 32) == 0 && (int64_t)B * H * (Fh / (kScanWaves * 32)) >= 32;
  p.fs = wide ? kScanWaves * 32 : kScanWaves * 16;
  const int64_t groups = (int64_t)B * H * (Fh / p.fs);
  int64_t nseg = ceil_div(256, groups);   // about one workgroup per compute unit
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
  aa.slice = p.fs;
  if (bf) return a.chunk == 128 ? launch_scan_dh<bf16, 128>(aa, s) : launch_scan_dh<bf16, 64>(aa, s);
  return a.chunk == 128 ? launch_scan_dh<float, 128>(aa, s) : launch_scan_dh<float, 64>(aa, s);
}

}  // namespace tango
