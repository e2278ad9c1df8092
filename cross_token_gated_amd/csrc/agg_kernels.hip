// agg_kernels.hip - gate aggregation on gfx950 MFMA.
//
// TANGO ("TANGO: Token-Aggregated Nonlinear Gating Operators ...", §2.1 eqs.
// 4-5, §2.2 eq. 6):
//     gbar_ia = sum_{j<=i} e^{l_ija} g_ja / (sum_{j<=i} e^{l_ija} + n_i e^{b_a}),
//     l_ija = tau_a q_ia . k_ja with unit-length q and k.
// WANGO window band (§2.2 eqs. 7-10 and the joint-normalisation paragraph):
// the same exp weights over the trailing window of W positions, plus the
// older-prefix numerator n_old and denominator z_old from the running sums,
// plus the null term, all in one ratio.
//
// Because |q.k| <= 1, every logit lies in [-tau, tau] with tau <= 20, so the
// weights are computed as e^{tau (s - 1)}: a fixed shift by the largest
// possible logit replaces the running maximum of softmax kernels.  The shift
// cancels in the ratio (the null and older-prefix terms are scaled by e^{-tau}
// to match) and every weight stays in [e^{-40}, 1], far from float32 limits.
// With no running maximum, partial sums over disjoint source ranges combine by
// plain addition and the accumulators are never rescaled.
//
// Workgroup: 8 waves (two per SIMD) over a BR-row destination tile and
// FS = 8 * WCOLS gate columns of one head.  Per step of 64 sources:
//   * the key block is staged once in LDS (double-buffered, fetched two steps
//     ahead);
//   * wave w computes S^T = K Q^T for destination block w against all 64
//     sources, exponentiates, and writes the weights to LDS -- one step
//     ahead, between the two halves of the current step's product -- and
//     takes its row sums with one MFMA against a fragment of ones per half;
//   * every wave multiplies its own WCOLS gate columns: gbar^T += G^T P^T, the
//     gates read straight from the packed layout in global memory (their k
//     order is the row order of the S^T accumulators), double-buffered in
//     registers.
// One barrier per step; every step issues the same loads, so the compiler's
// load-counter waits stay exact across the loop.
//
// TANGO load balance: with B*H*column-chunks*(tiles/2) >= 256 the long and the
// short tile of a causal pair share one workgroup.  Otherwise each long tile is
// split in two source ranges done by two workgroups, each writing a float32
// partial; the second to finish adds the two (a commutative sum, so the result
// does not depend on which finishes first) and writes gbar.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace tango {

namespace {

// Destination rows per tile and gate columns per wave.  The columns per wave
// (WIDE, 48, 32 or 16) are chosen per head width by a cost model (agg_wcols
// below); where the width is not a multiple of 8 waves' columns, the last
// column chunk has waves with fewer or no columns inside the head, which
// multiply copies and store nothing past the width.
template <typename T> struct AggCfg;
template <> struct AggCfg<bf16> { static constexpr int BR = 128, WIDE = 64; };
template <> struct AggCfg<float> { static constexpr int BR = 64, WIDE = 32; };
constexpr int kNarrow = 16;
constexpr int kMid = 32;
constexpr int kMid48 = 48;                // bf16 only
constexpr int kShortBR = 64;       // bf16 TANGO tiles of 64 rows, for grids that would underfill
constexpr int kFillItems = 256;    // work items that fill the 256 compute units once

constexpr int kWaves = 8;                 // two waves per SIMD
constexpr int BC = 64;                    // sources per step
constexpr int kAggThreads = 64 * kWaves;

enum JobKind { kFull = 0, kPart0 = 1, kPart1 = 2 };
struct Job {
  int tile, jb0, jb1, kind;   // destination tile; source steps jb0..jb1 (64 each)
  int64_t split_id;
};

// LDS operand layout.  The key block (BC sources x DH) and the weights
// (BR destinations x BC sources) are MFMA operands read by every wave.  A
// block of 16 rows x 32 k is stored as 256-byte regions, one per (chunk h,
// k group g) with g covering k = 8g .. 8g + 7 in the order of the fragment's
// slots (PPF chunks of 16 bytes per fragment: 1 for bf16, 2 for float32);
// row r of the block sits at slot r xor 2g of its region.  gfx950 serves a
// 16-byte LDS read 16 lanes (256 bytes) per clock and a 16-byte write 8 lanes
// (128 bytes) per clock, conflict-free when the lanes of the group hit
// distinct 16-byte slots modulo 256 or 128 bytes: an MFMA fragment read
// (lanes 16g .. 16g + 15: rows 0 .. 15 of group g) takes a permutation of one
// region, and the key loader's 8-lane groups (two rows x four groups; four
// consecutive lanes fetch the 64 contiguous bytes of one row, keeping its
// global loads coalesced) land on 8 distinct slots modulo 8.  Measured on
// gfx950 with SQ_LDS_BANK_CONFLICT: 8 LDS cycles per loader write
// instruction, against 16 with slot r xor g and 32 with slot r.
template <typename T> constexpr int frag_chunks() { return (int)sizeof(T) / 2; }
__device__ __forceinline__ int region_pos(int region, int r, int g) {
  return region * 256 + (r ^ (2 * g)) * 16;
}

template <typename T, int DH, int BR> struct AggLds {
  T ks[2][BC * DH];   // key blocks, region layout (16-source block jj, k block, chunk, group)
  T ps[2][BR * BC];   // weights, region layout (16-destination block, 32-source half, chunk, group)
  float den[kWaves][BR];
  int flag;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Index of accumulator element r of 16 x 16 block blk, lane `lane`, in a
// partial: element-major within a block, so each store instruction writes
// 256 contiguous bytes.
__device__ __forceinline__ int64_t part_index(int blk, int r, int lane) {
  return ((int64_t)blk * 4 + r) * 64 + lane;
}

template <typename T, int MODE, int DH, int WCOLS, int BR>
__global__ __launch_bounds__(kAggThreads) void agg_kernel(AggArgs a, int nfc, int rtiles,
                                                          int64_t items) {
  constexpr int FS = kWaves * WCOLS, NFB = WCOLS / 16, NIB = BR / 16;
  constexpr int JBW = NIB * (BC / 16) / kWaves;  // S^T source blocks per wave (one dest block)
  constexpr int NSPLIT = kWaves / NIB;           // waves sharing one destination block
  constexpr int KS = DH / 32;
  constexpr int SPT = BR / BC;                    // source steps per destination tile
  using L = AggLds<T, DH, BR>;
  constexpr int PE = 16 / (int)sizeof(T);        // elements per 16-byte piece
  constexpr int PPF = frag_chunks<T>();
  constexpr int KCH = (BC / 16) * KS * PPF;       // 64-piece chunks of a key block
  constexpr int KPT = (KCH + kWaves - 1) / kWaves;   // per wave (the last may be partial)
  static_assert(JBW >= 2 && JBW % 2 == 0, "tile shape");
  __shared__ L sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int li = lane & 15, lg = lane >> 4;
  const int wib = wave % NIB;                      // destination block of this wave's S^T
  const int wjb = (wave / NIB) * JBW;              // its first source block

  // Work item of this workgroup.  Consecutive items go to one XCD (workgroup
  // w runs on XCD w % 8), so the workgroups of one XCD share gate columns.
  const int64_t q8 = gridDim.x / 8;
  const int64_t item = (int64_t)(blockIdx.x % 8) * q8 + blockIdx.x / 8;
  if (item >= items) return;

  const int R = rtiles, half = R / 2;
  Job job0 = {0, 0, 0, kFull, 0}, job1 = {0, 0, 0, kFull, 0};
  int njobs = 1;
  int64_t grp;
  if (MODE == 0) {
    const int P = a.split ? 2 * half + (R & 1) : half + (R & 1);
    grp = item / P;
    const int p = (int)(item % P);
    if (a.split) {
      if (p == 2 * half) {
        job0 = {half, 0, (half + 1) * SPT - 1, kFull, 0};          // middle tile (R odd)
      } else {
        const int k = p >> 1, rl = R - 1 - k;                      // short tile k, long tile rl
        const int64_t sid = grp * half + (half - 1 - k);
        if ((p & 1) == 0) {
          job0 = {rl, (rl + 1 - half) * SPT, (rl + 1) * SPT - 1, kPart0, sid};
        } else {
          job0 = {rl, 0, (rl + 1 - half) * SPT - 1, kPart1, sid};
          job1 = {k, 0, (k + 1) * SPT - 1, kFull, 0};
          njobs = 2;
        }
      }
    } else {
      if (p == half) {
        job0 = {half, 0, (half + 1) * SPT - 1, kFull, 0};
      } else {
        job0 = {R - 1 - p, 0, (R - p) * SPT - 1, kFull, 0};
        job1 = {p, 0, (p + 1) * SPT - 1, kFull, 0};
        njobs = 2;
      }
    }
  } else {
    grp = item / R;
    const int r = (int)(item % R);
    // first source: the start of the chunk holding row i0 - W (the older
    // sources of that chunk are read pairwise here), or 0
    const int i0 = r * BR;
    const int lo = i0 >= a.window ? (i0 - a.window) / a.chunk * a.chunk : 0;
    job0 = {r, lo / BC, (r + 1) * SPT - 1, kFull, 0};
  }
  const int fc = (int)(grp % nfc);
  const int64_t bh = grp / nfc;
  const int h = (int)(bh % a.H);
  const int64_t b = bh / a.H;

  const int F = a.F, HD = a.H * DH, Fh = F / a.H, Tp = a.Tp;
  const int f_base = fc * FS + wave * WCOLS;          // within the head
  const bool has_cols = f_base < Fh;                   // wave-uniform; always true when FS divides Fh
  const int64_t col0 = (int64_t)h * Fh + f_base;       // global gate column
  const int64_t mseq = b * Tp;                         // first row of the sequence

  const float tau = __expf(fminf(a.theta[h], 2.995732273553991f));   // log 20
  const float ktau = tau * kLog2e;
  const float stau = sqrtf(tau), isd = 1.0f / sqrtf((float)DH);      // WANGO features
  const float escale = __expf(-tau);                   // e^{-tau}: the fixed shift
  const float null_w = a.null_bias ? __expf(a.null_bias[h] - tau) : 0.f;

  const T* __restrict__ qh = static_cast<const T*>(a.qh);
  const T* __restrict__ kh = static_cast<const T*>(a.kh);
  const T* __restrict__ gp = static_cast<const T*>(a.gp);
  T* __restrict__ gbar = static_cast<T*>(a.gbar);

  // key block jb -> registers -> LDS buffer.  Chunk c = wave + kWaves p of
  // the block (16-source block jj, k block kb, chunk ch); lane l fetches row
  // l / 4 and k group l % 4 of it.  A wave past the last chunk (small heads)
  // fetches a copy of chunk c mod KCH and does not store it, so that every
  // wave issues the same loads.
  // (The global addresses are split into a wave-uniform 64-bit base and a
  // 32-bit lane offset.)
  const int k_lane = (lane >> 2) * HD + (lane & 3) * 8;
  auto key_chunk = [&](int p, int& row0, int& col, int& off) {
    const int c = (wave + kWaves * p) % KCH;
    const int jj = c / (KS * PPF), kb = (c / PPF) % KS, ch = c % PPF;
    const int r = lane >> 2, g = lane & 3;
    row0 = jj * 16;
    col = kb * 32 + ch * PE;
    off = region_pos(((jj * KS + kb) * PPF + ch) * 4 + g, r, g);
  };
  auto key_fetch = [&](int jb, u32x4 (&kr)[KPT]) {
#pragma unroll
    for (int p = 0; p < KPT; ++p) {
      int row0, col, off;
      key_chunk(p, row0, col, off);
      const T* base = kh + (mseq + (int64_t)jb * BC + row0) * HD + h * DH + col;   // wave-uniform
      kr[p] = *reinterpret_cast<const u32x4*>(base + k_lane);
    }
  };
  auto key_stash = [&](int buf, const u32x4 (&kr)[KPT]) {
#pragma unroll
    for (int p = 0; p < KPT; ++p) {
      if (KCH % kWaves != 0 && wave + kWaves * p >= KCH) break;   // wave-uniform
      int row0, col, off;
      key_chunk(p, row0, col, off);
      *reinterpret_cast<u32x4*>(reinterpret_cast<unsigned char*>(sm.ks[buf]) + off) = kr[p];
    }
  };
  // MFMA fragment (16-row block rb, k block kb) of a region-layout tile
  auto lds_frag = [&](const T* tile, int nkb, int rb, int kb) -> Frag<T> {
    const unsigned char* base = reinterpret_cast<const unsigned char*>(tile) +
                                region_pos((rb * nkb + kb) * PPF * 4 + lg, li, lg);
    if constexpr (PPF == 1) {
      return load_frag<T>(reinterpret_cast<const T*>(base));
    } else {
      return join(load_quad<T>(reinterpret_cast<const T*>(base)),
                  load_quad<T>(reinterpret_cast<const T*>(base + 4 * 256)));
    }
  };
  // A wave past the head's width (narrow variant) reads the head's first
  // columns and multiplies them like the others; only its stores are
  // skipped.  Every step then issues the same loads and MFMAs in every wave,
  // which keeps the compiler's load-counter waits exact across the loop.
  const int64_t gcol0 = has_cols ? col0 : (int64_t)h * Fh;
  const int g_lane = (lg * F + li) * 8;   // packed_offset(blk, lg, col, F) - packed_offset(blk, 0, col - li, F)
  // 16-column blocks of this wave inside the head: with 48 columns a wave
  // can straddle the head's end (the head width is a multiple of 64); its
  // blocks past the end re-read the last block inside and are never stored.
  // Other widths keep constant offsets.
  constexpr bool kStraddle = 64 % WCOLS != 0;
  const int nvb = has_cols ? min(NFB, (Fh - f_base) / 16) : NFB;
  auto in_head = [&](int fb) { return kStraddle ? min(fb, nvb - 1) : fb; };
  auto gate_fetch = [&](int jb, int ks, Frag<T> (&gf)[NFB]) {
    const int64_t blk = (mseq + (int64_t)jb * BC) / 32 + ks;
    const T* base = gp + packed_offset(blk, 0, gcol0, F);   // wave-uniform
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb) gf[fb] = load_frag<T>(base + g_lane + in_head(fb) * 16 * 8);
  };

  // one destination tile over a range of source steps (called once or twice)
  auto run_job = [&](const Job job) {
    const int i0 = job.tile * BR;
    // B operand of S^T = K Q^T: column i of Q^T = query row i (linear k slots).
    Frag<T> qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = load_frag<T>(qh + (mseq + i0 + wib * 16 + li) * HD + h * DH + ks * 32 + lg * 8);

    // WANGO: phi(sqrt(tau) q) of the same fragment, for the older sources of
    // the chunk next to the window
    Frag<T> fqf[KS];
    if (MODE != 0) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) fqf[ks][e] = cvt<T>(phi_feature(stau * tof<T>(qf[ks][e]), isd));
    }

    f32x4 acc[NIB][NFB];
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib)
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb) acc[ib][fb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Row sums of this wave's weights.  bfloat16: a fragment of ones times
    // the weights of each 32-source half (every row of rsum then holds the
    // column sums); float32: plain adds in rsum[0], summed over lane groups
    // at the end.
    f32x4 rsum = {0.f, 0.f, 0.f, 0.f};
    Frag<T> ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = cvt<T>(1.0f);
    const int i_me = i0 + wib * 16 + li;     // this lane's destination in S^T
    // older sources of destination i read pairwise here: C floor((i-W)/C) <= j <= i-W
    const int jphi_lo = (MODE != 0 && i_me >= a.window) ? (i_me - a.window) / a.chunk * a.chunk : 0;

    // weights of source step jb (key block in ks[buf]) into ps[buf].  The
    // S^T accumulator starts at -1, so it holds s - 1 and the weight is
    // exp2(tau log2e (s - 1)) in one multiply.  A wave whose sources all lie at
    // or before its first destination needs no causal mask (TANGO: every step
    // but the diagonal ones).
    auto weights = [&](int jb, int buf) {
      const int j0 = jb * BC;
      // WANGO: does this step hold older sources of some row of the tile?
      const bool phi_step = MODE != 0 && i0 + BR - 1 >= a.window && j0 <= i0 + BR - 1 - a.window;
      const bool unmasked = MODE == 0 && j0 + (wjb + JBW) * 16 - 1 <= i0 + wib * 16;   // wave-uniform
      Quad<T> pq_even;
#pragma unroll
      for (int t = 0; t < JBW; ++t) {
        const int jj = wjb + t;   // wjb is even, so jj & 1 == t & 1
        f32x4 s = {-1.f, -1.f, -1.f, -1.f}, sphi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const Frag<T> kf = lds_frag(sm.ks[buf], KS, jj, ks);
          mma(s, kf, qf[ks]);
          if (phi_step) {
            Frag<T> fkf;
#pragma unroll
            for (int e = 0; e < 8; ++e) fkf[e] = cvt<T>(phi_feature(stau * tof<T>(kf[e]), isd));
            mma(sphi, fkf, fqf[ks]);
          }
        }
        Quad<T> pq;
        if (unmasked) {
          // the argument lies in [-2 tau log2 e, 0] >= -58: v_exp_f32 needs no range fix-up
#pragma unroll
          for (int r = 0; r < 4; ++r) pq[r] = cvt<T>(__builtin_amdgcn_exp2f(ktau * s[r]));
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = j0 + jj * 16 + lg * 4 + r;
            float p = 0.f;
            if (j <= i_me && (MODE == 0 || j > i_me - a.window)) {
              p = __builtin_amdgcn_exp2f(ktau * s[r]);
            } else if (phi_step && i_me >= a.window && j <= i_me - a.window && j >= jphi_lo) {
              p = escale * sphi[r];   // same e^{-tau} scale as the exp weights
            }
            pq[r] = cvt<T>(p);
          }
        }
        if constexpr (sizeof(T) == 2) {
          // blocks t - 1 and t make one half: a lane's 8 weights of column li
          if (t & 1) mma(rsum, ones, join(pq_even, pq));
          else pq_even = pq;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) rsum[0] += pq[r];
        }
        // the weights of sources 4 lg + r of block jj are slots r (jj even)
        // or 4 + r (jj odd) of this lane's fragment for the half jj / 2: for
        // bf16 the two blocks of a half make one 16-byte piece, written once
        // (half the write instructions of two 8-byte writes, and on gfx950
        // a sixth fewer bank-conflict cycles per LDS cycle: 0.24 against
        // 0.29); for float32 chunk 0 or 1 of the fragment
        unsigned char* base = reinterpret_cast<unsigned char*>(sm.ps[buf]) +
                              region_pos((wib * 2 + (jj >> 1)) * PPF * 4 + lg, li, lg);
        if constexpr (sizeof(T) == 2) {
          if (t & 1) store_frag<T>(reinterpret_cast<T*>(base), join(pq_even, pq));
        } else {
          store_quad<T>(reinterpret_cast<T*>(base + (t & 1) * 4 * 256), pq);
        }
      }
    };
    // gbar^T += G^T P^T over one half (32 sources) of the step in ps[buf]
    auto product = [&](int buf, int ks, const Frag<T> (&gf)[NFB]) {
#pragma unroll
      for (int ih = 0; ih < NIB; ih += 4) {
        Frag<T> pf[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) pf[q] = lds_frag(sm.ps[buf], 2, ih + q, ks);
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
          for (int q = 0; q < 4; ++q) mma(acc[ih + q][fb], gf[fb], pf[q]);
      }
    };

    // prologue: key steps jb0 and jb0+1 in LDS, weights of jb0
    {
      u32x4 kr[KPT];
      key_fetch(job.jb0, kr);
      key_stash(0, kr);
      __syncthreads();
      if (job.jb0 + 1 <= job.jb1) {
        key_fetch(job.jb0 + 1, kr);
        key_stash(1, kr);
      }
      weights(job.jb0, 0);
      __syncthreads();
    }
    // Every step issues the same global loads (past the last step they
    // re-read it, and such keys land in a buffer no later step reads): with
    // no load or consumer under a condition, the compiler's load-counter
    // waits stay exact across the loop instead of draining every load.
    Frag<T> ga[NFB], gb[NFB];
    gate_fetch(job.jb0, 0, ga);
    for (int jb = job.jb0; jb <= job.jb1; ++jb) {
      const int buf = (jb - job.jb0) & 1;
      const bool more = jb + 1 <= job.jb1;
      u32x4 kr[KPT];
      key_fetch(min(jb + 2, job.jb1), kr);
      gate_fetch(jb, 1, gb);
      product(buf, 0, ga);
      gate_fetch(min(jb + 1, job.jb1), 0, ga);
      if (more) weights(jb + 1, buf ^ 1);
      product(buf, 1, gb);
      key_stash(buf, kr);   // ks[buf] was last read by weights(jb) one step ago
      __syncthreads();
    }

    // ---- row sums: over lane groups, then over the waves sharing a block ----
    {
      const float rs = sizeof(T) == 2 ? rsum[0] : group_sum(rsum[0]);
      if (lg == 0) sm.den[wave / NIB][wib * 16 + li] = rs;
    }
    __syncthreads();
    float den[NIB];
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) {
      den[ib] = sm.den[0][ib * 16 + li];
#pragma unroll
      for (int q = 1; q < NSPLIT; ++q) den[ib] += sm.den[q][ib * 16 + li];
    }

    bool finish = job.kind == kFull;
    bool combine = false;              // add the partner's partial while storing
    int64_t obase = 0, odbase = 0;
    if (job.kind != kFull) {
      // Write this partial, then the second of the two workgroups combines.
      // The partials and the counter are accessed with agent-scope atomics
      // (coherent stores and loads that bypass the per-XCD L2s): an agent-
      // scope fence would instead write back and invalidate the whole L2 of
      // the XCD, evicting the keys and gates the other workgroups stream.
      const int slot = job.kind == kPart0 ? 0 : 1;
      const int64_t pbase = (job.split_id * 2 + slot) * (int64_t)BR * FS;
      if (has_cols) {
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
          for (int ib = 0; ib < NIB; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              __hip_atomic_store(a.part + pbase + part_index(ib * (FS / 16) + wave * NFB + fb, r, lane),
                                 acc[ib][fb][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (wave == 0 && lg == 0)
        for (int ib = 0; ib < NIB; ++ib)
          __hip_atomic_store(a.part_den + (job.split_id * 2 + slot) * BR + ib * 16 + li, den[ib],
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);   // this thread's partial stores are complete
      __syncthreads();                 // ... and every thread's
      if (tid == 0)
        sm.flag = __hip_atomic_fetch_add(&a.counters[job.split_id], 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      if (sm.flag == 1) {
        const int other = 1 - slot;
        obase = (job.split_id * 2 + other) * (int64_t)BR * FS;
        odbase = (job.split_id * 2 + other) * BR;
        if (tid == 0)
          __hip_atomic_store(&a.counters[job.split_id], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        combine = true;
        finish = true;
      }
    }

    if (finish && has_cols) {
      // The loads of a destination block (the partner's partial, or WANGO's
      // older-prefix terms) are issued together, one block ahead of its sums
      // and stores: left to itself, the compiler waits for each batch before
      // issuing the next, one memory round trip apiece.  The additions keep
      // their order (the stored values do not change).
      struct Extra {
        float part[NFB][4];
        f32x4 nold[NFB];
        float pden, zold;
      };
      auto epilogue = [&](auto comb) {
        constexpr bool C = decltype(comb)::value;
        auto fetch = [&](int ib, Extra& e) {
          const int i = i0 + ib * 16 + li;
          if constexpr (C) {
            e.pden = __hip_atomic_load(a.part_den + odbase + ib * 16 + li, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                e.part[fb][r] = __hip_atomic_load(a.part + obase + part_index(ib * (FS / 16) + wave * NFB + fb, r, lane),
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          if constexpr (MODE == 1) {
            e.zold = a.z_old[(mseq + i) * a.H + h];
#pragma unroll
            for (int fb = 0; fb < NFB; ++fb) {
              const int64_t nblk = ((mseq + i0) / 16 + ib) * (F / 16) + (col0 / 16 + in_head(fb));
              e.nold[fb] = *reinterpret_cast<const f32x4*>(a.n_old + (nblk * 64 + lane) * 4);
            }
          } else if constexpr (MODE == 2) {
            // the read-out of the state of this block's destination chunk,
            // n_old^T = S^T phi_Q^T and z_old likewise: the products the
            // scan's read-out would make, on the same bf16 parts
            constexpr int KE = DH / 32;
            const int dchunk = (i0 + ib * 16) / a.chunk;
            f32x4 nz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int fb = 0; fb < NFB; ++fb) e.nold[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (dchunk >= a.window / a.chunk) {   // block-uniform; earlier chunks have no state
              const T* st = static_cast<const T*>(a.states);
              const T* zt = static_cast<const T*>(a.zstates);
              const T* fq = static_cast<const T*>(a.fq);
              const int64_t dbase = (b * a.H + h) * (int64_t)(Tp / a.chunk) + dchunk;
              Frag<T> qb[KE];
#pragma unroll
              for (int ke = 0; ke < KE; ++ke) qb[ke] = load_frag<T>(fq + (mseq + i) * HD + h * DH + ke * 32 + lg * 8);
#pragma unroll
              for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
                for (int ke = 0; ke < KE; ++ke)
                  mma(e.nold[fb],
                      load_frag<T>(st + (((dbase * (Fh / 16) + f_base / 16 + in_head(fb)) * KE + ke) * 64 + lane) * 8),
                      qb[ke]);
#pragma unroll
              for (int ke = 0; ke < KE; ++ke) mma(nz, load_frag<T>(zt + ((dbase * KE + ke) * 64 + lane) * 8), qb[ke]);
            }
            e.zold = nz[0];
          }
        };
        auto store_block = [&](int ib, const Extra& e) {
          const int i = i0 + ib * 16 + li;
          // the two partials are added first: mine + other is the same float
          // whichever workgroup finishes last
          float dsum = den[ib];
          if constexpr (C) dsum += e.pden;
          dsum += null_w * (float)(i + 1);
          if constexpr (MODE != 0) dsum += escale * e.zold;
          // Options: the denominator for a later backward pass (one writer per
          // row: column chunk 0, wave 0); the numerator alone; rows stored in
          // reverse order (rows past the end are not stored then)
          if (a.den_out && fc == 0 && wave == 0 && lg == 0 && i < a.T) a.den_out[(mseq + i) * a.H + h] = dsum;
          const float inv = a.num_only ? 1.0f : 1.0f / dsum;
          const int64_t orow = a.rev_out ? mseq + (a.T - 1 - i) : mseq + i;
          const bool ostore = !a.rev_out || i < a.T;
#pragma unroll
          for (int fb = 0; fb < NFB; ++fb) {
            f32x4 num = acc[ib][fb];
            if constexpr (C) {
#pragma unroll
              for (int r = 0; r < 4; ++r) num[r] += e.part[fb][r];
            }
            if constexpr (MODE != 0) num += escale * e.nold[fb];
            // gbar is not head-padded: columns past the head's width are pad
            const int c = f_base + fb * 16 + lg * 4;
            if (c < a.Fho && ostore)
              store_quad<T>(gbar + orow * a.Fo + (int64_t)h * a.Fho + c, cvt_quad<T>(num * inv));
          }
        };
        Extra e0, e1;
        fetch(0, e0);
#pragma unroll
        for (int ib = 0; ib < NIB; ib += 2) {
          if (ib + 1 < NIB) fetch(ib + 1, e1);
          __builtin_amdgcn_sched_barrier(0);
          store_block(ib, e0);
          if (ib + 1 < NIB) {
            if (ib + 2 < NIB) fetch(ib + 2, e0);
            __builtin_amdgcn_sched_barrier(0);
            store_block(ib + 1, e1);
          }
        }
      };
      if (combine) epilogue(std::true_type{});
      else epilogue(std::false_type{});
    }
    __syncthreads();   // LDS is reused by the next job
  };
  run_job(job0);
  if (njobs == 2) run_job(job1);
}

__global__ void zero_i32_kernel(int* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

template <typename T, int MODE, int WC, int BR>
hipError_t launch_agg_w(const AggArgs& a, int nfc, int rtiles, int64_t items, hipStream_t s) {
  const int64_t q8 = ceil_div(items, 8);
  dim3 grid((unsigned)(8 * q8)), block(kAggThreads);
  switch (a.dh) {
    case 32: hipLaunchKernelGGL((agg_kernel<T, MODE, 32, WC, BR>), grid, block, 0, s, a, nfc, rtiles, items); break;
    case 64: hipLaunchKernelGGL((agg_kernel<T, MODE, 64, WC, BR>), grid, block, 0, s, a, nfc, rtiles, items); break;
    case 128: hipLaunchKernelGGL((agg_kernel<T, MODE, 128, WC, BR>), grid, block, 0, s, a, nfc, rtiles, items); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Gate columns per wave for a head width Fh (padded to a multiple of 64) and
// query/key width dh.  Each of the ceil(Fh / (kWaves wc)) column chunks of a
// destination tile recomputes the scores and weights, and a chunk costs the
// same whether or not every wave has columns (the waves past the width
// multiply copies), so the choice weighs the chunk count against the work
// per chunk: scores dh / 128, products wc / 16 and a fixed part 3.6 (the
// exponentials, the row sums, the epilogue; the narrower variants also run
// at a lower MFMA rate), in units of one 16-column product.  With 3.6 the
// choice is the fastest measured on gfx950 at T = 8192, dh = 128 (64-row
// tiles where the grid would underfill): 64 columns for Fh = 2048 (161 us
// against 198 with 32 and 281 with 16); 48 for Fh = 704 and 640 (two chunks
// of 384 that leave one or two wave slots idle, 86 us against 101 with 64,
// 112 with 32 and 153 with 16).  48 is a bf16 variant only.
template <typename T> int agg_wcols(int Fh, int dh) {
  const int cand[4] = {AggCfg<T>::WIDE, kMid, kNarrow, sizeof(T) == 2 ? kMid48 : kMid};
  int best = cand[0];
  double best_cost = 0.0;
  for (int c = 0; c < 4; ++c) {
    const int wc = cand[c];
    const double cost = (double)ceil_div(Fh, kWaves * wc) * (dh / 128.0 + wc / 16.0 + 3.6);
    if (c == 0 || cost < best_cost) {
      best = wc;
      best_cost = cost;
    }
  }
  return best;
}
template <typename T> int agg_fs(int Fh, int dh) { return kWaves * agg_wcols<T>(Fh, dh); }

// wc: gate columns per wave; br: destination rows per tile, AggCfg<T>::BR or
// (bf16 TANGO) kShortBR.
template <typename T, int MODE, int BR>
hipError_t launch_agg_wc(const AggArgs& a, int wc, int nfc, int rtiles, int64_t items, hipStream_t s) {
  if (wc == AggCfg<T>::WIDE) return launch_agg_w<T, MODE, AggCfg<T>::WIDE, BR>(a, nfc, rtiles, items, s);
  if (wc == kMid) return launch_agg_w<T, MODE, kMid, BR>(a, nfc, rtiles, items, s);
  if constexpr (sizeof(T) == 2) {
    if (wc == kMid48) return launch_agg_w<T, MODE, kMid48, BR>(a, nfc, rtiles, items, s);
  }
  if (wc == kNarrow) return launch_agg_w<T, MODE, kNarrow, BR>(a, nfc, rtiles, items, s);
  return hipErrorInvalidValue;
}
template <typename T, int MODE>
hipError_t launch_agg_t(const AggArgs& a, int wc, int nfc, int rtiles, int64_t items, int br, hipStream_t s) {
  constexpr int BR = AggCfg<T>::BR;
  if constexpr (MODE == 0 && BR != kShortBR) {
    if (br == kShortBR) return launch_agg_wc<T, MODE, kShortBR>(a, wc, nfc, rtiles, items, s);
  }
  if (br != BR) return hipErrorInvalidValue;
  return launch_agg_wc<T, MODE, BR>(a, wc, nfc, rtiles, items, s);
}

}  // namespace

AggPlan tango_agg_plan(int B, int Tp, int F, int H, int dh, bool bf) {
  AggPlan p;
  const int Fh = F / H;
  p.fs = bf ? agg_fs<bf16>(Fh, dh) : agg_fs<float>(Fh, dh);
  p.nfc = (int)ceil_div(Fh, p.fs);   // waves past the head's width skip
  const int64_t groups = (int64_t)B * H * p.nfc;
  auto shape = [&](int br) {
    p.br = br;
    p.rtiles = Tp / br;
    const int half = p.rtiles / 2;
    const int64_t pair_items = groups * (half + (p.rtiles & 1));
    p.split = pair_items < kFillItems ? 1 : 0;
    p.items = p.split ? groups * (2 * half + (p.rtiles & 1)) : pair_items;
    p.n_split_tiles = p.split ? groups * half : 0;
  };
  shape(bf ? AggCfg<bf16>::BR : AggCfg<float>::BR);
  // Few column chunks (narrow heads, one sequence) leave compute units idle
  // even with the long tiles split: halve the tile height to double the
  // items (each streams the same gate blocks for half the rows).
  if (bf && p.items < kFillItems && (p.fs == kWaves * AggCfg<bf16>::WIDE || p.fs == kWaves * kMid48))
    shape(kShortBR);
  return p;
}

hipError_t launch_tango_agg(const AggArgs& a, const AggPlan& p, bool bf, bool counters_clear,
                            hipStream_t s) {
  if (p.split && p.n_split_tiles > 0 && !counters_clear) {
    hipError_t e = launch_zero_i32(a.counters, p.n_split_tiles, s);
    if (e != hipSuccess) return e;
  }
  AggArgs aa = a;
  aa.split = p.split;
  return bf ? launch_agg_t<bf16, 0>(aa, p.fs / kWaves, p.nfc, p.rtiles, p.items, p.br, s)
            : launch_agg_t<float, 0>(aa, p.fs / kWaves, p.nfc, p.rtiles, p.items, p.br, s);
}

hipError_t launch_wango_band(const AggArgs& a, bool bf, hipStream_t s) {
  const int Fh = a.F / a.H;
  const int fs = bf ? agg_fs<bf16>(Fh, a.dh) : agg_fs<float>(Fh, a.dh);
  const int br = bf ? AggCfg<bf16>::BR : AggCfg<float>::BR;
  const int nfc = (int)ceil_div(Fh, fs);
  const int rtiles = a.Tp / br;
  const int64_t items = (int64_t)a.B * a.H * nfc * rtiles;
  if (a.states)   // the read-out of the chunk states in the epilogue
    return bf ? launch_agg_t<bf16, 2>(a, fs / kWaves, nfc, rtiles, items, br, s)
              : launch_agg_t<float, 2>(a, fs / kWaves, nfc, rtiles, items, br, s);
  return bf ? launch_agg_t<bf16, 1>(a, fs / kWaves, nfc, rtiles, items, br, s)
            : launch_agg_t<float, 1>(a, fs / kWaves, nfc, rtiles, items, br, s);
}

hipError_t launch_zero_i32(int* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_i32_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace tango
