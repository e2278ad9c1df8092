// gemm_kernels.hip - projection (KP) and output (KO) GEMMs of the TANGO/WANGO
// block on gfx950 MFMA.
//
// KP ("TANGO: Token-Aggregated Nonlinear Gating Operators ...", §2.1, eq. 2 and
// the head paragraph): for every (batch, position) row m,
//     [a | v | q | k] = (h_m * gain) [W_g; W_v; W_q; W_k]^T * r_m,
//     r_m = 1 / sqrt(mean(h_m^2) + eps)                          (RMSNorm)
// with the epilogue  g = a * sigmoid(a)  (stored in the packed gate layout),
// v stored row-major, and per head RoPE then unit length for q and k.  The
// RMSNorm row scale factors out of the product, so it is accumulated while the
// h tile streams through LDS and applied in the epilogue.
//
// KO (§2.1, eq. 3): out_m = h_m + (gbar_m * v_m) W_o^T, the gated product
// formed while the A tile is staged, the residual added in the epilogue.
//
// Both use a workgroup of four waves (eight for KO's wide tile) over a BM x BN
// output tile.  K
// streams through double-buffered LDS tiles of BK columns; global loads run D
// k-tiles ahead in registers and are converted (gating) only when they are
// written to LDS, so their latency overlaps D tiles of MFMA work.  Every
// 16 x 16 output block is an MFMA accumulator (see common.hpp).
//
// The KP input rows are prepared once by KX (one wave per row): the RMSNorm
// scale r_m and the parts of h_m * gain in the compute dtype, so the KP main
// loop only copies (the 34 or so column tiles of a row tile would otherwise
// each redo the conversion).
//
// In bf16 the weights are exact, but the activation operand of both products
// (h * gain, and gbar * v) is a float32 value.  The shape's operand_parts picks
// how it enters the MFMA: one part, bf16(e), the plain bf16 compute of the
// pages; or two parts, hi = bf16(e) and lo = bf16(e - hi), each multiplied
// into the same float32 accumulator, so the product sees e to about 2^-16
// relative instead of 2^-9 at twice the MFMA work.  Long stacks of shared-weight
// applications need the second part: at the first positions of a sequence
// (whose aggregate is their own gate, so their updates are the largest) the
// operand roundings compound over eight applications past 2e-2 of the output
// rms.
//
// Row tiles never straddle two sequences (the padded length is a multiple of
// 128), so a workgroup resolves its (batch, position) once.  The 1-D grid is
// mapped so that each of the eight XCDs (own L2 each) receives a contiguous
// range of tiles, walked in groups of GM row tiles with the row tile varying
// fastest (column tiles from the last): the A rows of a group stay in that
// XCD's L2 while the B tiles sweep.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace tango {

namespace {

constexpr int kThreads = 256;
constexpr int kGroupRows = 8;    // GM: row tiles per launch group
constexpr int kEpiRows = 64;     // output rows staged in LDS per epilogue pass

// BM x BN output tile, BK-wide k-tiles, WM x WN waves, register prefetch D
// k-tiles ahead, AS parts (1, or hi and lo) of the A operand; SW selects the
// LDS slot order (1: conflict-free loader writes, 0: the older order, see
// lds_slot).
template <int BM_, int BN_, int BK_, int WM_, int WN_, int D_, int AS_, int SW_ = 1>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, D = D_, AS = AS_, SW = SW_;
  static constexpr int WTM = BM / WM, WTN = BN / WN;   // wave tile
  static constexpr int IB = WTM / 16, JB = WTN / 16;   // 16 x 16 blocks per wave
  static constexpr int NT = WM * WN * 64;              // threads per workgroup
  static constexpr int CSTR = BN + 4;                  // row stride of the fp32 epilogue tile
  static_assert(NT == 256 || NT == 512, "four or eight waves");
  static_assert(BN <= 256 && BM % kEpiRows == 0 && BK % 32 == 0, "tile shape");
  static_assert(D >= 1 && D <= 4, "prefetch depth");
  static_assert(AS == 1 || AS == 2, "operand parts");
};

template <typename T, int AS> struct ProjCfg;
// (two parts keep the older slot order: with the conflict-free one the kernel
// needs two more VGPRs and drops from three waves per SIMD to two, 110 against
// 101 us)
template <> struct ProjCfg<bf16, 2> : TileCfg<128, 128, 32, 2, 2, 2, 2, 0> {};
template <> struct ProjCfg<bf16, 1> : TileCfg<128, 128, 32, 2, 2, 2, 1, 1> {};
template <> struct ProjCfg<float, 1> : TileCfg<64, 128, 32, 2, 2, 1, 1> {};
template <typename T, int AS> struct OutCfg;
// KO's K is the gate width (a multiple of 64): k-tiles of 64 halve its barriers
// (53 against 57 us at T = 8192, F = 2048, d = 512 with k-tiles of 32 and four
// tiles of prefetch).  In bf16 the A operand costs more to form than to
// multiply (gbar * v, then its parts), and every column tile of a row block
// forms it again: where 256 divides d the tile is 64 x 256 over eight waves
// (two per SIMD), which forms it half as often and re-reads the rows half as
// often (41 against 46 us at that shape with two parts); otherwise 64 x 128
// over four.
template <> struct OutCfg<bf16, 2> : TileCfg<64, 256, 64, 2, 4, 2, 2> {};
template <> struct OutCfg<bf16, 1> : TileCfg<64, 256, 64, 2, 4, 2, 1> {};
template <> struct OutCfg<float, 1> : TileCfg<64, 128, 32, 2, 2, 1, 1> {};
template <int AS> struct OutCfgNarrow : TileCfg<64, 128, 64, 2, 2, 2, AS> {};

template <typename T> constexpr int piece_elems() { return 16 / (int)sizeof(T); }

// LDS operand layout.  A tile of R rows x BK columns is stored as blocks of
// 16 rows x 32 columns; the 16-byte pieces of a block (row r, k group g =
// columns 8g .. 8g + 7, in PPF chunks h of PE elements: PPF = 1 for bf16, 2
// for float32) live in 256-byte regions, one per (chunk, group), at slot
// r xor 2g xor x, x the parity of (k block + chunk).  gfx950 serves a 16-byte
// LDS read 16 lanes (256 bytes) per clock and a 16-byte write 8 lanes (128
// bytes) per clock, each conflict-free when the lanes of the group hit
// distinct 16-byte slots modulo 256 or 128 bytes.  An MFMA fragment read (16
// lanes: rows 0..15 of one group) takes a permutation of one region; a loader
// write (consecutive lanes fetch 64 or 128 contiguous bytes of a row, which
// keeps the global loads coalesced) puts its 8 lanes -- two rows x four
// groups, or one row x (two k blocks or chunks) x four groups -- on 8
// distinct slots modulo 8.  Measured on gfx950 with SQ_LDS_BANK_CONFLICT: 8
// LDS cycles per loader write instruction, against 16 with slot r xor g and
// 32 with slot r.  SW = 0 keeps the older slot r xor g (2-way conflicted
// writes).
template <int SW> __device__ __forceinline__ int lds_slot(int r, int g, int x) {
  return SW ? r ^ (2 * g) ^ (x & 1) : r ^ g;
}
template <typename T> constexpr int frag_chunks() { return (int)sizeof(T) / 2; }   // PPF
template <class CF, typename T> constexpr int tile_chunks(int rows) {
  return rows / 16 * (CF::BK / 32) * frag_chunks<T>();
}
// Byte offset of piece (row, piece kp along the row) in a tile.
template <class CF, typename T>
__device__ __forceinline__ int piece_offset(int row, int kp) {
  constexpr int PE = 16 / (int)sizeof(T), PPF = frag_chunks<T>(), NKB = CF::BK / 32;
  const int kb = kp * PE / 32, within = kp % (32 / PE);
  const int g = within / PPF, h = within % PPF, r = row & 15;
  const int region = (((row >> 4) * NKB + kb) * PPF + h) * 4 + g;
  return region * 256 + lds_slot<CF::SW>(r, g, kb + h) * 16;
}
template <class CF, typename T> constexpr size_t ops_bytes() {
  return 2 * (size_t)tile_chunks<CF, T>(CF::AS * CF::BM + CF::BN) * 1024;
}
template <class CF> constexpr size_t epi_bytes() { return (size_t)kEpiRows * CF::CSTR * sizeof(float); }
// Operand buffers (reused for the epilogue tile), then BM row scales, then
// the RoPE frequencies of one head (at most 64 pairs, float64).
constexpr int kMaxPairs = 64;
template <class CF, typename T> constexpr size_t main_bytes() {
  return (ops_bytes<CF, T>() > epi_bytes<CF>() ? ops_bytes<CF, T>() : epi_bytes<CF>()) +
         (size_t)CF::BM * sizeof(float) + kMaxPairs * sizeof(double);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// v (the W_v projection) is stored in T with one bf16 operand part: the output
// GEMM rounds gbar * v to bf16 anyway.  With two parts (and in float32) it is
// float32, unrounded: the output GEMM then carries gbar * v to about 2^-16,
// and a bf16 v would add a rounding that compounds through stacked
// applications.
template <typename T, int AS> constexpr bool v_half() { return std::is_same<T, bf16>::value && AS == 1; }
// One 16-byte LDS piece per operand part.
template <int AS> struct Parts {
  u32x4 p[AS];
};

// Round PE float32 values to T parts: hi = T(e), and with AS = 2 also
// lo = T(e - hi) (e - hi is exact in float32).
template <typename T, int AS, int PE>
__device__ __forceinline__ Parts<AS> split_parts(const float (&e)[PE]) {
  Parts<AS> out;
  T* hi = reinterpret_cast<T*>(&out.p[0]);
#pragma unroll
  for (int q = 0; q < PE; ++q) hi[q] = cvt<T>(e[q]);
  if constexpr (AS == 2) {
    T* lo = reinterpret_cast<T*>(&out.p[1]);
#pragma unroll
    for (int q = 0; q < PE; ++q) lo[q] = cvt<T>(e[q] - tof<T>(hi[q]));
  }
  return out;
}

template <typename IO, int N> struct IOVec {
  typedef IO type __attribute__((ext_vector_type(N)));
};

template <int V> using IC = std::integral_constant<int, V>;

// Output tile of this workgroup (see the file header for the order).
struct TilePos {
  int64_t m_tile;
  int n_tile;
};
__device__ __forceinline__ TilePos tile_of(int64_t nm, int nn) {
  const int64_t L = blockIdx.x, NT = nm * nn;
  const int64_t q = NT / 8, r = NT % 8, x = L % 8;
  const int64_t t = x * q + (x < r ? x : r) + L / 8;   // contiguous range per XCD
  const int64_t gsz = (int64_t)kGroupRows * nn;
  const int64_t g = t / gsz, w = t - g * gsz;
  const int64_t first = g * kGroupRows;
  const int64_t rows = nm - first < kGroupRows ? nm - first : kGroupRows;
  // last column tile first: in KP those hold the queries and keys, whose
  // epilogue is the longest, so they start early instead of forming a tail
  return {first + w % rows, nn - 1 - (int)(w / rows)};
}

// The MFMA inner product of one BK-wide LDS tile for one wave.
// Fragment (row block rb, k block kb) of a tile, this lane.
template <class CF, typename T>
__device__ __forceinline__ Frag<T> lds_frag(const T* tile, int rb, int kb, int lane) {
  constexpr int PPF = frag_chunks<T>(), NKB = CF::BK / 32;
  const int r = lane & 15, g = lane >> 4;
  const unsigned char* base = reinterpret_cast<const unsigned char*>(tile) + ((rb * NKB + kb) * PPF * 4 + g) * 256;
  if constexpr (PPF == 1) {
    return load_frag<T>(reinterpret_cast<const T*>(base + lds_slot<CF::SW>(r, g, kb) * 16));
  } else {
    return join(load_quad<T>(reinterpret_cast<const T*>(base + lds_slot<CF::SW>(r, g, kb) * 16)),
                load_quad<T>(reinterpret_cast<const T*>(base + 4 * 256 + lds_slot<CF::SW>(r, g, kb + 1) * 16)));
  }
}

template <class CF, typename T>
__device__ __forceinline__ void tile_mma(f32x4 (&acc)[CF::IB][CF::JB], const T* __restrict__ As,
                                         const T* __restrict__ Bs, int wr, int wc, int lane) {
#pragma unroll
  for (int ks = 0; ks < CF::BK / 32; ++ks) {
    Frag<T> b[CF::JB];
#pragma unroll
    for (int j = 0; j < CF::JB; ++j) b[j] = lds_frag<CF, T>(Bs, wc * CF::JB + j, ks, lane);
#pragma unroll
    for (int i = 0; i < CF::IB; ++i) {
#pragma unroll
      for (int part = 0; part < CF::AS; ++part) {   // A parts live BM rows apart
        const Frag<T> a = lds_frag<CF, T>(As, part * (CF::BM / 16) + wr * CF::IB + i, ks, lane);
#pragma unroll
        for (int j = 0; j < CF::JB; ++j) mma(acc[i][j], a, b[j]);
      }
    }
  }
}

// Piece loaded by this thread in pass p: PR = BK / PE consecutive threads
// cover one row of the tile.
template <class CF, typename T> struct PiecePos {
  int row, kp;
};
template <class CF, typename T>
__device__ __forceinline__ PiecePos<CF, T> piece_pos(int tid, int p) {
  constexpr int PR = CF::BK / (16 / (int)sizeof(T)), RPP = CF::NT / PR;
  return {tid / PR + p * RPP, tid % PR};
}

// Main loop.  SA / SB supply this thread's 16-byte pieces of the A (BM x BK)
// and B (BN x BK) tiles (pass p: the piece at piece_pos(tid, p)):
// fetch(raw, p, k0) issues the global load for the k-tile starting at column
// k0, convert(raw, p) turns it into the 16-byte pieces stored to LDS (one per
// operand part).  At the top of step kt,
// LDS buffer kt & 1 holds tile kt and register set (kt + j) % D holds tile
// kt + j for j = 1..D.
template <class CF, typename T, class SA, class SB>
__device__ __forceinline__ void gemm_mainloop(f32x4 (&acc)[CF::IB][CF::JB], T* lds, int nk, SA& sa,
                                              SB& sb) {
  constexpr int PE = piece_elems<T>(), D = CF::D;
  constexpr int PA = tile_chunks<CF, T>(CF::BM) * 64 / CF::NT, PB = tile_chunks<CF, T>(CF::BN) * 64 / CF::NT;
  static_assert(PA >= 1 && PB >= 1, "every thread loads a piece of each tile");
  constexpr int TA = tile_chunks<CF, T>(CF::AS * CF::BM) * 64 * PE;   // elements
  constexpr int TB = tile_chunks<CF, T>(CF::BN) * 64 * PE;
  constexpr int PART = tile_chunks<CF, T>(CF::BM) * 64 * PE;          // A part stride
  const int tid = threadIdx.x, lane = tid & 63;
  int a_off[PA], b_off[PB];   // byte offsets of this thread's pieces in a tile
#pragma unroll
  for (int p = 0; p < PA; ++p) {
    const PiecePos<CF, T> pp = piece_pos<CF, T>(tid, p);
    a_off[p] = piece_offset<CF, T>(pp.row, pp.kp);
  }
#pragma unroll
  for (int p = 0; p < PB; ++p) {
    const PiecePos<CF, T> pp = piece_pos<CF, T>(tid, p);
    b_off[p] = piece_offset<CF, T>(pp.row, pp.kp);
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave / CF::WN, wc = wave % CF::WN;
  typename SA::raw ra[D][PA];
  typename SB::raw rb[D][PB];
  auto fetch = [&](auto set, int kt) {
    constexpr int s = decltype(set)::value;
#pragma unroll
    for (int p = 0; p < PA; ++p) sa.fetch(ra[s][p], p, kt * CF::BK);
#pragma unroll
    for (int p = 0; p < PB; ++p) sb.fetch(rb[s][p], p, kt * CF::BK);
  };
  auto stash = [&](auto set, int kt) {
    constexpr int s = decltype(set)::value;
    unsigned char* As = reinterpret_cast<unsigned char*>(lds + (kt & 1) * TA);
    unsigned char* Bs = reinterpret_cast<unsigned char*>(lds + 2 * TA + (kt & 1) * TB);
#pragma unroll
    for (int p = 0; p < PA; ++p) {
      const Parts<CF::AS> pa = sa.convert(ra[s][p], p);
#pragma unroll
      for (int part = 0; part < CF::AS; ++part)
        *reinterpret_cast<u32x4*>(As + part * PART * (int)sizeof(T) + a_off[p]) = pa.p[part];
    }
#pragma unroll
    for (int p = 0; p < PB; ++p) *reinterpret_cast<u32x4*>(Bs + b_off[p]) = sb.convert(rb[s][p], p);
  };
  // Fetches past the last tile re-read the last one (never stashed): every
  // step issues the same loads, so the wait before a stash only covers the
  // set being stashed.
  auto step = [&](auto set, int kt) {
    tile_mma<CF, T>(acc, lds + (kt & 1) * TA, lds + 2 * TA + (kt & 1) * TB, wr, wc, lane);
    if (kt + 1 < nk) stash(set, kt + 1);
    fetch(set, min(kt + 1 + D, nk - 1));
    __syncthreads();
  };
  fetch(IC<0>{}, 0);
  stash(IC<0>{}, 0);
  fetch(IC<1 % D>{}, min(1, nk - 1));
  if constexpr (D > 1) fetch(IC<2 % D>{}, min(2, nk - 1));
  if constexpr (D > 2) fetch(IC<3 % D>{}, min(3, nk - 1));
  if constexpr (D > 3) fetch(IC<4 % D>{}, min(4, nk - 1));
  __syncthreads();
  // step kt uses register set (kt + 1) % D; the loop is unrolled by D so that
  // the set is a compile-time index
  int kt = 0;
  for (; kt + D <= nk; kt += D) {
    step(IC<1 % D>{}, kt);
    if constexpr (D > 1) step(IC<2 % D>{}, kt + 1);
    if constexpr (D > 2) step(IC<3 % D>{}, kt + 2);
    if constexpr (D > 3) step(IC<4 % D>{}, kt + 3);
  }
  if (kt < nk) step(IC<1 % D>{}, kt);
  if constexpr (D > 1) if (kt + 1 < nk) step(IC<2 % D>{}, kt + 1);
  if constexpr (D > 2) if (kt + 2 < nk) step(IC<3 % D>{}, kt + 2);
}

// Rows of plain T matrices (the weights): one pointer per pass, at the
// piece's row and column; a row past the end points at a valid row and is
// replaced by zeros when stored.
template <typename T, int P> struct RowSource {
  struct raw {
    u32x4 v;
  };
  const T* ptr[P];
  bool ok[P];
  __device__ __forceinline__ void fetch(raw& r, int p, int k0) const {
    r.v = *reinterpret_cast<const u32x4*>(ptr[p] + k0);
  }
  __device__ __forceinline__ u32x4 convert(const raw& r, int p) const {
    return ok[p] ? r.v : u32x4{0u, 0u, 0u, 0u};
  }
};

// A of KP: the AS parts of the prepared rows (plain copies).
template <typename T, int P, int AS> struct PartsSource {
  struct raw {
    u32x4 v[AS];
  };
  const T* ptr[P];      // part 0 at the piece; part q lies q * part_stride further
  int64_t part_stride;
  __device__ __forceinline__ void fetch(raw& r, int p, int k0) const {
#pragma unroll
    for (int q = 0; q < AS; ++q) r.v[q] = *reinterpret_cast<const u32x4*>(ptr[p] + q * part_stride + k0);
  }
  __device__ __forceinline__ Parts<AS> convert(const raw& r, int) const {
    Parts<AS> out;
#pragma unroll
    for (int q = 0; q < AS; ++q) out.p[q] = r.v[q];
    return out;
  }
};

// A of KO: gbar * v, formed in float and rounded to T parts.
// Column of gate column n (0 .. F-1) in the head-padded gate layout: head a's
// columns start at a * Fhp.
__device__ __forceinline__ int pad_col(int n, int Fh, int Fhp) {
  return Fh == Fhp ? n : n + (n / Fh) * (Fhp - Fh);
}

// A piece of PE gates meets the PE values of v in VP 16-byte loads (one when
// v is stored in T, PE / 4 when it is float32).
template <typename T, int P, int AS> struct GatedSource {
  static constexpr int PE = piece_elems<T>();
  using VT = typename std::conditional<v_half<T, AS>(), T, float>::type;
  static constexpr int VE = 16 / (int)sizeof(VT);   // v values per 16-byte load
  static constexpr int VP = PE / VE;
  struct raw {
    u32x4 g;
    u32x4 v[VP];
  };
  const T* gptr[P];     // at the piece's row and column
  const VT* vptr[P];
  __device__ __forceinline__ void fetch(raw& r, int p, int k0) const {
    r.g = *reinterpret_cast<const u32x4*>(gptr[p] + k0);
#pragma unroll
    for (int q = 0; q < VP; ++q) r.v[q] = *reinterpret_cast<const u32x4*>(vptr[p] + k0 + VE * q);
  }
  __device__ __forceinline__ Parts<AS> convert(const raw& r, int) const {
    const T* ge = reinterpret_cast<const T*>(&r.g);
    const VT* ve = reinterpret_cast<const VT*>(&r.v[0]);
    float e[PE];
#pragma unroll
    for (int q = 0; q < PE; ++q) e[q] = tof<T>(ge[q]) * tof<VT>(ve[q]);
    return split_parts<T, AS, PE>(e);
  }
};

// Write the accumulator blocks that fall into epilogue pass `pass` (tile rows
// [64 pass, 64 pass + 64)), times the row scale rs[row] (or 1), to the fp32
// LDS tile Cs[64][CF::CSTR].
template <class CF>
__device__ __forceinline__ void acc_to_lds(const f32x4 (&acc)[CF::IB][CF::JB], float* Cs,
                                           const float* rs, int pass) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave / CF::WN, wc = wave % CF::WN, col = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int i = 0; i < CF::IB; ++i) {
    const int r0 = wr * CF::WTM + i * 16;
    if (r0 / kEpiRows != pass) continue;
#pragma unroll
    for (int j = 0; j < CF::JB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = r0 + grp * 4 + r;
        const float s = rs ? rs[row] : 1.0f;
        Cs[(row - pass * kEpiRows) * CF::CSTR + wc * CF::WTN + j * 16 + col] = acc[i][j][r] * s;
      }
  }
}

template <typename IO, int N>
__device__ __forceinline__ void load_io(const IO* p, float (&v)[N]) {
  const typename IOVec<IO, N>::type r = *reinterpret_cast<const typename IOVec<IO, N>::type*>(p);
#pragma unroll
  for (int q = 0; q < N; ++q) v[q] = (float)r[q];
}
template <typename IO, int N>
__device__ __forceinline__ void store_io(IO* p, const float (&v)[N]) {
  typename IOVec<IO, N>::type r;
#pragma unroll
  for (int q = 0; q < N; ++q) r[q] = cvt<IO>(v[q]);
  *reinterpret_cast<typename IOVec<IO, N>::type*>(p) = r;
}

}  // namespace

// ---------------------------------------------------------------------------
// KX: RMSNorm scales and operand parts of the KP input rows, one wave per
// padded row m:  rinv[m] = 1 / sqrt(mean(h_m^2) + eps)  ([TANGO] §2.1, the
// RMSNorm before eq. 2) and the AS parts of h_m * gain in T; rows past the end
// of a sequence are zero.  Grid: M_pad / 4 workgroups of 256.
// ---------------------------------------------------------------------------
template <typename T, typename IO, int AS>
__global__ __launch_bounds__(kThreads) void prep_kernel(ProjArgs args) {
  const int lane = threadIdx.x & 63;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < args.zero_n;
       i += (int64_t)gridDim.x * kThreads)
    args.zero[i] = 0;
  const int64_t m = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int d = args.d, Tp = args.Tp, T_len = args.T;
  const int64_t M = (int64_t)args.B * Tp;
  if (m >= M) return;
  const int64_t b = m / Tp;
  const int t = (int)(m - b * Tp);
  T* out = static_cast<T*>(args.xs) + m * d;
  const T* gain = static_cast<const T*>(args.gain);
  const IO* src = static_cast<const IO*>(args.x) + (b * T_len + (t < T_len ? t : 0)) * d;
  float ss = 0.f;
  for (int k = lane * 8; k < d; k += 64 * 8) {
    float e[8];
    if (t < T_len) {
      load_io<IO, 8>(src + k, e);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) e[q] = 0.f;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) ss += e[q] * e[q];
    if (gain) {
      const Frag<T> g = load_frag<T>(gain + k);
#pragma unroll
      for (int q = 0; q < 8; ++q) e[q] *= tof<T>(g[q]);
    }
    Frag<T> hi;
#pragma unroll
    for (int q = 0; q < 8; ++q) hi[q] = cvt<T>(e[q]);
    store_frag<T>(out + k, hi);
    if constexpr (AS == 2) {
      Frag<T> lo;
#pragma unroll
      for (int q = 0; q < 8; ++q) lo[q] = cvt<T>(e[q] - tof<T>(hi[q]));
      store_frag<T>(out + M * d + k, lo);
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) args.rinv[m] = t < T_len ? 1.0f / sqrtf(ss / (float)d + args.eps) : 0.f;
}

// ---------------------------------------------------------------------------
// KP: [W_g; W_v; W_q; W_k] projection of the prepared rows + epilogue.
// 1-D grid over (M_pad / BM) x ceil(N / BN) tiles, N = 2F + 2HD, M_pad = B * Tp.
// ---------------------------------------------------------------------------
template <typename T, typename IO, int AS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void proj_kernel(ProjArgs args) {
  using CF = ProjCfg<T, AS>;
  constexpr int PA = tile_chunks<CF, T>(CF::BM) / 4, PB = tile_chunks<CF, T>(CF::BN) / 4;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* lds = reinterpret_cast<T*>(smem_raw);
  constexpr size_t kRsOff = main_bytes<CF, T>() - kMaxPairs * sizeof(double) - CF::BM * sizeof(float);
  float* rs = reinterpret_cast<float*>(smem_raw + kRsOff);
  double* rev_freq = reinterpret_cast<double*>(smem_raw + kRsOff + CF::BM * sizeof(float));

  const int d = args.d, F = args.F, HD = args.HD, Tp = args.Tp;
  const int N = 2 * F + 2 * HD;
  const int64_t M = (int64_t)args.B * Tp;
  const TilePos tp = tile_of(M / CF::BM, (int)ceil_div(N, CF::BN));
  const int n0 = tp.n_tile * CF::BN;
  const int64_t m0 = tp.m_tile * CF::BM;
  const int64_t bseq = m0 / Tp;
  const int t0 = (int)(m0 - bseq * Tp);   // position of the tile's first row
  const int tid = threadIdx.x;

  PartsSource<T, PA, CF::AS> sa;
  sa.part_stride = M * d;
#pragma unroll
  for (int p = 0; p < PA; ++p) {
    const PiecePos<CF, T> pp = piece_pos<CF, T>(tid, p);
    sa.ptr[p] = static_cast<const T*>(args.xs) + (m0 + pp.row) * d + pp.kp * piece_elems<T>();
  }
  RowSource<T, PB> sb;
#pragma unroll
  for (int p = 0; p < PB; ++p) {
    const PiecePos<CF, T> pp = piece_pos<CF, T>(tid, p);
    const int n = n0 + pp.row;
    const T* w = static_cast<const T*>(args.w_g);
    if (n < F) w = static_cast<const T*>(args.w_g) + (int64_t)n * d;
    else if (n < 2 * F) w = static_cast<const T*>(args.w_v) + (int64_t)(n - F) * d;
    else if (n < 2 * F + HD) w = static_cast<const T*>(args.w_q) + (int64_t)(n - 2 * F) * d;
    else if (n < N) w = static_cast<const T*>(args.w_k) + (int64_t)(n - 2 * F - HD) * d;
    sb.ptr[p] = w + pp.kp * piece_elems<T>();
    sb.ok[p] = n < N;
  }

  f32x4 acc[CF::IB][CF::JB];
#pragma unroll
  for (int i = 0; i < CF::IB; ++i)
#pragma unroll
    for (int j = 0; j < CF::JB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  gemm_mainloop<CF, T>(acc, lds, d / CF::BK, sa, sb);

  const int dh = args.dh;
  const bool has_qk = n0 + CF::BN > 2 * F;
  // RMSNorm row scales, and for the query/key tiles the RoPE rotation rate of
  // pair c, base^(-2c/d_h) in revolutions per position (float64: positions
  // reach 65,535); both live past the operand buffers
  if (tid < CF::BM) rs[tid] = args.rinv[m0 + tid];
  if (has_qk && tid < dh / 2)
    rev_freq[tid] = args.rope_base > 0.f
        ? pow((double)args.rope_base, -2.0 * (double)tid / (double)dh) * 0.15915494309189533577
        : 0.0;
  __syncthreads();
  float* Cs = reinterpret_cast<float*>(smem_raw);

  if (n0 + CF::BN <= F) {
    // Gate tile: a lane holds column l % 16 of two stacked 16-row blocks, rows
    // 4 (l / 16) + r and 16 + 4 (l / 16) + r of a 32-row block: exactly the 8
    // slots of its piece of the packed layout, stored with SiLU applied.
    T* gp = static_cast<T*>(args.gp);
    const int lane = tid & 63, col = lane & 15, grp = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave / CF::WN, wc = wave % CF::WN;
    static_assert(CF::IB % 2 == 0, "32-row blocks");
#pragma unroll
    for (int i = 0; i < CF::IB; i += 2) {
      const int r0 = wr * CF::WTM + i * 16;
      float sl[4], sh[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sl[r] = rs[r0 + grp * 4 + r];
        sh[r] = rs[r0 + 16 + grp * 4 + r];
      }
#pragma unroll
      for (int j = 0; j < CF::JB; ++j) {
        Frag<T> out;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = acc[i][j][r] * sl[r], b = acc[i + 1][j][r] * sh[r];
          out[r] = cvt<T>(a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)));
          out[4 + r] = cvt<T>(b * __builtin_amdgcn_rcpf(1.0f + __expf(-b)));
        }
        store_frag<T>(gp + packed_offset((m0 + r0) / 32, grp,
                                         pad_col(n0 + wc * CF::WTN + j * 16 + col, args.Fh, args.Fhp), args.Fp),
                      out);
      }
    }
    return;
  }

  for (int pass = 0; pass < CF::BM / kEpiRows; ++pass) {
    if (pass) __syncthreads();   // the previous pass is done with Cs
    acc_to_lds<CF>(acc, Cs, rs, pass);
    __syncthreads();
    const int64_t mp = m0 + pass * kEpiRows;   // first row of this pass
    const int tpos = t0 + pass * kEpiRows;     // its position in the sequence
    constexpr int NRB = kEpiRows / 32;

    // gates: packed layout, 8 rows (one permuted 32-row group slot set) per item
    if (n0 < F) {
      T* gp = static_cast<T*>(args.gp);
      for (int it = tid; it < NRB * 4 * CF::BN; it += kThreads) {
        const int c = it % CF::BN, grp = (it / CF::BN) & 3, rb = it / (4 * CF::BN);
        const int n = n0 + c;
        if (n >= F) continue;
        Frag<T> out;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const float a = Cs[(rb * 32 + perm_slot(grp, s)) * CF::CSTR + c];
          out[s] = cvt<T>(a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)));
        }
        store_frag<T>(gp + packed_offset(mp / 32 + rb, grp, pad_col(n, args.Fh, args.Fhp), args.Fp), out);
      }
    }
    // v: row-major [M_pad, F], in T with one bf16 operand part, else float32
    // (v_half)
    if (v_half<T, AS>() && n0 + CF::BN > F && n0 < 2 * F) {
      T* v = static_cast<T*>(args.v);
      constexpr int P8 = CF::BN / 8;
      for (int it = tid; it < kEpiRows * P8; it += kThreads) {
        const int row = it / P8, c = (it % P8) * 8;
        const int n = n0 + c;
        if (n < F || n >= 2 * F) continue;   // F is a multiple of 64: pieces lie on one side
        Frag<T> o;
#pragma unroll
        for (int s = 0; s < 8; ++s) o[s] = cvt<T>(Cs[row * CF::CSTR + c + s]);
        store_frag<T>(v + (mp + row) * F + (n - F), o);
      }
    } else if (n0 + CF::BN > F && n0 < 2 * F) {
      float* v = static_cast<float*>(args.v);
      constexpr int P4 = CF::BN / 4;
      for (int it = tid; it < kEpiRows * P4; it += kThreads) {
        const int row = it / P4, c = (it % P4) * 4;
        const int n = n0 + c;
        if (n < F || n >= 2 * F) continue;
        *reinterpret_cast<f32x4*>(v + (mp + row) * F + (n - F)) =
            *reinterpret_cast<const f32x4*>(&Cs[row * CF::CSTR + c]);
      }
    }
    // queries and keys: RoPE on interleaved pairs, then unit length per head.
    // A thread takes 16 pairs (32 columns) of one row; the dh / 32 threads of a
    // (row, head) are consecutive lanes and reduce the squared norm together.
    if (has_qk) {
      const int c_lo = n0 < 2 * F ? 2 * F - n0 : 0;  // first q/k column in tile
      const int c_hi = min(CF::BN, N - n0);
      const int nq = (c_hi - c_lo) / 32;             // 32-column quarters per row
      const int qph = dh / 32;                       // quarters per head
      const float isd = 1.0f / sqrtf((float)dh);
      for (int item = tid; item < kEpiRows * nq; item += kThreads) {   // block-uniform trip count
        const int row = item / nq, q = item % nq;
        const int hcol = c_lo + q * 32;             // first column of this quarter in the tile
        const int pair0 = (q % qph) * 16;           // first pair within the head
        float u[32];
#pragma unroll
        for (int e4 = 0; e4 < 8; ++e4) {
          const f32x4 t4 = *reinterpret_cast<const f32x4*>(&Cs[row * CF::CSTR + hcol + e4 * 4]);
#pragma unroll
          for (int r = 0; r < 4; ++r) u[e4 * 4 + r] = t4[r];
        }
        if (args.rope_base > 0.f) {
          const double pos = (double)(tpos + row);
#pragma unroll
          for (int p = 0; p < 16; ++p) {
            const double rev = pos * rev_freq[pair0 + p];
            const float fr = (float)(rev - rint(rev));
            const float fs = __builtin_amdgcn_sinf(fr), fc = __builtin_amdgcn_cosf(fr);
            const float a0 = u[2 * p], a1 = u[2 * p + 1];
            u[2 * p] = a0 * fc - a1 * fs;
            u[2 * p + 1] = a0 * fs + a1 * fc;
          }
        }
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 32; ++e) ss += u[e] * u[e];
        for (int off = 1; off < qph; off <<= 1) ss += __shfl_xor(ss, off, 64);
        const float inv = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
        const int n = n0 + hcol;
        const bool is_q = n < 2 * F + HD;
        const int e0 = is_q ? n - 2 * F : n - 2 * F - HD;   // first column within q or k
        Frag<T> w[4];
#pragma unroll
        for (int e = 0; e < 32; ++e) w[e / 8][e % 8] = cvt<T>(u[e] * inv);
        T* dst = (is_q ? static_cast<T*>(args.qh) : static_cast<T*>(args.kh)) + (mp + row) * HD + e0;
#pragma unroll
        for (int c8 = 0; c8 < 4; ++c8) store_frag<T>(dst + c8 * 8, w[c8]);
        if (args.fq) {
          // WANGO features phi(sqrt(tau) u) ([TANGO] §2.2 eq. 8) of the stored
          // unit vector: queries go out in the permuted feature order of their
          // group of 32, keys back into the tile for the packed store below
          const float st = sqrtf(__expf(fminf(args.theta[e0 / dh], 2.995732273553991f)));
          float ph[32];
#pragma unroll
          for (int e = 0; e < 32; ++e) ph[e] = phi_feature(st * tof<T>(w[e / 8][e % 8]), isd);
          if (is_q) {
            Frag<T> fqv[4];
#pragma unroll
            for (int e = 0; e < 32; ++e) {
              const int slot = feature_slot(e);
              fqv[slot / 8][slot % 8] = cvt<T>(ph[e]);
            }
            T* fqd = static_cast<T*>(args.fq) + (mp + row) * HD + e0;
#pragma unroll
            for (int c8 = 0; c8 < 4; ++c8) store_frag<T>(fqd + c8 * 8, fqv[c8]);
          } else {
#pragma unroll
            for (int e4 = 0; e4 < 8; ++e4)
              *reinterpret_cast<f32x4*>(&Cs[row * CF::CSTR + hcol + e4 * 4]) =
                  f32x4{ph[e4 * 4], ph[e4 * 4 + 1], ph[e4 * 4 + 2], ph[e4 * 4 + 3]};
          }
        }
      }
      if (args.fk) {
        // key features in the source-packed layout, as the gates
        __syncthreads();
        const int k_lo = max(c_lo, 2 * F + HD - n0);
        if (k_lo < c_hi) {
          T* fk = static_cast<T*>(args.fk);
          const int ncols = c_hi - k_lo;
          for (int it = tid; it < NRB * 4 * ncols; it += kThreads) {
            const int c2 = k_lo + it % ncols, grp = (it / ncols) & 3, rb = it / (4 * ncols);
            Frag<T> out;
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2)
              out[s2] = cvt<T>(Cs[(rb * 32 + perm_slot(grp, s2)) * CF::CSTR + c2]);
            store_frag<T>(fk + packed_offset(mp / 32 + rb, grp, n0 + c2 - 2 * F - HD, HD), out);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// KO: out = x + (gbar * v) W_o^T.  1-D grid over (M_pad / BM) x (d / BN) tiles.
// ---------------------------------------------------------------------------
template <typename T, typename IO, class CF>
__global__ __launch_bounds__(CF::NT) void out_kernel(OutArgs args) {
  constexpr int PA = tile_chunks<CF, T>(CF::BM) * 64 / CF::NT, PB = tile_chunks<CF, T>(CF::BN) * 64 / CF::NT;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* lds = reinterpret_cast<T*>(smem_raw);
  const int d = args.d, F = args.F, T_len = args.T, Tp = args.Tp;
  const TilePos tp = tile_of((int64_t)args.B * Tp / CF::BM, d / CF::BN);
  const int n0 = tp.n_tile * CF::BN;
  const int64_t m0 = tp.m_tile * CF::BM;
  const int64_t bseq = m0 / Tp;
  const int t0 = (int)(m0 - bseq * Tp);
  const int tid = threadIdx.x;

  GatedSource<T, PA, CF::AS> sa;
#pragma unroll
  for (int p = 0; p < PA; ++p) {
    const PiecePos<CF, T> pp = piece_pos<CF, T>(tid, p);
    const int64_t off = (m0 + pp.row) * F + pp.kp * piece_elems<T>();
    sa.gptr[p] = static_cast<const T*>(args.gbar) + off;
    sa.vptr[p] = static_cast<const typename GatedSource<T, PA, CF::AS>::VT*>(args.v) + off;
  }
  RowSource<T, PB> sb;
#pragma unroll
  for (int p = 0; p < PB; ++p) {
    const PiecePos<CF, T> pp = piece_pos<CF, T>(tid, p);
    sb.ptr[p] = static_cast<const T*>(args.w_o) + (int64_t)(n0 + pp.row) * F + pp.kp * piece_elems<T>();
    sb.ok[p] = true;
  }

  f32x4 acc[CF::IB][CF::JB];
#pragma unroll
  for (int i = 0; i < CF::IB; ++i)
#pragma unroll
    for (int j = 0; j < CF::JB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  gemm_mainloop<CF, T>(acc, lds, F / CF::BK, sa, sb);

  float* Cs = reinterpret_cast<float*>(smem_raw);
  const IO* __restrict__ x = static_cast<const IO*>(args.x);
  IO* out = static_cast<IO*>(args.out);
  constexpr int P8 = CF::BN / 8;
  for (int pass = 0; pass < CF::BM / kEpiRows; ++pass) {
    if (pass) __syncthreads();   // the previous pass is done with Cs
    acc_to_lds<CF>(acc, Cs, nullptr, pass);
    __syncthreads();
    for (int it = tid; it < kEpiRows * P8; it += CF::NT) {
      const int row = it / P8, c = (it % P8) * 8;
      const int t = t0 + pass * kEpiRows + row;
      if (t >= T_len) continue;
      const int64_t off = (bseq * T_len + t) * d + n0 + c;
      float o[8];
      load_io<IO, 8>(x + off, o);
#pragma unroll
      for (int s = 0; s < 8; ++s) o[s] += Cs[row * CF::CSTR + c + s];
      store_io<IO, 8>(out + off, o);
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <typename T, typename IO, int AS>
hipError_t launch_proj_t(const ProjArgs& a, hipStream_t s) {
  using CF = ProjCfg<T, AS>;
  const int64_t M = (int64_t)a.B * a.Tp;
  hipLaunchKernelGGL((prep_kernel<T, IO, AS>), dim3((unsigned)(M / (kThreads / 64))), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int N = 2 * a.F + 2 * a.HD;
  const int64_t tiles = (M / CF::BM) * ceil_div(N, CF::BN);
  const size_t lds = main_bytes<CF, T>();
  hipLaunchKernelGGL((proj_kernel<T, IO, AS>), dim3((unsigned)tiles), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <typename T, typename IO, class CF>
hipError_t launch_out_cf(const OutArgs& a, hipStream_t s) {
  if (a.d % CF::BN != 0) return hipErrorInvalidValue;
  const int64_t tiles = ((int64_t)a.B * a.Tp / CF::BM) * (a.d / CF::BN);
  const size_t lds = main_bytes<CF, T>();
  hipLaunchKernelGGL((out_kernel<T, IO, CF>), dim3((unsigned)tiles), dim3(CF::NT), lds, s, a);
  return hipGetLastError();
}
template <typename T, typename IO, int AS>
hipError_t launch_out_t(const OutArgs& a, hipStream_t s) {
  if constexpr (std::is_same<T, bf16>::value) {
    if (a.d % OutCfg<T, AS>::BN != 0) return launch_out_cf<T, IO, OutCfgNarrow<AS>>(a, s);
  }
  return launch_out_cf<T, IO, OutCfg<T, AS>>(a, s);
}

// Pad columns of the head-padded packed gates: one 16-byte piece (8 rows of
// one column) per thread and item.
template <typename T>
__global__ void zero_pad_kernel(T* gp, int64_t M, int H, int Fh, int Fhp) {
  const int npad = Fhp - Fh, Fp = H * Fhp;
  const int64_t n_g = (M / 32) * 4 * H * (int64_t)npad;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_g; i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % npad);
    const int64_t r = i / npad;
    const int h = (int)(r % H);
    const int64_t bg = r / H;                               // (blk, grp)
    *reinterpret_cast<u32x4*>(gp + (bg * Fp + h * Fhp + Fh + c) * 8) = z;
  }
}

template <typename T, typename IO, int AS>
hipError_t launch_prep_t(const ProjArgs& a, hipStream_t s) {
  const int64_t M = (int64_t)a.B * a.Tp;
  hipLaunchKernelGGL((prep_kernel<T, IO, AS>), dim3((unsigned)(M / (kThreads / 64))), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_zero_pad(void* gp, int64_t M, int H, int Fh, int Fhp, bool bf, hipStream_t s) {
  if (Fh == Fhp) return hipSuccess;
  const unsigned grid = 1024;
  if (bf)
    hipLaunchKernelGGL(zero_pad_kernel<bf16>, dim3(grid), dim3(256), 0, s, static_cast<bf16*>(gp), M, H, Fh, Fhp);
  else
    hipLaunchKernelGGL(zero_pad_kernel<float>, dim3(grid), dim3(256), 0, s, static_cast<float*>(gp), M, H, Fh,
                       Fhp);
  return hipGetLastError();
}

// bf16 takes one or two operand parts (a.parts); float32 one.
hipError_t launch_prep(const ProjArgs& a, bool bf, bool io_bf, hipStream_t s) {
  if (bf && a.parts == 2) return io_bf ? launch_prep_t<bf16, bf16, 2>(a, s) : launch_prep_t<bf16, float, 2>(a, s);
  if (bf) return io_bf ? launch_prep_t<bf16, bf16, 1>(a, s) : launch_prep_t<bf16, float, 1>(a, s);
  return io_bf ? launch_prep_t<float, bf16, 1>(a, s) : launch_prep_t<float, float, 1>(a, s);
}

hipError_t launch_proj(const ProjArgs& a, bool bf, bool io_bf, hipStream_t s) {
  if (bf && a.parts == 2) return io_bf ? launch_proj_t<bf16, bf16, 2>(a, s) : launch_proj_t<bf16, float, 2>(a, s);
  if (bf) return io_bf ? launch_proj_t<bf16, bf16, 1>(a, s) : launch_proj_t<bf16, float, 1>(a, s);
  return io_bf ? launch_proj_t<float, bf16, 1>(a, s) : launch_proj_t<float, float, 1>(a, s);
}
hipError_t launch_out(const OutArgs& a, bool bf, bool io_bf, hipStream_t s) {
  if (bf && a.parts == 2) return io_bf ? launch_out_t<bf16, bf16, 2>(a, s) : launch_out_t<bf16, float, 2>(a, s);
  if (bf) return io_bf ? launch_out_t<bf16, bf16, 1>(a, s) : launch_out_t<bf16, float, 1>(a, s);
  return io_bf ? launch_out_t<float, bf16, 1>(a, s) : launch_out_t<float, float, 1>(a, s);
}

size_t proj_parts_bytes(int64_t rows, int d, bool bf, int parts) {
  return (size_t)(bf ? parts : 1) * (bf ? sizeof(bf16) : sizeof(float)) * rows * d;
}

namespace {
template <typename K> hipError_t raise_lds(K* k, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}
}  // namespace

// ---------------------------------------------------------------------------
// Backward of the aggregation ("TANGO: Token-Aggregated Nonlinear Gating
// Operators ...", §2.1 eqs. 4-5, §2.2 eqs. 6-10): the tiles of ds (and, for
// WANGO, dP) and the products by them.  With the forward's shifted weights
// w_ij = e^{tau (s_ij - 1)}, u_i = dgbar_i / den_i and delta_i = -u_i . gbar_i
// (bwd_kernels.hip) and dm_ij = u_i . g_j + delta_i,
//     ds_ij = tau w_ij dm_ij        (TANGO: j <= i; WANGO: the window i-W < j <= i),
//     dP_ij = e^{-tau} dm_ij        (WANGO: older pairs j <= i - W; dP = dL/d(p_i . a_j)),
//     dq_i = sum_j ds_ij k_j, dk_j = sum_i ds_ij q_i, dp_i = sum_j dP_ij a_j, da_j = sum_i dP_ij p_i,
//     dtheta += sum ds_ij s_ij.
//
// KD: one 128 x 128 tile (destination rows i of tile it, source rows j of
// tile jt) of one sequence and head per workgroup: TANGO every jt <= it,
// WANGO the nb "near" tiles jt = it - nb + 1 .. it that hold the window.
// S = Q_i K_j^T (k = d_h) and dW = U_i G_j^T (k = the head's gate columns)
// run one after the other on the main loop above, into two accumulator sets
// (WANGO's u and g rows carry delta and 1 in one extra column, so dW is dm).
// Each tile is stored in bf16 twice: transposed (rows j, for dk / da)
// straight from the accumulators, whose lanes hold 4 consecutive rows i of
// one column j, and by rows (for dq / dp) through LDS.  The workgroup also
// sums ds * s for dtheta.
//
// KM: one product for one 128-row tile r and one chunk of kBwdChunkTiles
// tiles along the sum: A = the rows of the tiles ((r, jt) by rows for dq / dp,
// (it, r) transposed for dk / da), B = the keys, queries or features
// transposed per head, k = the summed position.  Each chunk writes a float32
// partial, which the finish kernels add up.
//
// KW (WANGO older prefix, far tiles): per-tile sums a_j g^_j^T and p_i u^_i^T
// ([d_h] x [FhC]), their shifted prefix / suffix (bwd_kernels-side scan), and
// the read-outs dp_i += S_it u^_i, da_j += R_jt g^_j (e^{-tau} applied in the
// finish), all on the same main loop.
// ---------------------------------------------------------------------------
namespace {

using DsCfg = TileCfg<kBwdTile, kBwdTile, 32, 2, 2, 3, 1>;
// (d_h = 32 runs 64 B rows, the upper half zero: a load pass covers 64 rows)
template <int DH> using MmCfg = TileCfg<kBwdTile, (DH < 64 ? 64 : DH), 32, 2, 2, 3, 1>;
constexpr int kTileElems = kBwdTile * kBwdTile;
constexpr int kDsStride = kBwdTile + 8;   // bf16 per staged row (rows stay 16-byte aligned)
constexpr size_t kStageBytes = (size_t)kBwdTile * kDsStride * sizeof(bf16);
constexpr size_t kDsLds = ops_bytes<DsCfg, bf16>() > kStageBytes ? ops_bytes<DsCfg, bf16>() : kStageBytes;
constexpr float kLogTauMaxB = 2.995732273553991f;   // log 20: tau = exp(min(theta, log 20))

__host__ __device__ __forceinline__ int64_t tri_index(int i, int j) { return (int64_t)i * (i + 1) / 2 + j; }
// Index of tile (it, jt) among a (sequence, head)'s stored tiles.
template <bool W>
__device__ __forceinline__ int64_t tile_index(int it, int jt, int nb) {
  return W ? (int64_t)it * nb + (jt - it + nb - 1) : tri_index(it, jt);
}

// Stores a tile of values v(i, j) (this lane: rows r0 + 0..3 of column c, per
// accumulator block) transposed straight from the registers and by rows
// through LDS.
template <class CF, class Fn>
__device__ __forceinline__ void store_tile(bf16* dst_r, bf16* dst_t, bf16* st, Fn value) {
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave / CF::WN, wc = wave % CF::WN;
#pragma unroll
  for (int i = 0; i < CF::IB; ++i) {
    const int r0 = wr * CF::WTM + i * 16 + grp * 4;
#pragma unroll
    for (int j = 0; j < CF::JB; ++j) {
      const int c = wc * CF::WTN + j * 16 + col;
      bf16x4 q4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        q4[r] = (bf16)value(i, j, r, r0 + r, c);
        st[(r0 + r) * kDsStride + c] = q4[r];
      }
      *reinterpret_cast<bf16x4*>(dst_t + c * kBwdTile + r0) = q4;
    }
  }
  __syncthreads();
  for (int q = tid; q < kTileElems / 8; q += kThreads) {
    const int row = q >> 4, c8 = (q & 15) * 8;
    *reinterpret_cast<u32x4*>(dst_r + row * kBwdTile + c8) =
        *reinterpret_cast<const u32x4*>(st + row * kDsStride + c8);
  }
  __syncthreads();   // st is reused
}

template <bool W>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void ds_kernel(BwdArgs a, int64_t ntiles, int64_t items) {
  using CF = DsCfg;
  typedef bf16 T;
  constexpr int PA = tile_chunks<CF, T>(CF::BM) / 4, PB = tile_chunks<CF, T>(CF::BN) / 4;
  __shared__ __align__(16) unsigned char smem[kDsLds];
  __shared__ float red[kThreads / 64];
  T* lds = reinterpret_cast<T*>(smem);

  const int64_t q8 = gridDim.x / 8;
  const int64_t item = (int64_t)(blockIdx.x % 8) * q8 + blockIdx.x / 8;
  if (item >= items) return;
  const int64_t bh = item / ntiles;
  const int64_t t = item - bh * ntiles;
  int it, jt;
  if (W) {
    it = (int)(t / a.nb);
    jt = it - a.nb + 1 + (int)(t % a.nb);
    if (jt < 0) {         // before the first tile (workgroup-uniform)
      if (threadIdx.x == 0) a.part_theta[item] = 0.f;
      return;
    }
  } else {
    it = (int)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
    while (tri_index(it + 1, 0) <= t) ++it;
    while (tri_index(it, 0) > t) --it;
    jt = (int)(t - tri_index(it, 0));
  }
  const int h = (int)(bh % a.H);
  const int64_t mseq = (bh / a.H) * a.Tp;
  const int HD = a.H * a.dh, tid = threadIdx.x;
  const int64_t ri = mseq + (int64_t)it * kBwdTile, rj = mseq + (int64_t)jt * kBwdTile;

  f32x4 accS[CF::IB][CF::JB], accW[CF::IB][CF::JB];
#pragma unroll
  for (int i = 0; i < CF::IB; ++i)
#pragma unroll
    for (int j = 0; j < CF::JB; ++j) {
      accS[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      accW[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  PartsSource<T, PA, 1> sa;
  sa.part_stride = 0;
  RowSource<T, PB> sb;
  // S = Q_i K_j^T
#pragma unroll
  for (int p = 0; p < PA; ++p) {
    const PiecePos<CF, T> pp = piece_pos<CF, T>(tid, p);
    sa.ptr[p] = static_cast<const T*>(a.qh) + (ri + pp.row) * HD + h * a.dh + pp.kp * piece_elems<T>();
  }
#pragma unroll
  for (int p = 0; p < PB; ++p) {
    const PiecePos<CF, T> pp = piece_pos<CF, T>(tid, p);
    sb.ptr[p] = static_cast<const T*>(a.kh) + (rj + pp.row) * HD + h * a.dh + pp.kp * piece_elems<T>();
    sb.ok[p] = true;
  }
  gemm_mainloop<CF, T>(accS, lds, a.dh / CF::BK, sa, sb);   // ends with a barrier
  // dW = U_i G_j^T
#pragma unroll
  for (int p = 0; p < PA; ++p) {
    const PiecePos<CF, T> pp = piece_pos<CF, T>(tid, p);
    sa.ptr[p] = static_cast<const T*>(a.u_rm) + ((ri + pp.row) * a.H + h) * a.FhC + pp.kp * piece_elems<T>();
  }
#pragma unroll
  for (int p = 0; p < PB; ++p) {
    const PiecePos<CF, T> pp = piece_pos<CF, T>(tid, p);
    sb.ptr[p] = static_cast<const T*>(a.g_rm) + ((rj + pp.row) * a.H + h) * a.FhC + pp.kp * piece_elems<T>();
  }
  gemm_mainloop<CF, T>(accW, lds, a.FhC / CF::BK, sa, sb);

  // ds (and dP), their stores and dtheta
  const float tau = __expf(fminf(a.theta[h], kLogTauMaxB));
  const float ktau = tau * kLog2e;
  const float* delta = a.delta + (int64_t)h * a.B * a.Tp;
  const int lane = tid & 63, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave / CF::WN;
  float dl[CF::IB][4];   // TANGO: delta of this lane's rows (WANGO: already inside dW)
#pragma unroll
  for (int i = 0; i < CF::IB; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) dl[i][r] = W ? 0.f : delta[ri + wr * CF::WTM + i * 16 + grp * 4 + r];
  const int di = (it - jt) * kBwdTile;   // i - j = di + (row - col)
  float th = 0.f;
  auto ds_of = [&](int i, int j, int r, int row, int c) {
    const float sv = accS[i][j][r];
    const float w = __builtin_amdgcn_exp2f(ktau * (sv - 1.0f));
    const int ij = di + row - c;   // i - j
    const bool valid = W ? (ij >= 0 && ij < a.window) : ij >= 0;
    const float v = valid ? tau * w * (accW[i][j][r] + dl[i][r]) : 0.f;
    th += v * sv;
    return v;
  };
  const int64_t tix = bh * ntiles + (W ? tile_index<true>(it, jt, a.nb) : t);
  T* st = reinterpret_cast<T*>(smem);
  store_tile<CF>(static_cast<T*>(a.ds_rm) + tix * kTileElems, static_cast<T*>(a.ds_t) + tix * kTileElems, st,
                 ds_of);
  if (W) {
    const float escale = __expf(-tau);
    auto dp_of = [&](int i, int j, int r, int row, int c) {
      return di + row - c >= a.window ? escale * accW[i][j][r] : 0.f;
    };
    store_tile<CF>(static_cast<T*>(a.dp_rm) + tix * kTileElems, static_cast<T*>(a.dp_t) + tix * kTileElems, st,
                   dp_of);
  }
  th = wave_sum(th);
  if (lane == 0) red[wave] = th;
  __syncthreads();
  if (tid == 0) a.part_theta[bh * ntiles + t] = red[0] + red[1] + red[2] + red[3];
}

// A operand of KM: pieces of the rows of a run of tiles along k.
template <int DIR, bool W, int P> struct DsRowSource {
  struct raw {
    u32x4 v;
  };
  const bf16* tiles;   // the (sequence, head)'s first tile
  int off[P];          // row * 128 + piece column of each pass
  int r, kbase, nb;
  __device__ __forceinline__ void fetch(raw& x, int p, int k0) const {
    const int k = kbase + k0, kt = k >> 7;
    const int64_t tile = DIR == 0 ? tile_index<W>(r, kt, nb) : tile_index<W>(kt, r, nb);
    x.v = *reinterpret_cast<const u32x4*>(tiles + tile * kTileElems + off[p] + (k & (kBwdTile - 1)));
  }
  __device__ __forceinline__ Parts<1> convert(const raw& x, int) const {
    Parts<1> o;
    o.p[0] = x.v;
    return o;
  }
};

// Product `prod` (0 dq, 1 dk, 2 dp, 3 da) for row tile r, chunk c.
template <int PROD, bool W, int DH>
__device__ __forceinline__ void dsmm_job(const BwdArgs& a, int64_t ntiles, int nch, int64_t bh, int r, int c,
                                         bf16* lds) {
  using CF = MmCfg<DH>;
  typedef bf16 T;
  constexpr int DIR = PROD & 1;
  constexpr int PA = tile_chunks<CF, T>(CF::BM) / 4, PB = tile_chunks<CF, T>(CF::BN) / 4;
  const int nt = a.Tp / kBwdTile;
  // k tiles of this chunk.  TANGO: chunk c holds tiles 8c .. 8c + 7 of the
  // sum, DIR 0 those with jt <= r, DIR 1 those with it >= r.  WANGO: one chunk,
  // the near tiles of row tile r (nb <= 8 of them): DIR 0 jt = r - nb + 1 .. r,
  // DIR 1 it = r .. r + nb - 1, clipped to the sequence.
  int first, last;
  if (W) {
    first = DIR == 0 ? max(0, r - a.nb + 1) : r;
    last = DIR == 0 ? r : min(nt - 1, r + a.nb - 1);
  } else {
    first = c * kBwdChunkTiles;
    last = first + kBwdChunkTiles - 1;
    if (DIR == 0) {
      last = min(last, r);
    } else {
      first = max(first, r);
      last = min(last, nt - 1);
    }
  }
  if (first > last) return;   // workgroup-uniform
  const int tid = threadIdx.x;
  DsRowSource<DIR, W, PA> sa;
  const void* tiles = PROD == 0 ? a.ds_rm : PROD == 1 ? a.ds_t : PROD == 2 ? a.dp_rm : a.dp_t;
  sa.tiles = static_cast<const T*>(tiles) + bh * ntiles * kTileElems;
  sa.r = r;
  sa.kbase = first * kBwdTile;
  sa.nb = a.nb;
#pragma unroll
  for (int p = 0; p < PA; ++p) {
    const PiecePos<CF, T> pp = piece_pos<CF, T>(tid, p);
    sa.off[p] = pp.row * kBwdTile + pp.kp * piece_elems<T>();
  }
  RowSource<T, PB> sb;
  const void* bsrc = PROD == 0 ? a.kT : PROD == 1 ? a.qT : PROD == 2 ? a.aT : a.pT;
  const T* xT = static_cast<const T*>(bsrc) + bh * DH * (int64_t)a.Tp;
#pragma unroll
  for (int p = 0; p < PB; ++p) {
    const PiecePos<CF, T> pp = piece_pos<CF, T>(tid, p);
    sb.ptr[p] = xT + (int64_t)(pp.row % DH) * a.Tp + sa.kbase + pp.kp * piece_elems<T>();
    sb.ok[p] = pp.row < DH;
  }
  f32x4 acc[CF::IB][CF::JB];
#pragma unroll
  for (int i = 0; i < CF::IB; ++i)
#pragma unroll
    for (int j = 0; j < CF::JB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  gemm_mainloop<CF, T>(acc, lds, (last - first + 1) * (kBwdTile / CF::BK), sa, sb);

  const int64_t M = (int64_t)a.B * a.Tp;
  const int HD = a.H * DH, h = (int)(bh % a.H);
  const int64_t row0 = (bh / a.H) * a.Tp + (int64_t)r * kBwdTile;
  float* out = a.part + ((int64_t)PROD * nch + c) * M * HD + row0 * HD + h * DH;
  const int lane = tid & 63, col = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave / CF::WN, wc = wave % CF::WN;
#pragma unroll
  for (int i = 0; i < CF::IB; ++i)
#pragma unroll
    for (int j = 0; j < CF::JB; ++j) {
      const int e = wc * CF::WTN + j * 16 + col;
      if (e < DH)
#pragma unroll
        for (int q = 0; q < 4; ++q) out[(int64_t)(wr * CF::WTM + i * 16 + grp * 4 + q) * HD + e] = acc[i][j][q];
    }
}

template <bool W, int DH>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void dsmm_kernel(BwdArgs a, int64_t ntiles, int nch, int64_t items) {
  __shared__ __align__(16) unsigned char smem[ops_bytes<MmCfg<DH>, bf16>()];
  const int64_t q8 = gridDim.x / 8;
  const int64_t item = (int64_t)(blockIdx.x % 8) * q8 + blockIdx.x / 8;
  if (item >= items) return;
  const int nt = a.Tp / kBwdTile;
  const int64_t per_prod = (int64_t)a.B * a.H * nt * nch;
  const int prod = (int)(item / per_prod);
  int64_t rem = item - prod * per_prod;
  const int c = (int)(rem % nch);
  rem /= nch;
  const int r = (int)(rem % nt);
  const int64_t bh = rem / nt;
  bf16* lds = reinterpret_cast<bf16*>(smem);
  switch (prod) {
    case 0: dsmm_job<0, W, DH>(a, ntiles, nch, bh, r, c, lds); break;
    case 1: dsmm_job<1, W, DH>(a, ntiles, nch, bh, r, c, lds); break;
    case 2: if (W) dsmm_job<2, W, DH>(a, ntiles, nch, bh, r, c, lds); break;
    default: if (W) dsmm_job<3, W, DH>(a, ntiles, nch, bh, r, c, lds); break;
  }
}

// KW read-out: for tile t of (sequence, head) bh, out[row][e] = sum_f rows[row][f] state_t[e][f]
// (S: rows = augmented u of destination tile t; R: augmented g of source tile t).
template <int DH>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void state_readout_kernel(WStateArgs w) {
  using CF = MmCfg<DH>;
  typedef bf16 T;
  constexpr int PA = tile_chunks<CF, T>(CF::BM) / 4, PB = tile_chunks<CF, T>(CF::BN) / 4;
  __shared__ __align__(16) unsigned char smem[ops_bytes<CF, T>()];
  const int64_t id = blockIdx.x;
  const int t = (int)(id % w.nt);
  const int64_t bh = id / w.nt;
  const int h = (int)(bh % w.H);
  const int64_t row0 = (bh / w.H) * w.Tp + (int64_t)t * kBwdTile;
  const int tid = threadIdx.x;
  PartsSource<T, PA, 1> sa;
  sa.part_stride = 0;
#pragma unroll
  for (int p = 0; p < PA; ++p) {
    const PiecePos<CF, T> pp = piece_pos<CF, T>(tid, p);
    sa.ptr[p] = static_cast<const T*>(w.rows) + ((row0 + pp.row) * w.H + h) * w.FhC + pp.kp * piece_elems<T>();
  }
  const T* st = static_cast<const T*>(w.state) + ((bh * w.nt + t) * DH) * (int64_t)w.FhC;
  RowSource<T, PB> sb;
#pragma unroll
  for (int p = 0; p < PB; ++p) {
    const PiecePos<CF, T> pp = piece_pos<CF, T>(tid, p);
    sb.ptr[p] = st + (int64_t)(pp.row % DH) * w.FhC + pp.kp * piece_elems<T>();
    sb.ok[p] = pp.row < DH;
  }
  f32x4 acc[CF::IB][CF::JB];
#pragma unroll
  for (int i = 0; i < CF::IB; ++i)
#pragma unroll
    for (int j = 0; j < CF::JB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  gemm_mainloop<CF, T>(acc, reinterpret_cast<T*>(smem), w.FhC / CF::BK, sa, sb);
  const int HD = w.H * DH;
  float* out = w.out + row0 * HD + h * DH;
  const int lane = tid & 63, col = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave / CF::WN, wc = wave % CF::WN;
#pragma unroll
  for (int i = 0; i < CF::IB; ++i)
#pragma unroll
    for (int j = 0; j < CF::JB; ++j) {
      const int e = wc * CF::WTN + j * 16 + col;
      if (e < DH)
#pragma unroll
        for (int q = 0; q < 4; ++q) out[(int64_t)(wr * CF::WTM + i * 16 + grp * 4 + q) * HD + e] = acc[i][j][q];
    }
}

}  // namespace

hipError_t launch_tango_ds(const BwdArgs& a, const BwdPlan& p, hipStream_t s) {
  if (a.dh % 32 != 0 || a.FhC % 32 != 0 || a.Tp % kBwdTile != 0) return hipErrorInvalidValue;
  const int64_t q8 = ceil_div(p.items_ds, 8);
  if (a.window > 0)
    hipLaunchKernelGGL(ds_kernel<true>, dim3((unsigned)(8 * q8)), dim3(kThreads), 0, s, a, p.ntri, p.items_ds);
  else
    hipLaunchKernelGGL(ds_kernel<false>, dim3((unsigned)(8 * q8)), dim3(kThreads), 0, s, a, p.ntri, p.items_ds);
  return hipGetLastError();
}

template <bool W>
static hipError_t launch_dsmm_w(const BwdArgs& a, const BwdPlan& p, hipStream_t s) {
  const int64_t q8 = ceil_div(p.items_mm, 8);
  dim3 grid((unsigned)(8 * q8)), block(kThreads);
  switch (a.dh) {
    case 32: hipLaunchKernelGGL((dsmm_kernel<W, 32>), grid, block, 0, s, a, p.ntri, p.nch, p.items_mm); break;
    case 64: hipLaunchKernelGGL((dsmm_kernel<W, 64>), grid, block, 0, s, a, p.ntri, p.nch, p.items_mm); break;
    case 128: hipLaunchKernelGGL((dsmm_kernel<W, 128>), grid, block, 0, s, a, p.ntri, p.nch, p.items_mm); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_tango_dsmm(const BwdArgs& a, const BwdPlan& p, hipStream_t s) {
  return a.window > 0 ? launch_dsmm_w<true>(a, p, s) : launch_dsmm_w<false>(a, p, s);
}

hipError_t launch_wango_state_readout(const WStateArgs& w, hipStream_t s) {
  if (w.FhC % 32 != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((int64_t)w.B * w.H * w.nt)), block(kThreads);
  switch (w.dh) {
    case 32: hipLaunchKernelGGL(state_readout_kernel<32>, grid, block, 0, s, w); break;
    case 64: hipLaunchKernelGGL(state_readout_kernel<64>, grid, block, 0, s, w); break;
    case 128: hipLaunchKernelGGL(state_readout_kernel<128>, grid, block, 0, s, w); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t gemm_kernels_init() {
  hipError_t e;
#define TANGO_RAISE(K, BYTES) \
  if ((e = raise_lds(&K, BYTES)) != hipSuccess) return e;
  TANGO_RAISE((proj_kernel<bf16, bf16, 2>), (main_bytes<ProjCfg<bf16, 2>, bf16>()))
  TANGO_RAISE((proj_kernel<bf16, bf16, 1>), (main_bytes<ProjCfg<bf16, 1>, bf16>()))
  TANGO_RAISE((proj_kernel<bf16, float, 2>), (main_bytes<ProjCfg<bf16, 2>, bf16>()))
  TANGO_RAISE((proj_kernel<bf16, float, 1>), (main_bytes<ProjCfg<bf16, 1>, bf16>()))
  TANGO_RAISE((proj_kernel<float, bf16, 1>), (main_bytes<ProjCfg<float, 1>, float>()))
  TANGO_RAISE((proj_kernel<float, float, 1>), (main_bytes<ProjCfg<float, 1>, float>()))
  TANGO_RAISE((out_kernel<bf16, bf16, OutCfg<bf16, 2>>), (main_bytes<OutCfg<bf16, 2>, bf16>()))
  TANGO_RAISE((out_kernel<bf16, bf16, OutCfgNarrow<2>>), (main_bytes<OutCfgNarrow<2>, bf16>()))
  TANGO_RAISE((out_kernel<bf16, float, OutCfg<bf16, 2>>), (main_bytes<OutCfg<bf16, 2>, bf16>()))
  TANGO_RAISE((out_kernel<bf16, float, OutCfgNarrow<2>>), (main_bytes<OutCfgNarrow<2>, bf16>()))
  TANGO_RAISE((out_kernel<bf16, bf16, OutCfg<bf16, 1>>), (main_bytes<OutCfg<bf16, 1>, bf16>()))
  TANGO_RAISE((out_kernel<bf16, bf16, OutCfgNarrow<1>>), (main_bytes<OutCfgNarrow<1>, bf16>()))
  TANGO_RAISE((out_kernel<bf16, float, OutCfg<bf16, 1>>), (main_bytes<OutCfg<bf16, 1>, bf16>()))
  TANGO_RAISE((out_kernel<bf16, float, OutCfgNarrow<1>>), (main_bytes<OutCfgNarrow<1>, bf16>()))
  TANGO_RAISE((out_kernel<float, bf16, OutCfg<float, 1>>), (main_bytes<OutCfg<float, 1>, float>()))
  TANGO_RAISE((out_kernel<float, float, OutCfg<float, 1>>), (main_bytes<OutCfg<float, 1>, float>()))
#undef TANGO_RAISE
  return hipSuccess;
}

}  // namespace tango
