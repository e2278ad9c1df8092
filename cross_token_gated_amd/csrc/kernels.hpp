// kernels.hpp - argument blocks and launchers of the gfx950 kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tango {

// Rows of every intermediate buffer are padded per sequence to a multiple of
// this many positions; padded rows hold zeros.
constexpr int kRowPad = 128;

struct ProjArgs {
  const void* x;       // [B, T, d] in the I/O dtype
  const void* w_g;     // [F, d]
  const void* w_v;     // [F, d]
  const void* w_q;     // [HD, d]
  const void* w_k;     // [HD, d]
  const void* gain;    // [d] or null
  void* gp;            // packed gates [B*Tp/32][4][F][8]
  void* v;             // [B*Tp, F]: bf16 with one bf16 operand part, else float32
  void* qh;            // [B*Tp, HD]
  void* kh;            // [B*Tp, HD]
  void* fq;            // WANGO only (else null): phi(sqrt(tau) q) [B*Tp, HD], permuted feature order
  void* fk;            // WANGO only (else null): phi(sqrt(tau) k), source-packed [B*Tp/32][4][HD][8]
  const float* theta;  // [H], for the WANGO features
  void* xs;            // scratch: [parts][B*Tp, d] parts of h * gain (padded rows zero)
  float* rinv;         // scratch: [B*Tp] RMSNorm row scales
  int* zero;           // optional: zero_n ints the row-prep kernel clears (the
  int64_t zero_n;      //   aggregation's split counters), else null / 0
  int B, T, Tp, d, F, HD, dh;
  int Fh, Fhp, Fp;     // gate columns per head, padded to a multiple of 64, and H * Fhp:
                       // gp holds head a's column c at a * Fhp + c (v is not padded)
  float rope_base, eps;
  int parts;           // operand parts of h * gain in bf16 (1 or 2; float32: 1)
};

// Bytes of the operand parts xs for `rows` padded rows of width d (parts
// counts for bf16 only).
size_t proj_parts_bytes(int64_t rows, int d, bool bf, int parts);

struct OutArgs {
  const void* x;       // [B, T, d] in the I/O dtype
  const void* w_o;     // [d, F]
  const void* gbar;    // [B*Tp, F]
  const void* v;       // [B*Tp, F]: bf16 with one bf16 operand part, else float32
  void* out;           // [B, T, d] in the I/O dtype
  int B, T, Tp, d, F;
  int parts;           // operand parts of gbar * v in bf16 (1 or 2; float32: 1)
};

// Aggregation (TANGO full prefix, or the WANGO window band + combine).
struct AggArgs {
  const void* qh;          // [B*Tp, H*dh]
  const void* kh;          // [B*Tp, H*dh]
  const void* gp;          // packed gates
  void* gbar;              // [B*Tp, F]
  const float* theta;      // [H]
  const float* null_bias;  // [H] or null
  const float* n_old;      // WANGO: blocked [B*Tp/16][F/16][64][4]
  const float* z_old;      // WANGO: [B*Tp, H]
  // WANGO with the read-out in the band (instead of n_old, z_old): the chunk
  // states and the query features they are read out with (see ScanArgs)
  const void* states;
  const void* zstates;
  const void* fq;          // phi(sqrt(tau) q), permuted feature order [B*Tp, HD]
  float* part;             // TANGO split mode: partial numerators
  float* part_den;         // TANGO split mode: partial denominators
  int* counters;           // TANGO split mode: one per split tile
  int B, T, Tp, F, H, dh, window;   // F: gate columns of gp and n_old (head-padded)
  int Fo, Fho;             // gbar: [B*Tp, Fo] with Fho columns per head (not padded)
  int chunk;               // WANGO: n_old holds the state read-out at chunk boundaries
  int split;               // 1: split the long tiles in two (last finisher combines)
  // options (all off when zero / null):
  float* den_out;          // [B*Tp, H]: the ratio's denominator, e^{-tau} units (rows < T)
  int num_only;            // 1: write the numerator alone (no row sums, no null, no division)
  int rev_out;             // 1: row i of a sequence is stored at row T - 1 - i (rows < T only)
};

// WANGO older-prefix scan.
struct ScanArgs {
  const void* fq;          // phi(sqrt(tau) q), permuted feature order [B*Tp, HD]
  const void* fk;          // phi(sqrt(tau) k), source-packed [B*Tp/32][4][HD][8]
  const void* gp;
  float* n_old;            // blocked [B*Tp/16][F/16][64][4]
  float* z_old;            // [B*Tp, H]
  // Instead of n_old, z_old (when non-null): the state of every destination
  // chunk d >= window / chunk in the A-operand layout of the read-out, bf16
  // (or float32) fragments [B][H][Tp/chunk][Fh/16][dh/32][64 lanes], and the
  // z state likewise [B][H][Tp/chunk][dh/32][64 lanes]
  void* states;
  void* zstates;
  float* seg_state;        // segment sums: [B][H][column slice][nseg] blocks of dh x slice, accumulator order
  float* seg_z;            // [B][H][nseg][dh]
  int B, T, Tp, F, H, dh, window, chunk;
  int nseg, chunks_per_seg;
  int slice;               // gate columns per workgroup (64 or 128)
};

// Plan of the TANGO aggregation grid for a shape.
struct AggPlan {
  int fs;          // gate columns per workgroup
  int br;          // destination rows per tile
  int nfc;         // column chunks per head
  int rtiles;      // 64-row tiles per sequence
  int split;       // 1 = split mode
  int64_t items;   // work items
  int64_t n_split_tiles;
};

AggPlan tango_agg_plan(int B, int Tp, int F, int H, int dh, bool bf);

struct ScanPlan {
  int nseg, chunks_per_seg, fs;
};
ScanPlan wango_scan_plan(int B, int Tp, int F, int H, int chunk);

// bf: bf16 weights/activations (else float32); io_bf: bf16 x/out (else float32)
hipError_t launch_proj(const ProjArgs& a, bool bf, bool io_bf, hipStream_t s);
hipError_t launch_out(const OutArgs& a, bool bf, bool io_bf, hipStream_t s);
// counters_clear: the split counters were already cleared earlier on the
// stream (by the row-prep kernel of the same block); else a fill kernel runs.
hipError_t launch_tango_agg(const AggArgs& a, const AggPlan& p, bool bf, bool counters_clear,
                            hipStream_t s);
hipError_t launch_wango_band(const AggArgs& a, bool bf, hipStream_t s);
hipError_t launch_wango_scan(const ScanArgs& a, const ScanPlan& p, bool bf, hipStream_t s);
hipError_t launch_zero_i32(int* p, int64_t n, hipStream_t s);

// Raise the dynamic-LDS limit of the kernels that need more than 64 KB
// (once per device).
hipError_t gemm_kernels_init();

// Zero the pad columns (Fh .. Fhp-1 of every head) of the packed gates, [M
// rows][H * Fhp], before the projection fills the rest.
hipError_t launch_zero_pad(void* gp, int64_t M, int H, int Fh, int Fhp, bool bf, hipStream_t s);

// Row-prep kernel alone (RMSNorm scales and operand parts of h * gain).
hipError_t launch_prep(const ProjArgs& a, bool bf, bool io_bf, hipStream_t s);

// ---- backward of the TANGO aggregation -------------------------------------

struct BwdArgs {
  // inputs (bf16 unless noted)
  const void* qh;          // [B*Tp, H*dh] unit queries (forward)
  const void* kh;          // [B*Tp, H*dh] unit keys
  const void* gp;          // packed gates [B*Tp/32][4][Fp][8] (forward, head-padded)
  const void* gbar;        // [B*Tp, F] forward output
  const void* dgbar;       // [B*Tp, F] incoming gradient
  const float* den;        // [B*Tp, H] forward denominators (e^{-tau} units), float32
  const float* theta;      // [H]
  const float* null_bias;  // [H] or null
  // scratch
  void* u_rm;              // [B*Tp][H][FhC] u = dgbar / den, row-major
  void* g_rm;              // [B*Tp][H][FhC] gates, row-major
  void* qT;                // [B][H][dh][Tp] queries, transposed per head
  void* kT;                // [B][H][dh][Tp] keys, transposed per head
  void* q_rev;             // [B*Tp, H*dh] queries, every sequence reversed
  void* k_rev;             // keys, reversed
  void* u_rev_pk;          // packed reversed u, [B*Tp/32][4][Fp][8]
  float* delta;            // [H][B*Tp] float32
  void* ds_rm;             // [B*H][ntiles][128][128] ds tiles, rows i (destinations)
  void* ds_t;              // [B*H][ntiles][128][128] ds tiles transposed, rows j (sources)
  float* part;             // TANGO: [2][nch][B*Tp][H*dh] float32 chunk partials of dq (0) and dk (1);
                           // WANGO: [6][B*Tp][H*dh]: dq, dk (window), dp, da (near older pairs),
                           // dp, da (far older pairs, from the prefix states)
  float* part_theta;       // [B*H*ntiles] float32: sum of ds * s per tile
  // WANGO only (window > 0)
  int window;              // W
  int nb;                  // near tiles per row tile: source tiles it - nb + 1 .. it
  void* dp_rm;             // [B*H][ntiles][128][128] dP tiles (older pairs), rows i
  void* dp_t;              // transposed, rows j
  void* pT;                // [B][H][dh][Tp] phi(sqrt(tau) q), transposed per head
  void* aT;                // [B][H][dh][Tp] phi(sqrt(tau) k)
  void* p_rm;              // [B*Tp][H*dh] phi(sqrt(tau) q), row-major
  void* a_rm;              // phi(sqrt(tau) k)
  // outputs
  float* dq;               // [B*Tp, H*dh] float32 (zero on rows past the end)
  float* dk;               // [B*Tp, H*dh]
  float* dtheta;           // [H]
  float* dnull;            // [H] or null
  int* zero_ints;          // TANGO: the dg aggregation's split counters, cleared by the row prep; or null
  int64_t n_zero_ints;
  int B, T, Tp, H, dh;
  int F, Fh;               // gate columns (unpadded) in all and per head
  int Fhp, Fp;             // head-padded width of the packed gates, H * Fhp
  int FhC;                 // head width of u_rm / g_rm: TANGO Fhp; WANGO Fhp + 64, with delta (u)
                           // and 1 (g) in column Fhp, so that u . g over it is u . g + delta
};

constexpr int kBwdTile = 128;        // rows of a ds tile
constexpr int kBwdChunkTiles = 8;    // ds tiles per chunk of the dq / dk sums

struct BwdPlan {
  int FhC;
  int nt;              // 128-row tiles per sequence
  int64_t ntri;        // ds tiles per (sequence, head): TANGO nt (nt + 1) / 2, WANGO nt * nb
  int nch;             // chunks of kBwdChunkTiles tiles along a sum (WANGO: 1)
  int nb;              // WANGO: near tiles per row tile (0 for TANGO)
  int nprod;           // products of the tiles: 2 (dq, dk), WANGO 4 (and dp, da)
  int64_t items_ds;    // B * H * ntri
  int64_t items_mm;    // nprod * B * H * nt * nch (some empty)
};
BwdPlan tango_bwd_plan(int B, int Tp, int Fhp, int H);
BwdPlan wango_bwd_plan(int B, int Tp, int Fhp, int H, int window);
hipError_t launch_tango_bwd_prep(const BwdArgs& a, const BwdPlan& p, hipStream_t s, bool qk = true);
// ds tiles and their products (gemm_kernels.hip)
hipError_t launch_tango_ds(const BwdArgs& a, const BwdPlan& p, hipStream_t s);
hipError_t launch_tango_dsmm(const BwdArgs& a, const BwdPlan& p, hipStream_t s);
hipError_t launch_tango_bwd_finish(const BwdArgs& a, const BwdPlan& p, hipStream_t s);

// WANGO: the older-prefix states and their read-outs (gemm_kernels.hip), the
// feature layouts and the finish (bwd_kernels.hip)
struct WStateArgs {
  const void* aT;      // [B*H][dh][Tp] source features (S) / destination features (R)
  const void* xrm;     // [B*Tp][H][FhC] augmented g (S) / u (R), row-major
  float* tsum;         // [B*H][nt][dh][FhC] per-tile sums
  void* state;         // [B*H][nt][dh][FhC] bf16: S exclusive prefix / R suffix from tile t + nb
  const void* rows;    // [B*Tp][H][FhC] augmented u (S read-out) / g (R read-out)
  float* out;          // [B*Tp][H*dh] read-out partial
  int B, H, dh, Tp, FhC, nt, nb;
};
hipError_t launch_wango_state_sums(const WStateArgs& w, hipStream_t s);
hipError_t launch_wango_state_readout(const WStateArgs& w, hipStream_t s);
hipError_t launch_wango_state_scan(const WStateArgs& w, bool reverse, hipStream_t s);
hipError_t launch_wango_bwd_features(const BwdArgs& a, void* fq_perm, void* tmp_rm, const void* q_src,
                                     const void* k_src, void* fk_pk, hipStream_t s);
// theta_blk: [ceil(B*Tp*H*dh / 256)][H] float32 scratch
hipError_t launch_wango_bwd_finish(const BwdArgs& a, const BwdPlan& p, float* theta_blk, hipStream_t s);
// fq_perm, fk_pk: the reversed scan's destination (permuted) and source (packed)
// features, written here so that the scan does not redo them
hipError_t launch_wango_bwd_prep(const BwdArgs& a, const BwdPlan& p, void* fq_perm, void* fk_pk, hipStream_t s);
// Name of the kernel the backward prep launched last on this thread.
const char* bwd_last_step();

// ---- autoregressive decode -------------------------------------------------

constexpr int kDecChunk = 128;        // TANGO cache positions per workgroup
constexpr int kOutSplit = 4;          // K quarters of the decode output GEMM
constexpr int kDecMaxWindow = 2048;   // largest WANGO window of the decode kernels

struct DecArgs {
  int B;                   // sequences (one new token each)
  int Mp;                  // B rounded up to kRowPad (rows of the scratch operands)
  int d, F, H, dh, HD;
  int P;                   // state rows per sequence: TANGO capacity, WANGO window + 1
  int window;              // WANGO window W; 0 = TANGO
  int nch;                 // TANGO: chunks of kDecChunk positions per sequence
  float rope_base;
  const int* pos;          // [B] position of each new token (device)
  const void *w_g, *w_v, *w_q, *w_k, *w_o;
  const float* theta;
  const float* null_bias;  // or null
  void* kc;                // state: RoPE-rotated keys [B][P][HD] (normalised on read)
  void* gc;                // state: gates [B][P][F]
  float* S;                // WANGO state: [B][H][dh][F/H]
  float* z;                // WANGO state: [B][2][H][dh], the copy after position p in slot p % 2
  const void* xs;          // scratch: operand parts of h * gain [AS][Mp][d]
  const float* rinv;       // scratch: RMSNorm scales [Mp]
  void* v;                 // scratch: [Mp][F]
  void* q;                 // scratch: RoPE-rotated queries [Mp][HD] (normalised on read)
  float* part;             // scratch (TANGO): [B][nch][F + 64] partial sums
  void* gv;                // scratch: operand parts of gbar * v [AS][Mp][F]
  float* opart;            // scratch: output partials [kOutSplit][Mp][d]
  int* ocount;             // scratch: one counter per output tile, zero at entry
  const void* x;           // [B][d] in the I/O dtype
  void* out;               // [B][d] in the I/O dtype (may equal x)
};

// Operand parts of the decode GEMMs for the compute dtype (2 for bf16).
int decode_parts(bool bf);
hipError_t launch_decode(const DecArgs& a, bool bf, bool io_bf, hipStream_t s);

}  // namespace tango
