// bwd_kernels.hip - backward pass of the TANGO aggregation on gfx950.
//
// Differentiates the TANGO ratio ("TANGO: Token-Aggregated Nonlinear Gating
// Operators ...", §2.1 eqs. 4-5, §2.2 eq. 6) with respect to the unit query
// and key vectors, the gates, the temperature parameter and the null bias.
// With the forward's fixed shift (weights w_ij = e^{tau (s_ij - 1)}, the
// denominator den_i in the same e^{-tau} units, saved by the forward) and the
// incoming gradient dgbar:
//     u_i     = dgbar_i / den_i,          delta_i = -u_i . gbar_i
//     dg_j    = sum_{i>=j} w_ij u_i
//     ds_ij   = tau w_ij (u_i . g_j + delta_i)            (j <= i)
//     dq_i    = sum_j ds_ij k_j,          dk_j = sum_i ds_ij q_i
//     dtheta  = sum_ij ds_ij s_ij  (theta < log 20),  dnull = sum_i delta_i n_i e^{b - tau}
// (the common factor e^{tau} of the shifted weights cancels in every term).
//
// Kernels here (the ds tiles and the products by them are GEMM-shaped and live
// with the other GEMMs in gemm_kernels.hip):
//   * row prep: u (row-major, head width padded to the gates' Fhp) and delta;
//   * layout kernels: row-major <-> the packed [M/32][4][C][8] layout, with an
//     optional reversal of every sequence; per-head transposes of q and k;
//   * dg: the forward aggregation kernel on the time-reversed problem
//     (queries = reversed keys, keys = reversed queries, gates = reversed u),
//     numerator only, rows stored back in forward order;
//   * finish: the chunk partials of dq and dk added up, dtheta and dnull.
#include "common.hpp"
#include "kernels.hpp"

namespace tango {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLogTauMax = 2.995732273553991f;   // log 20: tau = exp(min(theta, log 20))

constexpr int kMaxBwdHeads = 256;  // one finish thread per head sums its shares

thread_local const char* t_step = "";   // kernel of the last launch (named in error messages)

// Row of position r (0..31) of a 32-row block in slot (grp, s) order.
__device__ __forceinline__ void slot_of_row(int r, int& grp, int& s) {
  if (r < 16) {
    grp = r >> 2;
    s = r & 3;
  } else {
    grp = (r - 16) >> 2;
    s = 4 + ((r - 16) & 3);
  }
}

// ---------------------------------------------------------------------------
// Row prep: u = dgbar / den and delta = -u . gbar per (row, head); u row-major
// [M][H][FhC] (zero past the head width and on rows past the sequence end),
// delta head-major [H][M].
template <typename T>
__global__ __launch_bounds__(256) void bwd_rows_kernel(BwdArgs a) {
  if (a.zero_ints) {   // counters of a later kernel (no separate clearing launch)
    const int64_t nthr = (int64_t)gridDim.x * gridDim.y * 256;
    for (int64_t z = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * 256 + threadIdx.x; z < a.n_zero_ints; z += nthr)
      a.zero_ints[z] = 0;
  }
  const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int h = blockIdx.y, lane = threadIdx.x & 63;
  if (m >= (int64_t)a.B * a.Tp) return;
  const int i = (int)(m % a.Tp);
  const bool live = i < a.T;
  const T* dg = static_cast<const T*>(a.dgbar) + m * a.F + (int64_t)h * a.Fh;
  const T* gb = static_cast<const T*>(a.gbar) + m * a.F + (int64_t)h * a.Fh;
  T* u = static_cast<T*>(a.u_rm) + (m * a.H + h) * a.FhC;
  const float rden = live ? 1.0f / a.den[m * a.H + h] : 0.f;
  float dot = 0.f;
  // 4 columns per lane (8-byte accesses; Fh and FhC are multiples of 4)
  for (int c = lane * 4; c < a.FhC; c += 256) {
    float uv[4] = {0.f, 0.f, 0.f, 0.f};
    if (live && c < a.Fh) {
      const Quad<T> d4 = load_quad<T>(dg + c), g4 = load_quad<T>(gb + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uv[e] = (float)d4[e] * rden;
        dot += uv[e] * (float)g4[e];
      }
    }
    store_quad<T>(u + c, cvt_quad<T>(f32x4{uv[0], uv[1], uv[2], uv[3]}));
  }
  dot = wave_sum(dot);
  if (lane == 0) {
    a.delta[(int64_t)h * a.B * a.Tp + m] = live ? -dot : 0.f;
    if (a.window > 0) u[a.Fhp] = (T)(live ? -dot : 0.f);   // WANGO: delta in the extra column
  }
}

// Row-major [rows][ld] -> packed [rows/32][4][ncols][8].  Packed column n is
// head n / dst_hw, column c = n % dst_hw of it, taken from source column
// (n / dst_hw) * src_hw + c when c < valid_w, else zero.  rev: packed row
// b*Tp + i holds source row b*Tp + T-1-i (rows i >= T are zero).  Through LDS
// in tiles of 32 rows x 32 packed columns (16-byte accesses on both sides):
// grid nblk * (ncols / 32) workgroups of 128.  ncols and dst_hw are multiples
// of 32, valid_w of 4, and src_hw >= dst_hw.
template <typename T>
__global__ __launch_bounds__(128) void pack_kernel(const T* __restrict__ src, int64_t ld, T* __restrict__ dst,
                                                   int ncols, int dst_hw, int src_hw, int valid_w, int Tp, int T_,
                                                   int rev) {
  __shared__ T tile[32][32 + 8];
  const int nct = ncols / 32;
  const int64_t blk = blockIdx.x / nct;
  const int n0 = (int)(blockIdx.x % nct) * 32;
  const int tid = threadIdx.x;
  {   // 32 rows x 4 pieces of 8 columns
    const int r = tid >> 2, p = tid & 3;
    const int64_t row = blk * 32 + r, b = row / Tp;
    const int i = (int)(row % Tp);
    const int n = n0 + p * 8, hd = n / dst_hw, c = n % dst_hw;
    u32x4 v = {0u, 0u, 0u, 0u};
    const bool live = !rev || i < T_;
    if (live && c < valid_w) {
      const int64_t srow = rev ? b * Tp + (T_ - 1 - i) : row;
      v = *reinterpret_cast<const u32x4*>(src + srow * ld + (int64_t)hd * src_hw + c);
      T* e8 = reinterpret_cast<T*>(&v);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c + e >= valid_w) e8[e] = (T)0.f;
    }
    *reinterpret_cast<u32x4*>(&tile[r][p * 8]) = v;
  }
  __syncthreads();
  {   // 4 slot groups x 32 columns, 8 rows each
    const int grp = tid >> 5, cl = tid & 31;
    T out[8];
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) out[s8] = tile[perm_slot(grp, s8)][cl];
    *reinterpret_cast<u32x4*>(dst + ((blk * 4 + grp) * (int64_t)ncols + n0 + cl) * 8) =
        *reinterpret_cast<const u32x4*>(out);
  }
}

// Packed gates [rows/32][4][H*src_hw][8] -> row-major [rows][H][dst_hw]
// (columns past valid_w zero; one_col >= 0: that column holds 1 on rows before
// the sequence end, the extra column of WANGO's augmented gates).  Through LDS
// in tiles of 32 rows x 64 columns: grid (rows / 32) * H * (dst_hw / 64).
template <typename T>
__global__ __launch_bounds__(256) void unpack_kernel(const T* __restrict__ gp, int src_F, T* __restrict__ dst,
                                                     int H, int src_hw, int dst_hw, int valid_w, int one_col, int Tp,
                                                     int T_) {
  __shared__ T tile[32][64 + 8];
  int64_t id = blockIdx.x;
  const int ct = (int)(id % (dst_hw / 64));
  id /= dst_hw / 64;
  const int hd = (int)(id % H);
  const int64_t blk = id / H;
  const int tid = threadIdx.x;
  {   // 4 slot groups x 64 columns, 8 rows (slots) each
    const int grp = tid >> 6, cl = tid & 63, c = ct * 64 + cl;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (c < valid_w) v = *reinterpret_cast<const u32x4*>(gp + packed_offset(blk, grp, (int64_t)hd * src_hw + c, src_F));
    const T* e8 = reinterpret_cast<const T*>(&v);
#pragma unroll
    for (int s = 0; s < 8; ++s) tile[perm_slot(grp, s)][cl] = e8[s];
  }
  __syncthreads();
  {   // 32 rows x 8 pieces of 8 columns
    const int r = tid >> 3, p = tid & 7;
    const int64_t row = blk * 32 + r;
    T out[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = ct * 64 + p * 8 + e;
      out[e] = (c == one_col && (int)(row % Tp) < T_) ? (T)1.0f : tile[r][p * 8 + e];
    }
    *reinterpret_cast<u32x4*>(dst + (row * H + hd) * (int64_t)dst_hw + ct * 64 + p * 8) =
        *reinterpret_cast<const u32x4*>(out);
  }
}


// Row-major copy with every sequence reversed (rows past the end zero).
template <typename T>
__global__ __launch_bounds__(256) void reverse_rows_kernel(const T* __restrict__ src, T* __restrict__ dst, int cols,
                                                           int Tp, int T_, int64_t rows) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= rows * cols) return;
  const int64_t row = id / cols;
  const int c = (int)(id % cols);
  const int64_t b = row / Tp;
  const int i = (int)(row % Tp);
  dst[id] = i < T_ ? src[(b * Tp + (T_ - 1 - i)) * cols + c] : (T)0.f;
}

// Row-major [B*Tp][H*C] -> per head transposed [B][H][C][Tp], through LDS in
// tiles of 64 positions x 32 columns (16-byte loads and stores on both sides).
// Grid: B * H * (C / 32) * (Tp / 64) workgroups of 256.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, T* __restrict__ dst, int H,
                                                        int C, int Tp) {
  __shared__ T tile[64][32 + 8];
  int64_t id = blockIdx.x;
  const int it = (int)(id % (Tp / 64));
  id /= Tp / 64;
  const int ct = (int)(id % (C / 32));
  id /= C / 32;
  const int h = (int)(id % H);
  const int64_t b = id / H;
  const int tid = threadIdx.x;
  {   // 64 rows x 4 pieces of 8 columns
    const int r = tid >> 2, p = tid & 3;
    const u32x4 v = *reinterpret_cast<const u32x4*>(
        src + (b * Tp + (int64_t)it * 64 + r) * (int64_t)H * C + (int64_t)h * C + ct * 32 + p * 8);
    *reinterpret_cast<u32x4*>(&tile[r][p * 8]) = v;
  }
  __syncthreads();
  {   // 32 columns x 8 pieces of 8 positions
    const int c = tid >> 3, p = tid & 7;
    T out[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = tile[p * 8 + e][c];
    *reinterpret_cast<u32x4*>(dst + ((b * H + h) * (int64_t)C + ct * 32 + c) * Tp + (int64_t)it * 64 + p * 8) =
        *reinterpret_cast<const u32x4*>(out);
  }
}


// WANGO feature layouts of phi(sqrt(tau) x) for x = q or k ([TANGO] §2.2 eq. 8),
// row-major [M][H*dh] (plain, and/or in the permuted feature order of each
// group of 32 that the scan reads for its destination features).
template <typename T>
__global__ __launch_bounds__(256) void phi_kernel(const T* __restrict__ src, T* __restrict__ plain,
                                                  T* __restrict__ perm, const float* theta, int H, int dh,
                                                  int64_t n) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= n) return;
  const int HD = H * dh;
  const int64_t m = id / HD;
  const int col = (int)(id % HD), h = col / dh, e = col % dh;
  const float st = sqrtf(__expf(fminf(theta[h], kLogTauMax)));
  const T v = (T)phi_feature(st * (float)src[id], 1.0f / sqrtf((float)dh));
  if (plain) plain[id] = v;
  if (perm) perm[m * HD + h * dh + (e / 32) * 32 + feature_slot(e % 32)] = v;
}

// Everything the WANGO backward derives from the unit queries and keys, in one
// pass over tiles of 64 positions x 32 columns (a group of 32 columns of one
// head), 16-byte accesses throughout:
//   forward order: q and k transposed per head; p = phi(sqrt(tau) q) and
//   a = phi(sqrt(tau) k) ([TANGO] §2.2 eq. 8) row-major and transposed;
//   the time-reversed problem of dg (destination row i' reads source row
//   T-1-i', zero past the end): the reversed q and k row-major, the
//   destination features phi(sqrt(tau) k_rev) in the permuted feature order of
//   each group of 32, and the source features phi(sqrt(tau) q_rev) packed
//   [M/32][4][H*dh][8].
// The same values as the transpose, reversal, phi and pack kernels would
// produce one launch at a time.  Grid: B * H * (dh / 32) * (Tp / 64).
template <typename T>
__global__ __launch_bounds__(256) void qk_prep_kernel(BwdArgs a, T* __restrict__ fq_perm, T* __restrict__ fk_pk) {
  __shared__ T tile[4][64][32 + 8];
  const int dh = a.dh, HD = a.H * dh, Tp = a.Tp;
  int64_t id = blockIdx.x;
  const int it = (int)(id % (Tp / 64));
  id /= Tp / 64;
  const int ct = (int)(id % (dh / 32));
  id /= dh / 32;
  const int h = (int)(id % a.H);
  const int64_t b = id / a.H;
  const int tid = threadIdx.x, r = tid >> 2, p8 = tid & 3;
  const float st = sqrtf(__expf(fminf(a.theta[h], kLogTauMax))), isd = 1.0f / sqrtf((float)dh);
  const int64_t col = (int64_t)h * dh + ct * 32 + p8 * 8;
  const T* qh = static_cast<const T*>(a.qh);
  const T* kh = static_cast<const T*>(a.kh);
  auto phi8 = [&](const u32x4& x) {
    const T* e8 = reinterpret_cast<const T*>(&x);
    u32x4 y;
    T* o8 = reinterpret_cast<T*>(&y);
#pragma unroll
    for (int e = 0; e < 8; ++e) o8[e] = (T)phi_feature(st * (float)e8[e], isd);
    return y;
  };
  // forward order: row-major features, then the four transposed tiles
  {
    const int64_t m = b * Tp + (int64_t)it * 64 + r;
    const u32x4 q8 = *reinterpret_cast<const u32x4*>(qh + m * HD + col);
    const u32x4 k8 = *reinterpret_cast<const u32x4*>(kh + m * HD + col);
    const u32x4 pv = phi8(q8), av = phi8(k8);
    *reinterpret_cast<u32x4*>(static_cast<T*>(a.p_rm) + m * HD + col) = pv;
    *reinterpret_cast<u32x4*>(static_cast<T*>(a.a_rm) + m * HD + col) = av;
    *reinterpret_cast<u32x4*>(&tile[0][r][p8 * 8]) = q8;
    *reinterpret_cast<u32x4*>(&tile[1][r][p8 * 8]) = k8;
    *reinterpret_cast<u32x4*>(&tile[2][r][p8 * 8]) = pv;
    *reinterpret_cast<u32x4*>(&tile[3][r][p8 * 8]) = av;
  }
  __syncthreads();
  {   // 32 columns x 8 pieces of 8 positions, per array
    const int c = tid >> 3, p = tid & 7;
    const int64_t dst = ((b * a.H + h) * (int64_t)dh + ct * 32 + c) * Tp + (int64_t)it * 64 + p * 8;
    T* outs[4] = {static_cast<T*>(a.qT), static_cast<T*>(a.kT), static_cast<T*>(a.pT), static_cast<T*>(a.aT)};
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      T out[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = tile[x][p * 8 + e][c];
      *reinterpret_cast<u32x4*>(outs[x] + dst) = *reinterpret_cast<const u32x4*>(out);
    }
  }
  __syncthreads();   // the tiles are reused below
  // reversed problem: destination rows it*64 .. it*64+63
  {
    const int i2 = it * 64 + r;
    const bool live = i2 < a.T;
    const int64_t m2 = b * Tp + i2, src = b * Tp + (live ? a.T - 1 - i2 : 0);
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 q8 = live ? *reinterpret_cast<const u32x4*>(qh + src * HD + col) : z;
    const u32x4 k8 = live ? *reinterpret_cast<const u32x4*>(kh + src * HD + col) : z;
    *reinterpret_cast<u32x4*>(static_cast<T*>(a.q_rev) + m2 * HD + col) = q8;
    *reinterpret_cast<u32x4*>(static_cast<T*>(a.k_rev) + m2 * HD + col) = k8;
    const u32x4 fq = phi8(k8), fk = phi8(q8);
    const T* f8 = reinterpret_cast<const T*>(&fq);
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[0][r][feature_slot(p8 * 8 + e)] = f8[e];
    *reinterpret_cast<u32x4*>(&tile[1][r][p8 * 8]) = fk;
  }
  __syncthreads();
  {
    const int64_t m2 = b * Tp + (int64_t)it * 64 + r;
    *reinterpret_cast<u32x4*>(fq_perm + m2 * HD + col) = *reinterpret_cast<const u32x4*>(&tile[0][r][p8 * 8]);
    // packed source features: two 32-row blocks, 4 slot groups x 32 columns each
    const int bb = tid >> 7, grp = (tid >> 5) & 3, cl = tid & 31;
    T out[8];
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) out[s8] = tile[1][bb * 32 + perm_slot(grp, s8)][cl];
    const int64_t blk = (b * Tp + (int64_t)it * 64) / 32 + bb;
    *reinterpret_cast<u32x4*>(fk_pk + ((blk * 4 + grp) * (int64_t)HD + h * dh + ct * 32 + cl) * 8) =
        *reinterpret_cast<const u32x4*>(out);
  }
}

// KW sums: per tile t of (sequence, head) bh, tsum[e][f] = sum over the
// tile's rows j of aT[e][j] x[j][f], x the augmented g (S) or u (R) rows as
// they lie (row-major).  A workgroup stages a 128-row x 64-column tile of x in
// LDS with 16-byte writes and assembles each MFMA B fragment (8 consecutive
// rows of one column) from 2-byte reads; the A fragments come straight from
// the per-head transposed features.  Wave w takes columns 16 w .. 16 w + 15 of
// the block and every d_h row, over the tile's four k-steps in order (the
// same MFMA sequence per output block as a GEMM over transposed operands).
// Grid: B*H * nt * (FhC / 64) workgroups of 256.
template <int DH>
__global__ __launch_bounds__(256) void state_sums_kernel(WStateArgs w) {
  typedef __bf16 T;
  constexpr int NE = DH / 16, XS = 64 + 8;   // row stride of the staged tile (16-byte aligned)
  __shared__ __align__(16) T xs[kBwdTile][XS];
  const int nfb = w.FhC / 64;
  int64_t id = blockIdx.x;
  const int fb = (int)(id % nfb);
  id /= nfb;
  const int t = (int)(id % w.nt);
  const int64_t bh = id / w.nt;
  const int h = (int)(bh % w.H);
  const int64_t b = bh / w.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const T* x = static_cast<const T*>(w.xrm);
  const int64_t row0 = b * w.Tp + (int64_t)t * kBwdTile;
  // every global load of the workgroup is issued before the first wait (left
  // alone, the compiler spreads them over the k-steps, one round trip each)
  const T* aT = static_cast<const T*>(w.aT) + bh * DH * (int64_t)w.Tp + (int64_t)t * kBwdTile;
  Frag<T> af[kBwdTile / 32][NE];
#pragma unroll
  for (int ks = 0; ks < kBwdTile / 32; ++ks)
#pragma unroll
    for (int eb = 0; eb < NE; ++eb) af[ks][eb] = load_frag<T>(aT + (int64_t)(eb * 16 + li) * w.Tp + ks * 32 + lg * 8);
  u32x4 xv[kBwdTile * 8 / 256];
#pragma unroll
  for (int pp = 0; pp < kBwdTile * 8 / 256; ++pp) {   // 128 rows x 8 pieces of 8 columns
    const int pc = tid + 256 * pp, r = pc >> 3, q = pc & 7;
    xv[pp] = *reinterpret_cast<const u32x4*>(x + ((row0 + r) * w.H + h) * w.FhC + fb * 64 + q * 8);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int pp = 0; pp < kBwdTile * 8 / 256; ++pp) {
    const int pc = tid + 256 * pp, r = pc >> 3, q = pc & 7;
    *reinterpret_cast<u32x4*>(&xs[r][q * 8]) = xv[pp];
  }
  __syncthreads();
  f32x4 acc[NE];
#pragma unroll
  for (int eb = 0; eb < NE; ++eb) acc[eb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < kBwdTile / 32; ++ks) {
    Frag<T> bf;
#pragma unroll
    for (int i = 0; i < 8; ++i) bf[i] = xs[ks * 32 + lg * 8 + i][wave * 16 + li];
#pragma unroll
    for (int eb = 0; eb < NE; ++eb) mma(acc[eb], af[ks][eb], bf);
  }
  float* out = w.tsum + ((bh * w.nt + t) * DH) * (int64_t)w.FhC + fb * 64 + wave * 16 + li;
#pragma unroll
  for (int eb = 0; eb < NE; ++eb)
#pragma unroll
    for (int r = 0; r < 4; ++r) out[(int64_t)(eb * 16 + lg * 4 + r) * w.FhC] = acc[eb][r];
}

// Shifted prefix (S) or suffix (R) over the tiles of the per-tile sums, stored
// in bf16: S[t] = sum_{t' <= t - nb} tsum[t'], R[t] = sum_{t' >= t + nb} tsum[t'].
// One thread per element; the tiles go in batches of kScanBatch whose loads are
// all issued before the first add (the loads do not depend on the sum).
constexpr int kScanBatch = 32;
__global__ __launch_bounds__(256) void state_scan_kernel(WStateArgs w, int reverse) {
  const int64_t E = (int64_t)w.dh * w.FhC;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)w.B * w.H * E) return;
  const int64_t bh = id / E, el = id % E;
  const float* ts = w.tsum + bh * w.nt * E + el;
  __bf16* st = static_cast<__bf16*>(w.state) + bh * w.nt * E + el;
  float acc = 0.f;
  for (int n0 = 0; n0 < w.nt; n0 += kScanBatch) {
    // step n visits tile t = n (prefix) or nt - 1 - n (suffix), adding the
    // tile nb before (after) it
    float v[kScanBatch];
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      const int n = n0 + u, t = reverse ? w.nt - 1 - n : n, src = reverse ? t + w.nb : t - w.nb;
      v[u] = (n < w.nt && src >= 0 && src < w.nt) ? ts[(int64_t)src * E] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      const int n = n0 + u, t = reverse ? w.nt - 1 - n : n;
      acc += v[u];
      if (n < w.nt) st[(int64_t)t * E] = (__bf16)acc;
    }
  }
}

// WANGO finish: dq = window part + sqrt(tau) phi'(sqrt(tau) q) (near + far dp),
// dk alike with da.  Each element's share of dtheta through the features,
// sqrt(tau) / 2 (dp phi'(sqrt(tau) q) q + da phi'(sqrt(tau) k) k), is summed per
// head within the workgroup: theta_blk[block][H].
__global__ __launch_bounds__(256) void wango_finish_kernel(BwdArgs a, float* theta_blk) {
  __shared__ float val[8];
  __shared__ int head[8];
  const int64_t M = (int64_t)a.B * a.Tp;
  const int HD = a.H * a.dh;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float share = 0.f;
  int h = -1;
  if (id < M * HD) {
    const int64_t m = id / HD;
    h = (int)(id % HD) / a.dh;
    const bool live = (int)(m % a.Tp) < a.T;
    const float tau = __expf(fminf(a.theta[h], kLogTauMax));
    const float st = sqrtf(tau), escale = __expf(-tau);   // far read-outs are unscaled
    const float isd = 1.0f / sqrtf((float)a.dh);
    const float* P = a.part;
    const float dp = P[2 * M * HD + id] + escale * P[4 * M * HD + id];
    const float da = P[3 * M * HD + id] + escale * P[5 * M * HD + id];
    const float q = (float)static_cast<const __bf16*>(a.qh)[id];
    const float k = (float)static_cast<const __bf16*>(a.kh)[id];
    const float xq = st * q, xk = st * k;
    const float fq = (xq > 0.f ? 1.0f : __expf(xq)) * isd;   // phi'
    const float fk = (xk > 0.f ? 1.0f : __expf(xk)) * isd;
    a.dq[id] = live ? P[id] + st * fq * dp : 0.f;
    a.dk[id] = live ? P[M * HD + id] + st * fk * da : 0.f;
    if (live) share = 0.5f * st * (dp * fq * q + da * fk * k);
  }
  // a wave spans at most two heads (d_h >= 32): two wave sums, then per head
  // the four waves' partials in order (the sum does not depend on timing)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h0 = __shfl(h, 0);
  int h1 = h != h0 ? h : -1;   // the other head of the wave, if any (the row may wrap to head 0)
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) h1 = max(h1, __shfl_xor(h1, o));
  const float lo = wave_sum(h == h0 ? share : 0.f), hi = wave_sum(h != h0 ? share : 0.f);
  if (lane == 0) {
    val[wave * 2] = lo;
    val[wave * 2 + 1] = hi;
    head[wave * 2] = h0;
    head[wave * 2 + 1] = h1;
  }
  __syncthreads();
  if (threadIdx.x < a.H) {
    float sum = 0.f;
    for (int t = 0; t < 8; ++t)
      if (head[t] == (int)threadIdx.x) sum += val[t];
    theta_blk[(int64_t)blockIdx.x * a.H + threadIdx.x] = sum;
  }
}

// Sums the chunk partials into dq, dk: a row of tile r takes the dq chunks
// 0 .. r / kBwdChunkTiles and the dk chunks r / kBwdChunkTiles .. (nt - 1) /
// kBwdChunkTiles (the chunks that hold its terms).
__global__ __launch_bounds__(256) void bwd_finish_kernel(BwdArgs a, int nch) {
  const int64_t M = (int64_t)a.B * a.Tp;
  const int HD = a.H * a.dh;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= M * HD) return;
  const int64_t m = id / HD;
  const int i = (int)(m % a.Tp);
  const int rc = (i / kBwdTile) / kBwdChunkTiles, lastc = (a.Tp / kBwdTile - 1) / kBwdChunkTiles;
  float sq = 0.f, sk = 0.f;
  for (int c = 0; c <= rc; ++c) sq += a.part[(int64_t)c * M * HD + id];
  for (int c = rc; c <= lastc; ++c) sk += a.part[((int64_t)nch + c) * M * HD + id];
  const bool live = i < a.T;
  a.dq[id] = live ? sq : 0.f;
  a.dk[id] = live ? sk : 0.f;
}

// Per head: dtheta from the per-item partials, dnull from delta.  One block
// per head.
__global__ __launch_bounds__(256) void bwd_scalars_kernel(BwdArgs a, int64_t ntri, const float* theta_blk) {
  __shared__ float red[2][256];
  const int h = blockIdx.x, tid = threadIdx.x;
  const float tau = __expf(fminf(a.theta[h], kLogTauMax));
  float th = 0.f, nb = 0.f;
  // tiles of head h: (b * H + h) * ntri + t
  for (int64_t b = 0; b < a.B; ++b)
    for (int64_t k = tid; k < ntri; k += 256) th += a.part_theta[(b * a.H + h) * ntri + k];
  if (theta_blk) {   // WANGO: the features' share, per finish workgroup
    const int64_t nblk = ceil_div((int64_t)a.B * a.Tp * a.H * a.dh, 256);
    for (int64_t x = tid; x < nblk; x += 256) th += theta_blk[x * a.H + h];
  }
  if (a.null_bias) {
    const float nw = __expf(a.null_bias[h] - tau);
    const int64_t M = (int64_t)a.B * a.Tp;
    for (int64_t m = tid; m < M; m += 256) {
      const int i = (int)(m % a.Tp);
      if (i < a.T) nb += a.delta[(int64_t)h * M + m] * (float)(i + 1) * nw;
    }
  }
  red[0][tid] = th;
  red[1][tid] = nb;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) {
      red[0][tid] += red[0][tid + s];
      red[1][tid] += red[1][tid + s];
    }
    __syncthreads();
  }
  if (tid == 0) {
    a.dtheta[h] = a.theta[h] < kLogTauMax ? red[0][0] : 0.f;
    if (a.dnull) a.dnull[h] = red[1][0];
  }
}

}  // namespace

BwdPlan tango_bwd_plan(int B, int Tp, int Fhp, int H) {
  BwdPlan p;
  p.FhC = Fhp;
  p.nt = Tp / kBwdTile;
  p.ntri = (int64_t)p.nt * (p.nt + 1) / 2;
  p.nch = (int)ceil_div(p.nt, kBwdChunkTiles);
  p.nb = 0;
  p.nprod = 2;
  p.items_ds = (int64_t)B * H * p.ntri;
  p.items_mm = p.nprod * (int64_t)B * H * p.nt * p.nch;
  return p;
}

BwdPlan wango_bwd_plan(int B, int Tp, int Fhp, int H, int window) {
  BwdPlan p;
  p.FhC = Fhp + 64;   // augmented rows: delta / 1 in column Fhp
  p.nt = Tp / kBwdTile;
  // near tiles: every window pair (i - j < W) lies in source tiles it - nb + 1 .. it
  p.nb = (int)ceil_div(window - 1, kBwdTile) + 1;
  if (p.nb > kBwdChunkTiles) p.nb = kBwdChunkTiles;   // (callers keep W <= 7 * 128 + 1)
  p.ntri = (int64_t)p.nt * p.nb;
  p.nch = 1;
  p.nprod = 4;
  p.items_ds = (int64_t)B * H * p.ntri;
  p.items_mm = p.nprod * (int64_t)B * H * p.nt;
  return p;
}

hipError_t launch_tango_bwd_prep(const BwdArgs& a, const BwdPlan& p, hipStream_t s, bool qk) {
  const int64_t M = (int64_t)a.B * a.Tp;
  const int HD = a.H * a.dh;
  typedef __bf16 T;
  t_step = "bwd_rows_kernel";
  hipLaunchKernelGGL(bwd_rows_kernel<T>, dim3((unsigned)ceil_div(M, 4), a.H), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // gates row-major from the packed forward layout
  if (p.FhC % 64 != 0 || a.dh % 32 != 0) return hipErrorInvalidValue;
  t_step = "unpack_kernel";
  hipLaunchKernelGGL(unpack_kernel<T>, dim3((unsigned)((M / 32) * a.H * (p.FhC / 64))), dim3(256), 0, s,
                     static_cast<const T*>(a.gp), a.Fp, static_cast<T*>(a.g_rm), a.H, a.Fhp, p.FhC, a.Fh,
                     a.window > 0 ? a.Fhp : -1, a.Tp, a.T);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t nblk = M / 32;
  if (qk) {
    // queries and keys transposed per head (the B operands of dk and dq)
    t_step = "transpose_kernel";
    const dim3 tgrid((unsigned)((int64_t)a.B * a.H * (a.dh / 32) * (a.Tp / 64)));
    hipLaunchKernelGGL(transpose_kernel<T>, tgrid, dim3(256), 0, s, static_cast<const T*>(a.qh),
                       static_cast<T*>(a.qT), a.H, a.dh, a.Tp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    t_step = "transpose_kernel";
    hipLaunchKernelGGL(transpose_kernel<T>, tgrid, dim3(256), 0, s, static_cast<const T*>(a.kh),
                       static_cast<T*>(a.kT), a.H, a.dh, a.Tp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // the reversed problem of dg: reversed queries / keys, reversed u packed
    // with the forward's head padding
    const int64_t nr = M * HD;
    t_step = "reverse_rows_kernel";
    hipLaunchKernelGGL(reverse_rows_kernel<T>, dim3((unsigned)ceil_div(nr, 256)), dim3(256), 0, s,
                       static_cast<const T*>(a.qh), static_cast<T*>(a.q_rev), HD, a.Tp, a.T, M);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    t_step = "reverse_rows_kernel";
    hipLaunchKernelGGL(reverse_rows_kernel<T>, dim3((unsigned)ceil_div(nr, 256)), dim3(256), 0, s,
                       static_cast<const T*>(a.kh), static_cast<T*>(a.k_rev), HD, a.Tp, a.T, M);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  t_step = "pack_kernel";
  hipLaunchKernelGGL(pack_kernel<T>, dim3((unsigned)(nblk * (a.Fp / 32))), dim3(128), 0, s,
                     static_cast<const T*>(a.u_rm), (int64_t)a.H * p.FhC, static_cast<T*>(a.u_rev_pk), a.Fp, a.Fhp,
                     p.FhC, a.Fh, a.Tp, a.T, 1);
  return hipGetLastError();
}

hipError_t launch_tango_bwd_finish(const BwdArgs& a, const BwdPlan& p, hipStream_t s) {
  const int64_t n = (int64_t)a.B * a.Tp * a.H * a.dh;
  hipLaunchKernelGGL(bwd_finish_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, a, p.nch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_scalars_kernel, dim3(a.H), dim3(256), 0, s, a, p.ntri, nullptr);
  return hipGetLastError();
}

hipError_t launch_wango_state_sums(const WStateArgs& w, hipStream_t s) {
  if (w.FhC % 64 != 0 || w.Tp % kBwdTile != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((int64_t)w.B * w.H * w.nt * (w.FhC / 64))), block(256);
  switch (w.dh) {
    case 32: hipLaunchKernelGGL(state_sums_kernel<32>, grid, block, 0, s, w); break;
    case 64: hipLaunchKernelGGL(state_sums_kernel<64>, grid, block, 0, s, w); break;
    case 128: hipLaunchKernelGGL(state_sums_kernel<128>, grid, block, 0, s, w); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_wango_state_scan(const WStateArgs& w, bool reverse, hipStream_t s) {
  const int64_t n = (int64_t)w.B * w.H * w.dh * w.FhC;
  hipLaunchKernelGGL(state_scan_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, w, reverse ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_wango_bwd_features(const BwdArgs& a, void* fq_perm, void* tmp_rm, const void* q_src,
                                     const void* k_src, void* fk_pk, hipStream_t s) {
  typedef __bf16 T;
  const int64_t M = (int64_t)a.B * a.Tp;
  const int HD = a.H * a.dh;
  const int64_t n = M * HD;
  const dim3 grid((unsigned)ceil_div(n, 256)), block(256);
  // destination features (permuted order) of q_src, source features of k_src packed
  t_step = "phi_kernel";
  hipLaunchKernelGGL(phi_kernel<T>, grid, block, 0, s, static_cast<const T*>(q_src), static_cast<T*>(nullptr),
                     static_cast<T*>(fq_perm), a.theta, a.H, a.dh, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  t_step = "phi_kernel";
  hipLaunchKernelGGL(phi_kernel<T>, grid, block, 0, s, static_cast<const T*>(k_src), static_cast<T*>(tmp_rm),
                     static_cast<T*>(nullptr), a.theta, a.H, a.dh, n);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t nblk = M / 32, nqk = nblk * 4 * HD;
  t_step = "pack_kernel";
  hipLaunchKernelGGL(pack_kernel<T>, dim3((unsigned)(nblk * (HD / 32))), dim3(128), 0, s,
                     static_cast<const T*>(tmp_rm), (int64_t)HD, static_cast<T*>(fk_pk), HD, HD, HD, HD, a.Tp, a.T, 0);
  return hipGetLastError();
}

hipError_t launch_wango_bwd_prep(const BwdArgs& a, const BwdPlan& p, void* fq_perm, void* fk_pk, hipStream_t s) {
  // the TANGO prep's augmented u and g rows and reversed packed u, then every
  // q/k-derived array (including the reversed scan's features) in one launch
  hipError_t e = launch_tango_bwd_prep(a, p, s, false);
  if (e != hipSuccess) return e;
  typedef __bf16 T;
  if (a.dh % 32 != 0 || a.Tp % 64 != 0) return hipErrorInvalidValue;
  t_step = "qk_prep_kernel";
  hipLaunchKernelGGL(qk_prep_kernel<T>, dim3((unsigned)((int64_t)a.B * a.H * (a.dh / 32) * (a.Tp / 64))), dim3(256),
                     0, s, a, static_cast<T*>(fq_perm), static_cast<T*>(fk_pk));
  return hipGetLastError();
}

const char* bwd_last_step() { return t_step; }

hipError_t launch_wango_bwd_finish(const BwdArgs& a, const BwdPlan& p, float* theta_blk, hipStream_t s) {
  if (a.H > kMaxBwdHeads) return hipErrorInvalidValue;
  const int64_t n = (int64_t)a.B * a.Tp * a.H * a.dh;
  hipLaunchKernelGGL(wango_finish_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, a, theta_blk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_scalars_kernel, dim3(a.H), dim3(256), 0, s, a, p.ntri, theta_blk);
  return hipGetLastError();
}

}  // namespace tango
