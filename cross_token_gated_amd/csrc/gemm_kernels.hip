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
// Both use a 256-thread workgroup (four waves in a 2 x 2 grid) over a BM x BN
// output tile; K streams through double-buffered LDS tiles of BK columns, and
// every 16 x 16 block is an MFMA accumulator (see common.hpp).
#include "common.hpp"
#include "kernels.hpp"

namespace tango {

namespace {

template <typename T> struct GemmCfg;
template <> struct GemmCfg<bf16> {
  static constexpr int BM = 128, BN = 128, BK = 64;
};
template <> struct GemmCfg<float> {
  static constexpr int BM = 64, BN = 128, BK = 32;
};

constexpr int kThreads = 256;

// LDS row stride of an operand tile (elements): BK plus 16 bytes of padding.
template <typename T> constexpr int op_stride() { return GemmCfg<T>::BK + 16 / (int)sizeof(T); }
// LDS row stride of the fp32 output tile.
constexpr int kCStride = 128 + 4;

template <typename T> constexpr int op_tile_elems(int rows) { return rows * op_stride<T>(); }

template <typename T> constexpr size_t gemm_lds_bytes() {
  using C = GemmCfg<T>;
  size_t ops = 2 * (size_t)(op_tile_elems<T>(C::BM) + op_tile_elems<T>(C::BN)) * sizeof(T);
  size_t out = (size_t)C::BM * kCStride * sizeof(float);
  return (ops > out ? ops : out) + (size_t)C::BM * sizeof(float);
}

// 16-byte piece = PE elements.
template <typename T> constexpr int piece_elems() { return 16 / (int)sizeof(T); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The MFMA inner product of one BK-wide LDS tile for one wave.
// Wave tile: WM x WN = (BM/2) x (BN/2); blocks IB x JB of 16 x 16.
template <typename T>
__device__ __forceinline__ void tile_mma(f32x4 (&acc)[GemmCfg<T>::BM / 32][GemmCfg<T>::BN / 32],
                                         const T* __restrict__ As, const T* __restrict__ Bs,
                                         int wr, int wc, int lane) {
  using C = GemmCfg<T>;
  constexpr int IB = C::BM / 32, JB = C::BN / 32, S = op_stride<T>();
  const int row = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < C::BK / 32; ++ks) {
    Frag<T> a[IB], b[JB];
#pragma unroll
    for (int i = 0; i < IB; ++i)
      a[i] = load_frag<T>(As + (wr * (C::BM / 2) + i * 16 + row) * S + ks * 32 + grp * 8);
#pragma unroll
    for (int j = 0; j < JB; ++j)
      b[j] = load_frag<T>(Bs + (wc * (C::BN / 2) + j * 16 + row) * S + ks * 32 + grp * 8);
#pragma unroll
    for (int i = 0; i < IB; ++i)
#pragma unroll
      for (int j = 0; j < JB; ++j) mma(acc[i][j], a[i], b[j]);
  }
}

// Generic double-buffered main loop.  load_a(pass, row, kpiece, kt) /
// load_b(row, kpiece, kt) return one 16-byte piece of the A (BM x BK) / B
// (BN x BK) tile of k-tile kt; `pass` is the compile-time index of the row
// pass (row = this thread's first row + pass * rows-per-pass).
template <typename T, typename LA, typename LB>
__device__ __forceinline__ void gemm_mainloop(f32x4 (&acc)[GemmCfg<T>::BM / 32][GemmCfg<T>::BN / 32],
                                              T* lds, int nk, LA load_a, LB load_b) {
  using C = GemmCfg<T>;
  constexpr int PR = C::BK / piece_elems<T>();     // pieces per row (8)
  constexpr int RPP = kThreads / PR;               // rows per pass (32)
  constexpr int PA = C::BM / RPP, PB = C::BN / RPP;
  constexpr int S = op_stride<T>();
  // tile addresses are computed from the LDS base (not picked from an array
  // of pointers), so every access stays a ds_read / ds_write
  constexpr int TA = op_tile_elems<T>(C::BM), TB = op_tile_elems<T>(C::BN);
  auto As = [&](int buf) { return lds + buf * TA; };
  auto Bs = [&](int buf) { return lds + 2 * TA + buf * TB; };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int prow = tid / PR, pcol = tid % PR;
  u32x4 ra[PA], rb[PB];
  auto fetch = [&](int kt) {
#pragma unroll
    for (int p = 0; p < PA; ++p) ra[p] = load_a(p, prow + p * RPP, pcol, kt);
#pragma unroll
    for (int p = 0; p < PB; ++p) rb[p] = load_b(prow + p * RPP, pcol, kt);
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PA; ++p)
      *reinterpret_cast<u32x4*>(As(buf) + (prow + p * RPP) * S + pcol * piece_elems<T>()) = ra[p];
#pragma unroll
    for (int p = 0; p < PB; ++p)
      *reinterpret_cast<u32x4*>(Bs(buf) + (prow + p * RPP) * S + pcol * piece_elems<T>()) = rb[p];
  };
  fetch(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) fetch(kt + 1);
    tile_mma<T>(acc, As(buf), Bs(buf), wr, wc, lane);
    if (kt + 1 < nk) stash(buf ^ 1);
    __syncthreads();
  }
}

// Write the wave accumulators, times the row scale rs[row] (or 1), to the fp32
// LDS tile Cs[BM][kCStride].
template <typename T>
__device__ __forceinline__ void acc_to_lds(const f32x4 (&acc)[GemmCfg<T>::BM / 32][GemmCfg<T>::BN / 32],
                                           float* Cs, const float* rs) {
  using C = GemmCfg<T>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1, col = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int i = 0; i < C::BM / 32; ++i)
#pragma unroll
    for (int j = 0; j < C::BN / 32; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wr * (C::BM / 2) + i * 16 + grp * 4 + r;
        const float s = rs ? rs[row] : 1.0f;
        Cs[row * kCStride + wc * (C::BN / 2) + j * 16 + col] = acc[i][j][r] * s;
      }
}

template <typename T> __device__ __forceinline__ u32x4 as_piece(const T* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// N consecutive residual-stream values (float32 or bf16) as floats.
template <typename IO, int N> struct IOVec {
  typedef IO type __attribute__((ext_vector_type(N)));
};
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
// KP: fused RMSNorm + [W_g; W_v; W_q; W_k] projection + epilogue.
// Grid: (ceil(N/BN), M_pad/BM) with N = 2F + 2HD, M_pad = B * Tp.
// ---------------------------------------------------------------------------
template <typename T, typename IO>
__global__ __launch_bounds__(kThreads) void proj_kernel(ProjArgs args) {
  using C = GemmCfg<T>;
  constexpr int PE = piece_elems<T>();
  constexpr int PR = C::BK / PE;
  constexpr int RPP = kThreads / PR;
  constexpr int PA = C::BM / RPP;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* lds = reinterpret_cast<T*>(smem_raw);
  float* rs = reinterpret_cast<float*>(smem_raw + gemm_lds_bytes<T>() - C::BM * sizeof(float));

  const int d = args.d, F = args.F, HD = args.HD, T_len = args.T, Tp = args.Tp;
  const int N = 2 * F + 2 * HD;
  const int n0 = blockIdx.x * C::BN;
  const int64_t m0 = (int64_t)blockIdx.y * C::BM;
  const IO* __restrict__ x = static_cast<const IO*>(args.x);
  const T* __restrict__ gain = static_cast<const T*>(args.gain);
  const int tid = threadIdx.x;
  const int prow = tid / PR, pcol = tid % PR;

  float ssq[PA];  // sums of squares of this thread's h pieces, per row pass
#pragma unroll
  for (int p = 0; p < PA; ++p) ssq[p] = 0.f;

  auto load_a = [&](int pass, int row, int kp, int kt) -> u32x4 {
    const int64_t m = m0 + row;
    const int64_t b = m / Tp, t = m % Tp;
    const int k = kt * C::BK + kp * PE;
    u32x4 z = {0u, 0u, 0u, 0u};
    if (t >= T_len) return z;
    float e[PE];
    load_io<IO, PE>(x + (b * T_len + t) * d + k, e);
    float sq = 0.f;
#pragma unroll
    for (int q = 0; q < PE; ++q) sq += e[q] * e[q];
    ssq[pass] += sq;
    u32x4 out;
    T* o = reinterpret_cast<T*>(&out);
    if (gain) {
#pragma unroll
      for (int q = 0; q < PE; ++q) o[q] = cvt<T>(e[q] * tof<T>(gain[k + q]));
    } else {
#pragma unroll
      for (int q = 0; q < PE; ++q) o[q] = cvt<T>(e[q]);
    }
    return out;
  };
  auto load_b = [&](int row, int kp, int kt) -> u32x4 {
    const int n = n0 + row;
    const int k = kt * C::BK + kp * PE;
    u32x4 z = {0u, 0u, 0u, 0u};
    const T* w;
    if (n < F) w = static_cast<const T*>(args.w_g) + (int64_t)n * d;
    else if (n < 2 * F) w = static_cast<const T*>(args.w_v) + (int64_t)(n - F) * d;
    else if (n < 2 * F + HD) w = static_cast<const T*>(args.w_q) + (int64_t)(n - 2 * F) * d;
    else if (n < N) w = static_cast<const T*>(args.w_k) + (int64_t)(n - 2 * F - HD) * d;
    else return z;
    return as_piece<T>(w + k);
  };

  f32x4 acc[C::BM / 32][C::BN / 32];
#pragma unroll
  for (int i = 0; i < C::BM / 32; ++i)
#pragma unroll
    for (int j = 0; j < C::BN / 32; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  gemm_mainloop<T>(acc, lds, d / C::BK, load_a, load_b);

  // RMSNorm row scales: reduce the squares over the PR threads of each row.
#pragma unroll
  for (int p = 0; p < PA; ++p) {
    float v = ssq[p];
#pragma unroll
    for (int off = 1; off < PR; off <<= 1) v += __shfl_xor(v, off, 64);
    if (pcol == 0) rs[prow + p * RPP] = 1.0f / sqrtf(v / (float)d + args.eps);
  }
  __syncthreads();
  float* Cs = reinterpret_cast<float*>(smem_raw);
  acc_to_lds<T>(acc, Cs, rs);
  __syncthreads();

  // ---- epilogue ----
  // gates: packed layout, 8 rows (one permuted 32-row group slot set) per item
  if (n0 < F) {
    T* gp = static_cast<T*>(args.gp);
    constexpr int NRB = C::BM / 32;
    for (int it = tid; it < NRB * 4 * C::BN; it += kThreads) {
      const int c = it % C::BN, grp = (it / C::BN) & 3, rb = it / (4 * C::BN);
      const int n = n0 + c;
      if (n >= F) continue;
      Frag<T> out;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float a = Cs[(rb * 32 + perm_slot(grp, s)) * kCStride + c];
        out[s] = cvt<T>(a / (1.0f + __expf(-a)));
      }
      store_frag<T>(gp + packed_offset(m0 / 32 + rb, grp, n, F), out);
    }
  }
  // features: row-major [M_pad, F]
  if (n0 + C::BN > F && n0 < 2 * F) {
    T* v = static_cast<T*>(args.v);
    constexpr int P8 = C::BN / 8;
    for (int it = tid; it < C::BM * P8; it += kThreads) {
      const int row = it / P8, c = (it % P8) * 8;
      const int n = n0 + c;
      if (n < F || n >= 2 * F) continue;
      Frag<T> out;
#pragma unroll
      for (int s = 0; s < 8; ++s) out[s] = cvt<T>(Cs[row * kCStride + c + s]);
      store_frag<T>(v + (m0 + row) * F + (n - F), out);
    }
  }
  // queries and keys: RoPE on interleaved pairs, then unit length per head
  if (n0 + C::BN > 2 * F) {
    const int dh = args.dh;
    const int half = dh >> 1;                      // lanes per (row, head)
    const int lane = tid & 63, wave = tid >> 6;
    const int per_wave = 64 / half;                // (row, head) items per wave pass
    const int sub = lane / half, c = lane % half;
    const int c_lo = n0 < 2 * F ? 2 * F - n0 : 0;  // first q/k column in tile
    const int c_hi = min(C::BN, N - n0);
    const int heads_in_tile = (c_hi - c_lo) / dh;
    const int items = C::BM * heads_in_tile;
    const double inv_freq = args.rope_base > 0.f
        ? pow((double)args.rope_base, -2.0 * (double)c / (double)dh) : 0.0;
    for (int base = wave * per_wave; base < items; base += 4 * per_wave) {
      const int item = base + sub;
      const bool ok = item < items;
      const int row = ok ? item / heads_in_tile : 0;
      const int hcol = c_lo + (ok ? item % heads_in_tile : 0) * dh;
      float u0 = ok ? Cs[row * kCStride + hcol + 2 * c] : 0.f;
      float u1 = ok ? Cs[row * kCStride + hcol + 2 * c + 1] : 0.f;
      if (args.rope_base > 0.f) {
        const int64_t pos = (m0 + row) % Tp;
        double ang = (double)pos * inv_freq;
        ang = fmod(ang, 6.283185307179586476925286766559);
        double sn, cs;
        sincos(ang, &sn, &cs);
        const float fs = (float)sn, fc = (float)cs;
        const float r0 = u0 * fc - u1 * fs, r1 = u0 * fs + u1 * fc;
        u0 = r0;
        u1 = r1;
      }
      float ss = u0 * u0 + u1 * u1;
      for (int off = 1; off < half; off <<= 1) ss += __shfl_xor(ss, off, 64);
      const float inv = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
      if (ok) {
        const int n = n0 + hcol;
        const bool is_q = n < 2 * F + HD;
        const int e = is_q ? n - 2 * F : n - 2 * F - HD;   // column within q or k
        T* dst = (is_q ? static_cast<T*>(args.qh) : static_cast<T*>(args.kh)) + (m0 + row) * HD + e;
        const T w0 = cvt<T>(u0 * inv), w1 = cvt<T>(u1 * inv);
        dst[2 * c] = w0;
        dst[2 * c + 1] = w1;
        if (args.fq) {
          // WANGO features phi(sqrt(tau) u) ([TANGO] §2.2 eq. 8) of the stored
          // unit vector: queries go out directly in the permuted feature order,
          // keys back into the tile for the packed store below
          const float st = sqrtf(__expf(fminf(args.theta[e / dh], 2.995732273553991f)));
          const float isd = 1.0f / sqrtf((float)dh);
          const float p0 = phi_feature(st * tof<T>(w0), isd), p1 = phi_feature(st * tof<T>(w1), isd);
          if (is_q) {
            T* fq = static_cast<T*>(args.fq) + (m0 + row) * HD + (e + 2 * c) / 32 * 32 +
                    feature_slot((e + 2 * c) % 32);
            fq[0] = cvt<T>(p0);
            fq[1] = cvt<T>(p1);
          } else {
            Cs[row * kCStride + hcol + 2 * c] = p0;
            Cs[row * kCStride + hcol + 2 * c + 1] = p1;
          }
        }
      }
    }
    if (args.fk) {
      // key features in the source-packed layout, as the gates
      __syncthreads();
      const int k_lo = max(c_lo, 2 * F + HD - n0);
      if (k_lo < c_hi) {
        T* fk = static_cast<T*>(args.fk);
        constexpr int NRB = C::BM / 32;
        const int ncols = c_hi - k_lo;
        for (int it = tid; it < NRB * 4 * ncols; it += kThreads) {
          const int c2 = k_lo + it % ncols, grp = (it / ncols) & 3, rb = it / (4 * ncols);
          Frag<T> out;
#pragma unroll
          for (int s2 = 0; s2 < 8; ++s2) out[s2] = cvt<T>(Cs[(rb * 32 + perm_slot(grp, s2)) * kCStride + c2]);
          store_frag<T>(fk + packed_offset(m0 / 32 + rb, grp, n0 + c2 - 2 * F - HD, HD), out);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// KO: out = x + (gbar * v) W_o^T.  Grid: (d/BN, M_pad/BM).
// ---------------------------------------------------------------------------
template <typename T, typename IO>
__global__ __launch_bounds__(kThreads) void out_kernel(OutArgs args) {
  using C = GemmCfg<T>;
  constexpr int PE = piece_elems<T>();
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* lds = reinterpret_cast<T*>(smem_raw);
  const int d = args.d, F = args.F, T_len = args.T, Tp = args.Tp;
  const int n0 = blockIdx.x * C::BN;
  const int64_t m0 = (int64_t)blockIdx.y * C::BM;
  const T* __restrict__ gbar = static_cast<const T*>(args.gbar);
  const T* __restrict__ v = static_cast<const T*>(args.v);
  const T* __restrict__ wo = static_cast<const T*>(args.w_o);

  auto load_a = [&](int, int row, int kp, int kt) -> u32x4 {
    const int64_t m = m0 + row;
    const int k = kt * C::BK + kp * PE;
    u32x4 ga = as_piece<T>(gbar + m * F + k);
    u32x4 va = as_piece<T>(v + m * F + k);
    const T* ge = reinterpret_cast<const T*>(&ga);
    const T* ve = reinterpret_cast<const T*>(&va);
    u32x4 out;
    T* o = reinterpret_cast<T*>(&out);
#pragma unroll
    for (int q = 0; q < PE; ++q) o[q] = cvt<T>(tof<T>(ge[q]) * tof<T>(ve[q]));
    return out;
  };
  auto load_b = [&](int row, int kp, int kt) -> u32x4 {
    const int k = kt * C::BK + kp * PE;
    return as_piece<T>(wo + (int64_t)(n0 + row) * F + k);
  };

  f32x4 acc[C::BM / 32][C::BN / 32];
#pragma unroll
  for (int i = 0; i < C::BM / 32; ++i)
#pragma unroll
    for (int j = 0; j < C::BN / 32; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  gemm_mainloop<T>(acc, lds, F / C::BK, load_a, load_b);

  float* Cs = reinterpret_cast<float*>(smem_raw);
  acc_to_lds<T>(acc, Cs, nullptr);
  __syncthreads();

  const IO* __restrict__ x = static_cast<const IO*>(args.x);
  IO* out = static_cast<IO*>(args.out);
  constexpr int P8 = C::BN / 8;
  for (int it = threadIdx.x; it < C::BM * P8; it += kThreads) {
    const int row = it / P8, c = (it % P8) * 8;
    const int64_t m = m0 + row;
    const int64_t b = m / Tp, t = m % Tp;
    if (t >= T_len) continue;
    const int64_t off = (b * T_len + t) * d + n0 + c;
    float o[8];
    load_io<IO, 8>(x + off, o);
#pragma unroll
    for (int s = 0; s < 8; ++s) o[s] += Cs[row * kCStride + c + s];
    store_io<IO, 8>(out + off, o);
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <typename T, typename IO>
hipError_t launch_proj_t(const ProjArgs& a, hipStream_t s) {
  using C = GemmCfg<T>;
  const int N = 2 * a.F + 2 * a.HD;
  dim3 grid((unsigned)ceil_div(N, C::BN), (unsigned)((int64_t)a.B * a.Tp / C::BM));
  hipLaunchKernelGGL((proj_kernel<T, IO>), grid, dim3(kThreads), gemm_lds_bytes<T>(), s, a);
  return hipGetLastError();
}

template <typename T, typename IO>
hipError_t launch_out_t(const OutArgs& a, hipStream_t s) {
  using C = GemmCfg<T>;
  dim3 grid((unsigned)(a.d / C::BN), (unsigned)((int64_t)a.B * a.Tp / C::BM));
  hipLaunchKernelGGL((out_kernel<T, IO>), grid, dim3(kThreads), gemm_lds_bytes<T>(), s, a);
  return hipGetLastError();
}

hipError_t launch_proj(const ProjArgs& a, bool bf, bool io_bf, hipStream_t s) {
  if (bf) return io_bf ? launch_proj_t<bf16, bf16>(a, s) : launch_proj_t<bf16, float>(a, s);
  return io_bf ? launch_proj_t<float, bf16>(a, s) : launch_proj_t<float, float>(a, s);
}
hipError_t launch_out(const OutArgs& a, bool bf, bool io_bf, hipStream_t s) {
  if (bf) return io_bf ? launch_out_t<bf16, bf16>(a, s) : launch_out_t<bf16, float>(a, s);
  return io_bf ? launch_out_t<float, bf16>(a, s) : launch_out_t<float, float>(a, s);
}

namespace {
template <typename K> hipError_t raise_lds(K* k, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}
}  // namespace

hipError_t gemm_kernels_init() {
  hipError_t e;
#define TANGO_RAISE(K, T) \
  if ((e = raise_lds(&K, gemm_lds_bytes<T>())) != hipSuccess) return e;
  TANGO_RAISE((proj_kernel<bf16, bf16>), bf16) TANGO_RAISE((proj_kernel<bf16, float>), bf16)
  TANGO_RAISE((proj_kernel<float, bf16>), float) TANGO_RAISE((proj_kernel<float, float>), float)
  TANGO_RAISE((out_kernel<bf16, bf16>), bf16) TANGO_RAISE((out_kernel<bf16, float>), bf16)
  TANGO_RAISE((out_kernel<float, bf16>), float) TANGO_RAISE((out_kernel<float, float>), float)
#undef TANGO_RAISE
  return hipSuccess;
}

}  // namespace tango
