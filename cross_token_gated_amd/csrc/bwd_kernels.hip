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
// Kernels:
//   * row prep: u (row-major, head width padded to a multiple of 256 gate
//     columns) and delta;
//   * layout kernels: row-major <-> the packed [M/32][4][C][8] layout, with an
//     optional reversal of every sequence;
//   * dg: the forward aggregation kernel on the time-reversed problem
//     (queries = reversed keys, keys = reversed queries, gates = reversed u),
//     numerator only, rows stored back in forward order;
//   * dqk: dq (DIR 0) or dk (DIR 1) over one 256-column gate chunk, per
//     workgroup one 128-row tile of "own" rows against 64-row steps of the
//     "other" rows; the chunk partials are summed by the finish kernel.
#include "common.hpp"
#include "kernels.hpp"

namespace tango {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBwdWaves = 8;                 // two per SIMD
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kOwnRows = 128;                // own rows per tile (one 16-row block per wave)
constexpr int kStep = 64;                    // other rows per step
constexpr int kChunk = 256;                  // gate columns per workgroup
constexpr int kChunkKB = kChunk / 32;        // MFMA k blocks of a chunk
constexpr float kLogTauMax = 2.995732273553991f;   // log 20: tau = exp(min(theta, log 20))

// LDS operand layout (as in the forward kernels): a 16-row x 32-k block is four
// 256-byte regions, one per k group g; row r sits at position r xor g.
__device__ __forceinline__ int region_pos(int region, int r, int g) {
  return region * 256 + (r ^ g) * 16;
}

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
  for (int c = lane; c < a.FhC; c += 64) {
    float uv = 0.f;
    if (live && c < a.Fh) {
      uv = (float)dg[c] * rden;
      dot += uv * (float)gb[c];
    }
    u[c] = (T)uv;
  }
  dot = wave_sum(dot);
  if (lane == 0) a.delta[(int64_t)h * a.B * a.Tp + m] = live ? -dot : 0.f;
}

// Row-major [rows][ld] -> packed [rows/32][4][ncols][8].  Packed column n is
// head n / dst_hw, column c = n % dst_hw of it, taken from source column
// (n / dst_hw) * src_hw + c when c < valid_w, else zero.  rev: packed row
// b*Tp + i holds source row b*Tp + T-1-i (rows i >= T are zero).
template <typename T>
__global__ __launch_bounds__(256) void pack_kernel(const T* __restrict__ src, int64_t ld, T* __restrict__ dst,
                                                   int ncols, int dst_hw, int src_hw, int valid_w, int Tp, int T_,
                                                   int rev, int64_t nblk) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_blk = (int64_t)4 * ncols;
  if (id >= nblk * per_blk) return;
  const int64_t blk = id / per_blk;
  const int grp = (int)((id / ncols) % 4), n = (int)(id % ncols);
  const int hd = n / dst_hw, c = n % dst_hw;
  T out[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int64_t row = blk * 32 + perm_slot(grp, s);
    const int64_t b = row / Tp;
    const int i = (int)(row % Tp);
    float v = 0.f;
    if (c < valid_w) {
      if (!rev) {
        v = (float)src[row * ld + (int64_t)hd * src_hw + c];
      } else if (i < T_) {
        v = (float)src[(b * Tp + (T_ - 1 - i)) * ld + (int64_t)hd * src_hw + c];
      }
    }
    out[s] = (T)v;
  }
  *reinterpret_cast<u32x4*>(dst + id * 8) = *reinterpret_cast<const u32x4*>(out);
}

// Packed gates [rows/32][4][H*src_hw][8] -> row-major [rows][H][dst_hw]
// (columns past valid_w zero).
template <typename T>
__global__ __launch_bounds__(256) void unpack_kernel(const T* __restrict__ gp, int src_F, T* __restrict__ dst,
                                                     int H, int src_hw, int dst_hw, int valid_w, int64_t rows) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_row = (int64_t)H * dst_hw;
  if (id >= rows * per_row) return;
  const int64_t row = id / per_row;
  const int n = (int)(id % per_row), hd = n / dst_hw, c = n % dst_hw;
  int grp, s;
  slot_of_row((int)(row % 32), grp, s);
  float v = 0.f;
  if (c < valid_w) v = (float)gp[packed_offset(row / 32, grp, (int64_t)hd * src_hw + c, src_F) + s];
  dst[id] = (T)v;
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

// ---------------------------------------------------------------------------
// dq (DIR 0) / dk (DIR 1) over one gate chunk.
//
// Own rows (fixed per job, one 16-row block per wave): DIR 0 destinations,
// DIR 1 sources.  Other rows (64 per step): DIR 0 the sources j <= own rows,
// DIR 1 the destinations i >= own rows.  Per step and wave, with accumulator
// blocks X[other][own] (other = rows, own = columns):
//   S  = K Q^T  (DIR 0: A = staged keys, B = own queries; DIR 1: A = staged
//        queries, B = own keys) -- the cosine s_ij minus 1 (the accumulator
//        starts at -1), so w = exp2(tau log2e (s - 1));
//   dW = u . g over the chunk (DIR 0: A = staged gate rows, B = own u rows;
//        DIR 1: A = staged u rows, B = own gate rows);
//   ds = tau w (dW + delta) with delta of the destination (chunk 0 only);
//   out^T (d_h x own) += P^T (d_h x other) ds^T with P the packed staged
//        keys (DIR 0) or queries (DIR 1), ds^T through a wave-private LDS
//        block in the packed k order.
// DIR 0 also sums ds * s for dtheta.
template <int DH> struct BwdLds {
  static constexpr int T1 = kStep * DH;            // elements: staged q or k rows, region layout
  static constexpr int T2 = kStep * kChunk;        // staged g or u rows, region layout
  static constexpr int T3 = kStep * DH;            // packed q or k, fragment order
  __bf16 t1[2][T1];
  __bf16 t2[2][T2];
  __bf16 t3[2][T3];
  __bf16 ds[kBwdWaves][16 * kStep];                // wave-private ds^T (own block x 64 other), region layout
  float dl[2][kStep];                              // DIR 1: delta of the staged destinations
  float red[kBwdWaves];
};

template <int DIR, int DH>
__global__ __launch_bounds__(kBwdThreads) void dqk_kernel(BwdArgs a, int rtiles, int nchunk, int64_t items) {
  typedef __bf16 T;
  constexpr int KS = DH / 32;                      // k blocks of d_h
  constexpr int NDB = DH / 16;                     // d_h blocks of the output
  constexpr int C1 = (kStep / 16) * KS;            // 1 KiB chunks of t1
  constexpr int C2 = (kStep / 16) * kChunkKB;      // of t2
  constexpr int C3 = NDB * 2;                      // of t3 (fragments)
  constexpr int P1 = (C1 + kBwdWaves - 1) / kBwdWaves;
  constexpr int P2 = (C2 + kBwdWaves - 1) / kBwdWaves;
  constexpr int P3 = (C3 + kBwdWaves - 1) / kBwdWaves;
  __shared__ BwdLds<DH> sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;

  const int64_t q8 = gridDim.x / 8;
  const int64_t item = (int64_t)(blockIdx.x % 8) * q8 + blockIdx.x / 8;
  if (item >= items) return;
  const int R = rtiles, half = (R + 1) / 2;
  const int p = (int)(item % half);
  int64_t grp = item / half;
  const int c = (int)(grp % nchunk);
  grp /= nchunk;
  const int h = (int)(grp % a.H);
  const int64_t b = grp / a.H;
  const int64_t mseq = b * a.Tp;
  const int HD = a.H * DH;

  const float tau = __expf(fminf(a.theta[h], kLogTauMax));
  const float ktau = tau * kLog2e;
  const bool first_chunk = c == 0;

  // tensors of the two sides
  const T* own_qk = static_cast<const T*>(DIR == 0 ? a.qh : a.kh);     // B operand of S
  const T* own_ug = static_cast<const T*>(DIR == 0 ? a.u_rm : a.g_rm);  // B operand of dW
  const T* oth_qk = static_cast<const T*>(DIR == 0 ? a.kh : a.qh);     // staged t1
  const T* oth_ug = static_cast<const T*>(DIR == 0 ? a.g_rm : a.u_rm);  // staged t2
  const T* oth_pk = static_cast<const T*>(DIR == 0 ? a.kp : a.qp);     // staged t3 (packed)
  const float* delta = a.delta + (int64_t)h * a.B * a.Tp + mseq;

  // staging: other rows [o0, o0 + 64) of this sequence into buffer `buf`
  auto fetch = [&](int o0, u32x4 (&r1)[P1], u32x4 (&r2)[P2], u32x4 (&r3)[P3], f32x4& rd) {
    // DIR 1: delta of the 64 destinations (every wave loads, wave 0 stores)
    if (DIR == 1) rd = *reinterpret_cast<const f32x4*>(delta + o0 + (lane & 15) * 4);
#pragma unroll
    for (int q = 0; q < P1; ++q) {
      const int cc = (wave + kBwdWaves * q) % C1;
      const int jj = cc / KS, kb = cc % KS;
      r1[q] = *reinterpret_cast<const u32x4*>(oth_qk + (mseq + o0 + jj * 16 + (lane >> 2)) * HD + h * DH +
                                              kb * 32 + (lane & 3) * 8);
    }
#pragma unroll
    for (int q = 0; q < P2; ++q) {
      const int cc = (wave + kBwdWaves * q) % C2;
      const int jj = cc / kChunkKB, kb = cc % kChunkKB;
      r2[q] = *reinterpret_cast<const u32x4*>(oth_ug + ((mseq + o0 + jj * 16 + (lane >> 2)) * a.H + h) * a.FhC +
                                              c * kChunk + kb * 32 + (lane & 3) * 8);
    }
#pragma unroll
    for (int q = 0; q < P3; ++q) {
      const int cc = (wave + kBwdWaves * q) % C3;
      const int db = cc >> 1, hf = cc & 1;
      r3[q] = *reinterpret_cast<const u32x4*>(
          oth_pk + packed_offset((mseq + o0) / 32 + hf, lg, (int64_t)h * DH + db * 16 + li, HD));
    }
  };
  auto stash = [&](int buf, const u32x4 (&r1)[P1], const u32x4 (&r2)[P2], const u32x4 (&r3)[P3],
                   const f32x4& rd) {
    if (DIR == 1 && wave == 0 && lane < 16) *reinterpret_cast<f32x4*>(&sm.dl[buf][lane * 4]) = rd;
#pragma unroll
    for (int q = 0; q < P1; ++q) {
      if (C1 % kBwdWaves != 0 && wave + kBwdWaves * q >= C1) break;   // wave-uniform
      const int cc = wave + kBwdWaves * q, jj = cc / KS, kb = cc % KS;
      const int r = lane >> 2, g = lane & 3;
      *reinterpret_cast<u32x4*>(reinterpret_cast<unsigned char*>(sm.t1[buf]) +
                                region_pos((jj * KS + kb) * 4 + g, r, g)) = r1[q];
    }
#pragma unroll
    for (int q = 0; q < P2; ++q) {
      if (C2 % kBwdWaves != 0 && wave + kBwdWaves * q >= C2) break;
      const int cc = wave + kBwdWaves * q, jj = cc / kChunkKB, kb = cc % kChunkKB;
      const int r = lane >> 2, g = lane & 3;
      *reinterpret_cast<u32x4*>(reinterpret_cast<unsigned char*>(sm.t2[buf]) +
                                region_pos((jj * kChunkKB + kb) * 4 + g, r, g)) = r2[q];
    }
#pragma unroll
    for (int q = 0; q < P3; ++q) {
      if (C3 % kBwdWaves != 0 && wave + kBwdWaves * q >= C3) break;
      const int cc = wave + kBwdWaves * q;
      *reinterpret_cast<u32x4*>(reinterpret_cast<unsigned char*>(sm.t3[buf]) + (cc * 64 + lane) * 16) = r3[q];
    }
  };
  auto region_frag = [&](const T* tile, int nkb, int rb, int kb) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const unsigned char*>(tile) +
                                            region_pos((rb * nkb + kb) * 4 + lg, li, lg));
  };

  float dtheta_part = 0.f;

  auto run_job = [&](int tile) {
    const int r0 = tile * kOwnRows;                 // own rows [r0, r0 + 128)
    const int own_row = r0 + wave * 16 + li;        // this lane's own row (B operand column)
    // steps of other rows: DIR 0 sources [0, r0 + 128), DIR 1 destinations [r0, Tp)
    const int s_first = DIR == 0 ? 0 : r0 / kStep;
    const int s_last = DIR == 0 ? (r0 + kOwnRows) / kStep - 1 : a.Tp / kStep - 1;

    bf16x8 bq[KS], bu[kChunkKB];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      bq[ks] = *reinterpret_cast<const bf16x8*>(own_qk + (mseq + own_row) * HD + h * DH + ks * 32 + lg * 8);
#pragma unroll
    for (int kf = 0; kf < kChunkKB; ++kf)
      bu[kf] = *reinterpret_cast<const bf16x8*>(own_ug + ((mseq + own_row) * a.H + h) * a.FhC + c * kChunk +
                                                kf * 32 + lg * 8);
    const float delta_own = DIR == 0 ? delta[own_row] : 0.f;

    f32x4 out[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) out[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    {
      __syncthreads();   // the previous job's last stash is done with the buffers
      u32x4 r1[P1], r2[P2], r3[P3];
      f32x4 rd = {0.f, 0.f, 0.f, 0.f};
      fetch(s_first * kStep, r1, r2, r3, rd);
      stash(0, r1, r2, r3, rd);
      if (s_first + 1 <= s_last) {
        fetch((s_first + 1) * kStep, r1, r2, r3, rd);
        stash(1, r1, r2, r3, rd);
      }
      __syncthreads();
    }
    for (int st = s_first; st <= s_last; ++st) {
      const int buf = (st - s_first) & 1;
      const int o0 = st * kStep;
      u32x4 r1[P1], r2[P2], r3[P3];
      f32x4 rd = {0.f, 0.f, 0.f, 0.f};
      fetch(min(st + 2, s_last) * kStep, r1, r2, r3, rd);   // past the end: re-read the last step
      unsigned char* dsb = reinterpret_cast<unsigned char*>(sm.ds[wave]);
      // S and dW of the four other blocks t side by side, k block by k block:
      // four independent accumulation chains in the MFMA pipeline
      f32x4 sacc[4], wacc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        sacc[t] = f32x4{-1.f, -1.f, -1.f, -1.f};
        wacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int t = 0; t < 4; ++t) mma(sacc[t], region_frag(sm.t1[buf], KS, t, ks), bq[ks]);
#pragma unroll
      for (int kf = 0; kf < kChunkKB; ++kf)
#pragma unroll
        for (int t = 0; t < 4; ++t) mma(wacc[t], region_frag(sm.t2[buf], kChunkKB, t, kf), bu[kf]);
#pragma unroll
      for (int t = 0; t < 4; ++t) {                    // other block t of the step
        float dsv[4];
        const f32x4 dl = DIR == 1 ? *reinterpret_cast<const f32x4*>(&sm.dl[buf][t * 16 + lg * 4])
                                  : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int other = o0 + t * 16 + lg * 4 + r;
          const bool valid = DIR == 0 ? other <= own_row : own_row <= other;   // source <= destination
          const float dlt = first_chunk ? (DIR == 0 ? delta_own : dl[r]) : 0.f;
          const float w = __builtin_amdgcn_exp2f(ktau * sacc[t][r]);
          const float v = valid ? tau * w * (wacc[t][r] + dlt) : 0.f;
          dsv[r] = v;
          if (DIR == 0) dtheta_part += v * (sacc[t][r] + 1.0f);
        }
        // ds^T of block t: rows 4 lg + r of the block are slots r (t even) or
        // 4 + r (t odd) of this lane's fragment for the half t / 2
        bf16x4 q4;
#pragma unroll
        for (int r = 0; r < 4; ++r) q4[r] = (T)dsv[r];
        *reinterpret_cast<bf16x4*>(dsb + region_pos((t >> 1) * 4 + lg, li, lg) + (t & 1) * 8) = q4;
      }
      // out^T += P^T ds^T over the two 32-row halves of the step
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const bf16x8 dfr = *reinterpret_cast<const bf16x8*>(dsb + region_pos(hf * 4 + lg, li, lg));
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8 pf = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const unsigned char*>(sm.t3[buf]) +
                                                             ((db * 2 + hf) * 64 + lane) * 16);
          mma(out[db], pf, dfr);
        }
      }
      __syncthreads();   // every wave is done with buffer buf; buf ^ 1 (stashed a step ago) is visible
      stash(buf, r1, r2, r3, rd);
    }
    // out^T block db: lane holds own row li, d_h columns 16 db + 4 lg + r
    float* dst = (DIR == 0 ? a.part_q : a.part_k) + ((int64_t)c * a.B * a.Tp + mseq + own_row) * HD + h * DH;
#pragma unroll
    for (int db = 0; db < NDB; ++db) *reinterpret_cast<f32x4*>(dst + db * 16 + lg * 4) = out[db];
  };

  run_job(p);
  if (R - 1 - p != p) run_job(R - 1 - p);

  if (DIR == 0) {
    const float s = wave_sum(dtheta_part);
    if (lane == 0) sm.red[wave] = s;
    __syncthreads();
    if (tid == 0) {
      float tot = 0.f;
      for (int w = 0; w < kBwdWaves; ++w) tot += sm.red[w];
      a.part_theta[item] = tot;
    }
  }
}

// Sums the chunk partials into dq, dk; dtheta and dnull per head.
__global__ __launch_bounds__(256) void bwd_finish_kernel(BwdArgs a, int nchunk) {
  const int64_t M = (int64_t)a.B * a.Tp;
  const int HD = a.H * a.dh;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id < M * HD) {
    const int64_t m = id / HD;
    const bool live = (int)(m % a.Tp) < a.T;
    float sq = 0.f, sk = 0.f;
    for (int cc = 0; cc < nchunk; ++cc) {
      sq += a.part_q[cc * M * HD + id];
      sk += a.part_k[cc * M * HD + id];
    }
    a.dq[id] = live ? sq : 0.f;
    a.dk[id] = live ? sk : 0.f;
  }
}

// Per head: dtheta from the per-item partials, dnull from delta.  One block
// per head.
__global__ __launch_bounds__(256) void bwd_scalars_kernel(BwdArgs a, int nchunk, int half) {
  __shared__ float red[2][256];
  const int h = blockIdx.x, tid = threadIdx.x;
  const float tau = __expf(fminf(a.theta[h], kLogTauMax));
  float th = 0.f, nb = 0.f;
  // items of head h: item = ((b * H + h) * nchunk + c) * half + p
  for (int64_t b = 0; b < a.B; ++b)
    for (int64_t k = tid; k < (int64_t)nchunk * half; k += 256)
      th += a.part_theta[((b * a.H + h) * nchunk) * half + k];
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

template <int DIR>
hipError_t launch_dqk(const BwdArgs& a, int rtiles, int nchunk, int64_t items, hipStream_t s) {
  const int64_t q8 = ceil_div(items, 8);
  dim3 grid((unsigned)(8 * q8)), block(kBwdThreads);
  switch (a.dh) {
    case 32: hipLaunchKernelGGL((dqk_kernel<DIR, 32>), grid, block, 0, s, a, rtiles, nchunk, items); break;
    case 64: hipLaunchKernelGGL((dqk_kernel<DIR, 64>), grid, block, 0, s, a, rtiles, nchunk, items); break;
    case 128: hipLaunchKernelGGL((dqk_kernel<DIR, 128>), grid, block, 0, s, a, rtiles, nchunk, items); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

BwdPlan tango_bwd_plan(int B, int Tp, int Fh, int H) {
  BwdPlan p;
  p.FhC = (int)ceil_div(Fh, kChunk) * kChunk;
  p.nchunk = p.FhC / kChunk;
  p.rtiles = Tp / kOwnRows;
  p.half = (p.rtiles + 1) / 2;
  p.items = (int64_t)B * H * p.nchunk * p.half;
  return p;
}

hipError_t launch_tango_bwd_prep(const BwdArgs& a, const BwdPlan& p, hipStream_t s) {
  const int64_t M = (int64_t)a.B * a.Tp;
  const int HD = a.H * a.dh;
  typedef __bf16 T;
  hipLaunchKernelGGL(bwd_rows_kernel<T>, dim3((unsigned)ceil_div(M, 4), a.H), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // gates row-major from the packed forward layout
  const int64_t ng = M * a.H * p.FhC;
  hipLaunchKernelGGL(unpack_kernel<T>, dim3((unsigned)ceil_div(ng, 256)), dim3(256), 0, s,
                     static_cast<const T*>(a.gp), a.Fp, static_cast<T*>(a.g_rm), a.H, a.Fhp, p.FhC, a.Fh, M);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // packed queries and keys (k order = rows), for the third products
  const int64_t nblk = M / 32;
  const int64_t nqk = nblk * 4 * HD;
  hipLaunchKernelGGL(pack_kernel<T>, dim3((unsigned)ceil_div(nqk, 256)), dim3(256), 0, s,
                     static_cast<const T*>(a.qh), (int64_t)HD, static_cast<T*>(a.qp), HD, HD, HD, HD, a.Tp, a.T, 0, nblk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(pack_kernel<T>, dim3((unsigned)ceil_div(nqk, 256)), dim3(256), 0, s,
                     static_cast<const T*>(a.kh), (int64_t)HD, static_cast<T*>(a.kp), HD, HD, HD, HD, a.Tp, a.T, 0, nblk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // the reversed problem of dg: reversed queries / keys, reversed u packed
  // with the forward's head padding
  const int64_t nr = M * HD;
  hipLaunchKernelGGL(reverse_rows_kernel<T>, dim3((unsigned)ceil_div(nr, 256)), dim3(256), 0, s,
                     static_cast<const T*>(a.qh), static_cast<T*>(a.q_rev), HD, a.Tp, a.T, M);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(reverse_rows_kernel<T>, dim3((unsigned)ceil_div(nr, 256)), dim3(256), 0, s,
                     static_cast<const T*>(a.kh), static_cast<T*>(a.k_rev), HD, a.Tp, a.T, M);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t nu = nblk * 4 * a.Fp;
  hipLaunchKernelGGL(pack_kernel<T>, dim3((unsigned)ceil_div(nu, 256)), dim3(256), 0, s,
                     static_cast<const T*>(a.u_rm), (int64_t)a.H * p.FhC, static_cast<T*>(a.u_rev_pk), a.Fp, a.Fhp,
                     p.FhC, a.Fh, a.Tp, a.T, 1, nblk);
  return hipGetLastError();
}

hipError_t launch_tango_dqk(const BwdArgs& a, const BwdPlan& p, hipStream_t s) {
  hipError_t e = launch_dqk<0>(a, p.rtiles, p.nchunk, p.items, s);
  if (e != hipSuccess) return e;
  return launch_dqk<1>(a, p.rtiles, p.nchunk, p.items, s);
}

hipError_t launch_tango_bwd_finish(const BwdArgs& a, const BwdPlan& p, hipStream_t s) {
  const int64_t n = (int64_t)a.B * a.Tp * a.H * a.dh;
  hipLaunchKernelGGL(bwd_finish_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, a, p.nchunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_scalars_kernel, dim3(a.H), dim3(256), 0, s, a, p.nchunk, p.half);
  return hipGetLastError();
}

}  // namespace tango
