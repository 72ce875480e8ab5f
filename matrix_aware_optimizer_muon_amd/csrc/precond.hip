// Newton-Muon right-preconditioner on gfx950 (Newton-Muon README, "What Is
// Newton-Muon?": each layer's gradient is right-multiplied by the inverse of
// the layer input's d x d second moment before the usual Muon step).
//
//   moment_kernel      S = X^T X / N + damping * I from N x d activations,
//                      or (accumulating form) Sigma <- beta Sigma + X^T X
//                      for one micro-batch; finalize_kernel then forms
//                      S = Sigma / N + damping * I from the running sums
//                      (bf16 MFMA with float32 accumulation for bf16
//                      activations, float32 MFMA for float32 ones); upper
//                      tiles, mirror-stored; the padded diagonal is set to 1
//                      so the padded matrix stays positive definite.
//   potrf / trsm / syrk_update    blocked right-looking Cholesky S = L L^T in
//                      float64 (64 x 64 blocks), with L^-1 formed alongside
//                      by blocked forward substitution of L X = I
//   sinv_store         S^-1 = L^-T L^-1 (summed in float64 during the
//                      factorisation), rounded to float32 and stored as three
//                      exact bf16 planes
//   apply_kernel       P = G S^-1 (block-wise for block-diagonal S), a float32
//                      product formed from exact bf16 planes on bf16 MFMA,
//                      read by the momentum phase in place of G.
#include "device_common.h"
#include "muon_internal.h"

namespace muon {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr int kThreads = 256;
constexpr int kCb = kCholBlock;   // Cholesky block edge (64)

__device__ __forceinline__ bf16x4_t lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
}

// ---------------------------------------------------------------- moment
// Tile of S for output rows [ti*BT, +BT) and columns [tj*BT, +BT): both
// operands are column blocks of the K-major activation slab (row r of X is
// one sample), so both are staged in natural [r][c] layout.
template <bool F32>
struct MomCfg;
template <> struct MomCfg<false> {
  using E = uint16_t;
  static constexpr int BT = 128, WT = 64, BK = 32, XPAD = 32;
};
template <> struct MomCfg<true> {
  using E = float;
  static constexpr int BT = 64, WT = 32, BK = 32, XPAD = 4;
};

// VEC: 16-byte aligned rows and d a multiple of a chunk (every chunk lies
// wholly inside or wholly outside the d columns).
template <bool F32, bool VEC>
__global__ __launch_bounds__(kThreads)
void moment_kernel(const void* __restrict__ acts, int64_t n_rows, int64_t ld, int d,
                   float* __restrict__ S, int dp, float inv_n, float damping, int accumulate, float beta,
                   float* __restrict__ part, int64_t split_rows) {
  using C = MomCfg<F32>;
  using E = typename C::E;
  constexpr int BT = C::BT, WT = C::WT, BK = C::BK;
  constexpr int LDX = BT + C::XPAD;
  constexpr int NB = WT / 32;
  constexpr int EPE = 16 / sizeof(E);
  constexpr int CPRX = BT / EPE;                 // 16-byte chunks per slab row
  constexpr int RPPX = kThreads / CPRX;
  constexpr int NPX = BK / RPPX;
  constexpr int TILE = BK * LDX;
  constexpr int EPP = WT + 8;
  static_assert(4 * 32 * EPP <= 2 * 2 * TILE * static_cast<int>(sizeof(E)) / 4, "epilogue staging");
  __shared__ __attribute__((aligned(16))) E smem[2 * 2 * TILE];   // [buf][operand][BK][LDX]

  // upper-triangle tile index -> (ti, tj)
  int ti = 0, rem = blockIdx.x;
  const int nt = dp / BT;
  while (rem >= nt - ti) { rem -= nt - ti; ++ti; }
  const int tj = ti + rem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int brow = tid / CPRX, bchunk = tid % CPRX;
  // sample rows of this block: all of them, or (split) range blockIdx.y
  const int64_t r_begin = static_cast<int64_t>(blockIdx.y) * split_rows;
  const int64_t r_end = r_begin + split_rows < n_rows ? r_begin + split_rows : n_rows;

  f32x16_t acc[NB][NB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // K pipeline: NR register sets of staged chunks (stage s in set s % NR)
  // and two LDS buffers.  Iteration kt requests stage kt+3, runs the MFMAs
  // of stage kt and stores stage kt+1 (requested two iterations earlier).
  // Every request is issued and stored (stage indices clamped, KT rounded
  // up to the unroll: stages past the rows are all zero), so the waits the
  // compiler places cover only the stage being stored.  A chunk outside the
  // tensor (rows past this block's range, columns past d) is loaded from a
  // clamped address and zeroed when it is stored.
  constexpr int NR = 4;
  const int ca = ti * BT + bchunk * EPE, cb = tj * BT + bchunk * EPE;   // this thread's columns
  const bool ca_ok = ca < d, cb_ok = cb < d;
  u32x4_t ra[NR][NPX], rb[NR][NPX];
  uint32_t rok[NR];                                  // bit q: row of chunk q inside the range
  auto load_chunk = [&](int64_t r, int c, bool ok) -> u32x4_t {
    if constexpr (VEC) {
      const int64_t rc = r < r_end ? r : r_end - 1;
      const size_t off = static_cast<size_t>(rc) * ld + (ok ? c : 0);
      return gld<u32x4_t>(static_cast<const E*>(acts) + off);
    } else {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (r >= r_end || !ok) return v;
      const size_t off = static_cast<size_t>(r) * ld + c;
      E tmp[EPE];
#pragma unroll
      for (int e = 0; e < EPE; ++e) tmp[e] = (c + e < d) ? gld<E>(static_cast<const E*>(acts) + off + e) : E(0);
      return __builtin_bit_cast(u32x4_t, tmp);
    }
  };
  const int KT0 = static_cast<int>((r_end - r_begin + BK - 1) / BK);
  const int KT = (KT0 + NR - 1) / NR * NR;
  auto gload = [&](int kt, u32x4_t (&a)[NPX], u32x4_t (&b)[NPX], uint32_t& ok) {
    ok = 0;
#pragma unroll
    for (int q = 0; q < NPX; ++q) {
      const int64_t r = r_begin + static_cast<int64_t>(kt) * BK + brow + q * RPPX;
      ok |= (r < r_end ? 1u : 0u) << q;
      a[q] = load_chunk(r, ca, ca_ok);
      b[q] = load_chunk(r, cb, cb_ok);
    }
  };
  auto sstore = [&](int buf, const u32x4_t (&a)[NPX], const u32x4_t (&b)[NPX], uint32_t ok) {
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < NPX; ++q) {
      const bool rq = (ok >> q) & 1u;
      *reinterpret_cast<u32x4_t*>(&smem[(buf * 2 + 0) * TILE + (brow + q * RPPX) * LDX + bchunk * EPE]) =
          rq && ca_ok ? a[q] : z;
      *reinterpret_cast<u32x4_t*>(&smem[(buf * 2 + 1) * TILE + (brow + q * RPPX) * LDX + bchunk * EPE]) =
          rq && cb_ok ? b[q] : z;
    }
  };

  gload(0, ra[0], rb[0], rok[0]);
  gload(min(1, KT - 1), ra[1], rb[1], rok[1]);
  gload(min(2, KT - 1), ra[2], rb[2], rok[2]);
  sstore(0, ra[0], rb[0], rok[0]);
  __syncthreads();
  for (int k4 = 0; k4 < KT; k4 += NR)
#pragma unroll
  for (int h = 0; h < NR; ++h) {
    const int kt = k4 + h, buf = h & 1;
    const E* la = smem + (buf * 2 + 0) * TILE;
    const E* lb = smem + (buf * 2 + 1) * TILE;
    gload(min(kt + 3, KT - 1), ra[(h + 3) % NR], rb[(h + 3) % NR], rok[(h + 3) % NR]);
    if constexpr (!F32) {
      const int g = lane >> 4, r = lane & 15;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int krow = ks * 16 + 8 * (g >> 1) + (r >> 2);
        bf16x8_t fa[NB], fb[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int col = wm * WT + i * 32 + 16 * (g & 1) + 4 * (r & 3);
          fa[i] = __builtin_shufflevector(lds_read_tr(&la[krow * LDX + col]),
                                          lds_read_tr(&la[(krow + 4) * LDX + col]), 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int col = wn * WT + j * 32 + 16 * (g & 1) + 4 * (r & 3);
          fb[j] = __builtin_shufflevector(lds_read_tr(&lb[krow * LDX + col]),
                                          lds_read_tr(&lb[(krow + 4) * LDX + col]), 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
    } else {
      const int k0 = (lane >> 5) * 16;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                la[(k0 + e) * LDX + wm * WT + i * 32 + (lane & 31)],
                lb[(k0 + e) * LDX + wn * WT + j * 32 + (lane & 31)], acc[i][j], 0, 0, 0);
      }
    }
    sstore(buf ^ 1, ra[(h + 1) % NR], rb[(h + 1) % NR], rok[(h + 1) % NR]);
    __syncthreads();
  }

  // epilogue: S = acc / N (+ damping on the diagonal; padded diagonal = 1),
  // or, accumulating, S = beta * S + acc (every element belongs to one
  // thread of one tile, so the read-modify-write needs no atomics)
  float* ep = reinterpret_cast<float*>(smem) + wave * (32 * EPP);
  const int row_base = ti * BT + wm * WT, col_base = tj * BT + wn * WT;
#pragma unroll
  for (int pi = 0; pi < NB; ++pi) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        ep[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * EPP + j * 32 + (lane & 31)] = acc[pi][j][r];
    __syncthreads();
    for (int s = lane; s < 32 * WT; s += 64) {
      const int row = s / WT, col = s % WT;
      const int gr = row_base + pi * 32 + row, gc = col_base + col;
      if (part) {   // split: raw partial sum of this row range, upper tile only
        part[static_cast<size_t>(blockIdx.y) * dp * dp + static_cast<size_t>(gr) * dp + gc] = ep[row * EPP + col];
        continue;
      }
      if (accumulate) {
        const float a = ep[row * EPP + col];
        const size_t o = static_cast<size_t>(gr) * dp + gc, om = static_cast<size_t>(gc) * dp + gr;
        S[o] = beta != 0.f ? fmaf(beta, S[o], a) : a;
        if (ti != tj) S[om] = beta != 0.f ? fmaf(beta, S[om], a) : a;
        continue;
      }
      float v = ep[row * EPP + col] * inv_n;
      if (gr == gc) v = gr < d ? v + damping : 1.0f;
      S[static_cast<size_t>(gr) * dp + gc] = v;
      if (ti != tj) S[static_cast<size_t>(gc) * dp + gr] = v;   // diagonal tiles hold both halves
    }
    __syncthreads();
  }
}

// Sum of the split partials (in split order, so the result does not depend
// on the schedule), then the same finish as the unsplit epilogue.  One block
// per 16-row quarter of a 64 x 64 sub-tile (a, b), a <= b, of the upper tile
// region: thread t adds the float4 at row t/16, columns 4(t%16).. over the
// splits; the mirror (b, a) is written through an LDS transpose so both
// stores are coalesced.  Diagonal sub-tiles keep their own values and have
// no mirror.
__global__ __launch_bounds__(kThreads)
void moment_reduce_kernel(const float* __restrict__ part, int splits, float* __restrict__ S, int d, int dp,
                          float inv_n, float damping, int accumulate, float beta) {
  __shared__ float T[16][65];
  const int quarter = blockIdx.x & 3;
  int a = 0, rem = blockIdx.x >> 2;
  const int ns = dp / 64;
  while (rem >= ns - a) { rem -= ns - a; ++a; }
  const int b = a + rem;
  const int c4 = (threadIdx.x & 15) * 4, row = threadIdx.x >> 4;
  const size_t slab = static_cast<size_t>(dp) * dp;
  const int gr = a * 64 + quarter * 16 + row;
  const size_t o = static_cast<size_t>(gr) * dp + b * 64 + c4;
  f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
  int sp = 0;
  for (; sp + 4 <= splits; sp += 4) {   // four loads in flight, added in split order
    const f32x4_t p0 = gld<f32x4_t>(part + (sp + 0) * slab + o), p1 = gld<f32x4_t>(part + (sp + 1) * slab + o);
    const f32x4_t p2 = gld<f32x4_t>(part + (sp + 2) * slab + o), p3 = gld<f32x4_t>(part + (sp + 3) * slab + o);
    sum += p0;
    sum += p1;
    sum += p2;
    sum += p3;
  }
  for (; sp < splits; ++sp) sum += gld<f32x4_t>(part + sp * slab + o);
  f32x4_t v;
  if (accumulate) {
    const f32x4_t old = gld<f32x4_t>(S + o);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = beta != 0.f ? fmaf(beta, old[e], sum[e]) : sum[e];
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int gc = b * 64 + c4 + e;
      v[e] = sum[e] * inv_n;
      if (gr == gc) v[e] = gr < d ? v[e] + damping : 1.0f;
    }
  }
  *reinterpret_cast<f32x4_t*>(S + o) = v;
  if (a == b) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) T[row][c4 + e] = v[e];
  __syncthreads();
  // mirror: 64 rows (columns of (a, b)) of 16 values; 4 threads per row
  const int mr = threadIdx.x >> 2, mc = (threadIdx.x & 3) * 4;
  f32x4_t m;
#pragma unroll
  for (int e = 0; e < 4; ++e) m[e] = T[mc + e][mr];
  *reinterpret_cast<f32x4_t*>(S + static_cast<size_t>(b * 64 + mr) * dp + a * 64 + quarter * 16 + mc) = m;
}

// ---------------------------------------------------------------- Cholesky
// 64 x 64 float64 block products from two LDS tiles (pitch kCb + 1): thread
// t owns the 4 x 4 register tile of rows 4*(t/16).., columns 4*(t%16).., so
// each K step reads 8 values for 16 multiply-adds.  TA: P is read as [m][i]
// (P^T), else [i][m]; TB: Q is read as [j][m] (Q^T), else [m][j].
template <bool TA, bool TB>
__device__ __forceinline__ void mm64_acc(const double (*P)[kCb + 1], const double (*Q)[kCb + 1],
                                         double (&c)[4][4]) {
  static_assert(kThreads == 256 && kCb == 64, "16 x 16 threads of 4 x 4 cover a 64 x 64 block");
  const int i0 = (threadIdx.x >> 4) * 4, j0 = (threadIdx.x & 15) * 4;
#pragma unroll 4
  for (int m = 0; m < kCb; ++m) {
    double a[4], b[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      a[r] = TA ? P[m][i0 + r] : P[i0 + r][m];
      b[r] = TB ? Q[j0 + r][m] : Q[m][j0 + r];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q) c[r][q] = fma(a[r], b[q], c[r][q]);
  }
}

__device__ __forceinline__ void zero44(double (&c)[4][4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) c[r][q] = 0.0;
}

// Load two 64 x 64 float64 blocks (leading dimension dp) into LDS tiles:
// all sixteen 16-byte loads of a thread are issued before the first LDS
// store, so the two blocks cost one memory latency, not sixteen.
typedef double f64x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void load_blocks(double (*P)[kCb + 1], const double* __restrict__ sp,
                                            double (*Q)[kCb + 1], const double* __restrict__ sq, int dp) {
  constexpr int kPer = kCb * kCb / 2 / kThreads;   // 16-byte pieces per thread and block
  f64x2_t vp[kPer], vq[kPer];
#pragma unroll
  for (int p = 0; p < kPer; ++p) {
    const int e = threadIdx.x + p * kThreads, row = e / (kCb / 2), col = (e % (kCb / 2)) * 2;
    vp[p] = gld<f64x2_t>(sp + row * static_cast<size_t>(dp) + col);
    vq[p] = gld<f64x2_t>(sq + row * static_cast<size_t>(dp) + col);
  }
#pragma unroll
  for (int p = 0; p < kPer; ++p) {
    const int e = threadIdx.x + p * kThreads, row = e / (kCb / 2), col = (e % (kCb / 2)) * 2;
    P[row][col] = vp[p][0];
    P[row][col + 1] = vp[p][1];
    Q[row][col] = vq[p][0];
    Q[row][col + 1] = vq[p][1];
  }
}

// Load one 64 x 64 float64 block (leading dimension dp) into an LDS tile,
// all of a thread's 16-byte loads issued before its first LDS store.
__device__ __forceinline__ void load_block(double (*P)[kCb + 1], const double* __restrict__ sp, int dp) {
  constexpr int kPer = kCb * kCb / 2 / kThreads;
  f64x2_t vp[kPer];
#pragma unroll
  for (int p = 0; p < kPer; ++p) {
    const int e = threadIdx.x + p * kThreads, row = e / (kCb / 2), col = (e % (kCb / 2)) * 2;
    vp[p] = gld<f64x2_t>(sp + row * static_cast<size_t>(dp) + col);
  }
#pragma unroll
  for (int p = 0; p < kPer; ++p) {
    const int e = threadIdx.x + p * kThreads, row = e / (kCb / 2), col = (e % (kCb / 2)) * 2;
    P[row][col] = vp[p][0];
    P[row][col + 1] = vp[p][1];
  }
}

// S (float32, dp x dp) -> L (float64, lower triangle; upper set to zero);
// L^-1's storage cleared (the right-hand side B of L X = I starts at zero off
// the diagonal blocks, which potrf_kernel writes) and so is the float64 sum
// that collects S^-1.
__global__ __launch_bounds__(kThreads) void to_f64_kernel(const float* __restrict__ S, double* __restrict__ L,
                                                          double* __restrict__ Li, double* __restrict__ sacc,
                                                          int dp) {
  const size_t n = static_cast<size_t>(dp) * dp;
  for (size_t k = blockIdx.x * static_cast<size_t>(kThreads) + threadIdx.x; k < n;
       k += static_cast<size_t>(gridDim.x) * kThreads) {
    const int i = static_cast<int>(k / dp), j = static_cast<int>(k % dp);
    L[k] = j <= i ? static_cast<double>(S[k]) : 0.0;
    Li[k] = 0.0;
    sacc[k] = 0.0;
  }
}

// The factor and L^-1 are built together, one 64-column block step jb at
// a time (right-looking):
//   potrf_kernel   D = L[jb][jb] and X[jb][jb] = D^-1
//   trsm_kernel    L[ib][jb] = A[ib][jb] D^-T            (ib > jb)
//                  X[jb][cb] = D^-1 B[jb][cb]            (cb < jb)
//   syrk_update    A[ib][kb] -= L[ib][jb] L[kb][jb]^T    (jb < kb <= ib)
//                  B[ib][cb] -= L[ib][jb] X[jb][cb]      (ib > jb, cb <= jb)
//                  Z[ib][cb] += X[jb][ib]^T X[jb][cb]    (ib <= cb <= jb)
// where X = L^-1 and B (held in the same storage, zero off the diagonal at
// the start) is the right-hand side of the block forward substitution
// L X = I: X[jb][cb] = D^-1 (I[jb][cb] - sum_{kb<jb} L[jb][kb] X[kb][cb]),
// each term subtracted at step kb once both of its factors are final.  Row
// jb of X is final after trsm_kernel of step jb, so the same launch also
// adds its term of S^-1 = L^-T L^-1 = sum_jb X[jb]^T X[jb] to the float64
// sum Z (upper blocks); a last launch adds the final row's term and
// sinv_store_kernel writes S^-1 (float32 values as bf16 planes).  The inverse and the product
// add blocks to launches the factorisation makes anyway.

// Diagonal block jb: factor in place and store D^-1 as X[jb][jb].
// Right-looking, with the block in registers: thread t holds the 4 x 4
// entries at rows 4(t/16).., columns 4(t%16).. of the trailing matrix (a)
// and of the running right-hand side of D X = I (x).  Two columns per
// barrier: the owners of columns k and k+1 publish them as they stand (k+1
// not yet reduced by k), and the owners of rows k and k+1 of x publish
// those rows (double-buffered in LDS).  Every thread then forms
//   l0_i = A[i][k] / sqrt(A[k][k]),
//   u_i  = A[i][k+1] - l0_i l0_{k+1}        (column k+1 reduced by column k),
//   l1_i = u_i / sqrt(u_{k+1}),
// (l0 zero for i <= k, l1 zero for i <= k+1, so the update leaves finished
// rows and columns alone), applies A[i][j] -= l0_i l0_j + l1_i l1_j and
// x[i][:] -= l0_i X[k][:] + l1_i X[k+1][:], with X[k][:] = x[k][:] / L[k][k]
// and X[k+1][:] = (x[k+1][:] - l0_{k+1} X[k][:]) / L[k+1][k+1] the finished
// rows of D^-1.  The step is a chain of latencies (LDS, barrier, rsqrt), so
// halving the barriers shortens the factor; the column loop is unrolled so
// register columns are static.  (One column per barrier with 4 x 4 tiles
// measured 29 us per block; with 2 x 2 tiles and 1024 threads, slower.)
// With P (an LDS tile) the block first applies the previous step's update
// to itself, A[jb][jb] -= L[jb][jb-1] L[jb][jb-1]^T (see step_kernel).
constexpr int kPotrfThreads = 256;
__device__ __forceinline__ void potrf_block(double* __restrict__ L, double* __restrict__ Li, int dp, int jb,
                                            uint32_t* __restrict__ flags, double (*P)[kCb + 1]) {
  static_assert(kPotrfThreads == kThreads && kPotrfThreads * 16 == kCb * kCb,
                "4 x 4 entries per thread cover the block");
  __shared__ double col0[2][kCb], col1[2][kCb];
  __shared__ double row0[2][kCb], row1[2][kCb];
  double* base = L + static_cast<size_t>(jb) * kCb * dp + jb * kCb;
  const int i0 = (threadIdx.x >> 4) * 4, j0 = (threadIdx.x & 15) * 4;
  double a[4][4], x[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[r][q] = base[(i0 + r) * static_cast<size_t>(dp) + j0 + q];
      x[r][q] = i0 + r == j0 + q ? 1.0 : 0.0;
    }
  if (P) {
    load_block(P, L + static_cast<size_t>(jb) * kCb * dp + (jb - 1) * kCb, dp);
    __syncthreads();
    double c[4][4];
    zero44(c);
    mm64_acc<false, true>(P, P, c);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q) a[r][q] -= c[r][q];
  }
  for (int k0 = 0; k0 < kCb; k0 += 4)
#pragma unroll
  for (int kq = 0; kq < 4; kq += 2) {
    const int k = k0 + kq, buf = (kq >> 1) & 1;
    if (j0 == k0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        col0[buf][i0 + r] = a[r][kq];
        col1[buf][i0 + r] = a[r][kq + 1];
      }
    }
    if (i0 == k0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        row0[buf][j0 + q] = x[kq][q];
        row1[buf][j0 + q] = x[kq + 1][q];
      }
    }
    __syncthreads();
    // a non-positive pivot gives NaN or inf, which propagates into S^-1,
    // and sets the flag
    const double p0 = col0[buf][k];
    const double rd0 = rsqrt(p0);
    const double l0k1 = col0[buf][k + 1] * rd0;          // L[k+1][k]
    const double p1 = col1[buf][k + 1] - l0k1 * l0k1;
    const double rd1 = rsqrt(p1);
    if (threadIdx.x == 0 && !(p0 > 0.0 && p1 > 0.0)) atomicOr(flags, 2u);
    double c0i[4], c0j[4], u_i[4], u_j[4], xk0[4], xk1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      c0i[r] = col0[buf][i0 + r] * rd0;
      c0j[r] = col0[buf][j0 + r] * rd0;
      u_i[r] = fma(-c0i[r], l0k1, col1[buf][i0 + r]);
      u_j[r] = fma(-c0j[r], l0k1, col1[buf][j0 + r]);
      xk0[r] = row0[buf][j0 + r] * rd0;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) xk1[r] = fma(-l0k1, xk0[r], row1[buf][j0 + r]) * rd1;
    if (i0 + 3 > k) {
      double li0[4], lj0[4], li1[4], lj1[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        li0[r] = i0 + r > k ? c0i[r] : 0.0;
        lj0[r] = j0 + r > k ? c0j[r] : 0.0;
        li1[r] = i0 + r > k + 1 ? u_i[r] * rd1 : 0.0;
        lj1[r] = j0 + r > k + 1 ? u_j[r] * rd1 : 0.0;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          a[r][q] = fma(-li1[r], lj1[q], fma(-li0[r], lj0[q], a[r][q]));
          x[r][q] = fma(-li1[r], xk1[q], fma(-li0[r], xk0[q], x[r][q]));
        }
    }
    if (j0 == k0) {   // columns k and k+1 of L (L[k][k] = p0 rd0, L[k+1][k+1] = p1 rd1)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        a[r][kq] = c0i[r];
        a[r][kq + 1] = u_i[r] * rd1;
      }
    }
    if (i0 == k0) {   // rows k and k+1 of D^-1
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        x[kq][q] = xk0[q];
        x[kq + 1][q] = xk1[q];
      }
    }
  }
  double* di = Li + static_cast<size_t>(jb) * kCb * dp + jb * kCb;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      base[(i0 + r) * static_cast<size_t>(dp) + j0 + q] = j0 + q <= i0 + r ? a[r][q] : 0.0;
      di[(i0 + r) * static_cast<size_t>(dp) + j0 + q] = x[r][q];
    }
}

// The first diagonal block (no previous step).
__global__ __launch_bounds__(kPotrfThreads) void potrf_kernel(double* __restrict__ L, double* __restrict__ Li, int dp,
                                                              uint32_t* __restrict__ flags) {
  potrf_block(L, Li, dp, 0, flags, nullptr);
}


// Step jb, after potrf_kernel: blocks [0, below) form the panel
// L[ib][jb] = A[ib][jb] D^-T (ib = jb + 1 + block); blocks [below, below + jb)
// finish row jb of L^-1 left of the diagonal, X[jb][cb] = D^-1 B[jb][cb].
__global__ __launch_bounds__(kThreads) void trsm_kernel(double* __restrict__ L, double* __restrict__ Li, int dp,
                                                        int jb, int below) {
  __shared__ double P[kCb][kCb + 1];
  __shared__ double Q[kCb][kCb + 1];
  const double* dinv = Li + static_cast<size_t>(jb) * kCb * dp + jb * kCb;
  const bool panel = static_cast<int>(blockIdx.x) < below;
  double* out = panel ? L + static_cast<size_t>(jb + 1 + blockIdx.x) * kCb * dp + jb * kCb
                      : Li + static_cast<size_t>(jb) * kCb * dp + (blockIdx.x - below) * kCb;
  double c[4][4];
  zero44(c);
  if (panel) {
    load_blocks(P, out, Q, dinv, dp);
    __syncthreads();
    mm64_acc<false, true>(P, Q, c);   // sum_m A[i][m] D^-1[j][m]
  } else {
    load_blocks(P, dinv, Q, out, dp);
    __syncthreads();
    mm64_acc<false, false>(P, Q, c);  // sum_m D^-1[i][m] B[m][j]
  }
  const int i0 = (threadIdx.x >> 4) * 4, j0 = (threadIdx.x & 15) * 4;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) out[(i0 + r) * static_cast<size_t>(dp) + j0 + q] = c[r][q];
}

// Step jb, after trsm_kernel: blocks [0, npairs) update the trailing matrix,
// A[ib][kb] -= L[ib][jb] L[kb][jb]^T for jb < kb <= ib; the next nrhs update
// the right-hand side of L X = I, B[ib][cb] -= L[ib][jb] X[jb][cb] for
// ib > jb, cb <= jb; the rest add row jb's term of S^-1,
// Z[ib][cb] += X[jb][ib]^T X[jb][cb] for ib <= cb <= jb.
__device__ __forceinline__ void syrk_task(double* __restrict__ L, double* __restrict__ Li, double* __restrict__ sacc,
                                          int dp, int jb, int npairs, int nrhs, int task, double (*P)[kCb + 1],
                                          double (*Q)[kCb + 1]) {
  double* out;
  double c[4][4];
  zero44(c);
  const int i0 = (threadIdx.x >> 4) * 4, j0 = (threadIdx.x & 15) * 4;
  if (task >= npairs + nrhs) {
    int ib = 0, rem = task - npairs - nrhs;   // upper pair index over 0..jb -> (ib, cb)
    while (rem >= jb + 1 - ib) { rem -= jb + 1 - ib; ++ib; }
    const int cb = ib + rem;
    load_blocks(P, Li + static_cast<size_t>(jb) * kCb * dp + ib * kCb, Q, Li + static_cast<size_t>(jb) * kCb * dp + cb * kCb,
                dp);
    out = sacc + static_cast<size_t>(ib) * kCb * dp + cb * kCb;
    __syncthreads();
    mm64_acc<true, false>(P, Q, c);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q) out[(i0 + r) * static_cast<size_t>(dp) + j0 + q] += c[r][q];
    return;
  }
  if (task < npairs) {
    int ib = jb + 1, rem = task;   // lower-triangle pair index -> (ib, kb); pair 0 is (jb+1, jb+1)
    while (rem >= ib - jb) { rem -= ib - jb; ++ib; }
    const int kb = jb + 1 + rem;
    load_blocks(P, L + static_cast<size_t>(ib) * kCb * dp + jb * kCb, Q, L + static_cast<size_t>(kb) * kCb * dp + jb * kCb,
                dp);
    out = L + static_cast<size_t>(ib) * kCb * dp + kb * kCb;
    __syncthreads();
    mm64_acc<false, true>(P, Q, c);
  } else {
    const int idx = task - npairs;
    const int ib = jb + 1 + idx / (jb + 1), cb = idx % (jb + 1);
    load_blocks(P, L + static_cast<size_t>(ib) * kCb * dp + jb * kCb, Q, Li + static_cast<size_t>(jb) * kCb * dp + cb * kCb,
                dp);
    out = Li + static_cast<size_t>(ib) * kCb * dp + cb * kCb;
    __syncthreads();
    mm64_acc<false, false>(P, Q, c);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) out[(i0 + r) * static_cast<size_t>(dp) + j0 + q] -= c[r][q];
}

__global__ __launch_bounds__(kThreads) void syrk_update_kernel(double* __restrict__ L, double* __restrict__ Li,
                                                               double* __restrict__ sacc, int dp, int jb, int npairs,
                                                               int nrhs) {
  __shared__ double P[kCb][kCb + 1];
  __shared__ double Q[kCb][kCb + 1];
  syrk_task(L, Li, sacc, dp, jb, npairs, nrhs, blockIdx.x, P, Q);
}

// Step jb's first launch: block 0 factors diagonal block jb after applying
// the previous step's update to it (pair 0 of that step's updates); blocks
// 1.. run the previous step's other updates (trailing matrix, right-hand
// side, S^-1 term), which the factor does not read, beside it.  So the
// update launch leaves the chain of dependent launches: two per step.
__global__ __launch_bounds__(kThreads) void step_kernel(double* __restrict__ L, double* __restrict__ Li,
                                                        double* __restrict__ sacc, int dp, int jb, int npairs,
                                                        int nrhs, uint32_t* __restrict__ flags) {
  __shared__ double P[kCb][kCb + 1];
  __shared__ double Q[kCb][kCb + 1];
  if (blockIdx.x == 0) potrf_block(L, Li, dp, jb, flags, P);
  else syrk_task(L, Li, sacc, dp, jb - 1, npairs, nrhs, blockIdx.x, P, Q);
}

// S^-1 from the float64 sum Z, which holds the upper blocks (ib <= jb); a
// lower block is the transpose of its mirror, staged through LDS so that
// reads and writes are both along rows.  Each value is rounded to float32
// and stored as its three bf16 planes.  One block per 64 x 64 block of S^-1,
// 16 rows per pass.
__device__ __forceinline__ void store_planes(uint16_t* sinv, size_t plane, size_t idx, double z) {
  const float x = static_cast<float>(z);
  const uint16_t h = f32_to_bf16(x);
  const float r = x - bf16_to_f32(h);               // exact
  const uint16_t m = f32_to_bf16(r);
  const uint16_t l = f32_to_bf16(r - bf16_to_f32(m));   // exact: at most 8 significant bits
  sinv[idx] = h;
  sinv[plane + idx] = m;
  sinv[2 * plane + idx] = l;
}

__global__ __launch_bounds__(kThreads) void sinv_store_kernel(const double* __restrict__ sacc,
                                                              uint16_t* __restrict__ Sinv, int dp) {
  __shared__ double T[16][kCb + 1];
  const int nb = dp / kCb;
  const size_t plane = static_cast<size_t>(dp) * dp;
  const int ib = blockIdx.x / nb, jb = blockIdx.x % nb;
  const int c = threadIdx.x & 63, r = threadIdx.x >> 6;
  for (int p = 0; p < kCb; p += 16) {
    if (ib <= jb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = p + r + 4 * q;
        const size_t idx = static_cast<size_t>(ib * kCb + row) * dp + jb * kCb + c;
        store_planes(Sinv, plane, idx, sacc[idx]);
      }
      continue;
    }
    // rows p..p+15 of lower block (ib, jb) = columns p..p+15 of Z[jb][ib]
    __syncthreads();
    for (int s = threadIdx.x; s < 16 * kCb; s += kThreads) {
      const int zr = s >> 4, zc = s & 15;   // row of Z[jb][ib], column p + zc
      T[zc][zr] = sacc[static_cast<size_t>(jb * kCb + zr) * dp + ib * kCb + p + zc];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = r + 4 * q;
      store_planes(Sinv, plane, static_cast<size_t>(ib * kCb + p + row) * dp + jb * kCb + c, T[row][c]);
    }
  }
}

// ---------------------------------------------------------------- apply
// P[i][k*d + j] = sum_c G[i][k*d + c] * Sinv_k[j][c]   (S^-1 is symmetric,
// so its rows are the K-contiguous operand).  The float32 product is formed
// on bf16 matrix cores: while a tile is staged, each float32 value x is
// split into three bf16 planes, x = h + m + l exactly (h = bf16(x),
// m = bf16(x - h), l = x - h - m, which has at most 8 significant bits), and
// the tile product sums the plane products i + j <= 2 with float32
// accumulation (bf16 products are exact in float32).  S^-1 arrives as its
// planes (the refresh stores them), so its tiles are staged as raw bits; a
// float32 gradient is split while staged.  A bf16 gradient is its own single
// plane, so P = G (h + m + l) is the float32 GEMM up to the order
// of the additions; a float32 gradient drops only the products of two small
// planes (each below 2^-16 of the leading one).  Output tiles of 128 rows
// of G by 64 columns (S^-1 rows), 4 waves of 64x32 (two 32x32 blocks of
// v_mfma_f32_32x32x16_bf16 sharing each S^-1 fragment), 32-deep K stages
// double-buffered in LDS with a padded row pitch (conflict-free 16-byte
// fragment reads).
constexpr int kApRows = 128, kApCols = 64, kApBK = 32, kApLDK = kApBK + 8;
constexpr int kApGPlane = kApRows * kApLDK;          // bf16 elements per gradient plane
constexpr int kApSPlane = kApCols * kApLDK;          // ... per S^-1 plane
// two stages of the gradient's planes (1 for bf16, 3 for float32) and S^-1's 3
template <bool GF32>
constexpr int ap_smem() { return 2 * ((GF32 ? 3 : 1) * kApGPlane + kSinvPlanes * kApSPlane); }

template <bool GF32, bool VEC>
__device__ __forceinline__ void apply_tile(const PrecondDev& pd, const ApplyTask& t, uint16_t* smem) {
  constexpr int WR = 64, WC = 32, MB = WR / 32, BK = kApBK, LDK = kApLDK, EPP = WC + 8;
  constexpr int NG = GF32 ? 3 : 1;                 // planes of the gradient tile
  constexpr int GPLANE = kApGPlane, SPLANE = kApSPlane;
  constexpr int STAGE = NG * GPLANE + kSinvPlanes * SPLANE;
  constexpr int GQ = kApRows / 64;                 // gradient chunks per thread and stage
  static_assert(2 * STAGE <= ap_smem<GF32>(), "stages fit");
  static_assert(4 * 32 * EPP * 4 <= 2 * STAGE * 2, "epilogue staging");
  const int d = pd.d, dp = pd.dp;
  const int r0 = t.tr * kApRows, c0 = t.tc * kApCols;   // rows of G, columns within block t.blk
  const int gcol0 = t.blk * d;                          // first column of the block in G and P
  const size_t splane = static_cast<size_t>(dp) * dp;
  const uint16_t* sinv = pd.sinv + static_cast<size_t>(t.blk) * kSinvPlanes * splane;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = tid >> 2, lk = (tid & 3) * 8;        // 64 rows x 4 chunks of 8 per pass

  f32x16_t acc[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;

  // NR register sets of staged operands (stage kt+s in set (kt+s) % NR),
  // used with static indices: the loop is unrolled by NR.
  // The gradient is staged as raw bits (8 bf16, or 8 float32 in two words
  // of four) and decoded only when the tile is stored, so no wait follows
  // a load.  Aligned rows (VEC) take a branch-free path: the address is clamped
  // into the tensor and a chunk outside it (rows past the end, columns past
  // d, which is a multiple of 8 there) is zeroed at decode time.
  constexpr int GW = GF32 ? 2 : 1;
  constexpr int NR = 4;
  u32x4_t gr[NR][GQ][GW];
  bool gok[NR][GQ];
  u32x4_t sb[NR][kSinvPlanes];
  // one chunk of the gradient: row r0+lrow+64q, 8 columns from kc
  auto gchunk = [&](int q, int kc, u32x4_t (&g)[GW], bool& ok) {
    const int gi = r0 + lrow + 64 * q;
    ok = gi < pd.rows && kc < d;
    if constexpr (VEC) {
      const int gic = gi < pd.rows ? gi : pd.rows - 1, kcc = kc < d ? kc : 0;
      const size_t off = static_cast<size_t>(gic) * pd.ld_grad + gcol0 + kcc;
      if constexpr (GF32) {
        g[0] = gld<u32x4_t>(static_cast<const float*>(pd.grad) + off);
        g[1] = gld<u32x4_t>(static_cast<const float*>(pd.grad) + off + 4);
      } else {
        g[0] = gld<u32x4_t>(static_cast<const uint16_t*>(pd.grad) + off);
      }
    } else {   // unaligned rows: element loads, packed into the same raw layout
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
      if (gi < pd.rows) {
        const size_t off = static_cast<size_t>(gi) * pd.ld_grad + gcol0 + kc;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (kc + e < d)
            v[e] = GF32 ? gld<float>(static_cast<const float*>(pd.grad) + off + e)
                        : bf16_to_f32(gld<uint16_t>(static_cast<const uint16_t*>(pd.grad) + off + e));
      }
      if constexpr (GF32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          g[0][e] = __float_as_uint(v[e]);
          g[1][e] = __float_as_uint(v[4 + e]);
        }
      } else {
        g[0] = pack8_bf16(v);   // exact: the values are bf16
      }
      ok = true;
    }
  };
  auto gload = [&](int k0, u32x4_t (&g)[GQ][GW], bool (&ok)[GQ], u32x4_t (&sv)[kSinvPlanes]) {
#pragma unroll
    for (int q = 0; q < GQ; ++q) gchunk(q, k0 + lk, g[q], ok[q]);
    // operand B: row c0+lrow of the S^-1 planes (padded to dp, always in bounds)
    const uint16_t* sp = sinv + static_cast<size_t>(c0 + lrow) * dp + k0 + lk;
#pragma unroll
    for (int pl = 0; pl < kSinvPlanes; ++pl) sv[pl] = gld<u32x4_t>(sp + pl * splane);
  };
  // split 8 floats into bf16 planes h, m, l and store them (16 bytes each)
  auto split_store = [&](const float* x, int nplanes, uint16_t* dst) {
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = x[e];
#pragma unroll
    for (int pl = 0; pl < 3; ++pl) {
      if (pl >= nplanes) break;
      u32x4_t w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = cvt2_bf16(r[2 * e], r[2 * e + 1]);
      *reinterpret_cast<u32x4_t*>(dst + pl * GPLANE) = w;
      if (pl + 1 < nplanes) {
        float hv[8];
        unpack8_bf16(w, hv);
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] -= hv[e];   // exact: the residual of a round-to-nearest
      }
    }
  };
  auto sstore = [&](int buf, const u32x4_t (&g)[GQ][GW], const bool (&ok)[GQ],
                    const u32x4_t (&sv)[kSinvPlanes]) {
    uint16_t* st = smem + buf * STAGE;
#pragma unroll
    for (int q = 0; q < GQ; ++q) {
      uint16_t* gs = st + (lrow + 64 * q) * LDK + lk;
      if constexpr (GF32) {
        float gv[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gv[e] = ok[q] ? __uint_as_float(g[q][0][e]) : 0.f;
          gv[4 + e] = ok[q] ? __uint_as_float(g[q][1][e]) : 0.f;
        }
        split_store(gv, NG, gs);
      } else {
        const u32x4_t z = {0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4_t*>(gs) = ok[q] ? g[q][0] : z;   // bf16: its own plane
      }
    }
    uint16_t* ss = st + NG * GPLANE + lrow * LDK + lk;
#pragma unroll
    for (int pl = 0; pl < kSinvPlanes; ++pl) *reinterpret_cast<u32x4_t*>(ss + pl * SPLANE) = sv[pl];
  };
  // K pipeline: LDS buffer kt&1 holds stage kt; iteration kt requests
  // stage kt+3 (into the set stage kt-1 left, stored two iterations ago),
  // runs the MFMAs of stage kt, then stores stage kt+1, requested two
  // iterations earlier, so a full iteration separates each load from its
  // use.  Stage indices past the end are clamped to the last stage and every
  // request is stored (the copies land in a buffer nobody reads again), so
  // on every path each set's loads are consumed before the set is reloaded
  // and the compiler's waits cover only the stage being stored.
  const int KT = dp / BK;                          // a multiple of 4 (dp is of 128)
  static_assert(NR == 4, "KT is a multiple of the unroll");
  gload(0, gr[0], gok[0], sb[0]);
  gload(BK, gr[1], gok[1], sb[1]);
  gload(2 * BK, gr[2], gok[2], sb[2]);
  sstore(0, gr[0], gok[0], sb[0]);
  __syncthreads();
  for (int k4 = 0; k4 < KT; k4 += NR)
#pragma unroll
  for (int h = 0; h < NR; ++h) {
    const int kt = k4 + h, buf = h & 1;
    gload(min(kt + 3, KT - 1) * BK, gr[(h + 3) % NR], gok[(h + 3) % NR], sb[(h + 3) % NR]);
    const uint16_t* st = smem + buf * STAGE;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kk = ks * 16 + 8 * (lane >> 5);
      bf16x8_t fa[MB][NG], fb[3];
#pragma unroll
      for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int pl = 0; pl < NG; ++pl)
          fa[b][pl] = *reinterpret_cast<const bf16x8_t*>(st + pl * GPLANE + (wm * WR + b * 32 + (lane & 31)) * LDK + kk);
#pragma unroll
      for (int pl = 0; pl < 3; ++pl)
        fb[pl] = *reinterpret_cast<const bf16x8_t*>(st + NG * GPLANE + pl * SPLANE + (wn * WC + (lane & 31)) * LDK + kk);
      // small products first
#pragma unroll
      for (int sum = 2; sum >= 0; --sum)
#pragma unroll
        for (int i = 0; i < NG; ++i) {
          const int j = sum - i;
          if (j >= 0 && j < 3) {
#pragma unroll
            for (int b = 0; b < MB; ++b) acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[b][i], fb[j], acc[b], 0, 0, 0);
          }
        }
    }
    sstore(buf ^ 1, gr[(h + 1) % NR], gok[(h + 1) % NR], sb[(h + 1) % NR]);
    __syncthreads();
  }
  // epilogue through LDS (each wave its own area): row segments of P, one
  // 32-row block at a time
  float* ep = reinterpret_cast<float*>(smem) + wave * (32 * EPP);
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    if (b > 0) __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) ep[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * EPP + (lane & 31)] = acc[b][r];
    __syncthreads();
    for (int s = lane; s < 32 * WC; s += 64) {
      const int row = s / WC, col = s % WC;
      const int gi = r0 + wm * WR + b * 32 + row, cj = c0 + wn * WC + col;
      if (gi < pd.rows && cj < d) pd.p[static_cast<size_t>(gi) * pd.ld_p + gcol0 + cj] = ep[row * EPP + col];
    }
  }
}

// One launch per gradient dtype, with the LDS its planes need (bf16: 50 KB,
// three blocks per CU; float32: 90 KB, one).
template <bool GF32>
__global__ __launch_bounds__(kThreads)
void apply_kernel(const PrecondDev* __restrict__ pds, const ApplyTask* __restrict__ tasks) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[ap_smem<GF32>()];   // [buf][G planes, S planes][BT][LDK]
  const ApplyTask t = tasks[blockIdx.x];
  const PrecondDev& pd = pds[t.tensor];
  if (pd.vec_grad) apply_tile<GF32, true>(pd, t, smem);   // uniform over the block
  else apply_tile<GF32, false>(pd, t, smem);
}

// S^-1 = I for every block (the state of a slot before its first refresh).
// Running sample count of an accumulating block: N <- beta N + n_rows.
__global__ void count_kernel(double* cnt, float beta, int64_t n_rows) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *cnt = static_cast<double>(beta) * *cnt + static_cast<double>(n_rows);
}

// S = Sigma / N + damping * I (padded diagonal 1); a block with no samples
// gives S = damping * I.
__global__ __launch_bounds__(kThreads) void finalize_kernel(const float* __restrict__ acc, const double* cnt,
                                                            float* __restrict__ S, int d, int dp, float damping) {
  const double n = *cnt;
  const float inv_n = n > 0.0 ? static_cast<float>(1.0 / n) : 0.f;
  const size_t total = static_cast<size_t>(dp) * dp;
  for (size_t k = blockIdx.x * static_cast<size_t>(kThreads) + threadIdx.x; k < total;
       k += static_cast<size_t>(gridDim.x) * kThreads) {
    const int i = static_cast<int>(k / dp), j = static_cast<int>(k % dp);
    float v = acc[k] * inv_n;
    if (i == j) v = i < d ? v + damping : 1.0f;
    S[k] = v;
  }
}

// Clears a block's running sum and count.
__global__ __launch_bounds__(kThreads) void clear_acc_kernel(float* __restrict__ acc, double* cnt, int dp) {
  const size_t total = static_cast<size_t>(dp) * dp;
  for (size_t k = blockIdx.x * static_cast<size_t>(kThreads) + threadIdx.x; k < total;
       k += static_cast<size_t>(gridDim.x) * kThreads)
    acc[k] = 0.f;
  if (blockIdx.x == 0 && threadIdx.x == 0) *cnt = 0.0;
}

__global__ __launch_bounds__(kThreads) void identity_kernel(uint16_t* __restrict__ sinv, int dp, int nblocks) {
  const size_t plane = static_cast<size_t>(dp) * dp;
  const size_t n = static_cast<size_t>(nblocks) * kSinvPlanes * plane;
  for (size_t k = blockIdx.x * static_cast<size_t>(kThreads) + threadIdx.x; k < n;
       k += static_cast<size_t>(gridDim.x) * kThreads) {
    const size_t e = k % plane;
    const bool lead = (k / plane) % kSinvPlanes == 0;   // h plane: 1 on the diagonal; m, l: 0
    sinv[k] = lead && e / dp == e % dp ? static_cast<uint16_t>(0x3F80u) : static_cast<uint16_t>(0u);
  }
}

}  // namespace

hipError_t launch_identity(uint16_t* sinv, int dp, int nblocks, hipStream_t s) {
  identity_kernel<<<256, kThreads, 0, s>>>(sinv, dp, nblocks);
  return hipGetLastError();
}

namespace {

// X^T X of one activation batch into `out`: normalised (inv_n, damping) or
// accumulated (out = beta * out + X^T X).
void launch_moment(const PrecondBlockDev& b, const void* acts, int64_t n_rows, int64_t ld, bool acts_f32, float* out,
                   float inv_n, float damping, int accumulate, float beta, hipStream_t s) {
  const int d = b.d, dp = b.dp;
  const size_t es = acts_f32 ? 4 : 2;
  const bool vec = (reinterpret_cast<uintptr_t>(acts) % 16 == 0) && ((ld * es) % 16 == 0) && (d * es) % 16 == 0;
  const int splits = b.part ? moment_splits(dp, acts_f32, n_rows) : 1;
  const int bk = acts_f32 ? MomCfg<true>::BK : MomCfg<false>::BK;
  const int64_t per = splits > 1 ? ((n_rows + splits - 1) / splits + bk - 1) / bk * bk : n_rows;
  const int used = static_cast<int>((n_rows + per - 1) / per);   // splits that hold rows
  float* part = used > 1 ? b.part : nullptr;
  const int nt = dp / (acts_f32 ? MomCfg<true>::BT : MomCfg<false>::BT);
  const dim3 grid(nt * (nt + 1) / 2, used);
  if (acts_f32) {
    if (vec)
      moment_kernel<true, true><<<grid, kThreads, 0, s>>>(acts, n_rows, ld, d, out, dp, inv_n, damping, accumulate,
                                                          beta, part, per);
    else
      moment_kernel<true, false><<<grid, kThreads, 0, s>>>(acts, n_rows, ld, d, out, dp, inv_n, damping, accumulate,
                                                           beta, part, per);
  } else {
    if (vec)
      moment_kernel<false, true><<<grid, kThreads, 0, s>>>(acts, n_rows, ld, d, out, dp, inv_n, damping, accumulate,
                                                           beta, part, per);
    else
      moment_kernel<false, false><<<grid, kThreads, 0, s>>>(acts, n_rows, ld, d, out, dp, inv_n, damping,
                                                            accumulate, beta, part, per);
  }
  if (part) {
    const int ns = dp / 64;
    moment_reduce_kernel<<<4 * (ns * (ns + 1) / 2), kThreads, 0, s>>>(part, used, out, d, dp, inv_n, damping, accumulate,
                                                                beta);
  }
}

// S (in b.s) -> float64 Cholesky factor -> its inverse -> S^-1 (float32).
void factor_and_invert(const PrecondBlockDev& b, uint32_t* flags, hipStream_t s) {
  const int dp = b.dp, nb = dp / kCb;
  double* sacc = reinterpret_cast<double*>(b.part);   // the scratch holds dp x dp float64
  to_f64_kernel<<<256, kThreads, 0, s>>>(b.s, b.l, b.li, sacc, dp);
  // update counts of step j: trailing pairs, right-hand-side blocks, S^-1 terms
  auto counts = [nb](int j, int& npairs, int& nrhs, int& nz) {
    const int below = nb - j - 1;
    npairs = below * (below + 1) / 2;
    nrhs = below * (j + 1);
    nz = (j + 1) * (j + 2) / 2;
  };
  for (int jb = 0; jb < nb; ++jb) {
    if (jb == 0) {
      potrf_kernel<<<1, kPotrfThreads, 0, s>>>(b.l, b.li, dp, flags);
    } else {
      int npairs, nrhs, nz;
      counts(jb - 1, npairs, nrhs, nz);   // npairs >= 1: pair 0, block (jb, jb), is the factor's own
      step_kernel<<<npairs + nrhs + nz, kThreads, 0, s>>>(b.l, b.li, sacc, dp, jb, npairs, nrhs, flags);
    }
    const int below = nb - jb - 1;
    if (below + jb > 0) trsm_kernel<<<below + jb, kThreads, 0, s>>>(b.l, b.li, dp, jb, below);
  }
  {
    int npairs, nrhs, nz;
    counts(nb - 1, npairs, nrhs, nz);     // the last step: its S^-1 term only
    syrk_update_kernel<<<npairs + nrhs + nz, kThreads, 0, s>>>(b.l, b.li, sacc, dp, nb - 1, npairs, nrhs);
  }
  sinv_store_kernel<<<nb * nb, kThreads, 0, s>>>(sacc, b.sinv, dp);
}

}  // namespace

hipError_t launch_precond_refresh(const PrecondBlockDev& b, const void* acts, int64_t n_rows, int64_t ld,
                                  bool acts_f32, float damping, uint32_t* flags, hipStream_t s) {
  const float inv_n = static_cast<float>(1.0 / static_cast<double>(n_rows));
  launch_moment(b, acts, n_rows, ld, acts_f32, b.s, inv_n, damping, 0, 0.f, s);
  factor_and_invert(b, flags, s);
  return hipGetLastError();
}

hipError_t launch_precond_accumulate(const PrecondBlockDev& b, const void* acts, int64_t n_rows, int64_t ld,
                                     bool acts_f32, float beta, hipStream_t s) {
  launch_moment(b, acts, n_rows, ld, acts_f32, b.acc, 0.f, 0.f, 1, beta, s);
  count_kernel<<<1, 64, 0, s>>>(b.cnt, beta, n_rows);
  return hipGetLastError();
}

hipError_t launch_precond_refresh_accumulated(const PrecondBlockDev& b, float damping, bool reset, uint32_t* flags,
                                              hipStream_t s) {
  finalize_kernel<<<256, kThreads, 0, s>>>(b.acc, b.cnt, b.s, b.d, b.dp, damping);
  factor_and_invert(b, flags, s);
  if (reset) clear_acc_kernel<<<256, kThreads, 0, s>>>(b.acc, b.cnt, b.dp);
  return hipGetLastError();
}

hipError_t launch_precond_apply(const PrecondDev* pds, const ApplyTask* tasks, int n_bf16, int n_f32, hipStream_t s) {
  if (n_bf16 > 0) apply_kernel<false><<<n_bf16, kThreads, 0, s>>>(pds, tasks);
  if (n_f32 > 0) apply_kernel<true><<<n_f32, kThreads, 0, s>>>(pds, tasks + n_bf16);
  return hipGetLastError();
}

}  // namespace muon
