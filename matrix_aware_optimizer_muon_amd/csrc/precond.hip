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
//                      float64 (64 x 64 blocks)
//   trinv_diag / trinv_offdiag    L^-1, blocked forward substitution
//   inv_product        S^-1 = L^-T L^-1, stored as float32
//   apply_kernel       P = G S^-1 (block-wise for block-diagonal S), float32
//                      MFMA, read by the momentum phase in place of G.
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

template <bool F32>
__global__ __launch_bounds__(kThreads)
void moment_kernel(const void* __restrict__ acts, int64_t n_rows, int64_t ld, int d, int vec,
                   float* __restrict__ S, int dp, float inv_n, float damping, int accumulate, float beta) {
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

  f32x16_t acc[NB][NB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // load one chunk (EPE elements) of the slab, zero outside the tensor
  auto load_chunk = [&](int64_t r, int c) -> u32x4_t {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (r >= n_rows || c >= d) return v;
    const size_t off = static_cast<size_t>(r) * ld + c;
    if (vec && c + EPE <= d) return gld<u32x4_t>(static_cast<const E*>(acts) + off);
    E tmp[EPE];
#pragma unroll
    for (int e = 0; e < EPE; ++e) tmp[e] = (c + e < d) ? gld<E>(static_cast<const E*>(acts) + off + e) : E(0);
    return __builtin_bit_cast(u32x4_t, tmp);
  };

  u32x4_t ra[NPX], rb[NPX];
  const int KT = static_cast<int>((n_rows + BK - 1) / BK);
  auto gload = [&](int kt) {
#pragma unroll
    for (int q = 0; q < NPX; ++q) {
      const int64_t r = static_cast<int64_t>(kt) * BK + brow + q * RPPX;
      ra[q] = load_chunk(r, ti * BT + bchunk * EPE);
      rb[q] = load_chunk(r, tj * BT + bchunk * EPE);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < NPX; ++q) {
      *reinterpret_cast<u32x4_t*>(&smem[(buf * 2 + 0) * TILE + (brow + q * RPPX) * LDX + bchunk * EPE]) = ra[q];
      *reinterpret_cast<u32x4_t*>(&smem[(buf * 2 + 1) * TILE + (brow + q * RPPX) * LDX + bchunk * EPE]) = rb[q];
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    const E* la = smem + (buf * 2 + 0) * TILE;
    const E* lb = smem + (buf * 2 + 1) * TILE;
    const bool more = kt + 1 < KT;
    if (more) gload(kt + 1);
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
    if (more) sstore(buf ^ 1);
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

// ---------------------------------------------------------------- Cholesky
// S (float32, dp x dp) -> L (float64, lower triangle; upper set to zero).
__global__ __launch_bounds__(kThreads) void to_f64_kernel(const float* __restrict__ S, double* __restrict__ L,
                                                          int dp) {
  const size_t n = static_cast<size_t>(dp) * dp;
  for (size_t k = blockIdx.x * static_cast<size_t>(kThreads) + threadIdx.x; k < n;
       k += static_cast<size_t>(gridDim.x) * kThreads) {
    const int i = static_cast<int>(k / dp), j = static_cast<int>(k % dp);
    L[k] = j <= i ? static_cast<double>(S[k]) : 0.0;
  }
}

// Factor the diagonal block jb in place (unblocked, in LDS).
__global__ __launch_bounds__(kThreads) void potrf_kernel(double* __restrict__ L, int dp, int jb,
                                                         uint32_t* __restrict__ flags) {
  __shared__ double T[kCb][kCb + 1];
  double* base = L + static_cast<size_t>(jb) * kCb * dp + jb * kCb;
  for (int s = threadIdx.x; s < kCb * kCb; s += kThreads) T[s / kCb][s % kCb] = base[(s / kCb) * static_cast<size_t>(dp) + s % kCb];
  __syncthreads();
  for (int k = 0; k < kCb; ++k) {
    if (threadIdx.x == 0) {
      const double piv = T[k][k];
      if (!(piv > 0.0)) atomicOr(flags, 2u);
      T[k][k] = sqrt(piv);   // NaN for a non-positive pivot; it propagates into S^-1
    }
    __syncthreads();
    const double dk = T[k][k];
    for (int i = k + 1 + threadIdx.x; i < kCb; i += kThreads) T[i][k] /= dk;
    __syncthreads();
    const int n = kCb - k - 1;   // trailing lower triangle of order n
    for (int s = threadIdx.x; s < n * n; s += kThreads) {
      const int i = k + 1 + s / n, j = k + 1 + s % n;
      if (j <= i) T[i][j] -= T[i][k] * T[j][k];
    }
    __syncthreads();
  }
  for (int s = threadIdx.x; s < kCb * kCb; s += kThreads) {
    const int i = s / kCb, j = s % kCb;
    base[i * static_cast<size_t>(dp) + j] = j <= i ? T[i][j] : 0.0;
  }
}

// Panel below the diagonal block: L[ib][jb] = A[ib][jb] L[jb][jb]^-T.
__global__ __launch_bounds__(kThreads) void trsm_kernel(double* __restrict__ L, int dp, int jb) {
  __shared__ double D[kCb][kCb + 1];
  __shared__ double X[kCb][kCb + 1];
  const int ib = jb + 1 + blockIdx.x;
  const double* dg = L + static_cast<size_t>(jb) * kCb * dp + jb * kCb;
  double* pb = L + static_cast<size_t>(ib) * kCb * dp + jb * kCb;
  for (int s = threadIdx.x; s < kCb * kCb; s += kThreads) {
    D[s / kCb][s % kCb] = dg[(s / kCb) * static_cast<size_t>(dp) + s % kCb];
    X[s / kCb][s % kCb] = pb[(s / kCb) * static_cast<size_t>(dp) + s % kCb];
  }
  __syncthreads();
  // row r of X solves x D^T = a: x_k = (a_k - sum_{m<k} x_m D[k][m]) / D[k][k]
  if (threadIdx.x < kCb) {
    const int r = threadIdx.x;
    for (int k = 0; k < kCb; ++k) {
      double v = X[r][k];
      for (int m = 0; m < k; ++m) v -= X[r][m] * D[k][m];
      X[r][k] = v / D[k][k];
    }
  }
  __syncthreads();
  for (int s = threadIdx.x; s < kCb * kCb; s += kThreads) pb[(s / kCb) * static_cast<size_t>(dp) + s % kCb] = X[s / kCb][s % kCb];
}

// Trailing update A[ib][kb] -= L[ib][jb] L[kb][jb]^T for jb < kb <= ib.
__global__ __launch_bounds__(kThreads) void syrk_update_kernel(double* __restrict__ L, int dp, int jb) {
  __shared__ double P[kCb][kCb + 1];
  __shared__ double Q[kCb][kCb + 1];
  int ib = jb + 1, rem = blockIdx.x;   // lower-triangle pair index -> (ib, kb)
  while (rem >= ib - jb) { rem -= ib - jb; ++ib; }
  const int kb = jb + 1 + rem;
  const double* pi = L + static_cast<size_t>(ib) * kCb * dp + jb * kCb;
  const double* pk = L + static_cast<size_t>(kb) * kCb * dp + jb * kCb;
  for (int s = threadIdx.x; s < kCb * kCb; s += kThreads) {
    P[s / kCb][s % kCb] = pi[(s / kCb) * static_cast<size_t>(dp) + s % kCb];
    Q[s / kCb][s % kCb] = pk[(s / kCb) * static_cast<size_t>(dp) + s % kCb];
  }
  __syncthreads();
  double* out = L + static_cast<size_t>(ib) * kCb * dp + kb * kCb;
  for (int s = threadIdx.x; s < kCb * kCb; s += kThreads) {
    const int i = s / kCb, j = s % kCb;
    double v = 0.0;
    for (int m = 0; m < kCb; ++m) v += P[i][m] * Q[j][m];
    out[i * static_cast<size_t>(dp) + j] -= v;
  }
}

// Inverse of each diagonal block of L (lower triangular, in LDS).
__global__ __launch_bounds__(kThreads) void trinv_diag_kernel(const double* __restrict__ L, double* __restrict__ Li,
                                                              int dp) {
  __shared__ double D[kCb][kCb + 1];
  __shared__ double X[kCb][kCb + 1];
  const int b = blockIdx.x;
  const double* dg = L + static_cast<size_t>(b) * kCb * dp + b * kCb;
  for (int s = threadIdx.x; s < kCb * kCb; s += kThreads) D[s / kCb][s % kCb] = dg[(s / kCb) * static_cast<size_t>(dp) + s % kCb];
  __syncthreads();
  // column c of D^-1 solves D x = e_c by forward substitution
  if (threadIdx.x < kCb) {
    const int c = threadIdx.x;
    for (int i = 0; i < kCb; ++i) {
      double v = i == c ? 1.0 : 0.0;
      for (int m = c; m < i; ++m) v -= D[i][m] * X[m][c];
      X[i][c] = i < c ? 0.0 : v / D[i][i];
    }
  }
  __syncthreads();
  double* out = Li + static_cast<size_t>(b) * kCb * dp + b * kCb;
  for (int s = threadIdx.x; s < kCb * kCb; s += kThreads) out[(s / kCb) * static_cast<size_t>(dp) + s % kCb] = X[s / kCb][s % kCb];
}

// Block row ib of L^-1 left of the diagonal:
// Li[ib][jb] = -Li[ib][ib] * sum_{kb=jb}^{ib-1} L[ib][kb] Li[kb][jb].
__global__ __launch_bounds__(kThreads) void trinv_offdiag_kernel(const double* __restrict__ L, double* __restrict__ Li,
                                                                 int dp, int ib) {
  __shared__ double P[kCb][kCb + 1];
  __shared__ double Q[kCb][kCb + 1];
  const int jb = blockIdx.x;
  double acc[kCb * kCb / kThreads];
#pragma unroll
  for (int q = 0; q < kCb * kCb / kThreads; ++q) acc[q] = 0.0;
  for (int kb = jb; kb < ib; ++kb) {
    const double* pl = L + static_cast<size_t>(ib) * kCb * dp + kb * kCb;
    const double* pq = Li + static_cast<size_t>(kb) * kCb * dp + jb * kCb;
    __syncthreads();
    for (int s = threadIdx.x; s < kCb * kCb; s += kThreads) {
      P[s / kCb][s % kCb] = pl[(s / kCb) * static_cast<size_t>(dp) + s % kCb];
      Q[s / kCb][s % kCb] = pq[(s / kCb) * static_cast<size_t>(dp) + s % kCb];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kCb * kCb / kThreads; ++q) {
      const int s = threadIdx.x + q * kThreads, i = s / kCb, j = s % kCb;
      double v = 0.0;
      for (int m = 0; m < kCb; ++m) v += P[i][m] * Q[m][j];
      acc[q] += v;
    }
  }
  // multiply by -Li[ib][ib]
  const double* pd = Li + static_cast<size_t>(ib) * kCb * dp + ib * kCb;
  __syncthreads();
  for (int s = threadIdx.x; s < kCb * kCb; s += kThreads) P[s / kCb][s % kCb] = pd[(s / kCb) * static_cast<size_t>(dp) + s % kCb];
#pragma unroll
  for (int q = 0; q < kCb * kCb / kThreads; ++q) {
    const int s = threadIdx.x + q * kThreads;
    Q[s / kCb][s % kCb] = acc[q];
  }
  __syncthreads();
  double* out = Li + static_cast<size_t>(ib) * kCb * dp + jb * kCb;
  for (int s = threadIdx.x; s < kCb * kCb; s += kThreads) {
    const int i = s / kCb, j = s % kCb;
    double v = 0.0;
    for (int m = 0; m <= i; ++m) v += P[i][m] * Q[m][j];
    out[i * static_cast<size_t>(dp) + j] = -v;
  }
}

// S^-1 = L^-T L^-1: block (ib, jb) = sum_{kb >= max(ib, jb)} Li[kb][ib]^T Li[kb][jb].
__global__ __launch_bounds__(kThreads) void inv_product_kernel(const double* __restrict__ Li, float* __restrict__ Sinv,
                                                               int dp) {
  __shared__ double P[kCb][kCb + 1];
  __shared__ double Q[kCb][kCb + 1];
  const int nb = dp / kCb;
  const int ib = blockIdx.x / nb, jb = blockIdx.x % nb;
  double acc[kCb * kCb / kThreads];
#pragma unroll
  for (int q = 0; q < kCb * kCb / kThreads; ++q) acc[q] = 0.0;
  for (int kb = ib > jb ? ib : jb; kb < nb; ++kb) {
    const double* pi = Li + static_cast<size_t>(kb) * kCb * dp + ib * kCb;
    const double* pj = Li + static_cast<size_t>(kb) * kCb * dp + jb * kCb;
    __syncthreads();
    for (int s = threadIdx.x; s < kCb * kCb; s += kThreads) {
      P[s / kCb][s % kCb] = pi[(s / kCb) * static_cast<size_t>(dp) + s % kCb];
      Q[s / kCb][s % kCb] = pj[(s / kCb) * static_cast<size_t>(dp) + s % kCb];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kCb * kCb / kThreads; ++q) {
      const int s = threadIdx.x + q * kThreads, i = s / kCb, j = s % kCb;
      double v = 0.0;
      for (int m = 0; m < kCb; ++m) v += P[m][i] * Q[m][j];
      acc[q] += v;
    }
  }
  float* out = Sinv + static_cast<size_t>(ib) * kCb * dp + jb * kCb;
#pragma unroll
  for (int q = 0; q < kCb * kCb / kThreads; ++q) {
    const int s = threadIdx.x + q * kThreads, i = s / kCb, j = s % kCb;
    out[i * static_cast<size_t>(dp) + j] = static_cast<float>(acc[q]);
  }
}

// ---------------------------------------------------------------- apply
// P[i][k*d + j] = sum_c G[i][k*d + c] * Sinv_k[j][c]   (S^-1 is symmetric,
// so its rows are the K-contiguous operand).  64x64 output tiles, 4 waves of
// 32x32, float32 MFMA 32x32x2; G (bf16 or float32) is converted to float32
// while it is staged.
__global__ __launch_bounds__(kThreads)
void apply_kernel(const PrecondDev* __restrict__ pds, const ApplyTask* __restrict__ tasks) {
  constexpr int BT = 64, WT = 32, BK = 32, LDA = BK + 4, EPP = WT + 8;
  constexpr int TILE = BT * LDA;
  static_assert(4 * 32 * EPP <= 4 * TILE, "epilogue staging");
  __shared__ __attribute__((aligned(16))) float smem[4 * TILE];   // [operand][buf][BT][LDA]
  auto sa = [&](int buf, int r, int k) -> float* { return smem + buf * TILE + r * LDA + k; };
  auto sb = [&](int buf, int r, int k) -> float* { return smem + (2 + buf) * TILE + r * LDA + k; };
  const ApplyTask t = tasks[blockIdx.x];
  const PrecondDev& pd = pds[t.tensor];
  const int d = pd.d, dp = pd.dp;
  const int r0 = t.tr * BT, c0 = t.tc * BT;            // rows of G, columns within block t.blk
  const int gcol0 = t.blk * d;                          // first column of the block in G and P
  const float* sinv = pd.sinv + static_cast<size_t>(t.blk) * dp * dp;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = tid >> 3, lk = (tid & 7) * 4;        // 32 rows x 8 chunks of 4 per pass

  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;

  f32x4_t ra[2], rb[2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = lrow + 32 * q;
      // operand A: G rows r0+row, columns k0+lk.. of the block (bounds-checked)
      const int gi = r0 + row, kc = k0 + lk;
      f32x4_t v = {0.f, 0.f, 0.f, 0.f};
      if (gi < pd.rows) {
        const size_t off = static_cast<size_t>(gi) * pd.ld_grad + gcol0 + kc;
        if (pd.vec_grad && kc + 4 <= d) {
          if (pd.grad_f32) {
            v = gld<f32x4_t>(static_cast<const float*>(pd.grad) + off);
          } else {
            const u32x2_t w = gld<u32x2_t>(static_cast<const uint16_t*>(pd.grad) + off);
            v[0] = __uint_as_float(w[0] << 16); v[1] = __uint_as_float(w[0] & 0xffff0000u);
            v[2] = __uint_as_float(w[1] << 16); v[3] = __uint_as_float(w[1] & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (kc + e < d)
              v[e] = pd.grad_f32 ? gld<float>(static_cast<const float*>(pd.grad) + off + e)
                                 : bf16_to_f32(gld<uint16_t>(static_cast<const uint16_t*>(pd.grad) + off + e));
        }
      }
      ra[q] = v;
      // operand B: rows c0+row of S^-1 (padded to dp, always in bounds)
      rb[q] = gld<f32x4_t>(sinv + static_cast<size_t>(c0 + row) * dp + k0 + lk);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      *reinterpret_cast<f32x4_t*>(sa(buf, lrow + 32 * q, lk)) = ra[q];
      *reinterpret_cast<f32x4_t*>(sb(buf, lrow + 32 * q, lk)) = rb[q];
    }
  };
  const int KT = dp / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) gload((kt + 1) * BK);
    const int k0 = (lane >> 5) * 16;
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(sa(buf, wm * WT + (lane & 31), k0 + kq * 4));
      const f32x4_t b = *reinterpret_cast<const f32x4_t*>(sb(buf, wn * WT + (lane & 31), k0 + kq * 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], acc, 0, 0, 0);
    }
    if (more) sstore(buf ^ 1);
    __syncthreads();
  }
  // epilogue through LDS: row segments of P
  float* ep = smem + wave * (32 * EPP);
#pragma unroll
  for (int r = 0; r < 16; ++r) ep[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * EPP + (lane & 31)] = acc[r];
  __syncthreads();
  for (int s = lane; s < 32 * WT; s += 64) {
    const int row = s / WT, col = s % WT;
    const int gi = r0 + wm * WT + row, cj = c0 + wn * WT + col;
    if (gi < pd.rows && cj < d) pd.p[static_cast<size_t>(gi) * pd.ld_p + gcol0 + cj] = ep[row * EPP + col];
  }
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

__global__ __launch_bounds__(kThreads) void identity_kernel(float* __restrict__ sinv, int dp, int nblocks) {
  const size_t n = static_cast<size_t>(nblocks) * dp * dp;
  for (size_t k = blockIdx.x * static_cast<size_t>(kThreads) + threadIdx.x; k < n;
       k += static_cast<size_t>(gridDim.x) * kThreads) {
    const size_t e = k % (static_cast<size_t>(dp) * dp);
    sinv[k] = (e / dp == e % dp) ? 1.0f : 0.0f;
  }
}

}  // namespace

hipError_t launch_identity(float* sinv, int dp, int nblocks, hipStream_t s) {
  identity_kernel<<<256, kThreads, 0, s>>>(sinv, dp, nblocks);
  return hipGetLastError();
}

namespace {

// X^T X of one activation batch into `out`: normalised (inv_n, damping) or
// accumulated (out = beta * out + X^T X).
void launch_moment(const void* acts, int64_t n_rows, int64_t ld, bool acts_f32, int d, int dp, float* out,
                   float inv_n, float damping, int accumulate, float beta, hipStream_t s) {
  const size_t es = acts_f32 ? 4 : 2;
  const int vec = (reinterpret_cast<uintptr_t>(acts) % 16 == 0) && ((ld * es) % 16 == 0);
  if (acts_f32) {
    const int nt = dp / MomCfg<true>::BT;
    moment_kernel<true><<<nt * (nt + 1) / 2, kThreads, 0, s>>>(acts, n_rows, ld, d, vec, out, dp, inv_n, damping,
                                                               accumulate, beta);
  } else {
    const int nt = dp / MomCfg<false>::BT;
    moment_kernel<false><<<nt * (nt + 1) / 2, kThreads, 0, s>>>(acts, n_rows, ld, d, vec, out, dp, inv_n, damping,
                                                                accumulate, beta);
  }
}

// S (in b.s) -> float64 Cholesky factor -> its inverse -> S^-1 (float32).
void factor_and_invert(const PrecondBlockDev& b, uint32_t* flags, hipStream_t s) {
  const int dp = b.dp, nb = dp / kCb;
  to_f64_kernel<<<256, kThreads, 0, s>>>(b.s, b.l, dp);
  for (int jb = 0; jb < nb; ++jb) {
    potrf_kernel<<<1, kThreads, 0, s>>>(b.l, dp, jb, flags);
    const int below = nb - jb - 1;
    if (below > 0) {
      trsm_kernel<<<below, kThreads, 0, s>>>(b.l, dp, jb);
      syrk_update_kernel<<<below * (below + 1) / 2, kThreads, 0, s>>>(b.l, dp, jb);
    }
  }
  trinv_diag_kernel<<<nb, kThreads, 0, s>>>(b.l, b.li, dp);
  for (int ib = 1; ib < nb; ++ib) trinv_offdiag_kernel<<<ib, kThreads, 0, s>>>(b.l, b.li, dp, ib);
  inv_product_kernel<<<nb * nb, kThreads, 0, s>>>(b.li, b.sinv, dp);
}

}  // namespace

hipError_t launch_precond_refresh(const PrecondBlockDev& b, const void* acts, int64_t n_rows, int64_t ld,
                                  bool acts_f32, float damping, uint32_t* flags, hipStream_t s) {
  const float inv_n = static_cast<float>(1.0 / static_cast<double>(n_rows));
  launch_moment(acts, n_rows, ld, acts_f32, b.d, b.dp, b.s, inv_n, damping, 0, 0.f, s);
  factor_and_invert(b, flags, s);
  return hipGetLastError();
}

hipError_t launch_precond_accumulate(const PrecondBlockDev& b, const void* acts, int64_t n_rows, int64_t ld,
                                     bool acts_f32, float beta, hipStream_t s) {
  launch_moment(acts, n_rows, ld, acts_f32, b.d, b.dp, b.acc, 0.f, 0.f, 1, beta, s);
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

hipError_t launch_precond_apply(const PrecondDev* pds, const ApplyTask* tasks, int n_tasks, hipStream_t s) {
  if (n_tasks <= 0) return hipSuccess;
  apply_kernel<<<n_tasks, kThreads, 0, s>>>(pds, tasks);
  return hipGetLastError();
}

}  // namespace muon
