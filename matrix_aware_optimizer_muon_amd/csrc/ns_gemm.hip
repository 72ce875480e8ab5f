// Quintic Newton-Schulz iteration of the Muon step on gfx950 MFMA (Muon blog
// by Venkatramana, section 3: X <- a X + b (X X^T) X + c (X X^T)^2 X, run in
// bfloat16 on the matrix units).  One iteration is three grouped launches,
// each over the tiles of every matrix at once:
//
//   kGram    A = s * X X^T          upper tiles only, mirror-stored   (K = n)
//   kSquare  B = b A + c A A        upper tiles only, mirror-stored   (K = m)
//   kBX      X = s * (a X + B X)    all tiles of m x n                (K = m)
//
// s folds the Frobenius normalisation into the first iteration (s = 1/||U||^2
// for the Gram, 1/||U|| for the update) so the norm never round-trips to the
// host.  All three are "rows x rows" products C[i][j] = sum_k P[i][k] Q[j][k]
// with both operands K-contiguous: A is symmetric, so A A = A A^T, and B X
// reads X^T, which the update epilogue writes alongside X.
//
// bf16 path: 128x128 output tile, 4 waves each owning 64x64 (2x2 blocks of
// v_mfma_f32_32x32x16_bf16), K staged through LDS 64 deep, double-buffered
// with register prefetch; two blocks fit per CU (74 KB LDS each) so one
// block's epilogue traffic overlaps the other's MFMA loop; X is held as a bf16 hi/lo pair so the a*X term
// keeps ~16 significant bits while the MFMA operand is the hi part.
// fp32 path: 64x64 tile, 4 waves of 32x32, v_mfma_f32_32x32x2f32.
#include "device_common.h"
#include "muon_internal.h"

namespace muon {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(1))) const u32x4_t gu32x4_t;   // global memory

constexpr int kThreads = 256;

template <bool F32> struct Cfg;
template <> struct Cfg<false> {
  using E = uint16_t;
  static constexpr int BT = kTileBf16, WT = kTileBf16 / 2, BK = 64, PAD = 8;
};
template <> struct Cfg<true> {
  using E = float;
  static constexpr int BT = kTileF32, WT = 32, BK = 32, PAD = 4;
};

template <bool F32, int PH>
__global__ __launch_bounds__(kThreads, 2)
void ns_gemm_kernel(const UnitDev* __restrict__ units, const GemmTask* __restrict__ tasks,
                    GemmParams p) {
  using C = Cfg<F32>;
  using E = typename C::E;
  constexpr int BT = C::BT, WT = C::WT, BK = C::BK;
  constexpr int LDP = BK + C::PAD;                 // LDS row pitch (elements)
  constexpr int NB = WT / 32;                      // 32x32 blocks per wave edge
  constexpr int EPE = 16 / sizeof(E);              // elements per 16-byte chunk
  constexpr int CPR = BK / EPE;                    // chunks per operand row
  constexpr int RPP = kThreads / CPR;              // rows per load pass
  constexpr int NPASS = BT / RPP;                  // load passes per operand
  constexpr int EPP = WT + 8;                      // epilogue LDS pitch (floats)
  static_assert(CPR * RPP == kThreads && NPASS * RPP == BT, "tile/thread mismatch");
  static_assert(4 * 32 * EPP * 4 <= 2 * 2 * BT * LDP * static_cast<int>(sizeof(E)),
                "epilogue staging must fit in the operand LDS");

  __shared__ __attribute__((aligned(16))) E lds[2][2][BT][LDP];
  __shared__ float red[4];

  const GemmTask t = tasks[blockIdx.x];
  const UnitDev& u = units[t.unit];
  const int mp = u.mp, np = u.np;
  const int ti = t.ti, tj = t.tj;

  const E* pa;
  const E* pb;
  int ld, K;
  if constexpr (PH == kGram) {
    pa = static_cast<const E*>(u.xh) + static_cast<size_t>(ti) * BT * np;
    pb = static_cast<const E*>(u.xh) + static_cast<size_t>(tj) * BT * np;
    ld = np; K = np;
  } else if constexpr (PH == kSquare) {
    pa = static_cast<const E*>(u.a) + static_cast<size_t>(ti) * BT * mp;
    pb = static_cast<const E*>(u.a) + static_cast<size_t>(tj) * BT * mp;
    ld = mp; K = mp;
  } else {
    pa = static_cast<const E*>(u.b) + static_cast<size_t>(ti) * BT * mp;
    pb = static_cast<const E*>(u.xt[p.xt_in]) + static_cast<size_t>(tj) * BT * mp;
    ld = mp; K = mp;
  }

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = tid / CPR, lchunk = tid % CPR;

  f32x16_t acc[NB][NB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Global (address space 1) views of the two operands, pre-offset to this
  // thread's first chunk; rows advance by RPP per load pass.
  const gu32x4_t* ga = (const gu32x4_t*)(pa + static_cast<size_t>(lrow) * ld + lchunk * EPE);
  const gu32x4_t* gb = (const gu32x4_t*)(pb + static_cast<size_t>(lrow) * ld + lchunk * EPE);
  const size_t pass_stride = static_cast<size_t>(RPP) * ld / EPE;   // in 16-byte chunks
  u32x4_t ra[NPASS], rb[NPASS];
#pragma unroll
  for (int q = 0; q < NPASS; ++q) {
    ra[q] = ga[q * pass_stride];
    rb[q] = gb[q * pass_stride];
  }
#pragma unroll
  for (int q = 0; q < NPASS; ++q) {
    *reinterpret_cast<u32x4_t*>(&lds[0][0][lrow + q * RPP][lchunk * EPE]) = ra[q];
    *reinterpret_cast<u32x4_t*>(&lds[0][1][lrow + q * RPP][lchunk * EPE]) = rb[q];
  }
  __syncthreads();

  const int KT = K / BK;
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) {
      const size_t koff = static_cast<size_t>(kt + 1) * (BK / EPE);
#pragma unroll
      for (int q = 0; q < NPASS; ++q) {
        ra[q] = ga[q * pass_stride + koff];
        rb[q] = gb[q * pass_stride + koff];
      }
    }
    if constexpr (!F32) {
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        bf16x8_t fa[NB], fb[NB];
        const int kk = ks * 16 + (lane >> 5) * 8;
#pragma unroll
        for (int i = 0; i < NB; ++i)
          fa[i] = *reinterpret_cast<const bf16x8_t*>(&lds[buf][0][wm * WT + i * 32 + (lane & 31)][kk]);
#pragma unroll
        for (int j = 0; j < NB; ++j)
          fb[j] = *reinterpret_cast<const bf16x8_t*>(&lds[buf][1][wn * WT + j * 32 + (lane & 31)][kk]);
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
    } else {
      // each lane half takes 16 consecutive k of the 32-deep slab; step e of
      // the MFMA pairs k = e (half 0) with k = 16 + e (half 1)
      const int k0 = (lane >> 5) * 16;
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        float4 fa[NB], fb[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i)
          fa[i] = *reinterpret_cast<const float4*>(&lds[buf][0][wm * WT + i * 32 + (lane & 31)][k0 + kq * 4]);
#pragma unroll
        for (int j = 0; j < NB; ++j)
          fb[j] = *reinterpret_cast<const float4*>(&lds[buf][1][wn * WT + j * 32 + (lane & 31)][k0 + kq * 4]);
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i].x, fb[j].x, acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i].y, fb[j].y, acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i].z, fb[j].z, acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i].w, fb[j].w, acc[i][j], 0, 0, 0);
          }
      }
    }
    if (more) {
#pragma unroll
      for (int q = 0; q < NPASS; ++q) {
        *reinterpret_cast<u32x4_t*>(&lds[buf ^ 1][0][lrow + q * RPP][lchunk * EPE]) = ra[q];
        *reinterpret_cast<u32x4_t*>(&lds[buf ^ 1][1][lrow + q * RPP][lchunk * EPE]) = rb[q];
      }
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  // Stage each wave's 32-row strip of accumulators in LDS, then write row
  // segments (natural layout) and column segments (mirror / X^T) as 16-byte
  // vector stores.
  float scale = 1.f;
  if constexpr (PH == kGram || PH == kBX) {
    if (p.first) {
      const float iv = unit_inv_norm(u.partials, u.k1_ntiles, p.eps, red);
      scale = PH == kGram ? iv * iv : iv;
    }
  }
  const bool mirror = (PH == kBX) || (ti != tj);
  float* ep = reinterpret_cast<float*>(&lds[0][0][0][0]) + wave * (32 * EPP);
  const int row_base = ti * BT + wm * WT;
  const int col_base = tj * BT + wn * WT;
  constexpr int SEGS = WT / 8;                       // row segments per strip row
  constexpr int RITER = 32 * SEGS / 64;              // row segments per lane
  constexpr int CITER = WT * 4 / 64;                 // column segments per lane

#pragma unroll
  for (int pi = 0; pi < NB; ++pi) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        ep[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * EPP + j * 32 + (lane & 31)] = acc[pi][j][r];
    __syncthreads();

#pragma unroll
    for (int q = 0; q < RITER; ++q) {
      const int s = lane + 64 * q;
      const int row = s / SEGS, cseg = s % SEGS;
      float v[8];
      const float4 v0 = *reinterpret_cast<const float4*>(&ep[row * EPP + cseg * 8]);
      const float4 v1 = *reinterpret_cast<const float4*>(&ep[row * EPP + cseg * 8 + 4]);
      v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
      v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
      const int gr = row_base + pi * 32 + row;
      const int gc = col_base + cseg * 8;
      if constexpr (PH == kGram) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= scale;
        st8<F32>(u.a, static_cast<size_t>(gr) * mp + gc, v);
      } else if constexpr (PH == kSquare) {
        float av[8];
        ld8<F32>(u.a, static_cast<size_t>(gr) * mp + gc, av);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = fmaf(p.b, av[e], p.c * v[e]);
        st8<F32>(u.b, static_cast<size_t>(gr) * mp + gc, v);
      } else {
        const size_t off = static_cast<size_t>(gr) * np + gc;
        float xm[8];
        if constexpr (F32) {
          ld8<true>(u.xh, off, xm);
        } else {
          float xl[8];
          ld8<false>(u.xh, off, xm);
          ld8<false>(u.xl, off, xl);
#pragma unroll
          for (int e = 0; e < 8; ++e) xm[e] += xl[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = scale * fmaf(p.a, xm[e], v[e]);
        if constexpr (F32) {
          st8<true>(u.xh, off, v);
        } else {
          float hi[8], lo[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            hi[e] = bf16_to_f32(f32_to_bf16(v[e]));
            lo[e] = v[e] - hi[e];
          }
          st8<false>(u.xh, off, hi);
          st8<false>(u.xl, off, lo);
        }
        *reinterpret_cast<float4*>(&ep[row * EPP + cseg * 8]) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(&ep[row * EPP + cseg * 8 + 4]) = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
    __syncthreads();

    if (mirror) {
#pragma unroll
      for (int q = 0; q < CITER; ++q) {
        const int s = lane + 64 * q;
        const int col = s % WT, rseg = s / WT;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = ep[(rseg * 8 + e) * EPP + col];
        const int gc = col_base + col;                 // mirror row
        const int gr = row_base + pi * 32 + rseg * 8;  // mirror column start
        if constexpr (PH == kGram) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] *= scale;
          st8<F32>(u.a, static_cast<size_t>(gc) * mp + gr, v);
        } else if constexpr (PH == kSquare) {
          float av[8];   // A is exactly symmetric off the diagonal tiles
          ld8<F32>(u.a, static_cast<size_t>(gc) * mp + gr, av);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = fmaf(p.b, av[e], p.c * v[e]);
          st8<F32>(u.b, static_cast<size_t>(gc) * mp + gr, v);
        } else {
          st8<F32>(u.xt[p.xt_in ^ 1], static_cast<size_t>(gc) * mp + gr, v);
        }
      }
    }
    __syncthreads();
  }
}

template <bool F32>
hipError_t launch_phase(int phase, const UnitDev* units, const GemmTask* tasks, int n,
                        const GemmParams& p, hipStream_t s) {
  switch (phase) {
    case kGram: ns_gemm_kernel<F32, kGram><<<n, kThreads, 0, s>>>(units, tasks, p); break;
    case kSquare: ns_gemm_kernel<F32, kSquare><<<n, kThreads, 0, s>>>(units, tasks, p); break;
    default: ns_gemm_kernel<F32, kBX><<<n, kThreads, 0, s>>>(units, tasks, p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int phase, bool f32, const UnitDev* units, const GemmTask* tasks,
                       int n_tasks, const GemmParams& p, hipStream_t s) {
  if (n_tasks <= 0) return hipSuccess;
  return f32 ? launch_phase<true>(phase, units, tasks, n_tasks, p, s)
             : launch_phase<false>(phase, units, tasks, n_tasks, p, s);
}

}  // namespace muon
