// HBM-bound phases of the Muon step on gfx950:
//
//   momentum_kernel  M' = mu M + (1-mu) G, the Nesterov look-ahead U, one
//                    partial sum of U^2 per tile (for the Frobenius
//                    normalisation), and U written into the NS workspace as
//                    the two-part X master (or float32) in the canonical
//                    short-side-first orientation.
//                    (Muon README, "Hyperparameter tuning"; Muon blog by
//                    Venkatramana, section 3: X = G / ||G||_F.)
//   update_kernel    W' = W - lr*wd*W - lr*scale*O with O = U/||U||, for
//                    ns_steps == 0 only (otherwise the last Newton-Schulz
//                    phase applies the update).
//
// Both walk tiles of 4096 elements in which every thread owns two 8-element
// row segments, so global traffic is 16-byte vector accesses along rows:
// 16 x 256 tiles for units whose X is U (a wave covers two 256-element runs
// of one row each), 64 x 64 tiles for units whose X is U^T, whose
// orientation swap goes through an LDS tile.  The partial sums are folded
// later, in a fixed order, by the first Newton-Schulz phase, so no block
// here waits on another.
#include "device_common.h"
#include "muon_internal.h"

namespace muon {
namespace {

constexpr int kThreads = 256;

// Store one 8-element row segment of the X master: bf16 hi and its int8
// correction (element offsets are shared, the correction array holds one
// byte per element), or float32.
template <bool F32>
__device__ __forceinline__ void store_seg(void* hi, void* lo, int64_t ld, int r, int c, const float* v) {
  const size_t off = static_cast<size_t>(r) * ld + c;
  if constexpr (F32) {
    st8_f32(hi, off, v);
  } else {
    u32x4_t h;
    u32x2_t q;
    master_encode8(v, h, q);
    gst(static_cast<uint16_t*>(hi) + off, h);
    gst(static_cast<int8_t*>(lo) + off, q);
  }
}

// One tile of the momentum phase; GF32: the gradient is float32 (else
// bf16), a compile-time choice so the tile's loads are straight-line code.
template <bool F32, bool GF32>
__device__ __forceinline__ void momentum_tile(const UnitDev& u, const EwTask& t, const K1Params& p,
                                              float (*tile)[kEwTile + 1], float* wsum) {
  const bool left = u.side == kLeft;
  const int r0 = t.tr * (left ? kEwRows : kEwTile), c0 = t.tc * (left ? kEwCols : kEwTile);
  const int seg_sh = left ? 5 : 3;                   // log2 of 8-element segments per tile row
  const int rows = u.rows, cols = u.cols;
  const float mu = p.mu;
  const float one_m = 1.0f - mu;
  float ss = 0.f;
  bool bad = false;

  // Interior tiles with 16-byte aligned rows take a branch-free path that
  // issues every load of the thread before the first use, so the load
  // latency is paid once per tile rather than once per access; edge tiles
  // go element by element where needed.
  const bool interior = r0 + (left ? kEwRows : kEwTile) <= rows && c0 + (left ? kEwCols : kEwTile) <= cols &&
                        u.vec_grad && u.vec_mom;
  int iq[2], jq[2], lrq[2], lcq[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int s = threadIdx.x + kThreads * q;
    lrq[q] = s >> seg_sh;
    lcq[q] = (s & ((1 << seg_sh) - 1)) * 8;
    iq[q] = r0 + lrq[q];
    jq[q] = c0 + lcq[q];
  }
  float g[2][8], m[2][8];
  if (interior) {
    ld8_f32(u.mom, static_cast<size_t>(iq[0]) * u.ld_mom + jq[0], m[0]);
    ld8_f32(u.mom, static_cast<size_t>(iq[1]) * u.ld_mom + jq[1], m[1]);
    const size_t og0 = static_cast<size_t>(iq[0]) * u.ld_grad + jq[0];
    const size_t og1 = static_cast<size_t>(iq[1]) * u.ld_grad + jq[1];
    if constexpr (GF32) {
      ld8_f32(u.grad, og0, g[0]);
      ld8_f32(u.grad, og1, g[1]);
    } else {
      ld8_bf16(u.grad, og0, g[0]);
      ld8_bf16(u.grad, og1, g[1]);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int e = 0; e < 8; ++e) g[q][e] = m[q][e] = 0.f;
      if (iq[q] < rows) {
        load_row8(u.grad, GF32, u.ld_grad, iq[q], jq[q], cols, u.vec_grad, g[q]);
        load_row8(u.mom, true, u.ld_mom, iq[q], jq[q], cols, u.vec_mom, m[q]);
      }
    }
  }

#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = iq[q], j0 = jq[q], lr = lrq[q], lc = lcq[q];
    float uv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float mn, un;
      if (p.sgd_form) {
        mn = fmaf(mu, m[q][e], g[q][e]);
        un = p.nesterov ? fmaf(mu, mn, g[q][e]) : mn;
      } else {
        mn = fmaf(mu, m[q][e], one_m * g[q][e]);
        un = p.nesterov ? fmaf(mu, mn, one_m * g[q][e]) : mn;
      }
      m[q][e] = mn;
      uv[e] = (i < rows && j0 + e < cols) ? un : 0.f;
    }
    if (interior) st8_f32(u.mom, static_cast<size_t>(i) * u.ld_mom + j0, m[q]);
    else if (i < rows) store_row8(u.mom, true, u.ld_mom, i, j0, cols, u.vec_mom, m[q]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ss = fmaf(uv[e], uv[e], ss);
      bad |= !isfinite(uv[e]);
    }
    if (left) {
      // X = U: rows of the unit stay rows (padding inside the tile gets
      // zeros; a 256-wide tile may reach past the padded width np)
      if (j0 < u.np) store_seg<F32>(u.xh[0], u.xl, u.np, i, j0, uv);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[lr][lc + e] = uv[e];
    }
  }
  if (!left) {
    // X = U^T: column segments of the tile become row segments of X
    __syncthreads();
    // eight lanes cover one X row (a 64-element run); LDS column reads at
    // pitch kEwTile + 1 put the 64 lanes in distinct banks
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int s = threadIdx.x + kThreads * q;
      const int xr = s >> 3, xs = s & 7;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = tile[xs * 8 + e][xr];
      store_seg<F32>(u.xh[0], u.xl, u.np, c0 + xr, r0 + xs * 8, v);
    }
  }

  // per-tile partial of sum(U^2), in a fixed order
  ss = wave_sum(ss);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) wsum[wave] = ss;
  if (__any(bad) && lane == 0) atomicOr(p.flags, 1u);
  __syncthreads();
  if (threadIdx.x == 0) gst(u.partials + t.local, (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]));
}

template <bool F32>
__global__ __launch_bounds__(kThreads) void momentum_kernel(const UnitDev* __restrict__ units,
                                                            const EwTask* __restrict__ tasks,
                                                            K1Params p) {
  __shared__ float tile[kEwTile][kEwTile + 1];
  __shared__ float wsum[kThreads / 64];
  const EwTask t = tasks[blockIdx.x];
  const UnitDev& u = units[t.unit];
  if (u.grad_f32) momentum_tile<F32, true>(u, t, p, tile, wsum);
  else momentum_tile<F32, false>(u, t, p, tile, wsum);
}

// X master of the stand-alone update (ns_steps == 0: the iterate the
// momentum phase wrote, buffer 0).
template <bool F32>
__device__ __forceinline__ void load_master_seg(const UnitDev& u, int r, int c, float* v) {
  const size_t off = static_cast<size_t>(r) * u.np + c;
  if constexpr (F32) {
    ld8_f32(u.xh[0], off, v);
  } else {
    master_decode8(gld<u32x4_t>(static_cast<const uint16_t*>(u.xh[0]) + off),
                   gld<u32x2_t>(static_cast<const int8_t*>(u.xl) + off), v);
  }
}

template <bool F32>
__global__ __launch_bounds__(kThreads) void update_kernel(const UnitDev* __restrict__ units,
                                                          const EwTask* __restrict__ tasks,
                                                          K5Params p) {
  __shared__ float tile[kEwTile][kEwTile + 1];
  __shared__ float red[4];
  const EwTask t = tasks[blockIdx.x];
  const UnitDev& u = units[t.unit];
  const bool left = u.side == kLeft;
  const int r0 = t.tr * (left ? kEwRows : kEwTile), c0 = t.tc * (left ? kEwCols : kEwTile);
  const int seg_sh = left ? 5 : 3;                   // log2 of 8-element segments per tile row
  const int rows = u.rows;
  // with no Newton-Schulz iteration O is the normalised U itself
  const float inv = unit_inv_norm(u.partials, u.k1_ntiles, p.eps, red);

  if (u.side == kRight) {
    // O[i][j] = X[j][i]: read X row segments (j fixed, i contiguous) into
    // the tile transposed.
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int s = threadIdx.x + kThreads * q;
      const int lj = s >> 3, li = (s & 7) * 8;
      float v[8];
      load_master_seg<F32>(u, c0 + lj, r0 + li, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[li + e][lj] = v[e];
    }
    __syncthreads();
  }

  const float decay = p.lr * p.weight_decay;
  const float step = p.lr * u.lr_scale;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int s = threadIdx.x + kThreads * q;
    const int lr = s >> seg_sh, lc = (s & ((1 << seg_sh) - 1)) * 8;
    const int i = r0 + lr, j0 = c0 + lc;
    if (i >= rows || j0 >= u.cols) continue;
    float o[8];
    if (!left) {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = tile[lr][lc + e];
    } else {
      load_master_seg<F32>(u, i, j0, o);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= inv;
    update_w8(u, i, j0, o, decay, step);
  }
}

}  // namespace

hipError_t launch_momentum(bool f32, const UnitDev* units, const EwTask* tasks, int n_tasks,
                           const K1Params& p, hipStream_t s) {
  if (n_tasks <= 0) return hipSuccess;
  if (f32)
    momentum_kernel<true><<<n_tasks, kThreads, 0, s>>>(units, tasks, p);
  else
    momentum_kernel<false><<<n_tasks, kThreads, 0, s>>>(units, tasks, p);
  return hipGetLastError();
}

hipError_t launch_update(bool f32, const UnitDev* units, const EwTask* tasks, int n_tasks,
                         const K5Params& p, hipStream_t s) {
  if (n_tasks <= 0) return hipSuccess;
  if (f32)
    update_kernel<true><<<n_tasks, kThreads, 0, s>>>(units, tasks, p);
  else
    update_kernel<false><<<n_tasks, kThreads, 0, s>>>(units, tasks, p);
  return hipGetLastError();
}

}  // namespace muon
