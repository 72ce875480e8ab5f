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
// Both walk tiles of 8192 elements in which every thread owns four 8-element
// row segments, so global traffic is 16-byte vector accesses along rows:
// 32 x 256 tiles for units whose X is U (a wave covers two 256-element runs
// of one row each; the 32 rows are one row of whole correction blocks, so
// each block's 16-byte lane chunks are written whole), 64 x 128 tiles (of U)
// for units whose X is U^T, whose orientation swap goes through an LDS tile.  The partial sums are folded
// later, in a fixed order, by the first Newton-Schulz phase, so no block
// here waits on another.
#include "device_common.h"
#include "muon_internal.h"

namespace muon {
namespace {

constexpr int kThreads = 256;
constexpr int kSegs = 4;   // 8-element row segments per thread and tile
static_assert(kEwRows * kEwCols == kThreads * kSegs * 8 && kEwRRows * kEwRCols == kThreads * kSegs * 8,
              "a tile is kSegs segments per thread");
// LDS tile of a momentum block: 64 x (128 + 1) floats for the transposed
// (right-side) walk (column reads at pitch 129 put the 64 lanes in distinct
// banks), 32 x (256 + 8) for the correction blocks of a left-side one (pitch
// 264 puts the two half-waves of a column read in different banks).
constexpr int kRightPitch = kEwRCols + 1;
constexpr int kLeftPitch = kEwCols + 8;
constexpr int kTileFloats = kEwRRows * kRightPitch > kEwRows * kLeftPitch ? kEwRRows * kRightPitch
                                                                          : kEwRows * kLeftPitch;

// Debug builds: an elementwise tile starts inside its unit, and the X rows
// (left side) or X columns (right side) it writes stay inside the padded
// master.
__device__ __forceinline__ bool ew_tile_in_bounds(const UnitDev& u, const EwTask& t) {
  const bool left = u.side == kLeft;
  const int r0 = t.tr * (left ? kEwRows : kEwRRows), c0 = t.tc * (left ? kEwCols : kEwRCols);
  if (t.tr < 0 || t.tc < 0 || r0 >= u.rows || c0 >= u.cols) return false;
  return left ? r0 + kEwRows <= u.mp : r0 + kEwRRows <= u.np;
}

// Store one 8-element row segment of X: the bf16 hi part of the master (its
// int8 corrections are written separately, in their blocked layout), or the
// float32 value.
template <bool F32>
__device__ __forceinline__ void store_seg(void* hi, int64_t ld, int r, int c, const float* v) {
  const size_t off = static_cast<size_t>(r) * ld + c;
  if constexpr (F32) st8_f32(hi, off, v);
  else gst(static_cast<uint16_t*>(hi) + off, pack8_bf16(v));
}

// Four consecutive X rows of one column (values x[0..3]) as their four int8
// master corrections, packed low byte first.
__device__ __forceinline__ uint32_t corr4(const float* x) {
  uint32_t w = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) w |= static_cast<uint32_t>(master_corr(x[e])) << (8 * e);
  return w;
}

// One tile of the momentum phase; GF32: the gradient is float32 (else
// bf16), a compile-time choice so the tile's loads are straight-line code.
template <bool F32, bool GF32>
__device__ __forceinline__ void momentum_tile(const UnitDev& u, const EwTask& t, const K1Params& p,
                                              float* tile, float* wsum) {
  const bool left = u.side == kLeft;
  const int r0 = t.tr * (left ? kEwRows : kEwRRows), c0 = t.tc * (left ? kEwCols : kEwRCols);
  const int seg_sh = left ? 5 : 4;                   // log2 of 8-element segments per tile row
  const int rows = u.rows, cols = u.cols;
  const float mu = p.mu;
  const float one_m = 1.0f - mu;
  float ss = 0.f;
  bool bad = false;

  // Interior tiles with 16-byte aligned rows take a branch-free path that
  // issues every load of the thread before the first use, so the load
  // latency is paid once per tile rather than once per access; edge tiles
  // go element by element where needed.
  const bool interior = r0 + (left ? kEwRows : kEwRRows) <= rows && c0 + (left ? kEwCols : kEwRCols) <= cols &&
                        u.vec_grad && u.vec_mom;
  int iq[kSegs], jq[kSegs], lrq[kSegs], lcq[kSegs];
#pragma unroll
  for (int q = 0; q < kSegs; ++q) {
    const int s = threadIdx.x + kThreads * q;
    lrq[q] = s >> seg_sh;
    lcq[q] = (s & ((1 << seg_sh) - 1)) * 8;
    iq[q] = r0 + lrq[q];
    jq[q] = c0 + lcq[q];
  }
  float g[kSegs][8], m[kSegs][8];
  if (interior) {
#pragma unroll
    for (int q = 0; q < kSegs; ++q) ld8_f32(u.mom, static_cast<size_t>(iq[q]) * u.ld_mom + jq[q], m[q]);
#pragma unroll
    for (int q = 0; q < kSegs; ++q) {
      const size_t og = static_cast<size_t>(iq[q]) * u.ld_grad + jq[q];
      if constexpr (GF32) ld8_f32(u.grad, og, g[q]);
      else ld8_bf16(u.grad, og, g[q]);
    }
  } else {
#pragma unroll
    for (int q = 0; q < kSegs; ++q) {
#pragma unroll
      for (int e = 0; e < 8; ++e) g[q][e] = m[q][e] = 0.f;
      if (iq[q] < rows) {
        load_row8(u.grad, GF32, u.ld_grad, iq[q], jq[q], cols, u.vec_grad, g[q]);
        load_row8(u.mom, true, u.ld_mom, iq[q], jq[q], cols, u.vec_mom, m[q]);
      }
    }
  }

#pragma unroll
  for (int q = 0; q < kSegs; ++q) {
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
      if (j0 < u.np) store_seg<F32>(u.xh[0], u.np, i, j0, uv);
      if constexpr (!F32) {
#pragma unroll
        for (int e = 0; e < 8; ++e) tile[lr * kLeftPitch + lc + e] = uv[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[lr * kRightPitch + lc + e] = uv[e];
    }
  }
  if (!left) {
    // X = U^T: column segments of the tile become row segments of X (128 X
    // rows of 64 elements; eight lanes cover one row); X rows past the
    // padded m (a 128-wide tile of a float32 unit padded to 64) are skipped
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kSegs; ++q) {
      const int s = threadIdx.x + kThreads * q;
      const int xr = s >> 3, xs = s & 7;
      if (c0 + xr >= u.mp) continue;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = tile[(xs * 8 + e) * kRightPitch + xr];
      store_seg<F32>(u.xh[0], u.np, c0 + xr, r0 + xs * 8, v);
    }
    if constexpr (!F32) {
      // corrections: the 128 x 64 X tile is 4 x 2 whole 32 x 32 blocks;
      // thread t writes lane l = t%64's 16 bytes of block t/64 and of block
      // t/64 + 4 (X row c0 + 32 bi + 8q + 4h + e, column r0 + 32 bj + l%32,
      // i.e. U-tile element [32 bj + l%32][32 bi + 8q + 4h + e])
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const int s = threadIdx.x + kThreads * q2;
        const int blk = s >> 6, l = s & 63;
        const int bi = blk >> 1, bj = blk & 1;
        if (c0 + 32 * bi >= u.mp) continue;
        const float* trow = &tile[(32 * bj + (l & 31)) * kRightPitch + 32 * bi + 4 * (l >> 5)];
        u32x4_t w;
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = corr4(trow + 8 * q);
        gst(static_cast<int8_t*>(u.xl) + corr_block_offset(u.np, c0 + 32 * bi, r0 + 32 * bj) + l * 16, w);
      }
    }
  } else if constexpr (!F32) {
    // corrections of a left tile: its 32 rows are one row of 32 x 32 blocks;
    // thread t writes lane l = t%64's 16 bytes of block t/64 and of block
    // t/64 + 4 (rows 8q + 4h + e, column 32 jb + l%32)
    __syncthreads();
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      const int s = threadIdx.x + kThreads * q2;
      const int jb = s >> 6, l = s & 63;
      const int col = c0 + 32 * jb;
      if (col >= u.np) continue;
      const float* tcol = &tile[4 * (l >> 5) * kLeftPitch + 32 * jb + (l & 31)];
      u32x4_t w;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = tcol[(8 * q + e) * kLeftPitch];
        w[q] = corr4(x);
      }
      gst(static_cast<int8_t*>(u.xl) + corr_block_offset(u.np, r0, col) + l * 16, w);
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
  __shared__ float tile[kTileFloats];
  __shared__ float wsum[kThreads / 64];
  const EwTask t = tasks[blockIdx.x];
  const UnitDev& u = units[t.unit];
  if constexpr (MUON_DEBUG_BOUNDS) {
    if (!ew_tile_in_bounds(u, t)) {
      if (threadIdx.x == 0) atomicOr(p.flags, kFlagBounds);
      return;
    }
  }
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
    const uint16_t* hp = static_cast<const uint16_t*>(u.xh[0]) + off;
    const int8_t* xl = static_cast<const int8_t*>(u.xl);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int hb = static_cast<int>(static_cast<uint32_t>(gld<uint16_t>(hp + e)) << 16);
      v[e] = __int_as_float(hb + 256 * static_cast<int>(gld<int8_t>(xl + corr_index(u.np, r, c + e))));
    }
  }
}

template <bool F32>
__global__ __launch_bounds__(kThreads) void update_kernel(const UnitDev* __restrict__ units,
                                                          const EwTask* __restrict__ tasks,
                                                          K5Params p) {
  __shared__ float tile[kEwRRows][kRightPitch];
  __shared__ float red[4];
  const EwTask t = tasks[blockIdx.x];
  const UnitDev& u = units[t.unit];
  if constexpr (MUON_DEBUG_BOUNDS) {
    if (!ew_tile_in_bounds(u, t)) {
      if (threadIdx.x == 0) atomicOr(p.flags, kFlagBounds);
      return;
    }
  }
  const bool left = u.side == kLeft;
  const int r0 = t.tr * (left ? kEwRows : kEwRRows), c0 = t.tc * (left ? kEwCols : kEwRCols);
  const int seg_sh = left ? 5 : 4;                   // log2 of 8-element segments per tile row
  const int rows = u.rows;
  // with no Newton-Schulz iteration O is the normalised U itself
  const float inv = unit_inv_norm(u.partials, u.k1_ntiles, p.eps, red);

  if (u.side == kRight) {
    // O[i][j] = X[j][i]: read X row segments (j fixed, i contiguous) into
    // the tile transposed (X rows past the padded m read as zeros)
#pragma unroll
    for (int q = 0; q < kSegs; ++q) {
      const int s = threadIdx.x + kThreads * q;
      const int lj = s >> 3, li = (s & 7) * 8;
      float v[8];
      if (c0 + lj < u.mp) {
        load_master_seg<F32>(u, c0 + lj, r0 + li, v);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[li + e][lj] = v[e];
    }
    __syncthreads();
  }

  const float decay = p.lr * p.weight_decay;
  const float step = p.lr * u.lr_scale;
#pragma unroll
  for (int q = 0; q < kSegs; ++q) {
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
