// HBM-bound phases of the Muon step on gfx950:
//
//   momentum_kernel  M' = mu M + (1-mu) G, Nesterov look-ahead U, the sum of
//                    squares of U (for the Frobenius normalisation), and U
//                    written into the NS workspace as a bf16 hi/lo pair (or
//                    float32) in the canonical short-side-first orientation.
//                    (Muon README, "Hyperparameter tuning"; Muon blog by
//                    Venkatramana, section 3: X = G / ||G||_F.)
//   update_kernel    W' = W - lr*wd*W - lr*scale*O, one round-to-nearest-even
//                    to bf16 (Muon README, "Usage": decoupled weight decay).
//
// Both walk 64x64 tiles of each matrix: every thread owns two 8-element row
// segments, so global traffic is 16-byte vector loads/stores along rows; the
// orientation swap needed for tall matrices goes through an LDS tile.
#include "muon_internal.h"

namespace muon {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even float32 -> bf16 (the conversion instruction of
// gfx950 via the compiler's fptrunc).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint4 pack8_bf16(const float* v) {
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w[e] = static_cast<uint32_t>(f32_to_bf16(v[2 * e])) |
           (static_cast<uint32_t>(f32_to_bf16(v[2 * e + 1])) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Split 8 float32 values into bf16 hi and lo parts (hi + lo carries ~16
// significant bits).
__device__ __forceinline__ void split8(const float* v, uint4& hi, uint4& lo) {
  float h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint16_t hb = f32_to_bf16(v[e]);
    h[e] = bf16_to_f32(hb);
    l[e] = v[e] - h[e];
  }
  hi = pack8_bf16(h);
  lo = pack8_bf16(l);
}

__device__ __forceinline__ void unpack8_bf16(const uint4& u, float* v) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(w[e] << 16);
    v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Store 8 values (one row segment) of an NS buffer: bf16 hi(/lo) or fp32.
template <bool F32>
__device__ __forceinline__ void store_seg(void* hi, void* lo, int64_t ld, int r, int c,
                                          const float* v) {
  if constexpr (F32) {
    float* p = static_cast<float*>(hi) + static_cast<size_t>(r) * ld + c;
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint4 h, l;
    split8(v, h, l);
    const size_t off = static_cast<size_t>(r) * ld + c;
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(hi) + off) = h;
    if (lo) *reinterpret_cast<uint4*>(static_cast<uint16_t*>(lo) + off) = l;
  }
}

template <bool F32>
__global__ __launch_bounds__(kThreads) void momentum_kernel(const UnitDev* __restrict__ units,
                                                            const EwTask* __restrict__ tasks,
                                                            K1Params p) {
  __shared__ float tile[kEwTile][kEwTile + 1];
  __shared__ float wsum[kThreads / 64];
  __shared__ int is_last;

  const EwTask t = tasks[blockIdx.x];
  const UnitDev& u = units[t.unit];
  const int r0 = t.tr * kEwTile, c0 = t.tc * kEwTile;
  const int rows = u.rows, cols = u.cols;
  const float mu = p.mu;
  const float one_m = 1.0f - mu;
  float ss = 0.f;
  bool bad = false;

#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int s = threadIdx.x + kThreads * q;
    const int lr = s >> 3, lc = (s & 7) * 8;
    const int i = r0 + lr, j0 = c0 + lc;
    float g[8], m[8], uv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { g[e] = 0.f; m[e] = 0.f; }
    const bool row_ok = i < rows;
    const bool full = row_ok && (j0 + 8 <= cols);
    if (row_ok) {
      if (u.grad_f32) {
        const float* gp = static_cast<const float*>(u.grad) + static_cast<size_t>(i) * u.ld_grad + j0;
        if (full && u.vec_grad) {
          const float4 a = *reinterpret_cast<const float4*>(gp);
          const float4 b = *reinterpret_cast<const float4*>(gp + 4);
          g[0] = a.x; g[1] = a.y; g[2] = a.z; g[3] = a.w;
          g[4] = b.x; g[5] = b.y; g[6] = b.z; g[7] = b.w;
        } else {
          for (int e = 0; e < 8; ++e) if (j0 + e < cols) g[e] = gp[e];
        }
      } else {
        const uint16_t* gp = static_cast<const uint16_t*>(u.grad) + static_cast<size_t>(i) * u.ld_grad + j0;
        if (full && u.vec_grad) {
          unpack8_bf16(*reinterpret_cast<const uint4*>(gp), g);
        } else {
          for (int e = 0; e < 8; ++e) if (j0 + e < cols) g[e] = bf16_to_f32(gp[e]);
        }
      }
      float* mp = u.mom + static_cast<size_t>(i) * u.ld_mom + j0;
      if (full && u.vec_mom) {
        const float4 a = *reinterpret_cast<const float4*>(mp);
        const float4 b = *reinterpret_cast<const float4*>(mp + 4);
        m[0] = a.x; m[1] = a.y; m[2] = a.z; m[3] = a.w;
        m[4] = b.x; m[5] = b.y; m[6] = b.z; m[7] = b.w;
      } else {
        for (int e = 0; e < 8; ++e) if (j0 + e < cols) m[e] = mp[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float mn, un;
        if (p.sgd_form) {
          mn = fmaf(mu, m[e], g[e]);
          un = p.nesterov ? fmaf(mu, mn, g[e]) : mn;
        } else {
          mn = fmaf(mu, m[e], one_m * g[e]);
          un = p.nesterov ? fmaf(mu, mn, one_m * g[e]) : mn;
        }
        m[e] = mn;
        uv[e] = (j0 + e < cols) ? un : 0.f;
      }
      if (full && u.vec_mom) {
        *reinterpret_cast<float4*>(mp) = make_float4(m[0], m[1], m[2], m[3]);
        *reinterpret_cast<float4*>(mp + 4) = make_float4(m[4], m[5], m[6], m[7]);
      } else {
        for (int e = 0; e < 8; ++e) if (j0 + e < cols) mp[e] = m[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) uv[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ss = fmaf(uv[e], uv[e], ss);
      bad |= !isfinite(uv[e]);
      tile[lr][lc + e] = uv[e];
    }
    // natural orientation: rows of the unit stay rows (padding gets zeros)
    store_seg<F32>(u.nat_hi, u.nat_lo, u.ld_nat, i, j0, uv);
  }
  __syncthreads();

  // transposed orientation: column segments of the tile become row segments
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int s = threadIdx.x + kThreads * q;
    const int lc = s & (kEwTile - 1), rseg = s >> 6;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[rseg * 8 + e][lc];
    store_seg<F32>(u.tr_hi, u.tr_lo, u.ld_tr, c0 + lc, r0 + rseg * 8, v);
  }

  // deterministic per-tile partial of sum(U^2)
  ss = wave_sum(ss);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) wsum[wave] = ss;
  if (__any(bad) && lane == 0) atomicOr(p.flags, 1u);
  __syncthreads();
  if (threadIdx.x == 0) {
    const float tot = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    u.partials[t.local] = tot;
    __threadfence();
    const uint32_t prev = atomicAdd(u.counter, 1u);
    is_last = (prev == static_cast<uint32_t>(u.k1_ntiles - 1));
  }
  __syncthreads();
  if (!is_last) return;

  // The last tile of this unit to finish folds the partials in a fixed
  // order (independent of which block ran last) and publishes 1/(||U||+eps).
  __threadfence();
  float acc = 0.f;
  for (int k = threadIdx.x; k < u.k1_ntiles; k += kThreads)
    acc += __builtin_nontemporal_load(&u.partials[k]);
  acc = wave_sum(acc);
  if (lane == 0) wsum[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float tot = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    *u.inv = 1.0f / (sqrtf(tot) + p.eps);
    *u.counter = 0u;
  }
}

template <bool F32>
__device__ __forceinline__ void load_master_seg(const UnitDev& u, int r, int c, float* v) {
  const size_t off = static_cast<size_t>(r) * u.np + c;
  if constexpr (F32) {
    const float* x = static_cast<const float*>(u.xh) + off;
    const float4 a = *reinterpret_cast<const float4*>(x);
    const float4 b = *reinterpret_cast<const float4*>(x + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    float h[8], l[8];
    unpack8_bf16(*reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(u.xh) + off), h);
    unpack8_bf16(*reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(u.xl) + off), l);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = h[e] + l[e];
  }
}

template <bool F32>
__global__ __launch_bounds__(kThreads) void update_kernel(const UnitDev* __restrict__ units,
                                                          const EwTask* __restrict__ tasks,
                                                          K5Params p) {
  __shared__ float tile[kEwTile][kEwTile + 1];
  const EwTask t = tasks[blockIdx.x];
  const UnitDev& u = units[t.unit];
  const int r0 = t.tr * kEwTile, c0 = t.tc * kEwTile;
  const int rows = u.rows, cols = u.cols;

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
  const float oscale = p.scale_by_inv ? *u.inv : 1.0f;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int s = threadIdx.x + kThreads * q;
    const int lr = s >> 3, lc = (s & 7) * 8;
    const int i = r0 + lr, j0 = c0 + lc;
    if (i >= rows) continue;
    float o[8];
    if (u.side == kRight) {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = tile[lr][lc + e];
    } else {
      load_master_seg<F32>(u, i, j0, o);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= oscale;
    const bool full = j0 + 8 <= cols;
    float w[8];
    if (u.param_f32) {
      float* wp = static_cast<float*>(u.param) + static_cast<size_t>(i) * u.ld_param + j0;
      if (full && u.vec_param) {
        const float4 a = *reinterpret_cast<const float4*>(wp);
        const float4 b = *reinterpret_cast<const float4*>(wp + 4);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
      } else {
        for (int e = 0; e < 8; ++e) w[e] = (j0 + e < cols) ? wp[e] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = w[e] - decay * w[e] - step * o[e];
      if (full && u.vec_param) {
        *reinterpret_cast<float4*>(wp) = make_float4(w[0], w[1], w[2], w[3]);
        *reinterpret_cast<float4*>(wp + 4) = make_float4(w[4], w[5], w[6], w[7]);
      } else {
        for (int e = 0; e < 8; ++e) if (j0 + e < cols) wp[e] = w[e];
      }
    } else {
      uint16_t* wp = static_cast<uint16_t*>(u.param) + static_cast<size_t>(i) * u.ld_param + j0;
      if (full && u.vec_param) {
        unpack8_bf16(*reinterpret_cast<const uint4*>(wp), w);
      } else {
        for (int e = 0; e < 8; ++e) w[e] = (j0 + e < cols) ? bf16_to_f32(wp[e]) : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = w[e] - decay * w[e] - step * o[e];
      if (full && u.vec_param) {
        *reinterpret_cast<uint4*>(wp) = pack8_bf16(w);
      } else {
        for (int e = 0; e < 8; ++e) if (j0 + e < cols) wp[e] = f32_to_bf16(w[e]);
      }
    }
    if (u.update_out) {
      float* op = u.update_out + static_cast<size_t>(i) * u.ld_out + j0;
      if (full && u.vec_out) {
        *reinterpret_cast<float4*>(op) = make_float4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<float4*>(op + 4) = make_float4(o[4], o[5], o[6], o[7]);
      } else {
        for (int e = 0; e < 8; ++e) if (j0 + e < cols) op[e] = o[e];
      }
    }
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
