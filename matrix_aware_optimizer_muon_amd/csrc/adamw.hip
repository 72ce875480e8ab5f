// AdamW for the parameters Muon does not take (Muon README, "Usage":
// embeddings, classifier heads, hidden gains and biases; lr 3e-4, betas
// (0.9, 0.95), weight decay 0.01), in the same step as the Muon matrices.
// Moments follow the recurrences of the Muon blog by Venkatramana, section
// 1, with the usual bias correction and eps:
//
//   M = b1 M + (1-b1) G,  V = b2 V + (1-b2) G^2,
//   W = W - lr*wd*W - lr * (M / (1-b1^t)) / (sqrt(V / (1-b2^t)) + eps).
//
// HBM-bound: 22 bytes per bf16 element (W 2+2, G 2, M 4+4, V 4+4), one
// launch over every AdamW tensor.  The step count t lives in the workspace
// and is advanced by a one-thread launch before the update, so a captured
// graph replays correctly.
#include <type_traits>

#include "device_common.h"
#include "muon_internal.h"

namespace muon {
namespace {

constexpr int kThreads = 256;

__global__ void adam_tick_kernel(AdamState* st, float beta1, float beta2) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  const uint32_t t = st->t + 1;
  st->t = t;
  const double bc1 = 1.0 - pow(double(beta1), double(t));
  const double bc2 = 1.0 - pow(double(beta2), double(t));
  st->inv_bc1 = float(1.0 / bc1);
  st->inv_sqrt_bc2 = float(1.0 / sqrt(bc2));
}

__global__ void adam_set_kernel(AdamState* st, uint32_t t) {
  if (threadIdx.x == 0 && blockIdx.x == 0) st->t = t;
}

// One AdamW element update in float32; returns the new parameter.
__device__ __forceinline__ float adamw_elem(float w, float g, float& m, float& v, const AdamParams& p,
                                            float lr, float inv_bc1, float inv_sqrt_bc2) {
  m = fmaf(p.beta1, m, (1.f - p.beta1) * g);
  v = fmaf(p.beta2, v, (1.f - p.beta2) * g * g);
  const float mh = m * inv_bc1;
  const float den = sqrtf(v) * inv_sqrt_bc2 + p.eps;
  return w - lr * p.weight_decay * w - lr * (mh / den);
}

// One thread's 8-element segment; WF32: the parameter and gradient are
// float32 (else bf16), a compile-time choice so that every load of a full
// segment is issued before the first wait.
template <bool WF32>
__device__ __forceinline__ void adamw_segment(const AdamDev& d, const AdamTask& tk, const AdamParams& p, float lr,
                                              float inv_bc1, float inv_sqrt_bc2, int64_t j0) {
  using W = typename std::conditional<WF32, float, uint16_t>::type;
  const int64_t r = tk.row;
  W* prow = static_cast<W*>(d.param) + r * d.ld_param;
  const W* grow = static_cast<const W*>(d.grad) + r * d.ld_grad;
  float* mrow = d.m + r * d.ld_mom;
  float* vrow = d.v + r * d.ld_mom;
  float w[8], g[8], m[8], v[8];
  const bool full = d.vec && j0 + 8 <= d.len;
  if (full) {
    ld8_f32(mrow, j0, m);
    ld8_f32(vrow, j0, v);
    ld8<WF32>(prow, j0, w);
    ld8<WF32>(grow, j0, g);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t j = j0 + e;
      w[e] = g[e] = m[e] = v[e] = 0.f;
      if (j < d.len) {
        if constexpr (WF32) {
          w[e] = gld<float>(prow + j);
          g[e] = gld<float>(grow + j);
        } else {
          w[e] = bf16_to_f32(gld<uint16_t>(prow + j));
          g[e] = bf16_to_f32(gld<uint16_t>(grow + j));
        }
        m[e] = gld<float>(mrow + j);
        v[e] = gld<float>(vrow + j);
      }
    }
  }
  bool bad = false;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bad |= !isfinite(g[e]);
    w[e] = adamw_elem(w[e], g[e], m[e], v[e], p, lr, inv_bc1, inv_sqrt_bc2);
  }
  if (full) {
    st8<WF32>(prow, j0, w);
    st8_f32(mrow, j0, m);
    st8_f32(vrow, j0, v);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t j = j0 + e;
      if (j < d.len) {
        if constexpr (WF32) gst(prow + j, w[e]);
        else gst(prow + j, f32_to_bf16(w[e]));
        gst(mrow + j, m[e]);
        gst(vrow + j, v[e]);
      }
    }
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(p.flags, 1u);
}

__global__ __launch_bounds__(kThreads) void adamw_kernel(const AdamDev* __restrict__ tensors,
                                                         const AdamTask* __restrict__ tasks, AdamParams p) {
  const AdamTask tk = tasks[blockIdx.x];
  const AdamDev& d = tensors[tk.tensor];
  const float lr = p.lr * d.lr_mult;
  const float inv_bc1 = p.state->inv_bc1, inv_sqrt_bc2 = p.state->inv_sqrt_bc2;
  const int64_t j0 = tk.c0 + int64_t(threadIdx.x) * 8;
  if (j0 >= d.len) return;
  if (d.f32) adamw_segment<true>(d, tk, p, lr, inv_bc1, inv_sqrt_bc2, j0);
  else adamw_segment<false>(d, tk, p, lr, inv_bc1, inv_sqrt_bc2, j0);
}

}  // namespace

hipError_t launch_adam_tick(AdamState* st, float beta1, float beta2, hipStream_t s) {
  adam_tick_kernel<<<1, 64, 0, s>>>(st, beta1, beta2);
  return hipGetLastError();
}

hipError_t launch_adam_set(AdamState* st, uint32_t t, hipStream_t s) {
  adam_set_kernel<<<1, 64, 0, s>>>(st, t);
  return hipGetLastError();
}

hipError_t launch_adamw(const AdamDev* tensors, const AdamTask* tasks, int n_tasks, const AdamParams& p,
                        hipStream_t s) {
  if (n_tasks <= 0) return hipSuccess;
  adamw_kernel<<<n_tasks, kThreads, 0, s>>>(tensors, tasks, p);
  return hipGetLastError();
}

}  // namespace muon
