// Device helpers shared by the gfx950 kernels: bf16 <-> float32 conversion
// and 16-byte vector accesses through address-space-1 (global) pointers, so
// the compiler emits global_load/store_dwordx4 rather than flat accesses
// (flat accesses also count against the LDS wait counter).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "muon_internal.h"

namespace muon {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
#define MUON_GLOBAL __attribute__((address_space(1)))

template <typename T>
__device__ __forceinline__ T gld(const void* p) {
  return *(const MUON_GLOBAL T*)p;
}
template <typename T>
__device__ __forceinline__ void gst(void* p, const T& v) {
  *(MUON_GLOBAL T*)p = v;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float32 -> bf16, round to nearest even (the compiler's fptrunc, which
// gfx950 implements with its bf16 conversion instruction).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two floats to bf16 (round to nearest even) packed in one word, a first,
// in one conversion instruction.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt2_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

__device__ __forceinline__ u32x4_t pack8_bf16(const float* v) {
  u32x4_t w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = cvt2_bf16(v[2 * e], v[2 * e + 1]);
  return w;
}

// A wave-uniform pointer held as a computed scalar value: a pointer read from
// a descriptor in memory may otherwise be re-read from it after each store
// (a scalar load and a wait per use), since the compiler is free to reload
// what it knows is unchanged rather than keep it in registers.
__device__ __forceinline__ int32_t sreg_i32(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t sreg_i64(int64_t v) {
  const uint64_t u = static_cast<uint64_t>(v);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}
template <typename T>
__device__ __forceinline__ T* sreg_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ void unpack8_bf16(const u32x4_t& w, float* v) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(w[e] << 16);
    v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
}

// Two-part X master of the bf16 Newton-Schulz path: hi = x rounded to bf16
// (the MFMA operand; here to nearest even) and an int8 correction q counted
// in the float32 bit pattern,
// x ~= float_from_bits(bits(hi) + 256 q).  Within hi's binade 256 float32
// ulps are ulp_bf16(hi)/256, so q carries 8 more bits below hi's last one
// (round-to-nearest-even gives |bits(x) - bits(hi)| <= 2^15, so |q| <= 128,
// kept in [-127, 127]).  Where the rounding carried hi up to a power of two
// the count runs in the binade below, and the decode, adding in the same bit
// space, lands there too.  Sign-magnitude patterns make the count a
// magnitude offset for negative x as well.  Integer arithmetic only: a
// subtraction and a rounding shift to encode, a shift-add to decode.  The
// decode holds for any hi within 2^15 bit steps of x whose q was counted
// against that hi: the B X epilogue writes its masters with hi rounded
// half-up at a threshold 128 steps below the tie (q in [-128, 127], same
// 128-step accuracy), which it packs with fewer instructions.
__device__ __forceinline__ void master_encode8(const float* v, u32x4_t& hi, u32x2_t& lo) {
  uint32_t q[8];
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const uint32_t hp = cvt2_bf16(v[e], v[e + 1]);
    hi[e >> 1] = hp;
    const int d0 = __float_as_int(v[e]) - static_cast<int>(hp << 16);
    const int d1 = __float_as_int(v[e + 1]) - static_cast<int>(hp & 0xFFFF0000u);
    q[e] = static_cast<uint32_t>(min(max((d0 + 128) >> 8, -127), 127)) & 0xFFu;
    q[e + 1] = static_cast<uint32_t>(min(max((d1 + 128) >> 8, -127), 127)) & 0xFFu;
  }
  lo[0] = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
  lo[1] = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
}

// The correction of one element: q = round((bits(x) - bits(bf16(x))) / 256),
// clamped to [-127, 127], as its byte.
__device__ __forceinline__ uint32_t master_corr(float x) {
  const uint32_t hb = static_cast<uint32_t>(f32_to_bf16(x)) << 16;
  const int d = __float_as_int(x) - static_cast<int>(hb);
  return static_cast<uint32_t>(min(max((d + 128) >> 8, -127), 127)) & 0xFFu;
}

// Layout of the correction array (one byte per element of the padded m_p x
// n_p master): 32 x 32 blocks of 1 KB, block (bi, bj) at (bi * n_p/32 + bj)
// KB; inside a block, the 16 bytes of lane l hold, in MFMA accumulator
// register order r = 4q + e, the elements at row 8q + 4(l/32) + e, column
// l%32 -- the positions the B X kernel's accumulators hold.
__device__ __forceinline__ size_t corr_block_offset(int np, int r0, int c0) {   // r0, c0 multiples of 32
  return (static_cast<size_t>(r0 >> 5) * (np >> 5) + (c0 >> 5)) * 1024;
}
__device__ __forceinline__ size_t corr_index(int np, int r, int c) {
  const int lr = r & 31;
  const int lane = (c & 31) + 32 * ((lr >> 2) & 1);
  const int reg = 4 * (lr >> 3) + (lr & 3);
  return corr_block_offset(np, r & ~31, c & ~31) + lane * 16 + reg;
}

__device__ __forceinline__ void master_decode8(const u32x4_t& hi, const u32x2_t& lo, float* v) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t h32 = (e & 1) ? (hi[e >> 1] & 0xFFFF0000u) : (hi[e >> 1] << 16);
    const int q = static_cast<int8_t>((lo[e >> 2] >> (8 * (e & 3))) & 0xFFu);
    v[e] = __int_as_float(static_cast<int>(h32) + q * 256);
  }
}

// 8 consecutive float32 or bf16 elements at element offset `off` of `base`.
__device__ __forceinline__ void ld8_f32(const void* base, size_t off, float* v) {
  const float* p = static_cast<const float*>(base) + off;
  const f32x4_t a = gld<f32x4_t>(p), b = gld<f32x4_t>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
}
__device__ __forceinline__ void st8_f32(void* base, size_t off, const float* v) {
  float* p = static_cast<float*>(base) + off;
  f32x4_t a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) { a[e] = v[e]; b[e] = v[4 + e]; }
  gst(p, a);
  gst(p + 4, b);
}
__device__ __forceinline__ void ld8_bf16(const void* base, size_t off, float* v) {
  unpack8_bf16(gld<u32x4_t>(static_cast<const uint16_t*>(base) + off), v);
}
__device__ __forceinline__ void st8_bf16(void* base, size_t off, const float* v) {
  gst(static_cast<uint16_t*>(base) + off, pack8_bf16(v));
}

template <bool F32>
__device__ __forceinline__ void ld8(const void* base, size_t off, float* v) {
  if constexpr (F32) ld8_f32(base, off, v); else ld8_bf16(base, off, v);
}
template <bool F32>
__device__ __forceinline__ void st8(void* base, size_t off, const float* v) {
  if constexpr (F32) st8_f32(base, off, v); else st8_bf16(base, off, v);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace muon

namespace muon {

// 1 / (||U||_F + eps) of one unit from its per-tile partial sums of squares,
// folded by the first 256 threads of the block in a fixed order (thread t
// takes partials t, t+256, ...; then a fixed shuffle tree and a fixed sum of
// the four wave totals), so every block that calls it, whatever its size
// (a multiple of 256 threads), gets the same bits.  `red` is 4 floats of
// shared memory.  Must be called by all threads.
__device__ __forceinline__ float unit_inv_norm(const float* partials, int n, float eps, float* red) {
  float acc = 0.f;
  if (threadIdx.x < 256)
    for (int k = threadIdx.x; k < n; k += 256) acc += gld<float>(partials + k);
  acc = wave_sum(acc);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if (wave < 4 && (threadIdx.x & 63) == 0) red[wave] = acc;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  return 1.0f / (sqrtf(tot) + eps);
}

}  // namespace muon

namespace muon {

// 8 elements of a row of a caller tensor (float32 or bf16), bounds- and
// alignment-aware: the vector path needs 16-byte alignment (`vec`) and the
// whole segment inside the row; otherwise elements are accessed one by one.
__device__ __forceinline__ void load_row8(const void* base, bool is_f32, int64_t ld, int i, int j0,
                                          int cols, bool vec, float* v) {
  const size_t off = static_cast<size_t>(i) * ld + j0;
  if (vec && j0 + 8 <= cols) {
    if (is_f32) ld8_f32(base, off, v); else ld8_bf16(base, off, v);
    return;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    v[e] = 0.f;
    if (j0 + e < cols)
      v[e] = is_f32 ? gld<float>(static_cast<const float*>(base) + off + e)
                    : bf16_to_f32(gld<uint16_t>(static_cast<const uint16_t*>(base) + off + e));
  }
}

__device__ __forceinline__ void store_row8(void* base, bool is_f32, int64_t ld, int i, int j0,
                                           int cols, bool vec, const float* v) {
  const size_t off = static_cast<size_t>(i) * ld + j0;
  if (vec && j0 + 8 <= cols) {
    if (is_f32) st8_f32(base, off, v); else st8_bf16(base, off, v);
    return;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (j0 + e < cols) {
      if (is_f32) gst(static_cast<float*>(base) + off + e, v[e]);
      else gst(static_cast<uint16_t*>(base) + off + e, f32_to_bf16(v[e]));
    }
  }
}

}  // namespace muon

namespace muon {

// Decoupled decay and the orthogonalised step for one 8-element row segment
// of a unit's weight: W' = W - lr*wd*W - lr*scale*O (Muon README, "Usage"),
// computed in float32 and stored with one rounding; O is also copied out if
// the caller asked for it.  Row i and columns j0.. are unit-local.
__device__ __forceinline__ void update_w8(const UnitDev& u, int i, int j0, const float* o,
                                          float decay, float step) {
  float w[8];
  load_row8(u.param, u.param_f32, u.ld_param, i, j0, u.cols, u.vec_param, w);
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] = w[e] - decay * w[e] - step * o[e];
  store_row8(u.param, u.param_f32, u.ld_param, i, j0, u.cols, u.vec_param, w);
  if (u.update_out) store_row8(u.update_out, true, u.ld_out, i, j0, u.cols, u.vec_out, o);
}

}  // namespace muon

namespace muon {

// update_w8 for a bf16 weight segment that was loaded ahead (whole segment
// inside the matrix, 16-byte aligned rows): the same float32 arithmetic and
// one rounding, so the result is bit-identical to update_w8's.
__device__ __forceinline__ void update_w8_loaded(const UnitDev& u, int i, int j0, const float* o, float decay,
                                                 float step, const u32x4_t& wraw) {
  float w[8];
  unpack8_bf16(wraw, w);
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] = w[e] - decay * w[e] - step * o[e];
  st8_bf16(u.param, static_cast<size_t>(i) * u.ld_param + j0, w);
  if (u.update_out) store_row8(u.update_out, true, u.ld_out, i, j0, u.cols, u.vec_out, o);
}

}  // namespace muon
