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
// host.  In the last iteration kBX applies the weight update itself
// (W' = W - lr*wd*W - lr*scale*X, Muon README "Usage") instead of storing X.
//
// Operands.  The Gram and the square are "rows x rows" products
// C[i][j] = sum_k P[i][k] Q[j][k] with both operands K-contiguous (A is
// symmetric, so A A = A A^T).  In B X the X operand is K-major (row k of X
// holds the n-direction): its tile is staged in LDS in its natural [k][j]
// layout and the MFMA fragments are read with gfx950's transposing LDS read
// (ds_read_b64_tr_b16), so no transposed copy of X is ever stored.
//
// The linear terms.  b A (square) and a X (B X) need the operand at the
// output tile's own positions.  Those values pass through the block's LDS
// anyway: A[i][j] = A[j][i] is row j, K index i of the square's second
// operand, and row i of X is K row i of B X's second operand.  While the K
// step that holds them sits in LDS, each lane reads the values of its own
// accumulator registers (MFMA output layout: four consecutive rows of one
// column per read) and adds (b/c) A or a X to the accumulators; the
// epilogue then only scales (by c, or by s).  For X this needs the int8
// correction of the bf16 master at the same positions, so the correction
// array is stored in that layout (32 x 32 blocks, 16 bytes per lane), read
// once per tile with one 16-byte load per block, and written back the same
// way from the accumulators.
//
// bf16 tile shapes (the planner picks one per matrix and phase):
//   kTileM  128 x 128 output tiles, 8 waves of 64 x 32 (2 x 1 blocks of
//           v_mfma_f32_32x32x16_bf16), 64-deep K stages in a two-stage
//           ring (64 KB of LDS): two blocks per CU, so one block's epilogue
//           overlaps the other's MFMA loop.
//   kTileL  256 x 256 output tiles, 8 waves of 128 x 64 (4 x 2 blocks, the
//           accumulators in 128 AGPRs), a 128 KB ring: one block per CU,
//           with half the operand bytes per flop of kTileM, which the
//           L2 -> LDS path needs to keep the MFMAs fed.
// The K stages are filled by direct-to-LDS loads (global_load_lds_dwordx4:
// no VGPR staging, no LDS store instructions).
// float32 path: 64x64 tile, 4 waves of 32x32, v_mfma_f32_32x32x2f32.
#include <type_traits>

#include "device_common.h"
#include "muon_internal.h"

namespace muon {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;       // LDS

// Tile configuration per precision, phase and shape.  BTM x BTN: output
// tile (rows x columns); NWM x NWN waves, each owning a (BTM/NWM) x
// (BTN/NWN) block of 32x32 MFMA tiles; BK: K depth of one LDS stage; NS:
// stages in the LDS ring (NS-1 in flight while one is consumed); OCC: the
// launch bound's minimum waves per SIMD.  DMAW: where a K step issues the
// next stage's copies: 0 right after the stage barrier, 2 after the first
// 16-deep slice of MFMAs (so the matrix pipe starts as soon as the first
// fragments arrive).  Measured: 2 makes the 256 x 256 kernels faster (4096 x
// 4096 square 102 -> 95 us, B X 120 -> 117 us per launch; GPT-2-small B X
// 106 -> 103.5 us) and the 128 x 128 ones slower (GPT-2-small Gram 60 -> 63
// us, GPT-2-XL square 1.57 -> 1.65 ms).
//   128 x 128: 8 waves of 64 x 32, 64 KB of stages, two blocks (four waves
//     per SIMD) per CU;
//   256 x 256: 8 waves of 128 x 64 (accumulators in the AGPRs), 128 KB of
//     stages, one block per CU.
// Measured alternatives, slower on every workload here: 256 x 128 with four
// waves of 128 x 64 (two blocks per CU, 32-deep stages, three of them, with
// or without the next stage's barrier moved before the last slice); 128 x
// 128 with four waves of 64 x 64; 32-deep stages with 3 or 4 in the ring.
template <bool F32, int PH, int TC> struct Cfg;
#ifndef MUON_PINGPONG
#define MUON_PINGPONG 1
#endif
template <int PH> struct Cfg<false, PH, kTileM> {
  using E = uint16_t;
  static constexpr int BTM = kTileEdgeM, BTN = kTileEdgeM, NWM = 2, NWN = 4, BK = 64, NS = 2, OCC = 2, DMAW = 0;
};
template <int PH> struct Cfg<false, PH, kTileL> {
  using E = uint16_t;
  static constexpr int BTM = kTileEdgeL, BTN = kTileEdgeL, NWM = 2, NWN = 4, BK = 64, NS = 2, OCC = 1, DMAW = 2;
};
template <int PH, int TC> struct Cfg<true, PH, TC> {
  using E = float;
  static constexpr int BTM = kTileF32, BTN = kTileF32, NWM = 2, NWN = 2, BK = 32, NS = 2, OCC = 2, DMAW = 0;
};

// LDS layout of a stage.  Tiles are stored unpadded as rows of 16-byte
// chunks, with the chunk order of each row XOR-swizzled so the MFMA
// fragment reads are free of bank conflicts.  gfx950's LDS serves 256 bytes
// per clock, i.e. a 16-byte read of 16 lanes at a time:
//   K-contiguous tile (row = M or N index, 8 chunks of K, 128 bytes): chunk
//     c of row r sits at position c ^ ((r / 2) % 8) (with 32-deep stages,
//     rows of 4 chunks: c ^ ((r / 4) % 4)).  Sixteen consecutive
//     rows read at one chunk then cover the 16 distinct 16-byte slots of a
//     256-byte bank line (the two rows sharing a line differ in r % 2, and
//     the eight of one parity in (r / 2) % 8); c ^ (r % 8) would put rows r
//     and r + 8 in one slot (a 2-way conflict, measured with the LDS bank
//     conflict counter);
//   K-major tile of B X (row = k, 16 or 32 chunks of columns): chunk c of
//     row k sits at position c ^ 4 (k % 4), which spreads the four rows a
//     transposing read touches over distinct banks.
template <int CPR>
__device__ __forceinline__ int swz_kc(int r, int c) {
  static_assert(CPR == 8 || CPR == 4, "K rows of 8 or 4 chunks");
  if constexpr (CPR == 8) return c ^ ((r >> 1) & 7);
  else return c ^ ((r >> 2) & 3);   // 64-byte rows: four share a bank line
}
__device__ __forceinline__ int swz_km(int k, int c) { return c ^ ((k & 3) << 2); }

// Wait until at most N vector-memory operations of this wave are pending
// (asm, so the compiler, which does not see the asm loads, keeps it).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for the stage ring.  A __syncthreads fence would also
// wait for every direct-to-LDS load in flight (they count as LDS writes)
// and drain the ring; here each wave only completes its own LDS reads
// (lgkmcnt(0): the buffer refilled after the barrier was read before it),
// and callers wait for the loads they need with wait_vmcnt.  The asm
// memory clobbers keep the compiler from moving memory accesses across.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Orders one wave's LDS writes before its other lanes read them back (the
// epilogue's staging area is private to the wave): a release and an acquire
// fence at wavefront scope around a wave barrier, so neither the compiler
// nor the hardware lets a read move above the writes it depends on.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Transposing LDS read (gfx950).  Within each 16-lane group the 8-byte words
// addressed by the lanes form a 16 x 4 matrix W[lane][e]; lane i receives
// W[4e + i/4][i%4] for e = 0..3.  If lane 4e+q points at X[k+e][j+4q..+3],
// lane i therefore gets X[k+e][j+i], e = 0..3: four consecutive k of one
// column, which is what an MFMA operand lane holds.
__device__ __forceinline__ bf16x4_t lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
}

// Direct-to-LDS loads of one stage (global_load_lds_dwordx4): instruction i
// of wave w (of NW) fills the 1 KB at chunk (i*NW + w)*64 of the tile, lane
// L writing chunk +L; aoff/boff hold each lane's byte offset of the global
// chunk that belongs there for i = 0 (swizzle included).  Instruction i
// lands NW*64 chunks further, a whole number of rows whose swizzle repeats,
// so its global chunk is the same offset from a base advanced by astep /
// bstep bytes (one VGPR per operand instead of one per instruction).  No
// VGPR holds the data and no LDS store instruction is issued.
//
// The instruction is written as inline asm (it has no register result): the
// compiler treats the builtin form as an LDS store and puts a wait for every
// outstanding vector-memory operation in front of the next LDS read, which
// would drain the ring.  The stage waits are therefore explicit
// (wait_vmcnt), and the asm's memory clobber keeps LDS accesses in order
// around it.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}

template <int NA, int NB, int NW, typename E>
__device__ __forceinline__ void issue_stage(const E* ga, const E* gb, uint32_t aoff, uint32_t boff, size_t astep,
                                            size_t bstep, uint32_t la, uint32_t lb, int wave, bool with_b) {
#pragma unroll
  for (int i = 0; i < NA; ++i)
    dma16(reinterpret_cast<const char*>(ga) + i * astep, aoff, la + (i * NW + wave) * 1024);
  if (with_b) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
      dma16(reinterpret_cast<const char*>(gb) + i * bstep, boff, lb + (i * NW + wave) * 1024);
  }
}

// LDS byte address of a shared-memory pointer.
template <typename E>
__device__ __forceinline__ uint32_t lds_addr(const E* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const E*)(p)));
}

// The lane's index in its wave, from the lane masks rather than the thread
// index: the epilogue recomputes its lane-derived offsets from it instead of
// keeping the K loop's copies alive through the loop (which spilled them).
__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time (a
// loop left rolled would index the accumulator array at run time and move
// it to scratch memory).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Fragments of one 16-deep K slice (bf16) for the wave's blocks.
template <bool KMAJOR_B, int NBM, int NBN, int WTM, int WTN, int BK, int BTN>
__device__ __forceinline__ void load_frags(const uint16_t* la, const uint16_t* lb, int ks, int lane, int wm, int wn,
                                           bf16x8_t (&fa)[NBM], bf16x8_t (&fb)[NBN]) {
  const int kc = ks * 2 + (lane >> 5);           // 16-byte chunk of K (8 bf16)
#pragma unroll
  for (int i = 0; i < NBM; ++i) {
    const int r = wm * WTM + i * 32 + (lane & 31);
    fa[i] = *reinterpret_cast<const bf16x8_t*>(&la[r * BK + swz_kc<BK / 8>(r, kc) * 8]);
  }
#pragma unroll
  for (int j = 0; j < NBN; ++j) {
    if constexpr (!KMAJOR_B) {
      const int r = wn * WTN + j * 32 + (lane & 31);
      fb[j] = *reinterpret_cast<const bf16x8_t*>(&lb[r * BK + swz_kc<BK / 8>(r, kc) * 8]);
    } else {
      // lane group g = lane/16 covers columns 16*(g%2).. and k-half g/2;
      // lane r of the group points at row k + r/4, columns 4*(r%4)..
      const int g = lane >> 4, r = lane & 15;
      const int krow = ks * 16 + 8 * (g >> 1) + (r >> 2);
      const int col = wn * WTN + j * 32 + 16 * (g & 1) + 4 * (r & 3);
      const int cofs = swz_km(krow, col >> 3) * 8 + (col & 7);   // rows krow and krow+4 swizzle alike
      const bf16x4_t lo = lds_read_tr(&lb[krow * BTN + cofs]);
      const bf16x4_t hi = lds_read_tr(&lb[(krow + 4) * BTN + cofs]);
      fb[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
}

// MFMAs of one BK-deep stage held in LDS (la: K-contiguous A tile, BTM rows
// of BK; lb: the B tile, K-contiguous like A or K-major, BK rows of BTN).
// The wave owns rows wm*WTM.. and columns wn*WTN.. of the block tile, as
// NBM x NBN tiles of 32x32.  bf16: the fragments of slice ks+1 are read
// before the MFMAs of slice ks are issued, and a scheduling barrier keeps
// the compiler from hoisting further slices, so the LDS reads overlap the
// MFMAs while only two slices' fragments occupy registers.  (Interleaving
// each read with an MFMA through scheduling-group barriers was measured:
// no faster with 64 x 32 wave tiles, 20 % slower with 128 x 64.)
template <bool F32, bool KMAJOR_B, int NBM, int NBN, int WTM, int WTN, int BK, int BTN, int WHEN = 0, typename E,
          typename H>
__device__ __forceinline__ void mma_stage(const E* la, const E* lb, f32x16_t (&acc)[NBM][NBN], int lane, int wm,
                                          int wn, H&& mid) {
  if constexpr (!F32) {
    constexpr int NKS = BK / 16;
    bf16x8_t fa[2][NBM], fb[2][NBN];
    load_frags<KMAJOR_B, NBM, NBN, WTM, WTN, BK, BTN>(la, lb, 0, lane, wm, wn, fa[0], fb[0]);
    if constexpr (WHEN == 1) {
      __builtin_amdgcn_sched_barrier(0);
      mid();
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (ks + 1 < NKS)
        load_frags<KMAJOR_B, NBM, NBN, WTM, WTN, BK, BTN>(la, lb, ks + 1, lane, wm, wn, fa[(ks + 1) & 1],
                                                         fb[(ks + 1) & 1]);
#pragma unroll
      for (int i = 0; i < NBM; ++i)
#pragma unroll
        for (int j = 0; j < NBN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks & 1][i], fb[ks & 1][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (WHEN == 2) {
        if (ks == 0) {
          mid();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  } else {
    if constexpr (WHEN != 0) mid();
    // v_mfma_f32_32x32x2f32: lane half h holds k = h*16 + e at step e of the
    // 32-deep slab, for both operands
    const int k0 = (lane >> 5) * 16;
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      f32x4_t fa[NBM], fb[NBN];
      const int kc = (k0 >> 2) + kq;                 // 16-byte chunk of K (4 floats)
#pragma unroll
      for (int i = 0; i < NBM; ++i) {
        const int r = wm * WTM + i * 32 + (lane & 31);
        fa[i] = *reinterpret_cast<const f32x4_t*>(&la[r * BK + swz_kc<BK / 4>(r, kc) * 4]);
      }
#pragma unroll
      for (int j = 0; j < NBN; ++j) {
        if constexpr (!KMAJOR_B) {
          const int r = wn * WTN + j * 32 + (lane & 31);
          fb[j] = *reinterpret_cast<const f32x4_t*>(&lb[r * BK + swz_kc<BK / 4>(r, kc) * 4]);
        } else {
          const int col = wn * WTN + j * 32 + (lane & 31);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int k = k0 + kq * 4 + e;
            fb[j][e] = lb[k * BTN + swz_km(k, col >> 2) * 4 + (col & 3)];
          }
        }
      }
#pragma unroll
      for (int i = 0; i < NBM; ++i)
#pragma unroll
        for (int j = 0; j < NBN; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][e], fb[j][e], acc[i][j], 0, 0, 0);
    }
  }
}

// An accumulator element, read in the epilogue.  The 128 accumulators of a
// 128 x 64 wave tile live in the AGPRs; reading them through an asm operand
// that must be an AGPR keeps them there until each is read (left to itself
// the register allocator copies them all to VGPRs where the K loop ends,
// which spills).  The compiler's hazard check does not cover these reads,
// so the epilogue first waits out the MFMA latency.  Smaller wave tiles keep
// their accumulators in VGPRs and read them plainly, as do the folds inside
// the K loop (the compiler then inserts the waits it needs).
template <bool AGPR>
__device__ __forceinline__ float acc_get(const f32x16_t& v, int r) {
  if constexpr (AGPR) {
    float x;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(x) : "a"(v[r]));
    return x;
  } else {
    return v[r];
  }
}

// MFMA 32x32 output layout: lane l, register r holds row 8*(r/4) + 4*(l/32)
// + r%4, column l%32 of its 32x32 block.  The "linear term" folds below read
// the operand in that layout: for r = 4q..4q+3 the four rows
// 8q + 4(l/32) + 0..3 of column l%32.

// B X: acc += a * X at the wave's output positions, during the K step that
// holds the block's rows of X (the K-major second operand, BK rows of BTN).
// bf16: X = the master hi (read from LDS with the transposing read) plus its
// int8 correction (xq: the part's blocks, loaded from the correction array
// one K step ahead).
// PART (a compile-time constant, so no branch joins accumulator blocks) is
// the wave's fold in this step: the block rows i whose 32 rows lie in the
// PART-th K step of the wave's rows (BK / 32 of them per step).  Each quad
// of rows is read, widened and added before the next, so few registers
// beside the accumulators are live.
template <int PART, bool F32, bool AGPR, int NBM, int NBN, int WTM, int WTN, int BK, int BTN, typename E>
__device__ __forceinline__ void fold_master(const E* lbx, int wn, int lane, float a,
                                            const u32x4_t (&xq)[BK / 32][NBN], f32x16_t (&acc)[NBM][NBN]) {
  static_assert(WTM % BK == 0, "a wave's rows start on a K step");
  static_for<0, NBM>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if constexpr ((i * 32) / BK == PART) {
      constexpr int kr = (i * 32) % BK;              // the block's first row inside the stage
#pragma unroll
      for (int j = 0; j < NBN; ++j) {
        const int c0 = wn * WTN + j * 32;
        if constexpr (!F32) {
          const int g = lane >> 4, r = lane & 15;
          const int col = c0 + 16 * (g & 1) + 4 * (r & 3);
          u32x2_t hw[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            // the four bf16 values as two words (element e in half e%2 of
            // word e/2)
            const int krow = kr + 8 * q + 4 * (g >> 1) + (r >> 2);
            hw[q] = __builtin_bit_cast(u32x2_t,
                                       lds_read_tr(&lbx[krow * BTN + swz_km(krow, col >> 3) * 8 + (col & 7)]));
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t qw = xq[i - PART * (BK / 32)][j][q];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t hb = (e & 1) ? (hw[q][e >> 1] & 0xFFFF0000u) : (hw[q][e >> 1] << 16);
              const int qq = static_cast<int8_t>((qw >> (8 * e)) & 0xFFu);
              const float x = __int_as_float(static_cast<int>(hb) + qq * 256);
              acc[i][j][4 * q + e] = fmaf(a, x, acc[i][j][4 * q + e]);
            }
            // AGPR accumulators: a quad at a time through the VGPRs
            if constexpr (AGPR) __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          const int col = c0 + (lane & 31);
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int krow = kr + 8 * q + 4 * (lane >> 5) + e;
              const float x = lbx[krow * BTN + swz_km(krow, col >> 2) * 4 + (col & 3)];
              acc[i][j][4 * q + e] = fmaf(a, x, acc[i][j][4 * q + e]);
            }
        }
      }
    }
  });
}

// B = b A + c A A: acc += (b/c) A at the wave's output positions (the
// epilogue scales by c).  A[i][j] = A[j][i]: row j of the second operand
// (K-contiguous, BK columns of K per row), K index i, so during the K step
// that holds k = the block's rows each lane reads four consecutive k of its
// column's row.  PART as for fold_master.
template <int PART, bool F32, bool AGPR, int NBM, int NBN, int WTM, int WTN, int BK, typename E>
__device__ __forceinline__ void fold_atile(const E* lb, int wn, int lane, float bc, f32x16_t (&acc)[NBM][NBN]) {
  constexpr int EPE = 16 / sizeof(E);        // elements per 16-byte chunk
  static_assert(WTM % BK == 0, "a wave's rows start on a K step");
  static_for<0, NBM>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if constexpr ((i * 32) / BK == PART) {
      constexpr int kr = (i * 32) % BK;
#pragma unroll
      for (int j = 0; j < NBN; ++j) {
        const int brow = wn * WTN + j * 32 + (lane & 31);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int k = kr + 8 * q + 4 * (lane >> 5);      // first of four consecutive k
          const int pos = brow * BK + swz_kc<BK / EPE>(brow, k / EPE) * EPE + (k % EPE);
          float x[4];
          if constexpr (!F32) {
            const u32x2_t w = *reinterpret_cast<const u32x2_t*>(&lb[pos]);
            x[0] = __uint_as_float(w[0] << 16);
            x[1] = __uint_as_float(w[0] & 0xFFFF0000u);
            x[2] = __uint_as_float(w[1] << 16);
            x[3] = __uint_as_float(w[1] & 0xFFFF0000u);
          } else {
            const f32x4_t w = *reinterpret_cast<const f32x4_t*>(&lb[pos]);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = w[e];
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] = fmaf(bc, x[e], acc[i][j][4 * q + e]);
          if constexpr (AGPR) __builtin_amdgcn_sched_barrier(0);   // a quad at a time
        }
      }
    }
  });
}

// One 32x32 block of a 32-row strip (block column j; v: the lane's 16
// values in accumulator register order) into the wave's LDS staging area in
// row-major order (pitch EPP floats).
template <int EPP>
__device__ __forceinline__ void stage_block(const float* v, int j, float* ep, int lane) {
#pragma unroll
  for (int r = 0; r < 16; ++r) ep[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * EPP + j * 32 + (lane & 31)] = v[r];
}

// The next bf16 master as B X writes it, from one 32x32 block of
// accumulators (16 values per lane in register order, already scaled): with
// y = bits(x) + 0x8080, hi = the upper half of y (x rounded to bf16 half-up
// with the threshold 1/256 ulp below the tie, so within a bf16 half-ulp plus
// 2^-8 of one) and the int8 correction q = byte 1 of y, xor 0x80.  Then
// d = bits(x) - bits(hi) = (y mod 2^16) - 0x8080 lies in [-32896, 32639] and
// q = floor((d + 128) / 256) in [-128, 127]: the decode bits(hi) + 256 q
// (master_decode8, the folds) lands within 128 float32 ulps of x, as with
// the round-to-nearest-even encoding of master_encode8, for either sign and
// across binades (bit-pattern arithmetic).  y replaces x in place; the
// function returns the 16 correction bytes in register order.
__device__ __forceinline__ u32x4_t encode_master16(float* v) {
  uint32_t y[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    y[r] = __float_as_uint(v[r]) + 0x8080u;
    v[r] = __uint_as_float(y[r]);
  }
  u32x4_t out;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    // byte 1 of y0, y1 (then y2, y3) into bytes 0, 1; then the two halves
    const uint32_t lo = __builtin_amdgcn_perm(y[4 * w + 1], y[4 * w], 0x0c0c0501u);
    const uint32_t hi = __builtin_amdgcn_perm(y[4 * w + 3], y[4 * w + 2], 0x0c0c0501u);
    out[w] = __builtin_amdgcn_perm(hi, lo, 0x05040100u) ^ 0x80808080u;
  }
  return out;
}

// Eight staged y patterns (encode_master16) to their eight bf16 hi halves,
// element 2e in the low half of word e.
__device__ __forceinline__ u32x4_t pack8_hi(const float* v) {
  u32x4_t w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = __builtin_amdgcn_perm(__float_as_uint(v[2 * e + 1]), __float_as_uint(v[2 * e]), 0x07060302u);
  return w;
}

template <bool F32, int PH, int TC, bool LAST>
__global__ __launch_bounds__((64 * Cfg<F32, PH, TC>::NWM * Cfg<F32, PH, TC>::NWN), (Cfg<F32, PH, TC>::OCC))
void ns_gemm_kernel(const UnitDev* __restrict__ units, const GemmTask* __restrict__ tasks, GemmParams p) {
  using C = Cfg<F32, PH, TC>;
  using E = typename C::E;
  constexpr int BTM = C::BTM, BTN = C::BTN, BK = C::BK, NWM = C::NWM, NWN = C::NWN;
  constexpr int NT = 64 * NWM * NWN;               // threads per block
  constexpr int WTM = BTM / NWM, WTN = BTN / NWN;  // wave tile
  constexpr int NBM = WTM / 32, NBN = WTN / 32;    // 32x32 MFMA tiles per wave
  constexpr bool KMAJOR_B = PH == kBX;             // X operand of B X is K-major
  constexpr int NS = C::NS;
  constexpr int EPE = 16 / sizeof(E);              // elements per 16-byte chunk
  constexpr int CPR = BK / EPE;                    // chunks per K-contiguous row
  constexpr int CPRX = BTN / EPE;                  // chunks per K-major row
  constexpr int T_A = BTM * BK, T_B = BTN * BK;    // the two operand tiles (elements)
  constexpr int NIA = T_A / EPE / NT;              // DMA instructions per lane per A tile
  constexpr int NIB = T_B / EPE / NT;              // ... and per B tile
  constexpr int STAGE = T_A + T_B;                 // A tile then B tile
  constexpr int EPP = WTN + 8;                     // epilogue LDS pitch (floats)
  constexpr int NFOLD = WTM / BK;                  // K steps holding a wave's rows (B X, square)
  constexpr bool FOLD = PH == kBX || PH == kSquare;
  // ping-pong K loop: the Gram phase of 256 x 256 tiles (one block per CU,
  // two groups of four waves, one wave of each on every SIMD).  Measured on
  // 4096 x 4096: Gram 101 -> 91 us per launch; the square and B X phases,
  // whose memory phases carry the fold (and for B X twice the LDS read
  // instructions: transposing 8-byte reads), ran 3 % faster and 25 % slower
  // and keep the plain loop.
  constexpr bool PING = !F32 && TC == kTileL && PH == kGram && MUON_PINGPONG;
  static_assert(!PING || (NS == 2 && NWM == 2 && NWN == 4 && BK % 32 == 0 && !FOLD), "ping-pong layout");
  constexpr bool AGPR = NBM * NBN >= 8;            // accumulators in the AGPRs (128 x 128 wave tiles)
  static_assert(NIA * NT * EPE == T_A && NIB * NT * EPE == T_B, "tile/thread mismatch");
  static_assert((CPR == 8 || CPR == 4) && (CPRX == 16 || CPRX == 32),
                "swizzles assume 8- or 4-chunk K rows and 16- or 32-chunk K-major rows");
  static_assert(BK % 32 == 0 && WTM % BK == 0 && NFOLD >= 1 && NFOLD <= 4, "a wave's rows fill whole K steps");
  static_assert(NWM * NWN * 32 * EPP * 4 <= NS * STAGE * static_cast<int>(sizeof(E)),
                "epilogue staging must fit in the operand LDS");
  static_assert(!LAST || PH == kBX, "only B X has a last-iteration variant");

  __shared__ __attribute__((aligned(16))) E smem[NS * STAGE];
  __shared__ float red[4];

  const GemmTask t = tasks[blockIdx.x];
  if (t.unit < 0) return;   // padding of the XCD-interleaved task order
  const UnitDev& u = units[t.unit];
  const int mp = u.mp, np = u.np;
  const int ti = t.ti, tj = t.tj;
  if constexpr (MUON_DEBUG_BOUNDS) {
    // debug build: the tile and its K extent lie inside the unit's padded
    // operands, and the symmetric products list upper tiles only
    const int out_cols = PH == kBX ? np : mp, kext = PH == kGram ? np : mp;
    const bool ok = ti >= 0 && tj >= 0 && (ti + 1) * BTM <= mp && (tj + 1) * BTN <= out_cols && kext >= BK &&
                    kext % BK == 0 && (PH == kBX || ti <= tj);
    if (!ok) {
      if (threadIdx.x == 0) atomicOr(p.flags, kFlagBounds);
      return;
    }
  }

  // The epilogue's scale, known before the K loop (so no control flow
  // joins while the accumulators are live).  The first Gram folds the
  // per-tile partial sums into s = 1/(||U|| + eps) (every block in the same
  // order; tile (0, 0) stores it) and scales by s^2.  The square scales by
  // c, in the first iteration by c s: B' = s B, so that the first B X,
  // s (a X + B X) = (s a) X + B' X, only needs s in the fold's coefficient
  // and its epilogue (which runs with its block alone on the CU at 256 x
  // 256) multiplies nothing.
  float scale = 1.f;
  float a_fold = p.a;                                // B X: coefficient of the a X fold
  if constexpr (PH == kGram) {
    if (p.first) {
      const float iv = unit_inv_norm(u.partials, u.k1_ntiles, p.eps, red);
      scale = iv * iv;
      if (ti == 0 && tj == 0 && threadIdx.x == 0) gst(u.norm, iv);
    }
  } else if constexpr (PH == kSquare) {
    scale = p.first ? p.c * gld<float>(u.norm) : p.c;
  } else {
    if (p.first) a_fold = p.a * gld<float>(u.norm);
  }

  // operand A: rows [ti*BTM, +BTM) over K; operand B: rows [tj*BTN, +BTN)
  // over K (Gram, square) or K rows x columns [tj*BTN, +BTN) (B X)
  const E* pa;
  const E* pb;
  int lda_g, ldb_g, K;
  const E* xcur = static_cast<const E*>(u.xh[p.x_in]);
  if constexpr (PH == kGram) {
    pa = xcur + static_cast<size_t>(ti) * BTM * np;
    pb = xcur + static_cast<size_t>(tj) * BTN * np;
    lda_g = ldb_g = np; K = np;
  } else if constexpr (PH == kSquare) {
    pa = static_cast<const E*>(u.a) + static_cast<size_t>(ti) * BTM * mp;
    pb = static_cast<const E*>(u.a) + static_cast<size_t>(tj) * BTN * mp;
    lda_g = ldb_g = mp; K = mp;
  } else {
    pa = static_cast<const E*>(u.b) + static_cast<size_t>(ti) * BTM * mp;
    pb = xcur + static_cast<size_t>(tj) * BTN;
    lda_g = mp; ldb_g = np; K = mp;
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / NWN, wn = wave % NWN;
  const int row_base = ti * BTM + wm * WTM;
  const int col_base = tj * BTN + wn * WTN;

  // B X, bf16: the int8 corrections of the X master at the wave's output
  // blocks (correction array: 32 x 32 blocks of 1 KB, row of blocks after
  // row of blocks, 16 bytes per lane in accumulator register order).  Only
  // one fold part's blocks are held at a time (XPP block rows): each part's
  // are requested a K step ahead, after the previous part's fold.
  constexpr int XPP = BK / 32;
  u32x4_t xq[XPP][NBN];
  auto load_xq = [&](auto partc) {
    constexpr int P = decltype(partc)::value;
    if constexpr (PH == kBX && !F32 && P < WTM / BK) {
      const int8_t* xl = static_cast<const int8_t*>(u.xl);
      const size_t nbc = static_cast<size_t>(np / 32);
#pragma unroll
      for (int i = 0; i < XPP; ++i)
#pragma unroll
        for (int j = 0; j < NBN; ++j) {
          const size_t bi = (row_base + (P * XPP + i) * 32) / 32, bj = (col_base + j * 32) / 32;
          xq[i][j] = gld<u32x4_t>(xl + (bi * nbc + bj) * 1024 + lane * 16);
        }
    }
  };

  // each lane's global byte offset (within a stage) of its first DMA chunk
  // per operand, and the advance of the global base per instruction (NW*64
  // chunks: whole rows, a multiple of the swizzle period of 16 K-contiguous
  // rows or 4 K-major rows)
  constexpr int NW = NWM * NWN;
  static_assert((NW * 64 / CPR) % 16 == 0 && (NW * 64 / CPRX) % 4 == 0 && 64 % CPRX == 0,
                "DMA instructions advance by whole swizzle periods");
  uint32_t aoff, boff;
  {
    const int c = wave * 64 + lane;                  // chunk position in the A tile
    const int ar = c / CPR;
    aoff = static_cast<uint32_t>((ar * lda_g + swz_kc<CPR>(ar, c % CPR) * EPE) * sizeof(E));
    if constexpr (KMAJOR_B) {
      const int k = c / CPRX;
      boff = static_cast<uint32_t>((k * ldb_g + swz_km(k, c % CPRX) * EPE) * sizeof(E));
    } else {
      boff = static_cast<uint32_t>((ar * ldb_g + swz_kc<CPR>(ar, c % CPR) * EPE) * sizeof(E));
    }
  }
  const size_t astep = static_cast<size_t>(NW * 64 / CPR) * lda_g * sizeof(E);
  const size_t bstep = static_cast<size_t>(KMAJOR_B ? NW * 64 / CPRX : NW * 64 / CPR) * ldb_g * sizeof(E);
  const uint32_t ring0 = lds_addr(smem);
  // diagonal tiles of the Gram and the square read the same rows as both
  // operands: the stage is loaded once and both fragment reads use it
  const bool diag = (PH == kGram || PH == kSquare) && ti == tj;
  // advance per K step: along the rows for K-contiguous tiles, down BK rows
  // for the K-major tile
  const size_t a_step = BK;
  const size_t b_step = KMAJOR_B ? static_cast<size_t>(BK) * ldb_g : BK;

  f32x16_t acc[NBM][NBN];
#pragma unroll
  for (int i = 0; i < NBM; ++i)
#pragma unroll
    for (int j = 0; j < NBN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = K / BK;
  const float bc = p.b / p.c;                        // square: b A folded as (b/c) A, scaled by c

  // The epilogue's 32-row strips: SEGS segments of 8 per row, RITER per lane
  // (row pass) and CITER per lane (column pass: mirror tiles, weight rows of
  // a tall matrix).
  constexpr int SEGS = WTN / 8;
  constexpr int RITER = 32 * SEGS / 64;
  constexpr int CITER = WTN * 4 / 64;
  static_assert(RITER == CITER, "row and column passes give a lane equally many segments");
  // Last B X, bf16 weights with aligned rows: the weight segments of every
  // strip (rows of W for a wide unit; columns of the tile, i.e. rows of W,
  // for a tall one) are requested together as the K loop ends, so the
  // strips wait on one HBM latency instead of one each (the K loop's
  // registers are free by then; the epilogue holds NBM * RITER segments).
  const bool wfast = LAST && !F32 && !u.param_f32 && u.vec_param;
  auto wseg = [&](int pi, int q, int ln, int& wi, int& wj) {
    const int sg = ln + 64 * q;
    if (u.side == kLeft) {
      wi = row_base + pi * 32 + sg / SEGS;
      wj = col_base + (sg % SEGS) * 8;
    } else {
      wi = col_base + sg % WTN;
      wj = row_base + pi * 32 + (sg / WTN) * 8;
    }
  };
  u32x4_t wbuf[NBM][RITER];
  auto load_w = [&](int pi, int ln, u32x4_t (&dst)[RITER]) {
#pragma unroll
    for (int q = 0; q < RITER; ++q) {
      int wi, wj;
      wseg(pi, q, ln, wi, wj);
      if (wi < u.rows && wj + 8 <= u.cols)
        dst[q] = gld<u32x4_t>(static_cast<const uint16_t*>(u.param) + static_cast<size_t>(wi) * u.ld_param + wj);
    }
  };

  // K pipeline: a ring of NS stages filled by direct-to-LDS loads.  Step kt
  // waits for its own stage (the stages issued after it may stay in
  // flight), passes a barrier (every wave's part of the stage has landed,
  // and every wave is done with step kt-1, whose buffer is refilled next),
  // issues stage kt+NS-1 into that buffer and runs the MFMAs of stage kt.
  // With more than two stages, indices past the end are clamped to the last
  // stage (its copy lands in a buffer nobody reads again), so every step has
  // the same NS-2 newer stages in flight and a fixed wait count.  With two
  // stages every step waits for everything, so the last step issues no copy.
  //
  // The linear term is folded during the NFOLD steps that hold the wave's
  // own rows (B X: rows of X; square: K indices of A).
  constexpr uint32_t STAGE_B = STAGE * sizeof(E), TILE_B = T_A * sizeof(E);
  using NoFold = std::integral_constant<int, -1>;
  auto nohook = [] {};
  if constexpr (PING) {
    // Ping-pong (256 x 256 tiles, one block per CU).  The two waves sharing
    // a SIMD belong to different groups (wave w runs on SIMD w % 4; group =
    // the wave's row half wm), and the groups alternate, one phase apart,
    // between MFMA phases (half a stage: NKS/2 slices of MFMAs from
    // registers) and memory phases (the fragment reads of the next half
    // stage, copy issue and waits, the fold), with a block barrier between
    // phases: at every moment one group feeds the matrix pipe while the
    // other prepares, instead of both idling at each stage's barrier.
    //   phase 4k   (memory): issue stage k+1 (its buffer's last reader, the
    //              other group, finished before this phase's barrier);
    //              read slices of half 0 of stage k;
    //   phase 4k+1 (MFMA)  : half 0;
    //   phase 4k+2 (memory): wait for this wave's part of stage k+1; read
    //              half 1;
    //   phase 4k+3 (MFMA)  : half 1.
    // Group 1 starts one barrier later and skips the last one, so both pass
    // the same number of barriers.  Every memory phase ends with its reads
    // complete (lgkmcnt(0) in the barrier), so a stage is visible to all
    // after the barrier that follows both groups' waits for it, and free
    // once both groups' last reads of it precede a barrier.
    constexpr int HALF = BK / 32;   // slices per half stage
    bf16x8_t fa[HALF][NBM], fb[HALF][NBN];
    auto read_half = [&](const E* cs, const E* csb, int h) {
#pragma unroll
      for (int q = 0; q < HALF; ++q)
        load_frags<KMAJOR_B, NBM, NBN, WTM, WTN, BK, BTN>(reinterpret_cast<const uint16_t*>(cs),
                                                         reinterpret_cast<const uint16_t*>(csb), h * HALF + q, lane,
                                                         wm, wn, fa[q], fb[q]);
    };
    auto mfma_half = [&]() {
#pragma unroll
      for (int q = 0; q < HALF; ++q)
#pragma unroll
        for (int i = 0; i < NBM; ++i)
#pragma unroll
          for (int j = 0; j < NBN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[q][i], fb[q][j], acc[i][j], 0, 0, 0);
    };
    auto phase_barrier = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      ring_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    auto pstage = [&](int k) {
      const E* cs = smem + (k & 1) * STAGE;
      const E* csb = diag ? cs : cs + T_A;
      if (k + 1 < KT) {
        const uint32_t ls = ring0 + ((k + 1) & 1) * STAGE_B;
        issue_stage<NIA, NIB, NW, E>(pa + (k + 1) * a_step, pb + (k + 1) * b_step, aoff, boff, astep, bstep, ls,
                                     ls + TILE_B, wave, !diag);
      }
      read_half(cs, csb, 0);
      phase_barrier();
      mfma_half();
      phase_barrier();
      wait_vmcnt<0>();
      read_half(cs, csb, 1);
      phase_barrier();
      mfma_half();
      if (wm == 0 || k + 1 < KT) phase_barrier();
    };
    issue_stage<NIA, NIB, NW, E>(pa, pb, aoff, boff, astep, bstep, ring0, ring0 + TILE_B, wave, !diag);
    wait_vmcnt<0>();
    ring_barrier();
    if (wm == 1) phase_barrier();
    for (int kt = 0; kt < KT; ++kt) pstage(kt);
  } else {
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) {
    const int sc = min(s, KT - 1);
    issue_stage<NIA, NIB, NW, E>(pa + sc * a_step, pb + sc * b_step, aoff, boff, astep, bstep, ring0 + s * STAGE_B,
                             ring0 + s * STAGE_B + TILE_B, wave, !diag);
  }
  // One K step; FP >= 0: the step holding part FP of the wave's own rows,
  // which also folds the linear term.  `hook` runs once the step's copy is
  // issued.
  auto kstep = [&](int kt, auto fpc, auto&& hook) {
    constexpr int FP = decltype(fpc)::value;
    if (diag) wait_vmcnt<(NS - 2) * NIA>();   // newer stages in flight: NS-2 of one operand each
    else wait_vmcnt<(NS - 2) * (NIA + NIB)>();
    ring_barrier();
    auto issue = [&] {
      if (NS > 2 || kt + 1 < KT) {   // with two stages the last step issues no copy
        const int nx = min(kt + NS - 1, KT - 1);
        const uint32_t ls = ring0 + ((kt + NS - 1) % NS) * STAGE_B;
        issue_stage<NIA, NIB, NW, E>(pa + nx * a_step, pb + nx * b_step, aoff, boff, astep, bstep, ls, ls + TILE_B,
                                     wave, !diag);
      }
    };
    if constexpr (C::DMAW == 0) issue();
    hook();
    const E* cs = smem + (kt % NS) * STAGE;
    const E* csb = diag ? cs : cs + T_A;
    if constexpr (FP >= 0) {
      if constexpr (PH == kBX) {
        fold_master<FP, F32, AGPR, NBM, NBN, WTM, WTN, BK, BTN>(csb, wn, lane, a_fold, xq, acc);
        load_xq(std::integral_constant<int, FP + 1>{});
      } else {
        fold_atile<FP, F32, AGPR, NBM, NBN, WTM, WTN, BK>(csb, wn, lane, bc, acc);
      }
    }
    mma_stage<F32, KMAJOR_B, NBM, NBN, WTM, WTN, BK, BTN, C::DMAW>(cs, csb, acc, lane, wm, wn, issue);
  };
  if constexpr (FOLD) {
    // the wave's rows are K steps f0 .. f0 + NFOLD - 1 (K index = tile row);
    // all waves pass the same steps and barriers, each with its own split
    const int f0 = (ti * BTM + wm * WTM) / BK;
    using Part0 = std::integral_constant<int, 0>;
    if (f0 == 0) load_xq(Part0{});
    for (int kt = 0; kt + 1 < f0; ++kt) kstep(kt, NoFold{}, nohook);
    if (f0 > 0) kstep(f0 - 1, NoFold{}, [&] { load_xq(Part0{}); });
    static_for<0, NFOLD>([&](auto pc) { kstep(f0 + decltype(pc)::value, pc, nohook); });
    for (int kt = f0 + NFOLD; kt < KT; ++kt) kstep(kt, NoFold{}, nohook);
  } else {
    for (int kt = 0; kt < KT; ++kt) kstep(kt, NoFold{}, nohook);
  }
  }
  const int el = lane_id();   // the epilogue's lane index
  if (wfast) static_for<0, NBM>([&](auto pc) { load_w(decltype(pc)::value, el, wbuf[decltype(pc)::value]); });
  if constexpr (PING) {
    // nothing in flight, every read of the ring done: group 0 passed the
    // last barrier after group 1's last reads, and group 1 (in its last
    // MFMA phase) reads no LDS while group 0 stages its epilogue
  } else if constexpr (NS == 2) {
    ring_barrier();    // no copy in flight; every wave is done reading the ring
  } else {
    wait_vmcnt<0>();   // the clamped copies of the last stage
    __syncthreads();   // the epilogue reuses the ring as staging
  }

  // ---------------------------------------------------------------- epilogue
  // The epilogue reads AGPR accumulators with inline asm, which the
  // compiler's hazard check does not see: wait out the MFMA result latency
  // first (24 wait states; the scheduling barriers keep every MFMA above the
  // wait and every read below it).
  if constexpr (AGPR) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Gram and square: the tiles above the diagonal are also stored transposed
  const bool mirror = PH == kBX ? (LAST && u.side == kRight) : (ti != tj);
  const float decay = p.lr * p.weight_decay;
  const float step = p.lr * u.lr_scale;
  float* ep = reinterpret_cast<float*>(smem) + wave * (32 * EPP);
  // the output pointers, kept in scalar registers for the whole epilogue;
  // so are the weight fields of the last iteration's update (wu: a copy of
  // the descriptor whose fields the update reads are pinned)
  void* const out_ab = PH == kGram ? sreg_ptr(u.a) : PH == kSquare ? sreg_ptr(u.b) : nullptr;
  void* const out_xh = PH == kBX ? sreg_ptr(u.xh[p.x_in ^ 1]) : nullptr;
  int8_t* const out_xl = PH == kBX ? sreg_ptr(static_cast<int8_t*>(u.xl)) : nullptr;
  UnitDev wu;
  if constexpr (LAST) {
    wu.param = sreg_ptr(u.param);
    wu.ld_param = sreg_i64(u.ld_param);
    wu.param_f32 = sreg_i32(u.param_f32);
    wu.vec_param = sreg_i32(u.vec_param);
    wu.update_out = sreg_ptr(u.update_out);
    wu.ld_out = sreg_i64(u.ld_out);
    wu.vec_out = sreg_i32(u.vec_out);
    wu.rows = sreg_i32(u.rows);
    wu.cols = sreg_i32(u.cols);
  }

  // Each wave stages one 32-row strip of its scaled accumulators in its own
  // LDS area (so the strips need no block barrier), then writes row segments
  // (natural layout) and, where needed, column segments (mirror tiles of A
  // and B; weight rows of a tall matrix in the last iteration) as 16-byte
  // vector accesses.  In B X (bf16, not last) each accumulator block read
  // for the strip also gives the int8 corrections of the next master, stored
  // straight from the registers (one 16-byte store per block).  acc and wbuf
  // are only ever indexed with constants (a runtime index would move the
  // arrays to scratch memory), so the strip loop is unrolled at compile time.
  const float es = PH == kBX ? 1.f : scale;          // B X: the scale is folded upstream
  const size_t nbc = static_cast<size_t>(np / 32);
  static_for<0, NBM>([&](auto pic) {
    constexpr int pi = decltype(pic)::value;
    // strip by strip: a later strip's accumulators stay in the AGPRs until
    // its turn (reading them all out at once would exceed the VGPRs)
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (pi > 0) wave_sync();      // the previous strip's reads are done
#pragma unroll
    for (int j = 0; j < NBN; ++j) {
      float v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = es * acc_get<AGPR>(acc[pi][j], r);
      if constexpr (PH == kBX && !F32 && !LAST) {
        // the strip then holds y = bits(x) + 0x8080, whose upper halves are hi
        const size_t bi = (row_base + pi * 32) / 32, bj = (col_base + j * 32) / 32;
        gst(out_xl + (bi * nbc + bj) * 1024 + el * 16, encode_master16(v));
      }
      stage_block<EPP>(v, j, ep, el);
    }
    wave_sync();

#pragma unroll
    for (int q = 0; q < RITER; ++q) {
      const int s = el + 64 * q;
      const int row = s / SEGS, cseg = s % SEGS;
      float v[8];
      const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(&ep[row * EPP + cseg * 8]);
      const f32x4_t v1 = *reinterpret_cast<const f32x4_t*>(&ep[row * EPP + cseg * 8 + 4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) { v[e] = v0[e]; v[4 + e] = v1[e]; }
      const int gr = row_base + pi * 32 + row;
      const int gc = col_base + cseg * 8;
      if constexpr (PH == kGram || PH == kSquare) {
        st8<F32>(out_ab, static_cast<size_t>(gr) * mp + gc, v);
      } else if constexpr (!LAST) {
        if constexpr (F32) st8<true>(out_xh, static_cast<size_t>(gr) * np + gc, v);
        else gst(static_cast<uint16_t*>(out_xh) + static_cast<size_t>(gr) * np + gc, pack8_hi(v));
      } else if (u.side == kLeft) {
        if (gr < wu.rows) {
          if (wfast && gc + 8 <= wu.cols) update_w8_loaded(wu, gr, gc, v, decay, step, wbuf[pi][q]);
          else update_w8(wu, gr, gc, v, decay, step);
        }
      }
    }

    if (mirror) {
#pragma unroll
      for (int q = 0; q < CITER; ++q) {
        const int s = el + 64 * q;
        const int col = s % WTN, rseg = s / WTN;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = ep[(rseg * 8 + e) * EPP + col];
        const int gc = col_base + col;                 // mirror row
        const int gr = row_base + pi * 32 + rseg * 8;  // mirror column start
        if constexpr (PH == kGram || PH == kSquare) {
          st8<F32>(out_ab, static_cast<size_t>(gc) * mp + gr, v);   // A and B are symmetric
        } else if constexpr (LAST) {
          // tall matrix: O[i][j] = X[j][i], so X column gc is weight row gc
          if (gc < wu.rows) {
            if (!F32 && wfast && gr + 8 <= wu.cols) update_w8_loaded(wu, gc, gr, v, decay, step, wbuf[pi][q]);
            else update_w8(wu, gc, gr, v, decay, step);
          }
        }
      }
    }
  });
}

template <bool F32, int PH, int TC, bool LAST>
void launch_one(const UnitDev* units, const GemmTask* tasks, int n, const GemmParams& p, hipStream_t s) {
  constexpr int nt = 64 * Cfg<F32, PH, TC>::NWM * Cfg<F32, PH, TC>::NWN;
  ns_gemm_kernel<F32, PH, TC, LAST><<<n, nt, 0, s>>>(units, tasks, p);
}

template <bool F32, int TC>
hipError_t launch_phase(int phase, const UnitDev* units, const GemmTask* tasks, int n,
                        const GemmParams& p, hipStream_t s) {
  switch (phase) {
    case kGram: launch_one<F32, kGram, TC, false>(units, tasks, n, p, s); break;
    case kSquare: launch_one<F32, kSquare, TC, false>(units, tasks, n, p, s); break;
    default:
      if (p.last) launch_one<F32, kBX, TC, true>(units, tasks, n, p, s);
      else launch_one<F32, kBX, TC, false>(units, tasks, n, p, s);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int phase, bool f32, int tile, const UnitDev* units, const GemmTask* tasks,
                       int n_tasks, const GemmParams& p, hipStream_t s) {
  if (n_tasks <= 0) return hipSuccess;
  if (f32) return launch_phase<true, kTileM>(phase, units, tasks, n_tasks, p, s);
  return tile == kTileL ? launch_phase<false, kTileL>(phase, units, tasks, n_tasks, p, s)
                        : launch_phase<false, kTileM>(phase, units, tasks, n_tasks, p, s);
}

}  // namespace muon
