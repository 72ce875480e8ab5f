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
// bf16 path: 128x128 output tile, 8 waves of 64x32 (2x1 blocks of
// v_mfma_f32_32x32x16_bf16), K staged through LDS 64 deep in a two-stage
// ring filled by direct-to-LDS loads (global_load_lds_dwordx4: no VGPR
// staging, no LDS store instructions); two blocks fit per CU (64 KB LDS
// each) so one block's epilogue overlaps the other's MFMA loop.  X is held
// as a bf16 hi/lo pair so the a*X term keeps ~16 significant bits while the MFMA
// operand is the hi part.
// fp32 path: 64x64 tile, 4 waves of 32x32, v_mfma_f32_32x32x2f32.
#include "device_common.h"
#include "muon_internal.h"

namespace muon {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(1))) const u32x4_t gu32x4_t;     // global memory
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;       // LDS

// Tile configuration per precision and phase (the defaults are the fastest
// measured; 32-deep stages in a 3- or 4-stage ring, MUON_BK_BF16=32, were 9 %
// slower on every workload).  BTM x BTN: output tile (rows x columns);
// NWM x NWN waves, each owning a (BTM/NWM) x (BTN/NWN) block of 32x32 MFMA
// tiles; BK: K depth of one LDS stage; NS: stages in the LDS ring (NS-1 in
// flight while one is consumed); OCC: blocks per CU the registers and LDS
// allow.  BTM x BTN: output tile (rows x columns).
#ifndef MUON_NS_BF16
#define MUON_NS_BF16 2
#endif
#ifndef MUON_BK_BF16
#define MUON_BK_BF16 64
#endif
#ifndef MUON_BX_NWN
#define MUON_BX_NWN 4
#endif
#ifndef MUON_BX_OCC
#define MUON_BX_OCC 2
#endif
template <bool F32, int PH> struct Cfg;
#ifndef MUON_G_NWN
#define MUON_G_NWN 4
#endif
template <int PH> struct Cfg<false, PH> {        // bf16, Gram and square
  using E = uint16_t;
  static constexpr int BTM = kTileGramBf16, BTN = kTileGramBf16, NWM = 2, NWN = MUON_G_NWN, BK = MUON_BK_BF16,
                       NS = MUON_NS_BF16;
  static constexpr int OCC = NS * BK <= 128 ? 2 : 1;    // ring of 2 x 32 KB or 4 x 16 KB: two blocks per CU
};
template <> struct Cfg<false, kBX> {             // bf16, B X
  using E = uint16_t;
  static constexpr int BTM = kTileBxRowsBf16, BTN = kTileBxColsBf16, NWM = kTileBxRowsBf16 / 64, NWN = MUON_BX_NWN,
                       BK = MUON_BK_BF16, NS = MUON_NS_BF16;
  static constexpr int OCC = NWM * NWN > 8 ? 1 : NS * BK <= 128 ? MUON_BX_OCC : 1;
};
template <int PH> struct Cfg<true, PH> {         // float32, all phases
  using E = float;
  static constexpr int BTM = kTileF32, BTN = kTileF32, NWM = 2, NWN = 2, BK = 32, NS = 2, OCC = 2;
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
//   K-major tile of B X (row = k, 16 chunks of columns): chunk c of row k
//     sits at position c ^ 4 (k % 4), which spreads the four rows a
//     transposing read touches over distinct banks.
template <int CPR>
__device__ __forceinline__ int swz_kc(int r, int c) {
  static_assert(CPR == 8 || CPR == 4, "K rows of 8 or 4 chunks");
  if constexpr (CPR == 8) return c ^ ((r >> 1) & 7);
  else return c ^ ((r >> 2) & 3);   // 64-byte rows: four share a bank line
}
__device__ __forceinline__ int swz_km(int k, int c) { return c ^ ((k & 3) << 2); }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

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

// Transposing LDS read (gfx950).  Within each 16-lane group the 8-byte words
// addressed by the lanes form a 16 x 4 matrix W[lane][e]; lane i receives
// W[4e + i/4][i%4] for e = 0..3.  If lane 4e+q points at X[k+e][j+4q..+3],
// lane i therefore gets X[k+e][j+i], e = 0..3: four consecutive k of one
// column, which is what an MFMA operand lane holds.
__device__ __forceinline__ bf16x4_t lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
}

// Direct-to-LDS loads of one stage (global_load_lds_dwordx4): instruction i
// of wave w fills the 1 KB at chunk (w*NI + i)*64 of the tile, lane L
// writing chunk +L; aoff/boff hold each lane's byte offset of the global
// chunk that belongs there (swizzle included).  No VGPR holds the data and
// no LDS store instruction is issued.
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

template <int NA, int NB, typename E>
__device__ __forceinline__ void issue_stage(const E* ga, const E* gb, const uint32_t (&aoff)[NA],
                                            const uint32_t (&boff)[NB], uint32_t la, uint32_t lb, int wave,
                                            bool with_b) {
#pragma unroll
  for (int i = 0; i < NA; ++i) dma16(ga, aoff[i], la + (wave * NA + i) * 1024);
  if (with_b) {
#pragma unroll
    for (int i = 0; i < NB; ++i) dma16(gb, boff[i], lb + (wave * NB + i) * 1024);
  }
}

// LDS byte address of a shared-memory pointer.
template <typename E>
__device__ __forceinline__ uint32_t lds_addr(const E* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const E*)(p)));
}

// MFMAs of one BK-deep stage held in LDS (la: K-contiguous A tile, BTM rows
// of BK; lb: the B tile, K-contiguous like A or K-major, BK rows of BTN).
// The wave owns rows wm*WTM.. and columns wn*WTN.. of the block tile, as
// NBM x NBN tiles of 32x32.
template <bool F32, bool KMAJOR_B, int NBM, int NBN, int WTM, int WTN, int BK, int BTN, typename E>
__device__ __forceinline__ void mma_stage(const E* la, const E* lb, f32x16_t (&acc)[NBM][NBN], int lane, int wm,
                                          int wn) {
  if constexpr (!F32) {
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t fa[NBM], fb[NBN];
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
#pragma unroll
      for (int i = 0; i < NBM; ++i)
#pragma unroll
        for (int j = 0; j < NBN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  } else {
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

// Accumulators of one 32-row strip (NBN tiles of 32x32) into the wave's LDS
// staging area, in row-major order (pitch EPP floats).  v_mfma 32x32 output:
// lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
template <int NBN, int EPP>
__device__ __forceinline__ void stage_strip(const f32x16_t (&row)[NBN], float* ep, int lane) {
#pragma unroll
  for (int j = 0; j < NBN; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      ep[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * EPP + j * 32 + (lane & 31)] = row[j][r];
}

// B X: the X master of the output tile's rows is part of the X operand (row
// r of X is K step r), so while a K step whose rows overlap the tile sits in
// LDS each lane copies out its own row segments: bf16 the hi half (the lo
// half is not an operand and comes from HBM), float32 all 8 values.
template <bool F32, int NBM, int RITER, int SEGS, int WTM, int BK, int BTN, typename E>
__device__ __forceinline__ void capture_master(const E* lbx, int kt, int kt0, int wm, int col0, int lane,
                                               u32x4_t (&pre0)[NBM][RITER], u32x4_t (&pre1)[NBM][RITER]) {
  static_assert(BK % 32 == 0, "32-row strips must not straddle K steps");
#pragma unroll
  for (int pi = 0; pi < NBM; ++pi) {
    const int r0 = wm * WTM + pi * 32;      // first tile row of the strip
    if (kt == kt0 + r0 / BK) {
#pragma unroll
      for (int q = 0; q < RITER; ++q) {
        const int sg = lane + 64 * q;
        const int k = r0 % BK + sg / SEGS, col = col0 + (sg % SEGS) * 8;
        if constexpr (F32) {
          pre0[pi][q] = *reinterpret_cast<const u32x4_t*>(&lbx[k * BTN + swz_km(k, col >> 2) * 4]);
          pre1[pi][q] = *reinterpret_cast<const u32x4_t*>(&lbx[k * BTN + swz_km(k, (col >> 2) + 1) * 4]);
        } else {
          pre0[pi][q] = *reinterpret_cast<const u32x4_t*>(&lbx[k * BTN + swz_km(k, col >> 3) * 8]);
        }
      }
    }
  }
}

// B = b A + c A A: the A tile (ti, tj) the epilogue combines is part of the
// A operand of the same block (rows ti, K columns tj), so each lane copies
// its row segments out of LDS during the K step that holds its columns,
// and the epilogue reads no A from memory.  A wave's WTN columns lie in one
// K step (WTN divides BK).
template <bool F32, int NBM, int RITER, int SEGS, int WTM, int WTN, int BK, typename E>
__device__ __forceinline__ void capture_atile(const E* la, int kt, int kt_cap, int wm, int wn, int lane,
                                              u32x4_t (&pre0)[NBM][RITER], u32x4_t (&pre1)[NBM][RITER]) {
  static_assert(BK % WTN == 0, "a wave's columns must lie in one K step");
  constexpr int EPE = 16 / sizeof(E);
  if (kt != kt_cap) return;
#pragma unroll
  for (int pi = 0; pi < NBM; ++pi)
#pragma unroll
    for (int q = 0; q < RITER; ++q) {
      const int sg = lane + 64 * q;
      const int r = wm * WTM + pi * 32 + sg / SEGS;            // tile row = A-operand row
      const int k = (wn * WTN + (sg % SEGS) * 8) % BK;         // column inside the K step
      pre0[pi][q] = *reinterpret_cast<const u32x4_t*>(&la[r * BK + swz_kc<BK / EPE>(r, k / EPE) * EPE]);
      if constexpr (F32)
        pre1[pi][q] = *reinterpret_cast<const u32x4_t*>(&la[r * BK + swz_kc<BK / EPE>(r, k / EPE + 1) * EPE]);
    }
}

template <bool F32, int PH>
__global__ __launch_bounds__((64 * Cfg<F32, PH>::NWM * Cfg<F32, PH>::NWN), (Cfg<F32, PH>::OCC))
void ns_gemm_kernel(const UnitDev* __restrict__ units, const GemmTask* __restrict__ tasks,
                    GemmParams p) {
  using C = Cfg<F32, PH>;
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
  static_assert(NIA * NT * EPE == T_A && NIB * NT * EPE == T_B, "tile/thread mismatch");
  static_assert((CPR == 8 || CPR == 4) && CPRX == 16, "swizzles assume 8- or 4-chunk K rows and 16-chunk K-major rows");
  static_assert(NWM * NWN * 32 * EPP * 4 <= NS * STAGE * static_cast<int>(sizeof(E)),
                "epilogue staging must fit in the operand LDS");

  __shared__ __attribute__((aligned(16))) E smem[NS * STAGE];
  __shared__ float red[4];

  const GemmTask t = tasks[blockIdx.x];
  if (t.unit < 0) return;   // padding of the XCD-interleaved task order
  const UnitDev& u = units[t.unit];
  // first iteration: B X applies the unit's 1/||U|| that the Gram phase
  // folded (every Gram block folds the same bits; one stores them); the
  // load is issued here so its latency hides behind the K loop
  const float first_scale = PH == kBX && p.first ? gld<float>(u.norm) : 1.f;
  const int mp = u.mp, np = u.np;
  const int ti = t.ti, tj = t.tj;

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

  // each lane's global element offset (within a stage) for its DMA chunks
  uint32_t aoff[NIA], boff[NIB];
#pragma unroll
  for (int i = 0; i < NIA; ++i) {
    const int c = (wave * NIA + i) * 64 + lane;      // chunk position in the A tile
    const int ar = c / CPR;
    aoff[i] = static_cast<uint32_t>((ar * lda_g + swz_kc<CPR>(ar, c % CPR) * EPE) * sizeof(E));
  }
#pragma unroll
  for (int i = 0; i < NIB; ++i) {
    const int c = (wave * NIB + i) * 64 + lane;      // chunk position in the B tile
    if constexpr (KMAJOR_B) {
      const int k = c / CPRX;
      boff[i] = static_cast<uint32_t>((k * ldb_g + swz_km(k, c % CPRX) * EPE) * sizeof(E));
    } else {
      const int br = c / CPR;
      boff[i] = static_cast<uint32_t>((br * ldb_g + swz_kc<CPR>(br, c % CPR) * EPE) * sizeof(E));
    }
  }
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

  // row segments of the epilogue: per 32-row strip, SEGS segments of 8 per
  // row, RITER per lane
  constexpr int SEGS = WTN / 8;
  constexpr int RITER = 32 * SEGS / 64;
  constexpr bool CAPTURE = KMAJOR_B || PH == kSquare;   // epilogue operand taken from LDS
  constexpr int NPRE = CAPTURE ? NBM : 1;
  u32x4_t pre0[NPRE][RITER], pre1[NPRE][RITER];     // master: hi (bf16) / first..last 4 (float32)
  u32x2_t preq[NPRE][RITER];                          // master: int8 corrections (bf16)
  const int kt0 = ti * BTM / BK;                     // K step of the tile's first row

  const int KT = K / BK;

  // B X, bf16: the epilogue's HBM operands are the lo half of the master
  // (the hi half is captured from LDS) and, in the last iteration, the
  // weight segments this lane updates (bf16 weights with aligned rows; the
  // segments are rows of W for a wide unit, columns of the tile for a tall
  // one, where X column j is weight row j).  They are requested once per
  // tile, behind the last K step's MFMAs.
  const int row_base = ti * BTM + wm * WTM;
  const int col_base = tj * BTN + wn * WTN;
  static_assert(!KMAJOR_B || RITER == WTN * 4 / 64, "row and column passes give a lane equally many segments");
  u32x4_t wpre[NPRE][RITER];
  const bool wfast = KMAJOR_B && !F32 && p.last && !u.param_f32 && u.vec_param;
  auto wseg = [&](int pi, int q, int& wi, int& wj) {
    const int sg = lane + 64 * q;
    if (u.side == kLeft) {
      wi = row_base + pi * 32 + sg / SEGS;
      wj = col_base + (sg % SEGS) * 8;
    } else {
      wi = col_base + sg % WTN;
      wj = row_base + pi * 32 + (sg / WTN) * 8;
    }
  };
  auto epilogue_loads = [&]() {
    if constexpr (KMAJOR_B && !F32) {
#pragma unroll
      for (int pi = 0; pi < NBM; ++pi)
#pragma unroll
        for (int q = 0; q < RITER; ++q) {
          const int sg = lane + 64 * q;
          const size_t off = static_cast<size_t>(row_base + pi * 32 + sg / SEGS) * np + col_base + (sg % SEGS) * 8;
          preq[pi][q] = gld<u32x2_t>(static_cast<const int8_t*>(u.xl) + off);
        }
      if (wfast) {
#pragma unroll
        for (int pi = 0; pi < NBM; ++pi)
#pragma unroll
          for (int q = 0; q < RITER; ++q) {
            int wi, wj;
            wseg(pi, q, wi, wj);
            if (wi < u.rows && wj + 8 <= u.cols)
              wpre[pi][q] = gld<u32x4_t>(static_cast<const uint16_t*>(u.param) + static_cast<size_t>(wi) * u.ld_param + wj);
          }
      }
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
  // stages every step waits for everything, so the last step issues no copy
  // and sends the epilogue's HBM loads out in its place: they overlap the
  // final MFMAs and the epilogue does not wait for a dead copy.
  constexpr uint32_t STAGE_B = STAGE * sizeof(E), TILE_B = T_A * sizeof(E);
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) {
    const int sc = min(s, KT - 1);
    issue_stage<NIA, NIB, E>(pa + sc * a_step, pb + sc * b_step, aoff, boff, ring0 + s * STAGE_B,
                             ring0 + s * STAGE_B + TILE_B, wave, !diag);
  }
  auto kstep = [&](int kt, bool tail) {
    if (diag) wait_vmcnt<(NS - 2) * NIA>();   // newer stages in flight: NS-2 of one operand each
    else wait_vmcnt<(NS - 2) * (NIA + NIB)>();
    ring_barrier();
    if (!tail) {
      const int nx = min(kt + NS - 1, KT - 1);
      const uint32_t ls = ring0 + ((kt + NS - 1) % NS) * STAGE_B;
      issue_stage<NIA, NIB, E>(pa + nx * a_step, pb + nx * b_step, aoff, boff, ls, ls + TILE_B, wave, !diag);
    }
    const E* cs = smem + (kt % NS) * STAGE;
    if constexpr (KMAJOR_B)
      capture_master<F32, NPRE, RITER, SEGS, WTM, BK, BTN>(cs + T_A, kt, kt0, wm, wn * WTN, lane, pre0, pre1);
    else if constexpr (PH == kSquare)
      capture_atile<F32, NPRE, RITER, SEGS, WTM, WTN, BK>(cs, kt, (tj * BTN + wn * WTN) / BK, wm, wn, lane, pre0, pre1);
    if (tail) epilogue_loads();
    mma_stage<F32, KMAJOR_B, NBM, NBN, WTM, WTN, BK, BTN>(cs, diag ? cs : cs + T_A, acc, lane, wm, wn);
  };
  if constexpr (NS == 2) {
    for (int kt = 0; kt < KT - 1; ++kt) kstep(kt, false);
    kstep(KT - 1, true);
    ring_barrier();    // no copy in flight; every wave is done reading the ring
  } else {
    for (int kt = 0; kt < KT; ++kt) kstep(kt, false);
    epilogue_loads();
    wait_vmcnt<0>();   // the clamped copies of the last stage
    __syncthreads();   // the epilogue reuses the ring as staging
  }

  // ---------------------------------------------------------------- epilogue
  // Each wave stages one 32-row strip of its accumulators in its own LDS
  // area (so the strips need no block barrier: one wave's LDS accesses take
  // effect in order), then writes row segments (natural layout) and, where
  // needed, column segments (mirror tiles of A and B; weight rows of a tall
  // matrix in the last iteration) as 16-byte vector accesses.
  float scale = 1.f;
  if constexpr (PH == kGram) {
    if (p.first) {
      const float iv = unit_inv_norm(u.partials, u.k1_ntiles, p.eps, red);
      scale = iv * iv;
      if (ti == 0 && tj == 0 && threadIdx.x == 0) gst(u.norm, iv);   // for the first B X phase
    }
  } else if constexpr (PH == kBX) {
    scale = first_scale;
  }
  const bool last = PH == kBX && p.last;
  const bool mirror = PH == kBX ? (last && u.side == kRight) : (ti != tj);
  const float decay = p.lr * p.weight_decay;
  const float step = p.lr * u.lr_scale;
  float* ep = reinterpret_cast<float*>(smem) + wave * (32 * EPP);
  constexpr int CITER = WTN * 4 / 64;                // column segments per lane
  // the output pointers, kept in scalar registers for the whole epilogue;
  // so are the weight fields of the last iteration's update (wu: a copy of
  // the descriptor whose fields the update reads are pinned)
  void* const out_ab = PH == kGram ? sreg_ptr(u.a) : PH == kSquare ? sreg_ptr(u.b) : nullptr;
  void* const out_xh = PH == kBX ? sreg_ptr(u.xh[p.x_in ^ 1]) : nullptr;
  int8_t* const out_xl = PH == kBX ? sreg_ptr(static_cast<int8_t*>(u.xl)) : nullptr;
  UnitDev wu;
  if (last) {
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

  // acc and the master registers are only ever indexed with constants (a
  // runtime index would move the whole array to scratch memory), so the
  // strip loop is unrolled.
#pragma unroll
  for (int pi = 0; pi < NBM; ++pi) {
    stage_strip<NBN, EPP>(acc[pi], ep, lane);

#pragma unroll
    for (int q = 0; q < RITER; ++q) {
      const int s = lane + 64 * q;
      const int row = s / SEGS, cseg = s % SEGS;
      float v[8];
      const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(&ep[row * EPP + cseg * 8]);
      const f32x4_t v1 = *reinterpret_cast<const f32x4_t*>(&ep[row * EPP + cseg * 8 + 4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) { v[e] = v0[e]; v[4 + e] = v1[e]; }
      const int gr = row_base + pi * 32 + row;
      const int gc = col_base + cseg * 8;
      if constexpr (PH == kGram) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= scale;
        st8<F32>(out_ab, static_cast<size_t>(gr) * mp + gc, v);
      } else if constexpr (PH == kSquare) {
        float av[8];                                      // A at this segment, captured from LDS
        if constexpr (F32) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            av[e] = __uint_as_float(pre0[pi][q][e]);
            av[4 + e] = __uint_as_float(pre1[pi][q][e]);
          }
        } else {
          unpack8_bf16(pre0[pi][q], av);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = fmaf(p.b, av[e], p.c * v[e]);
        st8<F32>(out_ab, static_cast<size_t>(gr) * mp + gc, v);
        if (mirror) {   // the mirror pass stores B^T from the staged values
          *reinterpret_cast<f32x4_t*>(&ep[row * EPP + cseg * 8]) = f32x4_t{v[0], v[1], v[2], v[3]};
          *reinterpret_cast<f32x4_t*>(&ep[row * EPP + cseg * 8 + 4]) = f32x4_t{v[4], v[5], v[6], v[7]};
        }
      } else {
        const size_t off = static_cast<size_t>(gr) * np + gc;
        float xm[8];
        if constexpr (F32) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xm[e] = __uint_as_float(pre0[pi][q][e]);
            xm[4 + e] = __uint_as_float(pre1[pi][q][e]);
          }
        } else {
          master_decode8(pre0[pi][q], preq[pi][q], xm);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = scale * fmaf(p.a, xm[e], v[e]);
        if (!last) {
          if constexpr (F32) {
            st8<true>(out_xh, off, v);
          } else {
            u32x4_t hq;
            u32x2_t lq;
            master_encode8(v, hq, lq);
            gst(static_cast<uint16_t*>(out_xh) + off, hq);
            gst(out_xl + off, lq);
          }
        } else if (u.side == kLeft) {
          if (gr < wu.rows) {
            if (wfast && gc + 8 <= wu.cols) update_w8_loaded(wu, gr, gc, v, decay, step, wpre[pi][q]);
            else update_w8(wu, gr, gc, v, decay, step);
          }
        } else {
          *reinterpret_cast<f32x4_t*>(&ep[row * EPP + cseg * 8]) = f32x4_t{v[0], v[1], v[2], v[3]};
          *reinterpret_cast<f32x4_t*>(&ep[row * EPP + cseg * 8 + 4]) = f32x4_t{v[4], v[5], v[6], v[7]};
        }
      }
    }

    if (mirror) {
#pragma unroll
      for (int q = 0; q < CITER; ++q) {
        const int s = lane + 64 * q;
        const int col = s % WTN, rseg = s / WTN;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = ep[(rseg * 8 + e) * EPP + col];
        const int gc = col_base + col;                 // mirror row
        const int gr = row_base + pi * 32 + rseg * 8;  // mirror column start
        if constexpr (PH == kGram) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] *= scale;
          st8<F32>(out_ab, static_cast<size_t>(gc) * mp + gr, v);
        } else if constexpr (PH == kSquare) {
          st8<F32>(out_ab, static_cast<size_t>(gc) * mp + gr, v);   // B is symmetric off the diagonal tiles
        } else {
          // tall matrix: O[i][j] = X[j][i], so X column gc is weight row gc
          if (gc < wu.rows) {
            if constexpr (!F32) {
              if (wfast && gr + 8 <= wu.cols) {
                update_w8_loaded(wu, gc, gr, v, decay, step, wpre[pi][q]);
                continue;
              }
            }
            update_w8(wu, gc, gr, v, decay, step);
          }
        }
      }
    }
  }
}

template <bool F32, int PH>
void launch_one(const UnitDev* units, const GemmTask* tasks, int n, const GemmParams& p, hipStream_t s) {
  constexpr int nt = 64 * Cfg<F32, PH>::NWM * Cfg<F32, PH>::NWN;
  ns_gemm_kernel<F32, PH><<<n, nt, 0, s>>>(units, tasks, p);
}

template <bool F32>
hipError_t launch_phase(int phase, const UnitDev* units, const GemmTask* tasks, int n,
                        const GemmParams& p, hipStream_t s) {
  switch (phase) {
    case kGram: launch_one<F32, kGram>(units, tasks, n, p, s); break;
    case kSquare: launch_one<F32, kSquare>(units, tasks, n, p, s); break;
    default: launch_one<F32, kBX>(units, tasks, n, p, s); break;
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
