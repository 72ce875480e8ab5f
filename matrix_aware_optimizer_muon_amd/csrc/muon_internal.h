// Internal types shared by the host planner (muon_host.cpp) and the gfx950
// kernels (*.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace muon {

// Output tiles of the Newton-Schulz GEMM phases.  A bf16 unit takes one tile
// edge for all three phases: 128 (kTileM) or, for large matrices, 256
// (kTileL), chosen per unit by the planner; float32 units use 64.  Every NS
// buffer of a unit is zero-padded to a multiple of its tile edge, which is
// exact under X X^T, A A and B X.
enum TileCfg : int32_t { kTileM = 0, kTileL = 1 };
constexpr int kTileCfgs = 2;
constexpr int kTileEdgeM = 128;
constexpr int kTileEdgeL = 256;
constexpr int kTileF32 = 64;
inline int tile_edge(bool f32, int cfg) { return f32 ? kTileF32 : cfg == kTileL ? kTileEdgeL : kTileEdgeM; }
// Tiles of the elementwise phases (momentum, update), 8192 elements each.
// A unit whose X is U itself (rows <= cols) is walked in kEwRows x kEwCols
// tiles along its rows, so each wave reads and writes runs of 256
// consecutive elements, and a tile's 32 rows are one row of whole 32 x 32
// correction blocks; a unit whose X is U^T is walked in kEwRRows x kEwRCols
// tiles (rows x columns of U) transposed through LDS.
constexpr int kEwRows = 32, kEwCols = 256;
constexpr int kEwRRows = 64, kEwRCols = 128;
// bf16 matrices whose short side is below this run their Newton-Schulz
// iteration on the float32 path: at such sizes the bf16 iteration's own
// rounding error approaches 2e-2 relative, and the float32 path costs
// nothing measurable.
constexpr int kMinBf16NsSide = 128;

enum Side : int32_t { kLeft = 0, kRight = 1 };

// One orthogonalisation problem ("unit"): a whole matrix, or one row block
// of a matrix registered with split_rows.  Stored shape rows x cols.  Left
// side (rows <= cols): X = U (m = rows, n = cols).  Right side: X = U^T
// (m = cols, n = rows).  X is kept in the canonical m x n orientation in the
// workspace, so the GEMM phases never see a transpose.
struct UnitDev {
  // caller tensors (views of this unit's rows)
  const void* grad;  int64_t ld_grad;  int32_t grad_f32;  int32_t vec_grad;
  float* mom;        int64_t ld_mom;   int32_t vec_mom;   int32_t pad0;
  void* param;       int64_t ld_param; int32_t param_f32; int32_t vec_param;
  float* update_out; int64_t ld_out;   int32_t vec_out;   int32_t pad1;
  int32_t rows, cols;        // stored shape of the unit
  int32_t side, m, n, mp, np, pad2;
  // workspace buffers (row-major, leading dimension np for X, mp for A/B).
  // bf16 NS: xh is X rounded to bf16 (the MFMA operand; nearest-even as the
  // momentum phase writes it, half-up just below the tie as B X writes it)
  // and xl one int8 correction per element counted against that xh (X ~=
  // the float32 with bits(xh) + 256 xl, i.e. xh + xl * ulp(xh)/256 within
  // xh's binade), stored in 32 x 32 blocks in the MFMA accumulator order
  // (corr_index in device_common.h); a and b are bf16.
  // float32 NS: xh is the float32 X, xl is unused, a and b are float32.
  // xh is double-buffered: the B X phase reads the whole current iterate as
  // an operand while its tiles write the next one; xl is read and written
  // only by the tile that owns each region.
  void* xh[2]; void* xl; void* a; void* b;
  float* partials;           // one partial sum of squares per momentum tile
  float* norm;               // 1 / (||U||_F + eps), folded by the first Gram phase
  int32_t k1_tile0, k1_ntiles;
  float lr_scale;            // shape scale * lr_mult
  int32_t pad3;
};

struct EwTask { int32_t unit, tr, tc, local; };      // tile (tr, tc) of a unit
struct GemmTask { int32_t unit, ti, tj, pad; };      // output tile (ti, tj)

struct K1Params {
  float mu;
  int32_t nesterov;
  int32_t sgd_form;
  uint32_t* flags;
};

struct GemmParams {
  float a, b, c;
  float eps;           // Frobenius normalisation guard
  int32_t first;       // first NS iteration: fold the norm scale in
  int32_t last;        // last NS iteration: apply the weight update in place of storing X
  int32_t x_in;        // which xh buffer holds the current iterate
  int32_t pad;
  float lr;            // weight update of the last iteration
  float weight_decay;
  uint32_t* flags;     // the handle's flag word (bounds checks of a debug build)
};

struct K5Params {      // stand-alone update, used when ns_steps == 0
  float lr;
  float weight_decay;
  float eps;
  int32_t pad;
  uint32_t* flags;     // the handle's flag word (bounds checks of a debug build)
};

// Flag word bits (muon_get_flags): 1 = a non-finite value in an update,
// 2 = a preconditioner factorisation failed, 4 = a task of a build with
// MUON_DEBUG_BOUNDS=1 failed its bounds check (the task was skipped).
constexpr uint32_t kFlagBounds = 4u;
#ifndef MUON_DEBUG_BOUNDS
#define MUON_DEBUG_BOUNDS 0
#endif

enum Phase : int32_t { kGram = 0, kSquare = 1, kBX = 2 };

// ---- Newton-Muon preconditioner ------------------------------------------
constexpr int kCholBlock = 64;    // Cholesky / inverse block edge (float64)
constexpr int kPrecondPad = 128;  // S and S^-1 are padded to multiples of this

// S^-1 is stored as three bf16 planes per block, h + m + l = the float32
// value exactly (h = bf16(x), m = bf16(x - h), l = x - h - m), so the apply
// reads operands its bf16 matrix cores take as they are.
constexpr int kSinvPlanes = 3;

// One preconditioned tensor of the apply phase: P = G S^-1 (block-wise).
struct PrecondDev {
  const void* grad; int64_t ld_grad; int32_t grad_f32; int32_t vec_grad;
  float* p;         int64_t ld_p;     // P, float32, rows x (d * nblocks)
  const uint16_t* sinv;               // nblocks inverses of the slot, kSinvPlanes bf16 dp x dp planes each
  int32_t rows, d, dp, nblocks;
};
struct ApplyTask { int32_t tensor, tr, tc, blk; };   // 128x64 tile (tr, tc) of block blk

// Buffers of one S^-1 block for a refresh.
struct PrecondBlockDev {
  float* s;        // S, float32, dp x dp
  double* l;       // Cholesky factor, float64
  double* li;      // its inverse, float64
  uint16_t* sinv;  // S^-1, kSinvPlanes bf16 planes
  float* acc;      // running sum of X^T X over micro-batches, float32, dp x dp
  double* cnt;     // its running sample count
  float* part;     // scratch shared by every block of every slot: the split partial sums of
                   // X^T X (moment_splits(dp) dp x dp float32 slabs), then the float64 dp x dp
                   // sum that collects S^-1 during the factorisation
  int32_t d, dp;
};

// Split of the second-moment product X^T X over ranges of sample rows: a
// d = 768 layer has only 21 upper tiles, so without it a batch occupies 21
// of the 256 CUs.  The split count aims at kMomentTargetBlocks blocks, keeps
// at least kMomentMinRows rows per range, and the partial sums are added in
// range order by a second pass (deterministic).
constexpr int kMomentTargetBlocks = 512;
constexpr int kMomentMaxSplits = 16;
constexpr int64_t kMomentMinRows = 256;
inline int moment_splits(int dp, bool f32, int64_t n_rows) {
  const int nt = dp / (f32 ? 64 : 128);
  const int tiles = nt * (nt + 1) / 2;
  int sp = (kMomentTargetBlocks + tiles - 1) / tiles;
  if (sp > kMomentMaxSplits) sp = kMomentMaxSplits;
  const int64_t by_rows = n_rows / kMomentMinRows + (n_rows % kMomentMinRows != 0);
  if (sp > by_rows) sp = static_cast<int>(by_rows);
  return sp < 1 ? 1 : sp;
}

// Launchers (defined in the .hip files).
// AdamW tensors (parameters Muon does not take).  Each is stepped as a set
// of "rows" of `len` elements; a tensor whose param, grad and moments are all
// contiguous is one row of rows*cols elements.
struct AdamDev {
  void* param; const void* grad; float* m; float* v;
  int64_t ld_param, ld_grad, ld_mom;   // elements between rows
  int64_t len;                         // elements per row
  int32_t f32;                         // param/grad float32 (else bf16)
  int32_t vec;                         // 16-byte aligned rows: vector accesses
  float lr_mult;
  int32_t pad;
};
constexpr int kAdamChunk = 2048;       // elements of one row per block (256 threads x 8)
struct AdamTask { int32_t tensor, row; int64_t c0; };
struct AdamState {                     // on the device, in the workspace
  uint32_t t;                          // steps taken
  float inv_bc1;                       // 1 / (1 - b1^t)
  float inv_sqrt_bc2;                  // 1 / sqrt(1 - b2^t)
  uint32_t pad;
};
struct AdamParams {
  float lr, beta1, beta2, eps, weight_decay;
  const AdamState* state;
  uint32_t* flags;
};

hipError_t launch_momentum(bool f32, const UnitDev* units, const EwTask* tasks, int n_tasks,
                           const K1Params& p, hipStream_t s);
hipError_t launch_gemm(int phase, bool f32, int tile, const UnitDev* units, const GemmTask* tasks,
                       int n_tasks, const GemmParams& p, hipStream_t s);
hipError_t launch_update(bool f32, const UnitDev* units, const EwTask* tasks, int n_tasks,
                         const K5Params& p, hipStream_t s);
hipError_t launch_precond_refresh(const PrecondBlockDev& b, const void* acts, int64_t n_rows, int64_t ld,
                                  bool acts_f32, float damping, uint32_t* flags, hipStream_t s);
hipError_t launch_precond_accumulate(const PrecondBlockDev& b, const void* acts, int64_t n_rows, int64_t ld,
                                     bool acts_f32, float beta, hipStream_t s);
hipError_t launch_precond_refresh_accumulated(const PrecondBlockDev& b, float damping, bool reset, uint32_t* flags,
                                              hipStream_t s);
// tasks: n_bf16 tiles of bf16-gradient tensors, then n_f32 of float32 ones
hipError_t launch_precond_apply(const PrecondDev* pds, const ApplyTask* tasks, int n_bf16, int n_f32, hipStream_t s);
hipError_t launch_identity(uint16_t* sinv, int dp, int nblocks, hipStream_t s);
hipError_t launch_adam_tick(AdamState* st, float beta1, float beta2, hipStream_t s);
hipError_t launch_adam_set(AdamState* st, uint32_t t, hipStream_t s);
hipError_t launch_adamw(const AdamDev* tensors, const AdamTask* tasks, int n_tasks, const AdamParams& p,
                        hipStream_t s);

}  // namespace muon
