// Host side of the Muon C ABI: validation, planning (units, sides, padding,
// tile lists, workspace carve-up), descriptor upload and kernel sequencing.
//
// Plan of one step:
//   adamw     (2 launches, only with kind-ADAMW tensors: count tick, update)
//             Muon README "Usage"
// then per NS-precision group, all matrices of the group at once:
//   momentum  (1 launch)      Muon README "Hyperparameter tuning"
//   ns_steps x {gram, square, bx}  (per phase one launch per tile shape,
//             on each lane's stream)   Muon blog sec. 3;
//             the last bx applies the update (Muon README "Usage")
//   update    (1 launch, only when ns_steps == 0)
#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/muon.h"
#include "muon_internal.h"

using namespace muon;

namespace {

thread_local std::string g_last_error;

// A host-side range naming the launches it encloses, for rocprofv3's marker
// trace (`--marker-trace`); with no tool attached a push and a pop cost a few
// tens of nanoseconds.
struct Range {
  explicit Range(const char* name) { roctxRangePushA(name); }
  ~Range() { roctxRangePop(); }
  Range(const Range&) = delete;
  Range& operator=(const Range&) = delete;
};

muon_status_t fail(muon_status_t s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct UnitPlan {
  int tensor = 0, block = 0;
  int64_t row0 = 0;
  int rows = 0, cols = 0, side = 0, m = 0, n = 0, mp = 0, np = 0;
  bool f32 = false;
  int tile[3] = {kTileM, kTileM, kTileM};   // GEMM tile shape (TileCfg) per phase
  float lr_scale = 1.f;
  size_t off_xh0 = 0, off_xh1 = 0, off_xl = 0, off_a = 0, off_b = 0;
  int k1_tile0 = 0, k1_ntiles = 0, k1_tr = 0, k1_tc = 0;
  int group_index = 0;  // index inside its dtype group
};

struct Group {
  bool f32 = false;
  int lane = 0;            // 0: caller's stream; l > 0: the handle's stream l
  std::vector<int> units;  // global unit ids
  std::vector<EwTask> ew;
  // per GEMM phase and tile shape (TileCfg): the tiles of the group's units
  // of that shape, in launch order (one launch per non-empty list)
  std::vector<GemmTask> gemm[3][kTileCfgs];
  size_t off_units = 0, off_ew = 0;
  size_t off_gemm[3][kTileCfgs] = {};
};

const char* kPhaseNames[3] = {"gram", "square", "bx"};
const int kLaunchOrder[kTileCfgs] = {kTileL, kTileM};   // per phase: the longer 256-tile launch first

// bf16 tile shape of a unit's GEMM phase.  The 256 x 256 tiles (one block
// of 128 x 64-wave tiles per CU) halve the operand bytes per flop and read
// a third of the LDS bytes per flop of the 128 x 128 ones.  Units are padded
// to 128 only: a phase of 256-tiles covers the unit's largest multiple of
// 256 with them and the strips beyond with 128-tiles (unit_tiles), in a
// second launch.  Measured (steps/s against 128-tiles everywhere):
//   B X     256 from m = 768: GPT-2-small (768) 474-476 against 466-470,
//           GPT-2-XL (1600) B X 6.1 against 6.4 ms per phase;
//   Gram    256 from m = 1536: GPT-2-XL Gram 2.9 against 3.1 ms per phase;
//           GPT-2-small's 256-tile Gram launches take 84 instead of 59 us
//           (few tiles, filling the chip in fewer, emptier waves);
//   square  256 where m is a multiple of 256 (GPT-2-small with it: 477-479)
//           or from m = 2048; GPT-2-XL's remainder strip makes its square
//           slower (1.86 against 1.66 ms per phase).
// 4096 x 4096: 256-tiles in every phase, 580 against 535 steps/s.
// MUON_TILE_POLICY 1 / 2 force 128 / 256 (measurement builds).
#ifndef MUON_TILE_POLICY
#define MUON_TILE_POLICY 0
#endif
int choose_tile(int m, int phase) {
  if (MUON_TILE_POLICY == 1) return kTileM;
  if (MUON_TILE_POLICY == 2) return kTileL;
  bool large = false;
  if (phase == kGram) large = m >= 1536;
  else if (phase == kSquare) large = m >= 2048 || (m >= 768 && m % 256 == 0);
  else large = m >= 768;
  return large ? kTileL : kTileM;
}

// suffix of a GEMM launch's phase name per tile edge
const char* tile_tag(bool f32, int cfg) { return !f32 && cfg == kTileL ? "x256" : ""; }

struct SlotPlan {
  int64_t d = 0;
  int nblocks = 0, dp = 0;
  size_t off_s = 0, off_l = 0, off_li = 0, off_sinv = 0;   // nblocks consecutive dp x dp blocks each
  size_t off_acc = 0, off_cnt = 0;                          // running X^T X sums and sample counts
};

struct Plan {
  std::vector<UnitPlan> units;
  std::vector<SlotPlan> slots;
  std::vector<int> prec_tensors;     // tensors with a preconditioner, in tensor order
  std::vector<size_t> off_p;         // their P buffers (float32, rows x cols)
  std::vector<ApplyTask> apply;
  size_t off_pdev = 0, off_apply = 0;
  int apply_bf16 = 0;                // apply tasks of bf16-gradient tensors, first in `apply`
  std::vector<Group> groups;  // by NS precision (bf16 first) and lane
  std::vector<int> adam_tensors;     // kind-ADAMW tensors, in tensor order
  std::vector<AdamTask> adam_tasks;
  size_t off_adam_dev = 0, off_adam_tasks = 0, off_adam_state = 0;
  size_t off_flags = 0, off_partials = 0, off_norms = 0;
  size_t off_mpart = 0;              // refresh scratch (moment partials, float64 S^-1 sum), all slots
  size_t meta_bytes = 0, total = 0;
  int total_k1_tiles = 0;
  int64_t zero_bytes = 0;  // bytes of NS buffers (zero-filled at init)
};

bool finite(float x) { return std::isfinite(x); }

float shape_scale(int64_t rows, int64_t cols, int mode) {
  switch (mode) {
    case MUON_SCALE_NONE: return 1.f;
    case MUON_SCALE_ORIGINAL: return std::sqrt(std::max(1.0, double(rows) / double(cols)));
    case MUON_SCALE_MATCH_RMS_ADAMW: return float(0.2 * std::sqrt(double(std::max(rows, cols))));
    case MUON_SCALE_SPECTRAL: return float(std::sqrt(double(rows) / double(cols)));
    default: return 1.f;
  }
}

muon_status_t validate(const muon_tensor_t* ts, int32_t n, const muon_precond_t* pcs, int32_t npc,
                       const muon_hparams_t* hp) {
  if (!hp) return fail(MUON_ERR_NULL_ARG, "hparams is NULL");
  if (n < 0) return fail(MUON_ERR_BAD_ARG, "n_tensors < 0");
  if (n > 0 && !ts) return fail(MUON_ERR_NULL_ARG, "tensors is NULL");
  if (npc < 0) return fail(MUON_ERR_BAD_ARG, "n_preconds < 0");
  if (npc > 0 && !pcs) return fail(MUON_ERR_NULL_ARG, "preconds is NULL");
  if (hp->ns_steps < 0 || hp->ns_steps > 64) return fail(MUON_ERR_BAD_ARG, "ns_steps must be in [0, 64]");
  if (!finite(hp->lr) || !finite(hp->momentum) || !finite(hp->weight_decay) || !finite(hp->eps) ||
      !finite(hp->ns_a) || !finite(hp->ns_b) || !finite(hp->ns_c))
    return fail(MUON_ERR_BAD_ARG, "non-finite hyper-parameter");
  if (hp->eps < 0.f) return fail(MUON_ERR_BAD_ARG, "eps must be >= 0");
  // the square phase folds b A into c (A A + (b/c) A)
  if (hp->ns_steps > 0 && hp->ns_c == 0.f)
    return fail(MUON_ERR_BAD_ARG, "ns_c must be nonzero (the quintic's A^2 coefficient)");
  if (hp->scale_mode < MUON_SCALE_NONE || hp->scale_mode > MUON_SCALE_SPECTRAL)
    return fail(MUON_ERR_BAD_ARG, "unknown scale_mode");
  if (hp->momentum_form != MUON_MOM_EMA && hp->momentum_form != MUON_MOM_SGD)
    return fail(MUON_ERR_BAD_ARG, "unknown momentum_form");
  if (!finite(hp->adam_lr) || !finite(hp->adam_eps) || !finite(hp->adam_weight_decay) ||
      !(hp->adam_beta1 >= 0.f && hp->adam_beta1 < 1.f) || !(hp->adam_beta2 >= 0.f && hp->adam_beta2 < 1.f) ||
      hp->adam_eps < 0.f)
    return fail(MUON_ERR_BAD_ARG, "AdamW hyper-parameters: finite lr, eps >= 0, decay, betas in [0, 1)");
  for (int32_t k = 0; k < npc; ++k) {
    if (pcs[k].d < 1 || pcs[k].nblocks < 1 || pcs[k].d > 16384 || pcs[k].nblocks > 64)
      return fail(MUON_ERR_BAD_SHAPE, "preconditioner " + std::to_string(k) + ": bad d or nblocks");
  }
  struct Range { uintptr_t lo, hi; int t; const char* what; };
  std::vector<Range> ranges;
  for (int32_t i = 0; i < n; ++i) {
    const muon_tensor_t& t = ts[i];
    const std::string who = "tensor " + std::to_string(i) + ": ";
    if (!t.param || !t.grad || !t.momentum) return fail(MUON_ERR_NULL_ARG, who + "param, grad and momentum are required");
    if (t.dtype != MUON_F32 && t.dtype != MUON_BF16) return fail(MUON_ERR_BAD_DTYPE, who + "dtype must be MUON_F32 or MUON_BF16");
    if (t.rows < 1 || t.cols < 1 || t.rows > (1 << 20) || t.cols > (1 << 20))
      return fail(MUON_ERR_BAD_SHAPE, who + "rows and cols must be in [1, 2^20]");
    if (t.ld_param < t.cols || t.ld_grad < t.cols || t.ld_momentum < t.cols)
      return fail(MUON_ERR_BAD_SHAPE, who + "leading dimensions must be >= cols");
    if (t.kind != MUON_KIND_MUON && t.kind != MUON_KIND_ADAMW)
      return fail(MUON_ERR_BAD_ARG, who + "kind must be MUON_KIND_MUON or MUON_KIND_ADAMW");
    const bool adam = t.kind == MUON_KIND_ADAMW;
    if (adam) {
      if (!t.exp_avg_sq) return fail(MUON_ERR_NULL_ARG, who + "an AdamW tensor needs exp_avg_sq");
      if (t.split_rows != 0 || t.precond != -1 || t.update_out)
        return fail(MUON_ERR_BAD_ARG, who + "an AdamW tensor takes no split_rows, precond or update_out");
      if (reinterpret_cast<uintptr_t>(t.exp_avg_sq) % 4) return fail(MUON_ERR_ALIGNMENT, who + "exp_avg_sq misaligned");
    } else if (t.exp_avg_sq) {
      return fail(MUON_ERR_BAD_ARG, who + "exp_avg_sq is only for AdamW tensors");
    }
    if (t.split_rows < 0 || (t.split_rows > 0 && t.rows % t.split_rows != 0))
      return fail(MUON_ERR_BAD_SHAPE, who + "split_rows must be 0 or divide rows");
    if (t.precond < -1 || t.precond >= npc) return fail(MUON_ERR_BAD_ARG, who + "precond slot out of range");
    if (t.precond >= 0) {
      const muon_precond_t& pc = pcs[t.precond];
      if (t.cols != pc.d * pc.nblocks)
        return fail(MUON_ERR_BAD_SHAPE, who + "cols must equal d * nblocks of its preconditioner");
    }
    if (!finite(t.lr_mult)) return fail(MUON_ERR_BAD_ARG, who + "lr_mult is not finite");
    const size_t es = t.dtype == MUON_F32 ? 4 : 2;
    if (reinterpret_cast<uintptr_t>(t.param) % es || reinterpret_cast<uintptr_t>(t.grad) % es ||
        reinterpret_cast<uintptr_t>(t.momentum) % 4 || reinterpret_cast<uintptr_t>(t.update_out) % 4)
      return fail(MUON_ERR_ALIGNMENT, who + "pointers must be aligned to their element size");
    const int64_t h = t.split_rows ? t.split_rows : t.rows;
    const int64_t m = std::min<int64_t>(h, t.cols), nn = std::max<int64_t>(h, t.cols);
    const int64_t TE = t.dtype == MUON_F32 ? kTileF32 : kTileEdgeM;   // units are padded to 128
    if (!adam && round_up(m, TE) * round_up(nn, TE) > (int64_t(1) << 31))
      return fail(MUON_ERR_UNSUPPORTED, who + "matrix too large for one orthogonalisation unit");
    auto add = [&](const void* p, int64_t ld, size_t esz, const char* what) {
      const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
      const uintptr_t hi = lo + (size_t((t.rows - 1) * ld + t.cols)) * esz;
      ranges.push_back({lo, hi, i, what});
    };
    add(t.param, t.ld_param, es, "param");
    add(t.grad, t.ld_grad, es, "grad");
    add(t.momentum, t.ld_momentum, 4, "momentum");
    if (t.update_out) add(t.update_out, t.cols, 4, "update_out");
    if (t.exp_avg_sq) add(t.exp_avg_sq, t.ld_momentum, 4, "exp_avg_sq");
  }
  std::sort(ranges.begin(), ranges.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t k = 1; k < ranges.size(); ++k)
    if (ranges[k].lo < ranges[k - 1].hi)
      return fail(MUON_ERR_ALIASING, std::string("buffers overlap: tensor ") + std::to_string(ranges[k - 1].t) +
                                         " " + ranges[k - 1].what + " and tensor " + std::to_string(ranges[k].t) +
                                         " " + ranges[k].what);
  return MUON_OK;
}

constexpr int kXcds = 8;   // MI355X: 8 accelerator complex dies, one L2 each
#ifndef MUON_LANES
#define MUON_LANES 2
#endif
constexpr int kLanes = MUON_LANES;       // lanes (streams) a large precision group is split into
constexpr int kLaneMinUnits = 4 * kLanes;    // matrices of one precision needed for that split
constexpr int64_t kLaneMaxBxTiles = 16384;   // ... and at most this many B X tiles per phase

// The output tiles of one unit's GEMM phase, appended to the lists of their
// shape (unit index gi within its group).  The Gram and the square compute
// the upper tiles (i <= j) of the mp x mp product, B X every tile of mp x np.
// A phase of 128-tiles (or float32 tiles) tiles the whole padded unit; a
// phase of 256-tiles covers [0, 256 floor(mp / 256)) x [0, 256 floor(np /
// 256)) with them and the remaining strips (at most 128 wide, as mp and np
// are multiples of 128) with 128 x 128 tiles: for the square products the
// upper tiles of the last column strip, for B X the last column strip and
// then the last row strip.  B X tiles go column by column: the tiles that
// run together then share one column strip of X and all of B (a unit's B is
// the smaller operand), so each strip of X comes from HBM about once.
void unit_tiles(const UnitPlan& u, int ph, int gi, std::vector<GemmTask> (&lists)[kTileCfgs]) {
  const int tc = u.tile[ph];
  const int te = tile_edge(u.f32, tc);
  const int nm = u.mp / te, nn = u.np / te;     // whole tiles of this shape
  std::vector<GemmTask>& main = lists[tc];
  if (ph != kBX) {
    for (int a = 0; a < nm; ++a)
      for (int b = a; b < nm; ++b) main.push_back({gi, a, b, 0});
  } else {
    for (int b = 0; b < nn; ++b)
      for (int a = 0; a < nm; ++a) main.push_back({gi, a, b, 0});
  }
  if (tc != kTileL) return;
  std::vector<GemmTask>& rest = lists[kTileM];
  const int r = te / kTileEdgeM;                // 128-tiles per 256-tile edge
  const int mm = u.mp / kTileEdgeM, mn = u.np / kTileEdgeM;
  if (ph != kBX) {
    for (int j = r * nm; j < mm; ++j)
      for (int i = 0; i <= j; ++i) rest.push_back({gi, i, j, 0});
  } else {
    for (int j = r * nn; j < mn; ++j)
      for (int i = 0; i < mm; ++i) rest.push_back({gi, i, j, 0});
    for (int j = 0; j < r * nn; ++j)
      for (int i = r * nm; i < mm; ++i) rest.push_back({gi, i, j, 0});
  }
}

// XCD-aware order of one phase's tiles.  The dispatcher hands block b to XCD
// b mod 8, and each XCD has its own L2, so tiles that share operand rows
// (the tiles of one matrix) should run on one XCD.  A matrix costing more
// than an eighth of the phase is cut into contiguous parts (row-major tile
// order) of about an eighth each; the parts and the remaining whole matrices
// are then assigned to XCDs longest-processing-time first.  Each XCD's
// sequence lists its tiles costliest first, and the sequences are
// interleaved so block 8*s + x runs the s-th tile of XCD x; shorter
// sequences are padded with empty tasks (unit = -1).
std::vector<GemmTask> xcd_order(const std::vector<GemmTask>& tiles, const std::vector<UnitPlan>& units,
                                const Group& g, int phase) {
  auto tile_cost = [&](const GemmTask& t) {
    const UnitPlan& u = units[g.units[t.unit]];
    return phase == kGram ? int64_t(u.np) : int64_t(u.mp);
  };
  std::vector<int64_t> ucost(g.units.size(), 0);
  std::vector<std::vector<GemmTask>> per_unit(g.units.size());
  int64_t total = 0;
  for (const GemmTask& t : tiles) {
    ucost[t.unit] += tile_cost(t);
    per_unit[t.unit].push_back(t);
    total += tile_cost(t);
  }
  const int64_t share = std::max<int64_t>(1, (total + kXcds - 1) / kXcds);
  struct Part { std::vector<GemmTask> tiles; int64_t cost = 0; };
  std::vector<Part> parts;
  for (size_t uidx = 0; uidx < per_unit.size(); ++uidx) {
    if (per_unit[uidx].empty()) continue;
    const int64_t k = ucost[uidx] > share ? (ucost[uidx] + share - 1) / share : 1;
    const int64_t target = (ucost[uidx] + k - 1) / k;
    parts.emplace_back();
    for (const GemmTask& t : per_unit[uidx]) {
      if (parts.back().cost >= target) parts.emplace_back();
      parts.back().tiles.push_back(t);
      parts.back().cost += tile_cost(t);
    }
  }
  std::stable_sort(parts.begin(), parts.end(), [](const Part& a, const Part& b) { return a.cost > b.cost; });
  std::vector<int64_t> load(kXcds, 0);
  std::vector<std::vector<GemmTask>> seq(kXcds);
  for (const Part& pt : parts) {
    const int x = int(std::min_element(load.begin(), load.end()) - load.begin());
    load[x] += pt.cost;
    seq[x].insert(seq[x].end(), pt.tiles.begin(), pt.tiles.end());
  }
  size_t longest = 0;
  for (int x = 0; x < kXcds; ++x) {
    std::stable_sort(seq[x].begin(), seq[x].end(),
                     [&](const GemmTask& a, const GemmTask& b) { return tile_cost(a) > tile_cost(b); });
    longest = std::max(longest, seq[x].size());
  }
  std::vector<GemmTask> out;
  out.reserve(longest * kXcds);
  for (size_t sidx = 0; sidx < longest; ++sidx)
    for (int x = 0; x < kXcds; ++x)
      out.push_back(sidx < seq[x].size() ? seq[x][sidx] : GemmTask{-1, 0, 0, 0});
  // drop trailing empty tasks
  while (!out.empty() && out.back().unit < 0) out.pop_back();
  return out;
}

// Self-check of a group's GEMM task lists, run on every plan: counted on the
// grid of g x g blocks (g: the 128-tile edge, 64 for float32 units), B X's
// tiles cover every block of each unit's m_p x n_p output exactly once, and
// the Gram's and the square's tiles every block on or above the diagonal
// exactly once, reaching below it only inside diagonal tiles (whose lower
// part they store directly; the other tiles are mirror-stored).
bool tiles_cover_exactly(const std::vector<UnitPlan>& units, const Group& g) {
  for (int ph = 0; ph < 3; ++ph) {
    std::vector<std::vector<uint8_t>> cnt(g.units.size());
    std::vector<int> gr(g.units.size()), gc(g.units.size());
    for (size_t gi = 0; gi < g.units.size(); ++gi) {
      const UnitPlan& u = units[g.units[gi]];
      const int e = tile_edge(u.f32, kTileM);
      if (u.mp % e || u.np % e) return false;
      gr[gi] = u.mp / e;
      gc[gi] = ph == kBX ? u.np / e : u.mp / e;
      cnt[gi].assign(size_t(gr[gi]) * gc[gi], 0);
    }
    for (int tc = 0; tc < kTileCfgs; ++tc)
      for (const GemmTask& t : g.gemm[ph][tc]) {
        if (t.unit < 0) continue;
        if (size_t(t.unit) >= g.units.size()) return false;
        const UnitPlan& u = units[g.units[t.unit]];
        const int r = tile_edge(u.f32, tc) / tile_edge(u.f32, kTileM);
        if (u.f32 && tc != kTileM) return false;
        for (int bi = t.ti * r; bi < (t.ti + 1) * r; ++bi)
          for (int bj = t.tj * r; bj < (t.tj + 1) * r; ++bj) {
            if (bi < 0 || bj < 0 || bi >= gr[t.unit] || bj >= gc[t.unit]) return false;
            if (ph != kBX && bi > bj) {
              if (t.ti != t.tj) return false;
              continue;
            }
            if (++cnt[t.unit][size_t(bi) * gc[t.unit] + bj] > 1) return false;
          }
      }
    for (size_t gi = 0; gi < g.units.size(); ++gi)
      for (int bi = 0; bi < gr[gi]; ++bi)
        for (int bj = ph == kBX ? 0 : bi; bj < gc[gi]; ++bj)
          if (cnt[gi][size_t(bi) * gc[gi] + bj] != 1) return false;
  }
  return true;
}

muon_status_t build_plan(const muon_tensor_t* ts, int32_t n, const muon_precond_t* pcs, int32_t npc,
                         const muon_hparams_t* hp, Plan& plan, bool single_lane = false) {
  muon_status_t st = validate(ts, n, pcs, npc, hp);
  if (st != MUON_OK) return st;
  plan = Plan();
  // Newton-Muon slots and preconditioned tensors
  for (int32_t k = 0; k < npc; ++k) {
    SlotPlan sp;
    sp.d = pcs[k].d;
    sp.nblocks = pcs[k].nblocks;
    sp.dp = int(round_up(sp.d, kPrecondPad));
    plan.slots.push_back(sp);
  }
  // apply tiles: those of bf16-gradient tensors first, then float32 ones
  // (each dtype has its own kernel, with the LDS its planes need)
  std::vector<ApplyTask> apply_f32;
  for (int32_t i = 0; i < n; ++i) {
    if (ts[i].precond < 0) continue;
    const int pi = int(plan.prec_tensors.size());
    plan.prec_tensors.push_back(i);
    const SlotPlan& sp = plan.slots[ts[i].precond];
    const int trs = int((ts[i].rows + 127) / 128), tcs = int((sp.d + 63) / 64);   // 128 x 64 tiles
    std::vector<ApplyTask>& dst = ts[i].dtype == MUON_F32 ? apply_f32 : plan.apply;
    for (int blk = 0; blk < sp.nblocks; ++blk)
      for (int r = 0; r < trs; ++r)
        for (int c = 0; c < tcs; ++c) dst.push_back({pi, r, c, blk});
  }
  plan.apply_bf16 = int(plan.apply.size());
  plan.apply.insert(plan.apply.end(), apply_f32.begin(), apply_f32.end());
  // AdamW tensors: rows of `len` elements in chunks of kAdamChunk; a fully
  // contiguous tensor is one row of rows*cols elements
  for (int32_t i = 0; i < n; ++i) {
    const muon_tensor_t& t = ts[i];
    if (t.kind != MUON_KIND_ADAMW) continue;
    const int ai = int(plan.adam_tensors.size());
    plan.adam_tensors.push_back(i);
    const bool flat = t.ld_param == t.cols && t.ld_grad == t.cols && t.ld_momentum == t.cols;
    const int64_t nrows = flat ? 1 : t.rows, len = flat ? t.rows * t.cols : t.cols;
    for (int64_t r = 0; r < nrows; ++r)
      for (int64_t c0 = 0; c0 < len; c0 += kAdamChunk) plan.adam_tasks.push_back({ai, int32_t(r), c0});
  }
  // units
  for (int32_t i = 0; i < n; ++i) {
    const muon_tensor_t& t = ts[i];
    if (t.kind == MUON_KIND_ADAMW) continue;
    const int64_t h = t.split_rows ? t.split_rows : t.rows;
    for (int64_t b = 0; b < t.rows / h; ++b) {
      UnitPlan u;
      u.tensor = i;
      u.block = int(b);
      u.row0 = b * h;
      u.rows = int(h);
      u.cols = int(t.cols);
      u.side = h > t.cols ? kRight : kLeft;
      u.m = int(std::min<int64_t>(h, t.cols));
      u.n = int(std::max<int64_t>(h, t.cols));
      u.f32 = t.dtype == MUON_F32 || u.m < kMinBf16NsSide;   // NS precision of the unit
      for (int ph = 0; ph < 3; ++ph) u.tile[ph] = u.f32 ? kTileM : choose_tile(u.m, ph);
      u.mp = int(round_up(u.m, tile_edge(u.f32, kTileM)));
      u.np = int(round_up(u.n, tile_edge(u.f32, kTileM)));
      u.lr_scale = shape_scale(h, t.cols, hp->scale_mode) * t.lr_mult;
      const int ewr = u.side == kLeft ? kEwRows : kEwRRows, ewc = u.side == kLeft ? kEwCols : kEwRCols;
      u.k1_tr = int((h + ewr - 1) / ewr);
      u.k1_tc = int((t.cols + ewc - 1) / ewc);
      u.k1_ntiles = u.k1_tr * u.k1_tc;
      u.k1_tile0 = plan.total_k1_tiles;
      plan.total_k1_tiles += u.k1_ntiles;
      plan.units.push_back(u);
    }
  }
  // groups: one per NS precision; a precision with many matrices is split
  // into lanes of about equal Newton-Schulz work (longest first), which
  // muon_step runs on separate streams so one lane's ramp-up and tail
  // overlap another's tiles.  The float32 group takes the lanes after the
  // bf16 group's while both fit in kLanes, so two small groups of different
  // precision (launch-bound chains) run side by side.
  int bf16_lanes = 0;
  for (int f = 0; f < 2; ++f) {
    std::vector<int> ids;
    for (size_t k = 0; k < plan.units.size(); ++k)
      if (plan.units[k].f32 == (f == 1)) ids.push_back(int(k));
    if (ids.empty()) continue;
    // lanes pay off when a phase is short (a few waves of tiles, so its
    // ramp and tail are a large share); with very many tiles more streams
    // only add cache contention
    int64_t bx_tiles = 0;
    for (int k : ids) {
      std::vector<GemmTask> lists[kTileCfgs];
      unit_tiles(plan.units[k], kBX, 0, lists);
      for (const auto& l : lists) bx_tiles += int64_t(l.size());
    }
    const int lanes = !single_lane && ids.size() >= size_t(kLaneMinUnits) && bx_tiles <= kLaneMaxBxTiles ? kLanes : 1;
    auto cost = [&](int k) {
      const UnitPlan& u = plan.units[k];
      return double(u.mp) * u.mp * (u.mp + 3.0 * u.np);
    };
    std::stable_sort(ids.begin(), ids.end(), [&](int a, int b) { return cost(a) > cost(b); });
    std::vector<Group> lg(lanes);
    std::vector<double> load(lanes, 0.0);
    for (int k : ids) {
      const int l = int(std::min_element(load.begin(), load.end()) - load.begin());
      load[l] += cost(k);
      lg[l].units.push_back(k);
    }
    const int lane0 = !single_lane && f == 1 && bf16_lanes + lanes <= kLanes ? bf16_lanes : 0;
    if (f == 0) bf16_lanes = lanes;
    for (int l = 0; l < lanes; ++l) {
      lg[l].f32 = f == 1;
      lg[l].lane = lane0 + l;
      std::sort(lg[l].units.begin(), lg[l].units.end());   // tensor order inside a lane
      for (size_t gi = 0; gi < lg[l].units.size(); ++gi) plan.units[lg[l].units[gi]].group_index = int(gi);
      plan.groups.push_back(std::move(lg[l]));
    }
  }
  // Small phases take 128-tiles.  A group's phase with fewer 256-tiles than
  // CUs runs them as one partial round, one block per CU; when the same
  // phase as 128-tiles fits in one round of the chip's block slots (two per
  // CU), those finish in about half the time, a 256-tile being four
  // 128-tiles' work on one CU.  (The Newton-Muon layer's six 768-row units,
  // 36 square and 108 B X 256-tiles: 1985 steps/s with them.)  Larger
  // phases keep the per-unit choice.
  constexpr int64_t kCUs = 256, kSlots128 = 2 * kCUs;
  for (Group& g : plan.groups) {
    if (g.f32 || MUON_TILE_POLICY != 0) continue;
    for (int ph = 0; ph < 3; ++ph) {
      int64_t n256 = 0, n128 = 0;   // the phase's 256-tiles, and its 128-tiles were every unit to take them
      for (int k : g.units) {
        const UnitPlan& u = plan.units[k];
        const int64_t rm = u.mp / kTileEdgeM, rn = (ph == kBX ? u.np : u.mp) / kTileEdgeM;
        n128 += ph == kBX ? rm * rn : rm * (rm + 1) / 2;
        if (u.tile[ph] == kTileL) {
          const int64_t lm = u.mp / kTileEdgeL, ln = (ph == kBX ? u.np : u.mp) / kTileEdgeL;
          n256 += ph == kBX ? lm * ln : lm * (lm + 1) / 2;
        }
      }
      if (n256 > 0 && n256 < kCUs && n128 <= kSlots128)
        for (int k : g.units) plan.units[k].tile[ph] = kTileM;
    }
  }
  // tile lists
  for (Group& g : plan.groups) {
    for (size_t gi = 0; gi < g.units.size(); ++gi) {
      const UnitPlan& u = plan.units[g.units[gi]];
      for (int r = 0; r < u.k1_tr; ++r)
        for (int c = 0; c < u.k1_tc; ++c) g.ew.push_back({int(gi), r, c, r * u.k1_tc + c});
      for (int ph = 0; ph < 3; ++ph) unit_tiles(u, ph, int(gi), g.gemm[ph]);
    }
    for (int ph = 0; ph < 3; ++ph)
      for (int tc = 0; tc < kTileCfgs; ++tc) g.gemm[ph][tc] = xcd_order(g.gemm[ph][tc], plan.units, g, ph);
    if (!tiles_cover_exactly(plan.units, g))
      return fail(MUON_ERR_UNSUPPORTED, "internal: GEMM tile lists do not cover the outputs exactly once");
  }
  // workspace: metadata first, then the NS buffers
  size_t off = 0;
  plan.off_flags = off; off += kAlign;
  plan.off_partials = off; off = align_up(off + sizeof(float) * plan.total_k1_tiles);
  plan.off_norms = off; off = align_up(off + sizeof(float) * plan.units.size());
  for (Group& g : plan.groups) {
    g.off_units = off; off = align_up(off + sizeof(UnitDev) * g.units.size());
    g.off_ew = off; off = align_up(off + sizeof(EwTask) * g.ew.size());
    for (int ph = 0; ph < 3; ++ph)
      for (int tc = 0; tc < kTileCfgs; ++tc) {
        g.off_gemm[ph][tc] = off;
        off = align_up(off + sizeof(GemmTask) * g.gemm[ph][tc].size());
      }
  }
  plan.off_pdev = off; off = align_up(off + sizeof(PrecondDev) * plan.prec_tensors.size());
  plan.off_apply = off; off = align_up(off + sizeof(ApplyTask) * plan.apply.size());
  plan.off_adam_dev = off; off = align_up(off + sizeof(AdamDev) * plan.adam_tensors.size());
  plan.off_adam_tasks = off; off = align_up(off + sizeof(AdamTask) * plan.adam_tasks.size());
  plan.off_adam_state = off; off = align_up(off + sizeof(AdamState));
  plan.meta_bytes = off;
  for (UnitPlan& u : plan.units) {
    const size_t es = u.f32 ? 4 : 2;
    const size_t xs = size_t(u.mp) * u.np * es, as = size_t(u.mp) * u.mp * es;
    u.off_xh0 = off; off = align_up(off + xs);
    u.off_xh1 = off; off = align_up(off + xs);
    if (!u.f32) { u.off_xl = off; off = align_up(off + size_t(u.mp) * u.np); }   // int8 master corrections
    u.off_a = off; off = align_up(off + as);
    u.off_b = off; off = align_up(off + as);
  }
  for (SlotPlan& sp : plan.slots) {
    const size_t blk = size_t(sp.dp) * sp.dp * sp.nblocks;
    sp.off_s = off; off = align_up(off + blk * sizeof(float));
    sp.off_l = off; off = align_up(off + blk * sizeof(double));
    sp.off_li = off; off = align_up(off + blk * sizeof(double));
    sp.off_sinv = off; off = align_up(off + blk * kSinvPlanes * sizeof(uint16_t));
    sp.off_acc = off; off = align_up(off + blk * sizeof(float));
    sp.off_cnt = off; off = align_up(off + size_t(sp.nblocks) * sizeof(double));
  }
  // scratch of the refresh (one at a time per handle): the split partials
  // of the second moment, then the float64 sum of S^-1
  size_t mpart = 0;
  for (const SlotPlan& sp : plan.slots) {
    const int splits = moment_splits(sp.dp, false, INT64_MAX);   // bf16 tiles split the most
    const size_t sq = size_t(sp.dp) * sp.dp;
    mpart = std::max({mpart, sq * sizeof(double), splits > 1 ? size_t(splits) * sq * sizeof(float) : size_t(0)});
  }
  if (mpart) { plan.off_mpart = off; off = align_up(off + mpart); }
  for (int ti : plan.prec_tensors) {
    plan.off_p.push_back(off);
    off = align_up(off + size_t(ts[ti].rows) * ts[ti].cols * sizeof(float));
  }
  plan.total = std::max<size_t>(off, kAlign);
  plan.zero_bytes = int64_t(plan.total - plan.meta_bytes);
  return MUON_OK;
}

std::vector<uint8_t> build_meta(const Plan& plan, const muon_tensor_t* ts, uint8_t* ws) {
  std::vector<uint8_t> meta(plan.meta_bytes, 0);
  for (const Group& g : plan.groups) {
    for (size_t gi = 0; gi < g.units.size(); ++gi) {
      const UnitPlan& up = plan.units[g.units[gi]];
      const muon_tensor_t& t = ts[up.tensor];
      const size_t es = t.dtype == MUON_F32 ? 4 : 2;   // element size of param/grad
      UnitDev d;
      std::memset(&d, 0, sizeof(d));
      if (t.precond < 0) {
        d.grad = static_cast<const uint8_t*>(t.grad) + size_t(up.row0) * t.ld_grad * es;
        d.ld_grad = t.ld_grad;
        d.grad_f32 = t.dtype == MUON_F32;
        d.vec_grad = reinterpret_cast<uintptr_t>(t.grad) % 16 == 0 && (t.ld_grad * es) % 16 == 0;
      } else {   // the momentum phase reads P = G S^-1 (float32, ld = cols)
        const size_t pi = size_t(std::find(plan.prec_tensors.begin(), plan.prec_tensors.end(), up.tensor) -
                                 plan.prec_tensors.begin());
        d.grad = ws + plan.off_p[pi] + size_t(up.row0) * t.cols * sizeof(float);
        d.ld_grad = t.cols;
        d.grad_f32 = 1;
        d.vec_grad = (t.cols * sizeof(float)) % 16 == 0;
      }
      d.mom = t.momentum + size_t(up.row0) * t.ld_momentum;
      d.ld_mom = t.ld_momentum;
      d.vec_mom = reinterpret_cast<uintptr_t>(t.momentum) % 16 == 0 && (t.ld_momentum * 4) % 16 == 0;
      d.param = static_cast<uint8_t*>(t.param) + size_t(up.row0) * t.ld_param * es;
      d.ld_param = t.ld_param;
      d.param_f32 = t.dtype == MUON_F32;
      d.vec_param = reinterpret_cast<uintptr_t>(t.param) % 16 == 0 && (t.ld_param * es) % 16 == 0;
      d.update_out = t.update_out ? t.update_out + size_t(up.row0) * t.cols : nullptr;
      d.ld_out = t.cols;
      d.vec_out = t.update_out && reinterpret_cast<uintptr_t>(t.update_out) % 16 == 0 && (t.cols * 4) % 16 == 0;
      d.rows = up.rows;
      d.cols = up.cols;
      d.side = up.side;
      d.m = up.m; d.n = up.n; d.mp = up.mp; d.np = up.np;
      d.xh[0] = ws + up.off_xh0;
      d.xh[1] = ws + up.off_xh1;
      d.xl = up.f32 ? nullptr : ws + up.off_xl;
      d.a = ws + up.off_a;
      d.b = ws + up.off_b;
      d.partials = reinterpret_cast<float*>(ws + plan.off_partials) + up.k1_tile0;
      d.norm = reinterpret_cast<float*>(ws + plan.off_norms) + g.units[gi];
      d.k1_tile0 = up.k1_tile0;
      d.k1_ntiles = up.k1_ntiles;
      d.lr_scale = up.lr_scale;
      std::memcpy(meta.data() + g.off_units + gi * sizeof(UnitDev), &d, sizeof(d));
    }
    auto put = [&](size_t o, const void* src, size_t bytes) {
      if (bytes) std::memcpy(meta.data() + o, src, bytes);
    };
    put(g.off_ew, g.ew.data(), g.ew.size() * sizeof(EwTask));
    for (int ph = 0; ph < 3; ++ph)
      for (int tc = 0; tc < kTileCfgs; ++tc)
        put(g.off_gemm[ph][tc], g.gemm[ph][tc].data(), g.gemm[ph][tc].size() * sizeof(GemmTask));
  }
  for (size_t pi = 0; pi < plan.prec_tensors.size(); ++pi) {
    const muon_tensor_t& t = ts[plan.prec_tensors[pi]];
    const SlotPlan& sp = plan.slots[t.precond];
    const size_t es = t.dtype == MUON_F32 ? 4 : 2;
    PrecondDev pd;
    std::memset(&pd, 0, sizeof(pd));
    pd.grad = t.grad;
    pd.ld_grad = t.ld_grad;
    pd.grad_f32 = t.dtype == MUON_F32;
    pd.vec_grad = reinterpret_cast<uintptr_t>(t.grad) % 16 == 0 && (t.ld_grad * es) % 16 == 0 && sp.d % 8 == 0;
    pd.p = reinterpret_cast<float*>(ws + plan.off_p[pi]);
    pd.ld_p = t.cols;
    pd.sinv = reinterpret_cast<const uint16_t*>(ws + sp.off_sinv);
    pd.rows = int(t.rows);
    pd.d = int(sp.d);
    pd.dp = sp.dp;
    pd.nblocks = sp.nblocks;
    std::memcpy(meta.data() + plan.off_pdev + pi * sizeof(PrecondDev), &pd, sizeof(pd));
  }
  if (!plan.apply.empty())
    std::memcpy(meta.data() + plan.off_apply, plan.apply.data(), plan.apply.size() * sizeof(ApplyTask));
  for (size_t ai = 0; ai < plan.adam_tensors.size(); ++ai) {
    const muon_tensor_t& t = ts[plan.adam_tensors[ai]];
    const size_t es = t.dtype == MUON_F32 ? 4 : 2;
    const bool flat = t.ld_param == t.cols && t.ld_grad == t.cols && t.ld_momentum == t.cols;
    AdamDev d;
    std::memset(&d, 0, sizeof(d));
    d.param = t.param;
    d.grad = t.grad;
    d.m = t.momentum;
    d.v = t.exp_avg_sq;
    d.ld_param = t.ld_param;
    d.ld_grad = t.ld_grad;
    d.ld_mom = t.ld_momentum;
    d.len = flat ? t.rows * t.cols : t.cols;
    d.f32 = t.dtype == MUON_F32;
    auto al = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
    d.vec = al(t.param) && al(t.grad) && al(t.momentum) && al(t.exp_avg_sq) &&
            (flat || ((t.ld_param * es) % 16 == 0 && (t.ld_grad * es) % 16 == 0 && (t.ld_momentum * 4) % 16 == 0));
    d.lr_mult = t.lr_mult;
    std::memcpy(meta.data() + plan.off_adam_dev + ai * sizeof(AdamDev), &d, sizeof(d));
  }
  if (!plan.adam_tasks.empty())
    std::memcpy(meta.data() + plan.off_adam_tasks, plan.adam_tasks.data(), plan.adam_tasks.size() * sizeof(AdamTask));
  return meta;
}

}  // namespace

struct muon_handle_s {
  Plan plan;
  muon_hparams_t hp;
  std::vector<muon_tensor_t> tensors;
  uint8_t* ws = nullptr;
  std::vector<uint8_t> meta;  // host copy of the uploaded descriptors (kept for the async copy)
  hipStream_t last_stream = nullptr;
  std::vector<hipStream_t> lane_streams;              // lanes 1.. (created when the plan has them)
  std::vector<hipEvent_t> ev_joins;                   // one per lane stream
  hipStream_t aux_stream = nullptr;                   // AdamW beside the Muon phases
  hipEvent_t ev_aux = nullptr, ev_adam = nullptr;
  hipEvent_t ev_fork = nullptr;
  std::vector<hipEvent_t> events;
  std::vector<std::string> phase_names;
  int static_device = -1;        // muon_init_static: the GPU whose scratch array holds the workspace
  uint64_t static_generation = 0;  // ... and which of its static inits this handle is
};

namespace {

// Enqueue one whole step.  With `ev` non-null, record ev[k] before launch k
// and ev[last] after the final one.
muon_status_t enqueue_step(muon_handle_t h, float lr, hipStream_t s, std::vector<hipEvent_t>* ev) {
  const Plan& plan = h->plan;
  const muon_hparams_t& hp = h->hp;
  size_t ek = 0;
  auto mark = [&]() -> bool {
    if (!ev) return true;
    return hipEventRecord((*ev)[ek++], s) == hipSuccess;
  };
  Range step_range("muon.step");
  if (!mark()) return fail(MUON_ERR_HIP, "hipEventRecord failed");
  if (!plan.apply.empty()) {
    Range r("muon.precond_apply");
    hipError_t e = launch_precond_apply(reinterpret_cast<const PrecondDev*>(h->ws + plan.off_pdev),
                                        reinterpret_cast<const ApplyTask*>(h->ws + plan.off_apply),
                                        plan.apply_bf16, int(plan.apply.size()) - plan.apply_bf16, s);
    if (e != hipSuccess || !mark()) return fail(MUON_ERR_HIP, std::string("precond apply launch: ") + hipGetErrorString(e));
  }
  // Lanes: the groups of lane l > 0 run on the handle's stream l, and the
  // AdamW launches on its auxiliary stream, all forked from `s` here (after
  // the preconditioner, which the momentum phase reads) and joined back into
  // it at the end (also under graph capture).  The timed variant keeps
  // everything on `s`, in order (AdamW first).
  const bool fork = !ev && (!h->lane_streams.empty() || h->aux_stream != nullptr);
  if (fork) {
    if (hipEventRecord(h->ev_fork, s) != hipSuccess) return fail(MUON_ERR_HIP, "lane fork failed");
    for (hipStream_t ls : h->lane_streams)
      if (hipStreamWaitEvent(ls, h->ev_fork, 0) != hipSuccess) return fail(MUON_ERR_HIP, "lane fork failed");
    if (h->aux_stream && hipStreamWaitEvent(h->aux_stream, h->ev_fork, 0) != hipSuccess)
      return fail(MUON_ERR_HIP, "lane fork failed");
  }
  auto launch_adam = [&](hipStream_t as) -> muon_status_t {
    Range r("muon.adamw");
    AdamState* st = reinterpret_cast<AdamState*>(h->ws + plan.off_adam_state);
    hipError_t e = launch_adam_tick(st, hp.adam_beta1, hp.adam_beta2, as);
    AdamParams ap{hp.adam_lr, hp.adam_beta1, hp.adam_beta2, hp.adam_eps, hp.adam_weight_decay, st,
                  reinterpret_cast<uint32_t*>(h->ws + plan.off_flags)};
    if (e == hipSuccess)
      e = launch_adamw(reinterpret_cast<const AdamDev*>(h->ws + plan.off_adam_dev),
                       reinterpret_cast<const AdamTask*>(h->ws + plan.off_adam_tasks), int(plan.adam_tasks.size()),
                       ap, as);
    if (e != hipSuccess || !mark()) return fail(MUON_ERR_HIP, std::string("adamw launch: ") + hipGetErrorString(e));
    return MUON_OK;
  };
  // AdamW is HBM-bound like the momentum phase: on its own stream it starts
  // once the first lane's momentum launch is done, beside the MFMA phases
  const bool adam_aside = fork && h->aux_stream != nullptr && !plan.adam_tasks.empty();
  if (!plan.adam_tasks.empty() && !adam_aside) {
    const muon_status_t st = launch_adam(s);
    if (st != MUON_OK) return st;
  }
  bool adam_pending = adam_aside;
  for (const Group& g : plan.groups) {
    if (g.units.empty()) continue;
    const hipStream_t gs = fork && g.lane > 0 ? h->lane_streams[g.lane - 1] : s;
    const UnitDev* units = reinterpret_cast<const UnitDev*>(h->ws + g.off_units);
    K1Params k1{hp.momentum, hp.nesterov, hp.momentum_form == MUON_MOM_SGD,
                reinterpret_cast<uint32_t*>(h->ws + plan.off_flags)};
    hipError_t e;
    {
      Range r("muon.momentum");
      e = launch_momentum(g.f32, units, reinterpret_cast<const EwTask*>(h->ws + g.off_ew), int(g.ew.size()), k1, gs);
    }
    if (e != hipSuccess || !mark()) return fail(MUON_ERR_HIP, std::string("momentum launch: ") + hipGetErrorString(e));
    if (adam_pending && g.lane == 0) {
      if (hipEventRecord(h->ev_adam, gs) != hipSuccess || hipStreamWaitEvent(h->aux_stream, h->ev_adam, 0) != hipSuccess)
        return fail(MUON_ERR_HIP, "adamw stream wait failed");
      const muon_status_t st = launch_adam(h->aux_stream);
      if (st != MUON_OK) return st;
      adam_pending = false;
    }
    for (int it = 0; it < hp.ns_steps; ++it) {
      GemmParams gp{hp.ns_a, hp.ns_b, hp.ns_c, hp.eps, it == 0, it == hp.ns_steps - 1, it & 1, 0,
                    lr, hp.weight_decay, reinterpret_cast<uint32_t*>(h->ws + plan.off_flags)};
      for (int ph = 0; ph < 3; ++ph)
        for (int tc : kLaunchOrder) {   // the 256-row tiles (the longer launches) first
          const std::vector<GemmTask>& tl = g.gemm[ph][tc];
          if (tl.empty()) continue;
          {
            static const char* const kRangeNames[3] = {"muon.gram", "muon.square", "muon.bx"};
            Range r(kRangeNames[ph]);
            e = launch_gemm(ph, g.f32, tc, units, reinterpret_cast<const GemmTask*>(h->ws + g.off_gemm[ph][tc]),
                            int(tl.size()), gp, gs);
          }
          if (e != hipSuccess || !mark())
            return fail(MUON_ERR_HIP, std::string(kPhaseNames[ph]) + " launch: " + hipGetErrorString(e));
        }
    }
    if (hp.ns_steps == 0) {   // otherwise the last B X phase applies the update
      K5Params k5{lr, hp.weight_decay, hp.eps, 0, reinterpret_cast<uint32_t*>(h->ws + plan.off_flags)};
      Range r("muon.update");
      e = launch_update(g.f32, units, reinterpret_cast<const EwTask*>(h->ws + g.off_ew), int(g.ew.size()), k5, gs);
      if (e != hipSuccess || !mark()) return fail(MUON_ERR_HIP, std::string("update launch: ") + hipGetErrorString(e));
    }
  }
  if (adam_pending) {
    const muon_status_t st = launch_adam(h->aux_stream);
    if (st != MUON_OK) return st;
  }
  if (fork) {
    for (size_t l = 0; l < h->lane_streams.size(); ++l)
      if (hipEventRecord(h->ev_joins[l], h->lane_streams[l]) != hipSuccess ||
          hipStreamWaitEvent(s, h->ev_joins[l], 0) != hipSuccess)
        return fail(MUON_ERR_HIP, "lane join failed");
    if (h->aux_stream && (hipEventRecord(h->ev_aux, h->aux_stream) != hipSuccess ||
                          hipStreamWaitEvent(s, h->ev_aux, 0) != hipSuccess))
      return fail(MUON_ERR_HIP, "lane join failed");
  }
  h->last_stream = s;
  return MUON_OK;
}

std::string plan_json(const Plan& plan, const muon_hparams_t& hp) {
  std::string s = "{\"units\":[";
  char buf[512];
  for (size_t i = 0; i < plan.units.size(); ++i) {
    const UnitPlan& u = plan.units[i];
    std::snprintf(buf, sizeof(buf),
                  "%s{\"tensor\":%d,\"block\":%d,\"row0\":%lld,\"rows\":%d,\"cols\":%d,\"side\":\"%s\","
                  "\"m\":%d,\"n\":%d,\"mp\":%d,\"np\":%d,\"ns\":\"%s\",\"tiles\":[%d,%d,%d],\"lr_scale\":%.9g,"
                  "\"k1_tiles\":%d}",
                  i ? "," : "", u.tensor, u.block, (long long)u.row0, u.rows, u.cols,
                  u.side == kLeft ? "left" : "right", u.m, u.n, u.mp, u.np, u.f32 ? "f32" : "bf16",
                  tile_edge(u.f32, u.tile[kGram]), tile_edge(u.f32, u.tile[kSquare]),
                  tile_edge(u.f32, u.tile[kBX]), double(u.lr_scale), u.k1_ntiles);
    s += buf;
  }
  s += "],\"groups\":[";
  bool first = true;
  for (const Group& g : plan.groups) {
    if (g.units.empty()) continue;
    auto real = [](const std::vector<GemmTask>& v) {
      return size_t(std::count_if(v.begin(), v.end(), [](const GemmTask& t) { return t.unit >= 0; }));
    };
    // per phase: real tiles and launched blocks (with the XCD padding) of all
    // tile shapes, and per shape the tile counts
    size_t tiles[3] = {}, blocks[3] = {};
    for (int ph = 0; ph < 3; ++ph)
      for (int tc = 0; tc < kTileCfgs; ++tc) {
        tiles[ph] += real(g.gemm[ph][tc]);
        blocks[ph] += g.gemm[ph][tc].size();
      }
    std::snprintf(buf, sizeof(buf),
                  "%s{\"ns\":\"%s\",\"lane\":%d,\"units\":%zu,\"momentum_tiles\":%zu,\"gram_tiles\":%zu,"
                  "\"square_tiles\":%zu,\"bx_tiles\":%zu,\"gram_blocks\":%zu,\"square_blocks\":%zu,"
                  "\"bx_blocks\":%zu,\"tiles_by_edge\":{",
                  first ? "" : ",", g.f32 ? "f32" : "bf16", g.lane, g.units.size(), g.ew.size(), tiles[0], tiles[1],
                  tiles[2], blocks[0], blocks[1], blocks[2]);
    s += buf;
    bool fe = true;
    for (int tc = 0; tc < kTileCfgs; ++tc) {
      if (g.gemm[kGram][tc].empty() && g.gemm[kBX][tc].empty()) continue;
      std::snprintf(buf, sizeof(buf), "%s\"%d\":[%zu,%zu,%zu]", fe ? "" : ",", tile_edge(g.f32, tc),
                    real(g.gemm[kGram][tc]), real(g.gemm[kSquare][tc]), real(g.gemm[kBX][tc]));
      s += buf;
      fe = false;
    }
    s += "}}";
    first = false;
  }
  s += "],\"preconds\":[";
  for (size_t k = 0; k < plan.slots.size(); ++k) {
    // s_offset / sinv_offset: workspace byte offsets of the slot's S blocks
    // (float32, dp x dp each) and of its S^-1 (three bf16 planes per block)
    std::snprintf(buf, sizeof(buf), "%s{\"d\":%lld,\"nblocks\":%d,\"dp\":%d,\"s_offset\":%zu,\"sinv_offset\":%zu}",
                  k ? "," : "", (long long)plan.slots[k].d, plan.slots[k].nblocks, plan.slots[k].dp,
                  plan.slots[k].off_s, plan.slots[k].off_sinv);
    s += buf;
  }
  std::snprintf(buf, sizeof(buf), "],\"apply_tiles\":%zu,\"adamw_tensors\":%zu,\"adamw_tasks\":%zu,"
                "\"launch_order\":[", plan.apply.size(), plan.adam_tensors.size(), plan.adam_tasks.size());
  s += buf;
  first = true;
  if (!plan.apply.empty()) {
    s += "\"precond_apply\"";
    first = false;
  }
  if (!plan.adam_tasks.empty()) {
    if (!first) s += ",";
    s += "\"adam_tick\",\"adamw\"";
    first = false;
  }
  for (const Group& g : plan.groups) {
    if (g.units.empty()) continue;
    const char* dt = g.f32 ? "f32" : "bf16";
    std::snprintf(buf, sizeof(buf), "%s\"momentum/%s\"", first ? "" : ",", dt);
    s += buf;
    first = false;
    for (int it = 0; it < hp.ns_steps; ++it)
      for (int ph = 0; ph < 3; ++ph)
        for (int tc : kLaunchOrder) {
          if (g.gemm[ph][tc].empty()) continue;
          std::snprintf(buf, sizeof(buf), ",\"%s/%s%s\"", kPhaseNames[ph], dt, tile_tag(g.f32, tc));
          s += buf;
        }
    if (hp.ns_steps == 0) {
      std::snprintf(buf, sizeof(buf), ",\"update/%s\"", dt);
      s += buf;
    }
  }
  std::snprintf(buf, sizeof(buf), "],\"workspace_bytes\":%zu,\"meta_bytes\":%zu}", plan.total, plan.meta_bytes);
  s += buf;
  return s;
}

}  // namespace

extern "C" {

void muon_default_hparams(muon_hparams_t* hp) {
  if (!hp) return;
  hp->lr = 0.02f;
  hp->momentum = 0.95f;
  hp->weight_decay = 0.01f;
  hp->eps = 1e-7f;
  hp->nesterov = 1;
  hp->ns_steps = 5;
  hp->ns_a = 3.4445f;
  hp->ns_b = -4.7750f;
  hp->ns_c = 2.0315f;
  hp->scale_mode = MUON_SCALE_ORIGINAL;
  hp->momentum_form = MUON_MOM_EMA;
  hp->adam_lr = 3e-4f;
  hp->adam_beta1 = 0.9f;
  hp->adam_beta2 = 0.95f;
  hp->adam_eps = 1e-8f;
  hp->adam_weight_decay = 0.01f;
}

muon_status_t muon_workspace_size(const muon_tensor_t* tensors, int32_t n_tensors, const muon_precond_t* preconds,
                                  int32_t n_preconds, const muon_hparams_t* hp, size_t* bytes) {
  if (!bytes) return fail(MUON_ERR_NULL_ARG, "bytes is NULL");
  Plan plan;
  muon_status_t st = build_plan(tensors, n_tensors, preconds, n_preconds, hp, plan);
  if (st != MUON_OK) return st;
  *bytes = plan.total;
  return MUON_OK;
}

muon_status_t muon_plan_describe(const muon_tensor_t* tensors, int32_t n_tensors, const muon_precond_t* preconds,
                                 int32_t n_preconds, const muon_hparams_t* hp, char* buf, size_t len,
                                 size_t* needed) {
  Plan plan;
  muon_status_t st = build_plan(tensors, n_tensors, preconds, n_preconds, hp, plan);
  if (st != MUON_OK) return st;
  const std::string js = plan_json(plan, *hp);
  if (needed) *needed = js.size() + 1;
  if (buf && len) {
    const size_t k = std::min(len - 1, js.size());
    std::memcpy(buf, js.data(), k);
    buf[k] = 0;
  }
  return MUON_OK;
}

}  // extern "C"

namespace {

// Static device scratch of muon_init_static, for callers that cannot
// allocate device memory.  Each GPU the library runs on holds one copy until
// the process ends; host code must use the address hipGetSymbolAddress
// returns for the current device (the array's name is a host-side stand-in).
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices] = {};
uint64_t g_static_gen[kMaxDevices] = {};

// The calling thread's current device and its scratch address (looked up
// once per device, with that device current).
muon_status_t static_scratch(int* dev_out, void** ptr_out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MUON_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MUON_ERR_UNSUPPORTED, "device index beyond the static scratch table");
  std::lock_guard<std::mutex> lk(g_static_mu);
  if (!g_static_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(MUON_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_static_ptr[dev] = ptr;
  }
  *dev_out = dev;
  *ptr_out = g_static_ptr[dev];
  return MUON_OK;
}

// Body shared by muon_init and muon_init_static: `plan` is built and checked
// against the workspace already.  With `with_streams` false the handle
// creates no streams or events: every launch of muon_step then runs on the
// caller's stream.
muon_status_t init_handle(muon_handle_t* out, Plan&& plan, const muon_tensor_t* tensors, int32_t n_tensors,
                          const muon_hparams_t* hp, void* workspace, void* stream, bool with_streams) {
  const uintptr_t wlo = reinterpret_cast<uintptr_t>(workspace), whi = wlo + plan.total;
  for (int32_t i = 0; i < n_tensors; ++i) {
    const muon_tensor_t& t = tensors[i];
    const size_t es = t.dtype == MUON_F32 ? 4 : 2;
    const void* ps[5] = {t.param, t.grad, t.momentum, t.update_out, t.exp_avg_sq};
    const int64_t lds[5] = {t.ld_param, t.ld_grad, t.ld_momentum, t.cols, t.ld_momentum};
    const size_t ess[5] = {es, es, 4, 4, 4};
    for (int k = 0; k < 5; ++k) {
      if (!ps[k]) continue;
      const uintptr_t lo = reinterpret_cast<uintptr_t>(ps[k]);
      const uintptr_t hi = lo + size_t((t.rows - 1) * lds[k] + t.cols) * ess[k];
      if (lo < whi && wlo < hi)
        return fail(MUON_ERR_ALIASING, "tensor " + std::to_string(i) + " overlaps the workspace");
    }
  }
  muon_handle_s* h = new (std::nothrow) muon_handle_s();
  if (!h) return fail(MUON_ERR_UNSUPPORTED, "host allocation failed");
  h->plan = std::move(plan);
  h->hp = *hp;
  h->tensors.assign(tensors, tensors + n_tensors);
  h->ws = static_cast<uint8_t*>(workspace);
  h->meta = build_meta(h->plan, tensors, h->ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemsetAsync(h->ws, 0, h->plan.total, s);
  if (e == hipSuccess) e = hipMemcpyAsync(h->ws, h->meta.data(), h->meta.size(), hipMemcpyHostToDevice, s);
  for (const SlotPlan& sp : h->plan.slots)   // S^-1 = I until the slot's first refresh
    if (e == hipSuccess) e = launch_identity(reinterpret_cast<uint16_t*>(h->ws + sp.off_sinv), sp.dp, sp.nblocks, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);  // the host copy of meta may be reused after init
  if (e != hipSuccess) {
    delete h;
    return fail(MUON_ERR_HIP, std::string("workspace initialisation: ") + hipGetErrorString(e));
  }
  h->last_stream = s;
  int max_lane = 0;
  for (const Group& g : h->plan.groups) max_lane = std::max(max_lane, g.lane);
  const bool aux = with_streams && !h->plan.adam_tasks.empty() && !h->plan.units.empty();
  if (with_streams && (max_lane > 0 || aux)) {
    e = hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming);
    if (aux && e == hipSuccess) e = hipStreamCreateWithFlags(&h->aux_stream, hipStreamNonBlocking);
    if (aux && e == hipSuccess) e = hipEventCreateWithFlags(&h->ev_aux, hipEventDisableTiming);
    if (aux && e == hipSuccess) e = hipEventCreateWithFlags(&h->ev_adam, hipEventDisableTiming);
    for (int l = 0; l < max_lane && e == hipSuccess; ++l) {
      hipStream_t ls = nullptr;
      hipEvent_t ej = nullptr;
      e = hipStreamCreateWithFlags(&ls, hipStreamNonBlocking);   // default priority
      if (e == hipSuccess) h->lane_streams.push_back(ls);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&ej, hipEventDisableTiming);
      if (e == hipSuccess) h->ev_joins.push_back(ej);
    }
    if (e != hipSuccess) {
      if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
      if (h->ev_aux) (void)hipEventDestroy(h->ev_aux);
      if (h->ev_adam) (void)hipEventDestroy(h->ev_adam);
      if (h->aux_stream) (void)hipStreamDestroy(h->aux_stream);
      for (hipEvent_t ej : h->ev_joins) (void)hipEventDestroy(ej);
      for (hipStream_t ls : h->lane_streams) (void)hipStreamDestroy(ls);
      delete h;
      return fail(MUON_ERR_HIP, std::string("lane streams: ") + hipGetErrorString(e));
    }
  }
  if (!h->plan.apply.empty()) h->phase_names.push_back("precond_apply");
  if (!h->plan.adam_tasks.empty()) h->phase_names.push_back("adamw");
  for (const Group& g : h->plan.groups) {
    if (g.units.empty()) continue;
    const std::string dt = std::string(g.f32 ? "/f32" : "/bf16") + (g.lane ? "@" + std::to_string(g.lane + 1) : "");
    h->phase_names.push_back("momentum" + dt);
    for (int it = 0; it < hp->ns_steps; ++it)
      for (int ph = 0; ph < 3; ++ph)
        for (int tc : kLaunchOrder) {
          if (g.gemm[ph][tc].empty()) continue;
          h->phase_names.push_back(std::string(kPhaseNames[ph]) + dt + tile_tag(g.f32, tc) + "#" +
                                   std::to_string(it + 1));
        }
    if (hp->ns_steps == 0) h->phase_names.push_back("update" + dt);
  }
  *out = h;
  return MUON_OK;
}

// A static handle may only launch while its init is the latest one on its
// GPU: a later muon_init_static reuses the same array for another plan.
muon_status_t check_live(muon_handle_t h) {
  if (h->static_device < 0) return MUON_OK;
  std::lock_guard<std::mutex> lk(g_static_mu);
  if (g_static_gen[h->static_device] != h->static_generation)
    return fail(MUON_ERR_BAD_ARG, "a later muon_init_static on this GPU has taken over the static scratch; "
                                  "initialise this handle again");
  return MUON_OK;
}

}  // namespace

extern "C" {

muon_status_t muon_init(muon_handle_t* out, const muon_tensor_t* tensors, int32_t n_tensors,
                        const muon_precond_t* preconds, int32_t n_preconds, const muon_hparams_t* hp,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!out) return fail(MUON_ERR_NULL_ARG, "out is NULL");
  *out = nullptr;
  Plan plan;
  muon_status_t st = build_plan(tensors, n_tensors, preconds, n_preconds, hp, plan);
  if (st != MUON_OK) return st;
  if (!workspace) return fail(MUON_ERR_NULL_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(MUON_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  if (workspace_bytes < plan.total)
    return fail(MUON_ERR_WORKSPACE_TOO_SMALL,
                "workspace has " + std::to_string(workspace_bytes) + " bytes, needs " + std::to_string(plan.total));
  return init_handle(out, std::move(plan), tensors, n_tensors, hp, workspace, stream, true);
}

muon_status_t muon_init_static(muon_handle_t* out, const muon_tensor_t* tensors, int32_t n_tensors,
                               const muon_precond_t* preconds, int32_t n_preconds, const muon_hparams_t* hp,
                               void* stream) {
  if (!out) return fail(MUON_ERR_NULL_ARG, "out is NULL");
  *out = nullptr;
  Plan plan;
  muon_status_t st = build_plan(tensors, n_tensors, preconds, n_preconds, hp, plan, /*single_lane=*/true);
  if (st != MUON_OK) return st;
  if (plan.total > kStaticScratchBytes)
    return fail(MUON_ERR_WORKSPACE_TOO_SMALL,
                "the request needs " + std::to_string(plan.total) + " bytes of workspace; the static scratch holds " +
                    std::to_string(kStaticScratchBytes) + " (use muon_init with a caller workspace)");
  int dev = -1;
  void* ptr = nullptr;
  if ((st = static_scratch(&dev, &ptr)) != MUON_OK) return st;
  uint64_t gen;
  {
    std::lock_guard<std::mutex> lk(g_static_mu);
    gen = ++g_static_gen[dev];
  }
  st = init_handle(out, std::move(plan), tensors, n_tensors, hp, ptr, stream, false);
  if (st != MUON_OK) return st;
  (*out)->static_device = dev;
  (*out)->static_generation = gen;
  return MUON_OK;
}

namespace {

PrecondBlockDev block_dev(muon_handle_t h, const SlotPlan& sp, int32_t block) {
  const size_t bo = size_t(block) * sp.dp * sp.dp;
  PrecondBlockDev b;
  b.s = reinterpret_cast<float*>(h->ws + sp.off_s) + bo;
  b.l = reinterpret_cast<double*>(h->ws + sp.off_l) + bo;
  b.li = reinterpret_cast<double*>(h->ws + sp.off_li) + bo;
  b.sinv = reinterpret_cast<uint16_t*>(h->ws + sp.off_sinv) + bo * kSinvPlanes;
  b.acc = reinterpret_cast<float*>(h->ws + sp.off_acc) + bo;
  b.cnt = reinterpret_cast<double*>(h->ws + sp.off_cnt) + block;
  b.part = h->plan.off_mpart ? reinterpret_cast<float*>(h->ws + h->plan.off_mpart) : nullptr;
  b.d = int(sp.d);
  b.dp = sp.dp;
  return b;
}

muon_status_t check_slot_block(muon_handle_t h, int32_t slot, int32_t block) {
  if (!h) return fail(MUON_ERR_NULL_ARG, "handle is NULL");
  if (check_live(h) != MUON_OK) return MUON_ERR_BAD_ARG;
  if (slot < 0 || size_t(slot) >= h->plan.slots.size()) return fail(MUON_ERR_BAD_ARG, "no such preconditioner slot");
  if (block < 0 || block >= h->plan.slots[size_t(slot)].nblocks) return fail(MUON_ERR_BAD_ARG, "no such block in the slot");
  return MUON_OK;
}

muon_status_t check_acts(const SlotPlan& sp, const void* acts, int64_t n_rows, int64_t ld, int32_t dtype) {
  if (!acts) return fail(MUON_ERR_NULL_ARG, "activations are NULL");
  if (dtype != MUON_F32 && dtype != MUON_BF16) return fail(MUON_ERR_BAD_DTYPE, "activations must be f32 or bf16");
  if (n_rows < 1 || ld < sp.d) return fail(MUON_ERR_BAD_SHAPE, "activations need n_rows >= 1 and ld >= d");
  const size_t es = dtype == MUON_F32 ? 4 : 2;
  if (reinterpret_cast<uintptr_t>(acts) % es) return fail(MUON_ERR_ALIGNMENT, "activations misaligned");
  return MUON_OK;
}

}  // namespace

muon_status_t muon_precond_accumulate(muon_handle_t h, int32_t slot, int32_t block, const void* acts,
                                      int64_t n_rows, int64_t ld, int32_t dtype, float beta, void* stream) {
  muon_status_t st = check_slot_block(h, slot, block);
  if (st != MUON_OK) return st;
  const SlotPlan& sp = h->plan.slots[size_t(slot)];
  if ((st = check_acts(sp, acts, n_rows, ld, dtype)) != MUON_OK) return st;
  if (!(beta >= 0.f && beta <= 1.f)) return fail(MUON_ERR_BAD_ARG, "beta must be in [0, 1]");
  hipStream_t s = static_cast<hipStream_t>(stream);
  Range r("muon.precond_accumulate");
  hipError_t e = launch_precond_accumulate(block_dev(h, sp, block), acts, n_rows, ld, dtype == MUON_F32, beta, s);
  if (e != hipSuccess) return fail(MUON_ERR_HIP, std::string("precond accumulate launch: ") + hipGetErrorString(e));
  h->last_stream = s;
  return MUON_OK;
}

muon_status_t muon_precond_refresh_accumulated(muon_handle_t h, int32_t slot, int32_t block, float damping,
                                               int32_t reset, void* stream) {
  muon_status_t st = check_slot_block(h, slot, block);
  if (st != MUON_OK) return st;
  if (!std::isfinite(damping) || damping < 0.f) return fail(MUON_ERR_BAD_ARG, "damping must be finite and >= 0");
  hipStream_t s = static_cast<hipStream_t>(stream);
  Range r("muon.precond_refresh_accumulated");
  hipError_t e = launch_precond_refresh_accumulated(block_dev(h, h->plan.slots[size_t(slot)], block), damping,
                                                    reset != 0,
                                                    reinterpret_cast<uint32_t*>(h->ws + h->plan.off_flags), s);
  if (e != hipSuccess) return fail(MUON_ERR_HIP, std::string("precond refresh launch: ") + hipGetErrorString(e));
  h->last_stream = s;
  return MUON_OK;
}

muon_status_t muon_precond_refresh(muon_handle_t h, int32_t slot, int32_t block, const void* acts, int64_t n_rows,
                                   int64_t ld, int32_t dtype, float damping, void* stream) {
  muon_status_t st = check_slot_block(h, slot, block);
  if (st != MUON_OK) return st;
  const SlotPlan& sp = h->plan.slots[size_t(slot)];
  if ((st = check_acts(sp, acts, n_rows, ld, dtype)) != MUON_OK) return st;
  if (!std::isfinite(damping) || damping < 0.f) return fail(MUON_ERR_BAD_ARG, "damping must be finite and >= 0");
  hipStream_t s = static_cast<hipStream_t>(stream);
  Range r("muon.precond_refresh");
  hipError_t e = launch_precond_refresh(block_dev(h, sp, block), acts, n_rows, ld, dtype == MUON_F32, damping,
                                        reinterpret_cast<uint32_t*>(h->ws + h->plan.off_flags), s);
  if (e != hipSuccess) return fail(MUON_ERR_HIP, std::string("precond refresh launch: ") + hipGetErrorString(e));
  h->last_stream = s;
  return MUON_OK;
}

muon_status_t muon_step(muon_handle_t h, float lr, void* stream) {
  if (!h) return fail(MUON_ERR_NULL_ARG, "handle is NULL");
  if (!std::isfinite(lr)) return fail(MUON_ERR_BAD_ARG, "lr is not finite");
  if (check_live(h) != MUON_OK) return MUON_ERR_BAD_ARG;
  return enqueue_step(h, lr < 0.f ? h->hp.lr : lr, static_cast<hipStream_t>(stream), nullptr);
}

muon_status_t muon_step_timed(muon_handle_t h, float lr, void* stream, float* phase_ms, int32_t max_phases,
                              int32_t* n_phases) {
  if (!h) return fail(MUON_ERR_NULL_ARG, "handle is NULL");
  if (!std::isfinite(lr)) return fail(MUON_ERR_BAD_ARG, "lr is not finite");
  if (check_live(h) != MUON_OK) return MUON_ERR_BAD_ARG;
  const size_t np = h->phase_names.size();
  if (h->events.size() < np + 1) {
    while (h->events.size() < np + 1) {
      hipEvent_t ev;
      if (hipEventCreate(&ev) != hipSuccess) return fail(MUON_ERR_HIP, "hipEventCreate failed");
      h->events.push_back(ev);
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  muon_status_t st = enqueue_step(h, lr < 0.f ? h->hp.lr : lr, s, &h->events);
  if (st != MUON_OK) return st;
  if (hipEventSynchronize(h->events[np]) != hipSuccess) return fail(MUON_ERR_HIP, "hipEventSynchronize failed");
  const size_t k = std::min<size_t>(np, max_phases > 0 ? size_t(max_phases) : 0);
  for (size_t i = 0; i < k; ++i) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, h->events[i], h->events[i + 1]) != hipSuccess)
      return fail(MUON_ERR_HIP, "hipEventElapsedTime failed");
    if (phase_ms) phase_ms[i] = ms;
  }
  if (n_phases) *n_phases = int32_t(np);
  return MUON_OK;
}

const char* muon_phase_name(muon_handle_t h, int32_t phase) {
  if (!h || phase < 0 || size_t(phase) >= h->phase_names.size()) return "";
  return h->phase_names[size_t(phase)].c_str();
}

muon_status_t muon_set_adam_step(muon_handle_t h, int64_t steps_taken, void* stream) {
  if (!h) return fail(MUON_ERR_NULL_ARG, "handle is NULL");
  if (check_live(h) != MUON_OK) return MUON_ERR_BAD_ARG;
  if (steps_taken < 0 || steps_taken > int64_t(UINT32_MAX) - 1) return fail(MUON_ERR_BAD_ARG, "step count out of range");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_adam_set(reinterpret_cast<AdamState*>(h->ws + h->plan.off_adam_state),
                                 uint32_t(steps_taken), s);
  if (e != hipSuccess) return fail(MUON_ERR_HIP, std::string("adam step set: ") + hipGetErrorString(e));
  h->last_stream = s;
  return MUON_OK;
}

muon_status_t muon_get_adam_step(muon_handle_t h, void* stream, int64_t* steps_taken) {
  if (!h || !steps_taken) return fail(MUON_ERR_NULL_ARG, "handle or output is NULL");
  if (check_live(h) != MUON_OK) return MUON_ERR_BAD_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  AdamState st;
  hipError_t e = hipMemcpyAsync(&st, h->ws + h->plan.off_adam_state, sizeof(st), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(MUON_ERR_HIP, std::string("adam step read: ") + hipGetErrorString(e));
  *steps_taken = int64_t(st.t);
  return MUON_OK;
}

muon_status_t muon_get_flags(muon_handle_t h, void* stream, int32_t reset, uint32_t* flags) {
  if (!h || !flags) return fail(MUON_ERR_NULL_ARG, "handle or flags is NULL");
  if (check_live(h) != MUON_OK) return MUON_ERR_BAD_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemcpy(&v, h->ws + h->plan.off_flags, sizeof(v), hipMemcpyDeviceToHost);
  if (e == hipSuccess && reset) {
    e = hipMemsetAsync(h->ws + h->plan.off_flags, 0, sizeof(uint32_t), s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
  }
  if (e != hipSuccess) return fail(MUON_ERR_HIP, std::string("flags: ") + hipGetErrorString(e));
  *flags = v;
  return MUON_OK;
}

muon_status_t muon_destroy(muon_handle_t h) {
  if (!h) return MUON_OK;
  hipError_t e = hipStreamSynchronize(h->last_stream);
  for (hipStream_t ls : h->lane_streams) {
    const hipError_t e2 = hipStreamSynchronize(ls);
    if (e == hipSuccess) e = e2;
    (void)hipStreamDestroy(ls);
  }
  if (h->aux_stream) {
    const hipError_t e2 = hipStreamSynchronize(h->aux_stream);
    if (e == hipSuccess) e = e2;
    (void)hipStreamDestroy(h->aux_stream);
  }
  for (hipEvent_t ej : h->ev_joins) (void)hipEventDestroy(ej);
  if (h->ev_aux) (void)hipEventDestroy(h->ev_aux);
  if (h->ev_adam) (void)hipEventDestroy(h->ev_adam);
  if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
  for (hipEvent_t ev : h->events) (void)hipEventDestroy(ev);
  delete h;
  if (e != hipSuccess) return fail(MUON_ERR_HIP, std::string("destroy: ") + hipGetErrorString(e));
  return MUON_OK;
}

const char* muon_status_str(muon_status_t s) {
  switch (s) {
    case MUON_OK: return "MUON_OK";
    case MUON_ERR_NULL_ARG: return "MUON_ERR_NULL_ARG";
    case MUON_ERR_BAD_SHAPE: return "MUON_ERR_BAD_SHAPE";
    case MUON_ERR_BAD_DTYPE: return "MUON_ERR_BAD_DTYPE";
    case MUON_ERR_ALIGNMENT: return "MUON_ERR_ALIGNMENT";
    case MUON_ERR_ALIASING: return "MUON_ERR_ALIASING";
    case MUON_ERR_WORKSPACE_TOO_SMALL: return "MUON_ERR_WORKSPACE_TOO_SMALL";
    case MUON_ERR_UNSUPPORTED: return "MUON_ERR_UNSUPPORTED";
    case MUON_ERR_HIP: return "MUON_ERR_HIP";
    case MUON_ERR_BAD_ARG: return "MUON_ERR_BAD_ARG";
  }
  return "MUON_ERR_UNKNOWN";
}

const char* muon_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
