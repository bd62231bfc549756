// The launch planner of the skinny GEMM (declared in qpn_plan.hpp): plain
// host C++, shared by the C ABI and the kernel launcher.
#include "qpn_plan.hpp"

namespace qpn {
namespace {

// Launch shapes. For the matrices of a ~27B dense decoder (hidden 5120) the
// launch comes from a table measured on MI355X: a sweep of activation stage x
// workgroup size x K slices x K split x stream depth, best graph-replayed time
// per launch at M = 1, 2, 4, 8, 16 (and, for gate_up, groups kept whole x
// split of the rest). Other shapes use a rule distilled from the same sweep:
//  * a workgroup holds TN n-tiles that share one staged copy of x (the
//    staging reads 2*M bytes of x per K element against 9*TN bytes of NVFP4
//    weights), TN = 2 up to M = 4 and 4 above;
//  * the rest of an 8-wavefront workgroup splits each n-tile's K range into
//    K slices, reduced through LDS, keeping >= kMinSliceUnits units a slice;
//  * K is split over workgroups only as far as the activation stage must be
//    cut to fit LDS (that reduction costs memory round trips at the tail);
//  * a stream depth of 3 units;
//  * the ring activation stage from kRingMinM rows on (at 8 and 16 rows it
//    wins on every matrix but one, at 4 it ties with the full stage);
//  * no whole groups (all groups split alike): a balanced grid needs the
//    shape's group count, and is only tabled where it was measured.
// An uneven-group row (waves == kUnevenWaves) serves only calls that leave
// the workgroup size, K slices, K split, whole groups and depth automatic
// and ask for the fp16 or fp32 epilogue on the MFMA path; the others take
// the next row of the shape.
struct TunedLaunch {
  int fmt;
  int64_t n, k;
  int m_max;  // entry applies to m <= m_max (entries of a shape in increasing m_max)
  int waves, k_slices, split, depth;
  int x_stage = kStageFull;
  int whole_groups = 0;
};

constexpr TunedLaunch kTuned[] = {
    // NVFP4 gate_up 34816 x 5120: 2176 n-tiles. 256 whole groups of 8 tiles
    // fill the 256 CUs evenly; the last 16 groups split K, a short tail of
    // small workgroups that share CUs with whole groups. Up to 2 rows the
    // tail is split four ways; from 3 rows five (4 units a range, so the
    // busiest CU streams 192 tile-units instead of 200): M = 6 18.61
    // against 19.23 us, M = 8 18.87 / 18.98 / 19.03 against 19.34 / 19.57 /
    // 19.66, M = 4 18.02 / 18.23 against 18.21 / 18.50 (three machines, ten
    // or twelve alternated rounds); at 1 row no better (17.64 / 17.77 /
    // 18.07 against 17.90 / 17.95 / 17.96), with SwiGLU worse (18.67 / 19.02
    // against 18.53 / 18.71). At 2 rows this grid beats groups of 4 tiles
    // with a full stage (18.05 against 18.51 us). From 9 rows on the fp16
    // and fp32 epilogues take the uneven grid: 256 workgroups of 9
    // wavefronts, 128 with 9 n-tiles and 128 with 8, no K split (M = 12
    // 19.80 against 20.60 for the five-way tail, M = 16 20.53 against 22.03;
    // against the four-way tail M = 9 18.67 / 19.74, M = 16 19.67 / 22.20).
    // At 8 rows it ties with the five-way tail (18.99 / 18.64 against 18.98
    // / 18.87), below that it is slower (M = 1 18.52 against 17.95).
    {kFmtNvfp4, 34816, 5120, 2, 8, 1, 4, 2, kStageRing, 256},
    {kFmtNvfp4, 34816, 5120, 8, 8, 1, 5, 2, kStageRing, 256},
    {kFmtNvfp4, 34816, 5120, 16, kUnevenWaves, 1, 1, 2, kStageRing, 256},
    {kFmtNvfp4, 34816, 5120, 16, 8, 1, 5, 2, kStageRing, 256},
    // NVFP4 down 5120 x 17408 (at M = 3 and 4 the ring at depth 3 measured 12.43 / 12.48 us
    // against 12.45 / 12.68 for the full stage at depth 2, eight alternated rounds)
    {kFmtNvfp4, 5120, 17408, 2, 8, 4, 1, 3}, {kFmtNvfp4, 5120, 17408, 4, 8, 2, 3, 3, kStageRing},
    {kFmtNvfp4, 5120, 17408, 8, 8, 2, 3, 2, kStageRing}, {kFmtNvfp4, 5120, 17408, 16, 8, 2, 3, 2, kStageRing},
    // NVFP4 qkv 7168 x 5120 and o_proj 5120 x 5120
    {kFmtNvfp4, 7168, 5120, 4, 8, 4, 1, 3}, {kFmtNvfp4, 7168, 5120, 8, 8, 4, 1, 2, kStageRing},
    {kFmtNvfp4, 7168, 5120, 16, 8, 2, 2, 2, kStageRing},
    {kFmtNvfp4, 5120, 5120, 4, 8, 4, 1, 3}, {kFmtNvfp4, 5120, 5120, 8, 8, 4, 1, 2, kStageRing},
    {kFmtNvfp4, 5120, 5120, 16, 8, 2, 3, 2},
    // NVFP4 lm_head 151936 x 5120
    {kFmtNvfp4, 151936, 5120, 1, 8, 4, 1, 3}, {kFmtNvfp4, 151936, 5120, 2, 4, 2, 1, 2, kStageRing},
    {kFmtNvfp4, 151936, 5120, 4, 8, 2, 1, 2}, {kFmtNvfp4, 151936, 5120, 16, 8, 1, 1, 2, kStageRing},
    // Per-GPU shapes of 4-way tensor parallelism (NVFP4): qkv 1792 x 5120,
    // o_proj 5120 x 1280, gate_up 8704 x 5120, down 5120 x 4352
    {kFmtNvfp4, 1792, 5120, 1, 4, 4, 1, 3}, {kFmtNvfp4, 1792, 5120, 8, 8, 2, 6, 2},
    {kFmtNvfp4, 5120, 1280, 8, 8, 4, 1, 2},
    {kFmtNvfp4, 8704, 5120, 1, 8, 2, 1, 3}, {kFmtNvfp4, 8704, 5120, 8, 4, 2, 6, 2, kStageRing, 256},
    {kFmtNvfp4, 5120, 4352, 1, 8, 4, 1, 3}, {kFmtNvfp4, 5120, 4352, 8, 8, 4, 1, 3},
    // FP8 qkv 7168 x 5120
    // (M = 2 takes the ring of M = 4: 8.60 against 8.70 us for the full stage, alternated rounds)
    {kFmtFp8, 7168, 5120, 1, 4, 2, 1, 2}, {kFmtFp8, 7168, 5120, 4, 4, 2, 1, 3, kStageRing},
    {kFmtFp8, 7168, 5120, 8, 4, 2, 1, 2, kStageRing}, {kFmtFp8, 7168, 5120, 16, 8, 2, 2, 2, kStageRing},
    // FP8 o_proj 5120 x 5120
    // (M = 1 at depth 2: 7.18 against 7.27 us at depth 3; M = 2 takes the ring of M = 3..8: 7.43
    // against 7.65 for the full stage at depth 4; alternated rounds)
    {kFmtFp8, 5120, 5120, 1, 4, 2, 1, 2},
    {kFmtFp8, 5120, 5120, 8, 4, 2, 1, 3, kStageRing}, {kFmtFp8, 5120, 5120, 16, 8, 2, 3, 2, kStageRing},
    // FP8 down 5120 x 17408
    {kFmtFp8, 5120, 17408, 1, 8, 4, 1, 2}, {kFmtFp8, 5120, 17408, 4, 4, 1, 3, 3, kStageRing},
    // (from 5 rows on depth 2: 17.50 / 19.13 us at M = 8 / 16 against 17.73 / 19.61 at depth 3)
    {kFmtFp8, 5120, 17408, 16, 8, 2, 3, 2, kStageRing},
};

// Whether an uneven-group row may serve this call (see TunedLaunch).
bool uneven_row_ok(const LaunchOverride& o) {
  return !o.waves && !o.k_slices && !o.split && !o.whole_groups && !o.depth &&
         (o.epilogue == kEpiNone || o.epilogue == kEpiF32) && !o.valu_dot && o.block_cols != 1;
}

const TunedLaunch* find_tuned(int fmt, int64_t n, int64_t k, int m, const LaunchOverride& o) {
  for (const TunedLaunch& t : kTuned)
    if (t.fmt == fmt && t.n == n && t.k == k && m <= t.m_max && (t.waves != kUnevenWaves || uneven_row_ok(o)))
      return &t;
  return nullptr;
}

}  // namespace

int ring_pieces(int waves, int k_slices, int m) { return (k_slices * m * 32 + waves * 64 - 1) / (waves * 64); }

bool shape_ok(int64_t n, int64_t k) {
  return n >= 0 && k >= 0 && k % 16 == 0 && n <= (int64_t(1) << 31) - 16 && k <= (int64_t(1) << 30);
}

size_t packed_bytes(int fmt, int64_t n, int64_t k) {
  if (!shape_ok(n, k)) return 0;
  const int64_t units = ceil_div(n, kTileN) * ceil_div(k, kUnitK);
  if (fmt == kFmtNvfp4) return static_cast<size_t>(units) * kNvUnitBytes;
  if (fmt == kFmtFp8) return static_cast<size_t>(units) * kF8UnitBytes;
  return 0;
}

bool plan_gemm(int fmt, int64_t n, int64_t k, int m, const LaunchOverride& o, GemmPlan* p) {
  if (fmt != kFmtNvfp4 && fmt != kFmtFp8) return false;
  if (m < 1 || m > kMaxM || n < 1 || k < 0) return false;
  if (!shape_ok(n, k)) return false;
  // the override's own ranges (0 is automatic for every field)
  if (o.split < 0 || o.waves < 0 || o.depth < 0 || o.k_slices < 0 || o.whole_groups < 0) return false;
  if (o.x_stage != 0 && o.x_stage != kStageFull && o.x_stage != kStageRing) return false;
  if (o.epilogue < kEpiNone || o.epilogue > kEpiF32) return false;
  if (o.valu_dot != 0 && o.valu_dot != 1) return false;
  if (o.block_cols < 0 || o.block_cols > 2) return false;
  const int64_t NT = ceil_div(n, kTileN);
  const int64_t KU = ceil_div(k, kUnitK);
  const int64_t unit_bytes = fmt == kFmtNvfp4 ? kNvUnitBytes : kF8UnitBytes;
  // unit offsets inside one wavefront's stream are 32-bit
  if (NT * KU * unit_bytes >= (int64_t(1) << 31)) return false;
  const int64_t max_ups = (static_cast<int64_t>(kLdsBudget) / (2 * m) - kRowPad) / kUnitK;
  if (max_ups < 1) return false;

  // A tuned launch for this shape fills in what the caller left automatic
  // (the argmax epilogue takes the plain GEMM's shape: on the 151936-row
  // head it measured the same as few, wide groups, 70.2 against 70.4 us at
  // M = 1 and 70.1 against 70.2 at M = 8).
  LaunchOverride w = o;
  int tuned_tn = 0;  // n-tiles per workgroup behind a tabled whole_groups (0: none tabled)
  const TunedLaunch* t = find_tuned(fmt, n, k, m, o);
  // An explicit request for the uneven grid takes nothing from a row of
  // another grid (its K split and slices do not apply there).
  if (t && o.waves == kUnevenWaves && t->waves != kUnevenWaves) t = nullptr;
  if (t) {
    if (!w.split) w.split = t->split;
    if (!w.waves) w.waves = t->waves;
    if (!w.k_slices) w.k_slices = t->k_slices;
    if (!w.depth) w.depth = t->depth;
    if (!w.x_stage) w.x_stage = t->x_stage;
    if (!w.whole_groups && !o.split && t->whole_groups) {
      w.whole_groups = t->whole_groups;
      tuned_tn = t->waves / t->k_slices;
    }
  }

  // The uneven-group grid: NVFP4, the fp16 or fp32 epilogue on the MFMA
  // path, one K slice, no K split, at most kUnevenWaves n-tiles a workgroup.
  const bool uneven = w.waves == kUnevenWaves;
  if (uneven) {
    if (fmt != kFmtNvfp4 || (o.epilogue != kEpiNone && o.epilogue != kEpiF32) || o.valu_dot || o.block_cols == 1)
      return false;
    if (w.k_slices > 1 || w.split > 1 || w.whole_groups <= 0 || w.whole_groups > NT) return false;
    if (ceil_div(NT, w.whole_groups) > kUnevenWaves) return false;
    if (w.depth && w.depth != 2 && w.depth != 3) return false;
  }

  // K ranges over workgroups: as few as a full activation stage allows.
  int64_t split = uneven ? 1 : w.split > 0 ? w.split : (KU ? ceil_div(KU, max_ups) : 1);
  if (split > KU) split = KU ? KU : 1;
  if (split < 1) split = 1;
  const int64_t ups = KU ? ceil_div(KU, split) : 0;
  if (KU) split = ceil_div(KU, ups);

  // n-tiles per workgroup first (from M), then as many K slices per n-tile
  // as the workgroup has room for and the K range supports.
  const int tn_target = m > 4 ? 4 : 2;
  int ks = uneven ? 1 : w.k_slices;
  if (!ks) {
    const int ks_room = 8 / tn_target;
    ks = 1;
    while (ks < ks_room && ceil_div(ups, 2 * ks) >= kMinSliceUnits) ks *= 2;
  }
  int waves = w.waves;
  if (!waves) {
    waves = tn_target * ks < 4 ? 4 : tn_target * ks > 8 ? 8 : tn_target * ks;
    if (waves < ks) waves = ks;
  }
  // The SwiGLU epilogue pairs gate and up n-tiles inside a workgroup, so it
  // needs an even number of n-tiles per workgroup (and N/2 on a tile
  // boundary): an automatic shape gives up K slices (or adds wavefronts) to
  // get there.
  if (o.epilogue == kEpiSwiglu) {
    if (n % (2 * kTileN)) return false;
    if (waves && ks && (waves / ks) % 2) {
      if (o.k_slices && o.waves) return false;
      if (!o.k_slices && ks > 1) ks /= 2;
      else if (!o.waves && waves < 8) waves *= 2;
      else return false;
    }
  }
  if (waves != 4 && waves != 8 && !uneven) return false;
  if (ks != 1 && ks != 2 && ks != 4 && ks != 8) return false;
  if (ks > waves) return false;
  if (o.epilogue == kEpiSwiglu && (waves / ks) % 2) return false;
  const int depth = w.depth ? w.depth : uneven ? 2 : 3;
  if (depth != 2 && depth != 3 && depth != 4 && depth != 6 && depth != 8) return false;
  // The packed-dot path: the plain epilogue, a full stage, depths 2..4, and
  // at most 4 rows (its cost grows with M; the MFMA's does not).
  if (o.valu_dot && (o.epilogue != kEpiNone || depth > 4 || m > 4 || o.x_stage == kStageRing)) return false;

  // Groups kept whole (split > 1 only): a whole group's workgroup covers
  // all KU units, so a full stage must hold them. A tabled count was chosen
  // for the table's n-tiles per workgroup; where the caller changed those,
  // it is scaled to keep the same n-tiles whole (the balanced grid).
  const int64_t groups = ceil_div(NT, waves / ks);
  if (tuned_tn && waves / ks != tuned_tn)
    w.whole_groups = static_cast<int>(static_cast<int64_t>(w.whole_groups) * tuned_tn / (waves / ks));
  const int64_t whole = split > 1 ? (w.whole_groups < groups ? w.whole_groups : groups) : groups;
  if (w.whole_groups < 0) return false;

  // Activation stage: the caller's choice is binding; a tuned or automatic
  // one falls back to the other stage when it is not possible. The ring
  // stage wins from kRingMinM rows on (its per-unit barriers cost more than
  // a small full stage saves).
  const bool full_ok = (split > 1 && whole > 0 ? KU : ups) <= max_ups;
  const bool ring_ok = depth <= 4 && ring_pieces(waves, ks, m) <= kRingMaxPieces &&
                       2 * static_cast<int64_t>(m) * k < (int64_t(1) << 31);
  int stage = o.valu_dot ? kStageFull : w.x_stage ? w.x_stage : (m >= kRingMinM ? kStageRing : kStageFull);
  if (stage != kStageFull && stage != kStageRing) return false;
  if (!o.x_stage && !o.valu_dot) {
    if (stage == kStageRing && !ring_ok) stage = kStageFull;
    if (stage == kStageFull && !full_ok) stage = kStageRing;
  }
  if (stage == kStageFull ? !full_ok : !ring_ok) return false;
  // Block columns: one activation row of NVFP4 weights, full stage, the MFMA
  // path; 1 demands it, 0 and 2 leave it off. Its decode skips the
  // per-weight scale multiply (45 instead of 66 VALU per unit), yet measured
  // 2-5% slower as a standalone launch (11.2 against 11.0 us on down at one
  // row, 18.2 against 17.9 on gate_up): the launch is bound by memory latency
  // and balance, not by the VALU, and the path adds four LDS permutes a unit.
  if (o.block_cols < 0 || o.block_cols > 2) return false;
  const int64_t staged = (split > 1 && whole > 0 ? KU : ups) * kUnitK + kRowPad;  // halves per staged row
  const bool bc_ok = m == 1 && fmt == kFmtNvfp4 && stage == kStageFull && !o.valu_dot &&
                     (staged + depth * kUnitK + 64) * static_cast<int64_t>(kHalfBytes) <=
                         static_cast<int64_t>(kLdsBudget);
  if (o.block_cols == 1 && !bc_ok) return false;
  p->block_cols = bc_ok && o.block_cols == 1 ? 1 : 0;

  p->split = static_cast<int>(split);
  p->whole_groups = uneven ? w.whole_groups : split > 1 ? static_cast<int>(whole) : 0;
  p->waves = waves;
  p->depth = depth;
  p->k_slices = ks;
  p->dot_rows = o.valu_dot ? (m <= 1 ? 1 : m <= 2 ? 2 : 4) : 0;
  p->units_per_split = static_cast<int>(ups);
  p->lds_stride = static_cast<int>((split > 1 && whole > 0 ? KU : ups) * kUnitK + kRowPad);
  p->x_stage = stage;
  p->lds_bytes = stage == kStageFull ? static_cast<size_t>(m) * p->lds_stride * kHalfBytes
                                     : static_cast<size_t>(ks) * kRingSlots * m * kRingRow * kHalfBytes;
  // ... plus the zero region the block-column B operand reads (DEPTH units and a chunk of slack)
  if (p->block_cols) p->lds_bytes += static_cast<size_t>(depth * kUnitK + 64) * kHalfBytes;
  // K slices reduce through the same LDS: one 16x16 fp32 tile per wavefront.
  const size_t red_bytes = ks > 1 ? static_cast<size_t>(waves) * 64 * kTileLaneBytes : 0;
  if (p->lds_bytes < red_bytes) p->lds_bytes = red_bytes;
  // ... and (SwiGLU) the up tiles handed to the gate wavefronts.
  const size_t xch_bytes = o.epilogue == kEpiSwiglu ? static_cast<size_t>(waves / ks / 2) * 64 * kTileLaneBytes : 0;
  if (p->lds_bytes < xch_bytes) p->lds_bytes = xch_bytes;
  if (o.epilogue < kEpiNone || o.epilogue > kEpiF32) return false;
  p->epilogue = o.epilogue;
  const size_t counters = (static_cast<size_t>(NT) * sizeof(int) + 255) & ~size_t(255);
  p->control_offset = counters;
  p->partials_offset = counters + kControlBytes;
  p->workspace_bytes = 0;
  if (split > 1)
    p->workspace_bytes =
        p->partials_offset + ((static_cast<size_t>(split) * m * n * sizeof(float) + 255) & ~size_t(255));
  if (o.epilogue == kEpiArgmax && p->workspace_bytes < p->partials_offset)
    p->workspace_bytes = p->partials_offset;  // the key slots of the control block
  return true;
}

int64_t gemm_grid(const GemmPlan& p, int64_t n) {
  if (p.waves == kUnevenWaves) return p.whole_groups;
  const int64_t groups = ceil_div(ceil_div(n, kTileN), p.waves / p.k_slices);
  const int64_t whole = p.split > 1 ? p.whole_groups : groups;
  return whole + (groups - whole) * (p.split > 1 ? p.split : 0);
}

bool plan_mlp(int fmt_up, int64_t n_up, int64_t k_up, int fmt_dn, int64_t n_dn, int64_t k_dn, int m,
              const MlpOverride& o, MlpPlan* p) {
  if (o.fused < 0 || o.fused > 2 || o.down_depth < 0 || o.stream_after < -1) return false;
  if (n_up % (2 * kTileN) || k_dn != n_up / 2) return false;
  LaunchOverride up_o, dn_o;
  up_o.epilogue = kEpiSwiglu;
  if (!plan_gemm(fmt_up, n_up, k_up, m, up_o, &p->up)) return false;
  if (!plan_gemm(fmt_dn, n_dn, k_dn, m, dn_o, &p->down)) return false;
  // The one-launch form: one workgroup size for both halves, and a
  // consumer that stages all of its K range before it streams (the h
  // staging waits for the producers; a ring stage would wait once per
  // unit). The kernels exist for NVFP4 with producer depths 2 and 3 and
  // consumer depths 2, 3, 4, 6 and 8.
  up_o.waves = kMlpWaves;
  dn_o.waves = kMlpWaves;
  dn_o.x_stage = kStageFull;
  dn_o.depth = o.down_depth;
  // Only on request: on the 27B shapes the one launch measures level with
  // the two (M = 1: 30.29 against 29.94 us, M = 2: 30.66 against 30.97; the
  // last producer's signal takes 2.5-3 us to reach the consumers, about what
  // the second launch costs).
  p->fusable = fmt_up == kFmtNvfp4 && fmt_dn == kFmtNvfp4 && o.fused == 1 &&
               plan_gemm(fmt_up, n_up, k_up, m, up_o, &p->up_fused) &&
               plan_gemm(fmt_dn, n_dn, k_dn, m, dn_o, &p->down_fused) && p->up_fused.dot_rows == 0 &&
               (p->up_fused.depth == 2 || p->up_fused.depth == 3) &&
               (p->up_fused.x_stage == kStageFull || ring_pieces(kMlpWaves, p->up_fused.k_slices, m) == 1) &&
               p->down_fused.dot_rows == 0 && p->down_fused.block_cols == 0 &&
               (p->down_fused.depth == 2 || p->down_fused.depth == 3 || p->down_fused.depth == 4 ||
                p->down_fused.depth == 6 || p->down_fused.depth == 8);
  if (o.fused == 1 && !p->fusable) return false;
  p->fused_requested = o.fused == 1;
  if (!p->fusable) {
    p->up_fused = p->up;
    p->down_fused = p->down;
  }
  p->producers = static_cast<int>(gemm_grid(p->up_fused, n_up));
  p->consumers = static_cast<int>(gemm_grid(p->down_fused, n_dn));
  // Consumers start streaming once most producers are done: the producers'
  // last workgroups leave CUs idle that the consumers' first units fill.
  p->stream_after = o.stream_after == -1 ? 0 : o.stream_after > 0 ? o.stream_after : p->producers / 2;
  if (p->stream_after > p->producers) p->stream_after = p->producers;
  p->lds_bytes = p->up_fused.lds_bytes > p->down_fused.lds_bytes ? p->up_fused.lds_bytes : p->down_fused.lds_bytes;
  const auto round256 = [](size_t b) { return (b + 255) & ~size_t(255); };
  const size_t up_ws = round256(p->up.workspace_bytes > p->up_fused.workspace_bytes ? p->up.workspace_bytes
                                                                                      : p->up_fused.workspace_bytes);
  const size_t dn_ws = round256(p->down.workspace_bytes > p->down_fused.workspace_bytes
                                    ? p->down.workspace_bytes
                                    : p->down_fused.workspace_bytes);
  p->down_ws_offset = up_ws;
  p->flags_offset = up_ws + dn_ws;
  p->counter_offset = p->flags_offset + static_cast<size_t>(p->consumers) * kMlpFlagLineBytes;
  p->workspace_bytes = p->counter_offset + kMlpControlBytes;
  return true;
}

}  // namespace qpn
