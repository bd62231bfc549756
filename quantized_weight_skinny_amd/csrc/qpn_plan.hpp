// Launch planning of the skinny GEMM: the constants the planner shares with
// the kernels, the launch override and plan, and the planner itself. Plain
// C++ (no HIP types), so that the planner also builds with the host compiler
// alone (the sanitizer test builds it with g++ -fsanitize=address,undefined).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace qpn {

// Packed layout: 16-row n-tiles, 256-element K units (see qpn_device.hpp).
constexpr int kTileN = 16;
constexpr int kUnitK = 256;
constexpr int kNvUnitBytes = 2304;
constexpr int kF8UnitBytes = 4096;
constexpr int kMaxM = 16;

constexpr int kFmtNvfp4 = 1;
constexpr int kFmtFp8 = 2;

constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int kStageFull = 1;  // the workgroup's whole K range of x staged before the stream
constexpr int kStageRing = 2;  // a three-unit ring per K slice, refilled alongside the stream

// Activation stage per workgroup: two workgroups of up to this size (plus a
// few bytes of static LDS) fit the 160 KiB of LDS in a CU.
constexpr size_t kLdsBudget = 79 * 1024;
constexpr int kMinSliceUnits = 4;
constexpr int kRingMinM = 5;
constexpr int kEpiNone = 0, kEpiSwiglu = 1, kEpiArgmax = 2, kEpiF32 = 3;  // GemmPlan::epilogue
// DOT template value of the block-column path (one activation row, NVFP4, full stage).
constexpr int kDotBlockCols = -1;
// The argmax epilogue's key slots in the workspace's control block: group g
// folds its best key of row m into slot (g % kArgmaxSubs, m) with a
// device-scope atomic max, so thousands of groups spread over 64 addresses
// per row.
constexpr int kArgmaxSubs = 64;
constexpr size_t kControlBytes = static_cast<size_t>(kArgmaxSubs) * kMaxM * sizeof(unsigned long long);
constexpr int kFixupBatch = 8;  // split-K partials loaded together by the last workgroup

// Workgroup size of the uneven-group grid: `whole_groups` workgroups share
// the n-tiles, one K slice each and no K split; the first NT % whole_groups
// of them take one n-tile more than the others, at most this many.
constexpr int kUnevenWaves = 9;

constexpr int kRowPad = 8;                  // fp16 pad per staged row (bank spread)
constexpr int kRingSlots = 3;               // units per K slice in the ring stage
constexpr int kRingRow = kUnitK + kRowPad;  // halves per row of a ring slot
constexpr int kRingMaxPieces = 2;           // x pieces per thread and unit in the ring stage
constexpr size_t kHalfBytes = 2;            // one fp16 activation
constexpr size_t kTileLaneBytes = 16;       // one lane's share of a 16x16 fp32 tile (4 floats)

// Launch plan of one GEMM call: the K range is cut into `split` pieces of
// `units_per_split` 256-element units (except for the first `whole_groups`
// groups of n-tiles, which take all of K in one workgroup); each workgroup of
// `waves` wavefronts handles `waves / k_slices` n-tiles of one piece. split > 1
// writes fp32 partial sums to the workspace; the last workgroup of a group to
// finish adds them in piece order.
struct LaunchOverride {
  int split = 0, waves = 0, depth = 0, k_slices = 0;  // 0 = automatic
  int epilogue = 0;  // 0: y[M, N]; 1: SwiGLU (h[M, N/2]); 2: greedy argmax per row; 3: fp32 y
  int x_stage = 0;   // 0 automatic; kStageFull; kStageRing
  int whole_groups = 0;  // with split > 1: leading n-tile groups kept whole (not split);
                         // with waves == kUnevenWaves: the workgroups of the uneven grid
  int valu_dot = 0;      // 1: the VALU packed-dot path instead of the MFMA
  int block_cols = 0;    // one activation row, NVFP4: 1 on, 0 and 2 off
};

struct GemmPlan {
  int split;
  int waves;
  int k_slices;    // wavefronts of a workgroup that split one n-tile's K range
  int dot_rows;    // 0: MFMA; 1, 2 or 4: the VALU packed-dot path for up to that many rows
  int block_cols;  // 1: MFMA output columns carry K-blocks (one activation row, NVFP4, full stage)
  int depth;       // units of the weight stream each wavefront keeps in flight
  int epilogue;    // 0 y[M, N]; 1 h[M, N/2] = silu(y[:, :N/2]) * y[:, N/2:]; 2 argmax of each row; 3 fp32 y
  int x_stage;     // kStageFull or kStageRing
  int whole_groups;  // split > 1: the first whole_groups groups of n-tiles take all of K;
                     // waves == kUnevenWaves: the workgroups of the uneven grid
  int units_per_split;
  int lds_stride;  // halves per staged activation row (full stage)
  size_t lds_bytes;
  // Workspace: one split-K arrival counter per n-tile (padded to 256 bytes),
  // a control block (the argmax epilogue's 64 x 16 key slots, 8 KiB), then
  // fp32 partials [split][m][n] from partials_offset (split > 1). 0 bytes
  // when neither split-K nor the argmax epilogue needs it.
  size_t control_offset;
  size_t partials_offset;
  size_t workspace_bytes;
};

// The MLP of a decoder layer, h = SwiGLU(x W_gu^T), y = h W_dn^T, as one
// launch: the gate_up workgroups (producers) write h with device-scope
// stores and count themselves in; the down workgroups (consumers), placed
// after them in the grid, issue their first weight units once
// `stream_after` producers have finished and stage h once all have. Every
// workgroup of the grid must be resident at once (the launcher checks the
// occupancy), so a consumer's wait never holds a slot a producer needs.
struct MlpOverride {
  int fused = 0;         // 0 automatic, 1 one launch (or fail), 2 two launches
  int down_depth = 0;    // stream depth of the consumers, 0 automatic
  int stream_after = 0;  // producers finished before consumers stream; 0 automatic, -1 at once
};

constexpr int kMlpWaves = 8;              // workgroup size of both halves of a fused launch
constexpr size_t kMlpControlBytes = 256;  // arrival counter and status word, padded
constexpr size_t kMlpFlagLineBytes = 128;  // each consumer's flag line (stream, go), after them

struct MlpPlan {
  GemmPlan up, down;             // the two-launch plans (each its own tuned shape)
  GemmPlan up_fused, down_fused; // the one-launch plans (kMlpWaves wavefronts, full-stage consumer)
  bool fusable;                  // the one-launch plans exist (the launcher still checks occupancy)
  bool fused_requested;          // the caller asked for one launch
  int producers, consumers;      // workgroups of the one-launch halves
  int stream_after;              // resolved: producers finished before consumers stream (0: at once)
  size_t lds_bytes;              // dynamic LDS of the one-launch kernel
  // Workspace: the gate_up GEMM's, the down GEMM's (each large enough for
  // either plan), then the control of the one-launch form: one flag line per
  // consumer from flags_offset, then the arrival counter and the status word
  // in the last kMlpControlBytes (from counter_offset).
  size_t down_ws_offset, flags_offset, counter_offset, workspace_bytes;
};

// Workgroups in the grid of a GEMM plan for an [n, k] weight.
int64_t gemm_grid(const GemmPlan& p, int64_t n);

// The MLP of gate_up [n_up, k_up] (gate rows first, then up rows) and down
// [n_dn, k_dn] with k_dn = n_up / 2, for m activation rows; false when the
// request is not possible.
bool plan_mlp(int fmt_up, int64_t n_up, int64_t k_up, int fmt_dn, int64_t n_dn, int64_t k_dn, int m,
              const MlpOverride& o, MlpPlan* plan);

// x pieces each thread stages per unit in the ring stage.
int ring_pieces(int waves, int k_slices, int m);

// The launch of one call, or false when the request is not possible.
bool plan_gemm(int fmt, int64_t n, int64_t k, int m, const LaunchOverride& o, GemmPlan* plan);

// Shapes the library takes: n * k / 2 must stay addressable and the kernels
// index rows with int.
bool shape_ok(int64_t n, int64_t k);

// Bytes of the packed form of an [n, k] weight (0 for an invalid request).
size_t packed_bytes(int fmt, int64_t n, int64_t k);

}  // namespace qpn
