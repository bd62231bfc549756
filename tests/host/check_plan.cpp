// Host driver of the launch planner and the C ABI's argument checks, built by
// tests/test_build_checks.py with g++ -fsanitize=address,undefined together
// with qpn_plan.cpp and qpn_checks.cpp (no HIP runtime, no device). It sweeps
// shapes, row counts and launch overrides, valid and not, through plan_gemm,
// the check_* functions and the entry points that need no device, and checks
// the invariants the kernels rely on for every plan the planner accepts.
// Prints "ok <plans accepted> <calls>" and exits 0, or names the first
// broken invariant and exits 1.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/qpn.h"
#include "../../quantized_weight_skinny_amd/csrc/qpn_checks.hpp"
#include "../../quantized_weight_skinny_amd/csrc/qpn_plan.hpp"

using namespace qpn;

namespace {

uint64_t g_state = 0x9e3779b97f4a7c15ull;
uint64_t next_u64() {  // splitmix64
  uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
template <typename T, size_t N>
T pick(const T (&a)[N]) {
  return a[next_u64() % N];
}

long g_calls = 0, g_plans = 0;

[[noreturn]] void fail(const char* what, int fmt, int64_t n, int64_t k, int m, const LaunchOverride& o) {
  printf("FAIL %s: fmt=%d n=%lld k=%lld m=%d override{split=%d waves=%d depth=%d k_slices=%d epilogue=%d "
         "x_stage=%d whole_groups=%d valu_dot=%d block_cols=%d}\n",
         what, fmt, static_cast<long long>(n), static_cast<long long>(k), m, o.split, o.waves, o.depth, o.k_slices,
         o.epilogue, o.x_stage, o.whole_groups, o.valu_dot, o.block_cols);
  exit(1);
}

#define REQUIRE(cond)                                  \
  do {                                                 \
    if (!(cond)) fail(#cond, fmt, n, k, m, o);         \
  } while (0)

// Every accepted plan: the launch shape the kernels are instantiated for, a
// K range that covers K exactly once, LDS within the budget and a workspace
// that holds what the kernels write there.
void check_plan(int fmt, int64_t n, int64_t k, int m, const LaunchOverride& o, const GemmPlan& p) {
  const int64_t NT = ceil_div(n, kTileN), KU = ceil_div(k, kUnitK);
  REQUIRE(fmt == kFmtNvfp4 || fmt == kFmtFp8);
  REQUIRE(m >= 1 && m <= kMaxM && n >= 1 && k >= 0);
  // The uneven-group grid: whole_groups workgroups of kUnevenWaves
  // wavefronts share the n-tiles (at most kUnevenWaves each), NVFP4, fp16 or
  // fp32 y on the MFMA path, one K slice, no split.
  const bool uneven = p.waves == kUnevenWaves;
  REQUIRE(p.waves == 4 || p.waves == 8 || uneven);
  if (uneven) {
    REQUIRE(fmt == kFmtNvfp4 && (p.epilogue == kEpiNone || p.epilogue == kEpiF32));
    REQUIRE(p.k_slices == 1 && p.split == 1 && (p.depth == 2 || p.depth == 3));
    REQUIRE(p.dot_rows == 0 && p.block_cols == 0);
    REQUIRE(p.whole_groups >= 1 && p.whole_groups <= NT && ceil_div(NT, p.whole_groups) <= kUnevenWaves);
    REQUIRE(gemm_grid(p, n) == p.whole_groups);
  }
  REQUIRE(p.k_slices == 1 || p.k_slices == 2 || p.k_slices == 4 || p.k_slices == 8);
  REQUIRE(p.k_slices <= p.waves && p.waves % p.k_slices == 0);
  REQUIRE(p.depth == 2 || p.depth == 3 || p.depth == 4 || p.depth == 6 || p.depth == 8);
  REQUIRE(p.x_stage == kStageFull || p.x_stage == kStageRing);
  REQUIRE(p.epilogue == o.epilogue);
  REQUIRE(p.split >= 1);
  if (KU) {
    REQUIRE(p.units_per_split >= 1);
    REQUIRE(static_cast<int64_t>(p.units_per_split) * p.split >= KU);
    REQUIRE(static_cast<int64_t>(p.units_per_split) * (p.split - 1) < KU);  // no empty K piece
  } else {
    REQUIRE(p.split == 1 && p.units_per_split == 0);
  }
  const int64_t groups = ceil_div(NT, p.waves / p.k_slices);
  if (p.split == 1) REQUIRE(p.whole_groups == 0 || uneven);
  else REQUIRE(p.whole_groups >= 0 && p.whole_groups <= groups);
  // unit offsets inside a stream are 32-bit
  REQUIRE(NT * KU * (fmt == kFmtNvfp4 ? kNvUnitBytes : kF8UnitBytes) < (int64_t(1) << 31));
  // LDS: the stage (and, with K slices, the reduction tiles) within the budget
  REQUIRE(p.lds_bytes <= kLdsBudget);
  if (p.x_stage == kStageFull) {
    const int64_t staged_units = p.split > 1 && p.whole_groups > 0 ? KU : p.units_per_split;
    REQUIRE(p.lds_stride == staged_units * kUnitK + kRowPad);
    REQUIRE(static_cast<size_t>(m) * p.lds_stride * kHalfBytes <= p.lds_bytes);
  } else {
    REQUIRE(p.depth <= 4);
    REQUIRE(ring_pieces(p.waves, p.k_slices, m) <= kRingMaxPieces);
    REQUIRE(static_cast<size_t>(p.k_slices) * kRingSlots * m * kRingRow * kHalfBytes <= p.lds_bytes);
    REQUIRE(2 * static_cast<int64_t>(m) * k < (int64_t(1) << 31));
  }
  if (p.k_slices > 1) REQUIRE(static_cast<size_t>(p.waves) * 64 * kTileLaneBytes <= p.lds_bytes);
  if (p.block_cols) {
    REQUIRE(m == 1 && fmt == kFmtNvfp4 && p.x_stage == kStageFull && p.dot_rows == 0);
    REQUIRE(o.block_cols == 1);
    REQUIRE(static_cast<size_t>(m) * p.lds_stride * kHalfBytes + (p.depth * kUnitK + 64) * kHalfBytes <=
            p.lds_bytes);
  }
  if (o.block_cols == 1) REQUIRE(p.block_cols == 1);
  if (p.dot_rows) {
    REQUIRE(p.dot_rows >= m && (p.dot_rows == 1 || p.dot_rows == 2 || p.dot_rows == 4));
    REQUIRE(p.x_stage == kStageFull && p.epilogue == kEpiNone && p.depth <= 4);
  }
  if (o.epilogue == kEpiSwiglu) {
    REQUIRE(n % (2 * kTileN) == 0);
    REQUIRE((p.waves / p.k_slices) % 2 == 0);
    REQUIRE(static_cast<size_t>(p.waves / p.k_slices / 2) * 64 * kTileLaneBytes <= p.lds_bytes);
  }
  // Workspace: counters (one int per n-tile), then the control block, then
  // the partial sums [split][m][n] in fp32.
  REQUIRE(p.control_offset >= static_cast<size_t>(NT) * sizeof(int) && p.control_offset % 256 == 0);
  REQUIRE(p.partials_offset == p.control_offset + kControlBytes && p.partials_offset % 16 == 0);
  if (p.split > 1)
    REQUIRE(p.workspace_bytes >= p.partials_offset + static_cast<size_t>(p.split) * m * n * sizeof(float));
  if (o.epilogue == kEpiArgmax) REQUIRE(p.workspace_bytes >= p.partials_offset);
  if (p.split == 1 && o.epilogue != kEpiArgmax) REQUIRE(p.workspace_bytes == 0);
  // A caller's explicit choice is binding.
  if (o.waves) REQUIRE(p.waves == o.waves);
  if (o.k_slices) REQUIRE(p.k_slices == o.k_slices);
  if (o.depth) REQUIRE(p.depth == o.depth);
  if (o.x_stage) REQUIRE(p.x_stage == o.x_stage);
}

const int64_t kNs[] = {-16, -1, 0, 1, 15, 16, 17, 31, 32, 48, 1000, 1792, 5120, 7168, 8704, 34816, 151936,
                       int64_t(1) << 20, (int64_t(1) << 31) - 16, (int64_t(1) << 31), INT64_MAX};
const int64_t kKs[] = {-256, -16, 0, 8, 16, 240, 256, 272, 1280, 4352, 5120, 17408, 65536, int64_t(1) << 20,
                       int64_t(1) << 30, (int64_t(1) << 30) + 16, INT64_MAX - 15};
const int kFmts[] = {0, kFmtNvfp4, kFmtFp8, 3};
const int kSplits[] = {0, 0, 0, 1, 2, 3, 4, 6, 7, 100, -1};
const int kWaves[] = {0, 0, 0, 4, 8, 9, 2, -4, 16};
const int kDepths[] = {0, 0, 0, 2, 3, 4, 6, 8, 5, -1};
const int kSlices[] = {0, 0, 0, 1, 2, 4, 8, 3, 16};
const int kEpis[] = {0, 0, 1, 2, 3, 4, -1};
const int kStages[] = {0, 0, kStageFull, kStageRing, 3};
const int kWhole[] = {0, 0, 1, 16, 256, 512, 100000, -1};
const int kFlags[] = {0, 0, 0, 1, 2, -1};

LaunchOverride random_override() {
  LaunchOverride o;
  o.split = pick(kSplits);
  o.waves = pick(kWaves);
  o.depth = pick(kDepths);
  o.k_slices = pick(kSlices);
  o.epilogue = pick(kEpis);
  o.x_stage = pick(kStages);
  o.whole_groups = pick(kWhole);
  o.valu_dot = pick(kFlags) == 1;
  o.block_cols = pick(kFlags);
  return o;
}

// A pointer value with a chosen alignment (never dereferenced).
const void* fake_ptr(int kind) {
  static const uintptr_t base = 0x7f0000001000ull;
  switch (kind % 5) {
    case 0: return nullptr;
    case 1: return reinterpret_cast<const void*>(base + 1);
    case 2: return reinterpret_cast<const void*>(base + 2);
    case 3: return reinterpret_cast<const void*>(base + 4);
    default: return reinterpret_cast<const void*>(base);
  }
}

void sweep_planner() {
  for (int fmt : kFmts)
    for (int64_t n : kNs)
      for (int64_t k : kKs)
        for (int m = -1; m <= kMaxM + 1; ++m)
          for (int r = 0; r < 24; ++r) {
            const LaunchOverride o = r == 0 ? LaunchOverride{} : random_override();
            GemmPlan p;
            memset(&p, 0xa5, sizeof p);
            ++g_calls;
            if (!plan_gemm(fmt, n, k, m, o, &p)) continue;
            ++g_plans;
            check_plan(fmt, n, k, m, o, p);
          }
}

void sweep_checks() {
  const size_t sizes[] = {0, 1, 15, 16, 2304, 4096, size_t(1) << 30, SIZE_MAX};
  const float scales[] = {1.0f, 0.5f, 0.0f, -1.0f, INFINITY, NAN, 1e-30f};
  for (int it = 0; it < 400000; ++it) {
    const int64_t n = pick(kNs), k = pick(kKs);
    const size_t bytes = pick(sizes);
    const auto P = [](int kind) { return fake_ptr(kind); };
    const int a = static_cast<int>(next_u64() % 5), b = static_cast<int>(next_u64() % 5),
              c = static_cast<int>(next_u64() % 5), d = static_cast<int>(next_u64() % 5);
    bool run = true;
    const auto u8 = [&](int kind) { return static_cast<const uint8_t*>(P(kind)); };
    const auto f32 = [&](int kind) { return static_cast<const float*>(P(kind)); };
    qpn_status st = QPN_OK;
    switch (it % 11) {
      case 0: st = check_pack_nvfp4(u8(a), u8(b), n, k, P(c), bytes, static_cast<const int32_t*>(P(d)), &run); break;
      case 1: st = check_pack_fp8(u8(a), n, k, P(c), bytes, static_cast<const int32_t*>(P(d)), &run); break;
      case 2: st = check_unpack_nvfp4(P(a), bytes, n, k, u8(b), u8(c), &run); break;
      case 3: st = check_unpack_fp8(P(a), bytes, n, k, u8(b), &run); break;
      case 4: st = check_absmax_f32(f32(a), n, f32(b), &run); break;
      case 5: st = check_quantize_nvfp4(f32(a), n, k, pick(scales), u8(b), u8(c), &run); break;
      case 6: st = check_quantize_fp8(f32(a), n, k, u8(b), f32(c), &run); break;
      case 7: st = check_fp8_absmax(u8(a), f32(b), n, k, f32(c), &run); break;
      case 8:
        st = check_requantize_fp8_nvfp4(u8(a), f32(b), n, k, pick(scales), u8(c), u8(d), &run);
        break;
      case 9:
        st = check_read_ceiling(P(a), bytes, static_cast<const uint32_t*>(P(b)),
                                static_cast<int32_t>(next_u64() % 5) - 1, pick(kFlags) * 2, &run);
        break;
      default: {
        qpn_weight w{};
        w.format = pick(kFmts);
        w.n = n;
        w.k = k;
        w.packed = P(a);
        w.row_scales = f32(b);
        w.tensor_scale = pick(scales);
        w.reserved = next_u64() % 16 == 0 ? 1 : 0;
        const LaunchOverride o = random_override();
        const int m = static_cast<int>(next_u64() % 19) - 1;
        GemmPlan p;
        st = check_gemm(P(c), next_u64() % 8 ? &w : nullptr, P(d), f32(static_cast<int>(next_u64() % 5)), m,
                        P(static_cast<int>(next_u64() % 5)), bytes, o, &p, &run);
        if (st == QPN_OK && run) {
          const int fmt = w.format;
          REQUIRE(bytes >= p.workspace_bytes);
          check_plan(fmt, n, k, m, o, p);
        }
      }
    }
    ++g_calls;
    if (st != QPN_OK && run) {
      printf("FAIL check %d: a failed check asks for a launch\n", it % 11);
      exit(1);
    }
  }
}

void sweep_entry_points() {
  for (int s = -2; s < 8; ++s)
    if (!qpn_status_string(static_cast<qpn_status>(s))) {
      printf("FAIL qpn_status_string(%d) is null\n", s);
      exit(1);
    }
  for (int fmt : kFmts)
    for (int64_t n : kNs)
      for (int64_t k : kKs) {
        const size_t pb = qpn_packed_bytes(fmt, n, k);
        const bool ok = (fmt == QPN_FMT_NVFP4 || fmt == QPN_FMT_FP8_E4M3) && shape_ok(n, k);
        if (!ok && pb != 0) {
          printf("FAIL qpn_packed_bytes(%d, %lld, %lld) = %zu for an invalid request\n", fmt,
                 static_cast<long long>(n), static_cast<long long>(k), pb);
          exit(1);
        }
        if (ok && n > 0 && k > 0 &&
            pb != static_cast<size_t>(ceil_div(n, 16) * ceil_div(k, 256)) * (fmt == QPN_FMT_NVFP4 ? 2304 : 4096)) {
          printf("FAIL qpn_packed_bytes(%d, %lld, %lld) = %zu\n", fmt, static_cast<long long>(n),
                 static_cast<long long>(k), pb);
          exit(1);
        }
        for (int r = 0; r < 8; ++r) {
          qpn_weight w{};
          w.format = fmt;
          w.n = n;
          w.k = k;
          qpn_launch l{};
          l.split_k = pick(kSplits);
          l.waves_per_group = pick(kWaves);
          l.depth = pick(kDepths);
          l.k_slices = pick(kSlices);
          l.epilogue = pick(kEpis);
          l.x_stage = pick(kStages);
          l.whole_groups = pick(kWhole);
          l.valu_dot = pick(kFlags);
          l.block_columns = pick(kFlags);
          const int32_t m = static_cast<int32_t>(next_u64() % 19) - 1;
          qpn_launch res;
          const qpn_status st = qpn_gemm_plan(&w, m, r ? &l : nullptr, &res);
          const size_t ws = qpn_workspace_bytes_tuned(&w, m, r ? &l : nullptr);
          g_calls += 2;
          if (st == QPN_OK) {
            // the resolved launch plans to itself
            qpn_launch again;
            if (qpn_gemm_plan(&w, m, &res, &again) != QPN_OK || memcmp(&res, &again, sizeof res) != 0 ||
                qpn_workspace_bytes_tuned(&w, m, &res) != ws) {
              printf("FAIL resolved launch does not replan to itself: fmt=%d n=%lld k=%lld m=%d\n", fmt,
                     static_cast<long long>(n), static_cast<long long>(k), m);
              exit(1);
            }
          } else if (ws != 0) {
            printf("FAIL workspace bytes %zu for a launch the planner rejects\n", ws);
            exit(1);
          }
        }
      }
}

// The fused MLP plans: both halves' plans valid, a one-launch form only with
// one workgroup size and a full-stage consumer, the workspace regions in
// order and large enough for either form.
void sweep_mlp() {
  const int64_t fs[] = {-16, 0, 16, 32, 48, 1000, 1024, 4352, 8704, 17408, int64_t(1) << 24};
  const int64_t ks[] = {-16, 0, 16, 256, 272, 5120, int64_t(1) << 20};
  const int64_t ns[] = {-1, 0, 1, 17, 512, 5120, 151936};
  const int fused[] = {0, 1, 2, 3, -1};
  const int depths[] = {0, 0, 2, 3, 4, 6, 8, 5};
  const int after[] = {0, 0, -1, 1, 160, 100000, -2};
  for (int it = 0; it < 200000; ++it) {
    const int64_t f = pick(fs), k = pick(ks), n = pick(ns);
    const int fmt_up = pick(kFmts), fmt_dn = pick(kFmts);
    const int m = static_cast<int>(next_u64() % 19) - 1;
    MlpOverride mo;
    mo.fused = pick(fused);
    mo.down_depth = pick(depths);
    mo.stream_after = pick(after);
    const int64_t n_up = 2 * f, k_dn = next_u64() % 16 ? f : f + 16;
    MlpPlan p;
    memset(&p, 0x5a, sizeof p);
    ++g_calls;
    if (!plan_mlp(fmt_up, n_up, k, fmt_dn, n, k_dn, m, mo, &p)) continue;
    ++g_plans;
    const LaunchOverride o{};  // for the failure message only
    const int fmt = fmt_up;
    REQUIRE(k_dn == n_up / 2 && n_up % 32 == 0 && m >= 1 && m <= kMaxM);
    REQUIRE(p.up.epilogue == kEpiSwiglu && p.down.epilogue == kEpiNone);
    if (p.fusable) {
      REQUIRE(fmt_up == kFmtNvfp4 && fmt_dn == kFmtNvfp4 && mo.fused != 2);
      REQUIRE(p.up_fused.waves == kMlpWaves && p.down_fused.waves == kMlpWaves);
      REQUIRE(p.down_fused.x_stage == kStageFull && p.down_fused.dot_rows == 0 && p.down_fused.block_cols == 0);
      REQUIRE(p.up_fused.depth == 2 || p.up_fused.depth == 3);
      REQUIRE(p.up_fused.x_stage == kStageFull || ring_pieces(kMlpWaves, p.up_fused.k_slices, m) == 1);
      if (mo.down_depth) REQUIRE(p.down_fused.depth == mo.down_depth);
      REQUIRE(p.producers == gemm_grid(p.up_fused, n_up) && p.consumers == gemm_grid(p.down_fused, n));
      REQUIRE(p.lds_bytes >= p.up_fused.lds_bytes && p.lds_bytes >= p.down_fused.lds_bytes);
      REQUIRE(p.lds_bytes <= kLdsBudget);
      REQUIRE(p.stream_after >= 0 && p.stream_after <= p.producers);
    } else {
      REQUIRE(mo.fused != 1);
    }
    REQUIRE(p.fused_requested == (mo.fused == 1));
    REQUIRE(p.down_ws_offset % 256 == 0 && p.flags_offset % 256 == 0);
    REQUIRE(p.down_ws_offset >= p.up.workspace_bytes && p.down_ws_offset >= p.up_fused.workspace_bytes);
    REQUIRE(p.flags_offset - p.down_ws_offset >= p.down.workspace_bytes);
    REQUIRE(p.flags_offset - p.down_ws_offset >= p.down_fused.workspace_bytes);
    REQUIRE(p.counter_offset == p.flags_offset + static_cast<size_t>(p.consumers) * kMlpFlagLineBytes);
    REQUIRE(p.workspace_bytes == p.counter_offset + kMlpControlBytes);
  }
  // the C entry points around it, with arbitrary arguments
  for (int it = 0; it < 100000; ++it) {
    qpn_weight up{}, dn{};
    up.format = pick(kFmts);
    dn.format = pick(kFmts);
    up.n = 2 * pick(fs);
    up.k = pick(ks);
    dn.n = pick(ns);
    dn.k = next_u64() % 8 ? up.n / 2 : pick(fs);
    up.packed = fake_ptr(static_cast<int>(next_u64() % 5));
    dn.packed = fake_ptr(static_cast<int>(next_u64() % 5));
    up.tensor_scale = dn.tensor_scale = 1.0f;
    up.row_scales = dn.row_scales = static_cast<const float*>(fake_ptr(4));
    qpn_mlp_launch l{};
    l.fused = pick(fused);
    l.down_depth = pick(depths);
    l.stream_after = pick(after);
    l.reserved = next_u64() % 16 == 0;
    const int32_t m = static_cast<int32_t>(next_u64() % 19) - 1;
    const size_t need = qpn_mlp_workspace_bytes(&up, &dn, m, next_u64() % 2 ? &l : nullptr);
    MlpOverride mo;
    bool run = false;
    qpn_status st = QPN_ERR_INVALID_ARG;
    MlpPlan p;
    if (to_mlp_override(&l, &mo))
      st = check_mlp(fake_ptr(static_cast<int>(next_u64() % 5)), &up, &dn, fake_ptr(static_cast<int>(next_u64() % 5)),
                     fake_ptr(static_cast<int>(next_u64() % 5)), m, fake_ptr(static_cast<int>(next_u64() % 5)),
                     next_u64() % 2 ? need : need / 2, mo, &p, &run);
    g_calls += 2;
    if (st != QPN_OK && run) {
      printf("FAIL check_mlp: a failed check asks for a launch\n");
      exit(1);
    }
  }
}

}  // namespace

int main() {
  sweep_planner();
  sweep_checks();
  sweep_entry_points();
  sweep_mlp();
  printf("ok %ld %ld\n", g_plans, g_calls);
  return 0;
}
