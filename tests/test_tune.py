"""The launch-shape tuner's host side: its candidates are exactly the launch
shapes the planner accepts (each once, resolved), they include the balanced
grids where a shape has more groups than CUs and the uneven grid where the
planner takes it, and a table entry spells out a launch. Timing needs a GPU and is not run here."""

import quantized_weight_skinny_amd as q
from quantized_weight_skinny_amd import tune


def test_candidates_are_valid_resolved_and_unique():
    for fmt, n, k, m in ((q.QPN_FMT_NVFP4, 34816, 5120, 1), (q.QPN_FMT_FP8_E4M3, 5120, 17408, 8),
                         (q.QPN_FMT_NVFP4, 100, 272, 3)):
        cands = tune.candidates(fmt, n, k, m, 256)
        assert cands
        keys = [tuple(c[f] for f in tune.FIELDS) for c in cands]
        assert len(keys) == len(set(keys))
        w = tune.planner_weight(fmt, n, k)
        for c in cands:
            p = q.qpn_gemm_plan(w, m, q.make_launch(c["split_k"], c["waves"], c["depth"], c["k_slices"],
                                                   x_stage=c["x_stage"], whole_groups=c["whole_groups"]))
            assert (p.waves_per_group, p.k_slices, p.split_k, p.depth, p.x_stage, p.whole_groups) == \
                tuple(c[f] for f in tune.FIELDS)


def test_balanced_grids_are_among_the_candidates():
    # gate_up: 2176 n-tiles, 272 groups of 8; 256 kept whole on 256 CUs
    cands = tune.candidates(q.QPN_FMT_NVFP4, 34816, 5120, 1, 256)
    assert any(c["waves"] == 8 and c["k_slices"] == 1 and c["split_k"] == 4 and c["whole_groups"] == 256
               for c in cands)
    # the planner's own choice for the shape is one of them
    assert tune.current_plan(q.QPN_FMT_NVFP4, 34816, 5120, 1) in cands


def test_uneven_grid_is_among_the_candidates():
    # gate_up at 16 rows: 256 workgroups of 9 wavefronts (8 or 9 n-tiles each),
    # the planner's own choice there; FP8 has no uneven grid
    cands = tune.candidates(q.QPN_FMT_NVFP4, 34816, 5120, 16, 256)
    uneven = [c for c in cands if c["waves"] == tune.UNEVEN_WAVES]
    assert {(c["depth"], c["x_stage"]) for c in uneven} == {(2, q.QPN_X_STAGE_RING), (3, q.QPN_X_STAGE_RING)}
    assert all((c["k_slices"], c["split_k"], c["whole_groups"]) == (1, 1, 256) for c in uneven)
    assert tune.current_plan(q.QPN_FMT_NVFP4, 34816, 5120, 16) in uneven
    # at one row the full stage fits as well
    assert len([c for c in tune.candidates(q.QPN_FMT_NVFP4, 34816, 5120, 1, 256)
                if c["waves"] == tune.UNEVEN_WAVES]) == 4
    assert not [c for c in tune.candidates(q.QPN_FMT_FP8_E4M3, 34816, 5120, 16, 256)
                if c["waves"] == tune.UNEVEN_WAVES]


def test_table_entry():
    kw = dict(waves=8, k_slices=1, split_k=4, depth=2, x_stage=q.QPN_X_STAGE_RING, whole_groups=256)
    assert tune.table_entry(q.QPN_FMT_NVFP4, 34816, 5120, 1, kw) == \
        "{kFmtNvfp4, 34816, 5120, 1, 8, 1, 4, 2, kStageRing, 256}"
    kw = dict(waves=9, k_slices=1, split_k=1, depth=2, x_stage=q.QPN_X_STAGE_RING, whole_groups=256)
    assert tune.table_entry(q.QPN_FMT_NVFP4, 34816, 5120, 16, kw) == \
        "{kFmtNvfp4, 34816, 5120, 16, kUnevenWaves, 1, 1, 2, kStageRing, 256}"
