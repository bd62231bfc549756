"""The launch-shape tuner end to end on a small shape: it times every finalist
and reports the planner's current launch among them."""

import pytest

import quantized_weight_skinny_amd as q
from quantized_weight_skinny_amd import tune

pytestmark = pytest.mark.gpu


def test_tune_small_shape():
    print("tune small shape", flush=True)
    res = tune.tune(q.QPN_FMT_NVFP4, 1024, 2048, 2, top=2, rounds=1, log=lambda *a: None)
    assert 2 <= len(res) <= 3
    assert all(us > 0 for us, _, _ in res)
    assert [us for us, _, _ in res] == sorted(us for us, _, _ in res)
    assert sum(1 for _, _, cur in res if cur) == 1
