"""The input generator's own records, checked against the rows it produced.

The update mask a sampler would hand the count gate is the generator's record
of the positions it rewrote (`rewritten`), next to their count (`touched`).
Both must agree with a direct comparison of consecutive block tensors, so
that a gate fed the mask decides as a gate comparing rows does.
"""

import numpy as np
import pytest

from workloads.synth import make_block_schedule


@pytest.mark.parametrize("schedule,dtype", [("redraw", "bf16"), ("unmask", "bf16"), ("poisson", "f32"),
                                            ("qnoise", "bf16")])
def test_rewritten_record_matches_the_rows(schedule, dtype):
    s = make_block_schedule(dtype=dtype, B=3, hq=4, hkv=2, d=16, lp=8, nb=12, steps=9, schedule=schedule,
                            redraw_range=(0, 4), unmask_range=(1, 3), poisson_lam=2.0, seed=11)
    assert s.rewritten.shape == (s.steps + 1, s.B, s.nb) and s.rewritten.dtype == np.uint8
    assert not s.rewritten[0].any()
    for t in range(1, s.steps + 1):
        changed = np.zeros((s.B, s.nb), dtype=bool)
        for cur, prev in ((s.q[t], s.q[t - 1]), (s.k[t], s.k[t - 1]), (s.v[t], s.v[t - 1])):
            changed |= (np.asarray(cur).view(np.uint8).reshape(s.B, s.nb, -1)
                        != np.asarray(prev).view(np.uint8).reshape(s.B, s.nb, -1)).any(axis=2)
        assert np.array_equal(s.rewritten[t].astype(bool), changed), (schedule, t)
        assert np.array_equal(s.rewritten[t].sum(axis=1), s.touched[t]), (schedule, t)


def test_generator_is_deterministic_with_the_record():
    # the same seed gives the same tensors and the same record
    a = make_block_schedule(B=2, hq=2, hkv=1, d=8, lp=4, nb=6, steps=3, schedule="poisson", seed=3)
    b = make_block_schedule(B=2, hq=2, hkv=1, d=8, lp=4, nb=6, steps=3, schedule="poisson", seed=3)
    for x, y in zip(a.q + a.k + a.v + [a.kp, a.vp], b.q + b.k + b.v + [b.kp, b.vp]):
        assert np.array_equal(x, y)
    assert np.array_equal(a.rewritten, b.rewritten)
