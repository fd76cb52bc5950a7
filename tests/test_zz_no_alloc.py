"""ba_prefix_attn_noalloc -- prefix attention with its split-KV partials in the
library's static per-GPU scratch instead of a caller workspace -- against
ba_prefix_attn on the same inputs, through the C-ABI: two calls in a row,
the second on a smaller input (so it reuses scratch the first left behind),
each bit-identical to ba_prefix_attn and within the parity bars of the CPU
oracle on every row."""

import numpy as np
import pytest
import torch

import oracle
from workloads import make_block_schedule
from tests.gpu_util import DEV, check_a, check_l, dev_in, host

pytestmark = pytest.mark.gpu

ba = pytest.importorskip("cached_split_attention_amd")
from cached_split_attention_amd import _lib  # noqa: E402


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# (B, hq, hkv, d, lp, nb, seed): GQA with 64-row tiles and a ragged last
# key split; then a smaller MHA problem with fewer splits
SHAPES = [(2, 8, 2, 128, 5000, 40, 81), (1, 4, 4, 128, 1500, 20, 82)]


def _one_call(shape, gated):
    B, hq, hkv, d, lp, nb, seed = shape
    s = make_block_schedule(dtype="bf16", B=B, hq=hq, hkv=hkv, d=d, lp=lp, nb=nb, steps=0, std=1.0,
                            schedule="none", seed=seed)
    q, kp, vp = dev_in(s.q[0], "bf16"), dev_in(s.kp, "bf16"), dev_in(s.vp, "bf16")
    rows = B * nb
    need = ba.ba_prefix_attn_workspace(q, kp, vp)
    assert 0 < need <= _lib.BA_NOALLOC_SCRATCH_BYTES, "the shape must use the split scratch"
    dec = None
    if gated:
        # every other head reused: its cache entries must stay untouched
        dec = torch.zeros(B, hq, device=DEV, dtype=torch.uint8)
        dec[:, ::2] = 1
    cache_a = torch.full((rows, hq, d), 7.0, device=DEV)
    cache_l = torch.full((rows, hq), -3.0, device=DEV)
    ws = torch.zeros(need, device=DEV, dtype=torch.uint8)
    a_ref, l_ref = cache_a.clone(), cache_l.clone()
    ba.ba_prefix_attn(q, kp, vp, a_ref, l_ref, ws, decision=dec)
    a, l = cache_a.clone(), cache_l.clone()
    ba.ba_prefix_attn_noalloc(q, kp, vp, a, l, decision=dec)
    torch.cuda.synchronize()
    print(f"shape {shape} gated={gated}: {need} bytes of split scratch", flush=True)
    assert torch.equal(a, a_ref), "A_out differs from ba_prefix_attn"
    assert torch.equal(l, l_ref), "L_out differs from ba_prefix_attn"
    ga = host(a).reshape(B, nb, hq, d)
    gl = host(l).reshape(B, nb, hq)
    for b in range(B):
        for h in range(hq):
            if gated and h % 2 == 0:
                assert (ga[b, :, h] == 7.0).all() and (gl[b, :, h] == -3.0).all(), "reused head written"
                continue
            wa, wl = oracle.prefix_rows(s, 0, b, h)
            check_a(ga[b, :, h], wa, f"A_out b{b} h{h}")
            check_l(gl[b, :, h], wl, f"L_out b{b} h{h}")


@pytest.mark.parametrize("gated", [False, True])
def test_noalloc_matches_workspace_call(gated):
    for shape in SHAPES:   # two calls in a row, the second smaller
        _one_call(shape, gated)
