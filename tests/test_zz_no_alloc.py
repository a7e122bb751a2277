"""The allocation-free decode call (pre_attn_decode_noalloc, the library's
per-GPU scratch as its workspace) against pre_attn_decode with a caller
workspace, through the C ABI: two calls in a row, the second with fewer tokens
and a smaller hidden size, each bit for bit equal to the plain call (the same
kernels), and a call whose workspace would not fit the scratch rejected."""

import sys

import numpy as np
import pytest
import torch

import synth
from tests import parity

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(S, K, nkv, seed):
    wl = synth.Workload(name=f"noalloc_s{S}_k{K}_nkv{nkv}", mode="decode", tokens=S, hidden=K, nkv=nkv,
                        max_pos=4096, num_pages=max(1, -(-S // 16) + 2), layout="random", skip_frac=0.1)
    return synth.make_workload(wl, seed=seed)


def _outputs(p):
    return p.outputs()


def test_noalloc_matches_workspace_call_twice():
    from kv_residual_add_amd import _binding as B
    from kv_residual_add_amd.runner import Problem

    for S, K, nkv, seed in ((40, 2048, 2, 5), (6, 1024, 1, 6)):  # the second call smaller
        _say(f"noalloc S={S} K={K} nkv={nkv}")
        inp = _case(S, K, nkv, seed)
        plain = Problem(inp)
        plain.run()
        want = plain.outputs()
        p = Problem(inp)
        a = p.args()
        B.pre_attn_decode_noalloc(*a[:-1])  # every argument but the workspace
        got = p.outputs()
        for k in want:
            assert np.array_equal(want[k].view(np.uint8), got[k].view(np.uint8)), k
        parity.check_written_sets(inp, got)


def test_noalloc_rejects_workspace_past_the_scratch():
    from kv_residual_add_amd import _binding as B
    from kv_residual_add_amd.runner import Problem

    inp = _case(64, 16384, 4, 7)
    p = Problem(inp)
    assert B.pa_workspace_bytes(p.dims, B.PA_MODE_DECODE) > (24 << 20)
    with pytest.raises(B.PaError) as e:
        B.pre_attn_decode_noalloc(*p.args()[:-1])
    assert e.value.status == B.PA_ERR_WORKSPACE
