"""GPU parity of paged_decode_step_static (the decode step that allocates
nothing, its scratch a fixed device array) against paged_decode_step with a
workspace: outputs and caches bitwise equal, on two calls in a row, the second
smaller, plus the oracle's tolerance on sampled outputs."""

import dataclasses

import numpy as np
import pytest
import torch

import paged_kv_cache_353_amd as pkv
from paged_kv_cache_353_amd import workloads as W
from tests.gpu_helpers import assert_close, host_inputs, oracle_step, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _clone(inp):
    return dataclasses.replace(inp, k_cache=inp.k_cache.clone(), v_cache=inp.v_cache.clone())


def _run(inp, static):
    out = torch.full_like(inp.q, float("nan"))
    fn = pkv.paged_decode_step_static if static else pkv.paged_decode_step
    fn(out, inp.q, inp.k_new, inp.v_new, inp.k_cache, inp.v_cache, inp.block_tables,
       inp.context_lens, inp.block_size, inp.scale, max_context_len=inp.max_context_len)
    torch.cuda.synchronize()
    return out


def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32)


def _compare(inp, what, pairs=None, dtype="bf16"):
    h = host_inputs(inp)
    a, b = _clone(inp), _clone(inp)
    ref = _run(a, static=False)
    got = _run(b, static=True)
    assert torch.equal(_bits(got), _bits(ref)), f"{what}: output differs from paged_decode_step"
    assert torch.equal(_bits(b.k_cache), _bits(a.k_cache)), f"{what}: K cache differs"
    assert torch.equal(_bits(b.v_cache), _bits(a.v_cache)), f"{what}: V cache differs"
    want = oracle_step(h, inp, pairs=pairs)
    return assert_close(got, want, dtype, pairs=pairs, what=what)


def test_static_step_two_calls_second_smaller():
    say("case: static step, llama8b-shaped batch then a small ragged one")
    big = W.llama8b_decode(DEV)
    rng = np.random.default_rng(11)
    pairs = sorted({(int(rng.integers(64)), int(rng.integers(32))) for _ in range(64)})
    worst = _compare(big, "static llama8b", pairs=pairs)
    say(f"  first call worst normwise error {worst:.2e}")
    lens = [0, 1, 2, 17, 300, 1025]
    small = W.build_decode_inputs(lens, 16, 4, 128, 16, "bf16", 120, seed=431, device=DEV)
    worst = _compare(small, "static small")
    say(f"  second call worst normwise error {worst:.2e}")


@pytest.mark.parametrize("dtype,D,G", [("f32", 64, 1), ("f16", 128, 2), ("f16", 64, 8), ("bf16", 64, 2), ("bf16", 128, 8)])
def test_static_step_other_shapes(dtype, D, G):
    say(f"case: static step dtype={dtype} D={D} G={G}")
    lens = [3, 16, 33, 257, 700]
    bs = 32
    nb = sum(-(-L // bs) for L in lens) + 2
    inp = W.build_decode_inputs(lens, 2 * G, 2, D, bs, dtype, nb, seed=440 + D + G, device=DEV)
    _compare(inp, f"static {dtype} D{D} G{G}", dtype=dtype)


def test_static_step_limits_are_refused():
    """Sizes beyond the fixed array and configurations of the many-column
    kernel raise on the host; nothing is launched."""
    say("case: static step limits")
    inp = W.build_decode_inputs([4] * 3, 6, 2, 64, 16, "bf16", 4, seed=450, device=DEV)
    out = torch.empty_like(inp.q)
    with pytest.raises(pkv.PKVError) as e:   # group 3: the many-column kernel's case
        pkv.paged_decode_step_static(out, inp.q, inp.k_new, inp.v_new, inp.k_cache, inp.v_cache,
                                     inp.block_tables, inp.context_lens, 16, 0.125,
                                     max_context_len=inp.max_context_len)
    assert e.value.status == 4   # PKV_ERR_UNSUPPORTED
    # 16385 units: one more than the array's counters hold
    S, hkv, d = 16385, 1, 64
    q = torch.zeros(S, 1, d, dtype=torch.bfloat16, device=DEV)
    kn = torch.zeros(S, hkv, d, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(1, hkv, 16, d, dtype=torch.bfloat16, device=DEV)
    bt = torch.zeros(S, 1, dtype=torch.int32, device=DEV)
    cl = torch.zeros(S, dtype=torch.int32, device=DEV)
    with pytest.raises(pkv.PKVError) as e:
        pkv.paged_decode_step_static(torch.empty_like(q), q, kn, kn.clone(), kc, kc.clone(), bt, cl, 16,
                                     0.125, max_context_len=16)
    assert e.value.status == 5   # PKV_ERR_WORKSPACE
