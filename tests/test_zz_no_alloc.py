"""The allocation-free entry point (plsh_alibi_attention_noalloc) against
the caller-workspace entry point it mirrors: same kernels, so the outputs
must be bitwise equal, on two calls in a row (the second smaller, so the
shared static scratch still holds the first call's larger record set)."""

import sys

import pytest
import torch

from approximate_long_context_amd import plsh, workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def _pair(w, seed):
    q, k, v = (x.to("cuda:0") for x in W.make_qkv(w))
    t = plsh.sample_tables(seed, w.n, w.sigma, w.s).to("cuda:0")
    ref = plsh.attention(q, k, v, w.sigma, w.s, t, causal=w.causal)
    out = torch.empty_like(q)
    got = plsh.attention_noalloc(q, k, v, w.sigma, w.s, t, causal=w.causal, out=out)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_equals_workspace_entry_two_calls():
    big = W.get("mistral-7b-n16384-s20")
    small = W.Workload("noalloc-small", 2, 4, 2, 700, 64, "bf16", False, [1.5, 6.0, 30.0, 300.0], 9)
    for w, seed in ((big, 0), (small, 5)):
        say("noalloc", w.name, "B", w.batch, "H", w.heads, "n", w.n, "d", w.d, "s", w.s)
        ref, got = _pair(w, seed)
        assert got.data_ptr() != ref.data_ptr()
        assert torch.equal(ref, got), w.name


def test_noalloc_fp32_path_needs_no_scratch():
    w = W.get("tiny-f32-n512")
    say("noalloc", w.name)
    ref, got = _pair(w, 0)
    assert torch.equal(ref, got)


def test_noalloc_refuses_beyond_scratch():
    """8 heads, n = 131072, s = 48 need 67.6 MB of records (> 64 MiB)."""
    w = W.get("long-n131072")
    say("noalloc capacity", w.name)
    q = torch.zeros((1, w.heads, w.n, w.d), dtype=torch.bfloat16, device="cuda:0")
    t = plsh.sample_tables(0, w.n, w.sigma, w.s).to("cuda:0")
    with pytest.raises(plsh.PlshError) as e:
        plsh.attention_noalloc(q, q, q, w.sigma, w.s, t, causal=True, out=torch.empty_like(q))
    assert e.value.status == plsh.PLSH_ERR_CAPACITY
