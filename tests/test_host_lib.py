"""Host half of libplsh (no GPU): exported symbols, hash sampler parity with
the oracle, table validation, work counts, and argument/error paths."""

import ctypes
import math
import os
import re
import subprocess

import numpy as np
import pytest

import oracle as orc
from approximate_long_context_amd import plsh

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "plsh.h")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(plsh.LIB_PATH):
        from approximate_long_context_amd import build
        build.build()
    return plsh.lib()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(plsh_[a-z_]+)\s*\(", src)))


def test_library_exports_exactly_the_declared_symbols():
    """The header's functions are exported, and nothing else is: the
    library's dynamic text symbols equal the declarations, both ways."""
    names = _declared()
    assert "plsh_alibi_attention" in names and "plsh_last_error" in names
    L = plsh.lib()
    for nm in names:
        assert hasattr(L, nm), nm
    dyn = subprocess.run(["nm", "-D", "--defined-only", plsh.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = sorted(m.group(1) for m in re.finditer(r"^[0-9a-f]+ T (\S+)$", dyn, flags=re.M))
    assert exported == names
    assert sorted(plsh.EXPORTED) == names


@pytest.mark.parametrize("seed,n,sigma,s", [
    (0, 512, [16.0], 8),
    (0, 4096, [2.0 ** h for h in range(1, 9)], 16),
    (7, 1, [3.0], 4),
    (7, 2, [1e-3, 1e12], 3),
    (123456789, 3001, [1e-3, 0.7, 1.19, 4.0, 64.0, 1e12], 11),
    (2 ** 64 - 1, 700, [256.0, 2.0], 53),
])
def test_sampler_bit_exact_with_oracle(seed, n, sigma, s):
    """Methodology §1-§2: (delta, u) draws and block starts agree bit for bit
    with the oracle's own SplitMix64 draws and full position scan."""
    t = plsh.sample_tables(seed, n, sigma, s)
    p = orc.sample_params(seed, sigma, s)
    assert np.array_equal(t.params, p)
    off, st = orc.tables_from_params(n, p)
    assert np.array_equal(t.offsets.astype(np.int64), off)
    assert np.array_equal(t.starts.astype(np.int64), st)
    plsh.validate_tables(t)


def test_sample_k_independent_of_s():
    a = plsh.sample_tables(5, 300, [8.0, 9.0], 4)
    b = plsh.sample_tables(5, 300, [8.0, 9.0], 9)
    for h in range(2):
        assert np.array_equal(a.params[h * 4:(h + 1) * 4], b.params[h * 9:h * 9 + 4])


def test_two_call_protocol_and_capacity():
    L = plsh.lib()
    sig = np.array([4.0])
    params = np.empty((2, 2))
    offsets = np.empty(3, dtype=np.int32)
    need = ctypes.c_int64(0)
    st = L.plsh_sample_tables(1, 100, 1, sig.ctypes.data, 2, params.ctypes.data, offsets.ctypes.data,
                              None, 0, ctypes.byref(need))
    assert st == plsh.PLSH_OK and need.value == offsets[-1]
    small = np.empty(need.value - 1, dtype=np.int32)
    st = L.plsh_sample_tables(1, 100, 1, sig.ctypes.data, 2, params.ctypes.data, offsets.ctypes.data,
                              small.ctypes.data, small.size, ctypes.byref(need))
    assert st == plsh.PLSH_ERR_CAPACITY and b"capacity" in L.plsh_last_error()


@pytest.mark.parametrize("bad", [float("nan"), 0.0, -1.0, float("inf"), 1e308, 1e-310, 5e300, 1e-285])
def test_sampler_rejects_bad_sigma(bad):
    """Scales outside [1e-280, 1e300] could draw an infinite or subnormal
    pitch: refused (an infinite pitch once sent the scan into a loop)."""
    with pytest.raises(plsh.PlshError) as e:
        plsh.sample_tables(0, 10, [1.0, bad], 2)
    assert e.value.status == plsh.PLSH_ERR_ARG


def test_sampler_accepts_the_range_ends():
    t = plsh.sample_tables(3, 50, [1e-280, 1e300], 4)
    assert np.all(np.isfinite(t.params)) and np.all(t.params[:, 0] > 0)
    plsh.validate_tables(t)


def test_sampler_rejects_bad_sizes():
    for n, s in [(0, 2), (5, 0), (-3, 1)]:
        with pytest.raises(plsh.PlshError) as e:
            plsh.sample_tables(0, n, [1.0], s)
        assert e.value.status == plsh.PLSH_ERR_ARG


def _corrupt(t, fn):
    t2 = plsh.Tables(t.n, t.heads, t.s, t.params.copy(), t.offsets.copy(), t.starts.copy())
    fn(t2)
    return t2


@pytest.mark.parametrize("name,fn", [
    ("first_not_zero", lambda t: t.starts.__setitem__(0, 1)),
    ("last_not_n", lambda t: t.starts.__setitem__(t.offsets[1] - 1, t.n - 1)),
    ("not_increasing", lambda t: t.starts.__setitem__(2, t.starts[1])),
    ("moved_boundary", lambda t: t.starts.__setitem__(1, t.starts[1] + 1)),
    ("u_out_of_range", lambda t: t.params.__setitem__((0, 1), t.params[0, 0] * 1.5)),
    ("delta_nan", lambda t: t.params.__setitem__((1, 0), float("nan"))),
    ("offsets_start", lambda t: t.offsets.__setitem__(0, 1)),
])
def test_validate_rejects_malformed_tables(name, fn):
    t = plsh.sample_tables(3, 200, [6.0, 20.0], 3)
    plsh.validate_tables(t)
    with pytest.raises(plsh.PlshError) as e:
        plsh.validate_tables(_corrupt(t, fn))
    assert e.value.status == plsh.PLSH_ERR_TABLE


@pytest.mark.parametrize("causal", [False, True])
def test_count_work_matches_oracle(causal):
    n, sig, s = 1500, [1.19, 7.0, 64.0, 256.0], 12
    t = plsh.sample_tables(9, n, sig, s)
    tabs = orc.starts_per_head(t.offsets, t.starts, len(sig), s)
    assert plsh.count_work(t, causal) == orc.work_counts(n, tabs, causal)


def _attn_args(**over):
    """Arguments for plsh_alibi_attention with dummy (never dereferenced) pointers."""
    L = plsh.lib()
    sig = np.array([2.0, 4.0, 8.0, 16.0])
    params = np.zeros((4 * 3, 2))
    tb = plsh._Tables(64, 4, 3, params.ctypes.data, None, None)
    a = dict(q=0x10000, k=0x20000, v=0x30000, out=0x40000, batch=1, n=64, heads=4, kv_heads=2,
             d=64, dtype=plsh.PLSH_BF16, sigma=sig.ctypes.data, s=3, tables=ctypes.byref(tb),
             causal=1, stream=None)
    a.update(over)
    keep = (sig, params, tb)
    return L, a, keep


def _call(**over):
    L, a, keep = _attn_args(**over)
    st = L.plsh_alibi_attention(a["q"], a["k"], a["v"], a["out"], a["batch"], a["n"], a["heads"],
                                a["kv_heads"], a["d"], a["dtype"], a["sigma"], a["s"], a["tables"],
                                a["causal"], a["stream"])
    return st, L.plsh_last_error().decode()


@pytest.mark.parametrize("over,status", [
    (dict(q=None), plsh.PLSH_ERR_ARG),
    (dict(n=0), plsh.PLSH_ERR_ARG),
    (dict(kv_heads=3), plsh.PLSH_ERR_ARG),
    (dict(s=0), plsh.PLSH_ERR_ARG),
    (dict(d=96), plsh.PLSH_ERR_UNSUPPORTED),
    (dict(s=300), plsh.PLSH_ERR_UNSUPPORTED),
    (dict(n=1 << 30), plsh.PLSH_ERR_UNSUPPORTED),
    (dict(dtype=7), plsh.PLSH_ERR_UNSUPPORTED),
    (dict(out=0x10000 + 64), plsh.PLSH_ERR_ARG),
    (dict(q=0x10004), plsh.PLSH_ERR_ARG),
])
def test_attention_argument_errors(over, status):
    st, msg = _call(**over)
    assert st == status, msg
    assert msg


def test_attention_rejects_n_beyond_32bit_row_offsets():
    """bf16 reaches a head's K/V rows through 32-bit byte offsets up to the
    end of the last 32-row tile; an n within 31 rows of that limit is refused
    before any device work, although the tensor is under 2^31 elements."""
    n = (1 << 24) - 1  # n * 128 < 2^31, (n + 31) * 128 * 2 > 2^32
    st, msg = _call(n=n, heads=1, kv_heads=1, d=128)
    assert st == plsh.PLSH_ERR_UNSUPPORTED and "too long" in msg, msg
    st, msg = _call(n=n, heads=1, kv_heads=1, d=128, dtype=plsh.PLSH_F32)
    assert st != plsh.PLSH_ERR_UNSUPPORTED, msg


def test_attention_table_mismatch():
    L, a, keep = _attn_args()
    sig, params, _ = keep
    tb = plsh._Tables(65, 4, 3, params.ctypes.data, None, None)
    st = L.plsh_alibi_attention(a["q"], a["k"], a["v"], a["out"], 1, 64, 4, 2, 64, plsh.PLSH_BF16,
                                sig.ctypes.data, 3, ctypes.byref(tb), 1, None)
    assert st == plsh.PLSH_ERR_TABLE


def test_attention_rejects_bad_sigma():
    L, a, keep = _attn_args()
    bad = np.array([2.0, float("nan"), 8.0, 16.0])
    st = L.plsh_alibi_attention(a["q"], a["k"], a["v"], a["out"], 1, 64, 4, 2, 64, plsh.PLSH_BF16,
                                bad.ctypes.data, 3, a["tables"], 1, None)
    assert st == plsh.PLSH_ERR_ARG


def test_attention_without_device_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st, msg = _call()
    assert st == plsh.PLSH_ERR_HIP, msg


def test_workspace_size_formula():
    """Records of the pre-pass: heads * ceil(n/32) records of 16 + 16 E + 1024
    bytes, E = s + 16 rounded up to even; none for fp32."""
    for n, heads, s in ((1, 1, 1), (512, 1, 8), (16384, 32, 20), (8193, 16, 124), (100, 3, 7), (100, 2, 125),
                        (700, 3, 255)):
        e = (s + 16 + 1) & ~1
        want = heads * ((n + 31) // 32) * (16 + 16 * e + 1024)
        assert plsh.workspace_size(n, heads, s, torch_dtype("bf16")) == want
        assert plsh.workspace_size(n, heads, s, torch_dtype("f32")) == 0
    nb = ctypes.c_int64(-1)
    L = plsh.lib()
    assert L.plsh_attention_workspace_size(0, 1, 1, plsh.PLSH_BF16, ctypes.byref(nb)) == plsh.PLSH_ERR_ARG
    assert L.plsh_attention_workspace_size(4, 1, 1, 9, ctypes.byref(nb)) == plsh.PLSH_ERR_UNSUPPORTED
    assert L.plsh_attention_workspace_size(4, 1, 1, plsh.PLSH_BF16, None) == plsh.PLSH_ERR_ARG


def torch_dtype(name):
    import torch
    return torch.bfloat16 if name == "bf16" else torch.float32


def _call_ws(ws, ws_bytes, **over):
    L, a, keep = _attn_args(**over)
    st = L.plsh_alibi_attention_ws(a["q"], a["k"], a["v"], a["out"], a["batch"], a["n"], a["heads"],
                                   a["kv_heads"], a["d"], a["dtype"], a["sigma"], a["s"], a["tables"],
                                   a["causal"], ws, ws_bytes, a["stream"])
    return st, L.plsh_last_error().decode()


def test_attention_ws_argument_errors():
    """The caller-workspace entry point checks its workspace before any device
    work: too small, null, misaligned, overlapping an operand; then the common
    argument checks as plsh_alibi_attention."""
    need = plsh.workspace_size(64, 4, 3, torch_dtype("bf16"))
    big = 0x4000000
    assert _call_ws(big, need - 1)[0] == plsh.PLSH_ERR_CAPACITY
    assert _call_ws(big, -1)[0] == plsh.PLSH_ERR_CAPACITY
    assert _call_ws(None, need)[0] == plsh.PLSH_ERR_ARG
    assert _call_ws(big + 8, need)[0] == plsh.PLSH_ERR_ARG
    L, a, keep = _attn_args()
    assert _call_ws(a["v"], need)[0] == plsh.PLSH_ERR_ARG   # overlaps v
    assert _call_ws(big, need, d=96)[0] == plsh.PLSH_ERR_UNSUPPORTED
    assert _call_ws(big, need, n=0)[0] == plsh.PLSH_ERR_ARG
    # fp32 needs no workspace: a null one of size 0 passes the checks
    import torch
    if not torch.cuda.is_available():
        st, msg = _call_ws(None, 0, dtype=plsh.PLSH_F32)
        assert st == plsh.PLSH_ERR_HIP, msg
        st, msg = _call_ws(big, need)
        assert st == plsh.PLSH_ERR_HIP, msg


def test_noalloc_argument_errors_before_any_device_work():
    """The allocation-free entry point: records beyond its 64 MiB static
    scratch are refused (PLSH_ERR_CAPACITY) before any device access, and
    the common argument checks apply; without a device it reports
    PLSH_ERR_HIP."""
    import torch
    L, a, keep = _attn_args()

    def call(**over):
        L2, b, keep2 = _attn_args(**over)
        st = L2.plsh_alibi_attention_noalloc(b["q"], b["k"], b["v"], b["out"], b["batch"], b["n"], b["heads"],
                                             b["kv_heads"], b["d"], b["dtype"], b["sigma"], b["s"], b["tables"],
                                             b["causal"], b["stream"])
        return st, L2.plsh_last_error().decode()

    assert call(q=None)[0] == plsh.PLSH_ERR_ARG
    assert call(d=96)[0] == plsh.PLSH_ERR_UNSUPPORTED
    # 8 heads, n = 131072, s = 48: 8 * 4096 * 2064 bytes of records > 64 MiB
    n, heads, s = 131072, 8, 48
    sig = np.full(heads, 64.0)
    params = np.zeros((heads * s, 2))
    tb = plsh._Tables(n, heads, s, params.ctypes.data, None, None)
    st = L.plsh_alibi_attention_noalloc(0x10000, 0x20000, 0x30000, 0x40000000, 1, n, heads, heads, 128,
                                        plsh.PLSH_BF16, sig.ctypes.data, s, ctypes.byref(tb), 1, None)
    assert st == plsh.PLSH_ERR_CAPACITY, L.plsh_last_error()
    assert b"scratch" in L.plsh_last_error()
    assert plsh.workspace_size(n, heads, s, torch.bfloat16) > (64 << 20)
    if not torch.cuda.is_available():
        assert call()[0] == plsh.PLSH_ERR_HIP


def test_records_entry_points_argument_errors_before_any_device_work():
    """plsh_alibi_records and plsh_alibi_attention_from_records refuse, before
    any device work: null tables or workspace, a misaligned workspace, one
    smaller than the records (PLSH_ERR_CAPACITY), s above 255, fp32 on the
    records path (PLSH_ERR_UNSUPPORTED), a workspace overlapping out; without
    a device the checked calls report PLSH_ERR_HIP."""
    import torch
    L, a, keep = _attn_args()
    need = plsh.workspace_size(64, 4, 3, torch.bfloat16)
    ws = 0x8000000

    def rec(tables=a["tables"], w=ws, nbytes=need):
        st = L.plsh_alibi_records(tables, 1, w, nbytes, None)
        return st, L.plsh_last_error().decode()

    def fwd(w=ws, nbytes=need, **over):
        b = dict(a, **over)
        st = L.plsh_alibi_attention_from_records(b["q"], b["k"], b["v"], b["out"], b["batch"], b["n"], b["heads"],
                                                 b["kv_heads"], b["d"], b["dtype"], b["sigma"], b["s"],
                                                 b["tables"], b["causal"], w, nbytes, None)
        return st, L.plsh_last_error().decode()

    assert rec(tables=None)[0] == plsh.PLSH_ERR_ARG
    assert rec(w=None)[0] == plsh.PLSH_ERR_ARG
    assert rec(w=ws + 8)[0] == plsh.PLSH_ERR_ARG
    st, msg = rec(nbytes=need - 16)
    assert st == plsh.PLSH_ERR_CAPACITY and "records need" in msg
    params = np.zeros((4 * 300, 2))
    big_s = plsh._Tables(64, 4, 300, params.ctypes.data, None, None)
    assert rec(tables=ctypes.byref(big_s))[0] == plsh.PLSH_ERR_UNSUPPORTED
    zero_n = plsh._Tables(0, 4, 3, params.ctypes.data, None, None)
    assert rec(tables=ctypes.byref(zero_n))[0] == plsh.PLSH_ERR_TABLE

    assert fwd(q=None)[0] == plsh.PLSH_ERR_ARG
    assert fwd(w=None)[0] == plsh.PLSH_ERR_ARG
    assert fwd(w=ws + 8)[0] == plsh.PLSH_ERR_ARG
    assert fwd(nbytes=need - 16)[0] == plsh.PLSH_ERR_CAPACITY
    assert fwd(dtype=plsh.PLSH_F32)[0] == plsh.PLSH_ERR_UNSUPPORTED
    assert fwd(w=a["out"])[0] == plsh.PLSH_ERR_ARG  # the records would overlap out
    if not torch.cuda.is_available():
        assert rec()[0] == plsh.PLSH_ERR_HIP
        assert fwd()[0] == plsh.PLSH_ERR_HIP


def test_lse_and_saved_backward_argument_errors():
    """plsh_alibi_attention_lse and plsh_alibi_attention_backward_saved check
    their extra operands before any device work: null or misaligned lse2 /
    out, fp32 (the MFMA path only); without a device the checks pass and the
    call reports PLSH_ERR_HIP."""
    import torch
    L, a, keep = _attn_args()
    big = 0x4000000

    def lse(lse2, ws=None, ws_bytes=0, **over):
        b = dict(a, **over)
        return L.plsh_alibi_attention_lse(b["q"], b["k"], b["v"], b["out"], b["batch"], b["n"], b["heads"],
                                          b["kv_heads"], b["d"], b["dtype"], b["sigma"], b["s"], b["tables"],
                                          b["causal"], lse2, ws, ws_bytes, b["stream"])

    def saved(out, lse2, **over):
        b = dict(a, **over)
        return L.plsh_alibi_attention_backward_saved(b["q"], b["k"], b["v"], out, lse2, 0x50000, 0x60000,
                                                     0x70000, 0x80000, b["batch"], b["n"], b["heads"],
                                                     b["kv_heads"], b["d"], b["dtype"], b["sigma"], b["s"],
                                                     b["tables"], b["causal"], b["stream"])
    assert lse(None) == plsh.PLSH_ERR_ARG
    assert lse(big + 4) == plsh.PLSH_ERR_ARG
    assert lse(a["q"]) == plsh.PLSH_ERR_ARG             # overlaps q
    assert lse(big, dtype=plsh.PLSH_F32) == plsh.PLSH_ERR_UNSUPPORTED
    need = plsh.workspace_size(64, 4, 3, torch.bfloat16)
    assert lse(big, big + 0x100000, need - 1) == plsh.PLSH_ERR_CAPACITY
    assert lse(big, big + 0x100008, need) == plsh.PLSH_ERR_ARG     # misaligned
    assert lse(big, a["v"], need) == plsh.PLSH_ERR_ARG            # overlaps v
    assert saved(None, big) == plsh.PLSH_ERR_ARG
    assert saved(big, None) == plsh.PLSH_ERR_ARG
    assert saved(big + 8, big + 0x100000) == plsh.PLSH_ERR_ARG
    assert saved(0x60000, big) == plsh.PLSH_ERR_ARG     # dq overlaps out
    assert saved(big, big + 0x100000, dtype=plsh.PLSH_F32) == plsh.PLSH_ERR_UNSUPPORTED
    if not torch.cuda.is_available():
        assert lse(big) == plsh.PLSH_ERR_HIP
        assert lse(big, big + 0x100000, need) == plsh.PLSH_ERR_HIP
        assert saved(big, big + 0x100000) == plsh.PLSH_ERR_HIP


def test_kernel_timer_without_launches():
    plsh.kernel_timer(True)
    assert plsh.kernel_timer_read() == (0, 0.0)
    plsh.kernel_timer(False)
    assert plsh.kernel_timer_read() == (0, 0.0)


def test_kernel_timer_read_rejects_null_pointers():
    import ctypes
    n = ctypes.c_int32(0)
    assert plsh.lib().plsh_kernel_timer_read(None, None) == plsh.PLSH_ERR_ARG
    assert plsh.lib().plsh_kernel_timer_read(ctypes.byref(n), None) == plsh.PLSH_ERR_ARG


def _exact_call(**over):
    L, a, keep = _attn_args(**over)
    st = L.plsh_exact_alibi_attention(a["q"], a["k"], a["v"], a["out"], a["batch"], a["n"], a["heads"],
                                      a["kv_heads"], a["d"], a["dtype"], a["sigma"], a["causal"],
                                      a["stream"])
    return st, L.plsh_last_error().decode()


@pytest.mark.parametrize("over,status", [
    (dict(q=None), plsh.PLSH_ERR_ARG),
    (dict(sigma=None), plsh.PLSH_ERR_ARG),
    (dict(n=0), plsh.PLSH_ERR_ARG),
    (dict(kv_heads=3), plsh.PLSH_ERR_ARG),
    (dict(d=96), plsh.PLSH_ERR_UNSUPPORTED),
    (dict(dtype=plsh.PLSH_F32), plsh.PLSH_ERR_UNSUPPORTED),
    (dict(n=1 << 30), plsh.PLSH_ERR_UNSUPPORTED),
    (dict(out=0x10000 + 64), plsh.PLSH_ERR_ARG),
    (dict(q=0x10004), plsh.PLSH_ERR_ARG),
])
def test_exact_attention_argument_errors(over, status):
    """plsh_exact_alibi_attention validates like the estimator (no table)."""
    st, msg = _exact_call(**over)
    assert st == status, msg
    assert msg


def test_exact_attention_rejects_bad_sigma_and_needs_a_device():
    import torch
    L, a, keep = _attn_args()
    bad = np.array([2.0, 0.0, 8.0, 16.0])
    st = L.plsh_exact_alibi_attention(a["q"], a["k"], a["v"], a["out"], 1, 64, 4, 2, 64, plsh.PLSH_BF16,
                                      bad.ctypes.data, 1, None)
    assert st == plsh.PLSH_ERR_ARG
    if not torch.cuda.is_available():
        st, msg = _exact_call()
        assert st == plsh.PLSH_ERR_HIP, msg


def test_walk_argument_errors_and_device():
    """plsh_alibi_attention_walk validates as the estimator, bf16 only."""
    import torch
    L, a, keep = _attn_args(dtype=plsh.PLSH_F32)
    args = [a[x] for x in ("q", "k", "v", "out", "batch", "n", "heads", "kv_heads", "d", "dtype", "sigma", "s",
                           "tables", "causal", "stream")]
    assert L.plsh_alibi_attention_walk(*args) == plsh.PLSH_ERR_UNSUPPORTED
    args[9] = plsh.PLSH_BF16
    args[0] = None
    assert L.plsh_alibi_attention_walk(*args) == plsh.PLSH_ERR_ARG
    args[0] = a["q"]
    args[8] = 96
    assert L.plsh_alibi_attention_walk(*args) == plsh.PLSH_ERR_UNSUPPORTED
    args[8] = 64
    if not torch.cuda.is_available():
        assert L.plsh_alibi_attention_walk(*args) == plsh.PLSH_ERR_HIP, L.plsh_last_error()


def _bwd_call(**over):
    L, a, keep = _attn_args(**over)
    b = dict(dout=0x50000, dq=0x60000, dk=0x70000, dv=0x80000)
    b.update({k: v for k, v in over.items() if k in b})
    st = L.plsh_alibi_attention_backward(a["q"], a["k"], a["v"], b["dout"], b["dq"], b["dk"], b["dv"],
                                         a["batch"], a["n"], a["heads"], a["kv_heads"], a["d"], a["dtype"],
                                         a["sigma"], a["s"], a["tables"], a["causal"], a["stream"])
    return st, L.plsh_last_error().decode()


@pytest.mark.parametrize("over,status", [
    (dict(dout=None), plsh.PLSH_ERR_ARG),
    (dict(dq=None), plsh.PLSH_ERR_ARG),
    (dict(dk=None), plsh.PLSH_ERR_ARG),
    (dict(dv=None), plsh.PLSH_ERR_ARG),
    (dict(dk=0x70008), plsh.PLSH_ERR_ARG),
    (dict(dq=0x50000 + 128), plsh.PLSH_ERR_ARG),   # dq overlaps dout
    (dict(dk=0x20000), plsh.PLSH_ERR_ARG),         # dk is k
    (dict(dv=0x70000 + 64), plsh.PLSH_ERR_ARG),    # dv overlaps dk
    (dict(n=0), plsh.PLSH_ERR_ARG),
    (dict(d=96), plsh.PLSH_ERR_UNSUPPORTED),
    (dict(dtype=plsh.PLSH_F32), plsh.PLSH_ERR_UNSUPPORTED),
])
def test_backward_argument_errors(over, status):
    """plsh_alibi_attention_backward rejects bad arguments before any launch
    (q, k, v, dout at 64 KiB steps; each gradient 16 KiB at most here)."""
    st, msg = _bwd_call(**over)
    assert st == status, msg
    assert msg


def test_backward_rejects_more_than_124_samples():
    L, a, keep = _attn_args()
    params = np.zeros((4 * 125, 2))
    tb = plsh._Tables(64, 4, 125, params.ctypes.data, None, None)
    st, msg = _bwd_call(s=125, tables=ctypes.byref(tb))
    assert st == plsh.PLSH_ERR_UNSUPPORTED, msg


def test_backward_without_device_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st, msg = _bwd_call()
    assert st == plsh.PLSH_ERR_HIP, msg


def _sample_dev_call(seed=1, heads=4, sigma=(2.0, 4.0, 8.0, 16.0), s=3, params=0x10000):
    sig = np.ascontiguousarray(sigma, dtype=np.float64)
    L = plsh.lib()
    st = L.plsh_sample_params_device(seed, heads, sig.ctypes.data if sigma is not None else None, s, params, None)
    return st, L.plsh_last_error().decode()


@pytest.mark.parametrize("over,status", [
    (dict(sigma=None), plsh.PLSH_ERR_ARG),
    (dict(params=None), plsh.PLSH_ERR_ARG),
    (dict(heads=0), plsh.PLSH_ERR_ARG),
    (dict(s=0), plsh.PLSH_ERR_ARG),
    (dict(heads=129, sigma=[1.0] * 129), plsh.PLSH_ERR_UNSUPPORTED),
    (dict(s=256), plsh.PLSH_ERR_UNSUPPORTED),
    (dict(sigma=(2.0, float("inf"), 8.0, 16.0)), plsh.PLSH_ERR_ARG),
    (dict(sigma=(2.0, -1.0, 8.0, 16.0)), plsh.PLSH_ERR_ARG),
    (dict(sigma=(2.0, 1e308, 8.0, 16.0)), plsh.PLSH_ERR_ARG),
    (dict(sigma=(2.0, 1e-310, 8.0, 16.0)), plsh.PLSH_ERR_ARG),
    (dict(params=0x10008), plsh.PLSH_ERR_ARG),
])
def test_device_sampler_argument_errors(over, status):
    st, msg = _sample_dev_call(**over)
    assert st == status, msg
    assert msg


def test_device_sampler_without_device_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st, msg = _sample_dev_call()
    assert st == plsh.PLSH_ERR_HIP, msg


@pytest.mark.parametrize("width", [1.0, 7.0, 7.5, 64.0, 1e6])
def test_fixed_block_tables_match_oracle_scan(width):
    """Fixed blocks (pitch w, offset 0) through plsh_build_tables equal the
    oracle's own scan of the same hash; integer w gives starts 0, w, 2w, ..."""
    n = 1000
    t = plsh.fixed_block_tables(n, [width, 2.0 * width], s=3)
    plsh.validate_tables(t)
    off, st = orc.tables_from_params(n, t.params)
    assert np.array_equal(t.offsets, off) and np.array_equal(t.starts, st)
    if float(width).is_integer():
        r0 = t.starts[t.offsets[0]:t.offsets[1]]
        want = np.unique(np.append(np.arange(0, n, int(width)), n))
        assert np.array_equal(r0, want)


def _near_integer_rows():
    """(delta, u) rows whose quotients (x + u) / delta hit integers exactly or
    land within a few ulp of one: integer and dyadic pitches with offsets 0
    and exact fractions, pitches one ulp off an integer or a third, and
    offsets one ulp below delta."""
    rows = []
    for d in (1.0, 2.0, 3.0, 5.0, 0.5, 0.25, 1.5, 2.5, 7.0, 64.0, 0.125, 1.0 / 3.0, 0.1, 6.0,
              10.0 / 3.0):
        for dd in (d, np.nextafter(d, 0.0), np.nextafter(d, np.inf)):
            for u in (0.0, dd / 2.0, dd / 3.0, np.nextafter(dd, 0.0), 2.0 ** -40, dd * 0.75):
                if 0.0 <= u < dd:
                    rows.append((dd, u))
    return np.array(rows, dtype=np.float64)


def test_build_tables_exact_near_integer_quotients():
    """The host scan's bins (a product with the pitch's reciprocal, the
    division taken wherever the product lies within its error bound of an
    integer) equal the oracle's plain floor((x + u) / delta) scan, start for
    start, where the quotient is an exact integer or within ulps of one."""
    params = _near_integer_rows()
    n = 2000
    t = plsh.build_tables(n, 1, len(params), params)
    off, st = orc.tables_from_params(n, t.params)
    assert np.array_equal(t.offsets, off) and np.array_equal(t.starts, st)


def test_build_tables_reproduces_the_sampler():
    t = plsh.sample_tables(11, 3000, [1.19, 16.0, 256.0], 7)
    b = plsh.build_tables(3000, 3, 7, t.params)
    assert np.array_equal(t.offsets, b.offsets) and np.array_equal(t.starts, b.starts)


@pytest.mark.parametrize("row", [(0.0, 0.0), (-1.0, 0.0), (float("nan"), 0.0), (4.0, -0.5), (4.0, 4.0),
                                 (float("inf"), 0.0), (1e-310, 0.0), (2.5e-308, 0.0)])
def test_build_tables_rejects_bad_rows(row):
    params = np.array([[8.0, 1.0], row], dtype=np.float64)
    with pytest.raises(plsh.PlshError) as e:
        plsh.build_tables(100, 1, 2, params)
    assert e.value.status == plsh.PLSH_ERR_ARG


def test_build_tables_capacity_protocol():
    L = plsh.lib()
    params = np.array([[3.0, 0.0]], dtype=np.float64)
    offsets = np.empty(2, dtype=np.int32)
    need = ctypes.c_int64(0)
    assert L.plsh_build_tables(30, 1, 1, params.ctypes.data, offsets.ctypes.data, None, 0,
                               ctypes.byref(need)) == plsh.PLSH_OK
    assert need.value == 11
    small_buf = np.empty(5, dtype=np.int32)
    assert L.plsh_build_tables(30, 1, 1, params.ctypes.data, offsets.ctypes.data, small_buf.ctypes.data, 5,
                               ctypes.byref(need)) == plsh.PLSH_ERR_CAPACITY


# ------------------------------------------------ binding argument checks ---
def _cpu_qkv(n=64, d=64, H=2, Hkv=1):
    import torch
    q = torch.zeros((1, H, n, d), dtype=torch.bfloat16)
    k = torch.zeros((1, Hkv, n, d), dtype=torch.bfloat16)
    return q, k, k.clone()


def test_binding_rejects_host_tables_before_any_call(monkeypatch):
    """A host Tables holds host addresses; the binding refuses it (and CPU
    tensors) before the library is called, so nothing is launched."""
    q, k, v = _cpu_qkv()
    t = plsh.sample_tables(0, 64, [4.0, 8.0], 3)
    real = plsh.lib()
    calls = []

    class Recorder:   # forwards the host-only size query, records anything else
        def __getattr__(self, name):
            if name == "plsh_attention_workspace_size":
                return getattr(real, name)
            return lambda *a: calls.append(name) or 0
    monkeypatch.setattr(plsh, "lib", lambda: Recorder())
    for fn in (plsh.attention, plsh.attention_library_workspace, plsh.attention_unfused,
               plsh.attention_walk, plsh.attention_reference, plsh.attention_with_lse):
        with pytest.raises(plsh.PlshError) as e:
            fn(q, k, v, [4.0, 8.0], 3, t, causal=True)
        assert "CUDA" in str(e.value) or "DeviceTables" in str(e.value)
    with pytest.raises(plsh.PlshError):
        plsh.attention_backward(q, k, v, q.clone(), [4.0, 8.0], 3, t, causal=True)
    with pytest.raises(plsh.PlshError):
        plsh.exact_alibi_attention(q, k, v, [4.0, 8.0])
    with pytest.raises(plsh.PlshError):
        plsh.debug_block_intervals(t)
    with pytest.raises(plsh.PlshError):
        plsh.sample_params_device(0, [4.0], 3, "cpu")
    assert calls == []


def test_binding_tables_check():
    """_require_device_tables: a host Tables, params of the wrong dtype,
    shape or device are refused."""
    import torch
    t = plsh.sample_tables(0, 64, [4.0, 8.0], 3)
    with pytest.raises(plsh.PlshError, match="DeviceTables"):
        plsh._require_device_tables(t, torch.device("cpu"))
    dt = t.to("cpu")   # a DeviceTables whose tensors happen to be on the CPU
    plsh._require_device_tables(dt, torch.device("cpu"))
    bad = plsh.DeviceTables(dt.n, dt.heads, dt.s, dt.params.float(), dt.offsets, dt.starts)
    with pytest.raises(plsh.PlshError, match="float64"):
        plsh._require_device_tables(bad, torch.device("cpu"))
    bad = plsh.DeviceTables(dt.n, dt.heads, dt.s, dt.params[:-1], dt.offsets, dt.starts)
    with pytest.raises(plsh.PlshError):
        plsh._require_device_tables(bad, torch.device("cpu"))
    with pytest.raises(plsh.PlshError):
        plsh._require_device_tables(dt, torch.device("cuda", 0))
