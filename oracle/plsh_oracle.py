"""Plain, slow fp64 CPU oracle for Positional-LSH ALiBi attention.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  Shares no code with
the HIP library or its binding.

Source: "Positional LSH: Binary Block Matrix Approximation for Attention with
Linear Biases" (Wolfson & Wagner), technical-summary pages.  Sections cited:
  Methodology §1  -- Positional LSH framework: L*_ij = exp(-|i-j|/sigma) is a
                     Laplacian kernel on token positions; random binning
                     (Rahimi-Recht) hashes integer positions into contiguous
                     bins; L* = E_h[M(h)].
  Methodology §2  -- Theorem 2.1: M~ = (1/s) sum_k M(h_k); spectral/max-norm
                     bounds; b_max ~ sigma log log n; Gamma law behind the bins.
  Methodology §3  -- Theorem 2.2: reduction of ALiBi attention to s randomized
                     short-context attentions without positional bias; output
                     error bounded by bias error over minimum biased row sum.
  Key results     -- O(1/sqrt(s)) decay; convergence of ||L*-M~||, ||T*-T~||.

Readings of what the pages leave open (each is listed in the design notes):
  * bin(x) = floor((x + u) / delta) in IEEE fp64 (add, then divide, then
    floor); pitch delta ~ Gamma(shape 2, scale sigma), offset u ~ U[0, delta).
  * random draws: SplitMix64 (Steele, Lea & Flood 2014), used as a counter-
    based generator: draw #i of a stream keyed by `seed` is the SplitMix64
    output function applied to seed + (i + 1) * 0x9E3779B97F4A7C15.
  * estimator: ratio of sums, T~ = D~^-1 (A o M~ o C) V with
    D~ = diag((A o M~ o C) 1), A = exp(Q K^T), C = causal mask (optional).
  * causal masking applies inside each block (M(h) o C).
  * logits are q.k with scale 1 (inputs arrive pre-scaled).

Parity status per function:
  sample_params            pinned (law: quadrature + KS; exact bit-match
                           against the host sampler is a product check)
  series_ln                pinned (math.log to 1 ulp over every exponent the
                           draws reach; exact at 1 and powers of two)
  bins / tables_from_params pinned (collision probability, structure)
  exact_alibi              pinned (library attention with additive bias;
                           sigma -> inf limit)
  lsh_estimate             pinned (brute force n <= 64, sigma limits, s = 1,
                           error-bound inequality, convex hull)
  lsh_estimate_multiplicity pinned (brute force)
  lsh_row_log_normaliser   pinned (brute-force row sums of A o (sum_k M) o C)
  mask_mean / matrix_errors pinned (variance identity, 1/sqrt(s) slope,
                           hand-worked spectral / max / Frobenius norms)
  work_counts              pinned (brute-force pair enumeration)
  lsh_estimate_grad /      pinned (central finite differences of the
  lsh_grad_rows /          block-walk lsh_estimate; subsets against the
  lsh_grad_keys            dense gradient)
"""

from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "splitmix64",
    "unit_open",
    "unit_halfopen",
    "sample_params",
    "series_ln",
    "bins",
    "block_starts",
    "tables_from_params",
    "starts_per_head",
    "block_intervals",
    "exact_alibi",
    "lsh_estimate",
    "lsh_estimate_multiplicity",
    "lsh_row_log_normaliser",
    "multiplicity_dense",
    "alibi_matrix",
    "mask_dense",
    "mask_mean",
    "matrix_errors",
    "work_counts",
    "lsh_estimate_grad",
    "lsh_grad_rows",
    "lsh_grad_keys",
]

# --------------------------------------------------------------------------
# Counter-based random draws (SplitMix64 output function, published form).
# --------------------------------------------------------------------------
_M64 = (1 << 64) - 1
_GOLDEN = 0x9E3779B97F4A7C15


def splitmix64(seed: int, index: int) -> int:
    """Draw #index of the SplitMix64 stream started at state `seed`."""
    z = (seed + (index + 1) * _GOLDEN) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def unit_open(z: int) -> float:
    """Top 53 bits mapped to the open interval (0, 1)."""
    return ((z >> 11) + 0.5) * (2.0 ** -53)


def unit_halfopen(z: int) -> float:
    """Top 53 bits mapped to [0, 1)."""
    return (z >> 11) * (2.0 ** -53)


def _draw_index(head: int, sample: int, draw: int) -> int:
    # one stream position per (head, sample, draw); independent of s so that
    # raising s only appends samples
    return ((head << 32) | sample) * 4 + draw


# Natural log for the draws.  The pages fix the law of the pitch (Gamma(2,
# sigma)) but no way of computing it; the draws use a logarithm made of IEEE
# double +, -, *, / alone, so that any implementation taking the same steps
# (host or device) draws the same bits: x = m 2^e with m in [sqrt(1/2),
# sqrt(2)) (exact), f = (m - 1) / (m + 1), ln m = 2 atanh f = 2 f (1 + f^2 p)
# with p = 1/3 + f^2/5 + ... + f^22/25 summed by Horner from the last term,
# and ln x = (e ln2_hi + ln m) + e ln2_lo.  |f| <= 0.172, so the first
# omitted term is below 2^-60 of ln m.
_LN2_HI = float.fromhex("0x1.62e42ff000000p-1")     # ln 2 to 32 significant bits
_LN2_LO = float.fromhex("-0x1.718432a1b0e26p-35")   # ln 2 - _LN2_HI, rounded
_SQRT2 = float.fromhex("0x1.6a09e667f3bcdp+0")      # sqrt(2), rounded


def series_ln(x: float) -> float:
    """ln x for finite x > 0 (normal), by the atanh series above."""
    m, e = math.frexp(x)           # x = m 2^e, m in [1/2, 1)
    m, e = m * 2.0, e - 1          # m in [1, 2)
    if m >= _SQRT2:
        m, e = m * 0.5, e + 1      # m in [sqrt(1/2), sqrt(2))
    f = (m - 1.0) / (m + 1.0)
    f2 = f * f
    p = 1.0 / 25.0
    for k in range(11, 0, -1):
        p = 1.0 / (2 * k + 1) + f2 * p
    lnm = 2.0 * f + (2.0 * f) * (f2 * p)
    return (e * _LN2_HI + lnm) + e * _LN2_LO


def sample_params(seed: int, sigma: Sequence[float], s: int) -> np.ndarray:
    """Random-binning hash parameters (delta, u) for every (head, sample).

    Methodology §1 (random binning features on positions) and §2 (Gamma law
    of the bins): pitch delta ~ Gamma(2, sigma) drawn as the sum of two
    exponentials, delta = -sigma (ln U1 + ln U2); offset u = delta * U3 with
    U3 ~ U[0, 1); ln is series_ln.  Returns float64 [heads * s, 2], row
    h * s + k.
    """
    heads = len(sigma)
    out = np.empty((heads * s, 2), dtype=np.float64)
    for h in range(heads):
        sg = float(sigma[h])
        for k in range(s):
            u1 = unit_open(splitmix64(seed, _draw_index(h, k, 0)))
            u2 = unit_open(splitmix64(seed, _draw_index(h, k, 1)))
            u3 = unit_halfopen(splitmix64(seed, _draw_index(h, k, 2)))
            delta = -sg * (series_ln(u1) + series_ln(u2))
            out[h * s + k, 0] = delta
            out[h * s + k, 1] = delta * u3
    return out


# --------------------------------------------------------------------------
# Blocks (Methodology §1: h partitions positions into contiguous bins).
# --------------------------------------------------------------------------
def bins(n: int, delta: float, u: float) -> np.ndarray:
    """bin(x) = floor((x + u) / delta) for x = 0..n-1 (fp64, kept as float)."""
    x = np.arange(n, dtype=np.float64)
    return np.floor((x + u) / delta)


def block_starts(n: int, delta: float, u: float) -> np.ndarray:
    """Block starts of one hash by a full scan: 0, every x whose bin differs
    from that of x-1, and finally n.  int64."""
    b = bins(n, delta, u)
    inner = np.nonzero(b[1:] != b[:-1])[0] + 1
    return np.concatenate([[0], inner, [n]]).astype(np.int64)


def tables_from_params(n: int, params: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """CSR boundary table (offsets, starts) derived by scanning every position
    of every (head, sample) row of `params`."""
    rows = []
    for r in range(params.shape[0]):
        rows.append(block_starts(n, float(params[r, 0]), float(params[r, 1])))
    offsets = np.zeros(len(rows) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum([len(x) for x in rows])
    return offsets, np.concatenate(rows)


def starts_per_head(offsets: np.ndarray, starts: np.ndarray, heads: int,
                    s: int) -> List[List[np.ndarray]]:
    """Split a CSR table into [head][sample] -> starts array."""
    out = []
    for h in range(heads):
        row = []
        for k in range(s):
            r = h * s + k
            row.append(np.asarray(starts[offsets[r]:offsets[r + 1]], dtype=np.int64))
        out.append(row)
    return out


def block_intervals(n: int, starts: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """[lo(x), hi(x)) of the block containing x, for x = 0..n-1."""
    x = np.arange(n)
    idx = np.searchsorted(starts, x, side="right") - 1
    return starts[idx], starts[idx + 1]


# --------------------------------------------------------------------------
# O1: exact ALiBi attention (Methodology §1: bias as Laplacian kernel).
# --------------------------------------------------------------------------
def _kv_head(h: int, heads: int, kv_heads: int) -> int:
    return h // (heads // kv_heads)


def exact_alibi(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                sigma: Sequence[float], causal: bool,
                rows: Optional[np.ndarray] = None,
                chunk: int = 256) -> np.ndarray:
    """T*_i = sum_j exp(q_i.k_j - |i-j|/sigma) v_j / sum_j exp(...), over
    j <= i when causal.  q [B,H,n,d], k/v [B,Hkv,n,d], fp64.  `rows`
    restricts the output to the given query rows (same for every (b,h));
    returns [B,H,len(rows) or n,d]."""
    B, H, n, d = q.shape
    Hkv = k.shape[1]
    rws = np.arange(n) if rows is None else np.asarray(rows)
    out = np.empty((B, H, len(rws), d), dtype=np.float64)
    j = np.arange(n)
    for b in range(B):
        for h in range(H):
            g = _kv_head(h, H, Hkv)
            kk, vv = k[b, g], v[b, g]
            for c0 in range(0, len(rws), chunk):
                ri = rws[c0:c0 + chunk]
                logits = q[b, h, ri] @ kk.T - np.abs(ri[:, None] - j[None, :]) / float(sigma[h])
                if causal:
                    logits = np.where(j[None, :] <= ri[:, None], logits, -np.inf)
                mx = logits.max(axis=1, keepdims=True)
                w = np.exp(logits - mx)
                out[b, h, c0:c0 + len(ri)] = (w @ vv) / w.sum(axis=1, keepdims=True)
    return out


# --------------------------------------------------------------------------
# O3: the LSH estimate (Methodology §2 Thm 2.1 mask mean; §3 Thm 2.2
# reduction to s short-context attentions, combined as a ratio of sums).
# --------------------------------------------------------------------------
def _block_stats_full(qh, kh, vh, starts, causal, max_elems=1 << 24):
    """For one hash: per-row (mu, Z, N) of plain attention restricted to the
    row's block (and to j <= i when causal).  Blocks of equal length are
    stacked into batched matmuls."""
    n, d = qh.shape
    mu = np.empty(n)
    Z = np.empty(n)
    N = np.empty((n, d))
    lens = np.diff(starts)
    for L in np.unique(lens):
        L = int(L)
        b0_all = starts[:-1][lens == L]
        step = max(1, max_elems // (L * L))
        tri = np.tril(np.ones((L, L), dtype=bool)) if causal else None
        for c0 in range(0, len(b0_all), step):
            b0 = b0_all[c0:c0 + step]
            pos = b0[:, None] + np.arange(L)[None, :]
            Sb = qh[pos] @ np.swapaxes(kh[pos], 1, 2)          # [nb, L, L]
            if causal:
                Sb = np.where(tri[None], Sb, -np.inf)
            m = Sb.max(axis=2)
            E = np.exp(Sb - m[:, :, None])
            flat = pos.reshape(-1)
            mu[flat] = m.reshape(-1)
            Z[flat] = E.sum(axis=2).reshape(-1)
            N[flat] = (E @ vh[pos]).reshape(-1, d)
    return mu, Z, N


def _block_stats_rows(qh, kh, vh, starts, causal, rows):
    """Same statistics for selected rows only: cost |B(i)| * d per row."""
    d = qh.shape[1]
    idx = np.searchsorted(starts, rows, side="right") - 1
    lo, hi = starts[idx], starts[idx + 1]
    mu = np.empty(len(rows))
    Z = np.empty(len(rows))
    N = np.empty((len(rows), d))
    for r, i in enumerate(rows):
        top = i + 1 if causal else hi[r]
        lg = kh[lo[r]:top] @ qh[i]
        m = lg.max()
        e = np.exp(lg - m)
        mu[r], Z[r], N[r] = m, e.sum(), e @ vh[lo[r]:top]
    return mu, Z, N


def lsh_estimate(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                 tables: List[List[np.ndarray]], causal: bool,
                 rows: Optional[np.ndarray] = None,
                 return_stats: bool = False):
    """T~ for every (b, h): for each hash k run plain attention (no bias)
    inside every block, keep per-row (mu_k, Z_k, N_k) = (max logit,
    sum exp, sum exp * v), then combine over hashes as a ratio of sums:
    T~_i = sum_k e^{mu_k - mu} N_k / sum_k e^{mu_k - mu} Z_k.
    `tables[h][k]` are block starts (0 ... n).  fp64 throughout."""
    B, H, n, d = q.shape
    Hkv = k.shape[1]
    s = len(tables[0])
    R = n if rows is None else len(rows)
    out = np.empty((B, H, R, d))
    for b in range(B):
        for h in range(H):
            g = _kv_head(h, H, Hkv)
            qh, kh, vh = q[b, h], k[b, g], v[b, g]
            mus = np.empty((s, R))
            Zs = np.empty((s, R))
            Ns = np.empty((s, R, d))
            for kk in range(s):
                st = np.asarray(tables[h][kk], dtype=np.int64)
                if rows is None:
                    mus[kk], Zs[kk], Ns[kk] = _block_stats_full(qh, kh, vh, st, causal)
                else:
                    mus[kk], Zs[kk], Ns[kk] = _block_stats_rows(qh, kh, vh, st, causal,
                                                                np.asarray(rows))
            m = mus.max(axis=0)
            wgt = np.exp(mus - m[None, :])
            out[b, h] = (wgt[:, :, None] * Ns).sum(axis=0) / (wgt * Zs).sum(axis=0)[:, None]
    return out


def lsh_row_log_normaliser(q: np.ndarray, k: np.ndarray, tables: List[List[np.ndarray]],
                           causal: bool, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """ln of each row's normaliser, ln sum_k sum_{j in B_k(i), j in J(i)}
    e^{q_i.k_j}: the diagonal of s D~ with D~ = diag((A o M~ o C) 1)
    (Methodology §3, Theorem 2.2), as [B, H, rows].  Per hash, the block
    maximum mu_k and sum Z_k of the block-walk statistics; over hashes,
    ln sum_k e^{mu_k} Z_k taken as max + ln sum e^{mu_k - max} Z_k."""
    B, H, n, d = q.shape
    Hkv = k.shape[1]
    s = len(tables[0])
    R = n if rows is None else len(rows)
    out = np.empty((B, H, R))
    zero_v = np.zeros((n, d))  # (the value sums are not needed)
    for b in range(B):
        for h in range(H):
            g = _kv_head(h, H, Hkv)
            qh, kh = q[b, h], k[b, g]
            mus = np.empty((s, R))
            Zs = np.empty((s, R))
            for kk in range(s):
                st = np.asarray(tables[h][kk], dtype=np.int64)
                if rows is None:
                    mus[kk], Zs[kk], _ = _block_stats_full(qh, kh, zero_v, st, causal)
                else:
                    mus[kk], Zs[kk], _ = _block_stats_rows(qh, kh, zero_v, st, causal, np.asarray(rows))
            m = mus.max(axis=0)
            out[b, h] = m + np.log((np.exp(mus - m[None, :]) * Zs).sum(axis=0))
    return out


def multiplicity_dense(n: int, starts_list: Sequence[np.ndarray], causal: bool) -> np.ndarray:
    """c_ij = #{k : i and j share a block of hash k} (times the causal mask),
    i.e. s * M~ o C, as an integer matrix.  For small n."""
    c = np.zeros((n, n), dtype=np.int64)
    for st in starts_list:
        c += mask_dense(n, st)
    if causal:
        c = np.tril(c)
    return c


def lsh_estimate_multiplicity(q, k, v, tables, causal):
    """The same estimator summed pair by pair with integer multiplicities:
    T~_i = sum_j c_ij e^{q_i.k_j} v_j / sum_j c_ij e^{q_i.k_j}.  Small n."""
    B, H, n, d = q.shape
    Hkv = k.shape[1]
    out = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            g = _kv_head(h, H, Hkv)
            c = multiplicity_dense(n, tables[h], causal).astype(np.float64)
            lg = q[b, h] @ k[b, g].T
            lg = np.where(c > 0, lg, -np.inf)
            w = c * np.exp(lg - lg.max(axis=1, keepdims=True))
            out[b, h] = (w @ v[b, g]) / w.sum(axis=1, keepdims=True)
    return out


# --------------------------------------------------------------------------
# O4: matrix errors (Methodology §2 Thm 2.1; Key results).
# --------------------------------------------------------------------------
def alibi_matrix(n: int, sigma: float) -> np.ndarray:
    """L*_ij = exp(-|i-j| / sigma)."""
    x = np.arange(n)
    return np.exp(-np.abs(x[:, None] - x[None, :]) / sigma)


def mask_dense(n: int, starts: np.ndarray) -> np.ndarray:
    """M(h)_ij = 1 when i and j fall in the same block of hash h."""
    blk = np.searchsorted(starts, np.arange(n), side="right") - 1
    return (blk[:, None] == blk[None, :]).astype(np.int64)


def mask_mean(n: int, starts_list: Sequence[np.ndarray]) -> np.ndarray:
    """M~ = (1/s) sum_k M(h_k)."""
    acc = np.zeros((n, n))
    for st in starts_list:
        acc += mask_dense(n, st)
    return acc / len(starts_list)


def matrix_errors(Lstar: np.ndarray, Mtilde: np.ndarray) -> dict:
    """max-norm, spectral norm (both matrices are symmetric, so the largest
    |eigenvalue| of the difference) and Frobenius norm of L* - M~."""
    D = Lstar - Mtilde
    ev = np.linalg.eigvalsh(D)
    return {"max": float(np.abs(D).max()),
            "spectral": float(np.abs(ev).max()),
            "fro": float(np.sqrt((D * D).sum()))}


# --------------------------------------------------------------------------
# O5: work counts (Methodology §3 Thm 2.2 cost structure).
# --------------------------------------------------------------------------
def work_counts(n: int, tables: List[List[np.ndarray]], causal: bool) -> Tuple[int, int]:
    """pairs_alg: in-block (i, j) pairs summed over every hash (the literal
    s-short-attention count); pairs_distinct: pairs in the union over hashes,
    counted once (nonzeros of M~ o C).  Per batch element, summed over heads."""
    alg = 0
    distinct = 0
    x = np.arange(n)
    for per_head in tables:
        ulo = np.full(n, n, dtype=np.int64)
        uhi = np.zeros(n, dtype=np.int64)
        for st in per_head:
            L = np.diff(st)
            alg += int((L * (L + 1) // 2).sum()) if causal else int((L * L).sum())
            lo, hi = block_intervals(n, st)
            ulo = np.minimum(ulo, lo)
            uhi = np.maximum(uhi, hi)
        if causal:
            distinct += int((x - ulo + 1).sum())
        else:
            distinct += int((uhi - ulo).sum())
    return alg, distinct


# --------------------------------------------------------------------------
# O6: gradients of the estimate for fixed hash tables (the pages train with
# the method: Experimental Validation).  With P_ij = c_ij e^{q_i.k_j} /
# sum_l c_il e^{q_i.k_l} and T~_i = sum_j P_ij v_j, an upstream gradient dO
# gives (c is a constant of the tables; the softmax Jacobian):
#   dV_j = sum_i P_ij dO_i,   dP_ij = dO_i . v_j,   D_i = sum_j P_ij dP_ij,
#   dS_ij = P_ij (dP_ij - D_i),   dQ_i = sum_j dS_ij k_j,   dK_j = sum_i dS_ij q_i.
# K and V gradients of a GQA group add over the group's query heads.
# --------------------------------------------------------------------------
def lsh_estimate_grad(q, k, v, do, tables, causal):
    """(dq, dk, dv) of sum(do * T~) for every element, dense per head (small n)."""
    B, H, n, d = q.shape
    Hkv = k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            g = _kv_head(h, H, Hkv)
            c = multiplicity_dense(n, tables[h], causal).astype(np.float64)
            lg = q[b, h] @ k[b, g].T
            lg = np.where(c > 0, lg, -np.inf)
            w = c * np.exp(lg - lg.max(axis=1, keepdims=True))
            p = w / w.sum(axis=1, keepdims=True)
            dp = do[b, h] @ v[b, g].T
            dvec = (p * dp).sum(axis=1, keepdims=True)
            ds = p * (dp - dvec)
            dq[b, h] = ds @ k[b, g]
            dk[b, g] += ds.T @ q[b, h]
            dv[b, g] += p.T @ do[b, h]
    return dq, dk, dv


def _row_probs(qi, kh, starts_list, i, n, causal):
    """Keys j with c_ij > 0 of row i and their normalised weights P_ij."""
    lo, hi = n, 0
    ivals = []
    for st in starts_list:
        a, bnd = _interval_of(st, i)
        if causal:
            bnd = min(bnd, i + 1)
        ivals.append((a, bnd))
        lo, hi = min(lo, a), max(hi, bnd)
    js = np.arange(lo, hi)
    c = np.zeros(len(js))
    for a, bnd in ivals:
        c[(js >= a) & (js < bnd)] += 1.0
    lg = kh[js] @ qi
    w = c * np.exp(lg - lg.max())
    return js, w / w.sum()


def _interval_of(starts, x):
    idx = np.searchsorted(starts, x, side="right") - 1
    return int(starts[idx]), int(starts[idx + 1])


def lsh_grad_rows(q, k, v, do, tables, causal, rows):
    """dq at the given query rows ([B, H, len(rows), d]): row-local."""
    B, H, n, d = q.shape
    Hkv = k.shape[1]
    out = np.zeros((B, H, len(rows), d))
    for b in range(B):
        for h in range(H):
            g = _kv_head(h, H, Hkv)
            for r, i in enumerate(rows):
                js, p = _row_probs(q[b, h, i], k[b, g], tables[h], int(i), n, causal)
                dp = v[b, g, js] @ do[b, h, i]
                ds = p * (dp - (p * dp).sum())
                out[b, h, r] = ds @ k[b, g, js]
    return out


def lsh_grad_keys(q, k, v, do, tables, causal, keys):
    """(dk, dv) at the given key positions ([B, Hkv, len(keys), d]).  The rows
    that weigh key j are those sharing a block with j in some hash (the
    same-bin relation is symmetric), i >= j when causal; each needs its own
    normalisation over its blocks."""
    B, H, n, d = q.shape
    Hkv = k.shape[1]
    dk = np.zeros((B, Hkv, len(keys), d))
    dv = np.zeros((B, Hkv, len(keys), d))
    for b in range(B):
        for h in range(H):
            g = _kv_head(h, H, Hkv)
            for r, j in enumerate(keys):
                j = int(j)
                lo, hi = n, 0
                for st in tables[h]:
                    a, bnd = _interval_of(st, j)
                    lo, hi = min(lo, a), max(hi, bnd)
                if causal:
                    lo = j
                for i in range(lo, hi):
                    js, p = _row_probs(q[b, h, i], k[b, g], tables[h], i, n, causal)
                    hit = np.nonzero(js == j)[0]
                    if len(hit) == 0:
                        continue
                    dp = v[b, g, js] @ do[b, h, i]
                    dvec = (p * dp).sum()
                    pij = p[hit[0]]
                    dv[b, g, r] += pij * do[b, h, i]
                    dk[b, g, r] += pij * (dp[hit[0]] - dvec) * q[b, h, i]
    return dk, dv

