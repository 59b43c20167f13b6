"""Pins for the fp64 oracle: checks against facts fixed by the pages and by
mathematics, never against the oracle itself.

Each pin is a function ``pin_xxx(lib)`` that raises AssertionError when the
oracle library ``lib`` violates it.  ``test_oracle_pins.py`` runs them on the
real oracle; ``test_oracle_mutants.py`` runs them on copies of the oracle with
one planted mistake each and requires every copy to fail at least one pin.

What pins what:
* worked example - CS336 Lecture 5 notes (GPUs, TPUs), Exercise 8: online
  softmax over [1, 3 | 2, 5] with printed m and l after each block.
* blocked identities - CS149 Lecture 9 notes (Efficiently Evaluating DNNs on
  GPUs), section 9: m = max of block maxima, l = sum_b e^{m_b - m} l_b.
* streaming and blocked evaluation - what PDC notes Lecture 4, section 4.13.3
  (one key at a time with a running o) and CS149 L9 notes Example 4 (key
  blocks with a per-block max) compute, done here with a vectorised merge of
  partial softmax states folded left to right or as a tree; block sizes that
  do not divide N as CS336 L5 notes Exercise 10 asks.
* brute force - the textbook formula O_i = sum_j e^{s_ij} V_j / sum_j e^{s_ij}
  (no max subtraction) in 50-digit decimal arithmetic.
* closed forms - Q = 0, constant V, causal row 0, N = 1.
* large logits - PDC notes 4.13.2: e^x overflows for x near 1000 unless the
  row maximum is subtracted.
* backward - finite differences of the 50-digit forward; the D identity of
  CS336 L5 notes Exercise 9; sum_j dV_j = sum_i dO_i; sum_j dK_j = 0.
* Nq queries against Nk keys (the last Nq positions, PDC notes Lecture 4
  section 4.9 key/value cache): 50-digit brute force with the shifted causal
  mask, Q = 0 closed form, and the blocked merge of per-chunk (O, lse) pairs
  (CS149 L9 notes section 9) that split-key attention relies on; its backward
  by finite differences of that brute force, the dV / dK sums, the D identity,
  and Nq = Nk against the square backward.
* MXFP8 decoding (CS336 L5 notes section 6.2: E4M3 values, one E8M0 scale
  per 32 elements): every E4M3 code against torch's float8_e4m3fn cast and
  the format's fixed points (1, 448, 2^-6, 2^-9, NaN); E8M0 against its
  definition 2^(e-127); the scale of element c is that of block c / 32.
"""
from __future__ import annotations

import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- helpers
def _rng(seed):
    return np.random.default_rng(seed)


def dec_forward(q, k, v, causal, scale, prec=50):
    """Textbook attention in Decimal: no max subtraction, no blocking.
    Returns (O, lse) as nested lists of Decimal."""
    getcontext().prec = prec
    N, d = len(q), len(q[0])
    sc = Decimal(scale)
    O, lse = [], []
    for i in range(N):
        w = []
        for j in range(N):
            if causal and j > i:
                w.append(Decimal(0))
                continue
            s = sum((q[i][c] * k[j][c] for c in range(d)), Decimal(0)) * sc
            w.append(s.exp())
        Z = sum(w, Decimal(0))
        O.append([sum((w[j] * v[j][c] for j in range(N)), Decimal(0)) / Z for c in range(d)])
        lse.append(Z.ln())
    return O, lse


def dec_forward_rect(q, k, v, causal, scale, prec=50):
    """Textbook attention of len(q) queries at the last positions of a
    len(k)-key sequence, in Decimal: query i sees keys j <= i + Nk - Nq under
    the causal mask.  Returns (O, lse) as nested lists of Decimal."""
    getcontext().prec = prec
    Nq, Nk, d = len(q), len(k), len(q[0])
    sc = Decimal(scale)
    O, lse = [], []
    for i in range(Nq):
        w = []
        for j in range(Nk):
            if causal and j > i + (Nk - Nq):
                w.append(Decimal(0))
                continue
            s = sum((q[i][c] * k[j][c] for c in range(d)), Decimal(0)) * sc
            w.append(s.exp())
        Z = sum(w, Decimal(0))
        O.append([sum((w[j] * v[j][c] for j in range(Nk)), Decimal(0)) / Z for c in range(d)])
        lse.append(Z.ln())
    return O, lse


def _to_dec(a):
    return [[Decimal(float(x)) for x in row] for row in np.asarray(a, dtype=np.float64)]


def _assert_close(a, b, rtol, atol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.abs(a - b)
    bound = atol + rtol * np.abs(b)
    assert np.all(err <= bound), f"{what}: max err {err.max():.3e} (worst excess {(err - bound).max():.3e})"


# ---------------------------------------------------------------- forward pins
def pin_worked_example(lib):
    """CS336 L5 notes Exercise 8, printed values."""
    with open(os.path.join(GOLDEN, "online_softmax_ex8.json")) as f:
        g = json.load(f)
    x = np.array(g["x"])
    # block-by-block online update as the notes state it (section 8.2):
    # m' = max(m, max block), l' = l e^{m - m'} + sum_block e^{x - m'}
    m, l = -math.inf, 0.0
    seen = []
    for lo, hi in g["blocks"]:
        blk = x[lo:hi]
        m_new = max(m, float(blk.max()))
        l = l * math.exp(m - m_new) + float(np.exp(blk - m_new).sum())
        m = m_new
        seen.append((m, l))
    assert seen[0][0] == g["after_block_1"]["m"]
    assert abs(seen[0][1] - g["after_block_1"]["l"]) < 1e-4
    assert seen[1][0] == g["after_block_2"]["m"]
    assert abs(seen[1][1] - g["after_block_2"]["l"]) < 1e-4
    # the oracle's one-shot softmax must land on the printed final state
    p, m1, l1 = oracle.softmax_row(x, lib=lib)
    assert m1 == g["after_block_2"]["m"]
    assert abs(l1 - g["after_block_2"]["l"]) < 1e-4
    assert abs(p[3] - g["softmax_of_x4"]["value"]) < 1e-3
    # and exactly on the online result (same quantity, different order)
    assert abs(l1 - seen[1][1]) < 1e-15 * 2


def pin_blocked_identity(lib):
    """CS149 L9 notes section 9: merging per-block (m_b, l_b, softmax_b)
    reproduces the one-shot softmax, for block splits that do not divide n."""
    rng = _rng(11)
    for n, cuts in [(37, [5, 17, 30]), (64, [1, 2, 40]), (9, [4]), (100, [33, 66, 99])]:
        x = rng.normal(0, 4, n)
        p, m, l = oracle.softmax_row(x, lib=lib)
        edges = [0] + cuts + [n]
        parts = [oracle.softmax_row(x[a:b], lib=lib) for a, b in zip(edges[:-1], edges[1:])]
        m_merged = max(mb for _, mb, _ in parts)
        l_merged = sum(math.exp(mb - m_merged) * lb for _, mb, lb in parts)
        assert m_merged == m
        assert abs(l_merged - l) <= 1e-14 * l
        f = np.concatenate([pb * lb * math.exp(mb - m_merged) for pb, mb, lb in parts])
        _assert_close(f / l_merged, p, 1e-14, 1e-300, "blocked softmax")
        # the plain definition, evaluated directly
        ref = np.exp(x - x.max()) / np.exp(x - x.max()).sum()
        _assert_close(p, ref, 1e-14, 1e-300, "softmax definition")


def _merge_states(a, b):
    """Combine the softmax states of two disjoint key sets, for every query
    row at once: a state is (m, l, o) with m the row maximum of the scores,
    l = sum e^{s - m} and o = sum e^{s - m} v over its keys (CS149 L9 notes
    section 9, the blocked-softmax identity).  m = -inf, l = 0, o = 0 is the
    state of no visible key and leaves the other operand unchanged."""
    ma, la, oa = a
    mb, lb, ob = b
    m = np.maximum(ma, mb)
    base = np.where(np.isfinite(m), m, 0.0)

    def weight(mx):
        return np.where(np.isfinite(mx), np.exp(np.where(np.isfinite(mx), mx, 0.0) - base), 0.0)

    wa, wb = weight(ma), weight(mb)
    return m, la * wa + lb * wb, oa * wa[:, None] + ob * wb[:, None]


def _key_range_state(q, k, v, causal, scale, j0, j1):
    """State (m, l, o) of keys j0 .. j1-1 for every query (query i sees key j
    when j <= i under the causal mask)."""
    s = scale * (q @ k[j0:j1].T)
    if causal:
        s = np.where(np.arange(j0, j1)[None, :] > np.arange(q.shape[0])[:, None], -np.inf, s)
    m = s.max(axis=1)
    base = np.where(np.isfinite(m), m, 0.0)
    p = np.where(np.isfinite(s), np.exp(s - base[:, None]), 0.0)
    return m, p.sum(axis=1), p @ v[j0:j1]


def _attention_by_merging(q, k, v, causal, scale, bk, tree):
    """O and lse from the states of key blocks of bk keys, merged left to
    right (tree=False; bk = 1 is the key-at-a-time online softmax of the PDC
    notes section 4.13.3) or pairwise as a balanced tree (tree=True)."""
    n = k.shape[0]
    states = [_key_range_state(q, k, v, causal, scale, j0, min(n, j0 + bk)) for j0 in range(0, n, bk)]
    if tree:
        while len(states) > 1:
            states = [_merge_states(states[i], states[i + 1]) if i + 1 < len(states) else states[i]
                      for i in range(0, len(states), 2)]
        m, l, o = states[0]
    else:
        m, l, o = states[0]
        for st in states[1:]:
            m, l, o = _merge_states((m, l, o), st)
    return o / l[:, None], m + np.log(l)


def pin_streaming_and_blocked(lib):
    rng = _rng(12)
    for N, d, causal in [(23, 5, False), (23, 5, True), (40, 8, True), (7, 3, False)]:
        q, k, v = rng.normal(size=(3, N, d))
        scale = 1 / math.sqrt(d)
        o, lse = oracle.attn_fwd(q, k, v, causal, scale, lib=lib)
        os_, ls_ = _attention_by_merging(q, k, v, causal, scale, 1, tree=False)
        _assert_close(os_, o, 1e-12, 1e-13, "streaming")
        _assert_close(ls_, lse, 1e-13, 1e-13, "streaming lse")
        for bk in (3, 4, 7, N):
            for tree in (False, True):
                ob, lb = _attention_by_merging(q, k, v, causal, scale, bk, tree)
                _assert_close(ob, o, 1e-12, 1e-13, f"blocked {bk} tree={tree}")
                _assert_close(lb, lse, 1e-13, 1e-13, f"blocked lse {bk} tree={tree}")


def pin_rows_sum_to_one(lib):
    rng = _rng(13)
    for causal in (False, True):
        q, k, v = rng.normal(size=(3, 2, 33, 6))
        o, lse, p = oracle.attn_fwd(q, k, v, causal, 0.4, return_p=True, lib=lib)
        assert np.all(p >= 0)
        _assert_close(p.sum(-1), np.ones((2, 33)), 1e-13, 0, "row sums")
        if causal:
            assert np.all(np.triu(p, 1) == 0), "causal P must vanish above the diagonal"
        # O is P V (definition) and lse = ln sum exp(s)
        _assert_close(o, p @ v, 1e-12, 1e-13, "O = P V")


def pin_constant_v(lib):
    rng = _rng(14)
    for causal in (False, True):
        q, k = rng.normal(size=(2, 29, 7))
        c = rng.normal(size=7)
        v = np.tile(c, (29, 1))
        o, _ = oracle.attn_fwd(q, k, v, causal, 0.3, lib=lib)
        _assert_close(o, np.tile(c, (29, 1)), 1e-13, 1e-13, "constant V")


def pin_q_zero(lib):
    rng = _rng(15)
    N, d = 31, 4
    k, v = rng.normal(size=(2, N, d))
    q = np.zeros((N, d))
    o, lse = oracle.attn_fwd(q, k, v, False, 0.5, lib=lib)
    _assert_close(o, np.tile(v.mean(0), (N, 1)), 1e-13, 1e-13, "Q=0 mean")
    _assert_close(lse, np.full(N, math.log(N)), 1e-14, 0, "Q=0 lse")
    o, lse = oracle.attn_fwd(q, k, v, True, 0.5, lib=lib)
    prefix = np.cumsum(v, axis=0) / np.arange(1, N + 1)[:, None]
    _assert_close(o, prefix, 1e-13, 1e-13, "Q=0 causal prefix mean")
    _assert_close(lse, np.log(np.arange(1, N + 1)), 1e-14, 1e-15, "Q=0 causal lse")


def pin_row0_and_single_key(lib):
    rng = _rng(16)
    q, k, v = rng.normal(size=(3, 12, 5))
    o, lse = oracle.attn_fwd(q, k, v, True, 0.7, lib=lib)
    _assert_close(o[0], v[0], 0, 0, "causal row 0")
    assert abs(lse[0] - 0.7 * float(q[0] @ k[0])) < 1e-14
    o, lse = oracle.attn_fwd(q[:1], k[:1], v[:1], False, 0.7, lib=lib)
    _assert_close(o[0], v[0], 0, 0, "N=1")
    assert abs(lse[0] - 0.7 * float(q[0] @ k[0])) < 1e-14


def pin_brute_force(lib):
    rng = _rng(17)
    for N, d, causal, spread in [(5, 3, False, 1.0), (6, 4, True, 2.0), (4, 2, False, 3.0),
                                 (6, 3, True, 1.0), (1, 4, True, 1.0)]:
        q, k, v = rng.normal(0, spread, size=(3, N, d))
        scale = 1 / math.sqrt(d)
        o, lse = oracle.attn_fwd(q, k, v, causal, scale, lib=lib)
        Od, Ld = dec_forward(_to_dec(q), _to_dec(k), _to_dec(v), causal, scale)
        _assert_close(o, np.array([[float(x) for x in r] for r in Od]), 1e-13, 1e-14, "brute O")
        _assert_close(lse, np.array([float(x) for x in Ld]), 1e-14, 1e-14, "brute lse")


def pin_large_logits(lib):
    """Logits near +-1000 (PDC notes 4.13.2) and the large-logit workload
    regime (Q, K ~ N(0, 9)): finite results equal to 50-digit brute force."""
    rng = _rng(18)
    for N, d, causal, qs in [(6, 4, False, 40.0), (6, 4, True, 40.0), (5, 8, False, 3.0)]:
        q = rng.normal(0, qs, size=(N, d))
        k = rng.normal(0, qs, size=(N, d))
        v = rng.normal(size=(N, d))
        scale = 1 / math.sqrt(d)
        o, lse = oracle.attn_fwd(q, k, v, causal, scale, lib=lib)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
        Od, Ld = dec_forward(_to_dec(q), _to_dec(k), _to_dec(v), causal, scale)
        _assert_close(o, np.array([[float(x) for x in r] for r in Od]), 1e-12, 1e-12, "large O")
        _assert_close(lse, np.array([float(x) for x in Ld]), 1e-14, 1e-12, "large lse")


def pin_rows_entry(lib):
    """The row-sampled entry point returns the head entry point's rows."""
    rng = _rng(19)
    for causal in (False, True):
        q, k, v = rng.normal(size=(3, 50, 6))
        o, lse = oracle.attn_fwd(q, k, v, causal, 0.35, lib=lib)
        rows = np.array([49, 0, 17, 3, 3, 31])
        orow, lrow = oracle.attn_fwd_rows(q, k, v, causal, 0.35, rows, lib=lib)
        _assert_close(orow, o[rows], 0, 0, "rows O")
        _assert_close(lrow, lse[rows], 0, 0, "rows lse")
        _, _, p = oracle.attn_fwd(q, k, v, causal, 0.35, return_p=True, lib=lib)
        _, _, prow = oracle.attn_fwd_rows(q, k, v, causal, 0.35, rows, return_p=True, lib=lib)
        _assert_close(prow, p[rows], 0, 0, "rows P")


# ---------------------------------------------------------------- backward pins
def pin_bwd_finite_differences(lib):
    """Gradient of L = sum(dO * O) by central differences of the 50-digit
    forward (independent of the oracle's forward and backward)."""
    rng = _rng(20)
    h = Decimal("1e-15")
    for N, d, causal in [(4, 3, False), (5, 2, True), (3, 4, True)]:
        q, k, v, do = rng.normal(size=(4, N, d))
        scale = 1 / math.sqrt(d)
        g = oracle.attn_bwd(q, k, v, do, causal, scale, lib=lib)
        base = {"q": _to_dec(q), "k": _to_dec(k), "v": _to_dec(v)}
        dod = _to_dec(do)

        def loss(t):
            O, _ = dec_forward(t["q"], t["k"], t["v"], causal, scale)
            return sum((O[i][c] * dod[i][c] for i in range(N) for c in range(d)), Decimal(0))

        for name in ("q", "k", "v"):
            fd = np.zeros((N, d))
            for i in range(N):
                for c in range(d):
                    t = {n: [row[:] for row in a] for n, a in base.items()}
                    t[name][i][c] = base[name][i][c] + h
                    lp = loss(t)
                    t[name][i][c] = base[name][i][c] - h
                    lm = loss(t)
                    fd[i, c] = float((lp - lm) / (2 * h))
            _assert_close(g["d" + name], fd, 1e-10, 1e-12, f"finite differences d{name}")


def pin_bwd_dq_rows(lib):
    """The row-wise dQ entry point returns the square backward's dQ rows
    (that backward is pinned by finite differences above)."""
    rng = _rng(23)
    for causal in (False, True):
        q, k, v, do = rng.normal(size=(4, 41, 7))
        g = oracle.attn_bwd(q, k, v, do, causal, 0.35, lib=lib)
        rows = np.array([40, 0, 13, 13, 1, 27])
        dq = oracle.attn_bwd_dq_rows(q, k, v, do, causal, 0.35, rows, lib=lib)
        _assert_close(dq, g["dq"][rows], 1e-12, 1e-13, "dq rows")


def pin_bwd_D_identity(lib):
    """CS336 L5 notes Exercise 9: sum_j P_ij dP_ij = sum_k dO_ik O_ik."""
    rng = _rng(21)
    for causal in (False, True):
        q, k, v, do = rng.normal(size=(4, 37, 8))
        g = oracle.attn_bwd(q, k, v, do, causal, 0.3, lib=lib)
        _, _, p = oracle.attn_fwd(q, k, v, causal, 0.3, return_p=True, lib=lib)
        dP = do @ v.T
        _assert_close(g["D"], (p * dP).sum(-1), 1e-12, 1e-12, "D identity")
        _assert_close(g["D"], (do * g["o"]).sum(-1), 1e-12, 1e-12, "D definition")


def pin_bwd_invariants(lib):
    """Rows of P sum to 1, so sum_j dV_j = sum_i dO_i; softmax is shift
    invariant along a row, so each row of dS sums to 0 and sum_j dK_j = 0."""
    rng = _rng(22)
    for causal in (False, True):
        q, k, v, do = rng.normal(size=(4, 45, 6))
        g = oracle.attn_bwd(q, k, v, do, causal, 0.4, lib=lib)
        _assert_close(g["dv"].sum(0), do.sum(0), 1e-12, 1e-12, "sum dV")
        _assert_close(g["dk"].sum(0), np.zeros(6), 0, 1e-12 * np.abs(g["dk"]).sum(), "sum dK")


# ---------------------------------------------------------------- Nq x Nk pins
def pin_rect_brute_force(lib):
    """Nq queries at the end of an Nk-key sequence: 50-digit brute force."""
    rng = _rng(31)
    for Nq, Nk, d, causal in [(3, 7, 3, True), (1, 6, 4, True), (4, 4, 2, True),
                              (5, 9, 3, False), (2, 5, 4, True), (6, 6, 3, False)]:
        q = rng.normal(0, 1.5, size=(Nq, d))
        k, v = rng.normal(0, 1.5, size=(2, Nk, d))
        scale = 1 / math.sqrt(d)
        o, lse = oracle.attn_fwd_rect(q, k, v, causal, scale, lib=lib)
        Od, Ld = dec_forward_rect(_to_dec(q), _to_dec(k), _to_dec(v), causal, scale)
        _assert_close(o, np.array([[float(x) for x in r] for r in Od]), 1e-13, 1e-14, "rect brute O")
        _assert_close(lse, np.array([float(x) for x in Ld]), 1e-14, 1e-14, "rect brute lse")


def pin_rect_q_zero(lib):
    """Q = 0: every visible key gets the same weight, so O_i is the mean of
    the visible V rows and lse_i = ln(number of visible keys)."""
    rng = _rng(32)
    Nq, Nk, d = 5, 13, 4
    k, v = rng.normal(size=(2, Nk, d))
    q = np.zeros((Nq, d))
    o, lse = oracle.attn_fwd_rect(q, k, v, False, 0.5, lib=lib)
    _assert_close(o, np.tile(v.mean(0), (Nq, 1)), 1e-13, 1e-13, "rect Q=0 mean")
    _assert_close(lse, np.full(Nq, math.log(Nk)), 1e-14, 0, "rect Q=0 lse")
    o, lse = oracle.attn_fwd_rect(q, k, v, True, 0.5, lib=lib)
    seen = np.arange(Nq) + (Nk - Nq) + 1
    _assert_close(o, np.stack([v[:n].mean(0) for n in seen]), 1e-13, 1e-13, "rect Q=0 causal")
    _assert_close(lse, np.log(seen), 1e-14, 1e-15, "rect Q=0 causal lse")


def pin_rect_merge(lib):
    """CS149 L9 notes section 9: attention over a split key range equals the
    merge of the per-chunk results, lse = ln sum_c e^{lse_c} and
    O = sum_c e^{lse_c - lse} O_c, for chunk sizes that do not divide Nk."""
    rng = _rng(33)
    Nq, Nk, d = 3, 23, 5
    q = rng.normal(size=(Nq, d))
    k, v = rng.normal(size=(2, Nk, d))
    o, lse, p = oracle.attn_fwd_rect(q, k, v, False, 0.6, return_p=True, lib=lib)
    _assert_close(p @ v, o, 1e-13, 1e-14, "rect O = P V")
    _assert_close(p.sum(-1), np.ones(Nq), 1e-14, 0, "rect P rows sum to 1")
    edges = [0, 4, 11, 12, 23]
    parts = [oracle.attn_fwd_rect(q, k[a:b], v[a:b], False, 0.6, lib=lib)
             for a, b in zip(edges[:-1], edges[1:])]
    m = np.max([lc for _, lc in parts], axis=0)
    w = [np.exp(lc - m) for _, lc in parts]
    lse_m = m + np.log(sum(w))
    o_m = sum(wc[:, None] * oc for wc, (oc, _) in zip(w, parts)) / sum(w)[:, None]
    _assert_close(lse_m, lse, 1e-14, 1e-14, "merged lse")
    _assert_close(o_m, o, 1e-13, 1e-14, "merged O")


def pin_rect_bwd_finite_differences(lib):
    """Gradient of L = sum(dO * O) for Nq queries at the end of Nk keys, by
    central differences of the 50-digit shifted-mask forward (independent of
    the oracle's forward and backward)."""
    rng = _rng(34)
    h = Decimal("1e-15")
    for Nq, Nk, d, causal in [(2, 5, 3, True), (3, 4, 2, False), (1, 4, 3, True), (3, 3, 2, True)]:
        q, do = rng.normal(size=(2, Nq, d))
        k, v = rng.normal(size=(2, Nk, d))
        scale = 1 / math.sqrt(d)
        g = oracle.attn_bwd_rect(q, k, v, do, causal, scale, lib=lib)
        base = {"q": _to_dec(q), "k": _to_dec(k), "v": _to_dec(v)}
        dod = _to_dec(do)

        def loss(t):
            O, _ = dec_forward_rect(t["q"], t["k"], t["v"], causal, scale)
            return sum((O[i][c] * dod[i][c] for i in range(Nq) for c in range(d)), Decimal(0))

        for name, rows in (("q", Nq), ("k", Nk), ("v", Nk)):
            fd = np.zeros((rows, d))
            for i in range(rows):
                for c in range(d):
                    t = {n: [row[:] for row in a] for n, a in base.items()}
                    t[name][i][c] = base[name][i][c] + h
                    lp = loss(t)
                    t[name][i][c] = base[name][i][c] - h
                    lm = loss(t)
                    fd[i, c] = float((lp - lm) / (2 * h))
            _assert_close(g["d" + name], fd, 1e-10, 1e-12, f"rect finite differences d{name}")


def pin_rect_bwd_invariants(lib):
    """For Nq queries against Nk keys: sum_j dV_j = sum_i dO_i (rows of P sum
    to 1), sum_j dK_j = 0 (each row of dS sums to 0), the D identity of CS336
    L5 notes Exercise 9, and O, lse equal to the rectangular forward's."""
    rng = _rng(35)
    for Nq, Nk, causal in [(13, 40, True), (40, 13, False), (29, 29, True)]:
        q, do = rng.normal(size=(2, Nq, 6))
        k, v = rng.normal(size=(2, Nk, 6))
        g = oracle.attn_bwd_rect(q, k, v, do, causal, 0.45, lib=lib)
        _assert_close(g["dv"].sum(0), do.sum(0), 1e-12, 1e-12, "rect sum dV")
        _assert_close(g["dk"].sum(0), np.zeros(6), 0, 1e-12 * np.abs(g["dk"]).sum(), "rect sum dK")
        o, lse = oracle.attn_fwd_rect(q, k, v, causal, 0.45, lib=lib)
        _assert_close(g["o"], o, 1e-13, 1e-14, "rect bwd O")
        _assert_close(g["lse"], lse, 1e-14, 1e-14, "rect bwd lse")
        _assert_close(g["D"], (do * o).sum(-1), 1e-12, 1e-12, "rect D definition")


def pin_rect_bwd_square(lib):
    """Nq = Nk is the square backward, pinned on its own above."""
    rng = _rng(36)
    for causal in (False, True):
        q, k, v, do = rng.normal(size=(4, 21, 5))
        a = oracle.attn_bwd(q, k, v, do, causal, 0.5, lib=lib)
        b = oracle.attn_bwd_rect(q, k, v, do, causal, 0.5, lib=lib)
        for n in ("dq", "dk", "dv"):
            _assert_close(b[n], a[n], 1e-13, 1e-13, f"rect square {n}")


def pin_mx_e4m3_codes(lib):
    """Every E4M3 code decodes to torch's float8_e4m3fn value (a separate
    implementation of the OCP format), and the format's fixed points hold."""
    import torch
    codes = np.arange(256, dtype=np.uint8).reshape(8, 32)
    scales = np.full((8, 1), 127, dtype=np.uint8)  # 2^0
    got = oracle.mx_decode(codes, scales, lib=lib).reshape(-1)
    ref = torch.from_numpy(codes.reshape(-1).copy()).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all(), "NaN codes"
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF], "exactly S.1111.111 is NaN"
    assert np.array_equal(got[~nan], ref[~nan]), "E4M3 values differ from torch's"
    fixed = {0x00: 0.0, 0x38: 1.0, 0xB8: -1.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9,
             0x07: 7 * 2.0 ** -9, 0x40: 2.0, 0x3C: 1.5}
    for c, val in fixed.items():
        assert got[c] == val, f"code {c:#04x}: {got[c]} != {val}"


def pin_mx_scales(lib):
    """E8M0 scale e multiplies by 2^(e - 127) (255 is NaN), and element c of a
    row takes the scale of block c // 32."""
    d = 128
    codes = np.full((3, d), 0x38, dtype=np.uint8)  # all 1.0
    scales = np.array([[127, 128, 126, 200], [0, 254, 127, 127], [255, 127, 1, 129]],
                      dtype=np.uint8)
    got = oracle.mx_decode(codes, scales, lib=lib)
    for r in range(3):
        for c in range(d):
            e = int(scales[r, c // 32])
            want = float("nan") if e == 255 else 2.0 ** (e - 127)
            if math.isnan(want):
                assert math.isnan(got[r, c]), f"({r},{c}) should be NaN"
            else:
                assert got[r, c] == want, f"({r},{c}): {got[r, c]} != {want}"
    # a value times its scale (sign and magnitude)
    codes = np.array([[0xC4] * 32 + [0x11] * 32], dtype=np.uint8)  # -3.0, 2^-9*... codes
    scales = np.array([[130, 100]], dtype=np.uint8)
    got = oracle.mx_decode(codes, scales, lib=lib)
    assert got[0, 0] == -3.0 * 8 and got[0, 40] == (1 + 1 / 8) * 2.0 ** -5 * 2.0 ** -27


FORWARD_PINS = [pin_worked_example, pin_blocked_identity, pin_streaming_and_blocked,
                pin_rows_sum_to_one, pin_constant_v, pin_q_zero, pin_row0_and_single_key,
                pin_brute_force, pin_large_logits, pin_rows_entry]
BACKWARD_PINS = [pin_bwd_finite_differences, pin_bwd_D_identity, pin_bwd_invariants,
                 pin_bwd_dq_rows]
RECT_PINS = [pin_rect_brute_force, pin_rect_q_zero, pin_rect_merge,
             pin_rect_bwd_finite_differences, pin_rect_bwd_invariants, pin_rect_bwd_square]
MX_PINS = [pin_mx_e4m3_codes, pin_mx_scales]
ALL_PINS = FORWARD_PINS + BACKWARD_PINS + RECT_PINS + MX_PINS
