"""GPU parity on the method's edge cases, through the C ABI, bit for bit.

Each case builds its inputs here by construction (no seeded workload), runs
them through the GPU library and the oracle side by side (tests/gpu_harness.py
Twin) and requires every stored field, every output and, before each
separate fold, the full rebuilt state to be bitwise equal:

  * the round-half-even fixture of tests/golden/arith_fixtures.json (exact
    .5 ties) in several heads, rows and column offsets;
  * rows whose largest magnitude lies below 2^-120 (stored as zeros), at
    exactly 2^-120, rows of subnormals, rows mixing a normal maximum with
    subnormal entries, and columns of subnormals, with and without smoothing;
  * bitwise-equal line energies: duplicated rows across the row 63 / 64
    boundary of the pick's ballot words, duplicated columns 63 / 64, the
    fixture pairs of pick_ties and pick_equal_rows, and planted lines whose
    picks land in every register block of the zeroing (row blocks 0..3,
    column entries 0..15) and in unused (-1) slots;
  * folds whose records make a fused multiply-add and a multiply-then-add
    differ (a CPU check below counts this on the oracle), with subnormal
    products and accumulators, rows that cancel exactly to +0, and rows
    that keep only the rounding error of gamma_n * line, which a
    multiply-then-add would turn into zero.

The rebuild applies records with K = 1 matrix-core steps; these cases pin,
in the product path, that such a step rounds like one fma (including
subnormal operands and results), since the oracle's rebuild is an fma chain.

The precondition checks (test_*_preconditions) run on the CPU with the
oracle only; the rest need the GPU.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_harness import D, Report, Twin, progress

F = np.float32
GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "arith_fixtures.json")


def _fixtures():
    with open(GOLD) as f:
        return json.load(f)


def _finish(rep):
    progress(f"    summary: {rep.summary()}")
    rep.check()
    assert sum(rep.nonbit.values()) == 0, rep.nonbit


def _bits(x):
    return np.ascontiguousarray(x, np.float32).view(np.uint32)


def _unit(rng, n):
    x = rng.standard_normal((n, D))
    return (x / np.linalg.norm(x, axis=1, keepdims=True)).astype(F)


def _tokens(rng, H, T, beta=None):
    """T tokens of the seeded distributions (q, k unit; v Gaussian;
    alpha = exp(-softplus(N(-3, 1))); beta = sigmoid(N(0, 1)) or fixed)."""
    toks = []
    for _ in range(T):
        q, k = _unit(rng, H), _unit(rng, H)
        v = rng.standard_normal((H, D)).astype(F)
        z = rng.standard_normal(H) - 3.0
        a = np.exp(-np.logaddexp(0.0, z)).astype(F)
        b = (1.0 / (1.0 + np.exp(-rng.standard_normal(H)))).astype(F) if beta is None else np.full(H, beta, F)
        toks.append((q, k, v, a, b))
    return toks


# ------------------------------------------------------------ exact ties

def half_even_state():
    """The round_half_even fixture row in 5 heads, at rows 17, 0, 63, 64,
    127, its entries shifted by 5 columns per head; everything else zero."""
    case = _fixtures()["round_half_even"]
    rows = [17, 0, 63, 64, 127]
    S0 = np.zeros((len(rows), D, D), F)
    for h, r in enumerate(rows):
        for i, x in case["row"].items():
            S0[h, r, (int(i) + 5 * h) % D] = F(x)
    return S0, rows, case


@pytest.mark.gpu
def test_round_half_even_fixture():
    S0, rows, case = half_even_state()
    tw = Twin(S0, C=0, smoothing=False)
    _finish(tw.rep)
    Q, rho = tw.L.codes().cpu().numpy(), tw.L.rho().cpu().numpy()
    for h, r in enumerate(rows):
        for i, c in case["expected_codes"].items():
            assert int(Q[h, r, (int(i) + 5 * h) % D]) == c, (h, r, i)
        assert rho[h, r] == F(case["expected_rho"])


# ------------------------------------------------- tiny and subnormal rows

def tiny_state(seed=3):
    """4 heads: random rows over six decades plus, per head, a row of
    2^-121 (below the 2^-120 threshold), a row whose maximum is exactly
    2^-120 with subnormal entries, a row of subnormals only, a row with a
    normal maximum and subnormal entries, a row whose maximum is the float
    just below 2^-120, a row spanning 2^-100 .. 2^-140, a row straddling
    2^-126, and a column of subnormals."""
    rng = np.random.default_rng(seed)
    H = 4
    S0 = (rng.standard_normal((H, D, D)) * 10.0 ** rng.integers(-3, 3, (H, D, 1))).astype(F)
    sub = lambda n: (rng.integers(1, 1 << 20, n) * rng.choice([-1, 1], n)).astype(np.float64) * 2.0 ** -149
    for h in range(H):
        o = 11 * h
        S0[h, (1 + o) % D] = F(2.0 ** -121) * rng.choice([-1, 1], D).astype(F)
        r = (2 + o) % D
        S0[h, r] = sub(D).astype(F)
        S0[h, r, (7 * h) % D] = F(2.0 ** -120)
        S0[h, (3 + o) % D] = sub(D).astype(F)
        r = (4 + o) % D
        S0[h, r] = sub(D).astype(F)
        S0[h, r, 5] = F(1.0)
        S0[h, (5 + o) % D] = np.nextafter(F(2.0 ** -120), F(0)) * rng.choice([-1, 1], D).astype(F)
        S0[h, (6 + o) % D] = (rng.standard_normal(D) * 2.0 ** -rng.integers(100, 141, D)).astype(F)
        S0[h, (7 + o) % D] = (2.0 ** -126 + sub(D) * rng.choice([-1, 1], D)).astype(F)
        S0[h, :, (100 + h) % D] = sub(D).astype(F)
    assert np.isfinite(S0).all()
    return S0


@pytest.mark.parametrize("C,smoothing,floor,fused", [(0, False, 1e-6, False), (4, True, 1e-6, False),
                                                      (4, True, 1e-30, True), (8, True, 1e-30, False)])
def test_tiny_rows_preconditions(C, smoothing, floor, fused):
    """The constructed state reaches the cases named above in the oracle:
    nonzero rows stored as zeros (tiny maxima), quantized rows holding
    subnormal entries, and without smoothing the threshold itself (a row
    at exactly 2^-120 is quantized, the float below it is not); with a tiny
    floor, a smoothing scale computed from a column of subnormals."""
    S0 = tiny_state()
    sub = (S0 != 0) & (np.abs(S0) < F(2.0 ** -126))
    assert sub.sum() > 1000
    for h in range(S0.shape[0]):
        ref = oracle.Head(C, 16, smoothing, floor).init(S0[h])
        nz = np.any(S0[h] != 0, axis=1)
        assert np.sum(nz & (ref.rho == 0)) >= 3
        assert np.sum((ref.rho > 0) & np.any(sub[h], axis=1)) >= 2
        o = 11 * h
        if not smoothing:
            assert ref.rho[(1 + o) % D] == 0 and ref.rho[(5 + o) % D] == 0 and ref.rho[(3 + o) % D] == 0
            assert ref.rho[(2 + o) % D] > 0 and ref.rho[(4 + o) % D] > 0
        if smoothing and floor < 1e-20:
            s = ref.sigma[(100 + h) % D]
            assert floor < s < 1e-15, s


@pytest.mark.gpu
@pytest.mark.parametrize("C,smoothing,floor,fused", [(0, False, 1e-6, False), (4, True, 1e-6, False),
                                                      (4, True, 1e-30, True), (8, True, 1e-30, False)])
def test_tiny_and_subnormal_rows(C, smoothing, floor, fused):
    """Init, two windows (every token, the rebuilt state before a separate
    fold, each fold) bitwise against the oracle."""
    S0 = tiny_state()
    rng = np.random.default_rng(4)
    tw = Twin(S0, C=C, smoothing=smoothing, sigma_floor=floor)
    for w in range(2):
        for t, tok in enumerate(_tokens(rng, S0.shape[0], 16)):
            last = t == 15
            tw.append(tok, fused=fused and last)
        if not fused:
            tw.fold()
    _finish(tw.rep)


# ------------------------------------------------------ equal energies

def tie_state():
    """6 heads with planted lines, C = 8.  Head 0: rows 63 and 64 identical
    and strongest, rows 5 and 100; columns in register entries m = 0..3.
    Head 1: columns 63 and 64 identical and strongest, columns in m = 4..6
    and 9, rows 40 and 70.  Head 2: one row in each row block (10, 45, 80,
    120) and columns in m = 10..13.  Head 3: a zero state but for row 20 and
    columns 115, 125 (m = 14, 15): three picks, then unused slots.  Heads 4
    and 5: the pick_equal_rows and pick_ties fixtures."""
    rng = np.random.default_rng(11)
    H = 6
    S0 = (rng.standard_normal((H, D, D)) * 0.01).astype(F)
    plan = {0: ([(63, 60.0), (5, 30.0), (100, 25.0)], [(3, 38.0), (9, 33.0), (18, 28.0), (30, 23.0)]),
            1: ([(40, 8.0), (70, 6.0)], [(63, 60.0), (33, 38.0), (44, 33.0), (50, 28.0), (75, 23.0)]),
            2: ([(10, 40.0), (45, 35.0), (80, 30.0), (120, 25.0)], [(83, 38.0), (90, 33.0), (100, 28.0),
                                                                   (110, 23.0)])}
    # a planted line holds s (1 + 0.1 z): its energy is about 128 s^2, far
    # above the noise; columns are written after rows (they own the crossings)
    for h, (rows, cols) in plan.items():
        for r, sc in rows:
            S0[h, r, :] = (sc * (1.0 + 0.1 * rng.standard_normal(D))).astype(F)
        for c, sc in cols:
            S0[h, :, c] = (sc * (1.0 + 0.1 * rng.standard_normal(D))).astype(F)
    S0[0, 64, :] = S0[0, 63, :]
    S0[1, :, 64] = S0[1, :, 63]
    S0[3] = 0.0
    S0[3, 20, :] = (rng.standard_normal(D) * 5).astype(F)
    S0[3, :, 115] = (rng.standard_normal(D) * 4).astype(F)
    S0[3, :, 125] = (rng.standard_normal(D) * 3).astype(F)
    g = _fixtures()
    S0[4] = 0.0
    line = (np.arange(1, D + 1) / 64.0).astype(F)
    S0[4, 9] = line
    S0[4, 5] = line
    S0[5] = 0.0
    S0[5, 3, :] = 1.0
    S0[5, :, 7] = 1.0
    return S0, g


def _tie_checks(idx):
    """Tie rules and leaf coverage on one set of picks [6][8]."""
    g = _fixtures()
    assert list(idx[0][:2]) == [63, 64], idx[0]
    assert list(idx[1][:2]) == [D + 63, D + 64], idx[1]
    assert list(idx[4][:1]) == g["pick_equal_rows"]["expected_idx"], idx[4]
    assert list(idx[5][:2]) == g["pick_ties"]["expected_idx"], idx[5]
    assert -1 in list(idx[3]) and -1 in list(idx[5])
    picks = [int(i) for h in range(4) for i in idx[h] if i >= 0]
    assert {i >> 5 for i in picks if i < D} == {0, 1, 2, 3}
    assert {(i - D) >> 3 for i in picks if i >= D} == set(range(16))


def test_ties_preconditions():
    S0, _ = tie_state()
    idx = [oracle.Head(8).init(S0[h]).idx for h in range(S0.shape[0])]
    _tie_checks(idx)


@pytest.mark.gpu
@pytest.mark.parametrize("fused", [True, False])
def test_equal_energy_ties_every_leaf(fused):
    """Init, then a window of beta = 0 tokens (every record's correction is
    a signed zero, so the rebuilt state is gamma_n B and the ties survive
    into the fold), then a window of regular tokens.  Picks, lines, codes,
    scales, outputs and records bitwise; the tie rules and the leaf coverage
    hold on the GPU's picks at init and after the first fold."""
    S0, _ = tie_state()
    H = S0.shape[0]
    rng = np.random.default_rng(12)
    tw = Twin(S0, C=8)
    _tie_checks(tw.L.comp_idx().cpu().numpy())
    for t, tok in enumerate(_tokens(rng, H, 16, beta=0.0)):
        tw.append(tok, fused=fused and t == 15)
    if not fused:
        tw.fold()
    _tie_checks(tw.L.comp_idx().cpu().numpy())
    for t, tok in enumerate(_tokens(rng, H, 16)):
        tw.append(tok, fused=fused and t == 15)
    if not fused:
        tw.fold()
    _finish(tw.rep)


# ------------------------------------------- rebuild: fma, subnormals, zeros

def stress_state(seed=21):
    """4 heads; rows 0..31 Gaussian with two outlier rows x50 (kept as row
    lines); rows 32..63 at 2^-100 .. 2^-118 (quantized tiny rows); rows
    64..95 with a magnitude 2^-(0..140) per entry; rows 96..127 at
    2^-121 .. 2^-135 (stored as zeros, so their rebuilt values come from the
    records alone); one outlier column x30."""
    rng = np.random.default_rng(seed)
    H = 4
    S0 = rng.standard_normal((H, D, D))
    S0[:, 32:64] *= 2.0 ** -rng.integers(100, 119, (H, 32, 1))
    S0[:, 64:96] *= 2.0 ** -rng.integers(0, 141, (H, 32, D))
    S0[:, 96:128] *= 2.0 ** -rng.integers(121, 136, (H, 32, 1))
    for h in range(H):
        S0[h, rng.choice(32, 2, replace=False)] *= 50.0
        S0[h, :, rng.integers(0, D)] *= 30.0
    return S0.astype(F)


def stress_tokens(seed=22, H=4, T=16):
    """Tokens whose keys reach the tiny rows at their own scale: entries of
    rows 32..63 scaled by 2^-(100..140) per token, of rows 96..127 by a
    per-row 2^-(128..145) for the whole window (subnormal products with
    corrections of order one, summed into subnormal entries), of rows
    64..95 by 2^-(0..60)."""
    rng = np.random.default_rng(seed)
    toks = _tokens(rng, H, T)
    f_rows = (2.0 ** -rng.integers(128, 146, (H, 32))).astype(F)
    for q, k, v, a, b in toks:
        k[:, 32:64] *= (2.0 ** -rng.integers(100, 141, (H, 32))).astype(F)
        k[:, 96:128] *= f_rows
        k[:, 64:96] *= (2.0 ** -rng.integers(0, 61, (H, 32))).astype(F)
    return toks


def current_mul_add(head):
    """The oracle head's current state rebuilt with each record applied as
    a rounded product followed by a rounded add (numpy float32), in place of
    the fused multiply-add: the rebuild a non-fused matrix step would give."""
    n = head.n
    gn = head.gam[n - 1] if n else F(1.0)
    S = (head.Q.astype(F) * (gn * head.rho)[:, None]) * head.sigma[None, :]
    for j in range(head.C):
        i = int(head.idx[j])
        if 0 <= i < D:
            S[i, :] = S[i, :] + gn * head.vec[j]
        elif i >= D:
            S[:, i - D] = S[:, i - D] + gn * head.vec[j]
    for i in range(n):
        w = (gn / head.gam[i]) * head.rk[i]
        S = (w[:, None] * head.ru[i][None, :]) + S
    return S.astype(F)


def _products_subnormal(head):
    """Nonzero record products w_i[r] u_i[c] below 2^-126, in float64."""
    n = head.n
    cnt = 0
    for i in range(n):
        w = ((head.gam[n - 1] / head.gam[i]) * head.rk[i]).astype(np.float64)
        p = w[:, None] * head.ru[i].astype(np.float64)[None, :]
        cnt += int(np.sum((p != 0) & (np.abs(p) < 2.0 ** -126)))
    return cnt


def _row_lines(head):
    return [int(i) for i in head.idx if 0 <= i < D]


def cancel_tokens(heads, rng, r_zero, r_keep, alpha_one=True):
    """A window whose first tokens are one-hot keys e_r with v = 0 and
    beta = 1, so each such record's correction is -B[r, :]: with alpha = 1
    for the whole window (alpha_one) the rebuilt row r cancels to +0
    exactly; with alpha = 1 only for the first token, a row line keeps
    exactly the rounding error of gamma_n * line, which a multiply-then-add
    cancels to zero.  The other tokens' keys are zero on those rows."""
    H = len(heads)
    toks = _tokens(rng, H, 16)
    special = [r_zero, r_keep]
    for t, (q, k, v, a, b) in enumerate(toks):
        for h in range(H):
            rows = [special[j][h] for j in range(2) if special[j] is not None]
            if t < len(rows):
                k[h] = 0.0
                k[h, rows[t]] = 1.0
                v[h] = 0.0
                b[h] = 1.0
            else:
                k[h, rows] = 0.0
            if alpha_one or t == 0:
                a[h] = 1.0
    return toks


def test_rebuild_stress_preconditions():
    """On the oracle alone: the stress window's rebuild differs from a
    multiply-then-add rebuild in many entries, with subnormal products and
    subnormal accumulators; the cancellation windows give +0 rows, and a
    row of pure rounding error that a multiply-then-add would zero."""
    S0 = stress_state()
    H = S0.shape[0]
    heads = [oracle.Head(4).init(S0[h]) for h in range(H)]
    for tok in stress_tokens(H=H):
        q, k, v, a, b = tok
        for h in range(H):
            heads[h].append(q[h], k[h], v[h], a[h], b[h])
    cur = np.stack([hd.dequant(2) for hd in heads])
    mul = np.stack([current_mul_add(hd) for hd in heads])
    ndiff = int(np.sum(_bits(cur) != _bits(mul)))
    nsub = int(np.sum((cur != 0) & (np.abs(cur) < F(2.0 ** -126))))
    nprod = sum(_products_subnormal(hd) for hd in heads)
    progress(f"    stress: fma vs mul-add differ in {ndiff}, subnormal entries {nsub}, subnormal products {nprod}")
    assert ndiff > 5000 and nsub > 1000 and nprod > 1000
    for hd in heads:
        hd.fold()
    rng = np.random.default_rng(23)
    r0 = [_row_lines(hd)[0] for hd in heads]
    r1 = [int(np.flatnonzero(hd.rho)[np.flatnonzero(hd.rho) != r][0]) for hd, r in zip(heads, r0)]
    for tok in cancel_tokens(heads, rng, r0, r1, alpha_one=True):
        q, k, v, a, b = tok
        for h in range(H):
            heads[h].append(q[h], k[h], v[h], a[h], b[h])
    cur = np.stack([hd.dequant(2) for hd in heads])
    for h in range(H):
        assert not _bits(cur[h, r0[h]]).any() and not _bits(cur[h, r1[h]]).any()
        assert _bits(cur[h]).any()
    for hd in heads:
        hd.fold()
    r2 = [_row_lines(hd)[0] for hd in heads]
    for tok in cancel_tokens(heads, rng, r2, None, alpha_one=False):
        q, k, v, a, b = tok
        for h in range(H):
            heads[h].append(q[h], k[h], v[h], a[h], b[h])
    cur = np.stack([hd.dequant(2) for hd in heads])
    mul = np.stack([current_mul_add(hd) for hd in heads])
    for h in range(H):
        assert np.sum(cur[h, r2[h]] != 0) >= 64, np.sum(cur[h, r2[h]] != 0)
        assert not np.any(mul[h, r2[h]]), "a multiply-then-add rebuild should cancel the row"


@pytest.mark.gpu
@pytest.mark.parametrize("fused", [False, True])
def test_rebuild_fma_subnormal_cancellation(fused):
    """The three stress windows on the GPU beside the oracle.  Without
    fused, the full rebuilt state (dequant view 2, which runs the fold's
    matrix-core rebuild) is compared bit for bit before each fold; with
    fused, the last token and its fold are one call (its own rebuild, from
    the weighted keys the append leaves) and the current-state view is
    compared after the window's 15th token."""
    S0 = stress_state()
    H = S0.shape[0]
    tw = Twin(S0, C=4)
    rng = np.random.default_rng(23)

    def window(toks, expect_zero=(), expect_residue=()):
        for t, tok in enumerate(toks):
            if fused and t == 15:
                got, ref = tw.current()
                tw.rep.fp("current15", got, ref)
            tw.append(tok, fused=fused and t == 15)
        if not fused:
            got, ref = tw.current()
            for h, r in expect_zero:
                assert not _bits(got[h, r]).any(), (h, r)
            for h, r in expect_residue:
                assert np.sum(got[h, r] != 0) >= 64, (h, r)
            tw.fold()

    window(stress_tokens(H=H))
    r0 = [_row_lines(hd)[0] for hd in tw.refs]
    r1 = [int(np.flatnonzero(hd.rho)[np.flatnonzero(hd.rho) != r][0]) for hd, r in zip(tw.refs, r0)]
    window(cancel_tokens(tw.refs, rng, r0, r1, alpha_one=True),
           expect_zero=[(h, r0[h]) for h in range(H)] + [(h, r1[h]) for h in range(H)])
    r2 = [_row_lines(hd)[0] for hd in tw.refs]
    window(cancel_tokens(tw.refs, rng, r2, None, alpha_one=False), expect_residue=[(h, r2[h]) for h in range(H)])
    _finish(tw.rep)


# ------------------------------------------------------------- resume

@pytest.mark.gpu
def test_resume_from_snapshot():
    """Prefix-caching use of the boundary state: a layer's whole buffer is
    copied to host memory at n = 7, restored into a fresh buffer with the
    same record count, and both layers continue through 41 more tokens
    (fused and separate folds, a partial window).  Every output and the
    whole state buffer stay bit-identical."""
    import dataclasses

    from quantized_recurrent_state_amd import leapq as lq
    from quantized_recurrent_state_amd import workloads
    wl = dataclasses.replace(workloads.WORKLOADS["tiny"], batch=2, heads=8, init="prefill", seed=55)
    H = wl.batch * wl.heads
    cfg = lq.make_config(wl.batch, wl.heads, wl.window, wl.n_comp)
    A = lq.Layer(cfg)
    lq.leapq_init_state(A, workloads.initial_state(wl, 0).reshape(H, D, D).cuda())
    oa = torch.empty(H, D, device="cuda")
    ob = torch.empty(H, D, device="cuda")

    def tok(t):
        q, k, v, a, b = workloads.token_inputs(wl, 0, t)
        return [x.reshape(H, D).cuda() for x in (q, k, v)] + [a.reshape(H).cuda(), b.reshape(H).cuda()]

    for t in range(7):
        lq.leapq_append(A, *tok(t), oa)
    snap = A.state.cpu()
    n_snap = A.n_records
    B = lq.Layer(cfg)
    B.state.copy_(snap.cuda())
    B.c.n_records = n_snap
    assert n_snap == 7
    for t in range(7, 52):
        args = tok(t)
        for L, o in ((A, oa), (B, ob)):
            if t == 31 and L.n_records == wl.window - 1:
                lq.leapq_append_fold(L, *args, o)
            else:
                lq.leapq_append(L, *args, o)
                if L.n_records == wl.window:
                    lq.leapq_fold(L)
        assert torch.equal(oa.view(torch.int32), ob.view(torch.int32)), t
        assert torch.equal(A.state, B.state), t
        assert A.n_records == B.n_records
    progress(f"    resume: 45 tokens after the snapshot, n = {A.n_records}, bit-identical")
