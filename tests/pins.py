"""Pins of the CPU oracle against facts fixed outside it.

Each pin takes a loaded oracle library handle `L` and raises AssertionError
when the oracle disagrees with:
  * hand-derived arithmetic fixtures (tests/golden/arith_fixtures.json),
  * the dense GDN recurrence written here in float64 numpy, which the windowed
    path must reproduce to rounding (LeapQuant B.2 window unrolling; B.1 no
    error inside a window),
  * closed-form special cases of the delta rule (LeapQuant App. A),
  * exact scaling and tree-automorphism equivariance of the quantizer,
  * planted outliers, a float64 brute-force argmax, textbook absmax int8.
The same pins run against deliberately broken copies of the oracle in
test_oracle_mutants.py, where each copy must fail at least one of them.
"""
import json
import os

import numpy as np
import torch

import oracle
from quantized_recurrent_state_amd import workloads

D = 128
GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(float(np.max(np.abs(b))), 1e-30))


def sparse_vec(d):
    v = np.zeros(D, np.float32)
    for i, x in d.items():
        v[int(i)] = np.float32(x)
    return v


# ---------------------------------------------------------------- inputs

def tiny_inputs(seed=0, tokens=16, heads=1, init="gauss", C=4, head=0):
    """Seeded tiny case: (S0 [heads,128,128], per-token (q, k, v, alpha, beta)
    of head `head`)."""
    wl = workloads.Workload("pin", 1, 1, heads, tokens, init=init, seed=seed, n_comp=C)
    S0 = workloads.initial_state(wl, 0).numpy()[0]
    toks = []
    for t in range(tokens):
        q, k, v, a, b = workloads.token_inputs(wl, 0, t)
        toks.append((q.numpy()[0, head], k.numpy()[0, head], v.numpy()[0, head],
                     np.float32(a.numpy()[0, head]), np.float32(b.numpy()[0, head])))
    return S0, toks


def np_gdn_f64(S, q, k, v, alpha, beta):
    """The dense GDN token step in float64 (decay, read with k, correction,
    rank-one write, read with q); S is [key row, value column]."""
    S *= alpha
    r = S.T @ k
    u = beta * (v - r)
    S += np.outer(k, u)
    return u, S.T @ q


# ---------------------------------------------------------------- pins

def pin_t128_fixtures(L):
    g = golden("arith_fixtures.json")
    for key in ("t128_sum_level0_pairs_i_with_i_plus_64", "t128_sum_levels_halve_from_32"):
        case = g[key]
        got = oracle.t128_sum(sparse_vec(case["nonzero"]), L)
        assert got == case["expected"], (key, got)
    for key in ("t128_dot_fma_on_lower_term", "t128_dot_upper_term_rounded"):
        case = g[key]
        got = oracle.t128_dot(sparse_vec(case["a"]), sparse_vec(case["b"]), L)
        assert got == case["expected"], (key, got)


def pin_t128_exact_integers(L):
    rng = np.random.default_rng(7)
    for _ in range(20):
        a = rng.integers(-1000, 1000, D).astype(np.float32)
        b = rng.integers(-1000, 1000, D).astype(np.float32)
        assert oracle.t128_sum(a, L) == float(a.astype(np.int64).sum())
        assert oracle.t128_dot(a, b, L) == float((a.astype(np.int64) * b.astype(np.int64)).sum())
        # a single nonzero term anywhere is returned unchanged
        j = int(rng.integers(0, D))
        e = np.zeros(D, np.float32)
        e[j] = a[j] + 0.5
        assert oracle.t128_sum(e, L) == float(e[j])


def pin_round_half_even(L):
    case = golden("arith_fixtures.json")["round_half_even"]
    R = np.zeros((D, D), np.float32)
    R[17] = sparse_vec(case["row"])
    h = oracle.Head(C=0, smoothing=False, L=L).init(R)
    want = np.zeros(D, np.int8)
    for i, c in case["expected_codes"].items():
        want[int(i)] = c
    assert np.array_equal(h.Q[17], want), h.Q[17][:12]
    assert h.rho[17] == np.float32(case["expected_rho"])
    others = np.delete(np.arange(D), 17)
    assert not h.Q[others].any() and not h.rho[others].any()


def pin_round_exact_product_once(L):
    """A code is the nearest integer to the exact product x * (127 / M), with
    one rounding: the fixture's entry lies a sliver above a .5 boundary, where
    rounding the fp32 product first lands on the tie and goes to the even code."""
    case = golden("arith_fixtures.json")["round_exact_product_once"]
    R = np.zeros((D, D), np.float32)
    R[40] = sparse_vec(case["row"])
    h = oracle.Head(C=0, smoothing=False, L=L).init(R)
    want = np.zeros(D, np.int8)
    for i, c in case["expected_codes"].items():
        want[int(i)] = c
    assert np.array_equal(h.Q[40], want), h.Q[40][:4]
    assert h.rho[40] == np.float32(case["expected_rho"])


def pin_pick_ties(L):
    g = golden("arith_fixtures.json")
    R = np.zeros((D, D), np.float32)
    R[3, :] = 1.0
    R[:, 7] = 1.0
    h = oracle.Head(C=2, smoothing=False, L=L).init(R)
    assert list(h.idx) == g["pick_ties"]["expected_idx"], list(h.idx)
    R = np.zeros((D, D), np.float32)
    line = (np.arange(1, D + 1) / 64.0).astype(np.float32)
    R[9] = line
    R[5] = line
    h = oracle.Head(C=1, smoothing=False, L=L).init(R)
    assert list(h.idx) == g["pick_equal_rows"]["expected_idx"], list(h.idx)


def pin_textbook_int8(L):
    """C=0 without smoothing is per-row symmetric absmax int8: scale = max|x|/127,
    code = round-half-even(x*127/max).  Computed here in float64; a code may
    differ only where the float64 value is within 1e-5 of a .5 boundary."""
    rng = np.random.default_rng(3)
    for trial in range(4):
        R = (rng.standard_normal((D, D)) * (10.0 ** rng.integers(-3, 3, (D, 1)))).astype(np.float32)
        h = oracle.Head(C=0, smoothing=False, L=L).init(R)
        M = np.abs(R.astype(np.float64)).max(axis=1)
        assert np.allclose(h.rho, M / 127.0, rtol=2e-7, atol=0)
        assert np.all(h.sigma == 1.0) and np.all(h.idx[:0] == -1)
        y = R.astype(np.float64) * (127.0 / M)[:, None]
        want = np.rint(y)
        diff = h.Q.astype(np.float64) != want
        near = np.abs(np.abs(y - np.trunc(y)) - 0.5) < 1e-5
        assert not np.any(diff & ~near), np.argwhere(diff & ~near)[:5]
        assert int(diff.sum()) <= 2


def pin_low_bit_textbook(L):
    """6- and 4-bit states with C = 0 and no smoothing are per-row symmetric
    absmax codes with 31 or 7 levels: scale = max|x| / L, code =
    round-half-even(x L / max), computed here in float64; every live row
    reaches +-L, no code exceeds L, and a code may differ only within 1e-5
    of a .5 boundary."""
    rng = np.random.default_rng(7)
    for bits, lv in ((6, 31.0), (4, 7.0)):
        for trial in range(3):
            R = (rng.standard_normal((D, D)) * (10.0 ** rng.integers(-3, 3, (D, 1)))).astype(np.float32)
            h = oracle.Head(C=0, smoothing=False, L=L, bits=bits).init(R)
            M = np.abs(R.astype(np.float64)).max(axis=1)
            assert np.allclose(h.rho, M / lv, rtol=2e-7, atol=0)
            y = R.astype(np.float64) * (lv / M)[:, None]
            want = np.rint(y)
            diff = h.Q.astype(np.float64) != want
            near = np.abs(np.abs(y - np.trunc(y)) - 0.5) < 1e-5
            assert not np.any(diff & ~near), (bits, np.argwhere(diff & ~near)[:5])
            assert np.abs(h.Q).max() == lv and np.all(np.abs(h.Q).max(axis=1) == lv)


def pin_low_bit_planted(L):
    """6- and 4-bit states pick the planted outlier lines of the tiny case
    as their compensators, as the int8 state does."""
    wl = workloads.Workload("pin", 1, 1, 4, 16, init="gauss", seed=0)
    G, lines = workloads.initial_state(wl, 0, return_lines=True)
    for bits in (6, 4):
        for h_ in range(4):
            want = set(int(r) for r in lines[0][0, h_]) | set(D + int(c) for c in lines[1][0, h_])
            got = oracle.Head(C=4, L=L, bits=bits).init(G.numpy()[0, h_]).idx
            assert set(int(i) for i in got) == want


def pin_low_bit_window(L):
    """A window from a 4-bit boundary equals the float64 dense recurrence
    from that boundary (outputs and rebuilt state to 1e-5); the fold then
    equals a fresh 4-bit quantization of the rebuilt state."""
    S0, toks = tiny_inputs(seed=45, tokens=16, init="prefill")
    h = oracle.Head(C=4, W=16, L=L, bits=4).init(S0[0])
    S = h.dequant(1).astype(np.float64)
    for (q, k, v, a, b) in toks:
        o, _ = h.append(q, k, v, a, b)
        _, o64 = np_gdn_f64(S, q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), float(a), float(b))
        assert rel(o, o64) < 1e-5
    cur = h.dequant(2)
    assert rel(cur, S) < 1e-5
    h.fold()
    want = oracle.Head(C=4, W=16, L=L, bits=4).init(cur)
    assert np.array_equal(h.Q, want.Q) and np.array_equal(h.rho, want.rho) and np.array_equal(h.idx, want.idx)


def pin_smoothing_closed_form(L):
    """Column c holds +-s_c (alternating signs) with s_c a power of 4, so the mean
    absolute value over the key rows is s_c and sigma_c = sqrt(s_c) exactly;
    a zero column takes the floor.  Rows then quantize x = R / sigma."""
    e = (np.arange(D) % 9) - 4
    s = np.power(4.0, e).astype(np.float32)
    sign = np.where(np.arange(D) % 2 == 0, 1.0, -1.0).astype(np.float32)
    R = (sign[:, None] * s[None, :]).astype(np.float32)
    R[:, 100] = 0.0
    h = oracle.Head(C=0, smoothing=True, sigma_floor=1e-6, L=L).init(R)
    want = np.sqrt(s.astype(np.float64)).astype(np.float32)
    want[100] = np.float32(1e-6)
    assert np.array_equal(h.sigma, want), np.flatnonzero(h.sigma != want)[:5]
    # every smoothed entry is +-sqrt(s_c); the row max is 16 (s=256), so codes
    # are round(127 * sqrt(s_c) / 16) with the row's sign (all products exact)
    mag = np.rint(127.0 * np.sqrt(s.astype(np.float64)) / 16.0)
    mag[100] = 0
    assert np.array_equal(np.abs(h.Q[0].astype(np.int64)), mag.astype(np.int64))
    assert np.all(np.sign(h.Q[1][mag > 0]) == -1)


def pin_scaling_exact(L):
    """Scaling the state by 4 leaves codes and picks unchanged and scales
    rho and sigma by 2 and the compensator lines by 4, exactly (with
    smoothing on; without smoothing any power of two scales rho by itself)."""
    S0, _ = tiny_inputs(seed=11, tokens=1)
    S = S0[0]
    a = oracle.Head(C=4, smoothing=True, L=L).init(S)
    b = oracle.Head(C=4, smoothing=True, L=L).init(S * np.float32(4.0))
    assert np.array_equal(a.Q, b.Q) and np.array_equal(a.idx, b.idx)
    assert np.array_equal(b.rho, a.rho * 2) and np.array_equal(b.vec, a.vec * 4)
    # extracted (zeroed) columns sit at the floor in both; the rest scale by 2
    floor = a.sigma == np.float32(1e-6)
    assert sorted(np.flatnonzero(floor) + D) == sorted(int(i) for i in a.idx if i >= D)
    assert np.array_equal(b.sigma[~floor], a.sigma[~floor] * 2)
    assert np.all(b.sigma[floor] == np.float32(1e-6))
    for p in (0.125, 8.0):
        a = oracle.Head(C=4, smoothing=False, L=L).init(S)
        b = oracle.Head(C=4, smoothing=False, L=L).init(S * np.float32(p))
        assert np.array_equal(a.Q, b.Q) and np.array_equal(a.idx, b.idx)
        assert np.array_equal(b.rho, a.rho * np.float32(p))
        assert np.array_equal(b.vec, a.vec * np.float32(p))


def pin_planted_outliers(L):
    """The tiny case plants 2 rows and 2 columns x50; with C=4 the four
    compensators are exactly those lines at init, and they stay the picks
    after a window of pure decay (beta = 0), where S = gamma B."""
    wl = workloads.Workload("pin", 1, 1, 4, 16, init="gauss", seed=0)
    S0, lines = workloads.initial_state(wl, 0, return_lines=True)
    for h_ in range(4):
        rows, cols = lines
        want = set(int(r) for r in rows[0, h_]) | set(D + int(c) for c in cols[0, h_])
        head = oracle.Head(C=4, L=L).init(S0.numpy()[0, h_])
        assert set(int(i) for i in head.idx) == want, (h_, head.idx, want)
        for t in range(16):
            q, k, v, a, b = workloads.token_inputs(wl, 0, t)
            head.append(q.numpy()[0, h_], k.numpy()[0, h_], v.numpy()[0, h_], a[0, h_], 0.0)
        head.fold()
        assert set(int(i) for i in head.idx) == want, (h_, head.idx, want)


def pin_planted_prefill_lines(L):
    """The prefilled initial states (512 dense tokens from zero) carry 1..4
    injected lines x20..100 per head; with C = 4 each injected line is among
    the compensators picked at init (planted ground truth)."""
    wl = workloads.Workload("pin", 1, 1, 8, 16, seed=1)
    S0, (line, is_row, active) = workloads.initial_state(wl, 0, return_lines=True)
    for h_ in range(8):
        want = {int(line[0, h_, j]) + (0 if bool(is_row[0, h_, j]) else D)
                for j in range(4) if bool(active[0, h_, j])}
        head = oracle.Head(C=4, L=L).init(S0.numpy()[0, h_])
        assert want <= set(int(i) for i in head.idx), (h_, head.idx, want)


def pin_keyrow_smoothing_is_transpose(L):
    """The other smoothing axis (smoothing per key row, int8 scales per value
    column; a CPU study only) applied to S equals the path's quantizer
    applied to the transpose of S, transposed, bit for bit: codes, scales,
    boundary state, lines, and each row pick of one is the same-numbered
    column pick of the other.  Random states with outlier lines (no exact
    row/column energy ties), with and without smoothing, C = 0 and 4."""
    rng = np.random.default_rng(17)
    for trial in range(4):
        S = (rng.standard_normal((D, D)) * 10.0 ** rng.uniform(-2, 1, (D, 1))).astype(np.float32)
        S[rng.integers(0, D, 2)] *= np.float32(20.0)
        S[:, rng.integers(0, D, 2)] *= np.float32(15.0)
        C, sm = (4, True) if trial < 2 else ((0, True) if trial == 2 else (4, False))
        Qa, ra, sa, ia, va, Ba = oracle.quantize_axis(S, C, sm, 1e-6, axis="key", L=L)
        Qb, rb, sb, ib, vb, Bb = oracle.quantize_axis(np.ascontiguousarray(S.T), C, sm, 1e-6, axis="value", L=L)
        assert np.array_equal(Qa, Qb.T)
        assert np.array_equal(ra.view(np.uint32), rb.view(np.uint32))
        assert np.array_equal(sa.view(np.uint32), sb.view(np.uint32))
        assert np.array_equal(Ba.view(np.uint32), np.ascontiguousarray(Bb.T).view(np.uint32))
        swap = [(-1 if i < 0 else (i + D if i < D else i - D)) for i in ib]
        assert list(ia) == swap, (list(ia), swap)
        assert np.array_equal(va.view(np.uint32), vb.view(np.uint32))


def pin_greedy_bruteforce(L):
    """Every greedy pick is the float64 argmax of the line energies of the
    matrix left after the earlier picks, unless the top two are within 1e-6."""
    rng = np.random.default_rng(5)
    for trial in range(6):
        R = rng.standard_normal((D, D)).astype(np.float32)
        R[rng.integers(0, D, 3)] *= np.float32(3 + trial)
        R[:, rng.integers(0, D, 3)] *= np.float32(2 + trial)
        h = oracle.Head(C=4, smoothing=bool(trial % 2), L=L).init(R)
        Rw = R.astype(np.float64)
        taken = set()
        for j in range(4):
            e = np.concatenate([(Rw ** 2).sum(axis=1), (Rw ** 2).sum(axis=0)])
            for t in taken:
                e[t] = -1.0
            order = np.argsort(-e, kind="stable")
            top, second = e[order[0]], e[order[1]]
            if (top - second) / top > 1e-6:
                assert h.idx[j] == order[0], (trial, j, h.idx[j], order[:3])
            else:
                assert h.idx[j] in (order[0], order[1])
            pick = int(h.idx[j])
            line = Rw[pick] if pick < D else Rw[:, pick - D]
            assert np.array_equal(h.vec[j], line.astype(np.float32))
            taken.add(pick)
            if pick < D:
                Rw[pick] = 0
            else:
                Rw[:, pick - D] = 0


def pin_reconstruction_bound(L):
    """After quantization every entry is within half a step rho_r*sigma_c of
    the input (plus a few fp32 roundings), and extracted lines come back
    exactly; for the int8 state and the 6- and 4-bit options.  Error budget:
    |code*rho*sigma - R| <= rho*sigma*(0.5 + 1200*2^-24)."""
    S0, _ = tiny_inputs(seed=2, tokens=1, heads=2)
    for sm, bits in ((True, 8), (False, 8), (True, 6), (False, 4), (True, 4)):
        for h_ in range(2):
            R = S0[h_]
            h = oracle.Head(C=4, smoothing=sm, L=L, bits=bits).init(R)
            res = h.dequant(0).astype(np.float64)
            B = h.dequant(1)
            step = h.rho.astype(np.float64)[:, None] * h.sigma.astype(np.float64)[None, :]
            lines = np.zeros((D, D), bool)
            for j, i in enumerate(h.idx):
                if i < 0:
                    continue
                if i < D:
                    lines[i, :] = True
                else:
                    lines[:, i - D] = True
            assert np.array_equal(B[lines], R[lines])
            err = np.abs(res - R.astype(np.float64))
            bound = step * (0.5 + 1200 * 2.0 ** -24)
            assert np.all(err[~lines] <= bound[~lines]), float(np.max(err[~lines] / bound[~lines]))
            assert not np.any(h.Q[lines])


def _window(L, S0, toks, C=4, smoothing=True, W=16):
    """Run one window through the oracle beside the float64 dense recurrence
    from the oracle's own dequantized boundary.  Returns the worst relative
    errors of o, u (per token) and of the state rebuilt at the window end."""
    h = oracle.Head(C=C, W=W, smoothing=smoothing, L=L).init(S0)
    S = h.dequant(1).astype(np.float64)
    eo = eu = 0.0
    for (q, k, v, a, b) in toks[:W]:
        o, u = h.append(q, k, v, a, b)
        u64, o64 = np_gdn_f64(S, q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                              float(a), float(b))
        eo, eu = max(eo, rel(o, o64)), max(eu, rel(u, u64))
    es = rel(h.dequant(2), S)
    return h, eo, eu, es


def pin_window_vs_dense_f64(L):
    """Within a window the windowed path equals the dense recurrence started
    from the dequantized boundary (exact in real arithmetic): o, u and the
    rebuilt state agree to 1e-5 relative."""
    for seed, init in ((0, "gauss"), (1, "prefill"), (4, "hard")):
        S0, toks = tiny_inputs(seed=seed, tokens=16, heads=1, init=init)
        for C, sm in ((4, True), (0, False), (2, True)):
            _, eo, eu, es = _window(L, S0[0], toks, C=C, smoothing=sm)
            assert eo < 1e-5 and eu < 1e-5 and es < 1e-5, (seed, C, sm, eo, eu, es)


def pin_beta_zero(L):
    """beta = 0 writes nothing: u = 0, o_t = gamma_t B^T q and the state at
    the window end is gamma_16 B (to rounding)."""
    S0, toks = tiny_inputs(seed=3, tokens=16)
    h = oracle.Head(C=4, L=L).init(S0[0])
    B = h.dequant(1).astype(np.float64)
    g = 1.0
    for (q, k, v, a, _) in toks:
        o, u = h.append(q, k, v, a, 0.0)
        g = float(np.float32(g * np.float64(a)))
        assert not u.any()
        assert rel(o, g * (B.T @ q.astype(np.float64))) < 1e-6
    assert rel(h.dequant(2), g * B) < 1e-6


def pin_overwrite_identity(L):
    """beta = 1 and q = k with |k| = 1 read back exactly what was written:
    o = (alpha S)^T k + (k.k)(v - (alpha S)^T k) = v."""
    S0, toks = tiny_inputs(seed=6, tokens=16, init="prefill")
    h = oracle.Head(C=4, L=L).init(S0[0])
    for (_, k, v, a, _) in toks:
        k64 = k.astype(np.float64)
        kn = (k64 / np.sqrt(k64 @ k64)).astype(np.float32)
        o, _ = h.append(kn, kn, v, a, 1.0)
        assert rel(o, v) < 2e-5, rel(o, v)


def pin_fold_invariants(L):
    """After a fold the buffer is empty and the current state equals the
    boundary; the fold's new boundary is within the quantization bound of the
    state rebuilt before it."""
    S0, toks = tiny_inputs(seed=8, tokens=16, init="prefill")
    h = oracle.Head(C=4, L=L).init(S0[0])
    for (q, k, v, a, b) in toks:
        h.append(q, k, v, a, b)
    S = h.dequant(2)
    h.fold()
    assert h.n == 0
    assert np.array_equal(h.dequant(2), h.dequant(1))
    step = h.rho.astype(np.float64)[:, None] * h.sigma.astype(np.float64)[None, :]
    err = np.abs(h.dequant(1).astype(np.float64) - S)
    assert np.all(err <= step * (0.5 + 1200 * 2.0 ** -24) + 1e-30)


def pin_xor_equivariance(L):
    """Relabelling key rows (with k and q) or value columns (with v) by
    i -> i XOR m, 0 < m < 64, is an automorphism of the canonical trees, so
    every output and every state field is permuted exactly."""
    S0, toks = tiny_inputs(seed=9, tokens=16, init="prefill")
    S = S0[0]
    for m in (1, 22, 63):
        p = np.arange(D) ^ m
        a = oracle.Head(C=4, L=L).init(S)
        b = oracle.Head(C=4, L=L).init(S[p])
        c = oracle.Head(C=4, L=L).init(S[:, p])
        for (q, k, v, al, be) in toks:
            oa, ua = a.append(q, k, v, al, be)
            ob, ub = b.append(q[p], k[p], v, al, be)
            oc, uc = c.append(q, k, v[p], al, be)
            assert np.array_equal(oa, ob) and np.array_equal(ua, ub)
            assert np.array_equal(oa[p], oc) and np.array_equal(ua[p], uc)
        for h in (a, b, c):
            h.fold()
        assert np.array_equal(a.Q[p], b.Q) and np.array_equal(a.rho[p], b.rho)
        assert np.array_equal(a.sigma, b.sigma)
        assert np.array_equal(a.Q[:, p], c.Q) and np.array_equal(a.sigma[p], c.sigma)
        assert np.array_equal(a.rho, c.rho)
        ia, ib, ic = list(a.idx), list(b.idx), list(c.idx)
        assert ib == [(int(p[i]) if i < D else i) for i in ia]
        assert ic == [(i if i < D else D + int(p[i - D])) for i in ia]


def pin_zero_state(L):
    """An all-zero state has no compensators, zero scales, floor smoothing,
    and the first token reads u = beta v and o = (k.q) u."""
    h = oracle.Head(C=4, sigma_floor=1e-6, L=L).init(np.zeros((D, D), np.float32))
    assert list(h.idx) == [-1] * 4 and not h.vec.any()
    assert not h.rho.any() and not h.Q.any() and np.all(h.sigma == np.float32(1e-6))
    _, toks = tiny_inputs(seed=10, tokens=1)
    q, k, v, a, b = toks[0]
    o, u = h.append(q, k, v, a, b)
    assert rel(u, np.float64(b) * v) < 1e-7
    kq = float(k.astype(np.float64) @ q.astype(np.float64))
    assert rel(o, kq * u.astype(np.float64)) < 1e-6


def pin_tiny_rows(L):
    """A row whose largest magnitude is below 2^-120 is stored as zeros."""
    R = np.zeros((D, D), np.float32)
    R[4, :] = np.float32(2.0 ** -121)
    R[5, :3] = np.float32(1.0)
    h = oracle.Head(C=0, smoothing=False, L=L).init(R)
    assert h.rho[4] == 0 and not h.Q[4].any()
    assert h.rho[5] == np.float32(1.0 / 127.0) and list(h.Q[5, :4]) == [127, 127, 127, 0]


def pin_dense_steps(L):
    """The fp32 and fp64 dense steps match the float64 numpy recurrence, and
    the bf16 step equals the fp32 step on the widened state followed by
    torch's round-to-nearest-even bf16 conversion."""
    S0, toks = tiny_inputs(seed=12, tokens=8, init="prefill")
    S32 = S0[0].copy()
    S64 = S0[0].astype(np.float64)
    Sn = S0[0].astype(np.float64)
    for (q, k, v, a, b) in toks:
        u32, o32 = oracle.gdn_step_f32(S32, q, k, v, a, b, L)
        u64, o64 = oracle.gdn_step_f64(S64, q, k, v, a, b, L)
        un, on = np_gdn_f64(Sn, q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                            float(np.float32(a)), float(np.float32(b)))
        assert rel(o32, on) < 1e-5 and rel(u32, un) < 1e-5
        assert rel(o64, on) < 1e-12 and rel(u64, un) < 1e-12
    Sb = torch.from_numpy(S0[0]).to(torch.bfloat16)
    bits = Sb.view(torch.int16).numpy().view(np.uint16).copy()
    Sw = Sb.to(torch.float32).numpy().copy()
    q, k, v, a, b = toks[0]
    ub, ob = oracle.gdn_step_bf16(bits, q, k, v, a, b, L)
    uw, ow = oracle.gdn_step_f32(Sw, q, k, v, a, b, L)
    assert np.array_equal(ob, ow) and np.array_equal(ub, uw)
    want = torch.from_numpy(Sw).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, want)


def pin_window_one(L):
    """W=1 quantizes after every token: each fold's input state equals the
    dense step from the previous boundary."""
    S0, toks = tiny_inputs(seed=13, tokens=4, init="prefill")
    h = oracle.Head(C=4, W=1, L=L).init(S0[0])
    for (q, k, v, a, b) in toks:
        S = h.dequant(1).astype(np.float64)
        o, u = h.append(q, k, v, a, b)
        _, o64 = np_gdn_f64(S, q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                            float(a), float(b))
        assert rel(o, o64) < 1e-5
        assert rel(h.dequant(2), S) < 1e-5
        h.fold()


def _ulps(a, b):
    """Distance in fp32 units in the last place (same-sign finite values)."""
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


def pin_gate_closed_forms(L):
    """Gate arithmetic against closed forms: softplus(0) = ln 2, so A = 1 and
    x = 0 give alpha = 1/2 and A = 2 gives 1/4; sigmoid(0) = 1/2 and
    sigmoid(-b) = 1 - sigmoid(b); large x make softplus(x) = x, very negative
    x make alpha round to 1; alpha falls as a grows.  Random arguments agree
    within one ulp with numpy's float64 logaddexp / exp, a different route to
    the same functions."""
    assert oracle.gate(0.0, 0.0, 0.0, 0.0, L) == (np.float32(0.5), np.float32(0.5))
    al, _ = oracle.gate(0.0, 0.0, np.float32(np.log(2.0)), 0.0, L)
    assert _ulps(al, np.float32(0.25)) <= 1
    al, _ = oracle.gate(30.0, 0.0, -3.0, 0.0, L)
    assert _ulps(al, np.float32(np.exp(-np.exp(-3.0) * 30.0))) <= 1
    al, be = oracle.gate(-40.0, 40.0, 2.0, 0.0, L)
    assert al == np.float32(1.0) and be == np.float32(1.0)
    al, _ = oracle.gate(0.5, 0.0, 0.0, -0.5, L)  # dt_bias shifts a
    assert al == np.float32(0.5)
    rng = np.random.default_rng(7)
    prev = 2.0
    for a in np.linspace(-6, 6, 49, dtype=np.float32):
        al, _ = oracle.gate(a, 0.0, 0.3, -1.0, L)
        assert al <= prev
        prev = al
    for _ in range(200):
        a, b, Al, dt = (np.float32(x) for x in rng.normal(0, 3, 4))
        al, be = oracle.gate(a, b, Al, dt, L)
        x = np.float64(a) + np.float64(dt)
        want_a = np.float32(np.exp(-np.exp(np.float64(Al)) * np.logaddexp(0.0, x)))
        want_b = np.float32(1.0 / (1.0 + np.exp(-np.float64(b))))
        assert _ulps(al, want_a) <= 1 and _ulps(be, want_b) <= 1, (a, b, Al, dt, al, want_a, be, want_b)
        _, be_neg = oracle.gate(a, -b, Al, dt, L)
        assert abs(np.float64(be) + np.float64(be_neg) - 1.0) <= 2.0 ** -23


def pin_l2norm(L):
    """L2 normalization: a power-of-two multiple of a unit vector comes back
    exactly; random vectors get unit norm to rounding and match x / |x| in
    float64 within 2 ulp; the scale applies after the normalization (exactly
    the unscaled result times the scale); eps sits under the root (a vector
    far below sqrt(eps) is divided by sqrt(eps), the zero vector stays 0)."""
    e = np.zeros(D, np.float32)
    e[37] = -8.0
    out = oracle.l2norm(e, 0.0, 1.0, L)
    assert out[37] == -1.0 and np.count_nonzero(out) == 1
    rng = np.random.default_rng(11)
    x = rng.normal(0, 3, D).astype(np.float32)
    u = oracle.l2norm(x, 0.0, 1.0, L)
    assert abs(np.linalg.norm(u.astype(np.float64)) - 1.0) < 1e-6
    want = (x.astype(np.float64) / np.linalg.norm(x.astype(np.float64))).astype(np.float32)
    assert np.max(_ulps(u, want)) <= 2
    s = np.float32(128 ** -0.5)
    assert np.array_equal(oracle.l2norm(x, 1e-6, s, L), oracle.l2norm(x, 1e-6, 1.0, L) * s)
    tiny = np.full(D, 1e-6, np.float32)
    got = oracle.l2norm(tiny, 1e-6, 1.0, L)
    assert rel(got, tiny.astype(np.float64) / np.sqrt(1e-6 + 128e-12)) < 1e-5
    assert not np.any(oracle.l2norm(np.zeros(D, np.float32), 1e-6, 1.0, L))


def pin_gated_window(L):
    """A window driven through the gate arithmetic equals the dense float64
    recurrence on the same gated inputs (normalized in float64) to 1e-5."""
    rng = np.random.default_rng(21)
    S0 = (rng.normal(0, 0.02, (D, D))).astype(np.float32)
    h = oracle.Head(C=4, W=16, L=L).init(S0)
    S = h.dequant(1).astype(np.float64)
    A_log, dt_bias = np.float32(np.log(4.0)), np.float32(-4.0)
    for t in range(16):
        q, k, v = (rng.normal(0, 1, D).astype(np.float32) for _ in range(3))
        a, b = (np.float32(x) for x in rng.normal(0, 1, 2))
        gq, gk, gv, al, be = oracle.gated_inputs(q, k, v, a, b, A_log, dt_bias, q_scale=0.125, L=L)
        o, _ = h.append(gq, gk, gv, al, be)
        q64 = q.astype(np.float64) / np.sqrt(np.sum(q.astype(np.float64) ** 2) + 1e-6) * 0.125
        k64 = k.astype(np.float64) / np.sqrt(np.sum(k.astype(np.float64) ** 2) + 1e-6)
        x = np.float64(a) + np.float64(dt_bias)
        al64 = np.exp(-np.exp(np.float64(A_log)) * np.logaddexp(0.0, x))
        be64 = 1.0 / (1.0 + np.exp(-np.float64(b)))
        _, o64 = np_gdn_f64(S, q64, k64, v.astype(np.float64), al64, be64)
        assert rel(o, o64) < 1e-5, (t, rel(o, o64))


def _kda_tokens(rng, T, spread=1.0):
    toks = []
    for _ in range(T):
        q = rng.normal(0, 1, D)
        k = rng.normal(0, 1, D)
        q, k = (x / np.linalg.norm(x) for x in (q, k))
        v = rng.normal(0, 1, D)
        alpha = np.exp(-np.logaddexp(0.0, rng.normal(-3.0, spread, D)))
        beta = 1.0 / (1.0 + np.exp(-rng.normal()))
        toks.append(tuple(np.float32(x) if np.ndim(x) == 0 else x.astype(np.float32)
                          for x in (q, k, v, alpha, beta)))
    return toks


def pin_kda_window_vs_dense_f64(L):
    """Per-channel decay ([LQ] App. A, D_t = Diag(alpha_t)): a window of
    appends equals the float64 dense recurrence with row-wise decay from the
    dequantized boundary (outputs and the rebuilt state to 1e-5), and the
    fold leaves an empty buffer whose boundary is the quantized state."""
    S0, _ = tiny_inputs(seed=31, tokens=1, init="gauss")
    rng = np.random.default_rng(31)
    h = oracle.Head(C=4, W=16, L=L, decay="channel").init(S0[0])
    S = h.dequant(1).astype(np.float64)
    for (q, k, v, a, b) in _kda_tokens(rng, 16, spread=1.5):
        o, u = h.append(q, k, v, a, b)
        S *= a.astype(np.float64)[:, None]
        r = S.T @ k.astype(np.float64)
        u64 = float(b) * (v.astype(np.float64) - r)
        S += np.outer(k.astype(np.float64), u64)
        o64 = S.T @ q.astype(np.float64)
        assert rel(o, o64) < 1e-5 and rel(u, u64) < 1e-5
    cur = h.dequant(2)
    assert rel(cur, S) < 1e-5
    want = oracle.quantize(cur, C=4, L=L)
    h.fold()
    assert h.n == 0 and np.array_equal(h.Q, want.Q) and np.array_equal(h.idx, want.idx)
    assert np.array_equal(h.dequant(2), h.dequant(1))


def pin_kda_uniform_is_gdn(L):
    """With the same decay on every channel, per-channel decay is the scalar
    (GDN) decay: the dense steps agree bit for bit, and the windowed paths,
    which round in different orders, agree to 1e-6."""
    S0, _ = tiny_inputs(seed=32, tokens=1, init="gauss")
    rng = np.random.default_rng(32)
    hk = oracle.Head(C=4, W=16, L=L, decay="channel").init(S0[0])
    hg = oracle.Head(C=4, W=16, L=L).init(S0[0])
    Sk = hk.dequant(1)
    Sg = Sk.copy()
    for (q, k, v, a, b) in _kda_tokens(rng, 16):
        a0 = np.float32(a[0])
        ok, _ = hk.append(q, k, v, np.full(D, a0, np.float32), b)
        og, _ = hg.append(q, k, v, a0, b)
        assert rel(ok, og) < 1e-6
        uk, dk = oracle.kda_step_f32(Sk, q, k, v, np.full(D, a0, np.float32), b, L)
        ug, dg = oracle.gdn_step_f32(Sg, q, k, v, a0, b, L)
        assert np.array_equal(dk, dg) and np.array_equal(uk, ug) and np.array_equal(Sk, Sg)
    assert rel(hk.dequant(2), hg.dequant(2)) < 1e-6


def pin_kda_dense_step(L):
    """The fp32 dense KDA step against numpy float64 (row-wise decay)."""
    rng = np.random.default_rng(33)
    S = rng.normal(0, 0.1, (D, D)).astype(np.float32)
    S64 = S.astype(np.float64)
    for (q, k, v, a, b) in _kda_tokens(rng, 8, spread=2.0):
        u, o = oracle.kda_step_f32(S, q, k, v, a, b, L)
        S64 *= a.astype(np.float64)[:, None]
        u64 = float(b) * (v.astype(np.float64) - S64.T @ k.astype(np.float64))
        S64 += np.outer(k.astype(np.float64), u64)
        assert rel(u, u64) < 1e-5 and rel(o, S64.T @ q.astype(np.float64)) < 1e-5
    assert rel(S, S64) < 1e-5


def pin_bf16_records(L):
    """Records whose corrections are kept in bf16: the token that makes a
    record reads out with its fp32 u (outputs equal to the fp32-record path
    until then), the stored u is that u rounded to nearest even in bf16
    (torch's conversion as the independent reference), every stored value is
    bf16, and a window stays within bf16 rounding of the float64 dense
    recurrence."""
    S0, toks = tiny_inputs(seed=41, tokens=16, init="gauss")
    hf = oracle.Head(C=4, W=16, L=L).init(S0[0])
    hb = oracle.Head(C=4, W=16, L=L, rec_u="bf16").init(S0[0])
    S = hb.dequant(1).astype(np.float64)
    for t, (q, k, v, a, b) in enumerate(toks):
        of, uf = hf.append(q, k, v, a, b)
        ob, ub = hb.append(q, k, v, a, b)
        if t == 0:
            assert np.array_equal(of, ob)
            want = torch.from_numpy(uf).to(torch.bfloat16).float().numpy()
            assert np.array_equal(ub, want)
        assert not np.any(ub.view(np.uint32) & 0xFFFF)
        _, o64 = np_gdn_f64(S, q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                            float(a), float(b))
        assert rel(ob, o64) < 5e-3
    assert rel(hb.dequant(2), S) < 5e-3


def _torch_e4m3(x):
    """torch's float8_e4m3fn rounding of fp32 values, as (codes uint8, values fp32)."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy(), t.float().numpy()


def pin_fp8_codec(L):
    """The oracle's E4M3 codec against torch's float8_e4m3fn: the value of
    every code (NaN codes aside, -0 included), and the code of every
    representable value, of every midpoint between neighbours (ties go to
    the even code) and of the floats next to those midpoints, of random
    values over every binade up to 448, and of fp32 subnormals."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    got = np.array([L.lqo_e4m3_to_f32(int(c)) for c in codes], np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    pos = np.unique(want[want > 0]).astype(np.float64)
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    near = np.concatenate([np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    rng = np.random.default_rng(23)
    rnd = (rng.uniform(1, 2, 4000) * 2.0 ** rng.integers(-12, 8, 4000)).astype(np.float32)
    sub = (rng.integers(1, 1 << 23, 200) * 2.0 ** -149).astype(np.float32)
    x = np.concatenate([pos.astype(np.float32), mids, near, rnd, sub, [np.float32(448.0), np.float32(0.0)]])
    x = np.concatenate([x, -x])
    wc, _ = _torch_e4m3(x)
    gc = np.array([L.lqo_f32_to_e4m3(float(v)) for v in x], np.uint8)
    bad = np.flatnonzero(gc != wc)
    assert bad.size == 0, (x[bad[:5]], gc[bad[:5]], wc[bad[:5]])


def pin_fp8_records(L):
    """Records whose corrections are kept in fp8: the token that makes a
    record reads out with its fp32 u; the stored u of each group of 32
    value columns (c % 4 = j) is torch's E4M3 rounding of u / s times s, with
    s a power of two that puts the group's largest magnitude in (224, 448]
    (or 2^-126 for a group that small); a window stays within fp8 rounding
    of the float64 dense recurrence."""
    S0, toks = tiny_inputs(seed=43, tokens=16, init="gauss")
    hf = oracle.Head(C=4, W=16, L=L).init(S0[0])
    h8 = oracle.Head(C=4, W=16, L=L, rec_u="fp8").init(S0[0])
    S = h8.dequant(1).astype(np.float64)
    worst = 0.0
    for t, (q, k, v, a, b) in enumerate(toks):
        of, uf = hf.append(q, k, v, a, b)
        o8, u8 = h8.append(q, k, v, a, b)
        if t == 0:
            assert np.array_equal(of, o8)
        # the record as h8 made it: its fp32 u is that of a twin of h8 with
        # fp32 records up to this token
        twin = h8.copy()
        twin.n -= 1
        twin.rec_u = "f32"
        _, u32 = twin.append(q, k, v, a, b)
        for j in range(4):
            g = u32[j::4]
            M = float(np.max(np.abs(g)))
            e = int(np.floor(np.log2(M / 224.0)))
            sc = [2.0 ** (e + d) for d in (-1, 0, 1) if 224.0 * 2.0 ** (e + d) < M <= 448.0 * 2.0 ** (e + d)]
            assert len(sc) == 1, (M, e)
            sc = np.float32(sc[0])
            _, want = _torch_e4m3(g / sc)
            assert np.array_equal(u8[j::4], (want * sc).astype(np.float32)), (t, j)
        _, o64 = np_gdn_f64(S, q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                            float(a), float(b))
        worst = max(worst, rel(o8, o64))
    assert worst < 0.05, worst
    assert rel(h8.dequant(2), S) < 0.05


def pin_rank1_fit(L):
    """Rank-one compensators by power sweeps: the start is the fp64 argmax
    row energy; after 8 sweeps a and b equal float64 power iteration from
    that row to 1e-5; a has unit norm; a planted rank-one pattern is
    captured (cosine > 0.99999) and the state is rebuilt from residual and
    pairs within half an int8 step per entry."""
    rng = np.random.default_rng(51)
    u, v = rng.normal(size=D), rng.normal(size=D)
    S = (3.0 * np.outer(u, v) + rng.normal(0, 0.05, (D, D))).astype(np.float32)
    h = oracle.quantize(S, C=4, L=L, fit="rank1")
    R = S.astype(np.float64)
    for j in range(4):
        a_j, b_j = h.vec[j, :D].astype(np.float64), h.vec[j, D:].astype(np.float64)
        energy = np.sum(R * R, axis=1)
        top = np.sort(energy)[::-1]
        if top[0] - top[1] > 1e-6 * top[0]:
            assert h.idx[j] == int(np.argmax(energy)), (j, h.idx[j])
        b = R[h.idx[j]].copy()
        for _ in range(8):
            a = R @ b
            a /= np.linalg.norm(a)
            b = R.T @ a
        assert rel(a_j, a) < 1e-5 and rel(b_j, b) < 1e-5, (j, rel(a_j, a), rel(b_j, b))
        assert abs(np.linalg.norm(a_j) - 1.0) < 1e-6
        R = R - np.outer(a_j, b_j)
    a0, b0 = h.vec[0, :D].astype(np.float64), h.vec[0, D:].astype(np.float64)
    assert abs(a0 @ u) / np.linalg.norm(u) > 0.99999
    assert abs(b0 @ v) / (np.linalg.norm(b0) * np.linalg.norm(v)) > 0.99999
    B = h.dequant(1).astype(np.float64)
    step = np.outer(h.rho, h.sigma).astype(np.float64)
    assert np.all(np.abs(B - S) <= 0.5 * step * (1 + 1e-5) + 1e-6 * np.abs(S).max())


def pin_rank1_window_and_fold(L):
    """A window with rank-one compensators equals the float64 dense
    recurrence from its boundary to 1e-5; the fold equals fitting and
    quantizing the current state, leaves an empty buffer, and the boundary
    then equals the current state."""
    S0, toks = tiny_inputs(seed=52, tokens=16, init="gauss")
    h = oracle.Head(C=4, W=16, L=L, fit="rank1").init(S0[0])
    S = h.dequant(1).astype(np.float64)
    for (q, k, v, a, b) in toks:
        o, _ = h.append(q, k, v, a, b)
        _, o64 = np_gdn_f64(S, q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                            float(a), float(b))
        assert rel(o, o64) < 1e-5
    cur = h.dequant(2)
    assert rel(cur, S) < 1e-5
    want = oracle.quantize(cur, C=4, L=L, fit="rank1")
    h.fold()
    assert h.n == 0 and np.array_equal(h.Q, want.Q) and np.array_equal(h.vec, want.vec)
    assert np.array_equal(h.dequant(2), h.dequant(1))


def pin_rank1_zero_state(L):
    """An all-zero state: no start row, zero pairs, zero codes."""
    h = oracle.quantize(np.zeros((D, D), np.float32), C=4, L=L, fit="rank1")
    assert list(h.idx[:4]) == [-1] * 4 and not np.any(h.vec) and not np.any(h.Q)


def _mgs64(Y):
    """Modified Gram-Schmidt in float64 over the rows of Y (slot order)."""
    A = np.array(Y, np.float64)
    for j in range(A.shape[0]):
        for i in range(j):
            A[j] -= (A[i] @ A[j]) * A[i]
        A[j] /= np.linalg.norm(A[j])
    return A


def pin_block_start_rows(L):
    """Block fit, cold start with no sweep: the slots start from the unit
    vectors of the rows in decreasing canonical energy, so the pairs are
    exactly those rows (a = e_r, b = R[r, :]), deflation zeroes exactly
    those rows and leaves the rest bitwise unchanged, and rows of zero
    energy are never a start."""
    rng = np.random.default_rng(61)
    R = rng.normal(0, 1, (D, D)).astype(np.float32)
    R[[5, 90, 17]] *= np.float32(8.0)
    R[[33, 34]] = 0.0
    Rd, idx, ab = oracle.fit_block(R, C=4, sweeps=0, L=L)
    energy = (R.astype(np.float64) ** 2).sum(1)
    order = list(np.argsort(-energy, kind="stable")[:4])
    assert list(idx[:4]) == [0, 1, 2, 3]
    for j, r in enumerate(order):
        e = np.zeros(D, np.float32)
        e[r] = 1.0
        assert np.array_equal(ab[j, :D], e) and np.array_equal(ab[j, D:], R[r]), j
    keep = np.ones(D, bool)
    keep[order] = False
    assert not np.any(Rd[order]) and np.array_equal(Rd[keep], R[keep])
    # a state with two nonzero rows: the other two slots stay unused
    Z = np.zeros((D, D), np.float32)
    Z[3], Z[70] = rng.normal(size=D), 2 * rng.normal(size=D)
    _, idx2, ab2 = oracle.fit_block(Z, C=4, sweeps=0, L=L)
    assert list(idx2[:4]) == [0, 1, -1, -1] and not np.any(ab2[2:])
    assert ab2[0, 70] == 1.0 and ab2[1, 3] == 1.0


def pin_block_fit_svd(L):
    """With many sweeps the block fit converges to the leading singular
    subspace: the pairs' sum equals the best rank-4 approximation (SVD,
    Eckart-Young) to 1e-4 relative, a is orthonormal to 1e-5, and the
    deflated matrix is the SVD tail."""
    rng = np.random.default_rng(62)
    U, _ = np.linalg.qr(rng.normal(size=(D, D)))
    V, _ = np.linalg.qr(rng.normal(size=(D, D)))
    s = np.concatenate([[40.0, 25.0, 15.0, 9.0], 1.0 / (1 + np.arange(D - 4))])
    R = ((U * s) @ V.T).astype(np.float32)
    Rd, idx, ab = oracle.fit_block(R, C=4, sweeps=60, L=L)
    A, B = ab[:4, :D].astype(np.float64), ab[:4, D:].astype(np.float64)
    assert list(idx[:4]) == [0, 1, 2, 3]
    assert np.abs(A @ A.T - np.eye(4)).max() < 1e-5
    u, sv, vt = np.linalg.svd(R.astype(np.float64))
    best = (u[:, :4] * sv[:4]) @ vt[:4]
    assert rel(A.T @ B, best) < 1e-4, rel(A.T @ B, best)
    assert rel(Rd, R.astype(np.float64) - best) < 1e-3


def pin_block_fit_steps(L):
    """Two warm-started sweeps equal float64 subspace iteration with
    modified Gram-Schmidt from the stored a's (z = R^T a, y = R z, then
    orthonormalize), followed by b = R^T a, to 1e-5."""
    rng = np.random.default_rng(63)
    R = (rng.normal(size=(D, D)) + 4 * np.outer(rng.normal(size=D), rng.normal(size=D))).astype(np.float32)
    start = _mgs64(rng.normal(size=(4, D))).astype(np.float32)
    ab0 = np.zeros((4, 2 * D), np.float32)
    ab0[:, :D] = start
    _, idx, ab = oracle.fit_block(R, C=4, idx=[0, 1, 2, 3], ab=ab0, warm=True, sweeps=2, L=L)
    R64 = R.astype(np.float64)
    A = _mgs64(start)
    for _ in range(2):
        A = _mgs64((R64 @ (R64.T @ A.T)).T)
    B = (R64.T @ A.T).T
    assert rel(ab[:4, :D], A) < 1e-5 and rel(ab[:4, D:], B) < 1e-5, (rel(ab[:4, :D], A), rel(ab[:4, D:], B))
    # a cold start from the same matrix differs (the start is the longest rows)
    _, _, abc = oracle.fit_block(R, C=4, sweeps=2, L=L)
    assert not np.array_equal(abc, ab)


def pin_block_warm_fixed_point(L):
    """A state that is exactly rank 4 in the span of the stored a's is
    captured by one warm sweep: the fitted a's span the stored ones (their
    4 x 4 matrix of cosines is orthogonal) and the deflated state is zero to
    1e-5 of its scale."""
    rng = np.random.default_rng(64)
    A0 = _mgs64(rng.normal(size=(4, D)))
    Vb = rng.normal(size=(4, D)) * np.array([[30.0], [12.0], [5.0], [2.0]])
    R = (A0.T @ Vb).astype(np.float32)
    ab0 = np.zeros((4, 2 * D), np.float32)
    ab0[:, :D] = A0.astype(np.float32)
    Rd, idx, ab = oracle.fit_block(R, C=4, idx=[0, 1, 2, 3], ab=ab0, warm=True, sweeps=1, L=L)
    P = ab[:4, :D].astype(np.float64) @ A0.T  # cosines between fitted and stored bases
    assert np.abs(P @ P.T - np.eye(4)).max() < 1e-5
    assert np.abs(Rd).max() < 1e-5 * np.abs(R).max()


def pin_block_zero_state(L):
    """An all-zero state: no start row, unused pairs, zero codes."""
    h = oracle.quantize(np.zeros((D, D), np.float32), C=4, L=L, fit="block")
    assert list(h.idx[:4]) == [-1] * 4 and not np.any(h.vec) and not np.any(h.Q)


def pin_block_window_and_fold(L):
    """With block pairs a window equals the float64 dense recurrence from
    its boundary to 1e-5 (the read is the rank-one read); the fold equals
    the block fit of the current state warm-started from the window's own
    pairs, followed by smoothing and rounding; the buffer is then empty."""
    S0, toks = tiny_inputs(seed=65, tokens=16, init="gauss")
    h = oracle.Head(C=4, W=16, L=L, fit="block").init(S0[0])
    assert list(h.idx[:4]) == [0, 1, 2, 3]
    S = h.dequant(1).astype(np.float64)
    for (q, k, v, a, b) in toks:
        o, _ = h.append(q, k, v, a, b)
        _, o64 = np_gdn_f64(S, q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                            float(a), float(b))
        assert rel(o, o64) < 1e-5
    cur = h.dequant(2)
    assert rel(cur, S) < 1e-5
    Rd, idx, ab = oracle.fit_block(cur, C=4, idx=h.idx, ab=h.vec, warm=True, sweeps=2, L=L)
    cold = oracle.quantize(cur, C=4, L=L, fit="block")
    h.fold()
    assert h.n == 0 and np.array_equal(h.vec, ab) and np.array_equal(h.idx, idx)
    assert not np.array_equal(h.vec, cold.vec)
    res = h.dequant(0).astype(np.float64)
    step = np.outer(h.rho, h.sigma).astype(np.float64)
    assert np.all(np.abs(res - Rd) <= 0.5 * step * (1 + 1e-5) + 1e-6 * np.abs(Rd).max())
    assert np.array_equal(h.dequant(2), h.dequant(1))


ALL = [
    pin_t128_fixtures, pin_t128_exact_integers, pin_round_half_even, pin_round_exact_product_once, pin_pick_ties,
    pin_textbook_int8, pin_smoothing_closed_form, pin_scaling_exact, pin_planted_outliers,
    pin_planted_prefill_lines, pin_keyrow_smoothing_is_transpose,
    pin_greedy_bruteforce, pin_reconstruction_bound, pin_window_vs_dense_f64, pin_beta_zero,
    pin_overwrite_identity, pin_fold_invariants, pin_xor_equivariance, pin_zero_state,
    pin_tiny_rows, pin_dense_steps, pin_window_one, pin_gate_closed_forms, pin_l2norm, pin_gated_window,
    pin_kda_window_vs_dense_f64, pin_kda_uniform_is_gdn, pin_kda_dense_step, pin_bf16_records,
    pin_fp8_codec, pin_fp8_records, pin_low_bit_textbook, pin_low_bit_planted, pin_low_bit_window,
    pin_rank1_fit, pin_rank1_window_and_fold, pin_rank1_zero_state,
    pin_block_start_rows, pin_block_fit_svd, pin_block_fit_steps, pin_block_warm_fixed_point,
    pin_block_zero_state, pin_block_window_and_fold,
]
