"""Host-side checks of the C ABI (no GPU): symbols, layout, validation.

Every call here returns before any HIP call (validation failures and the
host-only layout query), so it runs on a machine without a GPU.
"""
import ctypes
import os
import re

import pytest

from quantized_recurrent_state_amd import leapq as lq
from quantized_recurrent_state_amd import metrics
from tests.pins import golden

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # a 256-byte-aligned address that is never dereferenced
HEADER = os.path.join(ROOT, "include", "leapq.h")


def header_functions():
    text = open(os.path.join(ROOT, "include", "leapq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(leapq_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = header_functions()
    assert set(names) == set(lq.SYMBOLS), names
    L = lq.lib()
    for n in names:
        assert hasattr(L, n), n


def test_probe_library_loads():
    """The measurement probes (libleapq_probe.so, and libleapq_probe_agpr.so
    for the co-execution probe with AGPR accumulators) are built beside the
    library and export their entry points; a call with invalid arguments
    returns hipErrorInvalidValue (1) before any HIP call."""
    from quantized_recurrent_state_amd import profiling
    P = profiling.probe_lib()
    us = ctypes.c_float()
    assert P.lqp_append_pattern(0, 4, 16, 2, 512, 0, 10, ctypes.byref(us)) == 1
    assert P.lqp_append_pattern(16, 4, 16, 2, 512, 16, 10, ctypes.byref(us)) == 1  # n >= W
    assert P.lqp_append_pattern(16, 4, 16, 2, 100, 0, 10, ctypes.byref(us)) == 1   # not 16-byte pieces
    assert P.lqp_read_ceiling(0, 10, ctypes.byref(us)) == 1
    for agpr in (False, True):
        Q = profiling.probe_lib(agpr)
        assert Q.lqp_coexec(3, 0, 10, ctypes.byref(us)) == 1  # no mode 3
        assert Q.lqp_coexec(2, 70000, 10, ctypes.byref(us)) == 1  # more LDS than a workgroup gets


PAGE_TITLES = ("Recurrent-state quantization for linear attention", "LeapQuant")


def test_declarations_cite_pages():
    """Every entry point of include/leapq.h is preceded by a comment that
    names the page defining its operation, except the two utilities
    (status strings and the version), whose comments say they have none."""
    import re
    text = open(HEADER).read()
    decls = list(re.finditer(r"\n(?:int32_t|const char \*)\s*(leapq_\w+)\(", text))
    assert {m.group(1) for m in decls} == set(lq.SYMBOLS)
    for m in decls:
        before = text[:m.start() + 1]
        start = before.rfind("/*")
        end = before.rfind("*/")
        assert 0 <= start < end, m.group(1)
        between = before[end + 2:]
        assert not between.strip(), f"{m.group(1)}: no comment right above the declaration"
        comment = " ".join(re.sub(r"\n\s*\*", " ", before[start:end]).split())
        if m.group(1) in ("leapq_status_str", "leapq_version"):
            assert "no passage" in comment, m.group(1)
        else:
            assert any(t in comment for t in PAGE_TITLES), f"{m.group(1)} cites no page: {comment[:120]}"


def test_version_and_status_strings():
    assert lq.leapq_version() == 100
    for st in range(0, -8, -1):
        s = lq.status_str(st)
        assert s and s != "unknown status", st
    assert lq.status_str(-99) == "unknown status"


def layout(**kw):
    return lq.leapq_query_layout(lq.make_config(**kw))


def test_layout_sections_aligned_and_disjoint():
    for (B, H, W, C, dt) in ((1, 4, 16, 4, "f32"), (512, 32, 16, 4, "bf16"), (3, 5, 1, 0, "bf16"),
                             (2, 7, 64, 8, "f32")):
        L = layout(batch=B, heads=H, window=W, n_comp=C, in_dtype=dt)
        heads = B * H
        e = 2 if dt == "bf16" else 4  # record keys are stored in the input dtype
        secs = [("off_codes", heads * 128 * 128), ("off_row_scale", heads * 512), ("off_col_scale", heads * 512),
                ("off_comp_idx", heads * C * 4), ("off_comp_vec", heads * C * 512),
                ("off_rec_gamma", heads * W * 4), ("off_rec_k", heads * W * 128 * e), ("off_rec_u", heads * W * 512)]
        end = 0
        for name, size in secs:
            off = getattr(L, name)
            assert off % 256 == 0 and off >= end, (name, off, end)
            end = off + size
        assert L.total_bytes >= end and L.total_bytes % 256 == 0
        assert L.boundary_bytes_per_head == metrics.boundary_bytes(C)
        assert L.record_bytes_per_head == W * metrics.record_bytes(e)


def test_layout_matches_page_figures():
    g = golden("page_figures.json")
    L = layout(batch=1, heads=1)
    bpe = L.boundary_bytes_per_head / (128 * 128)
    f = g["boundary_bytes_per_element"]
    assert abs(bpe - f["value"]) <= f["printed_digits_tol"], bpe
    assert abs(f["fp32_bytes_per_element"] / bpe - f["storage_ratio"]) <= f["ratio_tol"]
    r = g["fp32_state_bytes_per_request"]
    s = r["shape"]
    fp32 = s["layers"] * s["heads"] * s["dk"] * s["dv"] * s["bytes_per_number"]
    assert abs(fp32 - r["value"]) <= r["printed_digits_tol"], fp32
    e = g["gpu_entries_matched"]
    assert e["folds"] * e["heads"] * e["entries_per_head"] == e["value"]
    assert e["entries_per_head"] == 128 * 128
    d = g["defaults"]
    assert (lq.make_config(1, 1).window, lq.make_config(1, 1).n_comp) == (d["window"], d["n_comp"])


def test_step_definition_matches_page():
    s = golden("page_figures.json")["step_definition"]
    step = metrics.step_ms(s["append_ms"], s["fold_extra_ms"], s["window"])
    assert abs(step - s["table_step_ms"]) <= s["tol_ms"], step
    budget = metrics.fold_budget_ms(s["append_ms"], s["window_kernel_ms"], s["window"])
    assert abs(budget - s["fold_budget_ms"]) <= s["budget_tol_ms"], budget


def test_bytes_model_values():
    # one head, bf16 inputs (bf16 record keys), W=16, C=4
    assert metrics.record_bytes() == 4 + 256 + 512
    assert metrics.append_bytes(0) == 21532
    assert sum(metrics.append_bytes(n) for n in range(16)) / 16 == 27322
    assert metrics.fold_bytes(16) == 51296
    assert metrics.window_bytes() / 16 == 30528
    # fp32 inputs: fp32 keys, 1,028-byte records
    assert metrics.append_bytes(0, in_bytes=4) == 22556
    assert metrics.fold_bytes(16, in_bytes=4) == 55392
    assert metrics.gdn_step_bytes(4) == 132360 and metrics.gdn_step_bytes(2) == 66824


# ---------------------------------------------------------------- validation

def cfg(**kw):
    base = dict(batch=2, heads=4, window=16, n_comp=4, smoothing=True, sigma_floor=1e-6, in_dtype="f32")
    base.update(kw)
    return lq.make_config(**base)


def fake_layer(c, n=0, state=FAKE):
    L = lq.leapq_layer()
    L.cfg = c
    L.state = state
    L.n_records = n
    return L


def call_append(L, q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, o=FAKE):
    vp = ctypes.c_void_p
    return lq.lib().leapq_append(ctypes.byref(L), vp(q), vp(k), vp(v), vp(a), vp(b), vp(o), None)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), lq.LEAPQ_ERR_RANGE), (dict(heads=0), lq.LEAPQ_ERR_RANGE),
    (dict(window=0), lq.LEAPQ_ERR_RANGE), (dict(window=65), lq.LEAPQ_ERR_RANGE),
    (dict(n_comp=-1), lq.LEAPQ_ERR_RANGE), (dict(n_comp=9), lq.LEAPQ_ERR_RANGE),
    (dict(sigma_floor=0.0), lq.LEAPQ_ERR_RANGE), (dict(sigma_floor=float("nan")), lq.LEAPQ_ERR_RANGE),
])
def test_config_ranges(kw, status):
    c = cfg(**kw)
    assert lq.lib().leapq_query_layout(ctypes.byref(c), ctypes.byref(lq.leapq_layout())) == status
    L = fake_layer(c)
    assert call_append(L) == status and L.n_records == 0


def test_config_shape_dtype_reserved():
    L_out = lq.leapq_layout()
    c = cfg()
    c.dk = 64
    assert lq.lib().leapq_query_layout(ctypes.byref(c), ctypes.byref(L_out)) == lq.LEAPQ_ERR_SHAPE
    c = cfg()
    c.in_dtype = 7
    assert lq.lib().leapq_query_layout(ctypes.byref(c), ctypes.byref(L_out)) == lq.LEAPQ_ERR_DTYPE
    c = cfg()
    c.smoothing = 2
    assert lq.lib().leapq_query_layout(ctypes.byref(c), ctypes.byref(L_out)) == lq.LEAPQ_ERR_RANGE
    c = cfg()
    c.rec_dtype = 5
    assert lq.lib().leapq_query_layout(ctypes.byref(c), ctypes.byref(L_out)) == lq.LEAPQ_ERR_DTYPE
    c = cfg()
    c.decay = 2
    assert lq.lib().leapq_query_layout(ctypes.byref(c), ctypes.byref(L_out)) == lq.LEAPQ_ERR_RANGE
    c = cfg(decay="channel", qk_norm=True)  # channel decay excludes normalized keys
    assert lq.lib().leapq_query_layout(ctypes.byref(c), ctypes.byref(L_out)) == lq.LEAPQ_ERR_RANGE
    assert lq.lib().leapq_query_layout(None, ctypes.byref(L_out)) == lq.LEAPQ_ERR_NULL
    assert lq.lib().leapq_query_layout(ctypes.byref(cfg()), None) == lq.LEAPQ_ERR_NULL


def test_append_pointer_checks():
    c = cfg()
    assert call_append(fake_layer(c, state=0)) == lq.LEAPQ_ERR_NULL
    assert call_append(fake_layer(c, state=FAKE + 16)) == lq.LEAPQ_ERR_ALIGN
    for key in ("q", "k", "v", "a", "b", "o"):
        assert call_append(fake_layer(c), **{key: 0}) == lq.LEAPQ_ERR_NULL, key
    for key in ("q", "k", "v", "o"):
        assert call_append(fake_layer(c), **{key: FAKE + 4}) == lq.LEAPQ_ERR_ALIGN, key
    assert lq.lib().leapq_append(None, *([ctypes.c_void_p(FAKE)] * 6), None) == lq.LEAPQ_ERR_NULL


def test_append_window_full_and_record_range():
    c = cfg(window=16)
    L = fake_layer(c, n=16)
    assert call_append(L) == lq.LEAPQ_ERR_WINDOW_FULL and L.n_records == 16
    L = fake_layer(c, n=17)
    assert call_append(L) == lq.LEAPQ_ERR_RANGE
    L = fake_layer(c, n=-1)
    assert lq.lib().leapq_fold(ctypes.byref(L), None) == lq.LEAPQ_ERR_RANGE and L.n_records == -1


def test_init_fold_dequant_checks():
    c = cfg()
    lib = lq.lib()
    vp = ctypes.c_void_p
    L = fake_layer(c)
    assert lib.leapq_init_state(ctypes.byref(L), None, None) == lq.LEAPQ_ERR_NULL
    assert lib.leapq_init_state(ctypes.byref(L), vp(FAKE + 8), None) == lq.LEAPQ_ERR_ALIGN
    assert lib.leapq_fold(None, None) == lq.LEAPQ_ERR_NULL
    assert lib.leapq_fold(ctypes.byref(fake_layer(c, state=FAKE + 128)), None) == lq.LEAPQ_ERR_ALIGN
    for what in (-1, 3):
        assert lib.leapq_dequant(ctypes.byref(L), what, vp(FAKE), None) == lq.LEAPQ_ERR_RANGE
    assert lib.leapq_dequant(ctypes.byref(L), 0, None, None) == lq.LEAPQ_ERR_NULL
    assert lib.leapq_dequant(ctypes.byref(L), 2, vp(FAKE + 4), None) == lq.LEAPQ_ERR_ALIGN


def test_gdn_decode_checks():
    lib = lq.lib()
    vp = ctypes.c_void_p
    c = cfg()
    args = [vp(FAKE)] * 8
    assert lib.leapq_gdn_decode(ctypes.byref(c), 5, *args, None) == lq.LEAPQ_ERR_DTYPE
    assert lib.leapq_gdn_decode(None, 0, *args, None) == lq.LEAPQ_ERR_NULL
    bad = list(args)
    bad[0] = None
    assert lib.leapq_gdn_decode(ctypes.byref(c), 0, *bad, None) == lq.LEAPQ_ERR_NULL
    bad = list(args)
    bad[1] = vp(FAKE + 2)
    assert lib.leapq_gdn_decode(ctypes.byref(c), 1, *bad, None) == lq.LEAPQ_ERR_ALIGN
    c.dv = 96
    assert lib.leapq_gdn_decode(ctypes.byref(c), 0, *args, None) == lq.LEAPQ_ERR_SHAPE


def call_append_fold(L, q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, o=FAKE):
    vp = ctypes.c_void_p
    return lq.lib().leapq_append_fold(ctypes.byref(L), vp(q), vp(k), vp(v), vp(a), vp(b), vp(o), None)


def test_append_fold_checks():
    """The fused last append + fold needs n_records == window - 1; failures
    leave n_records unchanged."""
    for W in (1, 16, 20, 64):
        c = cfg(window=W)
        for n in (0, W - 2, W, W + 1):
            if n == W - 1 or n < 0:
                continue
            L = fake_layer(c, n=n)
            assert call_append_fold(L) == lq.LEAPQ_ERR_RANGE and L.n_records == n, (W, n)
    c = cfg(window=16)
    assert call_append_fold(fake_layer(c, n=15, state=0)) == lq.LEAPQ_ERR_NULL
    assert call_append_fold(fake_layer(c, n=15, state=FAKE + 16)) == lq.LEAPQ_ERR_ALIGN
    for key in ("q", "k", "v", "a", "b", "o"):
        L = fake_layer(c, n=15)
        assert call_append_fold(L, **{key: 0}) == lq.LEAPQ_ERR_NULL and L.n_records == 15, key
    for key in ("q", "k", "v", "o"):
        assert call_append_fold(fake_layer(c, n=15), **{key: FAKE + 4}) == lq.LEAPQ_ERR_ALIGN, key


# ---------------------------------------------------------------- gated entry points

def gate_struct(A=FAKE, dt=FAKE, q_scale=0.125, eps=1e-6):
    g = lq.leapq_gate()
    g.A_log, g.dt_bias, g.q_scale, g.norm_eps = A, dt, q_scale, eps
    return g


def call_gated(L, g, fused=False, q=FAKE, a=FAKE):
    vp = ctypes.c_void_p
    fn = lq.lib().leapq_append_fold_gated if fused else lq.lib().leapq_append_gated
    gp = ctypes.byref(g) if g is not None else None
    return fn(ctypes.byref(L), gp, vp(q), vp(FAKE), vp(FAKE), vp(a), vp(FAKE), vp(FAKE), None)


@pytest.mark.parametrize("fused", [False, True])
def test_gated_checks(fused):
    c = cfg(qk_norm=True)
    n = 15 if fused else 0
    assert call_gated(fake_layer(c, n), None, fused) == lq.LEAPQ_ERR_NULL
    for kw, status in ((dict(A=0), lq.LEAPQ_ERR_NULL), (dict(dt=0), lq.LEAPQ_ERR_NULL),
                       (dict(A=FAKE + 2), lq.LEAPQ_ERR_ALIGN), (dict(dt=FAKE + 1), lq.LEAPQ_ERR_ALIGN),
                       (dict(eps=-1.0), lq.LEAPQ_ERR_RANGE), (dict(eps=float("nan")), lq.LEAPQ_ERR_RANGE),
                       (dict(eps=float("inf")), lq.LEAPQ_ERR_RANGE),
                       (dict(q_scale=float("nan")), lq.LEAPQ_ERR_RANGE),
                       (dict(q_scale=float("inf")), lq.LEAPQ_ERR_RANGE)):
        L = fake_layer(c, n)
        assert call_gated(L, gate_struct(**kw), fused) == status, kw
        assert L.n_records == n
    g = gate_struct()
    g.reserved[0] = 3
    assert call_gated(fake_layer(c, n), g, fused) == lq.LEAPQ_ERR_RANGE
    assert call_gated(fake_layer(c, n), gate_struct(), fused, q=0) == lq.LEAPQ_ERR_NULL
    assert call_gated(fake_layer(c, n), gate_struct(), fused, a=FAKE + 2) == lq.LEAPQ_ERR_ALIGN
    # window position
    bad_n = 3 if fused else 16
    expect = lq.LEAPQ_ERR_RANGE if fused else lq.LEAPQ_ERR_WINDOW_FULL
    assert call_gated(fake_layer(c, bad_n), gate_struct(), fused) == expect


def test_qk_norm_config_and_key_layout():
    out = lq.leapq_layout()
    c = cfg()
    c.qk_norm = 2
    assert lq.lib().leapq_query_layout(ctypes.byref(c), ctypes.byref(out)) == lq.LEAPQ_ERR_RANGE
    for dt, qk, e in (("bf16", False, 2), ("bf16", True, 4), ("f32", False, 4), ("f32", True, 4)):
        L = layout(batch=2, heads=4, window=16, n_comp=4, in_dtype=dt, qk_norm=qk)
        assert L.off_rec_u - L.off_rec_k >= 2 * 4 * 16 * 128 * e
        assert L.record_bytes_per_head == 16 * (4 + 128 * e + 512), (dt, qk)


# ---------------------------------------------------------------- per-channel decay

def test_channel_decay_layout_and_checks():
    for dt, e in (("bf16", 2), ("f32", 4)):
        L = layout(batch=2, heads=4, window=16, n_comp=4, in_dtype=dt, decay="channel")
        assert L.off_rec_k - L.off_rec_gamma >= 2 * 4 * 16 * 128 * 4
        assert L.record_bytes_per_head == 16 * (4 * 128 + 128 * e + 512), dt
    c = cfg(decay="channel")
    # the decay vector is read in 16-byte pieces
    assert call_append(fake_layer(c), a=FAKE + 4) == lq.LEAPQ_ERR_ALIGN
    assert call_append(fake_layer(c, n=16)) == lq.LEAPQ_ERR_WINDOW_FULL
    # the gates are scalar-decay gates
    assert call_gated(fake_layer(c), gate_struct()) == lq.LEAPQ_ERR_RANGE
    vp = ctypes.c_void_p
    args = [vp(FAKE)] * 8
    args[4] = vp(FAKE + 4)  # alpha
    assert lq.lib().leapq_gdn_decode(ctypes.byref(c), 0, *args, None) == lq.LEAPQ_ERR_ALIGN


# ---------------------------------------------------------------- bf16 record corrections

def test_bf16_corrections_layout_and_checks():
    for dt, e in (("bf16", 2), ("f32", 4)):
        L = layout(batch=2, heads=4, window=16, n_comp=4, in_dtype=dt, rec_dtype="bf16")
        assert L.total_bytes - L.off_rec_u >= 2 * 4 * 16 * 128 * 2
        assert L.record_bytes_per_head == 16 * (4 + 128 * e + 256), dt
    out = lq.leapq_layout()
    for kw in (dict(decay="channel"), dict(qk_norm=True)):
        c = cfg(rec_dtype="bf16", **kw)
        assert lq.lib().leapq_query_layout(ctypes.byref(c), ctypes.byref(out)) == lq.LEAPQ_ERR_RANGE, kw
    # the gated entry points keep fp32 corrections
    assert call_gated(fake_layer(cfg(rec_dtype="bf16")), gate_struct()) == lq.LEAPQ_ERR_RANGE


def test_fp8_corrections_layout_and_checks():
    for dt, e in (("bf16", 2), ("f32", 4)):
        L = layout(batch=2, heads=4, window=16, n_comp=4, in_dtype=dt, rec_dtype="fp8")
        assert L.total_bytes - L.off_rec_u >= 2 * 4 * 16 * 144
        assert L.record_bytes_per_head == 16 * (4 + 128 * e + 144), dt
        assert L.off_rec_u % 256 == 0
    out = lq.leapq_layout()
    for kw in (dict(decay="channel"), dict(qk_norm=True), dict(comp_fit="rank1"), dict(comp_fit="block")):
        c = cfg(rec_dtype="fp8", **kw)
        assert lq.lib().leapq_query_layout(ctypes.byref(c), ctypes.byref(out)) == lq.LEAPQ_ERR_RANGE, kw
    c = cfg()
    c.rec_dtype = 3
    assert lq.lib().leapq_query_layout(ctypes.byref(c), ctypes.byref(out)) == lq.LEAPQ_ERR_DTYPE
    c = cfg()
    c.in_dtype = lq.LEAPQ_FP8  # fp8 is a record format, not an input dtype
    assert lq.lib().leapq_query_layout(ctypes.byref(c), ctypes.byref(out)) == lq.LEAPQ_ERR_DTYPE
    assert call_gated(fake_layer(cfg(rec_dtype="fp8")), gate_struct()) == lq.LEAPQ_ERR_RANGE


def test_low_bit_layout_and_checks():
    for bits, nb in ((8, 16384), (6, 12288), (4, 8192)):
        L = layout(batch=2, heads=4, window=16, n_comp=4, state_bits=bits)
        assert L.boundary_bytes_per_head == nb + 1024 + 4 * 4 + 4 * 512, bits
        assert L.off_row_scale >= 8 * nb and L.off_row_scale % 256 == 0
    L0 = layout(batch=2, heads=4, state_bits=0)
    assert L0.boundary_bytes_per_head == 19472  # 0 means the int8 state
    out = lq.leapq_layout()
    for kw in (dict(state_bits=5), dict(state_bits=6, decay="channel"), dict(state_bits=4, comp_fit="rank1"),
               dict(state_bits=4, rec_dtype="bf16"), dict(state_bits=6, rec_dtype="fp8"),
               dict(state_bits=4, qk_norm=True)):
        c = cfg(**kw)
        assert lq.lib().leapq_query_layout(ctypes.byref(c), ctypes.byref(out)) == lq.LEAPQ_ERR_RANGE, kw
    assert call_gated(fake_layer(cfg(state_bits=4)), gate_struct()) == lq.LEAPQ_ERR_RANGE


# ---------------------------------------------------------------- rank-one compensators

def test_rank1_layout_and_checks():
    lines = layout(batch=2, heads=4, window=16, n_comp=4)
    r1 = layout(batch=2, heads=4, window=16, n_comp=4, comp_fit="rank1")
    # each compensator holds the pair (a, b): twice the vector bytes of a line
    assert r1.off_rec_gamma - r1.off_comp_vec >= 2 * 4 * 4 * 256 * 4
    assert r1.total_bytes - lines.total_bytes >= 2 * 4 * 4 * 128 * 4 - 256
    assert r1.record_bytes_per_head == lines.record_bytes_per_head
    out = lq.leapq_layout()
    c = cfg()
    c.comp_fit = -1
    assert lq.lib().leapq_query_layout(ctypes.byref(c), ctypes.byref(out)) == lq.LEAPQ_ERR_RANGE
    for kw in (dict(n_comp=5), dict(decay="channel"), dict(rec_dtype="bf16")):
        c = cfg(comp_fit="rank1", **kw)
        assert lq.lib().leapq_query_layout(ctypes.byref(c), ctypes.byref(out)) == lq.LEAPQ_ERR_RANGE, kw
    for C in (0, 1, 4):
        c = cfg(comp_fit="rank1", n_comp=C)
        assert lq.lib().leapq_query_layout(ctypes.byref(c), ctypes.byref(out)) == lq.LEAPQ_OK, C
    # the gated entry points keep line compensators
    assert call_gated(fake_layer(cfg(comp_fit="rank1")), gate_struct()) == lq.LEAPQ_ERR_RANGE


def test_block_fit_layout_and_checks():
    r1 = layout(batch=2, heads=4, window=16, n_comp=4, comp_fit="rank1")
    blk = layout(batch=2, heads=4, window=16, n_comp=4, comp_fit="block")
    # the block fit stores the same pairs as the rank-one fit
    for f in ("total_bytes", "off_comp_vec", "off_rec_gamma", "boundary_bytes_per_head"):
        assert getattr(blk, f) == getattr(r1, f), f
    out = lq.leapq_layout()
    c = cfg()
    c.comp_fit = 3
    assert lq.lib().leapq_query_layout(ctypes.byref(c), ctypes.byref(out)) == lq.LEAPQ_ERR_RANGE
    for kw in (dict(n_comp=5), dict(decay="channel"), dict(rec_dtype="bf16")):
        c = cfg(comp_fit="block", **kw)
        assert lq.lib().leapq_query_layout(ctypes.byref(c), ctypes.byref(out)) == lq.LEAPQ_ERR_RANGE, kw
    assert call_gated(fake_layer(cfg(comp_fit="block")), gate_struct()) == lq.LEAPQ_ERR_RANGE


# ---------------------------------------------------------------- per-request phases

def call_step(L, n_in=FAKE, n_out=FAKE + 4096, gate=None, a=FAKE):
    vp = ctypes.c_void_p
    gp = ctypes.byref(gate) if gate is not None else None
    return lq.lib().leapq_step(ctypes.byref(L), gp, vp(n_in), vp(n_out) if n_out else None, vp(FAKE), vp(FAKE),
                               vp(FAKE), vp(a), vp(FAKE), vp(FAKE), None)


def test_step_checks():
    c = cfg()  # batch 2
    assert call_step(fake_layer(c), n_in=0) == lq.LEAPQ_ERR_NULL
    assert call_step(fake_layer(c), n_in=FAKE + 2) == lq.LEAPQ_ERR_ALIGN
    assert call_step(fake_layer(c), n_out=FAKE + 4096 + 2) == lq.LEAPQ_ERR_ALIGN
    # n_out must not overlap n_in (batch 2: 8 bytes)
    assert call_step(fake_layer(c), n_out=FAKE) == lq.LEAPQ_ERR_RANGE
    assert call_step(fake_layer(c), n_out=FAKE + 4) == lq.LEAPQ_ERR_RANGE
    assert call_step(fake_layer(cfg(window=17))) == lq.LEAPQ_ERR_RANGE
    assert call_step(fake_layer(c), a=FAKE + 2) == lq.LEAPQ_ERR_ALIGN
    g = gate_struct()
    g.reserved[1] = 1
    assert call_step(fake_layer(cfg(qk_norm=True)), gate=g) == lq.LEAPQ_ERR_RANGE
    # the layer's host count is neither checked nor changed
    L = fake_layer(c, n=16)
    assert call_step(L, n_in=0) == lq.LEAPQ_ERR_NULL and L.n_records == 16
