"""ctypes wrapper of the C oracle (test infrastructure only).

Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark use this package.  It marshals numpy arrays into the C functions of
leapq_oracle.c and holds no arithmetic of its own beyond widening bf16 inputs
to fp32, which is exact.
"""
import ctypes
import os

import numpy as np

from . import build as _build

D = 128
_LIB = None


def lib(path=None):
    """Load (building if absent) the oracle shared object."""
    global _LIB
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _LIB = _bind(ctypes.CDLL(_build.LIB))
    return _LIB


def _bind(L):
    f32p = ctypes.POINTER(ctypes.c_float)
    i8p = ctypes.POINTER(ctypes.c_int8)
    i32p = ctypes.POINTER(ctypes.c_int32)
    f64p = ctypes.POINTER(ctypes.c_double)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    ci, cf, cd = ctypes.c_int, ctypes.c_float, ctypes.c_double
    sig = {
        "lqo_t128_sum": (cf, [f32p]),
        "lqo_t128_dot": (cf, [f32p, f32p]),
        "lqo_residual": (None, [i8p, f32p, f32p, f32p]),
        "lqo_boundary": (None, [i8p, f32p, f32p, ci, i32p, f32p, f32p]),
        "lqo_current": (None, [i8p, f32p, f32p, ci, i32p, f32p, ci, f32p, f32p, f32p, f32p]),
        "lqo_quantize": (None, [f32p, ci, ci, cf, i8p, f32p, f32p, i32p, f32p]),
        "lqo_init": (None, [f32p, ci, ci, cf, i8p, f32p, f32p, i32p, f32p]),
        "lqo_init_bits": (None, [f32p, ci, ci, cf, ci, i8p, f32p, f32p, i32p, f32p]),
        "lqo_fold_bits": (None, [i8p, f32p, f32p, ci, i32p, f32p, ci, f32p, f32p, f32p, ci, cf, ci]),
        "lqo_quantize_keyrow": (None, [f32p, ci, ci, cf, i8p, f32p, f32p, i32p, f32p]),
        "lqo_boundary_keyrow": (None, [i8p, f32p, f32p, ci, i32p, f32p, f32p]),
        "lqo_fold": (None, [i8p, f32p, f32p, ci, i32p, f32p, ci, f32p, f32p, f32p, ci, cf]),
        "lqo_append": (None, [i8p, f32p, f32p, ci, i32p, f32p, ci, f32p, f32p, f32p,
                              f32p, f32p, f32p, cf, cf, f32p]),
        "lqo_current_kda": (None, [i8p, f32p, f32p, ci, i32p, f32p, ci, f32p, f32p, f32p, f32p]),
        "lqo_fold_kda": (None, [i8p, f32p, f32p, ci, i32p, f32p, ci, f32p, f32p, f32p, ci, cf]),
        "lqo_append_kda": (None, [i8p, f32p, f32p, ci, i32p, f32p, ci, f32p, f32p, f32p,
                                  f32p, f32p, f32p, f32p, cf, f32p]),
        "lqo_kda_step_f32": (None, [f32p, f32p, f32p, f32p, f32p, cf, f32p, f32p]),
        "lqo_gdn_step_f32": (None, [f32p, f32p, f32p, f32p, cf, cf, f32p, f32p]),
        "lqo_gdn_step_f64": (None, [f64p, f64p, f64p, f64p, cd, cd, f64p, f64p]),
        "lqo_gdn_step_bf16": (None, [u16p, f32p, f32p, f32p, cf, cf, f32p, f32p]),
        "lqo_f32_to_bf16": (ctypes.c_uint16, [cf]),
        "lqo_round_bf16": (None, [f32p, ci]),
        "lqo_f32_to_e4m3": (ctypes.c_uint8, [cf]),
        "lqo_e4m3_to_f32": (cf, [ctypes.c_uint8]),
        "lqo_round_fp8_record": (None, [f32p]),
        "lqo_gate": (None, [cf, cf, cf, cf, f32p, f32p]),
        "lqo_quantize_r1": (None, [f32p, ci, ci, cf, i8p, f32p, f32p, i32p, f32p]),
        "lqo_init_r1": (None, [f32p, ci, ci, cf, i8p, f32p, f32p, i32p, f32p]),
        "lqo_fold_r1": (None, [i8p, f32p, f32p, ci, i32p, f32p, ci, f32p, f32p, f32p, ci, cf]),
        "lqo_current_r1": (None, [i8p, f32p, f32p, ci, f32p, ci, f32p, f32p, f32p, f32p]),
        "lqo_append_r1": (None, [i8p, f32p, f32p, ci, i32p, f32p, ci, f32p, f32p, f32p,
                                 f32p, f32p, f32p, cf, cf, f32p]),
        "lqo_fit_block": (None, [f32p, ci, i32p, f32p, ci, ci]),
        "lqo_quantize_block": (None, [f32p, ci, ci, cf, ci, i8p, f32p, f32p, i32p, f32p]),
        "lqo_init_block": (None, [f32p, ci, ci, cf, i8p, f32p, f32p, i32p, f32p]),
        "lqo_fold_block": (None, [i8p, f32p, f32p, ci, i32p, f32p, ci, f32p, f32p, f32p, ci, cf]),
        "lqo_l2norm": (None, [f32p, cf, cf, f32p]),
        "lqo_dim": (ci, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def _p(a, ct):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.POINTER(ct))


def f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns (uint16) to fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def t128_sum(f, L=None):
    L = L or lib()
    return float(L.lqo_t128_sum(_p(f32(f), ctypes.c_float)))


def t128_dot(a, b, L=None):
    L = L or lib()
    return float(L.lqo_t128_dot(_p(f32(a), ctypes.c_float), _p(f32(b), ctypes.c_float)))


def gate(a, b, A_log, dt_bias, L=None):
    """Decay and step size from the raw gate inputs (fp32 scalars)."""
    L = L or lib()
    al, be = ctypes.c_float(), ctypes.c_float()
    L.lqo_gate(float(np.float32(a)), float(np.float32(b)), float(np.float32(A_log)), float(np.float32(dt_bias)),
               ctypes.byref(al), ctypes.byref(be))
    return np.float32(al.value), np.float32(be.value)


def l2norm(x, eps=1e-6, scale=1.0, L=None):
    """(x * (1 / sqrt(T128(x . x) + eps))) * scale in fp32."""
    L = L or lib()
    out = np.zeros(D, np.float32)
    L.lqo_l2norm(_p(f32(x), ctypes.c_float), float(np.float32(eps)), float(np.float32(scale)),
                 _p(out, ctypes.c_float))
    return out


def gated_inputs(q, k, v, a, b, A_log, dt_bias, q_scale=1.0, eps=1e-6, normalize=True, L=None):
    """One head's token as the append sees it after the gate arithmetic:
    (q, k, v, alpha, beta), q and k L2-normalized (q also scaled) when
    `normalize`."""
    alpha, beta = gate(a, b, A_log, dt_bias, L)
    if normalize:
        q = l2norm(q, eps, q_scale, L)
        k = l2norm(k, eps, 1.0, L)
    return f32(q), f32(k), f32(v), alpha, beta


def quantize_axis(S, C=4, smoothing=True, sigma_floor=1e-6, axis="value", L=None):
    """Quantizes one fp32 state [128][128] as init does and returns
    (Q, rho, sigma, idx, vec, B) with B the boundary state.  axis="value"
    is the path's smoothing (sigma per value column, rho per key row);
    axis="key" is the study of the other axis (sigma per key row, rho per
    value column)."""
    L = L or lib()
    R = f32(S).reshape(D, D).copy()
    Q = np.zeros((D, D), np.int8)
    rho, sig = np.zeros(D, np.float32), np.zeros(D, np.float32)
    idx, vec = np.full(max(C, 1), -1, np.int32), np.zeros((max(C, 1), D), np.float32)
    B = np.zeros((D, D), np.float32)
    fp, ip = ctypes.c_float, ctypes.c_int8
    args = (_p(Q, ip), _p(rho, fp), _p(sig, fp))
    if axis == "value":
        L.lqo_quantize(_p(R, fp), C, int(smoothing), float(sigma_floor), *args, _p(idx, ctypes.c_int32),
                       _p(vec, fp))
        L.lqo_boundary(*args, C, _p(idx, ctypes.c_int32), _p(vec, fp), _p(B, fp))
    elif axis == "key":
        L.lqo_quantize_keyrow(_p(R, fp), C, int(smoothing), float(sigma_floor), *args, _p(idx, ctypes.c_int32),
                              _p(vec, fp))
        L.lqo_boundary_keyrow(*args, C, _p(idx, ctypes.c_int32), _p(vec, fp), _p(B, fp))
    else:
        raise ValueError("axis must be 'value' or 'key'")
    return Q, rho, sig, idx[:C], vec[:C], B


class Head:
    """One head's LeapQuant state held in numpy arrays, driven by the oracle.

    Q is int8 [128][128] in logical (key row, value column) order; rho and
    sigma are fp32 [128]; idx int32 [C]; vec fp32 [C][128]; records gam [W]
    (decay="scalar", GDN) or [W][128] (decay="channel", KDA), rk [W][128],
    ru [W][128]; n is the number of records in the window.
    """

    def __init__(self, C=4, W=16, smoothing=True, sigma_floor=1e-6, L=None, decay="scalar", rec_u="f32",
                 fit="lines", bits=8):
        self.L = L or lib()
        if bits not in (8, 6, 4):
            raise ValueError("bits must be 8, 6 or 4")
        if bits != 8 and (decay != "scalar" or fit != "lines"):
            raise ValueError("6- and 4-bit states are defined for scalar decay and line compensators")
        self.bits = int(bits)
        self.C, self.W, self.smoothing, self.floor = int(C), int(W), int(smoothing), float(sigma_floor)
        if decay not in ("scalar", "channel"):
            raise ValueError("decay must be 'scalar' or 'channel'")
        self.decay = decay
        self.kda = decay == "channel"
        if rec_u not in ("f32", "bf16", "fp8"):
            raise ValueError("rec_u must be 'f32', 'bf16' or 'fp8'")
        self.rec_u = rec_u
        if fit not in ("lines", "rank1", "block"):
            raise ValueError("fit must be 'lines', 'rank1' or 'block'")
        if fit != "lines" and self.kda:
            raise ValueError("rank-one and block compensators are defined for scalar decay")
        self.fit = fit
        # rank-one and block fits store and read the same pairs [a | b]
        self.r1 = fit in ("rank1", "block")
        self.block = fit == "block"
        self.Q = np.zeros((D, D), np.int8)
        self.rho = np.zeros(D, np.float32)
        self.sigma = np.ones(D, np.float32)
        self.idx = np.full(max(self.C, 1), -1, np.int32)
        # compensators: lines [C][128], or pairs [C][2 * 128] = [a | b] (rank-one
        # and block fits)
        self.vec = np.zeros((max(self.C, 1), 2 * D if self.r1 else D), np.float32)
        self.gam = np.zeros((max(self.W, 1), D) if self.kda else max(self.W, 1), np.float32)
        self.rk = np.zeros((max(self.W, 1), D), np.float32)
        self.ru = np.zeros((max(self.W, 1), D), np.float32)
        self.n = 0

    def _st(self):
        fp, ip = ctypes.c_float, ctypes.c_int8
        return (_p(self.Q, ip), _p(self.rho, fp), _p(self.sigma, fp), self.C,
                _p(self.idx, ctypes.c_int32), _p(self.vec, fp))

    def _rec(self):
        fp = ctypes.c_float
        return (self.n, _p(self.gam, fp), _p(self.rk, fp), _p(self.ru, fp))

    def init(self, S0):
        S0 = f32(S0).reshape(D, D)
        fp = ctypes.c_float
        if self.bits != 8:
            self.L.lqo_init_bits(_p(S0, fp), self.C, self.smoothing, self.floor, self.bits, _p(self.Q, ctypes.c_int8),
                                 _p(self.rho, fp), _p(self.sigma, fp), _p(self.idx, ctypes.c_int32), _p(self.vec, fp))
            self.n = 0
            return self
        fn = self.L.lqo_init_block if self.block else self.L.lqo_init_r1 if self.r1 else self.L.lqo_init
        fn(_p(S0, fp), self.C, self.smoothing, self.floor, _p(self.Q, ctypes.c_int8),
           _p(self.rho, fp), _p(self.sigma, fp), _p(self.idx, ctypes.c_int32), _p(self.vec, fp))
        self.n = 0
        return self

    def append(self, q, k, v, alpha, beta):
        """One token; returns (o, u) as fp32 arrays."""
        if self.n >= self.W:
            raise RuntimeError("window full: fold before the next append")
        q, k, v = f32(q), f32(k), f32(v)
        o = np.zeros(D, np.float32)
        fp = ctypes.c_float
        if self.kda:
            al = f32(alpha).reshape(D)
            self.L.lqo_append_kda(*self._st(), *self._rec(), _p(q, fp), _p(k, fp), _p(v, fp), _p(al, fp),
                                  float(np.float32(beta)), _p(o, fp))
        else:
            fn = self.L.lqo_append_r1 if self.r1 else self.L.lqo_append
            fn(*self._st(), *self._rec(), _p(q, fp), _p(k, fp), _p(v, fp),
               float(np.float32(alpha)), float(np.float32(beta)), _p(o, fp))
        self.n += 1
        if self.rec_u == "bf16":
            # the record keeps u rounded to bf16; this token's output used
            # the fp32 u (lqo_append above)
            self.L.lqo_round_bf16(_p(self.ru[self.n - 1], fp), D)
        elif self.rec_u == "fp8":
            # the record keeps u as fp8 with a power-of-two scale per group
            # of 32 value columns; this token's output used the fp32 u
            self.L.lqo_round_fp8_record(_p(self.ru[self.n - 1], fp))
        return o, self.ru[self.n - 1].copy()

    def fold(self):
        if self.bits != 8:
            self.L.lqo_fold_bits(*self._st(), *self._rec(), self.smoothing, self.floor, self.bits)
            self.n = 0
            return self
        if self.kda:
            fn = self.L.lqo_fold_kda
        elif self.block:
            fn = self.L.lqo_fold_block
        else:
            fn = self.L.lqo_fold_r1 if self.r1 else self.L.lqo_fold
        fn(*self._st(), *self._rec(), self.smoothing, self.floor)
        self.n = 0
        return self

    def dequant(self, what):
        out = np.zeros((D, D), np.float32)
        fp = ctypes.c_float
        if what == 0:
            self.L.lqo_residual(_p(self.Q, ctypes.c_int8), _p(self.rho, fp), _p(self.sigma, fp),
                                _p(out, fp))
        elif what in (1, 2) and self.r1:
            n = self.n if what == 2 else 0
            self.L.lqo_current_r1(_p(self.Q, ctypes.c_int8), _p(self.rho, fp), _p(self.sigma, fp), self.C,
                                  _p(self.vec, fp), n, _p(self.gam, fp), _p(self.rk, fp), _p(self.ru, fp),
                                  _p(out, fp))
        elif what == 1:
            self.L.lqo_boundary(*self._st(), _p(out, fp))
        elif what == 2:
            fn = self.L.lqo_current_kda if self.kda else self.L.lqo_current
            fn(*self._st(), *self._rec(), _p(out, fp))
        else:
            raise ValueError("what must be 0, 1 or 2")
        return out

    def copy(self):
        h = Head(self.C, self.W, self.smoothing, self.floor, self.L, self.decay, self.rec_u, self.fit, self.bits)
        for name in ("Q", "rho", "sigma", "idx", "vec", "gam", "rk", "ru"):
            setattr(h, name, getattr(self, name).copy())
        h.n = self.n
        return h


def fit_block(R, C=4, idx=None, ab=None, warm=False, sweeps=2, L=None):
    """The block fit alone on a copy of R: returns (deflated R, idx, ab).
    With warm, the live pairs of (idx, ab) are the start."""
    L = L or lib()
    R = f32(R).reshape(D, D).copy()
    idx = np.full(max(C, 1), -1, np.int32) if idx is None else np.array(idx, np.int32)
    ab = np.zeros((max(C, 1), 2 * D), np.float32) if ab is None else np.array(ab, np.float32)
    L.lqo_fit_block(_p(R, ctypes.c_float), int(C), _p(idx, ctypes.c_int32), _p(ab, ctypes.c_float), int(warm),
                    int(sweeps))
    return R, idx, ab


def quantize(R, C=4, smoothing=True, sigma_floor=1e-6, L=None, fit="lines"):
    """Quantize a full fp32 matrix; returns a fresh Head at n = 0."""
    return Head(C, 16, smoothing, sigma_floor, L, fit=fit).init(R)


def gdn_step_f32(S, q, k, v, alpha, beta, L=None):
    """Dense fp32 GDN token step, in place on S [128][128]; returns (u, o)."""
    L = L or lib()
    assert S.dtype == np.float32 and S.flags["C_CONTIGUOUS"]
    u = np.zeros(D, np.float32)
    o = np.zeros(D, np.float32)
    fp = ctypes.c_float
    L.lqo_gdn_step_f32(_p(S, fp), _p(f32(q), fp), _p(f32(k), fp), _p(f32(v), fp),
                       float(np.float32(alpha)), float(np.float32(beta)), _p(u, fp), _p(o, fp))
    return u, o


def kda_step_f32(S, q, k, v, alpha, beta, L=None):
    """Dense fp32 KDA token step (per-row decay alpha [128]), in place on S; returns (u, o)."""
    L = L or lib()
    assert S.dtype == np.float32 and S.flags["C_CONTIGUOUS"]
    u = np.zeros(D, np.float32)
    o = np.zeros(D, np.float32)
    fp = ctypes.c_float
    L.lqo_kda_step_f32(_p(S, fp), _p(f32(q), fp), _p(f32(k), fp), _p(f32(v), fp), _p(f32(alpha), fp),
                       float(np.float32(beta)), _p(u, fp), _p(o, fp))
    return u, o


def gdn_step_f64(S, q, k, v, alpha, beta, L=None):
    """Dense fp64 GDN token step, in place on S; returns (u, o)."""
    L = L or lib()
    assert S.dtype == np.float64 and S.flags["C_CONTIGUOUS"]
    dp = ctypes.c_double
    u = np.zeros(D, np.float64)
    o = np.zeros(D, np.float64)
    c = lambda a: np.ascontiguousarray(a, dtype=np.float64)
    L.lqo_gdn_step_f64(_p(S, dp), _p(c(q), dp), _p(c(k), dp), _p(c(v), dp), float(alpha),
                       float(beta), _p(u, dp), _p(o, dp))
    return u, o


def gdn_step_bf16(Sb, q, k, v, alpha, beta, L=None):
    """Dense bf16-state GDN token step, in place on Sb (uint16 bits); returns (u, o)."""
    L = L or lib()
    assert Sb.dtype == np.uint16 and Sb.flags["C_CONTIGUOUS"]
    u = np.zeros(D, np.float32)
    o = np.zeros(D, np.float32)
    fp = ctypes.c_float
    L.lqo_gdn_step_bf16(_p(Sb, ctypes.c_uint16), _p(f32(q), fp), _p(f32(k), fp), _p(f32(v), fp),
                        float(np.float32(alpha)), float(np.float32(beta)), _p(u, fp), _p(o, fp))
    return u, o

