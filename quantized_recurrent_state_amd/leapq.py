"""ctypes binding of libleapq (include/leapq.h), under the C names.

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libleapq.so.  Tensors are torch tensors (device memory); streams
are torch streams.  If the shared library is missing this module raises on
first use; there is no fallback implementation.
"""
import ctypes
import os

import torch

from . import build as _build

D = 128

LEAPQ_OK = 0
LEAPQ_ERR_NULL = -1
LEAPQ_ERR_SHAPE = -2
LEAPQ_ERR_RANGE = -3
LEAPQ_ERR_ALIGN = -4
LEAPQ_ERR_WINDOW_FULL = -5
LEAPQ_ERR_DTYPE = -6
LEAPQ_ERR_HIP = -7

LEAPQ_F32 = 0
LEAPQ_BF16 = 1
LEAPQ_FP8 = 2  # record corrections only

LEAPQ_DECAY_SCALAR = 0
LEAPQ_DECAY_CHANNEL = 1

LEAPQ_COMP_LINES = 0
LEAPQ_COMP_RANK1 = 1
LEAPQ_COMP_BLOCK = 2

LEAPQ_DEQ_RESIDUAL = 0
LEAPQ_DEQ_BOUNDARY = 1
LEAPQ_DEQ_CURRENT = 2

SYMBOLS = ("leapq_query_layout", "leapq_init_state", "leapq_append", "leapq_append_fold", "leapq_append_gated",
           "leapq_append_fold_gated", "leapq_step", "leapq_fold", "leapq_dequant", "leapq_gdn_decode",
           "leapq_status_str", "leapq_version")


class leapq_config(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("dk", ctypes.c_int32),
                ("dv", ctypes.c_int32), ("window", ctypes.c_int32), ("n_comp", ctypes.c_int32),
                ("smoothing", ctypes.c_int32), ("sigma_floor", ctypes.c_float),
                ("in_dtype", ctypes.c_int32), ("qk_norm", ctypes.c_int32), ("decay", ctypes.c_int32),
                ("rec_dtype", ctypes.c_int32), ("comp_fit", ctypes.c_int32), ("state_bits", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 2)]


class leapq_gate(ctypes.Structure):
    _fields_ = [("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p), ("q_scale", ctypes.c_float),
                ("norm_eps", ctypes.c_float), ("reserved", ctypes.c_int32 * 2)]


class leapq_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "total_bytes", "off_codes", "off_row_scale", "off_col_scale", "off_comp_idx", "off_comp_vec",
        "off_rec_gamma", "off_rec_k", "off_rec_u", "boundary_bytes_per_head", "record_bytes_per_head")]


class leapq_layer(ctypes.Structure):
    _fields_ = [("cfg", leapq_config), ("state", ctypes.c_void_p), ("n_records", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class LeapqError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} ({status})")


_LIB = None


def lib():
    """The loaded libleapq.so.  Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            raise RuntimeError(f"libleapq.so not found at {_build.LIB}; run __graft_entry__.build() "
                               "or python -m quantized_recurrent_state_amd.build")
        L = ctypes.CDLL(_build.LIB)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.leapq_query_layout.argtypes = [ctypes.POINTER(leapq_config), ctypes.POINTER(leapq_layout)]
        L.leapq_init_state.argtypes = [ctypes.POINTER(leapq_layer), vp, vp]
        L.leapq_append.argtypes = [ctypes.POINTER(leapq_layer), vp, vp, vp, vp, vp, vp, vp]
        L.leapq_append_fold.argtypes = [ctypes.POINTER(leapq_layer), vp, vp, vp, vp, vp, vp, vp]
        for f in ("leapq_append_gated", "leapq_append_fold_gated"):
            getattr(L, f).argtypes = [ctypes.POINTER(leapq_layer), ctypes.POINTER(leapq_gate), vp, vp, vp, vp, vp,
                                      vp, vp]
        L.leapq_step.argtypes = [ctypes.POINTER(leapq_layer), ctypes.POINTER(leapq_gate), vp, vp, vp, vp, vp, vp,
                                 vp, vp, vp]
        L.leapq_fold.argtypes = [ctypes.POINTER(leapq_layer), vp]
        L.leapq_dequant.argtypes = [ctypes.POINTER(leapq_layer), i32, vp, vp]
        L.leapq_gdn_decode.argtypes = [ctypes.POINTER(leapq_config), i32, vp, vp, vp, vp, vp, vp, vp, vp]
        for f in ("leapq_query_layout", "leapq_init_state", "leapq_append", "leapq_append_fold",
                  "leapq_append_gated", "leapq_append_fold_gated", "leapq_step", "leapq_fold", "leapq_dequant",
                  "leapq_gdn_decode", "leapq_version"):
            getattr(L, f).restype = i32
        L.leapq_status_str.argtypes = [i32]
        L.leapq_status_str.restype = ctypes.c_char_p
        L.leapq_version.argtypes = []
        _LIB = L
    return _LIB


def status_str(status):
    return lib().leapq_status_str(int(status)).decode()


def _check(status, what):
    if status != LEAPQ_OK:
        raise LeapqError(status, what)


def make_config(batch, heads, window=16, n_comp=4, smoothing=True, sigma_floor=1e-6, in_dtype="f32",
                qk_norm=False, decay="scalar", rec_dtype="f32", comp_fit="lines", state_bits=8):
    c = leapq_config()
    c.batch, c.heads, c.dk, c.dv = int(batch), int(heads), D, D
    c.window, c.n_comp, c.smoothing = int(window), int(n_comp), int(bool(smoothing))
    c.sigma_floor = float(sigma_floor)
    c.in_dtype = LEAPQ_BF16 if in_dtype in ("bf16", torch.bfloat16, LEAPQ_BF16) else LEAPQ_F32
    c.qk_norm = int(bool(qk_norm))
    c.decay = LEAPQ_DECAY_CHANNEL if decay in ("channel", LEAPQ_DECAY_CHANNEL) else LEAPQ_DECAY_SCALAR
    c.rec_dtype = (LEAPQ_BF16 if rec_dtype in ("bf16", torch.bfloat16, LEAPQ_BF16) else
                   LEAPQ_FP8 if rec_dtype in ("fp8", LEAPQ_FP8) else LEAPQ_F32)
    fits = {"lines": LEAPQ_COMP_LINES, "rank1": LEAPQ_COMP_RANK1, "block": LEAPQ_COMP_BLOCK}
    c.comp_fit = fits.get(comp_fit, comp_fit)
    c.state_bits = int(state_bits)
    return c


def _alpha_shape(cfg):
    H = cfg.batch * cfg.heads
    return (H, D) if cfg.decay == LEAPQ_DECAY_CHANNEL else (H,)


class Gate:
    """Gate parameters of a layer (leapq_gate): A_log and dt_bias are fp32
    device tensors [heads] (per model head); q_scale and norm_eps apply when
    the layer normalizes q and k (qk_norm)."""

    def __init__(self, A_log, dt_bias, q_scale=D ** -0.5, norm_eps=1e-6):
        if A_log.shape != dt_bias.shape or A_log.dim() != 1:
            raise ValueError("A_log and dt_bias: fp32 [heads]")
        for name, t in (("A_log", A_log), ("dt_bias", dt_bias)):
            if t.dtype != torch.float32 or not t.is_contiguous():
                raise ValueError(f"{name}: expected a contiguous float32 tensor")
        self.A_log, self.dt_bias = A_log, dt_bias
        self.c = leapq_gate()
        self.c.A_log, self.c.dt_bias = A_log.data_ptr(), dt_bias.data_ptr()
        self.c.q_scale, self.c.norm_eps = float(q_scale), float(norm_eps)


def leapq_query_layout(cfg):
    out = leapq_layout()
    _check(lib().leapq_query_layout(ctypes.byref(cfg), ctypes.byref(out)), "leapq_query_layout")
    return out


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dev_tensor(t, name, dtype, shape, device):
    if t.device != device or t.dtype != dtype or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on {device}, got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device} (contiguous={t.is_contiguous()})")


# ---- stored orders of the state sections (include/leapq.h); r, c are
# integer tensors (or ints) of key rows / value columns.
def _iperm(x):
    return x ^ (((x >> 2) & 1) * 3)


def code_offset(r, c):
    """Byte of code (r, c) within its head's 16384-byte block."""
    return (c & 3) * 4096 + (r >> 5) * 1024 + (_iperm(r & 31) + 32 * ((c >> 2) & 1)) * 16 + (c >> 3)


def corr_pos(c):
    """Position of value column c within a stored record correction."""
    return 32 * (c & 3) + 8 * (c >> 5) + 4 * ((c >> 2) & 1) + ((c >> 3) & 3)


class Layer:
    """One layer: config + its state buffer (torch uint8 tensor) + window count."""

    def __init__(self, cfg, device="cuda"):
        self.cfg = cfg
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self.layout = leapq_query_layout(cfg)
        n = int(self.layout.total_bytes)
        buf = torch.empty(n + 256, dtype=torch.uint8, device=self.device)
        off = (-buf.data_ptr()) % 256
        self._buf = buf
        self.state = buf[off:off + n]
        self.c = leapq_layer()
        self.c.cfg = cfg
        self.c.state = self.state.data_ptr()
        self.c.n_records = 0

    @property
    def heads(self):
        return self.cfg.batch * self.cfg.heads

    @property
    def n_records(self):
        return self.c.n_records

    @property
    def in_dtype(self):
        return torch.bfloat16 if self.cfg.in_dtype == LEAPQ_BF16 else torch.float32

    @property
    def key_dtype(self):
        """Element type of the stored record keys (include/leapq.h layout)."""
        return torch.bfloat16 if self.cfg.in_dtype == LEAPQ_BF16 and not self.cfg.qk_norm else torch.float32

    # ---- read-only views of the state sections (layout of include/leapq.h)
    def _sec(self, off, count, dtype, shape):
        nbytes = count * torch.tensor([], dtype=dtype).element_size()
        return self.state[off:off + nbytes].view(dtype).view(*shape)

    @property
    def state_bits(self):
        return self.cfg.state_bits if self.cfg.state_bits in (6, 4) else 8

    def codes_physical(self):
        """int8 [heads, bytes]: each head's codes in stored order (16384 bytes; 12288 or 8192 packed
        bytes with state_bits 6 or 4)."""
        H, nb = self.heads, D * D * self.state_bits // 8
        return self._sec(self.layout.off_codes, H * nb, torch.int8, (H, nb))

    def codes(self):
        """int8 [heads, 128(row), 128(column)] in logical order (the 6- and 4-bit layouts of
        include/leapq.h unpacked and sign-extended)."""
        r = torch.arange(D, device=self.device).view(D, 1)
        c = torch.arange(D, device=self.device).view(1, D)
        phys = self.codes_physical()
        if self.state_bits == 8:
            return phys[:, code_offset(r, c)]
        raw = phys.view(torch.uint8).to(torch.int32)
        w, p, m = c & 3, r >> 5, c >> 3
        l = _iperm(r & 31) + 32 * ((c >> 2) & 1)
        lo_byte = 2048 * w + 1024 * (p >> 1) + 16 * l + 8 * (p & 1) + 4 * (m >> 3) + (m & 3)
        val = (raw[:, lo_byte] >> (4 * ((m & 7) >> 2))) & 15
        if self.state_bits == 4:
            return torch.where(val >= 8, val - 16, val).to(torch.int8)
        hi_byte = 8192 + 1024 * w + 16 * l + 4 * p + (m & 3)
        val = val | (((raw[:, hi_byte] >> (2 * (m >> 2))) & 3) << 4)
        return torch.where(val >= 32, val - 64, val).to(torch.int8)

    def rho(self):
        return self._sec(self.layout.off_row_scale, self.heads * D, torch.float32, (self.heads, D))

    def sigma(self):
        return self._sec(self.layout.off_col_scale, self.heads * D, torch.float32, (self.heads, D))

    def comp_idx(self):
        C = max(self.cfg.n_comp, 0)
        return self._sec(self.layout.off_comp_idx, self.heads * C, torch.int32, (self.heads, C))

    def comp_vec(self):
        """Compensators [heads, C, 128] (lines) or [heads, C, 256] (rank-one pairs [a | b])."""
        C = max(self.cfg.n_comp, 0)
        w = 2 * D if self.cfg.comp_fit != LEAPQ_COMP_LINES else D
        return self._sec(self.layout.off_comp_vec, self.heads * C * w, torch.float32, (self.heads, C, w))

    def rec_gamma(self):
        """Record decays [heads, W] (scalar decay) or [heads, W, 128] (channel decay)."""
        W = self.cfg.window
        if self.cfg.decay == LEAPQ_DECAY_CHANNEL:
            return self._sec(self.layout.off_rec_gamma, self.heads * W * D, torch.float32, (self.heads, W, D))
        return self._sec(self.layout.off_rec_gamma, self.heads * W, torch.float32, (self.heads, W))

    def rec_k_physical(self):
        """Record keys [heads, W, 128] as stored (key_dtype, key-row order)."""
        W = self.cfg.window
        return self._sec(self.layout.off_rec_k, self.heads * W * D, self.key_dtype, (self.heads, W, D))

    def rec_u_physical(self):
        """Record corrections [heads, W, 128] as stored (fp32, or bf16 with rec_dtype bf16); with
        rec_dtype fp8 the tuple (E4M3 codes uint8 [heads, W, 128], scales fp32 [heads, W, 4])."""
        W = self.cfg.window
        if self.cfg.rec_dtype == LEAPQ_FP8:
            raw = self._sec(self.layout.off_rec_u, self.heads * W * (D + 16), torch.uint8, (self.heads, W, D + 16))
            return raw[:, :, :D], raw[:, :, D:].contiguous().view(torch.float32)
        dt = torch.bfloat16 if self.cfg.rec_dtype == LEAPQ_BF16 else torch.float32
        return self._sec(self.layout.off_rec_u, self.heads * W * D, dt, (self.heads, W, D))

    def rec_k(self):
        """Record keys [heads, W, 128] as fp32 (exact)."""
        return self.rec_k_physical().float()

    def rec_u(self):
        """Record corrections [heads, W, 128] in logical value-column order, as fp32 (fp8 codes are
        decoded with torch's float8_e4m3fn and multiplied by their group's scale)."""
        c = torch.arange(D, device=self.device)
        if self.cfg.rec_dtype == LEAPQ_FP8:
            codes, scales = self.rec_u_physical()
            vals = codes.contiguous().view(torch.float8_e4m3fn).float() * scales.repeat_interleave(32, dim=2)
            return vals[:, :, corr_pos(c)]
        return self.rec_u_physical()[:, :, corr_pos(c)].float()


def leapq_init_state(layer, S0, stream=None):
    _dev_tensor(S0, "S0", torch.float32, (layer.heads, D, D), layer.device)
    _check(lib().leapq_init_state(ctypes.byref(layer.c), _ptr(S0), _stream(stream, layer.device)),
           "leapq_init_state")


def leapq_append(layer, q, k, v, alpha, beta, o, stream=None):
    H, dt, dev = layer.heads, layer.in_dtype, layer.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(t, name, dt, (H, D), dev)
    _dev_tensor(alpha, "alpha", torch.float32, _alpha_shape(layer.cfg), dev)
    _dev_tensor(beta, "beta", torch.float32, (H,), dev)
    _dev_tensor(o, "o", torch.float32, (H, D), dev)
    _check(lib().leapq_append(ctypes.byref(layer.c), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                              _ptr(o), _stream(stream, dev)), "leapq_append")


def leapq_append_fold(layer, q, k, v, alpha, beta, o, stream=None):
    """The window's last token and the fold (leapq_append then leapq_fold)."""
    H, dt, dev = layer.heads, layer.in_dtype, layer.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(t, name, dt, (H, D), dev)
    _dev_tensor(alpha, "alpha", torch.float32, _alpha_shape(layer.cfg), dev)
    _dev_tensor(beta, "beta", torch.float32, (H,), dev)
    _dev_tensor(o, "o", torch.float32, (H, D), dev)
    _check(lib().leapq_append_fold(ctypes.byref(layer.c), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                   _ptr(o), _stream(stream, dev)), "leapq_append_fold")


def _gated_args(layer, gate, q, k, v, a, b, o):
    H, dt, dev = layer.heads, layer.in_dtype, layer.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(t, name, dt, (H, D), dev)
    _dev_tensor(a, "a", torch.float32, (H,), dev)
    _dev_tensor(b, "b", torch.float32, (H,), dev)
    _dev_tensor(o, "o", torch.float32, (H, D), dev)
    for name, t in (("A_log", gate.A_log), ("dt_bias", gate.dt_bias)):
        _dev_tensor(t, name, torch.float32, (layer.cfg.heads,), dev)
    return (ctypes.byref(layer.c), ctypes.byref(gate.c), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(o))


def leapq_append_gated(layer, gate, q, k, v, a, b, o, stream=None):
    """leapq_append with the gate arithmetic: a, b are the raw projections."""
    _check(lib().leapq_append_gated(*_gated_args(layer, gate, q, k, v, a, b, o), _stream(stream, layer.device)),
           "leapq_append_gated")


def leapq_append_fold_gated(layer, gate, q, k, v, a, b, o, stream=None):
    """leapq_append_fold with the gate arithmetic."""
    _check(lib().leapq_append_fold_gated(*_gated_args(layer, gate, q, k, v, a, b, o),
                                         _stream(stream, layer.device)), "leapq_append_fold_gated")


def leapq_step(layer, n_in, n_out, q, k, v, alpha, beta, o, gate=None, stream=None):
    """One token with a window phase per request: n_in, n_out int32 [batch]
    (n_out may be None); with a gate, alpha and beta are the raw a, b."""
    H, dt, dev = layer.heads, layer.in_dtype, layer.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(t, name, dt, (H, D), dev)
    _dev_tensor(alpha, "alpha", torch.float32, (H,) if gate is not None else _alpha_shape(layer.cfg), dev)
    _dev_tensor(beta, "beta", torch.float32, (H,), dev)
    _dev_tensor(o, "o", torch.float32, (H, D), dev)
    _dev_tensor(n_in, "n_in", torch.int32, (layer.cfg.batch,), dev)
    if n_out is not None:
        _dev_tensor(n_out, "n_out", torch.int32, (layer.cfg.batch,), dev)
    if gate is not None:
        for name, t in (("A_log", gate.A_log), ("dt_bias", gate.dt_bias)):
            _dev_tensor(t, name, torch.float32, (layer.cfg.heads,), dev)
    _check(lib().leapq_step(ctypes.byref(layer.c), ctypes.byref(gate.c) if gate is not None else None, _ptr(n_in),
                            _ptr(n_out) if n_out is not None else None, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                            _ptr(beta), _ptr(o), _stream(stream, dev)), "leapq_step")


def leapq_fold(layer, stream=None):
    _check(lib().leapq_fold(ctypes.byref(layer.c), _stream(stream, layer.device)), "leapq_fold")


def leapq_dequant(layer, what, out, stream=None):
    _dev_tensor(out, "S_out", torch.float32, (layer.heads, D, D), layer.device)
    _check(lib().leapq_dequant(ctypes.byref(layer.c), int(what), _ptr(out), _stream(stream, layer.device)),
           "leapq_dequant")


def leapq_gdn_decode(cfg, S, q, k, v, alpha, beta, o, stream=None):
    """Dense baseline step in place on S (fp32 or bf16 [heads, 128, 128])."""
    H = cfg.batch * cfg.heads
    dev = S.device
    if S.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("S must be float32 or bfloat16")
    _dev_tensor(S, "S", S.dtype, (H, D, D), dev)
    dt = torch.bfloat16 if cfg.in_dtype == LEAPQ_BF16 else torch.float32
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(t, name, dt, (H, D), dev)
    _dev_tensor(alpha, "alpha", torch.float32, _alpha_shape(cfg), dev)
    _dev_tensor(beta, "beta", torch.float32, (H,), dev)
    _dev_tensor(o, "o", torch.float32, (H, D), dev)
    sd = LEAPQ_BF16 if S.dtype == torch.bfloat16 else LEAPQ_F32
    _check(lib().leapq_gdn_decode(ctypes.byref(cfg), sd, _ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                  _ptr(beta), _ptr(o), _stream(stream, dev)), "leapq_gdn_decode")


def leapq_version():
    return int(lib().leapq_version())
