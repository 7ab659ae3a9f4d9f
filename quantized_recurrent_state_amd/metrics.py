"""Algorithmic byte counts and step definitions of the decode path.

Algorithmic bytes are what each kernel must move between HBM and the chip
for one head (no re-reads, no dense fp32 state):

  append, with n records already in the window (token n+1):
      read   codes 128*128 + rho, sigma 2*512 + compensators C*(4+512)
             (C*(4+1024) for rank-one pairs a, b)
             + q, k, v 3*128*e_in + alpha, beta 8 + records n*(4+128*e_in+512)
      write  record 4+128*e_in+512 + output 512
  (a record holds gamma and u in fp32 and the key in the input dtype e_in,
  which stores the token's k exactly; with per-channel decay (KDA) alpha and
  each record's gamma are 128-vectors: 512 bytes in place of 4)
  fold of n records:
      read   boundary (codes, scales, compensators) + n records
      write  boundary
  dense GDN step (baselines): read + write the state, plus q, k, v, alpha,
      beta and the output.

"Recurrent-state quantization for linear attention: a first GPU kernel"
(Where the time goes) defines the per-token step of the windowed path as a
window's appends plus its fold, divided by the window length; the fold's
share of window time is fold / (appends + fold).
"""
D = 128


def boundary_bytes(C=4, rank1=False, bits=8):
    """Bytes of one head's boundary state: the codes (int8, or packed 6- or
    4-bit codes), rho, sigma, and C compensators (an index and a line, or an
    index and a pair a, b)."""
    return D * D * bits // 8 + 2 * D * 4 + C * (4 + D * 4 * (2 if rank1 else 1))


def record_bytes(in_bytes=2, channel=False, u_bytes=4):
    """Bytes of one record: gamma (a 128-vector with per-channel decay) in
    fp32, k in the input dtype, u in fp32 (or bf16 as a lossy option)."""
    return 4 * (D if channel else 1) + D * in_bytes + D * u_bytes


def append_bytes(n, C=4, in_bytes=2, channel=False, u_bytes=4, rank1=False, bits=8):
    """Algorithmic bytes of one head's append with n records present."""
    gates = 4 * (D if channel else 1) + 4
    rec = record_bytes(in_bytes, channel, u_bytes)
    read = boundary_bytes(C, rank1, bits) + 3 * D * in_bytes + gates + n * rec
    write = rec + D * 4
    return read + write


def fold_bytes(n, C=4, in_bytes=2, channel=False, rank1=False):
    return 2 * boundary_bytes(C, rank1) + n * record_bytes(in_bytes, channel)


def init_bytes(C=4):
    return D * D * 4 + boundary_bytes(C)


def window_bytes(W=16, C=4, in_bytes=2, channel=False):
    """Bytes of one head over a whole window: W appends and one fold."""
    return (sum(append_bytes(n, C, in_bytes, channel) for n in range(W)) +
            fold_bytes(W, C, in_bytes, channel))


def gdn_step_bytes(state_bytes=4, in_bytes=2, channel=False):
    """Dense per-token step: state read + write, inputs, output."""
    return 2 * D * D * state_bytes + 3 * D * in_bytes + 4 * (D if channel else 1) + 4 + D * 4


def step_ms(append_ms, fold_extra_ms, W=16):
    """Mean per-token step: W appends plus the fold's extra time, over W."""
    return (W * append_ms + fold_extra_ms) / W


def fold_budget_ms(append_ms, target_step_ms, W=16):
    """Largest fold time (beyond an append) that keeps the step at target."""
    return W * (target_step_ms - append_ms)


def fold_share(append_total, fold_total):
    """Fold time over window time (appends + fold)."""
    return fold_total / (append_total + fold_total)
