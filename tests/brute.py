"""Arbitrary-precision brute force for tiny decode-attention cases (a pin for the
oracle, not a second oracle for the GPU).

It works on *logical* per-sequence arrays (no pool, no table), selects visible
keys by testing the span-02 page's visibility rule on every position
(``p <= last`` and, for sliding layers, ``qpos - p < window``), and forms the
softmax as ``exp(s_p) / sum exp(s_q)`` in 50-digit arithmetic with no max
subtraction.  Nothing here is shared with ``oracle/``.
"""
import mpmath

mpmath.mp.dps = 50


def _bf16(bits):
    # bf16 bits -> exact rational via float32 widening done by hand
    bits = int(bits)
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    if exp == 0:
        return sign * mpmath.mpf(man) * mpmath.mpf(2) ** (-133)
    return sign * (1 + mpmath.mpf(man) / 128) * mpmath.mpf(2) ** (exp - 127)


def attend(q_row, k_seq, v_seq, qpos, last, window):
    """One (row, head): q_row [hd] bits, k_seq/v_seq [ctx][hd] bits of its kv head."""
    hd = len(q_row)
    vis = [p for p in range(len(k_seq)) if p <= last and (window == 0 or qpos - p < window)]
    if not vis:
        return [mpmath.mpf(0)] * hd
    qv = [_bf16(x) for x in q_row]
    ex = {}
    for p in vis:
        s = mpmath.fsum(qv[d] * _bf16(k_seq[p][d]) for d in range(hd))
        ex[p] = mpmath.exp(s)
    z = mpmath.fsum(ex.values())
    return [mpmath.fsum(ex[p] * _bf16(v_seq[p][d]) for p in vis) / z for d in range(hd)]


def prep_head(x_bits, w_bits, cos_row, sin_row, rotary_dim, eps, rotate=True):
    """QK-norm + RoPE of one head in 50-digit arithmetic (a pin for the prep
    oracle).  The norm divides by the root of the mean square (plus eps); the
    weight (None = 1) scales each element; the first ``rotary_dim`` elements
    are rotated as complex numbers ``z_i = n_i + j n_{i + rotary_dim / 2}``
    multiplied by ``cos_i + j sin_i``.  Returns hd mpf values."""
    hd = len(x_bits)
    x = [_bf16(b) for b in x_bits]
    ms = mpmath.fsum(v * v for v in x) / hd
    r = 1 / mpmath.sqrt(ms + mpmath.mpf(eps))
    w = [mpmath.mpf(1)] * hd if w_bits is None else [_bf16(b) for b in w_bits]
    n = [x[d] * r * w[d] for d in range(hd)]
    y = list(n)
    if rotate and rotary_dim:
        h = rotary_dim // 2
        for i in range(h):
            z = mpmath.mpc(n[i], n[i + h]) * mpmath.mpc(mpmath.mpf(float(cos_row[i])), mpmath.mpf(float(sin_row[i])))
            y[i], y[i + h] = z.real, z.imag
    return y
