"""Exact-arithmetic brute-force model of NVFP4 quantisation, for pinning the oracle.

Written independently of oracle/ (no shared code): values are Python
Fractions, every fp32 rounding is done by `round_f32` below, and every
"nearest representable value" is an argmin over the full list of values of
the format.  Slow; meant for tiny inputs (a few 16-element blocks).
"""
from fractions import Fraction

F = Fraction

FLT_MAX = (F(2) - F(2) ** -23) * F(2) ** 127

# E2M1 magnitudes by code 0..7 (OCP MX FP4: 1 sign, 2 exponent bits, 1 mantissa bit)
E2M1_MAGS = [F(0), F(1, 2), F(1), F(3, 2), F(2), F(3), F(4), F(6)]


def e4m3_finite_positive():
    """(byte, value) for every finite non-negative E4M3 value (OCP: bias 7, max 448)."""
    out = []
    for b in range(0x7F):  # 0x7F is NaN
        e, m = b >> 3, b & 7
        v = F(m, 512) if e == 0 else F(8 + m, 8) * F(2) ** (e - 7)
        out.append((b, v))
    return out


E4M3_LIST = e4m3_finite_positive()
E4M3_VAL = dict(E4M3_LIST)


def round_f32(q):
    """Nearest IEEE binary32 value to the rational q, ties to even; None on overflow."""
    if q == 0:
        return F(0)
    s = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = F(2) ** (e - 23)
    k = a / quantum
    n = k.numerator // k.denominator
    rem = k - n
    if rem > F(1, 2) or (rem == F(1, 2) and n % 2 == 1):
        n += 1
    v = n * quantum
    if v > FLT_MAX:
        return None
    return s * v


def bf16_bits_to_fraction(u16):
    """(sign_bit, |value| as Fraction) of a bf16 bit pattern (finite only)."""
    s = (u16 >> 15) & 1
    e = (u16 >> 7) & 0xFF
    m = u16 & 0x7F
    assert e != 0xFF
    if e == 0:
        mag = F(m, 128) * F(2) ** -126
    else:
        mag = F(128 + m, 128) * F(2) ** (e - 127)
    return s, mag


def nearest_e4m3(t):
    """Byte of the E4M3 value nearest to t >= 0, ties to the even byte."""
    best = None
    for b, v in E4M3_LIST:
        d = abs(t - v)
        if best is None or d < best[0] or (d == best[0] and b % 2 == 0):
            best = (d, b)
    return best[1]


def nearest_e2m1_code(a):
    """Magnitude code nearest to a >= 0, ties to the even code."""
    best = None
    for c, v in enumerate(E2M1_MAGS):
        d = abs(a - v)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def sr_e2m1_code(a, u16):
    """Stochastic rounding of a >= 0 with the 16-bit draw u16.

    The two neighbours lo <= a < hi on the E2M1 grid; round up iff
    u16 < floor((a - lo) / (hi - lo) * 2^16).  a >= 6 gives 6.
    """
    if a >= 6:
        return 7
    lo_c = max(c for c, v in enumerate(E2M1_MAGS) if v <= a)
    lo, hi = E2M1_MAGS[lo_c], E2M1_MAGS[lo_c + 1]
    r = (a - lo) / (hi - lo)
    P = (r * 65536).numerator // (r * 65536).denominator
    return lo_c + 1 if u16 < P else lo_c


def tensor_scale(amax):
    if amax == 0:
        return F(1)
    s = round_f32(F(2688) / amax)
    return FLT_MAX if s is None else s


def quantize_blocks(x_bits, blocks, draws=None):
    """Quantise elements of x (list of bf16 bit patterns) grouped into blocks.

    blocks: list of lists of element indices (each one scale block).
    draws: None for round-to-nearest-even, else list of u16 per element.
    Returns (codes per element, scale byte per block, amax, s_enc).
    """
    vals = [bf16_bits_to_fraction(u) for u in x_bits]
    amax = max((v for _, v in vals), default=F(0))
    s_enc = tensor_scale(amax)
    codes = [None] * len(x_bits)
    sbytes = []
    for blk in blocks:
        am = max(vals[i][1] for i in blk)
        t1 = round_f32(am / 6)
        t = round_f32(t1 * s_enc)
        if t is None:
            t = FLT_MAX * 2  # overflow: nearest finite E4M3 is 448 either way
        sb = nearest_e4m3(t)
        sbytes.append(sb)
        S = E4M3_VAL[sb]
        f = F(0)
        if S > 0:
            f = round_f32(s_enc / S)
            if f is None:  # overflowing factor is clamped to FLT_MAX
                f = FLT_MAX
        for i in blk:
            sgn, mag = vals[i]
            y = round_f32(mag * f)
            if y is None:  # fp32 overflow: saturates like any |y| > 6
                y = FLT_MAX * 2
            if draws is None:
                c = nearest_e2m1_code(y)
            else:
                c = sr_e2m1_code(y, draws[i])
            codes[i] = (sgn << 3) | c
    return codes, sbytes, amax, s_enc


# --- MXFP4 (32-element blocks, UE8M0 scales, no tensor scale) --------------

def mx_exponent(amax):
    """The shared exponent e of an MXFP4 block: the integer with
    4 <= amax * 2^-e < 8 (amax * 2^-e then rounds onto [4, 6], the top binade
    of E2M1), clamped to [-127, 127]; -127 for amax = 0.  Found by search."""
    if amax == 0:
        return -127
    e = 0
    while amax * F(2) ** -e >= 8:
        e += 1
    while amax * F(2) ** -e < 4:
        e -= 1
    return min(max(e, -127), 127)


def mx_quantize_block(x_bits, draws=None):
    """(codes, scale byte) of one MXFP4 block given as bf16 bit patterns."""
    vals = [bf16_bits_to_fraction(u) for u in x_bits]
    e = mx_exponent(max(v for _, v in vals))
    codes = []
    for i, (sgn, mag) in enumerate(vals):
        y = round_f32(mag * F(2) ** -e)
        c = nearest_e2m1_code(y) if draws is None else sr_e2m1_code(y, draws[i])
        codes.append((sgn << 3) | c)
    return codes, e + 127
