"""Arithmetic identities that the HIP kernels rely on to give the oracle's bits
with fewer instructions, checked exhaustively on the CPU (no GPU, no oracle).

The first revision's tier transforms a stored group back as RN32(RN64(c * t))
with c = RN64(2^-2.5) (DAMP arXiv HTML, section 3.2 Eq.(3): the normalized
block-32 Hadamard transform).  Where t is an FP32 value (the decode's integer
inverse transform makes it one), the kernel computes fma(t, c_hi, RN32(t c_lo))
with c_hi = RN32(c) and c_lo = RN32(c - c_hi) in FP32 instead.  Both sides
scale exactly with powers of two while every product stays normal, so the
identity holds for every such t if it holds for every significand
t in [2^23, 2^24), which this test checks one by one."""
import numpy as np

C = float.fromhex("0x1.6a09e667f3bcdp-3")       # RN64(sqrt 2) / 8
C_HI = np.float32(C)
C_LO = np.float32(C - float(C_HI))


def _rn32_of_sum(p, a):
    """RN32(p + a), exactly, for float64 arrays with |a| <= |p|: s = RN64(p + a)
    rounds to RN32(p + a) unless it sits exactly on a midpoint between two FP32
    values (RN64 cannot cross one), where the error e = p + a - s decides."""
    s = p + a
    e = a - (s - p)                                # exact (Fast2Sum)
    r = s.astype(np.float32)
    rd = r.astype(np.float64)
    up = s > rd
    other = np.where(up, np.nextafter(r, np.float32(np.inf)), np.nextafter(r, np.float32(-np.inf)))
    mid = (s != rd) & (np.abs(s - rd) == np.abs(other.astype(np.float64) - s))
    pick_other = mid & (((e > 0) & up) | ((e < 0) & ~up))
    return np.where(pick_other, other, r)


def test_split_constant_scaling_equals_fp64_scaling_for_every_significand():
    bad_split = bad_plain = 0
    step = 1 << 21
    for lo in range(1 << 23, 1 << 24, step):
        t32 = np.arange(lo, lo + step, dtype=np.float64).astype(np.float32)
        t = t32.astype(np.float64)
        ref = (t * C).astype(np.float32)                      # RN32(RN64(c t))
        a = (t32 * C_LO).astype(np.float64)                   # RN32(t c_lo), an FP32 product
        got = _rn32_of_sum(t * float(C_HI), a)                # fma: t c_hi is exact in FP64
        bad_split += int(np.count_nonzero(got != ref))
        bad_plain += int(np.count_nonzero((t32 * C_HI) != ref))
    assert bad_split == 0
    # the check discriminates: the FP32 constant alone misses often
    assert bad_plain > 100_000


def test_rn32_of_sum_on_constructed_midpoints():
    one = 1.0
    ulp = 2.0 ** -23
    mid = one + ulp / 2                                       # between 1 and 1 + ulp
    p = np.array([mid, mid, mid, 3 * 2.0 ** 60])
    a = np.array([2.0 ** -60, -2.0 ** -60, 0.0, 2.0 ** 10])
    got = _rn32_of_sum(p, a)
    assert got[0] == np.float32(one + ulp)                    # above the midpoint
    assert got[1] == np.float32(one)                          # below it
    assert got[2] == np.float32(one)                          # a tie: to even
    assert got[3] == np.float32(3 * 2.0 ** 60)
