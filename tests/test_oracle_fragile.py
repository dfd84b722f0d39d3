"""Pins of oracle.lamp.fragile_flags, the statistic the parity reports count
as "within one fp32 ulp of a threshold" (CPU).

The values are worked by hand from the two stages of the look-ahead test
(figure captions: delta, tau): an entry is sensitive iff its exponential,
rounded to e4m3, is at least delta and its |logit| is at least T2.  Each
case puts one statistic a known number of fp32 steps from its threshold in
one chosen sub-block, so a wrong direction, a wrong step count or a wrong
sub-block index fails a case."""
import numpy as np

from oracle import lamp as L

T2 = float(np.float32(16 * 0.5 * np.log2(np.e)))   # tau = 2^-1
DELTA = 2.0 ** -8
# fp32 exponential at the e4m3 midpoint between 2^-9 and 2^-8: it rounds to
# the even code, 2^-8 = delta, so it passes the first stage; one fp32 step
# below it rounds to 2^-9 and fails
MID = 1.5 * 2.0 ** -9


def _steps(x, k):
    y = np.float32(x)
    for _ in range(abs(k)):
        y = np.nextafter(y, np.float32(np.inf if k > 0 else -np.inf))
    return float(y)


def _tile(c, e_val, s_val):
    """One row, 64 keys; entry 16c+5 carries (e_val, s_val); every other
    entry has e = 2^-20 (rounds to 0) and logit 0, so it is inactive."""
    e = np.full((1, 64), 2.0 ** -20)
    s2 = np.zeros((1, 64))
    e[0, 16 * c + 5] = e_val
    s2[0, 16 * c + 5] = s_val
    vis = np.ones((1, 64), dtype=bool)
    return e, s2, vis


def _bits(flags):
    return sum(int(f) << c for c, f in enumerate(flags))


def test_mid_point_exponential_is_what_the_first_stage_decides():
    from oracle.formats import round_e4m3
    assert round_e4m3(np.array([MID]))[0] == DELTA
    assert round_e4m3(np.array([_steps(MID, -1)]))[0] == 2.0 ** -9


def test_logit_one_step_below_threshold():
    e, s2, vis = _tile(2, 0.5, _steps(T2, -1))
    assert _bits(L.fragile_flags(e, s2, vis, DELTA, T2, 1)) == 0b0100
    e, s2, vis = _tile(2, 0.5, -_steps(T2, -1))          # negative logit: |s2|
    assert _bits(L.fragile_flags(e, s2, vis, DELTA, T2, 1)) == 0b0100


def test_logit_at_threshold_is_fragile_and_three_steps_above_needs_four():
    e, s2, vis = _tile(1, 0.5, T2)                        # passes, one step down fails
    assert _bits(L.fragile_flags(e, s2, vis, DELTA, T2, 1)) == 0b0010
    e, s2, vis = _tile(3, 0.5, _steps(T2, 3))             # three steps down still reach T2
    assert _bits(L.fragile_flags(e, s2, vis, DELTA, T2, 1)) == 0
    assert _bits(L.fragile_flags(e, s2, vis, DELTA, T2, 3)) == 0
    assert _bits(L.fragile_flags(e, s2, vis, DELTA, T2, 4)) == 0b1000


def test_exponential_one_step_below_the_delta_boundary():
    e, s2, vis = _tile(0, _steps(MID, -1), 2 * T2)
    assert _bits(L.fragile_flags(e, s2, vis, DELTA, T2, 1)) == 0b0001
    e, s2, vis = _tile(0, _steps(MID, 2), 2 * T2)
    assert _bits(L.fragile_flags(e, s2, vis, DELTA, T2, 1)) == 0
    assert _bits(L.fragile_flags(e, s2, vis, DELTA, T2, 3)) == 0b0001


def test_both_statistics_must_reach_their_thresholds():
    # the exponential is far below delta: no logit can flag the entry
    e, s2, vis = _tile(2, 2.0 ** -12, T2)
    assert _bits(L.fragile_flags(e, s2, vis, DELTA, T2, 1)) == 0
    # first stage off (delta <= 0): only the logit decides
    assert _bits(L.fragile_flags(e, s2, vis, 0.0, T2, 1)) == 0b0100
    # masked entries never count
    vis[0, 16 * 2 + 5] = False
    assert _bits(L.fragile_flags(e, s2, vis, 0.0, T2, 1)) == 0
