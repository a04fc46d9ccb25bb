"""Pins for the long-run schedule: closed forms of positions, resets, ramps."""
from oracle.schedule import bias_at, chunk_pos0, is_reset, reset_delta


def test_positions_and_resets():
    N, n, R = 5788, 757, 300
    assert [chunk_pos0(t, n, N, R) for t in (0, 1, 299)] == [0, 757, 757 * 299]
    assert chunk_pos0(300, n, N, R) == N
    assert chunk_pos0(301, n, N, R) == N + n
    assert chunk_pos0(600, n, N, R) == N
    assert [t for t in range(2000) if is_reset(t, R)] == [300, 600, 900, 1200, 1500, 1800]
    # before the reset at t=300 the full cache holds positions pos0-N .. pos0-1
    oldest = chunk_pos0(300, n, N, 0) - N
    assert reset_delta(oldest) == -(757 * 300 - N)
    # the delta that rebases the cache also maps the next write to N
    assert chunk_pos0(300, n, N, 0) + reset_delta(oldest) == chunk_pos0(300, n, N, R)


def test_bias_ramps():
    b = [bias_at(t) for t in range(2000)]
    assert min(b) == -4.0 and max(b) == 0.0
    peaks = [t for t in range(2000) if b[t] == -4.0]
    assert peaks == [152 + 200 * k for k in range(10)]
    assert b[150:155] == [0.0, -2.0, -4.0, -2.0, 0.0]
    # no ramp touches a reset chunk
    assert all(b[t] == 0.0 for t in range(300, 2000, 300))
