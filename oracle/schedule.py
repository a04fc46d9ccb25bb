"""Long-run streaming schedule: positions, resets and bias ramps (oracle).

Test infrastructure only (see ``oracle/__init__.py``).

Readings (the pages give the mechanisms, not the numbers):
* Positions are reset from time to time so that they stay bounded
  ("Why Live Video Generation Still Struggles With Timing", transcript:
  resetting or adjusting positional schedules; Runway Characters, abstract:
  a delta rotation when positions reset).  Here a reset happens before every
  chunk t that is a positive multiple of ``reset_every``; delta is minus the
  position of the oldest cached token, so the cache is rebased to start at 0.
* The cache bias is lowered and restored around prompt transitions
  (video-conductor, "Plastic Windows").  Here transition k starts at chunk
  ``first + k * spacing`` and the bias over its five chunks is
  [0, -depth/2, -depth, -depth/2, 0]: linear down over two chunks and back
  up over two, four intervals in all.
"""
from __future__ import annotations


def is_reset(t: int, reset_every: int) -> bool:
    return t > 0 and reset_every > 0 and t % reset_every == 0


def reset_delta(oldest_pos: int) -> int:
    """Delta that moves the oldest cached position to 0."""
    return -int(oldest_pos)


def chunk_pos0(t: int, n_new: int, n_slots: int, reset_every: int) -> int:
    """Position of the first token of chunk t when every reset rebases the
    full cache (n_slots tokens) to positions 0..n_slots-1."""
    if reset_every <= 0 or t < reset_every:
        return n_new * t
    return n_slots + n_new * (t % reset_every)


def bias_at(t: int, n_ramps: int = 10, first: int = 150, spacing: int = 200,
            depth: float = 4.0) -> float:
    """Cache bias for chunk t."""
    shape = (0.0, -depth / 2, -depth, -depth / 2, 0.0)
    for k in range(n_ramps):
        s = first + k * spacing
        if s <= t < s + len(shape):
            return shape[t - s]
    return 0.0
