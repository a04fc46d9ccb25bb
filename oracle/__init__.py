"""Oracle: a plain, slow, float64 CPU definition of the ring-cache chunk-attention path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (no kernels, headers, helpers or tables) and never imports it.

What it computes (all in float64 unless a stored format fixes the precision):

* ``e4m3``      -- the FP8 e4m3fn codec and per-vector absmax quantisation
                   used when K and V are written into the cache.
* ``rope``      -- rotary position encoding on adjacent pairs.
* ``ring``      -- the circular KV cache: slot assignment, write-time RoPE and
                   FP8 quantisation, delta re-rotation, ring advance.
* ``attention`` -- block-causal chunk attention of new queries over every
                   cached slot with the additive cache bias.
* ``schedule``  -- the long-run schedule: position resets and bias ramps.
* ``memory``    -- per-key attention mass and the scored content memory's
                   greedy selection (top-M with diminishing returns per block).
* ``projection``-- the QKV projection on FP8 operands that feeds the write.

The method is described in: Runway Characters: Serving a 57B Video Diffusion
Transformer for Real-Time Conversation (abstract) -- ring cache, RoPE and FP8
quantisation once per write, delta rotation on position reset; video-conductor
(daydream), "Plastic Windows" -- lowering the cache attention bias during
prompt transitions; StreamLTX project page (Training) and "Why Live Video
Generation Still Struggles With Timing" (transcript) -- bidirectional inside a
block, backward-only across blocks, anchors plus a sliding window; StreamLTX
("Why a long take does not slow down") -- anchor, scored content memory and
FIFO eviction.

Parity pins for every function live in ``tests/test_oracle_*.py``.  The one
reading that no pin can fix is the scale of the pages' "bias=0.3" (parity
unpinned; the oracle takes the bias as an additive term on scaled logits).
"""
