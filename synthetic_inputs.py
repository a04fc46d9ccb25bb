"""Seeded synthetic inputs and workload shapes for the ring-cache chunk-attention path.

This module is shared by the tests, the benchmark and the oracle's checks.  It
holds no arithmetic of the method itself: it draws N(0,1) samples, rounds them
to the storage type the GPU receives (bf16 by round-to-nearest-even, or fp32),
and describes the workload shapes.  Both the HIP path and the oracle are fed
the exact same values: bf16 and fp32 both convert exactly to float64.

The workloads stand in for model activations of the streaming systems on the
pages (no weights or datasets exist here):

* Runway Characters: Serving a 57B Video Diffusion Transformer for Real-Time
  Conversation (abstract): 240 attention calls per chunk, each over a
  5,788-slot cache of which 757 tokens are new.
* StreamLTX project page (Training): one-second blocks with 3 fps video and
  25 fps audio latents, causal masks on every path.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "e4m3_codes",
    "bf16_bits_from_f32",
    "bf16_bits_to_f64",
    "normal_bf16",
    "normal_f32",
    "Workload",
    "WORKLOADS",
]


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even) and return the
    16-bit patterns as uint16.  Input preparation only: the GPU receives these
    bits, the oracle receives the same values as float64."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = (u + 0x7FFF + lsb) >> 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 values of bfloat16 bit patterns."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def e4m3_codes(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniformly random finite OCP e4m3fn bytes (magnitude codes 0..0x7E,
    random sign): synthetic FP8 weights, given to both sides as codes."""
    mag = rng.integers(0, 0x7F, size=shape, dtype=np.uint8)
    sign = rng.integers(0, 2, size=shape, dtype=np.uint8) << 7
    return mag | sign


def normal_bf16(rng: np.random.Generator, shape) -> tuple[np.ndarray, np.ndarray]:
    """N(0,1) samples drawn as float32 and rounded to bf16.

    Returns (bits uint16, values float64) with identical numeric content."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    bits = bf16_bits_from_f32(x)
    return bits, bf16_bits_to_f64(bits)


def normal_f32(rng: np.random.Generator, shape) -> tuple[np.ndarray, np.ndarray]:
    """N(0,1) samples as float32.  Returns (float32 array, float64 copy)."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return x, x.astype(np.float64)


@dataclass(frozen=True)
class Workload:
    """Shape of one workload.  Seeds are the 0-based workload index."""

    name: str
    heads: int
    head_dim: int
    n_slots: int
    n_new: int
    kv_dtype: str  # "f32", "bf16" or "fp8"
    rope_base: float
    seed: int
    cache_bias: float = 0.0
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    # Tiny case: 96 slots = 3 history blocks of 32, then 32 new tokens at
    # positions 96..127 written over the oldest block.
    "tiny": Workload("tiny", heads=2, head_dim=64, n_slots=96, n_new=32,
                     kv_dtype="f32", rope_base=10000.0, seed=0, cache_bias=-0.5,
                     extra={"block_len": 32, "n_hist_blocks": 3}),
    # One layer of a streaming chunk: 757 new over a 5,788-slot fp8 ring,
    # 240 calls per chunk (4 denoising passes x 60 layers).
    "stream": Workload("stream", heads=40, head_dim=128, n_slots=5788, n_new=757,
                       kv_dtype="fp8", rope_base=10000.0, seed=1, cache_bias=0.0,
                       extra={"n_hist": 5031, "layers": 60, "passes": 4}),
    # Ring wrap and position reset on the streaming shapes.
    "wrap": Workload("wrap", heads=40, head_dim=128, n_slots=5788, n_new=757,
                     kv_dtype="fp8", rope_base=10000.0, seed=2, cache_bias=0.0,
                     extra={"heads_at": (4000, 5400), "delta": -3000}),
    # Joint audio-video: 1-second blocks, 1152 video and 25 audio tokens,
    # 9 history blocks + the current one, bf16 caches, no RoPE.
    "av": Workload("av", heads=32, head_dim=128, n_slots=11520, n_new=1152,
                   kv_dtype="bf16", rope_base=0.0, seed=3, cache_bias=0.0,
                   extra={"video_block": 1152, "audio_block": 25, "blocks": 10}),
    # Six-path joint audio-video block (StreamLTX project page, Training and
    # Data): the first block carries one latent frame more (4 + 3k video
    # frames of 16 x 24 tokens, 26 + 25k audio frames), and three prompt
    # segments (blocks 0-3, 4-6, 7-9) feed the text cross-attention; the
    # prompt lengths are not on the page (96-160 tokens stand in).
    "av6": Workload("av6", heads=32, head_dim=128, n_slots=1536 + 9 * 1152, n_new=1152,
                    kv_dtype="bf16", rope_base=0.0, seed=5, cache_bias=0.0,
                    extra={"video_first": 1536, "video_block": 1152, "audio_first": 26, "audio_block": 25,
                           "blocks": 10, "segment_of_block": [0, 0, 0, 0, 1, 1, 1, 2, 2, 2],
                           "prompt_tokens": [128, 96, 160]}),
    # Long run: 2000 chunks with eviction, resets every 300 chunks and
    # 10 bias ramps 0 -> -4 -> 0.
    "longrun": Workload("longrun", heads=40, head_dim=128, n_slots=5788, n_new=757,
                        kv_dtype="fp8", rope_base=10000.0, seed=4, cache_bias=0.0,
                        extra={"chunks": 2000, "reset_every": 300, "ramps": 10}),
}
