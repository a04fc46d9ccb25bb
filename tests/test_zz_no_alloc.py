"""rc_chunk_attention_noalloc against rc_chunk_attention (with a workspace the
caller allocates) through the C ABI: two calls in a row on one GPU, the
second with fewer queries, in shapes that split the key range (so the
library's fixed scratch array holds the split partials).  Both entry points
run the same kernels with the same split, so the outputs and lse must agree
bit for bit; the first call is also checked against the oracle."""
import sys

import numpy as np
import pytest
import torch

from autoregressive_video_diffusion_ring_amd import (Ring, rc_attention_noalloc_limit, rc_attention_workspace_bytes,
                                                     rc_chunk_attention, rc_chunk_attention_noalloc)
from gpu_helpers import DEV, assert_attention_close, inputs, oracle_from_gpu, oracle_rows, to_np64

pytestmark = pytest.mark.gpu


def setup_module(_):
    if not torch.cuda.is_available():
        pytest.skip("no GPU", allow_module_level=True)


def run_both(ring, q, n_q, q_pos0, q_block0, bias):
    out_a = torch.empty((n_q, ring.H, ring.d), dtype=torch.bfloat16, device=DEV)
    out_b = torch.empty_like(out_a)
    lse_a = torch.empty((ring.H, n_q), dtype=torch.float32, device=DEV)
    lse_b = torch.empty_like(lse_a)
    need = rc_attention_workspace_bytes(ring.struct, n_q)
    assert 0 < need <= rc_attention_noalloc_limit(), need  # the shape splits, and fits the scratch
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    rc_chunk_attention(ring.struct, q, n_q, q_pos0, q_block0, n_q, bias, 0.0, out_a, lse_a, ws, need)
    rc_chunk_attention_noalloc(ring.struct, q, n_q, q_pos0, q_block0, n_q, bias, 0.0, out_b, lse_b)
    torch.cuda.synchronize()
    return out_a, lse_a, out_b, lse_b


def test_noalloc_matches_workspace_entry_point():
    print("\n[gpu] no-alloc attention: fp8 d=128 N=5788 H=8, calls of 100 then 40 queries", flush=True)
    sys.stdout.flush()
    rng = np.random.default_rng(71)
    N, H, d = 5788, 8, 128
    ring = Ring(N, H, d, "fp8", 10000.0, device=DEV)
    hist = 5031
    kt, _ = inputs(rng, "fp8", (hist, H, d))
    vt, _ = inputs(rng, "fp8", (hist, H, d))
    ring.write(kt, vt, 0, 0)
    ring.advance(hist)
    kt, _ = inputs(rng, "fp8", (700, H, d))
    vt, _ = inputs(rng, "fp8", (700, H, d))
    ring.write(kt, vt, hist, 1)
    orc = oracle_from_gpu(ring, 10000.0)
    for n_q in (100, 40):
        qt, q64 = inputs(rng, "fp8", (n_q, H, d))
        out_a, lse_a, out_b, lse_b = run_both(ring, qt, n_q, hist, 1, -0.5)
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), n_q
        assert torch.equal(lse_a, lse_b), n_q
        if n_q == 100:
            ref, _ = oracle_rows(orc, q64, np.arange(n_q), hist, 1, n_q, -0.5)
            assert_attention_close(to_np64(out_b), ref, "fp8")
