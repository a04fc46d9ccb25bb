"""Pins for the oracle's scored content memory (oracle/memory.py and the
memory part of oracle/ring.py).

* key_mass: rows of the softmax sum to one (total mass = number of queries
  that see some slot); the Q = 0 closed form; equality with the attention
  oracle's output when V is the identity (out_i[s] is then p(i, s)); slot
  permutation invariance.
* select_memory: its kept set reaches the brute-force optimum of the
  objective over all subsets on small cases; gamma = 1 is top-M by score
  (library sort); a tiny gamma takes one token per block first.
* write_scored: hand-derived slot layouts, and invariants over long random
  runs (no token twice, the anchor untouched, n_mem = min(M, tokens ever
  evicted), the sliding part holds the most recent tokens); closed forms for
  scores increasing / decreasing with position (the memory then holds the
  most recently / earliest evicted tokens).
"""
import itertools
import math

import numpy as np
import pytest

from oracle.attention import chunk_attention
from oracle.memory import key_mass, memory_objective, select_memory, slot_score
from oracle.ring import Ring


def rand_cache(rng, H, N, d, blocks):
    k = rng.standard_normal((H, N, d))
    return k, np.asarray(blocks, dtype=np.int64)


# ---------------------------------------------------------------- key mass
@pytest.mark.parametrize("bias", [0.0, -0.7])
def test_mass_rows_sum_to_one(bias):
    rng = np.random.default_rng(0)
    H, N, d, n_q = 3, 40, 16, 12
    blocks = rng.integers(-1, 4, size=N)
    k, blk = rand_cache(rng, H, N, d, blocks)
    q = rng.standard_normal((n_q, H, d))
    m = key_mass(k, blk, q, 100, 1, 5, bias, 0.0, 10000.0)   # query blocks 1, 1.., 2.., 3..
    qb = 1 + np.arange(n_q) // 5
    sees = np.array([np.any((blk != -1) & (blk <= b)) for b in qb])
    assert np.allclose(m.sum(axis=1), sees.sum(), atol=1e-12)
    assert np.all(m[:, blk == -1] == 0) and np.all(m[:, blk > qb.max()] == 0)


def test_mass_zero_query_closed_form():
    rng = np.random.default_rng(1)
    H, N, d, n_q, beta = 2, 30, 8, 7, -0.9
    blk = np.array([0] * 10 + [1] * 8 + [2] * 7 + [-1] * 5)
    k = rng.standard_normal((H, N, d))
    q = np.zeros((n_q, H, d))
    m = key_mass(k, blk, q, 0, 2, n_q, beta, 0.0, 10000.0)
    w = np.where(blk == -1, 0.0, np.where(blk < 2, math.exp(beta), 1.0))
    expect = n_q * w / w.sum()
    assert np.allclose(m, expect[None, :], rtol=1e-13, atol=0)


def test_mass_equals_attention_with_identity_values():
    """With V = identity rows (d >= N), out_i[s] = p(i, s): the attention
    oracle's output, summed over queries, is the key mass."""
    rng = np.random.default_rng(2)
    H, N, d, n_q = 2, 24, 32, 9
    blk = rng.integers(0, 3, size=N)
    k = rng.standard_normal((H, N, d))
    v = np.zeros((H, N, d))
    v[:, np.arange(N), np.arange(N)] = 1.0
    q = rng.standard_normal((n_q, H, d))
    out, _ = chunk_attention(k, v, blk, q, 50, 1, 4, -0.4, 0.0, 10000.0)
    m = key_mass(k, blk, q, 50, 1, 4, -0.4, 0.0, 10000.0)
    assert np.allclose(out.sum(axis=0)[:, :N], m, atol=1e-13)


def test_mass_slot_permutation():
    rng = np.random.default_rng(3)
    H, N, d, n_q = 2, 33, 16, 10
    blk = rng.integers(-1, 3, size=N)
    k = rng.standard_normal((H, N, d))
    q = rng.standard_normal((n_q, H, d))
    perm = rng.permutation(N)
    a = key_mass(k, blk, q, 7, 2, n_q, -0.3, 0.0, 10000.0)
    b = key_mass(k[:, perm], blk[perm], q, 7, 2, n_q, -0.3, 0.0, 10000.0)
    assert np.allclose(a[:, perm], b, atol=1e-13)


# ---------------------------------------------------------------- selection
def scores_for(rng, H, N, kind="cont"):
    if kind == "ties":
        return rng.integers(0, 3, size=(H, N)).astype(np.float32)
    return rng.uniform(0, 1, size=(H, N)).astype(np.float32)


@pytest.mark.parametrize("seed", range(12))
def test_selection_reaches_brute_force_optimum(seed):
    rng = np.random.default_rng(100 + seed)
    N, H = 12, 2
    blk = rng.integers(0, 4, size=N)
    ks = scores_for(rng, H, N, "ties" if seed % 3 == 0 else "cont")
    cand = sorted(rng.choice(N, size=rng.integers(1, 11), replace=False).tolist())
    M = int(rng.integers(1, 8))
    gamma = [1.0, 0.5, 0.25, 0.9, 0.01][seed % 5]
    picks = select_memory(cand, blk, ks, M, gamma)
    assert len(picks) == min(M, len(cand)) and len(set(picks)) == len(picks) and set(picks) <= set(cand)
    best = max(memory_objective(c, blk, ks, gamma)
               for c in itertools.combinations(cand, min(M, len(cand))))
    got = memory_objective(picks, blk, ks, gamma)
    assert got >= best * (1 - 1e-12)


def test_selection_gamma_one_is_top_m():
    rng = np.random.default_rng(7)
    N, H, M = 60, 3, 17
    blk = rng.integers(0, 5, size=N)
    cand = list(range(N))
    # distinct scores: exactly the top M by score, in score order
    ks = rng.uniform(0, 1, size=(H, N)).astype(np.float32)
    total = np.array([slot_score(ks, s) for s in range(N)])
    assert select_memory(cand, blk, ks, M, 1.0) == np.argsort(-total, kind="stable")[:M].tolist()
    # many ties: the kept scores are the M largest (which tied slot stays is the tie rule's)
    ks = rng.integers(0, 6, size=(H, N)).astype(np.float32)
    total = ks.astype(np.float64).sum(axis=0)
    picks = select_memory(cand, blk, ks, M, 1.0)
    assert sorted(total[picks].tolist()) == sorted(np.sort(total)[::-1][:M].tolist())


def test_selection_tiny_gamma_spreads_over_blocks():
    """gamma -> 0: every block's best token first (blocks by their best
    score), then every block's second, and so on."""
    blk = np.array([0, 0, 0, 1, 1, 2, 2, 2, 2])
    ks = np.array([[5, 4, 3, 9, 1, 2, 8, 7, 6]], dtype=np.float32)
    picks = select_memory(list(range(9)), blk, ks, 6, 1e-20)
    assert picks == [3, 6, 0, 7, 1, 4]   # bests 9 (b1), 8 (b2), 5 (b0); then 7 (b2), 4 (b0), 1 (b1)


def test_slot_score_is_float64_head_sum():
    ks = np.array([[1.0], [2.0 ** -30], [-1.0 + 2.0 ** -23]], dtype=np.float32)
    assert slot_score(ks, 0) == (1.0 + 2.0 ** -30) + (-1.0 + 2.0 ** -23)


# ---------------------------------------------------------------- scored ring
def zeros(n):
    z = np.zeros((n, 1, 2))
    return z, z


def test_scored_write_by_hand():
    """N 12, anchor 2, memory 3 (slots 9..11), sliding part 2..8 (7 slots),
    chunks of 3 tokens; chunk b has positions 3b..3b+2.  Scores favour even
    positions (score = 1 for even, 0.5 for odd), gamma = 1."""
    N, A, M, n = 12, 2, 3, 3
    ring = Ring(N, 1, 2, "f32", 0.0, n_anchor=A, n_memory=M)
    def score():
        return np.where(ring.slot_pos % 2 == 0, 1.0, 0.5).astype(np.float32)[None, :]
    for b in range(3):                     # slots 0..8 fill: nothing evicted yet
        ring.write_scored(*zeros(n), n, 3 * b, b, score(), 1.0)
        ring.advance(n)
    assert ring.n_mem == 0 and ring.head == 2
    # chunk 3 overwrites slots 2, 3, 4 = positions 2, 3, 4 (blocks 0, 1, 1)
    ring.write_scored(*zeros(n), n, 9, 3, score(), 1.0)
    ring.advance(n)
    assert ring.n_mem == 3
    assert ring.slot_pos[9:].tolist() == [2, 3, 4] and ring.slot_block[9:].tolist() == [0, 1, 1]
    # chunk 4 overwrites slots 5, 6, 7 = positions 5, 6, 7; candidates 2, 3, 4 (memory) + 5, 6, 7:
    # even positions 2, 4, 6 score 1 -> memory keeps 2 and 4 in place, 6 moves into slot 10
    ring.write_scored(*zeros(n), n, 12, 4, score(), 1.0)
    assert ring.slot_pos[9:].tolist() == [2, 6, 4] and ring.slot_block[9:].tolist() == [0, 2, 1]
    assert ring.slot_pos[:2].tolist() == [0, 1] and ring.slot_block[5:8].tolist() == [4, 4, 4]
    assert ring.n_mem == 3 and ring.n_hist == 6   # anchor 2 + 4 sliding history tokens


@pytest.mark.parametrize("N,A,M,n,gamma,chunks", [(40, 0, 9, 5, 1.0, 30), (40, 6, 9, 7, 0.5, 30),
                                                   (25, 3, 4, 4, 0.25, 40), (30, 0, 12, 6, 1.0, 25)])
def test_scored_ring_invariants(N, A, M, n, gamma, chunks):
    rng = np.random.default_rng(N * 7 + M)
    ring = Ring(N, 2, 2, "f32", 0.0, n_anchor=A, n_memory=M)
    E = N - M
    evicted_total = 0
    for b in range(chunks):
        ks = rng.uniform(0, 1, size=(2, N)).astype(np.float32)
        before = ring.n_hist
        ring.write_scored(*(np.zeros((n, 2, 2)),) * 2, n, n * b, b, ks, gamma)
        evicted_total += before - ring.n_hist
        # a second pass of the same chunk changes nothing in the memory
        mem = (ring.slot_pos[E:].copy(), ring.slot_block[E:].copy())
        ring.write_scored(*(np.ones((n, 2, 2)),) * 2, n, n * b, b, ks, gamma)
        assert np.array_equal(ring.slot_pos[E:], mem[0]) and np.array_equal(ring.slot_block[E:], mem[1])
        ring.advance(n)
        written = ring.slot_block != -1
        toks = list(zip(ring.slot_pos[written].tolist(), ring.slot_block[written].tolist()))
        assert len(toks) == len(set(toks))                                  # no token twice
        assert ring.n_mem == min(M, evicted_total) == np.count_nonzero(ring.slot_block[E:] != -1)
        total = n * (b + 1)
        assert np.array_equal(ring.slot_pos[:A][ring.slot_block[:A] != -1], np.arange(min(A, total)))
        fifo = np.sort(ring.slot_pos[A:E][ring.slot_block[A:E] != -1])
        assert np.array_equal(fifo, np.arange(max(A, total - (E - A)), total))
        mem_pos = ring.slot_pos[E:][ring.slot_block[E:] != -1]
        assert np.all(mem_pos < max(A, total - (E - A))) and np.all(mem_pos >= A)


@pytest.mark.parametrize("increasing", [True, False])
def test_scored_ring_monotone_scores(increasing):
    """gamma = 1 with scores that rise (fall) with position: the memory holds
    the M most recently (earliest) evicted tokens."""
    N, A, M, n = 30, 0, 8, 5
    ring = Ring(N, 1, 2, "f32", 0.0, n_anchor=A, n_memory=M)
    E = N - M
    for b in range(12):
        sp = ring.slot_pos.astype(np.float64)
        ks = (sp + 1 if increasing else 1.0 / (sp + 1)).astype(np.float32)[None, :]
        ring.write_scored(*zeros(n), n, n * b, b, ks, 1.0)
        ring.advance(n)
        total = n * (b + 1)
        n_ev = max(0, total - E)                      # tokens pushed out of the sliding part
        mem = np.sort(ring.slot_pos[E:][ring.slot_block[E:] != -1])
        expect = np.arange(max(0, n_ev - M), n_ev) if increasing else np.arange(min(M, n_ev))
        assert np.array_equal(mem, expect)


def test_memory_argument_checks():
    with pytest.raises(ValueError):
        Ring(10, 1, 2, "f32", 0.0, n_anchor=4, n_memory=6)
    with pytest.raises(ValueError):
        Ring(10, 1, 2, "f32", 0.0, first_slot=8, n_memory=3)
    ring = Ring(10, 1, 2, "f32", 0.0, n_anchor=2, n_memory=3)
    with pytest.raises(ValueError):
        ring.write_scored(*zeros(6), 6, 0, 0, np.zeros((1, 10), np.float32), 1.0)   # > E - A = 5
    with pytest.raises(ValueError):
        ring.write_scored(*zeros(2), 2, 0, 0, np.zeros((1, 10), np.float32), 0.0)   # gamma not in (0, 1]
    assert ring.state() == (0, 0, 0, 0, 0, 0)
