"""Pins of the CPU oracle's Otil-style block selection.

Page: "Otil: Accelerating Diffusion Model Inference via Communication-Efficient
Multi-GPU Parallelism", Key designs 1-3 (8x8 square blocks, cosine
dissimilarity between a block and its previous value, top-k over the blocks not
yet visited in the round, round restart when every block has been visited).
Checks: closed forms of the dissimilarity (identical, negated, scaled,
orthogonal and zero blocks), the round-robin guarantee that every block is sent
exactly once per round, the top-k property with ties to the lower index, and
the state update (sent blocks replace the receiver's copy exactly).
"""
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(2024)


def _grid(n_by, n_bx, m):
    return n_by * 8 * n_bx * 8, n_bx * 8, m


def _put_block(x, i, grid_w, val):
    x[oracle.bs_block_tokens(i, grid_w)] = val


def test_block_tokens_are_the_8x8_squares_in_raster_order():
    n, gw, m = _grid(2, 3, 4)
    seen = np.zeros(n, int)
    for i in range(6):
        tok = oracle.bs_block_tokens(i, gw)
        rows, cols = tok // gw, tok % gw
        assert rows.max() - rows.min() == 7 and cols.max() - cols.min() == 7
        assert rows.min() == 8 * (i // 3) and cols.min() == 8 * (i % 3)
        seen[tok] += 1
    assert np.all(seen == 1)


def test_dissimilarity_closed_forms():
    n, gw, m = _grid(2, 3, 16)
    b = RNG.standard_normal((n, m)).astype(np.float32)
    a = b.copy()                                  # block 0: identical -> 0
    t = [oracle.bs_block_tokens(i, gw) for i in range(6)]
    a[t[1]] = -b[t[1]]                            # negated -> 2
    a[t[2]] = 4.0 * b[t[2]]                       # positive power-of-two scale -> 0
    # block 3: orthogonal (disjoint channel supports) -> 1
    a[t[3]] = 0.0
    a[t[3], :8] = 1.0
    b[t[3]] = 0.0
    b[t[3], 8:] = 1.0
    a[t[4]] = 0.0                                 # one zero block -> 1
    a[t[5]] = 0.0                                 # both zero -> 0
    b[t[5]] = 0.0
    d = oracle.bs_scores(a, b, gw)
    assert d[0] == 0.0 and d[2] == 0.0 and d[5] == 0.0
    assert d[1] == 2.0 and d[3] == 1.0 and d[4] == 1.0


def test_dissimilarity_is_scale_invariant_and_symmetric():
    n, gw, m = _grid(1, 2, 8)
    a = RNG.standard_normal((n, m)).astype(np.float32)
    b = RNG.standard_normal((n, m)).astype(np.float32)
    d = oracle.bs_scores(a, b, gw)
    assert np.all((d > 0.5) & (d < 1.5))   # independent blocks: cosine near 0
    assert np.allclose(oracle.bs_scores(b, a, gw), d, rtol=0, atol=1e-15)
    assert np.allclose(oracle.bs_scores(8.0 * a, 0.25 * b, gw), d, rtol=0, atol=1e-15)


@pytest.mark.parametrize("K,keep", [(16, 4), (16, 5), (12, 12), (7, 3), (5, 1)])
def test_round_robin_sends_every_block_once_per_round(K, keep):
    visited = np.zeros(K, bool)
    rounds = 3
    steps_per_round = -(-K // keep)
    counts = np.zeros(K, int)
    for step in range(rounds * steps_per_round):
        d = RNG.random(K)
        sel, visited = oracle.bs_select(d, visited, keep)
        assert sel.size == (keep if (step % steps_per_round) < steps_per_round - 1 else K - keep * (steps_per_round - 1))
        counts[sel] += 1
        if (step + 1) % steps_per_round == 0:
            assert np.all(counts == (step + 1) // steps_per_round)


def test_selection_is_top_k_of_unvisited_with_ties_to_lower_index():
    K, keep = 10, 3
    visited = np.zeros(K, bool)
    visited[[1, 4]] = True
    d = np.array([0.5, 0.9, 0.7, 0.7, 0.95, 0.1, 0.7, 0.2, 0.3, 0.6])
    sel, vis = oracle.bs_select(d, visited, keep)
    # unvisited scores: 0:.5 2:.7 3:.7 5:.1 6:.7 7:.2 8:.3 9:.6 -> top 3 = {2, 3, 6} (.7 ties, lower index first)
    assert sel.tolist() == [2, 3, 6]
    assert vis.tolist() == [False, True, True, True, True, False, True, False, False, False]
    # brute force on random small cases
    for _ in range(200):
        K = RNG.integers(2, 12)
        keep = RNG.integers(1, K + 1)
        vis0 = RNG.random(K) < 0.4
        d = RNG.integers(0, 4, K) / 4.0          # many exact ties
        sel, _ = oracle.bs_select(d, vis0, keep)
        cand = np.arange(K) if vis0.all() else np.flatnonzero(~vis0)
        ranked = sorted(cand, key=lambda i: (-d[i], i))
        assert sel.tolist() == sorted(ranked[:keep])


@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
def test_state_update_and_receiver(in_dtype):
    n, gw, m = _grid(3, 4, 24)
    K, keep = 12, 5
    a = RNG.standard_normal((n, m)).astype(np.float32)
    if in_dtype == "bf16":
        a = oracle.bf16_round(a)
    ahat = (a + 0.1 * RNG.standard_normal((n, m))).astype(np.float32)
    o = oracle.bs_compress_tensor(a, ahat, grid_w=gw, keep=keep, visited=np.zeros(K, bool),
                                  in_dtype=in_dtype)
    sent = np.zeros(n, bool)
    for i in o["selected"]:
        sent[oracle.bs_block_tokens(i, gw)] = True
    assert o["selected"].size == keep
    assert np.array_equal(o["ahat"][sent].view(np.uint32), a[sent].view(np.uint32))
    assert np.all(o["e"][sent] == 0.0)
    assert np.array_equal(o["ahat"][~sent].view(np.uint32), ahat[~sent].view(np.uint32))
    assert np.array_equal(o["e"][~sent].view(np.uint32), (a[~sent] - ahat[~sent]).view(np.uint32))
    rec = oracle.bs_decompress_tensor(o["packed"], ahat, grid_w=gw, keep=keep, in_dtype=in_dtype)
    assert np.array_equal(rec.view(np.uint32), o["ahat"].view(np.uint32))
    in_bytes = 2 if in_dtype == "bf16" else 4
    assert o["packed"].size == oracle.tensor_bytes("bs", n, m, keep=keep, in_bytes=in_bytes)


def test_page_rule_scores_against_the_previous_step_not_the_last_sent_copy():
    # Two steps on three blocks, one block sent per step. Step 1: block 2
    # changes most (its sign flips) and is sent; block 0 changes a lot too (it
    # turns by 90 degrees) but is not sent, so the receiver keeps its step-0
    # copy. Step 2: block 0 does not change any more, block 1 turns by 45
    # degrees. The page compares each block with the same block one step
    # earlier: block 0 scores 0, block 1 scores 1 - cos 45, so block 1 is sent.
    # Comparing with the copy last sent instead would score block 0 at 1
    # (orthogonal to the receiver's copy) and send it.
    n, gw, m = _grid(1, 3, 8)
    tok = [oracle.bs_block_tokens(i, gw) for i in range(3)]
    u = np.zeros(m, np.float32)
    u[0] = 1.0
    w = np.zeros(m, np.float32)
    w[1] = 1.0
    a0 = np.zeros((n, m), np.float32)
    for i in range(3):
        a0[tok[i]] = u
    a1 = a0.copy()
    a1[tok[0]] = w                    # turned by 90 degrees: 1 - cos = 1
    a1[tok[2]] = -u                   # flipped: 1 - cos = 2
    a2 = a1.copy()
    a2[tok[1]] = u + w                # 45 degrees from a1's block 1
    vis = np.zeros(3, bool)
    s1 = oracle.bs_compress_tensor(a1, a0, grid_w=gw, keep=1, visited=vis, prev=a0, in_dtype="f32")
    assert s1["selected"].tolist() == [2]
    s2 = oracle.bs_compress_tensor(a2, s1["ahat"], grid_w=gw, keep=1, visited=s1["visited"],
                                   prev=a1, in_dtype="f32")
    assert s2["scores"][0] == 0.0
    assert s2["scores"][1] == pytest.approx(1 - np.sqrt(0.5), abs=1e-12)
    assert s2["selected"].tolist() == [1]
    alt = oracle.bs_compress_tensor(a2, s1["ahat"], grid_w=gw, keep=1, visited=s1["visited"],
                                    score="last_sent", in_dtype="f32")
    assert alt["scores"][0] == 1.0 and alt["selected"].tolist() == [0]
    # after the warm-up the reconstruction is the previous activation, so the
    # first step may pass prev=None
    s1b = oracle.bs_compress_tensor(a1, a0, grid_w=gw, keep=1, visited=vis, in_dtype="f32")
    assert np.array_equal(s1b["packed"], s1["packed"])


def test_selected_override_follows_the_given_blocks():
    n, gw, m = _grid(2, 2, 8)
    a = RNG.standard_normal((n, m)).astype(np.float32)
    ahat = RNG.standard_normal((n, m)).astype(np.float32)
    o = oracle.bs_compress_tensor(a, ahat, grid_w=gw, keep=2, visited=np.zeros(4, bool),
                                  in_dtype="f32", selected=np.array([3, 0]))
    assert o["selected"].tolist() == [0, 3]
    assert o["visited"].tolist() == [True, False, False, True]
    head = o["packed"][:12].view(np.uint32)
    assert head.tolist() == [2, 0, 3]
