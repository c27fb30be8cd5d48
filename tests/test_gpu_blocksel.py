"""GPU parity of Otil-style block selection (RC_BLOCKSEL) against the CPU oracle.

Page: "Otil: Accelerating Diffusion Model Inference via Communication-Efficient
Multi-GPU Parallelism", Key designs 1-3: blocks are scored against the same
block at the previous step (the plan keeps that activation); the option
RC_BS_SCORE_LAST_SENT scores against the receiver's copy instead, and both are
checked. Every step is teacher-forced (the oracle starts from the GPU's
previous ahat and round state). The choice of
blocks rests on fp64 cosine scores whose last bits depend on summation order,
so the selection is checked for what is unique: if it equals the oracle's it
must match exactly; otherwise it must still be a valid top-k of the oracle's
scores within 1e-12, and the oracle re-run with that selection. Given the
selection, packed bytes (header, values, padding), e_t, ahat_t and the
receiver state must match bit for bit; over a round every block is sent once.
"""
import numpy as np
import pytest
import torch

from gpu_harness import DEV, bits, lib_view_f32, oracle, say, synth, to_device
from activation_residual_compression_amd import librescomp as rc

pytestmark = pytest.mark.gpu


def _valid_topk(sel, d, visited, keep, tol=1e-12):
    vis = np.array(visited, bool)
    if vis.all():
        vis[:] = False
    cand = np.flatnonzero(~vis)
    if len(sel) != min(keep, cand.size) or np.any(vis[sel]):
        return False
    rest = np.setdiff1d(cand, sel)
    return rest.size == 0 or d[sel].min() >= d[rest].max() - tol


def _run(wl, grid_w, keep, steps, check=None, zero_step=False, last_sent=False):
    B, n, m, dtype = wl.nb, wl.n, wl.m, wl.dtype
    K = n // 64
    in_dtype = "bf16" if dtype == "bf16" else "f32"
    score = "last_sent" if last_sent else "prev"
    flags = rc.RC_BS_SCORE_LAST_SENT if last_sent else 0
    with rc.Plan((B, n, m), dtype, "bs", grid_w=grid_w, keep_blocks=keep, flags=flags) as plan:
        assert plan.tensor_packed_bytes == oracle.tensor_bytes(
            "bs", n, m, keep=keep, in_bytes=2 if dtype == "bf16" else 4)
        _, a0 = wl.next()
        a = to_device(a0, dtype)
        ahat = a.float().clone()
        recon = ahat.clone()
        e = torch.zeros_like(ahat)
        packed = torch.empty(plan.packed_bytes, dtype=torch.uint8, device=DEV)
        prev = lib_view_f32(a0, dtype).copy()      # sender state (GPU's ahat)
        prev_a = lib_view_f32(a0, dtype).copy()    # the previous step's activation
        visited = [np.zeros(K, bool) for _ in range(B)]
        sent = [np.zeros(K, int) for _ in range(B)]
        tb = plan.tensor_packed_bytes
        for t in range(1, steps):
            if zero_step and t == 1:
                at = a0
            else:
                _, at = wl.next()
            a.copy_(to_device(at, dtype))
            packed.fill_(0xA5)
            plan.compress(a, ahat, e, packed)
            plan.decompress(packed, recon)
            torch.cuda.synchronize()
            pk, eh, ah, rh = packed.cpu().numpy(), e.cpu().numpy(), ahat.cpu().numpy(), recon.cpu().numpy()
            assert np.array_equal(bits(rh), bits(ah)), "receiver differs from sender"
            af = lib_view_f32(at, dtype)
            for b in (range(B) if check is None else check):
                tp = pk[b * tb:(b + 1) * tb]
                head = tp[:4 * (1 + keep)].view(np.uint32)
                gsel = head[1:1 + head[0]].astype(np.int64)
                o = oracle.bs_compress_tensor(af[b], prev[b], grid_w=grid_w, keep=keep,
                                              visited=visited[b], prev=prev_a[b], score=score,
                                              in_dtype=in_dtype)
                same = np.array_equal(gsel, o["selected"])
                say("[gpu] bs %s t=%d b=%d sent %d blocks, same as oracle: %s" % (score, t, b, gsel.size, same))
                if not same:
                    assert _valid_topk(gsel, o["scores"], visited[b], keep)
                    o = oracle.bs_compress_tensor(af[b], prev[b], grid_w=grid_w, keep=keep,
                                                  visited=visited[b], prev=prev_a[b], score=score,
                                                  in_dtype=in_dtype, selected=gsel)
                assert np.array_equal(tp, o["packed"])
                assert np.array_equal(bits(eh[b]), bits(o["e"]))
                assert np.array_equal(bits(ah[b]), bits(o["ahat"]))
                visited[b] = o["visited"]
                sent[b][gsel] += 1
            prev = ah
            prev_a = af
        return sent


@pytest.mark.parametrize("last_sent", [False, True])
def test_latent_rounds_every_block_once(last_sent):
    wl = synth.LatentWorkload(batch=2, height=32, width=64, m=64, steps=10)
    K, keep = 32, 8
    sent = _run(wl, 64, keep, steps=9, last_sent=last_sent)   # 8 compressed steps = 2 full rounds
    for s in sent:
        assert np.all(s == 2)


@pytest.mark.parametrize("keep", [1, 5, 32])
@pytest.mark.parametrize("last_sent", [False, True])
def test_latent_keep_sizes(keep, last_sent):
    wl = synth.LatentWorkload(batch=2, height=32, width=64, m=64, steps=5)
    _run(wl, 64, keep, steps=5, last_sent=last_sent)


def test_page_rule_and_last_sent_copy_pick_different_blocks():
    """The hand-built two-step case of the oracle pins (one block flips and is
    sent, one turns by 90 degrees and is not, then a third turns by 45 degrees):
    the page's rule sends the third block at step 2, the last-sent option the
    second; the GPU follows each rule."""
    gw, m = 24, 8
    n = 8 * gw
    tok = [oracle.bs_block_tokens(i, gw) for i in range(3)]
    u, w = np.zeros(m, np.float32), np.zeros(m, np.float32)
    u[0], w[1] = 1.0, 1.0
    a0 = np.zeros((n, m), np.float32)
    for i in range(3):
        a0[tok[i]] = u
    a1 = a0.copy()
    a1[tok[0]] = w
    a1[tok[2]] = -u
    a2 = a1.copy()
    a2[tok[1]] = u + w
    for flags, want in ((0, 1), (rc.RC_BS_SCORE_LAST_SENT, 0)):
        with rc.Plan((1, n, m), "f32", "bs", grid_w=gw, keep_blocks=1, flags=flags) as plan:
            ahat = to_device(a0[None], "f32")
            e = torch.zeros_like(ahat)
            packed = torch.empty(plan.packed_bytes, dtype=torch.uint8, device=DEV)
            heads = []
            for a in (a1, a2):
                plan.compress(to_device(a[None], "f32"), ahat, e, packed)
                torch.cuda.synchronize()
                heads.append(packed.cpu().numpy()[:8].view(np.uint32).tolist())
            say("[gpu] bs two-step case flags %d: %s" % (flags, heads))
            assert heads == [[1, 2], [1, want]]


@pytest.mark.parametrize("n,m,grid_w,keep", [(64, 4, 8, 1), (128, 8, 16, 1), (128, 4, 8, 2)])
def test_smallest_grids(n, m, grid_w, keep):
    # one 8 x 8 block (sent every step), one row of two blocks, and a column
    # of two blocks sent together; 4 to 8 channels
    _run(synth.WalkWorkload(batch=2, n=n, m=m, steps=4), grid_w, keep, steps=4)


def test_fp32_input_and_ragged_round():
    # 24 x 48 grid: 3 x 6 = 18 blocks, keep 7: rounds of 7, 7, 4
    wl = synth.WalkWorkload(batch=3, n=24 * 48, m=36, steps=6)
    _run(wl, 48, 7, steps=6)


def test_zero_change_step_takes_lowest_indices():
    wl = synth.LatentWorkload(batch=1, height=16, width=32, m=32, steps=3)
    _run(wl, 32, 3, steps=3, zero_step=True)


def test_full_size_latent_sampled():
    spec = synth.CONFIGS["latent_bs"]
    wl = synth.make("latent_bs", steps=4)
    _run(wl, spec["grid_w"], spec["keep_blocks"], steps=3, check=[0, wl.nb - 1])


def test_reset_state_restarts_the_round():
    wl = synth.LatentWorkload(batch=1, height=16, width=32, m=32, steps=4)
    _, a0 = wl.next()
    _, a1 = wl.next()
    with rc.Plan((1, wl.n, wl.m), "bf16", "bs", grid_w=32, keep_blocks=3) as plan:
        heads = []
        for _ in range(2):
            ahat = to_device(a0, "bf16").float()
            e = torch.zeros_like(ahat)
            packed = torch.empty(plan.packed_bytes, dtype=torch.uint8, device=DEV)
            plan.compress(to_device(a1, "bf16"), ahat, e, packed)
            torch.cuda.synchronize()
            heads.append(packed.cpu().numpy()[:16].view(np.uint32).copy())
            plan.reset_state()
        assert np.array_equal(heads[0], heads[1])


@pytest.mark.parametrize("chunk", [1, 2, 3])
def test_compress_send_and_decompress_many(chunk):
    wl = synth.LatentWorkload(batch=3, height=16, width=32, m=32, steps=2)
    _, a0 = wl.next()
    _, a1 = wl.next()
    kw = dict(grid_w=32, keep_blocks=3)
    with rc.Plan((3, wl.n, wl.m), "bf16", "bs", **kw) as p_ref, \
            rc.Plan((3, wl.n, wl.m), "bf16", "bs", **kw) as p_send:
        a = to_device(a1, "bf16")
        start = to_device(a0, "bf16").float()
        ah_r, e_r = start.clone(), torch.zeros_like(start)
        ah_s, e_s = start.clone(), torch.zeros_like(start)
        pk_r = torch.empty(p_ref.packed_bytes, dtype=torch.uint8, device=DEV)
        pk_s = torch.empty_like(pk_r)
        dst = torch.empty_like(pk_r)
        p_ref.compress(a, ah_r, e_r, pk_r)
        cs = torch.cuda.Stream()
        p_send.compress_send(a, ah_s, e_s, pk_s, dst, chunk, cs)
        cs.synchronize()
        torch.cuda.synchronize()
        for x, y in ((pk_s, pk_r), (dst, pk_r), (ah_s, ah_r), (e_s, e_r)):
            assert np.array_equal(bits(x.cpu().numpy()), bits(y.cpu().numpy()))
        states = [start.clone() + float(q) for q in range(3)]
        seq = [s.clone() for s in states]
        many = [s.clone() for s in states]
        for q in range(3):
            p_ref.decompress(pk_r, seq[q])
        p_ref.decompress_many([pk_r] * 3, many)
        torch.cuda.synchronize()
        for q in range(3):
            assert np.array_equal(bits(many[q].cpu().numpy()), bits(seq[q].cpu().numpy()))
