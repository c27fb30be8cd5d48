"""Batches past 2^31 elements: every kernel's offsets must be 64-bit.

One tensor's two steps come from the seeded flux generator; the batch repeats
them (640 copies of 1152 x 3072 = 2.26e9 elements, about 32 GB of state), so
every tensor must produce the same packed bytes and state. Sampled tensors
(first, middle, last) are checked against the oracle: bit for bit for the
quantisers, the sparsifier and block selection, by the low-rank tolerance
for low rank.
"""
import numpy as np
import pytest
import torch

from gpu_harness import DEV, bits, lib_view_f32, oracle, relF, say, synth, to_device
from activation_residual_compression_amd import librescomp as rc

pytestmark = pytest.mark.gpu

B, N_ROWS, N_COLS = 640, 1152, 3072


@pytest.fixture(scope="module")
def frames():
    free, _ = torch.cuda.mem_get_info()
    if free < 64 * 2 ** 30:
        pytest.skip("needs 64 GiB of free device memory")
    wl = synth.FluxWorkload(batch=1, n=N_ROWS, m=N_COLS, steps=2)
    _, a0 = wl.next()
    _, a1 = wl.next()
    return a0[0], a1[0]


@pytest.mark.parametrize("scheme,kw", [("q2", dict(group=128)), ("q1", dict(group=64)),
                                       ("nm", dict(nm_keep=2, nm_block=16)),
                                       ("lr", dict(rank=32, iters=2)),
                                       ("bs", dict(grid_w=144, keep_blocks=5))])
def test_batch_past_2_31_elements(frames, scheme, kw):
    assert B * N_ROWS * N_COLS > 2 ** 31
    a0, a1 = frames
    params = dict(kw)
    if scheme == "lr":
        q0 = synth.FluxWorkload(batch=1, n=N_ROWS, m=N_COLS, steps=1).q0(32)
        params["q0"] = np.repeat(q0, B, axis=0)
    say("[gpu] large %s: %d x %d x %d" % (scheme, B, N_ROWS, N_COLS))
    with rc.Plan((B, N_ROWS, N_COLS), "bf16", scheme, **params) as plan:
        a = to_device(a1, "bf16").unsqueeze(0).expand(B, N_ROWS, N_COLS).contiguous()
        ahat = to_device(a0, "bf16").float().unsqueeze(0).expand(B, N_ROWS, N_COLS).contiguous()
        recon = ahat.clone()
        e = torch.zeros_like(ahat)
        packed = torch.full((plan.packed_bytes,), 0xA5, dtype=torch.uint8, device=DEV)
        plan.compress(a, ahat, e, packed)
        plan.decompress(packed, recon)
        torch.cuda.synchronize()
        tb = plan.tensor_packed_bytes
        ref_pk = packed[:tb].cpu().numpy()
        ref_ah = ahat[0].cpu().numpy()
        ref_e = e[0].cpu().numpy()
        af, pf = lib_view_f32(a1, "bf16"), lib_view_f32(a0, "bf16")
        if scheme == "bs":  # 144-token grid rows: 8 x 18 blocks of 8 x 8 tokens per tensor
            o = oracle.bs_compress_tensor(af, pf, grid_w=144, keep=5,
                                          visited=np.zeros(N_ROWS // 64, bool), in_dtype="bf16")
        else:
            okw = {"group": kw["group"]} if "group" in kw else \
                ({"rank": 32, "iters": 2, "q0": q0[0]} if scheme == "lr" else {})
            o = oracle.compress_tensor(scheme, af, pf, **okw)
        if scheme == "lr":
            assert abs(relF(af, ref_ah) - relF(af, o["ahat"])) <= 1e-3
        else:
            assert np.array_equal(ref_pk, o["packed"])
            assert np.array_equal(bits(ref_ah), bits(o["ahat"]))
            assert np.array_equal(bits(ref_e), bits(o["e"]))
        for b in (1, B // 2, B - 1):
            assert np.array_equal(packed[b * tb:(b + 1) * tb].cpu().numpy(), ref_pk), b
            assert np.array_equal(bits(ahat[b].cpu().numpy()), bits(ref_ah)), b
            assert np.array_equal(bits(e[b].cpu().numpy()), bits(ref_e)), b
            assert np.array_equal(bits(recon[b].cpu().numpy()), bits(ref_ah)), b
        del a, ahat, recon, e, packed
    torch.cuda.empty_cache()
