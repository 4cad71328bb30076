"""The workspace-free live decoding call (its scratch in the library's static device array)
against the workspace call, through the C ABI: two calls in a row, the second on a smaller
shape, each compared bit for bit (the same kernels run on the same inputs)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def dev(a):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run(B, d, h, W, D, static):
    M = D.shape[0]
    Dn = torch.full((M,), 7, dtype=torch.uint8, device="cuda")
    tok = torch.full((M,), -1, dtype=torch.int32, device="cuda")
    conf = torch.full((M,), -5.0, dtype=torch.float32, device="cuda")
    if static:
        B.epoch_live_decode_static(d, h, W, D, Dn, tok, conf)
    else:
        n = B.epoch_decode_workspace_bytes(d)
        ws = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")  # stale contents
        B.epoch_live_decode(d, h, W, D, Dn, tok, conf, ws, n)
    torch.cuda.synchronize()
    return Dn.cpu().numpy(), tok.cpu().numpy(), conf.cpu().numpy()


def test_static_scratch_decode_matches_workspace_decode():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_sparse_amd import binding as B
    B.load()
    # first call: 768 positions, all live (the compute-bound LM head, 256-token partials);
    # second call: 96 positions with a quarter decoded (the streamed LM head, 128-token partials)
    shapes = [(24, 32, 256, 4096, True), (3, 32, 192, 2048, False)]
    for batch, block, H, V, all_live in shapes:
        hs, Wb, D = synth.decode_inputs(900 + batch, batch, block, H, V)
        if all_live:
            D[:] = 0
        d = B.make_decode_desc(batch, block, H, V)
        assert B.epoch_decode_workspace_bytes(d) <= B.EPOCH_DECODE_STATIC_SCRATCH_BYTES
        print(f"static decode vs workspace decode: batch {batch} block {block} H {H} V {V} "
              f"live {int((D == 0).sum())}", flush=True)
        h, W, Dd = dev(hs[0]), dev(Wb), dev(D)
        ref = run(B, d, h, W, Dd, static=False)
        got = run(B, d, h, W, Dd, static=True)
        for name, a, b in zip(("decoded_next", "tokens", "conf"), ref, got):
            assert np.array_equal(a, b), f"{name} differs from the workspace call"
        assert (ref[0] >= D).all() and ref[0].sum() > D.sum()   # the step committed something
