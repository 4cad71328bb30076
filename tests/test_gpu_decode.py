"""GPU parity of live-only output decoding (LM head on live positions, threshold commit)
through the C ABI, against the oracle on the same seeded inputs.

The GPU logits are bf16 products accumulated in fp32 on MFMA, the oracle's in double, so
decisions taken on them are compared exactly except where the pages' own near-tie rule
applies: a live row whose top-two logit gap is under 1e-2, or whose confidence lies within
1e-3 of tau, is reported (counted) instead of compared, and so is the commit outcome of its
sequence.  Confidences are compared within rtol 2e-3 on every other live row.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

GAP, NEAR_TAU, CONF_RTOL = 1e-2, 1e-3, 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_sparse_amd import binding
    binding.load()  # fails loudly when the library is missing


def dev(a):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class Decoder:
    def __init__(self, batch, block, hidden, vocab, tau=0.95):
        from block_diffusion_sparse_amd import binding as B
        self.B = B
        self.d = B.make_decode_desc(batch, block, hidden, vocab, tau)
        self.n = B.epoch_decode_workspace_bytes(self.d)
        self.ws = torch.empty(self.n, dtype=torch.uint8, device="cuda")
        self.block, self.tau = block, tau

    def __call__(self, h, W, D, tokens):
        M = D.shape[0]
        Dn = torch.empty(M, dtype=torch.uint8, device="cuda")
        tok = dev(tokens.copy())
        conf = torch.empty(M, dtype=torch.float32, device="cuda")
        self.B.epoch_live_decode(self.d, h, W, dev(D), Dn, tok, conf, self.ws, self.n)
        torch.cuda.synchronize()
        return Dn.cpu().numpy(), tok.cpu().numpy(), conf.cpu().numpy()


def compare(D, tokens, out, Dn, tok, conf, block, tau):
    """Compare one step; returns the number of reported (near-tie) rows."""
    live = D == 0
    near = live & ((out["gap"] < GAP) | (np.abs(out["conf"] - tau) < NEAR_TAU))
    ok = live & ~near
    np.testing.assert_allclose(conf[ok], out["conf"][ok], rtol=CONF_RTOL)
    assert (conf[~live] == 0).all()
    for b in range(D.shape[0] // block):
        sl = slice(b * block, (b + 1) * block)
        if near[sl].any():
            continue
        c = out["conf"][sl][live[sl]]
        if len(c) and not (c >= tau).any() and len(c) > 1:
            top2 = np.sort(c)[-2:]
            if top2[1] - top2[0] < NEAR_TAU * top2[1]:
                continue  # the fallback choice is a near tie
        assert np.array_equal(Dn[sl], out["D_next"][sl]), f"sequence {b}: commits differ"
        assert np.array_equal(tok[sl], out["token"][sl]), f"sequence {b}: tokens differ"
    return int(near.sum())


@pytest.mark.parametrize("shape", [(3, 24, 128, 512), (5, 13, 192, 384), (2, 64, 256, 1024)],
                         ids=["b3x24-h128-v512", "b5x13-h192-v384-ragged", "b2x64-h256-v1024"])
def test_small_decode_step(shape):
    batch, block, H, V = shape
    hs, Wb, D = synth.decode_inputs(40 + H, batch, block, H, V)
    dec = Decoder(batch, block, H, V)
    tokens = np.full(batch * block, -1, np.int32)
    Dn, tok, conf = dec(dev(hs[0]), dev(Wb), D, tokens)
    out = oracle.live_decode(hs[0], Wb, D, block, 0.95, token=tokens)
    reported = compare(D, tokens, out, Dn, tok, conf, block, 0.95)
    assert reported <= int((D == 0).sum()) // 4     # most live rows are compared exactly
    assert out["commits"] > 0 and (Dn >= D).all()


@pytest.mark.parametrize("shape", [(8, 32, 128, 384), (9, 32, 128, 384)],
                         ids=["b8x32-two-row-tiles-v384", "b9x32-three-row-tiles-v384"])
def test_lm_head_row_tiles_and_ragged_vocabulary(shape):
    """256 and 288 positions (two and three 128-row LM-head tiles, the last one ragged) with a
    vocabulary that is not a multiple of 256."""
    batch, block, H, V = shape
    hs, Wb, D = synth.decode_inputs(70 + batch, batch, block, H, V)
    dec = Decoder(batch, block, H, V)
    tokens = np.full(batch * block, -1, np.int32)
    Dn, tok, conf = dec(dev(hs[0]), dev(Wb), D, tokens)
    out = oracle.live_decode(hs[0], Wb, D, block, 0.95, token=tokens)
    reported = compare(D, tokens, out, Dn, tok, conf, block, 0.95)
    assert reported <= int((D == 0).sum()) // 4


@pytest.mark.parametrize("batch", [16, 20], ids=["512-live-streamed", "640-live-compute-tiles"])
def test_lm_head_on_both_sides_of_the_stream_limit(batch):
    """Every position live: 512 live rows are the most the streamed LM head takes (four
    128-row passes over each vocabulary slab), 640 go to the compute-bound tiles; both write
    the same 32-token partials."""
    block, H, V = 32, 128, 384
    hs, Wb, _ = synth.decode_inputs(55 + batch, batch, block, H, V)
    D = np.zeros(batch * block, np.uint8)
    dec = Decoder(batch, block, H, V)
    tokens = np.full(batch * block, -1, np.int32)
    Dn, tok, conf = dec(dev(hs[0]), dev(Wb), D, tokens)
    out = oracle.live_decode(hs[0], Wb, D, block, 0.95, token=tokens)
    reported = compare(D, tokens, out, Dn, tok, conf, block, 0.95)
    assert reported <= batch * block // 4


def test_lm_head_wide_vocabulary():
    """A vocabulary of at least 256 tokens per CU (65536 on 256 CUs) takes the eight-wave
    streamed LM head (256-token blocks); small hidden size keeps the oracle quick."""
    batch, block, H, V = 2, 32, 128, 65536
    hs, Wb, D = synth.decode_inputs(66, batch, block, H, V)
    dec = Decoder(batch, block, H, V)
    tokens = np.full(batch * block, -1, np.int32)
    Dn, tok, conf = dec(dev(hs[0]), dev(Wb), D, tokens)
    out = oracle.live_decode(hs[0], Wb, D, block, 0.95, token=tokens)
    reported = compare(D, tokens, out, Dn, tok, conf, block, 0.95)
    assert reported <= int((D == 0).sum()) // 4


def test_all_decoded_and_all_live():
    batch, block, H, V = 2, 32, 128, 256
    hs, Wb, _ = synth.decode_inputs(77, batch, block, H, V)
    dec = Decoder(batch, block, H, V)
    tokens = np.full(batch * block, 5, np.int32)
    D = np.ones(batch * block, np.uint8)
    Dn, tok, conf = dec(dev(hs[0]), dev(Wb), D, tokens)
    assert Dn.all() and (tok == 5).all() and (conf == 0).all()     # nothing left to decode
    D = np.zeros(batch * block, np.uint8)
    Dn, tok, conf = dec(dev(hs[0]), dev(Wb), D, tokens)
    out = oracle.live_decode(hs[0], Wb, D, block, 0.95, token=tokens)
    compare(D, tokens, out, Dn, tok, conf, block, 0.95)
    for b in range(batch):                                          # progress in every sequence
        assert Dn[b * block:(b + 1) * block].sum() >= 1


def test_block_decodes_to_completion():
    """Refinement steps until every position is decoded: D_{i+1} from the previous step's
    GPU mask, each step compared with the oracle on the same mask and hidden state."""
    batch, block, H, V, steps = 4, 32, 128, 512, 40
    hs, Wb, D = synth.decode_inputs(91, batch, block, H, V, steps=steps)
    D[:] = 0
    dec = Decoder(batch, block, H, V)
    Wd = dev(Wb)
    tokens = np.full(batch * block, -1, np.int32)
    for s in range(steps):
        Dn, tok, conf = dec(dev(hs[s]), Wd, D, tokens)
        out = oracle.live_decode(hs[s], Wb, D, block, 0.95, token=tokens)
        compare(D, tokens, out, Dn, tok, conf, block, 0.95)
        assert (Dn >= D).all() and Dn.sum() > D.sum()
        D, tokens = Dn, tok
        if D.all():
            break
    assert D.all() and s + 1 <= block and (tokens >= 0).all()


def test_decode_full_vocab_shape():
    """H = 2048, V = 32768 (a 64 MB bf16 LM head), two sequences of 32 positions."""
    batch, block, H, V = 2, 32, 2048, 32768
    hs, Wb, D = synth.decode_inputs(6, batch, block, H, V)
    dec = Decoder(batch, block, H, V)
    tokens = np.full(batch * block, -1, np.int32)
    Dn, tok, conf = dec(dev(hs[0]), dev(Wb), D, tokens)
    out = oracle.live_decode(hs[0], Wb, D, block, 0.95, token=tokens)
    assert compare(D, tokens, out, Dn, tok, conf, block, 0.95) <= int((D == 0).sum()) // 4
