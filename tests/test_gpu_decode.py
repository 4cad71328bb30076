"""GPU parity of live-only output decoding (LM head on live positions, threshold commit)
through the C ABI, against the oracle on the same seeded inputs.

The GPU's logits are exact bf16 x bf16 products accumulated in fp32 on MFMA, the oracle's are
summed in double.  Every fp32 sum on the GPU is a chain of at most n = H / 32 + 5 roundings
(H / 32 sequential 32-wide k-steps, each adding a sum of 32 products), so each logit is within
    B_t = gamma_n * max_v sum_k |h_tk| |w_vk|,   gamma_n = n u / (1 - n u), u = 2^-24
of the exact value (the standard bound for recursive summation).  Decisions are compared
exactly wherever this bound makes them unique: a live row whose top-two logit gap is under
2 B_t, or whose confidence lies within tau (2 B_t + 1e-5) of tau (1e-5 covers expf and the
fp32 partial sums of the softmax denominator), is reported instead of compared, and so is the
commit outcome of its sequence.  Confidences of the other live rows agree within a relative
2 B_t + 1e-5.  Reported rows are logged and capped at 3 % of the live rows (at least one).
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
# the most live rows the streamed LM head takes; more go to the compute-bound tiles
STREAM_MAX_ROWS = 128
CONF_EPS = 1e-5
REPORT_CAP = 0.03


def logit_bound(h_bits, W_bits):
    """Per-row bound B_t on the error of any fp32-accumulated logit of row t."""
    hf = synth.bf16_bits_to_f32(h_bits).astype(np.float64)
    Wf = synth.bf16_bits_to_f32(W_bits).astype(np.float64)
    n = hf.shape[1] // 32 + 5
    gamma = n * U / (1.0 - n * U)
    return gamma * (np.abs(hf) @ np.abs(Wf).T).max(axis=1)


def report_cap(D):
    return max(1, int(REPORT_CAP * int((D == 0).sum())))


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


def compare(D, tokens, out, Dn, tok, conf, block, tau, B):
    """Compare one step; B is the per-row logit error bound.  Returns the number of reported
    (near-tie) rows, after logging it."""
    live = D == 0
    crel = 2.0 * B + CONF_EPS
    near = live & ((out["gap"] < 2.0 * B) | (np.abs(out["conf"] - tau) < tau * crel))
    ok = live & ~near
    assert (np.abs(conf[ok] - out["conf"][ok]) <= crel[ok] * out["conf"][ok]).all(), \
        "confidence outside the fp32 accumulation bound"
    assert (conf[~live] == 0).all()
    for b in range(D.shape[0] // block):
        sl = slice(b * block, (b + 1) * block)
        if near[sl].any():
            continue
        c = out["conf"][sl][live[sl]]
        if len(c) and not (c >= tau).any() and len(c) > 1:
            order = np.argsort(-c, kind="stable")
            if c[order[0]] - c[order[1]] <= c[order[0]] * crel[sl][live[sl]][order[:2]].sum():
                continue  # the fallback choice is a near tie
        assert np.array_equal(Dn[sl], out["D_next"][sl]), f"sequence {b}: commits differ"
        assert np.array_equal(tok[sl], out["token"][sl]), f"sequence {b}: tokens differ"
    n_near = int(near.sum())
    print(f"decode parity: {n_near} of {int(live.sum())} live rows reported as near ties "
          f"(max logit bound {B.max():.2e})", flush=True)
    return n_near


@pytest.mark.parametrize("shape", [(3, 24, 128, 512), (5, 13, 192, 384), (2, 64, 256, 1024)],
                         ids=["b3x24-h128-v512", "b5x13-h192-v384-ragged", "b2x64-h256-v1024"])
def test_small_decode_step(shape):
    batch, block, H, V = shape
    hs, Wb, D = synth.decode_inputs(40 + H, batch, block, H, V)
    dec = Decoder(batch, block, H, V)
    tokens = np.full(batch * block, -1, np.int32)
    Dn, tok, conf = dec(dev(hs[0]), dev(Wb), D, tokens)
    out = oracle.live_decode(hs[0], Wb, D, block, 0.95, token=tokens)
    reported = compare(D, tokens, out, Dn, tok, conf, block, 0.95, logit_bound(hs[0], Wb))
    assert reported <= report_cap(D)
    assert out["commits"] > 0 and (Dn >= D).all()


@pytest.mark.parametrize("shape", [(8, 32, 128, 384), (9, 32, 128, 384)],
                         ids=["b8x32-v384", "b9x32-v384"])
def test_lm_head_row_tiles_and_ragged_vocabulary(shape):
    """256 and 288 positions (about 190 and 215 live rows: one ragged 256-row tile of the
    compute-bound LM head) with a vocabulary that is not a multiple of 256."""
    batch, block, H, V = shape
    hs, Wb, D = synth.decode_inputs(70 + batch, batch, block, H, V)
    dec = Decoder(batch, block, H, V)
    tokens = np.full(batch * block, -1, np.int32)
    Dn, tok, conf = dec(dev(hs[0]), dev(Wb), D, tokens)
    out = oracle.live_decode(hs[0], Wb, D, block, 0.95, token=tokens)
    reported = compare(D, tokens, out, Dn, tok, conf, block, 0.95, logit_bound(hs[0], Wb))
    assert reported <= report_cap(D)


@pytest.mark.parametrize("batch", [4, 5], ids=["128-live-streamed", "160-live-compute-tiles"])
def test_lm_head_on_both_sides_of_the_stream_limit(batch):
    """Every position live: 128 live rows are the most the streamed LM head takes (one
    128-row pass over each vocabulary slab; at this vocabulary four-wave work items of 128
    tokens, one partial each); 160 go to the compute-bound tiles (one ragged 256-row tile;
    256-token partials)."""
    block, H, V = 32, 128, 384
    hs, Wb, _ = synth.decode_inputs(55 + batch, batch, block, H, V)
    D = np.zeros(batch * block, np.uint8)
    dec = Decoder(batch, block, H, V)
    tokens = np.full(batch * block, -1, np.int32)
    Dn, tok, conf = dec(dev(hs[0]), dev(Wb), D, tokens)
    out = oracle.live_decode(hs[0], Wb, D, block, 0.95, token=tokens)
    reported = compare(D, tokens, out, Dn, tok, conf, block, 0.95, logit_bound(hs[0], Wb))
    assert reported <= report_cap(D)


@pytest.mark.parametrize("V", [65536, 65536 + 128], ids=["v65536", "v65664-half-last-block"])
def test_lm_head_wide_vocabulary(V):
    """A vocabulary of at least 256 tokens per CU (65536 on 256 CUs) takes the eight-wave
    streamed LM head (256-token blocks; with 65664 tokens the last block is half, its upper
    four waves past the vocabulary); small hidden size keeps the oracle quick."""
    batch, block, H = 2, 32, 128
    hs, Wb, D = synth.decode_inputs(66, batch, block, H, V)
    dec = Decoder(batch, block, H, V)
    tokens = np.full(batch * block, -1, np.int32)
    Dn, tok, conf = dec(dev(hs[0]), dev(Wb), D, tokens)
    out = oracle.live_decode(hs[0], Wb, D, block, 0.95, token=tokens)
    reported = compare(D, tokens, out, Dn, tok, conf, block, 0.95, logit_bound(hs[0], Wb))
    assert reported <= report_cap(D)


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
    assert compare(D, tokens, out, Dn, tok, conf, block, 0.95, logit_bound(hs[0], Wb)) <= report_cap(D)
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
        assert compare(D, tokens, out, Dn, tok, conf, block, 0.95,
                       logit_bound(hs[s], Wb)) <= report_cap(D)
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
    assert compare(D, tokens, out, Dn, tok, conf, block, 0.95,
                   logit_bound(hs[0], Wb)) <= report_cap(D)


def test_decode_bench_shape_sampled_sequences():
    """The largest decoding shape the benchmark times: 128 sequences of 64 positions from the
    8192-position sweep workload's seed (about 6080 live), H 2048, V 131072 (a 512 MiB bf16 LM
    head).  The GPU decodes every position, in the same launch configuration as the benchmark
    (the compute-bound LM-head tiles, a fixed grid walking 24 row tiles x 512 token blocks);
    the oracle decodes the first, a middle and the last sequence whole.  That is exact for
    them: a sequence's commits depend only on its own positions' logits."""
    w = synth.workload(5)
    batch, block, H, V = w.batch, w.block, w.hidden, 131072
    hs, Wb, D = synth.decode_inputs(w.seed, batch, block, H, V)
    assert int((D == 0).sum()) > 2 * 1024  # several row tiles of 256 live rows
    dec = Decoder(batch, block, H, V)
    tokens = np.full(batch * block, -1, np.int32)
    Dn, tok, conf = dec(dev(hs[0]), dev(Wb), D, tokens)
    rows = np.concatenate([np.arange(b * block, (b + 1) * block)
                           for b in (0, batch // 2, batch - 1)])
    h_s, D_s, t_s = hs[0][rows], D[rows], tokens[rows]
    out = oracle.live_decode(h_s, Wb, D_s, block, 0.95, token=t_s)
    assert compare(D_s, t_s, out, Dn[rows], tok[rows], conf[rows], block, 0.95,
                   logit_bound(h_s, Wb)) <= report_cap(D_s)
    # every position: a decoded one stays decoded with its token untouched; a live one commits
    # exactly when it gets a token, which is a vocabulary id
    live = D == 0
    assert (Dn[~live] == 1).all() and (tok[~live] == -1).all()
    assert ((tok[live] >= 0) == (Dn[live] == 1)).all() and (tok < V).all()


@pytest.mark.parametrize("n_live", [300, 500], ids=["300-live", "500-live"])
def test_lm_head_compute_tiles_ragged_second_row_tile(n_live):
    """The compute-bound LM head with two 256-row tiles, the second one ragged (44 and 244
    rows): fewer than four row tiles, so its walk's row supertile is two tiles tall."""
    batch, block, H, V = 16, 32, 128, 1024
    hs, Wb, _ = synth.decode_inputs(300 + n_live, batch, block, H, V)
    rng = np.random.default_rng(n_live)
    D = np.ones(batch * block, np.uint8)
    D[rng.choice(batch * block, size=n_live, replace=False)] = 0
    dec = Decoder(batch, block, H, V)
    tokens = np.full(batch * block, -1, np.int32)
    Dn, tok, conf = dec(dev(hs[0]), dev(Wb), D, tokens)
    out = oracle.live_decode(hs[0], Wb, D, block, 0.95, token=tokens)
    assert compare(D, tokens, out, Dn, tok, conf, block, 0.95,
                   logit_bound(hs[0], Wb)) <= report_cap(D)


def test_lm_head_compute_tiles_wide_hidden():
    """The compute-bound LM head at H = 1024 (32 K chunks) with 640 live rows (three 256-row
    tiles, the last ragged) over a vocabulary of 9 x 128 tokens (the last 256-token block half
    past the vocabulary)."""
    batch, block, H, V = 20, 32, 1024, 1152
    hs, Wb, _ = synth.decode_inputs(123, batch, block, H, V)
    D = np.zeros(batch * block, np.uint8)
    dec = Decoder(batch, block, H, V)
    tokens = np.full(batch * block, -1, np.int32)
    Dn, tok, conf = dec(dev(hs[0]), dev(Wb), D, tokens)
    out = oracle.live_decode(hs[0], Wb, D, block, 0.95, token=tokens)
    assert compare(D, tokens, out, Dn, tok, conf, block, 0.95,
                   logit_bound(hs[0], Wb)) <= report_cap(D)


@pytest.mark.parametrize("batch,H,V", [(41, 64, 257 * 128), (41, 192, 257 * 128),
                                       (7, 64, 513 * 128)],
                         ids=["six-row-tiles-one-chunk", "six-row-tiles-three-chunks",
                              "one-row-tile-257-blocks"])
def test_lm_head_compute_tiles_walk_several_tiles_per_workgroup(batch, H, V):
    """Enough compute-bound tiles that workgroups of the fixed grid walk several: 1312 live
    rows (six 256-row tiles, the last with 32 rows: a full row supertile of four and one of
    two) over 257 x 128 tokens (129 token blocks, the last half past the vocabulary; the last
    token supertile one block wide), and 224 live rows (one row tile) over 513 x 128 tokens
    (257 blocks: one more tile than a 256-CU grid).  A workgroup's copy cursor then crosses
    tile boundaries and row-tile changes, with K in one chunk (the first chunk of a tile is
    also its last) and in three."""
    block = 32
    hs, Wb, _ = synth.decode_inputs(130 + H, batch, block, H, V)
    D = np.zeros(batch * block, np.uint8)
    dec = Decoder(batch, block, H, V)
    tokens = np.full(batch * block, -1, np.int32)
    Dn, tok, conf = dec(dev(hs[0]), dev(Wb), D, tokens)
    out = oracle.live_decode(hs[0], Wb, D, block, 0.95, token=tokens)
    assert compare(D, tokens, out, Dn, tok, conf, block, 0.95,
                   logit_bound(hs[0], Wb)) <= report_cap(D)


@pytest.mark.parametrize("batch", [4, 20], ids=["128-live-streamed", "640-live-compute-tiles"])
def test_lm_head_largest_hidden_size(batch):
    """H = 16384, the largest hidden size the decoding call accepts (256 K chunks; the widest
    byte offsets of both LM heads' copies), on the streamed head and on the compute-bound tiles,
    over a ragged vocabulary of 3 x 128 tokens.  The fp32 accumulation bound is widest here
    (B_t near 7e-3, far above its value at H = 1024), and so is the band of rows whose
    decision it leaves open (a top-two gap under 2 B_t, a confidence within tau (2 B_t + 1e-5)
    of tau): about 3 % of the rows of these inputs, judged on the oracle's values alone; up to
    5 % may be reported here."""
    block, H, V = 32, 16384, 384
    hs, Wb, _ = synth.decode_inputs(160 + batch, batch, block, H, V)
    D = np.zeros(batch * block, np.uint8)
    dec = Decoder(batch, block, H, V)
    tokens = np.full(batch * block, -1, np.int32)
    Dn, tok, conf = dec(dev(hs[0]), dev(Wb), D, tokens)
    out = oracle.live_decode(hs[0], Wb, D, block, 0.95, token=tokens)
    assert compare(D, tokens, out, Dn, tok, conf, block, 0.95,
                   logit_bound(hs[0], Wb)) <= max(report_cap(D), -(-5 * batch * block // 100))


# token ids holding one and the same vocabulary row, placed so that the GPU meets their equal
# logits at every level of its max / argmax reductions: in one lane (5, 6, 21; on the
# compute-bound tiles, whose waves hold 128 tokens, also 69), across the lanes of a row (9),
# across the waves of a workgroup (197; on the streamed head, whose waves hold 32 tokens, also
# 69), across token blocks in the row reduction (261) and in the half-width last block (V - 5)
TIE_IDS = (5, 6, 9, 21, 69, 197, 261)


@pytest.mark.parametrize("batch,live_all", [(4, False), (24, True)],
                         ids=["streamed", "compute-tiles"])
def test_lm_head_exact_ties_take_the_lowest_token(batch, live_all):
    """Rows leaning toward a vocabulary row that several token ids share exactly.  A tied top
    token caps a row's confidence at 1/8, so no such row reaches tau and each sequence commits
    its most confident live row (one of the leaning rows): the committed tokens show the
    argmax.  The compute-bound tiles sum every token's logit in the same order, so the shared
    rows give bit-identical logits and the lowest id must win through every level at which
    partial maxima merge (lane, row, wave, token block).  The streamed LM head starts each
    work item's walk over the hidden dimension at a different chunk, so equal rows in
    different items round differently: there the tie is a near tie (gap 0 < 2 B_t) and any of
    the shared ids is a correct top token."""
    block, H, V = 32, 128, 1152
    hs, Wb, D = synth.decode_inputs(91 + batch, batch, block, H, V, lean_fraction=0.0)
    ids = TIE_IDS + (V - 5,)
    Wb = Wb.copy()
    for t in ids[1:]:
        Wb[t] = Wb[ids[0]]
    if live_all:
        D = np.zeros(batch * block, np.uint8)
    rng = np.random.default_rng(92 + batch)
    wf = synth.bf16_bits_to_f32(Wb[ids[0]]).astype(np.float32)
    h = synth.bf16_bits_to_f32(hs[0]).astype(np.float32)
    lean = rng.random(h.shape[0]) < 0.6
    h[lean] = wf * np.float32(8.0 / (0.02 * 0.02 * H)) + 0.5 * h[lean]
    hb = synth.f32_to_bf16_bits(h)
    dec = Decoder(batch, block, H, V)
    tokens = np.full(batch * block, -1, np.int32)
    Dn, tok, conf = dec(dev(hb), dev(Wb), D, tokens)
    out = oracle.live_decode(hb, Wb, D, block, 0.95, token=tokens)
    live = D == 0
    assert (live.sum() <= STREAM_MAX_ROWS) != live_all   # the intended LM-head path
    assert np.array_equal(Dn, out["D_next"])          # one fallback commit per sequence
    hot = live & (out["D_next"] == 1) & np.isin(out["token"], ids)
    assert hot.sum() == batch, int(hot.sum())
    assert (out["token"][hot] == ids[0]).all()        # the oracle's own tie rule
    if live_all:
        assert (tok[hot] == ids[0]).all(), np.unique(tok[hot])
    else:
        assert np.isin(tok[hot], ids).all(), np.unique(tok[hot])
    B = logit_bound(hb, Wb)
    crel = 2.0 * B + CONF_EPS
    assert (np.abs(conf[hot] - out["conf"][hot]) <= crel[hot] * out["conf"][hot]).all()
    print(f"exact ties: {int(hot.sum())} committed rows, tokens {np.unique(tok[hot]).tolist()} "
          f"({int(live.sum())} live)", flush=True)
