"""GPU parity of rollback (dory.rs `DoryState::rollback`, a chat turn that goes
back and rewrites the tail): the HIP path and the oracle take the same calls
and rollbacks, and must agree within the bars of any call.  q8_2f fields stay
frozen across a rollback below 64 rows (kv_cache.rs `truncate_last`), one-row
graphs replay at the earlier positions, and a rollback deeper than the windowed
rings keep changes nothing."""
import numpy as np
import pytest

from gpu_util import check_pair, run_pair, say
from looped_normalized_gpt_amd import synth
from oracle import oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def D():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from looped_normalized_gpt_amd import dory
    return dory


def _script(g, o, ops, loops, mode):
    """ops: token arrays (one call each) or ("rollback", n)."""
    res = []
    for op in ops:
        if isinstance(op, tuple):
            want = min(op[1], g.position())
            g.rollback(op[1])
            o.rollback(op[1])
            assert g.position() == o.pos() == want
        else:
            res += run_pair(g, o, [op], loops, mode)
    return res


def test_rollback_pages_case(D):
    """The pages' rollback test on their fixture: 9 tokens, back to 5, the rest."""
    cfg = dict(synth.config("pages"), window=50)
    w = synth.make_weights(cfg)
    ids = np.array([i * 3 % 11 for i in range(12)], np.int32)
    say("rollback pages 9, back to 5, 7")
    g = D.Dory(cfg, w, max_ctx=64, max_chunk=16)
    o = O.Oracle(cfg, w, max_ctx=64)
    res = _script(g, o, [ids[:9], ("rollback", 5), ids[5:]], 2, "per_loop")
    g.close()
    check_pair(res, 0.99999, 1e-4, "pages rollback")


def test_rollback_tiny_one_row_graphs_and_chunks(D):
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg)
    t = synth.make_tokens(200, cfg["vocab"], seq=21)
    say("rollback tiny: 100, 6 one-row, back to 97, 6 one-row, back to 40, 30")
    g = D.Dory(cfg, w, max_ctx=256, max_chunk=128)
    o = O.Oracle(cfg, w, max_ctx=256)
    ops = [t[:100]] + [t[i:i + 1] for i in range(100, 106)] + [("rollback", 97)] + \
          [t[i:i + 1] for i in range(150, 156)] + [("rollback", 40), t[160:190], ("rollback", 500)]
    res = _script(g, o, ops, 2, "last_loop")
    assert g.position() == o.pos() == 70
    g.close()
    check_pair(res, 0.99999, 1e-3, "tiny rollback")


Q8_LOGIT = 2e-2
KV128 = dict(synth.CONFIGS["tiny"], hidden=256, ffn=256, vocab=64, nh=16, nk=4, hd=128,
             pattern="S-*-S-", n_in=2, n_rec=2, n_out=2, window=64, weight_dtype="f32")


def test_rollback_q8_below_the_freeze_keeps_the_field(D):
    """Head dim 128 (the one-row decode kernel), q8_2f: the field freezes in the
    second call; after a rollback to position 20 the one-row graph replays at
    positions below 64 with the field on, a chunk crosses 64 again without a
    second freeze, and a batch takes the rolled-back sequence beside a fresh
    one.  Logit bar 2e-2: at this geometry the q8_2f codes of a few new key
    rows flip by one step between the GPU's and the oracle's fp32 keys, which
    leaves 4.6e-3 .. 9.1e-3 on every call with or without a rollback."""
    import torch
    cfg = KV128
    w = synth.make_weights(cfg)
    t = synth.make_tokens(200, cfg["vocab"], seq=22)
    g = D.Dory(cfg, w, max_ctx=256, max_chunk=64, max_seqs=2, kv_encoding="q8_2f")
    o = O.Oracle(cfg, w, max_ctx=256, max_seqs=2, kv_q8=True)
    say("rollback q8 hd128: 50 + 30, 5 one-row, back to 20, 5 one-row, 50")
    ops = [t[:50], t[50:80]] + [t[i:i + 1] for i in range(80, 85)]
    res = _script(g, o, ops, 2, "last_loop")
    before = [g.kv_field(od) for od in range(g.n_ord)]
    assert all(f[0] for f in before)
    ops = [("rollback", 20)] + [t[i:i + 1] for i in range(100, 105)]
    res += _script(g, o, ops, 2, "last_loop")
    # a batch: sequence 0 (rolled back below 64 rows, its fields frozen) beside
    # sequence 1 (10 rows, not frozen)
    g.forward(t[:10], 2, "last_loop", seq=1)
    o.forward(t[:10], 2, "last_loop", seq=1)
    for step in range(3):
        toks = np.array([t[170 + step], t[180 + step]], np.int32)
        loops = np.array([2, 3], np.int32)
        lg = g.forward_batch([0, 1], toks, loops, "last_loop")
        torch.cuda.synchronize()
        for i, sq in enumerate((0, 1)):
            ol, _ = o.forward(toks[i:i + 1], int(loops[i]), "last_loop", seq=sq)
            d = float(np.abs(lg[i].cpu().numpy() - ol).max())
            assert d <= Q8_LOGIT, (step, sq, d)
    # a chunk crossing position 64 again: no second freeze
    res += _script(g, o, [t[110:160]], 2, "last_loop")
    assert g.position() == o.pos() == 78
    for od in range(g.n_ord):
        fr, kcol, vcol = g.kv_field(od)
        assert fr and np.array_equal(kcol.view(np.uint32), before[od][1].view(np.uint32))
        assert np.array_equal(vcol.view(np.uint32), before[od][2].view(np.uint32))
    check_pair(res, 0.9999, Q8_LOGIT, "q8 rollback")
    g.close()


def test_rollback_errors_change_nothing(D):
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg)
    t = synth.make_tokens(300, cfg["vocab"], seq=23)
    g = D.Dory(cfg, w, max_ctx=512, max_chunk=16)
    for s in range(0, 300, 16):
        g.forward(t[s:s + 16], 1, "last_loop", logits=False)
    assert g.position() == 300
    # the sliding ring (window 64, 128 rows) keeps positions 172.. only
    with pytest.raises(Exception, match="deeper than the windowed rings keep"):
        g.rollback(100)
    with pytest.raises(Exception):
        g.rollback(-1)
    assert g.position() == 300
    g.rollback(236)          # the next row's window 173..235 is still held
    assert g.position() == 236
    g.close()


def test_rollback_2b_decode_at_context_2000(D):
    """Dory-2B, the decode launch configuration (one-row graphs) on a loaded
    context: 3 tokens, back by 2, 3 other tokens."""
    cfg = synth.config("2b")
    say("generating Dory-2B weights")
    w = synth.make_weights(cfg)
    n_ord = sum(1 for ch in cfg["pattern"] if ch != "-")
    k, v = synth.make_kv_rows(n_ord * 2000, cfg["nk"], cfg["hd"], cfg["hidden"], 31)
    k = k.reshape(n_ord, 1, 2000, cfg["nk"], cfg["hd"])
    v = v.reshape(n_ord, 1, 2000, cfg["nk"], cfg["hd"])
    g = D.Dory(cfg, w, max_ctx=2600, max_chunk=512)
    o = O.Oracle(cfg, w, max_ctx=2600)
    g.kv_load(k, v, "last_loop", 1)
    o.kv_load(k, v, "last_loop", 1)
    t = synth.make_tokens(6, cfg["vocab"], seq=24)
    say("2b rollback: ctx 2000, 3 decode, back to 2001, 3 decode")
    ops = [t[i:i + 1] for i in range(3)] + [("rollback", 2001)] + [t[i:i + 1] for i in range(3, 6)]
    res = _script(g, o, ops, 4, "last_loop")
    g.close()
    check_pair(res, 0.999, 5e-2, "2b rollback")
