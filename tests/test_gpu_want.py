"""GPU parity of the call variants dory.rs `Want::All` (the logits of every row
of a call) and `prompt_loops` (a last_loop call that wants no logits runs fewer
passes, `chunk_loops`): the HIP path against the oracle on the same calls."""
import numpy as np
import pytest

from gpu_util import say
from looped_normalized_gpt_amd import synth
from oracle import oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def D():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from looped_normalized_gpt_amd import dory
    return dory


def _all_pair(g, o, calls, loops, mode, tol, what):
    import torch
    worst = 0.0
    for toks in calls:
        lg = g.forward_all(toks, loops, mode)
        torch.cuda.synchronize()
        ol = o.forward_all(toks, loops, mode)
        gl = lg.cpu().numpy()
        assert gl.shape == ol.shape and np.isfinite(gl).all()
        d = float(np.abs(gl - ol).max())
        worst = max(worst, d)
        assert d <= tol, f"{what}: call of {len(toks)} rows, max |dlogit| {d:.3e} > {tol}"
    say(f"{what}: worst |dlogit| over every row {worst:.3e}")


def test_want_all_tiny(D):
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg)
    t = synth.make_tokens(120, cfg["vocab"], seq=41)
    say("want all tiny: 40, 1, 70 rows")
    for mode in ("last_loop", "per_loop"):
        g = D.Dory(cfg, w, max_ctx=256, max_chunk=128)
        o = O.Oracle(cfg, w, max_ctx=256)
        _all_pair(g, o, [t[:40], t[40:41], t[41:111]], 2, mode, 1e-3, f"tiny all {mode}")
        g.close()


def test_want_all_2b(D):
    """Dory-2B: a 100-row call (the head as the tiled MFMA GEMM) and a 48-row
    call (the skinny GEMM); bf16 operands as every projection of such a call."""
    cfg = synth.config("2b")
    say("generating Dory-2B weights")
    w = synth.make_weights(cfg)
    t = synth.make_tokens(148, cfg["vocab"], seq=42)
    g = D.Dory(cfg, w, max_ctx=1024, max_chunk=512)
    o = O.Oracle(cfg, w, max_ctx=1024)
    say("want all 2b: 100 + 48 rows, loops 2")
    _all_pair(g, o, [t[:100], t[100:148]], 2, "last_loop", 5e-2, "2b all")
    g.close()


def test_prompt_loops(D):
    """prompt_loops 1: logits-free last_loop calls (a chunk, then a batch)
    run one pass; calls that want logits run all of theirs."""
    import torch
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg)
    t = synth.make_tokens(80, cfg["vocab"], seq=43)
    g = D.Dory(cfg, w, max_ctx=256, max_chunk=64, max_seqs=2)
    o = O.Oracle(cfg, w, max_ctx=256, max_seqs=2)
    g.set_prompt_loops(1)
    o.set_prompt_loops(1)
    say("prompt_loops 1: 30 rows without logits, 1 with, batch without, batch with")
    for sq in (0, 1):
        assert g.forward(t[:30], 4, "last_loop", seq=sq, logits=False) is None
        o.forward(t[:30], 4, "last_loop", seq=sq, logits=False)
    worst = 0.0
    for step in range(3):
        toks = np.array([t[40 + step], t[50 + step]], np.int32)
        loops = np.array([4, 3], np.int32)
        g.forward_batch([0, 1], toks, loops, "last_loop", logits=False)
        for i in range(2):
            o.forward(toks[i:i + 1], int(loops[i]), "last_loop", seq=i, logits=False)
        lg = g.forward(t[60 + step:61 + step], 4, "last_loop", seq=step % 2)
        torch.cuda.synchronize()
        ol, _ = o.forward(t[60 + step:61 + step], 4, "last_loop", seq=step % 2)
        worst = max(worst, float(np.abs(lg.cpu().numpy() - ol).max()))
    assert worst <= 1e-3, worst
    # off again: the same logits-free call now runs all four passes, as the oracle's
    g.set_prompt_loops(0)
    o.set_prompt_loops(0)
    g.forward(t[70:75], 4, "last_loop", logits=False)
    o.forward(t[70:75], 4, "last_loop", logits=False)
    lg = g.forward(t[75:76], 4, "last_loop")
    torch.cuda.synchronize()
    ol, _ = o.forward(t[75:76], 4, "last_loop")
    assert float(np.abs(lg.cpu().numpy() - ol).max()) <= 1e-3
    with pytest.raises(Exception):
        g.set_prompt_loops(17)
    g.close()
