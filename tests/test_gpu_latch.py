"""GPU: the latch of a failed call (kv_cache.rs `append`: a failed transition is
terminal until the sequence is cleared), on the real library.  Failures are
injected on the host by the library's test hook (dory_debug_fail_launch): the
n-th launch of a call is refused before it is launched, the launches before it
run normally, nothing faults on the device.  The failed call reports
DORY_EDEVICE and latches its sequences; every later call on them is
DORY_ESTATE until dory_kv_reset; other sequences go on and still match the
oracle; after the reset the sequence matches the oracle run from scratch."""
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


def _logits(g, toks, loops, seq):
    import torch
    lg = g.forward(toks, loops, "last_loop", seq=seq)
    torch.cuda.synchronize()
    return lg.cpu().numpy()


@pytest.mark.parametrize("kind", ["chunk", "graph_replay", "graph_capture", "batch"])
@pytest.mark.parametrize("at", [1, 3, 11])
def test_failed_call_latches_until_reset(D, kind, at):
    import torch
    if kind == "graph_replay" and at != 1:
        pytest.skip("a graph replay is one launch")
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg)
    toks = synth.make_tokens(80, cfg["vocab"])
    say(f"latch kind={kind} at={at}")
    g = D.Dory(cfg, w, max_ctx=256, max_chunk=32, max_seqs=2)
    o1 = O.Oracle(cfg, w, max_ctx=256)
    g.forward(toks[:20], 2, "last_loop", seq=0)
    g.forward(toks[:20], 2, "last_loop", seq=1)
    o1.forward(toks[:20], 2, "last_loop")
    g.forward(toks[20:21], 2, "last_loop", seq=0)      # captures the one-row graph of sequence 0
    torch.cuda.synchronize()
    p0, p1 = g.position(0), g.position(1)
    lg = torch.empty((2, cfg["vocab"]), dtype=torch.float32, device=g.device)
    g.fail_launch(at)
    if kind == "chunk":
        rc = g.forward_rc(toks[21:30], 2, "last_loop", seq=0, logits=lg[0])
    elif kind == "graph_replay":
        rc = g.forward_rc(toks[21:22], 2, "last_loop", seq=0, logits=lg[0])
    elif kind == "graph_capture":
        rc = g.forward_rc(toks[21:22], 5, "last_loop", seq=0, logits=lg[0])
    else:
        rc = g.batch_rc([0, 1], [5, 6], [2, 3], "last_loop", logits=lg)
    g.fail_launch(0)
    torch.cuda.synchronize()
    assert rc == D.EDEVICE, rc
    assert g.latched(0)
    assert g.latched(1) == (kind == "batch")
    assert (g.position(0), g.position(1)) == (p0, p1)
    assert g.forward_rc(toks[21:22], 2, "last_loop", seq=0) == D.ESTATE
    assert g.batch_rc([1, 0], [1, 2], [1, 1]) == D.ESTATE
    with pytest.raises(D.DoryError):
        g.rollback(5, seq=0)
    if kind != "batch":
        # the other sequence was not touched: it goes on, as the oracle does
        d = np.abs(_logits(g, toks[40:45], 2, 1) - o1.forward(toks[40:45], 2, "last_loop")[0]).max()
        say(f"  other sequence after the failure: |dlogit| {d:.2e}")
        assert d <= 1e-3
    g.reset(0)
    assert not g.latched(0)
    o0 = O.Oracle(cfg, w, max_ctx=256)
    d = np.abs(_logits(g, toks[50:70], 2, 0) - o0.forward(toks[50:70], 2, "last_loop")[0]).max()
    d2 = np.abs(_logits(g, toks[70:71], 2, 0) - o0.forward(toks[70:71], 2, "last_loop")[0]).max()
    say(f"  reset sequence from scratch: |dlogit| {d:.2e}, one-row replay {d2:.2e}")
    assert d <= 1e-3 and d2 <= 1e-3
    g.close()


def test_q8_failure_across_the_freeze_then_reset(D):
    """q8_2f: a call across the 64-row freeze fails after the freeze was
    enqueued; the sequence latches; after the reset its prompt re-runs, freezes
    its fields again and matches the oracle."""
    import torch
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg)
    toks = synth.make_tokens(90, cfg["vocab"])
    g = D.Dory(cfg, w, max_ctx=256, max_chunk=64, kv_encoding="q8_2f")
    g.forward(toks[:60], 2, "last_loop", logits=None)
    g.fail_launch(12)
    rc = g.forward_rc(toks[60:70], 2, "last_loop")
    g.fail_launch(0)
    torch.cuda.synchronize()
    assert rc == D.EDEVICE and g.latched(0)
    g.reset(0)
    o = O.Oracle(cfg, w, max_ctx=256, kv_q8=True)
    for a, b in ((0, 60), (60, 70), (70, 71)):
        lg = g.forward(toks[a:b], 2, "last_loop")
        torch.cuda.synchronize()
        ol, _ = o.forward(toks[a:b], 2, "last_loop")
        assert np.abs(lg.cpu().numpy() - ol).max() <= 5e-3
    # (the fields come from each side's own fp32 keys and values, which agree to
    # rounding: a code may flip by one step, so the fields agree closely, not
    # bit for bit; bit-exactness from identical rows is tested elsewhere)
    frozen, kc, vc = g.kv_field(0)
    ofrozen, okc, ovc = o.kv_field(0)
    assert frozen and ofrozen
    assert np.allclose(kc, okc, rtol=1e-3, atol=1e-6) and np.allclose(vc, ovc, rtol=1e-3, atol=1e-6)
    g.close()
