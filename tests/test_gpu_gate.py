"""GPU parity of the confidence-gated early exit (dory.rs `Gate::Conf`,
`ExitRate`, `top_prob`): one-row calls with the gate on, against the oracle on
the same calls.  Decisions must agree token by token (the thresholds keep a
margin from every top probability the oracle sees), and so must the logits,
the counters and the exit rate."""
import numpy as np
import pytest

from gpu_util import say
from looped_normalized_gpt_amd import synth
from oracle import oracle as O

pytestmark = pytest.mark.gpu

KV128 = dict(synth.CONFIGS["tiny"], hidden=256, ffn=256, vocab=64, nh=16, nk=4, hd=128,
             pattern="S-*-S-", n_in=2, n_rec=2, n_out=2, window=64, weight_dtype="f32")


@pytest.fixture(scope="module")
def D():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from looped_normalized_gpt_amd import dory
    return dory


def _oracle_tops(cfg, w, t, th, n0, ntok):
    """The oracle's run under threshold th: per token (exited, top or None)."""
    o = O.Oracle(cfg, w, max_ctx=256)
    o.set_gate(th)
    o.forward(t[:n0], 3, "last_loop")
    out, prev = [], o.gate_stats()
    for i in range(n0, n0 + ntok):
        o.forward(t[i:i + 1], 3, "last_loop")
        st = o.gate_stats()
        out.append((st[1] > prev[1], st[2] if st[2] != prev[2] else None))
        prev = st
    return out


def _run_pair(D, cfg, w, t, th, n0, ntok, tol, what):
    import torch
    g = D.Dory(cfg, w, max_ctx=256, max_chunk=64)
    o = O.Oracle(cfg, w, max_ctx=256)
    g.set_gate(th)
    o.set_gate(th)
    lg = g.forward(t[:n0], 3, "last_loop")              # a multi-row call: no gate
    ol, _ = o.forward(t[:n0], 3, "last_loop")
    torch.cuda.synchronize()
    worst = float(np.abs(lg.cpu().numpy() - ol).max())
    exits = []
    for i in range(n0, n0 + ntok):
        lg = g.forward(t[i:i + 1], 3, "last_loop")
        torch.cuda.synchronize()
        ol, _ = o.forward(t[i:i + 1], 3, "last_loop")
        worst = max(worst, float(np.abs(lg.cpu().numpy() - ol).max()))
        gs, os_ = g.gate_stats(), o.gate_stats()
        assert gs[0] == os_[0] and gs[1] == os_[1], (what, i, gs, os_)   # the same decisions
        assert gs[3] == os_[3], (what, i, gs, os_)                       # the same exit rate (f32 steps)
        if os_[2] >= 0:  # d(top_prob)/top_prob = d(top logit) - sum_i p_i d(logit_i): within 2 tol
            assert abs(gs[2] - os_[2]) <= 2 * tol * os_[2], (what, i, gs, os_)
        exits.append(gs[1])
    g.close()
    assert worst <= tol, f"{what}: max |dlogit| {worst:.3e}"
    say(f"{what}: {ntok} gated tokens, {exits[-1]} left after one pass, worst |dlogit| {worst:.3e}")
    return exits[-1]


@pytest.mark.parametrize("geom", ["tiny", "kv128"])
def test_gate_never_and_always(D, geom):
    cfg = synth.config("tiny") if geom == "tiny" else KV128
    w = synth.make_weights(cfg)
    t = synth.make_tokens(60, cfg["vocab"], seq=51)
    # head dim 128: the 10-row first call's attention runs on bf16 MFMA operands
    # (the chunk attention at that head dim), which the later tokens' keys carry
    tol = 1e-3 if geom == "tiny" else 5e-3
    assert _run_pair(D, cfg, w, t, 2.0, 10, 20, tol, f"{geom} gate never") == 0
    assert _run_pair(D, cfg, w, t, 0.0, 10, 14, tol, f"{geom} gate always") == 14


def test_gate_mixed_threshold(D):
    """A threshold between the read-outs' top probabilities (the pages'
    fixture): some tokens leave after one pass, the others take two."""
    cfg = dict(synth.config("pages"), window=50)
    w = synth.make_weights(cfg)
    t = np.array([i * 5 % 11 for i in range(60)], np.int32)
    base = sorted(x for _, x in _oracle_tops(cfg, w, t, 2.0, 6, 40) if x is not None)
    best, margin = None, 0.0
    for th in ((a + b) / 2 for a, b in zip(base, base[1:])):   # between two of its top probabilities
        r = _oracle_tops(cfg, w, t, float(th), 6, 40)
        m = min(abs(x - th) / th for _, x in r if x is not None)
        if 0 < sum(e for e, _ in r) < 40 and m > margin:
            best, margin = float(th), m
    assert best is not None and margin > 0.02, margin
    say(f"pages gate: threshold {best:.4f}, margin {margin:.3f}")
    one = _run_pair(D, cfg, w, t, best, 6, 40, 1e-4, "pages gate mixed")
    assert 0 < one < 40


def test_gate_rules(D):
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg)
    t = synth.make_tokens(10, cfg["vocab"], seq=52)
    g = D.Dory(cfg, w, max_ctx=64, max_chunk=16, max_seqs=2)
    g.set_gate(0.5)
    with pytest.raises(Exception, match="last_loop"):
        g.forward(t[:1], 2, "per_loop")
    import torch
    g.set_tap(torch.zeros(64 * 16, device="cuda"))
    with pytest.raises(Exception, match="tap"):
        g.forward(t[:1], 2, "last_loop")
    g.set_tap(None)
    g.forward(t[:1], 2, "last_loop", seq=1)
    with pytest.raises(Exception, match="one-row"):
        g.forward_batch([0, 1], t[1:3], [2, 2], "last_loop")
    with pytest.raises(Exception):
        g.set_gate(-1.0)
    assert g.gate_stats(1)[0] == 1 and g.position(0) == 0
    g.close()


def test_gate_2b_decode_at_context_2000(D):
    """Dory-2B on a loaded context: gated tokens that never exit (read-outs,
    then two passes), and the ones the exit rate sends straight to two passes
    (the captured two-pass graph)."""
    cfg = synth.config("2b")
    say("generating Dory-2B weights")
    w = synth.make_weights(cfg)
    n_ord = sum(1 for ch in cfg["pattern"] if ch != "-")
    k, v = synth.make_kv_rows(n_ord * 2000, cfg["nk"], cfg["hd"], cfg["hidden"], 53)
    k = k.reshape(n_ord, 1, 2000, cfg["nk"], cfg["hd"])
    v = v.reshape(n_ord, 1, 2000, cfg["nk"], cfg["hd"])
    g = D.Dory(cfg, w, max_ctx=2100, max_chunk=512)
    o = O.Oracle(cfg, w, max_ctx=2100)
    g.kv_load(k, v, "last_loop", 1)
    o.kv_load(k, v, "last_loop", 1)
    # threshold 2: tokens 1..10 read out (each lowers the exit rate by a
    # tenth, below 0.35 after ten), tokens 11..14 go straight to two passes
    g.set_gate(2.0)
    o.set_gate(2.0)
    import torch
    t = synth.make_tokens(14, cfg["vocab"], seq=54)
    worst = 0.0
    say("2b gate: 14 tokens at context 2000 (10 read-outs, 4 straight to two passes)")
    for i in range(14):
        lg = g.forward(t[i:i + 1], 4, "last_loop")
        torch.cuda.synchronize()
        ol, _ = o.forward(t[i:i + 1], 4, "last_loop")
        worst = max(worst, float(np.abs(lg.cpu().numpy() - ol).max()))
        assert g.gate_stats()[:2] == o.gate_stats()[:2] and g.gate_stats()[3] == o.gate_stats()[3]
    g.close()
    assert worst <= 5e-2, worst
    say(f"2b gate: worst |dlogit| {worst:.3e}")


def test_gate_q8_across_the_freeze(D):
    """q8_2f cache at head dim 128: gated tokens at positions 58..71, so the
    read-out phase of the token at position 64 freezes the fields and its
    second pass rewrites the rows against them; threshold 2 (no exits)."""
    import torch
    cfg = KV128
    w = synth.make_weights(cfg)
    t = synth.make_tokens(80, cfg["vocab"], seq=55)
    g = D.Dory(cfg, w, max_ctx=256, max_chunk=64, kv_encoding="q8_2f")
    o = O.Oracle(cfg, w, max_ctx=256, kv_q8=True)
    g.forward(t[:58], 3, "last_loop", logits=False)
    o.forward(t[:58], 3, "last_loop", logits=False)
    g.set_gate(2.0)
    o.set_gate(2.0)
    worst = 0.0
    for i in range(58, 72):
        lg = g.forward(t[i:i + 1], 3, "last_loop")
        torch.cuda.synchronize()
        ol, _ = o.forward(t[i:i + 1], 3, "last_loop")
        worst = max(worst, float(np.abs(lg.cpu().numpy() - ol).max()))
        assert g.gate_stats()[:2] == o.gate_stats()[:2]
    for od in range(g.n_ord):
        assert g.kv_field(od)[0] and o.kv_field(od)[0]
    g.close()
    # bf16 chunk attention on the 58-row first call, and q8 codes of a few new
    # rows a step apart between the two sides' fp32 keys
    assert worst <= 2e-2, worst
    say(f"gate q8 across the freeze: worst |dlogit| {worst:.3e}")
