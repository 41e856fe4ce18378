"""GPU: the q8_2f codes and scales the forward itself writes, bit for bit.

The decode kernels encode the new row inside the attention kernel, the chunk
path in k_q8_write after k_prep; each writes the row it encodes (the rotated,
unit-normed key and the value, in fp32) to the kv tap (dory_debug_kv_tap).
Those rows, encoded by the oracle's encoder (kv_cache.rs `quant_row`) with the
slot's field, must give exactly the codes and scales the cache holds
(dory_kv_read) after the call: for every attention sub-layer, every kv head and
every row of the call, its last pass's rows (under last_loop a recurrent
layer's rows are those of the last loop).  Rows below position 64 of a layer
that froze its field in this call with no later pass are the freeze's
re-encoding of their dequantised codes (kv_cache.rs `freeze_cols`).  Covered:
a prompt call below the freeze, a call that crosses it, one-row decode calls
(the captured graph, head dim 128: the fused encoder of the one-row kernel),
a batch step, at Dory-2B and at the tiny geometry (head dim 16: one partial
32-channel key group)."""
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


def _last_pass_of_each_ordinal(cfg, loops):
    """(ordinal -> index of its last attention pass in the call, recurrent?)."""
    last, k = {}, 0
    n_in, n_rec = cfg["n_in"], cfg["n_rec"]
    walk = list(range(n_in)) + [n_in + j for _ in range(loops) for j in range(n_rec)] + \
        list(range(n_in + n_rec, len(cfg["pattern"])))
    ords = {}
    for li, ch in enumerate(cfg["pattern"]):
        if ch != "-":
            ords[li] = len(ords)
    for li in walk:
        if li in ords:
            last[ords[li]] = (k, n_in <= li < n_in + n_rec)
            k += 1
    return last, k


def _deq(codes, scales, group):
    g = np.repeat(scales, group)[: codes.size]
    return (codes.astype(np.float32) * g).astype(np.float32)


def _expected(x, col, group, refreeze):
    if refreeze:   # encoded without the field, then re-encoded by the freeze
        c0, s0 = O.q8_encode(x, None, group)
        x = _deq(c0, s0, group)
    return O.q8_encode(x, col, group)


def _check_call(g, cfg, seqs, positions, loops, tap, froze_here):
    """Every cache row the call wrote against the oracle's encoding of its tap row."""
    nk, hd = cfg["nk"], cfg["hd"]
    KV = nk * hd
    last, _ = _last_pass_of_each_ordinal(cfg, loops)
    checked = 0
    for o, (k, rec) in last.items():
        for r, (seq, p) in enumerate(zip(seqs, positions)):
            frozen, kcol, vcol = g.kv_field(o, 0, seq)
            kc, vc, ks, vs = g.kv_read(o, 0, p, seq)
            refreeze = froze_here[r] and p < 64 and not (rec and loops > 1)
            for kh in range(nk):
                xk = tap[k, r, 0, kh * hd:(kh + 1) * hd]
                xv = tap[k, r, 1, kh * hd:(kh + 1) * hd]
                ck, sk = _expected(xk, kcol[kh] if frozen else None, 32, refreeze and frozen)
                cv, sv = _expected(xv, vcol[kh] if frozen else None, hd, refreeze and frozen)
                assert np.array_equal(kc[kh], ck), (o, r, p, kh, "K codes")
                assert np.array_equal(ks[kh].view(np.uint32), sk.view(np.uint32)), (o, r, p, kh, "K scales")
                assert np.array_equal(vc[kh], cv), (o, r, p, kh, "V codes")
                assert vs[kh].view(np.uint32) == sv.view(np.uint32)[0], (o, r, p, kh, "V scale")
                checked += 1
    return checked


def _tapped(g, cfg, n, loops):
    import torch
    buf = torch.full((g.attn_passes(loops), n, 2, cfg["nk"] * cfg["hd"]), float("nan"),
                     dtype=torch.float32, device=g.device)
    g.set_kv_tap(buf)
    return buf


@pytest.mark.parametrize("geo", ["2b", "tiny"])
def test_forward_q8_writes_bit_exact(D, geo):
    import torch
    cfg = synth.config(geo, kv_encoding="q8_2f", full_window=300)
    w = synth.make_weights(cfg)
    loops = 2
    toks = synth.make_tokens(100, cfg["vocab"], seq=21)
    g = D.Dory(cfg, w, max_ctx=512, max_chunk=128, max_seqs=2, kv_encoding="q8_2f")
    total = 0
    pos = 0
    for n in (40, 40, 1, 1, 1):          # below the freeze, across it, then one-row calls (graph after the freeze)
        buf = _tapped(g, cfg, n, loops)
        g.forward(toks[pos:pos + n], loops, "last_loop", seq=0)
        torch.cuda.synchronize()
        tap = buf.cpu().numpy()
        assert np.isfinite(tap).all()
        froze = [pos <= 64 < pos + n] * n   # the call appends position 64: its slots freeze
        total += _check_call(g, cfg, [0] * n, list(range(pos, pos + n)), loops, tap, froze)
        say(f"{geo}: call of {n} rows at {pos}: codes and scales bit-exact")
        pos += n
    # a batch step: sequence 1 just below the freeze (its row freezes it), sequence 0 past it
    g.set_kv_tap(None)
    g.forward(toks[:64], loops, "last_loop", seq=1, logits=False)
    buf = _tapped(g, cfg, 2, loops)
    g.forward_batch([0, 1], toks[90:92], [loops, loops], "last_loop")
    torch.cuda.synchronize()
    tap = buf.cpu().numpy()
    total += _check_call(g, cfg, [0, 1], [pos, 64], loops, tap, [False, True])
    g.set_kv_tap(None)
    say(f"{geo}: {total} (layer, row, kv head) cache records bit-exact")
    g.close()
