"""GPU: dory_forward_chunk_noalloc (the entry point for callers that cannot
allocate) against dory_forward_chunk, through the C ABI.  Two sequences of one
handle get the same tokens: one through the ordinary entry point, one through
the no-allocation variant (its scratch a carve-out of the library's static
device array).  The logits agree within the oracle bars (the same kernels on
the same inputs), call after call: the first call of 8 rows, the second
smaller (3 rows), then one-row calls, then a longer run; and the device's free
memory does not move across the no-allocation calls."""
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


CASES = [("tiny", "last_loop", None, 1e-3), ("tiny", "per_loop", None, 1e-3), ("tiny", "last_loop", "q8_2f", 5e-3),
         ("2b", "last_loop", None, 5e-2), ("2b", "per_loop", None, 5e-2)]


@pytest.mark.parametrize("geo,mode,kv,tol", CASES)
def test_noalloc_matches_the_ordinary_entry_point(D, geo, mode, kv, tol):
    import torch
    cfg = synth.config(geo)
    w = synth.make_weights(cfg)
    loops = 3
    toks = synth.make_tokens(64, cfg["vocab"], seq=5)
    say(f"noalloc {geo} {mode} kv={kv}")
    g = D.Dory(cfg, w, max_ctx=512, max_chunk=64, max_seqs=2, kv_encoding=kv)
    o = O.Oracle(cfg, w, max_ctx=512, kv_q8=kv == "q8_2f")
    if mode == "per_loop":
        # per_loop slots of later loops come with the first ordinary call
        g.forward(toks[:1], loops, mode, seq=1, logits=False)
        g.reset(1)
    a = torch.empty(cfg["vocab"], dtype=torch.float32, device=g.device)
    b = torch.empty_like(a)
    calls = [(0, 8), (8, 11), (11, 12), (12, 13), (13, 20), (20, 21)]
    worst_pair, worst_ora = 0.0, 0.0
    moved = []
    for lo, hi in calls:
        g.forward(toks[lo:hi], loops, mode, seq=0, logits=a)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        g.forward_noalloc(toks[lo:hi], loops, mode, seq=1, logits=b)
        torch.cuda.synchronize()
        moved.append(torch.cuda.mem_get_info()[0] - free0)
        ga, gb = a.cpu().numpy(), b.cpu().numpy()
        ol, _ = o.forward(toks[lo:hi], loops, mode)
        d_pair = float(np.abs(ga - gb).max())
        d_ora = float(np.abs(gb - ol).max())
        worst_pair, worst_ora = max(worst_pair, d_pair), max(worst_ora, d_ora)
        assert d_pair <= tol, f"rows {lo}..{hi}: noalloc vs ordinary |dlogit| {d_pair:.3e}"
        assert d_ora <= tol, f"rows {lo}..{hi}: noalloc vs oracle |dlogit| {d_ora:.3e}"
        assert g.position(1) == hi
    say(f"  worst |dlogit|: noalloc vs ordinary {worst_pair:.2e}, vs oracle {worst_ora:.2e}; "
        f"free device memory moved by {moved} bytes across the no-allocation calls")
    assert all(m == 0 for m in moved), moved
    g.close()


def test_noalloc_rejects_what_it_cannot_take(D):
    import torch
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg)
    g = D.Dory(cfg, w, max_ctx=128, max_chunk=64)
    t = synth.make_tokens(9, cfg["vocab"])
    with pytest.raises(D.DoryError) as e:
        g.forward_noalloc(t, 2, "last_loop")
    assert e.value.rc == D.ERANGE
    with pytest.raises(D.DoryError) as e:
        g.forward_noalloc(t[:2], 4, "per_loop")       # per_loop slots not created yet
    assert e.value.rc == D.ESTATE
    assert g.position() == 0
    g.set_gate(0.7)
    with pytest.raises(D.DoryError) as e:
        g.forward_noalloc(t[:1], 2, "last_loop")
    assert e.value.rc == D.EINVAL
    g.close()
    torch.cuda.synchronize()
