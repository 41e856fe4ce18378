"""GPU parity at the Dory-2B geometry (hidden 2048, 16 q / 4 kv heads of 128,
ffn 5632, vocab 32000, 4/8/4 sub-layers, sliding window 1024, bf16 weights).

The oracle reads the same bf16 weight values (upcast exactly), so the bars
measure the kernels: cosine >= 0.999 for every residual state after every
sub-layer pass and max |dlogit| <= 5e-2.  Long contexts start from the same
synthetic cache rows loaded into both sides, so the oracle only computes the
tokens under test."""
import numpy as np
import pytest

from gpu_util import check_pair, run_pair, say
from looped_normalized_gpt_amd import synth
from oracle import oracle as O

pytestmark = pytest.mark.gpu

COS, DLOGIT = 0.999, 5e-2


@pytest.fixture(scope="module")
def model2b():
    import torch
    assert torch.cuda.is_available()
    cfg = synth.config("2b")
    say("generating Dory-2B weights")
    return cfg, synth.make_weights(cfg)


@pytest.fixture(scope="module")
def D():
    from looped_normalized_gpt_amd import dory
    return dory


def _rows(cfg, npos, n_slot, seed=4):
    n_ord = sum(1 for ch in cfg["pattern"] if ch != "-")
    k, v = synth.make_kv_rows(n_ord * n_slot * npos, cfg["nk"], cfg["hd"], cfg["hidden"], seed)
    shp = (n_ord, n_slot, npos, cfg["nk"], cfg["hd"])
    return k.reshape(shp), v.reshape(shp)


def test_2b_prompt_then_decode(model2b, D):
    cfg, w = model2b
    toks = synth.make_tokens(52, cfg["vocab"])
    say("2b last_loop prompt 48 + 4 decode")
    g = D.Dory(cfg, w, max_ctx=1024, max_chunk=512)
    o = O.Oracle(cfg, w, max_ctx=1024)
    calls = [toks[:48]] + [toks[i:i + 1] for i in range(48, 52)]
    check_pair(run_pair(g, o, calls, 4, "last_loop"), COS, DLOGIT, "2b prompt+decode")
    g.close()


def test_2b_decode_at_context_4096(model2b, D):
    """The benchmark's launch configuration: one-row calls (captured graph) at
    positions 4096.. with sliding windows full and the full layers reading 4097+
    keys."""
    cfg, w = model2b
    k, v = _rows(cfg, 4096, 1)
    say("2b kv_load 4096 + 3 decode")
    g = D.Dory(cfg, w, max_ctx=4096 + 512, max_chunk=512)
    o = O.Oracle(cfg, w, max_ctx=4096 + 512)
    g.kv_load(k, v, "last_loop", 1)
    o.kv_load(k, v, "last_loop", 1)
    toks = synth.make_tokens(3, cfg["vocab"], seq=5)
    calls = [toks[i:i + 1] for i in range(3)]
    check_pair(run_pair(g, o, calls, 4, "last_loop"), COS, DLOGIT, "2b ctx4096 decode")
    g.close()


def test_2b_decode_split_merge_paths(model2b, D):
    """One-row calls at context 4096 through both merges of the sliding
    layers' attention splits: inside the attention kernel (per kv head within
    one XCD; the default where the create-time XCD check passes) and the merge
    kernel.  Each matches the oracle; the two agree to fp32 rounding."""
    import torch
    cfg, w = model2b
    k, v = _rows(cfg, 4096, 1, seed=6)
    g = D.Dory(cfg, w, max_ctx=4096 + 512, max_chunk=512)
    o = O.Oracle(cfg, w, max_ctx=4096 + 512)
    g.kv_load(k, v, "last_loop", 1)
    o.kv_load(k, v, "last_loop", 1)
    assert g.xcd_merge(), "the create-time XCD check turned the in-kernel merge off on this device"
    toks = synth.make_tokens(3, cfg["vocab"], seq=9)
    calls = [toks[i:i + 1] for i in range(3)]
    fused = run_pair(g, o, calls, 4, "last_loop")
    check_pair(fused, COS, DLOGIT, "2b decode, in-kernel merge")
    # the same calls again from position 4096 with the merge kernel
    g.rollback(4096)
    assert not g.xcd_merge(False)
    sep = []
    for toks1 in calls:
        buf = torch.full((g.passes(4), 1, cfg["hidden"]), float("nan"), dtype=torch.float32, device=g.device)
        g.set_tap(buf)
        lg = g.forward(np.asarray(toks1, np.int32), 4, "last_loop", logits=True)
        torch.cuda.synchronize()
        sep.append((lg.cpu().numpy(), buf.cpu().numpy()))
    g.set_tap(None)
    for i, ((glg, _, gtap, otap), (slg, stap)) in enumerate(zip(fused, sep)):
        check_pair([(slg, fused[i][1], stap, otap)], COS, DLOGIT, f"2b decode call {i}, merge kernel")
        dt = float(np.abs(gtap - stap).max())
        dl = float(np.abs(glg - slg).max())
        say(f"call {i}: in-kernel vs merge kernel: max |dtap| {dt:.2e}, max |dlogit| {dl:.2e}")
        assert dt <= 1e-4 and dl <= 1e-3, f"call {i}: the two merges differ by {dt:.2e} (tap), {dl:.2e} (logits)"
    assert g.xcd_merge(True)
    g.close()


def test_2b_decode_grown_splits(model2b, D):
    """One-row calls whose full layers read 4501+ keys with max_ctx 4608: 64
    workgroups per kv head take 71-key splits (the grown split), so every
    workgroup's ninth load step holds keys."""
    cfg, w = model2b
    k, v = _rows(cfg, 4500, 1, seed=8)
    say("2b kv_load 4500 + 3 decode (grown splits)")
    g = D.Dory(cfg, w, max_ctx=4608, max_chunk=512)
    o = O.Oracle(cfg, w, max_ctx=4608)
    g.kv_load(k, v, "last_loop", 1)
    o.kv_load(k, v, "last_loop", 1)
    toks = synth.make_tokens(3, cfg["vocab"], seq=11)
    calls = [toks[i:i + 1] for i in range(3)]
    check_pair(run_pair(g, o, calls, 4, "last_loop"), COS, DLOGIT, "2b ctx4500 decode")
    g.close()


def test_2b_chunk_past_the_window(model2b, D):
    """A multi-row call whose rows cross the 1024-key sliding window, on a
    loaded context (the prefill path: tiled GEMMs, multi-row attention)."""
    cfg, w = model2b
    k, v = _rows(cfg, 1000, 1, seed=8)
    g = D.Dory(cfg, w, max_ctx=2048, max_chunk=512)
    o = O.Oracle(cfg, w, max_ctx=2048)
    g.kv_load(k, v, "last_loop", 1)
    o.kv_load(k, v, "last_loop", 1)
    toks = synth.make_tokens(40, cfg["vocab"], seq=6)
    say("2b chunk of 40 at 1000")
    check_pair(run_pair(g, o, [toks], 2, "last_loop"), COS, DLOGIT, "2b chunk past window")
    g.close()


def test_2b_per_loop_prompt(model2b, D):
    cfg, w = model2b
    toks = synth.make_tokens(33, cfg["vocab"], seq=7)
    say("2b per_loop loops 8: 32 + 1")
    g = D.Dory(cfg, w, max_ctx=1024, max_chunk=512)
    o = O.Oracle(cfg, w, max_ctx=1024)
    check_pair(run_pair(g, o, [toks[:32], toks[32:]], 8, "per_loop"), COS, DLOGIT, "2b per_loop")
    g.close()


def test_2b_q8_long_context_decode(model2b, D):
    """q8_2f cache, full_window 8192, context past the full ring's size: the
    loaded codes agree bit for bit, then decode steps agree within the bars."""
    cfg, w = model2b
    cfg = dict(cfg, full_window=8192)
    npos = 9000
    k, v = _rows(cfg, npos, 1, seed=10)
    say("2b q8 kv_load 9000 + 2 decode")
    g = D.Dory(cfg, w, max_ctx=npos + 512, max_chunk=512, kv_encoding="q8_2f")
    o = O.Oracle(cfg, w, max_ctx=npos + 512, kv_q8=True)
    g.kv_load(k, v, "last_loop", 1)
    o.kv_load(k, v, "last_loop", 1)
    for od in range(g.n_ord):
        for p in (npos - 1000, npos - 1):
            a, b = g.kv_read(od, 0, p), o.kv_read(od, 0, p)
            for x, y in zip(a, b):
                assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8)), (od, p)
        fg, kg, _ = g.kv_field(od)
        fo, ko, _ = o.kv_field(od)
        assert fg and fo and np.array_equal(kg.view(np.uint32), ko.view(np.uint32))
    toks = synth.make_tokens(2, cfg["vocab"], seq=11)
    check_pair(run_pair(g, o, [toks[:1], toks[1:]], 4, "last_loop"), COS, DLOGIT, "2b q8 decode")
    g.close()


def test_2b_long_chunk_on_loaded_context(model2b, D):
    """A 160-row call at position 3000: the MFMA chunk attention with several
    row blocks (the last one ragged) and several key splits per block."""
    cfg, w = model2b
    k, v = _rows(cfg, 3000, 1, seed=12)
    g = D.Dory(cfg, w, max_ctx=3200, max_chunk=512)
    o = O.Oracle(cfg, w, max_ctx=3200)
    g.kv_load(k, v, "last_loop", 1)
    o.kv_load(k, v, "last_loop", 1)
    toks = synth.make_tokens(161, cfg["vocab"], seq=13)
    say("2b chunk of 160 at 3000 + 1 decode")
    check_pair(run_pair(g, o, [toks[:160], toks[160:]], 2, "last_loop"), COS, DLOGIT, "2b long chunk")
    g.close()


def test_2b_q8_prompt_crosses_freeze_and_wrap(model2b, D):
    """q8_2f prompt in calls of 40, 30, 100, 30 rows: the field freezes inside
    the second call, the full ring (full_window 96 + 100 rows) wraps in the
    last, and every call's attention reads dequantised codes."""
    cfg, w = model2b
    cfg = dict(cfg, full_window=96)
    toks = synth.make_tokens(201, cfg["vocab"], seq=14)
    say("2b q8 prompt 40+30+100+30 + 1 decode")
    g = D.Dory(cfg, w, max_ctx=400, max_chunk=100, kv_encoding="q8_2f")
    o = O.Oracle(cfg, w, max_ctx=400, kv_q8=True)
    calls = [toks[:40], toks[40:70], toks[70:170], toks[170:200], toks[200:]]
    check_pair(run_pair(g, o, calls, 2, "last_loop"), COS, DLOGIT, "2b q8 prompt")
    g.close()


def test_2b_full_chunk_past_the_window(model2b, D):
    """The prefill benchmark's launch configuration: a 512-row call (the
    512-row GEMM kernels with split K, 16 row blocks of the MFMA chunk
    attention) on a loaded context of 700 rows, so the sliding layers' window
    cuts through the chunk; loops 1 keeps the oracle's share to seconds."""
    cfg, w = model2b
    k, v = _rows(cfg, 700, 1, seed=15)
    g = D.Dory(cfg, w, max_ctx=1300, max_chunk=512)
    o = O.Oracle(cfg, w, max_ctx=1300)
    g.kv_load(k, v, "last_loop", 1)
    o.kv_load(k, v, "last_loop", 1)
    toks = synth.make_tokens(513, cfg["vocab"], seq=16)
    say("2b chunk of 512 at 700 + 1 decode, loops 1")
    check_pair(run_pair(g, o, [toks[:512], toks[512:]], 1, "last_loop"), COS, DLOGIT, "2b full chunk")
    g.close()


def test_2b_chunks_at_the_projection_edges(model2b, D):
    """Calls of 16, 17, 64 and 65 rows: the few-row projection at one, two and
    four 16-row tiles (64 its largest), then the 128-row tiles with the SwiGLU
    epilogue from 65 rows on, each checked after every sub-layer pass."""
    cfg, w = model2b
    toks = synth.make_tokens(163, cfg["vocab"], seq=17)
    g = D.Dory(cfg, w, max_ctx=512, max_chunk=512)
    o = O.Oracle(cfg, w, max_ctx=512)
    calls = [toks[:16], toks[16:33], toks[33:97], toks[97:162], toks[162:]]
    say("2b chunks of 16, 17, 64, 65 + 1 decode")
    check_pair(run_pair(g, o, calls, 2, "last_loop"), COS, DLOGIT, "2b projection edges")
    g.close()


def test_2b_at_the_loop_maximum(model2b, D):
    """loops = 16, the most a call takes: a 24-row prompt, then one-row calls
    (the captured graph of 16 recurrent passes, replayed), every pass's
    residual checked."""
    cfg, w = model2b
    toks = synth.make_tokens(27, cfg["vocab"], seq=18)
    g = D.Dory(cfg, w, max_ctx=64, max_chunk=32)
    o = O.Oracle(cfg, w, max_ctx=64)
    calls = [toks[:24], toks[24:25], toks[25:26], toks[26:27]]
    say("2b at loops 16: prompt 24 + 3 decode")
    check_pair(run_pair(g, o, calls, 16, "last_loop"), COS, DLOGIT, "2b loops 16")
    g.close()


def test_2b_prefill_launch_configuration(model2b, D):
    """The prefill benchmark's exact launch configuration: a 512-row call under
    per_loop at loops 8 on a loaded context of 1100 rows per slot (past the
    1024-key sliding window, so the window cuts through the chunk), every one
    of its 72 sub-layer passes checked, then one decode row."""
    cfg, w = model2b
    k, v = _rows(cfg, 1100, 8, seed=19)
    g = D.Dory(cfg, w, max_ctx=1700, max_chunk=512)
    o = O.Oracle(cfg, w, max_ctx=1700)
    g.kv_load(k, v, "per_loop", 8)
    o.kv_load(k, v, "per_loop", 8)
    del k, v
    toks = synth.make_tokens(513, cfg["vocab"], seq=20)
    say("2b per_loop loops 8: a 512-row call at 1100 + 1 decode")
    check_pair(run_pair(g, o, [toks[:512], toks[512:]], 8, "per_loop"), COS, DLOGIT, "2b prefill configuration")
    g.close()

