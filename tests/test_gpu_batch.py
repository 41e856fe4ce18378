"""GPU parity of batched decode (dory_forward_batch): several sequences, each at
its own position, one token each, with different loop counts per row; checked
row by row against the oracle running each sequence on its own."""
import numpy as np
import pytest

from gpu_util import say
from looped_normalized_gpt_amd import synth
from oracle import oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def D():
    import torch
    assert torch.cuda.is_available()
    from looped_normalized_gpt_amd import dory
    return dory


def _prime(g, o, cfg, lens, mode, loops_fixed=None):
    """Prompts of different lengths, one sequence each (chunks of <= 40 rows)."""
    for s, n in enumerate(lens):
        toks = synth.make_tokens(n, cfg["vocab"], seq=20 + s)
        lp = loops_fixed[s] if loops_fixed is not None else 2
        for a in range(0, n, 40):
            g.forward(toks[a:a + 40], lp, mode, seq=s, logits=None)
            o.forward(toks[a:a + 40], lp, mode, seq=s, logits=False)


def _steps(g, o, cfg, nseq, steps, mode, loop_rows, tol, seqs_of=None):
    import torch
    rng = np.random.default_rng(7)
    worst = 0.0
    for t in range(steps):
        seqs = list(range(nseq)) if seqs_of is None else seqs_of(t)
        toks = rng.integers(0, cfg["vocab"], len(seqs)).astype(np.int32)
        loops = loop_rows(t, seqs)
        lg = g.forward_batch(seqs, toks, loops, mode)
        torch.cuda.synchronize()
        lg = lg.cpu().numpy()
        for i, s in enumerate(seqs):
            ol, _ = o.forward(toks[i:i + 1], int(loops[i]), mode, seq=s)
            d = float(np.abs(lg[i] - ol).max())
            worst = max(worst, d)
            assert d <= tol, f"step {t} row {i} (seq {s}, loops {loops[i]}): |dlogit| {d:.3e}"
    return worst


@pytest.mark.parametrize("mode", ["last_loop", "per_loop"])
def test_tiny_batch_matches_oracle(D, mode):
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg)
    nseq = 6
    lens = [5, 70, 33, 1, 64, 100]            # crosses the 64-key window on some rows
    g = D.Dory(cfg, w, max_ctx=160, max_chunk=64, max_seqs=8)
    o = O.Oracle(cfg, w, max_ctx=160, max_seqs=8)
    if mode == "per_loop":
        fixed = [1, 3, 2, 5, 2, 4]
        _prime(g, o, cfg, lens, mode, fixed)
        loop_rows = lambda t, seqs: np.array([fixed[s] for s in seqs], np.int32)
    else:
        _prime(g, o, cfg, lens, mode)
        loop_rows = lambda t, seqs: np.random.default_rng(100 + t).integers(1, 17, len(seqs)).astype(np.int32)
    say(f"tiny batch {mode}")
    worst = _steps(g, o, cfg, nseq, 6, mode, loop_rows, 1e-3)
    # a subset of the sequences, in another order
    worst = max(worst, _steps(g, o, cfg, nseq, 3, mode, loop_rows, 1e-3, seqs_of=lambda t: [4, 0, 2]))
    for s, n in enumerate(lens):
        assert g.position(s) == o.pos(s)
    say(f"tiny batch {mode}: worst |dlogit| {worst:.3e}")
    g.close()


def test_tiny_q8_batch_crosses_the_freeze(D):
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg)
    lens = [62, 63, 64, 90]                    # rows at positions 62..64 freeze during the steps
    g = D.Dory(cfg, w, max_ctx=160, max_chunk=64, max_seqs=4, kv_encoding="q8_2f")
    o = O.Oracle(cfg, w, max_ctx=160, max_seqs=4, kv_q8=True)
    _prime(g, o, cfg, lens, "last_loop")
    loop_rows = lambda t, seqs: np.array([3, 1, 2, 4], np.int32)[: len(seqs)]
    say("tiny q8 batch")
    worst = _steps(g, o, cfg, 4, 4, "last_loop", loop_rows, 5e-3)
    for s in range(4):
        fg, kg, _ = g.kv_field(0, 0, seq=s)
        fo, ko, _ = o.kv_field(0, 0, seq=s)
        assert fg == fo
    say(f"tiny q8 batch: worst |dlogit| {worst:.3e}")
    g.close()


def test_2b_batch_matches_oracle(D):
    cfg = synth.config("2b")
    w = synth.make_weights(cfg)
    lens = [100, 1100, 300, 2000]
    g = D.Dory(cfg, w, max_ctx=2100, max_chunk=512, max_seqs=4)
    o = O.Oracle(cfg, w, max_ctx=2100, max_seqs=4)
    n_ord = g.n_ord
    for s, n in enumerate(lens):
        k, v = synth.make_kv_rows(n_ord * n, cfg["nk"], cfg["hd"], cfg["hidden"], seed=30 + s)
        shp = (n_ord, 1, n, cfg["nk"], cfg["hd"])
        g.kv_load(k.reshape(shp), v.reshape(shp), "last_loop", 1, seq=s)
        o.kv_load(k.reshape(shp), v.reshape(shp), "last_loop", 1, seq=s)
    say("2b batch of 4 at contexts 100..2000")
    worst = _steps(g, o, cfg, 4, 2, "last_loop", lambda t, seqs: np.array([4, 1, 7, 2], np.int32), 5e-2)
    say(f"2b batch: worst |dlogit| {worst:.3e}")
    g.close()


def test_2b_q8_batch_matches_oracle(D):
    """The q8_2f batch kernel at head dim 128: four sequences with their caches
    loaded through the append rules, one whose row at position 64 freezes the
    field during the first step, one frozen long before, two past the 1024-key
    sliding window; each row with its own loop count."""
    cfg = synth.config("2b")
    w = synth.make_weights(cfg)
    lens = [64, 200, 1100, 1500]
    g = D.Dory(cfg, w, max_ctx=1600, max_chunk=512, max_seqs=4, kv_encoding="q8_2f")
    o = O.Oracle(cfg, w, max_ctx=1600, max_seqs=4, kv_q8=True)
    n_ord = g.n_ord
    for s, n in enumerate(lens):
        k, v = synth.make_kv_rows(n_ord * n, cfg["nk"], cfg["hd"], cfg["hidden"], seed=60 + s)
        shp = (n_ord, 1, n, cfg["nk"], cfg["hd"])
        g.kv_load(k.reshape(shp), v.reshape(shp), "last_loop", 1, seq=s)
        o.kv_load(k.reshape(shp), v.reshape(shp), "last_loop", 1, seq=s)
    say("2b q8 batch of 4 at contexts 64..1500")
    worst = _steps(g, o, cfg, 4, 2, "last_loop", lambda t, seqs: np.array([3, 1, 5, 2], np.int32), 5e-2)
    for s in range(4):
        for od in range(n_ord):
            fg, kg, _ = g.kv_field(od, 0, seq=s)
            fo, ko, _ = o.kv_field(od, 0, seq=s)
            assert fg and fo and np.array_equal(kg.view(np.uint32), ko.view(np.uint32)), (s, od)
    say(f"2b q8 batch: worst |dlogit| {worst:.3e}")
    g.close()


def test_tiny_batch_ids_past_the_table(D):
    """A batch whose rows carry ids at and past the vocabulary and negative
    ones (read as unsigned): zero embedding rows, as in one-sequence calls."""
    import torch
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg)
    g = D.Dory(cfg, w, max_ctx=64, max_chunk=16, max_seqs=4)
    o = O.Oracle(cfg, w, max_ctx=64, max_seqs=4)
    _prime(g, o, cfg, [5, 9, 12, 3], "last_loop")
    toks = np.array([cfg["vocab"], cfg["vocab"] + 7, -1, 3], np.int32)
    loops = np.array([2, 1, 3, 2], np.int32)
    lg = g.forward_batch(np.arange(4, dtype=np.int32), toks, loops, "last_loop")
    torch.cuda.synchronize()
    lg = lg.cpu().numpy()
    for s in range(4):
        ol, _ = o.forward(toks[s:s + 1], int(loops[s]), "last_loop", seq=s)
        d = float(np.abs(lg[s] - ol).max())
        assert d <= 1e-3, f"row {s} (id {toks[s]}): |dlogit| {d:.3e}"
    g.close()


def test_batch_errors_change_nothing(D):
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg)
    g = D.Dory(cfg, w, max_ctx=64, max_chunk=16, max_seqs=4)
    import ctypes as C
    def rc(seqs, loops, mode="last_loop"):
        sq = np.asarray(seqs, np.int32); tk = np.zeros(len(seqs), np.int32); lp = np.asarray(loops, np.int32)
        return D.lib.dory_forward_batch(g.h, len(sq), sq.ctypes.data_as(C.c_void_p), tk.ctypes.data_as(C.c_void_p),
                                        lp.ctypes.data_as(C.c_void_p), D.MODES[mode], None, None)
    assert rc([], []) == D.EINVAL                   # no row
    assert rc([0, 0], [1, 1]) == D.EINVAL           # a sequence twice
    assert rc([0, 4], [1, 1]) == D.EINVAL           # out of range
    assert rc([0, 1], [1, 17]) == D.EINVAL          # loops
    assert rc([0, 1, 2, 3, 0], [1] * 5) == D.ERANGE  # more rows than sequences
    g.forward(np.zeros(3, np.int32), 2, "per_loop", seq=1)
    assert rc([0, 1], [2, 2], "last_loop") == D.ESTATE   # seq 1 is per_loop
    assert rc([0, 1], [2, 3], "per_loop") == D.ESTATE    # seq 1 fixed at 2 loops
    assert [g.position(s) for s in range(4)] == [0, 3, 0, 0]
    assert rc([0, 1], [5, 2], "per_loop") == D.OK
    import torch
    torch.cuda.synchronize()
    assert [g.position(s) for s in range(4)] == [1, 4, 0, 0]
    g.close()


def test_2b_batch_of_64_in_the_benchmark_shape(D):
    """The batched benchmark's launch configuration: 64 rows in one call (skinny
    GEMMs on four 16-row tiles with split K, the 16-step decode attention, the
    multi-row merge) with loop counts drawn from 1..16, rows at different
    contexts.  Every row is one sequence's next token; six sampled rows are
    checked against the oracle run on that sequence alone."""
    import torch
    cfg = synth.config("2b")
    w = synth.make_weights(cfg)
    nseq = 64
    rng = np.random.default_rng(21)
    lens = rng.integers(40, 1300, nseq)            # some past the 1024-key window
    g = D.Dory(cfg, w, max_ctx=1400, max_chunk=512, max_seqs=nseq)
    n_ord = g.n_ord
    rows = {}
    for s in range(nseq):
        k, v = synth.make_kv_rows(n_ord * int(lens[s]), cfg["nk"], cfg["hd"], cfg["hidden"], seed=200 + s)
        shp = (n_ord, 1, int(lens[s]), cfg["nk"], cfg["hd"])
        rows[s] = (k.reshape(shp), v.reshape(shp))
        g.kv_load(rows[s][0], rows[s][1], "last_loop", 1, seq=s)
    seqs = np.arange(nseq, dtype=np.int32)
    toks = rng.integers(0, cfg["vocab"], nseq).astype(np.int32)
    loops = synth.make_loops(nseq, seed=22)
    say(f"2b batch of 64, loops {loops.min()}..{loops.max()}")
    lg = g.forward_batch(seqs, toks, loops, "last_loop")
    torch.cuda.synchronize()
    lg = lg.cpu().numpy()
    assert np.isfinite(lg).all()
    sample = [int(np.argmax(loops)), int(np.argmin(loops)), int(np.argmax(lens)), 5, 33, 62]
    worst = 0.0
    for s in sample:
        o = O.Oracle(cfg, w, max_ctx=1400)
        o.kv_load(rows[s][0], rows[s][1], "last_loop", 1)
        ol, _ = o.forward(toks[s:s + 1], int(loops[s]), "last_loop")
        o.close()
        d = float(np.abs(lg[s] - ol).max())
        worst = max(worst, d)
        assert d <= 5e-2, f"row {s} (context {lens[s]}, loops {loops[s]}): |dlogit| {d:.3e}"
    for s in range(nseq):
        assert g.position(s) == lens[s] + 1
    say(f"2b batch of 64: worst |dlogit| over rows {sample}: {worst:.3e}")
    g.close()


def test_2b_batch_past_64_rows(D):
    """96 sequences in one call: the first passes run on more than 64 rows (the
    128-row tile GEMMs, gate|up with SwiGLU in its epilogue and the sums of
    squares per 64 indices), later passes on the prefix of rows still looping
    (the few-row GEMMs, q|k|v|g split over K).  Sampled rows against the oracle
    run on their sequences alone."""
    import torch
    cfg = synth.config("2b")
    w = synth.make_weights(cfg)
    nseq = 96
    rng = np.random.default_rng(23)
    lens = rng.integers(20, 600, nseq)
    g = D.Dory(cfg, w, max_ctx=640, max_chunk=512, max_seqs=nseq)
    n_ord = g.n_ord
    rows = {}
    for s in range(nseq):
        k, v = synth.make_kv_rows(n_ord * int(lens[s]), cfg["nk"], cfg["hd"], cfg["hidden"], seed=400 + s)
        shp = (n_ord, 1, int(lens[s]), cfg["nk"], cfg["hd"])
        rows[s] = (k.reshape(shp), v.reshape(shp))
        g.kv_load(rows[s][0], rows[s][1], "last_loop", 1, seq=s)
    seqs = np.arange(nseq, dtype=np.int32)
    toks = rng.integers(0, cfg["vocab"], nseq).astype(np.int32)
    loops = synth.make_loops(nseq, seed=24)
    say(f"2b batch of 96, loops {loops.min()}..{loops.max()}, rows looping at pass 2: {(loops >= 2).sum()}")
    lg = g.forward_batch(seqs, toks, loops, "last_loop")
    torch.cuda.synchronize()
    lg = lg.cpu().numpy()
    assert np.isfinite(lg).all()
    sample = sorted({int(np.argmax(loops)), int(np.argmin(loops)), int(np.argmax(lens)), 0, 47, 95})
    worst = 0.0
    for s in sample:
        o = O.Oracle(cfg, w, max_ctx=640)
        o.kv_load(rows[s][0], rows[s][1], "last_loop", 1)
        ol, _ = o.forward(toks[s:s + 1], int(loops[s]), "last_loop")
        o.close()
        d = float(np.abs(lg[s] - ol).max())
        worst = max(worst, d)
        assert d <= 5e-2, f"row {s} (context {lens[s]}, loops {loops[s]}): |dlogit| {d:.3e}"
    for s in range(nseq):
        assert g.position(s) == lens[s] + 1
    say(f"2b batch of 96: worst |dlogit| over rows {sample}: {worst:.3e}")
    g.close()
