"""Pins of the oracle's whole forward: invariants the pages state, the pages' own
forward tests, an independent fp64 brute force on tiny inputs, and the error
rules of a call (CPU only)."""
import numpy as np
import pytest

from conftest import golden
from looped_normalized_gpt_amd import synth
from oracle import oracle as O
from ref_numpy import RefModel


@pytest.fixture(scope="module")
def pages():
    cfg = synth.config("pages")
    return cfg, synth.make_weights(cfg)


@pytest.fixture(scope="module")
def tiny():
    cfg = synth.config("tiny")
    return cfg, synth.make_weights(cfg)


def _run(cfg, w, ids, chunk, loops, mode, **kw):
    o = O.Oracle(cfg, w, max_ctx=max(256, len(ids)), **kw)
    lg = None
    for s in range(0, len(ids), chunk):
        lg, _ = o.forward(ids[s:s + chunk], loops, mode)
    return lg, o


def test_pages_fixture_weights_follow_the_lcg():
    """First draws of the fixture's LCG, written out from its definition."""
    cfg = synth.config("pages")
    w = synth.make_weights(cfg)
    s, want = 1, []
    for _ in range(3):
        s = (s * 1664525 + 1013904223) % 2 ** 32
        want.append(((s >> 8) / 2 ** 24 - 0.5) * 0.7)
    # the first sub-layer is sliding attention: its q matrix takes the first draws
    assert np.allclose(w["layers"][0]["wq"].ravel()[:3], want, atol=1e-7)
    assert w["layers"][1]["sg"][0] == np.float32(1.5) and w["layers"][0]["sq"][0] == np.float32(4.0)


def test_chunk_invariance_per_loop_pages_case(pages):
    g = golden("pages_fixture.json")["chunk_invariance"]
    cfg, w = pages
    cfg = dict(cfg, window=g["window"])
    ids = np.array([i * 7 % 11 for i in range(23)])
    out = [_run(cfg, w, ids, c, g["loops"], g["kv"])[0] for c in g["chunks"]]
    for o in out[1:]:
        assert np.abs(o - out[0]).max() < g["abs_tol"]


def test_last_loop_rewrites_in_place_pages_case(pages):
    g = golden("pages_fixture.json")["last_loop_rows"]
    cfg, w = pages
    cfg = dict(cfg, window=g["window"])
    lg, o = _run(cfg, w, np.array(g["ids"]), 64, g["loops"], g["kv"])
    for ord_ in range(o.n_ord):
        assert o.slot_rows(ord_, 0) == g["rows_per_slot"]
        assert o.slot_rows(ord_, 1) == 0
    assert np.isfinite(lg).all()


def test_last_loop_equals_per_loop_at_one_loop(tiny):
    cfg, w = tiny
    ids = synth.make_tokens(100, cfg["vocab"])
    a = _run(cfg, w, ids, 32, 1, "last_loop")[0]
    b = _run(cfg, w, ids, 32, 1, "per_loop")[0]
    assert np.array_equal(a, b)


def test_last_loop_rows_are_the_last_loops_rows(pages):
    """A first call on a fresh sequence computes the same under both modes; the
    last_loop slot then holds exactly per_loop's last-loop slot."""
    cfg, w = pages
    ids = np.arange(12) % 11
    la, oa = _run(cfg, w, ids, 12, 3, "last_loop")
    lb, ob = _run(cfg, w, ids, 12, 3, "per_loop")
    assert np.array_equal(la, lb)
    n_in, n_rec = cfg["n_in"], cfg["n_rec"]
    ords = [li for li, ch in enumerate(cfg["pattern"]) if ch != "-"]
    for o, li in enumerate(ords):
        rec = n_in <= li < n_in + n_rec
        for p in range(12):
            ka = oa.kv_read(o, 0, p)
            kb = ob.kv_read(o, 2 if rec else 0, p)
            assert np.array_equal(ka[0], kb[0]) and np.array_equal(ka[1], kb[1])


def test_every_residual_state_is_on_the_sphere(tiny):
    cfg, w = tiny
    o = O.Oracle(cfg, w, max_ctx=256)
    ids = synth.make_tokens(40, cfg["vocab"])
    for chunk in (ids[:37], ids[37:38], ids[38:]):
        _, tap = o.forward(chunk, 3, "last_loop", tap=True)
        assert tap.shape[0] == cfg["n_in"] + 3 * cfg["n_rec"] + cfg["n_out"]
        assert np.abs(np.linalg.norm(tap.astype(np.float64), axis=-1) - 1).max() < 1e-5


def test_wide_window_equals_full_attention(pages):
    cfg, w = pages
    ids = np.array([i * 5 % 11 for i in range(30)])
    both = dict(cfg, theta_s=cfg["theta_f"])
    a = _run(dict(both, window=1000), w, ids, 7, 2, "per_loop")[0]
    b = _run(dict(both, pattern=cfg["pattern"].replace("S", "*")), w, ids, 7, 2, "per_loop")[0]
    assert np.array_equal(a, b)


def test_gqa_forward_equals_replicated_kv_weights(tiny):
    cfg, w = tiny
    rep = cfg["nh"] // cfg["nk"]
    hd = cfg["hd"]
    w2 = {k: v for k, v in w.items() if k != "layers"}
    w2["layers"] = []
    for L in w["layers"]:
        L2 = dict(L)
        if L["kind"] == "attn":
            for name in ("wk", "wv"):
                m = L[name].reshape(cfg["nk"], hd, -1)
                L2[name] = np.repeat(m, rep, axis=0).reshape(cfg["nh"] * hd, -1)
        w2["layers"].append(L2)
    ids = synth.make_tokens(70, cfg["vocab"])
    a = _run(cfg, w, ids, 70, 2, "last_loop")[0]
    b = _run(dict(cfg, nk=cfg["nh"]), w2, ids, 70, 2, "last_loop")[0]
    assert np.allclose(a, b, atol=1e-6)


@pytest.mark.parametrize("mode", ["per_loop", "last_loop"])
def test_matches_independent_fp64_brute_force(pages, mode):
    cfg, w = pages
    ids = np.array([i * 3 % 11 for i in range(26)] + [11, -1])   # two ids past the table
    o = O.Oracle(cfg, w, max_ctx=64)
    ref = RefModel(cfg, w)
    for s, e in ((0, 9), (9, 10), (10, 23), (23, 28)):
        lg, tap = o.forward(ids[s:e], 2, mode, tap=True)
        rl, rt = ref.forward(ids[s:e], 2, mode)
        assert np.allclose(tap, rt, atol=2e-5), (s, e)
        assert np.allclose(lg, rl, atol=1e-4), (s, e)


def test_matches_brute_force_at_the_tiny_geometry(tiny):
    cfg, w = tiny
    ids = synth.make_tokens(90, cfg["vocab"])
    o = O.Oracle(cfg, w, max_ctx=128)
    ref = RefModel(cfg, w)
    for s, e in ((0, 70), (70, 71), (71, 90)):       # crosses the 64-key window
        lg, tap = o.forward(ids[s:e], 2, "last_loop", tap=True)
        rl, rt = ref.forward(ids[s:e], 2, "last_loop")
        assert np.allclose(tap, rt, atol=2e-5)
        assert np.allclose(lg, rl, atol=2e-4)


def test_q8_field_freezes_at_the_65th_row(tiny):
    cfg, w = tiny
    o = O.Oracle(cfg, w, max_ctx=256, kv_q8=True)
    ids = synth.make_tokens(66, cfg["vocab"])
    o.forward(ids[:64], 1, "last_loop", logits=False)
    assert o.kv_field(0)[0] is False
    o.forward(ids[64:65], 1, "last_loop", logits=False)
    fr, kcol, vcol = o.kv_field(0)
    assert fr and (kcol > 0).all() and (vcol > 0).all()
    # a chunk crossing the boundary freezes inside the call
    o2 = O.Oracle(cfg, w, max_ctx=256, kv_q8=True)
    o2.forward(ids[:60], 1, "last_loop", logits=False)
    o2.forward(ids[60:66], 1, "last_loop", logits=False)
    fr2, kcol2, _ = o2.kv_field(0)
    assert fr2 and np.array_equal(kcol, kcol2)


def test_q8_forward_tracks_fp32_forward(tiny):
    cfg, w = tiny
    ids = synth.make_tokens(100, cfg["vocab"])
    a = _run(cfg, w, ids, 50, 2, "last_loop")[0]
    b = _run(cfg, w, ids, 50, 2, "last_loop", kv_q8=True)[0]
    cos = np.dot(a, b) / np.linalg.norm(a) / np.linalg.norm(b)
    assert cos > 0.99


def test_call_errors_change_nothing(tiny):
    cfg, w = tiny
    o = O.Oracle(cfg, w, max_ctx=64)
    ids = synth.make_tokens(8, cfg["vocab"])
    assert o.forward_rc(ids, 0, "per_loop") == -1
    assert o.forward_rc(ids, 17, "per_loop") == -1
    assert o.forward_rc(ids[:0], 2, "per_loop") == -1
    assert o.forward_rc(ids, 2, 7) == -1
    assert o.pos() == 0
    assert o.forward_rc(ids, 2, "per_loop") == 0
    assert o.forward_rc(ids, 3, "per_loop") == -2        # per_loop loop count fixed
    assert o.forward_rc(ids, 2, "last_loop") == -2       # mode fixed until reset
    assert o.forward_rc(np.zeros(57, np.int32), 2, "per_loop") == -3   # 8 + 57 > 64
    assert o.pos() == 8
    o.reset()
    assert o.pos() == 0 and o.forward_rc(ids, 5, "last_loop") == 0
    assert o.forward_rc(ids, 9, "last_loop") == 0       # last_loop: any loop count per call


def test_attention_output_is_renormed_before_o(pages):
    """With values ~1e-4 the gated output's norm falls far below sqrt(eps); the
    justnorm over Q before O (dory.rs `attn_layer`) is then visible in the
    result, and the brute force, which keeps it, still agrees."""
    cfg, w = pages
    w2 = {k: v for k, v in w.items() if k != "layers"}
    w2["layers"] = [dict(L, wv=L["wv"] * np.float32(1e-4)) if L["kind"] == "attn" else L
                    for L in w["layers"]]
    ids = np.array([i * 3 % 11 for i in range(12)])
    o = O.Oracle(cfg, w2, max_ctx=64)
    ref = RefModel(cfg, w2)
    lg, tap = o.forward(ids, 2, "per_loop", tap=True)
    rl, rt = ref.forward(ids, 2, "per_loop")
    assert np.allclose(tap, rt, atol=2e-5) and np.allclose(lg, rl, atol=1e-4)


def test_rollback_keeps_the_prefix_a_new_turn_extends_pages_case(pages):
    """dory.rs test `rollback_keeps_the_prefix_a_new_turn_extends`: 9 tokens in
    one call, back to position 5, the rest from there: the logits of one token
    per call over all 12."""
    g = golden("pages_fixture.json")["rollback"]
    cfg, w = pages
    cfg = dict(cfg, window=g["window"])
    ids = np.array([i * 3 % 11 for i in range(12)], np.int32)
    want = _run(cfg, w, ids, g["reference_chunk"], g["loops"], g["kv"])[0]
    o = O.Oracle(cfg, w, max_ctx=64)
    o.forward(ids[:g["first_call"]], g["loops"], g["kv"])
    o.rollback(g["rollback_to"])
    assert o.pos() == g["rollback_to"]
    got, _ = o.forward(ids[g["rollback_to"]:], g["loops"], g["kv"])
    assert np.abs(got - want).max() < g["abs_tol"]


def test_rollback_equals_a_run_that_never_went_there(tiny):
    """Back to position 80 after 100 rows (q8_2f, last_loop, past the freeze),
    then other tokens: bit for bit the run that took the same calls up to 80
    and the new tokens next (the field froze from the same 64 rows)."""
    cfg, w = tiny
    ids = synth.make_tokens(100, cfg["vocab"])
    new = synth.make_tokens(12, cfg["vocab"], seq=3)
    a = O.Oracle(cfg, w, max_ctx=256, kv_q8=True)
    for s, e in ((0, 40), (40, 80), (80, 100)):
        a.forward(ids[s:e], 2, "last_loop", logits=False)
    a.rollback(80)
    assert a.pos() == 80 and all(a.slot_rows(od, 0) == 80 for od in range(a.n_ord))
    ga, _ = a.forward(new, 2, "last_loop")
    b = O.Oracle(cfg, w, max_ctx=256, kv_q8=True)
    for s, e in ((0, 40), (40, 80)):
        b.forward(ids[s:e], 2, "last_loop", logits=False)
    gb, _ = b.forward(new, 2, "last_loop")
    assert np.array_equal(ga, gb)
    for od in range(a.n_ord):
        for p in (79, 85, 91):
            for x, y in zip(a.kv_read(od, 0, p), b.kv_read(od, 0, p)):
                assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8))


def test_rollback_below_the_freeze_keeps_the_field(tiny):
    """kv_cache.rs `truncate_last` drops rows only and `append` freezes only
    while the field is empty: back to position 30 after the freeze, the field
    stays as it was, and the rows appended again past position 64 do not
    freeze it a second time."""
    cfg, w = tiny
    ids = synth.make_tokens(100, cfg["vocab"])
    o = O.Oracle(cfg, w, max_ctx=256, kv_q8=True)
    o.forward(ids[:50], 1, "last_loop", logits=False)
    o.forward(ids[50:100], 1, "last_loop", logits=False)
    before = [o.kv_field(od) for od in range(o.n_ord)]
    assert all(f[0] for f in before)
    o.rollback(30)
    assert o.pos() == 30 and o.slot_rows(0, 0) == 30
    new = synth.make_tokens(70, cfg["vocab"], seq=4)
    o.forward(new[:40], 1, "last_loop", logits=False)
    o.forward(new[40:], 1, "last_loop", logits=False)
    for od in range(o.n_ord):
        fr, kcol, vcol = o.kv_field(od)
        assert fr
        assert np.array_equal(kcol.view(np.uint32), before[od][1].view(np.uint32))
        assert np.array_equal(vcol.view(np.uint32), before[od][2].view(np.uint32))


def test_rollback_bounds(tiny):
    cfg, w = tiny
    o = O.Oracle(cfg, w, max_ctx=64)
    ids = synth.make_tokens(8, cfg["vocab"])
    o.forward(ids, 2, "per_loop")
    o.rollback(20)               # past the position: nothing to forget
    assert o.pos() == 8 and o.slot_rows(1, 1) == 8   # the recurrent layer's second loop slot
    with pytest.raises(Exception):
        o.rollback(-1)
    o.rollback(3)
    assert o.pos() == 3 and o.slot_rows(0, 0) == 3 and o.slot_rows(1, 1) == 3
    assert o.forward_rc(ids, 3, "per_loop") == -2    # the per_loop loop count stays fixed


def test_want_all_rows_pages_case(pages):
    """dory.rs `Want::All`: the head over every row of the call.  Its last row is
    the `Want::Last` logits bit for bit, and under per_loop (chunk invariant, the
    pages' test) row r equals the last logits of a call that ends at row r."""
    cfg, w = pages
    cfg = dict(cfg, window=5)
    ids = np.array([i * 7 % 11 for i in range(23)], np.int32)
    o = O.Oracle(cfg, w, max_ctx=64)
    allv = o.forward_all(ids, 2, "per_loop")
    o2 = O.Oracle(cfg, w, max_ctx=64)
    last, _ = o2.forward(ids, 2, "per_loop")
    assert np.array_equal(allv[-1], last)
    for r in (0, 4, 11, 17):
        o3 = O.Oracle(cfg, w, max_ctx=64)
        lr, _ = o3.forward(ids[:r + 1], 2, "per_loop")
        assert np.abs(allv[r] - lr).max() < 2e-4, r


def test_prompt_loops_caps_logits_free_last_loop_calls(tiny):
    """dory.rs `chunk_loops`: with prompt_loops 1, a last_loop call that wants no
    logits runs one pass (its cache rows equal a loops-1 call's); a call that
    wants logits, and per_loop, run every pass."""
    cfg, w = tiny
    ids = synth.make_tokens(40, cfg["vocab"])
    a = O.Oracle(cfg, w, max_ctx=128)
    a.set_prompt_loops(1)
    a.forward(ids[:30], 4, "last_loop", logits=False)
    b = O.Oracle(cfg, w, max_ctx=128)
    b.forward(ids[:30], 1, "last_loop", logits=False)
    c = O.Oracle(cfg, w, max_ctx=128)
    c.forward(ids[:30], 4, "last_loop", logits=False)
    for od in range(a.n_ord):
        for p in (0, 17, 29):
            ra, rb, rc = a.kv_read(od, 0, p), b.kv_read(od, 0, p), c.kv_read(od, 0, p)
            assert all(np.array_equal(x, y) for x, y in zip(ra, rb))
    assert not all(np.array_equal(x, y) for x, y in zip(a.kv_read(1, 0, 29), c.kv_read(1, 0, 29)))
    la, _ = a.forward(ids[30:], 4, "last_loop")       # logits wanted: four passes
    lc, _ = c.forward(ids[30:], 4, "last_loop")
    lb, _ = b.forward(ids[30:], 4, "last_loop")
    assert np.array_equal(la, lb) and not np.array_equal(la, lc)
    with pytest.raises(Exception):
        a.set_prompt_loops(17)


# ---------------------------------------------------------------- the early exit (Gate::Conf)

def test_top_prob_pages_case():
    """dory.rs test `top_prob_of_a_sure_row`, and the softmax maximum in fp64
    where no term is dropped (every logit within 20 of the top)."""
    lg = np.full(100, -30.0, np.float32)
    lg[7] = 30.0
    assert O.top_prob(lg) > 0.999
    assert abs(O.top_prob(np.array([1.0, 1.0], np.float32)) - 0.5) < 1e-5
    x = np.random.default_rng(3).uniform(-5, 5, 1000).astype(np.float32)
    e = np.exp(x.astype(np.float64) - x.max())
    assert abs(O.top_prob(x) - 1.0 / e.sum()) < 1e-7


def _gate_run(cfg, w, ids, th, loops=2):
    o = O.Oracle(cfg, w, max_ctx=256)
    o.set_gate(th)
    o.forward(ids[:8], loops, "last_loop")            # a multi-row call: no gate
    out = [o.forward(ids[i:i + 1], loops, "last_loop")[0] for i in range(8, len(ids))]
    return o, out


def test_gate_that_never_exits_equals_two_loops(tiny):
    """Threshold above 1: every token takes the second pass, read out or not,
    and rewrites the first read-out's rows: bit for bit a forward of loops 2
    (logits and cache rows).  The probes follow `ExitRate`: the rate falls by a
    tenth per read-out, so tokens 1..10 read out, then every eighth."""
    cfg, w = tiny
    ids = synth.make_tokens(28, cfg["vocab"], seq=6)
    g, got = _gate_run(cfg, w, ids, 2.0, loops=7)
    r = O.Oracle(cfg, w, max_ctx=256)
    r.forward(ids[:8], 7, "last_loop")
    want = [r.forward(ids[i:i + 1], 2, "last_loop")[0] for i in range(8, 28)]
    for a, b in zip(got, want):
        assert np.array_equal(a, b)
    for od in range(g.n_ord):
        assert g.slot_rows(od, 0) == r.slot_rows(od, 0) == 28
        for p in (8, 19, 27):
            assert all(np.array_equal(x, y) for x, y in zip(g.kv_read(od, 0, p), r.kv_read(od, 0, p)))
    rate = np.float32(1.0)
    for _ in range(11):       # read-outs at tokens 1..10 and 16 of the 20
        rate = np.float32(rate + np.float32(0.1) * (np.float32(0.0) - rate))
    tokens, one, last, got_rate = g.gate_stats()
    assert (tokens, one) == (20, 0) and got_rate == rate and 0 < last < 1


def test_gate_that_always_exits_equals_one_loop(tiny):
    """Threshold 0: every token leaves after its read-out (the rate stays 1, so
    every token reads out): bit for bit a forward of loops 1."""
    cfg, w = tiny
    ids = synth.make_tokens(20, cfg["vocab"], seq=7)
    g, got = _gate_run(cfg, w, ids, 0.0, loops=5)
    r = O.Oracle(cfg, w, max_ctx=256)
    r.forward(ids[:8], 5, "last_loop")
    want = [r.forward(ids[i:i + 1], 1, "last_loop")[0] for i in range(8, 20)]
    for a, b in zip(got, want):
        assert np.array_equal(a, b)
    assert g.gate_stats()[:2] == (12, 12) and g.gate_stats()[3] == 1.0


def test_gate_rules(tiny):
    cfg, w = tiny
    ids = synth.make_tokens(10, cfg["vocab"], seq=8)
    o = O.Oracle(cfg, w, max_ctx=64)
    o.set_gate(0.5)
    assert o.forward_rc(ids[:1], 2, "per_loop") == -1    # the gate works on the last-loop cache
    with pytest.raises(Exception):
        o.forward(ids[:1], 2, "last_loop", tap=True)      # gated calls take no tap
    with pytest.raises(Exception):
        o.set_gate(-0.1)
    # multi-row calls are not gated
    a, _ = o.forward(ids[:6], 3, "last_loop")
    b, _ = O.Oracle(cfg, w, max_ctx=64).forward(ids[:6], 3, "last_loop")
    assert np.array_equal(a, b) and o.gate_stats()[0] == 0
