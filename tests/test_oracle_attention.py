"""Pins of the oracle's attention: textbook attention (torch SDPA), GQA as
replication, the window as a mask, degenerate cases, and the q8_2f grid test of
the KV cache page (CPU only)."""
import numpy as np
import pytest
import torch

from conftest import golden
from looped_normalized_gpt_amd import synth
from oracle import oracle as O

RNG = np.random.default_rng(5)


def _sdpa(q, k, v, p, first):
    """torch scaled_dot_product_attention, fp64, one query row per head, with an
    explicit boolean mask over keys 0..p."""
    nh, hd = q.shape
    Q = torch.tensor(q, dtype=torch.float64).reshape(nh, 1, hd)
    K = torch.tensor(k[: p + 1], dtype=torch.float64).permute(1, 0, 2).contiguous()
    V = torch.tensor(v[: p + 1], dtype=torch.float64).permute(1, 0, 2).contiguous()
    mask = torch.zeros(nh, 1, p + 1, dtype=torch.bool)
    mask[:, :, first:] = True
    y = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=1 / np.sqrt(hd))
    return y.reshape(nh, hd).numpy()


@pytest.mark.parametrize("hd,n,first", [(8, 1, 0), (16, 40, 0), (16, 40, 33), (128, 300, 100)])
def test_mha_equals_textbook_attention(hd, n, first):
    nh = 4
    q = RNG.standard_normal((nh, hd)).astype(np.float32) * 3
    k = RNG.standard_normal((n, nh, hd)).astype(np.float32)
    v = RNG.standard_normal((n, nh, hd)).astype(np.float32)
    y = O.attend(q, k, v, n - 1, first)
    assert np.allclose(y, _sdpa(q, k, v, n - 1, first), atol=1e-6)


def test_gqa_equals_replicated_kv_heads_bit_exact():
    nh, nk, hd, n = 16, 4, 32, 50
    q = RNG.standard_normal((nh, hd)).astype(np.float32)
    k = RNG.standard_normal((n, nk, hd)).astype(np.float32)
    v = RNG.standard_normal((n, nk, hd)).astype(np.float32)
    y = O.attend(q, k, v, n - 1, 10)
    yr = O.attend(q, np.repeat(k, nh // nk, axis=1), np.repeat(v, nh // nk, axis=1), n - 1, 10)
    assert np.array_equal(y, yr)
    # and head h reads kv head h // 4: swapping kv heads 0 and 1 swaps q-head groups 0..3 and 4..7
    y2 = O.attend(q[[4, 5, 6, 7, 0, 1, 2, 3] + list(range(8, 16))], k[:, [1, 0, 2, 3]], v[:, [1, 0, 2, 3]], n - 1, 10)
    assert np.array_equal(y2[:4], y[4:8]) and np.array_equal(y2[4:8], y[:4])


def test_window_equals_masked_full_row_pages_case():
    g = golden("windowed_attend.json")
    rows, hd, hpk = g["rows"], g["hd"], g["heads_per_kv"]
    r, i = np.arange(rows)[:, None], np.arange(hd)[None, :]
    k = (((r * 13 + i * 5) % 29) / 29 - 0.5).astype(np.float32).reshape(rows, 1, hd)
    v = (((r * 7 + i * 3) % 31) / 31 - 0.5).astype(np.float32).reshape(rows, 1, hd)
    q = ((np.arange(hpk * hd) * 19 % 23) / 23 - 0.5).astype(np.float32).reshape(hpk, hd)
    assert 1 / np.sqrt(hd) == g["score_scale"]
    for w in g["windows"]:
        first = max(rows - w, 0)
        y, pr = O.attend(q, k, v, rows - 1, first, probs=True)
        # masked full row, in fp64: scores -inf before `first`
        s = np.einsum("hd,nd->hn", q.astype(np.float64), k[:, 0].astype(np.float64)) * g["score_scale"]
        s[:, :first] = -np.inf
        a = np.exp(s - s.max(1, keepdims=True))
        a /= a.sum(1, keepdims=True)
        assert np.allclose(y, a @ v[:, 0].astype(np.float64), atol=1e-6), w
        assert np.allclose(pr, a[:, first:], atol=1e-7)
        assert np.allclose(pr.sum(1), 1.0, atol=1e-6)


def test_degenerate_windows():
    nh, nk, hd, n = 4, 2, 16, 9
    q = RNG.standard_normal((nh, hd)).astype(np.float32)
    k = RNG.standard_normal((n, nk, hd)).astype(np.float32)
    v = RNG.standard_normal((n, nk, hd)).astype(np.float32)
    # one visible key (window 1): y is that key's value, whatever q is
    y = O.attend(q, k, v, n - 1, n - 1)
    assert np.allclose(y, np.repeat(v[n - 1], nh // nk, axis=0), atol=1e-7)
    # a single stored row at position 0
    y0 = O.attend(q, k[:1], v[:1], 0, 0)
    assert np.allclose(y0, np.repeat(v[0], nh // nk, axis=0), atol=1e-7)
    # equal keys give the plain mean of the values
    kk = np.repeat(k[:1], n, axis=0)
    assert np.allclose(O.attend(q, kk, v, n - 1, 0), np.repeat(v.mean(0), nh // nk, axis=0), atol=1e-6)


def _dummy_model(nh, nk, hd, kv_q8, max_ctx=128):
    cfg = dict(synth.CONFIGS["tiny"], hidden=8, ffn=8, vocab=4, nh=nh, nk=nk, hd=hd,
               pattern="*", n_in=1, n_rec=0, n_out=0, window=8)
    return O.Oracle(cfg, synth.make_weights(cfg), max_ctx=max_ctx, kv_q8=kv_q8)


def test_q8_attend_matches_f32_within_grid_pages_case():
    """The q8 cache reads like the fp32 one within the int8 grid (100 positions,
    crossing the freeze), from the KV cache page's own test."""
    g = golden("q8_grid.json")
    heads, hd, P = g["heads"], g["hd"], g["positions"]

    def row(p, salt):
        i = np.arange(heads * hd)
        x = ((i * 31 + p * 17 + salt * 7 + 3) % 97) / 97.0 - 0.5
        return np.where(i % 2 == 0, x * 4.0, x * 0.25).astype(np.float32).reshape(heads, hd)

    K = np.stack([row(p, 1) for p in range(P)])[None, None]
    V = np.stack([row(p, 2) for p in range(P)])[None, None]
    f, q8 = _dummy_model(heads, heads, hd, False), _dummy_model(heads, heads, hd, True)
    f.kv_load(K, V)
    q8.kv_load(K, V)
    q = ((np.arange(hd) * 13 + 5) % 89 / 89.0 - 0.5).astype(np.float32)
    qh = np.stack([q] * heads)
    kf = np.stack([f.kv_read(0, 0, p)[0] for p in range(P)])
    vf = np.stack([f.kv_read(0, 0, p)[1] for p in range(P)])
    rows8 = [q8.kv_read(0, 0, p) for p in range(P)]
    frozen, kcol, vcol = q8.kv_field(0)
    assert frozen
    yf, pf = O.attend(qh, kf, vf, P - 1, 0, probs=True)
    y8, p8 = O.attend_q8(qh, np.stack([r[0] for r in rows8]), np.stack([r[2] for r in rows8]),
                         np.stack([r[1] for r in rows8]), np.stack([r[3] for r in rows8]),
                         kcol, vcol, P - 1, 0, probs=True)
    for h in range(heads):
        scale = max(np.abs(yf[h]).max(), 1e-6)
        assert np.all(np.abs(yf[h] - y8[h]) <= scale * 0.03 + 1e-3)
        assert np.all(np.abs(pf[h] - p8[h]) < g["prob_tol"])
    assert q8.row_bytes() * 3 < f.row_bytes()


def test_q8_attend_equals_fp32_attend_on_dequantized_rows():
    """score = sum_g ks*<code,(q*kcol)> and y = (sum p*vs*code)*vcol are fp32
    attention over rows code*scale*field; checked frozen and not."""
    nh, nk, hd, n = 8, 2, 64, 30
    q = RNG.standard_normal((nh, hd)).astype(np.float32) * 4
    kc = RNG.integers(-127, 128, (n, nk, hd)).astype(np.int8)
    vc = RNG.integers(-127, 128, (n, nk, hd)).astype(np.int8)
    ks = RNG.uniform(0.001, 0.02, (n, nk, 2)).astype(np.float32)
    vs = RNG.uniform(0.001, 0.02, (n, nk)).astype(np.float32)
    for frozen in (False, True):
        kcol = RNG.uniform(0.5, 2, (nk, hd)).astype(np.float32) if frozen else None
        vcol = RNG.uniform(0.5, 2, (nk, hd)).astype(np.float32) if frozen else None
        kd = kc.astype(np.float64) * np.repeat(ks, 32, axis=2) * (1 if kcol is None else kcol)
        vd = vc.astype(np.float64) * vs[..., None] * (1 if vcol is None else vcol)
        y8 = O.attend_q8(q, kc, ks, vc, vs, kcol, vcol, n - 1, 3)
        # reference in fp64 through torch SDPA
        yr = _sdpa(q.astype(np.float64), np.repeat(kd, nh // nk, axis=1), np.repeat(vd, nh // nk, axis=1), n - 1, 3)
        assert np.allclose(y8, yr, rtol=2e-5, atol=1e-6), frozen
