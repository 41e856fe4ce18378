"""Seeded synthetic inputs for the Dory token forward: model geometries, weights,
tokens, loop counts and KV rows.

This module serves both the HIP path and the CPU oracle.  It holds none of the
method's arithmetic: it only draws numbers (NumPy PCG64), normalises weight rows
to unit length and rounds them to bf16, which is the input recipe, not a step of
the forward.

Geometries
----------
* ``tiny``: hidden 256, 16 q / 4 kv heads of 16, ffn 688, vocab 512, one
  attention+SwiGLU block in each of the input, recurrent and output stacks
  (sub-layer pattern ``S-*-S-``), loops 2, sliding window 64, fp32 weights.
* ``2b``: hidden 2048, 16 q / 4 kv heads of 128, ffn 5632, vocab 32000, 2/4/2
  attention+SwiGLU blocks (sub-layers ``S-*-`` | ``S-*-S-*-`` | ``S-*-``),
  sliding layers (window 1024) alternating with full ones, bf16 weights.
* ``pages``: the unit-test geometry of the Dory module page (dory.rs, test
  module, ``tiny``): hidden 16, ffn 16, 4 q / 2 kv heads of 8, vocab 11, pattern
  ``S-*-S-*-S-*-`` with 4/4/4 sub-layers, constant scale vectors and a 32-bit
  LCG for the matrices, reproduced from that fixture's published definition.

RoPE bases are the only ones the pages print (full 1e7, sliding 1e4).
"""
from __future__ import annotations

import numpy as np

MAX_LOOPS = 16

BASE = dict(theta_s=1.0e4, theta_f=1.0e7, full_window=0, kv_encoding="f32")

CONFIGS = {
    "tiny": dict(BASE, hidden=256, ffn=688, vocab=512, nh=16, nk=4, hd=16,
                 pattern="S-*-S-", n_in=2, n_rec=2, n_out=2, loops=2, window=64,
                 weight_dtype="f32", kv_mode="last_loop"),
    "2b": dict(BASE, hidden=2048, ffn=5632, vocab=32000, nh=16, nk=4, hd=128,
               pattern="S-*-S-*-S-*-S-*-", n_in=4, n_rec=8, n_out=4, loops=4,
               window=1024, weight_dtype="bf16", kv_mode="last_loop"),
    "pages": dict(BASE, hidden=16, ffn=16, vocab=11, nh=4, nk=2, hd=8,
                  pattern="S-*-S-*-S-*-", n_in=4, n_rec=4, n_out=4, loops=2,
                  window=5, weight_dtype="f32", kv_mode="per_loop"),
}


def config(name: str, **over) -> dict:
    """A copy of a named geometry with fields overridden."""
    c = dict(CONFIGS[name])
    c.update(over)
    assert len(c["pattern"]) == c["n_in"] + c["n_rec"] + c["n_out"]
    return c


# ---------------------------------------------------------------- bf16 rounding

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest even), returned as uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- weights

def _rownorm(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    w = rng.standard_normal((rows, cols), dtype=np.float32)
    n = np.sqrt(np.einsum("ij,ij->i", w, w, dtype=np.float64))
    w /= n[:, None].astype(np.float32)
    return w


def _uniform(rng, n, lo, hi, scale):
    return (scale * rng.uniform(lo, hi, size=n)).astype(np.float32)


MATRICES_ATTN = ("wq", "wk", "wv", "wg", "wo")
MATRICES_MLP = ("wgate", "wup", "wdown")


def make_weights(cfg: dict, seed: int = 1) -> dict:
    """Seeded weights for a geometry.

    Returns ``{"embed", "head", "logit_scale", "layers": [dict, ...]}`` with fp32
    arrays.  For a bf16 geometry every matrix is rounded to bf16 and the fp32
    arrays hold those values exactly; ``"<name>_bf16"`` keys hold the bit
    patterns.  Vectors are the effective (already folded) scales.
    """
    if cfg.get("fixture") == "lcg" or (cfg["hidden"] == 16 and cfg["vocab"] == 11):
        return _pages_fixture_weights(cfg)
    H, F, V = cfg["hidden"], cfg["ffn"], cfg["vocab"]
    Q, KV = cfg["nh"] * cfg["hd"], cfg["nk"] * cfg["hd"]
    rng = np.random.Generator(np.random.PCG64(seed))
    sH = float(np.sqrt(H))
    out = {"embed": _rownorm(rng, V, H), "layers": []}
    for kind in cfg["pattern"]:
        if kind == "-":
            L = {"kind": "mlp",
                 "wgate": _rownorm(rng, F, H), "wup": _rownorm(rng, F, H),
                 "wdown": _rownorm(rng, H, F),
                 "sg": _uniform(rng, F, 0.8, 1.2, sH), "su": _uniform(rng, F, 0.8, 1.2, sH),
                 "alpha": _uniform(rng, H, 0.05, 0.35, 1.0)}
        else:
            L = {"kind": "attn", "sliding": kind == "S",
                 "wq": _rownorm(rng, Q, H), "wk": _rownorm(rng, KV, H),
                 "wv": _rownorm(rng, KV, H), "wg": _rownorm(rng, Q, H),
                 "wo": _rownorm(rng, H, Q),
                 "sq": _uniform(rng, Q, 0.8, 1.2, float(cfg["hd"])),
                 "sg": _uniform(rng, Q, 0.5, 1.5, sH),
                 "alpha": _uniform(rng, H, 0.05, 0.35, 1.0)}
        out["layers"].append(L)
    out["head"] = _rownorm(rng, V, H)
    out["logit_scale"] = _uniform(rng, V, 0.8, 1.2, sH)
    if cfg["weight_dtype"] == "bf16":
        _round_bf16(out)
    return out


def _round_bf16(w: dict) -> None:
    for name in ("embed", "head"):
        b = bf16_bits(w[name])
        w[name + "_bf16"] = b
        w[name] = bf16_to_f32(b).reshape(w[name].shape)
    for L in w["layers"]:
        for name in (MATRICES_ATTN if L["kind"] == "attn" else MATRICES_MLP):
            b = bf16_bits(L[name])
            L[name + "_bf16"] = b
            L[name] = bf16_to_f32(b).reshape(L[name].shape)


def _pages_fixture_weights(cfg: dict) -> dict:
    """The Dory page's test fixture: matrices from the 32-bit LCG
    ``seed = seed*1664525 + 1013904223`` starting at seed 1, each value
    ``((seed >> 8) / 2**24 - 0.5) * 0.7``, drawn per sub-layer in pattern order
    (MLP: gate, up, down; attention: q, k, v, g, o), then embed and head.  Scale
    vectors are the fixture's constants (MLP sg 1.5, su 1.2, alpha 0.3; attention
    sq 4.0, sg 2.0, alpha 0.2; logit scale 3.0)."""
    H, F, V = cfg["hidden"], cfg["ffn"], cfg["vocab"]
    Q, KV = cfg["nh"] * cfg["hd"], cfg["nk"] * cfg["hd"]
    state = [1]

    def rnd(rows, cols):
        n = rows * cols
        vals = np.empty(n, dtype=np.float32)
        s = state[0]
        for i in range(n):
            s = (s * 1664525 + 1013904223) & 0xFFFFFFFF
            vals[i] = np.float32((np.float32(s >> 8) / np.float32(1 << 24) - np.float32(0.5)) * np.float32(0.7))
        state[0] = s
        return vals.reshape(rows, cols)

    layers = []
    for kind in cfg["pattern"]:
        if kind == "-":
            layers.append({"kind": "mlp", "wgate": rnd(F, H), "wup": rnd(F, H), "wdown": rnd(H, F),
                           "sg": np.full(F, 1.5, np.float32), "su": np.full(F, 1.2, np.float32),
                           "alpha": np.full(H, 0.3, np.float32)})
        else:
            layers.append({"kind": "attn", "sliding": kind == "S",
                           "wq": rnd(Q, H), "wk": rnd(KV, H), "wv": rnd(KV, H),
                           "wg": rnd(Q, H), "wo": rnd(H, Q),
                           "sq": np.full(Q, 4.0, np.float32), "sg": np.full(Q, 2.0, np.float32),
                           "alpha": np.full(H, 0.2, np.float32)})
    embed = rnd(V, H)
    head = rnd(V, H)
    return {"embed": embed, "head": head, "logit_scale": np.full(V, 3.0, np.float32),
            "layers": layers}


# ---------------------------------------------------------------- tokens, loops, KV rows

def make_tokens(n: int, vocab: int, seq: int = 0) -> np.ndarray:
    """Seeded token ids in [0, vocab): sequence ``seq`` draws from PCG64(2 + 1000*seq)."""
    rng = np.random.Generator(np.random.PCG64(2 + 1000 * seq))
    return rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def make_loops(n: int, seed: int = 3) -> np.ndarray:
    """Seeded per-token loop counts, uniform on 1..16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(1, MAX_LOOPS + 1, size=n, dtype=np.int64).astype(np.int32)


def make_kv_rows(npos: int, nk: int, hd: int, hidden: int, seed: int = 4):
    """Synthetic cache rows ``(K, V)``, each ``[npos][nk][hd]`` fp32: keys are
    random unit vectors per kv head (stored keys are normalised per head), values
    are N(0, 1/hidden), the spread of a projection of a unit vector by unit rows."""
    rng = np.random.Generator(np.random.PCG64(seed))
    k = rng.standard_normal((npos, nk, hd), dtype=np.float32)
    k /= np.sqrt(np.einsum("pkd,pkd->pk", k, k, dtype=np.float64))[..., None].astype(np.float32)
    v = (rng.standard_normal((npos, nk, hd), dtype=np.float32)
         * np.float32(1.0 / np.sqrt(hidden)))
    return np.ascontiguousarray(k), np.ascontiguousarray(v)
