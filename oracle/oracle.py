"""ctypes binding of the CPU oracle (liboracle.so).

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The oracle is a plain fp32
CPU forward of the Dory looped normalized GPT written from the pages of the
cortiq-engine crate ("dory.rs" and "kv_cache.rs"); it shares no code with the HIP
path.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# DORY_ORACLE_LIB names another build of the same source (the mutation tests plant
# mistakes in copies of the oracle and check that the pins catch them).
LIB_PATH = os.environ.get("DORY_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

PER_LOOP, LAST_LOOP = 0, 1
MODES = {"per_loop": PER_LOOP, "last_loop": LAST_LOOP}
ERRORS = {0: "ok", -1: "EINVAL", -2: "ESTATE", -3: "ERANGE", -4: "ENOMEM"}
KGROUP = 32

_f32p = C.POINTER(C.c_float)


class OraCfg(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("ffn", C.c_int32), ("vocab", C.c_int32),
                ("nh", C.c_int32), ("nk", C.c_int32), ("hd", C.c_int32),
                ("pattern", C.c_char_p), ("n_in", C.c_int32), ("n_rec", C.c_int32),
                ("n_out", C.c_int32), ("window", C.c_int32), ("full_window", C.c_int32),
                ("theta_s", C.c_double), ("theta_f", C.c_double),
                ("max_ctx", C.c_int32), ("max_seqs", C.c_int32), ("kv_q8", C.c_int32)]


class OraLayer(C.Structure):
    _fields_ = [(n, _f32p) for n in ("wq", "wk", "wv", "wg", "wo", "sq", "wgate", "wup",
                                     "wdown", "su", "sg", "alpha")]


class OraWeights(C.Structure):
    _fields_ = [("embed", _f32p), ("head", _f32p), ("logit_scale", _f32p),
                ("layers", C.POINTER(OraLayer))]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from oracle import build as _build
            _build.build()
        _lib = C.CDLL(LIB_PATH)
        L = _lib
        L.ora_create.argtypes = [C.POINTER(OraCfg), C.POINTER(OraWeights), C.POINTER(C.c_void_p)]
        L.ora_destroy.argtypes = [C.c_void_p]
        L.ora_forward.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_int32, C.c_int32,
                                  C.c_int32, C.c_void_p, C.c_void_p]
        L.ora_forward_want.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_int32, C.c_int32,
                                       C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]
        L.ora_set_prompt_loops.argtypes = [C.c_void_p, C.c_int32]
        L.ora_set_threads.argtypes = [C.c_int32]
        L.ora_set_gate.argtypes = [C.c_void_p, C.c_int32, C.c_float]
        L.ora_gate_stats.argtypes = [C.c_void_p, C.c_int32] + [C.c_void_p] * 4
        L.ora_top_prob.argtypes = [C.c_void_p, C.c_int32]
        L.ora_top_prob.restype = C.c_float
        L.ora_reset.argtypes = [C.c_void_p, C.c_int32]
        L.ora_rollback.argtypes = [C.c_void_p, C.c_int32, C.c_int64]
        L.ora_pos.argtypes = [C.c_void_p, C.c_int32]
        L.ora_pos.restype = C.c_int64
        L.ora_passes.argtypes = [C.c_void_p, C.c_int32]
        L.ora_slot_rows.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32]
        L.ora_slot_rows.restype = C.c_int64
        L.ora_kv_read.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_int64, C.c_void_p]
        L.ora_kv_field.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]
        L.ora_kv_load.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_int64,
                                  C.c_int32, C.c_void_p, C.c_void_p]
        L.ora_justnorm.argtypes = [C.c_void_p, C.c_int32]
        L.ora_slerp.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32]
        L.ora_rope_inv.argtypes = [C.c_int32, C.c_double, C.c_void_p]
        L.ora_rope_rotate.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_int64]
        L.ora_attend.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_int64,
                                 C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]
        L.ora_attend_q8.argtypes = [C.c_void_p] * 7 + [C.c_int64, C.c_int64, C.c_int32, C.c_int32,
                                                        C.c_int32, C.c_void_p, C.c_void_p]
        L.ora_q8_encode.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]
        L.ora_q8_freeze.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int32, C.c_int32, C.c_void_p]
        L.ora_silu_gate.argtypes = [C.c_float] * 4
        L.ora_silu_gate.restype = C.c_float
        L.ora_sigmoid_gate.argtypes = [C.c_float] * 3
        L.ora_sigmoid_gate.restype = C.c_float
    return _lib


def set_threads(n: int) -> int:
    """OpenMP threads of the oracle's loops (n <= 0: all the host's); returns
    the count in use.  Timing only: the results do not depend on it."""
    return lib().ora_set_threads(n)


def threads() -> int:
    return lib().ora_threads()


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


class OracleError(RuntimeError):
    def __init__(self, rc):
        super().__init__(f"oracle call failed: {ERRORS.get(rc, rc)}")
        self.rc = rc


def _check(rc):
    if rc != 0:
        raise OracleError(rc)


class Oracle:
    """The oracle model: ``cfg`` a geometry dict (see synth.CONFIGS), ``w`` the
    weights dict of fp32 arrays (bf16 geometries: the bf16 values upcast)."""

    def __init__(self, cfg: dict, w: dict, max_ctx: int = 4096, max_seqs: int = 1,
                 kv_q8: bool | None = None, full_window: int | None = None,
                 window: int | None = None):
        L = lib()
        self.cfg = dict(cfg)
        if kv_q8 is None:
            kv_q8 = cfg.get("kv_encoding", "f32") == "q8_2f"
        fw = cfg.get("full_window", 0) if full_window is None else full_window
        win = cfg["window"] if window is None else window
        self._keep = []
        self._pattern = cfg["pattern"].encode()
        self.c = OraCfg(cfg["hidden"], cfg["ffn"], cfg["vocab"], cfg["nh"], cfg["nk"], cfg["hd"],
                        self._pattern, cfg["n_in"], cfg["n_rec"], cfg["n_out"], win, fw,
                        cfg["theta_s"], cfg["theta_f"], max_ctx, max_seqs, int(bool(kv_q8)))
        self.kv_q8 = bool(kv_q8)
        layers = (OraLayer * len(cfg["pattern"]))()
        for i, Lw in enumerate(w["layers"]):
            for name in ("wq", "wk", "wv", "wg", "wo", "sq", "wgate", "wup", "wdown", "su", "sg", "alpha"):
                if name in Lw:
                    a = _f32(Lw[name])
                    self._keep.append(a)
                    setattr(layers[i], name, a.ctypes.data_as(_f32p))
        self._layers = layers
        emb, head, ls = _f32(w["embed"]), _f32(w["head"]), _f32(w["logit_scale"])
        self._keep += [emb, head, ls]
        self.w = OraWeights(emb.ctypes.data_as(_f32p), head.ctypes.data_as(_f32p),
                            ls.ctypes.data_as(_f32p), layers)
        h = C.c_void_p()
        _check(L.ora_create(C.byref(self.c), C.byref(self.w), C.byref(h)))
        self.h = h
        self.n_ord = sum(1 for ch in cfg["pattern"] if ch != "-")
        self.ngk = (cfg["hd"] + KGROUP - 1) // KGROUP

    def close(self):
        if self.h:
            lib().ora_destroy(self.h)
            self.h = None

    __del__ = close

    def passes(self, loops: int) -> int:
        return lib().ora_passes(self.h, loops)

    def forward(self, tokens, loops: int, kv_mode="last_loop", seq: int = 0,
                logits: bool = True, tap: bool = False):
        """One call (one chunk).  Returns (logits [vocab] or None, tap
        [passes][n][hidden] or None)."""
        mode = MODES[kv_mode] if isinstance(kv_mode, str) else kv_mode
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        n = int(tok.shape[0])
        lg = np.zeros(self.cfg["vocab"], np.float32) if logits else None
        tp = np.zeros((self.passes(loops), n, self.cfg["hidden"]), np.float32) if tap else None
        _check(lib().ora_forward(self.h, seq, _p(tok), n, loops, mode, _p(lg), _p(tp)))
        return lg, tp

    def forward_all(self, tokens, loops: int, kv_mode="last_loop", seq: int = 0):
        """One call whose logits are wanted for every row (dory.rs `Want::All`):
        returns logits [n][vocab]."""
        mode = MODES[kv_mode] if isinstance(kv_mode, str) else kv_mode
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        n = int(tok.shape[0])
        lg = np.zeros((n, self.cfg["vocab"]), np.float32)
        _check(lib().ora_forward_want(self.h, seq, _p(tok), n, loops, mode, 2, _p(lg), None))
        return lg

    def set_gate(self, th):
        """dory.rs `Gate::Conf(th)` for one-row calls; None turns it off."""
        _check(lib().ora_set_gate(self.h, 0 if th is None else 1, 0.0 if th is None else float(th)))

    def gate_stats(self, seq: int = 0):
        """(gated tokens, tokens out after one pass, last read-out's top
        probability, exit rate)."""
        t, o = C.c_int64(), C.c_int64()
        lt, r = C.c_float(), C.c_float()
        _check(lib().ora_gate_stats(self.h, seq, C.byref(t), C.byref(o), C.byref(lt), C.byref(r)))
        return t.value, o.value, lt.value, r.value

    def set_prompt_loops(self, n: int):
        """dory.rs `prompt_loops`: passes of a logits-free last_loop call (0: off)."""
        _check(lib().ora_set_prompt_loops(self.h, n))

    def forward_rc(self, tokens, loops, kv_mode, seq=0):
        """Raw status of a call (for the error-path tests)."""
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        mode = MODES[kv_mode] if isinstance(kv_mode, str) else kv_mode
        return lib().ora_forward(self.h, seq, _p(tok), int(tok.shape[0]), loops, mode, None, None)

    def reset(self, seq: int = -1):
        _check(lib().ora_reset(self.h, seq))

    def rollback(self, n: int, seq: int = 0):
        """Forget the rows from position n on (dory.rs `DoryState::rollback`)."""
        _check(lib().ora_rollback(self.h, seq, n))

    def pos(self, seq: int = 0) -> int:
        return lib().ora_pos(self.h, seq)

    def slot_rows(self, ord_: int, slot: int = 0, seq: int = 0) -> int:
        return lib().ora_slot_rows(self.h, seq, ord_, slot)

    def row_bytes(self) -> int:
        nk, hd = self.cfg["nk"], self.cfg["hd"]
        if self.kv_q8:
            return 2 * nk * hd + 4 * nk * self.ngk + 4 * nk
        return 8 * nk * hd

    def kv_read(self, ord_: int, slot: int, pos: int, seq: int = 0):
        """fp32: (K [nk][hd], V [nk][hd]); q8: (kcodes, vcodes, kscales [nk][ngk], vscales [nk])."""
        nk, hd = self.cfg["nk"], self.cfg["hd"]
        buf = np.zeros(self.row_bytes(), np.uint8)
        _check(lib().ora_kv_read(self.h, seq, ord_, slot, pos, _p(buf)))
        return split_row(buf, nk, hd, self.kv_q8)

    def kv_field(self, ord_: int, slot: int = 0, seq: int = 0):
        nk, hd = self.cfg["nk"], self.cfg["hd"]
        kc, vc = np.zeros((nk, hd), np.float32), np.zeros((nk, hd), np.float32)
        fr = lib().ora_kv_field(self.h, seq, ord_, slot, _p(kc), _p(vc))
        if fr < 0:
            raise OracleError(fr)
        return bool(fr), kc, vc

    def kv_load(self, k, v, kv_mode="last_loop", loops: int = 1, seq: int = 0):
        """k, v: [n_ord][n_slot][npos][nk][hd] fp32."""
        mode = MODES[kv_mode] if isinstance(kv_mode, str) else kv_mode
        k, v = _f32(k), _f32(v)
        _check(lib().ora_kv_load(self.h, seq, mode, loops, k.shape[2], k.shape[1], _p(k), _p(v)))


def split_row(buf: np.ndarray, nk: int, hd: int, q8: bool):
    """Splits one stored row (the layout of ora_kv_read and dory_kv_read)."""
    if not q8:
        f = buf.view(np.float32)
        return f[: nk * hd].reshape(nk, hd).copy(), f[nk * hd:].reshape(nk, hd).copy()
    ngk = (hd + KGROUP - 1) // KGROUP
    o = 0
    kc = buf[o:o + nk * hd].view(np.int8).reshape(nk, hd).copy(); o += nk * hd
    vc = buf[o:o + nk * hd].view(np.int8).reshape(nk, hd).copy(); o += nk * hd
    ks = buf[o:o + 4 * nk * ngk].view(np.float32).reshape(nk, ngk).copy(); o += 4 * nk * ngk
    vs = buf[o:o + 4 * nk].view(np.float32).copy()
    return kc, vc, ks, vs


# ------------------------------------------------------------------ stage functions

def justnorm(x):
    x = _f32(x).copy()
    lib().ora_justnorm(_p(x), x.size)
    return x


def slerp(x, o, alpha):
    x = _f32(x).copy()
    o, a = _f32(o), _f32(alpha)
    lib().ora_slerp(_p(x), _p(o), _p(a), x.size)
    return x


def rope_inv(hd: int, theta: float):
    inv = np.zeros(hd // 2, np.float32)
    lib().ora_rope_inv(hd, theta, _p(inv))
    return inv


def rope_rotate(row, inv, pos: int):
    r = _f32(row).copy()
    lib().ora_rope_rotate(_p(r), r.size, _p(_f32(inv)), pos)
    return r


def attend(q, k, v, p: int, first: int, probs: bool = False):
    """q [nh][hd]; k, v [p+1][nk][hd].  Returns y [nh][hd] (and probs [nh][n])."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    nh, hd = q.shape
    nk = k.shape[1]
    y = np.zeros((nh, hd), np.float32)
    pr = np.zeros((nh, p + 1 - first), np.float32) if probs else None
    lib().ora_attend(_p(q), _p(k), _p(v), p, first, nh, nk, hd, _p(y), _p(pr))
    return (y, pr) if probs else y


def attend_q8(q, kc, ks, vc, vs, kcol, vcol, p: int, first: int, probs: bool = False):
    q = _f32(q)
    nh, hd = q.shape
    nk = kc.shape[1]
    kc = np.ascontiguousarray(kc, np.int8)
    vc = np.ascontiguousarray(vc, np.int8)
    ks, vs = _f32(ks), _f32(vs)
    kcol = None if kcol is None else _f32(kcol)
    vcol = None if vcol is None else _f32(vcol)
    y = np.zeros((nh, hd), np.float32)
    pr = np.zeros((nh, p + 1 - first), np.float32) if probs else None
    lib().ora_attend_q8(_p(q), _p(kc), _p(ks), _p(vc), _p(vs), _p(kcol), _p(vcol), p, first,
                        nh, nk, hd, _p(y), _p(pr))
    return (y, pr) if probs else y


def q8_encode(x, col, group: int):
    x = _f32(x)
    n = x.size
    codes = np.zeros(n, np.int8)
    scales = np.zeros((n + group - 1) // group, np.float32)
    lib().ora_q8_encode(_p(x), None if col is None else _p(_f32(col)), n, group, _p(codes), _p(scales))
    return codes, scales


def q8_freeze(codes, scales, group: int):
    codes = np.ascontiguousarray(codes, np.int8).copy()
    scales = _f32(scales).copy()
    rows, hd = codes.shape
    col = np.zeros(hd, np.float32)
    lib().ora_q8_freeze(_p(codes), _p(scales), rows, hd, group, _p(col))
    return codes, scales, col


def silu_gate(a, sg, b, su):
    return lib().ora_silu_gate(a, sg, b, su)


def sigmoid_gate(y, g, sg):
    return lib().ora_sigmoid_gate(y, g, sg)


def top_prob(lg) -> float:
    """dory.rs `top_prob` on a row of logits."""
    a = np.ascontiguousarray(lg, dtype=np.float32)
    return float(lib().ora_top_prob(_p(a), int(a.shape[0])))
