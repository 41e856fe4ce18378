"""A second, independent brute-force forward in NumPy float64, used only to
cross-check the C oracle on tiny inputs.

It is written as whole-matrix algebra rather than the oracle's row loops: RoPE is
a complex multiplication, attention is a dense score matrix over every stored row
with an explicit window mask (minus infinity outside it), and the cache is a list
of per-position rows.  It follows the module summary of the Dory page (dory.rs):
attention, mlp, residual, loop and logits, and the per_loop / last_loop rules of
`stack` and `attn_layer`.  fp32 cache encoding only.
"""
import numpy as np

EPS = 1e-6


def _norm(x):
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + EPS)


def _rope(x, pos, inv):
    """x [..., t, heads, hd] rotated at positions pos [t]: pairs (j, j+hd/2) as complex numbers."""
    half = x.shape[-1] // 2
    z = x[..., :half] + 1j * x[..., half:]
    z = z * np.exp(1j * pos[:, None, None] * inv[None, None, :])
    return np.concatenate([z.real, z.imag], axis=-1)


class RefModel:
    def __init__(self, cfg, w, window=None, full_window=None):
        self.c = cfg
        self.w = w
        self.win = cfg["window"] if window is None else window
        fw = cfg.get("full_window", 0) if full_window is None else full_window
        self.fwin = fw if fw > 0 else 1 << 60
        hd = cfg["hd"]
        j = np.arange(hd // 2)
        self.inv = {k: np.power(cfg[t], -2.0 * j / hd).astype(np.float32).astype(np.float64)
                    for k, t in (("S", "theta_s"), ("F", "theta_f"))}
        self.kv = {}
        self.pos = 0

    def _attn(self, li, loop_i, h, mode):
        c, L = self.c, self.w["layers"][li]
        t = h.shape[0]
        nh, nk, hd = c["nh"], c["nk"], c["hd"]
        rec = c["n_in"] <= li < c["n_in"] + c["n_rec"]
        slot = loop_i if (mode == "per_loop" and rec) else 0
        kind = "S" if c["pattern"][li] == "S" else "F"
        pos = np.arange(self.pos, self.pos + t, dtype=np.float64)
        q = (h @ L["wq"].T.astype(np.float64)).reshape(t, nh, hd)
        k = (h @ L["wk"].T.astype(np.float64)).reshape(t, nk, hd)
        v = (h @ L["wv"].T.astype(np.float64)).reshape(t, nk, hd)
        g = h @ L["wg"].T.astype(np.float64)
        q = _norm(_rope(q, pos, self.inv[kind])) * L["sq"].reshape(nh, hd)
        k = _norm(_rope(k, pos, self.inv[kind]))
        key = (li, slot)
        K, V = self.kv.get(key, (np.zeros((0, nk, hd)), np.zeros((0, nk, hd))))
        if mode == "last_loop" and rec and loop_i > 0:
            K, V = K[:-t], V[:-t]
        K = np.concatenate([K, k])
        V = np.concatenate([V, v])
        self.kv[key] = (K, V)
        n = K.shape[0]
        W = self.win if kind == "S" else self.fwin
        e = np.arange(n)[None, :]
        p = pos.astype(np.int64)[:, None]
        visible = (e <= p) & (e > p - W)
        rep = nh // nk
        Kr = np.repeat(K, rep, axis=1)          # [n, nh, hd]
        Vr = np.repeat(V, rep, axis=1)
        s = np.einsum("thd,nhd->thn", q, Kr) / np.sqrt(hd)
        s = np.where(visible[:, None, :], s, -np.inf)
        s = s - s.max(-1, keepdims=True)
        a = np.exp(s)
        a /= a.sum(-1, keepdims=True)
        y = np.einsum("thn,nhd->thd", a, Vr).reshape(t, nh * hd)
        y = y / (1.0 + np.exp(-g * L["sg"]))
        y = _norm(y)
        return y @ L["wo"].T.astype(np.float64)

    def _mlp(self, li, h):
        L = self.w["layers"][li]
        a = (h @ L["wgate"].T.astype(np.float64)) * L["sg"]
        b = (h @ L["wup"].T.astype(np.float64)) * L["su"]
        z = _norm(a / (1.0 + np.exp(-a)) * b)
        return z @ L["wdown"].T.astype(np.float64)

    def _sub(self, li, loop_i, h, mode):
        out = self._mlp(li, h) if self.c["pattern"][li] == "-" else self._attn(li, loop_i, h, mode)
        alpha = self.w["layers"][li]["alpha"].astype(np.float64)
        xh, oh = _norm(h), _norm(out)
        return _norm(xh + alpha * (oh - xh))

    def forward(self, tokens, loops, mode):
        c = self.c
        tok = np.asarray(tokens, dtype=np.int64)
        V = c["vocab"]
        h = np.zeros((len(tok), c["hidden"]))
        ok = (tok >= 0) & (tok < V)
        h[ok] = self.w["embed"][tok[ok]]
        taps = []
        for li in range(c["n_in"]):
            h = self._sub(li, 0, h, mode)
            taps.append(h)
        inp = h.copy()
        state = inp.copy()
        for i in range(loops):
            h = _norm(state + inp)
            for li in range(c["n_in"], c["n_in"] + c["n_rec"]):
                h = self._sub(li, i, h, mode)
                taps.append(h)
            state = _norm(h)
        h = state
        for li in range(c["n_in"] + c["n_rec"], len(c["pattern"])):
            h = self._sub(li, 0, h, mode)
            taps.append(h)
        logits = (self.w["head"].astype(np.float64) @ h[-1]) * self.w["logit_scale"]
        self.pos += len(tok)
        return logits, np.stack(taps)
