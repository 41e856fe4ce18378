"""Helpers for the GPU parity tests: comparison metrics and paired runs of the
HIP path and the oracle on the same seeded inputs."""
import sys

import numpy as np


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def cos_rows(a, b):
    """Cosine between matching rows of two [..., H] arrays (fp64)."""
    a = np.asarray(a, np.float64).reshape(-1, a.shape[-1])
    b = np.asarray(b, np.float64).reshape(-1, b.shape[-1])
    na, nb = np.linalg.norm(a, axis=1), np.linalg.norm(b, axis=1)
    both_zero = (na == 0) & (nb == 0)
    c = (a * b).sum(1) / np.maximum(na * nb, 1e-300)
    c[both_zero] = 1.0
    return c


def run_pair(gpu, ora, calls, loops, mode, tap=True, logits=True):
    """Runs the same calls on the HIP path and the oracle.  Returns a list of
    (gpu_logits, ora_logits, gpu_tap, ora_tap) per call."""
    import torch
    out = []
    for toks in calls:
        toks = np.asarray(toks, np.int32)
        n = len(toks)
        buf = None
        if tap:
            buf = torch.full((gpu.passes(loops), n, gpu.cfg["hidden"]), float("nan"),
                             dtype=torch.float32, device=gpu.device)
            gpu.set_tap(buf)
        lg = gpu.forward(toks, loops, mode, logits=logits)
        torch.cuda.synchronize()
        glg = lg.cpu().numpy() if lg is not None else None
        gtap = buf.cpu().numpy() if tap else None
        olg, otap = ora.forward(toks, loops, mode, logits=logits, tap=tap)
        out.append((glg, olg, gtap, otap))
    if tap:
        gpu.set_tap(None)
    return out


def check_pair(res, cos_min, logit_tol, what=""):
    worst_cos, worst_lg = 1.0, 0.0
    for i, (glg, olg, gtap, otap) in enumerate(res):
        if gtap is not None:
            assert np.isfinite(gtap).all(), f"{what} call {i}: tap has non-finite values"
            c = cos_rows(gtap, otap)
            worst_cos = min(worst_cos, float(c.min()))
            assert c.min() >= cos_min, f"{what} call {i}: residual cosine {c.min():.7f} < {cos_min}"
        if glg is not None:
            d = float(np.abs(glg - olg).max())
            worst_lg = max(worst_lg, d)
            assert d <= logit_tol, f"{what} call {i}: max |dlogit| {d:.3e} > {logit_tol}"
    say(f"{what}: worst residual cosine {worst_cos:.8f}, worst |dlogit| {worst_lg:.3e}")
    return worst_cos, worst_lg
