"""Thin ctypes binding of libdory.so (the C ABI declared in include/dory.h).

Argument marshalling only: every step of the forward runs in the library's HIP
kernels.  PyTorch provides the device memory (weights, logits, taps) and the
stream.  Importing this module fails loudly when the library is not built.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdory.so")

OK, EINVAL, ESTATE, ERANGE, ENOMEM, EDEVICE = 0, -1, -2, -3, -4, -5
PER_LOOP, LAST_LOOP = 0, 1
KV_F32, KV_Q8_2F = 0, 1
W_F32, W_BF16 = 0, 1
MODES = {"per_loop": PER_LOOP, "last_loop": LAST_LOOP}
ERRNAMES = {0: "OK", -1: "EINVAL", -2: "ESTATE", -3: "ERANGE", -4: "ENOMEM", -5: "EDEVICE"}
KGROUP = 32


class DoryConfig(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("ffn", C.c_int32), ("vocab", C.c_int32),
                ("nh", C.c_int32), ("nk", C.c_int32), ("hd", C.c_int32),
                ("layer_pattern", C.c_char_p),
                ("n_in", C.c_int32), ("n_rec", C.c_int32), ("n_out", C.c_int32),
                ("window", C.c_int32), ("full_window", C.c_int32),
                ("rope_theta_sliding", C.c_double), ("rope_theta_full", C.c_double),
                ("max_ctx", C.c_int32), ("max_chunk", C.c_int32), ("max_seqs", C.c_int32),
                ("kv_encoding", C.c_int32), ("weight_dtype", C.c_int32)]


class DoryLayerWeights(C.Structure):
    _fields_ = [("wq", C.c_void_p), ("wk", C.c_void_p), ("wv", C.c_void_p), ("wg", C.c_void_p),
                ("wo", C.c_void_p), ("sq", C.c_void_p), ("wgate", C.c_void_p), ("wup", C.c_void_p),
                ("wdown", C.c_void_p), ("su", C.c_void_p), ("sg", C.c_void_p), ("alpha", C.c_void_p)]


class DoryWeights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("head", C.c_void_p), ("logit_scale", C.c_void_p),
                ("layers", C.POINTER(DoryLayerWeights))]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run python -m looped_normalized_gpt_amd.build")
    L = C.CDLL(LIB_PATH)
    vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
    L.dory_create.argtypes = [C.POINTER(DoryConfig), C.POINTER(DoryWeights), C.POINTER(vp)]
    L.dory_destroy.argtypes = [vp]
    L.dory_destroy.restype = None
    L.dory_last_error.argtypes = [vp]
    L.dory_last_error.restype = C.c_char_p
    L.dory_forward_chunk.argtypes = [vp, i32, vp, i32, i32, i32, vp, vp]
    L.dory_forward_batch.argtypes = [vp, i32, vp, vp, vp, i32, vp, vp]
    L.dory_kv_reset.argtypes = [vp, i32]
    L.dory_rollback.argtypes = [vp, i32, i64]
    L.dory_forward_chunk_all.argtypes = [vp, i32, vp, i32, i32, i32, vp, vp]
    L.dory_forward_chunk_noalloc.argtypes = [vp, i32, vp, i32, i32, i32, vp, vp]
    L.dory_set_prompt_loops.argtypes = [vp, i32]
    L.dory_set_gate.argtypes = [vp, i32, C.c_float]
    L.dory_gate_stats.argtypes = [vp, i32, vp, vp, vp, vp]
    L.dory_position.argtypes = [vp, i32]
    L.dory_position.restype = i64
    L.dory_latched.argtypes = [vp, i32]
    L.dory_debug_fail_launch.argtypes = [vp, i64]
    L.dory_debug_tap.argtypes = [vp, vp, i64]
    L.dory_debug_kv_tap.argtypes = [vp, vp, i64]
    L.dory_debug_xcd_merge.argtypes = [vp, i32]
    L.dory_kv_read.argtypes = [vp, i32, i32, i32, i64, vp]
    L.dory_kv_field.argtypes = [vp, i32, i32, i32, vp, vp]
    L.dory_kv_load.argtypes = [vp, i32, i32, i32, i64, i32, vp, vp]
    L.dory_q8_encode_rows.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
    L.dory_stage_bench.argtypes = [vp, i32, i32, vp]
    L.dory_probe.argtypes = [i32, vp, i64, i64, vp, vp, C.POINTER(C.c_double)]
    return L


lib = _load()


class DoryError(RuntimeError):
    def __init__(self, rc: int, msg: str):
        super().__init__(f"{ERRNAMES.get(rc, rc)}: {msg}")
        self.rc = rc


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _device_buffer(t, rows: int, cols: int, device, what: str):
    """A caller's output tensor, checked before the library writes rows x cols
    fp32 values through its pointer: contiguous float32 on the model's device
    with at least that many elements (else DoryError EINVAL, nothing called)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise DoryError(EINVAL, f"{what}: expected a torch tensor, got {type(t).__name__}")
    same = t.device.type == device.type and (device.index is None or t.device.index == device.index)
    if t.dtype != torch.float32 or not t.is_contiguous() or not same:
        raise DoryError(EINVAL, f"{what}: needs a contiguous float32 tensor on {device} "
                                f"(got {t.dtype}, contiguous={t.is_contiguous()}, {t.device})")
    if t.numel() < rows * cols:
        raise DoryError(EINVAL, f"{what}: {t.numel()} elements, the call writes {rows} x {cols}")
    return t


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


class Dory:
    """One model on the current GPU.  ``cfg``: a geometry dict (synth.CONFIGS
    layout); ``w``: weights from synth.make_weights (fp32 arrays, plus
    ``*_bf16`` bit patterns for bf16 geometries)."""

    def __init__(self, cfg: dict, w: dict, max_ctx: int = 4096, max_chunk: int = 512,
                 max_seqs: int = 1, kv_encoding: str | None = None, device: str = "cuda"):
        import torch
        self.cfg = dict(cfg)
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        kv = kv_encoding or cfg.get("kv_encoding", "f32")
        self.q8 = kv == "q8_2f"
        bf16 = cfg["weight_dtype"] == "bf16"
        self._t = []

        def mat(L, name):
            if bf16:
                a = torch.from_numpy(np.ascontiguousarray(L[name + "_bf16"]).view(np.int16))
                t = a.to(self.device).view(torch.bfloat16)
            else:
                t = torch.from_numpy(np.ascontiguousarray(L[name], dtype=np.float32)).to(self.device)
            self._t.append(t)
            return C.c_void_p(t.data_ptr())

        def vec(L, name):
            t = torch.from_numpy(np.ascontiguousarray(L[name], dtype=np.float32)).to(self.device)
            self._t.append(t)
            return C.c_void_p(t.data_ptr())

        nl = len(cfg["pattern"])
        layers = (DoryLayerWeights * nl)()
        for i, Lw in enumerate(w["layers"]):
            x = layers[i]
            if Lw["kind"] == "attn":
                x.wq, x.wk, x.wv, x.wg, x.wo = (mat(Lw, n) for n in ("wq", "wk", "wv", "wg", "wo"))
                x.sq, x.sg, x.alpha = vec(Lw, "sq"), vec(Lw, "sg"), vec(Lw, "alpha")
            else:
                x.wgate, x.wup, x.wdown = (mat(Lw, n) for n in ("wgate", "wup", "wdown"))
                x.sg, x.su, x.alpha = vec(Lw, "sg"), vec(Lw, "su"), vec(Lw, "alpha")
        self._layers = layers
        self._wts = DoryWeights(mat(w, "embed"), mat(w, "head"), vec(w, "logit_scale"), layers)
        self._pattern = cfg["pattern"].encode()
        self._cfg = DoryConfig(cfg["hidden"], cfg["ffn"], cfg["vocab"], cfg["nh"], cfg["nk"], cfg["hd"],
                               self._pattern, cfg["n_in"], cfg["n_rec"], cfg["n_out"],
                               cfg["window"], cfg.get("full_window", 0), cfg["theta_s"], cfg["theta_f"],
                               max_ctx, max_chunk, max_seqs, KV_Q8_2F if self.q8 else KV_F32,
                               W_BF16 if bf16 else W_F32)
        torch.cuda.synchronize(self.device)
        h = C.c_void_p()
        rc = lib.dory_create(C.byref(self._cfg), C.byref(self._wts), C.byref(h))
        if rc != OK:
            raise DoryError(rc, lib.dory_last_error(None).decode())
        self.h = h
        self.max_ctx, self.max_chunk, self.max_seqs = max_ctx, max_chunk, max_seqs
        self.n_ord = sum(1 for ch in cfg["pattern"] if ch != "-")
        self.ngk = (cfg["hd"] + KGROUP - 1) // KGROUP
        self._tap = None

    def close(self):
        if getattr(self, "h", None):
            lib.dory_destroy(self.h)
            self.h = None

    __del__ = close

    def _check(self, rc):
        if rc != OK:
            raise DoryError(rc, lib.dory_last_error(self.h).decode())

    def passes(self, loops: int) -> int:
        c = self.cfg
        return c["n_in"] + c["n_rec"] * loops + c["n_out"]

    def forward(self, tokens, loops: int, kv_mode="last_loop", seq: int = 0, logits=True, stream=None):
        """One call.  ``logits``: True (allocate), a device fp32 tensor [vocab],
        or False/None (no head).  Returns the logits tensor or None."""
        import torch
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        out = None
        if logits is True:
            out = torch.empty(self.cfg["vocab"], dtype=torch.float32, device=self.device)
        elif logits is not None and logits is not False:
            out = _device_buffer(logits, 1, self.cfg["vocab"], self.device, "forward: logits")
        mode = MODES[kv_mode] if isinstance(kv_mode, str) else kv_mode
        rc = lib.dory_forward_chunk(self.h, seq, tok.ctypes.data_as(C.c_void_p), int(tok.shape[0]), loops,
                                    mode, _stream(stream), _ptr(out))
        self._check(rc)
        return out

    def forward_noalloc(self, tokens, loops: int, kv_mode="last_loop", seq: int = 0, logits=None, stream=None):
        """dory_forward_chunk_noalloc (up to 8 rows, nothing allocated by the
        library): ``logits`` is a caller's device fp32 tensor [vocab] or None."""
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        if logits is not None:
            _device_buffer(logits, 1, self.cfg["vocab"], self.device, "forward_noalloc: logits")
        mode = MODES[kv_mode] if isinstance(kv_mode, str) else kv_mode
        self._check(lib.dory_forward_chunk_noalloc(self.h, seq, tok.ctypes.data_as(C.c_void_p), int(tok.shape[0]),
                                                   loops, mode, _stream(stream), _ptr(logits)))
        return logits

    def forward_all(self, tokens, loops: int, kv_mode="last_loop", seq: int = 0, stream=None):
        """One call with the logits of every row (dory_forward_chunk_all):
        returns a device fp32 tensor [n][vocab]."""
        import torch
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        out = torch.empty((int(tok.shape[0]), self.cfg["vocab"]), dtype=torch.float32, device=self.device)
        mode = MODES[kv_mode] if isinstance(kv_mode, str) else kv_mode
        self._check(lib.dory_forward_chunk_all(self.h, seq, tok.ctypes.data_as(C.c_void_p), int(tok.shape[0]),
                                               loops, mode, _stream(stream), _ptr(out)))
        return out

    def set_gate(self, th):
        """dory_set_gate: the confidence-gated early exit (None: off)."""
        self._check(lib.dory_set_gate(self.h, 0 if th is None else 1, 0.0 if th is None else float(th)))

    def gate_stats(self, seq: int = 0):
        """(gated tokens, tokens out after one pass, last read-out's top
        probability, exit rate)."""
        t, o = C.c_int64(), C.c_int64()
        lt, r = C.c_float(), C.c_float()
        self._check(lib.dory_gate_stats(self.h, seq, C.byref(t), C.byref(o), C.byref(lt), C.byref(r)))
        return t.value, o.value, lt.value, r.value

    def set_prompt_loops(self, n: int):
        """dory_set_prompt_loops: passes of a logits-free last_loop call (0: off)."""
        self._check(lib.dory_set_prompt_loops(self.h, n))

    def forward_batch(self, seqs, tokens, loops, kv_mode="last_loop", logits=True, stream=None):
        """One decode step of several sequences: row i = next token of seqs[i] with
        loops[i] passes.  Returns logits [nseq][vocab] (device) or None."""
        import torch
        sq = np.ascontiguousarray(seqs, dtype=np.int32)
        tk = np.ascontiguousarray(tokens, dtype=np.int32)
        lp = np.ascontiguousarray(loops, dtype=np.int32)
        out = None
        if logits is True:
            out = torch.empty((len(sq), self.cfg["vocab"]), dtype=torch.float32, device=self.device)
        elif logits is not None and logits is not False:
            out = _device_buffer(logits, len(sq), self.cfg["vocab"], self.device, "forward_batch: logits")
        mode = MODES[kv_mode] if isinstance(kv_mode, str) else kv_mode
        rc = lib.dory_forward_batch(self.h, len(sq), sq.ctypes.data_as(C.c_void_p), tk.ctypes.data_as(C.c_void_p),
                                    lp.ctypes.data_as(C.c_void_p), mode, _stream(stream), _ptr(out))
        self._check(rc)
        return out

    def forward_rc(self, tokens, loops, kv_mode, seq=0, logits=None):
        """Raw status of a call (error-path tests)."""
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        mode = MODES[kv_mode] if isinstance(kv_mode, str) else kv_mode
        if logits is not None:
            _device_buffer(logits, 1, self.cfg["vocab"], self.device, "forward_rc: logits")
        return lib.dory_forward_chunk(self.h, seq, tok.ctypes.data_as(C.c_void_p), int(tok.shape[0]), loops,
                                      mode, _stream(None), _ptr(logits))

    def batch_rc(self, seqs, tokens, loops, kv_mode="last_loop", logits=None):
        """Raw status of a batched call (error-path tests)."""
        sq = np.ascontiguousarray(seqs, dtype=np.int32)
        tk = np.ascontiguousarray(tokens, dtype=np.int32)
        lp = np.ascontiguousarray(loops, dtype=np.int32)
        mode = MODES[kv_mode] if isinstance(kv_mode, str) else kv_mode
        if logits is not None:
            _device_buffer(logits, len(sq), self.cfg["vocab"], self.device, "batch_rc: logits")
        return lib.dory_forward_batch(self.h, len(sq), sq.ctypes.data_as(C.c_void_p), tk.ctypes.data_as(C.c_void_p),
                                      lp.ctypes.data_as(C.c_void_p), mode, _stream(None), _ptr(logits))

    def latched(self, seq: int = 0) -> bool:
        """dory_latched: the sequence refuses calls until it is reset."""
        rc = lib.dory_latched(self.h, seq)
        if rc < 0:
            self._check(rc)
        return bool(rc)

    def fail_launch(self, n: int):
        """dory_debug_fail_launch: the n-th launch from now fails before it is
        launched (0: off)."""
        self._check(lib.dory_debug_fail_launch(self.h, n))

    def xcd_merge(self, on=None) -> bool:
        """dory_debug_xcd_merge: True/False selects the sliding layers'
        in-kernel split merge or the merge kernel for one-row calls (None:
        unchanged); returns whether the in-kernel merge is in use."""
        rc = lib.dory_debug_xcd_merge(self.h, -1 if on is None else int(bool(on)))
        if rc < 0:
            self._check(rc)
        return bool(rc)

    def reset(self, seq: int = -1):
        self._check(lib.dory_kv_reset(self.h, seq))

    def rollback(self, n: int, seq: int = 0):
        """Forget the sequence's rows from position n on (dory_rollback)."""
        self._check(lib.dory_rollback(self.h, seq, n))

    def position(self, seq: int = 0) -> int:
        return lib.dory_position(self.h, seq)

    def set_tap(self, buf):
        """buf: device fp32 tensor (or None to turn the tap off)."""
        if buf is not None:
            _device_buffer(buf, 1, buf.numel(), self.device, "set_tap: buffer")
        self._tap = buf
        self._check(lib.dory_debug_tap(self.h, _ptr(buf), 0 if buf is None else buf.numel()))

    def set_kv_tap(self, buf):
        """dory_debug_kv_tap: buf a device fp32 tensor [attention passes][n][2][KV],
        or None to turn the tap off."""
        if buf is not None:
            _device_buffer(buf, 1, buf.numel(), self.device, "set_kv_tap: buffer")
        self._kvtap = buf
        self._check(lib.dory_debug_kv_tap(self.h, _ptr(buf), 0 if buf is None else buf.numel()))

    def attn_passes(self, loops: int) -> int:
        c = self.cfg
        return sum((loops if c["n_in"] <= i < c["n_in"] + c["n_rec"] else 1)
                   for i, ch in enumerate(c["pattern"]) if ch != "-")

    def row_bytes(self) -> int:
        nk, hd = self.cfg["nk"], self.cfg["hd"]
        return 2 * nk * hd + 4 * nk * self.ngk + 4 * nk if self.q8 else 8 * nk * hd

    def kv_read(self, ord_: int, slot: int, pos: int, seq: int = 0):
        buf = np.zeros(self.row_bytes(), np.uint8)
        self._check(lib.dory_kv_read(self.h, seq, ord_, slot, pos, buf.ctypes.data_as(C.c_void_p)))
        return split_row(buf, self.cfg["nk"], self.cfg["hd"], self.q8)

    def kv_field(self, ord_: int, slot: int = 0, seq: int = 0):
        nk, hd = self.cfg["nk"], self.cfg["hd"]
        kc, vc = np.zeros((nk, hd), np.float32), np.zeros((nk, hd), np.float32)
        rc = lib.dory_kv_field(self.h, seq, ord_, slot, kc.ctypes.data_as(C.c_void_p),
                               vc.ctypes.data_as(C.c_void_p))
        if rc < 0:
            self._check(rc)
        return bool(rc), kc, vc

    def kv_load(self, k, v, kv_mode="last_loop", loops: int = 1, seq: int = 0):
        """k, v: host fp32 [n_ord][n_slot][npos][nk][hd]."""
        k = np.ascontiguousarray(k, dtype=np.float32)
        v = np.ascontiguousarray(v, dtype=np.float32)
        mode = MODES[kv_mode] if isinstance(kv_mode, str) else kv_mode
        self._check(lib.dory_kv_load(self.h, seq, mode, loops, k.shape[2], k.shape[1],
                                     k.ctypes.data_as(C.c_void_p), v.ctypes.data_as(C.c_void_p)))


STAGES = {"qkvg": 0, "attn": 1, "o": 2, "gateup": 3, "down": 4, "head": 5,
          "gemm_qkvg": 6, "gemm_o": 7, "gemm_gateup": 8, "gemm_down": 9, "attn_chunk": 10}


def stage_bench(model: "Dory", stage: str, reps: int, stream=None):
    """Launches one kernel of the forward `reps` times (see dory_stage_bench)."""
    model._check(lib.dory_stage_bench(model.h, STAGES[stage], reps, _stream(stream)))


def split_row(buf: np.ndarray, nk: int, hd: int, q8: bool):
    """One stored row in the layout of dory_kv_read."""
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


def q8_encode_rows(x, col, group: int, stream=None):
    """The isolated q8_2f encoder: x device fp32 [rows][n]; col device [n] or None."""
    import torch
    rows, n = x.shape
    ng = 1 if group >= n else (n + group - 1) // group
    codes = torch.empty((rows, n), dtype=torch.int8, device=x.device)
    scales = torch.empty((rows, ng), dtype=torch.float32, device=x.device)
    rc = lib.dory_q8_encode_rows(_ptr(x), _ptr(col), rows, n, group, _ptr(codes), _ptr(scales), _stream(stream))
    if rc != OK:
        raise DoryError(rc, lib.dory_last_error(None).decode())
    return codes, scales


def probe(kind: str, buf=None, iters: int = 0, sink=None, stream=None) -> float:
    """dory_probe: launches one peak probe ("stream": one read of the device
    tensor buf; "mfma": iters bf16 MFMA iterations) and returns the bytes or
    flops of the launch.  sink: a device tensor of at least 4 bytes."""
    work = C.c_double()
    k = {"stream": 0, "mfma": 1}[kind]
    nbytes = 0 if buf is None else buf.numel() * buf.element_size()
    rc = lib.dory_probe(k, _ptr(buf), nbytes, iters, _ptr(sink), _stream(stream), C.byref(work))
    if rc != OK:
        raise DoryError(rc, f"dory_probe({kind})")
    return work.value
