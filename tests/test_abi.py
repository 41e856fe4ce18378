"""The C ABI library: it loads without a GPU, exports every entry point that
include/dory.h declares, and rejects bad configurations and arguments before
touching the device (CPU only: no compute call is made)."""
import ctypes as C
import os
import re

import pytest

from conftest import ROOT
from looped_normalized_gpt_amd import synth

HEADER = os.path.join(ROOT, "include", "dory.h")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dory_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared()
    for want in ("dory_create", "dory_forward_chunk", "dory_kv_reset", "dory_destroy", "dory_last_error"):
        assert want in names


def test_library_exports_every_declared_symbol():
    from looped_normalized_gpt_amd import dory
    lib = C.CDLL(dory.LIB_PATH)
    missing = [n for n in declared() if not hasattr(lib, n)]
    assert not missing, missing


def _cfg(**over):
    from looped_normalized_gpt_amd.dory import DoryConfig, DoryLayerWeights, DoryWeights, W_F32, KV_F32
    c = synth.config("tiny")
    c.update(over)
    cfg = DoryConfig(c["hidden"], c["ffn"], c["vocab"], c["nh"], c["nk"], c["hd"], c["pattern"].encode(),
                     c["n_in"], c["n_rec"], c["n_out"], c["window"], c["full_window"], 1e4, 1e7,
                     over.get("max_ctx", 256), over.get("max_chunk", 128), 1, KV_F32, W_F32)
    layers = (DoryLayerWeights * len(c["pattern"]))()
    dummy = C.c_void_p(16)   # never dereferenced: the checks fail first
    for i, ch in enumerate(c["pattern"]):
        names = ("wgate", "wup", "wdown", "sg", "su", "alpha") if ch == "-" else \
                ("wq", "wk", "wv", "wg", "wo", "sq", "sg", "alpha")
        for n in names:
            setattr(layers[i], n, dummy)
    w = DoryWeights(dummy, dummy, dummy, layers)
    return cfg, w, layers


@pytest.mark.parametrize("over,msg", [
    (dict(hd=12), "hd must be"),
    (dict(nh=6), "nh must be"),
    (dict(pattern="S-*-S"), "pattern length"),
    (dict(n_in=0, n_rec=4, pattern="S-*-S-"), "every block"),
    (dict(ffn=690), "multiples of 8"),
    (dict(window=0), "window"),
    (dict(max_chunk=512, max_ctx=256), "max_chunk"),
])
def test_create_rejects_bad_geometry_before_any_device_work(over, msg):
    from looped_normalized_gpt_amd.dory import lib, EINVAL
    cfg, w, _ = _cfg(**over)
    h = C.c_void_p(123)
    assert lib.dory_create(C.byref(cfg), C.byref(w), C.byref(h)) == EINVAL
    assert h.value is None
    assert msg in lib.dory_last_error(None).decode()


def test_create_rejects_missing_weights():
    from looped_normalized_gpt_amd.dory import lib, EINVAL
    cfg, w, layers = _cfg()
    layers[3].wup = None
    h = C.c_void_p()
    assert lib.dory_create(C.byref(cfg), C.byref(w), C.byref(h)) == EINVAL
    assert "MLP weight at sub-layer 3" in lib.dory_last_error(None).decode()


def test_null_handles_and_encoder_arguments_are_rejected():
    from looped_normalized_gpt_amd.dory import lib, EINVAL
    assert lib.dory_forward_chunk(None, 0, None, 1, 1, 0, None, None) == EINVAL
    assert lib.dory_kv_reset(None, 0) == EINVAL
    assert lib.dory_rollback(None, 0, 0) == EINVAL
    assert lib.dory_set_prompt_loops(None, 1) == EINVAL
    assert lib.dory_set_gate(None, 1, C.c_float(0.5)) == EINVAL
    assert lib.dory_gate_stats(None, 0, None, None, None, None) == EINVAL
    assert lib.dory_forward_chunk_all(None, 0, None, 1, 1, 0, None, None) == EINVAL
    assert lib.dory_debug_tap(None, None, 0) == EINVAL
    assert lib.dory_q8_encode_rows(None, None, 1, 128, 32, None, None, None) == EINVAL
    x = C.c_void_p(16)
    assert lib.dory_q8_encode_rows(x, None, 1, 300, 32, x, x, None) == EINVAL   # n > 256
    assert lib.dory_q8_encode_rows(x, None, 1, 128, 16, x, x, None) == EINVAL   # group not 32 or >= n
    lib.dory_destroy(None)


def test_binding_checks_output_tensors_before_the_call():
    """The binding refuses a caller's output tensor that the library would
    write past or misread (dtype, contiguity, device, size), before any call."""
    import torch
    from looped_normalized_gpt_amd.dory import DoryError, _device_buffer
    dev = torch.device("cpu")
    ok = torch.empty(2 * 10, dtype=torch.float32)
    assert _device_buffer(ok, 2, 10, dev, "t") is ok
    assert _device_buffer(torch.empty(30), 2, 10, dev, "t").numel() == 30
    for bad in (torch.empty(19, dtype=torch.float32), torch.empty(20, dtype=torch.float64),
                torch.empty(10, 4, dtype=torch.float32)[:, ::2], [0.0] * 20):
        with pytest.raises(DoryError):
            _device_buffer(bad, 2, 10, dev, "t")
    with pytest.raises(DoryError):
        _device_buffer(ok, 2, 10, torch.device("cuda", 0), "t")


def test_probe_rejects_bad_arguments_before_any_launch():
    """dory_probe (the peak probes) checks its arguments first: no sink or
    work pointer, a stream read of a null or unaligned buffer, an MFMA loop of
    no or too many iterations, an unknown kind."""
    from looped_normalized_gpt_amd.dory import lib, EINVAL
    w = C.c_double()
    sink = C.c_void_p(64)   # never dereferenced: the checks fail first
    assert lib.dory_probe(0, None, 1 << 20, 0, sink, None, C.byref(w)) == EINVAL
    assert lib.dory_probe(0, sink, 1000, 0, sink, None, C.byref(w)) == EINVAL      # not a multiple of 16
    assert lib.dory_probe(0, sink, 0, 0, sink, None, C.byref(w)) == EINVAL
    assert lib.dory_probe(1, None, 0, 0, sink, None, C.byref(w)) == EINVAL          # no iterations
    assert lib.dory_probe(1, None, 0, (1 << 24) + 1, sink, None, C.byref(w)) == EINVAL
    assert lib.dory_probe(2, None, 0, 10, sink, None, C.byref(w)) == EINVAL
    assert lib.dory_probe(1, None, 0, 10, None, None, C.byref(w)) == EINVAL
    assert lib.dory_probe(1, None, 0, 10, sink, None, None) == EINVAL
