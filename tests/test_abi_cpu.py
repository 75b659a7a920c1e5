"""Host-side checks of the C ABI: the library loads, exports every function
include/llama_layer.h declares, and rejects bad arguments before it touches
the GPU (every case here returns from argument validation, so no HIP call is
made).  No GPU is needed."""
import ctypes
import os
import re
import subprocess

import pytest

import llama_decoder_block_amd as lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "llama_layer.h")
MODEL_HEADER = os.path.join(ROOT, "include", "llama_model.h")


def _declared_functions(header=HEADER, pattern=r"llama_layer_[a-z0-9_]+"):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(" + pattern + r")\s*\(", text)))


def _model_functions():
    return _declared_functions(MODEL_HEADER, r"llama_model_[a-z_]+|llama_sample")


def test_header_declares_the_abi():
    assert _declared_functions() == sorted(lib.EXPORTED)
    assert _model_functions() == sorted(lib.EXPORTED_MODEL)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (llama_[a-z0-9_]+)\b", out))
    for name in _declared_functions() + _model_functions():
        assert name in exported, name
        assert hasattr(lib.LIB, name)


def test_model_and_sampling_reject_bad_arguments():
    """Argument validation of the generation ABI returns before any HIP call."""
    h = ctypes.c_void_p()
    lw = (lib.LlamaLayerWeights * 1)(_weights())
    mw = lib.LlamaModelWeights(ctypes.c_void_p(4096), ctypes.c_void_p(4096), ctypes.c_void_p(4096), lw)
    cfg = lib.LlamaModelConfig(_cfg(), 0, 100)
    assert lib.LIB.llama_model_create(ctypes.byref(cfg), ctypes.byref(mw), None, ctypes.byref(h)) == \
        lib.LLAMA_ERR_INVALID  # no layers
    cfg = lib.LlamaModelConfig(_cfg(), 2, 1)
    assert lib.LIB.llama_model_create(ctypes.byref(cfg), ctypes.byref(mw), None, ctypes.byref(h)) == \
        lib.LLAMA_ERR_INVALID  # vocab < 2
    assert lib.LIB.llama_model_create(None, ctypes.byref(mw), None, ctypes.byref(h)) == lib.LLAMA_ERR_NULL
    fake = ctypes.c_void_p(4096)
    bad = [lib.make_sampling(temperature=-1.0), lib.make_sampling(top_p=0.0), lib.make_sampling(top_p=1.5),
           lib.make_sampling(repetition_penalty=0.5), lib.make_sampling(temperature=float("nan"))]
    for p in bad:
        assert lib.LIB.llama_sample(fake, 2, 100, 100, ctypes.byref(p), None, None, 0, fake, fake, None) == \
            lib.LLAMA_ERR_INVALID
    ok = lib.make_sampling(temperature=1.0)
    assert lib.LIB.llama_sample(fake, 2, 100, 100, ctypes.byref(ok), None, None, 0, None, fake, None) == \
        lib.LLAMA_ERR_NULL  # sampling needs uniforms
    pen = lib.make_sampling(repetition_penalty=1.3)
    assert lib.LIB.llama_sample(fake, 2, 100, 100, ctypes.byref(pen), None, None, 0, None, fake, None) == \
        lib.LLAMA_ERR_NULL  # the penalty needs a history
    assert lib.LIB.llama_sample(fake, 2, 100, 50, ctypes.byref(lib.make_sampling()), None, None, 0, None, fake,
                                None) == lib.LLAMA_ERR_INVALID  # ld < vocab
    assert lib.LIB.llama_sample(fake, 2, 1, 1, ctypes.byref(lib.make_sampling()), None, None, 0, None, fake,
                                None) == lib.LLAMA_ERR_INVALID  # vocab < 2


def test_strerror_covers_every_status():
    for st in (lib.LLAMA_OK, lib.LLAMA_ERR_NULL, lib.LLAMA_ERR_INVALID, lib.LLAMA_ERR_UNSUPPORTED,
               lib.LLAMA_ERR_CAPACITY, lib.LLAMA_ERR_HIP, lib.LLAMA_ERR_ALLOC):
        msg = lib.LIB.llama_layer_strerror(st).decode()
        assert msg and msg != "unknown status"
    assert lib.LIB.llama_layer_strerror(12345).decode() == "unknown status"


def _weights(ptr=4096):
    return lib.LlamaLayerWeights(*([ctypes.c_void_p(ptr)] * len(lib.WEIGHT_NAMES)))


def _create(cfg, w):
    h = ctypes.c_void_p()
    st = lib.LIB.llama_layer_create(ctypes.byref(cfg), ctypes.byref(w), None, ctypes.byref(h))
    return st, h


def _cfg(**kw):
    base = dict(d_model=512, n_heads=4, n_kv_heads=2, head_dim=128, d_ff=1408, max_pos=64,
                max_tokens=64, dtype="bf16")
    base.update(kw)
    return lib.make_config(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(n_heads=6, n_kv_heads=4), lib.LLAMA_ERR_INVALID),          # H % Hkv != 0
    (dict(head_dim=127, dtype="f32"), lib.LLAMA_ERR_INVALID),        # odd head_dim
    (dict(d_model=0), lib.LLAMA_ERR_INVALID),
    (dict(max_pos=-1), lib.LLAMA_ERR_INVALID),
    (dict(head_dim=64), lib.LLAMA_ERR_UNSUPPORTED),                  # bf16 needs dh 128
    (dict(d_ff=1400), lib.LLAMA_ERR_UNSUPPORTED),                    # bf16 needs f % 128 == 0
    (dict(d_model=520), lib.LLAMA_ERR_UNSUPPORTED),
    (dict(d_model=10240, n_heads=80, n_kv_heads=8), lib.LLAMA_ERR_UNSUPPORTED),  # no fragment-order norm
    (dict(d_model=12288, n_heads=96, n_kv_heads=8), lib.LLAMA_ERR_UNSUPPORTED),
])
def test_create_rejects_bad_configs(kw, status):
    st, h = _create(_cfg(**kw), _weights())
    assert st == status
    assert not h.value
    assert lib.LIB.llama_layer_last_error().decode()


def test_create_rejects_null_weights_and_bad_eps():
    w = _weights()
    w.w_up = None
    st, _ = _create(_cfg(), w)
    assert st == lib.LLAMA_ERR_NULL
    cfg = _cfg()
    cfg.rms_eps = float("nan")
    st, _ = _create(cfg, _weights())
    assert st == lib.LLAMA_ERR_INVALID
    st = lib.LIB.llama_layer_create(None, None, None, None)
    assert st == lib.LLAMA_ERR_NULL


def test_calls_reject_null_handle():
    p = ctypes.c_void_p(4096)
    assert lib.LIB.llama_layer_prefill(None, p, p, p, 1, 1, p, p, None) == lib.LLAMA_ERR_NULL
    assert lib.LIB.llama_layer_decode(None, p, p, p, 1, p, p, None) == lib.LLAMA_ERR_NULL
    assert lib.LIB.llama_layer_decode_noalloc(None, p, p, p, 1, p, p, None) == lib.LLAMA_ERR_NULL
    assert lib.LIB.llama_layer_prefill_paged(None, p, p, p, 1, 1, p, p, p, 1, 64, 1, None) == lib.LLAMA_ERR_NULL
    assert lib.LIB.llama_layer_decode_paged(None, p, p, p, 1, p, p, p, 1, 64, 1, None) == lib.LLAMA_ERR_NULL
    lib.LIB.llama_layer_destroy(None)  # no-op


def test_int8_cache_calls_reject_bad_arguments():
    """The int8 cache's calls check their pointers before any HIP call."""
    p = ctypes.c_void_p(4096)
    assert lib.LIB.llama_layer_decode_int8(None, p, p, p, 1, p, p, p, p, None) == lib.LLAMA_ERR_NULL
    assert lib.LIB.llama_layer_kv_quantize(None, p, p, 1, 1, p, p, p, p, None) == lib.LLAMA_ERR_NULL
    assert lib.LIB.llama_layer_kv_quantize(p, p, p, 1, 1, p, p, None, p, None) == lib.LLAMA_ERR_NULL
    assert lib.LIB.llama_layer_decode_int8(p, p, p, p, 1, p, p, None, p, None) == lib.LLAMA_ERR_NULL
    assert lib.LIB.llama_layer_prefill_int8(None, p, p, p, 1, 4, p, p, p, p, None) == lib.LLAMA_ERR_NULL
    assert lib.LIB.llama_layer_prefill_int8(p, p, p, p, 1, 4, p, p, p, None, None) == lib.LLAMA_ERR_NULL
    assert lib.LIB.llama_layer_prefill_paged_int8(None, p, p, p, 1, 4, p, p, p, p, p, 1, 64, 1, None) == \
        lib.LLAMA_ERR_NULL
    assert lib.LIB.llama_layer_decode_paged_int8(None, p, p, p, 1, p, p, p, p, p, 1, 64, 1, None) == lib.LLAMA_ERR_NULL
    # a scale pointer is checked before the handle is read (p is no handle)
    assert lib.LIB.llama_layer_decode_paged_int8(p, p, p, p, 1, p, p, None, p, p, 1, 64, 1, None) == \
        lib.LLAMA_ERR_NULL


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        lib._ptr(torch.zeros(4), "x")


def test_one_hip_runtime_in_the_process():
    """The library binds to the HIP runtime torch loaded (torch streams, events
    and memory are then valid inside it): exactly one libamdhip64 is mapped."""
    import re
    import torch  # noqa: F401
    maps = open("/proc/self/maps").read()
    runtimes = sorted(set(re.findall(r"/\S*libamdhip64\.so\S*", maps)))
    assert len(runtimes) == 1, runtimes


def test_ceiling_probes_reject_bad_arguments():
    """The ceiling entry points validate their arguments before any HIP call."""
    fake = ctypes.c_void_p(4096)
    flops = ctypes.c_double()
    assert lib.LIB.llama_layer_ceiling_mfma(10, None, ctypes.byref(flops), None) == lib.LLAMA_ERR_NULL
    assert lib.LIB.llama_layer_ceiling_mfma(10, fake, None, None) == lib.LLAMA_ERR_NULL
    assert lib.LIB.llama_layer_ceiling_mfma(0, fake, ctypes.byref(flops), None) == lib.LLAMA_ERR_INVALID
    assert lib.LIB.llama_layer_ceiling_read(None, 1024, fake, None) == lib.LLAMA_ERR_NULL
    assert lib.LIB.llama_layer_ceiling_read(fake, 0, fake, None) == lib.LLAMA_ERR_INVALID
    assert lib.LIB.llama_layer_ceiling_read(fake, 1000, fake, None) == lib.LLAMA_ERR_INVALID
    assert lib.LIB.llama_layer_ceiling_read(fake, 1040, fake, None) == lib.LLAMA_ERR_INVALID
    assert lib.LIB.llama_layer_ceiling_read(ctypes.c_void_p(4100), 1024, fake, None) == lib.LLAMA_ERR_INVALID
