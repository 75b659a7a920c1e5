"""Python binding of libllama_layer.so, the gfx950 decoder-layer library.

Argument marshalling only: torch tensors are turned into device pointers,
the current HIP stream is passed through, and status codes become
exceptions.  Every step of the layer runs in the library's HIP kernels; there
is no fallback of any kind — importing this package fails if the library has
not been built (``python llama_decoder_block_amd/build.py``).

The functions mirror the C ABI in include/llama_layer.h:

    handle = llama_layer_create(config, weights)
    llama_layer_prefill(handle, x, y, positions, B, T, k_cache, v_cache)
    llama_layer_decode(handle, x, y, positions, B, k_cache, v_cache)
    llama_layer_destroy(handle)

``LlamaLayer`` wraps a handle with the same calls.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libllama_layer.so")

LLAMA_OK = 0
LLAMA_ERR_NULL = -1
LLAMA_ERR_INVALID = -2
LLAMA_ERR_UNSUPPORTED = -3
LLAMA_ERR_CAPACITY = -4
LLAMA_ERR_HIP = -5
LLAMA_ERR_ALLOC = -6
LLAMA_F32 = 0
LLAMA_BF16 = 1

EXPORTED = ("llama_layer_create", "llama_layer_prefill", "llama_layer_decode", "llama_layer_decode_noalloc",
            "llama_layer_prefill_paged", "llama_layer_decode_paged",
            "llama_layer_kv_quantize", "llama_layer_prefill_int8", "llama_layer_decode_int8",
            "llama_layer_prefill_paged_int8", "llama_layer_decode_paged_int8",
            "llama_layer_destroy", "llama_layer_strerror", "llama_layer_last_error",
            "llama_layer_profile", "llama_layer_profile_read", "llama_layer_step_name",
            "llama_layer_ceiling_mfma", "llama_layer_ceiling_read")
EXPORTED_MODEL = ("llama_model_create", "llama_model_destroy", "llama_model_prefill",
                  "llama_model_decode", "llama_model_generate", "llama_sample")
LLAMA_LAYER_STEPS = 7


class LlamaLayerConfig(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_base", ctypes.c_float), ("max_pos", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("bidirectional", ctypes.c_int32)]


WEIGHT_NAMES = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


class LlamaLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_NAMES]


class LlamaModelConfig(ctypes.Structure):
    _fields_ = [("layer", LlamaLayerConfig), ("n_layers", ctypes.c_int32), ("vocab", ctypes.c_int32)]


class LlamaModelWeights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("layers", ctypes.POINTER(LlamaLayerWeights))]


class LlamaSampling(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_p", ctypes.c_float),
                ("repetition_penalty", ctypes.c_float), ("eos_id", ctypes.c_int32)]


class LlamaLayerError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python llama_decoder_block_amd/build.py` (hipcc, gfx950)")
    # torch first: the library then binds to the HIP runtime torch loaded
    # (one runtime per process, so torch streams and memory are valid here)
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.llama_layer_create.argtypes = [ctypes.POINTER(LlamaLayerConfig),
                                       ctypes.POINTER(LlamaLayerWeights), vp, ctypes.POINTER(vp)]
    lib.llama_layer_create.restype = ctypes.c_int
    lib.llama_layer_prefill.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp]
    lib.llama_layer_prefill.restype = ctypes.c_int
    lib.llama_layer_decode.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp]
    lib.llama_layer_decode.restype = ctypes.c_int
    lib.llama_layer_prefill_paged.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp, i32, i32, i32, vp]
    lib.llama_layer_prefill_paged.restype = ctypes.c_int
    lib.llama_layer_decode_paged.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, vp]
    lib.llama_layer_decode_paged.restype = ctypes.c_int
    lib.llama_layer_decode_noalloc.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp]
    lib.llama_layer_decode_noalloc.restype = ctypes.c_int
    lib.llama_layer_kv_quantize.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp, vp, vp]
    lib.llama_layer_kv_quantize.restype = ctypes.c_int
    lib.llama_layer_prefill_int8.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp]
    lib.llama_layer_prefill_int8.restype = ctypes.c_int
    lib.llama_layer_decode_int8.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, vp, vp]
    lib.llama_layer_prefill_paged_int8.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, i32, i32, i32, vp]
    lib.llama_layer_prefill_paged_int8.restype = ctypes.c_int
    lib.llama_layer_decode_paged_int8.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, i32, i32, i32, vp]
    lib.llama_layer_decode_paged_int8.restype = ctypes.c_int
    lib.llama_layer_decode_int8.restype = ctypes.c_int
    lib.llama_layer_destroy.argtypes = [vp]
    lib.llama_layer_destroy.restype = None
    lib.llama_layer_strerror.argtypes = [ctypes.c_int]
    lib.llama_layer_strerror.restype = ctypes.c_char_p
    lib.llama_layer_last_error.argtypes = []
    lib.llama_layer_last_error.restype = ctypes.c_char_p
    lib.llama_layer_profile.argtypes = [vp, ctypes.c_int]
    lib.llama_layer_profile.restype = ctypes.c_int
    lib.llama_layer_profile_read.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.c_int,
                                             ctypes.POINTER(ctypes.c_longlong)]
    lib.llama_layer_profile_read.restype = ctypes.c_int
    lib.llama_layer_step_name.argtypes = [ctypes.c_int]
    lib.llama_layer_step_name.restype = ctypes.c_char_p
    lib.llama_layer_ceiling_mfma.argtypes = [i32, vp, ctypes.POINTER(ctypes.c_double), vp]
    lib.llama_layer_ceiling_mfma.restype = ctypes.c_int
    lib.llama_layer_ceiling_read.argtypes = [vp, ctypes.c_uint64, vp, vp]
    lib.llama_layer_ceiling_read.restype = ctypes.c_int
    pp = ctypes.POINTER(vp)
    lib.llama_model_create.argtypes = [ctypes.POINTER(LlamaModelConfig), ctypes.POINTER(LlamaModelWeights),
                                       vp, ctypes.POINTER(vp)]
    lib.llama_model_create.restype = ctypes.c_int
    lib.llama_model_destroy.argtypes = [vp]
    lib.llama_model_destroy.restype = None
    lib.llama_model_prefill.argtypes = [vp, vp, i32, i32, pp, pp, vp, vp]
    lib.llama_model_prefill.restype = ctypes.c_int
    lib.llama_model_decode.argtypes = [vp, vp, vp, i32, pp, pp, vp, vp]
    lib.llama_model_decode.restype = ctypes.c_int
    lib.llama_sample.argtypes = [vp, i32, i32, i32, ctypes.POINTER(LlamaSampling), vp, vp, i32, vp, vp, vp]
    lib.llama_sample.restype = ctypes.c_int
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.llama_model_generate.argtypes = [vp, ip, i32, i32, i32, ctypes.POINTER(LlamaSampling),
                                         ctypes.POINTER(ctypes.c_float), pp, pp, ip, ip, vp]
    lib.llama_model_generate.restype = ctypes.c_int
    return lib


LIB = _load()


def _check(status: int):
    if status != LLAMA_OK:
        detail = LIB.llama_layer_last_error().decode(errors="replace")
        raise LlamaLayerError(status, f"{LIB.llama_layer_strerror(status).decode()}: {detail}")


def _stream_ptr(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t, name, dtype=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    return ctypes.c_void_p(t.data_ptr())


def make_config(d_model, n_heads, n_kv_heads, head_dim, d_ff, max_pos, max_tokens, dtype,
                rms_eps=1e-6, rope_base=10000.0, bidirectional=False) -> LlamaLayerConfig:
    return LlamaLayerConfig(int(d_model), int(n_heads), int(n_kv_heads), int(head_dim), int(d_ff),
                            float(rms_eps), float(rope_base), int(max_pos), int(max_tokens),
                            LLAMA_BF16 if dtype in ("bf16", LLAMA_BF16) else LLAMA_F32,
                            1 if bidirectional else 0)


def llama_layer_create(config: LlamaLayerConfig, weights: dict, stream=None) -> ctypes.c_void_p:
    import torch
    dt = torch.bfloat16 if config.dtype == LLAMA_BF16 else torch.float32
    w = LlamaLayerWeights(*[_ptr(weights[n], n, dt) for n in WEIGHT_NAMES])
    handle = ctypes.c_void_p()
    _check(LIB.llama_layer_create(ctypes.byref(config), ctypes.byref(w), _stream_ptr(stream),
                                  ctypes.byref(handle)))
    return handle


def llama_layer_prefill(handle, x, y, positions, B, T, k_cache, v_cache, stream=None):
    import torch
    _check(LIB.llama_layer_prefill(handle, _ptr(x, "x"), _ptr(y, "y"),
                                   _ptr(positions, "positions", torch.int32), int(B), int(T),
                                   _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache"),
                                   _stream_ptr(stream)))


def llama_layer_decode(handle, x, y, positions, B, k_cache, v_cache, stream=None):
    import torch
    _check(LIB.llama_layer_decode(handle, _ptr(x, "x"), _ptr(y, "y"),
                                  _ptr(positions, "positions", torch.int32), int(B),
                                  _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache"),
                                  _stream_ptr(stream)))


def llama_layer_prefill_paged(handle, x, y, positions, B, T, k_pages, v_pages, block_table, page_size,
                              stream=None):
    """Prefill over page pools [n_pages, Hkv, page_size, dh]; block_table
    [B, blocks_per_seq] int32 on the device."""
    import torch
    _check(LIB.llama_layer_prefill_paged(handle, _ptr(x, "x"), _ptr(y, "y"),
                                         _ptr(positions, "positions", torch.int32), int(B), int(T),
                                         _ptr(k_pages, "k_pages"), _ptr(v_pages, "v_pages"),
                                         _ptr(block_table, "block_table", torch.int32),
                                         int(block_table.shape[-1]), int(page_size), int(k_pages.shape[0]),
                                         _stream_ptr(stream)))


def llama_layer_decode_paged(handle, x, y, positions, B, k_pages, v_pages, block_table, page_size, stream=None):
    import torch
    _check(LIB.llama_layer_decode_paged(handle, _ptr(x, "x"), _ptr(y, "y"),
                                        _ptr(positions, "positions", torch.int32), int(B),
                                        _ptr(k_pages, "k_pages"), _ptr(v_pages, "v_pages"),
                                        _ptr(block_table, "block_table", torch.int32),
                                        int(block_table.shape[-1]), int(page_size), int(k_pages.shape[0]),
                                        _stream_ptr(stream)))


def llama_layer_decode_noalloc(handle, x, y, positions, B, k_cache, v_cache, stream=None):
    import torch
    _check(LIB.llama_layer_decode_noalloc(handle, _ptr(x, "x"), _ptr(y, "y"),
                                          _ptr(positions, "positions", torch.int32), int(B),
                                          _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache"),
                                          _stream_ptr(stream)))


def llama_layer_kv_quantize(handle, k_cache, v_cache, B, n_slots, k_codes, v_codes, k_scale, v_scale,
                            stream=None):
    """Slots [0, n_slots) of the bf16 caches [B, Hkv, max_pos, 128] -> int8
    codes [B, Hkv, max_pos, 128] and float32 scales [B, Hkv, max_pos]."""
    import torch
    _check(LIB.llama_layer_kv_quantize(handle, _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache"), int(B),
                                       int(n_slots), _ptr(k_codes, "k_codes", torch.int8),
                                       _ptr(v_codes, "v_codes", torch.int8), _ptr(k_scale, "k_scale", torch.float32),
                                       _ptr(v_scale, "v_scale", torch.float32), _stream_ptr(stream)))


def llama_layer_prefill_int8(handle, x, y, positions, B, T, k_codes, v_codes, k_scale, v_scale, stream=None):
    import torch
    _check(LIB.llama_layer_prefill_int8(handle, _ptr(x, "x"), _ptr(y, "y"),
                                        _ptr(positions, "positions", torch.int32), int(B), int(T),
                                        _ptr(k_codes, "k_codes", torch.int8), _ptr(v_codes, "v_codes", torch.int8),
                                        _ptr(k_scale, "k_scale", torch.float32),
                                        _ptr(v_scale, "v_scale", torch.float32), _stream_ptr(stream)))


def llama_layer_prefill_paged_int8(handle, x, y, positions, B, T, k_pages, v_pages, k_scale_pages, v_scale_pages,
                                   block_table, page_size, stream=None):
    """Prefill over int8 page pools: codes [n_pages, Hkv, page_size, 128] int8,
    scales [n_pages, Hkv, page_size] float32; block_table [B, blocks_per_seq]."""
    import torch
    _check(LIB.llama_layer_prefill_paged_int8(
        handle, _ptr(x, "x"), _ptr(y, "y"), _ptr(positions, "positions", torch.int32), int(B), int(T),
        _ptr(k_pages, "k_pages", torch.int8), _ptr(v_pages, "v_pages", torch.int8),
        _ptr(k_scale_pages, "k_scale_pages", torch.float32), _ptr(v_scale_pages, "v_scale_pages", torch.float32),
        _ptr(block_table, "block_table", torch.int32), int(block_table.shape[-1]), int(page_size),
        int(k_pages.shape[0]), _stream_ptr(stream)))


def llama_layer_decode_paged_int8(handle, x, y, positions, B, k_pages, v_pages, k_scale_pages, v_scale_pages,
                                  block_table, page_size, stream=None):
    import torch
    _check(LIB.llama_layer_decode_paged_int8(
        handle, _ptr(x, "x"), _ptr(y, "y"), _ptr(positions, "positions", torch.int32), int(B),
        _ptr(k_pages, "k_pages", torch.int8), _ptr(v_pages, "v_pages", torch.int8),
        _ptr(k_scale_pages, "k_scale_pages", torch.float32), _ptr(v_scale_pages, "v_scale_pages", torch.float32),
        _ptr(block_table, "block_table", torch.int32), int(block_table.shape[-1]), int(page_size),
        int(k_pages.shape[0]), _stream_ptr(stream)))


def llama_layer_decode_int8(handle, x, y, positions, B, k_codes, v_codes, k_scale, v_scale, stream=None):
    import torch
    _check(LIB.llama_layer_decode_int8(handle, _ptr(x, "x"), _ptr(y, "y"),
                                       _ptr(positions, "positions", torch.int32), int(B),
                                       _ptr(k_codes, "k_codes", torch.int8), _ptr(v_codes, "v_codes", torch.int8),
                                       _ptr(k_scale, "k_scale", torch.float32),
                                       _ptr(v_scale, "v_scale", torch.float32), _stream_ptr(stream)))


def llama_layer_destroy(handle):
    LIB.llama_layer_destroy(handle)


def llama_layer_profile(handle, enable: bool, step: int | None = None):
    """Per-step HIP event timing of later calls: every step, or only `step`
    (0 .. LLAMA_LAYER_STEPS - 1, two events per call); enable=False stops it."""
    mode = 0 if not enable else (1 if step is None else 2 + int(step))
    _check(LIB.llama_layer_profile(handle, mode))


def llama_layer_profile_read(handle):
    """{step name: total ms} over the calls recorded since profiling was
    enabled, and the number of those calls."""
    arr = (ctypes.c_double * LLAMA_LAYER_STEPS)()
    calls = ctypes.c_longlong()
    _check(LIB.llama_layer_profile_read(handle, arr, LLAMA_LAYER_STEPS, ctypes.byref(calls)))
    names = [LIB.llama_layer_step_name(i).decode() for i in range(LLAMA_LAYER_STEPS)]
    return dict(zip(names, list(arr))), int(calls.value)


def llama_layer_ceiling_mfma(n_iter: int, sink, stream=None) -> float:
    """Launch the MFMA-loop ceiling kernel on `stream` (default: torch's
    current stream); returns the flops it issues.  sink: a device tensor of at
    least 4 bytes, kept alive until the kernel has run."""
    flops = ctypes.c_double()
    _check(LIB.llama_layer_ceiling_mfma(int(n_iter), sink.data_ptr(), ctypes.byref(flops), _stream_ptr(stream)))
    return flops.value


def llama_layer_ceiling_read(buf, sink, stream=None):
    """Launch the streaming-read ceiling kernel over the device tensor `buf`
    (all of its bytes) on `stream`."""
    _check(LIB.llama_layer_ceiling_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                                        _stream_ptr(stream)))


class LlamaLayer:
    """One decoder layer bound to its weights (copied at construction)."""

    def __init__(self, config: LlamaLayerConfig, weights: dict, stream=None):
        self.config = config
        self.handle = llama_layer_create(config, weights, stream)

    def prefill(self, x, positions, k_cache, v_cache, y=None, stream=None):
        """x [B, T, d] -> y [B, T, d]; positions [B, T] int32; caches updated in place."""
        import torch
        B, T = int(x.shape[0]), int(x.shape[1])
        y = torch.empty_like(x) if y is None else y
        llama_layer_prefill(self.handle, x, y, positions, B, T, k_cache, v_cache, stream)
        return y

    def decode(self, x, positions, k_cache, v_cache, y=None, stream=None):
        """x [B, d] -> y [B, d]; positions [B] int32 (each sequence's cache length)."""
        import torch
        y = torch.empty_like(x) if y is None else y
        llama_layer_decode(self.handle, x, y, positions, int(x.shape[0]), k_cache, v_cache, stream)
        return y

    def kv_quantize(self, k_cache, v_cache, n_slots, k_codes, v_codes, k_scale, v_scale, stream=None):
        """Quantize slots [0, n_slots) of the bf16 caches into the int8 cache (codes, scales)."""
        llama_layer_kv_quantize(self.handle, k_cache, v_cache, int(k_cache.shape[0]), n_slots, k_codes, v_codes,
                                k_scale, v_scale, stream)

    def prefill_int8(self, x, positions, k_codes, v_codes, k_scale, v_scale, y=None, stream=None):
        """As prefill, over the int8 cache (codes and scales updated in place)."""
        import torch
        B, T = int(x.shape[0]), int(x.shape[1])
        y = torch.empty_like(x) if y is None else y
        llama_layer_prefill_int8(self.handle, x, y, positions, B, T, k_codes, v_codes, k_scale, v_scale, stream)
        return y

    def decode_int8(self, x, positions, k_codes, v_codes, k_scale, v_scale, y=None, stream=None):
        """As decode, over the int8 cache: codes [B, Hkv, max_pos, 128] int8,
        scales [B, Hkv, max_pos] float32, updated in place."""
        import torch
        y = torch.empty_like(x) if y is None else y
        llama_layer_decode_int8(self.handle, x, y, positions, int(x.shape[0]), k_codes, v_codes, k_scale, v_scale,
                                stream)
        return y

    def prefill_paged(self, x, positions, k_pages, v_pages, block_table, y=None, stream=None):
        """x [B, T, d]; pools [n_pages, Hkv, page, dh] (page size read from
        their shape); block_table [B, blocks_per_seq] int32."""
        import torch
        B, T = int(x.shape[0]), int(x.shape[1])
        y = torch.empty_like(x) if y is None else y
        llama_layer_prefill_paged(self.handle, x, y, positions, B, T, k_pages, v_pages, block_table,
                                  int(k_pages.shape[2]), stream)
        return y

    def decode_paged(self, x, positions, k_pages, v_pages, block_table, y=None, stream=None):
        import torch
        y = torch.empty_like(x) if y is None else y
        llama_layer_decode_paged(self.handle, x, y, positions, int(x.shape[0]), k_pages, v_pages, block_table,
                                 int(k_pages.shape[2]), stream)
        return y

    def prefill_paged_int8(self, x, positions, k_pages, v_pages, k_scale_pages, v_scale_pages, block_table, y=None,
                           stream=None):
        """As prefill_paged, over int8 pools (codes [n_pages, Hkv, page, 128]
        int8, scales [n_pages, Hkv, page] float32), updated in place."""
        import torch
        B, T = int(x.shape[0]), int(x.shape[1])
        y = torch.empty_like(x) if y is None else y
        llama_layer_prefill_paged_int8(self.handle, x, y, positions, B, T, k_pages, v_pages, k_scale_pages,
                                       v_scale_pages, block_table, int(k_pages.shape[2]), stream)
        return y

    def decode_paged_int8(self, x, positions, k_pages, v_pages, k_scale_pages, v_scale_pages, block_table, y=None,
                          stream=None):
        import torch
        y = torch.empty_like(x) if y is None else y
        llama_layer_decode_paged_int8(self.handle, x, y, positions, int(x.shape[0]), k_pages, v_pages,
                                      k_scale_pages, v_scale_pages, block_table, int(k_pages.shape[2]), stream)
        return y

    def decode_noalloc(self, x, positions, k_cache, v_cache, y, stream=None):
        """The allocation-free decode: y must be given (nothing is allocated)."""
        llama_layer_decode_noalloc(self.handle, x, y, positions, int(x.shape[0]), k_cache, v_cache, stream)
        return y

    def close(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            llama_layer_destroy(h)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------- generation stack

def make_sampling(temperature=0.0, top_p=1.0, repetition_penalty=1.0, eos_id=-1) -> LlamaSampling:
    return LlamaSampling(float(temperature), float(top_p), float(repetition_penalty), int(eos_id))


def _ptr_array(tensors, name):
    arr = (ctypes.c_void_p * len(tensors))()
    for i, t in enumerate(tensors):
        arr[i] = _ptr(t, f"{name}[{i}]").value
    return arr


def llama_sample(logits, params: LlamaSampling, history=None, history_len=None, uniforms=None, out=None,
                 stream=None):
    """One token per row of logits [B, V] (fp32); history [B, H] int32 with
    history_len [B] (for the repetition penalty), uniforms [B] fp32 (for
    temperature > 0).  Returns the int32 ids [B]."""
    import torch
    B, V = int(logits.shape[0]), int(logits.shape[1])
    out = torch.empty(B, dtype=torch.int32, device=logits.device) if out is None else out
    opt = lambda t, n, dt: None if t is None else _ptr(t, n, dt)  # noqa: E731
    _check(LIB.llama_sample(_ptr(logits, "logits", torch.float32), B, V, V, ctypes.byref(params),
                            opt(history, "history", torch.int32), opt(history_len, "history_len", torch.int32),
                            0 if history is None else int(history.shape[1]),
                            opt(uniforms, "uniforms", torch.float32), _ptr(out, "out", torch.int32),
                            _stream_ptr(stream)))
    return out


class LlamaModel:
    """Embedding, n_layers decoder layers, final RMSNorm and LM head (weights
    copied at construction), with prefill / decode logits and a native
    generation loop."""

    def __init__(self, layer_config: LlamaLayerConfig, n_layers: int, vocab: int, embed, final_norm,
                 lm_head, layer_weights: list, stream=None):
        import torch
        dt = torch.bfloat16 if layer_config.dtype == LLAMA_BF16 else torch.float32
        self.config = LlamaModelConfig(layer_config, int(n_layers), int(vocab))
        lw = (LlamaLayerWeights * len(layer_weights))(
            *[LlamaLayerWeights(*[_ptr(w[n], n, dt) for n in WEIGHT_NAMES]) for w in layer_weights])
        mw = LlamaModelWeights(_ptr(embed, "embed", dt), _ptr(final_norm, "final_norm", dt),
                               _ptr(lm_head, "lm_head", dt), lw)
        self.handle = ctypes.c_void_p()
        _check(LIB.llama_model_create(ctypes.byref(self.config), ctypes.byref(mw), _stream_ptr(stream),
                                      ctypes.byref(self.handle)))
        self.vocab = int(vocab)

    def prefill(self, ids, k_caches, v_caches, logits=None, stream=None):
        """ids [B, T] int32 (positions 0..T-1) -> the last position's logits [B, V] fp32."""
        import torch
        B, T = int(ids.shape[0]), int(ids.shape[1])
        logits = torch.empty(B, self.vocab, dtype=torch.float32, device=ids.device) if logits is None else logits
        _check(LIB.llama_model_prefill(self.handle, _ptr(ids, "ids", torch.int32), B, T,
                                       _ptr_array(k_caches, "k_caches"), _ptr_array(v_caches, "v_caches"),
                                       _ptr(logits, "logits", torch.float32), _stream_ptr(stream)))
        return logits

    def decode(self, ids, positions, k_caches, v_caches, logits=None, stream=None):
        """ids [B] int32 at positions [B] -> logits [B, V] fp32."""
        import torch
        B = int(ids.shape[0])
        logits = torch.empty(B, self.vocab, dtype=torch.float32, device=ids.device) if logits is None else logits
        _check(LIB.llama_model_decode(self.handle, _ptr(ids, "ids", torch.int32),
                                      _ptr(positions, "positions", torch.int32), B,
                                      _ptr_array(k_caches, "k_caches"), _ptr_array(v_caches, "v_caches"),
                                      _ptr(logits, "logits", torch.float32), _stream_ptr(stream)))
        return logits

    def generate(self, prompt, max_new: int, params: LlamaSampling, k_caches, v_caches, uniforms=None,
                 stream=None):
        """prompt: host int sequence [B][T]; uniforms: host [max_new][B] floats or
        None (greedy).  Returns the generated id lists (EOS not included)."""
        import numpy as np
        p = np.ascontiguousarray(np.asarray(prompt, dtype=np.int32))
        B, T = p.shape
        out = np.zeros((B, max_new), dtype=np.int32)
        n = np.zeros(B, dtype=np.int32)
        ip = ctypes.POINTER(ctypes.c_int32)
        u = None
        if uniforms is not None:
            u = np.ascontiguousarray(np.asarray(uniforms, dtype=np.float32).reshape(max_new, B))
        _check(LIB.llama_model_generate(
            self.handle, p.ctypes.data_as(ip), B, T, int(max_new), ctypes.byref(params),
            None if u is None else u.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
            _ptr_array(k_caches, "k_caches"), _ptr_array(v_caches, "v_caches"),
            out.ctypes.data_as(ip), n.ctypes.data_as(ip), _stream_ptr(stream)))
        return [out[b, :n[b]].tolist() for b in range(B)]

    def close(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            LIB.llama_model_destroy(h)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
