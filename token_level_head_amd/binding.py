"""Thin ctypes binding over libmhla.so (the C ABI in include/mhla.h).

Argument marshalling only: every function here forwards device pointers, sizes
and the current HIP stream to the C entry point of the same name, and turns a
non-zero status into :class:`MhlaError`.  All arithmetic runs in the library's
HIP kernels.  There is no fallback: if the library is not built, or no GPU is
present, the calls raise.
"""
import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
# MHLA_LIBRARY names another build of the same library (the sanitizer test loads an
# instrumented one); the default is the in-tree build.
LIB_PATH = os.environ.get("MHLA_LIBRARY") or os.path.join(PKG, "libmhla.so")

MHLA_OK = 0
MHLA_ERR_INVALID_ARG = -1
MHLA_ERR_UNSUPPORTED = -2
MHLA_ERR_NO_MEMORY = -3
MHLA_ERR_HIP = -4
MHLA_DTYPE_BF16 = 0
MHLA_DTYPE_F32 = 1
MHLA_PATH_STAGED = 0
MHLA_PATH_FUSED = 1
MHLA_PATH_PAIR = 2
MHLA_OPT_CAUSAL = 1
MHLA_OPT_NO_NORMALIZER = 2
MHLA_OPT_OUT_BF16 = 4
MHLA_OPT_W_PER_HEAD = 8
MHLA_NOALLOC_SCRATCH_BYTES = 256 << 20

# Every symbol include/mhla.h declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
SIGNATURES = {
    "mhla_forward": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I, _P]),
    "mhla_forward_f32": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I, _P]),
    "mhla_forward_noalloc": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I, _P]),
    "mhla_forward_ex": (_I, [_P, _P, _P, _I, _P, _P, _I64, _I64, _I64, _I64, _I64, ctypes.c_uint, _P]),
    "mhla_forward_blocks": (_I, [_P, _P, _P, _I, _P, _P, _I64, _I64, _I64, _I64, _I64, _P, _P, _I64, ctypes.c_uint,
                                 _P]),
    "mhla_workspace_bytes": (_I64, [_I64, _I64, _I64, _I64, _I64, _I]),
    "mhla_forward_path": (_I, [_I64, _I64, _I64, _I64, _I64, _I, _I]),
    "mhla_summary_floats": (_I64, [_I64]),
    "mhla_block_summaries": (_I, [_P, _P, _I, _P, _I64, _I64, _I64, _I64, _I64, _P]),
    "mhla_mix_summaries": (_I, [_P, _P, _P, _I64, _I64, _I64, _I, _I, _P]),
    "mhla_output": (_I, [_P, _P, _P, _I, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I, _P]),
    "mhla_unpack_summaries": (_I, [_P, _I64, _I64, _P, _P]),
    "mhla_decode_state_bytes": (_I64, [_I64, _I64, _I64, _I64]),
    "mhla_backward_workspace_bytes": (_I64, [_I64, _I64, _I64, _I64, _I64, _I]),
    "mhla_backward": (_I, [_P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I, _P]),
    "mhla_decode_step": (_I, [_P, _P, _P, _I, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _P]),
    "mhla_backward_ex": (_I, [_P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, ctypes.c_uint,
                              _P]),
    "mhla_decode_step_ex": (_I, [_P, _P, _P, _I, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, ctypes.c_uint,
                                 _P]),
    "mhla_release_workspace": (_I, [_P]),
    "mhla_debug_fail_workspace": (None, [_I]),
    "mhla_status_string": (ctypes.c_char_p, [_I]),
    "mhla_last_error": (ctypes.c_char_p, []),
    "mhla_version": (ctypes.c_char_p, []),
}


class MhlaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def load_library(path=LIB_PATH):
    """Load libmhla.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built: run `python -m token_level_head_amd.build` "
                               "(or __graft_entry__.build()) first")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status):
    if status != MHLA_OK:
        lib = load_library()
        raise MhlaError(status, f"{lib.mhla_status_string(status).decode()}: {lib.mhla_last_error().decode()}")


# ---- argument checks -------------------------------------------------------------
# The library sees raw addresses only, so the binding checks what an address cannot
# carry: element type, shape, density and device.  Everything is checked before the
# library is loaded or called; shapes and dtypes come first, then layout, then device.

def _tensor(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    return t


def _dtype(t, name, *allowed):
    if _tensor(t, name).dtype not in allowed:
        names = " or ".join(str(a).replace("torch.", "") for a in allowed)
        raise TypeError(f"{name} must be {names}, got {str(t.dtype).replace('torch.', '')}")


def _shape(t, name, shape):
    if tuple(_tensor(t, name).shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _numel(t, name, count):
    if _tensor(t, name).numel() < count:
        raise ValueError(f"{name} must hold at least {count} elements, got {t.numel()}")


def _device_of(**named):
    """Every given tensor is contiguous and on one GPU; returns that device."""
    tensors = [(n, t) for n, t in named.items() if t is not None]
    for n, t in tensors:
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous (dense row-major); got strides {tuple(t.stride())}")
    dev = None
    for n, t in tensors:
        if t.device.type != "cuda":
            raise ValueError(f"{n} must be on a GPU, got device {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{n} is on {t.device}, but the other tensors are on {dev}")
    return dev


def _same(ref, ref_name, **named):
    """The named tensors have ref's dtype and shape."""
    for n, t in named.items():
        _dtype(t, n, ref.dtype)
        _shape(t, n, ref.shape)


def _tokens(q, name="q", dims=4):
    _dtype(q, name, torch.bfloat16, torch.float32)
    if q.dim() != dims:
        lay = "[B, H, N, d]" if dims == 4 else "[B, H, d]"
        raise ValueError(f"{name} must be {lay}, got shape {tuple(q.shape)}")


def _mixing(W, H=None):
    """W is float32 [M, M] (or [H, M, M] when H is given and W has three dims); returns M."""
    _dtype(W, "W", torch.float32)
    if W.dim() == 2 or (H is not None and W.dim() == 3):
        M = W.shape[-1]
        want = (M, M) if W.dim() == 2 else (H, M, M)
        _shape(W, "W", want)
        return M
    raise ValueError(f"W must be [M, M]{' or [H, M, M]' if H is not None else ''}, got shape {tuple(W.shape)}")


def _launch(dev, stream):
    """(device context, stream handle) for a call whose tensors live on `dev`."""
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    elif stream.device != dev:
        raise ValueError(f"stream is on {stream.device}, but the tensors are on {dev}")
    return torch.cuda.device(dev), ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return MHLA_DTYPE_BF16
    if t.dtype == torch.float32:
        return MHLA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def mhla_forward(q, k, v, W, out, causal=False, stream=None):
    """bf16 q, k, v [B, H, N, d]; float32 W [M, M] and out [B, H, N, d]."""
    _dtype(q, "q", torch.bfloat16)
    _tokens(q)
    _same(q, "q", k=k, v=v)
    M = _mixing(W)
    _dtype(out, "out", torch.float32)
    _shape(out, "out", q.shape)
    ctx, s = _launch(_device_of(q=q, k=k, v=v, W=W, out=out), stream)
    B, H, N, d = q.shape
    with ctx:
        _check(load_library().mhla_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(W), _ptr(out), B, H, N, d, M,
                                           int(bool(causal)), s))
    return out


def mhla_forward_noalloc(q, k, v, W, out, causal=False, stream=None):
    """mhla_forward with its workspace in the library's fixed per-device scratch array
    (no allocation; workspaces above MHLA_NOALLOC_SCRATCH_BYTES are refused; calls that
    overlap on one device race)."""
    _dtype(q, "q", torch.bfloat16)
    _tokens(q)
    _same(q, "q", k=k, v=v)
    M = _mixing(W)
    _dtype(out, "out", torch.float32)
    _shape(out, "out", q.shape)
    ctx, s = _launch(_device_of(q=q, k=k, v=v, W=W, out=out), stream)
    B, H, N, d = q.shape
    with ctx:
        _check(load_library().mhla_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(W), _ptr(out), B, H, N, d, M,
                                                   int(bool(causal)), s))
    return out


def mhla_forward_f32(q, k, v, W, out, causal=False, stream=None):
    """float32 q, k, v [B, H, N, d]; float32 W [M, M] and out."""
    _dtype(q, "q", torch.float32)
    _tokens(q)
    _same(q, "q", k=k, v=v)
    M = _mixing(W)
    _dtype(out, "out", torch.float32)
    _shape(out, "out", q.shape)
    ctx, s = _launch(_device_of(q=q, k=k, v=v, W=W, out=out), stream)
    B, H, N, d = q.shape
    with ctx:
        _check(load_library().mhla_forward_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(W), _ptr(out), B, H, N, d, M,
                                               int(bool(causal)), s))
    return out


def _forward_opts(q, k, v, W, out, normalize):
    """Checks shared by mhla_forward_ex and mhla_forward_blocks; returns (M, option bits)."""
    _tokens(q)
    _same(q, "q", k=k, v=v)
    M = _mixing(W, H=q.shape[1])
    _dtype(out, "out", torch.float32, torch.bfloat16)
    _shape(out, "out", q.shape)
    opts = 0 if normalize else MHLA_OPT_NO_NORMALIZER
    if W.dim() == 3:
        opts |= MHLA_OPT_W_PER_HEAD
    if out.dtype == torch.bfloat16:
        opts |= MHLA_OPT_OUT_BF16
    return M, opts


def mhla_forward_ex(q, k, v, W, out, causal=False, normalize=True, stream=None):
    """q, k, v [B, H, N, d] bf16 or float32; W [M, M] float32, or [H, M, M] for one matrix
    per head; out [B, H, N, d] float32 or bfloat16 (which selects the bf16 output).
    normalize=False drops the normaliser."""
    M, opts = _forward_opts(q, k, v, W, out, normalize)
    opts |= MHLA_OPT_CAUSAL if causal else 0
    ctx, s = _launch(_device_of(q=q, k=k, v=v, W=W, out=out), stream)
    B, H, N, d = q.shape
    with ctx:
        _check(load_library().mhla_forward_ex(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(W), _ptr(out),
                                              B, H, N, d, M, opts, s))
    return out


def mhla_forward_blocks(q, k, v, W, out, order, offsets, max_block, normalize=True, stream=None):
    """Blocks as token lists: order [N] and offsets [M + 1] int32 device tensors (block b =
    order[offsets[b]:offsets[b+1]]), max_block >= the longest block.  W [M, M] or [H, M, M];
    out float32 or bfloat16, as for mhla_forward_ex.  Non-causal."""
    M, opts = _forward_opts(q, k, v, W, out, normalize)
    N = q.shape[2]
    _dtype(order, "order", torch.int32)
    _dtype(offsets, "offsets", torch.int32)
    _shape(order, "order", (N,))
    _shape(offsets, "offsets", (M + 1,))
    ctx, s = _launch(_device_of(q=q, k=k, v=v, W=W, out=out, order=order, offsets=offsets), stream)
    B, H, N, d = q.shape
    with ctx:
        _check(load_library().mhla_forward_blocks(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(W), _ptr(out),
                                                  B, H, N, d, M, _ptr(order), _ptr(offsets), int(max_block), opts,
                                                  s))
    return out


def mhla_workspace_bytes(B, H, N, d, M, causal=False):
    return int(load_library().mhla_workspace_bytes(B, H, N, d, M, int(bool(causal))))


def mhla_forward_path(B, H, N, d, M, causal=False, dtype=MHLA_DTYPE_BF16):
    """MHLA_PATH_STAGED, MHLA_PATH_FUSED or MHLA_PATH_PAIR: the kernels mhla_forward runs for these sizes."""
    return int(load_library().mhla_forward_path(B, H, N, d, M, int(bool(causal)), dtype))


def mhla_summary_floats(d):
    return int(load_library().mhla_summary_floats(d))


def mhla_release_workspace(stream=None):
    """Free the workspace the library keeps for `stream` (default: the current stream),
    in stream order; call it before a stream the library used is destroyed."""
    s = torch.cuda.current_stream() if stream is None else stream
    with torch.cuda.device(s.device):
        _check(load_library().mhla_release_workspace(ctypes.c_void_p(s.cuda_stream)))


def mhla_debug_fail_workspace(count):
    """Test hook: the next `count` calls that need workspace fail with MHLA_ERR_NO_MEMORY."""
    load_library().mhla_debug_fail_workspace(int(count))


def _summary_count(M, BH, d):
    return M * BH * (d * d + d)


def mhla_block_summaries(k, v, S, M, stream=None):
    """Stage 1 into S (float32, M * B*H * (d*d + d) elements, packed layout)."""
    _tokens(k, "k")
    _same(k, "k", v=v)
    B, H, N, d = k.shape
    _dtype(S, "S", torch.float32)
    _numel(S, "S", _summary_count(M, B * H, d))
    ctx, s = _launch(_device_of(k=k, v=v, S=S), stream)
    with ctx:
        _check(load_library().mhla_block_summaries(_ptr(k), _ptr(v), _dtype_code(k), _ptr(S), B, H, N, d, M, s))
    return S


def mhla_mix_summaries(S, W, St, BH, d, causal=False, precise=False, stream=None):
    """Stage 2: St = W-mix of S (both packed, float32)."""
    M = _mixing(W)
    for name, t in (("S", S), ("St", St)):
        _dtype(t, name, torch.float32)
        _numel(t, name, _summary_count(M, BH, d))
    ctx, s = _launch(_device_of(S=S, W=W, St=St), stream)
    with ctx:
        _check(load_library().mhla_mix_summaries(_ptr(S), _ptr(W), _ptr(St), BH, d, M, int(bool(causal)),
                                                 int(bool(precise)), s))
    return St


def mhla_output(q, k, v, St, W, out, causal=False, stream=None):
    """Stage 3 into out (float32 [B, H, N, d]).  k and v are read only when causal (they
    may be None otherwise)."""
    _tokens(q)
    if causal or k is not None or v is not None:
        _same(q, "q", k=k, v=v)
    M = _mixing(W)
    B, H, N, d = q.shape
    _dtype(St, "St", torch.float32)
    _numel(St, "St", _summary_count(M, B * H, d))
    _dtype(out, "out", torch.float32)
    _shape(out, "out", q.shape)
    ctx, s = _launch(_device_of(q=q, k=k, v=v, St=St, W=W, out=out), stream)
    with ctx:
        _check(load_library().mhla_output(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(St), _ptr(W), _ptr(out),
                                          B, H, N, d, M, int(bool(causal)), s))
    return out


def mhla_backward_workspace_bytes(B, H, N, d, M, causal=False):
    return int(load_library().mhla_backward_workspace_bytes(B, H, N, d, M, int(bool(causal))))


def mhla_backward(q, k, v, W, dy, dq, dk, dv, dW, causal=False, stream=None):
    """Gradients of sum(dy * forward(q, k, v, W)): q, k, v [B, H, N, d] bf16 or float32,
    dy and the outputs dq, dk, dv float32 [B, H, N, d], dW float32 [M, M]."""
    return mhla_backward_ex(q, k, v, W, dy, dq, dk, dv, dW, causal=causal, stream=stream)


def mhla_backward_ex(q, k, v, W, dy, dq, dk, dv, dW, causal=False, normalize=True, stream=None):
    """mhla_backward with options: normalize=False differentiates the form without the
    normaliser."""
    _tokens(q)
    _same(q, "q", k=k, v=v)
    M = _mixing(W)
    for name, t in (("dy", dy), ("dq", dq), ("dk", dk), ("dv", dv)):
        _dtype(t, name, torch.float32)
        _shape(t, name, q.shape)
    _dtype(dW, "dW", torch.float32)
    _shape(dW, "dW", (M, M))
    ctx, s = _launch(_device_of(q=q, k=k, v=v, W=W, dy=dy, dq=dq, dk=dk, dv=dv, dW=dW), stream)
    B, H, N, d = q.shape
    with ctx:
        opts = (MHLA_OPT_CAUSAL if causal else 0) | (0 if normalize else MHLA_OPT_NO_NORMALIZER)
        _check(load_library().mhla_backward_ex(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(W), _ptr(dy),
                                               _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dW), B, H, N, d, M, opts, s))
    return dq, dk, dv, dW


def mhla_decode_state_bytes(B, H, d, M):
    return int(load_library().mhla_decode_state_bytes(B, H, d, M))


def mhla_decode_step(q, k, v, W, state, out, C, t, stream=None):
    """One causal decoding step: q, k, v [B, H, d] (token t), out [B, H, d] float32,
    state a float32 device buffer of mhla_decode_state_bytes bytes; blocks of C tokens."""
    return mhla_decode_step_ex(q, k, v, W, state, out, C, t, stream=stream)


def mhla_decode_step_ex(q, k, v, W, state, out, C, t, normalize=True, stream=None):
    """mhla_decode_step with options: normalize=False writes the numerator alone; W may be
    [H, M, M] (one matrix per head)."""
    _tokens(q, dims=3)
    _same(q, "q", k=k, v=v)
    M = _mixing(W, H=q.shape[1])
    B, H, d = q.shape
    _dtype(state, "state", torch.float32)
    _numel(state, "state", ((M + 1) * (d * d + d) + d) * B * H)
    _dtype(out, "out", torch.float32)
    _shape(out, "out", q.shape)
    ctx, s = _launch(_device_of(q=q, k=k, v=v, W=W, state=state, out=out), stream)
    with ctx:
        opts = MHLA_OPT_CAUSAL | (0 if normalize else MHLA_OPT_NO_NORMALIZER)
        opts |= MHLA_OPT_W_PER_HEAD if W.dim() == 3 else 0
        _check(load_library().mhla_decode_step_ex(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(W), _ptr(state),
                                                  _ptr(out), B, H, d, M, C, t, opts, s))
    return out


def mhla_unpack_summaries(packed, d):
    """Host helper: packed float32 CPU tensor [..., d*d + d] -> (S [..., d, d], z [..., d])."""
    _dtype(packed, "packed", torch.float32)
    if packed.device.type != "cpu":
        raise ValueError(f"packed must be a host (CPU) tensor, got device {packed.device}")
    L = d * d + d
    if packed.dim() < 1 or packed.shape[-1] != L:
        raise ValueError(f"packed must be [..., {L}] for d = {d}, got shape {tuple(packed.shape)}")
    packed = packed.contiguous()
    count = packed.numel() // L
    lead = packed.shape[:-1]
    S = torch.empty((count, d, d), dtype=torch.float32)
    z = torch.empty((count, d), dtype=torch.float32)
    _check(load_library().mhla_unpack_summaries(_ptr(packed), count, d, _ptr(S), _ptr(z)))
    return S.reshape(*lead, d, d), z.reshape(*lead, d)


def mhla_status_string(status):
    return load_library().mhla_status_string(status).decode()


def mhla_last_error():
    return load_library().mhla_last_error().decode()


def mhla_version():
    return load_library().mhla_version().decode()
