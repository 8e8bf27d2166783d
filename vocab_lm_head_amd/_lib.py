"""ctypes binding of ``libvplmhead.so`` -- argument marshalling only.

Each function takes torch tensors that already live on the GPU, checks dtypes
and shapes, passes ``data_ptr()`` values and a HIP stream (the ``stream``
argument, else the current stream of the tensors' GPU) to the C entry point of
the same name, and raises ``VPError`` on a non-zero status.

Buffers a wrapper allocates itself (a workspace the caller did not pass, default
outputs) are allocated while that stream is current, so that torch's caching
allocator files them under the stream the kernels use: a temporary workspace
freed on return cannot be handed to other work before those kernels are done.
Every step of the computation runs in the library's HIP kernels; nothing here
computes a result.  If the library has not been built, importing this module
fails loudly -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import functools
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# VP_LMHEAD_LIB selects another build of the same library (e.g. the host-sanitized one)
LIB_PATH = os.environ.get("VP_LMHEAD_LIB") or os.path.join(_HERE, "libvplmhead.so")

VP_OK = 0
VP_ERR_SCRATCH = -7
NOALLOC_SCRATCH_BYTES = 64 << 20   # VP_NOALLOC_SCRATCH_BYTES of the header
DEFAULT_IGNORE_INDEX = -100

# symbol -> (restype, argtypes); the names and order follow include/vp_lmhead.h
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
SIGNATURES = {
    "vp_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "vp_shard_range": (ctypes.c_int, [_I64, _I32, _I32, ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
    "vp_padded_vocab": (ctypes.c_int, [_I64, _I32, _I64, ctypes.POINTER(_I64)]),
    "vp_embed_fwd": (ctypes.c_int, [_P, _I64, _P, _I64, _I64, _I64, _P, _P]),
    "vp_embed_bwd_workspace": (_SZ, [_I64, _I64, _I64, _I64]),
    "vp_embed_bwd": (ctypes.c_int, [_P, _I64, _P, _I64, _I64, _I64, _P, _P, _SZ, _P]),
    "vp_lmhead_ce_fwd_workspace": (_SZ, [_I64, _I64, _I64, _I64]),
    "vp_lmhead_ce_fwd": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _SZ, _P]),
    "vp_lmhead_ce_fwd_noalloc": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, _P, _P, _P, _P]),
    "vp_ce_combine": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I32, _I64, _P, _P, _P, _P]),
    "vp_lmhead_ce_bwd_workspace": (_SZ, [_I64, _I64, _I64, _I64]),
    "vp_lmhead_ce_bwd": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64,
                                        ctypes.c_float, _P, _P, _P, _SZ, _P]),
    "vp_lmhead_logits": (ctypes.c_int, [_P, _P, _I64, _I64, _I64, _I64, _P, _I64, _P]),
    "vp_logits_ce_stats": (ctypes.c_int, [_P, _I64, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "vp_ce_max": (ctypes.c_int, [_P, _I64, _I32, _P, _P]),
    "vp_logits_ce_bwd": (ctypes.c_int, [_P, _I64, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64,
                                        ctypes.c_float, _P, _P, _P, _SZ, _P]),
}


class VPError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first with `python vocab_lm_head_amd/build.py` "
            "(the HIP library is required; there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.vp_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != VP_OK:
        raise VPError(status, where)


def _stream(stream, device) -> int:
    """The given stream, else the current stream of the tensors' device."""
    s = torch.cuda.current_stream(device) if stream is None else stream
    return s.cuda_stream


def _on_stream(fn):
    """Run a wrapper with its ``stream`` argument (when given) as the current stream, so
    that every tensor it allocates belongs to that stream's memory pool."""
    @functools.wraps(fn)
    def call(*args, stream=None, **kwargs):
        if stream is None:
            return fn(*args, **kwargs)
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kwargs)
    return call


def _same_device(*tensors):
    devs = {t.device for t in tensors if t is not None}
    if len(devs) > 1:
        raise ValueError(f"all tensors must be on one GPU, got {sorted(map(str, devs))}")


def _workspace(workspace, need, device):
    """The caller's workspace (the library checks its size), else a new one."""
    if workspace is None:
        return alloc_workspace(need, device)
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return workspace


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _shape(t, shape, name):
    """Caller-provided buffers must have exactly the shape the kernels write or read."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {tuple(shape)}, got {tuple(t.shape)}")


def _need(t, dtype, ndim, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ---------------------------------------------------------------------------
def vp_shard_range(V: int, T: int, t: int):
    a, b = _I64(), _I64()
    _check(lib.vp_shard_range(int(V), int(T), int(t), ctypes.byref(a), ctypes.byref(b)),
           "vp_shard_range")
    return a.value, b.value


def vp_padded_vocab(V: int, T: int, multiple: int = 128) -> int:
    """Smallest V_pad >= V with every one of the T shards a multiple of `multiple` rows."""
    out = _I64()
    _check(lib.vp_padded_vocab(int(V), int(T), int(multiple), ctypes.byref(out)), "vp_padded_vocab")
    return out.value


@_on_stream
def vp_embed_fwd(ids, w_shard, vocab_start: int, vocab_end: int, out=None, stream=None):
    """Masked lookup of one shard: out[i] = w_shard[ids[i]-start] if owned, else 0."""
    _need(ids, torch.int64, 1, "ids")
    _need(w_shard, torch.bfloat16, 2, "w_shard")
    n, h = ids.shape[0], w_shard.shape[1]
    if w_shard.shape[0] != vocab_end - vocab_start:
        raise ValueError("w_shard rows must equal vocab_end - vocab_start")
    if out is None:
        out = torch.empty((n, h), dtype=torch.bfloat16, device=w_shard.device)
    _need(out, torch.bfloat16, 2, "out")
    if tuple(out.shape) != (n, h):
        raise ValueError("out must be [n, h]")
    _same_device(ids, w_shard, out)
    _check(lib.vp_embed_fwd(_ptr(ids), n, _ptr(w_shard), int(vocab_start), int(vocab_end), h,
                            _ptr(out), _stream(stream, out.device)), "vp_embed_fwd")
    return out


def vp_embed_bwd_workspace(n: int, h: int, vocab_start: int, vocab_end: int) -> int:
    return int(lib.vp_embed_bwd_workspace(n, h, vocab_start, vocab_end))


@_on_stream
def vp_embed_bwd(ids, dout, vocab_start: int, vocab_end: int, dw=None, workspace=None, stream=None):
    """Lookup weight gradient of one shard, ADDED to dw (fp32 [Vs, h]; zeros if not given):
    dw[ids[i] - start] += dout[i] for owned ids."""
    _need(ids, torch.int64, 1, "ids")
    _need(dout, torch.bfloat16, 2, "dout")
    n, h = dout.shape
    if ids.shape[0] != n:
        raise ValueError("ids and dout must have the same number of rows")
    vs = vocab_end - vocab_start
    if dw is None:
        dw = torch.zeros((vs, h), dtype=torch.float32, device=dout.device)
    _need(dw, torch.float32, 2, "dw")
    if tuple(dw.shape) != (vs, h):
        raise ValueError("dw must be [vocab_end - vocab_start, h]")
    need = vp_embed_bwd_workspace(n, h, vocab_start, vocab_end)
    workspace = _workspace(workspace, need, dout.device)
    _same_device(ids, dout, dw, workspace)
    _check(lib.vp_embed_bwd(_ptr(ids), n, _ptr(dout), int(vocab_start), int(vocab_end), h,
                            _ptr(dw), _ptr(workspace), workspace.numel() * workspace.element_size(),
                            _stream(stream, dw.device)), "vp_embed_bwd")
    return dw


def vp_lmhead_ce_fwd_workspace(n: int, h: int, vocab_start: int, vocab_end: int) -> int:
    return int(lib.vp_lmhead_ce_fwd_workspace(n, h, vocab_start, vocab_end))


def vp_lmhead_ce_bwd_workspace(n: int, h: int, vocab_start: int, vocab_end: int) -> int:
    return int(lib.vp_lmhead_ce_bwd_workspace(n, h, vocab_start, vocab_end))


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    """A byte tensor for a workspace (torch's allocator returns 256-byte aligned blocks)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


@_on_stream
def vp_lmhead_ce_fwd(hidden, w_shard, targets, vocab_start: int, vocab_end: int,
                     m_local=None, s_local=None, zy_local=None, workspace=None, stream=None):
    """Per-token (local max, local sum-exp, owned target logit) of one shard, fp32 [n] each."""
    _need(hidden, torch.bfloat16, 2, "hidden")
    _need(w_shard, torch.bfloat16, 2, "w_shard")
    _need(targets, torch.int64, 1, "targets")
    n, h = hidden.shape
    if w_shard.shape != (vocab_end - vocab_start, h) or targets.shape[0] != n:
        raise ValueError("shape mismatch between hidden, w_shard, targets and the vocab range")
    dev = hidden.device
    outs = []
    for t in (m_local, s_local, zy_local):
        if t is None:
            t = torch.empty(n, dtype=torch.float32, device=dev)
        _need(t, torch.float32, 1, "statistics output")
        if t.shape[0] != n:
            raise ValueError("statistics outputs must have n elements")
        outs.append(t)
    need = vp_lmhead_ce_fwd_workspace(n, h, vocab_start, vocab_end)
    workspace = _workspace(workspace, need, dev)
    _same_device(hidden, w_shard, targets, *outs, workspace)
    _check(lib.vp_lmhead_ce_fwd(_ptr(hidden), _ptr(w_shard), _ptr(targets), n, h, int(vocab_start),
                                int(vocab_end), _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]),
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream, dev)), "vp_lmhead_ce_fwd")
    return tuple(outs)


@_on_stream
def vp_lmhead_ce_fwd_noalloc(hidden, w_shard, targets, vocab_start: int, vocab_end: int,
                             m_local, s_local, zy_local, stream=None):
    """vp_lmhead_ce_fwd with the library's fixed per-GPU scratch instead of a workspace: the
    caller passes the three fp32 [n] outputs and nothing is allocated."""
    _need(hidden, torch.bfloat16, 2, "hidden")
    _need(w_shard, torch.bfloat16, 2, "w_shard")
    _need(targets, torch.int64, 1, "targets")
    n, h = hidden.shape
    if w_shard.shape != (vocab_end - vocab_start, h) or targets.shape[0] != n:
        raise ValueError("shape mismatch between hidden, w_shard, targets and the vocab range")
    for t in (m_local, s_local, zy_local):
        _need(t, torch.float32, 1, "statistics output")
        _shape(t, (n,), "statistics output")
    _same_device(hidden, w_shard, targets, m_local, s_local, zy_local)
    _check(lib.vp_lmhead_ce_fwd_noalloc(_ptr(hidden), _ptr(w_shard), _ptr(targets), n, h,
                                        int(vocab_start), int(vocab_end), _ptr(m_local),
                                        _ptr(s_local), _ptr(zy_local), _stream(stream, hidden.device)),
           "vp_lmhead_ce_fwd_noalloc")
    return m_local, s_local, zy_local


@_on_stream
def vp_ce_combine(m, s, zy, targets, ignore_index: int = DEFAULT_IGNORE_INDEX,
                  loss=None, lse=None, loss_mean=None, stream=None):
    """Merge [T, n] statistics -> (loss [n], lse [n], loss_mean [1]), fp32."""
    for t, nm in ((m, "m"), (s, "s"), (zy, "zy")):
        _need(t, torch.float32, 2, nm)
    _need(targets, torch.int64, 1, "targets")
    T, n = m.shape
    if s.shape != (T, n) or zy.shape != (T, n) or targets.shape[0] != n:
        raise ValueError("m, s, zy must be [T, n] and targets [n]")
    dev = m.device
    loss = torch.empty(n, dtype=torch.float32, device=dev) if loss is None else loss
    lse = torch.empty(n, dtype=torch.float32, device=dev) if lse is None else lse
    loss_mean = torch.empty(1, dtype=torch.float32, device=dev) if loss_mean is None else loss_mean
    for t, nm, size in ((loss, "loss", n), (lse, "lse", n), (loss_mean, "loss_mean", 1)):
        _need(t, torch.float32, 1, nm)
        if t.shape[0] != size:
            raise ValueError(f"{nm} must have {size} elements")
    _same_device(m, s, zy, targets, loss, lse, loss_mean)
    _check(lib.vp_ce_combine(_ptr(m), _ptr(s), _ptr(zy), _ptr(targets), n, T, int(ignore_index),
                             _ptr(loss), _ptr(lse), _ptr(loss_mean), _stream(stream, dev)),
           "vp_ce_combine")
    return loss, lse, loss_mean


@_on_stream
def vp_lmhead_ce_bwd(hidden, w_shard, targets, lse, vocab_start: int, vocab_end: int,
                     grad_scale: float, ignore_index: int = DEFAULT_IGNORE_INDEX,
                     dx=None, dw=None, workspace=None, stream=None):
    """(dx partial [n, h], dw [Vs, h]) in fp32 for one shard."""
    _need(hidden, torch.bfloat16, 2, "hidden")
    _need(w_shard, torch.bfloat16, 2, "w_shard")
    _need(targets, torch.int64, 1, "targets")
    _need(lse, torch.float32, 1, "lse")
    n, h = hidden.shape
    vs = vocab_end - vocab_start
    if w_shard.shape != (vs, h) or targets.shape[0] != n or lse.shape[0] != n:
        raise ValueError("shape mismatch between hidden, w_shard, targets, lse and the vocab range")
    dev = hidden.device
    dx = torch.empty((n, h), dtype=torch.float32, device=dev) if dx is None else dx
    dw = torch.empty((vs, h), dtype=torch.float32, device=dev) if dw is None else dw
    _need(dx, torch.float32, 2, "dx")
    _need(dw, torch.float32, 2, "dw")
    _shape(dx, (n, h), "dx")
    _shape(dw, (vs, h), "dw")
    need = vp_lmhead_ce_bwd_workspace(n, h, vocab_start, vocab_end)
    workspace = _workspace(workspace, need, dev)
    _same_device(hidden, w_shard, targets, lse, dx, dw, workspace)
    _check(lib.vp_lmhead_ce_bwd(_ptr(hidden), _ptr(w_shard), _ptr(targets), _ptr(lse), n, h,
                                int(vocab_start), int(vocab_end), int(ignore_index),
                                float(grad_scale), _ptr(dx), _ptr(dw), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream, dev)),
           "vp_lmhead_ce_bwd")
    return dx, dw


# ---------------------------------------------------------------------------
# materialised-logits comparator (not the fused path; it measures what that path saves)
def logits_ld(vs: int) -> int:
    """Row stride of stored fp32 logits: Vs rounded up to a multiple of 4."""
    return -(-int(vs) // 4) * 4


@_on_stream
def vp_lmhead_logits(hidden, w_shard, vocab_start: int, vocab_end: int, logits=None, stream=None):
    """fp32 logits [n, ld] of one shard (columns past Vs are zero)."""
    _need(hidden, torch.bfloat16, 2, "hidden")
    _need(w_shard, torch.bfloat16, 2, "w_shard")
    n, h = hidden.shape
    vs = vocab_end - vocab_start
    if w_shard.shape != (vs, h):
        raise ValueError("w_shard must be [vocab_end - vocab_start, h]")
    if logits is None:
        logits = torch.empty((n, logits_ld(vs)), dtype=torch.float32, device=hidden.device)
    _need(logits, torch.float32, 2, "logits")
    if logits.shape[0] != n:
        raise ValueError("logits must have n rows")
    _same_device(hidden, w_shard, logits)
    _check(lib.vp_lmhead_logits(_ptr(hidden), _ptr(w_shard), n, h, int(vocab_start), int(vocab_end),
                                _ptr(logits), logits.shape[1], _stream(stream, logits.device)),
           "vp_lmhead_logits")
    return logits


@_on_stream
def vp_logits_ce_stats(logits, targets, vocab_start: int, vocab_end: int, m_ref=None,
                       m_local=None, s_local=None, zy_local=None, stream=None):
    """(m, s, zy) fp32 [n] of one shard from its stored logits; with m_ref, s is taken
    about m_ref (the pages' second pass)."""
    _need(logits, torch.float32, 2, "logits")
    _need(targets, torch.int64, 1, "targets")
    n = logits.shape[0]
    _shape(targets, (n,), "targets")
    dev = logits.device
    outs = []
    for t in (m_local, s_local, zy_local):
        t = torch.empty(n, dtype=torch.float32, device=dev) if t is None else t
        _need(t, torch.float32, 1, "statistics output")
        _shape(t, (n,), "statistics output")
        outs.append(t)
    if m_ref is not None:
        _need(m_ref, torch.float32, 1, "m_ref")
        _shape(m_ref, (n,), "m_ref")
    _same_device(logits, targets, m_ref, *outs)
    _check(lib.vp_logits_ce_stats(_ptr(logits), logits.shape[1], _ptr(targets), n, int(vocab_start),
                                  int(vocab_end), _ptr(m_ref), _ptr(outs[0]), _ptr(outs[1]),
                                  _ptr(outs[2]), _stream(stream, dev)), "vp_logits_ce_stats")
    return tuple(outs)


@_on_stream
def vp_ce_max(m, out=None, stream=None):
    """Per-token maximum over the T rows of m [T, n]."""
    _need(m, torch.float32, 2, "m")
    T, n = m.shape
    out = torch.empty(n, dtype=torch.float32, device=m.device) if out is None else out
    _need(out, torch.float32, 1, "out")
    _shape(out, (n,), "out")
    _same_device(m, out)
    _check(lib.vp_ce_max(_ptr(m), n, T, _ptr(out), _stream(stream, m.device)), "vp_ce_max")
    return out


@_on_stream
def vp_logits_ce_bwd(logits, hidden, w_shard, targets, lse, vocab_start: int, vocab_end: int,
                     grad_scale: float, ignore_index: int = DEFAULT_IGNORE_INDEX,
                     dx=None, dw=None, workspace=None, stream=None):
    """(dx partial [n, h], dw [Vs, h]) fp32 from the stored logits (no recompute)."""
    _need(logits, torch.float32, 2, "logits")
    _need(hidden, torch.bfloat16, 2, "hidden")
    _need(w_shard, torch.bfloat16, 2, "w_shard")
    _need(targets, torch.int64, 1, "targets")
    _need(lse, torch.float32, 1, "lse")
    n, h = hidden.shape
    vs = vocab_end - vocab_start
    _shape(w_shard, (vs, h), "w_shard")
    _shape(targets, (n,), "targets")
    _shape(lse, (n,), "lse")
    if logits.shape[0] != n:
        raise ValueError("logits must have n rows")
    dev = hidden.device
    dx = torch.empty((n, h), dtype=torch.float32, device=dev) if dx is None else dx
    dw = torch.empty((vs, h), dtype=torch.float32, device=dev) if dw is None else dw
    _need(dx, torch.float32, 2, "dx")
    _need(dw, torch.float32, 2, "dw")
    _shape(dx, (n, h), "dx")
    _shape(dw, (vs, h), "dw")
    need = vp_lmhead_ce_bwd_workspace(n, h, vocab_start, vocab_end)
    workspace = _workspace(workspace, need, dev)
    _same_device(logits, hidden, w_shard, targets, lse, dx, dw, workspace)
    _check(lib.vp_logits_ce_bwd(_ptr(logits), logits.shape[1], _ptr(hidden), _ptr(w_shard),
                                _ptr(targets), _ptr(lse), n, h, int(vocab_start), int(vocab_end),
                                int(ignore_index), float(grad_scale), _ptr(dx), _ptr(dw),
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream, dev)), "vp_logits_ce_bwd")
    return dx, dw
