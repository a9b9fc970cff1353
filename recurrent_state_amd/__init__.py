"""Python binding of the Taylor-truncated causal attention library (gfx950 / MI355X).

Argument marshalling only: every function below forwards to the C entry point of
the same name in ``_lib/libtaylor_attn.so`` (declared in ``include/taylor_attn.h``)
with raw device pointers, sizes read off the tensor shapes, and the current HIP
stream.  All computation runs in the library's HIP kernels; nothing here does
any of the method's arithmetic, and there is no fallback: if the library is
missing the import of the binding functions fails loudly.

PyTorch provides device memory and streams.  torch is imported before the
library is loaded so that the library binds to the HIP runtime torch already
loaded (they share the soname ``libamdhip64.so.7``).
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libtaylor_attn.so")

TAYLOR_OK = 0
TAYLOR_ERR_INVALID_ARG = -1
TAYLOR_ERR_UNSUPPORTED = -2
TAYLOR_ERR_HIP = -3
TAYLOR_F32 = 0
TAYLOR_BF16 = 1
TAYLOR_READOUT_KERNEL = 0
TAYLOR_READOUT_CENTERED = 1

# Every symbol the header declares.
EXPORTS = (
    "taylor_status_string",
    "taylor_feature_width",
    "taylor_state_elems",
    "taylor_state_stride",
    "taylor_monomial_table",
    "taylor_supported",
    "taylor_prefill_chunk",
    "taylor_prefill_workspace_bytes",
    "taylor_state_init",
    "taylor_attn_prefill",
    "taylor_attn_prefill_into",
    "taylor_attn_prefill_into_static",
    "taylor_prefill_varlen_workspace_bytes",
    "taylor_attn_prefill_varlen",
    "taylor_attn_prefill_varlen_into",
    "taylor_prefill_backward_workspace_bytes",
    "taylor_attn_prefill_backward",
    "taylor_attn_decode_step",
)


class TaylorError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {taylor_status_string(status)} ({status})")
        self.status = status


class taylor_config(ctypes.Structure):
    """Mirror of the C struct taylor_config."""

    _fields_ = [
        ("n_terms", ctypes.c_int),
        ("d_k", ctypes.c_int),
        ("d_v", ctypes.c_int),
        ("chunk", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("in_dtype", ctypes.c_int),
        ("readout", ctypes.c_int),
    ]

    def __repr__(self):
        return (f"taylor_config(n_terms={self.n_terms}, d_k={self.d_k}, d_v={self.d_v}, chunk={self.chunk}, "
                f"scale={self.scale}, in_dtype={self.in_dtype}, readout={self.readout})")


def config(n_terms, d_k, d_v, chunk=0, scale=1.0, in_dtype=TAYLOR_F32, readout=TAYLOR_READOUT_KERNEL):
    if not isinstance(in_dtype, int):
        in_dtype = dtype_code(in_dtype)
    return taylor_config(n_terms, d_k, d_v, chunk, scale, in_dtype, readout)


_lib = None


def lib():
    """The loaded library (loaded on first use; raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (loads the HIP runtime the library must share)

    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m recurrent_state_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i, i64, p, f = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    cfgp = ctypes.POINTER(taylor_config)
    sig = {
        "taylor_status_string": (ctypes.c_char_p, [i]),
        "taylor_feature_width": (i, [i, i]),
        "taylor_state_elems": (i64, [cfgp]),
        "taylor_state_stride": (i64, [cfgp]),
        "taylor_monomial_table": (i, [i, i, p, p, ctypes.c_size_t]),
        "taylor_supported": (i, [cfgp]),
        "taylor_prefill_chunk": (i, [cfgp]),
        "taylor_prefill_workspace_bytes": (i64, [cfgp, i, i, i]),
        "taylor_state_init": (i, [p, i, i, cfgp, p]),
        "taylor_attn_prefill": (i, [p, p, p, p, p, p, i, i, i, cfgp, p]),
        "taylor_attn_prefill_into": (i, [p, p, p, p, p, p, p, i, i, i, cfgp, p]),
        "taylor_attn_prefill_into_static": (i, [p, p, p, p, p, p, i, i, i, cfgp, p]),
        "taylor_prefill_varlen_workspace_bytes": (i64, [cfgp, i, i, i, i64]),
        "taylor_attn_prefill_varlen": (i, [p, p, p, p, p, p, p, i, i, i, i64, cfgp, p]),
        "taylor_attn_prefill_varlen_into": (i, [p, p, p, p, p, p, p, p, i, i, i, i64, cfgp, p]),
        "taylor_prefill_backward_workspace_bytes": (i64, [cfgp, i, i, i]),
        "taylor_attn_prefill_backward": (i, [p, p, p, p, p, p, p, p, p, p, p, i, i, i, cfgp, p]),
        "taylor_attn_decode_step": (i, [p, p, p, p, p, i, i, cfgp, p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(rc, what):
    if rc != TAYLOR_OK:
        raise TaylorError(rc, what)
    return rc


def dtype_code(dtype):
    import torch

    if dtype == torch.float32:
        return TAYLOR_F32
    if dtype == torch.bfloat16:
        return TAYLOR_BF16
    raise TypeError(f"unsupported input dtype {dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _torch_dtype(code):
    import torch

    if code == TAYLOR_F32:
        return torch.float32
    if code == TAYLOR_BF16:
        return torch.bfloat16
    raise ValueError(f"cfg.in_dtype {code} is neither TAYLOR_F32 nor TAYLOR_BF16")


class _Args:
    """Checks the tensors of one call against the layout the C entry point assumes, before any pointer
    reaches the library: the ABI takes raw pointers and sizes, so it cannot see a wrong dtype, a
    transposed view or a short buffer itself (a kernel would then read or write past the allocation).
    Each tensor is checked for type, dtype, shape and contiguity as it comes; `done()` then checks
    that every tensor of the call sits on one device (a cuda device)."""

    def __init__(self, what):
        self.what = what
        self.seen = []

    def tensor(self, t, name, shape, dtype, optional=False):
        import torch

        if t is None:
            if optional:
                return None
            raise ValueError(f"{self.what}: {name} is required")
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{self.what}: {name} must be a torch.Tensor, not {type(t).__name__}")
        if t.dtype != dtype:
            raise TypeError(f"{self.what}: {name} has dtype {t.dtype}, expected {dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{self.what}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{self.what}: {name} must be contiguous (dense row-major)")
        self.seen.append((name, t))
        return t

    def rank(self, t, name, dims, last=None):
        """The leading sizes of a tensor whose shape defines the call's sizes (checked for rank and last dim)."""
        import torch

        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{self.what}: {name} must be a torch.Tensor, not {type(t).__name__}")
        if t.dim() != dims or (last is not None and t.shape[-1] != last):
            want = f"{dims}-D" + (f" with last dimension {last}" if last is not None else "")
            raise ValueError(f"{self.what}: {name} has shape {tuple(t.shape)}, expected {want}")
        return tuple(t.shape)

    def workspace(self, t, need):
        import torch

        if need == 0 and t is None:
            return None
        if t is None:
            raise ValueError(f"{self.what}: a workspace of {need} bytes is required")
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{self.what}: workspace must be a torch.Tensor, not {type(t).__name__}")
        if not t.is_contiguous():
            raise ValueError(f"{self.what}: workspace must be contiguous")
        if t.numel() * t.element_size() < need:
            raise ValueError(f"{self.what}: workspace holds {t.numel() * t.element_size()} bytes, needs {need}")
        self.seen.append(("workspace", t))
        return t

    def done(self):
        dev = None
        for name, t in self.seen:
            if t.device.type != "cuda":
                raise ValueError(f"{self.what}: {name} is on {t.device}; the library takes device (cuda) tensors")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"{self.what}: {name} is on {t.device}, other arguments on {dev}")


def _stream(stream, device):
    import torch

    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


# ---- host-only queries --------------------------------------------------------------------------


def taylor_status_string(status):
    return lib().taylor_status_string(int(status)).decode()


def taylor_feature_width(n_terms, d_k):
    return _check_nonneg(lib().taylor_feature_width(n_terms, d_k), "taylor_feature_width")


def _check_nonneg(v, what):
    if v < 0:
        raise TaylorError(int(v), what)
    return int(v)


def taylor_state_elems(cfg):
    return _check_nonneg(lib().taylor_state_elems(ctypes.byref(cfg)), "taylor_state_elems")


def taylor_state_stride(cfg):
    return _check_nonneg(lib().taylor_state_stride(ctypes.byref(cfg)), "taylor_state_stride")


def taylor_monomial_table(n_terms, d_k):
    """(idx int32 [W, max(n-1,1)], coef float64 [W]) exactly as the library exports them."""
    import numpy as np

    W = taylor_feature_width(n_terms, d_k)
    width = max(n_terms - 1, 1)
    idx = np.empty((W, width), dtype=np.int32)
    coef = np.empty(W, dtype=np.float64)
    rc = lib().taylor_monomial_table(n_terms, d_k, idx.ctypes.data, coef.ctypes.data, W)
    _check_nonneg(rc, "taylor_monomial_table")
    return idx, coef


def taylor_supported(cfg):
    return lib().taylor_supported(ctypes.byref(cfg))


def taylor_prefill_chunk(cfg):
    """Tokens per chunk the prefill kernels walk for this config (the matrix-core kernels ignore cfg.chunk)."""
    return _check_nonneg(lib().taylor_prefill_chunk(ctypes.byref(cfg)), "taylor_prefill_chunk")


def taylor_prefill_workspace_bytes(cfg, B, H, N):
    return _check_nonneg(lib().taylor_prefill_workspace_bytes(ctypes.byref(cfg), B, H, N),
                         "taylor_prefill_workspace_bytes")


def taylor_prefill_varlen_workspace_bytes(cfg, n_seqs, H, max_seqlen, total_tokens):
    return _check_nonneg(
        lib().taylor_prefill_varlen_workspace_bytes(ctypes.byref(cfg), n_seqs, H, max_seqlen, total_tokens),
        "taylor_prefill_varlen_workspace_bytes")


def taylor_prefill_backward_workspace_bytes(cfg, B, H, N):
    return _check_nonneg(lib().taylor_prefill_backward_workspace_bytes(ctypes.byref(cfg), B, H, N),
                         "taylor_prefill_backward_workspace_bytes")


# ---- device entry points ------------------------------------------------------------------------


def _check_prefill(what, q, k, v, o, states, workspace, cfg, need_ws=True):
    """Checks an equal-length prefill's tensors; returns (B, H, N).  q may be None only for a
    state-only call (o None)."""
    import torch

    a = _Args(what)
    B, H, N = a.rank(k, "k", 4, cfg.d_k)[:3]
    dt = _torch_dtype(cfg.in_dtype)
    a.tensor(q, "q", (B, H, N, cfg.d_k), dt, optional=o is None)
    a.tensor(k, "k", (B, H, N, cfg.d_k), dt)
    a.tensor(v, "v", (B, H, N, cfg.d_v), dt)
    a.tensor(o, "o", (B, H, N, cfg.d_v), torch.float32, optional=True)
    stride = taylor_state_stride(cfg)
    for name, st in zip(("state_in", "state_out") if len(states) == 2 else ("state",), states):
        a.tensor(st, name, (B, H, stride), torch.float32, optional=True)
    if need_ws:
        a.workspace(workspace, taylor_prefill_workspace_bytes(cfg, B, H, N))
    a.done()
    return B, H, N


def _check_varlen(what, q, k, v, o, states, workspace, cu_seqlens, max_seqlen, cfg):
    """Checks a ragged prefill's tensors; returns (H, T, n_seqs)."""
    import torch

    a = _Args(what)
    H, T = a.rank(k, "k", 3, cfg.d_k)[:2]
    n_seqs = a.rank(cu_seqlens, "cu_seqlens", 1)[0] - 1
    if n_seqs < 0:
        raise ValueError(f"{what}: cu_seqlens needs n_seqs + 1 >= 1 entries")
    a.tensor(cu_seqlens, "cu_seqlens", (n_seqs + 1,), torch.int32)
    dt = _torch_dtype(cfg.in_dtype)
    a.tensor(q, "q", (H, T, cfg.d_k), dt, optional=o is None)
    a.tensor(k, "k", (H, T, cfg.d_k), dt)
    a.tensor(v, "v", (H, T, cfg.d_v), dt)
    a.tensor(o, "o", (H, T, cfg.d_v), torch.float32, optional=True)
    stride = taylor_state_stride(cfg)
    for name, st in zip(("state_in", "state_out") if len(states) == 2 else ("state",), states):
        a.tensor(st, name, (n_seqs, H, stride), torch.float32, optional=True)
    a.workspace(workspace, taylor_prefill_varlen_workspace_bytes(cfg, n_seqs, H, int(max_seqlen), T))
    a.done()
    return H, T, n_seqs


def taylor_state_init(state, cfg, stream=None):
    """Zero a [B, H, stride] float32 state tensor (an empty history)."""
    import torch

    a = _Args("taylor_state_init")
    B, H = a.rank(state, "state", 3)[:2]
    a.tensor(state, "state", (B, H, taylor_state_stride(cfg)), torch.float32)
    a.done()
    _check(lib().taylor_state_init(_ptr(state), B, H, ctypes.byref(cfg), _stream(stream, state.device)),
           "taylor_state_init")


def taylor_attn_prefill(q, k, v, o, state, workspace, cfg, stream=None):
    """Causal prefill over [B, H, N, d] inputs; o [B, H, N, d_v] float32 or None; state in/out or None."""
    B, H, N = _check_prefill("taylor_attn_prefill", q, k, v, o, (state,), workspace, cfg)
    rc = lib().taylor_attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(state), _ptr(workspace), B, H, N,
                                   ctypes.byref(cfg), _stream(stream, k.device))
    _check(rc, "taylor_attn_prefill")


def taylor_attn_prefill_into(q, k, v, o, state_in, state_out, workspace, cfg, stream=None):
    """Causal prefill over [B, H, N, d] inputs from state_in (or None: empty history) into state_out
    (or None: discarded; the same tensor as state_in, or one that does not overlap it)."""
    B, H, N = _check_prefill("taylor_attn_prefill_into", q, k, v, o, (state_in, state_out), workspace, cfg)
    rc = lib().taylor_attn_prefill_into(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(state_in), _ptr(state_out),
                                        _ptr(workspace), B, H, N, ctypes.byref(cfg), _stream(stream, k.device))
    _check(rc, "taylor_attn_prefill_into")


def taylor_attn_prefill_into_static(q, k, v, o, state_in, state_out, cfg, stream=None):
    """taylor_attn_prefill_into with the library's static per-GPU workspace (no workspace argument, no
    allocation); calls that overlap in time on one GPU race."""
    B, H, N = _check_prefill("taylor_attn_prefill_into_static", q, k, v, o, (state_in, state_out), None, cfg,
                             need_ws=False)
    rc = lib().taylor_attn_prefill_into_static(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(state_in), _ptr(state_out),
                                               B, H, N, ctypes.byref(cfg), _stream(stream, k.device))
    _check(rc, "taylor_attn_prefill_into_static")


def taylor_attn_prefill_varlen(q, k, v, o, state, workspace, cu_seqlens, max_seqlen, cfg, stream=None):
    """Causal prefill of a ragged batch packed as [H, T, d]; cu_seqlens is a device int32 tensor of
    n_seqs + 1 offsets; o [H, T, d_v] float32 or None; state [n_seqs, H, stride] in/out or None."""
    H, T, n_seqs = _check_varlen("taylor_attn_prefill_varlen", q, k, v, o, (state,), workspace, cu_seqlens,
                                 max_seqlen, cfg)
    rc = lib().taylor_attn_prefill_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(state), _ptr(workspace),
                                          _ptr(cu_seqlens), n_seqs, H, int(max_seqlen), T, ctypes.byref(cfg),
                                          _stream(stream, k.device))
    _check(rc, "taylor_attn_prefill_varlen")


def taylor_attn_prefill_varlen_into(q, k, v, o, state_in, state_out, workspace, cu_seqlens, max_seqlen, cfg,
                                    stream=None):
    """Ragged-batch prefill (as taylor_attn_prefill_varlen) from state_in (or None: empty histories) into
    state_out (or None: discarded; the same tensor as state_in, or one that does not overlap it)."""
    H, T, n_seqs = _check_varlen("taylor_attn_prefill_varlen_into", q, k, v, o, (state_in, state_out), workspace,
                                 cu_seqlens, max_seqlen, cfg)
    rc = lib().taylor_attn_prefill_varlen_into(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(state_in), _ptr(state_out),
                                               _ptr(workspace), _ptr(cu_seqlens), n_seqs, H, int(max_seqlen), T,
                                               ctypes.byref(cfg), _stream(stream, k.device))
    _check(rc, "taylor_attn_prefill_varlen_into")


def taylor_attn_prefill_backward(q, k, v, o, g, state, dstate, dq, dk, dv, workspace, cfg, stream=None):
    """Gradients of a prefill over [B, H, N, d] inputs: dq, dk, dv (float32, written); dstate in/out
    (gradient of the final state in, of the incoming state out) or None; state: the forward's
    incoming state or None."""
    import torch

    a = _Args("taylor_attn_prefill_backward")
    B, H, N = a.rank(k, "k", 4, cfg.d_k)[:3]
    dt, f32 = _torch_dtype(cfg.in_dtype), torch.float32
    for t, name, d, ty in ((q, "q", cfg.d_k, dt), (k, "k", cfg.d_k, dt), (v, "v", cfg.d_v, dt), (o, "o", cfg.d_v, f32),
                           (g, "g", cfg.d_v, f32), (dq, "dq", cfg.d_k, f32), (dk, "dk", cfg.d_k, f32),
                           (dv, "dv", cfg.d_v, f32)):
        a.tensor(t, name, (B, H, N, d), ty)
    stride = taylor_state_stride(cfg)
    a.tensor(state, "state", (B, H, stride), f32, optional=True)
    a.tensor(dstate, "dstate", (B, H, stride), f32, optional=True)
    a.workspace(workspace, taylor_prefill_backward_workspace_bytes(cfg, B, H, N))
    a.done()
    rc = lib().taylor_attn_prefill_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(g), _ptr(state), _ptr(dstate),
                                            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), B, H, N,
                                            ctypes.byref(cfg), _stream(stream, k.device))
    _check(rc, "taylor_attn_prefill_backward")


def new_backward_workspace(cfg, B, H, N, device):
    """A workspace tensor of taylor_prefill_backward_workspace_bytes() bytes (None when none is needed)."""
    import torch

    n = taylor_prefill_backward_workspace_bytes(cfg, B, H, N)
    if n == 0:
        return None
    return torch.empty(((n + 15) // 16 * 16,), dtype=torch.uint8, device=device)


def taylor_attn_decode_step(q, k, v, o, state, cfg, stream=None):
    """One decode step over [B, H, d] inputs; o [B, H, d_v] float32; state updated in place."""
    import torch

    a = _Args("taylor_attn_decode_step")
    B, H = a.rank(k, "k", 3, cfg.d_k)[:2]
    dt = _torch_dtype(cfg.in_dtype)
    a.tensor(q, "q", (B, H, cfg.d_k), dt)
    a.tensor(k, "k", (B, H, cfg.d_k), dt)
    a.tensor(v, "v", (B, H, cfg.d_v), dt)
    a.tensor(o, "o", (B, H, cfg.d_v), torch.float32)
    a.tensor(state, "state", (B, H, taylor_state_stride(cfg)), torch.float32)
    a.done()
    rc = lib().taylor_attn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(state), B, H,
                                       ctypes.byref(cfg), _stream(stream, k.device))
    _check(rc, "taylor_attn_decode_step")


# ---- allocation helpers (torch owns the memory) -------------------------------------------------


def new_state(B, H, cfg, device, stream=None):
    """A zeroed [B, H, stride] float32 state tensor on ``device``."""
    import torch

    st = torch.empty((B, H, taylor_state_stride(cfg)), dtype=torch.float32, device=device)
    taylor_state_init(st, cfg, stream)
    return st


def new_workspace(cfg, B, H, N, device):
    """A workspace tensor of taylor_prefill_workspace_bytes() bytes (None when no workspace is needed)."""
    import torch

    n = taylor_prefill_workspace_bytes(cfg, B, H, N)
    if n == 0:
        return None
    return torch.empty(((n + 15) // 16 * 16,), dtype=torch.uint8, device=device)


def new_varlen_workspace(cfg, n_seqs, H, max_seqlen, total_tokens, device):
    """A workspace tensor of taylor_prefill_varlen_workspace_bytes() bytes (None when none is needed)."""
    import torch

    n = taylor_prefill_varlen_workspace_bytes(cfg, n_seqs, H, max_seqlen, total_tokens)
    if n == 0:
        return None
    return torch.empty(((n + 15) // 16 * 16,), dtype=torch.uint8, device=device)


def state_views(state, cfg):
    """Views (S [B, H, W, d_v], z [B, H, W]) of a [B, H, stride] state tensor."""
    W = taylor_feature_width(cfg.n_terms, cfg.d_k)
    S = state[..., : W * cfg.d_v].unflatten(-1, (W, cfg.d_v))
    z = state[..., W * cfg.d_v : W * (cfg.d_v + 1)]
    return S, z


# ---- differentiable op (forward and backward entry points under torch.autograd) ------------------

_AUTOGRAD_FN = None


def _autograd_fn():
    global _AUTOGRAD_FN
    if _AUTOGRAD_FN is None:
        import torch

        class _TaylorAttention(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, state, cfg):
                B, H, N = k.shape[:3]
                o = torch.empty((B, H, N, cfg.d_v), dtype=torch.float32, device=k.device)
                taylor_attn_prefill_into(q, k, v, o, state, None, new_workspace(cfg, B, H, N, k.device), cfg)
                ctx.save_for_backward(q, k, v, o, state)
                ctx.cfg = cfg
                return o

            @staticmethod
            def backward(ctx, g):
                q, k, v, o, state = ctx.saved_tensors
                cfg = ctx.cfg
                B, H, N = k.shape[:3]
                g = g.to(torch.float32).contiguous()
                dq = torch.empty(q.shape, dtype=torch.float32, device=k.device)
                dk = torch.empty(k.shape, dtype=torch.float32, device=k.device)
                dv = torch.empty(v.shape, dtype=torch.float32, device=k.device)
                # the final state is not an output of the op, so its gradient (dstate in) is zero
                dstate = torch.zeros_like(state) if state is not None and ctx.needs_input_grad[3] else None
                taylor_attn_prefill_backward(q, k, v, o, g, state, dstate, dq, dk, dv,
                                             new_backward_workspace(cfg, B, H, N, k.device), cfg)
                return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), dstate, None

        _AUTOGRAD_FN = _TaylorAttention
    return _AUTOGRAD_FN


def taylor_attention(q, k, v, cfg, state=None):
    """Causal Taylor attention as a differentiable op over contiguous [B, H, N, d] inputs (float32 or
    bfloat16 as cfg says): the forward is taylor_attn_prefill_into from `state` (a float32 [B, H,
    stride] incoming state, or None for an empty history), the backward taylor_attn_prefill_backward;
    returns o [B, H, N, d_v] float32.  q, k, v and `state` receive gradients when they require them
    (the truncated-kernel readout at n = 1..5, d_k = 16, d_v = 64)."""
    return _autograd_fn().apply(q, k, v, state, cfg)
