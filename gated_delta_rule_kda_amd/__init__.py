"""Python binding of libkda.so, the gfx950 Kimi Delta Attention (KDA) core.

Argument marshalling only: every step of the layer core runs in the HIP
kernels behind the C ABI declared in include/kda.h.  PyTorch provides device
memory and the current HIP stream; nothing here computes on tensors, and
there is no fallback: if libkda.so is missing every call raises.

    import gated_delta_rule_kda_amd as kda
    o, state, conv = kda.prefill(q, k, v, log_alpha, beta, cu_seqlens,
                                 g=g, conv_w=conv_w, state_in=S0)
    o = kda.decode_step(q, k, v, log_alpha, beta, state, g=g, conv_w=conv_w,
                        conv_state=conv)   # state and conv updated in place
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

HEAD_DIM = 128
F32, BF16 = 0, 1
ALGOS = {"auto": 0, "recurrent": 1, "chunked": 2, "chunked_throughput": 3, "chunked_latency": 4,
         "chunked_scan": 5}
GATES = {"log_alpha": 0, "lowrank": 1, "head": 2, "lowrank_softplus": 3, "log_alpha_unbounded": 4}
BETA_MODES = {"value": 0, "logit": 1}
OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_WORKSPACE_TOO_SMALL, ERR_HIP = range(5)

EXPORTS = ("kda_config_init", "kda_prefill_workspace_size", "kda_prefill", "kda_prefill_no_alloc",
           "kda_prefill_resolved_algo", "kda_decode_step",
           "kda_status_string", "kda_abi_version", "kda_state_bytes")


class KdaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("prologue", ctypes.c_int32), ("epilogue", ctypes.c_int32),
                ("algo", ctypes.c_int32), ("scale", ctypes.c_float),
                ("l2_eps", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("gate", ctypes.c_int32), ("gate_rank", ctypes.c_int32),
                ("beta_mode", ctypes.c_int32)]


_vp = ctypes.c_void_p


class PrefillArgs(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("cu_seqlens", _vp), ("total_tokens", ctypes.c_int64),
                ("q", _vp), ("k", _vp), ("v", _vp), ("log_alpha", _vp), ("beta", _vp), ("g", _vp),
                ("conv_w", _vp), ("conv_in", _vp), ("conv_out", _vp), ("rms_w", _vp),
                ("state_in", _vp), ("state_out", _vp), ("o", _vp), ("workspace", _vp),
                ("workspace_bytes", ctypes.c_size_t), ("state_in_slots", _vp), ("state_out_slots", _vp),
                ("gate_z", _vp), ("gate_w", _vp), ("gate_bias", _vp), ("gate_a", _vp)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q", _vp), ("k", _vp), ("v", _vp),
                ("log_alpha", _vp), ("beta", _vp), ("g", _vp), ("conv_w", _vp),
                ("conv_state", _vp), ("rms_w", _vp), ("state", _vp), ("slots", _vp), ("o", _vp),
                ("slots_out", _vp), ("gate_z", _vp), ("gate_w", _vp), ("gate_bias", _vp), ("gate_a", _vp)]


_lib: Optional[ctypes.CDLL] = None


def _init_device_runtime() -> None:
    """Initialise the HIP runtime (through torch, which shares it with this library) before
    the library registers its kernels: loading the library into an uninitialised runtime
    after worker threads have started has left every later launch failing with
    hipErrorNoDevice.  Nothing happens without a GPU."""
    try:
        import torch
    except ImportError:
        return
    if torch.cuda.is_available():
        torch.cuda.init()


def lib() -> ctypes.CDLL:
    """Load the in-tree libkda.so (raises when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m gated_delta_rule_kda_amd._build`")
        _init_device_runtime()
        L = ctypes.CDLL(LIB_PATH)
        L.kda_config_init.argtypes = [ctypes.POINTER(Config), ctypes.c_int32]
        L.kda_config_init.restype = None
        L.kda_prefill_workspace_size.argtypes = [ctypes.POINTER(Config), ctypes.c_int32,
                                                 ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)]
        L.kda_prefill_workspace_size.restype = ctypes.c_int32
        L.kda_prefill.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(PrefillArgs), _vp]
        L.kda_prefill.restype = ctypes.c_int32
        L.kda_prefill_no_alloc.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(PrefillArgs), _vp]
        L.kda_prefill_no_alloc.restype = ctypes.c_int32
        L.kda_prefill_resolved_algo.argtypes = [ctypes.POINTER(Config), ctypes.c_int32, ctypes.c_int64]
        L.kda_prefill_resolved_algo.restype = ctypes.c_int32
        L.kda_decode_step.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(DecodeArgs), _vp]
        L.kda_decode_step.restype = ctypes.c_int32
        L.kda_status_string.argtypes = [ctypes.c_int32]
        L.kda_status_string.restype = ctypes.c_char_p
        L.kda_abi_version.argtypes = []
        L.kda_abi_version.restype = ctypes.c_uint32
        L.kda_state_bytes.argtypes = [ctypes.c_int32]
        L.kda_state_bytes.restype = ctypes.c_size_t
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != OK:
        raise KdaError(status, lib().kda_status_string(status).decode())


def config(num_heads: int, io_dtype: str = "bf16", out_dtype: Optional[str] = None,
           prologue: bool = True, epilogue: bool = True, algo: str = "auto",
           scale: Optional[float] = None, l2_eps: float = 1e-6, rms_eps: float = 1e-6,
           head_dim: int = HEAD_DIM, gate: str = "log_alpha", gate_rank: int = 128,
           beta_mode: str = "value") -> Config:
    c = Config()
    lib().kda_config_init(ctypes.byref(c), num_heads)
    c.head_dim = head_dim
    c.io_dtype = _dtype_code(io_dtype)
    c.out_dtype = _dtype_code(out_dtype or io_dtype)
    c.prologue = int(bool(prologue))
    c.epilogue = int(bool(epilogue))
    c.algo = ALGOS[algo]
    c.scale = 1.0 / math.sqrt(head_dim) if scale is None else float(scale)
    c.l2_eps = float(l2_eps)
    c.rms_eps = float(rms_eps)
    c.gate = GATES[gate]
    c.gate_rank = int(gate_rank)
    c.beta_mode = BETA_MODES[beta_mode]
    return c


def _dtype_code(name: str) -> int:
    if name in ("bf16", "bfloat16"):
        return BF16
    if name in ("f32", "fp32", "float32"):
        return F32
    raise ValueError(f"unsupported dtype {name!r}")


def _torch_dtype(code: int):
    import torch
    return torch.bfloat16 if code == BF16 else torch.float32


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _on_stream(stream):
    """Context in which torch allocates for the launch stream: tensors this binding
    allocates (outputs, workspace) then belong to the stream the kernels run on, so
    torch's caching allocator does not hand their memory to other work while the
    kernels may still use it."""
    import contextlib
    import torch
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _expect(t, name: str, dtype, shape=None) -> None:
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _expect_device(dev, **tensors) -> None:
    """Every tensor given lives on `dev`, the GPU of q: the kernels take raw device pointers,
    so a host tensor or one on another GPU would be read as an address on this one."""
    if dev.type != "cuda":
        raise ValueError(f"q is on {dev}: the inputs must be GPU tensors")
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev} (the device of q)")


def _expect_gate(cfg, z, w, bias, a, T, H, io_t) -> None:
    import torch
    r = cfg.gate_rank
    _expect(z, "gate_z", io_t, (T, r))
    _expect(w, "gate_w", io_t, (H * HEAD_DIM, r))
    _expect(bias, "gate_bias", torch.float32, (H * HEAD_DIM,))
    _expect(a, "gate_a", torch.float32, (H,))


def workspace_size(cfg: Config, num_seqs: int, total_tokens: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().kda_prefill_workspace_size(ctypes.byref(cfg), num_seqs, total_tokens, ctypes.byref(n)))
    return n.value


def prefill(q, k, v, log_alpha, beta, cu_seqlens, *, g=None, conv_w=None, conv_in=None,
            conv_out=None, rms_w=None, state_in=None, state_out=None, o=None, workspace=None,
            state_in_slots=None, state_out_slots=None, gate_z=None, gate_w=None, gate_bias=None,
            gate_a=None, cfg: Optional[Config] = None, return_state: bool = True, return_conv: bool = True,
            stream=None, no_alloc: bool = False, **cfg_kwargs) -> Tuple[object, object, object]:
    """kda_prefill on torch tensors.  q, k, v, g: [T, H, 128]; log_alpha [T, H, 128] fp32;
    beta [T, H] fp32; cu_seqlens int32 [N+1] on the device.  Missing outputs are allocated.
    With state_in_slots / state_out_slots (int32 [N] on the device) the state and conv arrays
    are pools of rows [rows, H, 128, 128] / [rows, 3, 3, H*128] and sequence n reads row
    state_in_slots[n] and writes row state_out_slots[n]; outputs are then not allocated.
    With the low-rank gate (cfg.gate == "lowrank", or gate_z given) log_alpha may be None and
    gate_z [T, r], gate_w [H*128, r] (io dtype), gate_bias [H*128] and gate_a [H] (fp32) are used.
    gate "lowrank_softplus" takes the same factors and forms Kimi Linear's unbounded
    log alpha = -e^A softplus(z_down W_up^T + b).  With the scalar per-head gate
    (cfg.gate == "head") log_alpha is [T, H] fp32; with "log_alpha_unbounded" it is
    [T, H, 128] with any value <= 0.  With beta_mode "logit" beta holds the pre-activation
    and the kernels apply the sigmoid.  Outputs and the workspace that this function
    allocates are allocated on `stream` (default: the current stream).  With no_alloc the
    call goes to kda_prefill_no_alloc, which uses the library's static scratch in place of a
    workspace (pass o, and state_out / conv_out or return_state / return_conv False, for a
    call that allocates nothing at all).
    Returns (o, state_out, conv_out)."""
    import torch
    T, H = q.shape[0], q.shape[1]
    if cfg is None and gate_z is not None:
        cfg_kwargs.setdefault("gate", "lowrank")
        cfg_kwargs.setdefault("gate_rank", gate_z.shape[1])
    N = cu_seqlens.shape[0] - 1
    if cfg is None:
        io = "bf16" if q.dtype == torch.bfloat16 else "f32"
        cfg_kwargs.setdefault("io_dtype", io)
        cfg_kwargs.setdefault("prologue", conv_w is not None)
        cfg_kwargs.setdefault("epilogue", g is not None)
        cfg = config(H, **cfg_kwargs)
    elif cfg_kwargs:
        raise TypeError("pass either cfg or config keywords, not both")
    io_t, out_t = _torch_dtype(cfg.io_dtype), _torch_dtype(cfg.out_dtype)
    D = q.shape[2]
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g)):
        _expect(t, name, io_t, (T, H, D))
    _expect(log_alpha, "log_alpha", torch.float32, (T, H) if cfg.gate == GATES["head"] else (T, H, D))
    _expect_gate(cfg, gate_z, gate_w, gate_bias, gate_a, T, H, io_t)
    _expect(beta, "beta", torch.float32, (T, H))
    _expect(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    _expect(conv_w, "conv_w", torch.float32, (3, H * D, 4))
    _expect(state_in_slots, "state_in_slots", torch.int32, (N,))
    _expect(state_out_slots, "state_out_slots", torch.int32, (N,))
    rows_in = N if state_in_slots is None else (None if state_in is None else state_in.shape[0])
    rows_ci = N if state_in_slots is None else (None if conv_in is None else conv_in.shape[0])
    rows_out = N if state_out_slots is None else (None if state_out is None else state_out.shape[0])
    rows_co = N if state_out_slots is None else (None if conv_out is None else conv_out.shape[0])
    _expect(conv_in, "conv_in", io_t, (rows_ci, 3, 3, H * D))
    _expect(rms_w, "rms_w", torch.float32, (D,))
    _expect(state_in, "state_in", torch.float32, (rows_in, H, D, D))
    dev = q.device
    with _on_stream(stream):
        if o is None:
            o = torch.empty((T, H, D), dtype=out_t, device=dev)
        if state_out is None and return_state and state_out_slots is None:
            state_out = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
        if conv_out is None and return_conv and cfg.prologue and state_out_slots is None:
            conv_out = torch.empty((N, 3, 3, H * D), dtype=io_t, device=dev)
        need = 0 if no_alloc else workspace_size(cfg, N, T)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _expect(o, "o", out_t, (T, H, D))
    _expect(state_out, "state_out", torch.float32, (rows_out, H, D, D))
    _expect(conv_out, "conv_out", io_t, (rows_co, 3, 3, H * D))
    _expect_device(dev, q=q, k=k, v=v, log_alpha=log_alpha, beta=beta, cu_seqlens=cu_seqlens, g=g,
                   conv_w=conv_w, conv_in=conv_in, conv_out=conv_out, rms_w=rms_w, state_in=state_in,
                   state_out=state_out, o=o, workspace=workspace, state_in_slots=state_in_slots,
                   state_out_slots=state_out_slots, gate_z=gate_z, gate_w=gate_w, gate_bias=gate_bias,
                   gate_a=gate_a)
    a = PrefillArgs()
    a.num_seqs, a.cu_seqlens, a.total_tokens = N, _ptr(cu_seqlens), T
    a.q, a.k, a.v, a.log_alpha, a.beta, a.g = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                               _ptr(beta), _ptr(g))
    a.conv_w, a.conv_in, a.conv_out, a.rms_w = _ptr(conv_w), _ptr(conv_in), _ptr(conv_out), _ptr(rms_w)
    a.state_in, a.state_out, a.o = _ptr(state_in), _ptr(state_out), _ptr(o)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.state_in_slots, a.state_out_slots = _ptr(state_in_slots), _ptr(state_out_slots)
    a.gate_z, a.gate_w, a.gate_bias, a.gate_a = _ptr(gate_z), _ptr(gate_w), _ptr(gate_bias), _ptr(gate_a)
    fn = lib().kda_prefill_no_alloc if no_alloc else lib().kda_prefill
    _check(fn(ctypes.byref(cfg), ctypes.byref(a), _stream(stream)))
    return o, state_out, conv_out


def decode_step(q, k, v, log_alpha, beta, state, *, g=None, conv_w=None, conv_state=None,
                rms_w=None, slots=None, slots_out=None, o=None, gate_z=None, gate_w=None,
                gate_bias=None, gate_a=None, cfg: Optional[Config] = None, stream=None, **cfg_kwargs):
    """kda_decode_step on torch tensors: one token per request, q, k, v, g [B, H, 128];
    state [rows, H, 128, 128] and conv_state [rows, 3, 3, H*128] are pools updated in place:
    request b reads row slots[b] (b when None) and writes row slots_out[b] (its read row
    when None).  log_alpha is [B, H, 128] fp32, or [B, H] with cfg.gate == "head".
    Returns o [B, H, 128]."""
    import torch
    B, H, D = q.shape
    if cfg is None and gate_z is not None:
        cfg_kwargs.setdefault("gate", "lowrank")
        cfg_kwargs.setdefault("gate_rank", gate_z.shape[1])
    if cfg is None:
        io = "bf16" if q.dtype == torch.bfloat16 else "f32"
        cfg_kwargs.setdefault("io_dtype", io)
        cfg_kwargs.setdefault("prologue", conv_w is not None)
        cfg_kwargs.setdefault("epilogue", g is not None)
        cfg = config(H, **cfg_kwargs)
    elif cfg_kwargs:
        raise TypeError("pass either cfg or config keywords, not both")
    io_t, out_t = _torch_dtype(cfg.io_dtype), _torch_dtype(cfg.out_dtype)
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g)):
        _expect(t, name, io_t, (B, H, D))
    _expect(log_alpha, "log_alpha", torch.float32, (B, H) if cfg.gate == GATES["head"] else (B, H, D))
    _expect_gate(cfg, gate_z, gate_w, gate_bias, gate_a, B, H, io_t)
    _expect(beta, "beta", torch.float32, (B, H))
    n_slots = state.shape[0]
    _expect(state, "state", torch.float32, (n_slots, H, D, D))
    if slots is None and n_slots < B:
        raise ValueError("state has fewer rows than requests")
    _expect(conv_w, "conv_w", torch.float32, (3, H * D, 4))
    if conv_state is not None:
        _expect(conv_state, "conv_state", io_t, (conv_state.shape[0], 3, 3, H * D))
    _expect(rms_w, "rms_w", torch.float32, (D,))
    _expect(slots, "slots", torch.int32, (B,))
    _expect(slots_out, "slots_out", torch.int32, (B,))
    if slots_out is not None and slots is None and n_slots < B:
        raise ValueError("state has fewer rows than requests")
    if o is None:
        with _on_stream(stream):
            o = torch.empty((B, H, D), dtype=out_t, device=q.device)
    _expect(o, "o", out_t, (B, H, D))
    _expect_device(q.device, q=q, k=k, v=v, log_alpha=log_alpha, beta=beta, g=g, conv_w=conv_w,
                   conv_state=conv_state, rms_w=rms_w, state=state, slots=slots, slots_out=slots_out, o=o,
                   gate_z=gate_z, gate_w=gate_w, gate_bias=gate_bias, gate_a=gate_a)
    a = DecodeArgs()
    a.batch = B
    a.q, a.k, a.v, a.log_alpha, a.beta, a.g = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                               _ptr(beta), _ptr(g))
    a.conv_w, a.conv_state, a.rms_w = _ptr(conv_w), _ptr(conv_state), _ptr(rms_w)
    a.state, a.slots, a.o = _ptr(state), _ptr(slots), _ptr(o)
    a.slots_out = _ptr(slots_out)
    a.gate_z, a.gate_w, a.gate_bias, a.gate_a = _ptr(gate_z), _ptr(gate_w), _ptr(gate_bias), _ptr(gate_a)
    _check(lib().kda_decode_step(ctypes.byref(cfg), ctypes.byref(a), _stream(stream)))
    return o


def resolved_algo(cfg: Config, num_seqs: int = 1, total_tokens: int = 0) -> str:
    """Name of the prefill algorithm the library runs for `cfg`, `num_seqs` sequences and
    `total_tokens` tokens on the current device (AUTO and CHUNKED resolved)."""
    code = lib().kda_prefill_resolved_algo(ctypes.byref(cfg), num_seqs, total_tokens)
    if code < 0:
        raise KdaError(ERR_INVALID_ARGUMENT, "invalid configuration")
    return {v: k for k, v in ALGOS.items()}[code]


def abi_version() -> int:
    return lib().kda_abi_version()


def state_bytes(num_heads: int) -> int:
    return lib().kda_state_bytes(num_heads)
