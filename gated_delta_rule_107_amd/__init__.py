"""KDA (Kimi Delta Attention) hot path on MI355X: Python binding of libkda.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/kda.h.  PyTorch supplies device
memory and the current stream.  libkda.so is loaded on the first call; every
call raises ImportError if it has not been built
(``python -m gated_delta_rule_107_amd.build``).  There is no fallback path.

    o, S_T = chunk_fwd(q, k, v, log_alpha, beta, S0=None, chunk=64)
    o      = decode_step(state, q, k, v, log_alpha, beta)      # state updated in place
    o      = decode_verify(state, q, k, v, log_alpha, beta)    # n draft tokens, state untouched
    decode_commit(state, q, k, v, log_alpha, beta, n_accept)   # replay the accepted drafts

``gate=GATE_LOGITS`` makes every call read log_alpha as raw gate logits x, with the
log-decay -5 sigmoid(x) formed inside the kernels; ``qk_norm=True`` normalises q and k
per token inside the kernels (x / sqrt(sum x^2 + 1e-6)).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["KdaError", "Plan", "chunk_fwd", "chunk_fwd_noalloc", "decode_step", "decode_verify", "decode_commit",
           "default_plan", "workspace_bytes", "library_path", "ERRORS", "GATE_LOG_DECAY", "GATE_LOGITS"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libkda.so")

ERRORS = {0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_DTYPE", 4: "KDA_ERR_ALIGN",
          5: "KDA_ERR_UNSUPPORTED", 6: "KDA_ERR_WORKSPACE", 7: "KDA_ERR_HIP", 8: "KDA_ERR_ALIAS"}
DTYPE_F32, DTYPE_BF16 = 0, 1
GATE_LOG_DECAY, GATE_LOGITS = 0, 1
FLAG_GATE_LOGITS, FLAG_QK_L2NORM = 1, 2          # kda_input_flag_t


class KdaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


class Plan(ctypes.Structure):
    """kda_plan_t: segmentation, column blocking, optional launch-timing events, optional
    state checkpoints, packed sequences, the input flags and the lead form's segment-0 length."""
    _fields_ = [("n_segments", ctypes.c_int32), ("dv_block", ctypes.c_int32),
                ("launch_events", ctypes.POINTER(ctypes.c_void_p)), ("n_launch_events", ctypes.c_int32),
                ("state_ckpt", ctypes.c_void_p), ("ckpt_stride", ctypes.c_int64),
                ("cu_seqlens", ctypes.c_void_p), ("n_seqs", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("seg0_len", ctypes.c_int64)]

    def __repr__(self):
        lead = f", seg0_len={self.seg0_len}" if self.seg0_len else ""
        return f"Plan(n_segments={self.n_segments}, dv_block={self.dv_block}{lead})"


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m gated_delta_rule_107_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    lib.kda_chunk_fwd.restype = i32
    lib.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, i32,
                                  ctypes.POINTER(Plan), vp, sz, vp]
    lib.kda_chunk_fwd_noalloc.restype = i32
    lib.kda_chunk_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, i32,
                                          ctypes.POINTER(Plan), vp]
    lib.kda_decode_step.restype = i32
    u32 = ctypes.c_uint32
    lib.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, u32, vp]
    lib.kda_decode_verify.restype = i32
    lib.kda_decode_verify.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, u32, vp]
    lib.kda_decode_commit.restype = i32
    lib.kda_decode_commit.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, u32, vp]
    lib.kda_chunk_fwd_default_plan.restype = i32
    lib.kda_chunk_fwd_default_plan.argtypes = [i64, i64, i32, i32, i32, i32, i32, ctypes.POINTER(Plan)]
    lib.kda_chunk_fwd_workspace_bytes.restype = i32
    lib.kda_chunk_fwd_workspace_bytes.argtypes = [i64, i64, i32, i32, i32, i32, i32, ctypes.POINTER(Plan),
                                                  ctypes.POINTER(sz)]
    lib.kda_status_str.restype = ctypes.c_char_p
    lib.kda_status_str.argtypes = [i32]
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_abi_version.restype = i32
    lib.kda_abi_version.argtypes = []
    return lib


_lib_handle = None


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libkda.so (ctypes handle), loaded on first use; raises ImportError if it is not built."""
    global _lib_handle
    if _lib_handle is None:
        _lib_handle = _load()
    return _lib_handle


def _check(code: int):
    if code != 0:
        raise KdaError(code, lib().kda_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise KdaError(3, f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require(t: torch.Tensor, name: str, dtype: torch.dtype | None, shape: tuple, device):
    if not isinstance(t, torch.Tensor):
        raise KdaError(1, f"{name} must be a tensor")
    if dtype is not None and t.dtype != dtype:
        raise KdaError(3, f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise KdaError(2, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.device != device:
        raise KdaError(2, f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise KdaError(2, f"{name} must be contiguous")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def default_plan(B, T, H, dk, dv, chunk=64, dtype=torch.bfloat16) -> Plan:
    plan = Plan()
    code = DTYPE_BF16 if dtype == torch.bfloat16 else DTYPE_F32
    _check(lib().kda_chunk_fwd_default_plan(B, T, H, dk, dv, chunk, code, ctypes.byref(plan)))
    return plan


def workspace_bytes(B, T, H, dk, dv, chunk=64, dtype=torch.bfloat16, plan: Plan | None = None) -> int:
    n = ctypes.c_size_t(0)
    code = DTYPE_BF16 if dtype == torch.bfloat16 else DTYPE_F32
    _check(lib().kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, code,
                                              ctypes.byref(plan) if plan is not None else None,
                                              ctypes.byref(n)))
    return n.value


def _plan_copy(plan: Plan | None) -> Plan:
    p2 = Plan()
    if plan is not None:
        ctypes.memmove(ctypes.addressof(p2), ctypes.addressof(plan), ctypes.sizeof(Plan))
    return p2


def _flags(gate: int, qk_norm: bool) -> int:
    if gate not in (GATE_LOG_DECAY, GATE_LOGITS):
        raise KdaError(5, f"unknown gate mode {gate}")
    return (FLAG_GATE_LOGITS if gate == GATE_LOGITS else 0) | (FLAG_QK_L2NORM if qk_norm else 0)


def chunk_fwd(q, k, v, log_alpha, beta, S0=None, chunk: int = 64, plan: Plan | None = None,
              o=None, S_T=None, workspace=None, ckpt_stride: int = 0, state_ckpt=None, cu_seqlens=None,
              gate: int = GATE_LOG_DECAY, qk_norm: bool = False):
    """Chunked prefill: returns (o [B,T,H,dv] in q's dtype, S_T [B,H,dk,dv] float32), and with
    ``ckpt_stride`` > 0 also the state checkpoints [B, T // ckpt_stride, H, dk, dv] float32
    (the state after every ckpt_stride tokens; a multiple of ``chunk``).

    ``S_T`` may be passed as ``S0`` itself to advance the state in place.
    ``plan`` (a Plan) overrides the library's default segmentation / column blocking.
    ``cu_seqlens`` (int32 [N+1] on the device) packs N sequences along T of a single batch
    row; S0 / S_T are then [N, H, dk, dv].
    ``gate=GATE_LOGITS``: log_alpha holds raw gate logits (log-decay -5 sigmoid(x)).
    ``qk_norm=True``: q and k are L2-normalised per token inside the kernels.
    """
    if q.dim() != 4:
        raise KdaError(2, "q must be [B,T,H,dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise KdaError(2, "tensors must be on a GPU")
    dt = _dtype_code(q)
    _require(q, "q", q.dtype, (B, T, H, dk), dev)
    _require(k, "k", q.dtype, (B, T, H, dk), dev)
    _require(v, "v", q.dtype, (B, T, H, dv), dev)
    _require(log_alpha, "log_alpha", torch.float32, (B, T, H, dk), dev)
    _require(beta, "beta", torch.float32, (B, T, H), dev)
    NS = B
    if cu_seqlens is not None:
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise KdaError(2, "cu_seqlens must be [N+1] with N >= 1")
        _require(cu_seqlens, "cu_seqlens", torch.int32, (cu_seqlens.numel(),), dev)
        NS = cu_seqlens.numel() - 1
    if S0 is not None:
        _require(S0, "S0", torch.float32, (NS, H, dk, dv), dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    else:
        _require(o, "o", q.dtype, (B, T, H, dv), dev)
    if S_T is None:
        S_T = torch.empty((NS, H, dk, dv), dtype=torch.float32, device=dev)
    else:
        _require(S_T, "S_T", torch.float32, (NS, H, dk, dv), dev)
    flags = _flags(gate, qk_norm)
    if flags:
        plan = _plan_copy(plan)
        plan.flags = flags
    if cu_seqlens is not None:
        p2 = _plan_copy(plan)
        p2.cu_seqlens = cu_seqlens.data_ptr()
        p2.n_seqs = NS
        plan = p2
    if ckpt_stride:
        if ckpt_stride < 0 or ckpt_stride % chunk:
            raise KdaError(5, f"ckpt_stride ({ckpt_stride}) must be a positive multiple of chunk ({chunk})")
        nck = T // ckpt_stride
        if state_ckpt is None:
            state_ckpt = torch.empty((B, nck, H, dk, dv), dtype=torch.float32, device=dev)
        else:
            _require(state_ckpt, "state_ckpt", torch.float32, (B, nck, H, dk, dv), dev)
        p2 = _plan_copy(plan)
        if nck > 0:                          # (T < ckpt_stride: no checkpoint to write)
            p2.state_ckpt = state_ckpt.data_ptr()
            p2.ckpt_stride = ckpt_stride
        plan = p2
    nws = workspace_bytes(B, T, H, dk, dv, chunk, q.dtype, plan)
    if nws > 0:
        if workspace is None or workspace.numel() * workspace.element_size() < nws:
            workspace = torch.empty(nws, dtype=torch.uint8, device=dev)
    else:
        workspace = None
    code = lib().kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0),
                              _ptr(o), _ptr(S_T), B, T, H, dk, dv, chunk, dt,
                              ctypes.byref(plan) if plan is not None else None,
                              _ptr(workspace), nws, _stream(dev))
    _check(code)
    if ckpt_stride:
        return o, S_T, state_ckpt
    return o, S_T


def chunk_fwd_noalloc(q, k, v, log_alpha, beta, S0, o, S_T, chunk: int = 64, plan: Plan | None = None):
    """kda_chunk_fwd_noalloc: chunked prefill into caller-given ``o`` and ``S_T``, with the
    segment workspace held by the library (KDA_NOALLOC_SCRATCH_BYTES per GPU) instead of
    passed in.  Allocates nothing.  Plans needing more workspace raise KDA_ERR_WORKSPACE.
    Calls that may overlap in time on one GPU share that workspace and race."""
    if q.dim() != 4:
        raise KdaError(2, "q must be [B,T,H,dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise KdaError(2, "tensors must be on a GPU")
    dt = _dtype_code(q)
    _require(q, "q", q.dtype, (B, T, H, dk), dev)
    _require(k, "k", q.dtype, (B, T, H, dk), dev)
    _require(v, "v", q.dtype, (B, T, H, dv), dev)
    _require(log_alpha, "log_alpha", torch.float32, (B, T, H, dk), dev)
    _require(beta, "beta", torch.float32, (B, T, H), dev)
    if S0 is not None:
        _require(S0, "S0", torch.float32, (B, H, dk, dv), dev)
    _require(o, "o", q.dtype, (B, T, H, dv), dev)
    _require(S_T, "S_T", torch.float32, (B, H, dk, dv), dev)
    _check(lib().kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0),
                                      _ptr(o), _ptr(S_T), B, T, H, dk, dv, chunk, dt,
                                      ctypes.byref(plan) if plan is not None else None, _stream(dev)))
    return o, S_T


def _decode_inputs(state, q, k, v, log_alpha, beta, n_tok):
    """Checks the decode family's tensors; per-token tensors are [N,H,.] for a step
    (n_tok None) or [N,n,H,.]. Returns (N, H, dk, dv, n, dt, dev)."""
    if state.dim() != 4:
        raise KdaError(2, "state must be [N,H,dk,dv]")
    N, H, dk, dv = state.shape
    dev = state.device
    if dev.type != "cuda":
        raise KdaError(2, "tensors must be on a GPU")
    dt = _dtype_code(q)
    lead = (N, H) if n_tok is None else (N, n_tok, H)
    _require(state, "state", torch.float32, (N, H, dk, dv), dev)
    _require(q, "q", q.dtype, lead + (dk,), dev)
    _require(k, "k", q.dtype, lead + (dk,), dev)
    _require(v, "v", q.dtype, lead + (dv,), dev)
    _require(log_alpha, "log_alpha", torch.float32, lead + (dk,), dev)
    _require(beta, "beta", torch.float32, lead, dev)
    return N, H, dk, dv, dt, dev


def decode_step(state, q, k, v, log_alpha, beta, o=None, gate: int = GATE_LOG_DECAY, qk_norm: bool = False):
    """One recurrent step for N sequences; ``state`` [N,H,dk,dv] float32 is updated in place.
    q, k [N,H,dk], v [N,H,dv] (bf16 or float32), log_alpha [N,H,dk], beta [N,H] float32.
    Returns o [N,H,dv]."""
    N, H, dk, dv, dt, dev = _decode_inputs(state, q, k, v, log_alpha, beta, None)
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    else:
        _require(o, "o", q.dtype, (N, H, dv), dev)
    _check(lib().kda_decode_step(_ptr(state), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                _ptr(o), N, H, dk, dv, dt, _flags(gate, qk_norm), _stream(dev)))
    return o


def decode_verify(state, q, k, v, log_alpha, beta, o=None, gate: int = GATE_LOG_DECAY, qk_norm: bool = False):
    """Speculative decoding, verify: outputs of n draft tokens per sequence from ``state``
    [N,H,dk,dv], which is left unchanged.  q, k [N,n,H,dk], v [N,n,H,dv], log_alpha [N,n,H,dk],
    beta [N,n,H].  Returns o [N,n,H,dv] (draft j read after drafts 0..j)."""
    if q.dim() != 4:
        raise KdaError(2, "q must be [N,n,H,dk]")
    n = q.shape[1]
    N, H, dk, dv, dt, dev = _decode_inputs(state, q, k, v, log_alpha, beta, n)
    if o is None:
        o = torch.empty((N, n, H, dv), dtype=q.dtype, device=dev)
    else:
        _require(o, "o", q.dtype, (N, n, H, dv), dev)
    _check(lib().kda_decode_verify(_ptr(state), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                  _ptr(o), N, n, H, dk, dv, dt, _flags(gate, qk_norm), _stream(dev)))
    return o


def decode_commit(state, q, k, v, log_alpha, beta, n_accept, gate: int = GATE_LOG_DECAY, qk_norm: bool = False):
    """Speculative decoding, commit: advances ``state`` [N,H,dk,dv] in place by the first
    n_accept[i] (int32 [N] on the device, clamped to [0, n]) of sequence i's n draft tokens,
    given as for decode_verify.  Returns state."""
    if q.dim() != 4:
        raise KdaError(2, "q must be [N,n,H,dk]")
    n = q.shape[1]
    N, H, dk, dv, dt, dev = _decode_inputs(state, q, k, v, log_alpha, beta, n)
    _require(n_accept, "n_accept", torch.int32, (N,), dev)
    _check(lib().kda_decode_commit(_ptr(state), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                  _ptr(n_accept), N, n, H, dk, dv, dt, _flags(gate, qk_norm), _stream(dev)))
    return state
