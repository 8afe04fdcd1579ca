"""Transformer-FSQ latent decode on AMD MI355X: Python binding of libfsq.so.

The binding only marshals arguments: it checks tensor dtypes, shapes and
devices, takes their data pointers and the current HIP stream, and calls the
C ABI declared in include/fsq.h. Every step of the computation runs in the
library's HIP kernels. If the library has not been built the import of this
module succeeds but every call raises; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

# FSQ_LIBRARY_PATH: another build of the same library (A/B measurements);
# the in-tree build by default
_LIB_PATH = os.environ.get("FSQ_LIBRARY_PATH") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "lib", "libfsq.so")
EXPORTS = ("fsq_status_string", "fsq_append", "fsq_decode_workspace_bytes", "fsq_decode_attn",
           "fsq_decode_attn_timed", "fsq_decode_step", "fsq_decode_attn_recon",
           "fsq_decode_attn_rope", "fsq_append_levels", "fsq_decode_attn_levels",
           "fsq_decode_attn_levels_timed", "fsq_decode_plan_info", "fsq_decode_attn_noalloc",
           "fsq_decode_step_levels")

NOALLOC_SCRATCH_BYTES = 32 << 20   # FSQ_NOALLOC_SCRATCH_BYTES in include/fsq.h

FSQ_OK, FSQ_ERR_NULL, FSQ_ERR_SHAPE, FSQ_ERR_UNSUPPORTED, FSQ_ERR_WORKSPACE, FSQ_ERR_HIP = range(6)

_lib = None


class FsqError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libfsq.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m fsq_latent_decode_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.fsq_status_string.argtypes = [ctypes.c_int]
        L.fsq_status_string.restype = ctypes.c_char_p
        L.fsq_append.argtypes = [vp, vp, vp, i64, i32, i32, vp]
        L.fsq_append.restype = ctypes.c_int
        L.fsq_decode_workspace_bytes.argtypes = [i32, i32, i32, i64]
        L.fsq_decode_workspace_bytes.restype = sz
        L.fsq_decode_attn.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i64, vp, sz, vp]
        L.fsq_decode_attn.restype = ctypes.c_int
        L.fsq_decode_attn_timed.argtypes = L.fsq_decode_attn.argtypes + [vp, vp]
        L.fsq_decode_attn_timed.restype = ctypes.c_int
        L.fsq_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i64,
                                      vp, sz, vp]
        L.fsq_decode_step.restype = ctypes.c_int
        L.fsq_decode_step_levels.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                             i64, vp, sz, vp]
        L.fsq_decode_step_levels.restype = ctypes.c_int
        L.fsq_decode_attn_recon.argtypes = L.fsq_decode_attn.argtypes
        L.fsq_decode_attn_recon.restype = ctypes.c_int
        L.fsq_decode_plan_info.argtypes = [i32, i32, i32, i64, vp, vp, vp]
        L.fsq_decode_plan_info.restype = ctypes.c_int
        L.fsq_append_levels.argtypes = [vp, vp, vp, i64, i32, i32, i32, vp]
        L.fsq_append_levels.restype = ctypes.c_int
        L.fsq_decode_attn_levels.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i64, vp, sz, vp]
        L.fsq_decode_attn_levels.restype = ctypes.c_int
        L.fsq_decode_attn_levels_timed.argtypes = L.fsq_decode_attn_levels.argtypes + [vp, vp]
        L.fsq_decode_attn_levels_timed.restype = ctypes.c_int
        L.fsq_decode_attn_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i64, vp]
        L.fsq_decode_attn_noalloc.restype = ctypes.c_int
        f32 = ctypes.c_float
        L.fsq_decode_attn_rope.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i64, f32, f32,
                                           vp, sz, vp]
        L.fsq_decode_attn_rope.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().fsq_status_string(int(status)).decode()


def _check(rc: int, what: str) -> None:
    if rc != FSQ_OK:
        raise FsqError(rc, what)


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return int(getattr(stream, "cuda_stream", stream))


def _stream_obj(stream):
    """The call's stream as a torch stream object (the current stream for None;
    a raw hipStream_t handle is wrapped, not copied)."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(getattr(stream, "cuda_stream", stream)))


def _call_workspace(workspace, B, n_q, G, cap, device, stream) -> torch.Tensor:
    """The caller's workspace, or a new one allocated on the call's stream.

    A workspace made here is freed when the call returns, while its kernels may
    still be queued. Allocating it under the call's stream hands the block back
    to the caching allocator as that stream's memory, so it is reused only by
    work ordered after those kernels on the same stream."""
    if workspace is None:
        with torch.cuda.stream(_stream_obj(stream)):
            workspace = alloc_workspace(B, n_q, G, cap, device)
    _dev(workspace, "workspace", torch.uint8, 1)
    return workspace


LEVEL_BITS = {4: 2, 16: 4, 256: 8}


def bytes_per_token(G: int, levels: int = 16) -> int:
    return (G * LEVEL_BITS[levels] + 7) // 8


def fsq_append(x: torch.Tensor, E: torch.Tensor, codes: torch.Tensor, stream=None,
               levels: int = 16) -> None:
    """codes[t] = pack(FSQ(E x[t])) for every row of x.

    x [n, C] bf16, E [G, C] bf16, codes [n, ceil(G b/8)] uint8 (may be a row range
    of a cache tensor, e.g. cache[b, T:T+n]); levels L = 4, 16 (default) or 256."""
    _dev(x, "x", torch.bfloat16, 2)
    _dev(E, "E", torch.bfloat16, 2)
    _dev(codes, "codes", torch.uint8, 2)
    n, C = x.shape
    G = E.shape[0]
    if levels not in LEVEL_BITS:
        raise ValueError(f"levels must be one of {sorted(LEVEL_BITS)}")
    if E.shape[1] != C:
        raise ValueError(f"E is {tuple(E.shape)} but x has C={C}")
    P = bytes_per_token(G, levels)
    if tuple(codes.shape) != (n, P):
        raise ValueError(f"codes must be [{n}, {P}], got {tuple(codes.shape)}")
    if levels == 16:
        rc = lib().fsq_append(x.data_ptr(), E.data_ptr(), codes.data_ptr(), n, C, G, _stream(stream))
    else:
        rc = lib().fsq_append_levels(x.data_ptr(), E.data_ptr(), codes.data_ptr(), n, C, G, levels,
                                     _stream(stream))
    _check(rc, "fsq_append")


def decode_workspace_bytes(batch: int, n_q: int, G: int, seq_cap: int) -> int:
    return int(lib().fsq_decode_workspace_bytes(batch, n_q, G, seq_cap))


def decode_plan(batch: int, n_q: int, G: int, seq_cap: int) -> dict:
    """The split-K plan of fsq_decode_attn for these sizes: kernel name, chunks per
    sequence and tokens per chunk (with device_split, the split is chosen on the
    device from the actual lengths: at most that many chunks of at least that
    many tokens)."""
    k, sp, ch = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    _check(lib().fsq_decode_plan_info(batch, n_q, G, seq_cap, ctypes.byref(k), ctypes.byref(sp),
                                      ctypes.byref(ch)), "fsq_decode_plan_info")
    return {"kernel": "decode_stream_kernel" if k.value else "decode_split_kernel",
            "device_split": k.value == 2, "splits": sp.value, "chunk": ch.value}


def alloc_workspace(batch: int, n_q: int, G: int, seq_cap: int, device="cuda") -> torch.Tensor:
    """A device buffer for fsq_decode_attn (torch allocations are 256-byte aligned)."""
    n = decode_workspace_bytes(batch, n_q, G, seq_cap)
    if n == 0:
        raise ValueError("invalid sizes for the decode workspace")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _check_decode_args(q, codes, W_kv, seq_lens, out, n_kv, levels=16):
    _dev(q, "q", torch.bfloat16, 3)
    _dev(codes, "codes", torch.uint8, 3)
    _dev(W_kv, "W_kv", torch.bfloat16, 2)
    _dev(seq_lens, "seq_lens", torch.int32, 1)
    _dev(out, "out", torch.bfloat16, 3)
    B, n_q, d_h = q.shape
    G = W_kv.shape[1]
    if codes.shape[0] != B or codes.shape[2] != bytes_per_token(G, levels):
        raise ValueError(f"codes must be [{B}, cap, {bytes_per_token(G, levels)}], got {tuple(codes.shape)}")
    if W_kv.shape[0] != 2 * n_kv * d_h:
        raise ValueError(f"W_kv must have {2 * n_kv * d_h} rows, got {W_kv.shape[0]}")
    if seq_lens.shape[0] != B or tuple(out.shape) != (B, n_q, d_h):
        raise ValueError("seq_lens / out shape mismatch")
    return B, n_q, d_h, G, codes.shape[1]


def fsq_decode_step(x_new: torch.Tensor, E: torch.Tensor, q: torch.Tensor, codes: torch.Tensor,
                    W_kv: torch.Tensor, seq_lens: torch.Tensor, out: torch.Tensor, n_kv: int,
                    workspace: torch.Tensor | None = None, stream=None, levels: int = 16) -> torch.Tensor:
    """One decode step of one layer: codes[b, seq_lens[b] - 1] = pack(FSQ(E x_new[b]))
    for every sequence with 1 <= seq_lens[b] <= cap, then out = attention over the
    cache as in fsq_decode_attn. seq_lens already counts the new token.

    x_new [B, C] bf16, E [G, C] bf16; the other arguments as fsq_decode_attn
    (levels = 4 / 256: 2- / 8-bit codes, as fsq_decode_attn_levels)."""
    if levels not in LEVEL_BITS:
        raise ValueError(f"levels must be one of {sorted(LEVEL_BITS)}")
    B, n_q, d_h, G, cap = _check_decode_args(q, codes, W_kv, seq_lens, out, n_kv, levels)
    _dev(x_new, "x_new", torch.bfloat16, 2)
    _dev(E, "E", torch.bfloat16, 2)
    C = x_new.shape[1]
    if x_new.shape[0] != B or tuple(E.shape) != (G, C):
        raise ValueError(f"x_new must be [{B}, C] and E [{G}, C], got {tuple(x_new.shape)}, "
                         f"{tuple(E.shape)}")
    workspace = _call_workspace(workspace, B, n_q, G, cap, q.device, stream)
    if levels == 16:
        rc = lib().fsq_decode_step(x_new.data_ptr(), E.data_ptr(), q.data_ptr(), codes.data_ptr(),
                                   W_kv.data_ptr(), seq_lens.data_ptr(), out.data_ptr(), B, C, n_q, n_kv,
                                   d_h, G, cap, workspace.data_ptr(), workspace.numel(), _stream(stream))
        _check(rc, "fsq_decode_step")
    else:
        rc = lib().fsq_decode_step_levels(x_new.data_ptr(), E.data_ptr(), q.data_ptr(), codes.data_ptr(),
                                          W_kv.data_ptr(), seq_lens.data_ptr(), out.data_ptr(), B, C, n_q,
                                          n_kv, d_h, G, levels, cap, workspace.data_ptr(), workspace.numel(),
                                          _stream(stream))
        _check(rc, "fsq_decode_step_levels")
    return out


def fsq_decode_attn_levels(q: torch.Tensor, codes: torch.Tensor, W_kv: torch.Tensor,
                           seq_lens: torch.Tensor, out: torch.Tensor, n_kv: int, levels: int,
                           workspace: torch.Tensor | None = None, stream=None,
                           split_events=None) -> torch.Tensor:
    """fsq_decode_attn over a cache of L = levels codes per coordinate (4, 16, 256):
    codes [B, cap, ceil(G b/8)] uint8, z = code - L/2. With split_events the call
    goes through fsq_decode_attn_levels_timed."""
    if levels not in LEVEL_BITS:
        raise ValueError(f"levels must be one of {sorted(LEVEL_BITS)}")
    B, n_q, d_h, G, cap = _check_decode_args(q, codes, W_kv, seq_lens, out, n_kv, levels)
    workspace = _call_workspace(workspace, B, n_q, G, cap, q.device, stream)
    args = (q.data_ptr(), codes.data_ptr(), W_kv.data_ptr(), seq_lens.data_ptr(), out.data_ptr(), B, n_q,
            n_kv, d_h, G, levels, cap, workspace.data_ptr(), workspace.numel(), _stream(stream))
    if split_events is None:
        _check(lib().fsq_decode_attn_levels(*args), "fsq_decode_attn_levels")
    else:
        ev = [_event_handle(e) for e in split_events]
        _check(lib().fsq_decode_attn_levels_timed(*args, ev[0], ev[1]), "fsq_decode_attn_levels_timed")
    return out


def fsq_decode_attn(q: torch.Tensor, codes: torch.Tensor, W_kv: torch.Tensor, seq_lens: torch.Tensor,
                    out: torch.Tensor, n_kv: int, workspace: torch.Tensor | None = None,
                    stream=None, split_events=None) -> torch.Tensor:
    """One decode step of attention over the packed cache; writes and returns out.

    q [B, n_q, d_h] bf16, codes [B, cap, ceil(G/2)] uint8, W_kv [2 n_kv d_h, G] bf16,
    seq_lens [B] int32 (device), out [B, n_q, d_h] bf16. With split_events =
    (start, stop) (torch.cuda.Event with timing) the call goes through
    fsq_decode_attn_timed and the events bracket the split-K kernel."""
    B, n_q, d_h, G, cap = _check_decode_args(q, codes, W_kv, seq_lens, out, n_kv)
    workspace = _call_workspace(workspace, B, n_q, G, cap, q.device, stream)
    args = (q.data_ptr(), codes.data_ptr(), W_kv.data_ptr(), seq_lens.data_ptr(), out.data_ptr(),
            B, n_q, n_kv, d_h, G, cap, workspace.data_ptr(), workspace.numel(), _stream(stream))
    if split_events is None:
        _check(lib().fsq_decode_attn(*args), "fsq_decode_attn")
    else:
        ev = [_event_handle(e) for e in split_events]
        _check(lib().fsq_decode_attn_timed(*args, ev[0], ev[1]), "fsq_decode_attn_timed")
    return out


def fsq_decode_attn_noalloc(q: torch.Tensor, codes: torch.Tensor, W_kv: torch.Tensor,
                            seq_lens: torch.Tensor, out: torch.Tensor, n_kv: int, stream=None) -> torch.Tensor:
    """fsq_decode_attn with the library's fixed per-GPU scratch area as the
    workspace (no allocation by the library or here): for callers that cannot
    allocate. Calls that may overlap on one GPU share that area and must be
    serialised by the caller. Raises FsqError (FSQ_ERR_WORKSPACE) when the sizes
    need more than NOALLOC_SCRATCH_BYTES of workspace."""
    B, n_q, d_h, G, cap = _check_decode_args(q, codes, W_kv, seq_lens, out, n_kv)
    rc = lib().fsq_decode_attn_noalloc(q.data_ptr(), codes.data_ptr(), W_kv.data_ptr(), seq_lens.data_ptr(),
                                       out.data_ptr(), B, n_q, n_kv, d_h, G, cap, _stream(stream))
    _check(rc, "fsq_decode_attn_noalloc")
    return out


def fsq_decode_attn_recon(q: torch.Tensor, codes: torch.Tensor, W_kv: torch.Tensor,
                          seq_lens: torch.Tensor, out: torch.Tensor, n_kv: int,
                          workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """fsq_decode_attn computed with keys rebuilt per tile (K = Z W_k^T) instead of
    absorbed queries: the measured comparison. Same arguments and workspace."""
    B, n_q, d_h, G, cap = _check_decode_args(q, codes, W_kv, seq_lens, out, n_kv)
    workspace = _call_workspace(workspace, B, n_q, G, cap, q.device, stream)
    rc = lib().fsq_decode_attn_recon(q.data_ptr(), codes.data_ptr(), W_kv.data_ptr(),
                                     seq_lens.data_ptr(), out.data_ptr(), B, n_q, n_kv, d_h, G, cap,
                                     workspace.data_ptr(), workspace.numel(), _stream(stream))
    _check(rc, "fsq_decode_attn_recon")
    return out


def fsq_decode_attn_rope(q: torch.Tensor, codes: torch.Tensor, W_kv: torch.Tensor,
                         k_norm: torch.Tensor, seq_lens: torch.Tensor, out: torch.Tensor, n_kv: int,
                         rope_theta: float, norm_eps: float, workspace: torch.Tensor | None = None,
                         stream=None) -> torch.Tensor:
    """Decode with Eq. 5 keys in full: k^_t = RoPE_t(N_k(W_k z_t)) rebuilt per tile.
    k_norm [d_h] bf16 is the key-norm gain; q is already normalised and rotated.
    Other arguments as fsq_decode_attn."""
    B, n_q, d_h, G, cap = _check_decode_args(q, codes, W_kv, seq_lens, out, n_kv)
    _dev(k_norm, "k_norm", torch.bfloat16, 1)
    if k_norm.shape[0] != d_h:
        raise ValueError(f"k_norm must be [{d_h}], got {tuple(k_norm.shape)}")
    workspace = _call_workspace(workspace, B, n_q, G, cap, q.device, stream)
    rc = lib().fsq_decode_attn_rope(q.data_ptr(), codes.data_ptr(), W_kv.data_ptr(), k_norm.data_ptr(),
                                    seq_lens.data_ptr(), out.data_ptr(), B, n_q, n_kv, d_h, G, cap,
                                    float(rope_theta), float(norm_eps), workspace.data_ptr(),
                                    workspace.numel(), _stream(stream))
    _check(rc, "fsq_decode_attn_rope")
    return out


def _event_handle(ev) -> int:
    """The hipEvent_t behind a torch.cuda.Event (created on first record)."""
    if ev.cuda_event == 0:          # torch creates the event lazily
        ev.record()
    return ev.cuda_event
