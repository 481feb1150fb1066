"""Python binding of the MSA block-sparse attention library (libmsa.so, gfx950).

Argument marshalling only: torch provides device memory and the current HIP
stream; every step of the computation runs in the HIP kernels behind the C
ABI of include/msa.h.  There is no CPU fallback: without the built library
(or without a GPU) these functions raise.

    prob = Problem.from_lengths(len_q, len_kv, H, G, d, d_idx, B, k, "bf16", device)
    scores = index_score(prob, q_idx, k_idx)          # msa_index_score
    block_idx = topk_select(prob, scores)             # msa_topk_select
    out, lse = sparse_attn_fwd(prob, q, k, v, block_idx, return_lse=True)

Training support (the indexer's KL objective over the kept blocks):

    out, lse, mass = sparse_attn_fwd_mass(prob, q, k, v, block_idx)   # bf16 prefill
    kl, grad = indexer_kl(prob, scores, block_idx, mass)    # d kl / d scores
    dq_idx, dk_idx = indexer_bwd(prob, q_idx, k_idx, block_idx, grad)
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsa.so")
# Debug build: every index-driven gather is bounds-checked and failures are
# counted on the device (read them with debug_bounds_violations()).
DEBUG_LIB_PATH = os.path.join(_HERE, "libmsa_debug.so")

MSA_SUCCESS = 0
STATUS_NAMES = {0: "MSA_SUCCESS", 1: "MSA_ERR_NULL_POINTER", 2: "MSA_ERR_BAD_SHAPE",
                3: "MSA_ERR_UNSUPPORTED_DTYPE", 4: "MSA_ERR_MISALIGNED",
                5: "MSA_ERR_WORKSPACE_TOO_SMALL", 6: "MSA_ERR_DEVICE",
                7: "MSA_ERR_NOT_AVAILABLE"}
DTYPES = {"bf16": 0, "f32": 1}
SCHEDULES = {"auto": 0, "query_major": 1, "kv_major": 2}
EXPORTED = ("msa_index_score", "msa_topk_select", "msa_index_topk_workspace_size",
            "msa_index_topk", "msa_index_topk_hier_workspace_size", "msa_index_topk_hier",
            "msa_sparse_attn_workspace_size", "msa_sparse_attn_workspace_size_min",
            "msa_sparse_attn_rows_per_pass",
            "msa_sparse_attn_fwd", "msa_sparse_attn_fwd_noalloc", "msa_sparse_attn_fwd_mass",
            "msa_indexer_kl",
            "msa_indexer_bwd_workspace_size", "msa_indexer_bwd",
            "msa_sparse_attn_bwd_workspace_size", "msa_sparse_attn_bwd_workspace_size_min",
            "msa_sparse_attn_bwd_rows_per_pass", "msa_sparse_attn_bwd",
            "msa_set_profile_events", "msa_debug_bounds_violations", "msa_status_string",
            "msa_last_error_message", "msa_abi_version")


class MsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class CProblem(ctypes.Structure):
    """Mirror of msa_problem_t (include/msa.h)."""
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_groups", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("idx_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("schedule", ctypes.c_int32),
        ("max_q_len", ctypes.c_int32),
        ("max_kv_len", ctypes.c_int64),
        ("total_q", ctypes.c_int64),
        ("total_kv", ctypes.c_int64),
        ("softmax_scale", ctypes.c_float),
        ("cu_q", ctypes.c_void_p),
        ("cu_kv", ctypes.c_void_p),
    ]


_lib_handle = None
_lib_path = None
_loaded = {}


def _default_path() -> str:
    """libmsa.so, or libmsa_debug.so when MSA_LIBRARY=debug is set."""
    v = os.environ.get("MSA_LIBRARY", "release")
    if v not in ("release", "debug"):
        raise RuntimeError(f"MSA_LIBRARY must be 'release' or 'debug', not {v!r}")
    return DEBUG_LIB_PATH if v == "debug" else LIB_PATH


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """The library every call of this module goes through, loaded on first
    use (libmsa.so unless select_library() or MSA_LIBRARY chose another).
    Raises if it has not been built."""
    if _lib_handle is not None and path is None:
        return _lib_handle
    return select_library(path or _default_path())


def select_library(path: str) -> ctypes.CDLL:
    """Route every later call of this module through the library at `path`
    (LIB_PATH or DEBUG_LIB_PATH); both may be loaded in one process."""
    global _lib_handle, _lib_path
    lib = _loaded.get(path)
    if lib is None:
        lib = _open(path)
        _loaded[path] = lib
    _lib_handle, _lib_path = lib, path
    return lib


def current_library_path() -> Optional[str]:
    return _lib_path


def _open(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m block_sparse_long_msa_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(CProblem)
    vp, st = ctypes.c_void_p, ctypes.c_int
    lib.msa_index_score.argtypes = [P, vp, vp, vp, vp]
    lib.msa_index_score.restype = st
    lib.msa_topk_select.argtypes = [P, vp, vp, vp]
    lib.msa_topk_select.restype = st
    lib.msa_index_topk_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.msa_index_topk_workspace_size.restype = st
    lib.msa_index_topk.argtypes = [P, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.msa_index_topk.restype = st
    lib.msa_index_topk_hier_workspace_size.argtypes = [P, ctypes.c_int, ctypes.c_int,
                                                       ctypes.POINTER(ctypes.c_size_t)]
    lib.msa_index_topk_hier_workspace_size.restype = st
    lib.msa_index_topk_hier.argtypes = [P, vp, vp, ctypes.c_int, ctypes.c_int, vp, vp, vp,
                                        ctypes.c_size_t, vp]
    lib.msa_index_topk_hier.restype = st
    lib.msa_sparse_attn_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.msa_sparse_attn_workspace_size.restype = st
    lib.msa_sparse_attn_workspace_size_min.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.msa_sparse_attn_workspace_size_min.restype = st
    lib.msa_sparse_attn_rows_per_pass.argtypes = [P, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int64)]
    lib.msa_sparse_attn_rows_per_pass.restype = st
    lib.msa_sparse_attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.msa_sparse_attn_fwd.restype = st
    lib.msa_sparse_attn_fwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    lib.msa_sparse_attn_fwd_noalloc.restype = st
    lib.msa_sparse_attn_fwd_mass.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.msa_sparse_attn_fwd_mass.restype = st
    lib.msa_indexer_kl.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.msa_indexer_kl.restype = st
    lib.msa_indexer_bwd_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.msa_indexer_bwd_workspace_size.restype = st
    lib.msa_indexer_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.msa_indexer_bwd.restype = st
    lib.msa_sparse_attn_bwd_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.msa_sparse_attn_bwd_workspace_size.restype = st
    lib.msa_sparse_attn_bwd_workspace_size_min.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.msa_sparse_attn_bwd_workspace_size_min.restype = st
    lib.msa_sparse_attn_bwd_rows_per_pass.argtypes = [P, ctypes.c_size_t,
                                                      ctypes.POINTER(ctypes.c_int64)]
    lib.msa_sparse_attn_bwd_rows_per_pass.restype = st
    lib.msa_sparse_attn_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        ctypes.c_size_t, vp]
    lib.msa_sparse_attn_bwd.restype = st
    lib.msa_status_string.argtypes = [st]
    lib.msa_status_string.restype = ctypes.c_char_p
    lib.msa_last_error_message.argtypes = []
    lib.msa_last_error_message.restype = ctypes.c_char_p
    lib.msa_abi_version.argtypes = []
    lib.msa_abi_version.restype = ctypes.c_int
    lib.msa_set_profile_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    lib.msa_set_profile_events.restype = None
    lib.msa_debug_bounds_violations.argtypes = [ctypes.POINTER(ctypes.c_uint64),
                                                ctypes.POINTER(ctypes.c_uint64), st]
    lib.msa_debug_bounds_violations.restype = st
    return lib


def _check(status: int) -> None:
    if status != MSA_SUCCESS:
        msg = load_library().msa_last_error_message().decode()
        raise MsaError(status, msg)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


class Problem:
    """Shapes of one call sequence; owns the device offset arrays it points to."""

    def __init__(self, cu_q: torch.Tensor, cu_kv: torch.Tensor, len_q: Sequence[int],
                 len_kv: Sequence[int], num_q_heads: int, num_kv_groups: int, head_dim: int,
                 idx_dim: int, block_size: int, top_k: int, dtype: str = "bf16",
                 softmax_scale: Optional[float] = None, schedule: str = "auto"):
        if len(len_q) != len(len_kv):
            raise ValueError(f"len_q and len_kv need one entry per sequence "
                             f"(got {len(len_q)} and {len(len_kv)})")
        for name, cu in (("cu_q", cu_q), ("cu_kv", cu_kv)):
            if (cu.dtype != torch.int64 or not cu.is_cuda or not cu.is_contiguous()
                    or cu.numel() != len(len_q) + 1):
                raise ValueError(f"{name}: expected {len(len_q) + 1} contiguous int64 offsets on "
                                 f"the GPU, got {cu.dtype} {tuple(cu.shape)} on {cu.device}")
        self.cu_q, self.cu_kv = cu_q, cu_kv            # keep alive
        self.len_q, self.len_kv = list(len_q), list(len_kv)
        self.H, self.G, self.d, self.d_idx = num_q_heads, num_kv_groups, head_dim, idx_dim
        self.B, self.top_k, self.dtype = block_size, top_k, dtype
        self.scale = 1.0 / math.sqrt(head_dim) if softmax_scale is None else softmax_scale
        self.max_q_len = max(self.len_q) if self.len_q else 0
        self.max_kv_len = max(self.len_kv) if self.len_kv else 0
        self.total_q, self.total_kv = sum(self.len_q), sum(self.len_kv)
        self.nb_max = -(-self.max_kv_len // block_size)
        self.c = CProblem(len(self.len_q), num_q_heads, num_kv_groups, head_dim, idx_dim,
                          block_size, top_k, DTYPES[dtype], SCHEDULES[schedule], self.max_q_len,
                          self.max_kv_len, self.total_q, self.total_kv, self.scale,
                          cu_q.data_ptr(), cu_kv.data_ptr())

    @classmethod
    def from_lengths(cls, len_q, len_kv, num_q_heads, num_kv_groups, head_dim, idx_dim,
                     block_size, top_k, dtype="bf16", device="cuda", **kw) -> "Problem":
        cu_q = [0]
        cu_kv = [0]
        for a, b in zip(len_q, len_kv):
            cu_q.append(cu_q[-1] + a)
            cu_kv.append(cu_kv[-1] + b)
        dev = torch.device(device)
        return cls(torch.tensor(cu_q, dtype=torch.int64, device=dev),
                   torch.tensor(cu_kv, dtype=torch.int64, device=dev), len_q, len_kv,
                   num_q_heads, num_kv_groups, head_dim, idx_dim, block_size, top_k, dtype, **kw)

    def with_schedule(self, schedule: str) -> "Problem":
        return Problem(self.cu_q, self.cu_kv, self.len_q, self.len_kv, self.H, self.G, self.d,
                       self.d_idx, self.B, self.top_k, self.dtype, self.scale, schedule)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def ref(self):
        return ctypes.byref(self.c)


def _need(t: torch.Tensor, name: str, shape, dtype) -> None:
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on the GPU, got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device}")


def index_score(prob: Problem, q_idx: torch.Tensor, k_idx: torch.Tensor,
                scores: Optional[torch.Tensor] = None, stream: Optional[int] = None) -> torch.Tensor:
    """msa_index_score: block scores [G, total_q, NBmax] fp32."""
    _need(q_idx, "q_idx", (prob.total_q, prob.G, prob.d_idx), prob.torch_dtype)
    _need(k_idx, "k_idx", (prob.total_kv, prob.G, prob.d_idx), prob.torch_dtype)
    if scores is None:
        scores = torch.empty((prob.G, prob.total_q, prob.nb_max), dtype=torch.float32,
                             device=q_idx.device)
    _need(scores, "scores", (prob.G, prob.total_q, prob.nb_max), torch.float32)
    s = _stream(q_idx.device) if stream is None else stream
    _check(load_library().msa_index_score(prob.ref(), _ptr(q_idx), _ptr(k_idx), _ptr(scores), s))
    return scores


def topk_select(prob: Problem, scores: torch.Tensor, block_idx: Optional[torch.Tensor] = None,
                stream: Optional[int] = None) -> torch.Tensor:
    """msa_topk_select: kept blocks [G, total_q, k] int32, ascending, -1 padded."""
    _need(scores, "scores", (prob.G, prob.total_q, prob.nb_max), torch.float32)
    if block_idx is None:
        block_idx = torch.empty((prob.G, prob.total_q, prob.top_k), dtype=torch.int32,
                                device=scores.device)
    _need(block_idx, "block_idx", (prob.G, prob.total_q, prob.top_k), torch.int32)
    s = _stream(scores.device) if stream is None else stream
    _check(load_library().msa_topk_select(prob.ref(), _ptr(scores), _ptr(block_idx), s))
    return block_idx


def index_topk_workspace_size(prob: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().msa_index_topk_workspace_size(prob.ref(), ctypes.byref(n)))
    return n.value


def index_topk(prob: Problem, q_idx: torch.Tensor, k_idx: torch.Tensor,
               block_idx: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               stream: Optional[int] = None) -> torch.Tensor:
    """msa_index_topk: the kept blocks [G, total_q, k] int32 straight from the
    index tensors (index scoring and Top-k fused; no score tensor)."""
    _need(q_idx, "q_idx", (prob.total_q, prob.G, prob.d_idx), prob.torch_dtype)
    _need(k_idx, "k_idx", (prob.total_kv, prob.G, prob.d_idx), prob.torch_dtype)
    if block_idx is None:
        block_idx = torch.empty((prob.G, prob.total_q, prob.top_k), dtype=torch.int32,
                                device=q_idx.device)
    _need(block_idx, "block_idx", (prob.G, prob.total_q, prob.top_k), torch.int32)
    need = index_topk_workspace_size(prob)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_idx.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    s = _stream(q_idx.device) if stream is None else stream
    _check(load_library().msa_index_topk(prob.ref(), _ptr(q_idx), _ptr(k_idx), _ptr(block_idx),
                                         _ptr(workspace), wbytes, s))
    return block_idx


def index_topk_hier_workspace_size(prob: Problem, chunk_blocks: int, keep_chunks: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().msa_index_topk_hier_workspace_size(prob.ref(), chunk_blocks,
                                                             keep_chunks, ctypes.byref(n)))
    return n.value


def index_topk_hier(prob: Problem, q_idx: torch.Tensor, k_idx: torch.Tensor, chunk_blocks: int,
                    keep_chunks: int, block_idx: Optional[torch.Tensor] = None,
                    kept_chunks: Optional[torch.Tensor] = None, return_kept: bool = False,
                    workspace: Optional[torch.Tensor] = None, stream: Optional[int] = None):
    """msa_index_topk_hier: the hierarchical (coarse-to-fine) selection.
    Returns block_idx [G, total_q, k] int32, and with return_kept (or a given
    kept_chunks buffer) also the kept chunks [G, total_q, keep_chunks]."""
    _need(q_idx, "q_idx", (prob.total_q, prob.G, prob.d_idx), prob.torch_dtype)
    _need(k_idx, "k_idx", (prob.total_kv, prob.G, prob.d_idx), prob.torch_dtype)
    if block_idx is None:
        block_idx = torch.empty((prob.G, prob.total_q, prob.top_k), dtype=torch.int32,
                                device=q_idx.device)
    _need(block_idx, "block_idx", (prob.G, prob.total_q, prob.top_k), torch.int32)
    if kept_chunks is None and return_kept:
        kept_chunks = torch.empty((prob.G, prob.total_q, keep_chunks), dtype=torch.int32,
                                  device=q_idx.device)
    if kept_chunks is not None:
        _need(kept_chunks, "kept_chunks", (prob.G, prob.total_q, keep_chunks), torch.int32)
    need = index_topk_hier_workspace_size(prob, chunk_blocks, keep_chunks)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_idx.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    s = _stream(q_idx.device) if stream is None else stream
    _check(load_library().msa_index_topk_hier(prob.ref(), _ptr(q_idx), _ptr(k_idx), chunk_blocks,
                                              keep_chunks, _ptr(block_idx), _ptr(kept_chunks),
                                              _ptr(workspace), wbytes, s))
    if kept_chunks is not None:
        return block_idx, kept_chunks
    return block_idx


def workspace_size(prob: Problem) -> int:
    """msa_sparse_attn_workspace_size: bytes with which the forward runs at
    full speed (long KV-major prefills then run in passes of the library's
    preferred size; more workspace is not used)."""
    n = ctypes.c_size_t(0)
    _check(load_library().msa_sparse_attn_workspace_size(prob.ref(), ctypes.byref(n)))
    return n.value


def workspace_size_min(prob: Problem) -> int:
    """msa_sparse_attn_workspace_size_min: the least workspace the forward
    calls accept (the KV-major schedule runs in smaller passes below
    workspace_size)."""
    n = ctypes.c_size_t(0)
    _check(load_library().msa_sparse_attn_workspace_size_min(prob.ref(), ctypes.byref(n)))
    return n.value


def rows_per_pass(prob: Problem, workspace_bytes: int) -> int:
    """msa_sparse_attn_rows_per_pass: query rows per pass of the forward with
    a workspace of that many bytes."""
    n = ctypes.c_int64(0)
    _check(load_library().msa_sparse_attn_rows_per_pass(prob.ref(), workspace_bytes,
                                                        ctypes.byref(n)))
    return n.value


def sparse_attn_fwd(prob: Problem, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    block_idx: torch.Tensor, out: Optional[torch.Tensor] = None,
                    return_lse: bool = False, workspace: Optional[torch.Tensor] = None,
                    stream: Optional[int] = None, lse: Optional[torch.Tensor] = None
                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """msa_sparse_attn_fwd: (out [total_q, H, d], lse [total_q, H] or None).
    The LSE is written when return_lse is set or an `lse` buffer is given."""
    dt = prob.torch_dtype
    _need(q, "q", (prob.total_q, prob.H, prob.d), dt)
    _need(k, "k", (prob.total_kv, prob.G, prob.d), dt)
    _need(v, "v", (prob.total_kv, prob.G, prob.d), dt)
    _need(block_idx, "block_idx", (prob.G, prob.total_q, prob.top_k), torch.int32)
    if out is None:
        out = torch.empty((prob.total_q, prob.H, prob.d), dtype=dt, device=q.device)
    _need(out, "out", (prob.total_q, prob.H, prob.d), dt)
    if lse is None and return_lse:
        lse = torch.empty((prob.total_q, prob.H), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", (prob.total_q, prob.H), torch.float32)
    need = workspace_size(prob)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    s = _stream(q.device) if stream is None else stream
    _check(load_library().msa_sparse_attn_fwd(prob.ref(), _ptr(q), _ptr(k), _ptr(v),
                                              _ptr(block_idx), _ptr(out), _ptr(lse),
                                              _ptr(workspace), wbytes, s))
    return out, lse


def sparse_attn_fwd_noalloc(prob: Problem, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                            block_idx: torch.Tensor, out: Optional[torch.Tensor] = None,
                            return_lse: bool = False, stream: Optional[int] = None,
                            lse: Optional[torch.Tensor] = None
                            ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """msa_sparse_attn_fwd_noalloc: sparse_attn_fwd on the library's fixed
    device scratch instead of a workspace (the library allocates nothing;
    outputs are allocated here only when not given)."""
    dt = prob.torch_dtype
    _need(q, "q", (prob.total_q, prob.H, prob.d), dt)
    _need(k, "k", (prob.total_kv, prob.G, prob.d), dt)
    _need(v, "v", (prob.total_kv, prob.G, prob.d), dt)
    _need(block_idx, "block_idx", (prob.G, prob.total_q, prob.top_k), torch.int32)
    if out is None:
        out = torch.empty((prob.total_q, prob.H, prob.d), dtype=dt, device=q.device)
    _need(out, "out", (prob.total_q, prob.H, prob.d), dt)
    if lse is None and return_lse:
        lse = torch.empty((prob.total_q, prob.H), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", (prob.total_q, prob.H), torch.float32)
    s = _stream(q.device) if stream is None else stream
    _check(load_library().msa_sparse_attn_fwd_noalloc(prob.ref(), _ptr(q), _ptr(k), _ptr(v),
                                                      _ptr(block_idx), _ptr(out), _ptr(lse), s))
    return out, lse


def sparse_attn_fwd_mass(prob: Problem, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         block_idx: torch.Tensor, out: Optional[torch.Tensor] = None,
                         lse: Optional[torch.Tensor] = None, mass: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream: Optional[int] = None
                         ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """msa_sparse_attn_fwd_mass: (out [total_q, H, d], lse [total_q, H],
    block_mass [G, total_q, k] fp32)."""
    dt = prob.torch_dtype
    _need(q, "q", (prob.total_q, prob.H, prob.d), dt)
    _need(k, "k", (prob.total_kv, prob.G, prob.d), dt)
    _need(v, "v", (prob.total_kv, prob.G, prob.d), dt)
    _need(block_idx, "block_idx", (prob.G, prob.total_q, prob.top_k), torch.int32)
    if out is None:
        out = torch.empty((prob.total_q, prob.H, prob.d), dtype=dt, device=q.device)
    if lse is None:
        lse = torch.empty((prob.total_q, prob.H), dtype=torch.float32, device=q.device)
    if mass is None:
        mass = torch.empty((prob.G, prob.total_q, prob.top_k), dtype=torch.float32,
                           device=q.device)
    _need(out, "out", (prob.total_q, prob.H, prob.d), dt)
    _need(lse, "lse", (prob.total_q, prob.H), torch.float32)
    _need(mass, "block_mass", (prob.G, prob.total_q, prob.top_k), torch.float32)
    need = workspace_size(prob)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    s = _stream(q.device) if stream is None else stream
    _check(load_library().msa_sparse_attn_fwd_mass(prob.ref(), _ptr(q), _ptr(k), _ptr(v),
                                                   _ptr(block_idx), _ptr(out), _ptr(lse),
                                                   _ptr(mass), _ptr(workspace), wbytes, s))
    return out, lse, mass


def indexer_kl(prob: Problem, scores: torch.Tensor, block_idx: torch.Tensor,
               block_mass: torch.Tensor, kl: Optional[torch.Tensor] = None,
               grad: Optional[torch.Tensor] = None, stream: Optional[int] = None
               ) -> Tuple[torch.Tensor, torch.Tensor]:
    """msa_indexer_kl: (kl [G, total_q], grad [G, total_q, k]) fp32."""
    _need(scores, "scores", (prob.G, prob.total_q, prob.nb_max), torch.float32)
    _need(block_idx, "block_idx", (prob.G, prob.total_q, prob.top_k), torch.int32)
    _need(block_mass, "block_mass", (prob.G, prob.total_q, prob.top_k), torch.float32)
    if kl is None:
        kl = torch.empty((prob.G, prob.total_q), dtype=torch.float32, device=scores.device)
    if grad is None:
        grad = torch.empty((prob.G, prob.total_q, prob.top_k), dtype=torch.float32,
                           device=scores.device)
    _need(kl, "kl", (prob.G, prob.total_q), torch.float32)
    _need(grad, "grad", (prob.G, prob.total_q, prob.top_k), torch.float32)
    s = _stream(scores.device) if stream is None else stream
    _check(load_library().msa_indexer_kl(prob.ref(), _ptr(scores), _ptr(block_idx),
                                         _ptr(block_mass), _ptr(kl), _ptr(grad), s))
    return kl, grad


def indexer_bwd(prob: Problem, q_idx: torch.Tensor, k_idx: torch.Tensor,
                block_idx: torch.Tensor, grad: torch.Tensor,
                workspace: Optional[torch.Tensor] = None, stream: Optional[int] = None
                ) -> Tuple[torch.Tensor, torch.Tensor]:
    """msa_indexer_bwd: (dq_idx [total_q, G, d_idx], dk_idx [total_kv, G, d_idx]) fp32,
    the max-pooling backward of the kept slots' score gradients `grad`."""
    dt = prob.torch_dtype
    _need(q_idx, "q_idx", (prob.total_q, prob.G, prob.d_idx), dt)
    _need(k_idx, "k_idx", (prob.total_kv, prob.G, prob.d_idx), dt)
    _need(block_idx, "block_idx", (prob.G, prob.total_q, prob.top_k), torch.int32)
    _need(grad, "grad", (prob.G, prob.total_q, prob.top_k), torch.float32)
    dq = torch.empty((prob.total_q, prob.G, prob.d_idx), dtype=torch.float32, device=q_idx.device)
    dk = torch.empty((prob.total_kv, prob.G, prob.d_idx), dtype=torch.float32, device=q_idx.device)
    n = ctypes.c_size_t(0)
    _check(load_library().msa_indexer_bwd_workspace_size(prob.ref(), ctypes.byref(n)))
    if workspace is None and n.value > 0:
        workspace = torch.empty(n.value, dtype=torch.uint8, device=q_idx.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    s = _stream(q_idx.device) if stream is None else stream
    _check(load_library().msa_indexer_bwd(prob.ref(), _ptr(q_idx), _ptr(k_idx), _ptr(block_idx),
                                          _ptr(grad), _ptr(dq), _ptr(dk), _ptr(workspace), wbytes,
                                          s))
    return dq, dk


def sparse_attn_bwd_workspace_size(prob: Problem, minimum: bool = False) -> int:
    """msa_sparse_attn_bwd_workspace_size (single pass), or with `minimum`
    msa_sparse_attn_bwd_workspace_size_min (the least accepted)."""
    n = ctypes.c_size_t(0)
    lib = load_library()
    fn = lib.msa_sparse_attn_bwd_workspace_size_min if minimum else lib.msa_sparse_attn_bwd_workspace_size
    _check(fn(prob.ref(), ctypes.byref(n)))
    return n.value


def sparse_attn_bwd_rows_per_pass(prob: Problem, workspace_bytes: int) -> int:
    """msa_sparse_attn_bwd_rows_per_pass: query rows per pass of the backward
    with a workspace of that many bytes."""
    n = ctypes.c_int64(0)
    _check(load_library().msa_sparse_attn_bwd_rows_per_pass(prob.ref(), workspace_bytes,
                                                            ctypes.byref(n)))
    return n.value


def sparse_attn_bwd(prob: Problem, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    block_idx: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
                    dout: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                    stream: Optional[int] = None
                    ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """msa_sparse_attn_bwd: (dq [total_q, H, d], dk [total_kv, G, d], dv [total_kv, G, d])
    fp32, the Main Branch backward for the upstream gradient `dout`, given the
    forward's `out` and `lse` on the same inputs."""
    dt = prob.torch_dtype
    _need(q, "q", (prob.total_q, prob.H, prob.d), dt)
    _need(k, "k", (prob.total_kv, prob.G, prob.d), dt)
    _need(v, "v", (prob.total_kv, prob.G, prob.d), dt)
    _need(block_idx, "block_idx", (prob.G, prob.total_q, prob.top_k), torch.int32)
    _need(out, "out", (prob.total_q, prob.H, prob.d), dt)
    _need(lse, "lse", (prob.total_q, prob.H), torch.float32)
    _need(dout, "dout", (prob.total_q, prob.H, prob.d), dt)
    dq = torch.empty((prob.total_q, prob.H, prob.d), dtype=torch.float32, device=q.device)
    dk = torch.empty((prob.total_kv, prob.G, prob.d), dtype=torch.float32, device=q.device)
    dv = torch.empty((prob.total_kv, prob.G, prob.d), dtype=torch.float32, device=q.device)
    n = ctypes.c_size_t(0)
    _check(load_library().msa_sparse_attn_bwd_workspace_size(prob.ref(), ctypes.byref(n)))
    if workspace is None and n.value > 0:
        workspace = torch.empty(n.value, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    s = _stream(q.device) if stream is None else stream
    _check(load_library().msa_sparse_attn_bwd(prob.ref(), _ptr(q), _ptr(k), _ptr(v),
                                              _ptr(block_idx), _ptr(out), _ptr(lse), _ptr(dout),
                                              _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                              wbytes, s))
    return dq, dk, dv


def debug_bounds_violations(reset: bool = True) -> Tuple[int, int]:
    """msa_debug_bounds_violations: (failed, run) gather bounds checks counted
    on the current device since the last reset (the debug library only; the
    release one raises MSA_ERR_NOT_AVAILABLE).  Synchronises the device first."""
    torch.cuda.synchronize()
    v, c = ctypes.c_uint64(0), ctypes.c_uint64(0)
    _check(load_library().msa_debug_bounds_violations(ctypes.byref(v), ctypes.byref(c),
                                                      int(bool(reset))))
    return int(v.value), int(c.value)


class ProfileEvents:
    """Per-kernel timing via msa_set_profile_events: `with ProfileEvents(n) as ev:`
    around one library call; afterwards ev.events[i] was recorded right after
    the call's i-th kernel launch (torch.cuda.Event objects)."""

    def __init__(self, n: int, device=None):
        dev = torch.device("cuda") if device is None else torch.device(device)
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        stream = torch.cuda.current_stream(dev)
        for e in self.events:          # torch creates the HIP event on first record
            e.record(stream)
        self._arr = (ctypes.c_void_p * n)(*[e.cuda_event for e in self.events])

    def __enter__(self):
        load_library().msa_set_profile_events(self._arr, len(self.events))
        return self

    def __exit__(self, *exc):
        load_library().msa_set_profile_events(None, 0)
        return False


def msa_forward(prob: Problem, q, k, v, q_idx, k_idx, return_lse: bool = False):
    """The whole path: index_score -> topk_select -> sparse_attn_fwd."""
    scores = index_score(prob, q_idx, k_idx)
    block_idx = topk_select(prob, scores)
    out, lse = sparse_attn_fwd(prob, q, k, v, block_idx, return_lse=return_lse)
    return out, lse, block_idx, scores


# Names matching the C entry points.
msa_index_score = index_score
msa_topk_select = topk_select
msa_index_topk = index_topk
msa_index_topk_hier = index_topk_hier
msa_sparse_attn_fwd = sparse_attn_fwd
msa_sparse_attn_fwd_noalloc = sparse_attn_fwd_noalloc
msa_sparse_attn_fwd_mass = sparse_attn_fwd_mass
msa_indexer_kl = indexer_kl
msa_indexer_bwd = indexer_bwd
msa_sparse_attn_bwd = sparse_attn_bwd
