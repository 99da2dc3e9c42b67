"""MiniMax Sparse Attention (MSA) forward pass on AMD MI355X (gfx950).

Thin ctypes binding of ``include/msa.h`` (``libmsa.so``): argument marshalling
only.  Every step of the computation runs in the library's HIP kernels; torch
supplies device memory and the stream.  If the library has not been built the
import of a compute entry point raises; nothing falls back to another path.

Entry points (same names as the C ABI, without the ``msa_`` prefix):
``index_scores``, ``block_topk``, ``sparse_attn_fwd``, ``forward``,
``index_kl``, ``dense_attn_fwd``, ``dense_index_kl``, ``sparse_attn_bwd``, ``index_kl_bwd``,
``forward_noalloc``, ``workspace_size``; ``Problem`` mirrors ``msa_problem``.  Each compute call
takes an optional ``varlen`` (a ``Varlen``, mirroring ``msa_varlen``: per
sequence query and cache lengths, packed query rows, a page table); given,
the ``*_v`` variant of the C call is used.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsa.so")

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_WORKSPACE_TOO_SMALL, ERR_HIP = range(5)
OP_INDEX_SCORES, OP_BLOCK_TOPK, OP_SPARSE_ATTN, OP_FORWARD, OP_INDEX_KL, OP_SPARSE_ATTN_BWD, OP_INDEX_KL_BWD = range(7)
DTYPE_BF16, DTYPE_FP8_E4M3 = range(2)  # msa_dtype: element type of index_q / index_k
DEFAULT_CHUNK_ROWS, CHUNK_ALIGN = 131072, 8192  # MSA_DEFAULT_CHUNK_ROWS, MSA_CHUNK_ALIGN

EXPORTS = ("msa_workspace_size", "msa_index_scores", "msa_block_topk", "msa_sparse_attn_fwd", "msa_forward",
           "msa_index_scores_v", "msa_block_topk_v", "msa_sparse_attn_fwd_v", "msa_forward_v", "msa_index_kl",
           "msa_dense_attn_fwd", "msa_dense_index_kl", "msa_sparse_attn_bwd", "msa_index_kl_bwd",
           "msa_index_kl_teacher", "msa_index_kl_bwd_teacher", "msa_forward_noalloc", "msa_forward_marked",
           "msa_status_string")
NOALLOC_SCRATCH_BYTES = 128 << 20  # MSA_NOALLOC_SCRATCH_BYTES


class Problem(ctypes.Structure):
    """msa_problem: one MSA problem instance (see include/msa.h)."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_kv", ctypes.c_int32),
        ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("index_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("q_offset", ctypes.c_int64),
        ("softmax_scale", ctypes.c_float),
        ("index_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("chunk_rows", ctypes.c_int32),
    ]

    @classmethod
    def make(cls, batch, n_q, n_kv, h_q, h_kv, head_dim=128, index_dim=128, block_size=128, topk=16,
             q_offset=-1, softmax_scale=None, index_dtype=DTYPE_BF16, kv_dtype=DTYPE_BF16, chunk_rows=0):
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(head_dim)
        return cls(batch, n_q, n_kv, h_q, h_kv, head_dim, index_dim, block_size, topk, q_offset, softmax_scale,
                   index_dtype, kv_dtype, chunk_rows)

    @property
    def offset(self) -> int:
        return self.n_kv - self.n_q if self.q_offset == -1 else self.q_offset

    @property
    def n_blk(self) -> int:
        return -(-self.n_kv // self.block_size)


class Varlen(ctypes.Structure):
    """msa_varlen: variable-length batches and paged caches (device pointers)."""
    _fields_ = [
        ("qo_lens", ctypes.c_void_p), ("kv_lens", ctypes.c_void_p), ("q_starts", ctypes.c_void_p),
        ("total_q", ctypes.c_int32),
        ("page_table", ctypes.c_void_p), ("pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32),
    ]

    @classmethod
    def make(cls, qo_lens=None, kv_lens=None, q_starts=None, total_q=0, page_table=None, num_pages=0):
        """From int32 device tensors (or None); page_table is [batch, pages_per_seq]."""
        pps = int(page_table.shape[1]) if page_table is not None else 0
        v = cls(_ptr(qo_lens), _ptr(kv_lens), _ptr(q_starts), int(total_q), _ptr(page_table), pps, int(num_pages))
        v._keep = (qo_lens, kv_lens, q_starts, page_table)  # the tensors must outlive the calls
        return v


class MsaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_lib = None


def library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with `python -m block_sparse_long_qk_amd.build`")
        lib = ctypes.CDLL(path)
        P = ctypes.POINTER(Problem)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        lib.msa_workspace_size.argtypes = [P, ctypes.c_int, ctypes.POINTER(sz)]
        lib.msa_index_scores.argtypes = [P, vp, vp, vp, vp]
        lib.msa_block_topk.argtypes = [P, vp, vp, vp]
        lib.msa_sparse_attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.msa_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        V = ctypes.POINTER(Varlen)
        lib.msa_index_scores_v.argtypes = [P, V, vp, vp, vp, vp]
        lib.msa_block_topk_v.argtypes = [P, V, vp, vp, vp]
        lib.msa_sparse_attn_fwd_v.argtypes = [P, V, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.msa_forward_v.argtypes = [P, V, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.msa_index_kl.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.msa_dense_attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp]
        lib.msa_dense_index_kl.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.msa_sparse_attn_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.msa_index_kl_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.msa_index_kl_teacher.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.msa_index_kl_bwd_teacher.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.msa_forward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.msa_forward_marked.argtypes = [P, V, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, ctypes.POINTER(vp),
                                           ctypes.c_int, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_int)]
        for name in EXPORTS[:-1]:
            getattr(lib, name).restype = ctypes.c_int
        lib.msa_status_string.argtypes = [ctypes.c_int]
        lib.msa_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return library().msa_status_string(status).decode()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream, like=None):
    if stream is None:
        import torch
        dev = like.device if like is not None and hasattr(like, "device") else None
        return torch.cuda.current_stream(dev).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(x):
    return 0 if x is None else (x.numel() * x.element_size() if hasattr(x, "numel") else 0)


def _check(rc: int, what: str):
    if rc != OK:
        raise MsaError(rc, what)


# ---------------------------------------------------------------- argument checks
# The C ABI sees plain pointers and cannot tell a buffer's size, element type or
# device, so the binding checks every tensor against the sizes the problem
# implies (include/msa.h states the layouts) before the call: a wrong shape,
# dtype, a non-contiguous view or a host tensor raises ValueError and nothing
# reaches the library.
_BF16 = ("bfloat16",)
_F32 = ("float32",)
_F16 = ("float16",)
_I32 = ("int32",)
_FP8 = ("uint8", "float8_e4m3fn")


def _dtype_name(x) -> str:
    return str(x.dtype).replace("torch.", "")


def _elem(p_dtype: int):
    return _FP8 if p_dtype == DTYPE_FP8_E4M3 else _BF16


class _Args:
    """Collects the tensors of one call, each checked for element type,
    contiguity and size as it is added; device() then checks that all of
    them live on one GPU."""

    def __init__(self, what: str):
        self.what = what
        self.seen = []

    def add(self, x, name: str, dtypes, numel: int, optional: bool = False):
        if x is None:
            if optional:
                return None
            raise ValueError(f"{self.what}: {name} is required")
        if not (hasattr(x, "data_ptr") and hasattr(x, "is_contiguous")):
            raise ValueError(f"{self.what}: {name} must be a torch tensor, got {type(x).__name__}")
        if dtypes is not None and _dtype_name(x) not in dtypes:
            raise ValueError(f"{self.what}: {name} has dtype {_dtype_name(x)}, expected {' or '.join(dtypes)}")
        if not x.is_contiguous():
            raise ValueError(f"{self.what}: {name} must be contiguous")
        if x.numel() < numel:
            raise ValueError(f"{self.what}: {name} holds {x.numel()} elements, the problem needs {numel}")
        self.seen.append((name, x))
        return x

    def workspace(self, ws, nbytes: int):
        """The workspace tensor (any dtype) must hold the bytes passed to the call."""
        if ws is None:
            raise ValueError(f"{self.what}: workspace is required")
        self.add(ws, "workspace", None, 0)
        have = ws.numel() * ws.element_size()
        if nbytes > have:
            raise ValueError(f"{self.what}: workspace_bytes={nbytes} exceeds the workspace tensor ({have} bytes)")

    def device(self):
        dev = None
        for name, x in self.seen:
            if not getattr(x, "is_cuda", False):
                raise ValueError(f"{self.what}: {name} must be a GPU tensor (it is on {x.device})")
            if dev is None:
                dev = x.device
            elif x.device != dev:
                raise ValueError(f"{self.what}: {name} is on {x.device}, other arguments on {dev}")


def _rows(p: Problem, varlen) -> int:
    """Query rows of q, index_q and out: packed (total_q) or B * n_q."""
    if varlen is not None and varlen.q_starts:
        return int(varlen.total_q)
    return p.batch * p.n_q


def _kv_elems(p: Problem, varlen) -> int:
    if varlen is not None and varlen.page_table:
        return int(varlen.num_pages) * p.h_kv * p.block_size * p.head_dim
    return p.batch * p.h_kv * p.n_kv * p.head_dim


def _ik_elems(p: Problem, varlen) -> int:
    if varlen is not None and varlen.page_table:
        return int(varlen.num_pages) * p.block_size * p.index_dim
    return p.batch * p.n_kv * p.index_dim


def _varlen_args(a: _Args, p: Problem, varlen):
    """The descriptor's own device arrays (kept alive by Varlen.make)."""
    if varlen is None:
        return
    keep = getattr(varlen, "_keep", None)
    if keep is None:
        raise ValueError(f"{a.what}: build the Varlen with Varlen.make (its arrays are checked)")
    qo, kv, qs, pt = keep
    a.add(qo, "varlen.qo_lens", _I32, p.batch, optional=True)
    a.add(kv, "varlen.kv_lens", _I32, p.batch, optional=True)
    a.add(qs, "varlen.q_starts", _I32, p.batch, optional=True)
    if pt is not None:
        a.add(pt, "varlen.page_table", _I32, p.batch * int(varlen.pages_per_seq))
        if pt.dim() != 2 or pt.shape[0] != p.batch:
            raise ValueError(f"{a.what}: varlen.page_table must be [batch, pages_per_seq]")


def _index_args(a: _Args, p: Problem, index_q, index_k, varlen):
    a.add(index_q, "index_q", _elem(p.index_dtype), _rows(p, varlen) * p.h_kv * p.index_dim)
    a.add(index_k, "index_k", _elem(p.index_dtype), _ik_elems(p, varlen))


def _qkv_args(a: _Args, p: Problem, q, k, v, varlen, kv_dtypes=None, with_v=True):
    a.add(q, "q", _BF16, _rows(p, varlen) * p.h_q * p.head_dim)
    kvd = _elem(p.kv_dtype) if kv_dtypes is None else kv_dtypes
    a.add(k, "k", kvd, _kv_elems(p, varlen))
    if with_v:
        a.add(v, "v", kvd, _kv_elems(p, varlen))


def _bidx_numel(p: Problem) -> int:
    return p.batch * p.h_kv * p.n_q * p.topk


def _row_numel(p: Problem, heads: int) -> int:
    return p.batch * heads * p.n_q


def workspace_size(p: Problem, op: int) -> int:
    n = ctypes.c_size_t(0)
    _check(library().msa_workspace_size(ctypes.byref(p), op, ctypes.byref(n)), "msa_workspace_size")
    return n.value


def index_scores(p: Problem, index_q, index_k, pooled, stream=None, varlen: Varlen | None = None):
    """pooled[b, g, i, t] = max over visible j in block t of index_q[b, i, g] . index_k[b, j]."""
    a = _Args("index_scores")
    _index_args(a, p, index_q, index_k, varlen)
    a.add(pooled, "pooled", _F32, p.batch * p.h_kv * p.n_q * p.n_blk)
    _varlen_args(a, p, varlen)
    a.device()
    L, st = library(), _stream(stream, pooled)
    if varlen is None:
        rc = L.msa_index_scores(ctypes.byref(p), _ptr(index_q), _ptr(index_k), _ptr(pooled), st)
    else:
        rc = L.msa_index_scores_v(ctypes.byref(p), ctypes.byref(varlen), _ptr(index_q), _ptr(index_k), _ptr(pooled),
                                  st)
    _check(rc, "msa_index_scores")
    return pooled


def block_topk(p: Problem, pooled, block_idx, stream=None, varlen: Varlen | None = None):
    """block_idx[b, g, i] = local block + top-(k-1) other visible blocks, ascending, -1 padded."""
    a = _Args("block_topk")
    a.add(pooled, "pooled", _F32, p.batch * p.h_kv * p.n_q * p.n_blk)
    a.add(block_idx, "block_idx", _I32, _bidx_numel(p))
    _varlen_args(a, p, varlen)
    a.device()
    L, st = library(), _stream(stream, pooled)
    if varlen is None:
        rc = L.msa_block_topk(ctypes.byref(p), _ptr(pooled), _ptr(block_idx), st)
    else:
        rc = L.msa_block_topk_v(ctypes.byref(p), ctypes.byref(varlen), _ptr(pooled), _ptr(block_idx), st)
    _check(rc, "msa_block_topk")
    return block_idx


def sparse_attn_fwd(p: Problem, q, k, v, block_idx, out, lse=None, workspace=None, workspace_bytes=None,
                    stream=None, varlen: Varlen | None = None):
    """Softmax attention of every query head over its group's selected blocks."""
    nb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    a = _Args("sparse_attn_fwd")
    _qkv_args(a, p, q, k, v, varlen)
    a.add(block_idx, "block_idx", _I32, _bidx_numel(p))
    a.add(out, "out", _BF16, _rows(p, varlen) * p.h_q * p.head_dim)
    a.add(lse, "lse", _F32, _row_numel(p, p.h_q), optional=True)
    a.workspace(workspace, nb)
    _varlen_args(a, p, varlen)
    a.device()
    L, st = library(), _stream(stream, q)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), _ptr(out), _ptr(lse), _ptr(workspace), nb, st)
    if varlen is None:
        rc = L.msa_sparse_attn_fwd(ctypes.byref(p), *args)
    else:
        rc = L.msa_sparse_attn_fwd_v(ctypes.byref(p), ctypes.byref(varlen), *args)
    _check(rc, "msa_sparse_attn_fwd")
    return out


def forward(p: Problem, q, k, v, index_q, index_k, out, block_idx, lse=None, workspace=None, workspace_bytes=None,
            stream=None, varlen: Varlen | None = None):
    """The whole MSA forward pass: index scores, block top-k, sparse attention."""
    nb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    a = _Args("forward")
    _qkv_args(a, p, q, k, v, varlen)
    _index_args(a, p, index_q, index_k, varlen)
    a.add(out, "out", _BF16, _rows(p, varlen) * p.h_q * p.head_dim)
    a.add(block_idx, "block_idx", _I32, _bidx_numel(p))
    a.add(lse, "lse", _F32, _row_numel(p, p.h_q), optional=True)
    a.workspace(workspace, nb)
    _varlen_args(a, p, varlen)
    a.device()
    L, st = library(), _stream(stream, q)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(index_q), _ptr(index_k), _ptr(out), _ptr(block_idx), _ptr(lse),
            _ptr(workspace), nb, st)
    if varlen is None:
        rc = L.msa_forward(ctypes.byref(p), *args)
    else:
        rc = L.msa_forward_v(ctypes.byref(p), ctypes.byref(varlen), *args)
    _check(rc, "msa_forward")
    return out


def forward_marked(p: Problem, q, k, v, index_q, index_k, out, block_idx, lse, workspace, events, stream=None,
                   varlen: Varlen | None = None, workspace_bytes=None):
    """forward() with a HIP event recorded after each kernel it launches (for
    benchmarks).  events: torch.cuda.Event objects with timing enabled, each
    recorded once beforehand (so that the underlying event exists).  Returns
    the list of (kernel name, event before, event after) of the call."""
    nb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    a = _Args("forward_marked")
    _qkv_args(a, p, q, k, v, varlen)
    _index_args(a, p, index_q, index_k, varlen)
    a.add(out, "out", _BF16, _rows(p, varlen) * p.h_q * p.head_dim)
    a.add(block_idx, "block_idx", _I32, _bidx_numel(p))
    a.add(lse, "lse", _F32, _row_numel(p, p.h_q), optional=True)
    a.workspace(workspace, nb)
    _varlen_args(a, p, varlen)
    a.device()
    L, st = library(), _stream(stream, q)
    n = len(events)
    evs = (ctypes.c_void_p * n)(*[e.cuda_event for e in events])
    names = (ctypes.c_char_p * n)()
    used = ctypes.c_int(0)
    rc = L.msa_forward_marked(ctypes.byref(p), ctypes.byref(varlen) if varlen is not None else None, _ptr(q), _ptr(k),
                              _ptr(v), _ptr(index_q), _ptr(index_k), _ptr(out), _ptr(block_idx), _ptr(lse),
                              _ptr(workspace), nb, st, evs, n, names, ctypes.byref(used))
    _check(rc, "msa_forward_marked")
    return [(names[i].decode(), events[i], events[i + 1]) for i in range(used.value - 1)]


def forward_noalloc(p: Problem, q, k, v, index_q, index_k, out, block_idx, lse=None, stream=None):
    """forward() with the library's fixed device scratch as its workspace (no
    allocation anywhere; problems needing more than NOALLOC_SCRATCH_BYTES raise
    MsaError with ERR_WORKSPACE_TOO_SMALL).  Calls that overlap in time on one
    GPU share the scratch and race."""
    a = _Args("forward_noalloc")
    _qkv_args(a, p, q, k, v, None)
    _index_args(a, p, index_q, index_k, None)
    a.add(out, "out", _BF16, _rows(p, None) * p.h_q * p.head_dim)
    a.add(block_idx, "block_idx", _I32, _bidx_numel(p))
    a.add(lse, "lse", _F32, _row_numel(p, p.h_q), optional=True)
    a.device()
    L, st = library(), _stream(stream, q)
    rc = L.msa_forward_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(index_q), _ptr(index_k), _ptr(out),
                               _ptr(block_idx), _ptr(lse), st)
    _check(rc, "msa_forward_noalloc")
    return out


def index_kl(p: Problem, q, k, index_q, index_k, block_idx, lse, kl, workspace=None, workspace_bytes=None,
             stream=None, lse_index=None):
    """KL(teacher || student) per (b, g, query): the group-averaged main-branch
    distribution over the selected tokens against the softmax of the raw index
    scores over the same tokens; lse is the forward pass's output."""
    nb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    a = _Args("index_kl")
    _qkv_args(a, p, q, k, None, None, kv_dtypes=_BF16, with_v=False)
    _index_args(a, p, index_q, index_k, None)
    a.add(block_idx, "block_idx", _I32, _bidx_numel(p))
    a.add(lse, "lse", _F32, _row_numel(p, p.h_q))
    a.add(kl, "kl", _F32, _row_numel(p, p.h_kv))
    a.add(lse_index, "lse_index", _F32, _row_numel(p, p.h_kv), optional=True)
    a.workspace(workspace, nb)
    a.device()
    L, st = library(), _stream(stream, q)
    rc = L.msa_index_kl(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(index_q), _ptr(index_k), _ptr(block_idx), _ptr(lse),
                        _ptr(kl), _ptr(lse_index), _ptr(workspace), nb, st)
    _check(rc, "msa_index_kl")
    return kl


def teacher_shape(p: Problem):
    """Shape of index_kl_teacher's teacher (fp16): [B, H_kv, n_q, k + 1, block_size]."""
    return (p.batch, p.h_kv, p.n_q, p.topk + 1, p.block_size)


def index_kl_teacher(p: Problem, q, k, index_q, index_k, block_idx, lse, kl, lse_index, teacher, workspace=None,
                     workspace_bytes=None, stream=None):
    """index_kl, also storing the teacher's weight of every key of every
    (row, slot) in teacher (fp16, teacher_shape(p)) for index_kl_bwd_teacher."""
    nb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    a = _Args("index_kl_teacher")
    _qkv_args(a, p, q, k, None, None, kv_dtypes=_BF16, with_v=False)
    _index_args(a, p, index_q, index_k, None)
    a.add(block_idx, "block_idx", _I32, _bidx_numel(p))
    a.add(lse, "lse", _F32, _row_numel(p, p.h_q))
    a.add(kl, "kl", _F32, _row_numel(p, p.h_kv))
    a.add(lse_index, "lse_index", _F32, _row_numel(p, p.h_kv))
    a.add(teacher, "teacher", _F16, _row_numel(p, p.h_kv) * (p.topk + 1) * p.block_size)
    a.workspace(workspace, nb)
    a.device()
    L, st = library(), _stream(stream, q)
    rc = L.msa_index_kl_teacher(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(index_q), _ptr(index_k), _ptr(block_idx),
                                _ptr(lse), _ptr(kl), _ptr(lse_index), _ptr(teacher), _ptr(workspace), nb, st)
    _check(rc, "msa_index_kl_teacher")
    return kl, teacher


def index_kl_bwd_teacher(p: Problem, index_q, index_k, block_idx, teacher, lse_index, d_index_q, d_index_k,
                         dkl=None, workspace=None, workspace_bytes=None, stream=None):
    """index_kl_bwd with the teacher index_kl_teacher stored (no q, k, lse)."""
    nb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    a = _Args("index_kl_bwd_teacher")
    _index_args(a, p, index_q, index_k, None)
    a.add(block_idx, "block_idx", _I32, _bidx_numel(p))
    a.add(teacher, "teacher", _F16, _row_numel(p, p.h_kv) * (p.topk + 1) * p.block_size)
    a.add(lse_index, "lse_index", _F32, _row_numel(p, p.h_kv))
    a.add(d_index_q, "d_index_q", _elem(p.index_dtype), p.batch * p.n_q * p.h_kv * p.index_dim)
    a.add(d_index_k, "d_index_k", _elem(p.index_dtype), p.batch * p.n_kv * p.index_dim)
    a.add(dkl, "dkl", _F32, _row_numel(p, p.h_kv), optional=True)
    a.workspace(workspace, nb)
    a.device()
    L, st = library(), _stream(stream, index_q)
    rc = L.msa_index_kl_bwd_teacher(ctypes.byref(p), _ptr(index_q), _ptr(index_k), _ptr(block_idx), _ptr(teacher),
                                    _ptr(lse_index), _ptr(dkl), _ptr(d_index_q), _ptr(d_index_k), _ptr(workspace),
                                    nb, st)
    _check(rc, "msa_index_kl_bwd_teacher")
    return d_index_q, d_index_k


def sparse_attn_bwd(p: Problem, q, k, v, block_idx, out, lse, dout, dq, dk, dv, workspace=None,
                    workspace_bytes=None, stream=None):
    """Gradients dq, dk, dv of sparse_attn_fwd for the output gradient dout."""
    nb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    a = _Args("sparse_attn_bwd")
    _qkv_args(a, p, q, k, v, None, kv_dtypes=_BF16)
    a.add(block_idx, "block_idx", _I32, _bidx_numel(p))
    a.add(out, "out", _BF16, p.batch * p.n_q * p.h_q * p.head_dim)
    a.add(lse, "lse", _F32, _row_numel(p, p.h_q))
    a.add(dout, "dout", _BF16, p.batch * p.n_q * p.h_q * p.head_dim)
    a.add(dq, "dq", _BF16, p.batch * p.n_q * p.h_q * p.head_dim)
    a.add(dk, "dk", _BF16, _kv_elems(p, None))
    a.add(dv, "dv", _BF16, _kv_elems(p, None))
    a.workspace(workspace, nb)
    a.device()
    L, st = library(), _stream(stream, q)
    rc = L.msa_sparse_attn_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), _ptr(out), _ptr(lse),
                               _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), nb, st)
    _check(rc, "msa_sparse_attn_bwd")
    return dq, dk, dv


def index_kl_bwd(p: Problem, q, k, index_q, index_k, block_idx, lse, lse_index, d_index_q, d_index_k, dkl=None,
                 workspace=None, workspace_bytes=None, stream=None):
    """Gradients of sum(dkl * kl) into index_q and index_k, the teacher held
    fixed; lse_index is index_kl's output for the same inputs (dkl None: ones)."""
    nb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    a = _Args("index_kl_bwd")
    _qkv_args(a, p, q, k, None, None, kv_dtypes=_BF16, with_v=False)
    _index_args(a, p, index_q, index_k, None)
    a.add(block_idx, "block_idx", _I32, _bidx_numel(p))
    a.add(lse, "lse", _F32, _row_numel(p, p.h_q))
    a.add(lse_index, "lse_index", _F32, _row_numel(p, p.h_kv))
    a.add(d_index_q, "d_index_q", _elem(p.index_dtype), p.batch * p.n_q * p.h_kv * p.index_dim)
    a.add(d_index_k, "d_index_k", _elem(p.index_dtype), p.batch * p.n_kv * p.index_dim)
    a.add(dkl, "dkl", _F32, _row_numel(p, p.h_kv), optional=True)
    a.workspace(workspace, nb)
    a.device()
    L, st = library(), _stream(stream, q)
    rc = L.msa_index_kl_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(index_q), _ptr(index_k), _ptr(block_idx),
                            _ptr(lse), _ptr(lse_index), _ptr(dkl), _ptr(d_index_q), _ptr(d_index_k), _ptr(workspace),
                            nb, st)
    _check(rc, "msa_index_kl_bwd")
    return d_index_q, d_index_k


def dense_attn_fwd(p: Problem, q, k, v, out, lse=None, stream=None):
    """Dense causal GQA attention (every visible key): the warmup's main branch."""
    a = _Args("dense_attn_fwd")
    _qkv_args(a, p, q, k, v, None, kv_dtypes=_BF16)
    a.add(out, "out", _BF16, p.batch * p.n_q * p.h_q * p.head_dim)
    a.add(lse, "lse", _F32, _row_numel(p, p.h_q), optional=True)
    a.device()
    L, st = library(), _stream(stream, q)
    _check(L.msa_dense_attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), st),
           "msa_dense_attn_fwd")
    return out


def dense_index_kl(p: Problem, q, k, index_q, index_k, lse, kl, stream=None, lse_index=None):
    """index_kl over every visible token, with the dense attention's lse."""
    a = _Args("dense_index_kl")
    _qkv_args(a, p, q, k, None, None, kv_dtypes=_BF16, with_v=False)
    _index_args(a, p, index_q, index_k, None)
    a.add(lse, "lse", _F32, _row_numel(p, p.h_q))
    a.add(kl, "kl", _F32, _row_numel(p, p.h_kv))
    a.add(lse_index, "lse_index", _F32, _row_numel(p, p.h_kv), optional=True)
    a.device()
    L, st = library(), _stream(stream, q)
    _check(L.msa_dense_index_kl(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(index_q), _ptr(index_k), _ptr(lse), _ptr(kl),
                                _ptr(lse_index), st), "msa_dense_index_kl")
    return kl


# ---------------------------------------------------------------- allocation helpers (torch)
def alloc_outputs(p: Problem, device="cuda", lse: bool = True, op: int = OP_FORWARD) -> dict:
    """Output tensors and the workspace of one call, allocated with torch."""
    import torch
    o = {
        "out": torch.empty((p.batch, p.n_q, p.h_q, p.head_dim), dtype=torch.bfloat16, device=device),
        "block_idx": torch.empty((p.batch, p.h_kv, p.n_q, p.topk), dtype=torch.int32, device=device),
        "lse": torch.empty((p.batch, p.h_q, p.n_q), dtype=torch.float32, device=device) if lse else None,
    }
    if op == OP_INDEX_SCORES:
        o = {"pooled": torch.empty((p.batch, p.h_kv, p.n_q, p.n_blk), dtype=torch.float32, device=device)}
    nbytes = workspace_size(p, op)
    o["workspace"] = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    return o
