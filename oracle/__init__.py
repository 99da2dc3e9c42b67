"""Python face of the fp64 CPU oracle (``msa_oracle.c``).

TEST INFRASTRUCTURE: only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP path; its only common dependency is the seeded input generator
(``synth``), which holds none of the method's arithmetic.

The C library is built with gcc (``-O2 -fopenmp``, no fast-math) on first use,
or by ``build()``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_HERE, "liboracle.so")
SRC = os.path.join(_HERE, "msa_oracle.c")
_lib = None

_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_i64, _i32, _f64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_double


def build(force: bool = False) -> str:
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", SRC, "-o", tmp, "-lm"],
                       check=True)
        os.replace(tmp, LIB)
    return LIB


def _L():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(LIB)
        lib.oracle_pool.argtypes = [_u16p, _i64, _i64p, _u16p, _i64, _i32, _i32, _f64p, _i64]
        lib.oracle_select.argtypes = [_f64p, _i64, _i64, _i64p, _i32, _i32, _i32p]
        lib.oracle_attend.argtypes = [_u16p, _i64, _i64p, _i32p, _i32, _i32, _u16p, _u16p, _i64, _i32, _i32,
                                      _f64, _f64p, _f64p]
        lib.oracle_dense_gqa.argtypes = [_u16p, _i64, _i64p, _i32, _u16p, _u16p, _i64, _i32, _f64, _f64p, _f64p]
        lib.oracle_merge.argtypes = [_f64p, _f64p, _i64, _i32, _i32, _f64p, _f64p]
        lib.oracle_e4m3_decode.argtypes = [_u8p, _i64, _f64p]
        lib.oracle_pool_f8.argtypes = [_u8p, _i64, _i64p, _u8p, _i64, _i32, _i32, _f64p, _i64]
        lib.oracle_kl.argtypes = [_u16p, _i64, _i64p, _i32p, _i32, _i32, _u16p, _i64, _i32, _u16p, _u16p, _i32, _i32,
                                  _f64, _f64p]
        lib.oracle_attend_bwd.argtypes = [_u16p, _i64, _i64p, _i32p, _i32, _i32, _u16p, _u16p, _i64, _i32, _i32,
                                          _f64, _u16p, _f64p, _f64p, _f64p]
        lib.oracle_kl_bwd.argtypes = [_u16p, _i64, _i64p, _i32p, _i32, _i32, _u16p, _i64, _i32, _u16p, _u16p, _i32,
                                      _i32, _f64, _f64p, _f64p, _f64p]
        lib.oracle_kl_teacher.argtypes = [_u16p, _i64, _i64p, _i32p, _i32, _i32, _u16p, _i64, _i32, _i32, _f64,
                                           _f64p]
        for f in (lib.oracle_pool, lib.oracle_select, lib.oracle_attend, lib.oracle_dense_gqa, lib.oracle_merge,
                  lib.oracle_e4m3_decode, lib.oracle_pool_f8, lib.oracle_kl, lib.oracle_attend_bwd, lib.oracle_kl_bwd,
                  lib.oracle_kl_teacher):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what}: invalid argument")


def _u16(a):
    return np.ascontiguousarray(a, dtype=np.uint16)


def pool(iq_rows, pos, ik, bk: int) -> np.ndarray:
    """Pooled index scores [nrows, n_blk] (NaN after each row's local block).

    iq_rows [nrows, d_idx] bf16 bits; pos [nrows]; ik [n_kv, d_idx] bf16 bits.
    """
    iq_rows, ik = _u16(iq_rows), _u16(ik)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    n_kv, d_idx = ik.shape
    n_blk = -(-n_kv // bk)
    out = np.full((len(pos), n_blk), np.nan)
    _check(_L().oracle_pool(iq_rows, len(pos), pos, ik, n_kv, d_idx, bk, out, n_blk), "oracle_pool")
    return out


def index_values(x) -> np.ndarray:
    """Index inputs as fp64 values: bf16 bits (uint16) widened exactly, or
    E4M3 codes (uint8) through e4m3_decode."""
    x = np.asarray(x)
    if x.dtype == np.uint8:
        return e4m3_decode(x)
    return (np.ascontiguousarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(
        np.float64)


def pool_mm(iq_rows, pos, ik, bk: int, keys_per_step: int = 16384, ik_values=None) -> np.ndarray:
    """pool() (or pool_f8()) written with a library matrix product.

    The same definition as oracle_pool (page "MiniMax 发布 MSA…", section
    两个分支如何工作: score every visible key, max-pool to blocks): the scores of
    the rows against the keys are one fp64 product of the exact input values
    and each block keeps the max of its scores; a row's own (local) block is
    then pooled again over the keys up to the row's position only, and the
    blocks after it are not candidates (NaN).  Only the summation order inside
    each dot product differs from the plain loops (fp64, so by a few units in
    the last place).  The parity tests use it where the loops would take
    minutes (thousands of rows against a 1M-token cache).  Returns
    [nrows, n_blk], NaN after each row's local block, like pool().
    ik_values: index_values(ik), when the caller already holds it.
    """
    a = index_values(iq_rows)
    kv = index_values(ik) if ik_values is None else ik_values
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    n_kv = ik.shape[0]
    n_blk = -(-n_kv // bk)
    n = len(pos)
    out = np.full((n, n_blk), np.nan)
    if n == 0:
        return out
    if np.any(pos < 0) or np.any(pos >= n_kv) or a.shape[1] != ik.shape[1]:
        raise ValueError("pool_mm: invalid argument")
    local = pos // bk
    step = max(bk, keys_per_step // bk * bk)
    # every block up to the last one a row sees, all of its keys
    for j0 in range(0, int(pos.max()) + 1, step):
        j1 = min(j0 + step, n_kv)
        s = a @ kv[j0:j1].T
        nb = -(-(j1 - j0) // bk)
        if s.shape[1] < nb * bk:
            s = np.concatenate([s, np.full((n, nb * bk - s.shape[1]), -np.inf)], axis=1)
        out[:, j0 // bk:j0 // bk + nb] = s.reshape(n, nb, bk).max(axis=2)
    # the local block: only the keys j <= p count
    for r0 in range(0, n, 256):
        r1 = min(r0 + 256, n)
        keys = local[r0:r1, None] * bk + np.arange(bk)[None, :]
        sl = np.matmul(kv[np.minimum(keys, n_kv - 1)], a[r0:r1, :, None])[:, :, 0]
        sl[keys > pos[r0:r1, None]] = -np.inf
        out[np.arange(r0, r1), local[r0:r1]] = sl.max(axis=1)
    out[np.arange(n_blk)[None, :] > local[:, None]] = np.nan
    return out


def e4m3_decode(codes) -> np.ndarray:
    """OCP E4M3 codes (uint8) -> their values in fp64 (NaN for 0x7F / 0xFF)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    _check(_L().oracle_e4m3_decode(c.reshape(-1), c.size, out.reshape(-1)), "oracle_e4m3_decode")
    return out


def pool_f8(iq_rows, pos, ik, bk: int) -> np.ndarray:
    """pool() with E4M3 index inputs (uint8 codes)."""
    iq_rows = np.ascontiguousarray(iq_rows, dtype=np.uint8)
    ik = np.ascontiguousarray(ik, dtype=np.uint8)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    n_kv, d_idx = ik.shape
    n_blk = -(-n_kv // bk)
    out = np.full((len(pos), n_blk), np.nan)
    _check(_L().oracle_pool_f8(iq_rows, len(pos), pos, ik, n_kv, d_idx, bk, out, n_blk), "oracle_pool_f8")
    return out


def select(pooled, pos, bk: int, k: int) -> np.ndarray:
    """Selected blocks [nrows, k] int32: ascending, local included, -1 padded."""
    pooled = np.ascontiguousarray(pooled, dtype=np.float64)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    out = np.empty((len(pos), k), np.int32)
    _check(_L().oracle_select(pooled, pooled.shape[1], len(pos), pos, bk, k, out), "oracle_select")
    return out


def attend(q_rows, pos, sel, K, V, bk: int, scale: float):
    """Main-branch attention on a given block set.

    q_rows [nrows, G, d]; sel [nrows, k]; K, V [n_kv, d] -> (out [nrows, G, d], lse [nrows, G]).
    """
    q_rows, K, V = _u16(q_rows), _u16(K), _u16(V)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    n, G, d = q_rows.shape
    out = np.empty((n, G, d))
    lse = np.empty((n, G))
    _check(_L().oracle_attend(q_rows, n, pos, sel, sel.shape[1], G, K, V, K.shape[0], d, bk, scale, out, lse),
           "oracle_attend")
    return out, lse


def attend_bwd(q_rows, pos, sel, K, V, bk: int, scale: float, dO_rows):
    """Gradient of attend(): returns (dQ [n, G, d], dK [n_kv, d], dV [n_kv, d]),
    dK and dV summed over every row and head passed."""
    q_rows, K, V, dO_rows = _u16(q_rows), _u16(K), _u16(V), _u16(dO_rows)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    n, G, d = q_rows.shape
    dQ = np.zeros((n, G, d))
    dK = np.zeros((K.shape[0], d))
    dV = np.zeros((K.shape[0], d))
    _check(_L().oracle_attend_bwd(q_rows, n, pos, sel, sel.shape[1], G, K, V, K.shape[0], d, bk, scale, dO_rows, dQ,
                                  dK, dV), "oracle_attend_bwd")
    return dQ, dK, dV


def kl_bwd(q_rows, pos, sel, K, iq_rows, ik, bk: int, scale: float, w=None):
    """Gradient of sum_r w_r kl_r with respect to iq_rows and ik, the teacher
    held fixed: returns (d_iq [n, d_idx], d_ik [n_kv, d_idx])."""
    q_rows, K = _u16(q_rows), _u16(K)
    iq_rows, ik = _u16(iq_rows), _u16(ik)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    n, G, d = q_rows.shape
    w = np.ones(n) if w is None else np.ascontiguousarray(w, dtype=np.float64)
    d_iq = np.zeros((n, iq_rows.shape[1]))
    d_ik = np.zeros(ik.shape)
    _check(_L().oracle_kl_bwd(q_rows, n, pos, sel, sel.shape[1], G, K, K.shape[0], d, iq_rows, ik, iq_rows.shape[1],
                              bk, scale, w, d_iq, d_ik), "oracle_kl_bwd")
    return d_iq, d_ik


def kl(q_rows, pos, sel, K, iq_rows, ik, bk: int, scale: float) -> np.ndarray:
    """KL(teacher || student) per row over the selected blocks' visible tokens.

    q_rows [n, G, d]; sel [n, k]; K [n_kv, d]; iq_rows [n, d_idx]; ik [n_kv, d_idx] (bf16 bits) -> [n].
    """
    q_rows, K = _u16(q_rows), _u16(K)
    iq_rows, ik = _u16(iq_rows), _u16(ik)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    n, G, d = q_rows.shape
    out = np.empty(n)
    _check(_L().oracle_kl(q_rows, n, pos, sel, sel.shape[1], G, K, K.shape[0], d, iq_rows, ik, iq_rows.shape[1], bk,
                          scale, out), "oracle_kl")
    return out


def kl_teacher(q_rows, pos, sel, K, bk: int, scale: float) -> np.ndarray:
    """The teacher of kl() per row as a dense [n, n_kv] array (0 outside T)."""
    q_rows, K = _u16(q_rows), _u16(K)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    n, G, d = q_rows.shape
    out = np.empty((n, K.shape[0]))
    _check(_L().oracle_kl_teacher(q_rows, n, pos, sel, sel.shape[1], G, K, K.shape[0], d, bk, scale, out),
           "oracle_kl_teacher")
    return out


def dense_gqa(q_rows, pos, K, V, scale: float):
    """Dense causal GQA attention over every key j <= p."""
    q_rows, K, V = _u16(q_rows), _u16(K), _u16(V)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    n, G, d = q_rows.shape
    out = np.empty((n, G, d))
    lse = np.empty((n, G))
    _check(_L().oracle_dense_gqa(q_rows, n, pos, G, K, V, K.shape[0], d, scale, out, lse), "oracle_dense_gqa")
    return out, lse


def merge(o_parts, lse_parts):
    """LSE merge of partial results: o_parts [n, P, d], lse_parts [n, P] -> (o [n, d], lse [n])."""
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    n, P, d = o_parts.shape
    o = np.empty((n, d))
    lse = np.empty(n)
    _check(_L().oracle_merge(o_parts, lse_parts, n, P, d, o, lse), "oracle_merge")
    return o, lse


# ---------------------------------------------------------------- workload rows
def inputs_for_rows(w, b: int, g: int, rows, plant=None):
    """Host inputs of one (sequence, group) for the given query rows.

    Returns dict(pos, iq [n, d_idx], q [n, G, d], ik [pmax+1, d_idx]); iq and ik
    are bf16 bits, or E4M3 codes for an "fp8" workload.
    """
    x = inputs_for_rows_all(w, b, rows, plant)
    G = w.group
    return {"pos": x["pos"], "iq": np.ascontiguousarray(x["iq"][:, g, :]),
            "q": np.ascontiguousarray(x["q"][:, g * G:(g + 1) * G, :]), "ik": x["ik"]}


def inputs_for_rows_all(w, b: int, rows, plant=None, with_q: bool = True):
    """inputs_for_rows for every group at once: iq [n, h_kv, d_idx], q [n, h_q, d]
    (q None when with_q is false)."""
    import synth
    rows = np.asarray(rows, dtype=np.int64)
    plant = synth.plant_spec(w) if plant is None else plant
    pos = w.offset + rows
    iq = synth.host_iq_rows(w, b, rows, plant)
    if w.index_dtype == "fp8":
        iq = synth.to_e4m3(iq)
    q = synth.host_q_rows(w, b, rows) if with_q else None
    ik = _index_keys(w, b, plant)[:int(pos.max()) + 1]
    return {"pos": pos, "iq": iq, "q": q, "ik": ik}


def pool_for(w, iq_rows, pos, ik) -> np.ndarray:
    """pool() or pool_f8(), as the workload's index element type requires."""
    return (pool_f8 if w.index_dtype == "fp8" else pool)(iq_rows, pos, ik, w.block_size)


_ik_cache = {}


def _index_keys(w, b: int, plant):
    """index_k of one sequence (all n_kv tokens); the last one is kept, since
    every group and row of a sequence reads the same keys."""
    import synth
    key = (w, b)
    if key not in _ik_cache:
        _ik_cache.clear()
        ik = synth.host_ik(w, b, 0, w.n_kv, plant)
        _ik_cache[key] = synth.to_e4m3(ik) if w.index_dtype == "fp8" else ik
    return _ik_cache[key]


def kv_values_bf16(w, bits):
    """K or V rows as the attention sees them: the bf16 bits themselves, or,
    for a workload with FP8 K/V, the bf16 bits of the values their E4M3 codes
    represent (exact: every E4M3 value is a bf16 value)."""
    if getattr(w, "kv_dtype", "bf16") != "fp8":
        return bits
    import synth
    vals = e4m3_decode(synth.to_e4m3(bits)).astype(np.float32)
    return (vals.view(np.uint32) >> 16).astype(np.uint16)


def kv_for_blocks(w, b: int, g: int, sel):
    """K and V of one (sequence, group) with only the selected blocks filled.

    The arrays are full-length (so token positions keep their meaning) but are
    allocated with calloc, so untouched blocks cost no memory.
    """
    import synth
    K = np.zeros((w.n_kv, w.head_dim), np.uint16)
    V = np.zeros((w.n_kv, w.head_dim), np.uint16)
    blocks = np.unique(np.asarray(sel)[np.asarray(sel) >= 0])
    if 2 * len(blocks) > w.n_blk:   # most blocks: one generator pass over the whole head
        K[:] = kv_values_bf16(w, synth.host_kv(w, "k", b, g, 0, w.n_kv))
        V[:] = kv_values_bf16(w, synth.host_kv(w, "v", b, g, 0, w.n_kv))
        return K, V
    for t in blocks:
        j0, j1 = int(t) * w.block_size, min((int(t) + 1) * w.block_size, w.n_kv)
        K[j0:j1] = kv_values_bf16(w, synth.host_kv(w, "k", b, g, j0, j1))
        V[j0:j1] = kv_values_bf16(w, synth.host_kv(w, "v", b, g, j0, j1))
    return K, V


def forward_rows(w, b: int, g: int, rows, sel_given=None, plant=None):
    """The whole forward pass for some query rows of one (sequence, group).

    Returns dict(pos, pooled, sel, out [n, G, d], lse [n, G]); when ``sel_given``
    is passed, attention runs on that block set instead of the oracle's own.
    """
    x = inputs_for_rows(w, b, g, rows, plant)
    pooled = pool_for(w, x["iq"], x["pos"], x["ik"])
    sel = select(pooled, x["pos"], w.block_size, w.topk)
    use = sel if sel_given is None else np.asarray(sel_given, dtype=np.int32)
    K, V = kv_for_blocks(w, b, g, use)
    out, lse = attend(x["q"], x["pos"], use, K, V, w.block_size, w.scale)
    return {"pos": x["pos"], "pooled": pooled, "sel": sel, "out": out, "lse": lse}
