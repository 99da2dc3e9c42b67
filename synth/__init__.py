"""Seeded synthetic inputs for the MSA forward pass.

This module is the only code shared by the oracle side and the GPU side.  It
holds none of the method's arithmetic: it only produces input tensors (Q, K, V,
index-q, index-k) from a seed, either on the host (numpy, for the oracle) or on
the device (a HIP fill kernel in ``synth_dev.hip``, for the kernels), and the two
produce identical bits for every element.

Element generator
-----------------
Element ``e`` (flat index in the tensor's canonical layout) of tensor ``t``
under seed ``s``::

    key = sm64((s << 8) | t)
    h   = sm64(key + e)                 # all arithmetic mod 2**64
    x   = NT[h >> 48]                   # bf16 bit pattern

``sm64`` is Vigna's published SplitMix64 step (add the golden-ratio increment,
then the 30/27/31 xor-shift-multiply finaliser).  ``NT[u]`` is the bf16 (round to
nearest even, via fp32) of the standard normal quantile at ``(u + 0.5) / 65536``,
so values are ~N(0, 1) quantised to 2**16 levels with ``|x| <= 4.33``.

Planted structure
-----------------
The block-sparse workloads plant a few high-scoring key blocks per group (the
learned indexer's long-range stripes).  For group ``g``: a direction ``u_g`` (the
fp64 unit vector of generator values of tensor 6 at ``e = g * d_idx + c``) and
``m`` distinct block positions (successive hashes of tensor 7 modulo the block
count).  Then ``ik[j] <- bf16(fp32(ik[j]) + fp32(alpha * u_g))`` for every token
``j`` of those blocks (groups applied in ascending order) and
``iq[i, g] <- bf16(fp32(iq[i, g]) + fp32(beta * u_g))`` for every query row.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field
from statistics import NormalDist

import numpy as np

# Tensor ids of the element generator.
T_Q, T_K, T_V, T_IQ, T_IK, T_PLANT_DIR, T_PLANT_POS = 1, 2, 3, 4, 5, 6, 7
T_DO = 8  # the output gradient of the backward tests (q's layout)

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK64 = (1 << 64) - 1


def _sm64_int(x: int) -> int:
    """SplitMix64 step on a Python int (reference for the vectorised form)."""
    z = (x + 0x9E3779B97F4A7C15) & _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def _sm64_np(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = x + _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def stream_key(seed: int, tensor_id: int) -> int:
    return _sm64_int(((seed << 8) | tensor_id) & _MASK64)


# ---------------------------------------------------------------- bf16 helpers
def f32_to_bf16(x) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


_NT = None


def normal_table() -> np.ndarray:
    """The 65536-entry bf16 table of normal quantiles (built once per process)."""
    global _NT
    if _NT is None:
        nd = NormalDist()
        v = np.array([nd.inv_cdf((u + 0.5) / 65536.0) for u in range(65536)], dtype=np.float64)
        _NT = f32_to_bf16(v.astype(np.float32))
    return _NT


_GEN_CHUNK = 1 << 22   # elements per worker task of a large gen_range


def _gen_into(out: np.ndarray, key: np.uint64, start: int, nt: np.ndarray):
    e = np.arange(out.size, dtype=np.uint64) + np.uint64(start)
    with np.errstate(over="ignore"):
        h = _sm64_np(key + e)
    out[:] = nt[(h >> np.uint64(48)).astype(np.int64)]


def gen_range(seed: int, tensor_id: int, start: int, count: int) -> np.ndarray:
    """bf16 bits of elements start .. start+count-1 of one generated tensor.

    Large ranges are cut into pieces filled by a thread pool (numpy releases
    the interpreter lock inside its array operations); every element is still
    the same function of its index."""
    key = np.uint64(stream_key(seed, tensor_id))
    nt = normal_table()
    out = np.empty(count, dtype=np.uint16)
    if count <= _GEN_CHUNK:
        _gen_into(out, key, start, nt)
        return out
    from concurrent.futures import ThreadPoolExecutor
    workers = min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=workers) as ex:
        futs = [ex.submit(_gen_into, out[a:a + _GEN_CHUNK], key, start + a, nt) for a in range(0, count, _GEN_CHUNK)]
        for f in futs:
            f.result()
    return out


def gen_at(seed: int, tensor_id: int, idx) -> np.ndarray:
    """bf16 bits of the elements at the given flat indices."""
    key = np.uint64(stream_key(seed, tensor_id))
    e = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        h = _sm64_np(key + e)
    return normal_table()[(h >> np.uint64(48)).astype(np.int64)]


# ---------------------------------------------------------------- workloads
@dataclass(frozen=True)
class Workload:
    """One problem instance: shapes, causal offset, planting and seed."""
    name: str
    batch: int
    n_q: int
    n_kv: int
    h_q: int
    h_kv: int
    head_dim: int = 128
    index_dim: int = 128
    block_size: int = 128
    topk: int = 16
    q_offset: int = -1          # -1: bottom-right alignment, n_kv - n_q
    seed: int = 1
    plant_m: int = 0            # planted blocks per group (0: none)
    plant_alpha: float = 0.0    # amplitude added to planted index keys
    plant_beta: float = 0.0     # amplitude added to that group's index queries
    index_dtype: str = "bf16"   # "fp8": index_q / index_k are the bf16 values rounded to OCP E4M3
    kv_dtype: str = "bf16"      # "fp8": k / v are the bf16 values rounded to OCP E4M3
    v_outlier_shift: int = 0    # > 0: V channels V_OUTLIER_DIMS scaled by 2**shift (exact in bf16)

    @property
    def offset(self) -> int:
        return self.n_kv - self.n_q if self.q_offset < 0 else self.q_offset

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv

    @property
    def n_blk(self) -> int:
        return -(-self.n_kv // self.block_size)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def shapes(self) -> dict:
        B, nq, nkv = self.batch, self.n_q, self.n_kv
        return {
            "q": (B, nq, self.h_q, self.head_dim),
            "k": (B, self.h_kv, nkv, self.head_dim),
            "v": (B, self.h_kv, nkv, self.head_dim),
            "iq": (B, nq, self.h_kv, self.index_dim),
            "ik": (B, nkv, self.index_dim),
        }

    def replace(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


def _c_plant(d_idx: int) -> float:
    return 2.0 * d_idx ** 0.25


WORKLOADS = {
    # causal prefill, 4K tokens, 4 query heads on 1 KV head, index dim 64,
    # a random direction planted in the index keys of 3 blocks
    "prefill_4k": Workload("prefill_4k", 1, 4096, 4096, 4, 1, index_dim=64, seed=1,
                           plant_m=3, plant_alpha=2.0 * math.sqrt(64), plant_beta=0.0),
    # causal prefill, 32K tokens, 64/8 heads, 4 planted blocks per group
    "prefill_32k": Workload("prefill_32k", 1, 32768, 32768, 64, 8, seed=2,
                            plant_m=4, plant_alpha=_c_plant(128), plant_beta=_c_plant(128)),
    # causal prefill, 128K tokens, 64/8 heads, no planting
    "prefill_128k": Workload("prefill_128k", 1, 131072, 131072, 64, 8, seed=3),
    # decode: 64 sequences, one new query each, 256K-token cache
    "decode_256k": Workload("decode_256k", 64, 1, 262144, 64, 8, seed=4),
    # chunked prefill: 8192 queries at the end of a 1M-token cache, 8 planted blocks per group
    "chunked_1m": Workload("chunked_1m", 1, 8192, 1048576, 64, 8, seed=5,
                           plant_m=8, plant_alpha=_c_plant(128), plant_beta=_c_plant(128)),
}


# ---------------------------------------------------------------- planting
@dataclass
class Plant:
    blocks: list = field(default_factory=list)   # per group: planted block ids
    vec_k: np.ndarray | None = None              # [h_kv, d_idx] fp32, alpha * u_g
    vec_q: np.ndarray | None = None              # [h_kv, d_idx] fp32, beta * u_g


def plant_spec(w: Workload) -> Plant:
    if w.plant_m <= 0:
        return Plant()
    d = w.index_dim
    blocks, vk, vq = [], np.zeros((w.h_kv, d), np.float32), np.zeros((w.h_kv, d), np.float32)
    for g in range(w.h_kv):
        u = bf16_to_f32(gen_range(w.seed, T_PLANT_DIR, g * d, d)).astype(np.float64)
        u = u / np.sqrt(np.sum(u * u))
        vk[g] = (w.plant_alpha * u).astype(np.float32)
        vq[g] = (w.plant_beta * u).astype(np.float32)
        chosen, r = [], 0
        m = min(w.plant_m, w.n_blk)
        while len(chosen) < m:
            h = _sm64_int((stream_key(w.seed, T_PLANT_POS) + (g << 32) + r) & _MASK64)
            t = h % w.n_blk
            if t not in chosen:
                chosen.append(int(t))
            r += 1
        blocks.append(chosen)
    return Plant(blocks, vk, vq)


def _add_bf16(rows_bits: np.ndarray, vec: np.ndarray) -> np.ndarray:
    return f32_to_bf16(bf16_to_f32(rows_bits) + vec.astype(np.float32))


# ---------------------------------------------------------------- host tensors
def host_q(w: Workload, b: int, i0: int, i1: int) -> np.ndarray:
    """Q[b, i0:i1] as bf16 bits, shape [i1-i0, h_q, d]."""
    row = w.h_q * w.head_dim
    return gen_range(w.seed, T_Q, (b * w.n_q + i0) * row, (i1 - i0) * row).reshape(i1 - i0, w.h_q, w.head_dim)


# Outlier channels of V (workloads with v_outlier_shift > 0): a few value
# channels much larger than the rest, as activation outliers make them.  Their
# bf16 values are multiplied by a power of two by adding to the exponent field,
# which is exact; zeros stay zero.
V_OUTLIER_DIMS = (0, 100)


def _outlier_bits(x: np.ndarray, shift: int) -> np.ndarray:
    x = x.copy()
    cols = x[..., list(V_OUTLIER_DIMS)]
    nz = (cols & 0x7F80) != 0
    x[..., list(V_OUTLIER_DIMS)] = np.where(nz, cols + np.uint16(shift << 7), cols)
    return x


def host_kv(w: Workload, which: str, b: int, g: int, j0: int, j1: int) -> np.ndarray:
    """K or V[b, g, j0:j1] as bf16 bits, shape [j1-j0, d]."""
    tid = T_K if which == "k" else T_V
    base = ((b * w.h_kv + g) * w.n_kv + j0) * w.head_dim
    x = gen_range(w.seed, tid, base, (j1 - j0) * w.head_dim).reshape(j1 - j0, w.head_dim)
    if which == "v" and w.v_outlier_shift > 0:
        x = _outlier_bits(x, w.v_outlier_shift)
    return x


def host_kv_blocks(w: Workload, which: str, b: int, g: int, blocks) -> dict:
    """Selected 128-token blocks of K or V for one (batch, group): {block: [rows, d]}."""
    out = {}
    for t in sorted(set(int(x) for x in blocks if x >= 0)):
        j0 = t * w.block_size
        out[t] = host_kv(w, which, b, g, j0, min(j0 + w.block_size, w.n_kv))
    return out


def host_iq(w: Workload, b: int, i0: int, i1: int, plant: Plant | None = None) -> np.ndarray:
    """index-q[b, i0:i1] as bf16 bits, shape [i1-i0, h_kv, d_idx], planting applied."""
    row = w.h_kv * w.index_dim
    x = gen_range(w.seed, T_IQ, (b * w.n_q + i0) * row, (i1 - i0) * row).reshape(i1 - i0, w.h_kv, w.index_dim)
    plant = plant_spec(w) if plant is None else plant
    if plant.vec_q is not None:
        for g in range(w.h_kv):
            x[:, g, :] = _add_bf16(x[:, g, :], plant.vec_q[g])
    return x


def host_ik(w: Workload, b: int, j0: int, j1: int, plant: Plant | None = None) -> np.ndarray:
    """index-k[b, j0:j1] as bf16 bits, shape [j1-j0, d_idx], planting applied."""
    x = gen_range(w.seed, T_IK, (b * w.n_kv + j0) * w.index_dim, (j1 - j0) * w.index_dim)
    x = x.reshape(j1 - j0, w.index_dim)
    plant = plant_spec(w) if plant is None else plant
    if plant.vec_k is not None:
        for g in range(w.h_kv):
            for t in plant.blocks[g]:
                a, z = max(t * w.block_size, j0), min((t + 1) * w.block_size, j1)
                if a < z:
                    x[a - j0:z - j0] = _add_bf16(x[a - j0:z - j0], plant.vec_k[g])
    return x


def to_e4m3(bits: np.ndarray) -> np.ndarray:
    """OCP E4M3 codes (uint8) of bf16 bit patterns, rounded to nearest even by
    torch's float8_e4m3fn conversion (the same conversion the device inputs use)."""
    import torch
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    t = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(b.shape)


def _contiguous(rows: np.ndarray) -> bool:
    return len(rows) > 1 and bool(np.all(np.diff(rows) == 1))


def host_q_rows(w: Workload, b: int, rows) -> np.ndarray:
    """Q[b, rows] for arbitrary query rows, shape [len(rows), h_q, d]."""
    rows = np.asarray(rows, dtype=np.int64)
    if _contiguous(rows):
        return host_q(w, b, int(rows[0]), int(rows[-1]) + 1)
    row = w.h_q * w.head_dim
    idx = ((b * w.n_q + rows)[:, None] * row + np.arange(row)[None, :]).reshape(-1)
    return gen_at(w.seed, T_Q, idx).reshape(len(rows), w.h_q, w.head_dim)


def host_do_rows(w: Workload, b: int, rows) -> np.ndarray:
    """The output gradient dO[b, rows] (q's layout), shape [len(rows), h_q, d]."""
    rows = np.asarray(rows, dtype=np.int64)
    row = w.h_q * w.head_dim
    idx = ((b * w.n_q + rows)[:, None] * row + np.arange(row)[None, :]).reshape(-1)
    return gen_at(w.seed, T_DO, idx).reshape(len(rows), w.h_q, w.head_dim)


def device_dout(w: Workload, device="cuda:0"):
    """The output gradient dO of a workload (q's shape), generated on the device."""
    import torch
    t = torch.empty(w.shapes()["q"], dtype=torch.bfloat16, device=device)
    device_fill(w, "do", t)
    torch.cuda.synchronize(device)
    return t


def host_iq_rows(w: Workload, b: int, rows, plant: Plant | None = None) -> np.ndarray:
    """index-q[b, rows] for arbitrary query rows, shape [len(rows), h_kv, d_idx], planted."""
    rows = np.asarray(rows, dtype=np.int64)
    if _contiguous(rows):
        return host_iq(w, b, int(rows[0]), int(rows[-1]) + 1, plant)
    row = w.h_kv * w.index_dim
    idx = ((b * w.n_q + rows)[:, None] * row + np.arange(row)[None, :]).reshape(-1)
    x = gen_at(w.seed, T_IQ, idx).reshape(len(rows), w.h_kv, w.index_dim)
    plant = plant_spec(w) if plant is None else plant
    if plant.vec_q is not None:
        for g in range(w.h_kv):
            x[:, g, :] = _add_bf16(x[:, g, :], plant.vec_q[g])
    return x


def host_all(w: Workload) -> dict:
    """Every input tensor on the host (small workloads only)."""
    B = w.batch
    p = plant_spec(w)
    return {
        "q": np.stack([host_q(w, b, 0, w.n_q) for b in range(B)]),
        "k": np.stack([np.stack([host_kv(w, "k", b, g, 0, w.n_kv) for g in range(w.h_kv)]) for b in range(B)]),
        "v": np.stack([np.stack([host_kv(w, "v", b, g, 0, w.n_kv) for g in range(w.h_kv)]) for b in range(B)]),
        "iq": np.stack([host_iq(w, b, 0, w.n_q, p) for b in range(B)]),
        "ik": np.stack([host_ik(w, b, 0, w.n_kv, p) for b in range(B)]),
    }


# ---------------------------------------------------------------- device fill
_HERE = os.path.dirname(os.path.abspath(__file__))
DEV_LIB = os.path.join(_HERE, "libmsa_synth.so")
DEV_SRC = os.path.join(_HERE, "synth_dev.hip")
_dev = None


def build_device(force: bool = False) -> str:
    """Compile the device generator for gfx950 (hipcc, no GPU needed)."""
    import subprocess
    if force or not os.path.exists(DEV_LIB):
        tmp = DEV_LIB + ".tmp"
        cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               DEV_SRC, "-o", tmp]
        subprocess.run(cmd, check=True, stderr=subprocess.DEVNULL if not force else None)
        os.replace(tmp, DEV_LIB)
    return DEV_LIB


def _devlib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            build_device()
        lib = ctypes.CDLL(DEV_LIB)
        lib.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                   ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_fill.restype = ctypes.c_int
        lib.synth_add_rows.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_add_rows.restype = ctypes.c_int
        _dev = lib
    return _dev


def device_fill(w: Workload, name: str, tensor, stream=None, nt_dev=None):
    """Fill a device tensor (torch, bf16, canonical layout) with generator values."""
    import torch
    tid = {"q": T_Q, "k": T_K, "v": T_V, "iq": T_IQ, "ik": T_IK, "do": T_DO}[name]
    assert tensor.is_contiguous() and tensor.element_size() == 2
    assert tuple(tensor.shape) == w.shapes()["q" if name == "do" else name], (tensor.shape, w.shapes()[name])
    if nt_dev is None:
        nt_dev = torch.from_numpy(normal_table().view(np.int16).copy()).to(tensor.device)
    s = (stream or torch.cuda.current_stream(tensor.device)).cuda_stream
    rc = _devlib().synth_fill(tensor.data_ptr(), tensor.numel(), stream_key(w.seed, tid),
                              nt_dev.data_ptr(), s)
    if rc != 0:
        raise RuntimeError(f"synth_fill failed ({rc})")
    plant = plant_spec(w)
    if plant.vec_k is not None and name in ("iq", "ik"):
        lib = _devlib()
        for g in range(w.h_kv):
            if name == "iq":
                vec = torch.from_numpy(plant.vec_q[g].copy()).to(tensor.device)
                # rows (b, i, g): start g*d_idx, stride h_kv*d_idx, count batch*n_q
                rc = lib.synth_add_rows(tensor.data_ptr(), g * w.index_dim, w.h_kv * w.index_dim,
                                        w.batch * w.n_q, 0, w.index_dim, vec.data_ptr(), s)
                if rc != 0:
                    raise RuntimeError("synth_add_rows failed")
            else:
                vec = torch.from_numpy(plant.vec_k[g].copy()).to(tensor.device)
                for b in range(w.batch):
                    for t in plant.blocks[g]:
                        j0 = t * w.block_size
                        cnt = min(w.block_size, w.n_kv - j0)
                        rc = lib.synth_add_rows(tensor.data_ptr(), (b * w.n_kv + j0) * w.index_dim,
                                                w.index_dim, cnt, 0, w.index_dim, vec.data_ptr(), s)
                        if rc != 0:
                            raise RuntimeError("synth_add_rows failed")
            # keep vec alive until the stream has consumed it
            torch.cuda.current_stream(tensor.device).synchronize() if stream is None else stream.synchronize()
    return tensor


def device_inputs(w: Workload, device="cuda:0") -> dict:
    """All five input tensors of a workload, generated on the device.  With
    index_dtype "fp8", index_q and index_k are uint8 tensors of E4M3 codes;
    with kv_dtype "fp8", k and v are."""
    import torch
    nt = torch.from_numpy(normal_table().view(np.int16).copy()).to(device)
    out = {}
    for name, shp in w.shapes().items():
        t = torch.empty(shp, dtype=torch.bfloat16, device=device)
        device_fill(w, name, t, nt_dev=nt)
        if name == "v" and w.v_outlier_shift > 0:
            bits = t.view(torch.int16)
            for c in V_OUTLIER_DIMS:
                col = bits[..., c]
                col.copy_(torch.where((col & 0x7F80) != 0, col + (w.v_outlier_shift << 7), col))
        if (w.index_dtype == "fp8" and name in ("iq", "ik")) or (w.kv_dtype == "fp8" and name in ("k", "v")):
            t = t.to(torch.float8_e4m3fn).view(torch.uint8)
        out[name] = t
    torch.cuda.synchronize(device)
    return out
