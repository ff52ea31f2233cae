"""Seeded synthetic inputs for block-sparse GQA attention (MiniMax-style sparse attention).

This module draws random numbers, rounds them to the storage types the kernels consume
(bf16, or OCP fp8 e4m3fn with a per-tensor scale) and does shape bookkeeping. It holds
none of the method's arithmetic: no scores, no selection, no softmax. The CPU oracle, the
GPU tests and the benchmark all build their inputs here, so both sides of every parity
check see bit-identical values.

Determinism: every named tensor has its own child of ``numpy.random.SeedSequence(seed)``
(fixed child index per name), and large tensors are drawn in fixed-size chunks, each from
its own grandchild sequence. The values therefore depend only on (seed, name, shape), not
on the number of threads used to draw them.

Workloads follow the shapes of the pages: the MiniMax M3 attention shapes (Hq=64, Hkv=4,
D=128, 128-token blocks, top-16) from "Kernel optimization for MiniMax M3 on NVIDIA
Blackwell" (summary section), and the per-Q-tile block lists of "Sparse Attention"
(Chapters 1-3). The pages use plain synthetic Gaussian data ("Sparse Attention", Chapter 4:
all tests use synthetic data).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

# Child index of each named stream under SeedSequence(seed).
_STREAMS = {
    "q": 0, "k": 1, "v": 2, "q_idx": 3, "k_idx": 4,
    "bias_proxy": 5, "bias_main": 6, "lists": 7, "lengths": 8, "dout": 9,
}
_CHUNK = 1 << 22          # elements per independently seeded chunk
FP8_MAX = 448.0           # largest finite OCP e4m3fn magnitude


def _threads() -> int:
    n = os.environ.get("MSA_GEN_THREADS")
    if n:
        return max(1, int(n))
    return max(1, min(16, os.cpu_count() or 1))


def child(ss: np.random.SeedSequence, i: int) -> np.random.SeedSequence:
    """The i-th child of ``ss`` (what ``ss.spawn`` would give, without mutating ``ss``)."""
    return np.random.SeedSequence(ss.entropy, spawn_key=tuple(ss.spawn_key) + (i,),
                                  pool_size=ss.pool_size)


def _stream(seed: int, name: str) -> np.random.SeedSequence:
    return child(np.random.SeedSequence(seed), _STREAMS[name])


def normal_f32(ss: np.random.SeedSequence, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) float32 array of ``shape``, chunk-seeded so threads do not matter."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.float32)
    nchunk = max(1, -(-n // _CHUNK))
    kids = [child(ss, c) for c in range(nchunk)]

    def fill(c: int) -> None:
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        np.random.default_rng(kids[c]).standard_normal(out=out[lo:hi], dtype=np.float32)

    if nchunk == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunk)))
    if std != 1.0:
        out *= np.float32(std)
    return out.reshape(shape)


def grid_f32(ss: np.random.SeedSequence, shape) -> np.ndarray:
    """Values drawn uniformly from {-16, ..., 16} / 4: exact in bf16, and every dot product
    of up to 64 of them is exact in fp32 whatever the summation order."""
    rng = np.random.default_rng(ss)
    return (rng.integers(-16, 17, size=shape).astype(np.float32) / np.float32(4.0))


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """Round float32 to bfloat16, round-to-nearest-even (torch's CPU conversion)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def to_fp8(x: np.ndarray) -> tuple[torch.Tensor, float]:
    """Per-tensor quantisation to OCP fp8 e4m3fn: scale = amax / 448, value = RNE(x / scale)
    saturated to +-448. Returns (codes as torch.float8_e4m3fn, descale = scale)."""
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    scale = amax / FP8_MAX if amax > 0 else 1.0
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = (t / scale).clamp_(-FP8_MAX, FP8_MAX)
    return t.to(torch.float8_e4m3fn), scale


E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])   # magnitudes of codes 0..7


def to_mxfp4(x: np.ndarray) -> tuple[torch.Tensor, torch.Tensor]:
    """Prepares 4-bit index vectors (OCP MXFP4) from float32 rows [..., dp], dp % 32 == 0.

    Every 32 consecutive elements share the scale 2^X with X = floor(log2(amax)) - 2 (the
    largest E2M1 exponent), clamped to [-127, 127], X = 0 for an all-zero group; each element
    x / 2^X is rounded to the nearest E2M1 magnitude, ties to the code with a zero mantissa
    bit, magnitudes past 6 saturating to 6; the sign bit is set for negative x. Returns
    (packed codes uint8 [..., dp / 2], element 2i in the low nibble of byte i; E8M0 scale codes
    uint8 [..., dp / 32] = X + 127).
    """
    x = np.asarray(x, dtype=np.float64)
    dp = x.shape[-1]
    assert dp % 32 == 0, dp
    g = x.reshape(x.shape[:-1] + (dp // 32, 32))
    amax = np.abs(g).max(axis=-1)
    _, e = np.frexp(amax)                         # amax = f * 2^e, f in [0.5, 1)
    xexp = np.where(amax > 0, np.clip(e - 1 - 2, -127, 127), 0)
    mag = np.abs(g) / np.exp2(xexp)[..., None]
    mid = (E2M1_GRID[1:] + E2M1_GRID[:-1]) / 2
    lo = np.searchsorted(mid, mag, side="left")
    hi = np.searchsorted(mid, mag, side="right")
    k = np.where((lo != hi) & (lo % 2 == 1), hi, lo)   # a tie takes the even code
    codes = (k | np.where(g < 0, 8, 0)).astype(np.uint8).reshape(x.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return (torch.from_numpy(np.ascontiguousarray(packed)),
            torch.from_numpy(np.ascontiguousarray((xexp + 127).astype(np.uint8))))


def widen(t: torch.Tensor, descale: float = 1.0) -> np.ndarray:
    """Exact value of a stored bf16/fp8 tensor as float64 (times its descale)."""
    a = t.to(torch.float64).numpy()
    return a * descale if descale != 1.0 else a


# ----------------------------------------------------------------------------- configs

@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    n_q: tuple              # per-sequence query counts
    n_k: tuple              # per-sequence key counts
    hq: int
    hkv: int
    d: int = 128
    block: int = 128
    topk: int = 16
    dp: int = 64
    causal: bool = True
    dtype: str = "bf16"     # "bf16" or "fp8" for Q/K/V
    idx_dtype: str = "bf16"  # "bf16", "fp8" (e4m3fn, per-tensor scale) or "mxfp4" proxies
    lowrank: bool = False   # rank-8 per-group bias giving block reuse
    list_q: int = 1         # 1: per-query selection by the index branch; 128: given per-tile lists
    list_pool: int = 0      # per-tile lists: blocks drawn from range(list_pool)
    selector: int = 0       # per-tile lists chosen by the R1 (1) or R4 (4) selector, not drawn
    proxy: str = "normal"   # "normal" or "grid"
    length_seed_draw: Optional[tuple] = None  # decode: (R, lo_blocks, hi_blocks) drawn per seed

    @property
    def group(self) -> int:
        return self.hq // self.hkv


def _cfg(name, n, nk, **kw) -> Config:
    b = kw.pop("batch", 1)
    return Config(name=name, batch=b, n_q=tuple([n] * b), n_k=tuple([nk] * b), **kw)


# The five workloads, by what they are. Sizes: "Kernel optimization for MiniMax M3 on NVIDIA
# Blackwell" (summary: Hq=64, Hkv=4, D=128, block=128, topK=16) and "Sparse Attention"
# (Chapter 3: 16 of the 128-token blocks per Q128 tile).
CONFIGS = {
    # tiny MSA prefill: 2048 causal, Hq=16, Hkv=1, top-4, proxy dim 32
    "tiny": _cfg("tiny", 2048, 2048, hq=16, hkv=1, topk=4, dp=32),
    # per-Q-tile lists: 8192 non-causal, Hq=Hkv=16, 16 of 64 blocks per (tile, head)
    "qtile": _cfg("qtile", 8192, 8192, hq=16, hkv=16, topk=16, causal=False,
                  list_q=128, list_pool=64),
    # M3-shape prefill: 32768 causal, Hq=64, Hkv=4, top-16, proxy dim 64, rank-8 bias
    "m3": _cfg("m3", 32768, 32768, hq=64, hkv=4, topk=16, dp=64, lowrank=True),
    # long-context fp8 prefill: 131072 causal, M3 heads, fp8 e4m3 Q/K/V, bf16 proxies
    "m3_fp8_long": _cfg("m3_fp8_long", 131072, 131072, hq=64, hkv=4, topk=16, dp=64,
                        lowrank=True, dtype="fp8"),
    # decode: 64 requests x 1 query, key lengths uniform over multiples of 128 in [16K, 128K]
    "decode": Config(name="decode", batch=64, n_q=(), n_k=(), hq=64, hkv=4, topk=16, dp=64,
                     length_seed_draw=(64, 128, 1024)),
    # selector -> per-tile attention ("Sparse Attention", Chapter 4 benchmark): B=2, 4096
    # queries, 16K keys, 16 query heads on one KV head, 16 blocks per Q128 tile, non-causal
    "sel_r1": _cfg("sel_r1", 4096, 16384, batch=2, hq=16, hkv=1, topk=16, causal=False,
                   list_q=128, selector=1),
    "sel_r4": _cfg("sel_r4", 4096, 16384, batch=2, hq=16, hkv=1, topk=16, causal=False,
                   list_q=128, selector=4),
    # the same two workloads with the proxies quantised to fp8 e4m3 (low-precision scoring)
    "m3_fp8_long_i8": _cfg("m3_fp8_long_i8", 131072, 131072, hq=64, hkv=4, topk=16, dp=64,
                           lowrank=True, dtype="fp8", idx_dtype="fp8"),
    "decode_i8": Config(name="decode_i8", batch=64, n_q=(), n_k=(), hq=64, hkv=4, topk=16, dp=64,
                        length_seed_draw=(64, 128, 1024), idx_dtype="fp8"),
    # and with 4-bit (MXFP4) proxies ("Sparse Attention", Chapter 4: the FP4 scorer)
    "m3_fp8_long_i4": _cfg("m3_fp8_long_i4", 131072, 131072, hq=64, hkv=4, topk=16, dp=64,
                           lowrank=True, dtype="fp8", idx_dtype="mxfp4"),
    "decode_i4": Config(name="decode_i4", batch=64, n_q=(), n_k=(), hq=64, hkv=4, topk=16, dp=64,
                        length_seed_draw=(64, 128, 1024), idx_dtype="mxfp4"),
}


def custom(name="custom", n_q=(256,), n_k=None, **kw) -> Config:
    """A small config for tests. ``n_q``/``n_k`` are per-sequence lengths."""
    n_q = tuple(n_q)
    n_k = tuple(n_k) if n_k is not None else n_q
    return Config(name=name, batch=len(n_q), n_q=n_q, n_k=n_k, **kw)


def scaled(cfg: Config, n: int) -> Config:
    """The same workload at a different (single-sequence) length."""
    return Config(**{**cfg.__dict__, "name": f"{cfg.name}@{n}", "batch": 1,
                     "n_q": (n,), "n_k": (n,)})


# ----------------------------------------------------------------------------- cases

@dataclass
class Case:
    cfg: Config
    seed: int
    cu_q: np.ndarray            # int32 [B+1]
    cu_k: np.ndarray            # int32 [B+1]
    q: torch.Tensor             # [Tq, Hq, D] bf16 or float8_e4m3fn
    k: torch.Tensor             # [Tk, Hkv, D]
    v: torch.Tensor             # [Tk, Hkv, D]
    descale: tuple              # (dq, dk, dv); (1,1,1) for bf16
    q_idx: Optional[torch.Tensor] = None   # [Tq, Hkv, dp] bf16 / float8_e4m3fn, mxfp4: uint8 [.., dp/2]
    k_idx: Optional[torch.Tensor] = None   # [Tk, Hkv, dp]
    lists: Optional[np.ndarray] = None     # [Tq/list_q, Hkv, K] int32 for given lists
    softmax_scale: float = 0.0
    meta: dict = field(default_factory=dict)
    idx_descale: tuple = (1.0, 1.0)        # (descale of q_idx, of k_idx); (1, 1) for bf16
    q_idx_scale: Optional[torch.Tensor] = None   # mxfp4: E8M0 codes uint8 [Tq, Hkv, dp / 32]
    k_idx_scale: Optional[torch.Tensor] = None   # mxfp4: [Tk, Hkv, dp / 32]

    @property
    def total_q(self) -> int:
        return int(self.cu_q[-1])

    @property
    def total_k(self) -> int:
        return int(self.cu_k[-1])

    @property
    def max_q(self) -> int:
        return int(np.max(np.diff(self.cu_q))) if len(self.cu_q) > 1 else 0

    @property
    def max_k(self) -> int:
        return int(np.max(np.diff(self.cu_k))) if len(self.cu_k) > 1 else 0


def _lengths(cfg: Config, seed: int) -> tuple[np.ndarray, np.ndarray]:
    if cfg.length_seed_draw is not None:
        r, lo, hi = cfg.length_seed_draw
        rng = np.random.default_rng(_stream(seed, "lengths"))
        nk = 128 * rng.integers(lo, hi, size=r, endpoint=True)
        nq = np.ones(r, dtype=np.int64)
    else:
        nq = np.asarray(cfg.n_q, dtype=np.int64)
        nk = np.asarray(cfg.n_k, dtype=np.int64)
    cu_q = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(nk)]).astype(np.int32)
    return cu_q, cu_k


def _lowrank_factors(ss: np.random.SeedSequence, n_grp: int, width: int) -> np.ndarray:
    """One factor U_g (width x 8, entries N(0, 1/8)) per KV group, shared by both sides."""
    return normal_f32(ss, (n_grp, width, 8), std=math.sqrt(1.0 / 8.0))


def _add_lowrank(x: np.ndarray, side: str, cu: np.ndarray, u: np.ndarray, ss,
                 heads_per_factor: int, block: int) -> None:
    """Rank-8 bias giving block reuse (in place, float32).

    Query side, per head h of ``x`` with g = h // heads_per_factor:
    x[i, h] += U_g (a_h + 0.5 e_{i,h}), a_h and e_{i,h} ~ N(0, I_8).
    Key side, per KV head g: x[u, g] += U_g b_{g, block(u)}, b ~ N(0, I_8) constant over each
    128-token block of each sequence. Sub-streams of ``ss``: 0 offsets, 1 noise, 2 codes."""
    n_tok, n_head, _ = x.shape
    subs = [child(ss, i) for i in range(3)]
    if side == "q":
        a = normal_f32(subs[0], (n_head, 8))
        e = normal_f32(subs[1], (n_tok, n_head, 8))
        for h in range(n_head):
            coef = a[h][None, :] + np.float32(0.5) * e[:, h, :]
            x[:, h, :] += coef @ u[h // heads_per_factor].T
    else:
        nb_tot = sum(-(-int(cu[s + 1] - cu[s]) // block) for s in range(len(cu) - 1))
        codes = normal_f32(subs[2], (nb_tot, n_head, 8))
        blk_of_tok = np.empty(n_tok, dtype=np.int64)
        base = 0
        for s in range(len(cu) - 1):
            n = int(cu[s + 1] - cu[s])
            blk_of_tok[cu[s]:cu[s + 1]] = base + np.arange(n) // block
            base += -(-n // block)
        for h in range(n_head):
            x[:, h, :] += codes[blk_of_tok, h, :] @ u[h].T


def make_case(cfg: Config | str, seed: int = 0, with_proxies: Optional[bool] = None) -> Case:
    """Draw one seeded input set for ``cfg``."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    cu_q, cu_k = _lengths(cfg, seed)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    hq, hkv, d, dp = cfg.hq, cfg.hkv, cfg.d, cfg.dp
    g = hq // hkv

    q = normal_f32(_stream(seed, "q"), (tq, hq, d))
    k = normal_f32(_stream(seed, "k"), (tk, hkv, d))
    v = normal_f32(_stream(seed, "v"), (tk, hkv, d))
    if cfg.lowrank:
        ssm = [child(_stream(seed, "bias_main"), i) for i in range(3)]
        um = _lowrank_factors(ssm[0], hkv, d)
        _add_lowrank(q, "q", cu_q, um, ssm[1], g, cfg.block)
        _add_lowrank(k, "k", cu_k, um, ssm[2], 1, cfg.block)

    if cfg.dtype == "fp8":
        qs, dq = to_fp8(q)
        ks, dk = to_fp8(k)
        vs, dv = to_fp8(v)
        descale = (dq, dk, dv)
    elif cfg.dtype == "bf16":
        qs, ks, vs = to_bf16(q), to_bf16(k), to_bf16(v)
        descale = (1.0, 1.0, 1.0)
    else:
        raise ValueError(f"unknown dtype {cfg.dtype}")
    del q, k, v

    if with_proxies is None:
        with_proxies = cfg.list_q == 1
    q_idx = k_idx = None
    idx_descale = (1.0, 1.0)
    q_isc = k_isc = None
    if with_proxies:
        if cfg.proxy == "grid":
            qi = grid_f32(_stream(seed, "q_idx"), (tq, hkv, dp))
            ki = grid_f32(_stream(seed, "k_idx"), (tk, hkv, dp))
        else:
            qi = normal_f32(_stream(seed, "q_idx"), (tq, hkv, dp))
            ki = normal_f32(_stream(seed, "k_idx"), (tk, hkv, dp))
            if cfg.lowrank:
                ssp = [child(_stream(seed, "bias_proxy"), i) for i in range(3)]
                up = _lowrank_factors(ssp[0], hkv, dp)
                _add_lowrank(qi, "q", cu_q, up, ssp[1], 1, cfg.block)
                _add_lowrank(ki, "k", cu_k, up, ssp[2], 1, cfg.block)
        if cfg.idx_dtype == "fp8" and cfg.proxy == "grid":
            # every grid value {-16..16}/4 is an e4m3 code: stored as is, descale 1
            q_idx = torch.from_numpy(qi).to(torch.float8_e4m3fn)
            k_idx = torch.from_numpy(ki).to(torch.float8_e4m3fn)
        elif cfg.idx_dtype == "fp8":
            q_idx, dqi = to_fp8(qi)
            k_idx, dki = to_fp8(ki)
            idx_descale = (dqi, dki)
        elif cfg.idx_dtype == "mxfp4":
            q_idx, q_isc = to_mxfp4(qi)
            k_idx, k_isc = to_mxfp4(ki)
        elif cfg.idx_dtype == "bf16":
            q_idx, k_idx = to_bf16(qi), to_bf16(ki)
        else:
            raise ValueError(f"unknown idx_dtype {cfg.idx_dtype}")

    lists = None
    if cfg.list_q > 1 and cfg.selector == 0:
        lists = tile_lists(cfg, cu_q, seed)

    return Case(cfg=cfg, seed=seed, cu_q=cu_q, cu_k=cu_k, q=qs, k=ks, v=vs, descale=descale,
                q_idx=q_idx, k_idx=k_idx, lists=lists,
                softmax_scale=1.0 / math.sqrt(d), idx_descale=idx_descale,
                q_idx_scale=q_isc, k_idx_scale=k_isc)


def tile_lists(cfg: Config, cu_q: np.ndarray, seed: int) -> np.ndarray:
    """Per-(Q tile, KV head) block lists: ``topk`` distinct blocks drawn uniformly without
    replacement from ``range(list_pool)``, sorted ascending (the "Sparse Attention" page,
    Chapter 3, draws independent lists per Q128 tile). Shape [B * tiles_max, Hkv, K] with
    tiles_max = ceil(max_q / list_q); row s * tiles_max + t is tile t of sequence s (rows past
    a sequence's last tile hold -1)."""
    rng = np.random.default_rng(_stream(seed, "lists"))
    nq = np.diff(cu_q)
    tiles_max = -(-int(nq.max()) // cfg.list_q) if nq.size else 0
    out = np.full((len(nq) * tiles_max, cfg.hkv, cfg.topk), -1, dtype=np.int32)
    for s in range(len(nq)):
        for t in range(-(-int(nq[s]) // cfg.list_q)):
            for h in range(cfg.hkv):
                out[s * tiles_max + t, h] = np.sort(rng.choice(cfg.list_pool, cfg.topk,
                                                               replace=False))
    return out


def grad_output(case: Case, seed: Optional[int] = None) -> torch.Tensor:
    """Seeded upstream gradient dO for the backward: N(0, 1) bf16 [Tq, Hq, D]."""
    cfg = case.cfg
    ss = _stream(case.seed if seed is None else seed, "dout")
    return to_bf16(normal_f32(ss, (case.total_q, cfg.hq, cfg.d)))


def shared_lists(n_q: int, n_req: int, n_blocks: int, hkv: int, topk: int, seed: int) -> np.ndarray:
    """Per-query block lists [n_req * n_q, hkv, topk] in which the n_q queries of each request
    share one list per group: topk distinct blocks of the request's n_blocks, drawn uniformly
    without replacement and sorted (a workload whose block reuse nsb / N is hkv * topk / n_q)."""
    rng = np.random.default_rng(_stream(seed, "lists"))
    out = np.empty((n_req * n_q, hkv, topk), dtype=np.int32)
    for r in range(n_req):
        for g in range(hkv):
            out[r * n_q:(r + 1) * n_q, g] = np.sort(rng.choice(n_blocks, topk, replace=False))
    return out
