"""Seeded synthetic workloads for the block-sparse prefill path.

This module only *draws inputs*: Gaussian block-structured Q/K/V, rounded to
bf16 bit patterns or quantised to OCP e4m3fn codes with per-head scales,
ragged sequence lengths and a paged-KV page table.  It holds none of the
method's arithmetic (no pooling, scoring, thresholding or attention), so both
the fp64 oracle and the HIP path can consume what it produces without sharing
any code with each other.

Workload recipe (a synthetic stand-in for the long-context model workloads
that the FlashPrefill pages measure on; no benchmark item is reproduced):

* every tensor X (Q per query head, K and V per KV head) is
  ``X[t] = mu[block(t)] + 0.3 * eps[t]`` with ``mu[b] ~ N(0, I_d)`` per 128-token
  block and ``eps[t] ~ N(0, I_d)``, computed in fp32;
* vertical pattern: a unit vector ``u_g`` per KV head is added to every query
  of that group and ``3 * u_g`` to the keys of a few randomly chosen key blocks;
* slash pattern (optional): 16 unit vectors ``w_{g,r}`` per KV head; token t
  with ``r = (t // 128) % 16`` gets ``+w_{g,r}`` on its queries and
  ``+3 * w_{g,r}`` on its keys, so query block i and key block j share a
  component whenever ``(i - j) % 16 == 0`` (offsets of k * 2048 tokens);
* bf16 values are round-to-nearest-even of the fp32 values; fp8 values are
  ``code = RNE(x / s)`` saturated to +-448 with ``s = amax_head / 448`` (fp32).

Seeds: workload k uses ``SeedSequence(1000 + k)`` split into eight
independent streams (Q, K, V, vertical boosts, slash vectors, lengths, pages,
spare); every (sequence, head) gets its own child stream, so heads can be
drawn in parallel threads and the result does not depend on thread count.
"""
from __future__ import annotations

import hashlib
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

BLOCK = 128
HEAD_DIM = 128
NOISE_SD = 0.3
VERTICAL_GAIN = 3.0
SLASH_PERIOD_BLOCKS = 16
FP8_MAX = 448.0

_STREAM_Q, _STREAM_K, _STREAM_V, _STREAM_VERT, _STREAM_SLASH, _STREAM_LEN, _STREAM_PAGES, _STREAM_SPARE = range(8)


@dataclass
class Workload:
    """One synthetic prefill batch.

    Token-major packed layouts: ``q`` is ``[T, hq, d]`` and ``k``/``v`` are
    ``[T, hkv, d]`` with the sequences back to back (``cu_seqlens`` gives the
    offsets).  bf16 tensors hold raw bit patterns (uint16); fp8 tensors hold
    e4m3fn codes (uint8) with fp32 per-head scales.  When ``paged`` is set,
    ``k_cache``/``v_cache`` hold the same K/V values scattered into
    ``[num_pages, 128, hkv, d]`` pages at ``page_table[s, j]`` (logical block j
    of sequence s); unused tail slots of a page are zero and unused page-table
    entries are -1.
    """

    name: str
    hq: int
    hkv: int
    d: int
    block: int
    dtype: str
    lengths: list
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_scale: Optional[np.ndarray] = None
    k_scale: Optional[np.ndarray] = None
    v_scale: Optional[np.ndarray] = None
    alphas: tuple = (0.1,)
    n_sink: int = 1
    n_local: int = 4
    paged: bool = False
    page_table: Optional[np.ndarray] = None
    k_cache: Optional[np.ndarray] = None
    v_cache: Optional[np.ndarray] = None
    vertical_blocks: dict = field(default_factory=dict)

    @property
    def n_seqs(self) -> int:
        return len(self.lengths)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.lengths))

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int32)

    @property
    def seq_blocks(self) -> list:
        return [-(-int(n) // self.block) for n in self.lengths]

    @property
    def cu_blocks(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seq_blocks)]).astype(np.int32)

    @property
    def L(self) -> int:
        assert self.n_seqs == 1
        return int(self.lengths[0])

    def digests(self) -> dict:
        out = {}
        for name in ("q", "k", "v", "q_scale", "k_scale", "v_scale", "page_table", "k_cache", "v_cache"):
            a = getattr(self, name)
            if a is not None:
                out[name] = hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]
        return out


def _unit(rng: np.random.Generator, d: int) -> np.ndarray:
    x = rng.standard_normal(d)
    return (x / np.linalg.norm(x)).astype(np.float32)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def quantize_e4m3fn(x: np.ndarray):
    """fp32 values of one head -> (e4m3fn codes, fp32 scale) with scale = amax/448."""
    import torch

    amax = np.float32(np.max(np.abs(x)))
    scale = np.float32(amax / np.float32(FP8_MAX)) if amax > 0 else np.float32(1.0)
    y = np.clip(x / scale, -FP8_MAX, FP8_MAX).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def _draw_head(ss: np.random.SeedSequence, n: int, d: int, block: int, add, mean_scale: float = 1.0) -> np.ndarray:
    """fp32 [n, d] block-structured Gaussian head, plus additive pattern terms."""
    rng = np.random.default_rng(ss)
    nb = -(-n // block)
    mu = rng.standard_normal((nb, d), dtype=np.float32)
    if mean_scale != 1.0:
        mu *= np.float32(mean_scale)
    x = rng.standard_normal((n, d), dtype=np.float32)
    x *= np.float32(NOISE_SD)
    x += np.repeat(mu, block, axis=0)[:n]
    if add is not None:
        add(x)
    return x


def make_workload(
    name: str,
    hq: int,
    hkv: int,
    lengths: Sequence[int],
    *,
    seed: int,
    dtype: str = "bf16",
    vertical: Optional[int] = None,
    vertical_frac: float = 0.02,
    slash: bool = True,
    mean_scale: float = 1.0,
    vertical_gain: float = VERTICAL_GAIN,
    slash_period: int = SLASH_PERIOD_BLOCKS,
    paged: bool = False,
    alphas=(0.1,),
    n_sink: int = 1,
    n_local: int = 4,
    d: int = HEAD_DIM,
    block: int = BLOCK,
    threads: int = 8,
) -> Workload:
    """Draw one workload; ``vertical`` fixes the number of boosted key blocks per
    KV head (else ``round(vertical_frac * nb)`` per sequence).  ``mean_scale`` scales the
    per-block means, ``vertical_gain`` the key-side boost of the vertical and slash
    patterns and ``slash_period`` the slash spacing in blocks (the defaults give the
    standard workloads)."""
    assert hq % hkv == 0 and dtype in ("bf16", "fp8")
    lengths = [int(n) for n in lengths]
    group = hq // hkv
    streams = np.random.SeedSequence(seed).spawn(8)
    n_seqs = len(lengths)
    per_seq = [s.spawn(n_seqs) for s in streams]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(cu[-1])

    # pattern vectors per sequence (drawn serially: tiny)
    pattern = []
    vert_blocks = {}
    for s, n in enumerate(lengths):
        nb = -(-n // block)
        rv = np.random.default_rng(per_seq[_STREAM_VERT][s])
        rs = np.random.default_rng(per_seq[_STREAM_SLASH][s])
        nv = vertical if vertical is not None else int(round(vertical_frac * nb))
        nv = min(nv, nb)
        u = [_unit(rv, d) for _ in range(hkv)]
        vb = [np.sort(rv.choice(nb, size=nv, replace=False)) for _ in range(hkv)]
        w = [[_unit(rs, d) for _ in range(slash_period)] for _ in range(hkv)] if slash else None
        pattern.append((u, vb, w))
        for g in range(hkv):
            vert_blocks[(s, g)] = vb[g].tolist()

    def slash_rows(n, wg):
        r = (np.arange(n) // block) % slash_period
        return np.stack(wg)[r]

    def q_add(s, g):
        u, vb, w = pattern[s]

        def f(x):
            x += u[g]
            if w is not None:
                x += slash_rows(x.shape[0], w[g])
        return f

    def k_add(s, g):
        u, vb, w = pattern[s]

        def f(x):
            for b in vb[g]:
                x[b * block:(b + 1) * block] += np.float32(vertical_gain) * u[g]
            if w is not None:
                x += np.float32(vertical_gain) * slash_rows(x.shape[0], w[g])
        return f

    store = np.uint16 if dtype == "bf16" else np.uint8
    q = np.empty((T, hq, d), dtype=store)
    k = np.empty((T, hkv, d), dtype=store)
    v = np.empty((T, hkv, d), dtype=store)

    # fp8: per-head scales over the whole batch (a head's amax spans all sequences)
    raw = {} if dtype == "fp8" else None
    jobs = []
    for s, n in enumerate(lengths):
        hs_q = per_seq[_STREAM_Q][s].spawn(hq)
        hs_k = per_seq[_STREAM_K][s].spawn(hkv)
        hs_v = per_seq[_STREAM_V][s].spawn(hkv)
        for h in range(hq):
            jobs.append(("q", s, h, hs_q[h], q_add(s, h // group)))
        for g in range(hkv):
            jobs.append(("k", s, g, hs_k[g], k_add(s, g)))
            jobs.append(("v", s, g, hs_v[g], None))
    dst = {"q": q, "k": k, "v": v}

    def run(job):
        name_, s, h, ss, add = job
        n = lengths[s]
        x = _draw_head(ss, n, d, block, add, mean_scale)
        if dtype == "bf16":
            dst[name_][cu[s]:cu[s] + n, h, :] = round_to_bf16_bits(x)
        else:
            raw[(name_, s, h)] = x

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(run, jobs))

    q_scale = k_scale = v_scale = None
    if dtype == "fp8":
        q_scale = np.zeros(hq, np.float32)
        k_scale = np.zeros(hkv, np.float32)
        v_scale = np.zeros(hkv, np.float32)
        heads = [("q", h) for h in range(hq)] + [("k", g) for g in range(hkv)] + [("v", g) for g in range(hkv)]

        def quant(item):
            name_, h = item
            x = np.concatenate([raw[(name_, s, h)] for s in range(n_seqs)], axis=0)
            codes, sc = quantize_e4m3fn(x)
            dst[name_][:, h, :] = codes
            {"q": q_scale, "k": k_scale, "v": v_scale}[name_][h] = sc

        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(quant, heads))
        raw.clear()

    wl = Workload(name=name, hq=hq, hkv=hkv, d=d, block=block, dtype=dtype, lengths=lengths,
                  q=q, k=k, v=v, q_scale=q_scale, k_scale=k_scale, v_scale=v_scale,
                  alphas=tuple(alphas), n_sink=n_sink, n_local=n_local, paged=paged,
                  vertical_blocks=vert_blocks)
    if paged:
        _page(wl, np.random.default_rng(streams[_STREAM_PAGES]))
    return wl


def _page(wl: Workload, rng: np.random.Generator) -> None:
    """Scatter K/V into 128-token pages under a random page permutation."""
    B = wl.block
    nbs = wl.seq_blocks
    P = int(sum(nbs))
    perm = rng.permutation(P).astype(np.int32)
    max_pages = max(nbs)
    table = np.full((wl.n_seqs, max_pages), -1, dtype=np.int32)
    kc = np.zeros((P, B, wl.hkv, wl.d), dtype=wl.k.dtype)
    vc = np.zeros_like(kc)
    cu = wl.cu_seqlens
    cb = wl.cu_blocks
    for s, n in enumerate(wl.lengths):
        for j in range(nbs[s]):
            p = perm[cb[s] + j]
            table[s, j] = p
            t0 = cu[s] + j * B
            t1 = min(cu[s] + n, t0 + B)
            kc[p, :t1 - t0] = wl.k[t0:t1]
            vc[p, :t1 - t0] = wl.v[t0:t1]
    wl.page_table = table
    wl.k_cache = kc
    wl.v_cache = vc


# The five workloads: tiny, Qwen2.5-7B-shaped 32K GQA, Qwen3-30B-A3B-shaped 128K GQA,
# fp8 256K, and paged KV with 8 ragged sequences.
CONFIG_NAMES = {
    0: "tiny_h1_L4096_bf16",
    1: "gqa28x4_L32768_bf16",
    2: "gqa32x4_L131072_bf16",
    3: "gqa32x4_L262144_fp8",
    4: "paged8_gqa32x4_L4k-64k_bf16",
}


# An extra, sparser workload (not one of the five configurations): the 128K GQA shapes
# with the per-block means scaled down and strong vertical / slash patterns shared by the
# heads of each KV group, so that about 3.6% of causal blocks are kept at alpha = 0.1 --
# the retention the pages report for real models at 256K ([V1] Results) -- and the heads
# of a group choose largely the same blocks.
STRUCTURED_NAME = "structured_gqa32x4_L131072_bf16"
STRUCTURED_KNOBS = dict(mean_scale=0.3, vertical_gain=48.0, slash_period=64, vertical_frac=0.01)


def make_structured(threads: int = 8, L: int = 131072, hq: int = 32, hkv: int = 4, seed: int = 1102) -> Workload:
    """The structured extra workload (defaults: its 128K size); smaller L / head counts
    give the same recipe at test sizes."""
    name = STRUCTURED_NAME if (L, hq, hkv) == (131072, 32, 4) else f"structured_gqa{hq}x{hkv}_L{L}_bf16"
    return make_workload(name, hq, hkv, [L], seed=seed, alphas=(0.1,), n_sink=1, n_local=4, threads=threads,
                         **STRUCTURED_KNOBS)


def config_lengths(k: int) -> list:
    if k == 4:
        rng = np.random.default_rng(np.random.SeedSequence(1004).spawn(8)[_STREAM_LEN])
        return [int(x) for x in rng.integers(4096, 65536, size=8, endpoint=True)]
    return [{0: 4096, 1: 32768, 2: 131072, 3: 262144}[k]]


def make_config(k: int, threads: int = 8, dtype: Optional[str] = None) -> Workload:
    """Workload k of the five standard configurations (seed 1000 + k).  ``dtype="fp8"``
    with k = 2 gives the 128K workload quantised the way the 256K fp8 one is (same
    seed, so the same fp32 values before quantisation)."""
    seed = 1000 + k
    name = CONFIG_NAMES[k]
    if dtype is not None and dtype != {3: "fp8"}.get(k, "bf16"):
        if (k, dtype) != (2, "fp8"):
            raise ValueError(f"config {k} has no {dtype} variant")
        return make_workload("gqa32x4_L131072_fp8", 32, 4, [131072], seed=seed, dtype="fp8", vertical=20,
                             alphas=(0.1,), n_sink=1, n_local=4, threads=threads)
    if k == 0:
        return make_workload(name, 1, 1, [4096], seed=seed, vertical=4, slash=False,
                             alphas=(0.1,), n_sink=1, n_local=2, threads=threads)
    if k == 1:
        return make_workload(name, 28, 4, [32768], seed=seed, vertical=5,
                             alphas=(0.05, 0.1, 0.2), n_sink=1, n_local=4, threads=threads)
    if k == 2:
        return make_workload(name, 32, 4, [131072], seed=seed, vertical=20,
                             alphas=(0.1,), n_sink=1, n_local=4, threads=threads)
    if k == 3:
        return make_workload(name, 32, 4, [262144], seed=seed, dtype="fp8", vertical=41,
                             alphas=(0.1,), n_sink=1, n_local=4, threads=threads)
    if k == 4:
        return make_workload(name, 32, 4, config_lengths(4), seed=seed, paged=True,
                             alphas=(0.1,), n_sink=1, n_local=4, threads=threads)
    raise ValueError(f"unknown config {k}")


def device_tensors(wl: Workload, device="cuda"):
    """(q, k, v, q_scale, k_scale, v_scale) as torch tensors on `device`: bf16 bit
    patterns as torch.bfloat16, fp8 as uint8 e4m3fn codes plus fp32 scales."""
    import torch

    if wl.dtype == "bf16":
        def conv(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
        sc = (None, None, None)
    else:
        def conv(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(device)
        sc = tuple(torch.from_numpy(s).to(device) for s in (wl.q_scale, wl.k_scale, wl.v_scale))
    return (conv(wl.q), conv(wl.k), conv(wl.v)) + sc


def device_pages(wl: Workload, device="cuda"):
    """(k_cache, v_cache, page_table) of a paged workload as torch tensors (bf16, or
    uint8 e4m3fn codes whose scales are those of device_tensors)."""
    import torch

    assert wl.paged

    def conv(a):
        if wl.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return conv(wl.k_cache), conv(wl.v_cache), torch.from_numpy(wl.page_table).to(device)
