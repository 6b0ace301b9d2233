"""Plain fp64 CPU oracle for FlashPrefill block-sparse prefill attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call anything here.
It shares no code with the HIP path (no kernels, headers, helpers, tables or
pre/post-processing); the only thing both sides consume is the seeded input
generator in ``synth``.

Every function follows one step of the method as the pages describe it:

* [V1] "FlashPrefill: Near-Zero-Cost Sparsity Discovery for Ultra-Fast
  Long-Context Prefilling" (zhichai.net topic page), sections "Method 1.
  Instantaneous Pattern Discovery", "2. Dynamic Threshold Pruning" and
  "3. Index Compaction -> Physical Jumps";
* [V1-abs] the FlashPrefill abstract (insight.artgrammer.co.kr): one fast
  block search finds vertical, slash and block-sparse patterns together,
  and the threshold avoids sorting or accumulating scores;
* [V2] "FlashPrefill V2: Block-Sparse Prefill Attention for Long-Context LLM
  Serving" (shd-paper.top summary, English abstract): causal block-sparse
  prefill attention over paged KV with continuous batching, bf16 and FP8.

Readings taken where the pages are silent or garbled (each is repeated where
it is used):

* pooling is the arithmetic mean over a block's valid tokens;
* block score = (1/sqrt(d)) * qbar_i . kbar_j, so it equals the mean of the
  block's true attention logits;
* the undefined "global reweighting" is a row softmax over the causal blocks
  j <= i; any positive per-row factor cancels under the alpha * max rule, so
  the thresholded sets do not depend on this reading;
* the threshold compares P = exp(s - rowmax) >= alpha per (query head, query
  block) row, ties kept; alpha = 0 keeps everything;
* safety net: the first ``n_sink`` blocks and the ``n_local`` blocks ending at
  the diagonal are always kept (the page's sizes are garbled);
* lists are ascending, per query head, and always end with the diagonal;
* attention is causal inside the diagonal block, softmax scale 1/sqrt(d);
* varlen/paged: every sequence is processed on its own with queries and keys
  starting at token 0; the page table is addressing only, so it never appears
  here;
* the V2 "mean correction term" is named but not defined on the pages.  Kept
  outside the core above as a switchable assumption (``mean_correction``): every
  causal key block a list leaves out still enters the softmax, as n_j copies of
  its mean key with its mean value, so the pruned probability mass is restored
  approximately;
* group-shared lists (a PackGQA-style mode, beyond what the pages define): the
  list of a KV-head group is the union of its query heads' lists, and every
  query head of the group attends over that union (a superset of its own list);
* chunked / prefix-cached prefill (beyond the pages, which only name paged KV
  and continuous batching for serving): a chunk of len_q queries is the last
  len_q positions of a sequence whose K/V cache holds len_k tokens; query t sits
  at position len_k - len_q + t and sees keys up to that position; query blocks
  follow absolute positions (block I = positions 128I .. 128I+127) and a block's
  pooled query is the mean of the chunk's tokens in it; the selection of row I
  is the prefill rule over key blocks 0..I.

Precision: every floating-point step is fp64.  Inputs are the exact values of
the bf16 bit patterns or of ``e4m3fn_code * scale`` widened to fp64.

Pins (tests/test_oracle_pins.py) tie each function to something other than
itself: the bilinearity closed form of the block score, brute force on tiny
inputs with pure-Python loops, torch's fp64 scaled_dot_product_attention with
and without an explicit block mask, closed forms for alpha = 0 and alpha > 1,
monotonicity in alpha, GQA == MHA with repeated K/V, and the e4m3fn decoder
against torch.float8_e4m3fn.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

__all__ = [
    "decode_bf16", "decode_e4m3fn", "dequantize", "pool", "block_scores", "reweight",
    "keep_mask", "compact", "select_blocks", "attend_block", "sparse_attention",
    "dense_attention", "select_blocks_varlen", "sparse_attention_varlen", "dense_attention_varlen",
    "chunk_blocks", "pool_chunk", "select_blocks_chunked", "sparse_attention_chunked",
    "select_blocks_grouped", "mean_correction",
]


# --------------------------------------------------------------------------- inputs
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _e4m3fn_table() -> np.ndarray:
    """Value of every OCP FP8 E4M3FN byte from the format definition:
    1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, subnormals at
    exponent field 0, no infinities, and S.1111.111 the only NaN pattern."""
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            t[c] = np.nan
        elif e == 0:
            t[c] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            t[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


_E4M3FN = _e4m3fn_table()


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """e4m3fn codes (uint8) -> exact fp64 values."""
    return _E4M3FN[np.asarray(codes, dtype=np.uint8)]


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[T, H, d] e4m3fn codes with one fp32 scale per head -> fp64 code * scale.
    Each product is exact in fp64 (4-bit by 24-bit significands)."""
    return decode_e4m3fn(codes) * np.asarray(scales, dtype=np.float64)[None, :, None]


# ------------------------------------------------------------------ block discovery
def pool(x: np.ndarray, block: int) -> np.ndarray:
    """Mean-pool every ``block``-token block of x [L, H, d] -> [H, nb, d].

    [V1] Method 1: each block is represented by its mean vector (the
    "mean-proxy", valid under the within-block low-variance assumption).
    A partial last block is averaged over its valid tokens only."""
    L, H, d = x.shape
    nb = -(-L // block)
    out = np.empty((H, nb, d), dtype=np.float64)
    for b in range(nb):
        rows = x[b * block:min((b + 1) * block, L)]
        out[:, b, :] = rows.sum(axis=0) / rows.shape[0]
    return out


def block_scores(pq: np.ndarray, pk: np.ndarray, scale: float) -> np.ndarray:
    """Pooled block-score map s[h, i, j] = scale * pq[h, i] . pk[g(h), j] for j <= i,
    -inf above the diagonal.  [V1] Method 1: pooled queries against pooled keys give
    the (L/B)^2 map.  GQA: query head h reads KV head h // (Hq / Hkv)."""
    hq, nb, _ = pq.shape
    hkv = pk.shape[0]
    group = hq // hkv
    s = np.empty((hq, nb, nb), dtype=np.float64)
    upper = np.triu(np.ones((nb, nb), dtype=bool), k=1)
    for h in range(hq):
        s[h] = scale * (pq[h] @ pk[h // group].T)
        s[h][upper] = -np.inf
    return s


def reweight(s: np.ndarray) -> np.ndarray:
    """Row softmax numerators P = exp(s - max_{j<=i} s): the reading of [V1] Method 1's
    "global reweighting".  P lies in [0, 1] with the row maximum at 1; positions above
    the diagonal get 0."""
    m = np.max(s, axis=-1, keepdims=True)
    return np.exp(s - m)


def keep_mask(P: np.ndarray, alpha: float, n_sink: int, n_local: int) -> np.ndarray:
    """[V1] Method 2: keep block j of row i when its score reaches alpha times the row
    maximum (P >= alpha, since P is the score over its row max), and always keep the
    attention-sink blocks (j < n_sink) and the local window ending at the diagonal
    (i - n_local < j <= i).  Only causal blocks j <= i can be kept."""
    nb = P.shape[-1]
    i = np.arange(nb)[:, None]
    j = np.arange(nb)[None, :]
    causal = j <= i
    forced = (j < n_sink) | (j > i - n_local)
    return causal & ((P >= alpha) | forced)


def compact(keep: np.ndarray):
    """[V1] Method 3: turn each row of the block mask into a contiguous list of the kept
    block ids (ascending).  Returns (lists[h][i] -> int64 array, counts[h, i])."""
    hq, nb, _ = keep.shape
    lists = [[np.nonzero(keep[h, i])[0] for i in range(nb)] for h in range(hq)]
    counts = keep.sum(axis=-1).astype(np.int64)
    return lists, counts


def select_blocks(q: np.ndarray, k: np.ndarray, block: int, alpha: float, n_sink: int,
                  n_local: int, scale: Optional[float] = None) -> Dict[str, object]:
    """Discovery -> threshold -> compaction for one sequence.
    q [L, Hq, d] and k [L, Hkv, d] are fp64.  Returns pooled means, scores, P, the keep
    mask, lists and counts."""
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    pq = pool(q, block)
    pk = pool(k, block)
    s = block_scores(pq, pk, scale)
    P = reweight(s)
    keep = keep_mask(P, alpha, n_sink, n_local)
    lists, counts = compact(keep)
    return dict(pq=pq, pk=pk, s=s, P=P, keep=keep, lists=lists, counts=counts)


# ----------------------------------------------------------------------- attention
def attend_block(q: np.ndarray, k: np.ndarray, v: np.ndarray, blocks: Sequence[int], h: int,
                 i: int, block: int, scale: Optional[float] = None, want_lse: bool = False):
    """Output rows of query block i, head h, attending to the key blocks in ``blocks``.

    [V1] Method 3 / [V2]: the attention loop visits only the listed key blocks; inside
    them attention is causal (key c <= query t), softmax over the visited keys.  The
    query itself is always visible, so no row is empty when the diagonal is listed."""
    L, hq, d = q.shape
    group = hq // k.shape[1]
    g = h // group
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    t = np.arange(i * block, min((i + 1) * block, L))
    c = np.concatenate([np.arange(j * block, min((j + 1) * block, L)) for j in blocks])
    x = scale * (q[t, h, :] @ k[c, g, :].T)
    x = np.where(c[None, :] <= t[:, None], x, -np.inf)
    M = np.max(x, axis=1, keepdims=True)
    e = np.exp(x - M)
    den = e.sum(axis=1, keepdims=True)
    out = (e @ v[c, g, :]) / den
    if want_lse:
        return out, (M + np.log(den))[:, 0]
    return out


def sparse_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, lists, block: int,
                     scale: Optional[float] = None, want_lse: bool = False):
    """Causal GQA block-sparse attention for one sequence over the given lists
    (lists[h][i] = key block ids for query block i of head h).  -> O [L, Hq, d]
    (and LSE [Hq, L] in natural-log units of the scaled logits)."""
    L, hq, d = q.shape
    nb = -(-L // block)
    out = np.empty((L, hq, d), dtype=np.float64)
    lse = np.empty((hq, L), dtype=np.float64)
    for h in range(hq):
        for i in range(nb):
            r = attend_block(q, k, v, lists[h][i], h, i, block, scale, want_lse=True)
            out[i * block:(i + 1) * block, h, :] = r[0]
            lse[h, i * block:(i + 1) * block] = r[1]
    return (out, lse) if want_lse else out


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: Optional[float] = None,
                    want_lse: bool = False):
    """Plain causal GQA softmax attention, fp64: softmax(scale * q k^T, causal) v."""
    L, hq, d = q.shape
    group = hq // k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out = np.empty((L, hq, d), dtype=np.float64)
    lse = np.empty((hq, L), dtype=np.float64)
    causal = np.tril(np.ones((L, L), dtype=bool))
    for h in range(hq):
        g = h // group
        x = scale * (q[:, h, :] @ k[:, g, :].T)
        x = np.where(causal, x, -np.inf)
        M = np.max(x, axis=1, keepdims=True)
        e = np.exp(x - M)
        den = e.sum(axis=1, keepdims=True)
        out[:, h, :] = (e @ v[:, g, :]) / den
        lse[h] = (M + np.log(den))[:, 0]
    return (out, lse) if want_lse else out


# -------------------------------------------------------------------------- varlen
def _segments(cu_seqlens: Sequence[int]):
    cu = [int(x) for x in cu_seqlens]
    return [(cu[s], cu[s + 1]) for s in range(len(cu) - 1)]


def select_blocks_varlen(q, k, cu_seqlens, block, alpha, n_sink, n_local, scale=None) -> List[dict]:
    """[V2] continuous batching: discovery, threshold and compaction per sequence of a
    packed batch; the result for sequence s is exactly ``select_blocks`` on its slice."""
    return [select_blocks(q[a:b], k[a:b], block, alpha, n_sink, n_local, scale)
            for a, b in _segments(cu_seqlens)]


def sparse_attention_varlen(q, k, v, cu_seqlens, lists_per_seq, block, scale=None, want_lse=False):
    """Per-sequence sparse attention over a packed batch -> packed O [T, Hq, d]."""
    outs, lses = [], []
    for (a, b), lists in zip(_segments(cu_seqlens), lists_per_seq):
        o, l = sparse_attention(q[a:b], k[a:b], v[a:b], lists, block, scale, want_lse=True)
        outs.append(o)
        lses.append(l)
    out = np.concatenate(outs, axis=0)
    return (out, np.concatenate(lses, axis=1)) if want_lse else out


def dense_attention_varlen(q, k, v, cu_seqlens, scale=None):
    return np.concatenate([dense_attention(q[a:b], k[a:b], v[a:b], scale)
                           for a, b in _segments(cu_seqlens)], axis=0)


# ------------------------------------------------------------ chunked prefill
def chunk_blocks(len_q: int, len_k: int, block: int):
    """Absolute query blocks of a chunk of len_q queries ending at position len_k - 1:
    -> (I0, nq), the first block and the number of blocks the chunk touches."""
    off = len_k - len_q
    if len_q == 0:
        return off // block, 0
    return off // block, (len_k - 1) // block - off // block + 1


def pool_chunk(qc: np.ndarray, len_k: int, block: int) -> np.ndarray:
    """Pooled query means of a chunk qc [len_q, H, d] whose first query sits at
    position len_k - len_q: block I averages the chunk's queries at positions
    128I .. 128I+127 (a block the chunk enters mid-way is averaged over its part).
    -> [H, nq, d]."""
    len_q, H, d = qc.shape
    off = len_k - len_q
    I0, nq = chunk_blocks(len_q, len_k, block)
    out = np.empty((H, nq, d), dtype=np.float64)
    pos = off + np.arange(len_q)
    for r in range(nq):
        rows = qc[(pos // block) == I0 + r]
        out[:, r, :] = rows.sum(axis=0) / rows.shape[0]
    return out


def select_blocks_chunked(qc: np.ndarray, k: np.ndarray, block: int, alpha: float, n_sink: int,
                          n_local: int, scale: Optional[float] = None) -> Dict[str, object]:
    """Discovery -> threshold -> compaction for one chunk: row I (absolute query block,
    I0 <= I < I0 + nq) scores its pooled query against the pooled keys j <= I of the
    whole cache k [len_k, Hkv, d] and keeps blocks by the prefill rule.  Returns the
    pooled means, P, keep [hq, nq, nk] (row r = block I0 + r), lists[h][r], counts."""
    d = qc.shape[-1]
    len_k = k.shape[0]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    I0, nq = chunk_blocks(qc.shape[0], len_k, block)
    pq = pool_chunk(qc, len_k, block)
    pk = pool(k, block)
    hq, hkv, nk = pq.shape[0], pk.shape[0], pk.shape[1]
    group = hq // hkv
    P = np.zeros((hq, nq, nk), dtype=np.float64)
    keep = np.zeros((hq, nq, nk), dtype=bool)
    for h in range(hq):
        for r in range(nq):
            I = I0 + r
            s = scale * (pk[h // group, :I + 1] @ pq[h, r])
            p = np.exp(s - np.max(s))
            j = np.arange(I + 1)
            P[h, r, :I + 1] = p
            keep[h, r, :I + 1] = (p >= alpha) | (j < n_sink) | (j > I - n_local)
    lists = [[np.nonzero(keep[h, r])[0] for r in range(nq)] for h in range(hq)]
    counts = keep.sum(axis=-1).astype(np.int64)
    return dict(pq=pq, pk=pk, P=P, keep=keep, lists=lists, counts=counts, I0=I0, nq=nq)


def sparse_attention_chunked(qc: np.ndarray, k: np.ndarray, v: np.ndarray, lists, block: int,
                             scale: Optional[float] = None, want_lse: bool = False):
    """Chunk queries qc [len_q, Hq, d] (positions len_k - len_q ..) attend to the cache
    k, v [len_k, Hkv, d]: query at position p sees keys c <= p whose block is in
    lists[h][I - I0] for its block I = p // block.  -> O [len_q, Hq, d] (and LSE)."""
    len_q, hq, d = qc.shape
    len_k = k.shape[0]
    group = hq // k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    off = len_k - len_q
    I0, _ = chunk_blocks(len_q, len_k, block)
    out = np.empty((len_q, hq, d), dtype=np.float64)
    lse = np.empty((hq, len_q), dtype=np.float64)
    for t in range(len_q):
        p = off + t
        I = p // block
        for h in range(hq):
            g = h // group
            c = np.concatenate([np.arange(j * block, min((j + 1) * block, len_k)) for j in lists[h][I - I0]])
            c = c[c <= p]
            x = scale * (k[c, g, :] @ qc[t, h, :])
            M = np.max(x)
            e = np.exp(x - M)
            out[t, h, :] = (e @ v[c, g, :]) / e.sum()
            lse[h, t] = M + np.log(e.sum())
    return (out, lse) if want_lse else out


# ------------------------------------------------------- group-shared lists
def select_blocks_grouped(q: np.ndarray, k: np.ndarray, block: int, alpha: float, n_sink: int,
                          n_local: int, scale: Optional[float] = None) -> Dict[str, object]:
    """Per-head selection as in ``select_blocks``, then one list per KV-head group:
    the union of the keep masks of the group's query heads.  Returns the per-head
    result under ``heads`` plus the group keep mask, lists and counts."""
    per_head = select_blocks(q, k, block, alpha, n_sink, n_local, scale)
    keep = per_head["keep"]
    hq = keep.shape[0]
    hkv = k.shape[1]
    group = hq // hkv
    gkeep = np.zeros((hkv,) + keep.shape[1:], dtype=bool)
    for h in range(hq):
        gkeep[h // group] |= keep[h]
    lists, counts = compact(gkeep)
    return dict(heads=per_head, keep=gkeep, lists=lists, counts=counts)



# --------------------------------------- V2 mean correction (an assumption)
def mean_correction(q: np.ndarray, k: np.ndarray, v: np.ndarray, lists, block: int,
                    scale: Optional[float] = None, want_lse: bool = False):
    """ASSUMPTION, not defined on the pages (the [V2] abstract mentions a mean-based
    correction meant to reduce the sparse approximation's error, with no formula).
    Reading: sparse attention over the
    lists, plus every causal block j missing from the list of (h, i) entering the
    softmax as n_j copies of its mean key kbar_j with its mean value vbar_j:

        O_t = (sum_{c in C(t)} e^{s_tc} v_c + sum_{j pruned} n_j e^{scale q_t.kbar_j} vbar_j)
              / (sum_{c in C(t)} e^{s_tc} + sum_{j pruned} n_j e^{scale q_t.kbar_j}).

    Pruned blocks lie strictly below the diagonal (the diagonal is always listed), so
    all their keys are visible to every query of block i."""
    L, hq, d = q.shape
    group = hq // k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    nb = -(-L // block)
    kbar, vbar = pool(k, block), pool(v, block)
    n = np.array([min(block, L - j * block) for j in range(nb)], dtype=np.float64)
    out = np.empty((L, hq, d), dtype=np.float64)
    lse = np.empty((hq, L), dtype=np.float64)
    for h in range(hq):
        g = h // group
        for i in range(nb):
            t = np.arange(i * block, min((i + 1) * block, L))
            kept = np.asarray(lists[h][i], dtype=np.int64)
            c = np.concatenate([np.arange(j * block, min((j + 1) * block, L)) for j in kept])
            x = scale * (q[t, h, :] @ k[c, g, :].T)
            x = np.where(c[None, :] <= t[:, None], x, -np.inf)
            pruned = np.setdiff1d(np.arange(i + 1), kept)
            y = scale * (q[t, h, :] @ kbar[g, pruned, :].T) + np.log(n[pruned])[None, :]
            M = np.maximum(np.max(x, axis=1), np.max(y, axis=1) if pruned.size else -np.inf)[:, None]
            ex, ey = np.exp(x - M), np.exp(y - M)
            den = ex.sum(axis=1, keepdims=True) + ey.sum(axis=1, keepdims=True)
            out[t, h, :] = (ex @ v[c, g, :] + ey @ vbar[g, pruned, :]) / den
            lse[h, t] = (M + np.log(den))[:, 0]
    return (out, lse) if want_lse else out
