"""Pins of the fp64 oracle against things other than itself.

Each test names the step it pins.  Kinds: library routines (torch fp64 SDPA,
torch's bf16/float8 conversions), closed forms (bilinearity of the pooled score,
alpha = 0 and alpha > 1, single-key rows, equal keys), a hand-worked example, brute
force with pure-Python loops on tiny inputs, and invariants (forced blocks,
monotone in alpha, GQA == MHA with repeated K/V).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import synth

RNG = np.random.default_rng(7)


def rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- input decoding
def test_decode_bf16_matches_torch():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ours = O.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


def test_decode_e4m3fn_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def _torch_dequant(codes, scales):
    """Reference for code * scale[head]: torch's own e4m3fn decoder, one head at a time."""
    out = np.empty(codes.shape, dtype=np.float64)
    for h in range(codes.shape[1]):
        vals = torch.from_numpy(np.ascontiguousarray(codes[:, h])).view(torch.float8_e4m3fn).to(torch.float64)
        out[:, h] = (vals * float(np.float32(scales[h]))).numpy()
    return out


def test_dequantize_every_code_with_per_head_scales():
    """FP8 inputs (FlashPrefill V2 abstract, FP8 inference): the oracle consumes
    code * scale[head].  Every code 0..255 (zeros, subnormals, +-448, NaN) under three
    distinct fp32 scales, each head seeing the codes in its own order, against torch's
    float8_e4m3fn decoder times the head's scale.  A broadcast on the wrong axis or a
    division by the scale fails here."""
    rng = np.random.default_rng(11)
    scales = np.array([0.5, 3.25, 0.0123], dtype=np.float32)
    codes = np.empty((256, 3, 4), dtype=np.uint8)
    for h in range(3):
        for e in range(4):
            codes[:, h, e] = rng.permutation(256).astype(np.uint8)
    ours = O.dequantize(codes, scales)
    ref = _torch_dequant(codes, scales)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    one = codes == 0x38  # e4m3fn 1.0
    for h in range(3):
        assert np.all(ours[:, h][one[:, h]] == np.float64(scales[h]))
        assert np.max(np.abs(ours[:, h][fin[:, h]])) == 448.0 * np.float64(scales[h])


def test_dequantize_gqa_indexes_kv_scales_by_kv_head():
    """A GQA fp8 workload (4 query heads, 2 KV heads) with per-head scales that all
    differ: Q dequantises with its 4 scales, K and V with the 2 KV-head scales, each
    element equal to torch's decoding times the scale of its own head."""
    wl = synth.make_workload("t8", 4, 2, [300], seed=21, d=32, block=64, dtype="fp8")
    assert len(set(np.asarray(wl.q_scale).tolist())) == 4 and len(set(np.asarray(wl.k_scale).tolist())) == 2
    for codes, sc, H in ((wl.q, wl.q_scale, 4), (wl.k, wl.k_scale, 2), (wl.v, wl.v_scale, 2)):
        assert codes.shape[1] == H and np.asarray(sc).shape == (H,)
        assert np.array_equal(O.dequantize(codes, sc), _torch_dequant(codes, sc))


def test_fp8_workload_end_to_end_matches_sdpa():
    """FP8 end to end on the oracle side: selection from O.dequantize'd inputs equals the
    brute-force selection from torch-decoded values, and sparse attention over those
    lists equals fp64 SDPA (explicit block mask) on the torch-decoded values."""
    B = 64
    wl = synth.make_workload("t8e", 4, 2, [450], seed=23, d=32, block=B, dtype="fp8")
    q, k, v = (O.dequantize(wl.q, wl.q_scale), O.dequantize(wl.k, wl.k_scale),
               O.dequantize(wl.v, wl.v_scale))
    tq, tk, tv = (_torch_dequant(wl.q, wl.q_scale), _torch_dequant(wl.k, wl.k_scale),
                  _torch_dequant(wl.v, wl.v_scale))
    r = O.select_blocks(q, k, B, 0.2, 1, 2)
    bf = _brute_force_lists(tq, tk, B, 0.2, 1, 2)
    for h in range(wl.hq):
        for i, lst in enumerate(r["lists"][h]):
            assert list(lst) == bf[h][i]
    ours = O.sparse_attention(q, k, v, r["lists"], B)
    L = q.shape[0]
    g = wl.hq // wl.hkv
    for h in range(wl.hq):
        mask = np.zeros((L, L), dtype=bool)
        for t in range(L):
            allowed = set(int(x) for x in r["lists"][h][t // B])
            for c in range(t + 1):
                mask[t, c] = (c // B) in allowed
        ref = _sdpa(tq[:, h:h + 1], tk[:, h // g:h // g + 1], tv[:, h // g:h // g + 1], mask=mask[None])
        assert np.max(np.abs(ours[:, h] - ref[:, 0])) <= 1e-12
    assert r["counts"].sum() < wl.hq * (r["counts"].shape[1] * (r["counts"].shape[1] + 1)) // 2


def test_quantiser_codes_roundtrip_and_saturate():
    """Generator fp8 codes: per-head max |code| is 448 and code*scale is within half an
    e4m3 ulp of the source value (checked through torch's own decoder)."""
    x = (rand(300, 2, 16) * 3).astype(np.float32)
    for h in range(2):
        codes, s = synth.quantize_e4m3fn(x[:, h])
        vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        assert np.max(np.abs(vals)) == 448.0
        y = x[:, h].astype(np.float64) / float(s)
        # e4m3 relative spacing 2^-3 for normals, absolute 2^-9 for subnormals
        tol = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6)
        assert np.all(np.abs(vals - y) <= tol)


# ------------------------------------------------------------- pooling + scoring
def test_pooled_score_is_mean_of_token_logits():
    """P1 closed form (bilinearity): scale * mean(q_block) . mean(k_block) equals the
    mean over the B x B token pairs of scale * q_a . k_b, including a partial tail."""
    L, hq, hkv, d, B = 37, 4, 2, 16, 8
    q, k = rand(L, hq, d), rand(L, hkv, d)
    scale = 1 / math.sqrt(d)
    s = O.block_scores(O.pool(q, B), O.pool(k, B), scale)
    nb = -(-L // B)
    for h in range(hq):
        g = h // (hq // hkv)
        for i in range(nb):
            for j in range(i + 1):
                ta = range(i * B, min(L, (i + 1) * B))
                tb = range(j * B, min(L, (j + 1) * B))
                acc = 0.0
                for a in ta:
                    for b in tb:
                        acc += scale * float(np.dot(q[a, h], k[b, g]))
                acc /= len(ta) * len(tb)
                assert s[h, i, j] == pytest.approx(acc, rel=1e-12, abs=1e-13)
            assert np.all(np.isneginf(s[h, i, i + 1:]))


def test_pool_partial_block_divides_by_valid_rows():
    x = np.zeros((10, 1, 2))
    x[8:, 0, 0] = [3.0, 5.0]  # block 2 of size 4 has 2 valid rows
    p = O.pool(x, 4)
    assert p.shape == (1, 3, 2)
    assert p[0, 2, 0] == 4.0 and p[0, 0, 0] == 0.0


# ----------------------------------------------------------- hand-worked example
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    """A fixture under tests/golden/: '#' comment lines, then a JSON body."""
    with open(os.path.join(GOLDEN, name)) as f:
        return json.loads("".join(line for line in f if not line.lstrip().startswith("#")))


def test_hand_worked_selection():
    """Three 2-token blocks, d = 2, worked out by hand (tests/golden/hand_worked_selection.txt):
    the reweighted scores in closed form and the lists of five (alpha, sink, local) settings."""
    g = _golden("hand_worked_selection.txt")
    q = np.array(g["q"], float)[:, None, :]
    k = np.array(g["k"], float)[:, None, :]
    closed = {"1": 1.0, "exp(-sqrt(2))": math.exp(-math.sqrt(2)), "exp(-1/sqrt(2))": math.exp(-1 / math.sqrt(2))}
    for c in g["cases"]:
        r = O.select_blocks(q, k, g["block"], alpha=c["alpha"], n_sink=c["n_sink"], n_local=c["n_local"])
        for i, j, form in g["P"]:
            assert r["P"][0, i, j] == pytest.approx(closed[form], rel=1e-14)
        assert [list(x) for x in r["lists"][0]] == c["lists"], c


# ---------------------------------------------------------------- brute force
def _brute_force_lists(q, k, B, alpha, n_sink, n_local):
    """Independent pure-Python selection from token-level logits (tiny inputs only):
    block score = mean of scale * q_a . k_b over the token pairs of the two blocks,
    row max over causal blocks, keep = score/max-ratio test or forced block."""
    L, hq, d = q.shape
    g_size = hq // k.shape[1]
    scale = 1 / math.sqrt(d)
    nb = -(-L // B)
    out = []
    for h in range(hq):
        rows = []
        for i in range(nb):
            sc = []
            for j in range(i + 1):
                tot, n = 0.0, 0
                for a in range(i * B, min(L, (i + 1) * B)):
                    for b in range(j * B, min(L, (j + 1) * B)):
                        tot += scale * sum(q[a, h, c] * k[b, h // g_size, c] for c in range(d))
                        n += 1
                sc.append(tot / n)
            m = max(sc)
            lst = []
            for j in range(i + 1):
                ratio = math.exp(sc[j] - m)
                if ratio >= alpha or j < n_sink or j >= i - n_local + 1:
                    lst.append(j)
            rows.append(lst)
        out.append(rows)
    return out


@pytest.mark.parametrize("alpha,n_sink,n_local", [(0.0, 1, 1), (0.3, 1, 2), (0.7, 0, 1), (1.0, 2, 1), (1.5, 1, 3)])
def test_selection_matches_brute_force(alpha, n_sink, n_local):
    L, hq, hkv, d, B = 45, 4, 2, 8, 8
    rng = np.random.default_rng(11)
    q, k = rand(L, hq, d, rng=rng), rand(L, hkv, d, rng=rng)
    r = O.select_blocks(q, k, B, alpha, n_sink, n_local)
    bf = _brute_force_lists(q, k, B, alpha, n_sink, n_local)
    for h in range(hq):
        for i in range(len(bf[h])):
            assert list(r["lists"][h][i]) == bf[h][i]
            assert r["counts"][h, i] == len(bf[h][i])


# ---------------------------------------------------------------- closed forms
def _small_workload(seed=3, hq=4, hkv=2, lengths=(1000,), **kw):
    return synth.make_workload("t", hq, hkv, list(lengths), seed=seed, d=32, block=64, **kw)


def _f64(wl):
    if wl.dtype == "bf16":
        return O.decode_bf16(wl.q), O.decode_bf16(wl.k), O.decode_bf16(wl.v)
    return (O.dequantize(wl.q, wl.q_scale), O.dequantize(wl.k, wl.k_scale),
            O.dequantize(wl.v, wl.v_scale))


def test_alpha_zero_is_dense():
    """P4: alpha = 0 keeps every causal block and sparse attention equals dense."""
    wl = _small_workload()
    q, k, v = _f64(wl)
    r = O.select_blocks(q, k, 64, 0.0, 1, 1)
    nb = r["counts"].shape[1]
    assert np.array_equal(r["counts"], np.tile(np.arange(1, nb + 1), (wl.hq, 1)))
    sp = O.sparse_attention(q, k, v, r["lists"], 64)
    de = O.dense_attention(q, k, v)
    assert np.max(np.abs(sp - de)) <= 1e-12


@pytest.mark.parametrize("n_sink,n_local", [(1, 4), (2, 1), (0, 3), (5, 2)])
def test_alpha_above_one_keeps_exactly_forced_blocks(n_sink, n_local):
    """P5: for alpha > 1 the list is {0..min(n_sink, i+1)-1} U {max(0, i-n_local+1)..i}."""
    wl = _small_workload()
    q, k, _ = _f64(wl)
    r = O.select_blocks(q, k, 64, 1.0 + 1e-9, n_sink, n_local)
    for h in range(wl.hq):
        for i, lst in enumerate(r["lists"][h]):
            want = sorted(set(range(min(n_sink, i + 1))) | set(range(max(0, i - n_local + 1), i + 1)))
            assert list(lst) == want


def test_forced_blocks_argmax_and_monotone_in_alpha():
    """P3: sink/local blocks always present, the row argmax is kept for alpha <= 1, and
    kept sets nest as alpha grows; lists are strictly ascending and end at i (P6)."""
    wl = _small_workload(seed=5, lengths=(2000,))
    q, k, _ = _f64(wl)
    prev = None
    for alpha in [0.0, 0.01, 0.05, 0.1, 0.2, 0.5, 1.0]:
        r = O.select_blocks(q, k, 64, alpha, 1, 2)
        keep = r["keep"]
        nb = keep.shape[1]
        for h in range(wl.hq):
            for i in range(nb):
                lst = r["lists"][h][i]
                assert np.all(np.diff(lst) > 0) and lst[-1] == i and lst[0] >= 0
                assert 0 in lst and (i - 1 in lst or i == 0)
                assert int(np.argmax(r["s"][h, i, :i + 1])) in lst
        if prev is not None:
            assert np.all(keep <= prev)
        prev = keep


# ------------------------------------------------------------ attention pins
def _sdpa(q, k, v, mask=None, causal=False):
    """torch fp64 SDPA on CPU with [L, H, d] inputs (K/V already per query head)."""
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).permute(1, 0, 2)
    tv = torch.from_numpy(v).permute(1, 0, 2)
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, is_causal=causal)
    return o.permute(1, 0, 2).numpy()


def test_dense_matches_torch_sdpa():
    """P7: library routine, causal SDPA in fp64 on CPU; GQA via repeated K/V."""
    L, hq, hkv, d = 300, 4, 2, 32
    q, k, v = rand(L, hq, d), rand(L, hkv, d), rand(L, hkv, d)
    ours = O.dense_attention(q, k, v)
    ref = _sdpa(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), causal=True)
    assert np.max(np.abs(ours - ref)) <= 1e-12


def test_sparse_matches_sdpa_with_block_mask():
    """P8: sparse attention equals SDPA with the explicit token mask
    [block(c) in list(h, block(t))] and c <= t, built from the lists by brute force."""
    wl = _small_workload(seed=9, lengths=(700,))
    q, k, v = _f64(wl)
    B = 64
    r = O.select_blocks(q, k, B, 0.3, 1, 1)
    ours = O.sparse_attention(q, k, v, r["lists"], B)
    L = q.shape[0]
    g = wl.hq // wl.hkv
    for h in range(wl.hq):
        mask = np.zeros((L, L), dtype=bool)
        for t in range(L):
            for c in range(t + 1):
                mask[t, c] = (c // B) in set(r["lists"][h][t // B].tolist())
        ref = _sdpa(q[:, h:h + 1], k[:, h // g:h // g + 1], v[:, h // g:h // g + 1], mask=mask[None])
        assert np.max(np.abs(ours[:, h] - ref[:, 0])) <= 1e-12
    assert r["counts"].sum() < r["keep"].shape[0] * (r["keep"].shape[1] * (r["keep"].shape[1] + 1)) // 2


def test_attention_closed_forms():
    """P9: the first query sees only itself (O = V[0]); with all keys equal the softmax
    is uniform, so O[t] is the mean of V over the visible keys."""
    L, d, B = 200, 16, 64
    q, v = rand(L, 1, d), rand(L, 1, d)
    k = np.tile(rand(1, 1, d), (L, 1, 1))
    lists = [[np.array([0]), np.array([1]), np.array([0, 2]), np.array([1, 3])]]
    o = O.sparse_attention(q, k, v, lists, B)
    assert np.max(np.abs(o[0, 0] - v[0, 0])) <= 1e-15
    for t in [0, 5, 63, 64, 100, 130, 150, 199]:
        i = t // B
        vis = [c for c in range(t + 1) if c // B in lists[0][i]]
        assert np.max(np.abs(o[t, 0] - v[vis, 0].mean(axis=0))) <= 1e-12


def test_gqa_equals_mha_with_repeated_kv():
    """P10: a GQA run equals an MHA run with K/V repeated per query head."""
    wl = _small_workload(seed=13, lengths=(640,))
    q, k, v = _f64(wl)
    g = wl.hq // wl.hkv
    r1 = O.select_blocks(q, k, 64, 0.2, 1, 2)
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    r2 = O.select_blocks(q, kr, 64, 0.2, 1, 2)
    assert np.array_equal(r1["keep"], r2["keep"])
    o1 = O.sparse_attention(q, k, v, r1["lists"], 64)
    o2 = O.sparse_attention(q, kr, vr, r2["lists"], 64)
    assert np.max(np.abs(o1 - o2)) <= 1e-13


def test_varlen_dense_matches_block_diagonal_sdpa():
    """P11 (oracle side): a packed batch equals SDPA over the whole packed sequence
    with a block-diagonal causal mask (no attention across sequences)."""
    lengths = [100, 257, 64]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T, hq, d = cu[-1], 2, 16
    q, k, v = rand(T, hq, d), rand(T, hq, d), rand(T, hq, d)
    ours = O.dense_attention_varlen(q, k, v, cu)
    seg = np.repeat(np.arange(len(lengths)), lengths)
    mask = (seg[:, None] == seg[None, :]) & (np.arange(T)[None, :] <= np.arange(T)[:, None])
    ref = _sdpa(q, k, v, mask=mask[None])
    assert np.max(np.abs(ours - ref)) <= 1e-12


def test_varlen_sparse_rows_are_per_sequence():
    wl = _small_workload(seed=17, lengths=(300, 129, 64))
    q, k, v = _f64(wl)
    cu = wl.cu_seqlens
    sel = O.select_blocks_varlen(q, k, cu, 64, 0.2, 1, 1)
    o = O.sparse_attention_varlen(q, k, v, cu, [s["lists"] for s in sel], 64)
    for s in range(3):
        a, b = cu[s], cu[s + 1]
        r = O.select_blocks(q[a:b], k[a:b], 64, 0.2, 1, 1)
        assert np.array_equal(r["keep"], sel[s]["keep"])
        assert np.max(np.abs(O.sparse_attention(q[a:b], k[a:b], v[a:b], r["lists"], 64) - o[a:b])) == 0


def test_lse_matches_logsumexp():
    wl = _small_workload(seed=19, lengths=(256,))
    q, k, v = _f64(wl)
    r = O.select_blocks(q, k, 64, 0.1, 1, 1)
    _, lse = O.sparse_attention(q, k, v, r["lists"], 64, want_lse=True)
    h, t = 3, 200
    g = h // (wl.hq // wl.hkv)
    vis = [c for c in range(t + 1) if c // 64 in r["lists"][h][t // 64]]
    x = (q[t, h] @ k[vis, g].T) / math.sqrt(q.shape[-1])
    assert lse[h, t] == pytest.approx(float(torch.logsumexp(torch.from_numpy(x), 0)), rel=1e-13)


# ------------------------------------------------------------ chunked prefill
def test_chunk_blocks_closed_form():
    """Absolute query blocks a chunk touches, by hand: positions 172..299 lie in
    blocks 1 and 2; a whole sequence is blocks 0..2; positions 256..299 are block 2
    alone; an aligned chunk (128..299) starts at its own block; an empty chunk
    touches none."""
    assert O.chunk_blocks(128, 300, 128) == (1, 2)
    assert O.chunk_blocks(300, 300, 128) == (0, 3)
    assert O.chunk_blocks(44, 300, 128) == (2, 1)
    assert O.chunk_blocks(172, 300, 128) == (1, 2)
    assert O.chunk_blocks(0, 300, 128) == (2, 0)


def test_pool_chunk_partial_first_block_by_hand():
    """A chunk entering block 1 at position 150 (len_k 300, len_q 150): block 1
    averages positions 150..255 only, block 2 positions 256..299 (pure Python)."""
    qc = rand(150, 2, 3)
    got = O.pool_chunk(qc, 300, 128)
    assert got.shape == (2, 2, 3)
    for h in range(2):
        for e in range(3):
            b1 = [qc[t, h, e] for t in range(150) if (150 + t) // 128 == 1]
            b2 = [qc[t, h, e] for t in range(150) if (150 + t) // 128 == 2]
            assert len(b1) == 106 and len(b2) == 44
            assert got[h, 0, e] == pytest.approx(sum(b1) / 106, rel=1e-14, abs=1e-15)
            assert got[h, 1, e] == pytest.approx(sum(b2) / 44, rel=1e-14, abs=1e-15)


def test_chunked_with_whole_sequence_is_prefill():
    """len_q = len_k: pooled means, lists and outputs equal the prefill functions."""
    L, block = 5 * 16 + 7, 16
    q, k, v = rand(L, 4, 8), rand(L, 2, 8), rand(L, 2, 8)
    a = O.select_blocks_chunked(q, k, block, 0.2, 1, 2)
    b = O.select_blocks(q, k, block, 0.2, 1, 2)
    assert np.array_equal(a["pq"], b["pq"])
    assert np.array_equal(a["counts"], b["counts"])
    for h in range(4):
        for i in range(len(b["lists"][h])):
            assert np.array_equal(a["lists"][h][i], b["lists"][h][i])
    oa = O.sparse_attention_chunked(q, k, v, a["lists"], block)
    ob = O.sparse_attention(q, k, v, b["lists"], block)
    assert np.allclose(oa, ob, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("len_q", [1, 23, 48, 61])
def test_chunked_dense_equals_tail_of_full_attention(len_q):
    """All blocks kept: the chunk's outputs and LSE equal the last len_q rows of plain
    causal attention over the whole sequence (torch fp64 SDPA, bottom-right causal)."""
    L, block = 3 * 16 + 13, 16
    q, k, v = rand(L, 4, 8), rand(L, 2, 8), rand(L, 2, 8)
    sel = O.select_blocks_chunked(q[L - len_q:], k, block, 0.0, 1, 1)
    assert all(len(lst) == sel["I0"] + r + 1 for h in range(4) for r, lst in enumerate(sel["lists"][h]))
    out, lse = O.sparse_attention_chunked(q[L - len_q:], k, v, sel["lists"], block, want_lse=True)
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(np.repeat(k, 2, axis=1)).permute(1, 0, 2)
    vt = torch.from_numpy(np.repeat(v, 2, axis=1)).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True).permute(1, 0, 2).numpy()
    assert np.allclose(out, ref[L - len_q:], rtol=1e-10, atol=1e-12)
    x = (qt @ kt.transpose(1, 2)) / math.sqrt(8)
    x = x.masked_fill(~torch.ones(L, L, dtype=torch.bool).tril(), float("-inf"))
    assert np.allclose(lse, torch.logsumexp(x, dim=-1).numpy()[:, L - len_q:], rtol=1e-12, atol=1e-12)


def test_block_aligned_chunk_reuses_prefill_rows():
    """A chunk that starts on a block boundary has the prefill's pooled queries for its
    blocks, so its lists are the prefill lists of the same rows."""
    L, block = 6 * 16 + 5, 16
    q, k = rand(L, 4, 8), rand(L, 2, 8)
    full = O.select_blocks(q, k, block, 0.15, 1, 2)
    for start_block in (1, 3, 6):
        c = O.select_blocks_chunked(q[start_block * block:], k, block, 0.15, 1, 2)
        assert c["I0"] == start_block
        for h in range(4):
            for r in range(c["nq"]):
                assert np.array_equal(c["lists"][h][r], full["lists"][h][start_block + r])


def test_chunked_selection_brute_force():
    """Tiny chunk starting mid-block: pooled scores, threshold and forced blocks by
    pure-Python loops."""
    L, block, d = 5 * 4 + 2, 4, 3
    len_q = 9
    q, k = rand(len_q, 2, d), rand(L, 1, d)
    alpha, n_sink, n_local = 0.3, 1, 2
    sel = O.select_blocks_chunked(q, k, block, alpha, n_sink, n_local)
    off = L - len_q
    nk = -(-L // block)
    for h in range(2):
        for r in range(sel["nq"]):
            I = off // block + r
            qs = [t for t in range(len_q) if (off + t) // block == I]
            qbar = [sum(q[t, h, e] for t in qs) / len(qs) for e in range(d)]
            scores = []
            for j in range(I + 1):
                ks = [c for c in range(L) if c // block == j]
                kbar = [sum(k[c, 0, e] for c in ks) / len(ks) for e in range(d)]
                scores.append(sum(a * b for a, b in zip(qbar, kbar)) / math.sqrt(d))
            m = max(scores)
            want = [j for j in range(I + 1)
                    if math.exp(scores[j] - m) >= alpha or j < n_sink or j > I - n_local]
            assert list(sel["lists"][h][r]) == want
            assert I < nk



# ------------------------------------------------------- group-shared lists
def test_grouped_lists_are_unions_brute_force():
    """Group list = set union of the group's per-head lists (pure Python), ascending,
    a superset of each head's list, ending with the diagonal."""
    L, block = 6 * 16 + 3, 16
    q, k = rand(L, 6, 8), rand(L, 2, 8)
    sel = O.select_blocks_grouped(q, k, block, 0.2, 1, 2)
    heads = sel["heads"]["lists"]
    for g in range(2):
        for i in range(len(sel["lists"][g])):
            want = sorted(set().union(*[set(int(x) for x in heads[h][i]) for h in range(3 * g, 3 * g + 3)]))
            assert [int(x) for x in sel["lists"][g][i]] == want
            assert want[-1] == i


def test_grouped_with_one_head_per_group_is_per_head():
    L, block = 5 * 16, 16
    q, k = rand(L, 3, 8), rand(L, 3, 8)
    a = O.select_blocks_grouped(q, k, block, 0.1, 1, 1)
    b = O.select_blocks(q, k, block, 0.1, 1, 1)
    assert np.array_equal(a["keep"], b["keep"])


def test_grouped_alpha_zero_and_above_one():
    """alpha = 0 keeps every causal block for the group; alpha > 1 keeps exactly the
    forced blocks (closed forms, as for per-head lists)."""
    L, block = 5 * 16 + 9, 16
    q, k = rand(L, 4, 8), rand(L, 2, 8)
    nb = -(-L // block)
    full = O.select_blocks_grouped(q, k, block, 0.0, 1, 1)
    assert np.array_equal(full["keep"], np.broadcast_to(np.tril(np.ones((nb, nb), dtype=bool)), (2, nb, nb)))
    forced = O.select_blocks_grouped(q, k, block, 1.5, 2, 2)
    i = np.arange(nb)[:, None]
    j = np.arange(nb)[None, :]
    want = (j <= i) & ((j < 2) | (j > i - 2))
    assert np.array_equal(forced["keep"], np.broadcast_to(want, (2, nb, nb)))



# --------------------------------------- V2 mean correction (an assumption)
def test_mean_correction_is_noop_without_pruning():
    """Full lists: nothing is pruned, so the corrected output is plain attention
    (torch fp64 SDPA)."""
    L, block = 4 * 16 + 5, 16
    q, k, v = rand(L, 4, 8), rand(L, 2, 8), rand(L, 2, 8)
    nb = -(-L // block)
    full = [[np.arange(i + 1) for i in range(nb)] for _ in range(4)]
    out = O.mean_correction(q, k, v, full, block)
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(np.repeat(k, 2, axis=1)).permute(1, 0, 2)
    vt = torch.from_numpy(np.repeat(v, 2, axis=1)).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True).permute(1, 0, 2).numpy()
    assert np.allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_mean_correction_exact_for_constant_blocks():
    """Closed form: if every block's keys and values are constant inside the block, n_j
    copies of (kbar_j, vbar_j) are exactly the block, so the corrected sparse output
    equals dense attention whatever the lists prune (diagonal kept)."""
    L, block = 5 * 8, 8
    nb = L // block
    kb, vb = rand(nb, 2, 6), rand(nb, 2, 6)
    k = np.repeat(kb, block, axis=0)
    v = np.repeat(vb, block, axis=0)
    q = rand(L, 4, 6)
    rng = np.random.default_rng(5)
    lists = [[np.array(sorted(set(rng.choice(i + 1, size=rng.integers(1, i + 2), replace=False)) | {i}))
              for i in range(nb)] for _ in range(4)]
    out, lse = O.mean_correction(q, k, v, lists, block, want_lse=True)
    dense, dlse = O.dense_attention(q, k, v, want_lse=True)
    # pruned blocks lie below the diagonal, so all their keys are visible; the
    # diagonal block is listed and stays causal on both sides
    assert np.allclose(out, dense, rtol=1e-10, atol=1e-12)
    assert np.allclose(lse, dlse, rtol=1e-12, atol=1e-12)


def test_mean_correction_brute_force():
    """Tiny case by pure-Python loops over tokens and pruned blocks."""
    L, block, d = 3 * 4 + 1, 4, 3
    q, k, v = rand(L, 1, d), rand(L, 1, d), rand(L, 1, d)
    lists = [[np.array([0]), np.array([1]), np.array([0, 2]), np.array([3])]]
    out = O.mean_correction(q, k, v, lists, block)
    sc = 1 / math.sqrt(d)
    for t in range(L):
        i = t // block
        num = [0.0] * d
        den = 0.0
        for j in range(i + 1):
            toks = [c for c in range(j * block, min((j + 1) * block, L))]
            if j in lists[0][i]:
                for c in toks:
                    if c <= t:
                        w = math.exp(sc * sum(q[t, 0, e] * k[c, 0, e] for e in range(d)))
                        den += w
                        num = [num[e] + w * v[c, 0, e] for e in range(d)]
            else:
                kbar = [sum(k[c, 0, e] for c in toks) / len(toks) for e in range(d)]
                vbar = [sum(v[c, 0, e] for c in toks) / len(toks) for e in range(d)]
                w = len(toks) * math.exp(sc * sum(q[t, 0, e] * kbar[e] for e in range(d)))
                den += w
                num = [num[e] + w * vbar[e] for e in range(d)]
        assert np.allclose(out[t, 0], [x / den for x in num], rtol=1e-12, atol=1e-13)
