"""The seeded generator: determinism, structure of the patterns, fp8 codes, paging."""
import numpy as np

import oracle as O
import synth


def test_same_seed_same_bytes_and_thread_independent():
    a = synth.make_workload("a", 4, 2, [700, 300], seed=5, d=32, block=64, threads=1)
    b = synth.make_workload("a", 4, 2, [700, 300], seed=5, d=32, block=64, threads=4)
    c = synth.make_workload("a", 4, 2, [700, 300], seed=6, d=32, block=64)
    assert a.digests() == b.digests()
    assert a.digests()["q"] != c.digests()["q"]


def test_block_means_and_vertical_boost_present():
    wl = synth.make_workload("s", 2, 1, [128 * 40], seed=3, slash=False, vertical=4)
    k = O.decode_bf16(wl.k)[:, 0, :]
    q = O.decode_bf16(wl.q)
    # within-block noise sd ~0.3 around a per-block mean with sd ~1
    resid = k.reshape(40, 128, -1) - k.reshape(40, 128, -1).mean(axis=1, keepdims=True)
    assert 0.25 < resid.std() < 0.35
    # boosted key blocks align with the shared query direction
    u = (q.mean(axis=(0, 1)))
    proj = (k.reshape(40, 128, -1).mean(axis=1) @ u)
    top = set(np.argsort(proj)[-4:].tolist())
    assert top == set(wl.vertical_blocks[(0, 0)])


def test_fp8_workload_codes_and_scales():
    wl = synth.make_workload("f", 4, 2, [512], seed=4, dtype="fp8", d=32, block=64)
    assert wl.q.dtype == np.uint8 and wl.q_scale.shape == (4,)
    for arr in (wl.q, wl.k, wl.v):
        vals = O.decode_e4m3fn(arr)
        assert not np.isnan(vals).any()
        for h in range(arr.shape[1]):
            assert np.max(np.abs(vals[:, h])) == 448.0


def test_page_table_is_permutation_and_caches_hold_the_tokens():
    wl = synth.make_workload("p", 2, 2, [300, 64, 129], seed=8, d=16, block=64, paged=True)
    nbs = wl.seq_blocks
    assert nbs == [5, 1, 3]
    used = np.concatenate([wl.page_table[s, :nbs[s]] for s in range(3)])
    assert sorted(used.tolist()) == list(range(sum(nbs)))
    assert np.all(wl.page_table[1, 1:] == -1)
    cu = wl.cu_seqlens
    for s, n in enumerate(wl.lengths):
        for t in range(n):
            p = wl.page_table[s, t // 64]
            assert np.array_equal(wl.k_cache[p, t % 64], wl.k[cu[s] + t])
            assert np.array_equal(wl.v_cache[p, t % 64], wl.v[cu[s] + t])
        tail = n % 64
        if tail:
            p = wl.page_table[s, n // 64]
            assert not wl.k_cache[p, tail:].any()


def test_config_shapes():
    lens = synth.config_lengths(4)
    assert len(lens) == 8 and all(4096 <= n <= 65536 for n in lens)
    assert synth.config_lengths(2) == [131072]
    wl = synth.make_config(0)
    assert wl.q.shape == (4096, 1, 128) and wl.n_local == 2 and wl.alphas == (0.1,)


def test_structured_recipe_is_sparser_and_shared_within_groups():
    # same size and heads, standard recipe vs the structured one: far fewer kept blocks,
    # and the heads of a KV group keep largely the same blocks
    L, hq, hkv = 128 * 128, 8, 1
    std = synth.make_workload("std", hq, hkv, [L], seed=9)
    st = synth.make_structured(L=L, hq=hq, hkv=hkv, seed=9)
    dens, lift = {}, {}
    for tag, wl in (("std", std), ("structured", st)):
        q = O.decode_bf16(wl.q).astype(np.float64)
        k = O.decode_bf16(wl.k).astype(np.float64)
        keep = O.select_blocks(q, k, 128, 0.1, 1, 4)["keep"].reshape(hq, -1)
        nb = int(round(np.sqrt(keep.shape[1])))
        dens[tag] = keep.sum() / (hq * nb * (nb + 1) / 2)
        # chance that a block one head keeps is kept by another head of the group, over the
        # density (1 for independent heads)
        both = sum((keep[a] & keep[b]).sum() for a in range(hq) for b in range(hq) if a != b)
        lift[tag] = both / ((hq - 1) * keep.sum()) / dens[tag]
    assert dens["structured"] < 0.5 * dens["std"]
    assert lift["structured"] > 2.0 * lift["std"]


def test_default_knobs_leave_the_standard_recipe_unchanged():
    a = synth.make_workload("a", 2, 1, [900], seed=11, d=32, block=64)
    b = synth.make_workload("a", 2, 1, [900], seed=11, d=32, block=64, mean_scale=1.0,
                            vertical_gain=synth.VERTICAL_GAIN, slash_period=synth.SLASH_PERIOD_BLOCKS)
    assert a.digests() == b.digests()
    c = synth.make_workload("a", 2, 1, [900], seed=11, d=32, block=64, mean_scale=0.5)
    assert c.digests()["q"] != a.digests()["q"]
