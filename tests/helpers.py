"""Test utilities: moving synthetic workloads to the GPU, unpacking the library's
triangular-packed lists, and comparing them with the oracle under the stated rule
(exact, except non-forced blocks whose P lies within 1e-6 relative of alpha)."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
import synth

BAND_REL = 1e-6
TOL_BF16 = 2e-2
TOL_FP8 = 6e-2

# worst errors measured by the full-size tests; conftest prints them in the terminal
# summary, so they reach the log even when pytest runs quietly
MARGINS = []


def record_margin(line: str) -> None:
    MARGINS.append(line)


def have_gpu() -> bool:
    return torch.cuda.is_available()


def to_device(wl, device="cuda"):
    return synth.device_tensors(wl, device)


def to_device_paged(wl, device="cuda"):
    return synth.device_pages(wl, device)


def oracle_inputs(wl):
    """fp64 Q, K, V as the oracle consumes them (exact widening / dequantisation)."""
    if wl.dtype == "bf16":
        return O.decode_bf16(wl.q), O.decode_bf16(wl.k), O.decode_bf16(wl.v)
    return (O.dequantize(wl.q, wl.q_scale), O.dequantize(wl.k, wl.k_scale), O.dequantize(wl.v, wl.v_scale))


def unpack_lists(idx: np.ndarray, counts: np.ndarray, h: int, nb: int, total_tri: int, tri0: int = 0,
                 blk0: int = 0):
    """Lists of (h, i) for one sequence from the triangular-packed layout."""
    out = []
    base = h * total_tri + tri0
    for i in range(nb):
        c = int(counts[h, blk0 + i])
        s = base + i * (i + 1) // 2
        out.append(idx[s:s + max(c, 0)].copy())
    return out


def check_lists(gpu_lists, sel, alpha, n_sink, n_local, rows=None):
    """Compare GPU lists of every head (gpu_lists[h][i]) with the oracle's selection.

    Exact equality is required except for non-forced blocks inside the 1e-6 band
    around the threshold; every list must be strictly ascending, inside [0, i] and end
    with i.  Returns the number of in-band entries seen."""
    P = sel["P"]
    keep = sel["keep"]
    hq, nb, _ = P.shape
    rows = range(nb) if rows is None else rows
    ambiguous = 0
    for h in range(hq):
        for i in rows:
            lst = np.asarray(gpu_lists[h][i], dtype=np.int64)
            assert lst.size >= 1, (h, i)
            assert np.all(np.diff(lst) > 0), (h, i, lst)
            assert lst[0] >= 0 and lst[-1] == i, (h, i, lst)
            got = np.zeros(i + 1, dtype=bool)
            got[lst] = True
            want = keep[h, i, :i + 1]
            diff = np.nonzero(got != want)[0]
            if diff.size:
                j = np.arange(i + 1)
                forced = (j < n_sink) | (j > i - n_local)
                band = np.abs(P[h, i, :i + 1] - alpha) <= BAND_REL * alpha
                bad = [int(x) for x in diff if forced[x] or not band[x]]
                assert not bad, f"head {h} row {i}: blocks {bad} differ (P={P[h, i, bad]}, alpha={alpha})"
                ambiguous += diff.size
    return ambiguous
