"""GPU parity of the one-hot residual draw on long, shaped rows, through the
C ABI, against the CPU oracle.

With a one-hot draft ([SB] Exercise 4) the replacement is p without the
drafted token, drawn by Gumbel-max over the whole row. The cases shape the
rows in spans of 16384 entries: mass in one span only, spans emptied (every
entry -inf), the drafted token alone in its span, one span much heavier than
the rest; with a ragged end, rows that are not 16-byte aligned (the scalar
paths), fp32, every pass-1 chunk length, and a vocabulary of more than a
million entries with more pass-1 slots than one polling batch of the
decision.
"""
import numpy as np
import pytest

import oracle
from workloads import make_chain, round_bf16

from gpu_util import compare_chain, oracle_sample, run_sample

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

K = 16384  # the span length the rows are shaped in


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verify_amd as rsv
    rsv.lib()
    return torch.device("cuda:0")


def _shape_spans(inp, seed):
    """Per sequence, one of: mass spread over every span; all spans but one
    emptied; the drafted token alone in its span; one span much heavier than
    the rest. Applied to every target row, so whichever position is rejected
    has that shape."""
    rng = np.random.default_rng(seed)
    V = inp.meta["V"]
    nb = (V + K - 1) // K
    bf16 = inp.target.dtype == np.uint16
    ninf = np.uint16(0xFF80) if bf16 else np.float32(-np.inf)
    B, rows = inp.target.shape[0], inp.target.shape[1]
    for b in range(B):
        kind = b % 4
        for r in range(rows):
            row = inp.target[b, r]
            x = int(inp.draft_ids[b, min(r, inp.draft_ids.shape[1] - 1)])
            if kind == 1:
                keep = int(rng.integers(nb))
                for j in range(nb):
                    if j != keep:
                        lo, hi = j * K, min(V, (j + 1) * K)
                        xv = row[x] if lo <= x < hi else None
                        row[lo:hi] = ninf
                        if xv is not None:
                            row[x] = xv
            elif kind == 2:
                j = x // K
                lo, hi = j * K, min(V, (j + 1) * K)
                xv = row[x]
                row[lo:hi] = ninf
                row[x] = xv
            elif kind == 3:
                j = int(rng.integers(nb))
                lo, hi = j * K, min(V, (j + 1) * K)
                vals = (np.linspace(0, 1, hi - lo) * 4.0 + 3.0).astype(np.float32)
                row[lo:hi] = round_bf16(vals) if bf16 else vals
    return inp


@pytest.mark.parametrize("bf16,V", [(True, 3 * K + 776), (True, 3 * K + 777), (False, 2 * K + 3001)])
def test_onehot_shaped_rows_match_oracle(dev, bf16, V):
    inp = make_chain("onehot_rows", 48, 3, V, bf16=bf16, seed=51, target_sigma=3.0,
                     temperatures=(0.7, 1.0), one_hot=True, onehot_hit=0.5)
    _shape_spans(inp, 52)
    ref = oracle_sample(inp)
    # rejections at several positions, replacements from several spans
    rej = ref["n"] < 3
    assert rej.sum() >= 24
    spans = {int(ref["tokens"][b, ref["n"][b]]) // K for b in np.nonzero(rej)[0]}
    assert len(spans) >= 3
    for tiling in (None, (8, 0), (4, 0), (1, 0), (0, 3)):
        got = run_sample(inp, torch, dev, tiling=tiling)
        compare_chain(got, ref, label="onehot rows %s %d %s" % (bf16, V, tiling))


def test_onehot_long_rows(dev):
    """V just over 2^20 (65 spans, 4 x 65 pass-1 slots per sequence, more
    than one polling batch); some sequences hold their mass only in the last
    two spans."""
    V = 64 * K + 1000
    inp = make_chain("onehot_long_rows", 8, 4, V, bf16=True, seed=53, target_sigma=2.0,
                     temperatures=(1.0,), one_hot=True, onehot_hit=0.3)
    ninf = np.uint16(0xFF80)
    for b in range(0, 8, 2):
        for r in range(5):
            x = int(inp.draft_ids[b, min(r, 3)])
            xv = inp.target[b, r, x]
            inp.target[b, r, :63 * K] = ninf
            if x < 63 * K:
                inp.target[b, r, x] = xv
    ref = oracle_sample(inp)
    assert (ref["n"] < 4).sum() >= 4
    late = [b for b in range(0, 8, 2) if ref["n"][b] < 4]
    assert all(ref["tokens"][b, ref["n"][b]] >= 63 * K for b in late)
    for tiling in (None, (8, 0), (2, 0)):
        got = run_sample(inp, torch, dev, tiling=tiling)
        compare_chain(got, ref, label="onehot long rows %s" % (tiling,))
