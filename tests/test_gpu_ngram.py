"""GPU parity of the prompt-lookup / n-gram drafter against the CPU oracle,
through the C ABI. Integer work: drafts, counts and match positions are
bit-exact."""
import numpy as np
import pytest

import workloads
from oracle import ngram as og
from workloads import make_ngram

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verify_amd as rsv
    rsv.lib()
    return torch.device("cuda:0")


def _run(tokens, lengths, ngram, gamma, pad, dev, misalign=False):
    import rejection_sampling_verify_amd as rsv
    if misalign:
        # one extra leading column, then a view that starts 4 bytes in: rows are not 16-byte aligned
        wide = np.concatenate([np.full((tokens.shape[0], 1), -7, np.int32), tokens], axis=1)
        t = torch.from_numpy(wide).to(dev)[:, 1:]
    else:
        t = torch.from_numpy(tokens).to(dev)
    d, c, m = rsv.sv_ngram_draft(t, torch.from_numpy(lengths.astype(np.int32)).to(dev), ngram, gamma, pad)
    torch.cuda.synchronize()
    return d.cpu().numpy(), c.cpu().numpy(), m.cpu().numpy()


def _check(tokens, lengths, ngram, gamma, pad, dev, label, misalign=False):
    got = _run(tokens, lengths, ngram, gamma, pad, dev, misalign)
    ref = og.ngram_draft(tokens, lengths, ngram, gamma, pad)
    for name, g, r in zip(("draft", "count", "match"), got, ref):
        bad = np.argwhere(g != r)
        assert bad.size == 0, "%s: %s differs at %s (gpu %s, oracle %s)" % (
            label, name, bad[0].tolist(), g[tuple(bad[0])], r[tuple(bad[0])])
    print("[ngram parity] %s ok: matched %d of %d" % (label, int(np.sum(ref[2] >= 0)), len(lengths)), flush=True)
    return ref


CASES = {
    # name: (B, V, T_range, stride, ngram, gamma, pad, seed)
    "n1_pad_small_alphabet": (64, 5, (1, 200), 200, 1, 6, True, 1),
    "n3_lookup": (48, 40, (0, 3000), 3000, 3, 4, False, 2),
    "n3_pad_ragged_stride": (40, 60, (10, 5001), 5003, 3, 6, True, 3),   # stride not a multiple of 4
    "n4_lookup_long": (12, 1000, (9000, 20000), 20000, 4, 8, False, 4),  # several chunks
    "n2_pad_gamma1": (32, 8, (2, 700), 704, 2, 1, True, 5),
    "n16_lookup": (24, 3, (0, 400), 400, 16, 5, False, 6),
    "n1_lookup_cut_at_end": (48, 3, (0, 50), 52, 1, 6, False, 9),  # matches near the end: short continuations
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_ngram_parity(dev, name):
    B, V, T_range, stride, ngram, gamma, pad, seed = CASES[name]
    inp = make_ngram(name, B, V, T_range, ngram=ngram, gamma=gamma, pad=pad, seed=seed, stride=stride)
    ref = _check(inp.tokens, inp.lengths, ngram, gamma, pad, dev, name)
    assert np.any(ref[2] >= 0)


def test_ngram_misaligned_rows(dev):
    inp = make_ngram("misaligned", 16, 30, (50, 3000), ngram=3, gamma=6, pad=False, seed=7, stride=3000)
    _check(inp.tokens, inp.lengths, 3, 6, False, dev, "misaligned", misalign=True)
    _check(inp.tokens, inp.lengths, 3, 6, True, dev, "misaligned pad", misalign=True)


def test_ngram_edge_lengths(dev):
    """Lengths 0, 1, n, n + 1, the stride, above the stride and negative, in
    both modes; one row whose only match is at the very start of a long
    history (the scan crosses every chunk); one row with no match."""
    stride = 12000
    rows = []
    lens = []
    rng = np.random.default_rng(8)
    base = rng.integers(100, 200, stride).astype(np.int32)
    for T in (0, 1, 3, 4, stride, stride + 1, -5, 2):
        rows.append(base.copy())
        lens.append(T)
    far = np.arange(1000, 1000 + stride, dtype=np.int32)  # all distinct
    far[-3:] = far[:3]   # the tail trigram occurs only at the start
    rows.append(far)
    lens.append(stride)
    none = np.arange(5000, 5000 + stride, dtype=np.int32)
    rows.append(none)
    lens.append(stride)
    tokens = np.stack(rows)
    lengths = np.array(lens, np.int32)
    for pad in (False, True):
        for ngram, gamma in ((3, 6), (1, 4)):
            ref = _check(tokens, lengths, ngram, gamma, pad, dev, "edges n=%d pad=%d" % (ngram, pad))
            assert ref[1][5] == -1 and ref[1][6] == -1
    ref = og.ngram_draft(tokens, lengths, 3, 6, False)
    assert ref[2][8] == 0 and ref[2][9] == -1 and ref[1][9] == 0


def test_ngram_named_workload_full_size(dev):
    inp = workloads.make_extra("ngram_draft_qwen")
    ref = _check(inp.tokens, inp.lengths, inp.ngram, inp.gamma, inp.pad, dev, "ngram_draft_qwen")
    assert 0.3 < np.mean(ref[2] >= 0) < 0.9
