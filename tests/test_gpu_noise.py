"""The kernels' random primitives on the GPU, element by element, through the
C ABI's diagnostic entry points: Philox4x32-10 against the published
known-answer vectors and the oracle's Philox, and the word -> uniform / Gumbel
maps against the oracle and their fp64 definition."""
import json
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
import oracle  # noqa: E402

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verify_amd as rsv
    rsv.lib()
    return torch.device("cuda:0")


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32))


def _philox_gpu(ctr, key, dev):
    import rejection_sampling_verify_amd as rsv
    out = rsv.sv_debug_philox(_i32(ctr).to(dev), _i32(key).to(dev))
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint32)


def test_philox_known_answers(dev):
    kat = json.load(open(os.path.join(GOLDEN, "philox_kat.json")))
    ctr = np.array([[int(x, 16) for x in v["ctr"]] for v in kat["vectors"]], np.uint32)
    key = np.array([[int(x, 16) for x in v["key"]] for v in kat["vectors"]], np.uint32)
    want = np.array([[int(x, 16) for x in v["out"]] for v in kat["vectors"]], np.uint32)
    assert np.array_equal(_philox_gpu(ctr, key, dev), want)


def test_philox_matches_oracle(dev):
    rng = np.random.default_rng(5)
    n = 4096
    ctr = rng.integers(0, 1 << 32, size=(n, 4), dtype=np.uint64).astype(np.uint32)
    key = rng.integers(0, 1 << 32, size=(n, 2), dtype=np.uint64).astype(np.uint32)
    ctr[:64, 0] = np.arange(64)  # small counters, as the kernels use them
    ctr[:64, 1:] = 0
    got = _philox_gpu(ctr, key, dev)
    for i in range(0, n, 7):
        assert np.array_equal(got[i], oracle.philox4x32_10(ctr[i], key[i])), i


def _noise_gpu(words, dev):
    import rejection_sampling_verify_amd as rsv
    g, u = rsv.sv_debug_noise(_i32(words).to(dev))
    torch.cuda.synchronize()
    return g.cpu().numpy().astype(np.float64), u.cpu().numpy().astype(np.float64)


def _gumbel_tol(g):
    # fp32 evaluation of -ln(-ln U): about one rounding of the result plus the
    # relative error of the inner logarithm carried through the outer one.
    return 5e-7 + 2.5e-7 * np.abs(g)


def test_noise_maps_against_oracle(dev):
    """Words drawn through the kernels' counter layout; the oracle computes the
    same uniforms and Gumbel noise from the same counters."""
    seed, off = 0x1234_5678_9ABC, 3
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint32)
    words, gref, uref = [], [], []
    for b in range(3):
        for pos in range(4):
            for v in range(0, 4000, 3):
                w = oracle.philox4x32_10([v // 4, pos, b, 2 * off + 1], key)[v % 4]
                words.append(w)
                gref.append(oracle.gumbel(seed, off, b, pos, v))
                uref.append(np.nan)
            w = oracle.philox4x32_10([0, pos, b, 2 * off], key)[0]
            words.append(w)
            gref.append(np.nan)
            uref.append(oracle.accept_uniform(seed, off, b, pos))
    words = np.array(words, np.uint32)
    gref, uref = np.array(gref), np.array(uref)
    g, u = _noise_gpu(words, dev)
    mg, mu = ~np.isnan(gref), ~np.isnan(uref)
    assert np.array_equal(u[mu], uref[mu])  # exact: a 24-bit integer times 2^-24
    err = np.abs(g[mg] - gref[mg])
    print("[noise] max |G_gpu - G_oracle| = %.3g over %d words" % (err.max(), mg.sum()))
    assert np.all(err <= _gumbel_tol(gref[mg]))


def test_noise_maps_extreme_words(dev):
    """Every branch of the fp32 Gumbel evaluation: U near 0, near 1/2, near 1,
    against the fp64 definition G = -ln(-ln U), U = ((w >> 8) + 0.5) 2^-24."""
    j = np.concatenate([np.arange(0, 4096), np.arange((1 << 23) - 2048, (1 << 23) + 2048),
                        np.arange((1 << 24) - 65536, 1 << 24),
                        np.random.default_rng(6).integers(0, 1 << 24, 200000)]).astype(np.uint64)
    low = np.random.default_rng(7).integers(0, 256, j.size).astype(np.uint64)
    words = ((j << 8) | low).astype(np.uint32)
    g, u = _noise_gpu(words, dev)
    U = (j.astype(np.float64) + 0.5) * 2.0 ** -24
    gref = -np.log(-np.log(U))
    assert np.array_equal(u, j.astype(np.float64) * 2.0 ** -24)
    err = np.abs(g - gref)
    worst = int(np.argmax(err / _gumbel_tol(gref)))
    print("[noise] max |G - G_fp64| = %.3g; worst relative to tolerance at j=%d (G=%.6f)"
          % (err.max(), int(j[worst]), gref[worst]))
    assert np.all(err <= _gumbel_tol(gref))
    assert np.all(np.diff(g[np.argsort(j, kind="stable")]) >= 0)  # monotone in U


def test_wave_max(dev):
    """The wave-wide maximum the kernels use (row-local DPP steps, then the
    16- and 32-lane row swaps): every lane of every wave holds the group max,
    for maxima in every lane position and with -inf and ties."""
    import rejection_sampling_verify_amd as rsv
    rng = np.random.default_rng(8)
    groups = []
    for pos in range(64):  # the maximum in each lane position
        g = rng.standard_normal(64).astype(np.float32)
        g[pos] = 10.0 + pos
        groups.append(g)
    groups.append(np.full(64, -np.inf, np.float32))
    g = np.full(64, -np.inf, np.float32)
    g[37] = -5.0
    groups.append(g)
    groups.append(np.full(64, 3.25, np.float32))
    for _ in range(64):
        groups.append(rng.standard_normal(64).astype(np.float32) * 100)
    x = np.concatenate(groups)
    out = rsv.sv_debug_wave_max(torch.from_numpy(x).to(dev)).cpu().numpy()
    torch.cuda.synchronize()
    want = np.repeat(x.reshape(-1, 64).max(axis=1), 64)
    assert np.array_equal(out, want)


def test_read_stream_reads_every_word_once(dev):
    """The read-bandwidth yardstick reads each 16-byte word exactly once: the
    XOR of its per-wave folds equals the XOR of all words, for a ragged size
    and an odd grid."""
    import rejection_sampling_verify_amd as rsv
    rng = np.random.default_rng(9)
    for nwords, nblocks in ((4 * (1 << 20) + 12, 37), (4 * 1000, 2048), (4, 1)):
        h = rng.integers(0, 1 << 32, size=nwords, dtype=np.uint64).astype(np.uint32)
        buf = torch.from_numpy(h.view(np.int32)).to(dev)
        out = rsv.sv_debug_read_stream(buf, nblocks)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
        assert got == np.bitwise_xor.reduce(h), (nwords, nblocks)
