"""GPU parity at the edges of the rule and of the logits contract, through the
C ABI, against the CPU oracle.

[SB] "A From-Scratch Implementation" asks for care where a probability is
tiny; the cases here drive that through the kernels: a drafted token whose
draft probability underflows (a = 1) or whose target probability is zero
(a = 0), rows with masked (-inf) entries, a row with a single finite entry,
the empty-residual fallback (reachable only when p and q agree up to
rounding), logits outside the f16 range the packed maximum reads, and rows
that define no distribution (code SV_SEQ_BAD_LOGITS). Every case also runs at
the full pass-1 tile width (the packed bf16 paths) through the debug entry
point with a fixed tiling. Then: the sequence-index base (a batch split over
two calls reproduces one call), calls on a side stream with the wrappers'
own allocations, and a workspace left dirty by an aborted call.
"""
import numpy as np
import pytest

import oracle
from workloads import bf16_to_f32, make_chain, make_tree, round_bf16

from gpu_util import compare_chain, oracle_sample, run_sample, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BF16_PINF, BF16_NINF, BF16_NAN = 0x7F80, 0xFF80, 0x7FC0
BF16_HUGE, BF16_NHUGE = 0x7E00, 0xFE00  # +-2^125: outside the packed f16 reading


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verify_amd as rsv
    rsv.lib()
    return torch.device("cuda:0")


def _put(a, b, i, v, value):
    """Store `value` (a float, or a bf16 bit pattern for uint16 arrays) at [b, i, v]."""
    if a.dtype == np.uint16:
        a[b, i, v] = value if isinstance(value, (int, np.integer)) else round_bf16(np.float32([value]))[0]
    else:
        a[b, i, v] = np.float32(value)


def _both_tilings(inp, dev, **kw):
    """The library's own tiling and the full-width pass-1 tile (8 vectors per
    thread: the packed bf16 paths wherever a chunk is whole)."""
    return [run_sample(inp, torch, dev, **kw), run_sample(inp, torch, dev, tiling=(8, 0), **kw)]


@pytest.mark.parametrize("bf16", [True, False])
def test_empty_residual_fallback(dev, bf16):
    """p and q agree bit for bit except at the drafted token, whose draft
    logit (-40) is too small to move any normalizer sum and whose target logit
    (-100) makes a about e^-60: the residual has no candidate in fp32 (and in
    fp64), and both sides draw the correction from p at the rejected row with
    its noise."""
    B, G, V = 12, 2, 40000
    inp = make_chain("fallback", B, G, V, bf16=bf16, seed=501, target_sigma=1.0, draft_sigma=0.5,
                     temperatures=(1.0, 0.8))
    inp.draft[:, 0, :] = inp.target[:, 0, :]
    for b in range(B):
        x = int(inp.draft_ids[b, 0])
        _put(inp.target, b, 0, x, -100.0)
        _put(inp.draft, b, 0, x, -40.0)
    ref = oracle_sample(inp)
    assert np.all(ref["n"] == 0)
    assert np.all(ref["flags"] & oracle.FLAG_FALLBACK)
    for got in _both_tilings(inp, dev):
        compare_chain(got, ref, label="fallback bf16=%s" % bf16)
        assert np.all(got["residual_mass"] == 0.0)


@pytest.mark.parametrize("bf16", [True, False])
def test_masked_and_underflowing_probabilities(dev, bf16):
    """Masked (-inf) entries in target and draft rows; p(x) = 0 (a = 0, never
    accepted); q(x) = 0 (a = 1, always accepted); a draft logit so low that
    q(x) underflows fp32 (a = 1); a target row with one finite entry (p one-hot
    there); one-hot drafts over masked rows; greedy sequences over masked
    rows."""
    B, G, V = 24, 3, 40000
    inp = make_chain("masked", B, G, V, bf16=bf16, seed=502, target_sigma=2.0, draft_sigma=0.7,
                     temperatures=(0.0, 0.7, 1.0))
    rng = np.random.default_rng(502)
    neg_inf = BF16_NINF if bf16 else -np.inf
    for b in range(B):
        for i in range(G + 1):
            for v in rng.choice(V, size=400, replace=False):
                _put(inp.target, b, i, int(v), neg_inf)
        for i in range(G):
            for v in rng.choice(V, size=300, replace=False):
                _put(inp.draft, b, i, int(v), neg_inf)
        x0 = int(inp.draft_ids[b, 0])
        kind = b % 4
        if kind == 0:                 # p(x) = 0: rejected at position 0
            _put(inp.target, b, 0, x0, neg_inf)
        elif kind == 1:               # q(x) = 0: a = 1
            _put(inp.draft, b, 0, x0, neg_inf)
        elif kind == 2:               # q(x) underflows fp32 (l/T about -300)
            _put(inp.draft, b, 0, x0, -250.0)
        else:                         # a target row with a single finite entry: x0
            inp.target[b, 0, :] = neg_inf
            _put(inp.target, b, 0, x0, 1.5)
    ref = oracle_sample(inp)
    sampled = inp.temperature > 0
    assert np.all(ref["n"][sampled & (np.arange(B) % 4 == 0)] == 0)
    assert np.all(ref["n"][sampled & (np.arange(B) % 4 != 0)] >= 1)
    for got in _both_tilings(inp, dev):
        compare_chain(got, ref, label="masked bf16=%s" % bf16)
    # One-hot drafts over the same rows.
    oh = make_chain("masked_onehot", B, G, V, bf16=bf16, seed=503, target_sigma=2.0, one_hot=True,
                    temperatures=(1.0, 0.6))
    oh.target[:, :, :] = inp.target
    oh.target[:, 1, :] = neg_inf            # row 1: p one-hot at the drafted token
    for b in range(B):
        _put(oh.target, b, 1, int(oh.draft_ids[b, 1]), 0.25)
    ref = oracle_sample(oh)
    for got in _both_tilings(oh, dev):
        compare_chain(got, ref, label="masked one-hot bf16=%s" % bf16)


@pytest.mark.parametrize("one_hot", [False, True])
def test_pruning_bound_on_shifted_rows(dev, one_hot):
    """The draws' lane-level bound reads a vector's eight bf16 patterns as
    signed 16-bit integers: exact when some element is >= 0, 0 when all are
    negative. Rows shifted far below zero (every lane negative), rows shifted
    far above zero (every lane positive), and sequences whose drafts are all
    accepted and whose bonus row holds one logit of 2^125 (beyond the f16
    reading's range) must still draw exactly the oracle's tokens: residual,
    one-hot residual and bonus draws."""
    B, G, V = 18, 3, 20000
    inp = make_chain("shifted", B, G, V, bf16=True, seed=512, target_sigma=2.0, draft_sigma=0.7,
                     temperatures=(0.7, 1.0, 1.6), one_hot=one_hot)
    rng = np.random.default_rng(513)
    t = bf16_to_f32(inp.target)
    d = bf16_to_f32(inp.draft) if not one_hot else None
    huge = []
    for b in range(B):
        kind = b % 3
        if kind < 2:
            shift = np.float32(-80.0 if kind == 0 else 80.0)
            inp.target[b] = round_bf16(t[b] + shift)
            if not one_hot:
                inp.draft[b] = round_bf16(d[b] + shift)
        else:
            # Every draft accepted (q = p, or p one-hot at the drafted token),
            # then the bonus draw meets a logit of 2^125.
            if one_hot:
                for i in range(G):
                    inp.target[b, i, :] = BF16_NINF
                    inp.target[b, i, int(inp.draft_ids[b, i])] = round_bf16(np.float32([0.5]))[0]
            else:
                inp.draft[b] = inp.target[b, :G]
            h = int(rng.integers(V))
            inp.target[b, G, h] = BF16_HUGE
            huge.append((b, h))
    ref = oracle_sample(inp)
    for b, h in huge:
        assert ref["n"][b] == G and ref["tokens"][b, G] == h
    assert np.any(ref["n"][np.arange(B) % 3 < 2] < G)  # some shifted sequences end in a residual draw
    for got in _both_tilings(inp, dev):
        compare_chain(got, ref, check_diag=False, label="shifted rows one_hot=%s" % one_hot)


def test_logits_outside_the_packed_range(dev):
    """bf16 logits the packed f16 maximum cannot see: +-2^125, +inf, NaN.
    Greedy rows take the argmax (+inf the largest, lowest index among ties,
    huge finite values exactly); in sampled rows -2^125 is a token of
    probability 0; a sampled row with +inf or NaN, or without a finite entry,
    reports SV_SEQ_BAD_LOGITS, as does a bonus row without a finite entry;
    +inf in a bonus row is drawn."""
    B, G, V = 16, 3, 40000
    inp = make_chain("outside", B, G, V, bf16=True, seed=504, target_sigma=2.0, draft_sigma=0.7,
                     temperatures=(1.0,))
    inp.temperature[:8] = 0.0
    # Greedy sequences 0..7
    inp.target[0, 0, [100, 20000, 39999]] = BF16_PINF       # three +inf in chunks 0, 1 and the tail
    inp.target[0, 1, 5000] = BF16_HUGE
    inp.target[1, :, :] = BF16_NINF                         # every row -inf but two huge negatives
    inp.target[1, :, 17] = BF16_NHUGE
    inp.target[1, :, 30000] = BF16_NHUGE
    inp.target[2, 0, 123] = BF16_HUGE
    inp.target[2, 0, 124] = BF16_PINF
    inp.target[3, 2, :] = BF16_NINF                         # an all -inf row: argmax is index 0
    inp.draft_ids[0, 0] = 100
    inp.draft_ids[2, 0] = 124
    # Sampled sequences 8..15
    inp.target[8, 0, 777] = round_bf16(np.float32([60.0]))[0]   # p one-hot at 777 (to fp32 rounding)
    inp.draft_ids[8, 0] = 777
    inp.draft[9, 1, 5] = round_bf16(np.float32([60.0]))[0]      # q one-hot at 5: a(x) ~ 0 unless x = 5
    inp.target[10, 1, 9] = BF16_PINF                        # +inf in a scored row: bad logits
    inp.draft[11, 0, 9] = BF16_NAN                          # NaN in a draft row: bad logits
    inp.target[12, 2, :] = BF16_NINF                        # a scored row without a finite entry
    inp.target[13, G, :] = BF16_NINF                        # bonus row without a finite entry
    inp.target[14, G, [31, 33000]] = BF16_PINF              # +inf in the bonus row
    inp.target[15, 0, 3] = BF16_NHUGE                       # a huge negative logit is probability 0
    inp.draft_ids[15, 0] = 3
    for b in (13, 14):                                      # make sure every draft is accepted
        inp.draft[b, :, :] = inp.target[b, :G, :]
    ref = oracle_sample(inp)
    assert ref["tokens"][0, 0] == 100 and ref["n"][0] >= 1
    assert list(ref["n"][10:14]) == [oracle.SEQ_BAD_LOGITS] * 4
    assert ref["n"][14] == G and ref["tokens"][14, G] == 31
    for got in _both_tilings(inp, dev):
        compare_chain(got, ref, check_diag=False, label="outside the packed range")
        ok = ~np.isnan(ref["accept_prob"])
        assert np.array_equal(np.isnan(got["accept_prob"]), ~ok)
        assert np.abs(got["accept_prob"][ok] - ref["accept_prob"][ok]).max() <= 1e-5


def test_greedy_entry_point_outside_the_packed_range(dev):
    import rejection_sampling_verify_amd as rsv
    B, G, V = 6, 2, 40000
    rng = np.random.default_rng(505)
    tgt = round_bf16(rng.normal(0, 1, (B, G + 1, V)).astype(np.float32))
    tgt[0, 0, [7, 16390]] = BF16_PINF
    tgt[1, 1, :] = BF16_NINF
    tgt[2, 0, 20000] = BF16_HUGE
    tgt[3, 0, :] = BF16_NHUGE
    tgt[4, 2, 39998] = BF16_PINF
    ids = rng.integers(0, V, (B, G)).astype(np.int32)
    ids[0, 0] = 7
    ref = oracle.verify_greedy(tgt, ids)
    tok, n = rsv.spec_verify_greedy(to_dev(tgt, torch, dev), torch.from_numpy(ids).to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(n.cpu().numpy(), ref["n"]) and np.array_equal(tok.cpu().numpy(), ref["tokens"])


def test_split_batch_reproduces_one_call(dev):
    """seq_base: the two halves of a batch, called with the global index of
    their first sequence, give exactly the outputs of one call over the batch
    (chains with dense and one-hot drafts, sampled trees)."""
    import rejection_sampling_verify_amd as rsv
    for one_hot in (False, True):
        inp = make_chain("split", 24, 5, 30016, bf16=True, seed=506, target_sigma=3.0, draft_sigma=(0.3, 1.5),
                         temperatures=(0.0, 0.7, 1.0), one_hot=one_hot)
        full = run_sample(inp, torch, dev, diag=False)
        compare_chain(full, oracle_sample(inp), check_diag=False, label="split full")
        t = to_dev(inp.target, torch, dev)
        d = to_dev(inp.draft, torch, dev)
        ids = torch.from_numpy(inp.draft_ids).to(dev)
        temp = torch.from_numpy(inp.temperature).to(dev)
        parts = []
        for lo, hi in ((0, 11), (11, 24)):
            tok, n = rsv.spec_verify_sample(t[lo:hi], None if d is None else d[lo:hi], ids[lo:hi].contiguous(),
                                            temp[lo:hi].contiguous(), seed=0, offset=0, seq_base=lo)
            parts.append((tok, n))
        torch.cuda.synchronize()
        assert np.array_equal(np.concatenate([p[1].cpu().numpy() for p in parts]), full["n"])
        assert np.array_equal(np.concatenate([p[0].cpu().numpy() for p in parts]), full["tokens"])
    # Sampled trees.
    from workloads import make_tree_sample, tree_c5_structure
    parents, depth = tree_c5_structure()
    ts = make_tree_sample("split_tree", 10, 20016, parents, depth, bf16=True, seed=507, temperatures=(0.8, 1.0))
    args = [to_dev(ts.target, torch, dev), to_dev(ts.draft, torch, dev), torch.from_numpy(parents).to(dev),
            torch.from_numpy(depth).to(dev), torch.from_numpy(ts.node_tokens).to(dev),
            torch.from_numpy(ts.temperature).to(dev)]
    path, plen, token = rsv.spec_verify_tree_sample(*args, ts.max_depth, seed=5)
    halves = []
    for lo, hi in ((0, 4), (4, 10)):
        a = [x[lo:hi].contiguous() if i in (0, 1, 4, 5) else x for i, x in enumerate(args)]
        halves.append(rsv.spec_verify_tree_sample(*a, ts.max_depth, seed=5, seq_base=lo))
    torch.cuda.synchronize()
    for k, whole in enumerate((path, plen, token)):
        assert np.array_equal(np.concatenate([h[k].cpu().numpy() for h in halves]), whole.cpu().numpy())


def test_side_stream_with_default_allocations(dev):
    """Every verify wrapper called on a side stream, letting the wrapper
    allocate its outputs and workspace: the allocations belong to that stream
    (zeroed on it, reused only after its kernels), and results match the
    oracle."""
    import rejection_sampling_verify_amd as rsv
    side = torch.cuda.Stream()
    inp = make_chain("side", 16, 4, 20011, bf16=True, seed=508, target_sigma=2.0, draft_sigma=1.0,
                     temperatures=(0.0, 1.0))
    t, d = to_dev(inp.target, torch, dev), to_dev(inp.draft, torch, dev)
    ids, temp = torch.from_numpy(inp.draft_ids).to(dev), torch.from_numpy(inp.temperature).to(dev)
    torch.cuda.synchronize()
    for rep in range(3):
        with torch.cuda.stream(side):
            junk = torch.full((1 << 20,), 7, dtype=torch.int32, device=dev)  # recycled memory is not zero
        del junk
        tok, n = rsv.spec_verify_sample(t, d, ids, temp, stream=side)
        gtok, gn = rsv.spec_verify_greedy(t, ids, stream=side)
        side.synchronize()
        ref = oracle_sample(inp)
        assert np.array_equal(n.cpu().numpy(), ref["n"]) and np.array_equal(tok.cpu().numpy(), ref["tokens"])
        gref = oracle.verify_greedy(inp.target, inp.draft_ids)
        assert np.array_equal(gn.cpu().numpy(), gref["n"]) and np.array_equal(gtok.cpu().numpy(), gref["tokens"])
    from workloads import tree_c5_structure
    parents, depth = tree_c5_structure()
    tr = make_tree("side_tree", 8, 9001, parents, depth, bf16=True, seed=509, hit=0.6)
    path, plen, bonus = rsv.spec_verify_tree(to_dev(tr.target, torch, dev), torch.from_numpy(parents).to(dev),
                                             torch.from_numpy(depth).to(dev), torch.from_numpy(tr.node_tokens).to(dev),
                                             tr.max_depth, stream=side)
    side.synchronize()
    tref = oracle.verify_tree(tr.target, parents, depth, tr.node_tokens, tr.max_depth)
    assert np.array_equal(plen.cpu().numpy(), tref["path_len"]) and np.array_equal(bonus.cpu().numpy(), tref["bonus"])


def test_dirty_workspace_reports_internal_code(dev):
    """A workspace whose abort word is set (as a bounded wait that gave up
    leaves it) makes every decision report SV_SEQ_INTERNAL without waiting on
    it; sv_workspace_init returns it to a clean state for the next call. The
    word is set from the host, so every kernel still runs to its end."""
    import rejection_sampling_verify_amd as rsv
    inp = make_chain("dirty", 8, 3, 9001, bf16=True, seed=510, target_sigma=2.0, draft_sigma=1.0,
                     temperatures=(0.0, 1.0))
    ws = rsv.Workspace(dev).get(8, 4, 9001)
    ws.view(torch.int32)[1] = 1
    got = run_sample(inp, torch, dev, workspace=ws, diag=False)
    assert np.all(got["n"] == rsv.SV_SEQ_INTERNAL) and np.all(got["tokens"] == -1)
    rsv.sv_workspace_init(ws)
    compare_chain(run_sample(inp, torch, dev, workspace=ws), oracle_sample(inp), label="after init")
    assert int(ws.count_nonzero().item()) == 0
    # Greedy trees.
    from workloads import tree_c5_structure
    parents, depth = tree_c5_structure()
    tr = make_tree("dirty_tree", 4, 5001, parents, depth, bf16=True, seed=511, hit=0.6)
    wt = rsv.Workspace(dev).get(4, len(parents), 5001)
    args = (to_dev(tr.target, torch, dev), torch.from_numpy(parents).to(dev), torch.from_numpy(depth).to(dev),
            torch.from_numpy(tr.node_tokens).to(dev), tr.max_depth)
    wt.view(torch.int32)[1] = 1
    path, plen, bonus = rsv.spec_verify_tree(*args, workspace=wt)
    torch.cuda.synchronize()
    assert np.all(plen.cpu().numpy() == rsv.SV_SEQ_INTERNAL) and np.all(bonus.cpu().numpy() == -1)
    rsv.sv_workspace_init(wt)
    path, plen, bonus = rsv.spec_verify_tree(*args, workspace=wt)
    torch.cuda.synchronize()
    tref = oracle.verify_tree(tr.target, parents, depth, tr.node_tokens, tr.max_depth)
    assert np.array_equal(plen.cpu().numpy(), tref["path_len"]) and np.array_equal(path.cpu().numpy(), tref["path"])
    assert int(wt.count_nonzero().item()) == 0
