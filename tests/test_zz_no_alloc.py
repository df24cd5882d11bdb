"""The allocation-free entry point (spec_verify_sample_noalloc, its scratch a
static device array) against spec_verify_sample with a workspace, through the
C ABI, and against the oracle: two calls in a row on one GPU, the second
smaller, so that the second starts from the first one's leftover scratch.
Also: a call whose scratch need exceeds the static array is refused before
anything is launched."""
import numpy as np
import pytest

from workloads import make_chain

from gpu_util import compare_chain, oracle_sample, run_sample, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verify_amd as rsv
    rsv.lib()
    return torch.device("cuda:0")


def _noalloc(inp, dev, diag=True):
    import rejection_sampling_verify_amd as rsv
    B, G = inp.draft_ids.shape
    t, d = to_dev(inp.target, torch, dev), to_dev(inp.draft, torch, dev)
    ids, temp = torch.from_numpy(inp.draft_ids).to(dev), torch.from_numpy(inp.temperature).to(dev)
    tok = torch.full((B, G + 1), -7, dtype=torch.int32, device=dev)
    n = torch.full((B,), -7, dtype=torch.int32, device=dev)
    dg = None
    if diag:
        dg = {"accept_prob": torch.full((B, G), float("nan"), device=dev),
              "logz_target": torch.full((B, G), float("nan"), device=dev),
              "logz_draft": torch.full((B, G), float("nan"), device=dev),
              "residual_mass": torch.full((B,), float("nan"), device=dev)}
    torch.cuda.synchronize()
    rsv.spec_verify_sample_noalloc(t, d, ids, temp, tok, n, seed=inp.seed, offset=inp.offset, diag=dg,
                                   V=inp.meta.get("V", inp.V))
    torch.cuda.synchronize()
    out = {"tokens": tok.cpu().numpy(), "n": n.cpu().numpy()}
    if dg:
        for k, v in dg.items():
            out[k] = v.cpu().numpy().astype(np.float64)
    return out


def test_noalloc_matches_workspace_entry_point(dev):
    cases = [
        make_chain("noalloc_large", 96, 8, 128256, bf16=True, seed=601, target_sigma=3.0, boost="zipf",
                   draft_sigma=(0.2, 2.0), temperatures=(0.0, 0.7, 1.0)),
        make_chain("noalloc_small", 9, 3, 5003, bf16=True, seed=602, target_sigma=2.0, draft_sigma=0.8,
                   temperatures=(0.0, 1.0)),
        make_chain("noalloc_onehot", 40, 6, 30016, bf16=True, seed=603, target_sigma=3.0, one_hot=True,
                   temperatures=(1.0,)),
    ]
    for inp in cases:
        got = _noalloc(inp, dev)
        ref_ws = run_sample(inp, torch, dev)
        for key in ("tokens", "n", "accept_prob", "logz_target", "logz_draft"):
            assert np.array_equal(got[key], ref_ws[key], equal_nan=True), (inp.name, key)
        np.testing.assert_allclose(got["residual_mass"], ref_ws["residual_mass"], rtol=0, atol=1e-6)
        compare_chain(got, oracle_sample(inp), label="noalloc " + inp.name)


def test_noalloc_refuses_beyond_its_scratch(dev):
    """B = 4096, gamma = 16, V = 152064 needs more scratch than the static
    array holds: refused on the host (the pointers are never read)."""
    import ctypes
    import rejection_sampling_verify_amd as rsv
    B, G, V = 4096, 16, 152064
    assert rsv.sv_workspace_bytes(B, G + 1, V) > rsv.SV_NOALLOC_SCRATCH_BYTES
    small = torch.zeros(64, dtype=torch.int32, device=dev)
    P = ctypes.c_void_p(small.data_ptr())
    st = rsv.lib().spec_verify_sample_noalloc(P, V, None, 0, rsv.SV_DTYPE_BF16, P, P, B, G, V, 0, 0, 0, P, P, None,
                                              None)
    assert st == rsv.SV_ERR_SCRATCH_LIMIT
