"""GPU parity of the tree attention mask and position ids against the CPU
oracle, through the C ABI. Bit and integer work: bit-exact."""
import numpy as np
import pytest

import workloads
from oracle import trees
from workloads import make_tree_mask

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verify_amd as rsv
    rsv.lib()
    return torch.device("cuda:0")


def _run(parents, offsets, dev, packed=False, shared_B=None, misalign=False):
    import rejection_sampling_verify_amd as rsv
    par = torch.from_numpy(parents).to(dev)
    off = torch.from_numpy(offsets).to(dev) if offsets is not None else None
    B = shared_B if shared_B is not None else parents.shape[0]
    N = parents.shape[-1]
    out = None
    if misalign and not packed:
        buf = torch.zeros(B * N * N + 1, dtype=torch.bool, device=dev)
        out = buf[1:].view(B, N, N)  # starts one byte past an aligned address
    mask, pos = rsv.sv_tree_mask(par, off, B=B, packed=packed, out_mask=out)
    torch.cuda.synchronize()
    m = mask.cpu().numpy()
    if packed:
        m = m.view(np.uint32)
    return m.astype(np.uint8) if not packed else m, pos.cpu().numpy()


def _check(parents, offsets, dev, label, **kw):
    got_m, got_p = _run(parents, offsets, dev, **kw)
    B = kw.get("shared_B") or parents.shape[0]
    ref_m, ref_p = trees.tree_attn_batch(parents if parents.ndim == 2 else np.broadcast_to(parents, (B, len(parents))),
                                         offsets, packed=kw.get("packed", False))
    assert np.array_equal(got_p, ref_p), "%s: position ids differ at %s" % (label, np.argwhere(got_p != ref_p)[0])
    bad = np.argwhere(got_m != ref_m)
    assert bad.size == 0, "%s: mask differs at %d places, first %s" % (label, len(bad), bad[0].tolist())
    print("[tree-mask parity] %s ok (B=%d, N=%d)" % (label, B, parents.shape[-1]), flush=True)


SIZES = [1, 2, 31, 32, 33, 65, 255, 256, 257, 700, 1024]


@pytest.mark.parametrize("N", SIZES)
def test_tree_mask_parity_sizes(dev, N):
    inp = make_tree_mask("n%d" % N, 5, N, seed=N)
    _check(inp.parents, inp.offsets, dev, "bool N=%d" % N)
    _check(inp.parents, inp.offsets, dev, "packed N=%d" % N, packed=True)


def test_tree_mask_misaligned_output_and_shared_tree(dev):
    inp = make_tree_mask("odd", 7, 67, seed=3)
    _check(inp.parents, inp.offsets, dev, "misaligned", misalign=True)
    _check(inp.parents[0], inp.offsets, dev, "shared tree", shared_B=7)
    _check(inp.parents[0], None, dev, "shared tree, no offsets", shared_B=3)


def test_tree_mask_deep_chain_and_wide_star(dev):
    chain = make_tree_mask("chain", 2, 1024, seed=4, chain=True)
    _check(chain.parents, chain.offsets, dev, "chain 1024")
    star = np.zeros((2, 600), np.int32)
    star[:, 0] = -1
    _check(star, np.array([0, 9], np.int32), dev, "star 600")


def test_tree_mask_invalid_trees(dev):
    inp = make_tree_mask("bad", 5, 40, seed=5)
    par = inp.parents.copy()
    par[1, 0] = 0          # root without -1
    par[2, 10] = 10        # its own parent
    par[3, 7] = 30         # a parent after its child
    par[4, 5] = -1         # a second root
    _check(par, inp.offsets, dev, "invalid")
    got_m, got_p = _run(par, inp.offsets, dev)
    assert np.all(got_p[1:] == -1) and not got_m[1:].any() and np.all(got_p[0] >= 0)


def test_tree_mask_named_workload_full_size(dev):
    inp = workloads.make_extra("tree_mask_b256")
    _check(inp.parents, inp.offsets, dev, "tree_mask_b256")
    _check(inp.parents, inp.offsets, dev, "tree_mask_b256 packed", packed=True)
