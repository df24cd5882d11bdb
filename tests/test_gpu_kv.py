"""GPU parity of the KV-cache rollback against the CPU oracle, through the C
ABI. Byte work, so the bar is bit-exact: every byte of K and V (moved rows,
untouched prefix, untouched tail) and every new cache length."""
import numpy as np
import pytest

import workloads
from oracle import kv as okv
from workloads import make_kv_rollback

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verify_amd as rsv
    rsv.lib()
    return torch.device("cuda:0")


def _run(inp, dev, with_v=True, root=None, path=None, path_len=None):
    import rejection_sampling_verify_amd as rsv
    root = inp.root if root is None else root
    path = inp.path if path is None else path
    path_len = inp.path_len if path_len is None else path_len
    k_host = inp.cache_host(0)
    v_host = inp.cache_host(1) if with_v else None
    k = torch.from_numpy(k_host).to(dev)
    v = torch.from_numpy(v_host).to(dev) if with_v else None
    n = rsv.sv_kv_rollback(k, v, torch.from_numpy(root).to(dev), torch.from_numpy(path).to(dev),
                           torch.from_numpy(path_len).to(dev))
    torch.cuda.synchronize()
    got = {"k": k.cpu().numpy(), "len": n.cpu().numpy()}
    ref_k, ref_len = okv.kv_rollback(k_host, root, path, path_len)
    ref = {"k": ref_k, "len": ref_len}
    if with_v:
        got["v"] = v.cpu().numpy()
        ref["v"] = okv.kv_rollback(v_host, root, path, path_len)[0]
    return got, ref


def _assert_equal(got, ref, label):
    assert np.array_equal(got["len"], ref["len"]), (label, got["len"], ref["len"])
    for key in ("k", "v"):
        if key in ref:
            bad = np.argwhere(got[key] != ref[key])
            assert bad.size == 0, "%s %s differs at %d places, first (l, b, h, s, d) %s" % (
                label, key, len(bad), bad[0].tolist())
    print("[kv parity] %s ok: lengths %s" % (label, ref["len"][:12].tolist()), flush=True)


CASES = {
    # name: (L, B, H, S, D, elem_bytes, kind, P)
    "bf16_tree": (2, 9, 3, 96, 128, 2, "tree", None),
    "fp32_tree_row160": (2, 7, 2, 80, 40, 4, "tree", None),   # 10 vectors a row: chunks end mid-row
    "u8_tree": (1, 6, 4, 90, 128, 1, "tree", None),
    "bf16_row16": (1, 5, 2, 70, 8, 2, "tree", None),           # one vector a row
    "bf16_chain": (2, 8, 2, 64, 64, 2, "chain", 9),
    "bf16_sparse_long": (1, 6, 2, 2048, 128, 2, "sparse", 1024),
    "fp32_sparse_wide": (1, 4, 1, 1500, 1024, 4, "sparse", 700),  # 4 KiB rows
}


def _tree():
    return workloads.tree_c5_structure()[0]


@pytest.mark.parametrize("name", sorted(CASES))
def test_kv_rollback_parity(dev, name):
    L, B, H, S, D, es, kind, P = CASES[name]
    kw = dict(root_lo=0)
    if kind == "sparse":
        kw["root_hi"] = S - P - 5
    inp = make_kv_rollback(name, L, B, H, S, D, elem_bytes=es, seed=len(name), kind=kind,
                           parents=_tree() if kind == "tree" else None, P=P, **kw)
    got, ref = _run(inp, dev)
    _assert_equal(got, ref, name)
    if kind == "chain":
        assert np.array_equal(got["k"], inp.cache_host(0))  # a chain step moves nothing
    else:
        assert inp.moved_rows().sum() > 0


def test_kv_rollback_k_only(dev):
    inp = make_kv_rollback("k_only", 2, 6, 2, 80, 64, elem_bytes=2, seed=31, kind="tree", parents=_tree())
    got, ref = _run(inp, dev, with_v=False)
    _assert_equal(got, ref, "k only")


def test_kv_rollback_invalid_paths_left_alone(dev):
    """Invalid paths give length -1 and leave their sequence untouched; the
    valid sequences of the same call still roll back."""
    B, S = 8, 96
    inp = make_kv_rollback("invalid", 2, B, 2, S, 64, elem_bytes=2, seed=32, kind="tree", parents=_tree())
    path = inp.path.copy()
    plen = inp.path_len.copy()
    root = inp.root.copy()
    path[1, :3] = [1, 2, 3]; plen[1] = 3        # root not first
    path[2, :3] = [0, 5, 5]; plen[2] = 3        # not increasing
    path[3, :3] = [0, 9, 4]; plen[3] = 3        # decreasing
    plen[4] = 0                                 # empty
    root[5] = S - 2; path[5, :2] = [0, 3]; plen[5] = 2  # past the end
    plen[6] = path.shape[1] + 1                 # longer than the path array
    root[7] = -1                                # negative root
    got, ref = _run(inp, dev, root=root, path=path, path_len=plen)
    _assert_equal(got, ref, "invalid paths")
    assert list(got["len"][1:]) == [-1] * 7 and got["len"][0] >= 1


def test_kv_rollback_named_workload_full_size(dev):
    """The resident 32-layer workload (K and V of 8.6 GB each): new lengths
    for every sequence, and sampled (layer, sequence, head) slabs compared with
    the oracle on the same slab read back before the call."""
    import rejection_sampling_verify_amd as rsv
    inp = workloads.make_extra("kv_rollback_bf16_llama")
    L, B, H, S, D = inp.shape
    k = workloads.fill_kv_device(torch, torch.empty(inp.shape, dtype=torch.int16, device=dev), inp.seed, 0)
    v = workloads.fill_kv_device(torch, torch.empty(inp.shape, dtype=torch.int16, device=dev), inp.seed, 1)
    rng = np.random.default_rng(5)
    slabs = [(0, 0, 0), (L - 1, B - 1, H - 1)] + [tuple(int(x) for x in (rng.integers(L), rng.integers(B),
                                                                        rng.integers(H))) for _ in range(14)]
    before = [(k[l, b, h].cpu().numpy(), v[l, b, h].cpu().numpy()) for l, b, h in slabs]
    n = rsv.sv_kv_rollback(k, v, torch.from_numpy(inp.root).to(dev), torch.from_numpy(inp.path).to(dev),
                           torch.from_numpy(inp.path_len).to(dev))
    torch.cuda.synchronize()
    _, ref_len = okv.kv_rollback(np.zeros((1, B, 1, S, 1), np.int16), inp.root, inp.path, inp.path_len)
    assert np.array_equal(n.cpu().numpy(), ref_len)
    for (l, b, h), (k0, v0) in zip(slabs, before):
        for name, t, x0 in (("k", k, k0), ("v", v, v0)):
            ref, _ = okv.kv_rollback(x0[None, None, None], inp.root[b:b + 1], inp.path[b:b + 1],
                                     inp.path_len[b:b + 1])
            assert np.array_equal(t[l, b, h].cpu().numpy(), ref[0, 0, 0]), (name, l, b, h)
    print("[kv parity] full size: %d slabs ok, moved rows per layer-head %d" % (len(slabs),
                                                                            int(inp.moved_rows().sum())),
          flush=True)


def test_kv_rollback_per_layer_tensors(dev):
    """Caches kept as one tensor per layer (the page's key_cache[l]): the same
    result as the oracle on the stacked layers."""
    import rejection_sampling_verify_amd as rsv
    inp = make_kv_rollback("layers", 3, 7, 2, 96, 64, elem_bytes=2, seed=33, kind="tree", parents=_tree())
    k_host, v_host = inp.cache_host(0), inp.cache_host(1)
    ks = [torch.from_numpy(k_host[l].copy()).to(dev) for l in range(3)]
    vs = [torch.from_numpy(v_host[l].copy()).to(dev) for l in range(3)]
    n = rsv.sv_kv_rollback_layers(ks, vs, torch.from_numpy(inp.root).to(dev), torch.from_numpy(inp.path).to(dev),
                                  torch.from_numpy(inp.path_len).to(dev))
    torch.cuda.synchronize()
    ref_k, ref_len = okv.kv_rollback(k_host, inp.root, inp.path, inp.path_len)
    ref_v, _ = okv.kv_rollback(v_host, inp.root, inp.path, inp.path_len)
    assert np.array_equal(n.cpu().numpy(), ref_len)
    assert np.array_equal(np.stack([x.cpu().numpy() for x in ks]), ref_k)
    assert np.array_equal(np.stack([x.cpu().numpy() for x in vs]), ref_v)
    ks2 = [torch.from_numpy(k_host[l].copy()).to(dev) for l in range(3)]
    rsv.sv_kv_rollback_layers(ks2, None, torch.from_numpy(inp.root).to(dev), torch.from_numpy(inp.path).to(dev),
                              torch.from_numpy(inp.path_len).to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(np.stack([x.cpu().numpy() for x in ks2]), ref_k)
    print("[kv parity] per-layer tensors ok", flush=True)
