"""The rows composed as one decoding step uses them, on the GPU through the C
ABI, against the oracle composed the same way:

- chain: n-gram drafts -> one-hot verify -> KV rollback to keep = T + n;
- tree: tree mask / position ids -> sampled tree verify -> KV rollback to the
  accepted path.

Each GPU stage consumes the previous GPU stage's outputs and each oracle
stage the previous oracle stage's, so a mismatch anywhere shows downstream.
The seeds are ones where the oracle flags no near-tie or knife-edge, so every
stage is compared bit for bit."""
import numpy as np
import pytest

import oracle
from oracle import kv as okv
from oracle import ngram as og
from oracle import trees
from workloads import (bf16_to_f32, make_chain, make_kv_rollback, make_ngram, make_tree_mask, make_tree_sample,
                       round_bf16)

from gpu_util import NEAR_TIE, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verify_amd as rsv
    rsv.lib()
    return torch.device("cuda:0")


def _caches(B, S, seed):
    kv = make_kv_rollback("pipe_kv", 2, B, 2, S, 64, elem_bytes=2, seed=seed, kind="chain", P=2)
    return kv.cache_host(0), kv.cache_host(1)


def test_chain_step_drafter_verify_rollback(dev):
    import rejection_sampling_verify_amd as rsv
    B, V, gamma = 24, 3000, 5
    hist = make_ngram("pipe", B, V, (64, 900), ngram=2, gamma=gamma, pad=True, seed=41, stride=904)
    # drafter
    d_gpu, c_gpu, _ = rsv.sv_ngram_draft(torch.from_numpy(hist.tokens).to(dev),
                                         torch.from_numpy(hist.lengths).to(dev), 2, gamma, True)
    d_ref, c_ref, _ = og.ngram_draft(hist.tokens, hist.lengths, 2, gamma, True)
    assert np.array_equal(d_gpu.cpu().numpy(), d_ref) and np.array_equal(c_gpu.cpu().numpy(), c_ref)
    # target logits that favour the drafted tokens at some positions (so both
    # early and late rejections occur)
    inp = make_chain("pipe_target", B, gamma, V, bf16=True, seed=42, target_sigma=2.0, one_hot=True,
                     temperatures=(0.0, 0.8, 1.0))
    vals = bf16_to_f32(inp.target)
    rng = np.random.default_rng(43)
    for b in range(B):
        for i in range(gamma):
            if rng.random() < 0.8:
                vals[b, i, d_ref[b, i]] += 14.0
    inp.target = round_bf16(vals)
    ref = oracle.verify_sample(inp.target, None, d_ref, inp.temperature, seed=9, offset=2)
    assert np.all(ref["top_gap"] >= NEAR_TIE) and not np.any(ref["flags"] & oracle.FLAG_KNIFE_EDGE)
    tok, n = rsv.spec_verify_sample(to_dev(inp.target, torch, dev), None, d_gpu, torch.from_numpy(inp.temperature)
                                    .to(dev), seed=9, offset=2)
    n_gpu = n.cpu().numpy()
    assert np.array_equal(n_gpu, ref["n"]) and np.array_equal(tok.cpu().numpy(), ref["tokens"])
    assert len(set(n_gpu.tolist())) > 2
    # rollback: the verify pass wrote positions T - 1 (the last committed
    # token) .. T - 1 + gamma; keep T + n of them
    S = 1024
    k_host, v_host = _caches(B, S, 44)
    root = (hist.lengths - 1).astype(np.int32)
    path = np.full((B, gamma + 1), -1, np.int32)
    for b in range(B):
        path[b, :ref["n"][b] + 1] = np.arange(ref["n"][b] + 1)
    k, v = torch.from_numpy(k_host).to(dev), torch.from_numpy(v_host).to(dev)
    path_gpu = torch.full((B, gamma + 1), -1, dtype=torch.int32, device=dev)
    ar = torch.arange(gamma + 1, device=dev, dtype=torch.int32)
    path_gpu = torch.where(ar[None, :] <= n[:, None], ar[None, :].expand(B, -1), path_gpu).contiguous()
    new_len = rsv.sv_kv_rollback(k, v, torch.from_numpy(root).to(dev), path_gpu, (n + 1).to(torch.int32))
    ref_k, ref_len = okv.kv_rollback(k_host, root, path, ref["n"] + 1)
    assert np.array_equal(new_len.cpu().numpy(), hist.lengths + ref["n"])  # the page's keep = T + n
    assert np.array_equal(ref_len, hist.lengths + ref["n"])
    assert np.array_equal(k.cpu().numpy(), ref_k) and np.array_equal(v.cpu().numpy(), v_host)


def test_tree_step_mask_verify_rollback(dev):
    import rejection_sampling_verify_amd as rsv
    B, V = 16, 4000
    tm = make_tree_mask("pipe_tree", B, 21, seed=51, offset_range=(100, 800))
    parents = tm.parents[0]
    # mask and position ids for the packed forward pass (one shared tree)
    mask, pos = rsv.sv_tree_mask(torch.from_numpy(parents).to(dev), torch.from_numpy(tm.offsets).to(dev), B=B)
    ref_mask, ref_pos = trees.tree_attn_batch(parents, tm.offsets)
    assert np.array_equal(mask.cpu().numpy().astype(np.uint8), ref_mask)
    assert np.array_equal(pos.cpu().numpy(), ref_pos)
    depth = (ref_pos[0] - tm.offsets[0]).astype(np.int32)
    # sampled tree verify
    inp = make_tree_sample("pipe_tree", B, V, parents, depth, bf16=True, seed=52, temperatures=(0.7, 1.0),
                           target_sigma=2.0, zipf=0.0, draft_sigma=(0.3, 1.0))
    ref = oracle.verify_tree_sample(inp.target, inp.draft, parents, depth, inp.node_tokens, inp.temperature,
                                    inp.max_depth, seed=4, offset=1)
    assert np.all(ref["top_gap"] >= NEAR_TIE) and np.all(ref["margin"] >= 1e-4)
    path, plen, token = rsv.spec_verify_tree_sample(
        to_dev(inp.target, torch, dev), to_dev(inp.draft, torch, dev), torch.from_numpy(parents).to(dev),
        torch.from_numpy(depth).to(dev), torch.from_numpy(inp.node_tokens).to(dev),
        torch.from_numpy(inp.temperature).to(dev), inp.max_depth, seed=4, offset=1)
    assert np.array_equal(plen.cpu().numpy(), ref["path_len"]) and np.array_equal(path.cpu().numpy(), ref["path"])
    assert np.array_equal(token.cpu().numpy(), ref["token"])
    assert ref["path_len"].max() > 2
    # rollback to the accepted path: the root sits at its position id
    S = 1024
    k_host, v_host = _caches(B, S, 53)
    root = tm.offsets.astype(np.int32)
    k, v = torch.from_numpy(k_host).to(dev), torch.from_numpy(v_host).to(dev)
    new_len = rsv.sv_kv_rollback(k, v, torch.from_numpy(root).to(dev), path, plen)
    ref_k, ref_len = okv.kv_rollback(k_host, root, ref["path"], ref["path_len"])
    ref_v, _ = okv.kv_rollback(v_host, root, ref["path"], ref["path_len"])
    assert np.array_equal(new_len.cpu().numpy(), ref_len) and np.array_equal(ref_len, root + ref["path_len"])
    assert np.array_equal(k.cpu().numpy(), ref_k) and np.array_equal(v.cpu().numpy(), ref_v)
