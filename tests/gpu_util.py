"""Helpers shared by the GPU tests: move generated inputs to the device, run
the library, and compare with the oracle to the agreed bar."""
from __future__ import annotations

import numpy as np

import oracle

TOL_FP = 1e-5          # accept probabilities, log-normalizers, residual mass
NEAR_TIE = 1e-6        # relative top-two gap of the oracle's Gumbel-max scores


def to_dev(a, torch, dev):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


def run_sample(inp, torch, dev, diag=True, workspace=None, seed=None, offset=None, tiling=None, stream=None):
    import rejection_sampling_verify_amd as rsv
    t = to_dev(inp.target, torch, dev)
    d = to_dev(inp.draft, torch, dev)
    ids = torch.from_numpy(inp.draft_ids).to(dev)
    temp = torch.from_numpy(inp.temperature).to(dev)
    B, G = inp.draft_ids.shape
    dg = None
    if diag:
        dg = {"accept_prob": torch.full((B, G), float("nan"), dtype=torch.float32, device=dev),
              "logz_target": torch.full((B, G), float("nan"), dtype=torch.float32, device=dev),
              "logz_draft": torch.full((B, G), float("nan"), dtype=torch.float32, device=dev),
              "residual_mass": torch.full((B,), float("nan"), dtype=torch.float32, device=dev)}
    tok, n = rsv.spec_verify_sample(t, d, ids, temp, seed=inp.seed if seed is None else seed,
                                    offset=inp.offset if offset is None else offset, diag=dg,
                                    workspace=workspace, V=inp.meta.get("V", inp.V), tiling=tiling, stream=stream)
    torch.cuda.synchronize()
    out = {"tokens": tok.cpu().numpy(), "n": n.cpu().numpy()}
    if dg:
        for k, v in dg.items():
            out[k] = v.cpu().numpy().astype(np.float64)
    return out


def oracle_sample(inp, seed=None, offset=None):
    return oracle.verify_sample(inp.target, inp.draft, inp.draft_ids, inp.temperature,
                                seed=inp.seed if seed is None else seed,
                                offset=inp.offset if offset is None else offset, V=inp.meta.get("V", inp.V))


def compare_chain(got, ref, check_diag=True, label="", allow_excused=0):
    """Ids and lengths bit-exact except sequences the oracle marks as a Gumbel
    near-tie or an accept knife-edge; fp32 diagnostics within TOL_FP. At the
    fixed seeds of the tests no sequence is excused: the number excused must
    equal allow_excused (0 unless a case states otherwise). Returns a summary
    dict (the excused sequences)."""
    B = ref["n"].shape[0]
    excused = []
    for b in range(B):
        same = (got["n"][b] == ref["n"][b]) and np.array_equal(got["tokens"][b], ref["tokens"][b])
        if same:
            continue
        near_tie = ref["top_gap"][b] < NEAR_TIE
        knife = bool(ref["flags"][b] & oracle.FLAG_KNIFE_EDGE)
        assert near_tie or knife, (
            "%s sequence %d differs: gpu n=%d tokens=%s, oracle n=%d tokens=%s (gap %.3g, flags %d)"
            % (label, b, got["n"][b], got["tokens"][b].tolist(), ref["n"][b], ref["tokens"][b].tolist(),
               ref["top_gap"][b], ref["flags"][b]))
        excused.append(b)
    assert len(excused) == allow_excused, "%s: %d sequences excused (%s), expected %d" % (
        label, len(excused), excused, allow_excused)
    summary = {"B": B, "excused": excused}
    if check_diag and "accept_prob" in got:
        for key in ("accept_prob", "logz_target", "logz_draft"):
            g, r = got[key], ref[key]
            both_nan = np.isnan(g) & np.isnan(r)
            assert np.array_equal(np.isnan(g), np.isnan(r)), "%s %s NaN pattern differs" % (label, key)
            err = np.abs(np.where(both_nan, 0.0, g - r))
            assert err.max(initial=0.0) <= TOL_FP, "%s %s max error %.3g" % (label, key, err.max())
            summary[key + "_maxerr"] = float(err.max(initial=0.0))
        g, r = got["residual_mass"], ref["residual_mass"]
        ok = np.isnan(r) == np.isnan(g)
        for b in np.nonzero(~ok)[0]:
            assert b in excused, "%s residual_mass NaN pattern differs at %d" % (label, b)
        m = ~np.isnan(r) & ~np.isnan(g)
        m[excused] = False
        err = np.abs(g[m] - r[m])
        assert err.max(initial=0.0) <= TOL_FP, "%s residual_mass max error %.3g" % (label, err.max(initial=0.0))
        summary["residual_mass_maxerr"] = float(err.max(initial=0.0))
    return summary
