"""Helpers shared by the GPU parity tests: upload seeded inputs, run the HIP
path through the C ABI binding, run the oracle on the same arrays, compare."""
import sys

import numpy as np

import oracle
import workloads as W

TOL_PROB = 1e-5  # probabilities and residual masses, absolute (fp32 outputs)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    import torch
    return torch.device("cuda:0")


def to_dev(a, offset_elems=0):
    """numpy -> torch cuda.  bf16 arrays (uint16 bits) travel as int16.
    offset_elems > 0 places the tensor that many elements past an allocation
    start, so that its base is element- but not 16-byte aligned."""
    import torch
    a = np.ascontiguousarray(a)
    src = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
    if offset_elems == 0:
        return src.to(dev())
    flat = torch.empty(src.numel() + offset_elems, dtype=src.dtype, device=dev())
    view = flat[offset_elems:].view(src.shape)
    view.copy_(src.to(dev()))
    return view


def host(t):
    return t.detach().cpu().numpy()


def run_workload(w, offset=0, **kw):
    import speculative_decoding_verification_sample_amd as sv
    if w.kind == "sample":
        return sv.verify_sample(to_dev(w.target, offset), to_dev(w.draft, offset), to_dev(w.tokens),
                                to_dev(w.u_accept), to_dev(w.u_sample), w.temperature, w.top_p, **kw)
    if w.kind == "greedy":
        return sv.verify_greedy(to_dev(w.target, offset), to_dev(w.tokens), **kw)
    return sv.verify_tree(to_dev(w.target, offset), to_dev(w.parents), to_dev(w.tokens),
                          to_dev(w.anc_mask), **kw)


def check_sample(w, got, ref, requests=None):
    """Exact on unflagged requests, probabilities within 1e-5, invariants on
    every request.  `requests`: indices into the workload the oracle ran on
    (default all).  Returns the number of flagged requests."""
    idx = np.arange(w.B) if requests is None else np.asarray(requests)
    acc = host(got["accepted"])[idx]
    tok = host(got["tokens"])[idx]
    flags = ref["flags"]
    flagged = (flags & oracle.FLAG_AMBIGUOUS) != 0
    ok = ~flagged
    bad = ok & ((acc != ref["accepted"]) | (tok != ref["tokens"]).any(axis=1))
    if bad.any():
        b = int(np.nonzero(bad)[0][0])
        raise AssertionError(
            f"request {idx[b]}: gpu n={acc[b]} tokens={tok[b].tolist()} vs oracle "
            f"n={ref['accepted'][b]} tokens={ref['tokens'][b].tolist()} flags={flags[b]}")
    if "p" in got:
        edge = (flags & (oracle.FLAG_TOPP_EDGE | oracle.FLAG_TOPP_NEAR)) != 0
        p = host(got["p"])[idx]
        q = host(got["q"])[idx]
        np.testing.assert_allclose(p[~edge], ref["p"][~edge], atol=TOL_PROB, rtol=0)
        np.testing.assert_allclose(q[~edge], ref["q"][~edge], atol=TOL_PROB, rtol=0)
        same = (acc == ref["accepted"]) & ~edge
        S = host(got["residual_mass"])[idx]
        np.testing.assert_allclose(S[same], ref["S"][same], atol=TOL_PROB, rtol=0)
    # invariants on every request, flagged or not
    K, V = w.K, w.V
    drafts = w.tokens[idx]
    for r in range(len(idx)):
        n = int(acc[r])
        assert 0 <= n <= K
        assert (tok[r, :n] == drafts[r, :n]).all()
        assert 0 <= tok[r, n] < V
        assert (tok[r, n + 1:] == -1).all()
        if n < K and not (flags[r] & oracle.FLAG_FALLBACK) and acc[r] == ref["accepted"][r]:
            assert tok[r, n] != drafts[r, n], "replacement equals the rejected draft"
    return int(flagged.sum())


def check_greedy(w, got, ref):
    np.testing.assert_array_equal(host(got["accepted"]), ref["accepted"])
    np.testing.assert_array_equal(host(got["tokens"]), ref["tokens"])


def check_tree(w, got, ref):
    np.testing.assert_array_equal(host(got["path_len"]), ref["path_len"])
    np.testing.assert_array_equal(host(got["path_nodes"]), ref["path_nodes"])
    np.testing.assert_array_equal(host(got["tokens"]), ref["tokens"])


def subset(w, requests):
    """The same workload restricted to some requests (for oracle sampling)."""
    return W.subset(w, requests)
