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


def variants(ref, r):
    """The outcomes the oracle accepts for request r (an index into `ref`):
    the defined one and, where a row's nucleus edge lies within 1e-6 of
    top_p, the request with that row's cut moved by one tie group.  Each is
    (n, token, p[K], q[K], S)."""
    n = int(ref["accepted"][r])
    out = [(n, int(ref["tokens"][r, n]), ref["p"][r], ref["q"][r], float(ref["S"][r]))]
    if "alt_n" in ref:
        an = ref["alt_n"][r]
        for row, s in zip(*np.nonzero(an >= 0)):
            out.append((int(an[row, s]), int(ref["alt_token"][r, row, s]),
                        ref["alt_p"][r, row, s], ref["alt_q"][r, row, s],
                        float(ref["alt_S"][r, row, s])))
    return out


# a uniform within 1e-6 relative of its accept threshold or CDF step, or a
# residual mass near the level below which the draw falls back to p'
EXCLUDED = oracle.FLAG_ACCEPT_NEAR | oracle.FLAG_CDF_NEAR | oracle.FLAG_S_NEAR


def flag_counts(flags):
    """Requests per oracle flag, and the requests left out of the exact
    comparison (EXCLUDED)."""
    f = np.asarray(flags)
    return {"accept_near": int(((f & oracle.FLAG_ACCEPT_NEAR) != 0).sum()),
            "cdf_near": int(((f & oracle.FLAG_CDF_NEAR) != 0).sum()),
            "s_near": int(((f & oracle.FLAG_S_NEAR) != 0).sum()),
            "topp_near": int(((f & oracle.FLAG_TOPP_NEAR) != 0).sum()),
            "topp_edge": int(((f & oracle.FLAG_TOPP_EDGE) != 0).sum()),
            "excluded": int(((f & EXCLUDED) != 0).sum()),
            "requests": int(f.size)}


def check_sample(w, got, ref, requests=None):
    """The GPU's outcome against the oracle's, request by request.
      - accepted length and emitted token: equal to the defined outcome, or
        (a nucleus edge within 1e-6 of top_p) to one of the oracle's
        alternatives; requests whose uniform lies within 1e-6 relative of its
        threshold or CDF step, or whose residual mass lies near the level
        where the draw falls back to p', are left out and counted;
      - p'(x_i), q'(x_i): within 1e-5 of the defined or an alternative value,
        on every request;
      - S: within 1e-5 of the S of a variant with the GPU's accepted length;
      - invariants on every request.
    `requests`: indices into the workload the oracle ran on (default all).
    Returns flag_counts of the requests compared."""
    idx = np.arange(w.B) if requests is None else np.asarray(requests)
    acc = host(got["accepted"])[idx]
    tok = host(got["tokens"])[idx]
    flags = ref["flags"]
    excluded = (flags & EXCLUDED) != 0
    have_p = "p" in got
    if have_p:
        p = host(got["p"])[idx]
        q = host(got["q"])[idx]
        S = host(got["residual_mass"])[idx]
    for r in range(len(idx)):
        n = int(acc[r])
        vs = variants(ref, r)
        desc = (f"request {idx[r]}: gpu n={n} tokens={tok[r].tolist()} vs oracle "
                f"n={ref['accepted'][r]} tokens={ref['tokens'][r].tolist()} flags={flags[r]} "
                f"alternatives={[(v[0], v[1]) for v in vs[1:]]}")
        if not excluded[r]:
            assert 0 <= n <= w.K and any(n == v[0] and int(tok[r, n]) == v[1] for v in vs), desc
        if have_p:
            for i in range(w.K):
                err_p = min(abs(float(p[r, i]) - float(v[2][i])) for v in vs)
                err_q = min(abs(float(q[r, i]) - float(v[3][i])) for v in vs)
                assert err_p <= TOL_PROB and err_q <= TOL_PROB, \
                    f"{desc}: position {i} p={p[r, i]} q={q[r, i]} (err {err_p:.2e}, {err_q:.2e})"
            same_n = [v[4] for v in vs if v[0] == n]
            if same_n:
                err_S = min(abs(float(S[r]) - s) for s in same_n)
                assert err_S <= TOL_PROB, f"{desc}: S={S[r]} vs {same_n} (err {err_S:.2e})"
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
    return flag_counts(flags)


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


def oracle_parallel(w, requests=None, threads=None):
    """The oracle on `requests` of workload w (default all), one request per
    call, fanned out over host threads (the oracle's C code runs outside the
    interpreter lock).  Returns the oracle's fields for those requests, in
    their order."""
    import concurrent.futures as cf
    import os
    idx = np.arange(w.B) if requests is None else np.asarray(requests)
    n = threads or max(1, min(16, len(os.sched_getaffinity(0)), len(idx)))
    with cf.ThreadPoolExecutor(n) as ex:
        parts = list(ex.map(lambda r: oracle.verify_workload(W.subset(w, [r])), idx.tolist()))
    return {k: np.concatenate([p[k] for p in parts], axis=0) for k in parts[0]}
