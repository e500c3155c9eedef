"""GPU tests of the library's calls captured in a HIP graph (torch.cuda.CUDAGraph), the form the benchmark times.

Each graph is replayed several times.  Before every replay the program overwrites the graph's outputs and
workspace with eager fills, runs another eager call of the library on other inputs, and synchronises; every
replay's results must then be bit-identical to those of the same call made eagerly (same kernels, same plan,
a fixed reduction order).  The library records no memset or allocation into the graph: its kernels write
every output element and every workspace byte they later read.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si

pytestmark = pytest.mark.gpu

kdv = pytest.importorskip("speculative_decoding_tree_parent_amd")

REPLAYS = 4


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _b16(arrs):
    return torch.from_numpy(np.ascontiguousarray(np.concatenate(arrs)).view(np.int16)).cuda()


def _capture(call):
    """Warm the call up on a side stream, then capture it into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    return g


def _replay_and_check(g, bufs, refs, clobber, other_call):
    for rep in range(REPLAYS):
        for b in bufs:
            b.fill_(clobber[rep % len(clobber)])
        other_call()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, b, r in refs:
            assert torch.equal(b, r), f"replay {rep}: {name} differs from the eager call"


def test_tree_verify_graph_replays():
    inp = si.kimi(L=5553, T=15, seed=11, dist="unit")
    oth = si.kimi(L=1000, T=9, seed=12, dist="unit")
    dev, dev2 = si.to_device(inp), si.to_device(oth)
    dims = kdv.make_dims(**inp.dims())
    T, H, Dv = inp.T, inp.H, inp.dims()["v_head_dim"]
    out = torch.empty((T, H, Dv), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    mask = torch.empty((T, (T + 31) // 32), dtype=torch.int32, device="cuda")
    status = torch.empty((1,), dtype=torch.int32, device="cuda")
    ws = torch.zeros((kdv.verify_workspace_bytes(dims, T, inp.L),), dtype=torch.uint8, device="cuda")

    def call():
        kdv.verify_mla_attn_tree(dims, dev["q_nope"], dev["q_rope"], dev["w_uk"], dev["w_uv"], dev["c_kv"],
                                 dev["k_pe"], dev["page_table"], inp.L, dev["parent"], mask=mask, status=status,
                                 out=out, lse=lse, workspace=ws)

    def other_call():
        kdv.verify_mla_attn_tree(dims, dev2["q_nope"], dev2["q_rope"], dev2["w_uk"], dev2["w_uv"], dev2["c_kv"],
                                 dev2["k_pe"], dev2["page_table"], oth.L, dev2["parent"], lse=torch.empty(
                                     (oth.T, oth.H), dtype=torch.float32, device="cuda"))

    call()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    refs = [(n, b, b.clone()) for n, b in (("out", out), ("lse", lse), ("mask", mask), ("status", status))]
    g = _capture(call)
    _replay_and_check(g, [out, lse, mask, status, ws], refs, clobber=[0, 255, 7], other_call=other_call)


def test_batched_verify_graph_replays():
    Ls, Ts = [5553, 5553, 5553, 100], [15, 15, 15, 9]
    reqs = si.batch_inputs(si.KIMI_DIMS, Ls, Ts, seed=13, dist="unit")
    r0 = reqs[0]
    dims = kdv.make_dims(**r0.dims())
    dev = dict(q_nope=_b16([r.q_nope for r in reqs]), q_rope=_b16([r.q_rope for r in reqs]),
               w_uk=_b16([r0.w_uk]), w_uv=_b16([r0.w_uv]), c_kv=_b16([r0.c_kv]), k_pe=_b16([r0.k_pe]),
               page_table=torch.from_numpy(np.concatenate([r.page_table for r in reqs]).astype(np.int32)).cuda())
    mask, status = kdv.build_tree_masks([torch.from_numpy(r.parent.astype(np.int32)).cuda() for r in reqs])
    n, H, Dv = sum(Ts), r0.H, r0.dims()["v_head_dim"]
    out = torch.empty((n, H, Dv), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((n, H), dtype=torch.float32, device="cuda")
    ws = torch.zeros((kdv.verify_batch_workspace_bytes(dims, Ls, Ts),), dtype=torch.uint8, device="cuda")
    # the other call: one request of the same batch through the single-request path, into its own buffers
    one = si.to_device(reqs[3])

    def call():
        kdv.verify_mla_attn_batch(dims, dev["q_nope"], dev["q_rope"], dev["w_uk"], dev["w_uv"], dev["c_kv"],
                                  dev["k_pe"], dev["page_table"], Ls, Ts, mask, out=out, lse=lse, workspace=ws)

    def other_call():
        kdv.verify_mla_attn_tree(dims, one["q_nope"], one["q_rope"], one["w_uk"], one["w_uv"], one["c_kv"],
                                 one["k_pe"], one["page_table"], reqs[3].L, one["parent"])

    call()
    torch.cuda.synchronize()
    assert np.all(status.cpu().numpy() == 0)
    refs = [(n_, b, b.clone()) for n_, b in (("out", out), ("lse", lse))]
    g = _capture(call)
    _replay_and_check(g, [out, lse, ws], refs, clobber=[0, 3, 255], other_call=other_call)


def test_verify_step_graph_replays():
    """The whole verify step in one graph, device arrays only: best-first tree builder -> verify with its own
    ancestor mask -> greedy acceptance, with the built tree feeding the other two calls on the device."""
    T = 15
    logp, tok = si.draft_topk(7, 16, 4)
    rng = np.random.default_rng(9)
    inp = si.kimi(L=300, T=T, seed=5, dist="unit")
    d = si.to_device(inp)
    dims = kdv.make_dims(**inp.dims())
    lp, tk = torch.from_numpy(logp).cuda(), torch.from_numpy(tok).cuda()
    root = torch.tensor([42], dtype=torch.int32, device="cuda")
    # target predictions that mostly follow a drafted child (tree from the oracle's builder), so that acceptance
    # walks several levels
    b_parent, b_tokens, _ = oracle.build_draft_tree(logp, tok, T, 42)
    pr = rng.integers(0, 1 << 16, size=T).astype(np.int32)
    for p in range(T):
        kids = [c for c in range(T) if b_parent[c] == p]
        if kids and rng.random() < 0.9:
            pr[p] = b_tokens[kids[int(rng.integers(0, len(kids)))]]
    pred = torch.from_numpy(pr).cuda()
    res = {}

    def call():
        parent, tokens, n_nodes = kdv.build_draft_tree(lp, tk, T, root)
        out, _, mask, mstatus = kdv.verify_mla_attn_tree(dims, d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"],
                                                         d["c_kv"], d["k_pe"], d["page_table"], inp.L, parent)
        path, n_path, nxt, astatus = kdv.tree_accept(parent, tokens, pred)
        res.update(parent=parent, tokens=tokens, n_nodes=n_nodes, out=out, mask=mask, mstatus=mstatus, path=path,
                   n_path=n_path, next_token=nxt, astatus=astatus)

    call()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in res.items()}
    assert int(ref["n_nodes"].item()) == T and int(ref["mstatus"].item()) == 0 and int(ref["astatus"].item()) == 0
    g = _capture(call)
    n = int(ref["n_path"].item())
    for rep in range(REPLAYS):
        for v in res.values():
            v.fill_([0, 255, 7][rep % 3])
        kdv.build_tree_mask(d["parent"])  # other eager work of the library between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in res.items():
            if k == "path":  # entries past n_path are not part of the result
                assert torch.equal(v[:n], ref[k][:n]), f"replay {rep}: path differs from the eager call"
            else:
                assert torch.equal(v, ref[k]), f"replay {rep}: {k} differs from the eager call"
