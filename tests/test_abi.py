"""C ABI checks that need no GPU: the library loads, exports every function include/kdv.h declares,
and rejects bad arguments on the host with the documented status before anything is launched.

Argument errors are tested with fake (never dereferenced) addresses; KDV_SPLITS is set so that
workspace sizing does not query a device."""
import ctypes
import os
import re

import pytest

import speculative_decoding_tree_parent_amd as kdv

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kdv.h")

KIMI = dict(num_heads=64, qk_nope_dim=128, qk_rope_dim=64, kv_lora_rank=512, v_head_dim=128, sm_scale=192 ** -0.5)
TINY = dict(num_heads=4, qk_nope_dim=32, qk_rope_dim=16, kv_lora_rank=64, v_head_dim=32, sm_scale=48 ** -0.5)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kdv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(kdv.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(kdv.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code in range(-7, 1):
        s = kdv.kdv_status_string(code)
        assert s and "unknown" not in s
    assert "unknown" in kdv.kdv_status_string(-99)


@pytest.fixture
def fixed_splits(monkeypatch):
    monkeypatch.setenv("KDV_SPLITS", "4")


A = 0x10000  # fake, 64 KiB aligned, never dereferenced


def _call(dims, T=15, L=100, ws_bytes=1 << 40, **override):
    args = dict(q_nope=A, q_rope=A, w_uk=A, w_uv=A, c_kv=A, k_pe=A, pool_slots=1 << 20, page_table=A, L=L, T=T,
                mask=A, out=A, lse=None, workspace=A, workspace_bytes=ws_bytes, stream=None)
    args.update(override)
    return kdv.kdv_verify_mla_attn(dims, **args)


@pytest.mark.parametrize("field", ["q_nope", "q_rope", "w_uk", "w_uv", "c_kv", "k_pe", "page_table", "mask", "out",
                                   "workspace"])
def test_null_pointer_rejected(field, fixed_splits):
    assert _call(kdv.make_dims(**KIMI), **{field: None}) == kdv.KDV_ERR_NULL


@pytest.mark.parametrize("T,L", [(0, 10), (65, 10), (-1, 10), (15, -1)])
def test_bad_tree_or_prefix_rejected(T, L, fixed_splits):
    assert _call(kdv.make_dims(**KIMI), T=T, L=L) == kdv.KDV_ERR_SHAPE


@pytest.mark.parametrize("change", [dict(qk_nope_dim=64), dict(kv_lora_rank=256), dict(qk_rope_dim=32),
                                    dict(v_head_dim=64), dict(num_heads=0), dict(num_heads=129)])
def test_unsupported_dims_rejected(change, fixed_splits):
    d = dict(KIMI)
    d.update(change)
    assert _call(kdv.make_dims(**d)) == kdv.KDV_ERR_SHAPE
    assert kdv.kdv_verify_workspace_bytes(kdv.make_dims(**d), 15, 100) == 0


def test_bad_pool_rejected(fixed_splits):
    assert _call(kdv.make_dims(**KIMI), pool_slots=0) == kdv.KDV_ERR_SHAPE


@pytest.mark.parametrize("field,off", [("q_nope", 8), ("c_kv", 2), ("k_pe", 4), ("w_uk", 8), ("w_uv", 8),
                                       ("out", 8), ("workspace", 8), ("page_table", 2), ("mask", 1), ("lse", 2)])
def test_misaligned_rejected(field, off, fixed_splits):
    assert _call(kdv.make_dims(**KIMI), **{field: A + off}) == kdv.KDV_ERR_ALIGN


@pytest.mark.parametrize("dims", [KIMI, TINY])
def test_workspace_too_small_rejected(dims, fixed_splits):
    d = kdv.make_dims(**dims)
    need = kdv.kdv_verify_workspace_bytes(d, 15, 5553)
    assert need > 0
    assert _call(d, T=15, L=5553, ws_bytes=need - 1) == kdv.KDV_ERR_WORKSPACE
    assert _call(d, T=15, L=5553, ws_bytes=0) == kdv.KDV_ERR_WORKSPACE


def test_workspace_formula(fixed_splits):
    # header + q_cat (bf16) + split partials (bf16 O / l + fp32 (max, sum)), each region 256-byte aligned
    d = kdv.make_dims(**KIMI)
    T, L = 15, 5553
    S = kdv.kdv_verify_num_splits(d, T, L)
    assert S == 4
    M, Mp = T * 64, ((T * 64 + 63) // 64) * 64
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    expect = kdv.KDV_WS_HEADER + up(M * 576 * 2) + up(S * Mp * 512 * 2) + up(S * Mp * 8)
    assert kdv.kdv_verify_workspace_bytes(d, T, L) == expect


def test_split_count_never_exceeds_tiles(monkeypatch):
    monkeypatch.setenv("KDV_SPLITS", "1000")
    d = kdv.make_dims(**KIMI)
    assert kdv.kdv_verify_num_splits(d, 15, 0) == 1          # N = 15 -> one 64-row tile
    assert kdv.kdv_verify_num_splits(d, 15, 5553) == 87      # 5568 rows -> 87 tiles


def test_tree_mask_argument_errors():
    assert kdv.kdv_build_tree_mask(None, 7, A, None, None) == kdv.KDV_ERR_NULL
    assert kdv.kdv_build_tree_mask(A, 7, None, None, None) == kdv.KDV_ERR_NULL
    assert kdv.kdv_build_tree_mask(A, 0, A, None, None) == kdv.KDV_ERR_SHAPE
    assert kdv.kdv_build_tree_mask(A, 65, A, None, None) == kdv.KDV_ERR_SHAPE
    assert kdv.kdv_build_tree_mask(A + 2, 7, A, None, None) == kdv.KDV_ERR_ALIGN
    assert kdv.kdv_build_tree_mask(A, 7, A, A + 1, None) == kdv.KDV_ERR_ALIGN


def test_package_has_no_cpu_fallback():
    # the product package must not reach the oracle
    import inspect
    src = inspect.getsource(kdv)
    assert "oracle" not in src.replace("never by the product", "")


def test_tree_accept_argument_errors():
    ok = dict(parent=A, tokens=A, pred=A, T=15, path=A, n_path=A, next_token=A, status=None, stream=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return kdv.kdv_tree_accept(a["parent"], a["tokens"], a["pred"], a["T"], a["path"], a["n_path"],
                                   a["next_token"], a["status"], a["stream"])
    for field in ("parent", "tokens", "pred", "path", "n_path", "next_token"):
        assert call(**{field: None}) == kdv.KDV_ERR_NULL, field
    assert call(T=0) == kdv.KDV_ERR_SHAPE
    assert call(T=65) == kdv.KDV_ERR_SHAPE
    for field in ("parent", "tokens", "pred", "path", "n_path", "next_token", "status"):
        assert call(**{field: A + 2}) == kdv.KDV_ERR_ALIGN, field


def test_build_draft_tree_argument_errors():
    ok = dict(logp=A, tok=A, block=16, K=8, budget=32, root=A, parent=A, tokens=A, n=A)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return kdv.kdv_build_draft_tree(a["logp"], a["tok"], a["block"], a["K"], a["budget"], a["root"],
                                        a["parent"], a["tokens"], a["n"], None)
    for field in ("logp", "tok", "root", "parent", "tokens", "n"):
        assert call(**{field: None}) == kdv.KDV_ERR_NULL, field
    for bad in (dict(block=0), dict(block=64), dict(K=0), dict(K=65), dict(budget=0), dict(budget=65)):
        assert call(**bad) == kdv.KDV_ERR_SHAPE, bad
    for field in ("logp", "tok", "root", "parent", "tokens", "n"):
        assert call(**{field: A + 1}) == kdv.KDV_ERR_ALIGN, field


def _prefix(dims, L=100, T=15, ws_bytes=1 << 40, **override):
    args = dict(q_nope=A, q_rope=A, w_uk=A, w_uv=A, c_kv=A, k_pe=A, pool_slots=1 << 20, page_table=A, L=L, T=T,
                out=A, lse=A, workspace=A, workspace_bytes=ws_bytes, stream=None)
    args.update(override)
    return kdv.kdv_prefix_mla_attn(dims, **args)


@pytest.mark.parametrize("field", ["q_nope", "q_rope", "w_uk", "w_uv", "c_kv", "k_pe", "page_table", "out",
                                   "workspace"])
def test_prefix_null_pointer_rejected(field, fixed_splits):
    assert _prefix(kdv.make_dims(**KIMI), **{field: None}) == kdv.KDV_ERR_NULL


@pytest.mark.parametrize("T,L", [(15, 0), (15, -3), (0, 10), (65, 10)])
def test_prefix_bad_shape_rejected(T, L, fixed_splits):
    assert _prefix(kdv.make_dims(**KIMI), T=T, L=L) == kdv.KDV_ERR_SHAPE


@pytest.mark.parametrize("field,off", [("q_nope", 8), ("c_kv", 2), ("out", 8), ("workspace", 8), ("page_table", 2),
                                       ("lse", 2)])
def test_prefix_misaligned_rejected(field, off, fixed_splits):
    assert _prefix(kdv.make_dims(**KIMI), **{field: A + off}) == kdv.KDV_ERR_ALIGN


def test_prefix_workspace_too_small_rejected(fixed_splits):
    d = kdv.make_dims(**KIMI)
    assert kdv.kdv_verify_workspace_bytes(d, 15, 5553) > 0
    assert _prefix(d, T=15, L=5553, ws_bytes=0) == kdv.KDV_ERR_WORKSPACE
    assert _prefix(d, T=15, L=5553, ws_bytes=255) == kdv.KDV_ERR_WORKSPACE


def test_merge_argument_errors():
    ok = dict(out_a=A, lse_a=A, out_b=A, lse_b=A, rows=960, dv=128, out=A, lse=A)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return kdv.kdv_merge_attn_states(a["out_a"], a["lse_a"], a["out_b"], a["lse_b"], a["rows"], a["dv"],
                                         a["out"], a["lse"], None)
    for field in ("out_a", "lse_a", "out_b", "lse_b", "out"):
        assert call(**{field: None}) == kdv.KDV_ERR_NULL, field
    for bad in (dict(rows=0), dict(rows=-1), dict(dv=0), dict(dv=4), dict(dv=12), dict(dv=4104)):
        assert call(**bad) == kdv.KDV_ERR_SHAPE, bad
    for field, off in (("out_a", 8), ("out_b", 2), ("out", 8), ("lse_a", 2), ("lse_b", 1), ("lse", 2)):
        assert call(**{field: A + off}) == kdv.KDV_ERR_ALIGN, field


def _batch(dims, Ls, Ts, ws_bytes=1 << 40, C=None, **override):
    la, lp = kdv._host_i32(Ls)
    ta, tp = kdv._host_i32(Ts)
    args = dict(q_nope=A, q_rope=A, w_uk=A, w_uv=A, c_kv=A, k_pe=A, pool_slots=1 << 20, page_table=A, mask=A, out=A,
                lse=None, workspace=A, workspace_bytes=ws_bytes, stream=None)
    args.update(override)
    n = len(Ls) if C is None else C
    return kdv.kdv_verify_mla_attn_batch(dims, n, lp, tp, args["q_nope"], args["q_rope"], args["w_uk"],
                                         args["w_uv"], args["c_kv"], args["k_pe"], args["pool_slots"],
                                         args["page_table"], args["mask"], args["out"], args["lse"],
                                         args["workspace"], args["workspace_bytes"], args["stream"])


def test_batch_workspace_of_one_is_single(fixed_splits):
    d = kdv.make_dims(**KIMI)
    la, lp = kdv._host_i32([5553])
    ta, tp = kdv._host_i32([15])
    assert kdv.kdv_verify_batch_workspace_bytes(d, 1, lp, tp) == kdv.kdv_verify_workspace_bytes(d, 15, 5553)


def test_batch_workspace_formula(fixed_splits):
    # packed q_cat of all nodes + each request's split partials (KDV_SPLITS = 4 splits, capped by its tiles)
    d = kdv.make_dims(**KIMI)
    Ls, Ts = [5553, 0, 100], [15, 1, 33]
    la, lp = kdv._host_i32(Ls)
    ta, tp = kdv._host_i32(Ts)
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    rows = 0
    for L, T in zip(Ls, Ts):
        tiles = (L + T + 63) // 64
        want = min(4, tiles)
        tps = (tiles + want - 1) // want
        S = (tiles + tps - 1) // tps
        rows += S * ((T * 64 + 63) // 64) * 64
    expect = kdv.KDV_WS_HEADER + up(sum(Ts) * 64 * 576 * 2) + up(rows * 512 * 2) + up(rows * 8)
    assert kdv.kdv_verify_batch_workspace_bytes(d, 3, lp, tp) == expect


def test_batch_argument_errors(fixed_splits):
    d = kdv.make_dims(**KIMI)
    assert _batch(d, [10], [15], C=0) == kdv.KDV_ERR_SHAPE
    assert _batch(d, [10] * 17, [15] * 17) == kdv.KDV_ERR_SHAPE
    assert kdv.kdv_verify_mla_attn_batch(d, 1, None, None, A, A, A, A, A, A, 1 << 20, A, A, A, None, A, 1 << 40,
                                         None) == kdv.KDV_ERR_NULL
    for Ls, Ts in (([10, 10], [15, 0]), ([10, 10], [15, 65]), ([10, -1], [15, 3])):
        assert _batch(d, Ls, Ts) == kdv.KDV_ERR_SHAPE, (Ls, Ts)
    for field in ("q_nope", "page_table", "mask", "out", "workspace"):
        assert _batch(d, [10, 20], [15, 9], **{field: None}) == kdv.KDV_ERR_NULL, field
    for field, off in (("q_nope", 8), ("c_kv", 2), ("mask", 2), ("lse", 2), ("workspace", 8)):
        assert _batch(d, [10, 20], [15, 9], **{field: A + off}) == kdv.KDV_ERR_ALIGN, field
    la, lp = kdv._host_i32([5553, 20])
    ta, tp = kdv._host_i32([15, 9])
    need = kdv.kdv_verify_batch_workspace_bytes(d, 2, lp, tp)
    assert need > 0
    assert _batch(d, [5553, 20], [15, 9], ws_bytes=need - 1) == kdv.KDV_ERR_WORKSPACE


@pytest.mark.parametrize("splits", ["1", "3", "16", "63", "64", "100"])
def test_prefix_workspace_never_exceeds_verify(splits, monkeypatch):
    # sizing only (no call is made): a prefix pass's plan never has more splits than the full verify's
    monkeypatch.setenv("KDV_SPLITS", splits)
    for dims in (KIMI, dict(KIMI, num_heads=8), TINY):
        d = kdv.make_dims(**dims)
        for T in (1, 15, 32, 64):
            for L in (1, 63, 64, 65, 2048 * 64, 131072, 200000):
                p, v = kdv.kdv_prefix_workspace_bytes(d, T, L), kdv.kdv_verify_workspace_bytes(d, T, L)
                assert 0 < p <= v, (dims, T, L, p, v)
    assert kdv.kdv_prefix_workspace_bytes(kdv.make_dims(**KIMI), 15, 0) == 0


def test_tree_verify_argument_errors(fixed_splits):
    d = kdv.make_dims(**KIMI)

    def call(**kw):
        a = dict(parent=A, mask=A, status=None, q_nope=A, out=A)
        a.update(kw)
        return kdv.kdv_verify_mla_attn_tree(d, a["q_nope"], A, A, A, A, A, 1 << 20, A, 100, 15, a["parent"],
                                            a["mask"], a["status"], a["out"], None, A, 0, None)
    assert call(parent=None) == kdv.KDV_ERR_NULL
    assert call(mask=None) == kdv.KDV_ERR_NULL
    assert call(parent=A + 2) == kdv.KDV_ERR_ALIGN
    assert call(status=A + 1) == kdv.KDV_ERR_ALIGN
    assert call() == kdv.KDV_ERR_WORKSPACE  # workspace_bytes = 0: rejected before any launch


def test_mfma_probe_argument_errors():
    assert kdv.kdv_mfma_probe(10, None, 4, None) == kdv.KDV_ERR_NULL
    assert kdv.kdv_mfma_probe(0, A, 4, None) == kdv.KDV_ERR_SHAPE
    assert kdv.kdv_mfma_probe(10, A, 0, None) == kdv.KDV_ERR_SHAPE
    assert kdv.kdv_mfma_probe(10, A + 2, 4, None) == kdv.KDV_ERR_ALIGN


@pytest.mark.parametrize("scale", [0.0, -0.1, float("inf"), float("nan")])
def test_bad_softmax_scale_rejected(scale, fixed_splits):
    d = kdv.make_dims(**dict(KIMI, sm_scale=scale))
    assert _call(d) == kdv.KDV_ERR_SHAPE
    assert kdv.kdv_verify_workspace_bytes(d, 15, 100) == 0
