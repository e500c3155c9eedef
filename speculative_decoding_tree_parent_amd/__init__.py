"""Python binding of libkdv: DDTree tree-verify attention for MLA on MI355X (gfx950).

The functions named ``kdv_*`` are the C ABI of ``include/kdv.h`` one for one (plain integers for device
pointers and streams).  ``build_tree_mask``, ``verify_workspace_bytes`` and ``verify_mla_attn`` only
marshal torch tensors into those calls: every step of the computation runs in the HIP kernels of
``libkdv.so``.  There is no fallback: if the library is missing, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os

# torch ships its own HIP runtime (same soname as /opt/rocm's).  Loading it first makes libkdv.so bind to that
# same runtime instead of pulling a second one into the process.
import torch  # noqa: F401

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libkdv.so")

KDV_OK = 0
KDV_ERR_NULL = -1
KDV_ERR_SHAPE = -2
KDV_ERR_TREE = -3
KDV_ERR_ALIGN = -4
KDV_ERR_WORKSPACE = -5
KDV_ERR_HIP = -6
KDV_ERR_PAGE = -7
KDV_WS_HEADER = 256
KDV_NOALLOC_SCRATCH_BYTES = 32 << 20
KDV_MAX_TREE_NODES = 64
KDV_MAX_DRAFT_ENTRIES = 4096
KDV_MAX_BATCH = 16

EXPORTED = ("kdv_build_draft_tree", "kdv_build_tree_mask", "kdv_merge_attn_states", "kdv_prefix_mla_attn",
            "kdv_prefix_workspace_bytes",
            "kdv_tree_accept", "kdv_verify_batch_workspace_bytes", "kdv_verify_mla_attn_batch",
            "kdv_verify_workspace_bytes", "kdv_verify_mla_attn", "kdv_verify_mla_attn_profiled",
            "kdv_verify_mla_attn_tree", "kdv_verify_mla_attn_noalloc",
            "kdv_verify_num_splits", "kdv_verify_kernel_count", "kdv_mfma_probe", "kdv_status_string")


class KdvMlaDims(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("qk_nope_dim", ctypes.c_int32), ("qk_rope_dim", ctypes.c_int32),
                ("kv_lora_rank", ctypes.c_int32), ("v_head_dim", ctypes.c_int32), ("sm_scale", ctypes.c_float)]


class KdvError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {kdv_status_string(status)} ({status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libkdv.so not built at {LIB_PATH}; run `python speculative_decoding_tree_parent_amd/build.py`"
                          " (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    dims_p = ctypes.POINTER(KdvMlaDims)
    lib.kdv_build_tree_mask.argtypes = [vp, i32, vp, vp, vp]
    lib.kdv_build_tree_mask.restype = ctypes.c_int
    lib.kdv_build_draft_tree.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp, vp]
    lib.kdv_build_draft_tree.restype = ctypes.c_int
    lib.kdv_tree_accept.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, vp]
    lib.kdv_tree_accept.restype = ctypes.c_int
    lib.kdv_verify_workspace_bytes.argtypes = [dims_p, i32, i32]
    lib.kdv_verify_workspace_bytes.restype = sz
    lib.kdv_verify_num_splits.argtypes = [dims_p, i32, i32]
    lib.kdv_verify_num_splits.restype = i32
    lib.kdv_verify_kernel_count.argtypes = [dims_p, i32, i32]
    lib.kdv_verify_kernel_count.restype = i32
    lib.kdv_verify_mla_attn.argtypes = [dims_p, vp, vp, vp, vp, vp, vp, i64, vp, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.kdv_verify_mla_attn.restype = ctypes.c_int
    lib.kdv_verify_mla_attn_profiled.argtypes = [dims_p, vp, vp, vp, vp, vp, vp, i64, vp, i32, i32, vp, vp, vp, vp,
                                                 sz, vp, vp]
    lib.kdv_verify_mla_attn_profiled.restype = ctypes.c_int
    lib.kdv_verify_mla_attn_tree.argtypes = [dims_p, vp, vp, vp, vp, vp, vp, i64, vp, i32, i32, vp, vp, vp, vp, vp,
                                             vp, sz, vp]
    lib.kdv_verify_mla_attn_tree.restype = ctypes.c_int
    lib.kdv_verify_mla_attn_noalloc.argtypes = [dims_p, vp, vp, vp, vp, vp, vp, i64, vp, i32, i32, vp, vp, vp, vp]
    lib.kdv_verify_mla_attn_noalloc.restype = ctypes.c_int
    lib.kdv_verify_mla_attn_batch.argtypes = [dims_p, i32, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp,
                                              sz, vp]
    lib.kdv_verify_mla_attn_batch.restype = ctypes.c_int
    lib.kdv_verify_batch_workspace_bytes.argtypes = [dims_p, i32, vp, vp]
    lib.kdv_verify_batch_workspace_bytes.restype = sz
    lib.kdv_prefix_mla_attn.argtypes = [dims_p, vp, vp, vp, vp, vp, vp, i64, vp, i32, i32, vp, vp, vp, sz, vp]
    lib.kdv_prefix_mla_attn.restype = ctypes.c_int
    lib.kdv_prefix_workspace_bytes.argtypes = [dims_p, i32, i32]
    lib.kdv_prefix_workspace_bytes.restype = sz
    lib.kdv_merge_attn_states.argtypes = [vp, vp, vp, vp, i64, i32, vp, vp, vp]
    lib.kdv_merge_attn_states.restype = ctypes.c_int
    lib.kdv_mfma_probe.argtypes = [i32, vp, i32, vp]
    lib.kdv_mfma_probe.restype = ctypes.c_int
    lib.kdv_status_string.argtypes = [ctypes.c_int]
    lib.kdv_status_string.restype = ctypes.c_char_p
    return lib


_lib = _load()


# ------------------------------------------------------------------------------------------- C ABI, 1:1
def kdv_build_tree_mask(parent: int, T: int, mask: int, status: int | None, stream: int | None) -> int:
    return _lib.kdv_build_tree_mask(parent, T, mask, status, stream)


def kdv_build_draft_tree(logp: int, tok: int, block: int, K: int, budget: int, root_token: int, parent: int,
                         tokens: int, n_nodes: int, stream: int | None) -> int:
    return _lib.kdv_build_draft_tree(logp, tok, block, K, budget, root_token, parent, tokens, n_nodes, stream)


def kdv_tree_accept(parent: int, tokens: int, pred: int, T: int, path: int, n_path: int, next_token: int,
                    status: int | None, stream: int | None) -> int:
    return _lib.kdv_tree_accept(parent, tokens, pred, T, path, n_path, next_token, status, stream)


def kdv_verify_workspace_bytes(dims: KdvMlaDims, T: int, L: int) -> int:
    return _lib.kdv_verify_workspace_bytes(ctypes.byref(dims), T, L)


def kdv_verify_num_splits(dims: KdvMlaDims, T: int, L: int) -> int:
    return _lib.kdv_verify_num_splits(ctypes.byref(dims), T, L)


def kdv_verify_kernel_count(dims: KdvMlaDims, T: int, L: int) -> int:
    return _lib.kdv_verify_kernel_count(ctypes.byref(dims), T, L)


def kdv_verify_mla_attn(dims: KdvMlaDims, q_nope: int, q_rope: int, w_uk: int, w_uv: int, c_kv: int, k_pe: int,
                        pool_slots: int, page_table: int, L: int, T: int, mask: int, out: int, lse: int | None,
                        workspace: int, workspace_bytes: int, stream: int | None) -> int:
    return _lib.kdv_verify_mla_attn(ctypes.byref(dims), q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, pool_slots,
                                    page_table, L, T, mask, out, lse, workspace, workspace_bytes, stream)


def kdv_verify_mla_attn_profiled(dims: KdvMlaDims, q_nope: int, q_rope: int, w_uk: int, w_uv: int, c_kv: int,
                                 k_pe: int, pool_slots: int, page_table: int, L: int, T: int, mask: int, out: int,
                                 lse: int | None, workspace: int, workspace_bytes: int, stream: int | None,
                                 events: int) -> int:
    """`events`: address of 2 * kdv_verify_kernel_count() hipEvent_t handles: start/stop of each kernel (include/kdv.h)."""
    return _lib.kdv_verify_mla_attn_profiled(ctypes.byref(dims), q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, pool_slots,
                                             page_table, L, T, mask, out, lse, workspace, workspace_bytes, stream,
                                             events)


def kdv_verify_mla_attn_tree(dims: KdvMlaDims, q_nope: int, q_rope: int, w_uk: int, w_uv: int, c_kv: int, k_pe: int,
                             pool_slots: int, page_table: int, L: int, T: int, parent: int, mask: int,
                             status: int | None, out: int, lse: int | None, workspace: int, workspace_bytes: int,
                             stream: int | None) -> int:
    return _lib.kdv_verify_mla_attn_tree(ctypes.byref(dims), q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, pool_slots,
                                         page_table, L, T, parent, mask, status, out, lse, workspace,
                                         workspace_bytes, stream)


def kdv_verify_mla_attn_noalloc(dims: KdvMlaDims, q_nope: int, q_rope: int, w_uk: int, w_uv: int, c_kv: int,
                                k_pe: int, pool_slots: int, page_table: int, L: int, T: int, mask: int, out: int,
                                lse: int | None, stream: int | None) -> int:
    return _lib.kdv_verify_mla_attn_noalloc(ctypes.byref(dims), q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, pool_slots,
                                            page_table, L, T, mask, out, lse, stream)


def _host_i32(values):
    """(ctypes int32 array, its address) for a host array argument; None passes NULL."""
    if values is None:
        return None, None
    arr = (ctypes.c_int32 * len(values))(*[int(v) for v in values])
    return arr, ctypes.addressof(arr)


def kdv_verify_batch_workspace_bytes(dims: KdvMlaDims, C: int, L: int | None, T: int | None) -> int:
    """L, T: addresses of host int32 arrays (see _host_i32)."""
    return _lib.kdv_verify_batch_workspace_bytes(ctypes.byref(dims), C, L, T)


def kdv_verify_mla_attn_batch(dims: KdvMlaDims, C: int, L: int | None, T: int | None, q_nope: int, q_rope: int,
                              w_uk: int, w_uv: int, c_kv: int, k_pe: int, pool_slots: int, page_table: int,
                              mask: int, out: int, lse: int | None, workspace: int, workspace_bytes: int,
                              stream: int | None) -> int:
    """L, T: addresses of host int32 arrays of C entries (see _host_i32)."""
    return _lib.kdv_verify_mla_attn_batch(ctypes.byref(dims), C, L, T, q_nope, q_rope, w_uk, w_uv, c_kv, k_pe,
                                          pool_slots, page_table, mask, out, lse, workspace, workspace_bytes, stream)


def kdv_prefix_mla_attn(dims: KdvMlaDims, q_nope: int, q_rope: int, w_uk: int, w_uv: int, c_kv: int, k_pe: int,
                        pool_slots: int, page_table: int, L: int, T: int, out: int, lse: int | None, workspace: int,
                        workspace_bytes: int, stream: int | None) -> int:
    return _lib.kdv_prefix_mla_attn(ctypes.byref(dims), q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, pool_slots,
                                    page_table, L, T, out, lse, workspace, workspace_bytes, stream)


def kdv_prefix_workspace_bytes(dims: KdvMlaDims, T: int, L: int) -> int:
    return _lib.kdv_prefix_workspace_bytes(ctypes.byref(dims), T, L)


def kdv_merge_attn_states(out_a: int, lse_a: int, out_b: int, lse_b: int, rows: int, dv: int, out: int,
                          lse: int | None, stream: int | None) -> int:
    return _lib.kdv_merge_attn_states(out_a, lse_a, out_b, lse_b, rows, dv, out, lse, stream)


def kdv_mfma_probe(iters: int, sink: int, blocks: int, stream: int | None) -> int:
    return _lib.kdv_mfma_probe(iters, sink, blocks, stream)


def kdv_status_string(status: int) -> str:
    return _lib.kdv_status_string(status).decode()


# ------------------------------------------------------------------------------------------- torch marshalling
def make_dims(num_heads: int, qk_nope_dim: int, qk_rope_dim: int, kv_lora_rank: int, v_head_dim: int,
              sm_scale: float) -> KdvMlaDims:
    return KdvMlaDims(num_heads, qk_nope_dim, qk_rope_dim, kv_lora_rank, v_head_dim, sm_scale)


def _stream_handle(stream) -> int | None:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _ptr(t, dtype, what: str) -> int:
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


def _bf16_ptr(t, what: str) -> int:
    """Device address of a bf16 tensor given as torch.bfloat16 or as int16 bit patterns."""
    import torch
    return _ptr(t, torch.bfloat16 if t.dtype == torch.bfloat16 else torch.int16, what)


def new_workspace(nbytes: int, device) -> "torch.Tensor":
    """A device workspace of nbytes (zeroed, so that reading the KDV_DEBUG status word before any check is defined)."""
    import torch
    return torch.zeros((nbytes,), dtype=torch.uint8, device=device)


def debug_status(workspace) -> int:
    """The page-table status a call made with KDV_DEBUG set wrote into its workspace (KDV_OK or KDV_ERR_PAGE).
    Reads the device (synchronising with it)."""
    import torch
    return int(workspace[:4].view(torch.int32).item())


def build_tree_mask(parent, mask=None, status=None, stream=None):
    """parent: int32 [T] device tensor -> (mask uint32-as-int32 [T][W], status int32 [1])."""
    import torch
    T = parent.shape[0]
    W = (T + 31) // 32
    if mask is None:
        mask = torch.empty((T, W), dtype=torch.int32, device=parent.device)
    if status is None:
        status = torch.empty((1,), dtype=torch.int32, device=parent.device)
    rc = kdv_build_tree_mask(_ptr(parent, torch.int32, "parent"), T, _ptr(mask, torch.int32, "mask"),
                             _ptr(status, torch.int32, "status"), _stream_handle(stream))
    if rc != KDV_OK:
        raise KdvError(rc, "kdv_build_tree_mask")
    return mask, status


def build_draft_tree(logp, tok, budget: int, root_token, stream=None):
    """logp float32 [block][K], tok int32 [block][K], root_token int32 [1] (device tensors)
    -> (parent int32 [budget], tokens int32 [budget], n_nodes int32 [1])."""
    import torch
    block, K = logp.shape
    dev = logp.device
    parent = torch.empty((budget,), dtype=torch.int32, device=dev)
    tokens = torch.empty((budget,), dtype=torch.int32, device=dev)
    n_nodes = torch.empty((1,), dtype=torch.int32, device=dev)
    rc = kdv_build_draft_tree(_ptr(logp, torch.float32, "logp"), _ptr(tok, torch.int32, "tok"), block, K, budget,
                              _ptr(root_token, torch.int32, "root_token"), _ptr(parent, torch.int32, "parent"),
                              _ptr(tokens, torch.int32, "tokens"), _ptr(n_nodes, torch.int32, "n_nodes"),
                              _stream_handle(stream))
    if rc != KDV_OK:
        raise KdvError(rc, "kdv_build_draft_tree")
    return parent, tokens, n_nodes


def tree_accept(parent, tokens, pred, stream=None):
    """parent, tokens, pred: int32 [T] device tensors -> (path int32 [T], n_path, next_token, status: int32 [1])."""
    import torch
    T = parent.shape[0]
    dev = parent.device
    path = torch.empty((T,), dtype=torch.int32, device=dev)
    n_path = torch.empty((1,), dtype=torch.int32, device=dev)
    next_token = torch.empty((1,), dtype=torch.int32, device=dev)
    status = torch.empty((1,), dtype=torch.int32, device=dev)
    rc = kdv_tree_accept(_ptr(parent, torch.int32, "parent"), _ptr(tokens, torch.int32, "tokens"),
                         _ptr(pred, torch.int32, "pred"), T, _ptr(path, torch.int32, "path"),
                         _ptr(n_path, torch.int32, "n_path"), _ptr(next_token, torch.int32, "next_token"),
                         _ptr(status, torch.int32, "status"), _stream_handle(stream))
    if rc != KDV_OK:
        raise KdvError(rc, "kdv_tree_accept")
    return path, n_path, next_token, status


def verify_workspace_bytes(dims: KdvMlaDims, T: int, L: int) -> int:
    n = kdv_verify_workspace_bytes(dims, T, L)
    if n == 0:
        raise KdvError(KDV_ERR_SHAPE, "kdv_verify_workspace_bytes")
    return n


def verify_mla_attn(dims: KdvMlaDims, q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, page_table, L: int, mask, out=None,
                    lse=None, workspace=None, stream=None, pool_slots=None):
    """All tensors on the device; bf16 tensors may be torch.bfloat16 or int16 bit patterns.  pool_slots defaults
    to the pool's row count.

    Returns (out [T][H][Dv] bf16, lse [T][H] fp32 or None)."""
    import torch
    T = q_nope.shape[0]
    H = dims.num_heads

    bf = _bf16_ptr

    if out is None:
        out = torch.empty((T, H, dims.v_head_dim), dtype=torch.bfloat16, device=q_nope.device)
    if workspace is None:
        workspace = torch.zeros((verify_workspace_bytes(dims, T, L),), dtype=torch.uint8, device=q_nope.device)
    lse_ptr = None if lse is None else _ptr(lse, torch.float32, "lse")
    rc = kdv_verify_mla_attn(dims, bf(q_nope, "q_nope"), bf(q_rope, "q_rope"), bf(w_uk, "w_uk"), bf(w_uv, "w_uv"),
                             bf(c_kv, "c_kv"), bf(k_pe, "k_pe"), c_kv.shape[0] if pool_slots is None else pool_slots,
                             _ptr(page_table, torch.int32, "page_table"),
                             L, T, _ptr(mask, torch.int32, "mask"), bf(out, "out"), lse_ptr,
                             _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream_handle(stream))
    if rc != KDV_OK:
        raise KdvError(rc, "kdv_verify_mla_attn")
    return out, lse


def prefix_mla_attn(dims: KdvMlaDims, q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, page_table, L: int, out=None,
                    lse=None, workspace=None, stream=None, pool_slots=None):
    """Prefix part of a split verify step: every (node, head) row over the L prefix positions only.

    page_table: int32 [L] device tensor.  Returns (out [T][H][Dv] bf16, lse [T][H] fp32)."""
    import torch
    T = q_nope.shape[0]
    H = dims.num_heads

    bf = _bf16_ptr

    if out is None:
        out = torch.empty((T, H, dims.v_head_dim), dtype=torch.bfloat16, device=q_nope.device)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=q_nope.device)
    if workspace is None:
        n = kdv_prefix_workspace_bytes(dims, T, L)
        if n == 0:
            raise KdvError(KDV_ERR_SHAPE, "kdv_prefix_workspace_bytes")
        workspace = torch.zeros((n,), dtype=torch.uint8, device=q_nope.device)
    rc = kdv_prefix_mla_attn(dims, bf(q_nope, "q_nope"), bf(q_rope, "q_rope"), bf(w_uk, "w_uk"), bf(w_uv, "w_uv"),
                             bf(c_kv, "c_kv"), bf(k_pe, "k_pe"), c_kv.shape[0] if pool_slots is None else pool_slots,
                             _ptr(page_table, torch.int32, "page_table"), L, T, bf(out, "out"),
                             _ptr(lse, torch.float32, "lse"), _ptr(workspace, torch.uint8, "workspace"),
                             workspace.numel(), _stream_handle(stream))
    if rc != KDV_OK:
        raise KdvError(rc, "kdv_prefix_mla_attn")
    return out, lse


def merge_attn_states(out_a, lse_a, out_b, lse_b, out=None, lse=None, stream=None):
    """LSE merge of two attention results over disjoint KV position sets.

    out_a, out_b: bf16 [..., dv]; lse_a, lse_b: fp32 [...] (same leading shape).  Returns (out, lse)."""
    import torch
    dv = out_a.shape[-1]
    rows = lse_a.numel()
    if out_b.shape != out_a.shape or lse_b.shape != lse_a.shape or out_a.numel() != rows * dv:
        raise ValueError("merge_attn_states: shapes of the two parts differ")
    if out is None:
        out = torch.empty_like(out_a)
    if lse is None:
        lse = torch.empty_like(lse_a)
    rc = kdv_merge_attn_states(_ptr(out_a, torch.bfloat16, "out_a"), _ptr(lse_a, torch.float32, "lse_a"),
                               _ptr(out_b, torch.bfloat16, "out_b"), _ptr(lse_b, torch.float32, "lse_b"), rows, dv,
                               _ptr(out, torch.bfloat16, "out"), _ptr(lse, torch.float32, "lse"),
                               _stream_handle(stream))
    if rc != KDV_OK:
        raise KdvError(rc, "kdv_merge_attn_states")
    return out, lse


def build_tree_masks(parents, stream=None):
    """Packed ancestor masks of several trees (one kdv_build_tree_mask launch each), in the layout
    kdv_verify_mla_attn_batch takes.  parents: list of int32 device tensors.  Returns (mask int32 tensor,
    status int32 [len(parents)])."""
    import torch
    dev = parents[0].device
    words = [p.shape[0] * ((p.shape[0] + 31) // 32) for p in parents]
    mask = torch.empty((sum(words),), dtype=torch.int32, device=dev)
    status = torch.empty((len(parents),), dtype=torch.int32, device=dev)
    off = 0
    for i, (p, w) in enumerate(zip(parents, words)):
        rc = kdv_build_tree_mask(_ptr(p, torch.int32, "parent"), p.shape[0], mask.data_ptr() + 4 * off,
                                 status.data_ptr() + 4 * i, _stream_handle(stream))
        if rc != KDV_OK:
            raise KdvError(rc, "kdv_build_tree_mask")
        off += w
    return mask, status


def verify_batch_workspace_bytes(dims: KdvMlaDims, Ls, Ts) -> int:
    la, lp = _host_i32(Ls)
    ta, tp = _host_i32(Ts)
    n = kdv_verify_batch_workspace_bytes(dims, len(Ls), lp, tp)
    if n == 0:
        raise KdvError(KDV_ERR_SHAPE, "kdv_verify_batch_workspace_bytes")
    return n


def verify_mla_attn_batch(dims: KdvMlaDims, q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, page_table, Ls, Ts, mask,
                          out=None, lse=None, workspace=None, stream=None, pool_slots=None):
    """Batched verify over packed requests (include/kdv.h): q_nope [sum T][H][Dn], page_table [sum (L+T)],
    mask from build_tree_masks.  Returns (out [sum T][H][Dv] bf16, lse [sum T][H] fp32 or None)."""
    import torch
    n_nodes = int(sum(Ts))
    H = dims.num_heads

    bf = _bf16_ptr

    if out is None:
        out = torch.empty((n_nodes, H, dims.v_head_dim), dtype=torch.bfloat16, device=q_nope.device)
    if workspace is None:
        workspace = torch.zeros((verify_batch_workspace_bytes(dims, Ls, Ts),), dtype=torch.uint8,
                                device=q_nope.device)
    la, lp = _host_i32(Ls)
    ta, tp = _host_i32(Ts)
    lse_ptr = None if lse is None else _ptr(lse, torch.float32, "lse")
    rc = kdv_verify_mla_attn_batch(dims, len(Ls), lp, tp, bf(q_nope, "q_nope"), bf(q_rope, "q_rope"),
                                   bf(w_uk, "w_uk"), bf(w_uv, "w_uv"), bf(c_kv, "c_kv"), bf(k_pe, "k_pe"),
                                   c_kv.shape[0] if pool_slots is None else pool_slots,
                                   _ptr(page_table, torch.int32, "page_table"),
                                   _ptr(mask, torch.int32, "mask"), bf(out, "out"), lse_ptr,
                                   _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                   _stream_handle(stream))
    if rc != KDV_OK:
        raise KdvError(rc, "kdv_verify_mla_attn_batch")
    return out, lse


def verify_mla_attn_tree(dims: KdvMlaDims, q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, page_table, L: int, parent,
                         mask=None, status=None, out=None, lse=None, workspace=None, stream=None):
    """verify_mla_attn that builds the ancestor mask from `parent` (int32 [T] device tensor) in the same call.

    Returns (out, lse or None, mask int32 [T][W], status int32 [1])."""
    import torch
    T = q_nope.shape[0]
    H = dims.num_heads
    dev = q_nope.device

    bf = _bf16_ptr

    if mask is None:
        mask = torch.empty((T, (T + 31) // 32), dtype=torch.int32, device=dev)
    if status is None:
        status = torch.empty((1,), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((T, H, dims.v_head_dim), dtype=torch.bfloat16, device=dev)
    if workspace is None:
        workspace = torch.zeros((verify_workspace_bytes(dims, T, L),), dtype=torch.uint8, device=dev)
    lse_ptr = None if lse is None else _ptr(lse, torch.float32, "lse")
    rc = kdv_verify_mla_attn_tree(dims, bf(q_nope, "q_nope"), bf(q_rope, "q_rope"), bf(w_uk, "w_uk"),
                                  bf(w_uv, "w_uv"), bf(c_kv, "c_kv"), bf(k_pe, "k_pe"), c_kv.shape[0],
                                  _ptr(page_table, torch.int32, "page_table"), L, T, _ptr(parent, torch.int32, "parent"),
                                  _ptr(mask, torch.int32, "mask"), _ptr(status, torch.int32, "status"),
                                  bf(out, "out"), lse_ptr, _ptr(workspace, torch.uint8, "workspace"),
                                  workspace.numel(), _stream_handle(stream))
    if rc != KDV_OK:
        raise KdvError(rc, "kdv_verify_mla_attn_tree")
    return out, lse, mask, status
