"""CPU oracle for the DDTree verify step: tree construction, tree-verify MLA attention (fp64), the prefix/tail
split with its state merge, greedy accept.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py``; never by the product package.
"""
from .accept import tree_accept
from .build import build_draft_tree
from .split import merge_attn_states, prefix_mla_absorbed
from .ref import (KDV_ERR_TREE, KDV_OK, ancestor_path, gather_latent, tree_mask, tree_status, verify_inputs,
                  verify_mla_absorbed, verify_mla_explicit, visibility)

__all__ = ["KDV_OK", "KDV_ERR_TREE", "ancestor_path", "build_draft_tree", "gather_latent", "merge_attn_states", "prefix_mla_absorbed", "tree_accept", "tree_mask", "tree_status",
           "verify_inputs", "verify_mla_absorbed", "verify_mla_explicit", "visibility"]
