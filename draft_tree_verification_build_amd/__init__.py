"""One speculative-decoding draft-tree step on MI355X (gfx950).

The computation lives in libdtv.so (HIP kernels behind the C ABI of include/dtv.h);
``api`` marshals torch device tensors into those calls.
"""
from .api import (BF16, F32, DtvError, Tree, Workspace, bookkeeping, build_params, kv_compact, row_stats,
                  tree_attn, tree_attn_noalloc, tree_build_begin, tree_build_given, tree_build_step, tree_build_opt, tree_build_spine, tree_build_talon, tree_verify_greedy,
                  tree_verify_sample)

__all__ = ["BF16", "F32", "DtvError", "Tree", "Workspace", "bookkeeping", "build_params", "kv_compact", "row_stats",
           "tree_attn", "tree_attn_noalloc", "tree_build_begin", "tree_build_given", "tree_build_step", "tree_build_opt", "tree_build_spine", "tree_build_talon", "tree_verify_greedy",
           "tree_verify_sample"]
