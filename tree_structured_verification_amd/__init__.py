"""Tree-structured speculative verification on AMD Instinct MI355X (gfx950).

One verification round = four calls into the HIP library libtsv.so
(include/tsv.h): build_tree (or build_tree_topk / build_tree_fitted /
build_tree_expand), tree_verify_attn,
accept_walk, commit_path.
This package is the thin Python binding over that C ABI.
"""

from ._lib import (  # noqa: F401
    TSV_BF16,
    TSV_F32,
    TsvError,
    accept_walk,
    build_tree,
    build_tree_expand,
    build_tree_fitted,
    build_tree_noalloc,
    build_tree_topk,
    expanded_rows,
    fit_cost,
    kv_row_pitch,
    kv_rows,
    commit_path,
    compress_chains,
    lib,
    refresh_compressed,
    row_layout,
    select_global_budget,
    set_tree_method,
    status_string,
    tsv_cost,
    tsv_cost_fitted,
    tree_verify_attn,
    unfold_chains,
    workspace,
    workspace_size,
)
