"""The C-ABI library loads without a GPU, exports every symbol the header
declares, and rejects bad arguments on the host before any launch (CPU)."""

import ctypes
import os
import re

import pytest

import tree_structured_verification_amd as tsv
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "tsv.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(\w+)\s*\(", text, re.M)))


def test_all_declared_symbols_exported():
    names = _declared()
    assert names == sorted(["build_tree", "build_tree_topk", "build_tree_fitted", "build_tree_noalloc",
                            "build_tree_expand", "tree_verify_attn", "accept_walk",
                            "commit_path", "select_global_budget", "tsv_fit_cost",
                            "tsv_workspace_size", "tsv_status_string", "unfold_chains",
                            "compress_chains", "refresh_compressed", "tsv_set_tree_method"])
    lib = ctypes.CDLL(tsv._lib.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    assert tsv.status_string(0) == "ok"
    assert "workspace" in tsv.status_string(-3)
    assert tsv.status_string(123) == "unknown status"


def test_workspace_sizes():
    ws = tsv.workspace_size
    assert ws(0, 16, 16, 151936, 32, 32) > 0
    assert ws(0, 1, 65, 16, 8, 8) == 0              # gamma too large
    assert ws(0, 1, 4, 16, 8, 129) == 0             # N_max too large
    assert ws(1, 16, 1, 1, 1, 32, 4112, 32, 8, 128, 128, 1) > 0
    assert ws(1, 16, 1, 1, 1, 32, 4112, 30, 8, 128, 128, 1) == 0    # Hq % Hkv
    assert ws(2, 16, 16, 151936, 1, 32, dtype=1) > 0
    assert ws(3) == 0
    assert ws(4, 8, 3, 129280, 2, 8) > 0            # 7 expanded rows of top-2
    assert ws(4, 1, 11, 16, 2, 8) > 0               # 2047 rows x 2 = 4094 list entries
    assert ws(4, 1, 12, 16, 2, 8) == 0              # 4095 rows x 2 > 4096
    assert ws(4, 1, 6, 16, 4, 8) == 0               # 1365 rows x 4 > 4096
    assert ws(4, 1, 65, 16, 1, 8) == 0              # depth beyond 64
    # larger caps never need less workspace
    assert ws(1, 64, 1, 1, 1, 128, 32784, 32, 8, 128, 128, 1) >= ws(1, 16, 1, 1, 1, 32, 4112, 32, 8, 128, 128, 1)


def test_host_validation_without_launch():
    L = tsv.lib()
    nul = None
    # null pointers
    assert L.build_tree(nul, 1, 1, 1, 1, 1, None, nul, 1, nul, nul, nul, nul, nul, nul,
                        nul, 0, nul) == -1
    assert L.tree_verify_attn(nul, nul, nul, nul, nul, 64, nul, nul, nul, 1, 1, 1, 1, 1, 64,
                              64, 0, 0.1, nul, nul, nul, 0, nul) == -1
    assert L.accept_walk(nul, 0, 1, 1, 1, 1, nul, nul, nul, nul, nul, nul, nul, 0, nul) == -1
    assert L.commit_path(nul, nul, nul, nul, nul, 1, nul, nul, 1, 1, 1, 1, 1, 1, 1, 0, nul,
                         nul) == -1
    # non-null fake device addresses that are never dereferenced: argument
    # checks fail first, so nothing is launched
    p = ctypes.c_void_p(0x1000)
    assert L.build_tree(p, 1, 2, 8, 9, 2, None, nul, 4, p, p, p, p, p, p, p,
                        1 << 20, nul) == -1                       # top_k > V
    assert L.build_tree(p, 1, 2, 8, 2, 2, None, nul, 4, p, p, p, p, p, p, p,
                        16, nul) == -3                            # workspace too small
    cost = tsv.tsv_cost(1.0, 0.02, 1e-4, 1e-6, 0.5)
    assert L.build_tree(p, 1, 2, 8, 2, 2, ctypes.byref(cost), nul, 4, p, p, p, p, p, p, p,
                        1 << 20, nul) == -1                       # adaptive without prefix_len
    bad = tsv.tsv_cost(1.0, -0.02, 1e-4, 1e-6, 0.5)
    assert L.build_tree(p, 1, 2, 8, 2, 2, ctypes.byref(bad), p, 4, p, p, p, p, p, p, p,
                        1 << 20, nul) == -1                       # negative coefficient
    assert L.build_tree_topk(p, 1, 2, 8, 2, 2, None, nul, 4, p, p, p, p, p, p, nul, nul, p,
                             1 << 20, nul) == -1                  # top-k outputs are required
    assert L.build_tree_topk(p, 1, 2, 8, 9, 2, None, nul, 4, p, p, p, p, p, p, p, p, p,
                             1 << 20, nul) == -1                  # top_k > V
    assert L.build_tree_noalloc(p, 1, 2, 8, 9, 2, None, nul, 4, p, p, p, p, p, p,
                                nul) == -1                        # top_k > V
    assert L.build_tree_noalloc(p, 200, 32, 256, 128, 2, None, nul, 4, p, p, p, p, p, p,
                                nul) == -2                        # top-k table above 4 MiB
    badf = tsv.tsv_cost_fitted(1.0, 0.02, 1e-4, 1e-6, 0.5, -1e-3)
    assert L.build_tree_fitted(p, 1, 2, 8, 2, 2, ctypes.byref(badf), p, 4, p, p, p, p, p, p, p,
                               1 << 20, nul) == -1                # negative f
    assert L.build_tree_fitted(p, 1, 2, 8, 2, 2, None, nul, 4, p, p, p, p, p, p, p,
                               16, nul) == -3                     # workspace too small
    assert L.tree_verify_attn(p, p, p, p, p, 64, p, p, p, 1, 4, 10, 4, 3, 64, 64, 1, 0.1,
                              p, nul, p, 1 << 30, nul) == -1      # Hq % Hkv
    assert L.tree_verify_attn(p, p, p, p, p, 10, p, p, p, 1, 4, 10, 4, 2, 64, 64, 1, 0.1,
                              p, nul, p, 1 << 30, nul) == -1      # stride < Hkv * d
    assert L.tree_verify_attn(p, p, p, p, p, 1200, p, p, p, 1, 4, 10, 4, 2, 600, 64, 1, 0.1,
                              p, nul, p, 1 << 30, nul) == -2      # head dim > 576
    assert L.accept_walk(p, 1, 1, 4, 8, 65, p, p, p, p, p, p, p, 1 << 20, nul) == -2  # gamma
    assert L.unfold_chains(p, p, 4, 8, 4, p, p, nul, nul) == -1                # null output
    assert L.unfold_chains(p, p, 4, 129, 4, p, p, p, nul) == -1                # N_max > 128
    assert L.unfold_chains(p, p, 4, 8, 65, p, p, p, nul) == -1                 # gamma > 64
    assert L.select_global_budget(p, p, p, p, p, p, 4, 8, nul, 10, nul) == -1   # null table
    assert L.select_global_budget(p, p, p, p, p, p, 4, 129, p, 10, nul) == -1   # N_max > 128
    assert L.select_global_budget(p, p, p, p, p, p, 65, 128, p, 10, nul) == -2  # 8320 candidates
    assert L.select_global_budget(p, p, p, p, p, p, 4, 8, p, 0, nul) == -1      # empty table
    assert L.build_tree_expand(nul, 1, 2, 8, 2, 2, None, nul, 4, p, p, p, p, p, p, nul, nul, p,
                               1 << 20, nul) == -1                # null probabilities
    assert L.build_tree_expand(p, 1, 2, 8, 9, 2, None, nul, 4, p, p, p, p, p, p, nul, nul, p,
                               1 << 20, nul) == -1                # top_k > V
    assert L.build_tree_expand(p, 1, 6, 16, 4, 2, None, nul, 4, p, p, p, p, p, p, nul, nul, p,
                               1 << 20, nul) == -2                # list table too large
    assert L.build_tree_expand(p, 1, 3, 8, 2, 2, None, nul, 4, p, p, p, p, p, p, nul, nul, p,
                               16, nul) == -3                     # workspace too small
    assert L.build_tree_expand(p, 1, 3, 8, 2, 9, None, nul, 4, p, p, p, p, p, p, nul, nul, p,
                               1 << 20, nul) == -1                # budget > N_max
    assert L.commit_path(p, nul, p, p, p, 64, p, p, 1, 4, 8, 1, 64, 64, 2, 1, p, nul) == -1
    # compress_chains(rows, dtype, stride, E, c, tail, pl, nc, cl, cn, B, N, gamma, ent, n_ent, s)
    assert L.compress_chains(p, 1, 64, 64, 4, p, p, p, p, p, 2, 8, 4, p, nul, nul) == -1  # null
    assert L.compress_chains(p, 1, 32, 64, 4, p, p, p, p, p, 2, 8, 4, p, p, nul) == -1   # stride < E
    assert L.compress_chains(p, 1, 64, 64, 0, p, p, p, p, p, 2, 8, 4, p, p, nul) == -1   # c < 1
    assert L.compress_chains(p, 1, 64, 64, 1 << 17, p, p, p, p, p, 2, 8, 4, p, p, nul) == -1  # c
    assert L.compress_chains(p, 1, 64, 64, 4, p, p, p, p, p, 2, 129, 4, p, p, nul) == -1  # N_max
    assert L.compress_chains(p, 1, 1 << 25, 1 << 25, 4, p, p, p, p, p, 2, 8, 4, p, p,
                             nul) == -2                                                 # E > 2^24
    # refresh_compressed(rows, dtype, stride, E, c, pl, al, an, nc, cl, cn, ent, B, N, gamma,
    #                    comp, Lc_cap, tail, status, s)
    assert L.refresh_compressed(p, 1, 64, 64, 4, p, p, p, p, p, p, p, 2, 8, 4, p, 8, p, nul,
                                nul) == -1                                              # null status
    assert L.refresh_compressed(p, 1, 64, 64, 4, p, p, p, p, p, p, p, 2, 8, 4, p, -1, p, p,
                                nul) == -1                                              # Lc_cap < 0
    assert L.refresh_compressed(p, 1, 64, 64, 4, p, p, p, p, p, p, p, 2, 8, 65, p, 8, p, p,
                                nul) == -1                                              # gamma > 64


# The four calls of a round and the cost struct, exactly as the boundary
# fixes them (argument names, types and order), after comments are removed and
# whitespace is collapsed.
CONTRACT = [
    "typedef struct { double a, b, c, e, c_d; } tsv_cost;",
    "int build_tree(const float* marginals, int B, int gamma, int V, int top_k, int n_budget, "
    "const tsv_cost* cost, const int* prefix_len, int N_max, int* n_nodes, int* parent, "
    "int* token, int* depth, float* score, unsigned* anc_bits, void* ws, size_t ws_bytes, "
    "hipStream_t s);",
    "int tree_verify_attn(const void* q, const void* k_cache, const void* v_cache, "
    "const void* k_tree, const void* v_tree, long kv_row_stride, const int* prefix_len, "
    "const int* n_nodes, const unsigned* anc_bits, int B, int N_max, int L_cap, int Hq, "
    "int Hkv, int d_qk, int d_v, int dtype, float sm_scale, void* out, float* lse, void* ws, "
    "size_t ws_bytes, hipStream_t s);",
    "int accept_walk(const void* target_logits, int dtype, int B, int N_max, int V, int gamma, "
    "const int* n_nodes, const int* parent, const int* token, int* accept_len, "
    "int* accept_nodes, int* out_tokens, void* ws, size_t ws_bytes, hipStream_t s);",
    "int commit_path(void* k_cache, void* v_cache, int* prefix_len, const void* k_tree, "
    "const void* v_tree, long kv_row_stride, const int* accept_len, const int* accept_nodes, "
    "int B, int N_max, int L_cap, int Hkv, int d_k, int d_v, int gamma, int dtype, "
    "int* status, hipStream_t s);",
    "size_t tsv_workspace_size(int which, int B, int gamma, int V, int top_k, int N_max, "
    "int L_cap, int Hq, int Hkv, int d_qk, int d_v, int dtype);",
    "const char* tsv_status_string(int code);",
    "enum { TSV_F32 = 0, TSV_BF16 = 1 };",
]


def _flat_header():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"\s+", " ", text)
    return re.sub(r"\s*([(),;{}])\s*", r"\1", text)


def test_contract_prototypes_verbatim():
    flat = _flat_header()
    for decl in CONTRACT:
        norm = re.sub(r"\s*([(),;{}])\s*", r"\1", re.sub(r"\s+", " ", decl))
        assert norm in flat, decl
    for code, name in ((0, "TSV_OK"), (-1, "TSV_EINVAL"), (-2, "TSV_EUNSUPPORTED"),
                       (-3, "TSV_EWORKSPACE"), (-4, "TSV_EHIP")):
        assert re.search(rf"{name}={code}\b", flat.replace(" ", "")), name


def test_cost_struct_layout():
    assert ctypes.sizeof(tsv.tsv_cost) == 40
    assert [f for f, _ in tsv.tsv_cost._fields_] == ["a", "b", "c", "e", "c_d"]
    assert ctypes.sizeof(tsv.tsv_cost_fitted) == 48
    assert [f for f, _ in tsv.tsv_cost_fitted._fields_][:5] == ["a", "b", "c", "e", "c_d"]
    # the C side agrees: a header-only check compiled with the host compiler
    import shutil
    import subprocess
    import tempfile
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    src = ('#include "tsv.h"\n#include <stddef.h>\n'
           '_Static_assert(sizeof(tsv_cost) == 40, "tsv_cost");\n'
           '_Static_assert(offsetof(tsv_cost, c_d) == 32, "c_d");\n'
           '_Static_assert(sizeof(tsv_cost_fitted) == 48, "fitted");\n'
           'int main(void) { return 0; }\n')
    with tempfile.TemporaryDirectory() as d:
        f = os.path.join(d, "c.c")
        open(f, "w").write(src)
        r = subprocess.run([cc, "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                            "-I", "/opt/rocm/include", "-fsyntax-only", f],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_binding_requires_device_tensors():
    import torch
    with pytest.raises(ValueError):
        tsv.build_tree(torch.zeros(1, 2, 8), 2, 2, 4)
