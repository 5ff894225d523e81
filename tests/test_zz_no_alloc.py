"""The allocation-free tree verify (ssu_tree_verify_noalloc, the library's
per-GPU scratch in place of a caller workspace) against ssu_tree_verify on the
same inputs: outputs and stash bitwise equal, on two calls in a row (the second
smaller, so the scratch still holds the first call's larger contents), and the
size limit refused on the host. Collected last: it leaves the scratch used."""
import ctypes

import numpy as np
import pytest
import torch

from linear_rnn_recurrent_amd import (SsuError, TREE_SCRATCH_BYTES, inputs, ssu_tree_verify,
                                      ssu_tree_verify_noalloc, tree_workspace_bytes)
from gpu_helpers import TOL_F32, assert_bitwise, assert_close, gpu, oracle_tree, tol_for

pytestmark = pytest.mark.gpu


def _run(fn, w):
    T = {k: gpu(v) for k, v in w.tensors.items()}
    out = torch.full_like(T["x"], float("nan"))
    b, m, h, d = T["x"].shape
    S = {"replay_dA": torch.full((b, m, h), float("nan"), device="cuda"),
         "replay_dt": torch.full((b, m, h), float("nan"), device="cuda"),
         "replay_u": torch.full((b, m, h, d), float("nan"), device="cuda"),
         "replay_B": torch.full(tuple(T["B"].shape), float("nan"), device="cuda")}
    fn(T["x"], T["A"], T["B"], T["C"], T["dt"], T["state"], out, T["parent_ids"],
       depths=T["depths"], dt_bias=T["dt_bias"], D=T["D"], z=T["z"], dt_softplus=w.dt_softplus,
       state_indices=T["state_indices"], **S)
    return out, S


def _check_same(w):
    ref_out, ref_S = _run(ssu_tree_verify, w)
    out, S = _run(ssu_tree_verify_noalloc, w)
    torch.cuda.synchronize()
    assert_bitwise(out, ref_out, "outputs: noalloc vs workspace entry point")
    for k in S:
        assert_bitwise(S[k], ref_S[k], f"{k}: noalloc vs workspace entry point")
    return out


def test_noalloc_matches_the_workspace_entry_point_twice_second_smaller():
    # first call: the full 4 MiB (B64 G1 M128); second: B5 G2 M37 with padding
    big = inputs.tree_workload(batch=64, num_nodes=128, nheads=8, dim=64, dstate=128, ngroups=1,
                               pool_rows=70, seed=91, bc_std=128 ** -0.5, max_depth=16)
    assert tree_workspace_bytes(64, 1, 128) == TREE_SCRATCH_BYTES
    _check_same(big)
    small = inputs.tree_workload(batch=5, num_nodes=37, nheads=4, dim=64, dstate=64, ngroups=2,
                                 pool_rows=7, seed=92, bc_std=0.125, max_depth=6,
                                 indices=[6, -1, 0, 3, 2], io_dtype="f32", bc_dtype="f32",
                                 with_z=True)
    out = _check_same(small)
    # and to the oracle, as every tree-verify parity test
    out_ref, _ = oracle_tree(small, stash=True)
    assert_close(out.cpu(), out_ref, tol_for(out.dtype), "noalloc outputs vs oracle")


def test_noalloc_refuses_trees_beyond_the_scratch():
    w = inputs.tree_workload(batch=65, num_nodes=128, nheads=2, dim=64, dstate=64, ngroups=1,
                             pool_rows=65, seed=93, bc_std=0.125, max_depth=4)
    with pytest.raises(SsuError, match="scratch"):
        _run(ssu_tree_verify_noalloc, w)
