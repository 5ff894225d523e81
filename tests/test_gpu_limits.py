"""The size limits of the boundary on the GPU: the largest head dimension
(dim 4096, 64 row blocks per head) and the largest dstate (256) through decode,
both prefill kernels, replay and tree verify, and prefills whose every context
is empty, all against the fp64 oracle."""
import numpy as np
import pytest
import torch

from linear_rnn_recurrent_amd import inputs
from gpu_helpers import (TOL_F32, assert_bitwise, assert_close, f64, oracle_decode, oracle_replay,
                         oracle_tree, run_decode, run_replay, run_tree, tol_for)
from test_gpu_prefill import check_prefill, valu_kernel

pytestmark = pytest.mark.gpu

DIM_MAX = 4096


@pytest.mark.parametrize("dstate,state_dtype", [(128, "f32"), (256, "f16")])
def test_decode_at_the_largest_dim(dstate, state_dtype):
    w = inputs.decode_workload(batch=3, nheads=2, dim=DIM_MAX, dstate=dstate, ngroups=1, pool_rows=4,
                               seed=71, state_dtype=state_dtype, bc_std=dstate ** -0.5,
                               indices=[3, -1, 0])
    state0 = w["state"].clone()
    st, out = run_decode(w)
    st_ref, out_ref = oracle_decode(w)
    stc, outc = st.cpu(), out.cpu()
    assert_close(stc[[3, 0]], st_ref[[3, 0]], tol_for(stc.dtype), "state")
    assert_close(outc[[0, 2]], out_ref[[0, 2]], tol_for(outc.dtype), "out")
    assert_bitwise(stc[[1, 2]], state0[[1, 2]], "rows not addressed")
    assert_bitwise(outc[1], torch.zeros_like(outc[1]), "padding row output")


@pytest.mark.parametrize("io", ["bf16", "f32"])  # matrix-core and VALU kernels
def test_prefill_at_the_largest_dim(io):
    w = inputs.prefill_workload(batch=2, seq_len=40, nheads=1, dim=DIM_MAX, dstate=128, ngroups=1,
                                pool_rows=3, seed=72, io_dtype=io, bc_dtype=io, bc_std=128 ** -0.5,
                                ctx=[40, 33])
    check_prefill(w)
    check_prefill(w, stash=True)


def test_prefill_at_the_largest_dstate_on_both_kernels():
    # bf16 and fp16 on the matrix cores; fp16 with x off 16-byte alignment and
    # fp32 on the VALU kernel
    for io in ("bf16", "f16", "f32"):
        w = inputs.prefill_workload(batch=2, seq_len=70, nheads=2, dim=64, dstate=256, ngroups=1,
                                    pool_rows=2, seed=73, io_dtype=io, bc_dtype=io,
                                    bc_std=256 ** -0.5, ctx=[70, 38])
        check_prefill(w)
        if io == "f16":
            check_prefill(w, **valu_kernel(w))


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_prefill_with_every_context_empty(io):
    # no token of any row is live: outputs +0.0, state and stash rows untouched
    w = inputs.prefill_workload(batch=3, seq_len=37, nheads=2, dim=64, dstate=64, ngroups=1,
                                pool_rows=4, seed=74, io_dtype=io, bc_dtype=io, bc_std=0.125,
                                ctx=[0, -5, 0])
    state0 = w["state"].clone()
    st, out, _ = check_prefill(w)
    assert_bitwise(st.cpu(), state0, "state with every context empty")
    check_prefill(w, stash=True)


def test_replay_at_the_largest_dim():
    w = inputs.replay_workload(active_batch=3, seq_len=4, nheads=2, dim=DIM_MAX, dstate=128,
                               ngroups=1, pool_rows=4, seed=75, accepted=[4, 0, 2])
    state0 = w["state"].clone()
    st = run_replay(w)
    st_ref = oracle_replay(w)
    idx = f64(w["state_indices"]).astype(int)
    stc = st.cpu()
    assert_close(stc[idx[[0, 2]]], st_ref[idx[[0, 2]]], TOL_F32, "replayed rows")
    assert_bitwise(stc[idx[1]], state0[idx[1]], "row with nothing accepted")


def test_tree_verify_at_the_largest_dim():
    w = inputs.tree_workload(batch=2, num_nodes=20, nheads=1, dim=DIM_MAX, dstate=128, ngroups=1,
                             pool_rows=2, seed=76, bc_std=128 ** -0.5, max_depth=5)
    _, out, S = run_tree(w, stash=True)
    out_ref, S_ref = oracle_tree(w, stash=True)
    assert_close(out.cpu(), out_ref, tol_for(out.dtype), "out")
    assert_close(S["replay_u"].cpu(), S_ref["u"], TOL_F32, "x stash")
