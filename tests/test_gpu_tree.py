"""GPU parity of ssu_tree_verify (tree speculative verify) and of ssu_replay with
accepted node ids against the fp64 oracle."""
import numpy as np
import pytest
import torch

from linear_rnn_recurrent_amd import inputs, ssu_replay
from gpu_helpers import (TOL_F32, TOL_LOW, assert_bitwise, assert_close, f64, gpu,
                         oracle_replay, oracle_tree, run_prefill, run_replay, run_tree, tol_for)

import oracle

pytestmark = pytest.mark.gpu


def check_tree(w, stash=True):
    state0 = w["state"].clone()
    st, out, S = run_tree(w, stash=stash)
    out_ref, S_ref = oracle_tree(w, stash=stash)
    assert_bitwise(st, state0, "the committed state is read-only")
    idx = w["state_indices"]
    nb = w.dims["batch"]
    live = np.ones(nb, dtype=bool) if idx is None else f64(idx) >= 0
    outc = out.cpu()
    assert_close(outc[live], out_ref[live], tol_for(outc.dtype), "out (live rows)")
    if (~live).any():
        z = outc[torch.from_numpy(~live)]
        assert_bitwise(z, torch.zeros_like(z), "out of padding rows (+0.0)")
    if stash:
        for k_gpu, k_ref in (("replay_dA", "dA"), ("replay_dt", "dt"), ("replay_u", "u"),
                             ("replay_B", "B")):
            got = S[k_gpu].cpu()
            assert_close(got[live], S_ref[k_ref][live], TOL_F32, k_gpu)
            if (~live).any():
                assert torch.isnan(got[torch.from_numpy(~live)]).all(), k_gpu + " of padding rows"
        for b in np.nonzero(live)[0]:
            assert_bitwise(S["replay_u"][b].cpu(), w["x"][b].float(), "replay_u")
            assert_bitwise(S["replay_B"][b].cpu(), w["B"][b].float(), "replay_B")
    return out, S


def test_tree_verify_full_budget_workload():
    check_tree(inputs.tree_config())


def test_tree_verify_64_node_trees():
    check_tree(inputs.tree_config(seed=6, num_nodes=64))


@pytest.mark.parametrize("dstate", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("state_dtype", ["f32", "f16", "bf16"])
def test_dstate_and_state_dtype_matrix(dstate, state_dtype):
    w = inputs.tree_workload(batch=3, num_nodes=21, nheads=4, dim=64, dstate=dstate, ngroups=2,
                             pool_rows=5, seed=dstate + 1, state_dtype=state_dtype,
                             bc_std=dstate ** -0.5, max_depth=6)
    check_tree(w)


@pytest.mark.parametrize("io_dtype,bc_dtype", [("f32", "f32"), ("f16", "f16"), ("bf16", "f32"),
                                               ("f32", "bf16"), ("f16", "bf16")])
def test_io_and_bc_dtypes(io_dtype, bc_dtype):
    w = inputs.tree_workload(batch=2, num_nodes=13, nheads=4, dim=64, dstate=128, ngroups=1,
                             pool_rows=3, seed=7, io_dtype=io_dtype, bc_dtype=bc_dtype,
                             bc_std=128 ** -0.5, with_z=True)
    check_tree(w)


@pytest.mark.parametrize("shape,dstate", [("chain", 128), ("chain", 256), ("star", 64),
                                          ("random", 256)])
def test_full_budget_shapes(shape, dstate):
    # 128-node chains hold 8256 path entries: the largest LDS footprint
    w = inputs.tree_workload(batch=2, num_nodes=128, nheads=3, dim=64, dstate=dstate,
                             ngroups=1, pool_rows=4, seed=dstate, shape=shape,
                             bc_std=dstate ** -0.5)
    check_tree(w)


def test_depth_bound_and_bad_parent_ids():
    w = inputs.tree_workload(batch=3, num_nodes=40, nheads=4, dim=64, dstate=64, ngroups=2,
                             pool_rows=4, seed=9, bc_std=0.125, max_depth=9)
    dep = w["depths"].clone()
    dep[0] = torch.clamp(dep[0] - 2, min=0)          # truncated walks
    dep[1, ::3] = -5                                 # negative bound: node alone
    dep[2] = 1000                                    # bound far above the depth
    w.tensors["depths"] = dep
    par = w["parent_ids"].clone()
    par[1, 7] = 7                                    # itself
    par[2, 11] = 30                                  # a later node
    par[2, 12] = -9                                  # any negative id is a root
    w.tensors["parent_ids"] = par
    check_tree(w)
    w.tensors["depths"] = None
    check_tree(w)


def test_padding_rows_and_optional_inputs():
    w = inputs.tree_workload(batch=5, num_nodes=17, nheads=4, dim=64, dstate=128, ngroups=1,
                             pool_rows=8, seed=10, indices=[6, -1, 2, -1, 4], with_z=True,
                             bc_std=128 ** -0.5)
    check_tree(w)
    for opts in (dict(with_z=False, with_D=False), dict(with_bias=False, dt_softplus=False),
                 dict(indices="none")):
        w = inputs.tree_workload(batch=3, num_nodes=11, nheads=4, dim=64, dstate=64, ngroups=1,
                                 pool_rows=3, seed=11, bc_std=0.125, **opts)
        if opts.get("dt_softplus") is False:
            w.tensors["dt"] = w["dt"].abs() * 0.1
        check_tree(w)


@pytest.mark.parametrize("dim", [32, 100, 200])
def test_row_blocks_and_ragged_dim(dim):
    w = inputs.tree_workload(batch=2, num_nodes=19, nheads=3, dim=dim, dstate=128, ngroups=1,
                             pool_rows=3, seed=dim, bc_std=128 ** -0.5, with_z=True)
    check_tree(w)


def test_single_node_and_tiny_trees():
    for m in (1, 2, 9):
        w = inputs.tree_workload(batch=2, num_nodes=m, nheads=2, dim=16, dstate=16, ngroups=1,
                                 pool_rows=2, seed=20 + m, bc_std=0.25)
        check_tree(w)


def test_chain_tree_equals_gpu_prefill():
    w = inputs.tree_workload(batch=3, num_nodes=24, nheads=8, dim=64, dstate=128, ngroups=2,
                             pool_rows=4, seed=12, shape="chain", bc_std=128 ** -0.5,
                             with_z=True)
    _, out_t, S_t = run_tree(w, stash=True)
    wp = inputs.Workload("chain as prefill", "prefill", dict(w.dims, seq_len=24),
                         dict(w.tensors, context_lengths=None), w.dt_softplus)
    _, out_p, S_p = run_prefill(wp, stash=True)
    # the tree kernel sums the path in closed form, the prefill steps through it
    assert_close(out_t.cpu(), f64(out_p), 2 * TOL_LOW, "chain tree vs prefill (bf16 outputs)")
    for k in S_t:
        assert_bitwise(S_t[k], S_p[k], "stash " + k)


def _accepted_paths(w, rng):
    """A root-first accepted path per row (a prefix of a random node's path)."""
    par = f64(w["parent_ids"])
    dep = f64(w["depths"])
    nb, m = par.shape
    paths = []
    for b in range(nb):
        node = int(rng.integers(m))
        chain = [node]
        while len(chain) <= dep[b, node] and 0 <= par[b, chain[-1]] < chain[-1]:
            chain.append(int(par[b, chain[-1]]))
        paths.append(chain[::-1])
    return paths


def test_commit_accepted_path_through_node_ids():
    w = inputs.tree_workload(batch=6, num_nodes=48, nheads=8, dim=64, dstate=128, ngroups=1,
                             pool_rows=8, seed=13, bc_std=128 ** -0.5, max_depth=7,
                             indices=[5, 0, -1, 7, 3, 1])
    _, _, S = run_tree(w, stash=True)
    _, S_ref = oracle_tree(w, stash=True)
    rng = np.random.default_rng(0)
    paths = _accepted_paths(w, rng)
    L = 8
    ids = np.zeros((6, L), dtype=np.int32)
    acc = np.zeros(6, dtype=np.int32)
    for b, p in enumerate(paths):
        ids[b, :len(p)] = p
        acc[b] = len(p) if b != 4 else 0
    state0 = w["state"].clone()
    st = gpu(w["state"]).clone()
    ssu_replay(st, S["replay_dA"], S["replay_u"], S["replay_B"], S["replay_dt"],
               torch.from_numpy(acc).cuda(), state_indices=gpu(w["state_indices"]),
               accepted_node_ids=torch.from_numpy(ids).cuda())
    st_ref = f64(state0).copy()
    oracle.replay(st_ref, S_ref["dA"], S_ref["u"], S_ref["B"], S_ref["dt"], acc,
                  state_indices=f64(w["state_indices"]), node_ids=ids)
    assert_close(st.cpu(), st_ref, TOL_F32, "state after the path commit")
    idx = f64(w["state_indices"])
    still = np.setdiff1d(np.arange(8), idx[(idx >= 0) & (acc > 0)])
    assert_bitwise(st.cpu()[still], state0[still], "rows with nothing committed")


@pytest.mark.parametrize("max_accept", [3, 7, 12])
@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
def test_node_id_replay(max_accept, state_dtype):
    w = inputs.replay_workload(active_batch=7, seq_len=16, nheads=4, dim=64, dstate=64,
                               ngroups=2, pool_rows=9, seed=max_accept, state_dtype=state_dtype,
                               accepted=[0, 1, 3, 5, 20, 12, 2, 0], stash_batch=8,
                               indices=[8, 1, 2, -1, 4, 5, 6, 0])
    rng = np.random.default_rng(max_accept)
    ids = np.stack([rng.permutation(16)[:max_accept] for _ in range(8)]).astype(np.int32)
    ids[5, min(2, max_accept - 1)] = 16        # outside the stash: the row stops there
    ids[6, 0] = -1                             # stops before the first token
    w.tensors["node_ids"] = torch.from_numpy(ids)
    state0 = w["state"].clone()
    st = run_replay(w)
    st_ref = oracle_replay(w)
    assert_close(st.cpu(), st_ref, tol_for(st.dtype), "state")
    assert_bitwise(st.cpu()[[3, 7]], state0[[3, 7]], "rows nobody addresses")
    assert_bitwise(st.cpu()[8], state0[8], "row with accepted = 0")
    assert_bitwise(st.cpu()[6], state0[6], "row whose first node id is outside the stash")


def test_identity_node_ids_equal_plain_replay_bitwise():
    w = inputs.replay_workload(active_batch=4, seq_len=6, nheads=8, dim=64, dstate=128,
                               ngroups=1, pool_rows=6, seed=51, accepted=[6, 2, 0, 4])
    st_plain = run_replay(w)
    w.tensors["node_ids"] = torch.arange(6, dtype=torch.int32).repeat(4, 1).contiguous()
    st_ids = run_replay(w)
    assert_bitwise(st_ids, st_plain, "identity node ids vs plain replay")
