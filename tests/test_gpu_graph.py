"""The C-ABI entry points launch asynchronously on the caller's stream with no
allocation or synchronisation, so they can be recorded in a HIP graph. Each test
captures a sequence of calls, replays it several times with eager work and
synchronisations between the replays, and checks every replay against the same
calls run eagerly."""
import pytest
import torch

from linear_rnn_recurrent_amd import (SsuPool, inputs, ssu_decode, ssu_prefill, ssu_replay,
                                      ssu_tree_verify)
from gpu_helpers import assert_bitwise, gpu

pytestmark = pytest.mark.gpu


def _decode_inputs(seed):
    w = inputs.decode_workload(batch=8, nheads=16, dim=64, dstate=128, ngroups=2, pool_rows=12,
                               seed=seed, indices=[3, 0, -1, 7, 11, 5, -1, 9],
                               bc_std=128 ** -0.5)
    return w, {k: gpu(v) for k, v in w.tensors.items()}


def test_decode_sequence_in_graph_matches_eager_on_every_replay():
    w, T = _decode_inputs(101)
    steps = 3
    # eager reference: `steps` decodes from the initial pool, per replay round
    st_ref = T["state"].clone()
    out_ref = torch.empty_like(T["x"])
    st_g = T["state"].clone()
    out_g = torch.empty_like(T["x"])

    def run(st, out):
        for _ in range(steps):
            ssu_decode(T["x"], T["A"], T["B"], T["C"], T["dt"], st, out, dt_bias=T["dt_bias"],
                       D=T["D"], z=T["z"], state_indices=T["state_indices"])

    run(st_g, out_g)                   # warm up (and cache device attributes) eagerly
    st_g.copy_(T["state"])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(st_g, out_g)
    torch.cuda.synchronize()
    for rep in range(4):
        st_g.copy_(T["state"])         # eager work between replays
        st_ref.copy_(T["state"])
        torch.cuda.synchronize()
        g.replay()
        run(st_ref, out_ref)
        torch.cuda.synchronize()
        assert_bitwise(st_g, st_ref, f"state after replay {rep}")
        assert_bitwise(out_g, out_ref, f"out after replay {rep}")


def test_prefill_replay_and_pool_ops_in_graph_match_eager():
    w = inputs.prefill_workload(batch=4, seq_len=13, nheads=8, dim=64, dstate=64, ngroups=1,
                                pool_rows=6, seed=102, ctx=[13, 5, 0, 9], bc_std=0.125)
    T = {k: gpu(v) for k, v in w.tensors.items()}
    b, t, h, d = T["x"].shape
    acc = torch.tensor([4, 2, 0, 9], dtype=torch.int32, device="cuda")
    pool = SsuPool([(0, 0, (h, d, 64), torch.float32)], 6)
    saved = [torch.empty((1, h, d, 64), device="cuda")]

    def run(st, out, S):
        ssu_prefill(T["x"], T["A"], T["B"], T["C"], T["dt"], st, out, dt_bias=T["dt_bias"],
                    D=T["D"], z=T["z"], context_lengths=T["context_lengths"],
                    state_indices=T["state_indices"], replay_dA=S[0], replay_u=S[1],
                    replay_B=S[2], replay_dt=S[3])
        ssu_replay(st, S[0], S[1], S[2], S[3], acc, state_indices=T["state_indices"])
        pool.clear_slot(2)
        pool.capture(1, saved)

    def bufs():
        return [torch.zeros((b, t, h), device="cuda"), torch.zeros((b, t, h, d), device="cuda"),
                torch.zeros(tuple(T["B"].shape), device="cuda"), torch.zeros((b, t, h), device="cuda")]

    st_g, out_g, S_g = T["state"].clone(), torch.empty_like(T["x"]), bufs()
    run(st_g, out_g, S_g)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(st_g, out_g, S_g)
    torch.cuda.synchronize()
    for rep in range(3):
        st_g.copy_(T["state"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [st_g.clone(), out_g.clone()] + [s.clone() for s in S_g] + [saved[0].clone()]
        st_e, out_e, S_e = T["state"].clone(), torch.empty_like(T["x"]), bufs()
        run(st_e, out_e, S_e)
        torch.cuda.synchronize()
        want = [st_e, out_e] + S_e + [saved[0]]
        for i, (a, e) in enumerate(zip(got, want)):
            assert_bitwise(a, e, f"tensor {i} after replay {rep}")


def test_tree_verify_and_path_commit_in_graph_match_eager():
    # 128-node trees need more than 64 KiB of LDS: the first (eager) call enables it
    w = inputs.tree_workload(batch=3, num_nodes=128, nheads=4, dim=64, dstate=128, ngroups=1,
                             pool_rows=4, seed=103, indices=[2, -1, 0], bc_std=128 ** -0.5)
    T = {k: gpu(v) for k, v in w.tensors.items()}
    b, m, h, d = T["x"].shape
    acc = torch.tensor([3, 2, 4], dtype=torch.int32, device="cuda")
    ids = torch.tensor([[0, 1, 5, 9], [0, 2, 0, 0], [0, 3, 7, 200]], dtype=torch.int32,
                       device="cuda")

    def run(st, out, S):
        ssu_tree_verify(T["x"], T["A"], T["B"], T["C"], T["dt"], st, out, T["parent_ids"],
                        depths=T["depths"], dt_bias=T["dt_bias"], D=T["D"],
                        state_indices=T["state_indices"], replay_dA=S[0], replay_u=S[1],
                        replay_B=S[2], replay_dt=S[3])
        ssu_replay(st, S[0], S[1], S[2], S[3], acc, state_indices=T["state_indices"],
                   accepted_node_ids=ids)

    def bufs():
        return [torch.zeros((b, m, h), device="cuda"), torch.zeros((b, m, h, d), device="cuda"),
                torch.zeros(tuple(T["B"].shape), device="cuda"), torch.zeros((b, m, h), device="cuda")]

    st_g, out_g, S_g = T["state"].clone(), torch.zeros_like(T["x"]), bufs()
    run(st_g, out_g, S_g)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(st_g, out_g, S_g)
    torch.cuda.synchronize()
    for rep in range(3):
        st_g.copy_(T["state"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [st_g.clone(), out_g.clone()] + [s.clone() for s in S_g]
        st_e, out_e, S_e = T["state"].clone(), torch.zeros_like(T["x"]), bufs()
        run(st_e, out_e, S_e)
        torch.cuda.synchronize()
        want = [st_e, out_e] + S_e
        for i, (a, e) in enumerate(zip(got, want)):
            assert_bitwise(a, e, f"tensor {i} after replay {rep}")
