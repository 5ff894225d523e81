"""GPU parity of the layer-batched entry points (ssu_replay_layers,
ssu_state_clear_layers) against the fp64 oracle, and against the single-layer
entry points they batch."""
import numpy as np
import pytest
import torch

import oracle
from linear_rnn_recurrent_amd import (ReplayLayerTable, StateLayerTable, inputs, ssu_replay,
                                      ssu_replay_layers, ssu_state_clear_layers)
from gpu_helpers import assert_bitwise, assert_close, f64, gpu, tol_for

pytestmark = pytest.mark.gpu


def _layers(n, state_dtype="f32", **kw):
    base = dict(active_batch=6, seq_len=5, nheads=4, dim=64, dstate=64, ngroups=2, pool_rows=9,
                state_dtype=state_dtype, accepted=[5, 0, 3, 9, 1, 2, 0], stash_batch=7,
                indices=[8, 1, -1, 4, 2, 6, 0])
    base.update(kw)
    return [inputs.replay_workload(seed=100 + i, **base) for i in range(n)]


def _table(ws):
    T = [{k: gpu(v) for k, v in w.tensors.items()} for w in ws]
    table = ReplayLayerTable([t["state"] for t in T], [t["replay_dA"] for t in T],
                             [t["replay_u"] for t in T], [t["replay_B"] for t in T],
                             [t["replay_dt"] for t in T])
    return T, table


def _oracle(ws, active, ids=None):
    arrs = [{k: f64(v) for k, v in w.tensors.items()} for w in ws]
    states = [a["state"].copy() for a in arrs]
    stashes = [{"dA": a["replay_dA"], "u": a["replay_u"], "B": a["replay_B"], "dt": a["replay_dt"]}
               for a in arrs]
    oracle.replay_layers(states, stashes, arrs[0]["accepted_lengths"],
                         state_indices=arrs[0]["state_indices"], active_batch=active,
                         node_ids=ids)
    return states


@pytest.mark.parametrize("state_dtype", ["f32", "f16", "bf16"])
def test_replay_layers_matches_oracle_and_single_layer_calls(state_dtype):
    ws = _layers(5, state_dtype)
    state0 = [w["state"].clone() for w in ws]
    T, table = _table(ws)
    acc = T[0]["accepted_lengths"]
    idx = T[0]["state_indices"]
    ssu_replay_layers(table, acc, state_indices=idx, active_batch=6)
    ref = _oracle(ws, 6)
    for i, t in enumerate(T):
        assert_close(t["state"].cpu(), ref[i], tol_for(t["state"].dtype), f"layer {i} state")
        # the same layer through the single-layer entry point: bitwise equal
        single = gpu(state0[i]).clone()
        ssu_replay(single, t["replay_dA"], t["replay_u"], t["replay_B"], t["replay_dt"], acc,
                   state_indices=idx, active_batch=6)
        assert_bitwise(t["state"], single, f"layer {i}: batched vs single-layer replay")
        # pool rows 3, 5, 7 are not addressed; row 0 belongs to the poisoned entry 6
        assert_bitwise(t["state"].cpu()[[0, 3, 5, 7]], state0[i][[0, 3, 5, 7]], "untouched rows")


def test_replay_layers_with_node_ids_and_long_stash():
    ws = _layers(3, seq_len=12)
    T, table = _table(ws)
    rng = np.random.default_rng(5)
    ids = np.stack([rng.permutation(12)[:6] for _ in range(7)]).astype(np.int32)
    ids[3, 2] = 12  # outside the stash: that row stops after two tokens
    ssu_replay_layers(table, T[0]["accepted_lengths"], state_indices=T[0]["state_indices"],
                      active_batch=6, accepted_node_ids=torch.from_numpy(ids).cuda())
    ref = _oracle(ws, 6, ids)
    for i, t in enumerate(T):
        assert_close(t["state"].cpu(), ref[i], tol_for(t["state"].dtype), f"layer {i} state")


def test_replay_layers_full_size_two_layers():
    ws = [inputs.replay_workload(active_batch=32, seq_len=4, nheads=80, dim=64, dstate=128,
                                 ngroups=1, pool_rows=48, seed=200 + i, accepted=("uniform", 0, 4))
          for i in range(2)]
    for w in ws[1:]:  # shared accepted lengths and indices, per-layer stash and state
        w.tensors["accepted_lengths"] = ws[0]["accepted_lengths"]
        w.tensors["state_indices"] = ws[0]["state_indices"]
    T, table = _table(ws)
    ssu_replay_layers(table, T[0]["accepted_lengths"], state_indices=T[0]["state_indices"])
    ref = _oracle(ws, 32)
    for i, t in enumerate(T):
        assert_close(t["state"].cpu(), ref[i], tol_for(t["state"].dtype), f"layer {i} state")


def _byte_buffers(n_layers, rows, rb, cb, seed, conv_none=()):
    rng = np.random.default_rng(seed)
    rec = [rng.integers(1, 256, rows * rb, dtype=np.uint8) for _ in range(n_layers)]
    conv = [None if i in conv_none else rng.integers(1, 256, rows * cb + 3, dtype=np.uint8)
            for i in range(n_layers)]
    return rec, conv


@pytest.mark.parametrize("slot", [0, 3, 6, -1])
def test_state_clear_layers(slot):
    rows, rb, cb = 7, 80 * 64 * 128 * 4 // 64, 30   # conv rows of 30 bytes: unaligned rows
    rec, conv = _byte_buffers(4, rows, rb, cb, seed=slot + 10, conv_none=(2,))
    # a misaligned conv base too: layer 3's conv starts 3 bytes into its allocation
    g_rec = [torch.from_numpy(r.copy()).cuda() for r in rec]
    g_conv = [None if c is None else torch.from_numpy(c.copy()).cuda() for c in conv]
    views = [None if c is None else (c[3:] if i == 3 else c[:rows * cb]) for i, c in enumerate(g_conv)]
    table = StateLayerTable(g_rec, views)
    ssu_state_clear_layers(table, rows, slot, rb, cb)
    ref_conv = [None if c is None else c.copy() for c in conv]
    ref_views = [None if c is None else (c[3:] if i == 3 else c[:rows * cb]) for i, c in enumerate(ref_conv)]
    oracle.clear_layers(rec, ref_views, rows, slot, rb, cb)
    torch.cuda.synchronize()
    for i in range(4):
        np.testing.assert_array_equal(g_rec[i].cpu().numpy(), rec[i], err_msg=f"recurrent {i}")
        if conv[i] is not None:
            np.testing.assert_array_equal(g_conv[i].cpu().numpy(), ref_conv[i], err_msg=f"conv {i}")


def test_layer_batched_calls_in_graph_match_eager():
    ws = _layers(3)
    T, table = _table(ws)
    state0 = [t["state"].clone() for t in T]
    rows, rb = 5, 4096
    rec = [torch.randint(1, 255, (rows * rb,), dtype=torch.uint8, device="cuda") for _ in range(3)]
    rec0 = [r.clone() for r in rec]
    ctable = StateLayerTable(rec, [None] * 3)

    def run():
        ssu_replay_layers(table, T[0]["accepted_lengths"], state_indices=T[0]["state_indices"],
                          active_batch=6)
        ssu_state_clear_layers(ctable, rows, 2, rb, 0)

    run()
    torch.cuda.synchronize()
    want = [t["state"].clone() for t in T] + [r.clone() for r in rec]
    g = torch.cuda.CUDAGraph()
    for t, s0 in zip(T, state0):
        t["state"].copy_(s0)
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        for t, s0 in zip(T, state0):
            t["state"].copy_(s0)
        for r, r0 in zip(rec, rec0):
            r.copy_(r0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t["state"] for t in T] + rec
        for i, (a, e) in enumerate(zip(got, want)):
            assert_bitwise(a, e, f"tensor {i} after replay {rep}")
