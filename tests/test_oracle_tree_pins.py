"""Pins for the oracle's tree verify and node-id replay (CPU only).

Tree verify (TensorRT-Edge-LLM "Selective State Update" page,
invokeSelectiveStateUpdateDDTree) and the node-id form of the replay
(invokeMambaReplayReconstructBatched, acceptedNodeIds) are checked against
things other than the tree code itself:

* a chain tree is a prefill of the same tokens (outputs and stash);
* a star tree is one decode per node from the committed state;
* every node equals a prefill over the tokens of its own ancestor path, and
  the replay of that path through node ids gives the prefill's final state;
* a node depends on its ancestors only (perturbing any other node leaves it
  bitwise unchanged; perturbing an ancestor changes it);
* exact depths change nothing; zero depths turn the tree into a star;
* identity node ids are the plain replay; an id outside the stash ends the row;
* padding rows, read-only state;
* brute force against the pure-Python oracle, which writes each node's state in
  its unrolled form (a different formula from the C oracle's step-by-step path
  replay).

Plausible mistakes and the pin that catches each: walking the path node-first
instead of root-first (path == prefill), using the node's own B/C/x along the
path (path == prefill, golden T1), a missing decay of the committed state
(star == decode), off-by-one in the hop bound (golden T2, depths tests), sibling
leakage (ancestor-only), stash of the path instead of the node (chain == prefill
stash), node ids ignored by the replay (R5, path commit).
"""
import numpy as np
import pytest

import oracle
from oracle import ref_tiny
from linear_rnn_recurrent_amd import inputs


def _np(w):
    return {k: (None if v is None else v.double().numpy() if v.is_floating_point() else v.numpy())
            for k, v in w.tensors.items()}


def _stash(m, b, h, d, g, n):
    return {"dA": np.full((b, m, h), 7.0), "dt": np.full((b, m, h), 7.0),
            "u": np.full((b, m, h, d), 7.0), "B": np.full((b, m, g, n), 7.0)}


def _tree(a, impl=oracle, stash=False, **over):
    a = dict(a, **over)
    b, m, h, d = a["x"].shape
    out = np.full(a["x"].shape, 55.0)
    st = a["state"].copy()
    S = _stash(m, b, h, d, a["B"].shape[2], a["B"].shape[3]) if stash else None
    impl.tree(a["x"], a["A"], a["B"], a["C"], a["dt"], st, out, a["parent_ids"],
              depths=a.get("depths"), dt_bias=a.get("dt_bias"), D=a.get("D"), z=a.get("z"),
              dt_softplus=True, state_indices=a.get("state_indices"), stash=S)
    np.testing.assert_array_equal(st, a["state"])            # committed state read-only
    return out, S


def _prefill(a, stash=False, **over):
    a = dict(a, **over)
    b, t, h, d = a["x"].shape
    out = np.full(a["x"].shape, 66.0)
    st = a["state"].copy()
    S = _stash(t, b, h, d, a["B"].shape[2], a["B"].shape[3]) if stash else None
    oracle.prefill(a["x"], a["A"], a["B"], a["C"], a["dt"], st, out, dt_bias=a.get("dt_bias"),
                   D=a.get("D"), z=a.get("z"), state_indices=a.get("state_indices"), stash=S)
    return st, out, S


def _work(shape="random", seed=0, b=3, m=9, h=4, d=3, n=5, g=2, pool=5, **kw):
    kw.setdefault("with_z", True)
    return _np(inputs.tree_workload(batch=b, num_nodes=m, nheads=h, dim=d, dstate=n, ngroups=g,
                                    pool_rows=pool, seed=seed, state_dtype="f32", io_dtype="f32",
                                    bc_dtype="f32", bc_std=0.5, shape=shape, max_depth=4, **kw))


def test_chain_tree_is_prefill():
    a = _work("chain", seed=1)
    out_t, S_t = _tree(a, stash=True)
    _, out_p, S_p = _prefill(a, stash=True)
    np.testing.assert_allclose(out_t, out_p, rtol=1e-13, atol=1e-13)
    for k in S_t:
        np.testing.assert_array_equal(S_t[k], S_p[k])


def test_star_tree_is_one_decode_per_node():
    a = _work("star", seed=2)
    out_t, _ = _tree(a)
    for node in range(a["x"].shape[1]):
        st = a["state"].copy()
        out = np.zeros(a["x"][:, node].shape)
        oracle.decode(a["x"][:, node], a["A"], a["B"][:, node], a["C"][:, node], a["dt"][:, node],
                      st, out, dt_bias=a["dt_bias"], D=a["D"], z=a["z"][:, node],
                      state_indices=a["state_indices"])
        np.testing.assert_allclose(out_t[:, node], out, rtol=1e-13, atol=1e-13)


def _path(par, dep, b, node):
    chain = ref_tiny.ancestors(par, dep, b, node)
    return chain[::-1]                                       # root first


@pytest.mark.parametrize("seed", [3, 4])
def test_every_node_is_a_prefill_of_its_path(seed):
    a = _work("random", seed=seed, b=2, m=12)
    out_t, S_t = _tree(a, stash=True)
    for b in range(2):
        for node in range(12):
            p = _path(a["parent_ids"], a["depths"], b, node)
            sub = {k: (v[b:b + 1, p] if k in ("x", "z", "B", "C", "dt") else v) for k, v in a.items()}
            sub["state_indices"] = a["state_indices"][b:b + 1]
            st_p, out_p, _ = _prefill(sub)
            np.testing.assert_allclose(out_t[b, node], out_p[0, -1], rtol=1e-12, atol=1e-12)
            # committing the path from the tree's stash gives the prefill's final state
            st_r = a["state"].copy()
            ids = np.array([p + [0] * (12 - len(p))], dtype=np.int32)
            oracle.replay(st_r, S_t["dA"][b:b + 1], S_t["u"][b:b + 1], S_t["B"][b:b + 1],
                          S_t["dt"][b:b + 1], np.array([len(p)], dtype=np.int32),
                          state_indices=a["state_indices"][b:b + 1], node_ids=ids)
            np.testing.assert_allclose(st_r, st_p, rtol=1e-12, atol=1e-12)


def test_node_depends_on_its_ancestors_only():
    a = _work("random", seed=5, b=1, m=10)
    out0, _ = _tree(a)
    for node in range(10):
        anc = set(ref_tiny.ancestors(a["parent_ids"], a["depths"], 0, node))
        for other in range(10):
            pert = {k: v.copy() if isinstance(v, np.ndarray) else v for k, v in a.items()}
            for k in ("x", "B", "dt"):
                pert[k][0, other] += 0.75
            pert["C"][0, other] += 0.75 if other != node else 0.0
            out1, _ = _tree(pert)
            if other in anc:
                assert not np.array_equal(out1[0, node], out0[0, node]), (node, other)
            else:
                np.testing.assert_array_equal(out1[0, node], out0[0, node])


def test_exact_depths_change_nothing_and_zero_depths_make_a_star():
    a = _work("random", seed=6)
    out_d, _ = _tree(a)
    out_n, _ = _tree(a, depths=None)
    np.testing.assert_array_equal(out_d, out_n)
    out_0, _ = _tree(a, depths=np.zeros_like(a["depths"]))
    out_s, _ = _tree(a, parent_ids=np.full_like(a["parent_ids"], -1))
    np.testing.assert_array_equal(out_0, out_s)
    out_neg, _ = _tree(a, depths=np.full_like(a["depths"], -3))
    np.testing.assert_array_equal(out_neg, out_s)


def test_bad_parent_ids_end_the_walk():
    a = _work("chain", seed=7, b=1, m=6)
    par = a["parent_ids"].copy()
    par[0, 4] = 4          # itself
    par[0, 2] = 5          # a later node
    cut = a["parent_ids"].copy()
    cut[0, 4] = -1
    cut[0, 2] = -1
    out_bad, _ = _tree(a, parent_ids=par, depths=None)
    out_cut, _ = _tree(a, parent_ids=cut, depths=None)
    np.testing.assert_array_equal(out_bad, out_cut)


def test_node_id_replay_identity_and_early_stop():
    w = inputs.replay_workload(active_batch=3, seq_len=5, nheads=4, dim=3, dstate=4, ngroups=2,
                               pool_rows=4, seed=8, accepted=[5, 2, 4])
    a = _np(w)
    args = (a["replay_dA"], a["replay_u"], a["replay_B"], a["replay_dt"])
    st_plain = a["state"].copy()
    oracle.replay(st_plain, *args, a["accepted_lengths"], state_indices=a["state_indices"])
    st_ids = a["state"].copy()
    ident = np.tile(np.arange(5, dtype=np.int32), (3, 1))
    oracle.replay(st_ids, *args, a["accepted_lengths"], state_indices=a["state_indices"],
                  node_ids=ident)
    np.testing.assert_array_equal(st_ids, st_plain)
    # an id outside [0, seq_len) ends the row: same as accepting the tokens before it
    ids = ident.copy()
    ids[0, 3] = 5
    ids[2, 1] = -1
    st_stop = a["state"].copy()
    oracle.replay(st_stop, *args, a["accepted_lengths"], state_indices=a["state_indices"],
                  node_ids=ids)
    st_want = a["state"].copy()
    oracle.replay(st_want, *args, np.array([3, 2, 1], dtype=np.int32),
                  state_indices=a["state_indices"])
    np.testing.assert_array_equal(st_stop, st_want)
    # accepted beyond max_accept_len is clamped to it
    st_cap = a["state"].copy()
    oracle.replay(st_cap, *args, np.array([9, 9, 9], dtype=np.int32),
                  state_indices=a["state_indices"], node_ids=ident[:, :2].copy())
    st_two = a["state"].copy()
    oracle.replay(st_two, *args, np.array([2, 2, 2], dtype=np.int32),
                  state_indices=a["state_indices"])
    np.testing.assert_array_equal(st_cap, st_two)


def test_node_id_replay_order_matters():
    w = inputs.replay_workload(active_batch=1, seq_len=3, nheads=2, dim=2, dstate=4, ngroups=1,
                               pool_rows=2, seed=9, accepted=[3])
    a = _np(w)
    args = (a["replay_dA"], a["replay_u"], a["replay_B"], a["replay_dt"])
    st1 = a["state"].copy()
    oracle.replay(st1, *args, a["accepted_lengths"], state_indices=a["state_indices"],
                  node_ids=np.array([[2, 0, 1]], dtype=np.int32))
    st2 = a["state"].copy()
    ref_tiny.replay(st2, *args, a["accepted_lengths"], state_indices=a["state_indices"],
                    node_ids=np.array([[2, 0, 1]], dtype=np.int32))
    np.testing.assert_allclose(st1, st2, rtol=1e-13, atol=1e-13)
    st3 = a["state"].copy()
    oracle.replay(st3, *args, a["accepted_lengths"], state_indices=a["state_indices"])
    assert not np.allclose(st1, st3)


def test_padding_rows_and_stash_untouched():
    a = _work("random", seed=10, b=3, pool=6)
    a["state_indices"] = np.array([4, -1, 0], dtype=np.int32)
    out, S = _tree(a, stash=True)
    assert np.all(out[1] == 0.0) and not np.any(np.signbit(out[1]))
    for k in S:
        assert np.all(S[k][1] == 7.0), k
    assert np.all(np.isfinite(out))


@pytest.mark.parametrize("seed,shape,opts", [
    (11, "random", {}),
    (12, "chain", {"with_depths": False}),
    (13, "random", {"with_z": False, "with_D": False}),
    (14, "star", {"with_bias": False}),
])
def test_bruteforce_against_pure_python(seed, shape, opts):
    a = _work(shape, seed=seed, b=3, m=7, h=4, d=2, n=3, g=2, pool=4, **opts)
    if seed == 11:
        a["state_indices"][1] = -1
        a["depths"][0] = np.maximum(a["depths"][0] - 1, 0)   # truncated walks
        a["parent_ids"][2, 5] = 6                            # a bad id
    r = []
    for impl in (oracle, ref_tiny):
        out, S = _tree(a, impl=impl, stash=True)
        r.append([out] + [S[k] for k in ("dA", "u", "B", "dt")])
    for x, y in zip(*r):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# Layer-batched replay and clear (invokeMambaReplayReconstructBatched,
# invokeMambaStateClear)
# ---------------------------------------------------------------------------

def test_clear_layers_hand_case():
    """3 resident rows; recurrent rows of 8 bytes, conv rows of 5; layer 1 has no conv."""
    rec = [np.arange(1, 25, dtype=np.uint8), np.arange(101, 125, dtype=np.uint8)]
    conv = [np.arange(201, 216, dtype=np.uint8), None]
    oracle.clear_layers(rec, conv, 3, 1, 8, 5)
    for r0 in rec:
        assert np.all(r0[8:16] == 0) and np.all(r0[:8] != 0) and np.all(r0[16:] != 0)
    assert np.all(conv[0][5:10] == 0) and np.all(conv[0][:5] == np.arange(201, 206))
    assert np.all(conv[0][10:] == np.arange(211, 216))
    oracle.clear_layers(rec, conv, 3, -1, 8, 5)
    assert all(np.all(r0 == 0) for r0 in rec) and np.all(conv[0] == 0)


def test_replay_layers_is_one_replay_per_layer():
    ws = [inputs.replay_workload(active_batch=3, seq_len=4, nheads=2, dim=3, dstate=4, ngroups=1,
                                 pool_rows=4, seed=60 + i, accepted=[4, 1, 0],
                                 indices=[2, 0, 3]) for i in range(3)]
    arrs = [_np(w) for w in ws]
    acc = arrs[0]["accepted_lengths"]
    idx = arrs[0]["state_indices"]
    states = [a["state"].copy() for a in arrs]
    stashes = [{"dA": a["replay_dA"], "u": a["replay_u"], "B": a["replay_B"], "dt": a["replay_dt"]}
               for a in arrs]
    oracle.replay_layers(states, stashes, acc, state_indices=idx)
    for a, st in zip(arrs, states):
        want = a["state"].copy()
        ref_tiny.replay(want, a["replay_dA"], a["replay_u"], a["replay_B"], a["replay_dt"], acc,
                        state_indices=idx)
        np.testing.assert_allclose(st, want, rtol=1e-13, atol=1e-13)
