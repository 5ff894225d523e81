"""Pins for the oracle's fused gated-delta-rule decode step (FlashInfer
"flashinfer.gdn_fused_decode_step" page; formulas in oracle/gdn_oracle.c).

* the delta rule writes v at key k: with no decay (A_log -> -inf), beta -> 1 and
  k = c e_j, column j of every state row becomes (1 - c^2) S + c v exactly and
  every other column is untouched;
* decay 1/2: exp(A_log) = ln 2 and softplus(a + dt_bias) = 1 halve the state
  (hand-derived constants, k = 0 so the update term vanishes);
* conv: the pool keeps the last W-1 raw inputs (exact shift); a tap pattern of
  [1, 0, .., 0] feeds the oldest input through silu;
* GQA: value heads 2h, 2h+1 read q/k head h only; scale is linear in the output;
  None and 0 select 1/sqrt(D);
* the DS and SD conv-pool layouts agree; padding entries touch nothing;
* brute force against the pure-Python oracle, which expands the update
  (o = alpha S q + delta k.q) instead of reading the updated row.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import ref_tiny
from linear_rnn_recurrent_amd import inputs


def _np(w):
    out = {}
    for k, v in w.tensors.items():
        a = v.double() if v.is_floating_point() else v
        out[k] = np.ascontiguousarray(a.numpy())
    return out


def _run(a, hq, **kw):
    cs = a["conv_state"].copy()
    st = a["ssm_state"].copy()
    out = oracle.gdn_decode(a["hidden_states"], a["w_ba"], a["mixed_qkv"], a["conv_weight"],
                            a["conv_bias"], cs, a["A_log"], a["dt_bias"], kw.pop("scale", None),
                            st, a["state_indices"], num_q_heads=hq, **kw)
    return out, cs, st


def _small(seed=0, hq=2, hv=4, d=4, w=3, pool=3, b=2, **kw):
    return _np(inputs.gdn_workload(batch=b, hidden=6, num_q_heads=hq, num_v_heads=hv, head_dim=d,
                                   conv_width=w, pool_rows=pool, seed=seed, ssm_std=1.0, **kw))


def test_delta_rule_writes_v_at_key():
    hq, hv, d, w = 1, 1, 4, 2
    a = _small(seed=1, hq=hq, hv=hv, d=d, w=w, pool=1, b=1, indices=[0])
    j = 2
    a["A_log"][:] = -1.0e4                     # exp(A_log) = 0: no decay
    a["hidden_states"][:] = 0.0
    a["hidden_states"][0, 0] = 1.0
    a["w_ba"][:] = 0.0
    a["w_ba"][0, 0] = 60.0                     # beta = sigmoid(60) = 1 in fp64
    a["conv_weight"][:] = 0.0
    a["conv_bias"][:] = 0.0
    a["conv_weight"][:, w - 1] = 1.0           # y_c = silu(x_new)
    x = np.zeros(3 * d)
    x[:d] = [0.3, -0.2, 0.5, 0.1]              # q
    x[d + j] = 50.0                            # k = c e_j after the norm
    x[2 * d:] = [1.5, -2.0, 0.25, 3.0]         # v
    a["mixed_qkv"][0] = x
    out, cs, st = _run(a, hq)
    silu = lambda t: t / (1.0 + math.exp(-t))
    yk = silu(50.0)
    c = yk / math.sqrt(yk * yk + 1e-6)
    v = np.array([silu(t) for t in x[2 * d:]])
    S0 = a["ssm_state"][0, 0]
    want = S0.copy()
    want[:, j] = (1.0 - c * c) * S0[:, j] + c * v
    np.testing.assert_allclose(st[0, 0], want, rtol=1e-14, atol=1e-14)
    others = [i for i in range(d) if i != j]
    np.testing.assert_array_equal(st[0, 0][:, others], S0[:, others])
    q = np.array([silu(t) for t in x[:d]])
    q = q / math.sqrt(np.sum(q * q) + 1e-6) / math.sqrt(d)
    np.testing.assert_allclose(out[0, 0, 0], want @ q, rtol=1e-13, atol=1e-14)


def test_decay_one_half_without_update():
    a = _small(seed=2, hq=1, hv=2, d=4, w=2, pool=2, b=1, indices=[1])
    a["A_log"][:] = math.log(math.log(2.0))    # exp(A_log) = ln 2
    a["hidden_states"][:] = 0.0                # a = b = 0
    a["dt_bias"][:] = math.log(math.e - 1.0)   # softplus(0 + dt_bias) = 1
    a["mixed_qkv"][0, 2:2 * 4] = 0.0           # zero k channels (q of the single q/k head
    a["conv_bias"][4:8] = 0.0                  # is channels 0..3, k 4..7): k = 0
    a["conv_weight"][4:8] = 0.0
    out, cs, st = _run(a, 1)
    np.testing.assert_allclose(st[1], 0.5 * a["ssm_state"][1], rtol=1e-15, atol=0)
    np.testing.assert_array_equal(st[0], a["ssm_state"][0])


def test_conv_pool_shift_and_oldest_tap():
    a = _small(seed=3, w=4)
    cs0 = a["conv_state"].copy()
    out, cs, st = _run(a, 2)
    for b, s in enumerate(a["state_indices"]):
        np.testing.assert_array_equal(cs[s, :, :2], cs0[s, :, 1:])
        np.testing.assert_array_equal(cs[s, :, 2], a["mixed_qkv"][b])
    untouched = sorted(set(range(3)) - set(a["state_indices"].tolist()))
    np.testing.assert_array_equal(cs[untouched], cs0[untouched])


def test_gqa_map_and_scale():
    a = _small(seed=4, hq=2, hv=4, d=4)
    out1, _, _ = _run(a, 2)
    b = {k: v.copy() for k, v in a.items()}
    b["mixed_qkv"][:, 4:8] += 0.7              # q head 1 only
    out2, _, _ = _run(b, 2)
    np.testing.assert_array_equal(out2[:, :, :2], out1[:, :, :2])
    assert not np.allclose(out2[:, :, 2:], out1[:, :, 2:])
    o_def, _, _ = _run(a, 2, scale=None)
    o_zero, _, _ = _run(a, 2, scale=0.0)
    o_half, _, _ = _run(a, 2, scale=1.0 / math.sqrt(4) * 2.0)
    np.testing.assert_array_equal(o_def, o_zero)
    np.testing.assert_allclose(o_half, 2.0 * o_def, rtol=1e-13, atol=1e-15)


def test_layouts_agree_and_padding():
    ds = inputs.gdn_workload(batch=3, hidden=8, num_q_heads=1, num_v_heads=2, head_dim=4,
                             conv_width=3, pool_rows=4, seed=5, indices=[2, -1, 0])
    a = _np(ds)
    out_ds, cs_ds, st_ds = _run(a, 1)
    # the same pool stored as [P, W-1, qkv] rows, seen through strides
    flat = np.ascontiguousarray(a["conv_state"].transpose(0, 2, 1)).ravel()
    P, C, T = a["conv_state"].shape
    st = a["ssm_state"].copy()
    out_sd = oracle.gdn_decode(a["hidden_states"], a["w_ba"], a["mixed_qkv"], a["conv_weight"],
                               a["conv_bias"], flat, a["A_log"], a["dt_bias"], None, st,
                               a["state_indices"], num_q_heads=1,
                               conv_strides=(T * C, 1, C))
    np.testing.assert_array_equal(out_sd, out_ds)
    np.testing.assert_array_equal(flat.reshape(P, T, C).transpose(0, 2, 1), cs_ds)
    np.testing.assert_array_equal(st, st_ds)
    assert np.all(out_ds[1] == 0.0)
    np.testing.assert_array_equal(cs_ds[[1, 3]], a["conv_state"][[1, 3]])
    np.testing.assert_array_equal(st_ds[[1, 3]], a["ssm_state"][[1, 3]])


@pytest.mark.parametrize("seed,l2", [(6, True), (7, False)])
def test_bruteforce_against_pure_python(seed, l2):
    a = _small(seed=seed, hq=2, hv=4, d=4, w=4, pool=3, b=3, indices=[2, -1, 0])
    out, cs, st = _run(a, 2, use_qk_l2norm=l2)
    cs2 = a["conv_state"].copy()
    st2 = a["ssm_state"].copy()
    out2 = ref_tiny.gdn_decode(a["hidden_states"], a["w_ba"], a["mixed_qkv"], a["conv_weight"],
                               a["conv_bias"], cs2, a["A_log"], a["dt_bias"], None, st2,
                               a["state_indices"], 2, use_qk_l2norm=l2)
    np.testing.assert_allclose(out, np.array(out2), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st, st2, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(cs, cs2)
