"""GPU parity of ssu_gdn_decode (fused gated-delta-rule decode step) against the
fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from linear_rnn_recurrent_amd import inputs, ssu_gdn_decode
from gpu_helpers import TOL_F32, TOL_LOW, assert_bitwise, assert_close, gpu

pytestmark = pytest.mark.gpu


def _f64(t):
    a = t.detach().cpu()
    a = a.double() if a.is_floating_point() else a
    return np.ascontiguousarray(a.numpy())


def run_gdn(w, **over):
    T = {k: gpu(v) for k, v in w.tensors.items()}
    T.update(over)
    if w.tensors["conv_state"].is_contiguous() is False and "conv_state" not in over:
        # keep the strided (SD) view: rebuild it on the device from its pool
        base = w.tensors["conv_state"].transpose(1, 2).contiguous().cuda()
        T["conv_state"] = base.transpose(1, 2)
    d = w.dims
    out = ssu_gdn_decode(T["hidden_states"], T["w_ba"], T["mixed_qkv"], T["conv_weight"],
                         T["conv_bias"], T["conv_state"], T["A_log"], T["dt_bias"], d["scale"],
                         T["ssm_state"], T["state_indices"], num_q_heads=d["num_q_heads"],
                         use_qk_l2norm=d["use_qk_l2norm"])
    return out, T["conv_state"], T["ssm_state"]


def oracle_gdn(w):
    a = {k: _f64(v) for k, v in w.tensors.items()}
    d = w.dims
    out = oracle.gdn_decode(a["hidden_states"], a["w_ba"], a["mixed_qkv"], a["conv_weight"],
                            a["conv_bias"], a["conv_state"], a["A_log"], a["dt_bias"], d["scale"],
                            a["ssm_state"], a["state_indices"], num_q_heads=d["num_q_heads"],
                            use_qk_l2norm=d["use_qk_l2norm"])
    return out, a["conv_state"], a["ssm_state"]


def check_gdn(w):
    cs0 = w["conv_state"].clone()
    st0 = w["ssm_state"].clone()
    out, cs, st = run_gdn(w)
    out_r, cs_r, st_r = oracle_gdn(w)
    idx = w["state_indices"].numpy()
    live = idx >= 0
    outc = out.cpu()
    assert_close(outc[torch.from_numpy(live)], out_r[live], TOL_LOW, "out (live entries)")
    if (~live).any():
        zz = outc[torch.from_numpy(~live)]
        assert_bitwise(zz, torch.zeros_like(zz), "out of padding entries")
    rows = idx[live]
    stc = st.cpu()
    assert_close(stc[rows], st_r[rows], TOL_F32, "ssm_state (addressed slots)")
    # the conv pool holds raw bf16 inputs: its shift is exact
    csc = cs.cpu()
    if csc.numel():  # width 1 keeps no taps
        assert_bitwise(csc.contiguous(), torch.from_numpy(cs_r).to(torch.bfloat16).contiguous(),
                       "conv_state")
    free = np.setdiff1d(np.arange(stc.shape[0]), rows)
    if free.size:
        assert_bitwise(stc[free], st0[free], "ssm_state (slots nobody addresses)")
        if csc.numel():
            assert_bitwise(csc[free].contiguous(), cs0[free].contiguous(),
                           "conv_state (free slots)")
    return out


def test_qwen_shaped_layer_full_size():
    check_gdn(inputs.gdn_config())


@pytest.mark.parametrize("head_dim", [32, 64, 128, 256])
@pytest.mark.parametrize("hq,hv", [(2, 2), (2, 4), (1, 4), (1, 8)])
def test_head_dim_and_gqa(head_dim, hq, hv):
    w = inputs.gdn_workload(batch=3, hidden=96, num_q_heads=hq, num_v_heads=hv,
                            head_dim=head_dim, conv_width=4, pool_rows=5, seed=head_dim + hv)
    check_gdn(w)


@pytest.mark.parametrize("width", [1, 2, 3, 4, 8])
def test_conv_widths(width):
    w = inputs.gdn_workload(batch=2, hidden=64, num_q_heads=2, num_v_heads=4, head_dim=64,
                            conv_width=width, pool_rows=3, seed=width)
    check_gdn(w)


def test_sd_layout_padding_and_options():
    w = inputs.gdn_workload(batch=5, hidden=130, num_q_heads=2, num_v_heads=4, head_dim=128,
                            conv_width=4, pool_rows=8, seed=11, conv_layout="sd",
                            indices=[6, -1, 2, 0, -1])
    check_gdn(w)
    w = inputs.gdn_workload(batch=3, hidden=64, num_q_heads=2, num_v_heads=2, head_dim=64,
                            conv_width=4, pool_rows=4, seed=12, use_qk_l2norm=False, scale=0.3,
                            ssm_std=0.01)
    check_gdn(w)


def test_width4_dense_pool_off_word_alignment():
    # a dense width-4 pool whose taps are not 4-byte aligned takes the per-channel
    # conv path (aligned ones move channel pairs as 32-bit words)
    w = inputs.gdn_workload(batch=3, hidden=64, num_q_heads=2, num_v_heads=4, head_dim=64,
                            conv_width=4, pool_rows=4, seed=15, indices=[2, -1, 0])
    cs = w["conv_state"]
    flat = torch.empty(cs.numel() + 1, dtype=cs.dtype, device="cuda")
    view = flat[1:].view(cs.shape)
    view.copy_(cs.cuda())
    out, csg, st = run_gdn(w, conv_state=view)
    out_r, cs_r, st_r = oracle_gdn(w)
    idx = w["state_indices"].numpy()
    live = idx >= 0
    assert_close(out.cpu()[torch.from_numpy(live)], out_r[live], TOL_LOW, "out (live entries)")
    assert_close(st.cpu()[idx[live]], st_r[idx[live]], TOL_F32, "ssm_state")
    assert_bitwise(csg.cpu().contiguous(), torch.from_numpy(cs_r).to(torch.bfloat16).contiguous(),
                   "conv_state")


def test_padded_ssm_row_stride():
    w = inputs.gdn_workload(batch=3, hidden=64, num_q_heads=1, num_v_heads=2, head_dim=64,
                            conv_width=4, pool_rows=4, seed=13)
    st = w["ssm_state"]
    big = torch.full((4, 2 * 64 * 64 + 64), -7.0)
    big[:, : 2 * 64 * 64] = st.reshape(4, -1)
    gbig = big.cuda()
    gview = gbig.as_strided((4, 2, 64, 64), (2 * 64 * 64 + 64, 64 * 64, 64, 1))
    out, _, _ = run_gdn(w, ssm_state=gview)
    out_r, _, st_r = oracle_gdn(w)
    assert_close(out.cpu(), out_r, TOL_LOW, "out")
    got = gbig.cpu()
    assert_close(got[:, : 2 * 64 * 64].reshape(4, 2, 64, 64)[w["state_indices"].long()],
                 st_r[w["state_indices"].numpy()], TOL_F32, "ssm_state")
    assert torch.all(got[:, 2 * 64 * 64:] == -7.0)


def test_gdn_in_graph_matches_eager():
    w = inputs.gdn_workload(batch=4, hidden=64, num_q_heads=2, num_v_heads=4, head_dim=64,
                            conv_width=4, pool_rows=6, seed=14, indices=[5, -1, 0, 3])
    T = {k: gpu(v) for k, v in w.tensors.items()}
    cs0, st0 = T["conv_state"].clone(), T["ssm_state"].clone()
    out = torch.empty((4, 1, 4, 64), dtype=torch.bfloat16, device="cuda")

    def run():
        ssu_gdn_decode(T["hidden_states"], T["w_ba"], T["mixed_qkv"], T["conv_weight"],
                       T["conv_bias"], T["conv_state"], T["A_log"], T["dt_bias"], None,
                       T["ssm_state"], T["state_indices"], num_q_heads=2, out=out)

    run()
    run()
    torch.cuda.synchronize()
    want = [out.clone(), T["conv_state"].clone(), T["ssm_state"].clone()]
    g = torch.cuda.CUDAGraph()
    T["conv_state"].copy_(cs0)
    T["ssm_state"].copy_(st0)
    with torch.cuda.graph(g):
        run()
        run()
    for rep in range(3):
        T["conv_state"].copy_(cs0)
        T["ssm_state"].copy_(st0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, e) in enumerate(zip([out, T["conv_state"], T["ssm_state"]], want)):
            assert_bitwise(a, e, f"tensor {i} after replay {rep}")
