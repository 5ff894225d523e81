"""Strong and extreme decays on the GPU.

The selective state update with a strongly negative A*dt' has a closed form:
exp(A*dt') underflows to zero, so the state collapses to B*dt'*x of the last
token and each output to (x*(B.C)*dt' + D*x), gated (TensorRT-Edge-LLM,
"Selective State Update" page, the decode step of invokeSelectiveStateUpdate
with the decay term gone). Every kernel is run in that regime and compared
both with the fp64 oracle and with the closed form written out here.

The prefill kernels are also driven through every branch of their decay
handling: the rescaled VALU recurrence renormalises once when the running
product of decays leaves [1e-30, 1e30], walks a chunk token by token when the
product leaves that range inside the chunk, and applies a single decay below
1e-30 directly; the matrix-core kernel forms Q entry by entry when a 4-token
quad spans more than 2^64 of decay. Heads below take A*dt' of about -1e4,
-40, -10, -1 and isolated -100 tokens among mild ones (dt' stays <= 2 so that
the state stays O(1) and the outputs are well conditioned in fp32).
"""
import numpy as np
import pytest
import torch

import oracle
from linear_rnn_recurrent_amd import inputs, ssu_prefill, ssu_replay
from gpu_helpers import (TOL_F32, assert_close, f64, gpu, oracle_decode, oracle_prefill,
                         oracle_replay, oracle_tree, run_decode, run_prefill, run_replay,
                         run_tree, tol_for)
from test_gpu_prefill import check_prefill, valu_kernel

pytestmark = pytest.mark.gpu

COLLAPSE_A = -1.0e4  # with dt' = 1: exp(-1e4) is 0 in fp32 and in fp64


def silu(v):
    return v / (1.0 + np.exp(-v))


def strong_prefill_workload(io, bc, state_dtype="f32", seed=61, seq_len=130):
    """Six heads, one decay regime each (softplus off, no bias: dt' = dt)."""
    w = inputs.prefill_workload(batch=4, seq_len=seq_len, nheads=6, dim=64, dstate=128,
                                ngroups=2, pool_rows=6, seed=seed, state_dtype=state_dtype,
                                io_dtype=io, bc_dtype=bc, bc_std=128 ** -0.5,
                                ctx=[seq_len, seq_len - 33, 64, 33], with_bias=False,
                                dt_softplus=False)
    rng = np.random.default_rng(seed + 1000)
    b, t = w.dims["batch"], seq_len
    dt = rng.uniform(0.5, 1.5, (b, t, 6))
    A = np.array([COLLAPSE_A, -40.0, -10.0, -1.0, -50.0, 0.0])
    dt[:, :, 0] = 1.0                         # -1e4 per token: the collapse
    dt[:, :, 1] = 1.0                         # -40 per token
    dt[:, :, 4] *= 1e-3                       # -0.05 per token, and
    dt[:, 5::37, 4] = 2.0                     # an isolated -100 token every 37
    A[5] = float(w["A"][5])                   # the benchmark recipe's decay
    dt[:, :, 5] = np.exp(rng.uniform(np.log(4e-4), np.log(0.33), (b, t)))
    w.tensors["A"] = torch.from_numpy(A.astype(np.float32))
    w.tensors["dt"] = torch.from_numpy(dt.astype(np.float32))
    return w


def check_collapsed_head_state(w, st, head=0):
    """Closed form: after the last token the collapse head holds B_last x_last^T."""
    L = np.clip(f64(w["context_lengths"]), 0, w.dims["seq_len"]).astype(int)
    idx = f64(w["state_indices"])
    g = head // (w.dims["nheads"] // w.dims["ngroups"])
    stc = f64(st)
    for b in range(w.dims["batch"]):
        if L[b] == 0 or idx[b] < 0:
            continue
        x = f64(w["x"])[b, L[b] - 1, head]
        Bv = f64(w["B"])[b, L[b] - 1, g]
        want = np.outer(x, Bv)
        assert_close(stc[int(idx[b]), head], want, tol_for(st.dtype),
                     f"collapsed state of row {b} (B x of its last token)")


def check_collapsed_head_out(w, out, head=0):
    """Closed form of the collapse head's outputs: (x (B.C) + D x) silu(z)."""
    g = head // (w.dims["nheads"] // w.dims["ngroups"])
    x = f64(w["x"])[:, :, head]
    bc = np.einsum("btn,btn->bt", f64(w["B"])[:, :, g], f64(w["C"])[:, :, g])
    y = x * bc[:, :, None] + float(w["D"][head]) * x
    if w["z"] is not None:
        y = y * silu(f64(w["z"])[:, :, head])
    L = np.clip(f64(w["context_lengths"]), 0, w.dims["seq_len"]).astype(int)
    got = f64(out)[:, :, head]
    for b in range(w.dims["batch"]):
        assert_close(got[b, :L[b]], y[b, :L[b]], tol_for(out.dtype),
                     f"collapsed outputs of row {b}")


@pytest.mark.parametrize("io,bc,kernel", [("bf16", "bf16", "mm"), ("f16", "f16", "mm"),
                                          ("f32", "f32", "valu"), ("f16", "f16", "valu"),
                                          ("f32", "bf16", "valu")])
def test_prefill_decay_regimes(io, bc, kernel):
    # bf16/bf16 and fp16/fp16: the matrix-core kernel, or (fp16 x off 16-byte
    # alignment) the rescaled VALU recurrence, which also takes the other types
    w = strong_prefill_workload(io, bc)
    st, out, _ = check_prefill(w, **(valu_kernel(w) if kernel == "valu" else {}))
    check_collapsed_head_state(w, st.cpu())
    check_collapsed_head_out(w, out.cpu())


@pytest.mark.parametrize("io", ["bf16", "f16", "f32"])
def test_prefill_decay_regimes_fp16_state_and_stash(io):
    w = strong_prefill_workload(io, io, state_dtype="f16", seed=62)
    check_prefill(w)
    check_prefill(w, stash=True)


@pytest.mark.parametrize("io", ["bf16", "f16", "f32"])
def test_prefill_stash_then_replay_in_the_collapse(io):
    # the stash of an extreme-decay prefill replayed over the whole context
    # equals the plain prefill (the replay applies exp(dA) = 0 directly)
    w = strong_prefill_workload(io, io, seed=63)
    st_s, _, S = run_prefill(w, stash=True)
    acc = w["context_lengths"].clone()
    ssu_replay(st_s, S["replay_dA"], S["replay_u"], S["replay_B"], S["replay_dt"], gpu(acc),
               state_indices=gpu(w["state_indices"]))
    st_ref, _, _ = oracle_prefill(w)
    rows = f64(w["state_indices"]).astype(int)
    assert_close(st_s.cpu()[rows], st_ref[rows], TOL_F32, "stash + replay(ctx) vs oracle prefill")
    check_collapsed_head_state(w, st_s.cpu())


def test_prefill_long_sequences_on_the_valu_kernel_with_strong_decays():
    # 1100 tokens (137 staged chunks, many renormalisations), fp32 operands
    w = strong_prefill_workload("f32", "f32", seed=64, seq_len=1100)
    st, out, _ = check_prefill(w)
    check_collapsed_head_state(w, st.cpu())


@pytest.mark.parametrize("state_dtype,io", [("f32", "bf16"), ("f16", "bf16"), ("f32", "f32")])
def test_decode_collapse(state_dtype, io):
    w = inputs.decode_workload(batch=16, nheads=8, dim=64, dstate=128, ngroups=2, pool_rows=20,
                               seed=65, state_dtype=state_dtype, io_dtype=io, bc_dtype=io,
                               bc_std=128 ** -0.5, with_bias=False, dt_softplus=False)
    w.tensors["A"] = torch.full((8,), COLLAPSE_A)
    w.tensors["dt"] = torch.ones(16, 8)
    st, out = run_decode(w)
    st_ref, out_ref = oracle_decode(w)
    idx = f64(w["state_indices"]).astype(int)
    stc, outc = st.cpu(), out.cpu()
    assert_close(stc[idx], st_ref[idx], tol_for(stc.dtype), "state vs oracle")
    assert_close(outc, out_ref, tol_for(outc.dtype), "out vs oracle")
    # closed form, independent of the oracle
    x, Bm, Cm = f64(w["x"]), f64(w["B"]), f64(w["C"])
    g = np.arange(8) // 4
    want = np.einsum("bhd,bhn->bhdn", x, Bm[:, g])
    assert_close(stc[idx], want, tol_for(stc.dtype), "state = B x")
    y = (x * np.einsum("bhn,bhn->bh", Bm[:, g], Cm[:, g])[:, :, None]
         + f64(w["D"])[None, :, None] * x) * silu(f64(w["z"]))
    assert_close(outc, y, tol_for(outc.dtype), "out = (x (B.C) + D x) silu(z)")


@pytest.mark.parametrize("state_dtype", ["f32", "f16"])
def test_replay_collapse(state_dtype):
    w = inputs.replay_workload(active_batch=12, seq_len=4, nheads=8, dim=64, dstate=128,
                               ngroups=2, pool_rows=16, seed=66, state_dtype=state_dtype,
                               accepted=[0, 1, 2, 3, 4, 9, 1, 2, 3, 4, 4, 2])
    w.tensors["replay_dA"] = torch.full_like(w["replay_dA"], COLLAPSE_A)
    st = run_replay(w)
    st_ref = oracle_replay(w)
    acc = np.minimum(f64(w["accepted_lengths"]), 4).astype(int)
    idx = f64(w["state_indices"]).astype(int)
    moved = idx[acc > 0]
    stc = st.cpu()
    assert_close(stc[moved], st_ref[moved], tol_for(stc.dtype), "state vs oracle")
    g = np.arange(8) // 4
    for b in np.nonzero(acc > 0)[0]:
        k = acc[b] - 1  # the last applied token alone survives
        want = (f64(w["replay_dt"])[b, k][:, None, None] * f64(w["replay_u"])[b, k][:, :, None]
                * f64(w["replay_B"])[b, k][g][:, None, :])
        assert_close(stc[idx[b]], want, tol_for(stc.dtype), f"row {b}: state = DT u B")


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_tree_verify_collapse(io):
    # every node's output is its own step's alone: ancestors decay to nothing
    w = inputs.tree_workload(batch=4, num_nodes=40, nheads=8, dim=64, dstate=128, ngroups=2,
                             pool_rows=6, seed=67, io_dtype=io, bc_dtype=io, bc_std=128 ** -0.5,
                             max_depth=8, with_bias=False, dt_softplus=False)
    w.tensors["A"] = torch.full((8,), COLLAPSE_A)
    w.tensors["dt"] = torch.ones_like(w["dt"])
    _, out, S = run_tree(w, stash=True)
    out_ref, S_ref = oracle_tree(w, stash=True)
    outc = out.cpu()
    assert_close(outc, out_ref, tol_for(outc.dtype), "out vs oracle")
    x, Bm, Cm = f64(w["x"]), f64(w["B"]), f64(w["C"])
    g = np.arange(8) // 4
    bc = np.einsum("bmhn,bmhn->bmh", Bm[:, :, g], Cm[:, :, g])
    y = x * bc[..., None] + f64(w["D"])[None, None, :, None] * x
    assert_close(outc, y, tol_for(outc.dtype), "out = x (B.C) + D x")
    assert_close(S["replay_dA"].cpu(), S_ref["dA"], TOL_F32, "stash dA")


def test_strong_decay_prefill_equals_decode_steps_on_the_gpu():
    # the collapse heads of a short prefill against ssu_decode token by token
    from linear_rnn_recurrent_amd import ssu_decode
    w = strong_prefill_workload("bf16", "bf16", seed=68, seq_len=40)
    w.tensors["context_lengths"] = None
    T = {k: gpu(v) for k, v in w.tensors.items()}
    st_p, out_p, _ = run_prefill(w)
    st = T["state"].clone()
    for t in range(40):
        o = torch.empty_like(T["x"][:, t])
        ssu_decode(T["x"][:, t].contiguous(), T["A"], T["B"][:, t].contiguous(),
                   T["C"][:, t].contiguous(), T["dt"][:, t].contiguous(), st, o, D=T["D"],
                   z=T["z"][:, t].contiguous(), dt_softplus=False,
                   state_indices=T["state_indices"])
    assert_close(st_p.cpu(), f64(st), 2 * TOL_F32, "prefill vs repeated decode")
