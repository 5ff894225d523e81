"""GPU parity of ssu_prefill (with contextLengths and the replay stash) against the
fp64 oracle, plus the prefill/decode/replay invariants on the GPU itself."""
import numpy as np
import pytest
import torch

from linear_rnn_recurrent_amd import inputs, ssu_decode, ssu_replay
from gpu_helpers import (TOL_F32, TOL_LOW, assert_bitwise, assert_close, f64, gpu,
                         oracle_prefill, run_prefill, tol_for, touched_rows, untouched_rows)

pytestmark = pytest.mark.gpu


def lengths(w):
    T = w.dims["seq_len"]
    cl = w["context_lengths"]
    if cl is None:
        return np.full(w.dims["batch"], T)
    return np.clip(f64(cl), 0, T)


def check_prefill(w, stash=False):
    state0 = w["state"].clone()
    st, out, S = run_prefill(w, stash=stash)
    st_ref, out_ref, S_ref = oracle_prefill(w, stash=stash)
    idx = w["state_indices"]
    nb = w.dims["batch"]
    stc = st.cpu()
    if stash:
        assert_bitwise(stc, state0, "state must stay read-only in stash mode")
    else:
        rows = touched_rows(idx, nb)
        assert_close(stc[rows], st_ref[rows], tol_for(stc.dtype), "state (addressed rows)")
        free = untouched_rows(idx, w.dims["pool_rows"], nb)
        if free.size:
            assert_bitwise(stc[free], state0[free], "state (rows not addressed)")
    live = np.ones(nb, dtype=bool) if idx is None else f64(idx) >= 0
    outc = out.cpu()
    assert_close(outc[live], out_ref[live], tol_for(outc.dtype), "out (live rows)")
    L = lengths(w)
    zero_mask = np.zeros(outc.shape[:2], dtype=bool)
    for b in range(nb):
        zero_mask[b, int(L[b]):] = True
        if not live[b]:
            zero_mask[b, :] = True
    if zero_mask.any():
        z = outc[torch.from_numpy(zero_mask)]
        assert_bitwise(z, torch.zeros_like(z), "out beyond the context / padding rows (+0.0)")
    if stash:
        for k_gpu, k_ref in (("replay_dA", "dA"), ("replay_dt", "dt"), ("replay_u", "u"),
                             ("replay_B", "B")):
            got = S[k_gpu].cpu()
            assert_close(got[live], S_ref[k_ref][live], TOL_F32, k_gpu)
        # u and B are exact copies of the inputs (upcast) inside the context
        for b in np.nonzero(live)[0]:
            Lb = int(L[b])
            assert_bitwise(S["replay_u"][b, :Lb].cpu(), w["x"][b, :Lb].float(), "replay_u")
            assert_bitwise(S["replay_B"][b, :Lb].cpu(), w["B"][b, :Lb].float(), "replay_B")
    return st, out, S


def test_config2_full_size():
    check_prefill(inputs.config(2))


def test_config2_stash_mode_full_size():
    check_prefill(inputs.config(2), stash=True)


@pytest.mark.parametrize("stash", [False, True])
@pytest.mark.parametrize("io", ["f32", "f16"])
def test_config2_shape_on_the_valu_kernel(io, stash):
    # config 2's shape and recipe with fp32 or fp16 x/z/B/C: the rescaled VALU
    # recurrence over up to 512 tokens, where the running product of decays
    # (sum of A dt' near -100 at full length) leaves [1e-30, 1e30] and the
    # state is renormalised at a chunk start
    w = inputs.prefill_workload(batch=8, seq_len=512, nheads=80, dim=64, dstate=128,
                                ngroups=1, pool_rows=64, seed=2, state_dtype="f32",
                                io_dtype=io, bc_dtype=io, bc_std=1.0 / np.sqrt(128),
                                ctx=("uniform", 64, 512), zero_state=True)
    check_prefill(w, stash=stash)


@pytest.mark.parametrize("dstate", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("state_dtype", ["f32", "f16", "bf16"])
def test_dstate_and_state_dtype_matrix(dstate, state_dtype):
    w = inputs.prefill_workload(batch=3, seq_len=37, nheads=4, dim=64, dstate=dstate,
                                ngroups=2, pool_rows=5, seed=dstate, state_dtype=state_dtype,
                                bc_std=dstate ** -0.5, ctx=[37, 20, 1])
    check_prefill(w)


@pytest.mark.parametrize("io_dtype,bc_dtype", [("f32", "f32"), ("f16", "f16"), ("bf16", "f32"),
                                               ("f32", "bf16"), ("f16", "bf16")])
def test_io_and_bc_dtypes(io_dtype, bc_dtype):
    w = inputs.prefill_workload(batch=2, seq_len=21, nheads=4, dim=64, dstate=128, ngroups=1,
                                pool_rows=3, seed=3, io_dtype=io_dtype, bc_dtype=bc_dtype,
                                bc_std=128 ** -0.5, ctx=("none",))
    check_prefill(w)


def test_ragged_context_lengths_and_padding():
    # ctx: zero, negative (clamped to 0), full, beyond seq_len (clamped), odd; one padding row
    w = inputs.prefill_workload(batch=6, seq_len=45, nheads=4, dim=64, dstate=64, ngroups=2,
                                pool_rows=8, seed=4, ctx=[0, -3, 45, 100, 17, 33],
                                indices=[5, 1, 7, 0, -1, 3], bc_std=0.125)
    check_prefill(w)
    check_prefill(w, stash=True)


@pytest.mark.parametrize("dim", [32, 100, 200])
def test_row_blocks_and_ragged_dim(dim):
    w = inputs.prefill_workload(batch=2, seq_len=19, nheads=3, dim=dim, dstate=128, ngroups=1,
                                pool_rows=4, seed=dim, bc_std=128 ** -0.5, ctx=[19, 11])
    check_prefill(w)
    check_prefill(w, stash=True)


@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
def test_chunk_boundaries(state_dtype):
    # bf16 operands take the 32-token chunked closed form: lengths at, around and
    # across chunk ends, a one-token tail, strong decays (A dt' ~ -8 per token) and
    # weak ones in the same batch, the stash with the same lengths
    w = inputs.prefill_workload(batch=8, seq_len=97, nheads=4, dim=64, dstate=128, ngroups=2,
                                pool_rows=9, seed=31, state_dtype=state_dtype, bc_std=128 ** -0.5,
                                ctx=[32, 33, 31, 64, 65, 96, 97, 1])
    w.tensors["dt"][:, :, :2] = w["dt"][:, :, :2].abs() + 2.0
    check_prefill(w)
    check_prefill(w, stash=True)


@pytest.mark.parametrize("stash", [False, True])
def test_long_sequences_past_sixteen_chunks(stash):
    # bf16 operands: the decay tables cover 16 chunks (512 tokens) and are formed
    # again every 16 chunks; lengths across the 512- and 1024-token seams, one
    # just past a seam, one a single token
    w = inputs.prefill_workload(batch=4, seq_len=1100, nheads=2, dim=64, dstate=128, ngroups=1,
                                pool_rows=6, seed=41, bc_std=128 ** -0.5, ctx=[1100, 513, 1025, 1])
    check_prefill(w, stash=stash)


def test_large_batch_without_length_sort():
    w = inputs.prefill_workload(batch=300, seq_len=6, nheads=2, dim=64, dstate=16, ngroups=1,
                                pool_rows=320, seed=8, bc_std=0.25, ctx=("uniform", 0, 6))
    check_prefill(w)


@pytest.mark.parametrize("opts", [dict(with_z=False), dict(with_D=False),
                                  dict(dt_softplus=False, with_bias=False), dict(indices="none")])
def test_optional_inputs(opts):
    w = inputs.prefill_workload(batch=2, seq_len=24, nheads=4, dim=64, dstate=128, ngroups=1,
                                pool_rows=2, seed=9, bc_std=128 ** -0.5, ctx=[24, 9], **opts)
    if opts.get("dt_softplus") is False:
        w.tensors["dt"] = w["dt"].abs() * 0.1
    check_prefill(w)


def _decode_steps(w, steps):
    """Run ssu_decode token by token on a copy of the pool (all rows live)."""
    T = {k: gpu(v) for k, v in w.tensors.items()}
    st = T["state"].clone()
    outs = []
    for t in range(steps):
        out = torch.empty_like(T["x"][:, t])
        ssu_decode(T["x"][:, t].contiguous(), T["A"], T["B"][:, t].contiguous(),
                   T["C"][:, t].contiguous(), T["dt"][:, t].contiguous(), st, out,
                   dt_bias=T["dt_bias"], D=T["D"], z=T["z"][:, t].contiguous(),
                   dt_softplus=w.dt_softplus, state_indices=T["state_indices"])
        outs.append(out)
    return st, torch.stack(outs, 1)


def test_prefill_equals_repeated_decode():
    w = inputs.prefill_workload(batch=4, seq_len=20, nheads=8, dim=64, dstate=128, ngroups=2,
                                pool_rows=6, seed=21, bc_std=128 ** -0.5, ctx=("none",))
    st_p, out_p, _ = run_prefill(w)
    st_d, out_d = _decode_steps(w, 20)
    # prefill evaluates 32-token chunks in closed form on the matrix cores (bf16
    # operands; the rescaled recurrence otherwise), decode the direct recurrence:
    # equal up to each side's fp32 rounding
    assert_close(st_p.cpu(), f64(st_d), 2 * TOL_F32, "state: prefill vs repeated decode")
    assert_close(out_p.cpu(), f64(out_d), TOL_LOW, "out: prefill vs repeated decode")


def test_stash_then_replay_equals_prefill_with_accepted_context():
    w = inputs.prefill_workload(batch=5, seq_len=6, nheads=8, dim=64, dstate=128, ngroups=1,
                                pool_rows=7, seed=22, bc_std=128 ** -0.5, ctx=("none",))
    st_s, out_s, S = run_prefill(w, stash=True)
    accepted = torch.tensor([0, 6, 3, 1, 9], dtype=torch.int32, device="cuda")
    ssu_replay(st_s, S["replay_dA"], S["replay_u"], S["replay_B"], S["replay_dt"], accepted,
               state_indices=gpu(w["state_indices"]))
    st_k, _, _ = run_prefill(w, context_lengths=accepted)
    # rows with nothing accepted are bit-identical; the rest agree to rounding
    # (replay runs the direct recurrence, prefill the chunked closed form)
    idx = w["state_indices"].numpy()
    assert_bitwise(st_s[idx[0]], st_k[idx[0]], "row with accepted = 0")
    assert_close(st_s.cpu(), f64(st_k), 2 * TOL_F32, "stash + replay(k) vs prefill(contextLengths = k)")


def test_seq_len_one_equals_decode():
    w = inputs.prefill_workload(batch=3, seq_len=1, nheads=4, dim=64, dstate=64, ngroups=1,
                                pool_rows=4, seed=23, bc_std=0.125, ctx=("none",))
    st_p, out_p, _ = run_prefill(w)
    st_d, out_d = _decode_steps(w, 1)
    assert_close(st_p.cpu(), f64(st_d), 2 * TOL_F32, "state")
    assert_close(out_p.cpu(), f64(out_d), TOL_LOW, "out")
