"""GPU parity of ssu_prefill (with contextLengths and the replay stash) against the
fp64 oracle, plus the prefill/decode/replay invariants on the GPU itself."""
import numpy as np
import pytest
import torch

from linear_rnn_recurrent_amd import inputs, ssu_decode, ssu_replay
from gpu_helpers import (TOL_F32, TOL_LOW, assert_bitwise, assert_close, f64, gpu, misaligned,
                         oracle_prefill, oracle_prefill_magnitude, run_prefill, tol_for,
                         touched_rows, untouched_rows)

pytestmark = pytest.mark.gpu


def lengths(w):
    T = w.dims["seq_len"]
    cl = w["context_lengths"]
    if cl is None:
        return np.full(w.dims["batch"], T)
    return np.clip(f64(cl), 0, T)


def valu_kernel(w):
    """run_prefill overrides that put a 16-bit prefill on the VALU kernel."""
    return {"x": misaligned(gpu(w["x"]))} if w["x"].element_size() == 2 else {}


def check_prefill(w, stash=False, cancelling=False, **over):
    """cancelling: tolerances scaled by the magnitude of each value's terms (inputs
    whose sums cancel far below their terms) instead of by the value itself."""
    state0 = w["state"].clone()
    st, out, S = run_prefill(w, stash=stash, **over)
    st_ref, out_ref, S_ref = oracle_prefill(w, stash=stash)
    st_mag, out_mag = oracle_prefill_magnitude(w) if cancelling else (None, None)
    idx = w["state_indices"]
    nb = w.dims["batch"]
    stc = st.cpu()
    if stash:
        assert_bitwise(stc, state0, "state must stay read-only in stash mode")
    else:
        rows = touched_rows(idx, nb)
        assert_close(stc[rows], st_ref[rows], tol_for(stc.dtype), "state (addressed rows)",
                     None if st_mag is None else st_mag[rows])
        free = untouched_rows(idx, w.dims["pool_rows"], nb)
        if free.size:
            assert_bitwise(stc[free], state0[free], "state (rows not addressed)")
    live = np.ones(nb, dtype=bool) if idx is None else f64(idx) >= 0
    outc = out.cpu()
    assert_close(outc[live], out_ref[live], tol_for(outc.dtype), "out (live rows)",
                 None if out_mag is None else out_mag[live])
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


def config2_shape(io, seed=2):
    return inputs.prefill_workload(batch=8, seq_len=512, nheads=80, dim=64, dstate=128,
                                   ngroups=1, pool_rows=64, seed=seed, state_dtype="f32",
                                   io_dtype=io, bc_dtype=io, bc_std=1.0 / np.sqrt(128),
                                   ctx=("uniform", 64, 512), zero_state=True)


@pytest.mark.parametrize("stash", [False, True])
@pytest.mark.parametrize("io", ["f32", "f16"])
def test_config2_shape_on_the_valu_kernel(io, stash):
    # config 2's shape and recipe with fp32 or fp16 x/z/B/C on the rescaled VALU
    # recurrence (fp16 x placed off 16-byte alignment): over up to 512 tokens the
    # running product of decays (sum of A dt' near -100 at full length) leaves
    # [1e-30, 1e30] and the state is renormalised at a chunk start
    w = config2_shape(io)
    check_prefill(w, stash=stash, **valu_kernel(w))


@pytest.mark.parametrize("stash", [False, True])
def test_config2_shape_fp16_on_the_matrix_cores(stash):
    # fp16 x/z/B/C: B . C^T on the fp16 matrix cores as it is, the state and the
    # weighted x in scaled fp16 parts, x in two bf16 parts
    check_prefill(config2_shape("f16", seed=12), stash=stash)


@pytest.mark.parametrize("dstate", [32, 64, 128, 256])
@pytest.mark.parametrize("state_dtype", ["f32", "f16", "bf16"])
def test_fp16_operands_dstate_and_state_dtype_matrix(dstate, state_dtype):
    w = inputs.prefill_workload(batch=3, seq_len=70, nheads=4, dim=64, dstate=dstate,
                                ngroups=2, pool_rows=5, seed=100 + dstate, state_dtype=state_dtype,
                                io_dtype="f16", bc_dtype="f16", bc_std=dstate ** -0.5,
                                ctx=[70, 33, 1])
    check_prefill(w)
    check_prefill(w, stash=True)


def test_fp16_operands_over_wide_value_ranges():
    # the fp16 matrix-core path scales each state row and each row of the weighted
    # x by a power of two before cutting them into fp16 parts. Head 0: state rows
    # of ~1e3 to ~1e6 (past fp16's 65504); head 1: rows of ~1e-6; head 2: x up
    # to ~4e4, B ~30x the recipe, dt' ~ 1 and a weak decay, so that the weighted
    # x and the state pass fp16's range; small C and D keep the fp16 outputs in
    # range. A group per head. The state of head 2 sums terms of ~1e5 to values of
    # a few units, below fp32's resolution of its terms: tolerances are relative
    # to the magnitude of the terms.
    w = inputs.prefill_workload(batch=3, seq_len=100, nheads=4, dim=64, dstate=128,
                                ngroups=4, pool_rows=4, seed=91, io_dtype="f16", bc_dtype="f16",
                                bc_std=128 ** -0.5, ctx=[100, 64, 37])
    rng = np.random.default_rng(1091)
    st = w["state"].double().numpy()
    x, Bm, Cm = (w[k].double().numpy() for k in ("x", "B", "C"))
    st[:, 0] *= 1e6 * 10.0 ** rng.uniform(-3, 0, (st.shape[0], 64, 1))
    Cm[:, :, 0] *= 1e-3
    st[:, 1] *= 1e-6
    x[:, :, 2] *= 1e4
    Bm[:, :, 2] *= 30.0
    Cm[:, :, 2] *= 1e-3
    w.tensors["D"][2] = 0.01
    w.tensors["A"][2] = -0.05  # weak decay and dt' ~ 1: the state accumulates
    w.tensors["dt_bias"][2] = 1.0
    w.tensors["state"] = torch.from_numpy(st.astype(np.float32))
    for k, v in (("x", x), ("B", Bm), ("C", Cm)):
        w.tensors[k] = torch.from_numpy(v).to(torch.float16)
    assert np.isfinite(f64(w["x"])).all()
    assert np.abs(st[:, 0]).max() > 65504.0  # the cases this covers
    st_out, _, _ = check_prefill(w, cancelling=True)
    assert float(st_out[:, 2].abs().max()) > 65504.0
    check_prefill(w, stash=True, cancelling=True)


@pytest.mark.parametrize("dstate", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("state_dtype", ["f32", "f16", "bf16"])
def test_dstate_and_state_dtype_matrix(dstate, state_dtype):
    w = inputs.prefill_workload(batch=3, seq_len=37, nheads=4, dim=64, dstate=dstate,
                                ngroups=2, pool_rows=5, seed=dstate, state_dtype=state_dtype,
                                bc_std=dstate ** -0.5, ctx=[37, 20, 1])
    check_prefill(w)


@pytest.mark.parametrize("io_dtype,bc_dtype", [("f32", "f32"), ("f16", "f16"), ("bf16", "f32"),
                                               ("f32", "bf16"), ("f16", "bf16"), ("bf16", "f16")])
def test_io_and_bc_dtypes(io_dtype, bc_dtype):
    w = inputs.prefill_workload(batch=2, seq_len=21, nheads=4, dim=64, dstate=128, ngroups=1,
                                pool_rows=3, seed=3, io_dtype=io_dtype, bc_dtype=bc_dtype,
                                bc_std=128 ** -0.5, ctx=("none",))
    check_prefill(w)
    if io_dtype == bc_dtype == "f16":  # the matrix cores above, the VALU kernel here
        check_prefill(w, **valu_kernel(w))


@pytest.mark.parametrize("io", ["bf16", "f16"])
def test_ragged_context_lengths_and_padding(io):
    # ctx: zero, negative (clamped to 0), full, beyond seq_len (clamped), odd; one padding row
    w = inputs.prefill_workload(batch=6, seq_len=45, nheads=4, dim=64, dstate=64, ngroups=2,
                                pool_rows=8, seed=4, ctx=[0, -3, 45, 100, 17, 33],
                                indices=[5, 1, 7, 0, -1, 3], bc_std=0.125, io_dtype=io, bc_dtype=io)
    check_prefill(w)
    check_prefill(w, stash=True)


@pytest.mark.parametrize("io", ["bf16", "f16"])
@pytest.mark.parametrize("dim", [32, 100, 200])
def test_row_blocks_and_ragged_dim(dim, io):
    # dim 32 and 200 on the matrix cores (a partial row block), 100 on the VALU kernel
    w = inputs.prefill_workload(batch=2, seq_len=19, nheads=3, dim=dim, dstate=128, ngroups=1,
                                pool_rows=4, seed=dim, bc_std=128 ** -0.5, ctx=[19, 11],
                                io_dtype=io, bc_dtype=io)
    check_prefill(w)
    check_prefill(w, stash=True)


@pytest.mark.parametrize("state_dtype,io", [("f32", "bf16"), ("bf16", "bf16"), ("f32", "f16")])
def test_chunk_boundaries(state_dtype, io):
    # 16-bit operands take the 32-token chunked closed form: lengths at, around and
    # across chunk ends, a one-token tail, strong decays (A dt' ~ -8 per token) and
    # weak ones in the same batch, the stash with the same lengths
    w = inputs.prefill_workload(batch=8, seq_len=97, nheads=4, dim=64, dstate=128, ngroups=2,
                                pool_rows=9, seed=31, state_dtype=state_dtype, bc_std=128 ** -0.5,
                                io_dtype=io, bc_dtype=io, ctx=[32, 33, 31, 64, 65, 96, 97, 1])
    w.tensors["dt"][:, :, :2] = w["dt"][:, :, :2].abs() + 2.0
    check_prefill(w)
    check_prefill(w, stash=True)


@pytest.mark.parametrize("io", ["bf16", "f16"])
@pytest.mark.parametrize("stash", [False, True])
def test_long_sequences_past_sixteen_chunks(stash, io):
    # 16-bit operands: the decay tables cover 16 chunks (512 tokens) and are formed
    # again every 16 chunks; lengths across the 512- and 1024-token seams, one
    # just past a seam, one a single token
    w = inputs.prefill_workload(batch=4, seq_len=1100, nheads=2, dim=64, dstate=128, ngroups=1,
                                pool_rows=6, seed=41, bc_std=128 ** -0.5, io_dtype=io, bc_dtype=io,
                                ctx=[1100, 513, 1025, 1])
    check_prefill(w, stash=stash)


def test_large_batch_without_length_sort():
    w = inputs.prefill_workload(batch=300, seq_len=6, nheads=2, dim=64, dstate=16, ngroups=1,
                                pool_rows=320, seed=8, bc_std=0.25, ctx=("uniform", 0, 6))
    check_prefill(w)


@pytest.mark.parametrize("io", ["bf16", "f16"])
@pytest.mark.parametrize("opts", [dict(with_z=False), dict(with_D=False),
                                  dict(dt_softplus=False, with_bias=False), dict(indices="none")])
def test_optional_inputs(opts, io):
    w = inputs.prefill_workload(batch=2, seq_len=24, nheads=4, dim=64, dstate=128, ngroups=1,
                                pool_rows=2, seed=9, bc_std=128 ** -0.5, ctx=[24, 9],
                                io_dtype=io, bc_dtype=io, **opts)
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


@pytest.mark.parametrize("io", ["bf16", "f16"])
def test_prefill_equals_repeated_decode(io):
    w = inputs.prefill_workload(batch=4, seq_len=20, nheads=8, dim=64, dstate=128, ngroups=2,
                                pool_rows=6, seed=21, bc_std=128 ** -0.5, ctx=("none",),
                                io_dtype=io, bc_dtype=io)
    st_p, out_p, _ = run_prefill(w)
    st_d, out_d = _decode_steps(w, 20)
    # prefill evaluates 32-token chunks in closed form on the matrix cores (bf16 or
    # fp16 operands; the rescaled recurrence otherwise), decode the direct recurrence:
    # equal up to each side's fp32 rounding
    assert_close(st_p.cpu(), f64(st_d), 2 * TOL_F32, "state: prefill vs repeated decode")
    assert_close(out_p.cpu(), f64(out_d), TOL_LOW, "out: prefill vs repeated decode")


@pytest.mark.parametrize("io", ["bf16", "f16"])
def test_stash_then_replay_equals_prefill_with_accepted_context(io):
    w = inputs.prefill_workload(batch=5, seq_len=6, nheads=8, dim=64, dstate=128, ngroups=1,
                                pool_rows=7, seed=22, bc_std=128 ** -0.5, ctx=("none",),
                                io_dtype=io, bc_dtype=io)
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
