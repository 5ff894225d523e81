"""GPU parity of ssu_replay (MTP accepted-token commit) against the fp64 oracle."""
import numpy as np
import pytest
import torch

from linear_rnn_recurrent_amd import inputs, ssu_decode
from gpu_helpers import (TOL_F32, assert_bitwise, assert_close, f64, gpu, oracle_replay,
                         run_replay, tol_for)

pytestmark = pytest.mark.gpu


def check_replay(w):
    state0 = w["state"].clone()
    st = run_replay(w)
    st_ref = oracle_replay(w)
    stc = st.cpu()
    nb = w.active_batch
    idx = f64(w["state_indices"])[:nb] if w["state_indices"] is not None else np.arange(nb)
    k = np.minimum(f64(w["accepted_lengths"])[:nb], w.dims["seq_len"])
    moved = np.unique(idx[(idx >= 0) & (k > 0)])
    assert_close(stc[moved], st_ref[moved], tol_for(stc.dtype), "state (replayed rows)")
    still = np.setdiff1d(np.arange(stc.shape[0]), moved)
    if still.size:
        assert_bitwise(stc[still], state0[still], "state (rows with nothing to replay)")
    return st


def test_config4_mtp_replay():
    check_replay(inputs.config(4))


def test_entries_beyond_active_batch_are_not_read():
    # stash and accepted have 44 rows; rows 32..43 carry poison (accepted = 2^30)
    w = inputs.replay_workload(active_batch=32, seq_len=4, nheads=80, dim=64, dstate=128,
                               ngroups=1, pool_rows=48, seed=41, stash_batch=44)
    check_replay(w)


@pytest.mark.parametrize("dstate", [16, 64, 128, 256])
@pytest.mark.parametrize("state_dtype", ["f32", "f16", "bf16"])
def test_dstate_and_state_dtype_matrix(dstate, state_dtype):
    w = inputs.replay_workload(active_batch=6, seq_len=5, nheads=4, dim=40, dstate=dstate,
                               ngroups=2, pool_rows=9, seed=dstate, state_dtype=state_dtype,
                               accepted=[0, 1, 5, 9, 3, 2])
    check_replay(w)


def test_padding_rows_and_no_indices():
    w = inputs.replay_workload(active_batch=5, seq_len=3, nheads=4, dim=64, dstate=64,
                               ngroups=1, pool_rows=8, seed=42, accepted=[3, 3, 1, 2, 0],
                               indices=[6, -1, 2, -1, 4])
    check_replay(w)
    w = inputs.replay_workload(active_batch=4, seq_len=3, nheads=4, dim=64, dstate=64,
                               ngroups=1, pool_rows=4, seed=43, accepted=[3, 1, 0, 2],
                               indices="none")
    check_replay(w)


def test_replay_equals_repeated_decode_bitwise():
    w = inputs.replay_workload(active_batch=4, seq_len=4, nheads=8, dim=64, dstate=128,
                               ngroups=1, pool_rows=6, seed=44, accepted=[4, 2, 1, 3])
    st_r = run_replay(w)
    T = {k: gpu(v) for k, v in w.tensors.items()}
    st = T["state"].clone()
    for b in range(4):
        k = int(w["accepted_lengths"][b])
        for t in range(k):
            out = torch.empty((1, 8, 64), device="cuda")
            ssu_decode(T["replay_u"][b:b + 1, t].contiguous(), T["A"],
                       T["replay_B"][b:b + 1, t].contiguous(),
                       torch.zeros((1, 1, 128), device="cuda"),
                       T["replay_dt"][b:b + 1, t].contiguous(), st, out, dt_softplus=False,
                       state_indices=T["state_indices"][b:b + 1].contiguous())
    assert_bitwise(st_r, st, "replay(k) vs k decode steps")


def test_zero_active_batch_is_a_noop():
    w = inputs.replay_workload(active_batch=3, seq_len=2, nheads=2, dim=16, dstate=16,
                               ngroups=1, pool_rows=4, seed=45)
    w.active_batch = 0
    st = run_replay(w)
    torch.cuda.synchronize()
    assert_bitwise(st, w["state"], "state")
