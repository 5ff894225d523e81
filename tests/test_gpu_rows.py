"""GPU parity of the row-movement entry points (ssu_state_gather / _scatter /
_pack / _unpack) against the oracle: byte-exact."""
import numpy as np
import pytest
import torch

import oracle
from linear_rnn_recurrent_amd import (inputs, pack_workspace_bytes, ssu_state_gather,
                                      ssu_state_pack, ssu_state_scatter, ssu_state_unpack)
from gpu_helpers import assert_bitwise

pytestmark = pytest.mark.gpu


def _pool(shape, dtype=torch.float32, seed=0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype)


@pytest.mark.parametrize("dtype,shape", [(torch.float32, (12, 4, 64, 128)),
                                         (torch.bfloat16, (9, 3, 5)),       # 30-byte rows
                                         (torch.float16, (10, 7))])         # 14-byte rows
def test_gather_and_scatter(dtype, shape):
    pool = _pool(shape, dtype, seed=1)
    idx = torch.tensor([7, -1, 0, 3, 8, -1], dtype=torch.int32)
    active = torch.full((6,) + shape[1:], 9.0, dtype=dtype).cuda()
    ssu_state_gather(pool.cuda(), active, idx.cuda())
    want = oracle.gather(pool.numpy() if dtype == torch.float32 else pool.view(torch.int16).numpy(),
                         idx.numpy())
    got = active.cpu() if dtype == torch.float32 else active.cpu().view(torch.int16)
    np.testing.assert_array_equal(got.numpy(), want)
    # scatter modified rows back
    res = pool.clone().cuda()
    upd = (active.float() + 1.0).to(dtype)
    ssu_state_scatter(upd, res, idx.cuda())
    ref = pool.clone()
    ref_np = ref.numpy() if dtype == torch.float32 else ref.view(torch.int16).numpy()
    upd_np = upd.cpu().numpy() if dtype == torch.float32 else upd.cpu().view(torch.int16).numpy()
    oracle.scatter(upd_np, ref_np, idx.numpy())
    assert_bitwise(res, ref, "scatter")


def test_gather_strided_views():
    # rows of a padded pool (row stride > row bytes) and a strided active buffer
    big = _pool((8, 3, 40), seed=2)
    pool = big.reshape(8, 120)[:, :96].contiguous()
    padded = torch.zeros(8, 100)
    padded[:, :96] = pool
    view = padded[:, :96]                       # row stride 100 floats, rows dense
    act_buf = torch.zeros(5, 104).cuda()
    act = act_buf[:, :96]
    idx = torch.tensor([6, 2, -1, 7, 0], dtype=torch.int32)
    ssu_state_gather(view.cuda(), act, idx.cuda())
    want = oracle.gather(pool.numpy(), idx.numpy())
    np.testing.assert_array_equal(act.cpu().numpy(), want)
    assert torch.all(act_buf[:, 96:] == 0)      # nothing written past a row


@pytest.mark.parametrize("row_floats,stride_floats", [(10, 12), (4101, 4104)])
def test_gather_aligned_rows_with_tail(row_floats, stride_floats):
    # 16-byte aligned rows whose length is not a multiple of 16 bytes: whole
    # vectors in interleaved pieces, the tail bytes by the first piece; the
    # second case spans two pieces
    padded = _pool((7, stride_floats), seed=4)
    pool = padded[:, :row_floats]
    act_buf = torch.full((4, stride_floats + 4), -3.0).cuda()
    act = act_buf[:, :row_floats]
    idx = torch.tensor([5, -1, 0, 6], dtype=torch.int32)
    src = padded.cuda()[:, :row_floats]                 # row stride stride_floats
    ssu_state_gather(src, act, idx.cuda())
    want = oracle.gather(pool.contiguous().numpy(), idx.numpy())
    np.testing.assert_array_equal(act.cpu().numpy(), want)
    assert torch.all(act_buf[:, row_floats:] == -3.0)   # nothing written past a row
    res_buf = padded.clone().cuda()
    ssu_state_scatter(act, res_buf[:, :row_floats], idx.cuda())
    ref = padded.clone()
    ref_np = ref[:, :row_floats].numpy().copy()
    oracle.scatter(act.cpu().numpy(), ref_np, idx.numpy())
    ref[:, :row_floats] = torch.from_numpy(ref_np)
    assert_bitwise(res_buf, ref, "scatter")


def _pack_case(rows, homes, bystanders, dtype=torch.float32, seed=3, width=(2, 64, 128)):
    pool = _pool((rows,) + width, dtype, seed)
    h = torch.tensor(homes, dtype=torch.int32).cuda()
    by = torch.tensor(bystanders, dtype=torch.int32).cuda() if bystanders else None
    ws = torch.empty(pack_workspace_bytes(pool, len(homes), len(bystanders)), dtype=torch.uint8,
                     device="cuda")
    return pool, h, by, ws


@pytest.mark.parametrize("homes,bystanders", [
    ([3, 0, 1], []),                     # the page's case: homes not ascending
    ([5, 0, 4], [1, 2]),                 # live rows of other requests inside [0, B)
    ([0, 6, 2, 1], [3]),                 # members already in place (0, 2) are not copied
    ([0, 1, 2], []),                     # the whole cohort in place: nothing moves
    ([9, 8, 7, 6, 5], [0, 1, 2, 3, 4]),  # every slot a bystander
])
def test_pack_forward_unpack(homes, bystanders):
    pool, h, by, ws = _pack_case(10, homes, bystanders)
    g = pool.clone().cuda()
    ssu_state_pack(g, h, ws, bystanders=by)
    ref = pool.clone().numpy()
    saved = oracle.pack(ref, homes, bystanders)
    np.testing.assert_array_equal(g.cpu().numpy()[:len(homes)], ref[:len(homes)])
    # the forward updates the working slots, then they go home
    g[:len(homes)] += 1.0
    ref[:len(homes)] += 1.0
    ssu_state_unpack(g, h, ws, bystanders=by)
    oracle.unpack(ref, homes, bystanders, saved)
    live = sorted(set(homes) | set(bystanders) | set(range(len(homes), 10)))
    np.testing.assert_array_equal(g.cpu().numpy()[live], ref[live])


def test_pack_unpack_in_graph_match_eager():
    homes, bystanders = [5, 0, 4], [1, 2]
    pool, h, by, ws = _pack_case(8, homes, bystanders, seed=4)
    g = pool.clone().cuda()

    def run():
        ssu_state_pack(g, h, ws, bystanders=by)
        g[:3] *= 2.0
        ssu_state_unpack(g, h, ws, bystanders=by)

    run()
    torch.cuda.synchronize()
    want = g.clone()
    graph = torch.cuda.CUDAGraph()
    g.copy_(pool.cuda())
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        g.copy_(pool.cuda())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_bitwise(g, want, f"pool after replay {rep}")


def test_gather_config1_batch_full_size():
    w = inputs.config(1)
    pool = w["state"]
    idx = w["state_indices"]
    act = torch.empty((64,) + tuple(pool.shape[1:]), device="cuda")
    ssu_state_gather(pool.cuda(), act, idx.cuda())
    assert_bitwise(act, pool[idx.long()], "gathered rows")
