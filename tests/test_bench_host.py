"""bench.py's host side, on the CPU: the one-GPU contract, option checks, and the
algorithmic byte counts against sums of tensor sizes."""
import os
import subprocess
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from linear_rnn_recurrent_amd import inputs  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2 and "only --gpus 1" in r.stderr


def test_prefill_options_apply_to_the_prefill_configuration_only():
    r = _run("--config", "3", "--stash")
    assert r.returncode == 2 and "--config 2" in r.stderr


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def test_decode_bytes_of_the_default_workload():
    # every addressed state row read and written, x, z, out, B and C of every
    # row, the per-head scalars and dt; no padding at this workload
    w = inputs.config(1)
    T = w.tensors
    b, h, d = T["x"].shape
    row_bytes = h * d * T["state"].shape[-1] * T["state"].element_size()
    want = (2 * b * row_bytes + _nbytes(T["x"]) * 2 + _nbytes(T["z"]) + _nbytes(T["B"]) + _nbytes(T["C"])
            + _nbytes(T["dt"]) + _nbytes(T["A"]) + _nbytes(T["dt_bias"]) + _nbytes(T["D"])
            + _nbytes(T["state_indices"]))
    assert bench.decode_bytes(T, b) == want == 337_564_864


def test_prefill_stash_bytes_are_the_stash_minus_the_state_write():
    w = inputs.config(2)
    T = w.tensors
    L = T["context_lengths"].clamp(0, T["x"].shape[1]).tolist()
    b, t, h, d = T["x"].shape
    stash = (2 * b * t * h + b * t * h * d + T["B"].numel()) * 4
    state_write = b * h * d * T["state"].shape[-1] * T["state"].element_size()
    assert bench.prefill_bytes(T, L, True) - bench.prefill_bytes(T, L) == stash - state_write


def test_prefill_bytes_scale_with_the_operand_size():
    # fp32 x/z/out and B/C: every live token's activations cost twice the bf16 bytes
    w = inputs.config(2)
    T = dict(w.tensors)
    L = T["context_lengths"].clamp(0, T["x"].shape[1]).tolist()
    base = bench.prefill_bytes(T, L)
    for k in ("x", "z", "B", "C"):
        T[k] = T[k].to(torch.float32)
    b, t, h, d = T["x"].shape
    g, n = T["B"].shape[2], T["B"].shape[3]
    extra = sum(L) * (3 * h * d * 2 + 2 * g * n * 2) + sum(t - l for l in L) * h * d * 2
    assert bench.prefill_bytes(T, L) - base == extra
