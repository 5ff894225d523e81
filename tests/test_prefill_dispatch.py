"""Which prefill kernel a call takes, decided on the host and checked on the CPU.

The matrix-core prefill (x/z/out and B/C both bf16 or both fp16, dstate a
multiple of 32, dim a multiple of 8, 16-byte aligned x/out/z/x stash) forms its
offsets inside one batch row in 32 bits, so a row whose tokens span 2^31 bytes
or more (with a factor of two to spare: seq_len * max(nheads * dim, ngroups *
dstate) * 4 must stay below 2^31) goes to the VALU kernel, whose offsets are
64-bit. The host
predicate is compiled for the host alone (no device code, no GPU) and run here on
the boundary cases; no out-of-bounds case ever runs on a GPU.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# (name, fields, expected): fields override a bf16 H80 Dm64 N128 G1 T512 call
CASES = [
    ("config-2 shape", {}, 1),
    ("T 262144 at H128 Dm64", dict(nheads=128, seq_len=262144), 0),
    ("just below the bound", dict(nheads=64, dim=64, seq_len=(1 << 29) // 4096 - 1), 1),
    ("at the bound", dict(nheads=64, dim=64, seq_len=(1 << 29) // 4096), 0),
    ("B/C rows set the bound", dict(ngroups=64, dstate=256, nheads=64, dim=8, seq_len=(1 << 29) // 16384), 0),
    ("B/C rows just below", dict(ngroups=64, dstate=256, nheads=64, dim=8, seq_len=(1 << 29) // 16384 - 1), 1),
    ("fp16 x/z/out and B/C", dict(io="kF16", bc="kF16"), 1),
    ("fp16 x/z/out, bf16 B/C", dict(io="kF16"), 0),
    ("bf16 x/z/out, fp16 B/C", dict(bc="kF16"), 0),
    ("fp16 at dstate 16", dict(io="kF16", bc="kF16", dstate=16), 0),
    ("fp16 x not 16-byte aligned", dict(io="kF16", bc="kF16", x_off=2), 0),
    ("fp32 B/C", dict(bc="kF32"), 0),
    ("dstate 16", dict(dstate=16), 0),
    ("dim 100", dict(dim=100), 0),
    ("x not 16-byte aligned", dict(x_off=2), 0),
    ("out not 16-byte aligned", dict(out_off=8), 0),
    ("z not 16-byte aligned", dict(z_off=4), 0),
    ("x stash not 16-byte aligned", dict(u_off=4), 0),
    ("forced VALU waves", dict(waves=8), 0),
]


def _program():
    lines = ['#include "ssu_prefill_impl.h"', "#include <cstdio>",
             "static __attribute__((aligned(16))) char buf[256];", "int main() {"]
    for _, f, _ in CASES:
        lines.append("  {")
        lines.append("    ssu::PrefillParams p = {};")
        lines.append(f"    p.d.x = buf + {f.get('x_off', 0)}; p.d.out = buf + 64 + {f.get('out_off', 0)};")
        if "z_off" in f:
            lines.append(f"    p.d.z = buf + 128 + {f['z_off']};")
        if "u_off" in f:
            lines.append(f"    p.st_u = reinterpret_cast<float *>(buf + 192 + {f['u_off']});")
        lines.append(f"    p.d.io_dtype = ssu::{f.get('io', 'kBF16')}; p.d.bc_dtype = ssu::{f.get('bc', 'kBF16')};")
        lines.append(f"    p.d.dstate = {f.get('dstate', 128)}; p.d.dim = {f.get('dim', 64)};")
        lines.append(f"    p.d.nheads = {f.get('nheads', 80)}; p.d.ngroups = {f.get('ngroups', 1)};")
        lines.append(f"    p.seq_len = {f.get('seq_len', 512)}; p.waves_per_wg = {f.get('waves', 0)};")
        lines.append('    std::printf("%d\\n", (int)ssu::prefill_mm_fits(p));')
        lines.append("  }")
    lines.append("  return 0;\n}")
    return "\n".join(lines) + "\n"


@pytest.fixture(scope="module")
def decisions(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("dispatch")
    src, exe = d / "fits.hip", d / "fits"
    src.write_text(_program())
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "--cuda-host-only", "-O1", "-std=c++17",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "linear_rnn_recurrent_amd", "csrc"),
           str(src), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    return [int(v) for v in out]


@pytest.mark.parametrize("i", range(len(CASES)), ids=[c[0] for c in CASES])
def test_matrix_core_prefill_dispatch(decisions, i):
    name, _, want = CASES[i]
    assert decisions[i] == want, name
