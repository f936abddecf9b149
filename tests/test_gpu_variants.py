"""The environment switches of libsnm (SNM_LOG, SNM_FORCE_VARIANT), read once per process, so
each setting runs in a child process of its own (one at a time). Every forced variant must
give the oracle's product, and SNM_LOG must name the variant that ran.

Shapes: a V:2:16 product with V = 128 whose grid is too small for the large-tile kernel by
default (so 'large' changes the choice and 'wide' keeps it), the same for V:2:8 with V = 64
and the 64-row large-tile kernel (both storages), and a decode-shaped 2:4 product with C = 8
(the LDS-ring kernel by default, 'direct' forces the register kernel, 'generic' the generic
tiled kernel), on the canonical and the operand-major storage."""
import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest

import oracle
import workloads
from _parity import assert_fp16_close

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = textwrap.dedent("""
    import sys
    import numpy as np
    import torch
    sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
    import workloads
    import structured_sparse_matrix_amd as snm
    dev = torch.device("cuda:0")
    kind, out = sys.argv[1], sys.argv[2]
    if kind in ("vnm64", "vnm64t"):   # V = 64, ragged second column tile
        A = workloads.small_matrix(15, (1024, 2048), 0.02)
        B = workloads.small_matrix(16, (2048, 264))
        enc = snm.prune_encode_vnm_tiled if kind == "vnm64t" else snm.prune_encode_vnm
        mm = snm.spmm_vnm_tiled if kind == "vnm64t" else snm.spmm_vnm
        v, mi, cl = enc(torch.from_numpy(A).to(dev), 64, 8)
        Y = mm(v, mi, cl, torch.from_numpy(B).to(dev), 64, 8)
    elif kind == "vnm":
        A = workloads.small_matrix(11, (1024, 2048), 0.02)
        B = workloads.small_matrix(12, (2048, 512))
        v, mi, cl = snm.prune_encode_vnm(torch.from_numpy(A).to(dev), 128, 16)
        Y = snm.spmm_vnm(v, mi, cl, torch.from_numpy(B).to(dev), 128, 16)
    elif kind == "nmt":   # operand-major A, column-major B, C <= 32, K % 512 == 0
        A = workloads.small_matrix(13, (512, 1024), 0.02)
        X = workloads.small_matrix(14, (8, 1024))
        vt, mt = snm.prune_encode_nm_tiled(torch.from_numpy(A).to(dev))
        Y = snm.spmm_nm_tiled(vt, mt, 512, torch.from_numpy(X).to(dev).t())
    else:
        A = workloads.small_matrix(13, (512, 1024), 0.02)
        X = workloads.small_matrix(14, (8, 1024))   # column-major B: activations X[C][K]
        v, m = snm.prune_encode_nm(torch.from_numpy(A).to(dev))
        Y = snm.spmm_nm(v, m, torch.from_numpy(X).to(dev).t())
    torch.cuda.synchronize()
    np.save(out, Y.cpu().numpy())
""")


def _run(kind, force, tmp_path):
    script = tmp_path / "child.py"
    script.write_text(CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests")))
    out = tmp_path / f"{kind}_{force or 'default'}.npy"
    env = dict(os.environ, SNM_LOG="1")
    env.pop("SNM_FORCE_VARIANT", None)
    if force:
        env["SNM_FORCE_VARIANT"] = force
    print(f"variant child {kind} force={force!r}", flush=True)
    r = subprocess.run([sys.executable, str(script), kind, str(out)], env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("snm: ")]
    return np.load(out), lines


@pytest.mark.parametrize("force,expect", [("", "wide 128x128"), ("wide", "wide 128x128"),
                                          ("large", "large 128x512"), ("generic", "generic")])
def test_vnm_forced_variant_matches_oracle(force, expect, tmp_path):
    Y, lines = _run("vnm", force, tmp_path)
    A = workloads.small_matrix(11, (1024, 2048), 0.02)
    B = workloads.small_matrix(12, (2048, 512))
    ov, omi, ocl = oracle.prune_encode_vnm(A, 128, 16)
    assert_fp16_close(Y, oracle.spmm_vnm(ov, omi, ocl, 128, 16, B))
    assert any(ln.startswith("snm: spmm_vnm R=1024 K=2048 C=512 -> ") and ln.endswith(expect)
               for ln in lines), lines


@pytest.mark.parametrize("kind", ["vnm64", "vnm64t"])
@pytest.mark.parametrize("force,expect", [("", "wide 64x128"), ("wide", "wide 64x128"), ("large", "large 64x256")])
def test_vnm64_forced_variant_matches_oracle(kind, force, expect, tmp_path):
    """V = 64 (K' = 1024): the default grid (32 tiles of 64 x 256) is below the 64-row
    large-tile kernel's threshold, 'large' forces it (second column tile ragged: C = 264)."""
    Y, lines = _run(kind, force, tmp_path)
    A = workloads.small_matrix(15, (1024, 2048), 0.02)
    B = workloads.small_matrix(16, (2048, 264))
    ov, omi, ocl = oracle.prune_encode_vnm(A, 64, 8)
    assert_fp16_close(Y, oracle.spmm_vnm(ov, omi, ocl, 64, 8, B))
    op = "spmm_vnm_tiled" if kind == "vnm64t" else "spmm_vnm"
    assert any(ln.startswith(f"snm: {op} R=1024 K=2048 C=264 -> ") and ln.endswith(expect)
               for ln in lines), lines


@pytest.mark.parametrize("force,expect", [("", "skinny ring"), ("direct", "skinny"), ("generic", "generic"),
                                          ("unknown", "skinny ring")])
def test_nm_forced_variant_matches_oracle(force, expect, tmp_path):
    Y, lines = _run("nm", force, tmp_path)
    A = workloads.small_matrix(13, (512, 1024), 0.02)
    X = workloads.small_matrix(14, (8, 1024))
    ov, om = oracle.prune_encode_nm(A)
    assert_fp16_close(Y, oracle.spmm_nm(ov, om, np.ascontiguousarray(X.T)))
    assert lines == [f"snm: spmm_nm R=512 K=1024 C=8 -> {expect}"], lines


@pytest.mark.parametrize("force,expect", [("", "skinny ring"), ("direct", "skinny"), ("generic", "generic")])
def test_nm_tiled_forced_variant_matches_oracle(force, expect, tmp_path):
    Y, lines = _run("nmt", force, tmp_path)
    A = workloads.small_matrix(13, (512, 1024), 0.02)
    X = workloads.small_matrix(14, (8, 1024))
    ov, om = oracle.prune_encode_nm(A)
    assert_fp16_close(Y, oracle.spmm_nm(ov, om, np.ascontiguousarray(X.T)))
    assert lines == [f"snm: spmm_nm_tiled R=512 K=1024 C=8 -> {expect}"], lines
