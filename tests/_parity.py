"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import numpy as np

# Output tolerance for fp16 products (relative Frobenius and elementwise bars).
REL_FROB = 1e-3
ELEM = 1e-2


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_fp16_close(got, ref, what=""):
    """got: fp16 result; ref: float64 reference. Both bars must hold."""
    g = np.asarray(got).astype(np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - r)
    bound = ELEM * (1.0 + np.abs(r))
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} elements beyond 1e-2*(1+|ref|); worst err "
                           f"{err.max():.3e} at {np.unravel_index(np.argmax(err - bound), err.shape)}")
    nr = np.linalg.norm(r)
    rel = np.linalg.norm(g - r) / (nr if nr > 0 else 1.0)
    assert rel <= REL_FROB, f"{what}: relative Frobenius error {rel:.3e} > {REL_FROB}"
    return rel


def assert_bits_equal(got, ref, what=""):
    g = np.ascontiguousarray(got)
    r = np.ascontiguousarray(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    gv = g.view(np.uint16) if g.dtype == np.float16 else g
    rv = r.view(np.uint16) if r.dtype == np.float16 else r
    mism = gv != rv
    assert not mism.any(), f"{what}: {mism.sum()} of {mism.size} entries differ, first at {np.argwhere(mism)[0]}"
