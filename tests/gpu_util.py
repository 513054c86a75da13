"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def keep_from_mask(mask, M, N, d):
    """Per-sub-vector mask bytes (bit t = element t salient) -> keep[M, N] (1 = kept)."""
    m = np.asarray(mask, dtype=np.uint8).reshape(M, N // d)
    bits = (m[:, :, None] >> np.arange(d, dtype=np.uint8)[None, None, :]) & 1
    return (1 - bits).astype(np.uint8).reshape(M, N)


def mask_from_keep(keep, d):
    M, N = keep.shape
    sal = (1 - keep.astype(np.uint8)).reshape(M, N // d, d)
    return (sal << np.arange(d, dtype=np.uint8)[None, None, :]).sum(-1).astype(np.uint8).ravel()


def bits_equal(a, b):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    if a.shape != b.shape:
        return False
    if a.dtype.kind == "f":
        return np.array_equal(a.view(np.uint32 if a.itemsize == 4 else np.uint64),
                              b.astype(a.dtype).view(np.uint32 if a.itemsize == 4 else np.uint64))
    return np.array_equal(a, b)


def centroid_close(C, Cref, rel=1e-5):
    """Per-centroid max-norm tolerance: |C_k - Cref_k|_inf <= rel * |Cref_k|_inf."""
    C = np.asarray(C, np.float64)
    Cref = np.asarray(Cref, np.float64)
    scale = np.abs(Cref).max(1)
    err = np.abs(C - Cref).max(1)
    bad = err > rel * scale
    return not bad.any(), np.flatnonzero(bad)


def index_flips_allowed(X, hcol, rho, keep, d, C, idx_gpu, idx_ref, rel=1e-6):
    """Index differences are allowed only where the two centroids' weighted
    distances (float64) differ by less than rel * D(gpu choice)."""
    diff = np.flatnonzero(idx_gpu != idx_ref)
    if diff.size == 0:
        return True, diff
    M, N = X.shape
    nb = N // d
    Xs = X.reshape(-1, d).astype(np.float64)
    om = np.broadcast_to(hcol.reshape(nb, d)[None], (M, nb, d)).astype(np.float64)
    if rho is not None:
        om = om * rho.astype(np.float64)[:, None, None]
    if keep is not None:
        om = om * keep.reshape(M, nb, d)
    om = om.reshape(-1, d)
    Cd = C.astype(np.float64)
    dg = (om[diff] * (Xs[diff] - Cd[idx_gpu[diff]]) ** 2).sum(1)
    dr = (om[diff] * (Xs[diff] - Cd[idx_ref[diff]]) ** 2).sum(1)
    ok = (dg - dr) < rel * dg
    return bool(ok.all()), diff[~ok]


def check_select_properties(W, h, d, nnz, rp, col, val, mask):
    """The defining properties of the salient selection, on every element:
    nnz positions, CSR structure with ascending columns and exact values, the
    mask marking exactly those positions, no unselected score above a selected
    one, and among equal scores at the threshold the smaller linear indices
    selected.  Together they fix the selection uniquely."""
    M, N = W.shape
    assert rp[0] == 0 and rp[-1] == nnz and np.all(np.diff(rp) >= 0)
    rows = np.repeat(np.arange(M), np.diff(rp))
    same_row = rows[1:] == rows[:-1]
    assert np.all(col[1:][same_row] > col[:-1][same_row])
    assert np.all((col >= 0) & (col < N))
    assert bits_equal(val, W[rows, col])
    sel = np.zeros(M * N, bool)
    sel[rows.astype(np.int64) * N + col] = True
    assert sel.sum() == nnz
    keep = keep_from_mask(mask, M, N, d).ravel()
    assert np.array_equal(keep == 0, sel)
    s = (np.float32(h)[None, :] * (W * W)).ravel()
    if 0 < nnz < M * N:
        tau_in = s[sel].min()
        tau_out = s[~sel].max()
        assert tau_in >= tau_out
        if tau_in == tau_out:
            lin_in = np.flatnonzero(sel & (s == tau_in))
            lin_out = np.flatnonzero(~sel & (s == tau_in))
            assert lin_in.max() < lin_out.min()
