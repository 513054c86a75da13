"""ctypes face of the C oracle (test infrastructure).

``build()`` compiles ``vq_oracle.c`` with gcc (-O2 -fopenmp -ffp-contract=off)
into ``oracle/_build/liboracle.so``; every other function takes and returns
numpy arrays.  Nothing here touches a GPU.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vq_oracle.c")
_OUT_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_OUT_DIR, "liboracle.so")
_lib = None

CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(extra_flags=(), out_path=None, src=None):
    """Compile the oracle (or another copy of its source); returns the .so path."""
    out = out_path or _LIB_PATH
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *extra_flags, src or _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_P = ctypes.c_void_p
_LL = ctypes.c_longlong
_I = ctypes.c_int
_D = ctypes.c_double

_SIGS = {
    "orc_nnz": (_LL, [_LL, _LL, _D]),
    "orc_select": (_I, [_P, _P, _LL, _LL, _LL, _P, _P, _P, _P]),
    "orc_binorm": (None, [_P, _P, _LL, _LL, _P, _P, _P, _P, _P]),
    "orc_init": (_I, [_P, _LL, _I, _P, _I, _P]),
    "orc_assign": (None, [_P, _P, _P, _P, _LL, _LL, _I, _P, _I, _P, _LL, _P, _P, _I]),
    "orc_objective": (_D, [_P, _P, _P, _P, _LL, _LL, _I, _P, _P]),
    "orc_update": (_D, [_P, _P, _P, _P, _LL, _LL, _I, _P, _I, _P, _P]),
    "orc_residual": (None, [_P, _LL, _I, _P, _P, _P]),
    "orc_reconstruct": (None, [_LL, _LL, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "orc_select_subvectors": (_I, [_P, _P, _LL, _LL, _I, _LL, _P]),
    "orc_select_residual": (_I, [_P, _P, _P, _LL, _LL, _LL, _P]),
    "orc_keep_to_csr": (_LL, [_P, _P, _LL, _LL, _P, _P, _P]),
    "orc_column_order": (_I, [_P, _LL, _LL, _P]),
    "orc_fit_grouped": (_I, [_P, _P, _LL, _LL, _I, _I, _I, _I, _I, _D, _I, _I, _LL, _I, _I, _I, _I, _P, _P, _I,
                             _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "orc_vptq": (_I, [_P, _P, _LL, _LL, _I, _P, _I, _I, _P, _P, _P, _P]),
    "orc_qgemv": (_I, [_LL, _LL, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _LL, _P]),
    "orc_fit": (_I, [_P, _P, _LL, _LL, _I, _I, _I, _I, _I, _D, _I, _I, _P, _P, _I,
                     _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
}


def load(path=None):
    """Load the oracle library (building it first if it is absent)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        build(out_path=p)
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _ptr(a):
    # a ctypes pointer that holds a reference to the array, so that a
    # temporary converted copy stays alive until the C call returns
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def nnz(M, N, p, lib=None):
    return int((lib or load()).orc_nnz(M, N, p))


def select(W, h, nnz_, lib=None):
    lib = lib or load()
    W = _c(W, np.float32)
    h = _c(h, np.float32)
    M, N = W.shape
    row_ptr = np.zeros(M + 1, np.int32)
    col = np.zeros(max(nnz_, 1), np.int32)
    val = np.zeros(max(nnz_, 1), np.float32)
    keep = np.zeros(M * N, np.uint8)
    rc = lib.orc_select(_ptr(W), _ptr(h), M, N, nnz_, _ptr(row_ptr), _ptr(col), _ptr(val), _ptr(keep))
    if rc:
        raise RuntimeError("orc_select failed: %d" % rc)
    return row_ptr, col[:nnz_], val[:nnz_], keep.reshape(M, N)


def select_subvectors(W, h, d, n_sel, keep=None, lib=None):
    """keep (1 = kept) with every position of the n_sel most salient sub-vectors set to 0."""
    lib = lib or load()
    W = _c(W, np.float32)
    M, N = W.shape
    keep = np.ones((M, N), np.uint8) if keep is None else np.array(keep, dtype=np.uint8, copy=True, order="C")
    rc = lib.orc_select_subvectors(_ptr(W), _ptr(_c(h, np.float32)), M, N, d, int(n_sel), _ptr(keep))
    if rc:
        raise ValueError("orc_select_subvectors failed: %d" % rc)
    return keep


def select_residual(W, What, h, n_sel, keep=None, lib=None):
    """keep with the n_sel largest weighted residuals among kept positions set to 0."""
    lib = lib or load()
    W = _c(W, np.float32)
    M, N = W.shape
    keep = np.ones((M, N), np.uint8) if keep is None else np.array(keep, dtype=np.uint8, copy=True, order="C")
    rc = lib.orc_select_residual(_ptr(W), _ptr(_c(What, np.float32)), _ptr(_c(h, np.float32)), M, N,
                                 int(n_sel), _ptr(keep))
    if rc:
        raise ValueError("orc_select_residual failed: %d" % rc)
    return keep


def keep_to_csr(W, keep, lib=None):
    """CSR (row_ptr, col, val) of the positions with keep == 0."""
    lib = lib or load()
    W = _c(W, np.float32)
    M, N = W.shape
    keep = _c(keep, np.uint8)
    n = int((keep == 0).sum())
    row_ptr = np.zeros(M + 1, np.int32)
    col = np.zeros(max(n, 1), np.int32)
    val = np.zeros(max(n, 1), np.float32)
    got = lib.orc_keep_to_csr(_ptr(W), _ptr(keep), M, N, _ptr(row_ptr), _ptr(col), _ptr(val))
    assert got == n
    return row_ptr, col[:n], val[:n]


def binorm(W, h, lib=None):
    lib = lib or load()
    W = _c(W, np.float32)
    h = _c(h, np.float32)
    M, N = W.shape
    Wp = np.empty_like(W)
    r = np.empty(M, np.float32)
    c = np.empty(N, np.float32)
    hcol = np.empty(N, np.float32)
    rho = np.empty(M, np.float32)
    lib.orc_binorm(_ptr(W), _ptr(h), M, N, _ptr(Wp), _ptr(r), _ptr(c), _ptr(hcol), _ptr(rho))
    return Wp, r, c, hcol, rho


def init(X, d, perm, K, lib=None):
    """Returns (C [K, d], taken); taken < K means too few distinct sub-vectors."""
    lib = lib or load()
    X = _c(X, np.float32)
    perm = _c(perm, np.int32)
    n_sub = X.size // d
    C = np.zeros((K, d), np.float32)
    taken = lib.orc_init(_ptr(X), n_sub, d, _ptr(perm), K, _ptr(C))
    return C, int(taken)


def assign(X, hcol, rho, keep, d, C, subset=None, nthreads=0, lib=None):
    """X [M, N] (or [n_sub, d] with M,N implied by hcol/rho); returns (idx u16, dist f64)."""
    lib = lib or load()
    X = _c(X, np.float32)
    hcol = _c(hcol, np.float32)
    rho = _c(rho, np.float32)
    keep = _c(keep, np.uint8)
    C = _c(C, np.float32)
    N = hcol.size
    M = X.size // N
    K = C.shape[0]
    sub = None if subset is None else _c(subset, np.int64)
    n = (M * N // d) if sub is None else sub.size
    idx = np.zeros(n, np.uint16)
    dist = np.zeros(n, np.float64)
    lib.orc_assign(_ptr(X), _ptr(hcol), _ptr(rho), _ptr(keep), M, N, d, _ptr(C), K,
                   _ptr(sub), 0 if sub is None else sub.size, _ptr(idx), _ptr(dist), int(nthreads))
    return idx, dist


def objective(X, hcol, rho, keep, d, C, idx, lib=None):
    lib = lib or load()
    X = _c(X, np.float32)
    hcol = _c(hcol, np.float32)
    N = hcol.size
    M = X.size // N
    return float(lib.orc_objective(_ptr(X), _ptr(hcol), _ptr(_c(rho, np.float32)),
                                   _ptr(_c(keep, np.uint8)), M, N, d,
                                   _ptr(_c(C, np.float32)), _ptr(_c(idx, np.uint16))))


def update(X, hcol, rho, keep, d, idx, C, lib=None):
    """Returns (C_new, counts, J against the input C)."""
    lib = lib or load()
    X = _c(X, np.float32)
    hcol = _c(hcol, np.float32)
    N = hcol.size
    M = X.size // N
    Cn = np.array(C, dtype=np.float32, copy=True, order="C")
    K = Cn.shape[0]
    counts = np.zeros(K, np.int32)
    J = lib.orc_update(_ptr(X), _ptr(hcol), _ptr(_c(rho, np.float32)), _ptr(_c(keep, np.uint8)),
                       M, N, d, _ptr(_c(idx, np.uint16)), K, _ptr(Cn), _ptr(counts))
    return Cn, counts, float(J)


def residual(X, d, C, idx, lib=None):
    lib = lib or load()
    X = _c(X, np.float32)
    R = np.empty_like(X)
    lib.orc_residual(_ptr(X), X.size // d, d, _ptr(_c(C, np.float32)), _ptr(_c(idx, np.uint16)), _ptr(R))
    return R


def reconstruct(M, N, d, C1, idx1, C2=None, idx2=None, r=None, c=None,
                row_ptr=None, col=None, val=None, lib=None):
    lib = lib or load()
    What = np.empty((M, N), np.float32)
    lib.orc_reconstruct(M, N, d, _ptr(_c(C1, np.float32)), _ptr(_c(idx1, np.uint16)),
                        _ptr(_c(C2, np.float32)), _ptr(_c(idx2, np.uint16)),
                        _ptr(_c(r, np.float32)), _ptr(_c(c, np.float32)),
                        _ptr(_c(row_ptr, np.int32)), _ptr(_c(col, np.int32)),
                        _ptr(_c(val, np.float32)), _ptr(What))
    return What


def column_order(h, n_out, lib=None):
    """Column order of the grouped fit: the n_out columns with the largest h (ties:
    smaller index) ascending, then the rest ascending."""
    lib = lib or load()
    h = _c(h, np.float32)
    cols = np.zeros(h.size, np.int32)
    rc = lib.orc_column_order(_ptr(h), h.size, int(n_out), _ptr(cols))
    if rc:
        raise ValueError("orc_column_order failed: %d" % rc)
    return cols


def grouped_layout(N, d, n_out, d0, K0, T0, n_groups, K1, T1, K2, T2):
    """[(first column of the order, columns, d, K, T, K2, T2)] per group, in order."""
    groups = []
    if n_out > 0:
        groups.append((0, n_out, d0, K0, T0, 0, 0))
    nb = (N - n_out) // d
    w = -(-nb // n_groups) * d
    for g in range(n_groups):
        c0 = n_out + g * w
        groups.append((c0, min(w, N - c0), d, K1, T1, K2, T2))
    return groups


def fit_grouped(W, h, d, K1, T1, K2, T2, p, n_out, d0, K0, T0, n_groups, perm1_all, perm2_all,
                binorm=False, mask_outliers=True, nthreads=0, lib=None):
    """The grouped fit; returns cols, idx_all, cb_all, CSR, keep, What, J_all."""
    lib = lib or load()
    W = _c(W, np.float32)
    h = _c(h, np.float32)
    M, N = W.shape
    lay = grouped_layout(N, d, n_out, d0, K0, T0, n_groups, K1, T1, K2, T2)
    n_idx = sum(M * Ng // dg * (2 if K2g else 1) for _, Ng, dg, _, _, K2g, _ in lay)
    n_cb = sum(Kg * dg + K2g * dg for _, _, dg, Kg, _, K2g, _ in lay)
    n_J = sum(Tg + 1 + ((T2g + 1) if K2g else 0) for _, _, _, _, Tg, K2g, T2g in lay)
    nz = nnz(M, N, p, lib)
    out = {"cols": np.zeros(N, np.int32), "idx": np.zeros(n_idx, np.uint16), "cb": np.zeros(n_cb, np.float32),
           "row_ptr": np.zeros(M + 1, np.int32), "col": np.zeros(max(nz, 1), np.int32),
           "val": np.zeros(max(nz, 1), np.float32), "keep": np.zeros((M, N), np.uint8),
           "What": np.zeros((M, N), np.float32), "J": np.zeros(n_J), "layout": lay}
    rc = lib.orc_fit_grouped(_ptr(W), _ptr(h), M, N, d, K1, T1, K2, T2, float(p), int(bool(binorm)),
                             int(bool(mask_outliers)), int(n_out), d0, K0, T0, n_groups,
                             _ptr(_c(perm1_all, np.int32)), _ptr(_c(perm2_all, np.int32)), int(nthreads),
                             _ptr(out["cols"]), _ptr(out["idx"]), _ptr(out["cb"]), _ptr(out["row_ptr"]),
                             _ptr(out["col"]), _ptr(out["val"]), _ptr(out["keep"]), _ptr(out["What"]),
                             _ptr(out["J"]))
    if rc:
        raise RuntimeError("orc_fit_grouped failed: %d" % rc)
    out["col"] = out["col"][:nz]
    out["val"] = out["val"][:nz]
    return out


def inverse_hessian_factor(H, damp=0.01):
    """GPTQ's reading of the H^-1 that the error propagation reads: the upper
    Cholesky factor U (U^T U = Hd^-1) of the inverse of the damped Hessian
    Hd = H + damp * mean(diag H) * I, in float64 (numpy)."""
    H = np.asarray(H, dtype=np.float64)
    Hd = H + damp * float(np.mean(np.diag(H))) * np.eye(H.shape[0])
    Hinv = np.linalg.inv(Hd)
    Hinv = 0.5 * (Hinv + Hinv.T)
    return np.linalg.cholesky(Hinv).T


def vptq(W, U, V, C, B, lib=None):
    """Algorithm 1 on W [M x N] with column sub-vectors of length V, codebook C
    [K x V], block size B and the matrix U [N x N] (cast to float32, as the
    library receives it).  Returns idx [N, M/V], What [M, N] (fp32), E [M, N]
    (fp64) and gap [N, M/V]."""
    lib = lib or load()
    W = _c(W, np.float32)
    M, N = W.shape
    C = _c(C, np.float32)
    nv = M // V
    idx = np.zeros((N, nv), np.uint16)
    What = np.zeros((M, N), np.float32)
    E = np.zeros((M, N), np.float64)
    gap = np.zeros((N, nv), np.float64)
    rc = lib.orc_vptq(_ptr(W), _ptr(_c(U, np.float32)), M, N, V, _ptr(C), C.shape[0], int(B), _ptr(idx),
                      _ptr(What), _ptr(E), _ptr(gap))
    if rc:
        raise MemoryError("orc_vptq: allocation failed")
    return idx, What, E, gap


def qgemv(M, N, d, C1, idx1, X, C2=None, idx2=None, r=None, c=None,
          row_ptr=None, col=None, val=None, lib=None):
    """Y = X What^T in float64 (What as reconstruct writes it); X is [B x N]."""
    lib = lib or load()
    X = _c(np.atleast_2d(X), np.float32)
    B = X.shape[0]
    Y = np.empty((B, M), np.float64)
    rc = lib.orc_qgemv(M, N, d, _ptr(_c(C1, np.float32)), _ptr(_c(idx1, np.uint16)),
                       _ptr(_c(C2, np.float32)), _ptr(_c(idx2, np.uint16)),
                       _ptr(_c(r, np.float32)), _ptr(_c(c, np.float32)),
                       _ptr(_c(row_ptr, np.int32)), _ptr(_c(col, np.int32)),
                       _ptr(_c(val, np.float32)), _ptr(X), B, _ptr(Y))
    if rc:
        raise MemoryError("orc_qgemv: allocation failed")
    return Y


def fit(W, h, d, K1, T1, K2, T2, p, binorm=False, mask_outliers=True, perm1=None, perm2=None,
        nthreads=0, lib=None):
    """The whole pipeline; returns a dict of every output (raises on failure)."""
    lib = lib or load()
    W = _c(W, np.float32)
    h = _c(h, np.float32)
    M, N = W.shape
    n_sub = M * N // d
    nz = nnz(M, N, p, lib)
    out = {
        "idx1": np.zeros(n_sub, np.uint16), "C1": np.zeros((K1, d), np.float32),
        "idx2": np.zeros(n_sub, np.uint16), "C2": np.zeros((max(K2, 1), d), np.float32),
        "row_ptr": np.zeros(M + 1, np.int32), "col": np.zeros(max(nz, 1), np.int32),
        "val": np.zeros(max(nz, 1), np.float32), "keep": np.zeros((M, N), np.uint8),
        "Wp": np.zeros((M, N), np.float32), "r": np.ones(M, np.float32),
        "c": np.ones(N, np.float32), "hcol": h.copy(), "rho": np.ones(M, np.float32),
        "What": np.zeros((M, N), np.float32), "J": np.zeros(T1 + 1 + (T2 + 1 if K2 > 0 else 0)),
    }
    perm1 = _c(perm1, np.int32)
    perm2 = _c(perm2, np.int32) if perm2 is not None else perm1
    rc = lib.orc_fit(_ptr(W), _ptr(h), M, N, d, K1, T1, K2, T2, float(p), int(bool(binorm)),
                     int(bool(mask_outliers)), _ptr(perm1), _ptr(perm2), int(nthreads),
                     _ptr(out["idx1"]), _ptr(out["C1"]), _ptr(out["idx2"]), _ptr(out["C2"]),
                     _ptr(out["row_ptr"]), _ptr(out["col"]), _ptr(out["val"]), _ptr(out["keep"]),
                     _ptr(out["Wp"]), _ptr(out["r"]), _ptr(out["c"]), _ptr(out["hcol"]),
                     _ptr(out["rho"]), _ptr(out["What"]), _ptr(out["J"]))
    if rc:
        raise RuntimeError("orc_fit failed: %d" % rc)
    out["col"] = out["col"][:nz]
    out["val"] = out["val"][:nz]
    out["nnz"] = nz
    if K2 == 0:
        out["C2"] = None
    return out
