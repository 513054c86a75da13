"""Python binding of libvq (ctypes).  Argument marshalling only.

Every function takes torch tensors that already live on the GPU (PyTorch is
used for device memory and streams), passes their device pointers and the
current stream to the C ABI declared in include/vq.h, and raises VQError on
a non-zero status.  There is no fallback: if libvq.so is missing or no
gfx950 device is present the call fails.
"""
import ctypes
import math
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvq.so")

VQ_OK, VQ_ERR_INVALID, VQ_ERR_WORKSPACE, VQ_ERR_INIT, VQ_ERR_DEVICE, VQ_ERR_UNSUPPORTED = range(6)
STATUS_NAMES = {0: "VQ_OK", 1: "VQ_ERR_INVALID", 2: "VQ_ERR_WORKSPACE", 3: "VQ_ERR_INIT",
                4: "VQ_ERR_DEVICE", 5: "VQ_ERR_UNSUPPORTED"}


class VQError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), msg))
        self.status = status


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_D = ctypes.c_double


class FitParams(ctypes.Structure):
    _fields_ = [("M", _I64), ("N", _I64), ("d", _I), ("K1", _I), ("iters1", _I), ("K2", _I),
                ("iters2", _I), ("outlier_frac", _D), ("binorm", _I), ("mask_outliers", _I)]


class FitInputs(ctypes.Structure):
    _fields_ = [("W", _P), ("h", _P), ("perm1", _P), ("perm2", _P), ("C1_init", _P), ("C2_init", _P)]


class FitOutputs(ctypes.Structure):
    _fields_ = [("idx1", _P), ("C1", _P), ("idx2", _P), ("C2", _P), ("row_ptr", _P), ("col", _P),
                ("val", _P), ("mask", _P), ("Wp", _P), ("rscale", _P), ("cscale", _P), ("hcol", _P),
                ("rho", _P), ("W_hat", _P), ("J_hist", _P), ("bpw", _P), ("empty_hist", _P)]


class GroupedParams(ctypes.Structure):
    _fields_ = [("fit", FitParams), ("n_out", _I64), ("d0", _I), ("K0", _I), ("iters0", _I), ("n_groups", _I)]


class GroupedInputs(ctypes.Structure):
    _fields_ = [("W", _P), ("h", _P), ("perm1", _P), ("perm2", _P)]


class GroupedOutputs(ctypes.Structure):
    _fields_ = [("cols", _P), ("idx", _P), ("codebooks", _P), ("row_ptr", _P), ("col", _P), ("val", _P),
                ("mask", _P), ("W_hat", _P), ("J_hist", _P), ("bpw", _P)]


# name -> (restype, argtypes); every symbol declared in include/vq.h
SIGNATURES = {
    "vq_version": (ctypes.c_char_p, []),
    "vq_last_error": (ctypes.c_char_p, []),
    "vq_workspace_bytes": (_SZ, [_I64, _I64, _I, _I, _I, _I64]),
    "vq_sparse_select": (_I, [_P, _P, _I64, _I64, _I, _I64, _P, _P, _P, _P, _P, _SZ, _P]),
    "vq_binorm": (_I, [_P, _P, _I64, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "vq_init": (_I, [_P, _I64, _I64, _I, _P, _I, _P, _P, _SZ, _P]),
    "vq_assign": (_I, [_P, _P, _P, _P, _I64, _I64, _I, _P, _I, _P, _P, _P, _SZ, _P]),
    "vq_assign_noalloc": (_I, [_P, _P, _P, _P, _I64, _I64, _I, _P, _I, _P, _P, _P]),
    "vq_assign_exact_count": (_I, [_P, _SZ, _I64, _I, _P]),
    "vq_assign_exact_list": (_I64, [_P, _SZ, _I64, _I, _P, _I64, _P]),
    "vq_nnz": (_I64, [_I64, _I64, _D]),
    "vq_update": (_I, [_P, _P, _P, _P, _I64, _I64, _I, _P, _I, _P, _P, _P, _P, _SZ, _P]),
    "vq_objective": (_I, [_P, _P, _P, _P, _I64, _I64, _I, _P, _I, _P, _P, _P, _SZ, _P]),
    "vq_residual": (_I, [_P, _I64, _I64, _I, _P, _I, _P, _P, _P]),
    "vq_reconstruct": (_I, [_I64, _I64, _I, _P, _I, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P]),
    "vq_select_subvectors": (_I, [_P, _P, _I64, _I64, _I, _I64, _P, _P, _SZ, _P]),
    "vq_select_residual": (_I, [_P, _P, _P, _I64, _I64, _I, _I64, _P, _P, _SZ, _P]),
    "vq_mask_to_csr": (_I, [_P, _P, _I64, _I64, _I, _I64, _P, _P, _P, _P, _SZ, _P]),
    "vq_hessian_factor_workspace_bytes": (_SZ, [_I64]),
    "vq_hessian_factor": (_I, [_P, _I64, _D, _P, _P, _SZ, _P]),
    "vq_vptq_workspace_bytes": (_SZ, [_I64, _I64, _I]),
    "vq_vptq": (_I, [_P, _P, _I64, _I64, _I, _P, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "vq_qgemv_workspace_bytes": (_SZ, [_I64, _I64, _I, _I64]),
    "vq_qgemv": (_I, [_I64, _I64, _I, _P, _I, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _I64, _P, _P, _SZ,
                      _P]),
    "vq_fit": (_I, [ctypes.POINTER(FitParams), ctypes.POINTER(FitInputs), ctypes.POINTER(FitOutputs),
                    _P, _SZ, _P]),
    "vq_grouped_sizes": (_SZ, [ctypes.POINTER(GroupedParams), ctypes.POINTER(_I64), ctypes.POINTER(_I64),
                               ctypes.POINTER(_I64), ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
    "vq_fit_grouped": (_I, [ctypes.POINTER(GroupedParams), ctypes.POINTER(GroupedInputs),
                            ctypes.POINTER(GroupedOutputs), _P, _SZ, _P]),
    "vq_bits_per_weight_grouped": (_D, [ctypes.POINTER(GroupedParams)]),
    "vq_bits_per_weight": (_D, [_I64, _I64, _I, _I, _I, _I64, _I, _I]),
    "vq_timing_enable": (None, [_I]),
    "vq_timing_count": (_I, []),
    "vq_timing_get": (_I, [_I, ctypes.c_char_p, _I, ctypes.POINTER(_I), ctypes.POINTER(_I64),
                           ctypes.POINTER(_D), ctypes.POINTER(_D), ctypes.POINTER(_D)]),
}

_lib = None


def load(path=None):
    """Loads libvq.so; raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libvq.so is not built (%s); run __graft_entry__.build() or "
                           "python hessian_weighted_vector_amd/build.py" % p)
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(st):
    if st != VQ_OK:
        raise VQError(st, load().vq_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dtype(t, dt, name):
    if t is not None and t.dtype != dt:
        raise TypeError("%s must be %s, got %s" % (name, dt, t.dtype))


def workspace_bytes(M, N, d, K1, K2=0, nnz=0):
    return int(load().vq_workspace_bytes(M, N, d, K1, K2, nnz))


def workspace(M, N, d, K1, K2=0, nnz=0, device="cuda"):
    """A byte tensor large enough for every call with these sizes."""
    return torch.empty(max(workspace_bytes(M, N, d, K1, K2, nnz), 256), dtype=torch.uint8, device=device)


def nnz_of(M, N, p):
    """The library's salient count for an M x N matrix and fraction p."""
    n = int(load().vq_nnz(M, N, float(p)))
    if n < 0:
        raise VQError(VQ_ERR_INVALID, load().vq_last_error().decode())
    return n


def sparse_select(W, h, d, nnz, ws):
    _dtype(W, torch.float32, "W")
    M, N = W.shape
    dev = W.device
    row_ptr = torch.empty(M + 1, dtype=torch.int32, device=dev)
    col = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)
    val = torch.empty(max(nnz, 1), dtype=torch.float32, device=dev)
    mask = torch.empty(M * N // d, dtype=torch.uint8, device=dev)
    _check(load().vq_sparse_select(_ptr(W), _ptr(h), M, N, d, nnz, _ptr(row_ptr), _ptr(col), _ptr(val),
                                   _ptr(mask), _ptr(ws), ws.numel(), _stream()))
    return row_ptr, col[:nnz], val[:nnz], mask


def binorm(W, h, ws):
    M, N = W.shape
    Wp = torch.empty_like(W)
    r = torch.empty(M, dtype=torch.float32, device=W.device)
    c = torch.empty(N, dtype=torch.float32, device=W.device)
    hcol = torch.empty(N, dtype=torch.float32, device=W.device)
    rho = torch.empty(M, dtype=torch.float32, device=W.device)
    _check(load().vq_binorm(_ptr(W), _ptr(h), M, N, _ptr(Wp), _ptr(r), _ptr(c), _ptr(hcol), _ptr(rho),
                            _ptr(ws), ws.numel(), _stream()))
    return Wp, r, c, hcol, rho


def init(X, d, perm_host, K, ws):
    """perm_host: numpy int32 array (host)."""
    M, N = X.shape
    perm = np.ascontiguousarray(perm_host, dtype=np.int32)
    C = torch.empty((K, d), dtype=torch.float32, device=X.device)
    _check(load().vq_init(_ptr(X), M, N, d, perm.ctypes.data, K, _ptr(C), _ptr(ws), ws.numel(), _stream()))
    return C


def assign(X, hcol, rho, mask, d, C, ws, want_dist=False, idx=None, dist=None):
    _dtype(X, torch.float32, "X")
    _dtype(C, torch.float32, "C")
    _dtype(mask, torch.uint8, "mask")
    M, N = X.shape
    K = C.shape[0]
    n_sub = M * N // d
    if idx is None:
        idx = torch.empty(n_sub, dtype=torch.uint16, device=X.device)
    if want_dist and dist is None:
        dist = torch.empty(n_sub, dtype=torch.float32, device=X.device)
    _check(load().vq_assign(_ptr(X), _ptr(hcol), _ptr(rho), _ptr(mask), M, N, d, _ptr(C), K, _ptr(idx),
                            _ptr(dist) if want_dist else None, _ptr(ws), ws.numel(), _stream()))
    return (idx, dist) if want_dist else idx


def assign_exact_count(ws, n_sub, K):
    return int(load().vq_assign_exact_count(_ptr(ws), ws.numel(), n_sub, K, _stream()))


def assign_exact_list(ws, n_sub, K):
    """Sorted ids (numpy int32) of the sub-vectors the last assign re-searched exactly."""
    lib = load()
    n = int(lib.vq_assign_exact_list(_ptr(ws), ws.numel(), n_sub, K, None, 0, _stream()))
    if n < 0:
        raise VQError(VQ_ERR_INVALID, lib.vq_last_error().decode())
    out = np.zeros(max(n, 1), np.int32)
    m = int(lib.vq_assign_exact_list(_ptr(ws), ws.numel(), n_sub, K, out.ctypes.data, n, _stream()))
    if m != n:
        raise VQError(VQ_ERR_DEVICE, "exact-path list changed between reads")
    return np.sort(out[:n])


def update(X, hcol, rho, mask, d, idx, C, ws, want_counts=True, want_J=True):
    """In place on C; returns (counts, J tensor [1] float64)."""
    M, N = X.shape
    K = C.shape[0]
    counts = torch.empty(K, dtype=torch.int32, device=X.device) if want_counts else None
    J = torch.empty(1, dtype=torch.float64, device=X.device) if want_J else None
    _check(load().vq_update(_ptr(X), _ptr(hcol), _ptr(rho), _ptr(mask), M, N, d, _ptr(idx), K, _ptr(C),
                            _ptr(counts), _ptr(J), _ptr(ws), ws.numel(), _stream()))
    return counts, J


def objective(X, hcol, rho, mask, d, C, idx, ws):
    M, N = X.shape
    J = torch.empty(1, dtype=torch.float64, device=X.device)
    _check(load().vq_objective(_ptr(X), _ptr(hcol), _ptr(rho), _ptr(mask), M, N, d, _ptr(C), C.shape[0],
                               _ptr(idx), _ptr(J), _ptr(ws), ws.numel(), _stream()))
    return J


def residual(X, d, C, idx):
    M, N = X.shape
    R = torch.empty_like(X)
    _check(load().vq_residual(_ptr(X), M, N, d, _ptr(C), C.shape[0], _ptr(idx), _ptr(R), _stream()))
    return R


def reconstruct(M, N, d, C1, idx1, C2=None, idx2=None, rscale=None, cscale=None, row_ptr=None, col=None,
                val=None, out=None):
    W_hat = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=C1.device)
    _check(load().vq_reconstruct(M, N, d, _ptr(C1), C1.shape[0], _ptr(idx1), _ptr(C2),
                                 0 if C2 is None else C2.shape[0], _ptr(idx2), _ptr(rscale), _ptr(cscale),
                                 _ptr(row_ptr), _ptr(col), _ptr(val), _ptr(W_hat), _stream()))
    return W_hat


def select_subvectors(W, h, d, n_sel, mask, ws):
    """OR every bit of the n_sel most salient sub-vectors into mask (in place)."""
    M, N = W.shape
    _check(load().vq_select_subvectors(_ptr(W), _ptr(h), M, N, d, int(n_sel), _ptr(mask), _ptr(ws), ws.numel(),
                                       _stream()))
    return mask


def select_residual(W, W_hat, h, d, n_sel, mask, ws):
    """OR the n_sel largest weighted residuals among clear positions into mask (in place)."""
    M, N = W.shape
    _check(load().vq_select_residual(_ptr(W), _ptr(W_hat), _ptr(h), M, N, d, int(n_sel), _ptr(mask), _ptr(ws),
                                     ws.numel(), _stream()))
    return mask


def mask_to_csr(W, mask, d, nnz_cap, ws):
    """(row_ptr, col, val) of the held positions; row_ptr[M] is the full count."""
    M, N = W.shape
    row_ptr = torch.empty(M + 1, dtype=torch.int32, device=W.device)
    col = torch.empty(max(int(nnz_cap), 1), dtype=torch.int32, device=W.device)
    val = torch.empty(max(int(nnz_cap), 1), dtype=torch.float32, device=W.device)
    _check(load().vq_mask_to_csr(_ptr(W), _ptr(mask), M, N, d, int(nnz_cap), _ptr(row_ptr), _ptr(col), _ptr(val),
                                 _ptr(ws), ws.numel(), _stream()))
    return row_ptr, col, val


def hessian_factor(H, damp=0.01, ws=None):
    """U [N, N] (float32, upper): U^T U = (H + damp mean(diag H) I)^-1."""
    N = H.shape[0]
    U = torch.empty_like(H)
    if ws is None:
        ws = torch.empty(max(int(load().vq_hessian_factor_workspace_bytes(N)), 256), dtype=torch.uint8,
                         device=H.device)
    _check(load().vq_hessian_factor(_ptr(H), N, float(damp), _ptr(U), _ptr(ws), ws.numel(), _stream()))
    return U


def vptq(W, U, V, C, B=128, want_E=False, ws=None):
    """Algorithm 1 (column sub-vectors of length V): returns idx [N, M/V], W_hat [M, N]
    and, with want_E, E [M, N]."""
    M, N = W.shape
    dev = W.device
    idx = torch.empty((N, M // V), dtype=torch.uint16, device=dev)
    W_hat = torch.empty_like(W)
    E = torch.empty_like(W) if want_E else None
    if ws is None:
        ws = torch.empty(max(int(load().vq_vptq_workspace_bytes(M, N, V)), 256), dtype=torch.uint8, device=dev)
    _check(load().vq_vptq(_ptr(W), _ptr(U), M, N, V, _ptr(C), C.shape[0], int(B), _ptr(idx), _ptr(W_hat),
                          _ptr(E), _ptr(ws), ws.numel(), _stream()))
    return idx, W_hat, E


def qgemv_workspace_bytes(M, N, d, B):
    return int(load().vq_qgemv_workspace_bytes(M, N, d, B))


def qgemv(M, N, d, C1, idx1, X, C2=None, idx2=None, rscale=None, cscale=None, row_ptr=None, col=None,
          val=None, out=None, ws=None):
    """Y = X W_hat^T from the compressed form (X [B x N] -> Y [B x M], float32)."""
    B = X.shape[0]
    Y = out if out is not None else torch.empty((B, M), dtype=torch.float32, device=X.device)
    need = qgemv_workspace_bytes(M, N, d, B)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=X.device)
    _check(load().vq_qgemv(M, N, d, _ptr(C1), C1.shape[0], _ptr(idx1), _ptr(C2),
                           0 if C2 is None else C2.shape[0], _ptr(idx2), _ptr(rscale), _ptr(cscale),
                           _ptr(row_ptr), _ptr(col), _ptr(val), _ptr(X), B, _ptr(Y), _ptr(ws),
                           0 if ws is None else ws.numel(), _stream()))
    return Y


def grouped_params(M, N, d, K1, iters1, K2, iters2, outlier_frac, binorm, mask_outliers, n_out, d0, K0, iters0,
                   n_groups):
    return GroupedParams(FitParams(M, N, d, K1, iters1, K2, iters2, float(outlier_frac), int(bool(binorm)),
                                   int(bool(mask_outliers))), int(n_out), d0, K0, iters0, n_groups)


def grouped_sizes(params):
    """(workspace bytes, n_idx, n_codebook, n_J, n_perm1, n_perm2)."""
    v = [_I64(0) for _ in range(5)]
    ws = load().vq_grouped_sizes(ctypes.byref(params), *[ctypes.byref(x) for x in v])
    return (int(ws),) + tuple(int(x.value) for x in v)


def fit_grouped(W, h, params, perm1, perm2=None, ws=None):
    """The grouped fit; returns a dict of the outputs (device tensors; J and bpw on the host)."""
    M, N = W.shape
    dev = W.device
    wsb, n_idx, n_cb, n_J, n_p1, n_p2 = grouped_sizes(params)
    if wsb == 0:
        raise ValueError("the column groups do not split these sizes")
    nnz = nnz_of(M, N, params.fit.outlier_frac)
    o = {"cols": torch.empty(N, dtype=torch.int32, device=dev),
         "idx": torch.empty(max(n_idx, 1), dtype=torch.uint16, device=dev),
         "codebooks": torch.empty(max(n_cb, 1), dtype=torch.float32, device=dev),
         "row_ptr": torch.empty(M + 1, dtype=torch.int32, device=dev),
         "col": torch.empty(max(nnz, 1), dtype=torch.int32, device=dev),
         "val": torch.empty(max(nnz, 1), dtype=torch.float32, device=dev),
         "mask": torch.empty(M * N // params.fit.d, dtype=torch.uint8, device=dev),
         "W_hat": torch.empty_like(W)}
    J = np.zeros(max(n_J, 1), np.float64)
    bpw = np.zeros(1, np.float64)
    p1 = np.ascontiguousarray(perm1, dtype=np.int32)
    p2 = None if perm2 is None else np.ascontiguousarray(perm2, dtype=np.int32)
    if ws is None:
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    inputs = GroupedInputs(_ptr(W), _ptr(h), p1.ctypes.data, None if p2 is None else p2.ctypes.data)
    outputs = GroupedOutputs(_ptr(o["cols"]), _ptr(o["idx"]), _ptr(o["codebooks"]), _ptr(o["row_ptr"]),
                             _ptr(o["col"]), _ptr(o["val"]), _ptr(o["mask"]), _ptr(o["W_hat"]), J.ctypes.data,
                             bpw.ctypes.data)
    _check(load().vq_fit_grouped(ctypes.byref(params), ctypes.byref(inputs), ctypes.byref(outputs), _ptr(ws),
                                 ws.numel(), _stream()))
    o["col"] = o["col"][:nnz]
    o["val"] = o["val"][:nnz]
    o["J"] = J[:n_J]
    o["bpw"] = float(bpw[0])
    return o


def timing_enable(on=True):
    load().vq_timing_enable(int(bool(on)))


def timing_records():
    """[(name, K, launches, total_ms, min_ms, max_ms)] of the recorded step timings."""
    lib = load()
    out = []
    for i in range(lib.vq_timing_count()):
        buf = ctypes.create_string_buffer(64)
        K, n = _I(0), _I64(0)
        tot, mn, mx = _D(0), _D(0), _D(0)
        if lib.vq_timing_get(i, buf, 64, ctypes.byref(K), ctypes.byref(n), ctypes.byref(tot),
                             ctypes.byref(mn), ctypes.byref(mx)) == 0:
            out.append((buf.value.decode(), K.value, n.value, tot.value, mn.value, mx.value))
    return out


def bits_per_weight(M, N, d, K1, K2, nnz, cb_bits=32, binorm=False):
    return float(load().vq_bits_per_weight(M, N, d, K1, K2, nnz, cb_bits, int(bool(binorm))))


def fit(W, h, d, K1, iters1, K2=0, iters2=0, outlier_frac=0.0, binorm=False, mask_outliers=True,
        perm1=None, perm2=None, C1_init=None, C2_init=None, ws=None):
    """The whole pipeline on the GPU; returns a dict of device tensors + host J/bpw."""
    M, N = W.shape
    dev = W.device
    n_sub = M * N // d
    nnz = nnz_of(M, N, outlier_frac)
    if ws is None:
        ws = workspace(M, N, d, K1, K2, nnz, dev)
    o = {
        "idx1": torch.empty(n_sub, dtype=torch.uint16, device=dev),
        "C1": torch.empty((K1, d), dtype=torch.float32, device=dev),
        "idx2": torch.empty(n_sub if K2 > 0 else 1, dtype=torch.uint16, device=dev),
        "C2": torch.empty((max(K2, 1), d), dtype=torch.float32, device=dev),
        "row_ptr": torch.empty(M + 1, dtype=torch.int32, device=dev),
        "col": torch.empty(max(nnz, 1), dtype=torch.int32, device=dev),
        "val": torch.empty(max(nnz, 1), dtype=torch.float32, device=dev),
        "mask": torch.empty(n_sub, dtype=torch.uint8, device=dev),
        "W_hat": torch.empty((M, N), dtype=torch.float32, device=dev),
    }
    if binorm:
        o.update({"Wp": torch.empty_like(W), "rscale": torch.empty(M, dtype=torch.float32, device=dev),
                  "cscale": torch.empty(N, dtype=torch.float32, device=dev),
                  "hcol": torch.empty(N, dtype=torch.float32, device=dev),
                  "rho": torch.empty(M, dtype=torch.float32, device=dev)})
    nJ = iters1 + 1 + (iters2 + 1 if K2 > 0 else 0)
    J = np.zeros(nJ, np.float64)
    bpw = np.zeros(1, np.float64)
    empty = np.zeros(max(iters1 + (iters2 if K2 > 0 else 0), 1), np.int64)
    p1 = None if perm1 is None else np.ascontiguousarray(perm1, dtype=np.int32)
    p2 = None if perm2 is None else np.ascontiguousarray(perm2, dtype=np.int32)
    params = FitParams(M, N, d, K1, iters1, K2, iters2, float(outlier_frac), int(bool(binorm)),
                       int(bool(mask_outliers)))
    inputs = FitInputs(_ptr(W), _ptr(h), None if p1 is None else p1.ctypes.data,
                       None if p2 is None else p2.ctypes.data, _ptr(C1_init), _ptr(C2_init))
    g = lambda k: _ptr(o[k]) if k in o else None  # noqa: E731
    outputs = FitOutputs(g("idx1"), g("C1"), g("idx2"), g("C2"), g("row_ptr"), g("col"), g("val"), g("mask"),
                         g("Wp"), g("rscale"), g("cscale"), g("hcol"), g("rho"), g("W_hat"),
                         J.ctypes.data, bpw.ctypes.data, empty.ctypes.data)
    _check(load().vq_fit(ctypes.byref(params), ctypes.byref(inputs), ctypes.byref(outputs), _ptr(ws),
                         ws.numel(), _stream()))
    o["col"] = o["col"][:nnz]
    o["val"] = o["val"][:nnz]
    o["J"] = J
    o["empty"] = empty[:iters1 + (iters2 if K2 > 0 else 0)]
    o["bpw"] = float(bpw[0])
    o["nnz"] = nnz
    if K2 == 0:
        o["C2"] = None
        o["idx2"] = None
    return o
