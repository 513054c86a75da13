"""The CPU oracle (test infrastructure).

Plain fp64 C (``vq_oracle.c``) loaded through ctypes, plus the bits-per-weight
closed form in Python.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP library and never imports it.
"""
from .oracle import (build, load, nnz, select, select_subvectors, select_residual, keep_to_csr, binorm, init, assign, objective, update,
                     residual, reconstruct, qgemv, inverse_hessian_factor, vptq, fit,
                     column_order, grouped_layout, fit_grouped)
from .bits import bits_per_weight, bits_per_weight_grouped, compression_ratio_single

__all__ = ["build", "load", "nnz", "select", "select_subvectors", "select_residual", "keep_to_csr", "binorm", "init", "assign", "objective",
           "update", "residual", "reconstruct", "qgemv", "inverse_hessian_factor", "vptq", "fit", "column_order", "grouped_layout", "fit_grouped", "bits_per_weight",
           "compression_ratio_single", "bits_per_weight_grouped"]
