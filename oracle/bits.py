"""Bits-per-weight closed form (test infrastructure; part of the oracle).

VPTQ page, "End-to-End Quantization Pipeline" (compression ratio): original
bits over codebook bits plus index bits, with one ceil(log2 k)-bit index per
V-element vector and a [k, V] codebook of b_cb-bit entries.  The worked
example there (4096 x 4096, V = 8, k = 256, fp16 codebook) gives a ratio of
about 15.97, i.e. about 1.002 bits per weight.

Extended here to the stored form of this pipeline (the page gives no
accounting for the sparse part or the scales; this is a reading):
  bits = n_sub * (ceil(log2 K1) + ceil(log2 K2))      index matrices
       + d * (K1 + K2) * b_cb                          codebooks
       + 64 * nnz                                      CSR column + exact value
       + 32 * (M + 1)          if nnz > 0              CSR row pointer
       + 32 * (M + N)          if bi-normalized        row and column scales
  bpw  = bits / (M * N)
"""
import math


def _index_bits(K: int) -> int:
    return 0 if K <= 1 else math.ceil(math.log2(K))


def bits_per_weight(M, N, d, K1, K2, nnz, cb_bits=32, binorm=False):
    n_sub = M * N // d
    bits = n_sub * (_index_bits(K1) + (_index_bits(K2) if K2 > 0 else 0))
    bits += d * (K1 + (K2 if K2 > 0 else 0)) * cb_bits
    bits += 64 * nnz
    if nnz > 0:
        bits += 32 * (M + 1)
    if binorm:
        bits += 32 * (M + N)
    return bits / (M * N)


def bits_per_weight_grouped(M, N, groups, nnz, n_out, cb_bits=32, binorm=False):
    """Grouped form (VPTQ page, "Outlier Elimination" and its group partitioning:
    every group stores its own indices and codebooks).  groups = [(N_g, d_g, K_g,
    K2_g)]; one int32 per outlier column records which columns were held apart."""
    bits = 0
    for Ng, dg, Kg, K2g in groups:
        ns = M * Ng // dg
        bits += ns * (_index_bits(Kg) + (_index_bits(K2g) if K2g > 0 else 0))
        bits += dg * (Kg + (K2g if K2g > 0 else 0)) * cb_bits
    bits += 64 * nnz
    if nnz > 0:
        bits += 32 * (M + 1)
    if binorm:
        bits += 32 * (M + N)
    if n_out > 0:
        bits += 32 * n_out
    return bits / (M * N)


def compression_ratio_single(n_elem, V, k, orig_bits=16, cb_bits=16):
    """The page's ratio for one codebook: orig / (codebook + index bits)."""
    return (orig_bits * n_elem) / (V * k * cb_bits + n_elem * _index_bits(k) / V)
