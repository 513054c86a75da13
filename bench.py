#!/usr/bin/env python3
"""Benchmark of the weighted-VQ hot path on one MI355X.

One step = the whole per-matrix fit through the C ABI (vq_fit): salience
selection into the exact sparse correction, bi-normalization, codebook
seeding, T1 Lloyd iterations (weighted assignment + weighted-mean update) at
K1, residual, seeding, T2 iterations at K2, and reconstruction, on the
LLaMA-2-7B MLP workload (W 4096 x 11008, bf16 values held as fp32, d = 8,
K1 = 65536, T1 = 10, K2 = 256, T2 = 10, 1% salient, bi-normalized).  Inputs
are seeded synthetic arrays already resident in HBM.

value = sub-vector assignments per second over Lloyd iterations, whole step:
n_sub * (T1 + T2) / (wall time per step), in G/s.

The roofline entry is for the dominant kernel, the matrix-core search of the
stage-1 assignment (K = 65536): algorithmic flops = 32 per (sub-vector,
centroid) pair (the 2d = 16-term inner product, one multiply and one add
each) times n_sub * K pairs per launch, divided by that kernel's average
duration measured with HIP events on the stream it runs on, during the timed
steps.  The search runs on the fp16 matrix cores (each fp32 operand split
into two fp16 parts, two or three fp16 products per term, fp32
accumulation), so the peak is MI355X's dense fp16 figure.  The CPU baseline is the
C oracle's exhaustive float64 assignment against the same 65536-entry
codebook on a bounded sample of sub-vectors.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP16_MFMA_TFLOPS = 2500.0    # MI355X dense fp16 matrix peak
PEAK_FP32_MFMA_TFLOPS = 157.3     # MI355X dense fp32 matrix peak (what an fp32 search is bounded by)
PEAK_HBM_GBS = 8000.0             # MI355X HBM3E
PEAK_FP64_TFLOPS = 78.6           # MI355X float64 (vector and matrix)


def algorithmic_bytes_update(n_sub, M, N, d, K):
    # x (d fp32) + index (u16) + mask byte per sub-vector; hcol and rho; codebook in and out
    return n_sub * (4 * d + 2 + 1) + 4 * N + 4 * M + 2 * K * d * 4


def algorithmic_bytes_reconstruct(n_sub, M, N, d, K1, K2, nnz, binorm):
    b = n_sub * (4 * d + 2 + (2 if K2 else 0)) + 8 * nnz + 4 * (M + 1) + 4 * (K1 + K2) * d
    if binorm:
        b += 4 * (M + N)
    return b


def search_profile(kernel_src):
    """The committed counter summary of the 4096 x 11008 workload's stage-1 search,
    if it was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "assign_search_c4_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        prof = json.load(f)
    with open(kernel_src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    return prof if prof.get("kernel_src_sha256") == sha else None


def row_table(cfg, recs, nnz, oracle_ms):
    """Per-row GPU time per call (HIP events during the timed steps) against the row's
    roofline, with the oracle's CPU time for the same operation at the same size."""
    M, N, d, n_sub = cfg.M, cfg.N, cfg.d, cfg.n_sub
    rec = {(r[0], r[1]): r for r in recs}

    def ms(name, K):
        r = rec.get((name, K))
        return r[3] / r[2] if r else None

    def hbm(name, K, nbytes, key):
        t = ms(name, K)
        if t is None:
            return None
        out = {"gpu_ms": round(t, 4), "algorithmic_MB": round(nbytes / 1e6, 1),
               "GBs": round(nbytes / (t * 1e-3) / 1e9, 1), "frac_hbm": round(nbytes / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        if key in oracle_ms:
            out["oracle_ms"] = round(oracle_ms[key], 1)
        return out

    rows = {
        "A1_select": hbm("select", 0, 4 * M * N + 4 * N + 8 * nnz + 4 * (M + 1) + n_sub, "select"),
        "A2_binorm": hbm("binorm", 0, 8 * M * N + 8 * (M + N), "binorm") if cfg.binorm else None,
        "A5_update_stage1": hbm("update", cfg.K1, algorithmic_bytes_update(n_sub, M, N, d, cfg.K1), "update"),
        "A5_objective": hbm("objective", cfg.K1, n_sub * (4 * d + 3) + 4 * (M + N), "objective"),
        "A6_residual": hbm("residual", cfg.K1, n_sub * (8 * d + 2) + 4 * cfg.K1 * d, "residual"),
        "A7_reconstruct": hbm("reconstruct", cfg.K1, algorithmic_bytes_reconstruct(n_sub, M, N, d, cfg.K1, cfg.K2, nnz,
                                                                              cfg.binorm), "reconstruct"),
    }
    t = ms("init", cfg.K1)
    if t is not None:
        rows["A3_init"] = {"gpu_ms": round(t, 4), "note": "device gather + host walk over a hash set"}
        if "init" in oracle_ms:
            rows["A3_init"]["oracle_ms"] = round(oracle_ms["init"], 1)
    t = ms("assign_search", cfg.K1)
    if t is not None:
        fl = 32.0 * n_sub * cfg.K1
        rows["A4_assign_stage1"] = {"gpu_ms": round(t, 4), "algorithmic_TFLOP": round(fl / 1e12, 2),
                                    "TFLOPs": round(fl / (t * 1e-3) / 1e12, 1),
                                    "frac_fp16_mfma": round(fl / (t * 1e-3) / 1e12 / PEAK_FP16_MFMA_TFLOPS, 4)}
        if "assign" in oracle_ms:
            rows["A4_assign_stage1"]["oracle_ms"] = round(oracle_ms["assign"], 1)
    return {k: v for k, v in rows.items() if v is not None}


def cpu_rows(cfg, inp, nnz):
    """The oracle on each row at the workload's full size (one call each), on inputs the
    oracle makes itself or seeded synthetic indices; returns milliseconds per row."""
    import numpy as np

    import oracle
    out = {}

    def timed(key, f):
        t0 = time.perf_counter()
        r = f()
        out[key] = (time.perf_counter() - t0) * 1e3
        return r

    W, h = inp["W"], inp["h"]
    _, _, _, keep = timed("select", lambda: oracle.select(W, h, nnz))
    if cfg.binorm:
        Wp, r, c, hcol, rho = timed("binorm", lambda: oracle.binorm(W, h))
    else:
        Wp, r, c, hcol, rho = W, None, None, h, None
    C1, _ = timed("init", lambda: oracle.init(Wp, cfg.d, inp["perm1"], cfg.K1))
    g = np.random.default_rng([cfg.cid, 91])
    i1 = g.integers(0, cfg.K1, size=cfg.n_sub).astype(np.uint16)
    timed("update", lambda: oracle.update(Wp, hcol, rho, keep, cfg.d, i1, C1))
    timed("objective", lambda: oracle.objective(Wp, hcol, rho, keep, cfg.d, C1, i1))
    R = timed("residual", lambda: oracle.residual(Wp, cfg.d, C1, i1))
    if cfg.K2:
        C2, _ = oracle.init(R, cfg.d, inp["perm2"], cfg.K2)
        i2 = g.integers(0, cfg.K2, size=cfg.n_sub).astype(np.uint16)
    else:
        C2, i2 = None, None
    M, N = W.shape
    per = g.integers(0, 2 * max(1, nnz // M), size=M)
    rp = np.concatenate([[0], np.cumsum(per)]).astype(np.int32)
    col = np.concatenate([np.sort(g.choice(N, min(k, N), replace=False)) for k in per]).astype(np.int32)
    val = np.ones(col.size, np.float32)
    timed("reconstruct", lambda: oracle.reconstruct(M, N, cfg.d, C1, i1, C2, i2, r, c, rp, col, val))
    return out


def qgemv_inputs(cfg, inp):
    """Seeded compressed form of the workload's matrix for the fused product: the
    full codebook sizes, uniform indices, codebook rows drawn from the matrix,
    row/column scales when the workload bi-normalizes, and a CSR with about the
    workload's salient fraction per row holding the matrix's exact values."""
    import numpy as np
    g = np.random.default_rng([cfg.cid, 93])
    M, N, d, n_sub = cfg.M, cfg.N, cfg.d, cfg.n_sub
    flat = inp["W"].reshape(-1, d)
    C1 = flat[np.sort(g.choice(n_sub, cfg.K1, replace=False))].copy()
    K2 = cfg.K2
    C2 = (0.1 * flat[np.sort(g.choice(n_sub, K2, replace=False))]).astype(np.float32) if K2 else None
    i1 = g.integers(0, cfg.K1, n_sub).astype(np.uint16)
    i2 = g.integers(0, K2, n_sub).astype(np.uint16) if K2 else None
    r = g.uniform(0.5, 2.0, M).astype(np.float32) if cfg.binorm else None
    c = g.uniform(0.5, 2.0, N).astype(np.float32) if cfg.binorm else None
    per = g.integers(0, int(2 * cfg.p * N) + 1, size=M)
    rp = np.concatenate([[0], np.cumsum(per)]).astype(np.int32)
    col = np.concatenate([np.sort(g.choice(N, k, replace=False)) for k in per]).astype(np.int32)
    val = inp["W"][np.repeat(np.arange(M), per), col].copy()
    return dict(C1=C1, idx1=i1, C2=C2, idx2=i2, r=r, c=c, row_ptr=rp, col=col, val=val)


def qgemv_bytes(cfg, q, B):
    """Compressed bytes one fused-product call must move: indices, codebooks,
    scales, the CSR, the activations in and the outputs out."""
    M, N, d, n_sub = cfg.M, cfg.N, cfg.d, cfg.n_sub
    b = n_sub * 2 * (2 if q["C2"] is not None else 1) + q["C1"].nbytes
    b += q["C2"].nbytes if q["C2"] is not None else 0
    b += 4 * (M + N) if q["r"] is not None else 0
    b += q["row_ptr"].nbytes + q["col"].nbytes + q["val"].nbytes
    return b + 4 * B * (N + M)


def qgemv_bench(cfg, inp, run_oracle, reps=50):
    """The fused dequantize-and-multiply at one token (decode) and eight tokens,
    timed with HIP events on its stream, against HBM peak on the compressed bytes;
    beside it the materialized path (reconstruct, then a dense float32 product)
    and the oracle (float64, one token)."""
    import numpy as np
    import torch

    from hessian_weighted_vector_amd import vq
    q = qgemv_inputs(cfg, inp)
    M, N, d = cfg.M, cfg.N, cfg.d
    gq = {k: (None if v is None else torch.from_numpy(v).cuda()) for k, v in q.items()}
    args = (gq["C2"], gq["idx2"], gq["r"], gq["c"], gq["row_ptr"], gq["col"], gq["val"])
    out = {}
    for B in (1, 8):
        X = torch.from_numpy(np.random.default_rng([cfg.cid, 94, B]).standard_normal((B, N)).astype(np.float32)).cuda()
        Y = torch.empty((B, M), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(vq.qgemv_workspace_bytes(M, N, d, B), 256), dtype=torch.uint8, device="cuda")
        for _ in range(3):
            vq.qgemv(M, N, d, gq["C1"], gq["idx1"], X, *args, out=Y, ws=ws)
        torch.cuda.synchronize()
        vq.timing_enable(True)
        # keep the device busy while the host enqueues the calls, so that the
        # per-call events bracket back-to-back kernels and not launch gaps
        torch.cuda._sleep(int(2e7))
        for _ in range(reps):
            vq.qgemv(M, N, d, gq["C1"], gq["idx1"], X, *args, out=Y, ws=ws)
        torch.cuda.synchronize()
        rec = {(r[0], r[1]): r for r in vq.timing_records()}[("qgemv", cfg.K1)]
        vq.timing_enable(False)
        t = rec[3] / rec[2]
        nbytes = qgemv_bytes(cfg, q, B)
        e = {"gpu_us": round(t * 1e3, 2), "tokens_per_s": round(B / (t * 1e-3), 1),
             "compressed_MB": round(nbytes / 1e6, 2), "GBs": round(nbytes / (t * 1e-3) / 1e9, 1),
             "frac_hbm": round(nbytes / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
             "dense_fp32_equivalent_GBs": round(4.0 * M * N / (t * 1e-3) / 1e9, 1)}
        # the materialized path: write What, then a dense float32 product
        What = torch.empty((M, N), dtype=torch.float32, device="cuda")
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for _ in range(2):
            vq.reconstruct(M, N, d, gq["C1"], gq["idx1"], *args, out=What)
            torch.matmul(X, What.t())
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(10):
            vq.reconstruct(M, N, d, gq["C1"], gq["idx1"], *args, out=What)
            torch.matmul(X, What.t())
        ev[1].record()
        torch.cuda.synchronize()
        e["materialized_us"] = round(ev[0].elapsed_time(ev[1]) / 10 * 1e3, 1)
        del What
        if run_oracle and B == 1:
            import oracle
            Xh = X.cpu().numpy()
            t0 = time.perf_counter()
            oracle.qgemv(M, N, d, q["C1"], q["idx1"], Xh, q["C2"], q["idx2"], q["r"], q["c"], q["row_ptr"],
                         q["col"], q["val"])
            e["oracle_ms"] = round((time.perf_counter() - t0) * 1e3, 1)
        out["B%d" % B] = e
    return out


def correction_bench(cfg, inp, out, W, h, ws, run_oracle, reps=5):
    """The unified sparse correction on the fit's output: 0.25% salient sub-vectors
    and 0.5% largest weighted residuals ORed into the fit's mask, then the CSR.
    HIP-event time per call against the algorithmic bytes (one read of each input,
    the mask read and written, the CSR written); the oracle beside it on seeded
    inputs of the same size."""
    import numpy as np
    import torch

    from hessian_weighted_vector_amd import vq
    M, N, d, n_sub = cfg.M, cfg.N, cfg.d, cfg.n_sub
    n_sv, n_res = n_sub // 400, (M * N) // 200
    cap = out["nnz"] + n_sv * d + n_res
    What = vq.reconstruct(M, N, d, out["C1"], out["idx1"], out["C2"], out["idx2"], out.get("rscale"),
                          out.get("cscale"))
    torch.cuda.synchronize()
    vq.timing_enable(True)
    torch.cuda._sleep(int(2e7))
    for _ in range(reps):
        mask = out["mask"].clone()
        vq.select_subvectors(W, h, d, n_sv, mask, ws)
        vq.select_residual(W, What, h, d, n_res, mask, ws)
        rp, _, _ = vq.mask_to_csr(W, mask, d, cap, ws)
    torch.cuda.synchronize()
    rec = {r[0]: r for r in vq.timing_records()}
    vq.timing_enable(False)
    held = int(rp[-1].item())
    nb = {"select_subvectors": 4 * M * N + 4 * N + 2 * n_sub,
          "select_residual": 8 * M * N + 4 * N + 2 * n_sub,
          "mask_to_csr": n_sub + 12 * held + 4 * (M + 1)}
    res = {"held_positions": held, "n_subvectors": n_sv, "n_residuals": n_res}
    for k, b in nb.items():
        t = rec[k][3] / rec[k][2]
        res[k] = {"gpu_ms": round(t, 4), "algorithmic_MB": round(b / 1e6, 1),
                  "GBs": round(b / (t * 1e-3) / 1e9, 1), "frac_hbm": round(b / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    if run_oracle:
        import oracle
        Wn, hn = inp["W"], inp["h"]
        g = np.random.default_rng([cfg.cid, 96])
        C1 = Wn.reshape(-1, d)[np.sort(g.choice(n_sub, 4096, replace=False))].copy()
        Wq = oracle.reconstruct(M, N, d, C1, g.integers(0, 4096, n_sub).astype(np.uint16))
        keep = np.ones((M, N), np.uint8)
        t0 = time.perf_counter()
        keep = oracle.select_subvectors(Wn, hn, d, n_sv, keep=keep)
        t1 = time.perf_counter()
        keep = oracle.select_residual(Wn, Wq, hn, n_res, keep=keep)
        t2 = time.perf_counter()
        oracle.keep_to_csr(Wn, keep)
        t3 = time.perf_counter()
        res["select_subvectors"]["oracle_ms"] = round((t1 - t0) * 1e3, 1)
        res["select_residual"]["oracle_ms"] = round((t2 - t1) * 1e3, 1)
        res["mask_to_csr"]["oracle_ms"] = round((t3 - t2) * 1e3, 1)
    return res


def vptq_bench(cfg, inp, run_oracle, V=8, B=128):
    """VPTQ Algorithm 1 on the workload's matrix: the inverse-Hessian factor from
    H = X^T X of the workload's activations (float64 Cholesky and triangular
    inverse), then the column-by-column quantization with the workload's codebook
    size (codebook rows drawn from the matrix's column sub-vectors).  HIP-event
    times: the factor against the float64 peak (2N^3/3 flops), the float64 block
    updates against the float64 peak, the columns as distance pairs/s, and the
    number of decisions that took the exact float64 search; the oracle on one
    group of V rows at the full width."""
    import numpy as np
    import torch

    from hessian_weighted_vector_amd import synth, vq
    M, N, K = cfg.M, cfg.N, cfg.K1
    H = torch.from_numpy(synth.make_hessian(cfg.cid, cfg.N, cfg.T, cfg.n_ch, cfg.ch_gain)).cuda()
    W = torch.from_numpy(inp["W"]).cuda()
    g = np.random.default_rng([cfg.cid, 98])
    cols = inp["W"].T.reshape(-1, V)
    Cn = cols[np.sort(g.choice(cols.shape[0], K, replace=False))].copy()
    C = torch.from_numpy(Cn).cuda()
    ws_f = torch.empty(vq.load().vq_hessian_factor_workspace_bytes(N), dtype=torch.uint8, device="cuda")
    ws_v = torch.empty(vq.load().vq_vptq_workspace_bytes(M, N, V), dtype=torch.uint8, device="cuda")
    U = vq.hessian_factor(H, 0.01, ws=ws_f)
    vq.vptq(W, U, V, C, B, ws=ws_v)
    torch.cuda.synchronize()
    vq.timing_enable(True)
    t0 = time.perf_counter()
    U = vq.hessian_factor(H, 0.01, ws=ws_f)
    idx, What, _ = vq.vptq(W, U, V, C, B, ws=ws_v)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    rec = {(r[0], r[1]): r for r in vq.timing_records()}
    vq.timing_enable(False)
    t_f = rec[("hessian_factor", 0)][3]
    t_v = rec[("vptq", K)][3]
    gu = rec[("vptq_block_update", K)]
    gemm_flops = 0.0
    for s in range(0, N, B):
        s_end = min(s + B, N)
        gemm_flops += 2.0 * (N - s_end) * M * (s_end - s)
    f_flops = 2.0 * N ** 3 / 3.0
    pairs = float(N) * (M // V) * K
    res = {"V": V, "K": K, "B": B, "wall_ms": round(wall, 1),
           "hessian_factor": {"gpu_ms": round(t_f, 2), "flop": f_flops,
                              "TFLOPs": round(f_flops / (t_f * 1e-3) / 1e12, 2),
                              "frac_fp64": round(f_flops / (t_f * 1e-3) / 1e12 / PEAK_FP64_TFLOPS, 4)},
           "vptq_total_ms": round(t_v, 2),
           "block_update": {"gpu_ms": round(gu[3], 2), "launches": gu[2], "flop": gemm_flops,
                            "TFLOPs": round(gemm_flops / (gu[3] * 1e-3) / 1e12, 2),
                            "frac_fp64": round(gemm_flops / (gu[3] * 1e-3) / 1e12 / PEAK_FP64_TFLOPS, 4),
                            "note": "float64 vector units, each product rounded then added (the oracle's order)"},
           "exact_searches": rec[("vptq_exact_searches", K)][2] if ("vptq_exact_searches", K) in rec else None,
           "columns": {"gpu_ms": round(t_v - gu[3], 2),
                       "G_pairs_per_s": round(pairs / ((t_v - gu[3]) * 1e-3) / 1e9, 1),
                       "us_per_column": round((t_v - gu[3]) * 1e3 / N, 2)}}
    if run_oracle:
        import oracle
        Un = U.cpu().numpy()
        t0 = time.perf_counter()
        oracle.vptq(inp["W"][:V], Un, V, Cn, B)
        t_o = time.perf_counter() - t0
        res["oracle_ms_one_row_group"] = round(t_o * 1e3, 1)
        res["oracle_ms_full_extrapolated"] = round(t_o * 1e3 * (M // V), 0)
    return res


def grouped_bench(cfg, inp, W, h, plain_ms, run_oracle, d0=4, K0=4096, n_groups=1, outlier_frac=0.0, reps=2):
    """The grouped fit on the workload: the 1% of columns with the largest Hessian
    diagonal (rounded down to a multiple of 8) held apart with a v = 4, 4096-centroid
    codebook, the rest fitted as one group with the workload's codebooks.  The
    outlier columns take the place of the per-weight salient set here (fraction 0 by
    default), as in VPTQ's own configuration; with the workload's 1% salient weights
    most of those columns' weights would be masked.  Wall time
    per call beside the plain fit's step, the HIP-event time of the pieces the
    grouping adds (column order, gathers, scatters), and the assignment rate over all
    groups; the oracle's column order and one assignment pass over the outlier group,
    both at the full size."""
    import numpy as np
    import torch

    from hessian_weighted_vector_amd import vq
    M, N, d = cfg.M, cfg.N, cfg.d
    n_out = int(0.01 * N) // 8 * 8
    prm = vq.grouped_params(M, N, d, cfg.K1, cfg.T1, cfg.K2, cfg.T2, outlier_frac, cfg.binorm, True, n_out, d0,
                            K0, cfg.T1, n_groups)
    wsb, n_idx, n_cb, n_J, n_p1, n_p2 = vq.grouped_sizes(prm)
    ns0, ns1 = M * n_out // d0, M * (N - n_out) // d
    assert n_groups == 1 and n_p1 == ns0 + ns1 and n_p2 == (ns1 if cfg.K2 else 0)
    g = np.random.default_rng([cfg.cid, 99])
    p1 = np.concatenate([g.permutation(ns0), g.permutation(ns1)]).astype(np.int32)
    p2 = g.permutation(ns1).astype(np.int32) if cfg.K2 else None
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    vq.fit_grouped(W, h, prm, p1, p2, ws=ws)
    torch.cuda.synchronize()
    vq.timing_enable(True)
    t0 = time.perf_counter()
    for _ in range(reps):
        out = vq.fit_grouped(W, h, prm, p1, p2, ws=ws)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / reps
    recs = vq.timing_records()
    vq.timing_enable(False)
    added = sum(r[3] for r in recs if r[0] in ("column_order", "group_gather", "group_scatter")) / reps
    col = [r for r in recs if r[0] == "column_order"]
    iters = ns0 * cfg.T1 + ns1 * (cfg.T1 + cfg.T2)
    res = {"n_out": n_out, "d0": d0, "K0": K0, "n_groups": n_groups, "outlier_frac": outlier_frac,
           "ms": round(wall, 2),
           "plain_fit_ms": round(plain_ms, 2), "ms_added_by_grouping": round(added, 3),
           "column_order_ms": round(sum(r[3] for r in col) / reps, 4),
           "G_subvector_assignments_per_s": round(iters / (wall * 1e-3) / 1e9, 4),
           "bpw": round(out["bpw"], 4), "J_final_sum": float(out["J"][cfg.T1] + out["J"][-1])}
    if run_oracle:
        import oracle
        t0 = time.perf_counter()
        cols = oracle.column_order(inp["h"], n_out)
        res["oracle_column_order_ms"] = round((time.perf_counter() - t0) * 1e3, 1)
        Xo = np.ascontiguousarray(inp["W"][:, cols[:n_out]])
        C0 = Xo.reshape(-1, d0)[np.sort(g.choice(ns0, K0, replace=False))].copy()
        t0 = time.perf_counter()
        oracle.assign(Xo, inp["h"][cols[:n_out]], None, None, d0, C0)
        res["oracle_outlier_assign_pass_ms"] = round((time.perf_counter() - t0) * 1e3, 1)
    return res


def cold_warm_rows(cfg, out, W, h, nnz, ws, reps=10, scrub_mib=1024):
    """The HBM-bound rows timed cold and warm (HIP events on the library's stream).

    Cold: before every rep a resident scrub buffer of scrub_mib MiB (more than the
    256 MB Infinity Cache plus the L2s) is read once, so the call's inputs come
    from HBM and the caches hold only clean lines of another buffer.  Warm: the
    reps run back to back, as inside the Lloyd loop, where the 180 MB matrix of
    the 4096 x 11008 workload stays in the Infinity Cache.  Inputs are the fit's
    own state (matrix, weights, mask, indices, codebooks, CSR); the update
    restores its codebook before every rep."""
    import torch

    from hessian_weighted_vector_amd import vq
    M, N, d, n_sub = cfg.M, cfg.N, cfg.d, cfg.n_sub
    X = out["Wp"] if cfg.binorm else W
    hcol = out["hcol"] if cfg.binorm else h
    rho = out["rho"] if cfg.binorm else None
    mask = out["mask"]
    scrub = torch.ones(scrub_mib * (1 << 18), dtype=torch.float32, device="cuda")
    R = vq.residual(X, d, out["C1"], out["idx1"]) if cfg.K2 else None
    What = torch.empty((M, N), dtype=torch.float32, device="cuda")
    C1w = out["C1"].clone()
    C2w = out["C2"].clone() if cfg.K2 else None
    recon_args = (out["C2"], out["idx2"], out.get("rscale"), out.get("cscale"),
                  out["row_ptr"] if nnz else None, out["col"] if nnz else None, out["val"] if nnz else None)
    ops = [
        ("A1_select", ("select", 0), lambda: vq.sparse_select(W, h, d, nnz, ws), None,
         4 * M * N + 4 * N + 8 * nnz + 4 * (M + 1) + n_sub),
        ("A5_update_stage1", ("update", cfg.K1),
         lambda: vq.update(X, hcol, rho, mask, d, out["idx1"], C1w, ws, want_counts=False, want_J=False),
         lambda: C1w.copy_(out["C1"]), algorithmic_bytes_update(n_sub, M, N, d, cfg.K1)),
        ("A6_residual", ("residual", cfg.K1), lambda: vq.residual(X, d, out["C1"], out["idx1"]), None,
         n_sub * (8 * d + 2) + 4 * cfg.K1 * d),
        ("A7_reconstruct", ("reconstruct", cfg.K1),
         lambda: vq.reconstruct(M, N, d, out["C1"], out["idx1"], *recon_args, out=What), None,
         algorithmic_bytes_reconstruct(n_sub, M, N, d, cfg.K1, cfg.K2, nnz, cfg.binorm)),
    ]
    if cfg.K2:
        ops.insert(2, ("A5_update_stage2", ("update", cfg.K2),
                       lambda: vq.update(R, hcol, rho, mask, d, out["idx2"], C2w, ws, want_counts=False,
                                         want_J=False),
                       lambda: C2w.copy_(out["C2"]), algorithmic_bytes_update(n_sub, M, N, d, cfg.K2)))
    res = {}
    for name, key, fn, prep, nbytes in ops:
        e = {"algorithmic_MB": round(nbytes / 1e6, 1)}
        for mode in ("warm", "cold"):
            if prep:
                prep()
            fn()
            torch.cuda.synchronize()
            vq.timing_enable(True)
            for _ in range(reps):
                if prep:
                    prep()
                if mode == "cold":
                    scrub.sum()
                fn()
            torch.cuda.synchronize()
            r = {(x[0], x[1]): x for x in vq.timing_records()}[key]
            vq.timing_enable(False)
            t = r[3] / r[2]
            e[mode + "_ms"] = round(t, 4)
            e[mode + "_GBs"] = round(nbytes / (t * 1e-3) / 1e9, 1)
            e[mode + "_frac_hbm"] = round(nbytes / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        res[name] = e
    del scrub, R, What
    torch.cuda.empty_cache()
    return res


def config_rows(cfg_ids, steps_for, cpu_seconds):
    """One timed whole fit per workload (inputs resident in HBM, one untimed
    warm-up fit): step time, value, and the per-row times of the stage-1
    search, update and the reconstruction from HIP events inside the timed
    fits, each against its roofline; beside it the oracle's exhaustive
    assignment rate on a short seeded sample of the workload."""
    import numpy as np
    import torch

    import oracle
    from hessian_weighted_vector_amd import configs, synth, vq
    out_rows = {}
    for cid in cfg_ids:
        cfg = configs.get(cid)
        inp = synth.make_inputs(cfg)
        W = torch.from_numpy(inp["W"]).cuda()
        h = torch.from_numpy(inp["h"]).cuda()
        nnz = vq.nnz_of(cfg.M, cfg.N, cfg.p)
        ws = vq.workspace(cfg.M, cfg.N, cfg.d, cfg.K1, cfg.K2, nnz)
        fit = lambda: vq.fit(W, h, cfg.d, cfg.K1, cfg.T1, cfg.K2, cfg.T2, cfg.p, cfg.binorm, True,  # noqa: E731
                             inp["perm1"], inp["perm2"], ws=ws)
        fit()
        torch.cuda.synchronize()
        steps = steps_for(cfg)
        vq.timing_enable(True)
        t0 = time.perf_counter()
        for _ in range(steps):
            fit()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        rec = {(r[0], r[1]): r for r in vq.timing_records()}
        vq.timing_enable(False)
        n_sub = cfg.n_sub
        row = {"M": cfg.M, "N": cfg.N, "K1": cfg.K1, "K2": cfg.K2, "steps": steps, "step_ms": round(ms, 2),
               "value_G_subvector_assignments_per_s": round(n_sub * (cfg.T1 + cfg.T2) / (ms * 1e-3) / 1e9, 5)}

        def avg(key):
            r = rec.get(key)
            return r[3] / r[2] if r else None
        t = avg(("assign_search", cfg.K1))
        if t:
            fl = 32.0 * n_sub * cfg.K1
            row["A4_search_stage1_ms"] = round(t, 4)
            row["A4_frac_fp16_mfma"] = round(fl / (t * 1e-3) / 1e12 / PEAK_FP16_MFMA_TFLOPS, 4)
        t = avg(("update", cfg.K1))
        if t:
            row["A5_update_stage1_ms"] = round(t, 4)
            row["A5_frac_hbm_in_fit"] = round(algorithmic_bytes_update(n_sub, cfg.M, cfg.N, cfg.d, cfg.K1)
                                              / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        t = avg(("reconstruct", cfg.K1))
        if t:
            row["A7_reconstruct_ms"] = round(t, 4)
            row["A7_frac_hbm_in_fit"] = round(algorithmic_bytes_reconstruct(n_sub, cfg.M, cfg.N, cfg.d, cfg.K1,
                                                                            cfg.K2, nnz, cfg.binorm)
                                              / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        t = avg(("select", 0))
        if t:
            row["A1_select_ms"] = round(t, 4)
        del W, h, ws
        torch.cuda.empty_cache()
        if cpu_seconds > 0:
            c = cpu_baseline(cfg, inp, cpu_seconds)
            row["oracle_assign_G_per_s"] = c["value"]
            row["oracle_cores"] = c["cores"]
        out_rows[cfg.name] = row
        del inp
    return out_rows


def cpu_baseline(cfg, inp, seconds):
    """The oracle's assignment on a bounded sample (float64 exhaustive search)."""
    import numpy as np

    import oracle
    nthreads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    Wp, r, c, hcol, rho = oracle.binorm(inp["W"], inp["h"]) if cfg.binorm else (inp["W"], None, None, inp["h"], None)
    C, taken = oracle.init(Wp, cfg.d, inp["perm1"], cfg.K1)
    assert taken == cfg.K1
    chunk = 8192
    done, t_total, e0 = 0, 0.0, 0
    while t_total < seconds and e0 < cfg.n_sub:
        sub = np.sort(inp["perm1"][e0:e0 + chunk]).astype(np.int64)
        t0 = time.perf_counter()
        oracle.assign(Wp, hcol, rho, None, cfg.d, C, subset=sub, nthreads=nthreads)
        t_total += time.perf_counter() - t0
        done += sub.size
        e0 += chunk
    return {
        "value": done / t_total / 1e9,
        "unit": "G sub-vectors/s (one assignment pass, K=%d)" % cfg.K1,
        "cores": nthreads,
        "kind": "oracle",
        "sample": "%d seeded sub-vectors of the %dx%d%s matrix assigned against the %d-centroid seed "
                  "codebook (float64 direct form, exhaustive), %.1f s"
                  % (done, cfg.M, cfg.N, " bi-normalized" if cfg.binorm else "", cfg.K1, t_total),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", type=int, default=4, help="workload number 1..5 (default 4)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-qgemv", action="store_true", help="skip the fused dequantize-and-multiply rows")
    ap.add_argument("--no-correction", action="store_true", help="skip the unified sparse correction rows")
    ap.add_argument("--no-vptq", action="store_true", help="skip the VPTQ Algorithm 1 rows")
    ap.add_argument("--no-grouped", action="store_true", help="skip the grouped-fit row")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold/warm timing of the HBM rows")
    ap.add_argument("--no-configs", action="store_true", help="skip the one-fit rows of the other workloads")
    ap.add_argument("--breakdown", action="store_true", help="print per-step timings to stderr")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed steps, copy a buffer of this many MiB three times (a plain "
                         "copy of known size, to scale hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: each weight matrix is fitted on one device and there "
              "is no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from hessian_weighted_vector_amd import configs, synth, vq

    cfg = configs.get(args.config)
    inp = synth.make_inputs(cfg)
    torch.cuda.set_device(0)
    W = torch.from_numpy(inp["W"]).cuda()
    h = torch.from_numpy(inp["h"]).cuda()
    nnz = vq.nnz_of(cfg.M, cfg.N, cfg.p)
    ws = vq.workspace(cfg.M, cfg.N, cfg.d, cfg.K1, cfg.K2, nnz)

    def step():
        return vq.fit(W, h, cfg.d, cfg.K1, cfg.T1, cfg.K2, cfg.T2, cfg.p, cfg.binorm, True,
                      inp["perm1"], inp["perm2"], ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    vq.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        out = step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    recs = vq.timing_records()
    vq.timing_enable(False)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    n_sub = cfg.n_sub
    value = n_sub * (cfg.T1 + cfg.T2) / (ms_per_step * 1e-3) / 1e9

    rec = {(r[0], r[1]): r for r in recs}
    s1 = rec[("assign_search", cfg.K1)]
    avg_s1 = s1[3] / s1[2]
    flops = 32.0 * n_sub * cfg.K1
    achieved = flops / (avg_s1 * 1e-3) / 1e12
    src = os.path.join(ROOT, "hessian_weighted_vector_amd", "csrc", "vq_assign.hip")
    prof = search_profile(src) if cfg.cid == 4 else None
    roofline = {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_FP16_MFMA_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_MFMA_TFLOPS, 4),
                "traffic": prof.get("hbm_bytes_per_launch") if prof else None}

    extra = {"assign_stage1_ms": round(avg_s1, 3),
             "assign_stage1_Gsub_per_s": round(n_sub / (avg_s1 * 1e-3) / 1e9, 5),
             "assign_stage1_fp32_equivalent_vs_fp32_peak": round(achieved / PEAK_FP32_MFMA_TFLOPS, 4)}
    if prof:
        # executed matrix-core work from the counters (nominal = 32 flop per pair)
        ratio = prof["executed_mfma_flops_per_launch"] / prof["algorithmic_flops_per_launch"]
        extra["assign_stage1_executed_to_nominal_flops"] = round(ratio, 4)
        extra["assign_stage1_executed_frac_fp16_mfma"] = round(achieved * ratio / PEAK_FP16_MFMA_TFLOPS, 4)
    if ("assign", cfg.K1) in rec:
        a = rec[("assign", cfg.K1)]
        extra["assign_stage1_with_exact_ms"] = round(a[3] / a[2], 3)
    if cfg.K2 and ("assign_search", cfg.K2) in rec:
        a = rec[("assign_search", cfg.K2)]
        extra["assign_stage2_ms"] = round(a[3] / a[2], 4)
        extra["assign_stage2_Gsub_per_s"] = round(n_sub / (a[3] / a[2] * 1e-3) / 1e9, 4)
    if ("update", cfg.K1) in rec:
        u = rec[("update", cfg.K1)]
        ub = algorithmic_bytes_update(n_sub, cfg.M, cfg.N, cfg.d, cfg.K1)
        extra["update_stage1_us"] = round(u[3] / u[2] * 1e3, 2)
        extra["update_stage1_GBs"] = round(ub / (u[3] / u[2] * 1e-3) / 1e9, 1)
        extra["update_stage1_frac_hbm"] = round(extra["update_stage1_GBs"] / PEAK_HBM_GBS, 4)
    if ("reconstruct", cfg.K1) in rec:
        r_ = rec[("reconstruct", cfg.K1)]
        rb = algorithmic_bytes_reconstruct(n_sub, cfg.M, cfg.N, cfg.d, cfg.K1, cfg.K2, nnz, cfg.binorm)
        extra["reconstruct_us"] = round(r_[3] / r_[2] * 1e3, 2)
        extra["reconstruct_GBs"] = round(rb / (r_[3] / r_[2] * 1e-3) / 1e9, 1)
        extra["reconstruct_frac_hbm"] = round(extra["reconstruct_GBs"] / PEAK_HBM_GBS, 4)
    extra["J_final"] = float(out["J"][-1])
    extra["empty_centroids_per_update"] = [int(x) for x in out["empty"]]
    extra["bpw"] = out["bpw"]

    if args.breakdown:
        for r in sorted(recs, key=lambda r: -r[3]):
            print("%-14s K=%-6d launches=%-4d total=%9.3f ms avg=%9.4f ms min=%9.4f max=%9.4f"
                  % (r[0], r[1], r[2], r[3], r[3] / r[2], r[4], r[5]), file=sys.stderr)

    cpu = None
    oracle_ms = {}
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, inp, args.cpu_seconds)
        oracle_ms = cpu_rows(cfg, inp, nnz)
        oracle_ms["assign"] = n_sub / (cpu["value"] * 1e9) * 1e3   # full pass at the sampled rate
    extra["rows"] = row_table(cfg, recs, nnz, oracle_ms)
    if not args.no_qgemv:
        extra["rows"]["NEXT1_qgemv"] = qgemv_bench(cfg, inp, not args.no_cpu_baseline)
    if not args.no_vptq:
        extra["rows"]["NEXT2_vptq_algorithm1"] = vptq_bench(cfg, inp, not args.no_cpu_baseline)
    if not args.no_correction:
        extra["rows"]["NEXT3_unified_correction"] = correction_bench(cfg, inp, out, W, h, ws,
                                                                     not args.no_cpu_baseline)
    if not args.no_grouped:
        extra["rows"]["NEXT4_grouped_fit"] = grouped_bench(cfg, inp, W, h, ms_per_step, not args.no_cpu_baseline)
    if not args.no_cold:
        cw = cold_warm_rows(cfg, out, W, h, nnz, ws)
        for k, v in cw.items():
            extra["rows"].setdefault(k, {}).update({kk: vv for kk, vv in v.items() if kk != "algorithmic_MB"})
        for k in ("A5_update_stage1", "A5_update_stage2", "A7_reconstruct"):
            if k in cw:
                extra[k + "_frac_hbm_cold"] = cw[k]["cold_frac_hbm"]
                extra[k + "_frac_hbm_warm"] = cw[k]["warm_frac_hbm"]
    if not args.no_configs:
        del W, h, ws, out
        torch.cuda.empty_cache()
        others = [c for c in (1, 2, 3, 4, 5) if c != cfg.cid]
        rows = config_rows(others, lambda c: 1 if c.n_sub > 10_000_000 else (2 if c.n_sub > 1_000_000 else 5),
                           0.0 if args.no_cpu_baseline else 2.0)
        main_row = {"M": cfg.M, "N": cfg.N, "K1": cfg.K1, "K2": cfg.K2, "steps": args.steps,
                    "step_ms": round(ms_per_step, 2), "value_G_subvector_assignments_per_s": round(value, 5),
                    "A4_search_stage1_ms": round(avg_s1, 4), "A4_frac_fp16_mfma": roofline["frac"]}
        for k_src, k_dst in (("update_stage1_us", "A5_update_stage1_ms"), ("reconstruct_us", "A7_reconstruct_ms")):
            if k_src in extra:
                main_row[k_dst] = round(extra[k_src] / 1e3, 4)
        if "update_stage1_frac_hbm" in extra:
            main_row["A5_frac_hbm_in_fit"] = extra["update_stage1_frac_hbm"]
        if "reconstruct_frac_hbm" in extra:
            main_row["A7_frac_hbm_in_fit"] = extra["reconstruct_frac_hbm"]
        if cpu:
            main_row["oracle_assign_G_per_s"] = cpu["value"]
            main_row["oracle_cores"] = cpu["cores"]
        rows[cfg.name] = main_row
        extra["rows"]["configs"] = {configs.get(c).name: rows[configs.get(c).name] for c in (1, 2, 3, 4, 5)}

    line = {
        "metric": "sub-vectors assigned/s per Lloyd iter (G/s) + % FP32 peak; update/recon HBM GB/s",
        "value": round(value, 6),
        "unit": "G sub-vectors/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (search: fp16x2 split, f32 accumulate; f64 re-rank and sums)",
        "data": "synthetic (seeded StudentT weights, Gaussian activations with high-energy channels)",
        "config": {"workload": cfg.name, "M": cfg.M, "N": cfg.N, "d": cfg.d, "K1": cfg.K1, "T1": cfg.T1,
                   "K2": cfg.K2, "T2": cfg.T2, "outlier_frac": cfg.p, "nnz": nnz, "binorm": cfg.binorm,
                   "bf16_input": cfg.bf16, "n_sub": n_sub,
                   "value_def": "n_sub*(T1+T2)/step_time; step = full vq_fit incl. reconstruct"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
