#!/usr/bin/env python3
"""Benchmark of the TLR GEMM hot path on one MI355X.

Workload (default): TLR x TLR -> dense, fp64, N = 16384, b = 512 (32 x 32
tiles), op(A) = T, op(B) = N, alpha = 1, beta = 1, seeded synthetic ranks
min(64, max(4, round(64/(1+|i-j|)))) + U{0..4} and N(0,1)/sqrt(b) factors with
0.9^a column decay.  One step = one tlr_gemm_execute (all three stages of the
product) with every input already resident in HBM.  Plan analysis, descriptor
upload and input generation happen before the timed region.

Printed: one JSON line with the useful TFLOP/s (flops counted from rank
metadata for the chosen association order), the roofline of the dominant
kernel (the final-update launch, timed with HIP events on its own stream over
the timed steps), the whole-path roofline fraction, the same-chip dense
reference (the library's dense MFMA GEMM on the rebuilt N x N operands), and
the CPU oracle timed on a bounded sample of output tiles.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"f64": 78.6, "f32": 157.3, "f16": 2500.0, "bf16": 2500.0}   # MI355X dense MFMA TFLOP/s (datasheet)
# vector (non-matrix) ALU peaks: 256 CUs x 2.4 GHz x 128 fp64 / 256 fp32 flops per CU and clock
VECTOR_PEAK = {"f64": 78.6, "f32": 157.3}
ES = {"f64": 8, "f32": 4, "f16": 2, "bf16": 2}
HBM_PEAK_GBS = 8000.0
METRIC = "TLR GEMM useful TFLOP/s + % of roofline, fp64 TLRxTLR->dense N=16384"
DEFAULT_WORKLOAD = "3"

# Launch configuration the benchmark times for each workload unless --streams
# or --pipeline say otherwise: streams given to execute, and whether the
# rectangles alternate between two arenas on two streams.  The full-size GPU
# parity tests run exactly these configurations.
LAUNCH = {"1": {"streams": 1, "pipeline": False}, "2": {"streams": 1, "pipeline": False},
          "3": {"streams": 1, "pipeline": False}, "4": {"streams": 1, "pipeline": False},
          "5": {"streams": 1, "pipeline": False}, "dense_tlr": {"streams": 1, "pipeline": False}}


def launch_config(workload: str, streams=None, pipeline=None):
    """(n_streams, pipelined) for a workload: the LAUNCH entry, overridden by
    explicit values.  Pipelining needs two streams."""
    d = LAUNCH.get(workload, {"streams": 1, "pipeline": False})
    pipe = d["pipeline"] if pipeline is None else bool(pipeline)
    ns = d["streams"] if streams is None else int(streams)
    return max(ns, 2 if pipe else 1), pipe


def workload(name: str, dtype=None):
    """Inputs of a bench workload: "1".."5" are the seeded workloads of
    tlr_inputs.CONFIGS; "dense_tlr" is workload 2 with its operands swapped
    (a dense 4096 x 4096 A times the TLR operand), the dense x TLR product.
    ``dtype`` replaces the element type (the same draws, rounded to it)."""
    from tlr_inputs import CONFIGS, config_inputs
    if name == "dense_tlr":
        cfg = dict(CONFIGS[2])
        T_op, Bd, C = config_inputs(2, dtype=dtype)
        cfg["name"] = "dense_tlr_f64_n4096_b256_NN"
        A, B = Bd, T_op
    else:
        cfg = dict(CONFIGS[int(name)])
        A, B, C = config_inputs(int(name), dtype=dtype)
    if dtype and dtype != cfg["dtype"]:
        cfg["name"] = cfg["name"].replace("_" + cfg["dtype"] + "_", "_" + dtype + "_")
        cfg["dtype"] = dtype
    return cfg, A, B, C


def final_update_bytes(F3: float, N: int, b: int, es: int, beta: float) -> float:
    """Algorithmic HBM bytes of a final-update launch over the whole N x N C
    (square b x b tiles): C written once and read once when beta != 0, and the
    two operand panels read once.  The launch's flops are F3 = 2 N b sum(rank
    sums) in either association order, so the panels hold F3/(2b) (the N-long
    side: the right products T or the left products Y) plus F3/(2N) (the
    b-long side: U or Z) elements."""
    return es * (N * N * (2.0 if beta != 0 else 1.0) + F3 / (2.0 * b) + F3 / (2.0 * N))


def logical_flops(cfg, A, B, order: str) -> float:
    """Useful flops of the product in the given order counted with the logical
    ranks (16-bit operands store ranks rounded up to a multiple of 8; the
    zero columns are storage, not work): the same analysis on a 32-bit plan of
    the unrounded operands."""
    import numpy as np
    from hpc_linear_algebra_amd import tlrgemm as T
    from tlr_inputs import TLRTiles
    shp = lambda t: None if not isinstance(t, TLRTiles) else T.Shape(t.rows, t.cols, t.b,
                                                                      np.asarray(t.ranks, np.int32), t.has_diag)
    dense = A if not isinstance(A, TLRTiles) else (B if not isinstance(B, TLRTiles) else None)
    dr, dc = dense.shape if dense is not None else (0, 0)
    flag = T.TLR_PLAN_FORCE_LEFT if order == "left" else T.TLR_PLAN_FORCE_RIGHT
    p = T.tlr_gemm_analyze("f32", cfg["opA"], shp(A), cfg["opB"], shp(B), dr, dc, dr if dense is not None else 0,
                           cfg["N"], flags=flag)
    return T.tlr_plan_info(p)["useful_flops"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash(sixteen_bit: bool = False) -> str:
    from hpc_linear_algebra_amd.profiling import kernel_source_hash
    return kernel_source_hash(sixteen_bit)


def traffic_from_profiles(stage: int, workload_name: str, sixteen_bit: bool = False):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3
    counter runs of this workload, if they were taken on the current kernel
    source."""
    path = os.path.join(ROOT, "profiles", f"stage{stage}_traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    if d.get("kernel_hash") != kernel_hash(sixteen_bit):
        return None
    return d.get("bytes_per_launch")


def mfma_busy_from_profiles(stage: int, workload_name: str, sixteen_bit: bool = False):
    """MFMA busy fraction of the dominant kernel from a committed rocprofv3
    counter run of this workload, if it was taken on the current kernel
    source."""
    path = os.path.join(ROOT, "profiles", f"stage{stage}_mfma_{workload_name}.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    if d.get("kernel_hash") != kernel_hash(sixteen_bit):
        return None
    return d.get("mfma_busy")


def rebuild_dense_on_gpu(dev, t, dtype):
    """Dense N x N copy of a stored TLR operand, built with the library's own
    dense GEMM (U_ij V_ij^T per tile) and copies of the diagonal tiles."""
    import numpy as np
    import torch
    from hpc_linear_algebra_amd import tlrgemm as T
    N, b = t.rows, t.b
    tdt = torch.float64 if dtype == "f64" else torch.float32
    out = torch.zeros((N, N), dtype=tdt, device="cuda")       # column-major: out[col, row]
    sizes = t.row_sizes
    offs = np.concatenate([[0], np.cumsum(sizes)])[:-1]
    q = len(sizes)
    R = t.ranks
    es = 8 if dtype == "f64" else 4
    stream = torch.cuda.current_stream().cuda_stream
    oc = 0
    ocol = {}
    for i in range(q):
        for j in range(q):
            ocol[(i, j)] = oc
            oc += int(R[i, j])
    ic = 0
    icol = {}
    for j in range(q):
        for i in range(q):
            icol[(i, j)] = ic
            ic += int(R[i, j])
    base = out.data_ptr()
    for i in range(q):
        for j in range(q):
            r0, c0 = int(offs[i]), int(offs[j])
            cptr = base + (r0 + c0 * N) * es
            if t.has_diag and i == j:
                d = dev.diag[i * b * b:(i + 1) * b * b].view(b, b)[: sizes[i], : sizes[i]]
                out[c0:c0 + sizes[j], r0:r0 + sizes[i]] = d
                continue
            r = int(R[i, j])
            if r == 0:
                continue
            T.tlr_dense_gemm(dtype, "N", "T", sizes[i], sizes[j], r, 1.0,
                             dev.outer.data_ptr() + ocol[(i, j)] * b * es, b,
                             dev.inner.data_ptr() + icol[(i, j)] * b * es, b, 0.0, cptr, N, stream)
    torch.cuda.synchronize()
    return out


def padded_copy(t, rmax: int):
    """The TLR operand with every off-diagonal tile's factors padded with zero
    columns to rank min(rmax, tile sizes): the one-rank storage of the
    batched per-k comparator."""
    import copy
    import numpy as np
    p = copy.copy(t)
    p.U, p.V = dict(t.U), dict(t.V)
    p.ranks = np.array(t.ranks, copy=True)
    for key in list(p.U):
        u, v = p.U[key], p.V[key]
        want = min(rmax, u.shape[0], v.shape[0])
        if want > u.shape[1]:
            p.U[key] = np.concatenate([u, np.zeros((u.shape[0], want - u.shape[1]), u.dtype)], axis=1)
            p.V[key] = np.concatenate([v, np.zeros((v.shape[0], want - v.shape[1]), v.dtype)], axis=1)
            p.ranks[key] = want
    return p


def dense_reference_16(cfg, A, B, dtype, value, stream):
    """Same-chip dense reference of a 16-bit product: the N x N operands
    rebuilt in float32 by the library's dense GEMM, rounded to the 16-bit
    type, and multiplied by torch.matmul (hipBLASLt, 16-bit inputs, float
    accumulation), which is the vendor's tuned 16-bit GEMM."""
    import copy
    import torch
    from hpc_linear_algebra_amd.device import _TORCH, DeviceTLR, dense_to_device
    from tlr_inputs import TLRTiles
    N = cfg["N"]

    def rebuilt(t):
        if not isinstance(t, TLRTiles):
            return dense_to_device(t, dtype=dtype)
        t32 = copy.copy(t)
        t32.dtype = "f32"
        d = DeviceTLR(t32)
        out = rebuild_dense_on_gpu(d, t32, "f32").to(_TORCH[dtype])
        del d
        return out
    Ad, Bd = rebuilt(A), rebuilt(B)
    torch.matmul(Ad, Bd)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record(stream)
    for _ in range(reps):
        Cw = torch.matmul(Ad, Bd)
    e1.record(stream)
    torch.cuda.synchronize()
    dms = e0.elapsed_time(e1) / reps
    dense_tf = 2.0 * N ** 3 / (dms * 1e-3) / 1e12
    del Ad, Bd, Cw
    torch.cuda.empty_cache()
    return {"tflops": round(dense_tf, 3), "ms": round(dms, 3), "parity": round(value / dense_tf, 4),
            "note": "useful TFLOP/s of the TLR product / TFLOP/s of torch.matmul (hipBLASLt) on the rebuilt "
                    "N x N operands in the same 16-bit type"}


def cpu_baseline(cfg, A, B, C_in, useful_flops, budget_s=15.0):
    """The CPU oracle, timed on a bounded sample of output tiles."""
    import numpy as np
    from oracle import reference
    from tlr_inputs import tile_sizes
    try:
        from threadpoolctl import threadpool_info
        threads = max([x.get("num_threads", 1) for x in threadpool_info() if x.get("user_api") == "blas"] or [1])
    except Exception:
        threads = 1
    N, b = cfg["N"], cfg["b"]
    sz = tile_sizes(N, b)
    off = reference.offsets(sz)
    q = len(sz)
    rng = np.random.default_rng(7)
    order = [(int(x) // q, int(x) % q) for x in rng.permutation(q * q)]
    t0 = time.perf_counter()
    done = 0
    tm = {}
    for (i, j) in order:
        r0, r1, c0, c1 = off[i], off[i] + sz[i], off[j], off[j] + sz[j]
        cin = None if C_in is None else C_in[r0:r1, c0:c1]
        reference.gemm_reference_block(cfg["alpha"], cfg["opA"], A, cfg["opB"], B, cfg["beta"], cin,
                                       (r0, r1), (c0, c1), timings=tm)
        done += 1
        if time.perf_counter() - t0 > budget_s and done >= 2:
            break
    dt = time.perf_counter() - t0
    full_s = dt * (q * q) / done
    try:
        aff = len(os.sched_getaffinity(0))
    except Exception:
        aff = None
    return {"value": useful_flops / full_s / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "reconstruct_s": round(tm.get("reconstruct_s", 0.0), 3), "matmul_s": round(tm.get("matmul_s", 0.0), 3),
            "measured_s": round(dt, 3), "tiles": done, "tiles_total": q * q,
            "host_cpu_count": os.cpu_count(), "host_affinity": aff, "blas_threads": int(threads),
            "sample": f"{done} of {q*q} output tiles ({sz[0]}x{sz[0]}) rebuilt densely in fp64 from the row "
                      f"panel of op(A) and column panel of op(B) and multiplied with numpy BLAS; "
                      f"{dt:.2f} s measured ({tm.get('reconstruct_s', 0.0):.2f} s rebuilding panels, "
                      f"{tm.get('matmul_s', 0.0):.2f} s in the matmul), scaled by {q*q}/{done} to the whole "
                      f"product (host cpu_count={os.cpu_count()})"}


def bench_tlr_out(args):
    """The TLR-output product (C <- alpha A B + beta C, C in TLR format, every
    off-diagonal result tile truncated to a relative tolerance): expand C into
    a dense scratch, the dense-output product into it, compress it.  One step
    is all three; each is timed with its own event pair."""
    import numpy as np
    import torch
    from hpc_linear_algebra_amd.device import DeviceTLR, TLROutputGemm
    from tlr_inputs import TLR_OUT, tlr_out_inputs
    cfg = TLR_OUT
    N, b, dtype = cfg["N"], cfg["b"], cfg["dtype"]
    torch.cuda.set_device(0)
    log("bench: generating the TLR-output workload")
    A, B, C, omega = tlr_out_inputs()
    dA, dB, dC = DeviceTLR(A), DeviceTLR(B), DeviceTLR(C)
    g = TLROutputGemm(dtype, cfg["opA"], dA, cfg["opB"], dB, b, True, cfg["max_rank"])
    om = torch.from_numpy(np.ascontiguousarray(omega.T)).cuda()
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    from hpc_linear_algebra_amd import tlrgemm as T

    def step():
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record(stream)
        T.tlr_expand(dtype, N, N, b, True, dC.ranks_device().data_ptr(), dC.buffers(), 1.0, 0.0,
                     g.scratch.data_ptr(), N, g.ews.data_ptr(), g.ews.numel(), s)
        ev[1].record(stream)
        g.gemm(cfg["alpha"], dA, dB, cfg["beta"], g.scratch, [s])
        ev[2].record(stream)
        T.tlr_compress(dtype, N, N, b, True, g.scratch.data_ptr(), N, cfg["tol"], cfg["max_rank"], om.data_ptr(),
                       g.ranks.data_ptr(), g.diag.data_ptr(), g.outer.data_ptr(), g.inner.data_ptr(), g.capacity,
                       g.info.data_ptr(), g.cws.data_ptr(), g.cws.numel(), s)
        ev[3].record(stream)
        return ev
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # HIP events around every compression kernel group and every launch of
    # the product, on their streams
    T.tlr_compress_profile(args.steps)
    T.tlr_plan_profile(g.gemm.plan, args.steps)
    w0 = time.perf_counter()
    evs = [step() for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    group_ms, calls = T.tlr_compress_profile_read()
    _, prod_launch_ms, nexec = T.tlr_plan_profile_read(g.gemm.plan, g.gemm.info["launches"])
    T.tlr_plan_profile(g.gemm.plan, 0)
    assert nexec == args.steps
    phases = np.array([[e[k].elapsed_time(e[k + 1]) for k in range(3)] for e in evs])
    total = phases.sum(axis=1)
    ms = float(total.mean())
    R, _, _, _, info = g.host_result()
    F = g.gemm.info["useful_flops"]
    value = F / (ms * 1e-3) / 1e12
    es = ES[dtype]
    q = R.shape[0]
    out_elems = sum(int(R[i, j]) * (2 * b) for i in range(q) for j in range(q) if i != j) + q * b * b
    names = ["expand", "product", "compress"]
    dom = int(np.argmax(phases.mean(axis=0)))
    # the dominant kernel: the one-sided Jacobi SVD of the s x s cores (one
    # launch per step), bound by its own arithmetic; its work from the pair
    # visits and rotations it reports (info[3], info[4]): per visit a 2 x 2
    # Gram block (3 dot products over the k rows a core has, 6 k flops), per
    # rotation 2 columns of M and 2 of J (12 k flops), where k is the tile's
    # count of sketch basis columns (info[5] sums them; the mean stands in for
    # each tile's own)
    n_s = cfg["max_rank"] + 8           # sketch width
    sizes = [min(b, N - i * b) for i in range(q)]
    tiles = q * (q - 1)
    kbar = int(info[5]) / tiles

    def qr_flops(m, n, k):
        # per reflector j < k: w = A^T v and the rank-1 update on the
        # (m-j) x (n-j-1) block (4 flops an element), then the forming of the
        # k columns of Q the same way on (m-j) x (k-j-1)
        return sum(4.0 * (m - j) * ((n - j - 1) + (k - j - 1)) for j in range(min(m, k)))
    kr = int(round(kbar))
    qr_work = 0.5 * sum(qr_flops(sizes[i], n_s, kr) + qr_flops(sizes[j], kr, kr)
                        for i in range(q) for j in range(q) if i != j)   # one launch, the mean of the two
    qr_ms = (group_ms[2] + group_ms[4]) / (2 * calls)
    qr_tf = qr_work / (qr_ms * 1e-3) / 1e12
    visits, rotations = int(info[3]), int(info[4])
    jac_work = visits * 6.0 * kbar + rotations * 12.0 * kbar
    jac_ms = group_ms[5] / calls
    jac_tf = jac_work / (jac_ms * 1e-3) / 1e12
    vec_peak = VECTOR_PEAK[dtype]
    jacobi = {"bound": "alu", "achieved": round(jac_tf, 3), "peak": vec_peak, "unit": "TFLOP/s",
              "frac": round(jac_tf / vec_peak, 4), "traffic": None,
              "kernel": "one-sided Jacobi SVD of the s x s cores and the ranks (one launch per step)",
              "launch_ms": round(jac_ms, 4), "algorithmic_flops": jac_work,
              "work": {"pair_visits": visits, "rotations": rotations, "sketch_width": n_s,
                       "basis_columns_mean": round(kbar, 2)}}
    # the dominant kernel: the longest single launch of the step, the
    # product's or the compression's (each compression group but the tile
    # GEMMs is one launch)
    prod = [x / args.steps for x in prod_launch_ms]
    pl = int(np.argmax(prod))
    if prod[pl] > jac_ms:
        Lp = g.gemm.launches()[pl]
        ach = Lp["useful_flops"] / (prod[pl] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(ach, 3), "peak": PEAK[dtype], "unit": "TFLOP/s",
                    "frac": round(ach / PEAK[dtype], 4),
                    "traffic": traffic_from_profiles(Lp["stage"], cfg["name"]),
                    "kernel": f"the product's stage {Lp['stage']} launch" +
                              (" (final update, segmented-K)" if Lp["stage"] == 3 else ""),
                    "launch_ms": round(prod[pl], 4), "algorithmic_flops": Lp["useful_flops"]}
    else:
        roofline = jacobi
    cpu = None
    if not args.no_cpu:
        from oracle import recompress as rc
        from oracle import reference
        rng = np.random.default_rng(7)
        Cd = reference.reconstruct(C)
        t0 = time.perf_counter()
        done = 0
        off = reference.offsets([b] * q)
        for x in rng.permutation(q * q):
            i, j = int(x) // q, int(x) % q
            blk = reference.gemm_reference_block(cfg["alpha"], cfg["opA"], A, cfg["opB"], B, cfg["beta"],
                                                 Cd[off[i]:off[i] + b, off[j]:off[j] + b],
                                                 (off[i], off[i] + b), (off[j], off[j] + b))
            if i != j:
                rc.truncate_tile(blk, cfg["tol"])
            done += 1
            if time.perf_counter() - t0 > args.cpu_seconds and done >= 2:
                break
        dt = time.perf_counter() - t0
        cpu = {"value": F / (dt * q * q / done) / 1e12, "unit": "TFLOP/s", "kind": "oracle",
               "cores": os.cpu_count(),
               "sample": f"{done} of {q*q} output tiles: the exact tile (rebuilt panels, numpy BLAS) and its SVD "
                         f"truncation, {dt:.2f} s, scaled by {q*q}/{done}; the dense expansion of C is outside "
                         f"the timed loop"}
    out = {
        "metric": "TLR-output product useful TFLOP/s (expand C, dense-output product, compress), fp64 N=8192",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype, "data": "synthetic",
        "config": {"workload": cfg["name"], "N": N, "b": b, "opA": cfg["opA"], "opB": cfg["opB"],
                   "alpha": cfg["alpha"], "beta": cfg["beta"], "tol": cfg["tol"], "max_rank": cfg["max_rank"],
                   "useful_flops": F, "useful_flops_basis": "the product's useful flops from its ranks"},
        "phases_ms": {n: round(float(phases[:, k].mean()), 4) for k, n in enumerate(names)},
        "step_ms": {"mean": round(ms, 4), "median": round(float(np.median(total)), 4),
                    "min": round(float(total.min()), 4), "max": round(float(total.max()), 4)},
        "result": {"rank_sum": int(info[0]), "tiles_flagged": int(info[1]), "capacity_exceeded": int(info[2]),
                   "rank_min": int(min(R[i, j] for i in range(q) for j in range(q) if i != j)),
                   "rank_max": int(R.max()),
                   "memory_vs_dense": round(out_elems / float(N * N), 4)},
        "dominant_phase": names[dom],
        "compress_groups_ms": {g: round(x / calls, 4) for g, x in zip(T.COMPRESS_PROFILE_GROUPS, group_ms)},
        "roofline": roofline,
        "jacobi": jacobi,
        "panel_qr": {"bound": "alu", "achieved": round(qr_tf, 3), "peak": vec_peak, "unit": "TFLOP/s",
                     "frac": round(qr_tf / vec_peak, 4), "launch_ms": round(qr_ms, 4),
                     "algorithmic_flops": qr_work, "note": "two launches per step (the sketches, the projections); "
                     "each tile's basis columns replaced by their mean"},
        "cpu_baseline": cpu,
    }
    log(f"bench: {ms:.3f} ms/step ({', '.join(f'{n} {phases[:, k].mean():.3f}' for k, n in enumerate(names))}), "
        f"wall {wall * 1e3 / args.steps:.3f} ms/step")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="1..5: the seeded workloads (3, the N=16384 TLR x TLR product, is the metric's); "
                         "dense_tlr: workload 2 with the operands swapped; tlr_out: the TLR-output product "
                         "(N=8192, b=256, C in TLR format, compressed to a tolerance)")
    ap.add_argument("--dtype", default=None, choices=["f64", "f32", "f16", "bf16"],
                    help="element type in place of the workload's own (same draws, rounded to it)")
    ap.add_argument("--order", default="auto", choices=["auto", "left", "right"],
                    help="association order of every rectangle (auto: the planner's choice, fewer useful flops)")
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-GEMM reference")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--pipeline", type=int, default=None,
                    help="1: rectangles alternate between two workspace arenas on two streams "
                         "(default: the workload's LAUNCH entry)")
    ap.add_argument("--streams", type=int, default=None,
                    help="streams given to execute; with two or more the boundary regions of C run on their "
                         "own streams (default: the workload's LAUNCH entry)")
    ap.add_argument("--comparator", action="store_true",
                    help="also time the per-contraction-tile loop (one pass over C per k) on operands padded to "
                         "one rank: the batched-GEMM comparator the three-stage product is set against")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = (1 << 30) // 8
        src = torch.ones(n, dtype=torch.float64, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 8, "copy_bytes_written": n * 8, "dispatches": 3}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the TLR GEMM here runs on a single MI355X "
              "(multi-GPU sharding is a design note, not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.workload == "tlr_out":
        print(json.dumps(bench_tlr_out(args)), flush=True)
        return

    import numpy as np
    import torch
    from hpc_linear_algebra_amd import tlrgemm as T
    from hpc_linear_algebra_amd.device import _TORCH, DeviceTLR, TLRGemm, dense_to_device
    from tlr_inputs import TLRTiles

    torch.cuda.set_device(0)
    log(f"bench: generating workload {args.workload}")
    cfg, A, B, C_in = workload(args.workload, args.dtype)
    dtype, N = cfg["dtype"], cfg["N"]
    sixteen = dtype in ("f16", "bf16")
    dense_a, dense_b = not isinstance(A, TLRTiles), not isinstance(B, TLRTiles)
    dA = dense_to_device(A, dtype=dtype) if dense_a else DeviceTLR(A)
    dB = dense_to_device(B, dtype=dtype) if dense_b else DeviceTLR(B)
    dense_shape = A.shape if dense_a else (B.shape if dense_b else None)
    tdt = _TORCH[dtype]
    Cd = dense_to_device(C_in, dtype=dtype) if C_in is not None else torch.zeros((N, N), dtype=tdt, device="cuda")
    n_streams, pipelined = launch_config(args.workload, args.streams, args.pipeline)
    flags = (T.TLR_PLAN_PIPELINE if pipelined else 0) | \
        {"auto": 0, "left": T.TLR_PLAN_FORCE_LEFT, "right": T.TLR_PLAN_FORCE_RIGHT}[args.order]
    g = TLRGemm(dtype, cfg["opA"], None if dense_a else dA, cfg["opB"], None if dense_b else dB, ldc=N,
                dense_shape=dense_shape, ldb=N if (dense_a or dense_b) else 0, budget=cfg["budget"] or 0,
                n_streams=n_streams, flags=flags)
    info = g.info
    launches = g.launches()
    stream = torch.cuda.current_stream()
    side = [torch.cuda.Stream() for _ in range(n_streams - 1)]
    streams = [stream.cuda_stream] + [x.cuda_stream for x in side]
    log(f"bench: plan runs={info['runs']} launches={info['launches']} ws={info['workspace_bytes']/2**30:.2f} GiB "
        f"useful={info['useful_flops']:.4e}")
    # with beta != 0 every step starts from the same C: a pristine device copy
    # is restored before each step, outside the step's events
    C0 = Cd.clone() if cfg["beta"] != 0 else None

    def step():
        if C0 is not None:
            Cd.copy_(C0)
        e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        e[0].record(stream)
        g(cfg["alpha"], dA, dB, cfg["beta"], Cd, streams)
        e[1].record(stream)
        return e
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: K steps, one HIP event pair per step on streams[0] (the
    # execute joins its other streams back into it) and one around every
    # launch on the launch's own stream
    T.tlr_plan_profile(g.plan, args.steps)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    evs = [step() for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    step_ms = [a.elapsed_time(b) for (a, b) in evs]
    ms = sum(step_ms) / args.steps
    srt = sorted(step_ms)
    step_stats = {"mean": round(ms, 4), "median": round(srt[len(srt) // 2] if len(srt) % 2 else
                                                        0.5 * (srt[len(srt) // 2 - 1] + srt[len(srt) // 2]), 4),
                  "min": round(srt[0], 4), "max": round(srt[-1], 4)}
    stage_ms, launch_ms, nexec = T.tlr_plan_profile_read(g.plan, info["launches"])
    T.tlr_plan_profile(g.plan, 0)
    assert nexec == args.steps
    order = ",".join("left" if T.tlr_plan_rect(g.plan, r)["order"] == T.TLR_ORDER_LEFT else "right"
                     for r in range(info["runs"]))
    F = info["useful_flops"]
    F_stored = F
    basis = "ranks"
    if sixteen:
        # with one order for every rectangle the logical-rank count is exact; with
        # mixed orders the count stays on the stored (rounded-up) ranks
        if len(set(order.split(","))) == 1:
            F = logical_flops(cfg, A, B, order.split(",")[0])
            basis = "logical ranks"
        else:
            basis = "stored ranks (rounded up to multiples of 8; the rectangles use different orders)"
    value = F / (ms * 1e-3) / 1e12
    log(f"bench: {ms:.3f} ms/step (median {step_stats['median']:.3f}, min {step_stats['min']:.3f}, max "
        f"{step_stats['max']:.3f}), {value:.2f} useful TFLOP/s (wall {wall*1e3/args.steps:.3f} ms/step with the "
        f"restores of C)")

    # dominant kernel: the launch with the largest measured time
    per_launch = [x / args.steps for x in launch_ms]
    dom = int(np.argmax(per_launch))
    L = launches[dom]
    achieved = L["useful_flops"] / (per_launch[dom] * 1e-3) / 1e12
    peak = PEAK[dtype]
    es = ES[dtype]
    alg_bytes = info["algorithmic_bytes"] + (N * N * es if cfg["beta"] != 0 else 0)
    ai = F / alg_bytes
    roof = min(peak, HBM_PEAK_GBS * 1e9 * ai / 1e12)
    kname = (f"stage {L['stage']} launch (final update, segmented-K)" if L["stage"] == 3
             else f"stage {L['stage']} launch")
    lbytes = final_update_bytes(L["useful_flops"], N, cfg["b"], es, cfg["beta"]) if L["stage"] == 3 else None
    if lbytes is not None and lbytes / (HBM_PEAK_GBS * 1e9) > L["useful_flops"] / (peak * 1e12):
        # the launch's bytes take longer at 8 TB/s than its flops at the MFMA peak
        gbs = lbytes / (per_launch[dom] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic_from_profiles(L["stage"], cfg["name"], sixteen),
                    "kernel": kname, "launch_ms": round(per_launch[dom], 4), "algorithmic_bytes": lbytes,
                    "mfma_tflops": round(achieved, 3),
                    "mfma_busy": mfma_busy_from_profiles(L["stage"], cfg["name"], sixteen)}
    else:
        roofline = {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4), "traffic": traffic_from_profiles(L["stage"], cfg["name"], sixteen),
                    "kernel": kname, "launch_ms": round(per_launch[dom], 4),
                    "mfma_busy": mfma_busy_from_profiles(L["stage"], cfg["name"], sixteen)}

    dense = None
    if not args.no_dense and sixteen:
        log("bench: dense reference (rebuilt operands, torch.matmul = hipBLASLt 16-bit GEMM)")
        dense = dense_reference_16(cfg, A, B, dtype, value, stream)
    elif not args.no_dense:
        log("bench: dense reference (rebuilt operands, same MFMA kernel)")
        Ad = dA if dense_a else rebuild_dense_on_gpu(dA, A, dtype)
        Bd = dB if dense_b else rebuild_dense_on_gpu(dB, B, dtype)
        Cw = torch.zeros((N, N), dtype=Ad.dtype, device="cuda")
        s = stream.cuda_stream

        def dense_call():
            T.tlr_dense_gemm(dtype, cfg["opA"], cfg["opB"], N, N, N, cfg["alpha"], Ad.data_ptr(), N,
                             Bd.data_ptr(), N, cfg["beta"], Cw.data_ptr(), N, s)
        for _ in range(2):
            dense_call()
        torch.cuda.synchronize()
        reps = 10
        devs = []
        for _ in range(reps):
            e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            e[0].record(stream)
            dense_call()
            e[1].record(stream)
            devs.append(e)
        torch.cuda.synchronize()
        d_ms = sorted(a.elapsed_time(b) for (a, b) in devs)
        dms = sum(d_ms) / reps
        dense_tf = 2.0 * N ** 3 / (dms * 1e-3) / 1e12
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps_v = 3
        # context only: the vendor's GEMM (torch.matmul, rocBLAS / hipBLASLt) on the same operands
        torch.matmul(Ad, Bd)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps_v):
            Vw = torch.matmul(Ad, Bd)
        e1.record(stream)
        torch.cuda.synchronize()
        vms = e0.elapsed_time(e1) / reps_v
        del Vw
        dense = {"tflops": round(dense_tf, 3), "ms": round(dms, 3), "ms_min": round(d_ms[0], 3),
                 "ms_max": round(d_ms[-1], 3), "reps": reps,
                 "parity": round(value / dense_tf, 4),
                 "vendor_tflops": round(2.0 * N ** 3 / (vms * 1e-3) / 1e12, 3),
                 "note": "parity = useful TFLOP/s of the TLR product / TFLOP/s (2 N^3 per call) of the library's "
                         "dense MFMA GEMM on the rebuilt N x N operands, which equals the dense time multiplied by "
                         "useful flops / 2 N^3, divided by the TLR time; vendor_tflops: torch.matmul on the same "
                         "operands, for context"}
        if dense_a:
            Ad = None
        if dense_b:
            Bd = None
        del Ad, Bd, Cw
        torch.cuda.empty_cache()

    comparator = None
    if args.comparator and not (dense_a or dense_b):
        rmax = int(max(np.max(A.ranks), np.max(B.ranks)))
        log(f"bench: per-k comparator, ranks padded to {rmax}")
        Ap, Bp = padded_copy(A, rmax), padded_copy(B, rmax)
        dAp, dBp = DeviceTLR(Ap), DeviceTLR(Bp)
        gk = TLRGemm(dtype, cfg["opA"], dAp, cfg["opB"], dBp, ldc=N, flags=T.TLR_PLAN_PER_K)
        for _ in range(2):
            gk(cfg["alpha"], dAp, dBp, cfg["beta"], Cd, [stream.cuda_stream])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record(stream)
        for _ in range(reps):
            gk(cfg["alpha"], dAp, dBp, cfg["beta"], Cd, [stream.cuda_stream])
        e1.record(stream)
        torch.cuda.synchronize()
        kms = e0.elapsed_time(e1) / reps
        comparator = {"ms": round(kms, 3), "speedup": round(kms / ms, 3), "padded_rank": rmax,
                      "passes_over_C": gk.info["runs"], "executed_flops": gk.info["useful_flops"],
                      "note": "per contraction tile k: batched couplings, right products and updates of every "
                              "output tile at one common rank, C read and written once per k; speedup = its "
                              "time / the three-stage product's"}
        del gk, dAp, dBp, Ap, Bp
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        log("bench: CPU oracle baseline on a bounded sample")
        cpu = cpu_baseline(cfg, A, B, C_in, F, args.cpu_seconds)

    out = {
        "metric": METRIC if args.workload == DEFAULT_WORKLOAD and dtype == "f64" else
        f"TLR GEMM useful TFLOP/s + % of roofline, {cfg['name']}", "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": cfg["name"], "N": N, "b": cfg["b"], "opA": cfg["opA"], "opB": cfg["opB"],
                   "alpha": cfg["alpha"], "beta": cfg["beta"], "useful_flops": F, "order": order,
                   **({"stored_rank_flops": F_stored, "useful_flops_basis": basis} if sixteen else {}),
                   "runs": info["runs"], "groups": info["groups"], "streams": n_streams, "pipelined": pipelined,
                   "workspace_GiB": round(info["workspace_bytes"] / 2 ** 30, 3)},
        "roofline": roofline,
        "path_roofline": {"bound": "mfma" if roof >= peak else "hbm", "achieved": round(value, 3),
                          "roof": round(roof, 2), "unit": "TFLOP/s", "frac": round(value / roof, 4),
                          "arith_intensity": round(ai, 2)},
        "step_ms": step_stats,
        "stages_ms": {"stage1": round(stage_ms[0] / nexec, 4), "stage2": round(stage_ms[1] / nexec, 4),
                      "stage3": round(stage_ms[2] / nexec, 4), "side": round(stage_ms[4] / nexec, 4),
                      "execute": round(stage_ms[3] / nexec, 4)},
        "dense_reference": dense,
        "cpu_baseline": cpu,
    }
    if comparator is not None:
        out["per_k_comparator"] = comparator
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
