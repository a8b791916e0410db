"""Oracle references with their accumulation bounds, for the GEMM gate.

Each function returns a dict: ``ref`` (the oracle's fp64 reference on the
given FP8 operands), ``B`` (the accumulation bound of oracle.tolerance, for
every output) and, for the neighbour clause, ``rows`` (the output rows it is
checked on: all of them when the matrix unit's truncation D costs at most
2^30 products, else an even sample), ``R`` (ref - D on those rows) and
``Bf`` (the fp32 part of the bound on those rows).  Test helper only.
"""

import concurrent.futures
import functools

import numpy as np

from oracle import gemm, moe, quant, tolerance
from workloads import synth

A = tolerance.abs_codes
CLAUSE_PRODUCTS = 1 << 30


def clause_rows(M, N, K, budget=CLAUSE_PRODUCTS):
    """All rows when M N K <= budget products, else an even sample of rows
    within the budget."""
    if M * N * K <= budget:
        return np.arange(M)
    n = max(1, budget // (N * K))
    return np.unique(np.linspace(0, M - 1, n).astype(np.int64))


def truncation(aq, as_, wq, ws, mode):
    """oracle.tolerance.unit_truncation over column chunks in threads (small
    chunks stay in cache; numpy releases the GIL in the array operations).
    ws: per weight row (block, row mode) or one value (tensor)."""
    N = wq.shape[0]
    ws = np.asarray(ws, dtype=np.float32)
    per_row = mode != "tensor" and ws.size > 1
    starts = list(range(0, N, 256))

    def part(lo):
        sl = slice(lo, min(lo + 256, N))
        return tolerance.unit_truncation(aq, as_, wq[sl], ws[sl] if per_row else ws, mode)

    with concurrent.futures.ThreadPoolExecutor(16) as ex:
        return np.concatenate(list(ex.map(part, starts)), axis=1)


def _pack(ref, T, S1, K, mode, rows, D):
    B, Bf = tolerance.accumulation_bounds(T, S1, K, mode)
    return {"ref": ref, "B": B, "rows": rows, "R": ref[rows] - D, "Bf": Bf[rows]}


def block_rows(aq, as_, wq_rows, ws_rows, budget=CLAUSE_PRODUCTS):
    M, K = aq.shape
    ref = gemm.gemm_block_ref_rows(aq, as_, wq_rows, ws_rows)
    T = gemm.gemm_block_ref_rows(A(aq), np.abs(as_), A(wq_rows), np.abs(ws_rows))
    S1 = tolerance.truncation_terms(aq, as_, wq_rows, ws_rows, "block")
    rows = clause_rows(M, wq_rows.shape[0], K, budget)
    D = truncation(aq[rows], as_[rows], wq_rows, ws_rows, "block")
    return _pack(ref, T, S1, K, "block", rows, D)


def block(aq, as_, wq, ws):
    return block_rows(aq, as_, wq, np.repeat(np.asarray(ws, dtype=np.float32), 128, axis=0))


def tensor(aq, as_, wq, ws):
    M, K = aq.shape
    ref = gemm.gemm_tensor_ref(aq, as_, wq, ws)
    T = gemm.gemm_tensor_ref(A(aq), np.abs(as_), A(wq), np.abs(ws))
    S1 = tolerance.truncation_terms(aq, as_, wq, ws, "tensor")
    rows = clause_rows(M, wq.shape[0], K)
    D = truncation(aq[rows], as_, wq, ws, "tensor")
    return _pack(ref, T, S1, K, "tensor", rows, D)


def rows(aq, sa, wq, sw):
    M, K = aq.shape
    ref = gemm.gemm_rows_ref(aq, sa, wq, sw)
    T = gemm.gemm_rows_ref(A(aq), np.abs(sa), A(wq), np.abs(sw))
    S1 = tolerance.truncation_terms(aq, sa, wq, sw, "row")
    r = clause_rows(M, wq.shape[0], K)
    sar = np.asarray(sa, dtype=np.float32).reshape(-1)
    D = truncation(aq[r], sar if sar.size == 1 else sar[r], wq, sw, "row")
    return _pack(ref, T, S1, K, "row", r, D)


def grouped(aq, as_, wq, ws, offsets):
    """The grouped GEMM: each expert's rows against that expert's weight
    (rows in no segment: NaN reference, zero bounds, no clause)."""
    M, K = aq.shape
    E, N = wq.shape[0], wq.shape[1]
    ref = moe.grouped_gemm_ref(aq, as_, wq, ws, offsets)
    B = np.zeros((M, N))
    rows_all, R_all, Bf_all = [], [], []
    off = [int(v) for v in offsets]
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            d = block(aq[lo:hi], as_[lo:hi], wq[e], ws[e])
            B[lo:hi] = d["B"]
            rows_all.append(lo + d["rows"])
            R_all.append(d["R"])
            Bf_all.append(d["Bf"])
    cat = (lambda x: np.concatenate(x)) if rows_all else (lambda x: np.zeros((0, N)))
    return {"ref": ref, "B": B, "rows": cat(rows_all).astype(np.int64) if rows_all else
            np.zeros(0, np.int64), "R": cat(R_all), "Bf": cat(Bf_all)}


def select(d, idx):
    """The reference dict restricted to output rows ``idx`` (clause rows kept
    where they fall inside the selection, renumbered)."""
    idx = np.asarray(idx)
    pos = {int(r): i for i, r in enumerate(d["rows"])}
    keep = [(j, pos[int(r)]) for j, r in enumerate(idx) if int(r) in pos]
    return {"ref": d["ref"][idx], "B": d["B"][idx],
            "rows": np.array([j for j, _ in keep], dtype=np.int64),
            "R": d["R"][[i for _, i in keep]] if keep else d["R"][:0],
            "Bf": d["Bf"][[i for _, i in keep]] if keep else d["Bf"][:0]}


def check(out_bits, d):
    """The gate on every output, and the neighbour clause on the clause rows.
    Returns the two result dicts merged (clause keys from the second)."""
    r = tolerance.check(out_bits, d["ref"], d["B"])
    if len(d["rows"]):
        rc = tolerance.check(out_bits[d["rows"]], d["ref"][d["rows"]], d["B"][d["rows"]], d["R"],
                             d["Bf"])
        for k in ("max_ulp_vs_unit", "max_ulp_where_clause_holds", "n_clause_checked",
                  "n_clause_exempt", "neighbour_gate_ok"):
            r[k] = rc[k]
        r["ok"] = bool(r["ok"] and rc["ok"])
    return r


def parallel_rows(fn, bits, chunk):
    """fn over row chunks of ``bits`` in threads (numpy releases the GIL in
    the quantizer's array operations); returns the concatenated codes and
    scales.  ``chunk`` must respect the function's row grouping (a multiple
    of 128 for the 128x128 weight quantizer)."""
    starts = list(range(0, bits.shape[0], chunk))
    with concurrent.futures.ThreadPoolExecutor(8) as ex:
        parts = list(ex.map(lambda i: fn(bits[i:i + chunk]), starts))
    return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))


@functools.lru_cache(maxsize=2)
def workload(name):
    """The seeded bf16 inputs of a workload and the oracle's block-mode codes
    and scales of both operands (cached: several tests share them)."""
    d = synth.make_config(name)
    aq, as_ = parallel_rows(quant.quant_act_ref, d["A"], 256)
    wq, ws = parallel_rows(quant.quant_weight_block_ref, d["W"], 512)
    return d, aq, as_, wq, ws


def block_cols(aq, as_, wq, ws, cols, budget=CLAUSE_PRODUCTS):
    """The reference dict of the block GEMM restricted to output columns
    ``cols`` (weight rows), each column keeping its weight block's scales."""
    return block_rows(aq, as_, wq[cols], np.repeat(ws, 128, axis=0)[cols], budget)
