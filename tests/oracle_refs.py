"""Oracle references with their fp32 accumulation bound, for the GEMM gate.

Each function returns (ref, bound): the fp64 reference of the oracle on the
given FP8 operands and the elementwise bound B of oracle.tolerance, computed
from the same oracle GEMM on absolute codes and scales.  Test helper only.
"""

import numpy as np

from oracle import gemm, moe, tolerance

A = tolerance.abs_codes


def block(aq, as_, wq, ws):
    K = aq.shape[1]
    ref = gemm.gemm_block_ref(aq, as_, wq, ws)
    T = gemm.gemm_block_ref(A(aq), np.abs(as_), A(wq), np.abs(ws))
    return ref, tolerance.accumulation_bound(T, K, "block")


def block_rows(aq, as_, wq_rows, ws_rows):
    K = aq.shape[1]
    ref = gemm.gemm_block_ref_rows(aq, as_, wq_rows, ws_rows)
    T = gemm.gemm_block_ref_rows(A(aq), np.abs(as_), A(wq_rows), np.abs(ws_rows))
    return ref, tolerance.accumulation_bound(T, K, "block")


def tensor(aq, as_, wq, ws):
    K = aq.shape[1]
    ref = gemm.gemm_tensor_ref(aq, as_, wq, ws)
    T = gemm.gemm_tensor_ref(A(aq), np.abs(as_), A(wq), np.abs(ws))
    return ref, tolerance.accumulation_bound(T, K, "tensor")


def rows(aq, sa, wq, sw):
    K = aq.shape[1]
    ref = gemm.gemm_rows_ref(aq, sa, wq, sw)
    T = gemm.gemm_rows_ref(A(aq), np.abs(sa), A(wq), np.abs(sw))
    return ref, tolerance.accumulation_bound(T, K, "row")


def grouped(aq, as_, wq, ws, offsets):
    K = aq.shape[1]
    ref = moe.grouped_gemm_ref(aq, as_, wq, ws, offsets)
    T = moe.grouped_gemm_ref(A(aq), np.abs(as_), A(wq), np.abs(ws), offsets)
    return ref, tolerance.accumulation_bound(T, K, "block")


def take(refb, index):
    """The same selection of both arrays of a (ref, bound) pair."""
    ref, bound = refb
    return ref[index], np.broadcast_to(bound, ref.shape)[index]
