"""Helpers for the GPU parity tests: device upload, error metrics, oracle runs."""
from __future__ import annotations

import math
import os
import sys

import numpy as np

# Gates (max |err| / rms(y) of the oracle output):
#   fp32 I/O: 1e-4.
#   bf16 I/O: 2e-2 on the compute error, i.e. after allowing each element its
#   own output rounding to bf16 (at most 2^-8 |y|; the gate alone sits below the
#   rounding floor of the exact result when |y| reaches ~5x rms, which these
#   inputs do).
GATE_F32 = 1e-4
GATE_BF16 = 2e-2
BF16_HALF_ULP = 2.0 ** -8


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# Achieved errors of every compared output, kept for the summary printed at the end of the
# session: (test id, quantity, raw max|err|/rms, compute error or None).
RECORDS = []


def record(quantity, raw, comp=None):
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    RECORDS.append((test, quantity, float(raw), None if comp is None else float(comp)))


def to_dev(inp: dict, io: str, device="cuda"):
    import torch
    out = {}
    for k, v in inp.items():
        t = torch.from_numpy(np.ascontiguousarray(v))
        if k in ("x", "B", "C") and io == "bf16":
            t = t.to(torch.bfloat16)
        out[k] = t.to(device)
    return out


def state_to_dev(st: dict, device="cuda"):
    import torch
    return {k: torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(device) for k, v in st.items()}


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def err_metrics(y_gpu, y_ref, io: str):
    """(raw, compute) errors relative to rms(y_ref); compute removes the bf16 output quantum."""
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    if y_ref.size == 0:
        return 0.0, 0.0
    rms = math.sqrt(float(np.mean(y_ref * y_ref))) or 1.0
    d = np.abs(y_gpu - y_ref)
    raw = float(d.max()) / rms
    if io == "bf16":
        comp = float(np.maximum(d - BF16_HALF_ULP * np.abs(y_ref), 0.0).max()) / rms
    else:
        comp = raw
    return raw, comp


def gate(io: str) -> float:
    return GATE_BF16 if io == "bf16" else GATE_F32


def angle_err(a_gpu, a_ref):
    """Max |wrapped difference| of angles, relative to rms of the wrapped reference."""
    d = np.asarray(a_gpu, np.float64) - np.asarray(a_ref, np.float64)
    d = (d + math.pi) % (2 * math.pi) - math.pi
    ref = np.mod(np.asarray(a_ref, np.float64), 2 * math.pi)
    rms = math.sqrt(float(np.mean(ref * ref))) or 1.0
    return float(np.abs(d).max()) / rms if d.size else 0.0


def oracle_args(inp: dict):
    return (inp["x"], inp["B"], inp["C"], inp["dt"], inp["lam"], inp["theta"], inp["A"], inp["D"])


def head_slice(inp: dict, heads):
    """Restrict a workload's inputs to a subset of heads (sequences are independent per head)."""
    out = {}
    for k, v in inp.items():
        if k in ("A", "D"):
            out[k] = v[heads]
        elif k in ("b_bias", "c_bias"):
            out[k] = v[heads]
        elif k in ("b_norm_w", "c_norm_w"):
            out[k] = v
        else:
            out[k] = v[:, :, heads]
    return out
