"""Shared helpers for the GPU parity tests (inputs from synth, expectations from oracle)."""
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from oracle import ffn as offn


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> numpy uint16 bit patterns."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def rel_err(got, ref):
    """max |got - ref| / max |ref| over the whole output."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref)) / den) if den > 0 else float(np.max(np.abs(got)))


def token_rel_err(got, ref):
    """Largest per-token error: max over tokens t of max |got_t - ref_t| / max |ref_t|
    (each output row normalised by its own magnitude, so a wrong small row shows)."""
    got = np.asarray(got, dtype=np.float64).reshape(len(ref), -1)
    ref = np.asarray(ref, dtype=np.float64).reshape(len(ref), -1)
    if ref.size == 0:
        return 0.0
    den = np.max(np.abs(ref), axis=1)
    num = np.max(np.abs(got - ref), axis=1)
    return float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1.0), num)))


def oracle_bank(w13: torch.Tensor, w2: torch.Tensor):
    """Oracle dequant bank over bf16 expert weights living on any device (copied per expert on use)."""
    return offn.DequantBank(lambda e: bits(w13[e]), lambda e: bits(w2[e]))


def warm_bank(bank, experts, workers=8):
    """Dequantise the listed experts of an oracle bank ahead of use, several at once
    (numpy releases the interpreter lock inside its array loops)."""
    experts = list(experts)
    with ThreadPoolExecutor(max_workers=max(1, min(workers, len(experts)))) as ex:
        list(ex.map(bank.get, experts))
    return bank


def tol_for_layer():
    # bf16 rounding of the SwiGLU output h and of the final output, fp32 elsewhere;
    # max |err| / max |ref| of a layer output must stay within 1e-2.
    return 1e-2


def check_layer_out(name, got, ref, tol=None):
    """Assert both the whole-output and the per-token relative error are within the
    layer tolerance; returns (whole, per-token)."""
    tol = tol_for_layer() if tol is None else tol
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    e = rel_err(got, ref)
    et = token_rel_err(got, ref)
    say(f"  {name}: max rel err {e:.3e}, worst token {et:.3e}")
    assert e <= tol, f"{name}: max rel err {e}"
    assert et <= tol, f"{name}: worst per-token rel err {et}"
    return e, et
