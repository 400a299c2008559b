"""Shared helpers for the GPU parity tests (inputs from synth, expectations from oracle)."""
import sys

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
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / den) if den > 0 else float(np.max(np.abs(got)))


def oracle_bank(w13: torch.Tensor, w2: torch.Tensor):
    """Oracle dequant bank over bf16 expert weights living on any device (copied per expert on use)."""
    return offn.DequantBank(lambda e: bits(w13[e]), lambda e: bits(w2[e]))


def tol_for_layer():
    # bf16 rounding of the SwiGLU output h and of the final output, fp32 elsewhere;
    # max |err| / max |ref| of a layer output must stay within 1e-2.
    return 1e-2
