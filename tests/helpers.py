"""Shared helpers of the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

from differential_attention_causal_amd import diffattn as da
from differential_attention_causal_amd import synth
from oracle import diffattn_oracle as orc

DEV = "cuda:0"


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy() if t.dtype == torch.bfloat16 \
        else t.detach().cpu().double().numpy()


def draw(w, seed=None, with_dout=None):
    """Inputs on the GPU and their exact float64 host copies."""
    x = synth.make_inputs(w, DEV, seed=seed, with_dout=with_dout)
    torch.cuda.synchronize()
    return x, {k: np64(v) for k, v in x.items()}


def lam_pair(x, h, layer):
    """Device lambda state from the library and the oracle's lambda."""
    st = da.lambda_(x["lq1"], x["lk1"], x["lq2"], x["lk2"], layer)
    ls = orc.lambda_scalar(h["lq1"], h["lk1"], h["lq2"], h["lk2"], layer)
    return st, ls


def normwise_rel(a, ref, axes):
    """max |a - ref| / max |ref| over the given axes (per remaining index)."""
    num = np.max(np.abs(a - ref), axis=axes)
    den = np.max(np.abs(ref), axis=axes)
    return num / np.maximum(den, 1e-300)
