"""Shared helpers of the GPU parity tests."""
import struct

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


def lambda_state_tensor(lam: float, lam_init: float, device=DEV, exp_a=1.0, exp_b=1.0):
    """A hand-made device lambda state (for example lambda = 0 or 1), laid out as the
    library's diffattn_lambda_state: the float64 fields, then the float32 roundings of
    lambda, lambda_init and 1 - lambda_init."""
    raw = struct.pack(da.STATE_FMT, lam, lam_init, exp_a, exp_b, float(np.float32(lam)),
                      float(np.float32(lam_init)), float(np.float32(1.0 - lam_init)), 0.0)
    return torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(device)


def forward_groups(B, H, N):
    """Query groups per wave the bf16 forward uses: one (128-row blocks) when the problem
    has at most 384 blocks of 256 rows, else two (256-row blocks)."""
    return 1 if B * H * ((N + 255) // 256) <= 384 else 2


def row_flagged(ws, B, H, N, bh, row):
    """Whether the forward's fast pass flagged query row `row` of head bh (b H + h) for the
    fixup pass, from the row flags it leaves in its workspace: per block of 128 NG rows,
    4 NG words; bit m of word NG w + g is the row 4 NG m + NG w + g of the block."""
    ng = forward_groups(B, H, N)
    rb, fw = 128 * ng, 4 * ng
    nqb = (N + rb - 1) // rb
    qb, r = divmod(row, rb)
    m, rest = divmod(r, fw)
    word = rest            # NG w + g
    flags = ws.view(torch.int32).cpu().numpy()
    return bool((int(flags[fw * (bh * nqb + qb) + word]) >> m) & 1)
