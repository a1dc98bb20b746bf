"""Shared helpers of the GPU parity tests: host<->device transfers and the parity bars.

Parity bars: bf16 outputs max|gpu - oracle| <= 2e-2 * RMS(oracle) over the whole tensor; fp32
intermediates (inv_rms, lse) within 1e-4 relative error, measured against max(|value|, 1);
-inf where the oracle has -inf."""
import sys

import numpy as np
import torch

from oracle import mla_oracle as O

BF16_TOL = 2e-2
F32_RTOL = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bits_of(vals: np.ndarray) -> np.ndarray:
    return O.bf16_encode(vals)


def assert_bf16_parity(gpu_bits: np.ndarray, oracle_vals: np.ndarray, what: str, per_vector: bool = True) -> float:
    """max|gpu - oracle| <= 2e-2 * RMS(oracle).

    `oracle_vals` is the oracle's staged value BEFORE its final bf16 rounding: the GPU output is
    itself the rounding of its own accumulator, and comparing two independently rounded values
    would charge one bf16 quantum twice. With per_vector (the default) the RMS is taken over each
    output vector -- the last axis: one head's 128 output features, or one head's 192 query
    features -- since attention outputs of different rows have different scales (early prefill
    rows are single values, later rows averages); the whole-tensor ratio is reported too."""
    g = O.bf16_decode(gpu_bits)
    o = np.asarray(oracle_vals, np.float64)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU values"
    if not o.size:
        return 0.0
    err = np.abs(g - o)
    rms_all = float(np.sqrt(np.mean(o * o)))
    whole = float(err.max()) / max(rms_all, 1e-30)
    if per_vector:
        rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True))
        vec_err = err.max(axis=-1, keepdims=True)
        ok = (vec_err <= BF16_TOL * rms) | ((rms == 0) & (vec_err == 0))
        ratio = float(np.max(vec_err / np.maximum(rms, 1e-30)))
        say(f"  {what}: max per-vector |err|/rms = {ratio:.3e} (whole tensor {whole:.3e})")
        assert ok.all(), f"{what}: {int((~ok).sum())} vectors exceed {BF16_TOL} x their RMS (worst {ratio:.3e})"
        return ratio
    say(f"  {what}: max|err|/rms = {whole:.3e}")
    assert whole <= BF16_TOL, f"{what}: max|err| / rms {whole} > {BF16_TOL}"
    return whole


def assert_f32_parity(gpu: np.ndarray, oracle: np.ndarray, what: str, rtol: float = F32_RTOL,
                      magnitude=None) -> float:
    g = np.asarray(gpu, np.float64)
    o = np.asarray(oracle, np.float64)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    ninf = np.isneginf(o)
    assert np.array_equal(np.isneginf(g), ninf), f"{what}: -inf pattern differs"
    fin = ~ninf
    if not fin.any():
        return 0.0
    assert np.all(np.isfinite(g[fin])), f"{what}: non-finite GPU values"
    # Relative to max(|value|, magnitude, 1). lse is a logarithm whose zero is arbitrary (shifting
    # every score shifts it), so below magnitude 1 the bar is 1e-4 absolute -- a 1e-4 relative error
    # of exp(lse). Its error is that of the score dot products, whose relative error is measured
    # against the sum of the magnitudes of their terms (`magnitude`, from the oracle).
    ref = np.maximum(np.abs(o[fin]), 1.0)
    if magnitude is not None:
        ref = np.maximum(ref, np.asarray(magnitude, np.float64)[fin])
    rel = float(np.max(np.abs(g[fin] - o[fin]) / ref))
    say(f"  {what}: max rel err = {rel:.3e}")
    assert rel <= rtol, f"{what}: relative error {rel} > {rtol}"
    return rel
