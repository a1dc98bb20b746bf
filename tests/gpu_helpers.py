"""Shared helpers of the GPU parity tests: host<->device transfers and the parity bars.

Parity bars:
  * bf16 outputs: max|err| <= 2e-2 * RMS(oracle), by default per output vector (the last axis: one
    head's 128 outputs, one head's 192 query features, one cache row, one token's wo output),
    against the oracle's value o before its final bf16 rounding. A bf16 output carries the rounding
    of its own last step, which for an element several times its vector's RMS alone approaches the
    bar, so err is how much farther the GPU's output lies from o than the correctly rounded value
    bf16(o) does: err = |gpu - o| - |bf16(o) - o| (0 for a correctly rounded output). The plain
    ratio max|gpu - o| / RMS and the whole-tensor ratio are printed beside it;
  * fp32 intermediates (inv_rms, lse): relative error <= 1e-4 against max(|value|, 1, magnitude),
    where `magnitude` (lse only) is the oracle's sum of the absolute terms of the score dot
    products (decode_score_magnitude / prefill_score_magnitude); the ratio against max(|value|, 1)
    alone is printed beside it;
  * -inf exactly where the oracle has -inf."""
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
    """max|err| <= 2e-2 * RMS(oracle), err = |gpu - o| - |bf16(o) - o|.

    `oracle_vals` is the oracle's staged value o BEFORE its final bf16 rounding. The GPU output is
    a bf16 value, so it cannot come closer to o than bf16(o), the correctly rounded value; err is
    the distance beyond that (0 when the GPU returns bf16(o); about twice the GPU's own error before
    its rounding when that error moves it to the other bf16 neighbour). Charging the output's own
    rounding as well would let the bar fail on a correctly rounded exact result: an element 5 RMS
    large rounds by up to 5 * 2^-8 = 1.95e-2 RMS. With per_vector (the default) the RMS is taken
    over each output vector -- the last axis: one head's 128 output features, or one head's 192
    query features -- since attention outputs of different rows have different scales (early
    prefill rows are single values, later rows averages). The plain ratio max|gpu - o| / RMS and
    the whole-tensor ratio are printed too."""
    g = O.bf16_decode(gpu_bits)
    o = np.asarray(oracle_vals, np.float64)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU values"
    if not o.size:
        return 0.0
    plain = np.abs(g - o)
    err = np.maximum(plain - np.abs(O.bf16_decode(O.bf16_encode(o)) - o), 0.0)
    rms_all = float(np.sqrt(np.mean(o * o)))
    whole = float(plain.max()) / max(rms_all, 1e-30)
    if per_vector:
        rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True))
        vec_err = err.max(axis=-1, keepdims=True)
        ok = (vec_err <= BF16_TOL * rms) | ((rms == 0) & (vec_err == 0))
        ratio = float(np.max(vec_err / np.maximum(rms, 1e-30)))
        plain_ratio = float(np.max(plain.max(axis=-1, keepdims=True) / np.maximum(rms, 1e-30)))
        say(f"  {what}: max per-vector err/rms = {ratio:.3e} (plain |gpu - oracle|/rms {plain_ratio:.3e}, "
            f"whole tensor {whole:.3e})")
        assert ok.all(), f"{what}: {int((~ok).sum())} vectors exceed {BF16_TOL} x their RMS (worst {ratio:.3e})"
        return ratio
    ratio = float(err.max()) / max(rms_all, 1e-30)
    say(f"  {what}: max err/rms = {ratio:.3e} (plain {whole:.3e})")
    assert ratio <= BF16_TOL, f"{what}: max err / rms {ratio} > {BF16_TOL}"
    return ratio


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
    err = np.abs(g[fin] - o[fin])
    ref = np.maximum(np.abs(o[fin]), 1.0)
    literal = float(np.max(err / ref))
    if magnitude is not None:
        ref = np.maximum(ref, np.asarray(magnitude, np.float64)[fin])
    rel = float(np.max(err / ref))
    say(f"  {what}: max rel err = {rel:.3e} (against max(|value|, 1) alone: {literal:.3e})")
    assert rel <= rtol, f"{what}: relative error {rel} > {rtol}"
    return rel
