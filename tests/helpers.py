"""Shared helpers of the GPU parity tests: moving seeded bit arrays to the GPU,
reading outputs back as float64, and the parity metrics and gates.

Gates: max-abs / mean-abs error 2e-2 / 2e-3 for bf16 inputs and 1e-2 / 1e-3
for fp16 inputs; relative RMS error <= 1e-2 and cosine similarity >= 0.9999 on
top, because with long key ranges the outputs are small (|O| ~ 1e-2) and an
absolute bound alone would be loose.
"""
import sys

import numpy as np

TOL = {"bf16": (2e-2, 2e-3), "fp16": (1e-2, 1e-3)}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return t.cuda()


def i32_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def metrics(out: np.ndarray, ref: np.ndarray) -> dict:
    out = np.asarray(out, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    err = np.abs(out - ref)
    nref = np.linalg.norm(ref)
    nout = np.linalg.norm(out)
    return {
        "max_abs": float(err.max()) if err.size else 0.0,
        "mean_abs": float(err.mean()) if err.size else 0.0,
        "rel_rms": float(np.linalg.norm(out - ref) / nref) if nref > 0 else float(np.linalg.norm(out)),
        "cos": float(out @ ref / (nout * nref)) if nref > 0 and nout > 0 else 1.0,
        "finite": bool(np.isfinite(out).all()),
    }


# Relative half-ulp of a 16-bit type (round to nearest).
HALF_ULP = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}


def assert_parity(out, ref, in_dtype: str, what: str = "", partial_dtype: str = None) -> dict:
    """partial_dtype: the 16-bit type of key-split partial outputs, when the
    result went through them. Each partial row is rounded to that type before
    the combine, and the output rounds the combined value again, so each
    element may also be off by half an ulp of its own magnitude: the max-abs
    gate becomes |o - ref| <= max_abs + half_ulp * |ref| per element. (Only a
    peaked softmax, where an output row is nearly one value row with |O| up to
    ~4.6, makes that term matter: one bf16 ulp is 0.031 in [4, 8).)"""
    m = metrics(out, ref)
    mx, mean = TOL[in_dtype]
    log(f"parity {what}: " + " ".join(f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}"
                                      for k, v in m.items()))
    assert m["finite"], f"{what}: non-finite output"
    if partial_dtype in HALF_ULP:
        o = np.asarray(out, dtype=np.float64).ravel()
        r = np.asarray(ref, dtype=np.float64).ravel()
        excess = np.abs(o - r) - (mx + HALF_ULP[partial_dtype] * np.abs(r))
        assert excess.size == 0 or excess.max() <= 0, \
            f"{what}: max-abs {m['max_abs']:.3g} beyond {mx} + half an ulp of the partials"
    else:
        assert m["max_abs"] <= mx, f"{what}: max-abs {m['max_abs']:.3g} > {mx}"
    assert m["mean_abs"] <= mean, f"{what}: mean-abs {m['mean_abs']:.3g} > {mean}"
    if np.linalg.norm(np.asarray(ref)) > 0:
        assert m["rel_rms"] <= 1e-2, f"{what}: relative RMS {m['rel_rms']:.3g} > 1e-2"
        assert m["cos"] >= 0.9999, f"{what}: cosine {m['cos']:.6f} < 0.9999"
    return m


# lse tolerance. The kernels sum the row's probabilities as rounded to the P.V
# operand type (so that O's weights are exactly the ones it is normalised by):
# with one dominant key, l is then off by up to half an ulp of that type, i.e.
# a relative 2^-8 for bf16 and 2^-11 for fp16, and lse = m + ln l by about the
# same absolute amount; the rest (fp32 sums and scores) is far smaller.
LSE_TOL = {"bf16": 5e-3, "fp16": 2e-3}


def assert_lse(lse, ref, what: str = "", tol: float = None, dtype: str = "bf16") -> None:
    tol = LSE_TOL[dtype] if tol is None else tol
    lse = np.asarray(lse, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    inf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(lse), inf), f"{what}: -inf pattern differs"
    if (~inf).any():
        err = np.abs(lse[~inf] - ref[~inf]).max()
        log(f"lse {what}: max_abs={err:.3g}")
        assert err <= tol, f"{what}: lse error {err:.3g} > {tol}"
