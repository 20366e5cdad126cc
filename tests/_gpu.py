"""Helpers shared by the GPU tests: device copies of canonical inputs and the
tolerance check.  The oracle computes every expected value."""
import numpy as np

import oracle


def dev():
    import torch
    return torch.device("cuda:0")


def to_dev(a: np.ndarray):
    """numpy -> device tensor; uint16 bit patterns travel as int16."""
    import torch
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bf16_dev(bits: np.ndarray):
    import torch
    return to_dev(bits).view(torch.bfloat16)


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def pack_canonical(w: dict, flags: int = 0):
    import ffn_int4_g128_amd as q
    return q.pack(to_dev(w["qweight"]), to_dev(w["scales"]), to_dev(w["zeros"]), w["N"], w["K"],
                  flags)


def assert_within(got: np.ndarray, ref: np.ndarray, tol: np.ndarray, what: str):
    """|got - ref| <= tol elementwise (tol = C_TOL * sum|w*x| or a composite of it)."""
    err = np.abs(got - ref)
    bad = err > tol
    ratio = float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0
    if bad.any():
        i = np.unravel_index(np.argmax(err / np.maximum(tol, 1e-300)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} outside tolerance; worst at "
                             f"{i}: got {got[i]!r} ref {ref[i]!r} tol {tol[i]!r}")
    print(f"{what}: max err/tol = {ratio:.3g}", flush=True)
    return ratio
