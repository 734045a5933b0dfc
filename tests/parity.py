"""Parity helpers shared by the GPU tests.

Acceptance bar of the block: max-abs error <= 2e-2 * RMS(oracle) and cosine
similarity >= 0.9995, in float64 over the compared elements.

bf16 outputs: the output format alone carries an error of up to half a bf16
ulp per element, 2^(floor(log2|v|) - 8), which exceeds 2e-2 * RMS wherever an
output is larger than about 10 * RMS (heavy-tailed outputs such as the gated
residual at the Flux shape, or GELU outputs).  For bf16 outputs the max-abs
bar is therefore applied to the error in excess of that half ulp (taken at
the larger of |gpu| and |oracle|); the raw max-abs error and the format's own
floor, max |bf16(oracle) - oracle|, are printed for every comparison.  The
cosine bar is applied to the raw values.  fp32 outputs get no allowance.
"""
import numpy as np

MAX_ABS_FRAC = 2e-2
MIN_COS = 0.9995


def half_ulp_bf16(v):
    a = np.maximum(np.abs(np.asarray(v, np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 8.0)


def round_bf16_ref(v):
    import torch
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).double().numpy()


def stats(gpu, ref, quantum="bf16"):
    g = np.asarray(gpu, np.float64).ravel()
    r = np.asarray(ref, np.float64).ravel()
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    err = np.abs(g - r)
    raw = float(err.max()) if r.size else 0.0
    if quantum == "bf16" and r.size:
        excess = float(np.max(np.maximum(err - np.maximum(half_ulp_bf16(r), half_ulp_bf16(g)), 0.0)))
        floor = float(np.max(np.abs(round_bf16_ref(r) - r)))
    else:
        excess, floor = raw, 0.0
    den = float(np.linalg.norm(g) * np.linalg.norm(r))
    cos = float(np.dot(g, r) / den) if den > 0 else 1.0
    f = lambda x: x / rms if rms > 0 else 0.0
    return dict(max_abs=raw, rms=rms, ratio=f(raw), floor_ratio=f(floor), excess=excess, excess_ratio=f(excess),
                cos=cos)


def assert_parity(gpu, ref, name="", quantum="bf16", check_max_abs=True):
    s = stats(gpu, ref, quantum)
    print(f"[parity] {name}: max_abs/rms={s['ratio']:.3e} (bf16 floor {s['floor_ratio']:.3e}, "
          f"beyond half-ulp {s['excess_ratio']:.3e}) rms={s['rms']:.3e} cos={s['cos']:.7f}", flush=True)
    assert np.all(np.isfinite(np.asarray(gpu, np.float64))), f"{name}: non-finite output"
    if check_max_abs:
        assert s["excess"] <= MAX_ABS_FRAC * s["rms"], f"{name}: {s}"
    assert s["cos"] >= MIN_COS, f"{name}: {s}"
    return s


def dev_bf16(a):
    """float32 numpy array of bf16 values -> torch bf16 tensor on the GPU (exact)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda").to(torch.bfloat16)


def dev_f32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda")


def host(t):
    return t.float().cpu().numpy().astype(np.float64)
