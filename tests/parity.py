"""Parity helpers shared by the GPU tests: the acceptance bar of the block
(max |gpu - oracle| <= 2e-2 * RMS(oracle) and cosine >= 0.9995, both in
float64 over the compared elements) and small input conversions."""
import numpy as np

MAX_ABS_FRAC = 2e-2
MIN_COS = 0.9995


def stats(gpu, ref):
    g = np.asarray(gpu, np.float64).ravel()
    r = np.asarray(ref, np.float64).ravel()
    rms = float(np.sqrt(np.mean(r * r)))
    err = float(np.max(np.abs(g - r))) if r.size else 0.0
    den = float(np.linalg.norm(g) * np.linalg.norm(r))
    cos = float(np.dot(g, r) / den) if den > 0 else 1.0
    return dict(max_abs=err, rms=rms, ratio=err / rms if rms > 0 else 0.0, cos=cos)


def assert_parity(gpu, ref, name=""):
    s = stats(gpu, ref)
    print(f"[parity] {name}: max_abs={s['max_abs']:.3e} rms={s['rms']:.3e} "
          f"max_abs/rms={s['ratio']:.3e} cos={s['cos']:.7f}", flush=True)
    assert np.all(np.isfinite(np.asarray(gpu, np.float64))), f"{name}: non-finite output"
    assert s["max_abs"] <= MAX_ABS_FRAC * s["rms"], f"{name}: {s}"
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
