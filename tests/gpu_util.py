"""Helpers shared by the GPU parity tests (device transfer, tolerances, case printing)."""
import sys

import numpy as np

# Layer / GEMM tolerance (fp32 accumulate, fp16 out) against the fp64 oracle on identical
# dequantized weights: relative L2 <= 2e-3 and max |diff| <= 2e-2 * rms(reference).
REL_L2 = 2e-3
MAX_ABS_RMS = 2e-2


def dev(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t):
    return t.detach().cpu().numpy()


def case(msg):
    """Name the case on stdout before its GPU step (flushed, so a dead box still shows it)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def layer_errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = got - ref
    rms = np.sqrt(np.mean(ref * ref)) if ref.size else 0.0
    rel = np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300)
    mx = np.abs(diff).max() / max(rms, 1e-300) if diff.size else 0.0
    return rel, mx


def assert_layer_close(got, ref, what=""):
    assert np.all(np.isfinite(np.asarray(got, dtype=np.float64))), f"{what}: non-finite output"
    rel, mx = layer_errors(got, ref)
    assert rel <= REL_L2 and mx <= MAX_ABS_RMS, f"{what}: rel-L2 {rel:.3e}, max/rms {mx:.3e}"
    return rel, mx


def fp16_ulp(x):
    """Spacing of fp16 at |x| (subnormal spacing below 2^-14)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def assert_within_one_fp16_ulp(got16, ref64, what=""):
    """got16 (fp16) is ref64 rounded to fp16, give or take one fp16 ulp."""
    r16 = np.asarray(ref64).astype(np.float16).astype(np.float64)
    g = np.asarray(got16).astype(np.float64)
    bad = np.abs(g - r16) > fp16_ulp(r16) * 1.0000001
    assert not bad.any(), f"{what}: {bad.sum()} values off by more than 1 fp16 ulp"
