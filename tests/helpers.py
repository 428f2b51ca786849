"""Small host-side helpers for tests: exact bf16 encodings of values that are
representable, and the comparison rules used for GPU-vs-oracle parity."""
import numpy as np


def f64_to_bf16_bits_exact(x):
    """Encode float64 values that are exactly representable in bf16 (asserted)."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    if not np.array_equal(f.astype(np.float64), x):
        raise ValueError("value not representable in fp32")
    bits = f.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("value not representable in bf16")
    return (bits >> 16).astype(np.uint16)


def int_bf16(a):
    """Integer-valued array (|v| <= 256) -> exact bf16 bit patterns."""
    a = np.asarray(a)
    if np.any(np.abs(a) > 256):
        raise ValueError("integers above 256 are not all exact in bf16")
    return f64_to_bf16_bits_exact(a.astype(np.float64))


def bf16_bits_rne(x):
    """Round float64 -> float32 -> bf16 (nearest-even) bit patterns."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def score_close(gpu, ora, rel=1e-4, rms_frac=1e-6):
    """Scores: |gpu - ora| <= rel*|ora| + rms_frac*rms(ora) per slice (last axis)."""
    gpu = np.asarray(gpu, np.float64)
    ora = np.asarray(ora, np.float64)
    rms = np.sqrt(np.mean(ora ** 2, axis=-1, keepdims=True))
    bound = rel * np.abs(ora) + rms_frac * rms
    bad = np.abs(gpu - ora) > bound
    return (not bad.any()), float(np.max(np.abs(gpu - ora) / np.maximum(np.abs(ora), 1e-30))), int(bad.sum())


def lowrank_close(gpu, ora, rel=2e-3):
    """Low-rank outputs: |gpu - ora| <= rel*(|ora| + rms(ora_slice)) per slice (axis 0 = slice)."""
    gpu = np.asarray(gpu, np.float64)
    ora = np.asarray(ora, np.float64)
    axes = tuple(range(1, ora.ndim))
    rms = np.sqrt(np.mean(ora ** 2, axis=axes, keepdims=True))
    bound = rel * (np.abs(ora) + rms)
    err = np.abs(gpu - ora)
    return bool((err <= bound).all()), float((err / (np.abs(ora) + rms)).max())


def index_sets_agree(gpu_idx, ora_idx, ora_scores32, k, rel=1e-4):
    """Retained-set rule: exactly k unique ascending indices; the symmetric
    difference with the oracle set holds only tokens whose oracle score lies
    within rel of the oracle's k-th largest score.  Returns (ok, n_boundary)."""
    gpu_idx = np.asarray(gpu_idx)
    ora_idx = np.asarray(ora_idx)
    nb = 0
    for g in range(ora_idx.shape[0]):
        a = gpu_idx[g]
        if a.shape[0] != k or (k > 1 and np.any(np.diff(a) <= 0)):
            return False, -1
        if k == 0:
            continue
        sk = np.sort(ora_scores32[g].astype(np.float64))[::-1][k - 1]
        diff = np.setxor1d(a, ora_idx[g])
        if diff.size:
            if np.any(diff < 0) or np.any(diff >= ora_scores32.shape[1]):
                return False, -1
            if np.any(np.abs(ora_scores32[g][diff].astype(np.float64) - sk) > rel * abs(sk)):
                return False, -1
            nb += diff.size
    return True, nb


def bf16_close(gpu_bits, ora, ulps=1, abs_frac=2.0 ** -14):
    """bf16 outputs: within +-ulps bf16 ulps of the oracle's value rounded to bf16
    (nearest even), or within abs_frac * rms(slice) absolutely: for values below
    ~2^-6 of the slice's rms a bf16 ulp is smaller than the fp32 result's own error
    (hi/lo-split operands, fp32 accumulation: a few 2^-16 of the row scale).
    Axis 0 = slice.  Returns (ok, worst ulp distance among failures, or overall)."""
    gpu_bits = np.asarray(gpu_bits, np.uint16)
    ora = np.asarray(ora, np.float64)
    ob = bf16_bits_rne(ora)

    def ordered(b):
        b = b.astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)

    dist = np.abs(ordered(gpu_bits) - ordered(ob))
    g = (gpu_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    axes = tuple(range(1, ora.ndim))
    rms = np.sqrt(np.mean(ora ** 2, axis=axes, keepdims=True))
    ok = (dist <= ulps) | (np.abs(g - ora) <= abs_frac * rms)
    return bool(ok.all()), int(dist[~ok].max()) if (~ok).any() else int(dist.max())


def built_library():
    """True once libkvc.so exists: it is compiled here (hipcc, gfx950) when a fresh
    checkout has none; False only where hipcc is not installed."""
    import os
    import shutil
    from token_scoring_eviction_amd import build, kvc
    if not os.path.exists(kvc.LIB_PATH):
        if shutil.which(build.HIPCC) is None and not os.path.exists(build.HIPCC):
            return False
        build.build(verbose=False)
    return os.path.exists(kvc.LIB_PATH)
