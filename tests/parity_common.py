"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the float64 oracle on the same seeded bytes, and compare them."""

import sys

import numpy as np

from oracle import muon_oracle as orc

SCALE_NAMES = {0: orc.SCALE_NONE, 1: orc.SCALE_ORIGINAL, 2: orc.SCALE_MATCH_RMS_ADAMW, 3: orc.SCALE_SPECTRAL}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_f(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return float(num / den) if den > 0 else float(num)


def decode(arr, dtype):
    """Stored bytes (uint16 bf16 bits or float32) -> float64, exactly."""
    if dtype == "bf16":
        return orc.bf16_bits_to_f64(arr)
    return np.asarray(arr, np.float64)


def bf16_ulp_distance(a_bits, b_bits):
    """Distance in bf16 ulps between two uint16 bit arrays (ordered-int map)."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + x)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def to_device(torch, arr, dtype, device="cuda"):
    if dtype == "bf16":
        t = torch.from_numpy(arr.view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def from_device(torch, t, dtype):
    t = t.detach().cpu()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().astype(np.float32)


def oracle_step(W, G, M, dtype, hp, split_rows=0, lr=None, lr_mult=1.0, S_invs=None):
    """Oracle step on stored bytes; returns dict with M, O, W (float64) and,
    for bf16 params, W_bits (RNE of the float64 result)."""
    res = orc.muon_step(decode(W, dtype), decode(G, dtype), np.asarray(M, np.float64),
                        lr=hp.lr if lr is None else lr, weight_decay=hp.weight_decay,
                        momentum=hp.momentum, nesterov=bool(hp.nesterov), ns_steps=hp.ns_steps,
                        eps=hp.eps, coeffs=(hp.ns_a, hp.ns_b, hp.ns_c),
                        scale_mode=SCALE_NAMES[hp.scale_mode],
                        momentum_form="sgd" if hp.momentum_form == 1 else "ema",
                        split_rows=split_rows, lr_mult=lr_mult, S_invs=S_invs)
    if dtype == "bf16":
        res["W_bits"] = orc.f64_to_bf16_bits(res["W"])
    return res


def float32_hparams(hp):
    """The hyper-parameters exactly as the library sees them (float32)."""
    import ctypes
    out = {}
    for name, _ in hp._fields_:
        out[name] = getattr(hp, name)
    return out


def bf16_ulp(x):
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    ax = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_w_bf16(W_gpu_bits, ref, lr, scales, tol_o=2e-2):
    """New bf16 weights against the float64 oracle.

    W' = W - lr*wd*W - lr*s*O is rounded once to bf16, so the GPU result may
    differ from the exact W' by the rounding (at most half an ulp of W' per
    element) plus lr*s times the allowed deviation of O (tol_o relative in
    the Frobenius norm).  Returns (error, bound, fraction bitwise equal to
    RNE(W'))."""
    Wg = orc.bf16_bits_to_f64(W_gpu_bits)
    Wr = np.asarray(ref["W"], np.float64)
    s = np.asarray(scales, np.float64).reshape(-1, 1)
    err = float(np.linalg.norm(Wg - Wr))
    bound = (0.5 * float(np.linalg.norm(bf16_ulp(Wr))) * 1.001
             + lr * tol_o * float(np.linalg.norm(s * np.asarray(ref["O"], np.float64)))
             + 1e-6 * float(np.linalg.norm(Wr)))
    frac = float(np.mean(W_gpu_bits == ref["W_bits"]))
    return err, bound, frac


def check_w_update_elementwise(W_gpu_bits, W0_bits, O_gpu, lr, weight_decay, scales):
    """The fused weight update, element by element: given the GPU's own
    orthogonalised update O (read back through update_out), each new bf16
    weight must be one of the two bf16 neighbours of W - lr*wd*W - lr*s*O
    (decoupled decay, Muon README "Usage").  The kernel evaluates that in
    float32 and rounds once; its float32 roundings move the value by at most a
    few float32 ulps of the operands, which matters only where W and lr*s*O
    nearly cancel.  So |W'_gpu - W'| <= ulp_bf16(W') + 8 * 2^-24 (|W| +
    lr*s*|O|), with W' in float64.  Returns (max of |W'_gpu - W'| / that
    bound, fraction not bitwise equal to RNE(W'))."""
    s = np.asarray(scales, np.float64).reshape(-1, 1)
    W0 = orc.bf16_bits_to_f64(W0_bits)
    O = np.asarray(O_gpu, np.float64)
    W_exp = orc.apply_update(W0, O, lr, weight_decay, s)
    Wg = orc.bf16_bits_to_f64(np.asarray(W_gpu_bits))
    allowed = bf16_ulp(W_exp) + 8.0 * 2.0 ** -24 * (np.abs(W0) + lr * np.abs(s * O))
    ratio = np.abs(Wg - W_exp) / allowed
    exp_bits = orc.f64_to_bf16_bits(W_exp)
    off = np.asarray(W_gpu_bits) != exp_bits
    return (float(ratio.max()) if ratio.size else 0.0), (float(np.mean(off)) if off.size else 0.0)
