"""Shared helpers of the GPU tests: reading pool pages back and comparing with the oracle."""
from __future__ import annotations

import os

import numpy as np
import torch

from vcsynth import configs as C

TOL_CONTRACT = 5e-3   # max-abs bound on attention outputs (the contract)


# Relative rounding error of one softmax weight as it enters the value product, as a standard
# deviation per weight, per path:
#  * bf16 caches: the weight is rounded to nearest bf16 (8 significant bits), a relative error of
#    at most 2^-8 (half an ulp at the bottom of a binade) and no bias; a uniform error over
#    [-2^-8, 2^-8] has standard deviation 2^-8 / sqrt(3), an upper bound for the rounding.  The
#    weights are exponentials of a running maximum that moves lazily, so even the largest weight
#    of a row is in general not a power of two and carries this error.
#  * KIVI caches: three fp16 roundings (unit roundoff 2^-11), added in quadrature:
#      - the weight itself (fp16 operand of the value product);
#      - the weight times the token's value scale (the folded scale, one more rounding);
#      - the score: each channel's term code_c * fp16(q_c * s_c) carries a rounding of at most
#        2^-11 of itself; with N(0,1) data the terms code_c * s_c = k_c - min(group) have
#        E[(k - min)^2] ~ 5 over groups of 32 (min ~ -2, variance 1), so over d channels the
#        score error (in units of the softmax exponent, after the 1/sqrt(d) scale) has scale
#        2^-11 * sqrt(5 d) / sqrt(d) = 2^-11 * sqrt(5), a relative error of the weight.
#    sqrt(1 + 1 + 5) * 2^-11 ~ 1.3e-3.
SIGMA_W_BF16 = 2.0 ** -8 / np.sqrt(3.0)
SIGMA_W_KIVI = 2.0 ** -11 * np.sqrt(1.0 + 1.0 + 5.0)


def gate(spread, kivi: bool = False):
    """Per-element gate derived from the kernels' arithmetic.  An output element is
    sum_t w_t v_tc over the normalised softmax weights w_t; independent relative errors of
    standard deviation sigma on the weights give it an error of standard deviation at most
    sigma * spread_c, spread_c = sqrt(sum_t (w_t v_tc)^2), which the oracle returns with its
    output.  The gate allows 12 of those plus 1e-4 (fp32 accumulation over the keys), never more
    than the contract.  A long row's weights are spread out (about 3.5e-4 at 32K keys); a short
    row with one dominant key has that key's rounding alone (at most sqrt(3) sigma w |v| on the
    bf16 path), which the gate also covers."""
    s = SIGMA_W_KIVI if kivi else SIGMA_W_BF16
    return np.minimum(TOL_CONTRACT, 12.0 * s * np.asarray(spread, dtype=np.float64) + 1e-4)


# optional log of every comparison's error (path from the environment; off by default)
ERRLOG = os.environ.get("VC_PARITY_LOG")


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"


def bf16_tensor_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def unpack_codes(words: np.ndarray, bits: int, count: int) -> np.ndarray:
    """Codes 0..count-1 of a little-endian uint32 word stream, packed as documented in vc.h:
    code u of a word sits at bit (u%2)*16 + bits*(u/2)."""
    per = 32 // bits
    u = np.arange(count)
    w = words[..., u // per]
    uu = u % per
    shift = (uu % 2) * 16 + bits * (uu // 2)
    return ((w >> shift.astype(np.uint32)) & np.uint32((1 << bits) - 1)).astype(np.uint8)


def pool_tokens_bf16(pool, layer: int, r: int, g: int, n: int, d: int):
    """Read tokens [0, n) of (r, layer, g) back from a bf16 pool: (K [n][d], V [n][d]) float64."""
    pt = pool.page_table[r].cpu().numpy()
    npg = (n + 15) // 16
    ks, vs = [], []
    for p in range(npg):
        b = int(pt[p])
        ks.append(pool.k[layer, b, g].float().cpu().numpy())          # [16][d]
        vs.append(pool.v[layer, b, g].reshape(d, 16).float().cpu().numpy().T)  # [d][16] -> [16][d]
    k = np.concatenate(ks)[:n].astype(np.float64)
    v = np.concatenate(vs)[:n].astype(np.float64)
    return k, v


def pool_kivi(pool, layer: int, r: int, g: int, T: int, d: int):
    """Codes and (scale, zero) of (r, layer, g) from a KIVI pool, in the oracle's logical layout:
    kcodes [T][d], kscale/kzero [ceil(T/32)][d], vcodes [T][d], vscale/vzero [T][d/32]."""
    bits = pool.bits
    pt = pool.page_table[r].cpu().numpy()
    npg = (T + 15) // 16
    kc, vc_, vs, vz = [], [], [], []
    ks, kz = [], []
    for p in range(npg):
        b = int(pt[p])
        kw = pool.k[layer, b, g].cpu().numpy().view(np.uint32).reshape(16, d * bits // 32)
        kc.append(unpack_codes(kw, bits, d))                            # [16][d]
        vw = pool.v[layer, b, g].cpu().numpy().view(np.uint32).reshape(d, 16 * bits // 32)
        vc_.append(unpack_codes(vw, bits, 16).T)                        # [16][d]
        vsz = pool.v_sz[layer, b, g].cpu().numpy().view(np.float16)     # [d/32][2][16]
        vs.append(vsz[:, 0, :].T)
        vz.append(vsz[:, 1, :].T)
        if p % 2 == 0:
            ksz = pool.k_sz[layer, b, g].cpu().numpy().view(np.float16)  # [2][d]
            ks.append(ksz[0])
            kz.append(ksz[1])
    return dict(kcodes=np.concatenate(kc)[:T], vcodes=np.concatenate(vc_)[:T],
                kscale=np.stack(ks), kzero=np.stack(kz),
                vscale=np.concatenate(vs)[:T], vzero=np.concatenate(vz)[:T])


def assert_close(got: np.ndarray, want: np.ndarray, tol, what: str):
    """Every element within the contract and within its gate (a scalar, or one per element as
    ``gate`` returns).  Returns the largest error."""
    diff = np.abs(got - want)
    err = float(diff.max()) if got.size else 0.0
    tol = np.broadcast_to(np.asarray(tol, dtype=np.float64), diff.shape)
    ratio = diff / tol
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape) if got.size else ()
    if ERRLOG:
        with open(ERRLOG, "a") as f:
            f.write(f"{what}\tmax_abs={err:.3e}\tmax_ratio={float(ratio.max()) if got.size else 0.0:.3f}\n")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert err <= TOL_CONTRACT, f"{what}: max-abs error {err:.3e} > contract {TOL_CONTRACT:.0e}"
    assert not got.size or ratio[worst] <= 1.0, (
        f"{what}: error {float(diff[worst]):.3e} > derived gate {float(tol[worst]):.2e} at {worst}")
    return err


def tokens_match(tok_gpu, tok_or, gap_or, z_or, tie=1e-3):
    """Argmax tokens must be equal except at flagged near-tie rows, where the GPU's token must lie
    in the oracle's tie band (its oracle logit within `tie` of the maximum)."""
    tok_gpu = np.asarray(tok_gpu)
    bad = []
    for i in range(len(tok_or)):
        if tok_gpu[i] == tok_or[i]:
            continue
        if gap_or[i] < tie and z_or[i, tok_gpu[i]] >= z_or[i].max() - tie:
            continue
        bad.append((i, int(tok_gpu[i]), int(tok_or[i]), float(gap_or[i])))
    return bad


def ctx_bits_gpu_generator(cfg, r: int, l: int, g: int, n: int, stream: int, p0: int = 0) -> np.ndarray:
    """Context rows [p0, p0 + n) of (request r, layer l, kv head g) as uint16 [n][d], drawn by the
    seeded generator's GPU fill kernel (vcsynth), not by the attention library.  Bit-identical to
    vcsynth.tensors.kctx_bits / vctx_bits (pinned by a test), and much faster at full lengths."""
    from vcsynth import gpu as sg
    from vcsynth import tensors as T
    t = torch.empty((n, cfg.d), dtype=torch.int16, device="cuda")
    sg.fill_normal_bf16(t, [cfg.d, 1], T.ctx_index(cfg, r, l, g, p0, 0), cfg.seed, stream)
    out = t.cpu().numpy().view(np.uint16).copy()
    del t
    return out
