"""Comparison of the HIP path against the oracle, with the tolerances of the
contract:

* codes identical, except flips to the adjacent code where the oracle's
  argument Z/s sits at a rounding tie (within the float32 error the kernel's
  evaluation order can carry), on at most 1e-5 of the elements (for every
  code format: E4M3, E5M2 and INT8); every differing code is verified;
* alpha and s within 1e-6 relative;
* reconstructions within 1e-3 relative RMS of the oracle's reconstruction,
  and element by element within the float32 error of the kernel's arithmetic
  (plus one output rounding).

Large tensors are compared in full: the oracle runs on contiguous runs of
blocks on several host threads (one oracle call per run; blocks are
independent, so the result is the oracle's on the whole tensor).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import synth

FLIP_RATE = 1e-5
SCALAR_RTOL = 1e-6
RECON_RTOL = 1e-3
QMAX = 448.0
QMAX_OF = {"e4m3": 448.0, "e5m2": 57344.0, "int8": 127.0}
U32 = 2.0 ** -24          # float32 unit roundoff

# Owner step, per case: the rate of tie flips depends on the data, since its
# codes are decided on a float32 sum of decoded FP8 payloads, few-bit values
# whose rotated sums land on rounding ties far more often than bf16 data do
# in some small cases (2.7-5.4e-5 seen for two payloads without an own
# partial), and exactly on them in clusters (three exact ties in one block
# of 512).  The flips at inexact ties of one case are held to a Poisson
# bound of 1e-4; flips at exact ties are not capped per case.  The session
# total of all flips is held to the contract's 1e-5 like every other kind,
# and every flip is verified against the float32 bound of the sum.
OWNER_FLIP_RATE = 1e-4

#: Rate bound of each kind of comparison over the session.  "compress": the
#: operator's sender side, one rotation of exact bf16 inputs; "roundtrip":
#: the fidelity round trips (blocks explained by adjacent-code changes);
#: "owner": the owner step.
RATE_OF = {"compress": FLIP_RATE, "roundtrip": FLIP_RATE, "owner": FLIP_RATE}

# Flips and elements over every comparison of the session, per kind and code
# format: {(kind, fmt): [flips, elements]}.  A case may show a few
# tie-verified flips on its own (Poisson bound below); the session total of
# each kind must stay within its rate (checked when the session ends, in
# conftest.py, after every test file).
TOTALS: dict = {}


def tally(kind: str, fmt: str, flips: int, n: int) -> None:
    t = TOTALS.setdefault((kind, fmt), [0, 0])
    t[0] += int(flips)
    t[1] += int(n)


def session_report():
    """[(kind, fmt, flips, elements, rate bound, within bound)] of the session."""
    rows = []
    for (kind, fmt), (f, n) in sorted(TOTALS.items()):
        rate = RATE_OF[kind]
        rows.append((kind, fmt, f, n, rate, f <= rate * max(n, 1)))
    return rows


def session_check():
    """(report lines, every total within its rate) for the session's code
    comparisons."""
    rows = session_report()
    lines = []
    for kind, fmt, f, n, rate, ok in rows:
        lines.append(f"code flips [{kind} {fmt}]: {f} in {n} elements "
                     f"({f / max(n, 1):.2e}; bound {rate:g})" + ("" if ok else "  EXCEEDED"))
    ok = all(r[-1] for r in rows)
    if not ok:
        lines.append("FAILED: a session total of code flips exceeds its rate")
    return lines, ok


def threads() -> int:
    """Host threads for the oracle (the CPU share of one GPU: at most 16)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


#: Largest run of blocks handled by one oracle call or comparison step, in
#: blocks: small runs keep each step's temporaries (a few MB) reusable from
#: the heap instead of freshly mapped pages.
RUN_BLOCKS = 4096


def block_runs(m: int, nthreads: int | None = None, run: int | None = None):
    """Contiguous runs [lo, hi) of blocks covering 0..m: at most `run`
    blocks each, and at least one per thread when m allows."""
    nt = nthreads or threads()
    size = max(1, min(run or RUN_BLOCKS, -(-m // nt)))
    return [(lo, min(lo + size, m)) for lo in range(0, m, size)]


def run_blocks(fn, m: int, nthreads: int | None = None):
    """fn(lo, hi) over runs of blocks, on a thread pool (each oracle call is
    one C call, which releases the GIL).  Returns the list of results."""
    runs = block_runs(m, nthreads)
    if len(runs) == 1:
        return [fn(*runs[0])]
    with ThreadPoolExecutor(nthreads or threads()) as pool:
        return list(pool.map(lambda r: fn(*r), runs))


def oracle_compress(x_bits, B, tau=1.0, fmt="e4m3"):
    """oracle.compress of a flattened tensor, runs of blocks on host threads."""
    x = np.ascontiguousarray(x_bits).reshape(-1)
    m = x.size // B
    codes = np.empty(x.size, np.uint8)
    alpha = np.empty(m, np.float32)
    scale = np.empty(m, np.float32)

    def part(lo, hi):
        c, a, s = oracle.compress(x[lo * B:hi * B], B, tau, fmt=fmt)
        codes[lo * B:hi * B] = c.reshape(-1)
        alpha[lo:hi] = a
        scale[lo:hi] = s
    run_blocks(part, m)
    return codes, alpha, scale


def oracle_decompress(codes, alpha, scale, B, fmt="e4m3"):
    """oracle.decompress (bf16 bit patterns) of a flattened payload, runs of
    blocks on host threads."""
    c = np.ascontiguousarray(codes).reshape(-1)
    m = c.size // B
    y = np.empty(c.size, np.uint16)

    def part(lo, hi):
        y[lo * B:hi * B] = oracle.decompress(c[lo * B:hi * B], alpha[lo:hi], scale[lo:hi], B,
                                             fmt=fmt)
    run_blocks(part, m)
    return y


def oracle_accumulate(codes, alpha, scale, B, acc, fmt="e4m3"):
    """oracle.decompress_accumulate of a flattened payload into acc (float32,
    in place), runs of blocks on host threads."""
    c = np.ascontiguousarray(codes).reshape(-1)
    assert acc.dtype == np.float32 and acc.flags["C_CONTIGUOUS"] and acc.size == c.size
    a = acc.reshape(-1)

    def part(lo, hi):
        oracle.decompress_accumulate(c[lo * B:hi * B], alpha[lo:hi], scale[lo:hi], B,
                                     a[lo * B:hi * B], fmt=fmt)
    run_blocks(part, c.size // B)
    return acc


def bf16_rel_rms(y_bits, ref_bits) -> float:
    """Relative RMS of one bf16 tensor against another (runs on host threads)."""
    a = np.ascontiguousarray(y_bits).reshape(-1)
    b = np.ascontiguousarray(ref_bits).reshape(-1)

    def part(lo, hi):
        ya = synth.bits_to_f32(a[lo:hi]).astype(np.float64)
        yb = synth.bits_to_f32(b[lo:hi]).astype(np.float64)
        d = ya - yb
        return float(np.dot(d, d)), float(np.dot(yb, yb))
    res = run_blocks(part, a.size)
    num, den = sum(r[0] for r in res), sum(r[1] for r in res)
    return math.sqrt(num / den) if den > 0 else math.sqrt(num)


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


def compare_compress(x_bits, B, codes, alpha, scale, tau=1.0, fmt="e4m3", kind="compress"):
    """Check the GPU's (codes, alpha, scale) of x_bits against the oracle;
    every differing code is verified to be one the kernel's float32
    evaluation can give.  Returns a dict of statistics; raises
    AssertionError on a violation."""
    x_bits = np.ascontiguousarray(x_bits).reshape(-1)
    codes = np.ascontiguousarray(codes).reshape(-1)
    o_codes, o_alpha, o_scale = oracle_compress(x_bits, B, tau, fmt)
    bad = np.nonzero(codes != o_codes)[0]
    n = x_bits.size
    tally(kind, fmt, bad.size, n)
    assert bad.size <= allowed_flips(n), \
        f"{bad.size} code mismatches in {n} elements (allowed {allowed_flips(n):.1f})"
    for i in bad:
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
    (element-wise, one bf16 rounding plus the kernel's float32 error).
    Runs of blocks on host threads."""
    y_all = np.ascontiguousarray(y_bits).reshape(-1)
    c_all = np.ascontiguousarray(o_codes).reshape(-1)
    m = c_all.size // B

    def part(lo, hi):
        sl = slice(lo * B, hi * B)
        c, a, s = c_all[sl], o_alpha[lo:hi], o_scale[lo:hi]
        ref = oracle.reconstruct_f64(c, a, s, B, fmt=fmt)
        ref_bf16 = synth.bits_to_f32(oracle.decompress(c, a, s, B, fmt=fmt)).astype(np.float64)
        y = synth.bits_to_f32(y_all[sl]).astype(np.float64)
        # Element-wise: within one bf16 step of the exact value, plus the
        # kernel's float32 rounding relative to the block's largest output.
        blk_max = np.repeat(np.max(np.abs(ref.reshape(-1, B)), axis=1), B)
        # (bf16 subnormals, below 2^-126, are spaced 2^-133 apart.)
        tol = 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * blk_max + 2.0 ** -133
        worst = float(np.max(np.abs(y - ref) - tol))
        d = y - ref_bf16
        return worst, float(np.dot(d, d)), float(np.dot(ref_bf16, ref_bf16))

    res = run_blocks(part, m)
    worst = max(r[0] for r in res)
    num, den = sum(r[1] for r in res), sum(r[2] for r in res)
    r = math.sqrt(num / den) if den > 0 else math.sqrt(num)
    assert r <= RECON_RTOL, f"decompress rel RMS {r:.3g}"
    assert worst <= 0, f"decompress element error exceeds tolerance by {worst:.3g}"
    return {"rel_rms": r}


def compare_accumulate(got_acc, acc0, payloads, B, fmt="e4m3", out=None):
    """GPU float32 accumulator after acc0 += G'_p for the payloads, in order
    (each payload the oracle's own codes, alpha and s, so that the kernel is
    checked alone), against the oracle's (decompress_accumulate per payload),
    element by element.  Per payload the kernel's G'_p carries the float32
    error of an inverse FWHT of the decoded codes d_p (at most log2(B)
    roundings of partial sums bounded by |d_p|_1, times the factor
    f_p = s_p / (sqrt(B) alpha_p)) and of the factor and product (a few units
    of G'_p); the accumulator adds one rounding on each side:
        |acc - acc_oracle| <= sum_p 2^-23 (log2(B) |f_p| |d_p|_1 + 4 |G'_p|
                                           + 2 (|acc0| + sum_{q<=p} |G'_q|)),
    twice the first-order bound, plus a few subnormal steps.  Also the
    relative RMS against the oracle (<= 1e-6).  Runs of blocks on host
    threads.  out (float32, optional) receives the oracle's accumulator."""
    got = np.ascontiguousarray(got_acc).reshape(-1)
    a0 = np.ascontiguousarray(acc0, dtype=np.float32).reshape(-1)
    pays = [(np.ascontiguousarray(c).reshape(-1), np.asarray(a, np.float32).reshape(-1),
             np.asarray(s, np.float32).reshape(-1)) for c, a, s in payloads]
    m = got.size // B
    log_b = math.log2(B)

    def part(lo, hi):
        sl = slice(lo * B, hi * B)
        ref = a0[sl].copy()
        run = np.abs(ref).astype(np.float64)
        tol = np.zeros(ref.size)
        for c, a, s in pays:
            cc, aa, ss = c[sl], a[lo:hi], s[lo:hi]
            oracle.decompress_accumulate(cc, aa, ss, B, ref, fmt=fmt)
            g = np.abs(oracle.reconstruct_f64(cc, aa, ss, B, fmt=fmt))
            with np.errstate(divide="ignore", invalid="ignore"):
                f = np.where(aa != 0, ss.astype(np.float64) / (math.sqrt(B) * aa), 0.0)
            d1 = np.sum(np.abs(oracle.decode(cc, fmt)).reshape(-1, B), axis=1)
            run += g
            tol += 2.0 ** -23 * (log_b * np.repeat(np.abs(f) * d1, B) + 4 * g + 2 * run)
        tol += len(pays) * 4 * 2.0 ** -149
        if out is not None:
            out[sl] = ref
        diff = np.abs(got[sl].astype(np.float64) - ref)
        worst = float(np.max(diff - tol)) if diff.size else 0.0
        e = got[sl].astype(np.float64) - ref
        blk = np.repeat(np.max(run.reshape(-1, B), axis=1), B)
        ratio = float(np.max(diff / np.maximum(blk, 2.0 ** -149))) if diff.size else 0.0
        return worst, float(np.dot(e, e)), float(np.dot(ref.astype(np.float64), ref)), ratio

    res = run_blocks(part, m)
    worst = max(r[0] for r in res)
    num, den = sum(r[1] for r in res), sum(r[2] for r in res)
    r = math.sqrt(num / den) if den > 0 else math.sqrt(num)
    assert worst <= 0, f"accumulator element error exceeds its float32 bound by {worst:.3g}"
    assert r <= 1e-6, f"accumulate rel RMS {r:.3g}"
    return {"rel_rms": r, "max_err_over_block_magnitude": max(q[3] for q in res)}


#: Round-trip variants that rotate the block (their codes live in the
#: rotated domain).
ROTATING = {"taco", "ash", "hadamard"}
_CODE_VALUES = {}


def code_values(fmt: str) -> np.ndarray:
    """The distinct finite values of a format's codes, ascending."""
    if fmt not in _CODE_VALUES:
        v = oracle.decode(np.arange(256, dtype=np.uint8), fmt)
        _CODE_VALUES[fmt] = np.unique(v[np.isfinite(v)])
    return _CODE_VALUES[fmt]


def tie_changes(v, bound, fmt: str):
    """[(j, change)]: the elements j of a block whose code argument v[j]
    (exact, as the oracle defines it) lies within bound[j] of a rounding
    midpoint between the oracle's code value there and a neighbouring code
    value, with the change of code value (neighbour minus the oracle's) that
    a float32 evaluation on the other side of that midpoint gives."""
    vals = code_values(fmt)
    v = np.asarray(v, np.float64)
    o = oracle.decode(oracle.encode(v.astype(np.float32), fmt), fmt).astype(np.float64)
    i = np.searchsorted(vals, o)
    out = []
    for side in (-1, 1):
        q = i + side
        ok = (q >= 0) & (q < vals.size)
        nb = vals[np.clip(q, 0, vals.size - 1)]
        hit = ok & (np.abs(v - 0.5 * (o + nb)) <= bound)
        out += [(int(j), float(nb[j] - o[j])) for j in np.nonzero(hit)[0]]
    return out


def code_arguments(x_block, B, variant, fmt, tau, tensor_max):
    """(v, bound) of one block: each element's code argument as the oracle
    defines it (in double) and a bound on the float32 error of the kernel's
    evaluation of it.  The rotation accumulates at most log2(B) roundings of
    partial sums bounded by sum|x|; quotients and products add a few units
    of v."""
    qmax = QMAX_OF[fmt]
    xs = synth.bits_to_f32(x_block).astype(np.float64)
    if variant == "direct":
        return xs, np.zeros(B)
    if variant in ("ds", "tensor"):
        m = np.max(np.abs(xs)) if variant == "ds" else tensor_max
        v = xs * qmax / m if m > 0 else np.zeros(B)
        return v, 4 * U32 * np.abs(v)
    R = oracle.fwht(xs)
    ferr = np.log2(B) * U32 * np.sum(np.abs(xs))
    if variant == "taco":
        m = np.max(np.abs(R))
        v = qmax * R / m if m > 0 else np.zeros(B)
        return v, (qmax * ferr / m if m > 0 else 0.0) + 4 * U32 * np.abs(v)
    if variant == "hadamard":
        v = R / math.sqrt(B)
        return v, ferr / math.sqrt(B) + 4 * U32 * np.abs(v)
    alpha, _, z = oracle.ash_block(x_block, B, tau)            # "ash"
    return z, alpha * ferr / math.sqrt(B) + 8 * U32 * np.abs(z)


def _code_factor(x_block, B, variant, fmt, tau, tensor_delta):
    """c such that the oracle's round trip of a block is c * decode(q) in the
    code domain (H x' / sqrt(B) for the rotating variants, x' itself for the
    others): s/alpha (the operator), 1/alpha (ASH alone), s (DS alone), the
    tensor step, or 1 (direct cast, plain rotation)."""
    if variant in ("direct", "hadamard"):
        return 1.0
    if variant == "tensor":
        return tensor_delta
    if variant == "ds":
        m = float(np.max(np.abs(synth.bits_to_f32(x_block).astype(np.float64))))
        return float(np.float32(m / QMAX_OF[fmt]))
    _, a, sc = oracle.compress(x_block, B, tau, fmt=fmt)
    a, sc = float(a[0]), float(sc[0])
    if a == 0.0:
        return 0.0
    return 1.0 / a if variant == "ash" else sc / a


def compare_roundtrip(y_bits, x_bits, B, variant, fmt="e4m3", tau=1.0, xo=None):
    """GPU bf16 output of a fidelity round trip (taco_roundtrip) against the
    oracle's (roundtrip_variant), element by element.  Where no code
    differs, an element is within one bf16 rounding of the oracle's value
    plus the float32 error of the kernel's arithmetic relative to the
    block's largest value.  The round trip does not return its codes, so a
    tie flip shows only in its output, and one flip of a rotating variant
    moves every element of the block by about the code step over sqrt(B):
    below the bf16 noise of the other elements in the code domain, yet
    enough to take an element near zero past its bound.  A block beyond the
    bound must therefore be explained by flips at rounding ties: the
    elements whose code argument lies within the kernel's float32 error
    bound of a midpoint between the oracle's code and a neighbouring one
    are found (tie_changes), and some set of them (of the six whose flip
    alone best matches the difference), each moved to the other code of its
    tie, must bring the whole block within the element bound.  In the code domain (H x'/sqrt(B) for
    the rotating variants, x' itself for the others) the oracle's block is
    c * decode(q), so a flip at j changes it by c times the code step at j.
    The number of such blocks counts as flips against the rate.  Also the
    relative RMS (1e-3) against the oracle's output with those explained
    flips applied: with few, coarse codes one legitimate flip moves a small
    tensor's RMS by more than that (ASH alone in INT8 maps a block to values
    of RMS about 1, so one code step is a few percent of the block)."""
    import itertools
    y = synth.bits_to_f32(np.ascontiguousarray(y_bits).reshape(-1)).astype(np.float64)
    xb_all = np.ascontiguousarray(x_bits).reshape(-1)
    if xo is None:
        xo = oracle.roundtrip_variant(xb_all, B, variant, fmt, tau).reshape(-1)
    n = y.size
    xo2 = xo.reshape(-1, B)
    blk = np.max(np.abs(xo2), axis=1, keepdims=True)
    tol = (2.0 ** -8 * np.abs(xo2) + 2.0 ** -16 * blk + 2.0 ** -133)
    err = (y - xo).reshape(-1, B)
    over = np.nonzero(np.any(np.abs(err) > tol, axis=1))[0]
    tally("roundtrip", fmt, over.size, n)
    assert over.size <= allowed_flips(n), \
        f"{variant}/{fmt}: {over.size} blocks beyond the element bound in {n} elements"
    rot = variant in ROTATING
    tmax = delta = 0.0
    flipped = xo2.copy()
    if variant == "tensor" and over.size:
        tmax = float(np.max(np.abs(synth.bits_to_f32(xb_all).astype(np.float64))))
        delta = float(np.float32(tmax / QMAX_OF[fmt]))
    for k in over:
        e = err[k]
        xblock = xb_all[k * B:(k + 1) * B]
        c = _code_factor(xblock, B, variant, fmt, tau, delta)
        assert c != 0.0, f"{variant}/{fmt} block {k}: an all-zero block differs"
        v, vb = code_arguments(xblock, B, variant, fmt, tau, tmax)
        dom = oracle.fwht(e) / math.sqrt(B) if rot else e
        # Ties ranked by how much their flip alone lowers the difference in
        # the code domain; the six best are tried in every combination.
        ties = sorted(((abs(dom[j]) - abs(dom[j] - d * c), j, d * c)
                       for j, d in tie_changes(v, vb, fmt)), reverse=True)[:6]
        least = float(np.max(np.abs(e) - tol[k]))
        explained = False
        for size in range(1, len(ties) + 1):
            for sub in itertools.combinations(ties, size):
                change = np.zeros(B)
                for _, j, dc in sub:
                    change[j] += dc
                back = oracle.fwht(change) / math.sqrt(B) if rot else change
                # The kernel rounds its own value (the oracle's plus the
                # change) to bf16: the bound follows the larger magnitude.
                moved = np.abs(xo2[k] + back)
                t = np.maximum(tol[k], 2.0 ** -8 * moved + 2.0 ** -16 * np.max(moved) + 2.0 ** -133)
                excess = float(np.max(np.abs(e - back) - t * (1 + 1e-9)))
                least = min(least, excess)
                if excess <= 0:
                    explained = True
                    flipped[k] = xo2[k] + back
                    break
            if explained:
                break
        assert explained, (f"{variant}/{fmt} block {k}: error beyond the bound that no flips at "
                           f"its {len(ties)} rounding ties explain (least remaining excess "
                           f"{least:.3g})")
    ref = synth.bits_to_f32(oracle.double_to_bf16(flipped.reshape(-1))).astype(np.float64)
    r = rel_rms(y, ref)
    assert r <= RECON_RTOL, f"{variant}/{fmt}: reconstruction rel RMS {r:.3g}"
    return {"rel_rms": r, "flip_blocks": int(over.size)}


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


def oracle_reduce_compress(own_bits, payloads, B, tau=1.0, fmt="e4m3"):
    """oracle.reduce_compress of flattened tensors, runs of blocks on host
    threads.  own_bits: bf16 bit patterns or None; payloads: list of
    (codes, alpha, scale)."""
    pays = [(np.ascontiguousarray(c).reshape(-1), np.asarray(a, np.float32).reshape(-1),
             np.asarray(sc, np.float32).reshape(-1)) for c, a, sc in payloads]
    own = None if own_bits is None else np.ascontiguousarray(own_bits).reshape(-1)
    n = own.size if own is not None else pays[0][0].size
    m = n // B
    codes = np.empty(n, np.uint8)
    alpha = np.empty(m, np.float32)
    scale = np.empty(m, np.float32)

    def part(lo, hi):
        sl = slice(lo * B, hi * B)
        c, a, sc = oracle.reduce_compress(None if own is None else own[sl],
                                          [(pc[sl], pa[lo:hi], ps[lo:hi]) for pc, pa, ps in pays],
                                          B, tau, fmt=fmt)
        codes[sl] = c.reshape(-1)
        alpha[lo:hi] = a
        scale[lo:hi] = sc
    run_blocks(part, m)
    return codes, alpha, scale


def compare_reduce(own_bits, payloads, B, codes, alpha, scale, tau=1.0, fmt="e4m3",
                   cancelling=False):
    """Check the GPU owner step (codes, alpha, scale of own + sum of payload
    reconstructions) against the oracle.  The kernel decides the codes on a
    float32 rotated-domain sum of the own partial and every payload, the
    oracle on the exact sum: every code that differs must be the code of
    some value within the float32 error of that sum (rotated_sum_error,
    plus the oracle's own double rounding) around the exact value.  At a
    tie that is the adjacent code; near zero, where a format's codes are
    finer than that error (E5M2's reach far below it), it may be a few codes
    away.  A sum of a few decoded payloads can sit exactly on a midpoint
    between two codes: both are then equally near the exact sum, the
    oracle's choice is round-half-even's and the kernel's follows the sign
    of its float32 error, so such flips come in clusters of exact ties.  The
    flips at inexact ties are capped at OWNER_FLIP_RATE per case; every flip
    is counted in the session total.  The
    exact sum and its bound are formed only for the blocks that hold a
    differing code, so whole tensors of any size can be compared.

    cancelling: the sum cancels to a small fraction of its terms (own = x
    plus a payload compressed from -x leaves only the quantisation error).
    The rotated sum is then known only to that float32 error relative to a
    much smaller result, so the flip-rate and scalar tolerances of the
    operator cannot hold; instead every flip must be adjacent and inside the
    bound, and alpha and s must agree within the relative error that the
    same bound implies for the block's energy (Parseval) and maximum."""
    codes = np.ascontiguousarray(codes).reshape(-1)
    qmax = QMAX_OF[fmt]
    o_codes, o_alpha, o_scale = oracle_reduce_compress(own_bits, payloads, B, tau, fmt)
    n = o_codes.size
    M = n // B
    bad = np.nonzero(codes != o_codes)[0]
    if not cancelling:
        tally("owner", fmt, bad.size, n)
        # A coarse cap first, so that a broken result is not verified code by
        # code over the whole tensor; the per-case cap follows the checks.
        coarse = allowed_flips(n, 1e-3)
        assert bad.size <= coarse, \
            f"{bad.size} code mismatches in {n} elements (coarse cap {coarse:.1f})"
    # The blocks to examine: those with a differing code (every block when
    # the scalars are held to the bound as well).
    sel = np.arange(M) if cancelling else np.unique(bad // B)
    terms = len(payloads) + (own_bits is not None)
    x = e = None
    if sel.size:
        own_sel = None
        x = np.zeros((sel.size, B))
        if own_bits is not None:
            own_sel = np.ascontiguousarray(np.asarray(own_bits).reshape(M, B)[sel])
            x += synth.bits_to_f32(own_sel).astype(np.float64)
        pays_sel = []
        for c, a, sc in payloads:
            ps = (np.ascontiguousarray(np.asarray(c).reshape(M, B)[sel]),
                  np.asarray(a, np.float32).reshape(-1)[sel], np.asarray(sc, np.float32).reshape(-1)[sel])
            pays_sel.append(ps)
            x += oracle.reconstruct_f64(*ps, B, fmt=fmt).reshape(sel.size, B)
        e = rotated_sum_error(own_sel, pays_sel, B, fmt).reshape(sel.size, B)
        # The oracle's own rounding: it reconstructs every payload in double
        # and rotates the sum again, which leaves noise of order 2^-52 times
        # the block's L1 norm (enough to give an exact zero a sign).
        l1 = np.sum(np.abs(x), axis=1, keepdims=True)
        e = e + 2.0 ** -52 * (np.log2(B) + 2 * terms + 2) * l1
    pos = {int(k): q for q, k in enumerate(sel)}
    exact = 0
    for i in bad:
        k, j = divmod(int(i), B)
        q = pos[k]
        r = oracle.fwht(x[q])
        m = np.max(np.abs(r))
        v = qmax * r[j] / m
        cg, co = int(codes[i]), int(o_codes[i])
        bound = qmax * e[q, j] / m + 4 * U32 * abs(v)
        assert reachable(cg, v, bound, fmt), \
            f"element {i}: code {cg:#x} (oracle {co:#x}) is no code of a value within {bound:.3g} of {v!r}"
        dg, do = oracle.decode(np.array([cg, co], np.uint8), fmt)
        exact += abs(v - 0.5 * (dg + do)) <= 1e-12 * abs(v)
    if not cancelling:
        allowed = allowed_flips(n, OWNER_FLIP_RATE)
        assert bad.size - exact <= allowed, \
            (f"{bad.size} code mismatches in {n} elements, {exact} of them at exact ties "
             f"(allowed {allowed:.1f} others)")
    ea = max_rel(alpha, o_alpha)
    es = max_rel(scale, o_scale)
    if cancelling:
        R = np.stack([oracle.fwht(x[q]) for q in range(M)])
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


def compare_accumulate_n(got_acc, acc0, payloads, B, fmt="e4m3"):
    """GPU float32 accumulator after one multi-payload accumulate
    (acc0 += sum_p G'_p in one pass) against the oracle's
    (decompress_accumulate_n: the sum in double, rounded once), element by
    element and by relative RMS (<= 1e-6).  The kernel sums the payloads in
    the rotated domain, S = sum_p c_p d_p with c_p = sqrt(B) s_p / alpha_p
    (each product nearly exact, each of the P additions one rounding), then
    applies one inverse FWHT and the exact 1/B; so per element
        |err| <= 2^-24 ((P + 2 + log2 B) sum_p |s_p / alpha_p| |d_p|_1 / sqrt(B))
                 + 2^-23 (|acc0| + sum_p |G'_p|),
    which is held with a factor of 2.  Runs of blocks on host threads."""
    got = np.ascontiguousarray(got_acc).reshape(-1)
    a0 = np.ascontiguousarray(acc0, dtype=np.float32).reshape(-1)
    pays = [(np.ascontiguousarray(c).reshape(-1), np.asarray(a, np.float32).reshape(-1),
             np.asarray(sc, np.float32).reshape(-1)) for c, a, sc in payloads]
    P = len(pays)
    log_b = math.log2(B)

    def part(lo, hi):
        sl = slice(lo * B, hi * B)
        sub = [(c[sl], a[lo:hi], sc[lo:hi]) for c, a, sc in pays]
        ref = oracle.decompress_accumulate_n(sub, B, a0[sl].copy(), fmt)
        mag = np.abs(a0[sl]).astype(np.float64)
        t_blk = np.zeros(hi - lo)
        for c, a, sc in sub:
            mag += np.abs(oracle.reconstruct_f64(c, a, sc, B, fmt=fmt))
            with np.errstate(divide="ignore", invalid="ignore"):
                f = np.where(a != 0, sc.astype(np.float64) / a, 0.0)
            t_blk += np.abs(f) * np.sum(np.abs(oracle.decode(c, fmt)).reshape(-1, B), axis=1)
        tol = 2 * (2.0 ** -24 * (P + 2 + log_b) * np.repeat(t_blk, B) / math.sqrt(B)
                   + 2.0 ** -23 * mag) + 4 * P * 2.0 ** -149
        d = got[sl].astype(np.float64) - ref
        blk = np.repeat(np.max(mag.reshape(-1, B), axis=1), B)
        ratio = np.abs(d) / np.maximum(blk, 2.0 ** -149)
        return (float(np.max(np.abs(d) - tol)), float(np.dot(d, d)),
                float(np.dot(ref.astype(np.float64), ref)), float(np.max(ratio)))

    res = run_blocks(part, got.size // B)
    worst = max(r[0] for r in res)
    num, den = sum(r[1] for r in res), sum(r[2] for r in res)
    r = math.sqrt(num / den) if den > 0 else math.sqrt(num)
    assert worst <= 0, f"multi-payload accumulator beyond its float32 bound by {worst:.3g}"
    assert r <= 1e-6, f"multi-payload accumulate rel RMS {r:.3g}"
    return {"rel_rms": r, "max_err_over_block_magnitude": max(q[3] for q in res)}
