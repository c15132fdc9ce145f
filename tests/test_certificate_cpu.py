"""Host emulation of the encoder's fast scoring and of its certificate (CPU only).

The encode and Lloyd-assign kernels score every codeword approximately on the
matrix cores and only then decide the winner exactly (vq_device.hpp, vq_score.hpp):

  * fp16-split engine: codewords and residuals are split into fp16 hi + lo
    parts; the score ||c||^2 - 2<r, c> is accumulated in fp32 from the exact
    fp16 products -2 hi(c) hi(r), -2 lo(c) hi(r), -2 hi(c) lo(r) and the split
    norm term (||c||^2 2^-sigma as fp16 hi + lo, times the fp16 constant 2^sigma);
  * fp32 engine: 8 products -2 r_k c_k plus ||c||^2, accumulated in fp32.

Per group of GS (1, 2 or 4) consecutive codewords only the minimum score
survives, with the group's lane-local id packed into its low PACK bits; the two
smallest packed values p1 <= p2 decide the candidate group, its members are
resolved with the exact fp32 distance chain, and the winner is accepted when
  p2 - p1 > 1.25 (1 + 2^-20) (c_rr rr + c_w d_w + c_D dmax + 2^-20 + 2^-24 2^sigma + 2^-120),
  c_rr = 38/3 ALPHA + 2^(PACK-22) + 22/3 2^-24,  c_w = 2^-18 + 4.004 ALPHA,
  c_D = 2.2022 (ALPHA + 2^-24) + 2^(PACK-22),
the square-root-free upper bound of
  1.25 (2^-18 d_w + ALPHA (M_w + M_D) + 2^(PACK-22)(rr + dmax) + 2^-21 sqrt(M_D)
        + 2^-24 2^sigma + 2^-120),  M = (2 sqrt(rr) + sqrt(1.001 d))^2
that (a + b)^2 <= (1 + e) a^2 + (1 + 1/e) b^2 (e = 1/3 for M_w, 5/6 for M_D)
and sqrt(M) <= M/8 + 2 give.

The matrix-core accumulation order is not documented, so the emulation sums the
terms in several orders (sequential, reversed, pairwise, by increasing and
decreasing magnitude, random) with a fp32 rounding after every addition, and
once exactly. These tests check, on adversarial inputs (outlier rows with
max|r| = sqrt(cols), codewords at the +-2048 limit, fp16-subnormal split parts,
mixed signs and magnitudes, near and exact ties):
  1. every emulated score is within ALPHA (||r|| + ||c||)^2 + BETA of the exact
     value, BETA = 2^-22.5 (||r|| + ||c||) + 2^(sigma-25) + 2^-121 (fp16-subnormal
     split parts; the norm term's lo part is scaled by 2^-sigma), with at least
     4x margin on ALPHA;
  2. whenever the certificate accepts, the accepted index equals the
     exhaustive fp32 argmin of the oracle (ties to the lowest index).
"""
import math

import numpy as np
import pytest

import oracle

ALPHA = 2.0 ** -16
F32 = np.float32


# ------------------------------------------------------------------ fp16 split
def split16(x):
    """fp32 -> (hi, lo) fp16 halves: hi = RN16(x), lo = RN16(x - hi) (x - hi is
    exact in fp32); numpy's float16 conversion rounds to nearest even and keeps
    subnormals, as the device conversion does."""
    x = np.asarray(x, dtype=F32)
    hi = x.astype(np.float16)
    lo = (x - hi.astype(F32)).astype(np.float16)
    return hi, lo


def norm_terms(C):
    """Per-codeword split norm term as the kernel builds it: n = fp32(||c||^2 in
    fp64), sigma from the codebook's largest n, ns = n 2^-sigma, fp16 hi + lo,
    multiplied on the matrix core by the fp16 constant 2^sigma."""
    n = (C.astype(np.float64) ** 2).sum(axis=1).astype(F32)
    _, e = np.frexp(n.max())
    sg = max(int(e) - 14, 0)
    sig = F32(2.0 ** sg)
    ns = (n / sig).astype(F32)
    nh = ns.astype(np.float16)
    nl = (ns - nh.astype(F32)).astype(np.float16)
    return nh, nl, sig


def sigma_of(C):
    n = (C.astype(np.float64) ** 2).sum(axis=1).astype(F32)
    _, e = np.frexp(n.max())
    return max(int(e) - 14, 0)


def f16x_terms(R, C):
    """All product terms of the fp16-split score, [N, K, 26] fp32 (each exact)."""
    ch, cl = split16(C)
    rh, rl = split16(R)
    a_hi = (ch.astype(F32) * F32(-2)).astype(F32)   # -2 hi(c): exact in fp16 and fp32
    a_lo = (cl.astype(F32) * F32(-2)).astype(F32)
    rh32, rl32 = rh.astype(F32), rl.astype(F32)
    nh, nl, sig = norm_terms(C)
    t0 = a_hi[None, :, :] * rh32[:, None, :]         # first matrix-core product, low half
    t1 = a_lo[None, :, :] * rh32[:, None, :]         # first product, high half
    t2 = a_hi[None, :, :] * rl32[:, None, :]         # second product, low half
    tn = np.stack([nh.astype(F32) * sig, nl.astype(F32) * sig], axis=-1)  # second, high half
    N, K = R.shape[0], C.shape[0]
    first = np.concatenate([t0, t1], axis=2)
    second = np.concatenate([t2, np.broadcast_to(tn[None], (N, K, 2))], axis=2)
    return first.astype(F32), second.astype(F32)


def f32_terms(R, C):
    """fp32 engine: the 8 products -2 r_k c_k, each rounded to fp32 (the
    unfavourable reading of the matrix core's product), and ||c||^2 in fp32."""
    p = (F32(-2) * R[:, None, :]).astype(F32) * C[None, :, :].astype(F32)
    n = (C.astype(np.float64) ** 2).sum(axis=1).astype(F32)
    N = R.shape[0]
    return p.astype(F32), np.broadcast_to(n[None, :, None], (N, C.shape[0], 1)).astype(F32)


def acc_fp32(terms, order, rng=None):
    """Sum along the last axis in fp32 with a rounding after every addition, in
    the given order ('seq', 'rev', 'pair', 'inc', 'dec', 'rand'), or exactly
    rounded once ('exact')."""
    t = terms
    if order == "exact":
        s = np.zeros(t.shape[:-1], dtype=np.float64)
        flat = t.reshape(-1, t.shape[-1]).astype(np.float64)
        out = np.array([math.fsum(row) for row in flat]).reshape(t.shape[:-1])
        return out.astype(F32)
    if order == "rev":
        t = t[..., ::-1]
    elif order in ("inc", "dec"):
        idx = np.argsort(np.abs(t), axis=-1)
        if order == "dec":
            idx = idx[..., ::-1]
        t = np.take_along_axis(t, idx, axis=-1)
    elif order == "rand":
        idx = np.argsort(rng.random(t.shape), axis=-1)
        t = np.take_along_axis(t, idx, axis=-1)
    if order == "pair":
        cur = t
        while cur.shape[-1] > 1:
            if cur.shape[-1] % 2:
                cur = np.concatenate([cur, np.zeros(cur.shape[:-1] + (1,), F32)], axis=-1)
            cur = (cur[..., 0::2] + cur[..., 1::2]).astype(F32)
        return cur[..., 0]
    s = np.zeros(t.shape[:-1], dtype=F32)
    for k in range(t.shape[-1]):
        s = (s + t[..., k]).astype(F32)
    return s


ORDERS = ["seq", "rev", "pair", "inc", "dec", "rand", "exact"]


def scores(R, C, engine, order, rng):
    first, second = f16x_terms(R, C) if engine == "f16x" else f32_terms(R, C)
    s = acc_fp32(first, order, rng)
    s2 = acc_fp32(second, order, rng)
    return (s + s2).astype(F32)


def exact_scores(R, C):
    """||c||^2 - 2<r, c> of the fp32 values, summed exactly (fp64 products of fp32
    values are exact; fsum rounds once)."""
    out = np.empty((R.shape[0], C.shape[0]))
    C64 = C.astype(np.float64)
    cn = [math.fsum(c * c) for c in C64]
    for i, r in enumerate(R.astype(np.float64)):
        for j, c in enumerate(C64):
            out[i, j] = math.fsum(np.concatenate([[cn[j]], -2.0 * r * c]))
    return out


# ------------------------------------------------------------------ inputs
def make_case(kind, rng, K, n):
    """(R [n, 8], C [K, 8]) fp32 of one adversarial class."""
    if kind == "gauss":
        R = rng.standard_normal((n, 8))
        C = rng.standard_normal((K, 8))
    elif kind == "outlier_rows":
        # a normalized row of 7168 (or 2^20) elements with all its energy in one
        # element has max|v| = sqrt(cols)
        R = rng.standard_normal((n, 8)) * 0.01
        big = rng.choice([math.sqrt(7168), 1024.0], n) * rng.choice([-1, 1], n)
        R[np.arange(n), rng.integers(0, 8, n)] = big
        C = rng.standard_normal((K, 8))
        C[: K // 4] *= 30.0
        C[: K // 8, 0] = rng.choice([84.0, -84.0, 1000.0, -1000.0], K // 8)
    elif kind == "codebook_limit":
        R = rng.standard_normal((n, 8)) * 600.0
        C = rng.standard_normal((K, 8)) * 500.0
        C = np.clip(C, -2048, 2048)
        C[: K // 4, rng.integers(0, 8)] = rng.choice([2048.0, -2048.0], K // 4)
    elif kind == "subnormal_split":
        # values whose lo part (x - RN16(x)) is an fp16 subnormal, and values
        # below the fp16 normal range
        base = rng.choice([1.0, -1.0, 0.5, 2.0, 3.0], (K, 8))
        C = base * (1.0 + rng.integers(1, 2 ** 10, (K, 8)) * 2.0 ** -23)
        C[K // 2:] = rng.standard_normal((K - K // 2, 8)) * 2.0 ** -16
        Rb = rng.choice([1.0, -1.0, 0.25], (n, 8))
        R = Rb * (1.0 + rng.integers(1, 2 ** 12, (n, 8)) * 2.0 ** -23)
        R[n // 2:] = rng.standard_normal((n - n // 2, 8)) * 2.0 ** -15
    elif kind == "sigma_mix":
        # a few codewords at the +-2048 limit force the norm term's 2^-sigma
        # scaling (sigma = 12) while the residuals and the other codewords are
        # small: the scaled fp16 lo part then rounds at 2^(sigma-25) absolute
        R = rng.standard_normal((n, 8)) * 0.01
        C = rng.standard_normal((K, 8)) * 0.01
        C[: K // 8, rng.integers(0, 8)] = rng.choice([2048.0, -2048.0], K // 8)
    elif kind == "mixed":
        sc = 10.0 ** rng.uniform(-3, 3, 8)
        R = rng.standard_normal((n, 8)) * sc
        C = rng.standard_normal((K, 8)) * sc
    else:
        raise ValueError(kind)
    return R.astype(F32), C.astype(F32)


def near_tie_case(rng, K, n):
    """Codebooks with cross-group near and exact ties around each residual:
    codewords q and q + K/2 (always in different groups of 4) mirrored through
    r along a random direction (equal real distances, so the fp32 chain and the
    fast scores may order them differently), a copy of one codeword in another
    group and a copy one ulp away."""
    R = rng.standard_normal((n, 8)).astype(F32)
    cases = []
    for i in range(n):
        r = R[i].astype(np.float64)
        C = rng.standard_normal((K, 8))
        for q in range(0, K // 2 - 8):
            u = rng.standard_normal(8)
            u /= np.linalg.norm(u)
            t = rng.uniform(0.05, 1.5)
            C[q] = r + t * u
            C[q + K // 2] = r - t * u
        C = C.astype(F32)
        j = int(rng.integers(0, K // 2 - 8))
        C[K // 2 - 4] = C[j]                                   # exact duplicate, another group
        C[K // 2 - 3] = np.nextafter(C[j], np.float32(np.inf))  # one ulp away
        cases.append(C)
    return R, cases




# ------------------------------------------------------------------ search model
def lane_layout(K, GS):
    """Codeword -> (half h, lane-local group id g) of the 32x32 accumulator layout:
    codeword i = 32 tile + 8 (v // 4) + 4 h + v % 4 for accumulator entry v, and
    groups of GS consecutive entries: g = (16 / GS) tile + v // GS."""
    i = np.arange(K)
    tile, rem = i // 32, i % 32
    q, h, v4 = rem // 8, (rem % 8) // 4, rem % 4
    v = 4 * q + v4
    return h, (16 // GS) * tile + v // GS


def group_first(g, h, GS):
    gpt = 16 // GS
    tile, v0 = g // gpt, GS * (g % gpt)
    return tile * 32 + 8 * (v0 >> 2) + 4 * h + (v0 & 3)


def member(u):
    """Codeword offset of member u from its group's first codeword: groups cover
    consecutive accumulator entries, which map to codewords 8 (v // 4) + 4 h + v % 4."""
    return (u & 3) + 8 * (u >> 2)


def pack_bits(K, GS):
    return int(round(math.log2(16 * (K // 32) // GS)))


def pack(x, g, P):
    b = np.asarray(x, dtype=F32).view(np.uint32)
    return ((b & ~np.uint32((1 << P) - 1)) | np.uint32(g)).view(F32)


def _fma32(a, b, c):
    """fp32 fused multiply-add: the fp64 product-sum of fp32 operands rounded
    once to fp32 (exact but for rare double roundings, each within one ulp)."""
    return F32(float(F32(a)) * float(F32(b)) + float(F32(c)))


def cert_constants(P):
    """The kernel's fp32 constants (rounded from fp64 values raised by 2^-20)."""
    A, E24 = 2.0 ** -16, 2.0 ** -24
    PK = (1 << P) * 2.0 ** -22
    UP = 1.25 * (1.0 + 2.0 ** -20)
    return (F32(UP * (38.0 / 3.0 * A + PK + 22.0 / 3.0 * E24)), F32(UP * (2.0 ** -18 + 4.004 * A)),
            F32(UP * (2.2022 * (A + E24) + PK)), F32(UP * (2.0 ** -20 + 2.0 ** -120)), F32(UP * E24))


def delta_linear(rr, dw, dmax, P, sig, scale=1.25):
    """The kernel's bound in its fp32 operation order; scale replaces the 1.25
    of the bound (the constants are computed for 1.25 and rescaled)."""
    c_rr, c_w, c_d, c_0, c_s = (F32(c * (scale / 1.25)) for c in cert_constants(P))
    delta = _fma32(c_s, sig, c_0)
    delta = _fma32(c_d, dmax, delta)
    delta = _fma32(c_w, dw, delta)
    return _fma32(c_rr, rr, delta)


def delta_sqrt_form(rr, dw, dmax, P, sig):
    """The bound with its square roots, in fp64 (the form the linear one bounds)."""
    mw = (2.0 * math.sqrt(rr) + math.sqrt(1.001 * dw)) ** 2
    md = (2.0 * math.sqrt(rr) + math.sqrt(1.001 * dmax)) ** 2
    return 1.25 * (2.0 ** -18 * dw + 2.0 ** -16 * (mw + md) + (1 << P) * 2.0 ** -22 * (rr + dmax)
                   + 2.0 ** -21 * math.sqrt(md) + 2.0 ** -24 * sig + 2.0 ** -120)


def certified(p1, p2, rr, dw, dmax, P, sig, scale=1.25):
    """The acceptance test in the kernel's fp32 operation order."""
    return F32(F32(p2) - F32(p1)) > delta_linear(rr, dw, dmax, P, sig, scale)


def search(r, C, s, GS, scale=1.25, sig_override=None):
    """The kernel's decision for one vector from its scores s[K] with groups of
    GS codewords: returns (certified, accepted index). scale multiplies the
    bound (1.25 as built); sig_override replaces 2^sigma in it (to show that
    term is needed)."""
    K = C.shape[0]
    P = pack_bits(K, GS)
    h, g = lane_layout(K, GS)
    top = []
    for half in (0, 1):
        sel = np.where(h == half)[0]
        vals = []
        for gid in np.unique(g[sel]):
            members = sel[g[sel] == gid]
            assert len(members) == GS
            assert members.tolist() == [group_first(gid, half, GS) + member(u) for u in range(GS)]
            vals.append(pack(np.min(s[members]), gid, P))
        vals = np.sort(np.array(vals, dtype=F32))
        top.append((vals[0], vals[1]))
    (q0, n0), (q1, n1) = top
    p1 = min(q0, q1)
    p2 = min(max(q0, q1), min(n0, n1))
    hw = 0 if F32(p1).view(np.uint32) == F32(q0).view(np.uint32) else 1
    gid = int(F32(p1).view(np.uint32)) & ((1 << P) - 1)
    j0 = group_first(gid, hw, GS)
    d = [oracle.dist8(r, C[j0 + member(u)]) for u in range(GS)]
    wu = 0
    for u in range(1, GS):
        if d[u] < d[wu]:
            wu = u
    rr = oracle.dist8(r, np.zeros(8, F32))
    sig = F32(2.0 ** sigma_of(C)) if sig_override is None else F32(sig_override)
    ok = certified(F32(p1), F32(p2), F32(rr), F32(d[wu]), F32(max(d)), P, sig, scale)
    return bool(ok), j0 + member(wu)


# ------------------------------------------------------------------ tests
KINDS = ["gauss", "outlier_rows", "codebook_limit", "subnormal_split", "sigma_mix", "mixed"]


@pytest.mark.parametrize("engine", ["f16x", "f32"])
@pytest.mark.parametrize("kind", KINDS)
def test_score_error_within_bound(engine, kind):
    rng = np.random.default_rng(KINDS.index(kind) * 2 + (engine == "f32"))
    R, C = make_case(kind, rng, 64, 48)
    ex = exact_scores(R, C)
    rn = np.sqrt((R.astype(np.float64) ** 2).sum(axis=1))[:, None]
    cn = np.sqrt((C.astype(np.float64) ** 2).sum(axis=1))[None, :]
    quad = ALPHA * (rn + cn) ** 2
    sig_term = 2.0 ** (sigma_of(C) - 25) if engine == "f16x" else 0.0
    beta = 2.0 ** -22.5 * (rn + cn) + sig_term + 2.0 ** -121
    for order in ORDERS:
        s = scores(R, C, engine, order, rng).astype(np.float64)
        err = np.abs(s - ex)
        assert np.all(err <= quad + beta), (order, float(np.max(err - quad - beta)))
        # at least 4x margin on the quadratic term
        assert np.all(err <= 0.25 * quad + beta), (order, float(np.max((err - beta) / quad)))


@pytest.mark.parametrize("gs", [1, 2, 4, 8])
@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
@pytest.mark.parametrize("kind", KINDS)
def test_certificate_never_accepts_a_wrong_index(fmt, kind, gs):
    K = 256 if fmt == "vq3r" else 64
    rng = np.random.default_rng(100 + KINDS.index(kind) * 2 + (fmt == "vq4p") + 1000 * gs)
    R, C = make_case(kind, rng, K, 40)
    n_ok = 0
    for order in ("seq", "dec", "rand"):
        S = scores(R, C, "f16x", order, rng)
        for i in range(R.shape[0]):
            ok, w = search(R[i], C, S[i], gs)
            if ok:
                n_ok += 1
                assert w == oracle.argmin(R[i], C), (order, i)
    if kind in ("gauss", "mixed"):
        # not vacuous: ordinary data is certified almost always
        assert n_ok >= 0.8 * 3 * R.shape[0]
    if kind == "sigma_mix":
        assert n_ok >= 0.3 * 3 * R.shape[0]


@pytest.mark.parametrize("gs", [1, 2, 4, 8])
@pytest.mark.parametrize("fmt", ["vq3r", "vq4p"])
def test_certificate_with_near_and_exact_ties(fmt, gs):
    K = 256 if fmt == "vq3r" else 64
    rng = np.random.default_rng((11 if fmt == "vq3r" else 12) + 100 * gs)
    R, Cs = near_tie_case(rng, K, 30)
    wrong_unguarded = 0
    for i in range(R.shape[0]):
        C = Cs[i]
        want = oracle.argmin(R[i], C)
        for order in ("seq", "rev", "dec", "rand"):
            s = scores(R[i:i + 1], C, "f16x", order, rng)[0]
            ok, w = search(R[i], C, s, gs)
            if ok:
                assert w == want, (i, order)
            # the same decision with no margin at all does go wrong on these
            # inputs, so they exercise the bound
            ok0, w0 = search(R[i], C, s, gs, scale=0.0)
            wrong_unguarded += int(ok0 and w0 != want)
        # r equal to a codeword that has an exact copy in another group: a tie at
        # distance 0, never certified in favour of the higher index
        r_dup = C[K // 2 - 4].astype(F32)
        s = scores(r_dup[None], C, "f16x", "seq", rng)[0]
        ok, w = search(r_dup, C, s, gs)
        assert not ok or w == oracle.argmin(r_dup, C)
    assert wrong_unguarded > 0


def test_sigma_term_is_needed():
    """Without the 2^-24 2^sigma term (the round-to-2^(sigma-25) error of the
    scaled fp16 norm part) the certificate accepts wrong indices on codebooks
    that mix codewords at the +-2048 limit with small ones; with it, none."""
    rng = np.random.default_rng(5)
    wrong_with, wrong_without = 0, 0
    for trial in range(10):
        R, C = make_case("sigma_mix", rng, 256, 20)
        S = scores(R, C, "f16x", "rand", rng)
        for i in range(R.shape[0]):
            want = oracle.argmin(R[i], C)
            ok, w = search(R[i], C, S[i], 4)
            wrong_with += int(ok and w != want)
            ok0, w0 = search(R[i], C, S[i], 4, sig_override=0.0)
            wrong_without += int(ok0 and w0 != want)
    assert wrong_with == 0 and wrong_without > 0


@pytest.mark.parametrize("P", [4, 5, 6, 7])
def test_linear_bound_covers_the_square_root_form(P):
    """The kernel's square-root-free delta (fp32, its operation order) is never
    below the bound it replaces (square roots, fp64), over ||r||^2, d_w <= dmax
    and 2^sigma across many magnitudes, and within 5 % of it on residuals like
    the encoder's."""
    rng = np.random.default_rng(P)
    n = 20000
    rr = 10.0 ** rng.uniform(-12, 8, n)
    dw = rr * 10.0 ** rng.uniform(-8, 2, n)
    dmax = dw * 10.0 ** rng.uniform(0, 3, n)
    sig = 2.0 ** rng.integers(0, 13, n)
    sig[rng.random(n) < 0.3] = 0.0
    for a, b, c, g in zip(rr, dw, dmax, sig):
        a, b, c, g = F32(a), F32(b), F32(c), F32(g)
        lin = float(delta_linear(a, b, c, P, g))
        ref = delta_sqrt_form(float(a), float(b), float(c), P, float(g))
        assert lin >= ref, (a, b, c, g, lin, ref)
    # residuals like the encoder's: d_w about a third of ||r||^2, the winning
    # group's farthest member about 2-4 times it
    for _ in range(2000):
        a = 10.0 ** rng.uniform(-1, 1)
        a, b, c = F32(a), F32(a * rng.uniform(0.25, 0.45)), F32(a * rng.uniform(2.0, 4.0))
        ratio = float(delta_linear(a, b, c, P, F32(1))) / delta_sqrt_form(float(a), float(b), float(c), P, 1.0)
        assert 1.0 <= ratio <= 1.05, ratio
