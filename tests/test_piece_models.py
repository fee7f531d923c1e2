"""CPU pins of the two ways the library forms an fp32 product from 2-byte matrix-core pieces, against
the mathematics (no GPU, no library code):

- three bfloat16 pieces, x = x0 + x1 + x2 with x0 = bf16(x), x1 = bf16(x - x0), x2 = bf16(x - x0 - x1):
  the cut is exact for fp32 values of ordinary magnitude, so the six piece products that keep
  i + j <= 2 leave out only terms below 2^-23 |x||y|;
- two binary16 pieces after a power of two per block, x' = 2^e x with 2^13 <= 2^e max|x| < 2^14,
  x0 = f16(x'), x1 = f16(x' - x0): x' - x0 - x1 is at most 2^-9 (2^-22 of the block's largest
  element), and a product formed as x0 y0 + x0 y1 + x1 y0 with fp32 accumulation is as accurate,
  measured against fp64, as the fp32 matrix cores' product of the fp32 operands.

The accumulation model: k-slices as deep as the MFMA (16 for the 32x32x16 binary16 MFMA, 2 for the
32x32x2 fp32 one), each slice's sum of exact products rounded to fp32 once and added to an fp32
accumulator (slice by slice, and within a slice x0 y0, then x0 y1, then x1 y0)."""
import numpy as np
import torch

import dash_inputs as di


def top_exp(m):
    """e with 2^13 <= 2^e m < 2^14 (m > 0)."""
    _, e = np.frexp(np.float32(m))
    return 14 - int(e)


def pieces16(x, e):
    xs = np.ldexp(x.astype(np.float32), e).astype(np.float32)
    x0 = xs.astype(np.float16)
    x1 = (xs - x0.astype(np.float32)).astype(np.float16)  # the difference is exact in fp32
    return xs, x0.astype(np.float64), x1.astype(np.float64)


def accumulate(terms, K, BK=16):
    """fp32 accumulator over k-slices; terms(lo, hi) yields the exact slice sums to add in order."""
    acc = None
    for lo in range(0, K, BK):
        for t in terms(lo, lo + BK):
            t32 = t.astype(np.float32)
            acc = t32 if acc is None else (acc + t32).astype(np.float32)
    return acc.astype(np.float64)


def rel(P, R):
    return float(np.linalg.norm(P - R) / np.linalg.norm(R))


def test_bfloat16_three_piece_cut_is_exact():
    for seed, scale in ((801, 1.0), (802, 1e-20), (803, 1e20)):
        x = torch.from_numpy(di.gaussian((4096,), seed) * np.float32(scale))
        x0 = x.to(torch.bfloat16).float()
        r1 = x - x0
        x1 = r1.to(torch.bfloat16).float()
        r2 = r1 - x1
        x2 = r2.to(torch.bfloat16).float()
        assert torch.equal(x2, r2)                 # the last piece holds the rest exactly
        assert torch.equal(x0 + x1 + x2, x)        # so the cut is exact
        # the dropped products x1 y2, x2 y1, x2 y2 are below 2^-23 |x||y|
        y = x.flip(0)
        y0 = y.to(torch.bfloat16).float()
        y1 = (y - y0).to(torch.bfloat16).float()
        y2 = y - y0 - y1
        dropped = (x1.double() * y2.double() + x2.double() * y1.double() + x2.double() * y2.double()).abs()
        assert torch.all(dropped <= 2.0 ** -23 * (x.double() * y.double()).abs())


def test_binary16_two_piece_cut_bound():
    g = di.rng(811)
    for decades in (0, 6):
        x = di.gaussian((256, 256), 812 + decades)
        x = (x * np.exp(g.uniform(-decades * np.log(10), 0, (256, 1)))).astype(np.float32)
        e = top_exp(np.abs(x).max())
        xs, x0, x1 = pieces16(x, e)
        m = np.abs(xs).max()
        assert 2.0 ** 13 <= m < 2.0 ** 14
        err = np.abs(xs.astype(np.float64) - x0 - x1)
        assert err.max() <= 2.0 ** -9                     # absolute, in units of the scaled block
        assert err.max() <= 2.0 ** -22 * m


def test_binary16_three_products_as_accurate_as_fp32():
    B = 256
    for seed, decades in ((821, 0), (822, 4)):
        X = di.gaussian((B, B), seed)
        Y = di.gaussian((B, B), seed + 100)
        d = np.exp(di.rng(seed + 200).uniform(-decades * np.log(10), 0, B)).astype(np.float32)
        X = (X * d[None, :]).astype(np.float32)    # columns of X over several decades
        exact = X.astype(np.float64) @ Y.astype(np.float64)
        Xd, Yd = X.astype(np.float64), Y.astype(np.float64)
        fp32 = accumulate(lambda lo, hi: [Xd[:, lo:hi] @ Yd[lo:hi, :]], B, BK=2)  # the fp32 MFMA's depth
        ex, ey = top_exp(np.abs(X).max()), top_exp(np.abs(Y).max())
        _, x0, x1 = pieces16(X, ex)
        _, y0, y1 = pieces16(Y, ey)
        h2 = accumulate(lambda lo, hi: [x0[:, lo:hi] @ y0[lo:hi, :], x0[:, lo:hi] @ y1[lo:hi, :],
                                        x1[:, lo:hi] @ y0[lo:hi, :]], B)
        h2 = np.ldexp(h2, -(ex + ey))
        e32, e16 = rel(fp32, exact), rel(h2, exact)
        # the pieces' own error (exact accumulation) is below the fp32 accumulation's rounding
        e_op = rel(np.ldexp(x0 @ y0 + x0 @ y1 + x1 @ y0, -(ex + ey)), exact)
        print("decades", decades, "fp32 matrix cores", e32, "two-piece binary16", e16, "pieces alone", e_op)
        assert e16 <= e32
        assert e_op <= 0.5 * e32
        # dropping x1 y1 matters: with it the error is the same or smaller
        h2full = accumulate(lambda lo, hi: [x0[:, lo:hi] @ y0[lo:hi, :], x0[:, lo:hi] @ y1[lo:hi, :],
                                            x1[:, lo:hi] @ y0[lo:hi, :], x1[:, lo:hi] @ y1[lo:hi, :]], B)
        assert rel(np.ldexp(h2full, -(ex + ey)), exact) <= e16 * 1.01
        # a plausible mistake fails: the low piece not kept (x' cut to one binary16 piece)
        h1 = np.ldexp(accumulate(lambda lo, hi: [x0[:, lo:hi] @ y0[lo:hi, :]], B), -(ex + ey))
        assert rel(h1, exact) > 20 * e32
