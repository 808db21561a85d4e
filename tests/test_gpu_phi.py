"""The feature map phi(x) = ELU(x) + 1 ("Linear Attention 笔记" §2) as the kernels
compute it, checked value by value against its definition.

Through the summary stage with one token per block and V = 1, the normaliser of
block b is exactly the kernel's phi of each feature of token b: z_b[r] =
phi(k_b[r]) * 1 summed over one token (and every column of S_b holds the same
value).  So every input value can be fed once:

* bf16 path: all 65536 bfloat16 bit patterns.  The kernel rounds phi to bfloat16
  (nearest even) as an MFMA operand; the reference is the binary64 phi of the same
  value rounded once to bfloat16 (nearest even).  Each result must be bit-equal,
  except where the binary64 value lies within 2^-17 (relative) of the midpoint
  between two bfloat16 neighbours -- there the float32 evaluation (a few float32
  ulps of error, about 2^-21) may land on the other side, and the result must then
  be one of the two neighbours.  Results below the smallest normal float (x below
  about -87.3) may differ by at most 2^-126 in absolute terms.
* float32 path: the same 65536 values as float32, and 2^16 random float32 values in
  [-30, 30]; the result must be within 2 float32 ulps of the binary64 phi.
* NaN stays NaN, -inf gives 0; +inf gives NaN or +inf (x - max(x, 0) is inf - inf).
"""
import numpy as np
import pytest
import torch

import token_level_head_amd as mh

pytestmark = pytest.mark.gpu

D = 16
TOK = 65536 // D  # one token per block: M = N = 4096


def phi64(x):
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def bf16_bits_to_f64(bits):
    with np.errstate(invalid="ignore"):
        return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16_rne(y):
    """Round finite binary64 values >= 2^-126 to bfloat16 (8 significant bits), nearest
    even, directly from binary64 (no intermediate float32 rounding).  Returns
    (rounded value as float64, relative distance of y from the nearest rounding midpoint)."""
    y = np.asarray(y, dtype=np.float64)
    bits = y.view(np.uint64)
    drop = np.uint64(52 - 7)
    low_mask = (np.uint64(1) << drop) - np.uint64(1)
    trunc = bits & ~low_mask
    lo = trunc.view(np.float64)
    ulp = np.ldexp(1.0, np.frexp(np.where(lo == 0, 1.0, lo))[1] - 8)
    mid = lo + ulp / 2
    rem = bits & low_mask
    half = np.uint64(1) << (drop - np.uint64(1))
    odd = (trunc >> drop) & np.uint64(1)
    up = (rem > half) | ((rem == half) & (odd == 1))
    out = np.where(up, lo + ulp, lo)
    return out, np.abs(y - mid) / np.abs(y)


def kernel_phi(values, dtype):
    """phi of each value in `values` (65536 of them, as [TOK, D] tokens) through the summary
    stage with one token per block and V = 1: returns z [TOK, D] float32 and the S columns."""
    if dtype == torch.bfloat16:
        k = torch.from_numpy(values.astype(np.uint16).view(np.int16)).view(torch.bfloat16)
    else:
        k = torch.from_numpy(values.astype(np.float32))
    k = k.reshape(1, 1, TOK, D).cuda()
    v = torch.ones_like(k)
    L = D * D + D
    S = torch.full((TOK * L,), float("nan"), dtype=torch.float32, device="cuda")
    mh.mhla_block_summaries(k, v, S, TOK)
    torch.cuda.synchronize()
    packed = S.cpu().reshape(TOK, L)
    Sm, z = mh.mhla_unpack_summaries(packed, D)
    return z.numpy(), Sm.numpy()


def test_phi_bf16_path_every_bf16_value():
    bits = np.arange(65536, dtype=np.uint32)
    x = bf16_bits_to_f64(bits)
    z, Sm = kernel_phi(bits, torch.bfloat16)
    z = z.reshape(-1).astype(np.float64)
    # every column of S_b carries the same phi(k_b[r]) * 1
    assert np.array_equal(np.isnan(Sm), np.isnan(np.repeat(z.reshape(TOK, D, 1), D, axis=2)))
    assert np.allclose(Sm, np.repeat(z.reshape(TOK, D, 1), D, axis=2), rtol=0, atol=0, equal_nan=True)

    nan_in = np.isnan(x)
    assert np.all(np.isnan(z[nan_in])), "NaN inputs must give NaN"
    assert np.all(z[x == -np.inf] == 0.0)
    assert np.all(np.isnan(z[x == np.inf]) | (z[x == np.inf] == np.inf))

    fin = np.isfinite(x)
    ref = phi64(x[fin])
    got = z[fin]
    sub = ref < 2.0 ** -126  # results in the float32 subnormal range (x < about -87.3)
    assert np.all(np.abs(got[sub] - ref[sub]) <= 2.0 ** -126)
    r, dist = round_bf16_rne(ref[~sub])
    g = got[~sub]
    exact = g == r
    near_tie = dist <= 2.0 ** -17
    bad = ~exact & ~near_tie
    assert not np.any(bad), (f"{bad.sum()} values differ from RNE-bf16 of phi away from a rounding tie; "
                             f"first inputs {x[fin][~sub][bad][:8]}")
    # where a tie is close, the result is one of the two bfloat16 neighbours (<= 1 ulp away)
    ulp = np.ldexp(1.0, np.frexp(r)[1] - 8)
    assert np.all(np.abs(g - r) <= ulp)
    n_mismatch = int((~exact).sum())
    print(f"phi bf16 path: {exact.sum()} of {exact.size} normal results bit-equal to RNE-bf16(phi), "
          f"{n_mismatch} one ulp away next to a rounding tie; {int(sub.sum())} subnormal-range results")
    # bf16 x > 0: x + 1 is exact in binary64; it must round exactly as RNE does unless a tie is near
    pos = x[fin][~sub] > 0
    assert np.mean(exact[pos]) > 0.99


def test_phi_f32_path():
    bits = np.arange(65536, dtype=np.uint32)
    x_grid = bf16_bits_to_f64(bits)
    rng = np.random.default_rng(77)
    x_rand = rng.uniform(-30.0, 30.0, 65536).astype(np.float32).astype(np.float64)
    for x in (x_grid, x_rand):
        fin = np.isfinite(x)
        xs = np.where(fin, x, 0.0).astype(np.float32)
        z, _ = kernel_phi(xs, torch.float32)
        z = z.reshape(-1).astype(np.float64)
        ref = phi64(xs.astype(np.float64))
        normal = ref >= 2.0 ** -126
        ulp32 = np.ldexp(1.0, np.frexp(ref[normal])[1] - 24)
        err = np.abs(z[normal] - ref[normal]) / ulp32
        assert np.max(err) <= 2.0, (np.max(err), xs[normal][np.argmax(err)])
        assert np.all(np.abs(z[~normal] - ref[~normal]) <= 2.0 ** -126)
    # NaN stays NaN on the float32 path too
    xs = np.zeros(65536, dtype=np.float32)
    xs[::97] = np.nan
    z, _ = kernel_phi(xs, torch.float32)
    z = z.reshape(-1)
    assert np.all(np.isnan(z[::97])) and np.all(z[np.arange(65536) % 97 != 0] == 1.0)


@pytest.mark.parametrize("workload", ["fused", "staged", "causal"])
def test_nan_query_gives_nan_row(workload):
    """A NaN in q_t makes row t of Y NaN and leaves every other row finite (the output
    ratio reads q_t only for row t)."""
    shapes = {"fused": (2, 3, 256, 64, 16, False), "staged": (2, 3, 1024, 32, 8, False),
              "causal": (2, 3, 1024, 64, 8, True)}
    B, H, N, d, M, causal = shapes[workload]
    g = torch.Generator(device="cpu").manual_seed(5)
    q, k, v = (torch.randn((B, H, N, d), generator=g).to(torch.bfloat16) for _ in range(3))
    q[1, 2, 37, 5] = float("nan")
    W = torch.softmax(torch.randn((M, M), generator=g), dim=1)
    if causal:
        W = torch.tril(W)
    out = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    mh.mhla_forward(q.cuda(), k.cuda(), v.cuda(), W.cuda(), out, causal=causal)
    y = out.cpu()
    assert torch.isnan(y[1, 2, 37]).all()
    mask = torch.ones((B, H, N), dtype=torch.bool)
    mask[1, 2, 37] = False
    assert torch.isfinite(y[mask]).all()
