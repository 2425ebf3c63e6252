"""GPU numerics of the kernels' building blocks (include/kvrc_selftest.h).

The kernels are bit-identical to the float32 oracle only if (a) the device's
IEEE division and square root round exactly like the host's, and (b) the
shared-divisor division (reciprocal plus two corrections) returns the
correctly rounded quotient on its domain 2^-60 <= b <= 2^60,
2^-64 <= |a| <= 2^66. (a) is checked against numpy float32 on the host;
(b) against the device's IEEE division: exhaustively over every bf16
numerator in the domain (the kv values the norm divides) for 2^15 divisors,
and on 2^30 random float32 numerators (the quantisation divides float32 y).
"""
import numpy as np
import pytest
import torch

import latent_attention_kv_amd as k

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def run(a, b):
    qs, qi, rt = torch.empty_like(a), torch.empty_like(a), torch.empty_like(a)
    k.kvrc_selftest_arith(a, b, qs, qi, rt)
    torch.cuda.synchronize()
    return qs, qi, rt


def log_uniform(n, lo_exp, hi_exp, gen, signed=False):
    e = torch.randint(lo_exp, hi_exp, (n,), device=DEV, generator=gen, dtype=torch.int32)
    m = 1.0 + torch.rand(n, device=DEV, generator=gen, dtype=torch.float32)
    v = torch.ldexp(m, e.to(torch.float32)).to(torch.float32)
    if signed:
        v = torch.where(torch.rand(n, device=DEV, generator=gen) < 0.5, -v, v)
    return v


def bits(t):
    return t.view(torch.int32)


def bf16_numerators():
    allbits = torch.arange(65536, dtype=torch.int32, device=DEV) << 16
    v = allbits.view(torch.float32)
    mag = v.abs()
    keep = torch.isfinite(v) & (mag >= 2.0 ** -64) & (mag <= 2.0 ** 66)
    return v[keep].contiguous()


def special_divisors():
    out = []
    for e in range(-60, 61, 7):
        base = np.float32(2.0 ** e)
        out += [base, np.nextafter(base, np.float32(np.inf)), np.nextafter(base, np.float32(0)),
                np.float32(base * 1.5), np.float32(base * 1.999999)]
    out += [np.float32(x) for x in (1.0, 3.0, 7.0, 127.0, 1 / 3, 0.1, 2.5, 0.7071068)]
    arr = np.array(out, dtype=np.float32)
    arr = arr[(arr >= 2.0 ** -60) & (arr <= 2.0 ** 60)]
    return torch.from_numpy(arr).to(DEV)


def check_shared_equals_ieee(a, b):
    qs, qi, _ = run(a.contiguous(), b.contiguous())
    bad = bits(qs) != bits(qi)
    n = int(bad.sum().item())
    if n:
        i = int(torch.nonzero(bad)[0].item())
        pytest.fail(f"{n} mismatches, e.g. a={a[i].item()!r} b={b[i].item()!r} "
                    f"shared={qs[i].item()!r} ieee={qi[i].item()!r}")


def test_shared_division_all_bf16_numerators():
    g = torch.Generator(device=DEV).manual_seed(1234)
    A = bf16_numerators()
    divisors = torch.cat([special_divisors(), log_uniform(32768, -60, 60, g)])
    per = max(1, (32 << 20) // A.numel())
    for s in range(0, divisors.numel(), per):
        b = divisors[s:s + per]
        check_shared_equals_ieee(A.repeat(b.numel()), b.repeat_interleave(A.numel()))


def test_shared_division_random_float32_numerators():
    g = torch.Generator(device=DEV).manual_seed(99)
    n = 32 << 20
    for _ in range(32):
        a = log_uniform(n, -64, 66, g, signed=True)
        b = log_uniform(n, -60, 60, g)
        check_shared_equals_ieee(a, b)


def test_shared_division_quantisation_operands():
    """y / scale with scale = RN(amax / 127) and |y| <= amax: the operand mix of
    the int8 rows (including y = amax, whose quotient must round to 127)."""
    g = torch.Generator(device=DEV).manual_seed(7)
    n = 16 << 20
    amax = log_uniform(n, -40, 40, g)
    scale = amax / 127.0
    frac = torch.rand(n, device=DEV, generator=g) * 2 - 1
    y = (amax * frac).to(torch.float32)
    y[: n // 8] = amax[: n // 8]
    check_shared_equals_ieee(y, scale)
    qs, _, _ = run(amax.contiguous(), scale.contiguous())
    assert torch.all(torch.round(qs) == 127)


def test_device_ieee_division_and_sqrt_match_host():
    rng = np.random.Generator(np.random.PCG64(5))
    n = 1 << 22
    a = (rng.standard_normal(n) * np.exp2(rng.integers(-140, 120, n))).astype(np.float32)
    b = (rng.standard_normal(n) * np.exp2(rng.integers(-120, 120, n))).astype(np.float32)
    b[b == 0] = 1.0
    qs, qi, rt = run(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV))
    with np.errstate(all="ignore"):
        want_q = a / b
        want_r = np.sqrt(np.abs(a))
    np.testing.assert_array_equal(qi.cpu().numpy().view(np.int32), want_q.view(np.int32))
    _, _, rt = run(torch.from_numpy(np.abs(a)).to(DEV), torch.from_numpy(b).to(DEV))
    np.testing.assert_array_equal(rt.cpu().numpy().view(np.int32), want_r.view(np.int32))
