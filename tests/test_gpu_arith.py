"""GPU numerics of the kernels' building blocks (include/kvrc_selftest.h).

The kernels are bit-identical to the float32 oracle only if (a) the device's
IEEE division and square root round exactly like the host's, and (b) the
shared-divisor division (reciprocal plus two corrections) returns the
correctly rounded quotient on its domain 2^-60 <= b <= 2^60,
2^-64 <= |a| <= 2^66. (a) is checked against numpy float32 on the host;
(b) against the device's IEEE division: exhaustively over every bf16
numerator in the domain (the kv values the norm divides) for 2^15 divisors,
and on 2^30 random float32 numerators (the quantisation divides float32 y).
(b') The reciprocal routine (hardware estimate plus one Newton correction)
equals the host's IEEE 1/b for every float32 b in [2^-60, 2^60], and the
shared-divisor quotient equals the host's IEEE amax / d for the two row
scale divisors d = 127 and 448 and every float32 amax in [2^-64, 2^66].
(c) The float32 -> E4M3FN conversion of the fp8 rows equals the oracle's
encoder on every code value, every midpoint and its float32 neighbours, the
saturation range and random float32 values.
"""
import numpy as np
import pytest
import torch

import latent_attention_kv_amd as k
import oracle

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


# ---------------------------------------------------------------------------
# float32 -> FLOAT8 E4M3FN conversion of the kernels against the oracle's
# encoder (nearest value by search over the decoded code table, ties to the
# even code, saturating at 448; itself pinned to the format's definition).
# ---------------------------------------------------------------------------

def e4m3_codes_gpu(x):
    xs = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)
    code = torch.empty(xs.numel(), dtype=torch.uint8, device=DEV)
    k.kvrc_selftest_e4m3(xs, code)
    torch.cuda.synchronize()
    return code.cpu().numpy()


def check_e4m3(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    pad = (-x.size) % 4
    x = np.concatenate([x, np.zeros(pad, np.float32)])
    got, want = e4m3_codes_gpu(x), oracle.e4m3_encode_array(x)
    bad = np.flatnonzero(got != want)
    if bad.size:
        i = bad[0]
        pytest.fail(f"{bad.size} mismatches, e.g. x={x[i]!r} ({x.view(np.uint32)[i]:#010x}) "
                    f"gpu={got[i]:#04x} oracle={want[i]:#04x}")


def test_e4m3_values_midpoints_and_neighbours():
    t = np.array([oracle.e4m3_decode(c) for c in range(127)], dtype=np.float32)
    mids = ((t[:-1].astype(np.float64) + t[1:]) / 2).astype(np.float32)
    pts = [t, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
           np.nextafter(t, np.float32(0)), np.nextafter(t, np.float32(1e9))]
    big = np.array([448.0, 448.00003, 460.0, 463.99997, 464.0, 465.0, 480.0, 1e6, 3.4e38],
                   np.float32)
    tiny = np.array([0.0, 2.0 ** -10, np.nextafter(np.float32(2.0 ** -10), np.float32(1)),
                     np.nextafter(np.float32(2.0 ** -10), np.float32(0)), 2.0 ** -11, 1e-20,
                     1e-38, 1e-45, 2.0 ** -126], np.float32)
    x = np.concatenate(pts + [big, tiny])
    check_e4m3(np.concatenate([x, -x]))


def test_e4m3_random_float32():
    rng = np.random.Generator(np.random.PCG64(8))
    n = 1 << 24
    # every exponent from float32 denormals to beyond the E4M3FN range
    x = (rng.uniform(1, 2, n) * np.exp2(rng.integers(-150, 12, n))).astype(np.float32)
    x[rng.random(n) < 0.5] *= -1
    check_e4m3(x)
    bits = rng.integers(0, 1 << 32, 1 << 22, dtype=np.uint64).astype(np.uint32)
    y = bits.view(np.float32)
    check_e4m3(y[np.isfinite(y)])


def test_reciprocal_routine_every_float_of_the_domain():
    """All 1,006,632,961 float32 values in [2^-60, 2^60] (bit patterns
    0x21800000 .. 0x5D800000), in chunks; expected values are numpy's IEEE
    float32 division on the host."""
    lo, hi = 0x21800000, 0x5D800000
    chunk = 1 << 26
    b = torch.empty(chunk, dtype=torch.float32, device=DEV)
    r = torch.empty_like(b)
    bad = 0
    for start in range(lo, hi + 1, chunk):
        n = min(chunk, hi + 1 - start)
        torch.arange(start, start + n, dtype=torch.int32, device=DEV, out=bits(b[:n]))
        k.kvrc_selftest_recip(b[:n], r[:n])
        got = bits(r[:n]).cpu().numpy()
        hb = np.arange(start, start + n, dtype=np.int64).astype(np.uint32).view(np.float32)
        want = (np.float32(1.0) / hb).view(np.int32)
        miss = np.flatnonzero(got != want)
        if miss.size:
            print(f"[arith] recip mismatches in chunk at {start:#x}: {miss.size}, first b bits "
                  f"{start + int(miss[0]):#x}", flush=True)
        bad += miss.size
    assert bad == 0


@pytest.mark.parametrize("d", [127.0, 448.0])
def test_row_scale_divisors_every_float_of_the_domain(d):
    """amax / 127 (int8) and amax / 448 (E4M3FN) by the shared-divisor
    quotient, for all float32 amax in [2^-64, 2^66] (bit patterns
    0x1F800000 .. 0x60800000); expected values from numpy on the host."""
    lo, hi = 0x1F800000, 0x60800000
    chunk = 1 << 26
    a = torch.empty(chunk, dtype=torch.float32, device=DEV)
    b = torch.full((chunk,), d, dtype=torch.float32, device=DEV)
    qs, qi, rt = torch.empty_like(a), torch.empty_like(a), torch.empty_like(a)
    bad = 0
    for start in range(lo, hi + 1, chunk):
        n = min(chunk, hi + 1 - start)
        torch.arange(start, start + n, dtype=torch.int32, device=DEV, out=bits(a[:n]))
        k.kvrc_selftest_arith(a[:n], b[:n], qs[:n], qi[:n], rt[:n])
        got = bits(qs[:n]).cpu().numpy()
        ha = np.arange(start, start + n, dtype=np.int64).astype(np.uint32).view(np.float32)
        want = (ha / np.float32(d)).view(np.int32)
        miss = np.flatnonzero(got != want)
        if miss.size:
            print(f"[arith] /{d} mismatches in chunk at {start:#x}: {miss.size}", flush=True)
        bad += miss.size
    assert bad == 0
