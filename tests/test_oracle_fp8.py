"""Pins for the oracle's 8-bit cache: the E4M3 codec against the format's
definition (hand-worked code points, order, nearest-even by brute force,
saturation), the quantising slot write against the error bound that
definition implies, and decode over an 8-bit pool against the already
pinned fp32 path on the same values.  A quantized cache is one of the levers
that shrink each token's footprint and stack with paging (the vLLM
PagedAttention blog page, "Where it bites"); the format itself is OCP E4M3
with one bf16 scale per (token, kv head, side).  CPU only."""
import json
import os

import numpy as np
import pytest

import oracle
from workloads import bf16_bits_to_f32, f32_to_bf16_bits
from workloads.gen import fp8_region_bytes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FINITE = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)


def _value(text):
    if text == "nan":
        return float("nan")
    if text == "-0":
        return -0.0
    out = 1.0
    for part in text.split("*"):
        part = part.strip()
        out *= 2.0 ** int(part[2:]) if part.startswith("2^") else float(part)
    return out


# --- the codec ------------------------------------------------------------------
def test_code_points_from_the_format_definition():
    g = json.load(open(os.path.join(GOLDEN, "e4m3_code_points.json")))
    codes = np.array([int(c, 16) for c, _ in g["code_points"]], np.uint8)
    want = np.array([_value(v) for _, v in g["code_points"]])
    got = oracle.e4m3_decode(codes)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))  # -0 keeps its sign


def test_decode_is_monotone_and_sign_symmetric():
    """Codes 0x00..0x7E are the non-negative finite values in increasing
    order (a property of sign-magnitude floats with a biased exponent);
    setting the sign bit negates."""
    pos = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    assert pos[0] == 0.0 and pos[-1] == 448.0
    neg = oracle.e4m3_decode(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -pos)
    # the spacing doubles at each binade from the first normal up
    assert np.all(np.diff(pos[:9]) == 2.0 ** -9)
    assert np.all(np.diff(pos[0x70:0x79]) == 16.0)
    assert np.all(np.diff(pos[0x78:0x7F]) == 32.0)


def test_every_finite_code_round_trips():
    vals = oracle.e4m3_decode(FINITE).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), FINITE)


def _nearest_even_brute_force(x):
    """Nearest finite E4M3 value by exhaustive search; ties go to the even
    code (mantissa bit 0 clear); beyond 448 the nearest is 448."""
    mags = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # 0 .. 448
    out = np.empty(len(x), np.uint8)
    for i, xi in enumerate(np.asarray(x, np.float64)):
        a = min(abs(xi), 448.0)  # saturation; also keeps the distances exact
        dist = np.abs(mags - a)           # exact in double for these operands
        best = np.flatnonzero(dist == dist.min())
        c = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        out[i] = c | (0x80 if np.signbit(xi) else 0)
    return out


def test_encode_is_round_to_nearest_even_with_saturation():
    rng = np.random.default_rng(81)
    mags = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (mags[:-1] + mags[1:]) / 2          # every tie, exactly representable in fp32
    x = np.concatenate([
        rng.standard_normal(4000) * 50,
        rng.uniform(-2.0 ** -5, 2.0 ** -5, 2000),  # subnormal range and the first binade
        np.exp(rng.uniform(np.log(1e-4), np.log(460.0), 3000)),
        mids, -mids, mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20),
        [448.0, 449.0, 463.99, 500.0, 1e30, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11],
    ]).astype(np.float32)
    got = oracle.e4m3_encode(x)
    assert np.array_equal(got, _nearest_even_brute_force(x))


def test_encode_special_values():
    x = np.array([np.nan, -np.nan, np.inf, -np.inf, 464.0, -464.0, 463.9999, 0.0, -0.0],
                 np.float32)
    got = oracle.e4m3_encode(x)
    assert got[0] & 0x7F == 0x7F and got[1] & 0x7F == 0x7F      # NaN stays NaN
    assert list(got[2:]) == [0x7E, 0xFE, 0x7E, 0xFE, 0x7E, 0x00, 0x80]


# --- the quantising slot write -------------------------------------------------------
def _fp8_case(rng, nb, nkv, B, d, T):
    rk, rv = fp8_region_bytes(B, d)
    k = rng.integers(0, 256, (nb, nkv, rk), dtype=np.uint8)
    v = rng.integers(0, 256, (nb, nkv, rv), dtype=np.uint8)
    kn = f32_to_bf16_bits(rng.standard_normal((T, nkv, d)).astype(np.float32) * 3)
    vn = f32_to_bf16_bits(rng.standard_normal((T, nkv, d)).astype(np.float32) * 3)
    slots = rng.choice(nb * B, size=T, replace=False).astype(np.int64)
    return k, v, kn, vn, slots


def _read_back(k_pool, v_pool, B, d, blk, g, r, v_side):
    """Codes and scale of token slot r of (blk, g), read by the documented
    layout: K codes [B][d] then the scale groups (4 K scales, 4 V scales per
    4 slots, bf16) in the K buffer; V codes [d][B] in the V buffer."""
    if v_side:
        c = v_pool[blk, g].reshape(d, B)[:, r]
    else:
        c = k_pool[blk, g, :B * d].reshape(B, d)[r]
    at = B * d + 16 * (r // 4) + 8 * int(v_side) + 2 * (r % 4)
    bits = k_pool[blk, g, at:at + 2].view(np.uint16)
    return c, float(bf16_bits_to_f32(bits)[0])


def test_kv_write_fp8_error_bound_and_scale():
    """Each written row dequantises to within half an E4M3 step of its input:
    |x - x'| <= 2^-4 |x| for normal codes and <= 2^-10 s on the subnormal
    range, plus fp32 rounding of x / s; the largest |x| of a row maps to
    448 (code 0x7E with x's sign); 448 s equals max |x| to bf16 rounding."""
    rng = np.random.default_rng(82)
    nb, nkv, B, d, T = 12, 3, 16, 32, 40
    k, v, kn, vn, slots = _fp8_case(rng, nb, nkv, B, d, T)
    kn[5, 1, :] = 0                                   # an all-zero row
    k2, v2 = oracle.kv_write(k, v, kn, vn, slots)
    for i, slot in enumerate(slots):
        blk, r = divmod(int(slot), B)
        for g in range(nkv):
            for src, v_side in ((kn, False), (vn, True)):
                x = bf16_bits_to_f32(src[i, g]).astype(np.float64)
                c, s = _read_back(k2, v2, B, d, blk, g, r, v_side)
                amax = np.abs(x).max()
                if amax == 0:
                    assert s == 0.0 and not c.any()
                    continue
                assert abs(448.0 * s - amax) <= amax * 2.0 ** -8
                top = int(np.argmax(np.abs(x)))
                assert c[top] == (0xFE if x[top] < 0 else 0x7E)
                deq = oracle.e4m3_decode(c) * s
                bound = 2.0 ** -4 * np.abs(x) * (1 + 2.0 ** -20) + s * 2.0 ** -10
                assert np.all(np.abs(deq - x) <= bound)
                assert np.all(np.signbit(deq[x != 0]) == np.signbit(x[x != 0]))


def test_kv_write_fp8_touches_only_its_slots():
    """Skipped tokens (slot -1) write nothing; every byte outside the written
    slots' codes and scales is unchanged."""
    rng = np.random.default_rng(83)
    nb, nkv, B, d, T = 10, 2, 16, 64, 30
    k, v, kn, vn, slots = _fp8_case(rng, nb, nkv, B, d, T)
    slots[::3] = -1
    k2, v2 = oracle.kv_write(k, v, kn, vn, slots)
    touched_k = np.zeros(k.shape, bool)
    touched_v = np.zeros(v.shape, bool)
    for slot in slots[slots >= 0]:
        blk, r = divmod(int(slot), B)
        touched_k[blk, :, r * d:(r + 1) * d] = True
        touched_v[blk, :, r:B * d:B] = True
        for side in (0, 1):
            at = B * d + 16 * (r // 4) + 8 * side + 2 * (r % 4)
            touched_k[blk, :, at:at + 2] = True
    assert np.array_equal(k2[~touched_k], k[~touched_k])
    assert np.array_equal(v2[~touched_v], v[~touched_v])
    assert not np.array_equal(k2, k) and not np.array_equal(v2, v)


def _bf16(x):
    return np.array([x], np.float32).view(np.uint32).astype(np.uint32) >> 16


def test_gather_reads_the_region_layout_by_hand():
    """One token placed by hand: K codes at [r][i], V codes at [i][r], bf16
    scales in the K buffer's scale groups; gather returns decode(code) *
    scale at (token, dim)."""
    nb, B, d = 3, 16, 8
    rk, rv = fp8_region_bytes(B, d)
    k = np.zeros((nb, 1, rk), np.uint8)
    v = np.zeros((nb, 1, rv), np.uint8)
    r, i = 5, 3
    k[2, 0, r * d + i] = 0x38                     # 1.0
    v[2, 0, i * B + r] = 0x42                     # 2.5
    grp = B * d + 16 * (r // 4) + 2 * (r % 4)
    k[2, 0, grp:grp + 2] = np.array(_bf16(2.0), np.uint16).view(np.uint8)       # K scale
    k[2, 0, grp + 8:grp + 10] = np.array(_bf16(-4.0), np.uint16).view(np.uint8)  # V scale
    table = np.array([0, 2], np.int32)
    Kc, Vc = oracle.gather(k, v, table, 0, 2 * B)
    want_k = np.zeros((2 * B, d))
    want_v = np.zeros((2 * B, d))
    want_k[B + r, i] = 2.0
    want_v[B + r, i] = -10.0
    assert np.array_equal(Kc, want_k) and np.array_equal(Vc, want_v)


# --- decode over an 8-bit pool ------------------------------------------------------------
def _fp8_to_f32_pools(k8, v8, B, d):
    """The fp32 pools holding the same values, built from the documented layout."""
    nb, nkv = k8.shape[:2]
    kc = k8[..., :B * d].reshape(nb, nkv, B, d)
    vc = v8.reshape(nb, nkv, d, B)
    sc = bf16_bits_to_f32(k8[..., B * d:].view(np.uint16)).reshape(nb, nkv, B // 4, 2, 4)
    ks = sc[:, :, :, 0, :].reshape(nb, nkv, B)
    vs = sc[:, :, :, 1, :].reshape(nb, nkv, B)
    kval = oracle.e4m3_decode(kc) * ks[:, :, :, None]
    vval = oracle.e4m3_decode(vc) * vs[:, :, None, :]
    return kval.astype(np.float32), vval.astype(np.float32)


def _random_fp8_pools(rng, nb, nkv, B, d):
    rk, rv = fp8_region_bytes(B, d)
    k8 = np.empty((nb, nkv, rk), np.uint8)
    k8[..., :B * d] = rng.choice(FINITE, size=(nb, nkv, B * d))
    k8[..., B * d:] = f32_to_bf16_bits(
        (rng.uniform(1, 2, (nb, nkv, 2 * B)) * 2.0 ** -7).astype(np.float32)).view(
            np.uint8).reshape(nb, nkv, 4 * B)
    v8 = rng.choice(FINITE, size=(nb, nkv, rv)).astype(np.uint8)
    return k8, v8


def test_fp8_decode_equals_fp32_decode_of_the_same_values():
    """bf16 scales times 4-bit code significands are exact in fp32, so the
    fp32 oracle over those values must agree bit for bit with the 8-bit
    oracle (same doubles, same order); q is bf16 in both."""
    rng = np.random.default_rng(84)
    nb, nkv, B, d, S, Hq = 20, 2, 16, 32, 3, 4
    k8, v8 = _random_fp8_pools(rng, nb, nkv, B, d)
    q = f32_to_bf16_bits(rng.standard_normal((S, Hq, d)).astype(np.float32))
    tables = rng.permutation(nb)[:S * 4].reshape(S, 4).astype(np.int32)
    lens = np.array([1, 37, 64], np.int32)
    out8 = oracle.decode(k8, v8, q, tables, lens, d ** -0.5)
    k32, v32 = _fp8_to_f32_pools(k8, v8, B, d)
    assert np.all(np.isfinite(k32)) and np.all(np.isfinite(v32))
    out32 = oracle.decode(k32, v32, bf16_bits_to_f32(q), tables, lens, d ** -0.5)
    assert np.array_equal(out8, out32)


def test_fp8_zero_keys_give_mean_of_dequantised_values():
    """All K codes zero: every score is 0, weights are uniform, out is the
    mean of the dequantised V rows of the context."""
    rng = np.random.default_rng(85)
    nb, B, d, L = 4, 16, 16, 23
    rk, rv = fp8_region_bytes(B, d)
    k8 = np.zeros((nb, 1, rk), np.uint8)
    sc = k8[..., B * d:].view(np.uint16).reshape(nb, 1, B // 4, 2, 4)
    sc[:, :, :, 0, :] = _bf16(1.0)
    sc[:, :, :, 1, :] = _bf16(0.25)
    v8 = rng.choice(FINITE, size=(nb, 1, rv)).astype(np.uint8)
    q = f32_to_bf16_bits(rng.standard_normal((1, 2, d)).astype(np.float32))
    table = np.array([[3, 1]], np.int32)
    out = oracle.decode(k8, v8, q, table, np.array([L], np.int32), 0.3)
    rows = [oracle.e4m3_decode(v8[b, 0].reshape(d, B)[:, r]) * 0.25
            for b, n in ((3, B), (1, L - B)) for r in range(n)]
    want = np.mean(rows, axis=0)
    assert np.allclose(out[0, 0], want, rtol=0, atol=1e-12)
    assert np.allclose(out[0, 1], want, rtol=0, atol=1e-12)


def test_fp8_block_copy_copies_codes_and_scales():
    rng = np.random.default_rng(86)
    nb, nkv, B, d = 8, 2, 16, 32
    rk, rv = fp8_region_bytes(B, d)
    k = rng.integers(0, 256, (nb, nkv, rk), dtype=np.uint8)
    v = rng.integers(0, 256, (nb, nkv, rv), dtype=np.uint8)
    pairs = np.array([[1, 4], [1, 6], [7, 0]], np.int32)
    k2, v2 = oracle.block_copy(k, v, pairs)
    for src, dst in pairs:
        assert np.array_equal(k2[dst], k[src]) and np.array_equal(v2[dst], v[src])
    others = [b for b in range(nb) if b not in pairs[:, 1]]
    assert np.array_equal(k2[others], k[others]) and np.array_equal(v2[others], v[others])


def test_fp8_geometry_from_the_two_buffers():
    """Block size and head dim follow from the region sizes: R_k - R_v = 4B,
    R_v = B d; a pair that does not fit is refused."""
    k = np.zeros((2, 1, 16 * 68), np.uint8)
    v = np.zeros((2, 1, 16 * 64), np.uint8)
    assert oracle._geom(k, v) == (2, 16, 1, 64)
    with pytest.raises(ValueError):
        oracle._geom(k, np.zeros((2, 1, 16 * 68), np.uint8))


def test_fp8_dense_layout_is_rejected():
    """Dense copies are plain fp32 / bf16 arrays; an 8-bit dense call is refused."""
    k = np.zeros((1, 1, 4, 8), np.uint8)
    with pytest.raises(oracle.OracleError):
        oracle.decode_dense(k, k, np.zeros((1, 1, 8), np.uint16), np.array([1], np.int32), 1.0)
