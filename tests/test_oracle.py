"""Pins for the CPU oracle, each against something other than the oracle itself.

  * number formats: hand-derived bit patterns (tests/golden) and numpy's own
    float16 / float32 decoders over all 65536 patterns; MXFP4 (OCP Microscaling v1.0,
    which the pages name but do not define): the E2M1 value table, the same codes
    embedded in FP8 E4M3 and decoded by torch, and torch's own E8M0 decoder; IQ4_NL
    (ggml's type, which the pages name as an IQ-series format but do not define): the
    published 16-level table (tests/golden), a hand-worked row, and the reduction of an
    IQ4_NL product to the Q8_0 product on the same levels; IQ4_XS (ggml's super-block
    packing of those codes): a hand-built record exercising every sub-scale bit, and the
    reduction of an IQ4_XS product to the IQ4_NL product on its block scales;
  * row-id maps: exhaustive brute force by a stable sort on tiny inputs, numpy's
    stable argsort on random ones, and the invariants of the maps;
  * mul_mat_id: the dense all-experts product (numpy matmul) masked by ids, plain
    GEMM when E = k = 1, exact doubling when x doubles;
  * FFN: a dense MoE written with torch's matmul and silu, the shared-expert
    concatenation identity, one-hot routing, and a hand-derived worked example in
    closed form;
  * router (top-k + softmax over the picks): a full stable sort, numpy softmax,
    tie order, shift invariance, k = 1 and k = E, and a hand-computed example.
The op being pinned: "CUDA: better MoE implementation" (ik_llama.cpp PR #283
write-up), sections 1.2 (operands and semantics) and 2.1 (the three row maps).
"""
import itertools
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_pairs(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].strip()
        if line:
            b, v = line.split()
            rows.append((int(b, 16), float(v)))
    return rows


def normwise(got, ref):
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(np.asarray(got, np.float64) - ref).max() / (den if den > 0 else 1.0))


# --------------------------------------------------------------------- formats

def test_half_fixture():
    for bits, val in _read_pairs("fp16_values.txt"):
        got = oracle.half_to_double(bits)
        assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(bits)


def test_bf16_fixture():
    for bits, val in _read_pairs("bf16_values.txt"):
        assert oracle.bf16_to_double(bits) == val, hex(bits)


def test_half_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def test_bf16_sampled_patterns_match_numpy():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = np.array([oracle.bf16_to_double(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])


def test_q8_0_dequant_fixture_and_numpy():
    # One block: scale 2^-10 (0x1400), q = -127..-96 and a second row 0..31.
    qs = np.stack([np.arange(-127, -95), np.arange(0, 32)]).astype(np.int8)[None]
    d = np.array([[[0x1400], [0x1418]]], np.uint16).view(np.float16)
    got = oracle.dequant(qs, d)
    assert np.array_equal(got[0, 0], np.arange(-127, -95) / 1024.0)
    assert np.array_equal(got[0, 1], np.arange(0, 32) * 0.00099945068359375)
    rng = np.random.default_rng(0)
    qs, d = synth.gen.draw_q8_0(rng, 5, 96)
    ref = qs.astype(np.float64) * np.repeat(d.astype(np.float64), 32, axis=1)
    assert np.array_equal(oracle.dequant(qs, d), ref)


# --------------------------------------------------------------------- row ids

def _brute_maps(ids, E, B):
    T, k = ids.shape
    flat = [(t, s) for t in range(T) for s in range(k)]

    def bucket(ts):
        e = ids[ts]
        return e if 0 <= e < E else E

    order = sorted(range(T * k), key=lambda i: (bucket(flat[i]), i))
    s1 = [flat[i][0] * B + flat[i][1] % B for i in order]
    dd = [flat[i][0] * k + flat[i][1] for i in order]
    bounds = [sum(1 for ts in flat if bucket(ts) < e) for e in range(E + 1)]
    return np.array(s1), np.array(dd), np.array(bounds)


def _check_invariants(ids, E, B, s1, dd, b):
    T, k = ids.shape
    n = T * k
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    assert b[0] == 0 and np.all(np.diff(b) >= 0) and b[E] == int(valid.sum())
    assert np.array_equal(np.diff(b), np.bincount(flat[valid], minlength=E))
    assert np.array_equal(np.sort(dd), np.arange(n))           # bijection onto [0, T*k)
    if B == 1:
        assert np.array_equal(s1, dd // k)
    else:
        assert np.array_equal(s1, dd)
    for e in range(E):
        seg = dd[b[e]:b[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)                          # stable: (t, s) ascending
    tail = dd[b[E]:]
    assert np.all(~valid[tail]) and np.all(np.diff(tail) > 0)
    # gather by ids_src1 then scatter by ids_dst reproduces the per-slot source rows
    rows = np.arange(T * B)
    gathered = rows[s1]
    back = np.empty(n, np.int64)
    back[dd] = gathered
    want = (np.arange(n) // k) * B + (np.arange(n) % k) % B
    assert np.array_equal(back, want)


@pytest.mark.parametrize("E,T,k", [(1, 3, 1), (2, 2, 2), (3, 2, 2), (4, 3, 2), (2, 3, 3)])
def test_row_ids_exhaustive(E, T, k):
    values = list(range(-1, E + 1))       # includes out-of-range ids on both sides
    for combo in itertools.product(values, repeat=T * k):
        ids = np.array(combo, np.int32).reshape(T, k)
        for B in sorted({1, k}):
            s1, dd, b = oracle.row_ids(ids, E, B)
            r1, rd, rb = _brute_maps(ids, E, B)
            assert np.array_equal(s1, r1) and np.array_equal(dd, rd) and np.array_equal(b, rb)


@pytest.mark.parametrize("E,T,k,seed", [(8, 16, 2, 1), (64, 512, 6, 2), (128, 333, 8, 3),
                                        (512, 97, 12, 4), (1, 50, 1, 5), (5, 40, 7, 6)])
def test_row_ids_random_vs_stable_argsort(E, T, k, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-2, E + 2, size=(T, k)).astype(np.int32)   # duplicates and invalids
    for B in sorted({1, k}):
        s1, dd, b = oracle.row_ids(ids, E, B)
        flat = ids.reshape(-1)
        key = np.where((flat >= 0) & (flat < E), flat, E)
        order = np.argsort(key, kind="stable")
        assert np.array_equal(dd, order)
        assert np.array_equal(b, np.searchsorted(np.sort(key), np.arange(E + 1), side="left"))
        _check_invariants(ids, E, B, s1, dd, b)


@pytest.mark.parametrize("name", ["tiny", "lite", "dec1", "dec8", "skew"])
def test_row_ids_configs_invariants(name):
    cfg = synth.CONFIGS[name]
    ids = synth.make_inputs(cfg)["ids"] if cfg.kind == "mmid" else None
    if ids is None:
        ids = (synth.draw_ids_zipf(cfg.seed, cfg.n_tokens, cfg.n_experts, cfg.n_used, cfg.zipf_s)
               if cfg.routing == "zipf" else
               synth.draw_ids_uniform(cfg.seed, cfg.n_tokens, cfg.n_experts, cfg.n_used))
    s1, dd, b = oracle.row_ids(ids, cfg.n_experts, 1)
    assert b[-1] == cfg.n_tokens * cfg.n_used        # bounds' counts sum to T*k
    _check_invariants(ids, cfg.n_experts, 1, s1, dd, b)


# ------------------------------------------------------------------ mul_mat_id

# FP4 E2M1 magnitudes by code 0..7, from the table of the OCP Microscaling (MX) v1.0
# specification; codes 8..15 are the same values negated.
_E2M1 = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _e8m0_torch(x):
    """E8M0 bytes -> float64 through torch's float8_e8m0fnu decoder."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8))
    return t.view(torch.float8_e8m0fnu).to(torch.float64).numpy()


def _iq4nl_levels():
    """The 16 IQ4_NL levels from the golden file (ggml's table, cited there)."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "iq4nl_levels.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    assert [int(r[0]) for r in rows] == list(range(16))
    return np.array([float(r[1]) for r in rows])


def _numpy_iq4xs_scales(rec):
    """Per-block scales [..][rows][cols/32] of IQ4_XS records [..][rows][cols/256][8], read
    field by field: fp16 d, scales_h (2 bits per block), scales_l (a nibble per block)."""
    d = rec[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    sh = rec[..., 2].astype(np.int64) | (rec[..., 3].astype(np.int64) << 8)
    out = np.empty(rec.shape[:-1] + (8,))
    for j in range(8):
        lo = (rec[..., 4 + j // 2] >> (4 * (j % 2))) & 15
        hi = (sh >> (2 * j)) & 3
        out[..., j] = d * ((lo | (hi << 4)).astype(np.int64) - 32)
    return out.reshape(rec.shape[:-2] + (rec.shape[-2] * 8,))


def _numpy_dequant(qs, d):
    if qs.dtype == np.uint8 and d.ndim == qs.ndim + 1:   # IQ4_XS: IQ4_NL codes, super-blocks
        codes = np.stack([qs & 15, qs >> 4], axis=-1).reshape(qs.shape[:-1] + (2 * qs.shape[-1],))
        return _iq4nl_levels()[codes] * np.repeat(_numpy_iq4xs_scales(d), 32, axis=-1)
    if qs.dtype == np.uint8 and d.dtype == np.float16:   # IQ4_NL: MXFP4 packing, fp16 scale
        codes = np.stack([qs & 15, qs >> 4], axis=-1).reshape(qs.shape[:-1] + (2 * qs.shape[-1],))
        return _iq4nl_levels()[codes] * np.repeat(d.astype(np.float64), 32, axis=-1)
    if qs.dtype == np.uint8:   # MXFP4: low nibble = even column; table lookup; torch E8M0
        codes = np.stack([qs & 15, qs >> 4], axis=-1).reshape(qs.shape[:-1] + (2 * qs.shape[-1],))
        table = np.array(_E2M1 + tuple(-v for v in _E2M1))
        return table[codes] * np.repeat(_e8m0_torch(d), 32, axis=-1)
    return qs.astype(np.float64) * np.repeat(d.astype(np.float64), 32, axis=-1)


def test_e2m1_table_and_fp8_embedding():
    """Every E2M1 code against the format's table (sign included), and against torch's
    FP8 E4M3 decoder: E2M1 code (s, e, m) is the E4M3 pattern with the same sign, the
    exponent rebased from bias 1 to bias 7 and the mantissa bit on top of E4M3's three
    (the subnormal 0.5 is the normal E4M3 number 2^-1)."""
    import torch
    for c in range(16):
        v = oracle.e2m1_to_double(c)
        mag = _E2M1[c & 7]
        assert v == (-mag if c & 8 else mag) and math.copysign(1.0, v) == (-1.0 if c & 8 else 1.0)
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        if e == 0:
            bits = (s << 7) | ((6 << 3) if m else 0)
        else:
            bits = (s << 7) | ((e + 6) << 3) | (m << 2)
        t = torch.tensor([bits], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
        assert float(t[0]) == v, c


def test_e8m0_all_patterns_match_torch():
    got = np.array([oracle.e8m0_to_double(x) for x in range(256)])
    ref = _e8m0_torch(np.arange(256))
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[128] == 2.0 and got[126] == 0.5


def test_mxfp4_dequant_layout_and_values():
    """Byte i of a row holds column 2i (low nibble) and 2i+1 (high nibble); the 32
    columns of a block share one scale."""
    q = np.array([[0x21, 0x8F] + [0] * 14 + [0x77] * 16], dtype=np.uint8)   # 1 row, 64 columns
    d = np.array([[127, 129]], dtype=np.uint8)
    w = oracle.dequant(q[None], d[None])[0, 0]
    assert w.shape == (64,)
    assert (w[0], w[1], w[2], w[3]) == (0.5, 1.0, -6.0, -0.0)
    assert np.all(w[32:] == 6.0 * 4)     # code 7 = 6, scale 2^(129-127)
    qs, dd = synth.gen.draw_q8_0_stack(5, 2, 1, 3, 7, 96, wtype="mxfp4")
    assert np.array_equal(oracle.dequant(qs, dd), _numpy_dequant(qs, dd))


def test_iq4nl_levels_match_golden():
    """Every code's level against the published table (golden file), and the table's
    shape: strictly increasing, one level per code, ends at -127 and 113."""
    lv = _iq4nl_levels()
    assert np.array_equal([oracle.iq4nl_level(c) for c in range(16)], lv)
    assert np.all(np.diff(lv) > 0) and lv[0] == -127 and lv[15] == 113
    assert math.isnan(oracle.iq4nl_level(16)) and math.isnan(oracle.iq4nl_level(-1))


def test_iq4nl_dequant_worked_example():
    """Hand-worked row of 64 columns: byte 0 = 0x8F holds column 0 (low nibble, code 15,
    level 113) and column 1 (code 8, level 1); byte 1 = 0x07 holds column 2 (code 7,
    level -10) and column 3 (code 0, level -127); block 0's scale is fp16 0x3800 = 0.5.
    Block 1's bytes are all 0x9A (even columns code 10 = 25, odd ones code 9 = 13) with
    scale 0x4000 = 2: 50 and 26."""
    q = np.array([[0x8F, 0x07] + [0] * 14 + [0x9A] * 16], dtype=np.uint8)
    d = np.array([[0x3800, 0x4000]], dtype=np.uint16).view(np.float16)
    w = oracle.dequant(q[None], d[None])[0, 0]
    assert w.shape == (64,)
    assert (w[0], w[1], w[2], w[3]) == (56.5, 0.5, -5.0, -63.5)
    assert np.all(w[4:32:2] == -63.5) and np.all(w[5:32:2] == -63.5)   # zero bytes: code 0
    assert np.all(w[32::2] == 50.0) and np.all(w[33::2] == 26.0)
    qs, dd = synth.gen.draw_q8_0_stack(5, 2, 1, 3, 7, 96, wtype="iq4_nl")
    assert qs.dtype == np.uint8 and dd.dtype == np.float16 and qs.shape == (3, 7, 48)
    assert np.array_equal(oracle.dequant(qs, dd), _numpy_dequant(qs, dd))


@pytest.mark.parametrize("B_is_k", [False, True])
def test_mul_mat_id_iq4nl_is_q8_0_on_the_levels(B_is_k):
    """IQ4_NL with codes c and scales d is Q8_0 with q = level(c) and the same d: the
    oracle's IQ4_NL product must equal its (separately pinned) Q8_0 product bit for bit."""
    rng = np.random.default_rng(13)
    E, N, K, T, k = 5, 24, 128, 7, 2
    qs, d = synth.gen.draw_q8_0_stack(10, 2, 0, E, N, K, wtype="iq4_nl")
    codes = np.stack([qs & 15, qs >> 4], axis=-1).reshape(E, N, K)
    q8 = _iq4nl_levels()[codes].astype(np.int8)
    B = k if B_is_k else 1
    x = synth.f32_to_bf16_bits(rng.standard_normal((T * B, K)).astype(np.float32))
    ids = rng.integers(-1, E + 1, size=(T, k)).astype(np.int32)
    rw = synth.draw_route_w(5, T, k)
    for r in (None, rw):
        got = oracle.mul_mat_id(qs, d, x, "bf16", ids, r, B)
        assert np.array_equal(got, oracle.mul_mat_id(q8, d, x, "bf16", ids, r, B))
    ref = _dense_masked(_numpy_dequant(qs, d), synth.bf16_bits_to_f32(x).astype(np.float64), ids, B)
    assert normwise(oracle.mul_mat_id(qs, d, x, "bf16", ids, None, B), ref) < 1e-13


# Hand-built IQ4_XS super-block record: d = 1 (fp16 0x3C00); the 6-bit sub-scales of
# blocks 0..7 are 0, 1, 31, 32, 33, 47, 48, 63: low nibbles 0 1 15 0 1 15 0 15 (scales_l
# bytes 0x10 0x0F 0xF1 0xF0, low nibble first) and high bit pairs 0 0 1 2 2 2 3 3 (scales_h
# = 0xFA90); block scales d * (ls - 32) = -32 -31 -1 0 1 15 16 31.
_XS_REC = np.array([0x00, 0x3C, 0x90, 0xFA, 0x10, 0x0F, 0xF1, 0xF0], dtype=np.uint8)
_XS_SCALES = (-32.0, -31.0, -1.0, 0.0, 1.0, 15.0, 16.0, 31.0)


def test_iq4xs_block_scales_worked_example():
    assert tuple(oracle.iq4xs_block_scale(_XS_REC, j) for j in range(8)) == _XS_SCALES
    # one row of 256 columns: code 8 (level 1) everywhere but block 7, whose bytes are 0xF0
    # (even columns code 0 = -127, odd columns code 15 = 113)
    q = np.full((1, 1, 128), 0x88, dtype=np.uint8)
    q[0, 0, 112:] = 0xF0
    w = oracle.dequant(q, _XS_REC.reshape(1, 1, 1, 8))[0, 0]
    for j in range(7):
        assert np.all(w[32 * j:32 * j + 32] == _XS_SCALES[j])
    assert np.all(w[224::2] == -127 * 31.0) and np.all(w[225::2] == 113 * 31.0)
    qs, dd = synth.gen.draw_q8_0_stack(6, 2, 1, 3, 5, 512, wtype="iq4_xs")
    assert dd.shape == (3, 5, 2, 8) and dd.dtype == np.uint8
    assert np.array_equal(oracle.dequant(qs, dd), _numpy_dequant(qs, dd))


def test_mul_mat_id_iq4xs_is_iq4nl_on_the_block_scales():
    """With d a power of two (2^-8), every block scale d * (ls - 32) is exact in fp16, so an
    IQ4_XS matrix is the IQ4_NL matrix with those per-block scales and the same codes: the
    two oracle products must agree bit for bit."""
    rng = np.random.default_rng(14)
    E, N, K, T, k = 4, 12, 512, 6, 2
    qs, rec = synth.gen.draw_q8_0_stack(11, 2, 0, E, N, K, wtype="iq4_xs")
    rec[..., 0:2] = np.array([0x00, 0x1C], dtype=np.uint8)   # fp16 0x1C00 = 2^-8
    nl_d = _numpy_iq4xs_scales(rec).astype(np.float16)
    assert np.array_equal(nl_d.astype(np.float64), _numpy_iq4xs_scales(rec))
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    ids = rng.integers(-1, E + 1, size=(T, k)).astype(np.int32)
    rw = synth.draw_route_w(6, T, k)
    for r in (None, rw):
        got = oracle.mul_mat_id(qs, rec, x, "bf16", ids, r, 1)
        assert np.array_equal(got, oracle.mul_mat_id(qs, nl_d, x, "bf16", ids, r, 1))


def _dense_masked(W, X, ids, B):
    """Y_all[e][r] = W_e x_r for every expert and every src1 row (numpy matmul),
    then dst[t][s] = Y_all[ids[t][s]][t*B + s%B], zero for invalid ids."""
    E = W.shape[0]
    T, k = ids.shape
    Y_all = np.einsum("enk,rk->ern", W, X)
    out = np.zeros((T, k, W.shape[1]))
    for t in range(T):
        for s in range(k):
            e = ids[t, s]
            if 0 <= e < E:
                out[t, s] = Y_all[e, t * B + s % B]
    return out


@pytest.mark.parametrize("B_is_k", [False, True])
def test_mul_mat_id_q8_vs_dense_masked(B_is_k):
    rng = np.random.default_rng(11)
    E, N, K, T, k = 6, 40, 96, 9, 3
    qs, d = synth.gen.draw_q8_0_stack(7, 2, 0, E, N, K)
    B = k if B_is_k else 1
    x = synth.f32_to_bf16_bits(rng.standard_normal((T * B, K)).astype(np.float32))
    ids = rng.integers(-1, E + 1, size=(T, k)).astype(np.int32)
    rw = synth.draw_route_w(3, T, k)
    got = oracle.mul_mat_id(qs, d, x, "bf16", ids, None, B)
    ref = _dense_masked(_numpy_dequant(qs, d), synth.bf16_bits_to_f32(x).astype(np.float64), ids, B)
    assert normwise(got, ref) < 1e-13
    assert np.all(got[(ids < 0) | (ids >= E)] == 0.0)
    gw = oracle.mul_mat_id(qs, d, x, "bf16", ids, rw, B)
    refw = np.einsum("tsn,ts->tn", ref, rw.astype(np.float64))
    assert normwise(gw, refw) < 1e-13


def test_mul_mat_id_mxfp4_vs_dense_masked():
    rng = np.random.default_rng(12)
    E, N, K, T, k = 5, 24, 128, 7, 2
    qs, d = synth.gen.draw_q8_0_stack(8, 2, 0, E, N, K, wtype="mxfp4")
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    ids = rng.integers(-1, E + 1, size=(T, k)).astype(np.int32)
    rw = synth.draw_route_w(4, T, k)
    got = oracle.mul_mat_id(qs, d, x, "bf16", ids, None, 1)
    ref = _dense_masked(_numpy_dequant(qs, d), synth.bf16_bits_to_f32(x).astype(np.float64), ids, 1)
    assert normwise(got, ref) < 1e-13
    gw = oracle.mul_mat_id(qs, d, x, "bf16", ids, rw, 1)
    assert normwise(gw, np.einsum("tsn,ts->tn", ref, rw.astype(np.float64))) < 1e-13


def test_mul_mat_id_f32_tiny_vs_dense_masked():
    inp = synth.make_inputs("tiny")
    got = oracle.mul_mat_id(inp["w"], None, inp["x"], "f32", inp["ids"])
    ref = _dense_masked(inp["w"].astype(np.float64), inp["x"].astype(np.float64), inp["ids"], 1)
    assert normwise(got, ref) < 1e-14
    assert got.shape == (16, 2, 32)


def test_mul_mat_id_plain_gemm_when_one_expert():
    rng = np.random.default_rng(5)
    N, K, T = 33, 64, 7
    qs, d = synth.gen.draw_q8_0_stack(9, 2, 0, 1, N, K)
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    got = oracle.mul_mat_id(qs, d, x, "bf16", np.zeros((T, 1), np.int32))[:, 0, :]
    ref = synth.bf16_bits_to_f32(x).astype(np.float64) @ _numpy_dequant(qs, d)[0].T
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_mul_mat_id_doubling_x_doubles_exactly():
    rng = np.random.default_rng(8)
    E, N, K, T, k = 4, 16, 64, 5, 2
    qs, d = synth.gen.draw_q8_0_stack(4, 2, 0, E, N, K)
    xf = rng.standard_normal((T, K)).astype(np.float32)
    x1 = synth.f32_to_bf16_bits(xf)
    x2 = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(x1) * 2)
    ids = synth.draw_ids_uniform(1, T, E, k)
    assert np.array_equal(oracle.mul_mat_id(qs, d, x2, "bf16", ids),
                          2 * oracle.mul_mat_id(qs, d, x1, "bf16", ids))


# ------------------------------------------------------------------------- FFN

def _torch_dense_moe(inp):
    """Dense MoE in float64 with torch: every expert on every token, then masked
    by ids and weighted; shared experts added. Library matmul and silu only."""
    import torch
    F = torch.nn.functional

    def deq(name):
        return torch.from_numpy(_numpy_dequant(inp[name + "_qs"], inp[name + "_d"]))

    x = torch.from_numpy(synth.bf16_bits_to_f32(inp["x"]).astype(np.float64))
    G, U, D = deq("gate"), deq("up"), deq("down")
    E = G.shape[0]
    Y = torch.stack([(F.silu(x @ G[e].T) * (x @ U[e].T)) @ D[e].T for e in range(E)])  # [E][T][n_embd]
    ids = torch.from_numpy(inp["ids"].astype(np.int64))
    rw = torch.from_numpy(inp["route_w"].astype(np.float64))
    T, k = ids.shape
    out = torch.zeros(T, x.shape[1], dtype=torch.float64)
    for s in range(k):
        e = ids[:, s]
        ok = (e >= 0) & (e < E)
        sel = Y[e.clamp(0, E - 1), torch.arange(T)]
        out += torch.where(ok[:, None], rw[:, s:s + 1] * sel, torch.zeros_like(sel))
    if inp.get("sh_gate_qs") is not None:
        SG, SU, SD = deq("sh_gate"), deq("sh_up"), deq("sh_down")
        for j in range(SG.shape[0]):
            out += (F.silu(x @ SG[j].T) * (x @ SU[j].T)) @ SD[j].T
    return out.numpy()


@pytest.mark.parametrize("E,k,T,n_embd,n_ff,S", [(4, 4, 6, 64, 32, 0), (8, 3, 10, 96, 64, 2),
                                                  (16, 2, 5, 64, 96, 1)])
def test_ffn_vs_torch_dense_moe(E, k, T, n_embd, n_ff, S):
    inp = synth.make_custom_ffn(21 + E, E, k, T, n_embd, n_ff, S)
    got = oracle.ffn(inp)
    ref = _torch_dense_moe(inp)
    assert normwise(got, ref) < 1e-12


@pytest.mark.parametrize("E,k,T,n_embd,n_ff,S", [(4, 2, 5, 64, 96, 1), (8, 4, 3, 128, 64, 0)])
def test_ffn_mxfp4_vs_torch_dense_moe(E, k, T, n_embd, n_ff, S):
    inp = synth.make_custom_ffn(31 + E, E, k, T, n_embd, n_ff, S, wtype="mxfp4")
    assert inp["gate_qs"].dtype == np.uint8 and inp["gate_qs"].shape == (E, n_ff, n_embd // 2)
    assert normwise(oracle.ffn(inp), _torch_dense_moe(inp)) < 1e-12


@pytest.mark.parametrize("E,k,T,n_embd,n_ff,S", [(4, 2, 5, 64, 96, 1), (8, 4, 3, 128, 64, 0)])
def test_ffn_iq4nl_vs_torch_dense_moe(E, k, T, n_embd, n_ff, S):
    inp = synth.make_custom_ffn(41 + E, E, k, T, n_embd, n_ff, S, wtype="iq4_nl")
    assert inp["gate_qs"].dtype == np.uint8 and inp["gate_d"].dtype == np.float16
    assert normwise(oracle.ffn(inp), _torch_dense_moe(inp)) < 1e-12


@pytest.mark.parametrize("E,k,T,S", [(4, 2, 5, 1), (8, 4, 3, 0)])
def test_ffn_iq4xs_vs_torch_dense_moe(E, k, T, S):
    inp = synth.make_custom_ffn(45 + E, E, k, T, 256, 512, S, wtype="iq4_xs")
    assert inp["gate_d"].shape == (E, 512, 1, 8) and inp["down_d"].shape == (E, 256, 2, 8)
    assert normwise(oracle.ffn(inp), _torch_dense_moe(inp)) < 1e-12


def test_ffn_invalid_ids_contribute_nothing():
    inp = synth.make_custom_ffn(3, 6, 3, 7, 64, 32, 1)
    ids = inp["ids"].copy()
    ids[0, 1], ids[3, 0], ids[5, 2] = -1, 6, 1000
    inp["ids"] = ids
    assert normwise(oracle.ffn(inp), _torch_dense_moe(inp)) < 1e-12


def test_ffn_two_shared_equal_one_concatenated():
    inp = synth.make_custom_ffn(5, 8, 2, 6, 64, 32, 2)
    cat = dict(inp)
    cat["sh_gate_qs"] = inp["sh_gate_qs"].reshape(1, 64, 64)
    cat["sh_gate_d"] = inp["sh_gate_d"].reshape(1, 64, 2)
    cat["sh_up_qs"] = inp["sh_up_qs"].reshape(1, 64, 64)
    cat["sh_up_d"] = inp["sh_up_d"].reshape(1, 64, 2)
    cat["sh_down_qs"] = np.concatenate([inp["sh_down_qs"][0], inp["sh_down_qs"][1]], axis=1)[None]
    cat["sh_down_d"] = np.concatenate([inp["sh_down_d"][0], inp["sh_down_d"][1]], axis=1)[None]
    assert normwise(oracle.ffn(cat), oracle.ffn(inp)) < 1e-13


def test_ffn_one_hot_routing_isolates_a_slot():
    import torch
    F = torch.nn.functional
    inp = synth.make_custom_ffn(9, 8, 3, 5, 64, 32, 0)
    for s in range(3):
        one = dict(inp)
        rw = np.zeros_like(inp["route_w"])
        rw[:, s] = 1.0
        one["route_w"] = rw
        got = oracle.ffn(one)
        x = torch.from_numpy(synth.bf16_bits_to_f32(inp["x"]).astype(np.float64))
        ref = np.zeros_like(got)
        for t in range(5):
            e = inp["ids"][t, s]
            G, U, D = (torch.from_numpy(_numpy_dequant(inp[n + "_qs"][e], inp[n + "_d"][e]))
                       for n in ("gate", "up", "down"))
            ref[t] = ((F.silu(x[t] @ G.T) * (x[t] @ U.T)) @ D.T).numpy()
        assert normwise(got, ref) < 1e-13


def test_ffn_worked_example_closed_form():
    """Hand-built Q8_0 layer, n_embd = n_ff = 32, x = e_0 (bf16 1.0):
    expert 0: g_0 = 64*2^-6 = 1, u_0 = 32*2^-5 = 1, down column 0 = (c-16)*2^-4
        -> y_c = (c-16)/16 * silu(1) = (c-16)/16 * e/(1+e)
    expert 1: g_0 = -1, u_0 = 2, down column 0 = 1*2^-4
        -> y_c = silu(-1) * 2 / 16 = -1/(8(1+e))
    shared:   g_0 = 2, u_0 = 1, down column 0 = 16*2^-4 = 1 -> y_c = silu(2) = 2e^2/(1+e^2)
    every other gate row is zero, so silu(0) = 0 kills the rest.
    route_w = (0.75, 0.25) over experts (0, 1)."""
    n = 32

    def zeros():
        return np.zeros((1, n, n), np.int8), np.zeros((1, n, 1), np.uint16)

    def h(bits):
        return np.uint16(bits)

    gq, gd = [], []
    uq, ud = [], []
    dq, dd = [], []
    for g0, u0, dcol, dscale in ((64, 32, np.arange(n) - 16, 0x2C00), (-64, 64, np.ones(n), 0x2C00)):
        q, s = zeros(); q[0, 0, 0] = g0; s[0, 0, 0] = h(0x2400); gq.append(q); gd.append(s)   # 2^-6
        q, s = zeros(); q[0, 0, 0] = u0; s[0, 0, 0] = h(0x2800); uq.append(q); ud.append(s)   # 2^-5
        q, s = zeros(); q[0, :, 0] = dcol; s[0, :, 0] = h(dscale); dq.append(q); dd.append(s)  # 2^-4
    inp = {
        "gate_qs": np.concatenate(gq), "gate_d": np.concatenate(gd).view(np.float16),
        "up_qs": np.concatenate(uq), "up_d": np.concatenate(ud).view(np.float16),
        "down_qs": np.concatenate(dq), "down_d": np.concatenate(dd).view(np.float16),
        "x": np.array([[0x3F80] + [0] * (n - 1)], np.uint16), "xtype": "bf16",
        "ids": np.array([[0, 1]], np.int32), "route_w": np.array([[0.75, 0.25]], np.float32),
    }
    q, s = zeros(); q[0, 0, 0] = 64; s[0, 0, 0] = h(0x2800); inp["sh_gate_qs"], inp["sh_gate_d"] = q, s.view(np.float16)
    q, s = zeros(); q[0, 0, 0] = 32; s[0, 0, 0] = h(0x2800); inp["sh_up_qs"], inp["sh_up_d"] = q, s.view(np.float16)
    q, s = zeros(); q[0, :, 0] = 16; s[0, :, 0] = h(0x2C00); inp["sh_down_qs"], inp["sh_down_d"] = q, s.view(np.float16)
    e = math.e
    c = np.arange(n)
    want = 0.75 * (c - 16) / 16 * e / (1 + e) + 0.25 * (-1 / (8 * (1 + e))) + 2 * e * e / (1 + e * e)
    got = oracle.ffn(inp)[0]
    np.testing.assert_allclose(got, want, rtol=0, atol=4e-16 * 4)


# ------------------------------------------------------------------- generator

def test_generator_is_deterministic_and_in_range():
    a = synth.make_custom_ffn(17, 8, 2, 9, 64, 32, 1)
    b = synth.make_custom_ffn(17, 8, 2, 9, 64, 32, 1)
    for key in a:
        if isinstance(a[key], np.ndarray):
            assert np.array_equal(a[key], b[key]), key
    assert a["gate_qs"].min() >= -127 and a["gate_qs"].max() <= 127
    d = a["gate_d"].astype(np.float64)
    assert d.min() >= 0.5e-3 - 1e-6 and d.max() <= 1.5e-3 + 1e-6
    assert np.allclose(a["route_w"].astype(np.float64).sum(axis=1), 1.0, atol=1e-6)
    assert all(len(set(r)) == len(r) for r in a["ids"].tolist())   # without replacement


def test_zipf_routing_is_skewed():
    cfg = synth.CONFIGS["skew"]
    ids = synth.draw_ids_zipf(cfg.seed, cfg.n_tokens, cfg.n_experts, cfg.n_used, cfg.zipf_s)
    cnt = np.bincount(ids.ravel(), minlength=cfg.n_experts)
    assert cnt.sum() == cfg.n_tokens * cfg.n_used
    assert cnt.max() > 10 * cnt.mean() / 1.5 and cnt.min() < cnt.mean() / 2
    assert all(len(set(r)) == len(r) for r in ids.tolist())


# ---------------------------------------------------------------------- router
# The step ahead of the op: ids and routing weights from router logits (top-k,
# softmax renormalised over the picks).

def _softmax64(z):
    z = np.asarray(z, np.float64)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


@pytest.mark.parametrize("T,E,k,seed", [(9, 8, 2, 1), (40, 64, 6, 2), (7, 256, 8, 3), (3, 1024, 32, 4),
                                        (5, 33, 33, 5)])
def test_router_topk_vs_sort(T, E, k, seed):
    """Selection against a full stable sort by (-logit, index); weights against a
    softmax of the selected logits written with numpy."""
    lg = synth.draw_router_logits(seed, T, E)
    ids, w = oracle.router_topk(lg, k)
    order = np.array([np.lexsort((np.arange(E), -lg[t].astype(np.float64))) for t in range(T)])
    assert np.array_equal(ids, order[:, :k])
    want = _softmax64(np.take_along_axis(lg, ids, axis=1))
    np.testing.assert_allclose(w, want, rtol=1e-14, atol=0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)


def test_router_ties_go_to_the_lower_index():
    # logits from a 3-value set: many ties; picks among equals in index order
    lg = np.random.default_rng(7).integers(0, 3, size=(50, 40)).astype(np.float32)
    ids, w = oracle.router_topk(lg, 12)
    for t in range(50):
        row = lg[t]
        want = sorted(range(40), key=lambda e: (-row[e], e))[:12]
        assert ids[t].tolist() == want
        vals = row[ids[t]]
        # equal logits get equal weights
        for a in range(12):
            for b in range(12):
                if vals[a] == vals[b]:
                    assert w[t, a] == w[t, b]


def test_router_shift_invariance_and_special_cases():
    # logits on a 2^-10 grid, so adding 8 is exact in float32
    lg = (np.round(synth.draw_router_logits(11, 20, 32) * 1024) / 1024).astype(np.float32)
    ids, w = oracle.router_topk(lg, 4)
    ids2, w2 = oracle.router_topk(lg + np.float32(8.0), 4)
    assert np.array_equal(ids, ids2)
    np.testing.assert_allclose(w, w2, rtol=1e-12)
    ids1, w1 = oracle.router_topk(lg, 1)
    assert np.array_equal(ids1[:, 0], np.argmax(lg, axis=1)) and np.all(w1 == 1.0)
    idsE, wE = oracle.router_topk(lg, 32)                 # k = E: every expert, by logit
    assert all(sorted(r) == list(range(32)) for r in idsE.tolist())
    np.testing.assert_allclose(wE, np.take_along_axis(_softmax64(lg), idsE, axis=1), rtol=1e-13)


def test_router_worked_example():
    """Hand-computed: logits (1, ln 3, 0, ln 3) with k = 3 pick expert 1, then its
    equal expert 3, then expert 0, weighted e^{ln3}, e^{ln3}, e^1 over their sum."""
    l3 = np.float32(math.log(3.0))
    lg = np.array([[1.0, l3, 0.0, l3]], np.float32)
    ids, w = oracle.router_topk(lg, 3)
    assert ids.tolist() == [[1, 3, 0]]
    a = math.exp(float(l3))
    s = 2 * a + math.e
    np.testing.assert_allclose(w[0], [a / s, a / s, math.e / s], rtol=1e-15)


def test_router_nan_ranks_below_minus_inf():
    """Hand-derived: NaN ranks strictly below -inf (a NaN at index 0 against -inf at
    index 5), and non-finite picks get weight 0 when the largest pick is finite."""
    nan, inf = float("nan"), float("inf")
    lg = np.array([[nan, 1.0, 2.0, 3.0, 4.0, -inf]], np.float32)
    ids, w = oracle.router_topk(lg, 6)
    assert ids.tolist() == [[4, 3, 2, 1, 5, 0]]
    e = np.exp(np.array([0.0, -1.0, -2.0, -3.0]))
    np.testing.assert_allclose(w[0, :4], e / e.sum(), rtol=1e-15)
    assert w[0, 4] == 0.0 and w[0, 5] == 0.0
    # NaNs among themselves: lower index first, after every number
    lg2 = np.array([[nan, -inf, nan, 0.5, -inf]], np.float32)
    ids2, _ = oracle.router_topk(lg2, 5)
    assert ids2.tolist() == [[3, 1, 4, 0, 2]]


def test_router_non_finite_largest_pick():
    """Hand-derived limits of the softmax: an all-NaN row and an all -inf row weight
    every pick 1/k; with +inf picks, those share the weight and the rest get 0."""
    nan, inf = float("nan"), float("inf")
    ids, w = oracle.router_topk(np.full((1, 5), nan, np.float32), 3)
    assert ids.tolist() == [[0, 1, 2]]
    assert np.all(w == 1.0 / 3.0)
    ids, w = oracle.router_topk(np.array([[-inf, nan, -inf, -inf]], np.float32), 3)
    assert ids.tolist() == [[0, 2, 3]]
    assert np.all(w == 1.0 / 3.0)
    ids, w = oracle.router_topk(np.array([[-inf, nan, -inf]], np.float32), 3)
    assert ids.tolist() == [[0, 2, 1]]          # the NaN last, weighted as -inf
    assert np.all(w == 1.0 / 3.0)
    ids, w = oracle.router_topk(np.array([[1.0, inf, 3.0, inf, nan]], np.float32), 3)
    assert ids.tolist() == [[1, 3, 2]]
    assert w.tolist() == [[0.5, 0.5, 0.0]]


# ------------------------------------------------------- quantized-activation path
# Activation blocks of 32 columns: d = max|x|/127 (float32), q = rint(x/d) (float32,
# ties to even), value d*q.

def test_quantize_act_hand_derived():
    """A block whose largest value is 508 = 127 * 4 has d = 4 exactly, so every code is
    x/4 rounded by hand, ties to even: 63.5 -> 64, -0.5 -> 0, 1.5 -> 2, 2.5 -> 2,
    3.5 -> 4. A block of zeros has d = 0 and q = 0. Values are exact in bf16."""
    blk = [508.0, 254.0, -2.0, 3.0, 1.0, 2.5, -2.5, 3.5, 6.0, -6.0, 10.0, 14.0] + [0.0] * 20
    want = [127, 64, 0, 1, 0, 1, -1, 1, 2, -2, 2, 4] + [0] * 20
    x = np.array([blk + [0.0] * 32], np.float32)
    for typ, arr in (("f32", x), ("bf16", synth.f32_to_bf16_bits(x))):
        q, d = oracle.quantize_act(arr, typ)
        assert d.tolist() == [[4.0, 0.0]], typ
        assert q[0, :32].tolist() == want, typ
        assert not q[0, 32:].any()


def test_quantize_act_properties():
    """On random blocks: the largest element gets code +-127, codes keep the sign,
    |d*q - x| <= d/2 (rounding to the nearest code), and scaling a block by a power of
    two scales d by it and keeps the codes."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((40, 256)) * rng.uniform(0.01, 100, size=(40, 1))).astype(np.float32)
    q, d = oracle.quantize_act(x, "f32")
    xb = x.reshape(40, 8, 32).astype(np.float64)
    qb = q.reshape(40, 8, 32).astype(np.float64)
    db = d.astype(np.float64)[:, :, None]
    arg = np.abs(xb).argmax(axis=2)
    assert np.all(np.abs(np.take_along_axis(qb, arg[:, :, None], 2)) == 127)
    assert np.all((np.sign(qb) == np.sign(xb)) | (qb == 0))
    assert np.all(np.abs(db * qb - xb) <= db / 2 * (1 + 1e-6))
    assert np.abs(q).max() <= 127
    q2, d2 = oracle.quantize_act(x * np.float32(8.0), "f32")
    assert np.array_equal(q2, q) and np.array_equal(d2, d * np.float32(8.0))


def test_mul_mat_id_q8act_reduces_to_plain_when_quantization_is_exact():
    """Integer activations whose blocks each hold +-127 quantize exactly (d = 1, q = x),
    so the quantized-activation mul_mat_id must equal the plain one bit for bit, per slot
    and weighted, for one src1 row per token and one per slot."""
    rng = np.random.default_rng(8)
    E, k, T, K, N = 6, 3, 7, 96, 40
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    ids[2, 1] = -1
    inp = synth.make_custom_mmid(4, E, k, T, K, N, ids=ids)
    for B in (1, k):
        x = rng.integers(-127, 128, size=(T * B, K)).astype(np.float32)
        x[:, ::32] = 127.0
        q, d = oracle.quantize_act(x, "f32")
        assert np.all(d == 1.0) and np.array_equal(q.astype(np.float32), x)
        for rw in (None, inp["route_w"]):
            got = oracle.mul_mat_id_q8act(inp["w_qs"], inp["w_d"], q, d, ids, rw, B)
            ref = oracle.mul_mat_id(inp["w_qs"], inp["w_d"], x, "f32", ids, rw, B)
            assert np.array_equal(got, ref), (B, rw is None)


def test_mul_mat_id_q8act_equals_dense_masked_product():
    """Random activations: equals the dense all-experts product of the dequantized
    weights with the dequantized activations (numpy float64 matmul), masked by ids."""
    rng = np.random.default_rng(9)
    E, k, T, K, N = 5, 2, 9, 128, 24
    inp = synth.make_custom_mmid(6, E, k, T, K, N)
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    q, d = oracle.quantize_act(x, "bf16")
    xa = q.astype(np.float64) * np.repeat(d.astype(np.float64), 32, axis=1)
    W = oracle.dequant(inp["w_qs"], inp["w_d"])
    dense = np.einsum("enc,tc->ten", W, xa)
    want = np.stack([dense[t, inp["ids"][t]] for t in range(T)])
    got = oracle.mul_mat_id_q8act(inp["w_qs"], inp["w_d"], q, d, inp["ids"])
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def _bf16_round64(h):
    m, e = np.frexp(h)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def test_ffn_q8act_composition():
    """The quantized-activation FFN assembled from its steps with numpy: x quantized
    (the pinned quantizer), gate/up products of the dequantized weights (numpy float64
    matmul), silu(g)*u rounded to bf16 and quantized, the down product, the routing
    weights, then the shared experts."""
    E, k, T, n_embd, n_ff, S = 6, 2, 5, 96, 64, 1
    ids = np.random.default_rng(3).integers(0, E, size=(T, k)).astype(np.int32)
    ids[1, 1] = E + 2
    inp = synth.make_custom_ffn(12, E, k, T, n_embd, n_ff, S, ids=ids)
    got = oracle.ffn(inp, act_quant=True)
    Wg, Wu, Wd = (oracle.dequant(inp[n + "_qs"], inp[n + "_d"]) for n in ("gate", "up", "down"))
    Sg, Su, Sd = (oracle.dequant(inp["sh_" + n + "_qs"], inp["sh_" + n + "_d"]) for n in ("gate", "up", "down"))
    deq = lambda q, d: q.astype(np.float64) * np.repeat(d.astype(np.float64), 32, axis=1)
    xq = deq(*oracle.quantize_act(inp["x"], "bf16"))

    def expert(G, U, D, t):
        g, u = G @ xq[t], U @ xq[t]
        h = _bf16_round64(g / (1.0 + np.exp(-g)) * u).astype(np.float32)[None, :]
        return D @ deq(*oracle.quantize_act(h, "f32"))[0]

    want = np.zeros((T, n_embd))
    for t in range(T):
        for s in range(k):
            e = ids[t, s]
            if 0 <= e < E:
                want[t] += float(inp["route_w"][t, s]) * expert(Wg[e], Wu[e], Wd[e], t)
        want[t] += expert(Sg[0], Su[0], Sd[0], t)
    assert np.abs(got - want).max() <= 1e-12 * np.abs(want).max()
    # and it stays close to the unquantized layer (8-bit codes on both activations)
    plain = oracle.ffn(inp)
    assert np.abs(got - plain).max() / np.abs(plain).max() < 2e-2
