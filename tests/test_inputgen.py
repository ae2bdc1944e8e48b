"""The seeded input generator: Philox known answers, the normal table, the encoders and the
layer recipe (margin rule, Zipf popularity)."""
import numpy as np
import torch

from inputgen import layers as L
from inputgen import philox as px


def test_philox4x32_10_known_answers():
    """Known-answer vectors of Philox4x32-10 published with the Random123 library."""
    kat = [
        ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
        ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
        ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
         (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
    ]
    for ctr, key, out in kat:
        got = px.philox4x32_10(*[np.array([c], np.uint32) for c in ctr], *key)
        assert tuple(int(g[0]) for g in got) == out


def test_word_stream_is_position_independent():
    a = px.uniform_words(3, 4, 5, 0, 103)
    b = px.uniform_words(3, 4, 5, 37, 40)
    assert np.array_equal(a[37:77], b)
    assert not np.array_equal(px.uniform_words(3, 4, 6, 0, 8), a[:8])


def test_normal_table_symmetric_and_moments():
    t = px.NORMAL_TABLE.astype(np.int64)
    assert np.array_equal(t, -t[::-1])
    assert np.all(np.diff(t) > 0) and np.all(np.diff(px.NORMAL_TAIL.astype(np.int64)) > 0)
    z = px.normal_f32(9, 9, 0, 0, 1 << 20)
    assert abs(z.mean()) < 5e-3 and abs(z.var() - 1) < 6e-3
    # exact multiples of 2^-20
    assert np.all(z * 2 ** 20 == np.round(z * 2 ** 20))


def test_bf16_encoder_matches_torch_rne():
    v = px.normal_f32(1, 2, 0, 0, 100000) * np.float32(3.7)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(px.f32_to_bf16_bits(v), ref)


def test_e4m3fn_encoder_matches_torch_in_range():
    v = px.normal_f32(1, 3, 0, 0, 200000) * np.float32(120.0)
    v = np.concatenate([v[np.abs(v) <= 448], np.float32([448, -448, 2 ** -9, 2 ** -10, 3 * 2 ** -11, 0])])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = px.f32_to_e4m3fn(v)
    # torch keeps the sign of a value that rounds to zero; the encoder writes +0
    zero = (ref & 0x7F) == 0
    assert np.array_equal(got[~zero], ref[~zero]) and np.all(got[zero] == 0)
    # saturation instead of NaN
    assert px.f32_to_e4m3fn(np.float32([1000.0, -500.0, 464.0])).tolist() == [0x7E, 0xFE, 0x7E]


def test_e2m1_encoder_is_nearest_ties_to_even():
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    vals = np.concatenate([np.linspace(-7, 7, 2801), (grid[1:] + grid[:-1]) / 2])
    codes = px.e2m1_code(vals.astype(np.float32))
    for v, c in zip(vals, codes):
        mag = grid[c & 7] * (-1 if c & 8 else 1)
        d = np.abs(np.abs(v) - grid)
        best = np.flatnonzero(np.isclose(d, d.min()))
        if abs(v) > 6:
            assert c & 7 == 7
        elif len(best) == 1:
            assert c & 7 == best[0]
        else:  # tie: the even code
            assert c & 7 == [b for b in best if b % 2 == 0][0]
        assert np.sign(mag) in (0, np.sign(v))


def test_mxfp4_scale_puts_block_max_in_4_to_8():
    w = px.normal_f32(2, 2, 0, 0, 64 * 32).reshape(64, 32) * np.float32(0.02)
    codes, E = px.quantize_mxfp4_k32(w)
    amax = np.abs(w.reshape(2, 32, 32)).max(axis=1)
    r = amax / np.ldexp(1.0, E.astype(np.int64) - 127)
    assert np.all((r >= 4) & (r < 8))


def test_mxfp8_scale_puts_block_max_in_256_to_512_saturating_at_448():
    """OCP MXFP8 weights: E = floor(log2 amax) - 8, so the scaled block maximum lies in [256, 512)
    and codes above 448 saturate; every other element is the nearest E4M3 value."""
    w = px.normal_f32(2, 3, 0, 0, 64 * 32).reshape(64, 32) * np.float32(0.02)
    codes, E = px.quantize_mxfp8_k32(w)
    amax = np.abs(w.reshape(2, 32, 32)).max(axis=1)
    scale = np.ldexp(1.0, E.astype(np.int64) - 127)
    r = amax / scale
    assert np.all((r >= 256) & (r < 512))
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    scaled = w.astype(np.float64) / np.repeat(scale, 32, axis=0)
    assert np.all(np.abs(dec) <= 448)
    inside = np.abs(scaled) <= 448
    # nearest: at most half a step of the E4M3 grid (2^(e-3) for |v| in [2^e, 2^(e+1)), 2^-9 below 2^-6)
    e = np.floor(np.log2(np.maximum(np.abs(scaled), 2.0 ** -6)))
    assert np.all(np.abs(dec - scaled)[inside] <= (2.0 ** (e - 4))[inside] + 1e-12)
    assert np.all(dec[~inside] == np.sign(scaled[~inside]) * 448)


def test_int8_per_channel_scale_and_codes():
    """Int8 weights: s = amax / 127 per output column, the column maximum at code +-127, every
    code the nearest integer to w / s."""
    w = px.normal_f32(2, 4, 0, 0, 64 * 48).reshape(64, 48) * np.float32(0.02)
    codes, s = px.quantize_int8_per_channel(w)
    assert s.shape == (48,) and codes.dtype == np.int8
    assert np.allclose(s, np.abs(w).max(axis=0) / 127, rtol=1e-6)
    assert np.all(np.abs(codes.astype(np.int64)).max(axis=0) == 127)
    assert np.all(np.abs(codes - w.astype(np.float64) / s) <= 0.5 + 1e-5)


def test_generation_is_deterministic_and_seeded():
    s = L.CONFIGS["c1"]
    a, b = L.router_inputs(s), L.router_inputs(s)
    assert np.array_equal(a["x"], b["x"]) and np.array_equal(a["Wr"], b["Wr"])
    c = L.router_inputs(s.replace(seed=99))
    assert not np.array_equal(a["x"], c["x"])
    e1 = L.expert_weights(s, "routed", 3)
    assert np.array_equal(e1["down"], L.expert_weights(s, "routed", 3)["down"])
    assert not np.array_equal(e1["down"], L.expert_weights(s, "routed", 4)["down"])


def test_margin_rule_holds():
    s = L.LayerSpec("m", T=200, H=128, E=64, k=6, I=128, router="zipf", zipf_alpha=1.0,
                    calib_tokens=512, seed=4, margin=5e-3)
    r = L.router_inputs(s)
    logits = L.act_to_f64(r["x"], "bf16") @ L.act_to_f64(r["Wr"], "bf16") + r["bias"]
    assert np.all(L.topk_gap(logits, s.k) >= s.margin)
    assert (r["attempts"] > 0).any()  # the rule did fire at this margin


def test_zipf_targets():
    order = np.arange(256)
    for T, alpha in ((256, 1.0), (16384, 1.2)):
        t = L.zipf_targets(256, 8, T, alpha, order)
        assert abs(t.sum() - T * 8) < 1e-6 and t.max() <= T + 1e-9
        assert np.all(np.diff(t) <= 1e-9)  # rank order
    t = L.zipf_targets(256, 8, 16384, 1.2, order)
    assert t[0] == t[1] == 16384  # the two hottest experts are capped at one per token


def test_zipf_popularity_is_skewed():
    s = L.CONFIGS["c3"].replace(H=256, calib_tokens=2048)
    r = L.router_inputs(s)
    logits = L.act_to_f64(r["x"], "bf16") @ L.act_to_f64(r["Wr"], "bf16") + r["bias"]
    sel = np.argsort(-logits, axis=1)[:, :s.k]
    cnt = np.sort(np.bincount(sel.ravel(), minlength=s.E))[::-1]
    assert cnt[0] > 0.8 * s.T and cnt[0] > 20 * cnt.mean() * 0.5
    assert 200 <= (cnt > 0).sum() <= 250  # about 233 of 256 experts active at T = 256
