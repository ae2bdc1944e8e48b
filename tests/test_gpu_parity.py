"""Parity of the HIP path (through the C ABI) with the CPU oracle, element by element on the
same seeded inputs. Routing indices, offsets and the permutation must be identical; outputs
must meet the relative Frobenius bound of their precision (1e-5 fp32, 1e-2 bf16, 4e-2 fp8 and
MXFP4); routing weights within 1e-5."""
import numpy as np
import pytest
import torch

from expert_ffn_layer_amd import native as N
from expert_ffn_layer_amd.layer import PackedLayer, pack
from inputgen import gpu as G
from inputgen import layers as L
from inputgen import philox as px
from oracle import oracle as O

from _gpu import (build, host_weights, oracle_ffn_rows, oracle_full, oracle_tokens, rel_fro, run, say, spec_tol_of,
                  to_f64, tol_of)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    N.load()
    G.lib()
    yield


# ------------------------------------------------------------------ the input generator

@pytest.mark.parametrize("fmt", ["f32", "bf16", "fp8", "mxfp4", "mxfp8a8", "int8"])
def test_gpu_generator_is_bit_identical_to_numpy(fmt):
    K, Nn = 256, 384
    c, s = G.alloc_matrices(fmt, 2, K, Nn, DEV)
    G.fill_matrices(c, s, fmt, 7, 17, 3, K, Nn, K)
    for m in range(2):
        ref = L.store_matrix(L.draw_f32(7, 17, 3 + m, (K, Nn), K), fmt)
        assert np.array_equal(G.to_numpy_stored(c[m]), ref["w"])
        if s is not None:
            assert np.array_equal(G.to_numpy_stored(s[m]), ref["scale"])


def test_gpu_activations_bit_identical():
    spec = L.CONFIGS["c2"].replace(T=40, H=1024)
    x = G.to_numpy_stored(G.activations_attempt0(spec, DEV))
    assert np.array_equal(x, L.store_act(L.draw_f32(spec.seed, L.TID_X, 0, (spec.T, spec.H)), "bf16"))


# ------------------------------------------------------------------ packing

@pytest.mark.parametrize("fmt", ["f32", "bf16", "fp8", "mxfp4", "mxfp8a8", "int8"])
def test_pack_layout(fmt):
    """Unpack the packed bytes with numpy following the documented layout."""
    K, Nn = 256, 384
    c, s = G.alloc_matrices(fmt, 1, K, Nn, DEV)
    G.fill_matrices(c, s, fmt, 3, 16, 0, K, Nn, K)
    packed, pscale = pack(fmt, c, s, K, Nn)
    torch.cuda.synchronize()
    KP = {"f32": 16, "bf16": 32, "fp8": 64, "mxfp4": 128, "mxfp8a8": 64, "int8": 64}[fmt]
    NT, KT = Nn // 16, K // KP
    NTp = (Nn + 255) // 256 * 16  # features padded to a multiple of 256 with zero packets
    raw = packed.cpu().numpy().reshape(NTp, KT, 64, 16)
    assert not raw[NT:].any()
    raw = raw[:NT]
    stored = G.to_numpy_stored(c[0])
    if fmt == "mxfp4":
        codes = np.empty((K, Nn), np.uint8)
        codes[:, 0::2], codes[:, 1::2] = stored & 15, stored >> 4
        lanes = np.stack([raw & 15, raw >> 4], axis=-1).reshape(NT, KT, 64, 32)
    elif fmt in ("fp8", "mxfp8a8"):
        codes, lanes = stored, raw
    elif fmt == "int8":
        codes, lanes = stored, raw.view(np.int8)
    else:
        dt = np.float32 if fmt == "f32" else np.uint16
        codes, lanes = stored, raw.view(dt).reshape(NT, KT, 64, -1)
    run_len = KP // 4
    rebuilt = np.empty((K, Nn), codes.dtype)
    for l in range(64):
        n = np.arange(NT)[:, None] * 16 + l % 16
        for kt in range(KT):
            k0 = kt * KP + (l // 16) * run_len
            rebuilt[k0:k0 + run_len, n[:, 0]] = lanes[:, kt, l, :run_len].T
    assert np.array_equal(rebuilt, codes)
    if fmt == "fp8":
        assert np.array_equal(pscale.cpu().numpy().view(np.float32).reshape(s[0].shape), s[0].cpu().numpy())
    if fmt == "mxfp4":
        ps = pscale.cpu().numpy().reshape(NTp, KT, 64)[:NT]
        sc = G.to_numpy_stored(s[0])
        for l in range(64):
            for kt in range(KT):
                assert np.array_equal(ps[:, kt, l], sc[(kt * KP + (l // 16) * 32) // 32, np.arange(NT) * 16 + l % 16])
    if fmt == "int8":
        ps = pscale.cpu().numpy().view(np.float32)
        assert ps.size == NTp * 16
        assert np.array_equal(ps[:Nn], s[0].cpu().numpy()) and not ps[Nn:].any()
    if fmt == "mxfp8a8":
        # one exponent byte per lane per pair of packets: lane l of pair kt2 holds the exponent of
        # feature l % 16 of the tile, elements kt2 * 128 + (l // 16) * 32 .. + 32
        ps = pscale.cpu().numpy().reshape(NTp, K // 128, 64)[:NT]
        sc = G.to_numpy_stored(s[0])
        for l in range(64):
            for kt2 in range(K // 128):
                assert np.array_equal(ps[:, kt2, l], sc[kt2 * 4 + l // 16, np.arange(NT) * 16 + l % 16])


# ------------------------------------------------------------------ whole layer, small shapes

SMALL = [
    # name, spec overrides
    ("c1", L.CONFIGS["c1"]),
    ("bf16-shared-zipf", L.LayerSpec("s1", T=37, H=512, E=16, k=4, I=256, shared=True, router="zipf",
                                     zipf_alpha=1.0, calib_tokens=512, seed=31)),
    ("bf16-big-groups", L.LayerSpec("s2", T=300, H=256, E=4, k=2, I=128, seed=32)),
    ("fp8-shared", L.LayerSpec("s3", T=50, H=512, E=8, k=3, I=256, shared=True, w_routed="fp8",
                               w_shared="fp8", router="zipf", zipf_alpha=1.2, calib_tokens=512, seed=33)),
    ("mxfp4-bf16-shared", L.LayerSpec("s4", T=20, H=512, E=24, k=6, I=384, shared=True, w_routed="mxfp4",
                                      w_shared="bf16", seed=34)),
    ("one-token", L.LayerSpec("s5", T=1, H=256, E=8, k=8, I=128, seed=35)),
    ("k1-f32", L.LayerSpec("s6", T=70, H=384, E=3, k=1, I=256, act="f32", w_routed="f32", w_shared="f32",
                           shared=True, seed=36)),
    ("wide-E", L.LayerSpec("s7", T=9, H=256, E=300, k=7, I=128, seed=37)),
    # groups of several hundred rows: whole 256-row tiles, a padded last tile and a <= 128-row
    # remainder in the prefill kernel
    ("ragged-groups", L.LayerSpec("s8", T=600, H=512, E=6, k=2, I=256, shared=True, router="zipf",
                                  zipf_alpha=1.0, calib_tokens=512, seed=38)),
    ("ragged-groups-fp8", L.LayerSpec("s9", T=520, H=1024, E=5, k=2, I=512, shared=True, w_routed="fp8",
                                      w_shared="fp8", router="zipf", zipf_alpha=0.8, calib_tokens=512,
                                      seed=39)),
    # enough tokens for the router scores to run on the 256 x 256 MFMA tiles (split along H), with
    # a ragged last row tile
    ("many-tokens-router", L.LayerSpec("s10", T=2304, H=512, E=256, k=2, I=256, seed=40)),
    # MXFP4 routed experts in the prefill kernel, with a bf16 shared expert (one launch per
    # format) and with an MXFP4 one; fp8 routed with a bf16 shared expert
    ("mxfp4-bf16-prefill", L.LayerSpec("s11", T=600, H=512, E=6, k=2, I=256, shared=True, w_routed="mxfp4",
                                       w_shared="bf16", router="zipf", zipf_alpha=1.0, calib_tokens=512,
                                       seed=41)),
    ("mxfp4-prefill", L.LayerSpec("s12", T=520, H=1024, E=5, k=2, I=512, shared=True, w_routed="mxfp4",
                                  w_shared="mxfp4", seed=42)),
    ("fp8-bf16-prefill", L.LayerSpec("s13", T=600, H=512, E=6, k=2, I=256, shared=True, w_routed="fp8",
                                     w_shared="bf16", seed=43)),
    # W4A8 routed experts (MXFP4 weights x MXFP8 activations on the block-scaled MFMA): ragged
    # groups with a bf16 shared expert, and many small groups (half items) without one
    ("w4a8-bf16-shared", L.LayerSpec("s14", T=600, H=512, E=6, k=2, I=256, shared=True, w_routed="mxfp4a8",
                                     w_shared="bf16", router="zipf", zipf_alpha=1.0, calib_tokens=512,
                                     seed=44)),
    ("w4a8-small-groups", L.LayerSpec("s15", T=96, H=1024, E=24, k=4, I=512, w_routed="mxfp4a8", seed=45)),
    # the hybrid MXFP8-MXFP4 layer: W4A8 routed experts and a W8A8 MXFP8 shared expert, whose
    # 256-row items leave a row half empty (T = 300: 44 rows in the last item; T = 1: one row)
    ("hybrid-mx", L.LayerSpec("s16", T=300, H=512, E=6, k=2, I=256, shared=True, w_routed="mxfp4a8",
                              w_shared="mxfp8a8", router="zipf", zipf_alpha=1.0, calib_tokens=512, seed=46)),
    ("hybrid-mx-T200", L.LayerSpec("s17", T=200, H=1024, E=8, k=3, I=512, shared=True, w_routed="mxfp4a8",
                                   w_shared="mxfp8a8", seed=47)),
    ("hybrid-mx-one-token", L.LayerSpec("s18", T=1, H=512, E=4, k=2, I=256, shared=True, w_routed="mxfp4a8",
                                        w_shared="mxfp8a8", seed=48)),
    # Int8 W8A8 experts (int8 x int8 MFMA, exact int32 sums): ragged Zipf groups with an int8 shared
    # expert, many small groups without one, a single token
    ("int8-shared", L.LayerSpec("s19", T=600, H=512, E=6, k=2, I=256, shared=True, w_routed="int8",
                                w_shared="int8", router="zipf", zipf_alpha=1.0, calib_tokens=512, seed=49)),
    ("int8-small-groups", L.LayerSpec("s20", T=96, H=1024, E=24, k=4, I=512, w_routed="int8", seed=50)),
    ("int8-one-token", L.LayerSpec("s21", T=1, H=512, E=4, k=2, I=256, shared=True, w_routed="int8",
                                   w_shared="int8", seed=51)),
    # the limits the ABI accepts: 1024 experts (16 scores per lane of the top-k wave) and k = 16,
    # with a shared expert as group 1025 of the plan
    ("max-E-and-k", L.LayerSpec("s22", T=40, H=512, E=1024, k=16, I=256, shared=True, seed=52)),
    # the degenerate layer: one expert, k = 1, every token's weight 1 (a dense SwiGLU plus the
    # shared expert)
    ("single-expert", L.LayerSpec("s23", T=33, H=512, E=1, k=1, I=256, shared=True, seed=53)),
]


def _prefill_ok(spec):
    fmts = ("bf16", "fp8", "mxfp4")
    shared_fmts = fmts + (("mxfp8a8",) if spec.w_routed == "mxfp4a8" else ("int8",) if spec.w_routed == "int8" else ())
    return (spec.act == "bf16" and spec.w_routed in fmts + ("mxfp4a8", "int8")
            and (not spec.shared or spec.w_shared in shared_fmts) and spec.I % 256 == 0 and spec.H % 512 == 0)


@pytest.mark.parametrize("name,spec", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("path", ["auto", "decode", "prefill"])
def test_layer_small(name, spec, path):
    if path == "prefill" and not _prefill_ok(spec):
        pytest.skip("the prefill kernel takes bf16 activations, I % 256 == 0 and H % 512 == 0")
    say("layer", name, path, spec)
    lay, pl = build(spec, DEV, path)
    y, idx, w = run(spec, lay, pl)
    ref = oracle_full(spec, lay)
    assert np.array_equal(idx.cpu().numpy(), ref["topk_idx"])
    assert np.max(np.abs(w.cpu().numpy() - ref["topk_w"])) <= 1e-5
    err = rel_fro(to_f64(y), ref["y"])
    say("  rel. Frobenius error %.3e (bound %.0e)" % (err, tol_of(spec)))
    assert err <= tol_of(spec)
    # deterministic: a second call gives the same bits
    y2, idx2, w2 = run(spec, lay, pl)
    assert torch.equal(y, y2) and torch.equal(idx, idx2) and torch.equal(w, w2)


def test_layer_zero_tokens_is_a_no_op():
    spec = L.CONFIGS["c1"]
    lay, pl = build(spec, DEV)
    pl.set_tokens(0)
    y = torch.full((1, spec.H), 7.0, device=DEV)
    pl.forward(lay["x"], None, y)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


# ------------------------------------------------------------------ the four stages one by one

STAGE_SPECS = [
    ("bf16", L.LayerSpec("st", T=45, H=512, E=12, k=3, I=256, shared=True, router="zipf", zipf_alpha=1.0,
                         calib_tokens=512, seed=41)),
    ("mxfp4+bf16", L.LayerSpec("st4", T=20, H=512, E=24, k=6, I=384, shared=True, w_routed="mxfp4",
                               w_shared="bf16", seed=34)),
    ("fp8", L.LayerSpec("st8", T=40, H=512, E=8, k=2, I=256, shared=True, w_routed="fp8", w_shared="fp8",
                        seed=43)),
    ("mxfp4", L.LayerSpec("st44", T=24, H=512, E=8, k=2, I=256, shared=True, w_routed="mxfp4",
                          w_shared="mxfp4", seed=44)),
    ("mxfp4+bf16-T40", L.LayerSpec("st45", T=40, H=512, E=24, k=6, I=384, shared=True, w_routed="mxfp4",
                                   w_shared="bf16", seed=45)),
    ("bf16+mxfp4", L.LayerSpec("st46", T=20, H=512, E=24, k=6, I=384, shared=True, w_routed="bf16",
                               w_shared="mxfp4", seed=46)),
    ("fp8+bf16", L.LayerSpec("st47", T=20, H=512, E=8, k=2, I=256, shared=True, w_routed="fp8",
                             w_shared="bf16", seed=47)),
    ("bf16+fp8", L.LayerSpec("st48", T=20, H=512, E=8, k=2, I=256, shared=True, w_routed="bf16",
                             w_shared="fp8", seed=48)),
    ("mxfp4+fp8", L.LayerSpec("st49", T=20, H=512, E=8, k=2, I=256, shared=True, w_routed="mxfp4",
                              w_shared="fp8", seed=49)),
    ("w4a8+bf16", L.LayerSpec("st50", T=40, H=512, E=8, k=2, I=256, shared=True, w_routed="mxfp4a8",
                              w_shared="bf16", seed=50)),
    ("w4a8+w8a8", L.LayerSpec("st51", T=40, H=512, E=8, k=2, I=256, shared=True, w_routed="mxfp4a8",
                              w_shared="mxfp8a8", seed=51)),
    ("int8", L.LayerSpec("st52", T=40, H=512, E=8, k=2, I=256, shared=True, w_routed="int8",
                         w_shared="int8", seed=52)),
]


@pytest.mark.parametrize("name,spec", STAGE_SPECS, ids=[s[0] for s in STAGE_SPECS])
def test_stages_match_oracle_stage_by_stage(name, spec):
    lay, pl = build(spec, DEV)
    s = pl.shape
    T, k, E, H = spec.T, spec.k, spec.E, spec.H
    x = lay["x"].view(torch.bfloat16)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    N.moe_route(s, x, pl.Wr, lay["bias"], idx, w, pl.ws)
    ridx, rw, _ = O.route(lay["x_host"], lay["Wr_host"], lay["bias_host"], k, spec.act)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.max(np.abs(w.cpu().numpy() - rw)) <= 1e-5
    # permutation from the oracle's routing
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    st = torch.empty(T * k, dtype=torch.int32, device=DEV)
    ps = torch.empty(T * k, dtype=torch.int32, device=DEV)
    N.moe_permute(s, torch.from_numpy(ridx).to(DEV), off, st, ps, pl.ws)
    roff, rst, rps = O.permute(ridx, E)
    torch.cuda.synchronize()
    assert np.array_equal(off.cpu().numpy(), roff)
    assert np.array_equal(st.cpu().numpy(), rst) and np.array_equal(ps.cpu().numpy(), rps)
    # grouped FFN from the oracle's permutation
    yp = torch.empty((T * k, H), dtype=torch.bfloat16, device=DEV)
    ysh = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    N.moe_grouped_ffn(s, x, torch.from_numpy(roff).to(DEV), torch.from_numpy(rst).to(DEV), pl.routed, pl.shared,
                      yp, ysh, pl.ws)
    torch.cuda.synchronize()
    from _gpu import host_weights
    rt = host_weights(lay["routed"])
    sh = {kk: (None if v is None else v[0]) for kk, v in host_weights(lay["shared"]).items()}
    u = L.act_to_f64(lay["x_host"], "bf16")
    ref_perm = np.zeros((T * k, H))
    for e in range(E):
        r0, r1 = roff[e], roff[e + 1]
        if r1 > r0:
            one = {kk: (None if v is None else v[e]) for kk, v in rt.items()}
            ref_perm[r0:r1] = O.expert_ffn(u[rst[r0:r1]], one, spec.w_routed)
    ref_sh = O.expert_ffn(u, sh, spec.w_shared)
    e_r, e_s = rel_fro(to_f64(yp), ref_perm), rel_fro(to_f64(ysh), ref_sh)
    say("  %s: routed rows error %.3e, shared rows error %.3e" % (name, e_r, e_s))
    assert e_r <= 1e-2 and e_s <= 1e-2
    # combine from the oracle's intermediate rows (rounded to bf16, the act type)
    yp_ref = torch.from_numpy(ref_perm).to(torch.bfloat16).to(DEV)
    ysh_ref = torch.from_numpy(ref_sh).to(torch.bfloat16).to(DEV)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    N.moe_combine(s, yp_ref, torch.from_numpy(rps).to(DEV), torch.from_numpy(rw.astype(np.float32)).to(DEV),
                  ysh_ref, y)
    torch.cuda.synchronize()
    ypr, yshr = to_f64(yp_ref), to_f64(ysh_ref)
    ref_y = np.stack([O.combine_token(rw[t], ypr[rps[t * k:(t + 1) * k]], yshr[t]) for t in range(T)])
    assert rel_fro(to_f64(y), ref_y) <= 4e-3  # only the final bf16 rounding differs


# ------------------------------------------------------------------ fused routing + permutation

ROUTE_PERMUTE = [
    # (T, E, k): one token; a workgroup's 16 tokens exactly and one more; several workgroups with a
    # ragged last one; the largest fused sizes (T*k = 8192, 32 workgroups x 512 experts of histogram);
    # one expert; 125 workgroups; Zipf-skewed groups; past the fused limits (T*k > 8192; E > 512;
    # 2048 tokens or more, whose scores run on the prefill kernel): the separate kernels
    (1, 8, 2), (16, 128, 8), (17, 128, 8), (45, 300, 7), (255, 64, 6), (512, 512, 16), (64, 1, 1),
    (1024, 40, 8), (2000, 16, 4), (600, 256, 8), (1100, 64, 8), (40, 1024, 16), (2304, 8, 2),
]


@pytest.mark.parametrize("T,E,k", ROUTE_PERMUTE, ids=["T%d-E%d-k%d" % r for r in ROUTE_PERMUTE])
def test_route_permute_matches_oracle(T, E, k):
    """moe_route_permute against the oracle's route and permute, bit for bit (weights within
    1e-5), with the workspace filled with 0xFF first: the completion count the fused launch relies
    on is cleared by the score kernel of the same call. A second call gives the same bits."""
    zipf = T >= 600
    spec = L.LayerSpec("rp", T=T, H=256, E=E, k=k, I=128, router="zipf" if zipf else "uniform",
                       zipf_alpha=1.1 if zipf else 0.0, calib_tokens=512, seed=90 + T + E)
    lay, pl = build(spec, DEV)
    pl.ws.fill_(255)
    x = lay["x"].view(torch.bfloat16)
    ridx, rw, _ = O.route(lay["x_host"], lay["Wr_host"], lay["bias_host"], k, spec.act)
    roff, rst, rps = O.permute(ridx, E)
    outs = []
    for _ in range(2):
        idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
        w = torch.empty((T, k), dtype=torch.float32, device=DEV)
        off = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
        st = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
        ps = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
        N.moe_route_permute(pl.shape, x, pl.Wr, lay["bias"], idx, w, off, st, ps, pl.ws)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), ridx)
        assert np.max(np.abs(w.cpu().numpy() - rw)) <= 1e-5
        assert np.array_equal(off.cpu().numpy(), roff)
        assert np.array_equal(st.cpu().numpy(), rst) and np.array_equal(ps.cpu().numpy(), rps)
        outs.append((idx, w, off, st, ps))
    assert all(torch.equal(a, b) for a, b in zip(*outs))


# ------------------------------------------------------------------ full-size layers

# the DeepSeek-V4-Pro-shaped layer at a prefill batch: MXFP4 routed experts in the prefill
# kernel, the bf16 shared expert in a launch of its own; the same layer with W4A8 routed experts
# (MXFP8 activations on the block-scaled MFMA); and the hybrid MXFP8-MXFP4 layer (W4A8 routed, W8A8
# MXFP8 shared); the DeepSeek-V3-shaped prefill layer with Int8 W8A8 experts
FULL = ["c2", "c3", "c4", "c5", "v4p", "v4p-w4a8", "v4p-mx", "v3-int8", "c4-w4a8", "c4-mx", "c3-int8"]
# decode layers whose every output token is compared (the kernel widths the benchmark runs: bf16
# gate/up with 16-feature tiles and down with 64 at H = 4096; MXFP4, W4A8 and the hybrid scheme at
# H = 7168)
ALL_TOKENS = {"c2", "c4", "c4-w4a8", "c4-mx"}


def boundary_tokens(spec, roff, rst, block, groups=None):
    """Tokens of the first and last row of every `block`-row block of the listed groups (all
    routed groups when None), and of the shared group's blocks (rows in token order)."""
    E = spec.E
    out = set()
    for g in (range(E) if groups is None else groups):
        r0, r1 = int(roff[g]), int(roff[g + 1])
        for b0 in range(r0, r1, block):
            out.add(int(rst[b0]))
            out.add(int(rst[min(b0 + block, r1) - 1]))
    if spec.shared:
        for b0 in range(0, spec.T, block):
            out.add(b0)
            out.add(min(b0 + block, spec.T) - 1)
    return out


@pytest.mark.slow
@pytest.mark.parametrize("cfg", FULL)
def test_full_size_layer(cfg):
    """The bench's launch configuration at full size: routing and permutation identical for
    every token; outputs against the oracle on every token of the Qwen3 and V4-Pro decode layers,
    on the block boundaries of every group of more than one 64-row block of the V3 decode layers,
    and on a sample of the prefill layers (whose row tiles the next test covers group by group)."""
    spec = L.workload(cfg)
    say("full-size", cfg, spec)
    lay, pl = build(spec, DEV)
    y, idx, w = run(spec, lay, pl)
    say("  ran; oracle routing")
    ridx, rw, _ = O.route(lay["x_host"], lay["Wr_host"], lay["bias_host"], spec.k, spec.act)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.max(np.abs(w.cpu().numpy() - rw)) <= 1e-5
    # the permutation the layer used
    roff, rst, rps = O.permute(ridx, spec.E)
    s = pl.shape
    off = torch.empty(spec.E + 1, dtype=torch.int32, device=DEV)
    st = torch.empty(spec.T * spec.k, dtype=torch.int32, device=DEV)
    ps = torch.empty(spec.T * spec.k, dtype=torch.int32, device=DEV)
    N.moe_permute(s, idx, off, st, ps, pl.ws)
    torch.cuda.synchronize()
    assert np.array_equal(off.cpu().numpy(), roff)
    assert np.array_equal(st.cpu().numpy(), rst) and np.array_equal(ps.cpu().numpy(), rps)
    # routing and permutation as the layer runs them (one launch after the scores at decode sizes)
    x = lay["x"] if spec.act == "f32" else lay["x"].view(torch.bfloat16)
    idx2, w2 = torch.empty_like(idx), torch.empty_like(w)
    N.moe_route_permute(s, x, pl.Wr, lay["bias"], idx2, w2, off, st, ps, pl.ws)
    torch.cuda.synchronize()
    assert np.array_equal(idx2.cpu().numpy(), ridx) and np.max(np.abs(w2.cpu().numpy() - rw)) <= 1e-5
    assert np.array_equal(off.cpu().numpy(), roff)
    assert np.array_equal(st.cpu().numpy(), rst) and np.array_equal(ps.cpu().numpy(), rps)
    counts = np.diff(roff)
    hot = int(np.argmax(counts))
    rng = np.random.default_rng(7)
    if cfg in ALL_TOKENS:
        tokens = list(range(spec.T))
    elif spec.T <= 256:
        thick = [g for g in range(spec.E) if counts[g] > 64]
        tokens = sorted(boundary_tokens(spec, roff, rst, 64, thick) | set(rng.choice(spec.T, 8, replace=False).tolist()))
    else:
        tokens = sorted({0, spec.T - 1, int(rst[roff[hot]]), int(rst[roff[hot + 1] - 1]),
                         *rng.choice(spec.T, 8, replace=False).tolist()})
    say("  active experts %d, max rows %d; oracle on %d tokens" % ((counts > 0).sum(), counts.max(), len(tokens)))
    ref = oracle_tokens(spec, lay, ridx, rw, tokens)
    err = rel_fro(to_f64(y)[tokens], ref)
    say("  rel. Frobenius error on %d tokens %.3e (bound %.0e; specified %.0e)"
        % (len(tokens), err, tol_of(spec), spec_tol_of(spec)))
    assert err <= tol_of(spec)
    # no token far off either: the worst token's own error within the bound
    worst = max(rel_fro(to_f64(y)[t], r) for t, r in zip(tokens, ref))
    say("  worst single-token error %.3e" % worst)
    assert worst <= 2 * tol_of(spec)


@pytest.mark.slow
@pytest.mark.parametrize("cfg", ["c5"])
def test_full_size_prefill_rows_group_by_group(cfg):
    """The prefill layer's grouped FFN at full size, row tile by row tile: with the oracle's
    routing and permutation, the first and last row of every group, the first row of its last
    128-row block (the ragged tile: a half item or the last full item) and the same rows of the
    shared group are compared with the oracle's FFN of that row alone."""
    spec = L.workload(cfg)
    say("prefill rows", cfg, spec)
    lay, pl = build(spec, DEV)
    ridx, rw, _ = O.route(lay["x_host"], lay["Wr_host"], lay["bias_host"], spec.k, spec.act)
    roff, rst, rps = O.permute(ridx, spec.E)
    T, k, H = spec.T, spec.k, spec.H
    x = lay["x"].view(torch.bfloat16)
    yp = torch.empty((T * k, H), dtype=torch.bfloat16, device=DEV)
    ysh = torch.empty((T, H), dtype=torch.bfloat16, device=DEV) if spec.shared else None
    N.moe_grouped_ffn(pl.shape, x, torch.from_numpy(roff).to(DEV), torch.from_numpy(rst).to(DEV), pl.routed,
                      pl.shared, yp, ysh, pl.ws)
    torch.cuda.synchronize()
    rows = []  # (slot or -1 - token for the shared rows, token, expert)
    for g in range(spec.E):
        r0, r1 = int(roff[g]), int(roff[g + 1])
        if r1 > r0:
            for r in sorted({r0, r0 + 128 * ((r1 - r0 - 1) // 128), r1 - 1}):
                rows.append((r, int(rst[r]), g))
    if spec.shared:
        for t in sorted({0, 128 * ((T - 1) // 128), T - 1}):
            rows.append((-1 - t, t, -1))
    say("  %d rows over %d groups" % (len(rows), int((np.diff(roff) > 0).sum()) + (1 if spec.shared else 0)))
    res = oracle_ffn_rows(spec, lay, [(t, e) for _, t, e in rows])
    got = np.stack([to_f64(yp[r]) if r >= 0 else to_f64(ysh[-1 - r]) for r, _, _ in rows])
    ref = np.stack([res[(t, e)] for _, t, e in rows])
    err = rel_fro(got, ref)
    worst = max(rel_fro(a, b) for a, b in zip(got, ref))
    say("  rel. Frobenius error %.3e, worst row %.3e (bound %.0e)" % (err, worst, tol_of(spec)))
    assert err <= tol_of(spec) and worst <= 2 * tol_of(spec)


# layers at the V3 decode layer's width (H = 7168, I = 2048) on the decode kernel with a few
# experts, so every group spans several 64-row blocks with a ragged last one: the gate/up width of
# the V3 decode layers (32 features: their groups average 8 rows or more; bf16 and int8), down at
# 32 (bf16) and 64 (int8) features, four row tiles per block; every token compared
MID = [
    ("mid-bf16", L.LayerSpec("m1", T=200, H=7168, E=6, k=2, I=2048, shared=True, router="zipf", zipf_alpha=1.0,
                             calib_tokens=512, seed=81)),
    ("mid-int8", L.LayerSpec("m2", T=200, H=7168, E=6, k=2, I=2048, shared=True, w_routed="int8", w_shared="int8",
                             router="zipf", zipf_alpha=1.0, calib_tokens=512, seed=82)),
    # groups of several 256-row blocks (the decode kernel's largest items) with a ragged last one
    ("thick-bf16", L.LayerSpec("m3", T=700, H=1024, E=3, k=1, I=1024, shared=True, router="zipf", zipf_alpha=1.0,
                               calib_tokens=512, seed=83)),
    ("thick-f32", L.LayerSpec("m4", T=300, H=512, E=2, k=1, I=256, shared=True, act="f32", w_routed="f32",
                              w_shared="f32", seed=84)),
]


@pytest.mark.slow
@pytest.mark.parametrize("name,spec", MID, ids=[m[0] for m in MID])
def test_decode_widths_every_token(name, spec):
    say("mid", name, spec)
    lay, pl = build(spec, DEV, "decode")
    y, idx, w = run(spec, lay, pl)
    ridx, rw, _ = O.route(lay["x_host"], lay["Wr_host"], lay["bias_host"], spec.k, spec.act)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.max(np.abs(w.cpu().numpy() - rw)) <= 1e-5
    counts = np.bincount(ridx.reshape(-1), minlength=spec.E)
    say("  group rows %s" % counts.tolist())
    assert counts.max() > 128  # several 64-row blocks in one group
    tokens = list(range(spec.T))
    ref = oracle_tokens(spec, lay, ridx, rw, tokens)
    err = rel_fro(to_f64(y), ref)
    worst = max(rel_fro(to_f64(y)[t], ref[t]) for t in tokens)
    say("  rel. Frobenius error %.3e, worst token %.3e (bound %.0e)" % (err, worst, tol_of(spec)))
    assert err <= tol_of(spec) and worst <= 2 * tol_of(spec)


# the same width with groups of fewer than 8 rows on average: gate/up at 16 features per item
THIN = [
    ("thin-bf16", L.LayerSpec("m5", T=24, H=7168, E=12, k=2, I=2048, shared=True, seed=85)),
    ("thin-int8", L.LayerSpec("m6", T=24, H=7168, E=12, k=2, I=2048, shared=True, w_routed="int8", w_shared="int8",
                              seed=86)),
]


@pytest.mark.parametrize("name,spec", THIN, ids=[m[0] for m in THIN])
def test_decode_thin_groups_every_token(name, spec):
    say("thin", name, spec)
    lay, pl = build(spec, DEV, "decode")
    y, idx, w = run(spec, lay, pl)
    ridx, rw, _ = O.route(lay["x_host"], lay["Wr_host"], lay["bias_host"], spec.k, spec.act)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.max(np.abs(w.cpu().numpy() - rw)) <= 1e-5
    assert (spec.T * spec.k + spec.T) / (spec.E + 1) < 8  # the one-tile width
    tokens = list(range(spec.T))
    ref = oracle_tokens(spec, lay, ridx, rw, tokens)
    err = rel_fro(to_f64(y), ref)
    worst = max(rel_fro(to_f64(y)[t], ref[t]) for t in tokens)
    say("  rel. Frobenius error %.3e, worst token %.3e (bound %.0e)" % (err, worst, tol_of(spec)))
    assert err <= tol_of(spec) and worst <= 2 * tol_of(spec)


# ------------------------------------------------------------------ seeded sweep of random small layers

def _sweep_specs(n=24, seed=2024):
    """Random small layers over the supported combinations: formats, shared expert or not,
    Zipf or uniform routing, k up to 8, group sizes from empty to several 128-row blocks."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        act = "f32" if i % 8 == 0 else "bf16"
        if act == "f32":
            wr = ws = "f32"
        else:
            wr = str(rng.choice(["bf16", "fp8", "mxfp4", "mxfp4a8"]))
            ws = str(rng.choice(["bf16", "fp8", "mxfp4"]))
        prefill_shape = wr == "mxfp4a8" or rng.random() < 0.5
        H = int(rng.choice([512, 1024])) if prefill_shape else int(rng.choice([256, 384, 512]))
        I = int(rng.choice([256, 512])) if prefill_shape else int(rng.choice([128, 256, 384]))
        E = int(rng.choice([4, 8, 16, 40]))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.choice([1, 7, 33, 150, 420]))
        zipf = bool(rng.random() < 0.5) and E >= 8
        out.append(L.LayerSpec("sw%d" % i, T=T, H=H, E=E, k=k, I=I, shared=bool(rng.random() < 0.5), act=act,
                               w_routed=wr, w_shared=ws, router="zipf" if zipf else "uniform",
                               zipf_alpha=1.1 if zipf else 0.0, calib_tokens=256, seed=100 + i))
    return out


SWEEP = _sweep_specs()


@pytest.mark.parametrize("spec", SWEEP, ids=[s.name for s in SWEEP])
def test_layer_random_sweep(spec):
    """Every random layer on the automatic path, and on both explicit paths where the shape allows
    them: routing identical to the oracle's, outputs within the format's bound."""
    paths = ["auto", "decode"]
    if _prefill_ok(spec):
        paths.append("prefill")
    if spec.w_routed == "mxfp4a8" and not _prefill_ok(spec):
        pytest.skip("W4A8 needs the prefill shape constraints")
    say("sweep", spec)
    ref = None
    for path in paths:
        lay, pl = build(spec, DEV, path)
        y, idx, w = run(spec, lay, pl)
        if ref is None:
            ref = oracle_full(spec, lay)
        assert np.array_equal(idx.cpu().numpy(), ref["topk_idx"])
        assert np.max(np.abs(w.cpu().numpy() - ref["topk_w"])) <= 1e-5
        err = rel_fro(to_f64(y), ref["y"])
        say("  %s: rel. Frobenius error %.3e (bound %.0e)" % (path, err, tol_of(spec)))
        assert err <= tol_of(spec)


def _sweep_quantised_specs(n=12, seed=2025):
    """Random small layers over the activation-quantising formats (prefill path): W4A8 routed with a
    bf16 or W8A8 MXFP8 shared expert or none, Int8 W8A8 with or without a shared expert; group
    sizes from empty to several 256-row items, T from 1 up."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = ("w4a8", "hybrid", "int8")[i % 3]
        shared = kind == "hybrid" or bool(rng.random() < 0.5)
        wr = "int8" if kind == "int8" else "mxfp4a8"
        ws = {"w4a8": "bf16", "hybrid": "mxfp8a8", "int8": "int8"}[kind]
        H = int(rng.choice([512, 1024]))
        I = int(rng.choice([256, 512]))
        E = int(rng.choice([4, 8, 16, 40]))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.choice([1, 7, 33, 150, 420]))
        zipf = bool(rng.random() < 0.5) and E >= 8
        out.append(L.LayerSpec("swq%d" % i, T=T, H=H, E=E, k=k, I=I, shared=shared, w_routed=wr, w_shared=ws,
                               router="zipf" if zipf else "uniform", zipf_alpha=1.1 if zipf else 0.0,
                               calib_tokens=256, seed=300 + i))
    return out


SWEEP_Q = _sweep_quantised_specs()


@pytest.mark.parametrize("spec", SWEEP_Q, ids=[s.name for s in SWEEP_Q])
def test_layer_random_sweep_quantised(spec):
    """Each random quantised layer on its (prefill) path: routing identical to the oracle's, outputs
    within the bound, and a second call bit-identical."""
    say("sweep-q", spec)
    ref = None
    # each layer on both kernels (the automatic choice, then each one explicitly)
    for path in ("auto", "decode", "prefill"):
        lay, pl = build(spec, DEV, path)
        y, idx, w = run(spec, lay, pl)
        if ref is None:
            ref = oracle_full(spec, lay)
        assert np.array_equal(idx.cpu().numpy(), ref["topk_idx"])
        assert np.max(np.abs(w.cpu().numpy() - ref["topk_w"])) <= 1e-5
        err = rel_fro(to_f64(y), ref["y"])
        say("  %s: rel. Frobenius error %.3e (bound %.0e)" % (path, err, tol_of(spec)))
        assert err <= tol_of(spec)
        y2, _, _ = run(spec, lay, pl)
        assert torch.equal(y, y2)


# ------------------------------------------------------------------ activation quantisers, bit for bit

def _bf16_rows(rows):
    """float rows -> (their bf16 rounding as exact float64 values, the bf16 tensor on the device)."""
    bits = px.f32_to_bf16_bits(np.asarray(rows, np.float32))
    exact = px.bf16_bits_to_f32(bits).astype(np.float64)
    return exact, torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)


def _mxfp8_probe_rows(K, seed):
    """Rows whose 32-blocks reach every branch of the MXFP8 rule: normal rows over a wide range of
    scales, an all-zero row, -0.0 and entries far below their block maximum (the E4M3 subnormal grid
    after scaling), block maxima whose scaled value reaches [448, 512) (saturation) or sits just
    below it, exact E4M3 rounding ties, and bf16 subnormals (the exponent clamped at -127)."""
    rng = np.random.default_rng(seed)
    out = [rng.standard_normal(K) * 2.0 ** rng.uniform(-60, 60) for _ in range(24)]
    out.append(np.zeros(K))
    r = rng.standard_normal(K)
    r[::7] = -0.0
    r[1::5] *= 2.0 ** -rng.integers(8, 20, size=len(r[1::5]))
    out.append(r)
    # one block per maximum: 1.6875 (scaled 432, a tie between 416 and 448), 1.71875 (440, rounds up
    # to 448), 1.75 (448), 1.8125 (464), 1.96875 (504), each with a random sign
    r = rng.standard_normal(K) * 0.25
    for b, m in enumerate((1.6875, 1.71875, 1.75, 1.8125, 1.96875)):
        r[32 * (b % (K // 32)) + int(rng.integers(32))] = m * (1 if rng.random() < 0.5 else -1)
    out.append(r)
    # block maximum 1 (exponent -8), the other entries exact midpoints of the E4M3 grid at several
    # binades: (1 + (2j + 1) / 16) * 2^-m
    r = np.zeros(K)
    for b in range(K // 32):
        blk = [(1.0 + (2 * int(rng.integers(8)) + 1) / 16.0) * 2.0 ** -int(rng.integers(1, 12)) for _ in range(31)]
        r[32 * b:32 * b + 31] = np.array(blk) * np.where(rng.random(31) < 0.5, -1.0, 1.0)
        r[32 * b + 31] = 1.0
    out.append(r)
    out.append(rng.integers(-127, 128, size=K) * 2.0 ** -133)  # bf16 subnormals
    out.append(rng.standard_normal(K) * 2.0 ** 120)
    return np.stack(out)


@pytest.mark.parametrize("K", [32, 256, 7168])
def test_mxfp8_quantiser_matches_oracle_bit_for_bit(K):
    """The GPU's MXFP8 activation quantiser (the W4A8 layer's x) gives the oracle's codes and
    exponents exactly: both take each decision from exact values with the same rounding rule."""
    x, xd = _bf16_rows(_mxfp8_probe_rows(K, seed=900 + K))
    codes = torch.empty(xd.shape, dtype=torch.uint8, device=DEV)
    scales = torch.empty((xd.shape[0], K // 32), dtype=torch.uint8, device=DEV)
    N.moe_quantize_mxfp8(xd, codes, scales)
    torch.cuda.synchronize()
    rc, rs = O.mxfp8_quantize(x)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)
    # the probes reached saturation, the subnormal grid and signed zero
    assert (rc & 0x7F == 0x7E).any() and ((rc & 0x7F) > 0).any() and ((rc & 0x78) == 0).any()
    assert (rc == 0x80).any()


def _int8_probe_rows(K, seed):
    """Normal rows over a wide range of scales, an all-zero row, -0.0 entries, rows with maximum 127
    and 254 (factors 1 and 1/2, so half-integer and odd entries are exact rounding ties), a row with
    one dominant entry, bf16 subnormals."""
    rng = np.random.default_rng(seed)
    out = [rng.standard_normal(K) * 2.0 ** rng.uniform(-60, 60) for _ in range(12)]
    out.append(np.zeros(K))
    r = rng.standard_normal(K)
    r[::3] = -0.0
    out.append(r)
    for amax, ties in ((127.0, rng.integers(-40, 40, size=K) + 0.5), (254.0, 2.0 * rng.integers(-60, 60, size=K) + 1.0)):
        r = ties.astype(np.float64)
        r[int(rng.integers(K))] = amax if rng.random() < 0.5 else -amax
        out.append(r)
    r = rng.standard_normal(K) * 1e-3
    r[int(rng.integers(K))] = 1e3
    out.append(r)
    out.append(rng.integers(-127, 128, size=K) * 2.0 ** -133)
    return np.stack(out)


@pytest.mark.parametrize("K", [8, 520, 2048, 7168, 8192])
def test_int8_quantiser_matches_oracle_bit_for_bit(K):
    """The GPU's per-token int8 quantiser (the Int8 W8A8 layer's x and h) gives the oracle's codes
    and fp32 scales exactly, for each row-length variant of the kernel."""
    x, xd = _bf16_rows(_int8_probe_rows(K, seed=950 + K))
    codes = torch.empty(xd.shape, dtype=torch.int8, device=DEV)
    scales = torch.empty(xd.shape[0], dtype=torch.float32, device=DEV)
    N.moe_quantize_int8(xd, codes, scales)
    torch.cuda.synchronize()
    rc, rs = O.int8_quantize(x)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert (np.abs(rc) == 127).any() and (rs == 0).any()


# ------------------------------------------------------------------ hash routing

HASH_SPECS = [
    ("decode-bf16-shared", L.LayerSpec("h1", T=45, H=512, E=12, k=3, I=256, shared=True, seed=71), 37),
    ("prefill-fp8", L.LayerSpec("h2", T=600, H=512, E=6, k=2, I=256, shared=True, w_routed="fp8",
                                w_shared="fp8", seed=72), 1000),
    ("wide-E", L.LayerSpec("h3", T=9, H=256, E=300, k=7, I=128, seed=73), 5),
]


@pytest.mark.parametrize("name,spec,vocab", HASH_SPECS, ids=[h[0] for h in HASH_SPECS])
def test_hash_routing_matches_oracle(name, spec, vocab):
    """moe_route_hash against the oracle (indices bit-exact, weights within 1e-5), with some invalid
    ids and table entries mixed in; then the whole hash-routed layer."""
    say("hash", name, spec, vocab)
    lay, pl = build(spec, DEV)
    ids, table = L.hash_inputs(spec, vocab)
    ids[::7] = vocab + 3  # ids outside the table: all k pairs dropped
    table[1, 0] = spec.E  # an entry outside [0, E): that pair dropped
    if spec.k > 1:
        table[2, 1] = table[2, 0]  # a repeated expert: both pairs kept
    d_ids, d_tab = torch.from_numpy(ids).to(DEV), torch.from_numpy(table).to(DEV)
    x = lay["x"].view(torch.bfloat16)
    idx = torch.empty((spec.T, spec.k), dtype=torch.int32, device=DEV)
    w = torch.empty((spec.T, spec.k), dtype=torch.float32, device=DEV)
    N.moe_route_hash(pl.shape, x, pl.Wr, lay["bias"], d_ids, d_tab, idx, w, pl.ws)
    torch.cuda.synchronize()
    ridx, rw = O.route_hash(lay["x_host"], lay["Wr_host"], lay["bias_host"], ids, table, spec.k, spec.act)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.max(np.abs(w.cpu().numpy() - rw)) <= 1e-5
    y = torch.empty((spec.T, spec.H), dtype=torch.bfloat16, device=DEV)
    idx2 = torch.empty_like(idx)
    pl.forward_hash(x, lay["bias"], d_ids, d_tab, y, idx2)
    torch.cuda.synchronize()
    assert np.array_equal(idx2.cpu().numpy(), ridx)
    routed = host_weights(lay["routed"])
    shared = {kk: (None if v is None else v[0]) for kk, v in host_weights(lay["shared"]).items()} if spec.shared else None
    ref = O.layer(spec, lay["x_host"], lay["Wr_host"], lay["bias_host"], routed, shared, hash_routing=(ids, table))
    err = rel_fro(to_f64(y), ref["y"])
    say("  rel. Frobenius error %.3e (bound %.0e)" % (err, tol_of(spec)))
    assert err <= tol_of(spec)


# ------------------------------------------------------------------ weights in the logical layout

LOGICAL_SPECS = [
    ("f32", L.LayerSpec("l1", T=16, H=256, E=8, k=2, I=128, act="f32", w_routed="f32", w_shared="f32", seed=71)),
    ("bf16-shared-zipf", L.LayerSpec("l2", T=90, H=512, E=12, k=3, I=256, shared=True, router="zipf",
                                     zipf_alpha=1.0, calib_tokens=512, seed=72)),
    ("fp8-prefill", L.LayerSpec("l3", T=600, H=512, E=6, k=2, I=256, shared=True, w_routed="fp8", w_shared="fp8",
                                seed=73)),
    ("mxfp4+bf16", L.LayerSpec("l4", T=40, H=512, E=16, k=4, I=256, shared=True, w_routed="mxfp4",
                               w_shared="bf16", seed=74)),
    ("w4a8+mxfp8", L.LayerSpec("l5", T=200, H=512, E=8, k=2, I=256, shared=True, w_routed="mxfp4a8",
                               w_shared="mxfp8a8", seed=75)),
    ("int8", L.LayerSpec("l6", T=300, H=512, E=8, k=2, I=256, shared=True, w_routed="int8", w_shared="int8",
                         seed=76)),
]


@pytest.mark.parametrize("name,spec", LOGICAL_SPECS, ids=[g[0] for g in LOGICAL_SPECS])
def test_logical_weights_forward_matches_packed(name, spec):
    """moe_layer_forward_logical takes the router and the experts in the pages' row-major layout
    and packs them into its workspace each call; its results equal moe_layer_forward on the same
    weights packed once with moe_pack, bit for bit, on two calls in a row."""
    say("logical", name, spec)
    lay, pl = build(spec, DEV)
    x = lay["x"] if spec.act == "f32" else lay["x"].view(torch.bfloat16)
    Wr = lay["Wr"] if spec.act == "f32" else lay["Wr"].view(torch.bfloat16)
    ws = torch.empty(N.moe_logical_workspace_size(pl.shape), dtype=torch.uint8, device=DEV)
    for call in range(2):
        y2, idx2, w2 = run(spec, lay, pl)
        y1 = torch.full_like(y2, float("nan"))
        idx1 = torch.full_like(idx2, -7)
        w1 = torch.full_like(w2, float("nan"))
        N.moe_layer_forward_logical(pl.shape, x, Wr, lay["bias"], lay["routed"], lay["shared"], y1, idx1, w1, ws)
        torch.cuda.synchronize()
        assert torch.equal(idx1, idx2), call
        assert torch.equal(w1, w2), call
        assert torch.equal(y1, y2), (call, (y1.float() - y2.float()).abs().max().item())
        x.mul_(2.0)  # the second call on another batch


# ------------------------------------------------------------------ shared expert on a second stream

SIDE_SPECS = [
    # decode, one format, hot groups of more than 64 rows (thick gate/up blocks)
    ("decode-bf16-thick", L.LayerSpec("s1", T=300, H=512, E=6, k=2, I=256, shared=True, router="zipf",
                                      zipf_alpha=1.0, calib_tokens=512, seed=91), "decode"),
    # decode, MXFP4 routed and bf16 shared experts (two codecs in the one-stream launch)
    ("decode-mxfp4+bf16", L.LayerSpec("s2", T=40, H=512, E=16, k=4, I=256, shared=True, w_routed="mxfp4",
                                      w_shared="bf16", seed=92), "decode"),
    ("decode-fp8+mxfp4", L.LayerSpec("s3", T=33, H=512, E=8, k=2, I=256, shared=True, w_routed="fp8",
                                     w_shared="mxfp4", seed=93), "decode"),
    ("decode-f32", L.LayerSpec("s4", T=21, H=256, E=8, k=2, I=128, act="f32", w_routed="f32", w_shared="f32",
                               shared=True, seed=94), "decode"),
    ("decode-bf16+fp8", L.LayerSpec("s5", T=64, H=1024, E=32, k=4, I=512, shared=True, w_routed="bf16",
                                    w_shared="fp8", seed=95), "decode"),
    # groups of fewer than 8 rows at H = 4096: the all-groups gate/up launch takes one 16-feature
    # tile per item, the shared expert's own launch (24 rows in one group) two
    ("decode-bf16-widths", L.LayerSpec("s7", T=24, H=4096, E=12, k=2, I=1024, shared=True, seed=97), "decode"),
    # a prefill batch keeps one stream: the two entry points run the same launches
    ("prefill-fp8", L.LayerSpec("s6", T=600, H=512, E=6, k=2, I=256, shared=True, w_routed="fp8",
                                w_shared="fp8", seed=96), "prefill"),
]


@pytest.mark.parametrize("name,spec,path", SIDE_SPECS, ids=[g[0] for g in SIDE_SPECS])
def test_shared_expert_on_second_stream_matches_one_stream(name, spec, path):
    """At decode, moe_layer_forward runs a shared expert (bf16-activation formats) on a second
    stream beside the routing and the routed experts; moe_layer_forward_timed keeps one stream and
    one grouped launch over all groups. The shared expert's launch restricted to its own group gives
    every row the same arithmetic, so the two must agree bit for bit, on two calls in a row."""
    say("side", name, spec, path)
    lay, pl = build(spec, DEV, path=path)
    x = lay["x"] if spec.act == "f32" else lay["x"].view(torch.bfloat16)
    for call in range(2):
        y2, idx2, w2 = run(spec, lay, pl)
        y1 = torch.full_like(y2, float("nan"))
        idx1 = torch.full_like(idx2, -7)
        w1 = torch.full_like(w2, float("nan"))
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(N.TIMED_EVENTS)]
        for e in evs:
            e.record()  # creates the underlying HIP events
        N.moe_layer_forward_timed(pl.shape, x, pl.Wr, lay["bias"], pl.routed, pl.shared, y1, evs, idx1, w1, pl.ws)
        torch.cuda.synchronize()
        assert torch.equal(idx1, idx2), call
        assert torch.equal(w1, w2), call
        assert torch.equal(y1, y2), (call, (y1.float() - y2.float()).abs().max().item())
        # the second call on another batch: x scaled by two (exact in every activation format)
        x.mul_(2.0)


# ------------------------------------------------------------------ graph capture

GRAPH_SPECS = [
    ("decode-bf16-shared", L.LayerSpec("g1", T=45, H=512, E=12, k=3, I=256, shared=True, router="zipf",
                                       zipf_alpha=1.0, calib_tokens=512, seed=61)),
    ("prefill-fp8", L.LayerSpec("g2", T=600, H=512, E=6, k=2, I=256, shared=True, w_routed="fp8",
                                w_shared="fp8", seed=62)),
    ("w4a8", L.LayerSpec("g3", T=200, H=512, E=8, k=2, I=256, shared=True, w_routed="mxfp4a8",
                         w_shared="bf16", seed=63)),
    ("hybrid-mx", L.LayerSpec("g4", T=300, H=512, E=8, k=2, I=256, shared=True, w_routed="mxfp4a8",
                              w_shared="mxfp8a8", seed=64)),
    ("int8", L.LayerSpec("g5", T=300, H=512, E=8, k=2, I=256, shared=True, w_routed="int8",
                         w_shared="int8", seed=65)),
]


@pytest.mark.parametrize("name,spec", GRAPH_SPECS, ids=[g[0] for g in GRAPH_SPECS])
def test_layer_forward_captures_into_a_graph(name, spec):
    """Every entry point only enqueues on its stream (no host synchronisation, no allocation, no
    memset), so a whole layer forward can be captured in a HIP graph. The graph is replayed several
    times, with eager work and synchronisations between the replays, and every replay must equal
    the eager forward bit for bit (the plan and the zero row are rewritten by kernels each call)."""
    say("graph", name, spec)
    lay, pl = build(spec, DEV)
    y_ref, idx_ref, w_ref = run(spec, lay, pl)
    x = lay["x"].view(torch.bfloat16)
    y = torch.empty_like(y_ref)
    idx = torch.empty_like(idx_ref)
    w = torch.empty_like(w_ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pl.forward(x, lay["bias"], y, idx, w)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pl.forward(x, lay["bias"], y, idx, w)
    for rep in range(4):
        y.fill_(0)
        idx.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_ref), rep
        assert torch.equal(w, w_ref), rep
        assert torch.equal(y, y_ref), rep
        # eager work between the replays, on the same workspace
        run(spec, lay, pl)


def test_hash_routed_forward_captures_into_a_graph():
    """moe_layer_forward_hash captures like moe_layer_forward: every replay (with eager calls and
    synchronisations between them) equals the eager hash-routed forward bit for bit."""
    spec = L.LayerSpec("g6", T=45, H=512, E=12, k=3, I=256, shared=True, seed=66)
    lay, pl = build(spec, DEV)
    ids, table = L.hash_inputs(spec, 37)
    ids[::9] = 40  # some ids outside the table
    d_ids, d_tab = torch.from_numpy(ids).to(DEV), torch.from_numpy(table).to(DEV)
    x = lay["x"].view(torch.bfloat16)
    y_ref = torch.empty((spec.T, spec.H), dtype=torch.bfloat16, device=DEV)
    idx_ref = torch.empty((spec.T, spec.k), dtype=torch.int32, device=DEV)
    w_ref = torch.empty((spec.T, spec.k), dtype=torch.float32, device=DEV)
    pl.forward_hash(x, lay["bias"], d_ids, d_tab, y_ref, idx_ref, w_ref)
    torch.cuda.synchronize()
    y, idx, w = torch.empty_like(y_ref), torch.empty_like(idx_ref), torch.empty_like(w_ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pl.forward_hash(x, lay["bias"], d_ids, d_tab, y, idx, w)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pl.forward_hash(x, lay["bias"], d_ids, d_tab, y, idx, w)
    for rep in range(4):
        y.fill_(0)
        idx.fill_(-2)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_ref), rep
        assert torch.equal(w, w_ref), rep
        assert torch.equal(y, y_ref), rep
        run(spec, lay, pl)  # eager score-routed work between the replays, on the same workspace


# ------------------------------------------------------------------ exact ties in the router

def _tie_bias(E, k, rng):
    """Bias levels for a zeroed router: a few experts (fewer than k) at level 2, in the upper
    64-expert slices; a tied level-1 set spread over every slice, larger than the places left;
    the rest 0. The k-th place then falls inside the level-1 tie, and the lowest-indexed tied
    experts that fill it lie in more than one slice (scores e, e + 64, ... share a lane)."""
    b = np.zeros(E, np.float32)
    if E <= 64:
        b[:] = rng.integers(0, 3, size=E)
        return b
    n2 = max(1, k // 3)
    top = rng.choice(np.arange(E // 2, E), n2, replace=False)
    b[top] = 2.0
    stride = max(1, (E - 20) // (3 * k))
    tied = [e for e in range(20, E, stride) if b[e] == 0][:3 * k]
    b[tied] = 1.0
    need = k - n2
    assert len(tied) > need and tied[need - 1] >= 64  # the chosen tied experts straddle a slice boundary
    return b


@pytest.mark.parametrize("T", [33, 2304])
@pytest.mark.parametrize("E,k", [(40, 6), (300, 7), (1024, 16)])
def test_router_ties_go_to_the_lower_expert_index(T, E, k):
    """With the router matrix zeroed every score is exactly its bias, so tied biases put many
    experts at the k-th / (k+1)-th boundary: the k chosen are the largest scores with ties to the
    lower index, listed in ascending index, weighted by exp(b - max) renormalised; with no bias,
    experts 0..k-1 at 1/k each. The tied experts that fill the last places straddle the 64-expert
    slices a lane's scores come in (E = 300, 1024). T = 2304 takes the prefill kernel's split-K
    scores."""
    spec = L.LayerSpec("tie", T=T, H=512, E=E, k=k, I=256, seed=77)
    lay, pl = build(spec, DEV)
    pl.Wr.zero_()
    x = lay["x"].view(torch.bfloat16)
    rng = np.random.default_rng(5 + E)
    bias = _tie_bias(E, k, rng)
    for b in (bias, None):
        idx = torch.empty((T, spec.k), dtype=torch.int32, device=DEV)
        w = torch.empty((T, spec.k), dtype=torch.float32, device=DEV)
        N.moe_route(pl.shape, x, pl.Wr, None if b is None else torch.from_numpy(b).to(DEV), idx, w, pl.ws)
        torch.cuda.synchronize()
        bb = np.zeros(spec.E) if b is None else b.astype(np.float64)
        chosen = sorted(sorted(range(spec.E), key=lambda e: (-bb[e], e))[:spec.k])
        p = np.exp(bb[chosen] - bb[chosen].max())
        assert (idx.cpu().numpy() == np.array(chosen, np.int32)).all()
        assert np.abs(w.cpu().numpy() - p / p.sum()).max() <= 1e-6
        ridx, rw, _ = O.route(lay["x_host"], np.zeros_like(lay["Wr_host"]), b, spec.k, spec.act)
        assert np.array_equal(idx.cpu().numpy(), ridx) and np.abs(w.cpu().numpy() - rw).max() <= 1e-6
