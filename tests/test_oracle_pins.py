"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Sources of truth used here: the sizes the pages print (tests/golden/page_sizes.json),
textbook values of the number formats (OCP Microscaling v1.0 E2M1 and E8M0),
closed forms and identities of softplus and silu, brute force over all k-subsets
for top-k, exact invariants of the layer (zero input, zero routed weights, a
scale byte raised by one), a hand-worked two-expert layer
(tests/golden/two_expert_example.json), and for the optional pre-FFN RMSNorm
torch's float64 rms_norm, its fp32->bf16 cast, hand-worked rows and scale
invariance.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from moe_synth import CONFIGS, make_inputs, mxfp4_encode, pack_nibbles

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- formats

def test_e2m1_table_matches_textbook_values():
    # OCP MX v1.0, FP4 (E2M1) value table; code 8 is negative zero
    expected = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    got = oracle.e2m1_table()
    assert list(got) == expected
    assert np.signbit(got[8]) and not np.signbit(got[0])


def test_e8m0_values():
    assert oracle.e8m0_value(127) == 1.0
    assert oracle.e8m0_value(128) == 2.0
    assert oracle.e8m0_value(126) == 0.5
    assert oracle.e8m0_value(0) == 2.0 ** -127
    assert oracle.e8m0_value(254) == 2.0 ** 127
    assert np.isnan(oracle.e8m0_value(255))


def test_decode_nibble_order_and_block_scales():
    k = 64
    packed = np.zeros((1, k // 2), np.uint8)
    scales = np.full((1, k // 32), 127, np.uint8)
    packed[0, 0] = 0x24        # element 0 = 2 (low nibble), element 1 = 1
    packed[0, 15] = 0xF0       # element 30 = 0, element 31 = -6
    packed[0, 16] = 0x1A       # element 32 = -1, element 33 = 0.5 (second block)
    scales[0, 1] = 129         # second block scaled by 4
    v = oracle.decode_mxfp4(packed, scales, k)[0]
    assert v[0] == 2.0 and v[1] == 1.0
    assert v[30] == 0.0 and v[31] == -6.0
    assert v[32] == -4.0 and v[33] == 2.0
    assert np.count_nonzero(v) == 5


def test_decode_every_code_and_scale_by_brute_force():
    # each of the 256 byte values, under scales 110..140, element by element
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    packed = np.tile(np.arange(256, dtype=np.uint8), (31, 1))  # 31 rows x 256 bytes = 512 elements
    scales = np.repeat(np.arange(110, 141, dtype=np.uint8)[:, None], 16, axis=1)
    v = oracle.decode_mxfp4(packed, scales, 512)
    for r in range(31):
        sc = 2.0 ** (110 + r - 127)
        for b in range(256):
            assert v[r, 2 * b] == table[b & 15] * sc
            assert v[r, 2 * b + 1] == table[b >> 4] * sc


def test_packed_bytes_match_page_sizes():
    d = _load("page_sizes.json")
    eb = d["expert_bytes"]
    h, i = eb["hidden"], eb["inter"]
    per_expert = oracle.mxfp4_packed_bytes(2 * i, h) + oracle.mxfp4_packed_bytes(h, i)
    assert per_expert == 18_800_640
    assert abs(per_expert - eb["value_bytes_rounded"]) <= eb["round_to"] / 2
    for key in ("all_experts_bytes", "gpu_resident_experts_bytes", "cpu_resident_experts_bytes",
                "drafter_experts_bytes"):
        ent = d[key]
        assert abs(per_expert * ent["experts"] - ent["value_bytes_rounded"]) <= ent["round_to"] / 2, key


def test_generator_layout_sizes_match_page_sizes():
    # the generator's per-expert tensors at full size, checked on a 1-expert draw with small T
    cfg = CONFIGS["decode_t1_h5120_e384"].with_(n_experts=1, n_shared=0)
    inp = make_inputs(cfg, seed=0)
    nbytes = sum(t[0].numel() for t in (inp.gu_q, inp.gu_s, inp.dn_q, inp.dn_s))
    assert nbytes == 18_800_640


def test_layer_shape_constants_match_pages():
    shp = _load("page_sizes.json")["layer_shape"]
    for name in ("decode_t1_h5120_e384", "decode_t64_h5120_e384", "prefill_t4096_h5120_e384"):
        c = CONFIGS[name]
        assert (c.hidden, c.n_experts, c.top_k, c.inter, c.n_shared, c.shared_inter) == \
            (shp["hidden"], shp["n_experts"], shp["top_k"], shp["inter"], shp["n_shared"], shp["shared_inter"])
        assert (c.route_scale, c.swiglu_limit) == (shp["route_scale"], shp["swiglu_limit"])
    c = CONFIGS["skew_t16384_h5120_e128"]
    assert (c.n_experts, c.top_k) == (shp["drafter_n_experts"], shp["drafter_top_k"])


# ---------------------------------------------------------------- encoder (test harness) vs decoder

def test_encoder_round_trips_every_code_and_scale():
    table = oracle.e2m1_table()
    rng = np.random.default_rng(0)
    for sc in range(110, 141):
        codes = rng.integers(0, 16, size=(64, 32)).astype(np.uint8)
        codes[:, 0] = np.where(rng.random(64) < 0.5, 7, 15)  # a +-6 element fixes the block exponent
        vals = table[codes] * 2.0 ** (sc - 127)
        packed, scales = mxfp4_encode(torch.tensor(vals, dtype=torch.float32))
        assert np.all(scales.numpy() == sc)
        # equal values, code for code except -0 may encode as +0
        dec = oracle.decode_mxfp4(packed.numpy(), scales.numpy(), 32)
        assert np.array_equal(dec, vals)


def test_encoder_round_to_nearest_even_ties():
    # value / 2^scale -> expected magnitude; a 6.0 in the block pins the scale at 2^0
    cases = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0,
             6.5: 6.0, 7.99: 6.0, 0.26: 0.5, 2.6: 3.0, 4.9: 4.0, 5.1: 6.0}
    for v, want in cases.items():
        blk = np.zeros(32, np.float32)
        blk[0] = 6.0 if v < 6.0 else v
        blk[1] = v
        blk[2] = -v
        p, s = mxfp4_encode(torch.tensor(blk[None, :]))
        dec = oracle.decode_mxfp4(p.numpy(), s.numpy(), 32)[0]
        assert s.item() == 127
        assert dec[1] == want and dec[2] == -want, (v, dec[1], dec[2])


def test_encoder_zero_block_and_nibble_packing():
    p, s = mxfp4_encode(torch.zeros(2, 64))
    assert np.all(s.numpy() == 127) and np.all(p.numpy() == 0)
    codes = torch.tensor([[1, 2, 3, 4]], dtype=torch.int32)
    assert pack_nibbles(codes).tolist() == [[0x21, 0x43]]


# ---------------------------------------------------------------- elementwise closed forms

def test_sqrtsoftplus_closed_forms():
    ssp = oracle.sqrtsoftplus
    assert ssp(0.0) == pytest.approx(math.sqrt(math.log(2.0)), rel=1e-15)
    assert ssp(1.0) == pytest.approx(1.145976303209723, rel=1e-14)
    assert ssp(-1.0) == pytest.approx(0.5596978537731075, rel=1e-14)
    assert ssp(20.0) == pytest.approx(4.472135955230024, rel=1e-14)
    assert ssp(-20.0) == pytest.approx(4.5399929739090794e-05, rel=1e-12)
    assert ssp(1000.0) == pytest.approx(math.sqrt(1000.0), rel=1e-15)   # no overflow
    assert ssp(-1000.0) == 0.0
    z = np.linspace(-30, 30, 2001)
    # softplus(z) - softplus(-z) = z
    assert np.allclose(ssp(z) ** 2 - ssp(-z) ** 2, z, rtol=0, atol=1e-12)
    assert np.all(np.diff(ssp(z)) > 0)  # strictly increasing


def test_silu_and_clamp():
    assert oracle.silu(10.0) == pytest.approx(9.999546021312975, rel=1e-15)
    assert oracle.silu(4.0) == pytest.approx(3.928055160151634, rel=1e-15)
    assert oracle.silu(1.0) == pytest.approx(0.7310585786300049, rel=1e-15)
    z = np.linspace(-20, 20, 401)
    assert np.allclose(oracle.silu(z) - oracle.silu(-z), z, atol=1e-13)  # silu(z) - silu(-z) = z
    L = 10.0
    assert oracle.clamped_swiglu(12.0, -12.0, L) == oracle.silu(10.0) * -10.0
    assert oracle.clamped_swiglu(12.0, 3.0, L) == oracle.silu(10.0) * 3.0
    # the gate has no lower clamp; the up projection is clamped on both sides
    assert oracle.clamped_swiglu(-50.0, 1.0, L) == pytest.approx(-50.0 * math.exp(-50.0), rel=1e-12)
    assert oracle.clamped_swiglu(2.0, 50.0, L) == oracle.silu(2.0) * 10.0
    assert oracle.clamped_swiglu(2.0, -50.0, L) == oracle.silu(2.0) * -10.0
    assert oracle.clamped_swiglu(0.0, 5.0, L) == 0.0


# ---------------------------------------------------------------- router

def _route_given_logits(logits, k, rho=1.5, bias=None):
    """Drive the oracle router with chosen logits: x = e_0 and W_r[:, 0] = logits."""
    logits = np.asarray(logits, np.float32)
    e = logits.shape[0]
    x = np.zeros((1, 32), np.uint16)
    x[0, 0] = 0x3F80  # bf16 1.0
    wr = np.zeros((e, 32), np.float32)
    wr[:, 0] = logits
    return oracle.route(x, wr, bias, k, rho)


def _brute_force_topk(u, k):
    """The unique k-subset S with: i in S, j not in S => u_i > u_j or (u_i == u_j and i < j)."""
    e = len(u)
    found = []
    for sub in itertools.combinations(range(e), k):
        s = set(sub)
        ok = all((u[i] > u[j]) or (u[i] == u[j] and i < j) for i in s for j in range(e) if j not in s)
        if ok:
            found.append(s)
    assert len(found) == 1
    return found[0]


def test_topk_brute_force_small():
    rng = np.random.default_rng(1)
    for trial in range(300):
        e = int(rng.integers(2, 11))
        k = int(rng.integers(1, min(e, 4) + 1))
        # coarse values make exact ties frequent
        logits = rng.integers(-3, 4, size=e).astype(np.float32) * 0.5
        r = _route_given_logits(logits, k)
        u = r["u"][0]
        want = _brute_force_topk(list(u), k)
        got = r["idx"][0]
        assert set(int(i) for i in got) == want
        # selection order: u descending, ties by lower index
        for a, b in zip(got[:-1], got[1:]):
            assert u[a] > u[b] or (u[a] == u[b] and a < b)


def test_topk_bias_is_selection_only():
    # logits (1, -1, 0), bias (0, 0.7, 0), k = 2: selection by s + b, weights from s
    r = _route_given_logits([1.0, -1.0, 0.0], 2, bias=np.array([0.0, 0.7, 0.0], np.float32))
    assert list(r["idx"][0]) == [1, 0]
    s1, s0 = oracle.sqrtsoftplus(-1.0), oracle.sqrtsoftplus(1.0)
    b = float(np.float32(0.7))
    assert r["u"][0][1] == pytest.approx(s1 + b, rel=1e-15)
    assert r["w"][0][0] == pytest.approx(1.5 * s1 / (s1 + s0), rel=1e-14)


def test_weights_sum_to_route_scale():
    rng = np.random.default_rng(2)
    for k in (1, 2, 3, 6, 8):
        r = _route_given_logits(rng.standard_normal(40), k)
        assert r["w"][0].sum() == pytest.approx(1.5, rel=1e-15)
    r = _route_given_logits(rng.standard_normal(10), 1)
    assert r["w"][0][0] == 1.5


def test_zero_input_routes_to_lowest_indices_with_equal_weights():
    x = np.zeros((2, 64), np.uint16)
    wr = np.random.default_rng(3).standard_normal((32, 64)).astype(np.float32)
    r = oracle.route(x, wr, None, 6, 1.5)
    assert r["idx"].tolist() == [[0, 1, 2, 3, 4, 5]] * 2
    assert np.all(r["w"] == 0.25)
    assert np.all(r["gap"] == 0.0)


def test_gap_is_kth_minus_next():
    r = _route_given_logits([0.0, 3.0, 1.0, 2.0], 2)
    u = oracle.sqrtsoftplus(np.array([0.0, 3.0, 1.0, 2.0], np.float32).astype(np.float64))
    assert list(r["idx"][0]) == [1, 3]
    assert r["gap"][0] == u[3] - u[2]
    r = _route_given_logits([0.0, 3.0], 2)
    assert r["gap"][0] == np.inf


def test_valid_selections_near_tie():
    u = np.array([1.0, 1.0 - 0.5e-6, 0.5, 1.0 - 5e-6])
    assert oracle.valid_selections(u, 1, 0.0) == [[0]]
    assert sorted(oracle.valid_selections(u, 1, 1e-6)) == [[0], [1]]
    # exact ties keep the lower index only
    u = np.array([1.0, 1.0, 0.5])
    assert oracle.valid_selections(u, 1, 1e-6) == [[0]]
    u = np.array([2.0, 1.0, 1.0 - 0.2e-6, 0.3])
    assert sorted(oracle.valid_selections(u, 2, 1e-6)) == [[0, 1], [0, 2]]


# ---------------------------------------------------------------- permute

def test_permute_brute_force():
    rng = np.random.default_rng(4)
    for trial in range(50):
        e = int(rng.integers(1, 20))
        k = int(rng.integers(1, min(e, 5) + 1))
        t = int(rng.integers(0, 30))
        idx = np.stack([rng.permutation(e)[:k] for _ in range(t)]) if t else np.zeros((0, k), np.int64)
        p = oracle.permute(idx, e)
        flat = idx.reshape(-1)
        pos = 0
        for ex in range(e):
            assert p["expert_offsets"][ex] == pos
            for f in range(flat.shape[0]):  # ascending flat slot order within an expert
                if flat[f] == ex:
                    assert p["sorted_slots"][pos] == f
                    assert p["slot_pos"][f] == pos
                    pos += 1
        assert p["expert_offsets"][e] == flat.shape[0] == pos


# ---------------------------------------------------------------- experts: matmul vs explicit loops

def test_expert_mlp_against_explicit_loops():
    rng = np.random.default_rng(5)
    m, h, i = 3, 8, 5
    x = rng.standard_normal((m, h)) * 3
    wgu = rng.standard_normal((2 * i, h))
    wdn = rng.standard_normal((h, i))
    hh, o = oracle.expert_mlp(x, wgu, wdn, 2.0)
    for r in range(m):
        hr = []
        for c in range(i):
            g = sum(x[r, q] * wgu[c, q] for q in range(h))
            u = sum(x[r, q] * wgu[i + c, q] for q in range(h))
            g = min(g, 2.0)
            u = max(-2.0, min(u, 2.0))
            hr.append(g / (1 + math.exp(-g)) * u)
        assert np.allclose(hh[r], hr, rtol=1e-13, atol=1e-13)
        for c in range(h):
            assert o[r, c] == pytest.approx(sum(hr[q] * wdn[c, q] for q in range(i)), rel=1e-12, abs=1e-12)


def _tiny_inputs(**kw):
    cfg = CONFIGS["tiny_t8_h512_e32"].with_(**kw)
    return make_inputs(cfg, seed=0, device="cpu")


def test_layer_against_per_token_direct_sum():
    """The grouped/permuted/combined layer equals a per-token sum written out directly."""
    inp = _tiny_inputs()
    a = inp.oracle_args()
    out = oracle.layer_forward(**a)
    cfg = inp.cfg
    x = oracle.bf16_bits_to_f64(a["x_bits"])
    wsg = oracle.bf16_bits_to_f64(a["sh_gu"])
    wsd = oracle.bf16_bits_to_f64(a["sh_dn"])
    for t in range(cfg.tokens):
        y = oracle.expert_mlp(x[t:t + 1], wsg, wsd, cfg.swiglu_limit)[1][0]
        for j in range(cfg.top_k):
            e = int(out["idx"][t, j])
            wgu = oracle.decode_mxfp4(a["gu_q"][e], a["gu_s"][e], cfg.hidden)
            wdn = oracle.decode_mxfp4(a["dn_q"][e], a["dn_s"][e], cfg.inter)
            y = y + out["w"][t, j] * oracle.expert_mlp(x[t:t + 1], wgu, wdn, cfg.swiglu_limit)[1][0]
        assert np.allclose(out["y"][t], y, rtol=1e-12, atol=1e-12)


def test_layer_threads_give_the_single_thread_result():
    """Experts run on several threads write only their own rows: the same bits as one thread, and the per-token
    direct sum above still holds through them."""
    inp = _tiny_inputs(tokens=40)
    a = inp.oracle_args()
    one = oracle.layer_forward(**a)
    many = oracle.layer_forward(**a, workers=4)
    for key in ("idx", "w", "h_slot", "y_slot", "y_shared", "y"):
        assert np.array_equal(one[key], many[key]), key


# ---------------------------------------------------------------- whole-layer invariants

def test_zero_input_gives_zero_output():
    inp = _tiny_inputs()
    inp.x.zero_()
    out = oracle.layer_forward(**inp.oracle_args())
    assert np.all(out["y"] == 0.0)
    assert out["idx"].tolist() == [[0, 1, 2, 3, 4, 5]] * inp.cfg.tokens


def test_zero_routed_weights_give_shared_output():
    inp = _tiny_inputs()
    inp.gu_q.zero_()
    out = oracle.layer_forward(**inp.oracle_args())
    assert np.array_equal(out["y"], out["y_shared"])
    assert np.any(out["y_shared"] != 0.0)


def test_down_scale_plus_one_doubles_routed_part():
    inp = _tiny_inputs()
    base = oracle.layer_forward(**inp.oracle_args())
    inp.dn_s += 1
    dbl = oracle.layer_forward(**inp.oracle_args())
    assert np.array_equal(dbl["idx"], base["idx"])
    assert np.allclose(dbl["y"] - dbl["y_shared"], 2.0 * (base["y"] - base["y_shared"]), rtol=1e-14, atol=1e-14)


def test_no_shared_expert():
    inp = _tiny_inputs(n_shared=0)
    assert inp.sh_gu is None
    out = oracle.layer_forward(**inp.oracle_args())
    assert np.all(out["y_shared"] == 0.0)


# ---------------------------------------------------------------- hand-worked example

def _two_expert_inputs(d):
    s = d["shape"]
    h, i, e = s["hidden"], s["inter"], s["n_experts"]
    x = np.zeros((1, h), np.uint16)
    for pos, v in d["x"].items():
        x[0, int(pos)] = np.array([v], np.float32).view(np.uint32)[0] >> 16
    wr = np.zeros((e, h), np.float32)
    for r, c, v in d["router_w"]:
        wr[r, c] = v
    gu_q = np.zeros((e, 2 * i, h // 2), np.uint8)
    gu_s = np.full((e, 2 * i, h // 32), 127, np.uint8)
    dn_q = np.zeros((e, h, i // 2), np.uint8)
    dn_s = np.full((e, h, i // 32), 127, np.uint8)
    for ent in d["gu_q_bytes"]:
        gu_q[ent["expert"], ent["row"], ent["byte"]] = ent["value"]
    for ent in d["dn_q_bytes"]:
        dn_q[ent["expert"], ent["row"], ent["byte"]] = ent["value"]
    for ent in d["dn_s_bytes"]:
        dn_s[ent["expert"], ent["row"], ent["block"]] = ent["value"]
    bf = lambda v: np.array([v], np.float32).view(np.uint32)[0] >> 16  # noqa: E731
    sh_gu = np.zeros((2 * s["shared_inter"], h), np.uint16)
    sh_dn = np.zeros((h, s["shared_inter"]), np.uint16)
    for r, c, v in d["sh_gu"]:
        sh_gu[r, c] = bf(v)
    for r, c, v in d["sh_dn"]:
        sh_dn[r, c] = bf(v)
    return dict(x_bits=x, router_w=wr, router_bias=None, gu_q=gu_q, gu_s=gu_s, dn_q=dn_q, dn_s=dn_s,
                sh_gu=sh_gu, sh_dn=sh_dn, route_scale=s["route_scale"], swiglu_limit=s["swiglu_limit"])


def test_hand_worked_two_expert_layer():
    d = _load("two_expert_example.json")
    args = _two_expert_inputs(d)
    silu = lambda z: z / (1 + math.exp(-z))  # noqa: E731,F841
    ssp = lambda z: math.sqrt(math.log1p(math.exp(z)))  # noqa: E731,F841
    inter = d["intermediates"]
    for case in d["cases"]:
        out = oracle.layer_forward(top_k=case["top_k"], **args)
        assert out["idx"][0].tolist() == case["idx"]
        assert np.allclose(out["s"][0], inter["scores"]["value"], rtol=1e-14)
        assert np.allclose(out["w"][0], case["w"]["value"], rtol=1e-14)
        want = np.zeros(d["shape"]["hidden"])
        for pos, ent in case["y_nonzero"].items():
            assert eval(ent["expr"]) == pytest.approx(ent["value"], rel=1e-14)
            want[int(pos)] = ent["value"]
        assert np.allclose(out["y"][0], want, rtol=1e-13, atol=1e-13)
        assert out["y_shared"][0][2] == pytest.approx(inter["shared"]["o2"]["value"], rel=1e-15)
    # the expert-1 clamps fire: without them the value would be silu(12) * -12
    assert inter["expert1"]["h0"]["value"] == pytest.approx(silu(10) * -10, rel=1e-15)


def test_hand_worked_zero_input():
    d = _load("two_expert_example.json")
    args = _two_expert_inputs(d)
    args["x_bits"][:] = 0
    for k, w in ((1, [1.5]), (2, [0.75, 0.75])):
        out = oracle.layer_forward(top_k=k, **args)
        assert out["idx"][0].tolist() == list(range(k))
        assert out["w"][0].tolist() == w
        assert np.all(out["y"] == 0.0)


# ---------------------------------------------------------------- skewed routing claim

def test_zipf_bias_gives_twentyfold_hot_expert():
    """The skewed workload's hottest expert takes about 20x the mean load.

    Routing depends on x and W_r only through the logits, which are ~N(0, 1)
    for any hidden size, so a small hidden size gives the same load profile.
    """
    cfg = CONFIGS["skew_t16384_h5120_e128"].with_(hidden=256, inter=32, shared_inter=32, n_shared=0,
                                                    tokens=4096)
    inp = make_inputs(cfg, seed=0, device="cpu")
    r = oracle.route(inp.x.numpy().view(np.uint16), inp.router_w.numpy(), inp.router_bias.numpy(),
                     cfg.top_k, cfg.route_scale)
    load = np.bincount(r["idx"].reshape(-1), minlength=cfg.n_experts)
    ratio = load.max() / load.mean()
    assert 16.0 <= ratio <= 24.0, ratio


# ---------------------------------------------------------------- pre-FFN RMSNorm (eps 1e-20)

def _bf16_bits(values):
    """bf16 bits of values that are exact in bf16 (checked)."""
    t = torch.tensor(values, dtype=torch.float32)
    b = t.to(torch.bfloat16)
    assert torch.equal(b.float(), t)
    return b.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_torch_cast_and_ties_to_even():
    """fp64 -> bf16 rounding against torch's fp32 -> bf16 cast (nearest, ties to
    even) on fp32-exact values, plus hand-made ties."""
    g = np.random.default_rng(3)
    v = (g.standard_normal(20000) * np.exp2(g.integers(-20, 20, 20000))).astype(np.float32)
    # fp32 subnormals and the smallest normals, where bf16 steps by 2^-133
    sub = g.integers(-(1 << 24), 1 << 24, 4000).astype(np.int64)
    v = np.concatenate([v, (sub * 2.0 ** -149).astype(np.float32)])
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f64_to_bf16_bits(v.astype(np.float64)), want)
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 0.0, -0.0])
    got = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(ties))
    assert got.tolist() == [1.0, 1 + 2.0 ** -6, -1.0, 0.0, 0.0]
    assert oracle.f64_to_bf16_bits(np.array([-0.0]))[0] == 0x8000


def test_rmsnorm_hand_example():
    """x = (3, 4): mean square 12.5, so x/rms = (0.848528.., 1.131370..); the bf16
    neighbours are 217/256 and 145/128.  With gain (2, 1/2): 1.697.. -> 217/128,
    0.5657.. -> 145/256."""
    x = _bf16_bits([[3.0, 4.0]])
    one = _bf16_bits([1.0, 1.0])
    out = oracle.bf16_bits_to_f64(oracle.rmsnorm(x, one, 1e-20))
    assert out.tolist() == [[217 / 256, 145 / 128]]
    out = oracle.bf16_bits_to_f64(oracle.rmsnorm(x, _bf16_bits([2.0, 0.5]), 1e-20))
    assert out.tolist() == [[217 / 128, 145 / 256]]


def test_rmsnorm_special_rows():
    """A constant row maps to +-gain, a zero row to zero (eps keeps it finite), a
    one-hot row of width n to sqrt(n) at its place."""
    h = 64
    one = _bf16_bits([1.0] * h)
    rows = _bf16_bits([[0.375] * h, [-96.0] * h, [0.0] * h, [0.0] * 5 + [7.0] + [0.0] * (h - 6)])
    out = oracle.bf16_bits_to_f64(oracle.rmsnorm(rows, one, 1e-20))
    assert np.all(out[0] == 1.0) and np.all(out[1] == -1.0) and np.all(out[2] == 0.0)
    assert out[3, 5] == 8.0 and np.count_nonzero(out[3]) == 1   # sqrt(64) = 8


def test_rmsnorm_matches_torch_and_invariants():
    """Against torch's rms_norm in float64 (within half a bf16 step), exact under a
    power-of-two rescale of the input, linear in a power-of-two gain, and of unit
    RMS with unit gain (within bf16 rounding)."""
    g = np.random.default_rng(4)
    t, h = 16, 512
    xf = (g.standard_normal((t, h)) * np.exp2(g.integers(-6, 6, (t, 1)))).astype(np.float32)
    x = torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    gam = torch.from_numpy((1 + 0.1 * g.standard_normal(h)).astype(np.float32)).to(torch.bfloat16)
    gbits = gam.view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_bits_to_f64(oracle.rmsnorm(x, gbits, 1e-20))
    ref = torch.nn.functional.rms_norm(
        torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double(), (h,),
        weight=gam.double(), eps=1e-20).numpy()
    half_step = np.exp2(np.floor(np.log2(np.abs(ref))) - 8)
    assert np.all(np.abs(got - ref) <= half_step * (1 + 1e-9))
    x4 = oracle.f64_to_bf16_bits(oracle.bf16_bits_to_f64(x) * 4.0)
    assert np.array_equal(oracle.rmsnorm(x4, gbits, 1e-20), oracle.rmsnorm(x, gbits, 1e-20))
    g2 = oracle.f64_to_bf16_bits(oracle.bf16_bits_to_f64(gbits) * 0.5)
    assert np.array_equal(oracle.bf16_bits_to_f64(oracle.rmsnorm(x, g2, 1e-20)), got * 0.5)
    unit = oracle.bf16_bits_to_f64(oracle.rmsnorm(x, _bf16_bits([1.0] * h), 1e-20))
    assert np.allclose(np.sqrt(np.mean(unit ** 2, axis=1)), 1.0, atol=2 ** -8)


def test_layer_with_norm_is_scale_invariant_and_normalises_first():
    """With the norm on, the layer output does not change when the input is scaled
    by a power of two, and equals the norm-free layer on a row already normalised."""
    inp = _tiny_inputs()
    a = inp.oracle_args()
    h = inp.cfg.hidden
    gbits = torch.from_numpy(np.random.default_rng(5).normal(1, 0.1, h).astype(np.float32)) \
        .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert a["norm_gamma"] is None
    base = oracle.layer_forward(**dict(a, norm_gamma=gbits, norm_eps=1e-20))
    a8 = dict(a, x_bits=oracle.f64_to_bf16_bits(oracle.bf16_bits_to_f64(a["x_bits"]) * 8.0))
    scaled = oracle.layer_forward(**dict(a8, norm_gamma=gbits, norm_eps=1e-20))
    assert np.array_equal(base["y"], scaled["y"]) and np.array_equal(base["idx"], scaled["idx"])
    plain = oracle.layer_forward(**dict(a, x_bits=oracle.rmsnorm(a["x_bits"], gbits, 1e-20)))
    assert np.array_equal(base["y"], plain["y"])
    raw = oracle.layer_forward(**a)
    assert not np.array_equal(base["y"], raw["y"])


# ---------------------------------------------------------------- MXFP8 (E4M3) expert weights

def test_e4m3_table_textbook_values_and_torch():
    """E4M3 "fn": textbook codes, and every code against torch's float8_e4m3fn conversion."""
    t = oracle.e4m3_table()
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and math.copysign(1, t[0x80]) < 0
    assert t[0x38] == 1.0 and t[0x40] == 2.0 and t[0xC0] == -2.0 and t[0x3C] == 1.5
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0          # largest normal, no infinities
    assert t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9 and t[0x08] == 2.0 ** -6
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF]) and np.count_nonzero(np.isnan(t)) == 2
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(t), np.isnan(ref))
    ok = ~np.isnan(t)
    assert np.array_equal(t[ok], ref[ok])


def test_decode_mxfp8_brute_force():
    g = np.random.default_rng(21)
    codes = g.integers(0, 256, (3, 96)).astype(np.uint8)
    codes[codes == 0x7F] = 0x7E
    codes[codes == 0xFF] = 0xFE
    scales = g.integers(100, 150, (3, 3)).astype(np.uint8)
    got = oracle.decode_mxfp8(codes, scales, 96)
    for r in range(3):
        for i in range(96):
            assert got[r, i] == oracle.e4m3_value(codes[r, i]) * 2.0 ** (int(scales[r, i // 32]) - 127)


def test_mxfp8_encoder_nearest_and_block_scale():
    """The generator's MXFP8 encoder: block exponent floor(log2 amax) - 8, each code the nearest E4M3
    multiple of the block scale (ties to even), zero blocks scaled by 2^0."""
    from moe_synth import mxfp8_encode
    g = torch.Generator().manual_seed(5)
    w = torch.randn((8, 256), generator=g) * torch.exp2(torch.randint(-12, 4, (8, 1), generator=g).float())
    w[0, :32] = 0.0
    codes, scales = mxfp8_encode(w)
    c, s = codes.numpy(), scales.numpy()
    assert s[0, 0] == 127 and np.all(c[0, :32] % 128 == 0)
    table = oracle.e4m3_table()
    finite = np.where(np.isnan(table), np.inf, table)
    dec = oracle.decode_mxfp8(c, s, 256)
    wd = w.double().numpy()
    for r in range(8):
        for b in range(8):
            blk = wd[r, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            if amax == 0:
                continue
            assert int(s[r, b]) - 127 == math.floor(math.log2(amax)) - 8
            sc = 2.0 ** (int(s[r, b]) - 127)
            for i in range(32):
                v = min(max(blk[i] / sc, -448.0), 448.0)
                best = np.min(np.abs(finite - v))
                assert abs(dec[r, 32 * b + i] / sc - v) == best


def test_mxfp8_and_mxfp4_layers_agree_on_shared_values():
    """Weights whose values are exact in both codecs (E2M1 values times a power of two per block) give the
    same layer output through the MXFP8 and the MXFP4 decoders."""
    from moe_synth import mxfp4_encode, mxfp8_encode
    inp = _tiny_inputs()
    cfg = inp.cfg
    g = torch.Generator().manual_seed(6)
    e2m1 = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])

    def exact(rows, k):
        v = e2m1[torch.randint(0, 8, (rows, k), generator=g)] * torch.where(
            torch.rand((rows, k), generator=g) < 0.5, -1.0, 1.0)
        v[:, ::32] = 6.0  # every block reaches 6: the MXFP4 block exponent is exact
        return v * torch.exp2(torch.randint(-9, -5, (rows, k // 32), generator=g).float()).repeat_interleave(32, 1)

    gu = [exact(2 * cfg.inter, cfg.hidden) for _ in range(cfg.n_experts)]
    dn = [exact(cfg.hidden, cfg.inter) for _ in range(cfg.n_experts)]
    a = inp.oracle_args()
    enc4 = [mxfp4_encode(m) for m in gu], [mxfp4_encode(m) for m in dn]
    enc8 = [mxfp8_encode(m) for m in gu], [mxfp8_encode(m) for m in dn]
    a4 = dict(a, gu_q=[q.numpy() for q, _ in enc4[0]], gu_s=[s.numpy() for _, s in enc4[0]],
              dn_q=[q.numpy() for q, _ in enc4[1]], dn_s=[s.numpy() for _, s in enc4[1]])
    a8 = dict(a, gu_q=[q.numpy() for q, _ in enc8[0]], gu_s=[s.numpy() for _, s in enc8[0]],
              dn_q=[q.numpy() for q, _ in enc8[1]], dn_s=[s.numpy() for _, s in enc8[1]], expert_format="mxfp8")
    w4 = oracle.routed_expert_weights(a4["gu_q"], a4["gu_s"], a4["dn_q"], a4["dn_s"], 3, cfg.hidden, cfg.inter)
    w8 = oracle.routed_expert_weights(a8["gu_q"], a8["gu_s"], a8["dn_q"], a8["dn_s"], 3, cfg.hidden, cfg.inter,
                                      "mxfp8")
    assert np.array_equal(w4[0], gu[3].double().numpy()) and np.array_equal(w8[0], w4[0])
    assert np.array_equal(w8[1], w4[1])
    y4 = oracle.layer_forward(**a4)["y"]
    y8 = oracle.layer_forward(**a8)["y"]
    assert np.array_equal(y4, y8) and np.any(y4 != 0)
