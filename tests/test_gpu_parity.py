"""Parity of the HIP path (through the C ABI) with the CPU oracle on an MI355X.

Inputs are the seeded synthetic workloads; expert ids must match except at
oracle-reported near-ties, outputs must meet the relative-L2 / max-abs bar
(see tests/parity.py), integer outputs must match bit for bit.
"""

import numpy as np
import pytest
import torch

import mixture_experts_ffn_07_amd as moe
import oracle
from moe_synth import CONFIGS, make_inputs, make_router_inputs

from parity import (ORACLE_WORKERS, TIE_TOL, assert_bar, bf16_to_f64, check_layer, gpu_expert_ffn, gpu_layer,
                    gpu_permute, gpu_route, match_routing)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _oracle_route(cfg, x, router_w, bias):
    return oracle.route(x.cpu().numpy().view(np.uint16), router_w.cpu().numpy(),
                        None if bias is None else bias.cpu().numpy(), cfg.top_k, cfg.route_scale)


def _check_layer(inp, tokens=None, gpu=None):
    """Run the GPU layer (or take its results) and compare rows `tokens` (all if None) with the oracle."""
    return check_layer(inp, tokens=tokens, gpu=gpu, workers=ORACLE_WORKERS)


# ------------------------------------------------------------------ router


@pytest.mark.parametrize("name", list(CONFIGS))
def test_route_full_size(name):
    cfg = CONFIGS[name]
    x, wr, b = make_router_inputs(cfg, seed=0, device=DEV)
    idx, w, gap = gpu_route(cfg, x, wr, b)
    ref = _oracle_route(cfg, x, wr, b)
    alt = match_routing(idx.cpu().numpy(), w.cpu().numpy(), ref, cfg.route_scale)
    g = gap.cpu().numpy().astype(np.float64)
    same = np.array([t not in alt for t in range(cfg.tokens)])
    fin = np.isfinite(ref["gap"])
    assert np.all(np.abs(g[same & fin] - ref["gap"][same & fin]) <= 4e-6)
    assert np.all(np.isinf(g[~fin]))
    # weights sum to the route scale
    assert np.allclose(w.sum(dim=1).cpu().numpy(), cfg.route_scale, rtol=0, atol=4e-6)
    print(f"{name}: near-tie alternatives {len(alt)}, oracle gaps < 1e-6: {(ref['gap'] < TIE_TOL).sum()}")


@pytest.mark.parametrize("tokens", [64, 1030])
def test_route_exact_ties_resolve_to_lowest_index(tokens):
    """All router rows equal: every logit ties exactly (the MFMA router below 1024 tokens, the split-weight dense
    GEMM from 1024)."""
    cfg = CONFIGS["decode_t64_h5120_e384"].with_(tokens=tokens)
    x, wr, _ = make_router_inputs(cfg, seed=1, device=DEV)
    wr[:] = wr[7]  # every expert has the same router row: all logits tie exactly
    idx, w, gap = gpu_route(cfg, x, wr, None)
    assert torch.all(idx.cpu() == torch.arange(cfg.top_k, dtype=torch.int32)[None, :])
    assert torch.all(gap.cpu() == 0.0)
    assert torch.allclose(w.cpu(), torch.full_like(w.cpu(), cfg.route_scale / cfg.top_k), rtol=0, atol=1e-6)
    x.zero_()
    idx, w, _ = gpu_route(cfg, x, make_router_inputs(cfg, seed=2, device=DEV)[1], None)
    assert torch.all(idx.cpu() == torch.arange(cfg.top_k, dtype=torch.int32)[None, :])


@pytest.mark.parametrize("tokens", [256, 1500])
def test_route_duplicate_rows_tie(tokens):
    cfg = CONFIGS["tiny_t8_h512_e32"].with_(tokens=tokens)
    x, wr, _ = make_router_inputs(cfg, seed=3, device=DEV)
    wr[20] = wr[3]
    wr[31] = wr[3]
    idx, _, _ = gpu_route(cfg, x, wr, None)
    for row in idx.cpu().numpy().tolist():
        have = [e for e in (3, 20, 31) if e in row]
        if have:
            pos = [row.index(e) for e in have]
            # equal scores: taken lowest index first, adjacent in the selection order
            assert have == sorted(have) and pos == list(range(pos[0], pos[0] + len(pos)))
            assert have == [3, 20, 31][:len(have)]


# ------------------------------------------------------------------ permute


def _random_routing(t, e, k, seed, skew=False):
    rng = np.random.default_rng(seed)
    if skew:
        p = 1.0 / np.arange(1, e + 1) ** 1.2
        rows = [rng.choice(e, size=k, replace=False, p=p / p.sum()) for _ in range(t)]
    else:
        rows = [rng.permutation(e)[:k] for _ in range(t)]
    return np.array(rows, dtype=np.int32).reshape(t, k)


@pytest.mark.parametrize("t,e,k,skew", [(1, 384, 6, False), (3, 32, 6, False), (64, 384, 6, False),
                                        (170, 384, 6, False), (171, 384, 6, False), (4096, 384, 6, False),
                                        (16384, 128, 3, True), (1000, 1, 1, False), (2000, 1000, 16, False),
                                        (700, 2, 2, False)])
def test_permute_bit_exact(t, e, k, skew):
    idx = _random_routing(t, e, k, seed=t * 7 + e, skew=skew)
    cfg = CONFIGS["tiny_t8_h512_e32"].with_(tokens=t, n_experts=e, top_k=k)
    off, srt, pos = gpu_permute(cfg, torch.from_numpy(idx).to(DEV))
    ref = oracle.permute(idx, e)
    assert np.array_equal(off.cpu().numpy(), ref["expert_offsets"])
    assert np.array_equal(srt.cpu().numpy(), ref["sorted_slots"])
    assert np.array_equal(pos.cpu().numpy(), ref["slot_pos"])


# ------------------------------------------------------------------ experts and combine


@pytest.mark.parametrize("variant", ["tiny", "decode_t3", "ragged_k", "no_shared", "min_dims", "fp8", "fp8_ragged_k",
                                     "fp8_t2", "fp8_t5", "fp8_t8", "t200_sliced_shared", "t1100_dense_shared", "t2100_whole_round_shared",
                                     "t2100_whole_round_k64", "t2048_whole_round_one_chunk", "t12_skinny_shared",
                                     "t64_skinny_shared", "t127_skinny_shared", "t300_skinny_row_groups",
                                     "t512_skinny_row_groups"])
def test_expert_ffn(variant):
    """Routed slots and the shared expert against the oracle over every row.  From 2048 tokens the shared
    expert takes the whole-round dense kernel: at 2100 tokens with a ragged last row tile, 160 h columns (a
    144-column block and a ragged one), 352 output columns (320 and a ragged block) and K of 11 and 5 32-wide
    chunks; with K of 6 and 3 64-wide chunks (192 h columns, 384 output columns); at 2048 tokens with K of one
    chunk and fewer columns than one block.  Below 128 tokens, with both K multiples of 128, the skinny
    weight-streaming kernel over K ranges: 12 tokens (one row tile, K ranges of one chunk), 64 tokens, 127
    tokens (eight row tiles, the last ragged); up to 512 tokens in row groups of 128 (300: the last group
    ragged; 512: four whole groups)."""
    base = CONFIGS["tiny_t8_h512_e32"]
    cfg = {"tiny": base.with_(tokens=40),
           "t200_sliced_shared": base.with_(tokens=200, shared_inter=160),
           "t1100_dense_shared": base.with_(tokens=1100, hidden=384, shared_inter=224),
           "t2100_whole_round_shared": base.with_(tokens=2100, hidden=352, shared_inter=160),
           "t2100_whole_round_k64": base.with_(tokens=2100, hidden=384, shared_inter=192),
           "t12_skinny_shared": base.with_(tokens=12),
           "t64_skinny_shared": base.with_(tokens=64, shared_inter=384),
           "t127_skinny_shared": base.with_(tokens=127, hidden=640, shared_inter=256),
           "t300_skinny_row_groups": base.with_(tokens=300, hidden=384, shared_inter=256),
           "t512_skinny_row_groups": base.with_(tokens=512, shared_inter=128),
           "t2048_whole_round_one_chunk": base.with_(tokens=2048, hidden=32, inter=32, shared_inter=32, n_experts=4,
                                                     top_k=2),
           "fp8": base.with_(tokens=40, expert_format="mxfp8"),
           "fp8_t2": base.with_(tokens=2, expert_format="mxfp8"),
           "fp8_t5": base.with_(tokens=5, expert_format="mxfp8"),
           "fp8_t8": base.with_(tokens=8, hidden=640, inter=384, expert_format="mxfp8"),
           "fp8_ragged_k": base.with_(tokens=24, hidden=160, inter=96, shared_inter=224, expert_format="mxfp8"),
           "decode_t3": base.with_(tokens=3),
           "ragged_k": base.with_(tokens=24, hidden=160, inter=96, shared_inter=224),
           "no_shared": base.with_(tokens=16, n_shared=0, shared_inter=0),
           "min_dims": base.with_(tokens=20, hidden=32, inter=32, shared_inter=32, n_experts=4, top_k=2)}[variant]
    inp = make_inputs(cfg, seed=5, device=DEV)
    idx = _random_routing(cfg.tokens, cfg.n_experts, cfg.top_k, seed=11)
    perm = oracle.permute(idx, cfg.n_experts)
    off = torch.from_numpy(perm["expert_offsets"]).to(DEV)
    srt = torch.from_numpy(perm["sorted_slots"]).to(DEV)
    y_slot, y_sh = gpu_expert_ffn(inp, off, srt)
    a = inp.oracle_args()
    x = oracle.bf16_bits_to_f64(a["x_bits"])
    ref_slot = np.zeros((cfg.tokens * cfg.top_k, cfg.hidden))
    for e in range(cfg.n_experts):
        lo, hi = perm["expert_offsets"][e], perm["expert_offsets"][e + 1]
        if hi > lo:
            wgu, wdn = oracle.routed_expert_weights(a["gu_q"], a["gu_s"], a["dn_q"], a["dn_s"], e, cfg.hidden,
                                                    cfg.inter, cfg.expert_format)
            rows = perm["sorted_slots"][lo:hi] // cfg.top_k
            ref_slot[lo:hi] = oracle.expert_mlp(x[rows], wgu, wdn, cfg.swiglu_limit)[1]
    assert_bar(bf16_to_f64(y_slot), ref_slot, "y_slot")
    if cfg.n_shared:
        assert_bar(bf16_to_f64(y_sh), oracle.shared_expert(a["x_bits"], a["sh_gu"], a["sh_dn"],
                                                          cfg.swiglu_limit)[1], "y_shared")


def test_combine():
    from moe_synth import f32_to_bf16_bits
    t, k, h = 37, 6, 640
    g = torch.Generator().manual_seed(9)
    y_slot = f32_to_bf16_bits(torch.randn(t * k, h, generator=g))
    y_sh = f32_to_bf16_bits(torch.randn(t, h, generator=g))
    w = torch.rand(t, k, generator=g, dtype=torch.float32) * 1.5
    pos = torch.randperm(t * k, generator=g).to(torch.int32)
    cfg = moe.make_config(h, 32, k, 256)
    for shared in (y_sh, None):
        y = torch.empty(t, h, dtype=torch.int16, device=DEV)
        moe.moe_combine(cfg, y_slot.to(DEV), pos.to(DEV), w.to(DEV), None if shared is None else shared.to(DEV),
                        t, y)
        torch.cuda.synchronize()
        ref = oracle.combine(bf16_to_f64(y_slot), pos.numpy(), w.numpy().astype(np.float64),
                             None if shared is None else bf16_to_f64(shared), k)
        got = bf16_to_f64(y)
        # one bf16 rounding of an fp32 sum: within 2^-8 relative, plus fp32 accumulation error
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5)


# ------------------------------------------------------------------ whole layer


def test_layer_tiny_full():
    inp = make_inputs(CONFIGS["tiny_t8_h512_e32"], seed=0, device=DEV)
    stats, _, _ = _check_layer(inp)
    print("tiny:", stats)


def test_layer_decode_t1_full():
    inp = make_inputs(CONFIGS["decode_t1_h5120_e384"], seed=0, device=DEV)
    stats, ref, _ = _check_layer(inp)
    print("decode_t1:", stats, "experts", ref["idx"].tolist())


@pytest.mark.parametrize("tokens", [2, 6, 7])
def test_layer_decode_few_tokens_full(tokens):
    """Few-token decode at full size: T <= 6 takes the weight-streaming path, T = 7 the general one."""
    inp = make_inputs(CONFIGS["decode_t1_h5120_e384"].with_(tokens=tokens), seed=3, device=DEV)
    stats, _, alt = _check_layer(inp)
    print(f"decode T={tokens}:", stats, "near-tie alternatives", len(alt))


def _sample(n, count, seed, must=()):
    rng = np.random.default_rng(seed)
    s = set(int(v) for v in rng.choice(n, size=min(count, n), replace=False))
    s |= {0, n - 1} | set(int(v) for v in must)
    return sorted(s)


@pytest.mark.parametrize("name,count", [("decode_t64_h5120_e384", 12), ("prefill_t4096_h5120_e384", 10),
                                        ("skew_t16384_h5120_e128", 10), ("verify_t5_h5120_e384", 5),
                                        ("verify_t320_h5120_e384", 12), ("pro_t1_h7168_e384", 1)])
def test_layer_full_size_sampled(name, count):
    cfg = CONFIGS[name]
    inp = make_inputs(cfg, seed=0, device=DEV)
    gpu = gpu_layer(inp)
    must = ()
    if inp.router_bias is not None:  # include tokens routed to the hottest expert
        hot = int(torch.argmax(inp.router_bias).item())
        hits = np.nonzero((gpu[1].cpu().numpy() == hot).any(axis=1))[0]
        must = hits[:3]
        load = np.bincount(gpu[1].cpu().numpy().reshape(-1), minlength=cfg.n_experts)
        print(f"{name}: hottest expert load {load.max()} = {load.max() / load.mean():.1f}x mean")
    toks = _sample(cfg.tokens, count, seed=1, must=must)
    stats, _, alt = _check_layer(inp, tokens=toks, gpu=gpu)
    print(f"{name}: {len(toks)} sampled tokens {stats}, near-tie alternatives {len(alt)}")


@pytest.mark.parametrize("tokens", [1, 2, 3, 17])
def test_layer_small_token_counts(tokens):
    inp = make_inputs(CONFIGS["tiny_t8_h512_e32"].with_(tokens=tokens), seed=2, device=DEV)
    _check_layer(inp)


@pytest.mark.parametrize("tokens", [1, 2])
@pytest.mark.parametrize("variant", ["min_dims", "ragged_k", "no_shared", "k1", "all_experts", "k16", "wide_h",
                                     "too_wide_h", "scale_plus_one", "zero_routed", "v4pro_dims"])
def test_layer_one_two_tokens(tokens, variant):
    """One and two tokens take the vector-ALU routed projections; shapes around their limits."""
    base = CONFIGS["tiny_t8_h512_e32"].with_(tokens=tokens)
    cfg = {"min_dims": base.with_(hidden=32, inter=32, shared_inter=32, n_experts=4, top_k=2),
           "ragged_k": base.with_(hidden=160, inter=96, shared_inter=224),
           "no_shared": base.with_(n_shared=0, shared_inter=0),
           "k1": base.with_(top_k=1),
           "all_experts": base.with_(n_experts=8, top_k=8),  # both tokens pick every expert: 2-row tiles
           "k16": base.with_(top_k=16),
           "wide_h": base.with_(hidden=8192, inter=64, shared_inter=64, n_experts=8),
           "too_wide_h": base.with_(hidden=8224, inter=64, shared_inter=64, n_experts=8),
           "scale_plus_one": base,
           "zero_routed": base,
           "v4pro_dims": CONFIGS["decode_t1_h5120_e384"].with_(tokens=tokens, hidden=7168, inter=3072,
                                                                 shared_inter=3072, n_experts=16)}[variant]
    inp = make_inputs(cfg, seed=13 + tokens, device=DEV)
    if variant == "scale_plus_one":
        inp.dn_s += 1
        inp.gu_s += 1
    if variant == "zero_routed":
        inp.dn_q.zero_()
    stats, _, alt = _check_layer(inp)
    print(f"T={tokens} {variant}:", stats, "near-tie alternatives", len(alt))


@pytest.mark.parametrize("variant", ["two_tiles_per_expert", "three_chunks", "ragged_k_fallback", "down_one_chunk",
                                     "dense_shared_ragged", "dense_shared_one_chunk", "dense_shared_256_ragged",
                                     "sliced_shared_t128", "sliced_shared_t1023", "whole_round_router_ragged"])
def test_layer_many_rows_per_expert(variant):
    """Tiles of up to 128 rows (the pipelined grouped GEMM when K is a multiple of 128), sampled rows; from 1024
    tokens the shared expert takes the dense pipelined kernel (ragged last row tile and column block), from 128 to
    1023 tokens the same kernel over K slices plus their sum (one-chunk slices, fewer weight rows than a block);
    from 2048 tokens the whole-round dense kernel's 256-row block tiles, also for the router logits (40 experts:
    one 96-expert block, mostly past the end; K of 11 32-wide chunks over several K ranges)."""
    base = CONFIGS["tiny_t8_h512_e32"]
    cfg = {"two_tiles_per_expert": base.with_(tokens=1024),             # ~192 rows per expert
           "three_chunks": base.with_(tokens=600, n_experts=8, hidden=384, inter=128, shared_inter=256),
           "ragged_k_fallback": base.with_(tokens=700, n_experts=16, hidden=160, inter=96, shared_inter=224),
           "down_one_chunk": base.with_(tokens=500, n_experts=8, top_k=3, inter=128, shared_inter=128),
           "dense_shared_ragged": base.with_(tokens=1100, n_experts=8, hidden=384, inter=128, shared_inter=96),
           "dense_shared_one_chunk": base.with_(tokens=1031, n_experts=8, hidden=32, inter=32,
                                                shared_inter=32),
           # whole-round dense kernel: 256-row block tiles, ragged last row tile and column blocks
           "dense_shared_256_ragged": base.with_(tokens=8300, n_experts=8, hidden=256, inter=128,
                                                 shared_inter=160),
           "sliced_shared_t128": base.with_(tokens=128, n_experts=8, hidden=352, inter=128, shared_inter=96),
           "whole_round_router_ragged": base.with_(tokens=2100, n_experts=40, hidden=352, inter=128,
                                                   shared_inter=160),
           "sliced_shared_t1023": base.with_(tokens=1023, n_experts=16, hidden=256, inter=128,
                                             shared_inter=160)}[variant]
    inp = make_inputs(cfg, seed=21, device=DEV)
    gpu = gpu_layer(inp)
    stats, _, alt = _check_layer(inp, tokens=_sample(cfg.tokens, 40, seed=5), gpu=gpu)
    print(f"{variant}:", stats, "near-tie alternatives", len(alt))


@pytest.mark.parametrize("tokens,inter,experts", [(1500, 384, 8), (700, 256, 8), (2000, 640, 16)])
def test_layer_mx6_down_records(tokens, inter, experts):
    """96-row tiles: the gate/up epilogue writes h as two-term MXFP6 records for the MXFP6 down projection.
    Inter 384 and 640: the last 256-column block holds one valid 128-wide chunk of the two; ragged last row
    tiles; every row against the oracle."""
    cfg = CONFIGS["tiny_t8_h512_e32"].with_(tokens=tokens, n_experts=experts, hidden=384, inter=inter,
                                            shared_inter=128)
    inp = make_inputs(cfg, seed=41, device=DEV)
    gpu = gpu_layer(inp)
    load = np.bincount(gpu[1].cpu().numpy().reshape(-1), minlength=cfg.n_experts)
    assert load.sum() / max(1, np.count_nonzero(load)) > 16  # the 96-row tile table
    stats, _, alt = _check_layer(inp, gpu=gpu)
    print(f"mx6 down records T={tokens} I={inter}:", stats, "near-tie alternatives", len(alt))


@pytest.mark.parametrize("variant", ["hot_expert", "one_chunk", "two_rows_per_expert"])
def test_layer_small_tiles(variant):
    """32-row tiles of the pipelined grouped GEMM (K a multiple of 128, at most 16 rows per expert on average):
    a hot expert that spans many tiles, K of one 128-wide chunk, and a full-size-like spread of 1-5 rows."""
    base = CONFIGS["tiny_t8_h512_e32"]
    cfg = {"hot_expert": base.with_(tokens=400, n_experts=256, top_k=4, bias="zipf", zipf_alpha=1.0),
           "one_chunk": base.with_(tokens=50, n_experts=64, hidden=128, inter=128, shared_inter=128),
           "two_rows_per_expert": base.with_(tokens=64, n_experts=192, hidden=1024, inter=384,
                                             shared_inter=256)}[variant]
    inp = make_inputs(cfg, seed=31, device=DEV)
    gpu = gpu_layer(inp)
    load = np.bincount(gpu[1].cpu().numpy().reshape(-1), minlength=cfg.n_experts)
    assert load.sum() / max(1, np.count_nonzero(load)) <= 16
    if variant == "hot_expert":
        assert load.max() > 64, load.max()  # three or more tiles for one expert
    stats, _, alt = _check_layer(inp, gpu=gpu)
    print(f"{variant}: max load {load.max()}", stats, "near-tie alternatives", len(alt))


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 7, 8, 16])
def test_layer_top_k_range(k):
    inp = make_inputs(CONFIGS["tiny_t8_h512_e32"].with_(tokens=12, top_k=k), seed=3, device=DEV)
    _check_layer(inp)


@pytest.mark.parametrize("e,k", [(1, 1), (2, 2), (128, 3), (1000, 6)])
def test_layer_expert_counts(e, k):
    inp = make_inputs(CONFIGS["tiny_t8_h512_e32"].with_(tokens=24, n_experts=e, top_k=k, hidden=256, inter=64,
                                                         shared_inter=96), seed=4, device=DEV)
    _check_layer(inp)


@pytest.mark.parametrize("variant", ["min_dims", "ragged_k", "no_shared", "zipf_bias"])
def test_layer_shapes(variant):
    base = CONFIGS["tiny_t8_h512_e32"]
    cfg = {"min_dims": base.with_(hidden=32, inter=32, shared_inter=32),
           "ragged_k": base.with_(tokens=33, hidden=160, inter=96, shared_inter=224),
           "no_shared": base.with_(n_shared=0, shared_inter=0),
           "zipf_bias": base.with_(tokens=64, bias="zipf")}[variant]
    _check_layer(make_inputs(cfg, seed=6, device=DEV))


def test_layer_clamp_stress():
    cfg = CONFIGS["tiny_t8_h512_e32"].with_(tokens=32, x_std=40.0)
    inp = make_inputs(cfg, seed=7, device=DEV)
    _, ref, _ = _check_layer(inp)
    # the clamp must actually fire on a good share of the gate pre-activations
    a = inp.oracle_args()
    x = oracle.bf16_bits_to_f64(a["x_bits"])
    e = int(ref["idx"][0, 0])
    wgu, _ = oracle.routed_expert_weights(a["gu_q"], a["gu_s"], a["dn_q"], a["dn_s"], e, cfg.hidden, cfg.inter)
    g = x @ wgu[:cfg.inter].T
    assert np.mean(g > cfg.swiglu_limit) > 0.1


def test_layer_zero_input_gives_exact_zero():
    inp = make_inputs(CONFIGS["tiny_t8_h512_e32"], seed=8, device=DEV)
    inp.x.zero_()
    y, idx, w = gpu_layer(inp)
    assert torch.all(y == 0)
    assert torch.all(idx.cpu() == torch.arange(6, dtype=torch.int32)[None, :])


def test_layer_zero_routed_weights_gives_shared_output():
    inp = make_inputs(CONFIGS["tiny_t8_h512_e32"], seed=9, device=DEV)
    inp.gu_q.zero_()
    gpu = gpu_layer(inp)
    y = gpu[0]
    _check_layer(inp, gpu=gpu)
    ref_sh = oracle.shared_expert(inp.x.cpu().numpy().view(np.uint16), inp.sh_gu.cpu().numpy().view(np.uint16),
                                  inp.sh_dn.cpu().numpy().view(np.uint16), 10.0)[1]
    assert_bar(bf16_to_f64(y), ref_sh, "y vs shared")


def test_layer_down_scale_plus_one():
    inp = make_inputs(CONFIGS["tiny_t8_h512_e32"], seed=10, device=DEV)
    inp.dn_s += 1
    _check_layer(inp)


def test_layer_deterministic():
    inp = make_inputs(CONFIGS["tiny_t8_h512_e32"].with_(tokens=300), seed=11, device=DEV)
    a = gpu_layer(inp)
    b = gpu_layer(inp)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_layer_many_tokens_small_dims():
    """A large token count (multi-chunk permutation, many tiles) on a small layer, sampled."""
    cfg = CONFIGS["tiny_t8_h512_e32"].with_(tokens=1 << 18, hidden=64, inter=32, shared_inter=32)
    inp = make_inputs(cfg, seed=12, device=DEV)
    gpu = gpu_layer(inp)
    idx = gpu[1].cpu().numpy()
    assert idx.min() >= 0 and idx.max() < cfg.n_experts
    _check_layer(inp, tokens=_sample(cfg.tokens, 48, seed=2), gpu=gpu)


# ------------------------------------------------------------------ pre-FFN RMSNorm

def _norm_inputs(t, h, seed):
    """bf16 rows of scales 2^-30..2^30 with special rows (zero, constant, one huge element over tiny ones whose
    normalised values are bf16 subnormals), and a gain ~N(1, 0.1^2) with a few zeros and sign flips."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    x = torch.randn((t, h), generator=g) * torch.exp2(torch.randint(-30, 31, (t, 1), generator=g).float())
    if t > 1:
        x[1] = 0.0
    if t > 2:
        x[2] = 0.375
    if t > 3:
        x[3] = torch.randn(h, generator=g) * 2.0 ** -116
        x[3, 0] = 2.0 ** 20
    gam = 1.0 + 0.1 * torch.randn(h, generator=g)
    gam[:: 97] = 0.0
    gam[5:: 131] *= -1.0
    bits = lambda v: v.to(torch.bfloat16).view(torch.int16)  # noqa: E731
    return bits(x).to(DEV), bits(gam).to(DEV)


@pytest.mark.parametrize("t,h", [(1, 5120), (7, 5120), (3, 7168), (5, 32), (9, 8192), (4, 8224), (2, 65536),
                                 (1000, 512), (4096, 5120), (20000, 256)])
def test_rmsnorm_bit_exact(t, h):
    """moe_rmsnorm against the oracle bit for bit (single-pass rows up to 8192, two-pass beyond), in place too."""
    x, gam = _norm_inputs(t, h, seed=t * 7 + h)
    cfg = moe.make_config(h, 8, 2, 32)
    out = torch.empty_like(x)
    moe.moe_rmsnorm(cfg, gam, x, t, out)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(x.cpu().numpy().view(np.uint16), gam.cpu().numpy().view(np.uint16), 1e-20)
    got = out.cpu().numpy().view(np.uint16)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:4].tolist()}"
    if t > 3:
        sub = oracle.bf16_bits_to_f64(ref[3])
        assert np.any((sub != 0) & (np.abs(sub) < 2.0 ** -126)), "row 3 should reach bf16 subnormals"
    moe.moe_rmsnorm(cfg, gam, x, t, x)  # in place
    torch.cuda.synchronize()
    assert torch.equal(x, out)


@pytest.mark.parametrize("tokens,variant", [(1, "tiny"), (2, "tiny"), (1, "min_dims"), (2, "ragged_k"),
                                            (1, "no_shared"), (2, "v4pro_dims"), (5, "tiny"), (8, "tiny"),
                                            (64, "tiny"), (300, "tiny"), (17, "ragged_k")])
def test_layer_with_norm(tokens, variant):
    """The layer with the pre-FFN norm: in the router launch for one or two tokens (hidden <= 5120), a norm
    launch of its own otherwise; x itself is left as it was."""
    base = CONFIGS["tiny_t8_h512_e32"].with_(tokens=tokens, norm=True)
    cfg = {"tiny": base,
           "min_dims": base.with_(hidden=32, inter=32, shared_inter=32, n_experts=4, top_k=2),
           "ragged_k": base.with_(hidden=160, inter=96, shared_inter=224),
           "no_shared": base.with_(n_shared=0, shared_inter=0),
           "v4pro_dims": CONFIGS["decode_t1_h5120_e384"].with_(tokens=tokens, hidden=7168, inter=3072,
                                                                 shared_inter=3072, n_experts=16, norm=True)}[variant]
    inp = make_inputs(cfg, seed=40 + tokens, device=DEV)
    x0 = inp.x.clone()
    stats, _, alt = _check_layer(inp)
    assert torch.equal(inp.x, x0)
    print(f"norm T={tokens} {variant}:", stats, "near-tie alternatives", len(alt))


def test_layer_with_norm_decode_t1_full():
    """Full-size one-token layer with the norm: three launches, the norm inside the first."""
    inp = make_inputs(CONFIGS["decode_t1_h5120_e384_norm"], seed=0, device=DEV)
    stats, _, alt = _check_layer(inp)
    print("decode_t1 norm:", stats, "near-tie alternatives", len(alt))
    cfg = moe.config_from(inp.cfg)
    y = torch.empty((1, inp.cfg.hidden), dtype=torch.int16, device=DEV)
    names = [n for n, _ in moe.moe_layer_forward_timed(cfg, moe.weights_from(inp), inp.x, 1, y,
                                                       moe.workspace(cfg, 1, device=DEV))]
    assert names == ["norm_router_scores", "route_gate_up_shared_gate_up", "routed_down_shared_down_combine"]


def test_layer_with_norm_prefill_sampled():
    cfg = CONFIGS["prefill_t4096_h5120_e384"].with_(norm=True)
    inp = make_inputs(cfg, seed=0, device=DEV)
    gpu = gpu_layer(inp)
    stats, _, alt = _check_layer(inp, tokens=_sample(cfg.tokens, 6, seed=3), gpu=gpu)
    print("prefill norm sampled:", stats, "near-tie alternatives", len(alt))


def test_layer_with_norm_zero_input():
    inp = make_inputs(CONFIGS["tiny_t8_h512_e32"].with_(norm=True), seed=8, device=DEV)
    inp.x.zero_()
    y, idx, _ = gpu_layer(inp)
    assert torch.all(y == 0)
    assert torch.all(idx.cpu() == torch.arange(6, dtype=torch.int32)[None, :])



# ------------------------------------------------------------------ MXFP8 (E4M3) routed experts

@pytest.mark.parametrize("tokens,variant", [(1, "tiny"), (2, "tiny"), (5, "tiny"), (64, "tiny"), (300, "tiny"),
                                            (1, "min_dims"), (2, "ragged_k"), (7, "no_shared"), (3, "k16"),
                                            (2, "v4pro_dims"), (40, "norm"), (1, "norm"), (1, "v4pro_dims"),
                                            (2, "k1"), (1, "all_experts"), (1000, "few_experts"),
                                            (700, "ragged_k")])
def test_layer_fp8(tokens, variant):
    """MXFP8 experts: one and two tokens take the streaming kernels where their vector counts are built
    (up to 14 vectors per lane), every other shape the grouped GEMM."""
    base = CONFIGS["tiny_t8_h512_e32"].with_(tokens=tokens, expert_format="mxfp8")
    cfg = {"tiny": base,
           "min_dims": base.with_(hidden=32, inter=32, shared_inter=32, n_experts=4, top_k=2),
           "ragged_k": base.with_(hidden=160, inter=96, shared_inter=224),
           "no_shared": base.with_(n_shared=0, shared_inter=0),
           "k16": base.with_(top_k=16),
           "norm": base.with_(norm=True),
           "k1": base.with_(top_k=1),
           "all_experts": base.with_(n_experts=8, top_k=8),
           "few_experts": base.with_(n_experts=8, top_k=2),  # ~250 rows per expert: several 96-row tiles
           "v4pro_dims": CONFIGS["decode_t1_h5120_e384"].with_(tokens=tokens, hidden=7168, inter=3072,
                                                                 shared_inter=3072, n_experts=16,
                                                                 expert_format="mxfp8")}[variant]
    inp = make_inputs(cfg, seed=60 + tokens, device=DEV)
    stats, _, alt = _check_layer(inp)
    print(f"fp8 T={tokens} {variant}:", stats, "near-tie alternatives", len(alt))


@pytest.mark.parametrize("tokens", [16, 512])
def test_layer_fp8_every_code(tokens):
    """Every finite E4M3 code, under block scales 2^-20 .. 2^-12, in both projections of every expert
    (16 tokens: 16-row tiles; 512 tokens: 96-row tiles)."""
    cfg = CONFIGS["tiny_t8_h512_e32"].with_(tokens=tokens, expert_format="mxfp8", n_experts=8, top_k=4)
    inp = make_inputs(cfg, seed=70, device=DEV)
    g = torch.Generator().manual_seed(71)
    finite = torch.tensor([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=torch.uint8)
    for q, sc in ((inp.gu_q, inp.gu_s), (inp.dn_q, inp.dn_s)):
        n = q.numel()
        codes = finite[torch.arange(n) % len(finite)]
        q.copy_(codes[torch.randperm(n, generator=g)].reshape(q.shape).to(DEV))
        # scales that keep the expert outputs in a moderate range (values up to 448 * 2^-12)
        sc.copy_(torch.randint(107, 116, sc.shape, generator=g, dtype=torch.uint8).to(DEV))
    stats, _, alt = _check_layer(inp)
    print("fp8 every code:", stats, "near-tie alternatives", len(alt))


def test_layer_fp8_decode_t1_full():
    inp = make_inputs(CONFIGS["decode_t1_h5120_e384_fp8"], seed=0, device=DEV)
    stats, _, alt = _check_layer(inp)
    print("decode_t1 fp8:", stats, "near-tie alternatives", len(alt))
    cfg = moe.config_from(inp.cfg)
    y = torch.empty((1, inp.cfg.hidden), dtype=torch.int16, device=DEV)
    names = [n for n, _ in moe.moe_layer_forward_timed(cfg, moe.weights_from(inp), inp.x, 1, y,
                                                       moe.workspace(cfg, 1, device=DEV))]
    assert names == ["router_scores_shared_gate_up", "route_gate_up_shared_down", "routed_down_combine"]


@pytest.mark.parametrize("tokens", [2, 3, 5, 6])
def test_layer_fp8_few_tokens_full(tokens):
    """MXFP8 experts at 2-6 tokens at full size take the few-token MFMA kernels (E4M3 weights fed to the
    block-scaled instruction as its 8-bit operand, two-term MXFP8 x; the split-K down projection), not the
    grouped GEMM; every token against the oracle.  Two tokens: the vector-ALU gate/up with the MFMA down
    projection (the streaming down kernel holds at most 14 E4M3 vectors per lane).  From 7 tokens the staged
    x rows of H = 5120 pass the few-token kernels' 64 KB of LDS and both formats take the grouped GEMM."""
    cfg = CONFIGS["decode_t1_h5120_e384_fp8"].with_(tokens=tokens)
    inp = make_inputs(cfg, seed=100 + tokens, device=DEV)
    stats, _, alt = _check_layer(inp)
    print(f"fp8 T={tokens} full:", stats, "near-tie alternatives", len(alt))
    c = moe.config_from(cfg)
    y = torch.empty((tokens, cfg.hidden), dtype=torch.int16, device=DEV)
    names = [n for n, _ in moe.moe_layer_forward_timed(c, moe.weights_from(inp), inp.x, tokens, y,
                                                       moe.workspace(c, tokens, device=DEV))]
    assert names == ["router_shared_gate_up", "route_shared_down", "routed_gate_up", "routed_down", "combine"], names


def test_layer_fp8_prefill_sampled():
    cfg = CONFIGS["prefill_t4096_h5120_e384_fp8"]
    inp = make_inputs(cfg, seed=0, device=DEV)
    gpu = gpu_layer(inp)
    stats, _, alt = _check_layer(inp, tokens=_sample(cfg.tokens, 6, seed=4), gpu=gpu)
    print("prefill fp8 sampled:", stats, "near-tie alternatives", len(alt))


@pytest.mark.parametrize("e,k,tokens", [(1, 1, 3), (2, 2, 1), (128, 3, 40), (1000, 6, 2), (1000, 6, 24)])
def test_layer_fp8_expert_counts(e, k, tokens):
    """MXFP8 experts across expert counts and top-k (streaming kernels at one or two tokens, grouped GEMM
    otherwise)."""
    cfg = CONFIGS["tiny_t8_h512_e32"].with_(tokens=tokens, n_experts=e, top_k=k, expert_format="mxfp8")
    inp = make_inputs(cfg, seed=80 + e, device=DEV)
    stats, _, alt = _check_layer(inp)
    print(f"fp8 E={e} k={k} T={tokens}:", stats, "near-tie alternatives", len(alt))


@pytest.mark.parametrize("tokens", [1, 3, 5, 6, 8])
def test_layer_few_tokens_duplicate_router_rows(tokens):
    """The one-block routing of the few-token paths (tokens 5..8 take two tokens per wave): equal
    router rows give equal scores, taken lowest index first; the layer matches the oracle."""
    cfg = CONFIGS["tiny_t8_h512_e32"].with_(tokens=tokens)
    inp = make_inputs(cfg, seed=90 + tokens, device=DEV)
    inp.router_w[20] = inp.router_w[3]
    inp.router_w[31] = inp.router_w[3]
    y, idx, w = gpu_layer(inp)
    for row in idx.cpu().numpy().tolist():
        have = [e for e in (3, 20, 31) if e in row]
        if have:
            pos = [row.index(e) for e in have]
            assert have == [3, 20, 31][:len(have)] and pos == list(range(pos[0], pos[0] + len(pos)))
    stats, _, alt = _check_layer(inp, gpu=(y, idx, w))
    print(f"T={tokens} duplicate router rows:", stats, "near-tie alternatives", len(alt))
