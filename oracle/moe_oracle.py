"""Plain float64 CPU oracle of the DeepSeek-V4.1-Flash routed MoE FFN layer.

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the CPU
baseline of the benchmark, never by the product path.  It shares no code with
the HIP library.

What the layer computes, and where the pages state it:

* 384 routed experts, 6 used per token, 1 shared expert, expert width 2304 on
  a 5120-wide hidden state, ``routed_scaling_factor`` 1.5, ``swiglu_limit``
  10.0 -- max.pipelines.architectures.deepseekV41 API reference,
  ``DeepseekV41Config`` (class signature and its field entries); the same
  numbers in the checkpoint ``config.json`` shown on the "DeepSeek V4.1" atlas
  page (``n_routed_experts``, ``n_activated_experts``, ``n_shared_experts``,
  ``moe_inter_dim``, ``route_scale``, ``swiglu_limit``).
* The router's score function is ``"sqrtsoftplus"`` -- atlas page,
  ``config.json`` key ``score_func``.  The pages only name it.
* Experts are gated MLPs and the shared expert has width ``d_shared`` 2304 --
  "DeepSeek-V4.1-Flash" architecture sheet, table "Every architecture field"
  (rows ``ffns.moe.gated``, ``ffns.moe.d_shared``).
* Routed experts are stored as MXFP4 and everything else as BF16 -- Strata's
  DEEPSEEK41 notes, opening paragraph; 18.8 MB per routed expert -- same
  notes, table "Where it goes".  MXFP4 elements are ``float4_e2m1fnx2`` (two
  E2M1 codes a byte) -- API reference, ``SUPPORTED_ENCODINGS``; the scale is an
  E8M0 byte per 32 elements -- "DeepSeek-V4-Pro" record, KV-layout passage
  (``float8_e8m0`` scales, one per 32 values).

Readings taken where the pages are silent (each also listed in the design
notes of the repository):

* sqrtsoftplus(z) = sqrt(softplus(z)), softplus(z) = log(1 + e^z), applied to
  each logit on its own (no normalisation across experts).
* An optional per-expert router bias is added to the scores for *selection
  only*; the combine weights use the unbiased scores.
* Top-k order is by score descending, ties to the lower expert index.
* The k selected scores are renormalised to sum 1 and multiplied by the route
  scale.  The route scale applies to routed experts only; the shared expert's
  weight is 1.
* swiglu_limit L: the gate pre-activation is clamped to at most L (no lower
  clamp), the up pre-activation to [-L, L], before silu; h = silu(g) * u.  The
  same clamp applies to the shared expert.
* Gate/up weights of an expert are one [2I, H] matrix: rows 0..I-1 gate,
  rows I..2I-1 up.
* MXFP4 layout: element 2i of a row in the low nibble of byte i, element
  2i+1 in the high nibble; one E8M0 byte per 32 consecutive elements of a row,
  stored as a separate [rows, K/32] array.
* y = shared(x) + sum_j w_j * expert_{idx_j}(x); no residual.
* Optional pre-FFN norm (off unless a gain vector is given): the MAX API's
  ``DeepseekV41Config`` has ``rms_norm_eps`` = 1e-20 and the atlas page's
  ``config.json`` ``norm_eps`` = 1e-20, while the architecture sheet lists the
  norm type as not disclosed.  Reading: RMSNorm over the hidden dimension,
  x_n = x / sqrt(mean(x^2) + eps) * gamma with a bf16 gain gamma, its output
  rounded to bf16 (nearest, ties to even) before the router and the experts.
* Optional second expert-weight codec, MXFP8: the API reference lists
  ``float8_e4m3fn`` among ``SUPPORTED_ENCODINGS`` (and as ``DEFAULT_ENCODING``)
  and the checkpoint's dense ``dtype`` is ``"fp8"``.  Reading: E4M3 codes of
  the OCP "fn" kind (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
  infinities; S.1111.111 is NaN; largest value 448), one byte per element in
  row order, with the same E8M0 scale per 32 consecutive elements of a row as
  the MXFP4 weights (the block the "DeepSeek-V4-Pro" record gives for its
  e4m3 values).
"""

from __future__ import annotations

import itertools

import numpy as np

# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------



def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns: bf16 is the high half of binary32."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v) -> np.ndarray:
    """bf16 bit patterns of the values nearest to ``v`` (ties to an even significand).

    A normal bf16 has 8 significant bits: with v = m * 2^e, 0.5 <= |m| < 1,
    the rounded value is rint(m * 2^8) * 2^(e - 8), ``rint`` rounding halves to
    even.  Below 2^-126 bf16 is subnormal with the fixed step 2^-133.  Zeros
    keep their sign; overflow past the largest bf16 is not needed here.
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    r = np.where(np.abs(v) < 2.0 ** -126, np.rint(v * 2.0 ** 133) * 2.0 ** -133,
                 np.ldexp(np.rint(m * 256.0), e - 8))
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def rmsnorm(x_bits, gamma_bits, eps: float) -> np.ndarray:
    """RMSNorm of each row of bf16 ``x_bits`` with bf16 gain ``gamma_bits``,
    rounded to bf16 bits: x / sqrt(mean(x^2) + eps) * gamma (reading above)."""
    x = bf16_bits_to_f64(x_bits)
    g = bf16_bits_to_f64(gamma_bits)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return f64_to_bf16_bits(x * r * g)


def e2m1_value(code: int) -> float:
    """Value of one 4-bit E2M1 code, from the format's field definition.

    Exponent field 0 is subnormal: (-1)^s * 2^(1-bias) * (m / 2).
    Otherwise (-1)^s * 2^(e-bias) * (1 + m / 2).
    """
    code = int(code) & 0xF
    s = (code >> 3) & 1
    e = (code >> 1) & 0x3
    m = code & 1
    if e == 0:
        mag = 2.0 ** (1 - 1) * (m / 2.0)
    else:
        mag = 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


def e2m1_table() -> np.ndarray:
    """The 16 E2M1 values indexed by code (code 8 is -0.0)."""
    return np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e8m0_value(code) -> np.ndarray:
    """E8M0 scale: an unsigned biased exponent, 2^(code-127); 0xFF is NaN."""
    c = np.asarray(code).astype(np.int64)
    v = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, v)


def decode_mxfp4(packed, scales, k: int) -> np.ndarray:
    """Decode MXFP4 rows to float64.

    ``packed``: uint8 [..., k/2], two E2M1 codes a byte (even element in the
    low nibble).  ``scales``: uint8 [..., k/32], one E8M0 byte per 32
    consecutive elements.  Returns float64 [..., k], element
    i = E2M1(code_i) * 2^(scale_{i // 32} - 127).
    """
    packed = np.asarray(packed, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    assert packed.shape[-1] * 2 == k and scales.shape[-1] * 32 == k
    codes = np.empty(packed.shape[:-1] + (k,), dtype=np.uint8)
    codes[..., 0::2] = packed & 0x0F
    codes[..., 1::2] = packed >> 4
    values = e2m1_table()[codes]
    block_scale = np.repeat(e8m0_value(scales), 32, axis=-1)
    return values * block_scale




def e4m3_value(code: int) -> float:
    """Value of one 8-bit E4M3 code from its fields: exponent field 0 is
    subnormal, (-1)^s * 2^(1-7) * (m / 8); otherwise (-1)^s * 2^(e-7) * (1 + m / 8);
    e = 15 with m = 7 is NaN."""
    code = int(code) & 0xFF
    s = code >> 7
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 15 and m == 7:
        return float("nan")
    mag = 2.0 ** -6 * (m / 8.0) if e == 0 else 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return -mag if s else mag


def e4m3_table() -> np.ndarray:
    """The 256 E4M3 values indexed by code (code 0x80 is -0.0; 0x7F and 0xFF are NaN)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode_mxfp8(codes, scales, k: int) -> np.ndarray:
    """Decode MXFP8 rows to float64.

    ``codes``: uint8 [..., k], one E4M3 code per element.  ``scales``: uint8
    [..., k/32], one E8M0 byte per 32 consecutive elements.  Element
    i = E4M3(code_i) * 2^(scale_{i // 32} - 127).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    assert codes.shape[-1] == k and scales.shape[-1] * 32 == k
    return e4m3_table()[codes] * np.repeat(e8m0_value(scales), 32, axis=-1)


#: expert-weight codecs: name -> (decoder, elements per code byte)
EXPERT_FORMATS = {"mxfp4": (decode_mxfp4, 2), "mxfp8": (decode_mxfp8, 1)}


def mxfp4_packed_bytes(rows: int, k: int) -> int:
    """Bytes of an MXFP4 matrix [rows, k]: k/2 code bytes + k/32 scale bytes a row."""
    assert k % 32 == 0
    return rows * (k // 2 + k // 32)


# ---------------------------------------------------------------------------
# Elementwise functions
# ---------------------------------------------------------------------------


def softplus(z) -> np.ndarray:
    """log(1 + e^z), written as max(z, 0) + log1p(e^-|z|) so it never overflows."""
    z = np.asarray(z, dtype=np.float64)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def sqrtsoftplus(z) -> np.ndarray:
    """The ``sqrtsoftplus`` score of the checkpoint config: sqrt(softplus(z))."""
    return np.sqrt(softplus(z))


def silu(z) -> np.ndarray:
    """z * sigmoid(z) = z / (1 + e^-z)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def clamped_swiglu(g, u, limit: float) -> np.ndarray:
    """silu(min(g, L)) * clip(u, -L, L), the gated activation with ``swiglu_limit``."""
    g = np.minimum(np.asarray(g, dtype=np.float64), limit)
    u = np.clip(np.asarray(u, dtype=np.float64), -limit, limit)
    return silu(g) * u


# ---------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------


def router_logits(x_bits, router_w) -> np.ndarray:
    """Logits l[t, e] = sum_h x[t, h] * W_r[e, h], exact inputs, float64 matmul."""
    x = bf16_bits_to_f64(x_bits)
    w = np.asarray(router_w, dtype=np.float32).astype(np.float64)
    return x @ w.T


def _selection_order(u_row: np.ndarray) -> np.ndarray:
    """Expert indices sorted by (u descending, index ascending)."""
    e = np.arange(u_row.shape[0])
    return np.lexsort((e, -u_row))


def route_with_selection(s_row, idx_row, route_scale: float) -> np.ndarray:
    """Combine weights for a given selection: rho * s_i / sum of the selected s."""
    s_sel = np.asarray(s_row, dtype=np.float64)[np.asarray(idx_row)]
    total = s_sel.sum()
    if total == 0.0:
        return np.full(s_sel.shape, route_scale / s_sel.shape[0])
    return route_scale * s_sel / total


def route(x_bits, router_w, router_bias, top_k: int, route_scale: float) -> dict:
    """Router of the layer for every token row of ``x_bits``.

    Returns ``idx`` int32 [T, k] (rows in selection order), ``w`` float64
    [T, k], ``gap`` float64 [T] = u(k) - u(k+1) (+inf when k == E), and the
    intermediates ``logits``, ``s`` (scores) and ``u`` (selection scores).
    """
    logits = router_logits(x_bits, router_w)
    s = sqrtsoftplus(logits)
    u = s.copy()
    if router_bias is not None:
        u = u + np.asarray(router_bias, dtype=np.float32).astype(np.float64)[None, :]
    t_count, n_exp = s.shape
    idx = np.zeros((t_count, top_k), dtype=np.int32)
    w = np.zeros((t_count, top_k), dtype=np.float64)
    gap = np.full((t_count,), np.inf, dtype=np.float64)
    for t in range(t_count):
        order = _selection_order(u[t])
        idx[t] = order[:top_k]
        w[t] = route_with_selection(s[t], idx[t], route_scale)
        if top_k < n_exp:
            gap[t] = u[t, order[top_k - 1]] - u[t, order[top_k]]
    return {"idx": idx, "w": w, "gap": gap, "logits": logits, "s": s, "u": u}


def valid_selections(u_row, top_k: int, tol: float, max_pool: int = 16) -> list:
    """Every selection (as a list in selection order) that counts as correct.

    A selection S is correct when no expert left out beats an expert taken in,
    except by a margin of at most ``tol`` between two unequal scores; exactly
    equal scores go to the lower index.  With ``tol`` = 0 this is the single
    exact top-k.  Experts that could take part in a swap are those within
    ``tol`` of the k-th score; when more than ``max_pool`` of them exist the
    exact selection is the only one returned.
    """
    u_row = np.asarray(u_row, dtype=np.float64)
    order = _selection_order(u_row)
    exact = [int(e) for e in order[:top_k]]
    if tol <= 0.0 or top_k >= u_row.shape[0]:
        return [exact]
    kth = u_row[order[top_k - 1]]
    pool = [int(e) for e in order if u_row[e] >= kth - tol]
    if len(pool) > max_pool:
        return [exact]
    must = [e for e in order[:top_k] if u_row[e] > kth + tol]
    rest = [e for e in pool if e not in must]
    need = top_k - len(must)

    def beats(i, j):  # expert i may be taken while j is left out
        if u_row[i] > u_row[j] or (u_row[i] == u_row[j] and i < j):
            return True
        return u_row[i] != u_row[j] and u_row[j] - u_row[i] <= tol

    out = []
    for combo in itertools.combinations(rest, need):
        sel = set(must) | set(combo)
        left = [j for j in pool if j not in sel]
        if all(beats(i, j) for i in sel for j in left):
            out.append([int(e) for e in order if e in sel])
    return out


# ---------------------------------------------------------------------------
# Permutation of (token, slot) pairs into expert-contiguous order
# ---------------------------------------------------------------------------


def permute(idx, n_experts: int) -> dict:
    """Stable counting sort of the flat slots f = t*k + j by expert.

    ``expert_offsets`` [E+1]: start of each expert's run; ``sorted_slots``
    [T*k]: the flat slot at each position (ascending f within an expert);
    ``slot_pos`` [T*k]: the position of each flat slot (inverse permutation).
    """
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    sorted_slots = np.argsort(flat, kind="stable").astype(np.int32)
    slot_pos = np.empty_like(sorted_slots)
    slot_pos[sorted_slots] = np.arange(flat.shape[0], dtype=np.int32)
    return {"expert_offsets": offsets, "sorted_slots": sorted_slots, "slot_pos": slot_pos}


# ---------------------------------------------------------------------------
# Experts and combine
# ---------------------------------------------------------------------------


def expert_mlp(x, w_gate_up, w_down, limit: float):
    """A gated MLP: g = x W_g^T, u = x W_u^T, h = clamped_swiglu(g, u), o = h W_d^T.

    ``x`` float64 [M, H]; ``w_gate_up`` float64 [2I, H] (gate rows first);
    ``w_down`` float64 [H, I].  Returns (h [M, I], o [M, H]).
    """
    inter = w_down.shape[1]
    g = x @ w_gate_up[:inter].T
    u = x @ w_gate_up[inter:].T
    h = clamped_swiglu(g, u, limit)
    return h, h @ w_down.T


def shared_expert(x_bits, sh_gu_bits, sh_dn_bits, limit: float):
    """The always-on shared expert with bf16 weights; returns (h, o) in float64."""
    x = bf16_bits_to_f64(x_bits)
    return expert_mlp(x, bf16_bits_to_f64(sh_gu_bits), bf16_bits_to_f64(sh_dn_bits), limit)


def routed_expert_weights(gu_q, gu_s, dn_q, dn_s, e: int, hidden: int, inter: int, expert_format: str = "mxfp4"):
    """Decoded float64 gate/up [2I, H] and down [H, I] matrices of routed expert e."""
    decode = EXPERT_FORMATS[expert_format][0]
    w_gu = decode(np.asarray(gu_q[e]), np.asarray(gu_s[e]), hidden)
    w_dn = decode(np.asarray(dn_q[e]), np.asarray(dn_s[e]), inter)
    return w_gu, w_dn


def combine(y_slot, slot_pos, w, y_shared, top_k: int) -> np.ndarray:
    """y[t] = y_shared[t] + sum over j of w[t, j] * y_slot[slot_pos[t*k + j]]."""
    y_slot = np.asarray(y_slot, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    t_count = w.shape[0]
    y = np.zeros((t_count, y_slot.shape[1])) if y_shared is None else np.array(y_shared, dtype=np.float64)
    for t in range(t_count):
        for j in range(top_k):
            y[t] += w[t, j] * y_slot[slot_pos[t * top_k + j]]
    return y


def layer_forward(x_bits, router_w, router_bias, gu_q, gu_s, dn_q, dn_s, sh_gu, sh_dn,
                  top_k: int, route_scale: float, swiglu_limit: float,
                  tokens=None, selections=None, norm_gamma=None, norm_eps: float = 1e-20,
                  expert_format: str = "mxfp4", workers: int = 1) -> dict:
    """The whole layer for the rows ``tokens`` of ``x_bits`` (all rows if None).

    ``gu_q`` ... ``dn_s`` only need to support ``[e]`` (per-expert arrays of
    the packed layout).  ``sh_gu``/``sh_dn`` are None when there is no shared
    expert.  ``selections`` optionally replaces the routed selection of each
    row by one of the oracle's own ``valid_selections``.

    With ``norm_gamma`` (bf16 bits [H]) the rows are first RMS-normalised
    (``rmsnorm``) and the layer runs on the result.  ``expert_format`` names
    the routed experts' codec, "mxfp4" or "mxfp8".  ``workers`` > 1 runs the
    selected experts on that many threads (each writes only its own rows; every
    expert's arithmetic is the same as with one thread).

    Returns the router outputs, the permutation, ``h_slot`` [T*k, I] and
    ``y_slot`` [T*k, H] in position order, ``y_shared`` [T, H] and ``y`` [T, H].
    """
    x_bits = np.asarray(x_bits)
    if tokens is not None:
        x_bits = x_bits[np.asarray(tokens)]
    if norm_gamma is not None:
        x_bits = rmsnorm(x_bits, norm_gamma, norm_eps)
    t_count, hidden = x_bits.shape
    r = route(x_bits, router_w, router_bias, top_k, route_scale)
    idx, w = r["idx"], r["w"]
    if selections is not None:
        idx = np.asarray(selections, dtype=np.int32).reshape(t_count, top_k)
        w = np.stack([route_with_selection(r["s"][t], idx[t], route_scale) for t in range(t_count)]) \
            if t_count else w
    n_experts = np.asarray(router_w).shape[0]
    p = permute(idx, n_experts)
    x = bf16_bits_to_f64(x_bits)
    per_byte = EXPERT_FORMATS[expert_format][1]
    inter = (dn_q.shape[-1] if hasattr(dn_q, "shape") else np.asarray(dn_q[0]).shape[-1]) * per_byte
    h_slot = np.zeros((t_count * top_k, inter))
    y_slot = np.zeros((t_count * top_k, hidden))

    def one_expert(e):
        lo, hi = int(p["expert_offsets"][e]), int(p["expert_offsets"][e + 1])
        w_gu, w_dn = routed_expert_weights(gu_q, gu_s, dn_q, dn_s, e, hidden, inter, expert_format)
        rows = p["sorted_slots"][lo:hi] // top_k
        h_slot[lo:hi], y_slot[lo:hi] = expert_mlp(x[rows], w_gu, w_dn, swiglu_limit)

    used = [e for e in range(n_experts) if p["expert_offsets"][e + 1] > p["expert_offsets"][e]]
    if workers > 1 and len(used) > 1:
        from concurrent.futures import ThreadPoolExecutor

        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(max_workers=workers) as pool:
            list(pool.map(one_expert, used))
    else:
        for e in used:
            one_expert(e)
    if sh_gu is not None:
        h_sh, y_sh = shared_expert(x_bits, sh_gu, sh_dn, swiglu_limit)
    else:
        h_sh, y_sh = None, np.zeros((t_count, hidden))
    y = combine(y_slot, p["slot_pos"], w, y_sh, top_k)
    out = dict(r)
    out.update(p)
    out.update({"idx": idx, "w": w, "h_slot": h_slot, "y_slot": y_slot, "h_shared": h_sh,
                "y_shared": y_sh, "y": y})
    return out
