"""Plain CPU definition of the zero-computation-expert MoE layer (fp64).

TEST INFRASTRUCTURE ONLY -- imported by tests, the smoke check and the
benchmark's CPU-baseline leg; never by the product path. It shares no code,
table or constant with the HIP library.

Every function follows a passage of the "LongCat-Flash" llm-wiki entity page
(cited per function) or one of the readings listed where that page is silent:

  R-bias   the expert bias enters selection only: s = fl32(z + b) on the fp32
           router logit; the gates never see it.
  R-gate   gates are one softmax over all N+Z unbiased logits, read at the
           selected experts, not renormalised over the K chosen ones.
  R-ffn    an FFN expert is SiLU-gated: W2 (silu(W1 x) * (W3 x)), with the
           gate rows W1 stacked above the up rows W3 in one [2I, d] matrix.
  R-tie    selection order is (score descending, expert index ascending);
           -0 and +0 compare equal.
  R-upd    the bias update is applied to the N FFN experts only, computed in
           fp64 as mu*(K_e*T_all - N*T_i)/(K*N*T_all) and rounded once into
           the fp32 bias.
  R-fp8    fp8 weights are OCP E4M3FN codes with one fp32 scale per 128x128
           block; the dequantised weight is fl32(q * s).
  R-grp    for the device-level balance statistic the N FFN experts form D
           groups of N/D consecutive experts (the placement of expert
           parallelism over D devices); the Z zero experts are group D+1.
  R-lb     P_j is the mean over tokens of the softmax mass (all N+Z unbiased
           logits) in group j; f_j is group j's share of the T*K selected
           slots divided by its target share, K_e/(K*D) for each FFN group
           and (K-K_e)/K for the zero group, so routing at the target ratio
           K_e : (K-K_e), even over the FFN groups, has f_j = 1 everywhere.
  R-zl     the hidden z-loss is taken over the layer input hidden states,
           i running over d_model.
  R-a8     fp8 activations (with fp8 weights): each FFN expert's input row
           (the token's x) and its intermediate row (H, after rounding to
           bf16) are quantized per row: s = fl32(amax / 448) (1 for an
           all-zero row), q = RNE to E4M3FN of fl32(v / s) clamped to +-448,
           value q * s. Zero-computation experts see the exact x.

Precision: all arithmetic on activations is fp64 except where a step is
defined in fp32 (the selection score, the fp8 dequantised weight, the bias
written back), where the fp32 rounding is reproduced explicitly.
"""

import numpy as np

# ----------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) -> float64 values.

    A bf16 value is the upper half of an IEEE binary32 word, so the decode is
    exact: shift into the high half, reinterpret as fp32, widen.
    """
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def e4m3fn_value_table():
    """Value of each of the 256 OCP FP8 E4M3FN codes, from the format definition.

    Layout S.EEEE.MMM, exponent bias 7. Exponent field 0 is subnormal
    (value m/8 * 2^(1-7)); exponent 15 with mantissa 7 is NaN; the format has
    no infinities (so exponent 15 with mantissa 0..6 is an ordinary normal).
    """
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


def dequant_fp8_blocks(codes, scales, block=128):
    """fp8 block-scaled weight -> fp32 weight, w = fl32(q * s)   (reading R-fp8).

    codes:  uint8 [R, C]; scales: fp32 [R/block, C/block].
    q is exact in fp32 (every E4M3 value is), so the fp32 product rounds once.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    R, C = codes.shape
    assert R % block == 0 and C % block == 0
    q = e4m3fn_value_table()[codes].astype(np.float32)
    s = np.asarray(scales, dtype=np.float32)
    assert s.shape == (R // block, C // block)
    s_full = np.repeat(np.repeat(s, block, axis=0), block, axis=1)
    return (q * s_full).astype(np.float32)


def e4m3fn_encode(v):
    """fp32 values -> OCP E4M3FN codes, round to nearest, ties to even.

    Written from the format: normals are (1 + m/8) * 2^(e-7), e in 1..15
    (e = 15 allows m <= 6; the largest finite value is 448), subnormals are
    m/8 * 2^-6. |v| is split into its binary exponent, the fraction scaled to
    eighths and rounded half-to-even (np.rint); a carry out of the mantissa
    moves to the next exponent. Inputs must already lie in [-448, 448].
    """
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    if np.any(np.abs(v) > 448.0) or np.any(np.isnan(v)):
        raise ValueError("e4m3fn_encode needs finite inputs within +-448")
    sign = np.signbit(v).astype(np.uint8) << 7
    a = np.abs(v)
    codes = np.zeros(a.shape, dtype=np.uint8)
    sub = a < 2.0 ** -6
    # subnormal range: multiples of 2^-9
    m_sub = np.rint(a[sub] / 2.0 ** -9).astype(np.int64)       # 0..8 (8 = min normal)
    codes[sub] = np.where(m_sub == 8, 1 << 3, m_sub).astype(np.uint8)
    an = a[~sub]
    e = np.floor(np.log2(an)).astype(np.int64)
    # guard the floating log2 at exact powers of two
    e = np.where(2.0 ** (e + 1) <= an, e + 1, e)
    e = np.where(2.0 ** e > an, e - 1, e)
    m = np.rint((an / 2.0 ** e - 1.0) * 8.0).astype(np.int64)   # 0..8
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    codes[~sub] = (((e + 7) << 3) | m).astype(np.uint8)
    return codes | sign


def quantize_rows_fp8(v):
    """Per-row activation quantization (reading R-a8): fp32 rows -> (codes
    uint8, scale fp32 per row). s = fl32(amax / 448), 1 for an all-zero row;
    q = e4m3fn_encode(clamp(fl32(v / s), -448, 448))."""
    v = np.asarray(v, dtype=np.float32)
    amax = np.abs(v).max(axis=1)
    s = np.where(amax > 0, (amax / np.float32(448.0)).astype(np.float32), np.float32(1.0))
    s = s.astype(np.float32)
    q = np.clip((v / s[:, None]).astype(np.float32), -448.0, 448.0)
    return e4m3fn_encode(q), s


def dequant_rows_fp8(codes, scales):
    """q * s per row, in fp64 (every E4M3 value times an fp32 scale is exact
    in fp64)."""
    q = e4m3fn_value_table()[np.asarray(codes, dtype=np.uint8)]
    return q * np.asarray(scales, dtype=np.float64)[:, None]


def round_to_bf16(v):
    """fp64 -> fp32 -> bf16 (round to nearest even at each step), as fp64."""
    u = np.asarray(v, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# Routing  ("LongCat-Flash", section 2.1: router picks K of the N+Z experts;
#           bias update drives the mean FFN-expert count per token to K_e)
# ----------------------------------------------------------------------------


def router_logits(x, w_router):
    """z[t, i] = sum_k W_r[i, k] * x[t, k], accumulated in fp64.

    x: [T, d] (values), w_router: [E, d] (fp32 values). Returns fp64 [T, E].
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_router, dtype=np.float64)
    return x @ w.T


def selection_scores(z32, bias):
    """s = fl32(fl32(z) + b), with -0 mapped to +0   (readings R-bias, R-tie)."""
    z32 = np.asarray(z32, dtype=np.float32)
    b = np.asarray(bias, dtype=np.float32)
    s = (z32 + b[None, :]).astype(np.float32)
    s[s == 0] = np.float32(0.0)
    return s


def select_topk(z32, bias, k):
    """Top-K experts per token under (score desc, index asc)   (section 2.1, R-tie).

    z32: the fp32 router logits [T, E]; bias: fp32 [E].
    Returns int32 [T, K] in selection order. Uses a full lexicographic sort,
    which is independent of any partial-selection scheme.
    """
    s = selection_scores(z32, bias)
    T, E = s.shape
    assert 1 <= k <= E
    index_key = np.broadcast_to(np.arange(E), (T, E))
    # np.lexsort: the last key is primary.  Primary: -s ascending (s desc);
    # secondary: expert index ascending.
    order = np.lexsort((index_key, -s.astype(np.float64)), axis=-1)
    return order[:, :k].astype(np.int32)


def softmax_gates(z, idx):
    """Gates g[t, k] = softmax(z[t, :])[idx[t, k]] over all E experts (R-gate).

    "LongCat-Flash" section 2.3.2 names softmax gating spread over the experts;
    section 2.1's sum runs over all N+Z experts with weights g_i. Computed in
    fp64 with the usual max subtraction; not renormalised over the K chosen.
    Returns (g [T, K] fp64, p [T, E] fp64).
    """
    z = np.asarray(z, dtype=np.float64)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    p = e / e.sum(axis=1, keepdims=True)
    g = np.take_along_axis(p, np.asarray(idx, dtype=np.int64), axis=1)
    return g, p


def expert_counts(idx, n_experts):
    """T_i = number of (token, slot) pairs routed to expert i, for all E experts.

    "LongCat-Flash" section 2.1 defines T_i as the tokens routed to expert i;
    a token picks an expert at most once, so tokens and slots coincide.
    """
    return np.bincount(np.asarray(idx).ravel(), minlength=n_experts).astype(np.int64)


def permutation(idx, n_ffn):
    """Counting-sort permutation of the FFN slots.

    Slots are the flat positions j = t*K + k of idx. Returns
      offsets     int64 [N+1]  exclusive prefix sum of the FFN expert counts,
      perm        int64 [S]    FFN slot ids grouped by expert (expert ascending),
                               slot id ascending inside a group,
      row_of_slot int64 [T*K]  position of each slot in perm, -1 for slots that
                               went to a zero-computation expert.
    """
    flat = np.asarray(idx, dtype=np.int64).ravel()
    counts = np.array([np.count_nonzero(flat == e) for e in range(n_ffn)], dtype=np.int64)
    offsets = np.zeros(n_ffn + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    groups = [np.nonzero(flat == e)[0] for e in range(n_ffn)]
    perm = np.concatenate(groups) if groups else np.zeros(0, dtype=np.int64)
    row_of_slot = np.full(flat.shape[0], -1, dtype=np.int64)
    row_of_slot[perm] = np.arange(perm.shape[0])
    return offsets, perm.astype(np.int64), row_of_slot


# ----------------------------------------------------------------------------
# Experts and the layer  ("LongCat-Flash" section 2.1: MoE(x_t) = sum over the
#  N+Z experts of g_i E_i(x_t); a zero-computation expert returns x_t)
# ----------------------------------------------------------------------------


def silu(u):
    """silu(u) = u / (1 + exp(-u))."""
    with np.errstate(over="ignore"):
        return u / (1.0 + np.exp(-u))


def expert_gate_up(x_rows, w13):
    """First half of the SiLU-gated FFN expert (reading R-ffn): the
    intermediate h = silu(x W1^T) * (x W3^T), fp64, not rounded.

    x_rows: [m, d]; w13: [2I, d] with gate rows [0, I) and up rows [I, 2I).
    Returns [m, I].
    """
    x_rows = np.asarray(x_rows, dtype=np.float64)
    w13 = np.asarray(w13, dtype=np.float64)
    inter = w13.shape[0] // 2
    u = x_rows @ w13.T
    return silu(u[:, :inter]) * u[:, inter:]


def expert_ffn(x_rows, w13, w2):
    """SiLU-gated FFN expert (reading R-ffn).

    x_rows: [m, d]; w13: [2I, d] with gate rows [0, I) and up rows [I, 2I);
    w2: [d, I]. Returns [m, d] = (silu(x W1^T) * (x W3^T)) W2^T in fp64.
    """
    w2 = np.asarray(w2, dtype=np.float64)
    return expert_gate_up(x_rows, w13) @ w2.T


def expert_down_fp8_rows(h_codes, h_scales, w2):
    """Second half of the expert with fp8 activations (reading R-a8): the
    intermediate given as per-row E4M3FN codes and fp32 row scales, its value
    q * s (exact in fp64) times W2^T. h_codes: uint8 [m, I]; h_scales: [m];
    w2: [d, I]. Returns [m, d], fp64."""
    w2 = np.asarray(w2, dtype=np.float64)
    return dequant_rows_fp8(h_codes, h_scales) @ w2.T


def expert_ffn_a8(x_hat_rows, w13, w2):
    """SiLU-gated FFN expert with fp8 activations (readings R-ffn, R-a8):
    x_hat_rows are already quantized-dequantized; the intermediate
    h = silu(x W1^T) * (x W3^T) is rounded to bf16, quantized per row, and
    its dequantized value multiplies W2^T. fp64 otherwise."""
    h = round_to_bf16(expert_gate_up(x_hat_rows, w13))
    hq, hs = quantize_rows_fp8(h.astype(np.float32))
    return expert_down_fp8_rows(hq, hs, w2)


def combine_given_routing(x, idx, g, n_ffn, get_expert, tokens=None, a8=False):
    """y_t = sum_k g[t,k] * (E_{idx[t,k]}(x_t) if idx[t,k] < N else x_t).

    x: [T, d] fp64 values; idx/g: [T, K]; get_expert(e) -> (w13_e, w2_e).
    tokens: optional subset of token indices to evaluate (others not computed);
    returns y rows for `tokens` (all tokens when None), fp64.
    a8: FFN experts see each token row quantized per row to fp8 and quantize
    their intermediate likewise (reading R-a8); zero experts see exact x.
    """
    x = np.asarray(x, dtype=np.float64)
    idx = np.asarray(idx)
    g = np.asarray(g, dtype=np.float64)
    if tokens is None:
        tokens = np.arange(x.shape[0])
    tokens = np.asarray(tokens)
    y = np.zeros((tokens.shape[0], x.shape[1]), dtype=np.float64)
    sub_idx = idx[tokens]
    sub_g = g[tokens]
    # Zero-computation experts: identity, no FLOPs beyond the gate scaling.
    zero_mask = sub_idx >= n_ffn
    y += (sub_g * zero_mask).sum(axis=1)[:, None] * x[tokens]
    # FFN experts: evaluate each touched expert once on the tokens that chose it.
    x_ffn = x[tokens]
    if a8:
        xq, xs = quantize_rows_fp8(x_ffn.astype(np.float32))
        x_ffn = dequant_rows_fp8(xq, xs)
    for e in np.unique(sub_idx[~zero_mask]):
        rows, ks = np.nonzero(sub_idx == e)
        w13_e, w2_e = get_expert(int(e))
        if a8:
            out = expert_ffn_a8(x_ffn[rows], w13_e, w2_e)
        else:
            out = expert_ffn(x_ffn[rows], w13_e, w2_e)
        y[rows] += sub_g[rows, ks][:, None] * out
    return y


def combine_given_expert_outputs(x, idx, g, n_ffn, ffn_out):
    """The MoE sum of section 2.1 with each FFN slot's expert output given:
    y_t = sum_k g[t,k] * (ffn_out[t,k] if idx[t,k] < N else x_t), fp64.

    x: [T, d]; idx, g: [T, K]; ffn_out: [T, K, d] (rows of zero-expert slots
    are not read). Used where the expert outputs come from given
    intermediates (the fp8-activation expert's down half on given codes).
    """
    x = np.asarray(x, dtype=np.float64)
    idx = np.asarray(idx)
    g = np.asarray(g, dtype=np.float64)
    ffn_out = np.asarray(ffn_out, dtype=np.float64)
    ffn = idx < n_ffn
    v = np.where(ffn[:, :, None], ffn_out, x[:, None, :])
    return (g[:, :, None] * v).sum(axis=1)


def route(x, w_router, bias, k):
    """Routing half of the layer: logits, selection, gates, counts.

    Returns dict(z=fp64 [T,E], z32=fp32 [T,E], idx=int32 [T,K], g=fp64 [T,K],
    p=fp64 [T,E], counts=int64 [E]).
    """
    z = router_logits(x, w_router)
    z32 = z.astype(np.float32)
    idx = select_topk(z32, bias, k)
    g, p = softmax_gates(z, idx)
    counts = expert_counts(idx, z.shape[1])
    return dict(z=z, z32=z32, idx=idx, g=g, p=p, counts=counts)


def forward(x, w_router, bias, k, n_ffn, get_expert):
    """The whole layer: route, then combine over FFN and zero-computation experts.

    Returns (y fp64 [T, d], routing dict from `route`).
    """
    r = route(x, w_router, bias, k)
    y = combine_given_routing(x, r["idx"], r["g"], n_ffn, get_expert)
    return y, r


def dense_masked_forward(x, p_masked, n_ffn, get_expert):
    """The same sum evaluated densely: every FFN expert on every token.

    p_masked: [T, E] gate matrix, zero outside each token's selected experts.
    y = sum_{i<N} p[:, i] * E_i(x) + (sum_{i>=N} p[:, i]) * x.
    No permutation or gather: an independent evaluation of the MoE sum.
    """
    x = np.asarray(x, dtype=np.float64)
    p_masked = np.asarray(p_masked, dtype=np.float64)
    y = p_masked[:, n_ffn:].sum(axis=1)[:, None] * x
    for e in range(n_ffn):
        w13_e, w2_e = get_expert(e)
        y = y + p_masked[:, e][:, None] * expert_ffn(x, w13_e, w2_e)
    return y


# ----------------------------------------------------------------------------
# Expert-bias update  ("LongCat-Flash" section 2.1, the bias-adaptation law and
#  its symbols: mu adaptation rate, K_e target FFN count, T_i tokens routed to
#  expert i, T_all tokens in the global batch)
# ----------------------------------------------------------------------------


def bias_update(bias, counts, n_ffn, k, mu, k_e, t_all):
    """One step of the bias law, for the N FFN experts only (reading R-upd).

    delta_i = mu * (K_e/K * 1/N - T_i/(K*T_all)) is evaluated as the single
    fraction mu*(K_e*T_all - N*T_i) / (K*N*T_all) in fp64 (same value over the
    reals; exactly zero at the fixed point T_i = K_e*T_all/N), then
    b_i <- fl32(b_i + delta_i). Zero-computation experts keep their bias.
    Every operation below is one IEEE fp64 operation, in this order.
    """
    b = np.asarray(bias, dtype=np.float32).copy()
    counts = np.asarray(counts)
    den = float(k) * float(n_ffn) * float(t_all)
    for i in range(n_ffn):
        num = float(k_e) * float(t_all) - float(n_ffn) * float(counts[i])
        delta = (float(mu) * num) / den
        b[i] = np.float32(float(b[i]) + delta)
    return b


# ----------------------------------------------------------------------------
# Router-side statistics (forward values of the training-side terms)
# ----------------------------------------------------------------------------


def expert_groups(n_ffn, n_zero, n_groups):
    """Group of every expert (reading R-grp): FFN expert i is in group
    i // (n_ffn / n_groups); every zero-computation expert is in group
    n_groups (the page's group D+1, counted from 0 here)."""
    if n_groups < 1 or n_ffn % n_groups:
        raise ValueError("n_groups must divide n_ffn")
    gs = n_ffn // n_groups
    return np.array([i // gs for i in range(n_ffn)] + [n_groups] * n_zero, dtype=np.int64)


def load_balance_stats(z, counts, n_ffn, n_zero, k, n_groups, k_e, alpha):
    """Device-level load-balance loss with the zero experts as one extra
    group ("LongCat-Flash" section 2.1, load-balance control: L_LB = alpha *
    sum over the D+1 groups of f_j * P_j; the zero group drives the FFN to
    zero ratio toward K_e : (K - K_e)), under readings R-grp and R-lb.

    z: [T, E] router logits (unbiased); counts: [E] tokens per expert.
    Returns (L_LB, f[D+1], P[D+1]); T = 0 gives zeros.
    """
    z = np.asarray(z, dtype=np.float64)
    counts = np.asarray(counts, dtype=np.int64)
    T, E = z.shape
    D = n_groups
    grp = expert_groups(n_ffn, n_zero, D)
    f = np.zeros(D + 1)
    P = np.zeros(D + 1)
    if T == 0:
        return 0.0, f, P
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    p = e / e.sum(axis=1, keepdims=True)          # softmax over all N+Z experts
    target = np.array([k_e / (k * D)] * D + [(k - k_e) / k])
    for j in range(D + 1):
        P[j] = p[:, grp == j].sum(axis=1).mean()
        share = counts[grp == j].sum() / (T * k)  # share of the T*K selected slots
        # K_e = K sets no target for the zero group; its term is then 0.
        f[j] = share / target[j] if target[j] > 0 else 0.0
    return float(alpha * np.sum(f * P)), f, P


def hidden_z_loss(h, lam):
    """Hidden z-loss ("LongCat-Flash" section on training stability,
    activation stability: L_Z = (lambda / T) * sum_t (log sum_i exp|h_t^i|)^2),
    over the layer input hidden states h [T, d] (reading R-zl). The
    log-sum-exp is taken with its maximum factored out. T = 0 gives 0."""
    h = np.abs(np.asarray(h, dtype=np.float64))
    T = h.shape[0]
    if T == 0:
        return 0.0
    mx = h.max(axis=1)
    lse = mx + np.log(np.exp(h - mx[:, None]).sum(axis=1))
    return float(lam / T * np.sum(lse * lse))


# ----------------------------------------------------------------------------
# Backward of the layer (gradients of a scalar loss through y; the bias is
# used for selection only and has no gradient, selection itself is piecewise
# constant)
# ----------------------------------------------------------------------------


def silu_grad(a):
    """d silu(a) / da = sigma(a) * (1 + a * (1 - sigma(a)))."""
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-a))
    return s * (1.0 + a * (1.0 - s))


def expert_backward(x_rows, g, dy_rows, w13, w2):
    """One FFN expert's part of the backward (see layer_backward): for its
    rows x_rows [m, d] with gates g [m] and upstream gradients dy_rows [m, d],
    returns (dx_rows [m, d], dw13 [2I, d], dw2 [d, I], dg [m]), fp64."""
    x_rows = np.asarray(x_rows, dtype=np.float64)
    dy_rows = np.asarray(dy_rows, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    w13 = np.asarray(w13, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    inter = w2.shape[1]
    u = x_rows @ w13.T
    a, c = u[:, :inter], u[:, inter:]
    h = silu(a) * c
    v = h @ w2.T
    dg = np.sum(dy_rows * v, axis=1)
    dv = g[:, None] * dy_rows
    dh = dv @ w2
    du = np.concatenate([dh * c * silu_grad(a), dh * silu(a)], axis=1)
    return du @ w13, du.T @ x_rows, dv.T @ h, dg


def layer_backward(x, w_router, bias, k, n_ffn, get_expert, dy, idx=None):
    """Gradients of <dy, y> for y = MoE(x) ("LongCat-Flash" section 2.1: the
    sum over the K selected of N+Z experts, gates from one softmax over all
    experts, zero experts the identity), chain rule written out, fp64:

      g_tk = p_t[idx_tk], p_t = softmax(z_t), z_t = W_r x_t
      FFN slot (e = idx_tk < N):  u = W13_e x_t, a = u[:I], c = u[I:],
        h = silu(a) * c, v = W2_e h
      zero slot: v = x_t;   y_t = sum_k g_tk v_tk

      dg_tk = <dy_t, v_tk>;  dv = g_tk dy_t
      FFN: dh = W2_e^T dv;  dW2_e += dv h^T;  da = dh * c * silu'(a);
           dc = dh * silu(a);  du = [da; dc];  dW13_e += du x_t^T;
           dx_t += W13_e^T du
      zero: dx_t += dv
      router: dp_t[i] = sum_k dg_tk [i = idx_tk];  dz_t = p_t * (dp_t - <dp_t, p_t>);
              dW_r += dz_t x_t^T;  dx_t += W_r^T dz_t

    Returns dict(dx [T,d], dw_router [E,d], dw13 {e: [2I,d]}, dw2 {e: [d,I]},
    routing) with weight gradients for the touched FFN experts only.
    idx: optional [T, K] selection to use instead of the oracle's own (the
    gates are still the oracle's fp64 softmax at those experts).
    """
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    w_router = np.asarray(w_router, dtype=np.float64)
    r = route(x, w_router, bias, k)
    if idx is not None:
        idx = np.asarray(idx)
        g, p = softmax_gates(r["z"], idx)
        r = dict(r, idx=idx, g=g, p=p)
    idx, g, p = r["idx"], r["g"], r["p"]
    T, d = x.shape
    dx = np.zeros_like(x)
    dg = np.zeros(idx.shape)
    dw13, dw2 = {}, {}
    for e in np.unique(idx[idx < n_ffn]):
        rows, ks = np.nonzero(idx == e)
        w13_e, w2_e = get_expert(int(e))
        dxe, dw13[int(e)], dw2[int(e)], dg[rows, ks] = expert_backward(
            x[rows], g[rows, ks], dy[rows], w13_e, w2_e)
        np.add.at(dx, rows, dxe)
    zr, zk = np.nonzero(idx >= n_ffn)
    dg[zr, zk] = np.sum(dy[zr] * x[zr], axis=1)
    np.add.at(dx, zr, g[zr, zk][:, None] * dy[zr])
    dp = np.zeros_like(p)
    np.add.at(dp, (np.repeat(np.arange(T), idx.shape[1]), idx.ravel()), dg.ravel())
    dz = p * (dp - np.sum(dp * p, axis=1, keepdims=True))
    dx += dz @ w_router
    return dict(dx=dx, dw_router=dz.T @ x, dw13=dw13, dw2=dw2, dg=dg, dz=dz, routing=r)
