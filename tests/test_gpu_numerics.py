"""Numerical range and edge cases of every stage-1 kernel and the merge,
element by element against the fp64 oracle (gates in tests/_gpu_util.py,
widened below only by terms derived from the inputs' magnitudes).

* Peaked softmax: Q scaled x30, or the softmax scale x16, so that within a
  split scores jump far above the running reference, the lazy rescale of
  (l, acc) runs mid-split and, in the quantised kernels, fp16(p * 2^7)
  underflows for most tokens.
* Planted ramps: a few K rows late in every split whose scores each exceed
  all earlier ones by 6 nats (more than the 8 log2-unit slack), so every one
  of them forces a rescale over already accumulated state.
* Q = 0 (all scores equal): the output is mean(V) over the visible tokens and
  lse = ln L, checked against that closed form as well as the oracle.
* L = 1: the output is V_0 and lse the single score.
* Large magnitudes: dense bf16 / fp32 K, V of standard deviation 1e3 / 1e4;
  INT8 encoded from N(0,1) * 1e5 (scales near 2e3); INT4 encoded from
  N(0,1) * 1e5 (scales near 3e4, so n*s passes fp16's range and the kernel's
  rescaled pass runs); INT4 zero points shifted by fractions up to +-1e3, with
  and without scales that make z*s pass 65504.
* Tiny magnitudes: INT8 and INT4 caches encoded from N(0,1) * 1e-4 (every V
  scale an fp16 subnormal), held to the kernels' relative bound with no
  absolute allowance.

Gates beyond unit scale.  The standard gates assume unit-scale inputs.  A
kernel forms each score from fp32 terms whose magnitudes add up to
M = scale * sum_d |q_d| u_d, u_d being what the score's products carry
before they cancel: |k_d| for a dense cache, |s| (|b| + 128) for INT8 (its
codes enter offset by 128), |s| (n_d + |z|) for INT4 (codes and zero point
enter separately).  Its rounding error is a few units of 2^-24 M; the gate
allows E = 2^-20 M (16 units) per score, the largest M over the (request,
kv-head)'s query rows and tokens.  A score error E changes each softmax
weight by a factor within e^(+-E), so the LSE moves by at most E and a
normalised output by at most 2 E max|v|: the LSE gate adds E and the output
gates add 2 E max|v|.  With |V| far above 1, fp32 accumulation of p v over a
split adds its own rounding, allowed as 2^-16 max|v| (256 units of max|v|).
"""
import math

import numpy as np
import pytest
import torch

from decode_attention_paged_gqa_amd import workloads as W
from oracle import attention as OA
from oracle import quant as OQ
from tests import _gpu_util as U

pytestmark = pytest.mark.gpu
log = U.log

# one small workload per stage-1 kernel (and row-tile count), NHD or HND
FAMILIES = {
    "bf16_vec_g5": W.RAGGED_B64.scaled(name="num_bf16_vec_g5", batch=4, lengths="list",
                                       length_list=(1, 300, 1500, 65), pin_max=False),
    "bf16_vec_d64_g4": W.RAGGED_B64.scaled(name="num_bf16_vec_d64", batch=3, num_q_heads=16,
                                           head_dim=64, page_size=16, kv_layout="NHD",
                                           lengths="list", length_list=(40, 900, 17),
                                           pin_max=False),
    "bf16_mfma_r16": W.BF16_B16.scaled(name="num_bf16_mfma_r16", batch=3, q_per_req=4,
                                       causal=True, lengths="list", length_list=(7, 700, 1300)),
    "bf16_mfma_r20": W.BF16_B16.scaled(name="num_bf16_mfma_r20", batch=3, num_q_heads=40,
                                       q_per_req=4, causal=True, kv_layout="NHD",
                                       lengths="list", length_list=(90, 5, 1100)),
    "bf16_mfma_d64_g8": W.BF16_B16.scaled(name="num_bf16_mfma_d64", batch=3, num_q_heads=64,
                                          head_dim=64, lengths="list",
                                          length_list=(33, 1000, 260)),
    "fp32_vec_g2": W.TINY_FP32.scaled(name="num_fp32_vec_g2", batch=3, num_q_heads=4,
                                      num_kv_heads=2, lengths="list",
                                      length_list=(15, 700, 66), pool_pages=0),
    "fp32_mfma_g8": W.TINY_FP32.scaled(name="num_fp32_mfma_g8", batch=3, num_q_heads=16,
                                       num_kv_heads=2, head_dim=128, page_size=64,
                                       kv_layout="HND", lengths="list",
                                       length_list=(100, 1200, 3), pool_pages=0),
    "int8_g4": W.INT8_B32.scaled(name="num_int8_g4", batch=3, lengths="list",
                                 length_list=(64, 1500, 9)),
    "int8_fp32q_d64": W.INT8_B32.scaled(name="num_int8_fp32q_d64", batch=3, dtype="fp32",
                                        head_dim=64, kv_layout="NHD", lengths="list",
                                        length_list=(300, 1000, 2)),
    "int8_r20": W.INT8_B32.scaled(name="num_int8_r20", batch=3, num_q_heads=40, q_per_req=4,
                                  causal=True, lengths="list", length_list=(5, 129, 1400)),
    "int4_mtp_r16": W.INT4_MTP_B64.scaled(name="num_int4_r16", batch=3, lengths="list",
                                          length_list=(65, 1400, 6)),
    "int4_d64_q1": W.INT4_MTP_B64.scaled(name="num_int4_d64_q1", batch=3, head_dim=64,
                                         q_per_req=1, causal=False, kv_layout="NHD",
                                         lengths="list", length_list=(1000, 17, 300)),
    "int4_fp32q": W.INT4_MTP_B64.scaled(name="num_int4_fp32q", batch=3, dtype="fp32",
                                        lengths="list", length_list=(129, 800, 4)),
    "int4_r20": W.INT4_MTP_B64.scaled(name="num_int4_r20", batch=3, num_q_heads=40,
                                      kv_layout="NHD", lengths="list",
                                      length_list=(70, 1300, 10)),
}
FAM = list(FAMILIES)


def _out_dtype(w):
    return torch.float32 if (w.kv == W.KV_DENSE and w.dtype == "fp32") else torch.bfloat16


def _check_out(w, out, ref, label):
    if w.kv != W.KV_DENSE:
        U.check_quant(out, ref, label)
    elif w.dtype == "fp32":
        U.check_fp32(out, ref, label)
    else:
        U.check_bf16(out, ref, label)


def _score_terms(batch, scale):
    """Per (request, query head) [B, Hq]: the score magnitude M (see the module
    notes) maximised over the query's rows and the request's tokens, and
    max|v| over the request's tokens of the head's kv-head."""
    w = batch.w
    h = U.host_inputs(batch)
    nhd = batch.nhd
    if w.kv == W.KV_DENSE:
        u = np.abs(h["k"])
    elif w.kv == W.KV_INT8:
        codes = W.host_int(nhd(batch.k_pool)).astype(np.float64)
        s = np.abs(OQ.fp16_bits_to_f64(W.host_u16(nhd(batch.k_scale))))
        u = s[..., None] * (np.abs(codes) + 128.0)
    else:
        packed = W.host_int(nhd(batch.k_pool)).astype(np.int64)
        n = np.stack([packed & 15, packed >> 4], axis=-1).reshape(packed.shape[:-1] + (-1,))
        sz = OQ.fp16_bits_to_f64(W.host_u16(nhd(batch.k_scale)))
        s = np.repeat(np.abs(sz[..., 0]), 32, axis=-1)
        z = np.repeat(np.abs(sz[..., 1]), 32, axis=-1)
        u = s * (n + z)
    q = np.abs(h["q"])
    G = w.group
    M = np.zeros((w.batch, w.num_q_heads))
    vmax = np.zeros((w.batch, w.num_q_heads))
    for b, L in enumerate(batch.lengths):
        L = int(L)
        if L == 0:
            continue
        U_b = OA.gather_tokens(u, h["page_table"][b], L, w.page_size)      # [L, Hkv, D]
        V_b = OA.gather_tokens(h["v"], h["page_table"][b], L, w.page_size)
        for hh in range(w.num_q_heads):
            g = hh // G
            M[b, hh] = scale * float((q[b, :, hh] @ U_b[:, g].T).max())
            vmax[b, hh] = float(np.abs(V_b[:, g]).max())
    return M, vmax


def _compare(gpu, batch, S, label, scale=None, magnitudes=False, accumulate=False):
    """Partials, output and LSE against the oracle: the standard gates, plus,
    with ``magnitudes``, the score-rounding terms and, with ``accumulate``,
    the accumulation term of the module notes."""
    w = batch.w
    scale = w.softmax_scale if scale is None else scale
    o_ref, l_ref = U.oracle_partials(batch, S, scale=scale)
    out_ref, lse_ref = U.oracle_full(batch, scale=scale)
    out, lse, o, l = U.run_decode(gpu, batch, S, out_dtype=_out_dtype(w), scale=scale)
    o_extra = U.matrix_path_o_bound(batch)
    lse_tol = 1e-4
    if magnitudes or accumulate:
        M, vmax = _score_terms(batch, scale)
        E = 2.0 ** -20 * M if magnitudes else np.zeros_like(M)
        extra = 2 * E * vmax + (2.0 ** -16 * vmax if accumulate else 0.0)
        extra = extra[:, None, :, None, None]
        o_extra = extra if o_extra is None else o_extra + extra
        lse_tol = 1e-4 + E[:, None, :]
        log(f"  {label}: score magnitude M up to {M.max():.3e}, max|v| {vmax.max():.3e}")
    U.check_partials(U.to_np(o), U.to_np(l), o_ref, l_ref, label, o_extra=o_extra,
                     lse_tol=lse_tol if np.isscalar(lse_tol) else lse_tol[..., None])
    if magnitudes or accumulate:
        _bounded(w, U.to_np(out), out_ref, o_extra[..., 0], label + " out")
        U.check_lse(U.to_np(lse), lse_ref, label + " lse",
                    tol=np.broadcast_to(lse_tol, lse_ref.shape))
    else:
        _check_out(w, U.to_np(out), out_ref, label + " out")
        U.check_lse(U.to_np(lse), lse_ref, label + " lse")
    return U.to_np(out), U.to_np(lse)


# ---------------------------------------------------------------- peaked softmax
@pytest.mark.parametrize("fam", FAM)
def test_peaked_query(gpu, fam):
    w = FAMILIES[fam].scaled(amp=(30.0, 1.0, 1.0))
    log(f"peaked Q x30 {fam}")
    _compare(gpu, W.make_batch(w, device="cuda"), 3, f"{fam} Qx30", magnitudes=True)


@pytest.mark.parametrize("fam", FAM)
def test_scale_times_16(gpu, fam):
    w = FAMILIES[fam]
    log(f"softmax scale x16 {fam}")
    _compare(gpu, W.make_batch(w, device="cuda"), 2, f"{fam} scale x16",
             scale=16.0 * w.softmax_scale, magnitudes=True)


def _plant_ramp(batch, n_plant=6, step=6.0, c=4.0, seed=21):
    """Query rows of kv-head g set to c * u_g (plus a little noise) and, in every
    request, n_plant K rows at evenly spread positions written so that their
    scores are step, 2 step, ... (nats): each one above every earlier score by
    more than the kernels' rescale slack."""
    w = batch.w
    rng = np.random.default_rng(seed)
    D, G, Hkv = w.head_dim, w.group, w.num_kv_heads
    u = rng.standard_normal((Hkv, D))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    q = c * np.repeat(u, G, axis=0)[None, None] + 0.02 * rng.standard_normal(batch.q.shape)
    batch.q.copy_(torch.from_numpy(q).to(batch.q.dtype))
    pt = W.host_int(batch.page_table)
    kp = batch.nhd(batch.k_pool)
    ks = batch.nhd(batch.k_scale) if batch.k_scale is not None else None
    for b, L in enumerate(batch.lengths):
        L = int(L)
        if L < 2 * n_plant:
            continue
        for k in range(n_plant):
            t = int((k + 0.5) * L / n_plant)
            page, slot = int(pt[b, t // w.page_size]), t % w.page_size
            target = step * (k + 1)
            for g in range(Hkv):
                if w.kv == W.KV_DENSE:
                    row = target * math.sqrt(D) / c * u[g]
                    kp[page, slot, g] = torch.from_numpy(row).to(kp.dtype)
                elif w.kv == W.KV_INT8:
                    code = np.rint(127 * u[g] / np.abs(u[g]).max())
                    s = target * math.sqrt(D) / (c * float(u[g] @ code))
                    kp[page, slot, g] = torch.from_numpy(code).to(torch.int8)
                    ks[page, slot, g] = s
                else:
                    nib = np.where(u[g] > 0, 15, 0).astype(np.uint8)
                    s = target * math.sqrt(D) / (c * 7.5 * float(np.abs(u[g]).sum()))
                    kp[page, slot, g] = torch.from_numpy(nib[0::2] | (nib[1::2] << 4))
                    ks[page, slot, g, :, 0] = s
                    ks[page, slot, g, :, 1] = 7.5


@pytest.mark.parametrize("fam", FAM)
def test_planted_score_ramp(gpu, fam):
    w = FAMILIES[fam]
    log(f"planted score ramp {fam}")
    batch = W.make_batch(w, device="cuda")
    _plant_ramp(batch)
    torch.cuda.synchronize()
    _compare(gpu, batch, 2, f"{fam} ramp", magnitudes=True)


# ---------------------------------------------------------------- closed forms
def _visible(w, L, i):
    return OA.visible_length(int(L), w.q_per_req, i, w.causal)


@pytest.mark.parametrize("fam", FAM)
def test_zero_query_gives_mean_of_v(gpu, fam):
    w = FAMILIES[fam]
    log(f"Q = 0 {fam}")
    batch = W.make_batch(w, device="cuda")
    batch.q.zero_()
    out, lse = _compare(gpu, batch, 3, f"{fam} Q=0")
    h = U.host_inputs(batch)
    G = w.group
    mean = np.zeros_like(out)
    lnl = np.full(lse.shape, -np.inf)
    for b, L in enumerate(batch.lengths):
        V = OA.gather_tokens(h["v"], h["page_table"][b], int(L), w.page_size)
        for i in range(w.q_per_req):
            n = _visible(w, L, i)
            if n == 0:
                continue
            for hh in range(w.num_q_heads):
                mean[b, i, hh] = V[:n, hh // G].mean(axis=0)
            lnl[b, i] = math.log(n)
    _check_out(w, out, mean, f"{fam} Q=0 vs mean(V)")
    U.check_lse(lse, lnl, f"{fam} Q=0 lse vs ln L")


@pytest.mark.parametrize("fam", FAM)
def test_single_token_gives_v0(gpu, fam):
    base = FAMILIES[fam]
    # every MTP row sees the one token (not causal), so the kernel keeps its row count
    w = base.scaled(name=base.name + "_L1", lengths="list", length_list=(1,) * base.batch,
                    causal=False)
    log(f"L = 1 {fam}")
    batch = W.make_batch(w, device="cuda")
    out, lse = _compare(gpu, batch, 2, f"{fam} L=1")
    h = U.host_inputs(batch)
    G = w.group
    v0 = np.zeros_like(out)
    s0 = np.zeros(lse.shape)
    for b in range(w.batch):
        K = OA.gather_tokens(h["k"], h["page_table"][b], 1, w.page_size)
        V = OA.gather_tokens(h["v"], h["page_table"][b], 1, w.page_size)
        for i in range(w.q_per_req):
            for hh in range(w.num_q_heads):
                v0[b, i, hh] = V[0, hh // G]
                s0[b, i, hh] = w.softmax_scale * float(h["q"][b, i, hh] @ K[0, hh // G])
    _check_out(w, out, v0, f"{fam} L=1 vs V_0")
    U.check_lse(lse, s0, f"{fam} L=1 lse vs score")


# ---------------------------------------------------------------- large magnitudes
def _bounded(w, out, ref, bound, label):
    """|out - ref| <= bound + the output's own gate, element by element: half a
    bf16 ulp of ref + 1e-2 for a bf16 output, 1e-5 for an fp32 one (bound: the
    stage-1 partials' extra error bound, broadcastable to [B, q, Hq, 1]; the
    merge is a convex combination of partials, so it carries over)."""
    assert np.all(np.isfinite(out)), f"{label}: non-finite output"
    d = np.abs(out - ref)
    own = 1e-5 if _out_dtype(w) == torch.float32 else U.bf16_half_ulp(ref) + 1e-2
    excess = d - own - bound
    scale = float(np.max(np.abs(ref))) or 1.0
    log(f"  {label}: max|d|={float(d.max()):.3e} (max|ref| {scale:.3e}), "
        f"max bound {float(np.max(bound)):.3e}, relL2={U.rel_l2(out, ref):.3e}")
    assert float(excess.max()) <= 0, f"{label}: beyond the bound by {float(excess.max())}"


DENSE = [f for f in FAM if FAMILIES[f].kv == W.KV_DENSE]


@pytest.mark.parametrize("fam", DENSE)
def test_large_dense_values(gpu, fam):
    w = FAMILIES[fam].scaled(amp=(1e-3, 1e3, 1e4))
    log(f"large dense K, V {fam}")
    batch = W.make_batch(w, device="cuda")
    out, _ = _compare(gpu, batch, 3, f"{fam} K*1e3 V*1e4", magnitudes=True, accumulate=True)
    if w.dtype == "bf16":  # the scale-free bf16 gate holds at any magnitude
        assert U.rel_l2(out, U.bf16_rne_from_f64(U.oracle_full(batch)[0])) <= 1e-3


RANGE_CASES = [("int8", d, lay, qd) for d in (128, 64) for lay in ("NHD", "HND")
               for qd in ("bf16", "fp32")] + \
              [("int4", d, lay, qd) for d in (128, 64) for lay in ("NHD", "HND")
               for qd in ("bf16", "fp32")]


def _range_workload(kv, D, lay, qd, **kw):
    base = FAMILIES["int8_g4"] if kv == "int8" else FAMILIES["int4_mtp_r16"]
    return base.scaled(name=f"range_{kv}_d{D}_{lay.lower()}_{qd}", head_dim=D, kv_layout=lay,
                       dtype=qd, **kw)


@pytest.mark.parametrize("kv,D,lay,qd", RANGE_CASES,
                         ids=[f"{a}-d{b}-{c}-{d}" for a, b, c, d in RANGE_CASES])
def test_encoded_from_huge_values(gpu, kv, D, lay, qd):
    """K, V encoded from N(0,1) * 1e5 (Q * 1e-5 keeps the scores moderate):
    INT8 scales near 2e3 (b * s up to 4e5), INT4 scales near 3e4 (n * s up to
    5e5), both far past fp16's 65504."""
    w = _range_workload(kv, D, lay, qd, amp=(1e-5, 1e5, 1e5))
    log(f"encoded from N(0,1)*1e5: {w.name}")
    batch = W.make_batch(w, device="cuda")
    vs = U.host_inputs(batch)["v"]
    assert np.abs(vs).max() > 65504
    _compare(gpu, batch, 3, w.name, magnitudes=True, accumulate=True)


@pytest.mark.parametrize("overflow", [False, True], ids=["z_up_to_1e3", "z_and_s_past_fp16"])
@pytest.mark.parametrize("D,lay", [(128, "NHD"), (128, "HND"), (64, "NHD"), (64, "HND")])
def test_int4_large_zero_points(gpu, D, lay, overflow):
    """Every zero point shifted by a fraction in [-1000, 1000]; with ``overflow``
    the scales are also multiplied by 1000, so z*s (and v) pass 65504."""
    w = _range_workload("int4", D, lay, "bf16")
    log(f"int4 zero points up to 1e3 {w.name} overflow={overflow}")
    batch = W.make_batch(w, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(17)
    for sc in (batch.k_scale, batch.v_scale):
        shift = torch.rand(sc[..., 1].shape, generator=gen, device="cuda") * 2000.0 - 1000.0
        sc[..., 1] = (sc[..., 1].float() + shift).to(torch.float16)
        if overflow:
            sc[..., 0] = (sc[..., 0].float() * 1000.0).to(torch.float16)
    if overflow:  # keep the scores moderate: K grew with the scales
        batch.q.mul_(1e-5)
    torch.cuda.synchronize()
    v = U.host_inputs(batch)["v"]
    assert (np.abs(v).max() > 65504) == overflow
    _compare(gpu, batch, 3, w.name + (" s*1000" if overflow else ""), magnitudes=True,
             accumulate=True)


TINY_CASES = [(kv, d, lay) for kv in ("int8", "int4") for d in (128, 64) for lay in ("NHD", "HND")]


@pytest.mark.parametrize("kv,D,lay", TINY_CASES, ids=[f"{a}-d{b}-{c}" for a, b, c in TINY_CASES])
def test_tiny_scales(gpu, kv, D, lay):
    """K, V encoded from N(0,1) * 1e-4 (Q * 1e4 keeps the scores moderate):
    INT8 scales near 3e-6 and INT4 scales near 3e-5, fp16 subnormals.  The
    partials must hold the kernel's relative bound alone -- u (max|v| +
    max|n s| + max|z s|), the subnormal floor, and the score and accumulation
    terms of the module notes -- with no absolute allowance: at this scale an
    INT4 operand formed from a rounded s / 16, or an INT8 V' formed as
    fp16(b s / 2^7), would miss it by one to two orders of magnitude."""
    w = _range_workload(kv, D, lay, "bf16", amp=(1e4, 1e-4, 1e-4))
    log(f"tiny scales {w.name}")
    batch = W.make_batch(w, device="cuda")
    sc = OQ.fp16_bits_to_f64(W.host_u16(batch.nhd(batch.v_scale)))
    scales = sc[..., 0] if kv == "int4" else sc
    assert np.abs(scales).max() < 2.0 ** -14  # every V scale an fp16 subnormal
    S = 3
    o_ref, l_ref = U.oracle_partials(batch, S)
    _, _, o, _ = U.run_decode(gpu, batch, S)
    M, vmax = _score_terms(batch, w.softmax_scale)
    E = 2.0 ** -20 * M
    bound = U.fp16_pv_o_bound(batch) + (2 * E * vmax + 2.0 ** -16 * vmax)[:, None, :, None, None]
    d = np.abs(U.to_np(o) - o_ref)
    log(f"  max|dO| {float(d.max()):.3e}, max|O| {float(np.abs(o_ref).max()):.3e}, "
        f"bound up to {float(bound.max()):.3e}")
    excess = d - bound
    assert float(excess.max()) <= 0, f"beyond the relative bound by {float(excess.max()):.3e}"
