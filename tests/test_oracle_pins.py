"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle function to a library routine, a closed form, an
invariant the method guarantees, or brute force on tiny inputs, so that a
dropped term, a sign, an index or a transposed operand in the oracle fails
at least one of them.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import opt_he as O

TINY = synth.WORKLOADS["tiny"]


def rng(seed=0):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------
# bf16 rounding: bitwise against torch's float32 -> bfloat16 conversion
# ----------------------------------------------------------------------------

def _torch_bf16(x64):
    return torch.from_numpy(np.asarray(x64, np.float32)).to(torch.bfloat16).double().numpy()


def test_round_bf16_matches_torch_random():
    r = rng(1)
    x = (r.standard_normal(200000) * np.exp2(r.integers(-140, 120, 200000))).astype(np.float32)
    np.testing.assert_array_equal(O.round_bf16(x.astype(np.float64)), _torch_bf16(x))


def test_round_bf16_matches_torch_ties_and_edges():
    r = rng(2)
    hi = r.integers(0, 1 << 15, 5000, dtype=np.uint32) << 16
    hi |= r.integers(0, 2, 5000, dtype=np.uint32) << 31
    ties = (hi | np.uint32(0x8000)).view(np.float32)            # exactly halfway
    near = (hi | r.integers(0x7ff0, 0x8010, 5000, dtype=np.uint32)).view(np.float32)
    sub = (r.integers(1, 1 << 23, 5000, dtype=np.uint32)).view(np.float32)   # subnormals
    for x in (ties, near, sub):
        x = x[np.isfinite(x)]
        np.testing.assert_array_equal(O.round_bf16(x.astype(np.float64)), _torch_bf16(x))


def test_round_bf16_closed_forms():
    assert O.round_bf16(1.0 + 2.0 ** -8) == 1.0                  # tie -> even
    assert O.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6   # tie -> even (up)
    assert O.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -20) == 1.0 + 2.0 ** -7
    assert O.ulp_bf16(1.0) == 2.0 ** -7
    assert O.ulp_bf16(3.0) == 2.0 ** -6
    assert O.round_bf16(0.0) == 0.0


# ----------------------------------------------------------------------------
# LayerNorm
# ----------------------------------------------------------------------------

def test_layer_norm_matches_torch():
    r = rng(3)
    x = r.standard_normal((7, 96)) * 3 + 1.5
    g = r.standard_normal(96)
    b = r.standard_normal(96)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (96,), torch.from_numpy(g),
                                         torch.from_numpy(b), eps=1e-5).numpy()
    np.testing.assert_allclose(O.layer_norm(x, g, b), ref, rtol=1e-12, atol=1e-12)


def test_layer_norm_closed_forms():
    b = np.arange(8.0)
    np.testing.assert_array_equal(O.layer_norm(np.full((2, 8), 3.25), np.ones(8), b), np.tile(b, (2, 1)))
    x = np.array([[1.0, -1.0, 1.0, -1.0]])           # mean 0, variance 1
    np.testing.assert_allclose(O.layer_norm(x, np.ones(4), np.zeros(4), eps=0.0), x, rtol=0, atol=0)


# ----------------------------------------------------------------------------
# causal attention
# ----------------------------------------------------------------------------

def _brute_attention(q, k, v, q_pos0):
    H, Tq, D = q.shape
    out = np.zeros_like(q)
    for h in range(H):
        for i in range(Tq):
            last = q_pos0 + i
            s = [sum(q[h, i, c] * k[h, j, c] for c in range(D)) for j in range(last + 1)]
            m = max(s)
            e = [np.exp(x - m) for x in s]
            z = sum(e)
            for j in range(last + 1):
                out[h, i] += e[j] / z * v[h, j]
    return out


def test_attention_brute_force():
    r = rng(4)
    q, k, v = (r.standard_normal((2, 5, 3)) for _ in range(3))
    o, _ = O.causal_attention(q, k, v, 0)
    np.testing.assert_allclose(o, _brute_attention(q, k, v, 0), rtol=1e-12, atol=1e-12)
    # a query block that starts later (the cached-decode shape)
    k2, v2 = r.standard_normal((2, 9, 3)), r.standard_normal((2, 9, 3))
    q2 = r.standard_normal((2, 2, 3))
    o2, _ = O.causal_attention(q2, k2, v2, 7)
    np.testing.assert_allclose(o2, _brute_attention(q2, k2, v2, 7), rtol=1e-12, atol=1e-12)


def test_attention_matches_torch_sdpa():
    r = rng(5)
    q, k, v = (r.standard_normal((4, 33, 16)) for _ in range(3))
    o, _ = O.causal_attention(q, k, v, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True, scale=1.0).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_softmax_rows_and_mask():
    r = rng(6)
    q, k, v = (r.standard_normal((3, 12, 8)) * 4 for _ in range(3))
    _, p = O.causal_attention(q, k, v, 0)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert (p >= 0).all()
    assert (p[:, np.triu_indices(12, 1)[0], np.triu_indices(12, 1)[1]] == 0).all()


def test_attention_closed_forms():
    r = rng(7)
    q = r.standard_normal((2, 6, 4))
    v = r.standard_normal((2, 6, 4))
    k = np.zeros((2, 6, 4))                    # constant keys: uniform weights
    o, _ = O.causal_attention(q, k, v, 0)
    running_mean = np.cumsum(v, axis=1) / np.arange(1, 7)[None, :, None]
    np.testing.assert_allclose(o, running_mean, rtol=1e-12, atol=1e-12)
    k = r.standard_normal((2, 6, 4))
    o, _ = O.causal_attention(q, k, v, 0)
    np.testing.assert_allclose(o[:, 0], v[:, 0], rtol=0, atol=1e-15)   # first position sees itself only


def test_argmax_lowest_index_on_ties():
    x = np.array([[0.5, 2.0, 2.0, -1.0], [3.0, 3.0, 3.0, 3.0], [-1.0, -2.0, -1.0, -5.0]])
    np.testing.assert_array_equal(O.argmax_lowest(x), [1, 0, 0])


# ----------------------------------------------------------------------------
# LoRA fold / unfold
# ----------------------------------------------------------------------------

def test_lora_fused_equals_unfused_product():
    r = rng(8)
    W, A, B = r.standard_normal((40, 24)), r.standard_normal((4, 24)), r.standard_normal((40, 4))
    x = r.standard_normal((5, 24))
    s = 2.0
    Wf = O.lora_fuse(W, A, B, s, O.Precision("fp64"))
    unfused = x @ W.T + s * ((x @ A.T) @ B.T)       # W x + s B (A x)
    np.testing.assert_allclose(x @ Wf.T, unfused, rtol=1e-12, atol=1e-12)


def test_lora_delta_is_rank_sum_of_outer_products():
    r = rng(9)
    A, B = r.standard_normal((3, 7)), r.standard_normal((5, 3))
    expect = np.zeros((5, 7))
    for j in range(3):
        expect += np.outer(B[:, j], A[j])
    np.testing.assert_allclose(O.lora_delta(A, B, 1.5), 1.5 * expect, rtol=1e-14, atol=1e-14)


def test_lora_zero_B_is_identity_bitwise():
    W = synth.normal(0, "w", (64, 32))
    A = synth.normal(0, "a", (4, 32))
    B = torch.zeros((64, 4), dtype=torch.bfloat16)
    Wf = O.lora_fuse(W, A, B, 2.0, O.Precision("bf16"))
    np.testing.assert_array_equal(Wf, W.double().numpy())


def test_lora_round_trip_ulp_bound():
    prec = O.Precision("bf16")
    W = synth.normal(0, "rt.w", (256, 512))
    A = synth.normal(0, "rt.a", (16, 512))
    B = synth.normal(0, "rt.b", (256, 16))
    W64 = W.double().numpy()
    Wf = O.lora_fuse(W, A, B, 2.0, prec)
    assert np.array_equal(Wf, O.round_bf16(Wf))                      # stored as bf16
    Wr = O.lora_unfuse(Wf, A, B, 2.0, prec)
    err = np.abs(Wr - W64)
    bound = O.ulp_bf16(np.maximum(np.abs(W64), np.abs(Wf)))
    assert (err <= bound).all()
    assert (err == 0).mean() > 0.8                                    # most elements bit-exact
    # repeating the round trip does not drift further
    Wr2 = O.lora_unfuse(O.lora_fuse(Wr, A, B, 2.0, prec), A, B, 2.0, prec)
    assert (np.abs(Wr2 - W64) <= bound).all()


# ----------------------------------------------------------------------------
# whole decoder against Hugging Face's OPT (float64, CPU)
# ----------------------------------------------------------------------------

def _tiny_params(shape, seed=0):
    return synth.model_params(shape, seed)


def _hf_opt(shape, params, lora=None, scale=1.0, unfused_lora=False):
    from transformers import OPTConfig, OPTForCausalLM, OPTModel
    d = shape.d_model
    cfg = OPTConfig(vocab_size=shape.vocab, hidden_size=d, num_hidden_layers=shape.n_layers,
                    ffn_dim=shape.d_ffn, num_attention_heads=shape.n_heads,
                    max_position_embeddings=shape.max_pos, do_layer_norm_before=shape.norm == "pre",
                    word_embed_proj_dim=shape.embed_dim, activation_function="relu",
                    enable_bias=True, dropout=0.0, attention_dropout=0.0,
                    layerdrop=0.0, pad_token_id=1, tie_word_embeddings=True)
    cfg._attn_implementation = "eager"
    m = (OPTForCausalLM(cfg) if shape.head == "lm" else OPTModel(cfg)).double().eval()
    dec = m.model.decoder if shape.head == "lm" else m.decoder
    P = {k: v.double() for k, v in params.items()}
    with torch.no_grad():
        dec.embed_tokens.weight.copy_(P["E"])
        dec.embed_positions.weight.copy_(P["P"])
        if shape.norm == "pre":
            dec.final_layer_norm.weight.copy_(P["lnf.g"])
            dec.final_layer_norm.bias.copy_(P["lnf.b"])
        if shape.embed_dim != d:
            dec.project_in.weight.copy_(P["proj_in"])
            dec.project_out.weight.copy_(P["proj_out"])
        for i, lay in enumerate(dec.layers):
            W = P[f"L{i}.qkv.w"]
            bq = P[f"L{i}.qkv.b"]
            lin = {"q": (lay.self_attn.q_proj, W[:d], bq[:d]),
                   "k": (lay.self_attn.k_proj, W[d:2 * d], bq[d:2 * d]),
                   "v": (lay.self_attn.v_proj, W[2 * d:], bq[2 * d:]),
                   "out": (lay.self_attn.out_proj, P[f"L{i}.out.w"], P[f"L{i}.out.b"]),
                   "fc1": (lay.fc1, P[f"L{i}.fc1.w"], P[f"L{i}.fc1.b"]),
                   "fc2": (lay.fc2, P[f"L{i}.fc2.w"], P[f"L{i}.fc2.b"])}
            for name, (mod, w, b) in lin.items():
                mod.weight.copy_(w)
                mod.bias.copy_(b)
                if lora is not None:
                    A = lora[f"lora.L{i}.{name}.A"].double()
                    Bm = lora[f"lora.L{i}.{name}.B"].double()
                    if unfused_lora:
                        _attach_unfused(mod, A, Bm, scale)
                    else:
                        mod.weight.add_(scale * (Bm @ A))
            lay.self_attn_layer_norm.weight.copy_(P[f"L{i}.ln1.g"])
            lay.self_attn_layer_norm.bias.copy_(P[f"L{i}.ln1.b"])
            lay.final_layer_norm.weight.copy_(P[f"L{i}.ln2.g"])
            lay.final_layer_norm.bias.copy_(P[f"L{i}.ln2.b"])
        if shape.head == "lm":
            m.lm_head.weight = dec.embed_tokens.weight
    return m


def _attach_unfused(mod, A, Bm, scale):
    """Make a Linear compute W x + b + s B (A x) without folding."""
    base = mod.forward

    def fwd(x, base=base, A=A, Bm=Bm):
        return base(x) + scale * ((x @ A.T) @ Bm.T)
    mod.forward = fwd


@pytest.fixture(autouse=False)
def fp64_softmax(monkeypatch):
    """Hugging Face's eager attention upcasts softmax to float32; keep float64."""
    orig = torch.nn.functional.softmax

    def softmax(x, dim=None, _stacklevel=3, dtype=None):
        if x.dtype == torch.float64:
            dtype = None
        return orig(x, dim=dim, dtype=dtype)
    monkeypatch.setattr(torch.nn.functional, "softmax", softmax)


def test_decoder_matches_hf_opt_no_lora(fp64_softmax):
    shape = TINY.actor
    params = _tiny_params(shape)
    ids = synth.prompts(TINY).numpy()
    om = O.OracleModel(shape, params, O.Precision("fp64"))
    hf = _hf_opt(shape, params)
    with torch.no_grad():
        ref = hf(input_ids=torch.from_numpy(ids).long()).logits.numpy()
    np.testing.assert_allclose(om.forward_full(ids), ref, rtol=1e-10, atol=1e-12)


def test_decoder_lora_fused_matches_unfused_hf(fp64_softmax):
    shape = TINY.actor
    params = _tiny_params(shape)
    lora = synth.lora_params(shape, TINY.lora_rank)
    s = TINY.lora_scale
    ids = synth.prompts(TINY).numpy()
    om = O.OracleModel(shape, params, O.Precision("fp64"), lora=lora, lora_scale=s)
    hf = _hf_opt(shape, params, lora=lora, scale=s, unfused_lora=True)
    with torch.no_grad():
        ref = hf(input_ids=torch.from_numpy(ids).long()).logits.numpy()
    np.testing.assert_allclose(om.forward_full(ids), ref, rtol=1e-10, atol=1e-12)
    # and the adapters really change the output
    base = O.OracleModel(shape, params, O.Precision("fp64")).forward_full(ids)
    assert np.abs(base - ref).max() > 1e-4


def test_reward_model_matches_hf_opt_post_ln(fp64_softmax):
    shape = synth.ModelShape(n_layers=2, d_model=64, n_heads=4, d_ffn=128, vocab=300, max_pos=40,
                             dtype="fp32", norm="post", d_embed=32, head="scalar")
    params = synth.model_params(shape, seed=3)
    ids = synth.tokens(3, "rm.ids", (3, 20), shape.vocab).numpy()
    om = O.OracleModel(shape, params, O.Precision("fp64"))
    hf = _hf_opt(shape, params)
    with torch.no_grad():
        hs = hf(input_ids=torch.from_numpy(ids).long()).last_hidden_state.numpy()
    ref = hs[:, -1] @ params["score"].double().numpy()
    np.testing.assert_allclose(om.score(ids), ref, rtol=1e-10, atol=1e-12)


def test_zero_layer_closed_form():
    shape = synth.ModelShape(n_layers=0, d_model=32, n_heads=2, d_ffn=64, vocab=100, max_pos=20,
                             dtype="fp32")
    params = synth.model_params(shape, seed=4)
    ids = synth.tokens(4, "z.ids", (2, 9), 100).numpy()
    om = O.OracleModel(shape, params, O.Precision("fp64"))
    E, Pt = params["E"].double(), params["P"].double()
    h = E[torch.from_numpy(ids).long()] + Pt[2:11][None]
    z = torch.nn.functional.layer_norm(h, (32,), params["lnf.g"].double(), params["lnf.b"].double(), 1e-5)
    np.testing.assert_allclose(om.forward_full(ids), (z @ E.T).numpy(), rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# invariants of the method on the tiny workload
# ----------------------------------------------------------------------------

@pytest.fixture(scope="module")
def tiny_model():
    shape = TINY.actor
    params = _tiny_params(shape)
    lora = synth.lora_params(shape, TINY.lora_rank)
    return shape, params, lora


def test_causality_prefix_logits_unchanged(tiny_model):
    shape, params, lora = tiny_model
    om = O.OracleModel(shape, params, O.Precision("fp64"), lora=lora, lora_scale=TINY.lora_scale)
    ids = synth.tokens(5, "c.ids", (2, 20), shape.vocab).numpy()
    full = om.forward_full(ids)
    pre = om.forward_full(ids[:, :13])
    np.testing.assert_allclose(full[:, :13], pre, rtol=1e-12, atol=1e-13)
    changed = ids.copy()
    changed[:, 13:] = (changed[:, 13:] + 7) % shape.vocab
    np.testing.assert_allclose(om.forward_full(changed)[:, :13], pre, rtol=1e-12, atol=1e-13)


def test_row_independence(tiny_model):
    shape, params, lora = tiny_model
    om = O.OracleModel(shape, params, O.Precision("fp64"), lora=lora, lora_scale=TINY.lora_scale)
    ids = synth.tokens(6, "r.ids", (3, 11), shape.vocab).numpy()
    full = om.forward_full(ids)
    np.testing.assert_allclose(om.forward_full(ids[1:2]), full[1:2], rtol=1e-12, atol=1e-13)


def test_position_offset(tiny_model):
    shape, params, lora = tiny_model
    ids = synth.tokens(7, "p.ids", (2, 10), shape.vocab).numpy()
    ref = O.OracleModel(shape, params, O.Precision("fp64")).forward_full(ids)
    garbage = dict(params)
    P = params["P"].clone()
    P[:2] = 1000.0                                    # rows 0 and 1 are never read
    garbage["P"] = P
    np.testing.assert_array_equal(O.OracleModel(shape, garbage, O.Precision("fp64")).forward_full(ids), ref)
    moved = dict(params)
    P = params["P"].clone()
    P[2] = params["P"][3]                              # position 0 reads row 2
    moved["P"] = P
    out = O.OracleModel(shape, moved, O.Precision("fp64")).forward_full(ids)
    assert np.abs(out[:, 0] - ref[:, 0]).max() > 1e-6


@pytest.mark.parametrize("kind,tol", [("fp64", 1e-12), ("fp32", 1e-5), ("bf16", 1e-3)])
def test_cached_decode_equals_full_recompute(tiny_model, kind, tol):
    shape, params, lora = tiny_model
    om = O.OracleModel(shape, params, O.Precision(kind), lora=lora, lora_scale=TINY.lora_scale)
    prompts = synth.prompts(TINY).numpy()
    forced = synth.forced_tokens(TINY).numpy()
    _, lc = O.greedy_generate(om, prompts, TINY.gen_len, TINY.max_seq, forced=forced, mode="cached")
    _, ld = O.greedy_generate(om, prompts, TINY.gen_len, TINY.max_seq, forced=forced, mode="definition")
    for a, b in zip(lc, ld):
        scale = np.abs(b).max()
        assert np.abs(a - b).max() <= tol * scale


def test_greedy_picks_are_argmax_of_definition(tiny_model):
    shape, params, lora = tiny_model
    om = O.OracleModel(shape, params, O.Precision("fp64"), lora=lora, lora_scale=TINY.lora_scale)
    prompts = synth.prompts(TINY).numpy()
    picks, _ = O.greedy_generate(om, prompts, TINY.gen_len, TINY.max_seq, mode="cached")
    seq = np.concatenate([prompts, picks], axis=1)
    full = om.forward_full(seq[:, :-1])                 # logits after every prefix
    S = prompts.shape[1]
    np.testing.assert_array_equal(O.argmax_lowest(full[:, S - 1:]), picks)


def test_bf16_mode_stores_bf16_values(tiny_model):
    shape, params, lora = tiny_model
    # the tiny workload is fp32; use its bf16 twin to exercise the bf16 storage points
    shp = synth.ModelShape(**{**shape.__dict__, "dtype": "bf16"})
    p16 = synth.model_params(shp)
    l16 = synth.lora_params(shp, TINY.lora_rank)
    prec = O.Precision("bf16")
    om = O.OracleModel(shp, p16, prec, lora=l16, lora_scale=TINY.lora_scale)
    lw = om.layer(0)
    for k in ("qkv.w", "out.w", "fc1.w", "fc2.w"):
        assert np.array_equal(lw[k], O.round_bf16(lw[k]))
    _, cache = om.prefill(synth.prompts(TINY).numpy(), TINY.max_seq)
    for arr in (cache.k[0], cache.v[1]):
        assert np.array_equal(arr, O.round_bf16(arr))
    # bf16 storage stays close to the float64 definition at this size
    ids = synth.prompts(TINY).numpy()
    ref = O.OracleModel(shp, p16, O.Precision("fp64"), lora=l16, lora_scale=TINY.lora_scale).forward_full(ids)
    got = om.forward_full(ids)
    assert np.abs(got - ref).max() < 2e-2
    assert np.abs(got - ref).max() > 0                   # the rounding is really applied
