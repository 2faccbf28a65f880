"""Pins of the oracle's decoder forward (CPU only).

The pages print no logit values, so the forward is pinned by closed forms,
invariants, brute force and an independent library implementation of the
same architecture (transformers' Qwen2 decoder with its biases zeroed).
"""
import numpy as np
import pytest
import torch

from block_verify_amd.shapes import TINY, ModelShape
from block_verify_amd.synth import make_prompt, make_weights
from oracle.model import (OracleCache, OracleWeights, causal_attention, forward, full_recompute_logits, round_bf16,
                          prefill, rms_norm, rope_rotate_half)

MICRO = ModelShape("micro", 2, 64, 4, 2, 16, 96, 128)


def test_rmsnorm_constant_vector():
    x = np.full((1, 64), -3.0)
    y = rms_norm(x, np.ones(64), 1e-6)
    # |x| / sqrt(x^2 + eps) = 1 - eps/(2 x^2) + ...
    np.testing.assert_allclose(y, -np.ones((1, 64)) / np.sqrt(1 + 1e-6 / 9), rtol=0, atol=1e-15)


def test_rmsnorm_gain_and_scale_invariance():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 32))
    g = rng.standard_normal(32)
    a = rms_norm(x, g, 0.0)
    b = rms_norm(7.5 * x, g, 0.0)
    np.testing.assert_allclose(a, b, rtol=1e-13)
    np.testing.assert_allclose(np.mean((a / g) ** 2, axis=1), 1.0, rtol=1e-12)


def test_rope_identity_at_position_zero():
    x = np.random.default_rng(0).standard_normal((1, 3, 8))
    np.testing.assert_array_equal(rope_rotate_half(x, np.array([0]), 1e6), x)


def test_rope_hand_example_rotate_half_pairing():
    # d = 4, theta = 100: pair (0,2) turns by pos*1, pair (1,3) by pos*100^(-1/2) = pos*0.1
    x = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    pos = np.array([2])
    a0, a1 = 2.0, 0.2
    expect = [1 * np.cos(a0) - 3 * np.sin(a0), 2 * np.cos(a1) - 4 * np.sin(a1),
              3 * np.cos(a0) + 1 * np.sin(a0), 4 * np.cos(a1) + 2 * np.sin(a1)]
    np.testing.assert_allclose(rope_rotate_half(x, pos, 100.0)[0, 0], expect, rtol=1e-14)


def test_rope_norm_and_relative_position():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    rq = lambda p: rope_rotate_half(q, np.array([p]), 1e6)[0, 0]
    rk = lambda p: rope_rotate_half(k, np.array([p]), 1e6)[0, 0]
    np.testing.assert_allclose(np.linalg.norm(rq(777)), np.linalg.norm(q), rtol=1e-13)
    d1 = rq(1000) @ rk(990)
    d2 = rq(17) @ rk(7)
    np.testing.assert_allclose(d1, d2, rtol=1e-9)


def test_attention_single_key_returns_value():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 4, 16))
    k = rng.standard_normal((2, 1, 16))
    v = rng.standard_normal((2, 1, 16))
    o = causal_attention(q, k, v, np.array([0]), group=2).reshape(1, 4, 16)
    for h in range(4):
        np.testing.assert_allclose(o[0, h], v[h // 2, 0], rtol=1e-15)


def test_attention_matches_torch_sdpa_causal_gqa():
    rng = np.random.default_rng(3)
    T, M, nq, nkv, d = 37, 5, 6, 2, 16
    q = rng.standard_normal((M, nq, d))
    k = rng.standard_normal((nkv, T, d))
    v = rng.standard_normal((nkv, T, d))
    pos = np.arange(T - M, T)
    ours = causal_attention(q, k, v, pos, group=nq // nkv).reshape(M, nq, d)
    mask = torch.from_numpy(np.arange(T)[None, :] <= pos[:, None])
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(np.repeat(k, nq // nkv, axis=0))[None]
    tv = torch.from_numpy(np.repeat(v, nq // nkv, axis=0))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)[0].permute(1, 0, 2)
    np.testing.assert_allclose(ours, ref.numpy(), rtol=1e-12, atol=1e-12)


def _hf_qwen2_logits(shape, tensors, tokens):
    """Logits from transformers' Qwen2 decoder loaded with the same weights (biases zero)."""
    from transformers import Qwen2Config, Qwen2ForCausalLM
    from oracle.model import bf16_to_f64
    cfg = Qwen2Config(vocab_size=shape.vocab, hidden_size=shape.hidden, intermediate_size=shape.ffn,
                      num_hidden_layers=shape.n_layers, num_attention_heads=shape.n_q_heads,
                      num_key_value_heads=shape.n_kv_heads, head_dim=shape.head_dim,
                      rope_theta=shape.rope_theta, rms_norm_eps=shape.rms_eps,
                      tie_word_embeddings=False, max_position_embeddings=4096,
                      attn_implementation="eager")
    model = Qwen2ForCausalLM(cfg).to(torch.float64).eval()
    names = {n: i for i, (n, _, _) in enumerate(shape.tensor_specs())}
    t = lambda name: torch.from_numpy(bf16_to_f64(tensors[names[name]]))
    with torch.no_grad():
        model.model.embed_tokens.weight.copy_(t("embed"))
        for l, layer in enumerate(model.model.layers):
            layer.input_layernorm.weight.copy_(t(f"l{l}.attn_norm"))
            layer.self_attn.q_proj.weight.copy_(t(f"l{l}.wq"))
            layer.self_attn.k_proj.weight.copy_(t(f"l{l}.wk"))
            layer.self_attn.v_proj.weight.copy_(t(f"l{l}.wv"))
            for p in (layer.self_attn.q_proj, layer.self_attn.k_proj, layer.self_attn.v_proj):
                if p.bias is not None:
                    p.bias.zero_()
            layer.self_attn.o_proj.weight.copy_(t(f"l{l}.wo"))
            layer.post_attention_layernorm.weight.copy_(t(f"l{l}.mlp_norm"))
            layer.mlp.gate_proj.weight.copy_(t(f"l{l}.wgate"))
            layer.mlp.up_proj.weight.copy_(t(f"l{l}.wup"))
            layer.mlp.down_proj.weight.copy_(t(f"l{l}.wdown"))
        model.model.norm.weight.copy_(t("final_norm"))
        model.lm_head.weight.copy_(t("lm_head"))
        out = model(input_ids=torch.from_numpy(np.asarray(tokens, np.int64))[None])
    return out.logits[0].numpy()


def test_forward_matches_transformers_qwen2_tiny(tiny_weights):
    tokens = make_prompt(TINY.vocab, 40, seed=99)
    ours = full_recompute_logits(OracleWeights(TINY, tiny_weights), tokens, kv_bf16=False)
    ref = _hf_qwen2_logits(TINY, tiny_weights, tokens)
    # the library evaluates RoPE angles in float32; everything else is float64
    np.testing.assert_allclose(ours, ref, rtol=0, atol=2e-5)
    assert np.abs(ours).max() > 0.1


def test_forward_matches_transformers_nonunit_norm_gains():
    w = make_weights(MICRO, 7)
    rng = np.random.default_rng(8)
    for i, (_, shp, kind) in enumerate(MICRO.tensor_specs()):
        if kind == "norm":
            g = (1.0 + 0.5 * rng.standard_normal(shp)).astype(np.float32)
            w[i] = (g.view(np.uint32) >> 16).astype(np.uint16)
    tokens = make_prompt(MICRO.vocab, 23, seed=4)
    ours = full_recompute_logits(OracleWeights(MICRO, w), tokens, kv_bf16=False)
    ref = _hf_qwen2_logits(MICRO, w, tokens)
    np.testing.assert_allclose(ours, ref, rtol=0, atol=2e-5)


def test_incremental_cache_equals_full_recompute(tiny_weights):
    w = OracleWeights(TINY, tiny_weights)
    tokens = make_prompt(TINY.vocab, 24, seed=11)
    full = full_recompute_logits(w, tokens)
    c = OracleCache(TINY, 64)
    rows = [forward(w, c, tokens[:10])]
    for i in range(10, 24):
        rows.append(forward(w, c, tokens[i:i + 1]))
    np.testing.assert_allclose(np.concatenate(rows), full, rtol=0, atol=1e-10)


def test_block_rows_equal_sequential_rows(tiny_weights):
    w = OracleWeights(TINY, tiny_weights)
    prompt = make_prompt(TINY.vocab, 30, seed=12)
    block = make_prompt(TINY.vocab, 5, seed=13)
    c1 = OracleCache(TINY, 64)
    prefill(w, c1, prompt)
    c2 = c1.clone()
    rows = forward(w, c1, block)
    seq = np.concatenate([forward(w, c2, block[i:i + 1]) for i in range(5)])
    np.testing.assert_allclose(rows, seq, rtol=0, atol=1e-10)
    for l in range(TINY.n_layers):
        np.testing.assert_allclose(c1.k[l][:, :35], c2.k[l][:, :35], atol=1e-12)


def test_chunked_prefill_equals_unchunked(tiny_weights):
    w = OracleWeights(TINY, tiny_weights)
    prompt = make_prompt(TINY.vocab, 50, seed=14)
    a, b = OracleCache(TINY, 64), OracleCache(TINY, 64)
    la = prefill(w, a, prompt, chunk=64)
    lb = prefill(w, b, prompt, chunk=16)
    np.testing.assert_allclose(la, lb, atol=1e-10)
    assert a.length == b.length == 50
    for l in range(TINY.n_layers):
        np.testing.assert_allclose(a.v[l][:, :50], b.v[l][:, :50], atol=1e-12)


def test_trim_bounds_and_overwrite(tiny_weights):
    w = OracleWeights(TINY, tiny_weights)
    c = OracleCache(TINY, 16)
    forward(w, c, [1, 2, 3, 4])
    with pytest.raises(ValueError):
        c.trim(5)
    c.trim(2)
    assert c.length == 2
    with pytest.raises(ValueError):
        forward(w, c, list(range(15)))
    # positions past the trimmed length are rewritten by the next forward
    l_after = forward(w, c, [9])
    c2 = OracleCache(TINY, 16)
    ref = forward(w, c2, [1, 2, 9])
    np.testing.assert_allclose(l_after[0], ref[2], atol=1e-10)


def test_round_bf16_matches_torch_conversion():
    import torch
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.01171875, -3.0e-5, 65504.0]]).astype(np.float32)
    # halfway cases: bf16 neighbours 1 and 1+2^-7, midpoint 1+2^-8 ties to even (1.0)
    x = np.concatenate([x, np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_bf16(x.astype(np.float64)), ref)
    assert round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


def test_cache_stores_bf16_rounded_kv(tiny_weights):
    """Layer 0's K/V do not depend on earlier rounding: the bf16 cache holds exactly the
    rounded entries of the full-precision cache; later layers differ only slightly."""
    w = OracleWeights(TINY, tiny_weights)
    tokens = make_prompt(TINY.vocab, 20, seed=15)
    a, b = OracleCache(TINY, 32), OracleCache(TINY, 32, kv_bf16=False)
    la, lb = forward(w, a, tokens), forward(w, b, tokens)
    np.testing.assert_array_equal(a.k[0][:, :20], round_bf16(b.k[0][:, :20]))
    np.testing.assert_array_equal(a.v[0][:, :20], round_bf16(b.v[0][:, :20]))
    assert not np.array_equal(a.k[0][:, :20], b.k[0][:, :20])
    assert np.abs(la - lb).max() < 1e-2
