"""Pins of oracle.model (the plain transformer): an independent library
implementation (Hugging Face ``LlamaForCausalLM`` run in float64) plus closed
forms that hold for any correct implementation."""

import numpy as np
import pytest
import torch

from oracle.model import PlainModel, SlotEvaluator
from synthetic import get_workload
from synthetic.prompts import prompt_ids
from synthetic.weights import generate


def _hf_model(w, W):
    from transformers import LlamaConfig, LlamaForCausalLM
    cfg = LlamaConfig(vocab_size=w.vocab, hidden_size=w.d_model, intermediate_size=w.d_ffn,
                      num_hidden_layers=w.n_layers, num_attention_heads=w.n_heads,
                      num_key_value_heads=w.n_kv_heads, head_dim=w.head_dim,
                      rms_norm_eps=w.eps, rope_theta=w.rope_base, tie_word_embeddings=w.tied,
                      max_position_embeddings=4096, attention_bias=False, mlp_bias=False)
    cfg._attn_implementation = "eager"
    m = LlamaForCausalLM(cfg).double().eval()
    sd = {"model.embed_tokens.weight": W["embed"], "model.norm.weight": W["final_norm"],
          "lm_head.weight": W["lm_head"]}
    names = {"wq": "self_attn.q_proj", "wk": "self_attn.k_proj", "wv": "self_attn.v_proj",
             "wo": "self_attn.o_proj", "w_gate": "mlp.gate_proj", "w_up": "mlp.up_proj",
             "w_down": "mlp.down_proj", "attn_norm": "input_layernorm",
             "ffn_norm": "post_attention_layernorm"}
    for i, lw in enumerate(W["layers"]):
        for k, v in names.items():
            sd[f"model.layers.{i}.{v}.weight"] = lw[k]
    sd = {k: v.to(torch.float64) for k, v in sd.items()}
    m.load_state_dict(sd, strict=False)
    return m


@pytest.mark.parametrize("variant", [
    dict(),                                                        # tiny, tied, MHA
    dict(n_kv_heads=2, tied=False, gamma=0.9, n_layers=3),         # GQA, untied head
    dict(dtype="bf16", d_model=128, n_heads=2, n_kv_heads=1, head_dim=64, d_ffn=256,
         vocab=512, n_layers=2, tied=False),                       # bf16 storage, MQA
])
def test_forward_matches_transformers_llama(variant):
    w = get_workload("tiny_f32").scaled(**variant)
    W = generate(w)
    toks = prompt_ids("uniform", w.vocab, 40, 99, 0)
    hf = _hf_model(w, W)
    with torch.no_grad():
        ref = hf(torch.tensor(toks[None], dtype=torch.long)).logits[0].numpy()
    m = PlainModel(w, W)
    _, _, hs = m.prefill(list(toks))
    ours = m.logits(hs[-1])
    scale = np.abs(ref).max()
    # HF computes RMSNorm statistics and RoPE angles in float32: errors ~1e-7
    # relative. A dropped term, sign or transposed operand is O(1).
    assert np.abs(ours - ref).max() <= 1e-5 * max(1.0, scale)


def _tiny_model(**kw):
    w = get_workload("tiny_f32").scaled(**kw)
    return w, PlainModel(w, generate(w))


def test_attention_over_one_key_returns_its_value():
    w, m = _tiny_model(n_kv_heads=2)
    rng = np.random.default_rng(0)
    q = rng.normal(size=(w.n_heads, w.head_dim))
    K = rng.normal(size=(1, w.n_kv_heads, w.head_dim))
    V = rng.normal(size=(1, w.n_kv_heads, w.head_dim))
    out = m.attend(q, K, V).reshape(w.n_heads, w.head_dim)
    rep = w.n_heads // w.n_kv_heads
    for h in range(w.n_heads):
        assert np.allclose(out[h], V[0, h // rep], atol=1e-15)


def test_rmsnorm_has_unit_rms():
    w, m = _tiny_model()
    x = np.random.default_rng(1).normal(size=(5, w.d_model)) * 7.0
    y = m.rmsnorm(x, np.ones(w.d_model))
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0 / np.sqrt(1 + w.eps / np.mean(x * x, axis=-1)), rtol=1e-12)


def test_rope_preserves_norm_and_is_relative():
    w, m = _tiny_model()
    rng = np.random.default_rng(2)
    q = rng.normal(size=(1, 1, w.head_dim))
    k = rng.normal(size=(1, 1, w.head_dim))
    for p in (0, 3, 17, 400):
        assert np.isclose(np.linalg.norm(m.rope(q, np.array([p]))), np.linalg.norm(q), rtol=1e-13)
    dots = [float(np.sum(m.rope(q, np.array([p + 9])) * m.rope(k, np.array([p])))) for p in (0, 5, 123)]
    assert np.allclose(dots, dots[0], rtol=1e-11)
    assert np.allclose(m.rope(q, np.array([0])), q)


def test_incremental_slots_equal_full_recompute():
    w, m = _tiny_model(tied=False, gamma=0.9)
    toks = list(prompt_ids("uniform", w.vocab, 20, 5, 0))
    ev = SlotEvaluator(m)
    ev.begin(toks[:12])
    # extend the context through slots (anchor, t12, t13, ...) and then commit
    slot = (toks[11],)
    ev.eval_slots([slot])
    for t in toks[12:16]:
        slot = slot + (t,)
        ev.eval_slots([slot])
    _, _, hs = m.prefill(toks[:16])
    for depth in (1, 4, w.n_layers):
        assert np.allclose(ev.logits(slot, depth), m.logits(hs[depth][15]), atol=1e-12)
    ev.commit(toks[12])
    ev.commit(toks[13])
    assert ev.C == 13
    assert np.allclose(ev.logits((toks[13], toks[14], toks[15]), w.n_layers), m.logits(hs[-1][15]), atol=1e-12)
