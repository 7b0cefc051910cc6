"""Planted mistakes in the oracle (on the CPU) must fail its pins.

Each mutation below is a plausible slip in writing the forward pass: a transposed GQA head
mapping, a flipped RoPE rotation, SiLU on the wrong branch, a dropped per-head k norm. The
transformers pin (test_forward_matches_transformers_qwen3) must reject every one of them.
"""
import numpy as np
import pytest

import synth
import oracle
from oracle import model as om
from test_oracle_pins import MINI, _hf_model


def _orig_attention(q, K, V, pos):
    return ORIG["attention"](q, K, V, pos)


ORIG = {"attention": om.attention, "rope": om.rope, "silu": om.silu, "rmsnorm": om.rmsnorm}


def _attention_mod_mapping(q, K, V, q_pos):
    T, nq, d = q.shape
    nkv = K.shape[1]
    g = nq // nkv
    perm = [(h % nkv) * g + h // nkv for h in range(nq)]          # head h reads KV head h % nkv
    o = ORIG["attention"](q[:, perm, :], K, V, q_pos).reshape(T, nq, d)
    inv = np.argsort(perm)
    return o[:, inv, :].reshape(T, nq * d)


def _rope_flipped(x, cos, sin):
    return ORIG["rope"](x, cos, -sin)


MUTATIONS = {
    "gqa_mapping": ("attention", _attention_mod_mapping),
    "rope_sign": ("rope", _rope_flipped),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS) + ["silu_on_up"])
def test_transformers_pin_rejects_mutation(name, monkeypatch):
    torch = pytest.importorskip("torch")
    shape = MINI
    hf = _hf_model(shape, 5)
    ids = synth.token_ids(6, 40, shape.vocab)
    with torch.no_grad():
        ref = hf(torch.from_numpy(ids.astype(np.int64))[None]).logits[0].double().numpy()
    m = oracle.OracleModel(shape, 5)
    if name == "silu_on_up":
        for l in range(shape.n_layers):                            # swap the roles of gate and up
            w = m.layer(l)
            w["gate"], w["up"] = w["up"].copy(), w["gate"].copy()
    else:
        attr, fn = MUTATIONS[name]
        monkeypatch.setattr(om, attr, fn)
    got = oracle.OracleSession(m, oracle.ContiguousKV.for_shape(shape, 64), kv_round=False).forward(ids, all_logits=True)
    worst = max(om.nmse(got[t], ref[t]) for t in range(len(ids)))
    assert worst > 1e-6, f"mutation {name} went unnoticed (worst NMSE {worst:.3e})"
