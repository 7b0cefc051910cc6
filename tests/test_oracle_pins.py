"""Pins of the oracle against things other than itself: published vectors, closed forms,
brute force on tiny inputs, library routines (torch SDPA, transformers' Qwen3) and the
invariants the pages require (cached = recomputed, paged = contiguous bitwise, the
mutation faults are caught)."""
import json
import math
import os

import numpy as np
import pytest

import synth
import oracle
from oracle import model as om
from oracle.q8_0 import quantize_q8_0, dequantize_q8_0

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# A small shape with the real head width, used where the full tiny workload would be slow.
MINI = synth.ModelShape("mini", n_layers=2, hidden=256, n_q_heads=4, ffn=384, vocab=1000, n_kv_heads=2)


def test_splitmix64_published_vector():
    g = json.load(open(os.path.join(GOLDEN, "splitmix64_vector.json")))
    got = [synth.h(g["seed"], i) for i in range(len(g["outputs"]))]
    assert got == [int(x) for x in g["outputs"]]
    arr = synth.h_array(g["seed"], 0, len(g["outputs"]))
    assert [int(x) for x in arr] == [int(x) for x in g["outputs"]]


def test_weight_generator_moments_and_support():
    w = synth.bf16_bits_to_f32(synth.weight_bits(synth.weight_key(7, 3), (512, 1024)))
    assert abs(float(w.mean())) < 2e-4
    assert abs(float(w.std()) / 0.02 - 1.0) < 0.01
    # Irwin-Hall(4) support: |z| <= 131070 / std(S)
    assert float(np.abs(w).max()) <= 0.02 * 131070 / synth.IH4_STD * (1 + 2 ** -8)
    # chunked generation equals one-shot generation (counter based: no stream state)
    a = synth.weight_bits(99, (5 << 20,))
    b = np.concatenate([synth._weight_chunk(99, 0, 3 << 20), synth._weight_chunk(99, 3 << 20, 2 << 20)])
    assert np.array_equal(a, b)


def test_bf16_round_ties_to_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -(1.0 + 2 ** -8), 3.0, 0.0],
                 dtype=np.float32)
    want = np.array([1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -1.0, 3.0, 0.0], dtype=np.float32)
    assert np.array_equal(om.bf16_round(x), want)


def test_rmsnorm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 256)).astype(np.float32)
    y = om.rmsnorm(x, np.ones(256, np.float32), 1e-6)
    assert np.allclose(np.sqrt(np.mean(y.astype(np.float64) ** 2, axis=1)), 1.0, atol=1e-5)
    assert np.allclose(om.rmsnorm(4.0 * x, np.ones(256, np.float32), 1e-6), y, atol=1e-5)
    w = rng.standard_normal(256).astype(np.float32)
    assert np.allclose(om.rmsnorm(x, w, 1e-6), y * w, atol=1e-5)


def test_rope_closed_forms():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, 3, 128)).astype(np.float32)
    c0, s0 = om.rope_tables(1e6, np.array([0]))
    assert np.array_equal(om.rope(x, c0, s0), x)                 # position 0 is the identity
    pos = np.array([5, 777, 12799])
    c, s = om.rope_tables(1e6, pos)
    xs = np.repeat(x, 3, axis=0)
    y = om.rope(xs, c, s).astype(np.float64)
    # textbook complex form: (x_i + i x_{i+64}) * exp(i p theta^(-2i/128))
    z = xs[..., :64].astype(np.float64) + 1j * xs[..., 64:].astype(np.float64)
    ang = pos[:, None].astype(np.float64) * (1e6 ** (-np.arange(64) / 64.0))[None, :]
    zr = z * np.exp(1j * ang)[:, None, :]
    assert np.allclose(y[..., :64], zr.real, atol=1e-5) and np.allclose(y[..., 64:], zr.imag, atol=1e-5)
    # pair norms preserved
    assert np.allclose(np.abs(z), np.hypot(y[..., :64], y[..., 64:]), atol=1e-5)


def test_rope_relative_position():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 128)).astype(np.float32)
    k = rng.standard_normal((1, 1, 128)).astype(np.float32)

    def dot(p, s):
        cq, sq = om.rope_tables(1e6, np.array([p]))
        ck, sk = om.rope_tables(1e6, np.array([s]))
        return float(np.sum(om.rope(q, cq, sq).astype(np.float64) * om.rope(k, ck, sk)))

    assert abs(dot(10, 3) - dot(1007, 1000)) < 1e-4
    assert abs(dot(300, 0) - dot(9300, 9000)) < 1e-3


def test_silu_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 30.0, -200.0], dtype=np.float32)
    y = om.silu(z).astype(np.float64)
    assert y[0] == 0.0
    assert abs(y[1] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-7
    assert abs(y[2] + 1.0 / (1.0 + math.exp(1.0))) < 1e-7
    assert abs(y[3] - 30.0) < 1e-5 and y[4] == 0.0


def _attn_brute(q, K, V, pos):
    """Pure-Python float64 loops: softmax over visible keys, weighted sum of values."""
    T, nq, d = q.shape
    nkv = K.shape[1]
    g = nq // nkv
    o = np.zeros((T, nq, d))
    for t in range(T):
        for hh in range(nq):
            kv = hh // g
            js = [j for j in range(K.shape[0]) if j <= pos[t]]
            sc = [sum(float(q[t, hh, i]) * float(K[j, kv, i]) for i in range(d)) / math.sqrt(d) for j in js]
            mx = max(sc)
            e = [math.exp(s - mx) for s in sc]
            z = sum(e)
            for i in range(d):
                o[t, hh, i] = sum(e[a] * float(V[js[a], kv, i]) for a in range(len(js))) / z
    return o.reshape(T, nq * d)


@pytest.mark.parametrize("nq,nkv", [(4, 2), (8, 2), (2, 2)])
def test_attention_brute_force(nq, nkv):
    rng = np.random.default_rng(nq * 10 + nkv)
    T, n, d = 5, 9, 8
    q = rng.standard_normal((T, nq, d)).astype(np.float32)
    K = rng.standard_normal((n, nkv, d)).astype(np.float32)
    V = rng.standard_normal((n, nkv, d)).astype(np.float32)
    pos = np.array([0, 3, 4, 7, 8])
    assert np.allclose(om.attention(q, K, V, pos), _attn_brute(q, K, V, pos), atol=2e-6)


def test_attention_special_cases():
    rng = np.random.default_rng(3)
    d = 128
    K = rng.standard_normal((6, 2, d)).astype(np.float32)
    V = rng.standard_normal((6, 2, d)).astype(np.float32)
    q = rng.standard_normal((1, 4, d)).astype(np.float32)
    o = om.attention(q, K, V, np.array([0])).reshape(4, d)        # one visible key -> V exactly
    assert np.array_equal(o[0], V[0, 0]) and np.array_equal(o[1], V[0, 0]) and np.array_equal(o[2], V[0, 1])
    z = np.zeros((1, 4, d), np.float32)                               # uniform scores -> mean of visible V
    o = om.attention(z, K, V, np.array([4])).reshape(4, d)
    assert np.allclose(o[3], V[:5, 1].mean(axis=0), atol=1e-6)


def test_attention_vs_torch_sdpa():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    T, nq, nkv, d = 37, 8, 2, 128
    q = rng.standard_normal((T, nq, d)).astype(np.float32)
    K = rng.standard_normal((T, nkv, d)).astype(np.float32)
    V = rng.standard_normal((T, nkv, d)).astype(np.float32)
    got = om.attention(q, K, V, np.arange(T))
    g = nq // nkv
    tq = torch.from_numpy(q).double().permute(1, 0, 2)
    tk = torch.from_numpy(K).double().permute(1, 0, 2).repeat_interleave(g, dim=0)
    tv = torch.from_numpy(V).double().permute(1, 0, 2).repeat_interleave(g, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    ref = ref.permute(1, 0, 2).reshape(T, nq * d).numpy()
    assert np.allclose(got, ref, atol=1e-5)


def test_q8_0_exact_multiples_and_ties():
    d = np.float32(2.0 ** -10)
    row = np.zeros(64, np.float32)
    row[:32] = np.arange(-16, 16, dtype=np.float32) * d
    row[0] = -127 * d                                   # amax = 127 d -> scale exactly 2^-10
    row[32] = 127 * d
    row[33] = 2.5 * d                                   # exact tie -> away from zero
    row[34] = -2.5 * d
    row[35] = 0.49 * d
    scale, q = quantize_q8_0(row[None, :])
    assert scale.dtype == np.float16 and float(scale[0, 0]) == 2.0 ** -10 and float(scale[0, 1]) == 2.0 ** -10
    assert q[0, 0] == -127 and list(q[0, 1:32]) == list(range(-15, 16))
    assert q[0, 32] == 127 and q[0, 33] == 3 and q[0, 34] == -3 and q[0, 35] == 0
    assert np.array_equal(dequantize_q8_0(scale, q)[0, :32], row[:32])
    zero_s, zero_q = quantize_q8_0(np.zeros((1, 32), np.float32))   # all-zero block
    assert float(zero_s[0, 0]) == 0.0 and not zero_q.any()


def test_q8_0_error_bound():
    w = synth.bf16_bits_to_f32(synth.weight_bits(11, (64, 256)))
    scale, q = quantize_q8_0(w)
    deq = dequantize_q8_0(scale, q)
    amax = np.abs(w.reshape(64, 8, 32)).max(axis=2)
    d = amax / 127.0
    bound = d / 2 + 127 * np.abs(scale.astype(np.float64) - d)        # rounding + fp16 scale error
    err = np.abs(deq - w).reshape(64, 8, 32).max(axis=2)
    assert np.all(err <= bound * (1 + 1e-6) + 1e-12)
    assert np.all(np.abs(q) <= 127)


def test_affine4_exact_grid_ties_and_constant_groups():
    """AFFINE4_GS32 (Kipp Model Support, "Quantization (AFFINE4_GS32)"): values on the group's
    16-level grid come back exactly; half-way values round away from zero; a constant group has
    scale 0, codes 0 and the fp16 bias as its value."""
    from oracle.affine4 import quantize_affine4, dequantize_affine4
    d, b = 2.0 ** -8, -0.0625
    g0 = (b + d * np.arange(16)).astype(np.float32)
    row = np.concatenate([g0, g0[::-1], np.full(32, 0.03125, np.float32), np.zeros(32, np.float32)])
    row[64 + 1] = 0.0                                   # group 2: min 0, max 2^-5 -> d = 2^-5 / 15
    grid = np.concatenate([g0, g0]).astype(np.float32)
    grid[5] = np.float32(b + 2.5 * d)                   # tie: (v - bias) / scale = 2.5 -> 3
    grid[6] = np.float32(b + 0.49 * d)                  # -> 0
    scale, bias, q = quantize_affine4(grid[None, :])
    assert scale.dtype == np.float16 and float(scale[0, 0]) == d and float(bias[0, 0]) == b
    assert q[0, 5] == 3 and q[0, 6] == 0
    want = list(range(16)) * 2
    want[5], want[6] = 3, 0
    assert list(q[0]) == want
    deq = dequantize_affine4(scale, bias, q)[0]
    exact = [i for i in range(32) if i not in (5, 6)]
    assert np.array_equal(deq[exact], grid[exact].astype(np.float64))
    c = np.full((1, 32), 0.1, np.float32)               # constant group
    cs, cb, cq = quantize_affine4(c)
    assert float(cs[0, 0]) == 0.0 and not cq.any()
    assert dequantize_affine4(cs, cb, cq)[0, 0] == float(np.float16(np.float32(0.1)))
    rs, rb, rq = quantize_affine4(row[None, :])
    assert rq.max() <= 15 and np.array_equal(dequantize_affine4(rs, rb, rq)[0, :32], row[:32].astype(np.float64))


def test_affine4_error_bound():
    """Per group: |w - dequantised| <= scale/2 (code rounding) + 15 |scale - d| + |bias - min|
    (the fp16 roundings of the FP32 scale and minimum), and every code is in 0..15."""
    from oracle.affine4 import quantize_affine4, dequantize_affine4
    w = synth.bf16_bits_to_f32(synth.weight_bits(12, (64, 256)))
    scale, bias, q = quantize_affine4(w)
    deq = dequantize_affine4(scale, bias, q)
    g = w.reshape(64, 8, 32).astype(np.float64)
    mn, mx = g.min(axis=2), g.max(axis=2)
    d = (mx - mn) / 15
    s64, b64 = scale.astype(np.float64), bias.astype(np.float64)
    bound = s64 / 2 + 15 * np.abs(s64 - d) + np.abs(b64 - mn)
    err = np.abs(deq - w).reshape(64, 8, 32).max(axis=2)
    assert np.all(err <= bound * (1 + 1e-6) + 1e-12)
    assert q.max() <= 15 and np.all(scale.astype(np.float64) > 0)
    assert np.array_equal(deq.astype(np.float32).astype(np.float64), deq)   # the FP32 copy is exact


def test_affine4_size_matches_published_ratio():
    """Kipp Model Support, "Quantization (AFFINE4_GS32)": 5.0 bits per weight (16 bytes of codes +
    fp16 scale + fp16 bias per 32 weights); Kipp Roadmap, "Delivered since": about 2.6x smaller
    than BF16 -- the 4B shape with its seven projections in AFFINE4 and the tied embedding and
    norms in BF16 gives that ratio."""
    assert (16 + 2 + 2) * 8 / 32 == 5.0
    sh = synth.SHAPES["qwen3-4b-shape"]
    proj = sum(int(np.prod(s)) for nm, s in sh.layer_tensor_shapes().items() if nm in oracle.OracleModel.PROJ)
    norms = sum(int(np.prod(s)) for nm, s in sh.layer_tensor_shapes().items() if nm not in oracle.OracleModel.PROJ)
    emb = sh.vocab * sh.hidden * (1 if sh.tied else 2)
    bf16 = 2 * (sh.n_layers * (proj + norms) + emb + sh.hidden)
    a4 = sh.n_layers * (proj * 20 // 32 + 2 * norms) + 2 * (emb + sh.hidden)
    assert 2.55 <= bf16 / a4 <= 2.7


def test_parameter_inventory_matches_published_sizes():
    g = json.load(open(os.path.join(GOLDEN, "artifact_sizes.json")))
    sh = synth.SHAPES[g["shape"]]
    proj = sum(int(np.prod(s)) for nm, s in sh.layer_tensor_shapes().items() if nm in oracle.OracleModel.PROJ)
    norms = sum(int(np.prod(s)) for nm, s in sh.layer_tensor_shapes().items() if nm not in oracle.OracleModel.PROJ)
    emb = sh.vocab * sh.hidden * (1 if sh.tied else 2)
    bf16 = 2 * (sh.n_layers * (proj + norms) + emb + sh.hidden)
    q8 = sh.n_layers * (proj * 34 // 32 + 2 * norms) + 2 * (emb + sh.hidden)
    gib = 2.0 ** 30
    assert g["bf16_gib"] - g["tolerance_gib"] <= bf16 / gib <= g["bf16_gib"]
    assert g["q8_0_gib"] - g["tolerance_gib"] <= q8 / gib <= g["q8_0_gib"]


def _hf_model(shape, seed):
    torch = pytest.importorskip("torch")
    tr = pytest.importorskip("transformers")
    cfg = tr.Qwen3Config(vocab_size=shape.vocab, hidden_size=shape.hidden, intermediate_size=shape.ffn,
                         num_hidden_layers=shape.n_layers, num_attention_heads=shape.n_q_heads,
                         num_key_value_heads=shape.n_kv_heads, head_dim=shape.head_dim,
                         rms_norm_eps=shape.rms_eps, rope_theta=shape.rope_theta,
                         tie_word_embeddings=shape.tied, max_position_embeddings=4096,
                         attn_implementation="eager", torch_dtype=torch.float32)
    hf = tr.Qwen3ForCausalLM(cfg).float().eval()
    names = {"q": "self_attn.q_proj", "k": "self_attn.k_proj", "v": "self_attn.v_proj", "o": "self_attn.o_proj",
             "q_norm": "self_attn.q_norm", "k_norm": "self_attn.k_norm", "attn_norm": "input_layernorm",
             "ffn_norm": "post_attention_layernorm", "gate": "mlp.gate_proj", "up": "mlp.up_proj",
             "down": "mlp.down_proj"}
    sd = {"model.embed_tokens.weight": synth.tensor_bits(shape, seed, "embed"),
          "model.norm.weight": synth.tensor_bits(shape, seed, "final_norm")}
    if not shape.tied:
        sd["lm_head.weight"] = synth.tensor_bits(shape, seed, "lm_head")
    for l in range(shape.n_layers):
        for nm, hfn in names.items():
            sd[f"model.layers.{l}.{hfn}.weight"] = synth.tensor_bits(shape, seed, nm, l)
    sd = {k: torch.from_numpy(synth.bf16_bits_to_f32(v).copy()) for k, v in sd.items()}
    missing, unexpected = hf.load_state_dict(sd, strict=False)
    assert not unexpected and all(m == "lm_head.weight" for m in missing)
    if shape.tied:
        hf.tie_weights()
    return hf


@pytest.mark.parametrize("tied,theta", [(True, 1e6), (False, 5e6)])
def test_forward_matches_transformers_qwen3(tied, theta):
    """With the BF16 KV rounding switched off the oracle is the standard Qwen3 forward."""
    torch = pytest.importorskip("torch")
    shape = synth.reduced(MINI, tied=tied, rope_theta=theta)
    hf = _hf_model(shape, 5)
    ids = synth.token_ids(6, 45, shape.vocab)
    with torch.no_grad():
        ref = hf(torch.from_numpy(ids.astype(np.int64))[None]).logits[0].double().numpy()
    m = oracle.OracleModel(shape, 5)
    s = oracle.OracleSession(m, oracle.ContiguousKV.for_shape(shape, 64), kv_round=False)
    got = s.forward(ids, all_logits=True)
    for t in range(len(ids)):
        assert om.nmse(got[t], ref[t]) < 1e-9, t
        assert om.argmax(got[t]) == int(np.argmax(ref[t]))
    # incremental decode through the cache also matches the library's full forward
    s2 = oracle.OracleSession(m, oracle.ContiguousKV.for_shape(shape, 64), kv_round=False)
    s2.prefill(ids[:30])
    for t in range(30, 45):
        assert om.nmse(s2.decode(int(ids[t])), ref[t]) < 1e-9


def test_kv_rounding_is_the_only_deviation():
    """Storage contract: BF16 K/V changes logits slightly (well under the 5e-5 Phase-1 bound)."""
    m = oracle.OracleModel(MINI, 8)
    ids = synth.token_ids(9, 40, MINI.vocab)
    a = oracle.OracleSession(m, oracle.ContiguousKV.for_shape(MINI, 64)).forward(ids, all_logits=True)
    b = oracle.OracleSession(m, oracle.ContiguousKV.for_shape(MINI, 64), kv_round=False).forward(ids, all_logits=True)
    worst = max(om.nmse(a[t], b[t]) for t in range(len(ids)))
    assert 0 < worst < 5e-5


def test_zeroed_branches_reduce_to_embedding_lookup():
    """With o_proj and down_proj zeroed the residual stream stays E[id]; the tied logits then peak at id."""
    m = oracle.OracleModel(MINI, 10)
    for l in range(MINI.n_layers):
        w = m.layer(l)
        w["o"][:] = 0
        w["down"][:] = 0
    ids = synth.token_ids(11, 20, MINI.vocab)
    lg = oracle.OracleSession(m, oracle.ContiguousKV.for_shape(MINI, 32)).forward(ids, all_logits=True)
    e = m.embed[ids]
    want = om.rmsnorm(e, m.final_norm, MINI.rms_eps) @ m.embed.T
    assert np.allclose(lg, want, atol=1e-5)
    assert [om.argmax(r) for r in lg] == list(ids)


def test_cached_decode_equals_recompute():
    """Kipp Model Support, "What the gates check": cached decode = no-cache recomputation, NMSE <= 1e-6."""
    shape = MINI
    m = oracle.OracleModel(shape, 12)
    ids = synth.token_ids(13, 72, shape.vocab)
    full = oracle.OracleSession(m, oracle.ContiguousKV.for_shape(shape, 80)).forward(ids, all_logits=True)
    s = oracle.OracleSession(m, oracle.ContiguousKV.for_shape(shape, 80))
    s.prefill(ids[:40])
    for t in range(40, 72):
        lg = s.decode(int(ids[t]))
        assert om.nmse(lg, full[t]) <= 1e-6
        assert om.argmax(lg) == om.argmax(full[t])


def _run(shape, m, kv, ids, split=33):
    s = oracle.OracleSession(m, kv)
    out = [s.prefill(ids[:split])]
    for t in ids[split:]:
        out.append(s.decode(int(t)))
    return np.stack(out)


def test_paged_shuffled_equals_contiguous_bitwise():
    shape = MINI
    m = oracle.OracleModel(shape, 14)
    ids = synth.token_ids(15, 70, shape.vocab)
    ref = _run(shape, m, oracle.ContiguousKV.for_shape(shape, 96), ids)
    pool = 12
    table = synth.shuffled_blocks(16, pool)[:3]
    got = _run(shape, m, oracle.PagedKV.for_shape(shape, pool, table), ids)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("fault", [1, 2, 3, 4])
def test_mutation_faults_are_caught(fault):
    """Kipp Reproducing, "Mutation gate": the identity-layout tolerance gate and the adversarial
    block-table gate catch different classes of addressing defect."""
    shape = MINI
    m = oracle.OracleModel(shape, 14)
    ids = synth.token_ids(15, 70, shape.vocab)
    ref = _run(shape, m, oracle.ContiguousKV.for_shape(shape, 96), ids)
    ident = _run(shape, m, oracle.PagedKV.for_shape(shape, 3, np.arange(3), fault=fault), ids)
    shuf = _run(shape, m, oracle.PagedKV.for_shape(shape, 12, synth.shuffled_blocks(16, 12)[:3], fault=fault), ids)
    identity_gate_fails = max(om.nmse(a, b) for a, b in zip(ident, ref)) > 1e-6
    shuffled_gate_fails = not np.array_equal(shuf, ref)
    assert shuffled_gate_fails
    if fault == 1:
        assert not identity_gate_fails        # read-block is invisible under the identity table
    else:
        assert identity_gate_fails


def test_seeded_inputs_are_deterministic_and_in_range():
    ids = synth.token_ids(2003, 2048)
    assert ids.min() >= 0 and ids.max() < synth.VOCAB and np.array_equal(ids, synth.token_ids(2003, 2048))
    p = synth.shuffled_blocks(3003, 264)
    assert sorted(p.tolist()) == list(range(264))
    L = synth.context_lengths(synth.CONTEXT_SEED_8B, 32)
    assert L.min() >= 512 and L.max() <= 8192


def test_next_token_log_probs_closed_forms():
    """Kipp Roadmap, status v0.0.3 (multi-row scoring): a score is the natural log of the softmax
    probability of the next id. Uniform logits give -log V; two-level logits give closed forms."""
    V = 1000
    z = np.full((1, V), 3.25, dtype=np.float32)
    assert abs(om.next_token_log_probs(z, np.array([17]))[0] + math.log(V)) < 1e-12
    a, b = 2.0, -1.5
    z = np.full((2, V), b, dtype=np.float32)
    z[:, 5] = a
    got = om.next_token_log_probs(z, np.array([5, 6]))
    assert abs(got[0] + math.log1p((V - 1) * math.exp(b - a))) < 1e-12
    assert abs(got[1] - (b - a - math.log1p((V - 1) * math.exp(b - a)))) < 1e-12


def test_next_token_log_probs_invariants_and_torch():
    """Every target's probability sums to one, a constant shift changes nothing, large logits do
    not overflow, and torch's cross entropy (a library routine) gives the negated scores."""
    import torch
    rng = np.random.default_rng(5)
    z = (rng.standard_normal((4, 300)) * 4).astype(np.float32)
    all_t = np.stack([om.next_token_log_probs(z, np.full(4, t)) for t in range(300)], axis=1)
    assert np.allclose(np.exp(all_t).sum(axis=1), 1.0, atol=1e-12)
    t = np.array([0, 7, 299, 150])
    s = om.next_token_log_probs(z, t)
    assert np.allclose(om.next_token_log_probs(z.astype(np.float64) + 1e4, t), s, atol=1e-9)
    assert np.all(np.isfinite(om.next_token_log_probs(z * 1e3, t)))
    ce = torch.nn.functional.cross_entropy(torch.from_numpy(z.astype(np.float64)), torch.from_numpy(t),
                                           reduction="none").numpy()
    assert np.allclose(-ce, s, atol=1e-12)


def test_session_score_is_next_token_log_prob_of_every_row():
    """Scoring n ids gives the n-1 log-probabilities of ids[1:] under the logits of rows 0..n-2,
    each row's logits depending only on the ids up to it (checked against a fresh session per row)."""
    m = oracle.OracleModel(MINI, 21)
    ids = synth.token_ids(22, 9, MINI.vocab)
    sc = oracle.OracleSession(m, oracle.ContiguousKV.for_shape(MINI, 16)).score(ids)
    assert sc.shape == (8,)
    for i in (0, 3, 7):
        lg = oracle.OracleSession(m, oracle.ContiguousKV.for_shape(MINI, 16)).forward(ids[:i + 1])
        z = lg.astype(np.float64)
        want = z[ids[i + 1]] - (z.max() + math.log(np.exp(z - z.max()).sum()))
        assert abs(sc[i] - want) < 2e-5       # FP32 logits of a 1-row and a 9-row pass differ in rounding
    assert np.all(sc < 0)


def test_truncate_resume_equals_fresh_evaluation():
    """Kipp Model Support, "What the gates check": after a truncation, resuming gives the logits of
    the kept prefix plus the new ids evaluated from scratch; a truncation one position off fails."""
    m = oracle.OracleModel(MINI, 23)
    a, b, c = synth.token_ids(24, 37, MINI.vocab), synth.token_ids(25, 20, MINI.vocab), synth.token_ids(26, 11, MINI.vocab)
    ref = oracle.OracleSession(m, oracle.ContiguousKV.for_shape(MINI, 96)).forward(np.concatenate([a, c]),
                                                                                    all_logits=True)[len(a):]
    s = oracle.OracleSession(m, oracle.PagedKV.for_shape(MINI, 4, synth.shuffled_blocks(27, 4)[:3]))
    s.forward(np.concatenate([a, b]))
    s.truncate(len(a))
    got = s.forward(c, all_logits=True)
    assert s.pos == len(a) + len(c)
    assert max(om.nmse(g, r) for g, r in zip(got, ref)) < 1e-10
    s.truncate(len(a) - 1)
    off = s.forward(c, all_logits=True)
    assert max(om.nmse(g, r) for g, r in zip(off, ref)) > 1e-4
    with pytest.raises(ValueError):
        s.truncate(s.pos + 1)


def test_kv_q8_0_roundtrip_exact_on_the_grid():
    """Q8_0 KV rows (Kipp Roadmap, status v0.0.4): a block whose values are integers times a power
    of two, with max |x| = 127 times it, has scale exactly that power and quantises without error;
    an all-zero block stays zero; the read value is then exact in BF16 too."""
    rng = np.random.default_rng(31)
    q = rng.integers(-127, 128, size=(3, 8, 128)).astype(np.float64)
    q[..., ::32] = 127.0                     # every block reaches the full code range
    q[1, :, 32:64] = 0.0                     # one zero block per row of the second position
    q[2, :, ::32] = -127.0                   # the maximum magnitude taken by a negative value
    x = (q * 2.0 ** -10).astype(np.float32)
    got = om.kv_q8_0_roundtrip(x)
    assert got.shape == x.shape
    assert np.array_equal(got, x)
    scale, codes = quantize_q8_0(x.reshape(-1, 128))
    sc = scale.astype(np.float32).reshape(3, 8, 4)
    assert np.all(sc[0] == 2.0 ** -10) and np.all(sc[1][:, 1] == 0) and np.all(sc[2] == 2.0 ** -10)


def test_kv_q8_0_roundtrip_error_bound():
    """|read - x| <= 0.57 d + 2^-8 |read| per element, d = max|x| / 127 of the element's block (half a
    code step, the fp16 rounding of the scale over at most 127 codes, then the BF16 read)."""
    rng = np.random.default_rng(32)
    x = (rng.standard_normal((64, 8, 128)) * rng.uniform(0.01, 30, size=(64, 8, 1))).astype(np.float32)
    got = om.kv_q8_0_roundtrip(x).astype(np.float64)
    d = np.abs(x.astype(np.float64)).reshape(64, 8, 4, 32).max(axis=3, keepdims=True) / 127
    d = np.broadcast_to(d, (64, 8, 4, 32)).reshape(64, 8, 128)
    err = np.abs(got - x)
    assert np.all(err <= 0.57 * d + 2.0 ** -8 * np.abs(got) + 1e-30)
    assert err.max() > 0                     # it does quantise


def test_kv_q8_0_session_invariants():
    """With the Q8_0 KV cache: cached decode equals no-cache recomputation (NMSE <= 1e-6, same argmax),
    a shuffled block table equals the contiguous layout bitwise, and logits move from the BF16-cache
    ones by a small nonzero amount (the pages gate the option by a tolerance)."""
    shape = MINI
    m = oracle.OracleModel(shape, 33)
    ids = synth.token_ids(34, 60, shape.vocab)
    full = oracle.OracleSession(m, oracle.ContiguousKV.for_shape(shape, 64), kv_quant="q8_0").forward(ids, all_logits=True)
    s = oracle.OracleSession(m, oracle.ContiguousKV.for_shape(shape, 64), kv_quant="q8_0")
    s.prefill(ids[:35])
    for t in range(35, 60):
        lg = s.decode(int(ids[t]))
        assert om.nmse(lg, full[t]) <= 1e-6
        assert om.argmax(lg) == om.argmax(full[t])

    def run(kv):
        ss = oracle.OracleSession(m, kv, kv_quant="q8_0")
        out = [ss.prefill(ids[:33])]
        out += [ss.decode(int(t)) for t in ids[33:]]
        return np.stack(out)

    ref = run(oracle.ContiguousKV.for_shape(shape, 64))
    got = run(oracle.PagedKV.for_shape(shape, 12, synth.shuffled_blocks(35, 12)[:2]))
    assert np.array_equal(got, ref)
    bf = oracle.OracleSession(m, oracle.ContiguousKV.for_shape(shape, 64)).forward(ids, all_logits=True)
    worst = max(om.nmse(full[t], bf[t]) for t in range(len(ids)))
    assert 0 < worst < 1e-3, worst
    with pytest.raises(ValueError):
        oracle.OracleSession(m, oracle.ContiguousKV.for_shape(shape, 64), kv_quant="q4")


def test_nmse_closed_forms():
    """The gate's NMSE (Kipp Model Support, "What the gates check"; the pages do not define it,
    the reading is sum((y - ref)^2) / sum(ref^2) over one position's logits): closed forms that
    fail if the normaliser is the candidate's energy, if absolute instead of squared errors are
    summed, or if the sums are accumulated in FP32."""
    r = np.array([3.0, 4.0], dtype=np.float32)
    assert om.nmse(np.array([3.0, 4.5], dtype=np.float32), r) == 0.25 / 25.0
    assert om.nmse(r, r) == 0.0
    # normaliser is the reference's energy, not the candidate's: nmse(2r, r) = 1, nmse(r, 2r) = 1/4
    assert om.nmse(2 * r, r) == 1.0
    assert om.nmse(r, 2 * r) == 0.25
    # squared, not absolute, errors
    ones = np.ones(4, dtype=np.float32)
    assert om.nmse(np.array([1.5, 0.5, 1.0, 1.0], dtype=np.float32), ones) == 0.125
    # relative scaling y = (1 + c) r gives c^2 for any r
    rng = np.random.default_rng(3)
    z = rng.standard_normal(1000)
    assert abs(om.nmse((1 + 2.0 ** -10) * z, z) / 2.0 ** -20 - 1) < 1e-12
    # scale invariance
    y = z + 1e-3 * rng.standard_normal(1000)
    assert abs(om.nmse(7.5 * y, 7.5 * z) / om.nmse(y, z) - 1) < 1e-12
    # float64 accumulation over a full vocabulary of FP32 logits: every term is exact in float64
    big = np.full(synth.VOCAB, 1000.0, dtype=np.float32)
    off = big + np.float32(1e-3)                      # 1000.0009765625 in FP32: error 2^-10 exactly
    want = (2.0 ** -10) ** 2 / 1000.0 ** 2
    assert abs(om.nmse(off, big) / want - 1) < 1e-12


def test_argmax_lowest_index_on_ties():
    """Argmax ties go to the lowest index (the reading for greedy decoding; the pages fix none)."""
    assert om.argmax(np.array([0.0, 5.0, 5.0, 1.0], dtype=np.float32)) == 1
    assert om.argmax(np.full(17, -2.5, dtype=np.float32)) == 0
    assert om.argmax(np.array([-np.inf, -1.0, -1.0], dtype=np.float32)) == 1
    z = np.random.default_rng(4).standard_normal(synth.VOCAB).astype(np.float32)
    top = z.max() + 1
    z[100000] = top
    z[7] = top
    assert om.argmax(z) == 7
    z[7] = np.nextafter(top, np.float32(-np.inf))     # one ulp below: the later index wins
    assert om.argmax(z) == 100000
