"""GPU parity of the opt-in Q8_0 KV cache (Kipp Roadmap, status v0.0.4: about 1.9x smaller than
BF16, gated for tolerance and placement invariance). The library with kv_quant="q8_0" against the
oracle reading its K/V the same way (oracle.model.kv_q8_0_roundtrip): identical argmax and
full-logit NMSE <= 1e-4 at prefill and every decode position; codes and scales against the
oracle's quantiser; a shuffled block table bitwise equal to the identity one; batched equal to
isolated; pooled prefix reuse and copy on write over Q8_0 blocks."""
import numpy as np
import pytest

import synth
import oracle
from oracle import model as om
from oracle.q8_0 import quantize_q8_0
from parity_util import Gate, nmse

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_gqa_decoder_amd as lib
    lib.load()
    return lib


def say(*a):
    print("[gpu kvq8]", *a, flush=True)


def oracle_greedy(shape, seed, prompt, steps, kv=None):
    m = oracle.OracleModel(shape, seed)
    kv = kv or oracle.ContiguousKV.for_shape(shape, len(prompt) + steps + 1)
    s = oracle.OracleSession(m, kv, kv_quant="q8_0")
    logits = [s.prefill(prompt)]
    toks = []
    for _ in range(steps):
        toks.append(om.argmax(logits[-1]))
        logits.append(s.decode(toks[-1]))
    return logits, toks


def teacher_forced(sess, prompt, toks, vocab):
    lg = torch.empty(vocab, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    sess.prefill(prompt, lg, am)
    torch.cuda.synchronize()
    out = [(lg.cpu().numpy(), int(am.item()))]
    for t in toks:
        sess.decode(int(t), lg, am)
        torch.cuda.synchronize()
        out.append((lg.cpu().numpy(), int(am.item())))
    return out


def check(name, got, ref):
    gate = Gate(name)
    for i, ((lg, am), r) in enumerate(zip(got, ref)):
        gate.check(i, lg, r, am)
        assert am == int(np.argmax(lg))
    gate.assert_ok()


def test_kv_q8_pool_bytes(g):
    """Per position and KV head 2 x (128 codes + 4 fp16 scales) = 272 bytes instead of 512 (1.88x);
    no BF16 copy of any layer is kept."""
    shape = synth.TINY
    nb = 8
    mq = g.Model.from_shape(shape, seed=1001, kv_pool_blocks=nb, max_positions=64, kv_quant="q8_0")
    mb = g.Model.from_shape(shape, seed=1001, kv_pool_blocks=nb, max_positions=64)
    per = nb * 8 * 32
    assert mb.info().kv_pool_bytes == shape.n_layers * per * 512
    assert mq.info().kv_pool_bytes == shape.n_layers * per * 272
    mq.close()
    mb.close()


def test_kv_q8_codes_match_oracle(g):
    """Codes and scales written by the prefill (40 positions, one round) and by four decode steps
    through a shuffled table. Layer 0 sees the same inputs on both sides: its scales are equal and
    its codes equal except where x / d falls within FP32 noise of a rounding boundary. Deeper
    layers inherit upstream differences; their read-back values are bounded by NMSE."""
    shape = synth.TINY
    prompt = synth.token_ids(9, 40)
    toks = [7, 70000, 151935, 3]
    blocks = [5, 2]
    m = g.Model.from_shape(shape, seed=1001, kv_pool_blocks=8, max_positions=64, kv_quant="q8_0")
    s = g.Session(m, 64, block_ids=blocks)
    teacher_forced(s, prompt, toks, shape.vocab)
    n = len(prompt) + len(toks)
    ids = np.concatenate([prompt, toks])
    om_ = oracle.OracleModel(shape, 1001)
    raw = oracle.ContiguousKV.for_shape(shape, 64)                  # layer-0 inputs, unquantised
    oracle.OracleSession(om_, raw, kv_round=False).forward(ids)
    kvq = oracle.PagedKV.for_shape(shape, 8, blocks)
    oq = oracle.OracleSession(om_, kvq, kv_quant="q8_0")
    oq.prefill(prompt)
    for t in toks:
        oq.decode(t)
    K0, V0 = raw.read(0, n)
    kc, ks, vc, vs = s.read_kv_q8(0, 0, n)
    for x, codes, sbits in ((K0, kc, ks), (V0, vc, vs)):
        want_s, want_c = quantize_q8_0(np.asarray(x, np.float32).reshape(-1, 128))
        want_s = want_s.reshape(n, 8, 4).view(np.uint16)
        want_c = want_c.reshape(n, 8, 128)
        # a scale may differ by one fp16 step where the block maximum, computed in FP32 on both
        # sides from differently rounded projections, sits at an fp16 rounding boundary
        sdiff = sbits.astype(int) - want_s.astype(int)
        assert np.all(np.abs(sdiff) <= 1) and np.mean(sdiff != 0) < 0.01
        d = np.abs(np.asarray(x, np.float64)).reshape(n, 8, 4, 32).max(axis=3) / 127
        r = np.asarray(x, np.float64).reshape(n, 8, 4, 32) / np.maximum(d, 1e-30)[..., None]
        ambiguous = np.abs(np.abs(r - np.trunc(r)) - 0.5) < 1e-4
        diff = codes.reshape(n, 8, 4, 32).astype(int) - want_c.reshape(n, 8, 4, 32).astype(int)
        same = (sdiff == 0)[..., None]
        assert np.all((diff == 0) | (ambiguous & (np.abs(diff) == 1)) | (~same & (np.abs(diff) <= 1)))
        assert np.mean(diff != 0) < 0.001
    for layer in range(shape.n_layers):
        k, v = s.read_kv(layer, 0, n)
        K, V = kvq.read(layer, n)
        for got, want in ((synth.bf16_bits_to_f32(k), K), (synth.bf16_bits_to_f32(v), V)):
            assert nmse(got, want) < 1e-5, layer
            assert np.mean(got == want) > 0.9, layer
    s.close()
    m.close()


def test_kv_q8_quantiser_byte_exact_on_device_inputs(g):
    """The device's Q8_0 KV quantiser (prefill K/V write) against the oracle's quantiser
    (oracle.quantize_q8_0, the Q8_0 weight rule of Kipp Model Support, "Quantization (Q8_0)") on
    the very same FP32 inputs: V rows are stored without normalisation, so after a one-round prefill
    (40 rows, the GEMM path) the round's FP32 q|k|v projection left in the model's scratch holds
    exactly what the last layer's V quantiser read. Every code and every fp16 scale bit must match,
    with no tolerance. Two prompts: random ids, and one repeated id (identical rows, scales from
    equal maxima)."""
    shape = synth.TINY
    T = 40
    QD, QKV = shape.q_dim, shape.q_dim + 2 * shape.kv_dim
    for prompt in (synth.token_ids(19, T), np.full(T, 4242, dtype=np.int32)):
        m = g.Model.from_shape(shape, seed=1001, kv_pool_blocks=4, max_positions=64, kv_quant="q8_0")
        s = g.Session(m, 64, block_ids=[3, 1])
        lg = torch.empty(shape.vocab, device="cuda")
        s.prefill(prompt, lg)
        torch.cuda.synchronize()
        qkv = m.read_scratch("qkv", 0, T * QKV).reshape(T, QKV)
        v = np.ascontiguousarray(qkv[:, QD + shape.kv_dim:QD + 2 * shape.kv_dim], dtype=np.float32)
        want_s, want_c = quantize_q8_0(v.reshape(-1, 128))
        kc, ks, vc, vs = s.read_kv_q8(shape.n_layers - 1, 0, T)
        assert np.array_equal(vs, np.asarray(want_s).reshape(T, 8, 4).view(np.uint16))
        assert np.array_equal(vc, np.asarray(want_c).reshape(T, 8, 128))
        say("V quantiser byte-exact over", T * 8 * 128, "codes and", T * 8 * 4, "scales")
        s.close()
        m.close()


def test_tiny_kv_q8_parity(g):
    """Tiny decoder with the Q8_0 cache: the 16-token prompt and 16 greedy steps, then a 100-token
    prompt in ragged rounds of 48 (each later round's attention reads the earlier rounds' codes)."""
    wl = synth.WORKLOADS["tiny"]
    shape = wl.shape
    prompt = synth.token_ids(wl.ids_seed, wl.prompt)
    ref, toks = oracle_greedy(shape, wl.weight_seed, prompt, wl.decode)
    m = g.Model.from_shape(shape, seed=wl.weight_seed, kv_pool_blocks=8, max_positions=128, kv_quant="q8_0")
    s = g.Session(m, 64)
    check("tiny kv q8", teacher_forced(s, prompt, toks, shape.vocab), ref)
    s.close()
    m.close()
    say("ragged rounds")
    p2 = synth.token_ids(77, 100)
    ref2, toks2 = oracle_greedy(shape, 1001, p2, 3)
    m2 = g.Model.from_shape(shape, seed=1001, kv_pool_blocks=8, max_positions=128, max_round_tokens=48,
                            kv_quant="q8_0")
    s2 = g.Session(m2, 128)
    check("ragged rounds kv q8", teacher_forced(s2, p2, toks2, shape.vocab), ref2)
    s2.close()
    m2.close()


def test_kv_q8_paged_shuffled_equals_identity_bitwise(g):
    shape = synth.TINY
    prompt = synth.token_ids(5, 70)
    m = g.Model.from_shape(shape, seed=1001, kv_pool_blocks=16, max_positions=96, kv_quant="q8_0")
    a = g.Session(m, 96)
    free = [b for b in synth.shuffled_blocks(3001, 16).tolist() if b >= 3][:3]
    b = g.Session(m, 96, block_ids=free)
    toks = [11, 22, 33, 44, 55, 151935, 0]
    ra = teacher_forced(a, prompt, toks, shape.vocab)
    rb = teacher_forced(b, prompt, toks, shape.vocab)
    for (x, xa), (y, ya) in zip(ra, rb):
        assert np.array_equal(x, y) and xa == ya
    for layer in range(shape.n_layers):
        for u, w in zip(a.read_kv_q8(layer, 0, 77), b.read_kv_q8(layer, 0, 77)):
            assert np.array_equal(u, w)
    for o in (a, b, m):
        o.close()


@pytest.mark.parametrize("nseq", [4, 7])
def test_kv_q8_batched_equals_isolated_bitwise(g, nseq):
    shape = synth.TINY
    lens = [20, 45, 70, 33, 140, 1, 96][:nseq]
    m = g.Model.from_shape(shape, seed=1001, kv_pool_blocks=2 * 5 * len(lens), max_positions=160, kv_quant="q8_0")
    prompts = [synth.token_ids(100 + i, n) for i, n in enumerate(lens)]
    lg = torch.empty(shape.vocab, device="cuda")
    A = [g.Session(m, 160) for _ in lens]              # 5 blocks each
    Bs = [g.Session(m, 160) for _ in lens]
    for sa, sb, p in zip(A, Bs, prompts):
        sa.prefill(p, lg)
        sb.prefill(p, lg)
    blg = torch.empty(len(lens), shape.vocab, device="cuda")
    bam = torch.empty(len(lens), dtype=torch.int32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    for step in range(4):
        ids = [(1000 * step + 7 * i) % shape.vocab for i in range(len(lens))]
        m.eval_batch(A, ids, blg, bam)
        torch.cuda.synchronize()
        batched = blg.cpu().numpy()
        for i, sb in enumerate(Bs):
            sb.decode(ids[i], lg, am)
            torch.cuda.synchronize()
            assert np.array_equal(lg.cpu().numpy(), batched[i]), (step, i)
            assert int(am.item()) == int(bam[i].item())
    for o in A + Bs + [m]:
        o.close()


def _prefill(s, ids, vocab):
    lg = torch.empty(vocab, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    s.prefill(ids, lg, am)
    torch.cuda.synchronize()
    return lg.cpu().numpy(), int(am.item())


def _oracle_last(shape, seed, ids):
    s = oracle.OracleSession(oracle.OracleModel(shape, seed), oracle.ContiguousKV.for_shape(shape, len(ids) + 1),
                             kv_quant="q8_0")
    return s.forward(ids)


def test_kv_q8_pooled_prefix_reuse(g):
    """Pooled sessions over Q8_0 blocks: a warm prompt maps the cold one's published blocks, a
    truncation into a shared block copies it (codes and scales), and every result matches the
    oracle evaluating the whole prompt."""
    wl = synth.WORKLOADS["tiny"]
    shape, seed = wl.shape, wl.weight_seed
    P = synth.token_ids(51, 200)
    other = synth.token_ids(52, 60)
    m = g.Model.from_shape(shape, seed=seed, kv_pool_blocks=64, max_positions=512, kv_quant="q8_0")
    gate = Gate("pooled kv q8")
    a = g.Session(m, 512, pooled=True)
    la, ama = _prefill(a, P, shape.vocab)
    ref_p = _oracle_last(shape, seed, P)
    gate.check(0, la, ref_p, ama)
    a.close()
    b = g.Session(m, 512, pooled=True)
    lb, amb = _prefill(b, P, shape.vocab)
    assert b.reused == 192
    gate.check(1, lb, ref_p, amb)
    assert nmse(lb, la) <= 1e-8
    b.truncate(100)
    lt, amt = _prefill(b, other[:20], shape.vocab)
    gate.check(2, lt, _oracle_last(shape, seed, np.concatenate([P[:100], other[:20]])), amt)
    e = g.Session(m, 512, pooled=True)
    le, ame = _prefill(e, P, shape.vocab)
    assert e.reused == 192
    gate.check(3, le, ref_p, ame)
    gate.assert_ok()
    for o in (b, e, m):
        o.close()


def test_qwen3_0_6b_shape_kv_q8_parity(g):
    """The 0.6B-shape workload (28 layers, 348-id prompt, shuffled block table) with the Q8_0 cache,
    16 greedy decode steps."""
    wl = synth.WORKLOADS["0.6b"]
    shape = wl.shape
    prompt = synth.token_ids(wl.ids_seed, wl.prompt)
    steps = 16
    say("0.6b oracle")
    ref, toks = oracle_greedy(shape, wl.weight_seed, prompt, steps)
    nb = synth.blocks_for(wl.prompt + steps)
    table = synth.shuffled_blocks(wl.shuffle_seed, 4 * nb)[:nb]
    m = g.Model.from_shape(shape, seed=wl.weight_seed, kv_pool_blocks=4 * nb, max_positions=nb * 32,
                           kv_quant="q8_0")
    s = g.Session(m, nb * 32, block_ids=table)
    check("0.6b kv q8", teacher_forced(s, prompt, toks, shape.vocab), ref)
    s.close()
    m.close()
