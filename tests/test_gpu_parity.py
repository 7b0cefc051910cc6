"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on the same seeded
inputs. Gate (Kipp Model Support, "What the gates check"): identical argmax and full-logit
NMSE <= 1e-4 at prefill and at every decode position; paged KV bitwise equal to the contiguous
layout (Kipp Roadmap, status v0.0.2); batched evaluation equal to isolated evaluation."""
import hashlib
import os

import numpy as np
import pytest

import synth
import oracle
from oracle import model as om
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
    print("[gpu]", *a, flush=True)


_ORACLE_CACHE = {}


def oracle_greedy_cached(key, shape, seed, prompt, steps, scheme="bf16"):
    """oracle_greedy (with the logits of every prompt row), computed once per key for the whole
    test module."""
    if key not in _ORACLE_CACHE:
        _ORACLE_CACHE[key] = oracle_greedy(shape, seed, prompt, steps, scheme, prompt_rows=True)
    ref, toks, _ = _ORACLE_CACHE[key]
    return ref, toks


def oracle_prompt_rows(key):
    """Logits [len(prompt)][vocab] of every prompt position of a cached oracle_greedy run."""
    return _ORACLE_CACHE[key][2]


def oracle_greedy(shape, seed, prompt, steps, scheme="bf16", prompt_rows=False):
    """Oracle logits at the last prompt position and at each greedy decode step, and the
    greedy tokens fed at each step (and, with prompt_rows, the logits of every prompt row)."""
    m = oracle.OracleModel(shape, seed, scheme)
    s = oracle.OracleSession(m, oracle.ContiguousKV.for_shape(shape, len(prompt) + steps + 1))
    rows = s.forward(prompt, all_logits=True) if prompt_rows else None
    logits = [rows[-1] if prompt_rows else s.prefill(prompt)]
    toks = []
    for _ in range(steps):
        t = om.argmax(logits[-1])
        toks.append(t)
        logits.append(s.decode(t))
    return (logits, toks, rows) if prompt_rows else (logits, toks)


def gpu_teacher_forced(model, sess, prompt, toks, vocab):
    lg = torch.empty(vocab, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    out = []
    sess.prefill(prompt, lg, am)
    torch.cuda.synchronize()
    out.append((lg.cpu().numpy(), int(am.item())))
    for t in toks:
        sess.decode(int(t), lg, am)
        torch.cuda.synchronize()
        out.append((lg.cpu().numpy(), int(am.item())))
    return out


def test_weights_match_generator(g):
    shape = synth.TINY
    say("weights", shape.name)
    m = g.Model.from_shape(shape, seed=1001, kv_pool_blocks=4, max_positions=64)
    H = shape.hidden
    emb = synth.tensor_bits(shape, 1001, "embed")
    for r0 in (0, 77777, shape.vocab - 8):
        assert np.array_equal(m.read_weight("embed", -1, r0, 8, H), emb[r0:r0 + 8])
    for l in range(shape.n_layers):
        for nm, dims in shape.layer_tensor_shapes().items():
            if nm in synth.NORM_TENSORS:
                continue
            rows, cols = dims
            ref = synth.tensor_bits(shape, 1001, nm, l)
            for r0 in (0, rows // 2 + 3, rows - 5):
                n = min(5, rows - r0)
                assert np.array_equal(m.read_weight(nm, l, r0, n, cols), ref[r0:r0 + n]), (nm, l, r0)
    assert np.all(m.read_weight("final_norm", -1, 0, 1, H) == 0x3F80)
    m.close()


def test_untied_lm_head_generated(g):
    shape = synth.reduced(synth.TINY, tied=False, n_layers=1)
    m = g.Model.from_shape(shape, seed=7, kv_pool_blocks=2, max_positions=32)
    ref = synth.tensor_bits(shape, 7, "lm_head")
    assert np.array_equal(m.read_weight("lm_head", -1, 1000, 4, shape.hidden), ref[1000:1004])
    m.close()


def test_rope_table_matches_oracle(g):
    shape = synth.TINY
    m = g.Model.from_shape(shape, seed=1, kv_pool_blocks=2, max_positions=13000)
    c, s = m.read_rope(13000)
    rc, rs = om.rope_tables(shape.rope_theta, np.arange(13000))
    ulp = lambda a, b: np.abs(a.view(np.int32).astype(np.int64) - b.view(np.int32).astype(np.int64))
    assert ulp(c, rc).max() <= 1 and ulp(s, rs).max() <= 1
    say("rope ulp mismatches", int((ulp(c, rc) > 0).sum() + (ulp(s, rs) > 0).sum()))
    m.close()


def test_tiny_decoder_parity(g):
    """Tiny 2-layer decoder: 16-token prompt then 16 teacher-forced greedy steps, contiguous KV."""
    wl = synth.WORKLOADS["tiny"]
    shape = wl.shape
    prompt = synth.token_ids(wl.ids_seed, wl.prompt)
    say("tiny parity", shape.name)
    ref, toks = oracle_greedy(shape, wl.weight_seed, prompt, wl.decode)
    m = g.Model.from_shape(shape, seed=wl.weight_seed, kv_pool_blocks=4, max_positions=64)
    s = g.Session(m, 64)
    got = gpu_teacher_forced(m, s, prompt, toks, shape.vocab)
    gate = Gate("tiny")
    for i, ((lg, am), r) in enumerate(zip(got, ref)):
        gate.check(i, lg, r, am)
        assert am == int(np.argmax(lg))                       # device argmax = host argmax of GPU logits
    gate.assert_ok()
    s.close()
    m.close()


def test_ragged_multi_round_prefill(g):
    """A 100-token prompt in rounds of 48 (48 + 48 + 4): ragged tails in every kernel."""
    shape = synth.TINY
    prompt = synth.token_ids(77, 100)
    ref, toks = oracle_greedy(shape, 1001, prompt, 3)
    m = g.Model.from_shape(shape, seed=1001, kv_pool_blocks=8, max_positions=128, max_round_tokens=48)
    assert m.info().round_tokens == 48
    s = g.Session(m, 128)
    got = gpu_teacher_forced(m, s, prompt, toks, shape.vocab)
    gate = Gate("ragged rounds")
    for i, ((lg, am), r) in enumerate(zip(got, ref)):
        gate.check(i, lg, r, am)
    gate.assert_ok()
    # the same prompt in one round
    m1 = g.Model.from_shape(shape, seed=1001, kv_pool_blocks=8, max_positions=128)
    s1 = g.Session(m1, 128)
    one = gpu_teacher_forced(m1, s1, prompt, toks, shape.vocab)
    for (a, _), (b, _) in zip(got, one):
        assert nmse(a, b) <= 1e-8
    for o in (s, s1, m, m1):
        o.close()


def test_paged_shuffled_equals_identity_bitwise(g):
    shape = synth.TINY
    prompt = synth.token_ids(5, 70)
    m = g.Model.from_shape(shape, seed=1001, kv_pool_blocks=16, max_positions=96)
    a = g.Session(m, 96)                                                # blocks 0, 1, 2
    free = [b for b in synth.shuffled_blocks(3001, 16).tolist() if b >= 3][:3]
    b = g.Session(m, 96, block_ids=free)
    toks = [11, 22, 33, 44, 55, 151935, 0]
    ra = gpu_teacher_forced(m, a, prompt, toks, shape.vocab)
    rb = gpu_teacher_forced(m, b, prompt, toks, shape.vocab)
    for (x, xa), (y, ya) in zip(ra, rb):
        assert np.array_equal(x, y) and xa == ya
    for layer in range(shape.n_layers):
        ka, va = a.read_kv(layer, 0, 77)
        kb, vb = b.read_kv(layer, 0, 77)
        assert np.array_equal(ka, kb) and np.array_equal(va, vb)
    for o in (a, b, m):
        o.close()


def test_kv_cache_matches_oracle_storage(g):
    """K/V written through the block table are the BF16-rounded post-norm, post-RoPE k and v."""
    shape = synth.TINY
    prompt = synth.token_ids(9, 40)
    m = g.Model.from_shape(shape, seed=1001, kv_pool_blocks=8, max_positions=64)
    blocks = [5, 2]
    s = g.Session(m, 64, block_ids=blocks)
    lg = torch.empty(shape.vocab, device="cuda")
    s.prefill(prompt, lg)
    om_ = oracle.OracleModel(shape, 1001)
    kv = oracle.PagedKV.for_shape(shape, 8, blocks)
    oracle.OracleSession(om_, kv).prefill(prompt)
    for layer in range(shape.n_layers):
        k, v = s.read_kv(layer, 0, 40)
        kf = synth.bf16_bits_to_f32(k)
        vf = synth.bf16_bits_to_f32(v)
        K, V = kv.read(layer, 40)
        # layer 0: the same BF16 value, or one BF16 step apart where the FP32 inputs straddle a
        # rounding boundary (tiny elements may move further relative to themselves: FP32 rounding
        # of the projection is relative to the head's scale). Deeper layers inherit the upstream
        # differences, so only their overall agreement is bounded.
        for got, want in ((kf, K), (vf, V)):
            diff = np.abs(got - want)
            if layer == 0:
                scale = np.sqrt(np.mean(want.astype(np.float64) ** 2, axis=-1, keepdims=True))
                step = np.abs(want) * 2.0 ** -7 + scale * 2.0 ** -14
                assert np.all(diff <= step), (layer, float((diff - step).max()))
            assert nmse(got, want) < 1e-5, layer
            assert np.mean(diff == 0) > 0.9, layer
    s.close()
    m.close()


@pytest.mark.parametrize("nseq", [4, 7, 20])
def test_batched_equals_isolated_bitwise(g, nseq):
    """Up to four rows build their operands in the matvec prologues, more rows use the row
    kernels; both must give exactly what a single row gets."""
    shape = synth.TINY
    m = g.Model.from_shape(shape, seed=1001, kv_pool_blocks=128 * 4, max_positions=160)
    lens = [20, 45, 70, 33, 140, 1, 96, 64, 65, 31, 32, 127, 128, 129, 2, 3, 50, 77, 88, 99][:nseq]
    prompts = [synth.token_ids(100 + i, n) for i, n in enumerate(lens)]
    lg = torch.empty(shape.vocab, device="cuda")
    A = [g.Session(m, 160) for _ in lens]
    Bs = [g.Session(m, 160) for _ in lens]
    for sa, sb, p in zip(A, Bs, prompts):
        sa.prefill(p, lg)
        sb.prefill(p, lg)
    blg = torch.empty(len(lens), shape.vocab, device="cuda")
    bam = torch.empty(len(lens), dtype=torch.int32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    for step in range(6):
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


def test_batched_rows_past_the_lds_block_table(g):
    """The decode attention stages each workgroup's block-table entries in LDS (one per thread,
    256) when every workgroup of the launch fits; a row-batched launch walks three chunks per
    workgroup, so past 86,016 positions it reads the table from global memory instead. Such a
    launch (tiny shape, 5 rows, two of them at 86,105 positions) must equal each row stepped
    alone -- a one-row launch, which stages its table in LDS -- bit for bit, for 2 steps."""
    shape = synth.TINY
    lens = (86105, 3000, 86105, 100, 4000)
    nb = sum(synth.blocks_for(n + 4) for n in lens)
    m = g.Model.from_shape(shape, seed=1001, kv_pool_blocks=2 * nb + 8, max_positions=86112)
    lg = torch.empty(shape.vocab, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    A, Bs = [], []
    for i, n in enumerate(lens):
        p = synth.token_ids(400 + i, n - 1)                  # decode runs at context n
        a, b = g.Session(m, n + 4), g.Session(m, n + 4)
        a.prefill(p, lg)
        b.prefill(p, lg)
        A.append(a)
        Bs.append(b)
    blg = torch.empty(len(lens), shape.vocab, device="cuda")
    bam = torch.empty(len(lens), dtype=torch.int32, device="cuda")
    for step in range(2):
        ids = [(4099 * step + 17 * i + 3) % shape.vocab for i in range(len(lens))]
        m.eval_batch(A, ids, blg, bam)
        torch.cuda.synchronize()
        for i, sb in enumerate(Bs):
            sb.decode(ids[i], lg, am)
            torch.cuda.synchronize()
            assert torch.equal(lg.view(torch.int32), blg[i].view(torch.int32)), (step, i)
            assert int(am.item()) == int(bam[i].item())
    for o in A + Bs + [m]:
        o.close()


@pytest.mark.parametrize("lens", [(8193, 4096), (8193, 4096, 3000, 100, 4000)])
def test_batched_rows_needing_more_chunks_than_the_longest(g, lens):
    """Regression: a decode row's context is cut into chunks whose length grows in steps, so the
    chunk count is not monotonic in the context (8,193 positions give 26 chunks of 320, 4,096
    give 32 of 128). The attention grid must cover the largest count of any row, not the count of
    the longest row. Tiny shape, fused (2 rows) and row-kernel (5 rows) paths: every batched row
    equals its twin stepped alone, bit for bit, for 3 steps."""
    shape = synth.TINY
    nb = sum(synth.blocks_for(n + 4) for n in lens)
    m = g.Model.from_shape(shape, seed=1001, kv_pool_blocks=2 * nb + 8, max_positions=8256)
    lg = torch.empty(shape.vocab, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    A, Bs = [], []
    for i, n in enumerate(lens):
        p = synth.token_ids(300 + i, n - 1)                  # decode runs at context n
        a, b = g.Session(m, n + 4), g.Session(m, n + 4)
        a.prefill(p, lg)
        b.prefill(p, lg)
        A.append(a)
        Bs.append(b)
    blg = torch.empty(len(lens), shape.vocab, device="cuda")
    bam = torch.empty(len(lens), dtype=torch.int32, device="cuda")
    for step in range(3):
        ids = [(4099 * step + 13 * i + 5) % shape.vocab for i in range(len(lens))]
        m.eval_batch(A, ids, blg, bam)
        torch.cuda.synchronize()
        for i, sb in enumerate(Bs):
            sb.decode(ids[i], lg, am)
            torch.cuda.synchronize()
            assert torch.equal(lg.view(torch.int32), blg[i].view(torch.int32)), (lens, step, i)
            assert int(am.item()) == int(bam[i].item())
    for o in A + Bs + [m]:
        o.close()


def test_device_ids_and_errors(g):
    shape = synth.reduced(synth.TINY, n_layers=1)
    m = g.Model.from_shape(shape, seed=3, kv_pool_blocks=4, max_positions=40)
    s = g.Session(m, 40)
    lg = torch.empty(shape.vocab, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    s.prefill([1, 2, 3], lg, am)
    with pytest.raises(g.GqaError) as e:
        s.prefill([5, shape.vocab], lg, am)
    assert e.value.code == g.GQA_E_RANGE and s.position == 3
    with pytest.raises(g.GqaError):
        s.decode(-1, lg, am)
    assert s.position == 3
    # device-resident id: the previous argmax feeds the next step without a host round trip
    ref = torch.empty_like(lg)
    s2 = g.Session(m, 40)
    s2.prefill([1, 2, 3], lg, am)
    tok = int(am.item())
    s.decode(am, lg, am)                     # s reads its id from the device buffer
    s2.decode(tok, ref)
    torch.cuda.synchronize()
    assert torch.equal(lg, ref)
    m.check_device_error()
    bad = torch.tensor([shape.vocab + 5], dtype=torch.int32, device="cuda")
    s.decode(bad, lg, am)
    with pytest.raises(g.GqaError) as e:
        m.check_device_error()
    assert e.value.code == g.GQA_E_RANGE
    m.check_device_error()                   # flag cleared
    with pytest.raises(g.GqaError) as e:
        s.prefill(list(range(40)), lg, am)
    assert e.value.code == g.GQA_E_RANGE
    for o in (s, s2, m):
        o.close()


def test_prefill_device_ids(g):
    """eval_prefill_device (ids already in HBM) gives the bits of eval_prefill (host ids), across
    two rounds; an out-of-range device id is reported through the sticky device error."""
    shape = synth.reduced(synth.TINY, n_layers=2)
    m = g.Model.from_shape(shape, seed=5, kv_pool_blocks=8, max_positions=96, max_round_tokens=32)
    ids = synth.token_ids(17, 50)
    a, b = g.Session(m, 96), g.Session(m, 96)
    la, lb = torch.empty(shape.vocab, device="cuda"), torch.empty(shape.vocab, device="cuda")
    aa, ab = torch.empty(1, dtype=torch.int32, device="cuda"), torch.empty(1, dtype=torch.int32, device="cuda")
    a.prefill(ids, la, aa)
    b.prefill(torch.from_numpy(ids.astype(np.int32)).to("cuda"), lb, ab)
    torch.cuda.synchronize()
    assert a.position == b.position == 50
    assert torch.equal(la, lb) and torch.equal(aa, ab)
    m.check_device_error()
    bad = torch.tensor([3, shape.vocab], dtype=torch.int32, device="cuda")
    b.prefill(bad, lb, ab)
    with pytest.raises(g.GqaError) as e:
        m.check_device_error()
    assert e.value.code == g.GQA_E_RANGE
    assert b.position == 52
    for o in (a, b, m):
        o.close()


def test_pool_exhaustion_and_block_validation(g):
    shape = synth.reduced(synth.TINY, n_layers=1)
    m = g.Model.from_shape(shape, seed=3, kv_pool_blocks=4, max_positions=128)
    a = g.Session(m, 64)
    with pytest.raises(g.GqaError) as e:
        g.Session(m, 128)
    assert e.value.code == g.GQA_E_OOM
    with pytest.raises(g.GqaError):
        g.Session(m, 64, block_ids=[0, 3])      # block 0 is owned by a
    with pytest.raises(g.GqaError):
        g.Session(m, 64, block_ids=[3, 3])
    b = g.Session(m, 64, block_ids=[3, 2])
    assert m.info().free_blocks == 0
    a.close()
    b.close()
    assert m.info().free_blocks == 4
    m.close()


def test_q8_0_quantisation_bytes_match_oracle(g):
    shape = synth.reduced(synth.TINY, n_layers=1)
    m = g.Model.from_shape(shape, seed=1004, scheme="q8_0", kv_pool_blocks=2, max_positions=32)
    from oracle.q8_0 import quantize_q8_0
    for nm, dims in shape.layer_tensor_shapes().items():
        if nm in synth.NORM_TENSORS:
            continue
        rows, cols = dims
        w = synth.bf16_bits_to_f32(synth.tensor_bits(shape, 1004, nm, 0))
        sc, q = quantize_q8_0(w)
        for r0 in (0, rows - 7):
            gq, gs = m.read_q8(nm, 0, r0, 7, cols)
            assert np.array_equal(gq, q[r0:r0 + 7]), nm
            assert np.array_equal(gs, sc[r0:r0 + 7].view(np.uint16)), nm
    m.close()


def test_tiny_q8_0_parity(g):
    shape = synth.TINY
    prompt = synth.token_ids(2004, 40)
    ref, toks = oracle_greedy(shape, 1004, prompt, 8, scheme="q8_0")
    m = g.Model.from_shape(shape, seed=1004, scheme="q8_0", kv_pool_blocks=4, max_positions=64)
    s = g.Session(m, 64)
    got = gpu_teacher_forced(m, s, prompt, toks, shape.vocab)
    gate = Gate("tiny q8_0")
    for i, ((lg, am), r) in enumerate(zip(got, ref)):
        gate.check(i, lg, r, am)
    gate.assert_ok()
    s.close()
    m.close()


def test_affine4_codes_match_oracle(g):
    """AFFINE4_GS32 codes, scales and biases the library computes on the device equal the
    oracle's quantiser output, for rows of every projection kind (tiny shape)."""
    from oracle.affine4 import quantize_affine4
    shape = synth.TINY
    m = g.Model.from_shape(shape, seed=1001, scheme="affine4", kv_pool_blocks=2, max_positions=64)
    for l in range(shape.n_layers):
        for nm, dims in shape.layer_tensor_shapes().items():
            if nm in synth.NORM_TENSORS:
                continue
            rows, cols = dims
            w = synth.bf16_bits_to_f32(synth.tensor_bits(shape, 1001, nm, l))
            for r0 in (0, rows // 2 + 5, rows - 3):
                n = min(3, rows - r0)
                sc, bi, q = quantize_affine4(w[r0:r0 + n])
                gq, gs, gb = m.read_affine4(nm, l, r0, n, cols)
                assert np.array_equal(gq, q), (nm, l, r0)
                assert np.array_equal(gs, sc.view(np.uint16)) and np.array_equal(gb, bi.view(np.uint16)), (nm, l, r0)
    m.close()


def test_tiny_affine4_parity(g):
    """AFFINE4 tiny decoder against the oracle computing with the same dequantised weights: a
    16-token prompt (a round of few rows: matvec projections) and 16 teacher-forced decode steps,
    then a 100-token prompt in rounds of 48 (GEMMs over the FP16 dequantised copies, then a
    4-row matvec round) and 3 steps (gate: exact argmax, NMSE <= 1e-4)."""
    wl = synth.WORKLOADS["tiny"]
    shape = wl.shape
    prompt = synth.token_ids(wl.ids_seed, wl.prompt)
    say("tiny affine4 oracle")
    ref, toks = oracle_greedy(shape, wl.weight_seed, prompt, wl.decode, scheme="affine4")
    m = g.Model.from_shape(shape, seed=wl.weight_seed, scheme="affine4", kv_pool_blocks=8, max_positions=128,
                           max_round_tokens=48)
    s = g.Session(m, 128)
    got = gpu_teacher_forced(m, s, prompt, toks, shape.vocab)
    gate = Gate("tiny affine4")
    for i, ((lg, am), r) in enumerate(zip(got, ref)):
        gate.check(i, lg, r, am)
    long_prompt = synth.token_ids(61, 100)
    ref2, toks2 = oracle_greedy(shape, wl.weight_seed, long_prompt, 3, scheme="affine4")
    s2 = g.Session(m, 128)
    got2 = gpu_teacher_forced(m, s2, long_prompt, toks2, shape.vocab)
    for i, ((lg, am), r) in enumerate(zip(got2, ref2)):
        gate.check(100 + i, lg, r, am)
    gate.assert_ok()
    for o in (s, s2, m):
        o.close()


def test_affine4_batched_equals_isolated_bitwise(g):
    """AFFINE4 batched decode (7 rows: the staged split-K matvec) equals each row stepped alone
    (the whole-K matvec), bit for bit (Kipp Roadmap, status v0.0.2)."""
    shape = synth.TINY
    m = g.Model.from_shape(shape, seed=1001, scheme="affine4", kv_pool_blocks=64, max_positions=128)
    B = 7
    ss = [g.Session(m, 128) for _ in range(B)]
    twins = [g.Session(m, 128) for _ in range(B)]
    lg1 = torch.empty(shape.vocab, device="cuda")
    for b in range(B):
        p = synth.token_ids(70 + b, 5 + 3 * b)
        ss[b].prefill(p, lg1)
        twins[b].prefill(p, lg1)
    lg = torch.empty((B, shape.vocab), device="cuda")
    am = torch.empty(B, dtype=torch.int32, device="cuda")
    toks = [int(t) for t in synth.token_ids(80, B)]
    for step in range(3):
        m.eval_batch(ss, toks, lg, am)
        batched = lg.cpu().numpy()
        for b in range(B):
            twins[b].decode(toks[b], lg1)
            torch.cuda.synchronize()
            assert np.array_equal(batched[b], lg1.cpu().numpy()), (step, b)
        toks = [int(t) for t in am.cpu().numpy()]
    for o in ss + twins + [m]:
        o.close()


def test_qwen3_4b_affine4_reduced_depth_parity(g):
    """AFFINE4 at the 4B hidden sizes with 2 layers: a 300-token prompt (GEMMs over the FP16
    dequantised copies) and 3 teacher-forced decode steps (the whole-K matvec on the codes) over
    a shuffled paged KV, against the oracle (gate)."""
    wl = synth.WORKLOADS["4b-a4"]
    shape = synth.reduced(wl.shape, n_layers=2)
    prompt = synth.token_ids(wl.ids_seed, 300)
    say("4b affine4 depth-2 oracle")
    ref, toks = oracle_greedy(shape, wl.weight_seed, prompt, 3, scheme="affine4")
    nb = synth.blocks_for(len(prompt) + 4)
    m = g.Model.from_shape(shape, seed=wl.weight_seed, scheme="affine4", kv_pool_blocks=4 * nb,
                           max_positions=nb * 32)
    s = g.Session(m, nb * 32, block_ids=synth.shuffled_blocks(wl.shuffle_seed, 4 * nb)[:nb])
    got = gpu_teacher_forced(m, s, prompt, toks, shape.vocab)
    gate = Gate("4b affine4 depth 2")
    for i, ((lg, am), r) in enumerate(zip(got, ref)):
        gate.check(i, lg, r, am)
    gate.assert_ok()
    s.close()
    m.close()


@pytest.mark.parametrize("prefill", ["split", "fp16"])
def test_qwen3_0_6b_shape_parity(g, prefill):
    """0.6B shape: 28 layers, 348-token prompt, 64 teacher-forced greedy steps, paged KV with a
    shuffled block table drawn from a pool four times the session's size; prefill products with
    FP16 hi/lo activations (split) and with single FP16 activations (fp16)."""
    wl = synth.WORKLOADS["0.6b"]
    shape = wl.shape
    prompt = synth.token_ids(wl.ids_seed, wl.prompt)
    say("0.6b oracle")
    ref, toks = oracle_greedy_cached("0.6b", shape, wl.weight_seed, prompt, wl.decode)
    nb = synth.blocks_for(wl.prompt + wl.decode)
    table = synth.shuffled_blocks(wl.shuffle_seed, 4 * nb)[:nb]
    say("0.6b gpu", prefill)
    m = g.Model.from_shape(shape, seed=wl.weight_seed, kv_pool_blocks=4 * nb, max_positions=nb * 32,
                           prefill=prefill)
    s = g.Session(m, nb * 32, block_ids=table)
    got = gpu_teacher_forced(m, s, prompt, toks, shape.vocab)
    gate = Gate("0.6b " + prefill)
    for i, ((lg, am), r) in enumerate(zip(got, ref)):
        gate.check(i, lg, r, am)
    gate.assert_ok()
    s.close()
    m.close()


@pytest.mark.parametrize("prefill", ["split", "fp16"])
def test_qwen3_4b_shape_parity(g, prefill):
    """Qwen3-4B shape at its full prompt: 36 layers, hidden 2560, 32 Q / 8 KV heads, FFN 9728,
    the 2,048-token prompt prefilled in one round (the launch configuration bench.py times), then
    all 64 teacher-forced greedy decode steps over a shuffled paged KV; full-logit NMSE and exact
    argmax against the oracle at every position."""
    wl = synth.WORKLOADS["4b"]
    shape = wl.shape
    steps = wl.decode
    prompt = synth.token_ids(wl.ids_seed, wl.prompt)
    say("4b oracle (2048-token prefill, %d steps)" % steps)
    ref, toks = oracle_greedy_cached("4b", shape, wl.weight_seed, prompt, steps)
    nb = synth.blocks_for(wl.prompt + wl.decode)
    table = synth.shuffled_blocks(wl.shuffle_seed, 4 * nb)[:nb]
    say("4b gpu", prefill)
    m = g.Model.from_shape(shape, seed=wl.weight_seed, kv_pool_blocks=4 * nb, max_positions=nb * 32,
                           prefill=prefill)
    assert m.info().round_tokens >= wl.prompt
    s = g.Session(m, nb * 32, block_ids=table)
    got = gpu_teacher_forced(m, s, prompt, toks, shape.vocab)
    gate = Gate("4b " + prefill)
    for i, ((lg, am), r) in enumerate(zip(got, ref)):
        gate.check(i, lg, r, am)
    gate.assert_ok()
    s.close()
    m.close()


def _bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("q8_prefill", ["copy", "direct"])
def test_qwen3_4b_q8_0_reduced_depth_parity(g, q8_prefill):
    """Q8_0 at the 4B hidden sizes (hidden 2560, 32/8 heads, FFN 9728, tied vocab) with 4 layers,
    a 1,500-token prompt evaluated in rounds of 512 (two full rounds and a ragged one, so the
    attention of later rounds starts at pos0 > 0), then 3 teacher-forced decode steps over a
    shuffled paged KV: full-logit NMSE and exact argmax against the oracle, which dequantises
    the same Q8_0 bytes. Prefill GEMMs over the FP16 dequantised copies ("copy") or over the
    quants and scales directly ("direct")."""
    wl = synth.WORKLOADS["4b-q8"]
    shape = synth.reduced(wl.shape, n_layers=4)
    prompt = synth.token_ids(wl.ids_seed, 1500)
    steps = 3
    say("4b-q8 depth-4 oracle (1500-token prefill, %d steps)" % steps)
    ref, toks = oracle_greedy(shape, wl.weight_seed, prompt, steps, scheme="q8_0")
    nb = synth.blocks_for(len(prompt) + steps)
    table = synth.shuffled_blocks(wl.shuffle_seed, 4 * nb)[:nb]
    m = g.Model.from_shape(shape, seed=wl.weight_seed, scheme="q8_0", kv_pool_blocks=4 * nb,
                           max_positions=nb * 32, max_round_tokens=512, q8_prefill=q8_prefill)
    s = g.Session(m, nb * 32, block_ids=table)
    got = gpu_teacher_forced(m, s, prompt, toks, shape.vocab)
    gate = Gate("4b q8_0 depth 4 " + q8_prefill)
    for i, ((lg, am), r) in enumerate(zip(got, ref)):
        gate.check(i, lg, r, am)
    gate.assert_ok()
    s.close()
    m.close()


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
_REF_LOGITS = {}


def stored_oracle_ref(fname):
    """A stored oracle reference written by tests/golden/make_oracle_refs.py (oracle residual
    rows after the last layer, and the oracle's greedy tokens), as a dict of arrays."""
    path = os.path.join(GOLDEN, fname)
    if not os.path.exists(path):
        pytest.skip(f"stored oracle reference {fname} not generated (python tests/golden/make_oracle_refs.py)")
    z = np.load(path, allow_pickle=False)
    return {k: z[k] for k in z.files}


def stored_oracle_logits(fname, shape, seed, scheme):
    """Full-vocabulary oracle logits of every stored residual row: the oracle's own final norm
    and lm_head (oracle.final_logits) applied to the stored rows; cached per file."""
    if fname not in _REF_LOGITS:
        ref = stored_oracle_ref(fname)
        assert str(ref["shape"]) == shape.name and int(ref["weight_seed"]) == seed and str(ref["scheme"]) == scheme
        om_ = oracle.OracleModel(shape, seed, scheme)
        x = ref["x"]
        lg = oracle.final_logits(om_, x.reshape(-1, shape.hidden)).reshape(x.shape[:-1] + (shape.vocab,))
        _REF_LOGITS[fname] = (ref, lg)
    return _REF_LOGITS[fname]


def _ids_sha(ids):
    return hashlib.sha256(np.asarray(ids, dtype=np.int32).tobytes()).hexdigest()


@pytest.mark.parametrize("q8_prefill", ["copy", "direct"])
def test_qwen3_4b_q8_0_full_parity(g, q8_prefill):
    """The Q8_0 4B workload at full size against the oracle: 36 layers with the seven projections
    in Q8_0, the 12,800-token prompt prefilled in the device's rounds over a shuffled paged KV
    (pool four times the session's need), then all 32 teacher-forced greedy decode steps;
    full-logit NMSE and exact argmax at the prefill row and every decode position. The oracle's
    run (tens of CPU minutes) is stored by tests/golden/make_oracle_refs.py as residual rows,
    turned into logits here by the oracle's final norm and lm_head. Prefill GEMMs over the FP16
    dequantised copies ("copy", the benchmark's setting) or the quants and scales ("direct").
    The "copy" run also checks the last layer's attention output at the last prompt position
    (all 32 heads) against an FP64 softmax(q K^T / sqrt(128)) V over all 12,800 positions,
    computed on the host from the read-back rotated q and BF16 K/V."""
    wl = synth.WORKLOADS["4b-q8"]
    shape = wl.shape
    T = wl.prompt
    say("4b-q8 stored oracle logits")
    ref, ref_lg = stored_oracle_logits("oracle_ref_4b_q8_0.npz", shape, wl.weight_seed, "q8_0")
    prompt = synth.token_ids(wl.ids_seed, T)
    assert str(ref["prompt_sha"]) == _ids_sha(prompt) and int(ref["steps"]) == wl.decode
    toks = [int(t) for t in ref["toks"]]
    nb = synth.blocks_for(T + wl.decode + 1)
    table = synth.shuffled_blocks(wl.shuffle_seed, 4 * nb)[:nb]
    say("4b-q8 gpu (12800-token prompt, %d steps), prefill %s" % (wl.decode, q8_prefill))
    m = g.Model.from_shape(shape, seed=wl.weight_seed, scheme="q8_0", kv_pool_blocks=4 * nb,
                           max_positions=nb * 32, q8_prefill=q8_prefill)
    R = m.info().round_tokens
    assert T > R
    s = g.Session(m, nb * 32, block_ids=table)
    lg = torch.empty(shape.vocab, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    s.prefill(prompt, lg, am)
    torch.cuda.synchronize()
    got = [(lg.cpu().numpy(), int(am.item()))]

    if q8_prefill == "copy":
        # the prefill evaluates the last layer's attention for the last row only and stores it
        # as row 0 of the operand rows (times 16)
        nq, G = shape.n_q_heads, shape.n_q_heads // 8
        last0 = ((T - 1) // R) * R
        Tl = T - last0
        q = m.read_scratch("qrot", (Tl - 1) * nq * 128, nq * 128).reshape(nq, 128).astype(np.float64)
        o_hi = m.read_scratch("attn_hi", 0, nq * 128).astype(np.float64)
        o_lo = m.read_scratch("attn_lo", 0, nq * 128).astype(np.float64)
        o_gpu = ((o_hi + o_lo) / 16.0).reshape(nq, 128)
        kb, vb = s.read_kv(shape.n_layers - 1, 0, T)
        worst = 0.0
        for h in range(nq):
            kf = _bf16_to_f64(kb[:, h // G])
            vf = _bf16_to_f64(vb[:, h // G])
            sc = kf @ q[h] / np.sqrt(128.0)
            w = np.exp(sc - sc.max())
            ref_o = (w @ vf) / w.sum()
            worst = max(worst, float(np.sum((o_gpu[h] - ref_o) ** 2) / np.sum(ref_o ** 2)))
        say("4b-q8 attention of position %d over %d keys, 32 heads: worst NMSE %.3e" % (T - 1, T, worst))
        assert worst <= 1e-9

    for t in toks:
        s.decode(t, lg, am)
        torch.cuda.synchronize()
        got.append((lg.cpu().numpy(), int(am.item())))
    gate = Gate("4b q8_0 12800 + 32 steps " + q8_prefill)
    for i, (l, a) in enumerate(got):
        gate.check(i, l, ref_lg[i], a)
        assert a == om.argmax(l)
    gate.assert_ok()
    s.close()
    m.close()


def test_decode_across_chunk_length_change(g):
    """Decode attention cuts a context into chunks whose length grows with the context (64
    positions up to 4,096, then 128, ...). Tiny shape, a 4,094-token prompt over shuffled blocks,
    then five greedy decode steps at contexts 4,095 .. 4,099 -- across the change at 4,097: each
    step's logits equal those of prefilling the same tokens in a fresh session (matvec and split
    attention vs GEMM and flash attention) within NMSE 1e-5, same argmax unless the top-2
    margin is a near tie."""
    wl = synth.WORKLOADS["tiny"]
    shape = wl.shape
    T, steps = 4094, 5
    nb = synth.blocks_for(T + steps + 1)
    table = synth.shuffled_blocks(wl.shuffle_seed, 2 * nb)[:nb]
    m = g.Model.from_shape(shape, seed=wl.weight_seed, kv_pool_blocks=4 * nb, max_positions=nb * 32)
    s = g.Session(m, nb * 32, block_ids=table)
    prompt = synth.token_ids(wl.ids_seed, T)
    lg = torch.empty(shape.vocab, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    s.prefill(prompt, lg, am)
    torch.cuda.synchronize()
    seq = list(prompt)
    gate = Gate("tiny decode across the chunk-length change")
    lg2 = torch.empty(shape.vocab, device="cuda")
    for i in range(steps):
        tok = int(am.item())
        seq.append(tok)
        s.decode(tok, lg, am)
        torch.cuda.synchronize()
        s2 = g.Session(m, nb * 32)
        s2.prefill(np.array(seq, dtype=prompt.dtype), lg2)
        torch.cuda.synchronize()
        gate.check(len(seq) - 1, lg.cpu().numpy(), lg2.cpu().numpy(), int(am.item()))
        s2.close()
    w = gate.assert_ok()
    assert w <= 1e-5
    s.close()
    m.close()


def _rows(sess, ids, vocab):
    lg = torch.empty((len(ids), vocab), device="cuda")
    am = torch.empty(len(ids), dtype=torch.int32, device="cuda")
    sess.eval_n(ids, lg, am)
    torch.cuda.synchronize()
    return lg.cpu().numpy(), am.cpu().numpy()


def _scores(sess, ids):
    sc = torch.empty(len(ids) - 1, device="cuda")
    sess.eval_scored(ids, sc)
    torch.cuda.synchronize()
    return sc.cpu().numpy().astype(np.float64)


# Scores are log-probabilities taken in FP32 from FP32 logits. If every logit of a row is off
# by at most e, the row's score is off by at most 2e (the target's logit and the log-sum-exp
# each move by at most e); the FP32 log-softmax itself is held to 1e-4 against a float64 one of
# the same logits. So a row's score may differ from the oracle's by 2e + 1e-4, with e that
# row's largest logit error (the logits themselves pass the gate).
SCORE_FP32_TOL = 1e-4


def test_eval_n_every_row_parity(g):
    """Multi-row evaluation (Kipp Roadmap, status v0.0.2): the tiny decoder in rounds of 48, a
    100-token call (48 + 48 + 4 rows, every row of every round returned) and then a 37-token call
    (lm_head over row groups of 32 + 5); every row against the oracle's logits of the same
    positions (identical argmax, NMSE <= 1e-4), the device argmax equal to the host argmax, and
    the last row equal to what eval_prefill writes for the same call."""
    wl = synth.WORKLOADS["tiny"]
    shape = wl.shape
    ids = synth.token_ids(31, 137)
    say("eval_n tiny oracle")
    ref = oracle.OracleSession(oracle.OracleModel(shape, wl.weight_seed),
                               oracle.ContiguousKV.for_shape(shape, 160)).forward(ids, all_logits=True)
    m = g.Model.from_shape(shape, seed=wl.weight_seed, kv_pool_blocks=12, max_positions=160, max_round_tokens=48)
    s = g.Session(m, 160)
    a_lg, a_am = _rows(s, ids[:100], shape.vocab)
    b_lg, b_am = _rows(s, ids[100:], shape.vocab)
    assert s.position == 137
    lg, am = np.concatenate([a_lg, b_lg]), np.concatenate([a_am, b_am])
    gate = Gate("eval_n tiny")
    for i in range(137):
        gate.check(i, lg[i], ref[i], int(am[i]))
        assert am[i] == int(np.argmax(lg[i]))
    gate.assert_ok()
    s2 = g.Session(m, 160)
    last = torch.empty(shape.vocab, device="cuda")
    s2.prefill(ids[:100], last)
    torch.cuda.synchronize()
    assert nmse(a_lg[-1], last.cpu().numpy()) <= 1e-8
    for o in (s, s2, m):
        o.close()


def test_eval_scored_parity(g):
    """Multi-row scoring (Kipp Roadmap, status v0.0.3): 70 ids in rounds of 48 give 69 scores,
    each the log-probability of the next id; against the log-softmax (in float64) of the
    library's own eval_n logits within SCORE_FP32_TOL (which isolates the scoring kernel), and
    against the oracle within 2e + SCORE_FP32_TOL, e being the largest logit error. Fewer than
    two ids is an error."""
    wl = synth.WORKLOADS["tiny"]
    shape = wl.shape
    ids = synth.token_ids(33, 70)
    say("eval_scored tiny")
    om_ = oracle.OracleModel(shape, wl.weight_seed)
    ref_rows = oracle.OracleSession(om_, oracle.ContiguousKV.for_shape(shape, 96)).forward(ids, all_logits=True)
    ref = om.next_token_log_probs(ref_rows[:-1], ids[1:])
    m = g.Model.from_shape(shape, seed=wl.weight_seed, kv_pool_blocks=8, max_positions=96, max_round_tokens=48)
    s = g.Session(m, 96)
    got = _scores(s, ids)
    assert s.position == 70 and got.shape == (69,)
    s2 = g.Session(m, 96)
    lg, _ = _rows(s2, ids, shape.vocab)
    own = np.max(np.abs(got - om.next_token_log_probs(lg[:-1], ids[1:])))
    e = np.max(np.abs(lg[:-1].astype(np.float64) - ref_rows[:-1]))
    d = np.max(np.abs(got - ref))
    say("score |diff| vs oracle %.3g, vs own logits %.3g, largest logit error %.3g" % (d, own, e))
    assert own <= SCORE_FP32_TOL
    assert d <= 2 * e + SCORE_FP32_TOL
    with pytest.raises(g.GqaError):
        s2.eval_scored(ids[:1], torch.empty(1, device="cuda"))
    for o in (s, s2, m):
        o.close()


def test_multi_row_edges(g):
    """Edges of multi-row evaluation (tiny decoder, rounds of 48): n = 1, 32 (the largest matvec
    round), 33 (the smallest GEMM round, lm_head over the padded vocabulary) and 48 (a full
    round) rows of eval_n against the oracle; eval_scored with n = 2 (one score); eval_n on a
    pooled session; a session filled to its last position, after which one more token is a
    context overflow that leaves the position unchanged."""
    wl = synth.WORKLOADS["tiny"]
    shape = wl.shape
    m = g.Model.from_shape(shape, seed=wl.weight_seed, kv_pool_blocks=32, max_positions=256, max_round_tokens=48)
    om_ = oracle.OracleModel(shape, wl.weight_seed)
    gate = Gate("multi-row edges")
    k = 0
    for n in (1, 32, 33, 48):
        ids = synth.token_ids(90 + n, n)
        ref = oracle.OracleSession(om_, oracle.ContiguousKV.for_shape(shape, 64)).forward(ids, all_logits=True)
        s = g.Session(m, 64)
        lg, am = _rows(s, ids, shape.vocab)
        for i in range(n):
            gate.check(k, lg[i], ref[i], int(am[i]))
            assert am[i] == int(np.argmax(lg[i]))
            k += 1
        s.close()
    ids = synth.token_ids(95, 2)
    s = g.Session(m, 64)
    sc = _scores(s, ids)
    r = oracle.OracleSession(om_, oracle.ContiguousKV.for_shape(shape, 8)).score(ids)
    assert sc.shape == (1,) and abs(sc[0] - r[0]) < 2e-2
    s.close()
    ids = synth.token_ids(96, 40)
    ref = oracle.OracleSession(om_, oracle.ContiguousKV.for_shape(shape, 64)).forward(ids, all_logits=True)
    ps = g.Session(m, 64, pooled=True)
    lg, am = _rows(ps, ids, shape.vocab)
    for i in range(40):
        gate.check(k, lg[i], ref[i], int(am[i]))
        k += 1
    ps.close()
    gate.assert_ok()
    full = g.Session(m, 40)
    _prefill(full, synth.token_ids(97, 40), shape.vocab)
    assert full.position == 40
    with pytest.raises(g.GqaError):
        full.decode(5, torch.empty(shape.vocab, device="cuda"))
    with pytest.raises(g.GqaError):
        full.eval_n([1, 2], torch.empty((2, shape.vocab), device="cuda"))
    assert full.position == 40
    full.close()
    m.close()


def test_short_round_after_long_context(g):
    """A round of few rows over a long context splits its keys over several workgroups per KV
    head and merges the partials: the tiny decoder prefills 2,000 ids, then evaluates 10 more
    (eval_n: 2,010 keys, 8 key splits) and 1 more through eval_prefill; every row against the
    oracle's logits of the same positions (gate)."""
    wl = synth.WORKLOADS["tiny"]
    shape = wl.shape
    ids = synth.token_ids(98, 2011)
    say("short round oracle")
    ref = oracle.OracleSession(oracle.OracleModel(shape, wl.weight_seed),
                               oracle.ContiguousKV.for_shape(shape, 2048)).forward(ids, all_logits=True)
    nb = synth.blocks_for(2048)
    m = g.Model.from_shape(shape, seed=wl.weight_seed, kv_pool_blocks=2 * nb, max_positions=nb * 32)
    s = g.Session(m, nb * 32, block_ids=synth.shuffled_blocks(99, 2 * nb)[:nb])
    _prefill(s, ids[:2000], shape.vocab)
    lg, am = _rows(s, ids[2000:2010], shape.vocab)
    last, last_am = _prefill(s, ids[2010:], shape.vocab)
    gate = Gate("short round after a long context")
    for i in range(10):
        gate.check(2000 + i, lg[i], ref[2000 + i], int(am[i]))
    gate.check(2010, last, ref[2010], last_am)
    gate.assert_ok()
    s.close()
    m.close()


def test_truncate_resume_parity(g):
    """Truncate/resume (Kipp Model Support, "What the gates check"): prefill 40 ids, evaluate 20
    more, truncate back to 40, then evaluate 11 new ids (all rows) and 3 greedy decode steps over
    shuffled blocks: every position against the oracle evaluating the kept 40 plus the new ids
    from scratch. Truncating past the position is an error; truncating to 0 restarts the
    session."""
    wl = synth.WORKLOADS["tiny"]
    shape = wl.shape
    a, b, c = synth.token_ids(41, 40), synth.token_ids(42, 20), synth.token_ids(43, 11)
    say("truncate tiny oracle")
    osess = oracle.OracleSession(oracle.OracleModel(shape, wl.weight_seed), oracle.ContiguousKV.for_shape(shape, 96))
    ref_rows = osess.forward(np.concatenate([a, c]), all_logits=True)[len(a):]
    m = g.Model.from_shape(shape, seed=wl.weight_seed, kv_pool_blocks=16, max_positions=96)
    s = g.Session(m, 96, block_ids=synth.shuffled_blocks(44, 16)[:3])
    lg = torch.empty(shape.vocab, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    s.prefill(a, lg)
    s.eval_n(b, torch.empty((len(b), shape.vocab), device="cuda"))
    s.truncate(len(a))
    assert s.position == len(a)
    rows, row_am = _rows(s, c, shape.vocab)
    gate = Gate("truncate/resume")
    for i in range(len(c)):
        gate.check(len(a) + i, rows[i], ref_rows[i], int(row_am[i]))
    tok = int(row_am[-1])
    for step in range(3):
        want = osess.decode(tok)
        s.decode(tok, lg, am)
        torch.cuda.synchronize()
        gate.check(len(a) + len(c) + step, lg.cpu().numpy(), want, int(am.item()))
        tok = int(am.item())
    gate.assert_ok()
    with pytest.raises(g.GqaError):
        s.truncate(s.position + 1)
    s.truncate(0)
    s.prefill(a, lg)
    torch.cuda.synchronize()
    ref0 = oracle_greedy(shape, wl.weight_seed, a, 0)[0][0]
    g1 = Gate("truncate to 0")
    g1.check(0, lg.cpu().numpy(), ref0)
    g1.assert_ok()
    s.close()
    m.close()


def _prefill(sess, ids, vocab):
    lg = torch.empty(vocab, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    sess.prefill(ids, lg, am)
    torch.cuda.synchronize()
    return lg.cpu().numpy(), int(am.item())


def _oracle_last(shape, seed, ids):
    return oracle.OracleSession(oracle.OracleModel(shape, seed),
                                oracle.ContiguousKV.for_shape(shape, len(ids) + 1)).forward(ids)


def test_pooled_prefix_reuse_parity(g):
    """Content-addressed prefix blocks (Kipp Roadmap, status v0.0.3), tiny decoder. A pooled
    session prefills a 200-id prompt P and ends (publishing its 6 whole blocks); a second maps
    them and evaluates only the last 8 ids; a third shares P's first 100 ids (3 blocks reused);
    a 192-id prompt reuses 5 blocks (one id is always evaluated); a session truncated into a
    shared block writes a private copy, after which P still hits its intact blocks; greedy
    decode after a reused prefix. Every logit vector against the oracle evaluating the whole
    prompt from scratch (gate)."""
    wl = synth.WORKLOADS["tiny"]
    shape, seed = wl.shape, wl.weight_seed
    P = synth.token_ids(51, 200)
    other = synth.token_ids(52, 60)
    m = g.Model.from_shape(shape, seed=seed, kv_pool_blocks=64, max_positions=512)
    gate = Gate("pooled prefix reuse")
    say("pooled: cold prompt")
    a = g.Session(m, 512, pooled=True)
    la, _ = _prefill(a, P, shape.vocab)
    assert a.reused == 0
    ref_p = _oracle_last(shape, seed, P)
    gate.check(0, la, ref_p)
    a.close()
    assert m.info().cached_blocks == 6
    assert m.info().prefix_lookups == 1 and m.info().prefix_hits == 0     # the cold prompt's first block
    say("pooled: warm prompt")
    b = g.Session(m, 512, pooled=True)
    lb, amb = _prefill(b, P, shape.vocab)
    assert b.reused == 192
    assert m.info().prefix_hits == 6
    gate.check(1, lb, ref_p, amb)
    assert nmse(lb, la) <= 1e-8
    # greedy decode after the reused prefix, teacher-forced with the oracle's tokens
    osess = oracle.OracleSession(oracle.OracleModel(shape, seed), oracle.ContiguousKV.for_shape(shape, 256))
    r = osess.forward(P)
    lg = torch.empty(shape.vocab, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    for step in range(3):
        t = om.argmax(r)
        r = osess.decode(t)
        b.decode(t, lg, am)
        torch.cuda.synchronize()
        gate.check(2 + step, lg.cpu().numpy(), r, int(am.item()))
    say("pooled: shared first 100 ids")
    Q = np.concatenate([P[:100], other])
    c = g.Session(m, 512, pooled=True)
    lc, amc = _prefill(c, Q, shape.vocab)
    assert c.reused == 96
    gate.check(5, lc, _oracle_last(shape, seed, Q), amc)
    d = g.Session(m, 512, pooled=True)
    ld, amd = _prefill(d, P[:192], shape.vocab)
    assert d.reused == 160
    gate.check(6, ld, _oracle_last(shape, seed, P[:192]), amd)
    say("pooled: truncate into a shared block, copy on write")
    b.truncate(100)
    lt, amt = _prefill(b, other[:20], shape.vocab)
    gate.check(7, lt, _oracle_last(shape, seed, np.concatenate([P[:100], other[:20]])), amt)
    e = g.Session(m, 512, pooled=True)
    le, ame = _prefill(e, P, shape.vocab)
    assert e.reused == 192
    gate.check(8, le, ref_p, ame)
    gate.assert_ok()
    for o in (b, c, d, e, m):
        o.close()


def test_pooled_eviction_and_exhaustion(g):
    """A 16-block pool: a 150-id prompt X publishes 4 blocks; a 400-id prompt Y needs 13 blocks,
    so the least recently used of X's blocks (its first) is evicted, which breaks X's chain: X
    again reuses nothing and is still right. With every block held by fixed-table sessions, a
    pooled prefill fails with GQA_E_OOM and leaves the session at position 0."""
    wl = synth.WORKLOADS["tiny"]
    shape, seed = wl.shape, wl.weight_seed
    X, Y = synth.token_ids(53, 150), synth.token_ids(54, 400)
    m = g.Model.from_shape(shape, seed=seed, kv_pool_blocks=16, max_positions=512)
    gate = Gate("pooled eviction")
    s1 = g.Session(m, 512, pooled=True)
    gate.check(0, _prefill(s1, X, shape.vocab)[0], _oracle_last(shape, seed, X))
    s1.close()
    assert m.info().cached_blocks == 4 and m.info().free_blocks == 16
    s2 = g.Session(m, 512, pooled=True)
    l2, a2 = _prefill(s2, Y, shape.vocab)
    gate.check(1, l2, _oracle_last(shape, seed, Y), a2)
    s2.close()
    s3 = g.Session(m, 512, pooled=True)
    l3, a3 = _prefill(s3, X, shape.vocab)
    assert s3.reused == 0
    gate.check(2, l3, _oracle_last(shape, seed, X), a3)
    s3.close()
    gate.assert_ok()
    fixed = [g.Session(m, 32 * 8), g.Session(m, 32 * 8)]          # all 16 blocks (cached ones evicted)
    assert m.info().free_blocks == 0 and m.info().cached_blocks == 0
    s4 = g.Session(m, 512, pooled=True)
    with pytest.raises(g.GqaError):
        s4.prefill(X, torch.empty(shape.vocab, device="cuda"))
    assert s4.position == 0
    for o in fixed + [s4, m]:
        o.close()


def test_pooled_batched_decode(g):
    """Pooled sessions in batched decode: three sessions share a 70-id prefix (the last two
    reuse its 2 blocks), then 40 batched greedy steps cross block boundaries, so blocks are
    mapped on demand inside eval_batch; each row against the oracle (gate, teacher-forced)."""
    wl = synth.WORKLOADS["tiny"]
    shape, seed = wl.shape, wl.weight_seed
    pre = synth.token_ids(55, 70)
    tails = [synth.token_ids(56 + i, 5 + 7 * i) for i in range(3)]
    m = g.Model.from_shape(shape, seed=seed, kv_pool_blocks=64, max_positions=256)
    ss, ors, refs = [], [], []
    for i in range(3):
        ids = np.concatenate([pre, tails[i]])
        s = g.Session(m, 256, pooled=True)
        _prefill(s, ids, shape.vocab)
        if i:
            assert s.reused == 64
        s.publish()
        ss.append(s)
        o = oracle.OracleSession(oracle.OracleModel(shape, seed), oracle.ContiguousKV.for_shape(shape, 256))
        refs.append(o.forward(ids))
        ors.append(o)
    gate = Gate("pooled batched")
    lg = torch.empty((3, shape.vocab), device="cuda")
    am = torch.empty(3, dtype=torch.int32, device="cuda")
    for step in range(40):
        toks = [om.argmax(r) for r in refs]
        m.eval_batch(ss, toks, lg, am)
        torch.cuda.synchronize()
        got, ga = lg.cpu().numpy(), am.cpu().numpy()
        refs = [o.decode(t) for o, t in zip(ors, toks)]
        for i in range(3):
            gate.check(step * 3 + i, got[i], refs[i], int(ga[i]))
    gate.assert_ok()
    for o in ss + [m]:
        o.close()


def test_qwen3_4b_eval_n_and_scores_full_prompt(g):
    """Qwen3-4B shape at its full 2,048-token prompt in one round (the launch configuration
    bench.py times): eval_n returns every row (lm_head over 64 groups of 32 rows); all 2,048
    rows against the oracle's logits of the same positions (NMSE <= 1e-4; identical argmax,
    device argmax included, unless the gate's near-tie rule applies), and each of eval_scored's
    2,047 scores within 2e + SCORE_FP32_TOL of the oracle's, e being that row's largest logit
    error."""
    wl = synth.WORKLOADS["4b"]
    shape = wl.shape
    prompt = synth.token_ids(wl.ids_seed, wl.prompt)
    say("4b oracle rows")
    oracle_greedy_cached("4b", shape, wl.weight_seed, prompt, wl.decode)
    ref = oracle_prompt_rows("4b")
    nb = synth.blocks_for(wl.prompt + 1)
    m = g.Model.from_shape(shape, seed=wl.weight_seed, kv_pool_blocks=2 * nb, max_positions=nb * 32)
    s = g.Session(m, nb * 32, block_ids=synth.shuffled_blocks(wl.shuffle_seed, 2 * nb)[:nb])
    say("4b eval_n")
    lg = torch.empty((wl.prompt, shape.vocab), device="cuda")
    am = torch.empty(wl.prompt, dtype=torch.int32, device="cuda")
    s.eval_n(prompt, lg, am)
    torch.cuda.synchronize()
    am = am.cpu().numpy()
    lg = lg.cpu().numpy()
    gate = Gate("4b eval_n rows")
    err = np.empty(wl.prompt)
    for i in range(wl.prompt):
        gate.check(i, lg[i], ref[i], int(am[i]))
        err[i] = np.max(np.abs(lg[i].astype(np.float64) - ref[i]))
    gate.assert_ok()
    say("4b rows: largest logit error %.3g (median row %.3g)" % (err.max(), np.median(err)))
    e = np.array([r["nmse"] for r in gate.rows])
    for lo, hi in ((0, 1), (1, 4), (4, 16), (16, 64), (64, 256), (256, 1024), (1024, 2048)):
        say("4b rows at positions [%d, %d): median NMSE %.3e, worst %.3e" % (lo, hi, np.median(e[lo:hi]), e[lo:hi].max()))
    del lg
    s.reset()
    say("4b eval_scored")
    got = _scores(s, prompt)
    want = om.next_token_log_probs(ref[:-1], prompt[1:])
    d = np.abs(got - want)
    say("4b score largest |diff| %.3g" % d.max())
    assert np.all(d <= 2 * err[:-1] + SCORE_FP32_TOL)
    s.close()
    m.close()


def test_qwen3_8b_batched_32_sessions(g):
    """The 8B batched workload at full size: 36 layers, hidden 4096, untied lm_head, 32 sessions
    with contexts L_i ~ U{512..8192} (seed 4005), each prefilled alone over its own blocks, then
    all 128 batched decode steps (B = 32).
    (1) Oracle parity for the declared subset -- the shortest and the longest context and
        sessions 0 and 16 -- at the prefill row and all 128 steps, teacher-forced with the
        oracle's greedy tokens (full-logit NMSE, exact argmax; the oracle's run is stored by
        tests/golden/make_oracle_refs.py). The other rows follow their own device argmax.
    (2) Batched equals isolated bit for bit: every row of every batched step equals a twin
        session fed the same ids alone (logits and argmax), all 32 rows x 128 steps."""
    wl = synth.WORKLOADS["8b-batch"]
    shape = wl.shape
    lens = [int(x) for x in synth.context_lengths(synth.CONTEXT_SEED_8B, wl.n_seqs)]
    steps = wl.decode
    say("8b batch: stored oracle logits")
    ref, ref_lg = stored_oracle_logits("oracle_ref_8b_batch.npz", shape, wl.weight_seed, "bf16")
    sub = [int(i) for i in ref["sessions"]]
    assert [int(c) for c in ref["contexts"]] == [lens[i] for i in sub] and int(ref["steps"]) == steps
    assert sub[0] == int(np.argmin(lens)) and sub[1] == int(np.argmax(lens))
    rtoks = ref["toks"]
    need = sum(synth.blocks_for(n + steps) for n in lens)
    say("8b batch: contexts", min(lens), "..", max(lens), "total", sum(lens), "subset", sub)
    m = g.Model.from_shape(shape, seed=wl.weight_seed, kv_pool_blocks=2 * need + 64,
                           max_positions=8192 + steps + 64)
    V, B = shape.vocab, len(lens)
    lg = torch.empty(V, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    gates = {i: Gate("8b batch session %d (context %d)" % (i, lens[i])) for i in sub}
    A, Bs, nxt = [], [], []
    for i, n in enumerate(lens):
        p = synth.token_ids(wl.ids_seed, n, offset=i * 8192)
        if i in gates:
            assert str(ref["prompt_sha"][sub.index(i)]) == _ids_sha(p)
        a, b = g.Session(m, n + steps), g.Session(m, n + steps)
        a.prefill(p, lg, am)
        torch.cuda.synchronize()
        if i in gates:
            gates[i].check(0, lg.cpu().numpy(), ref_lg[sub.index(i)][0], int(am.item()))
        nxt.append(int(am.item()))
        b.prefill(p, lg)
        A.append(a)
        Bs.append(b)
    torch.cuda.synchronize()
    say("8b batch: prefilled 2 x 32 sessions")
    hist = torch.empty((steps, B, V), device="cuda")
    hist_am = torch.empty((steps, B), dtype=torch.int32, device="cuda")
    ids = np.empty((steps, B), dtype=np.int32)
    for step in range(steps):
        for k, i in enumerate(sub):
            nxt[i] = int(rtoks[k][step])
        ids[step] = nxt
        m.eval_batch(A, nxt, hist[step], hist_am[step])
        torch.cuda.synchronize()
        bam_h = hist_am[step].cpu().numpy()
        for k, i in enumerate(sub):
            gates[i].check(step + 1, hist[step, i].cpu().numpy(), ref_lg[k][step + 1], int(bam_h[i]))
        nxt = [int(x) for x in bam_h]
    say("8b batch: %d batched steps done" % steps)
    assert bool(torch.isfinite(hist).all())
    for gt in gates.values():
        gt.assert_ok()
    bad = torch.zeros(B, dtype=torch.int64, device="cuda")
    bad_am = torch.zeros(B, dtype=torch.int64, device="cuda")
    for i, sb in enumerate(Bs):
        for step in range(steps):
            sb.decode(int(ids[step, i]), lg, am)
            bad[i] += (lg.view(torch.int32) != hist[step, i].view(torch.int32)).sum()
            bad_am[i] += (am[0] != hist_am[step, i]).to(torch.int64)
    torch.cuda.synchronize()
    say("8b batch: isolated twins stepped; differing logit words per row:", bad.cpu().tolist())
    assert int(bad.sum()) == 0 and int(bad_am.sum()) == 0
    del hist
    for o in A + Bs + [m]:
        o.close()


def test_qwen3_8b_batched_row_reduced_depth_parity(g):
    """A batched row against the oracle at the 8B hidden sizes (hidden 4096, 32/8 heads, FFN
    12288, untied lm_head) with 4 layers: 8 sessions with contexts 512..1400 are prefilled alone,
    then 3 batched steps (B = 8, the split-K row path) teacher-force session 0 with the oracle's
    tokens; its prefill and batched logits match the oracle (NMSE, exact argmax)."""
    wl = synth.WORKLOADS["8b-batch"]
    shape = synth.reduced(wl.shape, n_layers=4)
    lens = [600, 512, 1400, 777, 1024, 900, 513, 1100]
    steps = 3
    p0 = synth.token_ids(wl.ids_seed, lens[0])
    say("8b depth-4 oracle (%d-token prefill, %d steps)" % (lens[0], steps))
    ref, toks = oracle_greedy(shape, wl.weight_seed, p0, steps)
    need = sum(synth.blocks_for(n + steps) for n in lens)
    m = g.Model.from_shape(shape, seed=wl.weight_seed, kv_pool_blocks=need + 16, max_positions=2048)
    lg = torch.empty(shape.vocab, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    sess, nxt = [], []
    gate = Gate("8b depth 4, batched row 0")
    for i, n in enumerate(lens):
        p = p0 if i == 0 else synth.token_ids(wl.ids_seed, n, offset=i * 8192)
        s = g.Session(m, n + steps)
        s.prefill(p, lg, am)
        torch.cuda.synchronize()
        if i == 0:
            gate.check(0, lg.cpu().numpy(), ref[0], int(am.item()))
        nxt.append(int(am.item()))
        sess.append(s)
    blg = torch.empty(len(lens), shape.vocab, device="cuda")
    bam = torch.empty(len(lens), dtype=torch.int32, device="cuda")
    for step in range(steps):
        nxt[0] = int(toks[step])
        m.eval_batch(sess, nxt, blg, bam)
        torch.cuda.synchronize()
        gate.check(step + 1, blg[0].cpu().numpy(), ref[step + 1], int(bam[0].item()))
        nxt = [int(x) for x in bam.cpu().numpy()]
    gate.assert_ok()
    for o in sess + [m]:
        o.close()
