"""The chained decode launches (any-order launches ordered by device arrival counters) against
the same launches issued as ordinary dependent launches, and the chain's bounded wait.

* Chained = unchained, bit for bit: while the decode gate/up matvec is being event-timed the
  library issues a decode's per-layer launches unchained; two sessions of one model decode the
  same tokens, one with that timing on and one without, and every step's logits and argmax must
  be equal (BF16 and Q8_0 weights, BF16 and Q8_0 KV caches, one to three rows).
* Bounded wait: with the test hook gqa_model_debug_chain_offset every chained launch waits for
  arrivals that never come; the call must still complete (each wait gives up after its bounded
  number of polls, later ones at once), gqa_model_check_device_error must report it, and once
  the offset is cleared a fresh session must decode exactly as before."""
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_gqa_decoder_amd as lib
    lib.load()
    return lib


def _sessions(g, m, nb, n):
    ss = []
    blocks = synth.shuffled_blocks(11, n * nb).tolist()
    for i in range(n):
        ss.append(g.Session(m, nb * 32, block_ids=blocks[i * nb:(i + 1) * nb]))
    return ss


def _chained_equals_unchained(g, shape, seed, prompt_len, steps, rows, scheme="bf16", kv_quant="bf16"):
    print(f"[gpu] chained = unchained: {shape.name} {scheme} kv {kv_quant}, {rows} row(s), "
          f"{prompt_len}-token prompts, {steps} steps", flush=True)
    nb = synth.blocks_for(prompt_len + 7 * (rows - 1) + steps + 1)
    m = g.Model.from_shape(shape, seed=seed, scheme=scheme, kv_pool_blocks=2 * rows * nb, max_positions=nb * 32,
                           kv_quant=kv_quant)
    a = _sessions(g, m, nb, 2 * rows)
    chained, unchained = a[:rows], a[rows:]
    V = shape.vocab
    la = torch.empty(rows, V, device="cuda")
    lb = torch.empty(rows, V, device="cuda")
    aa = torch.empty(rows, dtype=torch.int32, device="cuda")
    ab = torch.empty(rows, dtype=torch.int32, device="cuda")
    for r in range(rows):
        prompt = synth.token_ids(seed + 10 + r, prompt_len + 7 * r)      # different contexts per row
        chained[r].prefill(prompt, la[r], aa[r:r + 1])
        unchained[r].prefill(prompt, lb[r], ab[r:r + 1])
    torch.cuda.synchronize()
    for step in range(steps):
        toks = [int(t) for t in aa.tolist()]
        if rows == 1:
            chained[0].decode(toks[0], la[0], aa)
        else:
            m.eval_batch(chained, toks, la, aa)
        m.profile("decode_gateup")                # unchained while this class is recorded
        if rows == 1:
            unchained[0].decode(toks[0], lb[0], ab)
        else:
            m.eval_batch(unchained, toks, lb, ab)
        m.profile("none")
        torch.cuda.synchronize()
        assert torch.equal(la.view(torch.int32), lb.view(torch.int32)), (shape.name, scheme, kv_quant, step)
        assert torch.equal(aa, ab)
    m.check_device_error()
    for o in a + [m]:
        o.close()


def test_chained_decode_equals_unchained_bitwise(g):
    _chained_equals_unchained(g, synth.reduced(synth.Q06B, n_layers=4), 2001, 200, 4, 1)
    _chained_equals_unchained(g, synth.reduced(synth.Q06B, n_layers=4), 2002, 90, 3, 3)
    _chained_equals_unchained(g, synth.TINY, 2003, 40, 3, 1, scheme="q8_0")
    _chained_equals_unchained(g, synth.TINY, 2004, 40, 3, 2, kv_quant="q8_0")


def test_chain_wait_gives_up_and_is_reported(g):
    print("[gpu] chain bounded wait: tiny shape, unsatisfiable targets for one decode call", flush=True)
    shape = synth.TINY
    nb = synth.blocks_for(64)
    m = g.Model.from_shape(shape, seed=2005, kv_pool_blocks=4 * nb, max_positions=nb * 32)
    prompt = synth.token_ids(2006, 30)
    V = shape.vocab
    lg = torch.empty(V, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    # reference: a normal decode step
    s0 = g.Session(m, nb * 32)
    s0.prefill(prompt, lg, am)
    tok = int(am.item())
    s0.decode(tok, lg, am)
    torch.cuda.synchronize()
    ref_logits, ref_arg = lg.clone(), int(am.item())
    m.check_device_error()
    # the same step with every chained wait unsatisfiable
    s1 = g.Session(m, nb * 32)
    s1.prefill(prompt, lg, am)
    torch.cuda.synchronize()
    m.debug_chain_offset(1)
    s1.decode(tok, lg, am)
    torch.cuda.synchronize()                       # the call completes: every wait is bounded
    m.debug_chain_offset(0)
    with pytest.raises(g.GqaError) as e:
        m.check_device_error()
    assert e.value.code == g._lib.GQA_E_HIP and "gave up waiting" in str(e.value)
    m.check_device_error()                          # the flag was cleared by the report
    # normal operation again: a fresh session reproduces the reference step exactly
    s2 = g.Session(m, nb * 32)
    s2.prefill(prompt, lg, am)
    s2.decode(tok, lg, am)
    torch.cuda.synchronize()
    assert torch.equal(lg.view(torch.int32), ref_logits.view(torch.int32))
    assert int(am.item()) == ref_arg
    m.check_device_error()
    for o in (s0, s1, s2, m):
        o.close()
