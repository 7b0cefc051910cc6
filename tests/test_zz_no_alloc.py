"""The allocation-free single-row decode (gqa_session_eval_decode_static) against
gqa_session_eval_decode: two calls in a row through the C ABI, the second on a smaller model and
a shorter context, each bit-identical (logits and argmax) to the existing entry point on a twin
session (also with a Q8_0 KV cache); then a model whose scratch exceeds the static array is
refused before any work."""
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


def _twin_steps(g, shape, seed, prompt_len, steps, kv_quant="bf16"):
    """Prefill the same prompt in two sessions, then decode the same tokens through
    eval_decode (a) and eval_decode_static (b); every step's logits and argmax must be equal."""
    nb = synth.blocks_for(prompt_len + steps + 1)
    m = g.Model.from_shape(shape, seed=seed, kv_pool_blocks=2 * nb, max_positions=nb * 32, kv_quant=kv_quant)
    a = g.Session(m, nb * 32)
    b = g.Session(m, nb * 32, block_ids=[x for x in synth.shuffled_blocks(7, 2 * nb).tolist() if x >= nb])
    prompt = synth.token_ids(seed + 1, prompt_len)
    la, lb = torch.empty(shape.vocab, device="cuda"), torch.empty(shape.vocab, device="cuda")
    aa, ab = torch.empty(1, dtype=torch.int32, device="cuda"), torch.empty(1, dtype=torch.int32, device="cuda")
    a.prefill(prompt, la, aa)
    b.prefill(prompt, lb, ab)
    torch.cuda.synchronize()
    assert torch.equal(la, lb)
    for step in range(steps):
        tok = int(aa.item())
        a.decode(tok, la, aa)
        b.decode_static(tok, lb, ab)
        torch.cuda.synchronize()
        assert torch.equal(la.view(torch.int32), lb.view(torch.int32)), (shape.name, step)
        assert int(aa.item()) == int(ab.item())
    m.check_device_error()
    for o in (a, b, m):
        o.close()


def test_static_decode_equals_decode_two_calls(g):
    print("[gpu] static decode: 0.6B shape (6 layers), 300-token context", flush=True)
    _twin_steps(g, synth.reduced(synth.Q06B, n_layers=6), 1002, 300, 3)
    print("[gpu] static decode: tiny shape, 20-token context (smaller input)", flush=True)
    _twin_steps(g, synth.TINY, 1001, 20, 3)
    print("[gpu] static decode: tiny shape, Q8_0 KV cache, 40-token context", flush=True)
    _twin_steps(g, synth.TINY, 1001, 40, 3, kv_quant="q8_0")


def test_static_decode_refuses_what_does_not_fit(g):
    # a 2^21-entry vocabulary with 32 query heads needs more than the 2 MiB of static scratch;
    # refused at position 0, before any work is enqueued
    big = synth.ModelShape("wide-vocab", n_layers=1, hidden=1024, n_q_heads=32, ffn=3072, vocab=1 << 21)
    m = g.Model.from_shape(big, seed=5, kv_pool_blocks=2, max_positions=32)
    s = g.Session(m, 32)
    lg = torch.empty(big.vocab, device="cuda")
    with pytest.raises(g.GqaError) as ei:
        s.decode_static(7, lg)
    assert ei.value.code == g.GQA_E_INVALID and "2097152" in str(ei.value)
    assert s.position == 0
    for o in (s, m):
        o.close()
