"""Writes the stored oracle references of the two full-size workloads whose oracle runs take
too long to repeat inside a GPU test (tens of minutes of NumPy on a CPU):

* ``oracle_ref_4b_q8_0.npz`` -- the Qwen3-4B shape with Q8_0 projections: the 12,800-token
  prompt, then 32 greedy decode steps.
* ``oracle_ref_8b_batch.npz`` -- the Qwen3-8B shape (untied lm_head): the declared subset of
  the 32 batched sessions (the shortest context, the longest, and sessions 0 and 16), each
  prefilled alone and then decoded greedily for 128 steps.

Only ``oracle`` and ``synth`` are called. For every checked position the file keeps the
oracle's residual stream after the last layer (FP32, ``x[check][hidden]``) and the greedy
token fed at each step (the oracle's argmax at the previous check); a test rebuilds the
full-vocabulary logits with ``oracle.final_logits``, the oracle's own final norm and
lm_head, so the stored arrays stay small (a logit vector is 151,936 floats, a residual row
2,560 or 4,096).

Usage (from the repository root):  python tests/golden/make_oracle_refs.py [4b-q8] [8b-batch]
"""
import hashlib
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
import oracle  # noqa: E402
from oracle import model as om  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
SUBSET_8B_FIXED = (0, 16)


def say(*a):
    print(time.strftime("%H:%M:%S"), *a, flush=True)


def source_hashes():
    out = {}
    for rel in ("oracle/model.py", "oracle/q8_0.py", "synth/__init__.py"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            out[rel] = hashlib.sha256(f.read()).hexdigest()
    return out


def ids_hash(ids):
    return hashlib.sha256(np.asarray(ids, dtype=np.int32).tobytes()).hexdigest()


def greedy_residuals(model, prompt, steps, label):
    """Oracle residual rows at the last prompt position and after each greedy decode step,
    and the tokens fed (the argmax of the previous position's logits)."""
    shape = model.shape
    s = oracle.OracleSession(model, oracle.ContiguousKV.for_shape(shape, len(prompt) + steps + 1))
    t0 = time.time()
    x = [s.residual(prompt)[-1]]
    say(label, "prefill of", len(prompt), "tokens: %.0f s" % (time.time() - t0))
    toks = []
    for i in range(steps):
        t = om.argmax(oracle.final_logits(model, x[-1][None])[0])
        toks.append(t)
        x.append(s.residual([t])[-1])
        if (i + 1) % 16 == 0:
            say(label, "decode step", i + 1, "of", steps)
    return np.stack(x).astype(np.float32), np.asarray(toks, dtype=np.int32)


def make_4b_q8():
    wl = synth.WORKLOADS["4b-q8"]
    prompt = synth.token_ids(wl.ids_seed, wl.prompt)
    say("4b-q8: oracle model (Q8_0 projections)")
    m = oracle.OracleModel(wl.shape, wl.weight_seed, "q8_0")
    x, toks = greedy_residuals(m, prompt, wl.decode, "4b-q8")
    path = os.path.join(HERE, "oracle_ref_4b_q8_0.npz")
    np.savez(path, x=x, toks=toks, prompt_sha=ids_hash(prompt), shape=wl.shape.name,
             weight_seed=wl.weight_seed, ids_seed=wl.ids_seed, prompt_len=wl.prompt, steps=wl.decode,
             scheme="q8_0", sources=str(source_hashes()))
    say("wrote", path)


def subset_8b():
    lens = synth.context_lengths(synth.CONTEXT_SEED_8B, synth.WORKLOADS["8b-batch"].n_seqs)
    sub = [int(np.argmin(lens)), int(np.argmax(lens))] + [i for i in SUBSET_8B_FIXED]
    return lens, sub


def make_8b_batch():
    wl = synth.WORKLOADS["8b-batch"]
    lens, sub = subset_8b()
    say("8b-batch: sessions", sub, "contexts", [int(lens[i]) for i in sub])
    m = oracle.OracleModel(wl.shape, wl.weight_seed)
    xs, ts, hs = [], [], []
    for i in sub:
        p = synth.token_ids(wl.ids_seed, int(lens[i]), offset=i * 8192)
        x, toks = greedy_residuals(m, p, wl.decode, "8b session %d" % i)
        xs.append(x)
        ts.append(toks)
        hs.append(ids_hash(p))
    path = os.path.join(HERE, "oracle_ref_8b_batch.npz")
    np.savez(path, x=np.stack(xs), toks=np.stack(ts), sessions=np.asarray(sub, dtype=np.int32),
             contexts=np.asarray([int(lens[i]) for i in sub], dtype=np.int32), prompt_sha=np.asarray(hs),
             shape=wl.shape.name, weight_seed=wl.weight_seed, ids_seed=wl.ids_seed, steps=wl.decode,
             scheme="bf16", sources=str(source_hashes()))
    say("wrote", path)


if __name__ == "__main__":
    which = sys.argv[1:] or ["4b-q8", "8b-batch"]
    for w in which:
        {"4b-q8": make_4b_q8, "8b-batch": make_8b_batch}[w]()
