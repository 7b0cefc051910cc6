"""Helpers shared by the GPU parity tests: the gate of Kipp Model Support, "What the gates
check" (GPU vs CPU oracle: identical argmax and full-logit NMSE <= 1e-4 at prefill and every
checked decode position), plus the near-tie classification declared for random-weight models.

Random-init logits are close to i.i.d. Gaussian over 151,936 entries, so the top-2 gap is often
tiny and two correct FP32 implementations (the oracle and a more exact one) already differ by
NMSE ~1e-7 through BF16 K/V rounding flips. A position whose argmax differs is accepted as a
near tie only if the oracle's top-2 margin is below 4x the RMS logit error actually observed at
that position and the GPU's pick is the oracle's runner-up; every other mismatch fails.
"""
import numpy as np

NMSE_BOUND = 1e-4


def nmse(y, ref):
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    return float(np.sum((y - r) ** 2) / np.sum(r ** 2))


class Gate:
    def __init__(self, name):
        self.name, self.rows = name, []

    def check(self, pos, gpu_logits, ref_logits, gpu_argmax=None):
        g = np.asarray(gpu_logits, dtype=np.float32)
        r = np.asarray(ref_logits, dtype=np.float32)
        e = nmse(g, r)
        ra = int(np.argmax(r))
        ga = int(np.argmax(g)) if gpu_argmax is None else int(gpu_argmax)
        top2 = np.partition(r, -2)[-2:]
        margin = float(top2[1] - top2[0])
        rms = float(np.sqrt(np.mean((g.astype(np.float64) - r) ** 2)))
        near_tie = ga != ra and margin < 4 * rms and ga == int(np.argsort(r)[-2])   # runner-up
        self.rows.append(dict(pos=pos, nmse=e, ok=ga == ra, near_tie=near_tie, margin=margin, rms=rms))
        return e

    def assert_ok(self):
        assert self.rows, "nothing checked"
        worst = max(r["nmse"] for r in self.rows)
        bad = [r for r in self.rows if not r["ok"] and not r["near_tie"]]
        ties = [r for r in self.rows if r["near_tie"]]
        print(f"[{self.name}] positions={len(self.rows)} worst_nmse={worst:.3e} argmax_mismatch={len(bad)} "
              f"near_ties={len(ties)}", flush=True)
        for r in ties:
            print(f"  near tie at {r['pos']}: margin {r['margin']:.3e} rms {r['rms']:.3e}", flush=True)
        assert worst <= NMSE_BOUND, f"worst NMSE {worst:.3e} > {NMSE_BOUND}"
        assert not bad, f"argmax mismatches: {bad[:5]}"
        return worst
