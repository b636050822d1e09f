"""Comparison rules shared by the GPU parity tests.

Outputs: max |gpu - ref| <= 2e-2 * max |ref| per output tensor, against the
oracle run on the same bf16 inputs. Expert ids: identical as sets for every
token whose oracle gap between the k-th and (k+1)-th logit exceeds 1e-3;
where the gap is smaller several selections are correct, and the GPU's is
accepted when each chosen logit is within 1e-3 of the k-th largest.
"""
import numpy as np
import torch

REL_TOL = 2e-2
GAP = 1e-3


def to_np(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_rel_close(gpu, ref, name, tol=REL_TOL):
    g = to_np(gpu)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, f"{name}: shape {g.shape} vs {r.shape}"
    assert np.isfinite(g).all(), f"{name}: non-finite GPU values"
    err = float(np.max(np.abs(g - r))) if g.size else 0.0
    scale = float(np.max(np.abs(r))) if r.size else 0.0
    assert err <= tol * scale, (f"{name}: max|err| {err:.4e} > {tol} * max|ref| "
                                f"{scale:.4e} (ratio {err / max(scale, 1e-300):.3e})")
    return err / max(scale, 1e-300)


def gaps(logits: np.ndarray, k: int) -> np.ndarray:
    """l_(k) - l_(k+1) per token (inf when k equals the expert count)."""
    s = -np.sort(-logits.astype(np.float64), axis=1)
    if k >= s.shape[1]:
        return np.full(s.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


def check_ids(gpu_ids, ref_ids, ref_logits, k):
    """Gap rule on the expert ids. Returns the tokens whose set differs (all
    of them inside the tie band)."""
    g = np.asarray(gpu_ids.cpu() if torch.is_tensor(gpu_ids) else gpu_ids)
    r = np.asarray(ref_ids)
    gp = gaps(ref_logits, k)
    differ = []
    for t in range(g.shape[0]):
        assert len(set(g[t].tolist())) == k, f"token {t}: repeated ids {g[t]}"
        assert ((0 <= g[t]) & (g[t] < ref_logits.shape[1])).all(), f"token {t}: id out of range"
        if set(g[t].tolist()) != set(r[t].tolist()):
            assert gp[t] <= GAP, (f"token {t}: ids {sorted(g[t])} vs oracle {sorted(r[t])} "
                                  f"with gap {gp[t]:.3e} > {GAP}")
            kth = -np.sort(-ref_logits[t].astype(np.float64))[k - 1]
            assert (ref_logits[t][g[t]] >= kth - GAP).all(), f"token {t}: pick outside tie band"
            differ.append(t)
        # the ids come in descending logit order (ties within the band may swap)
        lg = ref_logits[t][g[t]].astype(np.float64)
        assert (np.diff(lg) <= GAP).all(), f"token {t}: ids not in descending logit order"
    return differ


def ref_selection(gpu_ids, logits, k):
    """Oracle ids and weights for every token, after the gap rule.

    Where the GPU's set differs from the oracle's (only inside the tie band,
    which check_ids verifies), the reference continues from the GPU's choice:
    the oracle's top-k softmax run on that token's logits with every expert
    outside the GPU's set masked to -inf, i.e. the renormalised softmax over
    exactly the GPU's experts. Returns (ids, w, tokens that differed)."""
    import oracle
    ref_ids, ref_w = oracle.topk_softmax(logits, k)
    differ = check_ids(gpu_ids, ref_ids, logits, k)
    if differ:
        g = np.asarray(gpu_ids.cpu() if torch.is_tensor(gpu_ids) else gpu_ids)
        masked = np.full((len(differ), logits.shape[1]), -np.inf, dtype=np.float32)
        for i, t in enumerate(differ):
            masked[i, g[t]] = logits[t, g[t]]
        ids2, w2 = oracle.topk_softmax(masked, k)
        for i, t in enumerate(differ):
            assert set(ids2[i].tolist()) == set(g[t].tolist())
            ref_ids[t], ref_w[t] = ids2[i], w2[i]
    return ref_ids, ref_w, differ
