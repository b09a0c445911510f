"""GPU-vs-oracle comparison protocol (tests only).

Bars (fixed in advance):
  * leaves: bit-exact for every key whose relative top-2 distance gap (over
    the parents, and over {parent} + its children) is >= 1e-4; an ambiguous
    key may take any of its near-tied candidates;
  * counts: bit-exact after the oracle adopts the GPU's choice for the
    ambiguous keys;
  * value sums: |gpu - oracle| <= (n - 1) * 2^-24 * sum|v| per slot and
    dimension (the fp32 recursive-summation bound, valid in any order) plus
    one fp32 ulp of slack for the stored result;
  * selections: equal sets for every tile whose importance gap
    (w_(P) - w_(P+1)) / w_(P) is >= 1e-4; for an ambiguous tile the GPU's set
    must be a valid top-P within that tolerance, and the oracle is re-run
    with the GPU's selection;
  * outputs: max |Y_gpu - Y_oracle| <= 2e-2 for bf16 inputs, 1e-4 for fp32
    inputs.
"""

import numpy as np

import oracle
import synth

AMBIG = 1e-4
Y_TOL = {"bf16": 2e-2, "f32": 1e-4}


def tensor_to_f64(t, dtype):
    """torch tensor (bf16 or fp32, any device) -> float64 numpy array."""
    import torch
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.to(torch.float64).numpy()


def check_stage1(inp, parents64, gpu_leaf, gpu_vsum, gpu_count, force_child=False):
    """Returns (oracle assignment dict with GPU choices adopted for ambiguous
    keys, vsum, count) after asserting the stage-1 bars."""
    ch = inp.f64("children")
    a = oracle.assign(inp.f64("K"), parents64, ch, force_child=force_child)
    amb = (a["gap_parent"] < AMBIG) | (a["gap_leaf"] < AMBIG)
    bad = (gpu_leaf != a["leaf"]) & ~amb
    assert not bad.any(), f"{bad.sum()} non-ambiguous keys assigned differently, first at {np.argwhere(bad)[:5]}"
    M0, C = inp.M0, inp.C
    # an ambiguous key's GPU leaf must at least be a slot of a valid shape
    assert ((gpu_leaf >= 0) & (gpu_leaf < M0 * (1 + C))).all()
    leaf = np.where(amb, gpu_leaf, a["leaf"])
    pst = leaf if C == 0 else np.where(leaf < M0, leaf, (leaf - M0) // C)
    vsum, count = oracle.aggregate(inp.f64("V"), leaf, M0, C)
    np.testing.assert_array_equal(gpu_count, count)
    # fp32 summation bound per slot and dimension
    # sum of |v| over each slot's keys (same slot membership as vsum)
    absum, _ = oracle.aggregate(np.abs(inp.f64("V")), leaf, M0, C)
    bound = np.maximum(count - 1, 0)[..., None] * 2.0 ** -24 * absum + 2.0 ** -23 * np.abs(vsum) + 1e-30
    err = np.abs(gpu_vsum - vsum)
    assert (err <= bound).all(), f"vsum outside the fp32 bound: max excess {(err - bound).max()}"
    a = dict(a)
    a["leaf"] = leaf
    a["pstar"] = pst
    a["n_ambiguous"] = int(amb.sum())
    return a, vsum, count


def tile_ambiguity(w, P):
    """w [..., ntiles, M0] -> bool [..., ntiles]: top-P boundary gap below the
    tolerance (never for P == 0 or P == M0)."""
    M0 = w.shape[-1]
    if P == 0 or P >= M0:
        return np.zeros(w.shape[:-1], dtype=bool)
    s = -np.sort(-w, axis=-1)
    wp, wn = s[..., P - 1], s[..., P]
    exact_tie_zero = (wp == 0) & (wn == 0)
    return ((wp - wn) <= AMBIG * wp) & ~exact_tie_zero


def check_selection(w_orc, sel_orc, sel_gpu, P):
    """Asserts the selection bar; returns the number of ambiguous tiles."""
    amb = tile_ambiguity(w_orc, P)
    B, H, nt = w_orc.shape[:3]
    for b in range(B):
        for h in range(H):
            for t in range(nt):
                g = set(sel_gpu[b, h, t].tolist())
                o = set(sel_orc[b, h, t].tolist())
                assert len(g) == P, f"tile {(b, h, t)}: duplicate selections {sorted(g)}"
                if not amb[b, h, t]:
                    assert g == o, f"tile {(b, h, t)}: gpu {sorted(g)} oracle {sorted(o)}"
                else:
                    w = w_orc[b, h, t]
                    inside = np.array(sorted(g))
                    outside = np.setdiff1d(np.arange(w.shape[0]), inside)
                    wp = -np.sort(-w)[P - 1]
                    if outside.size:
                        assert w[inside].min() >= w[outside].max() - AMBIG * wp - 1e-30
    return int(amb.sum())
