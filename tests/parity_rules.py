"""Comparison rules between the HIP path and the oracle (no method arithmetic).

* index sets: equal, or every block in the symmetric difference has an oracle
  score within 1e-5 (relative) of the oracle's k-th largest candidate score,
  with the sink and local blocks present;
* outputs: max-abs error <= 2e-3 (bf16 inputs, fp32 accumulation), against
  the oracle evaluated on the HIP path's own index set;
* fp32 summaries: within the worst-case bound of an fp32 sum of n terms in any
  order followed by a division, (n + 4) * 2^-24 * mean|x| per column.
"""
import numpy as np

OUT_ATOL = 2e-3
TIE_REL = 1e-5
U32 = 2.0 ** -24


def to_dev(a):
    """uint16 bf16 bits (numpy) -> torch bf16 on cuda:0."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda")


def from_dev_bf16(t):
    return t.view(__import__("torch").int16).cpu().numpy().view(np.uint16)


def mean_abs_blocks(x_u16, seq_len, bs):
    """per (pair, block, column) mean of |x| over the block's valid tokens (float64)."""
    from long_context_block_summary_amd.synth import bf16_to_f32
    B, H, _, d = x_u16.shape
    nb = -(-seq_len // bs)
    out = np.empty((B, H, nb, d), np.float64)
    full = seq_len // bs
    xa = np.abs(bf16_to_f32(x_u16[:, :, :full * bs]))
    if full:
        out[:, :, :full] = xa.reshape(B, H, full, bs, d).mean(axis=3)
    if nb > full:
        tail = np.abs(bf16_to_f32(x_u16[:, :, full * bs:seq_len]))
        out[:, :, full] = tail.mean(axis=2)
    return out


def summary_tolerance(x_u16, seq_len, bs):
    mabs = mean_abs_blocks(x_u16, seq_len, bs)
    n = min(bs, seq_len)
    return (n + 4) * U32 * mabs + 1e-30


def check_index_sets(gpu_idx, ora_idx, ora_scores, nb, n_sink, n_local, rel=TIE_REL):
    """Returns the number of (pair, block) differences exempted as near-ties.
    Raises AssertionError on a real mismatch."""
    gpu_idx = np.asarray(gpu_idx)
    ora_idx = np.asarray(ora_idx)
    assert gpu_idx.shape == ora_idx.shape, (gpu_idx.shape, ora_idx.shape)
    fixed = set(range(min(n_sink, nb))) | set(range(max(0, nb - n_local), nb))
    exempt = 0
    flat_g = gpu_idx.reshape(-1, gpu_idx.shape[-1])
    flat_o = ora_idx.reshape(-1, ora_idx.shape[-1])
    flat_s = ora_scores.reshape(-1, ora_scores.shape[-1])
    for p in range(flat_g.shape[0]):
        g, o = flat_g[p], flat_o[p]
        assert np.all(np.diff(g) > 0), f"pair {p}: not strictly ascending"
        assert g.min() >= 0 and g.max() < nb, f"pair {p}: out of range"
        sg, so = set(g.tolist()), set(o.tolist())
        assert fixed <= sg, f"pair {p}: sink/local missing"
        if sg == so:
            continue
        sel = np.array(sorted(so - fixed))
        tau = flat_s[p, sel].min()
        for j in sg ^ so:
            sj = flat_s[p, j]
            assert abs(sj - tau) <= rel * max(abs(sj), abs(tau)), \
                f"pair {p}: block {j} score {sj} vs k-th {tau}"
            exempt += 1
    return exempt
