"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and compare with the oracle.  The oracle never receives a value produced on the
GPU; the GPU may receive oracle-made lists and statistics."""
import numpy as np
import torch

import oracle
from sparse_attention_diffusion_amd import configs, rettn, synth

DEV = "cuda"
# output tolerances: max |dO| <= 1e-2 max |O_ref|, L1-relative error <= 3e-3
MAX_REL = 1e-2
L1_REL = 3e-3


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = np.abs(got - ref)
    return float(diff.max() / np.abs(ref).max()), float(diff.sum() / np.abs(ref).sum())


def assert_close(got, ref, max_rel=MAX_REL, l1_rel=L1_REL, what="O"):
    assert np.all(np.isfinite(np.asarray(got, dtype=np.float64))), f"{what}: non-finite values"
    mx, l1 = errors(got, ref)
    print(f"[err] {what}: max-rel {mx:.3e} L1-rel {l1:.3e}", flush=True)
    assert mx <= max_rel and l1 <= l1_rel, f"{what}: max-rel {mx:.3e} (<= {max_rel}), L1-rel {l1:.3e} (<= {l1_rel})"
    return mx, l1


class Worst:
    """Collects per-block errors of one compared step; check() asserts the
    tolerance on every block and prints the worst block of the step."""

    def __init__(self, what, max_rel=MAX_REL, l1_rel=L1_REL):
        self.what, self.max_rel, self.l1_rel = what, max_rel, l1_rel
        self.rows = []

    def add(self, got, ref, where):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        finite = bool(np.all(np.isfinite(got)))
        mx, l1 = errors(got, ref) if finite else (float("inf"), float("inf"))
        self.rows.append((mx, l1, where))

    def check(self):
        assert self.rows, f"{self.what}: nothing compared"
        wm = max(self.rows, key=lambda r: r[0])
        wl = max(self.rows, key=lambda r: r[1])
        print(f"[err] {self.what}: {len(self.rows)} blocks, worst max-rel {wm[0]:.3e} at {wm[2]}, "
              f"worst L1-rel {wl[1]:.3e} at {wl[2]}", flush=True)
        bad = [r for r in self.rows if not (r[0] <= self.max_rel and r[1] <= self.l1_rel)]
        assert not bad, f"{self.what}: {len(bad)} blocks out of tolerance, e.g. {bad[:3]}"
        return wm[0], wl[1]


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def residual_positions(sh, bh, rows):
    """Positions in one layer's flat R of rows `rows` of head bh, all d_pad
    columns ([len(rows), d_pad]).  The layout written out independently of
    the library (and checked against its rt_residual_index on the host):
    blocks of 64 rows padded past N; inside a block, for each 32-row half and
    8-column group, a run of 256 elements ordered (4-column half, row, column)."""
    D = sh.d_pad
    nb = (sh.N + 63) // 64
    row = np.asarray(rows, dtype=np.int64)[:, None]
    col = np.arange(D, dtype=np.int64)[None, :]
    r = row % 64
    run = (r // 32) * (D // 8) + col // 8
    return (bh * nb + row // 64) * 64 * D + run * 256 + (32 * ((col // 4) % 2) + r % 32) * 4 + col % 4


def r_rows(R, sh, b, h, rows):
    """Residual of head (b, h), rows `rows` (a slice or index array), as a host
    float64 array [rows, d_pad]."""
    pos = residual_positions(sh, b * sh.H + h, np.arange(sh.N)[rows])
    return host(R[torch.as_tensor(pos, device=R.device)])


def r_all(R, sh):
    """The whole residual of one layer as a host float64 array [B, H, N, d_pad]."""
    pos = np.stack([residual_positions(sh, bh, np.arange(sh.N)) for bh in range(sh.B * sh.H)])
    return host(R[torch.as_tensor(pos, device=R.device)]).reshape(sh.B, sh.H, sh.N, sh.d_pad)


def r_fill(R, sh, values):
    """Stores values [B, H, N, c] (c <= d_pad; missing columns and the padding
    rows become zero) into one layer's flat R."""
    values = np.asarray(values)
    full = np.zeros((sh.B, sh.H, sh.N, sh.d_pad), dtype=np.float64)
    full[..., :values.shape[-1]] = values
    pos = np.stack([residual_positions(sh, bh, np.arange(sh.N)) for bh in range(sh.B * sh.H)])
    R.zero_()
    R[torch.as_tensor(pos.reshape(-1), device=R.device)] = torch.as_tensor(full.reshape(-1), dtype=R.dtype,
                                                                            device=R.device)


def gpu_inputs(cfg, n_steps, seed=0):
    """Stored (q, k, v) per step, generated on the GPU."""
    return synth.steps(cfg, n_steps, seed=seed, device=DEV)


def empty_out(sh):
    return torch.zeros((sh.B, sh.H, sh.N, sh.d_pad), dtype=rettn.torch_dtype(sh), device=DEV)


def select(sh, q, k, forced):
    nb = rettn.num_blocks(sh)
    idx = torch.full((sh.B, sh.H, nb, sh.keep), -1, dtype=torch.int32, device=DEV)
    scores = torch.zeros((sh.B, sh.H, nb, nb), dtype=torch.float32, device=DEV)
    ws = torch.empty(rettn.select_workspace_bytes(sh), dtype=torch.uint8, device=DEV)
    rettn.rt_select_blocks(sh, q, k, forced, idx, scores, ws)
    torch.cuda.synchronize()
    return idx, scores


def oracle_lists(cfg_like, q, k, forced, keep):
    N, d = cfg_like["N"], cfg_like["d"]
    return oracle.select_blocks(host(q), host(k), N, d, keep, forced)


def valid_topk(scores_row, sel, keep, forced):
    """The list is ascending, holds the forced blocks, and every other chosen
    block beats every unchosen one by (score descending, index ascending)."""
    sel = [int(x) for x in sel]
    nb = len(scores_row)
    if sel != sorted(set(sel)) or len(sel) != min(keep, nb) or not set(forced) <= set(sel):
        return False
    chosen = [j for j in sel if j not in forced]
    other = [j for j in range(nb) if j not in sel]
    if not chosen or not other:
        return True
    worst = min(chosen, key=lambda j: (scores_row[j], -j))
    best = max(other, key=lambda j: (scores_row[j], -j))
    return (scores_row[worst], -worst) > (scores_row[best], -best)


def calibrate(sh, q, k, v, idx, cache, layer=0):
    o = empty_out(sh)
    rettn.rt_calibrate(sh, q, k, v, idx, cache, layer, o)
    return o


def sparse(sh, q, k, v, cache, layer=0, idx=None, variant=None):
    """Sparse step through rt_sparse_attn_reshape, or through the _ex entry
    point when a reshape variant ("r1" / "r2") is named."""
    o = empty_out(sh)
    if variant is None:
        rettn.rt_sparse_attn_reshape(sh, q, k, v, idx, cache, layer, o)
    else:
        rettn.rt_sparse_attn_reshape_ex(sh, q, k, v, idx, cache, layer, variant, o)
    return o


def block_rows(N, i):
    return slice(i * 64, min(N, (i + 1) * 64))


def sample_blocks(nb):
    return sorted(set([0, min(3, nb - 1), min(4, nb - 1), nb // 2, nb - 1]))


__all__ = ["configs", "synth", "rettn", "oracle"]
