"""Checks that tie the oracle to facts outside itself.

Each check takes the oracle module as an argument so that the mutation tests
can run the same checks against deliberately broken copies of the oracle.
Independent references used here: torch's CPU scaled-dot-product attention (a
library routine, with and without a boolean mask), torch's average pooling,
closed forms for uniform attention, and a shift-free float64 closed form.
"""
import itertools

import numpy as np
import torch
import torch.nn.functional as F

from sparse_attention_diffusion_amd import synth

BLOCK = 64


def sdpa64(q, k, v, N, d, mask=None):
    """Library attention in float64 on the CPU (softmax scale 1/sqrt(d))."""
    q, k, v = (torch.as_tensor(np.asarray(x, dtype=np.float64))[..., :N, :] for x in (q, k, v))
    m = None if mask is None else torch.as_tensor(mask)
    return F.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=1.0 / np.sqrt(d)).numpy()


def block_mask(idx, N):
    """Boolean [B,H,N,N] mask: query t may see key j iff block(j) is listed for block(t)."""
    B, H, nb, _ = idx.shape
    mask = np.zeros((B, H, N, N), dtype=bool)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                rows = slice(i * BLOCK, min((i + 1) * BLOCK, N))
                for j in idx[b, h, i]:
                    mask[b, h, rows, j * BLOCK: min((j + 1) * BLOCK, N)] = True
    return mask


def rel(a, b):
    """Max-relative difference; any non-finite value is an infinite error (a
    NaN would otherwise vanish inside Python's max of several errors)."""
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    if not (np.all(np.isfinite(a)) and np.all(np.isfinite(b))):
        return float("inf")
    return float(np.abs(a - b).max() / max(1e-300, np.abs(b).max()))


def small_case(N=200, d=24, D=32, B=1, H=2, keep=2, seed=3, scale=1.0):
    q0, k0, v0 = synth.random_qkv(B, H, N, d, D, seed=seed, scale=scale)
    q1, k1, v1 = synth.random_qkv(B, H, N, d, D, seed=seed + 100, scale=scale)
    # the step-1 inputs drift from step 0 like the denoising workloads do
    q1, k1, v1 = (0.98 * a + 0.2 * b for a, b in ((q0, q1), (k0, k1), (v0, v1)))
    return [t.numpy().astype(np.float64) for t in (q0, k0, v0, q1, k1, v1)]


# ---------------------------------------------------------------- pins
def pin_calibration_identity(orc):
    """Calibrating and then reshaping on the same inputs gives dense attention."""
    q, k, v, _, _, _ = small_case()
    N, d = 200, 24
    idx = orc.select_blocks(q, k, N, d, keep=2, forced=[0])
    st = orc.calibrate(q, k, v, idx, N, d)
    dense = sdpa64(q, k, v, N, d)
    o = orc.sparse_reshape(q, k, v, idx, st, N, d)
    return max(rel(st["o"], dense), rel(o, dense))


def pin_keep_all(orc):
    """keep = number of blocks: no residual, equal denominators, dense output at a later step."""
    q0, k0, v0, q1, k1, v1 = small_case()
    N, d = 200, 24
    nb = (N + BLOCK - 1) // BLOCK
    idx = orc.select_blocks(q0, k0, N, d, keep=nb)
    st = orc.calibrate(q0, k0, v0, idx, N, d)
    o = orc.sparse_reshape(q1, k1, v1, idx, st, N, d)
    err_r = float(np.abs(st["r"]).max())
    err_z = rel(st["z_sparse"], st["z_full"])
    return max(err_r, err_z, rel(o, sdpa64(q1, k1, v1, N, d)))


def pin_closed_form(orc, N=130, d=16, D=16, keep=2, forced=(1,), seed=5, B=1, H=1):
    """Oracle two-step result equals the shift-free float64 closed form."""
    q0, k0, v0, q1, k1, v1 = small_case(N=N, d=d, D=D, B=B, H=H, seed=seed)
    idx = orc.select_blocks(q0, k0, N, d, keep=keep, forced=forced)
    st = orc.calibrate(q0, k0, v0, idx, N, d)
    o = orc.sparse_reshape(q1, k1, v1, idx, st, N, d)
    ref = orc.closed_form_fp64(q1, k1, v1, q0, k0, v0, idx, N, d)
    return rel(o, ref)


def pin_shift_invariance(orc):
    """Moving the cached max by delta and scaling Z, R by e^-delta changes nothing."""
    q0, k0, v0, q1, k1, v1 = small_case()
    N, d = 200, 24
    idx = orc.select_blocks(q0, k0, N, d, keep=2)
    st = orc.calibrate(q0, k0, v0, idx, N, d)
    o = orc.sparse_reshape(q1, k1, v1, idx, st, N, d)
    delta = 3.7
    sh = dict(m=st["m"] + delta, z_full=st["z_full"] * np.exp(-delta),
              z_sparse=st["z_sparse"] * np.exp(-delta), r=st["r"] * np.exp(-delta))
    return rel(orc.sparse_reshape(q1, k1, v1, idx, sh, N, d), o)


def pin_partition(orc):
    """Kept numerator + residual = full numerator; 0 < Z_sparse <= Z_full; the
    stored max is the row max of the logits."""
    q, k, v, _, _, _ = small_case()
    N, d = 200, 24
    idx = orc.select_blocks(q, k, N, d, keep=2)
    st = orc.calibrate(q, k, v, idx, N, d)
    logits = np.einsum("bhtc,bhjc->bhtj", q[..., :N, :], k[..., :N, :]) / np.sqrt(d)
    err_m = float(np.abs(st["m"] - logits.max(axis=-1)).max())
    ok = bool(np.all(st["z_sparse"] > 0) and np.all(st["z_sparse"] <= st["z_full"] * (1 + 1e-12)))
    # the residual alone is the masked part of the dense output: check against masked SDPA
    mask = block_mask(idx, N)
    w_masked = (st["z_full"] - st["z_sparse"]) / st["z_full"]
    masked_only = sdpa64(q, k, v, N, d, mask=~mask)
    err_r = rel(st["r"] / st["z_full"][..., None], masked_only * w_masked[..., None])
    return max(err_m, err_r, 0.0 if ok else 1.0)


def pin_sparse_only(orc):
    """With a zero residual and equal denominators the reshape is plain
    block-sparse attention (library SDPA with the block mask)."""
    q0, k0, v0, q1, k1, v1 = small_case()
    N, d = 200, 24
    idx = orc.select_blocks(q0, k0, N, d, keep=2, forced=[3])
    shape = q1.shape[:-2] + (N,)
    st = dict(m=np.zeros(shape), z_full=np.ones(shape), z_sparse=np.ones(shape),
              r=np.zeros(shape + (q1.shape[-1],)))
    o = orc.sparse_reshape(q1, k1, v1, idx, st, N, d)
    return rel(o, sdpa64(q1, k1, v1, N, d, mask=block_mask(idx, N)))


def pin_uniform(orc):
    """q = 0: every logit is 0, so calibration gives m = 0, Z_full = N,
    Z_sparse = kept keys, R = sum of masked v; the next step's reshape is the
    mean over keys of (current v on kept keys, calibration v on masked keys)."""
    _, k0, v0, _, k1, v1 = small_case()
    N, d = 200, 24
    q = np.zeros_like(k0)
    idx = orc.select_blocks(k0, k0, N, d, keep=2, forced=[0])
    st = orc.calibrate(q, k0, v0, idx, N, d)
    mask = block_mask(idx, N)[:, :, :, :]  # [B,H,N,N] same row pattern per block
    kept_cnt = mask.sum(axis=-1)
    errs = [float(np.abs(st["m"]).max()), rel(st["z_full"], np.full_like(st["z_full"], N)),
            rel(st["z_sparse"], kept_cnt)]
    r_ref = np.einsum("bhtj,bhjc->bhtc", (~mask).astype(np.float64), v0[..., :N, :])
    errs.append(rel(st["r"], r_ref))
    o = orc.sparse_reshape(q, k1, v1, idx, st, N, d)
    mixed = (np.einsum("bhtj,bhjc->bhtc", mask.astype(np.float64), v1[..., :N, :]) + r_ref) / N
    errs.append(rel(o, mixed))
    return max(errs)


def pin_pooling(orc):
    """Block means (short last block included) equal torch's average pooling."""
    x = np.random.default_rng(7).standard_normal((2, 3, 177, 5))
    got = orc.pool_blocks(x, 177)
    t = torch.as_tensor(x).permute(0, 1, 3, 2).reshape(-1, 5, 177)
    ref = F.avg_pool1d(t, kernel_size=BLOCK, stride=BLOCK, ceil_mode=True, count_include_pad=False)
    ref = ref.reshape(2, 3, 5, -1).permute(0, 1, 3, 2).numpy()
    return rel(got, ref)


def pin_pooled_scores(orc):
    """Pooled logits equal alpha * mean-q . mean-k computed by brute force."""
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 1, 150, 6))
    k = rng.standard_normal((1, 1, 150, 6))
    got = orc.pooled_scores(q, k, 150, 6)
    ref = np.zeros((3, 3))
    for i, j in itertools.product(range(3), range(3)):
        qi = [q[0, 0, t] for t in range(150) if t // 64 == i]
        kj = [k[0, 0, t] for t in range(150) if t // 64 == j]
        ref[i, j] = float(np.dot(sum(qi) / len(qi), sum(kj) / len(kj))) / np.sqrt(6)
    return rel(got[0, 0], ref)


def selector_violations(orc, srow, keep, forced):
    """Count violations of the definition of the kept list for one row."""
    sel = orc.select_from_scores(srow, keep, forced)
    nb = len(srow)
    bad = 0
    if list(sel) != sorted(set(sel)) or len(sel) != min(keep, nb):
        bad += 1
    if not set(forced) <= set(sel):
        bad += 1
    chosen = [j for j in sel if j not in forced]
    other = [j for j in range(nb) if j not in sel]
    for a in chosen:
        for b in other:
            if not (srow[a] > srow[b] or (srow[a] == srow[b] and a < b)):
                bad += 1
    return bad


def pin_selector(orc):
    rng = np.random.default_rng(9)
    bad = 0
    for nb in (1, 2, 5, 9, 17):
        for keep in range(1, nb + 1):
            for forced in ([], [0], [nb - 1, 0]):
                if len(set(forced)) > keep:
                    continue
                srow = rng.standard_normal(nb).astype(np.float32)
                bad += selector_violations(orc, srow, keep, forced)
                tied = np.round(srow * 2) / 2  # many exact ties
                bad += selector_violations(orc, tied, keep, forced)
    return float(bad)


def pin_dense_attention(orc):
    """The oracle's dense attention equals library SDPA: ragged N, a true head
    dim of 72 stored padded to 80 (zero channels), several (b, h), and logits
    large enough that an unshifted exponential would overflow."""
    errs = []
    for N, d, D, scale in ((201, 72, 80, 1.0), (130, 16, 16, 24.0), (64, 64, 64, 0.5)):
        q, k, v = (t.numpy().astype(np.float64) for t in synth.random_qkv(2, 3, N, d, D, seed=N + d, scale=scale))
        o = orc.dense_attention(q, k, v, N, d)
        errs.append(rel(o, sdpa64(q, k, v, N, d)))
        if D > d:
            errs.append(float(np.abs(o[..., d:]).max()))
    return max(errs)


# ---------------------------------------------------------------- reshape variant R2
def pin_r2_calibration_identity(orc):
    """R2 on the calibration inputs gives dense attention (as R1 does)."""
    q, k, v, _, _, _ = small_case()
    N, d = 200, 24
    idx = orc.select_blocks(q, k, N, d, keep=2, forced=[1])
    st = orc.calibrate(q, k, v, idx, N, d)
    return rel(orc.sparse_reshape_r2(q, k, v, idx, st, N, d), sdpa64(q, k, v, N, d))


def pin_r2_keep_all(orc):
    """R2 with every block kept gives dense attention at a later step."""
    q0, k0, v0, q1, k1, v1 = small_case()
    N, d = 200, 24
    nb = (N + BLOCK - 1) // BLOCK
    idx = orc.select_blocks(q0, k0, N, d, keep=nb)
    st = orc.calibrate(q0, k0, v0, idx, N, d)
    return rel(orc.sparse_reshape_r2(q1, k1, v1, idx, st, N, d), sdpa64(q1, k1, v1, N, d))


def pin_r2_closed_form(orc):
    """R2 = r O_sparse + (1 - r) O_masked with library pieces: masked attention of
    the later step over the listed blocks, masked attention of the calibration
    step over the other blocks, and r = exp(logsumexp_kept - logsumexp_all) of
    the calibration logits."""
    q0, k0, v0, q1, k1, v1 = small_case(N=190)
    N, d = 190, 24
    idx = orc.select_blocks(q0, k0, N, d, keep=2, forced=[0])
    st = orc.calibrate(q0, k0, v0, idx, N, d)
    mask = block_mask(idx, N)
    o_sparse = sdpa64(q1, k1, v1, N, d, mask=mask)
    o_masked = sdpa64(q0, k0, v0, N, d, mask=~mask)
    s0 = torch.as_tensor(q0[..., :N, :]) @ torch.as_tensor(k0[..., :N, :]).transpose(-1, -2) / np.sqrt(d)
    lse_all = torch.logsumexp(s0, dim=-1)
    lse_kept = torch.logsumexp(s0.masked_fill(~torch.as_tensor(mask), float("-inf")), dim=-1)
    r = torch.exp(lse_kept - lse_all).numpy()[..., None]
    return rel(orc.sparse_reshape_r2(q1, k1, v1, idx, st, N, d), r * o_sparse + (1 - r) * o_masked)


def pin_r2_logit_offset(orc):
    """R2 ignores a uniform per-row logit offset at the sparse step: a padding
    channel that adds delta_t to every logit of row t (q_t[c] = delta_t sqrt(d),
    k_j[c] = 1) leaves the output unchanged."""
    q0, k0, v0, q1, k1, v1 = small_case()
    N, d, c = 200, 24, 30
    idx = orc.select_blocks(q0, k0, N, d, keep=2)
    st = orc.calibrate(q0, k0, v0, idx, N, d)
    o = orc.sparse_reshape_r2(q1, k1, v1, idx, st, N, d)
    delta = np.random.default_rng(7).uniform(-4.0, 6.0, size=q1.shape[:-1])
    q1s, k1s = q1.copy(), k1.copy()
    q1s[..., c] = delta * np.sqrt(d)
    k1s[..., c] = 1.0
    return rel(orc.sparse_reshape_r2(q1s, k1s, v1, idx, st, N, d), o)


ALL_PINS = {
    "calibration_identity": (pin_calibration_identity, 1e-10),
    "keep_all": (pin_keep_all, 1e-10),
    "closed_form": (pin_closed_form, 1e-10),
    "shift_invariance": (pin_shift_invariance, 1e-10),
    "partition": (pin_partition, 1e-10),
    "sparse_only": (pin_sparse_only, 1e-10),
    "uniform": (pin_uniform, 1e-12),
    "pooling": (pin_pooling, 1e-12),
    "pooled_scores": (pin_pooled_scores, 1e-12),
    "selector": (pin_selector, 0.0),
    "dense_attention": (pin_dense_attention, 1e-10),
    "r2_calibration_identity": (pin_r2_calibration_identity, 1e-10),
    "r2_keep_all": (pin_r2_keep_all, 1e-10),
    "r2_closed_form": (pin_r2_closed_form, 1e-10),
    "r2_logit_offset": (pin_r2_logit_offset, 1e-10),
}


def failing_pins(orc):
    """Names of the pins a given oracle module fails (exceptions count as failures)."""
    out = []
    for name, (fn, tol) in ALL_PINS.items():
        try:
            with np.errstate(all="ignore"):  # broken copies may overflow
                err = fn(orc)
            if not (err <= tol):
                out.append(name)
        except Exception:  # a broken oracle may also crash
            out.append(name)
    return out
