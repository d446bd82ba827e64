"""Plain, slow reference for Re-ttention sparse attention with a statistical reshape.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline may import this module.  It shares no code with the HIP kernels.

Source: the Re-ttention project page ("Re-ttention: Ultra Sparse Visual
Generation via Attention Statistical Reshape").

* Teaser paragraph: statistics cached across denoising steps reshape sparse
  attention so that the full attention distribution is recovered.
* Abstract: sparse attention attends to a small fraction of the tokens (the
  page reports 3.1%); renormalising the softmax over that fraction shifts the
  probabilities, and the reshape corrects the shift with the softmax statistics
  of earlier steps.
* Core-mechanism paragraph: the ratio of sparse to full softmax denominators is
  reused, and the contribution of masked-out tokens is cached as a residual.

The pages give the mechanism in words only.  The formulation written out here
(one reading of that paragraph, the one this library implements) is, per batch
b, head h, with alpha = 1/sqrt(d) for the true head dim d and 64-token blocks:

  selection   pooled means Qb_i, Kb_j of each block; S_ij = alpha <Qb_i, Kb_j>;
              I_i = forced blocks + best (keep - |forced|) others by
              (S_ij descending, j ascending), listed ascending.
  calibration s_j = alpha <q_t, k_j> over all keys, m = max_j s_j,
              p_j = exp(s_j - m), Z_full = sum_j p_j,
              Z_sparse = sum_{block(j) in I} p_j,
              R = sum_{block(j) not in I} p_j v_j,
              O = (sum_{block(j) in I} p_j v_j + R) / Z_full   (= dense attention).
  sparse step s_j over kept keys only, m, Z = sum e^{s-m}, N = sum e^{s-m} v,
              M = max(m, m_c),
              O = (N e^{m-M} + R_c e^{m_c-M}) / (Z e^{m-M} Z_full_c / Z_sparse_c).
  variant R2  (a second reading of the same paragraph, kept as an option: the
              cached ratio r_c = Z_sparse_c / Z_full_c weights the step's
              renormalised sparse output against the cached masked part)
              O = r_c N / Z + R_c / Z_full_c
                = r_c O_sparse + (1 - r_c) R_c / (Z_full_c - Z_sparse_c).

Everything is computed in ``dtype`` (float64 unless asked otherwise) from the
stored input values.
"""
import numpy as np

BLOCK = 64


def _np(x, dtype):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").float().numpy()
    return np.asarray(x, dtype=dtype)


def block_ranges(N, block=BLOCK):
    """[(start, stop)] of each token block; the last one may be short."""
    return [(s, min(s + block, N)) for s in range(0, N, block)]


def pool_blocks(x, N, block=BLOCK, dtype=np.float64):
    """Mean of each block's token vectors.  x: [..., N, D] -> [..., Nb, D]."""
    x = _np(x, dtype)
    parts = [x[..., a:b, :].sum(axis=-2) / dtype(b - a) for a, b in block_ranges(N, block)]
    return np.stack(parts, axis=-2)


def pooled_scores(q, k, N, d, block=BLOCK, dtype=np.float64):
    """Block-level logits S_ij = alpha <mean q of block i, mean k of block j>."""
    alpha = dtype(1.0) / np.sqrt(dtype(d))
    qb = pool_blocks(q, N, block, dtype)
    kb = pool_blocks(k, N, block, dtype)
    return alpha * (qb @ np.swapaxes(kb, -1, -2))


def select_from_scores(srow, keep, forced=()):
    """Kept key blocks for one query block: the forced ones plus the best
    remaining ones by (score descending, index ascending); ascending output."""
    nb = len(srow)
    if keep >= nb:
        return list(range(nb))
    fixed = sorted(set(int(j) for j in forced))
    assert len(fixed) <= keep
    rest = [j for j in range(nb) if j not in fixed]
    rest.sort(key=lambda j: (-float(srow[j]), j))
    return sorted(fixed + rest[: keep - len(fixed)])


def select_blocks(q, k, N, d, keep, forced=(), block=BLOCK, dtype=np.float64, scores=None):
    """Index lists [B, H, Nb, keep] (int32).  ``scores`` may supply S directly."""
    if scores is None:
        scores = pooled_scores(q, k, N, d, block, dtype)
    B, H, nb = scores.shape[0], scores.shape[1], scores.shape[2]
    out = np.zeros((B, H, nb, min(keep, nb)), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                out[b, h, i] = select_from_scores(scores[b, h, i], keep, forced)
    return out


def _kept_mask(idx_row, N, block):
    mask = np.zeros(N, dtype=bool)
    for j in idx_row:
        mask[j * block: min((j + 1) * block, N)] = True
    return mask


def dense_attention(q, k, v, N, d, dtype=np.float64):
    """softmax(alpha q k^T) v over all keys, row by row in blocks."""
    q, k, v = (_np(t, dtype) for t in (q, k, v))
    alpha = dtype(1.0) / np.sqrt(dtype(d))
    o = np.zeros(q.shape[:-2] + (N, q.shape[-1]), dtype=dtype)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            K, V = k[b, h, :N], v[b, h, :N]
            for a, e in block_ranges(N):
                s = alpha * (q[b, h, a:e] @ K.T)
                p = np.exp(s - s.max(axis=1, keepdims=True))
                o[b, h, a:e] = (p @ V) / p.sum(axis=1, keepdims=True)
    return o


def calibrate_rows(q, k, v, rows, idx_row, N, d, block=BLOCK, dtype=np.float64):
    """Calibration statistics for query rows ``rows`` of one head (q,k,v: [N, D]);
    all rows must lie in one query block whose kept list is ``idx_row``."""
    q, k, v = (_np(t, dtype) for t in (q, k, v))
    alpha = dtype(1.0) / np.sqrt(dtype(d))
    kept = _kept_mask(idx_row, N, block)
    K, V = k[:N], v[:N]
    s = alpha * (q[rows] @ K.T)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    z_full = p.sum(axis=1)
    z_sparse = p[:, kept].sum(axis=1)
    r = p[:, ~kept] @ V[~kept]
    num_kept = p[:, kept] @ V[kept]
    o = (num_kept + r) / z_full[:, None]
    return dict(o=o, m=m, z_full=z_full, z_sparse=z_sparse, r=r)


def sparse_reshape_rows(q, k, v, rows, idx_row, m_c, z_full_c, z_sparse_c, r_c, N, d,
                        block=BLOCK, dtype=np.float64):
    """Reshaped sparse attention for query rows ``rows`` of one head, given the
    cached statistics of those rows."""
    q, k, v = (_np(t, dtype) for t in (q, k, v))
    m_c, z_full_c, z_sparse_c, r_c = (_np(t, dtype) for t in (m_c, z_full_c, z_sparse_c, r_c))
    alpha = dtype(1.0) / np.sqrt(dtype(d))
    kept = _kept_mask(idx_row, N, block)
    K, V = k[:N][kept], v[:N][kept]
    s = alpha * (q[rows] @ K.T)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    z = p.sum(axis=1)
    n = p @ V
    big = np.maximum(m, m_c)
    num = n * np.exp(m - big)[:, None] + r_c * np.exp(m_c - big)[:, None]
    den = z * np.exp(m - big) * z_full_c / z_sparse_c
    return num / den[:, None]


def sparse_reshape_rows_r2(q, k, v, rows, idx_row, z_full_c, z_sparse_c, r_c, N, d,
                           block=BLOCK, dtype=np.float64):
    """Reshape variant R2 for query rows ``rows`` of one head: the step's sparse
    attention output over the kept keys (softmax renormalised over them),
    weighted by the cached ratio, plus the cached masked part R_c / Z_full_c.
    Both terms are free of any max shift (R_c and Z_full_c share one)."""
    q, k, v = (_np(t, dtype) for t in (q, k, v))
    z_full_c, z_sparse_c, r_c = (_np(t, dtype) for t in (z_full_c, z_sparse_c, r_c))
    alpha = dtype(1.0) / np.sqrt(dtype(d))
    kept = _kept_mask(idx_row, N, block)
    K, V = k[:N][kept], v[:N][kept]
    s = alpha * (q[rows] @ K.T)
    p = np.exp(s - s.max(axis=1)[:, None])
    o_sparse = (p @ V) / p.sum(axis=1)[:, None]
    return (z_sparse_c / z_full_c)[:, None] * o_sparse + r_c / z_full_c[:, None]


def sparse_reshape_r2(q, k, v, idx, cache, N, d, block=BLOCK, dtype=np.float64):
    """Reshape variant R2 over a whole layer with the cached statistics ``cache``."""
    q, k, v = (_np(t, dtype) for t in (q, k, v))
    B, H, _, D = q.shape
    o = np.zeros((B, H, N, D), dtype)
    for b in range(B):
        for h in range(H):
            for i, (a, e) in enumerate(block_ranges(N, block)):
                o[b, h, a:e] = sparse_reshape_rows_r2(
                    q[b, h], k[b, h], v[b, h], slice(a, e), idx[b, h, i], cache["z_full"][b, h, a:e],
                    cache["z_sparse"][b, h, a:e], cache["r"][b, h, a:e], N, d, block, dtype)
    return o


def calibrate(q, k, v, idx, N, d, block=BLOCK, dtype=np.float64):
    """Calibration step over a whole layer.  idx: [B, H, Nb, keep]."""
    q, k, v = (_np(t, dtype) for t in (q, k, v))
    B, H, _, D = q.shape
    out = dict(o=np.zeros((B, H, N, D), dtype), m=np.zeros((B, H, N), dtype),
               z_full=np.zeros((B, H, N), dtype), z_sparse=np.zeros((B, H, N), dtype),
               r=np.zeros((B, H, N, D), dtype))
    for b in range(B):
        for h in range(H):
            for i, (a, e) in enumerate(block_ranges(N, block)):
                st = calibrate_rows(q[b, h], k[b, h], v[b, h], slice(a, e), idx[b, h, i], N, d, block, dtype)
                for name, val in st.items():
                    out[name][b, h, a:e] = val
    return out


def sparse_reshape(q, k, v, idx, cache, N, d, block=BLOCK, dtype=np.float64):
    """Sparse step over a whole layer with the cached statistics ``cache``."""
    q, k, v = (_np(t, dtype) for t in (q, k, v))
    B, H, _, D = q.shape
    o = np.zeros((B, H, N, D), dtype)
    for b in range(B):
        for h in range(H):
            for i, (a, e) in enumerate(block_ranges(N, block)):
                o[b, h, a:e] = sparse_reshape_rows(
                    q[b, h], k[b, h], v[b, h], slice(a, e), idx[b, h, i],
                    cache["m"][b, h, a:e], cache["z_full"][b, h, a:e], cache["z_sparse"][b, h, a:e],
                    cache["r"][b, h, a:e], N, d, block, dtype)
    return o


def closed_form_fp64(q, k, v, q_c, k_c, v_c, idx, N, d, block=BLOCK):
    """Shift-free closed form of the reshaped output, evaluated row by row in
    float64 for tiny inputs.  With kept key set K of the row's query block,
    logits s now and s^c at the calibration step:

      O_t = (sum_{j in K} e^{s_tj} v_j + sum_{j not in K} e^{s^c_tj} v^c_j)
            * sum_{j in K} e^{s^c_tj} / (sum_{j in K} e^{s_tj} * sum_j e^{s^c_tj})
    """
    q, k, v, q_c, k_c, v_c = (_np(t, np.float64) for t in (q, k, v, q_c, k_c, v_c))
    B, H, _, D = q.shape
    alpha = 1.0 / np.sqrt(float(d))
    o = np.zeros((B, H, N, D))
    for b in range(B):
        for h in range(H):
            for t in range(N):
                kept_blocks = set(int(j) for j in idx[b, h, t // block])
                num = np.zeros(D)
                sum_now_kept = 0.0
                sum_cal_kept = 0.0
                sum_cal_all = 0.0
                for j in range(N):
                    e_cal = np.exp(alpha * float(np.dot(q_c[b, h, t], k_c[b, h, j])))
                    sum_cal_all += e_cal
                    if j // block in kept_blocks:
                        e_now = np.exp(alpha * float(np.dot(q[b, h, t], k[b, h, j])))
                        num += e_now * v[b, h, j]
                        sum_now_kept += e_now
                        sum_cal_kept += e_cal
                    else:
                        num += e_cal * v_c[b, h, j]
                o[b, h, t] = num * sum_cal_kept / (sum_now_kept * sum_cal_all)
    return o


def kept_flops(idx, N, d, block=BLOCK):
    """Multiply-add work of one sparse step on the kept blocks, counted as
    4 * d * sum over query blocks of (rows of the block) * (kept keys)."""
    idx = np.asarray(idx)
    ranges = block_ranges(N, block)
    sizes = np.array([e - a for a, e in ranges], dtype=np.int64)
    total = 0
    for i, (a, e) in enumerate(ranges):
        total += (e - a) * sizes[idx[..., i, :]].sum()
    return 4 * d * int(total)
