"""GPU parity of the HIP path (through the C ABI) against the oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_diffusion_amd import configs, rettn, synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def small_cfg(name, **over):
    c = dict(configs.CONFIGS[name])
    c.update(over)
    return c


# ------------------------------------------------------------------ selector
def block_constant_inputs(B, H, N, D, seed, dtype):
    """q, k constant inside every 64-token block with small integer entries, so
    pooled means and pooled logits (scale 1/8 for d = 64) are exact in float32
    on both sides, with many exact ties."""
    g = torch.Generator().manual_seed(seed)
    nb = (N + 63) // 64
    out = []
    for _ in range(2):
        vals = torch.randint(-2, 3, (B, H, nb, D), generator=g).float()
        x = vals.repeat_interleave(64, dim=2)[:, :, :N]
        out.append(x.to(torch.bfloat16 if dtype == "bf16" else torch.float32))
    return out


@pytest.mark.parametrize("N,keep,forced,dtype", [
    (1000, 5, [0, 7], "bf16"), (256, 2, [], "f32"), (64 * 37 + 5, 9, [0, 1, 2, 3], "bf16"),
    (65536, 9, [0, 1, 2, 3], "bf16"), (640, 10, [], "bf16"), (130, 1, [2], "bf16"),
    # more than 32 non-forced winners: the bitonic-sort path (and every block kept in the second case)
    (64 * 100, 45, [3], "bf16"), (64 * 40, 40, [0], "bf16"), (64 * 600 + 17, 40, [], "bf16"),
    # 257..320 key blocks: five 64-block chunks per lane sorted in a 512-key buffer
    (64 * 278, 40, [0, 1, 2, 3], "bf16"), (64 * 300, 300, [], "bf16"), (64 * 260 + 5, 100, [5], "bf16"),
    (64 * 278 + 48 - 64, 9, [0, 1, 2, 3], "bf16"),
])
def test_selector_exact_on_exact_scores(N, keep, forced, dtype):
    say("selector exact", N, keep, forced, dtype)
    B, H, D = 1, 2, 64
    q, k = block_constant_inputs(B, H, N, D, seed=N, dtype=dtype)
    sh = rettn.shape(B, H, N, 64, D, keep, dtype)
    idx, scores = gu.select(sh, q.to(gu.DEV), k.to(gu.DEV), forced)
    ref_scores = oracle.pooled_scores(gu.host(q), gu.host(k), N, 64)
    assert np.array_equal(scores.cpu().numpy().astype(np.float64), ref_scores)
    ref = oracle.select_blocks(gu.host(q), gu.host(k), N, 64, keep, forced)
    assert np.array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("B,H,N,D,keep,forced,dtype", [
    (1, 2, 64 * 100, 80, 9, [3], "bf16"),                   # d_pad 80, two 64-block chunks, rounds
    (1, 2, 64 * 278 - 16, 80, 40, [0, 1, 2, 3], "bf16"),    # d_pad 80, five chunks, bitonic sort
    (1, 2, 64 * 600 + 17, 80, 40, [], "bf16"),              # d_pad 80 above 512 blocks, bitonic: two-wave launch
    (1, 2, 64 * 600 + 17, 80, 9, [0], "bf16"),              # d_pad 80 above 512 blocks, rounds
    (1, 2, 64 * 300, 64, 20, [], "f32"),                    # float32 inputs, five chunks
    (1, 2, 64 * 700 + 5, 80, 40, [1], "f32"),               # float32, d_pad 80, sixteen chunks, bitonic
    (1, 48, 64 * 278 - 16, 64, 9, [0, 1, 2, 3], "bf16"),    # two query blocks per wave
    (1, 96, 64 * 278 - 16, 64, 9, [0, 1, 2, 3], "bf16"),    # four query blocks per wave
    (1, 96, 64 * 278 - 16, 64, 40, [0, 1, 2, 3], "bf16"),   # four per wave, bitonic sort
])
def test_selector_instantiations_exact(B, H, N, D, keep, forced, dtype):
    """Bit-exact lists and scores, on exactly representable inputs, for the
    selector instantiations the workload shapes above do not reach: d_pad 80
    with several 64-block chunks (and the two-wave launch that the bitonic
    path needs above 512 key blocks), float32 inputs with several chunks, and
    two and four query blocks per wave (chosen by the workgroup count).  The
    true head dim is 64 (scale 1/8, exact); channels 64.. are zero."""
    say("selector instantiation", B, H, N, D, keep, forced, dtype)
    d = 64
    q, k = block_constant_inputs(B, H, N, D, seed=N + H, dtype=dtype)
    q[..., d:] = 0
    k[..., d:] = 0
    sh = rettn.shape(B, H, N, d, D, keep, dtype)
    idx, scores = gu.select(sh, q.to(gu.DEV), k.to(gu.DEV), forced)
    hq, hk = gu.host(q), gu.host(k)
    ref_scores = oracle.pooled_scores(hq, hk, N, d)
    assert np.array_equal(scores.cpu().numpy().astype(np.float64), ref_scores)
    ref = oracle.select_blocks(hq, hk, N, d, keep, forced, scores=ref_scores)
    assert np.array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("name", ["tiny", "pixart512", "pixart1024", "cogvideox2b"])
def test_selector_on_workload(name):
    say("selector workload", name)
    cfg = configs.CONFIGS[name]
    sh = rettn.shape_of(cfg)
    forced = configs.forced_blocks(cfg)
    (q, k, v), = gu.gpu_inputs(cfg, 1)
    idx, scores = gu.select(sh, q, k, forced)
    idx, scores = idx.cpu().numpy(), scores.cpu().numpy()
    # the GPU list is a valid top-k of the GPU's own exported scores
    B, H, nb, _ = idx.shape
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                assert gu.valid_topk(scores[b, h, i], idx[b, h, i], cfg["keep"], forced), (b, h, i)
    # against the oracle's float64 scores: disagreements only at near-ties
    ref_scores = oracle.pooled_scores(gu.host(q), gu.host(k), cfg["N"], cfg["d"])
    ref = oracle.select_blocks(None, None, cfg["N"], cfg["d"], cfg["keep"], forced, scores=ref_scores)
    n_diff = 0
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                a, r = set(idx[b, h, i]), set(ref[b, h, i])
                if a == r:
                    continue
                n_diff += 1
                tau = min(ref_scores[b, h, i, j] for j in r if j not in forced)
                for j in a ^ r:
                    assert abs(ref_scores[b, h, i, j] - tau) < 1e-5, (b, h, i, j)
    assert n_diff <= max(1, B * H * nb // 1000)


# ------------------------------------------------------------------ attention
def bf16_round(x):
    """float64 array rounded to bf16 (nearest even) and back, on the CPU."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()


def oracle_rows(variant, qh, kh, vh, rows, idx_row, st, r, N, d):
    """The oracle's reshape of one query block for variant "r1" or "r2"."""
    if variant == "r2":
        return oracle.sparse_reshape_rows_r2(qh, kh, vh, rows, idx_row, st["z_full"], st["z_sparse"], r, N, d)
    return oracle.sparse_reshape_rows(qh, kh, vh, rows, idx_row, st["m"], st["z_full"], st["z_sparse"], r, N, d)


def oracle_layer(variant):
    return oracle.sparse_reshape_r2 if variant == "r2" else oracle.sparse_reshape


def run_full_parity(cfg, steps_to_check, seed=0, residual="f32", variant=None):
    """Oracle lists fed to the GPU; calibrate at step 0, reshape at later steps;
    the full layer is compared.  With a bf16 residual cache the later steps are
    checked against the oracle fed its residual rounded to bf16 and against the
    exact oracle, both to the same tolerance."""
    sh = rettn.shape_of(cfg)
    N, d = cfg["N"], cfg["d"]
    forced = configs.forced_blocks(cfg)
    n_steps = max(steps_to_check) + 1
    stepsin = gu.gpu_inputs(cfg, n_steps, seed)
    q0, k0, v0 = stepsin[0]
    ref_idx = gu.oracle_lists(cfg, q0, k0, forced, cfg["keep"])
    idx = torch.as_tensor(ref_idx).to(gu.DEV)
    cache = rettn.StatsCache(sh, 1, residual=residual)
    o_cal = gu.calibrate(sh, q0, k0, v0, idx, cache)
    torch.cuda.synchronize()
    ref_cal = oracle.calibrate(gu.host(q0), gu.host(k0), gu.host(v0), ref_idx, N, d)
    ref_cal_stored = dict(ref_cal, r=bf16_round(ref_cal["r"])) if residual == "bf16" else ref_cal
    tol = dict(max_rel=1e-5, l1_rel=1e-6) if cfg["dtype"] == "f32" else {}
    res = {"calibrate": gu.assert_close(gu.host(o_cal), ref_cal["o"], what="calibrate O", **tol)}
    t = cache.tensors(0)
    assert np.array_equal(t["idx"].cpu().numpy(), ref_idx)
    assert np.abs(gu.host(t["m"]) - ref_cal["m"]).max() <= 1e-4 * max(1.0, np.abs(ref_cal["m"]).max())
    for zname in ("z_full", "z_sparse"):
        zr = np.abs(gu.host(t[zname]) / ref_cal[zname] - 1).max()
        assert zr <= 1e-4, (zname, zr)
    r_l1 = np.abs(gu.r_all(t["R"], sh) - ref_cal["r"]).sum() / max(1e-30, np.abs(ref_cal["r"]).sum())
    assert r_l1 <= 3e-3, r_l1
    for s in steps_to_check:
        q, k, v = stepsin[s]
        o = gu.sparse(sh, q, k, v, cache, variant=variant)
        torch.cuda.synchronize()
        ref_o = oracle_layer(variant)(gu.host(q), gu.host(k), gu.host(v), ref_idx, ref_cal, N, d)
        res[f"step{s}"] = gu.assert_close(gu.host(o), ref_o, what=f"step {s} O", **tol)
        if residual == "bf16":
            ref_s = oracle_layer(variant)(gu.host(q), gu.host(k), gu.host(v), ref_idx, ref_cal_stored, N, d)
            res[f"step{s}_stored"] = gu.assert_close(gu.host(o), ref_s, what=f"step {s} O (rounded R)", **tol)
    cache.close()
    return res


def test_parity_tiny_f32():
    say("parity tiny f32")
    run_full_parity(configs.CONFIGS["tiny"], [1])


def test_parity_pixart512():
    say("parity pixart512")
    run_full_parity(configs.CONFIGS["pixart512"], [1, 9])


def test_parity_pixart1024():
    say("parity pixart1024")
    run_full_parity(configs.CONFIGS["pixart1024"], [1, 19])


def run_sampled_parity(cfg, heads, seed=0, n_steps=2, check_steps=(1,), residual="f32", variant=None):
    """Full-size layers: the GPU runs every row; the oracle checks sampled query
    blocks (first, text/video boundary, middle, ragged last) of sampled heads."""
    sh = rettn.shape_of(cfg)
    N, d, keep = cfg["N"], cfg["d"], cfg["keep"]
    forced = configs.forced_blocks(cfg)
    nb = configs.n_blocks(N)
    it = synth.StepInputs(cfg, seed=seed, device=gu.DEV)
    q0, k0, v0 = (synth.store(x, cfg["dtype"]) for x in it.next())
    ref_idx = np.zeros((sh.B, sh.H, nb, keep), dtype=np.int32)
    hq, hk = {}, {}
    for b, h in heads:
        hq[b, h] = gu.host(q0[b, h][None, None])
        hk[b, h] = gu.host(k0[b, h][None, None])
    # oracle lists for every head (pooling is cheap), so the GPU input is all-oracle
    for b in range(sh.B):
        for h in range(sh.H):
            qq, kk = gu.host(q0[b, h][None, None]), gu.host(k0[b, h][None, None])
            ref_idx[b, h] = oracle.select_blocks(qq, kk, N, d, keep, forced)[0, 0]
    idx = torch.as_tensor(ref_idx).to(gu.DEV)
    cache = rettn.StatsCache(sh, 1, residual=residual)
    o_cal = gu.calibrate(sh, q0, k0, v0, idx, cache)
    torch.cuda.synchronize()
    t = cache.tensors(0)
    cal_host = {bh: [gu.host(x[bh[0], bh[1]]) for x in (q0, k0, v0)] for bh in heads}
    blocks = gu.sample_blocks(nb)
    refs = {}
    for (b, h) in heads:
        qh, kh, vh = cal_host[b, h]
        for i in blocks:
            rows = gu.block_rows(N, i)
            st = oracle.calibrate_rows(qh, kh, vh, rows, ref_idx[b, h, i], N, d)
            refs[b, h, i] = st
            gu.assert_close(gu.host(o_cal[b, h, rows]), st["o"], what=f"cal O b{b} h{h} blk{i}")
            assert np.abs(gu.host(t["m"][b, h, rows]) - st["m"]).max() <= 1e-4 * max(1, np.abs(st["m"]).max())
            assert np.abs(gu.host(t["z_full"][b, h, rows]) / st["z_full"] - 1).max() <= 1e-4
            assert np.abs(gu.host(t["z_sparse"][b, h, rows]) / st["z_sparse"] - 1).max() <= 1e-4
            rl1 = np.abs(gu.r_rows(t["R"], sh, b, h, rows) - st["r"]).sum() / np.abs(st["r"]).sum()
            assert rl1 <= 3e-3, rl1
    for s in range(1, n_steps):
        q, k, v = (synth.store(x, cfg["dtype"]) for x in it.next())
        if s not in check_steps:
            continue
        o = gu.sparse(sh, q, k, v, cache, variant=variant)
        torch.cuda.synchronize()
        for (b, h) in heads:
            qh, kh, vh = (gu.host(x[b, h]) for x in (q, k, v))
            for i in blocks:
                rows = gu.block_rows(N, i)
                st = refs[b, h, i]
                ro = oracle_rows(variant, qh, kh, vh, rows, ref_idx[b, h, i], st, st["r"], N, d)
                gu.assert_close(gu.host(o[b, h, rows]), ro, what=f"step {s} O b{b} h{h} blk{i}")
                if residual == "bf16":
                    rs = oracle_rows(variant, qh, kh, vh, rows, ref_idx[b, h, i], st, bf16_round(st["r"]), N, d)
                    gu.assert_close(gu.host(o[b, h, rows]), rs, what=f"step {s} O (rounded R) b{b} h{h} blk{i}")
    cache.close()


def host32(t):
    """A whole device tensor as a float32 host array (converted per head later)."""
    return t.detach().float().cpu().numpy()


def check_stats(t, sh, b, h, rows, st, where):
    m = gu.host(t["m"][b, h, rows])
    assert np.abs(m - st["m"]).max() <= 1e-4 * max(1.0, np.abs(st["m"]).max()), ("m", where)
    for zname in ("z_full", "z_sparse"):
        assert np.abs(gu.host(t[zname][b, h, rows]) / st[zname] - 1).max() <= 1e-4, (zname, where)
    r = gu.r_rows(t["R"], sh, b, h, rows)
    assert np.abs(r - st["r"]).sum() <= 3e-3 * max(1e-30, np.abs(st["r"]).sum()), ("R", where)


def test_parity_cogvideox2b_all_heads():
    """cogvideox2b at full size through its whole 50-step schedule.  The
    oracle's lists for every head drive a calibration at step 0; the oracle
    checks, on all 60 (b, h), the first, text/video boundary, first video,
    middle and ragged last query blocks at the calibration step and at steps
    1, 25 and 49, and every query block of two heads at steps 0 and 49."""
    say("parity cogvideox2b all heads")
    cfg = configs.CONFIGS["cogvideox2b"]
    sh = rettn.shape_of(cfg)
    N, d, keep = cfg["N"], cfg["d"], cfg["keep"]
    forced = configs.forced_blocks(cfg)
    nb = configs.n_blocks(N)
    full_heads = [(0, 0), (1, 29)]
    sampled = gu.sample_blocks(nb)
    units = sorted({(b, h, i) for b in range(sh.B) for h in range(sh.H) for i in sampled}
                   | {(b, h, i) for b, h in full_heads for i in range(nb)})
    full_only = {(b, h, i) for b, h in full_heads for i in range(nb)} - {(b, h, i) for b, h, i in units
                                                                          if i in sampled}
    it = synth.StepInputs(cfg, seed=0, device=gu.DEV)
    q0, k0, v0 = it.next_stored()
    hq, hk, hv = host32(q0), host32(k0), host32(v0)
    ref_idx = oracle.select_blocks(hq, hk, N, d, keep, forced)  # every head
    cache = rettn.StatsCache(sh, 1)
    o = gu.calibrate(sh, q0, k0, v0, torch.as_tensor(ref_idx).to(gu.DEV), cache)
    torch.cuda.synchronize()
    t = cache.tensors(0)
    assert np.array_equal(t["idx"].cpu().numpy(), ref_idx)
    ho = host32(o)
    refs = {}
    w = gu.Worst("cogvideox2b calibration")
    for b in range(sh.B):
        for h in range(sh.H):
            kh, vh = hk[b, h].astype(np.float64), hv[b, h].astype(np.float64)
            qh = hq[b, h].astype(np.float64)
            for i in (i for (bb, hh, i) in units if (bb, hh) == (b, h)):
                rows = gu.block_rows(N, i)
                st = oracle.calibrate_rows(qh, kh, vh, rows, ref_idx[b, h, i], N, d)
                refs[b, h, i] = st
                w.add(ho[b, h, rows], st["o"], (b, h, i))
                check_stats(t, sh, b, h, rows, st, (b, h, i))
    w.check()
    for s in range(1, 50):
        q, k, v = it.next_stored()
        if s not in (1, 25, 49):
            continue
        o = gu.sparse(sh, q, k, v, cache)
        torch.cuda.synchronize()
        hq, hk, hv, ho = host32(q), host32(k), host32(v), host32(o)
        w = gu.Worst(f"cogvideox2b step {s}")
        for b in range(sh.B):
            for h in range(sh.H):
                kh, vh = hk[b, h].astype(np.float64), hv[b, h].astype(np.float64)
                qh = hq[b, h].astype(np.float64)
                for (bb, hh, i) in units:
                    if (bb, hh) != (b, h) or (s != 49 and (b, h, i) in full_only):
                        continue
                    rows = gu.block_rows(N, i)
                    st = refs[b, h, i]
                    ro = oracle.sparse_reshape_rows(qh, kh, vh, rows, ref_idx[b, h, i], st["m"], st["z_full"],
                                                    st["z_sparse"], st["r"], N, d)
                    w.add(ho[b, h, rows], ro, (b, h, i))
        w.check()
    cache.close()


def test_parity_pixart1024_bf16_residual():
    say("parity pixart1024 bf16 residual")
    run_full_parity(configs.CONFIGS["pixart1024"], [1, 19], residual="bf16")


def test_parity_cogvideox2b_sampled_bf16_residual():
    say("parity cogvideox2b sampled bf16 residual")
    cfg = configs.CONFIGS["cogvideox2b"]
    run_sampled_parity(cfg, heads=[(0, 3), (1, 17)], n_steps=4, check_steps=(3,), residual="bf16")


# ------------------------------------------------------------------ reshape variant R2
def test_parity_tiny_f32_r2():
    say("parity tiny f32 r2")
    run_full_parity(configs.CONFIGS["tiny"], [1], variant="r2")


def test_parity_pixart1024_r2():
    say("parity pixart1024 r2")
    run_full_parity(configs.CONFIGS["pixart1024"], [1, 19], variant="r2")


def test_parity_pixart512_r2_bf16_residual():
    say("parity pixart512 r2 bf16 residual")
    run_full_parity(configs.CONFIGS["pixart512"], [1, 9], residual="bf16", variant="r2")


def test_parity_cogvideox2b_sampled_r2():
    say("parity cogvideox2b sampled r2")
    cfg = configs.CONFIGS["cogvideox2b"]
    run_sampled_parity(cfg, heads=[(0, 7), (1, 23)], n_steps=4, check_steps=(1, 3), variant="r2")


def test_parity_cogvideox2b_sampled_r2_bf16_residual():
    """The d_pad 64 sparse kernel with both options at once (R2 epilogue,
    residual cached in bf16), against the exact oracle and against the oracle
    fed the rounded residual."""
    say("parity cogvideox2b sampled r2 bf16 residual")
    cfg = configs.CONFIGS["cogvideox2b"]
    run_sampled_parity(cfg, heads=[(0, 11), (1, 5)], n_steps=3, check_steps=(2,), residual="bf16", variant="r2")


def test_r1_through_ex_is_the_default_entry_point():
    """rt_sparse_attn_reshape_ex with RT_RESHAPE_R1 is bit-identical to
    rt_sparse_attn_reshape; R2 on the calibration inputs gives dense attention
    (the calibration identity, which both readings satisfy)."""
    say("r1 through ex; r2 calibration identity")
    cfg = small_cfg("pixart1024", H=4)
    sh = rettn.shape_of(cfg)
    (q0, k0, v0), (q1, k1, v1) = gu.gpu_inputs(cfg, 2, seed=21)
    idx, _ = gu.select(sh, q0, k0, configs.forced_blocks(cfg))
    cache = rettn.StatsCache(sh, 1)
    gu.calibrate(sh, q0, k0, v0, idx, cache)
    a = gu.sparse(sh, q1, k1, v1, cache)
    b = gu.sparse(sh, q1, k1, v1, cache, variant="r1")
    o2 = gu.sparse(sh, q0, k0, v0, cache, variant="r2")
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    gu.assert_close(gu.host(o2), oracle.dense_attention(gu.host(q0), gu.host(k0), gu.host(v0), cfg["N"], cfg["d"]))
    cache.close()


def test_bf16_residual_is_rounded_f32():
    """A bf16-residual cache holds the float32 residual rounded to nearest even;
    O, m, Z_full, Z_sparse and the list copy equal those of a float32 cache."""
    say("bf16 residual = rounded f32 residual")
    cfg = small_cfg("cogvideox2b", H=3)
    sh = rettn.shape_of(cfg)
    (q, k, v), = gu.gpu_inputs(cfg, 1, seed=11)
    idx, _ = gu.select(sh, q, k, configs.forced_blocks(cfg))
    c32, c16 = rettn.StatsCache(sh, 1), rettn.StatsCache(sh, 1, residual="bf16")
    o32 = gu.calibrate(sh, q, k, v, idx, c32)
    o16 = gu.calibrate(sh, q, k, v, idx, c16)
    torch.cuda.synchronize()
    t32, t16 = c32.tensors(0), c16.tensors(0)
    assert t16["R"].dtype == torch.bfloat16 and t32["R"].dtype == torch.float32
    assert torch.equal(o32, o16)
    for name in ("m", "z_full", "z_sparse", "idx"):
        assert torch.equal(t32[name], t16[name]), name
    assert torch.equal(t16["R"], t32["R"].to(torch.bfloat16))
    c32.close()
    c16.close()


# ------------------------------------------------------------------ identities on the GPU
@pytest.mark.parametrize("name", ["pixart512", "pixart1024"])
def test_gpu_calibration_identity(name):
    """Calibrate then reshape on the same inputs gives dense attention."""
    say("calibration identity", name)
    cfg = configs.CONFIGS[name]
    sh = rettn.shape_of(cfg)
    (q, k, v), = gu.gpu_inputs(cfg, 1, seed=3)
    idx, _ = gu.select(sh, q, k, configs.forced_blocks(cfg))
    cache = rettn.StatsCache(sh, 1)
    gu.calibrate(sh, q, k, v, idx, cache)
    o = gu.sparse(sh, q, k, v, cache)
    torch.cuda.synchronize()
    dense = oracle.dense_attention(gu.host(q), gu.host(k), gu.host(v), cfg["N"], cfg["d"])
    gu.assert_close(gu.host(o), dense)


def test_gpu_keep_all_identity():
    """keep = Nb: zero residual, equal denominators, dense output at later steps."""
    say("keep-all identity")
    cfg = small_cfg("pixart512", H=4, keep=16)
    sh = rettn.shape_of(cfg)
    stepsin = gu.gpu_inputs(cfg, 4, seed=4)
    q0, k0, v0 = stepsin[0]
    idx, _ = gu.select(sh, q0, k0, [])
    assert np.array_equal(idx.cpu().numpy()[0, 0, 0], np.arange(16))
    cache = rettn.StatsCache(sh, 1)
    gu.calibrate(sh, q0, k0, v0, idx, cache)
    torch.cuda.synchronize()
    t = cache.tensors(0)
    assert float(t["R"].abs().max()) == 0.0
    assert torch.equal(t["z_full"], t["z_sparse"])
    q, k, v = stepsin[3]
    o = gu.sparse(sh, q, k, v, cache)
    torch.cuda.synchronize()
    gu.assert_close(gu.host(o), oracle.dense_attention(gu.host(q), gu.host(k), gu.host(v), cfg["N"], cfg["d"]))


@pytest.mark.parametrize("name", ["pixart512", "pixart1024"])
def test_sparse_kernel_with_oracle_cache(name):
    """The sparse kernel alone, fed statistics and lists made by the oracle."""
    say("sparse kernel with oracle cache", name)
    cfg = configs.CONFIGS[name]
    sh = rettn.shape_of(cfg)
    N, d = cfg["N"], cfg["d"]
    (q0, k0, v0), (q1, k1, v1) = gu.gpu_inputs(cfg, 2, seed=5)
    ref_idx = gu.oracle_lists(cfg, q0, k0, [], cfg["keep"])
    ref_cal = oracle.calibrate(gu.host(q0), gu.host(k0), gu.host(v0), ref_idx, N, d)
    cache = rettn.StatsCache(sh, 1)
    t = cache.tensors(0)
    for name_ in ("m", "z_full", "z_sparse"):
        t[name_].copy_(torch.as_tensor(ref_cal[name_], dtype=torch.float32))
    gu.r_fill(t["R"], sh, ref_cal["r"])
    t["idx"].copy_(torch.as_tensor(ref_idx))
    cache.set_valid(0)
    o = gu.sparse(sh, q1, k1, v1, cache)  # lists from the cache
    torch.cuda.synchronize()
    ref = oracle.sparse_reshape(gu.host(q1), gu.host(k1), gu.host(v1), ref_idx, ref_cal, N, d)
    gu.assert_close(gu.host(o), ref)
    o2 = gu.sparse(sh, q1, k1, v1, cache, idx=torch.as_tensor(ref_idx).to(gu.DEV))  # explicit lists
    torch.cuda.synchronize()
    assert torch.equal(o, o2)


# ------------------------------------------------------------------ edge cases
@pytest.mark.parametrize("N,d,D,keep,forced,dtype", [
    (64, 64, 64, 1, [], "bf16"),        # one block
    (40, 64, 64, 1, [], "bf16"),        # one short block
    (100, 64, 64, 2, [], "bf16"),       # keep all, ragged
    (200, 64, 64, 1, [3], "bf16"),      # only the forced (short, last) block kept
    (333, 72, 80, 3, [1], "bf16"),      # padded head dim, ragged
    (333, 8, 64, 2, [], "bf16"),        # tiny true head dim
    (130, 64, 64, 2, [0], "f32"),
    (333, 72, 80, 2, [], "f32"),
])
@pytest.mark.parametrize("variant", ["r1", "r2"])
def test_edge_shapes(N, d, D, keep, forced, dtype, variant):
    say("edge", N, d, D, keep, forced, dtype, variant)
    B, H = 2, 3
    q0, k0, v0 = synth.random_qkv(B, H, N, d, D, seed=N + d, scale=1.5, dtype=dtype, device=gu.DEV)
    q1, k1, v1 = synth.random_qkv(B, H, N, d, D, seed=N + d + 1, scale=1.5, dtype=dtype, device=gu.DEV)
    sh = rettn.shape(B, H, N, d, D, keep, dtype)
    ref_idx = oracle.select_blocks(gu.host(q0), gu.host(k0), N, d, keep, forced)
    idx, _ = gu.select(sh, q0, k0, forced)
    cache = rettn.StatsCache(sh, 1)
    o_cal = gu.calibrate(sh, q0, k0, v0, torch.as_tensor(ref_idx).to(gu.DEV), cache)
    o = gu.sparse(sh, q1, k1, v1, cache, variant=variant)
    torch.cuda.synchronize()
    ref_cal = oracle.calibrate(gu.host(q0), gu.host(k0), gu.host(v0), ref_idx, N, d)
    ref = oracle_layer(variant)(gu.host(q1), gu.host(k1), gu.host(v1), ref_idx, ref_cal, N, d)
    tol = dict(max_rel=1e-5, l1_rel=1e-6) if dtype == "f32" else {}
    gu.assert_close(gu.host(o_cal), ref_cal["o"], what="calibrate", **tol)
    gu.assert_close(gu.host(o), ref, what="sparse", **tol)
    if D > d:
        assert float(o[..., d:].abs().max()) == 0.0 and float(o_cal[..., d:].abs().max()) == 0.0
    # the GPU selector agrees with the oracle on these random inputs (no near-ties expected)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)


@pytest.mark.parametrize("keep", [9, 1024])
def test_maximum_sequence_length(keep):
    """N = 65536 (1024 key blocks, the largest supported), with a few kept
    blocks and with every block kept: selector lists against the oracle's on
    exactly representable scores is covered elsewhere; here the oracle's lists
    drive calibration and a later sparse step, checked on sampled query blocks
    (first, middle, last)."""
    say("maximum N", keep)
    B, H, N, d = 1, 1, 65536, 64
    nb = N // 64
    forced = [0]
    (q0, k0, v0), (q1, k1, v1) = (synth.random_qkv(B, H, N, d, d, seed=s, scale=1.0, dtype="bf16", device=gu.DEV)
                                  for s in (41, 42))
    sh = rettn.shape(B, H, N, d, d, keep, "bf16")
    ref_idx = oracle.select_blocks(gu.host(q0), gu.host(k0), N, d, keep, forced)
    cache = rettn.StatsCache(sh, 1)
    o_cal = gu.calibrate(sh, q0, k0, v0, torch.as_tensor(ref_idx).to(gu.DEV), cache)
    o = gu.sparse(sh, q1, k1, v1, cache)
    torch.cuda.synchronize()
    qh0, kh0, vh0 = (gu.host(x[0, 0]) for x in (q0, k0, v0))
    qh1, kh1, vh1 = (gu.host(x[0, 0]) for x in (q1, k1, v1))
    for i in (0, nb // 2, nb - 1):
        rows = gu.block_rows(N, i)
        st = oracle.calibrate_rows(qh0, kh0, vh0, rows, ref_idx[0, 0, i], N, d)
        gu.assert_close(gu.host(o_cal[0, 0, rows]), st["o"], what=f"calibrate blk{i}")
        ro = oracle.sparse_reshape_rows(qh1, kh1, vh1, rows, ref_idx[0, 0, i], st["m"], st["z_full"],
                                        st["z_sparse"], st["r"], N, d)
        gu.assert_close(gu.host(o[0, 0, rows]), ro, what=f"sparse blk{i}")
    cache.close()


@pytest.mark.parametrize("keep,variant", [(1, "r1"), (2, "r1"), (3, "r1"), (9, "r1"), (1, "r2"), (9, "r2")])
def test_sparse_many_blocks_per_workgroup(keep, variant):
    """The sparse kernel where each persistent workgroup walks several query
    blocks (so the prefetch of the next block's tiles, lists and rows crosses
    block boundaries), against the oracle's reshape on sampled query blocks.
    The statistics cache is synthetic: any positive Z_full >= Z_sparse, any m
    and any R give a well-defined reshape, and m spans values far below and
    above the new scores (exercising the lazy max from the cached reference)."""
    say("sparse many blocks per workgroup", keep, variant)
    B, H, d = 2, 16, 64
    N = 64 * 170 + 23  # ragged last block
    nb = (N + 63) // 64
    q, k, v = synth.random_qkv(B, H, N, d, d, seed=70 + keep, scale=1.5, dtype="bf16", device=gu.DEV)
    g = np.random.default_rng(keep)
    idx = np.stack([np.sort(g.choice(nb, keep, replace=False)) for _ in range(B * H * nb)])
    idx = idx.reshape(B, H, nb, keep).astype(np.int32)
    idx[0, 0, :, -1] = nb - 1  # the ragged block in every list of one head
    idx[0, 0] = np.sort(idx[0, 0], axis=-1)
    for a in range(nb):  # keep lists of distinct blocks
        row = np.unique(idx[0, 0, a])
        while len(row) < keep:
            row = np.unique(np.append(row, g.integers(nb)))
        idx[0, 0, a] = row
    m_c = g.uniform(-2.0, 6.0, (B, H, N))
    z_s = g.uniform(0.5, 2.0, (B, H, N))
    z_f = z_s * g.uniform(1.0, 4.0, (B, H, N))
    r_c = g.normal(0.0, 0.5, (B, H, N, d))
    sh = rettn.shape(B, H, N, d, d, keep, "bf16")
    cache = rettn.StatsCache(sh, 1)
    t = cache.tensors(0)
    t["m"].copy_(torch.as_tensor(m_c, dtype=torch.float32))
    t["z_full"].copy_(torch.as_tensor(z_f, dtype=torch.float32))
    t["z_sparse"].copy_(torch.as_tensor(z_s, dtype=torch.float32))
    gu.r_fill(t["R"], sh, r_c)
    t["idx"].copy_(torch.as_tensor(idx))
    cache.set_valid(0)
    o = gu.sparse(sh, q, k, v, cache, variant=variant)
    torch.cuda.synchronize()
    # the oracle reads the statistics as stored (float32)
    m32, zf32, zs32, r32 = (x.astype(np.float32) for x in (m_c, z_f, z_s, r_c))
    qh, kh, vh, oh = gu.host(q), gu.host(k), gu.host(v), gu.host(o)
    got, ref = [], []
    for b in range(B):
        for h in range(H):
            for a in list(g.choice(nb - 1, 3, replace=False)) + [nb - 1]:
                rows = slice(64 * a, min(64 * a + 64, N))
                st = {"m": m32[b, h, rows], "z_full": zf32[b, h, rows], "z_sparse": zs32[b, h, rows]}
                ref.append(oracle_rows(variant, qh[b, h], kh[b, h], vh[b, h], rows, idx[b, h, a], st,
                                       r32[b, h, rows], N, d))
                got.append(oh[b, h, rows])
    gu.assert_close(np.concatenate(got), np.concatenate(ref))


@pytest.mark.parametrize("variant,residual", [("r1", "f32"), ("r2", "f32"), ("r1", "bf16"), ("r2", "bf16")])
def test_sparse_rows_beyond_the_reference_range(variant, residual):
    """Rows whose scores rise far above the reference the first walk takes P
    against: the cached row max (R1; set 200 below the scores for one head) or
    the first listed tile's row max (R2; every list of six heads ends with a
    key block scaled by 40, whose scores exceed the first tile's by far more
    than float32 exponentials hold).  Those blocks overflow on the first walk
    and are walked again with the per-tile maximum; with several query blocks
    per workgroup the blocks after a redone one must come out right too.  All
    sampled blocks are compared with the oracle (fed the stored residual:
    rounded to bf16 where the cache holds it in bf16)."""
    say("sparse rows beyond the reference range", variant, residual)
    B, H, d, keep = 2, 16, 64, 5
    N = 64 * 170 + 23
    nb = (N + 63) // 64
    hot = nb - 3
    q, k, v = synth.random_qkv(B, H, N, d, d, seed=123, scale=1.0, dtype="bf16", device=gu.DEV)
    k[:, :6, hot * 64:(hot + 1) * 64] *= 40.0
    # rows 0 and 32 of every block (the first row of each wave) never leave the
    # range, so the test of a block must look at every row, not one per wave
    first_rows = (np.arange(N) % 32) == 0
    q[:, :6, torch.as_tensor(first_rows, device=q.device)] = 0
    g = np.random.default_rng(11)
    idx = np.empty((B, H, nb, keep), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                pool = np.delete(np.arange(nb), hot)
                row = g.choice(pool, keep - 1 if h < 6 else keep, replace=False)
                idx[b, h, i] = np.sort(np.append(row, hot) if h < 6 else row)
    m_c = g.uniform(-2.0, 6.0, (B, H, N))
    m_c[:, 7, ~first_rows] = -200.0
    z_s = g.uniform(0.5, 2.0, (B, H, N))
    z_f = z_s * g.uniform(1.0, 4.0, (B, H, N))
    r_c = g.normal(0.0, 0.5, (B, H, N, d))
    sh = rettn.shape(B, H, N, d, d, keep, "bf16")
    cache = rettn.StatsCache(sh, 1, residual=residual)
    t = cache.tensors(0)
    t["m"].copy_(torch.as_tensor(m_c, dtype=torch.float32))
    t["z_full"].copy_(torch.as_tensor(z_f, dtype=torch.float32))
    t["z_sparse"].copy_(torch.as_tensor(z_s, dtype=torch.float32))
    gu.r_fill(t["R"], sh, r_c)
    t["idx"].copy_(torch.as_tensor(idx))
    cache.set_valid(0)
    o = gu.sparse(sh, q, k, v, cache, variant=variant)
    torch.cuda.synchronize()
    m32, zf32, zs32, r32 = (x.astype(np.float32) for x in (m_c, z_f, z_s, r_c))
    if residual == "bf16":
        r32 = bf16_round(r_c)
    qh, kh, vh, oh = gu.host(q), gu.host(k), gu.host(v), gu.host(o)
    # the data does leave the range: scores of the hot block exceed those of a
    # list's first block by more than 88 (e^88 is near the float32 limit)
    s_first = qh[0, 0, :64] @ kh[0, 0, idx[0, 0, 0, 0] * 64:idx[0, 0, 0, 0] * 64 + 64].T / np.sqrt(d)
    s_hot = qh[0, 0, :64] @ kh[0, 0, hot * 64:(hot + 1) * 64].T / np.sqrt(d)
    assert (s_hot.max(axis=1) - s_first.max(axis=1)).max() > 88.0
    got, ref = [], []
    for b in range(B):
        for h in range(H):
            for a in list(g.choice(nb - 1, 3, replace=False)) + [0, nb - 1]:
                rows = slice(64 * a, min(64 * a + 64, N))
                st = {"m": m32[b, h, rows], "z_full": zf32[b, h, rows], "z_sparse": zs32[b, h, rows]}
                ref.append(oracle_rows(variant, qh[b, h], kh[b, h], vh[b, h], rows, idx[b, h, a], st,
                                       r32[b, h, rows], N, d))
                got.append(oh[b, h, rows])
    gu.assert_close(np.concatenate(got), np.concatenate(ref))

@pytest.mark.parametrize("residual", ["f32", "bf16"])
def test_calibration_rows_beyond_the_first_block_range(residual):
    """Calibration at d_pad 64 first takes P against the row max of key block
    0.  For six heads a key block late in the sequence is scaled by 20, so
    many rows score it more than 64 ln 2 above block 0 and their first-walk
    row sums pass 2^64: waves holding such rows walk again with the per-block
    maximum.  That block is in none of the six heads' lists, so Z_sparse of
    such rows can lie far below float32's normal range (their kept mass can be
    e^-100 of the row's); it is compared where the oracle's is at least 1e-30
    and must be tiny elsewhere.  Every third
    32-row group of those heads has q = 0 (all scores 0, never out of range),
    so workgroups mix waves that walk again with waves that keep their first
    walk.  Output and statistics of sampled query blocks are compared with the
    oracle, on the six heads and on two heads without the scaled block; with
    the residual cached in bf16 as well (R within the same L1 bound)."""
    say("calibration rows beyond the first block's range", residual)
    B, H, d, keep = 1, 8, 64, 5
    N = 64 * 150 + 41
    nb = (N + 63) // 64
    hot = nb - 4
    q, k, v = synth.random_qkv(B, H, N, d, d, seed=321, scale=1.0, dtype="bf16", device=gu.DEV)
    k[:, :6, hot * 64:(hot + 1) * 64] *= 20.0
    calm = (np.arange(N) // 32) % 3 == 0
    q[:, :6, torch.as_tensor(calm, device=q.device)] = 0
    # the scaled block is masked for the six heads: R carries it (a kept block
    # that dominates would leave R = all - kept to float32 cancellation)
    g = np.random.default_rng(5)
    others = np.delete(np.arange(nb), hot)
    idx = np.sort(np.stack([[[g.choice(others if h < 6 else nb, keep, replace=False) for _ in range(nb)]
                             for h in range(H)] for _ in range(B)]), axis=-1).astype(np.int32)
    sh = rettn.shape(B, H, N, d, d, keep, "bf16")
    cache = rettn.StatsCache(sh, 1, residual=residual)
    o = gu.calibrate(sh, q, k, v, torch.as_tensor(idx).to(gu.DEV), cache)
    torch.cuda.synchronize()
    t = cache.tensors(0)
    qh, kh, vh, oh = gu.host(q), gu.host(k), gu.host(v), gu.host(o)
    # the data does leave the first walk's range: a row sum of exponentials
    # against block 0's max passes 2^64 once a score exceeds that max by
    # 64 ln 2 (scores scaled by 1/sqrt(d))
    s0 = qh[0, 0, 32:64] @ kh[0, 0, :64].T / np.sqrt(d)
    s_hot = qh[0, 0, 32:64] @ kh[0, 0, hot * 64:(hot + 1) * 64].T / np.sqrt(d)
    assert (s_hot.max(axis=1) - s0.max(axis=1)).max() > 64 * np.log(2.0)
    w = gu.Worst("calibration beyond the first block's range")
    tiny = 0
    for h in range(H):
        for i in sorted({0, 1, 2, 3, nb // 2, hot, nb - 1} | set(g.choice(nb, 3, replace=False).tolist())):
            rows = gu.block_rows(N, i)
            st = oracle.calibrate_rows(qh[0, h], kh[0, h], vh[0, h], rows, idx[0, h, i], N, d)
            w.add(oh[0, h, rows], st["o"], (h, i))
            m = gu.host(t["m"][0, h, rows])
            assert np.abs(m - st["m"]).max() <= 1e-4 * max(1.0, np.abs(st["m"]).max()), ("m", h, i)
            assert np.abs(gu.host(t["z_full"][0, h, rows]) / st["z_full"] - 1).max() <= 1e-4, ("z_full", h, i)
            zs, ok = gu.host(t["z_sparse"][0, h, rows]), st["z_sparse"] >= 1e-30
            assert np.abs(zs[ok] / st["z_sparse"][ok] - 1).max(initial=0.0) <= 1e-4, ("z_sparse", h, i)
            assert np.all(zs[~ok] <= 1e-29), ("z_sparse tiny", h, i)
            tiny += int((~ok).sum())
            r = gu.r_rows(t["R"], sh, 0, h, rows)
            assert np.abs(r - st["r"]).sum() <= 3e-3 * max(1e-30, np.abs(st["r"]).sum()), ("R", h, i)
    w.check()
    print(f"[info] {tiny} rows with Z_sparse below 1e-30", flush=True)
    cache.close()


@pytest.mark.parametrize("dtype,D,d", [("bf16", 64, 64), ("bf16", 80, 72), ("f32", 64, 64)])
def test_repeated_list_entries_count_once(dtype, D, d):
    """A non-decreasing list with repeated entries is read as the set of its
    blocks by calibration and by both sparse epilogues (bf16 and float32), as
    by the oracle; the list copy in the cache keeps the repeats."""
    say("repeated list entries", dtype, D)
    B, H, N, keep = 1, 2, 64 * 20 + 7, 6
    nb = (N + 63) // 64
    g = np.random.default_rng(D)
    idx = np.empty((B, H, nb, keep), dtype=np.int32)
    for h in range(H):
        for i in range(nb):
            picks = np.sort(g.choice(nb, 3, replace=False))
            row = np.sort(np.concatenate([picks, g.choice(picks, keep - 3)]))  # 3 distinct blocks, 3 repeats
            idx[0, h, i] = row
    idx[0, 0, 0] = [nb - 1] * keep  # one block only, the short last one
    q0, k0, v0 = synth.random_qkv(B, H, N, d, D, seed=90, scale=1.5, dtype=dtype, device=gu.DEV)
    q1, k1, v1 = synth.random_qkv(B, H, N, d, D, seed=91, scale=1.5, dtype=dtype, device=gu.DEV)
    sh = rettn.shape(B, H, N, d, D, keep, dtype)
    cache = rettn.StatsCache(sh, 1)
    didx = torch.as_tensor(idx).to(gu.DEV)
    o_cal = gu.calibrate(sh, q0, k0, v0, didx, cache)
    outs = {var: gu.sparse(sh, q1, k1, v1, cache, variant=var) for var in ("r1", "r2")}
    torch.cuda.synchronize()
    assert np.array_equal(cache.tensors(0)["idx"].cpu().numpy(), idx)
    ref_cal = oracle.calibrate(gu.host(q0), gu.host(k0), gu.host(v0), idx, N, d)
    tol = dict(max_rel=1e-5, l1_rel=1e-6) if dtype == "f32" else {}
    gu.assert_close(gu.host(o_cal), ref_cal["o"], what="calibrate", **tol)
    t = cache.tensors(0)
    assert np.abs(gu.host(t["z_sparse"]) / ref_cal["z_sparse"] - 1).max() <= 1e-4
    # the sparse steps read the GPU's own float32 calibration (L1 error about
    # 1e-6 already), so the two-step chain is held to 3e-6 in float32
    tol2 = dict(max_rel=1e-5, l1_rel=3e-6) if dtype == "f32" else {}
    for var, o in outs.items():
        ref = oracle_layer(var)(gu.host(q1), gu.host(k1), gu.host(v1), idx, ref_cal, N, d)
        gu.assert_close(gu.host(o), ref, what=f"sparse {var}", **tol2)
    cache.close()


def test_deterministic_bitwise():
    say("determinism")
    cfg = small_cfg("pixart1024", H=4)
    sh = rettn.shape_of(cfg)
    (q0, k0, v0), (q1, k1, v1) = gu.gpu_inputs(cfg, 2, seed=6)
    outs = []
    for _ in range(2):
        idx, sc = gu.select(sh, q0, k0, [])
        cache = rettn.StatsCache(sh, 1)
        oc = gu.calibrate(sh, q0, k0, v0, idx, cache)
        o = gu.sparse(sh, q1, k1, v1, cache)
        torch.cuda.synchronize()
        t = cache.tensors(0)
        outs.append([idx, sc, oc, o, t["m"].clone(), t["z_full"].clone(), t["z_sparse"].clone(), t["R"].clone()])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


# ------------------------------------------------------------------ schedule through the ABI
def test_schedule_pixart512_through_attention_step():
    say("schedule pixart512")
    cfg = configs.CONFIGS["pixart512"]
    sh = rettn.shape_of(cfg)
    N, d = cfg["N"], cfg["d"]
    stepsin = gu.gpu_inputs(cfg, cfg["steps"], seed=7)
    cache = rettn.StatsCache(sh, 1)
    ws = torch.empty(rettn.step_workspace_bytes(sh), dtype=torch.uint8, device=gu.DEV)
    q0, k0, v0 = stepsin[0]
    ref_idx = gu.oracle_lists(cfg, q0, k0, [], cfg["keep"])
    ref_cal = None
    for s, (q, k, v) in enumerate(stepsin):
        o = gu.empty_out(sh)
        did = rettn.rt_attention_step(sh, q, k, v, [], cache, 0, s, 0, o, ws)
        torch.cuda.synchronize()
        assert did == (s == 0)
        if s == 0:
            gpu_idx = cache.tensors(0)["idx"].cpu().numpy()
            assert np.array_equal(gpu_idx, ref_idx)
            ref_cal = oracle.calibrate(gu.host(q), gu.host(k), gu.host(v), ref_idx, N, d)
            ref = ref_cal["o"]
        else:
            ref = oracle.sparse_reshape(gu.host(q), gu.host(k), gu.host(v), ref_idx, ref_cal, N, d)
        gu.assert_close(gu.host(o), ref, what=f"step {s}")


@pytest.mark.parametrize("variant", ["r1", "r2"])
def test_schedule_with_reselection(variant):
    """rt_attention_step_ex with per-step reselection: every step's lists are
    the selector's on that step's q and k (compared with the oracle's), the
    cached statistics stay those of step 0, and each sparse step equals the
    oracle's reshape over the new lists."""
    say("schedule pixart512 reselect", variant)
    cfg = configs.CONFIGS["pixart512"]
    sh = rettn.shape_of(cfg)
    N, d, keep = cfg["N"], cfg["d"], cfg["keep"]
    nb = configs.n_blocks(N)
    stepsin = gu.gpu_inputs(cfg, 4, seed=17)
    cache = rettn.StatsCache(sh, 1)
    ws = torch.empty(rettn.step_workspace_bytes(sh), dtype=torch.uint8, device=gu.DEV)
    off = rettn.select_workspace_bytes(sh)
    ref_cal, changed = None, False
    for s, (q, k, v) in enumerate(stepsin):
        o = gu.empty_out(sh)
        did = rettn.rt_attention_step_ex(sh, q, k, v, [], cache, 0, s, 0, variant, True, o, ws)
        torch.cuda.synchronize()
        assert did == (s == 0)
        ref_idx = gu.oracle_lists(cfg, q, k, [], keep)
        got_idx = ws[off: off + sh.B * sh.H * nb * keep * 4].view(torch.int32).cpu().numpy()
        assert np.array_equal(got_idx.reshape(ref_idx.shape), ref_idx), f"step {s} lists"
        if s == 0:
            ref_cal = oracle.calibrate(gu.host(q), gu.host(k), gu.host(v), ref_idx, N, d)
            ref = ref_cal["o"]
            cal_idx = ref_idx
        else:
            assert np.array_equal(cache.tensors(0)["idx"].cpu().numpy(), cal_idx)  # cache keeps step 0's lists
            ref = oracle_layer(variant)(gu.host(q), gu.host(k), gu.host(v), ref_idx, ref_cal, N, d)
            changed = changed or not np.array_equal(ref_idx, cal_idx)
        gu.assert_close(gu.host(o), ref, what=f"step {s}")
    assert changed  # the lists did move, so reselection was exercised
    cache.close()


def test_cogvideox5b_full_schedule():
    """cogvideox5b: 42 layers share one cache allocation (19.3 GB); layers 0 and
    41 run the whole 50-step schedule through rt_attention_step with
    recalibration (and reselection) every 10 steps.  At every recalibration
    (0, 10, 20, 30, 40), the step after it and step 49, the oracle checks all
    96 (b, h) on three query blocks each (the text/video boundary, a middle
    block that varies with the head, the ragged last): the GPU's lists equal
    the oracle's (else differ only at a near-tie, and the block is skipped),
    the calibration output and statistics, and the reshaped sparse outputs."""
    say("cogvideox5b full schedule")
    cfg = configs.CONFIGS["cogvideox5b"]
    sh = rettn.shape_of(cfg)
    N, d, keep, period = cfg["N"], cfg["d"], cfg["keep"], cfg["period"]
    forced = configs.forced_blocks(cfg)
    nb = configs.n_blocks(N)
    cache = rettn.StatsCache(sh, cfg["layers"])
    ws = torch.empty(rettn.step_workspace_bytes(sh), dtype=torch.uint8, device=gu.DEV)
    compare = {0, 1, 10, 11, 20, 21, 30, 31, 40, 41, 49}
    units = [(b, h, i) for b in range(sh.B) for h in range(sh.H)
             for i in (3, 5 + (17 * (b * sh.H + h)) % (nb - 6), nb - 1)]
    n_ties = 0
    for layer in (0, cfg["layers"] - 1):
        it = synth.StepInputs(cfg, seed=1000 + layer, device=gu.DEV)
        refs = {}
        for s in range(cfg["steps"]):
            q, k, v = it.next_stored()
            o = gu.empty_out(sh)
            did = rettn.rt_attention_step(sh, q, k, v, forced, cache, layer, s, period, o, ws)
            torch.cuda.synchronize()
            assert did == (s % period == 0)
            if s not in compare:
                continue
            hq, hk, hv, ho = host32(q), host32(k), host32(v), host32(o)
            w = gu.Worst(f"cogvideox5b layer {layer} step {s} ({'calibration' if did else 'sparse'})")
            if did:
                t = cache.tensors(layer)
                lists = t["idx"].cpu().numpy()
                ref_scores = oracle.pooled_scores(hq, hk, N, d)
                refs = {}
            for b in range(sh.B):
                for h in range(sh.H):
                    kh, vh = hk[b, h].astype(np.float64), hv[b, h].astype(np.float64)
                    qh = hq[b, h].astype(np.float64)
                    for (bb, hh, i) in units:
                        if (bb, hh) != (b, h):
                            continue
                        rows = gu.block_rows(N, i)
                        if did:
                            ref_list = oracle.select_from_scores(ref_scores[b, h, i], keep, forced)
                            if set(lists[b, h, i]) != set(ref_list):  # only a near-tie may differ
                                tau = min(ref_scores[b, h, i, j] for j in ref_list if j not in forced)
                                assert all(abs(ref_scores[b, h, i, j] - tau) < 1e-5
                                           for j in set(lists[b, h, i]) ^ set(ref_list)), (layer, s, b, h, i)
                                n_ties += 1
                                continue
                            st = oracle.calibrate_rows(qh, kh, vh, rows, ref_list, N, d)
                            refs[b, h, i] = (st, ref_list)
                            w.add(ho[b, h, rows], st["o"], (b, h, i))
                            check_stats(t, sh, b, h, rows, st, (layer, s, b, h, i))
                        elif (b, h, i) in refs:
                            st, ref_list = refs[b, h, i]
                            ro = oracle.sparse_reshape_rows(qh, kh, vh, rows, ref_list, st["m"], st["z_full"],
                                                            st["z_sparse"], st["r"], N, d)
                            w.add(ho[b, h, rows], ro, (b, h, i))
            w.check()
    print(f"[case] cogvideox5b: {n_ties} (layer, step, block) lists skipped at near-ties", flush=True)
    assert n_ties <= len(units)  # near-ties are rare
    views = [cache.tensors(layer) for layer in (0, 1, cfg["layers"] - 1)]
    assert views[0]["valid"] == 1 and views[1]["valid"] == 0 and views[2]["valid"] == 1
    assert not torch.equal(views[0]["m"], views[2]["m"])
    cache.close()


# ------------------------------------------------------------------ token order (Hilbert)
@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 80), ("f32", 64), ("f32", 80)])
def test_permute_rows_bit_exact(dtype, D):
    """rt_permute_rows gathers and scatters whole rows exactly like the oracle's
    fancy indexing, for the Hilbert order and for a random permutation; the
    inverse undoes the gather."""
    import oracle.hilbert as oh
    say("permute rows", dtype, D)
    B, H, N = 2, 3, 13 * 30 * 45 // 5 + 7
    x = synth.random_qkv(B, H, N, D, D, seed=D, scale=1.0, dtype=dtype, device=gu.DEV)[0]
    sh = rettn.shape(B, H, N, D, D, 1, dtype)
    rng = np.random.default_rng(D)
    for perm in (rettn.rt_hilbert_order((13, 6, 45), 7), rng.permutation(N).astype(np.int32)):
        pd = torch.as_tensor(perm).to(gu.DEV)
        y, z = torch.empty_like(x), torch.empty_like(x)
        rettn.rt_permute_rows(sh, x, y, pd)
        rettn.rt_permute_rows(sh, y, z, pd, inverse=True)
        torch.cuda.synchronize()
        raw = x.cpu().view(torch.int16 if dtype == "bf16" else torch.float32).numpy()  # bit patterns
        ref = torch.as_tensor(oh.permute_rows(raw, perm)).view(x.dtype)
        assert torch.equal(y.cpu(), ref)
        assert torch.equal(z, x)


@pytest.mark.parametrize("name", ["pixart1024", "cogvideox2b"])
def test_hilbert_ordered_layer(name):
    """A layer in Hilbert token order: Q, K, V reordered on the device, lists,
    calibration and a later sparse step in that order, output put back; the
    oracle does the same with its own order and reorder.  cogvideox2b is
    checked on sampled query blocks of two heads."""
    import oracle.hilbert as oh
    say("hilbert ordered layer", name)
    cfg = configs.CONFIGS[name] if name == "pixart1024" else small_cfg(name, H=2)
    sh = rettn.shape_of(cfg)
    N, d, keep = cfg["N"], cfg["d"], cfg["keep"]
    forced = configs.forced_blocks(cfg)
    perm = rettn.rt_hilbert_order(cfg["grid"][1:], cfg["n_text"])
    assert np.array_equal(perm, oh.token_order(cfg["grid"][1:], cfg["n_text"]))
    pd = torch.as_tensor(perm).to(gu.DEV)
    (q0, k0, v0), (q1, k1, v1) = gu.gpu_inputs(cfg, 2, seed=23)

    def reorder(t):
        out = torch.empty_like(t)
        rettn.rt_permute_rows(sh, t, out, pd)
        return out
    pq0, pk0, pv0, pq1, pk1, pv1 = (reorder(t) for t in (q0, k0, v0, q1, k1, v1))
    gpu_idx, _ = gu.select(sh, pq0, pk0, forced)
    # oracle: its own reorder of the stored inputs, then the method, then back
    hq0, hk0, hv0, hq1, hk1, hv1 = (oh.permute_rows(gu.host(t), perm) for t in (q0, k0, v0, q1, k1, v1))
    ref_scores = oracle.pooled_scores(hq0, hk0, N, d)
    ref_idx = oracle.select_blocks(None, None, N, d, keep, forced, scores=ref_scores)
    gi = gpu_idx.cpu().numpy()
    for b, h, i in zip(*np.nonzero((gi != ref_idx).any(axis=-1))):  # disagreements only at near-ties
        a, r = set(gi[b, h, i]), set(ref_idx[b, h, i])
        tau = min(ref_scores[b, h, i, j] for j in r if j not in forced)
        assert all(abs(ref_scores[b, h, i, j] - tau) < 1e-5 for j in a ^ r), (b, h, i)
    idx = torch.as_tensor(ref_idx).to(gu.DEV)
    cache = rettn.StatsCache(sh, 1)
    pcal = gu.calibrate(sh, pq0, pk0, pv0, idx, cache)
    psp = gu.sparse(sh, pq1, pk1, pv1, cache)
    o_cal, o_sp = torch.empty_like(pcal), torch.empty_like(psp)
    rettn.rt_permute_rows(sh, pcal, o_cal, pd, inverse=True)
    rettn.rt_permute_rows(sh, psp, o_sp, pd, inverse=True)
    torch.cuda.synchronize()
    if name == "pixart1024":
        ref_cal = oracle.calibrate(hq0, hk0, hv0, ref_idx, N, d)
        gu.assert_close(gu.host(o_cal), oh.permute_rows(ref_cal["o"], perm, inverse=True), what="calibrate")
        ref = oracle.sparse_reshape(hq1, hk1, hv1, ref_idx, ref_cal, N, d)
        gu.assert_close(gu.host(o_sp), oh.permute_rows(ref, perm, inverse=True), what="sparse")
    else:
        nb = configs.n_blocks(N)
        pos = np.empty_like(perm)
        pos[perm] = np.arange(N)  # position of each original token in the new order
        for b, h in ((0, 0), (1, 1)):
            for i in gu.sample_blocks(nb):
                rows = gu.block_rows(N, i)  # rows of the reordered sequence
                st = oracle.calibrate_rows(hq0[b, h], hk0[b, h], hv0[b, h], rows, ref_idx[b, h, i], N, d)
                orig = perm[rows]
                gu.assert_close(gu.host(o_cal[b, h, orig]), st["o"], what=f"cal b{b} h{h} blk{i}")
                ro = oracle.sparse_reshape_rows(hq1[b, h], hk1[b, h], hv1[b, h], rows, ref_idx[b, h, i], st["m"],
                                                st["z_full"], st["z_sparse"], st["r"], N, d)
                gu.assert_close(gu.host(o_sp[b, h, orig]), ro, what=f"sparse b{b} h{h} blk{i}")
    cache.close()
