"""The five synthetic attention workloads this library is exercised on.

They are shaped after the text-to-image and text-to-video DiTs the Re-ttention
project page evaluates on (PixArt and CogVideoX, page "Re-ttention: Ultra Sparse
Visual Generation via Attention Statistical Reshape", section Abstract).  No
model weights are involved: only the attention shapes, the sparsity level
(about 3.1% of key blocks kept, Abstract) and a denoising schedule.

Fields
------
B, H, N      batch (2 = classifier-free-guidance pair), heads, tokens
d, d_pad     true head dim (sets the softmax scale) and the stored/padded dim
keep         kept key blocks per query block, forced blocks included
grid         ("image", Hg, Wg) or ("video", T, Hg, Wg) latent token grid
n_text       text tokens placed in front of the latent tokens
dtype        "f32" or "bf16" storage of Q, K, V and O
steps        denoising steps in one schedule
period       recalibration period (None = calibrate at step 0 only)
layers       attention layers, each with its own statistics cache
"""

BLOCK = 64

CONFIGS = {
    "tiny": dict(B=1, H=2, N=256, d=64, d_pad=64, keep=2, grid=("image", 16, 16), n_text=0,
                 dtype="f32", steps=2, period=None, layers=1),
    "pixart512": dict(B=2, H=16, N=1024, d=72, d_pad=80, keep=2, grid=("image", 32, 32), n_text=0,
                      dtype="bf16", steps=10, period=None, layers=1),
    "pixart1024": dict(B=2, H=16, N=4096, d=72, d_pad=80, keep=4, grid=("image", 64, 64), n_text=0,
                       dtype="bf16", steps=20, period=None, layers=1),
    "cogvideox2b": dict(B=2, H=30, N=17776, d=64, d_pad=64, keep=9, grid=("video", 13, 30, 45), n_text=226,
                        dtype="bf16", steps=50, period=None, layers=1),
    "cogvideox5b": dict(B=2, H=48, N=17776, d=64, d_pad=64, keep=9, grid=("video", 13, 30, 45), n_text=226,
                        dtype="bf16", steps=50, period=10, layers=42),
}

ORDER = ["tiny", "pixart512", "pixart1024", "cogvideox2b", "cogvideox5b"]


def n_blocks(N, block=BLOCK):
    return (N + block - 1) // block


def forced_blocks(cfg, block=BLOCK):
    """Key blocks that hold at least one text token; they are always kept."""
    nt = cfg["n_text"]
    return list(range(n_blocks(nt, block))) if nt > 0 else []


def grid_tokens(cfg):
    g = cfg["grid"]
    n = 1
    for s in g[1:]:
        n *= s
    return n


def check(cfg):
    assert grid_tokens(cfg) + cfg["n_text"] == cfg["N"], cfg
    assert cfg["d"] <= cfg["d_pad"]
    assert 1 <= cfg["keep"] <= n_blocks(cfg["N"])
    assert len(forced_blocks(cfg)) <= cfg["keep"]
    return cfg


for _c in CONFIGS.values():
    check(_c)
