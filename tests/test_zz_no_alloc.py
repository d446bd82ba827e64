"""rt_select_blocks_noalloc (no workspace argument, pooled means in the
library's own device scratch) against rt_select_blocks with a caller
workspace: two calls in a row, the second on a smaller input, so that the
second runs over scratch holding the first call's means.  Lists and scores
must be bit-identical."""
import numpy as np
import pytest
import torch

from sparse_attention_diffusion_amd import configs, rettn
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _run_noalloc(sh, q, k, forced):
    nb = rettn.num_blocks(sh)
    idx = torch.full((sh.B, sh.H, nb, sh.keep), -1, dtype=torch.int32, device=gu.DEV)
    sc = torch.zeros((sh.B, sh.H, nb, nb), dtype=torch.float32, device=gu.DEV)
    rettn.rt_select_blocks_noalloc(sh, q, k, forced, idx, sc)
    return idx, sc


def test_noalloc_selector_equals_workspace_selector():
    torch.cuda.init()
    cases = []
    for name in ("cogvideox5b", "pixart512"):  # the second call is the smaller one
        cfg = configs.CONFIGS[name]
        sh = rettn.shape_of(cfg)
        assert rettn.select_workspace_bytes(sh) <= rettn.SELECT_SCRATCH_BYTES
        (q, k, _v), = gu.gpu_inputs(cfg, 1, seed=31)
        cases.append((name, sh, q, k, configs.forced_blocks(cfg)))
    got = []
    for name, sh, q, k, forced in cases:  # two allocation-free calls in a row
        print("[case] noalloc", name, flush=True)
        got.append(_run_noalloc(sh, q, k, forced))
    torch.cuda.synchronize()
    for (name, sh, q, k, forced), (idx, sc) in zip(cases, got):
        ref_idx, ref_sc = gu.select(sh, q, k, forced)
        assert torch.equal(idx, ref_idx), name
        assert torch.equal(sc, ref_sc), name
        # and the lists are valid top-k lists of those scores (spot check)
        i_np, s_np = idx.cpu().numpy(), sc.cpu().numpy()
        for b, h, i in ((0, 0, 0), (sh.B - 1, sh.H - 1, i_np.shape[2] - 1)):
            assert gu.valid_topk(s_np[b, h, i], i_np[b, h, i], sh.keep, forced)
