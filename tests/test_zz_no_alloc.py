"""oda_local_attn_noalloc (for callers that cannot allocate: its scratch is a
fixed device array of the library) against oda_local_attn with a caller
workspace, through the C ABI.  Same kernels, so outputs and log-sum-exps
must match bit for bit.  Two calls in a row, the second with a smaller
input (fewer, shorter sequences, a paged cache, a larger group size), so
the shared scratch is reused with a different layout."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import conditional_sparse_attention_amd as C
    from _harness import Problem, from_dev_u16, to_dev_u16


def _wl(t0, *, layers, hq, hkv, layout, seed):
    t0 = np.asarray(t0, dtype=np.int64)
    return synth.Workload(f"noalloc-{hq}-{hkv}-{layout}", layers, hq, hkv, 128, len(t0), t0, 1, seed=seed,
                          head_seed=seed + 100, layout=layout, t_cap_slack=24)


def _compare(wl):
    pr = Problem(wl)
    inp = pr.step_inputs(0)
    L, B, Hq = wl.layers, wl.batch, wl.hq
    q, kc, vc = (to_dev_u16(inp[k]) for k in ("qL", "kL", "vL"))
    pos = pr.t0_dev.clone()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for l in range(L):
        out_ws = torch.zeros((B, Hq, 128), dtype=torch.int16, device="cuda")
        out_na = torch.full((B, Hq, 128), 0x7FC1, dtype=torch.int16, device="cuda")
        lse_ws = torch.zeros((B, Hq), dtype=torch.float32, device="cuda")
        lse_na = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
        C.oda_local_attn(pr.dims, l, pr.kv, pos, q[l], kc[l], vc[l], out_ws, lse_ws, pr.ws)
        C.oda_local_attn_noalloc(pr.dims, l, pr.kv, pos, q[l], kc[l], vc[l], out_na, lse_na, err)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev_u16(out_na), from_dev_u16(out_ws)), (wl.name, l)
        assert torch.equal(lse_na, lse_ws), (wl.name, l)
    assert int(err.item()) == 0
    assert pr.ws_error_word() == 0


def test_noalloc_local_attention_matches_workspace_entry_point():
    # first call: 6 sequences across t = 1, the s + w boundary and several
    # splits, two layers, 16/8 heads, contiguous cache
    _compare(_wl([0, 5, 2051, 2052, 3000, 6000], layers=2, hq=16, hkv=8, layout="contig", seed=61))
    # second call, smaller: 3 sequences, one layer, 32/8 heads (group 4), paged
    _compare(_wl([1, 700, 2500], layers=1, hq=32, hkv=8, layout="paged", seed=62))
