"""Reference replay of the trajectories the benchmark times, at full size.

The pages validate their implementation by replaying the same routing
policy and comparing actions, outputs and committed state
([On-Demand Attention notes §3.3, last paragraph; §4]).  Here the policy is
the benchmark's: the workload's random Xavier head, every decision taken by
the head, and the threshold tuned to the workload's call rate on an
all-local calibration pass over the same steps and then re-tuned on the ODA
step's own trajectory until it sends that share of the decisions to the
full branch (41.6% for the 16K batch of 8, 12.5% for the 128K batch of 4
with its far needles, 47% for the Qwen3-8B-shaped 64K batch of 16).  The GPU trajectory drives; for each of
8 steps the oracle checks

  * every recall score, every flag outside the tie band, the work list, the
    untouched full rows of unflagged sequences, every h_prev and pos, and
    the committed slots of the first and last layer;
  * local outputs: every (sequence, KV group) of the last layer, and a
    stride of earlier layers (a rotating KV group per sequence);
  * full outputs: every KV group of the last layer for every flagged
    sequence (the 64K batch of 16: its first four flagged sequences, one
    rotating group for the rest), and the layer stride.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from _harness import BigProblem, check_outputs

STEPS = 8
ALL_GROUPS_MAX = {2: 8, 3: 4, 4: 4}   # flagged sequences per step checked in every KV group


def stride_layers(L: int):
    return list(range(0, L - 1, max(1, L // 4)))


@pytest.fixture(scope="module", params=[2, 3, 4], ids=["w2-16k-b8", "w3-128k-b4", "w4-8b-64k-b16"])
def trajectory(request):
    key = request.param
    wl = synth.workloads()[key].replace(steps=STEPS)
    print(f"\n{wl.name}: calibrating theta for rate {wl.rate}", flush=True)
    bp = BigProblem(wl)
    theta = bp.calibrate_theta(STEPS, wl.rate)
    recs = {}
    for j in range(STEPS):
        rec = bp.run_step(j, theta, np.full(wl.batch, -1, np.int8))
        bp.check_step(rec)
        recs[j] = rec
        print(f"{wl.name} step {j}: theta {theta:.6f} flags {rec['flag'].tolist()}", flush=True)
    flags = list(bp.flags)
    # the checks below need only host records: release the device state
    bp.pr = None
    torch.cuda.empty_cache()
    yield key, wl, bp, recs, flags
    del bp, recs


def test_tuned_rate(trajectory):
    key, wl, bp, recs, flags = trajectory
    fl = np.array(flags)
    n = int(fl.sum())
    k = round(wl.rate * fl.size)
    print(f"{wl.name}: {n} of {fl.size} decisions full (target {wl.rate}: {k})", flush=True)
    # the trajectory exercises both branches, at the rate the threshold was tuned to
    assert 0 < n < fl.size
    assert abs(n - k) <= 1 + k // 20


def test_tuned_local_outputs(trajectory):
    key, wl, bp, recs, flags = trajectory
    L, B, Hkv = wl.layers, wl.batch, wl.hkv
    picks = [(j, "L", L - 1, b, g) for j in range(STEPS) for b in range(B) for g in range(Hkv)]
    picks += [(j, "L", l, b, (j + b + l) % Hkv) for j in range(STEPS) for b in range(B) for l in stride_layers(L)]
    n = check_outputs(bp, recs, picks, flags=flags)
    print(f"{wl.name}: {n} local outputs compared", flush=True)
    assert n == len(set(picks))


def _full_picks(key, wl, recs, layers_of):
    picks = []
    for j in range(STEPS):
        flagged = [int(b) for b in np.nonzero(recs[j]["flag"])[0]]
        for i, b in enumerate(flagged):
            for (l, gs) in layers_of(j, b, i):
                picks += [(j, "F", l, b, g) for g in gs]
    return picks


def test_tuned_full_outputs_last_layer(trajectory):
    key, wl, bp, recs, flags = trajectory
    L, Hkv = wl.layers, wl.hkv
    cap = ALL_GROUPS_MAX[key]
    picks = _full_picks(key, wl, recs, lambda j, b, i: [(L - 1, range(Hkv) if i < cap else [(j + b) % Hkv])])
    n = check_outputs(bp, recs, picks, flags=flags)
    print(f"{wl.name}: {n} full outputs of the last layer compared", flush=True)
    assert n == len(set(picks)) and n > 0


def test_tuned_full_outputs_layer_stride(trajectory):
    key, wl, bp, recs, flags = trajectory
    L, Hkv = wl.layers, wl.hkv
    cap = ALL_GROUPS_MAX[key]
    picks = _full_picks(key, wl, recs, lambda j, b, i: [(l, [(j + b + l) % Hkv]) for l in stride_layers(L)]
                        if i < cap else [])
    n = check_outputs(bp, recs, picks, flags=flags)
    print(f"{wl.name}: {n} full outputs of layers {stride_layers(L)} compared", flush=True)
    assert n == len(set(picks)) and n > 0
