"""Parity of the HIP path with the oracle on the full-size workloads (the
shapes and launch configuration bench.py times), on sampled outputs.

Every step checks all recall scores, flags (outside the tie band), the work
list, every h_prev and pos, the committed slots of the first and last
layer, and the attention outputs of sampled (layer, sequence, KV group)
triples against the oracle computed one by one.  A full-branch sample whose
sequence the step did not flag is moved to a flagged one; a sample outside
the workload's shape, or a comparison of nothing, fails.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from _harness import BigProblem


def run_workload(key, steps_force, samples, full_samples, *, perturb=True):
    wl = synth.workloads()[key]
    wl = wl.replace(steps=len(steps_force) + 1)
    bp = BigProblem(wl, head_perturb=perturb)
    for j, (theta, force) in enumerate(steps_force):
        rec = bp.run_step(j, theta, force)
        n_loc, n_full = bp.check(rec, samples(wl, j), full_samples(wl, j))
        assert n_loc >= 1 and (n_full >= 1 or not np.any(rec["flag"]))
        print(f"{wl.name} step {j}: flags {rec['flag'].tolist()}, {n_loc} local and {n_full} full outputs "
              f"compared", flush=True)
    del bp
    torch.cuda.empty_cache()


def _force(B, full=(), local=()):
    f = np.full(B, -1, np.int8)
    f[list(full)] = 1
    f[list(local)] = 0
    return f


def test_workload2_16k_b8():
    B = 8
    steps = [(0.0, _force(B, full=[0, 5])), (0.0, _force(B, full=[2], local=[0, 1])), (0.0, _force(B))]
    run_workload(2, steps,
                 lambda wl, j: [(27, j % B, 3), (13, (j + 3) % B, 7), (0, 1, 0)],
                 lambda wl, j: [(27, 0, 1), (27, 2, 6), (5, 5, 4), (27, 3, 0)])


def test_workload3_128k_b4_needles():
    B = 4
    # step 0 is needle-aligned: the full branch must find the far needle
    steps = [(0.0, _force(B, full=[1])), (0.0, _force(B, full=[3], local=[1])), (0.0, _force(B))]
    run_workload(3, steps,
                 lambda wl, j: [(27, j % B, 2), (3, 2, 5)],
                 lambda wl, j: [(27, 1, 3), (27, 3, 0), (10, 0, 7)])


def test_workload4_8b_64k_b16():
    B = 16
    steps = [(0.0, _force(B, full=[0, 9, 15])), (0.0, _force(B))]
    run_workload(4, steps,
                 lambda wl, j: [(35, j, 2), (0, 15, 7)],
                 lambda wl, j: [(35, 0, 1), (35, 9, 6), (17, 15, 0)])


def test_workload5_ragged_paged_b32():
    wl5 = synth.workloads()[5]
    B = wl5.batch
    longest = int(np.argmax(wl5.t0))
    shortest = int(np.argmin(wl5.t0))
    steps = [(0.0, np.where(np.arange(B) % 2 == 1, synth.bernoulli_force(wl5, 0), -1).astype(np.int8)),
             (0.0, _force(B, full=[longest, shortest]))]
    run_workload(5, steps,
                 lambda wl, j: [(27, longest, 3), (27, shortest, 5), (0, 7, 0)],
                 lambda wl, j: [(27, longest, 1), (27, shortest, 2), (6, 1, 7), (27, 3, 4)])


def test_workload5_4k_subbatch():
    B = 32
    steps = [(0.0, _force(B, full=list(range(0, B, 3)))), (0.0, _force(B))]
    run_workload("5-4k", steps,
                 lambda wl, j: [(27, 31, 3), (0, 0, 0)],
                 lambda wl, j: [(27, 0, 1), (27, 3, 6)])


def test_workload5_4k_all_flagged_whole_sequence_units():
    """Every sequence of the paged 4K batch flagged: 32 sequences x 8 KV heads
    fill the 256-unit round, so each sequence is a single split (whole
    sequence per unit, no partial merge)."""
    B = 32
    steps = [(0.0, _force(B, full=range(B)))]
    run_workload("5-4k", steps,
                 lambda wl, j: [(27, 31, 3)],
                 lambda wl, j: [(27, 0, 1), (13, 17, 4), (27, 31, 7)])


def test_paged_units_longer_than_one_table_window():
    """A paged cache of 2-row blocks with all 32 sequences flagged at 20K
    positions: the policy makes each (sequence, KV head) one unit of 20,001
    keys (10,001 blocks), more block-table entries than the full kernel's
    shared-memory copy holds at once (3,072 with 8 waves), so each unit is
    streamed in four windows of entries, the last one ragged."""
    B = 32
    t0 = np.full(B, 20000, dtype=np.int64)
    wl = synth.Workload("paged-20k-b32-block2", 2, 16, 8, 128, B, t0, 2, seed=61, head_seed=161, layout="paged",
                        block_size=2)
    bp = BigProblem(wl, head_perturb=True)
    rec = bp.run_step(0, 0.0, _force(B, full=range(B)))
    assert [ns for (_, ns, _) in rec["worklist"]] == [1] * B
    n_loc, n_full = bp.check(rec, [(1, 3, 2), (0, 30, 7)], [(1, 0, 0), (1, 31, 5), (0, 17, 3)])
    assert n_loc >= 2 and n_full >= 3
    print(f"{wl.name}: {n_loc} local and {n_full} full outputs compared", flush=True)
    del bp
    torch.cuda.empty_cache()
