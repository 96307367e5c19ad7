"""Test harness: device buffers for a synthetic workload, and a reference
replay of decode steps against the CPU oracle.

Replay protocol (after the pages' own consistency check, which replays the
same routing policy and compares outputs, actions and committed state): the
GPU trajectory drives.  Each step the oracle recomputes, from the same
inputs, every local output, the recall score from the GPU's h_prev / emb /
local output, the branch decision, every full output of the flagged
sequences, and the commit with the GPU's flags, and compares:
  * attention outputs   |gpu - oracle| <= 1e-2 + 1e-2 |oracle|
  * recall scores       |gpu - oracle| <= 1e-4 (1 + |oracle|)
  * flags               bit-exact unless |q_oracle - theta| < 1e-3
  * cache slot, h_prev, pos   bit-exact.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import synth
from oracle import (branch_rule, decode_attention, full_index_set, local_index_set, recall_score,
                    unpack_head)
import conditional_sparse_attention_amd as C
from conditional_sparse_attention_amd.step import StepBuffers, StepPlan

ATOL = RTOL = 1e-2
SCORE_TOL = 1e-4
TIE_BAND = 1e-3
DEV = "cuda"


def to_dev_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def from_dev_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def assert_close_bf16(gpu_bits: np.ndarray, ref: np.ndarray, what: str) -> None:
    gpu_bits, ref = np.asarray(gpu_bits), np.asarray(ref)
    if gpu_bits.size == 0 or gpu_bits.shape != ref.shape:
        raise AssertionError(f"{what}: nothing compared (gpu shape {gpu_bits.shape}, oracle shape {ref.shape})")
    g = synth.bf16_bits_to_f32(gpu_bits).astype(np.float64)
    err = np.abs(g - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    if np.any(bad):
        i = np.unravel_index(np.argmax(err - (ATOL + RTOL * np.abs(ref))), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst at {i}: "
                             f"gpu {g[i]} oracle {ref[i]}")


class Problem:
    """Device state of a workload: cache, step buffers, workspace, plan."""

    def __init__(self, wl: synth.Workload, *, theta: float = 0.0, head_perturb: bool = False,
                 device_fill: bool = False, lse: bool = True, host_cache: bool = True):
        self.wl = wl
        L, B, Hq, Hkv, d = wl.layers, wl.batch, wl.hq, wl.hkv, wl.head_dim
        self.paged = wl.layout == "paged"
        if self.paged:
            tables, nb = synth.paged_block_tables(wl)
            self.tables_np, self.num_blocks = tables, nb
            self.dims = C.make_dims(L, B, Hq, Hkv, kv_layout=C.ODA_KV_PAGED, block_size=wl.block_size,
                                    max_blocks_per_seq=tables.shape[1], num_blocks=nb,
                                    sink=wl.sink, window=wl.window)
            shape = (L, nb, Hkv, wl.block_size, d)
            self.tables = torch.from_numpy(tables).to(DEV)
        else:
            self.tables_np, self.tables = None, None
            self.dims = C.make_dims(L, B, Hq, Hkv, t_cap=wl.t_cap, sink=wl.sink, window=wl.window)
            shape = (L, B, Hkv, wl.t_cap, d)
        self.K = torch.zeros(shape, dtype=torch.int16, device=DEV)
        self.V = torch.zeros(shape, dtype=torch.int16, device=DEV)
        self.t0_dev = torch.from_numpy(wl.t0.astype(np.int32)).to(DEV)
        # host copy of the logical cache [L][B][Hkv][T][d] (small workloads only)
        self.host = None
        if host_cache:
            T = int(np.max(wl.t0)) + wl.steps
            self.host = {tag: np.zeros((L, B, Hkv, T, d), dtype=np.uint16) for tag in (synth.TAG_K, synth.TAG_V)}
            for tag in (synth.TAG_K, synth.TAG_V):
                for l in range(L):
                    for b in range(B):
                        for g in range(Hkv):
                            self.host[tag][l, b, g, :wl.t0[b]] = synth.cache_rows(wl, tag, l, b, g, 0, int(wl.t0[b]))
        if device_fill or not host_cache:
            import synth.device as sd
            for tag, buf in ((synth.TAG_K, self.K), (synth.TAG_V, self.V)):
                sd.fill_cache(buf, wl, tag, self.t0_dev, tables=self.tables, num_blocks=getattr(self, "num_blocks", 0))
        else:
            self._upload_cache()
        self.kv = C.make_kv(self.K, self.V, self.tables)
        nbytes = C.oda_workspace_bytes(self.dims)
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
        C.oda_workspace_init(self.dims, self.ws)
        self.blob = synth.head_blob(wl.hidden, wl.head_seed, perturb=head_perturb)
        self.head_P = None
        D = wl.hidden
        self.bufs = StepBuffers(
            pos=self.t0_dev.clone(),
            qL=torch.zeros((L, B, Hq, d), dtype=torch.int16, device=DEV),
            kL=torch.zeros((L, B, Hkv, d), dtype=torch.int16, device=DEV),
            vL=torch.zeros((L, B, Hkv, d), dtype=torch.int16, device=DEV),
            qF=torch.zeros((L, B, Hq, d), dtype=torch.int16, device=DEV),
            kF=torch.zeros((L, B, Hkv, d), dtype=torch.int16, device=DEV),
            vF=torch.zeros((L, B, Hkv, d), dtype=torch.int16, device=DEV),
            emb=torch.zeros((B, D), dtype=torch.int16, device=DEV),
            h_prev=to_dev_u16(synth.h_prev0(wl)),
            head_w=torch.from_numpy(self.blob).to(DEV),
            oL=torch.zeros((L, B, Hq, d), dtype=torch.int16, device=DEV),
            oF=torch.zeros((L, B, Hq, d), dtype=torch.int16, device=DEV),
            score=torch.zeros(B, dtype=torch.float32, device=DEV),
            flag=torch.zeros(B, dtype=torch.uint8, device=DEV),
            force=torch.full((B,), -1, dtype=torch.int8, device=DEV),
            lseL=torch.zeros((L, B, Hq), dtype=torch.float32, device=DEV) if lse else None,
            lseF=torch.zeros((L, B, Hq), dtype=torch.float32, device=DEV) if lse else None,
        )
        self.plan = StepPlan(self.dims, self.kv, self.ws, self.bufs, theta)

    def _upload_cache(self):
        wl = self.wl
        for tag, buf in ((synth.TAG_K, self.K), (synth.TAG_V, self.V)):
            host = self.host[tag]
            if not self.paged:
                arr = np.zeros(tuple(buf.shape), dtype=np.uint16)
                T = host.shape[3]
                arr[:, :, :, :T] = host
                buf.copy_(to_dev_u16(arr))
            else:
                arr = np.zeros(tuple(buf.shape), dtype=np.uint16)
                bs = wl.block_size
                for b in range(wl.batch):
                    n = int(wl.t0[b])
                    for p0 in range(0, n, bs):
                        blk = self.tables_np[b, p0 // bs]
                        p1 = min(p0 + bs, n)
                        arr[:, blk, :, :p1 - p0] = host[:, b, :, p0:p1]
                buf.copy_(to_dev_u16(arr))

    # ---------------------------------------------------------------- inputs
    def step_inputs(self, j: int) -> dict:
        wl = self.wl
        return {k: synth.step_tensor_all_layers(wl, k, j) for k in ("qL", "kL", "vL", "qF", "kF", "vF")} | \
            {"emb": synth.embedding(wl, j)}

    def upload_step(self, inp: dict) -> None:
        for k in ("qL", "kL", "vL", "qF", "kF", "vF"):
            getattr(self.bufs, k).copy_(to_dev_u16(inp[k]))
        self.bufs.emb.copy_(to_dev_u16(inp["emb"]))

    def set_force(self, force: np.ndarray) -> None:
        self.bufs.force.copy_(torch.from_numpy(np.asarray(force, dtype=np.int8)))

    # -------------------------------------------------------------- readback
    def cache_slot(self, l: int, b: int, p: int):
        """bf16 bits [2][Hkv][d] (K, V) of logical slot p."""
        if not self.paged:
            return (from_dev_u16(self.K[l, b, :, p]), from_dev_u16(self.V[l, b, :, p]))
        blk = int(self.tables_np[b, p // self.wl.block_size])
        r = p % self.wl.block_size
        return (from_dev_u16(self.K[l, blk, :, r]), from_dev_u16(self.V[l, blk, :, r]))

    def ws_error_word(self) -> int:
        return int(self.ws[:4].view(torch.int32).item())

    def worklist(self):
        off = C.oda_workspace_worklist_offset(self.dims)
        w = self.ws[off:].view(torch.int32)
        n = int(w[0].item())
        return decode_items(w[1:1 + n].cpu().numpy())

    def head_params(self):
        if self.head_P is None:
            self.head_P = unpack_head(self.blob, self.wl.hidden)
        return self.head_P


def full_nsplit(t: int, nflag: int, hkv: int, total: int = None) -> int:
    """Candidate A of the split policy stated in include/oda.h (one round):
    chunks of 1024 keys or more (at most 32 splits), cut finer, down to 256
    keys, while the F = nflag flagged sequences' Hkv heads would otherwise
    make fewer than 128 units; and at most the sequence's length-proportional
    share of one 256-unit round, floor(256 t / (total hkv)) but at least 1,
    where total is the flagged sequences' keys together (nflag * t when
    omitted: equal lengths)."""
    if total is None:
        total = nflag * t
    base = min(C.ODA_FULL_MAX_SPLITS, -(-t // C.ODA_FULL_MIN_CHUNK))
    per = nflag * hkv
    fine = min(C.ODA_FULL_MAX_SPLITS, -(-t // C.ODA_FULL_FINE_CHUNK), C.ODA_FULL_FILL_UNITS // per) if per else 0
    n = max(base, fine)
    if per and total > 0:
        share = (C.ODA_FULL_ROUND_UNITS * t) // (total * hkv)
        n = min(n, max(1, min(C.ODA_FULL_MAX_SPLITS, share)))
    return n


def full_nsplit_rounds(t: int, hkv: int, total: int) -> int:
    """Candidate B (several rounds): chunks of max(1024, ceil(total hkv /
    (4 * 256))) keys, at most 32 splits."""
    c = max(C.ODA_FULL_MIN_CHUNK, -(-total * hkv // (C.ODA_FULL_RAGGED_ROUNDS * C.ODA_FULL_ROUND_UNITS)))
    return max(1, min(C.ODA_FULL_MAX_SPLITS, -(-t // c)))


def full_splits(flags, ts, hkv: int) -> list:
    """Split counts of a step (0 for unflagged sequences): candidate B when
    its estimated time (include/oda.h) is below candidate A's, else A."""
    on = [int(f != 0) for f in flags]
    nflag = sum(on)
    total = sum(int(t) for f, t in zip(on, ts) if f)
    na = [full_nsplit(int(t), nflag, hkv, total) if f else 0 for f, t in zip(on, ts)]
    nb = [full_nsplit_rounds(int(t), hkv, total) if f else 0 for f, t in zip(on, ts)]

    R, K0 = C.ODA_FULL_ROUND_UNITS, C.ODA_FULL_UNIT_COST_KEYS

    def cost(ns):
        units = hkv * sum(ns)
        sizes = [-(-int(t) // n) for n, t in zip(ns, ts) if n > 0]
        longest, shortest = max(sizes, default=0), min(sizes, default=0)
        rounds = -(-units // R)
        even = -(-total * hkv // R) + (shortest if units > R else 0)
        return min(rounds * (longest + K0), max(even, longest) + rounds * K0)

    return nb if cost(nb) < cost(na) else na


def decode_items(items) -> list:
    """Work-list items (b << 20) | (nsplit << 10) | split as (b, nsplit, split)."""
    return [(int(x) >> 20, (int(x) >> 10) & 0x3FF, int(x) & 0x3FF) for x in items]


def want_worklist(flags, ts, hkv: int) -> list:
    """The oracle's work list (flagged sequences longest unit first, splits
    in order) for the split counts of the policy, as (b, nsplit, split)."""
    from oracle import full_worklist
    flags = [int(f != 0) for f in flags]
    ts = [int(t) for t in ts]
    ns = full_splits(flags, ts, hkv)
    return [(b, ns[b], s) for b, s in full_worklist(flags, ns, ts)]


def replay_step(pr: Problem, j: int, *, theta: float, force=None, check_layers=None, check_b=None,
                stats: dict = None) -> dict:
    """Run step j on the GPU, then check it against the oracle (small
    workloads with a host cache).  Returns per-step records."""
    wl = pr.wl
    L, B, Hq, Hkv, d = wl.layers, wl.batch, wl.hq, wl.hkv, wl.head_dim
    inp = pr.step_inputs(j)
    pr.upload_step(inp)
    if force is None:
        force = np.full(B, -1, dtype=np.int8)
    pr.set_force(force)
    pr.plan.set_theta(theta)
    pos_before = pr.bufs.pos.cpu().numpy().copy()
    h_prev_before = from_dev_u16(pr.bufs.h_prev)
    sentinel = np.full((L, B, Hq, d), 0x7FC1, dtype=np.uint16)  # NaN pattern: rows left untouched keep it
    pr.bufs.oF.copy_(to_dev_u16(sentinel))
    pr.plan.run()
    torch.cuda.synchronize()
    oL = from_dev_u16(pr.bufs.oL)
    oF = from_dev_u16(pr.bufs.oF)
    score = pr.bufs.score.cpu().numpy()
    flag = pr.bufs.flag.cpu().numpy()
    h_prev_after = from_dev_u16(pr.bufs.h_prev)
    pos_after = pr.bufs.pos.cpu().numpy()
    lseL = pr.bufs.lseL.cpu().numpy() if pr.bufs.lseL is not None else None
    assert pr.ws_error_word() == 0, "device error bits set"
    layers = range(L) if check_layers is None else check_layers
    bs = range(B) if check_b is None else check_b
    Kh, Vh = pr.host[synth.TAG_K], pr.host[synth.TAG_V]
    P = pr.head_params()
    # ---- local branch
    for l in layers:
        for b in bs:
            p = int(pos_before[b])
            ref = decode_attention(inp["qL"][l, b], Kh[l, b, :, :p], Vh[l, b, :, :p], inp["kL"][l, b],
                                   inp["vL"][l, b], local_index_set(p + 1, wl.sink, wl.window))
            assert_close_bf16(oL[l, b], ref, f"step {j} local l={l} b={b} pos={p}")
    # ---- score, rule
    for b in range(B):
        q = recall_score(P, h_prev_before[b], inp["emb"][b], oL[L - 1, b].reshape(-1))
        assert abs(float(score[b]) - q) <= SCORE_TOL * (1 + abs(q)), f"step {j} b={b}: score {score[b]} vs {q}"
        want = branch_rule(q, theta, int(force[b]))
        if force[b] >= 0 or abs(q - theta) >= TIE_BAND or not np.isfinite(q):
            assert int(flag[b]) == want, f"step {j} b={b}: flag {flag[b]} vs {want} (q={q}, theta={theta})"
        if stats is not None:
            stats.setdefault("q", []).append(q)
    # ---- work list
    assert pr.worklist() == want_worklist(flag, np.asarray(pos_before, np.int64) + 1, wl.hkv)
    # ---- full branch (flagged rows), untouched rows
    for b in range(B):
        if flag[b]:
            for l in layers:
                if b not in bs:
                    continue
                p = int(pos_before[b])
                ref = decode_attention(inp["qF"][l, b], Kh[l, b, :, :p], Vh[l, b, :, :p], inp["kF"][l, b],
                                       inp["vF"][l, b], full_index_set(p + 1))
                assert_close_bf16(oF[l, b], ref, f"step {j} full l={l} b={b} pos={p}")
        else:
            assert np.all(oF[:, b] == 0x7FC1), f"step {j}: full output of unflagged b={b} was written"
    # ---- commit (GPU flags drive), bit-exact
    assert np.array_equal(pos_after, pos_before + 1)
    for b in range(B):
        p = int(pos_before[b])
        chosen = "F" if flag[b] else "L"
        o_last = oF[L - 1, b] if flag[b] else oL[L - 1, b]
        assert np.array_equal(h_prev_after[b], o_last.reshape(-1)), f"step {j} b={b}: h_prev"
        for l in range(L):
            Kh[l, b, :, p] = inp["k" + chosen][l, b]
            Vh[l, b, :, p] = inp["v" + chosen][l, b]
            ks, vs = pr.cache_slot(l, b, p)
            assert np.array_equal(ks, Kh[l, b, :, p]) and np.array_equal(vs, Vh[l, b, :, p]), \
                f"step {j} l={l} b={b}: committed slot"
    return {"flag": flag.copy(), "score": score.copy(), "lseL": lseL}


class BigProblem:
    """A workload at full size: cache and per-step inputs filled on the
    device by the generator, no host copy of the cache.  The oracle checks
    sampled outputs, regenerating the rows it needs from G plus the slots
    committed by earlier steps (whose branch the recorded GPU flags give)."""

    def __init__(self, wl: synth.Workload, *, head_perturb: bool = False):
        import synth.device as sd
        self.sd = sd
        self.pr = Problem(wl, head_perturb=head_perturb, host_cache=False, lse=False)
        self.wl = wl
        self.flags = []      # GPU flags per step
        self.feed = {"qL": self.pr.bufs.qL, "qF": self.pr.bufs.qF, "kL": self.pr.bufs.kL, "vL": self.pr.bufs.vL,
                     "kF": self.pr.bufs.kF, "vF": self.pr.bufs.vF, "e": self.pr.bufs.emb}

    def reset(self) -> None:
        """Back to the state before step 0 (pos = t0, h_prev = its initial
        value).  Slots written by earlier passes lie at positions >= t0 and are
        rewritten by the new pass before any step reads them."""
        self.pr.bufs.pos.copy_(self.pr.t0_dev)
        self.pr.bufs.h_prev.copy_(to_dev_u16(synth.h_prev0(self.wl)))
        self.flags = []

    def calibrate_theta(self, steps: int, rate: float) -> float:
        """The benchmark's threshold for a target call rate: the steps run
        all-local (theta = +inf) and the threshold sends round(rate * B *
        steps) of their scores to the full branch; passes of the ODA step
        then re-tune it on its own trajectory (step.match_rate); the state
        is reset."""
        from conditional_sparse_attention_amd.step import match_rate, tune_theta
        B = self.wl.batch

        def run_pass(theta):
            self.reset()
            recs = [self.run_step(j, theta, np.full(B, -1, np.int8)) for j in range(steps)]
            return np.stack([r["score"] for r in recs]), np.stack([r["flag"] for r in recs])

        theta = match_rate(run_pass, tune_theta(run_pass(math.inf)[0], rate), rate)[0]
        self.reset()
        return theta

    def run_step(self, j: int, theta: float, force) -> dict:
        pr, wl = self.pr, self.wl
        pos_before = pr.bufs.pos.cpu().numpy().copy()
        assert np.all(pos_before == wl.t0 + j)
        self.sd.fill_step(self.feed, wl, pr.bufs.pos, pr.t0_dev)
        pr.set_force(force)
        pr.plan.set_theta(theta)
        h_prev_before = from_dev_u16(pr.bufs.h_prev)
        pr.bufs.oF.fill_(0x7FC1)
        pr.plan.run()
        torch.cuda.synchronize()
        rec = {"j": j, "pos": pos_before, "h_prev": h_prev_before, "oL": from_dev_u16(pr.bufs.oL),
               "oF": from_dev_u16(pr.bufs.oF), "score": pr.bufs.score.cpu().numpy().copy(),
               "flag": pr.bufs.flag.cpu().numpy().copy(), "worklist": pr.worklist(),
               "h_prev_after": from_dev_u16(pr.bufs.h_prev), "pos_after": pr.bufs.pos.cpu().numpy().copy(),
               "theta": theta, "force": np.asarray(force)}
        assert pr.ws_error_word() == 0
        self.flags.append(rec["flag"])
        return rec

    def history(self, l: int, b: int, g: int, j: int, rows: np.ndarray):
        """K, V bits [len(rows)][d] of logical positions `rows` as committed
        before step j."""
        return self._history(l, b, g, j, rows, self.flags, None)

    def _history(self, l, b, g, j, rows, flags, base):
        """As history(), with the GPU flags of steps < j given, and optionally
        a cached (lo, K, V) block of the initial cache covering the old rows."""
        wl = self.wl
        t0 = int(wl.t0[b])
        rows = np.asarray(rows, dtype=np.int64)
        K = np.zeros((len(rows), wl.head_dim), np.uint16)
        V = np.zeros_like(K)
        old = rows < t0
        if np.any(old):
            idx = np.nonzero(old)[0]
            r = rows[idx]
            if base is not None:
                lo, Kb, Vb = base
                assert r.min() >= lo and r.max() < lo + len(Kb)
                K[idx] = Kb[r - lo]
                V[idx] = Vb[r - lo]
            else:
                cuts = np.nonzero(np.diff(r) != 1)[0] + 1
                for seg_i, seg_r in zip(np.split(idx, cuts), np.split(r, cuts)):
                    lo, hi = int(seg_r[0]), int(seg_r[-1]) + 1
                    K[seg_i] = synth.cache_rows(wl, synth.TAG_K, l, b, g, lo, hi)
                    V[seg_i] = synth.cache_rows(wl, synth.TAG_V, l, b, g, lo, hi)
        for i in np.nonzero(~old)[0]:
            jj = int(rows[i]) - t0
            assert jj < j
            br = "F" if flags[jj][b] else "L"
            K[i] = synth.step_tensor(wl, "k" + br, jj, l)[b, g]
            V[i] = synth.step_tensor(wl, "v" + br, jj, l)[b, g]
        return K, V

    def check_step(self, rec: dict) -> None:
        """Every score, flag (outside the tie band), the work list, the
        untouched full rows of unflagged sequences, every h_prev and pos, and
        the committed slots of the first and the last layer."""
        wl, pr = self.wl, self.pr
        L, B = wl.layers, wl.batch
        j = rec["j"]
        P = pr.head_params()
        emb = synth.embedding(wl, j)
        flag = rec["flag"]
        for b in range(B):
            q = recall_score(P, rec["h_prev"][b], emb[b], rec["oL"][L - 1, b].reshape(-1))
            assert abs(float(rec["score"][b]) - q) <= SCORE_TOL * (1 + abs(q)), (j, b, rec["score"][b], q)
            f = int(rec["force"][b])
            if f >= 0 or abs(q - rec["theta"]) >= TIE_BAND:
                assert int(flag[b]) == branch_rule(q, rec["theta"], f), (j, b, q)
        assert rec["worklist"] == want_worklist(flag, np.asarray(rec["pos"], np.int64) + 1, wl.hkv)
        for b in range(B):
            if not flag[b]:
                assert np.all(rec["oF"][:, b] == 0x7FC1), "unflagged full rows written"
        assert np.array_equal(rec["pos_after"], rec["pos"] + 1)
        for b in range(B):
            o_last = rec["oF"][L - 1, b] if flag[b] else rec["oL"][L - 1, b]
            assert np.array_equal(rec["h_prev_after"][b], o_last.reshape(-1))
            p = int(rec["pos"][b])
            br = "F" if flag[b] else "L"
            for l in sorted({0, L - 1}):
                ks, vs = pr.cache_slot(l, b, p)
                assert np.array_equal(ks, synth.step_tensor(wl, "k" + br, j, l)[b])
                assert np.array_equal(vs, synth.step_tensor(wl, "v" + br, j, l)[b])

    def resolve_full(self, rec: dict, samples):
        """Full-branch samples of a step: (l, b, g) with an unflagged b is
        moved to the flagged sequence flagged[b % F]; none when F = 0."""
        flagged = [int(b) for b in np.nonzero(rec["flag"])[0]]
        out = []
        for (l, b, g) in samples:
            self._guard(l, b, g)
            if not flagged:
                continue
            out.append((l, b if rec["flag"][b] else flagged[b % len(flagged)], g))
        return out

    def _guard(self, l, b, g) -> None:
        wl = self.wl
        if not (0 <= l < wl.layers and 0 <= b < wl.batch and 0 <= g < wl.hkv):
            raise AssertionError(f"sample (l={l}, b={b}, g={g}) outside L={wl.layers}, B={wl.batch}, "
                                 f"Hkv={wl.hkv}")

    def check(self, rec: dict, samples, full_samples):
        """check_step(), then the attention outputs of the sampled (l, b, g)
        (local) and full_samples (full branch; see resolve_full).  Returns
        the numbers of local and full outputs compared."""
        self.check_step(rec)
        loc = []
        for (l, b, g) in samples:
            self._guard(l, b, g)
            loc.append((rec["j"], "L", l, b, g))
        full = [(rec["j"], "F", l, b, g) for (l, b, g) in self.resolve_full(rec, full_samples)]
        recs = {rec["j"]: rec}
        return (check_outputs(self, recs, loc, flags=self.flags, workers=1),
                check_outputs(self, recs, full, flags=self.flags, workers=1))


def check_outputs(bp: BigProblem, recs: dict, picks, *, flags, workers: int = None) -> int:
    """Attention outputs of `picks` = (j, kind, l, b, g), kind "L" or "F",
    against the oracle computed one by one from the regenerated history
    (the initial cache from G, later slots from the branch the GPU flags of
    earlier steps chose).  Picks are grouped by (l, b, g) so each history is
    generated once; groups run on a thread pool.  Returns the number of
    outputs compared (a full pick of an unflagged sequence is an error)."""
    import os
    from collections import defaultdict
    from concurrent.futures import ThreadPoolExecutor

    wl = bp.wl
    G = wl.hq // wl.hkv
    d = wl.head_dim
    by = defaultdict(list)
    for (j, kind, l, b, g) in picks:
        bp._guard(l, b, g)
        rec = recs[j]
        assert kind in ("L", "F")
        if kind == "F":
            assert rec["flag"][b], f"full sample of unflagged sequence {b} at step {j}"
        by[(l, b, g)].append((j, kind))

    def work(key):
        l, b, g = key
        items = sorted(set(by[key]))
        t0 = int(wl.t0[b])
        if any(k == "F" for _, k in items):
            lo, hi = 0, t0
        else:
            lo, hi = max(0, t0 - wl.window), t0
        # rows of the initial cache this group reads: all of them for a full
        # pick, else the sink and the last window before t0
        Kb = np.zeros((t0, d), np.uint16)
        Vb = np.zeros_like(Kb)
        have = np.zeros(t0, bool)
        for r0, r1 in ((0, min(wl.sink, t0)), (lo, hi)):
            if r1 > r0 and not have[r0:r1].all():
                Kb[r0:r1] = synth.cache_rows(wl, synth.TAG_K, l, b, g, r0, r1)
                Vb[r0:r1] = synth.cache_rows(wl, synth.TAG_V, l, b, g, r0, r1)
                have[r0:r1] = True
        n = 0
        for j, kind in items:
            rec = recs[j]
            p = int(rec["pos"][b])
            assert p == t0 + j
            S = local_index_set(p + 1, wl.sink, wl.window) if kind == "L" else full_index_set(p + 1)
            rows = S[S < p]
            assert have[rows[rows < t0]].all()
            K, V = bp._history(l, b, g, j, rows, flags, (0, Kb, Vb))
            Kh = np.zeros((1, p, d), np.uint16)
            Vh = np.zeros_like(Kh)
            Kh[0, rows] = K
            Vh[0, rows] = V
            qv = synth.step_tensor(wl, "q" + kind, j, l)[b, g * G:(g + 1) * G]
            kc = synth.step_tensor(wl, "k" + kind, j, l)[b, g:g + 1]
            vc = synth.step_tensor(wl, "v" + kind, j, l)[b, g:g + 1]
            ref = decode_attention(qv, Kh, Vh, kc, vc, S)
            got = (rec["oL"] if kind == "L" else rec["oF"])[l, b, g * G:(g + 1) * G]
            assert_close_bf16(got, ref, f"{wl.name} step {j} {kind} l={l} b={b} g={g} pos={p}")
            n += 1
        return n

    keys = sorted(by)
    if workers is None:
        workers = min(16, os.cpu_count() or 1)
    if workers <= 1 or len(keys) <= 1:
        return sum(work(k) for k in keys)
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return sum(ex.map(work, keys))
