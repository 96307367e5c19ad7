"""The C-ABI library loads, exports every symbol include/*.h declares,
answers host-only queries, and rejects bad arguments before launching
anything (these calls return before any device work, so they run on CPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

import conditional_sparse_attention_amd as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            src = open(os.path.join(ROOT, "include", h)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(oda_[a-z_]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(C.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = C.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_host_queries():
    assert C.oda_abi_version() == 1
    assert C.oda_head_param_count(2048) == 28325889   # the page's head size
    assert C.oda_head_param_count(0) == -1
    offs = C.oda_head_offsets(2048)
    assert offs[-1] == 28325889 and offs[0] == 0 and all(o % 4 == 0 for o in offs[:-1])


def test_head_offsets_agree_with_oracle_layout():
    from oracle import head_layout
    import numpy as np
    for D in (2048, 4096):
        offs = C.oda_head_offsets(D)
        sizes = [int(np.prod(s)) for _, s in head_layout(D)]
        assert offs == list(np.concatenate([[0], np.cumsum(sizes)]))


def test_workspace_and_dims_validation():
    ok = C.make_dims(28, 4, 16, 8, t_cap=131072 + 384)
    assert C.oda_workspace_bytes(ok) > 0
    bad = [
        C.make_dims(28, 33, 16, 8, t_cap=100),     # batch > 32
        C.make_dims(28, 4, 16, 8, head_dim=64, t_cap=100),
        C.make_dims(28, 4, 16, 6, t_cap=100),      # 16 % 6
        C.make_dims(28, 4, 64, 8, t_cap=100),      # G = 8 unsupported
        C.make_dims(0, 4, 16, 8, t_cap=100),
        C.make_dims(28, 4, 16, 8, t_cap=0),
        C.make_dims(28, 4, 16, 8, kv_layout=C.ODA_KV_PAGED, block_size=12, max_blocks_per_seq=4, num_blocks=8),
    ]
    for d in bad:
        with pytest.raises(C.OdaError):
            C.oda_workspace_bytes(d)


def test_entry_points_reject_bad_arguments_without_launching():
    lib = C.lib()
    d = C.make_dims(2, 2, 16, 8, t_cap=64)
    kv = C.oda_kv(None, None, None)
    ws_bytes = C.oda_workspace_bytes(d)
    dp, kp = ctypes.byref(d), ctypes.byref(kv)
    assert lib.oda_local_attn(dp, 0, kp, *([None] * 7), ws_bytes, None) == C.ODA_E_NULL
    assert lib.oda_full_attn_if(dp, 0, kp, *([None] * 7), ws_bytes, None) == C.ODA_E_NULL
    fake = 0x1000
    kv2 = C.oda_kv(fake, fake, None)
    args = (fake,) * 5  # pos, q, k_cur, v_cur, out
    assert lib.oda_local_attn(dp, 2, ctypes.byref(kv2), *args, None, fake, ws_bytes, None) == C.ODA_E_LAYER
    assert lib.oda_local_attn(dp, -1, ctypes.byref(kv2), *args, None, fake, ws_bytes, None) == C.ODA_E_LAYER
    assert lib.oda_local_attn(dp, 0, ctypes.byref(kv2), *args, None, fake, ws_bytes - 1, None) == C.ODA_E_WORKSPACE
    assert lib.oda_recall_score(dp, *([None] * 4), ctypes.c_float(0), *([None] * 5), ws_bytes, None) == C.ODA_E_NULL
    assert lib.oda_commit(dp, kp, *([None] * 10), ws_bytes, None) == C.ODA_E_NULL
    assert lib.oda_workspace_init(dp, None, ws_bytes, None) == C.ODA_E_NULL
    assert lib.oda_local_ranges(None, fake, fake, None) == C.ODA_E_NULL
    assert C.status_str(C.ODA_E_WORKSPACE).startswith("workspace")
    # alignment: 16 bytes for bf16 / float arrays and the workspace, 4 for int32 and lse
    odd = fake + 2
    k2 = ctypes.byref(kv2)
    assert lib.oda_local_attn(dp, 0, k2, fake, odd, fake, fake, fake, None, fake, ws_bytes, None) == C.ODA_E_ALIGN
    assert lib.oda_full_attn_if(dp, 0, k2, fake, fake, fake, fake, odd, None, fake, ws_bytes, None) == C.ODA_E_ALIGN
    assert lib.oda_local_attn(dp, 0, k2, *args, odd, fake, ws_bytes, None) == C.ODA_E_ALIGN
    assert lib.oda_local_attn(dp, 0, k2, *args, None, fake + 8, ws_bytes, None) == C.ODA_E_ALIGN
    assert lib.oda_local_attn(dp, 0, ctypes.byref(C.oda_kv(fake + 4, fake, None)), *args, None, fake, ws_bytes,
                              None) == C.ODA_E_ALIGN
    assert lib.oda_recall_score(dp, fake, odd, fake, fake, ctypes.c_float(0), None, fake, fake, fake, fake, ws_bytes,
                                None) == C.ODA_E_ALIGN
    assert lib.oda_recall_score(dp, fake, fake, fake, fake, ctypes.c_float(0), None, fake + 1, fake, fake, fake,
                                ws_bytes, None) == C.ODA_E_ALIGN
    assert lib.oda_commit(dp, k2, fake, fake, *([fake] * 6), odd, fake, ws_bytes, None) == C.ODA_E_ALIGN
    assert lib.oda_worklist(dp, fake, fake, fake + 4, ws_bytes, None) == C.ODA_E_ALIGN
    assert lib.oda_workspace_init(dp, fake + 4, ws_bytes, None) == C.ODA_E_ALIGN
    assert lib.oda_local_ranges(dp, fake + 2, fake, None) == C.ODA_E_ALIGN
    assert lib.oda_local_attn_noalloc(dp, 0, k2, *args, None, fake + 2, None) == C.ODA_E_ALIGN
    assert "aligned" in C.status_str(C.ODA_E_ALIGN)
    # the variant without a workspace: the same argument checks, and dims
    # whose split partials exceed the library's fixed scratch are refused
    assert lib.oda_local_attn_noalloc(dp, 0, kp, *([None] * 7), None) == C.ODA_E_NULL
    assert lib.oda_local_attn_noalloc(dp, 2, ctypes.byref(kv2), *args, None, None, None) == C.ODA_E_LAYER
    big = C.make_dims(1, 32, 64, 16, t_cap=64)   # 32 * 16 pairs x 16 splits x G 4 x 528 B = 17.3 MB
    assert 32 * 16 * 16 * 4 * 528 > C.ODA_NOALLOC_SCRATCH_BYTES
    assert lib.oda_local_attn_noalloc(ctypes.byref(big), 0, ctypes.byref(kv2), *args, None, None,
                                      None) == C.ODA_E_WORKSPACE


def test_decoder_layout_agrees_with_oracle_and_generator():
    """The library's layer blob offsets, the oracle's own layout statement
    and the generator's tensor list describe the same blob."""
    import numpy as np
    import synth
    from oracle import decoder as D
    for key in ("qwen3-1.7b", "tiny"):
        sh = synth.decoder_shapes()[key]
        dd = C.make_dec_dims(C.make_dims(sh.layers, 4, sh.hq, sh.hkv, t_cap=8192), sh.inter, sh.vocab,
                             sh.rope_theta, sh.eps)
        offs = C.oda_dec_layer_offsets(dd)
        lay = D.layer_layout(sh.hidden, sh.hq, sh.hkv, sh.head_dim, sh.inter)
        sizes = [int(np.prod(s)) for _, s in lay]
        assert offs == [0] + list(np.cumsum(sizes))
        assert C.oda_dec_layer_numel(dd) == D.layer_param_count(sh.hidden, sh.hq, sh.hkv, sh.head_dim, sh.inter)
        assert [n for n, _ in synth.dec_layer_tensors(sh)] == [n for n, _ in lay]


def test_decoder_rejects_bad_arguments_before_launching():
    import synth
    sh = synth.decoder_shapes()["tiny"]
    ok = C.make_dims(sh.layers, 4, sh.hq, sh.hkv, t_cap=8192)
    assert C.oda_dec_workspace_bytes(C.make_dec_dims(ok, sh.inter, sh.vocab)) > 0
    for inter, vocab in ((1000, sh.vocab), (sh.inter, 4000), (0, sh.vocab)):
        with pytest.raises(C.OdaError):
            C.oda_dec_workspace_bytes(C.make_dec_dims(ok, inter, vocab))
    dd = C.make_dec_dims(ok, sh.inter, sh.vocab)
    lib = C.lib()
    assert lib.oda_dec_layer(ctypes.byref(dd), 0, 2, None, None, None, None, None, None, None, None, None, 0, None,
                             0, None) == C.ODA_E_DIMS
    assert lib.oda_dec_layer(ctypes.byref(dd), 5, 0, None, None, None, None, None, None, None, None, None, 0, None,
                             0, None) == C.ODA_E_LAYER
    assert lib.oda_dec_layer(ctypes.byref(dd), 0, 0, None, None, None, None, None, None, None, None, None, 0, None,
                             0, None) == C.ODA_E_NULL
    assert lib.oda_dec_next_token(ctypes.byref(dd), None, None, None, None, None, None, None, 0, None) == C.ODA_E_NULL


def test_train_entry_points_reject_bad_arguments_before_launching():
    ok = C.make_train_dims(40, 2048, 151936)
    assert C.oda_train_workspace_bytes(ok) > 0
    for bad in (C.make_train_dims(0, 2048, 100), C.make_train_dims(70000, 2048, 100), C.make_train_dims(8, 100, 100),
                C.make_train_dims(8, 2048, 0), C.make_train_dims(8, 2048, 100, lam=-0.5)):
        with pytest.raises(C.OdaError):
            C.oda_train_workspace_bytes(bad)
    lib = C.lib()
    td = ctypes.byref(ok)
    fake = 1 << 20                          # never dereferenced: every call below returns before launching
    assert lib.oda_train_labels(td, None, fake, fake, fake, fake, fake, fake, fake, fake, 1 << 40, None) == C.ODA_E_NULL
    assert lib.oda_train_labels(td, fake + 2, fake, fake, fake, fake, fake, fake, fake, fake, 1 << 40,
                                None) == C.ODA_E_DIMS                    # lm_head not 16-byte aligned
    assert lib.oda_train_labels(td, fake, fake, fake, fake, fake, fake, fake, fake, fake, 0, None) == C.ODA_E_WORKSPACE
    args = [fake] * 13
    assert lib.oda_train_head_step(td, *args[:-1], None, 0, None) == C.ODA_E_NULL
    assert lib.oda_train_head_step(td, fake + 4, *args[1:], 1 << 40, None) == C.ODA_E_DIMS
    assert lib.oda_train_head_step(td, *args, 0, None) == C.ODA_E_WORKSPACE


def test_gdn_entry_points_reject_bad_arguments_before_launching():
    gd = C.make_gdn_dims(18, 8, 16)
    L, B, H, d, W = 18, 8, 16, 128, 4
    assert C.oda_gdn_state_bytes(gd) == L * B * 3 * H * d * d * 4 + L * B * 3 * (W - 1) * 3 * H * d * 2
    assert C.oda_gdn_conv_offset(gd) == L * B * 3 * H * d * d * 4
    for bad in (C.make_gdn_dims(18, 8, 16, head_dim=64), C.make_gdn_dims(18, 8, 16, conv_width=1),
                C.make_gdn_dims(0, 8, 16), C.make_gdn_dims(18, 0, 16), C.make_gdn_dims(18, 8, 65)):
        with pytest.raises(C.OdaError):
            C.oda_gdn_state_bytes(bad)
    lib = C.lib()
    g = ctypes.byref(gd)
    fake = 1 << 20
    f7 = [fake] * 7
    assert lib.oda_gdn_step(g, 0, 0, None, fake, None, *f7[:5], None) == C.ODA_E_NULL
    assert lib.oda_gdn_step(g, 0, 2, fake, fake, fake, *f7[:5], None) == C.ODA_E_DIMS
    assert lib.oda_gdn_step(g, 0, 1, fake, fake, None, *f7[:5], None) == C.ODA_E_NULL    # FULL needs flags
    assert lib.oda_gdn_step(g, 18, 0, fake, fake, None, *f7[:5], None) == C.ODA_E_LAYER
    assert lib.oda_gdn_step(g, 0, 0, fake + 8, fake, None, *f7[:5], None) == C.ODA_E_DIMS  # state not 16-byte aligned
    assert lib.oda_gdn_commit(g, None, fake, None) == C.ODA_E_NULL


def test_split_policy_constants_and_properties():
    """The binding's split-policy constants are the header's, and the policy
    the work-list tests expect keeps its stated properties: between 1 and 32
    splits, none empty; never more units than one round (256) unless a
    single split already makes more; never fewer splits than 1024-key
    chunks give (capped at 32) unless those would overflow the round; more
    only while the launch holds at most 128 units and then at most
    ceil(t / 256); sample values by hand."""
    from _harness import full_nsplit
    src = open(os.path.join(ROOT, "include", "oda.h")).read()
    for name in ("ODA_FULL_MIN_CHUNK", "ODA_FULL_FINE_CHUNK", "ODA_FULL_FILL_UNITS", "ODA_FULL_ROUND_UNITS",
                 "ODA_FULL_MAX_SPLITS", "ODA_FULL_RAGGED_ROUNDS", "ODA_FULL_UNIT_COST_KEYS"):
        m = re.search(r"#define\s+%s\s+(\d+)" % name, src)
        assert m and int(m.group(1)) == getattr(C, name), name
    ts = sorted(set([1, 2, 255, 256, 257, 1023, 1024, 1025, 2052, 4096, 4097, 9000, 16384, 32769, 131072, 262144]
                    + list(range(1, 70000, 997))))
    for hkv in (1, 2, 4, 8, 16):
        for nflag in (1, 2, 3, 5, 8, 16, 32):
            per = nflag * hkv
            for t in ts:
                n = full_nsplit(t, nflag, hkv)
                base = min(32, -(-t // 1024))
                chunk = -(-t // n)
                assert 1 <= n <= 32, (t, nflag, hkv, n)
                assert (n - 1) * chunk < t, (t, nflag, hkv, n)       # the last split is not empty
                assert per * n <= 256 or n == 1, (t, nflag, hkv, n)
                if per * base <= 256:
                    assert n >= base, (t, nflag, hkv, n)
                else:
                    assert n == max(1, 256 // per), (t, nflag, hkv, n)
                if n > base:
                    assert per * n <= 128 and -(-t // 256) >= n, (t, nflag, hkv, n)
    assert [full_nsplit(4096, f, 8) for f in (1, 2, 3, 4, 5)] == [16, 8, 5, 4, 4]
    assert [full_nsplit(t, 1, 8) for t in (1, 300, 8192, 16384, 131072)] == [1, 2, 16, 16, 32]
    assert [full_nsplit(131072, f, 8) for f in (1, 2, 3, 4, 32)] == [32, 16, 10, 8, 1]
    assert full_nsplit(16384, 3, 8) == 10 and full_nsplit(131072, 32, 16) == 1
    assert full_nsplit(4096, 1, 2) == 16 and full_nsplit(20000, 1, 2) == 32
    # the step's split counts: candidate A (one round) unless candidate B
    # (chunks of at least 1024 keys, four rounds' worth of units) costs less
    # in rounds x longest unit; every split non-empty
    from _harness import full_splits, full_nsplit_rounds
    rng = np.random.default_rng(3)
    for _ in range(300):
        hkv = int(rng.choice([2, 4, 8]))
        F = int(rng.integers(1, 33))
        ts = [int(t) for t in np.rint(np.exp(rng.uniform(np.log(1), np.log(262144), F)))]
        T = sum(ts)
        ns = full_splits([1] * F, ts, hkv)
        na = [full_nsplit(t, F, hkv, T) for t in ts]
        nb = [full_nsplit_rounds(t, hkv, T) for t in ts]
        assert ns in (na, nb)
        for t, n in zip(ts, ns):
            assert 1 <= n <= 32 and (n - 1) * -(-t // n) < t, (t, n)
        for t, n in zip(ts, nb):   # B: chunks of at least 1024 keys, so no split is tiny
            assert n == 1 or -(-t // n) >= min(1024, t) // 2
    # equal lengths that fill one round exactly keep A; three 128K sequences
    # (one round of 10 splits would leave units 6% longer than even) take B
    assert full_splits([1], [131073], 8) == [32]
    assert full_splits([1, 1], [131073] * 2, 8) == [16, 16]
    assert full_splits([1] * 3, [131073] * 3, 8) == [32] * 3
    assert full_splits([1] * 8, [16385] * 8, 8) == [4] * 8
    assert full_splits([1], [4097], 8) == [16]
    # a ragged mix: units handed out largest first to 256 workgroups finish
    # within 15% of the even share of all keys (one split per sequence per
    # head-round would leave the longest unit 40% over it)
    import heapq
    ts = [124661, 4388, 33000, 9000, 60000, 15000, 5000, 90000]
    ns = full_splits([1] * 8, ts, 8)
    units = sorted([-(-t // n) for t, n in zip(ts, ns) for _ in range(8 * n)], reverse=True)
    loads = [0] * 256
    for u in units:
        heapq.heapreplace(loads, loads[0] + u)
    even = sum(ts) * 8 / 256
    assert max(loads) <= 1.15 * even, (max(loads), even)
    na = [full_nsplit(t, 8, 8, sum(ts)) for t in ts]
    assert max(-(-t // n) for t, n in zip(ts, na)) > 1.4 * even

