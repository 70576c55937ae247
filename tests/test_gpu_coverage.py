"""GPU parity for accepted inputs the other suites leave out, each against
the CPU oracle element by element (with sentinel checks on the rows that are
not valid), plus exact pins that need no oracle:

  * attn_mask of rank 1, 2 and 3 and batch-broadcast rank-4 masks, in bool,
    f16 and f32, through the LDS-staged and the per-lane mask paths (onnx-
    tensorrt "TensorRT Custom Operator Schemas", TRT_Attention inputs: a mask
    of rank at most 4, broadcast to the attention shape);
  * lower_right causal attention with 0 < kv_len < q_len, whose first
    q_len - kv_len rows see no key and must come out as exact zeros;
  * exact-gather probes: one-hot keys and exactly representable values make
    softmax pick one key per row, so each output row must equal one V row
    bit for bit -- which row depends on every ragged offset, head map and
    causal alignment (2 x 2 forms x 3 causal kinds x f16 / bf16);
  * tree decoding with 128 drafts (TensorRT Edge-LLM "TensorRT Plugins
    Guide", AttentionPlugin: tree decoding; its INT4 GEMM section speaks of
    draft trees of 64 to 128 tokens), and NaN rows past the 128th draft;
  * split-KV outputs of |O| ~ 8 (f16 at D = 64 and 128);
  * the GQA_ATTN_VALIDATE=1 device-side length check;
  * the tile map read from per-workgroup records (written by the plan kernel
    into the workspace) against the map each workgroup builds itself (no
    workspace): bitwise equal outputs, and equal to the oracle.
"""
import dataclasses
import itertools
import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest
import torch

from gqa_attention_ragged_amd import capi, synth
from tests import parity, probes

pytestmark = pytest.mark.gpu

DEV = "cuda"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FORMS = ["padded_bhnd", "packed_nhd"]
CAUSALS = ["none", "upper_left", "lower_right"]


# ------------------------------------------------------------------ masks
def _mask_tensor(rng, shape, kind):
    """A seeded mask of the given shape: bool with 20% False, or additive
    with 20% -4.0 (f16 / f32)."""
    draw = rng.random(shape)
    if kind == "bool":
        return torch.from_numpy(draw >= 0.2)
    dt = {"f16": torch.float16, "f32": torch.float32}[kind]
    return torch.from_numpy(np.where(draw < 0.2, np.float32(-4.0), np.float32(0.0))).to(dt)


@pytest.mark.parametrize("layout", ["r1", "r2", "r3_bcast", "r3_heads", "b1", "b1_heads"])
@pytest.mark.parametrize("kind,aligned", [("bool", True), ("bool", False), ("f16", True),
                                          ("f16", False), ("f32", True)])
def test_mask_ranks_and_broadcasts(layout, kind, aligned):
    # Head-broadcast 1- and 2-byte masks whose key extent is a whole number
    # of 16-byte chunks take the LDS-staged path; the others (f32, per-head
    # masks, odd key extents) the per-lane path.
    seed = 7000 + ["r1", "r2", "r3_bcast", "r3_heads", "b1", "b1_heads"].index(layout) * 8 + \
        ["bool", "f16", "f32"].index(kind) * 2 + aligned
    rng = np.random.default_rng(seed)
    hq, hkv = 8, 2
    ql = np.array([31, 1, 70, 33])
    kl = np.maximum(rng.integers(1, 200, size=4), ql)
    c = synth.generate(seed=seed, q_lens=ql, kv_lens=kl, num_heads=hq, kv_num_heads=hkv,
                       head_dim=128, query_form="packed_nhd", kv_form="padded_bhnd",
                       n_kv=208, q_slack=2, kv_slack=0, dtype=torch.float16,
                       causal_kind="lower_right", device=DEV, name=f"mask-{layout}-{kind}-{aligned}")
    nq = int(ql.max())
    nk = 208 if aligned else 203  # 208 keys: 16-byte rows for 1- and 2-byte masks
    shape = {"r1": (nk,), "r2": (nq, nk), "r3_bcast": (1, nq, nk), "r3_heads": (hq, nq, nk),
             "b1": (1, 1, nq, nk), "b1_heads": (1, hq, nq, nk)}[layout]
    m = _mask_tensor(rng, shape, kind)
    c = dataclasses.replace(c, mask=m.to(DEV))
    parity.compare(c, parity.run_gpu(c))


@pytest.mark.parametrize("kind", ["bool", "f16"])
@pytest.mark.parametrize("causal", ["none", "upper_left"])
def test_batch_broadcast_mask_padded_q(kind, causal):
    # padded Q / packed KV with a [1, 1, N_q, N_kv] mask shared by the batch
    seed = 7100 + (kind == "f16") * 2 + (causal == "upper_left")
    rng = np.random.default_rng(seed)
    ql = rng.integers(1, 90, size=3)
    kl = rng.integers(1, 150, size=3)
    c = synth.generate(seed=seed, q_lens=ql, kv_lens=kl, num_heads=8, kv_num_heads=2,
                       head_dim=64, query_form="padded_bhnd", kv_form="packed_nhd",
                       n_q=96, q_slack=0, kv_slack=3, pass_query_lengths=True,
                       dtype=torch.bfloat16, causal_kind=causal, device=DEV,
                       name=f"bmask-{kind}-{causal}")
    m = _mask_tensor(rng, (1, 1, 96, 160), kind)
    c = dataclasses.replace(c, mask=m.to(DEV))
    parity.compare(c, parity.run_gpu(c))


# ------------------------------------------------- rows with no allowed key
def _row_values(case, out, b, i):
    """All heads of output row i of sequence b, as float32 [H, D]."""
    if case.query_form == "packed_nhd":
        r = int(np.sum(case.q_lens[:b])) + i
        return out[r].float()
    return out[b, :, i].float()


@pytest.mark.parametrize("qf,kf", list(itertools.product(FORMS, FORMS)))
@pytest.mark.parametrize("mask", [None, "bool"])
def test_lower_right_shorter_kv_rows_are_zero(qf, kf, mask):
    # kv_len < q_len: rows i < q_len - kv_len have no allowed key (zeros)
    seed = 7200 + FORMS.index(qf) * 4 + FORMS.index(kf) * 2 + (mask is not None)
    ql = np.array([70, 33, 5, 100, 40])
    kl = np.array([30, 1, 4, 99, 40])
    c = synth.generate(seed=seed, q_lens=ql, kv_lens=kl, num_heads=8, kv_num_heads=2,
                       head_dim=128, query_form=qf, kv_form=kf, n_q=104, n_kv=112, q_slack=3,
                       kv_slack=3, pass_query_lengths=True, dtype=torch.float16,
                       mask_kind=mask, mask_p=0.2, causal_kind="lower_right", device=DEV,
                       name=f"lr-short-{qf[:3]}-{kf[:3]}-{mask}")
    out = parity.run_gpu(c)
    parity.compare(c, out)
    for b in range(c.batch):
        for i in range(int(ql[b] - kl[b])):
            v = _row_values(c, out, b, i)
            assert torch.all(v == 0), (b, i)


def test_lower_right_shorter_kv_split_path():
    # the same with long keys: the split-KV path and its merge
    ql = np.array([700, 90])
    kl = np.array([500, 80])
    c = synth.generate(seed=7210, q_lens=ql, kv_lens=kl, num_heads=8, kv_num_heads=2,
                       head_dim=128, query_form="packed_nhd", kv_form="packed_nhd", q_slack=2,
                       kv_slack=2, dtype=torch.float16, causal_kind="lower_right", device=DEV,
                       name="lr-short-split")
    args = capi.make_args(c.q, c.k, c.v, c.mask, c.q, **c.kwargs())
    assert capi.gqa_attn_workspace_size(args) > 0  # the split path is taken
    out = parity.run_gpu(c)
    parity.compare(c, out)
    for b in range(c.batch):
        for i in range(int(ql[b] - kl[b])):
            assert torch.all(_row_values(c, out, b, i) == 0), (b, i)


# ------------------------------------------------------ exact-gather probes
@pytest.mark.parametrize("qf,kf", list(itertools.product(FORMS, FORMS)))
@pytest.mark.parametrize("causal", CAUSALS)
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_exact_gather_probe(qf, kf, causal, dtype):
    seed = 7300 + FORMS.index(qf) * 12 + FORMS.index(kf) * 6 + CAUSALS.index(causal) * 2 + (
        dtype == torch.bfloat16)
    c, expect, ks = probes.gather_probe(seed, qf, kf, causal, dtype, device=DEV)
    out = parity.run_gpu(c)
    raw = out.view(torch.int16).cpu()
    vraw = c.v.view(torch.int16).cpu()
    for (b, h, i), tgt in expect.items():
        got = raw[int(np.sum(c.q_lens[:b])) + i, h] if qf == "packed_nhd" else raw[b, h, i]
        if tgt is None:
            assert torch.all(got & 0x7FFF == 0), (b, h, i)  # zeros
            continue
        g, t = tgt
        want = vraw[int(ks[b]) + t, g] if kf == "packed_nhd" else vraw[b, g, t]
        assert torch.equal(got, want), (b, h, i, g, t)
    # and the oracle agrees (with the sentinel check on the rows not valid)
    parity.compare(c, out)


# ------------------------------------------------------------ 128-draft trees
def _tree128(seed, qf, kf, tree, q_lens, ctx, hq=8, hkv=2, dtype=torch.float16):
    ql = np.asarray(q_lens)
    kl = ql + np.asarray(ctx)
    n_q = 128 if qf == "padded_bhnd" else None
    return synth.generate(seed=seed, q_lens=ql, kv_lens=kl, num_heads=hq, kv_num_heads=hkv,
                          head_dim=128, query_form=qf, kv_form=kf, dtype=dtype, n_q=n_q,
                          n_kv=int(kl.max()) + 5 if kf != "paged" else int(kl.max()),
                          q_slack=3, kv_slack=2, pass_query_lengths=True, tree=tree,
                          page_size=64, device=DEV, name=f"tree128-{qf[:3]}-{kf[:3]}-{tree}")


@pytest.mark.parametrize("qf,kf", [("packed_nhd", "packed_nhd"), ("padded_bhnd", "padded_bhnd"),
                                   ("packed_nhd", "paged"), ("padded_bhnd", "packed_nhd")])
@pytest.mark.parametrize("tree", ["spec", "random", "chain"])
def test_tree_128_drafts(qf, kf, tree):
    seed = 7400 + ["packed_nhd", "padded_bhnd"].index(qf) * 10 + ["spec", "random",
                                                                   "chain"].index(tree) + \
        (kf == "paged") * 3 + (kf == "packed_nhd") * 5
    c = _tree128(seed, qf, kf, tree, q_lens=[128, 97, 65, 128], ctx=[300, 0, 77, 1000])
    parity.compare(c, parity.run_gpu(c))


def test_tree_more_than_128_drafts_gives_nan_rows():
    # packed Q: rows past the 128th draft of a sequence come out NaN (the
    # documented limit), every other row matches the oracle
    c = _tree128(7450, "packed_nhd", "packed_nhd", "random", q_lens=[150, 40], ctx=[200, 90])
    out = parity.run_gpu(c)
    rows = np.array([(b, h, i) for b in range(2) for h in (0, 5)
                     for i in range(min(int(c.q_lens[b]), 128))], dtype=np.int32)
    parity.compare(c, out, rows=rows)
    for i in range(128, 150):
        assert torch.isnan(out[i].float()).all(), i
    assert not torch.isnan(out[150:190].float()).any()


# ------------------------------------------------ split-KV with large |O|
@pytest.mark.parametrize("D", [64, 128])
def test_split_kv_large_outputs(D):
    # few query rows over long keys (the split path) with V = 8 + N(0, 1):
    # |O| ~ 8 straddles a binade of f16, where rounding each slice's output
    # before the merge would add up to 1.5 ulp; the merge of fp32 partials
    # rounds once and stays within max(2e-3, ulp(|O|))
    seed = 7500 + D
    ql = np.array([37, 5, 64])
    kl = np.array([2900, 1500, 2100])
    c = synth.generate(seed=seed, q_lens=ql, kv_lens=kl, num_heads=8, kv_num_heads=2,
                       head_dim=D, query_form="packed_nhd", kv_form="padded_bhnd",
                       n_kv=2944, q_slack=2, dtype=torch.float16, causal_kind="lower_right",
                       device=DEV, name=f"split-large-{D}")
    for b in range(3):
        c.v[b, :, :kl[b]] = (c.v[b, :, :kl[b]].float() + 8.0).to(torch.float16)
    args = capi.make_args(c.q, c.k, c.v, c.mask, c.q, **c.kwargs())
    assert capi.gqa_attn_workspace_size(args) > 0  # the split path is taken
    st = parity.compare(c, parity.run_gpu(c))
    assert st["ulp_relaxed"] > 0  # outputs beyond |O| = 4, where the ulp term is the bar


# ------------------------------------------------------ validate mode
_VALIDATE_SCRIPT = textwrap.dedent("""
    import sys, numpy as np, torch
    sys.path.insert(0, sys.argv[1])
    from gqa_attention_ragged_amd import capi, synth
    c = synth.generate(seed=7600, q_lens=[20, 7, 33], kv_lens=[40, 9, 50], num_heads=8,
                       kv_num_heads=2, head_dim=128, query_form="packed_nhd",
                       kv_form="padded_bhnd", n_kv=64, causal_kind="lower_right", device="cuda",
                       name="validate")
    out = synth.sentinel_like(c.q.shape, c.out_dtype, "cuda")
    # kv_lengths past N_kv = 64: rejected on the device before any attention kernel
    bad = c.kwargs()
    bad["kv_lengths"] = torch.tensor([40, 65, 50], dtype=torch.int32, device="cuda")
    args = capi.make_args(c.q, c.k, c.v, c.mask, out, **bad)
    st = capi.load().gqa_attn_forward(args, None, 0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == capi.GQA_ERR_INVALID_ARG, st
    assert "exceed k/v" in capi.last_error(), capi.last_error()
    raw = out.view(torch.int16).cpu()
    assert torch.all(raw == synth.SENTINEL_BITS[c.out_dtype]), "an attention kernel ran"
    # decreasing cumulative query lengths
    bad = c.kwargs()
    bad["query_lengths"] = torch.tensor([0, 20, 10, 60], dtype=torch.int32, device="cuda")
    args = capi.make_args(c.q, c.k, c.v, c.mask, out, **bad)
    st = capi.load().gqa_attn_forward(args, None, 0, torch.cuda.current_stream().cuda_stream)
    assert st == capi.GQA_ERR_INVALID_ARG and "non-decreasing" in capi.last_error()
    assert torch.all(out.view(torch.int16).cpu() == synth.SENTINEL_BITS[c.out_dtype])
    # the valid call runs and matches the oracle
    from tests import parity
    parity.compare(c, parity.run_gpu(c))
    print("validate ok")
""")


def test_validate_mode_rejects_before_launch():
    # GQA_ATTN_VALIDATE is read once per process: run in a child process
    env = dict(os.environ, GQA_ATTN_VALIDATE="1")
    r = subprocess.run([sys.executable, "-c", _VALIDATE_SCRIPT, ROOT], env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "validate ok" in r.stdout


# ------------------------------------------------------ tile-map records
def _run_ws(c, with_workspace):
    out = synth.sentinel_like(c.q.shape, c.out_dtype, DEV)
    args = capi.make_args(c.q, c.k, c.v, c.mask, out, **c.kwargs())
    n = capi.gqa_attn_workspace_size(args)
    assert n > 0  # the records are planned
    ws = torch.empty(n, dtype=torch.uint8, device=DEV) if with_workspace else None
    capi.gqa_attn_forward(args, ws, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("hq,hkv,causal,qf,dtype", [
    (16, 4, "lower_right", "packed_nhd", torch.float16),    # 4 head groups (no XCD remap)
    (32, 8, "lower_right", "packed_nhd", torch.bfloat16),   # 8 head groups: XCD remap
    (32, 8, "none", "padded_bhnd", torch.float16),
    (12, 4, "upper_left", "padded_bhnd", torch.bfloat16),   # groups of 3: one head per workgroup
])
def test_records_equal_in_kernel_map(hq, hkv, causal, qf, dtype):
    # at least 1024 workgroups, so that the call plans records
    rng = np.random.default_rng(7700 + hq + hkv)
    B = 64
    ql = rng.integers(0, 400, size=B)
    # at most 448 keys: no split-KV, so the call also runs without a workspace
    kl = ql + rng.integers(0, 40, size=B) if causal == "lower_right" else rng.integers(1, 440, size=B)
    n_q = int(ql.max()) + 3
    c = synth.generate(seed=7700 + hq, q_lens=ql, kv_lens=kl, num_heads=hq, kv_num_heads=hkv,
                       head_dim=128, query_form=qf, kv_form="padded_bhnd", dtype=dtype, n_q=n_q,
                       n_kv=int(kl.max()) + 5, pass_query_lengths=True, causal_kind=causal,
                       device=DEV, name=f"records-{hq}-{hkv}-{causal}-{qf}")
    a = _run_ws(c, True)
    b = _run_ws(c, False)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    parity.compare(c, a)


def test_split_kv_plans_no_records():
    # few rows over long keys, 8 head groups: about 128 workgroups split into
    # about 12 key slices; split grids take no records (the workspace holds
    # the partials only) and run as before
    rng = np.random.default_rng(7750)
    ql = rng.integers(1, 60, size=8)
    kl = ql + rng.integers(3000, 6000, size=8)
    c = synth.generate(seed=7750, q_lens=ql, kv_lens=kl, num_heads=32, kv_num_heads=8,
                       head_dim=128, query_form="packed_nhd", kv_form="padded_bhnd",
                       dtype=torch.bfloat16, n_kv=int(kl.max()) + 3, causal_kind="lower_right",
                       device=DEV, name="records-split")
    args = capi.make_args(c.q, c.k, c.v, c.mask, torch.empty_like(c.q), **c.kwargs())
    n = capi.gqa_attn_workspace_size(args)
    rows, heads, D = int(ql.sum()), 32, 128
    assert n > rows * heads * 2 * D * 4
    assert (n - 256) % (rows * heads * (D * 4 + 8)) == 0  # partials of S slices, no records
    parity.compare(c, parity.run_gpu(c))


@pytest.mark.parametrize("kind", ["prefill_split", "decode"])
def test_main_kernel_timer(kind):
    # the library's main-kernel timing window: one event pair per call
    # around the attention kernel (the merge / combine kernels outside),
    # calls past the window's size not timed, outputs unchanged; the timed
    # kernel fits inside the whole call that torch's events measure
    rng = np.random.default_rng(7760)
    if kind == "prefill_split":
        ql = rng.integers(1, 60, size=8)
        kl = ql + rng.integers(3000, 6000, size=8)
        c = synth.generate(seed=7760, q_lens=ql, kv_lens=kl, num_heads=32, kv_num_heads=8,
                           head_dim=128, query_form="packed_nhd", kv_form="padded_bhnd",
                           dtype=torch.bfloat16, n_kv=int(kl.max()) + 3,
                           causal_kind="lower_right", device=DEV, name="timer-prefill")
    else:
        kl = rng.integers(100, 20000, size=16)
        c = synth.generate(seed=7761, q_lens=np.ones(16, int), kv_lens=kl, num_heads=32,
                           kv_num_heads=8, head_dim=128, n_q=1, n_kv=int(kl.max()) + 5,
                           dtype=torch.float16, pass_query_lengths=False, device=DEV,
                           name="timer-decode")
    ref = parity.run_gpu(c)
    assert capi.timer_start(2) == capi.GQA_OK
    assert capi.timer_start(2) == capi.GQA_ERR_INVALID_ARG  # one window at a time
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    outs = []
    s.record()
    for _ in range(3):
        o = synth.sentinel_like(c.q.shape, c.out_dtype, c.q.device)
        outs.append(capi.attn_forward(c.q, c.k, c.v, c.mask, out=o, **c.kwargs()))
    e.record()
    torch.cuda.synchronize()
    st, ms, n = capi.timer_stop()
    assert st == capi.GQA_OK, capi.last_error()
    assert n == 2  # the third call is past the window
    whole = s.elapsed_time(e) / 3
    assert 0 < ms / n <= whole * 1.05, (ms / n, whole)
    for o in outs:
        assert torch.equal(o, ref)
    st, _, _ = capi.timer_stop()
    assert st == capi.GQA_ERR_INVALID_ARG  # closed


def test_main_kernel_timer_two_threads():
    # two threads, each on its own stream, call the library while one timing
    # window is open: every call's pair is its own (6 timed calls), and the
    # outputs are those of an untimed call
    import threading
    rng = np.random.default_rng(7770)
    ql = rng.integers(1, 200, size=6)
    kl = ql + rng.integers(0, 900, size=6)
    c = synth.generate(seed=7770, q_lens=ql, kv_lens=kl, num_heads=8, kv_num_heads=2,
                       head_dim=128, query_form="packed_nhd", kv_form="packed_nhd",
                       dtype=torch.float16, causal_kind="lower_right", device=DEV,
                       name="timer-threads")
    ref = parity.run_gpu(c)
    outs, errors = {}, []

    def work(k):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                res = []
                for _ in range(3):
                    o = synth.sentinel_like(c.q.shape, c.out_dtype, c.q.device)
                    res.append(capi.attn_forward(c.q, c.k, c.v, c.mask, out=o, **c.kwargs()))
                stream.synchronize()
            outs[k] = res
        except Exception as e:  # surfaced below
            errors.append(e)

    torch.cuda.synchronize()
    assert capi.timer_start(10) == capi.GQA_OK
    threads = [threading.Thread(target=work, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    st, ms, n = capi.timer_stop()
    assert not errors, errors
    assert st == capi.GQA_OK, capi.last_error()
    assert n == 6 and ms > 0
    for k in range(2):
        for o in outs[k]:
            assert torch.equal(o, ref)
