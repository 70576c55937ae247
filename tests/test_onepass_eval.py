"""Evaluation of a one-pass fp8 Q/DQ variant (CPU only; the variant is not
built).  TRT_QuantizedAttention (onnx-tensorrt "TensorRT Custom Operator
Schemas" page) quantizes the normalized P = exp(s - m) / l, which needs the
final row max m and sum l before any score is quantized: the GPU path runs a
statistics pass, then recomputes the scores.  A one-pass variant would
quantize exp(s - m_run) / qscale with the running max, accumulate the
dequantized values, and divide by the running sum at the end.  It is kept
only if it meets the 3e-2 parity bar on every seed; this test records that
it does not (rows with few allowed keys quantize large, very different
values), which is why the two-pass path stays."""
import numpy as np
import torch

from gqa_attention_ragged_amd import synth

FP8 = torch.float8_e4m3fn


def _q8(x):
    return torch.from_numpy(np.clip(x, -448.0, 448.0)).to(FP8).double().numpy()


def _one_pass(c, rows, tile=64):
    q = c.q.float().double().numpy()
    k = c.k.float().double().numpy()
    v = c.v.float().double().numpy()
    qs = float(np.float32(c.qscale))
    G = c.num_heads // c.kv_num_heads
    out = np.zeros((len(rows), q.shape[-1]))
    for r, (b, h, i) in enumerate(rows):
        g = h // G
        n = i + 1  # upper_left causal, q_len = kv_len
        s = (k[b, g, :n] @ q[b, h, i]) * c.scale
        m, l, o = -np.inf, 0.0, np.zeros(q.shape[-1])
        for t0 in range(0, n, tile):
            st = s[t0:t0 + tile]
            mn = max(m, st.max())
            a = np.exp(m - mn) if m > -np.inf else 0.0
            o, l = o * a, l * a
            e = np.exp(st - mn)
            o += (_q8(e / qs) * qs) @ v[b, g, t0:t0 + len(st)]
            l += e.sum()
            m = mn
        out[r] = o / l
    return out


def test_one_pass_fp8_variant_misses_the_bar(oracle_mod):
    worst = []
    for seed in range(2):
        c = synth.generate(seed=100 + seed, q_lens=[256], kv_lens=[256], num_heads=4,
                           kv_num_heads=1, head_dim=128, dtype=FP8, dist="round_normal",
                           causal_kind="upper_left", qdq="fp8",
                           qscale=float(np.float32(1 / 448.0)), pass_kv_lengths=False)
        res = oracle_mod.attention(c.q, c.k, c.v, c.mask, **c.kwargs())
        err = np.abs(_one_pass(c, res.rows) - res.out) - res.amb
        worst.append(float(err.max()))
    assert max(worst) > 3e-2, worst
