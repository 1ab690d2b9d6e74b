"""Benchmark of the CCA / CCGQA forward pass on one MI355X.

One step is one pass of the whole hot path over synthetic inputs resident in
HBM: a CCA prefill of the 4 x 2048-token batch (E = 2048, 8 latent heads of
64, compression 4) followed by one CCGQA decode step of 64 sequences against
a 32768-token latent cache (16 query / 4 kv heads of 64).  Both calls go
through libcca's C ABI on torch's current HIP stream.

Prints ONE JSON line.  ``value`` is prefill tokens per second of prefill time;
the decode step's HBM rate and the attention kernel's MFMA rate are reported
next to it.  A second timed pass launches the same kernels stage by stage
with HIP events between them to get per-kernel durations for the roofline.
A fourth pass times a training step on the prefill workload
(``cca_prefill_forward_train`` + ``cca_prefill_backward``, reported under
``train``).  The fp64 oracle is timed on the host cores on a bounded sample
of the same prefill workload (``cpu_baseline``).

    python bench.py [--steps K] [--warmup W] [--prefill WORKLOAD] [--no-cpu]
    python bench.py --compare     # CCGQA vs full-width MHA / GQA-8 prefill, and a T sweep
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CCA prefill tokens/sec and attn TFLOP/s vs MFMA peak; decode HBM GB/s"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 MFMA
PEAK_F32_MFMA_TFLOPS = 157.3


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--prefill", default="cca_prefill_b4_t2048")
    p.add_argument("--decode", default="ccgqa_decode_b64_l32768")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--compare", action="store_true",
                   help="prefill of ccgqa_prefill_t16384 next to full-width MHA and GQA-8 baselines "
                        "through the same kernels, plus a sequence-length sweep (prints its own JSON)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy 5 times (the reference "
                        "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


def calibrate_copy():
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)


def upload_weights(cca, T, W, dev):
    import torch
    dense = lambda a: None if a is None else torch.from_numpy(a).to(dev)
    return cca.Weights(T.to_device(W.w_qkv_s, dev), T.to_device(W.w_o_s, dev),
                       torch.from_numpy(W.q_seq_taps).to(dev), torch.from_numpy(W.k_seq_taps).to(dev),
                       torch.from_numpy(W.q_chan_taps).to(dev), torch.from_numpy(W.k_chan_taps).to(dev),
                       torch.from_numpy(W.tau).to(dev), dense(W.q_chan_dense), dense(W.k_chan_dense))


def grouped_reading(cca, T, sp, sd, P, D_weights, x, y, st, xt, yt, L, K, dev):
    """The prefill and decode workloads under the grouped channel-conv
    reading (dense d x d weights per lag and head, drawn from their own seeded
    stream): the prefill through cca_prefill_forward and its mixing stage
    alone (the MFMA channel conv plus the mixing kernel), and the decode step
    with its (k_s-1)+(k_c-1)-row window.  None when the shapes do not take it."""
    import torch
    from synth import add_chan_dense
    gp, gd = cca.make_config(sp, chan_conv="grouped"), cca.make_config(sd, chan_conv="grouped")
    if cca.validate_config(gp) != cca.CCA_OK or cca.validate_config(gd) != cca.CCA_OK:
        return None
    add_chan_dense(P.weights, sp, 0)
    add_chan_dense(D_weights, sd, 0)
    pw, dw = upload_weights(cca, T, P.weights, dev), upload_weights(cca, T, D_weights, dev)
    ws = T.workspace(cca.prefill_workspace_size(gp), dev)
    win = sd.seq_conv_k - 1 + sd.chan_conv_k - 1
    sdt = st.conv_q.dtype
    stg = cca.State(st.k_cache, st.v_cache, st.capacity,
                    torch.zeros((sd.batch, win, sd.e_q), dtype=sdt, device=dev),
                    torch.zeros((sd.batch, win, sd.e_kv), dtype=sdt, device=dev), st.vshift)
    dws = T.workspace(cca.decode_workspace_size(gd, L), dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(K)]
        for a, b_ in evs:
            a.record()
            fn()
            b_.record()
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b_) for a, b_ in evs) / K

    prefill = timed(lambda: cca.prefill_forward(gp, pw, x, y, ws))
    cca.stage_downproj(gp, pw, x, ws)
    mix = timed(lambda: cca.stage_convmix(gp, pw, ws))
    decode = timed(lambda: cca.decode_step(gd, dw, xt, L, stg, stg, yt, dws))
    flops = 2.0 * sp.batch * sp.seq_len * (sp.n_q_heads + sp.n_kv_heads) * sp.head_dim * \
        sp.chan_conv_k * sp.head_dim
    return {"reading": "grouped channel conv, dense d x d weights per lag and head",
            "prefill_ms": round(prefill, 4), "mix_stage_ms": round(mix, 4),
            "channel_conv_gflop": round(flops / 1e9, 3),
            "decode_ms": round(decode, 4)}


def algorithmic(sp, sd):
    """Algorithmic work per launch of each kernel (what the method must move or
    compute, not padded or masked work)."""
    B, T, E = sp.batch, sp.seq_len, sp.d_model
    eq, ekv, N = sp.e_q, sp.e_kv, sp.n_qkv
    esz = 2 if sp.dtype == "bf16" else 4
    Lk = sd.cache_len + 1
    return {
        # bytes: read qkv~ (fp32) + write q, k (16-bit) and v (storage type)
        "convmix_bytes": B * T * N * 4 + B * T * (eq + ekv) * 2 + B * T * ekv * esz,
        # causal latent attention: 2 matmuls of 2*d flops per visible (query, key) pair
        "attn_flops": 2 * 2 * B * sp.n_q_heads * sp.head_dim * T * (T + 1) / 2,
        "downproj_flops": 2 * B * T * N * E,
        "upproj_flops": 2 * B * T * E * eq,
        # decode attention streams K and V of Lk keys once
        "decode_attn_bytes": 2 * sd.batch * sd.n_kv_heads * Lk * sd.head_dim * 2,
    }


def measured_traffic():
    """HBM bytes per launch of each kernel from the committed counter summary
    (profiles/pmc_traffic.json), kept only while the kernel's sources still
    hash to what they were when the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return {}
    rec = json.load(open(path))
    out = {}
    for key, k in rec.get("kernels", {}).items():
        h = hashlib.sha256()
        for f in k["sources"]:
            h.update(open(os.path.join(ROOT, "efficient_transformer_attention_amd", "csrc", f), "rb").read())
        if h.hexdigest()[:16] == k["source_sha256_16"]:
            out[key] = k["bytes"]
    return out


def cpu_baseline(sp, seconds):
    """The fp64 oracle on the host cores: whole sequences of the prefill
    workload (the same synthetic sequence, repeated) until about `seconds`
    of wall time are spent."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing
        threads = len(os.sched_getaffinity(0))
    import oracle.cca as O
    from synth import make_prefill
    one = sp.with_(batch=1)
    P = make_prefill(one, seed=0)
    w = P.weights.f64()
    done, t0 = 0, time.perf_counter()
    while True:
        O.prefill(P.x, w, one)
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": done * one.seq_len / el, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": cpu_model, "wall_s": round(el, 2),
            "sample": f"{done} passes over one sequence of the prefill workload "
                      f"(T={one.seq_len}, E={one.d_model}, {one.n_q_heads}x{one.head_dim} heads; "
                      f"the workload has {sp.batch}), fp64 NumPy, {el:.1f} s wall"}


def paged_decode(cca, T, sd, dcfg, dw, xt, dl, L, st, K, dev, page=256):
    """cca_decode_step_paged over a paged copy of the decode cache: each
    sequence's rows cut into `page`-token pages stored in a seeded random
    order, timed with HIP events."""
    import numpy as np
    import torch
    B, H, cap, d = st.k_cache.shape
    mpps = (cap + page - 1) // page
    perm = torch.from_numpy(np.random.default_rng(2).permutation(B * mpps)).to(dev)

    def pages_of(c):
        padded = torch.zeros((B, H, mpps * page, d), dtype=c.dtype, device=dev)
        padded[:, :, :cap] = c
        blocks = padded.view(B, H, mpps, page, d).permute(0, 2, 1, 3, 4).reshape(B * mpps, H, page, d)
        out = torch.empty_like(blocks)
        out[perm] = blocks
        return out
    kp, vp = pages_of(st.k_cache), pages_of(st.v_cache)
    table = perm.view(B, mpps).to(torch.int32).contiguous()
    ps = cca.PagedState(kp, vp, table, page, st.conv_q.clone(), st.conv_k.clone(), st.vshift.clone())
    yt = torch.empty_like(xt)
    ws = T.workspace(cca.decode_workspace_size(dcfg, L), dev)
    cca.decode_step_paged(dcfg, dw, xt, dl, L, ps, ps, yt, ws)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for a, b_ in ev:
        a.record()
        cca.decode_step_paged(dcfg, dw, xt, dl, L, ps, ps, yt, ws)
        b_.record()
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b_) for a, b_ in ev) / K
    del kp, vp, ps, ws
    torch.cuda.empty_cache()
    return ms, page


def multi_decode(cca, T, sd, dcfg, dw, dl, Lmax, st, K, dev, m):
    """cca_decode_multi with m new tokens per sequence at the per-sequence
    lengths dl (clamped to Lmax), timed with HIP events."""
    import numpy as np
    import torch
    x = torch.from_numpy(np.random.default_rng(3).standard_normal(
        (sd.batch, m, sd.d_model)).astype(np.float32)).to(dev, torch.bfloat16)
    y = torch.empty_like(x)
    dlm = torch.clamp(dl, max=Lmax).contiguous()
    ws = T.workspace(cca.decode_multi_workspace_size(dcfg, m, Lmax), dev)
    cca.decode_multi(dcfg, dw, x, m, dlm, Lmax, st, st, y, ws)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for a, b_ in ev:
        a.record()
        cca.decode_multi(dcfg, dw, x, m, dlm, Lmax, st, st, y, ws)
        b_.record()
    torch.cuda.synchronize()
    del ws
    return sum(a.elapsed_time(b_) for a, b_ in ev) / K


def training_step(cca, T, sp, pcfg, pw, x, dev, K):
    """forward_train + backward on the prefill workload, timed with HIP events."""
    import torch
    from synth import make_upstream_grad
    dy = T.to_device(make_upstream_grad(sp, seed=0).dy_s, dev)
    y = torch.empty_like(x)
    tws = T.workspace(cca.train_workspace_size(pcfg), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = cca.Grads(torch.empty_like(x), torch.empty((sp.n_qkv, sp.d_model), **f32),
                  torch.empty((sp.d_model, sp.e_q), **f32), torch.empty((sp.e_q, sp.seq_conv_k), **f32),
                  torch.empty((sp.e_kv, sp.seq_conv_k), **f32),
                  torch.empty((sp.n_q_heads, sp.chan_conv_k), **f32),
                  torch.empty((sp.n_kv_heads, sp.chan_conv_k), **f32),
                  torch.empty((sp.n_q_heads,), **f32))
    for _ in range(2):
        cca.prefill_forward_train(pcfg, pw, x, y, tws)
        cca.prefill_backward(pcfg, pw, x, dy, g, tws)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for e in ev:
        e[0].record()
        cca.prefill_forward_train(pcfg, pw, x, y, tws)
        e[1].record()
        cca.prefill_backward(pcfg, pw, x, dy, g, tws)
        e[2].record()
    torch.cuda.synchronize()
    fwd = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    bwd = sum(e[1].elapsed_time(e[2]) for e in ev) / K
    print(f"[bench] training step: forward {fwd:.3f} ms backward {bwd:.3f} ms", file=sys.stderr,
          flush=True)
    B, Tn, d, H = sp.batch, sp.seq_len, sp.head_dim, sp.n_q_heads
    pairs = B * H * Tn * (Tn + 1) / 2
    del tws, g, dy, y
    torch.cuda.empty_cache()
    return {"workload": "the prefill workload above, forward_train + backward, seeded dy ~ N(0,1)",
            "forward_ms": round(fwd, 4), "backward_ms": round(bwd, 4),
            "step_ms": round(fwd + bwd, 4),
            "tokens_per_s": round(sp.tokens / ((fwd + bwd) * 1e-3), 1),
            "backward_over_forward": round(bwd / fwd, 3),
            # algorithmic flops of the backward: 5 matmuls of 2d flops per visible
            # pair (S recomputed, dP, dV, dQ, dK) plus the 4 gradient GEMMs
            "backward_gflop": round((5 * 2 * d * pairs + 2 * 2 * sp.tokens * sp.d_model * (sp.n_qkv + sp.e_q))
                                    / 1e9, 2)}


def compare(args):
    """The pages' prefill and backward comparisons reproduced with this
    library's kernels: CCGQA (ccgqa_prefill_t16384) against full-width MHA and
    GQA-8 at the same T, E and head size with the extras off (forward, then a
    training step: forward_train + backward), then a prefill sweep over T.  Context for
    the pages' own ratios, which they measure on other hardware."""
    import math
    import numpy as np
    import torch

    from efficient_transformer_attention_amd import cca, tensors as T
    from synth import COMPARISON_OVERRIDES, COMPARISONS, make_prefill, workload

    dev = "cuda:0"
    torch.cuda.set_device(0)
    K = max(2, min(args.steps, 5))

    def run(name, sp, train=False):
        P = make_prefill(sp, seed=0)
        W = P.weights
        if name in COMPARISONS:
            for a in (W.q_seq_taps, W.k_seq_taps, W.q_chan_taps, W.k_chan_taps):
                a[...] = COMPARISON_OVERRIDES["taps"]
            W.tau = np.full(sp.n_q_heads, 1.0 / math.sqrt(sp.head_dim), dtype=np.float32)
        pw = upload_weights(cca, T, W, dev)
        cfg = cca.make_config(sp)
        x = T.to_device(P.x_s, dev)
        y = torch.empty_like(x)
        ws = T.workspace(cca.prefill_workspace_size(cfg), dev)
        del P
        for _ in range(2):
            cca.prefill_forward(cfg, pw, x, y, ws)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        for e in ev:
            e[0].record()
            cca.prefill_forward(cfg, pw, x, y, ws)
            e[1].record()
            cca.stage_attention(cfg, pw, ws)
            e[2].record()
        torch.cuda.synchronize()
        pre = sum(a.elapsed_time(b) for a, b, _ in ev) / K
        att = sum(b.elapsed_time(c) for _, b, c in ev) / K
        flops = 2 * 2 * sp.batch * sp.n_q_heads * sp.head_dim * sp.seq_len * (sp.seq_len + 1) / 2
        r = {"T": sp.seq_len, "E": sp.d_model, "heads": f"{sp.n_q_heads}q/{sp.n_kv_heads}kv x {sp.head_dim}",
             "prefill_ms": round(pre, 4), "tokens_per_s": round(sp.tokens / (pre * 1e-3), 1),
             "attention_ms": round(att, 4), "attention_tflops": round(flops / (att * 1e-3) / 1e12, 1)}
        print(f"[compare] {name} T={sp.seq_len}: prefill {pre:.3f} ms, attention {att:.3f} ms",
              file=sys.stderr, flush=True)
        del ws
        if train:
            # forward_train + backward on the same shape (the pages' backward comparison)
            r["train"] = training_step(cca, T, sp, cfg, pw, x, dev, K)
            r["train"]["workload"] = "forward_train + backward on this shape, seeded dy ~ N(0,1)"
        del x, y, pw
        torch.cuda.empty_cache()
        return r

    main3 = ["ccgqa_prefill_t16384", "gqa8_prefill_t16384", "mha_prefill_t16384"]
    res = {n: run(n, workload(n), train=True) for n in main3}
    base = res["ccgqa_prefill_t16384"]
    ratios = {f"{n}_over_ccgqa": {"prefill": round(res[n]["prefill_ms"] / base["prefill_ms"], 3),
                                  "attention": round(res[n]["attention_ms"] / base["attention_ms"], 3),
                                  "backward": round(res[n]["train"]["backward_ms"]
                                                    / base["train"]["backward_ms"], 3)}
              for n in main3[1:]}
    sweep = []
    for n in ("ccgqa_prefill_t16384", "mha_prefill_t16384"):
        for t in (2048, 4096, 8192):
            r = run(n, workload(n).with_(seq_len=t))
            sweep.append(dict(r, shape=n))
    sweep += [dict(res[n], shape=n) for n in ("ccgqa_prefill_t16384", "mha_prefill_t16384")]
    print(json.dumps({"comparison": res, "ratios": ratios, "sweep": sweep, "steps": K,
                      "baselines": "same kernels, extras off (unit taps, no q-k-mean / value-shift / "
                                   "L2 norm, tau = 1/sqrt(d)); GQA-8 = 8 kv heads"}), flush=True)


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.compare:
        compare(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is a design note, not a measured configuration.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from efficient_transformer_attention_amd import cca, tensors as T
    from synth import make_decode, make_prefill, workload

    dev = "cuda:0"
    torch.cuda.set_device(0)
    sp, sd = workload(args.prefill), workload(args.decode)

    # ---- inputs (seeded, synthetic), resident in HBM before timing ----------
    t_gen = time.perf_counter()
    P = make_prefill(sp, seed=0)
    D = make_decode(sd, seed=0)
    print(f"[bench] inputs generated in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)
    pw = upload_weights(cca, T, P.weights, dev)
    dw = upload_weights(cca, T, D.weights, dev)
    pcfg, dcfg = cca.make_config(sp), cca.make_config(sd)
    x = T.to_device(P.x_s, dev)
    y = torch.empty_like(x)
    pws = T.workspace(cca.prefill_workspace_size(pcfg), dev)
    st = cca.State(T.to_device(D.k_cache_s, dev), T.to_device(D.v_cache_s, dev), D.capacity,
                   T.to_device(D.conv_q_s, dev), T.to_device(D.conv_k_s, dev),
                   T.to_device(D.vshift_s, dev))
    del D.k_cache_s, D.v_cache_s
    xt = T.to_device(D.x_s, dev)
    yt = torch.empty_like(xt)
    L = sd.cache_len
    dws = T.workspace(cca.decode_workspace_size(dcfg, L), dev)
    torch.cuda.synchronize()

    def step():
        cca.prefill_forward(pcfg, pw, x, y, pws)
        cca.decode_step(dcfg, dw, xt, L, st, st, yt, dws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    # ---- timed region 1: the public entry points ---------------------------
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record()
        cca.prefill_forward(pcfg, pw, x, y, pws)
        ev[i][1].record()
        cca.decode_step(dcfg, dw, xt, L, st, st, yt, dws)
        ev[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prefill_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    prefill_ms_median = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
    decode_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K
    ms_per_step = wall * 1e3 / K
    print(f"[bench] timed {K} steps: prefill {prefill_ms:.3f} ms decode {decode_ms:.3f} ms",
          file=sys.stderr, flush=True)

    # ---- timed region 2: stage by stage, HIP events between kernels --------
    names = ["downproj", "convmix", "attention", "upproj",
             "dec_downproj", "dec_mix", "dec_attention", "dec_upproj"]
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        e = sev[i]
        e[0].record()
        cca.stage_downproj(pcfg, pw, x, pws); e[1].record()
        cca.stage_convmix(pcfg, pw, pws); e[2].record()
        cca.stage_attention(pcfg, pw, pws); e[3].record()
        cca.stage_upproj(pcfg, pw, y, pws); e[4].record()
        cca.stage_decode_downproj(dcfg, dw, xt, L, dws); e[5].record()
        cca.stage_decode_mix(dcfg, dw, L, st, st, dws); e[6].record()
        cca.stage_decode_attention(dcfg, dw, L, st, dws); e[7].record()
        cca.stage_decode_upproj(dcfg, dw, L, yt, dws); e[8].record()
    torch.cuda.synchronize()
    stage_ms = {n: sum(sev[i][j].elapsed_time(sev[i][j + 1]) for i in range(K)) / K
                for j, n in enumerate(names)}

    # ---- timed region 2b: the two HBM-bound kernels with the Infinity Cache
    # flushed (a 512 MiB buffer written between iterations, outside the timed
    # region), so their reads come from HBM ----------------------------------
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = {"convmix": 0.0, "dec_attention": 0.0}
    for _ in range(K):
        cca.stage_downproj(pcfg, pw, x, pws)
        flush.fill_(1)
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        cca.stage_convmix(pcfg, pw, pws)
        b_.record()
        cca.stage_decode_downproj(dcfg, dw, xt, L, dws)
        cca.stage_decode_mix(dcfg, dw, L, st, st, dws)
        flush.fill_(2)
        c, d_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c.record()
        cca.stage_decode_attention(dcfg, dw, L, st, dws)
        d_.record()
        torch.cuda.synchronize()
        cold["convmix"] += a.elapsed_time(b_) / K
        cold["dec_attention"] += c.elapsed_time(d_) / K
    del flush

    # ---- timed region 3: the decode step with per-sequence cache lengths ---
    # (seeded lengths uniform in [L/2, L]; algorithmic bytes: each sequence's
    # own K and V rows)
    rng = np.random.default_rng(1)
    lens = rng.integers(L // 2, L + 1, size=sd.batch).astype(np.int32)
    dl = torch.from_numpy(lens).to(dev)
    cca.decode_step_varlen(dcfg, dw, xt, dl, L, st, st, yt, dws)
    vev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    for a, b_ in vev:
        a.record()
        cca.decode_step_varlen(dcfg, dw, xt, dl, L, st, st, yt, dws)
        b_.record()
    torch.cuda.synchronize()
    varlen_ms = sum(a.elapsed_time(b_) for a, b_ in vev) / K
    varlen_bytes = float(sum(2 * sd.n_kv_heads * (int(l) + 1) * sd.head_dim * 2 for l in lens))

    # ---- timed region 3b: the same step on a paged copy of the cache -------
    # (256-token pages in a seeded random order, the same per-sequence lengths)
    paged_ms, page = paged_decode(cca, T, sd, dcfg, dw, xt, dl, L, st, K, dev)

    # ---- timed region 3c: four new tokens per sequence in one step ---------
    # (the same lengths; the cache is read once for the four tokens)
    multi_m = 4
    multi_ms = multi_decode(cca, T, sd, dcfg, dw, dl, L - multi_m, st, K, dev, multi_m)

    # ---- timed region 3d: the fused down-projection + mixing prefill -------
    fused_ms = None
    if cca.validate_config(pcfg) == cca.CCA_OK and sp.n_q_heads == sp.n_kv_heads and \
            sp.head_dim == 64 and sp.seq_len % 128 == 0 and sp.dtype == "bf16":
        fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(K)]
        cca.prefill_forward_fused(pcfg, pw, x, y, pws)
        torch.cuda.synchronize()
        for a, b_ in fev:
            a.record()
            cca.prefill_forward_fused(pcfg, pw, x, y, pws)
            b_.record()
        torch.cuda.synchronize()
        fused_ms = sum(a.elapsed_time(b_) for a, b_ in fev) / K

    # ---- timed region 3e: the grouped channel-conv reading -----------------
    grouped = grouped_reading(cca, T, sp, sd, P, D.weights, x, y, st, xt, yt, L, K, dev)

    # ---- timed region 4: a training step on the prefill workload ----------
    # forward_train (the forward keeping its activations) then the backward
    # pass with a seeded upstream gradient; every gradient is computed
    train = training_step(cca, T, sp, pcfg, pw, x, dev, K)

    alg = algorithmic(sp, sd)
    attn_tflops = alg["attn_flops"] / (stage_ms["attention"] * 1e-3) / 1e12
    conv_gbs = alg["convmix_bytes"] / (stage_ms["convmix"] * 1e-3) / 1e9
    dec_gbs = alg["decode_attn_bytes"] / (stage_ms["dec_attention"] * 1e-3) / 1e9
    dec_step_gbs = alg["decode_attn_bytes"] / (decode_ms * 1e-3) / 1e9
    mfma_peak = PEAK_BF16_TFLOPS if sp.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS

    rooflines = {
        "dec_attention": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS,
                          "unit": "GB/s", "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                          "traffic": None},
        "attention": {"bound": "mfma", "achieved": round(attn_tflops, 1), "peak": mfma_peak,
                      "unit": "TFLOP/s", "frac": round(attn_tflops / mfma_peak, 4), "traffic": None},
        "convmix": {"bound": "hbm", "achieved": round(conv_gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(conv_gbs / PEAK_HBM_GBS, 4), "traffic": None},
    }
    for g in ("downproj", "upproj"):
        tf = alg[f"{g}_flops"] / (stage_ms[g] * 1e-3) / 1e12
        rooflines[g] = {"bound": "mfma", "achieved": round(tf, 1), "peak": mfma_peak,
                        "unit": "TFLOP/s", "frac": round(tf / mfma_peak, 4), "traffic": None}
    traffic = measured_traffic() if (args.prefill, args.decode) == (
        "cca_prefill_b4_t2048", "ccgqa_decode_b64_l32768") else {}
    for key, r in rooflines.items():
        r["traffic"] = traffic.get(key)
    dominant = max(stage_ms, key=stage_ms.get)
    dom_key = dominant if dominant in rooflines else "dec_attention"

    out = {
        "metric": METRIC,
        "value": round(sp.tokens / (prefill_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": sp.dtype, "data": "synthetic",
        "config": {
            "workload": f"{args.prefill} prefill (B={sp.batch}, T={sp.seq_len}, E={sp.d_model}, "
                        f"{sp.n_q_heads}q/{sp.n_kv_heads}kv x {sp.head_dim}) + {args.decode} decode step "
                        f"(B={sd.batch}, cache {sd.cache_len}, {sd.n_q_heads}q/{sd.n_kv_heads}kv x {sd.head_dim})",
            "global_batch": sp.batch, "seq_len": sp.seq_len, "parallelism": "single GPU",
            "value_is": "prefill tokens / prefill device time (HIP events)",
        },
        "prefill_ms": round(prefill_ms, 4),
        "prefill_ms_median": round(prefill_ms_median, 4),
        "decode_ms": round(decode_ms, 4),
        "decode_step_hbm_gbs": round(dec_step_gbs, 1),
        "decode_varlen": {"lengths": f"uniform in [{L // 2}, {L}], seeded", "ms": round(varlen_ms, 4),
                          "kv_bytes": varlen_bytes,
                          "step_hbm_gbs": round(varlen_bytes / (varlen_ms * 1e-3) / 1e9, 1),
                          "attention_traffic": traffic.get("dec_attention_varlen")},
        "decode_paged": {"page_size": page, "lengths": "as decode_varlen",
                         "pages": "seeded random order", "ms": round(paged_ms, 4),
                         "step_hbm_gbs": round(varlen_bytes / (paged_ms * 1e-3) / 1e9, 1)},
        "decode_multi": {"new_tokens": multi_m, "lengths": "as decode_varlen, minus the new tokens",
                         "ms": round(multi_ms, 4),
                         "tokens_per_s": round(sd.batch * multi_m / (multi_ms * 1e-3), 1),
                         "single_token_tokens_per_s": round(sd.batch / (varlen_ms * 1e-3), 1)},
        "prefill_fused_ms": None if fused_ms is None else round(fused_ms, 4),
        "grouped_chan_conv": grouped,
        "cold_cache": {
            "flush": "512 MiB written between iterations, outside the timed region",
            "convmix_ms": round(cold["convmix"], 4),
            "convmix_gbs": round(alg["convmix_bytes"] / (cold["convmix"] * 1e-3) / 1e9, 1),
            "dec_attention_ms": round(cold["dec_attention"], 4),
            "dec_attention_gbs": round(alg["decode_attn_bytes"] / (cold["dec_attention"] * 1e-3) / 1e9, 1),
        },
        "device": {"name": torch.cuda.get_device_name(0),
                   "compute_units": torch.cuda.get_device_properties(0).multi_processor_count},
        "train": train,
        "attn_tflops": round(attn_tflops, 1),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "roofline": dict(rooflines[dom_key], kernel=dom_key,
                         algorithmic_per_launch=(alg["decode_attn_bytes"] if dom_key == "dec_attention"
                                                 else None)),
        "rooflines": rooflines,
    }
    if not args.no_cpu:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(sp, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
