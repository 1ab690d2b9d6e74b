"""Benchmark of the CCA / CCGQA forward pass on one MI355X.

One step is one pass of the whole hot path over synthetic inputs resident in
HBM: a CCA prefill of the 4 x 2048-token batch (E = 2048, 8 latent heads of
64, compression 4) followed by one CCGQA decode step of 64 sequences against
a 32768-token latent cache (16 query / 4 kv heads of 64).  Both calls go
through libcca's C ABI on torch's current HIP stream.

Prints ONE JSON line.  ``value`` is prefill tokens per second of prefill time
(the K prefills of the timed steps back to back, then their K decode steps);
the decode step's HBM rate and the attention kernel's MFMA rate are reported
next to it, and under ``interleaved`` the same calls with each prefill right
after a decode step.  A second timed pass launches the kernels stage by stage,
each K times back to back between two HIP events, for per-kernel durations
(the roofline).
A fourth pass times a training step on the prefill workload
(``cca_prefill_forward_train`` + ``cca_prefill_backward``, reported under
``train``).  A fifth pass measures the two longer CCGQA prefill workloads
(8192 and 16384 tokens) on their own, kernel by kernel, under
``prefill_configs``.  The fp64 oracle is timed on the host cores on a bounded sample
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
    p.add_argument("--no-configs", action="store_true",
                   help="skip the per-kernel measurement of the 8192- and 16384-token CCGQA prefills")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--settle", type=float, default=0.3,
                   help="seconds of back-to-back steps before the warmup (clock settling)")
    p.add_argument("--compare", action="store_true",
                   help="prefill of ccgqa_prefill_t16384 next to full-width MHA and GQA-8 baselines "
                        "through the same kernels, plus a sequence-length sweep (prints its own JSON)")
    p.add_argument("--kernels-only", action="store_true",
                   help="only run the stage calls of the three bf16 prefill workloads and the decode "
                        "step, --steps times each (a short program for counter collection)")
    p.add_argument("--only", default="",
                   help="with --kernels-only: a comma-separated subset of cca_prefill_b4_t2048, "
                        "ccgqa_prefill_t8192, ccgqa_prefill_t16384, ccgqa_decode_b64_l32768")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy 5 times (the reference "
                        "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    p.add_argument("--summarize-profiles", metavar="DIR", default="",
                   help="write the profiles/ summaries from the rocprofv3 outputs under DIR "
                        "(layout in profile_summaries' docstring); needs no GPU")
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
    out = {
        # bytes the mixing step must move: read qkv~ once (16-bit in bf16 mode)
        # and write q, k (16-bit) and v (storage type) once
        "convmix_bytes": B * T * N * esz + B * T * (eq + ekv) * esz + B * T * ekv * esz,
        # causal latent attention: 2 matmuls of 2*d flops per visible (query, key) pair
        "attn_flops": 2 * 2 * B * sp.n_q_heads * sp.head_dim * T * (T + 1) / 2,
        "downproj_flops": 2 * B * T * N * E,
        "upproj_flops": 2 * B * T * E * eq,
    }
    if sd is not None:
        # decode attention streams K and V of Lk = L + 1 keys once
        out["decode_attn_bytes"] = 2 * sd.batch * sd.n_kv_heads * (sd.cache_len + 1) * sd.head_dim * 2
    return out


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
    """forward_train + backward on the prefill workload: the step and each half
    timed K calls back to back between two HIP events."""
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

    def step():
        cca.prefill_forward_train(pcfg, pw, x, y, tws)
        cca.prefill_backward(pcfg, pw, x, dy, g, tws)
    # the step, then each half on its own (the backward reads the activations
    # the last forward left in the workspace), each K calls back to back
    step_ms = launch_ms(step, K)
    fwd = launch_ms(lambda: cca.prefill_forward_train(pcfg, pw, x, y, tws), K)
    bwd = launch_ms(lambda: cca.prefill_backward(pcfg, pw, x, dy, g, tws), K)
    print(f"[bench] training step: forward {fwd:.3f} ms backward {bwd:.3f} ms", file=sys.stderr,
          flush=True)
    B, Tn, d, H = sp.batch, sp.seq_len, sp.head_dim, sp.n_q_heads
    pairs = B * H * Tn * (Tn + 1) / 2
    del tws, g, dy, y
    torch.cuda.empty_cache()
    return {"workload": "the prefill workload above, forward_train + backward, seeded dy ~ N(0,1)",
            "forward_ms": round(fwd, 4), "backward_ms": round(bwd, 4),
            "step_ms": round(step_ms, 4),
            "tokens_per_s": round(sp.tokens / (step_ms * 1e-3), 1),
            "backward_over_forward": round(bwd / fwd, 3),
            # algorithmic flops of the backward: 5 matmuls of 2d flops per visible
            # pair (S recomputed, dP, dV, dQ, dK) plus the 4 gradient GEMMs
            "backward_gflop": round((5 * 2 * d * pairs + 2 * 2 * sp.tokens * sp.d_model * (sp.n_qkv + sp.e_q))
                                    / 1e9, 2)}


def settle(fn, seconds=0.3):
    """Run fn back to back until `seconds` of wall time have passed, then
    wait for the device.  After an idle spell (the host drawing seeded
    inputs) the device takes a few tens of milliseconds of sustained load to
    raise its clocks: the prefill of the 4 x 2048-token workload goes from
    about 132 us to a steady 121-122 us over its first 200 calls.  Returns
    the number of calls."""
    import torch
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        fn()
        n += 1
        if n % 32 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def launch_ms(fn, n):
    """Average launch duration of fn (one kernel, or a short fixed sequence):
    0.05 s of untimed calls (the clocks settle under that kernel's own load),
    then n calls back to back between two HIP events on torch's current
    stream, the one the library launches on."""
    import torch
    settle(fn, 0.05)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(n):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


MIX_EVICT_BYTES = 512 << 20


def cold_convmix_ms(cca, T, cfg, pw, x, n, dev, call_bytes):
    """The mixing kernel with its input out of the 256 MiB Infinity Cache:
    nw workspaces, each holding the qkv~ that the down-projection wrote there,
    taken round-robin, so a call's input was last touched nw - 1 calls earlier,
    after at least MIX_EVICT_BYTES of other reads and writes.  One untimed
    pass over all of them and 0.05 s of round-robin calls (clock settling),
    then n calls back to back between two HIP events, the rotation carried
    on."""
    import torch
    nw = 1 + -(-MIX_EVICT_BYTES // int(call_bytes))
    wss = [T.workspace(cca.prefill_workspace_size(cfg), dev) for _ in range(nw)]
    for ws in wss:
        cca.stage_downproj(cfg, pw, x, ws)
    turn = [0]

    def rr():
        cca.stage_convmix(cfg, pw, wss[turn[0] % nw])
        turn[0] += 1
    settle(rr, 0.05)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(n):
        cca.stage_convmix(cfg, pw, wss[(turn[0] + i) % nw])
    b.record()
    torch.cuda.synchronize()
    del wss
    torch.cuda.empty_cache()
    return a.elapsed_time(b) / n, nw


def prefill_config(cca, T, name, K, dev):
    """One prefill workload on its own: cca_prefill_forward timed with HIP
    events (K iterations after two warm-up calls), then each stage's average
    launch duration (K calls back to back), then the mixing kernel with its
    input out of the Infinity Cache (its HBM figure).  Rooflines per kernel
    from the algorithmic work of algorithmic()."""
    import numpy as np
    import torch
    from synth import make_prefill, workload
    sp = workload(name)
    P = make_prefill(sp, seed=0)
    pw = upload_weights(cca, T, P.weights, dev)
    cfg = cca.make_config(sp)
    x = T.to_device(P.x_s, dev)
    y = torch.empty_like(x)
    ws = T.workspace(cca.prefill_workspace_size(cfg), dev)
    del P
    settle(lambda: cca.prefill_forward(cfg, pw, x, y, ws), 0.2)
    pre_ms = launch_ms(lambda: cca.prefill_forward(cfg, pw, x, y, ws), K)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for a, b_ in ev:
        a.record()
        cca.prefill_forward(cfg, pw, x, y, ws)
        b_.record()
    torch.cuda.synchronize()
    times = [a.elapsed_time(b_) for a, b_ in ev]
    st = {
        "downproj": launch_ms(lambda: cca.stage_downproj(cfg, pw, x, ws), K),
        "convmix": launch_ms(lambda: cca.stage_convmix(cfg, pw, ws), K),
        "attention": launch_ms(lambda: cca.stage_attention(cfg, pw, ws), K),
        "upproj": launch_ms(lambda: cca.stage_upproj(cfg, pw, y, ws), K),
    }
    del ws
    torch.cuda.empty_cache()
    alg = algorithmic(sp, None)
    cold, nw = cold_convmix_ms(cca, T, cfg, pw, x, K, dev, alg["convmix_bytes"])
    del x, y
    torch.cuda.empty_cache()
    peak = PEAK_BF16_TFLOPS if sp.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS

    def mfma(flops, ms):
        tf = flops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(tf, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(tf / peak, 4), "ms": round(ms, 4)}
    conv_cold = alg["convmix_bytes"] / (cold * 1e-3) / 1e9
    print(f"[bench] {name}: prefill {pre_ms:.3f} ms, attention {st['attention']:.3f} ms, "
          f"mixing {cold * 1e3:.1f} us cold", file=sys.stderr, flush=True)
    return {
        "shape": f"B={sp.batch}, T={sp.seq_len}, E={sp.d_model}, {sp.n_q_heads}q/{sp.n_kv_heads}kv x "
                 f"{sp.head_dim}, {sp.dtype}",
        "prefill_ms": round(pre_ms, 4),
        "per_call_events": {"prefill_ms_mean": round(sum(times) / K, 4),
                            "prefill_ms_median": round(float(np.median(times)), 4)},
        "tokens_per_s": round(sp.tokens / (pre_ms * 1e-3), 1),
        "stage_ms": {k: round(v, 4) for k, v in st.items()},
        "rooflines": {
            "attention": mfma(alg["attn_flops"], st["attention"]),
            "downproj": mfma(alg["downproj_flops"], st["downproj"]),
            "upproj": mfma(alg["upproj_flops"], st["upproj"]),
            "convmix": {"bound": "hbm", "achieved": round(conv_cold, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(conv_cold / PEAK_HBM_GBS, 4),
                        "ms": round(cold, 4), "bytes": alg["convmix_bytes"],
                        "timing": f"input out of the Infinity Cache ({nw} workspaces round-robin), "
                                  f"calls back to back",
                        "warm_ms": round(st["convmix"], 4)},
        },
    }


TRAIN_WORKLOAD = "train_cca_prefill_b4_t2048"
KERNEL_WORKLOADS = ("cca_prefill_b4_t2048", "ccgqa_prefill_t8192", "ccgqa_prefill_t16384",
                    "ccgqa_decode_b64_l32768")


def kernels_only(args):
    """The stage calls of the three bf16 prefill workloads and of the decode
    step, --steps times each after one warm-up call: a short program whose
    dispatches a counter pass can attribute to kernels."""
    import torch
    from efficient_transformer_attention_amd import cca, tensors as T
    from synth import make_decode, make_prefill, workload
    dev = "cuda:0"
    torch.cuda.set_device(0)
    only = [n for n in args.only.split(",") if n] or list(KERNEL_WORKLOADS)
    for name in ("cca_prefill_b4_t2048", "ccgqa_prefill_t8192", "ccgqa_prefill_t16384"):
        if name not in only:
            continue
        sp = workload(name)
        P = make_prefill(sp, seed=0)
        pw = upload_weights(cca, T, P.weights, dev)
        cfg = cca.make_config(sp)
        x = T.to_device(P.x_s, dev)
        y = torch.empty_like(x)
        ws = T.workspace(cca.prefill_workspace_size(cfg), dev)
        for _ in range(args.steps + 1):
            cca.stage_downproj(cfg, pw, x, ws)
            cca.stage_convmix(cfg, pw, ws)
            cca.stage_attention(cfg, pw, ws)
            cca.stage_upproj(cfg, pw, y, ws)
        torch.cuda.synchronize()
        print(f"[kernels] {name} done", file=sys.stderr, flush=True)
        del ws, x, y, pw, P
        torch.cuda.empty_cache()
    if TRAIN_WORKLOAD in only:
        # forward_train + backward on the B4 x T2048 prefill shape
        from synth import make_upstream_grad
        sp = workload("cca_prefill_b4_t2048")
        P = make_prefill(sp, seed=0)
        pw = upload_weights(cca, T, P.weights, dev)
        cfg = cca.make_config(sp)
        x = T.to_device(P.x_s, dev)
        y = torch.empty_like(x)
        dy = T.to_device(make_upstream_grad(sp, seed=0).dy_s, dev)
        tws = T.workspace(cca.train_workspace_size(cfg), dev)
        f32 = dict(dtype=torch.float32, device=dev)
        g = cca.Grads(torch.empty_like(x), torch.empty((sp.n_qkv, sp.d_model), **f32),
                      torch.empty((sp.d_model, sp.e_q), **f32),
                      torch.empty((sp.e_q, sp.seq_conv_k), **f32),
                      torch.empty((sp.e_kv, sp.seq_conv_k), **f32),
                      torch.empty((sp.n_q_heads, sp.chan_conv_k), **f32),
                      torch.empty((sp.n_kv_heads, sp.chan_conv_k), **f32),
                      torch.empty((sp.n_q_heads,), **f32))
        for _ in range(args.steps + 1):
            cca.prefill_forward_train(cfg, pw, x, y, tws)
            cca.prefill_backward(cfg, pw, x, dy, g, tws)
        torch.cuda.synchronize()
        print("[kernels] training step done", file=sys.stderr, flush=True)
        del tws, g, dy, x, y
        torch.cuda.empty_cache()
    if "ccgqa_decode_b64_l32768" not in only:
        return
    sd = workload("ccgqa_decode_b64_l32768")
    D = make_decode(sd, seed=0)
    dw = upload_weights(cca, T, D.weights, dev)
    cfg = cca.make_config(sd)
    st = cca.State(T.to_device(D.k_cache_s, dev), T.to_device(D.v_cache_s, dev), D.capacity,
                   T.to_device(D.conv_q_s, dev), T.to_device(D.conv_k_s, dev),
                   T.to_device(D.vshift_s, dev))
    xt = T.to_device(D.x_s, dev)
    yt = torch.empty_like(xt)
    ws = T.workspace(cca.decode_workspace_size(cfg, sd.cache_len), dev)
    for _ in range(args.steps + 1):
        cca.decode_step(cfg, dw, xt, sd.cache_len, st, st, yt, ws)
    torch.cuda.synchronize()
    print("[kernels] decode done", file=sys.stderr, flush=True)


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
        # as in the main run: clocks settled, K calls back to back between two
        # HIP events (the attention stage reads what the last prefill left)
        settle(lambda: cca.prefill_forward(cfg, pw, x, y, ws), 0.2)
        pre = launch_ms(lambda: cca.prefill_forward(cfg, pw, x, y, ws), K)
        att = launch_ms(lambda: cca.stage_attention(cfg, pw, ws), K)
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


# ---- profile summaries (rocprofv3 outputs -> profiles/) ---------------------

PROFILE_SOURCES = {
    "downproj": ["gemm.hip", "gemm_tile.h", "cca_device.h", "cca_launch.h"],
    "upproj": ["gemm.hip", "gemm_tile.h", "cca_device.h", "cca_launch.h"],
    "convmix": ["convmix.hip", "gemm_tile.h", "cca_device.h", "cca_launch.h"],
    "attention": ["attn_fwd.hip", "cca_device.h", "cca_launch.h"],
    "dec_attention": ["attn_decode.hip", "cca_device.h", "cca_launch.h"],
}
MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16 "
                 "SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU SQ_WAVES")


def _source_hash(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "efficient_transformer_attention_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def _counter_dispatches(path):
    """Per dispatch of a rocprofv3 counter pass (its rocpd database under
    path): kernel name, duration in ns and every counter summed over the
    instances that report it, in dispatch order."""
    import glob
    import sqlite3
    dbs = sorted(glob.glob(os.path.join(path, "**", "*.db"), recursive=True))
    if not dbs:
        raise FileNotFoundError(f"no rocpd database under {path}")
    rows = sqlite3.connect(dbs[0]).execute(
        "select dispatch_id, kernel_name, counter_name, value, duration from counters_collection").fetchall()
    out = {}
    for did, name, cn, v, dur in rows:
        d = out.setdefault(did, {"name": name, "dur_ns": float(dur)})
        d[cn] = d.get(cn, 0.0) + float(v)
    return [out[k] for k in sorted(out)]


def _stages(dispatches):
    """Label the libcca dispatches of a kernels-only run by pipeline stage
    (the first dispatch of every stage is the warm-up and is dropped)."""
    lab, prev = {}, None
    for d in dispatches:
        n = d["name"]
        if "convmix_prefill" in n:
            st = "convmix"
        elif "attn_fwd" in n:
            st = "attention"
        elif "gemm_nt_dma" in n:
            st = "upproj" if prev == "attention" else "downproj"
        elif "attn_decode_mfma" in n:
            st = "dec_attention"
        elif "attn_decode_combine" in n:
            st = "dec_combine"
        elif "convmix_decode" in n:
            st = "dec_mix"
        elif "splitk_reduce" in n:
            st = "dec_upproj_reduce"
        elif "gemm_nt_kernel" in n:
            st = "dec_upproj" if prev in ("dec_combine", "dec_attention") else "dec_downproj"
        else:
            continue
        prev = st
        lab.setdefault(st, []).append(d)
    return {k: v[1:] or v for k, v in lab.items()}


def _avg(ds, key):
    return sum(d.get(key, 0.0) for d in ds) / len(ds)


def profile_summaries(d):
    """Writes the profiles/ summaries from rocprofv3 outputs under d:
      d/trace        kernel trace (--kernel-trace --stats --output-format csv) of
                     `bench.py --steps 5 --warmup 1 --no-cpu`;
      d/<pass>_<w>   counter passes (rocpd output) of `bench.py --kernels-only
                     --steps 3 --only <w>` for pass in mfma (MFMA_COUNTERS),
                     fetch (FETCH_SIZE), write (WRITE_SIZE) and w in
                     KERNEL_WORKLOADS;
      d/fetch_copy, d/write_copy   the same two counters on `bench.py
                     --calibrate-copy` (a plain 1 GiB copy, which scales them).
    The command lines are recorded in the summaries."""
    import csv
    import glob
    from synth import workload
    prof = os.path.join(ROOT, "profiles")
    ws = list(KERNEL_WORKLOADS)
    run = "cd /tmp && rocprofv3"
    # ---- kernel trace of the default bench command
    stats = sorted(glob.glob(os.path.join(d, "trace", "**", "*kernel_stats.csv"), recursive=True))
    if stats:
        rows = list(csv.DictReader(open(stats[0])))
        lines = [
            "# Kernel durations: bench.py default run (prefill B4 x T2048, the 8192- and 16384-token "
            "CCGQA prefills, decode B64 x L32768)", "",
            "```", f"{run} --kernel-trace --stats --output-format csv -d gpurun_out/prof/trace -o run "
                   "-- python3 $REPO/bench.py --steps 5 --warmup 1 --no-cpu", "```", "",
            "| kernel | calls | average (us) | share |", "|---|---|---|---|"]
        for r in rows:
            lines.append(f"| `{r['Name'][:110]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                         f"{float(r['Percentage']):.1f}% |")
        open(os.path.join(prof, "kernel_trace_prefill_b4_t2048_t8192_t16384_decode_b64_l32768.md"),
             "w").write("\n".join(lines) + "\n")
    # ---- copy calibration of FETCH_SIZE / WRITE_SIZE
    if not os.path.isdir(os.path.join(d, "fetch_copy")) or not os.path.isdir(os.path.join(d, "write_copy")):
        print("no counter passes under " + d + ": kernel trace summary only", file=sys.stderr)
        return
    cf = [x for x in _counter_dispatches(os.path.join(d, "fetch_copy")) if "FETCH_SIZE" in x]
    cw = [x for x in _counter_dispatches(os.path.join(d, "write_copy")) if "WRITE_SIZE" in x]
    if not cf or not cw:
        print("no counter passes under " + d + ": kernel trace summary only", file=sys.stderr)
        return
    big = lambda xs, k: max(xs, key=lambda x: x[k])
    n_copy = 1 << 30
    fetch_factor = n_copy / (big(cf, "FETCH_SIZE")["FETCH_SIZE"] * 1024)
    write_factor = n_copy / (big(cw, "WRITE_SIZE")["WRITE_SIZE"] * 1024)
    # ---- per workload: MFMA utilisation and HBM traffic per stage
    mf_lines = ["# MFMA utilisation per kernel (rocprofv3 counters)", "",
                "MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs), the "
                "share of the kernel's cycles in which the matrix cores were busy (at whatever clock "
                "the chip ran); MFMA TFLOP/s = (SQ_INSTS_VALU_MFMA_MOPS_BF16 + _F16) x 512 / duration; "
                "algorithmic TFLOP/s counts only the product's own flops (no padding or masked "
                "work) against the 2.5 PFLOP/s bf16 peak.  Durations are those of the profiled run "
                "(short kernels run longer under the profiler).", "",
                "```", f"{run} --pmc {MFMA_COUNTERS} -d gpurun_out/prof/mfma_<w> -o k -- python3 "
                       "$REPO/bench.py --kernels-only --steps 3 --only <w>", "```", ""]
    tr_lines = ["# HBM traffic per launch (FETCH_SIZE, WRITE_SIZE)", "",
                "Each counter in its own pass, scaled by what it reads for a plain 1 GiB device copy "
                f"(factors: FETCH x{fetch_factor:.3f}, WRITE x{write_factor:.3f}).", "",
                "```",
                f"{run} --pmc FETCH_SIZE -d gpurun_out/prof/fetch_<w> -o k -- python3 $REPO/bench.py "
                "--kernels-only --steps 3 --only <w>",
                f"{run} --pmc WRITE_SIZE -d gpurun_out/prof/write_<w> -o k -- python3 $REPO/bench.py "
                "--kernels-only --steps 3 --only <w>",
                f"{run} --pmc FETCH_SIZE -d gpurun_out/prof/fetch_copy -o k -- python3 $REPO/bench.py "
                "--calibrate-copy",
                f"{run} --pmc WRITE_SIZE -d gpurun_out/prof/write_copy -o k -- python3 $REPO/bench.py "
                "--calibrate-copy", "```", ""]
    traffic = {"fetch_factor": round(fetch_factor, 4), "write_factor": round(write_factor, 4),
               "calibration": "1 GiB device copy", "kernels": {}}
    for w in ws:
        sp = workload(w)
        if sp.cache_len > 0:   # decode: the cache stream of one step
            alg = {"decode_attn_bytes": 2 * sp.batch * sp.n_kv_heads * (sp.cache_len + 1) * sp.head_dim * 2}
        else:
            alg = algorithmic(sp, None)
        mf = _stages(_counter_dispatches(os.path.join(d, f"mfma_{w}")))
        fe = _stages(_counter_dispatches(os.path.join(d, f"fetch_{w}")))
        wr = _stages(_counter_dispatches(os.path.join(d, f"write_{w}")))
        mf_lines += [f"## {w}", "", "| kernel | stage | avg (us) | MfmaUtil | MFMA TFLOP/s | "
                     "algorithmic TFLOP/s (of 2500) |", "|---|---|---|---|---|---|"]
        tr_lines += [f"## {w}", "", "| kernel | stage | FETCH (KiB) | WRITE (KiB) | scaled bytes | "
                     "algorithmic bytes | ratio |", "|---|---|---|---|---|---|---|"]
        for st, ds in mf.items():
            dur = _avg(ds, "dur_ns")
            cyc = _avg(ds, "GRBM_GUI_ACTIVE") / 8
            util = _avg(ds, "SQ_VALU_MFMA_BUSY_CYCLES") / (cyc * 1024) if cyc else 0.0
            mops = (_avg(ds, "SQ_INSTS_VALU_MFMA_MOPS_BF16") + _avg(ds, "SQ_INSTS_VALU_MFMA_MOPS_F16")) * 512
            af = {"downproj": "downproj_flops", "upproj": "upproj_flops", "attention": "attn_flops"}.get(st)
            atf = f"{alg[af] / (dur * 1e-9) / 1e12:.0f} ({alg[af] / (dur * 1e-9) / 1e12 / 25:.1f}%)" if af else "-"
            mf_lines.append(f"| `{ds[0]['name'][:70]}` | {st} | {dur / 1e3:.1f} | "
                            f"{100 * util:.1f}% | {mops / dur / 1e3:.0f} | {atf} |")
        for st in fe:
            if st not in wr:
                continue
            fk, wk = _avg(fe[st], "FETCH_SIZE"), _avg(wr[st], "WRITE_SIZE")
            byt = fk * 1024 * fetch_factor + wk * 1024 * write_factor
            ab = {"convmix": "convmix_bytes", "dec_attention": "decode_attn_bytes"}.get(st)
            abs_ = f"{alg[ab]:.4g} | {byt / alg[ab]:.3f}" if ab else "- | -"
            tr_lines.append(f"| `{fe[st][0]['name'][:70]}` | {st} | {fk:.1f} | {wk:.1f} | {byt:.4g} | {abs_} |")
            key = st if w in ("cca_prefill_b4_t2048", "ccgqa_decode_b64_l32768") else None
            if key in PROFILE_SOURCES:
                traffic["kernels"][key] = {"kernel": fe[st][0]["name"], "workload": w,
                                           "sources": PROFILE_SOURCES[key],
                                           "source_sha256_16": _source_hash(PROFILE_SOURCES[key]),
                                           "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                                           "bytes": int(byt)}
        mf_lines.append("")
        tr_lines.append("")
    # ---- training step: the attention backward kernels (and the rest of the
    # backward, without algorithmic figures), grouped by kernel
    tdir = os.path.join(d, f"mfma_{TRAIN_WORKLOAD}")
    if os.path.isdir(tdir):
        sp = workload("cca_prefill_b4_t2048")
        pairs = sp.batch * sp.n_q_heads * sp.seq_len * (sp.seq_len + 1) / 2
        bwd_flops = {"attn_bwd_dkdv": 4 * 2 * sp.head_dim * pairs,   # S, dP, dV, dK
                     "attn_bwd_dq": 3 * 2 * sp.head_dim * pairs}     # S, dP, dQ
        byname = {}
        for x in _counter_dispatches(tdir):
            if "cca" in x["name"]:
                byname.setdefault(x["name"], []).append(x)
        mf_lines += [f"## {TRAIN_WORKLOAD} (forward_train + backward on the B4 x T2048 shape)", "",
                     f"`--only {TRAIN_WORKLOAD}`; every kernel of the step, averaged over its "
                     "dispatches after the first.  Algorithmic flops of the two attention-backward "
                     "kernels: 2 d per visible (query, key) pair and matrix product, 4 products in "
                     "dK/dV (S, dP, dV, dK) and 3 in dQ (S, dP, dQ; S is recomputed in both).", "",
                     "| kernel | dispatches | avg (us) | MfmaUtil | MFMA TFLOP/s | algorithmic TFLOP/s "
                     "(of 2500) |", "|---|---|---|---|---|---|"]
        for name, ds in sorted(byname.items(), key=lambda kv: -sum(x["dur_ns"] for x in kv[1])):
            ds = ds[1:] or ds
            dur = _avg(ds, "dur_ns")
            cyc = _avg(ds, "GRBM_GUI_ACTIVE") / 8
            util = _avg(ds, "SQ_VALU_MFMA_BUSY_CYCLES") / (cyc * 1024) if cyc else 0.0
            mops = (_avg(ds, "SQ_INSTS_VALU_MFMA_MOPS_BF16") + _avg(ds, "SQ_INSTS_VALU_MFMA_MOPS_F16")) * 512
            fl = next((v for k, v in bwd_flops.items() if k in name), None)
            atf = f"{fl / (dur * 1e-9) / 1e12:.0f} ({fl / (dur * 1e-9) / 1e12 / 25:.1f}%)" if fl else "-"
            mf_lines.append(f"| `{name[:70]}` | {len(ds)} | {dur / 1e3:.1f} | {100 * util:.1f}% | "
                            f"{mops / dur / 1e3:.0f} | {atf} |")
        mf_lines.append("")
    open(os.path.join(prof, "mfma_util_prefill_b4_t2048_t8192_t16384_decode_b64_l32768.md"), "w").write(
        "\n".join(mf_lines) + "\n")
    open(os.path.join(prof, "hbm_traffic_prefill_b4_t2048_t8192_t16384_decode_b64_l32768.md"), "w").write(
        "\n".join(tr_lines) + "\n")
    json.dump(traffic, open(os.path.join(prof, "pmc_traffic.json"), "w"), indent=1)
    print("wrote profiles/ summaries", flush=True)


def main():
    args = parse()
    if args.summarize_profiles:
        profile_summaries(args.summarize_profiles)
        return
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.compare:
        compare(args)
        return
    if args.kernels_only:
        kernels_only(args)
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

    settle_steps = settle(step, args.settle)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] settled ({settle_steps} steps in {args.settle} s), warmup done", file=sys.stderr,
          flush=True)

    # ---- timed region 1: the public entry points ---------------------------
    # K steps: the K prefills back to back, then the K decode steps back to
    # back, with HIP events only around each of the two runs (an event
    # recorded between two calls idles the device while it is written)
    K = args.steps
    ea, eb, ed = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ea.record()
    for _ in range(K):
        cca.prefill_forward(pcfg, pw, x, y, pws)
    eb.record()
    for _ in range(K):
        cca.decode_step(dcfg, dw, xt, L, st, st, yt, dws)
    ed.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prefill_ms = ea.elapsed_time(eb) / K
    decode_ms = eb.elapsed_time(ed) / K
    ms_per_step = wall * 1e3 / K
    print(f"[bench] timed {K} steps: prefill {prefill_ms:.3f} ms decode {decode_ms:.3f} ms",
          file=sys.stderr, flush=True)

    # ---- timed region 1a: the same calls, each between two HIP events (the
    # spread of single calls; every call also carries the events' cost) ------
    evp = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    evd = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    for a, b_ in evp:
        a.record()
        cca.prefill_forward(pcfg, pw, x, y, pws)
        b_.record()
    for a, b_ in evd:
        a.record()
        cca.decode_step(dcfg, dw, xt, L, st, st, yt, dws)
        b_.record()
    torch.cuda.synchronize()
    prefill_times = [a.elapsed_time(b_) for a, b_ in evp]
    prefill_call_ms = sum(prefill_times) / K
    prefill_ms_median = float(np.median(prefill_times))
    decode_call_ms = sum(a.elapsed_time(b_) for a, b_ in evd) / K

    # ---- timed region 1b: the same calls interleaved, each prefill right
    # after a decode step (for reference: the clock falls during the memory-
    # bound decode step and the prefill that follows runs slower) ----------
    evi = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    for e in evi:
        e[0].record()
        cca.decode_step(dcfg, dw, xt, L, st, st, yt, dws)
        e[1].record()
        cca.prefill_forward(pcfg, pw, x, y, pws)
        e[2].record()
    torch.cuda.synchronize()
    inter_prefill_ms = sum(e[1].elapsed_time(e[2]) for e in evi) / K
    inter_decode_ms = sum(e[0].elapsed_time(e[1]) for e in evi) / K

    # ---- timed region 2: stage by stage, each stage's average launch
    # duration (K calls back to back between two HIP events, in pipeline order
    # so every stage reads what the one before it wrote) ---------------------
    stage_ms = {
        "downproj": launch_ms(lambda: cca.stage_downproj(pcfg, pw, x, pws), K),
        "convmix": launch_ms(lambda: cca.stage_convmix(pcfg, pw, pws), K),
        "attention": launch_ms(lambda: cca.stage_attention(pcfg, pw, pws), K),
        "upproj": launch_ms(lambda: cca.stage_upproj(pcfg, pw, y, pws), K),
        "dec_downproj": launch_ms(lambda: cca.stage_decode_downproj(dcfg, dw, xt, L, dws), K),
        "dec_mix": launch_ms(lambda: cca.stage_decode_mix(dcfg, dw, L, st, st, dws), K),
        "dec_attention": launch_ms(lambda: cca.stage_decode_attention(dcfg, dw, L, st, dws), K),
        "dec_upproj": launch_ms(lambda: cca.stage_decode_upproj(dcfg, dw, L, yt, dws), K),
    }

    # ---- timed region 2b: the two HBM-bound kernels reading from HBM: the
    # mixing kernel over workspaces taken round-robin (each call's input long
    # evicted from the Infinity Cache); decode attention's 2.15 GB stream is
    # eight times the cache, so its back-to-back time above is already cold --
    alg = algorithmic(sp, sd)
    cold_mix, mix_nw = cold_convmix_ms(cca, T, pcfg, pw, x, K, dev, alg["convmix_bytes"])
    cold = {"convmix": cold_mix, "dec_attention": stage_ms["dec_attention"]}

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

    # ---- timed region 5: the two longer CCGQA prefill workloads, each on
    # its own (per-kernel rooflines; the mixing kernel with a cold cache) --
    configs = {}
    if not args.no_configs:
        del pws
        torch.cuda.empty_cache()
        for name in ("ccgqa_prefill_t8192", "ccgqa_prefill_t16384"):
            configs[name] = prefill_config(cca, T, name, K, dev)

    attn_tflops = alg["attn_flops"] / (stage_ms["attention"] * 1e-3) / 1e12
    # the mixing kernel's HBM figure: its input out of the Infinity Cache (in
    # the pipeline it reads qkv~ that the down-projection has just left in the
    # cache; that warm time is reported next to it)
    conv_gbs = alg["convmix_bytes"] / (cold["convmix"] * 1e-3) / 1e9
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
                    "unit": "GB/s", "frac": round(conv_gbs / PEAK_HBM_GBS, 4), "traffic": None,
                    "bytes": alg["convmix_bytes"], "ms": round(cold["convmix"], 4),
                    "timing": f"input out of the Infinity Cache ({mix_nw} workspaces round-robin), "
                              f"calls back to back",
                    "warm_ms": round(stage_ms["convmix"], 4)},
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
        "settle": {"seconds": args.settle, "steps": settle_steps,
                   "why": "back-to-back steps before the warmup, so the timed steps run at settled clocks"},
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": sp.dtype, "data": "synthetic",
        "config": {
            "workload": f"{args.prefill} prefill (B={sp.batch}, T={sp.seq_len}, E={sp.d_model}, "
                        f"{sp.n_q_heads}q/{sp.n_kv_heads}kv x {sp.head_dim}) + {args.decode} decode step "
                        f"(B={sd.batch}, cache {sd.cache_len}, {sd.n_q_heads}q/{sd.n_kv_heads}kv x {sd.head_dim})",
            "global_batch": sp.batch, "seq_len": sp.seq_len, "parallelism": "single GPU",
            "value_is": "prefill tokens / prefill device time (K prefills back to back between two HIP events)",
        },
        "prefill_ms": round(prefill_ms, 4),
        "per_call_events": {"prefill_ms_mean": round(prefill_call_ms, 4),
                            "prefill_ms_median": round(prefill_ms_median, 4),
                            "decode_ms_mean": round(decode_call_ms, 4)},
        "interleaved": {"order": "decode step, then prefill, K times", "prefill_ms": round(inter_prefill_ms, 4),
                        "decode_ms": round(inter_decode_ms, 4),
                        "prefill_tokens_per_s": round(sp.tokens / (inter_prefill_ms * 1e-3), 1)},
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
            "method": f"mixing: {mix_nw} workspaces taken round-robin, so each call's input was last "
                      f"touched after at least {MIX_EVICT_BYTES >> 20} MiB of other traffic, calls back to "
                      f"back; decode attention: its stream is eight times the 256 MiB cache",
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
        "prefill_configs": configs,
    }
    if not args.no_cpu:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(sp, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
