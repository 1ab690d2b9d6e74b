"""GPU tests of the paged latent cache (cca_decode_step_paged,
cca_prefill_forward_paged) through the C ABI.

The cache rows of every sequence are scattered over pages in a seeded random
order; unused pages hold NaN, so a stray read shows up in the output.  The
paged step must equal the contiguous per-sequence-length step bit for bit
(same rows, same key chunking) and the fp64 oracle to the usual tolerance.
"""

import sys

import numpy as np
import pytest
import torch

import oracle.cca as O
from synth import CCAShape, make_decode, make_prefill
from gpu_helpers import assert_parity, lib, rel_l2, tens, upload_weights

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _upload_contig(D, dev="cuda"):
    T, L = tens(), lib()
    return L.State(k_cache=T.to_device(D.k_cache_s, dev), v_cache=T.to_device(D.v_cache_s, dev),
                   capacity=D.capacity, conv_q=T.to_device(D.conv_q_s, dev),
                   conv_k=T.to_device(D.conv_k_s, dev), vshift=T.to_device(D.vshift_s, dev))


def _paged_from(cache, page, mpps, seed, extra=3):
    """Scatter a contiguous [B, H, cap, d] device cache into [npages, H, page, d]
    pages in a random order; unused pages and rows past cap are NaN."""
    B, H, cap, d = cache.shape
    npages = B * mpps + extra
    perm = np.random.default_rng(seed).permutation(npages)
    table = perm[:B * mpps].reshape(B, mpps).astype(np.int32)
    pages = torch.full((npages, H, page, d), float("nan"), dtype=cache.dtype, device=cache.device)
    for b in range(B):
        for j in range(mpps):
            lo, hi = j * page, min((j + 1) * page, cap)
            if lo < hi:
                pages[table[b, j], :, :hi - lo] = cache[b, :, lo:hi]
    return pages, torch.from_numpy(table).to(cache.device)


def _gather(pages, table, b, rows):
    """Rows `rows` of sequence b from a paged cache, as [H, len(rows), d]."""
    page = pages.shape[2]
    t = table[b].cpu().numpy()
    return torch.stack([pages[int(t[r // page]), :, r % page] for r in rows], dim=1)


@pytest.mark.parametrize("page", [32, 64, 256])
def test_paged_decode_equals_contiguous_and_oracle(page):
    lens = [0, 1, 37, 1024, 2999, 3000]
    Lmax = 3000
    shape = CCAShape(batch=len(lens), seq_len=1, d_model=256, n_q_heads=8, n_kv_heads=2,
                     head_dim=64, rope_base=500000.0, cache_len=Lmax)
    _say(f"[paged] page={page} lens={lens}")
    D = make_decode(shape, seed=21, capacity=Lmax + 1)
    T, Lb = tens(), lib()
    cfg = Lb.make_config(shape)
    w = upload_weights(D.weights)
    x_t = T.to_device(D.x_s)
    dl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    ws = T.workspace(Lb.decode_workspace_size(cfg, Lmax))

    ref_st = _upload_contig(D)
    y_ref = torch.empty_like(x_t)
    Lb.decode_step_varlen(cfg, w, x_t, dl, Lmax, ref_st, ref_st, y_ref, ws)
    torch.cuda.synchronize()

    mpps = (Lmax + 1 + page - 1) // page
    src = _upload_contig(D)
    kp, table = _paged_from(src.k_cache, page, mpps, seed=page)
    vp, _ = _paged_from(src.v_cache, page, mpps, seed=page)
    pst = Lb.PagedState(kp, vp, table, page, src.conv_q, src.conv_k, src.vshift)
    y = torch.empty_like(x_t)
    Lb.decode_step_paged(cfg, w, x_t, dl, Lmax, pst, pst, y, ws)
    torch.cuda.synchronize()

    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    for b, L_ in enumerate(lens):
        got_k = _gather(kp, table, b, [L_])
        got_v = _gather(vp, table, b, [L_])
        assert torch.equal(got_k[:, 0].view(torch.int16), ref_st.k_cache[b, :, L_].view(torch.int16))
        assert torch.equal(got_v[:, 0].view(torch.int16), ref_st.v_cache[b, :, L_].view(torch.int16))
    for a, c in ((src.conv_q, ref_st.conv_q), (src.conv_k, ref_st.conv_k), (src.vshift, ref_st.vshift)):
        assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    # and the oracle, sequence by sequence
    wd = D.weights.f64()
    cq, ck, vs = D.state_f64()
    yy = T.to_f64(y)
    for b, L_ in enumerate(lens):
        K = D.cache_f64(b, "k")[None, :, :L_]
        V = D.cache_f64(b, "v")[None, :, :L_]
        ref, _ = O.decode_step(D.x[b:b + 1], wd, shape, K, V, cq[b:b + 1], ck[b:b + 1], vs[b:b + 1])
        assert_parity(yy[b:b + 1], ref, "bf16", f"paged b={b} L={L_}")


def test_paged_decode_f32_validation_mode():
    lens = [5, 700, 63]
    Lmax = 700
    shape = CCAShape(batch=3, seq_len=1, d_model=128, n_q_heads=4, n_kv_heads=2, head_dim=16,
                     dtype="f32", cache_len=Lmax)
    _say("[paged] f32")
    D = make_decode(shape, seed=5, capacity=Lmax + 1)
    T, Lb = tens(), lib()
    cfg = Lb.make_config(shape)
    src = _upload_contig(D)
    page = 64
    mpps = (Lmax + 1 + page - 1) // page
    kp, table = _paged_from(src.k_cache, page, mpps, seed=1)
    vp, _ = _paged_from(src.v_cache, page, mpps, seed=1)
    pst = Lb.PagedState(kp, vp, table, page, src.conv_q, src.conv_k, src.vshift)
    x_t = T.to_device(D.x_s)
    y = torch.empty_like(x_t)
    ws = T.workspace(Lb.decode_workspace_size(cfg, Lmax))
    Lb.decode_step_paged(cfg, upload_weights(D.weights), x_t,
                         torch.tensor(lens, dtype=torch.int32, device="cuda"), Lmax, pst, pst, y, ws)
    torch.cuda.synchronize()
    wd = D.weights.f64()
    cq, ck, vs = D.state_f64()
    yy = T.to_f64(y)
    for b, L_ in enumerate(lens):
        K = D.cache_f64(b, "k")[None, :, :L_]
        V = D.cache_f64(b, "v")[None, :, :L_]
        ref, _ = O.decode_step(D.x[b:b + 1], wd, shape, K, V, cq[b:b + 1], ck[b:b + 1], vs[b:b + 1])
        assert_parity(yy[b:b + 1], ref, "f32", f"paged f32 b={b} L={L_}")


def test_paged_prefill_then_decode_equals_contiguous():
    """Prefill writing pages, then three paged decode steps, against the same
    calls on a contiguous cache: every output and every cache row equal bit
    for bit."""
    shape = CCAShape(batch=2, seq_len=150, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                     rope_base=10000.0)
    _say(f"[paged] prefill then decode {shape}")
    P = make_prefill(shape, seed=8)
    T, Lb = tens(), lib()
    cfg = Lb.make_config(shape)
    w = upload_weights(P.weights)
    x = T.to_device(P.x_s)
    ws = T.workspace(Lb.prefill_workspace_size(cfg))
    B, H, d, steps, page = shape.batch, shape.n_kv_heads, shape.head_dim, 3, 64
    cap = shape.seq_len + steps
    sd = torch.bfloat16
    mk = lambda *s: torch.zeros(s, dtype=sd, device="cuda")
    cst = Lb.State(mk(B, H, cap, d), mk(B, H, cap, d), cap, mk(B, shape.seq_conv_k - 1, shape.e_q),
                   mk(B, shape.seq_conv_k - 1, shape.e_kv), mk(B, H // 2, d))
    mpps = (cap + page - 1) // page
    kp, table = _paged_from(cst.k_cache, page, mpps, seed=3)
    vp, _ = _paged_from(cst.v_cache, page, mpps, seed=3)
    pst = Lb.PagedState(kp, vp, table, page, mk(B, shape.seq_conv_k - 1, shape.e_q),
                        mk(B, shape.seq_conv_k - 1, shape.e_kv), mk(B, H // 2, d))
    y1, y2 = torch.empty_like(x), torch.empty_like(x)
    Lb.prefill_forward(cfg, w, x, y1, ws, cst)
    torch.cuda.synchronize()
    Lb.prefill_forward_paged(cfg, w, x, y2, ws, pst)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    for b in range(B):
        rows = list(range(shape.seq_len))
        assert torch.equal(_gather(kp, table, b, rows).view(torch.int16),
                           cst.k_cache[b, :, :shape.seq_len].view(torch.int16))
        assert torch.equal(_gather(vp, table, b, rows).view(torch.int16),
                           cst.v_cache[b, :, :shape.seq_len].view(torch.int16))
    dcfg = Lb.make_config(shape.with_(seq_len=1))
    rng = np.random.default_rng(4)
    for s_ in range(steps):
        L_ = shape.seq_len + s_
        xt = torch.from_numpy(rng.standard_normal((B, shape.d_model)).astype(np.float32)).to(
            "cuda", sd)
        dws = T.workspace(Lb.decode_workspace_size(dcfg, L_))
        ya, yb = torch.empty_like(xt), torch.empty_like(xt)
        dl = torch.full((B,), L_, dtype=torch.int32, device="cuda")
        Lb.decode_step_varlen(dcfg, w, xt, dl, L_, cst, cst, ya, dws)
        torch.cuda.synchronize()
        Lb.decode_step_paged(dcfg, w, xt, dl, L_, pst, pst, yb, dws)
        torch.cuda.synchronize()
        assert torch.equal(ya.view(torch.int16), yb.view(torch.int16)), s_
    for b in range(B):
        rows = list(range(cap))
        assert torch.equal(_gather(kp, table, b, rows).view(torch.int16),
                           cst.k_cache[b].view(torch.int16))
    assert rel_l2(T.to_f64(pst.conv_q), T.to_f64(cst.conv_q)) == 0.0


@pytest.mark.parametrize("page", [32, 256])
def test_paged_decode_full_length(page):
    """The decode workload's shape (B=64, 16 query / 4 kv heads of 64) at
    per-sequence lengths up to 32767.  Lk = 32768 keys split into two chunks
    of 16384 (the longest the chunking makes), so with 32-row pages one chunk
    spans 513 pages: the largest page list the attention kernel keeps in LDS.
    The paged step equals the contiguous per-sequence-length step bit for bit
    (outputs, new cache rows, rolled state); 8 sequences against the oracle."""
    from synth import workload
    Lmax = 32767
    shape = workload("ccgqa_decode_b64_l32768").with_(cache_len=Lmax)
    rng = np.random.default_rng(50 + page)
    lens = rng.integers(30000, Lmax + 1, size=shape.batch).astype(np.int32)
    lens[0], lens[1] = Lmax, 30000
    _say(f"[paged] full length page={page} B={shape.batch} Lmax={Lmax}")
    D = make_decode(shape, seed=51, capacity=Lmax + 1)
    T, Lb = tens(), lib()
    cfg = Lb.make_config(shape)
    w = upload_weights(D.weights)
    x_t = T.to_device(D.x_s)
    dl = torch.from_numpy(lens).to("cuda")
    ws = T.workspace(Lb.decode_workspace_size(cfg, Lmax))

    ref_st = _upload_contig(D)
    y_ref = torch.empty_like(x_t)
    Lb.decode_step_varlen(cfg, w, x_t, dl, Lmax, ref_st, ref_st, y_ref, ws)
    torch.cuda.synchronize()

    mpps = (Lmax + 1 + page - 1) // page
    src = _upload_contig(D)
    kp, table = _paged_from(src.k_cache, page, mpps, seed=page + 1)
    vp, _ = _paged_from(src.v_cache, page, mpps, seed=page + 1)
    del src.k_cache, src.v_cache
    pst = Lb.PagedState(kp, vp, table, page, src.conv_q, src.conv_k, src.vshift)
    y = torch.empty_like(x_t)
    Lb.decode_step_paged(cfg, w, x_t, dl, Lmax, pst, pst, y, ws)
    torch.cuda.synchronize()
    _say(f"[paged] full length page={page}: step done")

    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    for b, L_ in enumerate(lens):
        assert torch.equal(_gather(kp, table, b, [int(L_)])[:, 0].view(torch.int16),
                           ref_st.k_cache[b, :, L_].view(torch.int16))
        assert torch.equal(_gather(vp, table, b, [int(L_)])[:, 0].view(torch.int16),
                           ref_st.v_cache[b, :, L_].view(torch.int16))
    for a, c in ((pst.conv_q, ref_st.conv_q), (pst.conv_k, ref_st.conv_k),
                 (pst.vshift, ref_st.vshift)):
        assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    wd = D.weights.f64()
    cq, ck, vs = D.state_f64()
    yy = T.to_f64(y)
    for b in [0, 1] + sorted(rng.choice(np.arange(2, shape.batch), size=6, replace=False).tolist()):
        L_ = int(lens[b])
        K = D.cache_f64(b, "k")[None, :, :L_]
        V = D.cache_f64(b, "v")[None, :, :L_]
        ref, _ = O.decode_step(D.x[b:b + 1], wd, shape, K, V, cq[b:b + 1], ck[b:b + 1], vs[b:b + 1])
        assert_parity(yy[b:b + 1], ref, "bf16", f"paged full b={b} L={L_}")
