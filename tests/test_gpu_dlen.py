"""Device-resident length: the *_dlen calls against the oracle, and a whole
draft-verify-accept cycle captured once in a HIP graph and replayed.

The cycle follows the pages' decoding procedure (technical summary,
Methodology item 3): gamma sparse draft steps at lengths t+1 .. t+gamma,
one dense verify of gamma+1 queries at length t+gamma+1, then greedy
acceptance, which advances the device length by n+1.  Each replay is
checked against eager host-length calls at the length the replay saw, with
eager work and synchronisations between replays.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_draft_speculative_amd as sd
    sd.load()
    return sd


def f64(t):
    return t.detach().double().cpu().numpy()


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


@pytest.fixture(scope="module")
def c2(lib):
    cfg = synth.config("c2", extra=64)
    lay = synth.attention_layer(cfg, 0, device="cuda")
    idx_ref, _ = oracle.select_topk(f64(lay["q_text"]), f64(lay["k"]), cfg.text_start,
                                    cfg.vis_start, cfg.vis_len, cfg.topk)
    idx = torch.from_numpy(np.asarray(idx_ref, dtype=np.int32)).cuda()
    return cfg, lay, idx, np.asarray(idx_ref)


def test_dlen_calls_match_oracle(lib, c2):
    cfg, lay, idx, idx_np = c2
    kf, vf = f64(lay["k"]), f64(lay["v"])
    cap = cfg.capacity
    for t in (cfg.ctx, cfg.ctx + 17, cap - cfg.gamma - 1):
        seq = torch.tensor([t], dtype=torch.int32, device="cuda")
        q = lay["q_draft"][0].contiguous()
        out = lib.std_sparse_decode_attn_dlen(q, lay["k"], lay["v"], cap, seq, 1, cfg.vis_start,
                                              cfg.vis_len, idx)
        qv = lay["q_verify"]
        outv = lib.std_dense_verify_attn_dlen(qv, lay["k"], lay["v"], cap, seq, cfg.gamma + 1)
        torch.cuda.synchronize()
        ref = oracle.sparse_decode(f64(q), kf, vf, t + 1, cfg.vis_start, cfg.vis_len, idx_np)
        refv = oracle.dense_verify(f64(qv), kf, vf, t + cfg.gamma + 1)
        say(f"t={t}: sparse err {max_abs(f64(out), ref):.2e} dense err "
            f"{max_abs(f64(outv), refv):.2e}")
        assert max_abs(f64(out), ref) <= TOL
        assert max_abs(f64(outv), refv) <= TOL


@pytest.mark.parametrize("n_q", [10, 17])
def test_dlen_long_verify_matches_oracle(lib, c2, n_q):
    """Draft lengths of 9 and 16 (70 and 119 query rows per KV head: the
    128-row verify workgroups) with the length read on the device."""
    cfg, lay, _, _ = c2
    kf, vf = f64(lay["k"]), f64(lay["v"])
    cap = cfg.capacity
    g = torch.Generator(device="cuda").manual_seed(n_q)
    qv = (torch.randn(n_q, cfg.n_q_heads, cfg.head_dim, generator=g, device="cuda") * 1.5
          ).bfloat16()
    for t in (cfg.ctx, cfg.ctx + 31):
        seq = torch.tensor([t], dtype=torch.int32, device="cuda")
        out = lib.std_dense_verify_attn_dlen(qv, lay["k"], lay["v"], cap, seq, n_q)
        torch.cuda.synchronize()
        ref = oracle.dense_verify(f64(qv), kf, vf, t + n_q)
        say(f"n_q={n_q} t={t}: dense err {max_abs(f64(out), ref):.2e}")
        assert max_abs(f64(out), ref) <= TOL


def test_dlen_at_the_bound_equals_host_length(lib, c2):
    """With the device length equal to the bound the launch is the host-length
    launch: results are bitwise equal."""
    cfg, lay, idx, _ = c2
    L = cfg.verify_len
    seq = torch.tensor([L], dtype=torch.int32, device="cuda")
    a = lib.std_dense_verify_attn_dlen(lay["q_verify"], lay["k"], lay["v"], L, seq, 0)
    b = lib.std_dense_verify_attn(lay["q_verify"], lay["k"], lay["v"], L)
    q = lay["q_draft"][0].contiguous()
    c = lib.std_sparse_decode_attn_dlen(q, lay["k"], lay["v"], L, seq, 0, cfg.vis_start,
                                        cfg.vis_len, idx)
    d = lib.std_sparse_decode_attn(q, lay["k"], lay["v"], L, cfg.vis_start, cfg.vis_len, idx)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(c, d)


def test_graph_replayed_cycle(lib, c2):
    cfg, lay, idx, _ = c2
    G, cap = cfg.gamma, cfg.capacity
    dev = torch.device("cuda")
    shape = lib.attn_shape(cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim)
    ws_s = torch.zeros(lib.std_sparse_decode_workspace(shape, lay["k"], cap, cfg.vis_start,
                                                       cfg.vis_len, cfg.topk), dtype=torch.uint8,
                       device=dev)
    ws_d = torch.zeros(lib.std_dense_verify_workspace(shape, G + 1, lay["k"], cap),
                       dtype=torch.uint8, device=dev)
    seq = torch.tensor([cfg.ctx], dtype=torch.int32, device=dev)
    q_draft = [lay["q_draft"][j].contiguous() for j in range(G)]
    outs = [torch.empty_like(q_draft[0]) for _ in range(G)]
    out_v = torch.empty_like(lay["q_verify"])
    draft, logits = synth.accept_case(G, 4096, 0.7, seed=11)
    draft, logits = draft.to(dev), logits.to(dev)
    toks = torch.empty(G + 1, dtype=torch.int32, device=dev)
    n_out = torch.empty(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.Stream()
    calls = [lib.prepare_sparse_decode_dlen(q_draft[j], lay["k"], lay["v"], cfg.vis_start,
                                            cfg.vis_len, idx, outs[j], ws_s, seq, 1 + j,
                                            stream=stream)
             for j in range(G)]
    calls.append(lib.prepare_dense_verify_dlen(lay["q_verify"], lay["k"], lay["v"], out_v, ws_d,
                                               seq, G + 1, stream=stream))

    def cycle():
        for c in calls:
            c()
        lib.std_accept(draft, logits, out_tokens=toks, n_out=n_out, seq_len=seq)

    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        cycle()                                    # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    seq.fill_(cfg.ctx)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        cycle()
    torch.cuda.synchronize()
    seq.fill_(cfg.ctx)
    torch.cuda.synchronize()
    for rep in range(3):
        t = int(seq.item())
        graph.replay()
        torch.cuda.synchronize()
        # eager reference at the length this replay saw
        for j in range(G):
            ref = lib.std_sparse_decode_attn(q_draft[j], lay["k"], lay["v"], t + 1 + j,
                                             cfg.vis_start, cfg.vis_len, idx)
            torch.cuda.synchronize()
            assert max_abs(f64(outs[j]), f64(ref)) <= 1e-2, (rep, j)
        refv = lib.std_dense_verify_attn(lay["q_verify"], lay["k"], lay["v"], t + G + 1)
        torch.cuda.synchronize()
        assert max_abs(f64(out_v), f64(refv)) <= 1e-2, rep
        ref_toks, ref_n, _, _ = oracle.accept(draft.cpu().numpy(), f64(logits))
        assert toks.cpu().numpy().tolist() == list(ref_toks)
        assert int(n_out.item()) == ref_n
        assert int(seq.item()) == t + ref_n, "the accept step advances the device length"
        say(f"replay {rep}: t={t} -> {int(seq.item())}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_dlen_below_the_shortest_length_is_raised_to_it(lib, dtype):
    """A device length shorter than the call is defined for resolves to the
    shortest defined length (dense: n_q, so every query row sees a key;
    sparse: the end of the visual span, one past it when the key list would
    otherwise be empty), so the output is a defined attention result, never
    NaN."""
    g = torch.Generator(device="cpu").manual_seed(21)
    hq, hkv, d, vis_len, cap, n_q, topk = 8, 2, 128, 300, 400, 7, 32
    k = torch.randn(hkv, cap, d, generator=g).to(dtype)
    v = torch.randn(hkv, cap, d, generator=g).to(dtype)
    qv = torch.randn(n_q, hq, d, generator=g).to(dtype)
    q1 = torch.randn(hq, d, generator=g).to(dtype)
    idx = torch.stack([torch.sort(torch.randperm(vis_len, generator=g)[:topk])[0]
                       for _ in range(hkv)]).to(torch.int32)
    kc, vc, qvc, q1c, idxc = (t.cuda() for t in (k, v, qv, q1, idx))
    kf, vf = f64(k), f64(v)
    tol = 1e-5 if dtype == torch.float32 else TOL
    for dev_len in (-50, 0, 3):
        seq = torch.tensor([dev_len], dtype=torch.int32, device="cuda")
        outv = lib.std_dense_verify_attn_dlen(qvc, kc, vc, cap, seq, 0)
        out_s = lib.std_sparse_decode_attn_dlen(q1c, kc, vc, cap, seq, 1, 0, vis_len, idxc)
        out_0 = lib.std_sparse_decode_attn_dlen(q1c, kc, vc, cap, seq, 1, 0, vis_len,
                                                idxc[:, :0].contiguous())
        torch.cuda.synchronize()
        say(f"{dtype} device length {dev_len}")
        for o in (outv, out_s, out_0):
            assert torch.isfinite(o.float()).all()
        assert max_abs(f64(outv), oracle.dense_verify(f64(qv), kf, vf, n_q)) <= tol
        ref_s = oracle.sparse_decode(f64(q1), kf, vf, vis_len, 0, vis_len, idx.numpy())
        assert max_abs(f64(out_s), ref_s) <= tol
        ref_0 = oracle.sparse_decode(f64(q1), kf, vf, vis_len + 1, 0, vis_len,
                                     np.zeros((hkv, 0), np.int64))
        assert max_abs(f64(out_0), ref_0) <= tol
