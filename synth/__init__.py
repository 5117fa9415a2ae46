"""Seeded synthetic inputs for the StD hot path (shared by tests, bench, smoke).

This module only draws random inputs; it holds none of the method's
arithmetic.  Both the HIP path and the float64 oracle receive the tensors it
returns (the oracle reads back exactly the values the GPU received).

Workloads (the pages evaluate Qwen2-VL-7B-Instruct and LLaVA-OneVision-7B on
MLVU and VideoMME; neither weights nor datasets are available, so these
seeded tensors with the same head layout and context lengths stand in):

  c1  tiny, fp32: 4 query heads / 1 KV head / d 64; 1,024 visual + 64 text;
      64 planted salient visual keys (+3u); text and decode queries +2u;
      K=128, gamma=4.
  c2  Qwen2-VL-7B-shaped single layer, bf16: 28/4/128; 16,384 visual + 512
      text; 5% planted keys per KV head (+3u_h); K=1,024, gamma=5.
  c3  28 layers, bf16: 32,768 visual + 1,024 text; planted fraction per
      layer drawn from U[2%, 10%]; K=2,048, gamma=5.
  c4  28 layers, bf16 (~8 GB of KV): 140,000 visual + 2,048 text; planted
      keys in 64-token runs at random non-overlapping offsets covering 3% of
      the visual span; K=4,096, gamma=6.
  c5  toy decoder (4 layers, hidden 512, 8/2/64, MLP 1,536, vocab 8,192):
      8,192 visual embeddings (5% get +3u) + 128 uniform text ids; K=512.

Every K/V/Q entry is N(0,1) before planting.  The gamma+1 positions after
the context (the pending token and the drafts) get N(0,1) keys and values
like text; queries of group h (draft, verify and text) get +2*u_h.
"""

from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class AttnConfig:
    name: str
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    vis_len: int
    n_text: int
    topk: int
    gamma: int
    dtype: str                 # "f32" or "bf16"
    planted: tuple             # ("count", n) | ("frac", f) | ("frac_u", lo, hi) | ("runs", run, f)
    seed: int = 0
    prefix: int = 0            # non-visual positions before the visual span
    extra: int = 0             # further cache positions after ctx+gamma+1 (decode growth)

    @property
    def vis_start(self):
        return self.prefix

    @property
    def vis_end(self):
        return self.prefix + self.vis_len

    @property
    def text_start(self):
        return self.vis_end

    @property
    def ctx(self):
        return self.prefix + self.vis_len + self.n_text

    @property
    def capacity(self):
        return self.ctx + self.gamma + 1 + self.extra

    @property
    def verify_len(self):
        return self.ctx + self.gamma + 1

    def draft_len(self, j):
        """Valid length during draft step j (0-based): ctx + 1 + j."""
        return self.ctx + 1 + j

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


CONFIGS = {
    "c1": AttnConfig("c1", 1, 4, 1, 64, 1024, 64, 128, 4, "f32", ("count", 64)),
    "c2": AttnConfig("c2", 1, 28, 4, 128, 16384, 512, 1024, 5, "bf16", ("frac", 0.05)),
    "c3": AttnConfig("c3", 28, 28, 4, 128, 32768, 1024, 2048, 5, "bf16", ("frac_u", 0.02, 0.10)),
    "c4": AttnConfig("c4", 28, 28, 4, 128, 140000, 2048, 4096, 6, "bf16", ("runs", 64, 0.03)),
}


def config(name, **overrides):
    return replace(CONFIGS[name], **overrides) if overrides else CONFIGS[name]


def _seed(*parts):
    s = np.random.SeedSequence([int(p) & 0xFFFFFFFF for p in parts])
    return int(s.generate_state(1, dtype=np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)


def _gen(device, *parts):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def _planted_mask(cfg, layer, device):
    """Bool [H_kv][vis_len]: which visual keys get the salient direction."""
    g = _gen("cpu", cfg.seed, layer, 17)
    kind = cfg.planted[0]
    mask = torch.zeros(cfg.n_kv_heads, cfg.vis_len, dtype=torch.bool)
    if kind in ("count", "frac", "frac_u"):
        if kind == "count":
            n = cfg.planted[1]
        elif kind == "frac":
            n = int(round(cfg.planted[1] * cfg.vis_len))
        else:
            lo, hi = cfg.planted[1], cfg.planted[2]
            f = lo + (hi - lo) * torch.rand(1, generator=g).item()
            n = int(round(f * cfg.vis_len))
        for h in range(cfg.n_kv_heads):
            mask[h, torch.randperm(cfg.vis_len, generator=g)[:n]] = True
    elif kind == "runs":
        run, frac = cfg.planted[1], cfg.planted[2]
        n_runs = int(round(frac * cfg.vis_len / run))
        free = cfg.vis_len - n_runs * run
        for h in range(cfg.n_kv_heads):
            # sorted draws from [0, free] spaced by the run length give
            # uniformly placed, non-overlapping runs
            cuts = torch.sort(torch.randint(0, free + 1, (n_runs,), generator=g)).values
            for r in range(n_runs):
                s = int(cuts[r]) + r * run
                mask[h, s:s + run] = True
    else:
        raise ValueError(kind)
    return mask.to(device)


def attention_layer(cfg, layer=0, device="cpu"):
    """All inputs of one layer of an attention config, in the config dtype.

    Returns a dict with
      k, v       [H_kv][capacity][d]   KV cache (positions >= ctx hold the
                                       pending token and the gamma drafts)
      q_text     [H_q][n_text][d]      prefill text queries (text row i sits
                                       at position text_start + i)
      q_draft    [gamma][H_q][d]       query of draft step j (position ctx+j)
      q_verify   [gamma+1][H_q][d]     verify queries (positions ctx..ctx+gamma)
      u          [H_kv][d]             planted unit directions (fp32)
      planted    [H_kv][vis_len] bool  planted visual keys
    """
    hq, hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    g = _gen(device, cfg.seed, layer, 1)
    u = torch.randn(hkv, d, generator=g, device=device)
    u = u / u.norm(dim=1, keepdim=True)
    planted = _planted_mask(cfg, layer, device)
    k = torch.randn(hkv, cfg.capacity, d, generator=g, device=device)
    v = torch.randn(hkv, cfg.capacity, d, generator=g, device=device)
    kv_vis = k[:, cfg.vis_start:cfg.vis_end]
    kv_vis += 3.0 * planted.unsqueeze(-1).float() * u.unsqueeze(1)
    grp = torch.arange(hq, device=device) // (hq // hkv)
    uq = u[grp]                                    # direction of each query head
    q_text = torch.randn(hq, cfg.n_text, d, generator=g, device=device) + 2.0 * uq.unsqueeze(1)
    q_draft = torch.randn(cfg.gamma, hq, d, generator=g, device=device) + 2.0 * uq.unsqueeze(0)
    q_verify = torch.randn(cfg.gamma + 1, hq, d, generator=g, device=device) + 2.0 * uq.unsqueeze(0)
    dt = cfg.torch_dtype
    return {
        "k": k.to(dt).contiguous(), "v": v.to(dt).contiguous(),
        "q_text": q_text.to(dt).contiguous(),
        "q_draft": q_draft.to(dt).contiguous(),
        "q_verify": q_verify.to(dt).contiguous(),
        "u": u, "planted": planted,
    }


def accept_case(gamma, vocab, agree_prob, seed, dtype=torch.float32, n_ties=0):
    """Draft tokens and gamma+1 logit rows for the acceptance step.

    Logits are N(0,1); at each position the draft either equals the row's
    planted winner (probability ``agree_prob``) or is a different token.
    ``n_ties`` rows get an exact two-way tie at the top (same value at two
    token ids).  Returns (draft int32 [gamma], logits [gamma+1][vocab]).
    """
    g = _gen("cpu", seed, gamma, vocab, 23)
    logits = torch.randn(gamma + 1, vocab, generator=g)
    win = torch.randint(0, vocab, (gamma + 1,), generator=g)
    for i in range(gamma + 1):
        logits[i, win[i]] = 6.0 + torch.rand(1, generator=g).item()
    for i in range(min(n_ties, gamma + 1)):
        other = (int(win[i]) + 1 + int(torch.randint(0, vocab - 1, (1,), generator=g))) % vocab
        logits[i, other] = logits[i, win[i]]
    agree = torch.rand(gamma, generator=g) < agree_prob
    draft = torch.empty(gamma, dtype=torch.int32)
    for j in range(gamma):
        if agree[j]:
            draft[j] = int(win[j])
        else:
            draft[j] = (int(win[j]) + 1 + int(torch.randint(0, vocab - 1, (1,), generator=g))) % vocab
    return draft, logits.to(dtype)


# ----------------------------------------------------------------------------
# toy decoder (c5) inputs: random-init weights and a synthetic prompt

TOY_C5 = dict(n_layers=4, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=64,
              mlp=1536, vocab=8192, eps=1e-6, rope_theta=1e4,
              n_vis=8192, n_text=128, salient_frac=0.05, topk=512)

# a small decoder the GPU kernels take (head_dim 64) and the float64
# oracle still runs in seconds
TOY_GPU = dict(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
               mlp=512, vocab=512, eps=1e-6, rope_theta=1e4,
               n_vis=1024, n_text=32, salient_frac=0.05, topk=64)

TOY_TINY = dict(n_layers=2, hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16,
                mlp=128, vocab=256, eps=1e-6, rope_theta=1e4,
                n_vis=256, n_text=16, salient_frac=0.05, topk=32)


def toy_params(cfg, seed=0, std=0.02):
    """Random-init weights, N(0, std^2), RMSNorm weights 1; float64 numpy."""
    rng = np.random.Generator(np.random.PCG64(_seed(seed, 5)))
    hd, hq, hkv, d = cfg["hidden"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    f, vocab = cfg["mlp"], cfg["vocab"]

    def w(*shape):
        return rng.standard_normal(shape) * std

    layers = []
    for _ in range(cfg["n_layers"]):
        layers.append(dict(
            attn_norm=np.ones(hd), wq=w(hd, hq * d), wk=w(hd, hkv * d),
            wv=w(hd, hkv * d), wo=w(hq * d, hd), mlp_norm=np.ones(hd),
            w_gate=w(hd, f), w_up=w(hd, f), w_down=w(f, hd)))
    return dict(cfg=dict(cfg), embed=rng.standard_normal((vocab, hd)),
                layers=layers, final_norm=np.ones(hd), lm_head=w(hd, vocab))


def toy_prompt(cfg, seed=0):
    """(visual embeddings [n_vis][hidden] float64, text ids [n_text] int64)."""
    rng = np.random.Generator(np.random.PCG64(_seed(seed, 9)))
    n_vis, hd = cfg["n_vis"], cfg["hidden"]
    vis = rng.standard_normal((n_vis, hd))
    u = rng.standard_normal(hd)
    u /= np.linalg.norm(u)
    sal = rng.choice(n_vis, size=int(round(cfg["salient_frac"] * n_vis)), replace=False)
    vis[sal] += 3.0 * u
    text = rng.integers(0, cfg["vocab"], size=cfg["n_text"])
    return vis, text
