"""End-to-end example: a small decoder whose attention runs on the four calls.

The decoder is a standard pre-norm transformer (RMSNorm, rotary position
embedding with the rotate-half pairing, grouped-query attention, SwiGLU MLP,
untied LM head) with caller-supplied weights.  Every attention of the model
goes through the library:

* prefill        -- std_dense_verify_attn over the prompt in query chunks
                    (bottom-right causal alignment makes a chunk of n_q rows
                    ending at position p the causal rows of the prompt);
* selection      -- std_select_topk per layer on the prefill's rotated text
                    queries (technical summary, Methodology item 4), or the
                    streaming comparator's fixed lists (std_static_window_idx:
                    an attention sink plus a recent window of the visual span);
* draft step     -- std_sparse_decode_attn, one token at a time, over the
                    selected visual KV plus all other KV (Methodology item 2);
* verify         -- std_dense_verify_attn with the gamma+1 queries
                    (x_t, d_1..d_gamma) in one pass (Methodology items 2-3);
* acceptance     -- std_accept, greedy longest prefix plus the bonus token
                    (Methodology item 3); with an empty draft the same call
                    is the greedy argmax of one row.

Everything around attention (embeddings, norms, rotary embedding,
projections, MLP, LM head) is plain torch on the GPU: it is the model the
hot path sits in, not part of the path.  Drafted tokens write their K/V at
their own positions of the one shared cache; the verify pass rewrites
positions t..t+gamma and acceptance sets the valid length to t+n+1, so
rejected positions are overwritten later (Methodology item 3: accepted
tokens are appended to the context).
"""

import torch

from . import _lib


class ToyDecoder:
    """A decoder on one GPU with a KV cache of ``capacity`` positions.

    ``params`` holds the weights as float64 arrays: ``embed [vocab][hidden]``,
    per layer ``attn_norm, wq, wk, wv, wo, mlp_norm, w_gate, w_up, w_down``
    (matrices as [in][out]), ``final_norm`` and ``lm_head [hidden][vocab]``,
    plus ``cfg`` with n_q_heads, n_kv_heads, head_dim, eps and rope_theta.
    ``dtype`` is the cache and attention type (bf16 or fp32) and, unless
    ``matmul_dtype`` says otherwise, the projections' type; norms, the
    residual stream and the logits stay in fp32.  fp32 projections beside a
    bf16 cache keep the model's rows independent of how many rows a forward
    takes (a torch GEMM over 1 row and over gamma+1 rows may round
    differently), so a bf16-attention draft-verify loop can be compared
    token for token with bf16-attention greedy decoding.
    """

    def __init__(self, params, capacity, device="cuda", dtype=torch.bfloat16,
                 prefill_chunk=512, matmul_dtype=None):
        cfg = params["cfg"]
        self.cfg = cfg
        self.hq, self.hkv, self.d = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
        self.eps = float(cfg["eps"])
        self.dt = dtype
        self.mt = dtype if matmul_dtype is None else matmul_dtype
        self.dev = torch.device(device)
        self.capacity = int(capacity)
        self.chunk = int(prefill_chunk)

        def mat(a):
            return torch.as_tensor(a, dtype=self.mt, device=self.dev).contiguous()

        def vec(a):
            return torch.as_tensor(a, dtype=torch.float32, device=self.dev).contiguous()

        self.embed = vec(params["embed"])
        self.layers = []
        for lp in params["layers"]:
            self.layers.append({
                "attn_norm": vec(lp["attn_norm"]), "mlp_norm": vec(lp["mlp_norm"]),
                "wq": mat(lp["wq"]), "wk": mat(lp["wk"]), "wv": mat(lp["wv"]),
                "wo": mat(lp["wo"]), "w_gate": mat(lp["w_gate"]), "w_up": mat(lp["w_up"]),
                "w_down": mat(lp["w_down"])})
        self.final_norm = vec(params["final_norm"])
        self.lm_head = vec(params["lm_head"])
        self.vocab = self.lm_head.shape[1]

        n = len(self.layers)
        self.k = [torch.zeros(self.hkv, self.capacity, self.d, dtype=dtype, device=self.dev)
                  for _ in range(n)]
        self.v = [torch.zeros_like(self.k[0]) for _ in range(n)]

        half = self.d // 2
        inv = float(cfg["rope_theta"]) ** (-torch.arange(half, dtype=torch.float64) * 2.0 / self.d)
        ang = torch.arange(self.capacity, dtype=torch.float64)[:, None] * inv[None, :]
        self.cos = torch.cos(ang).to(torch.float32).to(self.dev)
        self.sin = torch.sin(ang).to(torch.float32).to(self.dev)

        self.shape = _lib.attn_shape(self.hq, self.hkv, self.d)
        self.ws_dense = self._ws(_lib.std_dense_verify_workspace(
            self.shape, self.chunk, self.k[0], self.capacity))
        self._ws_sparse = None
        self.out_tok = torch.empty(1, dtype=torch.int32, device=self.dev)
        self.n_one = torch.empty(1, dtype=torch.int32, device=self.dev)
        self.no_draft = torch.empty(0, dtype=torch.int32, device=self.dev)

    # ------------------------------------------------------------------ model
    def _ws(self, nbytes):
        return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=self.dev)

    def _rms(self, x, w):
        return x * torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + self.eps) * w

    def _rope(self, x, pos0, n):
        half = self.d // 2
        cos = self.cos[pos0:pos0 + n, None, :]
        sin = self.sin[pos0:pos0 + n, None, :]
        x1, x2 = x[..., :half], x[..., half:]
        return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], dim=-1)

    def _dense_attn(self, q, li, length):
        """Causal attention of the n_q rows ending at position length-1."""
        n = q.shape[0]
        out = torch.empty_like(q)
        for c0 in range(0, n, self.chunk):
            c1 = min(n, c0 + self.chunk)
            _lib.std_dense_verify_attn(q[c0:c1], self.k[li], self.v[li], length - n + c1,
                                       out=out[c0:c1], workspace=self.ws_dense)
        return out

    def forward(self, x, pos0, sparse=None, want_q_text=None):
        """Run the layers on x [T][hidden] (fp32) at positions pos0..pos0+T-1.

        Writes every layer's K/V at those positions and returns fp32 logits
        [T][vocab].  ``sparse`` = (idx per layer, vis_start, vis_len) selects
        the draft model (T must be 1).  ``want_q_text`` = (r0, r1) also
        returns each layer's rotated queries of rows r0..r1-1 as
        [H_q][r1-r0][d].
        """
        T = x.shape[0]
        length = pos0 + T
        hq, hkv, d = self.hq, self.hkv, self.d
        q_text = []
        for li, lp in enumerate(self.layers):
            h = self._rms(x, lp["attn_norm"]).to(self.mt)
            q = (h @ lp["wq"]).float().view(T, hq, d)
            k = (h @ lp["wk"]).float().view(T, hkv, d)
            v = (h @ lp["wv"]).to(self.dt).view(T, hkv, d)
            q = self._rope(q, pos0, T).to(self.dt).contiguous()
            k = self._rope(k, pos0, T).to(self.dt)
            self.k[li][:, pos0:length] = k.transpose(0, 1)
            self.v[li][:, pos0:length] = v.transpose(0, 1)
            if want_q_text is not None:
                r0, r1 = want_q_text
                q_text.append(q[r0:r1].transpose(0, 1).contiguous())
            if sparse is None:
                o = self._dense_attn(q, li, length)
            else:
                if T != 1:
                    raise ValueError("the draft model runs one token at a time")
                idx, vis_start, vis_len = sparse
                o = _lib.std_sparse_decode_attn(q[0], self.k[li], self.v[li], length, vis_start,
                                                vis_len, idx[li], workspace=self._sparse_ws(
                                                    idx[li].shape[1], vis_start, vis_len))[None]
            x = x + (o.reshape(T, hq * d).to(self.mt) @ lp["wo"]).float()
            h = self._rms(x, lp["mlp_norm"]).to(self.mt)
            g = torch.nn.functional.silu(h @ lp["w_gate"])
            x = x + ((g * (h @ lp["w_up"])) @ lp["w_down"]).float()
        logits = self._rms(x, self.final_norm) @ self.lm_head
        return (logits, q_text) if want_q_text is not None else logits

    def _sparse_ws(self, topk, vis_start, vis_len):
        key = (topk, vis_start, vis_len)
        if self._ws_sparse is None or self._ws_sparse[0] != key:
            nbytes = _lib.std_sparse_decode_workspace(self.shape, self.k[0], self.capacity,
                                                      vis_start, vis_len, topk)
            self._ws_sparse = (key, self._ws(nbytes))
        return self._ws_sparse[1]

    def argmax(self, logits_row, margins=None):
        """Greedy token of one fp32 logits row [1][vocab], on the device."""
        _lib.std_accept(self.no_draft, logits_row, out_tokens=self.out_tok, n_out=self.n_one,
                        margins=margins)
        return self.out_tok.clone()

    # --------------------------------------------------------------- decoding
    def prefill(self, vis_emb, text_ids, margin=None):
        """Prompt = visual embeddings [n_vis][hidden] then text ids.

        Returns (first token on the device, per-layer text queries);
        ``margin`` [1] fp32 receives top1 - top2 of the last prompt row.
        """
        vis = torch.as_tensor(vis_emb, dtype=torch.float32, device=self.dev)
        ids = torch.as_tensor(text_ids, dtype=torch.long, device=self.dev)
        x = torch.cat([vis, self.embed[ids]], dim=0)
        n_vis, n = vis.shape[0], x.shape[0]
        if n + 1 > self.capacity:
            raise ValueError("prompt does not fit the cache")
        logits, q_text = self.forward(x, 0, want_q_text=(n_vis, n))
        return self.argmax(logits[-1:].contiguous(), margin), q_text

    def select(self, q_text, prompt_len, vis_start, vis_len, topk):
        """Top-K visual positions per layer and KV head (fixed for decoding)."""
        n_text = q_text[0].shape[1]
        ws = self._ws(_lib.std_select_topk_workspace(self.shape, n_text, vis_start, vis_len,
                                                     topk, self.k[0], prompt_len))
        return [_lib.std_select_topk(q_text[li], self.k[li], prompt_len, prompt_len - n_text,
                                     vis_start, vis_len, topk, workspace=ws)
                for li in range(len(self.layers))]

    def select_static(self, vis_start, vis_len, sink, topk):
        """The streaming comparator's visual positions, the same for every
        layer: the first min(sink, topk) and the last topk - min(sink, topk)
        of the span (std_static_window_idx)."""
        idx = _lib.std_static_window_idx(self.hkv, vis_start, vis_len, sink, topk,
                                         device=self.dev)
        return [idx for _ in self.layers]

    def snapshot(self):
        return [t.clone() for t in self.k + self.v]

    def restore(self, snap):
        n = len(self.layers)
        for i in range(n):
            self.k[i].copy_(snap[i])
            self.v[i].copy_(snap[n + i])

    def decode_dense(self, first_tok, pos, n_new, margins=None):
        """Plain greedy decoding: n_new tokens starting with ``first_tok``
        (pending at position ``pos``).  One token per forward, no host sync
        inside the loop.  ``margins`` [n_new] fp32 receives top1 - top2 of
        every step's logits (entry 0 untouched)."""
        toks = [first_tok.view(1)]
        tok = first_tok.view(1)
        for i in range(1, n_new):
            logits = self.forward(self.embed[tok.long()], pos + i - 1)
            m = None if margins is None else margins[i:i + 1]
            tok = self.argmax(logits, m)
            toks.append(tok)
        return torch.cat(toks).tolist()

    def decode_std(self, first_tok, pos, n_new, idx, vis_start, vis_len, gamma):
        """Sparse-to-Dense decoding; returns (tokens, accepted n per cycle)."""
        out = [int(first_tok.item())]
        x_t = first_tok.view(1)
        t = pos
        accepted = []
        draft = torch.empty(gamma, dtype=torch.int32, device=self.dev)
        out_tokens = torch.empty(gamma + 1, dtype=torch.int32, device=self.dev)
        n_out = torch.empty(1, dtype=torch.int32, device=self.dev)
        sparse = (idx, vis_start, vis_len)
        nvtx = torch.cuda.nvtx                           # roctx ranges for a marker trace
        while len(out) < n_new:
            if t + gamma + 1 > self.capacity:
                raise ValueError("decoding ran past the cache capacity")
            tok = x_t
            nvtx.range_push("draft")
            for j in range(gamma):                      # sparse model drafts
                logits = self.forward(self.embed[tok.long()], t + j, sparse=sparse)
                tok = self.argmax(logits)
                draft[j:j + 1] = tok
            nvtx.range_pop()
            nvtx.range_push("verify")
            seq = torch.cat([x_t, draft])               # dense model verifies
            logits = self.forward(self.embed[seq.long()], t)
            nvtx.range_pop()
            nvtx.range_push("accept")
            _lib.std_accept(draft, logits, out_tokens=out_tokens, n_out=n_out)
            nvtx.range_pop()
            n = int(n_out.item())
            emitted = out_tokens[:n].tolist()
            accepted.append(n - 1)
            out.extend(emitted)
            x_t = out_tokens[n - 1:n].clone()           # the bonus is pending
            t += n
        return out[:n_new], accepted

