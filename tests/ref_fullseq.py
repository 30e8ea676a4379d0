"""An independent full-sequence reference decoder in numpy (float64).

Used only to pin the oracle.  It is written in a different form from the
oracle: the whole prompt is processed at once with matrix products and a causal
mask, K/V heads are expanded to the query heads with `repeat`, RoPE uses complex
exponentials and the softmax is scipy's.  Weight decoding uses numpy bit views.
The incremental, cached decode of the oracle must agree with it at every
position (K and V are rounded to bf16 before attention, since the decode step
reads them back from a bf16 cache).
"""
import numpy as np
import scipy.special
import torch


def bf16_to_f64(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_to_f64(a: np.ndarray) -> np.ndarray:
    return a.view(np.float16).astype(np.float64)


def round_bf16_f64(a: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.asarray(a, dtype=np.float64)).to(torch.float32).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


def dequant(lin) -> np.ndarray:
    if lin.s is None:
        return bf16_to_f64(lin.w)
    lo = (lin.w & 0x0F).astype(np.int64)
    hi = (lin.w >> 4).astype(np.int64)
    codes = np.empty((lin.rows, lin.cols), dtype=np.int64)
    codes[:, 0::2] = lo
    codes[:, 1::2] = hi
    scales = np.repeat(f16_to_f64(lin.s), 64, axis=1)
    return scales * (codes - 8).astype(np.float64)


def rmsnorm(x, g, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def rope(x, positions, theta):
    # x: [T, heads, d]; half-split pairs (i, i + d/2) as one complex number
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = np.outer(positions, inv)  # [T, half]
    rot = np.exp(1j * ang)[:, None, :]
    z = (x[..., :half] + 1j * x[..., half:]) * rot
    return np.concatenate([z.real, z.imag], axis=-1)


def forward(model, tokens):
    """Logits [T, V] for every prefix of `tokens`, plus the bf16-rounded K and V
    ([L][T][n_kv][d]) the decode step would have cached."""
    cfg = model.cfg
    T = len(tokens)
    H, d, nq, nkv = cfg.hidden, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    x = bf16_to_f64(model.embed[np.asarray(tokens)])
    pos = np.arange(T, dtype=np.float64)
    mask = np.triu(np.full((T, T), -np.inf), k=1)
    ks, vs = [], []
    for L in model.layers:
        h = rmsnorm(x, bf16_to_f64(L.attn_norm), cfg.rms_eps)
        y = h @ dequant(L.qkv).T
        if L.qkv_bias is not None:
            y = y + bf16_to_f64(L.qkv_bias)
        q = y[:, :nq * d].reshape(T, nq, d)
        k = y[:, nq * d:(nq + nkv) * d].reshape(T, nkv, d)
        v = y[:, (nq + nkv) * d:].reshape(T, nkv, d)
        q = rope(q, pos, cfg.rope_theta)
        k = round_bf16_f64(rope(k, pos, cfg.rope_theta))
        v = round_bf16_f64(v)
        ks.append(k)
        vs.append(v)
        group = nq // nkv
        kk = np.repeat(k, group, axis=1)  # [T, nq, d]
        vv = np.repeat(v, group, axis=1)
        s = np.einsum("thd,shd->hts", q, kk) / np.sqrt(d) + mask[None]
        p = scipy.special.softmax(s, axis=-1)
        o = np.einsum("hts,shd->thd", p, vv).reshape(T, nq * d)
        x = x + o @ dequant(L.o).T
        h = rmsnorm(x, bf16_to_f64(L.mlp_norm), cfg.rms_eps)
        I = cfg.intermediate
        if not cfg.n_experts:
            gu = h @ dequant(L.gate_up).T
            a = gu[:, :I] * scipy.special.expit(gu[:, :I]) * gu[:, I:]
            x = x + a @ dequant(L.down).T
        else:
            x = x + moe(cfg, L, h)
    h = rmsnorm(x, bf16_to_f64(model.final_norm), cfg.rms_eps)
    logits = h @ bf16_to_f64(model.head).T
    return logits, ks, vs


def moe(cfg, L, h):
    """Mixture-of-experts MLP of every row of h at once: the router's softmax
    over all experts (torch), the top_k experts by torch.topk on the fp32-rounded
    logits (the precision the decision is made in), every expert's SiLU-gated MLP
    evaluated for all rows as one batched product, and the chosen ones gathered
    and combined with their probabilities."""
    E, k, I, H = cfg.n_experts, cfg.top_k, cfg.intermediate, cfg.hidden
    z = torch.from_numpy(h @ bf16_to_f64(L.router).T)                  # [T, E]
    prob = torch.softmax(z, dim=-1)
    _, ids = torch.topk(z.to(torch.float32), k, dim=-1, sorted=True)   # [T, k]
    wgu = torch.from_numpy(dequant(L.gate_up)).reshape(E, 2 * I, H)
    wd = torch.from_numpy(dequant(L.down)).reshape(E, H, I)
    ht = torch.from_numpy(h)
    gu = torch.einsum("eoh,th->teo", wgu, ht)                           # [T, E, 2I]
    a = torch.nn.functional.silu(gu[..., :I]) * gu[..., I:]
    y = torch.einsum("ehi,tei->teh", wd, a)                             # [T, E, H]
    ysel = torch.gather(y, 1, ids[..., None].expand(-1, -1, H))         # [T, k, H]
    psel = torch.gather(prob, 1, ids)                                   # [T, k]
    return (psel[..., None] * ysel).sum(dim=1).numpy()
