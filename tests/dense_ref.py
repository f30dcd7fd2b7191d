"""Independent dense formulations used to pin the oracle (test code only).

Both work on one sequence's contiguous rows, with the mask written out as a
boolean matrix: query token i of an n-token step over L keys sits at position
L - n + i and sees keys a..L-n+i.  One uses numpy matrix products, the other
torch's CPU scaled_dot_product_attention in float64 with an explicit mask.
"""
import numpy as np
import torch


def visible_mask(L: int, n: int, a: int = 0) -> np.ndarray:
    j = np.arange(L)[None, :]
    p = (L - n + np.arange(n))[:, None]
    return (j <= p) & (j >= a)


def dense_numpy(q, k, v, scale, G, a=0):
    """q [n, Hq, D], k/v [L, Hkv, D] (float64 numpy) -> [n, Hq, D]."""
    n, hq, d = q.shape
    L = k.shape[0]
    ke = np.repeat(k, G, axis=1)  # kv head of q head h is h // G
    ve = np.repeat(v, G, axis=1)
    s = np.einsum("nhd,lhd->hnl", q, ke) * scale
    m = visible_mask(L, n, a)[None]
    s = np.where(m, s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    w = np.exp(s)
    w = w / w.sum(axis=-1, keepdims=True)
    return np.einsum("hnl,lhd->nhd", w, ve)


def dense_torch_sdpa(q, k, v, scale, G, a=0):
    qt = torch.from_numpy(q).permute(1, 0, 2)  # [Hq, n, D]
    kt = torch.from_numpy(np.repeat(k, G, axis=1)).permute(1, 0, 2).contiguous()
    vt = torch.from_numpy(np.repeat(v, G, axis=1)).permute(1, 0, 2).contiguous()
    mask = torch.from_numpy(visible_mask(k.shape[0], q.shape[0], a))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                         scale=float(scale))
    return o.permute(1, 0, 2).numpy()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()
