"""An independent torch formulation (float64, CPU) of the shifted-window layer, used as an
autograd reference by the oracle pins: roll, partition into windows, explicit RoPE, bias
matrix, region-label mask tensor, softmax, reverse."""

import math

import torch


def _windows(t, M):
    B, Hg, Wg, H, d = t.shape
    t = t.reshape(B, Hg // M, M, Wg // M, M, H, d).permute(0, 1, 3, 5, 2, 4, 6)
    return t.reshape(B, Hg // M, Wg // M, H, M * M, d)


def _unwindows(t, Hg, Wg, M):
    B, nWy, nWx, H, N, d = t.shape
    t = t.reshape(B, nWy, nWx, H, M, M, d).permute(0, 1, 4, 2, 5, 3, 6)
    return t.reshape(B, Hg, Wg, H, d)


def torch_layer(q, k, v, th, U, V, M, s):
    """Shifted window attention written with whole-tensor torch ops (float64)."""
    B, Hg, Wg, H, d = q.shape
    roll = lambda a: torch.roll(a, shifts=(-s, -s), dims=(1, 2))
    tq, tk, tv = (_windows(roll(a), M) for a in (q, k, v))
    n = torch.arange(M * M, dtype=torch.float64)
    rr, cc = torch.div(n, M, rounding_mode="floor"), n % M
    d4 = d // 4
    pos = torch.cat([rr[:, None].expand(M * M, d4), cc[:, None].expand(M * M, d4)], dim=1)  # [N, d/2]
    ang = pos[None] * th[:, None, :]                                                        # [H, N, d/2]
    cs, sn = torch.cos(ang), torch.sin(ang)

    def rot(t):
        a, b = t[..., 0::2], t[..., 1::2]
        return torch.stack([a * cs - b * sn, a * sn + b * cs], dim=-1).reshape(t.shape)

    logits = rot(tq) @ rot(tk).transpose(-1, -2) / math.sqrt(d) + (U @ V.transpose(-1, -2))
    lab = torch.zeros(Hg, Wg)
    cnt = 0
    sl = (lambda G: (slice(0, G - M), slice(G - M, G - s), slice(G - s, G))) if s else (lambda G: (slice(0, G),))
    for hs in sl(Hg):
        for ws in sl(Wg):
            lab[hs, ws] = cnt
            cnt += 1
    lw = lab.reshape(Hg // M, M, Wg // M, M).permute(0, 2, 1, 3).reshape(Hg // M, Wg // M, M * M)
    mask = torch.where(lw[..., :, None] == lw[..., None, :], 0.0, float("-inf")).double()
    logits = logits + mask[None, :, :, None]
    lse = torch.logsumexp(logits, dim=-1)
    o = torch.softmax(logits, dim=-1) @ tv
    out = torch.roll(_unwindows(o, Hg, Wg, M), shifts=(s, s), dims=(1, 2))
    lse_grid = torch.roll(_unwindows(lse[..., None], Hg, Wg, M)[..., 0], shifts=(s, s), dims=(1, 2))
    return out, lse_grid
