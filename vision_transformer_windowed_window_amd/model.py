"""FlashSwin-T forward pass on the GPU, composed from libwattn's C entry points.

FLASHSWIN: Unlocking Large Windows and Dense Tokens in Swin Vision Transformers with Memory
Efficient Attention -- "How it works": Swin's hierarchy with the fused window attention,
window-local 2D RoPE and the overlapping stem.  Every step runs in the library's kernels
(wattn_stem_conv, wattn_layernorm, wattn_swin_block, wattn_patch_merge_norm, wattn_linear,
wattn_token_mean); this module only uploads the parameters, allocates activations and calls
them in order on one stream.

Parameters come as a dict of arrays laid out as the library expects: stem_w [C][3][k][k],
stem_b, stem_ln_g, stem_ln_b; stages: list of dict(heads, blocks=[block dicts with the
wattn_block_params_t names], theta [H][16], merge=None or dict(ln_g, ln_b, w [2C][4C]));
norm_g, norm_b, head_w [classes][C], head_b.  Matrices are stored in bfloat16, norms, biases
and RoPE tables in float32.
"""

from __future__ import annotations

from . import (ACT_NONE, layernorm, linear, patch_merge_norm, stem_conv, swin_block, swin_block_workspace,
               token_mean)

_MATRICES = ("w_qkv", "w_proj", "w_fc1", "w_fc2")


def stage_window(grid: int, M: int, shift: int):
    """A stage whose grid side is not above M uses one window over the grid and no shift."""
    return (grid, 0) if grid <= M else (M, shift)


class FlashSwinT:
    def __init__(self, params: dict, *, p: int, M: int, device="cuda:0"):
        import torch

        self.p, self.M = p, M
        bf, f32 = torch.bfloat16, torch.float32
        dev = torch.device(device)

        def up(a, dt):
            return None if a is None else torch.as_tensor(a).to(dt).to(dev).contiguous()

        self.stem_w, self.stem_b = up(params["stem_w"], bf), up(params["stem_b"], f32)
        self.stem_ln = (up(params["stem_ln_g"], f32), up(params["stem_ln_b"], f32))
        self.stages = []
        for st in params["stages"]:
            blocks = []
            for blk in st["blocks"]:
                blocks.append({name: up(a, bf if name in _MATRICES else f32) for name, a in blk.items()})
            merge = None
            if st.get("merge") is not None:
                m = st["merge"]
                merge = (up(m["ln_g"], f32), up(m["ln_b"], f32), up(m["w"], bf))
            self.stages.append(dict(heads=st["heads"], blocks=blocks, theta=up(st.get("theta"), f32), merge=merge))
        self.norm = (up(params["norm_g"], f32), up(params["norm_b"], f32))
        self.head_w, self.head_b = up(params["head_w"], bf), up(params["head_b"], f32)
        self._ws = {}

    def _workspace(self, B, Hg, Wg, C, device):
        import torch

        key = (B, Hg, Wg, C)
        if key not in self._ws:
            self._ws[key] = torch.empty(swin_block_workspace(B, Hg, Wg, C), dtype=torch.uint8, device=device)
        return self._ws[key]

    def forward(self, img):
        """Class logits (float32 [B, classes]) of NHWC bfloat16 images [B, side, side, 3]."""
        import torch

        x = stem_conv(img, self.stem_w, self.stem_b, p=self.p)
        x = layernorm(x, *self.stem_ln)
        for st in self.stages:
            B, Hg, Wg, C = x.shape
            ws = self._workspace(B, Hg, Wg, C, x.device)
            for i, blk in enumerate(st["blocks"]):
                Mw, s = stage_window(Hg, self.M, 0 if i % 2 == 0 else self.M // 2)
                swin_block(x, dict(blk, theta=st["theta"]), H=st["heads"], M=Mw, shift=s, workspace=ws)
            if st["merge"] is not None:
                g, b, w = st["merge"]
                x = linear(patch_merge_norm(x, g, b), w, None, act=ACT_NONE)
        x = layernorm(x, *self.norm)
        return linear(token_mean(x), self.head_w, self.head_b, out_dtype=torch.float32)

    __call__ = forward
