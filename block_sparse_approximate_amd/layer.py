"""PyTorch modules around the MRA-2 kernels: an autograd function over the C
ABI's forward and backward calls, the self-attention module, and one
BERT-style encoder layer.

[MRA] architecture overview: MRA keeps BERT's encoder-only skeleton (feed-
forward block, residual connections and LayerNorm as in BERT); only the
self-attention module differs.  [MRA] "源码级原理", engineering notes: the
sequence length must be a multiple of the 32-token block, so inputs are
padded; here the padding tokens are masked out (mask 0), so they neither
attend nor are attended to, and are cut off again on return.

Every attention step runs in the HIP kernels (libmra.so); the projections,
LayerNorm and feed-forward block are ordinary torch layers.  There is no CPU
path: the modules raise on CPU tensors.
"""
from __future__ import annotations

import math

import torch
import torch.nn.functional as F

from . import attention, backward_workspace_size, prepare_backward, workspace_size


class MraAttentionFunction(torch.autograd.Function):
    """out = MRA-2(q, k, v) on [batch, heads, seq_len, 64 or 128] tensors; its
    backward is mra_attention_bwd (bf16 or fp32), which takes the forward's selection
    as fixed ([MRA] 第三步) and in full mode differentiates the low-res branch
    through the block means ([MRA] 第四步)."""

    @staticmethod
    def forward(ctx, q, k, v, mask, block_per_row, approx_mode, prior_first, prior_diag,
                score_ranking="row_normalized", scale_dim=0):
        B, H, N, d = q.shape
        ws = torch.empty(workspace_size(B, H, N, d, q.dtype, block_per_row, approx_mode), dtype=torch.uint8,
                         device=q.device)
        out = attention(q, k, v, mask, block_per_row, approx_mode, prior_first, prior_diag, workspace=ws,
                        score_ranking=score_ranking, scale_dim=scale_dim, save_stats=True)
        ctx.save_for_backward(q, k, v, out, ws, mask if mask is not None else torch.empty(0, device=q.device))
        ctx.has_mask = mask is not None
        ctx.args = (block_per_row, approx_mode, prior_first, prior_diag, scale_dim)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, ws, mask = ctx.saved_tensors
        mask = mask if ctx.has_mask else None
        block_per_row, approx_mode, prior_first, prior_diag, scale_dim = ctx.args
        B, H, N, d = q.shape
        bw = torch.empty(backward_workspace_size(B, H, N, d, q.dtype, block_per_row, approx_mode),
                         dtype=torch.uint8, device=q.device)
        call, grads = prepare_backward(q, k, v, out, dout.contiguous(), ws, mask, block_per_row, approx_mode,
                                       prior_first, prior_diag, bwd_workspace=bw, scale_dim=scale_dim)
        call()
        return grads[0], grads[1], grads[2], None, None, None, None, None, None, None


def mra_attention(q, k, v, mask=None, block_per_row=4, approx_mode="full", initial_prior_first_n_blocks=0,
                  initial_prior_diagonal_n_blocks=0, score_ranking="row_normalized"):
    """Differentiable MRA-2 attention on [batch, heads, seq_len, d] device
    tensors, d <= 128; mask is uint8 [batch, seq_len] (1 = valid) or None.
    Heads narrower than the kernels' 64 or 128 channels go to them
    zero-padded, with the logit scale of their own size ([MRA] engineering
    notes: the model pads small heads for the kernels; the zero channels
    change no sum), and the output is cut back to d channels."""
    d = q.shape[-1]
    if d > 128:
        raise ValueError("head_dim above 128 is not supported")
    hd = 64 if d <= 64 else 128
    if d == hd:
        return MraAttentionFunction.apply(q, k, v, mask, block_per_row, approx_mode, initial_prior_first_n_blocks,
                                          initial_prior_diagonal_n_blocks, score_ranking, 0)
    pad = lambda t: F.pad(t, (0, hd - d)).contiguous()
    out = MraAttentionFunction.apply(pad(q), pad(k), pad(v), mask, block_per_row, approx_mode,
                                     initial_prior_first_n_blocks, initial_prior_diagonal_n_blocks, score_ranking, d)
    return out[..., :d]


class MraSelfAttention(torch.nn.Module):
    """Query, key and value projections, head split, MRA-2 attention and head
    merge.  Parameters follow MraConfig ([MRA] MraConfig section):
    block_per_row, approx_mode, initial_prior_first_n_blocks,
    initial_prior_diagonal_n_blocks; score_ranking picks what step 2 ranks
    ("row_normalized" or "raw_logits").  head_dim = hidden_size / heads may
    be at most 128 (see mra_attention)."""

    def __init__(self, hidden_size=768, num_attention_heads=12, block_per_row=4, approx_mode="full",
                 initial_prior_first_n_blocks=0, initial_prior_diagonal_n_blocks=0, score_ranking="row_normalized"):
        super().__init__()
        if hidden_size % num_attention_heads != 0 or not 1 <= hidden_size // num_attention_heads <= 128:
            raise ValueError("hidden_size / num_attention_heads must be a whole number from 1 to 128")
        self.num_attention_heads = num_attention_heads
        self.head_dim = hidden_size // num_attention_heads
        self.query = torch.nn.Linear(hidden_size, hidden_size)
        self.key = torch.nn.Linear(hidden_size, hidden_size)
        self.value = torch.nn.Linear(hidden_size, hidden_size)
        self.block_per_row = block_per_row
        self.approx_mode = approx_mode
        self.prior_first = initial_prior_first_n_blocks
        self.prior_diag = initial_prior_diagonal_n_blocks
        self.score_ranking = score_ranking

    def _heads(self, x, B, N):
        return x.view(B, N, self.num_attention_heads, self.head_dim).transpose(1, 2).contiguous()

    def forward(self, hidden_states, attention_mask=None):
        """hidden_states [batch, seq_len, hidden]; attention_mask [batch,
        seq_len] (nonzero = valid) or None.  Any seq_len: it is padded to a
        multiple of 32 with masked tokens and cut back afterwards."""
        if not hidden_states.is_cuda:
            raise ValueError("MraSelfAttention runs on the GPU kernels only; move the module and inputs to cuda")
        B, N, _ = hidden_states.shape
        Np = max(32, math.ceil(N / 32) * 32)
        mask = None
        if attention_mask is not None or Np != N:
            mask = torch.ones(B, Np, dtype=torch.uint8, device=hidden_states.device)
            if attention_mask is not None:
                mask[:, :N] = (attention_mask != 0).to(torch.uint8)
            mask[:, N:] = 0
        x = F.pad(hidden_states, (0, 0, 0, Np - N)) if Np != N else hidden_states
        q = self._heads(self.query(x), B, Np)
        k = self._heads(self.key(x), B, Np)
        v = self._heads(self.value(x), B, Np)
        ctx = mra_attention(q, k, v, mask, self.block_per_row, self.approx_mode, self.prior_first, self.prior_diag,
                            self.score_ranking)
        ctx = ctx.transpose(1, 2).reshape(B, Np, -1)
        return ctx[:, :N]


class MraLayer(torch.nn.Module):
    """One encoder layer: MraSelfAttention, then BERT's self-output (dense,
    residual, LayerNorm), intermediate (dense, GELU) and output (dense,
    residual, LayerNorm) blocks.  Defaults follow MraConfig (hidden 768, 12
    heads, intermediate 3072, LayerNorm eps 1e-5).  Weights are random: no
    checkpoint is loaded."""

    def __init__(self, hidden_size=768, num_attention_heads=12, intermediate_size=3072, layer_norm_eps=1e-5,
                 **attention_kw):
        super().__init__()
        self.attention = MraSelfAttention(hidden_size, num_attention_heads, **attention_kw)
        self.attn_out = torch.nn.Linear(hidden_size, hidden_size)
        self.attn_norm = torch.nn.LayerNorm(hidden_size, eps=layer_norm_eps)
        self.intermediate = torch.nn.Linear(hidden_size, intermediate_size)
        self.out = torch.nn.Linear(intermediate_size, hidden_size)
        self.out_norm = torch.nn.LayerNorm(hidden_size, eps=layer_norm_eps)

    def forward(self, hidden_states, attention_mask=None):
        a = self.attention(hidden_states, attention_mask)
        h = self.attn_norm(self.attn_out(a) + hidden_states)
        return self.out_norm(self.out(F.gelu(self.intermediate(h))) + h)
