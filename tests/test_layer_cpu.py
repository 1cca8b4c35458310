"""CPU checks of the torch modules' argument handling (no kernel runs here)."""
import pytest
import torch

from block_sparse_approximate_amd import layer


def test_head_size_at_most_128():
    with pytest.raises(ValueError):
        layer.MraSelfAttention(hidden_size=512, num_attention_heads=2)     # 256
    assert layer.MraSelfAttention(hidden_size=256, num_attention_heads=2).head_dim == 128
    assert layer.MraSelfAttention(hidden_size=288, num_attention_heads=3).head_dim == 96
    with pytest.raises(ValueError):
        layer.MraSelfAttention(hidden_size=250, num_attention_heads=4)     # not whole
    assert layer.MraSelfAttention(hidden_size=256, num_attention_heads=4).head_dim == 64
    assert layer.MraSelfAttention(hidden_size=256, num_attention_heads=8).head_dim == 32
    assert layer.MraSelfAttention(hidden_size=16, num_attention_heads=2).head_dim == 8


def test_modules_refuse_cpu_inputs():
    # there is no CPU path: the attention runs in the HIP kernels only
    mod = layer.MraLayer(hidden_size=128, num_attention_heads=2, intermediate_size=256)
    with pytest.raises(ValueError):
        mod(torch.zeros(1, 64, 128))


def test_layer_shapes_follow_the_config():
    mod = layer.MraLayer(block_per_row=2, approx_mode="sparse", initial_prior_diagonal_n_blocks=3)
    assert mod.intermediate.out_features == 3072 and mod.attn_norm.eps == 1e-5
    assert mod.attention.num_attention_heads == 12 and mod.attention.prior_diag == 3
