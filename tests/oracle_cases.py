"""Small shared input builders for the CPU oracle tests (no arithmetic of the method)."""
import numpy as np

from long_context_split_amd import synth


def layer_np(lens, nq, seed, head_dim=256, scales=None, key_mix=0.0, max_blocks=None):
    inp = synth.make_layer(lens, nq, seed_base=seed, layer=0, device="cpu", scales=scales,
                           key_mix=key_mix, head_dim=head_dim, max_blocks=max_blocks)
    return inp.numpy()


def args(d):
    return (d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["context_lens"],
            d["k_scale"], d["v_scale"], d["softmax_scale"])


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))
