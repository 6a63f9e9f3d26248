"""Library reference for the oracle pins: transformers' GPT-2 in float64 on the CPU.

GPT-2 as implemented by an independent library (LayerNorm with epsilon 1e-5,
Conv1D projections stored [input][output], tanh GELU, causal attention scaled by
1/sqrt(head_dim), tied output head).  The packed synthetic checkpoint is mapped
onto its parameters by the checkpoint order the oracle reads; an offset, an
orientation or a formula mistake in the oracle therefore shows up as a logit
difference far above float32 rounding.
"""
from __future__ import annotations

import logging

import numpy as np
import torch

import synth


def _quiet() -> None:
    for name in ("transformers", "transformers.configuration_utils", "transformers.modeling_utils"):
        logging.getLogger(name).setLevel(logging.ERROR)


def build(w: np.ndarray, d: synth.Dims, f16: bool = False):
    """f16: binary16 weight storage (gpt2.s page, options, -h) -- the four block
    matrices and an untied output head are the checkpoint's values rounded to
    binary16 by numpy's conversion, while the embedding table keeps the binary32
    values."""
    _quiet()
    from transformers import GPT2Config, GPT2LMHeadModel

    cfg = GPT2Config(n_layer=d.n_layer, n_embd=d.d_model, n_head=d.n_head, n_inner=d.d_ff,
                     vocab_size=d.vocab, n_positions=d.n_pos_rows, activation_function="gelu_new",
                     resid_pdrop=0.0, embd_pdrop=0.0, attn_pdrop=0.0, layer_norm_epsilon=1e-5,
                     bos_token_id=0, eos_token_id=0, tie_word_embeddings=not f16)
    cfg._attn_implementation = "eager"
    with torch.device("meta"):
        model = GPT2LMHeadModel(cfg)
    off = synth.offsets(d)
    D, F = d.d_model, d.d_ff

    def t(name, shape, half=False):
        o, n = off[name]
        v = w[o:o + n]
        if half:
            v = v.astype(np.float16)
        return torch.from_numpy(v.astype(np.float64).reshape(shape))

    sd = {"transformer.wte.weight": t("wte", (d.vocab, D)),
          "transformer.wpe.weight": t("wpe", (d.n_pos_rows, D)),
          "transformer.ln_f.weight": t("lnf_g", (D,)),
          "transformer.ln_f.bias": t("lnf_b", (D,))}
    hf_names = {"ln1_g": ("ln_1.weight", (D,)), "ln1_b": ("ln_1.bias", (D,)),
                "attn_w": ("attn.c_attn.weight", (D, 3 * D)), "attn_b": ("attn.c_attn.bias", (3 * D,)),
                "attnproj_w": ("attn.c_proj.weight", (D, D)), "attnproj_b": ("attn.c_proj.bias", (D,)),
                "ln2_g": ("ln_2.weight", (D,)), "ln2_b": ("ln_2.bias", (D,)),
                "fc_w": ("mlp.c_fc.weight", (D, F)), "fc_b": ("mlp.c_fc.bias", (F,)),
                "mlpproj_w": ("mlp.c_proj.weight", (F, D)), "mlpproj_b": ("mlp.c_proj.bias", (D,))}
    for l in range(d.n_layer):
        for ours, (theirs, shape) in hf_names.items():
            sd[f"transformer.h.{l}.{theirs}"] = t(f"h{l}.{ours}", shape, half=f16 and ours.endswith("_w"))
    sd["lm_head.weight"] = t("wte", (d.vocab, D), half=True) if f16 else sd["transformer.wte.weight"]
    model = model.to_empty(device="cpu").double()
    missing, unexpected = model.load_state_dict(sd, strict=False)
    bad = [m for m in missing if not m.endswith("attn.bias") and not m.endswith("masked_bias")]
    assert not bad and not unexpected, (bad, unexpected)
    if not f16:
        model.tie_weights()
    model.eval()
    return model


@torch.no_grad()
def logits_all_positions(model, toks: np.ndarray) -> np.ndarray:
    ids = torch.from_numpy(np.asarray(toks, dtype=np.int64))[None, :]
    return model(input_ids=ids).logits[0].numpy()


@torch.no_grad()
def cache_all_positions(model, toks: np.ndarray, d: synth.Dims) -> np.ndarray:
    """The float64 keys and values of every position and layer, in the cachedStep
    layout: word (position*n_layer + layer)*2D + offset, keys then values."""
    ids = torch.from_numpy(np.asarray(toks, dtype=np.int64))[None, :]
    pkv = model(input_ids=ids, use_cache=True).past_key_values
    T, D = len(toks), d.d_model
    out = np.zeros((T, d.n_layer, 2 * D))
    for l in range(d.n_layer):
        lay = pkv.layers[l] if hasattr(pkv, "layers") else None
        k, v = (lay.keys, lay.values) if lay is not None else pkv[l]
        out[:, l, :D] = k[0].permute(1, 0, 2).reshape(T, D).numpy()   # [heads][T][dh] -> [T][heads*dh]
        out[:, l, D:] = v[0].permute(1, 0, 2).reshape(T, D).numpy()
    return out.reshape(-1)
