"""Per-module quantization schemes for a decoder layer's linear projections, resolved fail
closed, and the layer's projections executed with the scheme each module resolved to.

"feat(quantization): support compressed-tensors W8A8 and mixed modules" (Summary; Design and
Supported Execution Scheme; Notes for Reviewers) describes the rules followed here:

* a module's scheme comes from the quantization groups whose targets match it, the most
  specific match winning: an exact module name over a ``re:`` regular expression over a
  module type; two groups matching at the same specificity is an error (the order of the
  groups never decides); a module that an ignore entry matches stays unquantized (BF16),
  whatever the groups say (the page's hybrid checkpoint keeps a module in BF16 by listing
  it there);
* only schemes with a kernel are executable (per-channel W8A8 with dynamic per-token
  activations, its group-128 weight-scale variant, weight-only W8A16, unquantized BF16);
  any other resolved scheme is an error naming the module path, never a silent substitute;
* q/k/v and gate/up run as fused projections and must resolve to one scheme (an explicit
  error otherwise); o and down are selectable on their own, which gives mixed W8A8/BF16
  layers.

Execution: quantized modules run the library's kernels (per-token quantization and
w8a8_gemm, w8a8_gemm_g128 or w8a16_gemm).  Unquantized (BF16) modules are not on the int8
path: they run a plain bf16 library GEMM (``torch.matmul``, hipBLASLt on ROCm).
"""
from __future__ import annotations

import re
from dataclasses import dataclass, field

import torch

from . import _binding as lib

W8A8 = "w8a8"            # int8 per-channel weights, dynamic int8 per-token activations
W8A8_G128 = "w8a8_g128"  # the same with one weight scale per 128 input channels
W8A16 = "w8a16"          # int8 per-channel weights, bf16 activations
BF16 = "bf16"            # unquantized
EXECUTABLE = (W8A8, W8A8_G128, W8A16, BF16)

PROJECTIONS = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")
MODULE_TYPE = {"q_proj": "Linear", "k_proj": "Linear", "v_proj": "Linear", "o_proj": "Linear",
               "gate_proj": "Linear", "up_proj": "Linear", "down_proj": "Linear"}
FUSED = {"qkv": ("q_proj", "k_proj", "v_proj"), "o": ("o_proj",),
         "gate_up": ("gate_proj", "up_proj"), "down": ("down_proj",)}
FUSED_INPUT = {"qkv": "attn_in", "o": "attn_out", "gate_up": "mlp_in", "down": "mlp_mid"}


class SchemeError(ValueError):
    """A module's quantization cannot be resolved to an executable scheme; the message starts
    with the module path."""


@dataclass
class QuantGroup:
    """One quantization group: the scheme it assigns and the targets it applies to (exact
    module names, ``re:`` regular expressions over module paths, or module type names)."""
    name: str
    scheme: str
    targets: list = field(default_factory=list)


# specificity of a target match: exact path > regular expression > module type
_EXACT, _REGEX, _TYPE = 3, 2, 1


def _match(target: str, path: str, mtype: str) -> int:
    if target.startswith("re:"):
        return _REGEX if re.fullmatch(target[3:], path) else 0
    if target == path:
        return _EXACT
    if target == mtype:
        return _TYPE
    return 0


def resolve_module(path: str, mtype: str, groups, ignore=()) -> str:
    """The scheme of module ``path`` (of type ``mtype``): BF16 if an ignore entry matches it,
    else that of the group whose target matches it most specifically, else BF16.  Raises
    SchemeError when several groups match at the highest specificity or the scheme has no
    kernel."""
    if any(_match(t, path, mtype) for t in ignore):
        return BF16
    best, found = 0, []
    for grp in groups:
        spec = max((_match(t, path, mtype) for t in grp.targets), default=0)
        if spec > best:
            best, found = spec, [grp]
        elif spec == best and spec > 0:
            found.append(grp)
    if not found:
        return BF16
    if len(found) > 1:
        raise SchemeError(f"{path}: matched by groups "
                          f"{', '.join(repr(g.name) for g in found)} at the same specificity")
    if found[0].scheme not in EXECUTABLE:
        raise SchemeError(f"{path}: scheme '{found[0].scheme}' of group '{found[0].name}' has "
                          f"no kernel")
    return found[0].scheme


def resolve_layer(prefix: str, groups, ignore=()) -> dict:
    """Schemes of a decoder layer's fused projections {qkv, o, gate_up, down}, from its seven
    modules ``{prefix}.self_attn.{q,k,v,o}_proj`` and ``{prefix}.mlp.{gate,up,down}_proj``.
    A fused projection whose members resolve differently is an error naming them."""
    paths = {p: f"{prefix}.{'self_attn' if p[0] in 'qkvo' else 'mlp'}.{p}" for p in PROJECTIONS}
    per = {p: resolve_module(paths[p], MODULE_TYPE[p], groups, ignore) for p in PROJECTIONS}
    out = {}
    for fused, parts in FUSED.items():
        got = {per[p] for p in parts}
        if len(got) > 1:
            detail = ", ".join(f"{paths[p]} = {per[p]}" for p in parts)
            raise SchemeError(f"{paths[parts[0]]}: the fused {fused} projection needs one "
                              f"scheme for all of its modules ({detail})")
        out[fused] = per[parts[0]]
    return out


class FusedLinear:
    """One fused projection (its member modules' weights concatenated along N) executed in one
    scheme.  Weights: bf16 [N, K] on the GPU; bias fp32 [N] or None."""

    def __init__(self, scheme: str, weight: torch.Tensor, bias=None):
        if scheme not in EXECUTABLE:
            raise SchemeError(f"scheme '{scheme}' has no kernel")
        self.scheme = scheme
        self.bias = bias
        if scheme == BF16:
            self.w = weight.to(torch.bfloat16).contiguous()
        elif scheme == W8A8_G128:
            self.wq, self.ws = lib.quantize_per_group_int8(weight)
        else:
            self.wq, self.ws = lib.quantize_per_channel_int8(weight)

    def __call__(self, x: torch.Tensor, qx=None) -> torch.Tensor:
        """x: bf16 [M, K].  qx: this input already quantized per token (codes, scales), shared
        by the projections that read the same input."""
        if self.scheme == BF16:
            y = torch.matmul(x, self.w.t())
            return y if self.bias is None else (y.float() + self.bias).to(torch.bfloat16)
        if self.scheme == W8A16:
            return lib.w8a16_gemm(x, self.wq, self.ws, self.bias)
        q, s = qx if qx is not None else lib.quantize_per_token_int8(x)
        if self.scheme == W8A8_G128:
            return lib.w8a8_gemm_g128(q, s, self.wq, self.ws, self.bias)
        return lib.w8a8_gemm(q, s, self.wq, self.ws, self.bias)


class DecoderLinears:
    """The linear projections of one decoder layer, each fused projection in the scheme its
    modules resolved to (``resolve_layer``).  ``weights``: {module name: bf16 [N, K]} for the
    seven projections; ``biases``: optional {module name: fp32 [N]}."""

    def __init__(self, schemes: dict, weights: dict, biases=None):
        biases = biases or {}
        self.schemes = dict(schemes)
        self.proj = {}
        for fused, parts in FUSED.items():
            w = torch.cat([weights[p] for p in parts]).contiguous()
            bs = [biases.get(p) for p in parts]
            b = None if all(v is None for v in bs) else torch.cat(
                [v if v is not None else torch.zeros(weights[p].shape[0], device=w.device)
                 for v, p in zip(bs, parts)]).float().contiguous()
            self.proj[fused] = FusedLinear(schemes[fused], w, b)

    def run(self, inputs: dict) -> dict:
        """{fused projection: output} for the layer inputs {attn_in, attn_out, mlp_in,
        mlp_mid} (bf16 [M, K]); each input is quantized per token once for the W8A8
        projections that read it."""
        qx, out = {}, {}
        for fused, p in self.proj.items():
            key = FUSED_INPUT[fused]
            shared = None
            if p.scheme in (W8A8, W8A8_G128):
                if key not in qx:
                    qx[key] = lib.quantize_per_token_int8(inputs[key])
                shared = qx[key]
            out[fused] = p(inputs[key], shared)
        return out
