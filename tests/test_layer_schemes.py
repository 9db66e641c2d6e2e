"""Per-module scheme resolution of a decoder layer (host logic, no GPU): the rules of
"feat(quantization): support compressed-tensors W8A8 and mixed modules" (Summary; Design and
Supported Execution Scheme; Notes for Reviewers): exact > regex > type precedence, ambiguity
and unsupported schemes failing closed with the module path, ignored modules unquantized,
one scheme per fused q/k/v and gate/up projection, o and down free."""
import pytest

from int8_quantized_linear_amd.layer import (BF16, W8A8, W8A8_G128, W8A16, QuantGroup,
                                             SchemeError, resolve_layer, resolve_module)

P = "model.layers.0"


def test_type_target_quantizes_every_linear():
    g = [QuantGroup("group_0", W8A8, ["Linear"])]
    assert resolve_layer(P, g) == {"qkv": W8A8, "o": W8A8, "gate_up": W8A8, "down": W8A8}


def test_no_group_means_unquantized():
    assert resolve_layer(P, []) == {"qkv": BF16, "o": BF16, "gate_up": BF16, "down": BF16}


def test_precedence_exact_over_regex_over_type():
    g = [QuantGroup("by_type", W8A8, ["Linear"]),
         QuantGroup("by_regex", W8A16, [r"re:.*\.mlp\.down_proj"]),
         QuantGroup("by_name", W8A8_G128, [f"{P}.mlp.down_proj"])]
    assert resolve_module(f"{P}.mlp.down_proj", "Linear", g) == W8A8_G128
    assert resolve_module(f"{P}.mlp.down_proj", "Linear", g[:2]) == W8A16
    assert resolve_module(f"{P}.mlp.up_proj", "Linear", g) == W8A8
    # the order of the groups does not decide
    assert resolve_module(f"{P}.mlp.down_proj", "Linear", g[::-1]) == W8A8_G128


def test_equal_specificity_is_ambiguous_even_with_one_scheme():
    g = [QuantGroup("a", W8A8, [r"re:.*_proj"]), QuantGroup("b", W8A8, [r"re:.*\.o_proj"])]
    with pytest.raises(SchemeError, match=rf"^{P}\.self_attn\.o_proj: matched by groups 'a', 'b'"):
        resolve_module(f"{P}.self_attn.o_proj", "Linear", g)
    # a more specific target removes the ambiguity
    g.append(QuantGroup("c", W8A16, [f"{P}.self_attn.o_proj"]))
    assert resolve_module(f"{P}.self_attn.o_proj", "Linear", g) == W8A16


def test_unsupported_scheme_fails_closed_with_the_path():
    g = [QuantGroup("int4", "w4a16", ["Linear"])]
    with pytest.raises(SchemeError, match=rf"^{P}\.self_attn\.q_proj: scheme 'w4a16'"):
        resolve_layer(P, g)


def test_ignored_module_stays_bf16_and_mixes_with_w8a8():
    """The page's hybrid layer: W8A8 everywhere except the o projection, which the ignore
    list keeps in BF16."""
    g = [QuantGroup("group_0", W8A8, ["Linear"])]
    got = resolve_layer(P, g, ignore=[f"{P}.self_attn.o_proj", "lm_head"])
    assert got == {"qkv": W8A8, "o": BF16, "gate_up": W8A8, "down": W8A8}
    got = resolve_layer(P, g, ignore=[r"re:.*down_proj"])
    assert got["down"] == BF16 and got["gate_up"] == W8A8


@pytest.mark.parametrize("module,fused", [("k_proj", "qkv"), ("up_proj", "gate_up")])
def test_fused_projections_need_one_scheme(module, fused):
    part = "self_attn" if fused == "qkv" else "mlp"
    g = [QuantGroup("group_0", W8A8, ["Linear"])]
    with pytest.raises(SchemeError, match=f"fused {fused} projection needs one scheme"):
        resolve_layer(P, g, ignore=[f"{P}.{part}.{module}"])
    g2 = g + [QuantGroup("wo", W8A16, [f"{P}.{part}.{module}"])]
    with pytest.raises(SchemeError, match=rf"{P}\.{part}\.{module} = {W8A16}"):
        resolve_layer(P, g2)
