"""The oracle's geometry and split indices against the facts printed on the pages."""
import json
import os

from oracle import GEOMETRY, fp8_weight_elements, layout

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def test_projection_shapes():
    lay = layout()
    assert [lay["d_in_proj"], GEOMETRY["hidden"]] == FACTS["in_proj_shape_out_in"]["value"]
    assert [GEOMETRY["hidden"], lay["d_inner"]] == FACTS["out_proj_shape_out_in"]["value"]
    assert GEOMETRY["n_heads"] == FACTS["n_heads"]["value"]


def test_partitions_add_up():
    lay = layout()
    assert lay["z_width"] + lay["xbc_width"] + lay["dt_width"] == lay["d_in_proj"] == 10304
    assert lay["x_width"] + lay["b_width"] + lay["c_width"] == lay["conv_dim"] == 6144
    # head, middle, tail of an in_proj row, widths (I, conv_dim, num_heads)
    assert (lay["z_off"], lay["xbc_off"], lay["dt_off"]) == (0, 4096, 10240)
    assert (lay["z_width"], lay["xbc_width"], lay["dt_width"]) == (4096, 6144, 64)
    assert (lay["x_off"], lay["b_off"], lay["c_off"]) == (0, 4096, 5120)
    assert lay["dt_width"] == FACTS["n_heads"]["value"]
    assert lay["heads_per_group"] == 8 and lay["norm_group"] == 512


def test_weight_element_count():
    n = fp8_weight_elements(FACTS["n_mamba_layers"]["value"])
    assert n == 23 * (10304 * 2688 + 2688 * 4096) == 890_265_600
    assert abs(n - FACTS["per_token_reexpanded_elements_approx"]["value"]) / 890e6 < 5e-4


def test_ssm_widening_bytes():
    # 23 layers x 3 f32 tensors x 64 heads x 2 bytes widened (bf16 -> f32)
    f = FACTS
    assert f["n_mamba_layers"]["value"] * f["f32_ssm_params_per_layer"]["value"] * f["n_heads"]["value"] * 2 \
        == f["ssm_widening_bytes"]["value"]


def test_probe_shapes_are_the_projections():
    lay = layout()
    for m, n, k in FACTS["probe_shapes_mnk"]["value"][:5]:
        assert (n, k) in [(lay["d_in_proj"], GEOMETRY["hidden"]), (GEOMETRY["hidden"], lay["d_inner"])]
