"""Planted mistakes: each pin must be able to fail.

Every case below copies oracle/gs_oracle.cpp, changes one statement into a plausible
mistake (a comparison, a sign, a dropped term, a mask on the wrong quantity), builds the
copy with the oracle's own flags into a temporary directory and runs the pins named for
it against that build.  At least one of them must fail.  Nothing here touches the
committed oracle or its library, and nothing runs on a GPU.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from tests import test_oracle_camera_grad as cpins
from tests import test_oracle_charbonnier as chpins
from tests import test_oracle_densify as dpins
from tests import test_oracle_mip as mpins
from tests import test_oracle_overlap as opins
from tests import test_oracle_relocate as rpins
from tests import test_oracle_pins as pins
from tests import test_oracle_threshold_pins as tpins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "gs_oracle.cpp")


def _fd_smooth(seeds):
    def run(O):
        for s in seeds:
            pins.test_gradients_finite_difference_smooth(O, s, 1 + s % 8, (0, 1, 3)[s % 3])
    return run


def _fd_thresholded(cases):
    def run(O):
        for c in cases:
            tpins.fd_check_thresholded(O, *c)
    return run


def _pin(fn, *args):
    return lambda O: fn(O, *args)


def _with_mip(fn, *args):
    """A pin that needs the Mip-Splatting compensation switched on (its fixture's job)."""
    def run(O):
        O.set_mip_compensation(True)
        try:
            fn(O, *args)
        finally:
            O.set_mip_compensation(False)
    return run


# name: (statement as written in the oracle, the planted version, pins that must catch it)
MUTANTS = {
    "cap_at_or_above": (
        "capped = araw > R(kAlphaCap);",
        "capped = araw >= R(kAlphaCap);",
        [_pin(tpins.test_alpha_exactly_at_cap_passes_gradient)]),
    "capped_alpha_passes_gradient": (
        "    if (capped) continue;                // alpha = 0.99 does not depend on opacity or position\n",
        "",
        [_pin(tpins.test_capped_alpha_closed_form), _fd_thresholded([tpins.THR_CASES[6]])]),
    "clamp_mask_on_clamped_colour": (
        "gc[ch] = (!smooth && f.raw[ch] < R(0)) ? R(0) : GS(6 + ch);",
        "gc[ch] = (!smooth && f.rgb[ch] <= R(0)) ? R(0) : GS(6 + ch);",
        [_pin(tpins.test_colour_exactly_zero_passes_gradient)]),
    "clamp_mask_missing": (
        "gc[ch] = (!smooth && f.raw[ch] < R(0)) ? R(0) : GS(6 + ch);",
        "gc[ch] = GS(6 + ch);",
        [_pin(tpins.test_clamped_channel_closed_form), _fd_thresholded([tpins.THR_CASES[2]])]),
    "clamp_mask_missing_in_view_direction": (
        "for (int a = 0; a < 3; ++a) gdir[a] += gc[ch] * coef * f.dY[k][a];",
        "for (int a = 0; a < 3; ++a) gdir[a] += GS(6 + ch) * coef * f.dY[k][a];",
        [_pin(tpins.test_clamped_channel_adds_no_view_direction_term), _fd_thresholded([tpins.THR_CASES[2]])]),
    "view_direction_term_dropped": (
        "  if (K > 0) {\n",
        "  if (false) {\n",
        [_fd_smooth([1, 2])]),
    "conic_B_sign": (
        "gscreen[3 * n + g] += ge * dx * dy;",
        "gscreen[3 * n + g] -= ge * dx * dy;",
        [_fd_smooth([0, 1])]),
    "jacobian_depth_path_dropped": (
        "  dp[0] += dJ[0][2] * (-fx / pz2);\n",
        "",
        [_fd_smooth([0, 1])]),
    "quaternion_sign": (
        "gq[0] = R(2) * (-z * dR[0][1]",
        "gq[0] = R(2) * (z * dR[0][1]",
        [_fd_smooth([0, 1])]),
    "early_stop_disabled": (
        "      if (stop) break;\n",
        "",
        [_pin(pins.test_early_stop_and_contributor_count)]),
    "ssim_variance_derivative_sign": (
        "dsx[idx] = -(A1 * A2) / (B1 * B2 * B2);",
        "dsx[idx] = (A1 * A2) / (B1 * B2 * B2);",
        [_pin(pins.test_loss_gradient_finite_difference)]),
    # the method's constants and the other stages
    "dilation_dropped": (
        "constexpr double kDilation = 0.3;",
        "constexpr double kDilation = 0.0;",
        [_pin(pins.test_projected_spread, 10.0, 5.0), _pin(pins.test_projected_spread, 20.0, 2.5)]),
    "alpha_floor_one_in_256": (
        "constexpr double kAlphaMinInv = 255.0;",
        "constexpr double kAlphaMinInv = 256.0;",
        [_pin(pins.test_alpha_floor_is_one_in_255)]),
    "early_stop_threshold_looser": (
        "constexpr double kTStop = 1e-4;",
        "constexpr double kTStop = 1e-3;",
        [_pin(pins.test_early_stop_and_contributor_count),
         _pin(opins.test_overlap_counts_every_entry_at_or_above_the_floor)]),
    "extent_cut_smaller": (
        "constexpr double kExtentCut = 4.5;",
        "constexpr double kExtentCut = 3.0;",
        [_pin(pins.test_tiled_render_equals_untiled_below_extent_opacity)]),
    "tile_id_column_major": (
        "keys[pos] = (uint64_t(uint32_t(y * tx + x)) << 32) | dbits;",
        "keys[pos] = (uint64_t(uint32_t(x * ty + y)) << 32) | dbits;",
        [_pin(pins.test_sort_and_ranges_brute_force, 0), _pin(pins.test_sort_and_ranges_brute_force, 1)]),
    "ssim_window_sigma": (
        "const double sigma = 1.5;",
        "const double sigma = 2.0;",
        [_pin(pins.test_loss_matches_independent_separable_ssim)]),
    "loss_weights_swapped": (
        "out[0] = (R(1) - lambda) * L1 + lambda * (R(1) - SS);",
        "out[0] = lambda * L1 + (R(1) - lambda) * (R(1) - SS);",
        [_pin(pins.test_loss_gradient_finite_difference), _pin(pins.test_l1_subgradient_and_normaliser)]),
    "colour_clamp_dropped": (
        "f.rgb[ch] = smooth ? col : std::max(col, R(0));",
        "f.rgb[ch] = col;",
        [_pin(tpins.test_clamped_channel_closed_form)]),
    "sh_band1_sign": (
        "const R n10 = R(sh_norm(1, 0)), n11 = R(-sh_norm(1, 1));",
        "const R n10 = R(sh_norm(1, 0)), n11 = R(sh_norm(1, 1));",
        [_pin(pins.test_sh_printed_constants)]),
    "depth_order_reversed": (
        "    std::memcpy(&dbits, &depth[i], 4);\n",
        "    std::memcpy(&dbits, &depth[i], 4);\n    dbits = ~dbits;\n",
        [_pin(pins.test_sort_and_ranges_brute_force, 0), _pin(pins.test_two_gaussian_compositing,
                                                               "two_gaussians_nearest_first")]),
    "opacity_activation_exp": (
        "  f.ob = sigmoid_r(P(10));",
        "  f.ob = exp_r(P(10));",
        [_pin(pins.test_opacity_gradient_worked_example), _fd_smooth([0])]),
    # the trainer's variants and density control
    "camera_rotation_sign": (
        "out[0] += M[2][1] - M[1][2];",
        "out[0] += M[1][2] - M[2][1];",
        [_pin(cpins.test_camera_grad_matches_central_differences), _pin(cpins.test_position_only_is_the_pages_torque)]),
    "split_children_not_shrunk": (
        "if (shrink && k >= 3 && k < 6) th = th - lscale_shrink;",
        "",
        [_pin(dpins.test_hand_built_population)]),
    "relocated_donor_not_shrunk": (
        "for (int pl = 3; pl < 6; ++pl) params[pl * n + bd] = params[pl * n + bd] - lscale_shrink;",
        "",
        [_pin(rpins.test_hand_worked_population)]),
    "charbonnier_delta_kept": (
        "sl += double(root - delta);",
        "sl += double(root);",
        [_pin(chpins.test_zero_error_is_zero), _pin(chpins.test_single_element_closed_form)]),
    "mip_compensation_inverted": (
        "f.comp = std::sqrt(std::max(f.detv, R(0)) / f.det);",
        "f.comp = std::sqrt(f.det / std::max(f.detv, R(1e-30)));",
        [_with_mip(mpins.test_isotropic_closed_form)]),
    "adam_bias_correction_dropped": (
        "const R mh = m[k] / R(bc1), vh = v[k] / R(bc2);",
        "const R mh = m[k], vh = v[k];",
        [_pin(pins.test_adam_first_step_closed_form),
         _pin(pins.test_adam_zero_gradient_keeps_moving_with_momentum)]),
}


def _build(name, tmpdir):
    orig, planted, _ = MUTANTS[name]
    src = open(ORACLE_SRC).read()
    assert src.count(orig) == 1, f"{name}: the statement to change is not in the oracle exactly once"
    path = os.path.join(tmpdir, f"{name}.cpp")
    with open(path, "w") as f:
        f.write(src.replace(orig, planted))
    so = os.path.join(tmpdir, f"lib_{name}.so")
    subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC", path,
                    "-o", so], check=True, capture_output=True)
    return so


@pytest.fixture(scope="module")
def mutant_libs(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("oracle_mutants"))
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        libs = dict(zip(MUTANTS, ex.map(lambda n: _build(n, d), MUTANTS)))
    return libs


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_fails_a_pin(oracle, mutant_libs, name):
    caught = 0
    with oracle.library(mutant_libs[name]):
        for check in MUTANTS[name][2]:
            try:
                check(oracle)
            except AssertionError:
                caught += 1
    assert caught > 0, f"no pin caught the planted mistake {name}"


def test_unplanted_oracle_passes_the_same_pins(oracle):
    """The checks used above pass on the committed oracle (so a failure above is the
    planted mistake's doing)."""
    for _, _, checks in MUTANTS.values():
        for check in checks:
            check(oracle)
