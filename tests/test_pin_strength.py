"""Strength of the oracle's pins: each plausible mistake below is planted in a
copy of the oracle (its Python or its C combine; on the CPU, in a temporary
directory; the repository's oracle is never touched), and the oracle pin
tests run against the copy must fail.  An unmutated copy must pass them.  Not planted: dropping the slot
capacity check, which the token and pick range checks already enforce, so no
pin can tell the two apart."""
import shutil
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent

MUTATIONS = {
    "slot_index_swapped": ("return (src_idx * top_k + src_topk) * msg_bytes + byte_off",
                           "return (src_topk * top_k + src_idx) * msg_bytes + byte_off"),
    "count_index_swapped": ("return e * n_ranks + rk", "return rk * n_ranks + e"),
    "bf16_truncates": ("r = np.rint(ax / ulp) * ulp", "r = np.floor(ax / ulp) * ulp"),
    "bf16_rounds_half_up": ("r = np.rint(ax / ulp) * ulp", "r = np.floor(ax / ulp + 0.5) * ulp"),
    "gemm_wrong_expert": ("we = bf16_to_f32(w_bits[e])           # [N][K]",
                          "we = bf16_to_f32(w_bits[min(e + 1, El - 1)])"),
    "gemm_drops_last_k": ("xe = bf16_to_f32(x_bits[rows[sel]])",
                          "xe = bf16_to_f32(x_bits[rows[sel]]); xe[:, -1] = 0"),
    "combine_takes_remote_picks": ("local = (g >= lo) & (g < lo + n_experts_per_device)",
                                   "local = g >= 0"),
    "combine_drops_weight": ("weights = np.asarray(topk_w, dtype=np.float32)[rk][t_idx, k_idx]",
                             "weights = np.ones(t_idx.size, dtype=np.float32)"),
    "grouping_sort_key": ("order = np.lexsort((k, t, rk, e))", "order = np.lexsort((t, k, rk, e))"),
    "fp8_exponent_bias": ("(1.0 + mf / 8.0) * np.ldexp(1.0, (ef - 7))",
                          "(1.0 + mf / 8.0) * np.ldexp(1.0, (ef - 8))"),
    "fp8_weight_scale_index": (
        "sw = np.repeat(np.asarray(w_scale, dtype=np.float32)[e], 128, axis=0)",
        "sw = np.tile(np.asarray(w_scale, dtype=np.float32)[e], (128, 1))"),
    "election_off_by_one": ("if old == self.El - 1:",
                            "if old == self.El - 2 or (self.El == 1 and old == 0):"),
    "row_picks_rank_from_expert": ("return np.stack([gi % n_ranks, src[:, 0], src[:, 1]], axis=1)",
                                   "return np.stack([gi // n_ranks, src[:, 0], src[:, 1]], axis=1)"),
    "e4m3_encode_truncates": ("m = np.rint((2.0 * frac - 1.0) * 8.0).astype(np.int64)",
                              "m = np.floor((2.0 * frac - 1.0) * 8.0).astype(np.int64)"),
    "e4m3_encode_bias": ("code_n = np.minimum(((e + 7) << 3) | m, 0x7E)",
                         "code_n = np.minimum(((e + 8) << 3) | m, 0x7E)"),
    "e4m3_encode_subnormal_step": ("code_s = np.rint(a * 2.0 ** 9).astype(np.int64)",
                                   "code_s = np.rint(a * 2.0 ** 8).astype(np.int64)"),
    "quant_scale_range": ("scale = (amax / np.float32(448.0)).astype(np.float32)",
                          "scale = (amax / np.float32(240.0)).astype(np.float32)"),
    "fp8_swiglu_gate_up_swapped": ("""    gu = expert_rows_fp8(x1q, x1_scale, w1q, w1_scale, offsets, n_ranks, rows)
    half = gu.shape[1] // 2
    g, u = gu[:, :half], gu[:, half:]""", """    gu = expert_rows_fp8(x1q, x1_scale, w1q, w1_scale, offsets, n_ranks, rows)
    half = gu.shape[1] // 2
    u, g = gu[:, :half], gu[:, half:]"""),
}
# mistakes planted in the C combine
C_MUTATIONS = {
    "combine_descending_k": ("for (int64_t p = first[i]; p < first[i + 1]; ++p)",
                             "for (int64_t p = first[i + 1] - 1; p >= first[i]; --p)"),
    "combine_unfused": ("acc[j] = fmaf(w, bf16_value(row[j]), acc[j]);",
                        "acc[j] = w * bf16_value(row[j]) + acc[j];"),
}


def _copy_tree(dst: Path, mutation=None):
    shutil.copytree(ROOT / "oracle", dst / "oracle",
                    ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copytree(ROOT / "ep_synth", dst / "ep_synth",
                    ignore=shutil.ignore_patterns("__pycache__"))
    (dst / "tests").mkdir()
    shutil.copytree(ROOT / "tests" / "golden", dst / "tests" / "golden")
    for f in ["conftest.py",
              *[p.name for p in (ROOT / "tests").glob("test_oracle_*.py")]]:
        shutil.copy(ROOT / "tests" / f, dst / "tests" / f)
    for lib in (dst / "oracle").glob("*.so"):
        lib.unlink()                   # the copy builds its own combine library
    if mutation is not None:
        name, (before, after) = mutation
        src_file = dst / "oracle" / ("combine.c" if name in C_MUTATIONS else "__init__.py")
        src = src_file.read_text()
        assert before in src, "the oracle no longer holds the text this mutation replaces"
        src_file.write_text(src.replace(before, after))


def _pins(dst: Path):
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           "-m", "not gpu", "tests"], cwd=dst, capture_output=True, text=True,
                          timeout=600)


def test_pins_pass_on_an_unmutated_copy(tmp_path):
    _copy_tree(tmp_path)
    r = _pins(tmp_path)
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTATIONS) + sorted(C_MUTATIONS))
def test_planted_mistake_is_caught(tmp_path, name):
    _copy_tree(tmp_path, (name, {**MUTATIONS, **C_MUTATIONS}[name]))
    r = _pins(tmp_path)
    assert r.returncode != 0, f"{name} was not caught by any pin:\n{r.stdout[-1000:]}"
