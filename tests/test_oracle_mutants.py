"""Plant plausible mistakes in copies of the oracle source (on the CPU) and
show that the pins catch every one of them: a dropped term, a wrong sign, a
swapped operand, a wrong stride or index, a wrong tie rule, a missing
normalisation or weight."""
import os
import tempfile

import pytest

import oracle
import oracle_pins

MUTANTS = {
    "lora_term_dropped": ("? base + dot(z, Bt, b_off + n * r, r, dtype) : base", "? base : base"),
    "silu_sign": ("return v / (1.0 + exp(-v));", "return v / (1.0 + exp(v));"),
    "gate_up_swapped": ("a[i] = silu(g[i]) * g[I + i];", "a[i] = silu(g[I + i]) * g[i];"),
    "tie_to_higher_id": ("rank_value(lg[e]) > rank_value(lg[best])", "rank_value(lg[e]) >= rank_value(lg[best])"),
    "nan_not_ranked_last": ("return isnan(v) ? -INFINITY : v;", "return v;"),
    "b_stride": ("b_off + n * r", "b_off + n"),
    "w_stride": ("w_off + n * K", "w_off + n"),
    "adapter_expert_index": ("(int64_t)(l < 0 ? 0 : l) * E + e;", "(int64_t)e * L + (l < 0 ? 0 : l);"),
    "no_renormalisation": ("topk_w[t * k + j] = ex[j] / sum;", "topk_w[t * k + j] = ex[j];"),
    "adapter_major_keys": ("(int64_t)topk_ids[s] * Lb + (l < 0 ? L : l)", "(int64_t)(l < 0 ? L : l) * E + topk_ids[s]"),
    "base_only_gets_adapter0_lora": ("le * 2 * I * r, dtype, l >= 0, z1, g);", "le * 2 * I * r, dtype, 1, z1, g);"),
    "base_only_bucket_first": ("topk_ids[s] * Lb + (l < 0 ? L : l)", "topk_ids[s] * Lb + (l < 0 ? 0 : l + 1)"),
    "dense_b_block_offset": ("Bt, lc * N * r, dtype", "Bt, lc * r * K, dtype"),
    "dense_x_row_stride": ("xin[k] = elem(x, t * K + k, dtype);", "xin[k] = elem(x, t + k * T, dtype);"),
    "combine_weight_dropped": ("o[n] += w * d[n];", "o[n] += d[n];"),
    "x_transposed": ("xin[i] = elem(x, t * h + i, dtype);", "xin[i] = elem(x, i * T + t, dtype);"),
    "down_uses_up_half": ("lora_projection(a, I, h, r, w_dn,", "lora_projection(g + I, I, h, r, w_dn,"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    old, new = MUTANTS[name]
    src = open(oracle._SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib = oracle.load_library(oracle.compile_source(path, os.path.join(d, "libmutant.so")))
        monkeypatch.setattr(oracle, "_lib", lib)
        caught = []
        for check in oracle_pins.ALL_CHECKS:
            try:
                check()
            except (AssertionError, ValueError):
                caught.append(check.__name__)
                break
        assert caught, f"no pin caught mutant {name}"
