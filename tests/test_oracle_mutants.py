"""Plant plausible mistakes in a copy of the oracle source (on the CPU) and check
that at least one pin catches each of them."""
import pytest

import oracle
import oracle_pins

# (name, text in oracle.c, replacement, how many occurrences to replace (0 = all))
MUTATIONS = [
    ("sink only seeds the max, never joins the denominator",
     "double z = (sink == -INFINITY) ? 0.0 : exp(sink - m);", "double z = 0.0;", 1),
    ("sink multiplied by sm_scale", "(double)sinks[h]", "sm_scale * (double)sinks[h]", 0),
    ("GQA head mapping h % Hkv", "int g = h / group;", "int g = h % hkv;", 0),
    ("causal mask top-left aligned", "int64_t n = lk - lq + i + 1;", "int64_t n = i + 1;", 1),
    ("causal mask excludes the diagonal", "int64_t n = lk - lq + i + 1;",
     "int64_t n = lk - lq + i;", 1),
    ("sink seeded in every block", "*m = first ? sink : -INFINITY;", "*m = sink;", 1),
    ("accumulator not rescaled", "acc[d] = alpha * acc[d] + p * (double)vj[d];",
     "acc[d] = acc[d] + p * (double)vj[d];", 1),
    ("running scale not rescaled", "*dsum = alpha * (*dsum) + p;", "*dsum = *dsum + p;", 1),
    ("combine without block weights", "double w = exp(ms[c] - big);", "double w = 1.0;", 1),
    ("lse without the max", "*lse = m + log(z);", "*lse = log(z);", 1),
    ("dropped term of the dot product", "acc += (double)q[d] * (double)k[d];",
     "if (d) acc += (double)q[d] * (double)k[d];", 1),
    ("K used in place of V", "const float *vbase = v + ((int64_t)cu_k[b] * hkv + g) * d_head;",
     "const float *vbase = k + ((int64_t)cu_k[b] * hkv + g) * d_head;", 1),
    ("output not normalised", "out[d] /= z;", "out[d] /= 1.0;", 1),
    ("sign of the max shift flipped", "double p = exp(scratch[j] - m);",
     "double p = exp(m - scratch[j]);", 1),
]


@pytest.mark.parametrize("name,old,new,count", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, count):
    src = open(oracle.SOURCE).read()
    assert old in src, f"mutation anchor not found: {old}"
    mutated = src.replace(old, new) if count == 0 else src.replace(old, new, count)
    orc = oracle.build_variant(mutated, str(tmp_path))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught: {name}"
