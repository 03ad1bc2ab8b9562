"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is a copy of oracle.c with one plausible error (a dropped term, a
wrong sign or index, a swapped operand), compiled on the CPU into a temporary
library.  The pin battery of test_oracle_pins.py runs against it and at least
one pin has to fail.  The real oracle is never modified.
"""
import os

import pytest

import oracle
from oracle import build as obuild
from tests import test_oracle_pins as pins

# (name, text in oracle.c, replacement); each text must occur in the source.
MUTANTS = [
    ("wrong row in block", "int32_t row = j % block_size;",
     "int32_t row = (j + 1) % block_size;"),
    ("wrong logical block", "int32_t logical_block = j / block_size;",
     "int32_t logical_block = (j / block_size) / 2;"),
    ("GQA by modulo", "&s, h / group,", "&s, h % Hkv,"),
    ("scale dropped", "score[j] = scale * dot;", "score[j] = dot;"),
    ("no max subtraction", "score[j] = exp(score[j] - m);", "score[j] = exp(score[j]);"),
    ("sign flipped in exp", "score[j] = exp(score[j] - m);", "score[j] = exp(m - score[j]);"),
    ("not normalised", "double p = score[j] / l;", "double p = score[j];"),
    ("causal excludes diagonal", "pos + 1, scale);", "pos, scale);"),
    ("prefill ignores history", "int32_t pos = context_lens[b] - q_len + (t - cu_q_lens[b]);",
     "int32_t pos = (t - cu_q_lens[b]);"),
    ("append order reversed", "int32_t pos = context_lens[b] - n + t;",
     "int32_t pos = context_lens[b] - 1 - t;"),
    ("append heads swapped", "long src = ((long)(first + t) * Hkv + h) * D;",
     "long src = ((long)(first + t) * Hkv + (Hkv - 1 - h)) * D;"),
    ("merge drops l_p", "double w = lp * exp(m[(long)r * P + p] - M);",
     "double w = exp(m[(long)r * P + p] - M);"),
    ("V used as K", "dot += widen_bf16(q[d]) * widen_bf16(s->k_cache[off + d]);",
     "dot += widen_bf16(q[d]) * widen_bf16(s->v_cache[off + d]);"),
    ("K used as V", "out[d] += p * widen_bf16(s->v_cache[off + d]);",
     "out[d] += p * widen_bf16(s->k_cache[off + d]);"),
    ("bf16 widened wrongly", "uint32_t u = (uint32_t)bits << 16;",
     "uint32_t u = (uint32_t)bits << 15;"),
    ("online never rescales", "double alpha = exp(m - m_new); /* 0 on the first key */",
     "double alpha = 1.0;"),
    ("partition drops a key", "int32_t j1 = j0 + partition_size;",
     "int32_t j1 = j0 + partition_size - 1;"),
    ("head offset transposed", "return (((long)phys * Hkv + g) * block_size + row) * (long)D;",
     "return (((long)phys * Hkv + (Hkv - 1 - g)) * block_size + row) * (long)D;"),
    ("rope sign flipped", "dst[i] = a * c - b * s;", "dst[i] = a * c + b * s;"),
    ("rope cos and sin swapped", "double c = (double)cr[i], s = (double)sr[i];",
     "double c = (double)sr[i], s = (double)cr[i];"),
    ("rope table columns reversed", "double c = (double)cr[i], s = (double)sr[i];",
     "double c = (double)cr[half - 1 - i], s = (double)sr[half - 1 - i];"),
    ("rope pairs adjacent elements", "double a = widen_bf16(src[i]), b = widen_bf16(src[i + half]);",
     "double a = widen_bf16(src[i]), b = widen_bf16(src[i ^ 1]);"),
    ("rope position off by one", "pos[first + t] = context_lens[b] - n + t;",
     "pos[first + t] = context_lens[b] - n + t + 1;"),
    ("bf16 rounding through float", "double a = fabs(v);", "double a = fabs((double)(float)v);"),
    ("bf16 rounding truncates", "r = ldexp(nearbyint(ldexp(m, 8)), e - 8);",
     "r = ldexp(floor(ldexp(m, 8)), e - 8);"),
    ("block copy reversed", "memcpy(k_cache + dst[i] * per_block, k_cache + src[i] * per_block,",
     "memcpy(k_cache + src[i] * per_block, k_cache + dst[i] * per_block,"),
    ("block copy skips V", "memcpy(v_cache + dst[i] * per_block, v_cache + src[i] * per_block,",
     "memcpy(v_cache + dst[i] * per_block, v_cache + dst[i] * per_block,"),
]


def run_battery(orc, golden):
    """Returns the name of the first failing pin, or None if all pass."""
    for pin in pins.PINS:
        try:
            if pin in pins.NEEDS_GOLDEN:
                pin(orc, golden)
            else:
                pin(orc)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            return pin.__name__
    return None


def test_unmutated_source_passes(golden):
    assert run_battery(oracle.default(), golden) is None


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, golden, tmp_path):
    src = open(obuild.SRC).read()
    assert src.count(old) >= 1, f"mutation site missing: {old}"
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = obuild.compile_source(str(mutated), str(tmp_path / f"libmut_{abs(hash(name))}.so"))
    caught = run_battery(oracle.Oracle(lib), golden)
    assert caught is not None, f"planted mistake '{name}' passed every pin"
    os.remove(lib)
