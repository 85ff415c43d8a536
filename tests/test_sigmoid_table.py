"""The kernels' sigmoid table (gated_gqa_decode_amd/csrc/sigmoid_bf16_table.inc)
against its generator and against the oracle.

The generator evaluates sigmoid with 60-digit decimal arithmetic and rounds by
exact rational comparison; the oracle evaluates it in fp64 C and rounds the
fp64 value.  Two independent implementations agreeing on all 65,536 gates pin
both; the committed table must be exactly what the generator writes."""
import os
import sys

import numpy as np

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "gated_gqa_decode_amd", "csrc"))
import gen_sigmoid_table as gen  # noqa: E402


def test_committed_table_is_the_generators():
    with open(gen.OUT) as f:
        assert f.read() == gen.table_text()


def test_generator_agrees_with_the_oracle_on_every_gate():
    full = np.array(gen.full_table(), dtype=np.uint16)  # also checks the closed forms
    ref = oracle.sigmoid_table()
    nan = ((ref & 0x7F80) == 0x7F80) & ((ref & 0x7F) != 0)
    assert np.array_equal(full[~nan], ref[~nan])
    assert np.all(((full[nan] & 0x7F80) == 0x7F80) & ((full[nan] & 0x7F) != 0))


def test_closed_forms_at_the_table_edges():
    # just outside the table: |g| < 2^-9 gives 0.5, |g| >= 128 saturates
    assert gen.sigmoid_bf16_exact(0x3AFF) == 0x3F00      # 2^-9 * (1 - 2^-8)
    assert gen.sigmoid_bf16_exact(0xBAFF) == 0x3F00
    assert gen.sigmoid_bf16_exact(0x4300) == 0x3F80      # 128
    assert gen.sigmoid_bf16_exact(0xC300) == 0x0000      # -128
    assert gen.table_slot(0x3B00) == 0 and gen.table_slot(0xC2FF) == 4095
