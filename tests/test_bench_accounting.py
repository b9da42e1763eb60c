"""The benchmark's closed-form visible-pair counts equal the oracle's dense
masks (CPU)."""

import numpy as np
import pytest

import bench
import synth
from oracle import masks


def _count(lay):
    return sum(int(masks.visible_for_layout(lay, s).sum()) for s in range(lay.n_seqs))


@pytest.mark.parametrize("lay", [
    synth.causal_single(37, 1, 8),
    synth.packed_documents(seed=3, n_docs=4, lo=3, hi=90, H=1, D=8),
    synth.shared_prefix(prefix=13, n_suffix=3, suffix=7, H=1, D=8),
    synth.strip_thinking(n_turns=3, user=2, think=5, answer=3, H=1, D=8),
    synth.strip_thinking_duplicated(n_turns=3, user=2, think=5, answer=3, H=1, D=8),
    synth.strip_thinking_duplicated(n_turns=4, user=1, think=0, answer=2, H=1, D=8),
    synth.shared_prefix_groups(n_groups=3, prefix=5, n_suffix=2, suffix=4, pad=3, H=1, D=8),
    synth.paged_decode(seed=1, n_seqs=5, lo=3, hi=50, H=1, D=8),
    synth.Layout("x", "causal", "f32", 1, 8, [3, 5, 1], [7, 5, 2]),
    synth.prefix_lm(prefixes=(0, 4, 9, 30), lengths=(5, 17, 9, 12), H=1, D=8),
])
def test_closed_forms_match_oracle_small(lay):
    assert bench.visible_pairs(lay) == _count(lay)


def test_closed_forms_named_workloads():
    assert bench.visible_pairs(synth.config("causal_f32")) == 256 * 257 // 2
    lay = synth.config("strip_thinking")
    assert bench.visible_pairs(lay) == _count(lay) == 70788096
    lay = synth.config("shared_prefix")
    assert bench.visible_pairs(lay) == 83896320
    lay = synth.config("packed_documents")
    assert bench.visible_pairs(lay) == _count(lay)


def test_closed_form_duplicated_answers_full_size():
    lay = synth.config("strip_thinking_duplicated")
    assert bench.visible_pairs(lay) == _count(lay)


def test_closed_form_shared_prefix_groups_full_size():
    lay = synth.config("shared_prefix_groups")
    assert bench.visible_pairs(lay) == _count(lay)


def test_closed_form_prefix_lm_full_size():
    lay = synth.config("prefix_lm")
    assert bench.visible_pairs(lay) == _count(lay)
