"""The input harness (CPU): every workload's slot mapping gives each token its
own slot, and the uniqueness check catches a repeated slot."""

import numpy as np
import pytest

from packed_cache_decode_amd import synth


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_workload_slot_mappings_are_unique(name):
    inp = synth.generate(synth.WORKLOADS[name], with_kv=False)
    sm = inp.slot_mapping
    synth.assert_unique_slots(sm)
    assert sm.shape[0] == int(inp.seq_lens.sum())
    assert sm.min() >= 0 and sm.max() < inp.num_blocks * synth.WORKLOADS[name].block_size


def test_duplicate_slots_are_rejected_and_padding_may_repeat():
    synth.assert_unique_slots(np.array([5, -1, 7, -1, 0], np.int64))
    synth.assert_unique_slots(np.zeros(0, np.int64))
    with pytest.raises(ValueError, match="duplicate"):
        synth.assert_unique_slots(np.array([3, 9, 4, 9], np.int64))
