"""Host-side logic of the binding, without a GPU: the decode exchange-tag
bookkeeping (tags are 32-bit; a workspace is zeroed again before the tags
used since it was last zeroed would pass 2^32 - 1)."""
import torch

import attention_spark_ffn_amd as sf


def test_decode_tags_per_call():
    # A, B and C exchanges per layer, no C after the last layer of a launch,
    # up to 32 layers per launch
    assert sf.decode_tags(26, 1) == 77
    assert sf.decode_tags(1, 5) == 10
    assert sf.decode_tags(32, 1) == 95
    assert sf.decode_tags(33, 1) == 97
    assert sf.decode_tags(64, 2) == 2 * (192 - 2)
    assert sf.decode_tags(26, 0) == 0
    assert sf.decode_tags(0, 1) == -1 and sf.decode_tags(3, -1) == -1


def test_decode_workspace_tag_wrap():
    ws = sf.DecodeWorkspace(torch.zeros(256, dtype=torch.uint8))
    assert not ws.reserve(77) and ws.tags_used == 77
    # the last call that still fits ends exactly at tag 2^32 - 1
    ws.tags_used = sf.TAG_LIMIT - 77
    assert not ws.reserve(77) and ws.tags_used == sf.TAG_LIMIT
    # the next one would wrap: the workspace is zeroed first and the count restarts
    assert ws.reserve(77) and ws.tags_used == 77
    ws.tags_used = sf.TAG_LIMIT - 76
    assert ws.reserve(77) and ws.tags_used == 77
    # at 77 tags per token a workspace serves 55.8 million tokens between zeroings
    assert sf.TAG_LIMIT // sf.decode_tags(26, 1) == 55_778_796
