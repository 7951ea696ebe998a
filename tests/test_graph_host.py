"""Host logic of the decode-graph helper (no GPU): the bucket list and the
bucket choice follow the capture scheme of the "nano-vLLM learning note"
(ModelRunner.capture_cudagraph: 1, 2, 4, 8, then steps of 16 up to 512)."""

import pytest

from paged_kv_attention_16_amd.graph import DEFAULT_BUCKETS, bucket_for


def test_bucket_list():
    assert DEFAULT_BUCKETS[:5] == (1, 2, 4, 8, 16)
    assert DEFAULT_BUCKETS[-1] == 512
    assert all(b % 16 == 0 for b in DEFAULT_BUCKETS[4:])
    assert list(DEFAULT_BUCKETS) == sorted(set(DEFAULT_BUCKETS))


@pytest.mark.parametrize("batch,bucket", [(1, 1), (3, 4), (8, 8), (9, 16), (17, 32), (255, 256),
                                          (500, 512), (512, 512)])
def test_bucket_for(batch, bucket):
    assert bucket_for(batch) == bucket


def test_bucket_overflow():
    with pytest.raises(ValueError):
        bucket_for(513)
