"""Host-side arithmetic of the benchmark (no GPU): the read-ceiling probe's regions.

The probe reads `nbytes` at region offsets inside one device buffer; every region it
rotates over must end inside the buffer (a read past its end faults the GPU), and a read
larger than the buffer must be refused on the host.
"""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

MiB = 1024 * 1024


def buffer_total(max_bytes):
    region = (max_bytes + 4095) // 4096 * 4096
    return max(bench.ROTATION_BYTES + region, 2 * region)


@pytest.mark.parametrize("max_mib", [300, 440])
@pytest.mark.parametrize("nbytes", [1, 9_453_568, 66_125_824, 295_766_528, 361_400_000, 394_002_432 + 32_833_536,
                                    427_000_000, 470_000_000])
def test_ceiling_regions_stay_inside_the_buffer(max_mib, nbytes):
    total = buffer_total(max_mib * MiB)
    if (nbytes + 4095) // 4096 * 4096 > total:
        with pytest.raises(ValueError):
            bench.ReadCeiling.regions(total, nbytes)
        return
    read, region, regions = bench.ReadCeiling.regions(total, nbytes)
    assert read >= nbytes and region >= read
    assert regions >= 1
    assert (regions - 1) * region + read <= total  # the last region's read ends inside the buffer


def test_the_six_bit_lm_head_read_that_once_overran():
    """A 300 MiB probe buffer (812 MiB in all) holds one region of the 6-bit lm_head read
    (427 MB), not the two the old rule forced; the bits workload sizes its buffer for it."""
    nbytes = 128256 * 4096 * 6 // 8 + 4 * 128256 * 4096 // 64 + 2 * 4096 + 2 * 128256
    _, region, regions = bench.ReadCeiling.regions(buffer_total(300 * MiB), nbytes)
    assert regions == 1
    _, region, regions = bench.ReadCeiling.regions(buffer_total(440 * MiB), nbytes)
    assert regions == 2 and 2 * region <= buffer_total(440 * MiB)
