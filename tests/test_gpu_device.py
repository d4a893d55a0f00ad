"""The device query behind bench.py's run-time peak, on the GPU."""

import pytest
import torch

from exact_tiled_attention_attn_amd import attn

pytestmark = pytest.mark.gpu


def test_device_info_matches_torch_and_is_plausible():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    cus, clock_khz, mem_khz, bus_bits = attn.attn_device_info(0)
    print(f"device 0: {cus} CUs, {clock_khz / 1e3:.0f} MHz engine, {mem_khz / 1e3:.0f} MHz "
          f"memory, {bus_bits}-bit bus", flush=True)
    assert cus == torch.cuda.get_device_properties(0).multi_processor_count
    assert 500_000 <= clock_khz <= 5_000_000
    assert mem_khz > 0 and bus_bits > 0
    with pytest.raises(attn.AttnError):
        attn.attn_device_info(torch.cuda.device_count())
