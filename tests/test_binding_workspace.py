"""Host-side checks of the binding's default workspaces (no GPU): calls on
different streams of one device never share a workspace, and growing one
stream's workspace leaves the others alone."""
import torch

import moe_expert_routing_amd as M


def test_two_streams_get_distinct_workspaces(monkeypatch):
    monkeypatch.setattr(M, "_WORKSPACES", {})
    monkeypatch.setattr(M, "_new_workspace",
                        lambda n, dev: torch.zeros(n, dtype=torch.uint8))
    dev = torch.device("cuda", 0)
    a = M.workspace(dev, 1000, stream=0x1000)
    b = M.workspace(dev, 1000, stream=0x2000)
    assert a is not b and a.data_ptr() != b.data_ptr()
    # the same stream gets its cached buffer back
    assert M.workspace(dev, 500, stream=0x1000) is a
    assert M.cached_workspace(dev, stream=0x2000) is b
    # growth replaces only that stream's buffer
    big = M.workspace(dev, 1 << 20, stream=0x1000)
    assert big is not a and big.numel() >= 1 << 20
    assert M.workspace(dev, 1000, stream=0x2000) is b
    # another device with the same stream value is another key
    c = M.workspace(torch.device("cuda", 1), 1000, stream=0x2000)
    assert c is not b
    assert M.cached_workspace(dev, stream=0x3000) is None
