"""The slot ring with its HSA copy engine on the GPU (copies on chosen copy engines, ordered by
host threads): every byte a kernel reads from a slot is the layer last loaded into it, and every
gradient a kernel wrote lands in host memory, over repeated sliding sweeps whose slots are small
enough (1 MiB) to stay in the L2 caches between uses, with new contents every sweep, so a stale
cache line or a copy ordered wrongly against the kernels would show."""
import numpy as np
import pytest
import torch

import layer_sliding_offloaded_fwd_amd as sl

pytestmark = pytest.mark.gpu


def test_hsa_ring_sweeps_read_fresh_weights_and_land_gradients():
    n_slots, wb, gb, L, sweeps = 3, 1 << 20, 1 << 20, 8, 6
    print(f"hsa ring: {n_slots} slots of {wb} + {gb} bytes, {L} layers, {sweeps} sweeps",
          flush=True)
    dev = torch.empty(n_slots * (wb + gb), dtype=torch.uint8, device="cuda:0")
    c = torch.cuda.Stream()
    ring = sl.SlotRing(n_slots, wb, gb, dev, engine=sl.SLIDE_ENGINE_HSA)
    rng = np.random.default_rng(5)
    host_w = [torch.empty(wb, dtype=torch.uint8, pin_memory=True) for _ in range(L)]
    host_g = [torch.empty(gb, dtype=torch.uint8, pin_memory=True) for _ in range(L)]
    seen_f = torch.empty((L, wb // 4), dtype=torch.int32, device="cuda:0")
    seen_b = torch.empty((L, wb // 4), dtype=torch.int32, device="cuda:0")
    base = dev.data_ptr()

    def view(ptr, n):
        off = ptr - base
        return dev[off:off + n].view(torch.int32)

    try:
        for sweep in range(sweeps):
            for i in range(L):
                host_w[i].copy_(torch.from_numpy(rng.integers(0, 256, wb, dtype=np.uint8)))
            loaded = {i: ring.load(i, host_w[i]) for i in range(n_slots)}
            for i in range(L):                      # forward: a kernel reads the weights
                s = loaded.pop(i)
                w, _ = ring.acquire(s, c)
                with torch.cuda.stream(c):
                    torch.add(view(w, wb), 0, out=seen_f[i])
                ring.release(s, c)
                if i + n_slots < L:
                    loaded[i + n_slots] = ring.load(i + n_slots, host_w[i + n_slots])
            for i in range(L - 1, L - 1 - n_slots, -1):
                loaded[i] = ring.reuse(i)
            tickets = []
            for i in range(L - 1, -1, -1):          # backward: read again, write gradients
                s = loaded.pop(i)
                w, g = ring.acquire(s, c)
                with torch.cuda.stream(c):
                    torch.add(view(w, wb), 0, out=seen_b[i])
                    view(g, gb).fill_(1000 * sweep + i + 1)
                tickets.append((i, ring.flush(s, host_g[i], c)))
                ring.release(s, c)
                if i - n_slots >= 0:
                    loaded[i - n_slots] = ring.load(i - n_slots, host_w[i - n_slots])
            c.synchronize()
            for i, t in tickets:
                ring.wait_flush(t, 60000)
                assert ring.ticket_time(t) > 0
                assert torch.all(host_g[i].view(torch.int32) == 1000 * sweep + i + 1), \
                    f"sweep {sweep}: gradient of layer {i}"
            f, b = seen_f.cpu(), seen_b.cpu()
            for i in range(L):
                ref = host_w[i].view(torch.int32)
                assert torch.equal(f[i], ref), f"sweep {sweep}: forward read of layer {i}"
                assert torch.equal(b[i], ref), f"sweep {sweep}: backward read of layer {i}"
    finally:
        ring.close()
