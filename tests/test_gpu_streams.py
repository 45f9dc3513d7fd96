"""The entry points run in order on the caller's stream (torch's current stream, passed
through the C ABI), not on the null stream.

Each case makes a side stream spin for ~0.2 s (torch.cuda._sleep), then writes the
call's input on that stream and calls the entry point under it.  A launch on any other
stream would read the input before the write lands; on the caller's stream it must see
the written input, and its result must still be pending when the host returns (the
spin is still running).  The result is then compared bit for bit with the same call
made on the default stream with nothing pending.
"""
import pytest
import torch

import long_sequence_attention_rope3d_amd as r3d

pytestmark = pytest.mark.gpu

SPIN = 400_000_000  # shader clock cycles: ~0.2 s, far longer than the host needs to enqueue and query


def _rand(shape, seed, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype)


def test_attn_fwd_runs_on_the_current_stream(gpu):
    q, k, v = (_rand((1, 3, 700, 128), s).to(gpu) for s in (1, 2, 3))
    want, want_lse = r3d.attn_fwd(q, k, v, kv_chunk=256)
    torch.cuda.synchronize()
    q_in = torch.zeros_like(q)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        torch.cuda._sleep(SPIN)
        q_in.copy_(q)
        out, lse = r3d.attn_fwd(q_in, k, v, kv_chunk=256)
    assert not side.query(), "the call's work should still be queued behind the spin"
    side.synchronize()
    assert torch.equal(out, want) and torch.equal(lse, want_lse)


def test_joint_concat_permute_runs_on_the_current_stream(gpu):
    segs = [_rand((1, n, 4, 128), 10 + i).to(gpu) for i, n in enumerate((24, 7))]
    rope = r3d.Rope3D((2, 3, 4), (32, 48, 48))
    want = r3d.joint_concat_permute(segs, rope)
    torch.cuda.synchronize()
    seg0 = torch.zeros_like(segs[0])
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        torch.cuda._sleep(SPIN)
        seg0.copy_(segs[0])
        out = r3d.joint_concat_permute([seg0, segs[1]], rope)
    assert not side.query()
    side.synchronize()
    assert torch.equal(out, want)


def test_lse_merge_runs_on_the_current_stream(gpu):
    parts = _rand((3, 1, 2, 300, 64), 20, torch.float32).to(gpu)
    lses = _rand((3, 1, 2, 300), 21, torch.float32).to(gpu)
    want, want_lse = r3d.lse_merge(parts, lses)
    torch.cuda.synchronize()
    parts_in = torch.zeros_like(parts)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        torch.cuda._sleep(SPIN)
        parts_in.copy_(parts)
        out, lse = r3d.lse_merge(parts_in, lses)
    assert not side.query()
    side.synchronize()
    assert torch.equal(out, want) and torch.equal(lse, want_lse)


def test_attn_fwd_from_two_host_threads(gpu):
    """Two host threads each issue attn_fwd calls on their own stream with their own
    workspace and buffers (the library keeps no per-call state between calls; its error
    text is per thread): every result equals the single-threaded call, bit for bit, and
    a call that fails in one thread leaves the other thread's error text alone."""
    import threading
    shapes = [(1, 24, 4352, 128, 0), (1, 4, 300, 128, 1024)]   # a split 12-wave grid; an 8-wave split grid
    cases = []
    for i, (B, H, S, D, ch) in enumerate(shapes):
        q, k, v = (_rand((B, H, S if j == 0 else S + 700 * i, D), 30 + 3 * i + j).to(gpu) for j in range(3))
        want = r3d.attn_fwd(q, k, v, kv_chunk=ch)
        cases.append((q, k, v, ch, want))
    torch.cuda.synchronize()
    errors, msgs = [], {}

    def worker(idx):
        try:
            q, k, v, ch, (want_o, want_l) = cases[idx]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                ws = torch.empty(r3d.attn_fwd_workspace_size(*q.shape[:3], k.shape[2], q.shape[3], ch,
                                                             torch.bfloat16), dtype=torch.uint8, device=gpu)
                for _ in range(5):
                    o, l = r3d.attn_fwd(q, k, v, kv_chunk=ch, workspace=ws)
                    s.synchronize()
                    if not (torch.equal(o, want_o) and torch.equal(l, want_l)):
                        errors.append(f"thread {idx}: result differs")
                if idx == 0:
                    try:
                        r3d.attn_fwd(q, k, v, kv_chunk=-1)
                    except ValueError as e:
                        msgs[idx] = str(e)
                else:
                    msgs[idx] = r3d._lib.r3d_last_error().decode()
        except Exception as e:  # noqa: BLE001 (reported below)
            errors.append(f"thread {idx}: {e!r}")

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in ts), "a worker thread did not finish"
    assert not errors, errors
    assert "kv_chunk" in msgs[0] and msgs[1] == ""
