"""Helpers shared by the GPU tests (no arithmetic of the method here)."""
import numpy as np
import torch

import rotated_w4a8_group_amd as pq
import synth

SENT_U8 = 0xA5
SENT_F32 = np.uint32(0x7FC0DEAD)   # a NaN payload the kernels never write
SENT_BF16 = 0x7FC1


def dev():
    return torch.device("cuda:0")


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def records_for(pairs_l, theta_l):
    return np.stack([pq.build_records(p, t) for p, t in zip(pairs_l, theta_l)])


def guarded(shape, dtype, fill, guard=4096):
    """A contiguous tensor view of `shape` at the front of a larger sentinel-filled buffer;
    returns (view, whole buffer, number of view elements)."""
    n = int(np.prod(shape))
    buf = torch.empty(n + guard, dtype=dtype, device=dev())
    if dtype == torch.float32:
        buf.view(torch.int32).fill_(int(SENT_F32.view(np.int32)))
    elif dtype == torch.uint8:
        buf.fill_(SENT_U8)
    else:
        buf.view(torch.int16).fill_(SENT_BF16)
    return buf[:n].view(shape), buf, n


def prologue_gpu(wl, x, pairs_l, theta_l, cs_l, guard=True):
    rec = to_dev(records_for(pairs_l, theta_l))
    cs = to_dev(np.stack(cs_l))
    xd = to_dev(x)
    P, M, K, G = wl.P, x.shape[0], wl.K, wl.K // 128
    if guard:
        A, Ab, nA = guarded((P, M, K), torch.uint8, SENT_U8)
        S, Sb, nS = guarded((P, M, G), torch.float32, None)
        R, Rb, nR = guarded((P, M, G), torch.float32, None)
        pq.rotate_quant(xd, rec, cs, out=(A, S, R))
        torch.cuda.synchronize()
        assert torch.all(Ab[nA:] == SENT_U8)
        assert torch.all(Sb[nS:].view(torch.int32) == int(SENT_F32.view(np.int32)))
        assert torch.all(Rb[nR:].view(torch.int32) == int(SENT_F32.view(np.int32)))
        return A, S, R
    out = pq.rotate_quant(xd, rec, cs)
    torch.cuda.synchronize()
    return out


def packed_weights(w):
    return pq.pack_weights(to_dev(w.qweight), to_dev(w.qzeros), to_dev(w.scales))


def bf16_to_f64(t):
    return t.float().double().cpu().numpy()
