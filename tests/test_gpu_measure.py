"""The streaming-read calibration reads every word once (its XOR fold proves it)."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words,groups", [(4, 1), (4096 + 4, 7), (1 << 20, 0), (3 * (1 << 18) + 12, 300)])
def test_stream_read_folds_every_word(words, groups):
    from paged_kv_decode_07_amd import binding as pa
    rng = np.random.default_rng(words + groups)
    host = rng.integers(0, 2**32, size=words, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(65536, dtype=torch.int32, device="cuda")
    pa.stream_read(buf, sink, groups=groups)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


# The page stream reads, for every sequence, KV head and half, exactly the head's
# blocks of the pages its block table names (an id outside the pool reads page 0;
# a length outside [0, 16 * max_blocks] reads nothing): each wavefront's XOR fold
# is checked against the same fold over the host copy of those blocks.
NP_, MB = 1536, 256                    # pool pages; block-table row (the 4096-token window)
LENS = [0, 1, 15, 16, 17, 33, 300, 2047, 2048, 4096, 4097, -1, 129]


def _stream_inputs(fmt, seed):
    rng = np.random.default_rng(seed)
    words = {0: 16 * 8 * 64 // 2, 1: 8 * 16 * 64 // 4, 2: 8 * 16 * 32 // 4}[fmt]
    k = rng.integers(0, 2**32, size=NP_ * words, dtype=np.uint32)
    v = rng.integers(0, 2**32, size=NP_ * words, dtype=np.uint32)
    s = rng.integers(0, 2**32, size=NP_ * 8 * 2 * 16, dtype=np.uint32) if fmt else None
    tables = rng.integers(0, NP_, size=(len(LENS), MB)).astype(np.int32)
    tables[6, 3] = -5                   # inside sequence 6's 19 pages: reads page 0
    tables[12, 8] = NP_ + 7             # inside sequence 12's 9 pages: reads page 0
    return k, v, s, tables, np.array(LENS, np.int32)


def _host_blocks(fmt, k, v, s):
    """[pages][8 heads][words] of everything a head's wavefront folds from a page."""
    if fmt == 0:       # token-major BF16 rows: head g's 16 rows of 64 dims, K then V
        kk = k.view(np.uint16).reshape(NP_, 16, 8, 64).transpose(0, 2, 1, 3)
        vv = v.view(np.uint16).reshape(NP_, 16, 8, 64).transpose(0, 2, 1, 3)
        kk = np.ascontiguousarray(kk).reshape(NP_, 8, -1).view(np.uint32)
        vv = np.ascontiguousarray(vv).reshape(NP_, 8, -1).view(np.uint32)
        return np.concatenate([kk, vv], axis=2)
    kk, vv = k.reshape(NP_, 8, -1), v.reshape(NP_, 8, -1)
    return np.concatenate([kk, vv, s.reshape(NP_, 8, 32)], axis=2)


def _expected_folds(blocks, tables, lens, wph):
    per_word = np.bitwise_xor.reduce(blocks, axis=2)          # [pages][8]
    out = np.zeros((len(lens), 8 * wph), np.uint32)
    for b, L in enumerate(lens):
        n = -(-int(L) // 16) if 0 <= L <= 16 * MB else 0
        ids = np.where((tables[b, :n] >= 0) & (tables[b, :n] < NP_), tables[b, :n], 0)
        for g in range(8):
            for h in range(wph):
                sel = ids[n * h // wph: n * (h + 1) // wph]
                out[b, g * wph + h] = np.bitwise_xor.reduce(per_word[sel, g]) if len(sel) else 0
    return out


# every (format, wavefronts per head, ring) whose rings fit the LDS; BF16 pages with
# two wavefronts per head and three slots (192 KiB) are refused (test_abi_cpu.py)
STREAM_CASES = [(f, w, r) for f in (0, 1, 2) for w in (1, 2) for r in (1, 2, 3)
                if (f, w, r) != (0, 2, 3)]


@pytest.mark.parametrize("fmt,wph,ring", STREAM_CASES)
def test_page_stream_folds_each_heads_blocks(fmt, wph, ring):
    from paged_kv_decode_07_amd import binding as pa
    k, v, s, tables, lens = _stream_inputs(fmt, 100 + fmt)
    if fmt == 0:
        kd = torch.from_numpy(k.view(np.int16).reshape(NP_, 16, 8, 64)).cuda()
        vd = torch.from_numpy(v.view(np.int16).reshape(NP_, 16, 8, 64)).cuda()
        sd = None
    else:
        dt, w = (np.int8, 64) if fmt == 1 else (np.uint8, 32)
        kd = torch.from_numpy(k.view(dt).reshape(NP_, 8, 16, w)).cuda()
        vd = torch.from_numpy(v.view(dt).reshape(NP_, 8, 16, w)).cuda()
        sd = torch.from_numpy(s.view(np.float32).reshape(NP_, 8, 2, 16)).cuda()
    sink = pa.page_stream(kd, vd, sd, torch.from_numpy(tables).cuda(),
                          torch.from_numpy(lens).cuda(), waves_per_head=wph, ring=ring)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    want = _expected_folds(_host_blocks(fmt, k, v, s), tables, lens, wph)
    bad = np.argwhere(got != want)
    assert len(bad) == 0, f"first mismatching (sequence, wavefront): {bad[:4].tolist()}"
