"""The measurement probes behind kara_probe (include/kara.h): the copy probe
moves the bytes it claims, the loop probes report the work their launch
shapes imply and finish with finite results, and bad arguments are rejected
before anything is launched."""

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kara():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from decode_kv_cache_kara_amd import kara as k
    return k


def test_copy_probe_moves_bytes(kara):
    n = (1 << 20) + 48                      # not a multiple of one pass of the grid
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    work = kara.kara_probe(kara.KARA_PROBE_COPY, 1, dst, src=src)
    torch.cuda.synchronize()
    assert work == 2.0 * n
    assert torch.equal(dst, src)


@pytest.mark.parametrize("kind", [0, 1, 3])
def test_loop_probes(kara, kind):
    scratch = torch.full((kara.kara_probe_scratch_bytes() // 4,), float("nan"), device="cuda")
    iters = 7
    work = kara.kara_probe(kind, iters, scratch)
    torch.cuda.synchronize()
    n_threads = scratch.numel()             # one float per thread of the launch
    per_wave = {0: iters * 4 * 32768.0, 1: None, 3: iters * 2 * 2048.0}[kind]
    if kind == 1:
        assert work == n_threads * iters * 16.0
    else:
        assert work == (n_threads / 64) * per_wave
    assert torch.isfinite(scratch).all()


def test_probe_rejects_bad_arguments(kara):
    scratch = torch.empty(kara.kara_probe_scratch_bytes() // 4, device="cuda")
    with pytest.raises(kara.KaraError):
        kara.kara_probe(9, 1, scratch)
    with pytest.raises(kara.KaraError):
        kara.kara_probe(kara.KARA_PROBE_MFMA, 0, scratch)
    with pytest.raises(kara.KaraError):
        kara.kara_probe(kara.KARA_PROBE_MIX, 1, scratch[:16])
    with pytest.raises(ValueError):
        kara.kara_probe(kara.KARA_PROBE_COPY, 1, torch.zeros(64, dtype=torch.uint8, device="cuda"),
                        src=torch.zeros(32, dtype=torch.uint8, device="cuda"))
    odd = torch.zeros(17, dtype=torch.uint8, device="cuda")
    with pytest.raises(kara.KaraError):
        kara.kara_probe(kara.KARA_PROBE_COPY, 1, odd, src=odd.clone())


@pytest.mark.parametrize("D", [64, 128])
def test_paged_read_probe(kara, D):
    """The paged-read probe (decode attention's loads alone) runs over a
    fragmented cache with lengths around the split sizes, reports the K and V
    bytes of every cached token of the layer, leaves its 4-byte destination
    alone, and rejects a float32 shape before launching."""
    S, Lyr, Hq, Hkv, bs = 5, 2, 20, 4, 16
    lens = [1, 511, 512, 1025, 3000]
    nblk = [-(-L // bs) for L in lens]
    NB, MB = sum(nblk) + 3, max(nblk)
    g = torch.Generator().manual_seed(3)
    perm = torch.randperm(NB, generator=g).to(torch.int32)
    table = torch.full((S, MB), -1, dtype=torch.int32)
    cur = 0
    for b in range(S):
        table[b, :nblk[b]] = perm[cur:cur + nblk[b]]
        cur += nblk[b]
    pool = torch.randn((Lyr, 2, NB, Hkv, bs, D), device="cuda").to(torch.bfloat16)
    lens_h = torch.tensor(lens, dtype=torch.int32)
    dst = torch.zeros(1, dtype=torch.int32, device="cuda")
    shape = kara.kara_shape(Lyr, Hq, Hkv, D, bs, kara.dtype_code(torch.bfloat16))
    for layer in range(Lyr):
        nbytes = kara.kara_probe_paged_read(shape, layer, pool, table.cuda(), lens_h, lens_h.cuda(), dst)
        torch.cuda.synchronize()
        assert nbytes == sum(lens) * Hkv * 2 * D * 2
    assert int(dst.item()) == 0
    shape32 = kara.kara_shape(Lyr, Hq, Hkv, D, bs, kara.dtype_code(torch.float32))
    with pytest.raises(kara.KaraError) as e:
        kara.kara_probe_paged_read(shape32, 0, pool.float(), table.cuda(), lens_h, lens_h.cuda(), dst)
    assert e.value.status == kara.KARA_E_UNSUPPORTED


def test_read_and_write_probes(kara):
    """The read probe reads its buffer and leaves the sink alone; the write
    probe fills its buffer; both report their bytes."""
    n = (1 << 20) + 48
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert kara.kara_probe(kara.KARA_PROBE_READ, 1, sink, src=src) == float(n)
    dst = torch.zeros(n, dtype=torch.uint8, device="cuda")
    assert kara.kara_probe(kara.KARA_PROBE_WRITE, 1, dst) == float(n)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    assert int((dst.view(torch.int32)[2::4] == 0x5A5A5A5A).sum()) == n // 16   # every 16-byte piece written
