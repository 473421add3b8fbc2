"""The streaming probe through the C ABI: the copy moves every byte, the read leaves its
destination alone (but for at most one word), and bad arguments are refused on the host."""
import pytest
import torch

from linear_attention_beam_amd import binding as B

pytestmark = pytest.mark.gpu


def test_stream_probe_copy_and_read():
    g = torch.Generator(device="cuda").manual_seed(7)
    n = (48 << 20) + 4096                          # not a multiple of the grid's stride
    src = torch.randint(0, 2 ** 31 - 1, (n // 4,), generator=g, device="cuda", dtype=torch.int32)
    dst = torch.zeros_like(src)
    B.gdn_beam_stream_probe(dst, src, n, 0)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    # a shorter copy touches only its bytes
    dst.zero_()
    B.gdn_beam_stream_probe(dst, src, 4096, 0)
    torch.cuda.synchronize()
    assert torch.equal(dst[:1024], src[:1024]) and int(dst[1024:].abs().sum()) == 0
    # the read: at most the first word of its destination
    sink = torch.full((1024,), 5, device="cuda", dtype=torch.int32)
    B.gdn_beam_stream_probe(sink, src, n, 1)
    torch.cuda.synchronize()
    assert bool((sink[1:] == 5).all())


def test_stream_probe_write_pattern():
    """The write covers whole groups of 32 rows of 512 bytes and nothing past them."""
    rows = 3 * 32 + 5                               # a partial group at the end
    dst = torch.zeros(rows * 128, device="cuda", dtype=torch.float32)
    B.gdn_beam_stream_probe(dst, None, rows * 512, 2)
    torch.cuda.synchronize()
    assert bool((dst[:96 * 128] == 1.0).all()) and bool((dst[96 * 128:] == 0.0).all())


def test_stream_probe_refuses_bad_arguments():
    x = torch.zeros(1024, device="cuda", dtype=torch.int32)
    for args in ((x, x[1:], 64, 0),               # misaligned source
                 (x, x, 60, 0),                   # not a multiple of 16 bytes
                 (x, x, 64, 3),                   # no such mode
                 (None, x, 64, 1)):
        with pytest.raises(B.GdnBeamError) as e:
            B.gdn_beam_stream_probe(*args)
        assert e.value.status == B.GDN_ERR_INVALID_ARG
    B.gdn_beam_stream_probe(x, x, 0, 0)           # nothing to move
