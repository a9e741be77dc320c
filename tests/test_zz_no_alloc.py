"""gs_loss_ssim_static, the entry point that allocates nothing, against
gs_loss_ssim through the C ABI: identical loss, SSIM and gradient on two
calls in a row (the second on a smaller image, so its buffers hold the first
call's values beyond its own extent), no allocator call, and the largest and
over-large sizes."""
import ctypes as C

import numpy as np
import pytest

from differentiable_gaussian_splatting_amd import binding as B

pytestmark = pytest.mark.gpu


class CountingContext(B.Context):
    """A context whose allocator (torch's caching allocator) counts its calls."""

    def __init__(self):
        import torch
        self.torch = torch
        self.lib = B.load()
        self.device = torch.device("cuda", torch.cuda.current_device())
        self.stream = torch.cuda.current_stream(self.device)
        self.calls = 0
        dev_index, raw = self.device.index, self.stream.cuda_stream

        def _alloc(user, nbytes, strm):
            self.calls += 1
            return torch.cuda.caching_allocator_alloc(int(nbytes), dev_index, strm if strm else raw)

        def _free(user, ptr, nbytes, strm):
            torch.cuda.caching_allocator_delete(ptr)

        self._alloc_cb, self._free_cb = B.ALLOC_FN(_alloc), B.FREE_FN(_free)
        h = C.c_void_p()
        self.check(self.lib.gs_ctx_create(C.byref(h), C.c_void_p(raw), self._alloc_cb, self._free_cb, None), ctx=None)
        self.handle = h


@pytest.fixture(scope="module")
def cctx():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    c = CountingContext()
    yield c
    c.close()


def _images(rng, h, w, dev):
    import torch
    img = torch.from_numpy(rng.random((3, h, w), dtype=np.float32)).to(dev)
    tgt = torch.from_numpy(rng.random((3, h, w), dtype=np.float32)).to(dev)
    return img, tgt


@pytest.mark.parametrize("shapes", [((1080, 1920), (300, 517)), ((257, 1031), (17, 33))])
def test_static_ssim_equals_allocating_ssim(cctx, shapes):
    import torch
    rng = np.random.default_rng(90)
    for k, (h, w) in enumerate(shapes):
        img, tgt = _images(rng, h, w, cctx.device)
        dl_ref = torch.empty_like(img)
        dl = torch.full_like(img, np.nan)
        ref = B.gs_loss_ssim(cctx, img, tgt, dl_ref, 0.2)
        n0 = cctx.calls
        got = B.gs_loss_ssim_static(cctx, img, tgt, dl, 0.2)
        torch.cuda.synchronize()
        assert cctx.calls == n0, "the static variant called the allocator"
        assert got == ref, (k, got, ref)
        assert torch.equal(dl, dl_ref), k
        # the gradient alone (no sums): asynchronous, same values
        dl2 = torch.full_like(img, np.nan)
        assert B.gs_loss_ssim_static(cctx, img, tgt, dl2, 0.2, sums=False) is None
        torch.cuda.synchronize()
        assert cctx.calls == n0
        assert torch.equal(dl2, dl_ref), k


def test_static_ssim_size_limits(cctx):
    import torch
    rng = np.random.default_rng(91)
    # 2^21 pixels in a 32-pixel-wide column
    img, tgt = _images(rng, 1 << 16, 32, cctx.device)
    dl_ref, dl = torch.empty_like(img), torch.empty_like(img)
    ref = B.gs_loss_ssim(cctx, img, tgt, dl_ref, 0.2)
    got = B.gs_loss_ssim_static(cctx, img, tgt, dl, 0.2)
    assert got == ref and torch.equal(dl, dl_ref)
    del img, tgt, dl_ref, dl
    big, bt = _images(rng, 1081, 1940, cctx.device)   # 2,097,140 pixels: fits
    d = torch.empty_like(big)
    assert B.gs_loss_ssim_static(cctx, big, bt, d, 0.2) == B.gs_loss_ssim(cctx, big, bt, torch.empty_like(big), 0.2)
    over, ot = _images(rng, 1082, 1940, cctx.device)   # 2,099,080 pixels: over the limit
    with pytest.raises(B.GsError) as e:
        B.gs_loss_ssim_static(cctx, over, ot, torch.empty_like(over), 0.2)
    assert e.value.status == B.GS_ERR_OVERFLOW
    with pytest.raises(B.GsError) as e:
        B.gs_loss_ssim_static(cctx, over[:, :0], ot[:, :0], over[:, :0], 0.2)
    assert e.value.status == B.GS_ERR_INVALID_ARG
