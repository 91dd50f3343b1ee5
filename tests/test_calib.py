"""The synthetic loops of fa_calib.h (a measurement aid): every matrix-core mix and every LDS
read pattern launches, and two launches with the same data agree bit for bit (the matrix-core
checksums are also finite)."""
import pytest

pytestmark = pytest.mark.gpu


def test_every_mix_runs_and_repeats():
    import torch

    import io_aware_tiled_03_amd as fa
    g = torch.Generator().manual_seed(11)
    seed = (torch.randn(fa.CALIB_SEED_BYTES // 2, generator=g) * 0.5).to(torch.bfloat16).cuda()
    grid, iters = 8, 6
    for mix, name in enumerate(fa.calib_mixes()):
        print("calib mix", mix, name, flush=True)
        a = fa.calib_mfma(mix, grid, iters, seed, torch.empty(grid * 256, device="cuda"))
        b = fa.calib_mfma(mix, grid, iters, seed, torch.empty(grid * 256, device="cuda"))
        torch.cuda.synchronize()
        assert torch.isfinite(a).all(), name
        assert torch.equal(a, b), name
        assert fa.calib_flops(mix, grid, iters) > 0


def test_every_lds_pattern_runs_and_repeats():
    import torch

    import io_aware_tiled_03_amd as fa
    grid, iters = 4, 3
    for pat, name in enumerate(fa.calib_lds_patterns()):
        print("calib lds pattern", pat, name, flush=True)
        a = fa.calib_lds(pat, grid, iters, torch.empty(grid * 512, dtype=torch.int32, device="cuda"))
        b = fa.calib_lds(pat, grid, iters, torch.empty(grid * 512, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        assert torch.equal(a, b), name
        assert fa.calib_lds_bytes(pat, grid, iters) > 0


def test_hbm_read_checksum():
    """The streaming read folds every chunk once: workgroup b reads chunks [b*per, (b+1)*per)
    (per = ceil(chunks / grid)), its lane t the chunks t, t + 256, ... of that range, and the lane's
    checksum is the sum of their four-word XORs, which the test recomputes on the host."""
    import torch

    import io_aware_tiled_03_amd as fa
    g = torch.Generator().manual_seed(5)
    host = torch.randint(0, 2 ** 31 - 1, (1000 * 4 + 36,), generator=g, dtype=torch.int64)
    words = host.to(torch.int32)
    grid = 3
    out = fa.calib_hbm_read(words.cuda(), grid, torch.empty(grid * 256, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    w = words.numpy().astype("uint32").reshape(-1, 4)
    x = w[:, 0] ^ w[:, 1] ^ w[:, 2] ^ w[:, 3]
    per = -(-len(x) // grid)
    want = [int(x[b * per:min((b + 1) * per, len(x))][t::256].astype("uint64").sum() % 2 ** 32)
            for b in range(grid) for t in range(256)]
    got = (out.cpu().numpy().astype("int64") % 2 ** 32).tolist()
    assert got == want


def test_binding_rejects_short_buffers():
    import torch

    import io_aware_tiled_03_amd as fa
    seed = torch.zeros(fa.CALIB_SEED_BYTES // 2 - 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fa.calib_mfma(0, 2, 2, seed, torch.empty(512, device="cuda"))
    seed = torch.zeros(fa.CALIB_SEED_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fa.calib_mfma(0, 2, 2, seed, torch.empty(511, device="cuda"))
