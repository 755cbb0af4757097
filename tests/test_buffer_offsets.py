"""CPU model of the GEMM kernels' buffer-load addressing.

A raw buffer load (stride 0) on gfx950 range-checks only the per-lane offset:
a load whose per-lane offset is at or past the resource's size reads zeros,
any other load reads base + per-lane offset + scalar offset.  The kernels
rely on that check for ragged tiles and for the prefetch past a tile's last
K step, so every load must either fall wholly inside its resource or be
wholly out of range by its per-lane offset alone.  This test restates, in
numpy, the offsets each of the buffer-load GEMM kernels issues (the 128 x 128 tile
kernel's staging, the persistent 256 x 256 ring, the ping-pong kernel, the
skinny kernel) and checks that rule for the configs' shapes and ragged ones.
The ping-pong kernel also writes its outputs with range-checked buffer
stores: the model checks that every in-range store lands on its own output
row and columns, that every output is written exactly once, and that the
stores it drops are out of range by their per-lane offset.  It must be kept
in step with the kernels' index arithmetic in gemm.hip."""
import numpy as np
import pytest


def check(vo, so, size, num_records, what):
    vo = np.asarray(vo, dtype=np.int64).ravel()
    so = np.broadcast_to(np.asarray(so, dtype=np.int64), vo.shape)
    assert vo.min() >= 0 and (vo < 2 ** 32).all(), f"{what}: per-lane offset outside 32 bits"
    inr = vo < num_records
    lo = vo[inr] + so[inr]
    assert (lo >= 0).all(), what
    assert (lo + size <= num_records).all(), f"{what}: an in-range load reads past the resource"
    # a load partly in range would read a mix of data and zeros
    assert (vo[inr] + size <= num_records).all(), f"{what}: a load straddles the resource's end"


def tile128_loads(M, K, N):
    """128 x 128 tile kernel, staging through buffer loads (K % 64 == 0, no
    K chunks): steps 0 .. nsteps, the last one the prefetch past the end."""
    BM = BN = 128
    nsteps = K // 64
    c = np.arange(512)
    tid = np.arange(256)
    for m0 in range(0, M, BM):
        rows = min(M - m0, BM)
        for s in range(nsteps + 1):
            k = s * 64
            check((c >> 2) * K + (c & 3) * 16 + k, 0, 16, rows * K, f"codes m0={m0} s={s}")
    for n0 in range(0, N, BN):
        cols = min(N - n0, BN)
        for s in range(nsteps + 1):
            k = s * 64
            check((tid >> 1) * (K // 2) + (tid & 1) * 16 + (k >> 1), 0, 16, cols * (K // 2),
                  f"weights n0={n0} s={s}")


def r3_swz(r):
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 1)


def ring3_loads(M, K, N):
    """Persistent 256 x 256 ring (K % 128 == 0): every stage of every tile."""
    BBM = BBN = 256
    nsteps = K // 128
    wave = np.arange(8)[:, None, None]
    lane = np.arange(64)[None, :, None]
    i4 = np.arange(4)[None, None, :]
    i2 = np.arange(2)[None, None, :]
    a_vo = (lane >> 3) * K + (((lane & 7) ^ r3_swz(lane >> 3)) * 16)
    w_vo = (wave * 32 + (lane >> 2)) * (K // 2) + (((lane & 3) ^ ((lane >> 3) & 3)) * 16)
    for m0 in range(0, M, BBM):
        for st in range(nsteps):
            check(a_vo + (wave * 4 + i4) * (8 * K) + st * 128, 0, 16, (M - m0) * K,
                  f"ring codes m0={m0} st={st}")
    for n0 in range(0, N, BBN):
        for st in range(nsteps):
            check(w_vo + i2 * (16 * (K // 2)) + st * 64, 0, 16, (N - n0) * (K // 2),
                  f"ring weights n0={n0} st={st}")


def pp_loads(M, K, N, sw_sz=2, b_sz=2):
    """Ping-pong 256 x 256 kernel (K % 128 == 0): every stage of every tile
    (the step's K offset in the scalar offset, never past the tile's last
    step), and the scale staging."""
    nsteps = K // 128
    lw = np.arange(4)[:, None, None]
    lane = np.arange(64)[None, :, None]
    i8 = np.arange(8)[None, None, :]
    i4 = np.arange(4)[None, None, :]
    a_vo = (lw * 64 + (lane >> 3)) * K + (((lane & 7) ^ r3_swz(lane >> 3)) * 16) + i8 * (8 * K)
    swz = (0x78 >> (2 * i4)) & 3
    w_vo = (lw * 64 + i4 * 16 + (lane >> 2)) * (K // 2) + (((lane & 3) ^ swz) * 16)
    for m0 in range(0, M, 256):
        for st in range(nsteps):
            check(a_vo, st * 128, 16, (M - m0) * K, f"pp codes m0={m0} st={st}")
    for n0 in range(0, N, 256):
        for st in range(nsteps):
            check(w_vo, st * 64, 16, (N - n0) * (K // 2), f"pp weights n0={n0} st={st}")
    b = np.arange(4)[:, None]
    vo = b * 256 + np.arange(64)[None, :] * 4
    for n0 in range(0, N, 256):
        for sz, what in ((sw_sz, "scales"), (b_sz, "bias")):
            check(vo[: 256 * sz // 256], 0, 4, (N - n0) * sz, f"pp {what} n0={n0}")
    for m0 in range(0, M, 256):
        check(vo, 0, 4, (M - m0) * 4, f"pp row scales m0={m0}")


def pp_stores(M, N, esz, col_check=True):
    """Ping-pong kernel's output stores (N % 16 == 0): per tile, wave (wm, wn)
    lane (j, q) writes row wm*128 + 16 mt + j, columns wn*64 + 16 q .. +15;
    a lane whose columns start past N takes an offset past the resource
    (col_check=False leaves that out, for the test of the model)."""
    assert N % 16 == 0 and N * esz * 512 < 2 ** 32
    per = 16 // esz
    written = np.zeros((M, N), dtype=np.int32)
    wave = np.arange(8)[:, None, None, None]
    lane = np.arange(64)[None, :, None, None]
    mt = np.arange(8)[None, None, :, None]
    h = np.arange(16 // per)[None, None, None, :]
    wm, wn, j, q = wave & 1, wave >> 1, lane & 15, lane >> 4
    c0 = wn * 64 + 16 * q
    for m0 in range(0, M, 256):
        for n0 in range(0, N, 256):
            rows = min(M - m0, 256)
            nrec = (rows * N - n0) * esz
            off = ((wm * 128 + j) * N + c0) * esz
            if col_check:
                off = np.where(n0 + c0 < N, off, nrec)
            o = np.broadcast_to(off + mt * (16 * N * esz) + 16 * h, (8, 64, 8, 16 // per)).astype(np.int64)
            assert (o < 2 ** 32).all(), "store offset outside 32 bits"
            inr = o < nrec
            assert (o[inr] + 16 <= nrec).all(), "a store straddles the resource's end"
            row = np.broadcast_to(m0 + wm * 128 + mt * 16 + j, o.shape)[inr]
            col = np.broadcast_to(n0 + c0 + per * h, o.shape)[inr]
            # the in-range store's address is the one of its output
            assert np.array_equal(o[inr], ((row - m0) * N + (col - n0)) * esz)
            assert (row < M).all() and (col + per <= N).all()
            for e in range(per):
                np.add.at(written, (row, col + e), 1)
    assert (written == 1).all(), "an output written never or twice"


def skinny_loads(M, K, N):
    """Skinny-M kernel (M <= 64, K % 64 == 0)."""
    MT = 1 if M <= 16 else 2 if M <= 32 else 4
    nsteps = K // 64
    lane = np.arange(64)
    j, kq = lane & 15, lane >> 4
    a_off = j * K + kq * 16
    w_off = j * (K // 2) + kq * 8
    for st in range(nsteps):
        k0 = st * 64
        for mt in range(MT):
            check(a_off + mt * 16 * K + k0, 0, 16, M * K, f"skinny codes st={st}")
    for n0 in range(0, N, 16):
        for st in range(nsteps):
            check(w_off + (st * 64 >> 1), 0, 8, (N - n0) * (K // 2), f"skinny weights n0={n0}")


@pytest.mark.parametrize("M,K,N", [(100, 192, 130), (77, 1024, 40), (129, 2048, 200),
                                   (4096, 16384, 6144), (250, 64, 17)])
def test_tile128_staging_stays_in_bounds(M, K, N):
    tile128_loads(M, K, N)


@pytest.mark.parametrize("M,K,N", [(8192, 3840, 3840), (8192, 10240, 3840), (300, 2048, 520),
                                   (4100, 256, 4130), (4352, 384, 4112)])
def test_ring3_stays_in_bounds(M, K, N):
    ring3_loads(M, K, N)


@pytest.mark.parametrize("M,K,N", [(8192, 3840, 3840), (8192, 10240, 3840), (300, 2048, 528),
                                   (4100, 256, 4112), (4352, 384, 4128), (129, 256, 16)])
@pytest.mark.parametrize("sw_sz,b_sz", [(2, 2), (4, 4), (2, 4)])
def test_pingpong_loads_stay_in_bounds(M, K, N, sw_sz, b_sz):
    pp_loads(M, K, N, sw_sz, b_sz)


@pytest.mark.parametrize("M,N", [(300, 528), (4100, 272), (129, 16), (513, 4112), (1024, 3840)])
@pytest.mark.parametrize("esz", [2, 4])
def test_pingpong_stores_cover_each_output_once(M, N, esz):
    pp_stores(M, N, esz)


def test_store_model_catches_a_missing_column_check():
    # without the past-N redirect, a ragged tile's lanes beyond the last
    # column write the next row's first outputs
    with pytest.raises(AssertionError):
        pp_stores(300, 272, 2, col_check=False)


@pytest.mark.parametrize("M,K,N", [(32, 3840, 3840), (1, 64, 16), (33, 640, 129), (64, 4096, 272)])
def test_skinny_stays_in_bounds(M, K, N):
    skinny_loads(M, K, N)


def test_model_catches_a_scalar_offset_past_the_end():
    # the staging as it would be with the step's k in the scalar offset: the
    # prefetch past the last step on the tile's last row reads past the end
    M, K = 100, 192
    c = np.arange(512)
    rows = M
    with pytest.raises(AssertionError):
        check((c >> 2) * K + (c & 3) * 16, K, 16, rows * K, "k as scalar offset")
