"""The launch planners at other compute-unit counts (no GPU needed).

The plans balance tiles of 64 channels (or SSD units) over the device's
compute units, which the library reads from the device; SSM_NUM_CU overrides
the count.  A plan shows in the workspace it needs, so these tests derive the
expected plan by hand for a few shapes and compare the sizes: a chained plan
adds one ready flag per chunk to the header and a carried state per chunk, a
chunk-pair plan adds the pairs (P, S) and the carries, a plan of whole tiles
only the packed B/C records.
"""
import pytest

from selective_state_space_33_amd import ops

F32, BF16 = ops.SSM_DTYPE_F32, ops.SSM_DTYPE_BF16


def a256(x):
    return (x + 255) // 256 * 256


def fwd_expected(batch, L, dim, N, chained_chunks=0, split_tiles=0, pair_chunks=0, direct=False):
    """Workspace of the two-state-per-lane, 8-wavefront variant (N = 16): header words (+ flags), packed B/C
    records of whole 128-token trips (+ 32 rows of padding; none for fp32 storage, whose B and C the scan reads
    directly), and the chunk pairs and carries."""
    Lp = (L + 127) // 128 * 128
    npad = 16
    words = 4 + split_tiles * chained_chunks
    ws = a256(words * 4) + (0 if direct else a256((batch * Lp + 32) * 2 * npad * 4))
    K = chained_chunks or pair_chunks
    per = a256(split_tiles * K * 64 * npad * 4) if split_tiles else 0
    if chained_chunks:
        ws += per              # carries only
    elif pair_chunks:
        ws += 3 * per          # P, S and carries
    return ws


@pytest.mark.parametrize("cus,expect", [
    (256, dict(chained_chunks=4, split_tiles=64)),   # 320 tiles on 256 CUs: 64 left over, 4 chunks each
    (320, dict()),                                   # one tile per CU: every tile whole
    (300, dict(chained_chunks=8, split_tiles=20)),   # 20 left over: 300 / 20 = 15 chunks, at most 8
    (512, dict(pair_chunks=4, split_tiles=320)),     # under 3/4 of the CUs: chunk pairs, ~2 chunks per CU
])
def test_forward_plan_follows_the_cu_count(monkeypatch, cus, expect):
    monkeypatch.setenv("SSM_NUM_CU", str(cus))
    got = ops.lib().ssm_scan_workspace_size(5, 2048, 64 * 64, 16, BF16)
    assert got == fwd_expected(5, 2048, 64 * 64, 16, **expect)


def test_forward_plan_chunks_no_shorter_than_256_tokens(monkeypatch):
    """300 tokens allow at most 2 chunks: the chained and the chunk-pair plans both stop there."""
    monkeypatch.setenv("SSM_NUM_CU", "256")
    lib = ops.lib()
    assert lib.ssm_scan_workspace_size(5, 300, 64 * 64, 16, BF16) == fwd_expected(5, 300, 64 * 64, 16,
                                                                                   chained_chunks=2, split_tiles=64)
    monkeypatch.setenv("SSM_NUM_CU", "512")
    assert lib.ssm_scan_workspace_size(5, 300, 64 * 64, 16, BF16) == fwd_expected(5, 300, 64 * 64, 16,
                                                                                   pair_chunks=2, split_tiles=320)


def test_forward_plan_small_device(monkeypatch):
    """A 10-tile layer on an 8-CU device: 8 whole tiles, 2 left over in 4 chunks of the 1024 tokens."""
    monkeypatch.setenv("SSM_NUM_CU", "8")
    got = ops.lib().ssm_scan_workspace_size(1, 1024, 640, 16, F32)
    assert got == fwd_expected(1, 1024, 640, 16, chained_chunks=4, split_tiles=2, direct=True)
    # the same plan in bf16 packs B and C into records
    got = ops.lib().ssm_scan_workspace_size(1, 1024, 640, 16, BF16)
    assert got == fwd_expected(1, 1024, 640, 16, chained_chunks=4, split_tiles=2)


def bwd_expected(batch, L, dim, r=0, Ks=1, Kc=1):
    """Backward workspace for N <= 16: header words (+ the flags of both chained launches), packed B/C,
    checkpoints every 16 tokens, dB/dC partials per tile, dA/dD/dbias partials per chunk slot, carried adjoints
    and carried checkpoint-pass states."""
    Lp = (L + 127) // 128 * 128
    npad = 16
    ntd = (dim + 63) // 64
    T = batch * ntd
    slots = Ks if r else 1
    words = 4 + (r * Ks + r * Kc if r else 0)
    return (a256(words * 4) + a256((batch * Lp + 32) * 2 * npad * 4) + a256(T * (Lp // 16) * 64 * npad * 4)
            + 2 * a256(batch * ntd * Lp * npad * 4) + a256(slots * batch * dim * npad * 4)
            + 2 * a256(slots * batch * dim * 4) + a256(r * Ks * 64 * npad * 4) + a256(r * Kc * 64 * npad * 4))


def test_bwd_plan_follows_the_cu_count(monkeypatch):
    lib = ops.lib()
    monkeypatch.setenv("SSM_NUM_CU", "256")
    # 320 tiles: 64 left over; the backward's 4 chunks of blocks, the checkpoint pass's 4 chunks of 1024 tokens
    assert lib.ssm_scan_bwd_workspace_size(4, 4096, 5120, 16, 0, BF16) == bwd_expected(4, 4096, 5120, r=64, Ks=4, Kc=4)
    monkeypatch.setenv("SSM_NUM_CU", "320")
    assert lib.ssm_scan_bwd_workspace_size(4, 4096, 5120, 16, 0, BF16) == bwd_expected(4, 4096, 5120)


def test_bwd_checkpoint_chunks_are_clamped(monkeypatch):
    """One tile left over (257 tiles on 256 CUs): the backward cuts it into 8 chunks of blocks, and the checkpoint
    pass into no more than 8 chunks of at least 256 tokens -- one chunk for 150 tokens, 8 for 4096 (not 256)."""
    monkeypatch.setenv("SSM_NUM_CU", "256")
    lib = ops.lib()
    assert lib.ssm_scan_bwd_workspace_size(1, 150, 64 * 257, 16, 0, BF16) == bwd_expected(1, 150, 64 * 257, r=1, Ks=8,
                                                                                         Kc=1)
    assert lib.ssm_scan_bwd_workspace_size(1, 4096, 64 * 257, 16, 0, BF16) == bwd_expected(1, 4096, 64 * 257, r=1,
                                                                                          Ks=8, Kc=8)


def test_ssd_plan_follows_the_cu_count(monkeypatch):
    lib = ops.lib()
    monkeypatch.setenv("SSM_NUM_CU", "256")
    ws = lib.ssm_ssd_fwd_workspace_size(4, 4096, 80, 64, 128, BF16)   # 64 units left over, 4 segments each
    assert ws == a256((4 + 64 * 4) * 4) + a256(64 * 4 * 64 * 128 * 4)
    monkeypatch.setenv("SSM_NUM_CU", "320")
    assert lib.ssm_ssd_fwd_workspace_size(4, 4096, 80, 64, 128, BF16) == 0   # one unit per CU
