"""bench.py's host-side arithmetic (no GPU): the algorithmic byte counts behind `value` and the
roofline, the cold-HBM copy counts, and the fused launch's grid as the library picks it."""
import bench


def test_algorithmic_bytes_of_the_metric_workload():
    n, N = 4_194_304, 8                       # 16 MiB fp32 per rank, 8 ranks
    C = n // N
    assert bench.chunk_bytes(C) == 540_672    # codes + one fp32 scale per 128
    assert bench.fused_read_bytes(n, N) == 8_110_080
    assert bench.fused_write_bytes(n, N, 4) == 17_317_888
    assert bench.fused_bytes(n, N, 4) == 25_427_968
    assert bench.quantize_bytes(n, 4) == 21_102_592
    assert bench.rs_bytes(n, N) == 4_866_048
    assert bench.ag_bytes(n, N, 4) == 21_102_592
    assert bench.dda_bytes(32_768, N) == 589_824          # 8 x 64 KiB bf16 in, 64 KiB out
    assert bench.fused_bytes(134_217_728, N, 2) == 545_259_520   # 256 MiB bf16 per rank


def test_cold_copies_read_a_gib_between_reuses():
    assert bench.COLD_READ_BYTES == 1 << 30
    for read in (8 * bench.chunk_bytes(524_288), 16 << 20, 8 * 64 << 10, 2 << 20):
        c = bench.cold_copies(read)
        assert (c - 1) * read >= bench.COLD_READ_BYTES and c >= 2
    assert bench.cold_copies(8 * bench.chunk_bytes(524_288)) == 250


def test_fused_grid_matches_the_library_rule():
    # one vector per lane while the launch fits one round of 8,192 wavefronts, else two
    assert bench.fused_grid(4_194_304, 8, 4) == (256, 8)       # 16 MiB: two vectors, 8 slices
    assert bench.fused_grid(2_097_152, 8, 4) == (256, 7)       # 8 MiB: one vector fits one round
    assert bench.fused_grid(134_217_728, 8, 2) == (8_192, 7)   # bf16 output: always one vector
    assert bench.fused_grid(8_388_608, 8, 4) == (512, 8)       # 32 MiB
