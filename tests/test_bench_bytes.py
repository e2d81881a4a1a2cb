"""The algorithmic byte counts behind the bench's GB/s figures, checked
against the sizes the block formats fix (Q8_0: 34 bytes per 32 weights;
q8_1: 36 bytes per 32 values; fp32: 4 bytes) and against the per-expert and
per-layer figures they imply for the DS4.1 expert shape (hidden 4096,
expert intermediate 1024, top-8).  CPU only; nothing here touches a GPU."""

import bench

H, I, TOPK = 4096, 1024, 8
MATRIX = I * H // 32 * 34            # one expert matrix, 1024 x 4096 or 4096 x 1024


def test_one_expert_is_13_37_mb():
    assert MATRIX == 4_456_448
    gate_up = bench.gate_up_launch_bytes(1, 0, 0, H, I)
    down = bench.down_launch_bytes(1, 0, H, I)
    assert gate_up == 2 * MATRIX and down == MATRIX
    assert gate_up + down == 13_369_344


def test_single_column_layer_reads_eight_experts():
    """One column routed to eight distinct experts: 8 x 13.37 MB of weights,
    with activations, routing and outputs under 1% on top."""
    total = bench.layer_bytes(8, 8, 1, H, I, TOPK, 0)
    weights = 8 * 3 * MATRIX
    assert weights == 106_954_752
    assert weights < total < 1.01 * weights


def test_activation_terms():
    """Per route: h written by the gate/up launch and read by the down launch
    (fp32, 1024 values), y written (fp32, 4096 values); per column: x (fp32)
    and its q8_1 rows."""
    c, a, v = 5, 17, 40
    gu = bench.gate_up_launch_bytes(a, v, c, H, I)
    assert gu - 2 * a * MATRIX == c * (H // 32) * 36 + v * I * 4
    dn = bench.down_launch_bytes(a, v, H, I)
    assert dn - a * MATRIX == v * I * 4 + v * H * 4
    # the wide down reads the q8_1 rows of h instead of the fp32 ones
    assert bench.wide_down_bytes(a, v, H, I) - a * MATRIX == v * (I // 32) * 36 + v * H * 4


def test_shared_expert_slice():
    """Half of a 2048-wide shared expert: 1024 gate and up rows of 4096, and
    the 4096 down rows' 1024-value slice, each Q8_0."""
    rows, c = 1024, 8
    assert bench.shared_gate_up_bytes(c, H, rows) == 2 * rows * (H // 32) * 34 + c * rows * 4
    assert bench.shared_down_bytes(c, H, rows) == H * (rows // 32) * 34 + c * rows * 4 + c * H * 4
    with_share = bench.layer_bytes(23, 60, c, H, I, TOPK, rows)
    without = bench.layer_bytes(23, 60, c, H, I, TOPK, 0)
    weights_of_share = 2 * rows * (H // 32) * 34 + H * (rows // 32) * 34
    assert weights_of_share == 3 * MATRIX
    assert with_share - without == weights_of_share + c * rows * 4 * 2 + c * H * 4 * 2
