"""The algorithmic byte counts behind bench.py's GB/s figures, checked against
sums written out by hand for the configurations (no GPU)."""
import bench


def test_llama3_8b_layer_forward_bytes():
    # 8 x 8 K/V heads x 4096 rows x (256 B K + 256 B V); q bf16; 12 states of
    # (128 + 2) fp32 per (b, h_q) written and read; O + LSE fp32; 8 lengths
    kv, split, call = bench.algorithmic_bytes("contig", 8, 32, 8, 128, [4096] * 8, 12)
    assert kv == 8 * 8 * 4096 * 512 == 134_217_728
    states = 8 * 32 * 12 * 130 * 4
    assert split == kv + 8 * 32 * 128 * 2 + states + 8 * 4
    assert call == split + states + 8 * 32 * 129 * 4 == 137_610_272


def test_int8_sink_window_bytes():
    # 4 sinks + the newest 4096 positions of 16384, the newest 128 of them bf16
    # residual rows: 3972 int8 rows (128 + 128 code bytes + a 2-byte V scale),
    # 128 residual rows of 512 B, and the K scale rows of the touched groups
    # (group 0 for the sinks, groups 96 .. 126 for the window's int8 part)
    kv, _, call = bench.algorithmic_bytes("i8", 16, 32, 8, 128, [16384] * 16, 6, mask=(4, 4096))
    per_head = 3972 * 258 + 128 * 512 + (1 + 31) * 256
    assert kv == 16 * 8 * per_head
    assert call == 144_198_720


def test_paged_and_flashmask_bytes_count_only_what_is_read():
    # paged: one table entry per page of each request; masked keys never count
    kv, split, _ = bench.algorithmic_bytes("paged", 2, 4, 1, 128, [17, 0], 2)
    assert kv == 17 * 512
    assert split == kv + 2 * 4 * 128 * 2 + 2 * 4 * 2 * 130 * 4 + 2 * 4 + 2 * 4
    hidden = [[i % 3 == 0 for i in range(20)]]
    kv, split, _ = bench.algorithmic_bytes("contig", 1, 4, 1, 128, [20], 1, hidden=hidden)
    assert kv == 13 * 512
    assert split == kv + 4 * 128 * 2 + 4 * 130 * 4 + 4 + 2 * 2 * 16
