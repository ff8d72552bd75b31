"""Host side of the split-count study: the summary's counts and table, and the seeded draw.
Runs without a GPU."""

from attention_ulysses_a2a_amd import split_study as ss


def test_summary_counts_and_rows():
    lines = [
        {"split_study": "S=1024 H=1 D=64", "S": 1024, "H": 1, "D": 64, "n_tiles": 8,
         "us": {"1": 13.2, "4": 9.0}, "model_split": 4, "best_split": 4, "model_loss_pct": 0.0},
        {"split_study": "S=2304 H=1 D=64", "S": 2304, "H": 1, "D": 64, "n_tiles": 18,
         "us": {"4": 12.1, "8": 11.8}, "model_split": 4, "best_split": 8, "model_loss_pct": 2.54},
        {"split_study": "B=2 S=4608 H=6 D=128", "set": "random seed 5, 2 shapes", "B": 2, "S": 4608, "H": 6,
         "D": 128, "n_tiles": 432, "us": {"1": 80.0, "2": 74.8}, "model_split": 1, "best_split": 2,
         "model_loss_pct": 6.95},
    ]
    md = ss.summarize(lines, "python bench.py --split-study", "abc")
    assert "* grid: over 2 shapes the model's count is the fastest measured on 1, within 2 % on 1 and within 5 % on 2" in md
    assert "* random seed 5, 2 shapes: over 1 shapes" in md and "largest 6.95 %" in md
    assert "* all: over 3 shapes the model's count is the fastest measured on 1, within 2 % on 1 and within 5 % on 2; " \
           "mean loss 3.16 %, largest 6.95 %" in md
    assert "| grid | 1 | 2304 | 1 | 64 | 18 | 4 | 12.1 | 8 | 11.8 | +2.54 % |" in md
    assert "* B=2 S=4608 H=6 D=128: 1: 80.0, 2: 74.8" in md


def test_shape_sets():
    grid = ss.grid_shapes()
    assert len(grid) == 30 and all(b == 1 for b, _, _, _ in grid)
    a, b = ss.random_shapes(777, 40), ss.random_shapes(777, 40)
    assert a == b and len(a) == 40 and a != ss.random_shapes(778, 40)
    for B, S, H, D in a:
        assert B in (1, 2, 4) and 1 <= H <= 8 and D in (64, 128) and S % 8 == 0 and 512 <= S < 20000
        assert 8 <= B * H * ((S + 127) // 128) <= 1200
