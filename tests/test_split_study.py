"""Host side of the split-count study: the summary's counts and table.  Runs without a GPU."""

from attention_ulysses_a2a_amd import split_study as ss


def test_summary_counts_and_rows():
    lines = [
        {"split_study": "S=1024 H=1 D=64", "S": 1024, "H": 1, "D": 64, "n_tiles": 8,
         "us": {"1": 13.2, "4": 9.0}, "model_split": 4, "best_split": 4, "model_loss_pct": 0.0},
        {"split_study": "S=2304 H=1 D=64", "S": 2304, "H": 1, "D": 64, "n_tiles": 18,
         "us": {"4": 12.1, "8": 11.8}, "model_split": 4, "best_split": 8, "model_loss_pct": 2.54},
        {"split_study": "S=4608 H=6 D=128", "S": 4608, "H": 6, "D": 128, "n_tiles": 216,
         "us": {"1": 80.0, "2": 74.8}, "model_split": 1, "best_split": 2, "model_loss_pct": 6.95},
    ]
    md = ss.summarize(lines, "python bench.py --split-study", "abc")
    assert "Over 3 shapes the model's count is the fastest measured on 1, within 2 % on 1 and within 5 % on 2" in md
    assert "largest 6.95 %" in md
    assert "| 2304 | 1 | 64 | 18 | 4 | 12.1 | 8 | 11.8 | +2.54 % |" in md
    assert "* S=4608 H=6 D=128: 1: 80.0, 2: 74.8" in md
