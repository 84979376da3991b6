"""The fused layer's split table as profiled metadata (COMET paper review
§4.2.2): the compiled-in table, the JSON file it is stored in, and
MOE_TUNING_TABLE pointing the library at another file.  Host logic only
(moe_layer_default_movers makes no GPU call; without a GPU the library
assumes 256 compute units)."""
import contextlib
import json
import os

import pytest

import combine_topk_gate_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TABLE = os.path.join(ROOT, "combine_topk_gate_amd", "tuning", "mi355x.json")
WORKLOADS = ("qwen2", "mixtral", "phi35", "epshare", "epshare_b")


@contextlib.contextmanager
def tuning_table(path):
    old = os.environ.get("MOE_TUNING_TABLE")
    os.environ["MOE_TUNING_TABLE"] = path
    try:
        yield
    finally:
        if old is None:
            del os.environ["MOE_TUNING_TABLE"]
        else:
            os.environ["MOE_TUNING_TABLE"] = old


def plan(M, H, F, E, k, S=1, EL=0, dtype="bf16"):
    return moe.moe_layer_default_movers(moe.problem(M, H, F, E, k, S, dtype, 0, EL))


def _entry_plan(e):
    return plan(e["M"], e["H"], e["F"], e["E"], e["k"], e["S"], 0 if e["EL"] == e["E"] else e["EL"])


def test_committed_file_matches_compiled_table():
    with open(TABLE) as fh:
        entries = json.load(fh)["entries"]
    assert sorted(e["config"] for e in entries) == sorted(WORKLOADS)
    compiled = [_entry_plan(e) for e in entries]
    assert compiled == [e["n_mover"] for e in entries]
    with tuning_table(TABLE):
        assert [_entry_plan(e) for e in entries] == compiled


def _write(tmp_path, text, name="t.json"):
    p = tmp_path / name
    p.write_text(text)
    return str(p)


def test_file_entries_replace_the_compiled_table(tmp_path):
    text = json.dumps({
        "note": {"nested": [1, 2.5, "x", None, True]},  # skipped
        "entries": [
            {"n_mover": 8, "EL": 8, "S": 1, "k": 2, "E": 8, "F": 640, "H": 512, "M": 1000, "chain_us": 12.5},
            {"M": 2000, "H": 512, "F": 640, "E": 8, "k": 2, "S": 1, "EL": 8, "n_mover": 1000},
            {"M": 3000, "H": 512, "F": 640, "E": 8, "k": 2, "S": 1, "EL": 8, "n_mover": 0, "config": "a \"b\""},
            {"M": 4000, "H": 512, "F": 640, "E": 8, "k": 2, "S": 1, "EL": 8, "n_mover": -1},
        ],
    })
    with tuning_table(_write(tmp_path, text)):
        assert plan(1000, 512, 640, 8, 2) == 8
        assert plan(2000, 512, 640, 8, 2) == 0  # more combiners than CUs: the shared queue
        assert plan(3000, 512, 640, 8, 2) == 0
        assert plan(4000, 512, 640, 8, 2) == -1
        assert plan(5000, 512, 640, 8, 2) == -1  # not listed: the chain
        assert plan(1000, 512, 640, 8, 2, dtype="f32") == -1  # f32 layers always run the chain
    # back to the compiled-in table, where that shape is not listed
    assert plan(1000, 512, 640, 8, 2) == -1


def test_variable_change_rereads(tmp_path):
    a = _write(tmp_path, json.dumps({"entries": [{"M": 1000, "H": 512, "F": 640, "E": 8, "k": 2, "S": 1,
                                                  "EL": 8, "n_mover": 4}]}), "a.json")
    b = _write(tmp_path, json.dumps({"entries": [{"M": 1000, "H": 512, "F": 640, "E": 8, "k": 2, "S": 1,
                                                  "EL": 8, "n_mover": 16}]}), "b.json")
    with tuning_table(a):
        assert plan(1000, 512, 640, 8, 2) == 4
    with tuning_table(b):
        assert plan(1000, 512, 640, 8, 2) == 16
    with tuning_table(a):
        assert plan(1000, 512, 640, 8, 2) == 4


def test_empty_entries_run_the_chain(tmp_path):
    with tuning_table(_write(tmp_path, '{"entries": []}')):
        assert plan(8192, 4096, 14336, 8, 2) == -1


@pytest.mark.parametrize("text", [
    '{"entries": [{"M": 1000, "H": 512, "F": 640, "E": 8, "k": 2, "S": 1, "EL": 8}]}',  # n_mover missing
    '{"entries": [{"M": 1000.5, "H": 512, "F": 640, "E": 8, "k": 2, "S": 1, "EL": 8, "n_mover": 0}]}',
    '{"entries": [{"M": 1000, "H": 512, "F": 640, "E": 8, "k": 2, "S": 1, "EL": 8, "n_mover": -5}]}',
    '{"entries": [{"M": 1000, "H": 512, "F": 640, "E": 8, "k": 2, "S": 1, "EL": 8, "n_mover": 0}]} x',
    '{"entries": [{"M": 1000, "H": 512, "F": 640, "E": 8, "k": 2, "S": 1, "EL": 8, "n_mover": 0}',
    '{"entries": [{"M": "1000", "H": 512, "F": 640, "E": 8, "k": 2, "S": 1, "EL": 8, "n_mover": 0}]}',
    '{"table": []}',  # no entries
    '',
])
def test_unusable_file_is_reported(tmp_path, text):
    with tuning_table(_write(tmp_path, text)):
        assert plan(1000, 512, 640, 8, 2) == -2
        assert plan(1000, 512, 640, 8, 2, dtype="f32") == -1  # the chain needs no plan


def test_missing_file_is_reported(tmp_path):
    with tuning_table(str(tmp_path / "absent.json")):
        assert plan(8192, 4096, 14336, 8, 2) == -2
