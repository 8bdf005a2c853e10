"""The compiled-in tile table matches the committed sweep (CPU only)."""
import json

from scaled_dot_product_fa_amd import tune


def test_table_is_emitted_from_the_sweep():
    table = json.load(open(tune.TABLE_JSON))
    assert open(tune.TABLE_INC).read() == tune.emit(table)


def test_rules_name_valid_tiles_and_end_in_a_catch_all():
    table = json.load(open(tune.TABLE_JSON))
    rules = table["rules"]
    for dt in tune.DTYPES:
        for D in (64, 128):
            for causal in (False, True):
                rs = [r for r in rules if r["dtype"] == dt and r["D"] == D and r["causal"] == causal]
                assert rs, (dt, D, causal)
                assert all(r["tile"] in tune.TILES[D] for r in rs)
                assert rs[-1]["min_blocks256"] == 0 and rs[-1]["min_kv"] == 0
                mins = [(r["min_blocks256"], r["min_kv"]) for r in rs]
                assert mins == sorted(mins, reverse=True)


def test_the_sweep_covers_both_io_types():
    table = json.load(open(tune.TABLE_JSON))
    assert {r["dtype"] for r in table["results"]} == set(tune.DTYPES)
    assert {r["dtype"] for r in table["rules"]} == set(tune.DTYPES)


def test_rule_winners_are_the_sweep_winners():
    table = json.load(open(tune.TABLE_JSON))
    assert json.loads(json.dumps(tune.choose(table["results"]))) == table["rules"]
