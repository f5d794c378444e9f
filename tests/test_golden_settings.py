"""The paper's stated settings (golden fixture) agree with the workload table."""
import json
import os

from matrix_optimizers_amd.workloads import get, AdamWHP

HERE = os.path.dirname(os.path.abspath(__file__))


def test_paper_owner_share_uses_paper_settings():
    g = json.load(open(os.path.join(HERE, "golden", "paper_settings.json")))
    hp = get("paper_owner_share").hp
    assert hp.lr == g["muon"]["lr"] and hp.weight_decay == g["muon"]["weight_decay"]
    assert hp.momentum == g["muon"]["momentum"] and hp.ns_steps == g["muon"]["ns_steps"]
    assert hp.lr_adjust == g["muon"]["lr_adjust"]
    a = AdamWHP()
    assert (a.lr, a.weight_decay, a.beta1, a.beta2, a.eps) == (
        g["adamw"]["lr"], g["adamw"]["weight_decay"], g["adamw"]["beta1"], g["adamw"]["beta2"],
        g["adamw"]["eps"])
    # one rank of span 8 holds 2 of the 16 layers: 4 square + 2 MLP matrices per layer
    mats = get("paper_owner_share").matrices
    h, f = g["model"]["hidden"], g["model"]["intermediate"]
    assert len(mats) == 12
    assert sum(m.rows * m.cols for m in mats) == 2 * (4 * h * h + 2 * h * f)
