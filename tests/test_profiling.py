"""The committed rocprofv3 summaries and how bench.py reads them: each summary
is stamped with the hash of its own optimizer's kernel sources, and a figure is
used only while that hash matches the sources."""
import glob
import os
import re

from matrix_optimizers_amd import profiling as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def test_workloads_map_to_their_optimizer():
    assert P.family_of("soap_decoder_layer_h2048") == "soap"
    assert P.family_of("shampoo_decoder_layer_h2048") == "shampoo"
    for w in ("large_single", "decoder_layer_h2048", "batched_1024", "llama8b_4layers"):
        assert P.family_of(w) == "muon"


def test_family_sources_exist_and_hash_apart():
    shas = {}
    for fam, files in P.FAMILY_SOURCES.items():
        for rel in files:
            assert os.path.exists(os.path.join(os.path.dirname(P.__file__), rel)), rel
        shas[fam] = P.sources_sha256(fam)
        assert re.fullmatch(r"[0-9a-f]{64}", shas[fam])
    assert len(set(shas.values())) == len(shas)
    # every kernel source of the library belongs to some family
    csrc = os.path.join(os.path.dirname(P.__file__), "csrc")
    covered = {rel for files in P.FAMILY_SOURCES.values() for rel in files}
    for f in glob.glob(os.path.join(csrc, "*_kernels.hip")):
        assert "csrc/" + os.path.basename(f) in covered, f


def test_committed_summaries_match_the_current_sources():
    """Every machine-readable line of a committed summary carries the hash of
    its optimizer's current sources, so bench.py reports its figures."""
    seen = 0
    for f in glob.glob(os.path.join(PROFILES, "*.md")):
        for line in open(f):
            p = line.split()
            if len(p) == 7 and p[0] == "traffic" or len(p) == 6 and p[0] == "executed":
                assert p[-1] == P.sources_sha256(P.family_of(p[1])), (os.path.basename(f), p[1], p[2])
                seen += 1
    assert seen > 0


def test_a_stale_summary_is_not_read(tmp_path):
    good = P.sources_sha256("soap")
    stale = "0" * 64
    (tmp_path / "a.md").write_text(
        f"traffic soap_decoder_layer_h2048 so_solve 10 20 30 {stale}\n"
        f"executed soap_decoder_layer_h2048 so_solve 0.5 2.0 {stale}\n")
    assert P.read_traffic(str(tmp_path), "soap_decoder_layer_h2048", "so_solve") is None
    (tmp_path / "b.md").write_text(f"traffic soap_decoder_layer_h2048 so_solve 10 20 30 {good}\n")
    tr = P.read_traffic(str(tmp_path), "soap_decoder_layer_h2048", "so_solve")
    assert tr["read_bytes"] == 10 and tr["write_bytes"] == 20 and tr["source"] == "b.md"
    # a Muon workload never takes a SOAP-stamped line
    assert P.read_traffic(str(tmp_path), "large_single", "so_solve") is None
