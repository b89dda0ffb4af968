import json
import os

from paged_kv_cache_208_amd.roofline import ridge_point, HBM_GBPS, MFMA_F16_TFLOPS


def test_ridge_point_matches_the_pages_h100_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "roofline_h100.json")))
    r = ridge_point(g["peak_tflops"], g["peak_bw_gbps"])
    assert round(r, g["printed_digits"]) == g["ridge_flop_per_byte"]


def test_mi355x_ridges_put_decode_far_below_mfma_ridge():
    # decode attention does g FLOP per fp16 KV byte (g = 4 or 8 here)
    assert ridge_point(MFMA_F16_TFLOPS, HBM_GBPS) > 300
