"""GPU parity of FP8 caches whose last page is open: while a sequence's last
page holds fewer than 32 tokens its values are kept in token rows, and the
append that fills the page rewrites them as channel columns (the layout of
include/kvq.h). After every append of a sequence of calls that open, extend
and close pages (single tokens, chunks ending inside a page, chunks that close
one page and open the next, a chunk ending on a page boundary), the cache's
bytes equal the oracle's image bit for bit and decode -- the matrix-core FP8
kernel without rotary keys, the generic kernel with them -- stays within
tolerance of the oracle's fp64 attention. Shapes include head_dim 256 with
fp32 inputs (one page is the work of a whole 512-thread block)."""

import pytest
import torch

import harness as H
import kv_cache_quantisation_amd as kvq
import synth
from test_gpu_parity import small

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)

CHUNKS = [1, 1, 30, 5, 1, 1, 25, 1, 40, 23, 3, 1]   # closes pages at 32, 64, 128 and 96 inside a chunk
CASES = [
    # scheme, d, dtype, hg, rope
    (synth.FP8_E4M3, 128, torch.bfloat16, 4, 0.0),
    (synth.FP8_E5M2, 64, torch.bfloat16, 2, 0.0),
    (synth.FP8_E4M3, 256, torch.float32, 2, 0.0),
    (synth.FP8_E5M2, 256, torch.float32, 1, 10000.0),
    (synth.FP8_E4M3, 32, torch.float32, 2, 0.0),
    (synth.FP8_E4M3, 128, torch.bfloat16, 4, 500000.0),
]


@pytest.mark.parametrize("case", list(range(len(CASES))))
def test_fp8_open_page_rows_then_columns(case):
    scheme, d, dtype, hg, rope = CASES[case]
    T = sum(CHUNKS)
    w = small(scheme, 8, d, dtype, B=2, hg=hg, T=T, rope=rope)
    cfg = H.config(w, T + 20)
    cache = kvq.alloc_cache(cfg)
    oc = H.oracle_cache(w, T + 20)
    k, v = synth.keys_values(w, device=DEV)
    fmax = 57344.0 if scheme == synth.FP8_E5M2 else 448.0
    ks, vs = (x.to(DEV) for x in synth.fp8_scales(k, v, fmax))
    q = synth.query(w, device=DEV)
    t = 0
    for n in CHUNKS:
        kc, vc = k[:, t:t + n].contiguous(), v[:, t:t + n].contiguous()
        kvq.kvq_quantize_append(cfg, cache, 0, t, n, kc, vc, ks, vs)
        oc.append(0, H.host(kc), H.host(vc), H.host(ks), H.host(vs))
        t += n
        torch.cuda.synchronize()
        want, mask = oc.cache_image()
        H.compare_bytes(cache.cpu().numpy(), want, mask, f"case {case} after {t} tokens")
        out = H.decode(cfg, cache, 0, t, q, ks, vs)
        err = H.max_err(out, oc.decode(0, H.values(q), rope_theta=rope))
        assert err <= H.ATOL, (case, t, err)
