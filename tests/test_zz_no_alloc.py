"""The allocation-free MLA head (kvrc_mla_kv_head_paged_noalloc): its
static workspace in place of a caller's, the outputs of the entry point
with a workspace, bit for bit.

Two calls in a row on the one static array, the second with fewer tokens:
each must equal the workspace entry point's result on the same inputs (the
kernel is deterministic for a given He, so the outputs are the same bits).
The workspace entry point itself is checked against the float64 oracle in
test_gpu_mla.py.
"""
import numpy as np
import pytest
import torch

import gen
import latent_attention_kv_amd as k

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def dbf(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_cache(arr):
    if arr.dtype == np.uint16:
        return dbf(arr)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(DEV)


def host(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.cpu().numpy()


def run(case, noalloc):
    caches = {n: dev_cache(spec.numpy()) for n, spec in case["caches"].items()}
    ins = (dbf(case["x"]), dbf(case["w"]), dbf(case["gamma"]), dbf(case["cos"]),
           dbf(case["sin"]), torch.from_numpy(case["slot_mapping"]).to(DEV))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    if noalloc:
        k.kvrc_mla_kv_head_paged_noalloc(*ins, caches["k_cache"], caches["ckv_cache"],
                                         caches.get("ckv_scale"), alpha_kv=case["alpha"],
                                         eps=case["eps"], err_count=err)
    else:
        ws = torch.zeros(k.kvrc_mla_kv_head_workspace_bytes(case["x"].shape[0]),
                         dtype=torch.uint8, device=DEV)
        k.kvrc_mla_kv_head_paged(*ins, caches["k_cache"], caches["ckv_cache"],
                                 caches.get("ckv_scale"), workspace=ws, alpha_kv=case["alpha"],
                                 eps=case["eps"], err_count=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return {n: host(t) for n, t in caches.items()}


@pytest.mark.parametrize("kind", ["bf16", "int8"])
def test_noalloc_equals_the_workspace_entry_point(kind):
    """Two calls in a row, the second smaller: 9000 tokens (36 pairs of
    workgroups, a ragged last pair), then 700 tokens (3 pairs) on the same
    static array, which keeps the first call's contents."""
    for seed, S in ((570, 9000), (571, 700)):
        case = gen.mla_kv_head_case(seed, B=1, S=S, He=512, num_blocks=96, block_size=128,
                                    slot_kind="random", skip_frac=0.02, ckv_dtype=kind)
        want = run(case, noalloc=False)
        got = run(case, noalloc=True)
        for n in want:
            np.testing.assert_array_equal(got[n], want[n], err_msg=f"T={S} {n}")
        print(f"[noalloc] {kind} T={S}: bit-identical to the workspace entry point", flush=True)


def test_noalloc_rejects_tokens_beyond_its_workspace():
    T = k.MLA_NOALLOC_MAX_TOKENS + 1
    x = torch.zeros(T, 32, dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(576, 32, dtype=torch.bfloat16, device=DEV)
    g = torch.zeros(512, dtype=torch.bfloat16, device=DEV)
    cs = torch.zeros(T, 64, dtype=torch.bfloat16, device=DEV)
    slots = torch.full((T,), -1, dtype=torch.int64, device=DEV)
    kc = torch.zeros(1, 16, 1, 64, dtype=torch.bfloat16, device=DEV)
    ck = torch.zeros(1, 16, 1, 512, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(k.KvrcError, match="workspace"):
        k.kvrc_mla_kv_head_paged_noalloc(x, w, g, cs, cs, slots, kc, ck)
