"""Instruction mix of the compiled MFMA loops (gfx950 assembly, CPU only).

Per 64 score elements (one accumulator register per lane) the SiLU needs,
besides its two transcendentals (exp2, rcp), 3.5 other vector instructions in
the forward (scale, 1 + e, x * r, half a bf16 pack) and 7 in the key-owner
backward (SiLU and SiLU': scale, 1 + e, x * sg, two fused multiply-adds, the
product with dS, two half packs).  These tests hold the compiled tile bodies to
those counts (plus the key-owner's LDS swizzle addresses, under one per 64
elements) and the masked bodies to at most three more, so that a change which
makes the compiler add work in the hot loops is seen without a GPU.
"""
import collections
import os
import shutil

import pytest

from hstu_jagged_masked_amd import build as bld
from hstu_jagged_masked_amd import profiling

pytestmark = pytest.mark.skipif(not os.path.exists(bld.HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not available")


@pytest.fixture(scope="module")
def per_element(tmp_path_factory):
    """kernel -> sorted list of 'other VALU per 64 elements' over its SiLU blocks."""
    text = profiling.isa(str(tmp_path_factory.mktemp("isa")))
    out = collections.defaultdict(list)
    for line in text.splitlines()[1:]:
        left, _, right = line.partition("|")
        f = left.split()
        if right.strip():
            out[f[0]].append(float(right.split()[0]))
    return {k: sorted(v) for k, v in out.items()}


def test_forward_tile_is_the_silu_count(per_element):
    fwd = per_element["k_fwd_bf16"]
    assert fwd[0] <= 3.6, fwd          # unmasked tile: 3.5
    assert fwd[-1] <= 3.5 + 1.7, fwd   # masked tile: + field extract and and


def test_key_owner_step_is_the_silu_prime_count(per_element):
    for name in ("k_bwd_kv", "k_bwd_kv_p"):
        kv = per_element[name]
        assert kv[0] <= 7 + 1.2, (name, kv)      # unmasked step: 7 + swizzle addresses
        assert kv[-1] <= kv[0] + 3.1, (name, kv)  # masked: + extract, two ands


def test_every_mfma_kernel_has_silu_blocks(per_element):
    assert {"k_fwd_bf16", "k_bwd_kv", "k_bwd_kv_p", "k_bwd_q"} <= set(per_element)


def test_profile_names_of_the_key_owner_instantiations():
    """rocprofv3 and the assembly name the key-owner kernel's instantiations
    by their template arguments <store P, atomic dQ>; the summaries and the
    HBM-traffic table use the library's own timing names."""
    base = "void hstu::(anonymous namespace)::k_bwd_kv<{}>(unsigned short const*, int)"
    assert profiling.short_name(base.format("true, false")) == "k_bwd_kv_p"
    assert profiling.short_name(base.format("false, false")) == "k_bwd_kv"
    assert profiling.short_name(base.format("false, true")) == "k_bwd_kv_atomic"
    assert profiling.short_name("hstu::(anonymous namespace)::k_fwd_bf16(int)") == "k_fwd_bf16"
    mangled = "_ZN4hstu12_GLOBAL__N_18k_bwd_kvILb{}ELb{}EEEvPKtS3_"
    assert profiling.short_name_isa(mangled.format(1, 0)) == "k_bwd_kv_p"
    assert profiling.short_name_isa(mangled.format(0, 0)) == "k_bwd_kv"
    assert profiling.short_name_isa(mangled.format(0, 1)) == "k_bwd_kv_atomic"
