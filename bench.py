#!/usr/bin/env python3
"""Benchmark of the PIR database-multiplication scan on one MI355X.

One step = one pass of the whole scan path over both full-size databases:

  * RowSel, 48 GiB NTT-domain DB (N=4096, R=3 primes of 29 bits, P=12288,
    D0=D1=1024): a B=1 query (m=2) and a B=16 batch (m=32) sharing the tiled DB;
  * scalar-HE, 64 GiB int8 DB (M=K=262144): a B=1 query and a B=32 batch.

The tiled RowSel DB is built once by pirscan_layout_db and the tiled scalar DB
by pirscan_scalar_layout_db before timing (the databases are static).  All inputs are seeded synthetic data resident in HBM before the
timed region.  ``value`` = DB bytes scanned per step / step time (GB/s,
1 GB = 1e9 B).  Per-scan times come from HIP events on the stream the kernels
run on: around each scan call, and -- through the library's kernel-timer hook
-- around each scan's main kernel alone.  The ``roofline`` object is for the
main kernel that takes the most time, priced with its own launch duration.

Outside the step, ``next_rows`` measures VIPIR's ExpPack packing GEMM
H*C + (0|G) (section 3.6 size: N = 2^12, 3 primes, Dr = 256, n = 1280, a
15 GiB hint) for B = 1 and B = 16 the same way.

Also under ``next_rows``: the negacyclic NTT over the hint's 327680
polynomials (N = 2^12, three primes) -- the fused RNS decomposition + forward
transform of 5 GiB of integer coefficients, then the inverse and the forward
transform in place on the 15 GiB of residues.

Under ``config_rows``: the other configurations -- RowSel medium (3 GiB,
B = 1) on the int8 matrix-core scan and on the VALU scan, scalar 1 GiB (B = 1
and 8) on the tiled and the row-major entry points, the row-major entry point
pirscan_scalar_gemm_u32 at 64 GiB (B = 1 and 32), and the 48 GiB RowSel DB on
the VALU scan (B = 1 and 16) -- each timed the same way.

The ``cpu_baseline`` leg times the CPU oracle (oracle/, plain C) on the host
cores (count and CPU model reported) on bounded samples of the benchmark's own
device inputs, copied back first (copy time reported apart), and reports the
oracle's DB-scan rate for the same step mix, per scan, and on one thread for
the tiny and 1 GiB configurations.

The benchmark loads libpirscan_bench.so: the library's sources built with the
kernel-timing hooks of include/pirscan_bench.h.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
# 32-bit integer VALU rate of the multiply / min / select class: 256 CUs x 4
# SIMDs x 16 lanes per clock x 2.4 GHz (a probe measured v_mul_lo_u32,
# v_mul_hi_u32 and v_min_u32 at this rate and v_add_u32 at twice it)
VALU_INT32_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# integer operations per lazy (Harvey) butterfly with a Shoup product: three
# 32-bit multiplies and a subtraction for the twiddle product, a compare-and-
# subtract pair to keep one input below 2q, and one operation per output
NTT_OPS_PER_BUTTERFLY = 8
MFMA_INT8_PEAK_TOPS = 5000.0   # MI355X dense int8 MFMA, published (ops = 2 x MAC)
# VALU 32x32->64-bit multiply-add (v_mad_u64_u32): 256 CUs x 4 SIMDs x 16
# lanes per clock x 2.4 GHz = 39.3e12 MAC/s (half the issue rate of simple
# 32-bit ops such as v_add_u32, which run 32 lanes per SIMD per clock).
VALU_MAD64_PEAK_TMACS = 256 * 4 * 16 * 2.4e9 / 1e12

RS_N, RS_Q = 4096, [536813569, 536690689, 536641537]
RS_D0 = RS_D1 = 1024
SC_M = SC_K = 262144
EP_DR, EP_N = 256, 1280        # ExpPack: output ciphertexts, LWE dimension (same ring as RowSel)
# NTT over the hint's polynomials (VIPIR section 3.6: Dr x n polynomials of
# N = 2^12 over three primes); psi_r = g^((q_r - 1) / 2N) for the smallest
# generator g of each prime's group
NTT_PSI = [327210582, 176946644, 321217896]
NTT_COUNT = EP_DR * EP_N
# the scalar product at the pages' other shapes, on the 64 GiB database's bytes:
# VIPIR's hint DB * A (D/D0 = 2^20, n = 1280), the double-packing second fold
# (8N x D1 INT8 times D1 x (n+1), D1 = 2^17), and D/D0 = 2^20, 2^19, 2^17
N_LWE = 1280
SHAPE_SCANS = {
    "scalar_hint_64GiB_n1280": (1 << 20, 1 << 16, N_LWE),
    "scalar_fold2_4GiB_n1281": (8 * RS_N, 1 << 17, N_LWE + 1),
    "scalar_64GiB_D1_2e20_B1": (1 << 20, 1 << 16, 1),
    "scalar_64GiB_D1_2e20_B32": (1 << 20, 1 << 16, 32),
    "scalar_64GiB_D1_2e19_B1": (1 << 19, 1 << 17, 1),
    "scalar_64GiB_D1_2e19_B32": (1 << 19, 1 << 17, 32),
    "scalar_64GiB_D1_2e17_B1": (1 << 17, 1 << 19, 1),
    "scalar_64GiB_D1_2e17_B32": (1 << 17, 1 << 19, 32),
}
SEEDS = {"rowsel": 4, "scalar": 5, "exppack": 6, "ntt": 7, "scalar_1GiB": 2, "rowsel_medium": 3}
# the other configurations, reported beside the step: RowSel medium (3 GiB,
# D0 = D1 = 256, B = 1) on the matrix-core and on the VALU scan, scalar 1 GiB
# (M = K = 32768, B = 1 and 8) on the tiled and the row-major entry points, the
# row-major entry point at the 64 GiB configuration, and the 48 GiB RowSel DB
# on the VALU scan (B = 1 and 16)
RS_MED_D = 256
SC_SMALL = 32768
CPU_SAMPLE_POINTS = 64  # RowSel / ExpPack points the CPU baseline reads back (one RNS limb's first 64)
CPU_SAMPLE_ROWS = 2048  # scalar DB rows the CPU baseline reads back (512 MiB)

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
_CSRC = os.path.join(ROOT, "he_database_scan_amd", "csrc")
# The source file of each scan's main kernel (traffic figures are dropped once
# that file changes).
CONFIG_SCANS = {  # name -> main kernel (the step's four scans are in SCAN_KERNELS below)
    "scalar_64GiB_B1_rowmajor": "gemv_kernel",
    "scalar_64GiB_B32_rowmajor": "mfma_kernel<8, false>",
    "scalar_1GiB_B1": "gemv_tiled_kernel",
    "scalar_1GiB_B8": "mfma_kernel<4, true>",
    "scalar_1GiB_B1_rowmajor": "gemv_kernel",
    "scalar_1GiB_B8_rowmajor": "mfma_kernel<4, false>",
    "rowsel_3GiB_B1": "rowsel_packed_direct_kernel<1>",
    "rowsel_3GiB_B1_valu": "rowsel_kernel<2, 1, 4, 8>",
    "rowsel_48GiB_B1_valu": "rowsel_kernel<2, 1, 4, 8>",
    "rowsel_48GiB_B16_valu": "rowsel_kernel<32, 2, 4, 4>",
}
KERNEL_SOURCES = {
    **{name: os.path.join(_CSRC, "rowsel.hip" if "valu" in name else
                          "rowsel_mfma.hip" if name.startswith("rowsel") else "scalar.hip")
       for name in CONFIG_SCANS},
    "rowsel_48GiB_B1": os.path.join(_CSRC, "rowsel_mfma.hip"),
    "rowsel_48GiB_B16": os.path.join(_CSRC, "rowsel_mfma.hip"),
    "scalar_64GiB_B1": os.path.join(_CSRC, "scalar.hip"),
    "scalar_64GiB_B32": os.path.join(_CSRC, "scalar.hip"),
    "exppack_15GiB_B1": os.path.join(_CSRC, "rowsel_mfma.hip"),
    "exppack_15GiB_B16": os.path.join(_CSRC, "rowsel_mfma.hip"),
    **{name: os.path.join(_CSRC, "scalar.hip") for name in SHAPE_SCANS},
    "ntt_rns_fwd_hint": os.path.join(_CSRC, "ntt.hip"),
    "ntt_inv_hint": os.path.join(_CSRC, "ntt.hip"),
    "ntt_fwd_hint": os.path.join(_CSRC, "ntt.hip"),
}


def selected(spec: str, names, skip: bool) -> set:
    """The row names a comma-separated --shapes / --config-rows value picks
    (all, none, or names), empty when the matching --skip flag is set."""
    if skip or spec == "none":
        return set()
    if spec == "all":
        return set(names)
    want = {n for n in spec.split(",") if n}
    unknown = want - set(names)
    if unknown:
        raise SystemExit(f"unknown rows: {sorted(unknown)}")
    return want


def code_text(text: str) -> str:
    """A kernel source without its comments and blank lines: what the counters
    depend on (a comment edit keeps the profiled traffic valid)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln.strip())


def source_hash(path: str) -> str:
    """The kernel file's code together with the shared header it includes."""
    header = os.path.join(os.path.dirname(path), "internal.hpp")
    text = code_text(open(path).read()) + "\n" + code_text(open(header).read())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


class Workloads:
    """Device-resident inputs and outputs of the four scans."""

    def __init__(self):
        import torch

        import synth
        from he_database_scan_amd import pirscan

        self.torch, self.pirscan = torch, pirscan
        dev = torch.device("cuda:0")
        P = RS_N * len(RS_Q)
        self.shape = pirscan.RowselShape.make(RS_N, RS_Q, RS_D0, RS_D1)
        log("setup: RowSel 48 GiB DB (synthesise p-major, one-time relayout)")
        db = torch.empty((RS_D0, RS_D1, P), dtype=torch.int32, device=dev)
        synth.fill_residues_(db, SEEDS["rowsel"], synth.STREAM_ROWSEL_DB, RS_N, RS_Q)
        self.dbt = torch.empty(pirscan.layout_db_bytes(self.shape), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        pirscan.layout_db(self.shape, db, self.dbt)
        torch.cuda.synchronize()
        self.layout_s = time.perf_counter() - t0
        # the CPU baseline's sample: these points' p-major DB words, kept on the device
        self.rs_sample_pts = (RS_N, RS_N + CPU_SAMPLE_POINTS)
        self.rs_sample_db = db[:, :, self.rs_sample_pts[0]:self.rs_sample_pts[1]].contiguous()
        del db
        torch.cuda.empty_cache()
        self.ct, self.out, self.rws = {}, {}, {}
        for m in (2, 32):
            self.ct[m] = torch.empty((m, RS_D0, P), dtype=torch.int32, device=dev)
            synth.fill_residues_(self.ct[m], SEEDS["rowsel"], synth.STREAM_ROWSEL_CT, RS_N, RS_Q)
            self.out[m] = torch.empty((m, RS_D1, P), dtype=torch.int32, device=dev)
            nws = pirscan.rowsel_workspace_bytes(self.shape, m)
            self.rws[m] = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
        log("setup: scalar 64 GiB DB")
        self.sdb = torch.empty((SC_M, SC_K), dtype=torch.int8, device=dev)
        synth.fill_int8_(self.sdb, SEEDS["scalar"], synth.STREAM_SCALAR_DB)
        # the static DB is tiled once for the scan (the row-major bytes stay for
        # the other aspect ratios, which use the row-major entry point)
        self.sdbt = torch.empty(pirscan.scalar_layout_db_bytes(SC_M, SC_K), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        pirscan.scalar_layout_db(self.sdb, self.sdbt)
        torch.cuda.synchronize()
        self.slayout_s = time.perf_counter() - t0
        self.q, self.sout, self.ws = {}, {}, {}
        for B in (1, 32):
            self.q[B] = torch.empty((SC_K, B), dtype=torch.int32, device=dev)
            synth.fill_uint32_(self.q[B], SEEDS["scalar"], synth.STREAM_SCALAR_Q)
            self.sout[B] = torch.empty((SC_M, B), dtype=torch.int32, device=dev)
            self.ws[B] = torch.empty(pirscan.scalar_tiled_workspace_bytes(SC_M, SC_K, B), dtype=torch.uint8,
                                     device=dev)
        log("setup: ExpPack 15 GiB hint (synthesise p-major, one-time relayout)")
        self.eshape = pirscan.ExppackShape.make(RS_N, RS_Q, EP_DR, EP_N)
        h = torch.empty((EP_DR, EP_N, P), dtype=torch.int32, device=dev)
        synth.fill_residues_(h, SEEDS["exppack"], synth.STREAM_EXPPACK_H, RS_N, RS_Q)
        self.ht = torch.empty(pirscan.exppack_layout_h_bytes(self.eshape), dtype=torch.uint8, device=dev)
        pirscan.exppack_layout_h(self.eshape, h, self.ht)
        torch.cuda.synchronize()
        self.ep_sample_h = h[:, :, self.rs_sample_pts[0]:self.rs_sample_pts[1]].contiguous()
        del h
        torch.cuda.empty_cache()
        self.ec, self.eg, self.eout, self.ews = {}, {}, {}, {}
        for B in (1, 16):
            self.ec[B] = torch.empty((EP_N, 2 * B, P), dtype=torch.int32, device=dev)
            synth.fill_residues_(self.ec[B], SEEDS["exppack"], synth.STREAM_EXPPACK_C, RS_N, RS_Q)
            self.eg[B] = torch.empty((EP_DR, B, P), dtype=torch.int32, device=dev)
            synth.fill_residues_(self.eg[B], SEEDS["exppack"], synth.STREAM_EXPPACK_G, RS_N, RS_Q)
            self.eout[B] = torch.empty((EP_DR, 2 * B, P), dtype=torch.int32, device=dev)
            nws = pirscan.exppack_workspace_bytes(self.eshape, B)
            self.ews[B] = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
        torch.cuda.synchronize()

    def setup_ntt(self):
        """Integer coefficients of the hint's 327680 polynomials (5 GiB) and
        room for their three-limb transforms (15 GiB)."""
        torch, pirscan = self.torch, self.pirscan
        import synth

        dev = torch.device("cuda:0")
        log("setup: NTT over the hint's polynomials (5 GiB coefficients, 15 GiB residues)")
        self.nshape = pirscan.NttShape.make(RS_N, RS_Q, NTT_PSI)
        self.nplan = torch.empty(pirscan.ntt_plan_bytes(self.nshape), dtype=torch.uint8, device=dev)
        pirscan.ntt_plan_init(self.nshape, self.nplan)
        self.ncoef = torch.empty((NTT_COUNT, RS_N), dtype=torch.int32, device=dev)
        synth.fill_uint32_(self.ncoef, SEEDS["ntt"], synth.STREAM_NTT_IN)
        self.nres = torch.empty((NTT_COUNT, len(RS_Q), RS_N), dtype=torch.int32, device=dev)
        torch.cuda.synchronize()

    def ntt_scans(self):
        """The transform on either side of the scans, at the hint's size:
        fused RNS decomposition + forward NTT (integer coefficients in, three
        limbs out), then the inverse and the forward NTT in place.  Entries:
        (callable, residue bytes transformed, algorithmic HBM bytes, polynomials,
        butterflies, kind)."""
        pz, sh, plan = self.pirscan, self.nshape, self.nplan
        R = len(RS_Q)
        res_b = 4 * NTT_COUNT * R * RS_N
        coef_b = 4 * NTT_COUNT * RS_N
        bfly = NTT_COUNT * R * (RS_N // 2) * (RS_N.bit_length() - 1)
        return {
            "ntt_rns_fwd_hint": ((lambda: pz.ntt_rns_forward(sh, plan, self.ncoef, self.nres)),
                                 res_b, coef_b + res_b, NTT_COUNT, bfly, "ntt"),
            "ntt_inv_hint": ((lambda: pz.ntt_inverse(sh, plan, self.nres, self.nres)),
                             res_b, 2 * res_b, NTT_COUNT, bfly, "ntt"),
            "ntt_fwd_hint": ((lambda: pz.ntt_forward(sh, plan, self.nres, self.nres)),
                             res_b, 2 * res_b, NTT_COUNT, bfly, "ntt"),
        }

    def shape_scans(self, M, K, names):
        """The scalar product at the hint, second-fold and aspect-ratio shapes
        that view the leading M*K bytes of the 64 GiB database as [M][K]: that
        view is tiled once (as the step's DB is) and every listed shape scans
        the tiled copy.  Returns (tiled buffer, {name: scan})."""
        torch, pz = self.torch, self.pirscan
        import synth

        dev = torch.device("cuda:0")
        db = self.sdb.view(-1)[:M * K].view(M, K)
        tiled = torch.empty(pz.scalar_layout_db_bytes(M, K), dtype=torch.uint8, device=dev)
        pz.scalar_layout_db(db, tiled)
        out = {}
        for name in names:
            B = SHAPE_SCANS[name][2]
            q = torch.empty((K, B), dtype=torch.int32, device=dev)
            synth.fill_uint32_(q, SEEDS["scalar"], synth.STREAM_SCALAR_Q)
            o = torch.empty((M, B), dtype=torch.int32, device=dev)
            ws = torch.empty(pz.scalar_tiled_workspace_bytes(M, K, B), dtype=torch.uint8, device=dev)
            out[name] = ((lambda q=q, o=o, ws=ws, M=M, K=K: pz.scalar_gemm_u32_tiled(tiled, M, K, q, o, ws)),
                         M * K, M * K + 4 * K * B + 4 * M * B, B, M * K * B, "scalar")
        return tiled, out

    def rowmajor_scans(self):
        """pirscan_scalar_gemm_u32 -- the row-major entry point -- on the 64 GiB
        database's row-major bytes (the step scans the tiled copy)."""
        torch, pz = self.torch, self.pirscan
        dev = torch.device("cuda:0")
        self.rm_bufs, out = [], {}
        for B in (1, 32):
            q = self.q[B]
            o = torch.empty((SC_M, B), dtype=torch.int32, device=dev)
            ws = torch.empty(max(16, pz.scalar_workspace_bytes(SC_M, SC_K, B)), dtype=torch.uint8, device=dev)
            self.rm_bufs += [o, ws]
            out[f"scalar_64GiB_B{B}_rowmajor"] = (
                (lambda q=q, o=o, ws=ws: pz.scalar_gemm_u32(self.sdb, q, o, ws)),
                SC_M * SC_K, SC_M * SC_K + 4 * SC_K * B + 4 * SC_M * B, B, SC_M * SC_K * B, "scalar")
        return out

    def small_config_scans(self):
        """The two smaller configurations: scalar 1 GiB (M = K = 32768, B = 1
        and 8, tiled and row-major entry points) and RowSel medium (N = 4096,
        three primes, D0 = D1 = 256: 3 GiB, B = 1) on the matrix-core scan and
        on the VALU scan (each with its own one-time layout)."""
        torch, pz = self.torch, self.pirscan
        import synth

        dev = torch.device("cuda:0")
        log("setup: scalar 1 GiB and RowSel 3 GiB configurations")
        M = K = SC_SMALL
        sd = torch.empty((M, K), dtype=torch.int8, device=dev)
        synth.fill_int8_(sd, SEEDS["scalar_1GiB"], synth.STREAM_SCALAR_DB)
        st = torch.empty(pz.scalar_layout_db_bytes(M, K), dtype=torch.uint8, device=dev)
        pz.scalar_layout_db(sd, st)
        self.small = {"sdb": sd, "sdbt": st}
        out = {}
        for B in (1, 8):
            q = torch.empty((K, B), dtype=torch.int32, device=dev)
            synth.fill_uint32_(q, SEEDS["scalar_1GiB"], synth.STREAM_SCALAR_Q)
            o1 = torch.empty((M, B), dtype=torch.int32, device=dev)
            o2 = torch.empty((M, B), dtype=torch.int32, device=dev)
            w1 = torch.empty(pz.scalar_tiled_workspace_bytes(M, K, B), dtype=torch.uint8, device=dev)
            w2 = torch.empty(max(16, pz.scalar_workspace_bytes(M, K, B)), dtype=torch.uint8, device=dev)
            self.small[f"q{B}"] = q
            self.small[f"bufs{B}"] = (o1, o2, w1, w2)
            alg = M * K + 4 * K * B + 4 * M * B
            out[f"scalar_1GiB_B{B}"] = ((lambda q=q, o=o1, w=w1: pz.scalar_gemm_u32_tiled(st, M, K, q, o, w)),
                                        M * K, alg, B, M * K * B, "scalar")
            out[f"scalar_1GiB_B{B}_rowmajor"] = ((lambda q=q, o=o2, w=w2: pz.scalar_gemm_u32(sd, q, o, w)),
                                                 M * K, alg, B, M * K * B, "scalar")
        P, D = RS_N * len(RS_Q), RS_MED_D
        db = torch.empty((D, D, P), dtype=torch.int32, device=dev)
        synth.fill_residues_(db, SEEDS["rowsel_medium"], synth.STREAM_ROWSEL_DB, RS_N, RS_Q)
        ct = torch.empty((2, D, P), dtype=torch.int32, device=dev)
        synth.fill_residues_(ct, SEEDS["rowsel_medium"], synth.STREAM_ROWSEL_CT, RS_N, RS_Q)
        self.small["ct"] = ct
        rs_db = 4 * P * D * D
        for kind, suffix in ((pz.SCAN_AUTO, ""), (pz.SCAN_VALU, "_valu")):
            shape = pz.RowselShape.make(RS_N, RS_Q, D, D, scan=kind)
            dbt = torch.empty(pz.layout_db_bytes(shape), dtype=torch.uint8, device=dev)
            pz.layout_db(shape, db, dbt)
            o = torch.empty((2, D, P), dtype=torch.int32, device=dev)
            ws = torch.empty(pz.rowsel_workspace_bytes(shape, 2), dtype=torch.uint8, device=dev)
            self.small["rs" + suffix] = (shape, dbt, o, ws)
            out["rowsel_3GiB_B1" + suffix] = (
                (lambda shape=shape, dbt=dbt, o=o, ws=ws: pz.rowsel_modgemm(shape, 2, ct, dbt, o, ws)),
                rs_db, rs_db + 4 * P * 2 * (D + D), 1, P * 2 * D * D, "rowsel")
        torch.cuda.synchronize()
        del db
        torch.cuda.empty_cache()
        return out

    def valu48_scans(self):
        """The 48 GiB RowSel DB on the VALU scan (PIRSCAN_SCAN_VALU: the word
        layout and the 64-bit lazy-reduction kernel), B = 1 and 16.  Replaces
        the packed DB of the step (freed first) with its word layout."""
        torch, pz = self.torch, self.pirscan
        import synth

        dev = torch.device("cuda:0")
        P = RS_N * len(RS_Q)
        del self.dbt
        torch.cuda.empty_cache()
        log("setup: RowSel 48 GiB DB for the VALU scan (synthesise p-major, one-time word layout)")
        self.vshape = pz.RowselShape.make(RS_N, RS_Q, RS_D0, RS_D1, scan=pz.SCAN_VALU)
        db = torch.empty((RS_D0, RS_D1, P), dtype=torch.int32, device=dev)
        synth.fill_residues_(db, SEEDS["rowsel"], synth.STREAM_ROWSEL_DB, RS_N, RS_Q)
        self.vdbt = torch.empty(pz.layout_db_bytes(self.vshape), dtype=torch.uint8, device=dev)
        pz.layout_db(self.vshape, db, self.vdbt)
        torch.cuda.synchronize()
        del db
        torch.cuda.empty_cache()
        rs_db = 4 * P * RS_D0 * RS_D1
        out = {}
        self.vws = {}
        for m, B in ((2, 1), (32, 16)):
            self.vws[m] = torch.empty(pz.rowsel_workspace_bytes(self.vshape, m), dtype=torch.uint8, device=dev)
            out[f"rowsel_48GiB_B{B}_valu"] = (
                (lambda m=m: pz.rowsel_modgemm(self.vshape, m, self.ct[m], self.vdbt, self.out[m], self.vws[m])),
                rs_db, rs_db + 4 * P * m * (RS_D0 + RS_D1), B, P * m * RS_D0 * RS_D1, "rowsel")
        return out

    # name -> (callable, DB bytes, algorithmic HBM bytes, queries, macs, kind)
    def scans(self):
        P = RS_N * len(RS_Q)
        rs_db = 4 * P * RS_D0 * RS_D1
        sc_db = SC_M * SC_K
        pz = self.pirscan
        out = {}
        for m, B in ((2, 1), (32, 16)):
            ct, o, ws = self.ct[m], self.out[m], self.rws[m]
            out[f"rowsel_48GiB_B{B}"] = (
                (lambda ct=ct, o=o, m=m, ws=ws: pz.rowsel_modgemm(self.shape, m, ct, self.dbt, o, ws)),
                rs_db, rs_db + 4 * P * m * (RS_D0 + RS_D1), B, P * m * RS_D0 * RS_D1, "rowsel")
        for B in (1, 32):
            q, o, ws = self.q[B], self.sout[B], self.ws[B]
            out[f"scalar_64GiB_B{B}"] = (
                (lambda q=q, o=o, ws=ws: pz.scalar_gemm_u32_tiled(self.sdbt, SC_M, SC_K, q, o, ws)),
                sc_db, sc_db + 4 * SC_K * B + 4 * SC_M * B, B, SC_M * SC_K * B, "scalar")
        return out

    def next_scans(self):
        """ExpPack packing GEMM (the next row beyond the step): the 15 GiB hint
        is the streamed operand; C, G and out are per query."""
        P = RS_N * len(RS_Q)
        h_bytes = 4 * P * EP_DR * EP_N
        pz = self.pirscan
        out = {}
        for B in (1, 16):
            c, g, o, ws = self.ec[B], self.eg[B], self.eout[B], self.ews[B]
            alg = h_bytes + 4 * P * (EP_N * 2 * B + EP_DR * B + EP_DR * 2 * B)
            out[f"exppack_15GiB_B{B}"] = (
                (lambda c=c, g=g, o=o, ws=ws, B=B: pz.exppack_modgemm(self.eshape, B, c, self.ht, g, o, ws)),
                h_bytes, alg, B, P * EP_DR * 2 * B * EP_N, "exppack")
        return out


# int8 MACs the MFMA paths issue per algorithmic MAC: the scalar B>1 GEMM
# multiplies 4 query digit planes; RowSel / ExpPack multiply 4 x 4 limb pairs,
# and at m = 2 pad the 2 rows to a 16-row tile (x 8).
MFMA_MACS_PER_MAC = {"rowsel_48GiB_B1": 128, "rowsel_48GiB_B16": 16, "scalar_64GiB_B32": 4,
                     "exppack_15GiB_B1": 128, "exppack_15GiB_B16": 16, "rowsel_3GiB_B1": 128,
                     "scalar_64GiB_B32_rowmajor": 4, "scalar_1GiB_B8": 8, "scalar_1GiB_B8_rowmajor": 8,
                     **{name: 4 for name, (M, K, B) in SHAPE_SCANS.items() if B > 1}}
# scans on the VALU whose multiply work exceeds what HBM time allows: priced
# against the v_mad_u64_u32 rate (one per 32x32 -> 64-bit product)
VALU_BOUND = {"rowsel_48GiB_B16_valu"}
# shapes whose int8 MFMA work exceeds what HBM time allows: priced against the MFMA peak
MFMA_BOUND = {"scalar_hint_64GiB_n1280", "scalar_fold2_4GiB_n1281"}


def roofline_for(name, ms, db_bytes, alg_bytes, macs):
    """Every scan here is bound by HBM bandwidth at its shape; the MFMA scans
    also report the int8 MFMA utilisation they need.  ``ms`` is the main
    kernel's launch duration; its algorithmic bytes are the scan's (the
    streamed DB, the query operand once and the output once: the MFMA path's
    limb and output staging have exactly the sizes of ct and out)."""
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    rf = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
          "frac": achieved / HBM_PEAK_GBS}
    if name.startswith("ntt_"):
        # macs = butterflies per launch; the NTT kernels are bound by integer ALU issue
        tops = NTT_OPS_PER_BUTTERFLY * macs / (ms * 1e-3) / 1e12
        return {"bound": "alu", "achieved": tops, "peak": VALU_INT32_PEAK_TOPS, "unit": "TOP/s",
                "frac": tops / VALU_INT32_PEAK_TOPS, "hbm_GBps": achieved, "hbm_frac": achieved / HBM_PEAK_GBS}
    if name in VALU_BOUND:
        tmacs = macs / (ms * 1e-3) / 1e12
        return {"bound": "valu", "achieved": tmacs, "peak": VALU_MAD64_PEAK_TMACS, "unit": "TMAC/s",
                "frac": tmacs / VALU_MAD64_PEAK_TMACS, "hbm_GBps": achieved}
    if name.endswith("_valu"):
        rf["valu_mad64_TMACs"] = macs / (ms * 1e-3) / 1e12
        rf["valu_frac"] = rf["valu_mad64_TMACs"] / VALU_MAD64_PEAK_TMACS
    if name in MFMA_BOUND:
        tops = 2 * macs * MFMA_MACS_PER_MAC[name] / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": tops, "peak": MFMA_INT8_PEAK_TOPS, "unit": "TOP/s",
                "frac": tops / MFMA_INT8_PEAK_TOPS, "hbm_GBps": achieved}
    if name in MFMA_MACS_PER_MAC:
        tops = 2 * macs * MFMA_MACS_PER_MAC[name] / (ms * 1e-3) / 1e12
        rf["mfma_int8_TOPS"] = tops
        rf["mfma_frac"] = tops / MFMA_INT8_PEAK_TOPS
    return rf


def traffic_for(name):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    (profiles/traffic.json), or None if absent or the kernel source changed."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    ent = data.get(name)
    if not ent:
        return None
    if ent.get("source_sha256_16") != source_hash(KERNEL_SOURCES[name]):
        return None
    return ent.get("bytes_per_launch")


# The main kernel of each scan (the one the kernel timer, the roofline and the
# traffic refer to), in the order the benchmark first launches the scans.
# RowSel and ExpPack share kernel templates; their launches differ in grid
# size, and the scans are told apart by the (kernel, grid) group that appears
# first in dispatch order.
SCAN_KERNELS = {
    "rowsel_48GiB_B1": "rowsel_packed_direct_kernel<1>",
    "rowsel_48GiB_B16": "rowsel_packed_kernel<2, 2",
    "scalar_64GiB_B1": "gemv_tiled_kernel",
    "scalar_64GiB_B32": "mfma_kernel<8, true>",
    "exppack_15GiB_B1": "rowsel_packed_direct_kernel<1>",
    "exppack_15GiB_B16": "rowsel_packed_kernel<2, 2",
    **{name: CONFIG_SCANS[name] for name in ("scalar_64GiB_B1_rowmajor", "scalar_64GiB_B32_rowmajor",
                                             "scalar_1GiB_B1", "scalar_1GiB_B1_rowmajor", "scalar_1GiB_B8",
                                             "scalar_1GiB_B8_rowmajor", "rowsel_3GiB_B1", "rowsel_3GiB_B1_valu")},
    **{name: ("gemv_tiled_kernel" if B == 1 else "mfma_kernel<8, true>" if B <= 32 else
              "mfma_kernel<16, true>" if B <= 64 else "mfma_wide_kernel")
       for name, (M, K, B) in SHAPE_SCANS.items()},
    "rowsel_48GiB_B1_valu": CONFIG_SCANS["rowsel_48GiB_B1_valu"],
    "rowsel_48GiB_B16_valu": CONFIG_SCANS["rowsel_48GiB_B16_valu"],
    "ntt_rns_fwd_hint": "ntt_rns_kernel<12",
    "ntt_inv_hint": "ntt_kernel<12, true",
    "ntt_fwd_hint": "ntt_kernel<12, false",
}


# the scans the current run launches (all of SCAN_KERNELS unless row filters
# leave some out), in launch order: profile summaries attribute kernel groups
# to these only
RUN_SCANS = list(SCAN_KERNELS)


def assign_scan_groups(groups):
    """groups: {(kernel, grid): first dispatch id}.  Returns {scan: (kernel,
    grid)}, giving each scan of the run, in launch order, the earliest group of
    its kernel not yet taken."""
    taken, out = set(), {}
    for scan in RUN_SCANS:
        pat = SCAN_KERNELS[scan]
        cands = sorted((first, g) for g, first in groups.items() if g[0].startswith(pat) and g not in taken)
        if cands:
            out[scan] = cands[0][1]
            taken.add(cands[0][1])
    return out


def _short_kernel_name(name: str) -> str:
    for pre in ("void ", "pirscan::(anonymous namespace)::", "(anonymous namespace)::"):
        name = name.replace(pre, "")
    return name.split("(")[0]


def traffic_from_counters(fetch_csv: str, write_csv: str, calib_gib: float) -> dict:
    """Turns two rocprofv3 --pmc runs of this benchmark (FETCH_SIZE, then
    WRITE_SIZE, both with --calib-copy-gib) into HBM bytes per launch of each
    scan's dominant kernel.  Each counter is scaled by what it reads for the
    plain copy of calib_gib GiB (the largest copy kernel in the run)."""
    import csv
    import statistics

    def load(path, counter):
        vals, first = {}, {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            g = (_short_kernel_name(r["Kernel_Name"]), int(r["Grid_Size"]))
            vals.setdefault(g, []).append(float(r["Counter_Value"]))
            first[g] = min(first.get(g, 1 << 62), int(r["Dispatch_Id"]))
        return vals, first

    out = {"calibration": {}}
    per, every = {}, {}
    for kind, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        vals, first = load(path, counter)
        copies = [v for g, vs in vals.items() if "copy" in g[0].lower() for v in vs]
        if not copies:
            raise SystemExit(f"no copy kernel in {path}: run the profile with --calib-copy-gib")
        scale = calib_gib * 2**30 / (max(copies) * 1024.0)  # true bytes per counted byte
        out["calibration"][counter] = {"copy_bytes": calib_gib * 2**30, "counter_KiB": max(copies),
                                       "scale": scale}
        # every (kernel, grid) group of the run, the per-query passes around the
        # main kernels included
        for g, vs in vals.items():
            e = every.setdefault(g, {"kernel": g[0], "grid_size": g[1], "launches": len(vs), "first": first[g]})
            e[kind + "_bytes"] = statistics.median(vs) * 1024.0 * scale
        for scan, g in assign_scan_groups(first).items():
            per.setdefault(scan, {})[kind + "_bytes"] = statistics.median(vals[g]) * 1024.0 * scale
            per[scan]["kernel"] = g[0]
            per[scan]["grid_size"] = g[1]
    for scan, ent in per.items():
        if "fetch_bytes" in ent and "write_bytes" in ent:
            ent["bytes_per_launch"] = ent["fetch_bytes"] + ent["write_bytes"]
            ent["source_sha256_16"] = source_hash(KERNEL_SOURCES[scan])
            out[scan] = ent
    out["all_kernels"] = [{k: v for k, v in e.items() if k != "first"}
                          for e in sorted(every.values(), key=lambda e: e["first"])
                          if "fetch_bytes" in e and "write_bytes" in e]
    return out


# MI355X unit counts for the counter-derived rates
SIMDS = 256 * 4
MFMA_INT8_OPS_PER_SIMD_CLK = MFMA_INT8_PEAK_TOPS * 1e12 / (SIMDS * 2.4e9)  # 2035: the published peak at 2.4 GHz
COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
            "SQ_INSTS_VALU_MFMA_MOPS_I8", "SQ_BUSY_CU_CYCLES", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE"]


def counters_from(csv_paths) -> dict:
    """Per-scan figures from rocprofv3 --pmc collections of this benchmark
    (counters COUNTERS, summed over the chip's instances by rocprofv3):
    the dispatch's duration; GRBM_GUI_ACTIVE per XCD (the kernel's GPU clock
    cycles) and the achieved clock it implies; the MFMA busy fraction
    (SQ_VALU_MFMA_BUSY_CYCLES over SIMD cycles); the VALU busy fraction
    (SQ_ACTIVE_INST_VALU, in quad-cycles, over SIMD cycles); VALU and MFMA
    instructions issued; the counted int8 MFMA operations (512 per
    SQ_INSTS_VALU_MFMA_MOPS_I8) against the published peak and against the
    peak at the achieved clock.  Medians over each scan's dispatches."""
    import csv
    import statistics

    disp = {}
    for path in csv_paths:
        for r in csv.DictReader(open(path)):
            d = disp.setdefault(int(r["Dispatch_Id"]), {"kernel": _short_kernel_name(r["Kernel_Name"]),
                                                      "grid": int(r["Grid_Size"]), "c": {}})
            d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    groups, first = {}, {}
    for did, d in disp.items():
        g = (d["kernel"], d["grid"])
        groups.setdefault(g, []).append(d)
        first[g] = min(first.get(g, 1 << 62), did)
    out = {}
    for scan, g in assign_scan_groups(first).items():
        rows = []
        for d in groups[g]:
            c, ns = d["c"], d["ns"]
            gui = c.get("GRBM_GUI_ACTIVE", 0.0) / 8.0  # summed over the 8 XCDs
            if gui <= 0 or ns <= 0:
                continue
            simd_cycles = gui * SIMDS
            mops = c.get("SQ_INSTS_VALU_MFMA_MOPS_I8", 0.0) * 512
            rows.append({"ms": ns / 1e6, "gui_active_cycles": gui, "clock_GHz": gui / ns,
                         "mfma_busy": c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / simd_cycles,
                         "valu_busy": 4 * c.get("SQ_ACTIVE_INST_VALU", 0.0) / simd_cycles,
                         "valu_insts": c.get("SQ_INSTS_VALU", 0.0), "mfma_insts": c.get("SQ_INSTS_MFMA", 0.0),
                         "int8_ops": mops, "int8_TOPS": mops / ns / 1e3,
                         "int8_frac_published": mops / ns / 1e3 / MFMA_INT8_PEAK_TOPS,
                         "int8_frac_at_clock": mops / (simd_cycles * MFMA_INT8_OPS_PER_SIMD_CLK)})
        if rows:
            med = {k: statistics.median(r[k] for r in rows) for k in rows[0]}
            out[scan] = dict(med, kernel=g[0], grid_size=g[1], dispatches=len(rows))
    return out


def counters_markdown(res: dict) -> str:
    lines = ["| scan | main kernel | dispatches | ms | GUI cycles (per XCD) | clock GHz | MFMA busy | VALU busy | "
             "int8 TOP/s (counted) | of 5.0 POP/s | of peak at clock |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for scan, r in res.items():
        lines.append(f"| {scan} | `{r['kernel']}` | {r['dispatches']} | {r['ms']:.3f} | {r['gui_active_cycles']:.3e} | "
                     f"{r['clock_GHz']:.2f} | {r['mfma_busy']:.3f} | {r['valu_busy']:.3f} | {r['int8_TOPS']:.0f} | "
                     f"{r['int8_frac_published']:.3f} | {r['int8_frac_at_clock']:.3f} |")
    return "\n".join(lines)


def summarize_trace(trace_csv: str) -> str:
    """Markdown table of a rocprofv3 --kernel-trace CSV of this benchmark:
    launches grouped by (kernel, grid size), with the scan each main-kernel
    group belongs to."""
    import csv

    groups, first = {}, {}
    for r in csv.DictReader(open(trace_csv)):
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        g = (_short_kernel_name(r["Kernel_Name"]), grid)
        groups.setdefault(g, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6)
        first[g] = min(first.get(g, 1 << 62), int(r["Dispatch_Id"]))
    scan_of = {g: scan for scan, g in assign_scan_groups(first).items()}
    total = sum(sum(v) for v in groups.values())
    lines = ["| kernel | grid (work-items) | calls | avg ms | min ms | max ms | % of GPU time | scan (main kernel) |",
             "|---|---|---|---|---|---|---|---|"]
    for g, v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{g[0]}` | {g[1]} | {len(v)} | {sum(v) / len(v):.3f} | {min(v):.3f} | {max(v):.3f} | "
                     f"{100 * sum(v) / total:.2f} | {scan_of.get(g, '')} |")
    return "\n".join(lines)


def host_info():
    """The host this run is on: logical CPUs (hardware concurrency), what
    `nproc` reports for this process, the threads the oracle uses (the
    process's affinity set, capped by OMP_NUM_THREADS when set: the machine's
    CPU share) and the CPU model."""
    import subprocess

    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        nproc = int(subprocess.run(["nproc"], capture_output=True, text=True, check=True).stdout)
    except (OSError, ValueError, subprocess.CalledProcessError):
        nproc = None
    threads = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        threads = min(threads, int(cap))
    return {"hardware_concurrency": os.cpu_count(), "nproc": nproc, "affinity_cpus": len(os.sched_getaffinity(0)),
            "omp_num_threads": cap or None, "threads_used": threads, "cpu_model": model}


def cpu_baseline(w, budget_s: float = 2.0):
    """Times the CPU oracle (oracle/, plain C) on this machine's host cores, on
    bounded samples of the benchmark's own device inputs.  Each sample is
    copied back from device memory (the copy timed on its own), then the
    oracle's compute call is repeated until about ``budget_s`` seconds have
    been spent on it; only the compute is timed.  Also times the whole tiny
    RowSel and scalar 1 GiB configurations on one thread.  Returns (per-scan
    oracle rates in DB bytes/s on all threads, host info, sample text,
    device-to-host copy figures, single-thread rates)."""
    import torch

    import oracle
    import synth

    host = host_info()
    threads = host["threads_used"]
    a, b = w.rs_sample_pts
    npts, qr = b - a, [RS_Q[a // RS_N]]
    copies = {"bytes": 0, "s": 0.0}

    def fetch(t):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        h = t.contiguous().cpu()
        copies["s"] += time.perf_counter() - t0
        copies["bytes"] += h.numel() * h.element_size()
        return h.numpy()

    def u32(t):
        return fetch(t).view("uint32")

    def timed(fn):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= budget_s:
                return reps, dt

    rates, samples = {}, []
    rs_db = u32(w.rs_sample_db)
    h_s = u32(w.ep_sample_h)
    for m, B in ((2, 1), (32, 16)):
        ct = u32(w.ct[m][:, :, a:b])
        reps, dt = timed(lambda ct=ct: oracle.rowsel(ct, rs_db, npts, qr, nthreads=threads))
        rates[f"rowsel_48GiB_B{B}"] = reps * rs_db.nbytes / dt
        samples.append(f"rowsel_48GiB_B{B}: points {a}..{b - 1} x {RS_D0}x{RS_D1}, m={m}, {reps} reps in {dt:.1f} s")
    sc_db = fetch(w.sdb[:CPU_SAMPLE_ROWS]).view("int8")
    for B in (1, 32):
        Q = u32(w.q[B])
        reps, dt = timed(lambda Q=Q: oracle.scalar(sc_db, Q, nthreads=threads))
        rates[f"scalar_64GiB_B{B}"] = reps * sc_db.nbytes / dt
        samples.append(f"scalar_64GiB_B{B}: rows 0..{CPU_SAMPLE_ROWS - 1} x {SC_K}, B={B}, {reps} reps in {dt:.1f} s")
    for B in (1, 16):
        C, G = u32(w.ec[B][:, :, a:b]), u32(w.eg[B][:, :, a:b])
        reps, dt = timed(lambda C=C, G=G: oracle.exppack(h_s, C, G, npts, qr, nthreads=threads))
        rates[f"exppack_15GiB_B{B}"] = reps * h_s.nbytes / dt
        samples.append(f"exppack_15GiB_B{B}: points {a}..{b - 1} x {EP_DR}x{EP_N}, B={B}, {reps} reps in {dt:.1f} s")
    if hasattr(w, "ncoef"):
        npolys = threads
        coef = u32(w.ncoef[:npolys])
        res = oracle.ntt_rns(coef, RS_Q, NTT_PSI, nthreads=threads)
        R = len(RS_Q)
        for name, fn in (("ntt_rns_fwd_hint", lambda: oracle.ntt_rns(coef, RS_Q, NTT_PSI, nthreads=threads)),
                         ("ntt_inv_hint", lambda: oracle.ntt_batch(res, RS_Q, NTT_PSI, inverse=True, nthreads=threads)),
                         ("ntt_fwd_hint", lambda: oracle.ntt_batch(res, RS_Q, NTT_PSI, nthreads=threads))):
            reps, dt = timed(fn)
            rates[name] = reps * 4 * npolys * R * RS_N / dt
            samples.append(f"{name}: polynomials 0..{npolys - 1} x {R} limbs x N={RS_N}, {reps} reps in {dt:.1f} s")
    # one thread, whole configurations: tiny RowSel and scalar 1 GiB
    single = {}
    N, m, D0, D1 = 256, 2, 16, 8
    tq = [1073738753, 1073732609]
    P = N * len(tq)
    dev = torch.device("cuda:0")
    t_ct = torch.empty((m, D0, P), dtype=torch.int32, device=dev)
    t_db = torch.empty((D0, D1, P), dtype=torch.int32, device=dev)
    synth.fill_residues_(t_ct, 1, synth.STREAM_ROWSEL_CT, N, tq)
    synth.fill_residues_(t_db, 1, synth.STREAM_ROWSEL_DB, N, tq)
    ct, db = u32(t_ct), u32(t_db)
    reps, dt = timed(lambda: oracle.rowsel(ct, db, N, tq, nthreads=1))
    single["rowsel_tiny"] = {"GBps": reps * db.nbytes / dt / 1e9, "reps": reps, "s": dt}
    if getattr(w, "small", None):
        sdb = fetch(w.small["sdb"]).view("int8")
        for B in (1, 8):
            Q = u32(w.small[f"q{B}"])
            for label, nt in ((f"scalar_1GiB_B{B}", 1), (f"scalar_1GiB_B{B}_all_threads", threads)):
                t0 = time.perf_counter()
                oracle.scalar(sdb, Q, nthreads=nt)
                dt = time.perf_counter() - t0
                if nt == 1:
                    single[label] = {"GBps": sdb.nbytes / dt / 1e9, "reps": 1, "s": dt}
                else:
                    rates[f"scalar_1GiB_B{B}"] = sdb.nbytes / dt
        samples.append(f"scalar_1GiB_B1/B8: the whole 1 GiB DB, one pass each on 1 and on {threads} threads")
    d2h = {"bytes": copies["bytes"], "s": copies["s"],
           "GBps": copies["bytes"] / copies["s"] / 1e9 if copies["s"] > 0 else None}
    return rates, host, "; ".join(samples), d2h, single


def read_reference(torch, pirscan, bufs, steps, warmup, stream):
    """The library's read-stream reference (one non-temporal 16-byte read pass,
    no arithmetic) over each tiled database, timed like the scans: the HBM
    rate a plain read of the same buffer reaches on this device and run."""
    sink = torch.empty(256, dtype=torch.uint8, device="cuda:0")
    scans = {name: ((lambda b=b: pirscan.bench_read(b, sink)), b.numel() * b.element_size())
             for name, b in bufs.items()}
    _, times = time_scans(torch, pirscan, scans, steps, warmup, stream)
    out = {}
    for name, (call_ms, kern_ms) in times.items():
        nbytes = scans[name][1]
        k = sorted(kern_ms)[len(kern_ms) // 2]
        out[name] = {"bytes": nbytes, "kernel_ms": k, "kernel_ms_min": min(kern_ms),
                     "GBps": nbytes / (k * 1e-3) / 1e9, "frac": nbytes / (k * 1e-3) / 1e9 / HBM_PEAK_GBS}
    return out


def time_scans(torch, pirscan, scans, steps, warmup, stream):
    """Runs `warmup` untimed rounds of the scans, then times `steps` rounds:
    HIP events around each scan call and, through the library's kernel timer,
    around each call's main kernel.  Returns (wall seconds of the timed
    rounds, {scan: (call ms list, main-kernel ms list)})."""
    names = list(scans)
    for _ in range(warmup):
        for name in names:
            scans[name][0]()
    torch.cuda.synchronize()
    events = {name: [] for name in names}
    pirscan.kernel_timer_begin(steps * len(names))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        for name in names:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            scans[name][0]()
            e1.record(stream)
            events[name].append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = pirscan.kernel_timer_end(steps * len(names))
    if len(kms) != steps * len(names):
        raise RuntimeError(f"kernel timer recorded {len(kms)} of {steps * len(names)} launches")
    out = {}
    for i, name in enumerate(names):
        out[name] = ([e0.elapsed_time(e1) for e0, e1 in events[name]], kms[i::len(names)])
    return wall, out


def workload_entry(name, scan, call_ms, kernel_ms):
    fn, db_bytes, alg_bytes, queries, macs, kind = scan
    ms = sum(call_ms) / len(call_ms)
    kms = sum(kernel_ms) / len(kernel_ms)
    srt = sorted(call_ms)
    rf = roofline_for(name, kms, db_bytes, alg_bytes, macs)
    rf["traffic"] = traffic_for(name)
    if kind == "ntt":
        return {"ms": ms, "ms_min": srt[0], "ms_median": srt[len(srt) // 2],
                "kernel": SCAN_KERNELS[name], "kernel_ms": kms, "kernel_ms_min": min(kernel_ms),
                "polys_per_s": queries / (ms * 1e-3), "residue_GBps": db_bytes / (ms * 1e-3) / 1e9,
                "butterflies_per_s": macs / (kms * 1e-3), "roofline": rf}
    return {"ms": ms, "ms_min": srt[0], "ms_median": srt[len(srt) // 2],
            "kernel": SCAN_KERNELS[name], "kernel_ms": kms, "kernel_ms_min": min(kernel_ms),
            "db_GBps": db_bytes / (ms * 1e-3) / 1e9, "qps": queries / (ms * 1e-3),
            "hbm_frac": db_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "roofline": rf}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-shapes", action="store_true",
                    help="leave out the scalar hint / second-fold / D/D0 rows (profiling runs: their MFMA "
                         "launches share one grid size with the step's B=32 scan)")
    ap.add_argument("--shapes", default="all",
                    help="comma-separated scalar shape rows to run (all, none, or names of SHAPE_SCANS)")
    ap.add_argument("--config-rows", default="all",
                    help="comma-separated configuration rows to run (all, none, or names of CONFIG_SCANS)")
    ap.add_argument("--skip-config-rows", action="store_true",
                    help="leave out the other configurations' rows (profiling runs: the RowSel 3 GiB scan "
                         "shares a kernel and grid size with ExpPack B=1)")
    ap.add_argument("--calib-copy-gib", type=float, default=0.0,
                    help="also run one torch copy of this many GiB (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: write profiles/traffic.json from two rocprofv3 --pmc counter "
                         "collections (FETCH_SIZE, WRITE_SIZE) of this benchmark")
    ap.add_argument("--counters-from", nargs="+", metavar="PMC_CSV",
                    help="no GPU: write profiles/counters.json (and print a markdown table) from rocprofv3 --pmc "
                         "collections of this benchmark with the counters " + " ".join(COUNTERS))
    ap.add_argument("--counters-out", default=os.path.join(ROOT, "profiles", "counters.json"),
                    help="where --counters-from writes its JSON")
    ap.add_argument("--summarize-trace", metavar="TRACE_CSV",
                    help="no GPU: print a markdown table of a rocprofv3 --kernel-trace CSV of this benchmark")
    args = ap.parse_args()
    # the scans this run (or the run a profile summary below describes) launches
    want_cfg = selected(args.config_rows, CONFIG_SCANS, args.skip_config_rows)
    want_shapes = selected(args.shapes, SHAPE_SCANS, args.skip_shapes)
    RUN_SCANS[:] = [n for n in SCAN_KERNELS
                    if (n not in CONFIG_SCANS or n in want_cfg) and (n not in SHAPE_SCANS or n in want_shapes)]
    if args.counters_from:
        res = counters_from(args.counters_from)
        json.dump(res, open(args.counters_out, "w"), indent=1)
        print(counters_markdown(res))
        return
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    if args.traffic_from:
        res = traffic_from_counters(*args.traffic_from, calib_gib=args.calib_copy_gib or 4.0)
        json.dump(res, open(TRAFFIC_FILE, "w"), indent=1)
        print(json.dumps(res, indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (--gpus {args.gpus} requested); the scan would shard "
              "by points (RowSel, ExpPack) or by DB rows (scalar-HE) with no exchange", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    from he_database_scan_amd import pirscan

    # the benchmark build: the product sources with the kernel-timing hooks
    # (include/pirscan_bench.h), so each scan's main kernel is timed live
    pirscan.use_library(pirscan.BENCH_LIB_PATH)
    w = Workloads()
    scans = w.scans()
    stream = torch.cuda.current_stream()

    if args.calib_copy_gib > 0:
        n = int(args.calib_copy_gib * 2**30)
        a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        torch.cuda.empty_cache()

    log(f"warmup {args.warmup} steps, timing {args.steps} steps")
    wall, times = time_scans(torch, w.pirscan, scans, args.steps, args.warmup, stream)
    per = {name: workload_entry(name, scans[name], *times[name]) for name in scans}
    total_db = sum(v[1] for v in scans.values())
    ms_per_step = wall / args.steps * 1e3
    value = total_db * args.steps / wall / 1e9
    dominant = max(per, key=lambda k: per[k]["kernel_ms"])

    log("read reference: one plain read pass over each tiled database")
    read_ref = read_reference(torch, w.pirscan, {"rowsel_48GiB_db": w.dbt, "scalar_64GiB_db": w.sdbt},
                              args.steps, min(args.warmup, 1), stream)

    log("next rows: ExpPack packing GEMM")
    nscans = w.next_scans()
    _, ntimes = time_scans(torch, w.pirscan, nscans, args.steps, args.warmup, stream)
    next_rows = {name: workload_entry(name, nscans[name], *ntimes[name]) for name in nscans}

    nsteps = min(args.steps, 3)
    config_rows = None
    if want_cfg - {"rowsel_48GiB_B1_valu", "rowsel_48GiB_B16_valu"}:
        log("configuration rows: row-major entry point at 64 GiB, scalar 1 GiB, RowSel 3 GiB")
        cscans = w.rowmajor_scans()
        cscans.update(w.small_config_scans())
        cscans = {name: v for name, v in cscans.items() if name in want_cfg}
        _, ctimes = time_scans(torch, w.pirscan, cscans, args.steps, args.warmup, stream)
        config_rows = {name: workload_entry(name, cscans[name], *ctimes[name]) for name in cscans}
        del cscans, w.rm_bufs
        torch.cuda.empty_cache()

    shape_rows = None
    if want_shapes:
        log("next rows: scalar product at the hint, second-fold and D/D0 shapes")
        del w.sdbt  # the step's tiled DB; each [M][K] view below is tiled in turn
        torch.cuda.empty_cache()
        shape_rows = {}
        views = {}
        for name, (M, K, B) in SHAPE_SCANS.items():
            if name in want_shapes:
                views.setdefault((M, K), []).append(name)
        for (M, K), names in views.items():
            tiled, sscans = w.shape_scans(M, K, names)
            _, stimes = time_scans(torch, w.pirscan, sscans, nsteps, 1, stream)
            shape_rows.update({name: workload_entry(name, sscans[name], *stimes[name]) for name in sscans})
            del tiled, sscans
            torch.cuda.empty_cache()
        shape_rows = {name: shape_rows[name] for name in SHAPE_SCANS if name in shape_rows}

    if want_cfg & {"rowsel_48GiB_B1_valu", "rowsel_48GiB_B16_valu"}:
        log("configuration rows: the 48 GiB RowSel DB on the VALU scan")
        if hasattr(w, "sdbt"):
            del w.sdbt  # the step is done: room for the word layout beside the p-major DB
        vscans = {name: v for name, v in w.valu48_scans().items() if name in want_cfg}
        _, vtimes = time_scans(torch, w.pirscan, vscans, nsteps, 1, stream)
        config_rows = config_rows or {}
        config_rows.update({name: workload_entry(name, vscans[name], *vtimes[name]) for name in vscans})
        del vscans, w.vdbt, w.vws
        torch.cuda.empty_cache()

    w.setup_ntt()
    log("next rows: NTT / INTT over the hint's polynomials")
    tscans = w.ntt_scans()
    _, ttimes = time_scans(torch, w.pirscan, tscans, args.steps, args.warmup, stream)
    ntt_rows = {name: workload_entry(name, tscans[name], *ttimes[name]) for name in tscans}

    result = {
        "metric": "effective DB-scan GB/s and QPS at 48/64 GiB DB; % of HBM roofline",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32/s8 integer (exact)",
        "data": "synthetic (seeded SplitMix64, generated on device)",
        "config": {"workload": "rowsel-48GiB(B=1,B=16)+scalar-64GiB(B=1,B=32)",
                   "rowsel": {"N": RS_N, "R": len(RS_Q), "q": RS_Q, "P": RS_N * len(RS_Q),
                              "D0": RS_D0, "D1": RS_D1, "m": [2, 32]},
                   "scalar": {"M": SC_M, "K": SC_K, "B": [1, 32]},
                   "hbm_frac_of_step": value / HBM_PEAK_GBS,
                   "layout_db_once_ms": w.layout_s * 1e3, "scalar_layout_db_once_ms": w.slayout_s * 1e3},
        "roofline": dict(per[dominant]["roofline"], kernel=SCAN_KERNELS[dominant], scan=dominant),
        "hbm_read_reference": read_ref,
        "workloads": per,
        "config_rows": {"config": {"scalar_64GiB_rowmajor": {"M": SC_M, "K": SC_K, "B": [1, 32],
                                                             "entry_point": "pirscan_scalar_gemm_u32"},
                                   "scalar_1GiB": {"M": SC_SMALL, "K": SC_SMALL, "B": [1, 8],
                                                   "entry_points": ["pirscan_scalar_gemm_u32_tiled",
                                                                    "pirscan_scalar_gemm_u32"]},
                                   "rowsel_3GiB": {"N": RS_N, "R": len(RS_Q), "D0": RS_MED_D, "D1": RS_MED_D,
                                                   "m": 2, "scan": ["auto (int8 MFMA)", "valu"]},
                                   "rowsel_48GiB_valu": {"D0": RS_D0, "D1": RS_D1, "m": [2, 32], "scan": "valu",
                                                         "steps": nsteps}},
                        "workloads": config_rows},
        "next_rows": {"exppack": {"config": {"N": RS_N, "R": len(RS_Q), "Dr": EP_DR, "n": EP_N, "B": [1, 16],
                                             "hint_GiB": 4 * RS_N * len(RS_Q) * EP_DR * EP_N / 2**30},
                                  "workloads": next_rows},
                      "scalar_shapes": {"config": {name: {"M": M, "K": K, "B": B}
                                                   for name, (M, K, B) in SHAPE_SCANS.items()},
                                        "steps": nsteps, "workloads": shape_rows},
                      "ntt": {"config": {"N": RS_N, "R": len(RS_Q), "q": RS_Q, "psi": NTT_PSI,
                                         "polynomials": NTT_COUNT,
                                         "coef_GiB": 4 * NTT_COUNT * RS_N / 2**30,
                                         "residue_GiB": 4 * NTT_COUNT * len(RS_Q) * RS_N / 2**30},
                              "workloads": ntt_rows}},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (the oracle on samples of the device inputs, host cores)")
        rates, host, sample, d2h, single = cpu_baseline(w)
        t_cpu = sum(scans[n][1] / rates[n] for n in scans)
        result["cpu_baseline"] = {"value": total_db / t_cpu / 1e9, "unit": "GB/s", "cores": host["threads_used"],
                                  "kind": "oracle", "sample": sample, "host": host,
                                  "per_scan_GBps": {n: r / 1e9 for n, r in rates.items()},
                                  "gpu_over_oracle_step": value / (total_db / t_cpu / 1e9),
                                  "d2h_copy": d2h, "single_thread": single}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
