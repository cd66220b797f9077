"""GPU parity of the block-scaled FP8 GEMM (fwd / dgrad / wgrad) against the
CPU oracle on the same seeded bf16 inputs: full outputs at sizes the oracle
finishes in seconds (several 256x256 tiles, ragged token counts), and sampled
outputs at the full transformer-shaped sizes in the launch configuration the
benchmark uses.  The gates are described in tests/parity.py: relative
Frobenius <= 1e-3; every element within the bound of the GPU's FP8
matrix-core accumulation; max element relative error <= 5e-3 (against
max(|ref|, 1e-2)) wherever the hardware can attain it."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
import hw_accum
from parity import bf16_host_bits, dev, fmt, gemm_gates, host, random_bf16, say

pytestmark = pytest.mark.gpu

FWD, DGRAD, WGRAD, DGRAD_W, FWD_T = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def pf():
    import fp8_block_scaled_tile_amd as pf
    assert torch.cuda.is_available()
    return pf


# ---- one linear layer on both sides -----------------------------------------

def device_operands(pf, mode, x, w, dy):
    """Quantize on the device exactly as a training step does, returning
    (a, sa, b, sb, M, N, K) for the requested GEMM mode."""
    if mode == FWD:
        qa = pf.quant_act(dev(x), row=True)
        qw = pf.quant_weight(dev(w), transpose=False)
        return qa["q"], qa["s"], qw["q"], qw["s"]
    if mode == DGRAD:
        qa = pf.quant_act(dev(dy), row=True)
        qw = pf.quant_weight(dev(w), transpose=True)
        return qa["q"], qa["s"], qw["qt"], qw["s"]
    if mode == DGRAD_W:                  # the weight's own codes, no transposed copy
        qa = pf.quant_act(dev(dy), row=True)
        qw = pf.quant_weight(dev(w), transpose=False)
        return qa["q"], qa["s"], qw["q"], qw["s"]
    if mode == FWD_T:                    # the transposed weight codes
        qa = pf.quant_act(dev(x), row=True)
        qw = pf.quant_weight(dev(w), transpose=True)
        return qa["q"], qa["s"], qw["qt"], qw["s"]
    qa = pf.quant_act(dev(dy), row=False, col=True)
    qb = pf.quant_act(dev(x), row=False, col=True)
    return qa["qt"], qa["st"], qb["qt"], qb["st"]


def oracle_operands(mode, x, w, dy):
    if mode in (FWD, FWD_T):            # FWD_T computes FWD's products
        qa, sa = oracle.quant_rowwise(synth.bits(x))
        qw, _, sw = oracle.quant_weight(synth.bits(w), transpose=False)
        return qa, sa, qw, sw
    if mode in (DGRAD, DGRAD_W):        # DGRAD_W computes DGRAD's products
        qa, sa = oracle.quant_rowwise(synth.bits(dy))
        _, qwt, sw = oracle.quant_weight(synth.bits(w), transpose=True)
        return qa, sa, qwt, sw
    qa, sa = oracle.quant_colwise(synth.bits(dy))
    qb, sb = oracle.quant_colwise(synth.bits(x))
    return qa, sa, qb, sb


def make_inputs(T, d_in, d_out, seed):
    x = synth.normal((T, d_in), 1.0, seed, f"gemm/x/{T}x{d_in}")
    synth.with_outliers(x, max(1, d_in // 100), 20.0, seed, f"gemm/x/{T}x{d_in}")
    w = synth.normal((d_out, d_in), 0.02, seed, f"gemm/w/{d_out}x{d_in}")
    dy = synth.normal((T, d_out), 1e-3, seed, f"gemm/dy/{T}x{d_out}")
    return x.to(torch.bfloat16), w.to(torch.bfloat16), dy.to(torch.bfloat16)


def run_case(pf, mode, T, d_in, d_out, out_dtype, seed=0, accumulate=False):
    x, w, dy = make_inputs(T, d_in, d_out, seed)
    say("gemm", MODE_NAMES[mode], f"T={T} in={d_in} out={d_out}", out_dtype,
        "acc" if accumulate else "")
    a, sa, b, sb = device_operands(pf, mode, x, w, dy)
    M, N = a.shape[0], (b.shape[1] if mode in B_KN else b.shape[0])
    c0 = None
    out = None
    if accumulate:
        c0 = synth.normal((M, N), 1e-2, seed, "gemm/c0")
        out = dev(c0)
    c = pf.gemm_blockscaled(mode, a, sa, b, sb, out_dtype=out_dtype, out=out,
                            accumulate=accumulate)
    oa, osa, ob, osb = oracle_operands(mode, x, w, dy)
    omode = ORACLE_MODE[mode]
    assert np.array_equal(host(a), oa)
    assert np.array_equal(host(b).T if mode in B_KN else host(b), ob)
    ref = oracle.gemm_blockscaled(omode, oa, osa, ob, osb)
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    bound = hw_accum.bounds(omode, oa, osa, ob, osb, ii.ravel(), jj.ravel(), ref.ravel())
    if accumulate:
        ref = (c0.numpy() + ref).astype(np.float32)
        extra = 2.0 ** -22 * np.abs(ref.ravel())             # the final read-add-write
        bound = (bound[0] + extra, bound[1] + extra)
    # FWD reads X with outlier channels (x20): the named exemption of parity.py
    g = gemm_gates(device_values(c), ref, bound, out_dtype == torch.bfloat16,
                   literal=omode != FWD)
    say("   " + fmt(g))
    assert g["ok"], g
    return g


MODE_NAMES = {FWD: "fwd", DGRAD: "dgrad", WGRAD: "wgrad", DGRAD_W: "dgrad_w", FWD_T: "fwd_t"}
B_KN = (DGRAD_W, FWD_T)                  # modes whose b is stored [K][N]
ORACLE_MODE = {FWD: FWD, DGRAD: DGRAD, WGRAD: WGRAD, DGRAD_W: DGRAD, FWD_T: FWD}


def device_values(c):
    if c.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f32(bf16_host_bits(c))
    return host(c)


SMALL = [  # (T, d_in, d_out): several tiles, ragged token counts, N not % 256
    (256, 128, 256),
    (300, 512, 384),
    (129, 1024, 128),
    (1, 256, 256),
    (513, 384, 640),
    (1000, 768, 512),
]


@pytest.mark.parametrize("T,d_in,d_out", SMALL)
def test_fwd_small(pf, T, d_in, d_out):
    run_case(pf, FWD, T, d_in, d_out, torch.float32)
    run_case(pf, FWD, T, d_in, d_out, torch.bfloat16)


@pytest.mark.parametrize("T,d_in,d_out", SMALL)
def test_dgrad_small(pf, T, d_in, d_out):
    run_case(pf, DGRAD, T, d_in, d_out, torch.float32)
    run_case(pf, DGRAD, T, d_in, d_out, torch.bfloat16)


@pytest.mark.parametrize("T,d_in,d_out", SMALL)
def test_wgrad_small(pf, T, d_in, d_out):
    run_case(pf, WGRAD, T, d_in, d_out, torch.float32)
    run_case(pf, WGRAD, T, d_in, d_out, torch.float32, accumulate=True)


@pytest.mark.parametrize("T,d_in,d_out", SMALL)
def test_dgrad_from_weight_codes_small(pf, T, d_in, d_out):
    """DGRAD_W reads the weight's own codes W [out][in] through LDS transpose
    reads: the oracle's gates, and bit for bit the DGRAD result on the
    transposed copy (the fragments pair the same k in the same order)."""
    for dt in (torch.float32, torch.bfloat16):
        run_case(pf, DGRAD_W, T, d_in, d_out, dt)
    x, w, dy = make_inputs(T, d_in, d_out, 0)
    a, sa, bt, sb = device_operands(pf, DGRAD, x, w, dy)
    _, _, bw, _ = device_operands(pf, DGRAD_W, x, w, dy)
    for dt in (torch.float32, torch.bfloat16):
        c1 = pf.gemm_blockscaled(DGRAD, a, sa, bt, sb, out_dtype=dt)
        c2 = pf.gemm_blockscaled(DGRAD_W, a, sa, bw, sb, out_dtype=dt)
        assert torch.equal(c1, c2)


@pytest.mark.parametrize("T,d_in,d_out", SMALL)
def test_fwd_from_transposed_weight_codes_small(pf, T, d_in, d_out):
    """FWD_T reads the transposed weight codes W^T [in][out] through LDS
    transpose reads: the oracle's gates, and bit for bit the FWD result."""
    for dt in (torch.float32, torch.bfloat16):
        run_case(pf, FWD_T, T, d_in, d_out, dt)
    x, w, dy = make_inputs(T, d_in, d_out, 0)
    a, sa, bw, sb = device_operands(pf, FWD, x, w, dy)
    _, _, bt, _ = device_operands(pf, FWD_T, x, w, dy)
    for dt in (torch.float32, torch.bfloat16):
        c1 = pf.gemm_blockscaled(FWD, a, sa, bw, sb, out_dtype=dt)
        c2 = pf.gemm_blockscaled(FWD_T, a, sa, bt, sb, out_dtype=dt)
        assert torch.equal(c1, c2)


@pytest.mark.parametrize("mode", [FWD, DGRAD, WGRAD, DGRAD_W, FWD_T])
def test_split_k_paths(pf, mode):
    """Few output tiles and a long K: the K range is split across work-groups
    and reduced in a second kernel (FP32 and bf16 outputs, accumulate)."""
    T, d_in, d_out = (2048, 256, 256) if mode != WGRAD else (4096, 256, 256)
    if mode in (FWD, FWD_T):
        T, d_in, d_out = 256, 2048, 256
    elif mode in (DGRAD, DGRAD_W):
        T, d_in, d_out = 256, 256, 2048
    M = T if mode != WGRAD else d_out
    N = d_out if mode in (FWD, FWD_T) else d_in
    K = d_in if mode in (FWD, FWD_T) else (d_out if mode in (DGRAD, DGRAD_W) else T)
    assert pf.puro_fp8_gemm_workspace_bytes(mode, M, N, K) > 0
    run_case(pf, mode, T, d_in, d_out, torch.float32)
    run_case(pf, mode, T, d_in, d_out, torch.bfloat16)
    run_case(pf, mode, T, d_in, d_out, torch.float32, accumulate=True)


@pytest.mark.parametrize("mode,T,d_in,d_out", [
    (FWD, 1000, 768, 512),
    (DGRAD, 513, 384, 640),
    (FWD, 256, 2048, 256),      # split-K: the reduce kernel rounds
])
def test_bf16_output_is_rne_of_fp32(pf, mode, T, d_in, d_out):
    """The bf16 epilogue rounds the FP32 accumulator to nearest even: the
    bf16 output equals the oracle's RNE of the same GEMM's FP32 output, bit
    for bit (the tolerance gates alone would not tell RNE from truncation)."""
    x, w, dy = make_inputs(T, d_in, d_out, 21)
    say("bf16 rounding", MODE_NAMES[mode], f"T={T} in={d_in} out={d_out}")
    a, sa, b, sb = device_operands(pf, mode, x, w, dy)
    c32 = pf.gemm_blockscaled(mode, a, sa, b, sb, out_dtype=torch.float32)
    c16 = pf.gemm_blockscaled(mode, a, sa, b, sb, out_dtype=torch.bfloat16)
    want = oracle.f32_to_bf16_bits(host(c32).ravel())
    got = bf16_host_bits(c16).ravel()
    assert np.array_equal(got, want), f"{int(np.sum(got != want))} elements differ"


def test_tiny_forward_workload(pf):
    """X[256x512] N(0,1) with 4 outlier channels x50, W[512x512] N(0,0.02),
    seed 0: the complete output, FP32 and bf16."""
    spec = synth.workload("tiny_fwd").linears[0]
    t = synth.linear_inputs(spec, seed=0, need=("x", "w"))
    say("tiny_fwd workload")
    qa = pf.quant_act(dev(t["x"]), row=True)
    qw = pf.quant_weight(dev(t["w"]), transpose=False)
    y32 = pf.gemm_blockscaled(FWD, qa["q"], qa["s"], qw["q"], qw["s"], out_dtype=torch.float32)
    y16 = pf.gemm_blockscaled(FWD, qa["q"], qa["s"], qw["q"], qw["s"], out_dtype=torch.bfloat16)
    oq, os_ = oracle.quant_rowwise(synth.bits(t["x"]))
    wq, _, ws = oracle.quant_weight(synth.bits(t["w"]), transpose=False)
    ref = oracle.gemm_blockscaled(FWD, oq, os_, wq, ws)
    ii, jj = np.meshgrid(np.arange(ref.shape[0]), np.arange(ref.shape[1]), indexing="ij")
    bound = hw_accum.bounds(FWD, oq, os_, wq, ws, ii.ravel(), jj.ravel(), ref.ravel())
    # outlier channels x50: the named FWD exemption of parity.py
    g = gemm_gates(device_values(y32), ref, bound, False, literal=False)
    say("   fp32 " + fmt(g))
    assert g["ok"], g
    g = gemm_gates(device_values(y16), ref, bound, True, literal=False)
    say("   bf16 " + fmt(g))
    assert g["ok"], g
    exact = oracle.matmul_ref(synth.bits(t["x"]), synth.bits(t["w"]))
    say(f"   vs unquantized matmul: rel_fro={oracle.rel_fro(host(y32), exact):.3e}")


def test_closed_form_scaled_identity(pf):
    """W = 3.5 I quantizes to codes 0x7E with s = 2^-7 on the diagonal blocks;
    Y = X W^T equals the oracle bit for bit (one rounding per element)."""
    x = random_bf16((384, 512), seed=3, stream="ident/x")
    w = torch.zeros((512, 512), dtype=torch.float32)
    w.fill_diagonal_(3.5)
    w = w.to(torch.bfloat16)
    say("closed form 3.5 I")
    qa = pf.quant_act(dev(x), row=True)
    qw = pf.quant_weight(dev(w), transpose=False)
    y = pf.gemm_blockscaled(FWD, qa["q"], qa["s"], qw["q"], qw["s"], out_dtype=torch.float32)
    oq, os_ = oracle.quant_rowwise(synth.bits(x))
    wq, _, ws = oracle.quant_weight(synth.bits(w), transpose=False)
    ref = oracle.gemm_blockscaled(FWD, oq, os_, wq, ws)
    assert np.array_equal(host(y).view(np.uint32), ref.view(np.uint32))


def test_empty_tokens(pf):
    a = torch.empty((0, 256), dtype=torch.uint8, device="cuda:0")
    sa = torch.empty((2, 0), dtype=torch.float32, device="cuda:0")
    b = torch.zeros((256, 256), dtype=torch.uint8, device="cuda:0")
    sb = torch.zeros((2, 2), dtype=torch.float32, device="cuda:0")
    c = pf.gemm_blockscaled(FWD, a, sa, b, sb, out_dtype=torch.bfloat16)
    assert c.shape == (0, 256)


def test_gemm_deterministic(pf):
    x, w, dy = make_inputs(2048, 1024, 2048, 11)
    for mode in (FWD, WGRAD):
        say("gemm determinism", mode)
        a, sa, b, sb = device_operands(pf, mode, x, w, dy)
        c1 = pf.gemm_blockscaled(mode, a, sa, b, sb, out_dtype=torch.float32)
        c2 = pf.gemm_blockscaled(mode, a, sa, b, sb, out_dtype=torch.float32)
        assert torch.equal(c1, c2)


# ---- full transformer-shaped sizes, sampled outputs ----------------------------

def _sampled_check(mode, c_dev, out_dtype, oa, osa, ob, osb, n_samples, seed, literal=True):
    mode = ORACLE_MODE[mode]                         # the same products
    M, N = c_dev.shape
    rng = np.random.default_rng(seed)
    ii = rng.integers(0, M, n_samples)
    jj = rng.integers(0, N, n_samples)
    # whole first and last rows, and a whole column
    ii = np.concatenate([ii, np.zeros(N, np.int64), np.full(N, M - 1), np.arange(M)])
    jj = np.concatenate([jj, np.arange(N), np.arange(N), np.full(M, N // 2)])
    ref = oracle.gemm_blockscaled_at(mode, oa, osa, ob, osb, ii, jj)
    bound = hw_accum.bounds(mode, oa, osa, ob, osb, ii, jj, ref)
    return gemm_gates(device_values(c_dev)[ii, jj], ref, bound, out_dtype == torch.bfloat16,
                      literal=literal)


def _unquantized_at(mode, t, ii, jj, chunk=512):
    """The product of the unquantized bf16 operands at (ii[s], jj[s]), in
    double: the error of the whole FP8 path against a plain matmul is
    reported, not gated (the pages give no bound for it)."""
    if mode in (FWD, FWD_T):           # Y[i,j] = x[i,:] . w[j,:]
        L, R = t["x"].float().numpy(), t["w"].float().numpy()
    elif mode in (DGRAD, DGRAD_W):     # dX[i,j] = dy[i,:] . w[:,j]
        L, R = t["dy"].float().numpy(), t["w"].float().numpy().T
    else:                              # dW[i,j] = dy[:,i] . x[:,j]
        L, R = t["dy"].float().numpy().T, t["x"].float().numpy().T
    out = np.empty(len(ii), np.float64)
    for s0 in range(0, len(ii), chunk):
        li = L[ii[s0:s0 + chunk]].astype(np.float64)
        rj = R[jj[s0:s0 + chunk]].astype(np.float64)
        out[s0:s0 + chunk] = np.einsum("sk,sk->s", li, rj)
    return out


@pytest.mark.parametrize("name,mode,out_dtype", [
    ("qkv_fwd", FWD, torch.bfloat16),
    ("upgate_fwd", FWD, torch.bfloat16),
    ("down_bwd", DGRAD, torch.bfloat16),
    ("down_bwd", DGRAD_W, torch.bfloat16),
    ("down_bwd", WGRAD, torch.float32),
])
def test_workload_full_size_sampled(pf, name, mode, out_dtype):
    spec = synth.workload(name).linears[0]
    need = {FWD: ("x", "w"), DGRAD: ("w", "dy"), DGRAD_W: ("w", "dy"), WGRAD: ("x", "dy")}[mode]
    t = synth.linear_inputs(spec, seed=0, need=need)
    say("full-size", name, MODE_NAMES[mode])
    a, sa, b, sb = device_operands(pf, mode, t.get("x"), t.get("w"), t.get("dy"))
    c = pf.gemm_blockscaled(mode, a, sa, b, sb, out_dtype=out_dtype)
    oa, osa, ob, osb = oracle_operands(mode, t.get("x"), t.get("w"), t.get("dy"))
    assert np.array_equal(host(sa).view(np.uint32), osa.view(np.uint32))
    assert np.array_equal(host(sb).view(np.uint32), osb.view(np.uint32))
    # FWD reads X with outlier channels (QKV) or Student-t(3) tails (up/gate):
    # the named exemption of parity.py
    g = _sampled_check(mode, c, out_dtype, oa, osa, ob, osb, 20000, 1, literal=mode != FWD)
    say("   sampled " + fmt(g))
    assert g["ok"], g
    rng = np.random.default_rng(5)
    ii = rng.integers(0, c.shape[0], 4000)
    jj = rng.integers(0, c.shape[1], 4000)
    exact = _unquantized_at(mode, t, ii, jj)
    say(f"   vs unquantized matmul (4000 samples): "
        f"rel_fro={oracle.rel_fro(device_values(c)[ii, jj], exact):.3e}")


def test_block_stack_wgrad_split_sampled(pf):
    """out-proj weight gradient of the transformer-block workload:
    dW [2048 x 2048] over 32768 tokens, the split-K launch."""
    spec = synth.workload("block_stack").linears[1]
    t = synth.linear_inputs(spec, seed=0, need=("x", "dy"))
    say("block_stack out_proj wgrad (split-K)")
    a, sa, b, sb = device_operands(pf, WGRAD, t["x"], None, t["dy"])
    assert pf.puro_fp8_gemm_workspace_bytes(WGRAD, a.shape[0], b.shape[0], a.shape[1]) > 0
    c = pf.gemm_blockscaled(WGRAD, a, sa, b, sb, out_dtype=torch.float32)
    oa, osa, ob, osb = oracle_operands(WGRAD, t["x"], None, t["dy"])
    g = _sampled_check(WGRAD, c, torch.float32, oa, osa, ob, osb, 4000, 2)
    say("   sampled " + fmt(g))
    assert g["ok"], g


@pytest.mark.parametrize("linear,mode,out_dtype", [
    (0, FWD, torch.bfloat16),       # QKV forward, M = 32768 tokens
    (0, FWD_T, torch.bfloat16),     # the same from the transposed weight codes
    (2, DGRAD, torch.bfloat16),     # up/gate dgrad, dX [32768 x 2048], K = 16384
    (2, DGRAD_W, torch.bfloat16),   # the same from the weight's own codes
    (2, WGRAD, torch.float32),      # up/gate wgrad, dW [16384 x 2048], K = 32768 tokens
    # the step's other launches: with the two above and the split out-proj
    # wgrad, every GEMM the benchmark step runs is checked at its own shape
    (0, DGRAD_W, torch.bfloat16),   # QKV dgrad, K = 6144
    (0, WGRAD, torch.float32),      # QKV wgrad, dW [6144 x 2048]: split-K
    (1, FWD, torch.bfloat16),       # out-proj forward, 2048 -> 2048
    (1, DGRAD_W, torch.bfloat16),
    (2, FWD, torch.bfloat16),       # up/gate forward, Y [32768 x 16384]
    (3, FWD, torch.bfloat16),       # down forward, K = 8192
    (3, DGRAD_W, torch.bfloat16),   # down dgrad, dX [32768 x 8192]
    (3, WGRAD, torch.float32),      # down wgrad, dW [2048 x 8192]
])
def test_block_stack_headline_sampled(pf, linear, mode, out_dtype):
    """The transformer-block workload's own shapes (32768 tokens), quantized
    and multiplied in the launch configuration the benchmark step uses;
    20,000 random elements plus whole rows and a column against the oracle."""
    spec = synth.workload("block_stack").linears[linear]
    need = {FWD: ("x", "w"), FWD_T: ("x", "w"), DGRAD: ("w", "dy"), DGRAD_W: ("w", "dy"),
            WGRAD: ("x", "dy")}[mode]
    t = synth.linear_inputs(spec, seed=0, need=need)
    say("block_stack", spec.name, MODE_NAMES[mode], f"T={spec.tokens} in={spec.d_in} out={spec.d_out}")
    a, sa, b, sb = device_operands(pf, mode, t.get("x"), t.get("w"), t.get("dy"))
    c = pf.gemm_blockscaled(mode, a, sa, b, sb, out_dtype=out_dtype)
    oa, osa, ob, osb = oracle_operands(mode, t.get("x"), t.get("w"), t.get("dy"))
    assert np.array_equal(host(sa).view(np.uint32), osa.view(np.uint32))
    assert np.array_equal(host(sb).view(np.uint32), osb.view(np.uint32))
    # block inputs have outlier channels: FWD is the named exemption of parity.py
    g = _sampled_check(mode, c, out_dtype, oa, osa, ob, osb, 20000, 3,
                       literal=ORACLE_MODE[mode] != FWD)
    say("   sampled " + fmt(g))
    assert g["ok"], g


def test_operand_offsets_beyond_4gib(pf):
    """A [1280 x 2^22] codes (5 GiB): rows 1024 and up start more than 2^32
    bytes into A.  Only a few rows of A and B hold codes (seeded, both signs);
    every other output element is exactly zero, so a wrong row offset shows
    either as a mismatch or as a non-zero where zero is due."""
    M, N, K = 1280, 256, 1 << 22
    rows = np.array([0, 1, 700, 1100, 1279])
    cols = np.array([0, 5, 255])
    rng = np.random.default_rng(7)

    def codes(n):
        c = rng.integers(0, 0xFF, (n, K), dtype=np.uint8)
        c[c == 0x7F] = 0x7E                      # no NaN codes
        return c

    a_rows, b_rows = codes(len(rows)), codes(len(cols))
    sa = rng.uniform(0.5, 2.0, (K // 128, M)).astype(np.float32)
    sb = rng.uniform(0.5, 2.0, (N // 128, K // 128)).astype(np.float32)
    say("large offsets: FWD M=1280 N=256 K=2^22")
    A = torch.zeros((M, K), dtype=torch.uint8, device="cuda:0")
    A[torch.from_numpy(rows).cuda()] = torch.from_numpy(a_rows).cuda()
    B = torch.zeros((N, K), dtype=torch.uint8, device="cuda:0")
    B[torch.from_numpy(cols).cuda()] = torch.from_numpy(b_rows).cuda()
    c = pf.gemm_blockscaled(FWD, A, dev(torch.from_numpy(sa)), B, dev(torch.from_numpy(sb)),
                            out_dtype=torch.float32)
    got = host(c)
    del A, B
    a = np.zeros((M, K), np.uint8)
    a[rows] = a_rows
    b = np.zeros((N, K), np.uint8)
    b[cols] = b_rows
    ii, jj = (g.ravel() for g in np.meshgrid(rows, cols, indexing="ij"))
    ref = oracle.gemm_blockscaled_at(FWD, a, sa, b, sb, ii, jj)
    bound = hw_accum.bounds(FWD, a, sa, b, sb, ii, jj, ref, chunk=1)
    # codes drawn over the whole E4M3 range: the named exemption of parity.py
    g = gemm_gates(got[ii, jj], ref, bound, False, literal=False)
    say("   " + fmt(g))
    assert g["ok"], g
    nonzero = np.zeros((M, N), bool)
    nonzero[ii, jj] = True
    assert not np.any(got[~nonzero]), "output outside the populated rows/columns is not zero"


# ---- persistent launch: several units per work-group ---------------------------

def _operands_codes(rng, M, N, K, mode):
    """Random E4M3 codes (both signs, no NaN) and positive scales in the
    layouts of `mode`, host and device copies."""
    def codes(r, c):
        q = rng.integers(0, 0xFF, (r, c), dtype=np.uint8)
        q[(q & 0x7F) == 0x7F] = 0x7E
        return q
    a, b = codes(M, K), codes(N, K)
    sa = rng.uniform(0.25, 4.0, (K // 128, M)).astype(np.float32)
    sb_shape = {FWD: (N // 128, K // 128), DGRAD: (K // 128, N // 128), WGRAD: (K // 128, N)}[mode]
    sb = rng.uniform(0.25, 4.0, sb_shape).astype(np.float32)
    return a, sa, b, sb


@pytest.mark.parametrize("mode,M,N,K,out_dtype,accumulate", [
    (FWD, 70000, 1152, 512, torch.bfloat16, False),    # ragged M, half-inactive last column
    (DGRAD, 70000, 1152, 512, torch.float32, False),
    (FWD, 70000, 1152, 128, torch.bfloat16, False),    # one K-block per unit: an epilogue every step
    (DGRAD, 40000, 2048, 128, torch.bfloat16, False),
    (WGRAD, 8192, 8192, 256, torch.float32, False),    # 1024 units, 4 per work-group
    (WGRAD, 8192, 8192, 256, torch.float32, True),
    (WGRAD, 4000, 4224, 1024, torch.bfloat16, False),  # ragged M, N % 256 == 128
])
def test_persistent_multi_unit(pf, mode, M, N, K, out_dtype, accumulate):
    """More output tiles than compute units: every work-group runs several
    units back to back (the next unit's first K-block staged during the
    previous unit's last one, its epilogue overlapped with the next block).
    Sampled elements, whole first / last rows and a whole column."""
    rng = np.random.default_rng(M + N + K + mode)
    a, sa, b, sb = _operands_codes(rng, M, N, K, mode)
    say("persistent multi-unit", MODE_NAMES[mode], M, N, K, out_dtype,
        "acc" if accumulate else "")
    out = None
    c0 = None
    if accumulate:
        c0 = rng.normal(0.0, 1.0, (M, N)).astype(np.float32)
        out = dev(torch.from_numpy(c0))
    c = pf.gemm_blockscaled(mode, dev(torch.from_numpy(a)), dev(torch.from_numpy(sa)),
                            dev(torch.from_numpy(b)), dev(torch.from_numpy(sb)),
                            out_dtype=out_dtype, out=out, accumulate=accumulate)
    ii = rng.integers(0, M, 6000)
    jj = rng.integers(0, N, 6000)
    ii = np.concatenate([ii, np.zeros(N, np.int64), np.full(N, M - 1), np.arange(M)])
    jj = np.concatenate([jj, np.arange(N), np.arange(N), np.full(M, N - 1)])
    ref = oracle.gemm_blockscaled_at(mode, a, sa, b, sb, ii, jj)
    bound = hw_accum.bounds(mode, a, sa, b, sb, ii, jj, ref)
    if accumulate:
        ref = (c0[ii, jj] + ref).astype(np.float32)
        extra = 2.0 ** -22 * np.abs(ref)
        bound = (bound[0] + extra, bound[1] + extra)
    # codes drawn over the whole E4M3 range: the named exemption of parity.py
    g = gemm_gates(device_values(c)[ii, jj], ref, bound, out_dtype == torch.bfloat16,
                   literal=False)
    say("   " + fmt(g))
    assert g["ok"], g


@pytest.mark.parametrize("M,N,K,out_dtype", [
    (70000, 1152, 512, torch.bfloat16),     # several units per work-group, half last tile
    (40000, 2048, 128, torch.float32),      # one K-block per unit
    (3000, 384, 8192, torch.float32),       # split-K
])
@pytest.mark.parametrize("mode", [DGRAD, FWD])
def test_kn_modes_equal_on_random_codes(pf, M, N, K, out_dtype, mode):
    """Codes over the whole E4M3 range: DGRAD_W / FWD_T on b^T [K][N] give
    DGRAD's / FWD's result on b [N][K] bit for bit, through the persistent
    multi-unit walk, half-empty last column tiles and the split-K path."""
    rng = np.random.default_rng(M + N + K)
    a, sa, b, sb = _operands_codes(rng, M, N, K, mode)
    kn = DGRAD_W if mode == DGRAD else FWD_T
    say(MODE_NAMES[kn], "vs", MODE_NAMES[mode], "random codes", M, N, K, out_dtype)
    ad, sad, sbd = dev(torch.from_numpy(a)), dev(torch.from_numpy(sa)), dev(torch.from_numpy(sb))
    c1 = pf.gemm_blockscaled(mode, ad, sad, dev(torch.from_numpy(b)), sbd, out_dtype=out_dtype)
    c2 = pf.gemm_blockscaled(kn, ad, sad, dev(torch.from_numpy(np.ascontiguousarray(b.T))),
                             sbd, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)


# ---- streams and host threads ---------------------------------------------------

def _layer_on_stream(pf, x, w, stream):
    with torch.cuda.stream(stream):
        qa = pf.quant_act(x, row=True)
        qw = pf.quant_weight(w, transpose=False)
        y = pf.gemm_blockscaled(FWD, qa["q"], qa["s"], qw["q"], qw["s"], out_dtype=torch.bfloat16)
    return y


def test_non_default_stream_and_host_threads(pf):
    """Every call runs on the stream it is given (torch's current stream in
    the binding): a layer on a side stream, and four host threads each
    driving its own stream, reproduce the default-stream result bit for bit
    (the library keeps no mutable global state)."""
    import threading
    inputs = [make_inputs(1024, 1024, 1536, 40 + i)[:2] for i in range(4)]
    inputs = [(dev(x), dev(w)) for x, w in inputs]
    say("streams / host threads")
    ref = [_layer_on_stream(pf, x, w, torch.cuda.current_stream()) for x, w in inputs]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    got = _layer_on_stream(pf, inputs[0][0], inputs[0][1], side)
    side.synchronize()
    assert torch.equal(got.view(torch.int16), ref[0].view(torch.int16))
    results = [None] * 4
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            for _ in range(3):
                results[i] = _layer_on_stream(pf, inputs[i][0], inputs[i][1], s)
            s.synchronize()
        except Exception as e:          # reported below
            errors.append(e)
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i in range(4):
        assert torch.equal(results[i].view(torch.int16), ref[i].view(torch.int16)), i
