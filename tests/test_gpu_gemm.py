"""GPU bf16 products (the projections of one draft layer) against the fp64
product of the exact bf16 inputs: all three layouts, ragged edges in M, N and
K, fp32 and bf16 outputs, bias and accumulation."""
import numpy as np
import pytest
import torch

from block_sparse_cross_amd import binding, inputs
from tests.helpers import assert_close_f32, to_dev, to_f64, vals64

pytestmark = pytest.mark.gpu

NT, NN, TN = binding.SPLITKV_GEMM_NT, binding.SPLITKV_GEMM_NN, binding.SPLITKV_GEMM_TN


def operands(layout, M, N, K, seed):
    sa = (M, K) if layout != TN else (K, M)
    sb = (N, K) if layout == NT else (K, N)
    A = inputs.gen_matrix(sa[0], sa[1], seed, inputs.T_MAT, 1.0)
    B = inputs.gen_matrix(sb[0], sb[1], seed + 1, inputs.T_MAT, K ** -0.5)
    a, b = vals64(A), vals64(B)
    ref = (a if layout != TN else a.T) @ (b.T if layout == NT else b)
    return A, B, ref


def assert_close_bf16_out(got, ref, what):
    # one bf16 rounding of the fp32 result: |err| <= 2^-8 |ref| (+ fp32 accumulation)
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-4 * np.abs(ref).max()
    assert (err <= bound).all(), "%s: worst excess %.3e" % (what, float((err - bound).max()))


SHAPES = [(256, 256, 64), (8, 8, 8), (264, 136, 72), (1000, 520, 1032), (512, 768, 40),
          (2048, 1536, 2048)]


@pytest.mark.parametrize("layout", [NT, NN, TN])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_fp32_out(layout, M, N, K):
    A, B, ref = operands(layout, M, N, K, seed=M + N + K)
    C = binding.splitkv_gemm(layout, to_dev(A), to_dev(B))
    torch.cuda.synchronize()
    assert_close_f32(to_f64(C), ref, "gemm %d %dx%dx%d" % (layout, M, N, K))


@pytest.mark.parametrize("layout", [NT, NN, TN])
def test_gemm_bf16_out_bias_accumulate(layout):
    M, N, K = 392, 264, 328
    A, B, ref = operands(layout, M, N, K, seed=5)
    bias = np.random.default_rng(5).standard_normal(N).astype(np.float32)
    C0 = inputs.gen_matrix(M, N, 9, inputs.T_MAT, 1.0, dtype="fp32")
    Cd = to_dev(C0)
    binding.splitkv_gemm(layout, to_dev(A), to_dev(B), out=Cd, bias=to_dev(bias),
                         accumulate=True)
    Cb = binding.splitkv_gemm(layout, to_dev(A), to_dev(B), out_dtype=torch.bfloat16,
                              bias=to_dev(bias))
    torch.cuda.synchronize()
    assert_close_f32(to_f64(Cd), ref + bias[None, :] + C0, "accumulate + bias")
    assert_close_bf16_out(to_f64(Cb), ref + bias[None, :], "bf16 out + bias")


def test_gemm_sum_of_products_with_bias_once():
    # Eq. 5 shape: four products accumulated into one fp32 output, bias once
    M, N, K = 264, 520, 256
    C = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    bias = np.linspace(-1, 1, N).astype(np.float32)
    ref = np.zeros((M, N)) + bias[None, :]
    for p in range(4):
        A, B, r = operands(NT, M, N, K, seed=100 + 7 * p)
        binding.splitkv_gemm(NT, to_dev(A), to_dev(B), out=C, accumulate=True,
                             bias=to_dev(bias) if p == 0 else None)
        ref += r
    torch.cuda.synchronize()
    assert_close_f32(to_f64(C), ref, "sum of products")


def test_gemm_rejects_bad_shapes():
    x = torch.zeros((16, 12), dtype=torch.bfloat16, device="cuda")
    out = torch.full((16, 16), 3.0, dtype=torch.float32, device="cuda")
    st = binding.lib().splitkv_gemm(NT, 16, 16, 12, x.data_ptr(), x.data_ptr(), out.data_ptr(),
                                    binding.SPLITKV_FP32, None, 0, None)
    assert st == binding.SPLITKV_ERR_INVALID_ARG   # K % 8 != 0
    st = binding.lib().splitkv_gemm(7, 16, 16, 16, x.data_ptr(), x.data_ptr(), out.data_ptr(),
                                    binding.SPLITKV_FP32, None, 0, None)
    assert st == binding.SPLITKV_ERR_INVALID_ARG   # unknown layout
    torch.cuda.synchronize()
    assert (out == 3.0).all()


# Few output tiles and a long K: the K range is split over workgroups whose
# partial products are added into C atomically (the weight-gradient shapes).
@pytest.mark.parametrize("layout", [NT, NN, TN])
@pytest.mark.parametrize("M,N,K", [(256, 256, 2048), (1024, 512, 16384), (264, 8, 8200),
                                   (512, 1032, 4104)])
def test_gemm_split_k(layout, M, N, K):
    A, B, ref = operands(layout, M, N, K, seed=3 * M + N + K)
    bias = np.linspace(-2, 2, N).astype(np.float32)
    C = binding.splitkv_gemm(layout, to_dev(A), to_dev(B), bias=to_dev(bias))
    C0 = inputs.gen_matrix(M, N, 4, inputs.T_MAT, 1.0, dtype="fp32")
    Ca = to_dev(C0)
    binding.splitkv_gemm(layout, to_dev(A), to_dev(B), out=Ca, accumulate=True)
    torch.cuda.synchronize()
    assert_close_f32(to_f64(C), ref + bias[None, :], "split-K")
    assert_close_f32(to_f64(Ca), ref + C0, "split-K accumulate")


# More tiles than one round of the chip with a part-filled last round: the
# tiles of the full rounds keep all of K (plain stores), the last round's tiles
# split K (atomic adds), in one launch. 257 tiles: one tail tile in 4 splits;
# 320 tiles (the per-rank dWo shape with a shorter K): 64 tail tiles in 4.
@pytest.mark.parametrize("layout", [NT, NN, TN])
@pytest.mark.parametrize("M,N,K", [(256 * 257, 256, 2048), (5120, 4096, 2048), (3000, 5904, 1088)])
def test_gemm_tail_split(layout, M, N, K):
    A, B, ref = operands(layout, M, N, K, seed=M + K + layout)
    bias = np.random.default_rng(4).standard_normal(N).astype(np.float32)
    C = binding.splitkv_gemm(layout, to_dev(A), to_dev(B), bias=to_dev(bias))
    C0 = inputs.gen_matrix(M, N, 7, inputs.T_MAT, 1.0, dtype="fp32")
    Ca = to_dev(C0)
    binding.splitkv_gemm(layout, to_dev(A), to_dev(B), out=Ca, accumulate=True)
    torch.cuda.synchronize()
    assert_close_f32(to_f64(C), ref + bias[None, :], "tail split")
    assert_close_f32(to_f64(Ca), ref + C0, "tail split accumulate")


@pytest.mark.parametrize("layout", [NT, NN, TN])
@pytest.mark.parametrize("M,N,K", [(264, 520, 128), (1032, 512, 1024), (256, 256, 4096)])
def test_gemm_pair(layout, M, N, K):
    # op(A1) op(B1) + op(A2) op(B2) in one pass (incl. the split-K case 256 x 256)
    A1, B1, r1 = operands(layout, M, N, K, seed=11 + M)
    A2, B2, r2 = operands(layout, M, N, K, seed=12 + N)
    bias = np.linspace(-1, 1, N).astype(np.float32)
    C = binding.splitkv_gemm_pair(layout, to_dev(A1), to_dev(B1), to_dev(A2), to_dev(B2),
                                  bias=to_dev(bias))
    C0 = inputs.gen_matrix(M, N, 5, inputs.T_MAT, 1.0, dtype="fp32")
    Ca = to_dev(C0)
    binding.splitkv_gemm_pair(layout, to_dev(A1), to_dev(B1), to_dev(A2), to_dev(B2), out=Ca,
                              accumulate=True)
    torch.cuda.synchronize()
    assert_close_f32(to_f64(C), r1 + r2 + bias[None, :], "pair")
    assert_close_f32(to_f64(Ca), r1 + r2 + C0, "pair accumulate")


def test_gemm_pair_rejects_k_not_multiple_of_64():
    x = torch.zeros((16, 72), dtype=torch.bfloat16, device="cuda")
    out = torch.full((16, 16), 3.0, dtype=torch.float32, device="cuda")
    st = binding.lib().splitkv_gemm_pair(NT, 16, 16, 72, x.data_ptr(), x.data_ptr(),
                                         x.data_ptr(), x.data_ptr(), out.data_ptr(),
                                         binding.SPLITKV_FP32, None, 0, None)
    assert st == binding.SPLITKV_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert (out == 3.0).all()


@pytest.mark.parametrize("layout", [NT, NN, TN])
def test_gemm_bf16_accumulate(layout):
    # C bf16 read, added to, rounded once: C = bf16(C0 + A B)
    M, N, K = 136, 264, 192
    A, B, ref = operands(layout, M, N, K, seed=21)
    C0 = inputs.gen_matrix(M, N, 22, inputs.T_MAT, 1.0)          # bf16 bits
    Cd = to_dev(C0)
    binding.splitkv_gemm(layout, to_dev(A), to_dev(B), out=Cd, accumulate=True)
    torch.cuda.synchronize()
    assert_close_bf16_out(to_f64(Cd), ref + vals64(C0), "bf16 accumulate")
