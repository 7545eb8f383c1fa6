"""Shared set-up for the LoRA-linear GPU tests: seeded inputs, the HIP path through the C ABI,
and the oracle's reference values. Inputs come from layer_streamed_nf4_dequant_amd.inputs; the
oracle sees only those inputs (never a value the HIP path produced)."""

from __future__ import annotations

import numpy as np

from layer_streamed_nf4_dequant_amd import inputs, lib
from oracle import lora as olora
from oracle import nf4 as onf4

TOL = {"Y": 5e-3, "dX": 5e-3, "dA": 1e-2, "dB": 1e-2, "U": 5e-3, "G": 5e-3}


def bf16_dev(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def f32(bits):
    return onf4.bf16_to_f32(bits)


class Case:
    """One LoRA linear with host inputs (bf16 bit patterns / fp32 W) and device copies."""

    def __init__(self, T, K, N, r=16, scale=2.0, seed=0, base="nf4", B_zero=False, tag="case"):
        import torch
        self.T, self.K, self.N, self.r, self.s, self.base = T, K, N, r, scale, base
        key = (tag, T, K, N, r, base)
        self.W = inputs.weight_f32(N, K, seed, *key)
        self.A = inputs.lora_A_bf16(r, K, seed, *key)
        self.B = inputs.lora_B_bf16(N, r, seed, *key)
        if B_zero:
            self.B = np.zeros_like(self.B)
        self.X = inputs.act_bf16(T, K, seed, *key, "X")
        self.dY = inputs.act_bf16(T, N, seed, *key, "dY")
        self.dX_init = inputs.host_normal((T, K), 1.0, seed, *key, "dX0")    # for the F32_ADD mode
        self.g_init = inputs.host_normal((r * K + N * r,), 0.01, seed, *key, "g0")
        # oracle-side base weight: the exact bf16 operand the GEMM must use
        if base == "nf4":
            self.packed = onf4.pack(self.W)
            self.W_hat_bits = onf4.dequant_bf16(self.packed)
        else:
            self.W_hat_bits = inputs.to_bf16_bits(self.W)
        # device side
        self.Xd, self.Ad, self.Bd, self.dYd = (bf16_dev(a, torch) for a in (self.X, self.A, self.B, self.dY))
        if base == "nf4":
            self.Wd = lib.nf4_pack(torch.from_numpy(self.W).cuda())
        else:
            self.Wd = bf16_dev(self.W_hat_bits, torch)
        self.ws = torch.empty(max(lib.ws_bytes(T, K, N, r), 256), dtype=torch.uint8, device="cuda")

    def desc(self, W=None, transposed=False):
        return lib.linear_desc(self.T, self.K, self.N, self.r, self.s, self.Wd if W is None else W,
                               self.Ad, self.Bd, transposed=transposed)

    def w_transposed(self):
        """The bf16 W^T [K][N] the backward's transposed path reads: nf4_dequant's transposed
        output for an NF4 base, else the bf16 W transposed by torch."""
        if self.base == "nf4":
            return lib.nf4_dequant(self.Wd, "bf16_t")
        return self.Wd.t().contiguous()

    def gpu_fwd(self, adapters=True, W=None):
        import torch
        Y = torch.empty((self.T, self.N), dtype=torch.bfloat16, device="cuda")
        U = torch.empty((self.T, self.r), dtype=torch.bfloat16, device="cuda")
        lib.lora_linear_fwd(self.desc(W), self.Xd, Y, U, adapters=adapters, ws=self.ws)
        return Y, U

    def gpu_bwd(self, U, dx_mode=lib.DX_BF16_SET, grad_mode=lib.GRAD_SET, W=None, transposed=False):
        import torch
        if dx_mode == lib.DX_F32_ADD:
            dX = torch.from_numpy(self.dX_init).cuda()
        else:
            dX = torch.empty((self.T, self.K), dtype=torch.bfloat16, device="cuda")
        g0 = torch.from_numpy(self.g_init).cuda()
        dA = g0[: self.r * self.K].view(self.r, self.K).clone()
        dB = g0[self.r * self.K:].view(self.N, self.r).clone()
        lib.lora_linear_bwd(self.desc(W, transposed), self.Xd, self.dYd, U, dX, dA, dB, dx_mode=dx_mode,
                            grad_mode=grad_mode, ws=self.ws)
        return dX, dA, dB

    # ---- oracle ----
    def oracle_fwd(self, rows=None, adapters=True):
        X = f32(self.X) if rows is None else f32(self.X[rows])
        return olora.forward(X, f32(self.W_hat_bits), f32(self.A), f32(self.B), self.s, adapters)

    def oracle_bwd(self):
        return olora.backward(f32(self.X), f32(self.dY), f32(self.W_hat_bits), f32(self.A), f32(self.B),
                              self.s)


def to_np(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def assert_close(name, got, want, tol=None):
    err = olora.rel_l2(got, want)
    tol = TOL[name] if tol is None else tol
    assert err <= tol, f"{name}: rel L2 {err:.3e} > {tol:.1e}"
    return err
