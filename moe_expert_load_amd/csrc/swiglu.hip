// Backward of the SwiGLU activation of the two-projection expert.
//
// Source: "Moonshot AI 开源 MoonEP", 核心思想 (each expert projection is one
// contiguous [E+B, H_in, H_out] tensor; H' is the FFN intermediate size).
// The forward, act = silu(gate) * up, is fused into the first projection's
// GEMM epilogue (gemm.hip); its gradients need the stored gate and up:
//   d up   = d act * gate * s
//   d gate = d act * up * s * (1 + gate * (1 - s)),   s = 1 / (1 + e^-gate).
// Pure streaming: per row, 2H' bf16 of h13 and H' of d act in, 2H' out.
// One thread handles 8 columns (16-byte pieces of d act, gate, up, d gate
// and d up) of two rows at once, all six loads issued before any math; a
// workgroup walks whole rows so no index needs a division.  sigmoid uses the
// hardware reciprocal (1 ulp), far inside the bf16 rounding of the outputs.
#include "common.hpp"
#include "host.hpp"

namespace moonep {

constexpr int kSwiThreads = 256;

__device__ __forceinline__ void swiglu_grad(float g, float u, float d, float& dg, float& du) {
  const float s = __builtin_amdgcn_rcpf(1.f + __expf(-g));
  du = d * g * s;
  dg = d * u * s * (1.f + g * (1.f - s));
}

__global__ __launch_bounds__(kSwiThreads) void k_swiglu_bwd(const uint16_t* h13,
                                                          const uint16_t* dact, uint16_t* dh13,
                                                          int64_t rows, int Hp) {
  const int cpr = Hp / 8;                        // 16-byte pieces per d act row
  for (int64_t r0 = 2 * int64_t(blockIdx.x); r0 < rows; r0 += 2 * int64_t(gridDim.x)) {
    const int nr = r0 + 1 < rows ? 2 : 1;        // uniform per workgroup
    for (int c = threadIdx.x; c < cpr; c += kSwiThreads) {
      u32x4 gw[2], uw[2], dw[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if (k < nr) {
          const int64_t r = r0 + k;
          gw[k] = *reinterpret_cast<const u32x4*>(h13 + r * 2 * Hp + 8 * c);
          uw[k] = *reinterpret_cast<const u32x4*>(h13 + r * 2 * Hp + Hp + 8 * c);
          dw[k] = *reinterpret_cast<const u32x4*>(dact + r * Hp + 8 * c);
        }
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if (k < nr) {
          u32x4 og, ou;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float g0, u0, g1, u1;
            swiglu_grad(bf16_lo(gw[k][q]), bf16_lo(uw[k][q]), bf16_lo(dw[k][q]), g0, u0);
            swiglu_grad(bf16_hi(gw[k][q]), bf16_hi(uw[k][q]), bf16_hi(dw[k][q]), g1, u1);
            og[q] = pack_bf16x2(g0, g1);
            ou[q] = pack_bf16x2(u0, u1);
          }
          uint16_t* orow = dh13 + (r0 + k) * 2 * Hp;
          *reinterpret_cast<u32x4*>(orow + 8 * c) = og;
          *reinterpret_cast<u32x4*>(orow + Hp + 8 * c) = ou;
        }
      }
    }
  }
}

}  // namespace moonep

using namespace moonep;

extern "C" int moe_swiglu_backward(const moe_cfg* cfg, const moe_bf16* h13, const moe_bf16* dact,
                                   moe_bf16* dh13, hipStream_t stream) {
  const int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  const int64_t rows = int64_t(cfg->R) * cfg->S * cfg->K;
  if (rows == 0) return MOE_OK;
  if (!h13 || !dact || !dh13) return MOE_EINVAL;
  // in place (dh13 == h13) is allowed: every piece is read before the same
  // thread writes it; any other overlap with the inputs is not
  const uintptr_t o0 = reinterpret_cast<uintptr_t>(dh13);
  const uintptr_t o1 = o0 + size_t(rows) * 2 * cfg->Hp * 2;
  const uintptr_t d0 = reinterpret_cast<uintptr_t>(dact);
  const uintptr_t d1 = d0 + size_t(rows) * cfg->Hp * 2;
  const uintptr_t h0 = reinterpret_cast<uintptr_t>(h13);
  if (o0 < d1 && d0 < o1) return MOE_EINVAL;
  if (dh13 != h13 && o0 < h0 + (o1 - o0) && h0 < o1) return MOE_EINVAL;
  if (!aligned16(h13, dact, dh13)) return MOE_EINVAL;
  const int64_t pairs = (rows + 1) / 2;
  const int64_t grid = pairs < 4096 ? pairs : 4096;
  hipLaunchKernelGGL(k_swiglu_bwd, dim3((unsigned)grid), dim3(kSwiThreads), 0, stream,
                     reinterpret_cast<const uint16_t*>(h13), reinterpret_cast<const uint16_t*>(dact),
                     reinterpret_cast<uint16_t*>(dh13), rows, cfg->Hp);
  return hip_status();
}
