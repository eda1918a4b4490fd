// Host-side validation and scratch layout shared by the entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moonep.h"

namespace moonep {

inline int64_t i64(int32_t v) { return (int64_t)v; }

// Checks every requirement the header states for a configuration.
inline int check_cfg(const moe_cfg* c) {
  if (!c) return MOE_EINVAL;
  if (c->R < 1 || c->S < 0 || c->E < 1 || c->K < 1 || c->H < 8 || c->Hp < 8 || c->B < 0)
    return MOE_EINVAL;
  if (c->mode != MOE_MODE_TRAIN && c->mode != MOE_MODE_INFER) return MOE_EINVAL;
  if (c->E % c->R != 0 || c->K > c->E) return MOE_EINVAL;
  if (c->H % 8 != 0 || c->Hp % 8 != 0) return MOE_EINVAL;
  const int n = c->E / c->R;
  if (c->mode == MOE_MODE_TRAIN && c->B != n) return MOE_EINVAL;
  if (c->B > n) return MOE_EINVAL;
  if (c->E > MOE_MAX_E || c->R > MOE_MAX_R || c->K > MOE_MAX_K) return MOE_ELIMIT;
  if (i64(c->R) * i64(c->S) * i64(c->K) >= (int64_t(1) << 31)) return MOE_ELIMIT;
  // dispatch and its backward run one 256-thread workgroup per token, and one
  // launch holds fewer than 2^32 threads
  if (i64(c->R) * i64(c->S) >= (int64_t(1) << 24)) return MOE_ELIMIT;
  // byte extents the GEMM's 32-bit buffer offsets cover: one weight matrix,
  // and one rank's permuted rows
  const int64_t wide = c->H > c->Hp ? c->H : c->Hp;
  if (i64(c->H) * c->Hp * 2 >= (int64_t(1) << 32)) return MOE_ELIMIT;
  if (i64(c->S) * c->K * wide * 2 >= (int64_t(1) << 32)) return MOE_ELIMIT;
  return MOE_OK;
}

inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// Every bf16 / fp32 tensor is moved in 16-byte vectors (and the GEMMs load
// 16 bytes per lane straight into LDS), so tensor bases must be 16-byte
// aligned.  A null pointer passes (null checks are separate).
template <typename... P>
inline bool aligned16(const P*... p) {
  return (((reinterpret_cast<uintptr_t>(p) & 15) == 0) && ...);
}

// Plan scratch: chunk counts and the per-expert tables k_route reads.
struct PlanLayout {
  int64_t N;      // R*S*K slots
  int L;          // slots per wave sub-chunk (multiple of 64)
  int C;          // chunks of 16 sub-chunks (one workgroup each)
  int M;          // move capacity E + R - 1
  size_t off_cc, off_badc, off_taken, off_home_base, off_mptr, off_mcnt, off_cs_lo, off_cs_hi,
      off_cs_base, off_cs_dst, off_cs_b, off_cons, off_hpre, off_spre, off_rinfo, off_ocum,
      off_misc, bytes;
};

constexpr int kRouteWaves = 16;
constexpr size_t kMaxLds = 160 * 1024;   // LDS per workgroup on gfx950
#ifndef MOONEP_PLAN_CHUNKS
#define MOONEP_PLAN_CHUNKS 256
#endif
constexpr int kMaxChunks = MOONEP_PLAN_CHUNKS;

inline PlanLayout plan_layout(const moe_cfg* c) {
  PlanLayout p{};
  p.N = i64(c->R) * c->S * c->K;
  const int64_t per = int64_t(kRouteWaves) * 64 * kMaxChunks;
  p.L = (int)(64 * (p.N > 0 ? (p.N + per - 1) / per : 1));
  const int64_t ch = int64_t(kRouteWaves) * p.L;
  p.C = (int)((p.N + ch - 1) / ch);
  p.M = c->E + c->R - 1;
  size_t o = 0;
  auto take = [&](size_t ints) { size_t at = o; o += align256(ints * 4); return at; };
  p.off_cc = take(size_t(p.C > 0 ? p.C : 1) * c->E);
  p.off_badc = take(p.C > 0 ? p.C : 1);
  p.off_taken = take(c->E);
  p.off_home_base = take(c->E);
  p.off_mptr = take(c->E);
  p.off_mcnt = take(c->E);
  p.off_cs_lo = take(p.M);
  p.off_cs_hi = take(p.M);
  p.off_cs_base = take(p.M);
  p.off_cs_dst = take(p.M);
  p.off_cs_b = take(p.M);
  p.off_cons = take(c->E);
  p.off_hpre = take(size_t(c->E) + c->R);                 // R * (E/R + 1)
  p.off_spre = take(size_t(c->R) * (c->B + 1));
  p.off_rinfo = take(size_t(3) * c->R);
  p.off_ocum = take(p.M);
  p.off_misc = take(64);
  p.bytes = o;
  return p;
}

inline int32_t* ws_i32(void* ws, size_t off) {
  return reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + off);
}

inline int plan_ptrs_ok(const moe_plan* p) {
  return p && p->counts && p->load0 && p->cu_seqlens && p->slot_expert && p->n_redundant &&
         p->src_rank && p->moves && p->status && p->workspace;
}

inline int hip_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : MOE_EHIP;
}

// Raises a kernel's dynamic LDS limit once (needed above 64 KB on gfx950).
template <typename F>
inline int allow_lds(F* kernel, size_t bytes) {
  if (bytes > kMaxLds) return MOE_ELIMIT;
  if (bytes <= 65536) return MOE_OK;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  return e == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace moonep
