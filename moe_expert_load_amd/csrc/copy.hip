// HBM-bound steps: prefetch_weight, fused permute (dispatch), gate-weighted
// combine and reduce_grad, and the backward of combine and of dispatch.
// Every row moves as 16-byte vectors; a workgroup (dispatch) or a wave
// (combine and the backward kernels) owns a token, so its K routes are read
// once and broadcast with lane shuffles.
//
// Sources: "Kimi K3 模型结构（8）：训练并行，MoonEP 与四类等待", heading
// 在线规划、零拷贝、静态 shape (permute straight into expert-grouped places;
// combine multiplies each expert output by its own fp32 router weight);
// "Moonshot AI 开源 MoonEP", 核心思想 (prefetch_weight fills rows [E, E+B);
// reduce_grad folds each rank's slots of an expert into its home gradient and
// zeroes the consumed slots); "大规模 LLM 训练系统研究账本" §9.5 (the MoE
// backward keeps the permuted layout: the gradients of combine and dispatch
// are the transposed maps of the forward ones).
#include "common.hpp"
#include "host.hpp"

namespace moonep {

// ---------------------------------------------------------------------------
// prefetch: a fixed grid walks the copies of the slots in use.  Each
// workgroup first compacts a window of slot entries (slot id and expert)
// into LDS, in ascending slot order, so every workgroup builds the same list.
// Each used slot is then cut into CH chunks, chunk c moving vectors
// c*256 + tid + k*CH*256 (four per step), and the cnt*CH chunks are dealt
// out over the grid.  CH grows when few slots are used, so the grid stays
// full either way (a grid of (chunk, slot) pairs over every slot leaves most
// workgroups idle when a handful of slots hold an expert).
// ---------------------------------------------------------------------------
constexpr int kPfWin = 1024;   // slot entries compacted per window

__global__ __launch_bounds__(256) void k_prefetch(const u32x4* __restrict__ w_home,
                                                  u32x4* __restrict__ w_pref,
                                                  const int32_t* __restrict__ slot_expert,
                                                  int nslots, int E, int64_t nvec) {
  __shared__ int s_slot[kPfWin], s_exp[kPfWin];
  __shared__ int s_w[4];
  const int tid = threadIdx.x, wv = tid / kWave;
  for (int base = 0; base < nslots; base += kPfWin) {
    __syncthreads();                                          // last window's list is done
    int cnt = 0;
    for (int r0 = 0; r0 < kPfWin && base + r0 < nslots; r0 += 256) {
      const int i = base + r0 + tid;
      const int e = i < nslots ? slot_expert[i] : -1;
      const bool ok = e >= 0 && e < E;
      const uint64_t m = __ballot(ok);
      if (lane_id() == 0) s_w[wv] = __popcll(m);
      __syncthreads();
      int off = cnt, tot = 0;
      for (int x = 0; x < 4; ++x) {
        const int c = s_w[x];
        if (x < wv) off += c;
        tot += c;
      }
      if (ok) {
        const int p = off + __popcll(m & lanemask_lt());
        s_slot[p] = i;
        s_exp[p] = e;
      }
      cnt += tot;
      __syncthreads();                                        // s_w is reused
    }
    if (cnt == 0) continue;
    const int CH = max(64, ((int)gridDim.x + cnt - 1) / cnt);
    const int64_t stride = int64_t(CH) * 256;
    for (int vb = blockIdx.x; vb < cnt * CH; vb += gridDim.x) {
      const int j = vb / CH, c = vb - j * CH;
      const u32x4* src = w_home + int64_t(s_exp[j]) * nvec;
      u32x4* dst = w_pref + int64_t(s_slot[j]) * nvec;
      int64_t v = int64_t(c) * 256 + tid;
      constexpr int U = 4;       // loads in flight per thread (8 and 12 measured the same)
      for (; v + (U - 1) * stride < nvec; v += U * stride) {
        u32x4 a[U];
#pragma unroll
        for (int q = 0; q < U; ++q) a[q] = src[v + q * stride];
#pragma unroll
        for (int q = 0; q < U; ++q) dst[v + q * stride] = a[q];   // plain stores: 7 % faster here
      }
      for (; v < nvec; v += stride) dst[v] = src[v];
    }
  }
}

// ---------------------------------------------------------------------------
// dispatch: one workgroup per token; its 4 waves split the row (Q vectors per
// lane per pass), read it once and write it to each of its K destinations,
// so at any moment the workgroup's stores cover one whole destination row.
// Measured at the bench shape: 4 % faster than one wave per token; plain
// stores sustain a higher write rate than non-temporal ones here.
// ---------------------------------------------------------------------------
template <int Q>
__global__ __launch_bounds__(256) void k_dispatch(const u32x4* __restrict__ x,
                                                  u32x4* __restrict__ xperm,
                                                  const int32_t* __restrict__ route, int K,
                                                  int hv) {
  const int t = blockIdx.x;
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int myroute = lane < K ? route[int64_t(t) * K + lane] : -1;
  const u32x4* src = x + int64_t(t) * hv;
  for (int c0 = w * kWave * Q; c0 < hv; c0 += 4 * kWave * Q) {
    u32x4 v[Q];
#pragma unroll
    for (int u = 0; u < Q; ++u) {
      const int c = c0 + u * kWave + lane;
      if (c < hv) v[u] = src[c];
    }
    // Each token starts at its own k (t mod K), so the tokens in flight do
    // not all write their top-1 copy (the hot experts' segments) at once.
    for (int kk = 0; kk < K; ++kk) {
      const int k = (kk + t) % K;
      const int dst = __shfl(myroute, k, kWave);
      if (dst < 0) continue;
      u32x4* d = xperm + int64_t(dst) * hv;
#pragma unroll
      for (int u = 0; u < Q; ++u) {
        const int c = c0 + u * kWave + lane;
        if (c < hv) d[c] = v[u];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Dedup encoding of the route map and the two-phase dispatch it drives
// ("Kimi K3 模型结构（8）", 在线规划、零拷贝、静态 shape: a route whose
// destination rank already appeared among the token's earlier routes holds
// -(position) - 1 and carries no payload; the receiver copies the row it
// got once).  Positions are rows of the stacked [R*S*K] buffer.
// ---------------------------------------------------------------------------
constexpr int32_t kNoDest = INT32_MIN;

__global__ __launch_bounds__(256) void k_route_encode(const int32_t* __restrict__ route,
                                                      int32_t* __restrict__ enc, int ntok, int K,
                                                      int SK) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= ntok) return;
  const int32_t* r = route + int64_t(t) * K;
  int32_t* o = enc + int64_t(t) * K;
  for (int k = 0; k < K; ++k) {
    const int q = r[k];
    if (q < 0) { o[k] = kNoDest; continue; }
    const int d = q / SK;
    bool seen = false;
    for (int k2 = 0; k2 < k; ++k2) seen |= r[k2] >= 0 && r[k2] / SK == d;
    o[k] = seen ? -q - 1 : q;
  }
}

// send: one wave per token; its row is read once and written once per
// destination rank (entries >= 0).
template <int DU>
__global__ __launch_bounds__(256) void k_dispatch_send(const u32x4* __restrict__ x,
                                                       u32x4* __restrict__ xperm,
                                                       const int32_t* __restrict__ enc, int ntok,
                                                       int K, int hv) {
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= ntok) return;
  const int lane = lane_id();
  const int mine = lane < K ? enc[int64_t(t) * K + lane] : -1;
  const u32x4* src = x + int64_t(t) * hv;
  for (int c0 = 0; c0 < hv; c0 += kWave * DU) {
    u32x4 v[DU];
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      const int c = c0 + u * kWave + lane;
      if (c < hv) v[u] = src[c];
    }
    for (int k = 0; k < K; ++k) {
      const int dst = __shfl(mine, k, kWave);
      if (dst < 0) continue;
      u32x4* d = xperm + int64_t(dst) * hv;
#pragma unroll
      for (int u = 0; u < DU; ++u) {
        const int c = c0 + u * kWave + lane;
        if (c < hv) d[c] = v[u];
      }
    }
  }
}

// receive side: one wave per token; every entry -(q) - 1 copies the row that
// arrived on q's rank for this token (that rank's entry >= 0) into row q.
__global__ __launch_bounds__(256) void k_dispatch_expand(u32x4* __restrict__ xperm,
                                                         const int32_t* __restrict__ enc,
                                                         int ntok, int K, int SK, int hv) {
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= ntok) return;
  const int lane = lane_id();
  const int mine = lane < K ? enc[int64_t(t) * K + lane] : kNoDest;
  for (int k = 0; k < K; ++k) {
    const int e = __shfl(mine, k, kWave);
    if (e >= 0 || e == kNoDest) continue;
    const int q = -(e + 1);
    int src = -1;
    for (int k2 = 0; k2 < K && src < 0; ++k2) {
      const int f = __shfl(mine, k2, kWave);
      if (f >= 0 && f / SK == q / SK) src = f;
    }
    if (src < 0) continue;                      // never: the rank's first entry is >= 0
    const u32x4* s = xperm + int64_t(src) * hv;
    u32x4* d = xperm + int64_t(q) * hv;
    for (int c = lane; c < hv; c += kWave) d[c] = s[c];
  }
}

// ---------------------------------------------------------------------------
// combine: one wave per token; out = sum_k g_k * y[route_k] in fp32, k
// ascending, rounded once to bf16.  The rows of KB routes are loaded before
// any of them is accumulated, so KB * CU 16-byte loads per lane are in
// flight.
// ---------------------------------------------------------------------------
#ifndef MOONEP_COMBINE_KB
#define MOONEP_COMBINE_KB 8
#endif
template <int CU, int KB>
__device__ __forceinline__ void combine_rows(const u32x4* __restrict__ y,
                                             const float* __restrict__ gates,
                                             const int32_t* __restrict__ route,
                                             u32x4* __restrict__ out, int ntok, int K, int hv) {
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= ntok) return;
  const int lane = lane_id();
  const int myroute = lane < K ? route[int64_t(t) * K + lane] : -1;
  const float mygate = lane < K ? gates[int64_t(t) * K + lane] : 0.f;
  for (int c0 = 0; c0 < hv; c0 += kWave * CU) {
    float acc[CU][8];
#pragma unroll
    for (int u = 0; u < CU; ++u)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[u][q] = 0.f;
    for (int k0 = 0; k0 < K; k0 += KB) {
      u32x4 v[KB][CU];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int src = __shfl(myroute, min(k0 + kb, K - 1), kWave);
        const bool ok = k0 + kb < K && src >= 0;
        const u32x4* row = y + int64_t(ok ? src : 0) * hv;
#pragma unroll
        for (int u = 0; u < CU; ++u) {
          const int c = c0 + u * kWave + lane;
          // every y row is read exactly once: stream it past the caches
          v[kb][u] = (ok && c < hv) ? __builtin_nontemporal_load(row + c) : u32x4{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const float g = k0 + kb < K ? __shfl(mygate, min(k0 + kb, K - 1), kWave) : 0.f;
#pragma unroll
        for (int u = 0; u < CU; ++u) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[u][2 * q] = fmaf(g, bf16_lo(v[kb][u][q]), acc[u][2 * q]);
            acc[u][2 * q + 1] = fmaf(g, bf16_hi(v[kb][u][q]), acc[u][2 * q + 1]);
          }
        }
      }
    }
    u32x4* o = out + int64_t(t) * hv;
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const int c = c0 + u * kWave + lane;
      if (c < hv) {
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = pack_bf16x2(acc[u][2 * q], acc[u][2 * q + 1]);
        o[c] = w;
      }
    }
  }
}


template <int CU, int KB>
__global__ __launch_bounds__(256) void k_combine(const u32x4* __restrict__ y,
                                                 const float* __restrict__ gates,
                                                 const int32_t* __restrict__ route,
                                                 u32x4* __restrict__ out, int ntok, int K,
                                                 int hv) {
  combine_rows<CU, KB>(y, gates, route, out, ntok, K, hv);
}

// ---------------------------------------------------------------------------
// dispatch backward: dx[t] = sum over k of dxperm[route_k] (fp32 in ascending
// k, rounded once).  One workgroup per token: thread i takes vectors i + 256 u
// of the row, and the loads of KB routes' rows are all in flight before the
// sums (a wave per token, walking the 14 KB row in four passes, is 3 % slower).
// ---------------------------------------------------------------------------
template <int CU, int KB>
__global__ __launch_bounds__(256) void k_dispatch_bwd(const u32x4* __restrict__ dxperm,
                                                      const int32_t* __restrict__ route,
                                                      u32x4* __restrict__ dx, int K, int hv) {
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id();
  const int myroute = lane < K ? route[int64_t(t) * K + lane] : -1;
  for (int c0 = 0; c0 < hv; c0 += 256 * CU) {
    float acc[CU][8];
#pragma unroll
    for (int u = 0; u < CU; ++u)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[u][q] = 0.f;
    for (int k0 = 0; k0 < K; k0 += KB) {
      u32x4 v[KB][CU];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int src = __shfl(myroute, min(k0 + kb, K - 1), kWave);
        const bool ok = k0 + kb < K && src >= 0;
        const u32x4* row = dxperm + int64_t(ok ? src : 0) * hv;
#pragma unroll
        for (int u = 0; u < CU; ++u) {
          const int c = c0 + u * 256 + tid;
          // every dxperm row is read exactly once: stream it past the caches
          v[kb][u] = (ok && c < hv) ? __builtin_nontemporal_load(row + c) : u32x4{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const float g = k0 + kb < K ? 1.f : 0.f;         // the same sums as the combine
#pragma unroll
        for (int u = 0; u < CU; ++u) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[u][2 * q] = fmaf(g, bf16_lo(v[kb][u][q]), acc[u][2 * q]);
            acc[u][2 * q + 1] = fmaf(g, bf16_hi(v[kb][u][q]), acc[u][2 * q + 1]);
          }
        }
      }
    }
    u32x4* o = dx + int64_t(t) * hv;
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const int c = c0 + u * 256 + tid;
      if (c < hv) {
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = pack_bf16x2(acc[u][2 * q], acc[u][2 * q + 1]);
        o[c] = w;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// combine backward: one wave per token.  For each k,
//   dy[route_k] = g_k * dout[t]               (bf16 of the exact product)
//   dgates[t, k] = sum_h dout[t, h] * y[route_k, h]   (fp32, lanes then a
//                                                     DPP tree)
// dout is read once per token and each y row once; KB rows are in flight.
// ---------------------------------------------------------------------------
template <int CU, int KB>
__global__ __launch_bounds__(256) void k_combine_bwd(const u32x4* __restrict__ dout,
                                                     const u32x4* __restrict__ y,
                                                     const float* __restrict__ gates,
                                                     const int32_t* __restrict__ route,
                                                     u32x4* __restrict__ dy,
                                                     float* __restrict__ dgates, int ntok, int K,
                                                     int hv) {
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;   // whole waves leave together
  if (t >= ntok) return;
  const int lane = lane_id();
  const int myroute = lane < K ? route[int64_t(t) * K + lane] : -1;
  const float mygate = lane < K ? gates[int64_t(t) * K + lane] : 0.f;
  float mydot = 0.f;                                    // lane k: dgates[t, k]
  for (int c0 = 0; c0 < hv; c0 += kWave * CU) {
    u32x4 d[CU];
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const int c = c0 + u * kWave + lane;
      d[u] = c < hv ? __builtin_nontemporal_load(dout + int64_t(t) * hv + c) : u32x4{0, 0, 0, 0};
    }
    for (int k0 = 0; k0 < K; k0 += KB) {
      u32x4 v[KB][CU];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int src = wave_bcast(myroute, min(k0 + kb, K - 1));
        const bool ok = k0 + kb < K && src >= 0;
        const u32x4* row = y + int64_t(ok ? src : 0) * hv;
#pragma unroll
        for (int u = 0; u < CU; ++u) {
          const int c = c0 + u * kWave + lane;
          v[kb][u] = (ok && c < hv) ? __builtin_nontemporal_load(row + c) : u32x4{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if (k0 + kb >= K) break;                        // uniform
        const int dst = wave_bcast(myroute, k0 + kb);
        const float g = __int_as_float(wave_bcast(__float_as_int(mygate), k0 + kb));
        float part = 0.f;
#pragma unroll
        for (int u = 0; u < CU; ++u) {
          const int c = c0 + u * kWave + lane;
          u32x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float dl = bf16_lo(d[u][q]), dh = bf16_hi(d[u][q]);
            part = fmaf(dl, bf16_lo(v[kb][u][q]), part);
            part = fmaf(dh, bf16_hi(v[kb][u][q]), part);
            o[q] = mul_to_bf16(g, dl) | (mul_to_bf16(g, dh) << 16);
          }
          if (dst >= 0 && c < hv) dy[int64_t(dst) * hv + c] = o;
        }
        const float s = wave_sum_f(part);
        if (lane == k0 + kb) mydot += s;
      }
    }
  }
  if (lane < K) dgates[int64_t(t) * K + lane] = mydot;
}

// ---------------------------------------------------------------------------
// reduce_grad: grid (chunks, E); y-block i handles the i-th expert that has
// consumers.  Its consumers are the CSR entries of its moves (fill order);
// each receiver holds at most one of them, so they are placed by receiver
// rank and compacted, and the sum runs over ascending ranks.  Entries with
// b >= B (inference overflow) own no slot and are skipped.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_reduce_grad(f32x4* __restrict__ grad_home,
                                                     f32x4* __restrict__ grad_pref,
                                                     const int32_t* __restrict__ cons,
                                                     const int32_t* __restrict__ misc,
                                                     const int32_t* __restrict__ mptr,
                                                     const int32_t* __restrict__ mcnt,
                                                     const int32_t* __restrict__ cs_dst,
                                                     const int32_t* __restrict__ cs_b, int R,
                                                     int B, int64_t nvec) {
  __shared__ int s_rank[MOE_MAX_R];
  __shared__ int s_slot[MOE_MAX_R];
  __shared__ int s_n;
  if ((int)blockIdx.y >= misc[0]) return;
  const int e = cons[blockIdx.y];
  for (int r = threadIdx.x; r < R; r += blockDim.x) s_rank[r] = -1;
  __syncthreads();
  const int q0 = mptr[e], q1 = q0 + mcnt[e];
  for (int q = q0 + (int)threadIdx.x; q < q1; q += blockDim.x) {
    const int b = cs_b[q], d = cs_dst[q];
    if (b < B && (unsigned)d < (unsigned)R) s_rank[d] = d * B + b;
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int lane = lane_id();
    const uint64_t lt = lanemask_lt();
    int k = 0;
    for (int r0 = 0; r0 < R; r0 += kWave) {
      const int v = r0 + lane < R ? s_rank[r0 + lane] : -1;
      const uint64_t bal = __ballot(v >= 0);
      if (v >= 0) s_slot[k + (int)__popcll(bal & lt)] = v;
      k += (int)__popcll(bal);
    }
    if (lane == 0) s_n = k;
  }
  __syncthreads();
  const int ns = s_n;
  if (ns == 0) return;
  f32x4* home = grad_home + int64_t(e) * nvec;
  // U vectors per thread and pass, every load of a slot issued before its
  // sums, so each thread keeps U (1 + slots) loads in flight; the sum still
  // runs over ascending ranks per element
  constexpr int U = 4;
  const int64_t bd = blockDim.x;
  const int64_t stride = int64_t(gridDim.x) * bd * U;
  for (int64_t v0 = int64_t(blockIdx.x) * bd * U + threadIdx.x; v0 < nvec; v0 += stride) {
    f32x4 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + u * bd;
      if (v < nvec) acc[u] = home[v];
    }
    for (int s = 0; s < ns; ++s) {
      f32x4* p = grad_pref + int64_t(s_slot[s]) * nvec;
      f32x4 g[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t v = v0 + u * bd;
        if (v < nvec) g[u] = p[v];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t v = v0 + u * bd;
        if (v < nvec) {
          acc[u].x += g[u].x;
          acc[u].y += g[u].y;
          acc[u].z += g[u].z;
          acc[u].w += g[u].w;
          p[v] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + u * bd;
      if (v < nvec) home[v] = acc[u];
    }
  }
}

}  // namespace moonep

using namespace moonep;

extern "C" int moe_prefetch_weight(const moe_cfg* cfg, const moe_plan* plan,
                                   const moe_bf16* w_home, moe_bf16* w_pref, hipStream_t stream) {
  int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if (!plan || !plan->slot_expert) return MOE_EINVAL;
  const int64_t RB = int64_t(cfg->R) * cfg->B;
  if (RB == 0) return MOE_OK;
  if (!w_home || !w_pref) return MOE_EINVAL;
  if (!aligned16(w_home, w_pref)) return MOE_EINVAL;
  const int64_t nvec = int64_t(cfg->H) * cfg->Hp / 8;
  // enough workgroups to fill the chip (8 per CU); the grid depends on the
  // shape only, never on how many slots the plan uses
  const int grid = (int)std::min<int64_t>(2048, RB * 64);
  hipLaunchKernelGGL(k_prefetch, dim3(grid), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4*>(w_home), reinterpret_cast<u32x4*>(w_pref),
                     plan->slot_expert, (int)RB, cfg->E, nvec);
  return hip_status();
}

extern "C" int moe_dispatch(const moe_cfg* cfg, const moe_plan* plan, const moe_bf16* x,
                            moe_bf16* xperm, hipStream_t stream) {
  int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  const int ntok = cfg->R * cfg->S;
  if (ntok == 0) return MOE_OK;
  if (!plan || !plan->route || !x || !xperm) return MOE_EINVAL;
  if (!aligned16(x, xperm)) return MOE_EINVAL;
  const int hv = cfg->H / 8;
  const int q = (hv + 4 * kWave - 1) / (4 * kWave);   // vectors per lane for one pass
  const dim3 grid(ntok), block(256);
  const u32x4* xs = reinterpret_cast<const u32x4*>(x);
  u32x4* xd = reinterpret_cast<u32x4*>(xperm);
#define MOE_DISPATCH(N) \
  hipLaunchKernelGGL(k_dispatch<N>, grid, block, 0, stream, xs, xd, plan->route, cfg->K, hv)
  if (q <= 1) MOE_DISPATCH(1);
  else if (q <= 2) MOE_DISPATCH(2);
  else MOE_DISPATCH(4);                                // larger rows take several passes
#undef MOE_DISPATCH
  return hip_status();
}

extern "C" int moe_route_encode(const moe_cfg* cfg, const moe_plan* plan, int32_t* route_enc,
                                hipStream_t stream) {
  int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  const int ntok = cfg->R * cfg->S;
  if (ntok == 0) return MOE_OK;
  if (!plan || !plan->route || !route_enc) return MOE_EINVAL;
  hipLaunchKernelGGL(k_route_encode, dim3((ntok + 255) / 256), dim3(256), 0, stream, plan->route,
                     route_enc, ntok, cfg->K, cfg->S * cfg->K);
  return hip_status();
}

extern "C" int moe_dispatch_dedup(const moe_cfg* cfg, const int32_t* route_enc, const moe_bf16* x,
                                  moe_bf16* xperm, hipStream_t stream) {
  int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  const int ntok = cfg->R * cfg->S;
  if (ntok == 0) return MOE_OK;
  if (!route_enc || !x || !xperm) return MOE_EINVAL;
  if (!aligned16(x, xperm)) return MOE_EINVAL;
  const int hv = cfg->H / 8;
  const int du = (hv + kWave - 1) / kWave;
  const dim3 grid((ntok + 3) / 4), block(256);
  const u32x4* xs = reinterpret_cast<const u32x4*>(x);
  u32x4* xd = reinterpret_cast<u32x4*>(xperm);
#define MOE_SEND(N) \
  hipLaunchKernelGGL(k_dispatch_send<N>, grid, block, 0, stream, xs, xd, route_enc, ntok, cfg->K, hv)
  if (du <= 1) MOE_SEND(1);
  else if (du <= 2) MOE_SEND(2);
  else if (du <= 4) MOE_SEND(4);
  else if (du <= 8) MOE_SEND(8);
  else if (du <= 14) MOE_SEND(14);
  else MOE_SEND(16);
#undef MOE_SEND
  hipLaunchKernelGGL(k_dispatch_expand, grid, block, 0, stream, xd, route_enc, ntok, cfg->K,
                     cfg->S * cfg->K, hv);
  return hip_status();
}

extern "C" int moe_combine(const moe_cfg* cfg, const moe_plan* plan, const moe_bf16* y,
                           const float* gates, moe_bf16* out, hipStream_t stream) {
  int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  const int ntok = cfg->R * cfg->S;
  if (ntok == 0) return MOE_OK;
  if (!plan || !plan->route || !y || !gates || !out) return MOE_EINVAL;
  if (!aligned16(y, out)) return MOE_EINVAL;
  const int hv = cfg->Hp / 8;
  const int cu = (hv + kWave - 1) / kWave;
  const dim3 grid((ntok + 3) / 4), block(256);
  const u32x4* ys = reinterpret_cast<const u32x4*>(y);
  u32x4* od = reinterpret_cast<u32x4*>(out);
#define MOE_COMBINE(N)                                                                          \
  hipLaunchKernelGGL((k_combine<N, MOONEP_COMBINE_KB>), grid, block, 0, stream, ys, gates,        \
                     plan->route, od, ntok, cfg->K, hv)
  if (cu <= 1) MOE_COMBINE(1);
  else if (cu <= 2) MOE_COMBINE(2);
  else MOE_COMBINE(4);
#undef MOE_COMBINE
  return hip_status();
}

extern "C" int moe_combine_backward(const moe_cfg* cfg, const moe_plan* plan, const moe_bf16* dout,
                                    const moe_bf16* y, const float* gates, moe_bf16* dy,
                                    float* dgates, hipStream_t stream) {
  int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  const int ntok = cfg->R * cfg->S;
  if (ntok == 0) return MOE_OK;
  if (!plan || !plan->route || !dout || !y || !gates || !dy || !dgates) return MOE_EINVAL;
  if (!aligned16(dout, y, dy)) return MOE_EINVAL;
  const int hv = cfg->Hp / 8;
  const int cu = (hv + kWave - 1) / kWave;
  const dim3 grid((ntok + 3) / 4), block(256);
  const u32x4* ds = reinterpret_cast<const u32x4*>(dout);
  const u32x4* ys = reinterpret_cast<const u32x4*>(y);
  u32x4* dd = reinterpret_cast<u32x4*>(dy);
#define MOE_COMBINE_BWD(N)                                                                \
  hipLaunchKernelGGL((k_combine_bwd<N, 4>), grid, block, 0, stream, ds, ys, gates, plan->route, \
                     dd, dgates, ntok, cfg->K, hv)
  if (cu <= 1) MOE_COMBINE_BWD(1);
  else if (cu <= 2) MOE_COMBINE_BWD(2);
  else MOE_COMBINE_BWD(4);
#undef MOE_COMBINE_BWD
  return hip_status();
}

extern "C" int moe_dispatch_backward(const moe_cfg* cfg, const moe_plan* plan,
                                     const moe_bf16* dxperm, moe_bf16* dx, hipStream_t stream) {
  int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  const int ntok = cfg->R * cfg->S;
  if (ntok == 0) return MOE_OK;
  if (!plan || !plan->route || !dxperm || !dx) return MOE_EINVAL;
  if (!aligned16(dxperm, dx)) return MOE_EINVAL;
  const int hv = cfg->H / 8;
  const int cu = (hv + 255) / 256;                       // vectors per thread, one pass
  const dim3 grid(ntok), block(256);
  const u32x4* xs = reinterpret_cast<const u32x4*>(dxperm);
  u32x4* od = reinterpret_cast<u32x4*>(dx);
#define MOE_UNDISPATCH(N)                                                                   \
  hipLaunchKernelGGL((k_dispatch_bwd<N, 8>), grid, block, 0, stream, xs, plan->route, od, \
                     cfg->K, hv)
  if (cu <= 1) MOE_UNDISPATCH(1);
  else if (cu <= 2) MOE_UNDISPATCH(2);
  else MOE_UNDISPATCH(4);
#undef MOE_UNDISPATCH
  return hip_status();
}

extern "C" int moe_reduce_grad(const moe_cfg* cfg, const moe_plan* plan, float* grad_home,
                               float* grad_pref, hipStream_t stream) {
  int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if (!plan || !plan->workspace) return MOE_EINVAL;
  if (cfg->B == 0) return MOE_OK;
  if (!grad_home || !grad_pref) return MOE_EINVAL;
  if (!aligned16(grad_home, grad_pref)) return MOE_EINVAL;
  if ((int64_t(cfg->H) * cfg->Hp) % 4 != 0) return MOE_EINVAL;
  const PlanLayout L = plan_layout(cfg);
  void* ws = plan->workspace;
  const int64_t nvec = int64_t(cfg->H) * cfg->Hp / 4;
  int chunks = (int)std::min<int64_t>(256, (nvec + 256 * 16 - 1) / (256 * 16));
  if (chunks < 1) chunks = 1;
  hipLaunchKernelGGL(k_reduce_grad, dim3(chunks, cfg->E), dim3(256), 0, stream,
                     reinterpret_cast<f32x4*>(grad_home), reinterpret_cast<f32x4*>(grad_pref),
                     ws_i32(ws, L.off_cons), ws_i32(ws, L.off_misc), ws_i32(ws, L.off_mptr),
                     ws_i32(ws, L.off_mcnt), ws_i32(ws, L.off_cs_dst), ws_i32(ws, L.off_cs_b),
                     cfg->R, cfg->B, nvec);
  return hip_status();
}
