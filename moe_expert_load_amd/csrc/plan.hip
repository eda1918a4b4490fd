// Router histogram, deterministic Theorem-1 planner and route map.
//
// Method: "Kimi K3 模型结构（8）：训练并行，MoonEP 与四类等待" (blog.javazero.top),
// headings 定理 1 (fill an underloaded rank to exactly S*K from one overloaded
// rank, at most R-1 times) and 在线规划、零拷贝、静态 shape (the planner fixes
// every token's destination); "MoonEP : l'équilibrage parfait", Le théorème
// (lemma: a receiver's remote slots come from a single rank).
//
// Three launches, all sized from the configuration only:
//   k_count  C workgroups x 16 waves: per-chunk expert counts (ballot match)
//   k_plan   1 workgroup: column prefix of the chunk counts, T_e, loads, the
//            fills (wave 0), cu_seqlens per rank, per-expert route tables
//   k_route  C workgroups x 16 waves: stable rank of each slot inside its
//            expert, then its destination row
#include "common.hpp"
#include "host.hpp"

namespace moonep {

constexpr int kPlanThreads = kRouteWaves * kWave;  // 1024

struct PlanArgs {
  const int32_t* ids;
  int32_t N, R, S, E, K, B, mode, n, SK, L, C, M, nbits;
  int32_t *counts, *load0, *route, *cu, *slot_expert, *n_red, *src_rank, *moves, *status;
  int32_t *cc, *badc, *taken, *home_base, *mptr, *mcnt, *cs_lo, *cs_hi, *cs_base, *cs_dst, *cs_b,
      *cons, *misc;
};

// ---------------------------------------------------------------------------
// k_count: chunk c covers slots [c*16L, (c+1)*16L); wave w of it the L slots
// starting at c*16L + w*L.  Within a wave, lanes naming the same expert are
// grouped with a ballot per key bit and only the lowest such lane adds the
// group size, so LDS atomics are one per distinct expert per 64 slots.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPlanThreads) void k_count(PlanArgs a) {
  extern __shared__ int s_cnt[];
  __shared__ int s_bad;
  const int E = a.E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_cnt[e] = 0;
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const uint64_t lt = lanemask_lt();
  const int64_t base = int64_t(blockIdx.x) * kRouteWaves * a.L + int64_t(w) * a.L;
  int bad = 0;
  const int64_t lim = min<int64_t>(a.N, base + a.L);
  for (int64_t b0 = base; b0 < lim; b0 += 8 * kWave) {
    int ids8[8];                                  // 8 rounds of ids in flight
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = b0 + u * kWave + lane;
      ids8[u] = i < lim ? a.ids[i] : E;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = b0 + u * kWave + lane;
      int key = E;
      if (i < lim) {
        if ((unsigned)ids8[u] < (unsigned)E) key = ids8[u]; else bad = 1;
      }
      const uint64_t act = __ballot(key < E);
      if (act == 0) continue;
      const uint64_t m = match_any(key, a.nbits, act);
      if (key < E && (m & lt) == 0) atomicAdd(&s_cnt[key], (int)__popcll(m));
    }
  }
  if (bad) s_bad = 1;
  __syncthreads();
  int32_t* out = a.cc + int64_t(blockIdx.x) * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) out[e] = s_cnt[e];
  if (threadIdx.x == 0) a.badc[blockIdx.x] = s_bad;
}

// Exclusive prefix sum of arr[0..n) in LDS; every thread must call it.
// Returns the total.  scratch needs 17 ints.
__device__ int block_excl_scan(int* arr, int n, int* scratch) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int per = (n + kPlanThreads - 1) / kPlanThreads;
  const int b = min(n, tid * per), e = min(n, b + per);
  int s = 0;
  for (int i = b; i < e; ++i) s += arr[i];
  const int incl = wave_incl_scan(s);
  if (lane == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int v = lane < kRouteWaves ? scratch[lane] : 0;
    const int vi = wave_incl_scan(v);
    if (lane < kRouteWaves) scratch[lane] = vi - v;
    if (lane == kRouteWaves - 1) scratch[kRouteWaves] = vi;
  }
  __syncthreads();
  int run = scratch[wave] + incl - s;
  for (int i = b; i < e; ++i) {
    const int v = arr[i];
    arr[i] = run;
    run += v;
  }
  const int total = scratch[kRouteWaves];
  __syncthreads();
  return total;
}

// ---------------------------------------------------------------------------
// k_plan: one workgroup of 1024 threads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPlanThreads) void k_plan(PlanArgs a) {
  extern __shared__ int smem[];
  const int E = a.E, R = a.R, n = a.n, SK = a.SK, B = a.B, M = a.M, C = a.C;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  int* sT = smem;               // [E] T_e
  int* sTaken = sT + E;         // [E] slots of e moved away from home
  int* sMcnt = sTaken + E;      // [E] moves of e
  int* sMptr = sMcnt + E;       // [E] CSR start of e's moves
  int* sRun = sMptr + E;        // [E] scratch
  int* sLoad = sRun + E;        // [R] current load
  int* sLoad0 = sLoad + R;      // [R] initial load
  int* sCursor = sLoad0 + R;    // [R] next home expert a donor gives
  int* sRecv = sCursor + R;     // [R] fill index that filled rank r, or -1
  int* sFu = sRecv + R;         // [R] fill -> receiver
  int* sFo = sFu + R;           // [R] fill -> donor
  int* sFm0 = sFo + R;          // [R] fill -> first move
  int* sFm1 = sFm0 + R;         // [R] fill -> end move
  int* sMe = sFm1 + R;          // [M] move -> expert
  int* sMu = sMe + M;           // [M] move -> receiver
  int* sMlo = sMu + M;          // [M] move -> first in-expert rank
  int* sMhi = sMlo + M;         // [M] move -> end in-expert rank
  int* sMpos = sMhi + M;        // [M] move -> CSR position
  int* sScan = sMpos + M;       // [1024 + 32]
  __shared__ int sErr, sNm, sNf;

  if (tid == 0) { sErr = 0; sNm = 0; sNf = 0; }

  // 1. Column prefix over chunks: cc[c][e] <- sum of cc[c'][e], c' < c; T_e.
  // C <= kMaxChunks.  Each thread loads its whole share of a column in one
  // batch (one memory round trip), then writes the exclusive prefixes.
  {
    int P = 1;
    if (C > 1 && E <= kPlanThreads / 2) P = min(C, kPlanThreads / E);
    if (P == 1) {
      for (int e = tid; e < E; e += kPlanThreads) {
        int v[kMaxChunks];
#pragma unroll
        for (int u = 0; u < kMaxChunks; ++u) v[u] = u < C ? a.cc[int64_t(u) * E + e] : 0;
        int run = 0;
#pragma unroll
        for (int u = 0; u < kMaxChunks; ++u)
          if (u < C) { a.cc[int64_t(u) * E + e] = run; run += v[u]; }
        sT[e] = run;
      }
    } else {
      // P >= 2, so a part holds at most kMaxChunks / 2 chunks and P*E <= 1024
      const bool act = tid < P * E;
      const int e = tid % E, q = tid / E;
      const int c0 = q * C / P, c1 = (q + 1) * C / P;
      int v[kMaxChunks / 2];
      int sum = 0;
#pragma unroll
      for (int u = 0; u < kMaxChunks / 2; ++u) {
        v[u] = (act && c0 + u < c1) ? a.cc[int64_t(c0 + u) * E + e] : 0;
        sum += v[u];
      }
      if (act) sScan[tid] = sum;
      __syncthreads();
      if (act) {
        int run = 0;
        for (int q2 = 0; q2 < q; ++q2) run += sScan[q2 * E + e];
#pragma unroll
        for (int u = 0; u < kMaxChunks / 2; ++u)
          if (c0 + u < c1) { a.cc[int64_t(c0 + u) * E + e] = run; run += v[u]; }
        if (q == P - 1) sT[e] = run;
      }
    }
  }
  __syncthreads();

  // 2. Loads and validity.
  {
    int bad = 0;
    for (int c = tid; c < C; c += kPlanThreads) bad |= a.badc[c];
    if (bad) atomicOr(&sErr, MOE_STATUS_BAD_ID);
    int64_t tot = 0;
    for (int r = tid; r < R; r += kPlanThreads) {
      int s = 0;
      for (int j = 0; j < n; ++j) s += sT[r * n + j];
      sLoad[r] = s;
      sLoad0[r] = s;
      sRecv[r] = -1;
      sCursor[r] = r * n;
      tot += s;
    }
    for (int e = tid; e < E; e += kPlanThreads) { sTaken[e] = 0; sMcnt[e] = 0; sRun[e] = 0; }
    // total load must be R*S*K (it is unless ids were out of range)
    int t32 = (int)tot;  // R*S*K < 2^31
    t32 = wave_sum(t32);
    if (lane == 0) sScan[kPlanThreads + wave] = t32;
    __syncthreads();
    if (tid == 0) {
      int64_t all = 0;
      for (int w = 0; w < kRouteWaves; ++w) all += sScan[kPlanThreads + w];
      if (all != int64_t(R) * SK) atomicOr(&sErr, MOE_STATUS_UNBALANCED);
    }
    __syncthreads();
  }

  if (sErr & (MOE_STATUS_BAD_ID | MOE_STATUS_UNBALANCED)) {
    // No plan: leave every rank empty; k_route writes route = -1.
    for (int e = tid; e < E; e += kPlanThreads) { a.counts[e] = sT[e]; a.mcnt[e] = 0; }
    for (int r = tid; r < R; r += kPlanThreads) {
      a.load0[r] = sLoad0[r];
      a.n_red[r] = 0;
      a.src_rank[r] = -1;
    }
    for (int64_t i = tid; i < int64_t(R) * B; i += kPlanThreads) a.slot_expert[i] = -1;
    for (int64_t i = tid; i < int64_t(R) * (E + B + 1); i += kPlanThreads) a.cu[i] = 0;
    if (tid == 0) {
      a.status[0] = 0; a.status[1] = 0; a.status[2] = sErr; a.status[3] = 0;
      a.misc[0] = 0;
    }
    return;
  }

  // 3. The fills, on wave 0 (sequential by construction: at most R-1).
  if (wave == 0) {
    volatile int* vLoad = sLoad;
    volatile int* vT = sT;
    volatile int* vTaken = sTaken;
    volatile int* vMcnt = sMcnt;
    volatile int* vCursor = sCursor;
    volatile int* vRecv = sRecv;
    volatile int* vFu = sFu;
    volatile int* vFo = sFo;
    volatile int* vFm0 = sFm0;
    volatile int* vFm1 = sFm1;
    volatile int* vMe = sMe;
    volatile int* vMu = sMu;
    volatile int* vMlo = sMlo;
    volatile int* vMhi = sMhi;
    const uint64_t lt = lanemask_lt();
    int nm = 0, nf = 0, err = 0;
    for (int iter = 0; iter < R; ++iter) {
      // receiver: lowest-id rank that is underloaded now
      int u = -1;
      for (int r0 = 0; r0 < R; r0 += kWave) {
        const int r = r0 + lane;
        const uint64_t bal = __ballot(r < R && vLoad[r] < SK);
        if (bal) { u = r0 + __ffsll((unsigned long long)bal) - 1; break; }
      }
      if (u < 0) break;
      // donor: largest load, lowest id on ties
      int best = -1, bestr = R;
      for (int r = lane; r < R; r += kWave) {
        const int l = vLoad[r];
        if (l > best) { best = l; bestr = r; }
      }
#pragma unroll
      for (int d = kWave / 2; d >= 1; d >>= 1) {
        const int ob = __shfl_xor(best, d, kWave), orr = __shfl_xor(bestr, d, kWave);
        if (ob > best || (ob == best && orr < bestr)) { best = ob; bestr = orr; }
      }
      const int o = bestr;
      if (best <= SK) { err |= MOE_STATUS_INTERNAL; break; }
      const int need = SK - vLoad[u];
      int d = need;
      const int m0 = nm;
      int e0 = vCursor[o];
      const int eend = (o + 1) * n;
      // donor gives its home experts in ascending id, earliest slots first
      while (d > 0) {
        if (e0 >= eend) { err |= MOE_STATUS_INTERNAL; break; }
        const int e = e0 + lane;
        const bool in = e < eend;
        const int rem = in ? vT[e] - vTaken[e] : 0;
        const int incl = wave_incl_scan(rem);
        const int take = in ? min(max(d - (incl - rem), 0), rem) : 0;
        const uint64_t mvb = __ballot(take > 0);
        if (take > 0) {
          const int idx = nm + (int)__popcll(mvb & lt);
          const int lo = vTaken[e];
          if (idx < M) { vMe[idx] = e; vMu[idx] = u; vMlo[idx] = lo; vMhi[idx] = lo + take; }
          vTaken[e] = lo + take;
          vMcnt[e] = vMcnt[e] + 1;
        }
        nm += (int)__popcll(mvb);
        const int tot = __shfl(incl, kWave - 1, kWave);
        d -= min(d, tot);
        if (d == 0) {
          const uint64_t left = __ballot(in && rem - take > 0);
          e0 = left ? e0 + __ffsll((unsigned long long)left) - 1 : e0 + kWave;
        } else {
          e0 += kWave;
        }
      }
      if (err) break;
      if (nm > M) { err |= MOE_STATUS_INTERNAL; break; }
      if (lane == 0) {
        vCursor[o] = e0;
        vLoad[o] = vLoad[o] - need;
        vLoad[u] = SK;
        vFu[nf] = u;
        vFo[nf] = o;
        vFm0[nf] = m0;
        vFm1[nf] = nm;
        vRecv[u] = nf;
      }
      ++nf;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (lane == 0) {
      sNm = min(nm, M);
      sNf = nf;
      if (err) atomicOr(&sErr, err);
    }
  }
  __syncthreads();
  const int nm = sNm, nf = sNf;

  // 4. CSR of moves per expert, ordered by receiver rank (ascending).
  for (int e = tid; e < E; e += kPlanThreads) sMptr[e] = sMcnt[e];
  __syncthreads();
  block_excl_scan(sMptr, E, sScan);
  if (wave == 0) {
    volatile int* vRun = sRun;
    for (int r = 0; r < R; ++r) {
      const int f = sRecv[r];
      if (f < 0) continue;
      for (int m = sFm0[f] + lane; m < sFm1[f]; m += kWave) {
        const int e = sMe[m];
        const int k = vRun[e];
        vRun[e] = k + 1;
        sMpos[m] = sMptr[e] + k;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  __syncthreads();
  // experts that have consumers (ascending id), for reduce_grad
  for (int e = tid; e < E; e += kPlanThreads) sRun[e] = sMcnt[e] > 0 ? 1 : 0;
  __syncthreads();
  const int ncons = block_excl_scan(sRun, E, sScan);
  for (int e = tid; e < E; e += kPlanThreads)
    if (sMcnt[e] > 0) a.cons[sRun[e]] = e;
  if (tid == 0) a.misc[0] = ncons;

  // 5. cu_seqlens of every rank; home and move route bases.
  for (int r = wave; r < R; r += kRouteWaves) {
    const int f = sRecv[r];
    const int m0 = f >= 0 ? sFm0[f] : 0, m1 = f >= 0 ? sFm1[f] : 0;
    const int nred = m1 - m0;
    const int o = f >= 0 ? sFo[f] : -1;
    int32_t* cur = a.cu + int64_t(r) * (E + B + 1);
    if (lane == 0) cur[0] = 0;
    int carry = 0;
    for (int j0 = 0; j0 < E + B; j0 += kWave) {
      const int j = j0 + lane;
      int len = 0, mv = -1;
      if (j < E) {
        if (j / n == r) {
          len = sT[j] - sTaken[j];
        } else if (nred > B && j / n == o) {       // inference overflow row
          for (int m = m0 + B; m < m1; ++m)
            if (sMe[m] == j) { mv = m; break; }
          if (mv >= 0) len = sMhi[mv] - sMlo[mv];
        }
      } else if (j < E + B) {
        const int b = j - E;
        if (b < nred) { mv = m0 + b; len = sMhi[mv] - sMlo[mv]; }
      }
      const int incl = wave_incl_scan(len);
      const int start = carry + incl - len;
      if (j < E + B) cur[j + 1] = carry + incl;
      if (j < E && j / n == r) a.home_base[j] = r * SK + start - sTaken[j];
      if (mv >= 0) a.cs_base[sMpos[mv]] = r * SK + start - sMlo[mv];
      carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) {
      if (carry != SK) atomicOr(&sErr, MOE_STATUS_INTERNAL);
      if (a.mode == MOE_MODE_TRAIN && nred > B) atomicOr(&sErr, MOE_STATUS_CAPACITY);
    }
  }

  __syncthreads();
  if (sErr & MOE_STATUS_INTERNAL) {
    // Never expected (Theorem 1); keep every later step inside its buffers.
    for (int64_t i = tid; i < int64_t(R) * (E + B + 1); i += kPlanThreads) a.cu[i] = 0;
  }

  // 6. Outputs and route tables.
  for (int e = tid; e < E; e += kPlanThreads) {
    a.counts[e] = sT[e];
    a.taken[e] = sTaken[e];
    a.mptr[e] = sMptr[e];
    a.mcnt[e] = sMcnt[e];
  }
  for (int r = tid; r < R; r += kPlanThreads) {
    const int f = sRecv[r];
    a.load0[r] = sLoad0[r];
    a.n_red[r] = f >= 0 ? sFm1[f] - sFm0[f] : 0;
    a.src_rank[r] = f >= 0 ? sFo[f] : -1;
  }
  for (int64_t i = tid; i < int64_t(R) * B; i += kPlanThreads) {
    const int r = (int)(i / B), b = (int)(i % B);
    const int f = sRecv[r];
    int e = -1;
    if (f >= 0 && b < sFm1[f] - sFm0[f]) e = sMe[sFm0[f] + b];
    a.slot_expert[i] = e;
  }
  for (int m = tid; m < nm; m += kPlanThreads) {
    a.moves[4 * m + 0] = sMe[m];
    a.moves[4 * m + 1] = sMu[m];
    a.moves[4 * m + 2] = sMlo[m];
    a.moves[4 * m + 3] = sMhi[m];
    const int pos = sMpos[m];
    a.cs_lo[pos] = sMlo[m];
    a.cs_hi[pos] = sMhi[m];
    a.cs_dst[pos] = sMu[m];
    a.cs_b[pos] = m - sFm0[sRecv[sMu[m]]];
  }
  __syncthreads();
  if (tid == 0) {
    a.status[0] = nf;
    a.status[1] = nm;
    a.status[2] = sErr;
    a.status[3] = 0;
  }
}

// ---------------------------------------------------------------------------
// k_route: stable rank p of each slot inside its expert, then
//   p >= taken[e]: home_base[e] + p          (stays on the home rank)
//   otherwise:     cs_base[q] + p  for the move q of e with lo <= p < hi.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPlanThreads) void k_route(PlanArgs a) {
  extern __shared__ int s_cnt[];  // [16][E]
  const int E = a.E;
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const uint64_t lt = lanemask_lt();
  const int64_t base = int64_t(blockIdx.x) * kRouteWaves * a.L + int64_t(w) * a.L;
  const int64_t lim = min<int64_t>(a.N, base + a.L);
  const int st = a.status[2];
  if (st & (MOE_STATUS_BAD_ID | MOE_STATUS_UNBALANCED | MOE_STATUS_INTERNAL)) {
    for (int64_t i = base + lane; i < lim; i += kWave) a.route[i] = -1;
    return;
  }
  int* cnt = s_cnt + w * E;
  int* s_taken = s_cnt + kRouteWaves * E;     // [E] LDS copies of the
  int* s_home = s_taken + E;                  // [E] per-expert route tables
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    s_taken[e] = a.taken[e];
    s_home[e] = a.home_base[e];
  }
  for (int e = lane; e < E; e += kWave) cnt[e] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // pass A: per-wave counts
  for (int64_t b0 = base; b0 < lim; b0 += 8 * kWave) {
    int ids8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = b0 + u * kWave + lane;
      ids8[u] = i < lim ? a.ids[i] : E;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int key = ids8[u];
      const uint64_t act = __ballot(key < E);
      const uint64_t m = match_any(key, a.nbits, act);
      if (key < E && (m & lt) == 0) cnt[key] += (int)__popcll(m);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  __syncthreads();
  // exclusive prefix over the 16 waves, on top of the chunk's prefix
  const int32_t* ccp = a.cc + int64_t(blockIdx.x) * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = ccp[e];
    for (int ww = 0; ww < kRouteWaves; ++ww) {
      const int v = s_cnt[ww * E + e];
      s_cnt[ww * E + e] = run;
      run += v;
    }
  }
  __syncthreads();
  // pass B: ranks and destinations
  for (int64_t b0 = base; b0 < lim; b0 += 8 * kWave) {
   int ids8[8];
#pragma unroll
   for (int u = 0; u < 8; ++u) {
     const int64_t i = b0 + u * kWave + lane;
     ids8[u] = i < lim ? a.ids[i] : E;
   }
#pragma unroll
   for (int u = 0; u < 8; ++u) {
    const int64_t i = b0 + u * kWave + lane;
    const int key = ids8[u];
    const uint64_t act = __ballot(key < E);
    const uint64_t m = match_any(key, a.nbits, act);
    if (key < E) {
      const int p = cnt[key] + (int)__popcll(m & lt);
      int dest = -1;
      if (p >= s_taken[key]) {
        dest = s_home[key] + p;
      } else {
        const int q0 = a.mptr[key], q1 = q0 + a.mcnt[key];
        for (int q = q0; q < q1; ++q)
          if (p >= a.cs_lo[q] && p < a.cs_hi[q]) { dest = a.cs_base[q] + p; break; }
      }
      a.route[i] = dest;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (key < E && (m & lt) == 0) cnt[key] += (int)__popcll(m);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
   }
  }
}

static size_t plan_lds_bytes(const moe_cfg* c, const PlanLayout& L) {
  return sizeof(int) * (size_t(5) * c->E + size_t(8) * c->R + size_t(5) * L.M + kPlanThreads + 32);
}

}  // namespace moonep

using namespace moonep;

extern "C" int moe_plan_sizes(const moe_cfg* cfg, size_t sizes_out[MOE_PLAN_NARRAYS]) {
  const int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if (!sizes_out) return MOE_EINVAL;
  const PlanLayout L = plan_layout(cfg);
  const size_t E = cfg->E, R = cfg->R, B = cfg->B;
  sizes_out[0] = 4 * E;
  sizes_out[1] = 4 * R;
  sizes_out[2] = 4 * size_t(L.N);
  sizes_out[3] = 4 * R * (E + B + 1);
  sizes_out[4] = 4 * R * B;
  sizes_out[5] = 4 * R;
  sizes_out[6] = 4 * R;
  sizes_out[7] = 16 * size_t(L.M);
  sizes_out[8] = 16;
  sizes_out[9] = L.bytes;
  return MOE_OK;
}

extern "C" int moe_plan_run(const moe_cfg* cfg, const int32_t* topk_ids, const moe_plan* plan,
                            hipStream_t stream) {
  int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if (!plan_ptrs_ok(plan)) return MOE_EINVAL;
  const PlanLayout L = plan_layout(cfg);
  if (L.N > 0 && (!topk_ids || !plan->route)) return MOE_EINVAL;
  PlanArgs a;
  a.ids = topk_ids;
  a.N = (int32_t)L.N;
  a.R = cfg->R; a.S = cfg->S; a.E = cfg->E; a.K = cfg->K; a.B = cfg->B; a.mode = cfg->mode;
  a.n = cfg->E / cfg->R;
  a.SK = cfg->S * cfg->K;
  a.L = L.L; a.C = L.C; a.M = L.M; a.nbits = L.nbits;
  a.counts = plan->counts; a.load0 = plan->load0; a.route = plan->route; a.cu = plan->cu_seqlens;
  a.slot_expert = plan->slot_expert; a.n_red = plan->n_redundant; a.src_rank = plan->src_rank;
  a.moves = plan->moves; a.status = plan->status;
  void* ws = plan->workspace;
  a.cc = ws_i32(ws, L.off_cc); a.badc = ws_i32(ws, L.off_badc); a.taken = ws_i32(ws, L.off_taken);
  a.home_base = ws_i32(ws, L.off_home_base); a.mptr = ws_i32(ws, L.off_mptr);
  a.mcnt = ws_i32(ws, L.off_mcnt); a.cs_lo = ws_i32(ws, L.off_cs_lo);
  a.cs_hi = ws_i32(ws, L.off_cs_hi); a.cs_base = ws_i32(ws, L.off_cs_base);
  a.cs_dst = ws_i32(ws, L.off_cs_dst); a.cs_b = ws_i32(ws, L.off_cs_b);
  a.cons = ws_i32(ws, L.off_cons); a.misc = ws_i32(ws, L.off_misc);

  const size_t lds_count = sizeof(int) * cfg->E;
  const size_t lds_plan = plan_lds_bytes(cfg, L);
  const size_t lds_route = sizeof(int) * size_t(kRouteWaves + 2) * cfg->E;
  if ((rc = allow_lds(k_plan, lds_plan)) != MOE_OK) return rc;
  if ((rc = allow_lds(k_route, lds_route)) != MOE_OK) return rc;
  if (L.C > 0) hipLaunchKernelGGL(k_count, dim3(L.C), dim3(kPlanThreads), lds_count, stream, a);
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(kPlanThreads), lds_plan, stream, a);
  if (L.C > 0) hipLaunchKernelGGL(k_route, dim3(L.C), dim3(kPlanThreads), lds_route, stream, a);
  return hip_status();
}

extern "C" const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid configuration, pointer or rank range";
    case MOE_EHIP: return "HIP launch or runtime error";
    case MOE_ELIMIT: return "size beyond the library limits";
    default: return "unknown error code";
  }
}
