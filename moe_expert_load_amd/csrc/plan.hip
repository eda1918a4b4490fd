// Router histogram, deterministic Theorem-1 planner and route map.
//
// Method: "Kimi K3 模型结构（8）：训练并行，MoonEP 与四类等待" (blog.javazero.top),
// headings 定理 1 (fill an underloaded rank to exactly S*K from one overloaded
// rank, at most R-1 times) and 在线规划、零拷贝、静态 shape (the planner fixes
// every token's destination); "MoonEP : l'équilibrage parfait", Le théorème
// (lemma: a receiver's remote slots come from a single rank).
//
// Four launches, all sized from the configuration only:
//   k_count   C workgroups x 16 waves: per-chunk expert counts (LDS atomics)
//   k_colscan E/64 workgroups: prefix of the chunk counts over chunks, T_e
//   k_plan    1 workgroup: loads, the fills (wave 0: the loads alone for the
//             ascending construction, whose moves are then built one
//             wave per fill), per-rank row prefixes, per-expert route tables
//   k_route   C workgroups x 16 waves: stable rank of each slot inside its
//             expert, then its destination row
#include "common.hpp"
#include "host.hpp"

namespace moonep {

constexpr int kPlanThreads = kRouteWaves * kWave;  // 1024

template <int N>
struct IntTag {
  static constexpr int value = N;
};

struct PlanArgs {
  const int32_t* ids;
  int32_t N, R, S, E, K, B, mode, n, SK, L, C, M, policy;
  int32_t *counts, *load0, *route, *cu, *slot_expert, *n_red, *src_rank, *moves, *status;
  int32_t *cc, *badc, *taken, *home_base, *mptr, *mcnt, *cs_lo, *cs_hi, *cs_base, *cs_dst, *cs_b,
      *cons, *hpre, *spre, *rinfo, *ocum, *misc;
};

// ---------------------------------------------------------------------------
// k_count: chunk c covers slots [c*16L, (c+1)*16L); wave w of it the L slots
// starting at c*16L + w*L.  Every valid slot adds one to its expert's LDS
// counter (the LDS atomic unit serialises lanes that share an address).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPlanThreads) void k_count(PlanArgs a) {
  extern __shared__ int s_cnt[];
  __shared__ int s_bad;
  const int E = a.E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_cnt[e] = 0;
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  const int lane = lane_id(), w = threadIdx.x / kWave;
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
      if (i < lim) {
        if ((unsigned)ids8[u] < (unsigned)E) atomicAdd(&s_cnt[ids8[u]], 1); else bad = 1;
      }
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

// The same over two arrays of n elements at once (one pass, one set of
// barriers).  Returns the total of a1; *total2 gets the total of a2.
// scratch needs 34 ints.
__device__ int block_excl_scan2(int* a1, int* a2, int n, int* scratch, int* total2) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int per = (n + kPlanThreads - 1) / kPlanThreads;
  const int b = min(n, tid * per), e = min(n, b + per);
  int s1 = 0, s2 = 0;
  for (int i = b; i < e; ++i) {
    s1 += a1[i];
    s2 += a2[i];
  }
  const int i1 = wave_incl_scan(s1), i2 = wave_incl_scan(s2);
  if (lane == kWave - 1) {
    scratch[wave] = i1;
    scratch[17 + wave] = i2;
  }
  __syncthreads();
  if (wave == 0) {
    const int v1 = lane < kRouteWaves ? scratch[lane] : 0;
    const int v2 = lane < kRouteWaves ? scratch[17 + lane] : 0;
    const int w1 = wave_incl_scan(v1), w2 = wave_incl_scan(v2);
    if (lane < kRouteWaves) {
      scratch[lane] = w1 - v1;
      scratch[17 + lane] = w2 - v2;
    }
    if (lane == kRouteWaves - 1) {
      scratch[kRouteWaves] = w1;
      scratch[17 + kRouteWaves] = w2;
    }
  }
  __syncthreads();
  int r1 = scratch[wave] + i1 - s1, r2 = scratch[17 + wave] + i2 - s2;
  for (int i = b; i < e; ++i) {
    const int v1 = a1[i], v2 = a2[i];
    a1[i] = r1;
    a2[i] = r2;
    r1 += v1;
    r2 += v2;
  }
  const int t1 = scratch[kRouteWaves];
  *total2 = scratch[17 + kRouteWaves];
  __syncthreads();
  return t1;
}

// ---------------------------------------------------------------------------
// k_colscan: cc[c][e] <- sum of cc[c'][e] over c' < c, and T_e (the counts
// output).  A workgroup takes 64 experts; its 16 waves split the C chunks.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPlanThreads) void k_colscan(PlanArgs a) {
  constexpr int kPer = kMaxChunks / kRouteWaves;
  __shared__ int s_part[kRouteWaves][kWave];
  const int E = a.E, C = a.C;
  const int lane = lane_id(), g = threadIdx.x / kWave;
  const int e = blockIdx.x * kWave + lane;
  const int cpg = (C + kRouteWaves - 1) / kRouteWaves;     // <= kPer
  const int c0 = g * cpg;
  int v[kPer];
  int sum = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c = c0 + u;
    v[u] = (e < E && u < cpg && c < C) ? a.cc[int64_t(c) * E + e] : 0;
    sum += v[u];
  }
  s_part[g][lane] = sum;
  __syncthreads();
  int run = 0;
  for (int q = 0; q < g; ++q) run += s_part[q][lane];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c = c0 + u;
    if (e < E && u < cpg && c < C) {
      a.cc[int64_t(c) * E + e] = run;
      run += v[u];
    }
  }
  if (g == kRouteWaves - 1 && e < E) a.counts[e] = run;   // groups 0..15 cover all chunks
}

// No slots at all (S == 0): T_e = 0.
__global__ __launch_bounds__(kPlanThreads) void k_zero_counts(PlanArgs a) {
  for (int e = threadIdx.x; e < a.E; e += blockDim.x) a.counts[e] = 0;
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
  int* sLoad0 = sMptr + E;      // [R] initial load
  int* sRecv = sLoad0 + R;      // [R] fill index that filled rank r, or -1
  int* sFo = sRecv + R;         // [R] fill -> donor
  int* sFm0 = sFo + R;          // [R] fill -> first move
  int* sFm1 = sFm0 + R;         // [R] fill -> end move
  int* sMe = sFm1 + R;          // [M] move -> expert
  int* sMu = sMe + M;           // [M] move -> receiver
  int* sMlo = sMu + M;          // [M] move -> first in-expert rank
  int* sMhi = sMlo + M;         // [M] move -> end in-expert rank
  int* sMpos = sMhi + M;        // [M] move -> index among its expert's moves
  int* sHpre = sMpos + M;       // [R*(n+1)] per rank: prefix of home row lengths
  int* sSpre = sHpre + R * (n + 1);  // [R*(B+1)] per rank: prefix of prefetch rows
  int* sOcum = sSpre + R * (B + 1);  // [M] inclusive prefix over overflow moves
  int* sOt = sLoad0;            // [R] overflow rows per rank (after the fills)
  int* sScan = sOcum + M;       // [1024 + 32]
  __shared__ int sErr, sNm, sNf, sNov;

  if (tid == 0) { sErr = 0; sNm = 0; sNf = 0; sNov = 0; }

  // 1. T_e from k_colscan.
  for (int e = tid; e < E; e += kPlanThreads) sT[e] = a.counts[e];
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
      sLoad0[r] = s;
      a.load0[r] = s;
      sRecv[r] = -1;
      tot += s;
    }
    for (int e = tid; e < E; e += kPlanThreads) { sTaken[e] = 0; sMcnt[e] = 0; }
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

  // No plan: every rank empty, no moves; k_route writes route = -1.
  auto no_plan = [&]() {
    for (int e = tid; e < E; e += kPlanThreads) { a.counts[e] = sT[e]; a.mcnt[e] = 0; }
    for (int r = tid; r < R; r += kPlanThreads) {   // load0 is written in step 2
      a.n_red[r] = 0;
      a.src_rank[r] = -1;
    }
    for (int64_t i = tid; i < int64_t(R) * B; i += kPlanThreads) a.slot_expert[i] = -1;
    for (int64_t i = tid; i < int64_t(R) * (E + B + 1); i += kPlanThreads) a.cu[i] = 0;
    if (tid == 0) {
      a.status[0] = 0; a.status[1] = 0; a.status[2] = sErr; a.status[3] = 0;
      a.misc[0] = 0;
    }
  };
  if (sErr & (MOE_STATUS_BAD_ID | MOE_STATUS_UNBALANCED)) {
    no_plan();
    return;
  }

  // 3. The fills (sequential by construction: at most R-1).  Each picks the
  // lowest-id underloaded rank u and the most loaded rank o (lowest id on
  // ties) and moves SK - load(u) slots of o's home experts to u.  Wave 0
  // keeps every rank's load in registers (rank r in lane r % 64, slot r / 64
  // of RPL slots; RPL = 1 up to 64 ranks) and finds u and o with ballots.
  const bool ascending = a.policy != MOE_PLAN_LARGEST_FIRST;
  // Ascending construction: a donor gives its home experts in ascending id,
  // earliest slots first, so its fills take consecutive ranges of one list,
  // its experts' slots in id order.  The sequential part is then the loads
  // alone (receiver, donor, amount and where in the donor's list the fill
  // starts); the moves of every fill follow in parallel from where its range
  // meets the experts' ranges (step 3b).  Per-fill records, in arrays that
  // step 5 fills only after the moves are built:
  int* fNeed = sLoad0;          // [R] slots moved by fill f
  int* fG = sSpre;              // [R] start of f in its donor's list
  int* fUD = sScan + 32;        // [R] receiver | donor's fill ordinal << 16
  int* sFirst = sHpre;          // [E] donor ordinal of the fill that starts e
  int* sGtot = sHpre + E;       // [R] slots each rank gave away
  int* sLastD = sOcum;          // [E] donor ordinal of the fill that ends e
  auto fills_ascending = [&](auto rpl_tag) {
    constexpr int RPL = decltype(rpl_tag)::value;
    int ld[RPL], gv[RPL], dc[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int r = lane + kWave * i;
      ld[i] = r < R ? sLoad0[r] : 0;
      gv[i] = 0;                     // slots given so far (as a donor)
      dc[i] = 0;                     // fills given so far
    }
    // up to 64 ranks (at most 63 fills) the fill records stay in registers
    // (fill f in lane f) and are stored after the loop; otherwise lane 0
    // stores each one as it goes
    int r_o = 0, r_need = 0, r_g = 0, r_ud = 0, r_recv = -1;
    __builtin_amdgcn_s_waitcnt(0xc07f);        // lgkmcnt(0): ld is loaded
    int nf = 0, err = 0;
    for (int iter = 0; iter < R; ++iter) {
      int u = -1;
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        if (u < 0 && kWave * i < R) {
          const uint64_t bal = __ballot(lane + kWave * i < R && ld[i] < SK);
          if (bal) u = kWave * i + __ffsll((unsigned long long)bal) - 1;
        }
      }
      if (u < 0) break;
      int lb = -1;
#pragma unroll
      for (int i = 0; i < RPL; ++i)
        if (lane + kWave * i < R && ld[i] > lb) lb = ld[i];
      const int mx = wave_max(lb);
      if (mx <= SK) { err |= MOE_STATUS_INTERNAL; break; }
      int o = -1;
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        if (o < 0 && kWave * i < R) {
          const uint64_t bal = __ballot(lane + kWave * i < R && ld[i] == mx);
          if (bal) o = kWave * i + __ffsll((unsigned long long)bal) - 1;
        }
      }
      int lu = ld[0], go = gv[0], co = dc[0];
#pragma unroll
      for (int i = 1; i < RPL; ++i) {
        if (i == u / kWave) lu = ld[i];
        if (i == o / kWave) { go = gv[i]; co = dc[i]; }
      }
      lu = wave_bcast(lu, u % kWave);
      go = wave_bcast(go, o % kWave);
      co = wave_bcast(co, o % kWave);
      const int need = SK - lu;
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        if (lane + kWave * i == o) { ld[i] -= need; gv[i] += need; dc[i] += 1; }
        if (lane + kWave * i == u) ld[i] = SK;
      }
      if (RPL == 1) {
        if (lane == nf) { r_o = o; r_need = need; r_g = go; r_ud = u | (co << 16); }
        if (lane == u) r_recv = nf;
      } else if (lane == 0) {
        sFo[nf] = o;
        fNeed[nf] = need;
        fG[nf] = go;
        fUD[nf] = u | (co << 16);
        sRecv[u] = nf;
      }
      ++nf;
    }
    if (RPL == 1) {
      if (lane < nf) {
        sFo[lane] = r_o;
        fNeed[lane] = r_need;
        fG[lane] = r_g;
        fUD[lane] = r_ud;
      }
      if (lane < R) sRecv[lane] = r_recv;
    }
#pragma unroll
    for (int i = 0; i < RPL; ++i)
      if (lane + kWave * i < R) sGtot[lane + kWave * i] = gv[i];
    if (lane == 0) {
      sNf = nf;
      if (err) atomicOr(&sErr, err);
    }
  };

  // Largest-first policy: the donor's expert with the most slots still at
  // home (ties: lowest id), then the next, until the need is met; only the
  // last one chosen (L) gives part of its slots.  Pass 1 finds L and that
  // part by selecting in descending order of (remaining, -id); pass 2 walks
  // the donor's experts in ascending id and moves every expert ranked above
  // L in full, and L's part.  Moves are written as the fills go.
  auto fills_largest_first = [&](auto rpl_tag) {
    constexpr int RPL = decltype(rpl_tag)::value;
    const uint64_t lt = lanemask_lt();
    int ld[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int r = lane + kWave * i;
      ld[i] = r < R ? sLoad0[r] : 0;
    }
    int nm = 0, nf = 0, err = 0;
    for (int iter = 0; iter < R; ++iter) {
      int u = -1;
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        if (u < 0 && kWave * i < R) {
          const uint64_t bal = __ballot(lane + kWave * i < R && ld[i] < SK);
          if (bal) u = kWave * i + __ffsll((unsigned long long)bal) - 1;
        }
      }
      if (u < 0) break;
      int lb = -1;
#pragma unroll
      for (int i = 0; i < RPL; ++i)
        if (lane + kWave * i < R && ld[i] > lb) lb = ld[i];
      const int mx = wave_max(lb);
      if (mx <= SK) { err |= MOE_STATUS_INTERNAL; break; }
      int o = -1;
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        if (o < 0 && kWave * i < R) {
          const uint64_t bal = __ballot(lane + kWave * i < R && ld[i] == mx);
          if (bal) o = kWave * i + __ffsll((unsigned long long)bal) - 1;
        }
      }
      int lu = ld[0];
#pragma unroll
      for (int i = 1; i < RPL; ++i)
        if (i == u / kWave) lu = ld[i];
      lu = wave_bcast(lu, u % kWave);
      const int need = SK - lu;
      int d = need;
      const int m0 = nm;
      const int eend = (o + 1) * n;
      typedef __attribute__((address_space(3))) volatile int lds_vint;
      lds_vint* vT = (lds_vint*)sT;
      lds_vint* vTaken = (lds_vint*)sTaken;
      lds_vint* vMcnt = (lds_vint*)sMcnt;
      const int eb = o * n;
      // with at most 64 home experts the donor's remaining counts are read
      // once into registers (pass 1 does not change them)
      const int x0 = (n <= kWave && lane < n) ? vT[eb + lane] - vTaken[eb + lane] : 0;
      int prev_r = 0x7fffffff, prev_e = -1, L = -1, Lr = 0, Lamt = 0;
      for (int it = 0; it < n && d > 0; ++it) {
        int best_r = 0, best_e = 0x7fffffff;
        for (int c0 = eb; c0 < eend; c0 += kWave) {
          const int e = c0 + lane;
          int r = -1;
          if (e < eend) {
            const int x = n <= kWave ? x0 : vT[e] - vTaken[e];
            if (x > 0 && (x < prev_r || (x == prev_r && e > prev_e))) r = x;
          }
          const int mx2 = wave_max(r);
          if (mx2 <= 0) continue;                                  // uniform
          const uint64_t bal = __ballot(r == mx2);
          const int ce = c0 + __ffsll((unsigned long long)bal) - 1;
          if (mx2 > best_r || (mx2 == best_r && ce < best_e)) { best_r = mx2; best_e = ce; }
        }
        if (best_r <= 0) break;
        if (best_r >= d) { L = best_e; Lr = best_r; Lamt = d; d = 0; }
        else { d -= best_r; prev_r = best_r; prev_e = best_e; }
      }
      if (d > 0 || L < 0) { err |= MOE_STATUS_INTERNAL; break; }
      for (int c0 = eb; c0 < eend; c0 += kWave) {
        const int e = c0 + lane;
        int tk = 0, w = 0, take = 0;
        if (e < eend) {
          tk = vTaken[e];
          w = vMcnt[e];
          const int x = vT[e] - tk;
          if (e == L) take = Lamt;
          else if (x > 0 && (x > Lr || (x == Lr && e < L))) take = x;
        }
        const uint64_t mvb = __ballot(take > 0);
        if (take > 0) {
          const int idx = nm + (int)__popcll(mvb & lt);
          if (idx < M) { sMe[idx] = e; sMu[idx] = u; sMlo[idx] = tk; sMhi[idx] = tk + take; sMpos[idx] = w; }
          vTaken[e] = tk + take;
          vMcnt[e] = w + 1;
        }
        nm += (int)__popcll(mvb);
      }
      if (nm > M) { err |= MOE_STATUS_INTERNAL; break; }
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        if (lane + kWave * i == o) ld[i] -= need;
        if (lane + kWave * i == u) ld[i] = SK;
      }
      if (lane == 0) {
        sFo[nf] = o;
        sFm0[nf] = m0;
        sFm1[nf] = nm;
        sRecv[u] = nf;
      }
      ++nf;
    }
    if (lane == 0) {
      sNm = min(nm, M);
      sNf = nf;
      if (err) atomicOr(&sErr, err);
    }
  };
  if (wave == 0) {
    if (ascending) {
      if (R <= kWave) fills_ascending(IntTag<1>{});
      else if (R <= 4 * kWave) fills_ascending(IntTag<4>{});
      else fills_ascending(IntTag<MOE_MAX_R / kWave>{});
    } else {
      if (R <= kWave) fills_largest_first(IntTag<1>{});
      else if (R <= 4 * kWave) fills_largest_first(IntTag<4>{});
      else fills_largest_first(IntTag<MOE_MAX_R / kWave>{});
    }
  }
  __syncthreads();
  if (sErr & MOE_STATUS_INTERNAL) {
    // Never expected (Theorem 1): a donor ran dry or the moves overflowed.
    no_plan();
    return;
  }

  // 3b. Ascending construction: the moves of every fill.  Fill f takes the
  // range [G, G + need) of its donor's list (the donor's home experts' slots
  // in ascending expert id); every expert of the donor with a slot whose
  // range meets it gives one move, and the moves of a fill are listed in
  // ascending expert id after those of the fills before it.  One wave per
  // fill, one lane per expert of the donor: a prefix sum over the lanes
  // gives where each expert's slots start in the list, a ballot the moves.
  if (ascending) {
    // visit(f, body): calls body(e, p, t, lo, hi, k) on every lane whose
    // expert e (t slots, starting at p in the donor's list) gives fill f
    // its in-expert slots [lo, hi); k is the move's index among f's moves;
    // returns f's move count (every lane)
    auto visit = [&](int f, auto&& body) {
      const uint64_t lt = lanemask_lt();
      const int o = sFo[f], gs = fG[f], ge = gs + fNeed[f];
      int carry = 0, cnt = 0;
      for (int c0 = o * n; c0 < (o + 1) * n && carry < ge; c0 += kWave) {
        const int e = c0 + lane;
        const int t = e < (o + 1) * n ? sT[e] : 0;
        const int incl = wave_incl_scan(t);
        const int p = carry + incl - t;
        const bool mv = t > 0 && p < ge && p + t > gs;
        const uint64_t bal = __ballot(mv);
        if (mv) body(e, p, t, max(gs, p) - p, min(ge, p + t) - p, cnt + (int)__popcll(bal & lt));
        cnt += (int)__popcll(bal);
        carry += wave_bcast(incl, kWave - 1);
      }
      return cnt;
    };
    const int nf = sNf;
    for (int f = wave; f < nf; f += kRouteWaves) {
      const int cnt = visit(f, [&](int, int, int, int, int, int) {});
      if (lane == 0) sFm0[f] = cnt;                  // moves of f, scanned below
    }
    __syncthreads();
    if (wave == 0) {                                 // first and end move of each fill
      int carry = 0;
      for (int f0 = 0; f0 < nf; f0 += kWave) {
        const int f = f0 + lane;
        const int c = f < nf ? sFm0[f] : 0;
        const int incl = wave_incl_scan(c);
        if (f < nf) {
          sFm0[f] = carry + incl - c;
          sFm1[f] = carry + incl;
        }
        carry += wave_bcast(incl, kWave - 1);
      }
      if (lane == 0) {
        sNm = min(carry, M);
        if (carry > M) atomicOr(&sErr, MOE_STATUS_INTERNAL);
      }
    }
    __syncthreads();
    if (sErr & MOE_STATUS_INTERNAL) {
      no_plan();
      return;
    }
    // An expert's moves come from consecutive fills of its donor, so the
    // index of a move among its expert's moves is the distance in the
    // donor's fill order from the fill that takes the expert's first slot,
    // and the expert's move count that distance for the fill that takes its
    // last one (its taken slots: all, or up to where the donor stopped
    // giving).  sMpos holds the donor ordinal until step 4.
    for (int f = wave; f < nf; f += kRouteWaves) {
      const int ud = fUD[f], u = ud & 0xffff, d = ud >> 16, m0 = sFm0[f];
      const int gt = sGtot[sFo[f]];
      visit(f, [&](int e, int p, int t, int lo, int hi, int k) {
        const int idx = m0 + k;
        sMe[idx] = e;
        sMu[idx] = u;
        sMlo[idx] = lo;
        sMhi[idx] = hi;
        sMpos[idx] = d;
        if (lo == 0) sFirst[e] = d;
        const int taken = min(t, gt - p);
        if (hi == taken) {
          sLastD[e] = d;
          sTaken[e] = taken;
        }
      });
    }
    __syncthreads();
  }
  const int nm = sNm, nf = sNf;

  // 4. Moves per expert in fill order: CSR start of each expert.
  for (int e = tid; e < E; e += kPlanThreads) {
    if (ascending) sMcnt[e] = sTaken[e] > 0 ? sLastD[e] - sFirst[e] + 1 : 0;
    sMptr[e] = sMcnt[e];
  }
  if (ascending)
    for (int m = tid; m < nm; m += kPlanThreads) sMpos[m] -= sFirst[sMe[m]];
  __syncthreads();
  block_excl_scan(sMptr, E, sScan);

  // 5. Per rank: prefix of its home row lengths (over its experts), of its
  // prefetch rows (over its slots) and of its overflow rows (inference:
  // over its moves past the B slots); cu_seqlens follows in closed form.
  // Up to 32 ranks a wave takes a rank at a time (and the last wave lists
  // the experts that have moves, for reduce_grad); with more ranks the
  // first two are block-wide scans over all ranks at once (each rank's part
  // is a difference of the global prefix) with that list compacted in the
  // same scan.
  if (R <= 2 * kRouteWaves) {
    if (wave == kRouteWaves - 1) {
      const uint64_t lt = lanemask_lt();
      int k = 0;
      for (int e0 = 0; e0 < E; e0 += kWave) {
        const bool has = e0 + lane < E && sMcnt[e0 + lane] > 0;
        const uint64_t bal = __ballot(has);
        if (has) a.cons[k + (int)__popcll(bal & lt)] = e0 + lane;
        k += (int)__popcll(bal);
      }
      if (lane == 0) a.misc[0] = k;
    }
    for (int r = wave; r < R; r += kRouteWaves) {
      const int f = sRecv[r];
      const int m0 = f >= 0 ? sFm0[f] : 0, m1 = f >= 0 ? sFm1[f] : 0;
      const int nred = m1 - m0;
      int carry = 0;
      for (int t0 = 0; t0 < n; t0 += kWave) {
        const int t = t0 + lane;
        const int len = t < n ? sT[r * n + t] - sTaken[r * n + t] : 0;
        const int incl = wave_incl_scan(len);
        if (t < n) sHpre[r * (n + 1) + t] = a.hpre[r * (n + 1) + t] = carry + incl - len;
        carry += wave_bcast(incl, kWave - 1);
      }
      if (lane == 0) sHpre[r * (n + 1) + n] = a.hpre[r * (n + 1) + n] = carry;
      carry = 0;
      for (int b0 = 0; b0 < B; b0 += kWave) {
        const int b = b0 + lane;
        const int len = (b < B && b < nred) ? sMhi[m0 + b] - sMlo[m0 + b] : 0;
        const int incl = wave_incl_scan(len);
        if (b < B) sSpre[r * (B + 1) + b] = a.spre[r * (B + 1) + b] = carry + incl - len;
        carry += wave_bcast(incl, kWave - 1);
      }
      if (lane == 0) sSpre[r * (B + 1) + B] = a.spre[r * (B + 1) + B] = carry;
      carry = 0;
      for (int m = m0 + B + lane; m - lane < m1; m += kWave) {     // overflow moves
        const int len = m < m1 ? sMhi[m] - sMlo[m] : 0;
        const int incl = wave_incl_scan(len);
        if (m < m1) sOcum[m] = a.ocum[m] = carry + incl;
        carry += wave_bcast(incl, kWave - 1);
      }
      if (lane == 0) {
        sOt[r] = carry;
        a.rinfo[3 * r + 0] = carry;                 // overflow rows
        a.rinfo[3 * r + 1] = m0 + B;                // overflow moves [m0 + B, m1)
        a.rinfo[3 * r + 2] = m1;
      }
    }
    __syncthreads();
  } else {
    {
      int* tX = sHpre;               // [E] T - taken, then its global prefix
      int* tC = sOcum;               // [E] 1 where e has moves, then its prefix
      const int NH = R * (n + 1), NS = R * (B + 1);
      for (int e = tid; e < E; e += kPlanThreads) {
        tX[e] = sT[e] - sTaken[e];
        tC[e] = sMcnt[e] > 0;
      }
      for (int i = tid; i < NS; i += kPlanThreads) {
        const int r = i / (B + 1), b = i % (B + 1), f = sRecv[r];
        const int m0 = f >= 0 ? sFm0[f] : 0, nred = f >= 0 ? sFm1[f] - m0 : 0;
        sSpre[i] = (b < B && b < nred) ? sMhi[m0 + b] - sMlo[m0 + b] : 0;
      }
      __syncthreads();
      int ncons = 0;
      const int hx = block_excl_scan2(tX, tC, E, sScan, &ncons);
      block_excl_scan(sSpre, NS, sScan);
      constexpr int kPer = (MOE_MAX_E + MOE_MAX_R + kPlanThreads - 1) / kPlanThreads;
      int hv[kPer], sv[kPer];
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int i = tid + k * kPlanThreads;
        if (i < NH) {
          const int r = i / (n + 1), j = r * n + i % (n + 1);
          hv[k] = (j < E ? tX[j] : hx) - tX[r * n];
        }
        if (i < NS) sv[k] = sSpre[i] - sSpre[(i / (B + 1)) * (B + 1)];
      }
      for (int e = tid; e < E; e += kPlanThreads)
        if (sMcnt[e] > 0) a.cons[tC[e]] = e;
      if (tid == 0) a.misc[0] = ncons;
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int i = tid + k * kPlanThreads;
        if (i < NH) sHpre[i] = a.hpre[i] = hv[k];
        if (i < NS) sSpre[i] = a.spre[i] = sv[k];
      }
    }
    // overflow rows: ranks without moves past their B slots are written by one
    // thread each; the others (listed in the dead fill records) by a wave each
    int* sOvr = sScan + 32;
    for (int r = tid; r < R; r += kPlanThreads) {
      const int f = sRecv[r];
      const int m0 = f >= 0 ? sFm0[f] : 0, m1 = f >= 0 ? sFm1[f] : 0;
      if (m1 - m0 > B) {
        sOvr[atomicAdd(&sNov, 1)] = r;
      } else {
        sOt[r] = 0;
        a.rinfo[3 * r + 0] = 0;
        a.rinfo[3 * r + 1] = m0 + B;
        a.rinfo[3 * r + 2] = m1;
      }
    }
    __syncthreads();
    for (int q = wave; q < sNov; q += kRouteWaves) {
      const int r = sOvr[q], f = sRecv[r];
      const int m0 = sFm0[f], m1 = sFm1[f];
      int carry = 0;
      for (int m = m0 + B + lane; m - lane < m1; m += kWave) {     // overflow moves
        const int len = m < m1 ? sMhi[m] - sMlo[m] : 0;
        const int incl = wave_incl_scan(len);
        if (m < m1) sOcum[m] = a.ocum[m] = carry + incl;
        carry += wave_bcast(incl, kWave - 1);
      }
      if (lane == 0) {
        sOt[r] = carry;
        a.rinfo[3 * r + 0] = carry;                 // overflow rows
        a.rinfo[3 * r + 1] = m0 + B;                // overflow moves [m0 + B, m1)
        a.rinfo[3 * r + 2] = m1;
      }
    }
    __syncthreads();
  }

  // overflow rows of rank r below weight row j: prefix over its overflow
  // moves (ascending expert) with expert < j
  auto over_below = [&](int r, int j) {
    const int f = sRecv[r];
    if (f < 0) return 0;
    const int lo0 = sFm0[f] + B, hi0 = sFm1[f];
    if (hi0 <= lo0) return 0;
    int lo = lo0, hi = hi0;                                  // first move with e >= j
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sMe[mid] < j) lo = mid + 1; else hi = mid;
    }
    return lo > lo0 ? sOcum[lo - 1] : 0;
  };
  // rows of rank r before weight row j (j in [0, E+B])
  const bool infer = a.mode == MOE_MODE_INFER;
  auto cu_at = [&](int r, int j) {
    if (j <= E) {
      const int t = min(max(j - r * n, 0), n);
      return sHpre[r * (n + 1) + t] + (infer ? over_below(r, j) : 0);
    }
    return sHpre[r * (n + 1) + n] + sOt[r] + sSpre[r * (B + 1) + (j - E)];
  };
  if (C == 0) {
    // No slots: k_route does not run, so cu_seqlens is written here (with
    // slots, k_route writes it from the exported per-rank prefixes).
    const int W = E + B + 1;
    for (int i = tid; i < R * W; i += kPlanThreads) a.cu[i] = cu_at(i / W, i % W);
  }
  for (int e = tid; e < E; e += kPlanThreads) {
    const int h = e / n;
    a.home_base[e] = h * SK + cu_at(h, e) - sTaken[e];
  }
  for (int m = tid; m < nm; m += kPlanThreads) {
    const int u = sMu[m], f = sRecv[u], b = m - sFm0[f];
    const int row_start = b < B ? cu_at(u, E + b) : cu_at(u, sMe[m]);
    const int pos = sMptr[sMe[m]] + sMpos[m];
    if ((unsigned)pos >= (unsigned)M) {        // never expected; stay in bounds
      atomicOr(&sErr, MOE_STATUS_INTERNAL);
      continue;
    }
    a.cs_base[pos] = u * SK + row_start - sMlo[m];
    a.cs_lo[pos] = sMlo[m];
    a.cs_hi[pos] = sMhi[m];
    a.cs_dst[pos] = u;
    a.cs_b[pos] = b;
    a.moves[4 * m + 0] = sMe[m];
    a.moves[4 * m + 1] = u;
    a.moves[4 * m + 2] = sMlo[m];
    a.moves[4 * m + 3] = sMhi[m];
  }
  for (int r = tid; r < R; r += kPlanThreads) {
    const int f = sRecv[r];
    const int nred = f >= 0 ? sFm1[f] - sFm0[f] : 0;
    if (cu_at(r, E + B) != SK) atomicOr(&sErr, MOE_STATUS_INTERNAL);
    if (a.mode == MOE_MODE_TRAIN && nred > B) atomicOr(&sErr, MOE_STATUS_CAPACITY);
    a.n_red[r] = nred;
    a.src_rank[r] = f >= 0 ? sFo[f] : -1;
  }
  __syncthreads();
  if (sErr & MOE_STATUS_INTERNAL) {
    // Never expected (Theorem 1); keep every later step inside its buffers.
    for (int64_t i = tid; i < int64_t(R) * (E + B + 1); i += kPlanThreads) a.cu[i] = 0;
    __syncthreads();
  }

  // 6. Remaining outputs and route tables.
  for (int e = tid; e < E; e += kPlanThreads) {
    a.counts[e] = sT[e];
    a.taken[e] = sTaken[e];
    a.mptr[e] = sMptr[e];
    a.mcnt[e] = sMcnt[e];
  }
  for (int64_t i = tid; i < int64_t(R) * B; i += kPlanThreads) {
    const int r = (int)(i / B), b = (int)(i % B);
    const int f = sRecv[r];
    int e = -1;
    if (f >= 0 && b < sFm1[f] - sFm0[f]) e = sMe[sFm0[f] + b];
    a.slot_expert[i] = e;
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
// With kCsrLds the move tables are staged in LDS as well (when they fit).
// Every global read a workgroup needs before its first pass (its first 8
// rounds of ids, the status, the per-expert tables and its chunk prefix) is
// issued up front, so they share one memory round trip.
template <bool kCsrLds>
__global__ __launch_bounds__(kPlanThreads) void k_route(PlanArgs a) {
  constexpr int kEPer = MOE_MAX_E / kPlanThreads;            // experts per thread
  constexpr int kMPer = (MOE_MAX_E + MOE_MAX_R + kPlanThreads - 1) / kPlanThreads;
  extern __shared__ int s_cnt[];  // [16][E], then the per-expert tables
  const int E = a.E, M = a.M;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const uint64_t lt = lanemask_lt();
  const int64_t base = int64_t(blockIdx.x) * kRouteWaves * a.L + int64_t(w) * a.L;
  const int64_t lim = min<int64_t>(a.N, base + a.L);
  int* cnt = s_cnt + w * E;
  int* s_taken = s_cnt + kRouteWaves * E;     // [E] LDS copies of the
  int* s_home = s_taken + E;                  // [E] per-expert route tables
  int* s_mptr = s_home + E;                   // [E]  (kCsrLds only)
  int* s_mcnt = s_mptr + E;                   // [E]
  int* s_lo = s_mcnt + E;                     // [M]
  int* s_hi = s_lo + M;                       // [M]
  int* s_base = s_hi + M;                     // [M]

  auto load8 = [&](int64_t b0, int* ids8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = b0 + u * kWave + lane;
      ids8[u] = i < lim ? a.ids[i] : E;
    }
  };
  int first[8];
  load8(base, first);
  const int st = a.status[2];
  int t_taken[kEPer], t_home[kEPer], t_mptr[kEPer], t_mcnt[kEPer], t_cc[kEPer];
  const int32_t* ccp = a.cc + int64_t(blockIdx.x) * E;
#pragma unroll
  for (int k = 0; k < kEPer; ++k) {
    const int e = tid + k * kPlanThreads;
    if (e < E) {
      t_taken[k] = a.taken[e];
      t_home[k] = a.home_base[e];
      t_cc[k] = ccp[e];
      if (kCsrLds) { t_mptr[k] = a.mptr[e]; t_mcnt[k] = a.mcnt[e]; }
    }
  }
  int t_lo[kMPer], t_hi[kMPer], t_base[kMPer];
  if (kCsrLds) {
#pragma unroll
    for (int k = 0; k < kMPer; ++k) {
      const int q = tid + k * kPlanThreads;
      if (q < M) { t_lo[k] = a.cs_lo[q]; t_hi[k] = a.cs_hi[q]; t_base[k] = a.cs_base[q]; }
    }
  }
  // This workgroup's share of cu_seqlens (all zero when there is no plan):
  // rows of rank r before weight row j, from the per-rank prefixes of home
  // rows, prefetch rows and overflow rows (inference) that k_plan exported.
  auto write_cu = [&](bool ok) {
    const int n = a.n, B = a.B, W = E + B + 1, tot = a.R * W;
    const int per = (tot + gridDim.x - 1) / gridDim.x;
    const int i0 = blockIdx.x * per, i1 = min(tot, i0 + per);
    const bool infer = a.mode == MOE_MODE_INFER;
    for (int i = i0 + tid; i < i1; i += kPlanThreads) {
      int v = 0;
      if (ok) {
        const int r = i / W, j = i % W;
        const int32_t* hp = a.hpre + r * (n + 1);
        if (j <= E) {
          v = hp[min(max(j - r * n, 0), n)];
          if (infer) {
            // overflow moves of r ascend in expert id: count those below j
            const int lo0 = a.rinfo[3 * r + 1];
            int lo = lo0, hi = a.rinfo[3 * r + 2];
            while (lo < hi) {
              const int mid = (lo + hi) >> 1;
              if (a.moves[4 * mid] < j) lo = mid + 1; else hi = mid;
            }
            if (lo > lo0) v += a.ocum[lo - 1];
          }
        } else {
          v = hp[n] + a.rinfo[3 * r] + a.spre[r * (B + 1) + (j - E)];
        }
      }
      a.cu[i] = v;
    }
  };
  if (st & (MOE_STATUS_BAD_ID | MOE_STATUS_UNBALANCED | MOE_STATUS_INTERNAL)) {
    for (int64_t i = base + lane; i < lim; i += kWave) a.route[i] = -1;
    write_cu(false);
    return;
  }
#pragma unroll
  for (int k = 0; k < kEPer; ++k) {
    const int e = tid + k * kPlanThreads;
    if (e < E) {
      s_taken[e] = t_taken[k];
      s_home[e] = t_home[k];
      if (kCsrLds) { s_mptr[e] = t_mptr[k]; s_mcnt[e] = t_mcnt[k]; }
    }
  }
  if (kCsrLds) {
#pragma unroll
    for (int k = 0; k < kMPer; ++k) {
      const int q = tid + k * kPlanThreads;
      if (q < M) { s_lo[q] = t_lo[k]; s_hi[q] = t_hi[k]; s_base[q] = t_base[k]; }
    }
  }
  for (int e = lane; e < E; e += kWave) cnt[e] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // pass A: per-wave counts (LDS atomics; lanes sharing a key serialise)
  auto count8 = [&](const int* ids8) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if ((unsigned)ids8[u] < (unsigned)E) atomicAdd(&cnt[ids8[u]], 1);
  };
  count8(first);
  for (int64_t b0 = base + 8 * kWave; b0 < lim; b0 += 8 * kWave) {
    int ids8[8];
    load8(b0, ids8);
    count8(ids8);
  }
  write_cu(true);
  __syncthreads();
  // exclusive prefix over the 16 waves, on top of the chunk's prefix
#pragma unroll
  for (int k = 0; k < kEPer; ++k) {
    const int e = tid + k * kPlanThreads;
    if (e < E) {
      int run = t_cc[k];
      for (int ww = 0; ww < kRouteWaves; ++ww) {
        const int v = s_cnt[ww * E + e];
        s_cnt[ww * E + e] = run;
        run += v;
      }
    }
  }
  __syncthreads();
  // pass B: ranks and destinations.  Each slot takes a provisional rank
  // from one LDS fetch-add on its expert's counter (lanes of a round that
  // share an expert get consecutive values, in an order the hardware
  // picks); the lanes of every key that more than one lane holds are then
  // ranked again in lane order, one ballot per such key.  The counter ends
  // each round advanced by the round's slots of that expert either way.
  auto route8 = [&](int64_t b0, const int* ids8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = b0 + u * kWave + lane;
      const int key = ids8[u];
      const bool ok = key < E;
      int before = 0, p = 0;
      if (ok) {
        before = cnt[key];
        p = atomicAdd(&cnt[key], 1);
      }
      uint64_t pend = __ballot(ok && p != before);     // lanes not served first
      while (pend) {
        const int ld = __ffsll((unsigned long long)pend) - 1;
        const int k = wave_bcast(key, ld);
        const uint64_t m = __ballot(ok && key == k);
        if (ok && key == k) p = before + (int)__popcll(m & lt);
        pend &= ~m;
      }
      if (ok) {
        int dest = -1;
        if (p >= s_taken[key]) {
          dest = s_home[key] + p;
        } else if (kCsrLds) {
          const int q0 = s_mptr[key], q1 = q0 + s_mcnt[key];
          for (int q = q0; q < q1; ++q)
            if (p >= s_lo[q] && p < s_hi[q]) { dest = s_base[q] + p; break; }
        } else {
          const int q0 = a.mptr[key], q1 = q0 + a.mcnt[key];
          for (int q = q0; q < q1; ++q)
            if (p >= a.cs_lo[q] && p < a.cs_hi[q]) { dest = a.cs_base[q] + p; break; }
        }
        a.route[i] = dest;
      }
    }
  };
  route8(base, first);
  for (int64_t b0 = base + 8 * kWave; b0 < lim; b0 += 8 * kWave) {
    int ids8[8];
    load8(b0, ids8);
    route8(b0, ids8);
  }
}

static size_t plan_lds_bytes(const moe_cfg* c, const PlanLayout& L) {
  // the k_plan LDS layout: 4 arrays of E, 5 of R, 6 of M, R(n+1), R(B+1), scan scratch
  const size_t E = c->E, R = c->R, n = E / R, B = c->B;
  return sizeof(int) * (4 * E + 5 * R + 6 * size_t(L.M) + R * (n + 1) + R * (B + 1) +
                        kPlanThreads + 32);
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

extern "C" int moe_plan_run_policy(const moe_cfg* cfg, const int32_t* topk_ids,
                                   const moe_plan* plan, int32_t policy, hipStream_t stream) {
  int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if (policy != MOE_PLAN_ASCENDING && policy != MOE_PLAN_LARGEST_FIRST) return MOE_EINVAL;
  if (!plan_ptrs_ok(plan)) return MOE_EINVAL;
  const PlanLayout L = plan_layout(cfg);
  if (L.N > 0 && (!topk_ids || !plan->route)) return MOE_EINVAL;
  PlanArgs a;
  a.ids = topk_ids;
  a.N = (int32_t)L.N;
  a.R = cfg->R; a.S = cfg->S; a.E = cfg->E; a.K = cfg->K; a.B = cfg->B; a.mode = cfg->mode;
  a.n = cfg->E / cfg->R;
  a.SK = cfg->S * cfg->K;
  a.L = L.L; a.C = L.C; a.M = L.M;
  a.policy = policy;
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
  a.hpre = ws_i32(ws, L.off_hpre); a.spre = ws_i32(ws, L.off_spre);
  a.rinfo = ws_i32(ws, L.off_rinfo); a.ocum = ws_i32(ws, L.off_ocum);

  const size_t lds_count = sizeof(int) * cfg->E;
  const size_t lds_plan = plan_lds_bytes(cfg, L);
  const size_t lds_route = sizeof(int) * size_t(kRouteWaves + 2) * cfg->E;
  const size_t lds_route_csr = lds_route + sizeof(int) * (size_t(2) * cfg->E + size_t(3) * L.M);
  const bool csr_lds = lds_route_csr <= kMaxLds;
  if ((rc = allow_lds(k_plan, lds_plan)) != MOE_OK) return rc;
  if (csr_lds) {
    if ((rc = allow_lds(k_route<true>, lds_route_csr)) != MOE_OK) return rc;
  } else {
    if ((rc = allow_lds(k_route<false>, lds_route)) != MOE_OK) return rc;
  }
  if (L.C > 0) {
    hipLaunchKernelGGL(k_count, dim3(L.C), dim3(kPlanThreads), lds_count, stream, a);
    hipLaunchKernelGGL(k_colscan, dim3((cfg->E + kWave - 1) / kWave), dim3(kPlanThreads), 0,
                       stream, a);
  } else {
    hipLaunchKernelGGL(k_zero_counts, dim3(1), dim3(kPlanThreads), 0, stream, a);
  }
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(kPlanThreads), lds_plan, stream, a);
  if (L.C > 0) {
    if (csr_lds)
      hipLaunchKernelGGL((k_route<true>), dim3(L.C), dim3(kPlanThreads), lds_route_csr, stream, a);
    else
      hipLaunchKernelGGL((k_route<false>), dim3(L.C), dim3(kPlanThreads), lds_route, stream, a);
  }
  return hip_status();
}

extern "C" int moe_plan_run(const moe_cfg* cfg, const int32_t* topk_ids, const moe_plan* plan,
                            hipStream_t stream) {
  return moe_plan_run_policy(cfg, topk_ids, plan, MOE_PLAN_ASCENDING, stream);
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
