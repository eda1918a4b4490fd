// Grouped GEMM over the [E+B, H, H'] weight view, and its fp32 weight
// gradient, on gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Sources: "Moonshot AI 开源 MoonEP", 核心思想 (the grouped GEMM addresses
// experts only by row index of one [E+B, H, H'] tensor; cu_seqlens[E+B]
// picks the active rows; gradients mirror the layout in fp32 with rows
// [E, E+B) in a separate reduce buffer); "Kimi K3 模型结构（8）", rank 内部
// (per-expert row counts stay skewed inside a rank, so work is handed out by
// a load-aware scheduler rather than in a fixed order).
//
// Structure:
//   k_sched_*   one workgroup turns cu_seqlens into a flat work list on the
//               device (no host round trip: the grid never depends on it);
//   k_gemm<MODE> a persistent grid, one 256-thread workgroup per CU, pulls
//               256x256 output tiles from that list.  Consecutive work items
//               go to the 32 workgroups of one XCD (blockIdx % 8 picks the
//               XCD), so the A panel and the weight panels of neighbouring
//               tiles are shared in that XCD's L2.
// Tile: BM = BN = 256, BK = 64; 4 waves in a 2x2 grid, each 128x128 =
// 4x4 MFMA blocks of 32x32 with fp32 accumulators.  Both operands are
// staged through LDS (double buffered, 2 x 64 KB) in [row][k] order with a
// 16-byte-chunk XOR swizzle.  Operands whose k index is strided in memory
// (the weight [H][H'] in the forward; both operands of the weight
// gradient) are loaded as 8x8 bf16 blocks and transposed in registers
// before the LDS store.
#include <algorithm>

#include "common.hpp"
#include "host.hpp"

namespace moonep {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kGemmThreads = 256;
constexpr int kTileBytes = BM * BK * 2;          // 32 KB per operand tile
constexpr int kCRow = 272;                        // epilogue row pitch (bytes)
constexpr int kGemmLds = 4 * 128 * kCRow;         // >= A and B double buffered (128 KB)

enum { MODE_FWD = 0, MODE_WGRAD = 1 };

struct WorkItem {
  int32_t r, j, row0, rows;  // rank, weight row, first xperm row (absolute), row count
};

struct GemmArgs {
  const uint16_t* xperm;
  const uint16_t* w_home;
  const uint16_t* w_pref;
  const uint16_t* dy;
  uint16_t* y;
  float* grad_home;
  float* grad_pref;
  const WorkItem* items;
  const int32_t* nitems;
  int32_t H, Hp, E, B, SK;
};

// Byte offset of 16-byte chunk kc of row `row` in a [256][64] bf16 LDS tile.
__device__ __forceinline__ int lds_off(int row, int kc) {
  return row * (BK * 2) + ((kc ^ ((row >> 1) & 7)) << 4);
}

// Column c of an 8x8 bf16 block held as 8 rows (one u32x4 per row): the 8
// values in[0..7][c], packed two per dword.
__device__ __forceinline__ u32x4 transpose_col(const u32x4 (&in)[8], int c) {
  u32x4 out;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t a = in[2 * d][c >> 1], b = in[2 * d + 1][c >> 1];
    out[d] = (c & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
  }
  return out;
}

template <int MODE>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm(GemmArgs g) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave;
  const int wm = wv >> 1, wn = wv & 1;
  const int H = g.H, Hp = g.Hp;
  const int MDIM = MODE == MODE_FWD ? 0 : H;     // wgrad: output rows are h
  const int ntm = MODE == MODE_FWD ? 1 : (MDIM + BM - 1) / BM;
  const int ntn = (Hp + BN - 1) / BN;
  const int64_t total = int64_t(*g.nitems) * ntm * ntn;
  const int G = gridDim.x, per = G / 8;
  const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;

  for (int64_t q = 0;; ++q) {
    const int64_t w = q * G + int64_t(xcd) * per + local;
    if (w >= total) break;
    const int64_t item = w / (ntm * ntn);
    const int rest = (int)(w % (ntm * ntn));
    const int tm = rest / ntn, tn = rest % ntn;
    const WorkItem it = g.items[item];
    const int n0 = tn * BN;
    const int m0 = tm * BM;  // wgrad: first h of the tile
    // K extent: H for the forward, the segment length for the wgrad
    const int KD = MODE == MODE_FWD ? H : it.rows;
    const int nk = (KD + BK - 1) / BK;

    // Uniform (scalar) bases plus 32-bit per-lane element offsets, so the
    // loads use scalar-base addressing and few vector registers.
    const uint16_t* Ab = g.xperm + int64_t(it.row0) * H;
    const uint16_t* Bb;
    if (MODE == MODE_FWD)
      Bb = it.j < g.E ? g.w_home + int64_t(it.j) * H * Hp
                      : g.w_pref + (int64_t(it.r) * g.B + (it.j - g.E)) * H * Hp;
    else
      Bb = g.dy + int64_t(it.row0) * Hp;
    const int kg = tid & 7, cg = tid >> 3;   // 8x8 block: k group, column group
    // forward A: rows cg + 32i (masked to the segment), chunk kg
    uint32_t aoff = 0;
    int arow_lim = 0;
    if (MODE == MODE_FWD) {
      aoff = uint32_t(cg) * H + kg * 8;
      arow_lim = it.rows - cg;               // row cg + 32i valid iff 32i < arow_lim
    } else {
      aoff = uint32_t(kg * 8) * H + m0 + cg * 8;
    }
    const uint32_t boff = uint32_t(kg * 8) * Hp + n0 + cg * 8;
    const bool bcol_ok = n0 + cg * 8 < Hp;
    const bool acol_ok = MODE == MODE_FWD ? true : (m0 + cg * 8 < H);

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    u32x4 ra[8], rb[8];
    const u32x4 zero4 = {0, 0, 0, 0};
    // Global -> registers for k-tile kt.
    auto load = [&](int kt) {
      const int k0 = kt * BK;
      if (MODE == MODE_FWD) {
        const uint16_t* a = Ab + k0;
        const bool kok = k0 + kg * 8 < H;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          ra[i] = (kok && 32 * i < arow_lim)
                      ? *reinterpret_cast<const u32x4*>(a + aoff + uint32_t(32 * i) * H)
                      : zero4;
      } else {
        const uint16_t* a = Ab + int64_t(k0) * H;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          ra[i] = (acol_ok && k0 + kg * 8 + i < KD)
                      ? *reinterpret_cast<const u32x4*>(a + aoff + uint32_t(i) * H)
                      : zero4;
      }
      const uint16_t* b = Bb + int64_t(k0) * Hp;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        rb[i] = (bcol_ok && k0 + kg * 8 + i < KD)
                    ? *reinterpret_cast<const u32x4*>(b + boff + uint32_t(i) * Hp)
                    : zero4;
    };
    // Registers -> LDS buffer `buf`; 8x8 blocks are transposed on the way.
    // The swizzle of row cg + 32i is that of row cg, and rows 8cg + c share
    // it in pairs (c, c + 1), so every address is a per-lane base plus a
    // compile-time offset.
    const int st_lin = lds_off(cg, kg);                 // forward A rows cg + 32i
    int st_tr[4];                                       // rows 8cg + c, c = 2p, 2p+1
#pragma unroll
    for (int p2 = 0; p2 < 4; ++p2) st_tr[p2] = lds_off(cg * 8 + 2 * p2, kg) - 2 * p2 * (BK * 2);
    auto store = [&](int buf) {
      unsigned char* As = lds + buf * 2 * kTileBytes;
      unsigned char* Bs = As + kTileBytes;
      if (MODE == MODE_FWD) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          *reinterpret_cast<u32x4*>(As + st_lin + i * 32 * (BK * 2)) = ra[i];
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c)
          *reinterpret_cast<u32x4*>(As + st_tr[c >> 1] + c * (BK * 2)) = transpose_col(ra, c);
      }
#pragma unroll
      for (int c = 0; c < 8; ++c)
        *reinterpret_cast<u32x4*>(Bs + st_tr[c >> 1] + c * (BK * 2)) = transpose_col(rb, c);
    };
    // MFMA operand reads: row wm*128 + 32i + lane%32 (resp. wn) has the
    // swizzle of lane%32; only the 16-byte chunk 2s + lane/32 varies with s.
    int rd_a[BK / 16], rd_b[BK / 16];
#pragma unroll
    for (int s2 = 0; s2 < BK / 16; ++s2) {
      rd_a[s2] = lds_off(wm * 128 + (lane & 31), 2 * s2 + (lane >> 5));
      rd_b[s2] = lds_off(wn * 128 + (lane & 31), 2 * s2 + (lane >> 5));
    }

    if (nk > 0) {
      load(0);
      store(0);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const bool more = kt + 1 < nk;
      if (more) load(kt + 1);
      const unsigned char* As = lds + (kt & 1) * 2 * kTileBytes;
      const unsigned char* Bs = As + kTileBytes;
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        bf16x8 af[4], bfr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          af[i] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(As + rd_a[s] + i * 32 * (BK * 2)));
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bfr[j] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(Bs + rd_b[s] + j * 32 * (BK * 2)));
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (more) store((kt + 1) & 1);
      __syncthreads();
    }

    // Epilogue.  32x32 accumulator layout: lane l holds column l % 32 and
    // rows 8*(v/4) + 4*(l/32) + v%4 of its block for v = 0..15.
    if (MODE == MODE_FWD) {
      // Stage the wave's 128x128 bf16 sub-tile in LDS (rows padded to 272
      // bytes), then write whole 16-byte row chunks.
      unsigned char* Cs = lds + wv * (128 * kCRow);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int mm = 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            const int nn = 32 * j + (lane & 31);
            *reinterpret_cast<uint16_t*>(Cs + mm * kCRow + nn * 2) =
                (uint16_t)f32_to_bf16(acc[i][j][v]);
          }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      uint16_t* yb = g.y + int64_t(it.row0) * Hp;
#pragma unroll 4
      for (int c = lane; c < 128 * 16; c += kWave) {
        const int rr = c >> 4, cc = c & 15;
        const int m = wm * 128 + rr;
        const int n = n0 + wn * 128 + cc * 8;
        if (m < it.rows && n < Hp)
          *reinterpret_cast<u32x4*>(yb + uint32_t(m) * Hp + n) =
              *reinterpret_cast<const u32x4*>(Cs + rr * kCRow + cc * 16);
      }
      __syncthreads();
    } else {
      float* out = it.j < g.E ? g.grad_home + int64_t(it.j) * H * Hp
                              : g.grad_pref + (int64_t(it.r) * g.B + (it.j - g.E)) * H * Hp;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + wn * 128 + 32 * j + (lane & 31);
          if (n >= Hp) continue;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int h = m0 + wm * 128 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (h < H) out[uint32_t(h) * Hp + n] = acc[i][j][v];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Work lists.  Forward: one item per 256-row m-tile of every non-empty
// segment of ranks [rb, re), in (rank, weight row, m) order.  Weight
// gradient: one item per segment that owns a gradient row -- every home row
// of the rank (empty ones write zeros) and every non-empty prefetch row.
// ---------------------------------------------------------------------------
struct SchedArgs {
  const int32_t* cu;
  WorkItem* items;
  int32_t* nitems;
  int32_t rb, re, E, B, n, SK, cap;
};

template <int MODE>
__global__ __launch_bounds__(1024) void k_sched(SchedArgs s) {
  __shared__ int scratch[32];
  __shared__ int s_carry;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int rows = s.E + s.B;
  const int64_t total = int64_t(s.re - s.rb) * rows;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int64_t c0 = 0; c0 < total; c0 += 1024) {
    const int64_t idx = c0 + tid;
    int cnt = 0, r = 0, j = 0, lo = 0, len = 0;
    if (idx < total) {
      r = s.rb + (int)(idx / rows);
      j = (int)(idx % rows);
      const int32_t* cu = s.cu + int64_t(r) * (rows + 1);
      lo = cu[j];
      len = cu[j + 1] - lo;
      if (MODE == MODE_FWD) {
        cnt = (len + BM - 1) / BM;
      } else {
        const bool home = j < s.E && j / s.n == r;
        cnt = (home || (j >= s.E && len > 0)) ? 1 : 0;
      }
    }
    const int incl = wave_incl_scan(cnt);
    if (lane == kWave - 1) scratch[wave] = incl;
    __syncthreads();
    if (wave == 0) {
      const int v = lane < 16 ? scratch[lane] : 0;
      const int vi = wave_incl_scan(v);
      if (lane < 16) scratch[lane] = vi - v;
      if (lane == 15) scratch[16] = vi;
    }
    __syncthreads();
    const int base = s_carry + scratch[wave] + incl - cnt;
    for (int m = 0; m < cnt; ++m) {
      const int at = base + m;
      if (at < s.cap) {
        WorkItem w;
        w.r = r;
        w.j = j;
        if (MODE == MODE_FWD) {
          w.row0 = r * s.SK + lo + m * BM;
          w.rows = min(BM, len - m * BM);
        } else {
          w.row0 = r * s.SK + lo;
          w.rows = len;
        }
        s.items[at] = w;
      }
    }
    __syncthreads();
    if (tid == 0) s_carry += scratch[16];
    __syncthreads();
  }
  if (tid == 0) *s.nitems = min(s_carry, s.cap);
}

static int g_num_cus = 0;

static int num_cus() {
  if (g_num_cus > 0) return g_num_cus;
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    v = 256;
  g_num_cus = v;
  return v;
}

static int64_t fwd_capacity(const moe_cfg* c, int nranks) {
  return int64_t(nranks) * ((int64_t(c->S) * c->K + BM - 1) / BM + c->E + c->B);
}

static int64_t wgrad_capacity(const moe_cfg* c) { return int64_t(c->E) + int64_t(c->R) * c->B; }

static size_t gemm_ws_bytes(const moe_cfg* c) {
  const int64_t cap = std::max(fwd_capacity(c, c->R), wgrad_capacity(c));
  return 256 + size_t(cap) * sizeof(WorkItem);
}

static int launch_gemm(int mode, const moe_cfg* c, GemmArgs& g, SchedArgs& s, hipStream_t stream) {
  int rc;
  if (mode == MODE_FWD) {
    if ((rc = allow_lds(k_gemm<MODE_FWD>, kGemmLds)) != MOE_OK) return rc;
    hipLaunchKernelGGL(k_sched<MODE_FWD>, dim3(1), dim3(1024), 0, stream, s);
  } else {
    if ((rc = allow_lds(k_gemm<MODE_WGRAD>, kGemmLds)) != MOE_OK) return rc;
    hipLaunchKernelGGL(k_sched<MODE_WGRAD>, dim3(1), dim3(1024), 0, stream, s);
  }
  int G = num_cus();
  G = std::max(8, G - G % 8);
  if (mode == MODE_FWD)
    hipLaunchKernelGGL(k_gemm<MODE_FWD>, dim3(G), dim3(kGemmThreads), kGemmLds, stream, g);
  else
    hipLaunchKernelGGL(k_gemm<MODE_WGRAD>, dim3(G), dim3(kGemmThreads), kGemmLds, stream, g);
  return hip_status();
}

}  // namespace moonep

using namespace moonep;

extern "C" int moe_gemm_workspace_size(const moe_cfg* cfg, size_t* bytes_out) {
  const int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if (!bytes_out) return MOE_EINVAL;
  *bytes_out = gemm_ws_bytes(cfg);
  return MOE_OK;
}

extern "C" int moe_grouped_gemm(const moe_cfg* cfg, const moe_bf16* xperm, const moe_bf16* w_home,
                                const moe_bf16* w_pref, const int32_t* cu_seqlens, moe_bf16* y,
                                int32_t rank_begin, int32_t rank_end, void* workspace,
                                hipStream_t stream) {
  const int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if (rank_begin < 0 || rank_end > cfg->R || rank_begin > rank_end) return MOE_EINVAL;
  if (rank_begin == rank_end || cfg->S == 0) return MOE_OK;
  if (!xperm || !w_home || !cu_seqlens || !y || !workspace) return MOE_EINVAL;
  if (cfg->B > 0 && !w_pref) return MOE_EINVAL;
  GemmArgs g{};
  g.xperm = xperm; g.w_home = w_home; g.w_pref = w_pref; g.y = y;
  g.H = cfg->H; g.Hp = cfg->Hp; g.E = cfg->E; g.B = cfg->B; g.SK = cfg->S * cfg->K;
  SchedArgs s{};
  s.cu = cu_seqlens;
  s.nitems = reinterpret_cast<int32_t*>(workspace);
  s.items = reinterpret_cast<WorkItem*>(reinterpret_cast<char*>(workspace) + 256);
  s.rb = rank_begin; s.re = rank_end; s.E = cfg->E; s.B = cfg->B; s.n = cfg->E / cfg->R;
  s.SK = cfg->S * cfg->K;
  s.cap = (int32_t)fwd_capacity(cfg, rank_end - rank_begin);
  g.items = s.items;
  g.nitems = s.nitems;
  return launch_gemm(MODE_FWD, cfg, g, s, stream);
}

extern "C" int moe_grouped_gemm_wgrad(const moe_cfg* cfg, const moe_plan* plan,
                                      const moe_bf16* xperm, const moe_bf16* dy, float* grad_home,
                                      float* grad_pref, void* workspace, hipStream_t stream) {
  const int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if (cfg->mode != MOE_MODE_TRAIN) return MOE_EINVAL;
  if (!plan || !plan->cu_seqlens || !xperm || !dy || !grad_home || !workspace) return MOE_EINVAL;
  if (cfg->B > 0 && !grad_pref) return MOE_EINVAL;
  GemmArgs g{};
  g.xperm = xperm; g.dy = dy; g.grad_home = grad_home; g.grad_pref = grad_pref;
  g.H = cfg->H; g.Hp = cfg->Hp; g.E = cfg->E; g.B = cfg->B; g.SK = cfg->S * cfg->K;
  SchedArgs s{};
  s.cu = plan->cu_seqlens;
  s.nitems = reinterpret_cast<int32_t*>(workspace);
  s.items = reinterpret_cast<WorkItem*>(reinterpret_cast<char*>(workspace) + 256);
  s.rb = 0; s.re = cfg->R; s.E = cfg->E; s.B = cfg->B; s.n = cfg->E / cfg->R;
  s.SK = cfg->S * cfg->K;
  s.cap = (int32_t)wgrad_capacity(cfg);
  g.items = s.items;
  g.nitems = s.nitems;
  return launch_gemm(MODE_WGRAD, cfg, g, s, stream);
}
