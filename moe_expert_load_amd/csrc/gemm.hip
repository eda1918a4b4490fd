// Grouped GEMM over the [E+B, H, H'] weight view, its fp32 weight gradient
// and its data gradient, on gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Sources: "Moonshot AI 开源 MoonEP", 核心思想 (the grouped GEMM addresses
// experts only by row index of one [E+B, H, H'] tensor; cu_seqlens[E+B]
// picks the active rows; gradients mirror the layout in fp32 with rows
// [E, E+B) in a separate reduce buffer); "Kimi K3 模型结构（8）", rank 内部
// (per-expert row counts stay skewed inside a rank, so work is handed out by
// a load-aware scheduler rather than in a fixed order); "大规模 LLM 训练系统
// 研究账本" §9.5 (the backward runs over the rows dispatch laid out).
//
// Structure:
//   k_sched<MODE> one workgroup turns cu_seqlens into a flat work list on the
//               device (no host round trip: the grid never depends on it);
//   k_gemm<MODE> a persistent grid, one 256-thread workgroup per CU, pulls
//               256x256 output tiles from that list.  Consecutive work items
//               go to the 32 workgroups of one XCD (blockIdx % 8 picks the
//               XCD); inside bands of 8 row tiles of a segment the forward
//               and the data gradient go column tile by column tile, so the
//               CUs of one XCD share each weight panel across the band's row
//               tiles in that XCD's L2, and a long segment streams its rows
//               once per band rather than once per column tile.
//   k_wgrad     the weight gradient G = xperm_seg^T @ dy_seg (fp32) on
//               384 x 256 tiles with 8 waves (see its own comment).
//   MODE 0: y = xperm_seg @ W (forward); MODE 1: the weight gradient
//   (k_wgrad only); MODE 2: dxperm_seg = dy_seg @ W^T (data
//   gradient, over the forward's work list); MODE 3: the first projection
//   of a SwiGLU expert, act = silu(x W_gate) * (x W_up) with W13 = [W_gate |
//   W_up] in one [E+B, H, 2H'] tensor -- each 256-column tile takes 128
//   gate and the same 128 up columns, interleaved in 32-column blocks, so
//   every wave holds gate and up of the same outputs in its accumulators
//   and applies the activation in registers.
// Tile: BM = BN = 256, BK = 32; 4 waves in a 2x2 grid, each 128x128 =
// 4x4 MFMA blocks of 32x32 with fp32 accumulators (256 AGPRs per wave).
// Operands go from global memory straight into LDS (buffer_load ... lds,
// range-checked so ragged tails read zeros) through a 4-stage ring of
// separate LDS arrays, with 16-byte-chunk XOR swizzles that make every LDS
// read conflict free.  An operand whose k index is contiguous (the permuted
// activations in the forward; dy and the weight rows in the data gradient)
// is a "row tile" read with ds_read_b128; an operand whose k index is
// strided (the weight [H][H'] in the forward; x^T and dy in the weight
// gradient) is stored as loaded, [k][col], and read with the transposing
// ds_read_b64_tr_b16, which returns 4 consecutive k per lane.  Fragment
// reads of the next 16-deep substep are interleaved with the MFMAs of the
// current one.  The A operand of the forward and of the data gradient (a row
// tile) goes in pairs of k-tiles through three 32 KB buffers, so its loads
// are whole 128-byte lines: a CU keeps only about 64 L2 requests in flight,
// and that bound, not the matrix pipe, sets these kernels' speed.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "host.hpp"

namespace moonep {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int BM = 256, BN = 256;

// Work order of the forward: 0 = row tile major (each row tile's column
// tiles adjacent), 1 = column tile major inside a segment.
#ifndef MOONEP_FWD_NMAJOR
#define MOONEP_FWD_NMAJOR 1
#endif
constexpr int kGemmThreads = 256;

// Row-tile A operands interleave the two wave rows by 32-row blocks: wave
// row wm holds tile rows 64 i + 32 wm + [0, 32), i = 0..3, so a tile with
// few rows leaves both wave rows equally idle.
constexpr int kAWaveRow = 32;   // rows between the wave rows
constexpr int kABlock = 64;     // rows between a wave's row blocks

// Row tiles per band of the column-tile-major work order (a segment of at
// most this many row tiles is one band).
#ifndef MOONEP_GEMM_BAND
#define MOONEP_GEMM_BAND 8
#endif
constexpr int kBand = MOONEP_GEMM_BAND;

enum { MODE_FWD = 0, MODE_WGRAD = 1, MODE_DGRAD = 2, MODE_SWIGLU = 3 };

struct WorkItem {
  int32_t r, j, row0, rows;  // rank, weight row, first xperm row (absolute), row count
  int32_t first, cnt;        // row-tile lists: the segment's first item and its item count
};

struct GemmArgs {
  const uint16_t* xperm;
  const uint16_t* w_home;
  const uint16_t* w_pref;
  const uint16_t* dy;
  uint16_t* y;                // forward output; the data gradient's output (dxperm);
                              // the SwiGLU forward's activation
  uint16_t* h13;              // SwiGLU forward: gate and up outputs (optional)
  float* grad_home;
  float* grad_pref;
  const WorkItem* items;      // work list of this launch's tile class
  const int32_t* nitems;      // its item count
  int32_t H, Hp, E, B, SK;
};

// Cache-policy operand of the buffer-store builtin: non-temporal.
constexpr int kStoreNT = 2;

// Range-checked buffer resource over [base, base + bytes): loads past the end
// return zeros (per dword), which pads ragged row/K tails with zeros.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return u32x4{uint32_t(b), uint32_t(b >> 32) & 0xffffu, bytes, 0x00020000u};
}

// 16 bytes per lane from global memory straight into LDS (buffer_load ...
// lds): lane l writes lds_dst + 16*l; lds_dst must be wave-uniform.  Issued
// as inline assembly so the compiler does not pair every later LDS read with
// a wait for all such loads; the kernel waits for each stage itself
// (wait_vm) before the barrier that publishes it.
__device__ __forceinline__ void load_lds16(u32x4 rsrc, const unsigned char* lds_dst,
                                           uint32_t voff, uint32_t soff) {
  // every operand but voff is wave-uniform; make that explicit (scalar regs)
  const uint32_t l =
      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(lds_void*)lds_dst);
  u32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = (uint32_t)__builtin_amdgcn_readfirstlane((int)rsrc[q]);
  const uint32_t so = (uint32_t)__builtin_amdgcn_readfirstlane((int)soff);
  // one wait state between the scalar write of M0 and the LDS-DMA load that
  // reads it (a hazard of this GPU generation that the compiler's hazard pass
  // cannot see inside inline assembly)
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(l), "v"(voff), "s"(r), "s"(so) : "memory");
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Transposing LDS read: the 16 lanes of a group each name a 64-bit piece
// (4 bf16) of a 4-row x 16-column block; lane (a, c) = (i/4, i%4) receives
// column 4a + c of rows 0..3.  Used so that an operand stored [k][col] in
// LDS arrives as 8 consecutive k per lane, the MFMA layout.
__device__ __forceinline__ u32x2 lds_tr(const unsigned char* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ bf16x8 join(u32x2 lo, u32x2 hi) {
  return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Pipeline: kNST stages of BK-deep k-tiles.  BK = 64 (2 stages of 64 KB)
// makes every row of the k-contiguous forward operand a whole 128-byte line
// per stage; BK = 32 (4 stages of 32 KB) keeps more stages in flight.  Each
// stage's two operand tiles are separate LDS arrays so the compiler can
// tell a read of one stage from the in-flight direct loads of the others.
#ifndef MOONEP_GEMM_BK
#define MOONEP_GEMM_BK 32
#endif
#if MOONEP_GEMM_BK == 64
#define MOONEP_GEMM_STAGES 2
#elif !defined(MOONEP_GEMM_STAGES)
#define MOONEP_GEMM_STAGES 4
#endif
constexpr int kBK = MOONEP_GEMM_BK;
constexpr int kNST = MOONEP_GEMM_STAGES;
static_assert((kBK == 64 && kNST == 2) || (kBK == 32 && (kNST == 4 || kNST == 5)), "pipeline");
constexpr int kTile = 256 * kBK * 2;             // bytes per operand tile
__shared__ __attribute__((aligned(1024))) unsigned char g_sa0[kTile], g_sb0[kTile];
__shared__ __attribute__((aligned(1024))) unsigned char g_sa1[kTile], g_sb1[kTile];
#if MOONEP_GEMM_STAGES >= 4
__shared__ __attribute__((aligned(1024))) unsigned char g_sa2[kTile], g_sb2[kTile];
__shared__ __attribute__((aligned(1024))) unsigned char g_sa3[kTile], g_sb3[kTile];
#endif
#if MOONEP_GEMM_STAGES == 5
__shared__ __attribute__((aligned(1024))) unsigned char g_sa4[kTile], g_sb4[kTile];
#endif

template <int S>
__device__ __forceinline__ unsigned char* stage_a() {
  if constexpr (S == 0) return g_sa0;
  else if constexpr (S == 1) return g_sa1;
#if MOONEP_GEMM_STAGES >= 4
  else if constexpr (S == 2) return g_sa2;
  else if constexpr (S == 3) return g_sa3;
#endif
#if MOONEP_GEMM_STAGES == 5
  else if constexpr (S == 4) return g_sa4;
#endif
  else return nullptr;
}
template <int S>
__device__ __forceinline__ unsigned char* stage_b() {
  if constexpr (S == 0) return g_sb0;
  else if constexpr (S == 1) return g_sb1;
#if MOONEP_GEMM_STAGES >= 4
  else if constexpr (S == 2) return g_sb2;
  else if constexpr (S == 3) return g_sb3;
#endif
#if MOONEP_GEMM_STAGES == 5
  else if constexpr (S == 4) return g_sb4;
#endif
  else return nullptr;
}

// Paired row tiles: with MOONEP_GEMM_PAIRA, the k-contiguous A operand of
// the forward (xperm rows) and of the data gradient (dy rows) is loaded two
// k-tiles at a time, [256 rows][64 k] = 32 KB, so each 16-byte piece of a
// wave's 1 KB load is part of a whole 128-byte row line instead of half of
// one: the same bytes in half the L2 requests, and a CU keeps only about 64
// of those in flight.  Three pair buffers (96 KB) plus the four B stages
// (64 KB) fill the 160 KB of LDS.
#ifndef MOONEP_GEMM_PAIRA
#define MOONEP_GEMM_PAIRA 1
#endif
constexpr int kPairTile = 256 * 64 * 2;
__shared__ __attribute__((aligned(1024))) unsigned char g_pa0[kPairTile];
__shared__ __attribute__((aligned(1024))) unsigned char g_pa1[kPairTile];
__shared__ __attribute__((aligned(1024))) unsigned char g_pa2[kPairTile];

__device__ __forceinline__ unsigned char* pair_buf(int p) {
  const int b = p % 3;
  return b == 0 ? g_pa0 : b == 1 ? g_pa1 : g_pa2;
}

// Per-wave 16 KB staging area of the forward epilogue (reuses stage tiles).
__device__ __forceinline__ unsigned char* epilogue_area(int wv) {
#if MOONEP_GEMM_STAGES >= 4
  return wv == 0 ? g_sa0 : wv == 1 ? g_sa1 : wv == 2 ? g_sa2 : g_sa3;
#else
  return wv == 0 ? g_sa0 : wv == 1 ? g_sb0 : wv == 2 ? g_sa1 : g_sb1;
#endif
}

// A second per-wave 16 KB area, disjoint from every epilogue_area (the
// SwiGLU epilogue stages gate and up there beside the activation).
__device__ __forceinline__ unsigned char* epilogue_area2(int wv) {
#if MOONEP_GEMM_STAGES >= 4
  return wv == 0 ? g_sb0 : wv == 1 ? g_sb1 : wv == 2 ? g_sb2 : g_sb3;
#else
  return epilogue_area(wv) + 16384;     // the 2-stage arrays are 32 KB each
#endif
}

// Two fp32 values to a packed bf16 pair (lo in bits 0-15), rounded to
// nearest even by the hardware conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Workgroup barrier that orders this wave's LDS accesses around it but does
// not wait for outstanding global loads (the direct-to-LDS loads of later
// stages stay in flight; each wave waits for its own with wait_vm first).
__device__ __forceinline__ void barrier_lds() { asm volatile("s_barrier" ::: "memory"); }

// Tiles of one pipeline stage:
//  * "row tile" [256 rows][BK k] (forward A, k contiguous): 16-byte chunk kc
//    of row m is stored at chunk kc ^ ((m >> RSH) & (CPR - 1)) (CPR = BK/8
//    chunks per row, 2^RSH rows per 256 bytes), so 16 consecutive rows
//    reading one chunk hit 64 distinct banks;
//  * "col tile" [BK k][256 cols] (weights, dy, and x^T in the weight
//    gradient; columns contiguous): chunk c of row k is stored at
//    c ^ (4 * (k % 4)), so a transposing read of 4 rows x 4 chunks per 32
//    lanes is conflict free.
// Both are filled by buffer_load ... lds in whole 1 KB wave instructions;
// each lane fetches the global chunk whose swizzled position is its slot.
template <int MODE>
struct GemmTile {
  static constexpr int BK = kBK;
  static constexpr int ROWB = BK * 2;          // bytes per row-tile row
  static constexpr int CPR = BK / 8;           // 16-byte chunks per row-tile row
  static constexpr int RSH = CPR == 8 ? 1 : 2;  // rows per 256 bytes = 1 << RSH
  static constexpr int NI = kTile / 1024 / 4;  // 1 KB loads per wave per operand
  static constexpr int RPI = 1024 / ROWB;      // row-tile rows per load
};

// NBK: the tile class of this launch -- tiles of at most 64 NBK rows (4:
// any tile).  Each class runs as its own persistent launch over its own work
// list, so each kernel holds one instance of the k-loop.
template <int MODE, int NBK>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm(GemmArgs g) {
  static_assert(MODE != MODE_WGRAD && (NBK == 4 || NBK == 2 || NBK == 1), "mode, tile class");
  using T = GemmTile<MODE>;
  constexpr int BK = T::BK, ROWB = T::ROWB, CPR = T::CPR, RSH = T::RSH, NI = T::NI;
  static_assert(NI * 4096 == kTile && (CPR == 4 || CPR == 8), "tile geometry");
  constexpr int SUB = BK / 16;                 // MFMA k substeps per stage

  const int tid = threadIdx.x, lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wv >> 1, wn = wv & 1;
  // Operand tiles: A is always a "row tile" of k-contiguous rows; B is one
  // too in the data gradient and a "col tile" (k-strided rows) otherwise.
  constexpr bool kRowB = MODE == MODE_DGRAD;
  // Paired A tiles wherever A is a row tile (forward, data gradient, SwiGLU
  // projection).
  constexpr bool kPair = (MODE == MODE_FWD || MODE == MODE_DGRAD || MODE == MODE_SWIGLU) &&
                         MOONEP_GEMM_PAIRA && BK == 32 && kNST == 4;
  constexpr bool kSwi = MODE == MODE_SWIGLU;
  constexpr bool kNMajor =
      MODE == MODE_DGRAD || ((MODE == MODE_FWD || kSwi) && MOONEP_FWD_NMAJOR);
  const int H = g.H, Hp = g.Hp;
  const int WC = kSwi ? 2 * Hp : Hp;                     // weight / dy row length
  const int NOUT = MODE == MODE_DGRAD ? H : Hp;          // output columns
  // a SwiGLU tile yields 128 activation columns
  const int ntn = kSwi ? (Hp + BN / 2 - 1) / (BN / 2) : (NOUT + BN - 1) / BN;
  const int64_t total = int64_t(*g.nitems) * ntn;
  const int G = gridDim.x, per = G / 8;
  const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;

  // Per-lane pieces of the transposing reads (col tiles), see lds_tr:
  // G4 = lane/16 picks the k half (G4/2) and the column half (G4%2).
  const int G4 = lane >> 4, li = lane & 15;
  const int tr_k = 8 * (G4 >> 1) + (li >> 2);            // + 16 s + 4 h
  int tr_off[4];                                          // per 32-column block
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = (4 * j + 2 * (G4 & 1) + ((li & 3) >> 1)) ^ (4 * (li >> 2));
    tr_off[j] = tr_k * 512 + c * 16 + 8 * (li & 1);
  }
  // Row-tile MFMA reads, chunk 2 s + lane/32.  B (and a k-strided A):
  // row = wn*128 (wm*128) + 32 i + lane%32.  A row tiles interleave the two
  // wave rows by 32-row blocks, row = 64 i + 32 wm + lane%32, so a tile
  // with few rows leaves both wave rows equally idle (see kAStride).
  int ra_off[BK / 16], rb_off[BK / 16];
#pragma unroll
  for (int s = 0; s < BK / 16; ++s) {
    const int row = lane & 31, kc = 2 * s + (lane >> 5);
    const int sw = (kc ^ ((row >> RSH) & (CPR - 1))) << 4;
    ra_off[s] = (wm * kAWaveRow + row) * ROWB + sw;
    rb_off[s] = (wn * 128 + row) * ROWB + sw;
  }
  // Paired A tile reads: 128-byte rows, 8 chunks swizzled by (row / 2) % 8;
  // k-tile half h, substep s reads chunk 4 h + 2 s + lane/32.
  int rp_off[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int row = lane & 31, kc = 4 * h + 2 * s + (lane >> 5);
      rp_off[h][s] = (wm * kAWaveRow + row) * 128 + ((kc ^ ((row >> 1) & 7)) << 4);
    }

  // The work list is read-only here and every index is wave-uniform: read it
  // through the constant address space (scalar loads, counted by lgkmcnt),
  // so no wave has to wait for its vector-memory queue to fetch its next item.
  typedef __attribute__((address_space(4))) const WorkItem const_item;
  const const_item* items = (const const_item*)g.items;
  auto item_at = [&](int64_t i) {
    WorkItem v;
    v.r = items[i].r;
    v.j = items[i].j;
    v.row0 = items[i].row0;
    v.rows = items[i].rows;
    v.first = items[i].first;
    v.cnt = items[i].cnt;
    return v;
  };
  // Accumulators live across the persistent loop and are cleared per tile
  // (declared once here, the data gradient measured 2 % faster than with a
  // fresh array per tile).
  f32x16 acc[4][4];
  // Work index of this workgroup's q-th tile.
  auto work_index = [&](int64_t q) -> int64_t {
    return q * G + int64_t(xcd) * per + local;
  };
  const int arow = MODE == MODE_DGRAD ? Hp : H;          // A row length
  // Everything a tile's loads need: its place, its k-tile count, the two
  // range-checked operand resources and this lane's offsets into them.
  struct Tile {
    WorkItem it;
    int tn, KD, nk;
    u32x4 ra, rb;
    uint32_t goa[NI], gob[NI];
  };
  auto setup = [&](int64_t w) -> Tile {
    int tn;
    WorkItem it;
    if (kNMajor) {
      // Column-tile major inside bands of kBand row tiles of a segment: the
      // segment of row tiles [first, first + cnt) owns work
      // [first*ntn, (first + cnt)*ntn); band b holds its row tiles
      // [b*kBand, b*kBand + bc) and, inside the band, w is
      // (tn, row tile) = divmod(w - band start, bc).  Neighbouring work shares
      // one weight panel across the band's row tiles, and a long segment's
      // rows are streamed once per band instead of once per column tile.
      const WorkItem h = item_at(w / ntn);
      const int loc = (int)(w - int64_t(h.first) * ntn);
      const int b = loc / (kBand * ntn);
      const int bc = min(kBand, h.cnt - b * kBand);
      const int l = loc - b * kBand * ntn;
      tn = l / bc;
      it = item_at(h.first + b * kBand + l % bc);
    } else {
      tn = (int)(w % ntn);
      it = item_at(w / ntn);
    }
    const int n0 = tn * BN;
    const int KD = MODE == MODE_DGRAD ? Hp : H;
    // k-tiles, rounded up to whole passes over the stages (tiles past the end
    // load zeros; a ragged K is zeroed below)
    const int nk = ((KD + BK - 1) / BK + kNST - 1) / kNST * kNST;

    // Operand A: forward = xperm rows of the segment; data gradient = dy
    // rows (row tiles, k = h or h' contiguous).
    // Operand B: forward = weight W(r, j) [H][Hp] (col tile); data gradient
    // = W(r, j) read as W^T, i.e. rows h of W with k = h' contiguous (row
    // tile).
    const uint16_t* Abase = (MODE == MODE_DGRAD ? g.dy : g.xperm) + int64_t(it.row0) * arow;
    const uint16_t* Bbase = it.j < g.E ? g.w_home + int64_t(it.j) * H * WC
                                       : g.w_pref + (int64_t(it.r) * g.B + (it.j - g.E)) * H * WC;
    const uint32_t bbytes = uint32_t(H) * WC * 2;
    Tile X;
    X.it = it;
    X.tn = tn;
    X.KD = KD;
    X.nk = nk;
    X.ra = make_rsrc(Abase, uint32_t(it.rows) * arow * 2);
    X.rb = make_rsrc(Bbase, bbytes);

    // Per-lane global byte offsets of this wave's load instructions.
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int t = wv * NI + u;
      // row tile: load t covers rows t*RPI .. +RPI, 16-byte chunks swizzled
      const int rrow = t * T::RPI + lane / CPR;
      const int rkc = (lane % CPR) ^ ((rrow >> RSH) & (CPR - 1));
      // col tile: load t covers k rows 2t, 2t+1 of 256 columns
      const int crow = t * 2 + (lane >> 5);
      const int cc = (lane & 31) ^ (4 * (crow & 3));
      X.goa[u] = uint32_t(rrow) * arow * 2 + rkc * 16;
      // SwiGLU: 32-column block b of the tile is gate (b even) or up (b odd)
      // of activation columns tn*128 + (b/2)*32 + [0, 32).  Columns past the
      // activation width only feed accumulators that are never stored.
      const int col = kSwi ? ((cc >> 2) & 1) * Hp + tn * (BN / 2) + (cc >> 3) * 32 + 8 * (cc & 3)
                           : n0 + 8 * cc;
      if (kRowB) X.gob[u] = uint32_t(n0 + rrow) * Hp * 2 + rkc * 16;
      else X.gob[u] = uint32_t(crow) * WC * 2 + uint32_t(col) * 2;
    }
    return X;
  };
  // Direct loads of k-tile kt of tile X into stage S (= kt % kNST).
  auto issue_tile = [&](const Tile& X, auto S_, int kt) {
    constexpr int S = decltype(S_)::value;
    unsigned char* As = stage_a<S>();
    unsigned char* Bs = stage_b<S>();
    const uint32_t ka = uint32_t(kt) * BK * 2;
    const uint32_t kb = kRowB ? uint32_t(kt) * BK * 2 : uint32_t(kt) * BK * WC * 2;
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      load_lds16(X.ra, As + (wv * NI + u) * 1024, X.goa[u], ka);
      load_lds16(X.rb, Bs + (wv * NI + u) * 1024, X.gob[u], kb);
    }
  };
  // The first min(nk, kNST) k-tiles of tile X, one per stage.
  auto issue_first = [&](const Tile& X) {
    issue_tile(X, std::integral_constant<int, 0>(), 0);
    if (X.nk > 1) issue_tile(X, std::integral_constant<int, 1>(), 1);
    if constexpr (kNST >= 4) {
      if (X.nk > 2) issue_tile(X, std::integral_constant<int, 2 % kNST>(), 2);
      if (X.nk > 3) issue_tile(X, std::integral_constant<int, 3 % kNST>(), 3);
    }
    if constexpr (kNST == 5)
      if (X.nk > 4) issue_tile(X, std::integral_constant<int, 4 % kNST>(), 4);
  };
  for (int64_t q = 0;; ++q) {
    const int64_t w = work_index(q);
    if (w >= total) break;
    const Tile T = setup(w);
    const WorkItem it = T.it;
    const int tn = T.tn, KD = T.KD, nk = T.nk;
    const int n0 = tn * BN;
    const u32x4 ra = T.ra, rb = T.rb;
    uint32_t goa[NI], gob[NI];
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      goa[u] = T.goa[u];
      gob[u] = T.gob[u];
    }

    // paired A loads: load t (8 per wave) covers rows 8t .. 8t+7, whole lines
    uint32_t gop[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = (wv * 8 + u) * 8 + (lane >> 3);
      const int kc = (lane & 7) ^ ((row >> 1) & 7);
      gop[u] = uint32_t(row) * arow * 2 + kc * 16;
    }

#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // The k-loop for NB active MFMA row blocks per wave (a tile of at most
    // 64 NB rows): blocks past them are neither read nor multiplied.
    auto pipeline = [&](auto NB_) {
      constexpr int NB = decltype(NB_)::value;
      // Half h of the direct loads of k-tile kt into stage S (= kt % kNST):
      // A and B pieces u in [h*NI/2, (h+1)*NI/2).
      auto issue_part = [&](auto S_, int kt, int h) {
        constexpr int S = decltype(S_)::value;
        unsigned char* As = stage_a<S>();
        unsigned char* Bs = stage_b<S>();
        const uint32_t ka = uint32_t(kt) * BK * 2;
        const uint32_t kb = kRowB ? uint32_t(kt) * BK * 2 : uint32_t(kt) * BK * WC * 2;
  #pragma unroll
        for (int u2 = 0; u2 < NI / 2; ++u2) {
          const int u = h * (NI / 2) + u2;
          load_lds16(ra, As + (wv * NI + u) * 1024, goa[u], ka);
          load_lds16(rb, Bs + (wv * NI + u) * 1024, gob[u], kb);
        }
      };
      // Paired mode: B of k-tile kt into stage S; A pair p (k-tiles 2p, 2p+1).
      auto issue_b = [&](auto S_, int kt) {
        constexpr int S = decltype(S_)::value;
        unsigned char* Bs = stage_b<S>();
        const uint32_t kb = kRowB ? uint32_t(kt) * BK * 2 : uint32_t(kt) * BK * WC * 2;
  #pragma unroll
        for (int u = 0; u < NI; ++u) load_lds16(rb, Bs + (wv * NI + u) * 1024, gob[u], kb);
      };
      auto issue_a_pair = [&](int p) {
        unsigned char* Ap = pair_buf(p);
        const uint32_t ka = uint32_t(p) * 64 * 2;
  #pragma unroll
        for (int u = 0; u < 8; ++u) load_lds16(ra, Ap + (wv * 8 + u) * 1024, gop[u], ka);
      };
      // Half h of those loads (pieces u in [4h, 4h + 4)).
      auto issue_a_pair_half = [&](int p, int h) {
        unsigned char* Ap = pair_buf(p);
        const uint32_t ka = uint32_t(p) * 64 * 2;
  #pragma unroll
        for (int u2 = 0; u2 < 4; ++u2) {
          const int u = 4 * h + u2;
          load_lds16(ra, Ap + (wv * 8 + u) * 1024, gop[u], ka);
        }
      };
      auto read_frags_pair = [&](auto S_, int kt, int s, bf16x8 (&af)[4], bf16x8 (&bfr)[4]) {
        constexpr int S = decltype(S_)::value;
        const unsigned char* Ap = pair_buf(kt >> 1) + rp_off[kt & 1][s];
        const unsigned char* Bs = stage_b<S>();
  #pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i < NB)
            af[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Ap + i * kABlock * 128));
  #pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (NB == 0) {
          } else if (kRowB) {
            bfr[j] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(Bs + rb_off[s] + j * 32 * ROWB));
          } else {
            const unsigned char* p = Bs + tr_off[j] + wn * 256 + s * 16 * 512;
            bfr[j] = join(lds_tr(p), lds_tr(p + 4 * 512));
          }
        }
      };
      // Operand fragments of one 16-deep k substep of stage S.
      auto read_frags = [&](auto S_, int s, bf16x8 (&af)[4], bf16x8 (&bfr)[4]) {
        constexpr int S = decltype(S_)::value;
        const unsigned char* As = stage_a<S>();
        const unsigned char* Bs = stage_b<S>();
  #pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i >= NB) {
          } else {
            af[i] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(As + ra_off[s] + i * kABlock * ROWB));
          }
        }
  #pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (NB == 0) {
          } else if (kRowB) {
            bfr[j] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(Bs + rb_off[s] + j * 32 * ROWB));
          } else {
            const unsigned char* p = Bs + tr_off[j] + wn * 256 + s * 16 * 512;
            bfr[j] = join(lds_tr(p), lds_tr(p + 4 * 512));
          }
        }
      };
      // One row of MFMA blocks (A fragment I against the 4 B fragments);
      // nothing for a row block past this wave's NB active ones.
      auto mfma_row = [&](const bf16x8 (&af)[4], const bf16x8 (&bfr)[4], auto I_) {
        constexpr int I = decltype(I_)::value;
        if constexpr (I < NB) {
  #pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[I][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[I], bfr[j], acc[I][j], 0, 0, 0);
        }
      };
      auto mfma16 = [&](const bf16x8 (&af)[4], const bf16x8 (&bfr)[4]) {
  #pragma unroll
        for (int i = 0; i < NB; ++i)
  #pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      };
      // Interleave the 4*NB MFMAs just issued with the LDS reads of the next
      // fragments: one read between consecutive MFMAs keeps the matrix pipe fed
      // while the reads are in flight.
      auto interleave = [&]() {
        constexpr int NM = 4 * NB;                                    // MFMAs per substep
        constexpr int NR = NB == 0 ? 0 : NB + (kRowB ? 4 : 8);    // LDS reads
        constexpr int X = NM < NR ? NM : NR;
  #pragma unroll
        for (int x = 0; x < X; ++x) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        }
        if constexpr (NM > X) __builtin_amdgcn_sched_group_barrier(0x008, NM - X, 0);
        if constexpr (NR > X) __builtin_amdgcn_sched_group_barrier(0x100, NR - X, 0);
      };
      // Make stage S (k-tile kt) visible to every wave: each wave waits for
      // its own direct loads of the stage, then the barrier.
      // At publish(kt) the loads of k-tiles kt+1 .. kt+kNST-2 may stay in flight.
      auto publish = [&](int kt) {
        const int after = min(kNST - 2, nk - 1 - kt);
        if (kNST >= 5 && after >= 3) wait_vm<6 * NI>();
        else if (kNST >= 4 && after >= 2) wait_vm<4 * NI>();
        else if (kNST >= 3 && after == 1) wait_vm<2 * NI>();
        else wait_vm<0>();
        barrier_lds();
      };
      // k-tile kt in stage S.  On entry f0 holds its substep-0 fragments.
      bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
      auto step = [&](auto S_, int kt) {
        constexpr int S = decltype(S_)::value;
        constexpr int SN = (S + 1) % kNST;
        unsigned char* As = stage_a<S>();
        if ((kt + 1) * BK > KD) {
          // ragged K: row-tile chunks past the row length hold the next row's
          // data -- zero them and re-read this substep's fragments
          unsigned char* Bs = stage_b<S>();
          wait_vm<0>();
          barrier_lds();
          for (int x = tid; x < kTile / 16; x += kGemmThreads) {
            const int row = x / CPR, phys = x % CPR;
            const int kc = phys ^ ((row >> RSH) & (CPR - 1));
            if (kt * BK + kc * 8 >= KD) {
              *reinterpret_cast<u32x4*>(As + x * 16) = u32x4{0, 0, 0, 0};
              if (kRowB) *reinterpret_cast<u32x4*>(Bs + x * 16) = u32x4{0, 0, 0, 0};
            }
          }
          __syncthreads();
          read_frags(S_, 0, fa0, fb0);
        }
        // substeps 0 .. SUB-2: MFMAs on one fragment set while the next
        // substep's fragments are read into the other
        mfma16(fa0, fb0);
        read_frags(S_, 1, fa1, fb1);
        interleave();
        // Second half of the previous stage's refill (k-tile kt + kNST - 1;
        // its first half went out in the previous step's last substep), so a
        // stage's loads are spread over two substeps of MFMAs instead of one.
        // Loads keep their issue order, so publish's in-flight counts hold.
        __builtin_amdgcn_sched_barrier(0);
        if (kt > 0 && kt + kNST - 1 < nk)
          issue_part(std::integral_constant<int, (S + kNST - 1) % kNST>(), kt + kNST - 1, 1);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (SUB == 4) {
          mfma16(fa1, fb1);
          read_frags(S_, 2, fa0, fb0);
          interleave();
          mfma16(fa0, fb0);
          read_frags(S_, 3, fa1, fb1);
          interleave();
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);                    // lgkmcnt(0)
        // Last substep: its fragments are in registers, so its 16 MFMAs cover
        // the hand-over -- publish k-tile kt+1 (all waves are done with stage
        // S past that barrier), read substep 0 of the next stage (stale and
        // unused after the last k-tile) and start refilling stage S with
        // k-tile kt + kNST (the other half follows in the next step's first
        // substep) -- instead of the matrix pipe idling through it.
        mfma_row(fa1, fb1, std::integral_constant<int, 0>());
        __builtin_amdgcn_sched_barrier(0);
        if (kt + 1 < nk) publish(kt + 1);
        __builtin_amdgcn_sched_barrier(0);
        read_frags(std::integral_constant<int, SN>(), 0, fa0, fb0);
        mfma_row(fa1, fb1, std::integral_constant<int, 1>());
        __builtin_amdgcn_sched_barrier(0);
        if (kt + kNST < nk) issue_part(std::integral_constant<int, S>(), kt + kNST, 0);
        __builtin_amdgcn_sched_barrier(0);
        mfma_row(fa1, fb1, std::integral_constant<int, 2>());
        __builtin_amdgcn_sched_barrier(0);
        mfma_row(fa1, fb1, std::integral_constant<int, 3>());
        __builtin_amdgcn_sched_barrier(0);
      };

      // Paired mode.  Issue order (per wave): A0, B0, B1, A1, B2, B3, A2 before
      // the loop, then at step kt: B(kt+4), and for odd kt the pair
      // (kt+1)/2 + 2 (into the buffer of the pair just finished; its second
      // half goes out in the next step's first substep, before that step's
      // publish, so the counts below are unchanged).  Loads
      // complete in order, so at publish(kt+1) everything issued after B(kt+1)
      // may stay in flight: A(8) + B(4) + B(4) + A(8) = 24 loads for even kt,
      // B(4) + B(4) + A(8) = 16 for odd kt -- as long as all of them exist
      // (kt + 4 < nk); near the end everything is waited for.
      auto publish_pair = [&](int kt1) {
        const int kt = kt1 - 1;
        if (kt + 4 < nk) {
          if ((kt & 1) == 0) wait_vm<24>();
          else wait_vm<16>();
        } else {
          wait_vm<0>();
        }
        barrier_lds();
      };
      auto step_pair = [&](auto S_, int kt) {
        constexpr int S = decltype(S_)::value;
        constexpr int SN = (S + 1) % kNST;
        if ((kt + 1) * BK > KD) {
          // ragged K: chunks past the row length hold the next row's data --
          // zero them (both halves of the pair; B too when it is a row tile)
          unsigned char* Ap = pair_buf(kt >> 1);
          unsigned char* Bs = stage_b<S>();
          wait_vm<0>();
          barrier_lds();
          for (int x = tid; x < kPairTile / 16; x += kGemmThreads) {
            const int row = x / 8, phys = x % 8;
            const int kc = phys ^ ((row >> 1) & 7);
            if ((kt >> 1) * 64 + kc * 8 >= KD) *reinterpret_cast<u32x4*>(Ap + x * 16) = u32x4{0, 0, 0, 0};
          }
          if (kRowB) {
            for (int x = tid; x < kTile / 16; x += kGemmThreads) {
              const int row = x / CPR, phys = x % CPR;
              const int kc = phys ^ ((row >> RSH) & (CPR - 1));
              if (kt * BK + kc * 8 >= KD) *reinterpret_cast<u32x4*>(Bs + x * 16) = u32x4{0, 0, 0, 0};
            }
          }
          __syncthreads();
          read_frags_pair(S_, kt, 0, fa0, fb0);
        }
        mfma16(fa0, fb0);
        read_frags_pair(S_, kt, 1, fa1, fb1);
        interleave();
        // Second half of the A pair whose first half the previous (odd) step
        // issued: same issue order, so publish_pair's in-flight counts hold.
        __builtin_amdgcn_sched_barrier(0);
        if (!(kt & 1) && kt > 0 && 2 * (kt / 2 + 2) < nk) issue_a_pair_half(kt / 2 + 2, 1);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);                    // lgkmcnt(0)
        mfma_row(fa1, fb1, std::integral_constant<int, 0>());
        __builtin_amdgcn_sched_barrier(0);
        if (kt + 1 < nk) publish_pair(kt + 1);
        __builtin_amdgcn_sched_barrier(0);
        read_frags_pair(std::integral_constant<int, SN>(), kt + 1, 0, fa0, fb0);
        mfma_row(fa1, fb1, std::integral_constant<int, 1>());
        __builtin_amdgcn_sched_barrier(0);
        if (kt + kNST < nk) issue_b(std::integral_constant<int, S>(), kt + kNST);
        __builtin_amdgcn_sched_barrier(0);
        mfma_row(fa1, fb1, std::integral_constant<int, 2>());
        __builtin_amdgcn_sched_barrier(0);
        if ((kt & 1) && 2 * ((kt + 1) / 2 + 2) < nk) issue_a_pair_half((kt + 1) / 2 + 2, 0);
        __builtin_amdgcn_sched_barrier(0);
        mfma_row(fa1, fb1, std::integral_constant<int, 3>());
        __builtin_amdgcn_sched_barrier(0);
      };

      if (kPair && nk > 0) {                                      // then nk >= 4
        issue_a_pair(0);
        issue_b(std::integral_constant<int, 0>(), 0);
        issue_b(std::integral_constant<int, 1>(), 1);
        if (2 < nk) issue_a_pair(1);
        issue_b(std::integral_constant<int, 2>(), 2);
        issue_b(std::integral_constant<int, 3>(), 3);
        if (4 < nk) issue_a_pair(2);
        // k-tile 0 (A0, B0) has landed once B1, A1, B2, B3, A2 are all that
        // is left in flight
        if (nk >= 8) wait_vm<28>();
        else wait_vm<0>();
        barrier_lds();
        read_frags_pair(std::integral_constant<int, 0>(), 0, 0, fa0, fb0);
        for (int kt = 0; kt < nk; kt += 4) {
          step_pair(std::integral_constant<int, 0>(), kt);
          step_pair(std::integral_constant<int, 1>(), kt + 1);
          step_pair(std::integral_constant<int, 2>(), kt + 2);
          step_pair(std::integral_constant<int, 3>(), kt + 3);
        }
      } else if (nk > 0) {
      // k-tile 0 has landed once the later k-tiles of the first pass (2 NI
      // loads each) are all that is left in flight.
      {
        issue_first(T);
        const int later = min(nk, kNST) - 1;
        if constexpr (kNST >= 5) {
          if (later >= 4) wait_vm<4 * 2 * NI>();
        }
        if (later == 3) wait_vm<3 * 2 * NI>();
        else if (later == 2) wait_vm<2 * 2 * NI>();
        else if (later == 1) wait_vm<2 * NI>();
        else if (later == 0) wait_vm<0>();
      }
      barrier_lds();
      read_frags(std::integral_constant<int, 0>(), 0, fa0, fb0);
      // whole passes over the stages (the early exits never fire: nk is a
      // multiple of kNST)
      for (int kt = 0; kt < nk; kt += kNST) {
        step(std::integral_constant<int, 0>(), kt);
        if (kt + 1 >= nk) break;
        step(std::integral_constant<int, 1>(), kt + 1);
        if constexpr (kNST >= 4) {
          if (kt + 2 >= nk) break;
          step(std::integral_constant<int, 2 % kNST>(), kt + 2);
          if (kt + 3 >= nk) break;
          step(std::integral_constant<int, 3 % kNST>(), kt + 3);
        }
        if constexpr (kNST == 5) {
          if (kt + 4 >= nk) break;
          step(std::integral_constant<int, 4 % kNST>(), kt + 4);
        }
      }
      }
    };
    pipeline(std::integral_constant<int, NBK>());
    wait_vm<0>();
    __syncthreads();

    // Epilogue.  32x32 accumulator layout: lane l holds column l % 32 and
    // rows 8*(v/4) + 4*(l/32) + v%4 of its block for v = 0..15.
    if constexpr (kSwi) {
      // acc[i][2p] = gate and acc[i][2p+1] = up of activation columns
      // a0 + 32p + lane % 32.  Per half (64 rows), act = silu(gate) * up is
      // staged as bf16 in the wave's first area (144-byte rows: the two lane
      // halves, 4 rows apart, land on different banks) and, with h13 given,
      // gate and up in its second area (128-byte rows); then every staged
      // row piece goes out as one 16-byte store: act to act[:, a], gate to
      // h13[:, a], up to h13[:, H' + a].  sigmoid uses the hardware
      // reciprocal (1 ulp), far inside the bf16 rounding of the output.
      // with paired A tiles the stage arrays of A do not exist: the wave's
      // first area is its 16 KB of the pair buffers, as in the forward
      unsigned char* Ca = kPair ? (wv < 2 ? g_pa0 : g_pa1) + (wv & 1) * 16384 : epilogue_area(wv);
      unsigned char* Cg = epilogue_area2(wv);
      const int a0 = tn * (BN / 2) + wn * 64;
      const bool keep = g.h13 != nullptr;
      const int nout = keep ? 3 * 64 * 8 : 64 * 8;
      uint16_t* actb = g.y + int64_t(it.row0) * Hp;
      uint16_t* hb = keep ? g.h13 + int64_t(it.row0) * 2 * Hp : nullptr;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int lo = 4 * (lane >> 5), col2 = (lane & 31) * 2;
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const f32x16 ga = acc[2 * half + i2][2 * p], ua = acc[2 * half + i2][2 * p + 1];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int mm = 32 * i2 + 8 * (v >> 2) + (v & 3) + lo;
              const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-ga[v]));
              *reinterpret_cast<uint16_t*>(Ca + mm * 144 + 64 * p + col2) =
                  (uint16_t)f32_to_bf16(ga[v] * sg * ua[v]);
              if (keep) {
                *reinterpret_cast<uint16_t*>(Cg + mm * 128 + 64 * p + col2) =
                    (uint16_t)f32_to_bf16(ga[v]);
                *reinterpret_cast<uint16_t*>(Cg + 8192 + mm * 128 + 64 * p + col2) =
                    (uint16_t)f32_to_bf16(ua[v]);
              }
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll 4
        for (int c = lane; c < nout; c += kWave) {
          const int which = c >> 9, rr = (c >> 3) & 63, cc = c & 7;
          const int m = half * 128 + ((rr >> 5) << 6) + wm * kAWaveRow + (rr & 31);
          const int n = a0 + cc * 8;
          const unsigned char* src = which == 0 ? Ca + rr * 144 + cc * 16
                                                : Cg + (which - 1) * 8192 + rr * 128 + cc * 16;
          uint16_t* dst = which == 0 ? actb + uint32_t(m) * Hp + n
                                     : hb + uint32_t(m) * 2 * Hp + (which - 1) * Hp + n;
          if (m < it.rows && n < Hp)
            *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      __syncthreads();
    } else {
      // Per wave, two passes of 64 rows x 128 columns staged as bf16 in the
      // wave's own 16 KB stage array (256-byte rows; pairs of rows converted
      // by one hardware instruction), then whole 16-byte row chunks to global
      // memory (rows of NOUT columns).  All LDS reads of a pass are issued
      // before its stores, so the stores do not wait for one read each.
      unsigned char* Cs = kPair ? (wv < 2 ? g_pa0 : g_pa1) + (wv & 1) * 16384 : epilogue_area(wv);
      uint16_t* yb = g.y + int64_t(it.row0) * NOUT;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        unsigned char* cbase = Cs + 4 * (lane >> 5) * 256 + (lane & 31) * 2;
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x16 a = acc[2 * half + i2][j];
#pragma unroll
            for (int v = 0; v < 16; v += 2) {        // rows mm and mm + 1
              const int mm = 32 * i2 + 8 * (v >> 2) + (v & 3);
              const uint32_t p = cvt_pk_bf16(a[v], a[v + 1]);
              *reinterpret_cast<uint16_t*>(cbase + mm * 256 + 64 * j) = (uint16_t)p;
              *reinterpret_cast<uint16_t*>(cbase + (mm + 1) * 256 + 64 * j) = (uint16_t)(p >> 16);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // every LDS read of the pass first, then the stores
        u32x4 piece[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int c = lane + kWave * k, rr = c >> 4, cc = c & 15;
          piece[k] = *reinterpret_cast<const u32x4*>(Cs + rr * 256 + cc * 16);
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int c = lane + kWave * k, rr = c >> 4, cc = c & 15;
          const int m = half * 128 + ((rr >> 5) << 6) + wm * kAWaveRow + (rr & 31);
          const int n = n0 + wn * 128 + cc * 8;
          if (m < it.rows && n < NOUT)
            *reinterpret_cast<u32x4*>(yb + uint32_t(m) * NOUT + n) = piece[k];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// Weight gradient on 384 x 256 tiles (384 rows of G over h, 256 columns over
// h').  Like the other GEMMs, this kernel is bound by how fast one CU pulls
// operand lines through its L1 (a CU keeps about 64 requests in flight), not
// by the matrix pipe, so what counts is operand bytes per multiply-add: a
// 384 x 256 tile needs (384 + 256) / (384 * 256) of them per k, a sixth less
// than a 256 x 256 tile.  Its 384 KB of fp32 accumulators take 8 waves (2 per
// SIMD), each with 3 x 4 MFMA blocks of 32 x 32 (192 accumulator registers,
// which the compiler keeps in ordinary VGPRs: two waves per SIMD leave each
// 256 registers in all) and at most 64 other registers, so the layout is
// chosen to need few per-lane offsets:
//  * wave (wm, wn) = (wave % 4, wave / 4) takes the tile's 32-row blocks
//    wm + 4i (i < 3) and 32-column blocks wn + 2j (j < 4);
//  * a stage holds x^T as three [32 k][128 h] sub-tiles (256-byte rows) and
//    dy as one [32 k][256 h'] tile (512-byte rows), both stored as loaded
//    ("col tiles", k strided) with 16-byte chunk c of row k at c ^ 4 (k % 4),
//    and read with the transposing LDS read (see lds_tr), conflict free;
//  * every x^T load instruction fills 4 rows x 256 bytes of a sub-tile and
//    every dy load 2 rows x 512 bytes (whole 128-byte lines), so a lane's
//    global offset is one of three values plus a wave-uniform part.
// A wave keeps one set of fragments: the other wave on its SIMD runs its
// MFMAs while it waits for the next.  Four 40 KB stages fill the 160 KB of
// LDS.  The next tile's first pass is issued before the current tile's
// stores, as in k_gemm's weight gradient.
// ---------------------------------------------------------------------------
constexpr int WBM = 384;                 // h rows per tile
constexpr int kWThreads = 512;           // 8 waves
constexpr int kWSub = 32 * 128 * 2;      // one x^T sub-tile (8 KB)
constexpr int kWA = 3 * kWSub;           // x^T stage (24 KB)
constexpr int kWB = 32 * BN * 2;         // dy stage (16 KB)
constexpr int kWStage = kWA + kWB;       // one stage: x^T then dy (40 KB)
constexpr int kWNA = kWA / 1024 / 8;     // x^T loads per wave per k-tile (3)
constexpr int kWNB = kWB / 1024 / 8;     // dy loads per wave per k-tile (2)
constexpr int kWL = kWNA + kWNB;         // loads per wave per k-tile (5)
static_assert(kWNA == 3 && kWNB == 2 && 3 * kWL < 63, "weight-gradient tile");
__shared__ __attribute__((aligned(1024))) unsigned char g_wst[4 * kWStage];

__global__ __launch_bounds__(kWThreads, 1) void k_wgrad(GemmArgs g) {
  const int tid = threadIdx.x, lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wv & 3, wn = wv >> 2;
  const int H = g.H, Hp = g.Hp;
  const int ntm = (H + WBM - 1) / WBM, ntn = (Hp + BN - 1) / BN;
  const int per = gridDim.x / 8;
  const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;
  // XCD x owns the tiles of items [nitems[8+x], nitems[9+x]) (contiguous,
  // balanced by predicted time), so a segment's tiles share its x^T and dy
  // panels in that XCD's L2
  const int64_t wbeg = int64_t(g.nitems[8 + xcd]) * ntm * ntn;
  const int64_t wend = int64_t(g.nitems[9 + xcd]) * ntm * ntn;

  // Transposing fragment reads: lane group G4 = lane/16 takes k half G4/2
  // and column half G4%2 of a 32-column block; row k = tr_k (+4, +16 s) has
  // k % 4 = li / 4.  Block 4q + b of a 16-chunk row group sits at chunks
  // (4b + cl) ^ sw.  This wave's x^T blocks wm + 4i all have b = wm (sub-tile
  // i); its dy blocks wn + 2j have b = wn or wn + 2 (row group j / 2).
  const int G4 = lane >> 4, li = lane & 15;
  const int tr_k = 8 * (G4 >> 1) + (li >> 2);
  const int cl = 2 * (G4 & 1) + ((li & 3) >> 1), sw = 4 * (li >> 2);
  int pa = tr_k * 256 + (((4 * wm + cl) ^ sw) << 4) + 8 * (li & 1);
  int pb[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
    pb[e] = tr_k * 512 + (((4 * (2 * e + wn) + cl) ^ sw) << 4) + 8 * (li & 1);
  // Direct loads.  x^T load t (0..23 per stage) fills rows 4 (t % 8) + [0, 4)
  // of sub-tile t / 8: lane l takes row + l / 16 and stored chunk l % 16.
  // dy load t (0..15) fills rows 2t, 2t + 1: lane l takes row 2t + l / 32 and
  // stored chunk l % 32, whose logical chunk depends on t % 2.
  const uint32_t la = uint32_t(lane >> 4) * H * 2 + (((lane & 15) ^ (4 * (lane >> 4))) << 4);
  uint32_t lb[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
    lb[e] = uint32_t(lane >> 5) * Hp * 2 + (((lane & 31) ^ (4 * ((2 * e + (lane >> 5)) & 3))) << 4);

  typedef __attribute__((address_space(4))) const WorkItem const_item;
  const const_item* items = (const const_item*)g.items;
  struct Tile {
    int r, j, tm, tn, nk;
    u32x4 ra, rb;
  };
  auto setup = [&](int64_t w) -> Tile {
    const int64_t item = w / (ntm * ntn);
    const int rest = (int)(w % (ntm * ntn));
    Tile t;
    t.r = items[item].r;
    t.j = items[item].j;
    const int row0 = items[item].row0, rows = items[item].rows;
    t.tm = rest / ntn;
    t.tn = rest % ntn;
    t.nk = (rows + 31) / 32;              // the last k-tile's rows past the segment read zeros
    t.ra = make_rsrc(g.xperm + int64_t(row0) * H, uint32_t(rows) * H * 2);
    t.rb = make_rsrc(g.dy + int64_t(row0) * Hp, uint32_t(rows) * Hp * 2);
    return t;
  };
  // Loads of k-tile kt of tile X into its stage kt % 4 (this wave's pieces).
  auto issue = [&](const Tile& X, int kt) {
    unsigned char* st = g_wst + (kt & 3) * kWStage;
    const uint32_t ka = uint32_t(kt) * 32 * H * 2 + uint32_t(X.tm) * WBM * 2;
    const uint32_t kb = uint32_t(kt) * 32 * Hp * 2 + uint32_t(X.tn) * BN * 2;
#pragma unroll
    for (int u = 0; u < kWNA; ++u) {
      const int t = wv * kWNA + u;
      load_lds16(X.ra, st + t * 1024, la, ka + uint32_t(4 * (t & 7)) * H * 2 + (t >> 3) * 256);
    }
#pragma unroll
    for (int u = 0; u < kWNB; ++u) {
      const int t = wv * kWNB + u;
      load_lds16(X.rb, st + kWA + t * 1024, lb[u], kb + uint32_t(2 * t) * Hp * 2);
    }
  };
  // the first min(nk, 4) k-tiles of X, one per stage
  auto issue_first = [&](const Tile& X) {
    for (int kt = 0; kt < min(X.nk, 4); ++kt) issue(X, kt);
  };

  f32x16 acc[3][4];
  bf16x8 fa[3], fb[4];
  Tile nxt;
  bool have_nxt = false;
  for (int64_t w = wbeg + local; w < wend; w += per) {
    const bool carried = have_nxt;
    const Tile T = carried ? nxt : setup(w);
    const int nk = T.nk;
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // fragments of 16-deep substep s of the stage at st (its x^T sub-tile i,
    // its dy row group j / 2); qa, qb: this lane's offsets into the stage
    auto read_a = [&](int qa, int s, int i) {
      const unsigned char* p = g_wst + qa + s * 16 * 256 + i * kWSub;
      fa[i] = join(lds_tr(p), lds_tr(p + 4 * 256));
    };
    auto read_b = [&](const int (&qb)[2], int s, int j) {
      const unsigned char* p = g_wst + qb[j & 1] + kWA + s * 16 * 512 + (j >> 1) * 256;
      fb[j] = join(lds_tr(p), lds_tr(p + 4 * 512));
    };
    auto mfma_row = [&](int i) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    };

    if (nk > 0) {
      // k-tile 0 has landed once the later k-tiles of the first pass are
      // all that is left in flight.  A carried tile's first pass went out
      // before the previous tile's stores: a full tile's 192 store
      // instructions per wave follow it (more than the 63 a wave keeps in
      // flight, and completions count in issue order), and after a partial
      // tile's stores the wave waited for everything -- so at most 62
      // pending operations leave the whole first pass landed.
      if (carried) {
        wait_vm<62>();
      } else {
        issue_first(T);
        const int later = min(nk, 4) - 1;
        if (later == 3) wait_vm<3 * kWL>();
        else if (later == 2) wait_vm<2 * kWL>();
        else if (later == 1) wait_vm<kWL>();
        else wait_vm<0>();
      }
      barrier_lds();
      {
        int qb[2] = {pb[0], pb[1]};
#pragma unroll
        for (int j = 0; j < 4; ++j) read_b(qb, 0, j);
#pragma unroll
        for (int i = 0; i < 3; ++i) read_a(pa, 0, i);
      }
      for (int kt = 0; kt < nk; ++kt) {
        // this lane's offsets into the stage of k-tile kt and of kt + 1,
        // computed here (a few idle VALU cycles) rather than kept per stage
        const int so = (kt & 3) * kWStage, sn = ((kt + 1) & 3) * kWStage;
        const int qa = pa + so, qan = pa + sn;
        const int qb[2] = {pb[0] + so, pb[1] + so}, qbn[2] = {pb[0] + sn, pb[1] + sn};
        // substep 0; each fragment of substep 1 is read as soon as its last
        // use here has issued.  The wave runs this part at raised priority, so
        // of a SIMD's two waves the one in substep 0 issues first and the
        // pair settles into alternating phases (one multiplying while the
        // other waits on its loads or the barrier)
        __builtin_amdgcn_s_setprio(1);
        mfma_row(0);
        read_a(qa, 1, 0);
        mfma_row(1);
        read_a(qa, 1, 1);
        mfma_row(2);
#pragma unroll
        for (int j = 0; j < 4; ++j) read_b(qb, 1, j);
        read_a(qa, 1, 2);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        // k-tile kt+3 into the stage k-tile kt-1 has left (every wave passed
        // the barrier of the previous iteration after its reads of it)
        if (kt > 0 && kt + 3 < nk) issue(T, kt + 3);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);                    // lgkmcnt(0)
        // substep 1
        mfma_row(0);
        mfma_row(1);
        mfma_row(2);
        __builtin_amdgcn_sched_barrier(0);
        if (kt + 1 < nk) {
          // publish k-tile kt+1: k-tiles kt+2 and kt+3 may stay in flight
          // (loads complete in issue order); a carried tile's first pass has
          // landed already
          const int after = min(2, nk - 2 - kt);
          if (carried && kt + 1 < 4) {
          } else if (after >= 2) wait_vm<2 * kWL>();
          else if (after == 1) wait_vm<kWL>();
          else wait_vm<0>();
          barrier_lds();
#pragma unroll
          for (int j = 0; j < 4; ++j) read_b(qbn, 0, j);
#pragma unroll
          for (int i = 0; i < 3; ++i) read_a(qan, 0, i);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    wait_vm<0>();
    __syncthreads();
    // every wave is done with the stage arrays: the next tile's first pass
    have_nxt = w + per < wend;
    if (have_nxt) {
      nxt = setup(w + per);
      if (nxt.nk > 0) issue_first(nxt);
    }

    // fp32 gradient rows straight from the accumulators: each store writes
    // two whole 128-byte row pieces (lanes 0-31 and 32-63, four rows apart),
    // through a buffer resource over this tile's rows (the entry point keeps
    // them under 2 GiB), non-temporal (written once).  Row block wm + 4i,
    // column block wn + 2j.
    const int m0 = T.tm * WBM, n0 = T.tn * BN;
    float* out = T.j < g.E ? g.grad_home + int64_t(T.j) * H * Hp
                           : g.grad_pref + (int64_t(T.r) * g.B + (T.j - g.E)) * H * Hp;
    const int trows = min(WBM, H - m0);
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        out + int64_t(m0) * Hp, 0, int(uint32_t(trows) * Hp * 4), 0x00020000);
    int hb0 = wm * 32 + 4 * (lane >> 5);
    const int nb0 = n0 + wn * 32 + (lane & 31);
    asm volatile("" : "+v"(hb0));     // store offsets: computed here, not hoisted
    auto store_tile = [&](auto full_) {
      constexpr bool FULL = decltype(full_)::value;
#pragma unroll
      for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = nb0 + 64 * j;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int h = hb0 + 128 * i + 8 * (v >> 2) + (v & 3);
            if (FULL || (h < trows && n < Hp))
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][v]), orsrc,
                                                    int((uint32_t(h) * Hp + n) * 4), 0, kStoreNT);
          }
        }
    };
    if (m0 + WBM <= H && n0 + BN <= Hp) {
      store_tile(std::true_type());
    } else {
      store_tile(std::false_type());
      if (have_nxt) wait_vm<0>();      // see the carried wait above
    }
  }
}

// ---------------------------------------------------------------------------
// Work lists.  Forward: one item per 256-row m-tile of every non-empty
// segment of ranks [rb, re), in (rank, weight row, m) order.  Weight
// gradient: one item per segment that owns a gradient row -- every home row
// of the rank (empty ones write zeros) and every non-empty prefetch row.
//
// Forward-type lists (forward, data gradient, SwiGLU first projection) are
// split by tile height and the split is chosen per step by a cost model
// ("Kimi K3 模型结构（8）", rank 内部: expert token counts stay skewed inside a
// rank, so the GEMM schedule is picked from this step's counts before launch
// by a time estimate whose key coefficients are tuned offline; "MoonEP :
// l'équilibrage parfait", 3. Ordonnancement des GEMM d'experts).  On the
// device, from cu_seqlens and with no host round trip:
//  * a segment's full row tiles, and a last row tile of more than 128 rows,
//    go to class 4 (any tile); a last row tile of 65..128 rows to class 2,
//    of 1..64 rows to class 1 (the data gradient keeps the last tile of a
//    segment that has full tiles in class 4, beside the tiles it shares a
//    weight panel with).  Class c runs as its own persistent launch whose
//    tiles multiply only 2c of their 8 MFMA row blocks;
//  * a launch over n tiles of class c takes about L + ceil(n / G) t_c on G
//    workgroups, with t_c = c0 + nk (c1 + c2 c) per tile (nk = k-tiles);
//  * class 2 is folded into the class-4 list when the rounds it adds there
//    cost no more than its own launch, and class 1 likewise into the list
//    of the next larger class that still runs.
// A folded tail keeps its place right after its segment's other tiles, so
// each segment's items stay adjacent in every list.
// ---------------------------------------------------------------------------
struct SchedArgs {
  const int32_t* cu;
  WorkItem* items;        // class-4 list (weight gradient: its only list)
  WorkItem* items2;       // class-2 list
  WorkItem* items1;       // class-1 list
  int32_t* hdr;           // [0..2] items of the class 4, 2, 1 lists, [3] folds
                          // (bit 0: class 2 into 4, bit 1: class 1 folded, bit 2:
                          // into class 4), [4] predicted time in ns
  int32_t rb, re, E, B, n, SK, cap, cap_s;
  int32_t G, ntn, nk;     // persistent workgroups, column tiles, k-tiles per tile
  int32_t c0, c1, c2, cL; // cost model, picoseconds (see above; cL = per launch)
  int32_t small;          // 1 if the class-2 and class-1 launches run at all
  int32_t keep_multi;     // 1: the last tile of a multi-tile segment stays in class 4
};

template <int MODE>
__global__ __launch_bounds__(1024) void k_sched(SchedArgs s) {
  __shared__ int s_part[32];
  __shared__ int s_carry[3];
  __shared__ int s_fold;
  // weight gradient: predicted time of each item (k-tiles plus a fixed
  // part) and its exclusive prefix, for the XCD ranges
  constexpr int kMaxWItems = MODE == MODE_FWD ? 1 : 4096;
  __shared__ int s_wpre[kMaxWItems], s_wcost[kMaxWItems];
  __shared__ int s_wcarry, s_xcnt[8];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int rows = s.E + s.B;
  const int64_t total = int64_t(s.re - s.rb) * rows;
  if (tid < 3) s_carry[tid] = 0;
  if (tid < 8) s_xcnt[tid] = 0;
  if (tid == 0) { s_fold = 0; s_wcarry = 0; }
  __syncthreads();
  // Block-wide exclusive scan of one value per thread: returns the prefix
  // and leaves the chunk total in s_part[16].
  auto block_scan = [&](int v) {
    const int incl = wave_incl_scan(v);
    if (lane == kWave - 1) s_part[wave] = incl;
    __syncthreads();
    if (wave == 0) {
      const int x = lane < 16 ? s_part[lane] : 0;
      const int xi = wave_incl_scan(x);
      if (lane < 16) s_part[lane] = xi - x;
      if (lane == 15) s_part[16] = xi;
    }
    __syncthreads();
    const int pre = s_part[wave] + incl - v;
    return pre;
  };
  // The segment of chunk entry idx: rank, weight row, first row, rows, its
  // class-4 row tiles and the class (0, 1 or 2) of a separate last tile.
  auto segment = [&](int64_t idx, int& r, int& j, int& lo, int& len, int& c4, int& tc) {
    c4 = 0; tc = 0; r = 0; j = 0; lo = 0; len = 0;
    if (idx < total) {
      r = s.rb + (int)(idx / rows);
      j = (int)(idx % rows);
      const int32_t* cu = s.cu + int64_t(r) * (rows + 1);
      lo = cu[j];
      len = cu[j + 1] - lo;
      if (MODE == MODE_FWD) {
        const int cnt = (len + BM - 1) / BM;
        const int tail = len - (cnt - 1) * BM;         // rows of the last row tile
        tc = cnt == 0 || (s.keep_multi && cnt > 1) ? 0 : tail <= 64 ? 1 : tail <= 128 ? 2 : 0;
        c4 = cnt - (tc ? 1 : 0);
      } else {
        const bool home = j < s.E && j / s.n == r;
        c4 = (home || (j >= s.E && len > 0)) ? 1 : 0;
      }
    }
  };
  auto write_items = [&](WorkItem* list, int cap, int base, int r, int j, int lo, int len,
                         int m0, int cnt) {
    for (int m = 0; m < cnt; ++m) {
      const int at = base + m;
      if (at < cap) {
        WorkItem w;
        w.r = r;
        w.j = j;
        if (MODE == MODE_FWD) {
          w.row0 = r * s.SK + lo + (m0 + m) * BM;
          w.rows = min(BM, len - (m0 + m) * BM);
        } else {
          w.row0 = r * s.SK + lo;
          w.rows = len;
        }
        w.first = base;
        w.cnt = cnt;
        list[at] = w;
      }
    }
  };
  if (MODE == MODE_FWD) {
    // Pass 1: row tiles of each class.
    for (int64_t c0 = 0; c0 < total; c0 += 1024) {
      int r, j, lo, len, c4, tc;
      segment(c0 + tid, r, j, lo, len, c4, tc);
      const int v4 = wave_sum(c4), v2 = wave_sum(tc == 2), v1 = wave_sum(tc == 1);
      if (lane == 0) {
        atomicAdd(&s_carry[0], v4);
        atomicAdd(&s_carry[1], v2);
        atomicAdd(&s_carry[2], v1);
      }
    }
    __syncthreads();
    if (tid == 0) {
      // the cost model's choice of folds (tile counts = row tiles x ntn)
      const int64_t G = s.G, n4 = int64_t(s_carry[0]) * s.ntn;
      const int64_t n2 = int64_t(s_carry[1]) * s.ntn, n1 = int64_t(s_carry[2]) * s.ntn;
      auto rounds = [&](int64_t x) { return (x + G - 1) / G; };
      auto tile = [&](int c) { return int64_t(s.c0) + int64_t(s.nk) * (s.c1 + int64_t(s.c2) * c); };
      auto own = [&](int64_t x, int c) { return x > 0 ? s.cL + rounds(x) * tile(c) : int64_t(0); };
      const int64_t t4 = tile(4), t2 = tile(2);
      const bool f2 = n2 > 0 && (!s.small || (rounds(n4 + n2) - rounds(n4)) * t4 <= own(n2, 2));
      const int64_t m4 = n4 + (f2 ? n2 : 0), m2 = f2 ? 0 : n2;
      bool f1 = false, to4 = false;
      if (n1 > 0) {
        // fold into the smallest class that still runs, if that is cheaper
        if (!s.small) { f1 = true; to4 = true; }
        else if (m2 > 0) f1 = (rounds(m2 + n1) - rounds(m2)) * t2 <= own(n1, 1);
        else { f1 = (rounds(m4 + n1) - rounds(m4)) * t4 <= own(n1, 1); to4 = f1; }
      }
      const int64_t e4 = m4 + (to4 ? n1 : 0), e2 = m2 + (f1 && !to4 ? n1 : 0), e1 = f1 ? 0 : n1;
      const int64_t pred = own(e4, 4) + own(e2, 2) + own(e1, 1);
      s_fold = (f2 ? 1 : 0) | (f1 ? 2 : 0) | (to4 ? 4 : 0);
      s.hdr[4] = (int32_t)min<int64_t>(pred / 1000, 0x7fffffff);
      s_carry[0] = s_carry[1] = s_carry[2] = 0;
    }
    __syncthreads();
  }
  const int fold = s_fold;
  // Pass 2 (the only pass of the weight gradient): the lists, in layout
  // order; a folded last tile follows its segment's tiles in its new list.
  for (int64_t c0 = 0; c0 < total; c0 += 1024) {
    int r, j, lo, len, c4, tc;
    segment(c0 + tid, r, j, lo, len, c4, tc);
    // destination list of the last tile: 4, 2 or 1 (0: none)
    int dst = tc;
    if (tc == 2 && (fold & 1)) dst = 4;
    if (tc == 1 && (fold & 2)) dst = (fold & 4) ? 4 : 2;
    const int a4 = c4 + (dst == 4 ? 1 : 0), a2 = dst == 2 ? 1 : 0, a1 = dst == 1 ? 1 : 0;
    const int p4 = block_scan(a4);
    const int t4 = s_part[16];
    __syncthreads();
    const int p2 = block_scan(a2);
    const int t2 = s_part[16];
    __syncthreads();
    const int p1 = block_scan(a1);
    const int t1 = s_part[16];
    const int b4 = s_carry[0] + p4, b2 = s_carry[1] + p2, b1 = s_carry[2] + p1;
    if (MODE == MODE_WGRAD) {
      // an item's time: its k-tiles (rounded to whole passes of the stage
      // ring) plus about 12 k-tiles' worth of prologue and fp32 stores
      const int cost = a4 ? ((len + kBK - 1) / kBK + kNST - 1) / kNST * kNST + 12 : 0;
      __syncthreads();
      const int pc = block_scan(cost);
      const int tsum = s_part[16];
      if (a4 && b4 < kMaxWItems) { s_wpre[b4] = s_wcarry + pc; s_wcost[b4] = cost; }
      __syncthreads();
      if (tid == 0) s_wcarry += tsum;
    }
    write_items(s.items, s.cap, b4, r, j, lo, len, 0, a4);
    if (a2) write_items(s.items2, s.cap_s, b2, r, j, lo, len, c4, 1);
    if (a1) write_items(s.items1, s.cap_s, b1, r, j, lo, len, c4, 1);
    __syncthreads();
    if (tid == 0) { s_carry[0] += t4; s_carry[1] += t2; s_carry[2] += t1; }
    __syncthreads();
  }
  if (tid == 0) {
    s.hdr[0] = min(s_carry[0], s.cap);
    s.hdr[1] = MODE == MODE_FWD ? min(s_carry[1], s.cap_s) : 0;
    s.hdr[2] = MODE == MODE_FWD ? min(s_carry[2], s.cap_s) : 0;
    s.hdr[3] = fold;
    if (MODE != MODE_FWD) s.hdr[4] = 0;
  }
  if (MODE == MODE_WGRAD) {
    // XCD x takes the items whose time midpoint falls in [x/8, (x+1)/8) of
    // the total: contiguous, balanced ranges [hdr[8+x], hdr[9+x])
    __syncthreads();
    const int n = min(s_carry[0], s.cap);
    const int64_t tot = s_wcarry;
    if (n <= kMaxWItems && tot > 0) {
      for (int i = tid; i < n; i += 1024) {
        const int x = (int)min<int64_t>(7, (8 * (2 * int64_t(s_wpre[i]) + s_wcost[i])) / (2 * tot));
        atomicAdd(&s_xcnt[x], 1);
      }
      __syncthreads();
      if (tid == 0) {
        int acc = 0;
        for (int x = 0; x < 8; ++x) { s.hdr[8 + x] = acc; acc += s_xcnt[x]; }
        s.hdr[16] = acc;
      }
    } else if (tid == 0) {
      // no ranges: XCD 0 takes every item (cannot happen within the limits)
      s.hdr[8] = 0;
      for (int x = 1; x < 9; ++x) s.hdr[8 + x] = n;
    }
  }
}

// Compute units of the current device: the persistent grid's size.  The
// attribute query is cheap and asked on every launch, so nothing is cached
// across calls (or devices).
static int num_cus() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    v = 256;
  return v;
}

static int64_t fwd_capacity(const moe_cfg* c, int nranks) {
  return int64_t(nranks) * ((int64_t(c->S) * c->K + BM - 1) / BM + c->E + c->B);
}

static int64_t wgrad_capacity(const moe_cfg* c) { return int64_t(c->E) + int64_t(c->R) * c->B; }

// Forward-type lists: at most one last tile per segment goes to a small class.
static int64_t small_capacity(const moe_cfg* c, int nranks) {
  return int64_t(nranks) * (c->E + c->B);
}

// Workspace: a 256-byte header, then the work list (forward-type lists: the
// class-4, class-2 and class-1 lists).
static size_t fwd_ws_bytes(const moe_cfg* c, int nranks) {
  return 256 + size_t(fwd_capacity(c, nranks) + 2 * small_capacity(c, nranks)) * sizeof(WorkItem);
}

static size_t gemm_ws_bytes(const moe_cfg* c) {
  return std::max(fwd_ws_bytes(c, c->R), 256 + size_t(wgrad_capacity(c)) * sizeof(WorkItem));
}

// Cost model of the forward-type schedules, picoseconds: a 256x256 tile of
// class c (2c of 8 MFMA row blocks) over nk 32-deep k-tiles takes
// tile + nk (k + k_block c); a persistent launch adds `launch`.  Fitted by
// moe_expert_load_amd/calibrate.py to forward and data-gradient GEMM times
// on one MI355X (the SwiGLU projection uses the forward's).
struct CostModel { int32_t tile, k, k_block, launch; };
constexpr CostModel kCostFwd = {7118903, 522523, 125859, 0};
constexpr CostModel kCostDgrad = {5988999, 682007, 87206, 47041760};

// Average rows per home segment, S*K*R/E, below which a step's tails are a
// large enough share of its tiles for the class-2 and class-1 launches to
// pay for themselves (measured: decode-size steps gain, steps of about two
// row tiles per segment lose their launch cost).  The gate depends on the
// configuration only, so the launch sequence stays static.
constexpr int64_t kSmallClassRows = 512;

static SchedArgs sched_args(const moe_cfg* c, const int32_t* cu, void* workspace, int rb, int re,
                            int64_t cap, int64_t cap_s) {
  SchedArgs s{};
  s.cu = cu;
  s.hdr = reinterpret_cast<int32_t*>(workspace);
  s.items = reinterpret_cast<WorkItem*>(reinterpret_cast<char*>(workspace) + 256);
  s.items2 = s.items + cap;
  s.items1 = s.items2 + cap_s;
  s.rb = rb; s.re = re; s.E = c->E; s.B = c->B; s.n = c->E / c->R;
  s.SK = c->S * c->K;
  s.cap = (int32_t)cap;
  s.cap_s = (int32_t)cap_s;
  return s;
}

static SchedArgs fwd_sched_args(const moe_cfg* c, const int32_t* cu, void* workspace, int rb,
                                int re) {
  return sched_args(c, cu, workspace, rb, re, fwd_capacity(c, re - rb), small_capacity(c, re - rb));
}

template <int MODE>
static void launch_classes(GemmArgs& g, const SchedArgs& s, int G, hipStream_t stream) {
  g.items = s.items;
  g.nitems = s.hdr;
  hipLaunchKernelGGL((k_gemm<MODE, 4>), dim3(G), dim3(kGemmThreads), 0, stream, g);
  if (!s.small) return;                  // every tile folded into class 4
  g.items = s.items2;
  g.nitems = s.hdr + 1;
  hipLaunchKernelGGL((k_gemm<MODE, 2>), dim3(G), dim3(kGemmThreads), 0, stream, g);
  g.items = s.items1;
  g.nitems = s.hdr + 2;
  hipLaunchKernelGGL((k_gemm<MODE, 1>), dim3(G), dim3(kGemmThreads), 0, stream, g);
}

// The data gradient runs over the forward's work lists (the same row tiles).
static int launch_gemm(int mode, const moe_cfg* c, GemmArgs& g, SchedArgs& s, hipStream_t stream) {
  int G = num_cus();
  G = std::max(8, G - G % 8);
  if (mode == MODE_WGRAD) {
    hipLaunchKernelGGL(k_sched<MODE_WGRAD>, dim3(1), dim3(1024), 0, stream, s);
    g.items = s.items;
    g.nitems = s.hdr;
    hipLaunchKernelGGL(k_wgrad, dim3(G), dim3(kWThreads), 0, stream, g);
    return hip_status();
  }
  const int kdepth = mode == MODE_DGRAD ? c->Hp : c->H;
  s.G = G;
  s.ntn = mode == MODE_SWIGLU ? (c->Hp + BN / 2 - 1) / (BN / 2)
                              : ((mode == MODE_DGRAD ? c->H : c->Hp) + BN - 1) / BN;
  s.nk = ((kdepth + kBK - 1) / kBK + kNST - 1) / kNST * kNST;
  const CostModel& m = mode == MODE_DGRAD ? kCostDgrad : kCostFwd;
  s.c0 = m.tile; s.c1 = m.k; s.c2 = m.k_block; s.cL = m.launch;
  s.small = int64_t(c->S) * c->K * c->R < kSmallClassRows * c->E ? 1 : 0;
  // the data gradient's last tile shares its weight panel with the segment's
  // full tiles in one band: moving it to another launch reads the panel again,
  // which costs it more than the halved matrix work saves (measured)
  s.keep_multi = mode == MODE_DGRAD ? 1 : 0;
  hipLaunchKernelGGL(k_sched<MODE_FWD>, dim3(1), dim3(1024), 0, stream, s);
  if (mode == MODE_FWD) launch_classes<MODE_FWD>(g, s, G, stream);
  else if (mode == MODE_SWIGLU) launch_classes<MODE_SWIGLU>(g, s, G, stream);
  else launch_classes<MODE_DGRAD>(g, s, G, stream);
  return hip_status();
}

// The forward grouped GEMM with its work list in `workspace` (checked).
static int grouped_gemm_fwd(const moe_cfg* cfg, const moe_bf16* xperm, const moe_bf16* w_home,
                            const moe_bf16* w_pref, const int32_t* cu_seqlens, moe_bf16* y,
                            int32_t rank_begin, int32_t rank_end, void* workspace,
                            hipStream_t stream) {
  GemmArgs g{};
  g.xperm = xperm; g.w_home = w_home; g.w_pref = w_pref; g.y = y;
  g.H = cfg->H; g.Hp = cfg->Hp; g.E = cfg->E; g.B = cfg->B; g.SK = cfg->S * cfg->K;
  SchedArgs s = fwd_sched_args(cfg, cu_seqlens, workspace, rank_begin, rank_end);
  return launch_gemm(MODE_FWD, cfg, g, s, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free forward GEMM.  Its work list (the only scratch the GEMM
// uses) lives in `scratch`, a file-scope device array of fixed size; each
// device holds its own copy until the process ends.  In host code the name
// `scratch` is only a stand-in for the symbol: its device address on each
// device comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address is passed to kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call on each device).
static int scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ELIMIT;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
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
  if (!aligned16(xperm, w_home, w_pref, y, workspace)) return MOE_EINVAL;
  return grouped_gemm_fwd(cfg, xperm, w_home, w_pref, cu_seqlens, y, rank_begin, rank_end,
                          workspace, stream);
}

extern "C" int moe_grouped_gemm_noalloc(const moe_cfg* cfg, const moe_bf16* xperm,
                                        const moe_bf16* w_home, const moe_bf16* w_pref,
                                        const int32_t* cu_seqlens, moe_bf16* y,
                                        int32_t rank_begin, int32_t rank_end,
                                        hipStream_t stream) {
  const int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if (rank_begin < 0 || rank_end > cfg->R || rank_begin > rank_end) return MOE_EINVAL;
  // the work list of the listed ranks must fit the fixed scratch array
  if (fwd_ws_bytes(cfg, rank_end - rank_begin) > size_t(MOE_NOALLOC_SCRATCH_BYTES))
    return MOE_ELIMIT;
  if (rank_begin == rank_end || cfg->S == 0) return MOE_OK;
  if (!xperm || !w_home || !cu_seqlens || !y) return MOE_EINVAL;
  if (cfg->B > 0 && !w_pref) return MOE_EINVAL;
  if (!aligned16(xperm, w_home, w_pref, y)) return MOE_EINVAL;
  void* ws = nullptr;
  const int sp = scratch_ptr(&ws);
  if (sp != MOE_OK) return sp;
  return grouped_gemm_fwd(cfg, xperm, w_home, w_pref, cu_seqlens, y, rank_begin, rank_end, ws,
                          stream);
}

extern "C" int moe_grouped_gemm_swiglu(const moe_cfg* cfg, const moe_bf16* xperm,
                                       const moe_bf16* w13_home, const moe_bf16* w13_pref,
                                       const int32_t* cu_seqlens, moe_bf16* act, moe_bf16* h13,
                                       int32_t rank_begin, int32_t rank_end, void* workspace,
                                       hipStream_t stream) {
  const int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if (rank_begin < 0 || rank_end > cfg->R || rank_begin > rank_end) return MOE_EINVAL;
  // one [H][2H'] weight must fit the 32-bit buffer offsets
  if (int64_t(cfg->H) * cfg->Hp * 4 >= (int64_t(1) << 32)) return MOE_ELIMIT;
  if (rank_begin == rank_end || cfg->S == 0) return MOE_OK;
  if (!xperm || !w13_home || !cu_seqlens || !act || !workspace) return MOE_EINVAL;
  if (cfg->B > 0 && !w13_pref) return MOE_EINVAL;
  if (!aligned16(xperm, w13_home, w13_pref, act, h13, workspace)) return MOE_EINVAL;
  GemmArgs g{};
  g.xperm = xperm; g.w_home = w13_home; g.w_pref = w13_pref; g.y = act; g.h13 = h13;
  g.H = cfg->H; g.Hp = cfg->Hp; g.E = cfg->E; g.B = cfg->B; g.SK = cfg->S * cfg->K;
  SchedArgs s = fwd_sched_args(cfg, cu_seqlens, workspace, rank_begin, rank_end);
  return launch_gemm(MODE_SWIGLU, cfg, g, s, stream);
}

extern "C" int moe_grouped_gemm_dgrad(const moe_cfg* cfg, const moe_bf16* dy, const moe_bf16* w_home,
                                      const moe_bf16* w_pref, const int32_t* cu_seqlens,
                                      moe_bf16* dxperm, int32_t rank_begin, int32_t rank_end,
                                      void* workspace, hipStream_t stream) {
  const int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if (rank_begin < 0 || rank_end > cfg->R || rank_begin > rank_end) return MOE_EINVAL;
  if (rank_begin == rank_end || cfg->S == 0) return MOE_OK;
  if (!dy || !w_home || !cu_seqlens || !dxperm || !workspace) return MOE_EINVAL;
  if (cfg->B > 0 && !w_pref) return MOE_EINVAL;
  if (!aligned16(dy, w_home, w_pref, dxperm, workspace)) return MOE_EINVAL;
  GemmArgs g{};
  g.dy = dy; g.w_home = w_home; g.w_pref = w_pref; g.y = dxperm;
  g.H = cfg->H; g.Hp = cfg->Hp; g.E = cfg->E; g.B = cfg->B; g.SK = cfg->S * cfg->K;
  SchedArgs s = fwd_sched_args(cfg, cu_seqlens, workspace, rank_begin, rank_end);
  return launch_gemm(MODE_DGRAD, cfg, g, s, stream);
}

extern "C" int moe_grouped_gemm_wgrad(const moe_cfg* cfg, const moe_plan* plan,
                                      const moe_bf16* xperm, const moe_bf16* dy, float* grad_home,
                                      float* grad_pref, void* workspace, hipStream_t stream) {
  const int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if (cfg->mode != MOE_MODE_TRAIN) return MOE_EINVAL;
  // a 384-row fp32 gradient tile is stored through one 2 GiB buffer window
  if (uint64_t(WBM) * cfg->Hp * 4 >= (uint64_t(1) << 31)) return MOE_ELIMIT;
  if (!plan || !plan->cu_seqlens || !xperm || !dy || !grad_home || !workspace) return MOE_EINVAL;
  if (cfg->B > 0 && !grad_pref) return MOE_EINVAL;
  if (!aligned16(xperm, dy, grad_home, grad_pref, workspace)) return MOE_EINVAL;
  GemmArgs g{};
  g.xperm = xperm; g.dy = dy; g.grad_home = grad_home; g.grad_pref = grad_pref;
  g.H = cfg->H; g.Hp = cfg->Hp; g.E = cfg->E; g.B = cfg->B; g.SK = cfg->S * cfg->K;
  SchedArgs s = sched_args(cfg, plan->cu_seqlens, workspace, 0, cfg->R, wgrad_capacity(cfg), 0);
  return launch_gemm(MODE_WGRAD, cfg, g, s, stream);
}
