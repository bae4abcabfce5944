// Dense projections: C = A . W^T (+ R).  FT 3.1 (Q, K, V = LinearProjection(X))
// and the C x C output projection that returns the module to C channels
// (FT 3.5 block equation); the FFN projections of the block use the same
// kernels.
//
// A is [M][K] row-major (tokens x input channels), W is [N][K] row-major
// (output x input channels, the nn.Linear layout), so both MFMA operands read
// eight consecutive k values per lane straight from a row.
//
// bfloat16: 256x128 output tile per 256-thread workgroup (2x2 waves of
// 128x64, each a 4x2 grid of 32x32x16 MFMAs: the tall wave tile reads fewer
// LDS bytes per MFMA than a square 64x64 one), K staged through LDS in
// steps of 32 with two steps in flight -- copied straight into three LDS
// buffers (global_load_lds) when the K loop is unrolled, else through
// registers into two -- and workgroups mapped so that each XCD walks whole
// row panels of A (its L2 then serves the A panel to every column tile).
// float32: a plain LDS-tiled FMA kernel (small shapes only).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace hsmla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// bfloat16 MFMA kernel
//
// Workgroup tile BM x BN, WGM x WGN waves each owning (BM/WGM) x (BN/WGN) =
// FM x FN fragments of 32 x 32 (v_mfma_f32_32x32x16_bf16).  A and W tiles of
// BK k go through double-buffered LDS (16-byte loads staged in registers,
// PF steps ahead; rows padded by 16 bytes).  With NKT > 0 the K loop is
// unrolled completely (K = NKT * BK), which keeps the compiler's wait counts
// exact across iterations so the PF = 2 prefetch really stays in flight.
// The MFMA computes the transposed tile so each lane ends up with runs of 4
// consecutive output columns; the finished tile is staged in LDS as float32
// and written back row by row with 16-byte stores.  Tiles are remapped so
// each XCD walks whole row panels of A.
// ---------------------------------------------------------------------------

constexpr int kXcds = 8;
// With the unrolled K loop, each K step is copied straight into LDS (see
// the kernel); the register-staged pipeline serves the other shapes.
constexpr bool kDirectLds = true;

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8; a field at its maximum does not wait)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);

__device__ __forceinline__ uint4 ld16(const bf16* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// A pointer every lane holds the same value of, made visibly wave-uniform
// (scalar registers): the direct-to-LDS copies take a scalar base address.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// SITE only names the call site (one kernel symbol per projection, so
// profiles tell the four GEMMs apart); the code is the same.
template <int BM, int BN, int BK, int WGM, int WGN, int SITE, int PF, bool EDGE, int NKT,
          int BLK>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_mfma_bf16(
    const bf16* __restrict__ A, const bf16* __restrict__ W,
    const bf16* __restrict__ R, bf16* __restrict__ C, int M, int N, int K,
    int tiles_n, int tiles_total, int per_xcd) {
  constexpr int NT = 64 * WGM * WGN;         // threads
  constexpr int STR = BK + 8;                // bf16 per LDS row
  constexpr int FM = BM / WGM / 32, FN = BN / WGN / 32;
  constexpr int CPR = BK / 8;                // 16-byte chunks per row
  constexpr int LA = BM * CPR / NT;          // A chunks per thread
  constexpr int LW = BN * CPR / NT;          // W chunks per thread
  static_assert(BM * CPR % NT == 0 && BN * CPR % NT == 0, "tile/threads");
  constexpr int TN = BN / WGN;                 // wave tile width
  constexpr int CSTR = TN + 4;                 // floats per staged row
  constexpr int kTileBytes = 2 * (BM + BN) * STR * 2;
  constexpr int kStageBytes = WGM * WGN * 32 * CSTR * 4;
  // direct-to-LDS path: three unpadded buffers of one K step each
  constexpr bool kDma = kDirectLds && NKT > 0 && !EDGE && BK == 32;
  constexpr int kDmaBuf = (BM + BN) * BK * 2;
  constexpr int kDmaBytes = kDma ? 3 * kDmaBuf : 0;
  constexpr int kSmem0 = kTileBytes > kStageBytes ? kTileBytes : kStageBytes;
  __shared__ __attribute__((aligned(16))) char smem[kSmem0 > kDmaBytes ? kSmem0 : kDmaBytes];
  bf16 (*As)[BM * STR] = reinterpret_cast<bf16 (*)[BM * STR]>(smem);
  bf16 (*Ws)[BN * STR] = reinterpret_cast<bf16 (*)[BN * STR]>(smem + 2 * BM * STR * 2);

  const int b = blockIdx.x;
  const int tile = (b % kXcds) * per_xcd + b / kXcds;
  if (tile >= tiles_total) return;
  const int m0 = (tile / tiles_n) * BM;
  const int n0 = (tile % tiles_n) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = (wave / WGN) * (BM / WGM), wn = (wave % WGN) * (BN / WGN);

  uint4 ra[PF][LA], rw[PF][LW];
  // Without EDGE (M, N, K multiples of the tile) loads and LDS writes are
  // unconditional: no divergent branches, so the wait counts stay exact and
  // the loads stay in flight during the MFMAs.  With EDGE the address is
  // clamped into the matrix and chunks outside it are zeroed at the LDS
  // write.
  auto load_tile = [&](uint4 (&xa)[LA], uint4 (&xw)[LW], int k0) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int c = tid + NT * i;
      if constexpr ((BLK & 1) != 0) {
        // tile-blocked A: this tile's K step is one contiguous block
        xa[i] = ld16(A + ((size_t)(m0 / BM) * (K / BK) + k0 / BK) * (BM * BK) + (size_t)c * 8);
      } else {
        int gm = m0 + c / CPR, gk = k0 + (c % CPR) * 8;
        if (EDGE) { gm = min(gm, M - 1); gk = min(gk, K - 8); }
        xa[i] = ld16(A + (size_t)gm * K + gk);
      }
    }
#pragma unroll
    for (int i = 0; i < LW; ++i) {
      const int c = tid + NT * i;
      if constexpr ((BLK & 2) != 0) {
        xw[i] = ld16(W + ((size_t)(n0 / BN) * (K / BK) + k0 / BK) * (BN * BK) + (size_t)c * 8);
      } else {
        int gn = n0 + c / CPR, gk = k0 + (c % CPR) * 8;
        if (EDGE) { gn = min(gn, N - 1); gk = min(gk, K - 8); }
        xw[i] = ld16(W + (size_t)gn * K + gk);
      }
    }
  };
  auto store_tile = [&](const uint4 (&xa)[LA], const uint4 (&xw)[LW], int buf, int k0) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int c = tid + NT * i;
      const bool ok = !EDGE || (m0 + c / CPR < M && k0 + (c % CPR) * 8 < K);
      *reinterpret_cast<uint4*>(&As[buf][(c / CPR) * STR + (c % CPR) * 8]) =
          ok ? xa[i] : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < LW; ++i) {
      const int c = tid + NT * i;
      const bool ok = !EDGE || (n0 + c / CPR < N && k0 + (c % CPR) * 8 < K);
      *reinterpret_cast<uint4*>(&Ws[buf][(c / CPR) * STR + (c % CPR) * 8]) =
          ok ? xw[i] : uint4{0, 0, 0, 0};
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = NKT > 0 ? NKT : (K + BK - 1) / BK;
  const int frow = lane & 31;          // operand row within a 32-row fragment
  const int fk = (lane >> 5) * 8;      // operand k offset within a 16-k step
  auto read_frags = [&](int cur, int ks, bf16x8 (&af)[FM], bf16x8 (&wf)[FN]) {
#pragma unroll
    for (int t = 0; t < FM; ++t)
      af[t] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(
                      &As[cur][(wm + 32 * t + frow) * STR + ks + fk]));
#pragma unroll
    for (int t = 0; t < FN; ++t)
      wf[t] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(
                      &Ws[cur][(wn + 32 * t + frow) * STR + ks + fk]));
  };
  auto mfma_frags = [&](const bf16x8 (&af)[FM], const bf16x8 (&wf)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], af[i],
                                                            acc[i][j], 0, 0, 0);
  };
  auto compute = [&](int cur) {
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
      bf16x8 af[FM], wf[FN];
      read_frags(cur, ks, af, wf);
      mfma_frags(af, wf);
    }
  };
  if constexpr (kDma) {
    // Each K step of the A (W) tile is 16 (8) KB; every wave copies its
    // 1 KB units (16 rows x 64 bytes) straight into LDS
    // (global_load_lds_dwordx4: lane i's 16 bytes, from its own address,
    // land at the unit's base + 16 i), so no registers stage the tiles and
    // no LDS stores are issued.  A tile-blocked operand's unit is one
    // contiguous 1 KB of its K-step block; a row-major one's is 16 row
    // pieces of 64 bytes.
    // The LDS rows are unpadded (64 bytes); to keep the fragment reads free
    // of bank conflicts, slot i of a unit takes the chunk (row r, k-chunk
    // kc ^ ((r >> 2) & 3)) -- an XOR swizzle applied by choosing which
    // global chunk each lane loads, so the blocked layout itself is
    // unchanged and each unit still reads one contiguous 1 KB.  Three
    // buffers: tile kt is computed while tiles kt + 1 and kt + 2 load.
    // The waits are explicit (vmcnt counts this wave's copies in issue
    // order) and the barriers are plain s_barrier: a workgroup fence would
    // make the compiler wait for every copy in flight.
    static_assert(BM * BK * 2 % (1024 * WGM * WGN) == 0 && BN * BK * 2 % (1024 * WGM * WGN) == 0,
                  "whole 1 KB units per wave");
    static_assert(kGemmTileM % BM == 0, "A tiles split the blocked layout's row blocks");
    constexpr int UA = BM * BK * 2 / 1024 / (WGM * WGN);  // A units per wave
    constexpr int UW = BN * BK * 2 / 1024 / (WGM * WGN);  // W units per wave
    constexpr int kPerTile = UA + UW;                        // copies per wave per tile
    // this lane's chunk of a unit: its row and (swizzled) k-chunk
    auto swz_row = [&](int unit) { return (unit * 64 + lane) >> 2; };
    auto swz_kc = [&](int unit) {
      const int p = unit * 64 + lane;
      return (p & 3) ^ ((p >> 4) & 3);
    };
    // Tile-blocked operands hold kGemmTileM (A) and kGemmTileN (W) rows per
    // block.  An A tile of BM rows is a contiguous part of its block's K
    // step; a W unit (16 rows) lies in one block even where a tile of
    // another width starts mid-block.
    auto w_unit = [&](int kt, int unit) {
      if constexpr ((BLK & 2) != 0) {
        const int r0 = n0 + 16 * unit;
        const bf16* Wb = uniform_ptr(
            W + ((size_t)(r0 / kGemmTileN) * (K / BK) + kt) * (kGemmTileN * BK) +
            (size_t)(r0 % kGemmTileN) * BK);
        return Wb + (swz_row(unit) - 16 * unit) * BK + swz_kc(unit) * 8;
      } else {
        return uniform_ptr(W + (size_t)n0 * K + kt * BK) + swz_row(unit) * K +
               swz_kc(unit) * 8;
      }
    };
    auto issue = [&](int kt, int buf) {
      char* base = smem + buf * kDmaBuf;
      const bf16* Ab =
          (BLK & 1) ? uniform_ptr(A + ((size_t)(m0 / kGemmTileM) * (K / BK) + kt) *
                                          (kGemmTileM * BK) +
                                  (size_t)(m0 % kGemmTileM) * BK)
                    : uniform_ptr(A + (size_t)m0 * K + kt * BK);
      const int a_stride = (BLK & 1) ? BK : K;
#pragma unroll
      for (int i = 0; i < UA; ++i) {
        const int unit = wave * UA + i;
        __builtin_amdgcn_global_load_lds(
            (global_void_ptr)(Ab + swz_row(unit) * a_stride + swz_kc(unit) * 8),
            (lds_void_ptr)(base + unit * 1024), 16, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < UW; ++i) {
        const int unit = wave * UW + i;
        __builtin_amdgcn_global_load_lds((global_void_ptr)w_unit(kt, unit),
                                         (lds_void_ptr)(base + BM * BK * 2 + unit * 1024), 16,
                                         0, 0);
      }
    };
    auto frag = [&](const char* buf_base, int row, int kc) {
      return __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(
                      buf_base + row * 64 + ((kc ^ ((row >> 2) & 3)) * 16)));
    };
    issue(0, 0);
    issue(1, 1);
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      // tile kt has landed (this wave's copies of tile kt + 1 may be in
      // flight), then everyone's has, and everyone is done with kt - 1
      // (scheduling barriers: no copy may move across the wait + barrier)
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 1 < NKT)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(kPerTile));
      else
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 2 < NKT) issue(kt + 2, (kt + 2) % 3);
      const char* bA = smem + (kt % 3) * kDmaBuf;
      const char* bW = bA + BM * BK * 2;
      // The second 16-k half's fragment reads are interleaved with the
      // first half's MFMAs, and the wave's priority is raised while it
      // issues them (measured: QKV and FFN1 2-3 us faster).
      static_assert(BK == 32, "two 16-k halves per step");
      __builtin_amdgcn_s_setprio(1);
      {
        bf16x8 af0[FM], wf0[FN], af1[FM], wf1[FN];
        const int kc0 = lane >> 5, kc1 = 2 + (lane >> 5);
#pragma unroll
        for (int t = 0; t < FM; ++t) af0[t] = frag(bA, wm + 32 * t + frow, kc0);
#pragma unroll
        for (int t = 0; t < FN; ++t) wf0[t] = frag(bW, wn + 32 * t + frow, kc0);
#pragma unroll
        for (int t = 0; t < FM; ++t) af1[t] = frag(bA, wm + 32 * t + frow, kc1);
#pragma unroll
        for (int t = 0; t < FN; ++t) wf1[t] = frag(bW, wn + 32 * t + frow, kc1);
        mfma_frags(af0, wf0);
        mfma_frags(af1, wf1);
        // the first half's reads, then MFMA / read pairs, then the rest
        __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);
#pragma unroll
        for (int i = 0; i < FM + FN; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * FM * FN - (FM + FN), 0);
      }
      __builtin_amdgcn_s_setprio(0);
    }
    // the epilogue reuses the buffers: every wave's fragment reads are done
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  } else if constexpr (PF == 1) {
    load_tile(ra[0], rw[0], 0);
    store_tile(ra[0], rw[0], 0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) load_tile(ra[0], rw[0], (kt + 1) * BK);
      compute(cur);
      if (kt + 1 < nk) {
        store_tile(ra[0], rw[0], cur ^ 1, (kt + 1) * BK);
        __syncthreads();
      }
    }
  } else {
    static_assert(PF == 2 && NKT > 0 && NKT % 2 == 0,
                  "the two-tile prefetch needs an unrolled K loop");
    // Two tiles in flight: register set kt % 2 holds tile kt + 2's loads;
    // LDS buffer kt % 2 holds tile kt (measured: a third tile in flight
    // gains nothing).
    load_tile(ra[0], rw[0], 0);
#pragma unroll
    for (int q = 1; q < PF; ++q) load_tile(ra[q], rw[q], q * BK);
    store_tile(ra[0], rw[0], 0, 0);
    __syncthreads();
    // Within a step: issue tile kt + PF's loads first, then the first 16 k
    // of MFMAs, then write tile kt + 1 (loaded earlier) into the other LDS
    // buffer -- free since the barrier that ended step kt - 1 -- so the
    // writes overlap the second half's MFMAs; one barrier ends the step.
    // Scheduling barriers keep the compiler from sinking the loads and
    // writes behind the MFMAs (measured: a few percent on every projection;
    // reading both halves' fragments up front was slower).
    static_assert(BK == 32, "two 16-k halves per step");
    auto step = [&](auto set_c, auto buf_c, int kt) {
      constexpr int set = decltype(set_c)::value, nset = (set + 1) % PF;
      constexpr int buf = decltype(buf_c)::value;
      if (kt + PF < nk) load_tile(ra[set], rw[set], (kt + PF) * BK);
      __builtin_amdgcn_sched_barrier(0);
      {
        bf16x8 af[FM], wf[FN];
        read_frags(buf, 0, af, wf);
        mfma_frags(af, wf);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 1 < nk) store_tile(ra[nset], rw[nset], buf ^ 1, (kt + 1) * BK);
      __builtin_amdgcn_sched_barrier(0);
      {
        bf16x8 af[FM], wf[FN];
        read_frags(buf, 16, af, wf);
        mfma_frags(af, wf);
      }
      if (kt + 1 < nk) __syncthreads();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
#pragma unroll
    for (int kt = 0; kt < nk; kt += 2) {  // register set and buffer repeat
      step(I0{}, I0{}, kt);
      step(I1{}, I1{}, kt + 1);
    }
  }

  // Epilogue through LDS: each wave stages one 32-row fragment row of its
  // tile at a time as float32 in its own slice of the (now idle) tile
  // buffers, then writes those rows back with 16-byte stores by consecutive
  // lanes (R added in float32, one rounding to bf16).  The residual chunks
  // of the whole wave tile are loaded first, so their latency overlaps the
  // staging.  One workgroup barrier (the tile buffers are free); after it
  // each wave works in its own slice.
  float* Cs = reinterpret_cast<float*>(smem) + wave * 32 * CSTR;
  constexpr int CPRO = TN / 8;          // 16-byte output chunks per staged row
  constexpr int CPL = 32 * CPRO / 64;   // chunks per lane per fragment row
  uint4 rres[FM][CPL];
  if (R) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int q = 0; q < CPL; ++q) {
        const int c = lane + 64 * q;
        const int r = c / CPRO, cc = (c % CPRO) * 8;
        int gm = m0 + wm + 32 * i + r, gn = n0 + wn + cc;
        if (EDGE) { gm = min(gm, M - 1); gn = min(gn, N - 8); }
        // read once: streamed past the caches
        rres[i][q] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                                   reinterpret_cast<const u32x4*>(
                                                       R + (size_t)gm * N + gn)));
      }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int cc = 32 * j + 8 * g + 4 * (lane >> 5);
        *reinterpret_cast<float4*>(&Cs[frow * CSTR + cc]) =
            make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                        acc[i][j][4 * g + 3]);
      }
    // the slice is this wave's own: ordering the wave's LDS accesses is
    // enough (no workgroup barrier)
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const int c = lane + 64 * q;
      const int r = c / CPRO, cc = (c % CPRO) * 8;
      const int gm = m0 + wm + 32 * i + r, gn = n0 + wn + cc;
      const float4 lo = *reinterpret_cast<const float4*>(&Cs[r * CSTR + cc]);
      const float4 hi = *reinterpret_cast<const float4*>(&Cs[r * CSTR + cc + 4]);
      float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      if (R) {
        const uint32_t rw4[4] = {rres[i][q].x, rres[i][q].y, rres[i][q].z, rres[i][q].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[2 * t] += __uint_as_float(rw4[t] << 16);
          v[2 * t + 1] += __uint_as_float(rw4[t] & 0xffff0000u);
        }
      }
      if (!EDGE || (gm < M && gn < N)) {
        const u32x4 vv = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                          pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
        // BLK bit 2: C channel-planar, element (m, n) at
        // (n / 64) * M * 64 + m * 64 + n % 64 (a wave tile's 64 columns are
        // one plane, so its rows are one contiguous run)
        u32x4* dst = reinterpret_cast<u32x4*>(
            (BLK & 4) ? C + (size_t)(gn / 64) * ((size_t)M * 64) + (size_t)gm * 64 + gn % 64
                      : C + (size_t)gm * N + gn);
        // the QKV and FFN projections stream their outputs past the caches
        // (measured: FFN1 -8 us and QKV -2.5 us, the convs reading them
        // at most 1 us slower; the output projection's x1, read twice
        // more, gained nothing)
        if constexpr (SITE != 1)
          __builtin_nontemporal_store(vv, dst);
        else
          *dst = vv;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
}

template <int BM, int BN, int BK, int WGM, int WGN, int SITE, int PF, bool EDGE,
          int NKT, int BLK = 0>
void launch_tiles(const void* A, const void* W, const void* R, void* C, int M,
                  int N, int K, hipStream_t s) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int total = tiles_m * tiles_n;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  gemm_mfma_bf16<BM, BN, BK, WGM, WGN, SITE, PF, EDGE, NKT, BLK>
      <<<per_xcd * kXcds, 64 * WGM * WGN, 0, s>>>(
          static_cast<const bf16*>(A), static_cast<const bf16*>(W),
          static_cast<const bf16*>(R), static_cast<bf16*>(C), M, N, K, tiles_n,
          total, per_xcd);
}

// Shapes that are whole tiles with K = 128, 256, 384 or 1536 (the block's
// projections at C = 384, the module's at C = 128 and 256) get the unrolled
// K loop with copies straight into LDS; other whole-tile shapes a runtime K
// loop; ragged shapes the bounds-checked variant (plain layouts
// only).  blk: bit 0 A tile-blocked, bit 1 W tile-blocked.
template <int BM, int BN, int BK, int WGM, int WGN, int SITE, int PF, bool EDGE, int NKT>
void launch_blk(int blk, const void* A, const void* W, const void* R, void* C,
                int M, int N, int K, hipStream_t s) {
  switch (blk) {
    case 1: launch_tiles<BM, BN, BK, WGM, WGN, SITE, PF, EDGE, NKT, 1>(A, W, R, C, M, N, K, s); break;
    case 2: launch_tiles<BM, BN, BK, WGM, WGN, SITE, PF, EDGE, NKT, 2>(A, W, R, C, M, N, K, s); break;
    case 3: launch_tiles<BM, BN, BK, WGM, WGN, SITE, PF, EDGE, NKT, 3>(A, W, R, C, M, N, K, s); break;
    case 7:
      if constexpr (!EDGE && NKT > 0 && BN / WGN == 64)
        launch_tiles<BM, BN, BK, WGM, WGN, SITE, PF, EDGE, NKT, 7>(A, W, R, C, M, N, K, s);
      break;
    default: launch_tiles<BM, BN, BK, WGM, WGN, SITE, PF, EDGE, NKT, 0>(A, W, R, C, M, N, K, s); break;
  }
}

template <int BM, int BN, int BK, int WGM, int WGN, int SITE>
hipError_t run_tiles(const void* A, const void* W, const void* R, void* C, int M,
                     int N, int K, int blk, hipStream_t s) {
  if (M % BM || N % BN || K % BK) {
    if (blk) return hipErrorInvalidValue;
    launch_tiles<BM, BN, BK, WGM, WGN, SITE, 1, true, 0>(A, W, R, C, M, N, K, s);
  } else if (K == 12 * BK) {
    launch_blk<BM, BN, BK, WGM, WGN, SITE, 2, false, 12>(blk, A, W, R, C, M, N, K, s);
  } else if (K == 48 * BK) {
    launch_blk<BM, BN, BK, WGM, WGN, SITE, 2, false, 48>(blk, A, W, R, C, M, N, K, s);
  } else if (K == 8 * BK) {
    launch_blk<BM, BN, BK, WGM, WGN, SITE, 2, false, 8>(blk, A, W, R, C, M, N, K, s);
  } else if (K == 4 * BK) {
    launch_blk<BM, BN, BK, WGM, WGN, SITE, 2, false, 4>(blk, A, W, R, C, M, N, K, s);
  } else {
    launch_blk<BM, BN, BK, WGM, WGN, SITE, 1, false, 0>(blk, A, W, R, C, M, N, K, s);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// float32 FMA kernel
// ---------------------------------------------------------------------------

constexpr int kTM = 64, kTN = 64, kTK = 16;

__global__ __launch_bounds__(256) void gemm_f32(const float* __restrict__ A,
                                                const float* __restrict__ W,
                                                const float* __restrict__ R,
                                                float* __restrict__ C, int M,
                                                int N, int K) {
  __shared__ float As[kTK][kTM + 4];
  __shared__ float Bs[kTK][kTN + 4];
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  const int m0 = blockIdx.y * kTM, n0 = blockIdx.x * kTN;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += kTK) {
    for (int i = tid; i < kTM * kTK; i += 256) {
      const int mm = i / kTK, kk = i % kTK;
      const int gm = m0 + mm, gk = k0 + kk;
      As[kk][mm] = (gm < M && gk < K) ? A[(size_t)gm * K + gk] : 0.f;
    }
    for (int i = tid; i < kTN * kTK; i += 256) {
      const int nn = i / kTK, kk = i % kTK;
      const int gn = n0 + nn, gk = k0 + kk;
      Bs[kk][nn] = (gk < K && gn < N) ? W[(size_t)gn * K + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kTK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gm = m0 + ty * 4 + i;
    if (gm >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + tx * 4 + j;
      if (gn >= N) continue;
      float v = acc[i][j];
      if (R) v += R[(size_t)gm * N + gn];
      C[(size_t)gm * N + gn] = v;
    }
  }
}


// One tile shape for every projection: 256x128 with 2x2 waves of 128x64
// measured best on MI355X for all four projection shapes of the block
// (M = 65536; N, K = 1152, 384 / 384, 384 / 1536, 384 / 384, 1536); 128x128
// only where 256x128 tiles would leave CUs idle.
constexpr int kSmallTileBelow = 512;
template <int SITE>
hipError_t run_mfma(const void* A, const void* W, const void* R, void* C, int M,
                    int N, int K, int blk, hipStream_t s) {
  static_assert(kGemmTileM == 256 && kGemmTileN == 128 && kGemmTileK == 32,
                "the blocked layout follows the tile");
  // Launches that would give fewer than two 256x128 tiles per CU take
  // 128x128 tiles (2x2 waves of 64x64): twice the workgroups, where the
  // larger tile's lower LDS traffic per flop no longer matters.
  if (M % 128 == 0 && N % 128 == 0 && (int64_t)(M / 256) * (N / 128) < kSmallTileBelow) {
    if (K == 4 * kGemmTileK) {
      launch_blk<128, 128, 32, 2, 2, SITE, 2, false, 4>(blk, A, W, R, C, M, N, K, s);
      return hipGetLastError();
    }
    if (K == 8 * kGemmTileK) {
      launch_blk<128, 128, 32, 2, 2, SITE, 2, false, 8>(blk, A, W, R, C, M, N, K, s);
      return hipGetLastError();
    }
    if (K == 12 * kGemmTileK) {
      launch_blk<128, 128, 32, 2, 2, SITE, 2, false, 12>(blk, A, W, R, C, M, N, K, s);
      return hipGetLastError();
    }
  }
  return run_tiles<256, 128, 32, 2, 2, SITE>(A, W, R, C, M, N, K, blk, s);
}

}  // namespace

bool gemm_whole_tiles(int M, int N, int K) {
  return M % kGemmTileM == 0 && N % kGemmTileN == 0 && K % kGemmTileK == 0;
}

bool gemm_planar_ok(bool bf, int M, int N, int K, bool a_blocked, bool w_blocked) {
  return bf && a_blocked && w_blocked && gemm_whole_tiles(M, N, K) &&
         (K == 12 * kGemmTileK || K == 48 * kGemmTileK);
}

hipError_t launch_gemm(bool bf, const void* A, const void* W, const void* R,
                       void* C, int M, int N, int K, hipStream_t s,
                       GemmSite site, bool a_blocked, bool w_blocked, bool c_planar) {
  if (M == 0 || N == 0) return hipSuccess;
  const int blk = (a_blocked ? 1 : 0) | (w_blocked ? 2 : 0) | (c_planar ? 4 : 0);
  if (blk && (!bf || !gemm_whole_tiles(M, N, K))) return hipErrorInvalidValue;
  if (c_planar && !gemm_planar_ok(bf, M, N, K, a_blocked, w_blocked))
    return hipErrorInvalidValue;
  if (bf) {
    switch (site) {
      case GemmSite::kQkv: return run_mfma<0>(A, W, R, C, M, N, K, blk, s);
      case GemmSite::kOut: return run_mfma<1>(A, W, R, C, M, N, K, blk, s);
      case GemmSite::kFfn1: return run_mfma<2>(A, W, R, C, M, N, K, blk, s);
      default: return run_mfma<3>(A, W, R, C, M, N, K, blk, s);
    }
  } else {
    dim3 grid((N + kTN - 1) / kTN, (M + kTM - 1) / kTM);
    gemm_f32<<<grid, 256, 0, s>>>(static_cast<const float*>(A),
                                  static_cast<const float*>(W),
                                  static_cast<const float*>(R),
                                  static_cast<float*>(C), M, N, K);
  }
  return hipGetLastError();
}

}  // namespace hsmla
