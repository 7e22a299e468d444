// int8 x int8 -> int32 MFMA GEMM with the fused W8A8 scale epilogue (gfx950).
//
// acc[m,n] = sum_k xq[m,k] * wq[n,k]   (int32, exact; unsloth commit log of
//   test_diffusion_transformer_quant.py: int8 products, int32 accumulation)
// y[m,n]   = bf16(((fl32(acc) * a_scale[m]) * w_scale[n]) + bias[n])
//   (bias and y fp16 instead for fp16 layers; the same fp32 steps)
//   (Issue 5 probe, "Round two": the int8 scaled-MM result carries act_scale
//    and the fp32 per-channel weight scale)
//
// Design (CDNA4):
// * v_mfma_i32_32x32x32_i8 (on gfx950 it runs at the full int8 rate from a
//   single wave per SIMD; the 16x16x64 form sustains about half of it). The
//   MFMA "A" operand is a 32-row block of W and the "B" operand a 32-row block
//   of xq (both K-contiguous, no transpose), so each lane's 16 accumulators
//   are four runs of four consecutive output columns n of one output row m:
//   the epilogue stores 8 bytes of bf16 per run.
// * Two kernels. 256 x 256 tiles run on eight waves that take turns on the
//   matrix cores (gemm_pp_kernel, 64-byte K stages in a ring of four LDS
//   buffers; its comment gives the schedule). 128 x 128 and 64 x 64 tiles run
//   on four waves, each wave a WM x WN sub-tile of (WN/32)*(WM/32) MFMA
//   blocks, with K stages of 128 bytes (gemm_i8_kernel; within a stage the
//   fragment reads of k-step s+1 are interleaved with the MFMAs of k-step s).
// * Panels stream global -> LDS with buffer_load_dwordx4 ... lds (no VGPR
//   staging, no ds_write). One wave-instruction fills 1 KiB of LDS linearly
//   by lane; each lane picks the global 16-byte chunk that belongs at its LDS
//   slot, which realises an XOR swizzle of the 16-byte chunks so that the
//   ds_read_b128 of 8 consecutive rows hit distinct banks.
// * Four-wave kernel: a two-stage LDS ring; loads for stage kt+1 are issued
//   right after the barrier of stage kt; one barrier per stage; the wait
//   before it only counts this stage's loads (exact s_waitcnt vmcnt).
// * Filling the chip: 256 x 256 tiles run whole or as two 128-row halves
//   (the last round of an XCD's tiles when it is at most half full, every
//   tile when all of them fill at most half of the compute units; one
//   launch either way). K is split only on 128 x 128 and 64 x 64 tiles, with
//   int32 partial sums in the caller's workspace and a second kernel that
//   adds them before the epilogue.
// * Out-of-range rows read as zeros through the buffer descriptor's bound;
//   K-tail chunks are sent out of bounds, so ragged M, N and K need no branch.
// * Output stores are non-temporal, so the output does not evict the panels
//   the other tiles re-read from L2.
// * Tile order: every XCD (workgroups are dealt round-robin over the 8 XCDs)
//   takes a contiguous range of a grouped tile order (4 m-tiles per group),
//   so the tiles that run together on one XCD share W and xq panels in that
//   XCD's L2.
#include <type_traits>
#include <utility>

#include "row_groups.h"
#include "w8a8_device.h"
#include "w8a8_kernels.h"

namespace w8a8 {

namespace {

// Output stores are non-temporal: allocated in L2, the output tiles evict
// the W / xq panels that the other tiles of the launch are still re-reading
// (measured over the DiT block, 559 -> 522 us; out- and down-proj 12%
// faster).
constexpr int kOutAux = 2;

// s_waitcnt vmcnt(N) lgkmcnt(0): at most N vector-memory ops (this wave's
// newer panel loads) still in flight and every LDS read of this wave done.
// gfx9 encoding: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt in
// bits 6:4 (7 = no wait), lgkmcnt in bits 11:8.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Swizzled position of logical 16-byte chunk c of LDS row `row`. The LDS
// serves 16 lanes of a ds_read_b128 per cycle from 64 banks (256 bytes), and
// the 16 lanes read rows r..r+15 of one chunk; keying the XOR on row >> 1
// puts those 16 reads in 16 distinct 16-byte bank groups.
template <int BK>
__device__ __forceinline__ int swz(int row, int c) {
  if constexpr (BK == 128) return c ^ ((row >> 1) & 7);
  else return c ^ ((row >> 1) & 3);
}

// (tm, tn) of the workgroup: XCD-contiguous ranges of a grouped order.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int t = xcd * (T >> 3) + min(xcd, T & 7) + local;
  // m-tiles per group: 4 (measured over the DiT block: QKV 134 -> 130 us
  // against 8; 3 and 6 are within noise of 4, 17 is slower)
  constexpr int G = 4;
  const int group = t / (G * tiles_n);
  const int first_m = group * G;
  const int gm = min(G, tiles_m - first_m);
  const int r = t - group * G * tiles_n;
  tm = first_m + r % gm;
  tn = r / gm;
}

// Whole tiles of an XCD's run of tx tiles over its cpx compute units (cpx
// = 0: all whole): all of them but the last round when that round is at
// most half full, none when the whole run is (its tiles then run as
// halves, twice as many pieces of half the work, instead of as a split K).
__host__ __device__ inline int pp_whole_tiles(int tx, int cpx) {
  if (cpx <= 0) return tx;
  if (2 * tx <= cpx) return 0;
  const int rem = tx > cpx ? tx % cpx : 0;
  return (rem > 0 && 2 * rem <= cpx) ? tx - rem : tx;
}

// Block -> tile for the ping-pong kernel. XCD x (blockIdx & 7; the hardware
// hands workgroups to the XCDs in turn) takes the same contiguous run of
// tiles as tile_coords, in dispatch order. Beyond the run's whole tiles
// (pp_whole_tiles), each tile is split into two 128-row halves (half = 0,
// 1), numbered after the whole tiles (half = -1). Returns false for a
// block past its XCD's pieces.
__device__ __forceinline__ bool tile_coords_halves(int tiles_m, int tiles_n, int cpx, int& tm,
                                                   int& tn, int& half) {
  const int T = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int tx = (T >> 3) + (xcd < (T & 7) ? 1 : 0);
  const int whole = pp_whole_tiles(tx, cpx);
  int t = xcd * (T >> 3) + min(xcd, T & 7);
  half = -1;
  if (local < whole) {
    t += local;
  } else {
    const int h = local - whole;
    if (h >= 2 * (tx - whole)) return false;
    t += whole + (h >> 1);
    half = h & 1;
  }
  constexpr int G = 4;     // m-tiles per group, as tile_coords
  const int group = t / (G * tiles_n);
  const int first_m = group * G;
  const int gm = min(G, tiles_m - first_m);
  const int r = t - group * G * tiles_n;
  tm = first_m + r % gm;
  tn = r / gm;
  return true;
}

// Instruction order of one stage for the scheduler: the fragment reads of
// k-step 0, then per k-step its MFMAs in groups, each group followed by one
// fragment read of the next k-step and (in the first half of the stage) by
// panel loads for a later stage.
template <int KS, int KREADS, int KMFMA, int LOADS, int KSTEP>
__device__ __forceinline__ void sched_kstep() {
  constexpr int kPer = KMFMA / KREADS > 0 ? KMFMA / KREADS : 1;
  constexpr int kGroups = KMFMA / kPer < KREADS ? KMFMA / kPer : KREADS;
  constexpr int kIssueSteps = KS > 1 ? KS / 2 : 1;
  constexpr int kLoadsHere = KSTEP < kIssueSteps ? (LOADS + kIssueSteps - 1) / kIssueSteps : 0;
  constexpr int kLoadsPer = kLoadsHere / kGroups;
  constexpr bool kRead = KSTEP + 1 < KS;
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    __builtin_amdgcn_sched_group_barrier(0x008, kPer, 0);
    if constexpr (kRead) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if constexpr (kLoadsPer > 0) __builtin_amdgcn_sched_group_barrier(0x020, kLoadsPer, 0);
  }
  if constexpr (KMFMA - kPer * kGroups > 0)
    __builtin_amdgcn_sched_group_barrier(0x008, KMFMA - kPer * kGroups, 0);
  if constexpr (kRead && KREADS - kGroups > 0)
    __builtin_amdgcn_sched_group_barrier(0x100, KREADS - kGroups, 0);
  if constexpr (kLoadsHere - kLoadsPer * kGroups > 0)
    __builtin_amdgcn_sched_group_barrier(0x020, kLoadsHere - kLoadsPer * kGroups, 0);
}

template <int KS, int KREADS, int KMFMA, int LOADS, int... STEPS>
__device__ __forceinline__ void sched_stage(std::integer_sequence<int, STEPS...>) {
  __builtin_amdgcn_sched_group_barrier(0x100, KREADS, 0);
  (sched_kstep<KS, KREADS, KMFMA, LOADS, STEPS>(), ...);
}

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (or fp16) values, round to nearest even, packed
// low/high (v_cvt_pk_bf16_f32 on gfx950 for bf16).
template <bool F16>
__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
  if constexpr (F16) {
    const v2h h = __builtin_convertvector((v2f){lo, hi}, v2h);
    return __builtin_bit_cast(uint32_t, h);
  } else {
    const v2bf h = __builtin_convertvector((v2f){lo, hi}, v2bf);
    return __builtin_bit_cast(uint32_t, h);
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int BK, int S, bool HAS_BIAS, bool F16,
          bool SPLIT = false>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_i8_kernel(GemmArgs a, int tiles_m,
                                                                         int tiles_n, int vec_flags,
                                                                         int kps) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FM = WM / 32, FN = WN / 32;
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold 32x32 blocks");
  static_assert(BK == 64 || BK == 128, "stage = 2 or 4 32-byte MFMA k-steps");
  constexpr int KS = BK / 32;               // MFMA k-steps per stage
  constexpr int CH = BK / 16;               // 16-byte chunks per LDS row
  constexpr int RPI = 1024 / BK;            // LDS rows per wave-instruction
  constexpr int JW = BN * BK / 1024, JX = BM * BK / 1024;
  static_assert(JW % NW == 0 && JX % NW == 0, "panel loads must split evenly over waves");
  constexpr int LW = JW / NW, LX = JX / NW, LPS = LW + LX;
  static_assert(S == 2, "two LDS stages (double buffer)");
  static_assert(LPS < 64, "vmcnt range");
  constexpr int STAGE = (BM + BN) * BK;     // bytes per LDS stage (W rows then xq rows)

  // Two separate arrays (not one indexed by kt % 2): the compiler can then
  // prove that loads into one stage do not touch the other stage being read,
  // and interleave them.
  __shared__ __attribute__((aligned(1024))) int8_t lds0[STAGE];
  __shared__ __attribute__((aligned(1024))) int8_t lds1[STAGE];
  // the tile's activation scales, weight scales and bias, for the epilogue
  __shared__ __attribute__((aligned(16))) float lds_sa[BM];
  __shared__ __attribute__((aligned(16))) float lds_sw[BN];
  __shared__ __attribute__((aligned(16))) float lds_b[HAS_BIAS ? BN : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar
  const int wave_m = wave % WAVES_M, wave_n = wave / WAVES_M;
  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t M = a.M, N = a.N, K = a.K;

  const uint32_t rows_w = (uint32_t)min<int64_t>(BN, N - n0);
  const uint32_t rows_x = (uint32_t)min<int64_t>(BM, M - m0);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.wq + n0 * K, rows_w * (uint32_t)K);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.xq + m0 * K, rows_x * (uint32_t)K);
  // bytes of K this workgroup reads (chunks at or past it go out of bounds)
  const int kend = (int)min<int64_t>(K, (int64_t)min<int64_t>((int64_t)(blockIdx.y + 1) * kps,
                                                              (K + BK - 1) / BK) * BK);

  // Scales and bias of the tile into LDS (zero past M / N); the first stage
  // barrier of the K loop makes them visible to every wave.
  {
    const __amdgpu_buffer_rsrc_t r_sa = make_rsrc(a.a_scale + m0, rows_x * 4u);
    const __amdgpu_buffer_rsrc_t r_sw = make_rsrc(a.w_scale + n0, rows_w * 4u);
    for (int t = tid; t < BM; t += 64 * NW)
      lds_sa[t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_sa, t * 4, 0, 0));
    for (int t = tid; t < BN; t += 64 * NW)
      lds_sw[t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_sw, t * 4, 0, 0));
    if constexpr (HAS_BIAS) {
      const __amdgpu_buffer_rsrc_t r_b = make_rsrc(a.bias + n0, rows_w * 2u);
      for (int t = tid; t < BN; t += 64 * NW)
        lds_b[t] = half_to_f32<F16>(__builtin_amdgcn_raw_buffer_load_b16(r_b, t * 2, 0, 0));
    }
  }

  // Load j of the wave fills LDS rows (wave*L + j)*RPI + lane/CH; lane takes
  // the global chunk that belongs at its LDS slot under the swizzle.
  uint32_t off_w[LW], off_x[LX];
  int kc_w[LW], kc_x[LX];
#pragma unroll
  for (int j = 0; j < LW; ++j) {
    const int row = (wave * LW + j) * RPI + lane / CH;
    kc_w[j] = 16 * swz<BK>(row, lane % CH);
    off_w[j] = (uint32_t)row * (uint32_t)K + kc_w[j];
  }
#pragma unroll
  for (int j = 0; j < LX; ++j) {
    const int row = (wave * LX + j) * RPI + lane / CH;
    kc_x[j] = 16 * swz<BK>(row, lane % CH);
    off_x[j] = (uint32_t)row * (uint32_t)K + kc_x[j];
  }
  auto issue = [&](int kt, int8_t* st) {
    const int k0 = kt * BK;
    const int klim = kend - k0;
#pragma unroll
    for (int j = 0; j < LW; ++j) {
      // chunks past K (only in a K-tail stage) go out of bounds, branch-free
      const uint32_t keep = (uint32_t)((kc_w[j] - klim) >> 31);
      const uint32_t off = ((off_w[j] + k0) & keep) | (kOOB & ~keep);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, st + (wave * LW + j) * 1024, 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < LX; ++j) {
      const uint32_t keep = (uint32_t)((kc_x[j] - klim) >> 31);
      const uint32_t off = ((off_x[j] + k0) & keep) | (kOOB & ~keep);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, st + BN * BK + (wave * LX + j) * 1024, 16, off,
                                               0, 0, 0);
    }
  };

  v16i acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v16i{};

  // Fragment addresses: lane reads row 32*blk + lane%32 of its wave's rows,
  // 16-byte chunk (2*ks + lane/32) of the stage. The swizzle depends on the
  // low row bits only, so block b sits 32*BK*b bytes after block 0.
  const int frag_row = lane & 31, frag_half = lane >> 5;
  int fw_base[KS], fx_base[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    fw_base[ks] = (wave_n * WN + frag_row) * BK + 16 * swz<BK>(frag_row, 2 * ks + frag_half);
    fx_base[ks] = BN * BK + (wave_m * WM + frag_row) * BK + 16 * swz<BK>(frag_row, 2 * ks + frag_half);
  }
  // K stages of this workgroup: all of them, or with split K (grid.y > 1)
  // stages kb .. ke-1; loads past ke*BK go out of bounds (read nothing)
  const int nk_all = (int)((K + BK - 1) / BK);
  const int kb = (int)blockIdx.y * kps;
  const int ke = min(nk_all, kb + kps);

  // One stage: read the fragments of k-step 0, then run the MFMAs of each
  // k-step with the next k-step's fragment reads spread between them. With
  // ISSUE, the panel loads of stage kt+S-1 are spread over the first half of
  // the MFMAs, so the memory path drains while the matrix core works.
  auto stage = [&](int kt, const int8_t* st, int8_t* next, auto issue_tag) {
    constexpr bool ISSUE = decltype(issue_tag)::value;
    if constexpr (ISSUE) issue(kt + 1, next);
    v4i fw[KS][FN], fx[KS][FM];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int i = 0; i < FN; ++i)
        fw[ks][i] = *reinterpret_cast<const v4i*>(st + fw_base[ks] + 32 * BK * i);
#pragma unroll
      for (int j = 0; j < FM; ++j)
        fx[ks][j] = *reinterpret_cast<const v4i*>(st + fx_base[ks] + 32 * BK * j);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fw[ks][i], fx[ks][j], acc[i][j], 0, 0, 0);
    sched_stage<KS, FN + FM, FN * FM, ISSUE ? LPS : 0>(std::make_integer_sequence<int, KS>{});
  };

  // Double-buffered K loop: stage kt computes from one buffer while the
  // loads of stage kt+1 fill the other; each stage begins with this wave's
  // loads landed (vmcnt 0) and a barrier (everyone's loads landed, and
  // everyone done reading the buffer about to be refilled). The last stage's
  // "next" loads have K offsets past the end, so they only write zeros into
  // the idle buffer, which keeps every stage body identical.
  issue(kb, lds0);
  int kt = kb;
  for (; kt + 1 < ke; kt += 2) {
    wait_vmcnt_lgkm0<0>();
    stage_barrier();
    stage(kt, lds0, lds1, std::true_type{});
    wait_vmcnt_lgkm0<0>();
    stage_barrier();
    stage(kt + 1, lds1, lds0, std::true_type{});
  }
  if (kt < ke) {
    wait_vmcnt_lgkm0<0>();
    stage_barrier();
    stage(kt, lds0, lds1, std::true_type{});
  }

  // Split K: this workgroup's int32 partial sums, 16-byte stores of four
  // consecutive columns (N % 8 == 0 on this path) into slice blockIdx.y; the
  // reduction kernel adds the slices and applies the epilogue.
  if constexpr (SPLIT) {
    const __amdgpu_buffer_rsrc_t r_p =
        make_rsrc(a.partial + ((int64_t)blockIdx.y * M + m0) * N + n0,
                  (uint32_t)(((int64_t)(rows_x - 1) * N + rows_w) * 4));
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int ml = wave_m * WM + 32 * j + frag_row;
        const v16i& c = acc[i][j];
        // four-column runs q = 0..3 are elements 4q..4q+3: register sub-ranges
        const v4i run[4] = {c.lo.lo, c.lo.hi, c.hi.lo, c.hi.hi};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = wave_n * WN + 32 * i + 8 * q + 4 * frag_half;
          const uint32_t off = (nl < (int)rows_w) ? (uint32_t)(ml * N + nl) * 4u : kOOB;
          __builtin_amdgcn_raw_buffer_store_b128(run[q], r_p, off, 0, 0);
        }
      }
    return;
  }

  // Epilogue. Lane holds, for output row m = mb + lane%32, the columns
  // n = nb + 8*q + 4*(lane/32) + r in acc element 4*q + r (q, r = 0..3).
  // Branch-free: scales and bias come through buffer loads (zero past the
  // end), stores go through buffer stores whose offset is sent out of bounds
  // for columns >= N; rows >= M fall past the descriptor's bound.
  __builtin_amdgcn_sched_barrier(0);
  const int64_t ldo = a.ldo;
  const __amdgpu_buffer_rsrc_t r_out =
      make_rsrc(a.out + m0 * ldo + n0, (uint32_t)(((int64_t)(rows_x - 1) * ldo + rows_w) * 2));
  float sa[FM];
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int ml = wave_m * WM + 32 * j + frag_row;
    sa[j] = lds_sa[ml];
  }
  // Output tile staged through LDS (free after the K loop) when rows can be
  // written with 16-byte stores: each lane's four bf16 go to LDS, then every
  // thread writes 16 contiguous bytes of a row, so a wave stores two whole
  // 512-byte row segments per instruction. Layout: tile row r (BN*2 bytes),
  // 16-byte chunk c stored at chunk c ^ (r & 31), which keeps both the
  // column-wise writes and the row-wise reads free of bank conflicts.
  // The store path is chosen once per workgroup; each path is branch-free.
  constexpr bool kStageOut = (BN * 2 == 512) && (BM * BN * 2 <= 2 * STAGE);
  // visit(i, q, j, nl, ml, y01, y23) for every group of four outputs
  auto for_each_out = [&](auto&& visit) {
#pragma unroll
    for (int i = 0; i < FN; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = wave_n * WN + 32 * i + 8 * q + 4 * frag_half;
        const float4 sw4 = *reinterpret_cast<const float4*>(&lds_sw[nl]);
        float b4[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (HAS_BIAS) {
          const float4 bb = *reinterpret_cast<const float4*>(&lds_b[nl]);
          b4[0] = bb.x; b4[1] = bb.y; b4[2] = bb.z; b4[3] = bb.w;
        }
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          const int ml = wave_m * WM + 32 * j + frag_row;
          const v16i& c = acc[i][j];
          const float t0 = epilogue_f32<HAS_BIAS>(c[4 * q + 0], sa[j], sw4.x, b4[0]);
          const float t1 = epilogue_f32<HAS_BIAS>(c[4 * q + 1], sa[j], sw4.y, b4[1]);
          const float t2 = epilogue_f32<HAS_BIAS>(c[4 * q + 2], sa[j], sw4.z, b4[2]);
          const float t3 = epilogue_f32<HAS_BIAS>(c[4 * q + 3], sa[j], sw4.w, b4[3]);
          visit(nl, ml, pack_half2<F16>(t0, t1), pack_half2<F16>(t2, t3));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (kStageOut && (vec_flags & 4)) {
    wait_vmcnt_lgkm0<0>();
    stage_barrier();                      // every wave is done reading the K stages
    for_each_out([&](int nl, int ml, uint32_t y01, uint32_t y23) {
      const int c = nl >> 3;                                 // 16-byte chunk of the row
      int8_t* rowp = (ml < BM / 2 ? lds0 + ml * 512 : lds1 + (ml - BM / 2) * 512);
      *reinterpret_cast<v2u*>(rowp + 16 * (c ^ (ml & 31)) + 8 * frag_half) = (v2u){y01, y23};
    });
    __syncthreads();
    constexpr int kThreads = 64 * NW;
    constexpr int kRowsPerPass = kThreads / 32;
    const int c = tid & 31;
#pragma unroll 4
    for (int r = tid >> 5; r < BM; r += kRowsPerPass) {
      const int8_t* rowp = (r < BM / 2 ? lds0 + r * 512 : lds1 + (r - BM / 2) * 512);
      const v4i v = *reinterpret_cast<const v4i*>(rowp + 16 * (c ^ (r & 31)));
      // N % 8 == 0 here: the eight columns of a chunk are all valid or not
      const uint32_t off = (8 * c < (int)rows_w) ? (uint32_t)(r * ldo + 8 * c) * 2u : kOOB;
      __builtin_amdgcn_raw_buffer_store_b128(v, r_out, off, 0, kOutAux);
    }
  } else if (vec_flags & 1) {
    for_each_out([&](int nl, int ml, uint32_t y01, uint32_t y23) {
      // N % 4 == 0 here, so the four columns are all valid or all invalid
      const uint32_t off = (nl < (int)rows_w) ? (uint32_t)(ml * ldo + nl) * 2u : kOOB;
      __builtin_amdgcn_raw_buffer_store_b64((v2u){y01, y23}, r_out, off, 0, kOutAux);
    });
  } else {
    for_each_out([&](int nl, int ml, uint32_t y01, uint32_t y23) {
      const uint32_t base = (uint32_t)(ml * ldo + nl) * 2u;
      const uint32_t y[4] = {y01 & 0xffffu, y01 >> 16, y23 & 0xffffu, y23 >> 16};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t off = (nl + r < (int)rows_w) ? base + 2u * r : kOOB;
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)y[r], r_out, off, 0, kOutAux);
      }
    });
  }
  if (a.acc_debug) {
    const __amdgpu_buffer_rsrc_t r_acc =
        make_rsrc(a.acc_debug + m0 * N + n0, (uint32_t)(((int64_t)(rows_x - 1) * N + rows_w) * 4));
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int ml = wave_m * WM + 32 * j + frag_row;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = wave_n * WN + 32 * i + 8 * q + 4 * frag_half;
          const uint32_t base = (uint32_t)(ml * N + nl) * 4u;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t off = (nl + r < (int)rows_w) ? base + 4u * r : kOOB;
            __builtin_amdgcn_raw_buffer_store_b32(acc[i][j][4 * q + r], r_acc, off, 0, 0);
          }
        }
      }
  }
}

// Epilogue of the eight-wave kernels: the wave's 32 FM x 64 sub-tile (rows
// 32 FM grp.., columns 64 wn.. of the tile), scaled in the fp32 order of the
// oracle and stored as bf16 (fp16). With 16-byte output rows it is staged in
// the wave's own 16 KiB of LDS (`region`) and written as whole 128-byte row
// segments; no other wave touches the region, so no barrier is needed.
template <bool HAS_BIAS, bool F16, int HALVES = 1, int FM = 4>
__device__ __forceinline__ void gemm_pp_epilogue(const GemmArgs& a, const v16i (&acc)[2][FM],
                                                 const float* lds_sa, const float* lds_sw,
                                                 const float* lds_b, int8_t* region, int64_t m0,
                                                 int64_t n0, uint32_t rows_x, uint32_t rows_w,
                                                 int grp, int wn, int lane, int vec_flags) {
  constexpr int FN = 2;
  const int frag_row = lane & 31, frag_half = lane >> 5;
  const int64_t N = a.N;
  const int64_t ldo = a.ldo;
  const __amdgpu_buffer_rsrc_t r_out =
      make_rsrc(a.out + m0 * ldo + n0, (uint32_t)(((int64_t)(rows_x - 1) * ldo + rows_w) * 2));
  float sa[FM];
#pragma unroll
  for (int j = 0; j < FM; ++j) sa[j] = lds_sa[32 * FM * grp + 32 * j + frag_row];
  // visit(nl, ml, y01, y23): four outputs at wave-local column nl, row ml,
  // for the row blocks jb .. jb+jn-1
  auto for_each_out = [&](auto&& visit, int jb = 0, int jn = FM) {
#pragma unroll
    for (int i = 0; i < FN; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = 32 * i + 8 * q + 4 * frag_half;
        const float4 sw4 = *reinterpret_cast<const float4*>(&lds_sw[64 * wn + nl]);
        float b4[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (HAS_BIAS) {
          const float4 bb = *reinterpret_cast<const float4*>(&lds_b[64 * wn + nl]);
          b4[0] = bb.x; b4[1] = bb.y; b4[2] = bb.z; b4[3] = bb.w;
        }
#pragma unroll
        for (int j = jb; j < jb + jn; ++j) {
          const int ml = 32 * j + frag_row;
          const v16i& c = acc[i][j];
          const float t0 = epilogue_f32<HAS_BIAS>(c[4 * q + 0], sa[j], sw4.x, b4[0]);
          const float t1 = epilogue_f32<HAS_BIAS>(c[4 * q + 1], sa[j], sw4.y, b4[1]);
          const float t2 = epilogue_f32<HAS_BIAS>(c[4 * q + 2], sa[j], sw4.z, b4[2]);
          const float t3 = epilogue_f32<HAS_BIAS>(c[4 * q + 3], sa[j], sw4.w, b4[3]);
          visit(nl, ml, pack_half2<F16>(t0, t1), pack_half2<F16>(t2, t3));
        }
      }
    }
  };
  const int row_base = 32 * FM * grp, col_base = 64 * wn;
  if (vec_flags & 4) {
    // HALVES passes over 32 FM / HALVES rows each: rows of 128 bytes in the
    // region, 16-byte chunk c of row r at chunk c ^ ((r >> 1) & 7)
    constexpr int JN = FM / HALVES, ROWS = 32 * JN;
    const int c = lane & 7;
    const bool col_ok = col_base + 8 * c < (int)rows_w;
#pragma unroll
    for (int h = 0; h < HALVES; ++h) {
      for_each_out([&](int nl, int ml, uint32_t y01, uint32_t y23) {
        const int r = ml - ROWS * h;
        *reinterpret_cast<v2u*>(region + r * 128 + 16 * ((nl >> 3) ^ ((r >> 1) & 7)) + 8 * frag_half) =
            (v2u){y01, y23};
      }, JN * h, JN);
      __builtin_amdgcn_s_waitcnt(0xc07f);    // lgkmcnt(0): the wave's LDS writes are done
#pragma unroll 4
      for (int p = 0; p < ROWS / 8; ++p) {
        const int r = 8 * p + (lane >> 3);
        const v4i v = *reinterpret_cast<const v4i*>(region + r * 128 + 16 * (c ^ ((r >> 1) & 7)));
        const uint32_t o =
            col_ok ? (uint32_t)((row_base + ROWS * h + r) * ldo + col_base + 8 * c) * 2u : kOOB;
        __builtin_amdgcn_raw_buffer_store_b128(v, r_out, o, 0, kOutAux);
      }
    }
  } else if (vec_flags & 1) {
    for_each_out([&](int nl, int ml, uint32_t y01, uint32_t y23) {
      const int n = col_base + nl, m = row_base + ml;
      const uint32_t o = (n < (int)rows_w) ? (uint32_t)(m * ldo + n) * 2u : kOOB;
      __builtin_amdgcn_raw_buffer_store_b64((v2u){y01, y23}, r_out, o, 0, kOutAux);
    });
  } else {
    for_each_out([&](int nl, int ml, uint32_t y01, uint32_t y23) {
      const int n = col_base + nl, m = row_base + ml;
      const uint32_t base = (uint32_t)(m * ldo + n) * 2u;
      const uint32_t y[4] = {y01 & 0xffffu, y01 >> 16, y23 & 0xffffu, y23 >> 16};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t o = (n + r < (int)rows_w) ? base + 2u * r : kOOB;
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)y[r], r_out, o, 0, kOutAux);
      }
    });
  }
  if (a.acc_debug) {
    const __amdgpu_buffer_rsrc_t r_acc =
        make_rsrc(a.acc_debug + m0 * N + n0, (uint32_t)(((int64_t)(rows_x - 1) * N + rows_w) * 4));
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int m = row_base + 32 * j + frag_row;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = col_base + 32 * i + 8 * q + 4 * frag_half;
          const uint32_t base = (uint32_t)(m * N + n) * 4u;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t o = (n + r < (int)rows_w) ? base + 4u * r : kOOB;
            __builtin_amdgcn_raw_buffer_store_b32(acc[i][j][4 * q + r], r_acc, o, 0, 0);
          }
        }
      }
  }
}

// 256 x 256 tiles with eight waves in two groups that take turns on the
// matrix cores ("ping-pong"). Waves w and w + 4 share a SIMD; group g = w / 4
// owns output rows 128g .. 128g+127 of the tile and wave w % 4 of the group
// owns columns 64(w % 4) .. +63, so each wave holds a 128 x 64 sub-tile
// (2 x 4 blocks of 32 x 32, 128 accumulators per lane) and two waves fit on
// a SIMD. K runs in 64-byte stages (32 KiB of panels) through a ring of four
// LDS buffers; each stage takes two phases separated by workgroup barriers:
// in one, group 0 runs its 16 MFMAs of the stage from registers while group
// 1 reads its fragments of the stage into registers; in the next, the roles
// swap. So on every SIMD one wave issues MFMAs back to back while the other
// waits on LDS reads, panel loads and barriers. The panel loads of a stage
// go out from the read phases of both groups (group 0 the W panel, group 1
// the xq panel, four 1 KiB requests per wave), three stages ahead: the
// per-CU load path (about 64 bytes per clock) carries a steady half of its
// capacity, only waves that are not issuing MFMAs wait on it, and a request
// has about five phases to land. Group 0's epilogue runs alongside group
// 1's last MFMAs.
//
// A tile is whole (FM = 4: 256 x 256) or, in the last round of an XCD's
// tiles, one of two 128-row halves (FM = 2: 128 x 256, each wave a 64 x 64
// sub-tile, eight MFMAs per 64-byte slice of K). A half runs the same loop
// on stages of two slices, so each of its phases holds sixteen MFMAs per
// wave as a whole tile's does; group 1's waves 2 and 3, whose xq rows
// (128..) the half lacks, request nothing.
template <bool HAS_BIAS, bool F16, int FM>
__device__ __forceinline__ void pp_tile(const GemmArgs& a, int64_t m0, int64_t n0, int vec_flags,
                                        int kps, int8_t* ring, float* lds_sa, float* lds_sw,
                                        float* lds_b) {
  constexpr int BM = 64 * FM, BN = 256, BK = 64, KS = BK / 32;
  constexpr int FN = 2;
  constexpr int HALF = 256 * BK;             // the W panel of a 64-byte slice: 16 KiB
  constexpr int LPW = 4;                     // requests per requesting wave per slice
  // A stage is SUB slices of 64 bytes of K, each the W panel then the xq
  // panel (SUBB bytes), in a ring of NB buffers: whole tiles one slice per
  // stage in four 32 KiB buffers (three stages in flight ahead of the one
  // being read); halves, whose xq panel is half as tall, two slices per
  // stage in three 48 KiB buffers, so that a wave runs sixteen MFMAs per
  // phase as in a whole tile rather than eight, against the same barriers
  // and the same share of fragment reads
  constexpr int SUB = FM == 4 ? 1 : 2;
  constexpr int NB = FM == 4 ? 4 : 3;
  constexpr int SUBB = HALF + BM * BK;
  constexpr int SB = SUB * SUBB;
  constexpr int KST = KS * SUB;              // MFMA k-steps per stage

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wn = wave & 3;
  const int64_t M = a.M, N = a.N, K = a.K;

  const uint32_t rows_w = (uint32_t)min<int64_t>(BN, N - n0);
  const uint32_t rows_x = (uint32_t)min<int64_t>(BM, M - m0);
  const int kend = (int)min<int64_t>(K, (int64_t)min<int64_t>((int64_t)(blockIdx.y + 1) * kps,
                                                              (K + BK - 1) / BK) * BK);
  {
    const __amdgpu_buffer_rsrc_t r_sa = make_rsrc(a.a_scale + m0, rows_x * 4u);
    const __amdgpu_buffer_rsrc_t r_sw = make_rsrc(a.w_scale + n0, rows_w * 4u);
    // threads 0..255 the row scales (zero past the tile's rows), 256.. the
    // column scales
    if (tid < 256)
      lds_sa[tid] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_sa, tid * 4, 0, 0));
    else
      lds_sw[tid - 256] =
          __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_sw, (tid - 256) * 4, 0, 0));
    if constexpr (HAS_BIAS) {
      const __amdgpu_buffer_rsrc_t r_b = make_rsrc(a.bias + n0, rows_w * 2u);
      if (tid < BN) lds_b[tid] = half_to_f32<F16>(__builtin_amdgcn_raw_buffer_load_b16(r_b, tid * 2, 0, 0));
    }
  }

  // Requests: group 0 loads the W panel, group 1 the xq panel; wave wn of a
  // group fills rows 64wn .. 64wn+63 of its panel with four 1 KiB requests
  // (16 rows x 64 B each). Row 64wn + 16u + lane/4 takes 16-byte chunk
  // lane % 4 of LDS, which holds global chunk (lane % 4) ^ ((row >> 2) & 3),
  // and (row >> 2) & 3 = (lane >> 4) & 3 for every u.
  const __amdgpu_buffer_rsrc_t rsrc = grp == 0 ? make_rsrc(a.wq + n0 * K, rows_w * (uint32_t)K)
                                                : make_rsrc(a.xq + m0 * K, rows_x * (uint32_t)K);
  const int kc = 16 * ((lane & 3) ^ ((lane >> 4) & 3));
  const uint32_t lbase = (uint32_t)(64 * wn + (lane >> 2)) * (uint32_t)K + kc;
  const uint32_t rows16 = 16u * (uint32_t)K;
  const int pan = grp * HALF + wn * (LPW * 1024);   // this wave's LDS bytes within a stage
  // in halves, group 1's waves 2 and 3 would fill xq rows 128..255, which
  // the packed stage does not have: they request nothing
  const bool requests = grp == 0 || 64 * wn < BM;
  auto issue_one = [&](int kt, int8_t* st, int u) {
    if (!requests) return;
    const uint32_t k0 = (uint32_t)kt * BK;
    uint32_t b = lbase;
    asm volatile("" : "+v"(b));
    const uint32_t keep = (uint32_t)((kc - (kend - (int)k0)) >> 31);
    const uint32_t o = ((b + (uint32_t)u * rows16 + k0) & keep) | (kOOB & ~keep);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, st + pan + u * 1024, 16, o, 0, 0, 0);
  };

  v16i acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v16i{};

  // fragment address of k-step ks: row frag_row, chunk 2ks + frag_half under
  // the swizzle c ^ ((row >> 2) & 3), i.e. fb ^ (32 ks)
  const int frag_row = lane & 31, frag_half = lane >> 5;
  const int fb = frag_row * BK + 16 * (frag_half ^ ((frag_row >> 2) & 3));
  const int w_row0 = 64 * wn * BK, x_row0 = HALF + 32 * FM * grp * BK;

  v4i fw[KST][FN], fx[KST][FM];
  auto read_frags = [&](const int8_t* st) {
    int f = fb;
    asm volatile("" : "+v"(f));
#pragma unroll
    for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int8_t* p = st + sub * SUBB + (f ^ (32 * ks));
#pragma unroll
      for (int i = 0; i < FN; ++i)
        fw[sub * KS + ks][i] = *reinterpret_cast<const v4i*>(p + w_row0 + 32 * BK * i);
#pragma unroll
      for (int j = 0; j < FM; ++j)
        fx[sub * KS + ks][j] = *reinterpret_cast<const v4i*>(p + x_row0 + 32 * BK * j);
    }
  };
  // MFMAs of one stage, back to back at raised priority (a VMEM request in
  // the MFMA wave's stream would stall it behind the per-CU load queue)
  auto compute = [&]() {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < KST; ++ks)
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fw[ks][i], fx[ks][j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
  };

  // stages of SUB slices (a K slice of the tile's range that lies past
  // kend reads out of bounds: zeros, which add nothing); this kernel never
  // splits K, so the range starts at slice 0
  const int nk_all = (int)((K + BK - 1) / BK);
  const int kb = 0;
  const int ke = (nk_all + SUB - 1) / SUB;
  // a stage's requests: SUB x LPW per requesting wave
  auto issue_stage = [&](int t, int8_t* st) {
#pragma unroll
    for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
      for (int u = 0; u < LPW; ++u) issue_one(SUB * t + sub, st + sub * SUBB, u);
  };

  // Every wave runs the same loop body, read(t) | barrier | compute(t) |
  // barrier, with group 1 one phase behind group 0 (an extra barrier at the
  // start; group 1 skips the barrier after its last compute), so stage t is
  // read in phases 2t (group 0) and 2t+1 (group 1). Right after its
  // fragment reads of stage t, each wave requests its panel's part of stage
  // t+NB-1 into the buffer that stage t-1 left at the end of phase 2t-1
  // (group 0 the W panel in phase 2t, group 1 the xq panel in phase 2t+1),
  // so the loads go out from the waves that are not issuing MFMAs. Every
  // read phase sends exactly 4 SUB requests per requesting wave (past the
  // last stage they read out of bounds: no memory traffic, zeros into a
  // buffer no stage reads), so both waits are the constant
  // vmcnt((NB-2)*4*SUB) = vmcnt(8): a wave's requests of stage t+1 have
  // landed by the barrier that ends phase 2t+1.
  auto buf = [&](int i) { return ring + i * SB; };
#pragma unroll
  for (int i = 0; i < NB - 1; ++i) issue_stage(kb + i, buf(i));
  wait_vmcnt_lgkm0<(NB - 2) * SUB * LPW>();
  stage_barrier();
  if (grp == 1) stage_barrier();
  auto body = [&](int s, int8_t* st, int8_t* nxt) {
    read_frags(st);
    issue_stage(s + NB - 1, nxt);
    wait_vmcnt_lgkm0<(NB - 2) * SUB * LPW>();
    stage_barrier();
    compute();
    wait_vmcnt<(NB - 2) * SUB * LPW>();
    if (grp == 0 || s + 1 < ke) stage_barrier();
  };
  // (unrolled by NB, so that every access names its buffer)
  int s = kb;
  for (; s + NB - 1 < ke; s += NB) {
#pragma unroll
    for (int i = 0; i < NB; ++i) body(s + i, buf(i), buf((i + NB - 1) % NB));
  }
#pragma unroll
  for (int i = 0; i < NB - 1; ++i)
    if (s + i < ke) body(s + i, buf(i), buf((i + NB - 1) % NB));
  // every request of this wave (the last ones out of bounds) has written LDS
  wait_vmcnt<0>();
  __builtin_amdgcn_sched_barrier(0);

  // Staging (8 KiB per wave for whole tiles, half the sub-tile at a time; 4
  // KiB for halves), in a buffer that no request still in flight targets.
  // With n = ke - kb stages, the last requests (of stages n .. n+NB-2,
  // relative to kb) target buffers n .. n+NB-2 mod NB, never (n-1) mod NB,
  // and no stage is read after group 0's last barrier: group 0 stages in
  // buffer (n-1) mod NB. Group 1 stages after draining its own requests and
  // group 0's last barrier, by which group 0's requests of stage n (buffer
  // n mod NB) have landed: buffer n mod NB.
  const int n_st = ke - kb;
  const int pick = grp == 0 ? ((n_st - 1) % NB + NB) % NB : (n_st % NB + NB) % NB;
  constexpr int REGION = FM == 4 ? 8192 : 4096;
  gemm_pp_epilogue<HAS_BIAS, F16, 2, FM>(a, acc, lds_sa, lds_sw, lds_b, buf(pick) + wn * REGION, m0,
                                         n0, rows_x, rows_w, grp, wn, lane, vec_flags);
}

// cpx: compute units per XCD when tiles may be split into halves (0: never).
template <bool HAS_BIAS, bool F16>
__global__ __launch_bounds__(512) void gemm_pp_kernel(GemmArgs a, int tiles_m, int tiles_n,
                                                        int vec_flags, int kps, int cpx) {
  // the stage ring: 4 x 32 KiB for whole tiles, 3 x 48 KiB for halves
  __shared__ __attribute__((aligned(1024))) int8_t ring[3 * 48 * 1024];
  __shared__ __attribute__((aligned(16))) float lds_sa[256];
  __shared__ __attribute__((aligned(16))) float lds_sw[256];
  __shared__ __attribute__((aligned(16))) float lds_b[HAS_BIAS ? 256 : 1];
  int tm, tn, half;
  if (!tile_coords_halves(tiles_m, tiles_n, cpx, tm, tn, half)) return;
  if (half < 0) {
    pp_tile<HAS_BIAS, F16, 4>(a, (int64_t)tm * 256, (int64_t)tn * 256, vec_flags, kps, ring, lds_sa,
                              lds_sw, lds_b);
  } else {
    const int64_t m0 = (int64_t)tm * 256 + 128 * half;
    if (m0 < a.M)
      pp_tile<HAS_BIAS, F16, 2>(a, m0, (int64_t)tn * 256, vec_flags, kps, ring, lds_sa, lds_sw, lds_b);
  }
}

// Split K, second step: out[m, n..n+7] = epilogue(sum over the slices of
// the int32 partial sums), in the GEMM epilogue's fp32 order; one thread per
// eight columns (N % 8 == 0, out rows 16-byte aligned). The int32 sum is
// exact whatever the split, so the result is bit-identical to the one-pass
// GEMM.
template <bool HAS_BIAS, bool F16>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs a, int splits) {
  const int64_t n8 = a.N >> 3;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= a.M * n8) return;
  const int64_t m = g / n8, n = (g - m * n8) * 8;
  const int64_t slice = a.M * a.N;
  const int32_t* p = a.partial + m * a.N + n;
  int acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int sidx = 0; sidx < splits; ++sidx) {
    const int4 lo = *reinterpret_cast<const int4*>(p + sidx * slice);
    const int4 hi = *reinterpret_cast<const int4*>(p + sidx * slice + 4);
    acc[0] += lo.x; acc[1] += lo.y; acc[2] += lo.z; acc[3] += lo.w;
    acc[4] += hi.x; acc[5] += hi.y; acc[6] += hi.z; acc[7] += hi.w;
  }
  if (a.acc_debug) {
    int32_t* d = a.acc_debug + m * a.N + n;
    *reinterpret_cast<int4*>(d) = make_int4(acc[0], acc[1], acc[2], acc[3]);
    *reinterpret_cast<int4*>(d + 4) = make_int4(acc[4], acc[5], acc[6], acc[7]);
  }
  const float sa = a.a_scale[m];
  uint32_t y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float b0 = HAS_BIAS ? half_to_f32<F16>(a.bias[n + 2 * i]) : 0.f;
    const float b1 = HAS_BIAS ? half_to_f32<F16>(a.bias[n + 2 * i + 1]) : 0.f;
    const float t0 = epilogue_f32<HAS_BIAS>(acc[2 * i], sa, a.w_scale[n + 2 * i], b0);
    const float t1 = epilogue_f32<HAS_BIAS>(acc[2 * i + 1], sa, a.w_scale[n + 2 * i + 1], b1);
    y[i] = pack_half2<F16>(t0, t1);
  }
  *reinterpret_cast<uint4*>(a.out + m * a.ldo + n) = make_uint4(y[0], y[1], y[2], y[3]);
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int BK, int S>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t stream, int splits = 1, int kps = 0) {
  const int64_t tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
  const int64_t tiles = tiles_m * tiles_n;
  const int vec_flags = epilogue_vec_flags(a);
  if (splits == 1) kps = (int)((a.K + BK - 1) / BK);
  dim3 grid((unsigned)tiles, (unsigned)splits), block(64 * WAVES_M * WAVES_N);
  if constexpr (BM == BN) {
    if (splits > 1) {         // partial sums only: bias and output type do not matter
      hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, WAVES_M, WAVES_N, BK, S, false, false, true>),
                         grid, block, 0, stream, a, (int)tiles_m, (int)tiles_n, vec_flags, kps);
      return hipGetLastError();
    }
  }
#define W8A8_GEMM(B, H)                                                                    \
  hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, WAVES_M, WAVES_N, BK, S, B, H>), grid, block, 0, \
                     stream, a, (int)tiles_m, (int)tiles_n, vec_flags, kps)
  if (a.f16) {
    if (a.bias) W8A8_GEMM(true, true);
    else W8A8_GEMM(false, true);
  } else {
    if (a.bias) W8A8_GEMM(true, false);
    else W8A8_GEMM(false, false);
  }
#undef W8A8_GEMM
  return hipGetLastError();
}

// Blocks of the ping-pong kernel for T tiles, with tiles split into halves
// where tile_coords_halves does so (cpx compute units per XCD): 8 times the
// largest number of pieces of one XCD.
int64_t pp_blocks(int64_t T, int cpx) {
  int64_t most = 0;
  for (int x = 0; x < 8; ++x) {
    const int tx = (int)((T >> 3) + (x < (T & 7) ? 1 : 0));
    const int whole = pp_whole_tiles(tx, cpx);
    most = std::max<int64_t>(most, whole + 2 * (tx - whole));
  }
  return 8 * most;
}

// 256 x 256 tiles: the eight-wave ping-pong kernel. The last round of each
// XCD's tiles runs as 128-row halves when it is at most half full
// (4352 x 3072 x 9216, 612 tiles: 76 or 77 per XCD of 32 compute units,
// so 12 or 13 tiles in the last round become 24 or 26 halves), and every
// tile does when all of them fill at most half of the compute units
// (512 x 4096 x 12288: 96 tiles, 192 halves, 46.7 -> 42.1 us per product;
// K split in two with a reduction kernel took 51 us).
hipError_t launch_pp(const GemmArgs& a, hipStream_t stream) {
  constexpr int T = 256, BK = 64;
  const int64_t tiles_m = (a.M + T - 1) / T, tiles_n = (a.N + T - 1) / T;
  const int vec_flags = epilogue_vec_flags(a);
  const int kps = (int)((a.K + BK - 1) / BK);
  const int cus = device_cus();
  const int cpx = cus % 8 == 0 ? cus / 8 : 0;
  const dim3 grid((unsigned)pp_blocks(tiles_m * tiles_n, cpx)), block(512);
#define W8A8_PP(B, H)                                                                    \
  hipLaunchKernelGGL((gemm_pp_kernel<B, H>), grid, block, 0, stream, a, (int)tiles_m, \
                     (int)tiles_n, vec_flags, kps, cpx)
  if (a.f16) {
    if (a.bias) W8A8_PP(true, true);
    else W8A8_PP(false, true);
  } else {
    if (a.bias) W8A8_PP(true, false);
    else W8A8_PP(false, false);
  }
#undef W8A8_PP
  return hipGetLastError();
}

// Split-K plan for a shape: K is split in two (with K of at least 8 stages)
// when 128x128 tiles fill at most one round of the compute units (two 64 KiB
// 128x128 workgroups share a CU, so the split pairs overlap). Measured:
// 512x4096x4096 41 -> 31 us, 1024x4096x4096 49 -> 40 us, 512x4096x8192
// 49 -> 40 us (128 tiles). More splits lose: each adds a slice of int32
// partial sums, written and read back, except on 64x64 tiles, whose skinny
// products wait on the weight stream: up to four pieces there
// (64x3072x18432: 34 -> 30 us in three, 64x4096x4096: 34 -> 19 us in four).
// 256x256 tiles that fill at most half of the compute units run as halves
// instead (launch_pp), with no partial sums. splits = 1: no split.
struct SplitPlan {
  int splits = 1;
  int kps = 0;              // K stages per split
  int tile = 128;           // BM = BN of the split GEMM (128 or 64)
};

SplitPlan split_plan(int64_t M, int64_t N, int64_t K) {
  SplitPlan p;
  if ((N & 7) != 0 || N > (int64_t(1) << 21)) return p;
  int bm, bn;
  gemm_pick_tile(M, N, K, &bm, &bn);
  if (bm == 64) {
    // 64x64 tiles (M < 128), latency-bound on the weight stream: up to four
    // K pieces, so that about four 16 KiB workgroups stream per CU
    const int64_t tiles = ((M + 63) / 64) * ((N + 63) / 64);
    const int64_t nk = (K + 63) / 64;
    const int64_t s = std::min<int64_t>(4, (4 * (int64_t)device_cus()) / tiles);
    if (s < 2 || nk < 8 * s) return p;
    p.tile = 64;
    p.kps = (int)((nk + s - 1) / s);
    p.splits = (int)((nk + p.kps - 1) / p.kps);
    return p;
  }
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  const int64_t nk = (K + 127) / 128;
  if (bm != 128 || tiles > device_cus() || nk < 8) return p;
  p.tile = bm;
  p.kps = (int)((nk + 1) / 2);
  p.splits = (int)((nk + p.kps - 1) / p.kps);
  return p;
}

}  // namespace

// M >= 128: 256x256 tiles, unless 128x128 tiles finish first: a 128x128 tile takes
// about 0.6 of a 256x256 tile's time on the same K (measured on 512x4096x4096:
// 40 us in one round of 128 small tiles against 57 us for 32 large ones; on
// 512x4096x12288, 61 us in two rounds against 58 us in one), so the small
// tiles win only when their rounds over the compute units, times 0.6, are
// fewer than the large tiles' rounds.
void gemm_pick_tile(int64_t M, int64_t N, int64_t K, int* bm, int* bn) {
  (void)K;
  const int64_t cus = device_cus();
  if (M <= 64) { *bm = 64; *bn = 64; return; }
  if (M < 128) {
    // one 128-row tile reads each weight panel once where two 64-row tiles
    // read it twice; it pays when two K pieces of such tiles fill the chip
    // (100x3072x18432: 42 -> 32 us), not on narrow outputs, where 64x64
    // tiles split four ways keep more workgroups streaming (120x12288x3072:
    // 35 against 55 us)
    if (2 * ((N + 127) / 128) >= cus) { *bm = 128; *bn = 128; return; }
    *bm = 64; *bn = 64;
    return;
  }
  const int64_t r256 = (((M + 255) / 256) * ((N + 255) / 256) + cus - 1) / cus;
  const int64_t r128 = (((M + 127) / 128) * ((N + 127) / 128) + cus - 1) / cus;
  if (M >= 512 && N >= 512 && 5 * r256 <= 3 * r128) { *bm = 256; *bn = 256; return; }
  *bm = 128; *bn = 128;
}

size_t gemm_partial_bytes(int64_t M, int64_t N, int64_t K) {
  const SplitPlan p = split_plan(M, N, K);
  return p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)N * sizeof(int32_t) : 0;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  if (a.partial) {
    // split K only where the output takes the reduction's 16-byte stores
    const int vf = epilogue_vec_flags(a);
    const SplitPlan p = split_plan(a.M, a.N, a.K);
    if (p.splits > 1 && (vf & 4) && (!a.acc_debug || (vf & 2))) {
      if (hipError_t e = p.tile == 128 ? launch_cfg<128, 128, 2, 2, 128, 2>(a, stream, p.splits, p.kps)
                                       : launch_cfg<64, 64, 2, 2, 64, 2>(a, stream, p.splits, p.kps);
          e != hipSuccess)
        return e;
      const int64_t groups = a.M * (a.N >> 3);
      const dim3 grid((unsigned)((groups + 255) / 256)), block(256);
#define W8A8_RED(B, H) \
      hipLaunchKernelGGL((splitk_reduce_kernel<B, H>), grid, block, 0, stream, a, p.splits)
      if (a.f16) {
        if (a.bias) W8A8_RED(true, true);
        else W8A8_RED(false, true);
      } else {
        if (a.bias) W8A8_RED(true, false);
        else W8A8_RED(false, false);
      }
#undef W8A8_RED
      return hipGetLastError();
    }
  }
  GemmArgs one = a;
  one.partial = nullptr;
  int bm, bn;
  gemm_pick_tile(a.M, a.N, a.K, &bm, &bn);
  if (bm == 256) return launch_pp(one, stream);
  if (bm == 128) return launch_cfg<128, 128, 2, 2, 128, 2>(one, stream);
  return launch_cfg<64, 64, 2, 2, 64, 2>(one, stream);
}

}  // namespace w8a8
