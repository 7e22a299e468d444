// int8 x int8 -> int32 MFMA GEMM with the fused W8A8 scale epilogue (gfx950).
//
// acc[m,n] = sum_k xq[m,k] * wq[n,k]   (int32, exact; unsloth commit log of
//   test_diffusion_transformer_quant.py: int8 products, int32 accumulation)
// y[m,n]   = bf16(((fl32(acc) * a_scale[m]) * w_scale[n]) + bias[n])
//   (Issue 5 probe, "Round two": the int8 scaled-MM result carries act_scale
//    and the fp32 per-channel weight scale)
//
// Design (CDNA4):
// * v_mfma_i32_16x16x64_i8. The MFMA "A" operand is a 16-row block of W and
//   the "B" operand a 16-row block of xq (both K-contiguous, no transpose), so
//   each lane's accumulators are four consecutive output columns n of one
//   output row m: the epilogue stores 8 bytes of bf16 per lane and block.
// * A workgroup of NW waves computes a BM x BN tile, each wave a WM x WN
//   sub-tile held as (WN/16)*(WM/16) MFMA blocks.
// * Panels stream global -> LDS with buffer_load_dwordx4 ... lds (no VGPR
//   staging, no ds_write). One wave-instruction fills 1 KiB of LDS linearly
//   by lane; each lane picks the global 16-byte chunk that belongs at its LDS
//   slot, which realises an XOR swizzle of the 16-byte chunks so that the
//   ds_read_b128 of 8 consecutive rows hit distinct banks.
// * An S-stage LDS ring: loads for stage kt+S-1 are issued right after the
//   barrier of stage kt; one barrier per stage; the wait before it only
//   counts this stage's loads (exact s_waitcnt vmcnt).
// * Out-of-range rows read as zeros through the buffer descriptor's bound;
//   K-tail chunks are sent out of bounds, so ragged M, N and K need no branch.
// * Tile order: every XCD (workgroups are dealt round-robin over the 8 XCDs)
//   takes a contiguous range of a grouped tile order, so the tiles that run
//   together on one XCD share W and xq panels in that XCD's L2.
#include "w8a8_device.h"
#include "w8a8_kernels.h"

namespace w8a8 {

namespace {

constexpr uint32_t kOOB = 0x7ffffff0u;   // an offset past every descriptor bound

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

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

// Swizzled position of logical 16-byte chunk c of LDS row `row`.
template <int BK>
__device__ __forceinline__ int swz(int row, int c) {
  if constexpr (BK == 128) return c ^ (row & 7);
  else return c ^ ((row >> 1) & 3);
}

// (tm, tn) of the workgroup: XCD-contiguous ranges of a grouped order.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int t = xcd * (T >> 3) + min(xcd, T & 7) + local;
  constexpr int G = 8;                         // m-tiles per group
  const int group = t / (G * tiles_n);
  const int first_m = group * G;
  const int gm = min(G, tiles_m - first_m);
  const int r = t - group * G * tiles_n;
  tm = first_m + r % gm;
  tn = r / gm;
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int BK, int S, bool HAS_BIAS>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_i8_kernel(GemmArgs a, int tiles_m,
                                                                         int tiles_n, int vec_flags) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int CH = BK / 16;               // 16-byte chunks per LDS row
  constexpr int RPI = 1024 / BK;            // LDS rows per wave-instruction
  constexpr int JW = BN * BK / 1024, JX = BM * BK / 1024;
  static_assert(JW % NW == 0 && JX % NW == 0, "panel loads must split evenly over waves");
  constexpr int LW = JW / NW, LX = JX / NW, LPS = LW + LX;
  static_assert(LPS * (S - 1) < 64, "vmcnt range");
  constexpr int STAGE = (BM + BN) * BK;     // bytes per LDS stage (W rows then xq rows)

  __shared__ __attribute__((aligned(1024))) int8_t lds[S * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_m = wave % WAVES_M, wave_n = wave / WAVES_M;
  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t M = a.M, N = a.N, K = a.K;

  const uint32_t rows_w = (uint32_t)min<int64_t>(BN, N - n0);
  const uint32_t rows_x = (uint32_t)min<int64_t>(BM, M - m0);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.wq + n0 * K, rows_w * (uint32_t)K);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.xq + m0 * K, rows_x * (uint32_t)K);

  // Per-lane source of each of this wave's load instructions (stage-relative).
  uint32_t off_w[LW], off_x[LX];
  int kc_w[LW], kc_x[LX];
#pragma unroll
  for (int j = 0; j < LW; ++j) {
    const int row = (wave * LW + j) * RPI + lane / CH;
    const int c = swz<BK>(row, lane % CH);
    off_w[j] = (uint32_t)row * (uint32_t)K + 16u * c;
    kc_w[j] = 16 * c;
  }
#pragma unroll
  for (int j = 0; j < LX; ++j) {
    const int row = (wave * LX + j) * RPI + lane / CH;
    const int c = swz<BK>(row, lane % CH);
    off_x[j] = (uint32_t)row * (uint32_t)K + 16u * c;
    kc_x[j] = 16 * c;
  }

  auto issue = [&](int kt) {
    int8_t* st = lds + (kt % S) * STAGE;
    const int k0 = kt * BK;
#pragma unroll
    for (int j = 0; j < LW; ++j) {
      const uint32_t off = (k0 + kc_w[j] < K) ? off_w[j] + k0 : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, st + (wave * LW + j) * 1024, 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < LX; ++j) {
      const uint32_t off = (k0 + kc_x[j] < K) ? off_x[j] + k0 : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, st + BN * BK + (wave * LX + j) * 1024, 16, off,
                                               0, 0, 0);
    }
  };

  v4i acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  const int frag_row = lane & 15, frag_grp = lane >> 4;
  const int nk = (int)((K + BK - 1) / BK);

#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue(s);

  for (int kt = 0; kt < nk; ++kt) {
    if (kt + S - 2 < nk) wait_vmcnt_lgkm0<LPS * (S - 2)>();
    else wait_vmcnt_lgkm0<0>();
    stage_barrier();
    if (kt + S - 1 < nk) issue(kt + S - 1);
    const int8_t* sw = lds + (kt % S) * STAGE;
    const int8_t* sx = sw + BN * BK;
#pragma unroll
    for (int s = 0; s < BK / 64; ++s) {
      v4i fw[FN], fx[FM];
      const int c = 4 * s + frag_grp;
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int row = wave_n * WN + 16 * i + frag_row;
        fw[i] = *reinterpret_cast<const v4i*>(sw + row * BK + 16 * swz<BK>(row, c));
      }
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int row = wave_m * WM + 16 * j + frag_row;
        fx[j] = *reinterpret_cast<const v4i*>(sx + row * BK + 16 * swz<BK>(row, c));
      }
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fw[i], fx[j], acc[i][j], 0, 0, 0);
    }
  }

  // Epilogue. Lane holds D[n = nb + 4*(lane/16) + r][m = mb + lane%16], r=0..3.
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int64_t m = m0 + wave_m * WM + 16 * j + (lane & 15);
    if (m >= M) continue;
    const float sa = a.a_scale[m];
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int64_t n = n0 + wave_n * WN + 16 * i + 4 * (lane >> 4);
      if (n >= N) continue;
      const v4i c = acc[i][j];
      if (n + 3 < N) {
        const float sw0 = a.w_scale[n], sw1 = a.w_scale[n + 1];
        const float sw2 = a.w_scale[n + 2], sw3 = a.w_scale[n + 3];
        float b[4] = {0.f, 0.f, 0.f, 0.f};
        if (HAS_BIAS) {
#pragma unroll
          for (int r = 0; r < 4; ++r) b[r] = bf16_to_f32(a.bias[n + r]);
        }
        const uint32_t y0 = f32_to_bf16_rne(epilogue_f32<HAS_BIAS>(c[0], sa, sw0, b[0]));
        const uint32_t y1 = f32_to_bf16_rne(epilogue_f32<HAS_BIAS>(c[1], sa, sw1, b[1]));
        const uint32_t y2 = f32_to_bf16_rne(epilogue_f32<HAS_BIAS>(c[2], sa, sw2, b[2]));
        const uint32_t y3 = f32_to_bf16_rne(epilogue_f32<HAS_BIAS>(c[3], sa, sw3, b[3]));
        uint16_t* o = a.out + m * a.ldo + n;
        if (vec_flags & 1) {
          *reinterpret_cast<uint2*>(o) = make_uint2(y0 | (y1 << 16), y2 | (y3 << 16));
        } else {
          o[0] = (uint16_t)y0; o[1] = (uint16_t)y1; o[2] = (uint16_t)y2; o[3] = (uint16_t)y3;
        }
        if (a.acc_debug) {
          int32_t* d = a.acc_debug + m * N + n;
          if (vec_flags & 2) {
            *reinterpret_cast<int4*>(d) = make_int4(c[0], c[1], c[2], c[3]);
          } else {
            d[0] = c[0]; d[1] = c[1]; d[2] = c[2]; d[3] = c[3];
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (n + r < N) {
            const float b = HAS_BIAS ? bf16_to_f32(a.bias[n + r]) : 0.f;
            const float t = epilogue_f32<HAS_BIAS>(c[r], sa, a.w_scale[n + r], b);
            a.out[m * a.ldo + n + r] = (uint16_t)f32_to_bf16_rne(t);
            if (a.acc_debug) a.acc_debug[m * N + n + r] = c[r];
          }
        }
      }
    }
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int BK, int S>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t stream) {
  const int64_t tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
  const int64_t tiles = tiles_m * tiles_n;
  const int vec_flags = epilogue_vec_flags(a);
  dim3 grid((unsigned)tiles), block(64 * WAVES_M * WAVES_N);
  if (a.bias)
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, WAVES_M, WAVES_N, BK, S, true>), grid, block, 0,
                       stream, a, (int)tiles_m, (int)tiles_n, vec_flags);
  else
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, WAVES_M, WAVES_N, BK, S, false>), grid, block, 0,
                       stream, a, (int)tiles_m, (int)tiles_n, vec_flags);
  return hipGetLastError();
}

}  // namespace

void gemm_pick_tile(int64_t M, int64_t N, int64_t K, int* bm, int* bn) {
  (void)K;
  if (M >= 512 && N >= 512) { *bm = 256; *bn = 256; return; }
  if (M >= 128) { *bm = 128; *bn = 128; return; }
  if (M > 32) { *bm = 64; *bn = 64; return; }
  *bm = 32; *bn = 64;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  int bm, bn;
  gemm_pick_tile(a.M, a.N, a.K, &bm, &bn);
  if (bm == 256) return launch_cfg<256, 256, 2, 2, 64, 4>(a, stream);
  if (bm == 128) return launch_cfg<128, 128, 2, 2, 64, 4>(a, stream);
  if (bm == 64) return launch_cfg<64, 64, 2, 2, 64, 4>(a, stream);
  return launch_cfg<32, 64, 1, 4, 128, 4>(a, stream);
}

}  // namespace w8a8
