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
//   the accumulator lane layout gives each lane four consecutive output
//   columns n of one output row m: the epilogue stores 8 bytes of bf16 per
//   lane and per 16x16 block.
// * Workgroup of 256 threads (4 waves) computes a BM x BN tile; each wave a
//   WM x WN sub-tile held in registers as (WN/16)*(WM/16) MFMA blocks.
// * K advances in stages of 128 bytes. Each stage of the W and xq panels is
//   loaded from global memory with 16-byte loads (8 lanes per 128-byte row
//   segment), kept in registers while the previous stage is multiplied, then
//   written to the other half of a double-buffered LDS panel: one barrier per
//   stage. 16-byte chunks are XOR-swizzled by (row & 7) so the ds_read_b128
//   of 8 consecutive rows hit 8 distinct 16-byte bank groups.
// * Out-of-range rows and K chunks load as zeros, so ragged M, N and K
//   (K % 16 == 0) tails need no special path.
#include "w8a8_device.h"
#include "w8a8_kernels.h"

namespace w8a8 {

namespace {

constexpr int kBK = 128;  // bytes of K per LDS stage (two MFMA k-steps of 64)

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

template <int BM, int BN, int WAVES_M, int WAVES_N, bool HAS_BIAS>
__global__ __launch_bounds__(256) void gemm_i8_kernel(GemmArgs a, int tiles_m, int vec_flags) {
  static_assert(WAVES_M * WAVES_N == 4, "four waves per workgroup");
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FM = WM / 16, FN = WN / 16;
  static_assert(FM >= 1 && FN >= 1 && BM % 32 == 0 && BN % 32 == 0, "tile shape");
  constexpr int PA = BN / 32, PB = BM / 32;  // 16-byte loads per thread per stage

  __shared__ __attribute__((aligned(16))) int8_t lds_w[2][BN * kBK];
  __shared__ __attribute__((aligned(16))) int8_t lds_x[2][BM * kBK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_m = wave % WAVES_M, wave_n = wave / WAVES_M;

  const int tile = blockIdx.x;
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t M = a.M, N = a.N, K = a.K;

  // global -> register staging: thread covers row (tid/8 + 32p), chunk tid%8
  const int ld_row = tid >> 3, ld_chunk = tid & 7;
  uint4 rw[PA], rx[PB];

  auto load_stage = [&](int64_t k0) {
    const int64_t kc = k0 + 16 * ld_chunk;
    const bool kval = kc < K;
#pragma unroll
    for (int p = 0; p < PA; ++p) {
      const int64_t n = n0 + ld_row + 32 * p;
      rw[p] = (kval && n < N) ? *reinterpret_cast<const uint4*>(a.wq + n * K + kc)
                              : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      const int64_t m = m0 + ld_row + 32 * p;
      rx[p] = (kval && m < M) ? *reinterpret_cast<const uint4*>(a.xq + m * K + kc)
                              : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PA; ++p) {
      const int row = ld_row + 32 * p;
      *reinterpret_cast<uint4*>(&lds_w[buf][row * kBK + 16 * swz(row, ld_chunk)]) = rw[p];
    }
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      const int row = ld_row + 32 * p;
      *reinterpret_cast<uint4*>(&lds_x[buf][row * kBK + 16 * swz(row, ld_chunk)]) = rx[p];
    }
  };

  v4i acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  const int frag_row = lane & 15;   // row within a 16-row block
  const int frag_grp = lane >> 4;   // which 16-byte group of the 64-byte k-step

  const int nk = (int)((K + kBK - 1) / kBK);
  load_stage(0);
  store_stage(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_stage((int64_t)(kt + 1) * kBK);
#pragma unroll
    for (int s = 0; s < kBK / 64; ++s) {
      v4i fw[FN], fx[FM];
      const int chunk = 4 * s + frag_grp;
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int row = wave_n * WN + 16 * i + frag_row;
        fw[i] = *reinterpret_cast<const v4i*>(&lds_w[cur][row * kBK + 16 * swz(row, chunk)]);
      }
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int row = wave_m * WM + 16 * j + frag_row;
        fx[j] = *reinterpret_cast<const v4i*>(&lds_x[cur][row * kBK + 16 * swz(row, chunk)]);
      }
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fw[i], fx[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_stage(cur ^ 1);
    __syncthreads();
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

template <int BM, int BN, int WM_, int WN_>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t stream) {
  const int64_t tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
  const int64_t tiles = tiles_m * tiles_n;
  const int vec_flags = epilogue_vec_flags(a);
  dim3 grid((unsigned)tiles), block(256);
  if (a.bias)
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, WM_, WN_, true>), grid, block, 0, stream, a,
                       (int)tiles_m, vec_flags);
  else
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, WM_, WN_, false>), grid, block, 0, stream, a,
                       (int)tiles_m, vec_flags);
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
  if (bm == 256) return launch_cfg<256, 256, 2, 2>(a, stream);
  if (bm == 128) return launch_cfg<128, 128, 2, 2>(a, stream);
  if (bm == 64) return launch_cfg<64, 64, 2, 2>(a, stream);
  return launch_cfg<32, 64, 1, 4>(a, stream);
}

}  // namespace w8a8
