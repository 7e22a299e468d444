// Small-M W8A8 linear (M <= 32): fused, weight-streaming kernels (gfx950).
// Activations, bias and output are bf16, or all fp16 (same arithmetic).
//
// The int8 matmul route of the prior art requires more than 16 activation
// rows, so the AdaLN modulation and conditioning projections, which run at
// M = batch = 1, were kept out of int8 (unsloth commit log of
// test_diffusion_transformer_quant.py). Here they are served by kernels
// whose cost is streaming the int8 weight once from HBM.
//
// One wide workgroup per CU when the weight allows (see row_groups.h); its
// "weight waves" own 8 weight rows each over the whole K, read in 128-byte
// windows, and every CU quantises all M activation rows (per-row amax, scale
// = amax/127, exact half-to-even rounding) into LDS as int8 [M][K];
// workgroup 0 also hands xq and a_scale to the caller. Two kernels differ in
// who quantises and when the weight is requested:
//  * row modes (K <= 3072, rows held in registers): every wave quantises up
//    to three rows (M <= 3W) and is also a weight wave (or, beyond the
//    weight's row groups, a helper). A wave requests its rows before any
//    weight window (a wave's loads complete in order, so rows requested
//    behind its windows would arrive last), then its first kD0 windows, waits
//    for its rows, quantises them, and only then requests its remaining
//    windows: a wave that requests every window first stalls at issue once
//    the CU's request queue is full, and its rows wait behind the stall
//    (measured at M = 16 on 3072 -> 18432: 16.1 us with every window first,
//    15.0 us with kD0 = 8). All of a CU's rows are in flight at once, one
//    load latency for the lot.
//  * split roles: H "quantiser waves" own no weight rows. Before any weight
//    is requested (a workgroup barrier orders them) they request all their
//    rows into LDS as bf16 by LDS-DMA (buffer_load ... lds) and quantise them
//    in place; where the LDS slots do not fit, they hold two rows in
//    registers at a time (K <= 3072) or read longer rows twice from memory.
//    The weight waves request their windows at once and wait at a
//    second barrier; with one token block and more windows than a wave
//    keeps in flight, two weight waves share a row group, each streaming
//    half of K, and their int32 sums meet in LDS. Faster for long rows
//    (whose row-mode form quantised everything before the first weight
//    request) and where each quantiser has at most three rows (small N
//    leaves room for up to twelve quantisers); slower where four
//    quantisers carry many rows, whose VALU
//    time then serialises (17 / 32 rows on 3072 -> 18432: 15.5 / 21.5 us
//    in row modes, 20.0 / 27.5 us split).
// Streaming, in both: a weight wave requests up to 24 windows at once (one
// buffer_load_dwordx4 per window: lane l reads row l%8, 16-byte chunk l/8,
// so every instruction fetches 8 whole 128-byte lines). Each window is one
// v_mfma_i32_16x16x64_i8 per block of 8 tokens (up to 4 blocks, 3 for
// M <= 24). The loaded layout is the MFMA "A" layout if A-row i is read as
// weight row i%8 at chunk parity i/8: lane l holds A[l%16][k-group l/16] =
// row l%8, chunk 2*(l/16) + (l/8)%2 = l/8. The "B" operand is built the same
// way from LDS: column j = token j%8 at chunk parity j/8. Then
// D[n][t] + D[n+8][t+8] is the dot product of weight row n and token t over
// the window (the other two blocks of D are unused). Longer rows refill the
// windows as they are consumed, through a buffer descriptor bounded at the
// wave's rows, so rows past N and chunks past K read as zero, branch-free.
// The epilogue is the GEMM's, in the same fp32 order, so a row gives
// bit-identical results on either path.
#include "row_groups.h"
#include "w8a8_device.h"
#include "w8a8_kernels.h"

namespace w8a8 {

namespace {

constexpr int kQ = 6;                    // 16-byte chunks per lane of a row held in registers
constexpr int64_t kRegRowK = 64 * 8 * kQ;  // K up to this: whole rows fit in a wave's registers

// Row-mode kernel: windows in flight per wave (a K = 3072 row group whole),
// and of these, the ones requested before the wave's rows are quantised.
constexpr int kRowD = 24;
constexpr int kD0 = 8;

// Row modes: ONE_ROW: M <= W (a wave quantises at most one activation row,
// overlapped with the weight stream); TWO_ROWS and THREE_ROWS: up to two or
// three rows per wave (M <= 2W with up to three token blocks, M <= 3W with
// four). K <= kRegRowK.
// The value of a mode is the number of activation rows a wave holds in
// registers across its first weight requests.
enum Mode { ONE_ROW = 1, TWO_ROWS = 2, THREE_ROWS = 3 };

// Split kernel: weight waves + quantiser waves per workgroup, and the
// 128-byte windows a weight wave keeps in flight: 24 (a K = 3072 row group
// whole), fewer with three or four token blocks (whose LDS reads and
// accumulators leave no room for 24 within 128 registers).
constexpr int kMaxSplitWaves = 16;
constexpr int windows_in_flight(int TB) { return TB >= 4 ? 12 : TB >= 3 ? 16 : 24; }

// LDS row stride for the quantised activations: K rounded up to whole
// 128-byte windows plus 32 bytes. One quarter-wave of the "B" read takes 8
// tokens x 2 adjacent 16-byte chunks; with the stride an odd multiple of 32
// modulo 256 after the padding (or 32 itself), those 16 chunks fall into 16
// distinct 16-byte bank groups.
__host__ __device__ inline int xs_stride(int64_t K) { return (int)((K + 127) / 128) * 128 + 32; }

// Split kernel, how the quantiser waves hold their rows: kStaged, every row
// in LDS as bf16 (slot stride staged_stride, the int8 codes written over the
// slot's first K bytes), wherever 8 TB slots fit; otherwise kRegs, two rows
// in registers (K <= kRegRowK), or kTwoPass, longer rows read twice from
// memory.
constexpr int kRegs = 0, kStaged = 1, kTwoPass = 2;
__host__ __device__ inline int staged_stride(int64_t K) { return (int)((K + 127) / 128) * 256 + 32; }
constexpr size_t kMaxLds = 160 * 1024 - 1024;   // dynamic LDS a workgroup may take (static: sa_lds)


// Quantises the row chunks held in v (chunk lane + 64*u of the row, u < Q)
// with the row's scale into the LDS row xrow (and the global row qrow if
// write_q); returns the scale.
template <bool F16, int Q = kQ>
__device__ __forceinline__ float quantise_regs(const uint4 (&v)[Q], uint32_t nchunks, int lane,
                                               int8_t* xrow, int8_t* qrow, bool write_q) {
  uint32_t amax = 0;
#pragma unroll
  for (int u = 0; u < Q; ++u) amax = absmax_bits8(v[u], amax);
  amax = wave_max_u32(amax);
  const float s = row_scale<F16>(amax);
  const bool zero = (amax == 0);
  const bool exact_div = (__float_as_uint(s) & 0x7f800000u) == 0;
  const float r = (zero || exact_div) ? 0.0f : 1.0f / s;
#pragma unroll
  for (int u = 0; u < Q; ++u) {
    if (64u * u >= nchunks) break;        // wave-uniform: no chunk of this batch is in the row
    const uint32_t idx = lane + 64 * u;
    const uint2 q = quant8<F16>(v[u], s, r, zero, exact_div);
    if (idx < nchunks) {
      *reinterpret_cast<uint2*>(xrow + 8 * idx) = q;
      if (write_q) *reinterpret_cast<uint2*>(qrow + 8 * idx) = q;
    }
  }
  return s;
}

// Rows longer than 64*kQ chunks: an amax pass, then a quantise pass that
// reads the row again.
template <bool F16>
__device__ __forceinline__ float quantise_long(__amdgpu_buffer_rsrc_t rx, uint32_t nchunks, int lane,
                                               int8_t* xrow) {
  constexpr int U = 8;
  uint32_t amax = 0;
  for (uint32_t base = 0; base < nchunks; base += 64 * U) {
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = load16(rx, (base + lane + 64 * u) * 16u);
#pragma unroll
    for (int u = 0; u < U; ++u) amax = absmax_bits8(w[u], amax);
  }
  amax = wave_max_u32(amax);
  const float s = row_scale<F16>(amax);
  const bool zero = (amax == 0);
  const bool exact_div = (__float_as_uint(s) & 0x7f800000u) == 0;
  const float r = (zero || exact_div) ? 0.0f : 1.0f / s;
  for (uint32_t base = 0; base < nchunks; base += 64 * U) {
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = load16(rx, (base + lane + 64 * u) * 16u);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t idx = base + lane + 64 * u;
      const uint2 q = quant8<F16>(w[u], s, r, zero, exact_div);
      if (idx < nchunks) *reinterpret_cast<uint2*>(xrow + 8 * idx) = q;
    }
  }
  return s;
}

// Up to kMaxWaves waves per workgroup: three waves per SIMD. TB: blocks of 8
// tokens (1 to 4).
template <bool HAS_BIAS, int TB, int MODE, bool F16>
__global__ __launch_bounds__(64 * kMaxWaves) __attribute__((amdgpu_waves_per_eu(3, 8))) void small_m_rows_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, GemmArgs a, int8_t* __restrict__ xq_out,
    float* __restrict__ sa_out, int vec_flags, int G) {
  extern __shared__ __attribute__((aligned(16))) int8_t xs[];
  __shared__ float sa_lds[8 * TB];
  // two or three rows per wave: the epilogue scales and biases of each
  // wave's rows, parked here once they have landed (in registers across the
  // stream they would make these modes spill)
  constexpr int R = MODE;
  __shared__ float scl_lds[R >= 2 ? kMaxWaves : 1][16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int W = blockDim.x >> 6;
  const int M = (int)a.M;
  const int64_t K = a.K, N = a.N;
  const int ldxs = xs_stride(K);
  const int nwin = (int)((K + 127) / 128);
  // waves G.. of the workgroup own no weight rows: they only help quantise
  const int64_t n_base = ((int64_t)blockIdx.x * G + wave) * 8;
  const int rows_valid = wave < G ? (int)max<int64_t>(0, min<int64_t>(8, N - n_base)) : 0;
  const uint32_t nchunks = (uint32_t)(K >> 3);
  // epilogue scale and bias (row n_base + lane % 8), requested before anything else
  float sw1, bb1;
  load_row_scale<HAS_BIAS, F16>(a.w_scale, a.bias, n_base, rows_valid, lane, sw1, bb1);
  const bool write_q = blockIdx.x == 0;

  // weight windows: lane l reads row l%8, 16-byte chunk l/8 of window w
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(a.wq + (rows_valid > 0 ? n_base : 0) * K, (uint32_t)rows_valid * (uint32_t)K);
  const int chunk = lane >> 3;
  const uint32_t lane_off = (uint32_t)(lane & 7) * (uint32_t)K + 16u * chunk;
  auto wload = [&](int w) -> v4i {
    const bool in = 128 * w + 16 * chunk < K;          // chunks past K read as zero
    // non-temporal: the weight is streamed once; without the hint the loads
    // allocate in caches that a preceding write-heavy kernel left dirty, and
    // the stream waits on their write-back (measured: 21 against 14 us for
    // the 18432 x 3072 weight at M = 1 right after a DiT block)
    return __builtin_amdgcn_raw_buffer_load_b128(rw, in ? lane_off + 128u * w : kOOB, 0, 2);
  };
  v4i buf[kRowD];

  // ---- 1. activation quantisation into LDS, 2. weight requests ----
  // The K tail of each LDS row up to whole windows is never written: it only
  // meets weights that read as zero. Token rows >= M give unused columns.
  {
    // rows wave + W r (r < R) in registers across the first weight requests
    uint4 v[R][kQ];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int m = wave + W * r;
      if (r == 0 && wave >= M) continue;
      // past M the descriptor is empty: the loads read zero
      const __amdgpu_buffer_rsrc_t rx =
          make_rsrc(x + (int64_t)(m < M ? m : 0) * ldx, m < M ? (uint32_t)K * 2u : 0u);
#pragma unroll
      for (int u = 0; u < kQ; ++u) v[r][u] = load16(rx, (uint32_t)(lane + 64 * u) * 16u);
    }
    // the first kD0 weight requests go out right behind the row loads;
    // vmcnt(kD0) then waits for the rows only (loads complete in order)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < kD0; ++d) buf[d] = wload(d);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<kD0>();
    if constexpr (R >= 2) {
      if (lane < 8) {
        scl_lds[wave][lane] = sw1;
        scl_lds[wave][8 + lane] = bb1;
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int m = wave + W * r;
      if (m < M) {
        const float s = quantise_regs<F16>(v[r], nchunks, lane, xs + m * ldxs, xq_out + (int64_t)m * K,
                                           write_q);
        if (lane == 0) {
          sa_lds[m] = s;
          if (write_q) sa_out[m] = s;
        }
      }
    }
    // the remaining windows, once the rows are in LDS
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = kD0; d < kRowD; ++d) buf[d] = wload(d);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
  }
  if (rows_valid == 0) return;

  // ---- 3. weight streaming ----
  v4i acc[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) acc[t] = v4i{0, 0, 0, 0};
  const int8_t* xb = xs + (lane & 7) * ldxs + 16 * chunk;
  // window w: its LDS read(s) and MFMA(s); windows past the end multiply zero
  // weights, so the LDS read is kept inside the row (its last window)
  auto window = [&](int w, const v4i& wv) {
    const int wc = min(w, nwin - 1);
    v4i b[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) b[t] = *reinterpret_cast<const v4i*>(xb + 8 * t * ldxs + 128 * wc);
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv, b[t], acc[t], 0, 0, 0);
  };
#pragma unroll
  for (int d = 0; d < kRowD; ++d) {
    window(d, buf[d]);
    __builtin_amdgcn_sched_group_barrier(0x100, TB, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, TB, 0);
  }

  // ---- 4. epilogue ----
  // D[i][j] sits in lane 16*(i/4) + j, element i%4. Row n < 8 at token t < 8
  // is D[n][t] + D[n+8][t+8], whose second term is 40 lanes up; lanes 0-7
  // and 16-23 then hold rows nl..nl+3 (nl = 4*(lane/16)) of token lane%8.
  const int src = ((lane + 40) & 63) * 4;
  v4i sum[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) sum[t][r] = acc[t][r] + __builtin_amdgcn_ds_bpermute(src, acc[t][r]);
  float sw[4], bb[4];
  if constexpr (R >= 2) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sw[r] = scl_lds[wave][4 * ((lane >> 4) & 1) + r];
      bb[r] = scl_lds[wave][8 + 4 * ((lane >> 4) & 1) + r];
    }
  } else {
    gather4(sw1, 4 * ((lane >> 4) & 1), sw);
    gather4(bb1, 4 * ((lane >> 4) & 1), bb);
  }
  if ((lane & 8) != 0 || lane >= 32) return;
  const int nl = 4 * (lane >> 4);
  const int64_t n = n_base + nl;
#pragma unroll
  for (int blk = 0; blk < TB; ++blk) {
    const int m = 8 * blk + (lane & 7);
    if (m >= M) continue;
    const v4i c = sum[blk];
    const float sa = sa_lds[m];
    uint32_t y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = f32_to_half_rne<F16>(epilogue_f32<HAS_BIAS>(c[r], sa, sw[r], bb[r]));
    uint16_t* o = a.out + (int64_t)m * a.ldo + n;
    if (nl + 3 < rows_valid && (vec_flags & 1)) {
      *reinterpret_cast<uint2*>(o) = make_uint2(y[0] | (y[1] << 16), y[2] | (y[3] << 16));
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (nl + r < rows_valid) o[r] = (uint16_t)y[r];
    }
    if (a.acc_debug) {
      int32_t* dst = a.acc_debug + (int64_t)m * N + n;
      if (nl + 3 < rows_valid && (vec_flags & 2)) {
        *reinterpret_cast<int4*>(dst) = make_int4(c[0], c[1], c[2], c[3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (nl + r < rows_valid) dst[r] = c[r];
      }
    }
  }
}

// A row of more than 64*kQ chunks staged in LDS as bf16 (row): an amax pass,
// then a quantise pass that writes the int8 codes over the row's first K
// bytes. Codes of chunk batch b land on the bf16 bytes of chunks below half
// of the batch's first chunk, all read in earlier batches or earlier in this
// one (a wave's LDS accesses complete in order).
template <bool F16>
__device__ __forceinline__ float quantise_lds_long(int8_t* row, uint32_t nchunks, int lane) {
  constexpr int U = 8;
  uint32_t amax = 0;
  for (uint32_t base = 0; base < nchunks; base += 64 * U) {
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t idx = base + lane + 64 * u;
      w[u] = idx < nchunks ? *reinterpret_cast<const uint4*>(row + 16 * idx) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) amax = absmax_bits8(w[u], amax);
  }
  amax = wave_max_u32(amax);
  const float s = row_scale<F16>(amax);
  const bool zero = (amax == 0);
  const bool exact_div = (__float_as_uint(s) & 0x7f800000u) == 0;
  const float r = (zero || exact_div) ? 0.0f : 1.0f / s;
  for (uint32_t base = 0; base < nchunks; base += 64 * U) {
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t idx = base + lane + 64 * u;
      w[u] = idx < nchunks ? *reinterpret_cast<const uint4*>(row + 16 * idx) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t idx = base + lane + 64 * u;
      const uint2 q = quant8<F16>(w[u], s, r, zero, exact_div);
      if (idx < nchunks) *reinterpret_cast<uint2*>(row + 8 * idx) = q;
    }
  }
  return s;
}

// Workgroup: H quantiser waves (0..H-1), then S x G weight waves: wave
// H + p G + g streams part p (of S) of the windows of row group g. TB: blocks
// of 8 tokens (1 to 4). REFILL: a part has more windows than
// windows_in_flight(TB), which are refilled as they are consumed. QMODE: how
// the quantisers hold their rows (kRegs, kStaged, kTwoPass). With S > 1 the
// parts' int32 sums meet in LDS after the quantised rows (S x G x TB KiB,
// then G counters) and the last part to finish runs the epilogue.
template <bool HAS_BIAS, int TB, bool REFILL, int QMODE, bool F16>
__global__ __launch_bounds__(64 * kMaxSplitWaves) void small_m_split_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, GemmArgs a, int8_t* __restrict__ xq_out,
    float* __restrict__ sa_out, int vec_flags, int G, int H, int S) {
  extern __shared__ __attribute__((aligned(16))) int8_t xs[];
  __shared__ float sa_lds[8 * TB];

  constexpr int kD = windows_in_flight(TB);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = (int)a.M;
  const int64_t K = a.K, N = a.N;
  const int nwin = (int)((K + 127) / 128);
  const int ldxs = QMODE == kStaged ? staged_stride(K) : xs_stride(K);
  const uint32_t nchunks = (uint32_t)(K >> 3);
  const bool quantiser = wave < H;
  // a weight wave streams windows wlo .. whi-1 of weight rows n_base .. n_base+7
  const int ww = quantiser ? 0 : wave - H;
  const int grp = ww % G, part = ww / G;
  const int64_t n_base = ((int64_t)blockIdx.x * G + grp) * 8;
  const int rows_valid = quantiser ? 0 : (int)max<int64_t>(0, min<int64_t>(8, N - n_base));
  const int nwp = (nwin + S - 1) / S;
  const int wlo = part * nwp, whi = min(nwin, wlo + nwp);

  // weight windows: lane l reads row l%8, 16-byte chunk l/8 of window w
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(a.wq + (rows_valid > 0 ? n_base : 0) * K, (uint32_t)rows_valid * (uint32_t)K);
  const int chunk = lane >> 3;
  const uint32_t lane_off = (uint32_t)(lane & 7) * (uint32_t)K + 16u * chunk;
  auto wload = [&](int w) -> v4i {
    // chunks past K and windows of the other parts read as zero
    const bool in = w < whi && 128 * w + 16 * chunk < K;
    // non-temporal: the weight is streamed once; without the hint the loads
    // allocate in caches that a preceding write-heavy kernel left dirty, and
    // the stream waits on their write-back (measured: 21 against 14 us for
    // the 18432 x 3072 weight at M = 1 right after a DiT block)
    return __builtin_amdgcn_raw_buffer_load_b128(rw, in ? lane_off + 128u * w : kOOB, 0, 2);
  };
  // activation row m (rows past M: an empty descriptor, the loads read zero)
  auto row_rsrc = [&](int m) {
    return make_rsrc(x + (int64_t)(m < M ? m : 0) * ldx, m < M ? (uint32_t)K * 2u : 0u);
  };
  auto load_row = [&](uint4 (&v)[kQ], int m) {
    const __amdgpu_buffer_rsrc_t rx = row_rsrc(m);
#pragma unroll
    for (int u = 0; u < kQ; ++u) v[u] = load16(rx, (uint32_t)(lane + 64 * u) * 16u);
  };

  // The quantiser waves request their rows (all of them when staged, the
  // first two when held in registers) before any weight window is requested
  // (the first barrier orders them): queued behind a CU's weight stream,
  // they would arrive only as it drains. The two roles run apart between
  // the two barriers; every wave passes both.
  if (quantiser) {
    // ---- 1. quantisation into LDS: rows wave, wave + H, ... ----
    // The K tail of each LDS row up to whole windows is never written: it
    // only meets weights that read as zero. Token rows >= M give unused
    // columns.
    const int nr = wave < M ? (M - wave + H - 1) / H : 0;
    if constexpr (QMODE == kStaged) {
      // every row of this wave into its LDS slot as bf16 (LDS-DMA: lane l
      // of an instruction writes the 16 bytes at LDS base + 16*l), all
      // requested before any weight window
      const int row_bytes = (int)K * 2;
      for (int j = 0; j < nr; ++j) {
        const int m = wave + H * j;
        const __amdgpu_buffer_rsrc_t rx = row_rsrc(m);
        for (int c = 0; c < row_bytes; c += 1024)
          if (c + 16 * lane < row_bytes)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, xs + m * ldxs + c, 16, (uint32_t)(c + 16 * lane), 0,
                                                     0, 0);
      }
      lds_barrier();
      wait_vmcnt<0>();
      // each row read back whole (up to 64*kQ chunks; longer rows in two
      // passes over LDS) before its int8 codes overwrite its first K bytes
      for (int j = 0; j < nr; ++j) {
        const int m = wave + H * j;
        float s0;
        if (nchunks <= 64u * kQ) {
          uint4 v[kQ];
#pragma unroll
          for (int u = 0; u < kQ; ++u) {
            const uint32_t idx = lane + 64 * u;
            v[u] = idx < nchunks ? *reinterpret_cast<const uint4*>(xs + m * ldxs + 16 * idx)
                                 : make_uint4(0u, 0u, 0u, 0u);
          }
          s0 = quantise_regs<F16>(v, nchunks, lane, xs + m * ldxs, nullptr, false);
        } else {
          s0 = quantise_lds_long<F16>(xs + m * ldxs, nchunks, lane);
        }
        if (lane == 0) sa_lds[m] = s0;
      }
    } else if constexpr (QMODE == kRegs) {
      uint4 va[kQ], vb[kQ];
      load_row(va, wave);
      load_row(vb, wave + H);
      lds_barrier();
      // two rows in flight: the next row is requested as soon as a register
      // set is free; past the last row the requests are empty (read zero),
      // so every iteration issues the same loads and the waits stay exact
      for (int j = 0; j < nr; j += 2) {
        wait_vmcnt<kQ>();
        const int m0 = wave + H * j;
        const float s0 = quantise_regs<F16>(va, nchunks, lane, xs + m0 * ldxs, nullptr, false);
        if (lane == 0) sa_lds[m0] = s0;
        load_row(va, wave + H * (j + 2));
        wait_vmcnt<kQ>();
        const int m1 = wave + H * (j + 1);
        if (m1 < M) {
          const float s1 = quantise_regs<F16>(vb, nchunks, lane, xs + m1 * ldxs, nullptr, false);
          if (lane == 0) sa_lds[m1] = s1;
        }
        load_row(vb, wave + H * (j + 3));
      }
      wait_vmcnt<0>();                     // the empty requests past the last row
    } else {
      lds_barrier();
      for (int j = 0; j < nr; ++j) {
        const int m = wave + H * j;
        const float s = quantise_long<F16>(row_rsrc(m), nchunks, lane, xs + m * ldxs);
        if (lane == 0) sa_lds[m] = s;
      }
    }
    lds_barrier();
    // workgroup 0 hands the quantised rows and scales to the caller
    if (blockIdx.x == 0) {
      for (int m = wave; m < M; m += H) {
        for (uint32_t c = lane; c < (uint32_t)(K >> 4); c += 64)
          *reinterpret_cast<uint4*>(xq_out + (int64_t)m * K + 16 * c) =
              *reinterpret_cast<const uint4*>(xs + m * ldxs + 16 * c);
        if (lane == 0) sa_out[m] = sa_lds[m];
      }
    }
    return;
  }

  // ---- 2. weight requests ----
  // epilogue scale and bias (row n_base + lane % 8)
  float sw1, bb1;
  load_row_scale<HAS_BIAS, F16>(a.w_scale, a.bias, n_base, rows_valid, lane, sw1, bb1);
  int8_t* const parts_lds = xs + 8 * TB * ldxs;
  uint32_t* const done = reinterpret_cast<uint32_t*>(parts_lds + S * G * TB * 1024);
  if (S > 1 && wave == H && lane < G) done[lane] = 0u;
  lds_barrier();
  v4i buf[kD];
  if (rows_valid > 0) {
#pragma unroll
    for (int d = 0; d < kD; ++d) buf[d] = wload(wlo + d);
    __builtin_amdgcn_sched_barrier(0);     // all requests out before the barrier
  }
  lds_barrier();
  if (rows_valid == 0) return;

  // ---- 3. weight streaming ----
  v4i acc[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) acc[t] = v4i{0, 0, 0, 0};
  const int8_t* xb = xs + (lane & 7) * ldxs + 16 * chunk;
  // window w: its LDS read(s) and MFMA(s); windows past the end multiply zero
  // weights, so the LDS read is kept inside the row (its last window)
  auto window = [&](int w, const v4i& wv) {
    const int wc = min(w, nwin - 1);
    v4i b[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) b[t] = *reinterpret_cast<const v4i*>(xb + 8 * t * ldxs + 128 * wc);
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv, b[t], acc[t], 0, 0, 0);
  };
  if constexpr (!REFILL) {
#pragma unroll
    for (int d = 0; d < kD; ++d) {
      window(wlo + d, buf[d]);
      __builtin_amdgcn_sched_group_barrier(0x100, TB, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, TB, 0);
    }
  } else {
    for (int base = 0; base < nwp; base += kD) {
#pragma unroll
      for (int d = 0; d < kD; ++d) {
        window(wlo + base + d, buf[d]);
        buf[d] = wload(wlo + base + d + kD);
        __builtin_amdgcn_sched_group_barrier(0x100, TB, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, TB, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
  }
  if (S > 1) {
    // this part's sums into LDS; the last part of the group to arrive adds
    // the others' (int32, exact in any order) and runs the epilogue. The
    // counter's release orders the wave's stores before it, its acquire the
    // reads after it.
    v4i* const mine = reinterpret_cast<v4i*>(parts_lds) + (grp * S + part) * TB * 64;
#pragma unroll
    for (int t = 0; t < TB; ++t) mine[t * 64 + lane] = acc[t];
    uint32_t before = 0u;
    if (lane == 0)
      before = __hip_atomic_fetch_add(done + grp, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    before = __builtin_amdgcn_readfirstlane(before);
    if (before + 1u < (uint32_t)S) return;
    for (int p = 0; p < S; ++p) {
      if (p == part) continue;
      const v4i* const other = reinterpret_cast<const v4i*>(parts_lds) + (grp * S + p) * TB * 64;
#pragma unroll
      for (int t = 0; t < TB; ++t) acc[t] += other[t * 64 + lane];
    }
  }

  // ---- 4. epilogue ----
  // D[i][j] sits in lane 16*(i/4) + j, element i%4. Row n < 8 at token t < 8
  // is D[n][t] + D[n+8][t+8], whose second term is 40 lanes up; lanes 0-7
  // and 16-23 then hold rows nl..nl+3 (nl = 4*(lane/16)) of token lane%8.
  const int src = ((lane + 40) & 63) * 4;
  v4i sum[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) sum[t][r] = acc[t][r] + __builtin_amdgcn_ds_bpermute(src, acc[t][r]);
  float sw[4], bb[4];
  gather4(sw1, 4 * ((lane >> 4) & 1), sw);
  gather4(bb1, 4 * ((lane >> 4) & 1), bb);
  if ((lane & 8) != 0 || lane >= 32) return;
  const int nl = 4 * (lane >> 4);
  const int64_t n = n_base + nl;
#pragma unroll
  for (int blk = 0; blk < TB; ++blk) {
    const int m = 8 * blk + (lane & 7);
    if (m >= M) continue;
    const v4i c = sum[blk];
    const float sa = sa_lds[m];
    uint32_t y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = f32_to_half_rne<F16>(epilogue_f32<HAS_BIAS>(c[r], sa, sw[r], bb[r]));
    uint16_t* o = a.out + (int64_t)m * a.ldo + n;
    if (nl + 3 < rows_valid && (vec_flags & 1)) {
      *reinterpret_cast<uint2*>(o) = make_uint2(y[0] | (y[1] << 16), y[2] | (y[3] << 16));
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (nl + r < rows_valid) o[r] = (uint16_t)y[r];
    }
    if (a.acc_debug) {
      int32_t* dst = a.acc_debug + (int64_t)m * N + n;
      if (nl + 3 < rows_valid && (vec_flags & 2)) {
        *reinterpret_cast<int4*>(dst) = make_int4(c[0], c[1], c[2], c[3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (nl + r < rows_valid) dst[r] = c[r];
      }
    }
  }
}

// Quantiser waves for M rows next to G weight waves in the split kernel: one
// per row up to four rows, above that a multiple of four (the waves are
// dealt over the CU's four SIMDs in order, so each SIMD carries the same
// share of the rows), as many as fit beside the weight waves.
inline int quantiser_waves(int M, int G) {
  if (M <= 4) return M;
  const int fit = (kMaxSplitWaves - G) / 4;
  const int want = (M + 3) / 4;
  const int h = 4 * (want < fit ? want : fit);
  return h < M ? h : M;
}

template <bool HAS_BIAS, int TB, bool F16>
hipError_t launch_variant(const uint16_t* x, int64_t ldx, const GemmArgs& a, int8_t* xq_out,
                          float* a_scale_out, hipStream_t stream) {
  const RowGroupGrid g = row_group_grid(a.N);
  const int G = g.waves;
  const size_t lds = (size_t)(8 * TB) * (size_t)xs_stride(a.K);
  const int vf = epilogue_vec_flags(a);
  const int H = quantiser_waves((int)a.M, G);
  // The split kernel for rows too long for registers, and above 8 rows when
  // each quantiser wave has at most three rows to fetch; the row-mode kernel
  // otherwise (see the header).
  if (a.K > kRegRowK || (a.M > 8 && (a.M + H - 1) / H <= 3)) {
    // Rows longer than kRegRowK: down to one weight wave per workgroup, so
    // that a narrow weight still spreads over every CU (1 x 8192 -> 2048:
    // 13.8 -> 11.6 us, 12 x 8192 -> 1024: 18.3 -> 16.4 us; with shorter rows
    // the four-wave floor measured the same or better)
    const RowGroupGrid gs = a.K > kRegRowK ? row_group_grid(a.N, 1) : g;
    const int Gs = gs.waves, Hs = a.K > kRegRowK ? quantiser_waves((int)a.M, Gs) : H;
    // One token block with more windows than a wave keeps in flight: two
    // weight waves per row group, each streaming half of K, where the
    // workgroup has room for them
    const int nwin = (int)((a.K + 127) / 128);
    const int S = (TB == 1 && nwin > windows_in_flight(TB) && 2 * Gs + Hs <= kMaxSplitWaves) ? 2 : 1;
    const size_t parts = S > 1 ? (size_t)(S * Gs * TB * 1024 + 4 * Gs) : 0;
    const dim3 grid(gs.blocks), block(64 * (S * Gs + Hs));
#define W8A8_SMALL_M(REFILL, QMODE, LDS)                                                         \
  hipLaunchKernelGGL((small_m_split_kernel<HAS_BIAS, TB, REFILL, QMODE, F16>), grid, block,      \
                     (LDS) + parts, stream, x, ldx, a, xq_out, a_scale_out, vf, Gs, Hs, S)
    const size_t staged_lds = (size_t)(8 * TB) * (size_t)staged_stride(a.K);
    const bool refill = (nwin + S - 1) / S > windows_in_flight(TB);
    if (staged_lds + parts <= kMaxLds) {
      if (refill) W8A8_SMALL_M(true, kStaged, staged_lds);
      else W8A8_SMALL_M(false, kStaged, staged_lds);
    } else if (a.K > kRegRowK) {
      W8A8_SMALL_M(true, kTwoPass, lds);
    } else if (refill) {
      W8A8_SMALL_M(true, kRegs, lds);
    } else {
      W8A8_SMALL_M(false, kRegs, lds);
    }
#undef W8A8_SMALL_M
    return hipGetLastError();
  }
  // Above 8 rows, kMaxWaves waves quantise the rows whatever the weight rows
  // per workgroup (G groups), so the per-workgroup quantisation has three
  // waves per SIMD to hide its latency and spread its VALU work.
  const int threads = 64 * (TB >= 2 ? kMaxWaves : G);
  const dim3 grid(g.blocks), block(threads);
  // at most one, two or three activation rows per wave: one or two with one
  // token block, two with two or three (9 to 12 rows take the split kernel),
  // three with four; every M the launcher sends here fits (see launch_dtype)
#define W8A8_SMALL_M(MODE)                                                                           \
  hipLaunchKernelGGL((small_m_rows_kernel<HAS_BIAS, TB, MODE, F16>), grid, block, lds, stream, x, ldx, \
                     a, xq_out, a_scale_out, vf, G)
  const int64_t waves = threads / 64;
  if constexpr (TB == 4) {
    if (a.M > 3 * waves) return hipErrorInvalidValue;
    W8A8_SMALL_M(THREE_ROWS);
  } else {
    if (a.M > 2 * waves) return hipErrorInvalidValue;
    if constexpr (TB == 1) {
      if (a.M <= waves) W8A8_SMALL_M(ONE_ROW);
      else W8A8_SMALL_M(TWO_ROWS);
    } else {
      W8A8_SMALL_M(TWO_ROWS);
    }
  }
#undef W8A8_SMALL_M
  return hipGetLastError();
}

// Token blocks by M (launch_dtype) against the rows the row modes hold: one
// block (M <= 8) on at least kMinWaves waves, two or three on kMaxWaves.
static_assert(8 <= 2 * kMinWaves && 24 <= 2 * kMaxWaves && kSmallMWideRows <= 3 * kMaxWaves,
              "every small-M row count fits a row mode");
static_assert(kMaxWaves + 4 <= kMaxSplitWaves, "four quantiser waves fit beside every weight-wave count");

template <bool F16>
hipError_t launch_dtype(const uint16_t* x, int64_t ldx, const GemmArgs& a, int8_t* xq_out,
                        float* a_scale_out, hipStream_t stream) {
  if (a.bias) {
    if (a.M > 24) return launch_variant<true, 4, F16>(x, ldx, a, xq_out, a_scale_out, stream);
    if (a.M > 16) return launch_variant<true, 3, F16>(x, ldx, a, xq_out, a_scale_out, stream);
    return a.M > 8 ? launch_variant<true, 2, F16>(x, ldx, a, xq_out, a_scale_out, stream)
                   : launch_variant<true, 1, F16>(x, ldx, a, xq_out, a_scale_out, stream);
  }
  if (a.M > 24) return launch_variant<false, 4, F16>(x, ldx, a, xq_out, a_scale_out, stream);
  if (a.M > 16) return launch_variant<false, 3, F16>(x, ldx, a, xq_out, a_scale_out, stream);
  return a.M > 8 ? launch_variant<false, 2, F16>(x, ldx, a, xq_out, a_scale_out, stream)
                 : launch_variant<false, 1, F16>(x, ldx, a, xq_out, a_scale_out, stream);
}

}  // namespace

hipError_t launch_small_m(const uint16_t* x, int64_t ldx, const GemmArgs& a, int8_t* xq_out,
                          float* a_scale_out, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  if (a.M > kSmallMWideRows || a.K > (a.M > 16 ? kSmallMWideMaxK : kSmallMMaxK))
    return hipErrorInvalidValue;
  return a.f16 ? launch_dtype<true>(x, ldx, a, xq_out, a_scale_out, stream)
               : launch_dtype<false>(x, ldx, a, xq_out, a_scale_out, stream);
}

}  // namespace w8a8
