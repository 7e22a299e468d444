// Producers fused with the per-row int8 activation quantisation (host side).
//
// The modulated LayerNorm (in front of a DiT block's QKV and FFN-up linears)
// and GELU (in front of FFN-down) write the next linear's int8 codes and
// per-row scales directly instead of a bf16 row for a separate quantisation
// pass ("Qwen-Image-2.1 ...", section "Whole-pipeline follow-up": fused
// activation-quantisation, normalisation and activation kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

constexpr int kProducerLayerNorm = 0;   // (x - mean) rstd (1 + scale) + shift
constexpr int kProducerGelu = 1;        // z Phi(z)
constexpr int kProducerGeluTanh = 2;    // 0.5 z (1 + tanh(sqrt(2/pi)(z + 0.044715 z^3)))

// Longest rows the register-resident kernels take.
constexpr int64_t kProducerMaxK[3] = {16384, 32768, 32768};

struct ProducerArgs {
  int op;                       // kProducer*
  const uint16_t* x;            // bf16 [M, ldx]
  int64_t M, K, ldx;
  const uint16_t* shift;        // LayerNorm: bf16 [G, ld_mod], row m uses group m / rows_per_group
  const uint16_t* scale;
  int64_t ld_mod, rows_per_group;
  float eps;
  int8_t* xq;                   // [M, K]
  float* a_scale;               // [M]
  uint16_t* y;                  // bf16 [M, ldy] or nullptr: the producer's bf16 row
  int64_t ldy;
};

hipError_t launch_producer_quant(const ProducerArgs& a, hipStream_t stream);

}  // namespace w8a8
