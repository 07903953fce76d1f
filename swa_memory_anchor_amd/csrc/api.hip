// Host-side closed forms and status strings of the RMA C ABI.
//
// Sizes follow fluxbbs.com "EdgeRock-4B 开源：72 MiB 固定 KV，AIME 82.9 分", section
// "72 MiB 是怎么算出来的": per layer and sequence, K and V of a 1024-slot window,
// a 1024-record bank and a 256-record pending block for each of 4 KV groups at
// head width 256 in BF16 -- 9 MiB, i.e. 72 MiB over the 8 SWA||RMA layers.
#include "rma_device.h"

using namespace rma;

extern "C" size_t rma_layer_kv_bytes(int32_t batch) {
  if (batch <= 0) return 0;
  return static_cast<size_t>(batch) * 2 * kGroups * (kWindow + kBank + kBlock) * kDim *
         sizeof(uint16_t);
}

extern "C" size_t rma_layer_state_bytes(int32_t batch) {
  if (batch <= 0) return 0;
  const size_t per_seq_meta = static_cast<size_t>(kGroups) * kBank * (sizeof(float) + sizeof(int32_t)) +
                              static_cast<size_t>(kBlock) * (kGroups * sizeof(float) + sizeof(int32_t)) +
                              3 * sizeof(int32_t);
  return rma_layer_kv_bytes(batch) + static_cast<size_t>(batch) * per_seq_meta;
}

// FP8 variant: 1-byte codes plus one FP32 scale per K and V row.
extern "C" size_t rma_layer_state_fp8_bytes(int32_t batch) {
  if (batch <= 0) return 0;
  const size_t rows = static_cast<size_t>(2) * kGroups * (kWindow + kBank + kBlock);
  const size_t per_seq_meta = static_cast<size_t>(kGroups) * kBank * (sizeof(float) + sizeof(int32_t)) +
                              static_cast<size_t>(kBlock) * (kGroups * sizeof(float) + sizeof(int32_t)) +
                              3 * sizeof(int32_t);
  return static_cast<size_t>(batch) * (rows * (kDim + sizeof(float)) + per_seq_meta);
}

extern "C" const char *rma_status_str(rma_status s) {
  switch (s) {
    case RMA_OK: return "RMA_OK";
    case RMA_E_ARG: return "RMA_E_ARG: invalid argument";
    case RMA_E_ALIGN: return "RMA_E_ALIGN: pointer or stride not 16-byte aligned";
    case RMA_E_WORKSPACE: return "RMA_E_WORKSPACE: workspace missing or too small";
    case RMA_E_HIP: return "RMA_E_HIP: HIP launch error";
  }
  return "RMA_E_UNKNOWN";
}
