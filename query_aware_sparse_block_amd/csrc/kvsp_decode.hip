// The decode launcher for K/V pools in device memory. The kernel and its
// work decomposition are in kvsp_attend.h; pools in host memory are launched
// from kvsp_decode_host.hip.

#include "kvsp_attend.h"

namespace kvsp {

hipError_t launch_decode(const DecodeArgs& a, int dtype, int group_pad, int num_wgs,
                         hipStream_t stream) {
  return launch_decode_kind<false>(a, dtype, group_pad, num_wgs, stream);
}

int decode_chunk_quantum(int dtype, int D) {
  const int E = dtype == KVSP_F32 ? 4 : 2;
  const int sub = KVSP_SUB_TILE_BYTES / (D * E) < 16 ? 16 : KVSP_SUB_TILE_BYTES / (D * E);
  return kDecodeWaves * sub;
}

}  // namespace kvsp
