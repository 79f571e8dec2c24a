// The decode launcher for K/V pools in mapped pinned host memory: the same
// kernel (kvsp_attend.h) with row-major K loads, which cross PCIe in larger
// requests (SparPR news page: the full cache lives off the GPU and only what
// is selected crosses to it).

#include "kvsp_attend.h"

namespace kvsp {

hipError_t launch_decode_host(const DecodeArgs& a, int dtype, int group_pad, int num_wgs,
                              hipStream_t stream) {
  return launch_decode_kind<true>(a, dtype, group_pad, num_wgs, stream);
}

}  // namespace kvsp
