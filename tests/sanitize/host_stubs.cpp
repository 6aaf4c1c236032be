// Stand-ins for the HIP runtime and the kernel launchers, for the
// sanitizer build of the library's host code (validation, bank addressing,
// workspace sizing, the page manager) on a machine without a GPU. Every
// device query reports no device and every launch fails, as the real
// runtime does on such a machine, so each entry point runs its host logic
// and stops where it would enqueue work. Test infrastructure only.
#include <hip/hip_runtime.h>

#include "launch.hpp"

extern "C" {

hipError_t hipGetDevice(int *) { return hipErrorNoDevice; }
hipError_t hipDeviceGetAttribute(int *, hipDeviceAttribute_t, int) { return hipErrorNoDevice; }
const char *hipGetErrorString(hipError_t) { return "no device (host-only sanitizer build)"; }
hipError_t hipStreamBeginCapture(hipStream_t, hipStreamCaptureMode) { return hipErrorNoDevice; }
hipError_t hipStreamEndCapture(hipStream_t, hipGraph_t *g) {
  if (g) *g = nullptr;
  return hipErrorNoDevice;
}
hipError_t hipGraphInstantiate(hipGraphExec_t *, hipGraph_t, hipGraphNode_t *, char *, size_t) {
  return hipErrorNoDevice;
}
hipError_t hipGraphDestroy(hipGraph_t) { return hipSuccess; }
hipError_t hipGraphExecDestroy(hipGraphExec_t) { return hipSuccess; }
hipError_t hipGraphLaunch(hipGraphExec_t, hipStream_t) { return hipErrorNoDevice; }

}  // extern "C"

namespace pkv {

hipError_t launch_kv_write(const Bank &, const void *, const void *, const int32_t *, int32_t,
                           hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_decode(const DecodeArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_stream(const DecodeArgs &, int64_t, hipStream_t) {
  return hipErrorNoDevice;
}
int stream_waves(int, int, int, int num_cus) { return num_cus * 4; }
hipError_t launch_reduce(int32_t, int32_t, int32_t, int32_t, const int32_t *, int32_t, int32_t,
                         int32_t, const float *, const float *, const float *, void *, float *,
                         bool, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_prefill(const PrefillArgs &, hipStream_t) { return hipErrorNoDevice; }

}  // namespace pkv

// The allocation-free decode entry point without its device array: the
// scratch lookup reports no device, after the shared validation has run.
extern "C" int paged_decode_attn_noalloc(const pkv_pool *pool, int32_t plane_id,
                                         int32_t layer_id, const void *q, int32_t num_q_heads,
                                         const int32_t *page_table, int32_t page_table_stride,
                                         const int32_t *seq_lens, int32_t batch,
                                         int32_t max_seq_len, float scale, int32_t partition,
                                         void *out, float *lse, void *stream) {
  auto no_scratch = [](void **) { return pkv::set_error(PKV_ELAUNCH, "no device"); };
  return pkv::decode_scratch(pool, plane_id, layer_id, q, num_q_heads, page_table,
                             page_table_stride, seq_lens, batch, max_seq_len, scale, partition,
                             out, lse, +no_scratch, (size_t)PKV_SCRATCH_BYTES, stream);
}
