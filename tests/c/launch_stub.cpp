// Host stand-ins for the kernel launchers, for the sanitizer build of the
// plan and ABI code (tests/c/sanitize_host.cpp): no kernel is compiled, and
// every launch reports that no device is present.  The argument checks all
// run before the first launch, so they are exercised in full.
#include "kernels.hpp"

namespace fsdp {

hipError_t launch_copy(const Work*, int64_t, const void*, const PtrArray&, int, int, int, bool,
                       const Sink&) {
  return hipErrorNoDevice;
}
hipError_t launch_pack_cast(const Work*, int64_t, const void*, int, void*, int, bool,
                            const Sink&) {
  return hipErrorNoDevice;
}
hipError_t launch_rs_avg(const Work*, int64_t, const PtrArray&, int, int, float*, bool,
                         const Sink&) {
  return hipErrorNoDevice;
}
hipError_t launch_adamw(int64_t, const float*, float*, float*, float*, void*, int,
                        const AdamScalars&, const AdamScalars*, bool, const Sink&) {
  return hipErrorNoDevice;
}
hipError_t launch_fused(const Work*, int64_t, const PtrArray&, int, int, float*, float*, float*,
                        void*, int, const AdamScalars&, const AdamScalars*, bool, const Sink&) {
  return hipErrorNoDevice;
}
hipError_t launch_accumulate(int64_t, int, const PtrArray&, int, const PtrArray&, bool, bool,
                             const Sink&) {
  return hipErrorNoDevice;
}
hipError_t launch_allreduce(int64_t, int, const PtrArray&, int, const PtrArray&, int, bool,
                            const Sink&) {
  return hipErrorNoDevice;
}
hipError_t launch_copy_pairs(const Work*, int64_t, const PtrArray&, const PtrArray&, int, int,
                             bool, const Sink&) {
  return hipErrorNoDevice;
}
hipError_t launch_set_scalars(AdamScalars*, const AdamScalars&, const Sink&) {
  return hipErrorNoDevice;
}
hipError_t launch_fused_gather(const Work*, int64_t, const PtrArray&, int, int, float*, float*,
                               float*, void*, int, const AdamScalars&, const AdamScalars*, bool,
                               const Work*, int64_t, const void*, const PtrArray&, int, int, bool,
                               const Sink&) {
  return hipErrorNoDevice;
}
hipError_t StreamSink::launch(const void*, dim3, dim3, void**, unsigned) const {
  return hipErrorNoDevice;
}

}  // namespace fsdp
